// Global -> LDS staging of bf16 row tiles ([rows][D], D contiguous) for the
// gfx950 attention kernels.  A tile is fetched with 16-byte loads into
// registers first (issued one iteration ahead, so the loads overlap the MFMA
// work on the previous tile), then written to LDS in one or both of two forms:
//
//   row-major   [ROWS][D + 8]   operand reads of 8 consecutive d (16 bytes);
//   transposed  [D][ROWS + 8]   operand reads of 8 rows at one d, stored in the
//                               kperm order of attn_device.h so that one
//                               16-byte read returns a lane's 8 k slots.
//
// The +8 element pad per LDS row staggers consecutive rows across banks for the
// 16-byte operand reads.  Rows at or beyond S are zero-filled, so tail tiles
// need no special path in the loads.
#pragma once

#include "attn_device.h"

namespace attn {

template <int ROWS, int D, int NT = 256>
struct PairTile {
    static constexpr int RSTR = D + 8;      // row-major LDS stride (elements)
    static constexpr int TSTR = ROWS + 8;   // transposed LDS stride (elements)
    static constexpr int CPR = D / 8;       // 16-byte chunks per row
    static constexpr int UNITS = (ROWS / 2) * CPR;  // units of 2 rows x 8 columns
    static constexpr int PT = (UNITS + NT - 1) / NT;
    static_assert(ROWS % 32 == 0 && D % 32 == 0, "tile shape");
    static constexpr int ROW_ELEMS = ROWS * RSTR;
    static constexpr int TRANS_ELEMS = D * TSTR;

    u32x4 r0[PT], r1[PT];

    __device__ __forceinline__ void load(const uint16_t* __restrict__ g, int row0, int S, int tid) {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int u = tid + i * NT;
            u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
            if (UNITS % NT == 0 || u < UNITS) {
                const int p = u / CPR;
                const int col = (u % CPR) * 8;
                const int row = row0 + 2 * p;
                if (row < S) a = ldg16(g + (size_t)row * D + col);
                if (row + 1 < S) b = ldg16(g + (size_t)(row + 1) * D + col);
            }
            r0[i] = a;
            r1[i] = b;
        }
    }

    __device__ __forceinline__ void store_rows(uint16_t* s, int tid) const {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int u = tid + i * NT;
            if (UNITS % NT == 0 || u < UNITS) {
                const int p = u / CPR;
                const int col = (u % CPR) * 8;
                *reinterpret_cast<u32x4*>(s + (2 * p) * RSTR + col) = r0[i];
                *reinterpret_cast<u32x4*>(s + (2 * p + 1) * RSTR + col) = r1[i];
            }
        }
    }

    __device__ __forceinline__ void store_trans(uint16_t* s, int tid) const {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int u = tid + i * NT;
            if (UNITS % NT == 0 || u < UNITS) {
                const int p = u / CPR;
                const int col = (u % CPR) * 8;
                const int pos = kperm(2 * p);  // even; row 2p+1 lands at pos+1
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    *reinterpret_cast<uint32_t*>(s + (col + 2 * e) * TSTR + pos) = pack_lo(r0[i][e], r1[i][e]);
                    *reinterpret_cast<uint32_t*>(s + (col + 2 * e + 1) * TSTR + pos) = pack_hi(r0[i][e], r1[i][e]);
                }
            }
        }
    }
};

// Per-row fp32 statistics (LSE in log2 units, delta) for a tile of query rows.
template <int ROWS, int NT = 256>
struct RowStats {
    float a, b;
    // lse2 = LSE * log2(e); rows past S get +inf so exp2(s - lse2) is exactly 0.
    __device__ __forceinline__ void load(const float* __restrict__ lse, const float* __restrict__ delta,
                                         int row0, int S, int tid) {
        a = INFINITY;
        b = 0.f;
        if (tid < ROWS) {
            const int row = row0 + tid;
            if (row < S) {
                a = lse[row] * kLog2e;
                b = delta[row];
            }
        }
    }
    __device__ __forceinline__ void store(float* sa, float* sb, int tid) const {
        if (tid < ROWS) {
            sa[tid] = a;
            sb[tid] = b;
        }
    }
};

}  // namespace attn
