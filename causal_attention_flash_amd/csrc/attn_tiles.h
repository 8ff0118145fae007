// Global -> LDS staging of bf16 row tiles ([rows][D], D contiguous) for the
// gfx950 attention kernels.  A tile is fetched with 16-byte loads into
// registers first (issued an iteration ahead, so the loads overlap the MFMA work
// on earlier tiles), then written to LDS row-major as [ROWS][D + 8].
//
// Operand reads of 8 consecutive columns use 16-byte ds_read_b128; operand reads
// that contract over the rows use the transposing read (lds_tr_operand), so no
// tile is ever stored transposed.  The 8-element pad per row staggers
// consecutive rows across LDS banks for both kinds of read.  Rows at or beyond S
// are zero-filled, so tail tiles need no special path downstream of the load.
#pragma once

#include "attn_device.h"

namespace attn {

template <int ROWS, int D, int NT = 256>
struct RowTile {
    static constexpr int STR = D + 8;          // LDS row stride (elements)
    static constexpr int ELEMS = ROWS * STR;   // LDS footprint (elements)
    static constexpr int CPR = D / 8;          // 16-byte chunks per row
    static constexpr int CHUNKS = ROWS * CPR;
    static constexpr int PT = (CHUNKS + NT - 1) / NT;
    static_assert(ROWS % 32 == 0 && D % 32 == 0, "tile shape");

    u32x4 r[PT];

    __device__ __forceinline__ void load(const uint16_t* __restrict__ g, int row0, int S, int tid) {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int c = tid + i * NT;
            u32x4 a = {0u, 0u, 0u, 0u};
            if (CHUNKS % NT == 0 || c < CHUNKS) {
                const int row = row0 + c / CPR;
                if (row < S) a = ldg16(g + (size_t)row * D + (c % CPR) * 8);
            }
            r[i] = a;
        }
    }

    __device__ __forceinline__ void store(uint16_t* s, int tid) const {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int c = tid + i * NT;
            if (CHUNKS % NT == 0 || c < CHUNKS)
                *reinterpret_cast<u32x4*>(s + (c / CPR) * STR + (c % CPR) * 8) = r[i];
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
