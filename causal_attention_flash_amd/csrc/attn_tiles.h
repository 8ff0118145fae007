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

// Buffer resource covering `bytes` bytes from `base`.  Raw buffer loads through
// it are range-checked by the hardware: bytes at or beyond the end read as zero
// and nothing outside the range is accessed.  Dword 3 = 0x00020000 selects the
// 32-bit data format that untyped buffer loads require on gfx9-family parts.
// `bytes` must be the same in every lane; it is read from the first lane so that
// the descriptor lives in scalar registers (a clamp computed on the vector unit
// would otherwise make the compiler wrap each load in a per-lane loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

template <int ROWS, int D, int NT = 256>
struct RowTile {
    static constexpr int STR = D + 8;          // LDS row stride (elements)
    static constexpr int ELEMS = ROWS * STR;   // LDS footprint (elements)
    static constexpr int CPR = D / 8;          // 16-byte chunks per row
    static constexpr int CHUNKS = ROWS * CPR;
    static constexpr int PT = (CHUNKS + NT - 1) / NT;
    // Transposing reads cover whole 32-column output tiles (HeadDim::DB of
    // them), so when 32*DB > STR the last row's read runs past the tile by the
    // difference; a buffer holding tiles reserves this many elements after its
    // last tile.
    static constexpr int TR_SLACK = HeadDim<D>::DB * 32 > STR ? HeadDim<D>::DB * 32 - STR : 0;
    static_assert(ROWS % 32 == 0 && D % 16 == 0, "tile shape");

    u32x4 r[PT];

    // Rows row0 .. row0+ROWS-1 of the [S][D] matrix g; rows at or beyond S read
    // as zero (the buffer range ends at row S).
    __device__ __forceinline__ void load(const uint16_t* __restrict__ g, int row0, int S, int tid) {
        const int rows = max(0, min(S - row0, ROWS));
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(g + (size_t)row0 * D, rows * D * 2);
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int c = tid + i * NT;
            if (CHUNKS % NT == 0 || c < CHUNKS)
                r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, c * 16, 0, 0);
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

// Per-row fp32 statistics of a tile of query rows, in the form the backward
// accumulators start from: -LSE/scale (S - LSE/scale is the exponent of P
// before the factor scale*log2(e)) and -delta.  Rows past S get -inf, so P is
// exactly 0 there.  load() only issues the loads; the transform happens in
// store(), so no wait for the loads is placed at the point of issue.
template <int ROWS, int NT = 256>
struct RowStats {
    float l, d;
    bool ok;
    __device__ __forceinline__ void load(const float* __restrict__ lse, const float* __restrict__ delta,
                                         int row0, int S, int tid) {
        const int rows = max(0, min(S - row0, ROWS));
        const __amdgpu_buffer_rsrc_t rl = buffer_rsrc(lse + row0, rows * 4);
        const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(delta + row0, rows * 4);
        l = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, tid * 4, 0, 0));
        d = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rd, tid * 4, 0, 0));
        ok = tid < rows;
    }
    __device__ __forceinline__ void store(float* sa, float* sb, float rscale, int tid) const {
        if (tid < ROWS) {
            sa[tid] = ok ? -l * rscale : -INFINITY;
            sb[tid] = -d;
        }
    }
};

}  // namespace attn
