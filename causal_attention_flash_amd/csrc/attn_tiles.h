// Global -> LDS staging of 16-bit row tiles ([rows][D], D contiguous) for the
// gfx950 attention kernels, and the two LDS layouts the kernels read them from.
//
// Operand reads of 8 consecutive columns use 16-byte ds_read_b128; operand reads
// that contract over the rows use the transposing read (ds_read_b64_tr_b16), so
// no tile is ever stored transposed.  gfx950's LDS has 64 four-byte banks; a
// ds_read_b128 is served 16 lanes per cycle and a 64-bit read (the transposing
// one included) 32 lanes per cycle, and a cycle's lanes conflict when they touch
// one bank at different addresses (measured: each pattern's throughput and
// SQ_LDS_BANK_CONFLICT agree with this model).  The two reads cover:
// * row reads: 16 consecutive rows, one 16-byte chunk each;
// * transposing reads: 32 lanes over rows r .. r+3 (r % 4 == 0) and four
//   consecutive 16-byte chunks (64 bytes) of each.
// Both layouts below make both reads conflict-free.
//
// Padded layout (RowTile: tiles staged through registers).  Row r starts at
// element r * STR + (r / 4) * 8, with the row stride 2 * STR = 64 or 192 mod 256
// bytes: four consecutive rows then start 16 banks apart (their 64-byte windows
// of a transposing read are disjoint), and the extra 16 bytes after every fourth
// row shift the next group of four by 4 banks, so 16 consecutive rows start on
// 16 distinct 4-bank groups (row reads).  Addresses are linear in the lane's row,
// so every per-instruction part folds into the read's immediate offset.
//
// Swizzled layout (DTile in attn_direct.h: tiles loaded straight from HBM,
// which writes each wave's 1 KB contiguously, so rows cannot be padded): row r
// holds RP 16-byte slots (RP = D/8 rounded up to a power of two) and logical
// chunk c sits in slot c ^ slot_swizzle<RP>(r).  Rows of 128 bytes (RP = 8)
// start on bank 0 or 32 by row parity, so rows of equal parity need distinct
// slots; rows of 256 bytes (RP = 16) all start on bank 0, so 16 rows need 16
// distinct slots; rows of 64 bytes (RP = 4) start on 4 bank offsets by r % 4, so
// rows of equal r % 4 need distinct slots.  For the transposing read the
// swizzle moves each row's group of four chunks to a distinct group of slots
// (bit 2 of the slot differs between rows of equal parity at RP = 8; bits 2-3
// differ across the four rows at RP = 16).
#pragma once

#include "attn_device.h"

namespace attn {

constexpr int pow2_up(int x) { return x <= 1 ? 1 : 2 * pow2_up((x + 1) / 2); }

template <int RP>
__host__ __device__ __forceinline__ constexpr int slot_swizzle(int r) {
    static_assert(RP == 4 || RP == 8 || RP == 16, "rows of 4, 8 or 16 slots");
    return RP == 4 ? (r >> 2) & 3
         : RP == 8 ? (((r >> 1) & 1) << 2) | ((r >> 2) & 3)
                   : ((r & 3) << 2) | ((r >> 2) & 3);
}

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
    // row stride (elements): D rounded up to 32 or 96 mod 128 (64 or 192 mod 256 bytes)
    static constexpr int STR = (D % 128 <= 32) ? D - D % 128 + 32 : (D % 128 <= 96 ? D - D % 128 + 96 : D - D % 128 + 160);
    static_assert((2 * STR) % 256 == 64 || (2 * STR) % 256 == 192, "row stride");
    static constexpr int ELEMS = ROWS * STR + ROWS / 4 * 8;  // LDS footprint (elements)
    static constexpr int CPR = D / 8;          // 16-byte chunks per row
    static constexpr int CHUNKS = ROWS * CPR;
    static constexpr int PT = (CHUNKS + NT - 1) / NT;
    static_assert(ROWS % 32 == 0 && D % 16 == 0, "tile shape");
    // Transposing reads cover whole 32-column output tiles (HeadDim::DB of them);
    // the columns past D that they read are dead (computed, never stored) and
    // stay inside the row: 32 * DB <= STR.
    static_assert(HeadDim<D>::DB * 32 <= STR, "transposing reads stay inside the row");

    // element offset of (row, col)
    __host__ __device__ static __forceinline__ constexpr int at(int r, int col) { return r * STR + (r >> 2) * 8 + col; }
    // offset of row r0 (a multiple of 4), so that at(r0 + x, c) = base(r0) + at(x, c)
    __host__ __device__ static __forceinline__ constexpr int base(int r0) { return r0 * STR + (r0 >> 2) * 8; }

    // Row operand of rows r0 .. r0+31 (r0 a multiple of 4): lane (n, h) gets row
    // r0 + n, columns 16ks + 8h .. +7 (the A/B operand layout of attn_device.h).
    // rl = row_lane(lane), computed once.
    __device__ static __forceinline__ int row_lane(int lane) { return at(lane & 31, 8 * (lane >> 5)); }
    template <class E>
    __device__ static __forceinline__ typename E::V8 row_op(const uint16_t* T, int r0, int ks, int rl) {
        return as_op<E>(*reinterpret_cast<const u32x4*>(T + base(r0) + rl + ks * 16));
    }
    // Transposing operand contracting over rows r0 .. r0+15 (r0 a multiple of
    // 16), columns 32db + n: the lds_tr_operand lane map (attn_device.h).
    // tl = tr_lane(lane), computed once.
    __device__ static __forceinline__ int tr_lane(int lane) {
        const int g = lane >> 4, j = lane & 15;
        return at(4 * (g >> 1) + (j >> 2), 16 * (g & 1) + 4 * (j & 3));
    }
    template <class E>
    __device__ static __forceinline__ typename E::V8 tr_op(const uint16_t* T, int r0, int db, int tl) {
        const uint16_t* p = T + base(r0) + tl + db * 32;
        const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
        const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + at(8, 0)));
        return __builtin_bit_cast(typename E::V8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    }

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
                *reinterpret_cast<u32x4*>(s + at(c / CPR, (c % CPR) * 8)) = r[i];
        }
    }
};

// Per-row fp32 statistics of a tile of query rows, in the form the backward
// accumulators start from: -LSE/scale (S - LSE/scale is the exponent of P
// before the factor scale*log2(e)) and -delta.  Rows past S get -inf, so P is
// exactly 0 there.  load() only issues the loads; the transform happens in
// store(), so no wait for the loads is placed at the point of issue.  Without
// DELTA only -LSE/scale is loaded and stored (the caller forms delta).
template <int ROWS, int NT = 256, bool DELTA = true>
struct RowStats {
    float l, d;
    bool ok;
    __device__ __forceinline__ void load(const float* __restrict__ lse, const float* __restrict__ delta,
                                         int row0, int S, int tid) {
        const int rows = max(0, min(S - row0, ROWS));
        const __amdgpu_buffer_rsrc_t rl = buffer_rsrc(lse + row0, rows * 4);
        l = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, tid * 4, 0, 0));
        if constexpr (DELTA) {
            const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(delta + row0, rows * 4);
            d = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rd, tid * 4, 0, 0));
        }
        ok = tid < rows;
    }
    __device__ __forceinline__ void store(float* sa, float* sb, float rscale, int tid) const {
        if (tid < ROWS) {
            sa[tid] = ok ? -l * rscale : -INFINITY;
            if constexpr (DELTA) sb[tid] = -d;
        }
    }
};

}  // namespace attn
