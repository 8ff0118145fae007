// Direct global -> LDS staging of 16-bit row tiles ([rows][D], D contiguous) for
// the gfx950 attention kernels: buffer_load_dwordx4 ... lds writes each lane's 16
// bytes straight into LDS (at the wave's base + 16 * lane), with no register
// round trip and no ds_write.  The loads are asynchronous: a tile is usable once
// every wave's loads for it have drained (s_waitcnt vmcnt) and a barrier has
// passed; the kernels count their own loads for that.
//
// LDS layout: the swizzled row layout of attn_tiles.h (row r holds RP 16-byte
// slots, logical chunk c in slot c ^ slot_swizzle<RP>(r)).  A wave's load fills 64
// consecutive slots, and each lane fetches the logical chunk that belongs in its
// slot, so the swizzle costs nothing at load time.  Slots past the row's D/8
// chunks are loaded from an offset beyond the buffer range and read as zero.
// Rows at or beyond S also read as zero: the buffer range of a tile ends at row
// S.  Rows of 64 bytes (RP = 4) hold fp8 rows of 64 elements, read only as
// 16-byte row operands.
#pragma once

#include "attn_tiles.h"

namespace attn {


// Byte address within LDS of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Wait for every LDS read issued so far (s_waitcnt lgkmcnt(0)) and tie the raw
// halves of asynchronous reads to it, so that nothing (a use, a copy) reads them
// before the wait.  N counts 64-bit halves.
template <int N>
__device__ __forceinline__ void lds_wait(i16x4 (&x)[N]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(x[i]));
}

// Operand from the two halves of a transposing read.
template <class E>
__device__ __forceinline__ typename E::V8 tr_join(const i16x4 (&h)[2]) {
    const i16x8 r = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(typename E::V8, r);
}

// s_waitcnt vmcnt(n): at most n vector-memory operations of this wave still in
// flight (expcnt and lgkmcnt unconstrained).  n < 64.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    __builtin_amdgcn_sched_barrier(0);
}

// Barrier without the memory fence __syncthreads carries (the fence would wait
// for every load in flight, including prefetches of later tiles).  LDS reads
// issued before it have been consumed by the time a wave reaches it.
__device__ __forceinline__ void bare_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

template <int ROWS, int D, int NW>
struct DTile {
    static constexpr int CPR = D / 8;              // logical 16-byte chunks per row
    static constexpr int RP = pow2_up(CPR);        // slots per LDS row
    static constexpr int RS = RP * 8;              // LDS row stride (elements)
    static constexpr int ELEMS = ROWS * RS;        // LDS footprint (elements)
    static constexpr int LOADS = ROWS * RP / (64 * NW);  // load instructions per wave per tile
    static_assert(ROWS * RP % (64 * NW) == 0, "tile must split evenly over the waves");
    __host__ __device__ static __forceinline__ constexpr int sw(int r) { return slot_swizzle<RP>(r); }

    // Byte offsets (within the tile's global rows) each lane fetches, one per
    // load instruction; slots with no logical chunk get an offset past any range.
    struct Src {
        int off[LOADS];
        __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int p = (i * NW + wave) * 64 + lane;  // slot this lane fills
                const int row = p / RP, slot = p % RP;
                const int c = slot ^ sw(row);
                off[i] = c < CPR ? (row * D + c * 8) * 2 : 0x7fffff00;
            }
        }
    };

    // Issue the loads of rows row0 .. row0+ROWS-1 of the [S][D] matrix g into the
    // LDS tile t; rows at or beyond S read as zero.  row0 must be the same across
    // the wave (it is taken from the first lane, so the buffer descriptor stays in
    // scalar registers whatever the compiler concludes about its uniformity).
    __device__ static __forceinline__ void load(const uint16_t* __restrict__ g, int row0_, int S, uint16_t* t,
                                                const Src& src, int wave) {
        const int row0 = __builtin_amdgcn_readfirstlane(row0_);
        const int rows = max(0, min(S - row0, ROWS));
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(g + (size_t)row0 * D, rows * D * 2);
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(t + (i * NW + wave) * 512), 16, src.off[i], 0, 0,
                0);
    }

    // element offset of logical (row, col), col % 4 == 0
    __host__ __device__ static __forceinline__ int at(int r, int col) {
        return r * RS + ((((col >> 3) ^ sw(r)) << 3) | (col & 7));
    }
};

// Per-lane LDS offsets for the two operand reads of a swizzled tile (DTile or
// RowTile), computed once (the swizzle depends on the row modulo 16 only, and
// every row step the kernels add is a multiple of 16).
//   row[ks]   : 16-byte row operand, row n, columns 16ks + 8h .. +7
//   tr[db][e] : transposing read (the lds_tr_operand lane map) for columns
//               32db.., rows +0 (e = 0) and +8 (e = 1) of a 16-row step
template <class TILE, int D>
struct DOffsets {
    static constexpr int KS = HeadDim<D>::KSTEPS;
    static constexpr int DB = HeadDim<D>::DB;
    int row[KS];
    int tr[DB][2];
    __device__ __forceinline__ void init(int lane) {
        const int n = lane & 31, h = lane >> 5, g = lane >> 4, j = lane & 15;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) row[ks] = TILE::at(n, ks * 16 + 8 * h);
        const int rr = 4 * (g >> 1) + (j >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int col = db * 32 + 16 * (g & 1) + 4 * (j & 3);
            tr[db][0] = TILE::at(rr, col);
            tr[db][1] = TILE::at(rr + 8, col);
        }
    }
    // row operand of row r0 + n (r0 a multiple of 8)
    template <class E>
    __device__ __forceinline__ typename E::V8 row_op(const uint16_t* T, int r0, int ks) const {
        return as_op<E>(lds16(T + r0 * TILE::RS + row[ks]));
    }
    // Transposing read of the operand contracting over rows r0 .. r0+15 (r0 a
    // multiple of 16), columns 32db + n (the lds_tr_operand lane map), through the
    // compiler's builtin: it waits for the read where the operand is used.
    template <class E>
    __device__ __forceinline__ typename E::V8 tr_op(const uint16_t* T, int r0, int db) const {
        const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(T + r0 * TILE::RS + tr[db][0]));
        const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(T + r0 * TILE::RS + tr[db][1]));
        return __builtin_bit_cast(typename E::V8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    // The same read issued as inline assembly into two raw
    // halves.  The compiler does not see an LDS read there, so it adds no wait for
    // the loads in flight (which it would otherwise do before every transposing
    // read, unable to tell it from a load's LDS write).  The halves hold data only
    // after lds_wait() has taken them; tr_join() then forms the operand.  LDS
    // operations complete in order, so the compiler's own lgkmcnt waits for its
    // reads stay correct (only stricter) with these in flight.
    __device__ __forceinline__ void tr_async(const uint16_t* T, int r0, int db, i16x4 (&h)[2]) const {
        const uint32_t a0 = lds_addr(T + r0 * TILE::RS + tr[db][0]);
        const uint32_t a1 = lds_addr(T + r0 * TILE::RS + tr[db][1]);
        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(h[0]) : "v"(a0));
        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(h[1]) : "v"(a1));
    }
};

// Stores a wave's 32 x D output tile held in C registers (lane (n, h): row n,
// columns 32db + 8g + 4h + 0..3 in registers 4g .. 4g+3 of acc[db]), times the
// lane's s and rounded to E, to rows row0 .. row0+31 of the [S][D] matrix g (rows
// at or beyond S are skipped).  The tile goes through the wave's LDS scratch w
// (SCR elements, written and read by this wave only) in passes of up to 32 rows in
// DTile's swizzled layout, so that each global store instruction writes 64
// consecutive 16-byte chunks (whole rows) instead of 16 bytes of each of 32 rows.
// Returns with the wave's LDS reads of w complete.
template <class E, int D, int SCR>
__device__ __forceinline__ void store_tile_rows(uint16_t* w, const f32x16 (&acc)[HeadDim<D>::DB], float s,
                                                uint16_t* __restrict__ g, int row0, int S, int lane) {
    constexpr int CPR = D / 8;
    constexpr int PR = 32 * DTile<32, D, 1>::RS <= SCR ? 32 : 16;  // rows per pass
    using T = DTile<PR, D, 1>;
    static_assert(T::ELEMS <= SCR, "the scratch holds a pass");
    constexpr int CH = PR * CPR;  // 16-byte chunks per pass
    const int n = lane & 31, h = lane >> 5;
    const int rows = max(0, min(S - row0, 32));
#pragma unroll
    for (int p = 0; p < 32 / PR; ++p) {
        if (n >= p * PR && n < (p + 1) * PR) {
#pragma unroll
            for (int db = 0; db < HeadDim<D>::DB; ++db)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (!HeadDim<D>::live(db, q)) continue;
                    u32x2 u;
                    u[0] = E::pack2(acc[db][4 * q + 0] * s, acc[db][4 * q + 1] * s);
                    u[1] = E::pack2(acc[db][4 * q + 2] * s, acc[db][4 * q + 3] * s);
                    *reinterpret_cast<u32x2*>(w + T::at(n - p * PR, db * 32 + 8 * q + 4 * h)) = u;
                }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        uint16_t* gr = g + (size_t)(row0 + p * PR) * D;
#pragma unroll
        for (int i = 0; i < (CH + 63) / 64; ++i) {
            const int e = i * 64 + lane, row = e / CPR, c = e % CPR;
            if ((CH % 64 == 0 || e < CH) && p * PR + row < rows)
                *reinterpret_cast<u32x4*>(gr + (size_t)e * 8) = lds16(w + T::at(row, 8 * c));
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the scratch may be written again
    }
}

// The same for fp32 outputs (g is an [S][D] fp32 matrix): each lane's four values of a
// group are one 16-byte chunk of its row, laid out as a row of 2D 16-bit elements.
template <int D, int SCR>
__device__ __forceinline__ void store_tile_rows_f32(uint16_t* w, const f32x16 (&acc)[HeadDim<D>::DB], float s,
                                                    float* __restrict__ g, int row0, int S, int lane) {
    constexpr int CPR = D / 4;
    constexpr int PR = 32 * DTile<32, 2 * D, 1>::RS <= SCR ? 32 : 16;  // rows per pass
    using T = DTile<PR, 2 * D, 1>;
    static_assert(T::ELEMS <= SCR, "the scratch holds a pass");
    constexpr int CH = PR * CPR;
    const int n = lane & 31, h = lane >> 5;
    const int rows = max(0, min(S - row0, 32));
#pragma unroll
    for (int p = 0; p < 32 / PR; ++p) {
        if (n >= p * PR && n < (p + 1) * PR) {
#pragma unroll
            for (int db = 0; db < HeadDim<D>::DB; ++db)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (!HeadDim<D>::live(db, q)) continue;
                    f32x4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = acc[db][4 * q + i] * s;
                    *reinterpret_cast<f32x4*>(w + T::at(n - p * PR, 2 * (db * 32 + 8 * q + 4 * h))) = v;
                }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        float* gr = g + (size_t)(row0 + p * PR) * D;
#pragma unroll
        for (int i = 0; i < (CH + 63) / 64; ++i) {
            const int e = i * 64 + lane, row = e / CPR, c = e % CPR;
            if ((CH % 64 == 0 || e < CH) && p * PR + row < rows)
                *reinterpret_cast<u32x4*>(gr + (size_t)e * 4) = lds16(w + T::at(row, 8 * c));
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the scratch may be written again
    }
}

}  // namespace attn
