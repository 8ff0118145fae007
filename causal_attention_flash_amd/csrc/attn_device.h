// Device-side building blocks shared by the gfx950 attention kernels.
//
// MFMA used: v_mfma_f32_32x32x16_bf16 (one wave computes a 32x32 fp32 tile from
// a 32x16 and a 16x32 bf16 operand).  Register layouts, per lane l of the 64-lane
// wave, with h = l / 32 (the lane half) and n = l % 32:
//
//   A operand (32 x 16, row i, contraction index k): lane l holds row i = n and
//     eight consecutive k slots 8h .. 8h+7 (one bf16x8 register quad).
//   B operand (16 x 32, contraction index k, column j): lane l holds column j = n
//     and the same eight k slots 8h .. 8h+7.
//   C/D (32 x 32 fp32): lane l holds column j = n; register r in [0, 16) holds
//     row 8*(r/4) + 4*h + (r%4).
//
// Only the pairing of A's and B's k slots matters to a contraction, so any
// consistent relabelling of the contraction index is free.  The kernels use that
// to feed a C tile straight back as an operand: C registers 8c .. 8c+7 of a lane
// hold rows 16c + 8*(v/4) + 4h + (v%4), v = 0..7, so they form the k slots of
// one 16-deep contraction step whose k order is "rows 16c + {0..3, 8..11}" for
// h = 0 and "rows 16c + {4..7, 12..15}" for h = 1.  The operand on the other
// side is read from a row-major LDS tile in exactly that order by the gfx950
// transposing LDS read (lds_tr_operand below).
//
// This is the AMD counterpart of the problem the pages spend a section on
// (pairing softmax row statistics with accumulator lanes when the lane map is
// hidden; "Cooperative tensors ..." §8.5 and Forge "Attention kernel design").
// Here the lane map is fixed by the instruction, so the row statistics live in
// the lane that owns the row and the rescale is a per-lane multiply.
#pragma once

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 C tile held by register r of a lane in half h.
__device__ __forceinline__ int crow(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Head dimensions.  Contractions over d run in 16-deep MFMA steps (D / 16 of
// them, D a multiple of 16); outputs over d are built in 32-wide C tiles, so D =
// 80 uses three tiles of which the last has 16 live columns.  The dead columns
// are computed from whatever the operand reads return and never stored: in an
// MFMA, output row i depends on row i of A alone.
template <int D>
struct HeadDim {
    static_assert(D % 16 == 0 && D >= 32, "head dimension");
    static constexpr int KSTEPS = D / 16;        // 16-deep contraction steps over d
    static constexpr int DB = (D + 31) / 32;     // 32-wide output tiles over d
    // C registers 4g .. 4g+3 of output tile db hold d = 32 db + 8 g + 4 h + 0..3;
    // the whole group of 8 (both halves) is live or dead together.
    static constexpr bool live(int db, int g) { return db * 32 + 8 * g < D; }
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Operand for a contraction over the ROWS of a row-major bf16 LDS tile T (row
// stride STR elements): lane (n, h) receives T[r0 + kslot(v)][c0 + n] for
// v = 0..7, with kslot(v) = 8*(v/4) + 4*h + (v%4) -- the row order of C
// registers 8c .. 8c+7, so the result pairs with pack_operand() of a C tile.
//
// Built from two ds_read_b64_tr_b16.  That instruction works on groups of 16
// lanes: lane i of a group receives, as element k, element (i % 4) of the
// 4-element chunk addressed by lane 4k + i/4 of the same group.  Lane j of group
// g therefore addresses row r0 + 4*(g/2) + j/4 (plus 8 for the second read) at
// column c0 + 16*(g%2) + 4*(j%4).  c0 and STR must keep those 8-byte aligned.
template <int STR>
__device__ __forceinline__ bf16x8 lds_tr_operand(const uint16_t* T, int r0, int c0, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int row = r0 + 4 * (g >> 1) + (j >> 2);
    const int col = c0 + 16 * (g & 1) + 4 * (j & 3);
    const uint16_t* p = T + row * STR + col;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8 * STR));
    const i16x8 r = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, r);
}

// Two fp32 -> packed bf16 (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

// Eight consecutive C registers (8c .. 8c+7) -> one bf16x8 operand quad.
__device__ __forceinline__ bf16x8 pack_operand(const f32x16& acc, int c) {
    u32x4 u;
    u[0] = pack_bf16x2(acc[8 * c + 0], acc[8 * c + 1]);
    u[1] = pack_bf16x2(acc[8 * c + 2], acc[8 * c + 3]);
    u[2] = pack_bf16x2(acc[8 * c + 4], acc[8 * c + 5]);
    u[3] = pack_bf16x2(acc[8 * c + 6], acc[8 * c + 7]);
    return __builtin_bit_cast(bf16x8, u);
}

// acc + the sum of eight bf16 values, two per v_dot2_f32_bf16 (fp32 accumulate).
// The pairs are built element by element: a __builtin_bit_cast applied to one
// element of a vector register was seen to read element 0 for every index.
__device__ __forceinline__ float sum_bf16x8(const bf16x8& x, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{x[0], x[1]}, one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{x[2], x[3]}, one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{x[4], x[5]}, one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{x[6], x[7]}, one, acc, false);
    return acc;
}

// acc + the dot product of two bf16x8 vectors (fp32 accumulation, pairs built
// element by element as in sum_bf16x8).
__device__ __forceinline__ float dot_bf16x8(const bf16x8& x, const bf16x8& y, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{x[0], x[1]}, bf16x2{y[0], y[1]}, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{x[2], x[3]}, bf16x2{y[2], y[3]}, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{x[4], x[5]}, bf16x2{y[4], y[5]}, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{x[6], x[7]}, bf16x2{y[6], y[7]}, acc, false);
    return acc;
}

// 16-bit element types of the MFMA kernels.  A kernel templated on E uses
// E::V8 for its operand quads and E's MFMA, pack, dot and transposing-read
// helpers; everything else (fp32 accumulation, fp32 softmax statistics, the
// lane layouts above) is the same for both types.  Conversions from fp32 round
// to nearest even.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct Bf16 {
    using V8 = bf16x8;
    using V2 = bf16x2;
    static __device__ __forceinline__ f32x16 mma(const V8& a, const V8& b, const f32x16& c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma16(const V8& a, const V8& b, const f32x4& c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }
    // acc + a.lo*b.lo + a.hi*b.hi in fp32, on packed pairs
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(V2, a), __builtin_bit_cast(V2, b), acc, false);
    }
    static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
    static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
};

struct F16 {
    using V8 = f16x8;
    using V2 = f16x2;
    static __device__ __forceinline__ f32x16 mma(const V8& a, const V8& b, const f32x16& c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma16(const V8& a, const V8& b, const f32x4& c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float a, float b) {
        const f16x2 r = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, r);
    }
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(V2, a), __builtin_bit_cast(V2, b), acc, false);
    }
    static __device__ __forceinline__ float lo(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    }
    static __device__ __forceinline__ float hi(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
};

// fp8 (OCP E4M3) operands of v_mfma_f32_32x32x64_f8f6f4, for S^T = K Q^T only: a
// lane holds 32 values of its row (row lane % 32), at the contraction indices
// 32h .. 32h+31 of a 64-wide step, h = lane / 32 (the same map for both
// operands, so the instruction pairs equal indices; checked on the device
// against an fp64 dot product).  Format codes 0 select E4M3 for both operands;
// zero scale operands leave the products unscaled.  The instruction sums the
// exact fp8 products in fp32 with a narrower internal alignment than a serial
// fp32 sum (relative differences up to ~6e-5 on random 64-term sums, measured;
// one 448 and 63 terms of 0.0625 sum exactly).
typedef int i32x8 __attribute__((ext_vector_type(8)));
struct Fp8E4M3 {
    using Op = i32x8;
    static __device__ __forceinline__ f32x16 mma(const Op& a, const Op& b, const f32x16& c) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
    static __device__ __forceinline__ Op join(const u32x4& lo, const u32x4& hi) {
        const u32x4 v[2] = {lo, hi};
        return __builtin_bit_cast(Op, v);
    }
};

// Generic forms of the helpers above for an element type E.
template <class E>
__device__ __forceinline__ typename E::V8 as_op(const u32x4& u) {
    return __builtin_bit_cast(typename E::V8, u);
}
template <class E>
__device__ __forceinline__ typename E::V8 pack_op(const f32x16& acc, int c) {
    u32x4 u;
    u[0] = E::pack2(acc[8 * c + 0], acc[8 * c + 1]);
    u[1] = E::pack2(acc[8 * c + 2], acc[8 * c + 3]);
    u[2] = E::pack2(acc[8 * c + 4], acc[8 * c + 5]);
    u[3] = E::pack2(acc[8 * c + 6], acc[8 * c + 7]);
    return __builtin_bit_cast(typename E::V8, u);
}
// Per-lane sums of B operands of the 32x32x16 product, taken on the 16x16x32
// product.  As a 16x16x32 B operand, lane l is column l % 16 and contraction group
// g = l / 16 (A and B pair their values group by group, element by element, so how
// the hardware numbers a group's eight contraction indices does not matter here).
// This A operand is 1 in row 4g over group g and 0 elsewhere, so output register 0
// of lane l (row 4g, column l % 16) is the fp32 sum of lane l's own eight values.
template <class E>
__device__ __forceinline__ typename E::V8 lane_sum_selector(int lane) {
    const int i = lane & 15, g = lane >> 4;
    const uint32_t w = i == 4 * g ? E::pack2(1.0f, 1.0f) : 0u;
    return __builtin_bit_cast(typename E::V8, u32x4{w, w, w, w});
}

// acc + the sum of the eight values of x (fp32 accumulation)
template <class E>
__device__ __forceinline__ float sum8(const typename E::V8& x, float acc) {
    const u32x4 u = __builtin_bit_cast(u32x4, x);
    const uint32_t one = E::pack2(1.0f, 1.0f);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = E::dot2(u[i], one, acc);
    return acc;
}
// acc + the dot product of x and y (fp32 accumulation)
template <class E>
__device__ __forceinline__ float dot8(const typename E::V8& x, const typename E::V8& y, float acc) {
    const u32x4 u = __builtin_bit_cast(u32x4, x), w = __builtin_bit_cast(u32x4, y);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = E::dot2(u[i], w[i], acc);
    return acc;
}
template <class E, int STR>
__device__ __forceinline__ typename E::V8 lds_tr_op(const uint16_t* T, int r0, int c0, int lane) {
    return __builtin_bit_cast(typename E::V8, lds_tr_operand<STR>(T, r0, c0, lane));
}

// Reductions over the lane pair (l, l ^ 32).  v_permlane32_swap exchanges the
// upper half of its first register with the lower half of its second; given x in
// both, every lane ends up holding x[l % 32] in one result and x[l % 32 + 32] in
// the other, so a symmetric reduction of the two results is the pair reduction
// whichever result is which.
__device__ __forceinline__ float half_max(float x) {
    const uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over aligned groups of G lanes (G a power of two, at most 32), the result in
// every lane of the group: DPP adds within rows of 16 lanes (pairs, quads, the two
// halves of a row of 8, the two halves of 16), then one cross-row exchange.  Each
// step adds a lane's value and its partner's in either order, so every lane of a
// group ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float plus_dpp(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int G>
__device__ __forceinline__ float lane_group_sum(float x) {
    static_assert(G >= 1 && G <= 32 && (G & (G - 1)) == 0, "group of 1, 2, 4, 8, 16 or 32 lanes");
    if constexpr (G >= 2) x = plus_dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (G >= 4) x = plus_dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (G >= 8) x = plus_dpp<0x141>(x);  // row_half_mirror: the other quad of 8
    if constexpr (G >= 16) x = plus_dpp<0x140>(x); // row_mirror: the other 8 of 16
    if constexpr (G >= 32) x += __shfl_xor(x, 16);
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt vmcnt(0): every vector memory load issued so far has returned.
// Encoding (gfx9): vmcnt in bits 3:0 and 15:14 (0), expcnt in bits 6:4 and
// lgkmcnt in bits 11:8 at their maxima (no wait on those counters).  The
// scheduling barriers keep loads from being moved across the wait.
__device__ __forceinline__ void wait_vmem_all() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x4 lds16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Low halves of two words -> one word (a's low half in the low half).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
// High halves of two words -> one word (a's high half in the low half).
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Block order for a 1-D grid of nblk * BH blocks (BH = batch x heads): block b
// works on head b % BH at position rank = b / BH in its head's order of causal
// work, heaviest first.  Blocks are dispatched in index order as slots free up,
// so every head's heaviest blocks start first and the light ones pack in behind
// them (greedy list scheduling in decreasing order), which keeps the tail of the
// grid short.  The dispatcher assigns block b to XCD b % 8, so whenever BH is a
// multiple of 8 all blocks of one head run on one XCD and share its L2.
struct WorkItem {
    int head, rank;
};
__device__ __forceinline__ WorkItem heavy_first(int bid, int BH) { return {bid % BH, bid / BH}; }

// Issue priority of a causal workgroup by its share of the work: the heaviest
// quarter of the ranks (rank 0 heaviest, of nblk) 3, the next 2, then 1, the
// lightest quarter 0.  The heavy blocks are the grid's critical path; the waves of
// lighter ones sharing their SIMDs take the issue slots they leave.
__device__ __forceinline__ void weight_priority(int rank, int nblk) {
    const int p = 3 - (4 * rank) / nblk;
    if (p >= 3)
        __builtin_amdgcn_s_setprio(3);
    else if (p == 2)
        __builtin_amdgcn_s_setprio(2);
    else if (p == 1)
        __builtin_amdgcn_s_setprio(1);
}

// Grouped key/value heads: with H query heads per batch entry sharing H / GQ
// key/value heads, query head qh (index over batch x H) reads key/value head
// (qh / H) * (H / GQ) + (qh % H) / GQ (index over batch x H / GQ).  GQ = 1 is
// one key/value head per query head.
__device__ __forceinline__ int kv_head_of(int qh, int H, int GQ) { return (qh / H) * (H / GQ) + (qh % H) / GQ; }

}  // namespace attn
