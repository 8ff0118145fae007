// fp32 inputs: forward, dK/dV and dQ on the vector ALUs, fp32 throughout.
//
// Same method as the bf16 MFMA path (Forge RESEARCH.md §6: online softmax with a
// saved LSE; atomic-free backward recomputing P from the LSE; delta from the
// preprocess), laid out for exact fp32 products instead of matrix cores: G lanes
// share one row (a query, or a key for the dK/dV pass), each lane holding E = D/G
// consecutive columns (G = 2 at D = 64, else 4, for grids that fill the device;
// 8 for smaller ones, see kNarrowG), and dot products are finished with DPP adds
// inside the G-lane group (lane_group_sum).  The streamed rows are staged in LDS,
// where all groups read the same row (a broadcast).  This path serves fp32 callers
// and small problems; the bf16 kernels carry the throughput.
#include "attn_launch.h"
#include "attn_device.h"

namespace attn {

constexpr int kF32Tile = 32;  // streamed rows per LDS tile

// Row split: G lanes per row, E columns per lane, R rows per 256-thread block.
template <int D, int G_>
struct F32Split {
    static constexpr int G = G_;
    static constexpr int E = D / G;
    static constexpr int R = 256 / G;
    static_assert(D % G == 0 && E % 4 == 0, "head dimension");
};
// The wide split (fewest lane exchanges and repeated exps per score) serves grids
// whose row blocks cover the device at least twice; smaller grids take eight lanes
// per row (four at D = 80): a quarter of the rows per block, so four times the
// blocks, and a quarter of each lane's chain of dependent FMAs per score.
template <int D>
constexpr int kWideG = D <= 64 ? 2 : 4;
template <int D>
constexpr int kNarrowG = D == 80 ? 4 : 8;


// One tile of kF32Tile rows of D floats (rows row0 .. row0 + kF32Tile - 1, zero at
// and beyond S), held in registers between its loads and its store to LDS, so that
// the next tile's loads are in flight during the current tile's arithmetic.
template <int D>
struct F32Rows {
    static constexpr int CH = kF32Tile * D / 4;  // 16-byte chunks
    static constexpr int PT = (CH + 255) / 256;  // per thread
    f32x4 r[PT];
    __device__ __forceinline__ void load(const float* __restrict__ src, int row0, int S, int tid) {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int c = tid + i * 256;
            const int row = c / (D / 4), col = (c % (D / 4)) * 4;
            r[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if ((CH % 256 == 0 || c < CH) && row0 + row < S)
                r[i] = *reinterpret_cast<const f32x4*>(src + (size_t)(row0 + row) * D + col);
        }
    }
    __device__ __forceinline__ void store(float* dst, int tid) const {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int c = tid + i * 256;
            if (CH % 256 == 0 || c < CH) *reinterpret_cast<f32x4*>(dst + c * 4) = r[i];
        }
    }
};

template <int D, int GS>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, float* __restrict__ O,
                                                      float* __restrict__ LSE, int S, int nblk, int BH, int H, int GQ,
                                                      float c,
                                                      int causal) {
    constexpr int G = F32Split<D, GS>::G, R = F32Split<D, GS>::R, E = F32Split<D, GS>::E;
    __shared__ __attribute__((aligned(16))) float Ks[kF32Tile * D];
    __shared__ __attribute__((aligned(16))) float Vs[kF32Tile * D];
    const WorkItem wi = heavy_first(blockIdx.x, BH);
    const int head = wi.head;
    const int blk = nblk - 1 - wi.rank;
    const int q0 = blk * R;
    const size_t base = (size_t)head * S * D;
    const size_t kvbase = (size_t)kv_head_of(head, H, GQ) * S * D;
    const int tid = threadIdx.x;
    const int part = tid % G;
    const int q = q0 + tid / G;

    float qv[E], ov[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        qv[e] = q < S ? Q[base + (size_t)q * D + part * E + e] : 0.f;
        ov[e] = 0.f;
    }
    float m = -FLT_MAX, l = 0.f;
    const int kend = causal ? min(S, q0 + R) : S;
    F32Rows<D> kt, vt;
    kt.load(K + kvbase, 0, S, tid);
    vt.load(V + kvbase, 0, S, tid);
    for (int k0 = 0; k0 < kend; k0 += kF32Tile) {
        __syncthreads();  // the previous tile is no longer read
        kt.store(Ks, tid);
        vt.store(Vs, tid);
        __syncthreads();
        if (k0 + kF32Tile < kend) {
            kt.load(K + kvbase, k0 + kF32Tile, S, tid);
            vt.load(V + kvbase, k0 + kF32Tile, S, tid);
        }
        float sv[kF32Tile];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < kF32Tile; ++j) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) d = fmaf(qv[e], Ks[j * D + part * E + e], d);
            d = lane_group_sum<G>(d);
            const int key = k0 + j;
            const bool vis = key < S && (!causal || key <= q);
            sv[j] = vis ? d : -INFINITY;
            mx = fmaxf(mx, sv[j]);
        }
        // m is kept in raw score units and the exponent is (s - m) * c, so the
        // row maximum gets exactly exp2(0) = 1
        const float mn = fmaxf(m, mx);
        const float f = exp2f((m - mn) * c);
        m = mn;
        l *= f;
#pragma unroll
        for (int e = 0; e < E; ++e) ov[e] *= f;
#pragma unroll
        for (int j = 0; j < kF32Tile; ++j) {
            const float p = exp2f((sv[j] - m) * c);
            l += p;
#pragma unroll
            for (int e = 0; e < E; ++e) ov[e] = fmaf(p, Vs[j * D + part * E + e], ov[e]);
        }
    }
    if (q < S) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) O[base + (size_t)q * D + part * E + e] = ov[e] * inv;
        if (part == 0) LSE[(size_t)head * S + q] = l > 0.f ? (m * c + log2f(l)) * kLn2 : -INFINITY;
    }
}

// LDS of one dQ block (K and V tiles) or one dK/dV block (Q and dO tiles, then the
// rows' -LSE*log2(e) and delta), in floats.
template <int D>
constexpr int kF32Smem = 2 * kF32Tile * D + 2 * kF32Tile;

// dQ of query block `bid` (heaviest first over the BH heads).  DELTA_FROM_O:
// delta = rowsum(dO o O) is formed here from the O rows and written to DeltaOut;
// otherwise it is read from Delta.
template <int D, int GS, bool DELTA_FROM_O>
__device__ __forceinline__ void dq_f32_block(float* smem, int bid, const float* __restrict__ Q,
                                             const float* __restrict__ K, const float* __restrict__ V,
                                             const float* __restrict__ O, const float* __restrict__ dO,
                                             const float* __restrict__ LSE, const float* __restrict__ Delta,
                                             float* __restrict__ DeltaOut, float* __restrict__ dQ, int S, int nblk,
                                             int BH, int H, int GQ, float c, float scale, int causal) {
    constexpr int G = F32Split<D, GS>::G, R = F32Split<D, GS>::R, E = F32Split<D, GS>::E;
    float* Ks = smem;
    float* Vs = smem + kF32Tile * D;
    const WorkItem wi = heavy_first(bid, BH);
    const int head = wi.head;
    const int blk = nblk - 1 - wi.rank;
    const int q0 = blk * R;
    const size_t base = (size_t)head * S * D;
    const size_t kvbase = (size_t)kv_head_of(head, H, GQ) * S * D;
    const int tid = threadIdx.x;
    const int part = tid % G;
    const int q = q0 + tid / G;

    float qv[E], dov[E], acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const size_t off = base + (size_t)q * D + part * E + e;
        qv[e] = q < S ? Q[off] : 0.f;
        dov[e] = q < S ? dO[off] : 0.f;
        acc[e] = 0.f;
    }
    const float l2 = q < S ? LSE[(size_t)head * S + q] * kLog2e : INFINITY;
    float dl;
    if constexpr (DELTA_FROM_O) {
        float dsum = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e)
            dsum = fmaf(dov[e], q < S ? O[base + (size_t)q * D + part * E + e] : 0.f, dsum);
        dl = lane_group_sum<G>(dsum);
        if (part == 0 && q < S) DeltaOut[(size_t)head * S + q] = dl;
    } else {
        dl = q < S ? Delta[(size_t)head * S + q] : 0.f;
    }
    const int kend = causal ? min(S, q0 + R) : S;
    F32Rows<D> kt, vt;
    kt.load(K + kvbase, 0, S, tid);
    vt.load(V + kvbase, 0, S, tid);
    for (int k0 = 0; k0 < kend; k0 += kF32Tile) {
        __syncthreads();  // the previous tile is no longer read
        kt.store(Ks, tid);
        vt.store(Vs, tid);
        __syncthreads();
        if (k0 + kF32Tile < kend) {
            kt.load(K + kvbase, k0 + kF32Tile, S, tid);
            vt.load(V + kvbase, k0 + kF32Tile, S, tid);
        }
#pragma unroll 4
        for (int j = 0; j < kF32Tile; ++j) {
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                s = fmaf(qv[e], Ks[j * D + part * E + e], s);
                dp = fmaf(dov[e], Vs[j * D + part * E + e], dp);
            }
            s = lane_group_sum<G>(s);
            dp = lane_group_sum<G>(dp);
            const int key = k0 + j;
            const bool vis = key < S && (!causal || key <= q);
            const float p = vis ? exp2f(fmaf(s, c, -l2)) : 0.f;
            const float ds = p * (dp - dl);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = fmaf(ds, Ks[j * D + part * E + e], acc[e]);
        }
    }
    if (q < S) {
#pragma unroll
        for (int e = 0; e < E; ++e) dQ[base + (size_t)q * D + part * E + e] = acc[e] * scale;
    }
}

template <int D, int GS, bool DELTA_FROM_O>
__global__ __launch_bounds__(256) void dq_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                     const float* __restrict__ V, const float* __restrict__ O,
                                                     const float* __restrict__ dO, const float* __restrict__ LSE,
                                                     const float* __restrict__ Delta, float* __restrict__ DeltaOut,
                                                     float* __restrict__ dQ, int S, int nblk, int BH, int H, int GQ,
                                                     float c, float scale, int causal) {
    __shared__ __attribute__((aligned(16))) float smem[kF32Smem<D>];
    dq_f32_block<D, GS, DELTA_FROM_O>(smem, blockIdx.x, Q, K, V, O, dO, LSE, Delta, DeltaOut, dQ, S, nblk, BH, H,
                                      GQ, c, scale, causal);
}

// dK and dV of key block `bid` (heaviest first over the BH key/value heads).
// DELTA_FROM_O: each query tile's delta = rowsum(dO o O) is formed here from the
// dO and O rows, in the order of dq_f32_block with the same split (G lanes of an
// eight-lane group per row, E columns each, then the G-lane sum), so the same bits
// as the dQ pass; otherwise it is read from Delta.
template <int D, int GS, bool DELTA_FROM_O>
__device__ __forceinline__ void dkdv_f32_block(float* smem, int bid, const float* __restrict__ Q,
                                               const float* __restrict__ K, const float* __restrict__ V,
                                               const float* __restrict__ O, const float* __restrict__ dO,
                                               const float* __restrict__ LSE, const float* __restrict__ Delta,
                                               float* __restrict__ dK, float* __restrict__ dV, int S, int nblk, int BH,
                                               int H, int GQ, float c, float scale, int causal) {
    constexpr int G = F32Split<D, GS>::G, R = F32Split<D, GS>::R, E = F32Split<D, GS>::E;
    float* Qs = smem;
    float* Os = smem + kF32Tile * D;
    float* L2s = smem + 2 * kF32Tile * D;
    float* DLs = L2s + kF32Tile;
    const WorkItem wi = heavy_first(bid, BH);
    const int head = wi.head;
    const int blk = wi.rank;
    const int n0 = blk * R;
    const size_t base = (size_t)head * S * D;
    const int tid = threadIdx.x;
    const int part = tid % G;
    const int key = n0 + tid / G;

    float kv[E], vv[E], dk[E], dv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const size_t off = base + (size_t)key * D + part * E + e;
        kv[e] = key < S ? K[off] : 0.f;
        vv[e] = key < S ? V[off] : 0.f;
        dk[e] = 0.f;
        dv[e] = 0.f;
    }
    const int qstart = causal ? n0 : 0;
    // BH counts key/value heads here; the GQ query heads that read this one
    // all add into dk and dv
    const int Hkv = H / GQ;
    const int qh0 = (head / Hkv) * H + (head % Hkv) * GQ;
    // query tiles of the GQ query heads in turn; with the narrow split (E <= 16)
    // the next one is fetched into registers during the current one's arithmetic
    // (the wide split's four E-long row arrays leave no registers for it)
    constexpr bool PF = E <= 16;
    const int nq = (S - qstart + kF32Tile - 1) / kF32Tile;
    const int ntot = GQ * nq;
    F32Rows<D> qtl, otl;
    float l2n = INFINITY, dln = 0.f;
    // DELTA_FROM_O: lanes 0 .. G-1 of group tid / 8 hold E columns of dO and O of
    // row tid / 8 (the dQ split's partition)
    static_assert(kF32Tile * 8 == 256 && G <= 8, "eight lanes per query row of a tile");
    float dd[DELTA_FROM_O ? E : 1], oo[DELTA_FROM_O ? E : 1];
    auto fetch = [&](int i) {
        const int qh = qh0 + i / nq, qt = qstart + (i % nq) * kF32Tile;
        const size_t qbase = (size_t)qh * S * D;
        qtl.load(Q + qbase, qt, S, tid);
        otl.load(dO + qbase, qt, S, tid);
        if (tid < kF32Tile) {
            const int qq = qt + tid;
            l2n = qq < S ? LSE[(size_t)qh * S + qq] * kLog2e : INFINITY;
            if constexpr (!DELTA_FROM_O) dln = qq < S ? Delta[(size_t)qh * S + qq] : 0.f;
        }
        if constexpr (DELTA_FROM_O) {
            const int qq = qt + (tid >> 3), p8 = tid & 7;
            const bool on = qq < S && p8 < G;
            const size_t off = qbase + (size_t)qq * D + (on ? p8 : 0) * E;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                dd[e] = on ? dO[off + e] : 0.f;
                oo[e] = on ? O[off + e] : 0.f;
            }
        }
    };
    if (PF && ntot > 0) fetch(0);
    for (int i = 0; i < ntot; ++i) {
        const int qt0 = qstart + (i % nq) * kF32Tile;
        if (!PF) fetch(i);
        __syncthreads();  // the previous tile is no longer read
        qtl.store(Qs, tid);
        otl.store(Os, tid);
        if (tid < kF32Tile) {
            L2s[tid] = l2n;
            if constexpr (!DELTA_FROM_O) DLs[tid] = dln;
        }
        if constexpr (DELTA_FROM_O) {
            float dsum = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) dsum = fmaf(dd[e], oo[e], dsum);
            dsum = lane_group_sum<G>(dsum);
            if ((tid & 7) == 0) DLs[tid >> 3] = dsum;
        }
        __syncthreads();
        if (PF && i + 1 < ntot) fetch(i + 1);
#pragma unroll(E > 8 ? 1 : 4)  // wider rows keep 2 * E LDS values live per unrolled query
        for (int j = 0; j < kF32Tile; ++j) {
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                s = fmaf(kv[e], Qs[j * D + part * E + e], s);
                dp = fmaf(vv[e], Os[j * D + part * E + e], dp);
            }
            s = lane_group_sum<G>(s);
            dp = lane_group_sum<G>(dp);
            const int qq = qt0 + j;
            const bool vis = qq < S && (!causal || key <= qq);
            const float p = vis ? exp2f(fmaf(s, c, -L2s[j])) : 0.f;
            const float ds = p * (dp - DLs[j]);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                dv[e] = fmaf(p, Os[j * D + part * E + e], dv[e]);
                dk[e] = fmaf(ds, Qs[j * D + part * E + e], dk[e]);
            }
        }
    }
    if (key < S) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const size_t off = base + (size_t)key * D + part * E + e;
            dK[off] = dk[e] * scale;
            dV[off] = dv[e];
        }
    }
}

template <int D, int GS>
__global__ __launch_bounds__(256) void dkdv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                       const float* __restrict__ V, const float* __restrict__ dO,
                                                       const float* __restrict__ LSE,
                                                       const float* __restrict__ Delta, float* __restrict__ dK,
                                                       float* __restrict__ dV, int S, int nblk, int BH, int H, int GQ,
                                                       float c, float scale, int causal) {
    __shared__ __attribute__((aligned(16))) float smem[kF32Smem<D>];
    dkdv_f32_block<D, GS, false>(smem, blockIdx.x, Q, K, V, nullptr, dO, LSE, Delta, dK, dV, S, nblk, BH, H, GQ, c,
                                 scale, causal);
}

// The whole backward of a grid too small to fill the device, in one launch: blocks
// below ndq are dQ blocks (which also store delta), the rest dK/dV blocks, which form
// delta themselves, so the two kinds run side by side instead of one pass after the
// other.
template <int D, int GS>
__global__ __launch_bounds__(256) void bwd_f32_fused_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ O, const float* __restrict__ dO, const float* __restrict__ LSE,
    float* __restrict__ DeltaOut, float* __restrict__ dQ, float* __restrict__ dK, float* __restrict__ dV, int S,
    int nblk, int ndq, int BH, int BHkv, int H, int GQ, float c, float scale, int causal) {
    __shared__ __attribute__((aligned(16))) float smem[kF32Smem<D>];
    if ((int)blockIdx.x < ndq)
        dq_f32_block<D, GS, true>(smem, blockIdx.x, Q, K, V, O, dO, LSE, nullptr, DeltaOut, dQ, S, nblk, BH, H, GQ,
                                  c, scale, causal);
    else
        dkdv_f32_block<D, GS, true>(smem, (int)blockIdx.x - ndq, Q, K, V, O, dO, LSE, nullptr, dK, dV, S, nblk,
                                    BHkv, H, GQ, c, scale, causal);
}

template <int D, int GS>
static int f32_blocks(const LaunchArgs& a, int64_t units, int* nblk) {
    constexpr int R = F32Split<D, GS>::R;
    *nblk = (int)((a.S + R - 1) / R);
    const int64_t total = (int64_t)(*nblk) * units;
    return total > INT32_MAX ? -1 : (int)total;
}

// True where the wide split's grid over `units` heads would cover the device fewer
// than two times.
template <int D>
static bool f32_narrow(const LaunchArgs& a, int64_t units) {
    constexpr int R = F32Split<D, kWideG<D>>::R;
    return units * ((a.S + R - 1) / R) < 2 * (int64_t)cu_count();
}

template <int D, int GS>
static hipError_t fwd_f32_g(const LaunchArgs& a) {
    int nblk;
    const int total = f32_blocks<D, GS>(a, a.BH, &nblk);
    if (total < 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fwd_f32_kernel<D, GS>), dim3(total), dim3(256), 0, a.stream, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, (int)a.S, nblk, (int)a.BH, (int)a.H,
                       (int)(a.H / a.Hkv),
                       a.scale * kLog2e, a.causal);
    return hipGetLastError();
}

template <int D>
static hipError_t fwd_f32(const LaunchArgs& a) {
    return f32_narrow<D>(a, a.BH) ? fwd_f32_g<D, kNarrowG<D>>(a) : fwd_f32_g<D, kWideG<D>>(a);
}

template <int D, int GS, bool DELTA_FROM_O>
static hipError_t dq_f32_g(const LaunchArgs& a) {
    int nblk;
    const int total = f32_blocks<D, GS>(a, a.BH, &nblk);
    if (total < 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((dq_f32_kernel<D, GS, DELTA_FROM_O>), dim3(total), dim3(256), 0, a.stream, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (const float*)a.o_in, (const float*)a.dout, a.lse_in,
                       a.delta_in, a.delta, (float*)a.dq, (int)a.S, nblk, (int)a.BH, (int)a.H, (int)(a.H / a.Hkv),
                       a.scale * kLog2e, a.scale,
                       a.causal);
    return hipGetLastError();
}

template <int D, bool DELTA_FROM_O>
static hipError_t dq_f32(const LaunchArgs& a) {
    return f32_narrow<D>(a, a.BH) ? dq_f32_g<D, kNarrowG<D>, DELTA_FROM_O>(a)
                                  : dq_f32_g<D, kWideG<D>, DELTA_FROM_O>(a);
}

template <int D, int GS>
static hipError_t dkdv_f32_g(const LaunchArgs& a, int64_t bhkv) {
    int nblk;
    // one block per key block of each key/value head
    const int total = f32_blocks<D, GS>(a, bhkv, &nblk);
    if (total < 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((dkdv_f32_kernel<D, GS>), dim3(total), dim3(256), 0, a.stream, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (const float*)a.dout, a.lse_in, a.delta_in,
                       (float*)a.dk, (float*)a.dv, (int)a.S, nblk, (int)bhkv, (int)a.H, (int)(a.H / a.Hkv),
                       a.scale * kLog2e, a.scale, a.causal);
    return hipGetLastError();
}

template <int D>
static hipError_t dkdv_f32(const LaunchArgs& a) {
    const int64_t bhkv = a.BH / a.H * a.Hkv;
    return f32_narrow<D>(a, bhkv) ? dkdv_f32_g<D, kNarrowG<D>>(a, bhkv) : dkdv_f32_g<D, kWideG<D>>(a, bhkv);
}

// attn_bwd's passes: one fused launch when both take the narrow split, else the dQ
// pass (forming delta) and then the dK/dV pass.
template <int D>
static hipError_t bwd_f32(const LaunchArgs& a) {
    const int64_t bhkv = a.BH / a.H * a.Hkv;
    if (!f32_narrow<D>(a, a.BH) || !f32_narrow<D>(a, bhkv)) {
        const hipError_t e = dq_f32<D, true>(a);
        return e != hipSuccess ? e : dkdv_f32<D>(a);
    }
    constexpr int GS = kNarrowG<D>;
    int nblk;
    const int ndq = f32_blocks<D, GS>(a, a.BH, &nblk);
    const int nkv = f32_blocks<D, GS>(a, bhkv, &nblk);
    if (ndq < 0 || nkv < 0 || (int64_t)ndq + nkv > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_f32_fused_kernel<D, GS>), dim3(ndq + nkv), dim3(256), 0, a.stream, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (const float*)a.o_in, (const float*)a.dout, a.lse_in,
                       a.delta, (float*)a.dq, (float*)a.dk, (float*)a.dv, (int)a.S, nblk, ndq, (int)a.BH, (int)bhkv,
                       (int)a.H, (int)(a.H / a.Hkv), a.scale * kLog2e, a.scale, a.causal);
    return hipGetLastError();
}

hipError_t launch_fwd_f32(const LaunchArgs& a) {
    if (a.D == 64) return fwd_f32<64>(a);
    if (a.D == 80) return fwd_f32<80>(a);
    if (a.D == 96) return fwd_f32<96>(a);
    if (a.D == 128) return fwd_f32<128>(a);
    return hipErrorInvalidValue;
}
hipError_t launch_bwd_dq_f32(const LaunchArgs& a) {
    if (a.D == 64) return dq_f32<64, false>(a);
    if (a.D == 80) return dq_f32<80, false>(a);
    if (a.D == 96) return dq_f32<96, false>(a);
    if (a.D == 128) return dq_f32<128, false>(a);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_delta_f32(const LaunchArgs& a) {
    if (a.D == 64) return dq_f32<64, true>(a);
    if (a.D == 80) return dq_f32<80, true>(a);
    if (a.D == 96) return dq_f32<96, true>(a);
    if (a.D == 128) return dq_f32<128, true>(a);
    return hipErrorInvalidValue;
}
hipError_t launch_bwd_f32(const LaunchArgs& a) {
    if (a.D == 64) return bwd_f32<64>(a);
    if (a.D == 80) return bwd_f32<80>(a);
    if (a.D == 96) return bwd_f32<96>(a);
    if (a.D == 128) return bwd_f32<128>(a);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_dkdv_f32(const LaunchArgs& a) {
    if (a.D == 64) return dkdv_f32<64>(a);
    if (a.D == 80) return dkdv_f32<80>(a);
    if (a.D == 96) return dkdv_f32<96>(a);
    if (a.D == 128) return dkdv_f32<128>(a);
    return hipErrorInvalidValue;
}

}  // namespace attn
