// Decode attention: one new query row per (batch, query head) against a key/value
// cache, the query seeing every cached row of its sequence.  Forge RESEARCH.md §6,
// decode path ("forge generate"): one query row, a strided walk of the cache with a
// scalar online-softmax update, split into chunks over a long cache in a first pass
// and merged in a second.
//
// The step reads each cached key and value once and does a few flops per byte, so
// it is bound by HBM bandwidth; the layout serves that:
// * one workgroup per (sequence, key/value head, group of up to 8 query heads,
//   chunk of the cache), so the G query heads that share a key/value head read
//   its cache once;
// * a key row is read by a group of lanes with 16-byte loads (D*elem/16 of them,
//   rounded up to a power of two), consecutive lane groups on consecutive rows,
//   so a wave's loads cover whole rows and whole cache lines; loads are issued one
//   batch of two rows per lane group ahead of the arithmetic, as nontemporal loads
//   (each cache row is read once per call; measured 4-7% faster than plain loads
//   with batches of four rows, which also cost enough registers to leave part of
//   the grid waiting for a slot);
// * each lane keeps, per query head, the running max m, the running sum l and its
//   slice of the unnormalised output o (fp32, exponent in log2 units with
//   scale*log2(e) folded into q); the lane groups of a workgroup are merged by
//   shuffles within a wave and through LDS across waves;
// * with one chunk per sequence the first pass writes O and LSE directly;
//   otherwise it writes (m, l, o) partials to the workspace and the second pass
//   merges them: M = max m_c, L = sum l_c 2^(m_c - M), O = sum o_c 2^(m_c - M) / L.
//
// A sequence whose cache length is 0 has no visible key: O = 0, LSE = -inf.
#include "attn_launch.h"
#include "attn_device.h"

namespace attn {

namespace {

// 16-byte chunks of an element type, widened to fp32; fp32 -> element type.
template <class T>
struct Chunk;
template <>
struct Chunk<float> {
    static constexpr int E = 4;  // elements per 16 bytes
    static __device__ __forceinline__ void widen(const u32x4& u, float (&x)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(u[i]);
    }
};
template <class E16>
struct Chunk16 {
    static constexpr int E = 8;
    static __device__ __forceinline__ void widen(const u32x4& u, float (&x)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = E16::lo(u[i]);
            x[2 * i + 1] = E16::hi(u[i]);
        }
    }
};
template <>
struct Chunk<Bf16> : Chunk16<Bf16> {};
template <>
struct Chunk<F16> : Chunk16<F16> {};

constexpr int pow2_ceil(int x) { return x <= 1 ? 1 : 2 * pow2_ceil((x + 1) / 2); }

template <class T, int D>
struct DecodeCfg {
    static constexpr int E = Chunk<T>::E;
    static constexpr int CPR = D / E;              // 16-byte chunks per row
    static constexpr int DG = pow2_ceil(CPR);      // lanes per row
    static constexpr int NT = 256;                 // threads per workgroup
    static constexpr int R = NT / DG;              // rows in flight per workgroup
    static_assert(D % E == 0 && DG <= 32, "head dimension");
};

// Online-softmax state of one query head in one lane: running max m (log2
// units), running sum l and the lane's E output values o.
template <int E>
struct Run {
    float m, l, o[E];
};

// Merge (m2, l2, o2) into (m1, l1, o1); an empty state has m = -inf, l = 0, o = 0.
template <int E>
__device__ __forceinline__ void merge(Run<E>& a, float m2, float l2, const float (&o2)[E]) {
    const float M = fmaxf(a.m, m2);
    const float f1 = a.m == -INFINITY ? 0.f : fast_exp2(a.m - M);
    const float f2 = m2 == -INFINITY ? 0.f : fast_exp2(m2 - M);
    a.m = M;
    a.l = a.l * f1 + l2 * f2;
#pragma unroll
    for (int e = 0; e < E; ++e) a.o[e] = a.o[e] * f1 + o2[e] * f2;
}

// q . k over one lane's 16-byte slices (q pre-widened for fp32, packed for 16-bit)
template <class T>
struct SliceDot {
    static __device__ __forceinline__ float dot(const u32x4& q, const u32x4& k) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) s = T::dot2(q[i], k[i], s);
        return s;
    }
};
template <>
struct SliceDot<float> {
    static __device__ __forceinline__ float dot(const u32x4& q, const u32x4& k) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) s = fmaf(__uint_as_float(q[i]), __uint_as_float(k[i]), s);
        return s;
    }
};

}  // namespace

// Grid: B * H_kv * (G / GT) * nsplit workgroups, block index = ((b * H_kv + j) *
// (G / GT) + gt) * nsplit + split.
template <class T, int D, int GT>
__global__ __launch_bounds__(256) void decode_split_kernel(const void* __restrict__ Q, const void* __restrict__ K,
                                                           const void* __restrict__ V,
                                                           const int* __restrict__ kv_lens,
                                                           float* __restrict__ part_o, float* __restrict__ part_ml,
                                                           void* __restrict__ O, float* __restrict__ LSE, int H,
                                                           int Hkv, int L, int nsplit, int chunk, float c) {
    using Cfg = DecodeCfg<T, D>;
    constexpr int E = Cfg::E, CPR = Cfg::CPR, DG = Cfg::DG, R = Cfg::R, NT = Cfg::NT;
    constexpr int EB = 16 / E;  // bytes per element
    constexpr int U = 2;  // rows per lane group per batch of loads
    __shared__ float sm[NT / 64][GT][2];
    __shared__ float so[NT / 64][GT][D];

    const int G = H / Hkv, ngt = G / GT;
    int bid = blockIdx.x;
    const int split = bid % nsplit;
    bid /= nsplit;
    const int gt = bid % ngt;
    bid /= ngt;
    const int j = bid % Hkv, b = bid / Hkv;
    const int len = kv_lens ? min(max(kv_lens[b], 0), L) : L;
    const int k_begin = split * chunk;
    const int k_end = min(k_begin + chunk, len);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row0 = tid / DG, part = tid % DG;
    const bool act = part < CPR;
    const char* Kb = (const char*)K + ((size_t)b * Hkv + j) * (size_t)L * D * EB + (size_t)part * 16;
    const char* Vb = (const char*)V + ((size_t)b * Hkv + j) * (size_t)L * D * EB + (size_t)part * 16;

    // query slices as stored (the dot runs on the stored type with fp32
    // accumulation; scale*log2(e) multiplies the dot)
    u32x4 qs[GT];
    Run<E> run[GT];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
        const int h = j * G + gt * GT + g;
        qs[g] = u32x4{0u, 0u, 0u, 0u};
        if (act) qs[g] = ldg16((const char*)Q + ((size_t)b * H + h) * D * EB + (size_t)part * 16);
#pragma unroll
        for (int e = 0; e < E; ++e) run[g].o[e] = 0.f;
        run[g].m = -INFINITY;
        run[g].l = 0.f;
    }

    // Rows row0 + R*i of [k_begin, k_end), U per batch, loads one batch ahead.
    auto fetch = [&](u32x4 (&kk)[U], u32x4 (&vv)[U], int r) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int key = r + u * R;
            kk[u] = vv[u] = u32x4{0u, 0u, 0u, 0u};
            if (act && key < k_end) {
                kk[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kb + (size_t)key * D * EB));
                vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vb + (size_t)key * D * EB));
            }
        }
    };
    u32x4 kc[U], vc[U], kn[U], vn[U];
    int r = k_begin + row0;
    fetch(kc, vc, r);
    while (r < k_end) {  // uniform within a lane group
        fetch(kn, vn, r + U * R);
        // scores of the batch (rows past the chunk end: -inf, weight 0)
        float sc[U][GT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool valid = r + u * R < k_end;
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                const float s = lane_group_sum<DG>(SliceDot<T>::dot(qs[g], kc[u])) * c;
                sc[u][g] = valid ? s : -INFINITY;
            }
        }
        float vf[U][E];
#pragma unroll
        for (int u = 0; u < U; ++u) Chunk<T>::widen(vc[u], vf[u]);
        // one rescale per batch: the new reference is the max over the batch and
        // the running max (finite: the batch's first row is always in range)
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            Run<E>& st = run[g];
            float mn = st.m;
#pragma unroll
            for (int u = 0; u < U; ++u) mn = fmaxf(mn, sc[u][g]);
            const float f = fast_exp2(st.m - mn);  // 0 while the state is empty
            st.l *= f;
#pragma unroll
            for (int e = 0; e < E; ++e) st.o[e] *= f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float p = fast_exp2(sc[u][g] - mn);
                st.l += p;
#pragma unroll
                for (int e = 0; e < E; ++e) st.o[e] = fmaf(p, vf[u][e], st.o[e]);
            }
            st.m = mn;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            kc[u] = kn[u];
            vc[u] = vn[u];
        }
        r += U * R;
    }

    // merge the lane groups of each wave (xor over the row bits of the lane)
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
        for (int x = DG; x < 64; x <<= 1) {
            const float m2 = __shfl_xor(run[g].m, x), l2 = __shfl_xor(run[g].l, x);
            float o2[E];
#pragma unroll
            for (int e = 0; e < E; ++e) o2[e] = __shfl_xor(run[g].o[e], x);
            merge(run[g], m2, l2, o2);
        }
    }
    // then the waves, through LDS
    if (lane < DG && act) {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            if (part == 0) {
                sm[wave][g][0] = run[g].m;
                sm[wave][g][1] = run[g].l;
            }
#pragma unroll
            for (int e = 0; e < E; ++e) so[wave][g][part * E + e] = run[g].o[e];
        }
    }
    __syncthreads();
    if (wave != 0) return;
    // wave 0: lane d' handles output elements d' and d' + 64
#pragma unroll
    for (int g = 0; g < GT; ++g) {
        const int h = j * G + gt * GT + g;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) M = fmaxf(M, sm[w][g][0]);
        float f[NT / 64], Ls = 0.f;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) {
            f[w] = sm[w][g][0] == -INFINITY ? 0.f : fast_exp2(sm[w][g][0] - M);
            Ls += sm[w][g][1] * f[w];
        }
        const size_t bh = (size_t)b * H + h;
        for (int d = lane; d < D; d += 64) {
            float od = 0.f;
#pragma unroll
            for (int w = 0; w < NT / 64; ++w) od += so[w][g][d] * f[w];
            if (part_o) {
                part_o[(bh * nsplit + split) * D + d] = od;
            } else {
                const float x = Ls > 0.f ? od / Ls : 0.f;
                if constexpr (EB == 4)
                    reinterpret_cast<float*>(O)[bh * D + d] = x;
                else
                    reinterpret_cast<uint16_t*>(O)[bh * D + d] = (uint16_t)(T::pack2(x, 0.f) & 0xffffu);
            }
        }
        if (lane == 0) {
            if (part_ml) {
                part_ml[(bh * nsplit + split) * 2 + 0] = M;
                part_ml[(bh * nsplit + split) * 2 + 1] = Ls;
            } else {
                LSE[bh] = Ls > 0.f ? (M + __log2f(Ls)) * kLn2 : -INFINITY;
            }
        }
    }
}

// Second pass: one wave per (b, h) merges its nsplit <= 64 partials.  Lane s
// reads partial s's (m, l); the reference M and the total L are wave reductions;
// the weights 2^(m_s - M) go through LDS to the lanes that own the output
// elements, which then read the partial outputs with independent loads.
template <class T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml, void* __restrict__ O,
                                                          float* __restrict__ LSE, int nsplit) {
    constexpr int EB = 16 / Chunk<T>::E;
    __shared__ float wgt[64];
    const size_t bh = blockIdx.x;
    const int lane = threadIdx.x;
    float m = -INFINITY, l = 0.f;
    if (lane < nsplit) {
        m = part_ml[(bh * nsplit + lane) * 2];
        l = part_ml[(bh * nsplit + lane) * 2 + 1];
    }
    float M = m;
#pragma unroll
    for (int x = 1; x < 64; x <<= 1) M = fmaxf(M, __shfl_xor(M, x));
    const float f = m == -INFINITY ? 0.f : fast_exp2(m - M);
    float Ls = l * f;
#pragma unroll
    for (int x = 1; x < 64; x <<= 1) Ls += __shfl_xor(Ls, x);
    wgt[lane] = f;
    __syncthreads();
    const float* po = part_o + bh * nsplit * D;
    for (int d = lane; d < D; d += 64) {
        float od = 0.f;
#pragma unroll 8
        for (int sp = 0; sp < nsplit; ++sp) od = fmaf(po[(size_t)sp * D + d], wgt[sp], od);
        const float x = Ls > 0.f ? od / Ls : 0.f;
        if constexpr (EB == 4)
            reinterpret_cast<float*>(O)[bh * D + d] = x;
        else
            reinterpret_cast<uint16_t*>(O)[bh * D + d] = (uint16_t)(T::pack2(x, 0.f) & 0xffffu);
    }
    if (lane == 0) LSE[bh] = Ls > 0.f ? (M + __log2f(Ls)) * kLn2 : -INFINITY;
}

// Chunking of the cache: at least 256 rows per chunk, enough chunks that the
// first pass has about 2048 workgroups (measured 3-5% faster than 1024 at both
// decode workloads; 4096 no better), at most 64 chunks.
DecodePlan decode_plan(int64_t B, int64_t H, int64_t Hkv, int64_t L, int64_t D) {
    const int64_t G = H / Hkv;
    const int64_t gt = G % 8 == 0 ? 8 : G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1;
    const int64_t units = B * Hkv * (G / gt);
    int64_t nsplit = (2048 + units - 1) / units;
    const int64_t max_split = (L + 255) / 256;
    if (nsplit > max_split) nsplit = max_split;
    if (nsplit > 64) nsplit = 64;  // the merge pass reads one partial per lane
    if (nsplit < 1) nsplit = 1;
    int64_t chunk = (L + nsplit - 1) / nsplit;
    chunk = (chunk + 63) / 64 * 64;
    nsplit = (L + chunk - 1) / chunk;
    DecodePlan p;
    p.gt = (int)gt;
    p.nsplit = (int)nsplit;
    p.chunk = (int)chunk;
    // partial outputs [B*H][nsplit][D], then (m, l) [B*H][nsplit][2], fp32
    p.workspace_bytes = nsplit > 1 ? (size_t)(B * H * nsplit) * (size_t)(D + 2) * sizeof(float) : 0;
    return p;
}

namespace {

template <class T, int D, int GT>
hipError_t launch_decode_gt(const LaunchArgs& a, const DecodePlan& p, float* ws) {
    const int64_t G = a.H / a.Hkv;
    const int64_t B = a.BH / a.H;
    const int64_t grid = B * a.Hkv * (G / GT) * p.nsplit;
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    float* part_o = p.nsplit > 1 ? ws : nullptr;
    float* part_ml = p.nsplit > 1 ? ws + (size_t)a.BH * p.nsplit * D : nullptr;
    hipLaunchKernelGGL((decode_split_kernel<T, D, GT>), dim3((unsigned)grid), dim3(256), 0, a.stream, a.q, a.k, a.v,
                       a.kv_lens, part_o, part_ml, a.o, a.lse, (int)a.H, (int)a.Hkv, (int)a.S, p.nsplit, p.chunk,
                       a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nsplit == 1) return e;
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)a.BH), dim3(64), 0, a.stream, part_o, part_ml,
                       a.o, a.lse, p.nsplit);
    return hipGetLastError();
}

template <class T, int D>
hipError_t launch_decode_d(const LaunchArgs& a, const DecodePlan& p, float* ws) {
    if (p.gt == 8) return launch_decode_gt<T, D, 8>(a, p, ws);
    if (p.gt == 4) return launch_decode_gt<T, D, 4>(a, p, ws);
    if (p.gt == 2) return launch_decode_gt<T, D, 2>(a, p, ws);
    return launch_decode_gt<T, D, 1>(a, p, ws);
}

template <class T>
hipError_t launch_decode_t(const LaunchArgs& a, const DecodePlan& p, float* ws) {
    if (a.D == 64) return launch_decode_d<T, 64>(a, p, ws);
    if (a.D == 80) return launch_decode_d<T, 80>(a, p, ws);
    if (a.D == 96) return launch_decode_d<T, 96>(a, p, ws);
    if (a.D == 128) return launch_decode_d<T, 128>(a, p, ws);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const LaunchArgs& a, int dtype, float* workspace) {
    const DecodePlan p = decode_plan(a.BH / a.H, a.H, a.Hkv, a.S, a.D);
    if (dtype == 0) return launch_decode_t<float>(a, p, workspace);
    if (dtype == 1) return launch_decode_t<Bf16>(a, p, workspace);
    if (dtype == 2) return launch_decode_t<F16>(a, p, workspace);
    return hipErrorInvalidValue;
}

}  // namespace attn
