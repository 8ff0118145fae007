// Backward preprocess: delta_i = sum_d dO_id * O_id in fp32, once per query row.
//
// Forge RESEARCH.md §6, the "D term" paragraph: rowsum(dP o P) equals dO_i . O_i
// exactly, so it is computed once per row outside the two main backward kernels
// instead of per (query, key) pair (the hoist the page measures at 3.1x on a
// training step).  O here is the forward output as stored (fp32, bf16 or fp16).
//
// Memory-bound: each lane reads 16 bytes of O and of dO per row slice.  A row
// gets G lanes, the power of two at or above its D*elem/16 slices (lanes past
// the last slice contribute zero), which reduce their partial dots with
// cross-lane xors.
#include "attn_launch.h"
#include "attn_device.h"

namespace attn {

constexpr int pow2_at_least(int x) { return x <= 1 ? 1 : 2 * pow2_at_least((x + 1) / 2); }

template <int DT, int D>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(const void* __restrict__ O, const void* __restrict__ dO,
                                                             float* __restrict__ delta, int64_t rows) {
    constexpr int ELEM_BYTES = DT == 0 ? 4 : 2;  // attn_dtype: 0 f32, 1 bf16, 2 f16
    constexpr int SL = D * ELEM_BYTES / 16;  // 16-byte slices per row (8 .. 32)
    constexpr int G = pow2_at_least(SL);     // lanes per row
    constexpr int RPB = 256 / G;             // rows per block
    const int tid = threadIdx.x;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / G;
    const int part = tid % G;
    float acc = 0.f;
    if (row < rows && part < SL) {
        const size_t off = (size_t)row * D * ELEM_BYTES + (size_t)part * 16;
        const u32x4 a = ldg16((const char*)O + off);
        const u32x4 b = ldg16((const char*)dO + off);
        if constexpr (DT == 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc = fmaf(Bf16::lo(a[e]), Bf16::lo(b[e]), acc);
                acc = fmaf(Bf16::hi(a[e]), Bf16::hi(b[e]), acc);
            }
        } else if constexpr (DT == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc = fmaf(F16::lo(a[e]), F16::lo(b[e]), acc);
                acc = fmaf(F16::hi(a[e]), F16::hi(b[e]), acc);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = fmaf(__uint_as_float(a[e]), __uint_as_float(b[e]), acc);
        }
    }
#pragma unroll
    for (int s = 1; s < G; s <<= 1) acc += __shfl_xor(acc, s);
    if (row < rows && part == 0) delta[row] = acc;
}

template <int DT, int D>
static hipError_t launch_pre(const LaunchArgs& a) {
    constexpr int RPB = 256 / pow2_at_least(D * (DT == 0 ? 4 : 2) / 16);
    const int64_t rows = a.BH * a.S;
    const int64_t blocks = (rows + RPB - 1) / RPB;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_preprocess_kernel<DT, D>), dim3((unsigned)blocks), dim3(256), 0, a.stream,
                       a.o_in, a.dout, a.delta, rows);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_pre_type(const LaunchArgs& a) {
    if (a.D == 64) return launch_pre<DT, 64>(a);
    if (a.D == 80) return launch_pre<DT, 80>(a);
    if (a.D == 96) return launch_pre<DT, 96>(a);
    if (a.D == 128) return launch_pre<DT, 128>(a);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_preprocess(const LaunchArgs& a, int dtype) {
    if (dtype == 0) return launch_pre_type<0>(a);
    if (dtype == 1) return launch_pre_type<1>(a);
    if (dtype == 2) return launch_pre_type<2>(a);
    return hipErrorInvalidValue;
}

}  // namespace attn
