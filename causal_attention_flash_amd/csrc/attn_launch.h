// Internal launch interface between the C ABI (attn_api.hip) and the kernel
// files.  Arguments arrive here already validated: D in {64, 80, 96, 128} (64 or
// 128 for fp8 Q and K), S >= 1, B*H >= 1, B*H*S < 2^31 and S*D < 2^31, pointers
// non-null, aligned and non-overlapping, scale > 0 and finite.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct LaunchArgs {
    const void* q = nullptr;
    const void* k = nullptr;
    const void* v = nullptr;
    const void* o_in = nullptr;  // forward output, read where delta = rowsum(dO o O) is formed
    const void* dout = nullptr;
    const float* lse_in = nullptr;
    const float* delta_in = nullptr;
    void* o = nullptr;
    float* lse = nullptr;
    float* delta = nullptr;  // delta written by the preprocess or the dQ-with-delta pass
    void* dq = nullptr;
    void* dk = nullptr;
    void* dv = nullptr;
    float* dk_part = nullptr;  // grouped key/value heads: per-query-head fp32 dK, dV ([B,H,S,D])
    float* dv_part = nullptr;
    float* dq_acc = nullptr;  // atomic-dQ backward: fp32 dQ sums ([B,H,S,D], unscaled)
    const int* kv_lens = nullptr;  // decode: rows in use of each sequence's cache ([B]), or null
    int64_t BH = 0;  // batch * query heads
    int64_t H = 0;   // query heads per batch entry
    int64_t Hkv = 0; // key/value heads per batch entry (H is a multiple of Hkv)
    int64_t S = 0;   // sequence length (decode: cache rows L)
    int64_t D = 0;
    float scale = 0.f;
    float qk_descale = 1.f;  // fp8 Q/K: product of their dequantisation factors
    int causal = 1;
    hipStream_t stream = nullptr;
    // attn_bwd of small grids may run its passes on internal streams created on first
    // use; attn_bwd_noalloc clears this so that it creates nothing
    int side_streams = 1;
};

// Compute units of the current device (looked up once per device; 256 on MI355X
// if the query fails).
int cu_count();

hipError_t launch_fwd_bf16(const LaunchArgs& a);
// atomic-dQ backward: dK/dV pass that also adds dQ into a.dq_acc (D = 64, H = H_kv),
// the fill of the accumulator and the final dQ = scale * dq_acc
hipError_t launch_bwd_dkdv_dqa_bf16(const LaunchArgs& a);
hipError_t launch_bwd_dkdv_dqa_f16(const LaunchArgs& a);
hipError_t launch_dq_convert_bf16(const LaunchArgs& a);
hipError_t launch_dq_convert_f16(const LaunchArgs& a);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream);
// forward with fp8 (E4M3) Q and K, V and O of the named type
hipError_t launch_fwd_fp8qk_bf16(const LaunchArgs& a);
hipError_t launch_fwd_fp8qk_f16(const LaunchArgs& a);
hipError_t launch_bwd_dkdv_bf16(const LaunchArgs& a);
hipError_t launch_bwd_dq_bf16(const LaunchArgs& a);
// dQ pass that also forms delta from O and dO and writes it to a.delta
hipError_t launch_bwd_dq_delta_bf16(const LaunchArgs& a);
// dK, dV of each key/value head = sum of its query heads' fp32 partials (16-bit out)
hipError_t launch_group_sum_bf16(const LaunchArgs& a);

// The same kernels for fp16 tensors.
hipError_t launch_fwd_f16(const LaunchArgs& a);
hipError_t launch_bwd_dkdv_f16(const LaunchArgs& a);
hipError_t launch_bwd_dq_f16(const LaunchArgs& a);
hipError_t launch_bwd_dq_delta_f16(const LaunchArgs& a);
hipError_t launch_group_sum_f16(const LaunchArgs& a);

hipError_t launch_fwd_f32(const LaunchArgs& a);
hipError_t launch_bwd_dkdv_f32(const LaunchArgs& a);
// attn_bwd's passes (one query head per key/value head, or the fp32 grouped form):
// fused into one launch for grids too small to fill the device
hipError_t launch_bwd_f32(const LaunchArgs& a);
hipError_t launch_bwd_bf16(const LaunchArgs& a);
hipError_t launch_bwd_f16(const LaunchArgs& a);
hipError_t launch_bwd_dq_f32(const LaunchArgs& a);
hipError_t launch_bwd_dq_delta_f32(const LaunchArgs& a);

// Decode: q [B,H,D] against caches k, v [B,H_kv,L,D] (L in a.S); o [B,H,D], lse
// [B,H].  The cache is read in nsplit chunks of `chunk` rows by workgroups that
// each serve gt query heads of one key/value head; with nsplit > 1 the partials
// go to a workspace of workspace_bytes and a second pass merges them.
struct DecodePlan {
    int gt = 1, nsplit = 1, chunk = 0;
    size_t workspace_bytes = 0;
};
DecodePlan decode_plan(int64_t B, int64_t H, int64_t Hkv, int64_t L, int64_t D);
hipError_t launch_decode(const LaunchArgs& a, int dtype, float* workspace);

// delta = rowsum(dO o O) for any element type (0 = f32, 1 = bf16, 2 = f16: the
// attn_dtype codes).
hipError_t launch_bwd_preprocess(const LaunchArgs& a, int dtype);

}  // namespace attn
