// C ABI of libcausal_attn.so: argument validation, then kernel launches on the
// caller's stream.  The declarations and the contract are in include/attn.h.
//
// Validation happens before anything is enqueued: unsupported combinations are
// rejected loudly rather than run wrong (Iron "Kernel Engineering Guide", §2.5
// on selectors), and argument kinds and counts are checked up front, before any
// work (the TorchMetalKernel checks in "Cooperative tensors, reductions, and
// building a fused attention kernel", §12).
// Any combination outside the supported set returns a status; there is no
// fallback path.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/attn.h"
#include "attn_launch.h"

// Scratch of attn_bwd_noalloc: the fp32 delta vector of up to
// ATTN_NOALLOC_MAX_ROWS query rows.  In host code this name is a stand-in, not a
// device address: kernels and copies get the per-device address that
// hipGetSymbolAddress returns (scratch_on_current_device below).
static __device__ __align__(256) float scratch[ATTN_NOALLOC_MAX_ROWS];

namespace {

// Device address of `scratch` on the current device, looked up once per device
// (each GPU holds its own copy of the array at its own address); nullptr if the
// runtime reports an error.
constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

using attn::LaunchArgs;

int g_cus[kMaxDevices] = {};

struct Span {
    const void* p;
    size_t bytes;
};

bool overlaps(const Span& a, const Span& b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(attn_dtype dt) { return dt == ATTN_F32 ? 4 : 2; }
// bf16 and fp16 run the MFMA kernels; fp32 the vector-ALU kernels
bool is16(attn_dtype dt) { return dt == ATTN_BF16 || dt == ATTN_F16; }

// Sizes, D, dtype.  Sets *empty when there is nothing to compute.
attn_status check_shape(int64_t B, int64_t H, int64_t S, int64_t D, int dtype, bool* empty) {
    if (B < 0 || H < 0 || S < 0 || D < 0) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_ERR_UNSUPPORTED;
    if (D != 64 && D != 80 && D != 96 && D != 128) return ATTN_ERR_UNSUPPORTED;
    *empty = (B == 0 || H == 0 || S == 0);
    if (*empty) return ATTN_OK;
    // B*H*S < 2^31 and S*D < 2^31, checked without overflow.
    const int64_t lim = (int64_t)INT32_MAX;
    if (B > lim || H > lim || S > lim) return ATTN_ERR_SHAPE;
    if (B * H > lim || B * H * S > lim) return ATTN_ERR_SHAPE;
    if (S * D > lim) return ATTN_ERR_SHAPE;
    return ATTN_OK;
}

attn_status check_scale_causal(float scale, int causal) {
    if (causal != 0 && causal != 1) return ATTN_ERR_UNSUPPORTED;
    if (!(scale > 0.f) || !isfinite(scale)) return ATTN_ERR_UNSUPPORTED;
    return ATTN_OK;
}

attn_status check_ptrs(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (!p) return ATTN_ERR_NULL;
    for (const void* p : ps)
        if (!aligned16(p)) return ATTN_ERR_ALIGNMENT;
    return ATTN_OK;
}

attn_status check_alias(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (const Span& i : ins)
            if (overlaps(*o, i)) return ATTN_ERR_ALIAS;
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlaps(*o, *o2)) return ATTN_ERR_ALIAS;
    }
    return ATTN_OK;
}

attn_status from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// Grouped key/value heads: H_kv >= 1 dividing H (negative always rejected; any
// non-negative value is accepted for an empty problem).
attn_status check_groups(int64_t H, int64_t H_kv, bool empty) {
    if (H_kv < 0) return ATTN_ERR_SHAPE;
    if (empty) return ATTN_OK;
    return (H_kv >= 1 && H % H_kv == 0) ? ATTN_OK : ATTN_ERR_SHAPE;
}

struct Sizes {
    size_t tensor;  // bytes of one [B,H,S,D] tensor
    size_t rows;    // bytes of one [B,H,S] fp32 vector
};

Sizes sizes(int64_t B, int64_t H, int64_t S, int64_t D, attn_dtype dt) {
    const size_t n = (size_t)B * (size_t)H * (size_t)S;
    return {n * (size_t)D * (size_t)elem_bytes(dt), n * sizeof(float)};
}

LaunchArgs base_args(int64_t B, int64_t H, int64_t S, int64_t D, float scale, int causal, void* stream) {
    LaunchArgs a;
    a.BH = B * H;
    a.H = H;
    a.Hkv = H;
    a.S = S;
    a.D = D;
    a.scale = scale;
    a.causal = causal;
    a.stream = (hipStream_t)stream;
    return a;
}

attn_status run_preprocess(LaunchArgs a, attn_dtype dt) {
    return from_hip(attn::launch_bwd_preprocess(a, (int)dt));
}
attn_status run_dkdv(const LaunchArgs& a, attn_dtype dt) {
    return from_hip(dt == ATTN_BF16  ? attn::launch_bwd_dkdv_bf16(a)
                    : dt == ATTN_F16 ? attn::launch_bwd_dkdv_f16(a)
                                     : attn::launch_bwd_dkdv_f32(a));
}
attn_status run_dq(const LaunchArgs& a, attn_dtype dt) {
    return from_hip(dt == ATTN_BF16  ? attn::launch_bwd_dq_bf16(a)
                    : dt == ATTN_F16 ? attn::launch_bwd_dq_f16(a)
                                     : attn::launch_bwd_dq_f32(a));
}
// Workspace of the grouped backward: delta (B*H*S fp32), then for bf16/fp16 with more
// than one query head per key/value head the per-query-head fp32 dK and dV
// ([B,H,S,D] each), each region starting on a 256-byte boundary.
size_t round256(size_t n) { return (n + 255) / 256 * 256; }
size_t gqa_workspace(int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D, attn_dtype dt) {
    const Sizes z = sizes(B, H, S, D, dt);
    if (!is16(dt) || H_kv == H) return z.rows;
    const size_t part = (size_t)B * (size_t)H * (size_t)S * (size_t)D * sizeof(float);
    return round256(z.rows) + 2 * round256(part);
}
attn_status run_group_sum(const LaunchArgs& a, attn_dtype dt) {
    return from_hip(dt == ATTN_F16 ? attn::launch_group_sum_f16(a) : attn::launch_group_sum_bf16(a));
}
attn_status run_dq_delta(const LaunchArgs& a, attn_dtype dt) {
    return from_hip(dt == ATTN_BF16  ? attn::launch_bwd_dq_delta_bf16(a)
                    : dt == ATTN_F16 ? attn::launch_bwd_dq_delta_f16(a)
                                     : attn::launch_bwd_dq_delta_f32(a));
}
// The dQ pass, which forms delta, then the dK/dV pass that reads it, or both in one
// launch where the grids are too small to fill the device.
attn_status run_bwd_passes(const LaunchArgs& a, attn_dtype dt) {
    return from_hip(dt == ATTN_BF16  ? attn::launch_bwd_bf16(a)
                    : dt == ATTN_F16 ? attn::launch_bwd_f16(a)
                                     : attn::launch_bwd_f32(a));
}

}  // namespace

int attn::cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    if (g_cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        g_cus[dev] = n;
    }
    return g_cus[dev];
}

extern "C" {

const char* attn_status_string(attn_status s) {
    switch (s) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE:
            return "negative size, sizes beyond B*H*S < 2^31 and S*D < 2^31, or H_kv < 1 or not dividing H";
        case ATTN_ERR_UNSUPPORTED:
            return "unsupported: D must be 64, 80, 96 or 128 (64 or 128 with fp8 Q and K), dtype ATTN_F32, ATTN_BF16 "
                   "or ATTN_F16 (16-bit with fp8 Q and K), causal 0 or 1, scale and fp8 descale factors finite and > 0";
        case ATTN_ERR_ALIGNMENT: return "a device pointer is not 16-byte aligned";
        case ATTN_ERR_WORKSPACE: return "workspace is NULL or smaller than attn_bwd_workspace_bytes()";
        case ATTN_ERR_HIP: return "the HIP runtime reported an error at launch";
        case ATTN_ERR_ALIAS: return "an output buffer overlaps an input or another output";
        case ATTN_ERR_SCRATCH:
            return "attn_bwd_noalloc: B*H*S exceeds ATTN_NOALLOC_MAX_ROWS, the rows its static scratch holds";
    }
    return "unknown attn_status";
}

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                     int64_t S, int64_t D, float scale, int causal, attn_dtype dtype, void* stream) {
    return attn_fwd_gqa(q, k, v, o, lse, B, H, H, S, D, scale, causal, dtype, stream);
}

attn_status attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                         int64_t H_kv, int64_t S, int64_t D, float scale, int causal, attn_dtype dtype,
                         void* stream) {
    bool empty = false;
    attn_status st = check_shape(B, H, S, D, dtype, &empty);
    if (st == ATTN_OK) st = check_groups(H, H_kv, empty);
    if (st == ATTN_OK) st = check_scale_causal(scale, causal);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_ptrs({q, k, v, o, lse})) != ATTN_OK) return st;
    const Sizes z = sizes(B, H, S, D, dtype);
    const size_t zkv = z.tensor / (size_t)H * (size_t)H_kv;
    if ((st = check_alias({{o, z.tensor}, {lse, z.rows}}, {{q, z.tensor}, {k, zkv}, {v, zkv}})) != ATTN_OK)
        return st;
    LaunchArgs a = base_args(B, H, S, D, scale, causal, stream);
    a.Hkv = H_kv;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    return from_hip(dtype == ATTN_BF16  ? attn::launch_fwd_bf16(a)
                    : dtype == ATTN_F16 ? attn::launch_fwd_f16(a)
                                        : attn::launch_fwd_f32(a));
}

attn_status attn_fwd_fp8qk(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                           int64_t H, int64_t H_kv, int64_t S, int64_t D, float scale, float q_descale,
                           float k_descale, int causal, attn_dtype dtype, void* stream) {
    bool empty = false;
    attn_status st = check_shape(B, H, S, D, dtype, &empty);
    // the fp8 product contracts 64 values per instruction; V and O are 16-bit
    if (st == ATTN_OK && ((D != 64 && D != 128) || !is16(dtype))) st = ATTN_ERR_UNSUPPORTED;
    if (st == ATTN_OK) st = check_groups(H, H_kv, empty);
    if (st == ATTN_OK) st = check_scale_causal(scale, causal);
    if (st == ATTN_OK && (!(q_descale > 0.f) || !isfinite(q_descale) || !(k_descale > 0.f) ||
                          !isfinite(k_descale) || !isfinite(scale * q_descale * k_descale) ||
                          !(scale * q_descale * k_descale > 0.f)))
        st = ATTN_ERR_UNSUPPORTED;
    if (st != ATTN_OK || empty) return st;
    if ((st = check_ptrs({q, k, v, o, lse})) != ATTN_OK) return st;
    const Sizes z = sizes(B, H, S, D, dtype);
    const size_t zkv = z.tensor / (size_t)H * (size_t)H_kv;  // V: 16-bit elements
    if ((st = check_alias({{o, z.tensor}, {lse, z.rows}}, {{q, z.tensor / 2}, {k, zkv / 2}, {v, zkv}})) != ATTN_OK)
        return st;
    LaunchArgs a = base_args(B, H, S, D, scale, causal, stream);
    a.Hkv = H_kv;
    a.qk_descale = q_descale * k_descale;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    return from_hip(dtype == ATTN_BF16 ? attn::launch_fwd_fp8qk_bf16(a) : attn::launch_fwd_fp8qk_f16(a));
}

size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D, attn_dtype dtype) {
    bool empty = false;
    if (check_shape(B, H, S, D, dtype, &empty) != ATTN_OK || empty) return 0;
    return sizes(B, H, S, D, dtype).rows;
}

attn_status attn_bwd_preprocess(const void* o, const void* dout, float* delta, int64_t B, int64_t H, int64_t S,
                                int64_t D, attn_dtype dtype, void* stream) {
    bool empty = false;
    attn_status st = check_shape(B, H, S, D, dtype, &empty);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_ptrs({o, dout, delta})) != ATTN_OK) return st;
    const Sizes z = sizes(B, H, S, D, dtype);
    if ((st = check_alias({{delta, z.rows}}, {{o, z.tensor}, {dout, z.tensor}})) != ATTN_OK) return st;
    LaunchArgs a = base_args(B, H, S, D, 1.f, 1, stream);
    a.o_in = o;
    a.dout = dout;
    a.delta = delta;
    return run_preprocess(a, dtype);
}

attn_status attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                          const float* delta, void* dk, void* dv, int64_t B, int64_t H, int64_t S, int64_t D,
                          float scale, int causal, attn_dtype dtype, void* stream) {
    bool empty = false;
    attn_status st = check_shape(B, H, S, D, dtype, &empty);
    if (st == ATTN_OK) st = check_scale_causal(scale, causal);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_ptrs({q, k, v, dout, lse, delta, dk, dv})) != ATTN_OK) return st;
    const Sizes z = sizes(B, H, S, D, dtype);
    if ((st = check_alias({{dk, z.tensor}, {dv, z.tensor}}, {{q, z.tensor},
                                                              {k, z.tensor},
                                                              {v, z.tensor},
                                                              {dout, z.tensor},
                                                              {lse, z.rows},
                                                              {delta, z.rows}})) != ATTN_OK)
        return st;
    LaunchArgs a = base_args(B, H, S, D, scale, causal, stream);
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.lse_in = lse;
    a.delta_in = delta;
    a.dk = dk;
    a.dv = dv;
    return run_dkdv(a, dtype);
}

attn_status attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                        const float* delta, void* dq, int64_t B, int64_t H, int64_t S, int64_t D, float scale,
                        int causal, attn_dtype dtype, void* stream) {
    bool empty = false;
    attn_status st = check_shape(B, H, S, D, dtype, &empty);
    if (st == ATTN_OK) st = check_scale_causal(scale, causal);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_ptrs({q, k, v, dout, lse, delta, dq})) != ATTN_OK) return st;
    const Sizes z = sizes(B, H, S, D, dtype);
    if ((st = check_alias({{dq, z.tensor}}, {{q, z.tensor},
                                              {k, z.tensor},
                                              {v, z.tensor},
                                              {dout, z.tensor},
                                              {lse, z.rows},
                                              {delta, z.rows}})) != ATTN_OK)
        return st;
    LaunchArgs a = base_args(B, H, S, D, scale, causal, stream);
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.lse_in = lse;
    a.delta_in = delta;
    a.dq = dq;
    return run_dq(a, dtype);
}

attn_status attn_bwd_dq_delta(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, float* delta, void* dq, int64_t B, int64_t H, int64_t S, int64_t D,
                              float scale, int causal, attn_dtype dtype, void* stream) {
    bool empty = false;
    attn_status st = check_shape(B, H, S, D, dtype, &empty);
    if (st == ATTN_OK) st = check_scale_causal(scale, causal);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_ptrs({q, k, v, o, dout, lse, delta, dq})) != ATTN_OK) return st;
    const Sizes z = sizes(B, H, S, D, dtype);
    if ((st = check_alias({{dq, z.tensor}, {delta, z.rows}}, {{q, z.tensor},
                                                               {k, z.tensor},
                                                               {v, z.tensor},
                                                               {o, z.tensor},
                                                               {dout, z.tensor},
                                                               {lse, z.rows}})) != ATTN_OK)
        return st;
    LaunchArgs a = base_args(B, H, S, D, scale, causal, stream);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o_in = o;
    a.dout = dout;
    a.lse_in = lse;
    a.delta = delta;
    a.dq = dq;
    return run_dq_delta(a, dtype);
}

size_t attn_bwd_atomic_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D, attn_dtype dtype) {
    bool empty = false;
    if (check_shape(B, H, S, D, dtype, &empty) != ATTN_OK || empty || D != 64 || !is16(dtype)) return 0;
    const Sizes z = sizes(B, H, S, D, dtype);
    return round256(z.rows) + (size_t)B * (size_t)H * (size_t)S * (size_t)D * sizeof(float);
}

attn_status attn_bwd_atomic(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                            int64_t B, int64_t H, int64_t S, int64_t D, float scale, int causal, attn_dtype dtype,
                            void* stream) {
    bool empty = false;
    attn_status st = check_shape(B, H, S, D, dtype, &empty);
    if (st == ATTN_OK && (D != 64 || !is16(dtype))) st = ATTN_ERR_UNSUPPORTED;
    if (st == ATTN_OK) st = check_scale_causal(scale, causal);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_ptrs({q, k, v, o, dout, lse, dq, dk, dv})) != ATTN_OK) return st;
    const Sizes z = sizes(B, H, S, D, dtype);
    const size_t wsz = attn_bwd_atomic_workspace_bytes(B, H, S, D, dtype);
    if (!workspace || workspace_bytes < wsz) return ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_ERR_ALIGNMENT;
    if ((st = check_alias({{dq, z.tensor}, {dk, z.tensor}, {dv, z.tensor}, {workspace, wsz}},
                          {{q, z.tensor}, {k, z.tensor}, {v, z.tensor}, {o, z.tensor}, {dout, z.tensor},
                           {lse, z.rows}})) != ATTN_OK)
        return st;
    LaunchArgs a = base_args(B, H, S, D, scale, causal, stream);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o_in = o;
    a.dout = dout;
    a.lse_in = lse;
    a.delta = (float*)workspace;
    a.delta_in = (const float*)workspace;
    a.dq_acc = (float*)((char*)workspace + round256(z.rows));
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    if ((st = run_preprocess(a, dtype)) != ATTN_OK) return st;
    if ((st = from_hip(attn::launch_fill_zero(a.dq_acc, (int64_t)(z.tensor / 2), a.stream))) != ATTN_OK) return st;
    if ((st = from_hip(dtype == ATTN_BF16 ? attn::launch_bwd_dkdv_dqa_bf16(a) : attn::launch_bwd_dkdv_dqa_f16(a))) !=
        ATTN_OK)
        return st;
    return from_hip(dtype == ATTN_BF16 ? attn::launch_dq_convert_bf16(a) : attn::launch_dq_convert_f16(a));
}

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                     int64_t S, int64_t D, float scale, int causal, attn_dtype dtype, void* stream) {
    return attn_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H, S, D, scale, causal,
                        dtype, stream);
}

attn_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                             const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t S,
                             int64_t D, float scale, int causal, attn_dtype dtype, void* stream) {
    bool empty = false;
    attn_status st = check_shape(B, H, S, D, dtype, &empty);
    if (st == ATTN_OK) st = check_scale_causal(scale, causal);
    if (st != ATTN_OK || empty) return st;
    if (B * H * S > (int64_t)ATTN_NOALLOC_MAX_ROWS) return ATTN_ERR_SCRATCH;
    if ((st = check_ptrs({q, k, v, o, dout, lse, dq, dk, dv})) != ATTN_OK) return st;
    const Sizes z = sizes(B, H, S, D, dtype);
    if ((st = check_alias({{dq, z.tensor}, {dk, z.tensor}, {dv, z.tensor}},
                          {{q, z.tensor}, {k, z.tensor}, {v, z.tensor}, {o, z.tensor}, {dout, z.tensor},
                           {lse, z.rows}})) != ATTN_OK)
        return st;
    float* delta = static_cast<float*>(scratch_on_current_device());
    if (!delta) return ATTN_ERR_HIP;
    LaunchArgs a = base_args(B, H, S, D, scale, causal, stream);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o_in = o;
    a.dout = dout;
    a.lse_in = lse;
    a.delta = delta;
    a.delta_in = delta;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    // as attn_bwd: the dQ pass forms delta, then the dK/dV pass reads it (always on
    // `stream`: no internal streams, which would be created on first use)
    a.side_streams = 0;
    return run_bwd_passes(a, dtype);
}

attn_status attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                         int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D, float scale, int causal,
                         attn_dtype dtype, void* stream) {
    bool empty = false;
    attn_status st = check_shape(B, H, S, D, dtype, &empty);
    if (st == ATTN_OK) st = check_groups(H, H_kv, empty);
    if (st == ATTN_OK) st = check_scale_causal(scale, causal);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_ptrs({q, k, v, o, dout, lse, dq, dk, dv})) != ATTN_OK) return st;
    const Sizes z = sizes(B, H, S, D, dtype);
    const size_t zkv = z.tensor / (size_t)H * (size_t)H_kv;
    const size_t wsz = gqa_workspace(B, H, H_kv, S, D, dtype);
    if (!workspace || workspace_bytes < wsz) return ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_ERR_ALIGNMENT;
    if ((st = check_alias({{dq, z.tensor}, {dk, zkv}, {dv, zkv}, {workspace, wsz}},
                          {{q, z.tensor},
                           {k, zkv},
                           {v, zkv},
                           {o, z.tensor},
                           {dout, z.tensor},
                           {lse, z.rows}})) != ATTN_OK)
        return st;
    LaunchArgs a = base_args(B, H, S, D, scale, causal, stream);
    a.Hkv = H_kv;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o_in = o;
    a.dout = dout;
    a.lse_in = lse;
    a.delta = (float*)workspace;
    a.delta_in = (const float*)workspace;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    const bool partials = is16(dtype) && H_kv != H;
    if (partials) {
        char* w = (char*)workspace;
        const size_t part = (size_t)B * (size_t)H * (size_t)S * (size_t)D * sizeof(float);
        a.dk_part = (float*)(w + round256(z.rows));
        a.dv_part = (float*)(w + round256(z.rows) + round256(part));
    }
    // dQ first: it forms delta, which the dK/dV pass reads; with grouped heads in
    // bf16/fp16 the dK/dV pass leaves per-query-head partials that the group sum adds
    if ((st = run_bwd_passes(a, dtype)) != ATTN_OK) return st;
    return partials ? run_group_sum(a, dtype) : ATTN_OK;
}

// Decode shapes: B, H >= 0; H_kv >= 1 dividing H; L >= 1; B*H*L and L*D below
// 2^31 (B or H = 0 is an empty problem).
attn_status check_decode(int64_t B, int64_t H, int64_t H_kv, int64_t L, int64_t D, int dtype, bool* empty) {
    attn_status st = check_shape(B, H, L, D, dtype, empty);
    if (st != ATTN_OK) return st;
    if (H_kv < 0) return ATTN_ERR_SHAPE;
    if (*empty) return L == 0 ? ATTN_ERR_SHAPE : ATTN_OK;
    if (H_kv < 1 || H % H_kv != 0) return ATTN_ERR_SHAPE;
    return ATTN_OK;
}

size_t attn_decode_workspace_bytes(int64_t B, int64_t H, int64_t H_kv, int64_t L, int64_t D, attn_dtype dtype) {
    bool empty = false;
    if (check_decode(B, H, H_kv, L, D, dtype, &empty) != ATTN_OK || empty) return 0;
    return attn::decode_plan(B, H, H_kv, L, D).workspace_bytes;
}

attn_status attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* kv_lens, void* o,
                        float* lse, void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t H_kv,
                        int64_t L, int64_t D, float scale, attn_dtype dtype, void* stream) {
    bool empty = false;
    attn_status st = check_decode(B, H, H_kv, L, D, dtype, &empty);
    if (st == ATTN_OK) st = check_scale_causal(scale, 1);
    if (st != ATTN_OK || empty) return st;
    if ((st = check_ptrs({q, k_cache, v_cache, o, lse})) != ATTN_OK) return st;
    if (kv_lens && ((uintptr_t)kv_lens & 3u) != 0) return ATTN_ERR_ALIGNMENT;
    const size_t eb = (size_t)elem_bytes(dtype);
    const size_t zq = (size_t)B * (size_t)H * (size_t)D * eb;
    const size_t zkv = (size_t)B * (size_t)H_kv * (size_t)L * (size_t)D * eb;
    const size_t zl = (size_t)B * (size_t)H * sizeof(float);
    const size_t wsz = attn::decode_plan(B, H, H_kv, L, D).workspace_bytes;
    if (wsz > 0) {
        if (!workspace || workspace_bytes < wsz) return ATTN_ERR_WORKSPACE;
        if (!aligned16(workspace)) return ATTN_ERR_ALIGNMENT;
    }
    if ((st = check_alias({{o, zq}, {lse, zl}, {wsz > 0 ? workspace : nullptr, wsz}},
                          {{q, zq}, {k_cache, zkv}, {v_cache, zkv}, {kv_lens, kv_lens ? (size_t)B * 4 : 0}})) !=
        ATTN_OK)
        return st;
    LaunchArgs a = base_args(B, H, L, D, scale, 1, stream);
    a.Hkv = H_kv;
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.kv_lens = kv_lens;
    a.o = o;
    a.lse = lse;
    return from_hip(attn::launch_decode(a, (int)dtype, (float*)workspace));
}

size_t attn_bwd_gqa_workspace_bytes(int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D, attn_dtype dtype) {
    bool empty = false;
    if (check_shape(B, H, S, D, dtype, &empty) != ATTN_OK || empty) return 0;
    if (check_groups(H, H_kv, empty) != ATTN_OK) return 0;
    return gqa_workspace(B, H, H_kv, S, D, dtype);
}

}  // extern "C"
