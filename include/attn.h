/*
 * attn.h - fused causal scaled-dot-product attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libcausal_attn.so.  Plain pointers and sizes only; every pointer named
 * "device" is HIP device memory, every size is an element count unless it says
 * bytes.  The caller owns every buffer and the stream; the library never
 * allocates, frees, synchronises or keeps a pointer past the call.  Work is
 * enqueued asynchronously on `stream` (a hipStream_t; NULL = the default stream),
 * so buffers must stay alive until the stream has passed that point.
 *
 * What is computed (per batch b and head h, all indices in [0, S)):
 *
 *   s_ij  = scale * sum_d q_id k_jd
 *   query i sees key j iff (!causal || j <= i)            (top-left aligned mask)
 *   LSE_i = ln sum_{j visible} exp(s_ij)                  (natural log, fp32)
 *   P_ij  = exp(s_ij - LSE_i) for visible j, else 0
 *   O_i   = sum_j P_ij v_j
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j,   delta_i = dO_i . O_i,   dS_ij = P_ij (dP_ij - delta_i)
 *   dQ_i  = scale * sum_j dS_ij k_j,   dK_j = scale * sum_i dS_ij q_i
 *
 * Sources: attention as S = QK^T, row softmax, O = PV and the causal mask that
 * hides every key after the query's own position follow "Cooperative tensors,
 * reductions, and building a fused attention kernel" (§1, §5.3, §8.7).  The
 * online-softmax forward that saves one log-sum-exp per row, the three-stage
 * atomic-free backward (delta = rowsum(dO o O) preprocess, a dQ pass parallel
 * over queries, a dK/dV pass parallel over keys, both recomputing P from the
 * saved LSE) follow Forge
 * RESEARCH.md §6 "Fused attention design (flash-style)" and the Forge paper,
 * sections "Ecosystem survey" and "Attention kernel design".
 *
 * Layout: Q, K, V, O, dO, dQ, dK, dV are contiguous [B, H, S, D] (D innermost);
 * LSE and delta are contiguous [B, H, S] fp32.  Tensor element type is `dtype`
 * (ATTN_F32: float, ATTN_BF16: bfloat16 bit patterns, ATTN_F16: IEEE binary16
 * bit patterns); accumulation and all
 * softmax statistics are fp32 whatever the input type.  Outputs are written in
 * the input type, rounded to nearest even.
 *
 * Supported set: D in {64, 80, 96, 128} (the head dimensions of GPT-style
 * models; Forge RESEARCH.md §6 "Fused attention design" lists 64, 80 and 128 as
 * the tuned set and its pitfalls section compares backward variants up to
 * D = 96); dtype in {ATTN_F32, ATTN_BF16, ATTN_F16} (fp16 operands with fp32
 * accumulation and statistics are the form of the assembled kernel in §9 of
 * "Cooperative tensors, reductions, and building a fused attention kernel", and
 * the Forge paper measures its matmul2d with half operands); causal in {0, 1};
 * scale finite and > 0 (the forward takes each row's maximum over the raw
 * products, which commutes with the scaling only for a positive factor; a
 * scale <= 0, NaN or infinite -> ATTN_ERR_UNSUPPORTED); any S >= 1 (no
 * tile-multiple requirement).  Size limits, checked without overflow:
 * B*H*S < 2^31 (query rows; H counts query heads) and S*D < 2^31 (one head's
 * elements), every kernel indexing both in 32 bits; beyond either ->
 * ATTN_ERR_SHAPE.  B, H or S equal to 0 is an empty problem: ATTN_OK, nothing
 * enqueued, pointers not read.
 *
 * Errors: every argument is validated before anything is enqueued.  On any
 * error status nothing is launched and no output is touched.  ATTN_ERR_HIP
 * reports a launch failure read back with hipGetLastError (the stream may then
 * hold part of the work).  Outputs must not overlap inputs or each other
 * (ATTN_ERR_ALIAS).  All device pointers must be 16-byte aligned.
 *
 * Determinism: every entry point except attn_bwd_atomic uses no atomics, and its
 * results are bitwise identical run to run for the same inputs, sizes and
 * library build.  attn_bwd_atomic's dQ is the one exception (see there).
 */
#ifndef CAUSAL_ATTN_H
#define CAUSAL_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_dtype {
    ATTN_F32 = 0,  /* float32 tensors */
    ATTN_BF16 = 1, /* bfloat16 tensors (uint16 bit patterns) */
    ATTN_F16 = 2   /* IEEE fp16 tensors (uint16 bit patterns) */
} attn_dtype;

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
    ATTN_ERR_SHAPE = 2,       /* a negative size, sizes whose products overflow the limits, or a
                                 key/value head count that does not divide the query heads */
    ATTN_ERR_UNSUPPORTED = 3, /* D, dtype, causal flag or scale outside the supported set */
    ATTN_ERR_ALIGNMENT = 4,   /* a device pointer not aligned to 16 bytes */
    ATTN_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than attn_bwd_workspace_bytes() */
    ATTN_ERR_HIP = 6,         /* the HIP runtime reported an error when launching */
    ATTN_ERR_ALIAS = 7,       /* an output overlaps an input or another output */
    ATTN_ERR_SCRATCH = 8      /* attn_bwd_noalloc: more query rows than its static scratch holds */
} attn_status;

/*
 * Forward pass: O and LSE from Q, K, V.
 *   q, k, v : device, [B,H,S,D] of dtype, read only.
 *   o       : device, [B,H,S,D] of dtype, fully overwritten.
 *   lse     : device, [B,H,S] fp32, fully overwritten (natural-log log-sum-exp of
 *             the scaled, masked scores; the backward pass takes it back).
 *   scale   : multiplies QK^T before the softmax (typically 1/sqrt(D)).
 *   causal  : 1 = query i sees keys j <= i; 0 = every key.
 * Source: Forge RESEARCH.md §6 (online-softmax recurrence, divide by the row sum
 * once after the loop, L = m + log l saved per row).
 * Summation order: grids of few query blocks (B*H*ceil(S/128) up to 2/3 of the
 * device's workgroup slots at D = 64, up to all of them from D = 80 up) split each
 * block's keys between two waves and merge the two partial softmax states; a head's
 * O and LSE can therefore differ in the last bits between calls whose B*H or S put
 * them on different sides of that line (both within the accuracy the tests hold
 * them to).
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t B, int64_t H, int64_t S, int64_t D,
                     float scale, int causal, attn_dtype dtype, void* stream);

/*
 * Forward pass with grouped key/value heads (GQA): H query heads per batch entry
 * share H_kv key/value heads (H a multiple of H_kv, G = H / H_kv); query head h
 * reads key/value head h / G.  Source: Forge RESEARCH.md §6, the "GQA" index map
 * (kv_head = q_head / (n_heads / n_kv_heads), no repeated copies).
 *   q, o    : device, [B,H,S,D] of dtype.
 *   k, v    : device, [B,H_kv,S,D] of dtype, read only.
 *   lse     : device, [B,H,S] fp32.
 * attn_fwd is this call with H_kv = H.  Other rules as attn_fwd; H_kv < 1 or not
 * dividing H -> ATTN_ERR_SHAPE.
 */
attn_status attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D,
                         float scale, int causal, attn_dtype dtype, void* stream);

/*
 * Forward pass with fp8 Q and K (inference): the scores come from the fp8 matrix
 * instructions, the rest is attn_fwd_gqa.
 *   q          : device, [B,H,S,D] bytes, OCP FP8 E4M3 codes (sign, 4 exponent bits
 *                with bias 7, 3 mantissa bits; subnormals; no infinities; 0x7F and
 *                0xFF are NaN), read only; the values are code * q_descale.
 *   k          : device, [B,H_kv,S,D] E4M3 codes, read only; values code * k_descale.
 *   v          : device, [B,H_kv,S,D] of dtype (ATTN_BF16 or ATTN_F16), read only.
 *   o, lse     : as attn_fwd_gqa (o of dtype).
 *   q_descale, k_descale : finite, > 0 (per-tensor dequantisation factors).
 * Computes S = scale * q_descale * k_descale * (codes of Q)(codes of K)^T: the
 * products of two E4M3 values are exact and are summed in fp32 by
 * v_mfma_f32_32x32x64_f8f6f4, whose internal alignment is narrower than a serial
 * fp32 sum (relative differences up to ~6e-5 on random 64-term sums); then P, O
 * and LSE exactly as attn_fwd_gqa.  The E4M3 grid, its saturation at 448 and the
 * fp32 accumulation of fp8 products follow the Rigel paper (§5 "Is fp8
 * accelerated or emulated?" and §6 on accumulator width and the low-precision
 * formats); encoding to E4M3 (rounding, saturation, choice of the descale
 * factors) is the caller's.
 * Supported set: D in {64, 128}; dtype ATTN_BF16 or ATTN_F16; other rules as
 * attn_fwd_gqa; anything else -> ATTN_ERR_UNSUPPORTED.  No backward.
 */
attn_status attn_fwd_fp8qk(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D,
                           float scale, float q_descale, float k_descale, int causal,
                           attn_dtype dtype, void* stream);

/*
 * Bytes of device workspace attn_bwd needs: the fp32 delta vector, B*H*S*4 bytes.
 * delta_i = dO_i . O_i is formed once per query row and read by both backward
 * passes (Forge RESEARCH.md §6, the paragraph on the D term: it is needed by the
 * dK/dV and the dQ kernel and costs a cubic factor if formed per pair instead of
 * per row), so it is stored between them.  Returns 0 for an empty or invalid
 * problem (the same checks as attn_bwd).
 */
size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D, attn_dtype dtype);

/*
 * Backward pass: dQ, dK, dV from Q, K, V, the forward's O and LSE, and dO.
 *   q, k, v, o, dout : device, [B,H,S,D] of dtype, read only (o = the forward output).
 *   lse              : device, [B,H,S] fp32, read only (the forward's LSE).
 *   dq, dk, dv       : device, [B,H,S,D] of dtype, fully overwritten.
 *   workspace        : device, at least attn_bwd_workspace_bytes() bytes, owned by the
 *                      caller; clobbered; must not overlap any other argument.
 * Enqueues, in order: the dQ pass, which also forms delta = rowsum(dO o O) (fp32)
 * in the workspace, then the dK/dV pass, which reads it; for grids too small to
 * fill the device well (fp32 grids whose blocks cover it less than twice, 16-bit
 * D = 64 grids with one query head per key/value head whose dQ and dK/dV blocks fit
 * in three rounds) one launch runs the dQ blocks and dK/dV blocks side by side, the latter
 * forming delta themselves in the dQ pass's order: the same bits either way.
 * 16-bit grids (without the one-launch form) whose dQ pass and dK/dV pass(es) each
 * fit in one round of the device (D = 128, or D < 128 with S >= 2048)
 * form delta first, in the dQ pass's order, then run the dQ pass on `stream` and the
 * dK/dV pass (at D = 128 its dV and dK passes) on internal streams beside it, joined
 * back into `stream` with events before the call returns: work enqueued on `stream`
 * afterwards sees the whole backward, and the results are the same bits.  The
 * internal streams (default priority) and events are created on the first such call
 * on a device and kept until the process ends; a mutex orders such calls from several
 * host threads.  While `stream` is being captured into a graph the passes are
 * enqueued on `stream` alone.
 * Source: Forge RESEARCH.md §6 (the "D term" paragraph and the two-kernel,
 * atomic-free backward that recomputes P = exp(S - L) per tile).
 */
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse,
                     void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes,
                     int64_t B, int64_t H, int64_t S, int64_t D,
                     float scale, int causal, attn_dtype dtype, void* stream);

/*
 * attn_bwd without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The delta vector lives in a static device array of the
 * library (ATTN_NOALLOC_MAX_ROWS fp32 values, 8 MiB, held by every GPU the
 * library runs on until the process ends); the call allocates nothing.
 *   Arguments, outputs and errors as attn_bwd, without workspace and
 *   workspace_bytes; B*H*S > ATTN_NOALLOC_MAX_ROWS -> ATTN_ERR_SCRATCH (nothing
 *   enqueued).  Same kernels and results (bitwise) as attn_bwd, every pass on
 *   `stream` (never attn_bwd's internal streams, which would be created on first use).
 *   The stream must belong to the current device.  Every call on one GPU uses
 *   that GPU's single scratch array: calls that overlap on one GPU (other
 *   streams, other threads) race and must be ordered by the caller.  delta is
 *   fully written by the dQ pass before the dK/dV pass reads it, so nothing in
 *   the array needs to start at zero.
 */
#define ATTN_NOALLOC_MAX_ROWS (1 << 21)
attn_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse,
                             void* dq, void* dk, void* dv,
                             int64_t B, int64_t H, int64_t S, int64_t D,
                             float scale, int causal, attn_dtype dtype, void* stream);

/*
 * Bytes of device workspace attn_bwd_atomic needs: the fp32 delta vector (B*H*S*4
 * bytes, rounded up to 256) and the fp32 dQ accumulator (B*H*S*D*4 bytes).
 * Returns 0 for an empty, invalid or unsupported problem.
 */
size_t attn_bwd_atomic_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D, attn_dtype dtype);

/*
 * Backward pass with atomic dQ accumulation (opt-in; dQ is NOT bitwise
 * reproducible: the order of its fp32 additions varies from run to run).
 * Arguments, outputs and errors as attn_bwd, with a workspace of
 * attn_bwd_atomic_workspace_bytes() bytes.  Enqueues: delta = rowsum(dO o O)
 * (fp32), a fill of the dQ accumulator with zeros, one dK/dV pass that also adds
 * every (query block, key block) contribution to dQ into the accumulator with fp32
 * atomic adds, and dQ = scale * accumulator rounded to dtype.  dV is
 * bit-identical to attn_bwd's; dK equals it up to the rounding of delta, which
 * attn_bwd forms in its dQ pass.  This is the FlashAttention-2 fused backward that
 * Forge RESEARCH.md §6 describes as the atomic alternative to its separate,
 * deterministic dQ pass; it saves that pass's recomputation of S and dP.
 * Supported set: D = 64; dtype ATTN_BF16 or ATTN_F16; one query head per
 * key/value head; other rules as attn_bwd; anything else -> ATTN_ERR_UNSUPPORTED.
 */
attn_status attn_bwd_atomic(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse,
                            void* dq, void* dk, void* dv,
                            void* workspace, size_t workspace_bytes,
                            int64_t B, int64_t H, int64_t S, int64_t D,
                            float scale, int causal, attn_dtype dtype, void* stream);

/*
 * Backward pass with grouped key/value heads: dQ as attn_bwd; dK and dV of each
 * key/value head are the sums over the G query heads that read it (the chain
 * rule through the shared input).  bf16 or fp16 with G > 1: the dK/dV pass runs per query
 * head and leaves fp32 partials in the workspace, and a group-sum pass adds them
 * (no atomics; deterministic).  q, o, dout, dq: [B,H,S,D]; k, v, dk, dv:
 * [B,H_kv,S,D]; lse: [B,H,S]; workspace: attn_bwd_gqa_workspace_bytes() bytes.
 * Small grids run the dQ and dK/dV passes on internal streams as attn_bwd does
 * (the group sum follows the join on `stream`).
 * attn_bwd is this call with H_kv = H.  Source: Forge RESEARCH.md §6 ("GQA").
 */
/*
 * Bytes of device workspace attn_bwd_gqa needs: B*H*S*4 (delta), plus, for bf16 or fp16
 * with H_kv < H, 2*B*H*S*D*4 (the per-query-head fp32 dK and dV), each region
 * rounded up to 256 bytes.  Returns 0 for an empty or invalid problem.
 */
size_t attn_bwd_gqa_workspace_bytes(int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D,
                                    attn_dtype dtype);

attn_status attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse,
                         void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes,
                         int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D,
                         float scale, int causal, attn_dtype dtype, void* stream);

/*
 * The backward's stages, exposed one by one (same argument rules as attn_bwd).
 * attn_bwd is exactly attn_bwd_dq_delta + attn_bwd_dkdv on one stream.
 * attn_bwd_preprocess + attn_bwd_dkdv + attn_bwd_dq computes the same gradients
 * with delta formed by a separate pass (its fp32 sums may differ in the last bits).
 *   delta : device, [B,H,S] fp32; written by attn_bwd_preprocess and
 *           attn_bwd_dq_delta, read by attn_bwd_dkdv and attn_bwd_dq.
 */
attn_status attn_bwd_preprocess(const void* o, const void* dout, float* delta,
                                int64_t B, int64_t H, int64_t S, int64_t D,
                                attn_dtype dtype, void* stream);

attn_status attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                          const float* lse, const float* delta, void* dk, void* dv,
                          int64_t B, int64_t H, int64_t S, int64_t D,
                          float scale, int causal, attn_dtype dtype, void* stream);

attn_status attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                        const float* lse, const float* delta, void* dq,
                        int64_t B, int64_t H, int64_t S, int64_t D,
                        float scale, int causal, attn_dtype dtype, void* stream);

/*
 * dQ pass that also forms delta = rowsum(dO o O) for every query row from o and
 * dout (fp32 sums of the stored values) and writes it to delta (fully
 * overwritten; must not overlap the other arguments).
 */
attn_status attn_bwd_dq_delta(const void* q, const void* k, const void* v, const void* o,
                              const void* dout, const float* lse, float* delta, void* dq,
                              int64_t B, int64_t H, int64_t S, int64_t D,
                              float scale, int causal, attn_dtype dtype, void* stream);

/*
 * Decode attention: one new query row per (batch entry, query head) against a
 * key/value cache.  The query is the newest position, appended after its own key
 * and value, so it sees every cached row of its sequence: plain attention of one
 * row over the first n rows of the cache (Forge RESEARCH.md §6, the decode path
 * of "forge generate": one query row, a strided walk of the cache with an online
 * softmax, split into chunks over a long cache and merged in a second pass).
 *   q        : device, [B,H,D] of dtype, read only.
 *   k_cache,
 *   v_cache  : device, [B,H_kv,L,D] of dtype, read only; query head h of batch
 *              entry b reads cache head h / (H / H_kv) of b (grouped heads).
 *   kv_lens  : device int32 [B], rows in use of each sequence's cache (values
 *              are clamped to [0, L]); NULL = every sequence uses all L rows.
 *              A sequence with 0 rows gives O = 0 and LSE = -inf.
 *   o        : device, [B,H,D] of dtype, fully overwritten.
 *   lse      : device, [B,H] fp32, natural-log log-sum-exp of the scaled scores.
 *   workspace: device, attn_decode_workspace_bytes() bytes (may be NULL when
 *              that is 0); holds the per-chunk partial results.
 * Supported set: as attn_fwd for D, dtype and scale; H_kv >= 1 dividing H; L >= 1.
 * Deterministic (no atomics).
 */
size_t attn_decode_workspace_bytes(int64_t B, int64_t H, int64_t H_kv, int64_t L, int64_t D,
                                   attn_dtype dtype);

attn_status attn_decode(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* kv_lens, void* o, float* lse,
                        void* workspace, size_t workspace_bytes,
                        int64_t B, int64_t H, int64_t H_kv, int64_t L, int64_t D,
                        float scale, attn_dtype dtype, void* stream);

/*
 * Shader-clock sample, for measurement: launches n workgroups (1 <= n <=
 * ATTN_CLOCK_SAMPLE_MAX) on `stream`; workgroup i writes out[4i .. 4i+3] =
 * {shader-cycle counter (s_memtime: advances at the current shader clock),
 * 100 MHz reference counter (s_memrealtime), id of the XCC it ran on, 0}.
 *   out : device, n*4 uint64, 16-byte aligned, fully overwritten.
 * Two samples around a timed region give each XCC's average shader clock over it:
 * (cycles after - before) / ((ticks after - before) / 100 MHz); a throughput is
 * then read against the peak at that clock.  Source: Iron "Kernel Engineering
 * Guide", §6.1 (a cold GPU runs at a lower DVFS clock state; warm it before the
 * first sample).  Errors: n out of range -> ATTN_ERR_SHAPE; out NULL ->
 * ATTN_ERR_NULL; misaligned -> ATTN_ERR_ALIGNMENT.
 */
#define ATTN_CLOCK_SAMPLE_MAX 4096
attn_status attn_clock_sample(uint64_t* out, int64_t n, void* stream);

/*
 * Static, NUL-terminated description of a status code (never NULL; an unknown
 * value gives "unknown attn_status").  The statuses are the up-front argument
 * checks: argument kinds and counts are verified before any work, as
 * TorchMetalKernel does at construction ("Cooperative tensors, reductions, and
 * building a fused attention kernel", §12), and an unsupported combination is
 * rejected loudly instead of being run wrong (Iron "Kernel Engineering Guide",
 * §2.5 on dispatch selectors).
 */
const char* attn_status_string(attn_status status);

#ifdef __cplusplus
}
#endif

#endif /* CAUSAL_ATTN_H */
