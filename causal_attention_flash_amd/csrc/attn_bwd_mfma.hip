// Backward pass, bf16 inputs, fp32 accumulation (gfx950, v_mfma_f32_32x32x16_bf16).
//
// Structure: the atomic-free three-stage backward of Forge RESEARCH.md §6 and the
// Forge paper ("Ecosystem survey"): a preprocess computes delta = rowsum(dO o O)
// once per query row (attn_preprocess.hip); a dK/dV pass runs parallel over key
// tiles and loops over query tiles; a dQ pass runs parallel over query tiles and
// loops over key tiles.  Both recompute P = exp(S - L) from the saved
// log-sum-exp, so the backward needs no online rescale (Forge paper, "Attention
// kernel design").  Transposed products are obtained by
// swapping operand roles rather than moving data (same section): the dK/dV pass
// forms S = Q K^T and dP = dO V^T with keys on the lanes, and the dQ pass forms
// S^T = K Q^T and dP^T = V dO^T with queries on the lanes.
//
// Per-element work on a score tile, with L2 = LSE*log2(e):
//   P  = exp2(s*scale*log2(e) - L2)           (0 where masked)
//   dS = P o (dP - delta)
// dV += P^T dO, dK += scale * dS^T Q           (dK/dV pass)
// dQ += scale * dS K                           (dQ pass)
//
// Register and LDS budget (the pages' central finding is that this backward is
// bound by register pressure): each wave keeps its own K and V (dK/dV pass) or
// Q and dO (dQ pass) as MFMA operands in registers, plus two fp32 accumulators
// of 32 rows x D; the streamed operand tiles are double-buffered in LDS,
// row-major only: the contractions over their rows read them through the
// transposing LDS read.  The dK/dV pass stages its Q and dO tiles through
// registers into padded rows; the dQ pass loads its K and V tiles straight from
// HBM into swizzled rows (attn_direct.h).
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "attn_launch.h"
#include "attn_direct.h"

namespace attn {


// ============================================================== dK / dV pass

// MODE: 0 = dK and dV (one pass), 1 = dV only, 2 = dK only.  The one-accumulator
// passes are the pages' remedy for the register pressure of this pass (Forge
// paper, "Finding 3: register pressure dominates attention backward": separate
// dK and dV kernels, each holding one accumulator and recomputing what it needs).
template <int D, int BMQ, int NW_, int MODE = 0>
struct DkdvCfg {
    static constexpr int NW = NW_;
    static constexpr int NT = NW * 64;
    static constexpr int BNK = NW * 32;  // keys per workgroup (32 per wave)
    using QT = RowTile<BMQ, D, NT>;      // Q and dO tiles, padded rows
    static constexpr int QE = QT::ELEMS;
    static constexpr int KSTR = D + 8;   // DQA: row stride of each wave's copy of its K rows
    static constexpr int BUF_ELEMS = 2 * QE;   // Q, dO
    static constexpr int BUF_STATS = 2 * BMQ;  // -LSE/scale, -delta (fp32)
    // register budget: 256 VGPRs (two waves per SIMD) up to D = 96, and for the
    // one-accumulator passes at D = 128
    static constexpr int WAVES_PER_SIMD = (D <= 96 || MODE != 0) ? 2 : 1;
    static constexpr int KS = HeadDim<D>::KSTEPS;
    static constexpr int DB = HeadDim<D>::DB;
};

// One workgroup per (query head, key block): the query head's Q/dO/LSE/delta
// against the keys of its key/value head.  With one query head per key/value
// head (PARTIAL = false) dK and dV are final and stored as bf16.  With grouped
// key/value heads (PARTIAL = true) each query head's contribution is stored as
// fp32 at its own [query head] slot of dKp/dVp, and the sum over the G query
// heads of a key/value head is formed by bwd_group_sum_kernel.
//
// DQA (one query head per key/value head): the pass also forms dQ, FlashAttention-2
// style, with fp32 atomic adds (Forge RESEARCH.md §6 names atomics as the legal,
// nondeterministic alternative to a separate dQ pass).  Per 32-query block each wave
// holds dS for its 32 keys; dQ^T = K^T dS^T needs dS with queries on the lanes, so
// dS goes through a per-wave LDS tile [keys][queries] and both operands come from
// transposing reads (K^T from a per-wave copy of the wave's K rows).  Each wave
// stores its fp32 partial for the block in its own LDS slot (the dS tile lives at
// the start of the slot: it has been read by the time the partial is stored);
// after a barrier every thread sums the slots of the waves that had work for the
// block and adds its share to the fp32 accumulator dQacc in HBM (global atomic
// adds, zero sums skipped); a second barrier frees the slots.  (Summing in one
// slot with LDS atomics instead measured ~9x slower: eight waves' ds_add_f32 on
// the same addresses serialise.)
// The LDS of one dK/dV workgroup: the double-buffered Q and dO tiles, their row
// statistics and (DQA) the per-wave K rows and dQ slots.
template <int D, int BMQ, int NW, int MODE, bool DQA>
struct DkdvSmem {
    using Cfg = DkdvCfg<D, BMQ, NW, MODE>;
    static constexpr int KSTR = Cfg::KSTR, DQS = D + 1;
    __attribute__((aligned(16))) uint16_t smem[2 * Cfg::BUF_ELEMS];
    __attribute__((aligned(16))) float sstat[2 * Cfg::BUF_STATS];
    __attribute__((aligned(16))) uint16_t kst[DQA ? NW * 32 * KSTR + 32 : 1];
    __attribute__((aligned(16))) float dqs[DQA ? NW * 32 * DQS : 1];
};

// One dK/dV workgroup: key block `bid` in heavy-first order over the BH heads.
// DFLY (one query head per key/value head): each query tile's delta = rowsum(dO o O)
// is formed here from the tile's dO rows and the matching O rows, instead of being
// read from Delta.
template <class E, int D, int BMQ, int NW, bool PARTIAL, bool DQA, int MODE, bool DFLY>
__device__ __forceinline__ void dkdv_block(
    DkdvSmem<D, BMQ, NW, MODE, DQA>& lds, int bid, const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, float* __restrict__ dKp, float* __restrict__ dVp, int S, int nblk, int BH, int H,
    int GQ, float c, float scale, int causal, float* __restrict__ dQacc) {
    using Cfg = DkdvCfg<D, BMQ, NW, MODE>;
    using V8 = typename E::V8;
    constexpr int NT = Cfg::NT, BNK = Cfg::BNK;
    constexpr bool WANT_DK = MODE != 1, WANT_DV = MODE != 2;
    static_assert(MODE == 0 || !DQA, "atomic dQ runs in the one-pass form");
    constexpr int KSTR = Cfg::KSTR;
    constexpr int KS = Cfg::KS, DB = Cfg::DB;
    static_assert(!(DQA && PARTIAL), "atomic dQ is for one query head per key/value head");
    static_assert(!DQA || (32 * D) % (NW * 64) == 0, "the flush splits a block's 32 x D sums evenly");
    // LDS: [Q, dO][2] tiles and their statistics; DQA: each wave's K rows [32][STR]
    // and dQ slot [32 queries][DQS] (the odd row stride spreads a column's rows over
    // the banks), its dS tile [32 keys][DSTR] at the start of the slot
    constexpr int DSTR = 40, DQS = D + 1;
    static_assert(32 * DSTR * 2 <= 32 * DQS * 4, "the dS tile fits in the slot");
    static_assert(!DFLY || (!PARTIAL && !DQA), "delta formed in place: one query head per key/value head");
    uint16_t* smem = lds.smem;
    float* sstat = lds.sstat;
    uint16_t* kst = lds.kst;
    float* dqs = lds.dqs;

    const WorkItem wi = heavy_first(bid, BH);
    const int head = wi.head;
    const int kblk = wi.rank;  // low key blocks see the most queries: first
    const int n0 = kblk * BNK;
    const size_t base = (size_t)head * S * D;
    const size_t kvbase = (size_t)kv_head_of(head, H, GQ) * S * D;
    const uint16_t* Qh = Q + base;
    const uint16_t* dOh = dO + base;
    const float* Lh = LSE + (size_t)head * S;
    const float* Dh = DFLY ? nullptr : Delta + (size_t)head * S;
    const uint16_t* Oh = DFLY ? O + base : nullptr;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, n = lane & 31;
    const int kw0 = n0 + wave * 32;
    const int key = kw0 + n;  // the key this lane's C columns belong to

    // K and V as B operands (keys on the lanes), d = 16ks+8h..+7.
    V8 kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (key < S) {
            a = ldg16(K + kvbase + (size_t)key * D + ks * 16 + 8 * h);
            if (WANT_DK) b = ldg16(V + kvbase + (size_t)key * D + ks * 16 + 8 * h);
        }
        kf[ks] = as_op<E>(a);
        vf[ks] = as_op<E>(b);
    }
    uint16_t* kst_w = kst + wave * 32 * KSTR;
    float* slot_w = dqs + wave * 32 * DQS;
    uint16_t* dst_w = reinterpret_cast<uint16_t*>(slot_w);
    if constexpr (DQA) {
        // the wave's K rows, for the transposing reads of K^T (zero past S)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            *reinterpret_cast<u32x4*>(kst_w + n * KSTR + ks * 16 + 8 * h) = __builtin_bit_cast(u32x4, kf[ks]);
    }

    f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dkacc[db][r] = 0.f;
            dvacc[db][r] = 0.f;
        }

    const float rscale = 1.f / scale;
    const int t0 = causal ? n0 / BMQ : 0;
    const int ntiles = (S + BMQ - 1) / BMQ;

    typename Cfg::QT qt, ot;
    using QT = typename Cfg::QT;
    const int rl = QT::row_lane(lane), tl = QT::tr_lane(lane);
    RowStats<BMQ, NT, !DFLY> st;
    // DFLY: the tile's O rows, chunk for chunk beside its dO rows; a row's chunks are
    // held by QT::CPR consecutive lanes
    typename Cfg::QT otv;
    static_assert(!DFLY || (QT::CPR <= 16 && (QT::CPR & (QT::CPR - 1)) == 0 && QT::CHUNKS % NT == 0 &&
                            NT % QT::CPR == 0 && QT::CPR == 2 * KS),
                  "a row's chunks fill an aligned group within a 16-lane DPP row, two per contraction step");
    auto bufp = [&](int b) { return smem + b * Cfg::BUF_ELEMS; };
    auto stat = [&](int b) { return sstat + b * Cfg::BUF_STATS; };
    auto stage = [&](int b) {
        uint16_t* s = bufp(b);
        qt.store(s, tid);
        ot.store(s + Cfg::QE, tid);
        st.store(stat(b), stat(b) + BMQ, rscale, tid);
        if constexpr (DFLY) {
            // delta of each row, stored negated, in the dQ pass's order (so the same
            // bits as attn_bwd_dq_delta): two chains of dot8 over the row's chunks of
            // one parity (chunks h, h+2, h+4, ... for h = 0, 1; the running sum moves
            // two lanes per step), then the sum of the two chains
#pragma unroll
            for (int i = 0; i < QT::PT; ++i) {
                const int ch = tid + i * NT, j = ch % QT::CPR;
                float p = 0.f;
#pragma unroll
                for (int step = 0; step < QT::CPR / 2; ++step) {
                    // the chain so far, from lane j - 2 (DPP row_shr:2)
                    const float prev = step == 0 ? 0.f
                                                 : __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                       0, __builtin_bit_cast(int, p), 0x112, 0xF, 0xF, false));
                    const float mine = dot8<E>(as_op<E>(ot.r[i]), as_op<E>(otv.r[i]), prev);
                    p = (j >> 1) == step ? mine : p;
                }
                const float other = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                        0, __builtin_bit_cast(int, p), 0xB1, 0xF, 0xF, false));  // lane ^ 1
                if (j == QT::CPR - 2) stat(b)[BMQ + ch / QT::CPR] = -(p + other);
            }
        }
    };
    auto fetch = [&](int t) {
        qt.load(Qh, t * BMQ, S, tid);
        ot.load(dOh, t * BMQ, S, tid);
        st.load(Lh, Dh, t * BMQ, S, tid);
        if constexpr (DFLY) otv.load(Oh, t * BMQ, S, tid);
    };

    if (t0 < ntiles) {
        fetch(t0);
        stage(0);
    }
    // The K and V operand loads have landed before the first prefetch is issued;
    // otherwise they would still be outstanding where the loop starts and the
    // wait for them there would cover every later prefetch as well.
    wait_vmem_all();
    if (t0 + 1 < ntiles) fetch(t0 + 1);
    __syncthreads();

    // One query tile against this wave's 32 keys; MASK instantiates the causal
    // mask for tiles that cross the diagonal (query rows past S need no mask:
    // their statistic is -inf, so P is exactly 0 there).
    //
    // The accumulators start from the per-row statistics instead of zero, so the
    // MFMAs deliver S - LSE/scale and dP - delta directly (register r of a lane
    // holds query row crow(r, h)); then P = exp2(c * acc) with c = scale*log2(e),
    // and dS = P * acc.
    //
    // DQA: every wave runs the per-block barrier and flush, `active` or not (a
    // wave is inactive for a tile entirely before its first key).
    auto tile = [&](auto mask_tag, int b, int qt0, bool active) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const uint16_t* Qs = bufp(b);
        const uint16_t* dOs = Qs + Cfg::QE;
        const float* SIs = stat(b);
        const float* PIs = SIs + BMQ;
#pragma unroll
        for (int qb = 0; qb < BMQ / 32; ++qb) {
          if (!DQA || active) {
            f32x16 sacc, pacc;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int rl = qb * 32 + 8 * g + 4 * h;
                const f32x4 si = *reinterpret_cast<const f32x4*>(SIs + rl);
                f32x4 pi = {0.f, 0.f, 0.f, 0.f};
                if constexpr (WANT_DK) pi = *reinterpret_cast<const f32x4*>(PIs + rl);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sacc[4 * g + i] = si[i];
                    pacc[4 * g + i] = pi[i];
                }
            }
            // 32 queries x this wave's 32 keys: S - LSE/scale and dP - delta
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                sacc = E::mma(QT::template row_op<E>(Qs, qb * 32, ks, rl), kf[ks], sacc);
                if constexpr (WANT_DK) pacc = E::mma(QT::template row_op<E>(dOs, qb * 32, ks, rl), vf[ks], pacc);
            }
            // P and dS
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = fast_exp2(sacc[r] * c);
                if constexpr (MASK) p = key > qt0 + qb * 32 + crow(r, h) ? 0.f : p;
                // DQA: a key slot at or past S (zero K and V rows) has s = 0, so P =
                // exp(-LSE) can overflow; its dS reaches dQ through K^T dS^T (0 * inf
                // would be NaN), so it is zeroed.  The split passes leave such values
                // in columns that are never stored.
                if constexpr (DQA) p = key < S ? p : 0.f;
                sacc[r] = p;
                if constexpr (WANT_DK) pacc[r] *= p;
            }
            // dV^T += dO^T P ; dK^T += Q^T dS  (contraction over these 32 queries;
            // dO^T and Q^T read transposed from the row-major tiles)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                V8 pb{}, sb{};
                if constexpr (WANT_DV) pb = pack_op<E>(sacc, c2);
                if constexpr (WANT_DK) sb = pack_op<E>(pacc, c2);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int r0 = (qb * 2 + c2) * 16;
                    if constexpr (WANT_DV) dvacc[db] = E::mma(QT::template tr_op<E>(dOs, r0, db, tl), pb, dvacc[db]);
                    if constexpr (WANT_DK) dkacc[db] = E::mma(QT::template tr_op<E>(Qs, r0, db, tl), sb, dkacc[db]);
                }
            }
            if constexpr (DQA) {
                // dS (rounded as for dK) into the wave's [key][query] tile: lane n
                // holds key n, queries crow(r, h) = 8g + 4h + 0..3 for r = 4g..4g+3
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 u;
                    u[0] = E::pack2(pacc[4 * g + 0], pacc[4 * g + 1]);
                    u[1] = E::pack2(pacc[4 * g + 2], pacc[4 * g + 3]);
                    *reinterpret_cast<u32x2*>(dst_w + n * DSTR + 8 * g + 4 * h) = u;
                }
                // dQ^T (d x 32 queries) = K^T dS^T over this wave's 32 keys
                f32x16 dqp[DB];
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) dqp[db][r] = 0.f;
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const V8 sb = lds_tr_op<E, DSTR>(dst_w, c2 * 16, 0, lane);
#pragma unroll
                    for (int db = 0; db < DB; ++db)
                        dqp[db] = E::mma(lds_tr_op<E, KSTR>(kst_w, c2 * 16, db * 32, lane), sb, dqp[db]);
                }
                // the wave's partial: lane n holds query n, d = 32db + crow(r, h)
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) slot_w[n * DQS + db * 32 + crow(r, h)] = dqp[db][r];
            }
          }
          if constexpr (DQA) {
              __syncthreads();  // every active wave's partial for the block is stored
              // waves with work for this tile: all, or (causal) those whose first
              // key is at most the tile's last query
              const int last = qt0 + BMQ - 1 - n0;
              const int nact = !causal ? NW : last < 0 ? 0 : min(NW, last / 32 + 1);
              const size_t qrow0 = (size_t)head * S + qt0 + qb * 32;
#pragma unroll
              for (int i = 0; i < 32 * D / NT; ++i) {
                  const int e = tid + i * NT, row = e / D, col = e % D;
                  float v = 0.f;
                  for (int w = 0; w < nact; ++w) v += dqs[w * 32 * DQS + row * DQS + col];
                  if (qt0 + qb * 32 + row < S && v != 0.f) unsafeAtomicAdd(dQacc + (qrow0 + row) * D + col, v);
              }
              __syncthreads();  // slots free for the next block
          }
        }
    };

    for (int t = t0; t < ntiles; ++t) {
        const int b = (t - t0) & 1;
        const int qt0 = t * BMQ;
        // wave-uniform: skip query tiles entirely before this wave's first key
        const bool active = !causal || qt0 + BMQ - 1 >= kw0;
        if (DQA || active) {
            if (causal && qt0 < kw0 + 31)
                tile(std::true_type{}, b, qt0, active);
            else
                tile(std::false_type{}, b, qt0, active);
        }
        if (t + 1 < ntiles) {
            stage(b ^ 1);
            if (t + 2 < ntiles) fetch(t + 2);
        }
        __syncthreads();
    }

    if constexpr (PARTIAL && D == 64) {
        // as below, for the fp32 partials of grouped key/value heads (rows of D = 64
        // fp32 values fit the swizzled layout; the other head dims store directly)
        constexpr int SCR = 2 * Cfg::BUF_ELEMS / NW / 8 * 8;
        uint16_t* w = smem + wave * SCR;
        if (WANT_DK) store_tile_rows_f32<D, SCR>(w, dkacc, scale, dKp + base, kw0, S, lane);
        if (WANT_DV) store_tile_rows_f32<D, SCR>(w, dvacc, 1.f, dVp + base, kw0, S, lane);
    } else if (PARTIAL && key < S) {
        float* dKr = dKp + base + (size_t)key * D;
        float* dVr = dVp + base + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (!HeadDim<D>::live(db, g)) continue;
                const int d = db * 32 + 8 * g + 4 * h;
                f32x4 fk, fv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    fk[i] = dkacc[db][4 * g + i] * scale;
                    fv[i] = dvacc[db][4 * g + i];
                }
                if (WANT_DK) *reinterpret_cast<f32x4*>(dKr + d) = fk;
                if (WANT_DV) *reinterpret_cast<f32x4*>(dVr + d) = fv;
            }
    }
    if constexpr (!PARTIAL) {
        // The loop's last barrier has passed, so the tile buffers are free: each wave
        // stores dK and dV through its own share of them, whole rows per store
        // instruction.  (With one workgroup per CU nothing hides this pass's stores:
        // 16 bytes of 32 rows per instruction measured 5% slower at B=4 H=16 S=2048
        // D=64, 1-4% at D = 80, 96, 128; the less so the longer a workgroup runs.)
        constexpr int SCR = 2 * Cfg::BUF_ELEMS / NW / 8 * 8;
        uint16_t* w = smem + wave * SCR;
        if (WANT_DK) store_tile_rows<E, D, SCR>(w, dkacc, scale, dK + kvbase, kw0, S, lane);
        if (WANT_DV) store_tile_rows<E, D, SCR>(w, dvacc, 1.f, dV + kvbase, kw0, S, lane);
    } else if (!PARTIAL && key < S) {
        uint16_t* dKr = dK + kvbase + (size_t)key * D;
        uint16_t* dVr = dV + kvbase + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (!HeadDim<D>::live(db, g)) continue;
                const int d = db * 32 + 8 * g + 4 * h;
                u32x2 uk, uv;
                uk[0] = E::pack2(dkacc[db][4 * g + 0] * scale, dkacc[db][4 * g + 1] * scale);
                uk[1] = E::pack2(dkacc[db][4 * g + 2] * scale, dkacc[db][4 * g + 3] * scale);
                uv[0] = E::pack2(dvacc[db][4 * g + 0], dvacc[db][4 * g + 1]);
                uv[1] = E::pack2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]);
                if (WANT_DK) *reinterpret_cast<u32x2*>(dKr + d) = uk;
                if (WANT_DV) *reinterpret_cast<u32x2*>(dVr + d) = uv;
            }
    }

}

template <class E, int D, int BMQ, int NW, bool PARTIAL, bool DQA = false, int MODE = 0>
__global__ __launch_bounds__(NW * 64, (DkdvCfg<D, BMQ, NW, MODE>::WAVES_PER_SIMD)) void bwd_dkdv_mfma_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, float* __restrict__ dKp, float* __restrict__ dVp, int S,
    int nblk, int BH, int H, int GQ, float c, float scale, int causal, float* __restrict__ dQacc = nullptr) {
    __shared__ DkdvSmem<D, BMQ, NW, MODE, DQA> lds;
    dkdv_block<E, D, BMQ, NW, PARTIAL, DQA, MODE, false>(lds, blockIdx.x, Q, K, V, nullptr, dO, LSE, Delta, dK, dV,
                                                         dKp, dVp, S, nblk, BH, H, GQ, c, scale, causal, dQacc);
}

template <class E, int D, int BMQ, int NW, int MODE = 0>
static hipError_t launch_dkdv(const LaunchArgs& a) {
    using Cfg = DkdvCfg<D, BMQ, NW, MODE>;
    const int nblk = (int)((a.S + Cfg::BNK - 1) / Cfg::BNK);
    const int64_t total = (int64_t)nblk * a.BH;
    if (total > INT32_MAX) return hipErrorInvalidValue;
    const int GQ = (int)(a.H / a.Hkv);
    if (GQ == 1)
        hipLaunchKernelGGL((bwd_dkdv_mfma_kernel<E, D, BMQ, NW, false, false, MODE>), dim3((unsigned)total), dim3(Cfg::NT), 0,
                           a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                           (const uint16_t*)a.dout, a.lse_in, a.delta_in, (uint16_t*)a.dk, (uint16_t*)a.dv,
                           nullptr, nullptr, (int)a.S, nblk, (int)a.BH, (int)a.H, 1, a.scale * kLog2e, a.scale,
                           a.causal);
    else
        hipLaunchKernelGGL((bwd_dkdv_mfma_kernel<E, D, BMQ, NW, true, false, MODE>), dim3((unsigned)total), dim3(Cfg::NT), 0,
                           a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                           (const uint16_t*)a.dout, a.lse_in, a.delta_in, nullptr, nullptr, a.dk_part, a.dv_part,
                           (int)a.S, nblk, (int)a.BH, (int)a.H, GQ, a.scale * kLog2e, a.scale, a.causal);
    return hipGetLastError();
}

// dK and dV in two one-accumulator passes (MODE 1 then 2) on the stream.  At
// D = 128 the one-pass form holds both 32 x 128 accumulators (329 registers with
// the AGPRs: one wave per SIMD); each one-accumulator pass fits 256 and runs two,
// with 64-query tiles and eight waves.  Measured 2.6-3.5% faster for the pair of
// passes on 8191-token and 2048-token heads; at D = 96 the extra pass over Q and
// dO costs more than the occupancy gains (33% slower).
template <class E, int D, int BMQ, int NW>
static hipError_t launch_dkdv_split(const LaunchArgs& a) {
    const hipError_t e = launch_dkdv<E, D, BMQ, NW, 1>(a);
    return e != hipSuccess ? e : launch_dkdv<E, D, BMQ, NW, 2>(a);
}

template <class E>
static hipError_t launch_dkdv_type(const LaunchArgs& a) {
    if (a.D == 64) return launch_dkdv<E, 64, 64, 8>(a);
    if (a.D == 80) return launch_dkdv<E, 80, 64, 8>(a);
    if (a.D == 96) return launch_dkdv<E, 96, 64, 8>(a);
    if (a.D == 128) return launch_dkdv_split<E, 128, 64, 8>(a);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_dkdv_bf16(const LaunchArgs& a) { return launch_dkdv_type<Bf16>(a); }
hipError_t launch_bwd_dkdv_f16(const LaunchArgs& a) { return launch_dkdv_type<F16>(a); }

// ---------------------------------------------------- atomic dQ (fused backward)

__global__ __launch_bounds__(256) void fill_zero_kernel(f32x4* __restrict__ p, int64_t n4) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// dQ = scale * dQacc, rounded to the element type; groups of 8 elements
template <class E>
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ acc, uint16_t* __restrict__ dq,
                                                         int64_t n8, float scale) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(acc + i * 8);
        const f32x4 b = *reinterpret_cast<const f32x4*>(acc + i * 8 + 4);
        u32x4 u;
        u[0] = E::pack2(a[0] * scale, a[1] * scale);
        u[1] = E::pack2(a[2] * scale, a[3] * scale);
        u[2] = E::pack2(b[0] * scale, b[1] * scale);
        u[3] = E::pack2(b[2] * scale, b[3] * scale);
        *reinterpret_cast<u32x4*>(dq + i * 8) = u;
    }
}

static unsigned stream_blocks(int64_t n) { return (unsigned)std::min<int64_t>((n + 255) / 256, 256 * 16); }

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
    const int64_t n4 = n / 4;  // n is a multiple of 4 (whole rows of D floats)
    if (n4 == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(stream_blocks(n4)), dim3(256), 0, stream, (f32x4*)p, n4);
    return hipGetLastError();
}

template <class E>
static hipError_t launch_dkdv_dqa(const LaunchArgs& a) {
    if (a.D != 64 || a.H != a.Hkv) return hipErrorInvalidValue;
    using Cfg = DkdvCfg<64, 64, 8>;
    const int nblk = (int)((a.S + Cfg::BNK - 1) / Cfg::BNK);
    const int64_t total = (int64_t)nblk * a.BH;
    if (total > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dkdv_mfma_kernel<E, 64, 64, 8, false, true>), dim3((unsigned)total), dim3(Cfg::NT), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse_in, a.delta_in, (uint16_t*)a.dk, (uint16_t*)a.dv, nullptr,
                       nullptr, (int)a.S, nblk, (int)a.BH, (int)a.H, 1, a.scale * kLog2e, a.scale, a.causal,
                       a.dq_acc);
    return hipGetLastError();
}

template <class E>
static hipError_t launch_dq_convert(const LaunchArgs& a) {
    const int64_t n8 = a.BH * a.S * a.D / 8;
    if (n8 == 0) return hipSuccess;
    hipLaunchKernelGGL((dq_convert_kernel<E>), dim3(stream_blocks(n8)), dim3(256), 0, a.stream, a.dq_acc,
                       (uint16_t*)a.dq, n8, a.scale);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv_dqa_bf16(const LaunchArgs& a) { return launch_dkdv_dqa<Bf16>(a); }
hipError_t launch_bwd_dkdv_dqa_f16(const LaunchArgs& a) { return launch_dkdv_dqa<F16>(a); }
hipError_t launch_dq_convert_bf16(const LaunchArgs& a) { return launch_dq_convert<Bf16>(a); }
hipError_t launch_dq_convert_f16(const LaunchArgs& a) { return launch_dq_convert<F16>(a); }

// ====================================================== grouped key/value heads
//
// dK[b, j] = sum over g < GQ of dKp[b, j*GQ + g] (likewise dV), fp32 sums of the
// per-query-head contributions, rounded once to the output type.  Grid-stride over groups
// of 8 elements of [batch, key/value head, S, D].
template <class E>
__global__ __launch_bounds__(256) void bwd_group_sum_kernel(const float* __restrict__ dKp,
                                                            const float* __restrict__ dVp,
                                                            uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                                                            int64_t n8, int64_t head_elems, int GQ) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = i * 8;                // element of the [B, H_kv, S, D] output
        const int64_t kvh = e / head_elems;     // batch x key/value head
        const int64_t off = e - kvh * head_elems;
        const int64_t src0 = kvh * GQ * head_elems + off;  // query head kvh*GQ of the same batch entry
        f32x4 k0 = {0.f, 0.f, 0.f, 0.f}, k1 = k0, v0 = k0, v1 = k0;
        for (int g = 0; g < GQ; ++g) {
            const int64_t src = src0 + (int64_t)g * head_elems;
            k0 += *reinterpret_cast<const f32x4*>(dKp + src);
            k1 += *reinterpret_cast<const f32x4*>(dKp + src + 4);
            v0 += *reinterpret_cast<const f32x4*>(dVp + src);
            v1 += *reinterpret_cast<const f32x4*>(dVp + src + 4);
        }
        u32x4 uk, uv;
        uk[0] = E::pack2(k0[0], k0[1]);
        uk[1] = E::pack2(k0[2], k0[3]);
        uk[2] = E::pack2(k1[0], k1[1]);
        uk[3] = E::pack2(k1[2], k1[3]);
        uv[0] = E::pack2(v0[0], v0[1]);
        uv[1] = E::pack2(v0[2], v0[3]);
        uv[2] = E::pack2(v1[0], v1[1]);
        uv[3] = E::pack2(v1[2], v1[3]);
        *reinterpret_cast<u32x4*>(dK + e) = uk;
        *reinterpret_cast<u32x4*>(dV + e) = uv;
    }
}

template <class E>
static hipError_t launch_group_sum(const LaunchArgs& a) {
    const int64_t head_elems = a.S * a.D;
    const int64_t n8 = a.BH / a.H * a.Hkv * head_elems / 8;
    const int64_t want = (n8 + 255) / 256;
    const unsigned grid = (unsigned)(want < 8192 ? (want > 0 ? want : 1) : 8192);
    hipLaunchKernelGGL(bwd_group_sum_kernel<E>, dim3(grid), dim3(256), 0, a.stream, a.dk_part, a.dv_part,
                       (uint16_t*)a.dk, (uint16_t*)a.dv, n8, head_elems, (int)(a.H / a.Hkv));
    return hipGetLastError();
}

hipError_t launch_group_sum_bf16(const LaunchArgs& a) { return launch_group_sum<Bf16>(a); }
hipError_t launch_group_sum_f16(const LaunchArgs& a) { return launch_group_sum<F16>(a); }

// ================================================================== dQ pass

template <int D, int BNK, int NW_>
struct DqCfg {
    static constexpr int NW = NW_;
    static constexpr int NT = NW * 64;
    static constexpr int BMQ = NW * 32;  // queries per workgroup (32 per wave)
    // K and V tiles, two buffers each, loaded straight from HBM into swizzled
    // rows one iteration ahead.  (Staging them through registers into padded
    // rows measured 3-4.5% slower at D = 64 with the conflict-free layouts of
    // both, and 5-7% slower at D = 128 earlier; fetching two tiles ahead was
    // slower at every size.)
    using Tile = DTile<BNK, D, NW>;
    static constexpr int TE = Tile::ELEMS;  // one tile in LDS
    // K[2], V[2]
    static constexpr int SMEM_ELEMS = 4 * TE;
    // register budget: 168 VGPRs (3 waves per SIMD) fits D = 64 without spills,
    // 256 (two) fits D = 80 and 96
    static constexpr int WAVES_PER_SIMD = D == 64 ? 3 : (D <= 96 ? 2 : 1);
    static constexpr int KS = HeadDim<D>::KSTEPS;
    static constexpr int DB = HeadDim<D>::DB;
};

// One dQ workgroup: query block `bid` in heavy-first order over the BH heads, its
// K/V tiles in `smem` (Cfg::SMEM_ELEMS elements).  DELTA_FROM_O: delta =
// rowsum(dO o O) is formed here, from the O rows of this wave's queries (fp32 sums
// of bf16 products), and written to DeltaOut for the dK/dV pass; otherwise delta is
// read from Delta.
template <class E, int D, int BNK, int NW, bool DELTA_FROM_O>
__device__ __forceinline__ void dq_block(
    uint16_t* smem, int bid, const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta, float* __restrict__ DeltaOut,
    uint16_t* __restrict__ dQ, int S, int nblk, int BH, int H, int GQ, float c, float scale, int causal) {
    using Cfg = DqCfg<D, BNK, NW>;
    using V8 = typename E::V8;
    constexpr int BMQ = Cfg::BMQ;
    constexpr int KS = Cfg::KS, DB = Cfg::DB;
    constexpr int TE = Cfg::TE;

    const WorkItem wi = heavy_first(bid, BH);
    const int head = wi.head;
    const int qblk = nblk - 1 - wi.rank;  // high query blocks see the most keys: first
    const int q0 = qblk * BMQ;
    const size_t base = (size_t)head * S * D;
    const size_t kvbase = (size_t)kv_head_of(head, H, GQ) * S * D;
    const uint16_t* Kh = K + kvbase;
    const uint16_t* Vh = V + kvbase;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, n = lane & 31;
    const int qw0 = q0 + wave * 32;
    const int q = qw0 + n;  // the query this lane's C columns belong to

    const int kend = causal ? min(S, q0 + BMQ) : S;
    const int ntiles = (kend + BNK - 1) / BNK;

    // Tile t uses buffer t % 2.  Iteration t issues tile t + 1 into the buffers of
    // tile t - 1 (read in the previous iteration, free once the iteration's
    // barrier has passed), and waits for all of its own loads before that
    // barrier.  Tiles at or past ntiles load from row S (an empty buffer range) so
    // every path issues the same loads.
    auto kbuf = [&](int t) { return smem + (t & 1) * TE; };
    auto vbuf = [&](int t) { return smem + (2 + (t & 1)) * TE; };
    typename Cfg::Tile::Src src;
    DOffsets<typename Cfg::Tile, D> lo;
    lo.init(lane);
    auto load_t = [&](int t) {
        const int row = t < ntiles ? t * BNK : S;
        Cfg::Tile::load(Kh, row, S, kbuf(t), src, wave);
        Cfg::Tile::load(Vh, row, S, vbuf(t), src, wave);
    };
    src.init(wave, lane);
    load_t(0);

    V8 qf[KS], of[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (q < S) {
            a = ldg16(Q + base + (size_t)q * D + ks * 16 + 8 * h);
            b = ldg16(dO + base + (size_t)q * D + ks * 16 + 8 * h);
        }
        qf[ks] = as_op<E>(a);
        of[ks] = as_op<E>(b);
    }
    const float l2 = q < S ? LSE[(size_t)head * S + q] * kLog2e : INFINITY;
    float dl;
    if constexpr (DELTA_FROM_O) {
        // this lane holds half of the row (d = 16ks + 8h .. +7); its partner
        // lane l ^ 32 holds the other half
        float part = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 u = {0u, 0u, 0u, 0u};
            if (q < S) u = ldg16(O + base + (size_t)q * D + ks * 16 + 8 * h);
            part = dot8<E>(of[ks], as_op<E>(u), part);
        }
        dl = half_sum(part);
        if (h == 0 && q < S) DeltaOut[(size_t)head * S + q] = dl;
    } else {
        dl = q < S ? Delta[(size_t)head * S + q] : 0.f;
    }

    f32x16 dqacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;

    // One key tile against this wave's 32 queries; MASK instantiates the causal
    // and sequence-end mask for tiles that cross the diagonal or the end.
    auto tile = [&](auto mask_tag, int t, int k0) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const uint16_t* Ks = kbuf(t);
        const uint16_t* Vs = vbuf(t);
#pragma unroll
        for (int kb = 0; kb < BNK / 32; ++kb) {
            // S^T = K Q^T and dP^T = V dO^T: 32 keys x this wave's 32 queries
            f32x16 sacc, pacc;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sacc[r] = 0.f;
                pacc[r] = 0.f;
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                sacc = E::mma(lo.template row_op<E>(Ks, kb * 32, ks), qf[ks], sacc);
                pacc = E::mma(lo.template row_op<E>(Vs, kb * 32, ks), of[ks], pacc);
            }
            // K^T operands of this block's dQ product, read transposed from the K
            // tile (asynchronous: used after lds_wait)
            i16x4 kr[2][DB][2];
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                for (int db = 0; db < DB; ++db) lo.tr_async(Ks, (kb * 2 + c2) * 16, db, kr[c2][db]);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = fast_exp2(fmaf(sacc[r], c, -l2));
                if constexpr (MASK) {
                    const int kk = k0 + kb * 32 + crow(r, h);
                    p = ((causal && kk > q) || kk >= S) ? 0.f : p;
                }
                pacc[r] = p * (pacc[r] - dl);
            }
            // dQ^T += K^T dS^T (contraction over these 32 keys)
            lds_wait(reinterpret_cast<i16x4 (&)[2 * DB * 2]>(kr));
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const V8 sb = pack_op<E>(pacc, c2);
#pragma unroll
                for (int db = 0; db < DB; ++db) dqacc[db] = E::mma(tr_join<E>(kr[c2][db]), sb, dqacc[db]);
            }
        }
    };

    for (int t = 0; t < ntiles; ++t) {
        wait_vmcnt<0>();  // own loads of tile t
        bare_barrier();   // everyone's; tile t - 1 no longer read
        load_t(t + 1);
        const int k0 = t * BNK;
        // wave-uniform: skip key tiles entirely after this wave's last query
        if (!causal || k0 <= qw0 + 31) {
            if ((causal && k0 + BNK - 1 > qw0) || k0 + BNK > S)
                tile(std::true_type{}, t, k0);
            else
                tile(std::false_type{}, t, k0);
        }
    }
    wait_vmcnt<0>();  // no load into LDS outlives the workgroup

    if (q < S) {
        uint16_t* dQr = dQ + base + (size_t)q * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (!HeadDim<D>::live(db, g)) continue;
                u32x2 u;
                u[0] = E::pack2(dqacc[db][4 * g + 0] * scale, dqacc[db][4 * g + 1] * scale);
                u[1] = E::pack2(dqacc[db][4 * g + 2] * scale, dqacc[db][4 * g + 3] * scale);
                *reinterpret_cast<u32x2*>(dQr + db * 32 + 8 * g + 4 * h) = u;
            }
    }

}

template <class E, int D, int BNK, int NW, bool DELTA_FROM_O>
__global__ __launch_bounds__(NW * 64, (DqCfg<D, BNK, NW>::WAVES_PER_SIMD)) void bwd_dq_mfma_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
    const float* __restrict__ Delta, float* __restrict__ DeltaOut, uint16_t* __restrict__ dQ, int S, int nblk,
    int BH, int H, int GQ, float c, float scale, int causal) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[DqCfg<D, BNK, NW>::SMEM_ELEMS];
    dq_block<E, D, BNK, NW, DELTA_FROM_O>(smem, blockIdx.x, Q, K, V, O, dO, LSE, Delta, DeltaOut, dQ, S, nblk, BH, H,
                                          GQ, c, scale, causal);
}

template <class E, int D, int BNK, int NW, bool DELTA_FROM_O>
static hipError_t launch_dq(const LaunchArgs& a) {
    using Cfg = DqCfg<D, BNK, NW>;
    const int nblk = (int)((a.S + Cfg::BMQ - 1) / Cfg::BMQ);
    const int64_t total = (int64_t)nblk * a.BH;
    if (total > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dq_mfma_kernel<E, D, BNK, NW, DELTA_FROM_O>), dim3((unsigned)total), dim3(Cfg::NT), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.o_in, (const uint16_t*)a.dout, a.lse_in, a.delta_in, a.delta,
                       (uint16_t*)a.dq, (int)a.S, nblk, (int)a.BH, (int)a.H, (int)(a.H / a.Hkv), a.scale * kLog2e,
                       a.scale, a.causal);
    return hipGetLastError();
}

template <class E, bool DELTA_FROM_O>
static hipError_t launch_dq_type(const LaunchArgs& a) {
    if (a.D == 64) return launch_dq<E, 64, 64, 4, DELTA_FROM_O>(a);
    if (a.D == 80) return launch_dq<E, 80, 64, 4, DELTA_FROM_O>(a);
    if (a.D == 96) return launch_dq<E, 96, 64, 4, DELTA_FROM_O>(a);
    if (a.D == 128) return launch_dq<E, 128, 32, 4, DELTA_FROM_O>(a);
    return hipErrorInvalidValue;
}

// delta = rowsum(dO o O) for every query row, in exactly the dQ pass's order (lane n
// of a wave holds row n; lane half h sums chunks d = 16ks + 8h .. +7 in ks order with
// dot8, then the two halves are added), so that passes reading it produce the same
// bits as the dQ pass that forms delta itself.  128 rows per 256-thread block.
template <class E, int D>
__global__ __launch_bounds__(256) void delta_dq_order_kernel(const uint16_t* __restrict__ O,
                                                             const uint16_t* __restrict__ dO,
                                                             float* __restrict__ delta, int64_t rows) {
    constexpr int KS = HeadDim<D>::KSTEPS;
    const int lane = threadIdx.x & 63, h = lane >> 5;
    const int64_t row = (int64_t)blockIdx.x * 128 + (threadIdx.x >> 6) * 32 + (lane & 31);
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (row < rows) {
            a = ldg16(dO + row * D + ks * 16 + 8 * h);
            b = ldg16(O + row * D + ks * 16 + 8 * h);
        }
        part = dot8<E>(as_op<E>(a), as_op<E>(b), part);
    }
    const float dl = half_sum(part);
    if (h == 0 && row < rows) delta[row] = dl;
}

// Side streams of the concurrent small-grid backward (below), per device: created on
// first use with the default priority, never destroyed; one mutex orders the
// fork-join sequences of calls from several host threads.
namespace {
constexpr int kMaxDevices = 64;
struct SideStreams {
    hipStream_t st[2] = {nullptr, nullptr};
    hipEvent_t fork = nullptr;
    hipEvent_t join[2] = {nullptr, nullptr};
};
std::mutex g_side_mu;
SideStreams g_side[kMaxDevices];

hipError_t side_streams(SideStreams*& out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    SideStreams& sd = g_side[dev];
    if (sd.fork == nullptr) {
        for (int i = 0; i < 2; ++i) {
            if ((e = hipStreamCreateWithFlags(&sd.st[i], hipStreamNonBlocking)) != hipSuccess) return e;
            if ((e = hipEventCreateWithFlags(&sd.join[i], hipEventDisableTiming)) != hipSuccess) return e;
        }
        if ((e = hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming)) != hipSuccess) return e;
    }
    out = &sd;
    return hipSuccess;
}
}  // namespace

// The backward of a grid whose dQ pass and dK/dV pass(es) each fit in one round of the
// device (each alone would leave much of it idle): delta in the dQ pass's order on
// the caller's stream, then the dQ pass there and the dK/dV pass (at D = 128 its dV
// and dK passes, each on a side stream of its own) beside it, joined back into the
// caller's stream.  Same kernels and inputs as the serial passes: the same bits.
// With grouped key/value heads the dK/dV passes leave per-query-head partials, which
// the group sum enqueued after the join adds.
template <class E>
static hipError_t launch_bwd_concurrent(const LaunchArgs& a) {
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStreams* sd = nullptr;
    hipError_t e = side_streams(sd);
    if (e != hipSuccess) return e;
    const int64_t rows = a.BH * a.S;
    const unsigned grid = (unsigned)((rows + 127) / 128);
    const uint16_t* O = (const uint16_t*)a.o_in;
    const uint16_t* dO = (const uint16_t*)a.dout;
    if (a.D == 64) hipLaunchKernelGGL((delta_dq_order_kernel<E, 64>), dim3(grid), dim3(256), 0, a.stream, O, dO, a.delta, rows);
    else if (a.D == 80) hipLaunchKernelGGL((delta_dq_order_kernel<E, 80>), dim3(grid), dim3(256), 0, a.stream, O, dO, a.delta, rows);
    else if (a.D == 96) hipLaunchKernelGGL((delta_dq_order_kernel<E, 96>), dim3(grid), dim3(256), 0, a.stream, O, dO, a.delta, rows);
    else hipLaunchKernelGGL((delta_dq_order_kernel<E, 128>), dim3(grid), dim3(256), 0, a.stream, O, dO, a.delta, rows);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    LaunchArgs b = a;
    b.delta_in = a.delta;
    const int nside = a.D == 128 ? 2 : 1;
    if ((e = hipEventRecord(sd->fork, a.stream)) != hipSuccess) return e;
    for (int i = 0; i < nside; ++i)
        if ((e = hipStreamWaitEvent(sd->st[i], sd->fork, 0)) != hipSuccess) return e;
    if ((e = launch_dq_type<E, false>(b)) != hipSuccess) return e;
    LaunchArgs c = b;
    c.stream = sd->st[0];
    if (a.D == 128) {
        if ((e = launch_dkdv<E, 128, 64, 8, 1>(c)) != hipSuccess) return e;
        c.stream = sd->st[1];
        if ((e = launch_dkdv<E, 128, 64, 8, 2>(c)) != hipSuccess) return e;
    } else if ((e = launch_dkdv_type<E>(c)) != hipSuccess) {
        return e;
    }
    for (int i = 0; i < nside; ++i) {
        if ((e = hipEventRecord(sd->join[i], sd->st[i])) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(a.stream, sd->join[i], 0)) != hipSuccess) return e;
    }
    return hipSuccess;
}

// The whole backward of a small grid in one launch (D = 64, one query head per
// key/value head): blocks below ndq are dQ blocks (128 queries, storing delta), the
// rest four-wave dK/dV blocks of 128 keys that form each query tile's delta
// themselves (dkdv_block's DFLY), so the two kinds run side by side instead of one
// pass after the other, each of which would leave much of the device idle or end in
// a tail.
template <class E>
__global__ __launch_bounds__(256, 2) void bwd_small_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
    float* __restrict__ DeltaOut, uint16_t* __restrict__ dQ, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    int S, int nblk_q, int nblk_k, int ndq, int BH, int H, float c, float scale, int causal) {
    using DQ = DqCfg<64, 64, 4>;
    __shared__ union {
        __attribute__((aligned(16))) uint16_t dq[DQ::SMEM_ELEMS];
        DkdvSmem<64, 64, 4, 0, false> kv;
    } lds;
    if ((int)blockIdx.x < ndq)
        dq_block<E, 64, 64, 4, true>(lds.dq, blockIdx.x, Q, K, V, O, dO, LSE, nullptr, DeltaOut, dQ, S, nblk_q, BH, H,
                                     1, c, scale, causal);
    else
        dkdv_block<E, 64, 64, 4, false, false, 0, true>(lds.kv, (int)blockIdx.x - ndq, Q, K, V, O, dO, LSE, nullptr,
                                                        dK, dV, nullptr, nullptr, S, nblk_k, BH, H, 1, c, scale,
                                                        causal, nullptr);
}

// attn_bwd's passes for 16-bit inputs: the one-launch form where it applies (D = 64,
// one query head per key/value head, and the two kinds of blocks, two per CU, within
// three rounds of the device), else the dQ pass (forming delta) and then the dK/dV
// pass.  Measured: B=8 H=6 S=256 (one round) 0.0303 -> 0.0186 ms per step, B=8 H=12
// S=1024 (three rounds) 2% faster, B=4 H=16 S=2048 (four rounds) 3.4% slower.
template <class E>
static hipError_t launch_bwd_type(const LaunchArgs& a) {
    const int64_t nq = (a.S + 127) / 128;  // 128-query dQ blocks and 128-key dK/dV blocks
    if (a.D == 64 && a.H == a.Hkv && 2 * nq * a.BH <= 6 * (int64_t)cu_count()) {
        const int ndq = (int)(nq * a.BH);
        hipLaunchKernelGGL((bwd_small_kernel<E>), dim3(2 * ndq), dim3(256), 0, a.stream, (const uint16_t*)a.q,
                           (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.o_in,
                           (const uint16_t*)a.dout, a.lse_in, a.delta, (uint16_t*)a.dq, (uint16_t*)a.dk,
                           (uint16_t*)a.dv, (int)a.S, (int)nq, (int)nq, ndq, (int)a.BH, (int)a.H, a.scale * kLog2e,
                           a.scale, a.causal);
        return hipGetLastError();
    }
    if (a.side_streams) {
        // dQ and dK/dV passes side by side where each fits in one round by itself
        // (the D = 64 grids up to three rounds run as one launch above) and, below
        // D = 128, the sequences are long enough for the overlap to outweigh the
        // delta pass and the stream joins; not while the caller's stream is being
        // captured into a graph.  Backward, measured: D = 128 B=1 H=4 S=8191 724.5 ->
        // 371.6 us, B=1 H=8 S=4096 373.9 -> 209.2, B=1 H=16 S=2048 198.5 -> 123.1,
        // B=1 H=16 S=1024 107.5 -> 73.1; D = 96 B=1 H=12 S=2048 124.1 -> 105.4, D = 80
        // B=1 H=16 S=2048 115.2 -> 102.2; but D = 80 B=4 H=8 S=1024 +3.8%, D = 96 B=2
        // H=12 S=1024 +1.3%.
        const int dq_waves = a.D == 64 ? 3 : 2;  // occupancy of the 4-wave dQ blocks
        const int64_t dq_blocks = (a.S + 127) / 128 * a.BH, dkdv_blocks = (a.S + 255) / 256 * a.BH;
        if (dq_blocks <= (int64_t)cu_count() * dq_waves && dkdv_blocks <= cu_count() &&
            (a.D == 128 || a.S >= 2048)) {
            hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
            const hipError_t ce = hipStreamIsCapturing(a.stream, &cap);
            if (ce != hipSuccess) return ce;
            if (cap == hipStreamCaptureStatusNone) return launch_bwd_concurrent<E>(a);
        }
    }
    const hipError_t e = launch_dq_type<E, true>(a);
    return e != hipSuccess ? e : launch_dkdv_type<E>(a);
}

hipError_t launch_bwd_bf16(const LaunchArgs& a) { return launch_bwd_type<Bf16>(a); }
hipError_t launch_bwd_f16(const LaunchArgs& a) { return launch_bwd_type<F16>(a); }

hipError_t launch_bwd_dq_bf16(const LaunchArgs& a) { return launch_dq_type<Bf16, false>(a); }
hipError_t launch_bwd_dq_delta_bf16(const LaunchArgs& a) { return launch_dq_type<Bf16, true>(a); }
hipError_t launch_bwd_dq_f16(const LaunchArgs& a) { return launch_dq_type<F16, false>(a); }
hipError_t launch_bwd_dq_delta_f16(const LaunchArgs& a) { return launch_dq_type<F16, true>(a); }

}  // namespace attn
