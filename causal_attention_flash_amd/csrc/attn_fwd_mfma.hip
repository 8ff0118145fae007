// Forward pass, bf16 inputs, fp32 accumulation: O and LSE for one tile of queries
// per workgroup (gfx950, v_mfma_f32_32x32x16_bf16).
//
// Method: the FlashAttention-2 online softmax of Forge RESEARCH.md §6 ("Fused
// attention design"): per key tile, m_new = max(m, rowmax S), P = exp2(S - m_new)
// with scale*log2(e) folded into the exponent, l = l*factor + rowsum P,
// O = O*factor + P V, divide by l once after the loop, save L = m + log l.
// Causal tiles entirely above the diagonal are skipped and only tiles that cross
// the diagonal (or the sequence end) pay per-element masking (same section,
// "Causal masking"); masked scores are excluded with a mask that can never make
// exp produce NaN (the -inf - -inf hazard named there and in §6.3 of
// "Cooperative tensors, reductions, and building a fused attention kernel").
//
// gfx950 mapping:
// * NW waves per workgroup, split-Q: each wave owns QB blocks of 32 query rows
//   and never shares row statistics with another wave.  Small grids instead
//   split each query block's keys between two waves (FwdCfg::SPLIT): each
//   takes one 32-key half of every staged 64-key tile, with its own reference
//   point, and the two partial (m, l, O) are merged through LDS after the loop,
//   as the online softmax merges any two key ranges.
// * The score tile is computed transposed, S^T = K Q^T, so each lane owns one
//   query (C column) and the row max / row sum are per-lane reductions (the sum
//   on the matrix cores, see FwdCfg::MFMA_ROW_SUM) plus one exchange between the
//   two lane halves (v_permlane32_swap).
// * P^T, packed to bf16 straight from the C registers, is the B operand of
//   O^T += V^T P^T; V stays row-major in LDS and its transposed operand comes
//   from ds_read_b64_tr_b16, in the key order of the C registers.  The rescale
//   O *= factor is a per-lane multiply (no diag-matrix product).
// * The row max is not formed per tile.  P = exp2(s*c - m) is computed against
//   the row's reference point m, and m moves (to the row max, with O and l
//   rescaled and P formed again) only when some lane's sum of its P values
//   exceeds kPBound, i.e. when some P could: always on a row's first tile (m
//   starts at -FLT_MAX), after that only when scores grow past m by log2 of the
//   bound (64 for bf16 P, 15 for fp16).  fp32 accumulation and the P types
//   absorb values up to the bound; the result is the same function, only the
//   reference point of the exponent differs.
// * Software pipeline: K runs one tile ahead of V in LDS, so iteration t issues
//   the MFMAs of S^T for tile t+1 next to the exp/sum VALU work of tile t
//   (the MFMA unit works asynchronously from the VALU), then O += V_t P_t.
//   Q stays in registers for the whole loop; K/V tiles go from HBM straight to
//   LDS (buffer loads with the lds flag, swizzled rows) one tile ahead of their
//   use; one barrier per tile.
#include <type_traits>

#include "attn_launch.h"
#include "attn_direct.h"

namespace attn {


// Largest P value the loop lets through without moving the reference point:
// bf16 P (and fp32 O and l accumulation) holds 2^64 with room to spare for any
// sum over a row; fp16 P tops out at 65504.
template <class E>
constexpr float kPBound = std::is_same<E, F16>::value ? 0x1p15f : 0x1p64f;

// The S^T = K Q^T product: 16-bit Q and K of the element type E, or fp8 (E4M3)
// Q and K.  Op is the MFMA operand, STEPS the MFMAs per 32x32 score block, KD the
// 16-bit slots per K row in LDS (an fp8 row of D bytes is D/2 slots).
template <class E, int D, bool QK8>
struct QkOps {
    using Op = typename E::V8;
    static constexpr int STEPS = HeadDim<D>::KSTEPS;
    static constexpr int KD = D;
    static __device__ __forceinline__ f32x16 mma(const Op& a, const Op& b, const f32x16& c) { return E::mma(a, b, c); }
};
template <class E, int D>
struct QkOps<E, D, true> {
    using Op = Fp8E4M3::Op;
    static constexpr int STEPS = D / 64;
    static constexpr int KD = D / 2;
    static __device__ __forceinline__ f32x16 mma(const Op& a, const Op& b, const f32x16& c) {
        return Fp8E4M3::mma(a, b, c);
    }
};

// BN keys per tile: 32.  A 64-key tile's registers (the next tile's K operands,
// the V^T operands, two score sets) pass 256 VGPRs at D = 80, 96 and 128 and
// leave one wave per SIMD; 32-key tiles fit two there (measured 10-25% faster)
// and three at D = 64 (147 VGPRs; 2.5% faster than 64-key tiles at two).
template <int D, int QB, int NW_, bool QK8 = false, int BN_ = 32, bool SPLIT_ = false>
struct FwdCfg {
    static constexpr int NW = NW_;
    static constexpr int NT = NW * 64;
    // SPLIT: the waves form two key groups: wave w takes the query block w % (NW/2)
    // and, of each staged key tile, the 32-key half w / (NW/2), so a query block's
    // keys are shared by two waves whose partial (m, l, O) are merged at the end
    static constexpr bool SPLIT = SPLIT_;
    static constexpr int QW = SPLIT ? NW / 2 : NW;  // query blocks per workgroup
    static constexpr int BM = QW * 32 * QB;  // queries per workgroup
    static constexpr int BN = BN_;           // keys per staged tile
    static constexpr int KBW = SPLIT ? 1 : BN / 32;  // 32-key blocks a wave multiplies per tile
    // waves per SIMD the register budget is set for
    static constexpr int WAVES_PER_SIMD = D == 64 && BN == 32 ? 3 : 2;
    using Tile = DTile<BN, D, NW>;           // V tile
    static constexpr int TE = Tile::ELEMS;   // one V tile in LDS (elements)
    using KTile = DTile<BN, QK8 ? D / 2 : D, NW>;  // K tile (fp8 rows: D bytes)
    static constexpr int TK = KTile::ELEMS;
    // LDS buffers per operand: a tile is fetched during the iteration before its
    // use (fetching two or three ahead measured slower)
    static constexpr int NB = 2;
    static constexpr int P = NB - 1;
    static constexpr int KS = HeadDim<D>::KSTEPS;
    static constexpr int DB = HeadDim<D>::DB;
    // Paired query blocks (see the kernel): from D = 80 up two workgroups fill a
    // CU, and half as many workgroups, each with the same work, fill it evenly
    // (measured 2-5% faster where the pairs still cover every slot).  Where three
    // workgroups fill a CU (D = 64) pairs leave a third of it idle: 5% slower there.
    static constexpr bool PAIRABLE = D >= 80 && !QK8 && !SPLIT_;
    // Per-lane row sums of each tile's P on the matrix cores (two 16x16x32 products
    // against a selector, lane_sum_selector) instead of eight v_dot2, which hold the
    // MFMA pipe while they run: bitwise the same sums, 0.5-2% faster at D = 64; at
    // D = 128 (16-bit Q and K) the selector's registers would spill.
    static constexpr bool MFMA_ROW_SUM = D <= 96 || QK8;
    // the loop masks only a wave's last key tile: a wave's 32 * QB queries must
    // not reach into an earlier tile (else that tile also crosses the diagonal)
    static_assert(32 * QB <= BN, "a wave's queries must fit in one key tile");
    static_assert(!SPLIT || (BN == 64 && QB == 1 && NW % 2 == 0 && !QK8), "split tiles: two 32-key halves");
};

// QK8: Q and K hold fp8 (E4M3) bytes and c carries their dequantisation factors.
template <class E, int D, int QB, int NW, bool QK8, int BN_, bool SPLIT>
__global__ __launch_bounds__(NW * 64, (FwdCfg<D, QB, NW, QK8, BN_, SPLIT>::WAVES_PER_SIMD)) void fwd_mfma_kernel(const void* __restrict__ Q,
                                                       const void* __restrict__ K,
                                                       const uint16_t* __restrict__ V,
                                                       uint16_t* __restrict__ O, float* __restrict__ LSE,
                                                       int S, int nblk, int BH, int H, int GQ, float c,
                                                       int causal, int paired) {
    using Cfg = FwdCfg<D, QB, NW, QK8, BN_, SPLIT>;
    using V8 = typename E::V8;
    using QK = QkOps<E, D, QK8>;
    using QOp = typename QK::Op;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, TE = Cfg::TE, TK = Cfg::TK, NB = Cfg::NB, P = Cfg::P;
    // loads per wave of one K tile plus one V tile
    constexpr int LOADS2 = Cfg::KTile::LOADS + Cfg::Tile::LOADS;
    constexpr int KB = Cfg::KBW;  // 32-key blocks this wave multiplies per tile
    constexpr int QS = QK::STEPS, DB = Cfg::DB;
    // K[NB], V[NB]
    __shared__ __attribute__((aligned(16))) uint16_t smem[NB * (TK + TE)];

    // Work: one query block per workgroup, heaviest first (heavy_first), or, with
    // `paired` (Cfg::PAIRABLE configurations only), a pair of query blocks j and
    // nblk-1-j per workgroup, one after the other: in a causal head every pair
    // holds the same number of key tiles, so the workgroups finish together
    // instead of the heaviest blocks running on alone at the end of the grid.
    const WorkItem wi = heavy_first(blockIdx.x, BH);
    const int head = wi.head, rank = wi.rank;
    const int nparts = Cfg::PAIRABLE && paired && nblk - 1 - rank != rank ? 2 : 1;
    // causal blocks differ in work: the heavy ones get the SIMDs first (measured
    // 1.3% faster at B=4 H=16 S=2048 D=64, 0.6% at one 8191-token D = 128 head;
    // the same in the dQ pass gained nothing)
    if (causal && !paired) weight_priority(rank, nblk);
    for (int part = 0; part < nparts; ++part) {
        if (part > 0) __syncthreads();  // every wave is done with the LDS of the first block
        const int qblk = part == 0 ? nblk - 1 - rank : rank;  // most work first
        const int q0 = qblk * BM;
        const size_t base = (size_t)head * S * D;
        const size_t kvbase = (size_t)kv_head_of(head, H, GQ) * S * D;
        // Q and K rows as 16-bit slots (QK::KD per row; fp8 rows of D bytes are D / 2)
        const uint16_t* Qh = (const uint16_t*)Q + (QK8 ? base / 2 : base);
        const uint16_t* Kh = (const uint16_t*)K + (QK8 ? kvbase / 2 : kvbase);
        const uint16_t* Vh = V + kvbase;

        const int tid = threadIdx.x;
        const int lane = tid & 63, wave = tid >> 6;
        const int h = lane >> 5, n = lane & 31;
        const int qg = Cfg::SPLIT ? wave % Cfg::QW : wave;  // query block of the workgroup
        const int koff = Cfg::SPLIT ? 32 * (wave / Cfg::QW) : 0;  // this wave's rows of a tile
        const int qw0 = q0 + qg * 32 * QB;

        const int kend = causal ? min(S, q0 + BM) : S;
        const int ntiles = (kend + BN - 1) / BN;  // tiles the workgroup stages
        // tiles this wave multiplies: the causal ones up to its last query; split:
        // those whose half of the tile starts before the wave's key limit
        const int klim = causal ? min(S, qw0 + 32 * QB) : S;
        const int nw = Cfg::SPLIT ? max(0, (klim - koff + BN - 1) / BN)
                                  : causal ? min(ntiles, (qw0 + 32 * QB - 1) / BN + 1) : ntiles;

        auto kbuf = [&](int t) { return smem + (t % NB) * TK; };
        auto vbuf = [&](int t) { return smem + NB * TK + (t % NB) * TE; };
        typename Cfg::Tile::Src src;
        src.init(wave, lane);
        typename Cfg::KTile::Src ksrc;
        ksrc.init(wave, lane);
        DOffsets<typename Cfg::Tile, D> lo;
        lo.init(lane);
        const V8 rsel = lane_sum_selector<E>(lane);  // used where Cfg::MFMA_ROW_SUM
        // K row operand offsets: 16-bit, the DOffsets row reads; fp8, two 16-byte
        // chunks per step (indices 64s + 32h .. +31: slots 32s + 16h and +8)
        int k8[QK8 ? QS : 1][2];
        if constexpr (QK8) {
    #pragma unroll
            for (int st = 0; st < QS; ++st) {
                k8[st][0] = Cfg::KTile::at(n, st * 32 + 16 * h);
                k8[st][1] = Cfg::KTile::at(n, st * 32 + 16 * h + 8);
            }
        }

        // Q as the B operand of S^T = K Q^T: lane holds query qw0+32qb+n; 16-bit:
        // d = 16ks+8h..+7; fp8: d = 64s+32h..+31.
        QOp qf[QB][QS];
    #pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int q = qw0 + qb * 32 + n;
    #pragma unroll
            for (int st = 0; st < QS; ++st) {
                const uint16_t* row = Qh + (size_t)q * QK::KD;
                if constexpr (QK8) {
                    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
                    if (q < S) {
                        a = ldg16(row + st * 32 + 16 * h);
                        b = ldg16(row + st * 32 + 16 * h + 8);
                    }
                    qf[qb][st] = Fp8E4M3::join(a, b);
                } else {
                    u32x4 u = {0u, 0u, 0u, 0u};
                    if (q < S) u = ldg16(row + st * 16 + 8 * h);
                    qf[qb][st] = as_op<E>(u);
                }
            }
        }

        f32x16 oacc[QB][DB];
        float m[QB], l[QB];
    #pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            m[qb] = -FLT_MAX;
            l[qb] = 0.f;
    #pragma unroll
            for (int db = 0; db < DB; ++db)
    #pragma unroll
                for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
        }

        // K rows of tile t as A operands of S^T = K Q^T: kf[kb][st] holds key
        // t*BN + 32kb + n, at the contraction indices of the Q operand.
        auto load_k = [&](QOp (&kf)[KB][QS], int t) {
            const uint16_t* Ks = kbuf(t);
    #pragma unroll
            for (int kb = 0; kb < KB; ++kb)
    #pragma unroll
                for (int st = 0; st < QS; ++st) {
                    if constexpr (QK8) {
                        const uint16_t* r = Ks + kb * 32 * Cfg::KTile::RS;
                        kf[kb][st] = Fp8E4M3::join(lds16(r + k8[st][0]), lds16(r + k8[st][1]));
                    } else {
                        kf[kb][st] = lo.template row_op<E>(Ks, koff + kb * 32, st);
                    }
                }
        };
        // S^T tile from K operands already in registers; the first contraction step
        // starts from a zero accumulator.
        auto mma_scores = [&](f32x16 (&sacc)[QB][KB], const QOp (&kf)[KB][QS]) {
    #pragma unroll
            for (int st = 0; st < QS; ++st)
    #pragma unroll
                for (int kb = 0; kb < KB; ++kb)
    #pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        sacc[qb][kb] = QK::mma(kf[kb][st], qf[qb][st], st == 0 ? f32x16{} : sacc[qb][kb]);
        };

        // One key tile t: softmax of its scores `cur` and O += V_t P_t.  With NEXT,
        // the scores of tile t+1 are computed into `nxt` in the same straight-line
        // block as this tile's exp work, so the MFMAs run under the VALU work.
        // MASK instantiates the per-element causal / sequence-end mask; only a
        // wave's last tile can need it (its earlier tiles lie entirely below the
        // diagonal and before S), and the last tile has no successor.
        auto step = [&](auto mask_tag, auto next_tag, f32x16 (&cur)[QB][KB], f32x16 (&nxt)[QB][KB], int t) {
            constexpr bool MASK = decltype(mask_tag)::value;
            constexpr bool NEXT = decltype(next_tag)::value;
            QOp kf[KB][QS];
            if constexpr (NEXT) load_k(kf, t + 1);
            // V^T operands, read transposed from the V tile (asynchronous: used after lds_wait)
            i16x4 vr[KB * 2][DB][2];
            {
                const uint16_t* Vs = vbuf(t);
    #pragma unroll
                for (int ks = 0; ks < KB * 2; ++ks)
    #pragma unroll
                    for (int db = 0; db < DB; ++db) lo.tr_async(Vs, koff + ks * 16, db, vr[ks][db]);
            }

            // ---- mask (raw scores; only a wave's last tile)
            const int k0 = t * BN + koff;
            if constexpr (MASK) {
    #pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int q = qw0 + qb * 32 + n;
    #pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
    #pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = k0 + kb * 32 + crow(r, h);
                            const bool kill = (causal && key > q) || key >= S;
                            cur[qb][kb][r] = kill ? -INFINITY : cur[qb][kb][r];
                        }
                }
            }

            if constexpr (NEXT) mma_scores(nxt, kf);

            // ---- P = exp2(s*c - m) rounded to bf16 against the reference point
            // m; the row sum adds the same rounded values the PV product
            // multiplies, so numerator and denominator of O = (P V) / l carry the
            // same rounding (a row whose weight sits on one key reproduces that
            // key's V row).  The raw scores stay in `cur` for the rare path.
            V8 pf[QB][KB * 2];
            float ls[QB];
            auto probs = [&]() {
    #pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    ls[qb] = 0.f;
                    f32x4 rs = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        f32x16 e;
    #pragma unroll
                        for (int r = 0; r < 16; ++r) e[r] = fast_exp2(fmaf(cur[qb][kb][r], c, -m[qb]));
                        pf[qb][2 * kb] = pack_op<E>(e, 0);
                        pf[qb][2 * kb + 1] = pack_op<E>(e, 1);
                        if constexpr (Cfg::MFMA_ROW_SUM) {
                            rs = E::mma16(rsel, pf[qb][2 * kb], rs);
                            rs = E::mma16(rsel, pf[qb][2 * kb + 1], rs);
                        } else {
                            ls[qb] = sum8<E>(pf[qb][2 * kb], ls[qb]);
                            ls[qb] = sum8<E>(pf[qb][2 * kb + 1], ls[qb]);
                        }
                    }
                    if constexpr (Cfg::MFMA_ROW_SUM) ls[qb] = rs[0];
                }
            };
            probs();
            // The reference point stays put while every P is at most kPBound:
            // no lane's sum of its P values (all >= 0) above the bound means no
            // single P above it, so the tile needs no row max.  Otherwise
            // (wave-uniform; a row's first tile, where m starts at -FLT_MAX and
            // every P is infinite, and after that only when a row's scores grow
            // past its reference point by log2 of the bound) m moves to the row
            // max, O and l are rescaled and P is formed again.
            bool big = false;
    #pragma unroll
            for (int qb = 0; qb < QB; ++qb) big |= !(ls[qb] <= kPBound<E>);
            if (__builtin_amdgcn_ballot_w64(big) != 0) {
                asm volatile("");
    #pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    float v = -INFINITY;
    #pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
    #pragma unroll
                        for (int r = 0; r < 16; ++r) v = fmaxf(v, cur[qb][kb][r]);
                    // c > 0, so the max commutes with the scaling
                    const float mn = fmaxf(m[qb], half_max(v) * c);
                    const float f = fast_exp2(m[qb] - mn);
                    m[qb] = mn;
                    l[qb] *= f;
    #pragma unroll
                    for (int db = 0; db < DB; ++db)
    #pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= f;
                }
                probs();
            }
    #pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                l[qb] += ls[qb];
            }
            lds_wait(reinterpret_cast<i16x4 (&)[(KB * 2) * DB * 2]>(vr));
            V8 vf[KB * 2][DB];
    #pragma unroll
            for (int ks = 0; ks < KB * 2; ++ks)
    #pragma unroll
                for (int db = 0; db < DB; ++db) vf[ks][db] = tr_join<E>(vr[ks][db]);
            // ---- O^T += V^T P^T
    #pragma unroll
            for (int ks = 0; ks < KB * 2; ++ks)
    #pragma unroll
                for (int db = 0; db < DB; ++db)
    #pragma unroll
                    for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = E::mma(vf[ks][db], pf[qb][ks], oacc[qb][db]);
        };

        // ---- prologue: loads of K_0, then (K_{i+1}, V_i) for i < P, straight into
        // LDS.  Iteration t reads K_{t+1} and V_t and issues K_{t+1+P} and V_{t+P}
        // into the buffers of K_t and V_{t-1} (read in the previous iteration, so
        // free once the iteration's barrier has passed).  Each wave then finds the
        // tiles it needs complete once at most 2 (P - 1) tiles of its own loads are
        // outstanding: that count is the same in every iteration.  A tile index at
        // or past ntiles loads from row S: an empty buffer range, so the tile reads
        // as zeros and the count of loads stays the same on every path.
        auto row_of = [&](int t) { return t < ntiles ? t * BN : S; };
        auto load_kt = [&](int t) { Cfg::KTile::load(Kh, row_of(t), S, kbuf(t), ksrc, wave); };
        auto load_vt = [&](int t) { Cfg::Tile::load(Vh, row_of(t), S, vbuf(t), src, wave); };
        load_kt(0);
    #pragma unroll
        for (int i = 0; i < P; ++i) {
            load_kt(i + 1);
            load_vt(i);
        }
        wait_vmcnt<P * LOADS2>();  // K_0 landed
        bare_barrier();

        f32x16 sa[QB][KB], sb[QB][KB];
        if (nw > 0) {
            QOp kf[KB][QS];
            load_k(kf, 0);
            mma_scores(sa, kf);
        }

        // Iteration t: wait for K_{t+1} and V_t (own loads, then everyone's), issue
        // the loads of K_{t+1+P} and V_{t+P}, compute.
        auto iteration = [&](int t, f32x16 (&cur)[QB][KB], f32x16 (&nxt)[QB][KB]) {
            wait_vmcnt<(P - 1) * LOADS2>();
            bare_barrier();
            load_kt(t + 1 + P);
            load_vt(t + P);
            if (t + 1 < nw)
                step(std::false_type{}, std::true_type{}, cur, nxt, t);
            else if (t + 1 == nw)
                step(std::true_type{}, std::false_type{}, cur, nxt, t);
        };
        for (int t = 0; t < ntiles; t += 2) {
            iteration(t, sa, sb);
            if (t + 1 < ntiles) iteration(t + 1, sb, sa);
        }
        // no load may still be writing this workgroup's LDS when it exits
        wait_vmcnt<0>();

        if constexpr (Cfg::SPLIT) {
            // Merge the two key groups of each query block through LDS (the tile
            // buffers are free once every wave has passed this barrier): the second
            // group's waves store m, their lane's share of l and O; the first group's
            // waves rescale both to the larger reference point and add.  A group with
            // no tiles holds m = -FLT_MAX, l = 0, O = 0 and adds nothing.
            constexpr int ITEMS = 2 + DB * 16;
            static_assert(Cfg::QW * ITEMS * 64 * 4 <= (int)sizeof(smem), "the merge fits in the tile buffers");
            float* mb = reinterpret_cast<float*>(smem) + qg * ITEMS * 64 + lane;
            __syncthreads();
            if (koff != 0) {
                mb[0] = m[0];
                mb[64] = l[0];
    #pragma unroll
                for (int db = 0; db < DB; ++db)
    #pragma unroll
                    for (int r = 0; r < 16; ++r) mb[(2 + db * 16 + r) * 64] = oacc[0][db][r];
            }
            __syncthreads();
            if (koff != 0) continue;
            const float m1 = mb[0], l1 = mb[64];
            const float mn = fmaxf(m[0], m1);
            const float f0 = fast_exp2(m[0] - mn), f1 = fast_exp2(m1 - mn);
            m[0] = mn;
            l[0] = l[0] * f0 + l1 * f1;
    #pragma unroll
            for (int db = 0; db < DB; ++db)
    #pragma unroll
                for (int r = 0; r < 16; ++r) oacc[0][db][r] = oacc[0][db][r] * f0 + mb[(2 + db * 16 + r) * 64] * f1;
        }

        // ---- epilogue: O = O / l (l == 0 -> 0), LSE = (m + log2 l) * ln 2
        uint16_t* Oh = O + base;
        float* Lh = LSE + (size_t)head * S;
    #pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int q = qw0 + qb * 32 + n;
            const float lt = half_sum(l[qb]);
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            if (q < S) {
    #pragma unroll
                for (int db = 0; db < DB; ++db)
    #pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        if (!HeadDim<D>::live(db, g)) continue;
                        u32x2 u;
                        u[0] = E::pack2(oacc[qb][db][4 * g + 0] * inv, oacc[qb][db][4 * g + 1] * inv);
                        u[1] = E::pack2(oacc[qb][db][4 * g + 2] * inv, oacc[qb][db][4 * g + 3] * inv);
                        *reinterpret_cast<u32x2*>(Oh + (size_t)q * D + db * 32 + 8 * g + 4 * h) = u;
                    }
                if (h == 0) Lh[q] = lt > 0.f ? (m[qb] + __log2f(lt)) * kLn2 : -INFINITY;
            }
        }
    }

}

template <class E, int D, int QB, int NW, bool QK8, int BN, bool SPLIT = false>
static hipError_t launch_fwd(const LaunchArgs& a) {
    using Cfg = FwdCfg<D, QB, NW, QK8, BN, SPLIT>;
    const int nblk = (int)((a.S + Cfg::BM - 1) / Cfg::BM);
    // pairs when one query block per workgroup would not fit in one round of the
    // device's workgroup slots (CUs x workgroups per CU) and the pairs still cover
    // every slot (fewer workgroups than slots leave CUs idle)
    const int64_t slots = (int64_t)cu_count() * Cfg::WAVES_PER_SIMD * 4 / Cfg::NW;
    const int paired = Cfg::PAIRABLE && a.causal && (int64_t)nblk * a.BH > slots &&
                               (int64_t)((nblk + 1) / 2) * a.BH >= slots
                           ? 1
                           : 0;
    const int64_t total = (int64_t)(paired ? (nblk + 1) / 2 : nblk) * a.BH;
    if (total > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fwd_mfma_kernel<E, D, QB, NW, QK8, BN, SPLIT>), dim3((unsigned)total), dim3(Cfg::NT), 0, a.stream,
                       a.q, a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, (int)a.S, nblk, (int)a.BH,
                       (int)a.H, (int)(a.H / a.Hkv), a.scale * a.qk_descale * kLog2e, a.causal, paired);
    return hipGetLastError();
}

// The forward for one head dim: split key groups (64-query workgroups, each staged
// key tile shared by two waves instead of four) where the unsplit grid is small
// against one round of the device's workgroup slots, since such a grid is bound by
// its longest waves, whose tile chains the split halves; else one query block (or,
// from D = 80 up, a pair of blocks) per workgroup.  The line, measured (forward):
// at D = 64 (three workgroups per CU) two thirds of a round: B=2 H=16 S=2048 (2/3)
// 32.9 -> 27.5 us, B=4 H=12 S=1024 18.7 -> 13.9, B=8 H=6 S=256 7.7 -> 6.2, but
// B=6 H=12 S=1024 (3/4) +3.5%, B=8 H=12 S=1024 (one round) +6%, B=4 H=16 S=2048 +6%,
// B=8 H=16 S=2048 +19%; from D = 80 up (two per CU) one round: D = 128 B=1 H=8
// S=4096 (1/2) 77.9 -> 55.9 us, B=1 H=4 S=8191 148.9 -> 105.1, B=1 H=24 S=2048 (3/4)
// 46.1 -> 39.8, B=1 H=16 S=4096 (one round) 91.5 -> 86.2, D = 80 B=1 H=24 S=2048
// 36.1 -> 29.7, but B=2 H=32 S=2048 (two rounds, paired) +17%.
template <class E, int D>
static hipError_t launch_fwd_dim(const LaunchArgs& a) {
    using Cfg = FwdCfg<D, 1, 4, false, 32>;
    const int64_t slots = (int64_t)cu_count() * Cfg::WAVES_PER_SIMD * 4 / Cfg::NW;
    const int64_t blocks = (a.S + Cfg::BM - 1) / Cfg::BM * a.BH;
    const bool split = D == 64 ? 3 * blocks <= 2 * slots : blocks <= slots;
    if (split) return launch_fwd<E, D, 1, 4, false, 64, true>(a);
    return launch_fwd<E, D, 1, 4, false, 32>(a);
}

template <class E>
static hipError_t launch_fwd_type(const LaunchArgs& a) {
    if (a.D == 64) return launch_fwd_dim<E, 64>(a);
    if (a.D == 80) return launch_fwd_dim<E, 80>(a);
    if (a.D == 96) return launch_fwd_dim<E, 96>(a);
    if (a.D == 128) return launch_fwd_dim<E, 128>(a);
    return hipErrorInvalidValue;
}

template <class E>
static hipError_t launch_fwd_fp8qk_type(const LaunchArgs& a) {
    // (fp8 rows of 64 bytes: a 32-key K tile is too small to split over 4 waves' loads)
    if (a.D == 64) return launch_fwd<E, 64, 1, 4, true, 64>(a);
    if (a.D == 128) return launch_fwd<E, 128, 1, 4, true, 32>(a);
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_bf16(const LaunchArgs& a) { return launch_fwd_type<Bf16>(a); }
hipError_t launch_fwd_f16(const LaunchArgs& a) { return launch_fwd_type<F16>(a); }
hipError_t launch_fwd_fp8qk_bf16(const LaunchArgs& a) { return launch_fwd_fp8qk_type<Bf16>(a); }
hipError_t launch_fwd_fp8qk_f16(const LaunchArgs& a) { return launch_fwd_fp8qk_type<F16>(a); }

}  // namespace attn
