// Fused chunked gated delta rule scan for gfx950 (CDNA4).
//
// Method: the gated delta rule named on "flashinfer.gdn_prefill" (the chunked
// GDN scan) with the argument semantics of
// "flashinfer.cudnn.cudnn_chunk_gated_delta_rule" (Parameters).  Per chunk of
// C = 64 tokens (aligned to the sequence start), with G_i the in-chunk
// cumulative sum of ln(a), gamma_i = exp(G_i), and S0 the [V, K] state on
// entry, the chunk (UT / WY) form of the recurrence is
//
//   A_ij  = b_i (k_i . k_j) exp(G_i - G_j)           j < i   (strictly lower)
//   T'    = (I + A)^-1                                        (UT transform)
//   Vnew  = T' ( b o (V - diag(gamma) K S0^T) )               (rows scaled by b)
//   O     = scale [ diag(gamma) Q S0^T + ((Q K^T) o D) Vnew ],  D_ij = exp(G_i-G_j), j <= i
//   S_L   = gamma_L S0 + Vnew^T diag(exp(G_L - G)) K
//
// which equals the token recurrence exactly in real arithmetic.  L2
// normalisation is folded into per-row factors (rk, rq) so the MFMA operands
// are the caller's exact q/k values.
//
// Mapping to the hardware.  One workgroup (4 waves) scans one value head of
// one sequence; two workgroups share a CU (LDS < 80 KB, <= 256 VGPRs) so one
// can run matrix work while the other waits or solves.
//   * The fp32 state lives in MFMA accumulators for the whole sequence: wave
//     w owns state rows v in [32w, 32w+32) as four 32x32 tiles of S^T.
//   * Accumulators are reused directly as B operands (S0^T, Z, Vnew): the
//     contraction index of those products is permuted to the accumulator's
//     row order and the LDS-side operand is read with the same permutation.
//   * Per chunk: [L] stage K and Q in LDS; [A] one pass over the 128-wide
//     contraction gives K S~^T and S~ Q^T for the wave's own state rows plus
//     its Gram tiles and row norms, and one wave forms the next chunk's gate
//     prefix sums and decay rows (two row sets alternate); [B] A (fp32)
//     and P into LDS while the next chunk's K, Q loads are in flight; [C] the
//     four 16x16 diagonal inverses by forward substitution (one per wave), the
//     16->32 merges and the 32->64 merge on MFMA; [D] Vnew, O and the state
//     update.
//   * Global accesses go through buffer resources whose range ends at the
//     chunk's last valid token, so ragged tails load zeros and drop stores
//     without branches.
//   * Value heads that share a q/k head are mapped to workgroups that land on
//     the same XCD at the same time, so their q/k reads meet in that L2.
//   * bf16 inputs run v_mfma_f32_32x32x16_bf16 / 16x16x16 (fp32 accumulate);
//     fp32 inputs run the fp32 MFMAs so they keep fp32 accuracy.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdn_device.h"

namespace gdn {
namespace {

using namespace dev;

static_assert(kGateWave == 2, "the gate rows ride on the third wave's Gram pass");

template <typename IO> struct Smem {
    static constexpr bool BF = is_bf<IO>::value;
    static constexpr int KLD = BF ? kKqLd : 132;   // K, Q rows (elements of IO; bf16 rows permuted, see kq_row)
    static constexpr int OLD = 68;               // T', P rows (elements of IO)
    static constexpr int FLD = 68;               // fp32 64x64 work matrix (A, inverse blocks)
    static constexpr int KB = C * KLD * (int)sizeof(IO);
    static constexpr int K_OFF = 0;
    static constexpr int Q_OFF = K_OFF + KB;
    static constexpr int P_OFF = Q_OFF + KB;
    static constexpr int T_OFF = P_OFF + C * OLD * (int)sizeof(IO);
    static constexpr int AF_OFF = T_OFF + C * OLD * (int)sizeof(IO);
    // diagonal 16x16 blocks of A, transposed: NT[b][m][4 (i % 4) + i / 4] = A[16b + i][16b + m]
    // (column m, rows grouped by i % 4); block stride padded against bank conflicts
    static constexpr int NTS = 16 * 16 + 4;
    static constexpr int NT_OFF = AF_OFF + C * FLD * 4;
    static constexpr int ROW_OFF = NT_OFF + 4 * NTS * 4;
    static constexpr int BYTES = ROW_OFF + (kRowsTotal * C + 4) * 4;
    static_assert(!BF || BYTES <= 80 * 1024, "two workgroups per CU");
    static_assert(!BF || 4 * kStageBytes <= C * FLD * 4, "four staging blocks in the A area");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(Q_OFF % 16 == 0 && AF_OFF % 16 == 0 && T_OFF % 16 == 0 &&
                  ROW_OFF % 16 == 0, "align");
};

// bf16: two workgroups per CU (LDS < 80 KB) need <= 256 registers per lane;
// fp32 (LDS-bound to one workgroup per CU) keeps the full register file.
template <typename IO, int MODE, bool CK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(is_bf<IO>::value ? 2 : 1,
                                                                    is_bf<IO>::value ? 2 : 1))) void
fused_scan_kernel(const ScanParams p) {
    constexpr bool OUT = MODE == kScan;     // map modes produce no output rows
    constexpr bool PREP = MODE == kPrep;    // preparation only: no state, no v
    constexpr bool USEQ = OUT || PREP;      // q, its norms and the output tile P
    constexpr bool HASV = MODE != kMapM && !PREP;   // the M map scans v = 0
    using L = Smem<IO>;
    using M = Mma<IO>;
    using frag = typename M::frag;
    constexpr bool BF = L::BF;
    constexpr int E = M::E;
    constexpr int S32 = 32 / (2 * E);       // 32x32 MFMA steps per 32-wide contraction block
    constexpr int S16 = 16 / (4 * M::E16);  // 16x16 MFMA steps per 16-wide contraction block

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    IO *Ks = reinterpret_cast<IO *>(smem + L::K_OFF);
    IO *Qs = reinterpret_cast<IO *>(smem + L::Q_OFF);
    IO *Ps = reinterpret_cast<IO *>(smem + L::P_OFF);
    IO *Ts = reinterpret_cast<IO *>(smem + L::T_OFF);
    float *Af = reinterpret_cast<float *>(smem + L::AF_OFF);
    float *RF = reinterpret_cast<float *>(smem + L::ROW_OFF);     // per-row factors
    float *NT = reinterpret_cast<float *>(smem + L::NT_OFF);      // transposed diagonal blocks of A
    // factor row `which`, gate rows of set `set`; gamma_L of a set
    auto rf_set = [&](int which, int set) { return RF + (which < kGateRows ? which + set * NROWF : which) * C; };
    auto gamma_l = [&](int set) -> float & { return RF[kRowsTotal * C + set]; };
    auto igamma_l = [&](int set) -> float & { return RF[kRowsTotal * C + 2 + set]; };   // 1 / gamma_L

    // ---- work item: XCD-aware so the r value heads of one q/k head meet in one L2
    const int r = p.r;
    const int b = blockIdx.x;
    const int within = b % (8 * r);
    const int pidx = (b / (8 * r)) * 8 + (within & 7);
    const int items = p.segs ? p.seg_cap : p.N;
    if (pidx >= items * p.Hqk) return;
    const int item = pidx / p.Hqk, hq = pidx % p.Hqk;
    const int h = hq * r + (within >> 3);
    int n;
    int64_t bos, eos;
    bool first = true, last = true;
    if (p.segs) {
        if (item >= *p.nsegs) return;
        const SegEntry e = p.segs[item];
        n = e.n;
        bos = e.bos;
        eos = e.eos;
        first = e.first != 0;
        last = e.last != 0;
        if ((MODE == kMapN || MODE == kMapM) && last) return;   // maps: all but the last segment
        if constexpr (PREP) {   // a range of chunks: only the segments that start in it
            const int sc0 = (int)((bos - load_cu(p.cu, n, p.cu_i64)) / C);
            if (sc0 < p.ph_c0 || (p.ph_len > 0 && sc0 >= p.ph_c0 + p.ph_len)) return;
        }
    } else {
        n = item;
        bos = load_cu(p.cu, n, p.cu_i64);
        eos = load_cu(p.cu, n + 1, p.cu_i64);
    }
    const int64_t map_off = ((int64_t)item * p.Hv + h) * kMapBytes;
    const int64_t srow = state_row(p.sidx, p.sidx_i64, p.pool_rows, n);

    // ---- initial state: S[b] holds S^T rows k = 32b + acc_row(r, h32), column v0
    f32x16 S[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) S[bb] = zero16();
    {
        const int tid = threadIdx.x, lane = tid & 63, ws = tid >> 6;
        const int h32 = lane >> 5, v0 = ws * 32 + (lane & 31);
        if (MODE == kScan) {
            // a pooled state is read and written in place: the first segment of a
            // split sequence takes it from the workspace (copied there by the
            // fix-up), so no work item reads a row another one may be writing
            if (!first || (p.sidx && !last))
                load_state<BF>(S, reinterpret_cast<const char *>(p.ws_sin) + map_off, D * 4, GDN_F32, v0, h32);
            else if (p.s_in && srow >= 0)
                load_state<BF>(S, p.s_in + srow * p.si_n + h * p.si_h, p.si_v, p.si_dt, v0, h32);
        } else if (MODE == kMapM) {           // identity: S^T[k][v0] = (k == v0)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) S[bb][rr] = (state_k<BF>(bb, rr, h32) == v0) ? 1.f : 0.f;
        }
    }

    const int nchunks = (int)((eos - bos + C - 1) / C);
    // chunks of the sequence before this work item (segments start on chunk bounds)
    const int seq_chunk0 = (CK && p.segs) ? (int)((bos - load_cu(p.cu, n, p.cu_i64)) / C) : 0;
    float sigma = 1.f;          // true state = sigma * S (uniform across the workgroup)
    // Gate rows of one chunk into set `set`, on the gate wave (lane i = token i of
    // the chunk): the in-chunk log-gate cumsum G, gamma = exp(G), 1 / gamma,
    // exp(G_L - G), b (zero past the chunk end) and gamma_L.
    auto gate_rows = [&](const Prefetch<IO> &g, int Lch, int set, int lane) {
        const bool valid = lane < Lch;
        const float ga = p.g ? gate_value(g.g, p.g_dt) : 1.f;
        const float gb = p.beta ? gate_value(g.b, p.b_dt) : 1.f;
        const float G = wave_prefix_sum(valid ? fmaxf(__logf(ga), -80.f) : 0.f);
        const float GL = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 63));
        const float gam = __expf(G);
        rf_set(RG_, set)[lane] = G;
        rf_set(GM_, set)[lane] = gam;
        rf_set(IG_, set)[lane] = __expf(-G);
        rf_set(DC_, set)[lane] = __expf(GL - G);
        rf_set(FB_, set)[lane] = valid ? gb : 0.f;
        gamma_l(set) = __expf(GL);   // the same value from every lane
        igamma_l(set) = __expf(-GL);
    };
    // The gates run two chunks ahead of K and Q: chunk c + 1's gate rows are
    // written during chunk c (phase [A], gate wave), from values loaded during
    // chunk c - 1.
    Prefetch<IO> pf, pf_g0;   // pf_g0: chunk 0's gates (gate wave)
    const int ws0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (nchunks > 0) {
        issue_loads<IO>(pf, p, chunk_at(bos, eos, 0), hq, h, threadIdx.x, threadIdx.x & 63, ws0);
        if (ws0 == kGateWave) {
            issue_gates(pf_g0, p, chunk_at(bos, eos, 0), h, threadIdx.x & 63);
            issue_gates(pf, p, chunk_at(bos, eos, 1), h, threadIdx.x & 63);
        }
    }
    // Wait for the first chunk's loads (and chunk 1's gates) here, once.  In the
    // loop the prefetches are retired by the wait for chunk c's V, so the chunk
    // head needs no vector-memory wait; without this the loop entry would make
    // the head wait for everything outstanding, the previous chunk's output
    // stores included.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (nchunks > 0 && ws0 == kGateWave) gate_rows(pf_g0, chunk_at(bos, eos, 0).L, 0, threadIdx.x & 63);

    for (int c = 0; c < nchunks; ++c) {
        const ChunkRef ch = chunk_at(bos, eos, c);
        const int Lc = ch.L;
        // Lane indices are re-derived from an opaque copy each chunk so that the
        // compiler recomputes per-element addresses and masks (a few ALU ops)
        // instead of hoisting hundreds of them out of the loop into registers.
        int tid_o = threadIdx.x;
        asm volatile("" : "+v"(tid_o));
        const int tid = tid_o, lane = tid & 63;
        const int ws = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int h32 = lane >> 5, l32 = lane & 31;
        const int v0 = ws * 32 + l32;
        const int gset = c & 1;
        auto rf = [&](int which) { return rf_set(which, gset); };

        // ---- [L] stage K and Q (this chunk's gate rows are already in set gset)
        if constexpr (BF) {
            const int rq4 = tid >> 4, cg = tid & 15;
#pragma unroll
            for (int mat = 0; mat < 2; ++mat)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    *reinterpret_cast<i32x4 *>((mat ? Qs : Ks) + kq_off(4 * rq4 + t, 8 * cg)) = pf.kq[mat][t];
        } else {
            const int r0 = tid >> 5, cg = tid & 31;
#pragma unroll
            for (int mat = 0; mat < 2; ++mat)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    *reinterpret_cast<f32x4 *>((mat ? Qs : Ks) + (r0 + 8 * j) * L::KLD + 4 * cg) = pf.kq[mat][j];
        }
        __syncthreads();

        // ---- [A] Gram tiles; row norms from their operands
        // The true state is sigma * S~.  After this chunk it is
        //   gamma_L sigma S~ + K^T U  =  sigma' (S~ + K^T U / sigma'),  sigma' = gamma_L sigma,
        // so the decay costs no per-element work; when sigma' gets small it is
        // folded back into S~ (renorm) to keep U / sigma' in range.
        const float gLc =
            __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, gamma_l(gset))));
        const float sig_next = sigma * gLc;
        const bool renorm = !(sig_next >= kRenorm);
        const bool fast = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(
                              int, rf(RG_)[C - 1]))) > kFastDecay;
        // Gram tiles (bi, bj) = (0,0) (1,0) (1,1) of K K^T ("A" tiles) and Q K^T ("P"
        // tiles), each computed transposed: register rows are the column index
        // j = 32 bj + acc_row, the lane is the row index i = 32 bi + l32.
        // One pass over the 128-wide contraction reads, per step, the fragments of
        // K_0, K_1, Q_0, Q_1 (K_b / Q_b = rows 32b .. 32b+31) once and feeds:
        //   X = K S~^T and (S~ Q^T) for this wave's 32 state rows (S~ as the A operand
        //   gives the transpose), four accumulator chains;
        //   this wave's Gram tiles (first operand = K rows of the column block):
        //     wave 0: A(0,0) = K_0 K_0 (two accumulators: even / odd steps)   norms of K_0, Q_1
        //     wave 1: A(1,0) = K_0 K_1, P(1,1) = K_1 Q_1      norms of K_1
        //     wave 2: A(1,1) = K_1 K_1 (two accumulators); then the next chunk's
        //             gate rows (kGateWave)
        //     wave 3: P(0,0) = K_0 Q_0, P(1,0) = K_0 Q_1      norms of Q_0
        //   the squared row norms (dot2 on the fragments).
        // The contraction runs in the state's register order (natural for bf16,
        // accumulator order for fp32); the next step's fragments are read while
        // this step's MFMAs run.
        f32x16 gt[2] = {zero16(), zero16()};
        f32x16 X[2] = {zero16(), zero16()}, Y[2] = {zero16(), zero16()};
        const ChunkRef next = chunk_at(bos, eos, c + 1);
        {
            constexpr int NK = 4 * S32;
            auto frag_at = [&](const IO *M, int blk, int k) -> frag {
                if constexpr (BF) return ld_kq(M, 32 * blk + l32, k, h32);
                else return ld_acc<IO>(M, L::KLD, 32 * blk + l32, 32 * (k / S32), k % S32, h32);
            };
            auto sq = [&](const frag &f, float acc) {   // acc + the squares of f's elements
                if constexpr (BF) return sumsq8_acc(f, acc);
                else return acc + f * f;
            };
            // 1 / |row| (or 1 without the norm); a K row's factor also goes into
            // its 1 / gamma entry, which only the A tiles read
            auto put_norm = [&](float ss, int which, int blk) {
                ss += __shfl_xor(ss, 32);
                if (h32 == 0) {
                    const int row = 32 * blk + l32;
                    const float r = p.l2norm ? __builtin_amdgcn_rsqf(ss + 1e-6f) : 1.f;
                    rf(which)[row] = r;
                    if (which == RK_) rf(IG_)[row] *= r;
                }
            };
            auto pass = [&](auto role) {
                constexpr int R = decltype(role)::value;
                frag fk[2][2], fq[2][2];
                auto load = [&](int k, int st) {
                    fk[st][0] = frag_at(Ks, 0, k);
                    fk[st][1] = frag_at(Ks, 1, k);
                    if constexpr (USEQ) {
                        fq[st][0] = frag_at(Qs, 0, k);
                        fq[st][1] = frag_at(Qs, 1, k);
                    }
                };
                float ssa = 0.f, ssb = 0.f;
                load(0, 0);
#pragma unroll
                for (int k = 0; k < NK; ++k) {
                    const int cur = k & 1;
                    if (k + 1 < NK) load(k + 1, cur ^ 1);
                    const frag k0 = fk[cur][0], k1 = fk[cur][1];
                    if constexpr (!PREP) {
                        const frag sf = acc_frag<IO>(S[k / S32], k % S32);
                        X[0] = M::run(k0, sf, X[0]);
                        X[1] = M::run(k1, sf, X[1]);
                        if constexpr (OUT) {
                            Y[0] = M::run(sf, fq[cur][0], Y[0]);
                            Y[1] = M::run(sf, fq[cur][1], Y[1]);
                        }
                    }
                    if constexpr (R == 0) {
                        gt[cur] = M::run(k0, k0, gt[cur]);
                        ssa = sq(k0, ssa);
                        if constexpr (USEQ) ssb = sq(fq[cur][1], ssb);
                    } else if constexpr (R == 1) {
                        gt[0] = M::run(k0, k1, gt[0]);
                        ssa = sq(k1, ssa);
                        if constexpr (USEQ) gt[1] = M::run(k1, fq[cur][1], gt[1]);
                    } else if constexpr (R == 2) {
                        gt[cur] = M::run(k1, k1, gt[cur]);
                    } else if constexpr (USEQ) {
                        gt[0] = M::run(k0, fq[cur][0], gt[0]);
                        gt[1] = M::run(k0, fq[cur][1], gt[1]);
                        ssb = sq(fq[cur][0], ssb);
                    }
                }
                if constexpr (R == 0) {
                    gt[0] += gt[1];
                    put_norm(ssa, RK_, 0);
                    if constexpr (USEQ) put_norm(ssb, RQ_, 1);
                } else if constexpr (R == 1) {
                    put_norm(ssa, RK_, 1);
                } else if constexpr (R == 2) {
                    gt[0] += gt[1];
                } else if constexpr (USEQ) {
                    put_norm(ssb, RQ_, 0);
                }
            };
            if (ws == 0) pass(std::integral_constant<int, 0>{});
            else if (ws == 1) pass(std::integral_constant<int, 1>{});
            else if (ws == kGateWave) {   // also the next chunk's gate rows (the other set)
                pass(std::integral_constant<int, 2>{});
                gate_rows(pf, next.L, gset ^ 1, lane);
            }
            else pass(std::integral_constant<int, 3>{});
        }
        __syncthreads();

        // ---- [B] next chunk's K, Q and the gates of chunk c + 2 in flight; A (fp32)
        // and P into LDS.  bf16: half of the K, Q loads go out here, the rest after
        // the tiles are formed, so that a wave does not stall on a long run of load
        // issues
        if constexpr (BF) {
            issue_kq_part(pf, p, next, hq, tid, 0);
            issue_kq_part(pf, p, next, hq, tid, 1);
        } else {
            issue_loads<IO>(pf, p, next, hq, h, tid, lane, ws);
            if (ws == kGateWave) issue_gates(pf, p, chunk_at(bos, eos, c + 2), h, lane);
        }
        {
            // Lane row i = 32 bi + l32; register 4 jj + t is column j = 32 bj + 8 jj + 4 h32 + t.
            //   A = b_i rk_i rk_j (k_i . k_j) exp(G_i - G_j)   for j < i   (fp32)
            //   P = c rq_i rk_j (q_i . k_j) exp(G_i - G_j)      for j <= i  (slow)
            //   P = q_i . k_j                                  for j <= i  (fast: the row
            //       and column factors move to the output rows and to the shared Vnew
            //       operand, see [D])
            // Four consecutive columns are stored at once; every factor read is
            // issued before the first store.
            // Wave w < 3 holds A tile (0,0), (1,0), (1,1); wave 1 also P tile (1,1) and
            // wave 3 P tiles (0,0) and (1,0); the map modes need no P.
            // diagonal tiles only (bi == bj): row - column = l32 - 4 h32 - 8 jj - t
            const int dlane = l32 - 4 * h32;
            auto mask_row = [&](f32x4 &v, int jj, int keep_diag) {
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = dlane > 8 * jj + t - keep_diag ? v[t] : 0.f;
            };
            auto a_tile = [&](const f32x16 &acc, int bi, int bj) {
                const int i = 32 * bi + l32, jb = 32 * bj + 4 * h32;
                f32x4 v[4];
                if (fast) {   // (b_i rk_i gamma_i) (rk_j / gamma_j) (k_i . k_j); IG_ holds rk_j / gamma_j
                    const float ea = rf(FB_)[i] * rf(RK_)[i] * rf(GM_)[i];
                    f32x4 ig[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) ig[jj] = ld4(rf(IG_) + jb + 8 * jj);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                        for (int t = 0; t < 4; ++t) v[jj][t] = ea * ig[jj][t] * acc[4 * jj + t];
                } else {
                    const float fi = rf(FB_)[i] * rf(RK_)[i], Gi = rf(RG_)[i];
                    f32x4 rk[4], G4[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        rk[jj] = ld4(rf(RK_) + jb + 8 * jj);
                        G4[jj] = ld4(rf(RG_) + jb + 8 * jj);
                    }
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            v[jj][t] = fi * rk[jj][t] * acc[4 * jj + t] * __expf(fminf(Gi - G4[jj][t], 0.f));
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    if (bi == bj) mask_row(v[jj], jj, 0);
                    *reinterpret_cast<f32x4 *>(Af + i * L::FLD + jb + 8 * jj) = v[jj];
                }
                if (bi == bj) {   // this lane's row lies in diagonal block 2 bi + (l32 >= 16)
                    const int hi = l32 >= 16;
                    const int ir = l32 & 15;
                    float *nt = NT + (2 * bi + hi) * L::NTS + 4 * (ir & 3) + (ir >> 2);
#pragma unroll
                    for (int jr = 0; jr < 2; ++jr)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            nt[(8 * jr + 4 * h32 + t) * 16] = hi ? v[2 + jr][t] : v[jr][t];
                }
            };
            auto p_tile = [&](const f32x16 &acc, int bi, int bj) {
                const int i = 32 * bi + l32, jb = 32 * bj + 4 * h32;
                f32x4 v[4];
                if (fast) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                        for (int t = 0; t < 4; ++t) v[jj][t] = acc[4 * jj + t];
                } else {
                    const float fi = p.scale * rf(RQ_)[i], Gi = rf(RG_)[i];
                    f32x4 rk[4], G4[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        rk[jj] = ld4(rf(RK_) + jb + 8 * jj);
                        G4[jj] = ld4(rf(RG_) + jb + 8 * jj);
                    }
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            v[jj][t] = fi * rk[jj][t] * acc[4 * jj + t] * __expf(fminf(Gi - G4[jj][t], 0.f));
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    if (bi == bj) mask_row(v[jj], jj, 1);
                    if constexpr (BF) {
                        const bf16x4 b4 = {(bf16)v[jj][0], (bf16)v[jj][1], (bf16)v[jj][2], (bf16)v[jj][3]};
                        *reinterpret_cast<bf16x4 *>(Ps + i * L::OLD + jb + 8 * jj) = b4;
                    } else {
                        *reinterpret_cast<f32x4 *>(Ps + i * L::OLD + jb + 8 * jj) = v[jj];
                    }
                }
            };
            if (ws < 3) a_tile(gt[0], ws > 0, ws == 2);
            if constexpr (USEQ) {
                if (ws == 3) {
                    p_tile(gt[0], 0, 0);
                    p_tile(gt[1], 1, 0);
                }
                if (ws == 1) p_tile(gt[1], 1, 1);
            }
            if constexpr (BF) {
                issue_kq_part(pf, p, next, hq, tid, 2);
                issue_kq_part(pf, p, next, hq, tid, 3);
                if (ws == kGateWave) issue_gates(pf, p, chunk_at(bos, eos, c + 2), h, lane);
            }
            if (PREP && ws == 0) {   // the row factors without the lazy scale, lane = token
                const float rk = rf(RK_)[lane], gam = rf(GM_)[lane], dec = rf(DC_)[lane];
                rf(FZ_)[lane] = gam * rk;
                rf(FU_)[lane] = rk * dec;
                rf(FY_)[lane] = (p.scale * gam) * rf(RQ_)[lane];
            } else if (ws == 0) {   // row factors of [D], lane = token
                const float rk = rf(RK_)[lane], gam = rf(GM_)[lane], dec = rf(DC_)[lane];
                rf(FZ_)[lane] = sigma * (gam * rk);
                rf(FU_)[lane] = renorm ? rk * dec : (rk * dec) / sig_next;
                if constexpr (OUT) {
                    // a renormalising fast chunk carries its state term as (Y sigma) gamma_L,
                    // so its output rows take 1 / gamma_L instead of sigma (see [D])
                    const float base = (p.scale * gam) * rf(RQ_)[lane];
                    rf(FY_)[lane] = fast && renorm ? base * igamma_l(gset) : sigma * base;
                }
            }
        }
        __syncthreads();

        // ---- [C] this chunk's V in flight (first read in [D]); T' = (I + A)^-1: each
        // wave solves one 16x16 diagonal block, then the blocks are merged (16->32->64)
        VRegs vcur;       // fp32: one element per register, accumulator layout
        VWide vwide;      // bf16: 16-byte loads, moved to the accumulator layout through LDS in [D]
        if constexpr (HASV) {
            if constexpr (!BF) issue_v<IO>(vcur, p, ch, h, h32, v0);   // bf16: inside the solve below
        } else {
#pragma unroll
            for (int e = 0; e < 32; ++e) vcur.x[e] = 0u;
        }
        {
            // (1) wave w: D = (I + N)^-1 for the strictly lower 16x16 diagonal block N
            // of rows 16w .. 16w+15, by right-looking forward substitution.  Lane =
            // (column c, row class r): it holds D[r + 4k][c], k = 0..3.  Step m
            // broadcasts x_m = D[m][c] inside the lane quad (DPP) and subtracts
            // N[r + 4k][m] x_m (zero for rows at or above m, as N is strictly lower),
            // with N[r + 4k][m] read from the transposed copy one step ahead.
            const int c = lane >> 2, rq = lane & 3;
            const float *nt = NT + ws * L::NTS + 4 * rq;
            float x[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) x[k] = rq + 4 * k == c ? 1.f : 0.f;
            f32x4 ncol[2];
            ncol[0] = ld4(nt);
#pragma unroll
            for (int m = 0; m < 15; ++m) {
                if (m + 1 < 15) ncol[(m + 1) & 1] = ld4(nt + (m + 1) * 16);
                // bf16 V: one of the four 16-byte loads every fourth step
                if constexpr (BF && HASV) {
                    if (m % 4 == 0) issue_v_wide_part(vwide, p, ch, h, ws, lane, m / 4);
                }
                const float xm = quad_bcast(x[m >> 2], m & 3);
#pragma unroll
                for (int k = 0; k < 4; ++k) x[k] = fmaf(-ncol[m & 1][k], xm, x[k]);
            }
            const float bcol = rf(FB_)[16 * ws + c];
            float *blk = Af + (16 * ws) * L::FLD + 16 * ws;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = rq + 4 * k;
                blk[i * L::FLD + c] = x[k];
                Ts[(16 * ws + i) * L::OLD + 16 * ws + c] = (IO)(x[k] * bcol);
                if ((ws & 1) == 0) Ts[(16 * ws + i) * L::OLD + 16 * ws + 16 + c] = (IO)0.f;
            }
        }
        __syncthreads();
        // (2) 16 -> 32: T'_{2x+1,2x} = -D_{2x+1} A_{2x+1,2x} D_{2x}, x = 0, 1
        auto merge16 = [&](int x2) {
            const int g = lane >> 4, nn = lane & 15;
            const int lo = 32 * x2, hi = 32 * x2 + 16;
            f32x4 R = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < S16; ++s)
                R = M::run16(ld16_row<IO>(Af, L::FLD, hi + nn, lo, s, g), ld16_col<IO>(Af, L::FLD, lo + nn, lo, s, g), R);
            const float bcol = rf(FB_)[lo + nn];
            f32x4 Tq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < S16; ++s)
                Tq = M::run16(ld16_row<IO>(Af, L::FLD, hi + nn, hi, s, g), acc16_frag<IO>(R, s), Tq);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int i = hi + 4 * g + rr;
                Af[i * L::FLD + lo + nn] = -Tq[rr];
                Ts[i * L::OLD + lo + nn] = (IO)(-Tq[rr] * bcol);
            }
        };
        if constexpr (BF) {
            // the two 16 -> 32 merges on waves 0 and 1; then the four 16x16 blocks
            // (r, c) of T''_21 = -T'_22 A_21 T''_11 on the four waves: wave (r, c) forms
            // R = A_21 T''_11[:, c] (both 16-row halves) and -T'_22[r, :] R.  T''_11 is
            // read as its column-scaled copy from Ts (transposing loads), so the
            // product carries the column scale that Ts holds.
            if (ws < 2) merge16(ws);
            __syncthreads();
            const int r = ws >> 1, cc = ws & 1;
            const int g = lane >> 4, n = lane & 15;
            typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
            // T''_11 rows 8g .. 8g+7 of column 16 cc + n: source lane j points at row
            // 8g + j/4 (+4), columns 16 cc + 4 (j%4) .. +3
            const bf16 *tp = Ts + (8 * g + (n >> 2)) * L::OLD + 16 * cc + 4 * (n & 3);
            const s16x4 t_lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)tp);
            const s16x4 t_hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(tp + 4 * L::OLD));
            const bf16x8 tb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(t_lo, t_hi, 0, 1, 2, 3, 4, 5, 6, 7));
            auto row8 = [&](int row, int c0, int c1) {   // Af[row][c0 .. c0+3], Af[row][c1 .. c1+3] as bf16
                const f32x4 a = ld4(Af + row * L::FLD + c0), b = ld4(Af + row * L::FLD + c1);
                return bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3], (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
            };
            f32x4 R[2];
#pragma unroll
            for (int rp = 0; rp < 2; ++rp)
                R[rp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row8(32 + 16 * rp + n, 8 * g, 8 * g + 4), tb,
                                                               f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            // contraction over the 32 rows of R in the order the accumulators hold
            // them: slots 0..3 of group g are rows 4g .. 4g+3, slots 4..7 rows 16 + 4g ..
            const bf16x8 rb = {(bf16)R[0][0], (bf16)R[0][1], (bf16)R[0][2], (bf16)R[0][3],
                               (bf16)R[1][0], (bf16)R[1][1], (bf16)R[1][2], (bf16)R[1][3]};
            const f32x4 T21 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row8(32 + 16 * r + n, 32 + 4 * g, 48 + 4 * g), rb,
                                                                     f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) Ts[(32 + 16 * r + 4 * g + rr) * L::OLD + 16 * cc + n] = (IO)(-T21[rr]);
        } else if (ws == 0) {
            merge16(0);
            merge16(1);
            // (3) 32 -> 64: T'_21 = -T'_22 A_21 T'_11, then the column scale b
            f32x16 R2 = zero16();
#pragma unroll
            for (int s = 0; s < S32; ++s)       // R2 = A_21 T'_11 (contraction order as in ld_acc)
                R2 = M::run(ld_acc<IO>(Af, L::FLD, 32 + l32, 0, s, h32), ld_acc_t<IO>(Af, L::FLD, l32, 0, s, h32), R2);
            f32x16 T21 = zero16();
#pragma unroll
            for (int s = 0; s < S32; ++s)
                T21 = M::run(ld_acc<IO>(Af, L::FLD, 32 + l32, 32, s, h32), acc_frag<IO>(R2, s), T21);
            const float bcol = rf(FB_)[l32];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) Ts[(32 + acc_row(rr, h32)) * L::OLD + l32] = (IO)(-T21[rr] * bcol);
        }
        __syncthreads();

        if constexpr (PREP) {
            // T', P (their used blocks, as 16-byte pieces), the row factors without
            // the lazy scale and the chunk's decay scalars into its workspace slot
            static_assert(!PREP || BF, "prepared chunks are bf16");
            char *slot = p.prep + (((int64_t)item * p.prep_cps + c) * p.Hv + h) * kPrepSlot;
            for (int u = tid; u < kPrepPieces; u += 256) {
                const int row = u < 128 ? u >> 2 : 32 + ((u - 128) >> 3);
                const int pc = u < 128 ? (u & 3) : ((u - 128) & 7);
                // rows of the LDS tiles are 8-byte aligned: two 8-byte reads per piece
                const u32x2 t0 = *reinterpret_cast<const u32x2 *>(Ts + row * L::OLD + 8 * pc);
                const u32x2 t1 = *reinterpret_cast<const u32x2 *>(Ts + row * L::OLD + 8 * pc + 4);
                const u32x2 p0 = *reinterpret_cast<const u32x2 *>(Ps + row * L::OLD + 8 * pc);
                const u32x2 p1 = *reinterpret_cast<const u32x2 *>(Ps + row * L::OLD + 8 * pc + 4);
                *reinterpret_cast<i32x4 *>(slot + kPrepT + 16 * u) =
                    i32x4{(int)t0[0], (int)t0[1], (int)t1[0], (int)t1[1]};
                *reinterpret_cast<i32x4 *>(slot + kPrepP + 16 * u) =
                    i32x4{(int)p0[0], (int)p0[1], (int)p1[0], (int)p1[1]};
            }
            if (tid < 3 * C) reinterpret_cast<float *>(slot + kPrepRows)[tid] = rf(FZ_ + tid / C)[tid % C];
            if (tid == 0)
                *reinterpret_cast<f32x4 *>(slot + kPrepScalars) =
                    f32x4{gamma_l(gset), igamma_l(gset), rf(RG_)[C - 1], 0.f};
        } else {

        // ---- [D] Vnew, output and state update for this wave's 32 state rows
        //   Z' = V - FZ o (K S~^T)       Vnew = T' Z'   (T' = T diag(b))
        //   ub = FU o Vnew  (bf16 operand of the state update S~ += K^T ub)
        //   output, computed transposed (lane = token t, registers = 4 consecutive v):
        //     fast: O^T = FY_t [ (S~ Q^T) + ub^T P^T ]   (P = masked q.k, see [B]); on a
        //           renormalising chunk ub carries no 1 / sigma', so the state term
        //           enters as (S~ Q^T) sigma gamma_L and FY_t = c gamma_t rq_t / gamma_L
        //     slow: O^T = FY_t (S~ Q^T) + Vnew^T P^T
        // Z' = V - FZ o X, as the bf16 operand of Vnew = T' Z'
        frag zb[2][S32];
        {
            // bf16 V: this wave's 64 x 32 block goes through its own 4 KB of the
            // (now free) A area and comes back with transposing reads as 4
            // consecutive tokens of one column: registers 4q .. 4q+3 of tile ib.
            float vv[2][16];
            if constexpr (BF && HASV) {
                bf16 *Vw = reinterpret_cast<bf16 *>(smem + L::AF_OFF + ws * kStageBytes);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<i32x4 *>(Vw + (16 * j + (lane >> 2)) * 32 + 8 * (lane & 3)) = vwide.x[j];
                const int i = lane & 15, g16 = (lane >> 4) & 1;
                typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
#pragma unroll
                for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const bf16 *src = Vw + (32 * ib + 8 * q + 4 * h32 + (i >> 2)) * 32 + 16 * g16 + 4 * (i & 3);
                        const bf16x4 x =
                            __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)src));
#pragma unroll
                        for (int t = 0; t < 4; ++t) vv[ib][4 * q + t] = (float)x[t];
                    }
            }
            f32x4 fz[2][4];   // read as one batch (one wait instead of one per read)
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) fz[ib][jj] = ld4(rf(FZ_) + 32 * ib + 8 * jj + 4 * h32);
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int rr = 4 * jj + t;
                        X[ib][rr] = fmaf(-fz[ib][jj][t], X[ib][rr], BF && HASV ? vv[ib][rr] : vreg_at(vcur, 16 * ib + rr, BF));
                    }
                }
#pragma unroll
                for (int st = 0; st < S32; ++st) zb[ib][st] = acc_frag<IO>(X[ib], st);
            }
        }
        // Vnew = T' Z'   (T' lower block-triangular: skip the zero upper 32x32 block)
        typename M::frag tf[3][S32];   // T' blocks (0,0), (1,0), (1,1), read as one batch
#pragma unroll
        for (int s = 0; s < S32; ++s) {
            tf[0][s] = ld_acc<IO>(Ts, L::OLD, l32, 0, s, h32);
            tf[1][s] = ld_acc<IO>(Ts, L::OLD, 32 + l32, 0, s, h32);
            tf[2][s] = ld_acc<IO>(Ts, L::OLD, 32 + l32, 32, s, h32);
        }
        f32x16 Vn[2] = {zero16(), zero16()};
#pragma unroll
        for (int s = 0; s < S32; ++s) {
            Vn[0] = M::run(tf[0][s], zb[0][s], Vn[0]);
            Vn[1] = M::run(tf[1][s], zb[0][s], Vn[1]);
            Vn[1] = M::run(tf[2][s], zb[1][s], Vn[1]);
        }
        if constexpr (OUT) {
            if (!fast) {   // slow: FY_t (S~ Q^T) + Vnew^T P^T, with its own Vnew operand
                frag nb[2][S32];
#pragma unroll
                for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                    for (int s = 0; s < S32; ++s) nb[ib][s] = acc_frag<IO>(Vn[ib], s);
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const float fy = rf(FY_)[32 * ib + l32];
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) Y[ib][rr] *= fy;
#pragma unroll
                    for (int jb = 0; jb <= ib; ++jb)
#pragma unroll
                        for (int s = 0; s < S32; ++s)
                            Y[ib] = M::run(nb[jb][s], ld_acc<IO>(Ps, L::OLD, 32 * ib + l32, 32 * jb, s, h32), Y[ib]);
                }
            }
        }
        frag ub[2][S32];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            f32x4 fu[4];   // one batch per block of 32 rows
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) fu[jj] = ld4(rf(FU_) + 32 * ib + 8 * jj + 4 * h32);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int t = 0; t < 4; ++t) Vn[ib][4 * jj + t] *= fu[jj][t];
#pragma unroll
            for (int s = 0; s < S32; ++s) ub[ib][s] = acc_frag<IO>(Vn[ib], s);
        }
        if constexpr (OUT) {
            if (fast) {
                frag pfr[3][S32];   // P blocks (0,0), (1,0), (1,1), read as one batch
#pragma unroll
                for (int s = 0; s < S32; ++s) {
                    pfr[0][s] = ld_acc<IO>(Ps, L::OLD, l32, 0, s, h32);
                    pfr[1][s] = ld_acc<IO>(Ps, L::OLD, 32 + l32, 0, s, h32);
                    pfr[2][s] = ld_acc<IO>(Ps, L::OLD, 32 + l32, 32, s, h32);
                }
                if (renorm) {   // sigma and gamma_L are both normal numbers; their product may not be
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) Y[ib][rr] = (Y[ib][rr] * sigma) * gLc;
                }
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
                    for (int jb = 0; jb <= ib; ++jb)
#pragma unroll
                        for (int s = 0; s < S32; ++s) Y[ib] = M::run(ub[jb][s], pfr[ib + jb][s], Y[ib]);
                    const float fy = rf(FY_)[32 * ib + l32];
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) Y[ib][rr] *= fy;
                }
            }
            // store (rows past the chunk end fall outside the buffer range)
            if constexpr (BF) {
                // through this wave's staging block in the A area (free again), then 16
                // rows of 64 B per store instruction instead of 32 rows of 16 B
                char *st = smem + L::AF_OFF + ws * kStageBytes;
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) stage_out_tile(st, Y[ib], ib, l32, h32);
                // (read back and stored one 16-row group per step of the state update)
            } else {
                // lane = token 32 ib + l32, registers 4q..4q+3 = v 32 ws + 8q + 4 h32 + 0..3
                constexpr int ES = (int)sizeof(IO);
                const auto ro = rsrc(p.out + ch.t0 * p.o_st + h * p.o_sh, (Lc - 1) * p.o_st + D * ES);
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const int base = (32 * ib + l32) * p.o_st + (32 * ws + 4 * h32) * ES;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4 f4 = {Y[ib][4 * q], Y[ib][4 * q + 1], Y[ib][4 * q + 2], Y[ib][4 * q + 3]};
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, f4), ro, base + 8 * q * ES, 0, 0);
                    }
                }
            }
        }
        if (renorm) {
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) S[bb][rr] *= sig_next;
            sigma = 1.f;
        } else {
            sigma = sig_next;
        }
        {   // S~ += K^T ub: the four state tiles are independent chains; the K^T
            // fragments of the next contraction step are read while this step runs
            constexpr int NU = 2 * S32;
            frag kt[2][4];
            auto load_kt = [&](int k, frag (&f)[4]) {
                const int ib = k / S32, st = k % S32;
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    if constexpr (BF) f[bb] = ld_acc_tr(Ks, 32 * bb, 32 * ib, st, lane);
                    else f[bb] = ld_acc_t<float>(Ks, L::KLD, 32 * bb + l32, 32 * ib, st, h32);
                }
            };
            load_kt(0, kt[0]);
#pragma unroll
            for (int k = 0; k < NU; ++k) {
                const int cur = k & 1;
                if (k + 1 < NU) load_kt(k + 1, kt[cur ^ 1]);
                if constexpr (OUT && BF) {   // output rows 16k .. 16k+15 of this wave's columns
                    const char *st = smem + L::AF_OFF + ws * kStageBytes;
                    const auto ro = rsrc(p.out + ch.t0 * p.o_st + h * p.o_sh, (Lc - 1) * p.o_st + D * 2);
                    const int gq = lane & 3, t = 16 * k + (lane >> 2);
                    const i32x4 o16 = staged_out(st, t, gq);
                    __builtin_amdgcn_raw_buffer_store_b128(o16, ro, t * p.o_st + (32 * ws + 8 * gq) * 2, 0, 0);
                }
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) S[bb] = M::run(kt[cur][bb], ub[k / S32][k % S32], S[bb]);
            }
        }
        // ---- state checkpoint at a full chunk that ends on a checkpoint boundary:
        // the lazy scale is folded into the state first (a renorm), then stored
        if constexpr (CK) {
            const int done = seq_chunk0 + c + 1;
            if (Lc == C && done % p.ck_every == 0 && done / p.ck_every <= p.ck_per_seq) {
                if (sigma != 1.f) {
#pragma unroll
                    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) S[bb][rr] *= sigma;
                    sigma = 1.f;
                }
                const int64_t slot = (int64_t)n * p.ck_per_seq + done / p.ck_every - 1;
                store_state<BF>(S, p.ck + slot * p.ck_n + h * p.ck_h, p.ck_v, p.ck_dt, v0, h32);
            }
        }
        }   // !PREP
        __syncthreads();
    }

    // ---- final state (scan: the caller's output state, by the last segment only;
    // maps: the workspace)
    const bool write_caller = MODE == kScan && last && p.s_out && srow >= 0;
    if (write_caller || MODE == kMapN || MODE == kMapM) {
        if (sigma != 1.f) {
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) S[bb][rr] *= sigma;
        }
        const int tid = threadIdx.x, lane = tid & 63, ws = tid >> 6;
        const int h32 = lane >> 5, v0 = ws * 32 + (lane & 31);
        if (MODE == kScan)
            store_state<BF>(S, p.s_out + srow * p.so_n + h * p.so_h, p.so_v, p.so_dt, v0, h32);
        else
            store_state<BF>(S, reinterpret_cast<char *>(MODE == kMapN ? p.ws_n : p.ws_m) + map_off, D * 4, GDN_F32, v0,
                        h32);
    }
}


template <typename IO, int MODE>
hipError_t launch(const ScanParams &p, hipStream_t stream) {
    const int64_t items = p.segs ? p.seg_cap : p.N;
    const int64_t pairs = items * p.Hqk;
    const int64_t blocks = ((pairs + 7) / 8) * 8 * p.r;
    if (blocks == 0) return hipSuccess;
    if (MODE == kScan && p.ck)   // the scan that also writes state checkpoints
        hipLaunchKernelGGL((fused_scan_kernel<IO, kScan, true>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((fused_scan_kernel<IO, MODE, false>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prep(const ScanParams &p, hipStream_t stream) { return launch<bf16, kPrep>(p, stream); }

hipError_t launch_fused_scan(const ScanParams &p, bool io_bf16, int mode, hipStream_t stream) {
    if (io_bf16) {
        if (mode == kMapN) return launch<bf16, kMapN>(p, stream);
        if (mode == kMapM) return launch<bf16, kMapM>(p, stream);
        return launch<bf16, kScan>(p, stream);
    }
    if (mode == kMapN) return launch<float, kMapN>(p, stream);
    if (mode == kMapM) return launch<float, kMapM>(p, stream);
    return launch<float, kScan>(p, stream);
}

}  // namespace gdn
