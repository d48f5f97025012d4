// Pipelined chunked gated delta rule scan for gfx950: one workgroup of eight
// waves per (sequence, value head), for launches that leave CUs to spare.
//
// The method and every per-element step are those of the four-wave scan in
// gdn_scan.hip ("flashinfer.gdn_prefill", the chunked GDN scan; arguments as in
// "flashinfer.cudnn.cudnn_chunk_gated_delta_rule", Parameters): the same MFMA
// products in the same accumulation order, the same row factors, inverses and
// merges, so the two kernels give bitwise-identical results and either may run
// a given work item.  What differs is the schedule.  A chunk's work splits into
//   preparation  (needs only q, k, g, beta): Gram tiles and row norms, the
//                formation of A and P, the four 16x16 diagonal inverses and the
//                16 -> 32 -> 64 merges giving T', the row factors;
//   state work   (needs the state): K S~^T and S~ Q^T, Z', Vnew = T' Z', the
//                output and the state update.
// In the four-wave kernel both run one after the other on the same waves, so a
// chunk costs the sum of the two chains (~11.9 K cycles with one workgroup per
// CU).  Here waves 4..7 prepare chunk c + 1 while waves 0..3 (each owning 32
// state rows, as before) run the state work of chunk c; K, Q, P, T' and the
// row factors are double-buffered by chunk parity.  Each SIMD holds one wave
// of each role, so one role's MFMA and LDS latencies overlap the other's work.
// The iteration's five barrier intervals and what fills them are listed at the
// role loops below; one iteration takes ~9.8 K cycles (measured per interval
// with s_memtime), bound by the preparation's chain of five dependent steps.
//
// 147.5 KB of LDS, so one workgroup per CU: chosen when the launch has at most
// one work item per CU.  With more, two four-wave workgroups per CU overlap
// in the same way and the part runs at its power limit, where the extra LDS
// reads of the separate Gram pass would cost.  bf16 q/k/v only, no
// checkpoints, not in the split path's map modes.
#include <hip/hip_runtime.h>

#include "gdn_device.h"

namespace gdn {
namespace {

using namespace dev;

struct PipedSmem {
    static constexpr int KLD = kKqLd;   // K, Q rows (bf16, rows permuted, see kq_row)
    static constexpr int OLD = 68;      // T', P rows (bf16)
    static constexpr int FLD = 68;      // fp32 64x64 work matrix (A, inverse blocks)
    static constexpr int KB = C * KLD * 2;
    static constexpr int OB = C * OLD * 2;
    static constexpr int K_OFF = 0;                   // [2] by chunk parity
    static constexpr int Q_OFF = K_OFF + 2 * KB;      // [2]
    static constexpr int P_OFF = Q_OFF + 2 * KB;      // [2]
    static constexpr int T_OFF = P_OFF + 2 * OB;      // [2]
    static constexpr int AF_OFF = T_OFF + 2 * OB;
    static constexpr int VO_OFF = AF_OFF + C * FLD * 4;   // a staging block per state wave: V in, output out
    static constexpr int NTS = 16 * 16 + 4;
    static constexpr int NT_OFF = VO_OFF + 4 * kStageBytes;
    static constexpr int ROW_OFF = NT_OFF + 4 * NTS * 4;  // row factors, [2] sets by chunk parity
    static constexpr int BYTES = ROW_OFF + (2 * NROWF * C + 4) * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(Q_OFF % 16 == 0 && P_OFF % 16 == 0 && T_OFF % 16 == 0 && AF_OFF % 16 == 0 &&
                  VO_OFF % 16 == 0 && NT_OFF % 16 == 0 && ROW_OFF % 16 == 0, "align");
};

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void piped_scan_kernel(
    const ScanParams p) {
    using L = PipedSmem;
    using M = Mma<bf16>;
    using frag = M::frag;
    constexpr int S32 = 2;   // 32x32x16 steps per 32-wide contraction block

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    float *Af = reinterpret_cast<float *>(smem + L::AF_OFF);
    float *NT = reinterpret_cast<float *>(smem + L::NT_OFF);
    float *RF = reinterpret_cast<float *>(smem + L::ROW_OFF);
    // buffers of chunk x (by parity)
    auto kbuf = [&](int x) { return reinterpret_cast<bf16 *>(smem + L::K_OFF + (x & 1) * L::KB); };
    auto qbuf = [&](int x) { return reinterpret_cast<bf16 *>(smem + L::Q_OFF + (x & 1) * L::KB); };
    auto pbuf = [&](int x) { return reinterpret_cast<bf16 *>(smem + L::P_OFF + (x & 1) * L::OB); };
    auto tbuf = [&](int x) { return reinterpret_cast<bf16 *>(smem + L::T_OFF + (x & 1) * L::OB); };
    auto rows = [&](int which, int x) { return RF + ((x & 1) * NROWF + which) * C; };
    auto gamma_l = [&](int x) -> float & { return RF[2 * NROWF * C + (x & 1)]; };
    auto igamma_l = [&](int x) -> float & { return RF[2 * NROWF * C + 2 + (x & 1)]; };   // 1 / gamma_L

    // ---- work item (XCD-aware as in the four-wave scan)
    const int r = p.r;
    const int b = blockIdx.x;
    const int within = b % (8 * r);
    const int pidx = (b / (8 * r)) * 8 + (within & 7);
    if (pidx >= p.N * p.Hqk) return;
    const int n = pidx / p.Hqk, hq = pidx % p.Hqk;
    const int h = hq * r + (within >> 3);
    const int64_t bos = load_cu(p.cu, n, p.cu_i64), eos = load_cu(p.cu, n + 1, p.cu_i64);
    const int64_t srow = state_row(p.sidx, p.sidx_i64, p.pool_rows, n);
    const int nchunks = (int)((eos - bos + C - 1) / C);
    const int ws0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool is_state = ws0 < 4;

    // Gate rows of chunk x into its set, on the gate wave (lane = token).
    auto gate_rows = [&](const Prefetch<bf16> &g, int Lch, int x, int lane) {
        const bool valid = lane < Lch;
        const float ga = p.g ? gate_value(g.g, p.g_dt) : 1.f;
        const float gb = p.beta ? gate_value(g.b, p.b_dt) : 1.f;
        const float G = wave_prefix_sum(valid ? fmaxf(__logf(ga), -80.f) : 0.f);
        const float GL = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 63));
        const float gam = __expf(G);
        rows(RG_, x)[lane] = G;
        rows(GM_, x)[lane] = gam;
        rows(IG_, x)[lane] = __expf(-G);
        rows(DC_, x)[lane] = __expf(GL - G);
        rows(FB_, x)[lane] = valid ? gb : 0.f;
        gamma_l(x) = __expf(GL);
        igamma_l(x) = __expf(-GL);
    };
    // The preparation wave that loads the gates and forms the gate rows.  Its gate
    // loads of chunk c + 3 go out in interval 5 after its K, Q loads of that chunk,
    // where the wave's A(1,1) pass leaves time for them: queued behind the other
    // waves' 16-byte loads for the memory unit's address processing, the two small
    // loads hold the issuing wave ~500 cycles, and issued later (intervals 3, 4)
    // they also became part of the wait before the K, Q staging of interval 4.
    constexpr int kGateW = 4 + kGateWave;

    // State waves: S[b] holds S~^T rows k in natural operand order, column v0.
    // pf: the preparation waves' K, Q and gate prefetch; the state waves keep the
    // next chunk's V in pf.kq[0] (16-byte loads, as VWide).
    f32x16 S[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) S[bb] = zero16();
    Prefetch<bf16> pf;
    if (is_state) {
        const int lane = threadIdx.x & 63, h32 = lane >> 5, v0 = ws0 * 32 + (lane & 31);
        if (p.s_in && srow >= 0)
            load_state<true>(S, p.s_in + srow * p.si_n + h * p.si_h, p.si_v, p.si_dt, v0, h32);
    } else if (nchunks > 0) {
        const int tp = threadIdx.x - 256, lane = threadIdx.x & 63;
        issue_loads<bf16>(pf, p, chunk_at(bos, eos, 0), hq, h, tp, lane, ws0);
        if (ws0 == kGateW) issue_gates(pf, p, chunk_at(bos, eos, 0), h, lane);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        const int rq4 = tp >> 4, cg = tp & 15;
#pragma unroll
        for (int mat = 0; mat < 2; ++mat)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                *reinterpret_cast<i32x4 *>((mat ? qbuf(0) : kbuf(0)) + kq_off(4 * rq4 + t, 8 * cg)) = pf.kq[mat][t];
        if (ws0 == kGateW) gate_rows(pf, chunk_at(bos, eos, 0).L, 0, lane);
        if (nchunks > 1) {
            issue_loads<bf16>(pf, p, chunk_at(bos, eos, 1), hq, h, tp, lane, ws0);
            if (ws0 == kGateW) issue_gates(pf, p, chunk_at(bos, eos, 1), h, lane);
        }
    }
    __syncthreads();

    // The two roles run separate loops with the same barriers (one more before
    // the loop, five per iteration), so each role's registers are allocated for
    // its own code only.  Iteration c:
    //   interval  state waves                             preparation waves
    //   1         V staging, Z', Vnew, ub of chunk c      A and P of chunk c + 1, row factors
    //   2         output products and staging (c)         diagonal inverses (c + 1)
    //   3         output stores, state update (c);        16 -> 32 merges (c + 1); gate rows of c + 2
    //             V loads of chunk c + 1
    //   4         K S~^T, S~ Q^T of chunk c + 1           32 -> 64 merge (c + 1); K, Q of c + 2 staged
    //   5         -                                       Gram tiles and norms of chunk c + 2
    // sigma: scale of the true state (sigma S~) at the start of the wave's chunk;
    // the preparation waves track it one chunk ahead with the same arithmetic.
    if (is_state) {
        float sigma = 1.f;
        f32x16 X[2] = {zero16(), zero16()}, Y[2] = {zero16(), zero16()};
        // X = K S~^T and Y = S~ Q^T of chunk x over contraction steps k0 .. k0 + 3
        // (the next step's fragments read while the current one runs)
        auto xy_half = [&](auto k0c, int x, int lane) {
            constexpr int k0 = decltype(k0c)::value;
            const int h32 = lane >> 5, l32 = lane & 31;
            const bf16 *Ks = kbuf(x), *Qs = qbuf(x);
            frag fk[2][2], fq[2][2];
            auto load = [&](int k, int st) {
                fk[st][0] = ld_kq(Ks, l32, k, h32);
                fk[st][1] = ld_kq(Ks, 32 + l32, k, h32);
                fq[st][0] = ld_kq(Qs, l32, k, h32);
                fq[st][1] = ld_kq(Qs, 32 + l32, k, h32);
            };
            load(k0, 0);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int k = k0 + kk, cur = kk & 1;
                if (kk + 1 < 4) load(k + 1, cur ^ 1);
                const frag sf = acc_frag<bf16>(S[k / S32], k % S32);
                X[0] = M::run(fk[cur][0], sf, X[0]);
                X[1] = M::run(fk[cur][1], sf, X[1]);
                Y[0] = M::run(sf, fq[cur][0], Y[0]);
                Y[1] = M::run(sf, fq[cur][1], Y[1]);
            }
        };
        __syncthreads();   // (the preparation's Gram tiles of chunk 0)
        for (int c = -1; c < nchunks; ++c) {
            int tid_o = threadIdx.x;
            asm volatile("" : "+v"(tid_o));
            const int tid = tid_o, lane = tid & 63;
            const int ws = __builtin_amdgcn_readfirstlane(tid >> 6);
            const int h32 = lane >> 5, l32 = lane & 31;
            const bool on = c >= 0;
            auto rf = [&](int which) { return rows(which, c); };
            const float gLc =
                __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, gamma_l(c))));
            const float sig_next = sigma * gLc;
            const bool renorm = !(sig_next >= kRenorm);
            const bool fast = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(
                                  int, rf(RG_)[C - 1]))) > kFastDecay;
            const ChunkRef ch = chunk_at(bos, eos, c);
            const int Lc = ch.L;
            const bf16 *Ks = kbuf(c);
            char *st = smem + L::VO_OFF + ws * kStageBytes;
            bf16 *Vw = reinterpret_cast<bf16 *>(st);

            // ---- interval 1: Z' = V - FZ o X, Vnew = T' Z', ub = FU o Vnew (slow
            // path: the output products with their own Vnew operand)
            frag ub[2][S32];
            if (on) {
                frag zb[2][S32];
                {
                    // V through this wave's staging block, back as 4 consecutive tokens of one
                    // column (transposing reads): registers 4q .. 4q+3 of tile ib
                    float vv[2][16];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *reinterpret_cast<i32x4 *>(Vw + (16 * j + (lane >> 2)) * 32 + 8 * (lane & 3)) = pf.kq[0][j];
                    const int i = lane & 15, g16 = (lane >> 4) & 1;
                    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const bf16 *src = Vw + (32 * ib + 8 * q + 4 * h32 + (i >> 2)) * 32 + 16 * g16 + 4 * (i & 3);
                            const bf16x4 xv =
                                __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)src));
#pragma unroll
                            for (int t = 0; t < 4; ++t) vv[ib][4 * q + t] = (float)xv[t];
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
                                X[ib][rr] = fmaf(-fz[ib][jj][t], X[ib][rr], vv[ib][rr]);
                            }
                        }
#pragma unroll
                        for (int st = 0; st < S32; ++st) zb[ib][st] = acc_frag<bf16>(X[ib], st);
                    }
                }
                const bf16 *Ts = tbuf(c), *Ps = pbuf(c);
                // Vnew = T' Z'   (T' lower block-triangular: the upper 32x32 block is zero)
                frag tf[3][S32];   // T' blocks (0,0), (1,0), (1,1), read as one batch
#pragma unroll
                for (int s = 0; s < S32; ++s) {
                    tf[0][s] = ld_acc<bf16>(Ts, L::OLD, l32, 0, s, h32);
                    tf[1][s] = ld_acc<bf16>(Ts, L::OLD, 32 + l32, 0, s, h32);
                    tf[2][s] = ld_acc<bf16>(Ts, L::OLD, 32 + l32, 32, s, h32);
                }
                f32x16 Vn[2] = {zero16(), zero16()};
#pragma unroll
                for (int s = 0; s < S32; ++s) {
                    Vn[0] = M::run(tf[0][s], zb[0][s], Vn[0]);
                    Vn[1] = M::run(tf[1][s], zb[0][s], Vn[1]);
                    Vn[1] = M::run(tf[2][s], zb[1][s], Vn[1]);
                }
                if (!fast) {   // FY_t (S~ Q^T) + Vnew^T P^T, with its own Vnew operand
                    frag nb[2][S32];
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                        for (int s = 0; s < S32; ++s) nb[ib][s] = acc_frag<bf16>(Vn[ib], s);
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) {
                        const float fy = rf(FY_)[32 * ib + l32];
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) Y[ib][rr] *= fy;
#pragma unroll
                        for (int jb = 0; jb <= ib; ++jb)
#pragma unroll
                            for (int s = 0; s < S32; ++s)
                                Y[ib] = M::run(nb[jb][s], ld_acc<bf16>(Ps, L::OLD, 32 * ib + l32, 32 * jb, s, h32),
                                               Y[ib]);
                    }
                }
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
                    for (int s = 0; s < S32; ++s) ub[ib][s] = acc_frag<bf16>(Vn[ib], s);
                }
            }
            __syncthreads();

            // ---- interval 2: fast path output O^T = FY_t [S~ Q^T + ub^T P^T] (a
            // renormalising chunk: the state term as (S~ Q^T) sigma gamma_L, and FY_t
            // with 1 / gamma_L); the output tile staged through this wave's 4 KB: rows
            // t of its 32 columns (64 B), 16-byte granules of row t rotated by
            // (t / 4) % 4 against bank conflicts
            if (on) {
                if (fast) {
                    if (renorm) {   // sigma and gamma_L are both normal numbers; their product may not be
#pragma unroll
                        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                            for (int rr = 0; rr < 16; ++rr) Y[ib][rr] = (Y[ib][rr] * sigma) * gLc;
                    }
                    const bf16 *Ps = pbuf(c);
                    frag pfr[3][S32];   // P blocks (0,0), (1,0), (1,1), read as one batch
#pragma unroll
                    for (int s = 0; s < S32; ++s) {
                        pfr[0][s] = ld_acc<bf16>(Ps, L::OLD, l32, 0, s, h32);
                        pfr[1][s] = ld_acc<bf16>(Ps, L::OLD, 32 + l32, 0, s, h32);
                        pfr[2][s] = ld_acc<bf16>(Ps, L::OLD, 32 + l32, 32, s, h32);
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
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) stage_out_tile(st, Y[ib], ib, l32, h32);
            }
            __syncthreads();

            // ---- interval 3: S~ += K^T ub (after the renorm fold), one 16-row group
            // of output stores per step; then the next chunk's V
            if (on) {
                if (renorm) {
#pragma unroll
                    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) S[bb][rr] *= sig_next;
                }
                constexpr int NU = 2 * S32;
                frag kt[2][4];
                auto load_kt = [&](int k, frag (&f)[4]) {
                    const int ib = k / S32, st = k % S32;
#pragma unroll
                    for (int bb = 0; bb < 4; ++bb) f[bb] = ld_acc_tr(Ks, 32 * bb, 32 * ib, st, lane);
                };
                const auto ro = rsrc(p.out + ch.t0 * p.o_st + h * p.o_sh, (Lc - 1) * p.o_st + D * 2);
                load_kt(0, kt[0]);
#pragma unroll
                for (int k = 0; k < NU; ++k) {
                    const int cur = k & 1;
                    if (k + 1 < NU) load_kt(k + 1, kt[cur ^ 1]);
                    const int gq = lane & 3, t = 16 * k + (lane >> 2);
                    const i32x4 o16 = staged_out(st, t, gq);
                    __builtin_amdgcn_raw_buffer_store_b128(o16, ro, t * p.o_st + (32 * ws + 8 * gq) * 2, 0, 0);
#pragma unroll
                    for (int bb = 0; bb < 4; ++bb) S[bb] = M::run(kt[cur][bb], ub[k / S32][k % S32], S[bb]);
                }
            }
            if (c + 1 < nchunks) {   // as issue_v_wide_part, into pf.kq[0]
                const ChunkRef nx = chunk_at(bos, eos, c + 1);
                const auto rv = rsrc(p.v + nx.t0 * p.v_st + h * p.v_sh, (nx.L - 1) * p.v_st + D * 2);
                const int vo = (lane >> 2) * p.v_st + (32 * ws + 8 * (lane & 3)) * 2;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    pf.kq[0][j] = __builtin_amdgcn_raw_buffer_load_b128(rv, vo + 16 * j * p.v_st, 0, 0);
            }
            __syncthreads();

            // ---- interval 4: X and Y of chunk c + 1 from the updated state (interval 5
            // leaves the LDS to the preparation's Gram pass)
            if (c + 1 < nchunks) {
                X[0] = X[1] = Y[0] = Y[1] = zero16();
                xy_half(std::integral_constant<int, 0>{}, c + 1, lane);
                xy_half(std::integral_constant<int, 4>{}, c + 1, lane);
            }
            __syncthreads();
            __syncthreads();
            if (on) sigma = renorm ? 1.f : sig_next;
        }

        // ---- final state
        if (p.s_out && srow >= 0) {
            if (sigma != 1.f) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb)
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) S[bb][rr] *= sigma;
            }
            const int lane = threadIdx.x & 63, h32 = lane >> 5, v0 = ws0 * 32 + (lane & 31);
            store_state<true>(S, p.s_out + srow * p.so_n + h * p.so_h, p.so_v, p.so_dt, v0, h32);
        }
    } else {
        float sigma = 1.f;
        const int pw = ws0 & 3;   // role within the preparation waves
        // Gram tiles of the chunk being prepared (transposed: lane = row i,
        // registers = column j), kept from interval 5 to the next interval 1
        f32x16 X[2] = {zero16(), zero16()};
        // Gram tiles and row norms of chunk x; tiles as in the four-wave scan:
        // 0: A(0,0) (even / odd steps), norms of K_0 and Q_1; 1: A(1,0), P(1,1),
        // norm of K_1; 2: A(1,1) (even / odd); 3: P(0,0), P(1,0), norm of Q_0
        auto gram = [&](int x, int lane) {
            const int h32 = lane >> 5, l32 = lane & 31;
            const bf16 *Ks = kbuf(x), *Qs = qbuf(x);
            // 1 / |row| (or 1 without the norm); a K row's factor also goes into
            // its 1 / gamma entry, which only the A tiles read
            auto put_norm = [&](float ss, int which, int blk) {
                ss += __shfl_xor(ss, 32);
                if (h32 == 0) {
                    const int row = 32 * blk + l32;
                    const float rr = p.l2norm ? __builtin_amdgcn_rsqf(ss + 1e-6f) : 1.f;
                    rows(which, x)[row] = rr;
                    if (which == RK_) rows(IG_, x)[row] *= rr;
                }
            };
            X[0] = X[1] = zero16();
            auto pass = [&](auto role) {
                constexpr int R = decltype(role)::value;
                constexpr int NK = 4 * S32;
                frag fa[2][3];
                auto load = [&](int k, int st) {
                    if constexpr (R == 0) {
                        fa[st][0] = ld_kq(Ks, l32, k, h32);
                        fa[st][1] = ld_kq(Qs, 32 + l32, k, h32);
                    } else if constexpr (R == 1) {
                        fa[st][0] = ld_kq(Ks, l32, k, h32);
                        fa[st][1] = ld_kq(Ks, 32 + l32, k, h32);
                        fa[st][2] = ld_kq(Qs, 32 + l32, k, h32);
                    } else if constexpr (R == 2) {
                        fa[st][0] = ld_kq(Ks, 32 + l32, k, h32);
                    } else {
                        fa[st][0] = ld_kq(Ks, l32, k, h32);
                        fa[st][1] = ld_kq(Qs, l32, k, h32);
                        fa[st][2] = ld_kq(Qs, 32 + l32, k, h32);
                    }
                };
                float ssa = 0.f, ssb = 0.f;
                load(0, 0);
#pragma unroll
                for (int k = 0; k < NK; ++k) {
                    const int cur = k & 1;
                    if (k + 1 < NK) load(k + 1, cur ^ 1);
                    if constexpr (R == 0) {   // k0, q1
                        X[cur] = M::run(fa[cur][0], fa[cur][0], X[cur]);
                        ssa = sumsq8_acc(fa[cur][0], ssa);
                        ssb = sumsq8_acc(fa[cur][1], ssb);
                    } else if constexpr (R == 1) {   // k0, k1, q1
                        X[0] = M::run(fa[cur][0], fa[cur][1], X[0]);
                        ssa = sumsq8_acc(fa[cur][1], ssa);
                        X[1] = M::run(fa[cur][1], fa[cur][2], X[1]);
                    } else if constexpr (R == 2) {   // k1
                        X[cur] = M::run(fa[cur][0], fa[cur][0], X[cur]);
                    } else {   // k0, q0, q1
                        X[0] = M::run(fa[cur][0], fa[cur][1], X[0]);
                        X[1] = M::run(fa[cur][0], fa[cur][2], X[1]);
                        ssb = sumsq8_acc(fa[cur][1], ssb);
                    }
                }
                if constexpr (R == 0) {
                    X[0] += X[1];
                    put_norm(ssa, RK_, 0);
                    put_norm(ssb, RQ_, 1);
                } else if constexpr (R == 1) {
                    put_norm(ssa, RK_, 1);
                } else if constexpr (R == 2) {
                    X[0] += X[1];
                } else {
                    put_norm(ssb, RQ_, 0);
                }
            };
            if (pw == 0) pass(std::integral_constant<int, 0>{});
            else if (pw == 1) pass(std::integral_constant<int, 1>{});
            else if (pw == 2) pass(std::integral_constant<int, 2>{});
            else pass(std::integral_constant<int, 3>{});
        };
        if (nchunks > 0) gram(0, threadIdx.x & 63);
        // gamma_L and the last log-gate cumsum of the chunk the next iteration
        // prepares, read one interval early (with the LDS still free of the state
        // waves' V staging that opens interval 1)
        auto uniform_f = [](float v) {
            return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
        };
        float gl_next = 1.f, glog_next = 0.f;
        if (nchunks > 0) {
            gl_next = uniform_f(gamma_l(0));
            glog_next = uniform_f(rows(RG_, 0)[C - 1]);
        }
        __syncthreads();
        for (int c = -1; c < nchunks; ++c) {
            int tid_o = threadIdx.x;
            asm volatile("" : "+v"(tid_o));
            const int tid = tid_o, lane = tid & 63;
            const int ws = __builtin_amdgcn_readfirstlane(tid >> 6);
            const int h32 = lane >> 5, l32 = lane & 31;
            const int x = c + 1;   // the chunk being prepared
            const bool on = x < nchunks, on2 = c + 2 < nchunks;
            auto rf = [&](int which) { return rows(which, x); };
            const float gLc = gl_next;
            const float sig_next = sigma * gLc;
            const bool renorm = !(sig_next >= kRenorm);
            const bool fast = glog_next > kFastDecay;
            bf16 *Ts = tbuf(x);

            // ---- interval 1: A (fp32) and P of chunk x from the Gram tiles, row
            // factors of the state work.  Lane row i = 32 bi + l32; register 4 jj + t
            // is column j = 32 bj + 8 jj + 4 h32 + t.
            //   A = b_i rk_i rk_j (k_i . k_j) exp(G_i - G_j)   for j < i   (fp32)
            //   P = c rq_i rk_j (q_i . k_j) exp(G_i - G_j)      for j <= i  (slow)
            //   P = q_i . k_j                                  for j <= i  (fast)
            if (on) {
                bf16 *Ps = pbuf(x);
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
                            for (int t = 0; t < 4; ++t) nt[(8 * jr + 4 * h32 + t) * 16] = hi ? v[2 + jr][t] : v[jr][t];
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
                        const bf16x4 b4 = {(bf16)v[jj][0], (bf16)v[jj][1], (bf16)v[jj][2], (bf16)v[jj][3]};
                        *reinterpret_cast<bf16x4 *>(Ps + i * L::OLD + jb + 8 * jj) = b4;
                    }
                };
                if (pw < 3) a_tile(X[0], pw > 0, pw == 2);
                if (pw == 3) {
                    p_tile(X[0], 0, 0);
                    p_tile(X[1], 1, 0);
                }
                if (pw == 1) p_tile(X[1], 1, 1);
                if (pw == 3) {   // row factors of the state work (the wave with no A tile), lane = token
                    const float rk = rf(RK_)[lane], gam = rf(GM_)[lane], dec = rf(DC_)[lane];
                    rf(FZ_)[lane] = sigma * (gam * rk);
                    rf(FU_)[lane] = renorm ? rk * dec : (rk * dec) / sig_next;
                    const float base = (p.scale * gam) * rf(RQ_)[lane];
                    rf(FY_)[lane] = fast && renorm ? base * igamma_l(x) : sigma * base;
                }
            }
            __syncthreads();

            // ---- interval 2: D = (I + N)^-1 for the strictly lower 16x16 diagonal
            // block N of rows 16 pw .. 16 pw + 15, by forward substitution (lane =
            // column cc and row class rq; the pivot is broadcast inside the lane quad)
            if (on) {
                const int cc = lane >> 2, rq = lane & 3;
                const float *nt = NT + pw * L::NTS + 4 * rq;
                float xs[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) xs[k] = rq + 4 * k == cc ? 1.f : 0.f;
                // all 15 columns in one batch, so that no step of the chain waits on the
                // read of its column (one step ahead measured the same on its own)
                f32x4 ncol[15];
#pragma unroll
                for (int m = 0; m < 15; ++m) ncol[m] = ld4(nt + m * 16);
#pragma unroll
                for (int m = 0; m < 15; ++m) {
                    const float xm = quad_bcast(xs[m >> 2], m & 3);
#pragma unroll
                    for (int k = 0; k < 4; ++k) xs[k] = fmaf(-ncol[m][k], xm, xs[k]);
                }
                const float bcol = rf(FB_)[16 * pw + cc];
                float *blk = Af + (16 * pw) * L::FLD + 16 * pw;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int i = rq + 4 * k;
                    blk[i * L::FLD + cc] = xs[k];
                    Ts[(16 * pw + i) * L::OLD + 16 * pw + cc] = (bf16)(xs[k] * bcol);
                    if ((pw & 1) == 0) Ts[(16 * pw + i) * L::OLD + 16 * pw + 16 + cc] = (bf16)0.f;
                }
            }
            __syncthreads();

            // ---- interval 3: 16 -> 32 merges (waves 4, 5): T'_{2x+1,2x} =
            // -D_{2x+1} A_{2x+1,2x} D_{2x}; the gate rows of chunk c + 2 (their row
            // set was last read by the state work of chunk c)
            if (on && pw < 2) {
                const int g = lane >> 4, nn = lane & 15;
                const int lo = 32 * pw, hi = 32 * pw + 16;
                f32x4 R = {0.f, 0.f, 0.f, 0.f};
                R = M::run16(ld16_row<bf16>(Af, L::FLD, hi + nn, lo, 0, g), ld16_col<bf16>(Af, L::FLD, lo + nn, lo, 0, g),
                             R);
                const float bcol = rf(FB_)[lo + nn];
                f32x4 Tq = {0.f, 0.f, 0.f, 0.f};
                Tq = M::run16(ld16_row<bf16>(Af, L::FLD, hi + nn, hi, 0, g), acc16_frag<bf16>(R, 0), Tq);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int i = hi + 4 * g + rr;
                    Af[i * L::FLD + lo + nn] = -Tq[rr];
                    Ts[i * L::OLD + lo + nn] = (bf16)(-Tq[rr] * bcol);
                }
            }
            if (on2 && ws == kGateW) gate_rows(pf, chunk_at(bos, eos, c + 2).L, c + 2, lane);
            __syncthreads();

            // ---- interval 4: 32 -> 64 merge on the four waves, wave (r, cc) forming
            // block (r, cc) of T''_21 = -T'_22 A_21 T''_11 (T''_11 read as its
            // column-scaled copy with transposing loads); K and Q of chunk c + 2
            // staged (their buffers were last read by the state update of chunk c),
            // half of the K, Q loads of chunk c + 3
            if (on) {
                const int rr2 = pw >> 1, cc = pw & 1;
                const int g = lane >> 4, nn = lane & 15;
                typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
                const bf16 *tp = Ts + (8 * g + (nn >> 2)) * L::OLD + 16 * cc + 4 * (nn & 3);
                const s16x4 t_lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)tp);
                const s16x4 t_hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(tp + 4 * L::OLD));
                const bf16x8 tb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(t_lo, t_hi, 0, 1, 2, 3, 4, 5, 6, 7));
                auto row8 = [&](int row, int c0, int c1) {
                    const f32x4 a = ld4(Af + row * L::FLD + c0), bq = ld4(Af + row * L::FLD + c1);
                    return bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3], (bf16)bq[0], (bf16)bq[1], (bf16)bq[2],
                                  (bf16)bq[3]};
                };
                f32x4 R[2];
#pragma unroll
                for (int rp = 0; rp < 2; ++rp)
                    R[rp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row8(32 + 16 * rp + nn, 8 * g, 8 * g + 4), tb,
                                                                   f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                const bf16x8 rb = {(bf16)R[0][0], (bf16)R[0][1], (bf16)R[0][2], (bf16)R[0][3],
                                   (bf16)R[1][0], (bf16)R[1][1], (bf16)R[1][2], (bf16)R[1][3]};
                const f32x4 T21 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row8(32 + 16 * rr2 + nn, 32 + 4 * g, 48 + 4 * g),
                                                                         rb, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                for (int q = 0; q < 4; ++q) Ts[(32 + 16 * rr2 + 4 * g + q) * L::OLD + 16 * cc + nn] = (bf16)(-T21[q]);
            }
            const int tp = tid - 256;
            if (on2) {
                const int rq4 = tp >> 4, cg = tp & 15;
#pragma unroll
                for (int mat = 0; mat < 2; ++mat)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        *reinterpret_cast<i32x4 *>((mat ? qbuf(c + 2) : kbuf(c + 2)) + kq_off(4 * rq4 + t, 8 * cg)) =
                            pf.kq[mat][t];
            }
            if (c + 3 < nchunks) {
                issue_kq_part(pf, p, chunk_at(bos, eos, c + 3), hq, tp, 0);
                issue_kq_part(pf, p, chunk_at(bos, eos, c + 3), hq, tp, 1);
            }
            __syncthreads();

            // ---- interval 5: Gram tiles and norms of chunk c + 2 (its gamma_L and last
            // log-gate cumsum for the next iteration); the other half of the K, Q loads
            // and the gate loads of chunk c + 3
            if (on2) {
                gl_next = uniform_f(gamma_l(c + 2));
                glog_next = uniform_f(rows(RG_, c + 2)[C - 1]);
                gram(c + 2, lane);
            }
            if (c + 3 < nchunks) {
                issue_kq_part(pf, p, chunk_at(bos, eos, c + 3), hq, tp, 2);
                issue_kq_part(pf, p, chunk_at(bos, eos, c + 3), hq, tp, 3);
                if (ws == kGateW) issue_gates(pf, p, chunk_at(bos, eos, c + 3), h, lane);
            }
            __syncthreads();
            if (on) sigma = renorm ? 1.f : sig_next;
        }
    }
}

}  // namespace

hipError_t launch_piped_scan(const ScanParams &p, hipStream_t stream) {
    const int64_t pairs = (int64_t)p.N * p.Hqk;
    const int64_t blocks = ((pairs + 7) / 8) * 8 * p.r;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(piped_scan_kernel, dim3((unsigned)blocks), dim3(512), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdn
