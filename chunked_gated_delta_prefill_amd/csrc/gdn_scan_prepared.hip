// The chunked gated delta rule scan over prepared chunks, for gfx950: the
// state-dependent half of the scan, for launches that leave CUs to spare.
//
// Method and per-element steps are those of the four-wave scan in gdn_scan.hip
// ("flashinfer.gdn_prefill": the chunked GDN scan and, in its Cake GDN CP
// section, the stage order T precompute -> ... -> prefill; arguments as in
// "flashinfer.cudnn.cudnn_chunk_gated_delta_rule", Parameters).  Everything of
// a chunk that does not depend on the state (Gram tiles and norms, A, the UT
// transform T' = (I + A)^-1 diag(b), the output tile P, the gate rows) was
// computed for all chunks at once by the preparation pass (the kPrep mode of
// the four-wave scan kernel) into a workspace slot per (chunk, value head).
// What is left is a serial chain per (sequence, value head).
//
// The rows of the state evolve independently, so a value head's 128 state rows
// are split over 4 / NP workgroups (NP = 1 or 2), each on its own CU, each
// holding NP blocks of 32 rows.  A workgroup has three wave roles:
//
//   recurrence waves (NP, one per 32-row block; the state in MFMA accumulators):
//     X = K S~^T,  Z' = V - FZ o X,  Vnew = T' Z',  ub = FU o Vnew,
//     S~ += K^T ub   (after the lazy-decay renorm fold)
//   output waves (NP, the same rows):
//     Y = S~ Q^T (the state's bf16 operand fragments, passed through LDS),
//     O^T = FY [Y + ub^T P^T]  (or the entry-wise form), bf16 rows to `out`
//   loader waves (2): every other global load of the coming chunks (K, Q, T', P,
//     the row factors and the decay scalars) and their LDS staging, two chunks
//     in flight in registers; the output waves load and stage V (one chunk in
//     flight), so the recurrence waves issue no loads at all
//
// Per chunk, two barrier intervals:
//
//   interval  recurrence                 output              loaders
//   1         X, Z', Vnew, ub (to LDS)   Y = S~ Q^T; P and   loads of chunk c + 2
//                                        FY read ahead; V
//                                        of c + 1 into LDS,
//                                        V loads of c + 2
//   2         renorm fold, update, S~    output products,    chunk c + 1 into LDS
//             fragments (to LDS)         staging, stores
//
// A wave here has its SIMD to itself, so every LDS read waited on next to its
// use costs its whole latency: each wave reads what a phase needs in one batch
// (the recurrence wave after its X pass, the output wave a whole interval ahead).
//
// With one or two blocks of rows per CU, each CU reads K, K^T, Q and the
// exchange tiles for 32 or 64 state rows instead of 128: the LDS traffic per
// CU, which bounds a chunk when one CU holds a whole head, drops 2-4 times.
//
// Every product is the four-wave scan's MFMA sequence with the same operands
// in the same order and every row factor the same expression, so the results
// are bitwise those of the four-wave and the pipelined scans.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdn_device.h"

namespace gdn {
namespace {

using namespace dev;

template <int NP> struct PreparedSmem {
    static constexpr int KLD = kKqLd;   // K, Q rows (bf16, rows permuted, see kq_row)
    static constexpr int OLD = 68;      // T', P rows (bf16)
    static constexpr int KB = C * KLD * 2;
    static constexpr int OB = C * OLD * 2;
    static constexpr int FRAG_BYTES = 64 * 16;                 // one operand fragment of a wave
    static constexpr int K_OFF = 0;                            // [2] by chunk parity
    static constexpr int Q_OFF = K_OFF + 2 * KB;
    static constexpr int T_OFF = Q_OFF + KB;
    static constexpr int P_OFF = T_OFF + OB;                   // [2] by chunk parity
    static constexpr int SB_OFF = P_OFF + 2 * OB;              // S~ fragments [block][8 steps]
    static constexpr int UB_OFF = SB_OFF + NP * 8 * FRAG_BYTES;   // ub fragments [block][4]
    static constexpr int NB_OFF = UB_OFF + NP * 4 * FRAG_BYTES;   // Vnew fragments (entry-wise path)
    static constexpr int VO_OFF = NB_OFF + NP * 4 * FRAG_BYTES;   // output staging block per block
    static constexpr int VB = C * 32 * 2;                         // V of one chunk and block: [64 tokens][32] bf16
    static constexpr int V_OFF = VO_OFF + NP * kStageBytes;       // [2][NP] by chunk parity
    static constexpr int ROW_OFF = V_OFF + 2 * NP * VB;           // FZ, FU, FY [2][64] each; scalars [2][4]
    static constexpr int BYTES = ROW_OFF + (6 * C + 8) * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(Q_OFF % 16 == 0 && T_OFF % 16 == 0 && P_OFF % 16 == 0 && SB_OFF % 16 == 0 &&
                  VO_OFF % 16 == 0 && V_OFF % 16 == 0 && ROW_OFF % 16 == 0, "align");
};

// Row and 16-byte piece of piece u of a prepared tile (rows 0..31: 4 pieces,
// rows 32..63: 8 pieces).
__device__ __forceinline__ int piece_row(int u) { return u < 128 ? u >> 2 : 32 + ((u - 128) >> 3); }
__device__ __forceinline__ int piece_col(int u) { return u < 128 ? 8 * (u & 3) : 8 * ((u - 128) & 7); }

__device__ __forceinline__ void put_piece(bf16 *M, int ld, int u, i32x4 x) {
    // tile rows are 8-byte aligned: two 8-byte writes
    bf16 *d = M + piece_row(u) * ld + piece_col(u);
    *reinterpret_cast<u32x2 *>(d) = u32x2{(unsigned)x[0], (unsigned)x[1]};
    *reinterpret_cast<u32x2 *>(d + 4) = u32x2{(unsigned)x[2], (unsigned)x[3]};
}

// The wave-uniform value of a float every lane holds.  (Taking the uniform
// value of one lane of a loaded vector, readfirstlane(v[i]), is folded by this
// compiler into readfirstlane(v[0]) for every i, so only plain floats go
// through readfirstlane here.)
__device__ __forceinline__ float uniform(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// One chunk in flight to the loader waves' registers (thread lt of 128).
struct LoaderSet {
    i32x4 k[8], q[8];   // K, Q pieces u = lt + 128 j: row u / 16, 16 bytes at column 8 (u % 16)
    i32x4 t[3], p[3];   // T', P pieces lt + 128 j (384 pieces)
    float bz, bu, by;   // row factors of token lt (lt < 64)
    float gl, igl, G;   // gamma_L, 1 / gamma_L, G_L
};

// NP = 1 runs 256 threads, one wave per SIMD, for which the compiler would take up
// to 512 registers per lane and then move values between the VGPRs and the
// accumulation registers (~480 such moves per chunk on the recurrence chain).  The
// declared bound of 512 threads (two waves per SIMD) holds it to 256 VGPRs, which it
// fits without spills; the launch stays at 256 threads.
template <int NP>
__global__ __launch_bounds__(NP == 1 ? 512 : 128 * NP + 128) void prepared_scan_kernel(const ScanParams p) {
    using L = PreparedSmem<NP>;
    using M = Mma<bf16>;
    using frag = M::frag;
    constexpr int S32 = 2;          // 32x32x16 steps per 32-wide contraction block
    constexpr int SLICES = 4 / NP;  // workgroups per value head

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    auto kbuf = [&](int x) { return reinterpret_cast<bf16 *>(smem + L::K_OFF + (x & 1) * L::KB); };
    bf16 *Qs = reinterpret_cast<bf16 *>(smem + L::Q_OFF);
    bf16 *Ts = reinterpret_cast<bf16 *>(smem + L::T_OFF);
    auto pbuf = [&](int x) { return reinterpret_cast<bf16 *>(smem + L::P_OFF + (x & 1) * L::OB); };
    // V of chunk x for the workgroup's block i, staged by that block's output wave
    auto vbuf = [&](int x, int i) { return reinterpret_cast<bf16 *>(smem + L::V_OFF + ((x & 1) * NP + i) * L::VB); };
    // operand fragment f of block i in one of the exchange areas (16 bytes per lane)
    auto xfrag = [&](int off, int nf, int i, int f, int lane) {
        return reinterpret_cast<bf16x8 *>(smem + off + ((i * nf + f) * 64 + lane) * 16);
    };
    float *RW = reinterpret_cast<float *>(smem + L::ROW_OFF);
    auto fzr = [&](int x) { return RW + (x & 1) * C; };            // FZ of chunk x
    auto fur = [&](int x) { return RW + (2 + (x & 1)) * C; };      // FU
    auto fyr = [&](int x) { return RW + (4 + (x & 1)) * C; };      // FY
    auto scal = [&](int x) { return RW + 6 * C + 4 * (x & 1); };   // gamma_L, 1 / gamma_L, G_L

    // ---- work item: (sequence, value head, slice of 32 NP state rows); the r value
    // heads of a q/k head and the slices of each get workgroup ids 8 apart (one XCD)
    const int r = p.r;
    const int b = blockIdx.x;
    const int group = 8 * r * SLICES;
    const int within = b % group;
    const int pidx = (b / group) * 8 + (within & 7);
    if (pidx >= p.N * p.Hqk) return;
    const int rest = within >> 3;
    const int n = pidx / p.Hqk, hq = pidx % p.Hqk;
    const int h = hq * r + rest % r, slice = rest / r;
    const int64_t bos = load_cu(p.cu, n, p.cu_i64), eos = load_cu(p.cu, n + 1, p.cu_i64);
    const int64_t srow = state_row(p.sidx, p.sidx_i64, p.pool_rows, n);
    const int nchunks = (int)((eos - bos + C - 1) / C);
    const int ws0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // the chunks this launch runs: [c0, cend), all of them unless the host splits
    // the scan into ranges so that the preparation of the next range overlaps it
    const int c0 = p.ph_c0 & -kPrepChunks;   // a whole number of preparation segments (the host's ranges)
    const int cend = p.ph_len > 0 && c0 + p.ph_len < nchunks ? c0 + p.ph_len : nchunks;
    if (c0 > 0 && c0 >= nchunks) return;   // the sequence ended in an earlier range
    const bool resumed = c0 > 0;
    // S~ and sigma of 32-row block vb where the previous range left them: register
    // group j (accumulator registers 4 j .. 4 j + 3) of lane l at 16 (64 j + l)
    // bytes, sigma after the 64 groups
    auto resume_rsrc = [&](int vb) {
        return rsrc(p.resume + (((int64_t)n * p.Hv + h) * 4 + vb) * kResumeFloats, kResumeFloats * 4);
    };
    auto resume_sigma = [&](int vb) {
        return uniform(__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(resume_rsrc(vb), 64 * 64 * 4, 0, 0)));
    };

    if (ws0 < NP) {
        // ================= recurrence waves =================
        const int vb = slice * NP + ws0;   // this wave's block of 32 state rows
        f32x16 S[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) S[bb] = zero16();
        float sigma = 1.f;
        if (resumed) {
            const int lane = threadIdx.x & 63;
            const auto rr = resume_rsrc(vb);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const f32x4 x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, 16 * (64 * j + lane), 0, 0));
#pragma unroll
                for (int t = 0; t < 4; ++t) S[j >> 2][4 * (j & 3) + t] = x[t];
            }
            sigma = resume_sigma(vb);
        } else {
            const int lane = threadIdx.x & 63, h32 = lane >> 5, v0 = 32 * vb + (lane & 31);
            if (p.s_in && srow >= 0)
                load_state<true>(S, p.s_in + srow * p.si_n + h * p.si_h, p.si_v, p.si_dt, v0, h32);
        }
        // the state's bf16 operand fragments (natural order), kept for this wave's X
        // pass and written to LDS for its output wave
        frag sfr[4 * S32];
        auto state_frags = [&](int lane) {
#pragma unroll
            for (int k = 0; k < 4 * S32; ++k) {
                sfr[k] = acc_frag<bf16>(S[k / S32], k % S32);
                *xfrag(L::SB_OFF, 8, ws0, k, lane) = sfr[k];
            }
        };
        state_frags(threadIdx.x & 63);
        __syncthreads();   // chunk c0 staged by the loaders

        for (int c = c0; c < cend; ++c) {
            int tid_o = threadIdx.x;
            asm volatile("" : "+v"(tid_o));
            const int lane = tid_o & 63;
            const int h32 = lane >> 5, l32 = lane & 31;
            const float gLc = uniform(scal(c)[0]);
            const float sig_next = sigma * gLc;
            const bool renorm = !(sig_next >= kRenorm);
            const bool fast = uniform(scal(c)[2]) > kFastDecay;
            const bf16 *Ks = kbuf(c);
            const float *FZr = fzr(c), *FUr = fur(c);
            const bf16 *Vb = vbuf(c, ws0);

            // ---- interval 1: X = K S~^T (the next step's K fragments read while the
            // current step runs), Z', Vnew, ub.  After the X pass everything Z', Vnew and ub
            // read from LDS is read at once (the T' fragments, the FZ and FU rows, and V,
            // staged by the output wave and read as 4 consecutive tokens of one column), so
            // its latency is paid once.
            f32x16 X[2] = {zero16(), zero16()};
            {
                frag fk[2][2];
                auto load = [&](int k, int st) {
                    fk[st][0] = ld_kq(Ks, l32, k, h32);
                    fk[st][1] = ld_kq(Ks, 32 + l32, k, h32);
                };
                load(0, 0);
#pragma unroll
                for (int k = 0; k < 4 * S32; ++k) {
                    const int cur = k & 1;
                    if (k + 1 < 4 * S32) load(k + 1, cur ^ 1);
                    X[0] = M::run(fk[cur][0], sfr[k], X[0]);
                    X[1] = M::run(fk[cur][1], sfr[k], X[1]);
                }
            }
            frag tf[3][S32];   // T' blocks (0,0), (1,0), (1,1)
            // (with NP = 2 the FU rows come later, while the Vnew products run: reading them
            // here too would exceed that kernel's 256 registers)
            f32x4 fz[2][4], fu[2][4];
#pragma unroll
            for (int s = 0; s < S32; ++s) {
                tf[0][s] = ld_acc<bf16>(Ts, L::OLD, l32, 0, s, h32);
                tf[1][s] = ld_acc<bf16>(Ts, L::OLD, 32 + l32, 0, s, h32);
                tf[2][s] = ld_acc<bf16>(Ts, L::OLD, 32 + l32, 32, s, h32);
            }
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    fz[ib][jj] = ld4(FZr + 32 * ib + 8 * jj + 4 * h32);
                    if constexpr (NP == 1) fu[ib][jj] = ld4(FUr + 32 * ib + 8 * jj + 4 * h32);
                }
            bf16x4 vx[2][4];
            {
                const int i = lane & 15, g16 = (lane >> 4) & 1;
                typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
#pragma unroll
                for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const bf16 *src = Vb + (32 * ib + 8 * q + 4 * h32 + (i >> 2)) * 32 + 16 * g16 + 4 * (i & 3);
                        vx[ib][q] =
                            __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)src));
                    }
            }
            frag zb[2][S32];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int rr = 4 * jj + t;
                        X[ib][rr] = fmaf(-fz[ib][jj][t], X[ib][rr], (float)vx[ib][jj][t]);
                    }
#pragma unroll
                for (int st = 0; st < S32; ++st) zb[ib][st] = acc_frag<bf16>(X[ib], st);
            }
            // Vnew = T' Z'   (T' lower block-triangular: the upper 32x32 block is zero)
            f32x16 Vn[2] = {zero16(), zero16()};
#pragma unroll
            for (int s = 0; s < S32; ++s) {
                Vn[0] = M::run(tf[0][s], zb[0][s], Vn[0]);
                Vn[1] = M::run(tf[1][s], zb[0][s], Vn[1]);
                Vn[1] = M::run(tf[2][s], zb[1][s], Vn[1]);
            }
            if constexpr (NP != 1) {
#pragma unroll
                for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) fu[ib][jj] = ld4(FUr + 32 * ib + 8 * jj + 4 * h32);
            }
            if (!fast) {   // the entry-wise output path takes Vnew itself
#pragma unroll
                for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                    for (int s = 0; s < S32; ++s)
                        *xfrag(L::NB_OFF, 4, ws0, S32 * ib + s, lane) = acc_frag<bf16>(Vn[ib], s);
            }
            frag ub[2][S32];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int t = 0; t < 4; ++t) Vn[ib][4 * jj + t] *= fu[ib][jj][t];
#pragma unroll
                for (int s = 0; s < S32; ++s) {
                    ub[ib][s] = acc_frag<bf16>(Vn[ib], s);
                    *xfrag(L::UB_OFF, 4, ws0, S32 * ib + s, lane) = ub[ib][s];
                }
            }
            __syncthreads();

            // ---- interval 2: renorm fold, S~ += K^T ub; the next chunk's S~ fragments
            if (renorm) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb)
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) S[bb][rr] *= sig_next;
            }
            {
                constexpr int NU = 2 * S32;
                frag kt[2][4];
                auto load_kt = [&](int k, frag (&f)[4]) {
                    const int ib = k / S32, st = k % S32;
#pragma unroll
                    for (int bb = 0; bb < 4; ++bb) f[bb] = ld_acc_tr(Ks, 32 * bb, 32 * ib, st, lane);
                };
                load_kt(0, kt[0]);
#pragma unroll
                for (int k = 0; k < NU; ++k) {
                    const int cur = k & 1;
                    if (k + 1 < NU) load_kt(k + 1, kt[cur ^ 1]);
#pragma unroll
                    for (int bb = 0; bb < 4; ++bb) S[bb] = M::run(kt[cur][bb], ub[k / S32][k % S32], S[bb]);
                }
            }
            sigma = renorm ? 1.f : sig_next;
            if (c + 1 < cend) state_frags(lane);
            __syncthreads();
        }

        if (cend < nchunks) {   // S~ and sigma as they are, for the next range
            const int lane = threadIdx.x & 63;
            const auto rr = resume_rsrc(vb);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const f32x4 x = {S[j >> 2][4 * (j & 3)], S[j >> 2][4 * (j & 3) + 1], S[j >> 2][4 * (j & 3) + 2],
                                 S[j >> 2][4 * (j & 3) + 3]};
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), rr, 16 * (64 * j + lane), 0, 0);
            }
            if (lane == 0) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, sigma), rr, 64 * 64 * 4, 0, 0);
        } else if (p.s_out && srow >= 0) {   // ---- final state (each slice writes its own rows)
            if (sigma != 1.f) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb)
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) S[bb][rr] *= sigma;
            }
            const int lane = threadIdx.x & 63, h32 = lane >> 5, v0 = 32 * vb + (lane & 31);
            store_state<true>(S, p.s_out + srow * p.so_n + h * p.so_h, p.so_v, p.so_dt, v0, h32);
        }
    } else if (ws0 < 2 * NP) {
        // ================= output waves =================
        const int w = ws0 - NP;             // the block of rows (and the recurrence wave) this wave outputs
        const int vb = slice * NP + w;
        float sigma = resumed ? resume_sigma(vb) : 1.f;
        // V of this block for the recurrence wave, one chunk in flight in registers and
        // staged into LDS ([64 tokens][32] bf16) a chunk before it is used: the output
        // wave waits through most of the first interval, the recurrence wave does not
        VWide vw;
        auto stage_v = [&](int x, int lane) {
            bf16 *Vb = vbuf(x, w);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<i32x4 *>(Vb + (16 * j + (lane >> 2)) * 32 + 8 * (lane & 3)) = vw.x[j];
        };
        auto issue_v = [&](int x, int lane) {
            const ChunkRef ch = chunk_at(bos, eos, x);
#pragma unroll
            for (int j = 0; j < 4; ++j) issue_v_wide_part(vw, p, ch, h, vb, lane, j);
        };
        if (cend > c0) {
            issue_v(c0, threadIdx.x & 63);
            stage_v(c0, threadIdx.x & 63);
            if (c0 + 1 < cend) issue_v(c0 + 1, threadIdx.x & 63);
        }
        __syncthreads();   // chunk c0 staged by the loaders

        for (int c = c0; c < cend; ++c) {
            int tid_o = threadIdx.x;
            asm volatile("" : "+v"(tid_o));
            const int lane = tid_o & 63;
            const int h32 = lane >> 5, l32 = lane & 31;
            const float gLc = uniform(scal(c)[0]);
            const float sig_next = sigma * gLc;
            const bool renorm = !(sig_next >= kRenorm);
            const bool fast = uniform(scal(c)[2]) > kFastDecay;
            const ChunkRef ch = chunk_at(bos, eos, c);
            const int Lc = ch.L;

            // ---- interval 1: Y = S~ Q^T (the state as the A operand gives its transpose:
            // lane = token, registers = 4 consecutive v); this chunk's P fragments and
            // output row factors (staged in the previous interval) read here for interval 2
            const bf16 *Ps = pbuf(c);
            const float *FYr = fyr(c);
            frag pfr[3][S32];   // P blocks (0,0), (1,0), (1,1)
#pragma unroll
            for (int s = 0; s < S32; ++s) {
                pfr[0][s] = ld_acc<bf16>(Ps, L::OLD, l32, 0, s, h32);
                pfr[1][s] = ld_acc<bf16>(Ps, L::OLD, 32 + l32, 0, s, h32);
                pfr[2][s] = ld_acc<bf16>(Ps, L::OLD, 32 + l32, 32, s, h32);
            }
            const float fyv[2] = {FYr[l32], FYr[32 + l32]};
            f32x16 Y[2] = {zero16(), zero16()};
            {
                frag fq[2][2];
                auto load = [&](int k, int st) {
                    fq[st][0] = ld_kq(Qs, l32, k, h32);
                    fq[st][1] = ld_kq(Qs, 32 + l32, k, h32);
                };
                load(0, 0);
#pragma unroll
                for (int k = 0; k < 4 * S32; ++k) {
                    const int cur = k & 1;
                    if (k + 1 < 4 * S32) load(k + 1, cur ^ 1);
                    const frag sf = *xfrag(L::SB_OFF, 8, w, k, lane);
                    Y[0] = M::run(sf, fq[cur][0], Y[0]);
                    Y[1] = M::run(sf, fq[cur][1], Y[1]);
                }
            }
            // V of chunk c + 1 into its buffer (last read by the recurrence wave in the first
            // interval of chunk c - 1), then the loads of chunk c + 2
            if (c + 1 < cend) stage_v(c + 1, lane);
            if (c + 2 < cend) issue_v(c + 2, lane);
            __syncthreads();

            // ---- interval 2: the output rows of chunk c (the recurrence wave's ub, or
            // Vnew on the entry-wise path, read first)
            frag uf[2 * S32];
#pragma unroll
            for (int f = 0; f < 2 * S32; ++f) uf[f] = *xfrag(fast ? L::UB_OFF : L::NB_OFF, 4, w, f, lane);
            if (fast) {   // O^T = FY_t [S~ Q^T + ub^T P^T] (renormalising: the state term as (S~ Q^T) sigma gamma_L)
                if (renorm) {
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
                        for (int s = 0; s < S32; ++s) Y[ib] = M::run(uf[S32 * jb + s], pfr[ib + jb][s], Y[ib]);
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) Y[ib][rr] *= fyv[ib];
                }
            } else {      // FY_t (S~ Q^T) + Vnew^T P^T
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) Y[ib][rr] *= fyv[ib];
#pragma unroll
                    for (int jb = 0; jb <= ib; ++jb)
#pragma unroll
                        for (int s = 0; s < S32; ++s) Y[ib] = M::run(uf[S32 * jb + s], pfr[ib + jb][s], Y[ib]);
                }
            }
            // staged through this block's staging block, then 16 rows of 64 bytes per store
            char *st = smem + L::VO_OFF + w * kStageBytes;
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) stage_out_tile(st, Y[ib], ib, l32, h32);
            const auto ro = rsrc(p.out + ch.t0 * p.o_st + h * p.o_sh, (Lc - 1) * p.o_st + D * 2);
            const int gq = lane & 3;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int t = 16 * k + (lane >> 2);
                const i32x4 o16 = staged_out(st, t, gq);
                __builtin_amdgcn_raw_buffer_store_b128(o16, ro, t * p.o_st + (32 * vb + 8 * gq) * 2, 0, 0);
            }
            sigma = renorm ? 1.f : sig_next;
            __syncthreads();
        }
    } else {
        // ================= loader waves =================
        const int lt = threadIdx.x - 128 * NP;   // 0..127
        const int64_t slot_stride = (int64_t)p.Hv * kPrepSlot;
        const char *slot0 =
            p.prep + ((int64_t)(nchunks > 0 ? p.seg_first[n] : 0) * p.prep_cps * p.Hv + h) * kPrepSlot;
        float sigma = resumed ? resume_sigma(slice * NP) : 1.f;   // the lazy scale at the start of the chunk being staged
        LoaderSet set0, set1;
        auto issue = [&](LoaderSet &d, int x) {
            const ChunkRef ch = chunk_at(bos, eos, x);
            const auto rk = rsrc(p.k + ch.t0 * p.k_st + hq * p.k_sh, ch.L > 0 ? (ch.L - 1) * p.k_st + D * 2 : 0);
            const auto rq = rsrc(p.q + ch.t0 * p.q_st + hq * p.q_sh, ch.L > 0 ? (ch.L - 1) * p.q_st + D * 2 : 0);
            const auto rs = rsrc(slot0 + x * slot_stride, kPrepSlot);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int u = lt + 128 * j, row = u >> 4, col = 16 * (u & 15);
                d.k[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, row * p.k_st + col, 0, 0);
                d.q[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, row * p.q_st + col, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                d.t[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, kPrepT + 16 * (lt + 128 * j), 0, 0);
                d.p[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, kPrepP + 16 * (lt + 128 * j), 0, 0);
            }
            if (lt < C) {
                d.bz = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, kPrepRows + 4 * lt, 0, 0));
                d.by = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, kPrepRows + 4 * (C + lt), 0, 0));
                d.bu = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(rs, kPrepRows + 4 * (2 * C + lt), 0, 0));
            }
            d.gl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, kPrepScalars, 0, 0));
            d.igl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, kPrepScalars + 4, 0, 0));
            d.G = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, kPrepScalars + 8, 0, 0));
        };
        // chunk x from its register set into LDS; the row factors with the lazy scale
        // at the chunk's start (the four-wave scan's expressions)
        auto stage = [&](const LoaderSet &d, int x) {
            bf16 *Ks = kbuf(x);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int u = lt + 128 * j, row = u >> 4, col = 8 * (u & 15);
                *reinterpret_cast<i32x4 *>(Ks + kq_off(row, col)) = d.k[j];
                *reinterpret_cast<i32x4 *>(Qs + kq_off(row, col)) = d.q[j];
            }
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                put_piece(Ts, L::OLD, lt + 128 * j, d.t[j]);
                put_piece(pbuf(x), L::OLD, lt + 128 * j, d.p[j]);
            }
            const float gL = uniform(d.gl), igL = uniform(d.igl), G = uniform(d.G);
            const float sig_next = sigma * gL;
            const bool renorm = !(sig_next >= kRenorm);
            const bool fast = G > kFastDecay;
            if (lt < C) {
                fzr(x)[lt] = sigma * d.bz;
                fur(x)[lt] = renorm ? d.bu : d.bu / sig_next;
                fyr(x)[lt] = fast && renorm ? d.by * igL : sigma * d.by;
            }
            if (lt == 0) {
                scal(x)[0] = gL;
                scal(x)[1] = igL;
                scal(x)[2] = G;
            }
            sigma = renorm ? 1.f : sig_next;
        };
        if (cend > c0) {
            issue(set0, c0);
            if (c0 + 1 < cend) issue(set1, c0 + 1);
            stage(set0, c0);
        }
        __syncthreads();
        // Chunk c's set holds chunk c + 2 after interval 1 of chunk c; the other set
        // (chunk c + 1, loaded an iteration earlier) is staged in interval 2.  The loop
        // runs two chunks per trip so that each set is a fixed group of registers.
        auto body = [&](LoaderSet &mine, LoaderSet &other, int c) {
            // Chunk c + 1's loads (an iteration old) are waited for before chunk c + 2's
            // are issued: the compiler cannot count the conditional row loads, so a wait
            // after that issue (in interval 2) also waits for the new loads (4 x 8192
            // tokens: -3.4%; one 65,536-token sequence, once the recurrence waves no
            // longer load V and the loaders' staging bounds the second interval: -8%)
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            if (c + 2 < cend) issue(mine, c + 2);
            __syncthreads();
            if (c + 1 < cend) stage(other, c + 1);
            __syncthreads();
        };
        for (int c = c0; c < cend; c += 2) {
            body(set0, set1, c);
            if (c + 1 < cend) body(set1, set0, c + 1);
        }
    }
}

}  // namespace

hipError_t launch_prepared_scan(const ScanParams &p, int np, hipStream_t stream) {
    const int64_t pairs = (int64_t)p.N * p.Hqk;
    const int64_t blocks = ((pairs + 7) / 8) * 8 * p.r * (4 / np);
    if (blocks == 0) return hipSuccess;
    if (np == 1)
        hipLaunchKernelGGL(prepared_scan_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(prepared_scan_kernel<2>, dim3((unsigned)blocks), dim3(384), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdn
