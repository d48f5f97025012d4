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
//   T     = (I + A)^-1 diag(b)                                (UT transform)
//   Vnew  = T (V - diag(gamma) K S0^T)
//   O     = scale [ diag(gamma) Q S0^T + ((Q K^T) o D) Vnew ],  D_ij = exp(G_i-G_j), j <= i
//   S_L   = gamma_L S0 + Vnew^T diag(exp(G_L - G)) K
//
// which equals the token recurrence exactly in real arithmetic.  L2
// normalisation is folded into per-row factors (rk, rq) so the MFMA operands
// are the caller's exact q/k values.
//
// Mapping to the hardware (one workgroup per sequence and per group of RG
// value heads that share one q/k head; 4 waves per value head):
//   * the fp32 state of each value head lives in MFMA accumulators for the
//     whole sequence: wave w of a head owns state rows v in [32w, 32w+32) as
//     four 32x32 accumulator tiles of S^T (rows k, columns v);
//   * the accumulator layout is reused directly as the B operand of the next
//     products (S0^T in K S0^T / Q S0^T, and Z / Vnew in T Z, P Vnew and the
//     state update): the contraction index of those products is permuted to
//     match the accumulator's row order, and the LDS-side operand is read
//     with the same permutation, so the state never leaves registers;
//   * K, Q, K^T (bf16 path), T and P are staged in LDS; the intra-chunk
//     inverse is computed with 16-row diagonal blocks by forward substitution
//     and two block-merge steps;
//   * the bf16 path runs v_mfma_f32_32x32x16_bf16 (fp32 accumulate); the fp32
//     path runs v_mfma_f32_32x32x2_f32 so fp32 inputs keep fp32 accuracy.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;
constexpr int D = kHeadDim;

// ----------------------------------------------------------------- MFMA ----
// 32x32 MFMA lane layout (wave64): lane l, row/col index l % 32, half h = l / 32.
//   A operand: row m = l % 32, contraction slots owned by half h.
//   B operand: col n = l % 32, contraction slots owned by half h.
//   Accumulator (16 fp32): col n = l % 32, row 8*(r/4) + 4*h + r%4 for reg r.
template <typename OT> struct Mma;
template <> struct Mma<bf16> {
    static constexpr int E = 8;                     // operand elements per lane
    typedef bf16x8 frag;
    __device__ static f32x16 run(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma<float> {
    static constexpr int E = 1;
    typedef float frag;
    __device__ static f32x16 run(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

// Row of accumulator register r for half h.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// "Accumulator order" operand fragment: step s of a 32-wide contraction
// block starting at cb; slot e of half h holds contraction index
// cb + acc_row(s*E + e, h).  Read from row `row` of a row-major LDS matrix.
template <typename OT>
__device__ __forceinline__ typename Mma<OT>::frag ld_acc_order(const OT *M, int ld, int row, int cb, int s, int h) {
    if constexpr (std::is_same<OT, bf16>::value) {
        const bf16 *p = M + row * ld + cb + 16 * s + 4 * h;
        const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(p);
        const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(p + 8);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
        return M[row * ld + cb + acc_row(s, h)];
    }
}

// Same contraction order, but the LDS matrix is stored transposed
// (element (row, idx) at M[idx * ld + row]); fp32 path only.
__device__ __forceinline__ float ld_acc_order_t(const float *M, int ld, int row, int cb, int s, int h) {
    return M[(cb + acc_row(s, h)) * ld + row];
}

// Natural-order fragment (both operands from LDS): step s covers contraction
// [2E*s, 2E*s + 2E); half h holds E consecutive indices.
template <typename OT>
__device__ __forceinline__ typename Mma<OT>::frag ld_natural(const OT *M, int ld, int row, int s, int h) {
    if constexpr (std::is_same<OT, bf16>::value) {
        return *reinterpret_cast<const bf16x8 *>(M + row * ld + 16 * s + 8 * h);
    } else {
        return M[row * ld + 2 * s + h];
    }
}

// Accumulator registers of step s as an operand fragment (accumulator order).
template <typename OT>
__device__ __forceinline__ typename Mma<OT>::frag acc_frag(const f32x16 &a, int s) {
    if constexpr (std::is_same<OT, bf16>::value) {
        bf16x8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (bf16)a[8 * s + e];
        return f;
    } else {
        return a[s];
    }
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    return z;
}

__device__ __forceinline__ float load_gate(const void *p, int64_t off, int dt) {
    if (dt == GDN_F32) return static_cast<const float *>(p)[off];
    if (dt == GDN_BF16) return (float)static_cast<const bf16 *>(p)[off];
    return (float)static_cast<const _Float16 *>(p)[off];
}

__device__ __forceinline__ int64_t load_cu(const void *cu, int i, int is64) {
    return is64 ? static_cast<const int64_t *>(cu)[i] : (int64_t) static_cast<const int32_t *>(cu)[i];
}

// ---------------------------------------------------------- LDS layout ----
template <typename IO, int RG> struct Smem {
    static constexpr bool BF = std::is_same<IO, bf16>::value;
    static constexpr int KLD = BF ? 136 : 132;   // K, Q rows (elements)
    static constexpr int TLD = 72;               // K^T rows (bf16 path)
    static constexpr int FLD = 68;               // fp32 64x64 (A, then T)
    static constexpr int OLD = BF ? 72 : 68;     // IO-typed 64x64 operands (T copy, P)
    static constexpr int RLD = 33;               // merge scratch
    static constexpr int K_OFF = 0;
    static constexpr int Q_OFF = K_OFF + C * KLD * (int)sizeof(IO);
    static constexpr int KT_OFF = Q_OFF + C * KLD * (int)sizeof(IO);
    static constexpr int ROW_OFF = KT_OFF + (BF ? D * TLD * 2 : 0);   // rk[64], rq[64]
    static constexpr int HEAD_OFF = ROW_OFF + 2 * C * 4;
    // per head: Tf (fp32), Tb (bf16 copy, bf16 path only), P, R, G/gam/dec/bet
    static constexpr int TF = 0;
    static constexpr int TB = TF + C * FLD * 4;
    static constexpr int P = TB + (BF ? C * OLD * 2 : 0);
    static constexpr int R = P + C * OLD * (int)sizeof(IO);
    static constexpr int SC = R + 32 * RLD * 4;
    static constexpr int HEAD_BYTES = SC + 4 * C * 4;
    static constexpr int BYTES = HEAD_OFF + RG * HEAD_BYTES;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(Q_OFF % 16 == 0 && KT_OFF % 16 == 0 && HEAD_OFF % 16 == 0 && HEAD_BYTES % 16 == 0, "align");
};

template <typename IO, int RG>
__global__ __launch_bounds__(256 * RG) void fused_scan_kernel(const ScanParams p) {
    using L = Smem<IO, RG>;
    using M = Mma<IO>;
    using frag = typename M::frag;
    constexpr bool BF = L::BF;
    constexpr int E = M::E;
    constexpr int S32 = 32 / (2 * E);       // MFMA steps per 32-wide contraction block
    constexpr int NT = 256 * RG;

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    IO *Ks = reinterpret_cast<IO *>(smem + L::K_OFF);
    IO *Qs = reinterpret_cast<IO *>(smem + L::Q_OFF);
    bf16 *KTs = reinterpret_cast<bf16 *>(smem + L::KT_OFF);
    float *rks = reinterpret_cast<float *>(smem + L::ROW_OFF);
    float *rqs = rks + C;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = wave >> 2, ws = wave & 3;
    const int h32 = lane >> 5, l32 = lane & 31;

    char *hbase = smem + L::HEAD_OFF + grp * L::HEAD_BYTES;
    float *Tf = reinterpret_cast<float *>(hbase + L::TF);
    IO *Pm = reinterpret_cast<IO *>(hbase + L::P);
    float *Rs = reinterpret_cast<float *>(hbase + L::R);
    float *Gs = reinterpret_cast<float *>(hbase + L::SC);
    float *gams = Gs + C, *decs = Gs + 2 * C, *bets = Gs + 3 * C;
    const IO *Top;
    int TOLD;
    if constexpr (BF) {
        Top = reinterpret_cast<const IO *>(hbase + L::TB);
        TOLD = L::OLD;
    } else {
        Top = reinterpret_cast<const IO *>(Tf);
        TOLD = L::FLD;
    }

    const int HG = p.Hv / RG;
    const int n = blockIdx.x / HG, hg = blockIdx.x % HG;
    const int h = hg * RG + grp;              // this wave's value head
    const int hq = (hg * RG) / p.r;           // shared q/k head
    const int64_t bos = load_cu(p.cu, n, p.cu_i64), eos = load_cu(p.cu, n + 1, p.cu_i64);
    const int v0 = ws * 32 + l32;             // this lane's state row v

    const IO *qg = static_cast<const IO *>(p.q);
    const IO *kg = static_cast<const IO *>(p.k);
    const IO *vg = static_cast<const IO *>(p.v);
    IO *og = static_cast<IO *>(p.out);

    // ---- initial state: S[b] holds S^T rows k = 32b + acc_row(r, h32), column v0
    f32x16 S[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) S[b] = zero16();
    if (p.s_in) {
        const int64_t base = (int64_t)n * p.si_n + (int64_t)h * p.si_h + (int64_t)v0 * p.si_v;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k0 = 32 * b + 8 * j + 4 * h32;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    float x;
                    if (p.si_dt == GDN_F32) x = static_cast<const float *>(p.s_in)[base + k0 + t];
                    else x = (float)static_cast<const bf16 *>(p.s_in)[base + k0 + t];
                    S[b][4 * j + t] = x;
                }
            }
    }

    const int nchunks = (int)((eos - bos + C - 1) / C);
    for (int c = 0; c < nchunks; ++c) {
        const int64_t t0 = bos + (int64_t)c * C;
        const int Lc = (int)min((int64_t)C, eos - t0);

        // ---- phase 1: stage K, Q (+K^T), row norms; gates and in-chunk cumsum

        if constexpr (BF) {
            // unit = (matrix, 4-row quad, 8-column group): 4 x 16-byte rows
            for (int u = tid; u < 512; u += NT) {
                const int mat = u >> 8, rq = (u >> 4) & 15, cg = u & 15;
                const bf16 *src = mat ? qg : kg;
                const int64_t st = mat ? p.q_st : p.k_st;
                const int64_t off = (int64_t)hq * (mat ? p.q_sh : p.k_sh) + 8 * cg;
                bf16x8 x[4];
                float ss[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int i = 4 * rq + t;
                    if (i < Lc) {
                        x[t] = *reinterpret_cast<const bf16x8 *>(src + (t0 + i) * st + off);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) x[t][e] = (bf16)0.f;
                    }
                    float a = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) a += (float)x[t][e] * (float)x[t][e];
                    ss[t] = a;
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) {
#pragma unroll
                    for (int o = 1; o < 16; o <<= 1) ss[t] += __shfl_xor(ss[t], o);
                }
                IO *dst = mat ? Qs : Ks;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    *reinterpret_cast<bf16x8 *>(dst + (4 * rq + t) * L::KLD + 8 * cg) = x[t];
                if (cg == 0) {
                    float *rn = mat ? rqs : rks;
#pragma unroll
                    for (int t = 0; t < 4; ++t) rn[4 * rq + t] = p.l2norm ? rsqrtf(ss[t] + 1e-6f) : 1.f;
                }
                if (mat == 0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        bf16x4 col = {x[0][e], x[1][e], x[2][e], x[3][e]};
                        *reinterpret_cast<bf16x4 *>(KTs + (8 * cg + e) * L::TLD + 4 * rq) = col;
                    }
                }
            }
        } else {
            // unit = (matrix, row, 4-float group)
            for (int u = tid; u < 2 * C * 32; u += NT) {
                const int mat = u >> 11, i = (u >> 5) & 63, cg = u & 31;
                const float *src = reinterpret_cast<const float *>(mat ? qg : kg);
                const int64_t st = mat ? p.q_st : p.k_st;
                const int64_t off = (int64_t)hq * (mat ? p.q_sh : p.k_sh) + 4 * cg;
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
                if (i < Lc) x = *reinterpret_cast<const f32x4 *>(src + (t0 + i) * st + off);
                float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
#pragma unroll
                for (int o = 1; o < 32; o <<= 1) ss += __shfl_xor(ss, o);
                float *dst = reinterpret_cast<float *>(mat ? Qs : Ks);
                *reinterpret_cast<f32x4 *>(dst + i * L::KLD + 4 * cg) = x;
                if (cg == 0) (mat ? rqs : rks)[i] = p.l2norm ? rsqrtf(ss + 1e-6f) : 1.f;
            }
        }

        if (ws == 0) {   // one wave per value head: gates and the in-chunk log-gate cumsum
            const int i = lane;
            const bool valid = i < Lc;
            float a = 1.f, b = 1.f;
            if (valid && p.g) a = load_gate(p.g, (t0 + i) * p.g_st + (int64_t)h * p.g_sh, p.g_dt);
            if (valid && p.beta) b = load_gate(p.beta, (t0 + i) * p.b_st + (int64_t)h * p.b_sh, p.b_dt);
            float G = valid ? fmaxf(__logf(a), -80.f) : 0.f;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float y = __shfl_up(G, o);
                if (lane >= o) G += y;
            }
            const float GL = __shfl(G, 63);
            Gs[i] = G;
            gams[i] = __expf(G);
            decs[i] = __expf(GL - G);
            bets[i] = valid ? b : 0.f;
        }
        __syncthreads();

        // ---- phase 2: Gram tiles K K^T and Q K^T (lower 32x32 tiles) -> A (fp32) and P per head
        for (int tile = wave; tile < 6; tile += 4 * RG) {
            const int isq = tile >= 3, tt = tile - 3 * isq;
            const int bi = tt > 0, bj = tt == 2;
            const IO *As = isq ? Qs : Ks;
            f32x16 acc = zero16();
#pragma unroll
            for (int s = 0; s < D / (2 * E); ++s) {
                const frag a = ld_natural<IO>(As, L::KLD, 32 * bi + l32, s, h32);
                const frag bb = ld_natural<IO>(Ks, L::KLD, 32 * bj + l32, s, h32);
                acc = M::run(a, bb, acc);
            }
            const int j = 32 * bj + l32;
            const float rkj = rks[j];
#pragma unroll
            for (int hh = 0; hh < RG; ++hh) {
                char *hb = smem + L::HEAD_OFF + hh * L::HEAD_BYTES;
                float *Tfh = reinterpret_cast<float *>(hb + L::TF);
                IO *Ph = reinterpret_cast<IO *>(hb + L::P);
                const float *Gh = reinterpret_cast<const float *>(hb + L::SC);
                const float *bh = Gh + 3 * C;
                const float Gj = Gh[j];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = 32 * bi + acc_row(r, h32);
                    if (!isq) {
                        const float val = (j < i) ? bh[i] * rks[i] * rkj * acc[r] * __expf(Gh[i] - Gj) : 0.f;
                        Tfh[i * L::FLD + j] = val;
                    } else {
                        const float val = (j <= i) ? rqs[i] * rkj * acc[r] * __expf(Gh[i] - Gj) : 0.f;
                        Ph[i * L::OLD + j] = (IO)val;
                    }
                }
            }
        }
        __syncthreads();

        // ---- phase 3: T = (I + A)^-1 diag(b), 16-row diagonal blocks then two merges
        if (ws == 0) {
            const int b = lane >> 4, cc = lane & 15;
            float *blk = Tf + (16 * b) * L::FLD + 16 * b;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == cc) ? 1.f : 0.f;
#pragma unroll
            for (int i = 1; i < 16; ++i) {
                float s = 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) s += blk[i * L::FLD + m] * x[m];
                if (i > cc) x[i] = -s;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) blk[i * L::FLD + cc] = x[i];
            if ((b & 1) == 0) {
#pragma unroll
                for (int i = 0; i < 16; ++i) blk[i * L::FLD + 16 + cc] = 0.f;
            }
        }
        __syncthreads();
        const int tg = tid & 255;
        float rv[4];
#pragma unroll
        for (int e = 0; e < 2; ++e) {      // R = A_{2x+1,2x} Dinv_{2x}
            const int idx = tg + 256 * e, x2 = idx >> 8, i = (idx >> 4) & 15, j = idx & 15;
            const float *Ar = Tf + (32 * x2 + 16 + i) * L::FLD + 32 * x2;
            const float *Dc = Tf + (32 * x2) * L::FLD + 32 * x2 + j;
            float a = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) a += Ar[m] * Dc[m * L::FLD];
            Rs[x2 * 256 + i * 16 + j] = a;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 2; ++e) {      // T_{2x+1,2x} = -Dinv_{2x+1} R
            const int idx = tg + 256 * e, x2 = idx >> 8, i = (idx >> 4) & 15, j = idx & 15;
            const float *Dr = Tf + (32 * x2 + 16 + i) * L::FLD + 32 * x2 + 16;
            float a = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) a += Dr[m] * Rs[x2 * 256 + m * 16 + j];
            Tf[(32 * x2 + 16 + i) * L::FLD + 32 * x2 + j] = -a;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 4; ++e) {      // R2 = A_{21} T_{11}   (32x32 blocks)
            const int idx = tg + 256 * e, i = idx >> 5, j = idx & 31;
            const float *Ar = Tf + (32 + i) * L::FLD;
            float a = 0.f;
#pragma unroll
            for (int m = 0; m < 32; ++m) a += Ar[m] * Tf[m * L::FLD + j];
            rv[e] = a;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = tg + 256 * e;
            Rs[(idx >> 5) * L::RLD + (idx & 31)] = rv[e];
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 4; ++e) {      // T_{21} = -T_{22} R2
            const int idx = tg + 256 * e, i = idx >> 5, j = idx & 31;
            const float *Tr = Tf + (32 + i) * L::FLD + 32;
            float a = 0.f;
#pragma unroll
            for (int m = 0; m < 32; ++m) a += Tr[m] * Rs[m * L::RLD + j];
            Tf[(32 + i) * L::FLD + j] = -a;
        }
        __syncthreads();
        for (int idx = tg; idx < 3 * 1024; idx += 256) {   // T <- T diag(b), operand copy
            const int blk = idx >> 10, w = idx & 1023;
            const int i = 32 * (blk >= 1) + (w >> 5), j = 32 * (blk == 2) + (w & 31);
            const float t = Tf[i * L::FLD + j] * bets[j];
            if constexpr (BF) reinterpret_cast<bf16 *>(hbase + L::TB)[i * L::OLD + j] = (bf16)t;
            else Tf[i * L::FLD + j] = t;
        }
        __syncthreads();

        // ---- phase 4: state products for this wave's 32 state rows.  Stages are
        // ordered so that at most two 64x32 accumulator pairs are live at once.
        frag sb[4][S32];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int s = 0; s < S32; ++s) sb[b][s] = acc_frag<IO>(S[b], s);
        // Z = V - gamma * rk * (K S0^T)
        frag zb[2][S32];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            float vreg[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 32 * ib + acc_row(r, h32);
                vreg[r] = (i < Lc) ? (float)vg[(t0 + i) * p.v_st + (int64_t)h * p.v_sh + v0] : 0.f;
            }
            f32x16 X = zero16();
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int s = 0; s < S32; ++s)
                    X = M::run(ld_acc_order<IO>(Ks, L::KLD, 32 * ib + l32, 32 * b, s, h32), sb[b][s], X);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 32 * ib + acc_row(r, h32);
                X[r] = vreg[r] - gams[i] * rks[i] * X[r];
            }
#pragma unroll
            for (int s = 0; s < S32; ++s) zb[ib][s] = acc_frag<IO>(X, s);
        }
        __builtin_amdgcn_sched_barrier(0);
        // Vnew = T Z   (T lower block-triangular: skip the zero upper 32x32 block)
        f32x16 Vn[2] = {zero16(), zero16()};
#pragma unroll
        for (int s = 0; s < S32; ++s) {
            Vn[0] = M::run(ld_acc_order<IO>(Top, TOLD, l32, 0, s, h32), zb[0][s], Vn[0]);
            Vn[1] = M::run(ld_acc_order<IO>(Top, TOLD, 32 + l32, 0, s, h32), zb[0][s], Vn[1]);
            Vn[1] = M::run(ld_acc_order<IO>(Top, TOLD, 32 + l32, 32, s, h32), zb[1][s], Vn[1]);
        }
        __builtin_amdgcn_sched_barrier(0);
        frag nb[2][S32];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int s = 0; s < S32; ++s) nb[ib][s] = acc_frag<IO>(Vn[ib], s);
        // O = scale [ gamma * rq * (Q S0^T) + P Vnew ], one 32-row block at a time
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            f32x16 Y = zero16();
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int s = 0; s < S32; ++s)
                    Y = M::run(ld_acc_order<IO>(Qs, L::KLD, 32 * ib + l32, 32 * b, s, h32), sb[b][s], Y);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 32 * ib + acc_row(r, h32);
                Y[r] *= gams[i] * rqs[i];
            }
#pragma unroll
            for (int jb = 0; jb <= ib; ++jb)
#pragma unroll
                for (int s = 0; s < S32; ++s)
                    Y = M::run(ld_acc_order<IO>(Pm, L::OLD, 32 * ib + l32, 32 * jb, s, h32), nb[jb][s], Y);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 32 * ib + acc_row(r, h32);
                if (i < Lc) og[(t0 + i) * p.o_st + (int64_t)h * p.o_sh + v0] = (IO)(Y[r] * p.scale);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // S <- gamma_L S + K^T (rk * dec * Vnew)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 32 * ib + acc_row(r, h32);
                Vn[ib][r] *= rks[i] * decs[i];
            }
        frag ub[2][S32];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int s = 0; s < S32; ++s) ub[ib][s] = acc_frag<IO>(Vn[ib], s);
        const float gL = gams[C - 1];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int r = 0; r < 16; ++r) S[b][r] *= gL;
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int s = 0; s < S32; ++s) {
                    frag a;
                    if constexpr (BF) a = ld_acc_order<bf16>(KTs, L::TLD, 32 * b + l32, 32 * ib, s, h32);
                    else a = ld_acc_order_t(reinterpret_cast<const float *>(Ks), L::KLD, 32 * b + l32, 32 * ib, s, h32);
                    S[b] = M::run(a, ub[ib][s], S[b]);
                }
        }
        __syncthreads();
    }

    // ---- final state
    if (p.s_out) {
        const int64_t base = (int64_t)n * p.so_n + (int64_t)h * p.so_h + (int64_t)v0 * p.so_v;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k0 = 32 * b + 8 * j + 4 * h32;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float x = S[b][4 * j + t];
                    if (p.so_dt == GDN_F32) static_cast<float *>(p.s_out)[base + k0 + t] = x;
                    else static_cast<bf16 *>(p.s_out)[base + k0 + t] = (bf16)x;
                }
            }
    }
}

template <typename IO, int RG>
hipError_t launch(const ScanParams &p, hipStream_t stream) {
    const int64_t blocks = (int64_t)p.N * (p.Hv / RG);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((fused_scan_kernel<IO, RG>), dim3((unsigned)blocks), dim3(256 * RG), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fused_scan(const ScanParams &p, bool io_bf16, int rg, hipStream_t stream) {
    if (io_bf16) return rg == 2 ? launch<bf16, 2>(p, stream) : launch<bf16, 1>(p, stream);
    return launch<float, 1>(p, stream);
}

}  // namespace gdn
