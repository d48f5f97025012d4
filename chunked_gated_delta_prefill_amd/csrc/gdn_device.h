// Device helpers shared by the scan kernels (gdn_scan.hip, gdn_scan_piped.hip):
// MFMA operand layouts, LDS operand reads, buffer loads of one chunk, gate
// decoding, DPP reductions and state I/O.  Internal; included by .hip files only.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdn_internal.h"

namespace gdn {
namespace dev {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;
constexpr int D = kHeadDim;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, gfx9-family data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
    const int n = bytes <= 0 ? 0 : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, kRsrcWord3);
}

// ----------------------------------------------------------------- MFMA ----
// 32x32 MFMA lane layout (wave64): lane l, index l % 32, half h = l / 32.
//   A operand: row m = l % 32; B operand: col n = l % 32; contraction slots
//   owned by half h.  Accumulator (16 fp32): col n = l % 32, row
//   8*(r/4) + 4*h + r%4 for register r.
// 16x16 MFMA: lane l, index l % 16, group g = l / 16.  Accumulator (4 fp32):
//   col n = l % 16, row 4*g + r.
template <typename OT> struct Mma;
template <> struct Mma<bf16> {
    static constexpr int E = 8;                     // 32x32 operand elements per lane
    static constexpr int E16 = 4;                   // 16x16 operand elements per lane
    typedef bf16x8 frag;
    typedef bf16x4 frag16;
    __device__ static f32x16 run(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static f32x4 run16(frag16 a, frag16 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma<float> {
    static constexpr int E = 1;
    static constexpr int E16 = 1;
    typedef float frag;
    typedef float frag16;
    __device__ static f32x16 run(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    __device__ static f32x4 run16(frag16 a, frag16 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// Row of 32x32 accumulator register r for half h.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <typename T> struct is_bf : std::is_same<T, bf16> {};

// 32x32 operand, accumulator order: step s of a 32-wide contraction block at
// cb; slot e of half h holds index cb + acc_row(s*E + e, h).  Row-major LDS.
template <typename OT, typename ST>
__device__ __forceinline__ typename Mma<OT>::frag ld_acc(const ST *M, int ld, int row, int cb, int s, int h) {
    if constexpr (is_bf<OT>::value && is_bf<ST>::value) {
        const bf16 *p = M + row * ld + cb + 16 * s + 4 * h;
        const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(p);
        const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(p + 8);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    } else if constexpr (is_bf<OT>::value) {        // fp32 LDS -> bf16 operand
        const float *p = M + row * ld + cb + 16 * s + 4 * h;
        const f32x4 lo = *reinterpret_cast<const f32x4 *>(p);
        const f32x4 hi = *reinterpret_cast<const f32x4 *>(p + 8);
        bf16x8 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) { f[e] = (bf16)lo[e]; f[4 + e] = (bf16)hi[e]; }
        return f;
    } else {
        return M[row * ld + cb + acc_row(s, h)];
    }
}

// Same order, element (row, idx) stored at M[idx * ld + row] (column read).
template <typename OT, typename ST>
__device__ __forceinline__ typename Mma<OT>::frag ld_acc_t(const ST *M, int ld, int row, int cb, int s, int h) {
    if constexpr (is_bf<OT>::value) {
        bf16x8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (bf16)(float)M[(cb + acc_row(8 * s + e, h)) * ld + row];
        return f;
    } else {
        return M[(cb + acc_row(s, h)) * ld + row];
    }
}

// Accumulator registers of step s as a 32x32 operand (accumulator order).
template <typename OT>
__device__ __forceinline__ typename Mma<OT>::frag acc_frag(const f32x16 &a, int s) {
    if constexpr (is_bf<OT>::value) {
        bf16x8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (bf16)a[8 * s + e];
        return f;
    } else {
        return a[s];
    }
}

// 16x16 operands, accumulator order: step s, slot e of group g holds index
// 4*g + s*E16 + e.  Row read (row-major) and column read variants, from fp32 LDS.
template <typename OT>
__device__ __forceinline__ typename Mma<OT>::frag16 ld16_row(const float *M, int ld, int row, int cb, int s, int g) {
    if constexpr (is_bf<OT>::value) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(M + row * ld + cb + 4 * g);
        return bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
    } else {
        return M[row * ld + cb + 4 * g + s];
    }
}
template <typename OT>
__device__ __forceinline__ typename Mma<OT>::frag16 ld16_col(const float *M, int ld, int col, int rb, int s, int g) {
    if constexpr (is_bf<OT>::value) {
        bf16x4 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = (bf16)M[(rb + 4 * g + e) * ld + col];
        return f;
    } else {
        return M[(rb + 4 * g + s) * ld + col];
    }
}
template <typename OT>
__device__ __forceinline__ typename Mma<OT>::frag16 acc16_frag(const f32x4 &a, int s) {
    if constexpr (is_bf<OT>::value) {
        return bf16x4{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
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

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}

__device__ __forceinline__ int64_t load_cu(const void *cu, int i, int is64) {
    return is64 ? static_cast<const int64_t *>(cu)[i] : (int64_t) static_cast<const int32_t *>(cu)[i];
}

// Row of the caller's state buffers used by sequence n: n itself, or its entry
// in the state index array (-1 when that entry is outside [0, rows)).
__device__ __forceinline__ int64_t state_row(const void *sidx, int is64, int64_t rows, int n) {
    if (!sidx) return n;
    const int64_t ix = load_cu(sidx, n, is64);
    return (ix >= 0 && ix < rows) ? ix : -1;
}

// Gate loads keep the raw bits; they are converted when first used, so the
// load is not waited for when it is issued.
__device__ __forceinline__ uint32_t gate_bits(__amdgpu_buffer_rsrc_t r, int off, int dt) {
    return dt == GDN_F32 ? __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0)
                         : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ float gate_value(uint32_t bits, int dt) {
    if (dt == GDN_F32) return __builtin_bit_cast(float, bits);
    if (dt == GDN_BF16) return bf16_bits_to_float(bits & 0xffffu);
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(bits & 0xffffu));
}

// ---------------------------------------------------------- LDS layout ----
// Per-row factor arrays (64 floats each), written once per chunk.  The state
// is held as S = sigma * S~ (sigma a per-sequence scalar, see the kernel); c
// is the query scale:
//   RG  in-chunk log-gate cumsum G_i   GM gamma_i = exp(G_i)   IG 1 / gamma_i, then rk_i / gamma_i
//   DC  exp(G_L - G_i)                 FB b_i                  (b also scales T' columns)
//   RK  rk_i, RQ rq_i  (1 without L2 norm; computed with the Gram tiles, which also fold rk_i into IG)
//   FZ  sigma gamma_i rk_i   (rows of K S~^T)     FY  c sigma gamma_i rq_i  (output rows)
//   FU  rk_i exp(G_L - G_i) / sigma'   (state update; without / sigma' on renorm)
//   (FY is c gamma_i rq_i / gamma_L on a renormalising chunk of the fast path, whose
//   output takes the state term as (S~ Q^T) sigma gamma_L: no factor of 1 / sigma',
//   which can reach 2^40 e^60, meets the raw q.k of the output tile)
// The gate rows RG .. FB come in two sets, for chunks of even and odd index:
// one wave writes the next chunk's set while the current one is in use.  Row
// `which` of set 1 sits at NROWF + which; after all rows, gamma_L of each set.
enum { RG_ = 0, GM_ = 1, IG_ = 2, DC_ = 3, FB_ = 4, RK_ = 5, RQ_ = 6, FZ_ = 7, FY_ = 8, FU_ = 9, NROWF = 10 };
constexpr int kGateRows = 5;                  // RG_ .. FB_
constexpr int kRowsTotal = NROWF + kGateRows;
constexpr int kGateWave = 2;                  // the wave that loads and converts the gates
constexpr float kFastDecay = -60.f;   // G_L above this: exp(G_i - G_j) = gamma_i / gamma_j is safe
constexpr float kRenorm = 0x1p-40f;   // sigma below this is folded back into the state


// Element e of each lane quad, broadcast to the quad (DPP quad_perm [e, e, e, e]).
__device__ __forceinline__ float quad_bcast(float v, int e) {
    const int b = __builtin_bit_cast(int, v);
    switch (e) {
        case 0: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0x00, 0xf, 0xf, false));
        case 1: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0x55, 0xf, 0xf, false));
        case 2: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0xaa, 0xf, 0xf, false));
        default: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0xff, 0xf, 0xf, false));
    }
}

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

// acc + the sum of squares of 8 bf16 values (products exact in fp32, fp32
// accumulation), as one chain of four dot2 steps into the running sum.
__device__ __forceinline__ float sumsq8_acc(bf16x8 x, float acc) {
    const bf16x2 x0 = __builtin_shufflevector(x, x, 0, 1), x1 = __builtin_shufflevector(x, x, 2, 3);
    const bf16x2 x2 = __builtin_shufflevector(x, x, 4, 5), x3 = __builtin_shufflevector(x, x, 6, 7);
    acc = __builtin_amdgcn_fdot2_f32_bf16(x0, x0, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(x1, x1, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(x2, x2, acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(x3, x3, acc, false);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts of 1, 2, 4, 8 inside
// each 16-lane row, then the row totals carried across rows.
template <int CTRL, int ROWS> __device__ __forceinline__ float dpp_add(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xf, true));
}
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x = dpp_add<0x111, 0xf>(x);   // row_shr:1
    x = dpp_add<0x112, 0xf>(x);   // row_shr:2
    x = dpp_add<0x114, 0xf>(x);   // row_shr:4
    x = dpp_add<0x118, 0xf>(x);   // row_shr:8
    x = dpp_add<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
    x = dpp_add<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

// bf16 K and Q tiles in LDS: rows of 128 values padded to kKqLd (272 bytes, 4
// banks past a multiple of the 64 four-byte banks), row r stored at row
// kq_row(r), which transposes each aligned group of 16 rows as a 4 x 4 block
// (r = 4a + b goes to 4b + a).  A half-wave's 8-byte LDS reads finish in one
// pass only when they touch 64 distinct banks.  The transposing K^T reads of the
// state update take 4 consecutive tokens x 64 bytes per half-wave: after the
// permutation those rows sit 16 banks apart, so the half-wave covers all 64
// banks (with consecutive rows 4 banks apart they overlapped two-way).  16-byte
// operand reads of 16 consecutive rows at one column still land on 16 distinct
// bank quads, and the 16-byte staging writes run along one row, so neither
// conflicts.  The permutation is a per-lane constant for every access, so it
// costs no address arithmetic beyond the base.
constexpr int kKqLd = 136;
__device__ __forceinline__ int kq_row(int r) { return (r & ~15) | (4 * (r & 3) + ((r >> 2) & 3)); }
__device__ __forceinline__ int kq_off(int row, int col) { return kq_row(row) * kKqLd + col; }
// 32x32 operand in natural order from a K or Q tile: step s covers columns
// [16 s, 16 s + 16), half h holds the 8 consecutive columns 16 s + 8 h ..
__device__ __forceinline__ bf16x8 ld_kq(const bf16 *M, int row, int s, int h) {
    return *reinterpret_cast<const bf16x8 *>(M + kq_off(row, 16 * s + 8 * h));
}

// 32x32 bf16 A operand of a product contracting over tokens, rows = K columns
// [m0, m0 + 32), read straight from row-major K with the transposing LDS load
// (within 16 lanes, output lane i element e comes from source lane i/4 + 4e,
// element i%4; source lane j points at token t0 + j/4 and at the 4 columns of
// output lanes 4 (j%4) .. 4 (j%4) + 3).  Slots follow the accumulator order of
// ld_acc: tokens cb + 16s + 4h + {0..3} and the same + 8.  Operand row m holds
// K column m0 + m with bits 2 and 3 of m swapped, so that the product's
// accumulator register r of half h is column m0 + 16 (r/8) + 8h + r%8: the
// state's natural operand order.  With PERM = false operand row m is column
// m0 + m (a plain operand of a column-major read).
//
// Ks is a K tile in the row order of kq_row.
template <bool PERM = true>
__device__ __forceinline__ bf16x8 ld_acc_tr(const bf16 *Ks, int m0, int cb, int s, int lane) {
    const int i = lane & 15, h = lane >> 5, g16 = (lane >> 4) & 1;
    const int q = i & 3, qs = PERM ? ((q & 1) << 1) | (q >> 1) : q;
    const bf16 *p = Ks + kq_off(cb + 16 * s + 4 * h + (i >> 2), m0 + 16 * g16 + 4 * qs);
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
    // 8 tokens further down: kq_row(r + 8) = kq_row(r) + 2 for r % 16 < 8
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 2 * kKqLd));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// K, Q and the gates of the next chunk, loaded while the current chunk runs
// (consumed only after the chunk's last barrier, so no wait is forced early).
template <typename IO> struct Prefetch;
template <> struct Prefetch<bf16> {
    i32x4 kq[2][4];      // K and Q: 4 rows x 8 columns per thread
    uint32_t g, b;       // raw gate bits of token `lane` (wave 0)
};
template <> struct Prefetch<float> {
    f32x4 kq[2][8];      // K and Q: 8 rows x 4 columns per thread
    uint32_t g, b;
};
// This chunk's V in accumulator layout (rows 32*ib + acc_row(r, h32), column
// v0), one element per register; loaded at the start of the chunk and first
// read in the last phase.
struct VRegs {
    uint32_t x[32];
};
__device__ __forceinline__ float vreg_at(const VRegs &v, int e, bool bf) {
    return bf ? bf16_bits_to_float(v.x[e] & 0xffffu) : __builtin_bit_cast(float, v.x[e]);
}

struct ChunkRef {
    int64_t t0;
    int L;
};

// bf16 K and Q, part t of four: rows 4 (tid / 16) + t, 16 bytes at column 8 (tid % 16)
// (four full rows per wave and instruction).
__device__ __forceinline__ void issue_kq_part(Prefetch<bf16> &pf, const ScanParams &p, ChunkRef ch, int hq, int tid,
                                              int t) {
    const int L = ch.L;
    const auto rk = rsrc(p.k + ch.t0 * p.k_st + hq * p.k_sh, L > 0 ? (L - 1) * p.k_st + D * 2 : 0);
    const auto rq = rsrc(p.q + ch.t0 * p.q_st + hq * p.q_sh, L > 0 ? (L - 1) * p.q_st + D * 2 : 0);
    const int rq4 = tid >> 4, cg = tid & 15;
    pf.kq[0][t] = __builtin_amdgcn_raw_buffer_load_b128(rk, (4 * rq4 + t) * p.k_st + 16 * cg, 0, 0);
    pf.kq[1][t] = __builtin_amdgcn_raw_buffer_load_b128(rq, (4 * rq4 + t) * p.q_st + 16 * cg, 0, 0);
}

// gate and beta of token `lane` (raw bits; 0 when the input is absent)
template <typename IO>
__device__ __forceinline__ void issue_gates(Prefetch<IO> &pf, const ScanParams &p, ChunkRef ch, int h, int lane) {
    const int L = ch.L;
    pf.g = 0;
    pf.b = 0;
    if (p.g) {
        const auto rg = rsrc(p.g + ch.t0 * p.g_st + h * p.g_sh, L > 0 ? (L - 1) * p.g_st + 4 : 0);
        pf.g = gate_bits(rg, lane * p.g_st, p.g_dt);
    }
    if (p.beta) {
        const auto rb = rsrc(p.beta + ch.t0 * p.b_st + h * p.b_sh, L > 0 ? (L - 1) * p.b_st + 4 : 0);
        pf.b = gate_bits(rb, lane * p.b_st, p.b_dt);
    }
}

// Loads one chunk's K, Q (and, on wave 0, gates) into registers.
template <typename IO>
__device__ __forceinline__ void issue_loads(Prefetch<IO> &pf, const ScanParams &p, ChunkRef ch, int hq, int h,
                                            int tid, int lane, int ws) {
    if constexpr (is_bf<IO>::value) {
#pragma unroll
        for (int t = 0; t < 4; ++t) issue_kq_part(pf, p, ch, hq, tid, t);
    } else {
        const int L = ch.L;
        const auto rk = rsrc(p.k + ch.t0 * p.k_st + hq * p.k_sh, L > 0 ? (L - 1) * p.k_st + D * 4 : 0);
        const auto rq = rsrc(p.q + ch.t0 * p.q_st + hq * p.q_sh, L > 0 ? (L - 1) * p.q_st + D * 4 : 0);
        const int r0 = tid >> 5, cg = tid & 31;
        const int vk = r0 * p.k_st + 16 * cg, vq = r0 * p.q_st + 16 * cg;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            pf.kq[0][j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, vk + 8 * j * p.k_st, 0, 0));
            pf.kq[1][j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, vq + 8 * j * p.q_st, 0, 0));
        }
    }
}

template <typename IO>
__device__ __forceinline__ void issue_v(VRegs &vr, const ScanParams &p, ChunkRef ch, int h, int h32, int v0) {
    constexpr bool BF = is_bf<IO>::value;
    constexpr int ES = (int)sizeof(IO);
    const int L = ch.L;
    const bool full = L == C;
    const auto rv = rsrc(p.v + ch.t0 * p.v_st + h * p.v_sh, L > 0 ? (L - 1) * p.v_st + D * ES : 0);
    const int vv = 4 * h32 * p.v_st + v0 * ES;
    auto vall = [&](bool in_soffset) {
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const int ro = (32 * (e >> 4) + 8 * ((e & 15) >> 2) + (e & 3)) * p.v_st;
            if constexpr (BF)
                vr.x[e] = in_soffset ? __builtin_amdgcn_raw_buffer_load_b16(rv, vv, ro, 0)
                                     : __builtin_amdgcn_raw_buffer_load_b16(rv, vv + ro, 0, 0);
            else
                vr.x[e] = in_soffset ? __builtin_amdgcn_raw_buffer_load_b32(rv, vv, ro, 0)
                                     : __builtin_amdgcn_raw_buffer_load_b32(rv, vv + ro, 0, 0);
        }
    };
    if (full) vall(true);
    else vall(false);
}

// bf16 V: each wave loads the 64 x 32 block of its own state columns with
// 16-byte loads (token 16 j + lane / 4, columns 32 ws + 8 (lane % 4) .. + 8);
// rows past the chunk end fall outside the buffer range and load zeros.
struct VWide {
    i32x4 x[4];
};
__device__ __forceinline__ void issue_v_wide_part(VWide &vw, const ScanParams &p, ChunkRef ch, int h, int ws, int lane,
                                                  int j) {
    const int L = ch.L;
    const auto rv = rsrc(p.v + ch.t0 * p.v_st + h * p.v_sh, L > 0 ? (L - 1) * p.v_st + D * 2 : 0);
    const int vo = (lane >> 2) * p.v_st + (32 * ws + 8 * (lane & 3)) * 2;
    vw.x[j] = __builtin_amdgcn_raw_buffer_load_b128(rv, vo + 16 * j * p.v_st, 0, 0);
}

// A wave's 64 x 32 staging block in LDS (bf16 V in, bf16 output out): kStageBytes
// per wave.  V goes in as 64-byte rows (token t at 64 t).  Output goes in by
// granule columns: granule g (columns 8 g .. 8 g + 7) of token t at g kStageCol
// + 16 t, the column stride padded by 64 bytes.  Staged from the transposed
// output tile (lane = token, registers 4 q .. 4 q + 3 = columns 8 q + 4 h32 +
// 0..3), the two lane halves first trade 8-byte pieces (permlane32 swap) so that
// every lane holds 8 consecutive columns, granule 2 p + h32: each half-wave then
// writes 512 contiguous bytes with 16-byte stores, and a quarter-wave reading 4
// tokens x 4 granules (the 64-byte output rows) touches 64 distinct banks.  An
// LDS probe under SQ_LDS_BANK_CONFLICT measured both patterns conflict-free; the
// earlier row-major block with rotated granules took 8-byte writes with ~4.5
// conflict cycles each.
constexpr int kStageCol = 64 * 16 + 64;
constexpr int kStageBytes = 4 * kStageCol;

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
    return __builtin_bit_cast(unsigned, bf16x2{(bf16)a, (bf16)b});
}
// Output rows 32 ib .. 32 ib + 31 of accumulator tile Y into the staging block.
__device__ __forceinline__ void stage_out_tile(char *st, const f32x16 &Y, int ib, int l32, int h32) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
        const int q0 = 2 * pp, q1 = 2 * pp + 1;
        const unsigned a0 = pack_bf16(Y[4 * q0], Y[4 * q0 + 1]), a1 = pack_bf16(Y[4 * q0 + 2], Y[4 * q0 + 3]);
        const unsigned b0 = pack_bf16(Y[4 * q1], Y[4 * q1 + 1]), b1 = pack_bf16(Y[4 * q1 + 2], Y[4 * q1 + 3]);
        // lanes 0..31 keep a (granule q0, columns +0..3) and take the other half's a
        // (columns +4..7); lanes 32..63 take the other half's b and keep their own
        const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
        *reinterpret_cast<i32x4 *>(st + (2 * pp + h32) * kStageCol + 16 * (32 * ib + l32)) =
            i32x4{(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
    }
}
// Granule g (16 bytes) of staged output token t.
__device__ __forceinline__ i32x4 staged_out(const char *st, int t, int g) {
    return *reinterpret_cast<const i32x4 *>(st + g * kStageCol + 16 * t);
}

__device__ __forceinline__ ChunkRef chunk_at(int64_t bos, int64_t eos, int c) {
    ChunkRef ch;
    ch.t0 = bos + (int64_t)c * C;
    const int64_t rem = eos - ch.t0;
    ch.L = rem <= 0 ? 0 : (rem >= C ? C : (int)rem);
    return ch;
}

// ---- state I/O: accumulator tiles S[b] (S^T rows k, column v0) <-> a V-major
// [128][128] block at `base` with row stride `rs` bytes.  Register r of half h32
// holds k = 32 b + acc_row(r, h32) in accumulator order (NAT = false) or
// k = 32 b + 16 (r / 8) + 8 h32 + r % 8 in natural operand order (NAT = true).
template <bool NAT> __device__ __forceinline__ int state_k(int bb, int r, int h32) {
    return NAT ? 32 * bb + 16 * (r >> 3) + 8 * h32 + (r & 7) : 32 * bb + acc_row(r, h32);
}

template <bool NAT>
__device__ __forceinline__ void load_state(f32x16 (&S)[4], const char *base, int rs, int dt, int v0, int h32) {
    const auto r = rsrc(base, (int64_t)D * rs);
    if (dt == GDN_F32) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {     // registers 4j .. 4j+3 hold 4 consecutive k
                const f32x4 x = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, v0 * rs + 4 * state_k<NAT>(bb, 4 * j, h32), 0, 0));
#pragma unroll
                for (int t = 0; t < 4; ++t) S[bb][4 * j + t] = x[t];
            }
    } else {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x4 x = __builtin_bit_cast(
                    bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, v0 * rs + 2 * state_k<NAT>(bb, 4 * j, h32), 0, 0));
#pragma unroll
                for (int t = 0; t < 4; ++t) S[bb][4 * j + t] = (float)x[t];
            }
    }
}

template <bool NAT>
__device__ __forceinline__ void store_state(const f32x16 (&S)[4], char *base, int rs, int dt, int v0, int h32) {
    const auto r = rsrc(base, (int64_t)D * rs);
    if (dt == GDN_F32) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x4 x;
#pragma unroll
                for (int t = 0; t < 4; ++t) x[t] = S[bb][4 * j + t];
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), r,
                                                       v0 * rs + 4 * state_k<NAT>(bb, 4 * j, h32), 0, 0);
            }
    } else {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x4 x;
#pragma unroll
                for (int t = 0; t < 4; ++t) x[t] = (bf16)S[bb][4 * j + t];
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), r,
                                                      v0 * rs + 2 * state_k<NAT>(bb, 4 * j, h32), 0, 0);
            }
    }
}

constexpr int64_t kMapBytes = (int64_t)D * D * 4;   // one fp32 [128][128] block of the workspace
// s_waitcnt operand for vmcnt(0) alone (expcnt and lgkmcnt at their maximum)
constexpr int kWaitVmcnt0 = 0x0F70;


}  // namespace dev
}  // namespace gdn
