// Internal interface between the host layer (gdn_api.hip) and the kernels
// (gdn_scan.hip).  Not installed; the public ABI is include/gdn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

constexpr int kHeadDim = 128;   // K = V = 128 (every shape on the API page)
constexpr int kChunk = 64;      // tokens per chunk, aligned to each sequence start

// One work item of the split path: a run of whole chunks of one sequence.
struct SegEntry {
    int64_t bos, eos;          // token range [bos, eos)
    int32_t n;                 // sequence
    int32_t first, last;       // first / last segment of its sequence
    int32_t pad;
};

// Kernel modes: the scan proper, or one of the two segment maps of the split
// path (S_end = S_start M + N): N = scan from a zero state, M = scan of the
// identity with v = 0.  Map modes write no output rows.  kPrep runs only the
// state-independent preparation of single chunks (one work item per chunk
// entry of the table) and writes it to the prepared-chunk workspace.
enum ScanMode { kScan = 0, kMapN = 1, kMapM = 2, kPrep = 3 };

constexpr int kPrepChunks = 8;   // chunks per work item of the preparation pass

// One prepared chunk of one value head (bf16 q/k/v), as kPrep writes it and the
// prepared scan reads it.  T' = (I + A)^-1 diag(b) and the output tile P are
// stored as 16-byte pieces of their used blocks (rows 0..31: columns 0..31;
// rows 32..63: columns 0..63), row-major bf16 (a row of 64 holds 8 pieces);
// then the sigma-free row factors and the chunk's decay scalars.
constexpr int kPrepPieces = 32 * 4 + 32 * 8;                 // 16-byte pieces of one tile
constexpr int kPrepT = 0;                                     // T' pieces
constexpr int kPrepP = kPrepT + kPrepPieces * 16;             // P pieces
constexpr int kPrepRows = kPrepP + kPrepPieces * 16;          // [64] each: gamma_i rk_i, c gamma_i rq_i, rk_i exp(G_L - G_i)
constexpr int kPrepScalars = kPrepRows + 3 * kChunk * 4;      // gamma_L, 1 / gamma_L, G_L
constexpr int kPrepSlot = 13312;                              // bytes per (chunk, value head)
static_assert(kPrepScalars + 16 <= kPrepSlot && kPrepSlot % 256 == 0, "prepared slot");

// Everything one scan launch needs.  Per-row strides are in bytes and fit in
// 32 bits with 64 rows of headroom (the host checks); per-head and
// per-sequence strides are 64-bit.
struct ScanParams {
    const char *q, *k, *v;
    int32_t q_st, k_st, v_st;       // token strides (bytes)
    int64_t q_sh, k_sh, v_sh;       // head strides (bytes)
    const char *g;                  // nullptr: all ones
    int32_t g_st, g_dt;             // token stride (bytes), dtype
    int64_t g_sh;
    const char *beta;               // nullptr: all ones
    int32_t b_st, b_dt;
    int64_t b_sh;
    const void *cu;
    int32_t cu_i64;
    const char *s_in;               // nullptr: zero initial state
    int64_t si_n, si_h;             // bytes
    int32_t si_v, si_dt;            // row stride (bytes), dtype
    char *s_out;                    // nullptr: no final state
    int64_t so_n, so_h;
    int32_t so_v, so_dt;
    char *out;
    int32_t o_st;
    int64_t o_sh;
    float scale;
    int32_t N, Hqk, Hv, r;          // r = Hv / Hqk
    int32_t l2norm;
    // split path (segs == nullptr: one work item per sequence)
    const SegEntry *segs;
    const int32_t *nsegs;           // number of valid entries (device)
    int32_t seg_cap;                // entries the grid covers
    float *ws_n, *ws_m, *ws_sin;    // [seg_cap][Hv][128][128] fp32, V-major
    // state checkpoints (ck == nullptr: none): slot n * ck_per_seq + i holds the
    // state after (i + 1) * ck_every chunks of sequence n
    char *ck;
    int64_t ck_n, ck_h;             // slot and head strides (bytes)
    int32_t ck_v, ck_dt;            // row stride (bytes), dtype
    int32_t ck_per_seq, ck_every;   // slots per sequence, chunks between checkpoints
    // indexed state pool (sidx == nullptr: states indexed by sequence): sequence n
    // uses row sidx[n] of s_in / s_out; rows outside [0, pool_rows) mean no state
    const void *sidx;
    int32_t sidx_i64;
    int64_t pool_rows;
    // prepared chunks: chunk c of sequence n is slot ((seg_first[n] * prep_cps + c)
    // * Hv + h) * kPrepSlot, where the table (the split path's plan kernel) holds
    // segments of prep_cps chunks; kPrep writes the chunks of one segment per
    // work item
    char *prep;
    const int32_t *seg_first;
    int32_t prep_cps;
    // a range of chunks of every sequence (ph_len == 0: from ph_c0 to the end):
    // kPrep prepares only the segments that start in it, the prepared scan runs
    // only its chunks.  A range that does not end a sequence leaves the lazily
    // scaled state S~ and its scale sigma in `resume` (kResumeFloats per
    // (sequence, value head, 32-row block)), where the next range takes them up
    // exactly.
    int32_t ph_c0, ph_len;
    float *resume;
};
constexpr int kResumeFloats = 64 * 64 + 64;   // S~ (64 accumulator registers x 64 lanes), then sigma

// Fix-up of the split path: per (sequence, value head), serially over its
// segments, S_in(i+1) = S_in(i) M_i + N_i.
struct FixParams {
    const SegEntry *segs;
    const int32_t *seg_first;       // [N + 1] first segment of each sequence
    const char *s_in;               // caller's initial state (nullptr: zero)
    int64_t si_n, si_h;
    int32_t si_v, si_dt;
    const float *ws_n, *ws_m;
    float *ws_sin;
    int32_t N, Hv;
    const void *sidx;               // as ScanParams::sidx
    int32_t sidx_i64;
    int64_t pool_rows;
};

// One decode step (gdn_decode_step): byte strides over (sequence, head).
struct DecodeParams {
    const char *q, *k, *v, *g, *beta;
    int64_t q_sn, q_sh, k_sn, k_sh, v_sn, v_sh;
    int64_t g_sn, g_sh, b_sn, b_sh;
    int32_t io_dt, g_dt, b_dt;
    const char *s_in;
    int64_t si_n, si_h, si_v;
    int32_t si_dt;
    char *s_out;
    int64_t so_n, so_h, so_v;
    int32_t so_dt;
    char *out;
    int64_t o_sn, o_sh;
    float scale;
    int32_t l2norm, N, Hv, r;
    // indexed state pool (sidx == nullptr: state row n for sequence n): sequence n
    // uses row sidx[n] of s_in / s_out; rows outside [0, pool_rows) mean no state
    const void *sidx;
    int32_t sidx_i64;
    int64_t pool_rows;
};
hipError_t launch_decode(const DecodeParams &p, hipStream_t stream);

// Fused chunked scan: one workgroup per (sequence or segment, value head).
// io_bf16 selects bf16 q/k/v/out (bf16 MFMA) or fp32 (fp32 MFMA).
hipError_t launch_fused_scan(const ScanParams &p, bool io_bf16, int mode, hipStream_t stream);
// The eight-wave pipelined scan (bf16, scan mode, no checkpoints); same results
// as launch_fused_scan, one workgroup per CU.
hipError_t launch_piped_scan(const ScanParams &p, hipStream_t stream);
// The preparation of every chunk (kPrep over the chunk table, bf16), then the
// scan that consumes it; same results as launch_fused_scan.
hipError_t launch_prep(const ScanParams &p, hipStream_t stream);
// np = blocks of 32 state rows per workgroup (1 or 2): 4 / np workgroups per value head.
hipError_t launch_prepared_scan(const ScanParams &p, int np, hipStream_t stream);

// Split plan: cu_seqlens -> segment table of at most `cap` entries of `lseg`
// tokens (a multiple of the chunk), one entry for an empty sequence.
hipError_t launch_plan(const void *cu, int cu_i64, int N, int64_t lseg, SegEntry *segs, int32_t *nsegs,
                       int32_t *seg_first, int cap, hipStream_t stream);

hipError_t launch_fixup(const FixParams &f, hipStream_t stream);

}  // namespace gdn
