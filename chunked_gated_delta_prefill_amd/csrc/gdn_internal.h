// Internal interface between the host layer (gdn_api.hip) and the kernels
// (gdn_scan.hip).  Not installed; the public ABI is include/gdn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

constexpr int kHeadDim = 128;   // K = V = 128 (every shape on the API page)
constexpr int kChunk = 64;      // tokens per chunk, aligned to each sequence start

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
};

// Fused chunked scan: one workgroup per (sequence, value head).  io_bf16
// selects bf16 q/k/v/out (bf16 MFMA) or fp32 (fp32 MFMA).
hipError_t launch_fused_scan(const ScanParams &p, bool io_bf16, hipStream_t stream);

}  // namespace gdn
