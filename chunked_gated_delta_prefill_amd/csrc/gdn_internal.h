// Internal interface between the host layer (gdn_api.hip) and the kernels
// (gdn_scan.hip).  Not installed; the public ABI is include/gdn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

constexpr int kHeadDim = 128;   // K = V = 128 (every shape on the API page)
constexpr int kChunk = 64;      // tokens per chunk, aligned to each sequence start

// Everything one scan launch needs.  Strides are in elements.
struct ScanParams {
    const void *q, *k, *v;
    int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh;
    const void *g;                  // nullptr: all ones
    int64_t g_st, g_sh;
    int32_t g_dt;
    const void *beta;               // nullptr: all ones
    int64_t b_st, b_sh;
    int32_t b_dt;
    const void *cu;
    int32_t cu_i64;
    const void *s_in;               // nullptr: zero initial state
    int64_t si_n, si_h, si_v;
    int32_t si_dt;
    void *s_out;                    // nullptr: no final state
    int64_t so_n, so_h, so_v;
    int32_t so_dt;
    int32_t state_vec;              // state rows are 16-byte aligned (vector I/O)
    void *out;
    int64_t o_st, o_sh;
    float scale;
    int32_t N, Hqk, Hv, r;          // r = Hv / Hqk
    int32_t l2norm;
};

// Fused chunked scan: one workgroup per (sequence, group of `rg` value heads
// sharing one q/k head).  io_bf16 selects bf16 q/k/v/out (bf16 MFMA) or fp32
// (fp32 MFMA).  rg is 1 or 2 and must divide r.
hipError_t launch_fused_scan(const ScanParams &p, bool io_bf16, int rg, hipStream_t stream);

}  // namespace gdn
