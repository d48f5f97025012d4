// Split path of the scan for few long sequences: the plan (cu_seqlens ->
// segment table) and the state fix-up that chains the segments' maps.  The
// segment maps themselves and the final per-segment scan run the scan kernel
// (gdn_scan.hip) in its map and scan modes.  This is the context-parallel flow
// of "flashinfer.gdn_prefill" (Cake GDN CP section: per-segment map
// precompute, state fix-up, then the prefill of every segment from its fixed-up
// entry state) on one GPU; the recurrence is affine in the state, so a segment
// maps its entry state S to S M + N.
#include <hip/hip_runtime.h>

#include "gdn_device.h"

namespace gdn {
namespace {

using namespace dev;

// Plan: cu_seqlens -> segment table.  One workgroup; sequences in tiles of 256
// with a block-wide inclusive scan of their segment counts.
__global__ __launch_bounds__(256) void plan_kernel(const void *cu, int cu_i64, int N, int64_t lseg, SegEntry *segs,
                                                   int32_t *nsegs, int32_t *seg_first, int cap) {
    __shared__ int32_t part[256];
    const int tid = threadIdx.x;
    int base = 0;
    for (int n0 = 0; n0 < N; n0 += 256) {
        const int n = n0 + tid;
        int cnt = 0;
        int64_t bos = 0, eos = 0;
        if (n < N) {
            bos = load_cu(cu, n, cu_i64);
            eos = load_cu(cu, n + 1, cu_i64);
            const int64_t len = eos - bos;
            cnt = len <= 0 ? 1 : (int)((len + lseg - 1) / lseg);   // an empty sequence keeps one entry
        }
        part[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int v = tid >= off ? part[tid - off] : 0;
            __syncthreads();
            part[tid] += v;
            __syncthreads();
        }
        const int first = base + part[tid] - cnt;
        const int tile_total = part[255];
        if (n < N) {
            seg_first[n] = first;
            for (int sgi = 0; sgi < cnt; ++sgi) {
                const int idx = first + sgi;
                if (idx < cap) {
                    SegEntry e;
                    e.bos = bos + sgi * lseg;
                    e.eos = eos < bos + (sgi + 1) * lseg ? eos : bos + (sgi + 1) * lseg;
                    e.n = n;
                    e.first = sgi == 0;
                    e.last = sgi == cnt - 1;
                    e.pad = 0;
                    segs[idx] = e;
                }
            }
        }
        base += tile_total;
        __syncthreads();
    }
    if (tid == 0) {
        seg_first[N] = base;
        *nsegs = base < cap ? base : cap;
    }
}

// State fix-up: per (sequence, value head), S_in(i+1) = S_in(i) M_i + N_i over
// its segments, in fp32 (v_mfma_f32_32x32x2_f32).  With the state held as
// accumulator tiles of S^T (rows k, columns v):
//   (S M)^T[k][v] = sum_v' M[v'][k] S^T[v'][v]
// the accumulator is the B operand (contraction v' in accumulator order) and
// M, staged V-major in LDS, is read column-wise as the A operand.
__global__ __launch_bounds__(256) void fixup_kernel(const FixParams f) {
    constexpr int MLD = 132;
    __shared__ __attribute__((aligned(16))) float Ms[D * MLD];
    const int n = blockIdx.x / f.Hv, h = blockIdx.x % f.Hv;
    const int s0 = f.seg_first[n], cnt = f.seg_first[n + 1] - s0;
    if (cnt <= 1) return;
    const int tid = threadIdx.x, lane = tid & 63, ws = tid >> 6;
    const int h32 = lane >> 5, l32 = lane & 31, v0 = ws * 32 + l32;
    f32x16 S[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) S[bb] = zero16();
    const int64_t srow = state_row(f.sidx, f.sidx_i64, f.pool_rows, n);
    if (f.s_in && srow >= 0) load_state<false>(S, f.s_in + srow * f.si_n + h * f.si_h, f.si_v, f.si_dt, v0, h32);
    if (f.sidx)   // the first segment of a pooled sequence starts from this copy
        store_state<false>(S, reinterpret_cast<char *>(f.ws_sin) + ((int64_t)s0 * f.Hv + h) * kMapBytes, D * 4,
                           GDN_F32, v0, h32);
    for (int i = 0; i + 1 < cnt; ++i) {
        const int64_t off = ((int64_t)(s0 + i) * f.Hv + h) * kMapBytes;
        const float *Mg = reinterpret_cast<const float *>(reinterpret_cast<const char *>(f.ws_m) + off);
        // N_i (the product's accumulator) and M_i are fetched together, M in two
        // batches of eight 16-byte loads per thread, so a step waits for memory
        // about twice instead of once per load (232 -> 172 us for 15 steps of
        // 32 heads); the products themselves, 256 fp32 32x32x2 MFMAs per wave,
        // take about 7 us per step
        f32x16 Sn[4];
        load_state<false>(Sn, reinterpret_cast<const char *>(f.ws_n) + off, D * 4, GDN_F32, v0, h32);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            f32x4 t[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int u = tid + 256 * (8 * half + e), row = u >> 5, c4 = u & 31;
                t[e] = *reinterpret_cast<const f32x4 *>(Mg + row * D + 4 * c4);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int u = tid + 256 * (8 * half + e), row = u >> 5, c4 = u & 31;
                *reinterpret_cast<f32x4 *>(Ms + row * MLD + 4 * c4) = t[e];
            }
        }
        __syncthreads();
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int st = 0; st < 16; ++st)
                    Sn[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(Ms[(32 * cb + acc_row(st, h32)) * MLD + 32 * mb + l32],
                                                                  S[cb][st], Sn[mb], 0, 0, 0);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) S[bb] = Sn[bb];
        store_state<false>(S, reinterpret_cast<char *>(f.ws_sin) + ((int64_t)(s0 + i + 1) * f.Hv + h) * kMapBytes, D * 4,
                    GDN_F32, v0, h32);
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_plan(const void *cu, int cu_i64, int N, int64_t lseg, SegEntry *segs, int32_t *nsegs,
                       int32_t *seg_first, int cap, hipStream_t stream) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, cu, cu_i64, N, lseg, segs, nsegs, seg_first, cap);
    return hipGetLastError();
}

hipError_t launch_fixup(const FixParams &f, hipStream_t stream) {
    const int64_t blocks = (int64_t)f.N * f.Hv;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(fixup_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, f);
    return hipGetLastError();
}

}  // namespace gdn
