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
// with a block-wide inclusive scan of their segment counts, then the entries of
// the tile's sequences written by all threads together (one long sequence can
// hold a thousand one-chunk entries).
__global__ __launch_bounds__(256) void plan_kernel(const void *cu, int cu_i64, int N, int64_t lseg, SegEntry *segs,
                                                   int32_t *nsegs, int32_t *seg_first, int cap) {
    __shared__ int32_t part[256], tfirst[256], tcnt[256];
    __shared__ int64_t tbos[256], teos[256];
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
        tfirst[tid] = first;
        tcnt[tid] = cnt;
        tbos[tid] = bos;
        teos[tid] = eos;
        if (n < N) seg_first[n] = first;
        __syncthreads();
        const int ns = N - n0 < 256 ? N - n0 : 256;
        for (int sq = 0; sq < ns; ++sq) {
            const int c = tcnt[sq], f = tfirst[sq];
            const int64_t b0 = tbos[sq], e0 = teos[sq];
            for (int sgi = tid; sgi < c; sgi += 256) {
                const int idx = f + sgi;
                if (idx < cap) {
                    SegEntry e;
                    e.bos = b0 + sgi * lseg;
                    e.eos = e0 < b0 + (sgi + 1) * lseg ? e0 : b0 + (sgi + 1) * lseg;
                    e.n = n0 + sq;
                    e.first = sgi == 0;
                    e.last = sgi == c - 1;
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
//
// Rows of the state evolve independently (row v of S M needs row v of S only),
// so one workgroup takes one block of 32 state rows of a (sequence, head) and
// its wave w forms columns 32w .. 32w+31 of those rows: 64 MFMAs per step
// instead of 256.  After each step the four column blocks meet in LDS (Sx, in
// register order) to form the next step's B operand.  The next M and N are
// loaded into registers while the current products run.  The four row blocks
// of a head get workgroup ids 8 apart (one XCD), so M is fetched into one L2.
constexpr int kFixRowBlocks = D / 32;

__device__ __forceinline__ void load_block(f32x16 &S, const float *base, int bb, int v0, int h32) {
    const auto r = rsrc(base, (int64_t)D * D * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {   // registers 4j .. 4j+3 hold 4 consecutive k
        const f32x4 x = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (v0 * D + state_k<false>(bb, 4 * j, h32)) * 4, 0, 0));
#pragma unroll
        for (int t = 0; t < 4; ++t) S[4 * j + t] = x[t];
    }
}
__device__ __forceinline__ void store_block(const f32x16 &S, float *base, int bb, int v0, int h32) {
    const auto r = rsrc(base, (int64_t)D * D * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f32x4 x = {S[4 * j], S[4 * j + 1], S[4 * j + 2], S[4 * j + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), r,
                                               (v0 * D + state_k<false>(bb, 4 * j, h32)) * 4, 0, 0);
    }
}

struct MPieces {
    f32x4 x[16];
};
__device__ __forceinline__ void load_m(MPieces &m, const float *Mg, int tid) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int u = tid + 256 * e;
        m.x[e] = *reinterpret_cast<const f32x4 *>(Mg + (u >> 5) * D + 4 * (u & 31));
    }
}
__device__ __forceinline__ void put_m(float *Ms, int ld, const MPieces &m, int tid) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int u = tid + 256 * e;
        *reinterpret_cast<f32x4 *>(Ms + (u >> 5) * ld + 4 * (u & 31)) = m.x[e];
    }
}

__global__ __launch_bounds__(256) void fixup_kernel(const FixParams f) {
    constexpr int MLD = 132;
    __shared__ __attribute__((aligned(16))) float Ms[D * MLD];
    __shared__ __attribute__((aligned(16))) f32x4 Sx[4][4][64];   // [column block][register quad][lane]
    const int b = blockIdx.x;
    const int rb = (b >> 3) % kFixRowBlocks, pair = 8 * (b / (8 * kFixRowBlocks)) + (b & 7);
    if (pair >= f.N * f.Hv) return;
    const int n = pair / f.Hv, h = pair % f.Hv;
    const int s0 = f.seg_first[n], cnt = f.seg_first[n + 1] - s0;
    if (cnt <= 1) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int ws = __builtin_amdgcn_readfirstlane(tid >> 6);   // the column block this wave forms
    const int h32 = lane >> 5, l32 = lane & 31, v0 = 32 * rb + l32;
    f32x16 S[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) S[bb] = zero16();
    const int64_t srow = state_row(f.sidx, f.sidx_i64, f.pool_rows, n);
    if (f.s_in && srow >= 0) load_state<false>(S, f.s_in + srow * f.si_n + h * f.si_h, f.si_v, f.si_dt, v0, h32);
    auto map_at = [&](const float *base, int i) {
        return reinterpret_cast<const float *>(reinterpret_cast<const char *>(base) +
                                               ((int64_t)(s0 + i) * f.Hv + h) * kMapBytes);
    };
    auto sin_at = [&](int i) {
        return reinterpret_cast<float *>(reinterpret_cast<char *>(f.ws_sin) + ((int64_t)(s0 + i) * f.Hv + h) * kMapBytes);
    };
    // a pooled sequence's first segment starts from this copy (each wave its column block)
    if (f.sidx) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)   // constant indices keep S in registers
            if (bb == ws) store_block(S[bb], sin_at(0), bb, v0, h32);
    }
    // M_i in 16 16-byte pieces per thread: row u / 32, columns 4 (u % 32) .. +3
    // (u = tid + 256 e), held in registers from its load to its LDS store
    MPieces mreg;
    f32x16 Nn;
    load_m(mreg, map_at(f.ws_m, 0), tid);
    load_block(Nn, map_at(f.ws_n, 0), ws, v0, h32);
    put_m(Ms, MLD, mreg, tid);
    __syncthreads();
    for (int i = 0; i + 1 < cnt; ++i) {
        f32x16 Sn = Nn;
        const bool more = i + 2 < cnt;
        if (more) {   // the next step's M and N in flight during this step's products
            load_m(mreg, map_at(f.ws_m, i + 1), tid);
            load_block(Nn, map_at(f.ws_n, i + 1), ws, v0, h32);
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int st = 0; st < 16; ++st)
                Sn = __builtin_amdgcn_mfma_f32_32x32x2f32(Ms[(32 * cb + acc_row(st, h32)) * MLD + 32 * ws + l32],
                                                          S[cb][st], Sn, 0, 0, 0);
        store_block(Sn, sin_at(i + 1), ws, v0, h32);
        if (!more) break;   // the last segment's entry state was the last one needed
#pragma unroll
        for (int j = 0; j < 4; ++j) Sx[ws][j][lane] = f32x4{Sn[4 * j], Sn[4 * j + 1], Sn[4 * j + 2], Sn[4 * j + 3]};
        __syncthreads();   // every wave's products are done: Ms may be rewritten, Sx read
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 x = Sx[bb][j][lane];
#pragma unroll
                for (int t = 0; t < 4; ++t) S[bb][4 * j + t] = x[t];
            }
        put_m(Ms, MLD, mreg, tid);
        __syncthreads();   // M_{i+1} staged, and Sx read by every wave before it is rewritten
    }
}

}  // namespace

hipError_t launch_plan(const void *cu, int cu_i64, int N, int64_t lseg, SegEntry *segs, int32_t *nsegs,
                       int32_t *seg_first, int cap, hipStream_t stream) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, cu, cu_i64, N, lseg, segs, nsegs, seg_first, cap);
    return hipGetLastError();
}

hipError_t launch_fixup(const FixParams &f, hipStream_t stream) {
    const int64_t pairs = (int64_t)f.N * f.Hv;
    const int64_t blocks = ((pairs + 7) / 8) * 8 * kFixRowBlocks;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(fixup_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, f);
    return hipGetLastError();
}

}  // namespace gdn
