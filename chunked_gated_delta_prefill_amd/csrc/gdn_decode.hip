// One recurrent decode step of the gated delta rule on gfx950: the token that
// follows a prefill, consuming the V-major state the scan hands over
// ("flashinfer.gdn_prefill": the chunked scan builds the recurrent state before
// the decode loop takes over; "flashinfer.cudnn", Linear attention: the state
// crosses as [N, H, V, K] in float32 or bfloat16).  Per sequence n and value
// head h, with the old state S (rows v, columns k):
//
//     S' = a S + u k^T,   u = b (v - a S k)
//     o  = scale S' q  = scale (a (S q) + u (k . q))
//
// The step reads and writes the whole state once, so it is bound by HBM.  One
// workgroup of 4 waves covers 64 state rows of one (n, h); a row is 128 fp32
// values held by 32 lanes (4 consecutive columns each), so one 16-byte load
// per lane and row, and the two row sums (S k, S q) reduce over those 32 lanes.
// All eight rows of a wave are loaded before the first is used; state rows
// are streamed with non-temporal loads and stores (0.212 -> 0.179 ms on 256
// sequences x 32 heads).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(unsigned short b) { return __uint_as_float((uint32_t)b << 16); }

// round to nearest even (the hardware conversion)
__device__ __forceinline__ unsigned short f32_to_bf16(float f) { return __builtin_bit_cast(unsigned short, (__bf16)f); }

// four consecutive values as fp32; STREAM marks data read or written once
// (the state rows) as non-temporal, so it does not displace the q/k rows that
// the value heads of one q/k head share in the caches
template <bool STREAM = false>
__device__ __forceinline__ f32x4 load4(const char *base, int dt) {
    if (dt == GDN_F32) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(base);
        return STREAM ? __builtin_nontemporal_load(p) : *p;
    }
    const u16x4 *p = reinterpret_cast<const u16x4 *>(base);
    const u16x4 b = STREAM ? __builtin_nontemporal_load(p) : *p;
    return f32x4{bf16_to_f32(b[0]), bf16_to_f32(b[1]), bf16_to_f32(b[2]), bf16_to_f32(b[3])};
}

__device__ __forceinline__ void store4_stream(char *base, int dt, f32x4 x) {
    if (dt == GDN_F32) {
        __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(base));
    } else {
        const u16x4 b = {f32_to_bf16(x[0]), f32_to_bf16(x[1]), f32_to_bf16(x[2]), f32_to_bf16(x[3])};
        __builtin_nontemporal_store(b, reinterpret_cast<u16x4 *>(base));
    }
}

__device__ __forceinline__ float load1(const char *base, int dt) {
    if (dt == GDN_F32) return *reinterpret_cast<const float *>(base);
    const unsigned short b = *reinterpret_cast<const unsigned short *>(base);
    if (dt == GDN_BF16) return bf16_to_f32(b);
    return __half2float(__ushort_as_half(b));
}

// sum over the 32 lanes of a half-wave
__device__ __forceinline__ float sum32(float x) {
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) x += __shfl_xor(x, o, 32);
    return x;
}

constexpr int kRowsPerBlock = 64;
constexpr int kRowsPerWave = 16;   // 8 pairs of rows, one row per half-wave

__global__ __launch_bounds__(256) void decode_kernel(const DecodeParams p) {
    const int blocks_per_head = kHeadDim / kRowsPerBlock;
    const int64_t nh = blockIdx.x / blocks_per_head;
    const int rb = blockIdx.x % blocks_per_head;
    const int n = (int)(nh / p.Hv), h = (int)(nh % p.Hv), hq = h / p.r;
    const int tid = threadIdx.x, lane = tid & 63, ws = tid >> 6;
    const int c4 = (lane & 31) * 4, sub = lane >> 5;
    const int es_io = p.io_dt == GDN_F32 ? 4 : 2;

    // q, k columns c4 .. c4+3 in fp32, optionally L2-normalised over the 128 columns
    f32x4 qv = load4(p.q + n * p.q_sn + hq * p.q_sh + c4 * es_io, p.io_dt);
    f32x4 kv = load4(p.k + n * p.k_sn + hq * p.k_sh + c4 * es_io, p.io_dt);
    if (p.l2norm) {
        const float sq = sum32(qv[0] * qv[0] + qv[1] * qv[1] + qv[2] * qv[2] + qv[3] * qv[3]);
        const float sk = sum32(kv[0] * kv[0] + kv[1] * kv[1] + kv[2] * kv[2] + kv[3] * kv[3]);
        const float rq = __builtin_amdgcn_rsqf(sq + 1e-6f), rk = __builtin_amdgcn_rsqf(sk + 1e-6f);
        qv *= rq;
        kv *= rk;
    }
    const float kq = sum32(kv[0] * qv[0] + kv[1] * qv[1] + kv[2] * qv[2] + kv[3] * qv[3]);
    const float a = p.g ? load1(p.g + n * p.g_sn + h * p.g_sh, p.g_dt) : 1.f;
    const float b = p.beta ? load1(p.beta + n * p.b_sn + h * p.b_sh, p.b_dt) : 1.f;

    // the sequence's state row: n itself, or its entry in the pool index
    int64_t srow = n;
    if (p.sidx) {
        const int64_t ix = p.sidx_i64 ? reinterpret_cast<const int64_t *>(p.sidx)[n]
                                      : (int64_t)reinterpret_cast<const int32_t *>(p.sidx)[n];
        srow = (ix >= 0 && ix < p.pool_rows) ? ix : -1;
    }
    // this wave's rows: v = 64 rb + 16 ws + 2 j + sub
    const int v0 = kRowsPerBlock * rb + kRowsPerWave * ws + sub;
    const int es_si = p.si_dt == GDN_F32 ? 4 : 2, es_so = p.so_dt == GDN_F32 ? 4 : 2;
    const char *si = (p.s_in && srow >= 0) ? p.s_in + srow * p.si_n + h * p.si_h + c4 * es_si : nullptr;
    char *so = (p.s_out && srow >= 0) ? p.s_out + srow * p.so_n + h * p.so_h + c4 * es_so : nullptr;
    const char *vrow = p.v + n * p.v_sn + h * p.v_sh;
    f32x4 s[8];
    float vv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int v = v0 + 2 * j;
        s[j] = si ? load4<true>(si + (int64_t)v * p.si_v, p.si_dt) : f32x4{0.f, 0.f, 0.f, 0.f};
        vv[j] = load1(vrow + v * es_io, p.io_dt);
    }
    char *orow = p.out + n * p.o_sn + h * p.o_sh;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int v = v0 + 2 * j;
        const f32x4 x = s[j];
        const float sk = sum32(x[0] * kv[0] + x[1] * kv[1] + x[2] * kv[2] + x[3] * kv[3]);
        const float sq = sum32(x[0] * qv[0] + x[1] * qv[1] + x[2] * qv[2] + x[3] * qv[3]);
        const float u = b * (vv[j] - a * sk);
        if (so) {
            f32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = fmaf(a, x[e], u * kv[e]);
            store4_stream(so + (int64_t)v * p.so_v, p.so_dt, y);
        }
        if ((lane & 31) == 0) {
            const float o = p.scale * fmaf(a, sq, u * kq);
            if (p.io_dt == GDN_F32) *reinterpret_cast<float *>(orow + v * 4) = o;
            else *reinterpret_cast<unsigned short *>(orow + v * 2) = f32_to_bf16(o);
        }
    }
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream) {
    const int64_t blocks = (int64_t)p.N * p.Hv * (kHeadDim / kRowsPerBlock);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(decode_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdn
