// Host side of the C ABI declared in include/gdn.h: argument validation
// (no device access), device/arch checks, work planning and kernel enqueue.
//
// Error convention follows the pages: invalid inputs and unsupported
// configurations fail closed with a reason and no fallback ("flashinfer.
// gdn_prefill", Cake GDN CP section; "flashinfer.cudnn", Linear attention:
// the engine declines what it cannot serve and says why).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

const char *dt_name(int dt) {
    switch (dt) {
        case GDN_F32: return "f32";
        case GDN_BF16: return "bf16";
        case GDN_F16: return "f16";
        case GDN_I32: return "i32";
        case GDN_I64: return "i64";
        default: return "?";
    }
}

size_t dt_size(int dt) {
    switch (dt) {
        case GDN_F32: case GDN_I32: return 4;
        case GDN_BF16: case GDN_F16: return 2;
        case GDN_I64: return 8;
        default: return 0;
    }
}

int64_t numel(const gdn_tensor *t) {
    int64_t n = 1;
    for (int i = 0; i < t->ndim; ++i) n *= t->sizes[i];
    return n;
}

// Shape/stride checks shared by every tensor argument.
int check_basic(const gdn_tensor *t, const char *name, int ndim, std::string &msg, bool inner_contig = true) {
    if (t->ndim != ndim) {
        msg = std::string(name) + ": expected " + std::to_string(ndim) + " dims, got " + std::to_string(t->ndim);
        return GDN_ERR_INVALID_ARGUMENT;
    }
    if (dt_size(t->dtype) == 0) {
        msg = std::string(name) + ": unknown dtype code " + std::to_string(t->dtype);
        return GDN_ERR_INVALID_ARGUMENT;
    }
    for (int i = 0; i < ndim; ++i) {
        if (t->sizes[i] < 0 || t->strides[i] < 0) {
            msg = std::string(name) + ": negative size or stride";
            return GDN_ERR_INVALID_ARGUMENT;
        }
    }
    if (inner_contig && ndim > 0 && t->sizes[ndim - 1] > 1 && t->strides[ndim - 1] != 1) {
        msg = std::string(name) + ": innermost dimension must be contiguous (stride 1)";
        return GDN_ERR_INVALID_ARGUMENT;
    }
    if (t->data == nullptr && numel(t) > 0) {
        msg = std::string(name) + ": data is NULL";
        return GDN_ERR_INVALID_ARGUMENT;
    }
    return GDN_OK;
}

bool aligned16(const void *p, size_t esz, const int64_t *strides, int n) {
    if (reinterpret_cast<uintptr_t>(p) % 16) return false;
    for (int i = 0; i < n; ++i)
        if ((strides[i] * (int64_t)esz) % 16) return false;
    return true;
}

std::mutex g_dev_mu;
int g_dev_checked[64];   // 0 unknown, 1 gfx950, 2 other

int check_device(std::string &msg) {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        msg = "no HIP device visible";
        return GDN_ERR_NO_DEVICE;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        msg = "hipGetDevice failed";
        return GDN_ERR_NO_DEVICE;
    }
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (dev >= 0 && dev < 64 && g_dev_checked[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            msg = "hipGetDeviceProperties failed";
            return GDN_ERR_HIP;
        }
        g_dev_checked[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (g_dev_checked[dev] == 2) {
            msg = std::string("device ") + std::to_string(dev) + " is " + prop.gcnArchName +
                  "; this library is built for gfx950 only";
            return GDN_ERR_ARCH;
        }
    }
    if (dev >= 0 && dev < 64 && g_dev_checked[dev] == 2) {
        msg = "current device is not gfx950";
        return GDN_ERR_ARCH;
    }
    return GDN_OK;
}

}  // namespace

extern "C" const char *gdn_last_error(void) { return g_last_error.c_str(); }

extern "C" void gdn_release_workspace(void) {}

extern "C" int gdn_chunk_prefill(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v,
                                 const gdn_tensor *g, const gdn_tensor *beta, float scale,
                                 const gdn_tensor *cu_seqlens, const gdn_tensor *initial_state,
                                 const gdn_tensor *output_state, int use_qk_l2norm,
                                 int batch_invariant, const gdn_tensor *out, void *stream) {
    g_last_error.clear();
    std::string msg;
    int rc;
    if (!q || !k || !v || !cu_seqlens || !out)
        return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, cu_seqlens and out are required");

    // ---- q, k, v, out
    if ((rc = check_basic(q, "q", 3, msg))) return fail(rc, msg);
    if ((rc = check_basic(k, "k", 3, msg))) return fail(rc, msg);
    if ((rc = check_basic(v, "v", 3, msg))) return fail(rc, msg);
    if ((rc = check_basic(out, "out", 3, msg))) return fail(rc, msg);
    const int io = q->dtype;
    if (io == GDN_F16)
        return fail(GDN_ERR_UNSUPPORTED, "q/k/v in f16 are not supported (f32 or bf16)");
    if (io != GDN_F32 && io != GDN_BF16)
        return fail(GDN_ERR_INVALID_ARGUMENT, std::string("q: dtype ") + dt_name(io) + " is not a float type");
    if (k->dtype != io || v->dtype != io || out->dtype != io)
        return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v and out must share one dtype");
    const int64_t T = q->sizes[0], Hqk = q->sizes[1], Hv = v->sizes[1];
    if (q->sizes[2] != gdn::kHeadDim || k->sizes[2] != gdn::kHeadDim || v->sizes[2] != gdn::kHeadDim ||
        out->sizes[2] != gdn::kHeadDim)
        return fail(GDN_ERR_UNSUPPORTED, "head_dim must be 128 for q, k, v and out");
    if (k->sizes[0] != T || k->sizes[1] != Hqk)
        return fail(GDN_ERR_INVALID_ARGUMENT, "k must have the shape of q");
    if (v->sizes[0] != T || out->sizes[0] != T || out->sizes[1] != Hv)
        return fail(GDN_ERR_INVALID_ARGUMENT, "v and out must be [T, Hv, 128] with q's T");
    if (Hqk < 1 || Hv < 1)
        return fail(GDN_ERR_INVALID_ARGUMENT, "head counts must be positive");
    if (Hv % Hqk != 0)
        return fail(GDN_ERR_UNSUPPORTED, "Hv must be a multiple of Hqk (each q/k head serves Hv/Hqk value heads)");
    if (T > ((int64_t)1 << 40) || Hv > 65536)
        return fail(GDN_ERR_UNSUPPORTED, "problem too large");
    const size_t esz = dt_size(io);
    if (T > 0 && (!aligned16(q->data, esz, q->strides, 2) || !aligned16(k->data, esz, k->strides, 2)))
        return fail(GDN_ERR_UNSUPPORTED, "q and k rows must be 16-byte aligned (pointer and token/head strides)");

    // ---- gates
    if (g) {
        if ((rc = check_basic(g, "g", 2, msg, false))) return fail(rc, msg);
        if (g->sizes[0] != T || g->sizes[1] != Hv)
            return fail(GDN_ERR_INVALID_ARGUMENT, "g must be [T, Hv]");
        if (g->dtype != GDN_F32 && g->dtype != GDN_BF16 && g->dtype != GDN_F16)
            return fail(GDN_ERR_INVALID_ARGUMENT, "g must be f32, bf16 or f16");
    }
    if (beta) {
        if ((rc = check_basic(beta, "beta", 2, msg, false))) return fail(rc, msg);
        if (beta->sizes[0] != T || beta->sizes[1] != Hv)
            return fail(GDN_ERR_INVALID_ARGUMENT, "beta must be [T, Hv]");
        if (beta->dtype != GDN_F32 && beta->dtype != io)
            return fail(GDN_ERR_INVALID_ARGUMENT, "beta must be f32 or q's dtype");
    }

    // ---- cu_seqlens
    if ((rc = check_basic(cu_seqlens, "cu_seqlens", 1, msg))) return fail(rc, msg);
    if (cu_seqlens->dtype != GDN_I32 && cu_seqlens->dtype != GDN_I64)
        return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens must be i32 or i64");
    if (cu_seqlens->sizes[0] < 1 || cu_seqlens->data == nullptr)
        return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens must hold N + 1 >= 1 entries");
    if (cu_seqlens->sizes[0] > 1 && cu_seqlens->strides[0] != 1)
        return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens must be contiguous");
    const int64_t N = cu_seqlens->sizes[0] - 1;
    if (N > ((int64_t)1 << 24)) return fail(GDN_ERR_UNSUPPORTED, "too many sequences");

    // ---- states
    const gdn_tensor *st[2] = {initial_state, output_state};
    const char *st_name[2] = {"initial_state", "output_state"};
    for (int i = 0; i < 2; ++i) {
        if (!st[i]) continue;
        if ((rc = check_basic(st[i], st_name[i], 4, msg))) return fail(rc, msg);
        if (st[i]->dtype != GDN_F32 && st[i]->dtype != GDN_BF16)
            return fail(GDN_ERR_INVALID_ARGUMENT, std::string(st_name[i]) + " must be f32 or bf16");
        if (st[i]->sizes[0] != N || st[i]->sizes[1] != Hv || st[i]->sizes[2] != gdn::kHeadDim ||
            st[i]->sizes[3] != gdn::kHeadDim)
            return fail(GDN_ERR_INVALID_ARGUMENT, std::string(st_name[i]) + " must be [N, Hv, 128, 128]");
    }
    if (initial_state && output_state && initial_state->data == output_state->data && N > 0)
        return fail(GDN_ERR_ALIAS, "output_state must not alias initial_state");
    if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_ARGUMENT, "scale must be finite");

    // ---- device
    if ((rc = check_device(msg))) return fail(rc, msg);
    if (N == 0) return GDN_OK;

    gdn::ScanParams p{};
    p.q = q->data; p.k = k->data; p.v = v->data;
    p.q_st = q->strides[0]; p.q_sh = q->strides[1];
    p.k_st = k->strides[0]; p.k_sh = k->strides[1];
    p.v_st = v->strides[0]; p.v_sh = v->strides[1];
    p.g = g ? g->data : nullptr;
    p.g_st = g ? g->strides[0] : 0; p.g_sh = g ? g->strides[1] : 0; p.g_dt = g ? g->dtype : GDN_F32;
    p.beta = beta ? beta->data : nullptr;
    p.b_st = beta ? beta->strides[0] : 0; p.b_sh = beta ? beta->strides[1] : 0;
    p.b_dt = beta ? beta->dtype : GDN_F32;
    p.cu = cu_seqlens->data; p.cu_i64 = cu_seqlens->dtype == GDN_I64;
    p.s_in = initial_state ? initial_state->data : nullptr;
    if (initial_state) {
        p.si_n = initial_state->strides[0]; p.si_h = initial_state->strides[1];
        p.si_v = initial_state->strides[2]; p.si_dt = initial_state->dtype;
    }
    p.s_out = output_state ? output_state->data : nullptr;
    if (output_state) {
        p.so_n = output_state->strides[0]; p.so_h = output_state->strides[1];
        p.so_v = output_state->strides[2]; p.so_dt = output_state->dtype;
    }
    p.state_vec = 0;
    p.out = out->data; p.o_st = out->strides[0]; p.o_sh = out->strides[1];
    p.scale = scale == 0.0f ? 1.0f / std::sqrt((float)gdn::kHeadDim) : scale;
    p.N = (int32_t)N; p.Hqk = (int32_t)Hqk; p.Hv = (int32_t)Hv; p.r = (int32_t)(Hv / Hqk);
    p.l2norm = use_qk_l2norm != 0;
    (void)batch_invariant;   // the fused scan never splits a sequence

    const bool bf = io == GDN_BF16;
    const int rg = 1;
    hipError_t e = gdn::launch_fused_scan(p, bf, rg, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
    return GDN_OK;
}
