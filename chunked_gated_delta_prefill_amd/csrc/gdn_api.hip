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
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

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

// No two elements of a written tensor share an address: its dims, taken in
// order of increasing stride (size-1 dims skipped), each start past the whole
// extent of the dims before them.
bool no_self_overlap(const gdn_tensor *t) {
    int order[4];
    int n = 0;
    for (int i = 0; i < t->ndim; ++i) {
        if (t->sizes[i] == 0) return true;   // no elements
        if (t->sizes[i] > 1) order[n++] = i;
    }
    for (int a = 1; a < n; ++a)   // insertion sort by stride
        for (int b = a; b > 0 && t->strides[order[b]] < t->strides[order[b - 1]]; --b) std::swap(order[b], order[b - 1]);
    int64_t extent = 1;   // elements spanned by the dims taken so far
    for (int a = 0; a < n; ++a) {
        const int d = order[a];
        if (t->strides[d] < extent) return false;
        extent = t->strides[d] * (t->sizes[d] - 1) + extent;
    }
    return true;
}

constexpr int64_t kMinSegment = 1024;   // shortest segment of the split path (16 chunks)

std::mutex g_dev_mu;
int g_dev_checked[64];   // 0 unknown, 1 gfx950, 2 other
int g_dev_cus[64];

int check_device(std::string &msg, int *dev_out, int *cus_out) {
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
        g_dev_cus[dev] = prop.multiProcessorCount;
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
    *dev_out = dev;
    *cus_out = (dev >= 0 && dev < 64 && g_dev_cus[dev] > 0) ? g_dev_cus[dev] : 256;
    return GDN_OK;
}

// Workspace of the split path: cached per (device, stream), grown on demand
// (the cached shape-specific workspace of "flashinfer.gdn_prefill", Cake GDN CP
// section).  A superseded buffer is never freed while the library may still
// use it: work enqueued earlier on the stream, or a HIP graph captured from an
// earlier call, keeps its address in kernel arguments.  Superseded buffers are
// kept on a retired list until gdn_release_workspace.  Growth is refused while
// the stream is capturing (an allocation is not capturable): an eager call of
// the largest shape on the stream sizes the workspace first.  Growth rounds up
// by half again, so a run of slowly growing calls retires few buffers.
//
// The prepared plan of a long launch also keeps a side stream (non-blocking, so
// it never waits on the legacy default stream by itself) and its events: the
// preparation of later chunk ranges runs there while the caller's stream scans
// the earlier ones (fork and join by events, so a captured graph holds both
// branches).
constexpr int kPhases = 4;                  // chunk ranges of a long prepared launch
constexpr int64_t kPhaseMinChunks = 64;     // average chunks per sequence below which it runs as one range
struct Workspace {
    void *ptr = nullptr;
    size_t bytes = 0;
    hipStream_t side = nullptr;
    hipEvent_t ev[kPhases] = {};            // ev[0]: range 0 prepared (fork); ev[i]: range i prepared
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::vector<std::pair<int, void *>> g_ws_retired;   // (device, buffer)

int get_workspace(int dev, hipStream_t st, size_t need, void **out, std::string &msg) {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    Workspace &w = g_ws[{dev, st}];
    if (w.bytes < need) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
            (void)hipGetLastError();
            msg = "hipStreamIsCapturing failed";
            return GDN_ERR_HIP;
        }
        if (cs != hipStreamCaptureStatusNone) {
            msg = "the split path needs " + std::to_string(need) + " bytes of workspace on this stream but has " +
                  std::to_string(w.bytes) + "; it cannot grow during graph capture (run one eager call of the "
                  "largest shape on the capture stream first)";
            return GDN_ERR_UNSUPPORTED;
        }
        const size_t grow = w.bytes + w.bytes / 2;
        const size_t bytes = need > grow ? need : grow;
        void *fresh = nullptr;
        if (hipMalloc(&fresh, bytes) != hipSuccess) {
            (void)hipGetLastError();
            msg = "workspace allocation of " + std::to_string(bytes) + " bytes failed";
            return GDN_ERR_HIP;
        }
        if (w.ptr) g_ws_retired.push_back({dev, w.ptr});
        w.ptr = fresh;
        w.bytes = bytes;
    }
    *out = w.ptr;
    return GDN_OK;
}

// The side stream and events of (dev, st), created on first use.  They are not
// created while `st` is capturing (a graph then runs the launch as one range,
// with bitwise the same results): *side stays nullptr.
int get_side(int dev, hipStream_t st, hipStream_t *side, hipEvent_t **ev, std::string &msg) {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    Workspace &w = g_ws[{dev, st}];
    *side = nullptr;
    if (!w.side) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
            (void)hipGetLastError();
            msg = "hipStreamIsCapturing failed";
            return GDN_ERR_HIP;
        }
        if (cs != hipStreamCaptureStatusNone) return GDN_OK;
        hipStream_t s = nullptr;
        if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) {
            (void)hipGetLastError();
            msg = "side stream creation failed";
            return GDN_ERR_HIP;
        }
        for (int i = 0; i < kPhases; ++i) {
            if (hipEventCreateWithFlags(&w.ev[i], hipEventDisableTiming) != hipSuccess) {
                (void)hipGetLastError();
                for (int j = 0; j < i; ++j) (void)hipEventDestroy(w.ev[j]);
                (void)hipStreamDestroy(s);
                msg = "event creation failed";
                return GDN_ERR_HIP;
            }
        }
        w.side = s;
    }
    *side = w.side;
    *ev = w.ev;
    return GDN_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Scratch of the no-allocation entry point (gdn_chunk_prefill_noalloc): the
// split path's workspace in one fixed device array.  Every GPU the library
// runs on holds its own copy until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address is looked
// up once per device (hipGetSymbolAddress, with the device current) and only
// that address is passed to kernels.  On a 256-CU gfx950 part every split plan
// needs at most 120 MiB.
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_dev[64];   // device address of `scratch` per device (nullptr: not looked up yet)

int scratch_address(int dev, void **out, std::string &msg) {
    if (dev < 0 || dev >= 64) {
        msg = "device index out of range for the no-allocation scratch";
        return GDN_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            msg = std::string("hipGetSymbolAddress of the scratch array failed: ") + hipGetErrorString(e);
            return GDN_ERR_HIP;
        }
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return GDN_OK;
}

}  // namespace

extern "C" const char *gdn_last_error(void) { return g_last_error.c_str(); }

extern "C" void gdn_release_workspace(void) {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto &kv : g_ws) {
        Workspace &w = kv.second;
        (void)hipSetDevice(kv.first.first);
        if (w.side) {
            (void)hipStreamSynchronize(w.side);
            for (int i = 0; i < kPhases; ++i) (void)hipEventDestroy(w.ev[i]);
            (void)hipStreamDestroy(w.side);
        }
        if (w.ptr) {
            (void)hipStreamSynchronize(kv.first.second);
            (void)hipFree(w.ptr);
        }
    }
    for (auto &r : g_ws_retired) {   // their users were enqueued before the current buffers' users
        (void)hipSetDevice(r.first);
        (void)hipFree(r.second);
    }
    (void)hipSetDevice(cur);
    g_ws.clear();
    g_ws_retired.clear();
    (void)hipGetLastError();
}

namespace {

// The host plan of one prefill call, from host-known sizes only (no device
// reads, so a call stays graph-capturable).
struct Plan {
    int kind;       // enum gdn_plan_kind
    int64_t lseg;   // segment length of the split path (0 without a split)
    int np;         // prepared scan: blocks of 32 state rows per workgroup (1 or 2)
};
// Largest prepared-chunk workspace (one slot per chunk and value head, ~208 bytes
// per token and head) a call takes; beyond it the pipelined scan prepares each
// chunk beside the state work instead.
constexpr double kPrepBudget = 8.0 * (1ull << 30);

Plan make_plan(int64_t N, int64_t T, int64_t Hv, bool bf, bool ck, bool batch_invariant, int cus) {
    // Split path (T precompute -> MN precompute -> state fix-up -> CP prefill) when
    // one work item per (sequence, head) leaves the GPU under-filled and the
    // sequences are long on average.  A split sequence runs three passes over each
    // segment (two maps, then the scan) plus one fix-up step per segment boundary,
    // and the split multiplies the work items, which may push a launch from one
    // to two workgroups per CU.  The two plans are compared in units of one chunk
    // at one workgroup per CU: a launch of W items costs one unit per chunk while
    // W <= CUs and 1.6 per round of two workgroups per CU above that (measured:
    // 5.0 and 7.9 us per chunk), a fix-up step and the extra launches about one
    // unit per segment.  Measured on 8 sequences of 8192 tokens (32 heads): the
    // fixed rule used before split them into 2 segments, 1.10 ms against 0.64 ms
    // unsplit.  Never with batch_invariant (the split changes the reduction order
    // of a sequence).  The host knows only T and N, so the plan uses the average
    // sequence length.
    const int64_t fill = 2 * (int64_t)cus;
    int64_t lseg = 0;
    if (!batch_invariant && N > 0 && N * Hv < fill && T > 0 && T >= 4 * kMinSegment * N) {
        lseg = (T * Hv + fill - 1) / fill;
        lseg = (lseg + gdn::kChunk - 1) / gdn::kChunk * gdn::kChunk;
        if (lseg < kMinSegment) lseg = kMinSegment;
        if (lseg >= T) lseg = 0;   // no sequence is long enough to split
    }
    if (lseg > 0) {
        auto per_chunk = [&](int64_t items) {
            return items <= cus ? 1.0 : 1.6 * (double)((items + fill - 1) / fill);
        };
        const int64_t avg = (T + N - 1) / N;
        const int64_t P = (avg + lseg - 1) / lseg;
        const double unsplit = (double)((avg + gdn::kChunk - 1) / gdn::kChunk) * per_chunk(N * Hv);
        const double split = (double)(lseg / gdn::kChunk) *
                                 (2.0 * per_chunk(N * (P - 1) * Hv) + per_chunk(N * P * Hv)) + (double)P;
        if (!(split < unsplit)) lseg = 0;
    }
    if (lseg > 0) return {GDN_PLAN_SPLIT, lseg, 0};
    // At most one work item per CU: the chain of chunks of one work item bounds
    // the call.  With CUs to spare for two or four per (sequence, head), the
    // state-independent preparation of every chunk runs first, in parallel over
    // all chunks ("T precompute"), and the scan that consumes it spreads each
    // head's state rows over 4 / np CUs.  Otherwise the pipelined scan prepares
    // chunk c + 1 beside the state work of chunk c.  Both give bitwise the results
    // of the four-wave scan, so the choice keeps batch_invariant results
    // independent of the batch.
    const double prep_bytes =
        (double)(T / ((int64_t)gdn::kChunk * gdn::kPrepChunks) + N + 1) * gdn::kPrepChunks * Hv * gdn::kPrepSlot;
    if (bf && !ck && N * Hv <= cus && prep_bytes > kPrepBudget) return {GDN_PLAN_PIPELINED_SCAN, 0, 0};
    if (bf && !ck && N * Hv <= cus) {
        if (N * Hv * 4 <= cus) return {GDN_PLAN_PREPARED_SCAN, 0, 1};
        if (N * Hv * 2 <= cus) return {GDN_PLAN_PREPARED_SCAN, 0, 2};
        return {GDN_PLAN_PIPELINED_SCAN, 0, 0};
    }
    return {GDN_PLAN_SCAN, 0, 0};
}

int prefill_impl(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v, const gdn_tensor *g,
                 const gdn_tensor *beta, float scale, const gdn_tensor *cu_seqlens, const gdn_tensor *initial_state,
                 const gdn_tensor *output_state, int use_qk_l2norm, int batch_invariant, const gdn_tensor *ckpt,
                 int32_t ck_per_seq, int64_t ck_interval, const gdn_tensor *state_indices, const gdn_tensor *out,
                 void *stream, bool noalloc = false) {
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
    // v rows are read and out rows written in 16-byte pieces
    if (T > 0 && (!aligned16(v->data, esz, v->strides, 2) || !aligned16(out->data, esz, out->strides, 2)))
        return fail(GDN_ERR_UNSUPPORTED, "v and out rows must be 16-byte aligned (pointer and token/head strides)");
    if (!no_self_overlap(out))
        return fail(GDN_ERR_UNSUPPORTED, "out must not overlap itself (e.g. a head stride below 128 elements)");

    // Per-row offsets inside one 64-token chunk are 32-bit; rows must not overlap.
    const int64_t kRowLimit = ((int64_t)1 << 31) / (gdn::kChunk + 1);
    const gdn_tensor *rows[4] = {q, k, v, out};
    for (const gdn_tensor *t : rows)
        if (T > 1 && (t->strides[0] < gdn::kHeadDim || t->strides[0] * (int64_t)esz >= kRowLimit))
            return fail(GDN_ERR_UNSUPPORTED, "token strides of q, k, v and out must be >= 128 elements "
                                             "and < 32 MiB");

    // ---- gates
    if (g) {
        if ((rc = check_basic(g, "g", 2, msg, false))) return fail(rc, msg);
        if (g->sizes[0] != T || g->sizes[1] != Hv)
            return fail(GDN_ERR_INVALID_ARGUMENT, "g must be [T, Hv]");
        if (g->dtype != GDN_F32 && g->dtype != GDN_BF16 && g->dtype != GDN_F16)
            return fail(GDN_ERR_INVALID_ARGUMENT, "g must be f32, bf16 or f16");
        if (T > 1 && g->strides[0] * (int64_t)dt_size(g->dtype) >= kRowLimit)
            return fail(GDN_ERR_UNSUPPORTED, "g token stride too large");
    }
    if (beta) {
        if ((rc = check_basic(beta, "beta", 2, msg, false))) return fail(rc, msg);
        if (beta->sizes[0] != T || beta->sizes[1] != Hv)
            return fail(GDN_ERR_INVALID_ARGUMENT, "beta must be [T, Hv]");
        if (beta->dtype != GDN_F32 && beta->dtype != io)
            return fail(GDN_ERR_INVALID_ARGUMENT, "beta must be f32 or q's dtype");
        if (T > 1 && beta->strides[0] * (int64_t)dt_size(beta->dtype) >= kRowLimit)
            return fail(GDN_ERR_UNSUPPORTED, "beta token stride too large");
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
    // one workgroup per (sequence, value head), rounded up to groups of 8 q/k heads
    if ((N + 8) * Hv > ((int64_t)1 << 30))
        return fail(GDN_ERR_UNSUPPORTED, "too many (sequence, value head) pairs for one launch");

    // ---- states
    const gdn_tensor *st[2] = {initial_state, output_state};
    const char *st_name[2] = {"initial_state", "output_state"};
    for (int i = 0; i < 2; ++i) {
        if (!st[i]) continue;
        if ((rc = check_basic(st[i], st_name[i], 4, msg))) return fail(rc, msg);
        if (st[i]->dtype != GDN_F32 && st[i]->dtype != GDN_BF16)
            return fail(GDN_ERR_INVALID_ARGUMENT, std::string(st_name[i]) + " must be f32 or bf16");
        if ((!state_indices && st[i]->sizes[0] != N) || st[i]->sizes[1] != Hv || st[i]->sizes[2] != gdn::kHeadDim ||
            st[i]->sizes[3] != gdn::kHeadDim)
            return fail(GDN_ERR_INVALID_ARGUMENT, std::string(st_name[i]) + " must be [N, Hv, 128, 128]");
    }
    for (int i = 0; i < 2; ++i) {
        if (!st[i] || N == 0 || st[i]->sizes[0] == 0) continue;
        const int64_t se = (int64_t)dt_size(st[i]->dtype);
        if (!aligned16(st[i]->data, (size_t)se, st[i]->strides, 3) || st[i]->strides[2] < gdn::kHeadDim ||
            st[i]->strides[2] * se * gdn::kHeadDim >= kRowLimit)
            return fail(GDN_ERR_UNSUPPORTED, std::string(st_name[i]) +
                                                 ": rows must be 16-byte aligned, >= 128 elements apart (pointer and strides)");
    }
    if (output_state && !no_self_overlap(output_state))
        return fail(GDN_ERR_UNSUPPORTED, "output_state must not overlap itself");
    if (!state_indices && initial_state && output_state && initial_state->data == output_state->data && N > 0)
        return fail(GDN_ERR_ALIAS, "output_state must not alias initial_state");
    if (state_indices) {
        if ((rc = check_basic(state_indices, "state_indices", 1, msg))) return fail(rc, msg);
        if (state_indices->dtype != GDN_I32 && state_indices->dtype != GDN_I64)
            return fail(GDN_ERR_INVALID_ARGUMENT, "state_indices must be i32 or i64");
        if (state_indices->sizes[0] != N || (N > 0 && state_indices->data == nullptr))
            return fail(GDN_ERR_INVALID_ARGUMENT, "state_indices must hold N entries");
    }
    if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_ARGUMENT, "scale must be finite");

    // ---- state checkpoints
    if (ckpt) {
        if ((rc = check_basic(ckpt, "checkpoints", 4, msg))) return fail(rc, msg);
        if (ckpt->dtype != GDN_F32 && ckpt->dtype != GDN_BF16)
            return fail(GDN_ERR_INVALID_ARGUMENT, "checkpoints must be f32 or bf16");
        if (ck_per_seq < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "checkpoints_per_sequence must be >= 1");
        if (ck_interval < gdn::kChunk || ck_interval % gdn::kChunk != 0 || ck_interval > ((int64_t)1 << 30))
            return fail(GDN_ERR_UNSUPPORTED, "checkpoint_interval must be a positive multiple of 64 tokens");
        if (ckpt->sizes[0] != N * ck_per_seq || ckpt->sizes[1] != Hv || ckpt->sizes[2] != gdn::kHeadDim ||
            ckpt->sizes[3] != gdn::kHeadDim)
            return fail(GDN_ERR_INVALID_ARGUMENT, "checkpoints must be [N * checkpoints_per_sequence, Hv, 128, 128]");
        const int64_t se = (int64_t)dt_size(ckpt->dtype);
        if (N > 0 && (!aligned16(ckpt->data, (size_t)se, ckpt->strides, 3) || ckpt->strides[2] < gdn::kHeadDim ||
                      ckpt->strides[2] * se * gdn::kHeadDim >= kRowLimit))
            return fail(GDN_ERR_UNSUPPORTED, "checkpoints: rows must be 16-byte aligned, >= 128 elements apart");
        if (!no_self_overlap(ckpt))
            return fail(GDN_ERR_UNSUPPORTED, "checkpoints must not overlap itself");
        if (N > 0 && ((initial_state && ckpt->data == initial_state->data) ||
                      (output_state && ckpt->data == output_state->data)))
            return fail(GDN_ERR_ALIAS, "checkpoints must not alias initial_state or output_state");
    }

    // ---- device
    int dev = 0, cus = 256;
    if ((rc = check_device(msg, &dev, &cus))) return fail(rc, msg);
    if (N == 0) return GDN_OK;

    gdn::ScanParams p{};
    const int64_t es = (int64_t)esz;
    p.q = static_cast<const char *>(q->data);
    p.k = static_cast<const char *>(k->data);
    p.v = static_cast<const char *>(v->data);
    p.q_st = (int32_t)(q->strides[0] * es); p.q_sh = q->strides[1] * es;
    p.k_st = (int32_t)(k->strides[0] * es); p.k_sh = k->strides[1] * es;
    p.v_st = (int32_t)(v->strides[0] * es); p.v_sh = v->strides[1] * es;
    if (g) {
        const int64_t ge = (int64_t)dt_size(g->dtype);
        p.g = static_cast<const char *>(g->data);
        p.g_st = (int32_t)(g->strides[0] * ge); p.g_sh = g->strides[1] * ge; p.g_dt = g->dtype;
    }
    if (beta) {
        const int64_t be = (int64_t)dt_size(beta->dtype);
        p.beta = static_cast<const char *>(beta->data);
        p.b_st = (int32_t)(beta->strides[0] * be); p.b_sh = beta->strides[1] * be; p.b_dt = beta->dtype;
    }
    p.cu = cu_seqlens->data; p.cu_i64 = cu_seqlens->dtype == GDN_I64;
    if (initial_state) {
        const int64_t se = (int64_t)dt_size(initial_state->dtype);
        p.s_in = static_cast<const char *>(initial_state->data);
        p.si_n = initial_state->strides[0] * se; p.si_h = initial_state->strides[1] * se;
        p.si_v = (int32_t)(initial_state->strides[2] * se); p.si_dt = initial_state->dtype;
    }
    if (output_state) {
        const int64_t se = (int64_t)dt_size(output_state->dtype);
        p.s_out = static_cast<char *>(output_state->data);
        p.so_n = output_state->strides[0] * se; p.so_h = output_state->strides[1] * se;
        p.so_v = (int32_t)(output_state->strides[2] * se); p.so_dt = output_state->dtype;
    }
    p.out = static_cast<char *>(out->data);
    p.o_st = (int32_t)(out->strides[0] * es); p.o_sh = out->strides[1] * es;
    p.scale = scale == 0.0f ? 1.0f / std::sqrt((float)gdn::kHeadDim) : scale;
    p.N = (int32_t)N; p.Hqk = (int32_t)Hqk; p.Hv = (int32_t)Hv; p.r = (int32_t)(Hv / Hqk);
    if (state_indices) {
        p.sidx = state_indices->data;
        p.sidx_i64 = state_indices->dtype == GDN_I64;
        p.pool_rows = initial_state ? initial_state->sizes[0] : 0;
    }
    if (ckpt) {
        const int64_t se = (int64_t)dt_size(ckpt->dtype);
        p.ck = static_cast<char *>(ckpt->data);
        p.ck_n = ckpt->strides[0] * se; p.ck_h = ckpt->strides[1] * se;
        p.ck_v = (int32_t)(ckpt->strides[2] * se); p.ck_dt = ckpt->dtype;
        p.ck_per_seq = ck_per_seq; p.ck_every = (int32_t)(ck_interval / gdn::kChunk);
    }
    p.l2norm = use_qk_l2norm != 0;
    const bool bf = io == GDN_BF16;
    hipStream_t hs = static_cast<hipStream_t>(stream);

    Plan plan = make_plan(N, T, Hv, bf, p.ck != nullptr, batch_invariant != 0, cus);
    // the no-allocation entry point has no room for prepared chunks: the
    // pipelined scan gives the same results without a workspace
    if (noalloc && plan.kind == GDN_PLAN_PREPARED_SCAN) plan.kind = GDN_PLAN_PIPELINED_SCAN;
    const int64_t lseg = plan.lseg;
    hipError_t e;
    if (plan.kind == GDN_PLAN_PREPARED_SCAN) {
        // table of segments of kPrepChunks chunks (the split path's plan kernel), the
        // prepared chunks (one preparation work item per segment and head), then
        // the scan over them.  A long launch whose scan leaves at least half the
        // CUs free runs in kPhases ranges of chunks: the preparation of range 0
        // first, then the scan of each range on this stream while the side stream
        // prepares the later ones on the free CUs.  The scan leaves S~ and its
        // scale between ranges as they are, so the results are bitwise those of
        // one range.  (Measured: one 65,536-token sequence on 32 heads, 128 scan
        // workgroups, -7%; 2 x 32,768 tokens, 256 scan workgroups, +6%.)
        const int64_t lprep = (int64_t)gdn::kChunk * gdn::kPrepChunks;
        const int64_t cap = T / lprep + N + 1;
        const size_t seg_bytes = align_up((size_t)cap * sizeof(gdn::SegEntry), 256);
        const size_t first_bytes = align_up((size_t)(N + 2) * sizeof(int32_t), 256);
        const size_t prep_bytes = (size_t)cap * gdn::kPrepChunks * (size_t)Hv * gdn::kPrepSlot;
        const int64_t avg_chunks = N > 0 ? ((T + N - 1) / N + gdn::kChunk - 1) / gdn::kChunk : 0;
        const int64_t scan_wgs = N * Hv * (4 / plan.np);
        int nph = avg_chunks >= kPhaseMinChunks && 2 * scan_wgs <= cus ? kPhases : 1;
        // range length: a whole number of preparation segments, so every segment
        // falls in one range; the last range runs to the end of every sequence
        const int64_t ph = ((avg_chunks + kPhases - 1) / kPhases + gdn::kPrepChunks - 1) / gdn::kPrepChunks *
                           gdn::kPrepChunks;
        const size_t resume_bytes = (size_t)N * Hv * 4 * gdn::kResumeFloats * sizeof(float);
        hipStream_t side = nullptr;
        hipEvent_t *ev = nullptr;
        if (nph > 1) {
            if ((rc = get_side(dev, hs, &side, &ev, msg))) return fail(rc, msg);
            if (!side) nph = 1;
        }
        void *wsp = nullptr;
        if ((rc = get_workspace(dev, hs, seg_bytes + first_bytes + prep_bytes + (nph > 1 ? resume_bytes : 0), &wsp,
                                msg)))
            return fail(rc, msg);
        char *w = static_cast<char *>(wsp);
        gdn::SegEntry *segs = reinterpret_cast<gdn::SegEntry *>(w);
        int32_t *seg_first = reinterpret_cast<int32_t *>(w + seg_bytes);
        int32_t *nsegs = seg_first + (N + 1);
        gdn::ScanParams pp = p;
        pp.segs = segs;
        pp.nsegs = nsegs;
        pp.seg_cap = (int32_t)cap;
        pp.prep = w + seg_bytes + first_bytes;
        pp.prep_cps = gdn::kPrepChunks;
        gdn::ScanParams ps = p;
        ps.prep = pp.prep;
        ps.prep_cps = gdn::kPrepChunks;
        ps.seg_first = seg_first;
        if (nph == 1) {
            if ((e = gdn::launch_plan(p.cu, p.cu_i64, (int)N, lprep, segs, nsegs, seg_first, (int)cap, hs)) !=
                    hipSuccess ||
                (e = gdn::launch_prep(pp, hs)) != hipSuccess ||
                (e = gdn::launch_prepared_scan(ps, plan.np, hs)) != hipSuccess)
                return fail(GDN_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
            return GDN_OK;
        }
        float *resume = reinterpret_cast<float *>(w + seg_bytes + first_bytes + prep_bytes);
        auto range = [&](gdn::ScanParams q, int i) {
            q.ph_c0 = (int32_t)(i * ph);
            q.ph_len = i + 1 < nph ? (int32_t)ph : 0;
            q.resume = resume;
            return q;
        };
        if ((e = gdn::launch_plan(p.cu, p.cu_i64, (int)N, lprep, segs, nsegs, seg_first, (int)cap, hs)) != hipSuccess ||
            (e = gdn::launch_prep(range(pp, 0), hs)) != hipSuccess || (e = hipEventRecord(ev[0], hs)) != hipSuccess ||
            (e = hipStreamWaitEvent(side, ev[0], 0)) != hipSuccess)
            return fail(GDN_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
        for (int i = 1; i < nph; ++i)
            if ((e = gdn::launch_prep(range(pp, i), side)) != hipSuccess || (e = hipEventRecord(ev[i], side)) != hipSuccess)
                return fail(GDN_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
        for (int i = 0; i < nph; ++i)
            if ((i > 0 && (e = hipStreamWaitEvent(hs, ev[i], 0)) != hipSuccess) ||
                (e = gdn::launch_prepared_scan(range(ps, i), plan.np, hs)) != hipSuccess)
                return fail(GDN_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
        return GDN_OK;
    }
    if (lseg == 0) {
        if (plan.kind == GDN_PLAN_PIPELINED_SCAN) e = gdn::launch_piped_scan(p, hs);
        else e = gdn::launch_fused_scan(p, bf, gdn::kScan, hs);
        if (e != hipSuccess) return fail(GDN_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
        return GDN_OK;
    }
    const int64_t cap = T / lseg + N + 1;
    const size_t seg_bytes = align_up((size_t)cap * sizeof(gdn::SegEntry), 256);
    const size_t first_bytes = align_up((size_t)(N + 2) * sizeof(int32_t), 256);
    const size_t map_bytes = (size_t)cap * (size_t)Hv * gdn::kHeadDim * gdn::kHeadDim * sizeof(float);
    const size_t ws_bytes = seg_bytes + first_bytes + 3 * map_bytes;
    void *wsp = nullptr;
    if (noalloc) {
        if (ws_bytes > kScratchBytes)
            return fail(GDN_ERR_UNSUPPORTED, "the split plan needs " + std::to_string(ws_bytes) +
                                                 " bytes of scratch; the no-allocation entry point holds " +
                                                 std::to_string(kScratchBytes));
        if ((rc = scratch_address(dev, &wsp, msg))) return fail(rc, msg);
    } else if ((rc = get_workspace(dev, hs, ws_bytes, &wsp, msg))) {
        return fail(rc, msg);
    }
    char *w = static_cast<char *>(wsp);
    gdn::SegEntry *segs = reinterpret_cast<gdn::SegEntry *>(w);
    int32_t *seg_first = reinterpret_cast<int32_t *>(w + seg_bytes);
    int32_t *nsegs = seg_first + (N + 1);
    p.segs = segs;
    p.nsegs = nsegs;
    p.seg_cap = (int32_t)cap;
    p.ws_n = reinterpret_cast<float *>(w + seg_bytes + first_bytes);
    p.ws_m = reinterpret_cast<float *>(w + seg_bytes + first_bytes + map_bytes);
    p.ws_sin = reinterpret_cast<float *>(w + seg_bytes + first_bytes + 2 * map_bytes);
    gdn::FixParams f{};
    f.segs = segs;
    f.seg_first = seg_first;
    f.s_in = p.s_in; f.si_n = p.si_n; f.si_h = p.si_h; f.si_v = p.si_v; f.si_dt = p.si_dt;
    f.ws_n = p.ws_n; f.ws_m = p.ws_m; f.ws_sin = p.ws_sin;
    f.N = (int32_t)N; f.Hv = (int32_t)Hv;
    f.sidx = p.sidx; f.sidx_i64 = p.sidx_i64; f.pool_rows = p.pool_rows;
    if ((e = gdn::launch_plan(p.cu, p.cu_i64, (int)N, lseg, segs, nsegs, seg_first, (int)cap, hs)) != hipSuccess ||
        (e = gdn::launch_fused_scan(p, bf, gdn::kMapN, hs)) != hipSuccess ||
        (e = gdn::launch_fused_scan(p, bf, gdn::kMapM, hs)) != hipSuccess ||
        (e = gdn::launch_fixup(f, hs)) != hipSuccess ||
        (e = gdn::launch_fused_scan(p, bf, gdn::kScan, hs)) != hipSuccess)
        return fail(GDN_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
    return GDN_OK;
}

}  // namespace

extern "C" int gdn_chunk_prefill(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v,
                                 const gdn_tensor *g, const gdn_tensor *beta, float scale,
                                 const gdn_tensor *cu_seqlens, const gdn_tensor *initial_state,
                                 const gdn_tensor *output_state, int use_qk_l2norm,
                                 int batch_invariant, const gdn_tensor *out, void *stream) {
    return prefill_impl(q, k, v, g, beta, scale, cu_seqlens, initial_state, output_state, use_qk_l2norm,
                        batch_invariant, nullptr, 0, 0, nullptr, out, stream);
}

extern "C" int gdn_chunk_prefill_noalloc(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v,
                                         const gdn_tensor *g, const gdn_tensor *beta, float scale,
                                         const gdn_tensor *cu_seqlens, const gdn_tensor *initial_state,
                                         const gdn_tensor *output_state, int use_qk_l2norm,
                                         int batch_invariant, const gdn_tensor *out, void *stream) {
    return prefill_impl(q, k, v, g, beta, scale, cu_seqlens, initial_state, output_state, use_qk_l2norm,
                        batch_invariant, nullptr, 0, 0, nullptr, out, stream, true);
}

extern "C" int gdn_chunk_prefill_checkpointed(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v,
                                              const gdn_tensor *g, const gdn_tensor *beta, float scale,
                                              const gdn_tensor *cu_seqlens, const gdn_tensor *initial_state,
                                              const gdn_tensor *output_state, int use_qk_l2norm,
                                              int batch_invariant, const gdn_tensor *checkpoints,
                                              int32_t checkpoints_per_sequence, int64_t checkpoint_interval,
                                              const gdn_tensor *out, void *stream) {
    if (!checkpoints) {
        g_last_error = "checkpoints is required (use gdn_chunk_prefill without checkpoints)";
        return GDN_ERR_INVALID_ARGUMENT;
    }
    return prefill_impl(q, k, v, g, beta, scale, cu_seqlens, initial_state, output_state, use_qk_l2norm,
                        batch_invariant, checkpoints, checkpoints_per_sequence, checkpoint_interval, nullptr, out,
                        stream);
}

extern "C" int gdn_chunk_prefill_pooled(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v,
                                        const gdn_tensor *g, const gdn_tensor *beta, float scale,
                                        const gdn_tensor *cu_seqlens, const gdn_tensor *state_pool,
                                        const gdn_tensor *state_indices, int use_qk_l2norm, int batch_invariant,
                                        const gdn_tensor *out, void *stream) {
    if (!state_pool || !state_indices) {
        g_last_error = "state_pool and state_indices are required";
        return GDN_ERR_INVALID_ARGUMENT;
    }
    return prefill_impl(q, k, v, g, beta, scale, cu_seqlens, state_pool, state_pool, use_qk_l2norm, batch_invariant,
                        nullptr, 0, 0, state_indices, out, stream);
}

namespace {

int decode_impl(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v, const gdn_tensor *g,
                const gdn_tensor *beta, float scale, const gdn_tensor *state_in, const gdn_tensor *state_out,
                const gdn_tensor *state_indices, int use_qk_l2norm, const gdn_tensor *out, void *stream) {
    g_last_error.clear();
    std::string msg;
    int rc;
    if (!q || !k || !v || !out) return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v and out are required");
    if ((rc = check_basic(q, "q", 3, msg))) return fail(rc, msg);
    if ((rc = check_basic(k, "k", 3, msg))) return fail(rc, msg);
    if ((rc = check_basic(v, "v", 3, msg))) return fail(rc, msg);
    if ((rc = check_basic(out, "out", 3, msg))) return fail(rc, msg);
    const int io = q->dtype;
    if (io == GDN_F16) return fail(GDN_ERR_UNSUPPORTED, "q/k/v in f16 are not supported (f32 or bf16)");
    if (io != GDN_F32 && io != GDN_BF16)
        return fail(GDN_ERR_INVALID_ARGUMENT, std::string("q: dtype ") + dt_name(io) + " is not a float type");
    if (k->dtype != io || v->dtype != io || out->dtype != io)
        return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v and out must share one dtype");
    const int64_t N = q->sizes[0], Hqk = q->sizes[1], Hv = v->sizes[1];
    if (q->sizes[2] != gdn::kHeadDim || k->sizes[2] != gdn::kHeadDim || v->sizes[2] != gdn::kHeadDim ||
        out->sizes[2] != gdn::kHeadDim)
        return fail(GDN_ERR_UNSUPPORTED, "head_dim must be 128 for q, k, v and out");
    if (k->sizes[0] != N || k->sizes[1] != Hqk) return fail(GDN_ERR_INVALID_ARGUMENT, "k must have the shape of q");
    if (v->sizes[0] != N || out->sizes[0] != N || out->sizes[1] != Hv)
        return fail(GDN_ERR_INVALID_ARGUMENT, "v and out must be [N, Hv, 128] with q's N");
    if (Hqk < 1 || Hv < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "head counts must be positive");
    if (Hv % Hqk != 0)
        return fail(GDN_ERR_UNSUPPORTED, "Hv must be a multiple of Hqk (each q/k head serves Hv/Hqk value heads)");
    if (N > ((int64_t)1 << 24) || Hv > 65536) return fail(GDN_ERR_UNSUPPORTED, "problem too large");
    if (N * Hv > ((int64_t)1 << 29))   // two workgroups per (sequence, value head)
        return fail(GDN_ERR_UNSUPPORTED, "too many (sequence, value head) pairs for one launch");
    const size_t esz = dt_size(io);
    if (N > 0 && (!aligned16(q->data, esz, q->strides, 2) || !aligned16(k->data, esz, k->strides, 2)))
        return fail(GDN_ERR_UNSUPPORTED, "q and k rows must be 16-byte aligned (pointer and sequence/head strides)");
    if (g) {
        if ((rc = check_basic(g, "g", 2, msg, false))) return fail(rc, msg);
        if (g->sizes[0] != N || g->sizes[1] != Hv) return fail(GDN_ERR_INVALID_ARGUMENT, "g must be [N, Hv]");
        if (g->dtype != GDN_F32 && g->dtype != GDN_BF16 && g->dtype != GDN_F16)
            return fail(GDN_ERR_INVALID_ARGUMENT, "g must be f32, bf16 or f16");
    }
    if (beta) {
        if ((rc = check_basic(beta, "beta", 2, msg, false))) return fail(rc, msg);
        if (beta->sizes[0] != N || beta->sizes[1] != Hv) return fail(GDN_ERR_INVALID_ARGUMENT, "beta must be [N, Hv]");
        if (beta->dtype != GDN_F32 && beta->dtype != io)
            return fail(GDN_ERR_INVALID_ARGUMENT, "beta must be f32 or q's dtype");
    }
    const gdn_tensor *st[2] = {state_in, state_out};
    const char *st_name[2] = {"state_in", "state_out"};
    for (int i = 0; i < 2; ++i) {
        if (!st[i]) continue;
        if ((rc = check_basic(st[i], st_name[i], 4, msg))) return fail(rc, msg);
        if (st[i]->dtype != GDN_F32 && st[i]->dtype != GDN_BF16)
            return fail(GDN_ERR_INVALID_ARGUMENT, std::string(st_name[i]) + " must be f32 or bf16");
        if ((!state_indices && st[i]->sizes[0] != N) || st[i]->sizes[1] != Hv || st[i]->sizes[2] != gdn::kHeadDim ||
            st[i]->sizes[3] != gdn::kHeadDim)
            return fail(GDN_ERR_INVALID_ARGUMENT, std::string(st_name[i]) + " must be [N, Hv, 128, 128]");
        if (N > 0 && st[i]->sizes[0] > 0 && !aligned16(st[i]->data, dt_size(st[i]->dtype), st[i]->strides, 3))
            return fail(GDN_ERR_UNSUPPORTED, std::string(st_name[i]) + ": rows must be 16-byte aligned (pointer and strides)");
    }
    if (state_in && state_out && state_in->data == state_out->data && N > 0) {
        bool same = state_in->dtype == state_out->dtype;
        for (int i = 0; i < 4; ++i) same = same && state_in->strides[i] == state_out->strides[i];
        if (!same)
            return fail(GDN_ERR_ALIAS, "state_out may share state_in's buffer only as the identical view (in-place update)");
    }
    if (state_indices) {
        if ((rc = check_basic(state_indices, "state_indices", 1, msg))) return fail(rc, msg);
        if (state_indices->dtype != GDN_I32 && state_indices->dtype != GDN_I64)
            return fail(GDN_ERR_INVALID_ARGUMENT, "state_indices must be i32 or i64");
        if (state_indices->sizes[0] != N || (N > 0 && state_indices->data == nullptr))
            return fail(GDN_ERR_INVALID_ARGUMENT, "state_indices must hold N entries");
    }
    if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_ARGUMENT, "scale must be finite");
    int dev = 0, cus = 256;
    if ((rc = check_device(msg, &dev, &cus))) return fail(rc, msg);
    if (N == 0) return GDN_OK;

    gdn::DecodeParams p{};
    if (state_indices) {
        p.sidx = state_indices->data;
        p.sidx_i64 = state_indices->dtype == GDN_I64;
        p.pool_rows = state_in->sizes[0];
    }
    const int64_t es = (int64_t)esz;
    p.q = static_cast<const char *>(q->data); p.q_sn = q->strides[0] * es; p.q_sh = q->strides[1] * es;
    p.k = static_cast<const char *>(k->data); p.k_sn = k->strides[0] * es; p.k_sh = k->strides[1] * es;
    p.v = static_cast<const char *>(v->data); p.v_sn = v->strides[0] * es; p.v_sh = v->strides[1] * es;
    p.io_dt = io;
    if (g) {
        const int64_t ge = (int64_t)dt_size(g->dtype);
        p.g = static_cast<const char *>(g->data); p.g_sn = g->strides[0] * ge; p.g_sh = g->strides[1] * ge;
        p.g_dt = g->dtype;
    }
    if (beta) {
        const int64_t be = (int64_t)dt_size(beta->dtype);
        p.beta = static_cast<const char *>(beta->data); p.b_sn = beta->strides[0] * be; p.b_sh = beta->strides[1] * be;
        p.b_dt = beta->dtype;
    }
    if (state_in) {
        const int64_t se = (int64_t)dt_size(state_in->dtype);
        p.s_in = static_cast<const char *>(state_in->data);
        p.si_n = state_in->strides[0] * se; p.si_h = state_in->strides[1] * se; p.si_v = state_in->strides[2] * se;
        p.si_dt = state_in->dtype;
    }
    if (state_out) {
        const int64_t se = (int64_t)dt_size(state_out->dtype);
        p.s_out = static_cast<char *>(state_out->data);
        p.so_n = state_out->strides[0] * se; p.so_h = state_out->strides[1] * se; p.so_v = state_out->strides[2] * se;
        p.so_dt = state_out->dtype;
    }
    p.out = static_cast<char *>(out->data); p.o_sn = out->strides[0] * es; p.o_sh = out->strides[1] * es;
    p.scale = scale == 0.0f ? 1.0f / std::sqrt((float)gdn::kHeadDim) : scale;
    p.l2norm = use_qk_l2norm != 0;
    p.N = (int32_t)N; p.Hv = (int32_t)Hv; p.r = (int32_t)(Hv / Hqk);
    const hipError_t e = gdn::launch_decode(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
    return GDN_OK;
}

}  // namespace

extern "C" int gdn_decode_step(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v,
                               const gdn_tensor *g, const gdn_tensor *beta, float scale,
                               const gdn_tensor *state_in, const gdn_tensor *state_out, int use_qk_l2norm,
                               const gdn_tensor *out, void *stream) {
    return decode_impl(q, k, v, g, beta, scale, state_in, state_out, nullptr, use_qk_l2norm, out, stream);
}

extern "C" int gdn_decode_step_pooled(const gdn_tensor *q, const gdn_tensor *k, const gdn_tensor *v,
                                      const gdn_tensor *g, const gdn_tensor *beta, float scale,
                                      const gdn_tensor *state_pool, const gdn_tensor *state_indices,
                                      int use_qk_l2norm, const gdn_tensor *out, void *stream) {
    if (!state_pool || !state_indices) {
        g_last_error = "state_pool and state_indices are required";
        return GDN_ERR_INVALID_ARGUMENT;
    }
    return decode_impl(q, k, v, g, beta, scale, state_pool, state_pool, state_indices, use_qk_l2norm, out, stream);
}

extern "C" int gdn_prefill_plan(int64_t num_seqs, int64_t num_tokens, int64_t num_v_heads, int io_dtype,
                                int checkpoints, int batch_invariant, int num_cus, int *kind,
                                int64_t *segment_length) {
    if (!kind || !segment_length) {
        g_last_error = "kind and segment_length are required";
        return GDN_ERR_INVALID_ARGUMENT;
    }
    if (num_seqs < 0 || num_tokens < 0 || num_v_heads < 1 || num_cus < 1 ||
        (io_dtype != GDN_F32 && io_dtype != GDN_BF16)) {
        g_last_error = "invalid sizes or dtype";
        return GDN_ERR_INVALID_ARGUMENT;
    }
    // the size limits gdn_chunk_prefill applies (a plan only for a call it would accept)
    if (num_tokens > ((int64_t)1 << 40) || num_v_heads > 65536 || num_seqs > ((int64_t)1 << 24) ||
        (num_seqs + 8) * num_v_heads > ((int64_t)1 << 30)) {
        g_last_error = "problem too large";
        return GDN_ERR_UNSUPPORTED;
    }
    const Plan plan = make_plan(num_seqs, num_tokens, num_v_heads, io_dtype == GDN_BF16, checkpoints != 0,
                                batch_invariant != 0, num_cus);
    *kind = plan.kind;
    *segment_length = plan.lseg;
    return GDN_OK;
}
