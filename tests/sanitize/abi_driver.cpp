// Driver for the sanitizer build of the host layer (tests/test_sanitizers.py):
// the argument validation of every entry point and the host planner, run on a
// machine without a GPU.  Descriptors carry fake, never-dereferenced device
// pointers; a call that passes validation stops at the device check
// (GDN_ERR_NO_DEVICE).  Exit status 0 when every call returns the expected
// code; sanitizer reports are the test's real subject.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <limits>

#include "gdn.h"

namespace {

const uintptr_t kFake = 0x7f0000000000ull;
int failures = 0;

gdn_tensor tensor(std::initializer_list<int64_t> sizes, int dt, uintptr_t ptr = kFake) {
    gdn_tensor t;
    std::memset(&t, 0, sizeof(t));
    t.data = reinterpret_cast<void *>(ptr);
    t.dtype = dt;
    t.ndim = (int32_t)sizes.size();
    int i = 0;
    for (int64_t s : sizes) t.sizes[i++] = s;
    int64_t acc = 1;
    for (int d = t.ndim - 1; d >= 0; --d) {
        t.strides[d] = acc;
        acc *= t.sizes[d];
    }
    return t;
}

void expect(const char *what, int got, int want) {
    if (got != want) {
        std::printf("FAIL %s: got %d want %d (%s)\n", what, got, want, gdn_last_error());
        ++failures;
    } else if (got != GDN_OK && std::strlen(gdn_last_error()) == 0) {
        std::printf("FAIL %s: no message\n", what);
        ++failures;
    }
}

struct Args {
    gdn_tensor q, k, v, g, beta, cu, s0, s1, out;
    float scale = 0.f;
    Args(int64_t T = 100, int64_t N = 2, int64_t Hqk = 2, int64_t Hv = 4, int dt = GDN_BF16)
        : q(tensor({T, Hqk, 128}, dt)), k(tensor({T, Hqk, 128}, dt)), v(tensor({T, Hv, 128}, dt)),
          g(tensor({T, Hv}, GDN_F32)), beta(tensor({T, Hv}, GDN_F32)), cu(tensor({N + 1}, GDN_I32)),
          s0(tensor({N, Hv, 128, 128}, GDN_F32, kFake + (1ull << 30))),
          s1(tensor({N, Hv, 128, 128}, GDN_F32, kFake + (1ull << 31))),
          out(tensor({T, Hv, 128}, dt, kFake + (1ull << 32))) {}
    int call(bool noalloc = false) const {
        auto f = noalloc ? gdn_chunk_prefill_noalloc : gdn_chunk_prefill;
        return f(&q, &k, &v, &g, &beta, scale, &cu, &s0, &s1, 1, 1, &out, nullptr);
    }
};

}  // namespace

int main() {
    // ---- prefill validation
    {
        Args a;
        expect("valid call, no device", a.call(), GDN_ERR_NO_DEVICE);
        expect("valid call (no allocation), no device", a.call(true), GDN_ERR_NO_DEVICE);
    }
    {
        Args a;
        expect("missing q", gdn_chunk_prefill(nullptr, &a.k, &a.v, &a.g, &a.beta, 0.f, &a.cu, &a.s0, &a.s1, 1, 1,
                                              &a.out, nullptr), GDN_ERR_INVALID_ARGUMENT);
    }
    { Args a; a.q.ndim = 2; expect("q ndim", a.call(), GDN_ERR_INVALID_ARGUMENT); }
    { Args a; a.q.ndim = 7; expect("q ndim beyond 4", a.call(), GDN_ERR_INVALID_ARGUMENT); }
    { Args a; a.q.sizes[2] = a.k.sizes[2] = 64; expect("head dim", a.call(), GDN_ERR_UNSUPPORTED); }
    { Args a; a.v.sizes[1] = a.out.sizes[1] = 3; expect("head ratio", a.call(), GDN_ERR_UNSUPPORTED); }
    { Args a; a.k.dtype = GDN_F32; expect("k dtype", a.call(), GDN_ERR_INVALID_ARGUMENT); }
    { Args a; a.q.dtype = a.k.dtype = a.v.dtype = a.out.dtype = GDN_F16; expect("f16", a.call(), GDN_ERR_UNSUPPORTED); }
    { Args a; a.q.dtype = 99; expect("bad dtype code", a.call(), GDN_ERR_INVALID_ARGUMENT); }
    { Args a; a.v.strides[0] = -512; expect("negative stride", a.call(), GDN_ERR_INVALID_ARGUMENT); }
    { Args a; a.v.data = reinterpret_cast<void *>(kFake + 8); expect("misaligned v", a.call(), GDN_ERR_UNSUPPORTED); }
    { Args a; a.out.strides[1] = 64; expect("out heads overlap", a.call(), GDN_ERR_UNSUPPORTED); }
    { Args a; a.out.strides[0] = 0; expect("out tokens alias", a.call(), GDN_ERR_UNSUPPORTED); }
    { Args a; a.s1 = a.s0; expect("state alias", a.call(), GDN_ERR_ALIAS); }
    { Args a; a.s1.strides[1] = 128 * 64; expect("output_state overlap", a.call(), GDN_ERR_UNSUPPORTED); }
    { Args a; a.cu.strides[0] = 2; a.cu.sizes[0] = 3; expect("cu strided", a.call(), GDN_ERR_INVALID_ARGUMENT); }
    { Args a; a.cu.sizes[0] = 0; expect("cu empty", a.call(), GDN_ERR_INVALID_ARGUMENT); }
    { Args a; a.scale = std::numeric_limits<float>::quiet_NaN(); expect("scale NaN", a.call(), GDN_ERR_INVALID_ARGUMENT); }
    { Args a; a.scale = std::numeric_limits<float>::infinity(); expect("scale inf", a.call(), GDN_ERR_INVALID_ARGUMENT); }
    { Args a; a.q.strides[0] = 1ll << 40; a.k.strides[0] = 1ll << 40; expect("huge token stride", a.call(), GDN_ERR_UNSUPPORTED); }
    {   // a problem beyond the size limits
        Args a((int64_t)1 << 41, 1, 1, 1);
        expect("too many tokens", a.call(), GDN_ERR_UNSUPPORTED);
    }
    {   // the largest sizes still accepted reach the device check
        Args a(0, (int64_t)1 << 20, 16, 32);
        a.s0.data = a.s1.data = nullptr;
        expect("empty batch, many sequences", gdn_chunk_prefill(&a.q, &a.k, &a.v, &a.g, &a.beta, 0.f, &a.cu, nullptr,
                                                                nullptr, 1, 0, &a.out, nullptr), GDN_ERR_NO_DEVICE);
    }
    // ---- checkpointed and pooled forms
    {
        Args a;
        gdn_tensor ck = tensor({2 * 3, 4, 128, 128}, GDN_F32, kFake + (1ull << 33));
        expect("checkpointed valid", gdn_chunk_prefill_checkpointed(&a.q, &a.k, &a.v, &a.g, &a.beta, 0.f, &a.cu, &a.s0,
                                                                    &a.s1, 1, 1, &ck, 3, 128, &a.out, nullptr),
               GDN_ERR_NO_DEVICE);
        expect("checkpoint interval", gdn_chunk_prefill_checkpointed(&a.q, &a.k, &a.v, &a.g, &a.beta, 0.f, &a.cu,
                                                                     &a.s0, &a.s1, 1, 1, &ck, 3, 100, &a.out, nullptr),
               GDN_ERR_UNSUPPORTED);
        expect("checkpoints missing", gdn_chunk_prefill_checkpointed(&a.q, &a.k, &a.v, &a.g, &a.beta, 0.f, &a.cu,
                                                                     &a.s0, &a.s1, 1, 1, nullptr, 3, 128, &a.out,
                                                                     nullptr), GDN_ERR_INVALID_ARGUMENT);
        gdn_tensor pool = tensor({9, 4, 128, 128}, GDN_BF16, kFake + (1ull << 34));
        gdn_tensor idx = tensor({2}, GDN_I64, kFake + (1ull << 35));
        expect("pooled valid", gdn_chunk_prefill_pooled(&a.q, &a.k, &a.v, &a.g, &a.beta, 0.f, &a.cu, &pool, &idx, 1,
                                                        0, &a.out, nullptr), GDN_ERR_NO_DEVICE);
        idx.sizes[0] = 3;
        expect("pool index count", gdn_chunk_prefill_pooled(&a.q, &a.k, &a.v, &a.g, &a.beta, 0.f, &a.cu, &pool, &idx,
                                                            1, 0, &a.out, nullptr), GDN_ERR_INVALID_ARGUMENT);
    }
    // ---- decode step
    {
        gdn_tensor q = tensor({3, 2, 128}, GDN_BF16), k = tensor({3, 2, 128}, GDN_BF16);
        gdn_tensor v = tensor({3, 4, 128}, GDN_BF16), out = tensor({3, 4, 128}, GDN_BF16, kFake + (1ull << 32));
        gdn_tensor s = tensor({3, 4, 128, 128}, GDN_F32, kFake + (1ull << 30));
        expect("decode valid", gdn_decode_step(&q, &k, &v, nullptr, nullptr, 0.f, &s, &s, 1, &out, nullptr),
               GDN_ERR_NO_DEVICE);
        gdn_tensor s2 = s;
        s2.dtype = GDN_BF16;
        expect("decode alias", gdn_decode_step(&q, &k, &v, nullptr, nullptr, 0.f, &s, &s2, 1, &out, nullptr),
               GDN_ERR_ALIAS);
        gdn_tensor idx = tensor({3}, GDN_I32, kFake + (1ull << 35));
        expect("decode pooled valid", gdn_decode_step_pooled(&q, &k, &v, nullptr, nullptr, 0.f, &s, &idx, 1, &out,
                                                             nullptr), GDN_ERR_NO_DEVICE);
    }
    // ---- the planner over a grid of sizes, extremes included
    const int64_t counts[] = {0, 1, 2, 7, 32, 256, 1 << 24, (1 << 24) + 1, INT64_MAX};
    const int64_t tokens[] = {0, 1, 63, 4096, 65536, 1ll << 40, (1ll << 40) + 1, 1ll << 62, INT64_MAX};
    const int64_t heads[] = {0, 1, 4, 32, 65536, 65537, INT64_MAX};
    const int cus[] = {1, 80, 256, 1 << 20};
    long plans = 0;
    for (int64_t N : counts)
        for (int64_t T : tokens)
            for (int64_t Hv : heads)
                for (int cu : cus)
                    for (int dt : {GDN_F32, GDN_BF16})
                        for (int bi = 0; bi < 2; ++bi) {
                            int kind = -1;
                            int64_t seg = -1;
                            const int rc = gdn_prefill_plan(N, T, Hv, dt, 0, bi, cu, &kind, &seg);
                            if (rc == GDN_OK) {
                                ++plans;
                                if (kind < 0 || kind > 3 || seg < 0 || (kind != GDN_PLAN_SPLIT && seg != 0) ||
                                    (kind == GDN_PLAN_SPLIT && (seg % 64 != 0 || bi))) {
                                    std::printf("FAIL plan N=%lld T=%lld Hv=%lld: kind %d seg %lld\n", (long long)N,
                                                (long long)T, (long long)Hv, kind, (long long)seg);
                                    ++failures;
                                }
                            } else if (rc != GDN_ERR_INVALID_ARGUMENT && rc != GDN_ERR_UNSUPPORTED) {
                                ++failures;
                            }
                        }
    expect("plan without outputs", gdn_prefill_plan(1, 64, 4, GDN_BF16, 0, 0, 256, nullptr, nullptr),
           GDN_ERR_INVALID_ARGUMENT);
    gdn_release_workspace();
    std::printf("host layer driver: %s (%ld valid plans)\n", failures ? "FAILED" : "ok", plans);
    return failures ? 1 : 0;
}
