"""C-ABI checks that need no GPU: the library loads, exports every function
include/gdn.h declares, and rejects bad arguments before touching a device
(descriptors carry fake, never-dereferenced pointers)."""
import ctypes
import math
import os
import re

import pytest

import chunked_gated_delta_prefill_amd as lib
from chunked_gated_delta_prefill_amd import (GDN_BF16, GDN_F16, GDN_F32, GDN_I32, GDN_I64,
                                             make_tensor)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7f0000000000          # 16-byte aligned, never dereferenced
OK, INVALID, UNSUPPORTED, ALIAS, NO_DEVICE, ARCH, HIPERR = range(7)


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "gdn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_\w+)\s*\(", text)))


def test_exports_every_declared_function():
    names = _declared_functions()
    assert names == ["gdn_chunk_prefill", "gdn_chunk_prefill_checkpointed", "gdn_chunk_prefill_noalloc",
                     "gdn_chunk_prefill_pooled",
                     "gdn_decode_step", "gdn_decode_step_pooled", "gdn_last_error", "gdn_prefill_plan",
                     "gdn_release_workspace"]
    L = lib.load()
    for n in names:
        assert hasattr(L, n), n


def _contig(sizes):
    st, acc = [], 1
    for s in reversed(sizes):
        st.append(acc)
        acc *= s
    return list(reversed(st))


def _t(sizes, dt=GDN_BF16, ptr=FAKE, strides=None):
    return make_tensor(ptr, dt, sizes, strides or _contig(sizes))


def _args(T=100, N=2, Hqk=2, Hv=4, dt=GDN_BF16, **over):
    a = dict(q=_t([T, Hqk, 128], dt), k=_t([T, Hqk, 128], dt), v=_t([T, Hv, 128], dt),
             g=_t([T, Hv], GDN_F32), beta=_t([T, Hv], GDN_F32), scale=0.0,
             cu=_t([N + 1], GDN_I32), s0=_t([N, Hv, 128, 128], GDN_F32, FAKE + (1 << 30)),
             s1=_t([N, Hv, 128, 128], GDN_F32, FAKE + (1 << 31)), l2=1, bi=1,
             out=_t([T, Hv, 128], dt, FAKE + (1 << 32)))
    a.update(over)
    return a


def _call(a):
    return lib.call_raw(a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["cu"], a["s0"],
                        a["s1"], a["l2"], a["bi"], a["out"], None)


CASES = {
    "q_missing": (dict(q=None), INVALID),
    "out_missing": (dict(out=None), INVALID),
    "cu_missing": (dict(cu=None), INVALID),
    "q_ndim": (dict(q=_t([100, 256], GDN_BF16)), INVALID),
    "head_dim_64": (dict(q=_t([100, 2, 64]), k=_t([100, 2, 64])), UNSUPPORTED),
    "head_ratio": (dict(v=_t([100, 3, 128]), out=_t([100, 3, 128]), g=_t([100, 3], GDN_F32),
                        beta=_t([100, 3], GDN_F32), s0=None, s1=None), UNSUPPORTED),
    "f16_inputs": (dict(q=_t([100, 2, 128], GDN_F16), k=_t([100, 2, 128], GDN_F16),
                        v=_t([100, 4, 128], GDN_F16), out=_t([100, 4, 128], GDN_F16)), UNSUPPORTED),
    "k_dtype": (dict(k=_t([100, 2, 128], GDN_F32)), INVALID),
    "k_shape": (dict(k=_t([99, 2, 128])), INVALID),
    "inner_stride": (dict(q=_t([100, 2, 128], strides=[512, 256, 2])), INVALID),
    "negative_stride": (dict(v=_t([100, 4, 128], strides=[-512, 128, 1])), INVALID),
    "alias": (dict(s1=_t([2, 4, 128, 128], GDN_F32, FAKE + (1 << 30))), ALIAS),
    "g_shape": (dict(g=_t([100, 2], GDN_F32)), INVALID),
    "g_dtype": (dict(g=_t([100, 4], GDN_I32)), INVALID),
    "beta_dtype": (dict(beta=_t([100, 4], GDN_F16)), INVALID),
    "cu_dtype": (dict(cu=_t([3], GDN_F32)), INVALID),
    "cu_strided": (dict(cu=_t([3], GDN_I64, strides=[2])), INVALID),
    "state_shape": (dict(s0=_t([3, 4, 128, 128], GDN_F32)), INVALID),
    "state_dtype": (dict(s1=_t([2, 4, 128, 128], GDN_F16, FAKE + (1 << 31))), INVALID),
    "scale_nan": (dict(scale=math.nan), INVALID),
    "misaligned_q": (dict(q=_t([100, 2, 128], ptr=FAKE + 2)), UNSUPPORTED),
    "misaligned_stride": (dict(q=_t([100, 2, 128], strides=[260, 130, 1]),
                               k=_t([100, 2, 128], strides=[260, 130, 1])), UNSUPPORTED),
    "null_data": (dict(v=_t([100, 4, 128], ptr=None)), INVALID),
    "out_dtype": (dict(out=_t([100, 4, 128], GDN_F32)), INVALID),
    "bad_dtype_code": (dict(g=_t([100, 4], 17)), INVALID),
    # v and out move in 16-byte pieces: pointer and token/head byte strides must be multiples of 16
    "misaligned_v": (dict(v=_t([100, 4, 128], ptr=FAKE + 8)), UNSUPPORTED),
    "misaligned_v_stride": (dict(v=_t([100, 4, 128], strides=[516, 129, 1])), UNSUPPORTED),
    "misaligned_out": (dict(out=_t([100, 4, 128], ptr=FAKE + (1 << 32) + 2)), UNSUPPORTED),
    "misaligned_out_stride": (dict(out=_t([100, 4, 128], GDN_BF16, FAKE + (1 << 32), strides=[520, 130, 1])), UNSUPPORTED),
    # out must not overlap itself: heads 64 elements apart, or heads of one token running into the next
    "out_head_stride_below_128": (dict(out=_t([100, 4, 128], GDN_BF16, FAKE + (1 << 32), strides=[512, 64, 1])), UNSUPPORTED),
    "out_tokens_overlap_heads": (dict(out=_t([100, 4, 128], GDN_BF16, FAKE + (1 << 32), strides=[128, 128, 1])), UNSUPPORTED),
    "out_broadcast_heads": (dict(out=_t([100, 4, 128], GDN_BF16, FAKE + (1 << 32), strides=[128, 0, 1])), UNSUPPORTED),
    "output_state_overlap": (dict(s1=_t([2, 4, 128, 128], GDN_F32, FAKE + (1 << 31),
                                         strides=[4 * 16384, 128 * 64, 128, 1])), UNSUPPORTED),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_rejected_before_any_device_access(name):
    over, code = CASES[name]
    rc, msg = _call(_args(**over))
    assert rc == code, (rc, msg)
    assert msg, "a failed call must leave a message"


def test_interleaved_out_layouts_validate():
    """Non-overlapping out layouts other than the contiguous one pass validation
    (token-major with padding, head-major): no device exists, so the call stops
    at the device check."""
    if _has_gpu():
        pytest.skip("a valid descriptor with fake pointers must not reach a real GPU")
    for st in ([1024, 128, 1], [128, 100 * 128, 1]):
        rc, msg = _call(_args(out=_t([100, 4, 128], GDN_BF16, FAKE + (1 << 32), strides=st)))
        assert rc == NO_DEVICE, (st, rc, msg)


def test_fp32_inputs_and_bf16_state_validate():
    a = _args(dt=GDN_F32, beta=_t([100, 4], GDN_F32), s0=_t([2, 4, 128, 128], GDN_BF16, FAKE + (1 << 30)))
    if _has_gpu():
        pytest.skip("a valid descriptor with fake pointers must not reach a real GPU")
    rc, msg = _call(a)
    assert rc == NO_DEVICE, (rc, msg)


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def test_valid_call_without_gpu_reports_no_device():
    if _has_gpu():
        pytest.skip("a valid descriptor with fake pointers must not reach a real GPU")
    rc, msg = _call(_args())
    assert rc == NO_DEVICE and "device" in msg


def test_optional_arguments_may_be_null():
    if _has_gpu():
        pytest.skip("a valid descriptor with fake pointers must not reach a real GPU")
    rc, _ = _call(_args(g=None, beta=None, s0=None, s1=None))
    assert rc == NO_DEVICE


def test_release_workspace_without_gpu():
    lib.load().gdn_release_workspace()


# ---- gdn_decode_step (one token per sequence: q, k [N, Hqk, 128], v, out [N, Hv, 128])

def _dargs(N=3, Hqk=2, Hv=4, dt=GDN_BF16, **over):
    a = dict(q=_t([N, Hqk, 128], dt), k=_t([N, Hqk, 128], dt), v=_t([N, Hv, 128], dt),
             g=_t([N, Hv], GDN_F32), beta=_t([N, Hv], GDN_F32), scale=0.0,
             s0=_t([N, Hv, 128, 128], GDN_F32, FAKE + (1 << 30)),
             s1=_t([N, Hv, 128, 128], GDN_F32, FAKE + (1 << 31)), l2=1,
             out=_t([N, Hv, 128], dt, FAKE + (1 << 32)))
    a.update(over)
    return a


def _dcall(a):
    return lib.call_decode_raw(a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["s0"], a["s1"],
                               a["l2"], a["out"], None)


DECODE_CASES = {
    "q_missing": (dict(q=None), INVALID),
    "out_missing": (dict(out=None), INVALID),
    "head_dim_64": (dict(q=_t([3, 2, 64]), k=_t([3, 2, 64])), UNSUPPORTED),
    "head_ratio": (dict(v=_t([3, 3, 128]), out=_t([3, 3, 128]), g=None, beta=None, s0=None, s1=None),
                   UNSUPPORTED),
    "f16_inputs": (dict(q=_t([3, 2, 128], GDN_F16), k=_t([3, 2, 128], GDN_F16), v=_t([3, 4, 128], GDN_F16),
                        out=_t([3, 4, 128], GDN_F16)), UNSUPPORTED),
    "v_batch": (dict(v=_t([4, 4, 128])), INVALID),
    "g_shape": (dict(g=_t([3, 2], GDN_F32)), INVALID),
    "beta_dtype": (dict(beta=_t([3, 4], GDN_F16)), INVALID),
    "state_shape": (dict(s0=_t([3, 4, 128, 64], GDN_F32)), INVALID),
    "state_dtype": (dict(s1=_t([3, 4, 128, 128], GDN_I32, FAKE + (1 << 31))), INVALID),
    "alias_other_dtype": (dict(s1=_t([3, 4, 128, 128], GDN_BF16, FAKE + (1 << 30))), ALIAS),
    "alias_other_strides": (dict(s1=_t([3, 4, 128, 128], GDN_F32, FAKE + (1 << 30),
                                       strides=[4 * 128 * 256, 128 * 256, 256, 1])), ALIAS),
    "misaligned_state": (dict(s0=_t([3, 4, 128, 128], GDN_F32, FAKE + 4)), UNSUPPORTED),
    "scale_inf": (dict(scale=math.inf), INVALID),
}


@pytest.mark.parametrize("name", sorted(DECODE_CASES))
def test_decode_rejected_before_any_device_access(name):
    over, code = DECODE_CASES[name]
    rc, msg = _dcall(_dargs(**over))
    assert rc == code, (rc, msg)
    assert msg


def test_decode_in_place_view_is_accepted():
    if _has_gpu():
        pytest.skip("a valid descriptor with fake pointers must not reach a real GPU")
    a = _dargs(s1=_t([3, 4, 128, 128], GDN_F32, FAKE + (1 << 30)))
    rc, msg = _dcall(a)
    assert rc == NO_DEVICE, (rc, msg)
    rc, _ = _dcall(_dargs(g=None, beta=None, s0=None, s1=None))
    assert rc == NO_DEVICE


# ---- gdn_chunk_prefill_checkpointed (N = 2 sequences, P = 3 slots each)

def _ccall(ck=None, per_seq=3, interval=128, **over):
    a = _args(**over)
    if ck is None:
        ck = _t([6, 4, 128, 128], GDN_F32, FAKE + (1 << 33))
    return lib.call_checkpointed_raw(a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["cu"], a["s0"],
                                     a["s1"], a["l2"], a["bi"], ck, per_seq, interval, a["out"], None)


CKPT_CASES = {
    "interval_not_chunk_multiple": (dict(interval=100), UNSUPPORTED),
    "interval_zero": (dict(interval=0), UNSUPPORTED),
    "per_seq_zero": (dict(per_seq=0, ck=_t([0, 4, 128, 128], GDN_F32, FAKE + (1 << 33))), INVALID),
    "slots_mismatch": (dict(ck=_t([5, 4, 128, 128], GDN_F32, FAKE + (1 << 33))), INVALID),
    "dtype": (dict(ck=_t([6, 4, 128, 128], GDN_F16, FAKE + (1 << 33))), INVALID),
    "aliases_output_state": (dict(ck=_t([6, 4, 128, 128], GDN_F32, FAKE + (1 << 31))), ALIAS),
    "misaligned": (dict(ck=_t([6, 4, 128, 128], GDN_F32, FAKE + (1 << 33) + 8)), UNSUPPORTED),
}


@pytest.mark.parametrize("name", sorted(CKPT_CASES))
def test_checkpointed_rejected_before_any_device_access(name):
    rc, msg = _ccall(**CKPT_CASES[name][0])
    assert rc == CKPT_CASES[name][1], (rc, msg)
    assert msg


def test_checkpointed_requires_checkpoints():
    a = _args()
    rc, msg = lib.call_checkpointed_raw(a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["cu"], a["s0"],
                                        a["s1"], a["l2"], a["bi"], None, 1, 64, a["out"], None)
    assert rc == INVALID and msg


def test_checkpointed_valid_call_without_gpu():
    if _has_gpu():
        pytest.skip("a valid descriptor with fake pointers must not reach a real GPU")
    rc, msg = _ccall()
    assert rc == NO_DEVICE, (rc, msg)


# ---- gdn_chunk_prefill_pooled (N = 2 sequences, a pool of 5 rows)

def _pcall(pool="default", idx="default", **over):
    a = _args(**over)
    pool = _t([5, 4, 128, 128], GDN_F32, FAKE + (1 << 30)) if pool == "default" else pool
    idx = _t([2], GDN_I32, FAKE + (1 << 34)) if idx == "default" else idx
    return lib.call_pooled_raw(a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["cu"], pool, idx,
                               a["l2"], a["bi"], a["out"], None)


POOL_CASES = {
    "pool_missing": (dict(pool=None), INVALID),
    "indices_missing": (dict(idx=None), INVALID),
    "indices_dtype": (dict(idx=_t([2], GDN_F32, FAKE + (1 << 34))), INVALID),
    "indices_count": (dict(idx=_t([3], GDN_I64, FAKE + (1 << 34))), INVALID),
    "pool_heads": (dict(pool=_t([5, 2, 128, 128], GDN_F32, FAKE + (1 << 30))), INVALID),
    "pool_dtype": (dict(pool=_t([5, 4, 128, 128], GDN_F16, FAKE + (1 << 30))), INVALID),
}


@pytest.mark.parametrize("name", sorted(POOL_CASES))
def test_pooled_rejected_before_any_device_access(name):
    rc, msg = _pcall(**POOL_CASES[name][0])
    assert rc == POOL_CASES[name][1], (rc, msg)
    assert msg


def test_pooled_valid_call_without_gpu():
    if _has_gpu():
        pytest.skip("a valid descriptor with fake pointers must not reach a real GPU")
    rc, msg = _pcall()
    assert rc == NO_DEVICE, (rc, msg)


def test_decode_pooled_argument_checks():
    a = _dargs()
    pool = _t([7, 4, 128, 128], GDN_F32, FAKE + (1 << 30))
    bad = [(None, _t([3], GDN_I32, FAKE + (1 << 34)), INVALID),
           (pool, None, INVALID),
           (pool, _t([2], GDN_I32, FAKE + (1 << 34)), INVALID),
           (pool, _t([3], GDN_F32, FAKE + (1 << 34)), INVALID),
           (_t([7, 2, 128, 128], GDN_F32, FAKE + (1 << 30)), _t([3], GDN_I64, FAKE + (1 << 34)), INVALID)]
    for pl, ix, code in bad:
        rc, msg = lib.call_decode_pooled_raw(a["q"], a["k"], a["v"], a["g"], a["beta"], 0.0, pl, ix, 1, a["out"], None)
        assert rc == code and msg, (rc, msg)
    if not _has_gpu():
        rc, msg = lib.call_decode_pooled_raw(a["q"], a["k"], a["v"], a["g"], a["beta"], 0.0, pool,
                                             _t([3], GDN_I32, FAKE + (1 << 34)), 1, a["out"], None)
        assert rc == NO_DEVICE, (rc, msg)


def test_launch_size_limits():
    """(sequence, value head) counts whose grid would not fit one launch are refused."""
    N, Hv = 1 << 24, 128
    a = _args(T=N, N=N, Hqk=1, Hv=Hv, g=None, beta=None, s0=None, s1=None,
              q=_t([N, 1, 128]), k=_t([N, 1, 128]), v=_t([N, Hv, 128]), out=_t([N, Hv, 128], ptr=FAKE + (1 << 40)))
    rc, msg = _call(a)
    assert rc == UNSUPPORTED and "launch" in msg, (rc, msg)
    d = _dargs(N=N, Hqk=1, Hv=Hv, g=None, beta=None, s0=None, s1=None, q=_t([N, 1, 128]), k=_t([N, 1, 128]),
               v=_t([N, Hv, 128]), out=_t([N, Hv, 128], ptr=FAKE + (1 << 40)))
    rc, msg = _dcall(d)
    assert rc == UNSUPPORTED and "launch" in msg, (rc, msg)
