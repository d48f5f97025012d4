"""MI355X (gfx950) chunked gated delta rule prefill: Python binding.

Argument marshalling only: every step of the scan runs in the HIP library
``libgdn.so`` (built from ``csrc/`` by ``build.py``) behind the C ABI in
``include/gdn.h``.  There is no other implementation here and no fallback: if
the library is missing or refuses a call, an exception is raised.

The entry points mirror the C functions::

    gdn_chunk_prefill(q, k, v, g, beta, scale, cu_seqlens, initial_state,
                      output_state, use_qk_l2norm, batch_invariant, out,
                      stream=None)
    gdn_chunk_prefill_noalloc(q, k, v, g, beta, scale, cu_seqlens, initial_state,
                              output_state, use_qk_l2norm, batch_invariant, out,
                              stream=None)
    gdn_chunk_prefill_checkpointed(q, k, v, g, beta, scale, cu_seqlens,
                                   initial_state, output_state, use_qk_l2norm,
                                   batch_invariant, checkpoints,
                                   checkpoints_per_sequence, checkpoint_interval,
                                   out, stream=None)
    gdn_chunk_prefill_pooled(q, k, v, g, beta, scale, cu_seqlens, state_pool,
                             state_indices, use_qk_l2norm, batch_invariant, out,
                             stream=None)
    gdn_decode_step(q, k, v, g, beta, scale, state_in, state_out,
                    use_qk_l2norm, out, stream=None)
    gdn_decode_step_pooled(q, k, v, g, beta, scale, state_pool, state_indices,
                           use_qk_l2norm, out, stream=None)

All tensors are torch CUDA (HIP) tensors; ``out`` and ``output_state`` are
written in place.  See include/gdn.h for shapes, dtypes and error codes.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")

GDN_F32, GDN_BF16, GDN_F16, GDN_I32, GDN_I64 = 0, 1, 2, 3, 4
STATUS = {0: "GDN_OK", 1: "GDN_ERR_INVALID_ARGUMENT", 2: "GDN_ERR_UNSUPPORTED", 3: "GDN_ERR_ALIAS",
          4: "GDN_ERR_NO_DEVICE", 5: "GDN_ERR_ARCH", 6: "GDN_ERR_HIP"}


class GdnTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("sizes", ctypes.c_int64 * 4), ("strides", ctypes.c_int64 * 4)]


class GdnError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code


_lib = None


def load():
    """Loads libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(or python -m chunked_gated_delta_prefill_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(GdnTensor)
        lib.gdn_chunk_prefill.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, P, ctypes.c_int,
                                          ctypes.c_int, P, ctypes.c_void_p]
        lib.gdn_chunk_prefill.restype = ctypes.c_int
        lib.gdn_chunk_prefill_noalloc.argtypes = lib.gdn_chunk_prefill.argtypes
        lib.gdn_chunk_prefill_noalloc.restype = ctypes.c_int
        lib.gdn_chunk_prefill_checkpointed.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, P, ctypes.c_int,
                                                       ctypes.c_int, P, ctypes.c_int32, ctypes.c_int64, P,
                                                       ctypes.c_void_p]
        lib.gdn_chunk_prefill_checkpointed.restype = ctypes.c_int
        lib.gdn_chunk_prefill_pooled.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, P, ctypes.c_int, ctypes.c_int,
                                                 P, ctypes.c_void_p]
        lib.gdn_chunk_prefill_pooled.restype = ctypes.c_int
        lib.gdn_decode_step.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, ctypes.c_int, P, ctypes.c_void_p]
        lib.gdn_decode_step.restype = ctypes.c_int
        lib.gdn_decode_step_pooled.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, ctypes.c_int, P,
                                               ctypes.c_void_p]
        lib.gdn_decode_step_pooled.restype = ctypes.c_int
        lib.gdn_last_error.argtypes = []
        lib.gdn_last_error.restype = ctypes.c_char_p
        lib.gdn_release_workspace.argtypes = []
        lib.gdn_release_workspace.restype = None
        lib.gdn_prefill_plan.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                         ctypes.POINTER(ctypes.c_int64)]
        lib.gdn_prefill_plan.restype = ctypes.c_int
        _lib = lib
    return _lib


def make_tensor(data_ptr, dtype_code, sizes, strides):
    """A gdn_tensor descriptor from raw values (used by tests with fake pointers)."""
    t = GdnTensor()
    t.data = data_ptr
    t.dtype = dtype_code
    t.ndim = len(sizes)
    for i, (s, st) in enumerate(zip(sizes, strides)):
        t.sizes[i] = s
        t.strides[i] = st
    return t


def _dtype_code(dt):
    import torch
    return {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16, torch.float16: GDN_F16,
            torch.int32: GDN_I32, torch.int64: GDN_I64}.get(dt, -1)


def describe(t):
    """gdn_tensor descriptor of a torch tensor (None stays None)."""
    if t is None:
        return None
    return make_tensor(t.data_ptr(), _dtype_code(t.dtype), list(t.shape), list(t.stride()))


def call_raw(q, k, v, g, beta, scale, cu_seqlens, initial_state, output_state, use_qk_l2norm,
             batch_invariant, out, stream):
    """Calls the C function on descriptors; returns the status code and message."""
    lib = load()
    ref = lambda d: None if d is None else ctypes.byref(d)
    rc = lib.gdn_chunk_prefill(ref(q), ref(k), ref(v), ref(g), ref(beta), ctypes.c_float(scale),
                               ref(cu_seqlens), ref(initial_state), ref(output_state),
                               int(bool(use_qk_l2norm)), int(bool(batch_invariant)), ref(out), stream)
    return rc, (lib.gdn_last_error() or b"").decode()


def _stream_handle(stream, q):
    if stream is None:
        import torch
        return torch.cuda.current_stream(q.device).cuda_stream if q.is_cuda else None
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return stream


def gdn_chunk_prefill(q, k, v, g, beta, scale, cu_seqlens, initial_state, output_state,
                      use_qk_l2norm, batch_invariant, out, stream=None):
    """Enqueues the scan on ``stream`` (default: torch's current stream of q's device)."""
    stream = _stream_handle(stream, q)
    rc, msg = call_raw(describe(q), describe(k), describe(v), describe(g), describe(beta),
                       0.0 if scale is None else float(scale), describe(cu_seqlens),
                       describe(initial_state), describe(output_state), use_qk_l2norm,
                       batch_invariant, describe(out), stream)
    if rc != 0:
        raise GdnError(rc, msg)


def gdn_chunk_prefill_noalloc(q, k, v, g, beta, scale, cu_seqlens, initial_state, output_state,
                              use_qk_l2norm, batch_invariant, out, stream=None):
    """gdn_chunk_prefill without any device allocation (the split path's workspace
    is the library's fixed scratch array)."""
    stream = _stream_handle(stream, q)
    lib = load()
    ref = lambda d: None if d is None else ctypes.byref(d)
    rc = lib.gdn_chunk_prefill_noalloc(ref(describe(q)), ref(describe(k)), ref(describe(v)), ref(describe(g)),
                                       ref(describe(beta)), ctypes.c_float(0.0 if scale is None else float(scale)),
                                       ref(describe(cu_seqlens)), ref(describe(initial_state)),
                                       ref(describe(output_state)), int(bool(use_qk_l2norm)),
                                       int(bool(batch_invariant)), ref(describe(out)), stream)
    if rc != 0:
        raise GdnError(rc, (lib.gdn_last_error() or b"").decode())


def call_checkpointed_raw(q, k, v, g, beta, scale, cu_seqlens, initial_state, output_state, use_qk_l2norm,
                          batch_invariant, checkpoints, per_seq, interval, out, stream):
    """Calls gdn_chunk_prefill_checkpointed on descriptors; returns the status code and message."""
    lib = load()
    ref = lambda d: None if d is None else ctypes.byref(d)
    rc = lib.gdn_chunk_prefill_checkpointed(ref(q), ref(k), ref(v), ref(g), ref(beta), ctypes.c_float(scale),
                                            ref(cu_seqlens), ref(initial_state), ref(output_state),
                                            int(bool(use_qk_l2norm)), int(bool(batch_invariant)), ref(checkpoints),
                                            int(per_seq), int(interval), ref(out), stream)
    return rc, (lib.gdn_last_error() or b"").decode()


def gdn_chunk_prefill_checkpointed(q, k, v, g, beta, scale, cu_seqlens, initial_state, output_state,
                                   use_qk_l2norm, batch_invariant, checkpoints, checkpoints_per_sequence,
                                   checkpoint_interval, out, stream=None):
    """The scan, also writing the state every ``checkpoint_interval`` tokens of each sequence into
    ``checkpoints`` ([N * checkpoints_per_sequence, Hv, 128, 128])."""
    stream = _stream_handle(stream, q)
    rc, msg = call_checkpointed_raw(describe(q), describe(k), describe(v), describe(g), describe(beta),
                                    0.0 if scale is None else float(scale), describe(cu_seqlens),
                                    describe(initial_state), describe(output_state), use_qk_l2norm,
                                    batch_invariant, describe(checkpoints), checkpoints_per_sequence,
                                    checkpoint_interval, describe(out), stream)
    if rc != 0:
        raise GdnError(rc, msg)


def call_pooled_raw(q, k, v, g, beta, scale, cu_seqlens, state_pool, state_indices, use_qk_l2norm, batch_invariant,
                    out, stream):
    """Calls gdn_chunk_prefill_pooled on descriptors; returns the status code and message."""
    lib = load()
    ref = lambda d: None if d is None else ctypes.byref(d)
    rc = lib.gdn_chunk_prefill_pooled(ref(q), ref(k), ref(v), ref(g), ref(beta), ctypes.c_float(scale),
                                      ref(cu_seqlens), ref(state_pool), ref(state_indices), int(bool(use_qk_l2norm)),
                                      int(bool(batch_invariant)), ref(out), stream)
    return rc, (lib.gdn_last_error() or b"").decode()


def gdn_chunk_prefill_pooled(q, k, v, g, beta, scale, cu_seqlens, state_pool, state_indices, use_qk_l2norm,
                             batch_invariant, out, stream=None):
    """The scan on an indexed state pool: sequence n reads and rewrites ``state_pool[state_indices[n]]``."""
    stream = _stream_handle(stream, q)
    rc, msg = call_pooled_raw(describe(q), describe(k), describe(v), describe(g), describe(beta),
                              0.0 if scale is None else float(scale), describe(cu_seqlens), describe(state_pool),
                              describe(state_indices), use_qk_l2norm, batch_invariant, describe(out), stream)
    if rc != 0:
        raise GdnError(rc, msg)


def call_decode_raw(q, k, v, g, beta, scale, state_in, state_out, use_qk_l2norm, out, stream):
    """Calls gdn_decode_step on descriptors; returns the status code and message."""
    lib = load()
    ref = lambda d: None if d is None else ctypes.byref(d)
    rc = lib.gdn_decode_step(ref(q), ref(k), ref(v), ref(g), ref(beta), ctypes.c_float(scale), ref(state_in),
                             ref(state_out), int(bool(use_qk_l2norm)), ref(out), stream)
    return rc, (lib.gdn_last_error() or b"").decode()


def gdn_decode_step(q, k, v, g, beta, scale, state_in, state_out, use_qk_l2norm, out, stream=None):
    """Enqueues one decode step on ``stream``; ``state_out`` may be ``state_in`` (in place)."""
    stream = _stream_handle(stream, q)
    rc, msg = call_decode_raw(describe(q), describe(k), describe(v), describe(g), describe(beta),
                              0.0 if scale is None else float(scale), describe(state_in), describe(state_out),
                              use_qk_l2norm, describe(out), stream)
    if rc != 0:
        raise GdnError(rc, msg)


def call_decode_pooled_raw(q, k, v, g, beta, scale, state_pool, state_indices, use_qk_l2norm, out, stream):
    """Calls gdn_decode_step_pooled on descriptors; returns the status code and message."""
    lib = load()
    ref = lambda d: None if d is None else ctypes.byref(d)
    rc = lib.gdn_decode_step_pooled(ref(q), ref(k), ref(v), ref(g), ref(beta), ctypes.c_float(scale),
                                    ref(state_pool), ref(state_indices), int(bool(use_qk_l2norm)), ref(out), stream)
    return rc, (lib.gdn_last_error() or b"").decode()


def gdn_decode_step_pooled(q, k, v, g, beta, scale, state_pool, state_indices, use_qk_l2norm, out, stream=None):
    """One decode step on an indexed pool: sequence n reads and rewrites ``state_pool[state_indices[n]]``."""
    stream = _stream_handle(stream, q)
    rc, msg = call_decode_pooled_raw(describe(q), describe(k), describe(v), describe(g), describe(beta),
                                     0.0 if scale is None else float(scale), describe(state_pool),
                                     describe(state_indices), use_qk_l2norm, describe(out), stream)
    if rc != 0:
        raise GdnError(rc, msg)


PLAN_NAMES = {0: "scan", 1: "pipelined_scan", 2: "split", 3: "prepared_scan"}


def prefill_plan(num_seqs, num_tokens, num_v_heads, io_dtype, checkpoints, batch_invariant, num_cus):
    """gdn_prefill_plan: (plan name, segment length) of a prefill call with these
    sizes on a device with num_cus CUs (host only, no device needed)."""
    lib = load()
    kind, seg = ctypes.c_int(-1), ctypes.c_int64(-1)
    rc = lib.gdn_prefill_plan(int(num_seqs), int(num_tokens), int(num_v_heads), _dtype_code(io_dtype),
                              int(bool(checkpoints)), int(bool(batch_invariant)), int(num_cus), ctypes.byref(kind),
                              ctypes.byref(seg))
    if rc != 0:
        raise RuntimeError(f"gdn_prefill_plan failed ({rc}): {(lib.gdn_last_error() or b'').decode()}")
    return PLAN_NAMES[kind.value], seg.value


def release_workspace():
    load().gdn_release_workspace()
