"""CPU oracle for the gated delta rule prefill scan.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  Nothing here is imported by, or
imports, the HIP library; the two share no code.

``run`` wraps the C token-by-token recurrence (``gdn_oracle.c``, fp64 by
default, fp32 on request).  ``chunked`` holds a second, independent CPU form
(the chunked UT/WY algebra in numpy fp64) used to pin the chunk algebra.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIBS = {}


def _lib(mutant: int = 0):
    if mutant not in _LIBS:
        path = _build.lib_path(mutant)
        if not os.path.exists(path):
            _build.build(mutant)
        lib = ctypes.CDLL(path)
        for sfx, cty in (("f64", ctypes.c_double), ("f32", ctypes.c_float)):
            fn = getattr(lib, "gdn_oracle_run_" + sfx)
            P = ctypes.POINTER(cty)
            fn.argtypes = [P, P, P, P, P, ctypes.c_double, ctypes.POINTER(ctypes.c_int64),
                           ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                           ctypes.c_int64, P, ctypes.c_int, P, P, ctypes.c_int]
            fn.restype = ctypes.c_int
        _LIBS[mutant] = lib
    return _LIBS[mutant]


def _arr(x, dt):
    if x is None:
        return None
    if hasattr(x, "detach"):                    # torch tensor: exact upcast via fp64
        import torch
        x = x.detach().cpu().to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(dt, copy=False))


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return os.cpu_count() or 1


def run(q, k, v, g=None, beta=None, scale=0.0, cu_seqlens=None, initial_state=None,
        use_qk_l2norm=False, precision="f64", nthreads=None, mutant=0):
    """Token-by-token recurrence over a packed varlen batch.

    q, k: [T, Hqk, K]; v: [T, Hv, V]; g, beta: [T, Hv] or None (ones);
    cu_seqlens: [N+1]; initial_state: [N, Hv, V, K] or None (zeros).
    Inputs may be numpy arrays or CPU torch tensors of any float dtype; they
    are upcast exactly.  Returns (out [T, Hv, V], final_state [N, Hv, V, K])
    as numpy arrays of the requested precision.
    """
    dt = np.float64 if precision == "f64" else np.float32
    cty = ctypes.c_double if precision == "f64" else ctypes.c_float
    q, k, v = _arr(q, dt), _arr(k, dt), _arr(v, dt)
    g, beta, s0 = _arr(g, dt), _arr(beta, dt), _arr(initial_state, dt)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens),
                              dtype=np.int64)
    T, Hqk, K = q.shape
    Hv, V = v.shape[1], v.shape[2]
    N = cu.shape[0] - 1
    assert k.shape == q.shape and v.shape[0] == T and int(cu[-1]) == T
    out = np.zeros((T, Hv, V), dtype=dt)
    fin = np.zeros((N, Hv, V, K), dtype=dt)
    P = ctypes.POINTER(cty)

    def ptr(a):
        return None if a is None else a.ctypes.data_as(P)

    fn = getattr(_lib(mutant), "gdn_oracle_run_" + precision)
    rc = fn(ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), float(scale),
            cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), N, Hqk, Hv, K, V,
            ptr(s0), int(bool(use_qk_l2norm)), ptr(out), ptr(fin),
            int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle: bad arguments")
    return out, fin
