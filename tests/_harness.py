"""Shared helpers for the parity tests: run a workload on the GPU through the
C ABI, run the oracle on the same values, and compare."""
import sys

import numpy as np
import torch

import gdn_workloads as W
import oracle

BF16_TOL = 2e-2      # max normalised error, bf16 configurations
F32_TOL = 1e-4       # max normalised error, fp32 configurations


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# (label, out error, state error, tolerance) of every oracle comparison in the
# session; printed at the end of the run (tests/conftest.py)
RECORDS = []


def record(label, e_out, e_state, tol):
    RECORDS.append((label, float(e_out), None if e_state is None else float(e_state), tol))


def run_gpu(gdn, w: W.Workload, batch_invariant=True, out=None, output_state=None, stream=None):
    """Runs the HIP scan on device copies of w; returns (out, final_state) on the device."""
    dev = torch.device("cuda", 0)
    wd = w if w.q.is_cuda else w.to(dev)
    if out is None:
        out = torch.empty(wd.T, wd.Hv, 128, dtype=wd.q.dtype, device=dev)
    if output_state is None and wd.state_dtype is not None:
        output_state = torch.empty(wd.N, wd.Hv, 128, 128, dtype=wd.state_dtype, device=dev)
    gdn.gdn_chunk_prefill(wd.q, wd.k, wd.v, wd.g, wd.beta, wd.scale, wd.cu_seqlens, wd.initial_state,
                          output_state, wd.use_qk_l2norm, batch_invariant, out, stream)
    torch.cuda.synchronize()
    return out, output_state


def run_oracle(w: W.Workload, precision="f64"):
    """Oracle on the exact values of w (upcast); returns numpy (out, final_state)."""
    return oracle.run(w.q, w.k, w.v, w.g, w.beta, w.scale, w.cu_seqlens, w.initial_state,
                      w.use_qk_l2norm, precision=precision)


def nerr(gpu, ref):
    """max_i |gpu_i - ref_i| / max_i |ref_i| (0 for empty tensors)."""
    g = gpu.detach().float().cpu().numpy() if hasattr(gpu, "detach") else np.asarray(gpu)
    r = np.asarray(ref)
    if r.size == 0:
        return 0.0
    return float(np.max(np.abs(g.astype(np.float64) - r)) / max(float(np.max(np.abs(r))), 1e-12))


def check(gdn, w, tol, batch_invariant=True, label=""):
    say(f"[gpu] {label or w.name}: T={w.T} N={w.N} Hqk={w.Hqk} Hv={w.Hv} "
        f"dtype={w.q.dtype} batch_invariant={batch_invariant}")
    out, fin = run_gpu(gdn, w, batch_invariant)
    ref_out, ref_fin = run_oracle(w.to("cpu") if w.q.is_cuda else w)
    e_out = nerr(out, ref_out)
    e_fin = nerr(fin, ref_fin) if fin is not None else 0.0
    say(f"      max normalised error: out {e_out:.3e}  state {e_fin:.3e}  (tol {tol:g})")
    record(f"{label or w.name} bi={int(bool(batch_invariant))}", e_out, e_fin if fin is not None else None, tol)
    assert np.isfinite(e_out) and e_out <= tol, f"out error {e_out}"
    assert np.isfinite(e_fin) and e_fin <= tol, f"final state error {e_fin}"
    return out, fin


def nerr_dev(gpu, ref):
    """nerr for large tensors: gpu (a device tensor) against ref (a host fp64
    array), compared on the device in fp64 slices."""
    if ref.size == 0:
        return 0.0
    g = gpu.reshape(-1)
    r = np.ascontiguousarray(ref).reshape(-1)
    step = 1 << 26
    num, den = 0.0, 0.0
    for i in range(0, r.size, step):
        rr = torch.from_numpy(r[i:i + step]).to(g.device)
        num = max(num, float((g[i:i + step].double() - rr).abs().max()))
        den = max(den, float(rr.abs().max()))
    return num / max(den, 1e-12)
