"""Host-side pieces of bench.py (no GPU): the kernel names it reports (from
the library's host plan) and the one-GPU guard."""
import os
import subprocess
import sys

import torch

from types import SimpleNamespace

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _shape(lengths, Hv, dtype=torch.bfloat16):
    """What the plan reads: N, T, Hv and the q dtype (no data generated)."""
    return SimpleNamespace(N=len(lengths), T=sum(lengths), Hv=Hv, q=torch.empty(0, dtype=dtype))


# sequence lengths of the five workloads (the varlen and many-short ones only
# need their count and total here)
SHAPES = {
    "tiny_fp32": _shape([37, 91], 2, torch.float32),
    "varlen_bf16": _shape([1904] * 7 + [1902], 32),
    "long_single": _shape([65536], 32),
    "many_short": _shape([126] * 256, 32),
    "large_batch": _shape([8192] * 32, 32),
}


PREPARED = "prepared: plan_kernel, fused_scan_kernel (preparation), prepared_scan_kernel"


def test_scan_kernel_labels_of_the_five_workloads():
    cus = 256
    expect = {   # (batch_invariant 0, batch_invariant 1)
        "tiny_fp32": ("fused_scan_kernel", "fused_scan_kernel"),        # fp32 q/k/v
        "varlen_bf16": ("piped_scan_kernel", "piped_scan_kernel"),      # 256 work items = CUs
        "many_short": ("fused_scan_kernel", "fused_scan_kernel"),       # 8192 work items
        "large_batch": ("fused_scan_kernel", "fused_scan_kernel"),      # 1024 work items
    }
    for name, (k0, k1) in expect.items():
        w = SHAPES[name]
        assert bench.scan_kernels(w, 0, cus) == k0, name
        assert bench.scan_kernels(w, 1, cus) == k1, name
    w = SHAPES["long_single"]
    assert bench.scan_kernels(w, 0, cus).startswith("split")           # one sequence on 32 heads
    assert bench.scan_kernels(w, 1, cus) == PREPARED
    assert bench.scan_kernels(w, 1, cus, checkpoints=True) == "fused_scan_kernel"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_max_norm_err_on_host_tensors():
    """bench.max_norm_err: max |got - ref| / max |ref| over the whole tensor."""
    import numpy as np
    ref = np.array([[1.0, -4.0], [2.0, 0.5]])
    got = torch.tensor([[1.0, -3.9], [2.2, 0.5]])
    assert abs(bench.max_norm_err(got, ref) - 0.2 / 4.0) < 1e-6
    assert bench.max_norm_err(got[:0], ref[:0]) == 0.0
