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


def _fake_rocpd(path, trace=None, counters=None):
    """A database with the two rocpd views bench.py reads: kernels (name,
    start, end in ns) and counters_collection (dispatch_id, kernel_name,
    counter_name, value)."""
    import sqlite3
    os.makedirs(os.path.dirname(path), exist_ok=True)
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, start integer, end integer)")
    con.execute("create table counters_collection (dispatch_id integer, kernel_name text, counter_name text, "
                "value real)")
    for row in trace or []:
        con.execute("insert into kernels values (?, ?, ?)", row)
    for row in counters or []:
        con.execute("insert into counters_collection values (?, ?, ?, ?)", row)
    con.commit()
    con.close()


def test_plan_summary_groups_dispatches_into_calls(tmp_path):
    """bench.summarize_plan: gdn dispatches are grouped into calls of the plan's
    kernel sequence (other kernels ignored), durations averaged per position,
    traffic scaled by the copy's counters, per-wave counts derived."""
    seq = bench.PLAN_SEQUENCE["split"]
    names = ["_ZN3gdn12_GLOBAL__N_111plan_kernelEv", "_ZN3gdn12_GLOBAL__N_117fused_scan_kernelILi1E",
             "_ZN3gdn12_GLOBAL__N_117fused_scan_kernelILi2E", "gdn::anon::fixup_kernel",
             "_ZN3gdn12_GLOBAL__N_117fused_scan_kernelILi0E"]
    base = tmp_path / "case"
    trace, t = [], 0
    for call in range(3):
        trace.append(("at::native::copy_kernel", t, t + 999))   # not a gdn kernel
        for i, n in enumerate(names):
            trace.append((n, t, t + 1000 * (i + 1) + call))      # position i lasts ~(i + 1) us
            t += 10000
    _fake_rocpd(str(base / "trace" / "a.db"), trace=trace)
    disp = [(len(names) * call + i, n) for call in range(3) for i, n in enumerate(names)]   # launch order
    for sub, cnt in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        _fake_rocpd(str(base / sub / "a.db"), counters=[(d, n, cnt, 2.0) for d, n in disp])
    _fake_rocpd(str(base / "sq1" / "a.db"),
                counters=[(d, n, c, v) for d, n in disp for c, v in (("SQ_WAVES", 4.0), ("SQ_INSTS_VALU", 400.0))])
    _fake_rocpd(str(base / "sq2" / "a.db"),
                counters=[(d, n, c, v) for d, n in disp
                          for c, v in (("SQ_LDS_BANK_CONFLICT", 1.0), ("SQ_ACTIVE_INST_LDS", 4.0))])
    _fake_rocpd(str(tmp_path / "copy_fetch" / "a.db"), counters=[(1, "copyBuffer", "FETCH_SIZE", 524288.0)])
    _fake_rocpd(str(tmp_path / "copy_write" / "a.db"), counters=[(1, "copyBuffer", "WRITE_SIZE", 1048576.0)])
    w = SimpleNamespace(name="long_single", N=1, T=65536, Hqk=16, Hv=32, q=torch.empty(0, dtype=torch.bfloat16))
    out = tmp_path / "summary.txt"
    bench.summarize_plan(str(base), str(out), w, 0, "split", {"trace": "cmd"}, 1000.0, 2)
    kv, block = {}, "head"
    for line in out.read_text().splitlines():
        if line.startswith("["):
            block = line.strip("[]")
        elif "=" in line and not line.startswith("#"):
            a, b = line.split("=", 1)
            kv[(block, a.strip())] = b.strip()
    assert [b for b in dict.fromkeys(k[0] for k in kv) if b != "head"] == seq
    # the last 2 calls: position i lasts (i + 1) us + call index (1, 2) ns
    for i, name in enumerate(seq):
        assert abs(float(kv[(name, "average_us")]) - (i + 1 + 0.0015)) < 1e-3
        assert float(kv[(name, "fetch_bytes")]) == 2.0 * 1024 * 2.0   # 2 KiB, fetch scale 2
        assert float(kv[(name, "write_bytes")]) == 2.0 * 1024 * 1.0
        assert float(kv[(name, "valu_per_wave")]) == 100.0
        assert float(kv[(name, "lds_conflict_ratio")]) == 0.25
    # the call spans 4 gaps of 10 us and the last kernel (5 us + call index ns); the kernels alone sum to 15 us
    assert abs(float(kv[("head", "call_average_us")]) - (45 + 0.0015)) < 1e-3
    assert abs(float(kv[("head", "kernel_time_us")]) - (15 + 5 * 0.0015)) < 1e-3
    assert float(kv[("head", "hbm_bytes_per_call")]) == 5 * 3 * 2048.0
    # a run whose dispatches do not follow the plan's sequence is refused
    import pytest
    with pytest.raises(ValueError):
        bench.summarize_plan(str(base), str(out), w, 0, "prepared_scan", {}, 1000.0, 2)


def _kv(path):
    kv, block = {}, "head"
    for line in open(path).read().splitlines():
        if line.startswith("["):
            block = line.strip("[]")
        elif "=" in line and not line.startswith("#"):
            a, b = line.split("=", 1)
            kv[(block, a.strip())] = b.strip()
    return kv


def test_plan_summary_of_overlapping_ranges(tmp_path):
    """A prepared call in four chunk ranges: the preparation of ranges 1-3
    overlaps the scan of range 0 (started in either order), so a kernel's
    figures sum its dispatches and the call time is the span of the call."""
    plan_k, prep_k, scan_k = ("gdn::plan_kernel", "_ZN3gdn12_GLOBAL__N_117fused_scan_kernelILi3E",
                              "_ZN3gdn12_GLOBAL__N_120prepared_scan_kernelILi1EEEv")
    # (name, start us, duration us) within a call; prep 1 starts before scan 0
    call = [(plan_k, 0, 1), (prep_k, 2, 10), (prep_k, 12.5, 10), (scan_k, 13, 20), (prep_k, 23, 10),
            (prep_k, 33.5, 10), (scan_k, 34, 20), (scan_k, 55, 20), (scan_k, 76, 20)]
    enq = [0, 1, 2, 4, 5, 3, 6, 7, 8]   # dispatch (enqueue) order: the side stream's preparations first
    base = tmp_path / "case"
    trace, disp = [], []
    for c in range(3):
        t0 = 1000.0 * c
        trace += [(n, int((t0 + s0) * 1000), int((t0 + s0 + d) * 1000)) for n, s0, d in call]
        disp += [(9 * c + i, call[j][0]) for i, j in enumerate(enq)]
    _fake_rocpd(str(base / "trace" / "a.db"), trace=trace)
    for sub, cnt in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        _fake_rocpd(str(base / sub / "a.db"), counters=[(d, n, cnt, 1.0) for d, n in disp])
    for sub in ("sq1", "sq2"):
        _fake_rocpd(str(base / sub / "a.db"), counters=[(d, n, "SQ_WAVES", 4.0) for d, n in disp])
    _fake_rocpd(str(tmp_path / "copy_fetch" / "a.db"), counters=[(1, "copyBuffer", "FETCH_SIZE", 1048576.0)])
    _fake_rocpd(str(tmp_path / "copy_write" / "a.db"), counters=[(1, "copyBuffer", "WRITE_SIZE", 1048576.0)])
    w = SimpleNamespace(name="long_single", N=1, T=65536, Hqk=16, Hv=32, q=torch.empty(0, dtype=torch.bfloat16))
    out = tmp_path / "summary.txt"
    bench.summarize_plan(str(base), str(out), w, 1, "prepared_scan", {}, 1000.0, 2)
    kv = _kv(out)
    seq = bench.PLAN_SEQUENCE["prepared_scan"]
    for name, n, us in zip(seq, (1, 4, 4), (1.0, 40.0, 80.0)):
        assert int(kv[(name, "dispatches_per_call")]) == n
        assert abs(float(kv[(name, "average_us")]) - us) < 1e-6
        assert float(kv[(name, "fetch_bytes")]) == n * 1024.0
    assert abs(float(kv[("head", "call_average_us")]) - 96.0) < 1e-6
    assert abs(float(kv[("head", "kernel_time_us")]) - 121.0) < 1e-6
    assert float(kv[("head", "hbm_bytes_per_call")]) == 2 * 9 * 1024.0


def test_table_from_bench_lines(tmp_path):
    line = {"config": {"workload": "large_batch", "batch_invariant": False}, "plan": "scan", "kernel_ms": 2.0,
            "value": 1.25e8, "tflops": 520.0, "mfma_frac": 0.208,
            "roofline": {"achieved": 3200.0, "frac": 0.4, "traffic": 7.2e9, "algorithmic_bytes": 6.64e9},
            "max_norm_err": {"out": 7e-3, "state": 4e-3}}
    f = tmp_path / "lines.txt"
    f.write_text("noise\n" + __import__("json").dumps(line) + "\n")
    t = bench.render_table(str(f)).splitlines()
    assert len(t) == 3 and t[2].startswith("| large_batch | 0 | scan | 2.000 | 125.0 M | 520 (20.8%) | 3200 (40.0%)")
    assert "| 1.08 |" in t[2] and "7.0e-03, 4.0e-03" in t[2]
