"""Benchmark of the chunked gated delta rule prefill scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload large_batch]

One step = one gdn_chunk_prefill call over the whole synthetic batch (inputs
already resident in HBM).  The call first repeats untimed for --settle-ms
(300 ms) so the GPU's clocks settle, then runs W warmup calls, then K timed
calls.  Prints one JSON line with the throughput
(tokens/s), the roofline of the dominant kernel and the CPU oracle baseline.

Default workload: 32 sequences x 8192 tokens, Hqk = 16, Hv = 32, d = 128, bf16
q/k/v/out, fp32 gates and state, in-kernel L2 norm, batch_invariant off.

Algorithmic work (chunk length 64, whatever the kernels use internally):
  flop/token  = Hv (6 d^2 + 3 C d) + Hqk (2 C d)           (MFMA work)
  bytes/token = q, k (2 Hqk d 2B) + v, out (2 Hv d 2B) + g, beta (2 Hv 4B)
  bytes/seq   = initial + final state (2 Hv d^2 4B)

Decode step (gdn_decode_step): ``--decode`` times one recurrent step for 256
sequences (Hqk 16, Hv 32, bf16, fp32 state updated in place) and prints its
own JSON line; it reads and writes the whole state once, so its roofline is
HBM: bytes/step = state (2 Hv d^2 4B per sequence) + q, k, v, out, g, beta.

Every configuration: ``--all`` prints one JSON line per workload (the five
recipes of gdn_workloads.py) and batch_invariant mode, each with its host plan,
the fp32 oracle's timing (all host threads, and one item on one thread) and the
timed run's error against it, plus the varlen batch with cold caches (its inputs
fit the 256 MiB last-level cache: ``--cold-cache`` writes 512 MiB before each
timed call and takes the rate from the calls' own events); ``--table FILE``
renders such lines as a markdown table.

Other modes (used to produce the committed rocprofv3 summaries):
  --copy-calibration   a plain device copy of known size (for PMC scaling)
  --summarize-plan DIR OUT  one call's kernels (trace, traffic, SQ counters) from
                       the rocprofv3 output dirs DIR/{trace,fetch,write,sq1,sq2}
  --summarize-pmc DIR  (with --decode) the decode kernel's traffic summary
  --summarize-trace DIR OUT  kernel-trace statistics (rocpd .db) into a text summary
"""
import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
D, C = 128, 64
KERNEL = "fused_scan_kernel"
DECODE_KERNEL = "decode_kernel"
DECODE_SRCS = [os.path.join(ROOT, "chunked_gated_delta_prefill_amd", "csrc", "gdn_decode.hip")]
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_kernel_decode_batch.txt")


def algorithmic(w):
    """(MFMA flops, HBM bytes) the method itself needs for workload w."""
    import torch
    T, N, Hqk, Hv = w.T, w.N, w.Hqk, w.Hv
    io = w.q.element_size()
    esz = lambda t: 0 if t is None else t.element_size()
    flops = T * (Hv * (6 * D * D + 3 * C * D) + Hqk * (2 * C * D))
    byts = T * (2 * Hqk * D * io + 2 * Hv * D * io + Hv * (esz(w.g) + esz(w.beta)))
    s_out = 0 if w.state_dtype is None else torch.empty(0, dtype=w.state_dtype).element_size()
    byts += N * Hv * D * D * (esz(w.initial_state) + s_out)
    return flops, byts


def scan_kernels(w, batch_invariant, cus, checkpoints=False, noalloc=False):
    """Kernels one prefill call launches, from the library's own host plan
    (gdn_prefill_plan, no device needed)."""
    import chunked_gated_delta_prefill_amd as gdn
    kind, _ = gdn.prefill_plan(w.N, w.T, w.Hv, w.q.dtype, checkpoints, batch_invariant, cus)
    if noalloc and kind == "prepared_scan":   # the no-allocation entry point runs the pipelined scan
        kind = "pipelined_scan"
    return {"scan": KERNEL, "pipelined_scan": "piped_scan_kernel",
            "prepared_scan": "prepared: plan_kernel, fused_scan_kernel (preparation), prepared_scan_kernel",
            "split": "split: plan_kernel, fused_scan_kernel (maps N, M), fixup_kernel, fused_scan_kernel"}[kind]


def kernel_source_sha(srcs):
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(path, srcs):
    """HBM bytes per launch measured by rocprofv3 PMC runs, if they were taken
    on the current kernel source; else None."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha(srcs):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, max_seqs):
    """The oracle as it stands (the fp32 token-by-token C recurrence, all host
    cores) timed on the first max_seqs sequences (0: all of them).  Returns the
    baseline record and the oracle's (out, final_state) for that sample."""
    import gdn_workloads as W
    import oracle
    import torch
    take = w.N if max_seqs <= 0 else min(max_seqs, w.N)
    cu = w.cu_seqlens.cpu().to(torch.int64)
    end = int(cu[take])
    sub = W.Workload("sample", w.q[:end].cpu(), w.k[:end].cpu(), w.v[:end].cpu(),
                     None if w.g is None else w.g[:end].cpu(),
                     None if w.beta is None else w.beta[:end].cpu(), cu[:take + 1].clone(),
                     None if w.initial_state is None else w.initial_state[:take].cpu(),
                     w.state_dtype, w.use_qk_l2norm, w.scale)
    threads = oracle.default_threads()
    oracle.run(sub.q[:1], sub.k[:1], sub.v[:1], None, None, 0.0, [0, 1], None, False, precision="f32",
               nthreads=1)   # load the library
    t = time.perf_counter()
    ref = oracle.run(sub.q, sub.k, sub.v, sub.g, sub.beta, sub.scale, sub.cu_seqlens, sub.initial_state,
                     sub.use_qk_l2norm, precision="f32", nthreads=threads)
    dt = time.perf_counter() - t
    part = "all" if take == w.N else f"the first {take} of"
    rec = {"value": round(end / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{part} {w.N} sequences ({end} tokens, all {w.Hv} v-heads), fp32 token-by-token "
                     f"oracle, {dt:.1f} s wall"}
    # one (sequence, v-head) item on one thread: the rate one core gives, as tokens/s
    # of the whole head count (the first non-empty sequence, v-head 0 and its q/k head)
    n0 = next((i for i in range(take) if int(cu[i + 1]) > int(cu[i])), None)
    if n0 is not None:
        b0, e0 = int(cu[n0]), int(cu[n0 + 1])
        one = lambda x: None if x is None else x[b0:e0, :1]
        t = time.perf_counter()
        oracle.run(one(sub.q), one(sub.k), one(sub.v), one(sub.g), one(sub.beta), sub.scale, [0, e0 - b0],
                   None if sub.initial_state is None else sub.initial_state[n0:n0 + 1, :1], sub.use_qk_l2norm,
                   precision="f32", nthreads=1)
        dt1 = time.perf_counter() - t
        rec["per_core"] = {"value": round((e0 - b0) / dt1 / w.Hv, 1), "unit": "tokens/s",
                           "sample": f"sequence {n0} ({e0 - b0} tokens), v-head 0, one thread, {dt1:.2f} s; "
                                     f"divided by the {w.Hv} v-heads"}
    return rec, ref, take, end


def max_norm_err(got, ref):
    """max_i |got_i - ref_i| / max_i |ref_i| over a whole tensor; got on the
    device, ref a host array (compared on the device, in slices)."""
    import numpy as np
    import torch
    if ref.size == 0:
        return 0.0
    flat_g = got.reshape(-1)
    flat_r = np.ascontiguousarray(ref).reshape(-1)
    step = 1 << 27
    num, den = 0.0, 0.0
    for i in range(0, flat_r.size, step):
        r = torch.from_numpy(flat_r[i:i + step]).to(got.device, dtype=torch.float32)
        num = max(num, float((flat_g[i:i + step].float() - r).abs().max()))
        den = max(den, float(r.abs().max()))
    return num / max(den, 1e-12)


def achievable_peaks():
    """Measured in the bench process: a large bf16 GEMM (torch.mm, 8192^3) and a
    1 GiB device-to-device copy (read + write bytes)."""
    import torch
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.mm(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    reps = 10
    for _ in range(reps):
        torch.mm(a, b)
    e1.record()
    torch.cuda.synchronize()
    mm_tflops = 2 * n ** 3 * reps / (e0.elapsed_time(e1) / 1e3) / 1e12
    del a, b
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"bf16_mm_tflops": round(mm_tflops, 1), "copy_gbs": round(copy_gbs, 1)}


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}))


def _db_files(d):
    return sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))


def _pmc_values(d, name_part, counter):
    """Per-dispatch values of `counter` for kernels whose name contains
    name_part, from rocprofv3's rocpd database(s) under d."""
    import sqlite3
    vals = {}
    for f in _db_files(d):
        con = sqlite3.connect(f)
        for disp, kname, cname, v in con.execute(
                "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
            if name_part in kname and cname == counter:
                vals[(f, disp)] = vals.get((f, disp), 0.0) + float(v)
        con.close()
    return list(vals.values())


def _kernel_stats(d):
    """(name, calls, average ns, total ns, percent) rows from rocprofv3 --kernel-trace."""
    import sqlite3
    rows = []
    for f in _db_files(d):
        con = sqlite3.connect(f)
        rows += con.execute("select name, total_calls, average, total_duration, percentage from top_kernels").fetchall()
        con.close()
    return rows


def _dispatch_durations(d, name_part):
    """Per-dispatch durations (microseconds, in launch order) of the kernels
    whose name contains name_part, from the rocpd 'kernels' view."""
    import sqlite3
    out = []
    for f in _db_files(d):
        con = sqlite3.connect(f)
        try:
            cur = con.execute("select * from kernels")
            cols = [c[0] for c in cur.description]
            ni, si, ei = cols.index("name"), cols.index("start"), cols.index("end")
            for row in cur.fetchall():
                if name_part in str(row[ni]):
                    out.append((row[si], (row[ei] - row[si]) / 1e3))
        except (sqlite3.Error, ValueError):
            pass
        con.close()
    return [dur for _, dur in sorted(out)]


def summarize_trace(base, out_path, command, last=0, kernel=KERNEL):
    rows = _kernel_stats(base)
    lines = [f"# rocprofv3 --kernel-trace --stats summary (rocpd top_kernels; durations in microseconds)",
             f"# command: {command}",
             "# kernel | calls | average_us | total_us | percent"]
    for name, calls, avg, tot, pct in rows[:12]:
        short = name.replace("(anonymous namespace)", "anon").replace("void ", "")
        short = short[:short.rfind("(")] if "(" in short else short
        lines.append(f"{short[:100]} | {calls} | {avg:.3f} | {tot:.1f} | {pct:.2f}")
    durs = _dispatch_durations(base, kernel)
    if durs and last > 0:
        tail = durs[-last:]
        lines.append(f"# {kernel}: the last {len(tail)} dispatches (the timed steps, warmup excluded)")
        lines.append(f"timed_dispatches = {len(tail)}")
        lines.append(f"timed_average_us = {statistics.fmean(tail):.3f}")
        lines.append(f"timed_median_us = {statistics.median(tail):.3f}")
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


DECODE_TRAFFIC_TITLE = ("# HBM traffic of decode_kernel, decode_batch workload (256 one-token sequences, Hqk 16, Hv 32, "
                        "fp32 state updated in place)")


def summarize_pmc(base, cmd_fetch, cmd_write, cmd_cf, cmd_cw, launch_alg_bytes, kernel, out_path, srcs, title):
    """Reads four rocprofv3 --pmc output dirs (kernel FETCH_SIZE, WRITE_SIZE;
    copy FETCH_SIZE, WRITE_SIZE) and writes the traffic summary file."""
    kf = _pmc_values(os.path.join(base, "pmc_fetch"), kernel, "FETCH_SIZE")
    kw = _pmc_values(os.path.join(base, "pmc_write"), kernel, "WRITE_SIZE")
    cf = _pmc_values(os.path.join(base, "pmc_copy_fetch"), "copyBuffer", "FETCH_SIZE")
    cw = _pmc_values(os.path.join(base, "pmc_copy_write"), "copyBuffer", "WRITE_SIZE")
    copy_bytes = float(1 << 30)
    # counters are KiB per dispatch; the copy reads and writes copy_bytes once
    f_fac = copy_bytes / (statistics.median(cf) * 1024.0)
    w_fac = copy_bytes / (statistics.median(cw) * 1024.0)
    fetch = statistics.median(kf) * 1024.0 * f_fac
    write = statistics.median(kw) * 1024.0 * w_fac
    lines = [
        title,
        "# rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by the same counter",
        "# read for a plain 1 GiB device-to-device copy (bench.py --copy-calibration).",
        f"# kernel FETCH_SIZE command: {cmd_fetch}",
        f"# kernel WRITE_SIZE command: {cmd_write}",
        f"# copy FETCH_SIZE command:   {cmd_cf}",
        f"# copy WRITE_SIZE command:   {cmd_cw}",
        f"kernel_source_sha = {kernel_source_sha(srcs)}",
        f"dispatches_fetch = {len(kf)}",
        f"dispatches_write = {len(kw)}",
        f"raw_fetch_kib_median = {statistics.median(kf):.1f}",
        f"raw_write_kib_median = {statistics.median(kw):.1f}",
        f"copy_fetch_kib = {statistics.median(cf):.1f}",
        f"copy_write_kib = {statistics.median(cw):.1f}",
        f"fetch_scale = {f_fac:.4f}",
        f"write_scale = {w_fac:.4f}",
        f"fetch_bytes_per_launch = {fetch:.0f}",
        f"write_bytes_per_launch = {write:.0f}",
        f"hbm_bytes_per_launch = {fetch + write:.0f}",
        f"algorithmic_bytes_per_launch = {launch_alg_bytes:.0f}",
        f"traffic_over_algorithmic = {(fetch + write) / launch_alg_bytes:.3f}",
    ]
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


# Kernels one gdn_chunk_prefill call launches, in launch order, per host plan
# (gdn_prefill_plan); the fused scan kernel runs in several modes.
# The kernels of one call of each plan, in launch order.  A call opens with the
# first of them; a kernel named more than once is told apart by its occurrence
# in the call.  The prepared plan of a long launch runs the preparation and the
# scan once per chunk range (the later ranges' preparation on a side stream,
# beside the scan), so each of its labels may cover several dispatches.
PLAN_SEQUENCE = {
    "scan": ["fused_scan_kernel"],
    "pipelined_scan": ["piped_scan_kernel"],
    "prepared_scan": ["plan_kernel", "fused_scan_kernel (preparation)", "prepared_scan_kernel"],
    "split": ["plan_kernel", "fused_scan_kernel (map N)", "fused_scan_kernel (map M)", "fixup_kernel",
              "fused_scan_kernel (segment scan)"],
}
GDN_KERNELS = ("fused_scan_kernel", "piped_scan_kernel", "prepared_scan_kernel", "plan_kernel", "fixup_kernel",
               "decode_kernel")
ALL_SRCS = [os.path.join(ROOT, "chunked_gated_delta_prefill_amd", "csrc", f)
            for f in ("gdn_api.hip", "gdn_scan.hip", "gdn_scan_piped.hip", "gdn_scan_prepared.hip", "gdn_split.hip",
                      "gdn_device.h", "gdn_internal.h")]
SQ_PASSES = (
    "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_INSTS_VMEM SQ_WAVE_CYCLES SQ_BUSY_CYCLES",
    "SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS "
    "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_WAIT_ANY SQ_INSTS_SMEM",
)


def _gdn_base(name):
    for k in GDN_KERNELS:
        if k in str(name):
            return k
    return None


def _group_calls(names, seq):
    """Splits the gdn kernel names of a run (in start or dispatch order) into
    calls of the plan's kernels and labels them: returns (call index, label
    index) of every dispatch.  Every call must hold every label, each the same
    number of times as in the first call."""
    bases = [s.split(" (")[0] for s in seq]
    res, call, occ, counts = [], -1, {}, []
    for i, n in enumerate(names):
        b = _gdn_base(n)
        cands = [j for j, x in enumerate(bases) if x == b]
        if not cands:
            raise ValueError(f"dispatch {i} is {n}, not a kernel of {seq}")
        if b == bases[0] and (call < 0 or occ.get(b, 0) >= bases.count(b)):
            call, occ = call + 1, {}
            counts.append([0] * len(seq))
        if call < 0:
            raise ValueError(f"dispatch {i} is {n}, before the first {bases[0]}")
        k = occ.get(b, 0)
        lab = cands[0] if len(cands) == 1 else (cands[k] if k < len(cands) else None)
        if lab is None:
            raise ValueError(f"dispatch {i}: {n} once too often in a call of {seq}")
        occ[b] = k + 1
        counts[call][lab] += 1
        res.append((call, lab))
    for c, cnt in enumerate(counts):
        if 0 in cnt or cnt != counts[0]:
            raise ValueError(f"call {c} launches {cnt} of {seq}, the first call {counts[0]}")
    return res


def _trace_calls(d, seq):
    """Durations (us) of the gdn dispatches in the trace under d, grouped into
    calls: (per label: its dispatches' summed duration per call, per label:
    dispatches per call, per call: span from the first start to the last
    end, which counts overlapping kernels once)."""
    import sqlite3
    rows = []
    for f in _db_files(d):
        con = sqlite3.connect(f)
        cur = con.execute("select * from kernels")
        cols = [c[0] for c in cur.description]
        ni, si, ei = cols.index("name"), cols.index("start"), cols.index("end")
        rows += [(r[si], r[ei], r[ni]) for r in cur.fetchall() if _gdn_base(r[ni])]
        con.close()
    rows.sort()
    lab = _group_calls([r[2] for r in rows], seq)
    ncalls = lab[-1][0] + 1 if lab else 0
    per = [[0.0] * ncalls for _ in seq]
    cnt = [0] * len(seq)
    lo, hi = [None] * ncalls, [None] * ncalls
    for (s0, e0, _), (c, j) in zip(rows, lab):
        per[j][c] += (e0 - s0) / 1e3
        cnt[j] += c == 0
        lo[c] = s0 if lo[c] is None else min(lo[c], s0)
        hi[c] = e0 if hi[c] is None else max(hi[c], e0)
    return per, cnt, [(b - a) / 1e3 for a, b in zip(lo, hi)]


def _pmc_calls(d, seq):
    """{counter: per-position lists over calls} of the gdn dispatches under d."""
    import sqlite3
    disp = {}
    for f in _db_files(d):
        con = sqlite3.connect(f)
        for did, kname, cname, v in con.execute(
                "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
            if _gdn_base(kname):
                e = disp.setdefault((f, did), [kname, {}])
                e[1][cname] = e[1].get(cname, 0.0) + float(v)
        con.close()
    order = sorted(disp)
    lab = _group_calls([disp[k][0] for k in order], seq)
    ncalls = lab[-1][0] + 1 if lab else 0
    out = {}
    for k, (c, j) in zip(order, lab):
        for cname, v in disp[k][1].items():
            out.setdefault(cname, [[0.0] * ncalls for _ in seq])[j][c] += v
    return out


def summarize_plan(base, out_path, w, bi, plan, commands, alg_bytes, timed_calls):
    """One summary file per (workload, batch_invariant): every kernel the call
    launches with its trace duration, HBM traffic (FETCH_SIZE / WRITE_SIZE
    scaled by a plain copy's counters) and SQ counters.  base holds the
    rocprofv3 output dirs trace, fetch, write, sq1, sq2 and, one level up,
    copy_fetch, copy_write."""
    seq = PLAN_SEQUENCE[plan]
    med = statistics.median
    tr, ndisp, spans = _trace_calls(os.path.join(base, "trace"), seq)
    fe = _pmc_calls(os.path.join(base, "fetch"), seq)["FETCH_SIZE"]
    wr = _pmc_calls(os.path.join(base, "write"), seq)["WRITE_SIZE"]
    sq = {**_pmc_calls(os.path.join(base, "sq1"), seq), **_pmc_calls(os.path.join(base, "sq2"), seq)}
    up = os.path.dirname(base.rstrip("/"))
    cf = _pmc_values(os.path.join(up, "copy_fetch"), "copyBuffer", "FETCH_SIZE")
    cw = _pmc_values(os.path.join(up, "copy_write"), "copyBuffer", "WRITE_SIZE")
    f_fac = float(1 << 30) / (med(cf) * 1024.0)
    w_fac = float(1 << 30) / (med(cw) * 1024.0)
    lines = [f"# Kernels of one gdn_chunk_prefill call: {plan} plan, workload {w.name} ({w.N} sequences, {w.T} "
             f"tokens, Hqk {w.Hqk}, Hv {w.Hv}, {str(w.q.dtype).replace('torch.', '')}), batch_invariant {bi}",
             "# durations: rocprofv3 --kernel-trace, the last timed calls (warmup excluded);",
             "#   a kernel's figures sum its dispatches in the call; call_average_us spans the call from its first",
             "#   kernel's start to its last kernel's end (overlapping kernels counted once);",
             "# traffic: rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (KiB, median over calls), each",
             "#   scaled by the same counter read for a plain 1 GiB device-to-device copy;",
             "# SQ counters: median per call, summed over the device.  Derived: per_wave = INSTS / SQ_WAVES;",
             "#   mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (SQ_BUSY_CYCLES / 32 shader engines);",
             "#   lds_conflict_ratio = SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS"]
    lines += [f"# {k} command: {c}" for k, c in commands.items()]
    lines += [f"kernel_source_sha = {kernel_source_sha(ALL_SRCS)}",
              f"fetch_scale = {f_fac:.4f}", f"write_scale = {w_fac:.4f}"]
    tot_us, tot_bytes = 0.0, 0.0
    for i, name in enumerate(seq):
        durs = tr[i][-timed_calls:]
        fb = med(fe[i]) * 1024.0 * f_fac
        wb = med(wr[i]) * 1024.0 * w_fac
        tot_us += statistics.fmean(durs)
        tot_bytes += fb + wb
        lines += ["", f"[{name}]", f"timed_calls = {len(durs)}", f"dispatches_per_call = {ndisp[i]}",
                  f"average_us = {statistics.fmean(durs):.3f}", f"median_us = {med(durs):.3f}",
                  f"fetch_bytes = {fb:.0f}", f"write_bytes = {wb:.0f}",
                  f"hbm_gbs = {(fb + wb) / (statistics.fmean(durs) * 1e3):.1f}"]
        vals = {c: med(v[i]) for c, v in sq.items() if v[i]}
        lines += [f"{c} = {vals[c]:.0f}" for c in sorted(vals)]
        waves = vals.get("SQ_WAVES", 0.0)
        if waves:
            for c in ("VALU", "MFMA", "LDS", "SALU", "VMEM"):
                if f"SQ_INSTS_{c}" in vals:
                    lines.append(f"{c.lower()}_per_wave = {vals[f'SQ_INSTS_{c}'] / waves:.1f}")
        if vals.get("SQ_BUSY_CYCLES") and "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
            lines.append(f"mfma_busy = {vals['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024 / (vals['SQ_BUSY_CYCLES'] / 32):.3f}")
        if vals.get("SQ_ACTIVE_INST_LDS") and "SQ_LDS_BANK_CONFLICT" in vals:
            lines.append(f"lds_conflict_ratio = {vals['SQ_LDS_BANK_CONFLICT'] / vals['SQ_ACTIVE_INST_LDS']:.3f}")
    call_us = statistics.fmean(spans[-timed_calls:])
    at = next(i for i, x in enumerate(lines) if x.startswith("kernel_source_sha"))
    lines[at:at] = [f"call_average_us = {call_us:.3f}", f"kernel_time_us = {tot_us:.3f}",
                    f"hbm_bytes_per_call = {tot_bytes:.0f}", f"algorithmic_bytes_per_call = {alg_bytes:.0f}",
                    f"traffic_over_algorithmic = {tot_bytes / alg_bytes:.3f}"]
    os.makedirs(os.path.dirname(out_path) or ".", exist_ok=True)
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def plan_profile_path(workload, bi, plan):
    return os.path.join(ROOT, "profiles", f"plan_{plan}_{workload}_bi{int(bi)}.txt")


def read_plan_traffic(path):
    """HBM bytes per call from a per-plan summary taken on the current sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if line.startswith("["):
            break
        if "=" in line and not line.startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha(ALL_SRCS):
        return None
    try:
        return float(kv["hbm_bytes_per_call"])
    except (KeyError, ValueError):
        return None


TABLE_HEAD = ("| Workload | batch_invariant | plan | call (ms) | tokens/s | TFLOP/s (% bf16 peak) | "
              "algorithmic GB/s (% of 8 TB/s) | measured traffic / algorithmic | max_norm_err out, state |\n"
              "|---|---|---|---|---|---|---|---|---|")


def render_table(path):
    """Markdown table of the JSON lines in `path` (bench.py --all output)."""
    rows = [TABLE_HEAD]
    for line in open(path):
        line = line.strip()
        if not line.startswith("{"):
            continue
        r = json.loads(line)
        cfg, rf, e = r["config"], r["roofline"], r.get("max_norm_err") or {}
        tr = rf.get("traffic")
        if tr is None:   # the plan's committed summary, when it was taken on the current sources
            for b in dict.fromkeys((int(cfg["batch_invariant"]), 0)):
                path = plan_profile_path(cfg["workload"], b, r.get("plan", "?"))
                if os.path.exists(path):
                    tr = read_plan_traffic(path)
                    break
        err = (f"{e['out']:.1e}, " + ("-" if e.get("state") is None else f"{e['state']:.1e}")) if e else "-"
        ratio = "-" if tr is None else f"{tr / rf['algorithmic_bytes']:.2f}"
        name = cfg["workload"] + (" (cold caches)" if "cache" in cfg else "")
        rows.append(f"| {name} | {int(cfg['batch_invariant'])} | {r.get('plan', '?')} | "
                    f"{r['kernel_ms']:.3f} | {r['value'] / 1e6:.1f} M | {r['tflops']:.0f} ({100 * r['mfma_frac']:.1f}%) | "
                    f"{rf['achieved']:.0f} ({100 * rf['frac']:.1f}%) | "
                    f"{ratio} | {err} |")
    return "\n".join(rows)


def decode_bytes(w):
    """Algorithmic HBM bytes of one decode step on w: q, k, v, out, gates, and
    the fp32 state read and written once."""
    io = w.q.element_size()
    return w.N * (2 * w.Hqk * D * io + 2 * w.Hv * D * io + w.Hv * 8) + 2 * w.N * w.Hv * D * D * 4


def settle(args, step):
    """A GPU that has idled (input generation, the oracle of the previous
    workload) takes tens of milliseconds of work to reach its steady clocks, so
    the call is repeated for settle_ms of wall time before the W warmup calls
    (measured on the 256-sequence batch after 3 s idle: the first 20 calls ran
    23% slower than the steady state, the 32 x 8192 batch 3.5%)."""
    import torch
    t_end = time.perf_counter() + args.settle_ms / 1e3
    while time.perf_counter() < t_end:
        for _ in range(4):
            step()
        torch.cuda.synchronize()


def bench_decode(args, gdn, W):
    """One decode step per timed step over decode_batch; one JSON line."""
    import torch
    import oracle
    w = W.decode_batch(device="cuda")
    state = w.initial_state.clone()
    out = torch.empty(w.T, w.Hv, D, dtype=w.q.dtype, device="cuda")
    stream = torch.cuda.current_stream()
    byts = decode_bytes(w)

    def step():
        gdn.gdn_decode_step(w.q, w.k, w.v, w.g, w.beta, w.scale, state, state, w.use_qk_l2norm, out, stream)

    settle(args, step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in evs]
    kern_ms = statistics.mean(launch_ms)
    ms_step = wall * 1e3 / args.steps
    achieved = byts / (kern_ms / 1e3) / 1e9
    # reference: a plain 1 GiB device-to-device copy (reads and writes 1 GiB each)
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(5):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) * 5 / (a.elapsed_time(b) / 1e3) / 1e9
    del src, dst
    res = {
        "metric": "GDN decode step tokens/s (one token per sequence), 1 GPU",
        "value": round(w.N / (ms_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "sequences": w.N, "hqk": w.Hqk, "hv": w.Hv, "head_dim": D,
                   "state": "float32", "in_place": True, "l2norm": w.use_qk_l2norm},
        "kernel_ms": round(kern_ms, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": read_traffic(DECODE_TRAFFIC_FILE, DECODE_SRCS), "kernel": DECODE_KERNEL,
                     "algorithmic_bytes": byts, "device_copy_gbs": round(copy_gbs, 1)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        wc = W.decode_batch(device="cpu")
        threads = oracle.default_threads()
        t = time.perf_counter()
        reps = 0
        while time.perf_counter() - t < 2.0:
            oracle.run(wc.q, wc.k, wc.v, wc.g, wc.beta, wc.scale, wc.cu_seqlens, wc.initial_state,
                       wc.use_qk_l2norm, precision="f32", nthreads=threads)
            reps += 1
        dt = (time.perf_counter() - t) / reps
        res["cpu_baseline"] = {"value": round(wc.N / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "sample": f"the whole batch ({wc.N} sequences x {wc.Hv} v-heads), fp32 oracle, "
                                         f"{reps} runs of {dt * 1e3:.0f} ms"}
    print(json.dumps(res), flush=True)


def bench_prefill(args, gdn, w, bi, peaks, cold=False):
    """Times gdn_chunk_prefill on workload w (already on the device) and returns
    the result record with the timed run's output and final state (for
    with_oracle); cold: L2 and last-level cache flushed before every timed call."""
    import torch
    flops, byts = algorithmic(w)

    out = torch.empty(w.T, w.Hv, D, dtype=w.q.dtype, device="cuda")
    fin = None if w.state_dtype is None else torch.empty(w.N, w.Hv, D, D, dtype=w.state_dtype, device="cuda")
    stream = torch.cuda.current_stream()
    ck_every = args.checkpoint_interval
    if ck_every:
        per_seq = max(1, max(w.lengths()) // ck_every)
        ck = torch.empty(w.N * per_seq, w.Hv, D, D, dtype=torch.float32, device="cuda")
        byts += sum(L // ck_every for L in w.lengths()) * w.Hv * D * D * 4   # checkpoint writes

    if args.pooled:
        pool = w.initial_state.clone()
        pidx = torch.arange(w.N - 1, -1, -1, dtype=torch.int32, device="cuda")

    def step():
        if args.pooled:
            gdn.gdn_chunk_prefill_pooled(w.q, w.k, w.v, w.g, w.beta, w.scale, w.cu_seqlens, pool, pidx,
                                         w.use_qk_l2norm, bool(bi), out, stream)
        elif ck_every:
            gdn.gdn_chunk_prefill_checkpointed(w.q, w.k, w.v, w.g, w.beta, w.scale, w.cu_seqlens, w.initial_state,
                                               fin, w.use_qk_l2norm, bool(bi), ck, per_seq,
                                               ck_every, out, stream)
        else:
            fn = gdn.gdn_chunk_prefill_noalloc if args.noalloc else gdn.gdn_chunk_prefill
            fn(w.q, w.k, w.v, w.g, w.beta, w.scale, w.cu_seqlens, w.initial_state, fin, w.use_qk_l2norm,
               bool(bi), out, stream)

    # cold caches: a 512 MiB write (twice the 256 MiB last-level cache) before each
    # timed call, outside its event pair; the rate then comes from the calls' events
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if cold else None
    settle(args, step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # per-launch durations with events on the launch stream (one kernel per call)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(evs):
        if cold:
            flush.fill_(i & 255)
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in evs]
    ms_step = statistics.mean(launch_ms) if cold else wall * 1e3 / args.steps
    del flush
    kern_ms = statistics.mean(launch_ms)
    value = w.T / (ms_step / 1e3)
    achieved = byts / (kern_ms / 1e3) / 1e9
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan, _ = gdn.prefill_plan(w.N, w.T, w.Hv, w.q.dtype, bool(ck_every), bool(bi), cus)
    if args.noalloc and plan == "prepared_scan":
        plan = "pipelined_scan"
    # measured traffic of the whole call, from the plan's committed summary when it
    # was taken on the current sources for this workload (plain entry point only)
    traffic = None
    if args.variant is None and not (ck_every or args.pooled or args.noalloc):
        for b in dict.fromkeys((int(bi), 0)):
            path = plan_profile_path(w.name, b, plan)
            if os.path.exists(path):
                traffic = read_plan_traffic(path)
                break
    res = {
        "metric": "GDN prefill tokens/s and TFLOP/s (% of MI355X bf16 MFMA peak), 1 GPU",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.q.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "sequences": w.N, "tokens": w.T, "hqk": w.Hqk, "hv": w.Hv,
                   "head_dim": D, "state": str(w.initial_state.dtype).replace("torch.", "")
                   if w.initial_state is not None else None, "l2norm": w.use_qk_l2norm,
                   "batch_invariant": bool(bi),
                   **({"checkpoint_interval": ck_every} if ck_every else {}),
                   **({"entry": "gdn_chunk_prefill_noalloc"} if args.noalloc else {}),
                   **({"pooled": True} if args.pooled else {}),
                   **({"cache": "cold (512 MiB write before each call; rate from the calls' events)"}
                      if cold else {})},
        "tflops": round(flops / (ms_step / 1e3) / 1e12, 2),
        "mfma_frac": round(flops / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "kernel_ms": round(kern_ms, 4),
        "kernel_ms_p20_p80": [round(sorted(launch_ms)[int(0.2 * (len(launch_ms) - 1))], 4),
                              round(sorted(launch_ms)[int(0.8 * (len(launch_ms) - 1))], 4)],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": scan_kernels(w, bi, cus, bool(ck_every), args.noalloc),
                     "algorithmic_bytes": byts, "algorithmic_flops": flops},
        "cpu_baseline": None,
        # the realised sequence boundaries of the seeded workload
        "cu_seqlens": [int(x) for x in w.cu_seqlens.cpu().tolist()],
    }
    res["plan"] = plan
    res["achievable"] = {**peaks, "mfma_frac_of_mm": round(flops / (ms_step / 1e3) / 1e12 / peaks["bf16_mm_tflops"], 4),
                         "hbm_frac_of_copy": round(achieved / peaks["copy_gbs"], 4)}
    return res, out, fin


def with_oracle(args, timed, oracle_ref):
    """Adds the oracle baseline (cpu_baseline()'s return value, timed after the
    GPU runs) and each timed run's own error against it to the records of
    bench_prefill; returns the records."""
    rec, (ro, rf), take, end = oracle_ref
    recs = []
    for res, out, fin in timed:
        res["cpu_baseline"] = rec
        # the timed run's own output and final state against the oracle (same sample)
        if args.pooled:   # the pool is updated in place by every step: no fixed reference
            res["max_norm_err"] = None
        else:
            res["max_norm_err"] = {"out": max_norm_err(out[:end], ro),
                                   "state": None if fin is None else max_norm_err(fin[:take], rf),
                                   "reference": "fp32 oracle", "sample": rec["sample"].split(" (")[0]}
        recs.append(res)
    return recs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large_batch")
    ap.add_argument("--variant", default=None)
    ap.add_argument("--batch-invariant", type=int, default=0)
    ap.add_argument("--cpu-sample-seqs", type=int, default=0, help="sequences the oracle runs (0: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-pmc", default=None)
    ap.add_argument("--pmc-commands", default="{}")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("DIR", "OUT"), default=None)
    ap.add_argument("--decode", action="store_true", help="time the decode step instead of the prefill")
    ap.add_argument("--noalloc", action="store_true",
                    help="time gdn_chunk_prefill_noalloc (no workspace: the pipelined scan where the allocating "
                         "entry point prepares chunks)")
    ap.add_argument("--pooled", action="store_true",
                    help="states in an indexed pool (gdn_chunk_prefill_pooled, reversed index order)")
    ap.add_argument("--checkpoint-interval", type=int, default=0,
                    help="tokens between state checkpoints (gdn_chunk_prefill_checkpointed); 0 = plain scan")
    ap.add_argument("--settle-ms", type=int, default=300,
                    help="untimed calls for this long before the warmup calls, so the clocks settle (0: none)")
    ap.add_argument("--cold-cache", action="store_true",
                    help="flush L2 and the last-level cache (512 MiB write) before each timed call")
    ap.add_argument("--all", action="store_true",
                    help="one JSON line per configuration (all five) and batch_invariant mode, and the varlen batch "
                         "with cold caches")
    ap.add_argument("--table", default=None, metavar="FILE",
                    help="markdown table of the JSON lines in FILE (the output of --all)")
    ap.add_argument("--summarize-plan", nargs=2, metavar=("DIR", "OUT"), default=None,
                    help="per-kernel summary of a plan's rocprofv3 runs under DIR (trace, fetch, write, sq1, sq2)")
    ap.add_argument("--cus", type=int, default=256, help="with --summarize-plan: compute units the plan assumed")
    ap.add_argument("--trace-command", default="?")
    ap.add_argument("--trace-kernel", default=KERNEL, help="with --summarize-trace: kernel name to average")
    ap.add_argument("--trace-last", type=int, default=0,
                    help="with --summarize-trace: also average the last N dispatches of the scan kernel")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the scan shards across GPUs by heads and sequences with no communication, "
              "which is not built here", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace[0], args.summarize_trace[1], args.trace_command, args.trace_last,
                        args.trace_kernel)
        return

    import torch

    import chunked_gated_delta_prefill_amd as gdn
    import gdn_workloads as W

    gdn.load()
    if args.decode:
        if args.summarize_pmc:
            cmds = json.loads(args.pmc_commands)
            summarize_pmc(args.summarize_pmc, cmds.get("fetch", "?"), cmds.get("write", "?"),
                          cmds.get("copy_fetch", "?"), cmds.get("copy_write", "?"),
                          decode_bytes(W.decode_batch(device="cpu")), kernel=DECODE_KERNEL,
                          out_path=DECODE_TRAFFIC_FILE, srcs=DECODE_SRCS, title=DECODE_TRAFFIC_TITLE)
            return
        bench_decode(args, gdn, W)
        return
    if args.table:
        print(render_table(args.table))
        return
    if args.summarize_plan:
        import torch
        w = W.make(args.workload, device="cpu", variant=args.variant)
        plan, _ = gdn.prefill_plan(w.N, w.T, w.Hv, w.q.dtype, False, bool(args.batch_invariant), args.cus)
        summarize_plan(args.summarize_plan[0], args.summarize_plan[1], w, args.batch_invariant, plan,
                       json.loads(args.pmc_commands), algorithmic(w)[1], args.trace_last or 20)
        return
    peaks = achievable_peaks()
    # The oracle runs after a workload's GPU runs (the GPU is not left idle
    # between its warmup and the timed calls), once per workload.
    if args.all:
        # one line per configuration and batch_invariant mode
        for name in W.CONFIG_NAMES:
            w = W.make(name, device="cuda", variant=args.variant)
            timed = [bench_prefill(args, gdn, w, bi, peaks) for bi in (0, 1)]
            if name == "varlen_bf16":   # part of its inputs stays in the last-level cache: also cold
                timed.append(bench_prefill(args, gdn, w, 0, peaks, cold=True))
            recs = ([r for r, _, _ in timed] if args.no_cpu_baseline
                    else with_oracle(args, timed, cpu_baseline(w, args.cpu_sample_seqs)))
            for r in recs:
                print(json.dumps(r), flush=True)
            del w, timed
            torch.cuda.empty_cache()
        return
    w = W.make(args.workload, device="cuda", variant=args.variant)
    timed = [bench_prefill(args, gdn, w, args.batch_invariant, peaks, cold=args.cold_cache)]
    res = (timed[0][0] if args.no_cpu_baseline
           else with_oracle(args, timed, cpu_baseline(w, args.cpu_sample_seqs))[0])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
