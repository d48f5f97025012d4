"""GPU invariants of the scan through the C ABI: API identities, batch
invariance, determinism, strided views, state chaining and edge cases."""
import numpy as np
import pytest
import torch

import gdn_workloads as W
from _harness import BF16_TOL, F32_TOL, nerr, record, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _w(lengths=(100, 37, 64), Hqk=2, Hv=4, dtype=torch.bfloat16, seed=21, **kw):
    return W.build(list(lengths), Hqk, Hv, dtype, seed=seed, **kw)


def test_api_defaults_are_bitwise(gdn):
    """g = None == all ones; beta = None == all ones; scale 0 == 1/sqrt(128)."""
    w = _w()
    say("[gpu] api defaults")
    o1, f1 = run_gpu(gdn, W.Workload(**{**w.__dict__, "g": None, "beta": None}), True)
    ones = torch.ones_like(w.g)
    o2, f2 = run_gpu(gdn, W.Workload(**{**w.__dict__, "g": ones, "beta": ones.clone()}), True)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    o3, f3 = run_gpu(gdn, W.Workload(**{**w.__dict__, "scale": 1.0 / np.sqrt(128.0)}), True)
    o4, f4 = run_gpu(gdn, w, True)
    assert torch.equal(o3, o4) and torch.equal(f3, f4)


@pytest.mark.parametrize("gate", ["sigmoid", "strong"])
def test_batch_invariance_across_scan_kernels(gdn, gate):
    """Launches with at most half as many work items as CUs run the prepared
    scan, with at most one per CU the eight-wave pipelined scan, larger ones the
    four-wave scan; all must give bitwise the same results, or batch_invariant
    results would depend on the batch size.  A
    batch with more work items than CUs is compared with sequences of it run
    alone and with a sub-batch below the threshold.  "strong" gates put half
    of the sequences on the entry-wise exp path (chunk log-decay below -60)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    Hqk, Hv = 2, 4
    N = cus // Hv + 9
    gen = torch.Generator().manual_seed(61)
    lens = torch.randint(0, 300, (N,), generator=gen).tolist()
    lens[0], lens[5], lens[7] = 0, 64, 1000
    w = W.build(lens, Hqk, Hv, torch.bfloat16, seed=62)
    if gate == "strong":
        t = torch.arange(w.T)
        seq = torch.searchsorted(w.cu_seqlens.to(torch.int64)[1:], t, right=True)
        w = W.Workload(**{**w.__dict__, "g": torch.where((seq % 2 == 1).unsqueeze(1), torch.full_like(w.g, 0.2), w.g)})
    say(f"[gpu] batch invariance across kernels: {N * Hv} work items ({cus} CUs), gate={gate}")
    out, fin = run_gpu(gdn, w, True)
    cu = w.cu_seqlens.tolist()
    for n in (0, 5, 7, 11, N - 1):
        sub = W.slice_item(w, n, range(w.Hv))
        sub = W.Workload(**{**sub.__dict__, "q": w.q[cu[n]:cu[n + 1]], "k": w.k[cu[n]:cu[n + 1]]})
        o1, f1 = run_gpu(gdn, sub, True)
        assert torch.equal(o1, out[cu[n]:cu[n + 1]]), n
        assert torch.equal(f1[0], fin[n]), n
    m = cus // Hv - 3   # a leading sub-batch below the threshold
    head = W.Workload(**{**w.__dict__, "q": w.q[:cu[m]], "k": w.k[:cu[m]], "v": w.v[:cu[m]], "g": w.g[:cu[m]],
                         "beta": w.beta[:cu[m]], "cu_seqlens": w.cu_seqlens[:m + 1],
                         "initial_state": w.initial_state[:m]})
    o2, f2 = run_gpu(gdn, head, True)
    assert torch.equal(o2, out[:cu[m]])
    assert torch.equal(f2, fin[:m])
    ro, rf = run_oracle(head)
    assert nerr(o2, ro) <= BF16_TOL and nerr(f2, rf) <= BF16_TOL
    # sub-batches that take the prepared scan with 2 and 4 CUs per head
    for m in (cus // (2 * Hv), cus // (4 * Hv)):
        head = W.Workload(**{**w.__dict__, "q": w.q[:cu[m]], "k": w.k[:cu[m]], "v": w.v[:cu[m]], "g": w.g[:cu[m]],
                             "beta": w.beta[:cu[m]], "cu_seqlens": w.cu_seqlens[:m + 1],
                             "initial_state": w.initial_state[:m]})
        assert gdn.prefill_plan(m, cu[m], Hv, torch.bfloat16, False, True, cus)[0] == "prepared_scan"
        o3, f3 = run_gpu(gdn, head, True)
        assert torch.equal(o3, out[:cu[m]]), m
        assert torch.equal(f3, fin[:m]), m


def test_run_to_run_bitwise(gdn):
    w = _w(seed=22)
    say("[gpu] run-to-run determinism")
    o1, f1 = run_gpu(gdn, w, True)
    o2, f2 = run_gpu(gdn, w, True)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_batch_invariance_bitwise(gdn, dtype):
    """With batch_invariant a sequence's output and state do not depend on the
    rest of the batch or on its position in it."""
    lens = [150, 3, 77, 0, 64]
    w = W.build(lens, 2, 4, dtype, seed=23)
    say(f"[gpu] batch invariance {dtype}")
    out, fin = run_gpu(gdn, w, True)
    cu = w.cu_seqlens.tolist()
    for n in (0, 2, 4):
        sub = W.slice_item(w, n, range(w.Hv))
        sub = W.Workload(**{**sub.__dict__, "q": w.q[cu[n]:cu[n + 1]], "k": w.k[cu[n]:cu[n + 1]]})
        o1, f1 = run_gpu(gdn, sub, True)
        assert torch.equal(o1, out[cu[n]:cu[n + 1]]), n
        assert torch.equal(f1[0], fin[n]), n
    # the same sequences in reverse order
    order = list(reversed(range(len(lens))))
    rev = W.Workload(
        "rev", torch.cat([w.q[cu[n]:cu[n + 1]] for n in order]), torch.cat([w.k[cu[n]:cu[n + 1]] for n in order]),
        torch.cat([w.v[cu[n]:cu[n + 1]] for n in order]), torch.cat([w.g[cu[n]:cu[n + 1]] for n in order]),
        torch.cat([w.beta[cu[n]:cu[n + 1]] for n in order]),
        torch.tensor([0] + list(np.cumsum([lens[n] for n in order])), dtype=torch.int64),
        w.initial_state[order].contiguous(), w.state_dtype, w.use_qk_l2norm)
    o2, f2 = run_gpu(gdn, rev, True)
    cu2 = rev.cu_seqlens.tolist()
    for pos, n in enumerate(order):
        assert torch.equal(o2[cu2[pos]:cu2[pos + 1]], out[cu[n]:cu[n + 1]])
        assert torch.equal(f2[pos], fin[n])


def test_strided_views_of_fused_qkv(gdn):
    """q, k, v as views into one fused [T, 2*Hqk + Hv, 128] buffer (token stride
    larger than the tensor's own row) give bitwise the contiguous result."""
    w = _w(seed=24)
    say("[gpu] strided q/k/v views")
    T, Hqk, Hv = w.T, w.Hqk, w.Hv
    fused = torch.empty(T, 2 * Hqk + Hv, 128, dtype=w.q.dtype)
    fused[:, :Hqk] = w.q
    fused[:, Hqk:2 * Hqk] = w.k
    fused[:, 2 * Hqk:] = w.v
    fd = fused.to(DEV)
    sv = W.Workload(**{**w.to(DEV).__dict__, "q": fd[:, :Hqk], "k": fd[:, Hqk:2 * Hqk], "v": fd[:, 2 * Hqk:]})
    assert sv.q.stride(0) == (2 * Hqk + Hv) * 128 and not sv.q.is_contiguous()
    o1, f1 = run_gpu(gdn, sv, True)
    o2, f2 = run_gpu(gdn, w, True)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_cu_seqlens_int32_equals_int64(gdn):
    w = _w(seed=25)
    say("[gpu] int32 vs int64 cu_seqlens")
    o1, f1 = run_gpu(gdn, W.Workload(**{**w.__dict__, "cu_seqlens": w.cu_seqlens.to(torch.int32)}), True)
    o2, f2 = run_gpu(gdn, W.Workload(**{**w.__dict__, "cu_seqlens": w.cu_seqlens.to(torch.int64)}), True)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, BF16_TOL), (torch.float32, F32_TOL)])
def test_state_chaining_matches_whole(gdn, dtype, tol):
    """Two calls passing the fp32 state (split inside a chunk) match one call."""
    w = W.build([300], 2, 4, dtype, seed=26, gate="long")
    say(f"[gpu] state chaining {dtype}")
    out, fin = run_gpu(gdn, w, True)
    cut = 141
    a = W.Workload(**{**w.__dict__, "q": w.q[:cut], "k": w.k[:cut], "v": w.v[:cut], "g": w.g[:cut],
                      "beta": w.beta[:cut], "cu_seqlens": torch.tensor([0, cut])})
    oa, fa = run_gpu(gdn, a, True)
    b = W.Workload(**{**w.__dict__, "q": w.q[cut:], "k": w.k[cut:], "v": w.v[cut:], "g": w.g[cut:],
                      "beta": w.beta[cut:], "cu_seqlens": torch.tensor([0, 300 - cut]),
                      "initial_state": fa.cpu()})
    ob, fb = run_gpu(gdn, b, True)
    ro, rf = run_oracle(w)
    assert nerr(torch.cat([oa, ob]), ro) <= tol and nerr(fb, rf) <= tol
    assert nerr(torch.cat([oa, ob]).float(), out.float().cpu().numpy()) <= tol


def test_zero_gate_resets_state(gdn):
    """a_t = 0 (hard reset) inside a chunk: finite and matching the oracle."""
    w = _w(lengths=(130,), seed=27)
    g = w.g.clone()
    g[[5, 70, 129]] = 0.0
    w = W.Workload(**{**w.__dict__, "g": g})
    say("[gpu] zero gates")
    out, fin = run_gpu(gdn, w, True)
    ro, rf = run_oracle(w)
    assert torch.isfinite(out).all() and torch.isfinite(fin).all()
    assert nerr(out, ro) <= BF16_TOL and nerr(fin, rf) <= BF16_TOL


def test_strong_decay_slow_path(gdn):
    """Gates small enough that a chunk's total log-decay passes -60 (entry-wise
    exp path) still match the oracle."""
    w = _w(lengths=(200, 64), seed=28)
    w = W.Workload(**{**w.__dict__, "g": torch.full_like(w.g, 0.2)})
    say("[gpu] strong decay")
    out, fin = run_gpu(gdn, w, True)
    ro, rf = run_oracle(w)
    assert nerr(out, ro) <= BF16_TOL and nerr(fin, rf) <= BF16_TOL


@pytest.mark.parametrize("lengths,bi", [((7 * 64 + 13, 130, 64), True), ((8200, 300), False)])
def test_decay_regime_alternating_by_chunk(gdn, lengths, bi):
    """Chunks alternate between mild gates and gates strong enough for the
    entry-wise exp path (total log-decay below -60), so consecutive chunks of one
    sequence take different paths and renormalise the lazy decay at different
    points; the second case is long enough to take the split path."""
    w = _w(lengths=lengths, seed=33)
    t = torch.arange(w.T)
    starts = w.cu_seqlens.to(torch.int64)
    seq = torch.searchsorted(starts[1:], t, right=True)
    chunk = (t - starts[seq]) // 64
    strong = (chunk % 2 == 1).unsqueeze(1)
    g = torch.where(strong, torch.full_like(w.g, 0.2), w.g)
    w = W.Workload(**{**w.__dict__, "g": g})
    say(f"[gpu] alternating decay regimes {lengths} batch_invariant={bi}")
    out, fin = run_gpu(gdn, w, bi)
    ro, rf = run_oracle(w)
    assert nerr(out, ro) <= BF16_TOL and nerr(fin, rf) <= BF16_TOL


@pytest.mark.parametrize("bi", [True, False])
def test_renorm_chunk_with_extreme_decay(gdn, bi):
    """Chunk 0 leaves the lazy decay scale just above the renormalisation
    threshold (log-decay -27.5 over the chunk, sigma ~1.1e-12 > 2^-40); chunk 1
    has a log-decay of -59, still above the entry-wise exp limit of -60, so the
    chunk renormalises with sigma' = sigma gamma_L ~ 3e-38.  Factors of 1 / sigma'
    must not reach the output products (they would overflow bf16 and fp32).
    Raw q/k with the in-kernel norm, so q.k is not bounded by 1."""
    w = _w(lengths=(300, 64 * 3 + 5), Hqk=2, Hv=4, seed=37)
    t = torch.arange(w.T)
    starts = w.cu_seqlens.to(torch.int64)
    seq = torch.searchsorted(starts[1:], t, right=True)
    chunk = ((t - starts[seq]) // 64).unsqueeze(1)
    g = torch.where(chunk == 0, torch.full_like(w.g, float(np.exp(-27.5 / 64))),
                    torch.where(chunk == 1, torch.full_like(w.g, float(np.exp(-59.0 / 64))), w.g))
    w = W.Workload(**{**w.__dict__, "g": g})
    say(f"[gpu] renormalising chunk with log-decay -59 after -27.5, batch_invariant={bi}")
    out, fin = run_gpu(gdn, w, bi)
    assert torch.isfinite(out).all() and torch.isfinite(fin).all()
    ro, rf = run_oracle(w)
    e1, e2 = nerr(out, ro), nerr(fin, rf)
    record(f"renorm chunk, extreme decay bi={int(bi)}", e1, e2, BF16_TOL)
    say(f"      out {e1:.3e} state {e2:.3e}")
    assert e1 <= BF16_TOL and e2 <= BF16_TOL


def test_bf16_gates_and_fp16_gate(gdn):
    w = _w(seed=29)
    say("[gpu] gate dtypes")
    ref = run_gpu(gdn, w, True)
    for gdt in (torch.bfloat16, torch.float16):
        w2 = W.Workload(**{**w.__dict__, "g": w.g.to(gdt), "beta": w.beta.to(torch.bfloat16)})
        out, fin = run_gpu(gdn, w2, True)
        ro, rf = run_oracle(w2)
        assert nerr(out, ro) <= BF16_TOL and nerr(fin, rf) <= BF16_TOL
    del ref


def test_no_output_state_writes_nothing_else(gdn):
    w = _w(seed=30)
    say("[gpu] output_state NULL")
    wd = w.to(DEV)
    out = torch.full((w.T, w.Hv, 128), 7.0, dtype=w.q.dtype, device=DEV)
    gdn.gdn_chunk_prefill(wd.q, wd.k, wd.v, wd.g, wd.beta, 0.0, wd.cu_seqlens, wd.initial_state, None,
                          True, True, out)
    torch.cuda.synchronize()
    ro, _ = run_oracle(w)
    assert nerr(out, ro) <= BF16_TOL


# ---- split path: segment maps, state fix-up, per-segment scan (batch_invariant off)

@pytest.mark.parametrize("gate", ["sigmoid", "long"])
def test_split_path_matches_oracle(gdn, gate):
    """Few long sequences (N * Hv far below two work items per CU) take the split
    path; empty and single-chunk sequences ride along."""
    w = W.build([14000, 5000, 0, 1500, 64], 2, 4, torch.bfloat16, seed=31, gate=gate)
    say(f"[gpu] split path bf16 gate={gate}")
    out, fin = run_gpu(gdn, w, False)
    ro, rf = run_oracle(w)
    e1, e2 = nerr(out, ro), nerr(fin, rf)
    record(f"split path bf16 gate={gate} bi=0", e1, e2, BF16_TOL)
    say(f"      split: out {e1:.3e} state {e2:.3e}")
    assert e1 <= BF16_TOL and e2 <= BF16_TOL
    assert torch.equal(fin[2].cpu(), w.initial_state[2])
    o_u, f_u = run_gpu(gdn, w, True)
    assert not torch.equal(out, o_u), "the split path was not taken (results bitwise equal to the unsplit scan)"
    assert nerr(out.float(), o_u.float().cpu().numpy()) <= BF16_TOL
    assert nerr(fin, f_u.cpu().numpy()) <= BF16_TOL


def test_split_path_fp32(gdn):
    w = W.build([8000, 1025, 3300], 2, 2, torch.float32, seed=32, gate="long")
    say("[gpu] split path fp32")
    out, fin = run_gpu(gdn, w, False)
    ro, rf = run_oracle(w)
    e1, e2 = nerr(out, ro), nerr(fin, rf)
    record("split path fp32 bi=0", e1, e2, F32_TOL)
    say(f"      split fp32: out {e1:.3e} state {e2:.3e}")
    assert e1 <= F32_TOL and e2 <= F32_TOL


def test_split_path_no_states(gdn):
    w = W.build([6000, 2500], 2, 4, torch.bfloat16, seed=33, state_in=None, state_out=None)
    say("[gpu] split path without states")
    out, _ = run_gpu(gdn, w, False)
    ro, _ = run_oracle(w)
    assert nerr(out, ro) <= BF16_TOL


def test_split_path_odd_heads(gdn):
    """3 q/k heads, 6 value heads: the fix-up's (sequence, head) pairs (6) and the
    scan's (item, q/k head) pairs are not multiples of the 8 XCDs."""
    w = W.build([9000, 300], 3, 6, torch.bfloat16, seed=34, gate="long")
    say("[gpu] split path, odd head counts")
    out, fin = run_gpu(gdn, w, False)
    ro, rf = run_oracle(w)
    assert nerr(out, ro) <= BF16_TOL and nerr(fin, rf) <= BF16_TOL


def test_split_path_bf16_states(gdn):
    w = W.build([10000, 0, 2400], 2, 4, torch.bfloat16, seed=34, state_in=torch.bfloat16,
                state_out=torch.bfloat16, gate="long")
    say("[gpu] split path bf16 states")
    out, fin = run_gpu(gdn, w, False)
    ro, rf = run_oracle(w)
    assert nerr(out, ro) <= BF16_TOL and nerr(fin, rf) <= BF16_TOL
    assert torch.equal(fin[1].cpu(), w.initial_state[1])


@pytest.mark.parametrize("case", ["long_single", "four_8192", "uneven"])
def test_prepared_plan_equals_pipelined_scan(gdn, case):
    """The prepared plan (every chunk's preparation in parallel, then the scan
    over it with each head's state rows spread over 4 CUs for the 65,536-token
    sequence on 32 heads and four uneven sequences on 8 heads, over 2 CUs for
    4 x 8192 tokens on 32 heads; the first two leave half the CUs free and run
    in four chunk ranges, the later ranges prepared beside the scan of the
    earlier ones, and the uneven sequences end in different ranges) and the
    pipelined scan (the no-allocation entry point's plan for the same launch)
    give bitwise the same output and final state."""
    if case == "long_single":
        w = W.make(2, device="cuda")
    elif case == "four_8192":
        w = W.build([8192] * 4, 16, 32, torch.bfloat16, seed=64, device="cuda", name="four_8192")
    else:
        w = W.build([20000, 3000, 2373, 9000], 4, 8, torch.bfloat16, seed=65, device="cuda", name="uneven")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert gdn.prefill_plan(w.N, w.T, w.Hv, w.q.dtype, False, True, cus)[0] == "prepared_scan"
    res = []
    for fn in (gdn.gdn_chunk_prefill, gdn.gdn_chunk_prefill_noalloc):
        out = torch.full((w.T, w.Hv, 128), float("nan"), dtype=w.q.dtype, device=DEV)
        fin = torch.full((w.N, w.Hv, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
        fn(w.q, w.k, w.v, w.g, w.beta, w.scale, w.cu_seqlens, w.initial_state, fin, w.use_qk_l2norm, True, out)
        torch.cuda.synchronize()
        res.append((out, fin))
    say(f"[gpu] prepared plan vs pipelined scan, {w.name}")
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
