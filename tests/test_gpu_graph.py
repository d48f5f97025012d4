"""The entry points under HIP graph capture: after one warm-up call on the
capture stream (which sizes the split path's workspace) a call enqueues only
kernels, so it can be captured; every replay must reproduce the eager result
bitwise.  Outputs are poisoned between replays (eager work on the stream) so a
replay that writes nothing is caught."""
import pytest
import torch

import gdn_workloads as W
from _harness import say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _replays_match(call, outs, label, replays=3):
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call()                       # warm-up on the capture stream
        s.synchronize()
        ref = [o.clone() for o in outs]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            call()
        for r in range(replays):
            for o in outs:
                o.fill_(float("nan"))
            g.replay()
            s.synchronize()
            for i, (o, e) in enumerate(zip(outs, ref)):
                assert torch.equal(o, e), f"{label}: replay {r} output {i} differs from the eager result"
    say(f"[gpu] graph {label}: {replays} replays bitwise equal")


@pytest.mark.parametrize("case", ["scan", "split", "prepared"])
def test_prefill_graph_replay(gdn, case):
    if case == "split":      # one long sequence on few heads: plan, maps, fix-up and scan kernels
        w = W.build([8200, 100], 1, 4, torch.bfloat16, seed=51, gate="long").to(DEV)
    elif case == "prepared":  # batch_invariant, few work items: the prepared plan in chunk ranges, the
        # later ranges prepared on the side stream (fork and join captured)
        w = W.build([16384, 5000], 2, 4, torch.bfloat16, seed=58).to(DEV)
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        assert gdn.prefill_plan(w.N, w.T, w.Hv, w.q.dtype, False, True, cus)[0] == "prepared_scan"
    else:
        w = W.build([300, 64, 1, 129], 2, 4, torch.bfloat16, seed=52).to(DEV)
    out = torch.empty(w.T, w.Hv, 128, dtype=w.q.dtype, device=DEV)
    fin = torch.empty(w.N, w.Hv, 128, 128, dtype=torch.float32, device=DEV)
    call = lambda: gdn.gdn_chunk_prefill(w.q, w.k, w.v, w.g, w.beta, 0.0, w.cu_seqlens, w.initial_state, fin,
                                         True, case != "split", out)
    _replays_match(call, [out, fin], "prefill " + case)


def test_decode_graph_replay(gdn):
    w = W.decode_batch(device=DEV, N=16)
    out = torch.empty(w.T, w.Hv, 128, dtype=w.q.dtype, device=DEV)
    s_out = torch.empty_like(w.initial_state)
    call = lambda: gdn.gdn_decode_step(w.q, w.k, w.v, w.g, w.beta, 0.0, w.initial_state, s_out, True, out)
    _replays_match(call, [out, s_out], "decode")


def test_two_streams_concurrently(gdn):
    """Split-path calls on two streams at once use separate workspaces."""
    w1 = W.build([4096], 1, 4, torch.bfloat16, seed=53, gate="long").to(DEV)
    w2 = W.build([4100], 1, 4, torch.bfloat16, seed=54, gate="long").to(DEV)
    res = []
    for w in (w1, w2):
        out = torch.empty(w.T, w.Hv, 128, dtype=w.q.dtype, device=DEV)
        fin = torch.empty(w.N, w.Hv, 128, 128, dtype=torch.float32, device=DEV)
        gdn.gdn_chunk_prefill(w.q, w.k, w.v, w.g, w.beta, 0.0, w.cu_seqlens, w.initial_state, fin, True, False, out)
        res.append((out, fin))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    got = []
    for w, s in ((w1, s1), (w2, s2)):
        out = torch.full((w.T, w.Hv, 128), float("nan"), dtype=w.q.dtype, device=DEV)
        fin = torch.full((w.N, w.Hv, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            gdn.gdn_chunk_prefill(w.q, w.k, w.v, w.g, w.beta, 0.0, w.cu_seqlens, w.initial_state, fin, True, False,
                                  out)
        got.append((out, fin))
    torch.cuda.synchronize()
    for (o, f), (eo, ef) in zip(got, res):
        assert torch.equal(o, eo) and torch.equal(f, ef)
    say("[gpu] two streams: both results bitwise equal to the single-stream runs")


def test_graph_survives_workspace_growth(gdn):
    """A graph captured from a small split-path call keeps its workspace after a
    larger eager split call on the same stream grows the cached workspace: the
    superseded buffer is retired, not freed, so replays still write the small
    call's results bitwise."""
    small = W.build([8200, 100], 1, 4, torch.bfloat16, seed=55, gate="long").to(DEV)
    large = W.build([40000, 3000], 1, 4, torch.bfloat16, seed=56, gate="long").to(DEV)
    assert gdn.prefill_plan(small.N, small.T, small.Hv, small.q.dtype, False, False, 256)[0] == "split"
    assert gdn.prefill_plan(large.N, large.T, large.Hv, large.q.dtype, False, False, 256)[0] == "split"

    def bufs(w):
        return (torch.empty(w.T, w.Hv, 128, dtype=w.q.dtype, device=DEV),
                torch.empty(w.N, w.Hv, 128, 128, dtype=torch.float32, device=DEV))

    def call(w, out, fin):
        gdn.gdn_chunk_prefill(w.q, w.k, w.v, w.g, w.beta, 0.0, w.cu_seqlens, w.initial_state, fin, True, False, out)

    so, sf = bufs(small)
    lo, lf = bufs(large)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call(small, so, sf)                 # sizes the stream's workspace for the small call
        s.synchronize()
        ref = (so.clone(), sf.clone())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            call(small, so, sf)
        call(large, lo, lf)                 # grows the workspace (eager, same stream)
        s.synchronize()
        for r in range(3):
            so.fill_(float("nan"))
            sf.fill_(float("nan"))
            g.replay()
            s.synchronize()
            assert torch.equal(so, ref[0]) and torch.equal(sf, ref[1]), f"replay {r} after growth differs"
            call(large, lo, lf)             # eager work on the stream between replays
            s.synchronize()
    say("[gpu] graph replays after workspace growth: bitwise equal")


def test_growth_during_capture_is_refused(gdn):
    """A split call that would have to grow the workspace while its stream is
    capturing is refused (UNSUPPORTED) and enqueues nothing."""
    w = W.build([8200, 100], 1, 4, torch.bfloat16, seed=57, gate="long").to(DEV)
    out = torch.zeros(w.T, w.Hv, 128, dtype=w.q.dtype, device=DEV)
    fin = torch.zeros(w.N, w.Hv, 128, 128, dtype=torch.float32, device=DEV)
    # the library's one-time device query happens here, outside the capture
    gdn.gdn_chunk_prefill(w.q[:64], w.k[:64], w.v[:64], w.g[:64], w.beta[:64], 0.0,
                          torch.tensor([0, 64], dtype=torch.int32, device=DEV), None, None, True, True, out[:64])
    torch.cuda.synchronize()
    out.zero_()
    s = torch.cuda.Stream()                 # a new stream: no workspace yet
    code = None
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            try:
                gdn.gdn_chunk_prefill(w.q, w.k, w.v, w.g, w.beta, 0.0, w.cu_seqlens, w.initial_state, fin, True,
                                      False, out)
            except gdn.GdnError as e:
                code = e.code
            out.add_(1.0)                   # keep the captured graph non-empty
        g.replay()
        s.synchronize()
    assert code == 2, code
    assert torch.equal(out, torch.ones_like(out)) and torch.equal(fin, torch.zeros_like(fin))
    say("[gpu] workspace growth during capture: refused")


def test_release_and_reuse(gdn):
    """gdn_release_workspace frees the cached workspaces and destroys the side
    streams and events of prepared calls in chunk ranges; the next calls on the
    same stream create them again and give bitwise the same results."""
    cases = [(W.build([8200, 100], 1, 4, torch.bfloat16, seed=59, gate="long").to(DEV), False, "split"),
             (W.build([16384, 5000], 2, 4, torch.bfloat16, seed=60).to(DEV), True, "prepared")]
    for w, bi, label in cases:
        res = []
        for _ in range(2):
            out = torch.full((w.T, w.Hv, 128), float("nan"), dtype=w.q.dtype, device=DEV)
            fin = torch.full((w.N, w.Hv, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
            gdn.gdn_chunk_prefill(w.q, w.k, w.v, w.g, w.beta, 0.0, w.cu_seqlens, w.initial_state, fin, True, bi, out)
            torch.cuda.synchronize()
            res.append((out, fin))
            gdn.release_workspace()
        assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1]), label
        say(f"[gpu] release and reuse, {label}: bitwise equal")
