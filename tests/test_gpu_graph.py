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


@pytest.mark.parametrize("split", [False, True])
def test_prefill_graph_replay(gdn, split):
    if split:   # one long sequence on few heads: plan, maps, fix-up and scan kernels
        w = W.build([8200, 100], 1, 4, torch.bfloat16, seed=51, gate="long").to(DEV)
    else:
        w = W.build([300, 64, 1, 129], 2, 4, torch.bfloat16, seed=52).to(DEV)
    out = torch.empty(w.T, w.Hv, 128, dtype=w.q.dtype, device=DEV)
    fin = torch.empty(w.N, w.Hv, 128, 128, dtype=torch.float32, device=DEV)
    call = lambda: gdn.gdn_chunk_prefill(w.q, w.k, w.v, w.g, w.beta, 0.0, w.cu_seqlens, w.initial_state, fin,
                                         True, not split, out)
    _replays_match(call, [out, fin], "prefill split" if split else "prefill")


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
