"""The library's host plan (gdn_prefill_plan, no GPU): which kernels a prefill
call runs for the five workloads and around the thresholds of the split cost
model and the pipelined scan."""
import pytest
import torch

import chunked_gated_delta_prefill_amd as gdn

BF, F32 = torch.bfloat16, torch.float32


def plan(N, T, Hv, dt=BF, ck=False, bi=False, cus=256):
    return gdn.prefill_plan(N, T, Hv, dt, ck, bi, cus)


def test_the_five_workloads():
    assert plan(2, 128, 2, F32) == ("scan", 0)                      # fp32 q/k/v: four-wave scan
    assert plan(8, 15230, 32) == ("pipelined_scan", 0)             # 256 work items = CUs
    assert plan(1, 65536, 32) == ("split", 4096)                    # one long sequence: 16 segments
    assert plan(1, 65536, 32, bi=True) == ("prepared_scan", 0)     # batch_invariant: never split
    assert plan(256, 32280, 32) == ("scan", 0)                      # 8192 work items
    assert plan(32, 262144, 32) == ("scan", 0)                      # the 32 x 8192 batch


def test_split_cost_model():
    # 8 x 8192 on 32 heads: two segments per sequence cost more than the unsplit scan
    assert plan(8, 8 * 8192, 32)[0] == "pipelined_scan"
    # 4 x 16384: four segments, the maps and the scan at two workgroups per CU: still unsplit
    assert plan(4, 4 * 16384, 32)[0] == "prepared_scan"                 # 128 work items: 2 CUs each
    # 2 x 32768: eight segments pay off
    assert plan(2, 2 * 32768, 32) == ("split", 4096)
    # an average below four shortest segments is never split
    assert plan(1, 4 * 1024 - 64, 4)[0] == "prepared_scan"
    assert plan(1, 4 * 1024, 4) == ("split", 1024)


def test_prepared_scan_threshold_and_exclusions():
    assert plan(16, 16 * 100, 4)[0] == "prepared_scan"             # 64 work items: 4 CUs each
    assert plan(32, 32 * 100, 4)[0] == "prepared_scan"             # 128 work items: 2 CUs each
    assert plan(33, 33 * 100, 4)[0] == "pipelined_scan"            # 132 work items
    assert plan(64, 64 * 100, 4)[0] == "pipelined_scan"            # 256 work items
    assert plan(65, 65 * 100, 4)[0] == "scan"                      # 260 work items
    assert plan(16, 16 * 100, 4, cus=128)[0] == "prepared_scan"    # 64 work items, 2 CUs each
    assert plan(64, 64 * 100, 4, cus=128)[0] == "scan"             # fewer CUs
    assert plan(8, 800, 4, dt=F32)[0] == "scan"                    # fp32 q/k/v
    assert plan(8, 800, 4, ck=True)[0] == "scan"                   # checkpoints
    assert plan(0, 0, 4) == ("prepared_scan", 0)                   # empty batch: no work items
    assert plan(0, 100000, 4) == ("prepared_scan", 0)              # no sequences: never split


def test_prepared_workspace_budget():
    """The prepared chunks take ~208 bytes per token and value head; past 8 GiB the
    plan keeps the preparation inside the pipelined scan."""
    slot, per_seg = 13312, 8 * 64
    def prep_bytes(N, T, Hv):
        return (T // per_seg + N + 1) * 8 * Hv * slot
    T_ok = 1 << 20                                   # one sequence of 2^20 tokens, 32 heads: ~6.5 GiB
    assert prep_bytes(1, T_ok, 32) <= 8 << 30
    assert plan(1, T_ok, 32, bi=True)[0] == "prepared_scan"
    T_big = 3 << 19                                  # 1.5 x 2^20 tokens: ~9.8 GiB
    assert prep_bytes(1, T_big, 32) > 8 << 30
    assert plan(1, T_big, 32, bi=True)[0] == "pipelined_scan"


@pytest.mark.parametrize("args", [(-1, 0, 4), (1, -1, 4), (1, 64, 0)])
def test_invalid_sizes_are_rejected(args):
    with pytest.raises(RuntimeError):
        gdn.prefill_plan(*args, BF, False, False, 256)
    with pytest.raises(RuntimeError):
        gdn.prefill_plan(1, 64, 4, torch.float16, False, False, 256)
    with pytest.raises(RuntimeError):
        gdn.prefill_plan(1, 64, 4, BF, False, False, 0)


@pytest.mark.parametrize("args", [(1, (1 << 40) + 64, 4), (1, 1 << 20, 65537), ((1 << 24) + 1, 1 << 24, 1),
                                  (1 << 20, 1 << 30, 4096), (1, 1 << 62, 4)])
def test_sizes_the_prefill_refuses_get_no_plan(args):
    """The planner applies the prefill's own size limits (UNSUPPORTED), so no
    plan exists for a call the prefill would reject, and T * Hv cannot overflow."""
    L = gdn.load()
    import ctypes
    kind, seg = ctypes.c_int(-1), ctypes.c_int64(-1)
    rc = L.gdn_prefill_plan(*args, gdn.GDN_BF16, 0, 0, 256, ctypes.byref(kind), ctypes.byref(seg))
    assert rc == 2, rc
    assert kind.value == -1 and seg.value == -1
