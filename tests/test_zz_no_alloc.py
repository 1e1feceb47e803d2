"""tree_gdn_scan_noalloc, the scan entry point that allocates nothing (its
device plan and parent-state slots live in the library's static scratch
array), against tree_gdn_scan with a caller workspace: bitwise the same
outputs and states, over two calls in a row with the second on a smaller
trie, under both schedules, with and without `states`."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import prefix_tree_packed_plan_amd as ptp
from prefix_tree_packed_plan_amd import _lib
from workloads import make_scan_inputs, make_workload

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _noalloc(plan, t, o, states=None, sched=_lib.SCHED_LEVEL, scale=1.0):
    lib = _lib.load()
    n, h_qk, d_k = t["q"].shape
    h_v, d_v = t["v"].shape[1:]
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.tree_gdn_scan_noalloc(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), t["g"].data_ptr(),
                                   t["beta"].data_ptr(), o.data_ptr(), None,
                                   states.data_ptr() if states is not None else None, n, h_qk, h_v, d_k, d_v,
                                   float(scale), 1 if t["q"].dtype == torch.bfloat16 else 0, sched, plan.handle,
                                   stream)
    return rc


def _cases():
    wl = make_workload(4, DEV, conv=False)  # 55 segments, 26 parents: 52 MiB of parent slots
    rng = np.random.default_rng(3)
    parents = np.array([-1, -1] + [int(rng.integers(0, i)) for i in range(2, 20)], np.int32)
    lens = rng.choice([1, 5, 31, 32, 33, 64, 100, 129], size=20).astype(np.int32)
    small = make_scan_inputs(int(lens.sum()), 2, 4, 128, 128, "bf16", DEV, seed=5)
    return [(wl.parents, wl.seg_lens, wl.tensors), (parents, lens, small)]


@pytest.mark.parametrize("sched", ["level", "rescan"])
@pytest.mark.parametrize("with_states", [False, True])
def test_noalloc_scan_equals_the_workspace_scan(sched, with_states):
    code = _lib.SCHEDULES[sched]
    for i, (parents, lens, t) in enumerate(_cases()):
        plan = ptp.tree_plan(parents, lens, 4)
        say(f"noalloc call {i}: N={plan.n_tokens} segments={plan.n_seg} sched={sched} states={with_states}")
        want_o, want_s = ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, return_states=True,
                                           schedule=sched)
        if not with_states:
            want_o = ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, schedule=sched)
        o = torch.full_like(t["v"], float("nan"))
        st = torch.full_like(want_s, float("nan")) if with_states else None
        assert _noalloc(plan, t, o, st, code) == 0, _lib.load().tree_last_error()
        torch.cuda.synchronize()
        assert torch.equal(o, want_o)
        if with_states:
            assert torch.equal(st, want_s)


def test_noalloc_rejects_a_call_beyond_the_scratch():
    """The RL batch trie's 93 parent states (186 MiB) do not fit the 64 MiB
    array: rejected before any device work; with `states` passed (no parent
    slots needed) the same trie runs and matches."""
    wl = make_workload(5, DEV, conv=False)
    t = wl.tensors
    plan = ptp.tree_plan(wl.parents, wl.seg_lens, 4)
    o = torch.zeros_like(t["v"])
    say("noalloc over-size rejection")
    assert _noalloc(plan, t, o, None, _lib.SCHED_LEVEL) == -5
    assert b"static maximum" in _lib.load().tree_last_error()
    torch.cuda.synchronize()
    assert not o.any()
    want_o, want_s = ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, return_states=True,
                                       schedule="level")
    st = torch.empty_like(want_s)
    assert _noalloc(plan, t, o, st, _lib.SCHED_LEVEL) == 0
    torch.cuda.synchronize()
    assert torch.equal(o, want_o) and torch.equal(st, want_s)
