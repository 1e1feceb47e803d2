"""GPU parity of the tree Mamba2 (SSD) forward (tree_ssd_scan through the C
ABI) against the per-path oracle (oracle/ssd.py): outputs and every
segment's final state on ragged forests, and sampled segments plus exact
properties on the RL batch trie with Mamba2-2.7B-shaped heads."""
import sys

import numpy as np
import pytest
import torch

from tests import parity
from workloads import SSD_SHAPE, make_ssd_inputs, make_workload

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
Y_F32_ATOL = 1e-4  # fp32 inputs and outputs, fp32 arithmetic


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rand_trie(seed, n_seg, lens_choices, n_roots=1):
    rng = np.random.default_rng(seed)
    parents = [-1] * n_roots + [int(rng.integers(0, i)) for i in range(n_roots, n_seg)]
    return np.array(parents, np.int32), rng.choice(lens_choices, size=n_seg).astype(np.int32)


def host(t):
    return {k: parity.to_np(v) for k, v in t.items()}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 2, 128, 64), (2, 4, 128, 64), (2, 4, 128, 32), (2, 4, 64, 32)])
def test_ssd_matches_the_oracle(dtype, shape):
    """Ragged forest (1..40-token segments: whole 16-token chunks and tails,
    fan-outs), given root states, D on; outputs and every final state."""
    from oracle import ssd as ossd
    ptp = __import__("prefix_tree_packed_plan_amd")
    G, H, N, P = shape
    parents, lens = rand_trie(81, 18, [1, 3, 16, 17, 33, 40], n_roots=2)
    n = int(lens.sum())
    say(f"ssd dtype={dtype} groups={G} heads={H} d_state={N} head_dim={P} N={n}")
    t = make_ssd_inputs(n, G, H, N, P, dtype, DEV, seed=3)
    g = torch.Generator().manual_seed(4)
    init = (torch.randn((2, H, N, P), generator=g) * 0.3).to(DEV)
    plan = ptp.tree_plan(parents, lens, 4)
    y, st = ptp.tree_ssd_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], plan, D=t["D"], return_states=True,
                              init_states=init)
    torch.cuda.synchronize()
    hh = host(t)
    ry, rs = ossd.tree_ssd_reference(parents, lens, hh["x"], hh["dt"], hh["A"], hh["B"], hh["C"], hh["D"],
                                     init_states=parity.to_np(init))
    ey = parity.out_err(y, ry, what="ssd output") if dtype == "bf16" else float(np.abs(parity.to_np(y) - ry).max())
    es = float(parity.state_rel_err(parity.to_np(st), rs).max())
    say(f"  y {ey:.3e}  state {es:.3e}")
    assert ey <= (parity.OUT_ATOL if dtype == "bf16" else Y_F32_ATOL)
    assert es <= parity.STATE_RTOL


def test_ssd_workspace_slots_equal_states_output_and_zero_step():
    """Without `states` the parents' states go through workspace slots: the
    outputs are bitwise those of the run that writes `states`.  With dt = 0
    everywhere y = D x exactly (the state stays zero)."""
    ptp = __import__("prefix_tree_packed_plan_amd")
    parents, lens = rand_trie(82, 12, [5, 16, 40], n_roots=1)
    n = int(lens.sum())
    t = make_ssd_inputs(n, 1, 2, 128, 64, "bf16", DEV, seed=5)
    plan = ptp.tree_plan(parents, lens, 4)
    y1, _ = ptp.tree_ssd_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], plan, D=t["D"], return_states=True)
    y2 = ptp.tree_ssd_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], plan, D=t["D"])
    zero = ptp.tree_ssd_scan(t["x"], torch.zeros_like(t["dt"]), t["A"], t["B"], t["C"], plan, D=t["D"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(zero, t["x"])  # D = 1


def test_ssd_rl_batch_sampled_segments_and_determinism():
    """RL batch trie (N = 428,843) with 80 heads of 64, d_state 128: sampled
    segments of every level (heads 0, 41 and 79) against the oracle on their
    root paths; two runs are bitwise equal."""
    from oracle import ssd as ossd
    ptp = __import__("prefix_tree_packed_plan_amd")
    wl = make_workload(5, None, conv=False, scan=False)
    s = SSD_SHAPE
    n = wl.n_tokens
    t = make_ssd_inputs(n, s["n_groups"], s["n_heads"], s["d_state"], s["head_dim"], "bf16", DEV, seed=0)
    plan = ptp.tree_plan(wl.parents, wl.seg_lens, 4)
    say(f"ssd rl_batch N={n}")
    y1, st = ptp.tree_ssd_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], plan, D=t["D"], return_states=True)
    y2 = ptp.tree_ssd_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], plan, D=t["D"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    segs = parity.sample_segments(wl.parents, wl.seg_lens, 4, seed=1)
    heads = np.array([0, 41, 79])
    hh = {k: parity.to_np(v) for k, v in t.items()}
    ry, rs = ossd.tree_ssd_reference(wl.parents, wl.seg_lens, hh["x"], hh["dt"], hh["A"], hh["B"], hh["C"],
                                     hh["D"], segments=segs, heads=heads)
    off = np.concatenate([[0], np.cumsum(wl.seg_lens)])
    for sg in segs:
        rows = np.arange(off[sg], off[sg + 1])
        ey = parity.out_err(y1[torch.as_tensor(rows, device=DEV)][:, heads], ry[rows][:, heads], what="ssd output")
        es = float(parity.state_rel_err(parity.to_np(st[sg][heads]), rs[sg][heads]).max())
        say(f"  segment {sg}: y {ey:.3e}  state {es:.3e}")
        assert ey <= parity.OUT_ATOL and es <= parity.STATE_RTOL


@pytest.mark.parametrize("case", ["no_decay", "full_forget", "large_step"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ssd_degenerate_decay(case, dtype):
    """The decay at its limits, given root states, D on; outputs and every
    final state against the oracle.  no_decay: A dt -> 0, the state sums every
    token of the path.  full_forget: A dt = -80 at every token with a small
    step (A = -8000, dt = 0.01), so the state holds only the last token's
    write.  large_step: the same decay through dt = 5 (A = -16), which also
    scales the writes and puts outputs in the hundreds; the fp32 path carries
    its products as split bf16 (2^-16 of the sum of the terms' magnitudes), so
    there its bar is 1e-4 of the largest output rather than 1e-4 absolute."""
    from oracle import ssd as ossd
    ptp = __import__("prefix_tree_packed_plan_amd")
    G, H, N, P = 2, 4, 128, 64
    parents, lens = rand_trie(83, 18, [1, 3, 16, 17, 33, 40, 64], n_roots=2)
    n = int(lens.sum())
    say(f"ssd degenerate decay {case} dtype={dtype} N={n}")
    t = make_ssd_inputs(n, G, H, N, P, dtype, DEV, seed=6)
    A, dt = {"no_decay": (-1e-6, 0.05), "full_forget": (-8000.0, 0.01), "large_step": (-16.0, 5.0)}[case]
    t["A"] = torch.full_like(t["A"], A)
    t["dt"] = torch.full_like(t["dt"], dt)
    g = torch.Generator().manual_seed(7)
    init = (torch.randn((2, H, N, P), generator=g) * 0.3).to(DEV)
    plan = ptp.tree_plan(parents, lens, 4)
    y, st = ptp.tree_ssd_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], plan, D=t["D"], return_states=True,
                              init_states=init)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all() and torch.isfinite(st).all()
    hh = host(t)
    ry, rs = ossd.tree_ssd_reference(parents, lens, hh["x"], hh["dt"], hh["A"], hh["B"], hh["C"], hh["D"],
                                     init_states=parity.to_np(init))
    ey = parity.out_err(y, ry, what="ssd output") if dtype == "bf16" else float(np.abs(parity.to_np(y) - ry).max())
    es = float(parity.state_rel_err(parity.to_np(st), rs).max())
    say(f"  y {ey:.3e} (max |y| {np.abs(ry).max():.3e})  state {es:.3e}")
    f32_bar = Y_F32_ATOL * (np.abs(ry).max() if case == "large_step" else 1.0)
    assert ey <= (parity.OUT_ATOL if dtype == "bf16" else f32_bar)
    assert es <= parity.STATE_RTOL
