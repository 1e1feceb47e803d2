"""GPU parity of the backward: the HIP conv backward (through the C ABI)
against the autograd oracle (oracle/grad.py) on ragged forests, and exact
properties at the full RL batch size."""
import sys

import numpy as np
import pytest
import torch

from tests import parity
from workloads import make_conv_inputs, make_workload

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rand_trie(seed, n_seg, lens_choices, n_roots=1):
    rng = np.random.default_rng(seed)
    parents = [-1] * n_roots + [int(rng.integers(0, i)) for i in range(n_roots, n_seg)]
    lens = rng.choice(lens_choices, size=n_seg)
    return np.array(parents, np.int32), np.array(lens, np.int32)


def rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W", [1, 2, 4])
@pytest.mark.parametrize("C", [13, 96])
@pytest.mark.parametrize("act", [None, "silu"])
def test_conv_backward_matches_the_oracle(dtype, W, C, act):
    """Short segments and many children, so successor windows reach into
    grandchildren and root contexts; bias and given contexts on."""
    from oracle import grad as ograd
    ptp = __import__("prefix_tree_packed_plan_amd")
    parents, lens = rand_trie(61, 40, [1, 2, 3, 5, 9, 70], n_roots=3)
    n = int(lens.sum())
    say(f"conv backward dtype={dtype} W={W} C={C} act={act} N={n}")
    t = make_conv_inputs(n, C, W, dtype, DEV, seed=7, with_bias=True)
    dy = make_conv_inputs(n, C, W, dtype, DEV, seed=8)["x"]
    init = make_conv_inputs(3 * max(W - 1, 1), C, W, dtype, DEV, seed=9)["x"][: 3 * (W - 1)]
    init = init.reshape(3, W - 1, C).contiguous()
    plan = ptp.tree_plan(parents, lens, W)
    dx, dw, db, dctx = ptp.tree_conv_backward(t["x"], t["w"], dy, plan, bias=t["bias"], act=act, init_ctx=init)
    torch.cuda.synchronize()
    f = parity.to_np
    rx, rw, rb, rc = ograd.tree_conv_vjp(parents, lens, f(t["x"]), f(t["w"]), f(dy), bias=f(t["bias"]), act=act,
                                         init_ctx=f(init))
    ex = parity.out_err(dx, rx) if dtype == "bf16" else float(np.abs(f(dx) - rx).max())
    say(f"  dx {ex:.3e}  dw {rel(f(dw), rw):.3e}  dbias {rel(f(db), rb):.3e}")
    assert ex <= (parity.OUT_ATOL if dtype == "bf16" else 1e-4)
    assert rel(f(dw), rw) <= 1e-5 and rel(f(db), rb) <= 1e-5
    if W > 1:
        assert rel(f(dctx), rc) <= 1e-5


def test_conv_backward_full_size_properties_and_determinism():
    """RL batch trie, C = 8192: dbias = sum of dy and the current-token tap
    dw[:, W-1] = sum of dy * x (exact fp64 sums on the host side); two runs
    are bitwise equal."""
    ptp = __import__("prefix_tree_packed_plan_amd")
    wl = make_workload(5, DEV, scan=False)
    s, t = wl.spec, wl.tensors
    say(f"conv backward rl_batch N={wl.n_tokens} C={s.channels}")
    dy = make_conv_inputs(wl.n_tokens, s.channels, s.conv_width, "bf16", DEV, seed=3)["x"]
    bias = torch.zeros(s.channels, dtype=torch.bfloat16, device=DEV)
    plan = ptp.tree_plan(wl.parents, wl.seg_lens, s.conv_width)
    dx1, dw1, db1, _ = ptp.tree_conv_backward(t["x"], t["w"], dy, plan, bias=bias)
    dx2, dw2, db2, _ = ptp.tree_conv_backward(t["x"], t["w"], dy, plan, bias=bias)
    torch.cuda.synchronize()
    assert torch.equal(dx1, dx2) and torch.equal(dw1, dw2) and torch.equal(db1, db2)
    want_b = dy.double().sum(0)
    want_w = (dy.double() * t["x"].double()).sum(0)
    eb = float((db1.double() - want_b).abs().max() / want_b.abs().max())
    ew = float((dw1[:, -1].double() - want_w).abs().max() / want_w.abs().max())
    say(f"  dbias rel {eb:.3e}  dw[:, W-1] rel {ew:.3e}")
    assert eb <= 1e-4 and ew <= 1e-4
