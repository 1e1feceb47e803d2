"""GPU parity of the backward: the HIP conv backward (through the C ABI)
against the autograd oracle (oracle/grad.py) on ragged forests, and exact
properties at the full RL batch size."""
import sys

import numpy as np
import pytest
import torch

from tests import parity
from workloads import make_conv_inputs, make_scan_inputs, make_workload

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
    ex = parity.out_err(dx, rx, what="conv backward dx") if dtype == "bf16" else float(np.abs(f(dx) - rx).max())
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


# ---------------------------------------------------------------- scan backward

def _randn(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * std).to(DEV)


def _scan_grads(ptp, plan, t, do, scale, init=None, dstates=None, states=None):
    if states is None:
        _, states = ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, scale=scale,
                                      return_states=True, init_states=init, schedule="level")
    return ptp.tree_gdn_scan_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], do, plan, states, scale=scale,
                                      init_states=init, dstates=dstates)


# Max-norm relative error of every gradient against the fp64 oracle.  The
# arithmetic is fp32 throughout; "Tree Training" appendix B.8 reports fp32
# backward errors below 2e-5 for its SSM hybrid, the bar taken here
# (measured: about 2e-6 at most).
SCAN_GRAD_RTOL = 2e-5
GRAD_NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dinit")


@pytest.mark.parametrize("dtype,d", [("f32", 32), ("bf16", 32), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("heads", [(1, 1), (1, 2), (2, 4), (1, 4)])
def test_scan_backward_matches_the_oracle(dtype, d, heads):
    """Ragged forest (segments of 1..40 tokens: whole 16-token chunks and
    tails, chains and fan-outs), given root states and final-state
    gradients, scale != 1; every gradient against autograd of the fp64
    token-by-token oracle."""
    from oracle import gdn as ogdn
    from oracle import grad as ograd
    ptp = __import__("prefix_tree_packed_plan_amd")
    h_qk, h_v = heads
    parents, lens = rand_trie(71, 12 if d == 128 else 16, [1, 3, 16, 17, 33, 40], n_roots=2)
    n = int(lens.sum())
    say(f"scan backward dtype={dtype} d={d} heads={h_qk}/{h_v} N={n}")
    t = make_scan_inputs(n, h_qk, h_v, d, d, dtype, DEV, seed=11)
    do = make_scan_inputs(n, h_qk, h_v, d, d, dtype, DEV, seed=12)["v"]
    init = _randn((2, h_v, d, d), 13, 0.3)
    dst = _randn((len(parents), h_v, d, d), 14, 0.1)
    f = parity.to_np
    plan = ptp.tree_plan(parents, lens, 4)
    states = None
    if d == 64:  # no forward kernel at this size: take the oracle's final states
        _, st = ogdn.tree_gdn_reference(parents, lens, f(t["q"]), f(t["k"]), f(t["v"]), f(t["g"]), f(t["beta"]),
                                        0.6, init_states=f(init))
        states = torch.tensor(st, dtype=torch.float32, device=DEV)
    got = _scan_grads(ptp, plan, t, do, 0.6, init=init, dstates=dst, states=states)
    torch.cuda.synchronize()
    ref = ograd.tree_gdn_vjp(parents, lens, f(t["q"]), f(t["k"]), f(t["v"]), f(t["g"]), f(t["beta"]), f(do),
                             scale=0.6, init_states=f(init), dstates=f(dst))
    errs = {nm: rel(f(a), b) for nm, a, b in zip(GRAD_NAMES, got, ref)}
    say("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= SCAN_GRAD_RTOL, errs


@pytest.mark.parametrize("dtype,d", [("f32", 32), ("bf16", 128)])
@pytest.mark.parametrize("shape", ["roots_only", "deep_chain"])
def test_scan_backward_paired_heads_level_launches(dtype, d, shape):
    """Two value heads per q/k head: the first head of each pair stores its
    part of dq and dk and the second adds to it one launch later, with level
    l's first heads sharing a launch with level l + 1's second heads.  The
    end cases of that schedule: a forest of roots only (one level: the first
    heads, then the second heads alone) and a chain of six levels."""
    from oracle import grad as ograd
    ptp = __import__("prefix_tree_packed_plan_amd")
    if shape == "roots_only":
        parents = np.array([-1, -1, -1], np.int32)
        lens = np.array([5, 16, 40], np.int32)
    else:
        parents = np.array([-1, 0, 1, 2, 3, 4], np.int32)
        lens = np.array([17, 3, 16, 1, 20, 9], np.int32)
    n = int(lens.sum())
    say(f"scan backward paired heads {shape} dtype={dtype} d={d} N={n}")
    t = make_scan_inputs(n, 2, 4, d, d, dtype, DEV, seed=41)
    do = make_scan_inputs(n, 2, 4, d, d, dtype, DEV, seed=42)["v"]
    plan = ptp.tree_plan(parents, lens, 4)
    got = _scan_grads(ptp, plan, t, do, 0.8)
    torch.cuda.synchronize()
    f = parity.to_np
    ref = ograd.tree_gdn_vjp(parents, lens, f(t["q"]), f(t["k"]), f(t["v"]), f(t["g"]), f(t["beta"]), f(do),
                             scale=0.8)
    errs = {nm: rel(f(a), b) for nm, a, b in zip(GRAD_NAMES, got, ref)}
    say("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= SCAN_GRAD_RTOL, errs


def test_scan_backward_single_token_segments_and_zero_gradients():
    """Degenerate shapes: a chain of one-token segments under a root of one
    token, and a zero upstream gradient (every gradient exactly zero)."""
    from oracle import grad as ograd
    ptp = __import__("prefix_tree_packed_plan_amd")
    parents = np.array([-1, 0, 1, 2, 2, 4], np.int32)
    lens = np.array([1, 1, 1, 1, 2, 1], np.int32)
    n = int(lens.sum())
    t = make_scan_inputs(n, 1, 1, 32, 32, "f32", DEV, seed=21)
    do = make_scan_inputs(n, 1, 1, 32, 32, "f32", DEV, seed=22)["v"]
    plan = ptp.tree_plan(parents, lens, 4)
    got = _scan_grads(ptp, plan, t, do, 1.0)
    f = parity.to_np
    ref = ograd.tree_gdn_vjp(parents, lens, f(t["q"]), f(t["k"]), f(t["v"]), f(t["g"]), f(t["beta"]), f(do))
    for nm, a, b in zip(GRAD_NAMES, got, ref):
        assert rel(f(a), b) <= SCAN_GRAD_RTOL, nm
    zero = _scan_grads(ptp, plan, t, torch.zeros_like(do), 1.0)
    for nm, a in zip(GRAD_NAMES, zero):
        assert not bool(a.abs().max()), nm


def test_scan_backward_full_size_determinism_and_linearity():
    """RL batch trie (16 q/k and 32 value heads of 128): two runs are bitwise equal, and the
    gradients are linear in the upstream gradient: grads(do) = grads(do on
    even tokens) + grads(do on odd tokens) to fp32 rounding."""
    ptp = __import__("prefix_tree_packed_plan_amd")
    wl = make_workload(5, DEV, conv=False)
    s, t = wl.spec, wl.tensors
    say(f"scan backward rl_batch N={wl.n_tokens} heads={s.h_qk}/{s.h_v}")
    plan = ptp.tree_plan(wl.parents, wl.seg_lens, s.conv_width)
    _, states = ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, return_states=True,
                                  schedule="level")
    do1 = make_scan_inputs(wl.n_tokens, s.h_qk, s.h_v, s.d_k, s.d_v, "bf16", DEV, seed=31)["v"]
    # Split do1 into its even-token and odd-token rows: the parts are
    # independent and their sum is exactly do1.
    even = (torch.arange(wl.n_tokens, device=DEV) % 2 == 0).view(-1, 1, 1)
    half = torch.where(even, do1, torch.zeros_like(do1))
    rest = torch.where(even, torch.zeros_like(do1), do1)
    assert torch.equal(half + rest, do1)
    ws = torch.empty(int(ptp.load().tree_gdn_scan_backward_workspace_bytes(plan.handle, s.h_qk, s.h_v, s.d_k,
                                                                           s.d_v)), dtype=torch.uint8, device=DEV)
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"])
    a = ptp.tree_gdn_scan_backward(*args, do1, plan, states, workspace=ws)
    b = ptp.tree_gdn_scan_backward(*args, do1, plan, states, workspace=ws)
    torch.cuda.synchronize()
    for nm, x, y in zip(GRAD_NAMES, a, b):
        assert torch.equal(x, y), nm
    h1 = ptp.tree_gdn_scan_backward(*args, half, plan, states, workspace=ws)
    h2 = ptp.tree_gdn_scan_backward(*args, rest, plan, states, workspace=ws)
    torch.cuda.synchronize()
    for nm, x, y, z in zip(GRAD_NAMES, a, h1, h2):
        e = float((x.double() - y.double() - z.double()).abs().max() / x.double().abs().max().clamp_min(1e-30))
        say(f"  linearity {nm} {e:.2e}")
        assert e <= 1e-4, nm


def test_scan_backward_full_size_sampled_path_against_the_oracle():
    """RL batch trie at full size, upstream gradient only on the leaf with the
    shortest root path: the gradients on that path (value heads 0 and 1, which
    share q/k head 0) match the oracle run on the path as a chain, and every
    gradient off the path is exactly zero."""
    from oracle import grad as ograd
    ptp = __import__("prefix_tree_packed_plan_amd")
    wl = make_workload(5, DEV, conv=False)
    s, t = wl.spec, wl.tensors
    parents, lens = np.asarray(wl.parents), np.asarray(wl.seg_lens)
    off = np.concatenate([[0], np.cumsum(lens)])
    leaves = sorted(set(range(len(parents))) - set(int(p) for p in parents if p >= 0))

    def path(sg):
        out = []
        while sg >= 0:
            out.append(sg)
            sg = int(parents[sg])
        return out[::-1]

    leaf = min(leaves, key=lambda x: sum(int(lens[p]) for p in path(x)))
    segs = path(leaf)
    rows = np.concatenate([np.arange(off[p], off[p + 1]) for p in segs])
    say(f"scan backward sampled path: leaf {leaf}, {len(segs)} segments, {len(rows)} tokens")
    plan = ptp.tree_plan(parents, lens, s.conv_width)
    _, states = ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, return_states=True,
                                  schedule="level")
    src = make_scan_inputs(wl.n_tokens, s.h_qk, s.h_v, s.d_k, s.d_v, "bf16", DEV, seed=41)["v"]
    on_leaf = torch.zeros(wl.n_tokens, dtype=torch.bool, device=DEV)
    on_leaf[int(off[leaf]):int(off[leaf + 1])] = True
    do = torch.where(on_leaf.view(-1, 1, 1), src, torch.zeros_like(src))
    got = ptp.tree_gdn_scan_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], do, plan, states)
    torch.cuda.synchronize()
    on_path = torch.zeros(wl.n_tokens, dtype=torch.bool, device=DEV)
    on_path[torch.as_tensor(rows, device=DEV)] = True
    for nm, a in zip(GRAD_NAMES[:5], got[:5]):
        assert not bool(a[~on_path].abs().max()), nm
    f = parity.to_np
    r = torch.as_tensor(rows, device=DEV)
    chain = np.arange(-1, len(segs) - 1, dtype=np.int32)
    plens = np.array([lens[p] for p in segs], np.int32)
    ref = ograd.tree_gdn_vjp(chain, plens, f(t["q"][r, 0:1]), f(t["k"][r, 0:1]), f(t["v"][r, 0:2]),
                             f(t["g"][r, 0:2]), f(t["beta"][r, 0:2]), f(do[r, 0:2]))
    mine = (got[0][r, 0:1], got[1][r, 0:1], got[2][r, 0:2], got[3][r, 0:2], got[4][r, 0:2])
    errs = {nm: rel(f(a), b) for nm, a, b in zip(GRAD_NAMES, mine, ref)}
    say("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= SCAN_GRAD_RTOL, errs
