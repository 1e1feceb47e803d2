"""GPU parity on the scan's degenerate cases and extreme trie shapes, against
the oracle (through the C ABI).

Gates at their limits: no decay with full writes (g = 0, beta = 1: the
state accumulates over whole paths, the hardest case for its precision), no
writes (beta = 0), complete forgetting at every token (g = -40), and a random
mix of these.  Trie shapes: a deep chain run one launch per level, and one
wide level of single-token segments.
"""
import sys

import numpy as np
import pytest
import torch

from tests import parity
from workloads import make_scan_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
RAGGED = [1, 2, 3, 5, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 200, 300]


def _lib():
    import prefix_tree_packed_plan_amd as ptp
    return ptp


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rand_trie(seed, n_seg, lens_choices, n_roots=1):
    rng = np.random.default_rng(seed)
    parents = [-1] * n_roots + [int(rng.integers(0, i)) for i in range(n_roots, n_seg)]
    lens = rng.choice(lens_choices, size=n_seg)
    return np.array(parents, np.int32), np.array(lens, np.int32)


def _gates(case, n, h_v, seed):
    gen = torch.Generator(device="cpu").manual_seed(seed)
    if case == "no_decay":
        g, b = torch.zeros(n, h_v), torch.ones(n, h_v)
    elif case == "no_write":
        g = -torch.nn.functional.softplus(torch.randn(n, h_v, generator=gen))
        b = torch.zeros(n, h_v)
    elif case == "full_forget":
        g, b = torch.full((n, h_v), -40.0), torch.sigmoid(torch.randn(n, h_v, generator=gen))
    else:  # mix
        g = torch.where(torch.rand(n, h_v, generator=gen) < 0.5, 0.0, -40.0)
        b = (torch.rand(n, h_v, generator=gen) < 0.5).float()
    return g.to(DEV).contiguous(), b.to(DEV).contiguous()


@pytest.mark.parametrize("case", ["no_decay", "no_write", "full_forget", "mix"])
@pytest.mark.parametrize("dtype,d,h_qk,h_v", [("f32", 32, 1, 2), ("bf16", 64, 1, 2), ("bf16", 128, 2, 4)])
def test_scan_degenerate_gates(case, dtype, d, h_qk, h_v):
    """Both schedules agree bit for bit, from zero and from given root
    states, and match the oracle.  Without writes and from zero states the
    outputs and states are exactly zero."""
    ptp = _lib()
    parents, lens = rand_trie(31, 20, RAGGED, n_roots=2)
    n = int(lens.sum())
    say(f"degenerate gates {case} dtype={dtype} d={d} heads={h_qk}/{h_v} N={n}")
    t = make_scan_inputs(n, h_qk, h_v, d, d, dtype, DEV, seed=21)
    t["g"], t["beta"] = _gates(case, n, h_v, 22)
    plan = ptp.tree_plan(parents, lens, 4)
    gen = torch.Generator(device="cpu").manual_seed(23)
    init = (torch.randn(2, h_v, d, d, generator=gen) * 0.1).to(DEV)
    for init_states in (None, init):
        kw = {} if init_states is None else {"init_states": init_states}
        o1, s1 = ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, scale=0.75,
                                   return_states=True, schedule="level", **kw)
        o2, s2 = ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, scale=0.75,
                                   return_states=True, schedule="rescan", **kw)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(s1, s2)
        assert torch.isfinite(o1.float()).all() and torch.isfinite(s1).all()
        if case == "no_write" and init_states is None:
            assert not o1.float().abs().max().item() and not s1.abs().max().item()
        eo, es = parity.scan_errors_full(parents, lens, t["q"], t["k"], t["v"], t["g"], t["beta"], o1, s1,
                                         scale=0.75, init_states=init_states)
        say(f"  init={'given' if init_states is not None else 'zero'}: out {eo:.3e}  state {es:.3e}")
        assert eo <= parity.out_atol(dtype) and es <= parity.STATE_RTOL


def test_deep_chain_one_launch_per_level():
    """A chain of 400 segments of 1-5 tokens forced onto the level schedule
    (400 launches, each segment starting from its parent's state in a
    workspace slot or in `states`) equals the rescan and the oracle."""
    ptp = _lib()
    rng = np.random.default_rng(41)
    lens = rng.integers(1, 6, size=400).astype(np.int32)
    parents = np.arange(-1, len(lens) - 1, dtype=np.int32)
    n = int(lens.sum())
    say(f"deep chain: 400 levels, N={n}")
    t = make_scan_inputs(n, 2, 4, 128, 128, "bf16", DEV, seed=42)
    plan = ptp.tree_plan(parents, lens, 4)
    o1, s1 = ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, return_states=True,
                               schedule="level")
    o2 = ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, schedule="level")
    o3, s3 = ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, return_states=True,
                               schedule="rescan")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o1, o3) and torch.equal(s1, s3)
    eo, es = parity.scan_errors_full(parents, lens, t["q"], t["k"], t["v"], t["g"], t["beta"], o1, s1)
    say(f"  out {eo:.3e}  state {es:.3e}")
    assert eo <= parity.OUT_ATOL and es <= parity.STATE_RTOL


def test_wide_level_of_single_token_segments():
    """One 100-token root with 3000 children of 1-3 tokens: a level of 3000
    segments x 4 value heads, each a partial chunk starting from the root's
    state.  Both schedules agree bit for bit; sampled leaves match the
    oracle."""
    ptp = _lib()
    rng = np.random.default_rng(43)
    lens = np.concatenate([[100], rng.integers(1, 4, size=3000)]).astype(np.int32)
    parents = np.array([-1] + [0] * 3000, np.int32)
    n = int(lens.sum())
    say(f"wide level: 3000 children, N={n}")
    t = make_scan_inputs(n, 2, 4, 128, 128, "bf16", DEV, seed=44)
    plan = ptp.tree_plan(parents, lens, 4)
    o1, s1 = ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, return_states=True,
                               schedule="level")
    o2, s2 = ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, return_states=True,
                               schedule="rescan")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    segs = [1, 2, 1500, 2999, 3000]
    eo, es = parity.scan_errors_sampled(parents, lens, t["q"], t["k"], t["v"], t["g"], t["beta"], o1, s1, segs)
    say(f"  out {eo:.3e}  state {es:.3e}")
    assert eo <= parity.OUT_ATOL and es <= parity.STATE_RTOL


@pytest.mark.parametrize("case", ["no_decay", "full_forget", "mix"])
@pytest.mark.parametrize("dtype,d,h_qk,h_v", [("f32", 32, 1, 2), ("bf16", 128, 2, 4)])
def test_scan_backward_degenerate_gates(case, dtype, d, h_qk, h_v):
    """The scan backward under the degenerate gates, from given root states
    and final-state gradients: every gradient against autograd of the fp64
    token-by-token oracle, within the backward's 2e-5 bar (max-norm
    relative).  The gate gradient is measured against the larger of its own
    and the beta gradient's max-norm: both are sums over a token's row of the
    same products, and under complete forgetting the true dg vanishes (about
    1e-17 here) while the fp32 chunk sums of its terms, of dbeta's size, leave
    rounding of that size (about 6e-8)."""
    from oracle import grad as ograd
    ptp = _lib()
    parents, lens = rand_trie(51, 12, [1, 3, 16, 17, 33, 40], n_roots=2)
    n = int(lens.sum())
    say(f"scan backward, degenerate gates {case} dtype={dtype} d={d} heads={h_qk}/{h_v} N={n}")
    t = make_scan_inputs(n, h_qk, h_v, d, d, dtype, DEV, seed=52)
    t["g"], t["beta"] = _gates(case, n, h_v, 53)
    do = make_scan_inputs(n, h_qk, h_v, d, d, dtype, DEV, seed=54)["v"]
    gen = torch.Generator(device="cpu").manual_seed(55)
    init = (torch.randn(2, h_v, d, d, generator=gen) * 0.3).to(DEV)
    dst = (torch.randn(len(parents), h_v, d, d, generator=gen) * 0.1).to(DEV)
    plan = ptp.tree_plan(parents, lens, 4)
    _, states = ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, scale=0.6,
                                  return_states=True, init_states=init, schedule="level")
    got = ptp.tree_gdn_scan_backward(t["q"], t["k"], t["v"], t["g"], t["beta"], do, plan, states, scale=0.6,
                                     init_states=init, dstates=dst)
    torch.cuda.synchronize()
    f = parity.to_np
    ref = ograd.tree_gdn_vjp(parents, lens, f(t["q"]), f(t["k"]), f(t["v"]), f(t["g"]), f(t["beta"]), f(do),
                             scale=0.6, init_states=f(init), dstates=f(dst))
    names = ("dq", "dk", "dv", "dg", "dbeta", "dinit")
    errs = {}
    for nm, a, b in zip(names, got, ref):
        scale = np.abs(b).max()
        if nm == "dg":
            scale = max(scale, np.abs(ref[4]).max())
        errs[nm] = float(np.abs(f(a) - b).max() / max(scale, 1e-30))
    say("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    say(f"  max |dg| {np.abs(f(got[3])).max():.3e} (oracle {np.abs(ref[3]).max():.3e}), "
        f"max |dbeta| {np.abs(ref[4]).max():.3e}")
    assert max(errs.values()) <= 2e-5, errs


@pytest.mark.parametrize("h_qk,h_v", [(2, 4)])
def test_scan_decay_classes(h_qk, h_v):
    """The d = 128 kernel drops terms of a chunk's rows 16..31 by the largest
    gamma of those rows (lo pass of K S0 at <= 2^-10, Q S0 at <= 2^-12, all
    of K S0 at <= 2^-18).  Gates built so that chunks land on each side of
    every threshold: g = 0 except at row 16 of a chunk, where it sets
    G_16 = ln(target); so gamma is 1 on rows 0..15 and the target on rows
    16..31.  Both schedules agree bit for bit and match the oracle."""
    ptp = _lib()
    targets = [2.0 ** e for e in (-9, -10.5, -11, -12.5, -15, -18.5, -20, -30)]
    rng = np.random.default_rng(61)
    lens = np.array([32 * 6, 32 * 5 + 17, 32 * 4, 20, 32 * 3 + 31], np.int32)
    parents = np.array([-1, 0, 0, 1, 2], np.int32)
    n = int(lens.sum())
    say(f"decay classes N={n}")
    t = make_scan_inputs(n, h_qk, h_v, 128, 128, "bf16", DEV, seed=62)
    g = torch.zeros(n, h_v)
    off = np.concatenate([[0], np.cumsum(lens)])
    k = 0
    for s in range(len(lens)):
        for c0 in range(int(off[s]), int(off[s + 1]), 32):
            if c0 + 16 < off[s + 1]:
                for hh in range(h_v):
                    g[c0 + 16, hh] = float(np.log(targets[(k + hh) % len(targets)]))
                k += 1
    t["g"] = g.to(DEV).contiguous()
    plan = ptp.tree_plan(parents, lens, 4)
    gen = torch.Generator(device="cpu").manual_seed(63)
    init = (torch.randn(1, h_v, 128, 128, generator=gen) * 0.3).to(DEV)
    o1, s1 = ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, return_states=True,
                               init_states=init, schedule="level")
    o2, s2 = ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, return_states=True,
                               init_states=init, schedule="rescan")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    eo, es = parity.scan_errors_full(parents, lens, t["q"], t["k"], t["v"], t["g"], t["beta"], o1, s1,
                                     init_states=init)
    say(f"  out {eo:.3e}  state {es:.3e}")
    assert eo <= parity.OUT_ATOL and es <= parity.STATE_RTOL
