"""Pins of the backward oracle (oracle/grad.py): every gradient against
central finite differences of the NumPy forward oracle (oracle/conv.py,
oracle/gdn.py), which shares no code with it, on small forests with given
root contexts and states; and invariances of the tree structure."""
import numpy as np
import pytest

from oracle import conv as oconv
from oracle import gdn as ogdn
from oracle import grad as ograd

EPS = 1e-6


def forest(rng, n_seg, max_len, n_roots):
    parents = [-1] * n_roots + [int(rng.integers(0, i)) for i in range(n_roots, n_seg)]
    return np.array(parents, np.int32), rng.integers(1, max_len + 1, n_seg).astype(np.int32)


def fd_check(loss, arr, grad, rng, n_pick=10, rtol=1e-6):
    """Central differences of `loss` at n_pick random entries of `arr`."""
    flat = arr.reshape(-1)
    for i in rng.choice(flat.size, size=min(n_pick, flat.size), replace=False):
        keep = flat[i]
        flat[i] = keep + EPS
        lp = loss()
        flat[i] = keep - EPS
        lm = loss()
        flat[i] = keep
        fd = (lp - lm) / (2 * EPS)
        g = grad.reshape(-1)[i]
        assert abs(fd - g) <= rtol * max(1.0, abs(g)), (i, fd, g)


@pytest.mark.parametrize("W,act,with_bias", [(4, None, False), (4, "silu", True), (2, "silu", False), (1, None, True)])
def test_conv_gradients_are_finite_differences_of_the_forward(W, act, with_bias):
    rng = np.random.default_rng(40 + W)
    parents, lens = forest(rng, 9, 4, n_roots=2)  # short segments: windows reach grandparents and contexts
    n, C = int(lens.sum()), 3
    x = rng.standard_normal((n, C))
    w = rng.standard_normal((C, W))
    b = rng.standard_normal(C) if with_bias else None
    ctx = rng.standard_normal((2, W - 1, C))
    dy = rng.standard_normal((n, C))
    dx, dw, db, dctx = ograd.tree_conv_vjp(parents, lens, x, w, dy, bias=b, act=act, init_ctx=ctx)

    def loss():
        return float((oconv.tree_conv_reference(parents, lens, x, w, b, act, init_ctx=ctx) * dy).sum())

    fd_check(loss, x, dx, rng)
    fd_check(loss, w, dw, rng)
    if with_bias:
        fd_check(loss, b, db, rng)
    if W > 1:
        fd_check(loss, ctx, dctx, rng)


def test_gdn_gradients_are_finite_differences_of_the_forward():
    rng = np.random.default_rng(50)
    parents, lens = forest(rng, 7, 5, n_roots=2)
    n, h_qk, h_v, dk, dv = int(lens.sum()), 1, 2, 3, 4
    q = rng.standard_normal((n, h_qk, dk)) * 0.5
    k = rng.standard_normal((n, h_qk, dk)) * 0.5
    v = rng.standard_normal((n, h_v, dv))
    g = -np.log1p(np.exp(rng.standard_normal((n, h_v))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((n, h_v))))
    init = rng.standard_normal((2, h_v, dk, dv)) * 0.3
    do = rng.standard_normal((n, h_v, dv))
    dstates = rng.standard_normal((len(parents), h_v, dk, dv))
    grads = ograd.tree_gdn_vjp(parents, lens, q, k, v, g, beta, do, scale=0.7, init_states=init, dstates=dstates)

    def loss():
        o, st = ogdn.tree_gdn_reference(parents, lens, q, k, v, g, beta, 0.7, init_states=init)
        return float((o * do).sum() + (st * dstates).sum())

    for arr, gr in zip((q, k, v, g, beta, init), grads):
        fd_check(loss, arr, gr, rng, n_pick=8)


def test_split_chain_gradients_equal_one_segment():
    """Cutting a sequence into a parent-child chain changes nothing."""
    rng = np.random.default_rng(51)
    lens = np.array([3, 1, 4, 2], np.int32)
    n = int(lens.sum())
    chain = np.array([-1, 0, 1, 2], np.int32)
    one_p, one_l = np.array([-1], np.int32), np.array([n], np.int32)
    x, w, dy = rng.standard_normal((n, 2)), rng.standard_normal((2, 4)), rng.standard_normal((n, 2))
    a = ograd.tree_conv_vjp(chain, lens, x, w, dy, act="silu")
    b = ograd.tree_conv_vjp(one_p, one_l, x, w, dy, act="silu")
    for u, z in zip(a, b):
        if u is not None:
            assert np.allclose(u, z, rtol=1e-12, atol=1e-12)
    q, k = rng.standard_normal((n, 1, 3)), rng.standard_normal((n, 1, 3))
    v, do = rng.standard_normal((n, 1, 3)), rng.standard_normal((n, 1, 3))
    g, beta = -np.abs(rng.standard_normal((n, 1))), rng.uniform(0.1, 0.9, (n, 1))
    ga = ograd.tree_gdn_vjp(chain, lens, q, k, v, g, beta, do)
    gb = ograd.tree_gdn_vjp(one_p, one_l, q, k, v, g, beta, do)
    for u, z in zip(ga[:5], gb[:5]):
        assert np.allclose(u, z, rtol=1e-12, atol=1e-12)


def test_sibling_gradients_add_up_in_the_parent():
    """Two identical children with the same upstream gradients give the
    parent's inputs exactly the gradient of one child doubled (plus the
    parent's own outputs' part): the parent state and context receive the
    sum over children."""
    rng = np.random.default_rng(52)
    lens_one = np.array([4, 3], np.int32)
    lens_two = np.array([4, 3, 3], np.int32)
    par_one, par_two = np.array([-1, 0], np.int32), np.array([-1, 0, 0], np.int32)
    C, W = 2, 4
    xp, xc = rng.standard_normal((4, C)), rng.standard_normal((3, C))
    dyp, dyc = rng.standard_normal((4, C)), rng.standard_normal((3, C))
    w = rng.standard_normal((C, W))
    g1 = ograd.tree_conv_vjp(par_one, lens_one, np.r_[xp, xc], w, np.r_[dyp, dyc])
    g0 = ograd.tree_conv_vjp(par_one, lens_one, np.r_[xp, xc], w, np.r_[dyp, 0 * dyc])
    g2 = ograd.tree_conv_vjp(par_two, lens_two, np.r_[xp, xc, xc], w, np.r_[dyp, dyc, dyc])
    # parent rows: own part + 2 x (child part)
    assert np.allclose(g2[0][:4], g0[0][:4] + 2 * (g1[0][:4] - g0[0][:4]), rtol=1e-12, atol=1e-12)


def test_planted_grad_oracle_mistakes_are_caught(monkeypatch):
    """A conv window off by one token, or the roots' initial states swapped,
    must fail the finite-difference pins."""
    orig_rows = ograd._window_rows

    def shifted(parents, seg_lens, width):
        r = orig_rows(parents, seg_lens, width)
        r[:, :-1] = r[:, 1:]  # every window one token too new
        return r

    monkeypatch.setattr(ograd, "_window_rows", shifted)
    with pytest.raises(AssertionError):
        test_conv_gradients_are_finite_differences_of_the_forward(4, None, False)
    monkeypatch.setattr(ograd, "_window_rows", orig_rows)
    monkeypatch.setattr(ograd, "roots_of", lambda parents: list(reversed([i for i, p in enumerate(parents) if p < 0])))
    with pytest.raises(AssertionError):
        test_gdn_gradients_are_finite_differences_of_the_forward()
