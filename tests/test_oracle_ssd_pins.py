"""Pins of the Mamba2 (SSD) oracle (oracle/ssd.py) against what the
mathematics fixes independently of its token loop: the masked-matrix (dual)
form of the whole path, closed forms of special cases, and the tree
invariants of "Tree Training" section 3.1 Eq. 6; planted mistakes must fail
them."""
import numpy as np
import pytest

from oracle import ssd as ossd


def inputs(rng, L, H, G, N, P):
    x = rng.standard_normal((L, H, P))
    dt = np.log1p(np.exp(rng.standard_normal((L, H))))  # softplus: dt > 0
    A = -np.exp(rng.standard_normal(H) * 0.5)            # A < 0
    B = rng.standard_normal((L, G, N)) / np.sqrt(N)
    C = rng.standard_normal((L, G, N)) / np.sqrt(N)
    D = rng.standard_normal(H)
    return x, dt, A, B, C, D


def dual_form(x, dt, A, B, C, D, init=None):
    """y_t = sum_{s<=t} (C_t . B_s) exp(A (cum_t - cum_s)) dt_s x_s
             + exp(A cum_t) S0^T C_t + D x_t, cum_t = sum_{r<=t} dt_r:
    the whole path as one masked matrix product per head, no recurrence."""
    L, H, P = x.shape
    G = B.shape[1]
    y = np.zeros((L, H, P))
    for h in range(H):
        g = h // (H // G)
        cum = np.cumsum(dt[:, h])
        decay = np.exp(A[h] * (cum[:, None] - cum[None, :]))
        M = np.tril((C[:, g] @ B[:, g].T) * decay) * dt[None, :, h]
        y[:, h] = M @ x[:, h] + D[h] * x[:, h]
        if init is not None:
            y[:, h] += np.exp(A[h] * cum)[:, None] * (C[:, g] @ init[h])
    return y


@pytest.mark.parametrize("G", [1, 2])
def test_recurrence_equals_the_dual_form(G):
    rng = np.random.default_rng(70 + G)
    L, H, N, P = 23, 4, 5, 3
    x, dt, A, B, C, D = inputs(rng, L, H, G, N, P)
    init = rng.standard_normal((H, N, P))
    y, _ = ossd.ssd_on_path(x, dt, A, B, C, D, init=init)
    assert np.allclose(y, dual_form(x, dt, A, B, C, D, init), rtol=1e-12, atol=1e-12)


def test_single_token_closed_form():
    rng = np.random.default_rng(71)
    x, dt, A, B, C, D = inputs(rng, 1, 2, 1, 4, 3)
    y, snaps = ossd.ssd_on_path(x, dt, A, B, C, D, snap_at=[0])
    for h in range(2):
        want = dt[0, h] * float(C[0, 0] @ B[0, 0]) * x[0, h] + D[h] * x[0, h]
        assert np.allclose(y[0, h], want, rtol=1e-14)
        assert np.allclose(snaps[0][h], dt[0, h] * np.outer(B[0, 0], x[0, h]), rtol=1e-14)


def test_no_decay_is_a_cumulative_sum():
    """A = 0: S_t = sum_{s<=t} dt_s B_s x_s^T, summed with np.cumsum."""
    rng = np.random.default_rng(72)
    L, N, P = 9, 3, 2
    x, dt, _, B, C, _ = inputs(rng, L, 1, 1, N, P)
    A = np.zeros(1)
    y, _ = ossd.ssd_on_path(x, dt, A, B, C)
    terms = dt[:, 0, None, None] * B[:, 0, :, None] * x[:, 0, None, :]
    S = np.cumsum(terms, axis=0)
    assert np.allclose(y[:, 0], np.einsum("tnp,tn->tp", S, C[:, 0]), rtol=1e-12, atol=1e-12)


def test_zero_step_keeps_the_state():
    """dt = 0 (the pages' padding): the state passes through unchanged."""
    rng = np.random.default_rng(73)
    x, _, A, B, C, D = inputs(rng, 5, 2, 1, 3, 2)
    dt = np.zeros((5, 2))
    init = rng.standard_normal((2, 3, 2))
    y, snaps = ossd.ssd_on_path(x, dt, A, B, C, D, init=init, snap_at=[4])
    assert np.array_equal(snaps[4], init)
    for t in range(5):
        assert np.allclose(y[t], np.einsum("hnp,n->hp", init, C[t, 0]) + D[:, None] * x[t], rtol=1e-14)


def test_tree_invariants():
    """Branchless chain = one sequence; every path through a shared segment
    gives it the same bits; a forest is independent trees; a given root
    state is the path's initial state."""
    rng = np.random.default_rng(74)
    lens = np.array([4, 3, 5, 2], np.int32)
    n = int(lens.sum())
    x, dt, A, B, C, D = inputs(rng, n, 2, 1, 3, 2)
    chain = np.array([-1, 0, 1, 2], np.int32)
    y1, s1 = ossd.tree_ssd_reference(chain, lens, x, dt, A, B, C, D)
    y2, s2 = ossd.tree_ssd_reference(np.array([-1], np.int32), np.array([n], np.int32), x, dt, A, B, C, D)
    assert np.array_equal(y1, y2) and np.array_equal(s1[-1], s2[0])
    # a fork: segments 1 and 2 both children of 0 (tree_ssd_reference checks
    # the shared root comes out identical from both paths)
    fork = np.array([-1, 0, 0, 2], np.int32)
    yf, _ = ossd.tree_ssd_reference(fork, lens, x, dt, A, B, C, D)
    off = np.concatenate([[0], np.cumsum(lens)])
    alone, _ = ossd.ssd_on_path(np.r_[x[:4], x[off[2]:]], np.r_[dt[:4], dt[off[2]:]], A,
                                np.r_[B[:4], B[off[2]:]], np.r_[C[:4], C[off[2]:]], D)
    assert np.array_equal(yf[off[2]:], alone[4:])
    init = rng.standard_normal((1, 2, 3, 2))
    yi, _ = ossd.tree_ssd_reference(chain, lens, x, dt, A, B, C, D, init_states=init)
    yd = dual_form(x, dt, A, B, C, D, init[0])
    assert np.allclose(yi, yd, rtol=1e-12, atol=1e-12)


def test_planted_oracle_mistakes_are_caught(monkeypatch):
    """Decay applied after the write, or the step missing from the input,
    or the wrong group for a head, must fail the dual-form pin."""
    orig = ossd.ssd_on_path

    def decay_after(x, dt, A, B, C, D=None, heads=None, init=None, snap_at=(), dtype=np.float64):
        x, dt, A, B, C = (np.asarray(a, dtype) for a in (x, dt, A, B, C))
        L, H, P = x.shape
        G, N = B.shape[1], B.shape[2]
        S = np.zeros((H, N, P)) if init is None else np.array(init, dtype)
        y = np.zeros((L, H, P))
        for t in range(L):
            grp = np.arange(H) // (H // G)
            S = S + dt[t][:, None, None] * B[t, grp][:, :, None] * x[t][:, None, :]
            S = np.exp(dt[t] * A)[:, None, None] * S
            y[t] = np.einsum("hnp,hn->hp", S, C[t, grp]) + (0 if D is None else np.asarray(D)[:, None] * x[t])
        return y, {}

    def no_step(x, dt, A, B, C, D=None, heads=None, init=None, snap_at=(), dtype=np.float64):
        x, dt, A, B, C = (np.asarray(a, dtype) for a in (x, dt, A, B, C))
        L, H, P = x.shape
        G, N = B.shape[1], B.shape[2]
        grp = np.arange(H) // (H // G)
        S = np.zeros((H, N, P)) if init is None else np.array(init, dtype)
        y = np.zeros((L, H, P))
        for t in range(L):
            S = np.exp(dt[t] * A)[:, None, None] * S + B[t, grp][:, :, None] * x[t][:, None, :]
            y[t] = np.einsum("hnp,hn->hp", S, C[t, grp]) + (0 if D is None else np.asarray(D)[:, None] * x[t])
        return y, {}

    def wrong_group(x, dt, A, B, C, D=None, **kw):
        return orig(x, dt, A, np.asarray(B)[:, ::-1], C, D, **kw)

    for bad in (decay_after, no_step, wrong_group):
        monkeypatch.setattr(ossd, "ssd_on_path", bad)
        with pytest.raises(AssertionError):
            test_recurrence_equals_the_dual_form(2)
        monkeypatch.setattr(ossd, "ssd_on_path", orig)
