"""Pins for the CPU oracle, against things other than the oracle itself.

Each test names what fixes the expected value: a library routine, a closed
form of the recurrence, an invariant that the per-path definition implies,
an independent brute force, the chunked (WY/UT) form of the method, or the
number the pages print.  CPU only.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import conv as oconv
from oracle import gdn as ogdn
from oracle import trie as otrie
from oracle.brute import _prev_token_fn, conv_brute, gdn_brute
from tests import parity

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_trie(rng, n_seg, max_len, n_roots=1):
    parents = [-1] * n_roots
    for i in range(n_roots, n_seg):
        parents.append(int(rng.integers(0, i)))
    lens = rng.integers(1, max_len + 1, size=n_seg).tolist()
    return np.array(parents, np.int32), np.array(lens, np.int32)


def scan_inputs(rng, n, h_qk, h_v, d_k, d_v, gscale=1.0):
    q = rng.standard_normal((n, h_qk, d_k))
    k = rng.standard_normal((n, h_qk, d_k))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((n, h_v, d_v))
    g = -np.log1p(np.exp(rng.standard_normal((n, h_v)))) * gscale
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((n, h_v))))
    return q, k, v, g, beta


# --------------------------------------------------------------------- conv

@pytest.mark.parametrize("act", [None, "silu"])
@pytest.mark.parametrize("W", [2, 4])
def test_conv_chain_matches_torch_conv1d(act, W):
    """A branchless trie is one sequence: the tree conv must equal the library
    depthwise conv1d (left padding W-1, trailing outputs dropped)."""
    rng = np.random.default_rng(1)
    lens = np.array([7, 1, 3, 12], np.int32)          # a chain of 4 segments
    parents = np.array([-1, 0, 1, 2], np.int32)
    n, C = int(lens.sum()), 5
    x = rng.standard_normal((n, C))
    w = rng.standard_normal((C, W))
    b = rng.standard_normal(C)
    y = oconv.tree_conv_reference(parents, lens, x, w, bias=b, act=act)
    xt = torch.from_numpy(x.T[None].copy())
    ref = torch.nn.functional.conv1d(xt, torch.from_numpy(w[:, None, :].copy()),
                                     torch.from_numpy(b), padding=W - 1, groups=C)[0, :, :n].T
    if act == "silu":
        ref = torch.nn.functional.silu(ref)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_conv_onehot_reads_path_history_bitwise():
    """With w[:, W-1-s] = 1 and all other taps 0, y[t] is exactly the input s
    steps back along t's own path (zero before the root), across segment
    starts, ancestors shorter than W-1 and several roots."""
    rng = np.random.default_rng(2)
    parents, lens = rand_trie(rng, 40, 3, n_roots=3)
    n, C, W = int(lens.sum()), 3, 4
    x = rng.standard_normal((n, C))
    prev, _, _ = _prev_token_fn(parents, lens)
    for s in range(W):
        w = np.zeros((C, W))
        w[:, W - 1 - s] = 1.0
        y = oconv.tree_conv_reference(parents, lens, x, w)
        for t in range(n):
            j = t
            for _ in range(s):
                j = None if j is None else prev(j)
            expect = np.zeros(C) if j is None else x[j]
            assert np.array_equal(y[t], expect), (s, t)


@pytest.mark.parametrize("act", [None, "silu"])
def test_conv_tree_matches_brute_force(act):
    rng = np.random.default_rng(3)
    parents, lens = rand_trie(rng, 30, 6, n_roots=2)
    n, C, W = int(lens.sum()), 4, 4
    x = rng.standard_normal((n, C))
    w = rng.standard_normal((C, W))
    b = rng.standard_normal(C)
    y = oconv.tree_conv_reference(parents, lens, x, w, bias=b, act=act)
    np.testing.assert_allclose(y, conv_brute(parents, lens, x, w, b, act), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------- gdn

@pytest.mark.parametrize("h_qk,h_v,d_k,d_v", [(1, 1, 5, 3), (2, 4, 4, 6)])
def test_gdn_tree_matches_matrix_form_brute_force(h_qk, h_v, d_k, d_v):
    """d_k != d_v so that a transposed state or operand cannot pass."""
    rng = np.random.default_rng(4)
    parents, lens = rand_trie(rng, 12, 5, n_roots=2)
    q, k, v, g, beta = scan_inputs(rng, int(lens.sum()), h_qk, h_v, d_k, d_v)
    o, st = ogdn.tree_gdn_reference(parents, lens, q, k, v, g, beta, scale=0.7)
    ob, sb = gdn_brute(parents, lens, q, k, v, g, beta, scale=0.7)
    np.testing.assert_allclose(o, ob, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(st, sb, rtol=1e-11, atol=1e-12)


def test_gdn_closed_form_orthonormal_keys():
    """Distinct standard-basis keys never overlap, so the erase term vanishes
    and M_t = sum_{j<=t} (gamma_t / gamma_j) b_j v_j k_j^T."""
    rng = np.random.default_rng(5)
    L, d_k, d_v = 9, 9, 4
    k = np.eye(d_k)[rng.permutation(d_k)][:, None, :]
    q = rng.standard_normal((L, 1, d_k))
    v = rng.standard_normal((L, 1, d_v))
    g = -rng.random((L, 1))
    b = rng.random((L, 1))
    o, snaps = ogdn.gdn_on_path(q, k, v, g, b, snap_at=[L - 1])
    G = np.cumsum(g[:, 0])
    for t in range(L):
        M = sum(np.exp(G[t] - G[j]) * b[j, 0] * np.outer(v[j, 0], k[j, 0]) for j in range(t + 1))
        np.testing.assert_allclose(o[t, 0], M @ q[t, 0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(snaps[L - 1][0], M.T, rtol=1e-13, atol=1e-14)


def test_gdn_beta_zero_gives_zero():
    rng = np.random.default_rng(6)
    q, k, v, g, beta = scan_inputs(rng, 20, 1, 2, 4, 4)
    o, snaps = ogdn.gdn_on_path(q, k, v, g, np.zeros_like(beta), snap_at=[19])
    assert np.all(o == 0) and np.all(snaps[19] == 0)


def test_gdn_single_token():
    """One token from a zero state: o = scale * b (k . q) v."""
    rng = np.random.default_rng(7)
    q, k, v, g, beta = scan_inputs(rng, 1, 1, 1, 6, 5)
    o, _ = ogdn.gdn_on_path(q, k, v, g, beta, scale=0.5)
    np.testing.assert_allclose(o[0, 0], 0.5 * beta[0, 0] * (k[0, 0] @ q[0, 0]) * v[0, 0], rtol=1e-14)


def test_gdn_no_decay_full_erase_copies_values():
    """g = 0, beta = 1, q = k = e_1: the state holds only the latest value,
    so o_t = v_t up to fp64 rounding of v_{t-1} + (v_t - v_{t-1}) (read after
    the write, erase before the write)."""
    rng = np.random.default_rng(8)
    L, d = 15, 4
    e = np.zeros((L, 1, d))
    e[:, 0, 0] = 1.0
    v = rng.standard_normal((L, 1, 3))
    o, _ = ogdn.gdn_on_path(e, e, v, np.zeros((L, 1)), np.ones((L, 1)))
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-14)


def test_gdn_scalar_closed_form():
    """d_k = d_v = 1: s_t = a_t (1 - b_t k_t^2) s_{t-1} + b_t k_t v_t is a
    scalar linear recurrence with s_t = sum_j prod_{i>j} c_i * b_j k_j v_j."""
    rng = np.random.default_rng(9)
    L = 12
    k = rng.uniform(-1, 1, (L, 1, 1))
    q = rng.uniform(-1, 1, (L, 1, 1))
    v = rng.standard_normal((L, 1, 1))
    g = -rng.random((L, 1))
    b = rng.random((L, 1))
    o, _ = ogdn.gdn_on_path(q, k, v, g, b)
    c = np.exp(g[:, 0]) * (1 - b[:, 0] * k[:, 0, 0] ** 2)
    for t in range(L):
        s = sum(np.prod(c[j + 1:t + 1]) * b[j, 0] * k[j, 0, 0] * v[j, 0, 0] for j in range(t + 1))
        np.testing.assert_allclose(o[t, 0, 0], s * q[t, 0, 0], rtol=1e-12, atol=1e-14)


def chunk_form(parents, lens, q, k, v, g, beta, scale=1.0):
    """The method's chunked algebra with one chunk per segment, written from
    the "Tree Training" appendix A.2 equations (WY/UT transform, parent-state
    routing of Eq. 10), in fp64 with an exact triangular solve.  Per chunk
    with start state S0 and G = cumsum(g):
        (I + A) U = diag(b) V - diag(b*gamma) K S0,  A_ij = b_i e^{G_i-G_j} k_i.k_j (j<i)
        O = scale*(diag(gamma) Q S0 + ((Q K^T) o Gamma_incl) U)
        S_end = gamma_L S0 + (diag(gamma_L/gamma) K)^T U"""
    off = otrie.segment_offsets(lens)
    h_qk, d_k = q.shape[1], q.shape[2]
    h_v, d_v = v.shape[1], v.shape[2]
    grp = h_v // h_qk
    o = np.zeros(v.shape)
    st = np.zeros((len(lens), h_v, d_k, d_v))
    for s in range(len(lens)):
        a, e = off[s], off[s + 1]
        for h in range(h_v):
            S0 = st[parents[s], h] if parents[s] >= 0 else np.zeros((d_k, d_v))
            K, Q, V = k[a:e, h // grp], q[a:e, h // grp], v[a:e, h]
            G = np.cumsum(g[a:e, h])
            b = beta[a:e, h]
            gam = np.exp(G)
            Gam = np.tril(np.exp(np.tril(G[:, None] - G[None, :])))
            A = np.tril(b[:, None] * (K @ K.T) * Gam, -1)
            U = np.linalg.solve(np.eye(e - a) + A, b[:, None] * V - (b * gam)[:, None] * (K @ S0))
            o[a:e, h] = scale * (gam[:, None] * (Q @ S0) + ((Q @ K.T) * Gam) @ U)
            st[s, h] = gam[-1] * S0 + (np.exp(G[-1] - G)[:, None] * K).T @ U
    return o, st


def test_gdn_oracle_matches_chunked_form_of_the_method():
    """Pins the readings "output after the write" and "decay before the
    erase" to the pages' chunk algebra (which keeps the diagonal in the
    output mask and applies the cumulative decay to the erase term)."""
    rng = np.random.default_rng(10)
    parents, lens = rand_trie(rng, 10, 24, n_roots=2)
    q, k, v, g, beta = scan_inputs(rng, int(lens.sum()), 2, 4, 8, 6)
    o, st = ogdn.tree_gdn_reference(parents, lens, q, k, v, g, beta, scale=1.3)
    oc, sc = chunk_form(parents, lens, q, k, v, g, beta, scale=1.3)
    np.testing.assert_allclose(o, oc, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(st, sc, rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------- tree invariants

def test_branchless_trie_equals_plain_sequence_bitwise():
    rng = np.random.default_rng(11)
    lens = np.array([5, 9, 1, 7], np.int32)
    n = int(lens.sum())
    q, k, v, g, beta = scan_inputs(rng, n, 1, 2, 4, 4)
    x = rng.standard_normal((n, 3))
    w = rng.standard_normal((3, 4))
    chain = np.array([-1, 0, 1, 2], np.int32)
    one = (np.array([-1], np.int32), np.array([n], np.int32))
    o1, s1 = ogdn.tree_gdn_reference(chain, lens, q, k, v, g, beta)
    o2, s2 = ogdn.tree_gdn_reference(*one, q, k, v, g, beta)
    assert np.array_equal(o1, o2) and np.array_equal(s1[-1], s2[0])
    assert np.array_equal(oconv.tree_conv_reference(chain, lens, x, w),
                          oconv.tree_conv_reference(*one, x, w))


def test_forest_equals_independent_calls_bitwise():
    rng = np.random.default_rng(12)
    pa, la = rand_trie(rng, 6, 5)
    pb, lb = rand_trie(rng, 5, 5)
    na, nb = int(la.sum()), int(lb.sum())
    q, k, v, g, beta = scan_inputs(rng, na + nb, 1, 1, 4, 3)
    parents = np.concatenate([pa, np.where(pb >= 0, pb + len(pa), -1)]).astype(np.int32)
    lens = np.concatenate([la, lb])
    o, st = ogdn.tree_gdn_reference(parents, lens, q, k, v, g, beta)
    oa, sa = ogdn.tree_gdn_reference(pa, la, q[:na], k[:na], v[:na], g[:na], beta[:na])
    ob, sb = ogdn.tree_gdn_reference(pb, lb, q[na:], k[na:], v[na:], g[na:], beta[na:])
    assert np.array_equal(o, np.concatenate([oa, ob]))
    assert np.array_equal(st, np.concatenate([sa, sb]))


def test_sibling_order_and_duplicate_subtrees():
    """Permuting sibling subtrees permutes the outputs; identical sibling
    subtrees on identical inputs give identical outputs (bitwise)."""
    rng = np.random.default_rng(13)
    # root(4) with children A(3) and B(5); A has child A1(2).
    q, k, v, g, beta = scan_inputs(rng, 14, 1, 1, 4, 4)
    x = rng.standard_normal((14, 2))
    w = rng.standard_normal((2, 4))
    p1, l1 = np.array([-1, 0, 1, 0], np.int32), np.array([4, 3, 2, 5], np.int32)
    # same trie with B first: root, B, A, A1
    perm = np.r_[0:4, 9:14, 4:9]
    p2, l2 = np.array([-1, 0, 0, 2], np.int32), np.array([4, 5, 3, 2], np.int32)
    o1, s1 = ogdn.tree_gdn_reference(p1, l1, q, k, v, g, beta)
    o2, s2 = ogdn.tree_gdn_reference(p2, l2, q[perm], k[perm], v[perm], g[perm], beta[perm])
    assert np.array_equal(o1[perm], o2)
    assert np.array_equal(s1[[0, 3, 1, 2]], s2)
    y1 = oconv.tree_conv_reference(p1, l1, x, w)
    y2 = oconv.tree_conv_reference(p2, l2, x[perm], w)
    assert np.array_equal(y1[perm], y2)
    # duplicate: root(4) with two identical children of 6 tokens.
    pd, ld = np.array([-1, 0, 0], np.int32), np.array([4, 6, 6], np.int32)
    idx = np.r_[0:10, 4:10]
    od, sd = ogdn.tree_gdn_reference(pd, ld, q[idx], k[idx], v[idx], g[idx], beta[idx])
    assert np.array_equal(od[4:10], od[10:16]) and np.array_equal(sd[1], sd[2])


def test_every_path_through_a_segment_agrees():
    """The oracle runs every root-to-leaf path and raises if two paths give a
    shared segment different results; a tree with many leaves must pass and
    every row and state must be filled."""
    rng = np.random.default_rng(14)
    parents, lens = rand_trie(rng, 25, 4)
    n = int(lens.sum())
    q, k, v, g, beta = scan_inputs(rng, n, 1, 1, 3, 3)
    o, st = ogdn.tree_gdn_reference(parents, lens, q, k, v, g, beta)
    assert not np.isnan(o).any() and not np.isnan(st).any()
    y = oconv.tree_conv_reference(parents, lens, rng.standard_normal((n, 2)), rng.standard_normal((2, 4)))
    assert not np.isnan(y).any()


def test_segment_subset_matches_full_run():
    rng = np.random.default_rng(15)
    parents, lens = rand_trie(rng, 15, 6)
    n = int(lens.sum())
    q, k, v, g, beta = scan_inputs(rng, n, 2, 4, 4, 4)
    o, st = ogdn.tree_gdn_reference(parents, lens, q, k, v, g, beta)
    seg = [7, 11]
    os_, ss = ogdn.tree_gdn_reference(parents, lens, q, k, v, g, beta, segments=seg, heads=[1, 3])
    off = otrie.segment_offsets(lens)
    for s in seg:
        assert np.array_equal(os_[off[s]:off[s + 1]][:, [1, 3]], o[off[s]:off[s + 1]][:, [1, 3]])
        assert np.array_equal(ss[s][[1, 3]], st[s][[1, 3]])


# ------------------------------------------------------------------ the POR

def test_por_matches_printed_example():
    gold = json.load(open(os.path.join(GOLDEN, "por_example.json")))
    # root of 81k tokens with two 1k children: 83k in the trie, 164k repeated.
    parents = np.array([-1, 0, 0], np.int32)
    lens = np.array([81000, 1000, 1000], np.int32)
    assert int(lens.sum()) == gold["n_tree"]
    assert otrie.path_token_count(parents, lens) == gold["n_base"]
    assert round(100 * otrie.por(parents, lens), 1) == gold["por_percent_rounded"]


def test_bad_tries_rejected():
    for parents, lens in (([-1, 1], [1, 1]), ([-1, 0], [1, 0]), ([0], [1]), ([-1, 5], [1, 1])):
        with pytest.raises(ValueError):
            otrie.check_trie(np.array(parents), np.array(lens))


def test_oracle_on_tiny_workload_every_path():
    """The tiny workload through the shared generator: every path is run,
    shared segments agree bitwise, and the chain-of-one-path view of a leaf
    gives the same rows as the tree run."""
    from workloads import make_workload
    wl = make_workload(1, device="cpu")
    t = {k: v.double().numpy() for k, v in wl.tensors.items()}
    o, st = ogdn.tree_gdn_reference(wl.parents, wl.seg_lens, t["q"], t["k"], t["v"], t["g"], t["beta"])
    y = oconv.tree_conv_reference(wl.parents, wl.seg_lens, t["x"], t["w"])
    assert not np.isnan(o).any() and not np.isnan(st).any() and not np.isnan(y).any()
    # leaf 3's path is segments 0, 1, 3: run it as one plain sequence.
    idx = otrie.path_token_index([0, 1, 3], wl.seg_lens)
    op, snaps = ogdn.gdn_on_path(t["q"][idx], t["k"][idx], t["v"][idx], t["g"][idx], t["beta"][idx],
                                 snap_at=[len(idx) - 1])
    off = otrie.segment_offsets(wl.seg_lens)
    assert np.array_equal(op[-16:], o[off[3]:off[4]]) and np.array_equal(snaps[len(idx) - 1], st[3])
    assert round(otrie.por(wl.parents, wl.seg_lens), 4) == round(1 - 192 / 448, 4)


# ------------------------------------------------------- partition gateways

def test_conv_root_context_is_the_eq11_concatenation():
    """Eq. 11, y = Conv([ctx; x])[W-1:]: a root's given context computed by
    prepending it to the path and dropping the first W-1 outputs; in a
    forest, root r reads context r (roots in segment order)."""
    rng = np.random.default_rng(21)
    for W in (2, 4):
        x = rng.standard_normal((9, 5))
        w = rng.standard_normal((5, W))
        ctx = rng.standard_normal((W - 1, 5))
        assert np.array_equal(oconv.conv_on_path(x, w, ctx=ctx),
                              oconv.conv_on_path(np.concatenate([ctx, x]), w)[W - 1:])
        parents, lens = np.array([-1, 0, -1, 2]), np.array([3, 2, 4, 1])
        xs = rng.standard_normal((10, 5))
        init = rng.standard_normal((2, W - 1, 5))
        y = oconv.tree_conv_reference(parents, lens, xs, w, init_ctx=init)
        assert np.array_equal(y[:5], oconv.conv_on_path(np.concatenate([init[0], xs[:5]]), w)[W - 1:])
        assert np.array_equal(y[5:], oconv.conv_on_path(np.concatenate([init[1], xs[5:]]), w)[W - 1:])


def test_conv_context_out_is_the_path_walk():
    """The W-1 inputs ending at a segment's last token, by walking the path
    token by token and, past the root, into its given context (newest
    first)."""
    rng = np.random.default_rng(22)
    W, C = 4, 3
    parents, lens = rand_trie(rng, 12, 3, n_roots=2)
    n = int(lens.sum())
    x = rng.standard_normal((n, C))
    init = rng.standard_normal((2, W - 1, C))
    got = oconv.conv_context_reference(parents, lens, x, W, init_ctx=init)
    prev, _, start = _prev_token_fn(parents, lens)
    roots = [s for s in range(len(parents)) if parents[s] < 0]
    for s in range(len(parents)):
        root = s
        while parents[root] >= 0:
            root = parents[root]
        j, m = start[s] + int(lens[s]) - 1, 0
        for back in range(W - 1):  # row W-2-back is `back` steps before the last token
            if back > 0 and j is not None:
                j = prev(j)
            if j is None:
                m += 1
                want = init[roots.index(root)][W - 1 - m]
            else:
                want = x[j]
            assert np.array_equal(got[s, W - 2 - back], want), (s, back)


def test_partition_gateway_reproduces_the_uncut_trie():
    """Section 3.3 / appendix B.7: cutting a subtree off into its own
    partition, whose root starts from the parent's final state and conv
    context, reproduces the uncut trie bitwise (conv and recurrence)."""
    rng = np.random.default_rng(23)
    W, C = 4, 4
    parents, lens = rand_trie(rng, 14, 4, n_roots=1)
    n = int(lens.sum())
    off = otrie.segment_offsets(lens)
    x = rng.standard_normal((n, C))
    wts = rng.standard_normal((C, W))
    q, k, v, g, beta = scan_inputs(rng, n, 1, 2, 3, 4)
    yF = oconv.tree_conv_reference(parents, lens, x, wts)
    oF, sF = ogdn.tree_gdn_reference(parents, lens, q, k, v, g, beta)
    for c in [s for s in range(1, len(parents)) if parents[s] >= 0][:4]:
        keep, pa, ia, subl, pb, ib = parity.split_subtree(parents, c)
        rows = lambda segs: np.concatenate([np.arange(off[s], off[s + 1]) for s in segs])
        ra, rb = rows(keep), rows(subl)
        la, lb = lens[keep], lens[subl]
        ctxA = oconv.conv_context_reference(pa, la, x[ra], W)
        oA, sA = ogdn.tree_gdn_reference(pa, la, q[ra], k[ra], v[ra], g[ra], beta[ra])
        par = ia[int(parents[c])]
        yB = oconv.tree_conv_reference(pb, lb, x[rb], wts, init_ctx=ctxA[par][None])
        oB, sB = ogdn.tree_gdn_reference(pb, lb, q[rb], k[rb], v[rb], g[rb], beta[rb], init_states=sA[par][None])
        assert np.array_equal(yB, yF[rb]) and np.array_equal(oB, oF[rb])
        assert np.array_equal(sB, sF[subl])
        assert np.array_equal(oA, oF[ra]) and np.array_equal(sA, sF[keep])
