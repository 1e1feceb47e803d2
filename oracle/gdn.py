"""Oracle for the tree Gated DeltaNet forward (test infrastructure only).

Definition ("Tree Training" section 3.2 "SSM Layers (GDN)", Eq. 10: a
segment starts from the final state of its parent, a root from zero; Eq. 6:
the result equals the standalone forward of any path through the segment).
So the oracle runs the plain gated delta rule token by token over every
root-to-leaf path on its own.

Per value head h (query/key head hq = h // (H_v / H_qk)), state S [d_k, d_v]
starting at zero, and for each token t of the path in order:

    S   <- exp(g_t) * S                      (decay first)
    u   <- beta_t * (v_t - S^T k_t)          (erase what the key holds)
    S   <- S + k_t u^T                       (write)
    o_t <- S^T (scale * q_t)                 (read after the write)

which is S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t
stored transposed ([d_k, d_v], the orientation of the appendix's state
tensor).  Every segment's state after its last token is recorded.
"""
from __future__ import annotations

import numpy as np

from .trie import check_trie, leaf_paths, path_token_index, root_path, roots_of, segment_offsets


def _token_step(S, a, b, kt, vt, qt, scale):
    """One token for all heads at once.  S [H, dk, dv]; a, b [H];
    kt, qt [H, dk]; vt [H, dv].  Returns (S_new, o [H, dv])."""
    S = S * a[:, None, None]
    u = b[:, None] * (vt - np.einsum("hkv,hk->hv", S, kt))
    S = S + kt[:, :, None] * u[:, None, :]
    o = np.einsum("hkv,hk->hv", S, scale * qt)
    return S, o


def gdn_on_path(q, k, v, g, beta, scale=1.0, snap_at=(), heads=None,
                init=None, dtype=np.float64):
    """Gated delta rule over one path.

    q, k [L, H_qk, d_k]; v [L, H_v, d_v]; g, beta [L, H_v].
    heads: value heads to run (default all).  init: [len(heads), d_k, d_v]
    initial state (default zero).  Returns (o [L, len(heads), d_v],
    {pos: state after token pos for pos in snap_at}).
    """
    q = np.asarray(q, dtype=dtype)
    k = np.asarray(k, dtype=dtype)
    v = np.asarray(v, dtype=dtype)
    g = np.asarray(g, dtype=dtype)
    beta = np.asarray(beta, dtype=dtype)
    L, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    if h_v % h_qk:
        raise ValueError("value heads must be a multiple of query/key heads")
    heads = np.arange(h_v) if heads is None else np.asarray(heads, dtype=np.int64)
    hq = heads // (h_v // h_qk)
    S = (np.zeros((len(heads), d_k, d_v), dtype=dtype) if init is None
         else np.array(init, dtype=dtype, copy=True))
    o = np.zeros((L, len(heads), d_v), dtype=dtype)
    snaps = {}
    want = set(int(p) for p in snap_at)
    for t in range(L):
        S, o[t] = _token_step(S, np.exp(g[t, heads]), beta[t, heads],
                              k[t, hq], v[t, heads], q[t, hq], dtype(scale))
        if t in want:
            snaps[t] = S.copy()
    return o, snaps


def tree_gdn_reference(parents, seg_lens, q, k, v, g, beta, scale=1.0,
                       segments=None, heads=None, dtype=np.float64, init_states=None):
    """Per-path gated delta rule over the packed trie.

    Returns (o [N, H_v, d_v], states [n_seg, H_v, d_k, d_v]) in `dtype`,
    NaN where not computed.  init_states [n_roots, H_v, d_k, d_v]: the
    state each root starts from (roots in segment order; default zero; a
    partition gateway hands it across a cut, appendix B.7).  With
    segments=None every root-to-leaf path is run and a segment shared by
    several paths must come out bitwise identical from each (Eq. 6).  With
    a list of segments only the root paths of those segments are run;
    `heads` restricts the value heads.
    """
    parents, seg_lens = check_trie(parents, seg_lens)
    q = np.asarray(q)
    h_v, d_v = np.asarray(v).shape[1:]
    d_k = q.shape[2]
    n = int(np.sum(seg_lens))
    heads = np.arange(h_v) if heads is None else np.asarray(heads, dtype=np.int64)
    off = segment_offsets(seg_lens)
    rank = {r: i for i, r in enumerate(roots_of(parents))}
    o = np.full((n, h_v, d_v), np.nan, dtype=dtype)
    st = np.full((len(parents), h_v, d_k, d_v), np.nan, dtype=dtype)
    done = np.zeros(len(parents), dtype=bool)
    paths = leaf_paths(parents) if segments is None else [root_path(parents, s) for s in segments]
    for path in paths:
        idx = path_token_index(path, seg_lens)
        ends, pos = [], 0
        for s in path:
            pos += int(seg_lens[s])
            ends.append(pos - 1)
        init = None if init_states is None else np.asarray(init_states)[rank[path[0]]][heads]
        op, snaps = gdn_on_path(q[idx], k[idx], v[idx], g[idx], beta[idx], scale,
                                snap_at=ends, heads=heads, init=init, dtype=dtype)
        pos = 0
        for s, e in zip(path, ends):
            m = int(seg_lens[s])
            rows = op[pos:pos + m]
            if done[s]:
                same = (np.array_equal(o[off[s]:off[s + 1]][:, heads], rows)
                        and np.array_equal(st[s][heads], snaps[e]))
                if not same:
                    raise AssertionError(f"segment {s}: paths disagree (gdn)")
            else:
                o[off[s]:off[s + 1], heads] = rows
                st[s, heads] = snaps[e]
                done[s] = True
            pos += m
    return o, st
