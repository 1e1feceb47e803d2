"""Oracle for the tree Mamba2 (SSD) forward with a forked state (test
infrastructure only).

Definition.  The tree-recurrence 0.1.0 project page lists forking the Mamba2
state as work not yet done ("Not yet": per-depth batches that start from
initial states, padded with a step dt of zero after its softplus so that
padding leaves the state alone); its "How a tree runs" section gives the
fork rule the GDN scan already follows: a segment starts from its parent's
final state.  "Tree Training" section 3.1 Eq. 6 fixes what the fork must
reproduce: the standalone forward of any root-to-leaf path through a
segment.  The pages do not write the Mamba2 recurrence out; the reading
taken is the selective state-space recurrence of the Mamba2 (SSD) layer,
per head h with scalar decay rate A_h < 0, step dt_t >= 0 (after softplus),
input x_t [P], and B_t, C_t [N] of the head's group (head h uses group
h // (H / G)):

    S_t = exp(dt_t A_h) S_{t-1} + dt_t B_t x_t^T      (S [N, P])
    y_t = S_t^T C_t + D_h x_t

So the oracle runs this recurrence token by token over every root-to-leaf
path on its own, each root from zero (or a given initial state), and records
every segment's state after its last token.
"""
from __future__ import annotations

import numpy as np

from .trie import check_trie, leaf_paths, path_token_index, root_path, roots_of, segment_offsets


def ssd_on_path(x, dt, A, B, C, D=None, heads=None, init=None, snap_at=(), dtype=np.float64):
    """Mamba2 recurrence over one path.

    x [L, H, P]; dt [L, H]; A [H]; B, C [L, G, N]; D [H] or None.
    heads: heads to run (default all).  init: [len(heads), N, P] initial
    state (default zero).  Returns (y [L, len(heads), P], {pos: state after
    token pos for pos in snap_at}).
    """
    x = np.asarray(x, dtype=dtype)
    dt = np.asarray(dt, dtype=dtype)
    A = np.asarray(A, dtype=dtype)
    B = np.asarray(B, dtype=dtype)
    C = np.asarray(C, dtype=dtype)
    L, n_heads, p = x.shape
    n_groups, n = B.shape[1], B.shape[2]
    if n_heads % n_groups:
        raise ValueError("heads must be a multiple of groups")
    heads = np.arange(n_heads) if heads is None else np.asarray(heads, dtype=np.int64)
    grp = heads // (n_heads // n_groups)
    Dh = np.zeros(len(heads), dtype=dtype) if D is None else np.asarray(D, dtype=dtype)[heads]
    S = np.zeros((len(heads), n, p), dtype=dtype) if init is None else np.array(init, dtype=dtype, copy=True)
    y = np.zeros((L, len(heads), p), dtype=dtype)
    snaps = {}
    want = set(int(s) for s in snap_at)
    for t in range(L):
        a = np.exp(dt[t, heads] * A[heads])                      # decay first
        S = a[:, None, None] * S + (dt[t, heads][:, None, None] * B[t, grp][:, :, None] * x[t, heads][:, None, :])
        y[t] = np.einsum("hnp,hn->hp", S, C[t, grp]) + Dh[:, None] * x[t, heads]  # read after the write
        if t in want:
            snaps[t] = S.copy()
    return y, snaps


def tree_ssd_reference(parents, seg_lens, x, dt, A, B, C, D=None, segments=None, heads=None,
                       init_states=None, dtype=np.float64):
    """Per-path Mamba2 recurrence over the packed trie.

    Returns (y [N, H, P], states [n_seg, H, N_state, P]) in `dtype`, NaN where
    not computed.  init_states [n_roots, H, N_state, P]: the state each root
    starts from (roots in segment order; default zero).  With segments=None
    every root-to-leaf path is run and a segment shared by several paths must
    come out bitwise identical from each (Eq. 6); otherwise only the root
    paths of the given segments.  `heads` restricts the heads.
    """
    parents, seg_lens = check_trie(parents, seg_lens)
    x = np.asarray(x)
    n_heads, p = x.shape[1], x.shape[2]
    n_state = np.asarray(B).shape[2]
    ntok = int(np.sum(seg_lens))
    heads = np.arange(n_heads) if heads is None else np.asarray(heads, dtype=np.int64)
    off = segment_offsets(seg_lens)
    rank = {r: i for i, r in enumerate(roots_of(parents))}
    y = np.full((ntok, n_heads, p), np.nan, dtype=dtype)
    st = np.full((len(parents), n_heads, n_state, p), np.nan, dtype=dtype)
    done = np.zeros(len(parents), dtype=bool)
    paths = leaf_paths(parents) if segments is None else [root_path(parents, s) for s in segments]
    dt = np.asarray(dt)
    B, C = np.asarray(B), np.asarray(C)
    for path in paths:
        idx = path_token_index(path, seg_lens)
        ends, pos = [], 0
        for s in path:
            pos += int(seg_lens[s])
            ends.append(pos - 1)
        init = None if init_states is None else np.asarray(init_states)[rank[path[0]]][heads]
        yp, snaps = ssd_on_path(x[idx], dt[idx], A, B[idx], C[idx], D, heads=heads, init=init,
                                snap_at=ends, dtype=dtype)
        pos = 0
        for s, e in zip(path, ends):
            m = int(seg_lens[s])
            rows = yp[pos:pos + m]
            if done[s]:
                same = (np.array_equal(y[off[s]:off[s + 1]][:, heads], rows)
                        and np.array_equal(st[s][heads], snaps[e]))
                if not same:
                    raise AssertionError(f"segment {s}: paths disagree (ssd)")
            else:
                y[off[s]:off[s + 1], heads] = rows
                st[s, heads] = snaps[e]
                done[s] = True
            pos += m
    return y, st
