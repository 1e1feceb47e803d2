"""Oracle for the tree-aware causal depthwise conv1d (test infrastructure only).

Definition ("Tree Training" section 3.2, "Causal convolution", Eq. 11, and
the tree-recurrence 0.1.0 page: each short conv reads the last inputs of its
own path): run the ordinary causal depthwise conv over every root-to-leaf
path on its own.  The conv is the cross-correlation with W-1 zeros padded on
the left, tap W-1 multiplying the current token (the convention of a
depthwise conv1d whose weight is [C, W]):

    y[t, c] = act( sum_{i=0}^{W-1} w[c, i] * xpad[t + i, c] + bias[c] ),
    xpad    = [0 (W-1 rows); x_path].

The context a segment sees is the raw input of the W-1 path tokens before it
(the saved context in the appendix's conv routine is the tail of the
concatenated inputs), act is none or SiLU.

A root may be given the W-1 inputs that precede it (a partition gateway of
the same paper, section 3.3 and appendix B.7, hands the conv state across a
cut); they take the place of the zero padding, which is Eq. 11's
y = Conv([ctx; x])[W-1:] with ctx the given rows.
"""
from __future__ import annotations

import numpy as np

from .trie import check_trie, leaf_paths, path_token_index, root_path, roots_of, segment_offsets


def conv_on_path(xp, w, bias=None, act=None, dtype=np.float64, ctx=None):
    """Causal depthwise conv of one path.  xp [L, C], w [C, W] -> y [L, C].
    ctx [W-1, C]: the inputs in front of the path, oldest first (default
    zeros)."""
    xp = np.asarray(xp, dtype=dtype)
    w = np.asarray(w, dtype=dtype)
    L, C = xp.shape
    W = w.shape[1]
    pad = np.zeros((W - 1, C), dtype=dtype) if ctx is None else np.asarray(ctx, dtype=dtype).reshape(W - 1, C)
    xpad = np.concatenate([pad, xp], axis=0)
    y = np.zeros((L, C), dtype=dtype)
    for i in range(W):
        y += w[:, i][None, :] * xpad[i:i + L]
    if bias is not None:
        y += np.asarray(bias, dtype=dtype)[None, :]
    if act in ("silu", "swish"):
        y = y / (1.0 + np.exp(-y))
    elif act not in (None, "none"):
        raise ValueError(f"unknown activation {act!r}")
    return y


def tree_conv_reference(parents, seg_lens, x, w, bias=None, act=None,
                        segments=None, dtype=np.float64, init_ctx=None):
    """Per-path conv over the packed trie.

    x [N, C] (any float dtype, upcast exactly) -> y [N, C] in `dtype`.
    init_ctx [n_roots, W-1, C]: the inputs in front of each root (roots in
    segment order; default zeros).  With segments=None every root-to-leaf
    path is run and every segment that several paths share must come out
    bitwise identical from each of them (Eq. 6).  With a list of segments
    only the root paths of those segments are run; rows of other segments
    are left as NaN.
    """
    parents, seg_lens = check_trie(parents, seg_lens)
    x = np.asarray(x, dtype=dtype)
    off = segment_offsets(seg_lens)
    rank = {r: i for i, r in enumerate(roots_of(parents))}
    y = np.full(x.shape, np.nan, dtype=dtype)
    done = np.zeros(len(parents), dtype=bool)
    paths = leaf_paths(parents) if segments is None else [root_path(parents, s) for s in segments]
    for path in paths:
        idx = path_token_index(path, seg_lens)
        ctx = None if init_ctx is None else np.asarray(init_ctx)[rank[path[0]]]
        yp = conv_on_path(x[idx], w, bias, act, dtype, ctx=ctx)
        pos = 0
        for s in path:
            n = int(seg_lens[s])
            rows = yp[pos:pos + n]
            if done[s]:
                if not np.array_equal(y[off[s]:off[s + 1]], rows):
                    raise AssertionError(f"segment {s}: paths disagree (conv)")
            else:
                y[off[s]:off[s + 1]] = rows
                done[s] = True
            pos += n
    return y


def conv_context_reference(parents, seg_lens, x, width, init_ctx=None, dtype=np.float64):
    """For every segment, the W-1 inputs of its path ending at its last token,
    oldest first: [n_seg, W-1, C].  Before a root they are the root's given
    context rows (init_ctx [n_roots, W-1, C]) or zeros."""
    parents, seg_lens = check_trie(parents, seg_lens)
    x = np.asarray(x, dtype=dtype)
    h = int(width) - 1
    rank = {r: i for i, r in enumerate(roots_of(parents))}
    out = np.zeros((len(parents), h, x.shape[1]), dtype=dtype)
    for s in range(len(parents)):
        path = root_path(parents, s)
        rows = x[path_token_index(path, seg_lens)]
        pad = (np.zeros((h, x.shape[1]), dtype=dtype) if init_ctx is None
               else np.asarray(init_ctx, dtype=dtype)[rank[path[0]]].reshape(h, x.shape[1]))
        full = np.concatenate([pad, rows], axis=0)
        out[s] = full[full.shape[0] - h:]
    return out
