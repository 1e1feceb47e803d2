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
"""
from __future__ import annotations

import numpy as np

from .trie import check_trie, leaf_paths, path_token_index, root_path, segment_offsets


def conv_on_path(xp, w, bias=None, act=None, dtype=np.float64):
    """Causal depthwise conv of one path.  xp [L, C], w [C, W] -> y [L, C]."""
    xp = np.asarray(xp, dtype=dtype)
    w = np.asarray(w, dtype=dtype)
    L, C = xp.shape
    W = w.shape[1]
    xpad = np.concatenate([np.zeros((W - 1, C), dtype=dtype), xp], axis=0)
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
                        segments=None, dtype=np.float64):
    """Per-path conv over the packed trie.

    x [N, C] (any float dtype, upcast exactly) -> y [N, C] in `dtype`.
    With segments=None every root-to-leaf path is run and every segment that
    several paths share must come out bitwise identical from each of them
    (Eq. 6).  With a list of segments only the root paths of those segments
    are run; rows of other segments are left as NaN.
    """
    parents, seg_lens = check_trie(parents, seg_lens)
    x = np.asarray(x, dtype=dtype)
    off = segment_offsets(seg_lens)
    y = np.full(x.shape, np.nan, dtype=dtype)
    done = np.zeros(len(parents), dtype=bool)
    paths = leaf_paths(parents) if segments is None else [root_path(parents, s) for s in segments]
    for path in paths:
        idx = path_token_index(path, seg_lens)
        yp = conv_on_path(x[idx], w, bias, act, dtype)
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
