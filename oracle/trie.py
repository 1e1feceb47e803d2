"""Trie bookkeeping for the oracle (test infrastructure only).

A trie is given as parents[i] (-1 for a root) and seg_lens[i] > 0, with the
segments' tokens packed one after another in index order (the depth-first
serialisation, "Tree Training" section 3.1 Eq. 8).  A path is the list of
segments from a root down to a leaf; its tokens are the concatenation of the
segments' packed index ranges.
"""
from __future__ import annotations

import numpy as np


def _check(parents, seg_lens):
    parents = np.asarray(parents, dtype=np.int64)
    seg_lens = np.asarray(seg_lens, dtype=np.int64)
    n = parents.shape[0]
    if n == 0 or seg_lens.shape != (n,):
        raise ValueError("parents and seg_lens must be non-empty and of equal length")
    if np.any(seg_lens <= 0):
        raise ValueError("every segment needs at least one token")
    for i, p in enumerate(parents):
        if p < -1 or p >= n or p == i:
            raise ValueError(f"bad parent {p} for segment {i}")
    # Reject cycles: every walk towards the root must end within n steps.
    for i in range(n):
        j, steps = i, 0
        while j >= 0:
            j = int(parents[j])
            steps += 1
            if steps > n:
                raise ValueError("parents contain a cycle")
    return parents, seg_lens


def segment_offsets(seg_lens):
    """off[i] = first packed token of segment i; off[n] = total tokens."""
    seg_lens = np.asarray(seg_lens, dtype=np.int64)
    off = np.zeros(seg_lens.shape[0] + 1, dtype=np.int64)
    np.cumsum(seg_lens, out=off[1:])
    return off


def children_of(parents):
    kids = [[] for _ in range(len(parents))]
    for i, p in enumerate(parents):
        if p >= 0:
            kids[int(p)].append(i)
    return kids


def roots_of(parents):
    """Roots in segment order (the order initial states and contexts use)."""
    return [i for i, p in enumerate(parents) if int(p) < 0]


def leaves_of(parents):
    kids = children_of(parents)
    return [i for i in range(len(parents)) if not kids[i]]


def root_path(parents, s):
    """Segments from the root down to segment s (inclusive)."""
    out = []
    j = int(s)
    while j >= 0:
        out.append(j)
        j = int(parents[j])
    return out[::-1]


def leaf_paths(parents, seg_lens=None):
    if seg_lens is not None:
        _check(parents, seg_lens)
    return [root_path(parents, leaf) for leaf in leaves_of(parents)]


def path_token_index(path, seg_lens):
    off = segment_offsets(seg_lens)
    return np.concatenate([np.arange(off[s], off[s + 1]) for s in path])


def path_token_count(parents, seg_lens):
    """Sum over root-to-leaf paths of the path length: the token count of the
    serialisation that repeats every shared prefix ("Tree Training" Eq. 7)."""
    parents, seg_lens = _check(parents, seg_lens)
    return int(sum(sum(int(seg_lens[s]) for s in p) for p in leaf_paths(parents)))


def por(parents, seg_lens):
    """Potential overlap ratio, "Tree Training" section 4.1 Eq. 12:
    1 - (tokens in the trie) / (tokens of the prefix-repeating serialisation)."""
    return 1.0 - float(np.sum(seg_lens)) / float(path_token_count(parents, seg_lens))


def check_trie(parents, seg_lens):
    return _check(parents, seg_lens)
