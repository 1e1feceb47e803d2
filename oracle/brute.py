"""Independent fp64 brute forces used to pin the oracle (test infrastructure).

These use different formulations from conv.py / gdn.py on purpose, so that a
slip in one is not repeated in the other:

* conv_brute walks "previous token on my path" pointers per token instead of
  building path index lists.
* gdn_brute keeps the state in the [d_v, d_k] orientation and applies the
  recurrence as explicit matrix products,
      M_t = a_t M_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = M_t q_t,
  with a_t = exp(g_t), over each segment's own root path.

Pure Python loops over tokens: small inputs only.
"""
from __future__ import annotations

import numpy as np


def _prev_token_fn(parents, seg_lens):
    parents = [int(p) for p in parents]
    seg_lens = [int(n) for n in seg_lens]
    start, seg_of = [], []
    pos = 0
    for s, n in enumerate(seg_lens):
        start.append(pos)
        seg_of.extend([s] * n)
        pos += n

    def prev(t):
        s = seg_of[t]
        if t > start[s]:
            return t - 1
        p = parents[s]
        if p < 0:
            return None
        return start[p] + seg_lens[p] - 1

    return prev, seg_of, start


def conv_brute(parents, seg_lens, x, w, bias=None, act=None):
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    W = w.shape[1]
    prev, _, _ = _prev_token_fn(parents, seg_lens)
    y = np.zeros_like(x)
    for t in range(x.shape[0]):
        acc = np.zeros(x.shape[1])
        j, back = t, 0
        while j is not None and back < W:
            acc += w[:, W - 1 - back] * x[j]
            j = prev(j)
            back += 1
        if bias is not None:
            acc += np.asarray(bias, dtype=np.float64)
        if act == "silu":
            acc = acc / (1.0 + np.exp(-acc))
        y[t] = acc
    return y


def gdn_brute(parents, seg_lens, q, k, v, g, beta, scale=1.0):
    """Returns (o [N, H_v, d_v], states [n_seg, H_v, d_k, d_v]) in fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    n_tok, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    group = h_v // h_qk
    prev, seg_of, start = _prev_token_fn(parents, seg_lens)
    n_seg = len(seg_lens)
    o = np.zeros((n_tok, h_v, d_v))
    states = np.zeros((n_seg, h_v, d_k, d_v))
    eye = np.eye(d_k)
    for s in range(n_seg):
        last = start[s] + int(seg_lens[s]) - 1
        # The token sequence of s's root path, found by walking backwards.
        seq = []
        t = last
        while t is not None:
            seq.append(t)
            t = prev(t)
        seq.reverse()
        for h in range(h_v):
            hq = h // group
            M = np.zeros((d_v, d_k))
            for t in seq:
                kt = k[t, hq][:, None]
                vt = v[t, h][:, None]
                M = np.exp(g[t, h]) * M @ (eye - beta[t, h] * kt @ kt.T) + beta[t, h] * vt @ kt.T
                if seg_of[t] == s:
                    o[t, h] = M @ (scale * q[t, hq])
            states[s, h] = M.T
    return o, states
