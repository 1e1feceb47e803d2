"""Oracle for the backward of the tree conv and the tree Gated DeltaNet
(test infrastructure only).

Definition.  The tree forward computes every token's output once ("Tree
Training" section 3.1, Eq. 6); the loss weights each token's output once, so
given the upstream gradient of every output (and, optionally, of every
segment's final recurrent state or conv context, as a partition gateway
relays them), the input gradients are the vector-Jacobian product of the tree
forward.  A segment reads its parent's final state, so the parent's state
receives the sum of the contributions of all its children (section 3.2 and
appendix A.2: sibling chunks share one parent state tensor and their
gradients accumulate in it); likewise a parent's last W-1 inputs receive the
conv gradients of every child's first tokens.

This module writes the tree forward token by token in fp64 torch on the CPU,
each segment in index order starting from its parent's final state (or the
root's given state, or zero) and with the conv window walked back along the
path (into the root's given context, or zeros), and differentiates it with
torch.autograd.  It is pinned against central finite differences of the
NumPy forward oracle (conv.py, gdn.py), an implementation it shares no code
with.  Small inputs only: the recurrence is a Python loop over tokens.
"""
from __future__ import annotations

import numpy as np

from .trie import check_trie, roots_of, segment_offsets


def _torch():
    import torch
    return torch


def _window_rows(parents, seg_lens, width):
    """For every token t, the W source rows of its conv window, oldest first
    (the last is t itself).  A row is a packed token index, or -1 - j for row
    j of the flattened root contexts [n_roots * (W-1)] (root r's row m is
    r (W-1) + m, oldest first)."""
    parents, seg_lens = check_trie(parents, seg_lens)
    off = segment_offsets(seg_lens)
    rank = {r: i for i, r in enumerate(roots_of(parents))}
    n = int(off[-1])
    rows = np.zeros((n, width), np.int64)
    for s in range(len(parents)):
        root = s
        while parents[root] >= 0:
            root = parents[root]
        for p in range(int(seg_lens[s])):
            t = int(off[s]) + p
            seg, pos, back = s, p, 0
            for i in range(width - 1, -1, -1):  # i = W-1 is t itself, then one step back each
                if seg is None:
                    back += 1
                    rows[t, i] = -1 - (rank[root] * (width - 1) + (width - 1 - back))
                    continue
                rows[t, i] = int(off[seg]) + pos
                if pos > 0:
                    pos -= 1
                elif parents[seg] >= 0:
                    seg = int(parents[seg])
                    pos = int(seg_lens[seg]) - 1
                else:
                    seg = None
    return rows


def tree_conv_vjp(parents, seg_lens, x, w, dy, bias=None, act=None, init_ctx=None):
    """Gradients of sum(dy * y) for y = tree conv(x, w, bias, act, init_ctx).

    x, dy [N, C]; w [C, W]; bias [C] or None; init_ctx [n_roots, W-1, C] or
    None (zeros).  Returns (dx [N, C], dw [C, W], dbias [C] or None,
    dinit_ctx [n_roots, W-1, C]) in fp64.
    """
    torch = _torch()
    parents, seg_lens = check_trie(parents, seg_lens)
    x = torch.tensor(np.asarray(x, np.float64), requires_grad=True)
    wt = torch.tensor(np.asarray(w, np.float64), requires_grad=True)
    n, c = x.shape
    width = wt.shape[1]
    n_roots = len(roots_of(parents))
    ctx0 = np.zeros((n_roots, width - 1, c)) if init_ctx is None else np.asarray(init_ctx, np.float64)
    ctx = torch.tensor(ctx0, requires_grad=True)
    b = None if bias is None else torch.tensor(np.asarray(bias, np.float64), requires_grad=True)
    rows = _window_rows(parents, seg_lens, width)
    src = torch.cat([x, ctx.reshape(-1, c)])  # context row j sits at N + j
    idx = torch.tensor(np.where(rows >= 0, rows, n + (-1 - rows)))
    xhat = src[idx]                                   # [N, W, C], oldest first
    z = (xhat * wt.t().unsqueeze(0)).sum(1)
    if b is not None:
        z = z + b
    y = z * torch.sigmoid(z) if act == "silu" else z
    (y * torch.tensor(np.asarray(dy, np.float64))).sum().backward()
    return (x.grad.numpy(), wt.grad.numpy(), None if b is None else b.grad.numpy(), ctx.grad.numpy())


def tree_gdn_vjp(parents, seg_lens, q, k, v, g, beta, do, scale=1.0, init_states=None, dstates=None):
    """Gradients of sum(do * o) + sum(dstates * states) for the tree gated
    delta rule (the recurrence of gdn.py), every segment starting from its
    parent's final state.

    q, k [N, H_qk, d_k]; v, do [N, H_v, d_v]; g, beta [N, H_v];
    init_states [n_roots, H_v, d_k, d_v] or None (zero); dstates [n_seg,
    H_v, d_k, d_v] or None (no gradient on the final states).  Value head h
    uses q/k head h // (H_v / H_qk).  Returns (dq, dk, dv, dg, dbeta,
    dinit_states) in fp64.
    """
    torch = _torch()
    parents, seg_lens = check_trie(parents, seg_lens)
    f = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)  # noqa: E731
    q, k, v, g, beta = f(q), f(k), f(v), f(g), f(beta)
    n, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    grp = torch.arange(h_v) // (h_v // h_qk)
    roots = roots_of(parents)
    rank = {r: i for i, r in enumerate(roots)}
    init0 = np.zeros((len(roots), h_v, d_k, d_v)) if init_states is None else np.asarray(init_states, np.float64)
    init = torch.tensor(init0, requires_grad=True)
    off = segment_offsets(seg_lens)
    do_t = torch.tensor(np.asarray(do, np.float64))
    loss = torch.zeros((), dtype=torch.float64)
    final = {}
    for s in range(len(parents)):
        S = final[int(parents[s])] if parents[s] >= 0 else init[rank[s]]
        for t in range(int(off[s]), int(off[s + 1])):
            kt, qt = k[t][grp], q[t][grp]                      # [H_v, d_k]
            S = torch.exp(g[t]).view(h_v, 1, 1) * S            # decay
            u = beta[t].view(h_v, 1) * (v[t] - torch.einsum("hkv,hk->hv", S, kt))
            S = S + kt.unsqueeze(2) * u.unsqueeze(1)           # write
            o = scale * torch.einsum("hkv,hk->hv", S, qt)      # read after the write
            loss = loss + (o * do_t[t]).sum()
        final[s] = S
        if dstates is not None:
            loss = loss + (S * torch.tensor(np.asarray(dstates[s], np.float64))).sum()
    loss.backward()
    return tuple(a.grad.numpy() for a in (q, k, v, g, beta, init))
