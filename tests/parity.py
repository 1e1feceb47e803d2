"""Helpers shared by the GPU parity tests and the smoke check.

The bar (fp64 oracle on the same bf16/fp32 inputs):
  * outputs (o, y): max abs error <= 2e-2 beyond the rounding of the output
    format itself, i.e. |out - ref| <= 2e-2 + half an ulp of the output dtype
    at |ref| (bf16 spacing is 0.0625 for |ref| in [8, 16), so even the exactly
    rounded answer can sit 0.031 from the reference there);
  * segment final states: per (segment, value head), max-norm relative error
    max|S_gpu - S_ref| / max|S_ref| <= 1e-4.
"""
from __future__ import annotations

import numpy as np

from oracle import conv as oconv
from oracle import gdn as ogdn
from oracle import trie as otrie

OUT_ATOL = 2e-2
STATE_RTOL = 1e-4
# fp32 inputs and outputs: the scan carries every product as hi + lo bf16
# (2^-17 relative per operand, fp32 accumulation), so its outputs sit near
# 1e-6 of the fp64 result at these sizes; 1e-4 keeps two orders of margin and
# fails an output path that drops the lo parts (~2e-3 on the tiny trie).
OUT_ATOL_F32 = 1e-4


def out_atol(dtype) -> float:
    """The output bar for inputs of `dtype` ("f32"/"bf16" or a torch dtype)."""
    return OUT_ATOL_F32 if str(dtype) in ("f32", "torch.float32") else OUT_ATOL


def to_np(t):
    return t.detach().cpu().double().numpy()


def half_ulp(ref, torch_dtype):
    """Half the spacing of `torch_dtype` numbers at |ref| (0 for fp32 and wider)."""
    import torch
    if torch_dtype != torch.bfloat16:
        return np.zeros_like(ref)
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def out_err(gpu_t, ref, rows=None, cols=None):
    """Max over elements of |gpu - ref| - half_ulp(ref): the output error beyond
    the output format's own rounding."""
    g = to_np(gpu_t)
    if rows is not None:
        g = g[rows]
    if cols is not None:
        g = g[..., cols] if g.ndim == 2 else g[:, cols]
    return float((np.abs(g - ref) - half_ulp(ref, gpu_t.dtype)).max())


def state_rel_err(s_gpu, s_ref):
    """Per (segment, head) max-norm relative error; arrays [..., d_k, d_v]."""
    num = np.abs(s_gpu - s_ref).max(axis=(-2, -1))
    den = np.maximum(np.abs(s_ref).max(axis=(-2, -1)), 1e-30)
    return num / den


def sample_segments(parents, lens, k, seed=0):
    """The end of the longest path, the longest root, and k-2 random segments."""
    parents = np.asarray(parents)
    lens = np.asarray(lens)
    paths = otrie.leaf_paths(parents)
    longest = max(paths, key=lambda p: sum(int(lens[s]) for s in p))
    roots = np.flatnonzero(parents < 0)
    picks = [longest[-1], int(roots[np.argmax(lens[roots])])]
    rng = np.random.default_rng(seed)
    while len(picks) < k and len(picks) < len(parents):
        s = int(rng.integers(0, len(parents)))
        if s not in picks:
            picks.append(s)
    return picks


def scan_errors_full(parents, lens, q, k, v, g, beta, o_gpu, st_gpu, scale=1.0, heads=None,
                     init_states=None):
    """Run the oracle on every path (optionally a head subset) and compare all
    rows / states.  Returns (max abs output error, max state rel error)."""
    tq, tk, tv, tg_, tb = (to_np(x) for x in (q, k, v, g, beta))
    init = None if init_states is None else to_np(init_states)
    o_ref, s_ref = ogdn.tree_gdn_reference(parents, lens, tq, tk, tv, tg_, tb, scale, heads=heads,
                                           init_states=init)
    hs = np.arange(tv.shape[1]) if heads is None else np.asarray(heads)
    sg = to_np(st_gpu)[:, hs]
    return out_err(o_gpu, o_ref[:, hs], cols=hs), float(state_rel_err(sg, s_ref[:, hs]).max())


def scan_errors_sampled(parents, lens, q, k, v, g, beta, o_gpu, st_gpu, segments, heads, scale=1.0):
    """For each sampled segment, run the oracle over its root path for the given
    value heads only; compare the rows and states of every segment on the path."""
    import torch
    worst_o, worst_s = 0.0, 0.0
    for s in segments:
        path = otrie.root_path(parents, s)
        idx = torch.as_tensor(otrie.path_token_index(path, lens), device=q.device)
        sel = lambda t: to_np(t.index_select(0, idx))  # noqa: E731
        ends = np.cumsum([int(lens[p]) for p in path]) - 1
        op, snaps = ogdn.gdn_on_path(sel(q), sel(k), sel(v), sel(g), sel(beta), scale,
                                     snap_at=ends, heads=heads)
        worst_o = max(worst_o, out_err(o_gpu.index_select(0, idx), op, cols=heads))
        for p, e in zip(path, ends):
            sg = to_np(st_gpu[p])[heads]
            worst_s = max(worst_s, float(state_rel_err(sg, snaps[int(e)]).max()))
    return worst_o, worst_s


def conv_errors(parents, lens, x, w, y_gpu, bias=None, act=None, segments=None, channels=None,
                init_ctx=None):
    """Max abs error of the tree conv against the per-path oracle; with
    `segments`, only those segments' root paths (and `channels` subset)."""
    import torch
    cs = slice(None) if channels is None else channels
    tw = to_np(w)[cs]
    tb = None if bias is None else to_np(bias)[cs]
    if segments is None:
        ctx = None if init_ctx is None else to_np(init_ctx)[:, :, cs]
        ref = oconv.tree_conv_reference(parents, lens, to_np(x)[:, cs], tw, tb, act, init_ctx=ctx)
        return out_err(y_gpu, ref, cols=cs)
    worst = 0.0
    for s in segments:
        path = otrie.root_path(parents, s)
        idx = torch.as_tensor(otrie.path_token_index(path, lens), device=x.device)
        yp = oconv.conv_on_path(to_np(x.index_select(0, idx))[:, cs], tw, tb, act)
        worst = max(worst, out_err(y_gpu.index_select(0, idx), yp, cols=cs))
    return worst


def split_subtree(parents, c):
    """Cut segment c's subtree out of a trie (host bookkeeping, no
    arithmetic).  Returns (keep, parents_keep, index_keep, sub,
    parents_sub, index_sub): the kept and cut segment lists in original
    order, each with parents renumbered into its own list and a map
    original -> new index; c becomes the root of the cut part."""
    parents = [int(p) for p in parents]
    sub = {c}
    for i in range(c + 1, len(parents)):
        if parents[i] in sub:
            sub.add(i)
    keep = [i for i in range(len(parents)) if i not in sub]
    subl = sorted(sub)

    def renumber(segs):
        idx = {s: i for i, s in enumerate(segs)}
        return np.array([idx.get(parents[s], -1) if s != c else -1 for s in segs], np.int32), idx

    pa, ia = renumber(keep)
    pb, ib = renumber(subl)
    return keep, pa, ia, subl, pb, ib
