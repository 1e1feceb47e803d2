"""Helpers shared by the GPU parity tests and the smoke check.

The bar (fp64 oracle on the same bf16/fp32 inputs):
  * outputs (o, y): max abs error |out - ref| <= 2e-2 wherever a correctly
    rounded bf16 output can meet it, i.e. where half a bf16 ulp at |ref| is
    below 2e-2 (|ref| < 8).  From |ref| = 8 on the bf16 spacing is 0.0625 or
    more, so even the exactly rounded answer can sit 0.031 or more from the
    reference; there the bar is 2e-2 beyond that half ulp;
  * segment final states: per (segment, value head), max-norm relative error
    max|S_gpu - S_ref| / max|S_ref| <= 1e-4.
"""
from __future__ import annotations

import os
import sys

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


# Every output and state comparison of the session, for the run's summary
# (tests/conftest.py prints the worst of each kind after the tests).
RECORDS: list = []


def _record(kind, **vals):
    RECORDS.append(dict(kind=kind, test=os.environ.get("PYTEST_CURRENT_TEST", "").split(" (")[0], **vals))


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


def rounding_allowance(ref, torch_dtype):
    """What the output bar allows beyond 2e-2 at |ref|: half a bf16 ulp where
    that alone exceeds 2e-2 (|ref| >= 8), zero elsewhere and for fp32."""
    hu = half_ulp(ref, torch_dtype)
    return np.where(hu >= OUT_ATOL, hu, 0.0)


def out_errs(gpu_t, ref, rows=None, cols=None):
    """Output errors of gpu_t against ref: a dict with the raw max abs error,
    the max error beyond the output format's own rounding (|gpu - ref| -
    half_ulp) and the asserted measure (|gpu - ref| - rounding_allowance),
    which the bar holds to OUT_ATOL."""
    g = to_np(gpu_t)
    if rows is not None:
        g = g[rows]
    if cols is not None:
        g = g[..., cols] if g.ndim == 2 else g[:, cols]
    d = np.abs(g - ref)
    return {"raw": float(d.max()),
            "beyond_rounding": float((d - half_ulp(ref, gpu_t.dtype)).max()),
            "asserted": float((d - rounding_allowance(ref, gpu_t.dtype)).max())}


def out_err(gpu_t, ref, rows=None, cols=None, log=True, what="output"):
    """The asserted output error (see out_errs); the raw and beyond-rounding
    figures are printed to stderr."""
    e = out_errs(gpu_t, ref, rows, cols)
    _record(what, dtype=str(gpu_t.dtype).replace("torch.", ""), **e)
    if log:
        print(f"    output error: raw max abs {e['raw']:.3e}, beyond bf16 rounding {e['beyond_rounding']:.3e}, "
              f"asserted {e['asserted']:.3e}", file=sys.stderr, flush=True)
    return e["asserted"]


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
    es = float(state_rel_err(sg, s_ref[:, hs]).max())
    _record("state", rel=es)
    return out_err(o_gpu, o_ref[:, hs], cols=hs, what="scan output"), es


def _gdn_path_task(a):
    """One oracle run (a process-pool task): a path's inputs for a block of
    value heads (and their query/key heads) -> (outputs, end-of-segment states)."""
    q, k, v, g, beta, scale, ends = a
    return ogdn.gdn_on_path(q, k, v, g, beta, scale, snap_at=ends)


def oracle_workers():
    """Worker processes for the pooled oracle: the CPUs this process may use,
    at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def run_pooled(fn, tasks, workers=None, timeout_s=600):
    """[fn(t) for t in tasks] in a pool of fresh (spawned) interpreters that
    import nothing but the oracle; one task runs in this process.  The pool
    is terminated on any failure or after timeout_s, so a worker that cannot
    start ends the call with an error rather than a wait."""
    if len(tasks) <= 1:
        return [fn(t) for t in tasks]
    import multiprocessing as mp
    pool = mp.get_context("spawn").Pool(min(len(tasks), workers or oracle_workers()))
    try:
        return pool.map_async(fn, tasks, chunksize=1).get(timeout_s)
    finally:
        pool.terminate()
        pool.join()


def scan_errors_sampled(parents, lens, q, k, v, g, beta, o_gpu, st_gpu, segments, heads=None, scale=1.0,
                        workers=None):
    """For each sampled segment, run the oracle over its root path and compare
    the rows and final states of every segment on the path.  heads=None
    checks every value head: the oracle runs in a spawned process pool, one
    task per (segment, block of value heads sharing query/key heads).
    Returns (asserted output error, max state rel error)."""
    import torch

    h_qk, h_v = q.shape[1], v.shape[1]
    grp = h_v // h_qk
    if heads is None:
        n_blk = min(h_qk, max(1, (workers or oracle_workers()) // max(1, len(segments))))
        while h_qk % n_blk:
            n_blk -= 1
        qb = h_qk // n_blk
        blocks = [np.arange(b * qb * grp, (b + 1) * qb * grp) for b in range(n_blk)]
    else:
        blocks = [np.asarray([h]) for h in heads]
    tasks, meta = [], []
    for s in segments:
        path = otrie.root_path(parents, s)
        idx = torch.as_tensor(otrie.path_token_index(path, lens), device=q.device)
        ends = np.cumsum([int(lens[p]) for p in path]) - 1
        host = {n: to_np(t.index_select(0, idx)) for n, t in (("q", q), ("k", k), ("v", v), ("g", g),
                                                               ("beta", beta))}
        for hs in blocks:
            # A block is one value head or whole query/key groups, so inside
            # the task value head j uses sliced query/key head j // (its group).
            qh = np.unique(hs // grp)
            tasks.append((host["q"][:, qh], host["k"][:, qh], host["v"][:, hs], host["g"][:, hs],
                          host["beta"][:, hs], scale, ends))
            meta.append((path, idx, ends, hs))
    results = run_pooled(_gdn_path_task, tasks, workers)
    worst_o, worst_s = 0.0, 0.0
    raw = 0.0
    for (path, idx, ends, hs), (op, snaps) in zip(meta, results):
        e = out_errs(o_gpu.index_select(0, idx), op, cols=hs)
        _record("scan output", dtype=str(o_gpu.dtype).replace("torch.", ""), **e)
        worst_o = max(worst_o, e["asserted"])
        raw = max(raw, e["raw"])
        for p, en in zip(path, ends):
            sg = to_np(st_gpu[p])[hs]
            worst_s = max(worst_s, float(state_rel_err(sg, snaps[int(en)]).max()))
    _record("state", rel=worst_s)
    print(f"    sampled scan check: {len(segments)} segments x {sum(len(b) for b in blocks)} value heads, "
          f"output raw max abs {raw:.3e}, asserted {worst_o:.3e}, state rel {worst_s:.3e}",
          file=sys.stderr, flush=True)
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
        return out_err(y_gpu, ref, cols=cs, what="conv output")
    worst = 0.0
    for s in segments:
        path = otrie.root_path(parents, s)
        idx = torch.as_tensor(otrie.path_token_index(path, lens), device=x.device)
        yp = oconv.conv_on_path(to_np(x.index_select(0, idx))[:, cs], tw, tb, act)
        worst = max(worst, out_err(y_gpu.index_select(0, idx), yp, cols=cs, what="conv output"))
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
