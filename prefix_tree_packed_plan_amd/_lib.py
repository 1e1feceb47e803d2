"""ctypes binding of libtreegdn.so (include/tree_gdn.h).

Argument marshalling only: PyTorch provides device memory and the current
HIP stream; every step of the forward runs in the library's kernels.  There
is no fallback: if the library is missing or a call fails, an exception is
raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtreegdn.so")

TREE_OK = 0
ERRORS = {
    -1: "TREE_ERR_INVALID_ARG",
    -2: "TREE_ERR_BAD_TREE",
    -3: "TREE_ERR_SIZE",
    -4: "TREE_ERR_UNSUPPORTED",
    -5: "TREE_ERR_WORKSPACE",
    -6: "TREE_ERR_HIP",
}
DTYPE_F32, DTYPE_BF16 = 0, 1
ACT_NONE, ACT_SILU = 0, 1
SCHED_LEVEL, SCHED_RESCAN, SCHED_AUTO = 0, 1, 2
SCHEDULES = {"level": SCHED_LEVEL, "rescan": SCHED_RESCAN, "auto": SCHED_AUTO}
FORK_MIN_SAVED_TOKENS = 256  # the header's default price of one extra launch

# Every function the header declares, with its ctypes signature.
_P, _I32, _I64, _SZ, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float


class PlanStats(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int64),
        ("path_tokens", ctypes.c_int64),
        ("max_path_tokens", ctypes.c_int64),
        ("por", ctypes.c_double),
        ("n_seg", ctypes.c_int32),
        ("n_roots", ctypes.c_int32),
        ("n_leaves", ctypes.c_int32),
        ("n_parents", ctypes.c_int32),
        ("n_levels", ctypes.c_int32),
        ("conv_width", ctypes.c_int32),
        ("path_entries", ctypes.c_int64),
    ]


SIGNATURES = {
    "tree_plan": (ctypes.c_int, [_P, _P, _I32, _I32, ctypes.POINTER(_P)]),
    "tree_plan_free": (None, [_P]),
    "tree_plan_query": (ctypes.c_int, [_P, ctypes.POINTER(PlanStats)]),
    "tree_plan_conv_history": (ctypes.c_int, [_P, _P]),
    "tree_plan_levels": (ctypes.c_int, [_P, _P, _P]),
    "tree_plan_paths": (ctypes.c_int, [_P, _P, _P]),
    "tree_plan_choose_schedule": (ctypes.c_int, [_P, _I64, ctypes.POINTER(_I32)]),
    "tree_plan_device_bytes": (_SZ, [_P]),
    "tree_plan_upload": (ctypes.c_int, [_P, _P, _SZ, _P]),
    "tree_conv": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "tree_conv_backward_workspace_bytes": (_SZ, [_P, _I32]),
    "tree_conv_backward": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _P, _P, _SZ,
                                          _P, _SZ, _P]),
    "tree_scan_workspace_bytes": (_SZ, [_P, _I32, _I32, _I32, _I32]),
    "tree_workspace_bytes": (_SZ, [_P, _I32, _I32, _I32, _I32]),
    "tree_gdn_scan": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32,
                                     _F, _I32, _I32, _P, _P, _SZ, _P, _SZ, _P]),
    "tree_gdn_scan_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32,
                                             _F, _I32, _I32, _P, _P]),
    "tree_gdn_scan_backward_workspace_bytes": (_SZ, [_P, _I32, _I32, _I32, _I32]),
    "tree_gdn_scan_backward": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64,
                                              _I32, _I32, _I32, _I32, _F, _I32, _P, _P, _SZ, _P, _SZ, _P]),
    "tree_ssd_scan": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32,
                                     _P, _P, _SZ, _P, _SZ, _P]),
    "tree_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load():
    """Load the library (once).  Raises OSError if it has not been built."""
    global _lib
    if _lib is None:
        # torch bundles its own HIP runtime under the same soname
        # (libamdhip64.so.7).  Loading torch first makes the library's
        # dependency bind to that runtime, so torch's tensors, streams and
        # the kernels here share one HIP runtime and one device context.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is missing: build it with "
                          "`python -m prefix_tree_packed_plan_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class TreeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


def _check(rc):
    if rc != TREE_OK:
        raise TreeError(rc, load().tree_last_error().decode())


# --------------------------------------------------------------------- plan

class TreePlan:
    """Host plan of a packed trie (tree_plan), plus its device copies."""

    def __init__(self, parents, seg_lens, conv_width: int = 4):
        lib = load()
        self._parents = np.ascontiguousarray(parents, dtype=np.int32)
        self._lens = np.ascontiguousarray(seg_lens, dtype=np.int32)
        if self._parents.shape != self._lens.shape or self._parents.ndim != 1:
            raise ValueError("parents and seg_lens must be 1-D and of equal length")
        h = _P()
        _check(lib.tree_plan(self._parents.ctypes.data, self._lens.ctypes.data,
                             int(self._parents.shape[0]), int(conv_width), ctypes.byref(h)))
        self._h = h
        st = PlanStats()
        _check(lib.tree_plan_query(self._h, ctypes.byref(st)))
        self.stats = {f: getattr(st, f) for f, _ in PlanStats._fields_}
        self._dev = {}

    @property
    def handle(self):
        return self._h

    @property
    def n_tokens(self) -> int:
        return int(self.stats["n_tokens"])

    @property
    def n_seg(self) -> int:
        return int(self.stats["n_seg"])

    @property
    def conv_width(self) -> int:
        return int(self.stats["conv_width"])

    @property
    def n_roots(self) -> int:
        return int(self.stats["n_roots"])

    def conv_history(self) -> np.ndarray:
        w1 = self.conv_width - 1
        out = np.zeros((self.n_seg, max(w1, 0)), np.int32)
        if w1 > 0:
            _check(load().tree_plan_conv_history(self._h, out.ctypes.data))
        return out

    def levels(self):
        ls = np.zeros(self.stats["n_levels"] + 1, np.int32)
        order = np.zeros(self.n_seg, np.int32)
        _check(load().tree_plan_levels(self._h, ls.ctypes.data, order.ctypes.data))
        return ls, order

    def paths(self):
        """Rescan walks: (path_off [n_leaves + 1], path_seg [path_entries]);
        an entry is a segment the walk writes, or ~segment if another walk
        writes it."""
        n = int(self.stats["path_entries"])
        off = np.zeros(self.stats["n_leaves"] + 1, np.int32)
        seg = np.zeros(max(n, 1), np.int32)
        _check(load().tree_plan_paths(self._h, off.ctypes.data, seg.ctypes.data))
        return off, seg[:n]

    def choose_schedule(self, fork_min_saved_tokens: int = FORK_MIN_SAVED_TOKENS) -> str:
        """The fork/rescan policy: "level" when the prefix tokens forking saves
        reach fork_min_saved_tokens per extra launch, else "rescan"."""
        out = _I32()
        _check(load().tree_plan_choose_schedule(self._h, int(fork_min_saved_tokens), ctypes.byref(out)))
        return {SCHED_LEVEL: "level", SCHED_RESCAN: "rescan"}[out.value]

    def device_bytes(self) -> int:
        return int(load().tree_plan_device_bytes(self._h))

    def on_device(self, device):
        """The plan's device copy on `device` (uploaded once, stream-ordered)."""
        import torch
        dev = torch.device(device)
        key = dev.index if dev.index is not None else torch.cuda.current_device()
        if key not in self._dev:
            buf = torch.empty(self.device_bytes(), dtype=torch.uint8, device=dev)
            stream = torch.cuda.current_stream(buf.device).cuda_stream
            _check(load().tree_plan_upload(self._h, buf.data_ptr(), buf.numel(), stream))
            torch.cuda.current_stream(buf.device).synchronize()
            self._dev[key] = buf
        return self._dev[key]

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.tree_plan_free(h)
            self._h = None


def tree_plan(parents, seg_lens, conv_width: int = 4) -> TreePlan:
    return TreePlan(parents, seg_lens, conv_width)


# ------------------------------------------------------------------ kernels

def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name, dtype=None, device=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _need_shape(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _workspace(workspace, need, dev):
    """The caller's workspace (a device tensor of at least `need` bytes) or a
    new one; returns (tensor or None, bytes)."""
    import torch
    if workspace is None:
        if need <= 0:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", device=dev)
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise ValueError(f"workspace has {nbytes} bytes, needs {need}")
    return workspace, nbytes


def tree_conv(x, w, plan: TreePlan, bias=None, act: Optional[str] = None, out=None,
              init_ctx=None, return_ctx: bool = False, ctx_out=None):
    """y = tree-aware causal depthwise conv of x [N, C] with w [C, W].

    init_ctx [n_roots, W-1, C]: the inputs in front of each root (default
    zeros).  With return_ctx (or ctx_out given) also returns the W-1 path
    inputs ending at each segment's last token, [n_seg, W-1, C]."""
    import torch
    _need(x, "x")
    _need(w, "w", x.dtype, x.device)
    if x.dim() != 2 or w.dim() != 2 or w.shape[0] != x.shape[1] or w.shape[1] != plan.conv_width:
        raise ValueError("shapes must be x [N, C], w [C, W] with W = plan conv width")
    if bias is not None:
        _need(bias, "bias", x.dtype, x.device)
        _need_shape(bias, "bias", (x.shape[1],))
    w1 = plan.conv_width - 1
    if init_ctx is not None:
        _need(init_ctx, "init_ctx", x.dtype, x.device)
        if tuple(init_ctx.shape) != (plan.n_roots, w1, x.shape[1]):
            raise ValueError("init_ctx must be [n_roots, W-1, C]")
    if return_ctx and ctx_out is None:
        ctx_out = torch.empty((plan.n_seg, w1, x.shape[1]), dtype=x.dtype, device=x.device)
    if ctx_out is not None:
        _need(ctx_out, "ctx_out", x.dtype, x.device)
        if tuple(ctx_out.shape) != (plan.n_seg, w1, x.shape[1]):
            raise ValueError("ctx_out must be [n_seg, W-1, C]")
    y = torch.empty_like(x) if out is None else out
    _need(y, "out", x.dtype, x.device)
    _need_shape(y, "out", x.shape)
    a = {None: ACT_NONE, "none": ACT_NONE, "silu": ACT_SILU, "swish": ACT_SILU}[act]
    dplan = plan.on_device(x.device)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    _check(load().tree_conv(x.data_ptr(), w.data_ptr(), bias.data_ptr() if bias is not None else None,
                            y.data_ptr(), init_ctx.data_ptr() if init_ctx is not None else None,
                            ctx_out.data_ptr() if ctx_out is not None else None,
                            x.shape[0], x.shape[1], _dtype_code(x), a, plan.handle, dplan.data_ptr(),
                            dplan.numel(), stream))
    if return_ctx:
        return y, ctx_out
    return y


def tree_conv_backward(x, w, dy, plan: TreePlan, bias=None, act: Optional[str] = None, init_ctx=None,
                       dx=None, workspace=None):
    """Gradients of the tree conv: (dx [N, C] in x's dtype, dw [C, W] fp32,
    dbias [C] fp32 or None, dinit_ctx [n_roots, W-1, C] fp32 or None).
    dy is the gradient of the conv output (same dtype as x)."""
    import torch
    _need(x, "x")
    dev = x.device
    _need(w, "w", x.dtype, dev)
    _need(dy, "dy", x.dtype, dev)
    if x.dim() != 2 or dy.shape != x.shape or w.dim() != 2 or w.shape[0] != x.shape[1]:
        raise ValueError("shapes must be x, dy [N, C] and w [C, W]")
    n, c = x.shape
    w1 = w.shape[1] - 1
    if w.shape[1] != plan.conv_width:
        raise ValueError("w's width must be the plan's conv width")
    if bias is not None:
        _need(bias, "bias", x.dtype, dev)
        _need_shape(bias, "bias", (c,))
    if init_ctx is not None:
        _need(init_ctx, "init_ctx", x.dtype, dev)
        if tuple(init_ctx.shape) != (plan.n_roots, w1, c):
            raise ValueError("init_ctx must be [n_roots, W-1, C]")
    dx = torch.empty_like(x) if dx is None else dx
    _need(dx, "dx", x.dtype, dev)
    _need_shape(dx, "dx", x.shape)
    dw = torch.empty((c, w1 + 1), dtype=torch.float32, device=dev)
    db = torch.empty(c, dtype=torch.float32, device=dev) if bias is not None else None
    dctx = torch.empty((plan.n_roots, w1, c), dtype=torch.float32, device=dev) if w1 > 0 else None
    lib = load()
    need = int(lib.tree_conv_backward_workspace_bytes(plan.handle, c))
    workspace, ws_bytes = _workspace(workspace, need, dev)
    a = {None: ACT_NONE, "silu": ACT_SILU}[act]
    dplan = plan.on_device(dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    p = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    _check(lib.tree_conv_backward(x.data_ptr(), w.data_ptr(), p(bias), dy.data_ptr(), p(init_ctx), dx.data_ptr(),
                                  dw.data_ptr(), p(db), p(dctx), n, c, _dtype_code(x), a, plan.handle,
                                  dplan.data_ptr(), dplan.numel(), p(workspace), ws_bytes, stream))
    return dx, dw, db, dctx


def tree_gdn_scan(q, k, v, g, beta, plan: TreePlan, scale: float = 1.0, return_states: bool = False,
                  out=None, states=None, workspace=None, init_states=None, schedule: str = "auto",
                  fork_min_saved_tokens: int = FORK_MIN_SAVED_TOKENS):
    """Tree gated delta rule: o [N, H_v, d_v] (and states [n_seg, H_v, d_k, d_v] fp32).

    init_states [n_roots, H_v, d_k, d_v] fp32: the states the roots start
    from (default zero).  schedule: "level" (fork), "rescan" or "auto"
    (plan.choose_schedule(fork_min_saved_tokens)); all give the same bits."""
    import torch
    _need(q, "q")
    dev = q.device
    _need(k, "k", q.dtype, dev)
    _need(v, "v", q.dtype, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[0] != q.shape[0]:
        raise ValueError("shapes must be q, k [N, H_qk, d_k] and v [N, H_v, d_v]")
    n, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    if g.shape != (n, h_v) or beta.shape != (n, h_v):
        raise ValueError("g and beta must be [N, H_v]")
    o = torch.empty_like(v) if out is None else out
    _need(o, "out", q.dtype, dev)
    _need_shape(o, "out", v.shape)
    if return_states and states is None:
        states = torch.empty((plan.n_seg, h_v, d_k, d_v), dtype=torch.float32, device=dev)
    if states is not None:
        _need(states, "states", torch.float32, dev)
        _need_shape(states, "states", (plan.n_seg, h_v, d_k, d_v))
    if init_states is not None:
        _need(init_states, "init_states", torch.float32, dev)
        if tuple(init_states.shape) != (plan.n_roots, h_v, d_k, d_v):
            raise ValueError("init_states must be [n_roots, H_v, d_k, d_v]")
    if schedule not in SCHEDULES:
        raise ValueError(f"schedule must be one of {sorted(SCHEDULES)}")
    if schedule == "auto":
        schedule = plan.choose_schedule(fork_min_saved_tokens)
    sched = SCHEDULES[schedule]
    lib = load()
    need = 0
    if sched == SCHED_LEVEL:
        need = int(lib.tree_scan_workspace_bytes(plan.handle, h_v, d_k, d_v, int(states is not None)))
    workspace, ws_bytes = _workspace(workspace, need, dev)
    dplan = plan.on_device(dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    _check(lib.tree_gdn_scan(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
                             o.data_ptr(), init_states.data_ptr() if init_states is not None else None,
                             states.data_ptr() if states is not None else None,
                             n, h_qk, h_v, d_k, d_v, float(scale), _dtype_code(q), sched,
                             plan.handle, dplan.data_ptr(), dplan.numel(),
                             workspace.data_ptr() if workspace is not None else None, ws_bytes, stream))
    if return_states:
        return o, states
    return o


def tree_gdn_scan_backward(q, k, v, g, beta, do, plan: TreePlan, states, scale: float = 1.0,
                           init_states=None, dstates=None, workspace=None):
    """Gradients of the tree gated delta rule, given the upstream gradient do
    [N, H_v, d_v] of the outputs (and optionally dstates [n_seg, H_v, d_k,
    d_v] of every segment's final state) and the forward's final states
    `states` [n_seg, H_v, d_k, d_v] fp32 (tree_gdn_scan(..., return_states=True)).

    Returns fp32 (dq [N, H_qk, d_k], dk [N, H_qk, d_k], dv [N, H_v, d_v],
    dg [N, H_v], dbeta [N, H_v], dinit_states [n_roots, H_v, d_k, d_v])."""
    import torch
    _need(q, "q")
    dev = q.device
    f32 = torch.float32
    _need(k, "k", q.dtype, dev)
    _need(v, "v", q.dtype, dev)
    _need(do, "do", q.dtype, dev)
    _need(g, "g", f32, dev)
    _need(beta, "beta", f32, dev)
    _need(states, "states", f32, dev)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[0] != q.shape[0] or do.shape != v.shape:
        raise ValueError("shapes must be q, k [N, H_qk, d_k] and v, do [N, H_v, d_v]")
    n, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    if g.shape != (n, h_v) or beta.shape != (n, h_v):
        raise ValueError("g and beta must be [N, H_v]")
    st_shape = (plan.n_seg, h_v, d_k, d_v)
    if tuple(states.shape) != st_shape:
        raise ValueError("states must be [n_seg, H_v, d_k, d_v]")
    if dstates is not None:
        _need(dstates, "dstates", f32, dev)
        if tuple(dstates.shape) != st_shape:
            raise ValueError("dstates must be [n_seg, H_v, d_k, d_v]")
    if init_states is not None:
        _need(init_states, "init_states", f32, dev)
        if tuple(init_states.shape) != (plan.n_roots, h_v, d_k, d_v):
            raise ValueError("init_states must be [n_roots, H_v, d_k, d_v]")
    dq = torch.empty((n, h_qk, d_k), dtype=f32, device=dev)
    dk = torch.empty((n, h_qk, d_k), dtype=f32, device=dev)
    dv = torch.empty((n, h_v, d_v), dtype=f32, device=dev)
    dg = torch.empty((n, h_v), dtype=f32, device=dev)
    db = torch.empty((n, h_v), dtype=f32, device=dev)
    dinit = torch.empty((plan.n_roots, h_v, d_k, d_v), dtype=f32, device=dev)
    lib = load()
    need = int(lib.tree_gdn_scan_backward_workspace_bytes(plan.handle, h_qk, h_v, d_k, d_v))
    workspace, ws_bytes = _workspace(workspace, need, dev)
    dplan = plan.on_device(dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    p = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    _check(lib.tree_gdn_scan_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
                                      do.data_ptr(), p(dstates), p(init_states), states.data_ptr(),
                                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dg.data_ptr(), db.data_ptr(),
                                      dinit.data_ptr(), n, h_qk, h_v, d_k, d_v, float(scale), _dtype_code(q),
                                      plan.handle, dplan.data_ptr(), dplan.numel(), p(workspace), ws_bytes,
                                      stream))
    return dq, dk, dv, dg, db, dinit


def tree_ssd_scan(x, dt, A, B, C, plan: TreePlan, D=None, return_states: bool = False, out=None, states=None,
                  workspace=None, init_states=None):
    """Tree Mamba2 (SSD) forward: y [N, n_heads, head_dim] (and states
    [n_seg, n_heads, d_state, head_dim] fp32).

    x [N, n_heads, head_dim]; dt [N, n_heads] fp32 (after softplus); A
    [n_heads] fp32 (< 0); B, C [N, n_groups, d_state] (x's dtype); D
    [n_heads] fp32 or None; init_states [n_roots, n_heads, d_state,
    head_dim] fp32 or None."""
    import torch
    _need(x, "x")
    dev = x.device
    f32 = torch.float32
    _need(dt, "dt", f32, dev)
    _need(A, "A", f32, dev)
    _need(B, "B", x.dtype, dev)
    _need(C, "C", x.dtype, dev)
    if x.dim() != 3 or B.dim() != 3 or C.shape != B.shape or B.shape[0] != x.shape[0]:
        raise ValueError("shapes must be x [N, H, P] and B, C [N, G, d_state]")
    n, n_heads, head_dim = x.shape
    n_groups, d_state = B.shape[1], B.shape[2]
    if dt.shape != (n, n_heads) or A.shape != (n_heads,):
        raise ValueError("dt must be [N, H] and A [H]")
    if D is not None:
        _need(D, "D", f32, dev)
        if D.shape != (n_heads,):
            raise ValueError("D must be [H]")
    y = torch.empty_like(x) if out is None else out
    _need(y, "out", x.dtype, dev)
    _need_shape(y, "out", x.shape)
    if return_states and states is None:
        states = torch.empty((plan.n_seg, n_heads, d_state, head_dim), dtype=f32, device=dev)
    if states is not None:
        _need(states, "states", f32, dev)
        _need_shape(states, "states", (plan.n_seg, n_heads, d_state, head_dim))
    if init_states is not None:
        _need(init_states, "init_states", f32, dev)
        if tuple(init_states.shape) != (plan.n_roots, n_heads, d_state, head_dim):
            raise ValueError("init_states must be [n_roots, H, d_state, P]")
    lib = load()
    need = int(lib.tree_scan_workspace_bytes(plan.handle, n_heads, d_state, head_dim, int(states is not None)))
    workspace, ws_bytes = _workspace(workspace, need, dev)
    dplan = plan.on_device(dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    p = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    _check(lib.tree_ssd_scan(x.data_ptr(), dt.data_ptr(), A.data_ptr(), B.data_ptr(), C.data_ptr(), p(D),
                             y.data_ptr(), p(init_states), p(states), n, n_groups, n_heads, d_state, head_dim,
                             _dtype_code(x), plan.handle, dplan.data_ptr(), dplan.numel(), p(workspace), ws_bytes,
                             stream))
    if return_states:
        return y, states
    return y
