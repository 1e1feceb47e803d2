"""Seeded synthetic tries and tensors for the five benchmark workloads.

Workloads (segment lengths in tokens, heads as query/key heads / value heads):

1. tiny:     root 64 -> 2 children of 32 -> 2 leaves of 16 each (7 segments,
             192 tokens); 1/1 heads, d_k = d_v = 32, fp32; conv 96 channels.
2. grpo:     one 2048-token prompt with 8 completions of 1024 tokens
             (10,240 tokens); 16/16 heads, d = 128, bf16; conv 3*16*128.
3. chains:   16 independent roots, lengths uniform in [512, 8192]; 16/32
             heads, d = 128, bf16; conv 2*16*128 + 32*128 = 8192 channels.
4. agentic:  one trie of depth 6 (root depth 0, leaves depth 5), branching
             uniform in {1,2,3} per inner node, lengths uniform [64, 1024].
5. rl_batch: 32 prompts [1024, 4096], 8 completions each [256, 2048]; every
             completion forks with probability 1/4 into 2 continuations
             [128, 512].

All tries are numbered in depth-first pre-order, so parents[i] < i.

Value recipe: q, k ~ N(0,1) L2-normalised per (token, head) in fp32 without
epsilon and then cast; v ~ N(0,1); g = -softplus(N(0,1)) in fp32;
beta = sigmoid(N(0,1)) in fp32; conv input x ~ N(0,1); conv weights with
standard deviation 0.5.  Every tensor has its own generator seeded from
(seed, tensor id), so the draws do not depend on the order of creation.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

# Tensor ids for the per-tensor generators.
_TID = {"q": 1, "k": 2, "v": 3, "g": 4, "beta": 5, "x": 6, "w": 7, "bias": 8,
        "ssd_x": 9, "ssd_dt": 10, "ssd_A": 11, "ssd_B": 12, "ssd_C": 13}


@dataclass(frozen=True)
class ConfigSpec:
    cid: int
    name: str
    h_qk: int
    h_v: int
    d_k: int
    d_v: int
    dtype: str  # "f32" or "bf16"
    channels: int
    conv_width: int = 4


CONFIGS: Dict[int, ConfigSpec] = {
    1: ConfigSpec(1, "tiny", 1, 1, 32, 32, "f32", 96),
    2: ConfigSpec(2, "grpo", 16, 16, 128, 128, "bf16", 3 * 16 * 128),
    3: ConfigSpec(3, "chains", 16, 32, 128, 128, "bf16", 2 * 16 * 128 + 32 * 128),
    4: ConfigSpec(4, "agentic", 16, 32, 128, 128, "bf16", 2 * 16 * 128 + 32 * 128),
    5: ConfigSpec(5, "rl_batch", 16, 32, 128, 128, "bf16", 2 * 16 * 128 + 32 * 128),
}


def _trie_tiny(rng):
    parents = [-1, 0, 1, 1, 0, 4, 4]
    lens = [64, 32, 16, 16, 32, 16, 16]
    return parents, lens


def _trie_grpo(rng):
    return [-1] + [0] * 8, [2048] + [1024] * 8


def _trie_chains(rng):
    lens = rng.integers(512, 8192, size=16, endpoint=True).tolist()
    return [-1] * 16, lens


def _trie_agentic_once(rng):
    parents, lens = [], []

    def node(depth, parent):
        me = len(parents)
        parents.append(parent)
        lens.append(int(rng.integers(64, 1024, endpoint=True)))
        if depth < 5:
            for _ in range(int(rng.integers(1, 3, endpoint=True))):
                node(depth + 1, me)

    node(0, -1)
    return parents, lens


def _trie_rl_batch(rng):
    parents, lens = [], []
    for _ in range(32):
        root = len(parents)
        parents.append(-1)
        lens.append(int(rng.integers(1024, 4096, endpoint=True)))
        for _ in range(8):
            comp = len(parents)
            parents.append(root)
            lens.append(int(rng.integers(256, 2048, endpoint=True)))
            if rng.random() < 0.25:
                for _ in range(2):
                    parents.append(comp)
                    lens.append(int(rng.integers(128, 512, endpoint=True)))
    return parents, lens


def _n_leaves(parents):
    has_child = set(p for p in parents if p >= 0)
    return sum(1 for i in range(len(parents)) if i not in has_child)


def make_trie(cid: int, seed: int = 0):
    """Return (parents, seg_lens, seed_used) as int32 numpy arrays.

    For the agentic trie the seed is stepped until the realisation has
    24k-40k tokens and 28-52 leaves (the stated "~32k tokens, ~40 leaves").
    """
    if cid == 4:
        s = seed
        while True:
            rng = np.random.default_rng([s, 0])
            parents, lens = _trie_agentic_once(rng)
            n = sum(lens)
            if 24_000 <= n <= 40_000 and 28 <= _n_leaves(parents) <= 52:
                break
            s += 1
        return np.asarray(parents, np.int32), np.asarray(lens, np.int32), s
    rng = np.random.default_rng([seed, 0])
    fn = {1: _trie_tiny, 2: _trie_grpo, 3: _trie_chains, 5: _trie_rl_batch}[cid]
    parents, lens = fn(rng)
    return np.asarray(parents, np.int32), np.asarray(lens, np.int32), seed


# ----------------------------------------------------------------------------
# Tensors (torch: the GPU path needs device tensors; CPU tests use device="cpu")
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _gen(device, seed, name):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + _TID[name])
    return g


def _randn(shape, device, seed, name, std=1.0):
    torch = _torch()
    t = torch.randn(shape, generator=_gen(device, seed, name), device=device,
                    dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def _tdtype(dtype):
    torch = _torch()
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def make_scan_inputs(n_tokens, h_qk, h_v, d_k, d_v, dtype, device="cpu", seed=0):
    """q, k [N,H_qk,d_k] and v [N,H_v,d_v] in `dtype`; g, beta [N,H_v] fp32."""
    torch = _torch()
    td = _tdtype(dtype)
    out = {}
    for name, shape in (("q", (n_tokens, h_qk, d_k)), ("k", (n_tokens, h_qk, d_k))):
        t = _randn(shape, device, seed, name)
        t = t / t.norm(dim=-1, keepdim=True)
        out[name] = t.to(td).contiguous()
    out["v"] = _randn((n_tokens, h_v, d_v), device, seed, "v").to(td).contiguous()
    out["g"] = (-torch.nn.functional.softplus(
        _randn((n_tokens, h_v), device, seed, "g"))).contiguous()
    out["beta"] = torch.sigmoid(_randn((n_tokens, h_v), device, seed, "beta")).contiguous()
    return out


def make_conv_inputs(n_tokens, channels, width, dtype, device="cpu", seed=0,
                     with_bias=False):
    """x [N,C] and w [C,W] in `dtype` (w std 0.5); optional bias [C]."""
    td = _tdtype(dtype)
    out = {
        "x": _randn((n_tokens, channels), device, seed, "x").to(td).contiguous(),
        "w": _randn((channels, width), device, seed, "w", std=0.5).to(td).contiguous(),
    }
    if with_bias:
        out["bias"] = _randn((channels,), device, seed, "bias", std=0.5).to(td).contiguous()
    return out


# Mamba2-2.7B-shaped heads for the tree Mamba2 (SSD) scan: 80 heads of 64,
# d_state 128, one B/C group.
SSD_SHAPE = {"n_groups": 1, "n_heads": 80, "d_state": 128, "head_dim": 64}


def make_ssd_inputs(n_tokens, n_groups, n_heads, d_state, head_dim, dtype, device="cpu", seed=0):
    """Mamba2 (SSD) inputs at the ranges of Mamba2's initialisation: x, B, C
    ~ N(0, 1) in `dtype` (x [N,H,P], B and C [N,G,d_state]); dt [N,H] fp32
    log-uniform on [0.001, 0.1] (a step after softplus); A [H] fp32 =
    -exp(U[log 1, log 16]); D [H] fp32 = 1."""
    torch = _torch()
    td = _tdtype(dtype)
    u_dt = torch.rand((n_tokens, n_heads), generator=_gen(device, seed, "ssd_dt"), device=device)
    u_a = torch.rand((n_heads,), generator=_gen(device, seed, "ssd_A"), device=device)
    lo, hi = float(np.log(1e-3)), float(np.log(1e-1))
    return {
        "x": _randn((n_tokens, n_heads, head_dim), device, seed, "ssd_x").to(td).contiguous(),
        "dt": torch.exp(lo + (hi - lo) * u_dt).contiguous(),
        "A": (-torch.exp(u_a * float(np.log(16.0)))).contiguous(),
        "B": _randn((n_tokens, n_groups, d_state), device, seed, "ssd_B").to(td).contiguous(),
        "C": _randn((n_tokens, n_groups, d_state), device, seed, "ssd_C").to(td).contiguous(),
        "D": torch.ones((n_heads,), device=device, dtype=torch.float32),
    }


@dataclass
class Workload:
    spec: ConfigSpec
    parents: np.ndarray
    seg_lens: np.ndarray
    seed: int
    tensors: Dict[str, object] = field(default_factory=dict)

    @property
    def n_tokens(self) -> int:
        return int(self.seg_lens.sum())


def make_workload(cid: int, device: Optional[str] = None, seed: int = 0,
                  conv: bool = True, scan: bool = True) -> Workload:
    """Trie plus (optionally) its tensors on `device` (None: trie only)."""
    spec = CONFIGS[cid]
    parents, lens, used = make_trie(cid, seed)
    wl = Workload(spec, parents, lens, used)
    if device is not None:
        n = wl.n_tokens
        if scan:
            wl.tensors.update(make_scan_inputs(n, spec.h_qk, spec.h_v, spec.d_k,
                                               spec.d_v, spec.dtype, device, seed))
        if conv:
            wl.tensors.update(make_conv_inputs(n, spec.channels, spec.conv_width,
                                               spec.dtype, device, seed))
    return wl

