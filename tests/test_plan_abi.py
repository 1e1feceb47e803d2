"""Host plan and C-ABI checks that need no GPU.

tree_plan is host-only, so the real library is called here; nothing in this
file launches a kernel.  Expected values come from independent walks over the
parent array written in this file or from the oracle's trie helpers.
"""
import ctypes
import json
import os
import re

import numpy as np
import pytest

from oracle import trie as otrie
from oracle.brute import _prev_token_fn
from prefix_tree_packed_plan_amd import _lib
from workloads import CONFIGS, make_trie

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tree_gdn.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tree_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_header_symbol():
    lib = _lib.load()
    names = header_functions()
    assert "tree_plan" in names and "tree_gdn_scan" in names and "tree_conv" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def rand_trie(rng, n_seg, max_len, n_roots=1):
    parents = [-1] * n_roots + [int(rng.integers(0, i)) for i in range(n_roots, n_seg)]
    return np.array(parents, np.int32), rng.integers(1, max_len + 1, n_seg).astype(np.int32)


@pytest.mark.parametrize("cid", sorted(CONFIGS))
def test_plan_stats_match_the_trie(cid):
    parents, lens, _ = make_trie(cid)
    plan = _lib.TreePlan(parents, lens, 4)
    st = plan.stats
    leaves = otrie.leaves_of(parents)
    assert st["n_tokens"] == int(lens.sum())
    assert st["n_seg"] == len(parents)
    assert st["n_leaves"] == len(leaves)
    assert st["n_roots"] == int((parents < 0).sum())
    assert st["n_parents"] == len(parents) - len(leaves)
    assert st["path_tokens"] == otrie.path_token_count(parents, lens)
    assert st["max_path_tokens"] == max(sum(int(lens[s]) for s in p) for p in otrie.leaf_paths(parents))
    assert abs(st["por"] - otrie.por(parents, lens)) < 1e-12


def test_plan_por_printed_example():
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "por_example.json")))
    plan = _lib.TreePlan([-1, 0, 0], [81000, 1000, 1000], 4)
    assert plan.stats["n_tokens"] == gold["n_tree"]
    assert plan.stats["path_tokens"] == gold["n_base"]
    assert round(100 * plan.stats["por"], 1) == gold["por_percent_rounded"]


@pytest.mark.parametrize("W", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_conv_history_is_the_path_history(W, seed):
    """hist[s][W-2-j] must be the packed row j+1 steps before segment s's first
    token along its path (walked token by token); m steps before the root
    it is the code -1 - (r (W-1) + W-1-m) of row W-1-m of root r's context
    (r = the root's rank among the roots in segment order)."""
    rng = np.random.default_rng(seed)
    parents, lens = rand_trie(rng, 50, 4, n_roots=3)
    plan = _lib.TreePlan(parents, lens, W)
    hist = plan.conv_history()
    prev, _, start = _prev_token_fn(parents, lens)
    rank = {r: i for i, r in enumerate(s for s in range(len(parents)) if parents[s] < 0)}
    for s in range(len(parents)):
        root = s
        while parents[root] >= 0:
            root = parents[root]
        j, m = start[s], 0
        for back in range(1, W):
            if j is not None:
                j = prev(j)
            if j is None:
                m += 1
                want = -1 - (rank[root] * (W - 1) + (W - 1 - m))
            else:
                want = j
            assert hist[s, W - 1 - back] == want, (s, back)


def test_levels_respect_depth_and_longest_first():
    rng = np.random.default_rng(4)
    parents, lens = rand_trie(rng, 80, 50, n_roots=2)
    plan = _lib.TreePlan(parents, lens, 4)
    ls, order = plan.levels()
    depth = np.zeros(len(parents), int)
    for i, p in enumerate(parents):
        depth[i] = 0 if p < 0 else depth[p] + 1
    assert sorted(order.tolist()) == list(range(len(parents)))
    assert ls[0] == 0 and ls[-1] == len(parents) and len(ls) == depth.max() + 2
    for lvl in range(len(ls) - 1):
        segs = order[ls[lvl]:ls[lvl + 1]]
        assert np.all(depth[segs] == lvl)
        assert np.all(np.diff(lens[segs]) <= 0)


@pytest.mark.parametrize("parents,lens,code", [
    ([-1, 1], [3, 3], -2),        # self parent
    ([-1, 2, 0], [3, 3, 3], -2),  # parent after child
    ([-1, 0], [3, 0], -2),        # empty segment
    ([-2], [3], -2),              # parent below -1
])
def test_bad_trees_are_rejected(parents, lens, code):
    with pytest.raises(_lib.TreeError) as ei:
        _lib.TreePlan(parents, lens, 4)
    assert ei.value.code == code


def test_argument_errors_need_no_device():
    lib = _lib.load()
    h = ctypes.c_void_p()
    p = np.array([-1], np.int32)
    n = np.array([5], np.int32)
    assert lib.tree_plan(p.ctypes.data, n.ctypes.data, 0, 4, ctypes.byref(h)) == -2
    assert lib.tree_plan(p.ctypes.data, n.ctypes.data, 1, 9, ctypes.byref(h)) == -1
    assert lib.tree_plan(None, n.ctypes.data, 1, 4, ctypes.byref(h)) == -1
    plan = _lib.TreePlan(p, n, 4)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    # token count mismatch
    big = 1 << 20
    assert lib.tree_conv(fake, fake, None, fake, None, None, 6, 8, 1, 0, plan.handle, fake, big, None) == -3
    # bad activation / dtype
    assert lib.tree_conv(fake, fake, None, fake, None, None, 5, 8, 1, 7, plan.handle, fake, big, None) == -1
    assert lib.tree_conv(fake, fake, None, fake, None, None, 5, 8, 5, 0, plan.handle, fake, big, None) == -1
    assert lib.tree_conv(fake, fake, None, fake, None, None, 5, 8, 1, 0, plan.handle, None, big, None) == -1
    # context out aliasing an input
    assert lib.tree_conv(fake, fake, None, ctypes.c_void_p(0x2000), None, fake, 5, 8, 1, 0, plan.handle,
                         fake, big, None) == -1
    scan = lib.tree_gdn_scan
    args = [fake] * 6 + [None, fake]  # q, k, v, g, beta, o, init_states, states
    assert scan(*args, 5, 2, 3, 128, 128, 1.0, 1, 0, plan.handle, fake, big, fake, 1 << 30, None) == -4
    assert scan(*args, 5, 1, 1, 48, 48, 1.0, 1, 0, plan.handle, fake, big, fake, 1 << 30, None) == -4
    assert scan(*args, 5, 1, 1, 128, 128, 1.0, 0, 0, plan.handle, fake, big, fake, 1 << 30, None) == -4
    assert scan(*args, 5, 1, 1, 128, 128, 1.0, 0, 0, plan.handle, fake, big, fake, 1 << 30, None) == -4
    assert scan(*args, 4, 1, 1, 128, 128, 1.0, 1, 0, plan.handle, fake, big, fake, 1 << 30, None) == -3
    assert scan(*args, 5, 1, 1, 128, 128, 1.0, 1, 9, plan.handle, fake, big, fake, 1 << 30, None) == -1
    assert b"schedule" in lib.tree_last_error()


def test_device_plan_must_be_an_upload_of_this_plan():
    """Every entry point rejects, before any launch, a device plan whose byte
    count is below the plan's device size (WORKSPACE) and one that
    tree_plan_upload never filled from this plan (INVALID_ARG), with every
    other argument valid.  No upload can run without a GPU, so here every
    pointer is unknown; the GPU tests cover accepted uploads and a buffer
    uploaded from another plan."""
    lib = _lib.load()
    parents, lens, _ = make_trie(2)
    plan = _lib.TreePlan(parents, lens, 4)
    n = plan.n_tokens
    dbytes = plan.device_bytes()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced
    other, other2 = ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)  # outputs may not alias inputs
    ws = 1 << 40
    calls = {
        "tree_conv": lambda b: lib.tree_conv(fake, fake, None, other, None, None, n, 64, 1, 0, plan.handle,
                                             fake, b, None),
        "tree_conv_backward": lambda b: lib.tree_conv_backward(fake, fake, None, other, None, other2, fake, None,
                                                               None, n, 64, 1, 0, plan.handle, fake, b, fake,
                                                               ws, None),
        "tree_gdn_scan": lambda b: lib.tree_gdn_scan(*([fake] * 6), None, None, n, 16, 16, 128, 128, 1.0, 1, 0,
                                                     plan.handle, fake, b, fake, ws, None),
        "tree_gdn_scan_backward": lambda b: lib.tree_gdn_scan_backward(
            *([fake] * 6), None, None, fake, *([fake] * 5), None, n, 16, 16, 128, 128, 1.0, 1, plan.handle, fake,
            b, fake, ws, None),
        "tree_ssd_scan": lambda b: lib.tree_ssd_scan(fake, fake, fake, fake, fake, None, fake, None, None, n, 1, 8,
                                                     128, 64, 1, plan.handle, fake, b, fake, ws, None),
    }
    for name, call in calls.items():
        assert call(dbytes - 1) == -5, name
        assert b"dplan" in lib.tree_last_error(), name
        assert call(dbytes) == -1, name
        assert b"not an upload of this plan" in lib.tree_last_error(), name
    assert lib.tree_plan_upload(plan.handle, fake, dbytes - 1, None) == -5


def test_tree_workspace_bytes_per_schedule():
    """tree_workspace_bytes(plan, h_v, d_k, d_v, sched): the parent state
    slots under the level schedule, nothing under rescan, auto resolved by
    the fork/rescan policy."""
    lib = _lib.load()
    for cid in (2, 5):
        parents, lens, _ = make_trie(cid)
        plan = _lib.TreePlan(parents, lens, 4)
        slots = plan.stats["n_parents"] * 32 * 128 * 128 * 4
        assert lib.tree_workspace_bytes(plan.handle, 32, 128, 128, _lib.SCHED_LEVEL) == slots
        assert lib.tree_workspace_bytes(plan.handle, 32, 128, 128, _lib.SCHED_RESCAN) == 0
        auto = slots if plan.choose_schedule() == "level" else 0
        assert lib.tree_workspace_bytes(plan.handle, 32, 128, 128, _lib.SCHED_AUTO) == auto
    chain = _lib.TreePlan([-1, 0, 1], [10, 10, 10], 4)
    assert chain.choose_schedule() == "rescan"
    assert lib.tree_workspace_bytes(chain.handle, 4, 32, 32, _lib.SCHED_AUTO) == 0
    assert lib.tree_workspace_bytes(chain.handle, 4, 32, 32, _lib.SCHED_LEVEL) == 2 * 4 * 32 * 32 * 4
    assert lib.tree_workspace_bytes(None, 4, 32, 32, _lib.SCHED_LEVEL) == 0


def test_workspace_size_and_check():
    lib = _lib.load()
    parents, lens, _ = make_trie(2)
    plan = _lib.TreePlan(parents, lens, 4)
    need = lib.tree_scan_workspace_bytes(plan.handle, 16, 128, 128, 0)
    assert need == 1 * 16 * 128 * 128 * 4  # one parent (the prompt)
    assert lib.tree_scan_workspace_bytes(plan.handle, 16, 128, 128, 1) == 0
    fake = ctypes.c_void_p(0x1000)
    n = plan.n_tokens
    rc = lib.tree_gdn_scan(*([fake] * 6), None, None, n, 16, 16, 128, 128, 1.0, 1, 0, plan.handle, fake,
                           1 << 20, fake, need - 1, None)
    assert rc == -5


def test_library_shares_torchs_hip_runtime():
    """The binding loads torch first so that the library's libamdhip64.so.7
    dependency binds to torch's copy: one HIP runtime per process."""
    _lib.load()
    maps = open("/proc/self/maps").read()
    hip = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(hip) == 1, hip


# ------------------------------------------------------------ rescan walks

def _decode(e):
    return (int(e), True) if e >= 0 else (int(~e), False)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_rescan_walks_are_the_leaf_paths_with_one_owner_each(seed):
    rng = np.random.default_rng(30 + seed)
    parents, lens = rand_trie(rng, 60, 40, n_roots=1 + seed)
    plan = _lib.TreePlan(parents, lens, 4)
    off, seg = plan.paths()
    walks = [[_decode(e) for e in seg[off[w]:off[w + 1]]] for w in range(len(off) - 1)]
    want = {tuple(p) for p in otrie.leaf_paths(parents)}
    assert {tuple(s for s, _ in w) for w in walks} == want and len(walks) == len(want)
    assert plan.stats["path_entries"] == sum(len(p) for p in want)
    plen = [sum(int(lens[s]) for s, _ in w) for w in walks]
    assert all(a >= b for a, b in zip(plen, plen[1:])), "longest walk first"
    owners = {}
    for w, walk in enumerate(walks):
        for s, own in walk:
            if own:
                assert s not in owners, f"segment {s} written twice"
                owners[s] = walk[-1][0]
    assert sorted(owners) == list(range(len(parents)))
    # The owner is the lowest-indexed leaf whose root path holds the segment.
    for s in range(len(parents)):
        assert owners[s] == min(p[-1] for p in want if s in p)


def _expected_schedule(parents, lens, t):
    saved = otrie.path_token_count(parents, lens) - int(np.sum(lens))
    depth = np.zeros(len(parents), int)
    for i, p in enumerate(parents):
        depth[i] = 0 if p < 0 else depth[p] + 1
    extra = int(depth.max())
    return "level" if extra == 0 or saved >= t * extra else "rescan"


def test_fork_rescan_policy():
    rng = np.random.default_rng(7)
    cases = [(np.array([-1, 0, 1, 2], np.int32), np.array([50, 9, 70, 3], np.int32)),  # chain
             (np.array([-1, -1, -1], np.int32), np.array([5, 6, 7], np.int32)),          # forest
             (np.array([-1, 0, 0], np.int32), np.array([1000, 10, 10], np.int32))]       # fork
    cases += [rand_trie(rng, 30, 200, n_roots=2) for _ in range(4)]
    cases += [make_trie(c)[:2] for c in sorted(CONFIGS)]
    for parents, lens in cases:
        plan = _lib.TreePlan(parents, lens, 4)
        for t in (0, 1, 10, 999, 1000, 1001, 4096, 1 << 20, 1 << 40):
            assert plan.choose_schedule(t) == _expected_schedule(parents, lens, t), (parents, t)
    chain = _lib.TreePlan([-1, 0, 1], [10, 10, 10], 4)
    assert chain.choose_schedule(1) == "rescan" and chain.choose_schedule(0) == "level"
    lib = _lib.load()
    out = ctypes.c_int32()
    assert lib.tree_plan_choose_schedule(chain.handle, -1, ctypes.byref(out)) == -1


def test_schedule_constants_match_the_header():
    text = open(HEADER).read()
    val = lambda name: int(re.search(rf"#define {name}\s+\(?(-?\d+)", text).group(1))  # noqa: E731
    assert val("TREE_SCHED_LEVEL") == _lib.SCHED_LEVEL
    assert val("TREE_SCHED_RESCAN") == _lib.SCHED_RESCAN
    assert val("TREE_SCHED_AUTO") == _lib.SCHED_AUTO
    assert val("TREE_FORK_MIN_SAVED_TOKENS") == _lib.FORK_MIN_SAVED_TOKENS


@pytest.mark.parametrize("cid", sorted(CONFIGS))
def test_scan_backward_workspace_size_and_checks(cid):
    """Workspace = checkpoint start states (every 8th 16-token chunk of a
    segment) + one start-state
    gradient per segment + the [16, 16] T, KK, QK tiles of every chunk + the
    re-run scratch of the largest level's work-groups (7 states each) (+
    per-value-head dq, dk when more than two value heads share a q/k head;
    two add straight into dq, dk), fp32; undersized workspaces and bad
    arguments are rejected before any device work."""
    lib = _lib.load()
    parents, lens, _ = make_trie(cid)
    s = CONFIGS[cid]
    plan = _lib.TreePlan(parents, lens, 4)
    depth = np.zeros(len(parents), np.int64)
    for i, p in enumerate(parents):
        depth[i] = depth[p] + 1 if p >= 0 else 0
    chunks = [int(sum((lens[i] + 15) // 16 for i in range(len(parents)) if depth[i] == lv))
              for lv in range(int(depth.max()) + 1)]
    dd = s.d_k * s.d_v
    levels = np.bincount(depth)
    total = sum(chunks)

    ckpts = int(sum((int((lens[i] + 15) // 16) + 7) // 8 for i in range(len(parents))))

    def base(h_v):
        return (ckpts + len(parents)) * h_v * dd + total * h_v * 3 * 16 * 16 + int(levels.max()) * h_v * 7 * dd

    want = base(s.h_v)
    if s.h_v > 2 * s.h_qk:
        want += 2 * int(lens.sum()) * s.h_v * s.d_k
    need = lib.tree_gdn_scan_backward_workspace_bytes(plan.handle, s.h_qk, s.h_v, s.d_k, s.d_v)
    assert need == 4 * want
    # Four value heads per q/k head: the per-value-head parts are needed.
    need4 = lib.tree_gdn_scan_backward_workspace_bytes(plan.handle, 1, 4, s.d_k, s.d_v)
    assert need4 == 4 * (base(4) + 2 * int(lens.sum()) * 4 * s.d_k)

    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    bwd = lib.tree_gdn_scan_backward
    n = plan.n_tokens
    dt = 0 if s.dtype == "f32" else 1

    def call(n_tok=n, h_qk=s.h_qk, h_v=s.h_v, d=s.d_k, dtype=dt, ws=need, states=fake):
        return bwd(*([fake] * 6), None, None, states, *([fake] * 5), None, n_tok, h_qk, h_v, d, d, 1.0, dtype,
                   plan.handle, fake, 1 << 20, fake, ws, None)

    assert call(ws=need - 1) == -5
    assert call(n_tok=n + 1) == -3
    assert call(d=48) == -4
    assert call(h_qk=3, h_v=4) == -4
    assert call(dtype=7) == -1
    assert call(states=None) == -1


def test_ssd_scan_argument_checks_need_no_device():
    """tree_ssd_scan validates sizes, head/group counts, dtype, compiled sizes
    and the workspace before any device work."""
    lib = _lib.load()
    parents, lens, _ = make_trie(2)
    plan = _lib.TreePlan(parents, lens, 4)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    n = plan.n_tokens
    need = lib.tree_scan_workspace_bytes(plan.handle, 8, 128, 64, 0)
    assert need == 1 * 8 * 128 * 64 * 4  # one parent state slot per head

    def call(n_tok=n, groups=1, heads=8, d_state=128, head_dim=64, dtype=1, ws=need, states=None, x=fake):
        return lib.tree_ssd_scan(x, fake, fake, fake, fake, None, fake, None, states, n_tok, groups, heads, d_state,
                                 head_dim, dtype, plan.handle, fake, 1 << 20, fake, ws, None)

    assert call(n_tok=n - 1) == -3
    assert call(groups=3) == -4
    assert call(d_state=96) == -4
    assert call(head_dim=128) == -4
    assert call(dtype=5) == -1
    assert call(ws=need - 1) == -5
    assert call(x=None) == -1
    assert b"tree_ssd_scan" in lib.tree_last_error()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without the built library every entry point raises."""
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libtreegdn.so"))
    with pytest.raises(OSError, match="is missing"):
        _lib.load()
    with pytest.raises(OSError, match="is missing"):
        _lib.tree_plan(np.array([-1, 0], np.int32), np.array([3, 2], np.int32), 4)


def test_noalloc_scan_rejects_sizes_beyond_its_scratch_without_a_device():
    """tree_gdn_scan_noalloc checks that the device plan and the parent slots
    fit its static array before touching the device: the RL batch trie's 93
    parent states of 32 heads (186 MiB) exceed TREE_NOALLOC_SCRATCH_BYTES."""
    lib = _lib.load()
    text = open(HEADER).read()
    cap = re.search(r"#define TREE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    cap = int(cap.group(1)) << int(cap.group(2))
    parents, lens, _ = make_trie(5)
    plan = _lib.TreePlan(parents, lens, 4)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced
    need = lib.tree_scan_workspace_bytes(plan.handle, 32, 128, 128, 0)
    assert need + plan.device_bytes() > cap
    rc = lib.tree_gdn_scan_noalloc(*([fake] * 6), None, None, plan.n_tokens, 16, 32, 128, 128, 1.0, 1,
                                   _lib.SCHED_LEVEL, plan.handle, None)
    assert rc == -5 and b"static maximum" in lib.tree_last_error()
    # the usual argument checks come first
    assert lib.tree_gdn_scan_noalloc(*([fake] * 6), None, None, plan.n_tokens + 1, 16, 32, 128, 128, 1.0, 1,
                                     _lib.SCHED_LEVEL, plan.handle, None) == -3
