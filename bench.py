"""Benchmark: unique tokens/s of the tree conv + tree Gated DeltaNet forward.

    python bench.py [--steps K] [--warmup W] [--config 1..5] [--no-cpu-baseline]

One step is one pass of the whole hot path over the resident synthetic batch:
tree_conv over x [N, C] and tree_gdn_scan over q, k, v, g, beta under the
fork/rescan policy (--schedule auto; the RL batch trie forks: one launch per
trie level).  After the timed steps the other schedule is timed on the same
trie (fork_vs_rescan in the output).  Inputs are generated on the GPU before timing; W untimed
steps, then K timed steps between two synchronisations.  Kernel times come
from HIP events recorded on the stream the kernels are launched on.

Prints ONE JSON line (rank 0, one GPU).  The default workload is the large RL
batch trie (32 prompts x 8 completions, a quarter of the completions forking
into 2 continuations; N = 428,843 unique tokens; 16 query/key and 32 value
heads of 128; bf16; conv over 8192 channels, width 4).  --config 1..4 times
the other workloads the same way; below 2 GB of step traffic a 1 GiB scratch
write separates the steps so that they read from HBM, and the step time is
then the kernels' HIP events.  The CPU baseline runs the oracle on every core
the process may use, over a bounded sample of whole paths.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published


def scan_bwd_flops_per_token(s):
    """Algorithmic flops per token of the scan backward: per value head, the
    ten [16, d] x [d, d] contractions of a 16-token chunk (forward re-run:
    K S0 and K^T U; backward: K S0, Q S0, K dS1, dO S0^T, dV S0^T, U dS1^T,
    Q^T dO and K^T dV), 2 * 16 * d_k * d_v each, per 16 tokens; the
    [16, 16]-sized products (about 14% more) are not counted."""
    return s.h_v * 10 * 2 * s.d_k * s.d_v


def scan_bytes_per_token(s):
    """Algorithmic HBM bytes per token of the scan: read q, k (H_qk*d_k bf16
    each), v (H_v*d_v), g and beta (H_v fp32 each); write o (H_v*d_v)."""
    e = 2 if s.dtype == "bf16" else 4
    return 2 * s.h_qk * s.d_k * e + 2 * s.h_v * s.d_v * e + 2 * s.h_v * 4


def conv_bytes_per_token(s):
    """Read x and write y, C channels each."""
    e = 2 if s.dtype == "bf16" else 4
    return 2 * s.channels * e


# Sources whose change invalidates a kernel's committed counter summary.
FWD_SOURCES = ("gdn_scan.hip", "gdn_scan_d128.hip", "tree_conv.hip")
SSD_SOURCES = ("ssd_scan.hip", "chunk_mfma.hpp")


def kernel_source_hash(files=FWD_SOURCES):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "prefix_tree_packed_plan_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload, files=FWD_SOURCES):
    """The committed counter summary of `kernel` on `workload` (bytes per
    launch, launches per step), or None when the summary is missing or the
    kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(f"{kernel}:{workload}")
    if not entry or entry.get("source_hash") != kernel_source_hash(files):
        return None
    return entry


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_task(a):
    """One CPU-baseline task (run in a worker process): the oracle's conv over
    a block of channels, or its token-by-token recurrence over a block of
    value heads, on one root-to-leaf path.  Returns the seconds it took."""
    import time as _t

    from threadpoolctl import threadpool_limits

    from oracle import conv as oconv
    from oracle import gdn as ogdn

    kind, arrays = a
    with threadpool_limits(1):
        t0 = _t.perf_counter()
        if kind == "conv":
            oconv.conv_on_path(arrays[0], arrays[1])
        else:
            ogdn.gdn_on_path(*arrays)
        return _t.perf_counter() - t0


def _path_tasks(wl, path, head_blocks, chan_blocks):
    """The oracle work of one path, split into (kind, host arrays) tasks."""
    import torch

    from oracle import trie as otrie

    t = wl.tensors
    s = wl.spec
    idx = torch.as_tensor(otrie.path_token_index(path, wl.seg_lens), device=t["x"].device)
    # fp32 host copies (the inputs are bf16 or fp32, so exact); the oracle
    # itself computes in fp64
    host = {k: v.index_select(0, idx).float().cpu().numpy() for k, v in t.items() if k != "w"}
    w = t["w"].float().cpu().numpy()
    grp = s.h_v // s.h_qk
    tasks = []
    for c0, c1 in chan_blocks:
        tasks.append(("conv", (np.ascontiguousarray(host["x"][:, c0:c1]), w[c0:c1])))
    for h0, h1 in head_blocks:
        q0, q1 = h0 // grp, (h1 - 1) // grp + 1
        tasks.append(("gdn", (host["q"][:, q0:q1], host["k"][:, q0:q1], host["v"][:, h0:h1], host["g"][:, h0:h1],
                              host["beta"][:, h0:h1])))
    return tasks, int(idx.numel())


def cpu_baseline(wl, budget_tokens_per_core=2500):
    """The oracle as it stands (fp64 NumPy, the conv and the token-by-token
    recurrence on every root-to-leaf path) on the host's cores: one worker
    process per core the process may use, BLAS threads 1, tasks = (path x
    block of value heads) and (path x block of conv channels).  A bounded
    sample of whole paths (in leaf order, about budget_tokens_per_core path
    tokens per core) is timed and scaled to every path, since the oracle's
    cost is linear in path tokens.  A single-core figure is timed on the
    GRPO group trie (its first path)."""
    import multiprocessing as mp

    import numpy as np  # noqa: F401

    from oracle import trie as otrie
    from workloads import make_workload

    cores = len(os.sched_getaffinity(0))
    s = wl.spec
    grp = s.h_v // s.h_qk
    hb = max(grp, (s.h_v // cores // grp) * grp or grp)  # value heads per task: whole q/k groups
    head_blocks = [(h, min(h + hb, s.h_v)) for h in range(0, s.h_v, hb)]
    cb = 1024
    chan_blocks = [(c, min(c + cb, s.channels)) for c in range(0, s.channels, cb)]
    total_path = otrie.path_token_count(wl.parents, wl.seg_lens)
    tasks, done_tok, n_paths = [], 0, 0
    for path in otrie.leaf_paths(wl.parents):
        tt, L = _path_tasks(wl, path, head_blocks, chan_blocks)
        tasks += tt
        done_tok += L
        n_paths += 1
        if done_tok >= budget_tokens_per_core * cores:
            break
    pool = mp.get_context("spawn").Pool(cores)
    try:
        tiny = ("conv", (np.zeros((4, 8), np.float32), np.zeros((8, 4), np.float32)))
        pool.map(_oracle_task, [tiny] * cores, chunksize=1)  # workers started, imports done
        t0 = time.perf_counter()
        cpu_s = sum(pool.map_async(_oracle_task, tasks, chunksize=1).get(900))
        wall = time.perf_counter() - t0
    finally:
        pool.terminate()
        pool.join()
    full_wall = wall * total_path / done_tok
    # single core, GRPO group trie (16/16 heads of 128, C = 6144), first path
    g2 = make_workload(2, "cpu")
    path2 = otrie.leaf_paths(g2.parents)[0]
    t2, L2 = _path_tasks(g2, path2, [(0, g2.spec.h_v)], [(0, g2.spec.channels)])
    one = sum(_oracle_task(a) for a in t2)
    return {
        "value": wl.n_tokens / full_wall,
        "unit": "unique tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{n_paths} whole root-to-leaf paths ({done_tok} of {total_path} path tokens; conv over all "
                   f"{s.channels} channels, the token-by-token recurrence over all {s.h_v} value heads), "
                   f"{len(tasks)} tasks on {cores} worker processes (fp64 NumPy, BLAS threads 1): {wall:.1f} s wall, "
                   f"{cpu_s:.1f} s of task time; scaled linearly to every path"),
        "cpu_model": _cpu_model(),
        "wall_s_sample": wall,
        "wall_s_full_job_projected": full_wall,
        "path_tokens_per_s": total_path / full_wall,
        "single_core_grpo_path_tokens_per_s": L2 / one,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5,
                    help="workload: 1 tiny, 2 GRPO group, 3 chains, 4 agentic trie, 5 RL batch trie (default)")
    ap.add_argument("--schedule", choices=["auto", "level", "rescan"], default="auto",
                    help="scan schedule of the timed step (auto = the fork/rescan policy)")
    ap.add_argument("--no-rescan-compare", action="store_true",
                    help="skip the untimed-by-the-step comparison run of the rescan schedule")
    ap.add_argument("--no-backward", action="store_true", help="skip the separately timed conv and scan backward")
    ap.add_argument("--no-ssd", action="store_true", help="skip the separately timed tree Mamba2 (SSD) scan")
    ap.add_argument("--extras", action="store_true",
                    help="time the backward and the SSD scan on workloads other than the RL batch trie too")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="before timing, run one plain 1 GiB device copy (a counter reference for profiles)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the tree forward here is a single-GPU path "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    extras = args.config == 5 or args.extras

    import torch

    import prefix_tree_packed_plan_amd as ptp
    from workloads import make_workload

    dev = "cuda:0"
    wl = make_workload(args.config, dev)
    s, t = wl.spec, wl.tensors
    lib = ptp.load()
    # Host plan build, timed on its own (median of 5 builds; excluded from the step).
    builds = []
    for _ in range(5):
        t0 = time.perf_counter()
        plan = ptp.tree_plan(wl.parents, wl.seg_lens, s.conv_width)
        builds.append(time.perf_counter() - t0)
    plan_build_ms = 1e3 * sorted(builds)[len(builds) // 2]
    st = plan.stats
    y = torch.empty_like(t["x"])
    o = torch.empty_like(t["v"])
    ws_bytes = int(lib.tree_scan_workspace_bytes(plan.handle, s.h_v, s.d_k, s.d_v, 0))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    # Plan upload (host-to-device copy of the plan's device mirror into a
    # buffer allocated beforehand), timed from the host around the call and a
    # synchronisation, median of 5.
    plan.on_device(dev)
    ubuf = torch.empty(plan.device_bytes(), dtype=torch.uint8, device=dev)
    ustream = torch.cuda.current_stream(ubuf.device)
    uploads = []
    for _ in range(5):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        rc = lib.tree_plan_upload(plan.handle, ubuf.data_ptr(), ubuf.numel(), ustream.cuda_stream)
        ustream.synchronize()
        uploads.append(time.perf_counter() - t0)
        if rc != 0:
            raise RuntimeError(f"tree_plan_upload failed: {rc}")
    plan_upload_ms = 1e3 * sorted(uploads)[len(uploads) // 2]
    del ubuf
    sched = plan.choose_schedule() if args.schedule == "auto" else args.schedule
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        del src

    n = wl.n_tokens
    state_bytes = 2 * st["n_parents"] * s.h_v * s.d_k * s.d_v * 4  # write + read once
    conv_b = n * conv_bytes_per_token(s)
    scan_b = n * scan_bytes_per_token(s) + (state_bytes if sched == "level" else 0)
    # Below 2 GB the step's inputs would stay in the last-level cache from one
    # step to the next: write a 1 GiB scratch buffer between steps (outside
    # the kernels' events) so that every step reads from HBM.
    flush = None
    if conv_b + scan_b < (2 << 30):
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(ev=None, k=0):
        if flush is not None:
            flush.fill_(k & 0xFF)
        if ev:
            ev[0].record()
        ptp.tree_conv(t["x"], t["w"], plan, out=y)
        if ev:
            ev[1].record()
        ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, out=o, workspace=ws,
                          schedule=sched)
        if ev:
            ev[2].record()

    for k in range(args.warmup):
        step(k=k)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k], k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    conv_t = [e[0].elapsed_time(e[1]) for e in events]
    scan_t = [e[1].elapsed_time(e[2]) for e in events]
    conv_ms = sum(conv_t) / args.steps
    scan_ms = sum(scan_t) / args.steps
    if flush is None:
        ms_per_step = 1e3 * wall / args.steps
        timing = "wall clock over the timed steps (synchronised on both sides)"
    else:
        # the flush writes sit between the steps: the step time is the events'
        ms_per_step = conv_ms + scan_ms
        timing = ("HIP events around the conv and the scan of each step; a 1 GiB scratch write between steps "
                  f"(working set {(conv_b + scan_b) / 1e9:.3f} GB < 2 GB); wall clock incl. the writes "
                  f"{1e3 * wall / args.steps:.3f} ms per step")

    # After the timed steps: the other schedule on the same trie, so the
    # work a fork saves shows up as measured scan time.
    other = None
    if not args.no_rescan_compare and st["n_levels"] > 1:
        alt = "rescan" if sched == "level" else "level"
        reps = max(3, min(args.steps, 10))
        for _ in range(2):
            ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, out=o, workspace=ws,
                              schedule=alt)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for r in range(reps):
            if flush is not None:
                flush.fill_(r & 0xFF)
            ev[r][0].record()
            ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, out=o, workspace=ws,
                              schedule=alt)
            ev[r][1].record()
        torch.cuda.synchronize()
        other = {"schedule": alt, "scan_ms": sum(e[0].elapsed_time(e[1]) for e in ev) / reps, "reps": reps}

    # The conv backward on the same trie (timed on its own, outside the step):
    # dy of the conv output -> dx, dw, dbias.
    bwd = None
    if extras and not args.no_backward:
        dy = torch.empty_like(t["x"]).normal_()
        bias0 = torch.zeros(s.channels, dtype=t["x"].dtype, device=dev)
        dx = torch.empty_like(t["x"])
        bws = torch.empty(max(int(lib.tree_conv_backward_workspace_bytes(plan.handle, s.channels)), 1),
                          dtype=torch.uint8, device=dev)
        for _ in range(2):
            ptp.tree_conv_backward(t["x"], t["w"], dy, plan, bias=bias0, dx=dx, workspace=bws)
        reps = max(3, min(args.steps, 10))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            ptp.tree_conv_backward(t["x"], t["w"], dy, plan, bias=bias0, dx=dx, workspace=bws)
        ev[1].record()
        torch.cuda.synchronize()
        bms = ev[0].elapsed_time(ev[1]) / reps
        bb = 3 * wl.n_tokens * conv_bytes_per_token(s) // 2  # read x and dy, write dx
        bwd = {"tree_conv_backward": {"ms": bms, "bytes": bb, "GB/s": bb / bms / 1e6,
                                      "roofline_frac": bb / (HBM_PEAK_GBS * 1e9) / (bms * 1e-3), "reps": reps}}
        del dy, dx, bws
        # The scan backward: do of the scan output -> dq, dk, dv, dg, dbeta,
        # from the forward's segment states.
        states = torch.empty((st["n_seg"], s.h_v, s.d_k, s.d_v), dtype=torch.float32, device=dev)
        ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, out=o, states=states,
                          schedule="level")
        do = torch.empty_like(t["v"]).normal_()
        sws = torch.empty(int(lib.tree_gdn_scan_backward_workspace_bytes(plan.handle, s.h_qk, s.h_v, s.d_k, s.d_v)),
                          dtype=torch.uint8, device=dev)
        sargs = (t["q"], t["k"], t["v"], t["g"], t["beta"], do, plan, states)
        ptp.tree_gdn_scan_backward(*sargs, workspace=sws)
        reps = 3
        ev[0].record()
        for _ in range(reps):
            ptp.tree_gdn_scan_backward(*sargs, workspace=sws)
        ev[1].record()
        torch.cuda.synchronize()
        sms = ev[0].elapsed_time(ev[1]) / reps
        fl = wl.n_tokens * scan_bwd_flops_per_token(s)
        bwd["tree_gdn_scan_backward"] = {
            "ms": sms, "unique_tokens_per_s": wl.n_tokens / sms * 1e3, "flops": fl, "TFLOP/s": fl / sms / 1e9,
            # The dense products run on bf16 MFMA with fp32 operands split into
            # hi + lo (two or three passes each); fp32-accurate results.
            "roofline": {"bound": "mfma", "dtype": "bf16 (fp32 operands as hi + lo)",
                         "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": fl / sms / 1e9 / BF16_MFMA_PEAK_TFLOPS,
                         "frac_of_fp32_peak": fl / sms / 1e9 / FP32_MFMA_PEAK_TFLOPS},
            "workspace_GiB": sws.numel() / 2**30, "reps": reps}
        del states, do, sws

    # The tree Mamba2 (SSD) scan on the same trie, Mamba2-2.7B-shaped heads
    # (timed on its own, outside the step).
    ssd = None
    if extras and not args.no_ssd:
        from workloads import SSD_SHAPE, make_ssd_inputs
        sh = SSD_SHAPE
        si = make_ssd_inputs(wl.n_tokens, sh["n_groups"], sh["n_heads"], sh["d_state"], sh["head_dim"], "bf16", dev)
        yb = torch.empty_like(si["x"])
        ssws = torch.empty(max(int(lib.tree_scan_workspace_bytes(plan.handle, sh["n_heads"], sh["d_state"],
                                                                  sh["head_dim"], 0)), 1), dtype=torch.uint8, device=dev)
        sargs = (si["x"], si["dt"], si["A"], si["B"], si["C"], plan)
        for _ in range(2):
            ptp.tree_ssd_scan(*sargs, D=si["D"], out=yb, workspace=ssws)
        reps = max(3, min(args.steps, 10))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            ptp.tree_ssd_scan(*sargs, D=si["D"], out=yb, workspace=ssws)
        ev[1].record()
        torch.cuda.synchronize()
        yms = ev[0].elapsed_time(ev[1]) / reps
        # x, y (H * P bf16 each), B, C (G * d_state bf16 each), dt (H fp32) per
        # token, plus one write and one read of each parent's state.
        per_tok = 2 * sh["n_heads"] * sh["head_dim"] * 2 + 2 * sh["n_groups"] * sh["d_state"] * 2 + sh["n_heads"] * 4
        sb = wl.n_tokens * per_tok + 2 * st["n_parents"] * sh["n_heads"] * sh["d_state"] * sh["head_dim"] * 4
        sc = load_traffic("tree_ssd_scan", s.name, SSD_SOURCES)
        st_b = None if sc is None else sc["bytes_per_launch"] * sc["launches"]
        ssd = {"tree_ssd_scan": {
            "ms": yms, "unique_tokens_per_s": wl.n_tokens / yms * 1e3, "bytes": sb, "GB/s": sb / yms / 1e6,
            "roofline": {"bound": "hbm", "achieved": sb / yms / 1e6, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": sb / (HBM_PEAK_GBS * 1e9) / (yms * 1e-3),
                         "traffic_per_call": st_b,
                         "traffic_over_algorithmic": None if st_b is None else st_b / sb},
            "shape": dict(sh, dtype="bf16"), "launches": st["n_levels"], "reps": reps}}
        del si, yb, ssws

    n_levels = st["n_levels"] if sched == "level" else 1
    kernels = {
        "tree_conv": {"ms": conv_ms, "ms_median": statistics.median(conv_t), "ms_min": min(conv_t),
                      "bytes": conv_b, "launches": 1, "GB/s": conv_b / conv_ms / 1e6},
        "tree_gdn_scan": {"ms": scan_ms, "ms_median": statistics.median(scan_t), "ms_min": min(scan_t),
                          "bytes": scan_b, "launches": n_levels, "GB/s": scan_b / scan_ms / 1e6},
    }
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    kd = kernels[dom]
    # Algorithmic bytes per launch over the mean launch time (the same as the
    # per-step ratio when a step has several launches).
    achieved = kd["bytes"] / kd["launches"] / (kd["ms"] / kd["launches"] * 1e-3) / 1e9
    counters = load_traffic(dom, s.name)
    roofline = {
        "bound": "hbm",
        "kernel": dom,
        "achieved": achieved,
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": achieved / HBM_PEAK_GBS,
        # counter-measured HBM bytes per launch (rocprofv3 FETCH_SIZE and
        # WRITE_SIZE, scaled by a plain copy's reading), null when the kernel
        # sources changed since they were taken
        "traffic": None if counters is None else counters["bytes_per_launch"],
        "traffic_per_step": None if counters is None else counters["bytes_per_launch"] * counters["launches"],
        "algorithmic_bytes_per_launch": kd["bytes"] / kd["launches"],
        "algorithmic_bytes_per_step": kd["bytes"],
        "traffic_over_algorithmic": (None if counters is None
                                     else counters["bytes_per_launch"] * counters["launches"] / kd["bytes"]),
    }
    out = {
        "metric": "unique tokens/sec of tree conv+GDN forward",
        "value": n / (ms_per_step * 1e-3),
        "unit": "unique tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic",
        "config": {
            "workload": (f"{s.name}: {st['n_seg']} segments, {st['n_levels']} levels, {st['n_leaves']} leaves, "
                         f"N={n} unique tokens ({st['path_tokens']} path tokens), heads {s.h_qk} qk / {s.h_v} v, "
                         f"d_k=d_v={s.d_k}, conv C={s.channels} W={s.conv_width}"),
            "n_unique_tokens": n,
            "path_tokens": st["path_tokens"],
            "work_saved_vs_rescan": st["path_tokens"] / n,
            "por": st["por"],
            "scan_schedule": sched,
            "parallelism": "1 GPU",
        },
        "timing": timing,
        # per-step HIP event times (conv + scan) over the timed steps
        "event_ms_per_step": {"mean": conv_ms + scan_ms,
                              "median": statistics.median([a + b for a, b in zip(conv_t, scan_t)]),
                              "min": min(a + b for a, b in zip(conv_t, scan_t))},
        "roofline": roofline,
        "kernels": kernels,
        "roofline_combined_frac": ((conv_b + scan_b) / (HBM_PEAK_GBS * 1e9)) / ((conv_ms + scan_ms) * 1e-3),
        "plan": {"build_ms": plan_build_ms, "upload_ms": plan_upload_ms, "device_bytes": plan.device_bytes(),
                 "note": "host plan build and its upload into an allocated buffer (medians of 5), outside the timed steps"},
    }
    if bwd is not None:
        out["backward"] = bwd
    if ssd is not None:
        out["ssd"] = ssd
    if other is not None:
        fork_ms = scan_ms if sched == "level" else other["scan_ms"]
        rescan_ms = other["scan_ms"] if sched == "level" else scan_ms
        out["fork_vs_rescan"] = {"fork_scan_ms": fork_ms, "rescan_scan_ms": rescan_ms,
                                 "measured_speedup": rescan_ms / fork_ms,
                                 "path_tokens_over_n": st["path_tokens"] / n,
                                 "rescan_reps": other["reps"]}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
