"""Benchmark: unique tokens/s of the tree conv + tree Gated DeltaNet forward.

    python bench.py [--steps K] [--warmup W] [--config 5] [--no-cpu-baseline]

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
heads of 128; bf16; conv over 8192 channels, width 4).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

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


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("gdn_scan.hip", "gdn_scan_d128.hip", "tree_conv.hip"):
        with open(os.path.join(ROOT, "prefix_tree_packed_plan_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload):
    """Measured HBM bytes per launch from the committed counter summary, or
    None when the summary is missing or the kernels changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(f"{kernel}:{workload}")
    if not entry or entry.get("source_hash") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


def cpu_baseline(wl, budget_s=15.0):
    """The oracle as it stands, on one core, over a bounded sample: whole
    root-to-leaf paths (conv over all channels, the token-by-token recurrence
    over all value heads) in leaf order until about `budget_s` seconds of
    work.  Scaled to the whole job (every path), since the oracle's cost is
    linear in path tokens."""
    import numpy as np  # noqa: F401
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import conv as oconv
    from oracle import gdn as ogdn
    from oracle import trie as otrie

    s = wl.spec
    t = wl.tensors
    w = t["w"].double().cpu().numpy()
    total_path = otrie.path_token_count(wl.parents, wl.seg_lens)
    done_tok, spent, n_paths = 0, 0.0, 0
    with threadpool_limits(1):
        for path in otrie.leaf_paths(wl.parents):
            idx = otrie.path_token_index(path, wl.seg_lens)
            it = torch.as_tensor(idx, device=t["x"].device)
            host = {k: v.index_select(0, it).double().cpu().numpy() for k, v in t.items() if k != "w"}
            t0 = time.perf_counter()
            oconv.conv_on_path(host["x"], w)
            ogdn.gdn_on_path(host["q"], host["k"], host["v"], host["g"], host["beta"])
            spent += time.perf_counter() - t0
            done_tok += len(idx)
            n_paths += 1
            if spent >= budget_s:
                break
    full_s = spent * total_path / done_tok
    return {
        "value": wl.n_tokens / full_s,
        "unit": "unique tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{n_paths} whole root-to-leaf paths ({done_tok} of {total_path} path tokens): conv over all "
                   f"{s.channels} channels and the token-by-token recurrence over all {s.h_v} value heads, "
                   f"{spent:.1f} s on 1 core (fp64 NumPy); scaled linearly to every path"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--schedule", choices=["auto", "level", "rescan"], default="auto",
                    help="scan schedule of the timed step (auto = the fork/rescan policy)")
    ap.add_argument("--no-rescan-compare", action="store_true",
                    help="skip the untimed-by-the-step comparison run of the rescan schedule")
    ap.add_argument("--no-backward", action="store_true", help="skip the separately timed conv and scan backward")
    ap.add_argument("--no-ssd", action="store_true", help="skip the separately timed tree Mamba2 (SSD) scan")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="before timing, run one plain 1 GiB device copy (a counter reference for profiles)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the tree forward here is a single-GPU path "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import prefix_tree_packed_plan_amd as ptp
    from workloads import make_workload

    dev = "cuda:0"
    wl = make_workload(args.config, dev)
    s, t = wl.spec, wl.tensors
    plan = ptp.tree_plan(wl.parents, wl.seg_lens, s.conv_width)
    st = plan.stats
    y = torch.empty_like(t["x"])
    o = torch.empty_like(t["v"])
    lib = ptp.load()
    ws_bytes = int(lib.tree_scan_workspace_bytes(plan.handle, s.h_v, s.d_k, s.d_v, 0))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    plan.on_device(dev)
    sched = plan.choose_schedule() if args.schedule == "auto" else args.schedule
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        del src
    torch.cuda.synchronize()

    def step(ev=None):
        if ev:
            ev[0].record()
        ptp.tree_conv(t["x"], t["w"], plan, out=y)
        if ev:
            ev[1].record()
        ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, out=o, workspace=ws,
                          schedule=sched)
        if ev:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    conv_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    scan_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    ms_per_step = 1e3 * wall / args.steps

    # After the timed steps: the other schedule on the same trie, so the
    # work a fork saves shows up as measured scan time.
    other = None
    if not args.no_rescan_compare:
        alt = "rescan" if sched == "level" else "level"
        reps = max(3, min(args.steps, 10))
        for _ in range(2):
            ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, out=o, workspace=ws,
                              schedule=alt)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            ptp.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, out=o, workspace=ws,
                              schedule=alt)
        ev[1].record()
        torch.cuda.synchronize()
        other = {"schedule": alt, "scan_ms": ev[0].elapsed_time(ev[1]) / reps, "reps": reps}

    # The conv backward on the same trie (timed on its own, outside the step):
    # dy of the conv output -> dx, dw, dbias.
    bwd = None
    if not args.no_backward:
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
    if not args.no_ssd:
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
        ssd = {"tree_ssd_scan": {
            "ms": yms, "unique_tokens_per_s": wl.n_tokens / yms * 1e3, "bytes": sb, "GB/s": sb / yms / 1e6,
            "roofline": {"bound": "hbm", "achieved": sb / yms / 1e6, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": sb / (HBM_PEAK_GBS * 1e9) / (yms * 1e-3)},
            "shape": dict(sh, dtype="bf16"), "launches": st["n_levels"], "reps": reps}}
        del si, yb, ssws

    n = wl.n_tokens
    state_bytes = 2 * st["n_parents"] * s.h_v * s.d_k * s.d_v * 4  # write + read once
    conv_b = n * conv_bytes_per_token(s)
    scan_b = n * scan_bytes_per_token(s) + (state_bytes if sched == "level" else 0)
    n_levels = st["n_levels"] if sched == "level" else 1
    kernels = {
        "tree_conv": {"ms": conv_ms, "bytes": conv_b, "launches": 1,
                      "GB/s": conv_b / conv_ms / 1e6},
        "tree_gdn_scan": {"ms": scan_ms, "bytes": scan_b, "launches": n_levels,
                          "GB/s": scan_b / scan_ms / 1e6},
    }
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    kd = kernels[dom]
    achieved = kd["bytes"] / kd["launches"] / (kd["ms"] / kd["launches"] * 1e-3) / 1e9
    traffic = load_traffic(dom, s.name)
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
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
        },
        "kernels": kernels,
        "roofline_combined_frac": ((conv_b + scan_b) / (HBM_PEAK_GBS * 1e9)) / ((conv_ms + scan_ms) * 1e-3),
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
