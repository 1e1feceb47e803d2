"""Calibrate the fork/rescan policy's launch price on this GPU.

    python -m prefix_tree_packed_plan_amd.calibrate_policy [--heads 16 32] [--reps 20]

Times tree_gdn_scan under both schedules on RL-batch-shaped tries (P prompts
of R tokens, each followed by 8 completions of 384 tokens; bf16, d = 128) and
prints one row per trie, then the threshold fork_min_saved_tokens that loses
the least total time over the grid when the policy picks by it (the policy:
fork when the prefix tokens saved reach the threshold per extra launch,
"How a tree runs" on the tree-recurrence 0.1.0 project page).  Inputs are
seeded synthetic tensors made on the device.
"""
from __future__ import annotations

import argparse

import numpy as np


def rl_trie(prompts: int, prompt_len: int, completions: int = 8, completion_len: int = 384):
    parents, lens = [], []
    for _ in range(prompts):
        root = len(parents)
        parents.append(-1)
        lens.append(prompt_len)
        for _ in range(completions):
            parents.append(root)
            lens.append(completion_len)
    return np.array(parents, np.int32), np.array(lens, np.int32)


def time_schedules(parents, lens, h_qk, h_v, reps, device="cuda:0"):
    import torch

    from . import _lib
    from workloads import make_scan_inputs
    n = int(lens.sum())
    t = make_scan_inputs(n, h_qk, h_v, 128, 128, "bf16", device, seed=1)
    plan = _lib.TreePlan(parents, lens, 4)
    o = torch.empty_like(t["v"])
    out = {}
    for sched in ("level", "rescan"):
        def run():
            _lib.tree_gdn_scan(t["q"], t["k"], t["v"], t["g"], t["beta"], plan, out=o, schedule=sched)
        for _ in range(3):
            run()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            run()
        ev[1].record()
        torch.cuda.synchronize()
        out[sched] = ev[0].elapsed_time(ev[1]) / reps
    saved = int(plan.stats["path_tokens"]) - n
    extra = int(plan.stats["n_levels"]) - 1
    return saved, extra, out["level"], out["rescan"]


def best_threshold(rows):
    """The threshold with the least summed loss against the faster schedule
    (rows: saved, extra, level_ms, rescan_ms)."""
    cands = sorted({0} | {r[0] // max(r[1], 1) for r in rows} | {r[0] // max(r[1], 1) + 1 for r in rows})
    def loss(t):
        tot = 0.0
        for saved, extra, lv, rs in rows:
            pick = lv if extra == 0 or saved >= t * extra else rs
            tot += pick - min(lv, rs)
        return tot
    return min(cands, key=lambda t: (loss(t), t)), loss


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--heads", type=int, nargs=2, default=[16, 32], metavar=("H_QK", "H_V"))
    ap.add_argument("--reps", type=int, default=20)
    args = ap.parse_args()
    rows = []
    print("prompts prompt_len saved_tokens extra_launches fork_ms rescan_ms", flush=True)
    for p in (1, 4, 16, 64):
        for r in (16, 64, 256, 1024, 4096):
            parents, lens = rl_trie(p, r)
            row = time_schedules(parents, lens, args.heads[0], args.heads[1], args.reps)
            rows.append(row)
            print(p, r, row[0], row[1], f"{row[2]:.4f}", f"{row[3]:.4f}", flush=True)
    t, loss = best_threshold(rows)
    print(f"best fork_min_saved_tokens = {t} (summed loss {loss(t):.4f} ms; "
          f"always fork: {loss(0):.4f} ms)", flush=True)


if __name__ == "__main__":
    main()
