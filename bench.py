"""Benchmark of shared-prompt tree attention, forward + backward, on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole path over one batch of synthetic replay
trees: prompt prefill, response replay forward, replay backward (prompt
seeds summed over every branch) and prefill backward.  Inputs are resident
in HBM before the timed region.  The metric is useful tree-masked TFLOP/s:
14 * head_dim FLOPs (4d forward, 10d backward) per valid (query row, key)
pair and query head, divided by the step time.

Prints one JSON line.  Besides the headline numbers it carries:
  step_ms_median     median step time of a second pass that also times
                     each entry point (the headline is the mean over the
                     timed steps)
  breakdown_ms       time per entry point (HIP events between the calls)
  roofline           the dominant kernel's own duration (HIP events recorded
                     by the library around that kernel) against the bf16
                     MFMA peak (and, as frac_of_measured_ceiling, against
                     the random-operand rate of mfma_ceiling below); per
                     launch, its measured HBM bytes, the algorithmic bytes
                     and the achieved HBM bandwidth
  flattened_baseline the same attention computed the way flattened context
                     parallelism does it: every (prompt, response) pair as
                     its own causal sequence, with the same kernels
  cpu_baseline       the float64 oracle on a bounded sample, host cores
  mfma_ceiling       measured after the timed work: the GPU's sustained dense
                     bf16 MFMA rate on register operands, constant and random
                     (data like the attention operands), and each kernel's
                     rate over the random-operand figure
  also               the same measurement for further workloads (response-heavy
                     and long-mixed by default; long-mixed with 3 timed steps)

Other modes print one JSON line of their own instead: --dq-ab (the two dQ
strategies), --split-sweep and --tile-split-sweep (the data the replay
load-balancing models are fitted to), --mfma-ceiling (the sustained bf16
MFMA rate of the GPU on register operands); --summarize writes profiles/
summaries from rocprofv3 output.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12  # 256 CUs x 2.4 GHz x 4096 flop/clk/CU
HBM_GBPS = 8000.0

# Algorithmic FLOPs per valid pair and query head, per head_dim, of each
# main kernel: forward S and PV; dQ kernel recomputes S and dP and forms dQ;
# dK/dV kernel recomputes S and dP and forms dV and dK.  With the fused dQ
# strategy the dK/dV kernel also forms dQ (10) and no dQ kernel runs.
KERNEL_FLOPS_PER_PAIR_DIM = {"fwd": 4, "dq": 6, "dkv": 8}
FUSED_FLOPS_PER_PAIR_DIM = {"fwd": 4, "dq": 0, "dkv": 10}


def flops_per_pair_dim(kind, fused):
    return (FUSED_FLOPS_PER_PAIR_DIM if fused else KERNEL_FLOPS_PER_PAIR_DIM)[kind]


ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
def traffic_file(workload):
    """Where the HBM bytes per launch measured on a workload are stored."""
    return os.path.join(PROFILES, f"roofline_traffic_{workload}.json")
# Sources each main kernel is built from; a stored traffic figure is only
# reported while these are unchanged.
KERNEL_SOURCES = {
    "fwd": ["attn_fwd.hip", "device_common.h"],
    "dq": ["attn_bwd.hip", "device_common.h"],
    "dkv": ["attn_bwd.hip", "device_common.h"],
}
KERNEL_SYMBOLS = {"fwd": "fwd_kernel", "dq": "dq_kernel", "dkv": "dkv_kernel"}


def kernel_source_hash(kind):
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "shared_prompt_tree_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_workload(command):
    """The workload a profiled bench.py command ran (its --workload, else the
    default)."""
    import re

    m = re.search(r"--workload[ =](\S+)", command or "")
    return m.group(1) if m else "prompt_heavy"


def stored_traffic(kind, workload):
    """HBM bytes per launch measured by rocprofv3 for this kernel, if the
    measurement was taken on this workload and the current sources; else
    None."""
    try:
        with open(traffic_file(workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload:
        return None
    k = rec.get("kernels", {}).get(kind)
    if not k or k.get("source_hash") != kernel_source_hash(kind):
        return None
    return k.get("hbm_bytes_per_launch")


def stored_launch_traffic(kind, workload):
    """Measured HBM (read, write) bytes of each launch of a main kernel in one
    step, in call order, from the stored profile of this workload and the
    current sources; None when there is none.  The profiled run times one
    step twice, so its launches repeat the step's sequence."""
    try:
        with open(traffic_file(workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(kind)
    if rec.get("workload") != workload or not k or k.get("source_hash") != kernel_source_hash(kind):
        return None
    r, w = k.get("read_bytes", []), k.get("write_bytes", [])
    if len(r) < 2 or len(r) != len(w):
        return None
    # launches c = 0, 1 of every step, averaged over the profiled steps
    return [(sum(r[c::2]) / len(r[c::2]), sum(w[c::2]) / len(w[c::2])) for c in range(2)]


# Which entry point issues launch c (0, 1) of a main kernel in one step.
LAUNCH_CALLS = {"fwd": ("prefill", "replay_fwd"), "dq": ("replay_bwd", "prefill_bwd"),
                "dkv": ("replay_bwd", "prefill_bwd")}


def algorithmic_bytes(tree, kind, call, fused=False):
    """Least HBM traffic of one launch: every operand read once and every
    result written once (the pre-transposed copies and work lists the
    kernels also read are not counted).
      fwd prefill     Q, K, V in; O, LSE out (prompt)
      fwd replay      Q_R, K_R, V_R, K_P, V_P in; O_R, LSE_R out
      dq              Q, dO, LSE, D of the query rows and the K, V they read
                      in; dQ out
      dkv replay_bwd  Q_R, dO_R, LSE_R, D_R and K, V of prompt and responses
                      in; dK_R, dV_R (I/O dtype) and the float32 prompt seeds
                      out
      dkv prefill_bwd Q_P, dO_P, LSE_P, D_P, K_P, V_P and the float32 seeds
                      in; dK_P, dV_P out
      (fused dQ strategy: the dK/dV launch also writes dQ of its rows once)"""
    esz = 4 if tree.dtype == "f32" else 2
    hq, hkv, d = tree.hq, tree.hkv, tree.d
    tp, tr = tree.prompt_tokens, tree.resp_tokens
    q_rows = lambda n: n * hq * d * esz       # Q, O, dO or dQ of n tokens
    kv_rows = lambda n: n * hkv * d * esz     # K, V, dK or dV of n tokens
    seeds = tp * hkv * d * 4
    rows = tp if call in ("prefill", "prefill_bwd") else tr
    if kind == "fwd":
        keys = tp if call == "prefill" else tp + tr
        return q_rows(rows) + 2 * kv_rows(keys) + q_rows(rows) + rows * hq * 4
    if kind == "dq":
        keys = tp if call == "prefill_bwd" else tp + tr
        return 2 * q_rows(rows) + 2 * rows * hq * 4 + 2 * kv_rows(keys) + q_rows(rows)
    dq_out = q_rows(rows) if fused else 0
    if call == "replay_bwd":
        return (2 * q_rows(tr) + 2 * tr * hq * 4 + 2 * kv_rows(tp + tr) + 2 * kv_rows(tr)
                + 2 * seeds + dq_out)
    return (2 * q_rows(tp) + 2 * tp * hq * 4 + 2 * kv_rows(tp) + 2 * seeds + 2 * kv_rows(tp)
            + dq_out)


def launch_report(tree, kind, ms, stored, fused=(False, False)):
    """Per launch of the dominant kernel in one step: its own duration and
    FLOP rate, its measured HBM bytes (rocprofv3 counters of the stored
    profile, null without one), the algorithmic bytes and the achieved HBM
    bandwidth."""
    from shared_prompt_tree_amd import workloads as wl

    pc = wl.pair_counts(tree)
    pairs = {"prefill": pc["prefill"], "prefill_bwd": pc["prefill"],
             "replay_fwd": pc["replay_prompt"] + pc["replay_own"],
             "replay_bwd": pc["replay_prompt"] + pc["replay_own"]}
    out = []
    for c, call in enumerate(LAUNCH_CALLS[kind]):
        fz = kind != "fwd" and fused[c]
        flops = pairs[call] * tree.hq * tree.d * flops_per_pair_dim(kind, fz)
        alg = algorithmic_bytes(tree, kind, call, fz)
        rec = {"call": call, "ms": round(ms[c], 4),
               "tflops": round(flops / (ms[c] * 1e-3) / 1e12, 2) if ms[c] > 0 else None,
               "algorithmic_bytes": int(alg), "hbm_bytes": None, "hbm_gbps": None,
               "hbm_over_algorithmic": None}
        if stored is not None:
            hbm = stored[c][0] + stored[c][1]
            rec["hbm_bytes"] = int(round(hbm))
            rec["hbm_read_bytes"] = int(round(stored[c][0]))
            rec["hbm_gbps"] = round(hbm / (ms[c] * 1e-3) / 1e9, 1) if ms[c] > 0 else None
            rec["hbm_over_algorithmic"] = round(hbm / alg, 2) if alg > 0 else None
        out.append(rec)
    return out


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="prompt_heavy")
    p.add_argument("--also", default="response_heavy,long_mixed",
                   help="comma-separated further workloads measured the same way "
                        "('none' to skip); each is timed with at most ALSO_STEPS[name] "
                        "steps and ALSO_WARMUP[name] warmup steps")
    p.add_argument("--no-flattened", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-workers", type=int, default=0)
    p.add_argument("--summarize", nargs="+", metavar="DIR",
                   help="write profiles/ summaries from rocprofv3 output directories "
                        "(kernel-trace stats, FETCH_SIZE and WRITE_SIZE passes) and exit")
    p.add_argument("--summarize-command", default="",
                   help="the profiling command recorded in the summaries")
    p.add_argument("--dq-strategy", choices=["auto", "separate", "fused"], default="auto",
                   help="how the backward forms dQ (auto: the library's cost model)")
    p.add_argument("--dq-ab", action="store_true",
                   help="instead of the benchmark: time the two backward calls with each dQ "
                        "strategy, alternating, on each workload of --workload and --also, "
                        "and print one JSON line")
    p.add_argument("--split-sweep", action="store_true",
                   help="instead of the benchmark: time the replay forward and backward "
                        "calls of a few few-row replay shapes at forced prompt-column chunk "
                        "counts (the data the column-split model's constants are fitted "
                        "to), and print one JSON line")
    p.add_argument("--tile-split-sweep", action="store_true",
                   help="instead of the benchmark: time the replay backward of short-prompt, "
                        "many-branch shapes at forced prompt-tile split targets (the data the "
                        "split rule is fitted to), and print one JSON line")
    p.add_argument("--mfma-ceiling", action="store_true",
                   help="instead of the benchmark: the sustained dense bf16 MFMA rate of "
                        "this GPU on register operands (libmfmaceiling.so), with constant and "
                        "with random bf16 operands, and print one JSON line")
    p.add_argument("--ceiling-seconds", type=float, default=2.0,
                   help="how long the MFMA-rate measurement runs each operand kind (after "
                        "the timed work in a benchmark run, 0 to skip; or in --mfma-ceiling)")
    p.add_argument("--copy-calibration-mib", type=int, default=1024,
                   help="size of a plain device copy run after the timed region, used to "
                        "scale HBM byte counters in profiling runs (0 to skip)")
    return p.parse_args()


# Further workloads whose step takes over a second are timed with fewer
# steps, so the default run stays within a few minutes.
ALSO_STEPS = {"long_mixed": 3}
ALSO_WARMUP = {"long_mixed": 1}


def fail(msg):
    print(msg, file=sys.stderr, flush=True)
    sys.exit(2)


DQ_STRATEGY_CODES = {"auto": 0, "separate": 1, "fused": 2}
DQ_STRATEGY_NAMES = {1: "separate", 2: "fused"}


def measure_workload(name, steps, warmup, flattened=True, fms_hint=None, dq_strategy="auto"):
    import torch

    from shared_prompt_tree_amd import ops
    from shared_prompt_tree_amd import workloads as wl

    spec = wl.SPECS[name]
    tree = wl.make_tree(spec)
    dev = torch.device("cuda:0")
    t = wl.make_tensors(tree, spec.seed, device=dev, value_scale=spec.value_scale)
    prob = ops.TreeProblem.from_tree(tree, device=dev,
                                     dq_strategy=DQ_STRATEGY_CODES[dq_strategy])
    # the strategy each backward call uses (the cost model's choice for auto)
    used = {call: ops.tree_attn_dq_strategy_of(prob, op)
            for call, op in (("replay_bwd", ops.OP_REPLAY_BWD),
                             ("prefill_bwd", ops.OP_PREFILL_BWD))}
    fused = tuple(used[c] == ops.DQ_FUSED for c in ("replay_bwd", "prefill_bwd"))
    torch.cuda.synchronize()

    def step():
        return ops.tree_attention_forward_backward(prob, t)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # whole steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3 / steps
    ms = ev0.elapsed_time(ev1) / steps

    # per entry point, and every main kernel's own duration
    names = ["prefill", "replay_fwd", "replay_bwd", "prefill_bwd"]
    part = {n: 0.0 for n in names}
    kern = {k: 0.0 for k in ("fwd", "dq", "dkv")}
    kinds = {"fwd": ops.KERNEL_FWD, "dq": ops.KERNEL_DQ, "dkv": ops.KERNEL_DKV}

    def new_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    per_step = []
    kern_launch = {(k, c): 0.0 for k in kern for c in range(2)}
    for _ in range(steps):
        evs = [new_event() for _ in range(5)]
        # kernel events: fwd in prefill and replay_fwd, dq and dkv in both bwd calls
        kev = {(k, c): (new_event(), new_event()) for k in kern for c in range(2)}
        torch.cuda.synchronize()
        evs[0].record()
        ops.tree_attn_set_kernel_events(kinds["fwd"], *kev[("fwd", 0)])
        o_p, lse_p = ops.tree_attn_prefill(prob, t["q_p"], t["k_p"], t["v_p"])
        evs[1].record()
        ops.tree_attn_set_kernel_events(kinds["fwd"], *kev[("fwd", 1)])
        o_r, lse_r = ops.tree_attn_replay_fwd(prob, t["k_p"], t["v_p"], t["q_r"], t["k_r"],
                                              t["v_r"])
        evs[2].record()
        ops.tree_attn_set_kernel_events(kinds["dq"], *kev[("dq", 0)])
        ops.tree_attn_set_kernel_events(kinds["dkv"], *kev[("dkv", 0)])
        dq_r, dk_r, dv_r, dks, dvs = ops.tree_attn_replay_bwd(
            prob, t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], o_r, lse_r, t["do_r"])
        evs[3].record()
        ops.tree_attn_set_kernel_events(kinds["dq"], *kev[("dq", 1)])
        ops.tree_attn_set_kernel_events(kinds["dkv"], *kev[("dkv", 1)])
        ops.tree_attn_prefill_bwd(prob, t["q_p"], t["k_p"], t["v_p"], o_p, lse_p, t["do_p"],
                                  dks, dvs)
        evs[4].record()
        for k in kinds.values():
            ops.tree_attn_set_kernel_events(k)
        torch.cuda.synchronize()
        per_step.append(evs[0].elapsed_time(evs[4]))
        for i, n in enumerate(names):
            part[n] += evs[i].elapsed_time(evs[i + 1]) / steps
        for (k, c), (a, b) in kev.items():
            kern[k] += a.elapsed_time(b) / steps
            kern_launch[(k, c)] += a.elapsed_time(b) / steps

    pairs = wl.pair_counts(tree)
    useful = wl.useful_flops(tree)
    hq, d = tree.hq, tree.d
    rep = {
        "ms_per_step": ms,
        "wall_ms_per_step": wall_ms,
        "useful_tflop_per_step": useful / 1e12,
        "tflops": useful / (ms * 1e-3) / 1e12,
        # median of the per-step times of the second (per entry point) pass
        "step_ms_median": round(sorted(per_step)[len(per_step) // 2], 4),
        "breakdown_ms": {k: round(v, 4) for k, v in part.items()},
        "kernel_ms": {k: round(v, 4) for k, v in kern.items()},
    }
    # algorithmic FLOPs of each kernel kind over one step (the dQ and dK/dV
    # kernels per backward call, by the dQ strategy it used)
    call_pairs = {"prefill": pairs["prefill"],
                  "replay": pairs["replay_prompt"] + pairs["replay_own"]}
    kflops = {"fwd": pairs["tree"] * hq * d * 4}
    for k in ("dq", "dkv"):
        kflops[k] = sum(call_pairs[c] * hq * d * flops_per_pair_dim(k, fz)
                        for c, fz in (("replay", fused[0]), ("prefill", fused[1])))
    dom = max(kern, key=kern.get)
    achieved = kflops[dom] / (kern[dom] * 1e-3) / 1e12
    stored = stored_launch_traffic(dom, name)
    fpd = sorted({flops_per_pair_dim(dom, fz) for fz in fused})
    rep["dq_strategy"] = {c: DQ_STRATEGY_NAMES[v] for c, v in used.items()}
    # largest-first placement of the unsplit replay items of one head group /
    # kv head onto one XCD's 32 CUs: makespan over mean load (1 = perfect)
    rep["replay_schedule_balance"] = {k: round(wl.schedule_balance(tree, k), 4)
                                      for k in ("dq", "dkv")}
    rep["roofline"] = {
        "kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
        "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": None if stored is None else round(sum(r + w for r, w in stored) / len(stored)),
        "flops_per_pair_per_dim": fpd[0] if len(fpd) == 1 else fpd,
        "launches_per_step": 2, "ms_per_step": round(kern[dom], 4),
        "launches": launch_report(tree, dom, [kern_launch[(dom, c)] for c in range(2)], stored,
                                  fused),
    }
    rep["kernel_tflops"] = {k: round(kflops[k] / (kern[k] * 1e-3) / 1e12, 2) if kern[k] > 0
                            else None for k in kern}
    # forward (prefill + replay_fwd) and backward (replay_bwd + prefill_bwd)
    # on their own useful FLOPs (4d and 10d per pair), and the whole step
    # with 12d per pair (no recompute counted) beside the 14d convention
    base = pairs["tree"] * hq * d
    fwd_ms = part["prefill"] + part["replay_fwd"]
    bwd_ms = part["replay_bwd"] + part["prefill_bwd"]
    rep["phases"] = {}
    for ph, pms, f in (("fwd", fwd_ms, 4), ("bwd", bwd_ms, 10)):
        tf = base * f / (pms * 1e-3) / 1e12 if pms > 0 else 0.0
        rep["phases"][ph] = {"ms": round(pms, 4), "useful_tflops": round(tf, 2),
                             "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}
    rep["useful_tflops_12d"] = round(base * 12 / (ms * 1e-3) / 1e12, 2)

    if flattened:
        ftree = wl.flattened_tree(tree)
        ft = wl.flatten_tensors(tree, t)
        fprob = ops.TreeProblem.from_tree(ftree, device=dev)

        def fstep():
            o, l = ops.tree_attn_prefill(fprob, ft["q_p"], ft["k_p"], ft["v_p"])
            ops.tree_attn_prefill_bwd(fprob, ft["q_p"], ft["k_p"], ft["v_p"], o, l, ft["do_p"])

        fstep()
        torch.cuda.synchronize()
        fsteps = max(1, min(steps, 5 if fms_hint is None else fms_hint))
        ev0.record()
        for _ in range(fsteps):
            fstep()
        ev1.record()
        torch.cuda.synchronize()
        fms = ev0.elapsed_time(ev1) / fsteps
        rep["flattened_baseline"] = {
            "ms_per_step": round(fms, 3),
            "useful_tflops": round(useful / (fms * 1e-3) / 1e12, 2),
            "work_ratio": round(pairs["flattened"] / pairs["tree"], 3),
            "speedup_of_tree": round(fms / ms, 3),
            "note": "same kernels over one causal sequence per (prompt, response) pair; "
                    "same tree-masked numerator",
        }
        del ft
    rep["config"] = {
        "workload": name, "groups": tree.n_groups, "q_heads": tree.hq, "kv_heads": tree.hkv,
        "head_dim": tree.d, "prompt_len": spec.prompt_len, "branches_per_group": spec.g,
        "resp_len": list(spec.resp), "prompt_tokens": tree.prompt_tokens,
        "response_tokens": tree.resp_tokens, "seed": spec.seed,
        "valid_pairs_per_head": pairs["tree"],
    }
    rep["_tree"] = tree
    rep["_tensors"] = t
    return rep


def dq_strategy_ab(names, steps):
    """Same-box A/B of the dQ strategies: on each workload, the replay and
    prefill backward calls timed with HIP events, the separate pass and the
    fused kernel alternating (two rounds each, ``steps`` calls per round, the
    per-strategy figure is the mean of its rounds).  Useful backward TFLOP/s
    count 10d per valid pair and query head.  The float32 dQ atomic bytes of
    the fused kernel (d floats per query row and key tile it reads) are
    reported with the rate they were added at."""
    import torch

    from shared_prompt_tree_amd import ops
    from shared_prompt_tree_amd import workloads as wl

    dev = torch.device("cuda:0")
    out = {"metric": "dQ strategy A/B: backward call times", "unit": "ms", "rounds": 2,
           "steps": steps, "workloads": []}
    for name in names:
        spec = wl.SPECS[name]
        tree = wl.make_tree(spec)
        t = wl.make_tensors(tree, spec.seed, device=dev, value_scale=spec.value_scale)
        prob = ops.TreeProblem.from_tree(tree, device=dev)
        o_p, lse_p = ops.tree_attn_prefill(prob, t["q_p"], t["k_p"], t["v_p"])
        o_r, lse_r = ops.tree_attn_replay_fwd(prob, t["k_p"], t["v_p"], t["q_r"], t["k_r"],
                                              t["v_r"])
        pc = wl.pair_counts(tree)
        useful = {"replay_bwd": (pc["replay_prompt"] + pc["replay_own"]) * tree.hq * tree.d * 10,
                  "prefill_bwd": pc["prefill"] * tree.hq * tree.d * 10}
        visits = {"replay_bwd": 0, "prefill_bwd": 0}
        for P, rs in zip(tree.prompt_lens, tree.resp_lens):
            visits["prefill_bwd"] += causal_tile_visits(P)
            for r in rs:
                visits["replay_bwd"] += r * (-(-P // 256)) + causal_tile_visits(r)
        times = {st: {"replay_bwd": [], "prefill_bwd": []} for st in ("separate", "fused")}
        for _ in range(2):
            for st in ("separate", "fused"):
                prob.dq_strategy = DQ_STRATEGY_CODES[st]
                e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                res = ops.tree_attn_replay_bwd(prob, t["k_p"], t["v_p"], t["q_r"], t["k_r"],
                                               t["v_r"], o_r, lse_r, t["do_r"])
                ops.tree_attn_prefill_bwd(prob, t["q_p"], t["k_p"], t["v_p"], o_p, lse_p,
                                          t["do_p"], res[3], res[4])
                torch.cuda.synchronize()
                tr = tp = 0.0
                for _ in range(steps):
                    e[0].record()
                    res = ops.tree_attn_replay_bwd(prob, t["k_p"], t["v_p"], t["q_r"],
                                                   t["k_r"], t["v_r"], o_r, lse_r, t["do_r"])
                    e[1].record()
                    ops.tree_attn_prefill_bwd(prob, t["q_p"], t["k_p"], t["v_p"], o_p, lse_p,
                                              t["do_p"], res[3], res[4])
                    e[2].record()
                    torch.cuda.synchronize()
                    tr += e[0].elapsed_time(e[1]) / steps
                    tp += e[1].elapsed_time(e[2]) / steps
                times[st]["replay_bwd"].append(tr)
                times[st]["prefill_bwd"].append(tp)
                print(f"[ab] {name} {st}: replay_bwd {tr:.3f} ms, prefill_bwd {tp:.3f} ms",
                      file=sys.stderr, flush=True)
        rec = {"workload": name}
        for st, calls in times.items():
            rec[st] = {}
            for call, ts in calls.items():
                ms = sum(ts) / len(ts)
                r = {"ms": round(ms, 4), "rounds_ms": [round(x, 4) for x in ts],
                     "useful_tflops": round(useful[call] / (ms * 1e-3) / 1e12, 1)}
                if st == "fused":
                    ab = visits[call] * tree.hq * tree.d * 4
                    r["atomic_bytes"] = int(ab)
                    r["atomic_tbps"] = round(ab / (ms * 1e-3) / 1e12, 3)
                rec[st][call] = r
        prob.dq_strategy = 0
        rec["auto_chooses"] = {c: DQ_STRATEGY_NAMES[ops.tree_attn_dq_strategy_of(prob, op)]
                               for c, op in (("replay_bwd", ops.OP_REPLAY_BWD),
                                             ("prefill_bwd", ops.OP_PREFILL_BWD))}
        out["workloads"].append(rec)
        del t, o_p, lse_p, o_r, lse_r, res
        torch.cuda.empty_cache()
    return out


# Replay shapes where the prompt column split matters (32 query / 8 kv heads,
# head_dim 128, bf16): (prompt, branch lengths).  The 520-workgroup shape is
# two full rounds of 256 CUs plus 8 workgroups; 264 is one round plus 8.
SPLIT_SWEEP_SHAPES = {
    "13x260 behind 32768 (520 wg)": (32768, [260] * 13),
    "8x512 behind 32768 (prompt-heavy replay, 512 wg)": (32768, [512] * 8),
    "8x64 behind 131072 (64 wg)": (131072, [64] * 8),
    "16x200 behind 65536 (512 wg)": (65536, [200] * 16),
    "11x150 behind 2048 (264 wg)": (2048, [150] * 11),
    # short prompt, many long branches: the prompt key tiles are split over
    # branch ranges in the backward (not a column-split shape)
    "24x4096 behind 256": (256, [4096] * 24),
}
SPLIT_SWEEP_S = (1, 2, 3, 4, 6, 8, 12, 16, 24, 32)


def split_sweep(steps):
    """Replay forward and backward (separate dQ pass) call times at forced
    prompt-column chunk counts S, and the makespan model's own choice."""
    import torch

    from shared_prompt_tree_amd import ops
    from shared_prompt_tree_amd import workloads as wl

    dev = torch.device("cuda:0")
    out = {"metric": "replay call times by prompt-column chunks", "unit": "ms",
           "steps": steps, "shapes": []}
    for label, (P, rs) in SPLIT_SWEEP_SHAPES.items():
        tree = wl.Tree([P], [rs], 32, 8, 128, "bf16")
        t = wl.make_tensors(tree, 1, device=dev)
        prob = ops.TreeProblem.from_tree(tree, device=dev, dq_strategy=ops.DQ_SEPARATE)
        auto = {"replay_fwd": ops.tree_attn_prompt_col_splits_of(prob, ops.OP_REPLAY_FWD),
                "replay_bwd": ops.tree_attn_prompt_col_splits_of(prob, ops.OP_REPLAY_BWD)}
        rec = {"shape": label, "prompt": P, "branches": rs, "model_chooses": auto, "by_s": {}}
        for S in SPLIT_SWEEP_S:
            if S > max(1, -(-P // 64)):
                continue
            prob.prompt_col_splits = S
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]

            def call():
                o, lse = ops.tree_attn_replay_fwd(prob, t["k_p"], t["v_p"], t["q_r"], t["k_r"],
                                                  t["v_r"])
                e[1].record()
                ops.tree_attn_replay_bwd(prob, t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"],
                                         o, lse, t["do_r"])

            call()
            torch.cuda.synchronize()
            tf = tb = 0.0
            for _ in range(steps):
                e[0].record()
                call()
                e[2].record()
                torch.cuda.synchronize()
                tf += e[0].elapsed_time(e[1]) / steps
                tb += e[1].elapsed_time(e[2]) / steps
            rec["by_s"][S] = {"replay_fwd_ms": round(tf, 4), "replay_bwd_ms": round(tb, 4)}
            print(f"[sweep] {label} S={S}: fwd {tf:.3f} ms, bwd {tb:.3f} ms", file=sys.stderr,
                  flush=True)
        out["shapes"].append(rec)
        del t
        torch.cuda.empty_cache()
    return out


# Short-prompt, many-branch replays: a prompt key tile reads every response
# row of its group, so it is split over branch ranges.  (prompt, [branch
# lengths per group]) with 32 query / 8 kv heads, head_dim 128, bf16; the
# response-heavy workload itself is measured too.
TILE_SPLIT_SHAPES = {
    "24x4096 behind 256": (256, [[4096] * 24]),
    "2 groups of 32x1024 behind 512": (512, [[1024] * 32, [1024] * 32]),
    "16x2048 behind 1024": (1024, [[2048] * 16]),
    "8 groups of 8x512 behind 128": (128, [[512] * 8] * 8),
}
# split rule targets tried: max(longest branch, rows read by all key tiles x
# Hkv / slots) for these slot counts, and no split
TILE_SPLIT_SLOTS = (64, 128, 256, 512, 1024, 2048, 4096)


def key_rows_total(tree):
    """Rows read by all key-stationary replay items of one kv head: each own
    tile the rows of its branch at or after it, each prompt tile every row
    of its group."""
    total = 0
    for p, rs in zip(tree.prompt_lens, tree.resp_lens):
        for r in rs:
            n = -(-r // 256)
            total += n * r - 256 * n * (n - 1) // 2
        total += -(-p // 256) * sum(rs)
    return total


def mfma_ceiling(seconds):
    """Sustained dense bf16 MFMA rate on register operands: the instruction
    rate (constant operands) and what the power limit allows on data like
    the attention operands (random bf16 values of variance ~1).  The second
    is the ceiling the kernels' matrix work runs against."""
    import ctypes

    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "shared_prompt_tree_amd",
                        "lib", "libmfmaceiling.so")
    if not os.path.exists(path):
        fail(f"{path} is missing: build it with python -m shared_prompt_tree_amd.build")
    lib = ctypes.CDLL(path)
    lib.mfma_ceiling_run.argtypes = [ctypes.c_int, ctypes.c_double,
                                     ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int)]
    lib.mfma_ceiling_run.restype = ctypes.c_int
    out = {"metric": "sustained dense bf16 MFMA rate, register operands, 2 waves/SIMD",
           "unit": "TFLOP/s", "peak": round(PEAK_BF16_TFLOPS, 1), "seconds_each": seconds}
    for kind, rnd in (("constant", 0), ("random", 1)):
        tf, first, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int()
        rc = lib.mfma_ceiling_run(rnd, seconds, ctypes.byref(tf), ctypes.byref(first),
                                  ctypes.byref(n))
        if rc != 0:
            fail(f"mfma_ceiling_run({kind}) failed with {rc}")
        out[kind] = {"tflops": round(tf.value, 1),
                     "pct_of_peak": round(100 * tf.value / PEAK_BF16_TFLOPS, 1),
                     "first_launch_tflops": round(first.value, 1), "launches": n.value}
        print(f"[ceiling] {kind} operands: {tf.value:.1f} TFLOP/s "
              f"({100 * tf.value / PEAK_BF16_TFLOPS:.1f}% of peak; first launch "
              f"{first.value:.1f}) over {n.value} launches", file=sys.stderr, flush=True)
    return out


def tile_split_sweep(steps):
    """Replay backward call times at forced prompt-tile split targets, and
    the rule's own choice."""
    import torch

    from shared_prompt_tree_amd import ops
    from shared_prompt_tree_amd import workloads as wl

    dev = torch.device("cuda:0")
    out = {"metric": "replay backward call time by prompt-tile split target", "unit": "ms",
           "steps": steps, "shapes": []}
    shapes = dict(TILE_SPLIT_SHAPES)
    shapes["response_heavy"] = None
    for label, shp in shapes.items():
        if shp is None:
            tree = wl.make_tree(wl.SPECS["response_heavy"])
        else:
            tree = wl.Tree([shp[0]] * len(shp[1]), shp[1], 32, 8, 128, "bf16")
        t = wl.make_tensors(tree, 2, device=dev)
        prob = ops.TreeProblem.from_tree(tree, device=dev, dq_strategy=ops.DQ_SEPARATE)
        o, lse = ops.tree_attn_replay_fwd(prob, t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"])
        longest = max((r for rs in tree.resp_lens for r in rs), default=1)
        total = key_rows_total(tree)
        targets = {f"slots {n}": max(longest, -(-total * tree.hkv // n)) for n in TILE_SPLIT_SLOTS}
        targets["no split"] = max(sum(rs) for rs in tree.resp_lens)
        rec = {"shape": label, "rule_splits": ops.tree_attn_prompt_tile_splits_of(prob),
               "by_target": {}}
        for name, tgt in targets.items():
            prob.prompt_tile_split_rows = int(tgt)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ops.tree_attn_replay_bwd(prob, t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], o,
                                     lse, t["do_r"])
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                ops.tree_attn_replay_bwd(prob, t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"],
                                         o, lse, t["do_r"])
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            rec["by_target"][name] = {"rows": int(tgt),
                                      "splits": ops.tree_attn_prompt_tile_splits_of(prob),
                                      "replay_bwd_ms": round(ms, 4)}
            print(f"[tile-sweep] {label} {name} (target {tgt}, splits "
                  f"{rec['by_target'][name]['splits']}): {ms:.3f} ms", file=sys.stderr, flush=True)
        out["shapes"].append(rec)
        del t, o, lse
        torch.cuda.empty_cache()
    return out


def causal_tile_visits(n, tile=256):
    """Key tiles read by the rows of an n-token causal segment:
    sum over k = 1..n of ceil(k / tile)."""
    m, q = divmod(n, tile)
    return tile * m * (m + 1) // 2 + q * (m + 1)


def cpu_baseline(tree, t, workers):
    """The float64 oracle on a bounded sample of the workload: for one query
    head per worker, the flattened (prompt, first branch) sequence of group 0,
    evaluated on its last 16384 prompt rows and its first 512 response rows
    (the whole key range each), in a process pool."""
    import multiprocessing as mp

    import numpy as np
    import torch

    import oracle  # the oracle is only used for this baseline

    g, i = 0, int(tree.group_branch_cu[0])
    P = int(tree.prompt_cu[1])
    r0, r1 = int(tree.resp_cu[i]), int(tree.resp_cu[i + 1])
    n_resp = min(512, r1 - r0)
    rows = np.concatenate([np.arange(max(0, P - 16384), P), np.arange(P, P + n_resp)])
    heads = list(range(min(workers, tree.hq)))
    seqs = []
    for h in heads:
        kv = h * tree.hkv // tree.hq

        def cat(a, b, hh):
            return torch.cat([t[a][:P, hh], t[b][r0:r1, hh]]).to("cpu", torch.float64).numpy()

        seqs.append((cat("q_p", "q_r", h), cat("k_p", "k_r", kv), cat("v_p", "v_r", kv),
                     cat("do_p", "do_r", h)))
    scale = 1.0 / math.sqrt(tree.d)
    global _CPU_SEQS, _CPU_ROWS, _CPU_SCALE
    _CPU_SEQS, _CPU_ROWS, _CPU_SCALE = seqs, rows, scale
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(len(heads)) as pool:
        pool.map(_cpu_unit, range(len(heads)))
    dt = time.perf_counter() - t0
    pairs = int(sum(int(r) + 1 for r in rows)) * len(heads)
    flops = pairs * tree.d * 14
    return {
        "value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": len(heads),
        "kind": "oracle", "seconds": round(dt, 2),
        "sample": f"{len(heads)} query heads x {len(rows)} rows (last {P - int(rows[0])} "
                  f"prompt rows, first {n_resp} response rows of branch 0, group 0) of the "
                  f"flattened sequence, full key range per row, forward+backward, float64",
    }


_CPU_SEQS = _CPU_ROWS = _CPU_SCALE = None


def _cpu_unit(k):
    from threadpoolctl import threadpool_limits

    import oracle

    q, kk, v, do = _CPU_SEQS[k]
    with threadpool_limits(1):
        oracle.causal_unit(q, kk, v, do, _CPU_SCALE, rows=_CPU_ROWS)
    return k


def _csv_rows(dirs, suffix):
    import csv
    import glob

    out = []
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True):
            with open(f) as fh:
                out.extend(csv.DictReader(fh))
    return out


def summarize(dirs, command):
    """profiles/ summaries from rocprofv3 CSV output (kernel_stats,
    kernel_trace and counter_collection files)."""
    os.makedirs(PROFILES, exist_ok=True)
    lines = []
    stats = _csv_rows(dirs, "_kernel_stats.csv")
    if stats:
        lines.append("kernel                      calls   avg ms    total ms   share")
        for r in stats:
            name = r["Name"]
            short = next((k for k, v in KERNEL_SYMBOLS.items() if v in name), None)
            label = short or name.split("(")[0][:26]
            if short == "fwd":  # the 12-wave and 8-wave launches of the forward kernel
                label += " (12 waves)" if ("Li12E" in name or ", 12>" in name) else " (8 waves)"
            lines.append(f"{label:26s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e6:8.3f} "
                         f"{float(r['TotalDurationNs']) / 1e6:10.3f}  {float(r['Percentage']):5.1f}%")
    counters = {}
    for r in _csv_rows(dirs, "_counter_collection.csv"):
        counters.setdefault(r["Counter_Name"], []).append(r)
    traffic = {}
    calib = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = counters.get(ctr, [])
        copy = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        big = max(copy) if copy else 0.0
        # the calibration copy moves 1 GiB = 1048576 KiB each way
        calib[ctr] = 1048576.0 / big if big > 0 else None
        for kind, sym in KERNEL_SYMBOLS.items():
            vals = [float(r["Counter_Value"]) for r in rows if sym in r["Kernel_Name"]]
            if vals and calib[ctr]:
                traffic.setdefault(kind, {})[ctr] = [v * 1024 * calib[ctr] for v in vals]
    if traffic:
        lines.append("")
        lines.append("HBM bytes per launch (KiB counter x 1024 x calibration), launches in order:")
        lines.append(f"calibration from a 1 GiB device copy: FETCH_SIZE x{calib['FETCH_SIZE']:.3f}, "
                     f"WRITE_SIZE x{calib['WRITE_SIZE']:.3f}")
        rec = {"kernels": {}, "calibration": calib, "command": command,
               "workload": profiled_workload(command)}
        for kind, d in traffic.items():
            f = d.get("FETCH_SIZE", [])
            w = d.get("WRITE_SIZE", [])
            lines.append(f"{kind:4s} read  GB: " + " ".join(f"{x / 1e9:.3f}" for x in f))
            lines.append(f"{kind:4s} write GB: " + " ".join(f"{x / 1e9:.3f}" for x in w))
            if f and w:
                per = (sum(f) + sum(w)) / max(len(f), len(w))
                rec["kernels"][kind] = {"hbm_bytes_per_launch": round(per),
                                        "source_hash": kernel_source_hash(kind),
                                        "read_bytes": [round(x) for x in f],
                                        "write_bytes": [round(x) for x in w]}
        with open(traffic_file(rec["workload"]), "w") as fh:
            json.dump(rec, fh, indent=1)
    other = {c: v for c, v in counters.items() if c not in ("FETCH_SIZE", "WRITE_SIZE")}
    if other:
        dispatched = [(kind, sym) for kind, sym in KERNEL_SYMBOLS.items()
                      if any(sym in r["Kernel_Name"] for rows in other.values() for r in rows)]
        if dispatched:
            lines.append("")
            lines.append("counter totals per kernel (summed over dispatches):")
        for kind, sym in dispatched:
            row = []
            for c in sorted(other):
                v = sum(float(r["Counter_Value"]) for r in other[c] if sym in r["Kernel_Name"])
                row.append(f"{c}={v:.4g}")
            lines.append(f"{kind}: " + " ".join(row))
        if "GRBM_GUI_ACTIVE" in other:
            # Engine clock while each kernel ran: GRBM_GUI_ACTIVE sums the
            # active cycles of the 8 XCDs at the engine clock, over the
            # dispatch's own start/end timestamps (ns).  The plain copy is a
            # reference that does not load the matrix units.
            rows = other["GRBM_GUI_ACTIVE"]
            if rows and "Start_Timestamp" in rows[0]:
                lines.append("")
                lines.append("engine clock while the kernel ran (GRBM_GUI_ACTIVE / 8 / dispatch "
                             "time), GHz:")
                for kind, sym in list(KERNEL_SYMBOLS.items()) + [
                        ("copy", "copyBuffer"), ("mfma_loop_constant", "mfma_loop_constant"),
                        ("mfma_loop_random", "mfma_loop_random")]:
                    rs = [r for r in rows if sym in r["Kernel_Name"]]
                    if kind == "copy" and rs:  # the 1 GiB calibration copy only
                        rs = [max(rs, key=lambda r: int(r["End_Timestamp"]) -
                                  int(r["Start_Timestamp"]))]
                    ns = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rs)
                    if ns > 0:
                        cyc = sum(float(r["Counter_Value"]) for r in rs) / 8
                        lines.append(f"{kind}: {cyc / ns:.3f} over {len(rs)} dispatches, "
                                     f"{ns / 1e6:.3f} ms")
        need = ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY")
        if all(c in other for c in need):
            # Per-wave time split: waiting on dependencies (waitcnt, barrier),
            # ready but not issued (units busy with other waves), issuing.
            def tot(c, sym):
                return sum(float(r["Counter_Value"]) for r in other[c] if sym in r["Kernel_Name"])
            lines.append("")
            lines.append("share of wave time (SQ_WAVE_CYCLES): waiting on dependencies "
                         "(SQ_WAIT_ANY), ready but not issued (SQ_WAIT_INST_ANY), issuing "
                         "(SQ_ACTIVE_INST_ANY; with SQ_ACTIVE_INST_SCA, its scalar share):")
            for kind, sym in dispatched:
                w = tot("SQ_WAVE_CYCLES", sym)
                if w <= 0:
                    continue
                act = tot("SQ_ACTIVE_INST_ANY", sym)
                sca = (f" (scalar {tot('SQ_ACTIVE_INST_SCA', sym) / act:.2f} of it)"
                       if "SQ_ACTIVE_INST_SCA" in other and act > 0 else "")
                lines.append(f"{kind}: wait {tot('SQ_WAIT_ANY', sym) / w:.2f}, wait for issue "
                             f"{tot('SQ_WAIT_INST_ANY', sym) / w:.2f}, issuing {act / w:.2f}{sca}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in other and "GRBM_GUI_ACTIVE" in other:
            # GRBM_GUI_ACTIVE sums the active cycles of the 8 XCDs; each of the
            # 1024 SIMDs can keep its matrix unit busy for all of them.
            lines.append("")
            lines.append("MFMA busy share of SIMD cycles while the GPU was active "
                         "(SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 * 1024)):")
            for kind, sym in KERNEL_SYMBOLS.items():
                busy = sum(float(r["Counter_Value"]) for r in other["SQ_VALU_MFMA_BUSY_CYCLES"]
                           if sym in r["Kernel_Name"])
                act = sum(float(r["Counter_Value"]) for r in other["GRBM_GUI_ACTIVE"]
                          if sym in r["Kernel_Name"])
                if act > 0:
                    lines.append(f"{kind}: {busy / (act / 8 * 1024):.3f}")
    head = ["rocprofv3 summary", f"command: {command}", ""]
    return "\n".join(head + lines) + "\n"


def main():
    args = parse()
    if args.summarize:
        print(summarize(args.summarize, args.summarize_command), end="")
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        fail("bench.py measures one GPU: the library has no multi-GPU path; "
             "run with --gpus 1")
    import torch

    if not torch.cuda.is_available():
        fail("no GPU visible")
    from shared_prompt_tree_amd import ops

    ops.library()  # fail loudly if the HIP library is missing
    if args.mfma_ceiling:
        print(json.dumps(mfma_ceiling(args.ceiling_seconds)), flush=True)
        return
    if args.tile_split_sweep:
        print(json.dumps(tile_split_sweep(args.steps)), flush=True)
        return
    if args.split_sweep:
        print(json.dumps(split_sweep(args.steps)), flush=True)
        return
    if args.dq_ab:
        names = [args.workload] + ([] if args.also in ("", "none") else
                                   [n for n in args.also.split(",") if n != args.workload])
        print(json.dumps(dq_strategy_ab(names, args.steps)), flush=True)
        return
    print(f"[bench] workload {args.workload}: warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)
    main_rep = measure_workload(args.workload, args.steps, args.warmup, not args.no_flattened,
                                dq_strategy=args.dq_strategy)
    print(f"[bench] {args.workload}: {main_rep['ms_per_step']:.2f} ms/step, "
          f"{main_rep['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        workers = args.cpu_workers or min(16, os.cpu_count() or 1)
        cpu = cpu_baseline(main_rep["_tree"], main_rep["_tensors"], workers)
        print(f"[bench] cpu baseline {cpu['value']} TFLOP/s in {cpu['seconds']} s",
              file=sys.stderr, flush=True)
    main_rep.pop("_tree")
    main_rep.pop("_tensors")
    torch.cuda.empty_cache()
    also = []
    names = [] if args.also in ("", "none") else args.also.split(",")
    for aname in [n for n in names if n != args.workload]:
        a_steps = min(args.steps, ALSO_STEPS.get(aname, args.steps))
        a_warm = min(args.warmup, ALSO_WARMUP.get(aname, args.warmup))
        print(f"[bench] workload {aname}: warmup {a_warm}, steps {a_steps}", file=sys.stderr,
              flush=True)
        a = measure_workload(aname, a_steps, a_warm, not args.no_flattened,
                             fms_hint=1 if aname in ALSO_STEPS else None,
                             dq_strategy=args.dq_strategy)
        a.pop("_tree")
        a.pop("_tensors")
        also.append({
            "workload": aname, "value": round(a["tflops"], 2), "unit": "TFLOP/s",
            "steps": a_steps, "warmup": a_warm,
            "ms_per_step": round(a["ms_per_step"], 3), "step_ms_median": a["step_ms_median"],
            "pct_of_bf16_peak": round(100 * a["tflops"] / PEAK_BF16_TFLOPS, 2),
            "breakdown_ms": a["breakdown_ms"], "kernel_ms": a["kernel_ms"],
            "kernel_tflops": a["kernel_tflops"], "roofline": a["roofline"],
            "phases": a["phases"], "useful_tflops_12d": a["useful_tflops_12d"],
            "dq_strategy": a["dq_strategy"],
            "replay_schedule_balance": a["replay_schedule_balance"],
            "flattened_baseline": a.get("flattened_baseline"), "config": a["config"],
        })
        print(f"[bench] {aname}: {a['ms_per_step']:.2f} ms/step, {a['tflops']:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if args.copy_calibration_mib > 0:
        # A plain copy of known size, outside the timed region: profiling runs
        # scale the HBM byte counters of the kernels above by what the same
        # counters read for this kernel.
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ceiling = None
    if args.ceiling_seconds > 0:
        # After the timed work, on the same GPU: the matrix units' sustained
        # rate on register operands, with data like the attention operands
        # (random) and without (constant), and each kernel's rate against
        # the former.  The power-limited clock makes the first well below the
        # published peak, and it varies from GPU to GPU.
        ceiling = mfma_ceiling(args.ceiling_seconds)
        rnd = ceiling["random"]["tflops"]
        ceiling["kernel_frac_of_random"] = {
            rep["config"]["workload"]: {k: round(v / rnd, 3) for k, v in rep["kernel_tflops"].items()}
            for rep in [main_rep] + also}
        for rep in [main_rep] + also:
            # the dominant kernel against what this GPU sustains on such data
            rep["roofline"]["frac_of_measured_ceiling"] = round(
                rep["roofline"]["achieved"] / rnd, 4)
    line = {
        "metric": "tree-attention fwd+bwd useful TFLOP/s per GPU",
        "value": round(main_rep["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_rep["ms_per_step"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_bf16_peak": round(100 * main_rep["tflops"] / PEAK_BF16_TFLOPS, 2),
        "config": main_rep["config"],
        "useful_tflop_per_step": round(main_rep["useful_tflop_per_step"], 3),
        "wall_ms_per_step": round(main_rep["wall_ms_per_step"], 3),
        "step_ms_median": main_rep["step_ms_median"],
        "breakdown_ms": main_rep["breakdown_ms"],
        "kernel_ms": main_rep["kernel_ms"],
        "kernel_tflops": main_rep["kernel_tflops"],
        "phases": main_rep["phases"],
        "useful_tflops_12d": main_rep["useful_tflops_12d"],
        "dq_strategy": main_rep["dq_strategy"],
        "replay_schedule_balance": main_rep["replay_schedule_balance"],
        "roofline": main_rep["roofline"],
        "flattened_baseline": main_rep.get("flattened_baseline"),
        "cpu_baseline": cpu,
        "mfma_ceiling": ceiling,
        "also": also or None,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
