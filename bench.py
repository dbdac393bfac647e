#!/usr/bin/env python3
"""Benchmark of the fused attention-KL hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
already resident in HBM: skl_forward (one-pass forward), then the gradients
of both settings, optimise P2 (student) and optimise P1 (teacher).  By default
they come from one skl_backward_joint call (a joint dK kernel and a joint dQ
kernel that share each pair's logits and exponentials between the settings;
the library's fastest way to compute all four gradients).  --bwd-algo split
makes skl_backward_student and skl_backward_teacher calls instead, each a dK
kernel and a dQ kernel; fused_atomic the fused kernel with its workspace
clear and dQ convert.  W untimed warm-up steps, then exactly K timed steps
between two device synchronisations.

Prints ONE JSON line.  `value` is the step's algorithmic TFLOP/s
(2*pairs*[(d1+d2) + (d1+3*d2) + (3*d1+d2)] per step / step time).  The
`roofline` object describes the kernel that takes the most time per step,
timed with HIP events recorded by the library itself around that kernel on
its launch stream: `achieved` is its share of the algorithmic flops (logits a
split backward kernel recomputes count half) over its mean launch time, and
`mfma_work_tflops` the rate of all the MFMA work it issues; `noncausal` times
the same calls on the same inputs without the causal mask; `cpu_baseline` is
the float64 CPU oracle timed on a bounded causal sub-problem of the same
workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
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

METRIC = "fwd/bwd ms & TFLOP/s, causal 64K, H=32, d=128 bf16; % of MFMA peak"
DEFAULT_WORKLOAD = "causal_64k_h32_d128_q1x4"
KERNEL_SOURCES = {
    "fwd_kernel": ["fwd.hip", "skl_device.h", "skl_internal.h"],
    "bwd_dk_kernel": ["bwd_split.hip", "skl_device.h", "skl_internal.h"],
    "bwd_dq_kernel": ["bwd_split.hip", "skl_device.h", "skl_internal.h"],
    "bwd_fused_kernel": ["bwd.hip", "skl_device.h", "skl_internal.h"],
    "bwd_joint_dk_kernel": ["bwd_joint.hip", "skl_device.h", "skl_internal.h"],
    "bwd_joint_dq_kernel": ["bwd_joint.hip", "skl_device.h", "skl_internal.h"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.txt")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def code_text(path: str) -> str:
    """A source file's code without its comments, whitespace collapsed: an
    edit to comments or layout leaves the hash (and so the recorded counter
    figures) valid.  C-family files lose // and /* */ comments (the kernel
    sources have no string literal containing them), Python files their
    full-line # comments."""
    import re

    with open(path, encoding="utf-8") as fh:
        text = fh.read()
    if path.endswith(".py"):
        text = "\n".join(ln for ln in text.splitlines() if not ln.lstrip().startswith("#"))
    else:
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "attention_kl_divergence_skl_amd")
    # the build script carries per-source compiler flags, so it is hashed too
    for path in [os.path.join(pkg, "csrc", f) for f in KERNEL_SOURCES[kernel]] + [os.path.join(pkg, "build.py")]:
        h.update(code_text(path).encode())
    return h.hexdigest()[:16]


def kernel_traffic(kernel: str, phase: str, workload: str):
    """HBM bytes per launch (FETCH + WRITE, calibrated) from the committed
    counter summary, only if it was taken on the current kernel source.

    Lines of the summary look like
      traffic <workload> <phase> <kernel> <source_sha> <bytes_per_launch>
    """
    try:
        with open(TRAFFIC_FILE) as fh:
            lines = fh.read().splitlines()
    except OSError:
        return None
    sha = source_sha(kernel)
    for ln in lines:
        f = ln.split()
        if len(f) == 6 and f[0] == "traffic" and f[1:5] == [workload, phase, kernel, sha]:
            return float(f[5])
    return None


def cpu_baseline(w, n_sub: int):
    """Oracle (float64, numpy) on the leading n_sub x n_sub causal block of head
    (0, 0): forward plus both backward settings; the rate is the same
    algorithmic flop count the GPU value uses, for that sub-problem."""
    import numpy as np

    import oracle
    from attention_kl_divergence_skl_amd import synth, workmodel

    q1, k1, q2, k2 = synth.head_inputs(w.with_(NQ=n_sub, NK=n_sub), 0, 0)
    g = synth.head_grad(w.with_(NQ=n_sub, NK=n_sub), 0, 0)
    threads = None
    try:
        import threadpoolctl

        threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=None)
    except Exception:  # noqa: BLE001 - report unknown
        threads = None
    args = (q1, k1, q2, k2, w.scale1, w.scale2, w.causal)
    t0 = time.perf_counter()
    oracle.head_forward(*args)
    oracle.head_backward(*args, g, "student")
    oracle.head_backward(*args, g, "teacher")
    dt = time.perf_counter() - t0
    wk = workmodel.work(1, 1, n_sub, n_sub, w.d1, w.d2, w.causal)
    flops = wk.fwd_flops + wk.student_flops + wk.teacher_flops
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads or len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"float64 oracle forward + student + teacher backward on the leading "
                   f"{n_sub}x{n_sub} {'causal ' if w.causal else ''}block of head (0,0), "
                   f"{dt:.1f} s wall; host has {os.cpu_count()} cores"),
        "seconds": dt,
    }


def copy_calibration(nbytes: int, reps: int) -> None:
    """Kernels of known traffic, for scaling HBM byte counters: a plain copy
    (reads and writes nbytes) and a sum reduction of the same buffer (reads
    nbytes, writes a few bytes), each `reps` times."""
    import torch

    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    total = torch.empty((), dtype=torch.float32, device="cuda")
    for _ in range(reps):
        torch.sum(src, dim=0, out=total)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "sum_bytes_read": nbytes,
                      "reps": reps}), flush=True)


def kernel_flops(w, wk, phase: str, algo: str):
    """Flops each main kernel of a phase must do (its own MFMA work)."""
    P = wk.pairs
    if phase == "fwd":
        return {"fwd_kernel": wk.fwd_flops}
    if phase == "joint":  # both logits once + the four gradient GEMMs, split over two kernels
        per = 2 * P * 2 * (w.d1 + w.d2)
        return {"bwd_joint_dk_kernel": per, "bwd_joint_dq_kernel": per}
    dg = w.d2 if phase == "student" else w.d1
    if algo == "split":
        per = 2 * P * (w.d1 + w.d2 + dg)  # both logits again + one gradient GEMM
        return {"bwd_dk_kernel": per, "bwd_dq_kernel": per}
    return {"bwd_fused_kernel": wk.student_flops if phase == "student" else wk.teacher_flops}


def kernel_alg_flops(w, wk, phase: str, algo: str):
    """Algorithmic flops attributed to each main kernel of a phase: the
    phase's algorithmic count (each pair's logits once, each gradient GEMM
    once) shared out so that the kernels of a phase sum to it.  A kernel that
    recomputes logits another kernel also forms is credited half of them."""
    P = wk.pairs
    if phase == "fwd":
        return {"fwd_kernel": wk.fwd_flops}
    if phase == "joint":
        half = (wk.student_flops + wk.teacher_flops) // 2
        return {"bwd_joint_dk_kernel": half, "bwd_joint_dq_kernel": half}
    dg = w.d2 if phase == "student" else w.d1
    if algo == "split":
        per = P * (w.d1 + w.d2) + 2 * P * dg  # half of the logits + its own gradient GEMM
        return {"bwd_dk_kernel": per, "bwd_dq_kernel": per}
    return {"bwd_fused_kernel": wk.student_flops if phase == "student" else wk.teacher_flops}


def hbm_report(alg_bytes: int, traffic, ms: float):
    """Per-kernel HBM figures: compulsory bytes and, with a counter figure for
    the current source, the achieved GB/s (counter bytes / kernel time), its
    fraction of the 8 TB/s peak and the counter/compulsory ratio."""
    out = {"alg_bytes": int(alg_bytes), "hbm_bytes": traffic, "hbm_gbs": None, "hbm_frac": None,
           "traffic_ratio": None}
    if traffic:
        from attention_kl_divergence_skl_amd import workmodel

        gbs = traffic / (ms * 1e-3) / 1e9
        out.update(hbm_gbs=gbs, hbm_frac=gbs / workmodel.PEAK_HBM_GBS, traffic_ratio=traffic / alg_bytes)
    return out


def kernel_alg_bytes(w, phase: str, algo: str):
    """Compulsory HBM bytes of each main kernel of a phase: every input it
    reads once, the per-row vectors it reads, and the outputs it writes once
    (a workspace is an implementation cost and is not counted)."""
    e = 2 if w.dtype == "bf16" else 4
    BH = w.B * w.H
    inputs = BH * (w.NQ + w.NK) * (w.d1 + w.d2) * e
    rowvec = BH * w.NQ * 4
    if phase == "fwd":
        return {"fwd_kernel": inputs + 3 * rowvec}
    if phase == "joint":
        return {"bwd_joint_dk_kernel": inputs + 4 * rowvec + BH * w.NK * (w.d1 + w.d2) * e,
                "bwd_joint_dq_kernel": inputs + 4 * rowvec + BH * w.NQ * (w.d1 + w.d2) * e}
    dg = w.d2 if phase == "student" else w.d1
    rv = (3 if phase == "student" else 4) * rowvec
    if algo == "split":
        return {"bwd_dk_kernel": inputs + rv + BH * w.NK * dg * e,
                "bwd_dq_kernel": inputs + rv + BH * w.NQ * dg * e}
    return {"bwd_fused_kernel": inputs + rv + BH * (w.NQ + w.NK) * dg * e}


def other_mask_leg(skl, torch, np, w, t, phases, algo, ws_s, ws_t, peak_tf, steps: int):
    """The same inputs and calls without the causal mask (twice the pairs):
    one untimed step, then `steps` timed ones; each call timed with events
    around it on the current stream."""
    from attention_kl_divergence_skl_amd import workmodel

    wn = w.with_(causal=False)
    wk = workmodel.work(wn.B, wn.H, wn.NQ, wn.NK, wn.d1, wn.d2, False, 2 if wn.dtype == "bf16" else 4)
    alg = {"fwd": wk.fwd_flops, "student": wk.student_flops, "teacher": wk.teacher_flops,
           "joint": wk.student_flops + wk.teacher_flops}
    q1, k1, q2, k2, g = t["q1"], t["k1"], t["q2"], t["k2"], t["g"]
    ev = {p: [] for p in phases}

    def one(record):
        kl, l1, l2 = None, None, None
        for p in ("fwd", "student", "teacher", "joint"):
            if p not in phases:
                continue
            if record:
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record()
            if p == "fwd":
                kl, l1, l2 = skl.skl_forward(q1, k1, q2, k2, wn.scale1, wn.scale2, False)
            elif p == "joint":
                skl.skl_backward_joint(q1, k1, q2, k2, l1, l2, kl, g, wn.scale1, wn.scale2, False, ws=ws_t)
            elif p == "student":
                skl.skl_backward_student(q1, k1, q2, k2, l1, l2, g, wn.scale1, wn.scale2, False, algo=algo, ws=ws_s)
            else:
                skl.skl_backward_teacher(q1, k1, q2, k2, l1, l2, kl, g, wn.scale1, wn.scale2, False,
                                         algo=algo, ws=ws_t)
            if record:
                e[1].record()
                ev[p].append(e)

    one(False)
    torch.cuda.synchronize()
    log(f"no mask: untimed step done; timing {steps}")
    t0 = time.perf_counter()
    for _ in range(steps):
        one(True)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / steps * 1e3
    out = {"workload": f"{w.name} without the causal mask", "causal": False, "steps": steps,
           "ms_per_step": ms_step}
    step_flops = sum(alg[p] for p in phases)
    out["tflops"] = step_flops / (ms_step * 1e-3) / 1e12
    out["pct_peak"] = 100.0 * out["tflops"] / peak_tf
    out["phases"] = {}
    for p in phases:
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev[p]]))
        tf = alg[p] / (ms * 1e-3) / 1e12
        out["phases"][p] = {"call_ms": ms, "algorithmic_tflops": tf, "pct_peak": 100.0 * tf / peak_tf}
    log(f"no mask: {ms_step:.1f} ms per step, {out['tflops']:.1f} TFLOP/s")
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--mask", choices=["workload", "causal", "none"], default="workload",
                    help="run the workload's shapes and inputs with causal masking or without "
                         "(default: as the workload defines it)")
    ap.add_argument("--phases", default="fwd,student,teacher",
                    help="comma list of fwd, student, teacher, joint (profiling aid; the default is the "
                         "full step; with --bwd-algo joint, the default, student and teacher become joint)")
    ap.add_argument("--bwd-algo", default="joint", choices=["joint", "split", "fused_atomic"],
                    help="joint (default): both settings in one skl_backward_joint call; split: the "
                         "student and teacher calls")
    ap.add_argument("--noncausal-steps", type=int, default=2,
                    help="timed steps of the same inputs without the mask (reported beside the main line; 0: skip)")
    ap.add_argument("--cpu-sub", type=int, default=16384, help="side of the causal block the oracle times")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MiB",
                    help="only run a plain copy and a sum reduction of this many MiB (counter calibration) and exit")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the attention-KL kernels here run on a single MI355X "
              "(sharding across GPUs is described, not implemented); use --gpus 1.",
              file=sys.stderr, flush=True)
        return 2

    import numpy as np
    import torch

    import attention_kl_divergence_skl_amd as skl
    from attention_kl_divergence_skl_amd import synth, workmodel

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.copy_calib:
        copy_calibration(args.copy_calib << 20, 5)
        return 0
    skl.load()

    w = synth.WORKLOADS[args.workload]
    traffic_key = w.name  # counter figures are recorded per workload as it is defined
    if args.mask != "workload":
        if w.causal != (args.mask == "causal"):
            traffic_key = f"{w.name}_mask_{args.mask}"
        w = w.with_(causal=args.mask == "causal")
    phases = [p for p in args.phases.split(",") if p]
    algo = args.bwd_algo
    if algo == "joint" and any(p in ("student", "teacher") for p in phases):
        phases = [p for p in phases if p not in ("student", "teacher", "joint")] + ["joint"]
    for p in phases:
        if p not in ("fwd", "student", "teacher", "joint"):
            raise SystemExit(f"unknown phase {p}")
    log(f"workload {w.name}: generating inputs")
    t0 = time.perf_counter()
    t = synth.device_inputs(w, "cuda")
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    q1, k1, q2, k2, g = t["q1"], t["k1"], t["q2"], t["k2"], t["g"]
    ebytes = 2 if w.dtype == "bf16" else 4
    wk = workmodel.work(w.B, w.H, w.NQ, w.NK, w.d1, w.d2, w.causal, ebytes)

    # Workspaces (fused algorithm only) are allocated once, outside the timed region.
    def ws_for(teacher):
        if algo == "joint":
            n = skl.skl_backward_joint_workspace_size(q1, k1, q2, k2) if teacher else 0
        else:
            n = skl.skl_backward_workspace_size(q1, k1, q2, k2, teacher, algo)
        return torch.empty(n // 4, dtype=torch.float32, device="cuda") if n else None

    ws_s, ws_t = ws_for(False), ws_for(True)
    kflops = {p: kernel_flops(w, wk, p, algo) for p in phases}
    kalg = {p: kernel_alg_flops(w, wk, p, algo) for p in phases}
    kbytes = {p: kernel_alg_bytes(w, p, algo) for p in phases}
    kev = {p: [] for p in phases}   # per call: events around its main kernels
    pev = {p: [] for p in phases}   # per call: events around the whole call

    def new_events(n):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for x in e:
            x.record()  # torch creates the HIP event on first record; the library re-records
        return e

    def step(record: bool):
        out = {}
        kl = l1 = l2 = None
        for p in ("fwd", "student", "teacher", "joint"):
            if not (p in phases or (p == "fwd" and phases != ["fwd"])):
                continue
            rec = record and p in phases
            if rec:
                ke = new_events(len(kflops[p]) + 1)
                ce = new_events(2)
                skl.skl_set_kernel_events(ke)
                ce[0].record()
            if p == "fwd":
                kl, l1, l2 = skl.skl_forward(q1, k1, q2, k2, w.scale1, w.scale2, w.causal)
            elif p == "joint":
                out["j"] = skl.skl_backward_joint(q1, k1, q2, k2, l1, l2, kl, g, w.scale1, w.scale2, w.causal,
                                                  ws=ws_t)
            elif p == "student":
                out["s"] = skl.skl_backward_student(q1, k1, q2, k2, l1, l2, g, w.scale1, w.scale2, w.causal,
                                                    algo=algo, ws=ws_s)
            else:
                out["t"] = skl.skl_backward_teacher(q1, k1, q2, k2, l1, l2, kl, g, w.scale1, w.scale2,
                                                    w.causal, algo=algo, ws=ws_t)
            if rec:
                ce[1].record()
                skl.skl_set_kernel_events([])
                kev[p].append(ke)
                pev[p].append(ce)
        return out

    # Extra HBM of one step: peak allocation beyond resident inputs and outputs.
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    o = step(False)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    out_bytes = 3 * w.B * w.H * w.NQ * 4
    out_bytes += sum(x.numel() * x.element_size() for v in o.values() for x in v)
    held_ws = sum(x.numel() * 4 for x in (ws_s, ws_t) if x is not None)
    extra = peak - out_bytes + held_ws
    del o

    for i in range(args.warmup):
        step(False)
        torch.cuda.synchronize()
        log(f"warm-up step {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"{args.steps} timed steps in {elapsed:.3f} s")

    peak_tf = workmodel.PEAK_BF16_DENSE_TFLOPS if w.dtype == "bf16" else workmodel.PEAK_FP32_MFMA_TFLOPS
    alg = {"fwd": wk.fwd_flops, "student": wk.student_flops, "teacher": wk.teacher_flops,
           "joint": wk.student_flops + wk.teacher_flops}
    report, kernels = {}, []
    for p in phases:
        call_ms = float(np.mean([a.elapsed_time(b) for a, b in pev[p]]))
        ks = {}
        for i, (name, fl) in enumerate(kflops[p].items()):
            times = [e[i].elapsed_time(e[i + 1]) for e in kev[p]]
            kms = float(np.mean(times))
            tf = fl / (kms * 1e-3) / 1e12
            atf = kalg[p][name] / (kms * 1e-3) / 1e12
            # tflops / pct_mfma_peak: the kernel's own MFMA work (matrix-core use);
            # alg_tflops / pct_peak_alg: its share of the algorithmic count (both
            # from the mean time; the min and median over the timed launches
            # are reported beside it).
            ks[name] = {"ms": kms, "ms_min": float(np.min(times)), "ms_median": float(np.median(times)),
                        "tflops": tf, "pct_mfma_peak": 100.0 * tf / peak_tf,
                        "alg_tflops": atf, "pct_peak_alg": 100.0 * atf / peak_tf}
            # HBM: compulsory bytes, and the calibrated counter bytes of the
            # committed summary when it was taken on the current source.
            ks[name].update(hbm_report(kbytes[p][name], kernel_traffic(name, p, traffic_key), kms))
            kernels.append((kms, p, name, kalg[p][name], fl))
        report[p] = {"call_ms": call_ms, "algorithmic_tflops": alg[p] / (call_ms * 1e-3) / 1e12,
                     "kernels": ks}
    step_flops = sum(alg[p] for p in phases)
    ms_step = elapsed / args.steps * 1e3
    kms, dom_phase, dom_name, dom_flops, dom_mfma = max(kernels)
    ach = dom_flops / (kms * 1e-3) / 1e12
    mfma_rate = dom_mfma / (kms * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": step_flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N_Q": w.NQ, "N_K": w.NK, "d1": w.d1, "d2": w.d2,
                   "causal": w.causal, "step": "+".join(phases), "bwd_algo": algo},
        "phases": report,
        "extra_hbm_bytes": int(extra),
        "materialised_bytes": int(wk.materialised_bytes),
        "roofline": {
            "kernel": f"{dom_name} ({dom_phase})",
            "bound": "mfma",
            "achieved": ach,
            "peak": peak_tf,
            "unit": "TFLOP/s",
            "frac": ach / peak_tf,
            "traffic": kernel_traffic(dom_name, dom_phase, traffic_key),
            **{k: v for k, v in report[dom_phase]["kernels"][dom_name].items()
               if k in ("alg_bytes", "hbm_gbs", "traffic_ratio", "hbm_frac")},
            "flops_per_launch": dom_flops,
            "mfma_work_flops_per_launch": dom_mfma,
            "mfma_work_tflops": mfma_rate,
            "mfma_work_frac": mfma_rate / peak_tf,
        },
        "cpu_baseline": None,
    }
    if args.noncausal_steps > 0 and w.causal and "fwd" in phases:
        res["noncausal"] = other_mask_leg(skl, torch, np, w, t, phases, algo, ws_s, ws_t, peak_tf,
                                          args.noncausal_steps)
    if not args.no_cpu_baseline:
        log(f"timing the oracle on a {args.cpu_sub}x{args.cpu_sub} block")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sub)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
