#!/usr/bin/env python3
"""Throughput of libcce's flash cut-cross-entropy head, forward + backward.

One step = forward + backward (g = 1) over one batch of the synthetic
workload M=8192 tokens, H=2560, V=262144, 8-bit affine head (group 64),
softcap 30 -- the largest single-GPU workload at H=2560, V=262144.  Inputs are
resident in HBM and workspaces preallocated before the timed region.  The
step is one call of cce_forward_backward: under a softcap of at most 40, or
with none, a single pass (the logits computed once), otherwise its forward
and backward passes after one front.  The `two_calls` field times cce_forward +
cce_backward (the backward recomputes the logits) on the same inputs; the
skips always take their calls, and a dense head (--dense) takes
cce_dense_forward_backward alike (the single pass under a softcap of at most
40, its dW last).  Each step is timed
between its own pair of HIP events; the median is reported.

Prints one JSON line.  `value` is supervised tokens per second of fwd+bwd.
`roofline` is for the kernel family with the most time per step, timed live
with HIP events on the launch stream (include/cce_profile.h), against the
MI355X dense bf16 MFMA peak.  `cpu_baseline` times the fp64 CPU oracle on a
bounded sample of the same workload's tokens.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0
COPY_BYTES = 1 << 30        # calibration copy: reads and writes exactly this many bytes
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_M8192_H2560_V262144_8bit.txt")


def _code_only(text):
    """C/C++ source without comments and blank lines (string literals in these
    sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash():
    """Hash of the code of the HIP sources (comments excluded); a traffic
    measurement is valid only for the kernels it was taken on."""
    import hashlib
    d = os.path.join(ROOT, "linear_cross_entropy_libcce_amd", "csrc")
    hsh = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        hsh.update(f.encode())
        hsh.update(_code_only(open(os.path.join(d, f)).read()).encode())
    return hsh.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when it is missing or was taken on different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["%s.fetch_bytes_per_launch" % kernel]) + float(kv["%s.write_bytes_per_launch" % kernel])
    except KeyError:
        return None


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def cpu_baseline(inp, seconds, M_eff):
    """The oracle, untuned, on a bounded token sample; scaled to tokens/s."""
    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    import oracle
    act = np.arange(inp["M"]) if inp["mask"] is None else np.flatnonzero(inp["mask"])
    rng = np.random.default_rng(0)
    t0 = time.perf_counter()
    oracle.cce(inp, tokens=act[:1])
    per_tok = max(time.perf_counter() - t0, 1e-6)
    # a random sample of the supervised tokens (all of them when there are
    # few), repeated until the sample has taken about `seconds`
    n = int(max(1, min(64, len(act), seconds / per_tok)))
    reps = int(max(1, min(10000, seconds / (n * per_tok))))
    toks = rng.choice(act, size=n, replace=False)
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.cce(inp, tokens=toks)
    dt = time.perf_counter() - t0
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": n * reps / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "nproc": os.cpu_count(), "cpu_model": model,
            "sample": "fwd+bwd of %d random supervised tokens of the full workload%s (%.1f s)"
                      % (n, "" if reps == 1 else ", %d times" % reps, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3,
                    help="synthetic workload index (0-4); 3 is the measured configuration")
    ap.add_argument("--tokens", type=int, default=None,
                    help="override M (e.g. 1024: one GPU's share of workload 3 split over 8 GPUs)")
    ap.add_argument("--group", type=int, default=None, help="override the quantization group (32, 64, 128)")
    ap.add_argument("--sb-dtype", type=str, default=None, choices=["f32", "bf16", "f16"],
                    help="override the storage of scales and biases")
    ap.add_argument("--bias", type=str, default=None, choices=["symmetric", "affine"],
                    help="head kind: symmetric (bias = -zero_point*scale, the workload's own) or affine "
                         "(a float head min/max-quantized, bias = group minimum: every row has b' != 0)")
    ap.add_argument("--skip", type=str, default=None, metavar="BLOCK_EPS,FILTER_EPS",
                    help="opt-in backward skips (e.g. 1e-5,1e-5): forward with block maxima, backward skipping")
    ap.add_argument("--path", type=str, default="auto", choices=["auto", "calls"],
                    help="auto: the single pass cce_forward_backward where the head allows it (softcap in (0, 40]), "
                         "else cce_forward + cce_backward; calls: always the two calls")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays (launch-bound small M)")
    ap.add_argument("--dense", action="store_true",
                    help="a trainable dense bf16 head of the workload's shape (forward, dh and dW)")
    ap.add_argument("--prepared", action="store_true",
                    help="prepare the frozen head once (cce_head_prepare) before the timed steps; the steps then "
                         "skip the per-call derivation of its per-row data")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain device copy of COPY_BYTES (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the head is data-parallel over tokens with no "
              "communication, so a %d-GPU run is %d independent copies of this one; "
              "run with --gpus 1." % (args.gpus, args.gpus), file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_cross_entropy_libcce_amd import cce
    from linear_cross_entropy_libcce_amd import synthetic as syn

    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("calibration copy of %d bytes done" % COPY_BYTES)

    w = syn.WORKLOADS[args.workload]
    import dataclasses
    if args.tokens is not None:
        w = dataclasses.replace(w, M=args.tokens, name="%s, M=%d" % (w.name, args.tokens))
    if args.group is not None:
        w = dataclasses.replace(w, group=args.group, name="%s, group %d" % (w.name, args.group))
    if args.sb_dtype is not None:
        w = dataclasses.replace(w, sb_dtype=args.sb_dtype, name="%s, %s scales" % (w.name, args.sb_dtype))
    if args.bias is not None and args.bias != w.bias:
        w = dataclasses.replace(w, bias=args.bias, name="%s, %s head" % (w.name, args.bias))
    dev = torch.device("cuda:0")
    if args.dense:
        if args.skip or args.group or args.sb_dtype or args.prepared:
            sys.exit("--dense takes no quantization, skip or preparation options")
        w = dataclasses.replace(w, name="%s shape, dense bf16 head" % w.name.split(" 4-bit")[0].split(" 8-bit")[0])
        log("generating a dense head of workload %d's shape (%s)" % (args.workload, w.name))
        inp = syn.make_dense(w.M, w.H, w.V, syn.seed_for(args.workload), softcap=w.softcap, targets=w.targets,
                             zipf_a=w.zipf_a, mask=w.mask, mask_frac=w.mask_frac)
        head = cce.dense_head_from_numpy(inp, dev)
        ws_f = torch.empty(cce.dense_forward_workspace_bytes(head, inp["M"]), dtype=torch.uint8, device=dev)
        ws_b = torch.empty(cce.dense_backward_workspace_bytes(head, inp["M"]), dtype=torch.uint8, device=dev)
        dw = torch.empty((inp["V"], inp["H"]), dtype=torch.float32, device=dev)
    else:
        log("generating workload %d (%s)" % (args.workload, w.name))
        inp = syn.make_inputs(w, syn.seed_for(args.workload))
        head = cce.head_from_numpy(inp, dev)
        if args.prepared:
            cce.cce_head_prepare(head)
            torch.cuda.synchronize()
            w = dataclasses.replace(w, name="%s, prepared head" % w.name)
        ws_f = torch.empty(cce.forward_workspace_bytes(head, inp["M"]), dtype=torch.uint8, device=dev)
        ws_b = torch.empty(cce.backward_workspace_bytes(head, inp["M"]), dtype=torch.uint8, device=dev)
    M, H, V = inp["M"], inp["H"], inp["V"]
    M_eff = M if inp["mask"] is None else int(inp["mask"].sum())
    h, t, m = cce.tokens_from_numpy(inp, dev)
    logp = torch.empty(M, dtype=torch.float32, device=dev)
    lse = torch.empty(M, dtype=torch.float32, device=dev)
    dh = torch.empty((M, H), dtype=torch.float32, device=dev)
    block_eps = filter_eps = 0.0
    if args.skip:
        block_eps, filter_eps = (float(x) for x in args.skip.split(","))
    bmx = torch.empty((M, cce.n_blocks(head)), dtype=torch.float32, device=dev) if args.skip else None

    def fwd():
        if args.dense:
            cce.cce_dense_forward(h, head, t, m, workspace=ws_f, out=(logp, lse))
        elif args.skip:
            cce.cce_forward_ex(h, head, t, m, block_max=bmx, workspace=ws_f, out=(logp, lse))
        else:
            cce.cce_forward(h, head, t, m, workspace=ws_f, out=(logp, lse))

    def bwd():
        if args.dense:
            cce.cce_dense_backward(h, head, t, lse, None, m, workspace=ws_b, out=dh, dw_out=dw)
        elif args.skip:
            cce.cce_backward_ex(h, head, t, lse, None, m, block_max=bmx, block_eps=block_eps, filter_eps=filter_eps,
                                workspace=ws_b, out=dh)
        else:
            cce.cce_backward(h, head, t, lse, None, m, workspace=ws_b, out=dh)

    def calls():
        fwd()
        bwd()

    # one call (cce_forward_backward, cce_dense_forward_backward) without
    # skips: the single pass where the head allows it (0 < softcap <= 40), else
    # its two passes; the skips take the two calls
    combined = not args.skip and args.path != "calls"
    # the logits once: a softcap in (0, 40], or none on a quantized head (its
    # uncapped single pass)
    fused = combined and (0.0 < inp["softcap"] <= 40.0 or (inp["softcap"] == 0.0 and not args.dense))
    if combined:
        nb = (cce.dense_forward_backward_workspace_bytes(head, M) if args.dense
              else cce.forward_backward_workspace_bytes(head, M))
        ws_fb = torch.empty(nb, dtype=torch.uint8, device=dev)

    def fused_step():
        if args.dense:
            cce.cce_dense_forward_backward(h, head, t, None, m, workspace=ws_fb, out=(logp, lse, dh), dw_out=dw)
        else:
            cce.cce_forward_backward(h, head, t, None, m, workspace=ws_fb, out=(logp, lse, dh))

    step = fused_step if combined else calls
    fb_name = "cce_dense_forward_backward" if args.dense else "cce_forward_backward"
    calls_name = "cce_dense_forward + cce_dense_backward" if args.dense else "cce_forward + cce_backward"
    log("step: %s" % (("%s (%s)" % (fb_name, "single pass" if fused else "two passes"))
                      if combined else calls_name))

    log("warmup %d steps" % args.warmup)
    for _ in range(args.warmup):
        step()
        if combined:
            calls()
    torch.cuda.synchronize()

    def replayable(fn):
        if not args.graph:
            return fn
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        torch.cuda.synchronize()
        log("captured one step in a HIP graph")
        return graph.replay

    def timed(fn):
        """Per-step milliseconds, each step between its own pair of events."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(args.steps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]

    log("timing %d steps" % args.steps)
    wall0 = time.perf_counter()
    per = timed(replayable(step))
    wall = time.perf_counter() - wall0
    ms = float(np.median(per))
    ms_mean = float(np.mean(per))
    log("%.3f ms/step median, %.3f mean (wall %.3f ms/step)" % (ms, ms_mean, 1e3 * wall / args.steps))

    # the forward and the backward alone (same inputs), and the two calls as
    # a step when the single pass is the one timed above
    ms_fwd = float(np.median(timed(fwd)))
    ms_bwd = float(np.median(timed(bwd)))
    log("forward %.3f ms, backward %.3f ms (median)" % (ms_fwd, ms_bwd))
    two_calls = None
    if combined:
        ms_calls = float(np.median(timed(replayable(calls))))
        two_calls = {"ms_per_step": round(ms_calls, 4), "tokens_per_s": round(M_eff / (ms_calls * 1e-3), 1),
                     "tflops": round((8.0 if args.dense else 6.0) * M_eff * V * H / (ms_calls * 1e-3) / 1e12, 1)}
        log("cce_forward + cce_backward: %.3f ms/step (median)" % ms_calls)

    # per-kernel timing pass (same steps, events around every launch)
    log("per-kernel timing pass")
    cce.profile_read()
    cce.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = cce.profile_read()
    cce.profile_enable(False)
    per_step = {k: (n / args.steps, tot / args.steps) for k, (n, tot) in prof.items()}
    for k, (n, tot) in sorted(per_step.items(), key=lambda kv: -kv[1][1]):
        log("  %-10s %5.1f launches/step  %8.3f ms/step" % (k, n, tot))

    # MFMA work per step: forward logits and dh always, the backward's logit
    # recompute unless the single pass ran (and dW for a dense head)
    gemms = (3.0 if fused else 4.0) if args.dense else (2.0 if fused else 3.0)
    exec_flops = 2.0 * gemms * M_eff * V * H
    if args.dense:
        head_bytes = 2 * V * H
    else:
        sb_size = 4 if inp.get("sb_dtype", "f32") == "f32" else 2
        head_bytes = V * (H * inp["bits"] // 8) + 2 * sb_size * V * (H // inp["group"])  # codes + scales, biases
    head_gbs = 2.0 * head_bytes / (ms * 1e-3) / 1e9                   # the head is read by both passes
    tflops = exec_flops / (ms * 1e-3) / 1e12
    per_kernel_flops = {"tile_fwd": 2.0 * M_eff * V * H, "tile_bwd": 2.0 * M_eff * V * H,
                        "tile_fused": 2.0 * M_eff * V * H,
                        "dh_gemm": 2.0 * M_eff * V * H, "dw_gemm": 2.0 * M_eff * V * H}
    dom = max(per_step, key=lambda k: per_step[k][1])
    n_l, t_l = per_step[dom]
    roof = None
    if dom in per_kernel_flops:
        flop_launch = per_kernel_flops[dom] / n_l
        achieved = flop_launch / (t_l / n_l * 1e-3) / 1e12
        default_cfg = (args.tokens is None and not args.skip and args.group is None and args.sb_dtype is None
                       and not args.dense and args.bias in (None, "symmetric"))
        tb = measured_traffic(dom) if (args.workload == 3 and default_cfg) else None
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": tb,
                "traffic_GB_per_s": None if tb is None else round(tb / (t_l / n_l * 1e-3) / 1e9, 1),
                "flop_per_launch": flop_launch, "avg_launch_ms": round(t_l / n_l, 4)}
        if args.skip:
            roof["note"] = "dense-equivalent flops: skipped pairs are counted but do no work"

    cpu = None
    if not args.no_cpu_baseline and not args.dense:
        log("cpu baseline: oracle on a token sample (~%.0f s)" % args.cpu_seconds)
        cpu = cpu_baseline(inp, args.cpu_seconds, M_eff)

    out = {
        "metric": "CCE fwd+bwd tokens/s and % bf16 MFMA peak at H=2560,V=262144",
        "value": round(M_eff / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_mean": round(ms_mean, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": M, "M_supervised": M_eff, "H": H, "V": V,
                   "head": "dense bf16" if args.dense else "quantized",
                   "bits": 16 if args.dense else inp["bits"], "group": None if args.dense else inp["group"],
                   "sb_dtype": None if args.dense else inp.get("sb_dtype", "f32"),
                   "bias": None if args.dense else w.bias, "softcap": inp["softcap"],
                   "g": 1.0,
                   "skip": None if not args.skip else {"block_eps": block_eps, "filter_eps": filter_eps},
                   "hip_graph": bool(args.graph),
                   "step": ("%s (single pass)" % fb_name if fused else
                            ("%s (two passes)" % fb_name if combined else calls_name))},
        "ms_fwd": round(ms_fwd, 4),
        "ms_bwd": round(ms_bwd, 4),
        "two_calls": two_calls,
        "tflops": round(tflops, 1),
        "flops_counted": (("6*M_eff*V*H (logits once, dh, dW)" if fused else "8*M_eff*V*H (forward, recompute, dh, dW)")
                          if args.dense else
                          ("4*M_eff*V*H (logits once, dh)" if fused else "6*M_eff*V*H (logits, recompute, dh)"))
        + (" (dense-equivalent: skipped pairs counted)" if args.skip else ""),
        "pct_bf16_peak": round(100.0 * tflops / BF16_PEAK_TFLOPS, 2),
        "tflops_6mvh": round(6.0 * M_eff * V * H / (ms * 1e-3) / 1e12, 1),
        # the same step priced as a forward plus a recomputing backward (logits twice, dh): the rate such a
        # design would need for this throughput, as a fraction of the peak
        "pct_bf16_peak_6mvh": round(100.0 * 6.0 * M_eff * V * H / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2),
        "head_GB_per_s": round(head_gbs, 1),
        "kernel_ms_per_step": {k: round(v[1], 4) for k, v in per_step.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
