"""Benchmark of one tree-verification step on one MI355X.

A step is the whole hot path over one input set, issued on one HIP stream:
    spec_tree_mask_build, spec_tree_attention (one layer's KV), spec_tree_softmax
    (target rows, and draft rows at T > 0), spec_tree_reject_sample (whose final walk
    also writes the accepted path, the result of spec_accept_path).
Workload (default): the Llama-3-8B-shaped step -- one request, a 60-node EAGLE-2
tree (top-k 10, depth 6), 4096 cached tokens, 32 query / 8 KV heads, head_dim 128,
bf16 KV, fp32 logits over a 128256-token vocabulary, T = 1.  Synthetic, seeded.

Timing: W warm-up steps, then K steps bracketed by synchronize + HIP events.  Each
step reads one of R input replicas in turn (distinct device buffers, 8 x ~80 MB)
so the working set is far larger than the 256 MB last-level cache and the numbers
are HBM numbers.  A second timed pass records events around every stage to report
per-call durations; the call holding the longest kernel (tree attention) gives the
roofline entry, the logit softmax a second one.  Measured HBM traffic per call comes
from the committed counter summary under profiles/ while the kernel sources match.  The CPU oracle is timed on the host on full steps of the same
workload.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tree-verify steps/sec + attn/sampling HBM GB/s (8B-shape, 60-node tree, 4k ctx)"
HBM_PEAK_GBS = 8000.0
COPY_ELEMS = 1 << 27  # fp32: 512 MiB read and 512 MiB written per copy
# HBM bytes per call measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (scaled by the
# same counters on a plain copy); valid only while the sources listed there are unchanged
COUNTERS_MD = os.path.join(ROOT, "profiles", "attention_softmax_llama8b_60node_ctx4096_hbm_counters.md")


def measured_traffic():
    """{call: bytes} from the counter summary, for calls whose kernel sources still
    hash to the values recorded with the counters."""
    import hashlib
    import re

    if not os.path.exists(COUNTERS_MD):
        return {}
    text = open(COUNTERS_MD).read()
    shas = dict(re.findall(r"^- sha256 (\S+): ([0-9a-f]{64})", text, flags=re.M))
    calls = re.findall(r"^- traffic_bytes (\S+): (\d+) \(sources: ([^)]*)\)", text, flags=re.M)
    out = {}
    for call, nbytes, srcs in calls:
        ok = True
        for src in srcs.split(","):
            src = src.strip()
            path = os.path.join(ROOT, src)
            if src not in shas or not os.path.exists(path) or \
                    hashlib.sha256(open(path, "rb").read()).hexdigest() != shas[src]:
                ok = False
        out[call] = int(nbytes) if ok else None
    return out


def roofline_entry(kernel, nbytes, us, traffic):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "bytes_per_launch": int(nbytes),
            "avg_launch_us": round(float(us), 3)}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--temperature", type=float, default=1.0)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run four plain 512 MiB device-to-device copies (the reference kernel whose "
                         "FETCH_SIZE / WRITE_SIZE counters scale the traffic of the step's kernels)")
    return ap.parse_args()


def algorithmic_bytes(inp):
    """Bytes the step must move at least once: KV of every request (prompt + tree),
    Q and O, the target logits, and the draft logits when T > 0."""
    B, n_max, hq, hkv, d = inp["B"], inp["n_max"], inp["hq"], inp["hkv"], inp["d"]
    el = 2 if inp["bf16"] else 4
    kv_tokens = int(np.sum(inp["ctx_len"] + inp["n_nodes"]))
    attn = 2 * kv_tokens * hkv * d * el + 2 * B * n_max * hq * d * el
    logits = B * n_max * inp["V"] * 4
    sampling = logits * (2 if inp["T"] > 0 else 1)
    return attn, logits, sampling


def copy_calibration():
    import torch

    a = torch.ones(COPY_ELEMS, device="cuda")
    b = torch.empty_like(a)
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": a.numel() * 4, "bytes_written": b.numel() * 4,
                                           "launches": 4}}))


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from tree_verification_masked_amd import synth
    from tree_verification_masked_amd.step import VerifyStep, to_device

    torch.cuda.set_device(0)
    T = args.temperature if args.config != 3 else None
    inp = synth.make_config(args.config, seed=args.seed, T=T)
    dev = to_device(inp)
    step = VerifyStep(dev)
    big = [k for k in ("q", "k", "v", "tgt_logits", "dft_logits") if k in dev]
    replicas = [{k: dev[k].clone() for k in big} for _ in range(args.replicas)]
    stream = torch.cuda.current_stream()

    def run_steps(n, first=0, events=None):
        for i in range(n):
            r = replicas[(first + i) % len(replicas)]
            if events is None:
                step.run(replica=r)
                continue
            ev = events[i]
            ev[0].record(stream)
            step.mask()
            ev[1].record(stream)
            if step.with_attention:
                step.attention(None, r["q"], r["k"], r["v"])
            ev[2].record(stream)
            step.softmax(None, r["tgt_logits"], r.get("dft_logits"))
            ev[3].record(stream)
            ev[4].record(stream)
            step.reject(None, r["tgt_logits"], r.get("dft_logits"))  # writes the accepted path too
            ev[5].record(stream)
            ev[6].record(stream)

    # warm-up, then the clean timed region
    run_steps(args.warmup)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    run_steps(args.steps, first=args.warmup)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    assert int(step.status.item()) == 0, f"device status {int(step.status.item())}"

    # instrumented region: events around every stage of every step
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    run_steps(args.steps, first=0, events=evs)
    torch.cuda.synchronize()
    stage = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(6)] for e in evs]) * 1e3  # us
    st_mean = stage.mean(axis=0)
    names = ["mask_build", "attention", "softmax_pair", "-", "reject_sample", "-"]

    attn_b, logit_b, samp_b = algorithmic_bytes(inp)
    traffic = measured_traffic()
    step_b = attn_b + samp_b
    sm_us = st_mean[2]
    samp_us = st_mean[2] + st_mean[4] + st_mean[5]
    res = {
        "metric": METRIC,
        "value": round(1e3 / ms_per_step, 1),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 attention (fp32 accumulate), fp32 logits (fp64 sums)",
        "data": "synthetic (seeded; no dataset or weights)",
        "config": {
            "workload": synth.CONFIGS[args.config], "batch": inp["B"], "n_nodes": int(inp["n_nodes"].max()),
            "ctx": int(inp["ctx_len"].max()), "hq": inp["hq"], "hkv": inp["hkv"], "head_dim": inp["d"],
            "vocab": inp["V"], "T": inp["T"], "replicas": args.replicas, "launch": "stream (no graph)",
        },
        "step_bytes": step_b,
        "step_gbs": round(step_b / (ms_per_step * 1e-3) / 1e9, 1),
        "step_frac_of_hbm": round(step_b / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "attn_gbs": round(attn_b / (st_mean[1] * 1e-6) / 1e9, 1),
        "sampling_gbs": round(samp_b / (samp_us * 1e-6) / 1e9, 1),
        "stage_us": {n: round(float(v), 2) for n, v in zip(names, st_mean) if n != "-"},
        # the longest kernel of the step is the attention kernel; events bracket its call
        # (the attention kernel and the split combine), so the entry covers both
        "roofline": roofline_entry("spec_tree_attention call: attn_mfma_kernel<128> + attn_combine_kernel",
                                   attn_b, st_mean[1], traffic.get("spec_tree_attention")),
        "stage_roofline": {
            "softmax_pair": roofline_entry("spec_tree_softmax_pair call: softmax_stats_kernel + softmax_merge_kernel",
                                           samp_b, sm_us, traffic.get("spec_tree_softmax_pair")),
        },
    }

    if not args.no_cpu_baseline:
        import oracle

        threads = oracle.set_threads(min(16, os.cpu_count() or 1))
        n, t_start = 0, time.perf_counter()
        while True:
            oracle.verify_step(inp)
            n += 1
            if time.perf_counter() - t_start >= args.cpu_seconds:
                break
        el = time.perf_counter() - t_start
        res["cpu_baseline"] = {"value": round(n / el, 4), "unit": "steps/s", "cores": threads, "kind": "oracle",
                               "sample": f"{n} full steps of the same workload (all attention rows, lazy walk), "
                                         f"{el:.1f} s"}
    print(json.dumps(res))


if __name__ == "__main__":
    main()
