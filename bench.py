"""Benchmark of one tree-verification step on one MI355X.

A step is the whole hot path over one input set:
    spec_tree_attention (one layer's KV; given the parent links, the launch builds
    the ancestor rows of spec_tree_mask_build itself), spec_tree_softmax_pair
    (target and draft rows at T > 0; spec_tree_softmax at T = 0),
    spec_tree_reject_sample (whose final walk also writes the accepted path, the
    result of spec_accept_path).
The attention shares no data with the other two calls, so it can run on a second HIP
stream beside them, forked from and joined back into the timing stream by events.
``--streams auto`` (the default) times a short run of each form before the timed
region and keeps the faster: at the default workload the three calls in order on one
stream win (the attention kernel's registers leave no room on its CUs for the other
kernels' workgroups), at long contexts or large batches the second stream does
(the attention then outlasts the sampling half).  ``--streams one|two`` fixes it.
Workload (default): the Llama-3-8B-shaped step -- one request, a 60-node EAGLE-2
tree (top-k 10, depth 6), 4096 cached tokens, 32 query / 8 KV heads, head_dim 128,
bf16 KV, fp32 logits over a 128256-token vocabulary, T = 1.  Synthetic, seeded.

Timing: W warm-up steps, then K steps bracketed by synchronize + HIP events, queued
behind a short spin kernel so that the events time the GPU, not Python's launch rate.  Each
step reads one of R input replicas in turn (distinct device buffers, 8 x ~80 MB)
so the working set is far larger than the 256 MB last-level cache and the numbers
are HBM numbers.  A second timed pass records events around every stage to report
per-stage durations.  The call holding the longest kernel (tree attention) gives the
roofline entry and the logit softmax a second one; each is timed back to back on its
own, so no event sits between its kernels.  Measured HBM traffic per call comes
from the committed counter summary under profiles/ while the kernel sources match.
The sampling branch (logit pass + sampler), the step's critical path, is timed the
same way and reported with its own roofline entry.  A host-driven loop (no spin
ahead of it) gives the rate a serving loop on this host sees.  The request is then
verified under 2048 independent uniform sets for the accepted-length distribution
(tau, per-depth acceptance).  The CPU oracle is timed on the host on full steps of the same
workload (multi-threaded, and on one thread), and checks the first 32 of those
trials (near-tie and identical counts).  A third pass with one event per step
boundary gives the p10 / p50 / p90 of single steps.  After the timed regions come a
32-layer-equivalent step (32 attention calls over their own KV beside one sampling
pass), and, under "next_rows", the KV commit that follows a step (one layer, and 32
layers in one call, the deepest path of the tree, on a scratch copy of the cache) and
the draft-tree construction (EAGLE-2 and best-first).  Prints one JSON line.

``--cost-table PREFIX`` instead sweeps the step over (batch, context, nodes) and writes
the verify-latency table (PREFIX.json, PREFIX.md) that cost_table.CostTable reads.
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
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
COPY_ELEMS = 1 << 27  # fp32: 512 MiB read and 512 MiB written per copy
# HBM bytes per call measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (scaled by the
# same counters on a plain copy); valid only while the sources listed there are unchanged
COUNTERS_MD = os.path.join(ROOT, "profiles", "verify_step_llama8b_60node_ctx4096_hbm_counters.md")


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


def roofline_entry(kernel, nbytes, us, traffic, flops=0):
    """HBM roofline entry, or the bf16 MFMA one when the call's arithmetic intensity is
    above the ridge (peak FLOP/s / peak bytes/s)."""
    if flops and flops / nbytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        tf = flops / (us * 1e-6) / 1e12
        return {"kernel": kernel, "bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                "flops_per_launch": int(flops), "bytes_per_launch": int(nbytes), "avg_launch_us": round(float(us), 3)}
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
    ap.add_argument("--streams", choices=("auto", "one", "two", "step"), default="auto",
                    help="one: the separate calls on one stream; two: the attention on a second stream beside the "
                         "logit pass and the sampler; step: the single spec_tree_verify_step call (the attention's "
                         "split combine inside the logit pass's launch); auto: time a short run of each, keep the "
                         "fastest")
    ap.add_argument("--overlap", action="store_true", help="the same as --streams two")
    ap.add_argument("--fork", choices=("start", "after_softmax"), default="start",
                    help="with --overlap: where the second stream branches off, at the step's start or after "
                         "the logit pass")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cost-table", metavar="PREFIX", default=None,
                    help="sweep (batch, context, nodes) and write PREFIX.json and PREFIX.md: the verify-latency "
                         "table a cost-aware tree harness calibrates on")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run four plain 512 MiB device-to-device copies (the reference kernel whose "
                         "FETCH_SIZE / WRITE_SIZE counters scale the traffic of the step's kernels)")
    return ap.parse_args()


def internal_rows(inp):
    """Node rows whose node has at least one child (the rows whose draft logits the
    sampler reads: a leaf's draft row takes no part)."""
    n = 0
    for b in range(inp["B"]):
        nb, par = int(inp["n_nodes"][b]), inp["parent"][b]
        n += len({int(par[c]) for c in range(1, nb)})
    return n


def algorithmic_bytes(inp):
    """Bytes the step must move at least once: KV of every request (prompt + tree),
    Q and O, the target logits of every node row, and at T > 0 the draft logits of
    the rows of nodes with children."""
    B, n_max, hq, hkv, d = inp["B"], inp["n_max"], inp["hq"], inp["hkv"], inp["d"]
    el = 2 if inp["bf16"] else 4
    kv_tokens = int(np.sum(inp["ctx_len"] + inp["n_nodes"]))
    attn = 2 * kv_tokens * hkv * d * el + 2 * B * n_max * hq * d * el
    logits = B * n_max * inp["V"] * 4
    sampling = logits + (internal_rows(inp) * inp["V"] * 4 if inp["T"] > 0 else 0)
    return attn, logits, sampling


def attention_flops(inp):
    """Matrix FLOPs of the attention call: S = Q K^T and O = P V for every node and query
    head against every key of its request (prompt and tree; ancestors are masked after
    the product), 2 FLOPs per multiply-add."""
    n = inp["n_nodes"].astype(np.int64)
    return int(4 * inp["hq"] * inp["d"] * np.sum(n * (inp["ctx_len"].astype(np.int64) + n)))


def copy_calibration():
    import torch

    a = torch.ones(COPY_ELEMS, device="cuda")
    b = torch.empty_like(a)
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": a.numel() * 4, "bytes_written": b.numel() * 4,
                                           "launches": 4}}))


_SLEEP_CYCLES_PER_MS = None


def prefill(ms=20.0):
    """Hold the GPU on a short spin kernel while the host queues the timed work behind
    it, so that the timed region measures the GPU and not the Python launch rate."""
    global _SLEEP_CYCLES_PER_MS
    import torch

    if _SLEEP_CYCLES_PER_MS is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = 1e6 / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(_SLEEP_CYCLES_PER_MS * ms))


def run_steps(step, replicas, stream, n, first=0, events=None):
    """n steps, rotating over the input replicas; with events, 7 events per step
    bracket the stages (mask build unless the attention builds the ancestor rows
    itself, attention, softmax, -, reject + path, -)."""
    for i in range(n):
        r = replicas[(first + i) % len(replicas)]
        if events is None:
            if getattr(step, "_plans", None):
                step.run_fast((first + i) % len(replicas))  # the recorded calls of replica r
            else:
                step.run(replica=r)
            continue
        ev = events[i]
        ev[0].record(stream)
        if not step.fold_mask:  # (folded: the attention call builds the ancestor rows itself)
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


def host_prefill_ms(host_us_per_step, steps):
    """A spin long enough for the host to queue `steps` steps behind it (with margin)."""
    return max(20.0, 1.5 * host_us_per_step * steps / 1e3 + 5.0)


def gpu_time_us(fn, iters, warmup, stream=None):
    """GPU time per call of fn() (us), fn issued `iters` times back to back after
    `warmup` untimed calls, queued behind a spin sized from the host's measured
    queueing time per call.  Returns (us per call, host us per call, host ahead)."""
    import torch

    h = time.perf_counter()
    for i in range(warmup):
        fn(i)
    host_us = (time.perf_counter() - h) * 1e6 / max(warmup, 1)
    torch.cuda.synchronize()
    pre = host_prefill_ms(host_us, iters)
    prefill(pre)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    h = time.perf_counter()
    for i in range(iters):
        fn(i)
    queued_ms = (time.perf_counter() - h) * 1e3
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / iters, queued_ms * 1e3 / iters, queued_ms < pre


def time_steps(step, replicas, stream, steps, warmup, info=None):
    """(ms per step over a clean timed region, mean us per stage from an instrumented pass).
    The spin kernel ahead of each timed region is sized from the host's measured
    queueing time per step, so the GPU never waits for the host inside the region;
    `info` (a dict) receives that time and whether the host finished queueing first."""
    import torch

    h = time.perf_counter()
    run_steps(step, replicas, stream, warmup)
    host_us = (time.perf_counter() - h) * 1e6 / max(warmup, 1)
    torch.cuda.synchronize()
    pre = host_prefill_ms(host_us, steps)
    prefill(pre)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    h = time.perf_counter()
    run_steps(step, replicas, stream, steps, first=warmup)
    queued_ms = (time.perf_counter() - h) * 1e3
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / steps
    if info is not None:
        info.update(host_queue_us_per_step=round(queued_ms * 1e3 / steps, 2), spin_ms=round(pre, 1),
                    host_ahead=bool(queued_ms < pre))
    assert int(step.status.item()) == 0, f"device status {int(step.status.item())}"
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
    prefill(2 * pre)  # this pass records seven events per step as well
    run_steps(step, replicas, stream, steps, first=0, events=evs)
    torch.cuda.synchronize()
    stage = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(6)] for e in evs]) * 1e3  # us
    return ms_per_step, stage.mean(axis=0)


def time_calls(call, replicas, iters=200):
    """Average duration (us) of one library call issued back to back, rotating over the
    input replicas, queued behind a spin kernel: the call's kernels and the gaps
    between them, without the per-stage events of the instrumented pass."""
    us, _, _ = gpu_time_us(lambda i: call(replicas[i % len(replicas)]), iters, 10)
    return us


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def step_percentiles(step, replicas, stream, steps, first=0):
    """Per-step durations (us) of the clean step sequence from one event at every step
    boundary on the caller's stream (which the step joins), as p10 / p50 / p90; each
    event adds its own small cost to the step it closes."""
    import torch

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    h = time.perf_counter()
    step.run(replica=replicas[first % len(replicas)])
    torch.cuda.synchronize()
    prefill(host_prefill_ms((time.perf_counter() - h) * 1e6, steps))
    ev[0].record(stream)
    for i in range(steps):
        if getattr(step, "_plans", None):
            step.run_fast((first + i) % len(replicas))
        else:
            step.run(replica=replicas[(first + i) % len(replicas)])
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    d = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]) * 1e3
    return {"p10": round(float(np.percentile(d, 10)), 2), "p50": round(float(np.percentile(d, 50)), 2),
            "p90": round(float(np.percentile(d, 90)), 2), "mean": round(float(d.mean()), 2), "steps": steps}


def deepest_paths(parent, n_nodes):
    """Per request, the root-to-leaf path to the first deepest node (a full accept)."""
    B, n_max = parent.shape
    path = np.zeros((B, n_max), np.int32)
    L = np.zeros(B, np.int32)
    for b in range(B):
        depth = np.zeros(n_max, np.int64)
        for i in range(1, int(n_nodes[b])):
            depth[i] = depth[parent[b, i]] + 1
        j, chain = int(np.argmax(depth[: int(n_nodes[b])])), []
        while j > 0:
            chain.append(j)
            j = int(parent[b, j])
        chain = [0] + chain[::-1]
        path[b, : len(chain)] = chain
        L[b] = len(chain) - 1
    return path, L


def time_layers_step(step, dev, replicas, stream, layers=32, iters=20, warmup=3):
    """The 32-layer-equivalent step: one attention call per layer over its own KV
    buffers (the same Q), beside one sampling pass (two streams, as the step).
    Returns us per step and the attention bytes' rate."""
    import torch

    kv = [(torch.randn_like(dev["k"]), torch.randn_like(dev["v"])) for _ in range(layers)]
    side = step.side if step.side is not None else stream

    def one(r):
        if side is not stream:
            step.ev_fork.record(stream)
            side.wait_event(step.ev_fork)
        if not step.fold_mask:
            step.mask(side)
        for k, v in kv:
            step.attention(side, r["q"], k, v)
        if side is not stream:
            step.ev_join.record(side)
        step.softmax(stream, r["tgt_logits"], r.get("dft_logits"))
        step.reject(stream, r["tgt_logits"], r.get("dft_logits"))
        if side is not stream:
            stream.wait_event(step.ev_join)

    us, _, _ = gpu_time_us(lambda i: one(replicas[i % len(replicas)]), iters, warmup, stream)
    del kv
    return us


def time_kv_commit(step, dev, k_src, v_src, stream, iters=200, layers=1):
    """The commit after the step (``layers`` layers' K and V, in one call: one layer, or
    a whole model's cache stacked on a leading axis) along each tree's deepest path
    (every draft token accepted, the most rows a commit moves), timed on a scratch copy
    of the cache with back-to-back calls.  Repeating a commit is valid on a contiguous
    cache (it copies the same rows again); a paged one has its pages released by the
    first call, so it is not timed here."""
    import torch

    from tree_verification_masked_amd import binding as Bd

    if dev.get("block_table") is not None or not step.with_attention:
        return None
    if layers == 1:
        k, v = k_src.clone(), v_src.clone()
    else:
        k = k_src.unsqueeze(0).repeat(layers, *([1] * k_src.dim()))
        v = v_src.unsqueeze(0).repeat(layers, *([1] * v_src.dim()))
    Bn = dev["B"]
    new_len = torch.zeros(Bn, dtype=torch.int32, device=k.device)
    status = torch.zeros(1, dtype=torch.int32, device=k.device)
    path_h, L = deepest_paths(dev["parent"].cpu().numpy(), dev["n_nodes"].cpu().numpy())
    path, acc = torch.from_numpy(path_h).to(k.device), torch.from_numpy(L).to(k.device)

    def call():
        Bd.spec_tree_kv_commit(k, v, dev["ctx_len"], dev["n_nodes"], path, acc, new_len, status=status)

    us, _, _ = gpu_time_us(lambda i: call(), iters, 10, stream)
    L = L.astype(np.int64)
    assert int(status.item()) == 0, f"device status {int(status.item())}"
    assert np.array_equal(new_len.cpu().numpy(), dev["ctx_len"].cpu().numpy() + 1 + L)
    el = k.element_size()
    moved = layers * int(L.sum()) * dev["hkv"] * dev["d"] * el * 2 * 2  # K and V rows, read once, written once
    del k, v
    return {"call": f"spec_tree_kv_commit ({layers} layer{'s' if layers > 1 else ''}, contiguous KV)",
            "layers": layers, "us": round(us, 2),
            "accept_len": [int(x) for x in L], "bytes_moved": moved,
            "gbs": round(moved / (us * 1e-6) / 1e9, 2), "iters": iters,
            "note": "deepest path of each tree; back-to-back calls queued behind a spin kernel, on a scratch "
                    "copy after the timed region"}


def time_tree_build(seed, iters=100, V=128256, k=10, depth=6, n_final=60, select_k=None, policy="layer"):
    """Draft-tree construction on the GPU for the 60-node verify tree: init, the expand
    rounds (top-10 over a 128256-token vocabulary; EAGLE-2 layer rounds or best-first
    pops) and the rerank, with the draft rows of every round already resident
    (generated once, per node path).  The rows a round reads are its algorithmic bytes."""
    sk = k if select_k is None else select_k
    import torch

    import synth
    from tree_verification_masked_amd.draft_tree import DraftTree

    dt = DraftTree(1, 1024, sk, V)
    root = torch.tensor([int(np.random.default_rng(seed).integers(V))], dtype=torch.int32, device="cuda")
    dt.init(root)
    rounds, row_bytes = [], 0
    for _ in range(depth):  # one untimed build fixes each round's frontier and rows
        st = dt.host_state()
        rows = np.zeros((1, sk, V), np.float32)
        fc = int(st["frontier_count"][0])
        for j in range(fc):
            nd, path = int(st["frontier"][0, j]), []
            while nd >= 0:
                path.append(int(st["token"][0, nd]))
                nd = int(st["parent"][0, nd])
            rows[0, j] = synth.path_row(seed, tuple(path[::-1]), V)
        rounds.append(torch.from_numpy(rows).cuda())
        row_bytes += fc * V * 4
        dt.expand(rounds[-1], 1.0, k, sk, policy=policy)
    out = dt.rerank(n_final)
    torch.cuda.synchronize()
    ref = [t.clone() for t in out]

    def build():
        dt.init(root)
        for r in rounds:
            dt.expand(r, 1.0, k, sk, policy=policy)
        dt.rerank(n_final, out=out)

    us, host_us, ahead = gpu_time_us(lambda i: build(), iters, 5)
    assert int(dt.status.item()) == 0 and all(torch.equal(a, b) for a, b in zip(out, ref))
    kind = f"EAGLE-2 top-{k}, depth {depth}" if policy == "layer" else \
        f"best-first top-{k}, {depth} rounds of {sk} pops"
    return {"call": f"spec_tree_build_init + {depth} x spec_tree_expand + spec_tree_rerank (1 request)",
            "workload": f"{kind}, {n_final} nodes, vocabulary {V}, T_d = 1",
            "us_per_tree": round(us, 2), "host_queue_us_per_tree": round(host_us, 1), "host_ahead": bool(ahead),
            "draft_row_bytes": row_bytes,
            "gbs": round(row_bytes / (us * 1e-6) / 1e9, 1), "iters": iters,
            "note": "the drafter's rows are inputs (resident); its forward passes are not part of this"}


def gpu_tree_builder(row_of, root_token, T_d, top_k, depth, n_final):
    """The EAGLE-2 tree of a workload built on the GPU by the library's own calls
    (spec_tree_build_init, ``depth`` spec_tree_expand rounds, spec_tree_rerank), the
    drafter's rows supplied per frontier node by ``row_of(path)``; returns the
    flattened tree and each node's root path (the input hook of synth.make_config)."""
    import torch

    from tree_verification_masked_amd.draft_tree import DraftTree

    V = int(np.asarray(row_of((int(root_token),))).shape[0])
    dt = DraftTree(1, 1024, top_k, V)
    dt.init(torch.tensor([int(root_token)], dtype=torch.int32, device="cuda"))

    def path_of(st, nd):
        out = []
        while nd >= 0:
            out.append(int(st["token"][0, nd]))
            nd = int(st["parent"][0, nd])
        return tuple(out[::-1])

    for _ in range(depth):
        st = dt.host_state()
        fc = int(st["frontier_count"][0])
        if fc == 0:
            break
        rows = np.zeros((1, top_k, V), np.float32)
        for j in range(fc):
            rows[0, j] = row_of(path_of(st, int(st["frontier"][0, j])))
        dt.expand(torch.from_numpy(rows).cuda(), T_d, top_k, top_k)
    parent, tokens, n_nodes, cand_id = dt.rerank(n_final)
    st = dt.host_state()
    assert int(st["status"][0]) == 0, f"tree build status {int(st['status'][0])}"
    n = int(n_nodes[0].item())
    ids = cand_id[0, :n].cpu().numpy()
    return parent[0, :n].cpu().numpy(), tokens[0, :n].cpu().numpy(), [path_of(st, int(i)) for i in ids]


COST_GRID = {"batch": (1, 2, 4, 8), "ctx": (1024, 4096, 16384), "n_nodes": (16, 32, 64)}


def cost_table(args):
    """Verify latency of the whole step (and its attention and sampling calls) over
    (batch, context, nodes): random breadth-first trees (branching 1..4, depth <= 8),
    Llama-3-8B head geometry, bf16 KV, vocabulary 128256.  One input at the largest
    point; every point takes the first B requests, the first N nodes of each tree and
    context C, each in enough replicas to exceed the last-level cache."""
    import torch

    import synth
    from tree_verification_masked_amd.step import VerifyStep, to_device

    torch.cuda.set_device(0)
    cuda = torch.device("cuda")
    bm, cm, nm = max(COST_GRID["batch"]), max(COST_GRID["ctx"]), max(COST_GRID["n_nodes"])
    inp = synth.make_config(6, seed=args.seed, T=args.temperature, with_kv=False, grid=(bm, cm, nm))
    par = inp["parent"]
    assert np.all(par[:, 0] == -1) and np.all(par[:, 1:] < np.arange(1, nm)[None, :])  # prefixes are trees
    base = to_device(inp)
    g = torch.Generator(device=cuda)
    g.manual_seed(args.seed)
    hq, hkv, d = inp["hq"], inp["hkv"], inp["d"]
    qf = torch.randn((bm, nm, hq, d), generator=g, device=cuda, dtype=torch.bfloat16)
    kf = torch.randn((bm, cm + nm, hkv, d), generator=g, device=cuda, dtype=torch.bfloat16)
    vf = torch.randn((bm, cm + nm, hkv, d), generator=g, device=cuda, dtype=torch.bfloat16)
    stream = torch.cuda.current_stream()
    V = inp["V"]
    rows = []
    for Bn in COST_GRID["batch"]:
        for ctx in COST_GRID["ctx"]:
            for N in COST_GRID["n_nodes"]:
                pt = dict(base)
                for key in ("parent", "tokens", "tgt_logits", "dft_logits", "u_accept", "u_sample"):
                    pt[key] = base[key][:Bn, :N].contiguous()
                pt.update(B=Bn, n_max=N, kv_capacity=ctx + N, max_kv_len=ctx + N,
                          n_nodes=torch.full((Bn,), N, dtype=torch.int32, device=cuda),
                          ctx_len=torch.full((Bn,), ctx, dtype=torch.int32, device=cuda))
                kv_b = 2 * Bn * (ctx + N) * hkv * d * 2
                lg_b = Bn * N * V * 4 * (2 if inp["T"] > 0 else 1)
                reps = int(min(32, max(2, -(-(1 << 30) // (kv_b + lg_b)))))
                replicas = []
                for _ in range(reps):
                    replicas.append({"q": qf[:Bn, :N].clone(), "k": kf[:Bn, : ctx + N].clone(),
                                     "v": vf[:Bn, : ctx + N].clone(), "tgt_logits": pt["tgt_logits"].clone(),
                                     "dft_logits": pt["dft_logits"].clone()})
                pt.update(q=replicas[0]["q"], k=replicas[0]["k"], v=replicas[0]["v"])
                step = VerifyStep(pt).one_call()
                ms, st = time_steps(step, replicas, stream, args.steps, args.warmup)
                rows.append({"batch": Bn, "ctx": ctx, "n_nodes": N, "step_us": round(ms * 1e3, 2),
                             "attention_us": round(float(st[1]), 2),
                             "sampling_us": round(float(st[2] + st[4]), 2), "replicas": reps,
                             "mean_accept_len": round(float(step.accept_len.float().mean().item()), 3)})
                if not step.fold_mask:
                    rows[-1]["mask_us"] = round(float(st[0]), 2)
                print(json.dumps({"cost_point": rows[-1]}), flush=True)
                del replicas, step, pt
                torch.cuda.empty_cache()
    meta = {"what": "verify latency of one tree-verification step (one layer's attention, its ancestor rows built "
                    "from the parent links, + full-vocabulary sampling) on one MI355X, HIP events, inputs resident "
                    "in HBM; the step is the single spec_tree_verify_step call (the attention's split combine in the "
                    "logit pass's launch); the attention and sampling columns come from a pass of the separate calls "
                    "with events around each stage",
            "workload": synth.CONFIGS[6], "T": inp["T"], "hq": hq, "hkv": hkv, "head_dim": d, "vocab": V,
            "steps": args.steps, "warmup": args.warmup, "seed": args.seed, "grid": COST_GRID,
            "command": " ".join(["python", "bench.py"] + sys.argv[1:])}
    with open(args.cost_table + ".json", "w") as f:
        json.dump({"meta": meta, "rows": rows}, f, indent=1)
    with open(args.cost_table + ".md", "w") as f:
        f.write("# Verify-latency cost table (one MI355X)\n\n")
        f.write(f"{meta['what']}.  Workload: {meta['workload']}; T = {meta['T']}.  "
                f"{args.steps} timed steps per point after {args.warmup} warm-up steps.\n\n")
        f.write(f"Command: `{meta['command']}`\n\n")
        f.write("| batch | ctx | nodes | step us | attention us | sampling us | mean accept len |\n")
        f.write("|---:|---:|---:|---:|---:|---:|---:|\n")
        for r in rows:
            f.write(f"| {r['batch']} | {r['ctx']} | {r['n_nodes']} | {r['step_us']} | {r['attention_us']} | "
                    f"{r['sampling_us']} | {r['mean_accept_len']} |\n")
    print(json.dumps({"cost_table": args.cost_table, "points": len(rows)}))


def acceptance_trials(inp, dev, n_trials=2048, batch=256, seed=0):
    """The step's request verified under n_trials independent sets of uniforms (the
    tree, its tokens and logit rows fixed): the distribution of the accepted length
    L and of tau = L + 1 tokens per step (the bonus included).  Runs the library's
    softmax and sampling calls on `batch` copies of the request at a time.  Returns
    (summary dict, first batch's inputs and outputs for the oracle check)."""
    import torch

    import synth
    from tree_verification_masked_amd.step import VerifyStep

    n, V = inp["n_max"], inp["V"]
    rows = {k: dev[k][:1].expand(batch, n, V).contiguous() for k in ("tgt_logits", "dft_logits") if k in dev}
    small = dict(parent=np.repeat(inp["parent"][:1], batch, 0), tokens=np.repeat(inp["tokens"][:1], batch, 0),
                 n_nodes=np.repeat(inp["n_nodes"][:1], batch, 0), ctx_len=np.zeros(batch, np.int32))
    d = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in small.items()}
    d.update(rows, B=batch, n_max=n, V=V, T=inp["T"], Td=inp["Td"], max_kv_len=n)
    st = VerifyStep(d, with_attention=False)
    Ls, first = [], None
    for i in range(-(-n_trials // batch)):
        rng = synth.rng_for(seed, 12345, i)
        ua, us = synth.uniforms(rng, (batch, n)), synth.uniforms(rng, (batch, n))
        d["u_accept"], d["u_sample"] = torch.from_numpy(ua).cuda(), torch.from_numpy(us).cuda()
        st.softmax()
        st.reject()
        r = st.results()
        assert int(r["status"][0]) == 0
        Ls.append(r["accept_len"].copy())
        if first is None:
            first = dict(small, u_accept=ua, u_sample=us, out=r)
    L = np.concatenate(Ls)[:n_trials]
    depth = np.zeros(n, np.int64)
    for i in range(1, int(inp["n_nodes"][0])):
        depth[i] = depth[inp["parent"][0, i]] + 1
    D = int(depth.max())
    ge = [float((L >= k).mean()) for k in range(D + 1)]
    return {
        "trials": int(L.size),
        "what": "the timed request under independent uniform sets (tree, tokens and logits fixed)",
        "mean_accept_len": round(float(L.mean()), 4),
        "tau_mean": round(float(L.mean()) + 1, 4),
        "accept_len_hist": np.bincount(L, minlength=D + 1).tolist(),
        "p_accept_len_ge": [round(x, 4) for x in ge[1:]],
        "per_depth_acceptance": [round(ge[k] / ge[k - 1], 4) if ge[k - 1] > 0 else None for k in range(1, D + 1)],
    }, first


def oracle_check(inp, first, m=32):
    """The oracle on the first m of the acceptance trials: near-tie requests (flag on
    the oracle's path) and requests whose GPU outputs equal the oracle's."""
    import oracle

    sub = {k: first[k][:m] for k in ("parent", "tokens", "n_nodes", "u_accept", "u_sample")}
    tgt = np.broadcast_to(inp["tgt_logits"][:1], (m,) + inp["tgt_logits"].shape[1:])
    dft = np.broadcast_to(inp["dft_logits"][:1], (m,) + inp["dft_logits"].shape[1:]) if inp["T"] > 0 else None
    r = oracle.reject_sample(tgt, dft, inp["T"], inp["Td"], sub["tokens"], sub["parent"], sub["n_nodes"],
                             sub["u_accept"] if inp["T"] > 0 else None, sub["u_sample"] if inp["T"] > 0 else None)
    r.update(oracle.accept_path(r["accepted_child"], r["term_token"], sub["tokens"], sub["n_nodes"]))
    g = first["out"]
    ties = same = 0
    for b in range(m):
        pn = r["path_nodes"][b]
        if r["tie_flags"][b][pn[pn >= 0]].any():
            ties += 1
        if all(np.array_equal(g[k][b], r[k][b]) for k in ("path_nodes", "out_tokens", "accepted_child",
                                                          "term_token")):
            same += 1
    return {"trials": m, "near_tie_requests": ties, "identical_to_oracle": same}


def host_driven(step, replicas, steps):
    """Steps/s of a loop that the host drives with no spin ahead of it: the host's
    issue time included (the replayed calls of compile())."""
    import torch

    torch.cuda.synchronize()
    t = time.perf_counter()
    for i in range(steps):
        step.run_fast(i % len(replicas))
    torch.cuda.synchronize()
    el = time.perf_counter() - t
    return {"steps_per_s": round(steps / el, 1), "us_per_step": round(el * 1e6 / steps, 2), "steps": steps}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus == 1 and args.cost_table:
        cost_table(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    from tree_verification_masked_amd.step import VerifyStep, to_device

    torch.cuda.set_device(0)
    T = args.temperature if args.config != 3 else None
    inp = synth.make_config(args.config, seed=args.seed, T=T, tree_builder=gpu_tree_builder)
    dev = to_device(inp)
    big = [k for k in ("q", "k", "v", "tgt_logits", "dft_logits") if k in dev]
    replicas = [{k: dev[k].clone() for k in big} for _ in range(args.replicas)]
    stream = torch.cuda.current_stream()

    def make_step(mode):
        s = VerifyStep(dev)
        if mode == "two":
            s.overlap(fork=args.fork)  # the attention on a second stream
        elif mode == "step":
            s.one_call()
        s.compile(replicas, stream)  # the timed steps replay recorded calls: less host time per step
        return s

    mode = "two" if args.overlap else args.streams
    probe = None
    if mode == "auto":  # a short timed run of each form; the timed region uses the faster
        probe = {}
        for m in ("one", "two", "step"):
            ms, _ = time_steps(make_step(m), replicas, stream, 50, 10)
            probe[m] = round(ms * 1e3, 2)
        mode = min(probe, key=probe.get)
    step = make_step(mode)

    # warm-up, the clean timed region, then an instrumented pass with events around
    # every stage of every step
    timing = {}
    ms_per_step, st_mean = time_steps(step, replicas, stream, args.steps, args.warmup, timing)
    pct = step_percentiles(step, replicas, stream, args.steps)
    names = ["mask_build" if not step.fold_mask else "-", "attention", "softmax_pair", "-", "reject_sample", "-"]

    attn_b, logit_b, samp_b = algorithmic_bytes(inp)
    traffic = measured_traffic()
    # the two bandwidth calls on their own, back to back (their roofline entries)
    attn_us = time_calls(lambda r: step.attention(None, r["q"], r["k"], r["v"]), replicas) \
        if step.with_attention else float("nan")
    pair_us = time_calls(lambda r: step.softmax(None, r["tgt_logits"], r.get("dft_logits")), replicas)

    def branch(r):  # the sampling branch: the logit pass, then the sampler (with its walk)
        step.softmax(None, r["tgt_logits"], r.get("dft_logits"))
        step.reject(None, r["tgt_logits"], r.get("dft_logits"))

    branch_us = time_calls(branch, replicas)
    reject_us = time_calls(lambda r: step.reject(None, r["tgt_logits"], r.get("dft_logits")), replicas)
    step_b = attn_b + samp_b
    samp_us = st_mean[2] + st_mean[4] + st_mean[5]
    # one stream runs the parts in turn; two streams run the attention beside the sampling half
    crit_us = attn_us + branch_us if step.side is None else max(attn_us, branch_us)
    if step.composite:  # one call on one stream: its three launches in turn are the whole step
        crit_us = ms_per_step * 1e3
    hd = host_driven(step, replicas, args.steps)
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
            "vocab": inp["V"], "T": inp["T"], "replicas": args.replicas,
            "launch": "one spec_tree_verify_step call: attention, logit pass with the split combine, sampler "
                      "(one stream, no graph)" if step.composite else "one stream (no graph)" if step.side is None else
                      ("two streams: the attention (ancestor rows built in its launch) beside softmax + sampling "
                       "(no graph)" if step.fork == "start"
                       else "two streams: the attention beside the sampling, after the logit pass (no graph)"),
        },
        # one event per step boundary: the distribution of single steps (the events'
        # own cost included, so the mean sits a little above ms_per_step)
        "step_us_percentiles": pct,
        # the host's queueing time per step and whether it stayed ahead of the GPU
        "host_queue": timing,
        "step_bytes": step_b,
        "step_gbs": round(step_b / (ms_per_step * 1e-3) / 1e9, 1),
        "step_frac_of_hbm": round(step_b / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        # HBM bytes per single-call step from the counters (null for another form or stale counters)
        "step_traffic": traffic.get("spec_tree_verify_step") if step.composite else None,
        "attn_gbs": round(attn_b / (attn_us * 1e-6) / 1e9, 1),
        "sampling_gbs": round(samp_b / (samp_us * 1e-6) / 1e9, 1),
        "stage_us": {n: round(float(v), 2) for n, v in zip(names, st_mean) if n != "-"},
        # the longest kernel of the step is the attention kernel; events bracket its call
        # (the attention kernel and the split combine), so the entry covers both
        # avg_launch_us: the call timed back to back on its own (time_calls); stage_us
        # holds the same calls inside the step, each bracketed by events
        "roofline": roofline_entry("spec_tree_attention call: attn_mfma_kernel<128> + attn_combine_kernel",
                                   attn_b, attn_us, traffic.get("spec_tree_attention"), attention_flops(inp)),
        "stage_roofline": {
            # the logit pass alone: chunk partials of both logit arrays, one launch
            "softmax_pair": roofline_entry("spec_tree_softmax_pair call: softmax_stats_kernel (target and draft "
                                           "rows, chunk partials only)",
                                           samp_b, pair_us, traffic.get("spec_tree_softmax_pair")),
            # the sampling half of the step: the logit pass and the sampler, against the
            # bytes of one pass over both logit arrays
            "sampling_branch": roofline_entry("spec_tree_softmax_pair + spec_tree_reject_sample calls: "
                                              "softmax_stats_kernel, sample_kernel",
                                              samp_b, branch_us, traffic.get("sampling_branch")),
        },
        # the step's parts, each timed back to back on its own: one stream runs them in
        # turn; with two streams the attention runs beside the sampling half
        "critical_path": {
            "branch": ("spec_tree_verify_step: the attention kernel, the logit pass with the split combine, the "
                       "sampler (the whole step)" if step.composite else
                       "attention, then softmax_pair + reject_sample" if step.side is None else
                       "softmax_pair + reject_sample (the attention branch runs beside it)" if branch_us >= attn_us
                       else "attention (the sampling half runs beside it)"),
            "us": round(crit_us, 2),
            "share_of_step": round(crit_us / (ms_per_step * 1e3), 3),
            "reject_sample_us": round(reject_us, 2), "softmax_pair_us": round(pair_us, 2),
            "sampling_half_us": round(branch_us, 2),
            "attention_call_us": round(attn_us, 2),
        },
        # the same replayed steps driven by the host with nothing queued ahead: what a
        # serving loop on this host gets, host issue time included
        "host_driven": hd,
        # the stream form the timed steps used, and (auto) the short runs that chose it
        "streams": {"used": mode, "probe_us_per_step": probe},
    }
    acc, first = acceptance_trials(inp, dev, seed=args.seed)
    res["acceptance"] = acc
    if "k" in dev and dev.get("block_table") is None:
        res["next_rows"] = {
            "kv_commit": time_kv_commit(step, dev, replicas[0]["k"], replicas[0]["v"], stream),
            # every layer of a 32-layer model (the Llama-3-8B depth) in one call
            "kv_commit_32_layers": time_kv_commit(step, dev, replicas[0]["k"], replicas[0]["v"], stream, layers=32),
        }
    res.setdefault("next_rows", {})["tree_build"] = time_tree_build(args.seed)
    # the best-first (heap) variant: 16 rounds of 4 pops, top-8 children
    if step.with_attention and dev.get("block_table") is None:
        us32 = time_layers_step(step, dev, replicas, stream)
        res["step_32_layers"] = {
            "what": "32 attention calls (one per layer, each over its own KV buffers) beside one sampling "
                    "pass; the pages name no layer count, so this is a secondary figure",
            "us_per_step": round(us32, 2), "steps_per_s": round(1e6 / us32, 1),
            "attention_gbs": round(32 * attn_b / (us32 * 1e-6) / 1e9, 1)}
    res["next_rows"]["tree_build_best_first"] = time_tree_build(args.seed, k=8, depth=16, select_k=4,
                                                                policy="best_first")

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
                                         f"{el:.1f} s", "cpu": cpu_model(), "host_cores": os.cpu_count()}
        # the same oracle on one thread, a few steps (about 1 / threads of the rate)
        oracle.set_threads(1)
        n1, t_start = 0, time.perf_counter()
        while True:
            oracle.verify_step(inp)
            n1 += 1
            if time.perf_counter() - t_start >= args.cpu_seconds / 2:
                break
        el1 = time.perf_counter() - t_start
        res["cpu_baseline"]["single_thread"] = {"value": round(n1 / el1, 4), "unit": "steps/s", "cores": 1,
                                                "sample": f"{n1} full steps, {el1:.1f} s"}
        oracle.set_threads(threads)
        res["acceptance"]["oracle_check"] = oracle_check(inp, first)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
