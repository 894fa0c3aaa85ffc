#!/usr/bin/env python3
"""Throughput of the Domino draft-head hot path on one MI355X.

One step = one draft block for every sequence of the batch: the
block-parallel base logits (domino_base_logits, LM-head GEMM on the MFMA
cores) followed by the 16-step causal-correction chain (domino_draft_chain),
inputs resident in HBM.  Metric: draft blocks per second.

Prints one JSON line.  `roofline` covers the launch that takes the most time
per step (the chain's persistent kernel or the LM-head GEMM), with its
algorithmic bytes (or flops) per launch divided by its average duration from
HIP events that the library records on the launch stream right around it
inside the timed region (domino_set_timing_events); `traffic` comes from the
committed rocprofv3 counter summary when it was taken on the current sources.  `cpu_baseline` times the oracle on a bounded sample of the same
workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MFMA_F32_PEAK_TFLOPS = 157.3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="qwen3_4b_b1")
    ap.add_argument("--chain-mode", type=int, default=0)
    ap.add_argument("--logits", action="store_true", help="also write the final logits")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only copy 256 MiB once on the device (counter calibration under rocprofv3 --pmc)")
    return ap.parse_args()


def copy_probe():
    """One 256 MiB device-to-device copy: a kernel of known traffic for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": src.numel() * 4, "copy_probe_bytes_written": dst.numel() * 4}))


def algorithmic_traffic(cfg, B, write_logits):
    """Bytes each launch must move and flops it must do, from the method's definition.

    base:  the LM-head GEMM, L^base = H W_lm^T (W_lm once, H, L^base out).
    chain: the P sequential steps; every step reads W2, the GRU weights, the
           state half of W1, one base-logit row and the fed-back embedding
           rows, whatever the kernel keeps on chip between steps.
    """
    es = 2 if cfg.dtype == "bf16" else 4
    d, V, Hs, r, P = cfg.hidden, cfg.vocab, cfg.gru_hidden, cfg.rank, cfg.block
    M = B * P
    base_bytes = V * d * es + M * d * es + M * V * 4
    base_flops = 2.0 * M * V * d
    step = (V * r * es                      # W2
            + 3 * Hs * (d + Hs) * es        # W_ih, W_hh
            + r * Hs * es                   # state half of W1
            + B * V * 4                     # base-logit row of this position
            + B * d * es                    # embedding rows of the fed-back tokens
            + (B * V * 4 if write_logits else 0))
    chain_bytes = P * step + M * r * 4 + M * 4  # + H half of the bottleneck in, tokens out
    chain_flops = 2.0 * P * B * (3 * Hs * (d + Hs) + r * Hs + V * r)
    return {"base": (base_bytes, base_flops), "chain": (chain_bytes, chain_flops), "chain_step_bytes": step}


def tree_traffic(cfg, B):
    """Bytes and flops of one tree call: the top-M pass over every base-logit row, then
    N rounds that each read the GRU weights, the state half of W1 and, per sequence,
    M rows of W2, M base-logit entries, one embedding row and two fp64 states."""
    es = 2 if cfg.dtype == "bf16" else 4
    d, V, Hs, r, P, N, M = cfg.hidden, cfg.vocab, cfg.gru_hidden, cfg.rank, cfg.block, cfg.nodes, cfg.topm
    topm_bytes = B * P * V * 4
    rnd = 3 * Hs * (d + Hs) * es + r * Hs * es + B * (M * r * es + M * 4 + d * es + 2 * Hs * 8)
    byts = topm_bytes + B * P * d * es + r * d * es + N * rnd
    flops = 2.0 * B * N * (3 * Hs * (d + Hs) + r * Hs + M * r) + 2.0 * B * P * r * d
    return byts, flops


def source_digest():
    """sha256 of the HIP sources; counter summaries are valid only for the sources they were taken on."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "draft_head_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_sha256") != source_digest() or kernel_key not in t.get("kernels", {}):
        return None
    k = t["kernels"][kernel_key]
    return (k["fetch_kib"] * t["fetch_scale"] + k["write_kib"] * t["write_scale"]) * 1024.0


def cpu_baseline(cfg, w, inp, target_s):
    """The oracle (plain C, OpenMP) on whole blocks of the same workload."""
    import numpy as np

    import oracle
    m = oracle.Model.from_config(cfg, w)
    done, t_start = 0, time.perf_counter()
    B = inp["t0"].size
    while True:
        b = done % B
        H = np.ascontiguousarray(inp["H"][b:b + 1])
        Lb = m.base_logits(H)
        if cfg.tree:
            m.tree(H, Lb, inp["t0"][b:b + 1], cfg.nodes, cfg.topm)
        else:
            m.chain(H, Lb, inp["t0"][b:b + 1], want_logits=False)
        done += 1
        el = time.perf_counter() - t_start
        if el >= target_s or done >= 64:
            break
    return {"value": done / el, "unit": "draft blocks/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{done} whole blocks (one sequence each: base logits + "
                      f"{f'{cfg.nodes}-node tree' if cfg.tree else f'{cfg.block}-step chain'}) of {cfg.name}, {el:.1f} s"}


def main():
    args = parse()
    if args.copy_probe:
        return copy_probe()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (see the sharding notes); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import draft_head_amd as dh
    import synth

    for so in ("synth/libsynth.so", "draft_head_amd/libdomino.so"):
        if not os.path.exists(os.path.join(ROOT, so)):
            import __graft_entry__
            __graft_entry__.build()
            break

    cfg = synth.CONFIGS[args.config]
    B = cfg.batch
    print(f"bench: generating {cfg.name} weights", file=sys.stderr, flush=True)
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    head = dh.DraftHead.from_config(cfg, w, "cuda:0")
    H = head.upload(inp["H"])
    t0 = head.upload(inp["t0"])
    dev = head.device
    P, V = cfg.block, cfg.vocab
    Lb = torch.empty((B, P, V), dtype=torch.float32, device=dev)
    toks = torch.empty((B, P), dtype=torch.int32, device=dev)
    logits = torch.empty((B, P, V), dtype=torch.float32, device=dev) if args.logits else None
    if cfg.tree:
        N, Mc = cfg.nodes, cfg.topm
        tree_out = {k: torch.empty((B, N), dtype=torch.int32, device=dev) for k in ("parents", "tokens", "depth")}
        tree_scores = torch.empty((B, N), dtype=torch.float64, device=dev)
        ws = torch.zeros(dh.domino_tree_workspace_size(head.dims, B, N, Mc), dtype=torch.uint8, device=dev)
    else:
        ws = head.workspace(B)
    dh.set_chain_mode(args.chain_mode)
    stream = torch.cuda.current_stream()

    def step():
        dh.domino_base_logits(head.dims, head.weights, H, B, Lb, stream)
        if cfg.tree:
            dh.domino_tree_draft(head.dims, head.weights, H, Lb, t0, B, N, Mc, tree_out["parents"],
                                 tree_out["tokens"], tree_out["depth"], tree_scores, ws, ws.numel(), stream)
        else:
            dh.domino_draft_chain(head.dims, head.weights, H, Lb, t0, B, toks, logits, ws, ws.numel(), stream)

    print("bench: warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert dh.DraftHead.device_status(ws) == 0

    # whole-step timing: no events inside, wall clock and bracketing events
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(K):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_per_step = e0.elapsed_time(e1) / K

    # durations of the main launch of each call: the library records these
    # events on the launch stream right around it
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for e in evs:  # torch creates the HIP event on its first record
        for x in e:
            x.record(stream)
    torch.cuda.synchronize()
    for i in range(K):
        dh.domino_set_timing_events(*evs[i])
        step()
    torch.cuda.synchronize()
    dh.domino_set_timing_events()
    t_base = np.mean([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    t_chain = np.mean([e[2].elapsed_time(e[3]) for e in evs]) * 1e-3
    assert dh.DraftHead.device_status(ws) == 0

    tr = algorithmic_traffic(cfg, B, args.logits)
    if cfg.tree:
        tr["chain"] = tree_traffic(cfg, B)
    peak_mfma = MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    kernel_key = {"base": "base_gemm", "chain": "chain_steps"}
    kernels = {}
    for name, t in (("base", t_base), ("chain", t_chain)):
        byts, flops = tr[name]
        ai = flops / byts
        ridge = peak_mfma * 1e12 / (HBM_PEAK_GBS * 1e9)
        if ai < ridge:
            kernels[name] = {"bound": "hbm", "achieved": byts / t / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        else:
            kernels[name] = {"bound": "mfma", "achieved": flops / t / 1e12, "peak": peak_mfma, "unit": "TFLOP/s"}
        k = kernels[name]
        k["frac"] = k["achieved"] / k["peak"]
        k["traffic"] = measured_traffic(cfg.name, kernel_key[name])
        k["us"] = t * 1e6
        k["algorithmic_bytes"] = byts
        k["flops"] = flops
    dom = "chain" if t_chain >= t_base else "base"
    roof = {kk: kernels[dom][kk] for kk in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    if cfg.tree:
        roof["kernel"] = "tree launches (domino_tree_draft)" if dom == "chain" else "LM-head GEMM (domino_base_logits)"
    else:
        one_launch = args.chain_mode == 2 or (args.chain_mode == 0 and B <= 8)
        roof["kernel"] = (("domino_draft_chain steps (" + ("chain_persistent, one launch" if one_launch
                                                           else "three launches per step") + ")")
                          if dom == "chain" else "LM-head GEMM (domino_base_logits)")

    value = B / (ms_per_step * 1e-3)
    out = {
        "metric": "draft blocks/sec (16-pos Domino chain, Qwen3-4B shape) + % of HBM/MFMA peak",
        "value": value,
        "unit": "draft blocks/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "block": P, "hidden": cfg.hidden, "vocab": V,
                   "gru_hidden": cfg.gru_hidden, "rank": cfg.rank, "chain_mode": args.chain_mode,
                   "write_logits": bool(args.logits), "parallelism": "none (one GPU)",
                   **({"tree_nodes": cfg.nodes, "tree_topm": cfg.topm} if cfg.tree else {})},
        "roofline": roof,
        "kernels": kernels,
        "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        print("bench: oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, w, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
