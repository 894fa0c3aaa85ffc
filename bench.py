#!/usr/bin/env python3
"""Throughput of the Domino draft-head hot path on one MI355X.

One step = one draft block for every sequence of the batch: the
block-parallel base logits (domino_base_logits, LM-head GEMM on the MFMA
cores) followed by the 16-step causal-correction chain (domino_draft_chain),
inputs resident in HBM.  Metric: draft blocks per second.

Prints one JSON line.  `roofline` covers the call that takes the most time
per step, with its algorithmic bytes (or flops) per launch divided by its
average duration from HIP events recorded on the launch stream inside the
timed region.  `cpu_baseline` times the oracle on a bounded sample of the same
workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
"""
import argparse
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
    return ap.parse_args()


def algorithmic_traffic(cfg, B, write_logits):
    """Bytes each call must move and flops it must do, from the method's definition."""
    es = 2 if cfg.dtype == "bf16" else 4
    d, V, Hs, r, P = cfg.hidden, cfg.vocab, cfg.gru_hidden, cfg.rank, cfg.block
    M = B * P
    base_bytes = V * d * es + M * d * es + M * V * 4           # W_lm once, H, L^base out
    base_flops = 2.0 * M * V * d
    step = (V * r * es                      # W2
            + 3 * Hs * (d + Hs) * es        # W_ih, W_hh
            + r * Hs * es                   # state half of W1
            + B * V * 4                     # base-logit row of this position
            + B * d * es                    # embedding rows of the fed-back tokens
            + (B * V * 4 if write_logits else 0))
    chain_bytes = P * step + M * d * es + r * d * es + M * 4  # + H half of W1 once, tokens out
    chain_flops = 2.0 * P * B * (3 * Hs * (d + Hs) + r * (d + Hs) + V * r)
    return {"base": (base_bytes, base_flops), "chain": (chain_bytes, chain_flops), "chain_step_bytes": step}


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
        m.chain(H, Lb, inp["t0"][b:b + 1], want_logits=False)
        done += 1
        el = time.perf_counter() - t_start
        if el >= target_s or done >= 64:
            break
    return {"value": done / el, "unit": "draft blocks/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{done} whole blocks (one sequence each: base logits + {cfg.block}-step chain) of "
                      f"{cfg.name}, {el:.1f} s"}


def main():
    args = parse()
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
    ws = head.workspace(B)
    dh.set_chain_mode(args.chain_mode)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dh.domino_base_logits(head.dims, head.weights, H, B, Lb, stream)
        if ev is not None:
            ev[1].record(stream)
        dh.domino_draft_chain(head.dims, head.weights, H, Lb, t0, B, toks, logits, ws, ws.numel(), stream)
        if ev is not None:
            ev[2].record(stream)

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

    # per-call durations, events on the launch stream around each call
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    t_base = np.mean([a.elapsed_time(b) for a, b, _ in evs]) * 1e-3
    t_chain = np.mean([b.elapsed_time(c) for _, b, c in evs]) * 1e-3
    assert dh.DraftHead.device_status(ws) == 0

    tr = algorithmic_traffic(cfg, B, args.logits)
    peak_mfma = MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
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
        k["us"] = t * 1e6
        k["algorithmic_bytes"] = byts
        k["flops"] = flops
    dom = "chain" if t_chain >= t_base else "base"
    roof = {kk: kernels[dom][kk] for kk in ("bound", "achieved", "peak", "unit", "frac")}
    roof["traffic"] = None
    roof["kernel"] = "domino_draft_chain" if dom == "chain" else "domino_base_logits"

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
                   "write_logits": bool(args.logits), "parallelism": "none (one GPU)"},
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
