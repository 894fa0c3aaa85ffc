#!/usr/bin/env python3
"""Throughput of the Domino draft-head hot path on one MI355X.

One step = one draft block for every sequence of the batch: the
block-parallel base logits (domino_base_logits, LM-head GEMM on the MFMA
cores) followed by the 16-step causal-correction chain (domino_draft_chain),
or the best-first tree (domino_tree_draft) for the tree workload, inputs
resident in HBM.  Metric: draft blocks per second.

Prints one JSON line.  The headline (`value`, `roofline`, ...) is the
Qwen3-4B-shaped chain at batch 1; `configs` holds the same record for the
batch-32 and Qwen3-8B chains and the tree.  In every record:
  value        B * K / the wall time of K timed steps (HIP events around them)
  step_ms      median / p10 / p90 of the K per-step times
  roofline     the launch that takes the most time per step, its algorithmic
               bytes (or flops) per launch over its mean duration from HIP
               events the library records on the launch stream right around
               it (domino_bench.h); `traffic` from the committed rocprofv3
               counter summary when it was taken on the current sources;
               `compulsory_frac` counts every weight once instead
  parity       the GPU tokens (or tree) of the timed steps against the oracle
               on sampled sequences, under the margin rule
`cpu_baseline` times the oracle on a bounded sample of the headline workload;
`infinity_cache` times the batch-32 chain cold, warm and in place.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--extra a,b,c | --extra none]
"""
import argparse
import glob
import hashlib
import json
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MFMA_F32_PEAK_TFLOPS = 157.3
METRIC = "draft blocks/sec (16-pos Domino chain, Qwen3-4B shape) + % of HBM/MFMA peak"
MARGIN_FIRM = 1e-2              # tokens must agree where the oracle's top-2 margin exceeds this
EXTRA = ("qwen3_4b_b32", "qwen3_8b_b16", "qwen3_4b_tree", "qwen3_4b_b1_sampled")
PARITY_SAMPLE = {"qwen3_4b_b1": [0], "qwen3_4b_b32": [0, 31], "qwen3_8b_b16": [0, 15], "qwen3_4b_tree": [0, 7],
                 "qwen3_4b_b1_sampled": [0]}
# workloads that are a base config run another way: (base config, temperature, seed)
SAMPLED = {"qwen3_4b_b1_sampled": ("qwen3_4b_b1", 1.0, 20260)}


def log(*a):
    print("bench:", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="qwen3_4b_b1", help="headline workload")
    ap.add_argument("--extra", default=",".join(EXTRA), help="comma-separated extra workloads, or 'none'")
    ap.add_argument("--extra-steps", type=int, default=50)
    ap.add_argument("--chain-mode", type=int, default=0)
    ap.add_argument("--logits", action="store_true", help="also write the final logits")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-cache-probe", action="store_true")
    ap.add_argument("--no-input-table", action="store_true",
                    help="chain calls compute W_ih x from the embedding instead of reading the per-token table")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only copy 256 MiB once on the device (counter calibration under rocprofv3 --pmc)")
    ap.add_argument("--oracle-tiny-1t", action="store_true", help=argparse.SUPPRESS)
    return ap.parse_args()


def copy_probe():
    """One 256 MiB device-to-device copy: a kernel of known traffic for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": src.numel() * 4, "copy_probe_bytes_written": dst.numel() * 4}))


# ---- algorithmic bytes and flops ---------------------------------------------------------
def algorithmic_traffic(cfg, B, write_logits, table=False):
    """Bytes each launch must move and flops it must do, from the method's definition.

    base:  the LM-head GEMM, L^base = H W_lm^T (W_lm once, H, L^base out).
    chain: the P sequential steps; every step reads W2, the GRU weights, the
           state half of W1, one base-logit row and the fed-back embedding
           rows, whatever the kernel keeps on chip between steps.  With the
           per-token input table (table=True) a step reads one table row
           (3 Hs fp32) per sequence instead of W_ih and an embedding row.
    chain_compulsory: the same work with every weight counted once.
    """
    es = 2 if cfg.dtype == "bf16" else 4
    d, V, Hs, r, P = cfg.hidden, cfg.vocab, cfg.gru_hidden, cfg.rank, cfg.block
    M = B * P
    base_bytes = V * d * es + M * d * es + M * V * 4
    base_flops = 2.0 * M * V * d
    logits = V * 4 if write_logits else 0
    if table:
        weights = V * r * es + 3 * Hs * Hs * es + r * Hs * es     # W2, W_hh, W1 state half
        per_seq = V * 4 + 3 * Hs * 4 + logits                     # base row, table row, logits
        gru_flops = 3 * Hs * Hs
    else:
        weights = V * r * es + 3 * Hs * (d + Hs) * es + r * Hs * es   # W2, W_ih + W_hh, W1 state half
        per_seq = V * 4 + d * es + logits                            # base row, embedding row, logits
        gru_flops = 3 * Hs * (d + Hs)
    step = weights + B * per_seq
    tail = M * r * 4 + M * 4                                      # H half of the bottleneck in, tokens out
    chain_bytes = P * step + tail
    chain_flops = 2.0 * P * B * (gru_flops + r * Hs + V * r)
    compulsory = weights + P * B * per_seq + tail
    return {"base": (base_bytes, base_flops), "chain": (chain_bytes, chain_flops), "chain_step_bytes": step,
            "chain_compulsory": compulsory}


def tree_traffic(cfg, B, table=False):
    """Bytes and flops of one tree call: the top-M pass over every base-logit row, then
    N rounds that each read the GRU weights, the state half of W1 and, per sequence,
    M rows of W2, M base-logit entries, one embedding row and two fp64 states.  With the
    fp64 input table a round reads W_hh and one table row (3 Hs fp64) per sequence
    instead of W_ih and an embedding row."""
    es = 2 if cfg.dtype == "bf16" else 4
    d, V, Hs, r, P, N, M = cfg.hidden, cfg.vocab, cfg.gru_hidden, cfg.rank, cfg.block, cfg.nodes, cfg.topm
    topm_bytes = B * P * V * 4
    gru_w = 3 * Hs * (Hs if table else d + Hs) * es
    x_row = 3 * Hs * 8 if table else d * es
    rnd = gru_w + r * Hs * es + B * (M * r * es + M * 4 + x_row + 2 * Hs * 8)
    byts = topm_bytes + B * P * d * es + r * d * es + N * rnd
    flops = 2.0 * B * N * (3 * Hs * (Hs if table else d + Hs) + r * Hs + M * r) + 2.0 * B * P * r * d
    compulsory = topm_bytes + B * P * d * es + r * d * es + gru_w + r * Hs * es + \
        N * B * (M * r * es + M * 4 + x_row + 2 * Hs * 8)
    return byts, flops, compulsory


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


def host_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


# ---- the GPU side ----------------------------------------------------------------------------
class Workload:
    """Device buffers of one workload and its step()."""

    def __init__(self, cfg, weights, inputs, chain_mode, write_logits, temperature=0.0, seed=0, table=True):
        import torch

        import draft_head_amd as dh
        self.dh, self.torch, self.cfg = dh, torch, cfg
        self.head = dh.DraftHead.from_config(cfg, weights, "cuda:0")
        # the per-token GRU input table: built once per set of weights, before any timed step
        self.table = None
        if table:  # fp32 for the chain, fp64 for the tree
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            t = self.head.prepare_input_table_f64() if cfg.tree else self.head.prepare_input_table()
            e1.record()
            torch.cuda.synchronize()
            call = "domino_prepare_input_table_f64" if cfg.tree else "domino_prepare_input_table"
            self.table = {"prepare_ms": e0.elapsed_time(e1), "bytes": t.numel() * t.element_size(),
                          "note": f"{call}, once per set of weights; not part of a step"}
        self.H = self.head.upload(inputs["H"])
        self.t0 = self.head.upload(inputs["t0"])
        dev, B, P, V = self.head.device, cfg.batch, cfg.block, cfg.vocab
        self.B = B
        self.Lb = torch.empty((B, P, V), dtype=torch.float32, device=dev)
        self.toks = torch.empty((B, P), dtype=torch.int32, device=dev)
        self.logits = torch.empty((B, P, V), dtype=torch.float32, device=dev) if write_logits else None
        if cfg.tree:
            N = cfg.nodes
            self.tree = {k: torch.empty((B, N), dtype=torch.int32, device=dev) for k in ("parents", "tokens", "depth")}
            self.scores = torch.empty((B, N), dtype=torch.float64, device=dev)
            self.ws = self.head.workspace(B, dh.OP_TREE, N, cfg.topm)
        else:
            self.ws = self.head.workspace(B)
        self.chain_mode = chain_mode
        self.temperature, self.seed = temperature, seed
        self.stream = torch.cuda.current_stream()

    def base(self):
        self.dh.domino_base_logits(self.head.dims, self.head.weights, self.H, self.B, self.Lb, self.stream)

    def draft(self):
        dh, c = self.dh, self.cfg
        if c.tree:
            dh.domino_tree_draft(self.head.dims, self.head.weights, self.H, self.Lb, self.t0, self.B, c.nodes, c.topm,
                                 self.tree["parents"], self.tree["tokens"], self.tree["depth"], self.scores, self.ws,
                                 self.ws.numel(), self.stream)
        elif self.temperature > 0:
            dh.domino_draft_chain_sampled(self.head.dims, self.head.weights, self.H, self.Lb, self.t0, self.B,
                                          self.temperature, self.seed, self.toks, self.logits, self.ws,
                                          self.ws.numel(), self.stream)
        else:
            dh.domino_draft_chain(self.head.dims, self.head.weights, self.H, self.Lb, self.t0, self.B, self.toks,
                                  self.logits, self.ws, self.ws.numel(), self.stream)

    def step(self):
        self.base()
        self.draft()

    def check(self):
        self.dh.domino_device_status(self.ws, self.stream)  # raises on a flagged device status


def time_steps(wl, K, warmup):
    """Warm up, then K timed steps with an event between consecutive steps."""
    import numpy as np
    torch = wl.torch
    wl.dh.set_chain_mode(wl.chain_mode)
    for _ in range(warmup):
        wl.step()
    torch.cuda.synchronize()
    wl.check()
    # the throughput: K back-to-back steps between two events, nothing in between
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(wl.stream)
    for _ in range(K):
        wl.step()
    e1.record(wl.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    wl.check()
    total_ms = e0.elapsed_time(e1)
    # the distribution: K more steps with an event between consecutive ones
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    ev[0].record(wl.stream)
    for i in range(K):
        wl.step()
        ev[i + 1].record(wl.stream)
    torch.cuda.synchronize()
    wl.check()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(K)])
    return {"ms_per_step": total_ms / K, "wall_s_timed": wall,
            "step_ms": {"median": float(np.median(per)), "p10": float(np.percentile(per, 10)),
                        "p90": float(np.percentile(per, 90)), "min": float(per.min()), "max": float(per.max())}}


def time_launches(wl, K):
    """Mean (and median) duration of the main launch(es) of each call from events the
    library records on the launch stream right around them."""
    import numpy as np
    torch, dh = wl.torch, wl.dh
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for e in evs:  # torch creates the HIP event on its first record
        for x in e:
            x.record(wl.stream)
    torch.cuda.synchronize()
    for i in range(K):
        dh.domino_set_timing_events(*evs[i])
        wl.step()
    torch.cuda.synchronize()
    dh.domino_set_timing_events()
    wl.check()
    tb = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    tc = np.array([e[2].elapsed_time(e[3]) for e in evs]) * 1e-3
    return float(tb.mean()), float(tc.mean()), float(np.median(tb)), float(np.median(tc))


def roofline_record(cfg, B, t_base, t_chain, write_logits, chain_mode, table=False, workload=None):
    tr = algorithmic_traffic(cfg, B, write_logits, table)
    if cfg.tree:
        byts, flops, comp = tree_traffic(cfg, B, table)
        tr["chain"], tr["chain_compulsory"] = (byts, flops), comp
    peak_mfma = MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    kernel_key = {"base": "base_gemm", "chain": "chain_steps"}
    kernels = {}
    for name, t in (("base", t_base), ("chain", t_chain)):
        byts, flops = tr[name]
        ridge = peak_mfma * 1e12 / (HBM_PEAK_GBS * 1e9)
        if flops / byts < ridge:
            k = {"bound": "hbm", "achieved": byts / t / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        else:
            k = {"bound": "mfma", "achieved": flops / t / 1e12, "peak": peak_mfma, "unit": "TFLOP/s"}
        k["frac"] = k["achieved"] / k["peak"]
        k["traffic"] = measured_traffic(workload or cfg.name, kernel_key[name])
        k["us"] = t * 1e6
        k["algorithmic_bytes"] = byts
        k["flops"] = flops
        if k["traffic"] is not None:
            k["traffic_frac"] = k["traffic"] / t / 1e9 / HBM_PEAK_GBS
        kernels[name] = k
    c = kernels["chain"]
    c["compulsory_bytes"] = tr["chain_compulsory"]
    c["compulsory_frac"] = tr["chain_compulsory"] / t_chain / 1e9 / HBM_PEAK_GBS
    c["basis"] = ("streamed bytes: W2 and the GRU weights charged at every step, whatever stays on chip; "
                  "compulsory_frac charges every weight once")
    dom = "chain" if t_chain >= t_base else "base"
    roof = {kk: kernels[dom][kk] for kk in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    if dom == "chain":
        roof["compulsory_frac"] = c["compulsory_frac"]
        roof["kernel"] = "tree launches (domino_tree_draft)" if cfg.tree else "domino_draft_chain steps"
    else:
        roof["kernel"] = "LM-head GEMM (domino_base_logits)"
    return roof, kernels


def chain_schedule(wl):
    """Which schedule the library ran: the persistent one writes its step clocks."""
    import numpy as np
    if wl.cfg.tree:
        if wl.cfg.dtype == "bf16":
            return "tree: one launch per round (bottleneck, score and pop, next GRU step)", None
        return "tree: three launches per round", None
    dh, torch = wl.dh, wl.torch
    off = dh.domino_chain_stamp_offset(wl.head.dims, wl.B)
    n = wl.cfg.block + 1
    wl.ws[off:off + 8 * n].zero_()
    wl.step()
    torch.cuda.synchronize()
    st = wl.ws[off:off + 8 * n].view(torch.int64).cpu().numpy().astype(np.int64)
    if np.all(st > 0):
        return "one persistent launch for all steps", (np.diff(st) * 10e-3).tolist()  # 100 MHz ticks -> us
    if wl.cfg.dtype == "bf16" and min(wl.B, 32) <= 16:
        return "two launches per step (GRU; bottleneck and W2 in one launch)", None
    return "three launches per step (GRU; bottleneck; W2)", None


def cache_probe(wl, reps=10):
    """Infinity Cache evidence for the chain's W2 reuse: the chain timed cold (a 512 MiB
    write before each call evicts the 256 MB cache), warm (back to back, same inputs) and
    in place (right after the LM-head GEMM, as in a step), plus the step clocks of the
    persistent schedule (step 1 streams W2 into the chip, steps 2..P reuse it)."""
    import numpy as np
    torch, dh = wl.torch, wl.dh
    scratch = torch.empty(128 << 20, dtype=torch.float32, device=wl.head.device)
    wl.base()

    def timed(prep):
        out = []
        for _ in range(reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            for x in e:
                x.record(wl.stream)
            prep()
            dh.domino_set_timing_events(None, None, *e)
            wl.draft()
            dh.domino_set_timing_events()
            torch.cuda.synchronize()
            out.append(e[0].elapsed_time(e[1]) * 1e3)
        wl.check()
        return float(np.median(out))

    cold = timed(lambda: scratch.fill_(1.0))
    warm = timed(lambda: None)
    in_place = timed(wl.base)
    sched, steps = chain_schedule(wl)
    rec = {"chain_us_cold": cold, "chain_us_warm": warm, "chain_us_in_place": in_place, "schedule": sched,
           "evict_bytes": scratch.numel() * 4}
    if steps:
        rec["step_us"] = steps
        rec["step1_over_mean_rest"] = steps[0] / float(np.mean(steps[1:-1])) if len(steps) > 2 else None
    del scratch
    return rec


# ---- the oracle (CPU leg: baseline timing and parity of sampled sequences) -----------------------
def oracle_tokens_check(m, H, Lb_ref, t0, g_tokens):
    """Margin rule: the free-running oracle must produce the GPU's tokens up to its first
    near tie (top-2 margin <= MARGIN_FIRM); past a tolerated divergence the oracle is re-run
    with the GPU's tokens fed back and must agree wherever its margin is firm."""
    import numpy as np
    r_t, _, r_m = m.chain(H, Lb_ref, t0, want_logits=False)
    firm_checked, mism, near = 0, 0, int((r_m <= MARGIN_FIRM).sum())
    forced_needed = False
    for b in range(g_tokens.shape[0]):
        for p in range(g_tokens.shape[1]):
            if r_m[b, p] <= MARGIN_FIRM:
                if g_tokens[b, p] != r_t[b, p]:
                    forced_needed = True
                break
            firm_checked += 1
            mism += int(g_tokens[b, p] != r_t[b, p])
    if forced_needed:
        f_t, _, f_m = m.chain(H, Lb_ref, t0, forced=g_tokens, want_logits=False)
        firm = f_m > MARGIN_FIRM
        mism += int((firm & (f_t != g_tokens)).sum())
    return firm_checked, mism, near


def parity_chain(cfg, w, inp, g_tokens, sample, oracle_runs=None):
    import numpy as np

    import oracle
    m = oracle.Model.from_config(cfg, w)
    tot_firm, tot_mis, tot_near = 0, 0, 0
    for b in sample:
        H = np.ascontiguousarray(inp["H"][b:b + 1])
        Lb = oracle_runs.get(b) if oracle_runs else None
        if Lb is None:
            Lb = m.base_logits(H)
        f, mi, ne = oracle_tokens_check(m, H, Lb, inp["t0"][b:b + 1], g_tokens[b:b + 1])
        tot_firm, tot_mis, tot_near = tot_firm + f, tot_mis + mi, tot_near + ne
    return {"sequences": list(sample), "positions_checked": tot_firm, "mismatches": tot_mis, "near_ties": tot_near,
            "ok": tot_mis == 0,
            "rule": "timed tokens vs the oracle (its own base logits): equal at every position up to the first "
                    "oracle top-2 margin <= 1e-2, then equal wherever the forced-prefix oracle's margin > 1e-2"}


def parity_sampled(cfg, w, inp, Lb_gpu, g_tokens, sample, T, seed):
    """The sampled chain: tokens against the oracle's draws on the same fp32 base logits, under
    the margin rule on the perturbed logits L + T g (forced-prefix past a tolerated divergence)."""
    import numpy as np

    import oracle
    m = oracle.Model.from_config(cfg, w)
    checked, mism, near = 0, 0, 0
    for b in sample:
        H = np.ascontiguousarray(inp["H"][b:b + 1])
        f_t, _, f_m = m.chain_sampled(H, np.ascontiguousarray(Lb_gpu[b:b + 1]), inp["t0"][b:b + 1], T, seed, seq0=b,
                                      forced=g_tokens[b:b + 1], want_logits=False)
        firm = f_m > MARGIN_FIRM
        checked += int(firm.sum())
        near += int((~firm).sum())
        mism += int((firm & (f_t != g_tokens[b:b + 1])).sum())
    return {"sequences": list(sample), "positions_checked": checked, "mismatches": mism, "near_ties": near,
            "ok": mism == 0, "temperature": T, "seed": seed,
            "rule": "timed draws vs the oracle's Gumbel-max draws on the same base logits and noise: equal wherever "
                    "the oracle's top-2 margin of L + T g exceeds 1e-2 (forced prefix)"}


def parity_tree(cfg, w, inp, Lb_gpu, g_tree, g_scores, sample):
    import numpy as np

    import oracle
    m = oracle.Model.from_config(cfg, w)
    bad, max_err = 0, 0.0
    for b in sample:
        o = m.tree(np.ascontiguousarray(inp["H"][b:b + 1]), np.ascontiguousarray(Lb_gpu[b:b + 1]),
                   inp["t0"][b:b + 1], cfg.nodes, cfg.topm)
        for k in ("parents", "tokens", "depth"):
            bad += int(not np.array_equal(o[k][0], g_tree[k][b]))
        fin = np.isfinite(o["scores"][0])
        max_err = max(max_err, float(np.max(np.abs(o["scores"][0][fin] - g_scores[b][fin]), initial=0.0)))
    return {"sequences": list(sample), "structure_mismatches": bad, "max_score_err": max_err,
            "ok": bad == 0 and max_err <= 1e-9,
            "rule": "the timed trees vs the oracle tree on the same fp32 base logits: parents, tokens and depth "
                    "equal, scores within 1e-9"}


def cpu_baseline(cfg, w, inp, target_s):
    """The oracle (plain C, OpenMP) on whole blocks of the headline workload; the same oracle
    runs then check the GPU's timed tokens of those sequences."""
    import numpy as np

    import oracle
    m = oracle.Model.from_config(cfg, w)
    done, t_start = 0, time.perf_counter()
    B = inp["t0"].size
    lbs = {}
    while True:
        b = done % B
        H = np.ascontiguousarray(inp["H"][b:b + 1])
        Lb = m.base_logits(H)
        if cfg.tree:
            m.tree(H, Lb, inp["t0"][b:b + 1], cfg.nodes, cfg.topm)
        else:
            m.chain(H, Lb, inp["t0"][b:b + 1], want_logits=False)
        lbs.setdefault(b, Lb)
        done += 1
        el = time.perf_counter() - t_start
        if el >= target_s or done >= 64:
            break
    rec = {"value": done / el, "unit": "draft blocks/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"{done} whole blocks (one sequence each: base logits + "
                     f"{f'{cfg.nodes}-node tree' if cfg.tree else f'{cfg.block}-step chain'}) of {cfg.name}, "
                     f"{el:.1f} s"}
    return rec, lbs


def oracle_tiny_single_thread():
    """Runs in a child process with OMP_NUM_THREADS=1: the tiny fp32 block on one core."""
    import oracle
    import synth
    cfg = synth.CONFIGS["tiny_f32"]
    m = oracle.Model.from_config(cfg, synth.make_weights(cfg))
    inp = synth.make_inputs(cfg)
    n, t = 0, time.perf_counter()
    while time.perf_counter() - t < 2.0 or n < 3:
        m.chain(inp["H"], m.base_logits(inp["H"]), inp["t0"], want_logits=False)
        n += 1
    el = time.perf_counter() - t
    print(json.dumps({"blocks_per_s": n / el, "ms_per_block": el / n * 1e3, "threads": oracle.num_threads(),
                      "blocks": n}))


def tiny_1t():
    env = dict(os.environ, OMP_NUM_THREADS="1")
    res = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-tiny-1t"], env=env,
                         capture_output=True, text=True, timeout=120)
    if res.returncode != 0:
        return {"error": res.stderr[-300:]}
    rec = json.loads(res.stdout.strip().splitlines()[-1])
    rec["workload"] = "tiny_f32 (batch 1, block 16, d 256, V 4096, Hs 128, r 32, fp32)"
    return rec


# ---- one workload end to end ---------------------------------------------------------------------
def verify_inputs_record(wl, reps=50):
    """The tree's verification inputs (ancestor-only mask, positions, tokens) from the timed
    trees: launch time by events around the call, bytes = what it reads and writes."""
    import numpy as np
    torch, dh = wl.torch, wl.dh
    B, N = wl.B, wl.cfg.nodes
    E = N + 1
    mask = torch.empty((B, E, E), dtype=torch.uint8, device=wl.head.device)
    pos = torch.empty((B, E), dtype=torch.int32, device=wl.head.device)
    tok = torch.empty((B, E), dtype=torch.int32, device=wl.head.device)
    run = lambda: dh.domino_tree_verify_inputs(wl.tree["parents"], wl.tree["tokens"], wl.t0, None, B, N, mask, pos,
                                               tok, wl.stream)
    run()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(wl.stream)
    for _ in range(reps):
        run()
    ev[1].record(wl.stream)
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / reps
    byts = B * (2 * N * 4 + 4) + B * (E * E + 2 * E * 4)
    return {"us": us, "bytes": byts, "bound": "latency (one 64-lane workgroup per tree)",
            "achieved_gbs": byts / us * 1e-3}, (mask.cpu().numpy(), pos.cpu().numpy(), tok.cpu().numpy())


def run_workload(cfg, args, steps, warmup, weights, parity_lbs=None, label=None, temperature=0.0, seed=0):
    import numpy as np
    import synth
    inp = synth.make_inputs(cfg)
    wl = Workload(cfg, weights, inp, args.chain_mode, args.logits, temperature, seed, table=not args.no_input_table)
    name = label or cfg.name
    log(f"{name}: timing {steps} steps")
    t = time_steps(wl, steps, warmup)
    g_tokens = wl.toks.cpu().numpy()
    g_tree = {k: v.cpu().numpy() for k, v in wl.tree.items()} if cfg.tree else None
    g_scores = wl.scores.cpu().numpy() if cfg.tree else None
    Lb_gpu = wl.Lb.cpu().numpy() if (cfg.tree or temperature > 0) else None
    t_base, t_chain, tb_med, tc_med = time_launches(wl, steps)
    roof, kernels = roofline_record(cfg, cfg.batch, t_base, t_chain, args.logits, args.chain_mode, wl.table is not None,
                                    workload=name)
    kernels["base"]["us_median"], kernels["chain"]["us_median"] = tb_med * 1e6, tc_med * 1e6
    sched, step_us = chain_schedule(wl)
    rec = {"value": cfg.batch / (t["ms_per_step"] * 1e-3), "unit": "draft blocks/s",
           "ms_per_step": t["ms_per_step"], "step_ms": t["step_ms"], "steps": steps, "warmup": warmup,
           "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
           "config": {"workload": name, "batch": cfg.batch, "block": cfg.block, "hidden": cfg.hidden,
                      "vocab": cfg.vocab, "gru_hidden": cfg.gru_hidden, "rank": cfg.rank,
                      "chain_mode": args.chain_mode, "write_logits": bool(args.logits), "schedule": sched,
                      "input_table": wl.table is not None,
                      **({"temperature": temperature, "seed": seed} if temperature > 0 else {}),
                      **({"tree_nodes": cfg.nodes, "tree_topm": cfg.topm} if cfg.tree else {})},
           "roofline": roof, "kernels": kernels, "wall_s_timed": t["wall_s_timed"]}
    if step_us:
        rec["chain_step_us"] = [round(x, 2) for x in step_us]
    if wl.table is not None:
        rec["input_table"] = wl.table
    if cfg.name == "qwen3_4b_b32" and not args.no_cache_probe and temperature == 0:
        log(f"{cfg.name}: cache probe")
        rec["infinity_cache"] = cache_probe(wl)
    verify = None
    if cfg.tree:
        rec["verify_inputs"], verify = verify_inputs_record(wl)
    del wl
    import torch
    torch.cuda.empty_cache()
    if not args.no_parity:
        log(f"{cfg.name}: oracle parity")
        sample = [b for b in PARITY_SAMPLE.get(name, [0]) if b < cfg.batch]
        if cfg.tree:
            rec["parity"] = parity_tree(cfg, weights, inp, Lb_gpu, g_tree, g_scores, sample)
            import oracle
            o = oracle.tree_verify_inputs(g_tree["parents"], g_tree["tokens"], inp["t0"])
            rec["verify_inputs"]["parity"] = {"ok": all(np.array_equal(x, y) for x, y in zip(verify, o)),
                                              "rule": "mask, positions and tokens bit-exact against the oracle"}
        elif temperature > 0:
            rec["parity"] = parity_sampled(cfg, weights, inp, Lb_gpu, g_tokens, sample, temperature, seed)
        else:
            rec["parity"] = parity_chain(cfg, weights, inp, g_tokens, sample, parity_lbs)
    return rec, inp, g_tokens


def main():
    args = parse()
    if args.copy_probe:
        return copy_probe()
    if args.oracle_tiny_1t:
        return oracle_tiny_single_thread()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (see the sharding notes); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import draft_head_amd as dh  # noqa: F401  (fails loudly when the HIP library is missing)
    import synth

    for so in ("synth/libsynth.so", "draft_head_amd/libdomino.so"):
        if not os.path.exists(os.path.join(ROOT, so)):
            import __graft_entry__
            __graft_entry__.build()
            break

    base, T, seed = SAMPLED.get(args.config, (args.config, 0.0, 0))
    cfg = synth.CONFIGS[base]
    cache = {}

    def weights_of(c):
        key = (c.weight_seed, c.hidden, c.vocab, c.gru_hidden, c.rank, c.dtype)
        if key not in cache:
            cache.clear()
            log(f"generating weights for {c.name}")
            cache[key] = synth.make_weights(c)
        return cache[key]

    w = weights_of(cfg)
    head, inp, g_tokens = run_workload(cfg, dataclass_args(args, parity=(T > 0 or cfg.tree) and not args.no_parity), args.steps,
                                       args.warmup, w, label=args.config, temperature=T, seed=seed)
    out = {"metric": METRIC, "value": head["value"], "unit": "draft blocks/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": head["dtype"], "data": "synthetic",
           "config": {**head["config"], "parallelism": "none (one GPU)"},
           "step_ms": head["step_ms"], "roofline": head["roofline"], "kernels": head["kernels"],
           "wall_s_timed": head["wall_s_timed"]}
    for k in ("chain_step_us", "parity", "verify_inputs", "input_table"):
        if k in head:
            out[k] = head[k]
    if not args.no_cpu_baseline:
        log("oracle baseline")
        out["cpu_baseline"], lbs = cpu_baseline(cfg, w, inp, args.cpu_seconds)
        out["cpu_baseline"]["host"] = host_info()
        out["cpu_baseline"]["tiny_f32_single_thread"] = tiny_1t()
        if not args.no_parity and not cfg.tree and T == 0:
            out["parity"] = parity_chain(cfg, w, inp, g_tokens, sorted(lbs)[:4], lbs)
    elif not args.no_parity and not cfg.tree and T == 0:
        out["parity"] = parity_chain(cfg, w, inp, g_tokens, PARITY_SAMPLE.get(cfg.name, [0]))
    extra = [] if args.extra in ("", "none") else [e for e in args.extra.split(",") if e != cfg.name]
    if extra:
        out["configs"] = {}
    for name in extra:
        base, T, seed = SAMPLED.get(name, (name, 0.0, 0))
        c = synth.CONFIGS[base]
        try:
            rec, _, _ = run_workload(c, args, args.extra_steps, min(args.warmup, 10), weights_of(c), label=name,
                                     temperature=T, seed=seed)
        except Exception as e:  # a failing extra workload is reported, never hides the headline
            rec = {"error": f"{type(e).__name__}: {e}"}
        out["configs"][name] = rec
    print(json.dumps(out), flush=True)


def dataclass_args(args, parity):
    """The headline's parity comes from the CPU-baseline leg's own oracle runs."""
    a = argparse.Namespace(**vars(args))
    a.no_parity = not parity
    return a


if __name__ == "__main__":
    main()
