"""GPU parity of the best-first tree and its top-M candidate lists against the oracle.

Both sides receive the same fp32 base logits (the oracle's own, or a seeded
draw at the full shape), so every decision is taken on identical inputs; the
tree is scored in fp64 on both sides.  Parents, tokens and depths must be
identical, scores equal within 1e-9.
"""
import numpy as np
import pytest
import torch

import draft_head_amd as dh
import oracle
import synth
from gpu_common import say, weights_for
from helpers import small_config

pytestmark = pytest.mark.gpu

SCORE_TOL = 1e-9


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    dh.lib()
    yield
    torch.cuda.synchronize()


def _gpu_tree(cfg, w, H, Lb, t0, N, M):
    head = dh.DraftHead.from_config(cfg, w)
    out, ws = head.tree_draft(head.upload(H), head.upload(Lb), head.upload(t0), N, M, check=False)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}, dh.DraftHead.device_status(ws)


def _compare(g, o, label):
    for k in ("parents", "tokens", "depth"):
        assert np.array_equal(g[k], o[k]), f"{label}: {k} differ\n{g[k]}\n{o[k]}"
    fin = np.isfinite(o["scores"])
    assert np.array_equal(fin, np.isfinite(g["scores"]))
    assert np.all(np.abs(g["scores"][fin] - o["scores"][fin]) <= SCORE_TOL), label


@pytest.mark.parametrize("d,V,Hs,r,P,B,N,M,dtype", [
    (16, 37, 8, 8, 4, 2, 16, 3, "f32"),
    (64, 1003, 40, 24, 6, 3, 16, 8, "bf16"),
    (96, 2051, 64, 64, 16, 5, 16, 64, "bf16"),
    (48, 515, 16, 16, 5, 9, 40, 5, "bf16"),      # more sequences than one GRU pass
    (32, 300, 8, 32, 3, 2, 64, 256, "f32"),      # largest budget and candidate count
    (32, 64, 8, 8, 1, 2, 10, 4, "bf16"),         # one position: the tree runs out of nodes
    (3080, 1000, 1288, 64, 2, 3, 8, 16, "bf16"),  # GRU k blocks past the preloaded ones, ragged last block
    (64, 777, 24, 16, 3, 17, 12, 6, "bf16"),      # three GRU passes (sequences 16..)
    (128, 1500, 32, 256, 4, 3, 12, 16, "bf16"),   # the largest rank: full bottleneck vector in the pop
    (32, 300, 8, 32, 3, 2, 64, 256, "bf16"),     # bf16 (one launch per round): four groups of 64 candidates
    (64, 700, 16, 48, 4, 3, 20, 65, "bf16"),     # one candidate past a group of 64
    (64, 500, 16, 16, 4, 2, 1, 8, "bf16"),       # a single round: no GRU step in the round's launch
])
def test_tree_matches_oracle(d, V, Hs, r, P, B, N, M, dtype):
    cfg = small_config(d=d, V=V, Hs=Hs, r=r, P=P, B=B, dtype=dtype, biases=True)
    say(f"case tree d={d} V={V} Hs={Hs} r={r} P={P} B={B} N={N} M={M} {dtype}")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    m = oracle.Model.from_config(cfg, w)
    Lb = m.base_logits(inp["H"])
    g, st = _gpu_tree(cfg, w, inp["H"], Lb, inp["t0"], N, M)
    assert st == 0
    o = m.tree(inp["H"], Lb, inp["t0"], N, M)
    _compare(g, o, "small")


def test_tree_workspace_reuse_and_layout_change():
    """Calls on one workspace: the hand-off words of an earlier call (same
    rounds, an older epoch) must never pass, and a call with another layout of
    the same workspace clears them first."""
    cfg = small_config(d=96, V=1201, Hs=32, r=64, P=6, B=5, dtype="bf16", biases=True)
    say("case tree workspace reuse")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    m = oracle.Model.from_config(cfg, w)
    Lb = m.base_logits(inp["H"])
    head = dh.DraftHead.from_config(cfg, w)
    H, L, t0 = head.upload(inp["H"]), head.upload(Lb), head.upload(inp["t0"])
    ws = head.workspace(cfg.batch, dh.OP_TREE, 16, 12)
    outs = []
    for N, M, B in ((16, 12, 5), (16, 12, 5), (9, 12, 3), (16, 12, 5)):
        out, _ = head.tree_draft(H[:B], L[:B], t0[:B], N, M, workspace=ws, check=False)
        torch.cuda.synchronize()
        assert dh.DraftHead.device_status(ws) == 0
        g = {k: v.cpu().numpy() for k, v in out.items()}
        o = m.tree(np.ascontiguousarray(inp["H"][:B]), np.ascontiguousarray(Lb[:B]), inp["t0"][:B], N, M)
        _compare(g, o, f"reuse N={N} B={B}")
        outs.append(g)
    for k in ("parents", "tokens", "depth", "scores"):
        assert np.array_equal(outs[0][k], outs[1][k]) and np.array_equal(outs[0][k], outs[3][k])


def test_tree_single_candidate_and_zero_correction():
    cfg = small_config(d=32, V=211, Hs=16, r=16, P=6, B=3, dtype="bf16", biases=False)
    say("case tree M=1 / W2=0")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    m = oracle.Model.from_config(cfg, w)
    Lb = m.base_logits(inp["H"])
    g, _ = _gpu_tree(cfg, w, inp["H"], Lb, inp["t0"], 9, 1)
    assert g["tokens"][:, :6].tolist() == np.argmax(Lb, axis=-1).tolist()
    assert np.all(g["parents"][:, 6:] == -1) and np.all(g["tokens"][:, 6:] == -1)
    w0 = dict(w)
    w0["w2"] = np.zeros_like(w["w2"])
    m0 = oracle.Model.from_config(cfg, w0)
    g0, _ = _gpu_tree(cfg, w0, inp["H"], Lb, inp["t0"], 16, 4)
    _compare(g0, m0.tree(inp["H"], Lb, inp["t0"], 16, 4), "zero correction")


def test_tree_bad_first_token_flagged():
    cfg = small_config(d=32, V=101, Hs=16, r=16, P=3, B=2, dtype="bf16")
    say("case tree bad first token")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    m = oracle.Model.from_config(cfg, w)
    Lb = m.base_logits(inp["H"])
    g, st = _gpu_tree(cfg, w, inp["H"], Lb, np.array([cfg.vocab, 3], np.int32), 8, 4)
    assert st == dh.STATUS_BAD_FIRST_TOKEN
    o = m.tree(inp["H"], Lb, np.array([0, 3], np.int32), 8, 4)  # drafted from token 0 instead
    _compare(g, o, "bad first token")
    head = dh.DraftHead.from_config(cfg, w)
    with pytest.raises(dh.DominoError) as ei:
        head.tree_draft(head.upload(inp["H"]), head.upload(Lb), head.upload(np.array([-1, 3], np.int32)), 8, 4)
    assert ei.value.status == dh.ERR_FIRST_TOKEN


def test_tree_full_size():
    key = "qwen3_4b_tree"
    cfg = synth.CONFIGS[key]
    say(f"case tree full {key}")
    w = weights_for("qwen3_4b_b1")  # same weights (seed 4)
    inp = synth.make_inputs(cfg)
    # base logits with the distribution of H W_lm^T at these shapes (std ~ 1.01), drawn directly
    Lb = synth.normal((cfg.batch, cfg.block, cfg.vocab), 1.0, cfg.input_seed, 20, "f32")
    head = dh.DraftHead.from_config(cfg, w)
    out, ws = head.tree_draft(head.upload(inp["H"]), head.upload(Lb), head.upload(inp["t0"]), cfg.nodes, cfg.topm)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    o = oracle.Model.from_config(cfg, w).tree(inp["H"], Lb, inp["t0"], cfg.nodes, cfg.topm)
    _compare(g, o, key)


def test_tree_full_size_after_gpu_base_logits():
    """The whole tree path at full size: the GPU's LM-head GEMM gives L^base, and both the
    GPU tree and the oracle tree take exactly those fp32 values (the tree is a function of
    its L^base input), at the bench's batch, budget and candidate count."""
    key = "qwen3_4b_tree"
    cfg = synth.CONFIGS[key]
    say(f"case tree full {key} with the GPU's own base logits")
    w = weights_for("qwen3_4b_b1")
    inp = synth.make_inputs(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    H = head.upload(inp["H"])
    Lb = head.base_logits(H)
    out, _ = head.tree_draft(H, Lb, head.upload(inp["t0"]), cfg.nodes, cfg.topm)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    o = oracle.Model.from_config(cfg, w).tree(inp["H"], Lb.cpu().numpy(), inp["t0"], cfg.nodes, cfg.topm)
    _compare(g, o, key + " (GPU base logits)")


@pytest.mark.parametrize("kind", ["random", "ties", "constant", "ascending", "small_v", "wide", "wide_m256",
                                  "wide_m1", "one_wave_heavy", "signed_zero_max"])
def test_candidates_match_oracle_topm(kind):
    say(f"case top-M {kind}")
    B, P, V, M = 2, 3, 5003, 64
    rng = np.random.default_rng(5)
    if kind.startswith("wide") or kind == "one_wave_heavy":
        B, P, V = 1, 2, 151936
        M = {"wide_m256": 256, "wide_m1": 1}.get(kind, 64)
        Lb = rng.standard_normal((B, P, V)).astype(np.float32)
        if kind == "one_wave_heavy":
            # every segment's large values sit on the elements its first wave
            # scans, so the other waves' thresholds admit too many candidates
            # and the kernel takes its iterative path
            per = (V + 7) // 8
            v = np.arange(V)
            Lb[:, :, (v - (v // per) * per) % 256 < 64] += 10.0
    elif kind == "random":
        Lb = rng.standard_normal((B, P, V)).astype(np.float32)
    elif kind == "ties":
        Lb = (np.round(rng.standard_normal((B, P, V)) * 2) / 2).astype(np.float32)
        Lb[0, 0, :10] = -0.0
        Lb[0, 0, 10:20] = 0.0
    elif kind == "signed_zero_max":
        # the largest value is zero, stored as -0.0 and +0.0 in turn, so the
        # threshold sits exactly at zero and -0.0 must count as +0.0
        Lb = -np.abs(rng.standard_normal((B, P, V))).astype(np.float32) - np.float32(1e-3)
        v = np.arange(V)
        Lb[:, :, v % 7 == 0] = -0.0
        Lb[:, :, v % 7 == 3] = 0.0
    elif kind == "constant":
        Lb = np.full((B, P, V), 0.25, np.float32)
    elif kind == "ascending":
        Lb = np.tile(np.linspace(-3, 3, V, dtype=np.float32), (B, P, 1))
    else:
        V, M = 70, 70
        Lb = rng.standard_normal((B, P, V)).astype(np.float32)
    dims = dh.make_dims(16, V, 8, 8, P, "bf16")
    x = torch.from_numpy(np.ascontiguousarray(Lb)).cuda()
    idx = torch.empty((B, P, M), dtype=torch.int32, device="cuda")
    val = torch.empty((B, P, M), dtype=torch.float32, device="cuda")
    ws = torch.zeros(dh.domino_workspace_size(dims, B, dh.OP_CANDIDATES, 0, M), dtype=torch.uint8, device="cuda")
    dh.domino_tree_candidates(dims, x, B, M, idx, val, ws, ws.numel())
    torch.cuda.synchronize()
    gi, gv = idx.cpu().numpy(), val.cpu().numpy()
    for b in range(B):
        for p in range(P):
            row = Lb[b, p] + np.float32(0.0)  # -0 counts as +0 on both sides
            oi, ov = oracle.topm(row, M)
            assert np.array_equal(gi[b, p], oi), (kind, b, p)
            assert np.array_equal(gv[b, p], ov)


# ---- the tree with the per-token fp64 input table ------------------------------------
@pytest.mark.parametrize("d,V,Hs,dtype", [(64, 1003, 40, "bf16"), (96, 2051, 64, "bf16"), (16, 37, 8, "f32"),
                                          (3080, 1000, 1288, "bf16"), (32, 300, 8, "f32")])
def test_input_table_f64_exact(d, V, Hs, dtype):
    """E W_ih^T in fp64: the products are exact, so the table equals the exact sum up
    to fp64 rounding (a K-term bound), and the oracle's own fp64 product within it."""
    cfg = small_config(d=d, V=V, Hs=Hs, r=16, P=3, B=2, dtype=dtype)
    say(f"case input table fp64 d={d} V={V} Hs={Hs} {dtype}")
    w = synth.make_weights(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    T = head.prepare_input_table_f64().cpu().numpy()
    from helpers import widen
    E, Wd = widen(w["embed"], dtype), widen(w["w_ih"], dtype)
    exact = E @ Wd.T
    bound = 4.0 * d * 2.0 ** -53 * (np.abs(E) @ np.abs(Wd).T) + 1e-300  # both sides round
    assert np.all(np.abs(T - exact) <= bound)


@pytest.mark.parametrize("d,V,Hs,r,P,B,N,M,dtype", [
    (16, 37, 8, 8, 4, 2, 16, 3, "f32"),
    (96, 2051, 64, 64, 16, 5, 16, 64, "bf16"),
    (48, 515, 16, 16, 5, 9, 40, 5, "bf16"),
    (3080, 1000, 1288, 64, 2, 3, 8, 16, "bf16"),
    (64, 777, 24, 16, 3, 17, 12, 6, "bf16"),
])
def test_tree_with_table_matches_oracle(d, V, Hs, r, P, B, N, M, dtype):
    cfg = small_config(d=d, V=V, Hs=Hs, r=r, P=P, B=B, dtype=dtype, biases=True)
    say(f"case tree with table d={d} V={V} Hs={Hs} r={r} P={P} B={B} N={N} M={M} {dtype}")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    m = oracle.Model.from_config(cfg, w)
    Lb = m.base_logits(inp["H"])
    head = dh.DraftHead.from_config(cfg, w)
    head.prepare_input_table_f64()
    out, ws = head.tree_draft(head.upload(inp["H"]), head.upload(Lb), head.upload(inp["t0"]), N, M, check=False)
    torch.cuda.synchronize()
    assert dh.DraftHead.device_status(ws) == 0
    g = {k: v.cpu().numpy() for k, v in out.items()}
    _compare(g, m.tree(inp["H"], Lb, inp["t0"], N, M), "tree with table")


def test_tree_with_table_full_size_after_gpu_base_logits():
    key = "qwen3_4b_tree"
    cfg = synth.CONFIGS[key]
    say(f"case tree with table full {key}")
    w = weights_for("qwen3_4b_b1")
    inp = synth.make_inputs(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    head.prepare_input_table_f64()
    H = head.upload(inp["H"])
    Lb = head.base_logits(H)
    out, _ = head.tree_draft(H, Lb, head.upload(inp["t0"]), cfg.nodes, cfg.topm)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    o = oracle.Model.from_config(cfg, w).tree(inp["H"], Lb.cpu().numpy(), inp["t0"], cfg.nodes, cfg.topm)
    _compare(g, o, key + " (table)")
    del head
    torch.cuda.empty_cache()
