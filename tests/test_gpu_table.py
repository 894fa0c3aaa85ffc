"""GPU parity of the per-token GRU input table (domino_prepare_input_table) and
of the chain calls that read it instead of multiplying W_ih by an embedding
row at every step.

The table is E W_ih^T with fp32 accumulation: every entry is checked against
the exact product within the a-priori fp32 bound of a K-term dot product, and
against the oracle's fp64 product of the same operands (its base-logit
routine with E as the rows and W_ih as the head).  The chain with the table
is compared with the oracle's chain (which computes W_ih x itself) under the
same rules as the chain without it; its schedules agree to the bit.
"""
import functools

import numpy as np
import pytest
import torch

import draft_head_amd as dh
import oracle
import synth
from gpu_common import compare_chain, gemm_bound, say, weights_for
from helpers import row_rel_err, small_config, widen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    dh.lib()
    yield
    torch.cuda.synchronize()


@pytest.fixture(params=[0, 1, 2], ids=["persistent", "stepwise", "persistent-streamed"])
def chain_mode(request):
    prev = dh.set_chain_mode(request.param)
    yield request.param
    dh.set_chain_mode(prev)


def _oracle_table(cfg, w, rows=None):
    """The oracle's fp64 E W_ih^T (rounded once to fp32) for the given token rows."""
    mt = oracle.Model(cfg.hidden, 3 * cfg.gru_hidden, cfg.gru_hidden, cfg.rank, cfg.block, cfg.dtype,
                      {**w, "lm_head": w["w_ih"]})
    E = w["embed"] if rows is None else np.ascontiguousarray(w["embed"][rows])
    return mt.base_logits(E)


def _check_table(T, E, Wih, dtype, label):
    Ed, Wd = widen(E, dtype), widen(Wih, dtype)
    exact = Ed @ Wd.T
    bound = gemm_bound(Ed, Wd) + np.abs(exact) * 2.0 ** -24
    err = np.abs(T.astype(np.float64) - exact)
    assert np.all(err <= bound), f"{label}: worst excess {(err - bound).max():.3e}"


# d, V, Hs, dtype: few rows (split-k tiles), many rows with k a multiple of 64
# (the LDS-ring kernel, ragged rows and columns), many rows otherwise (128 x
# 128 tiles), fp32
TABLE_SHAPES = [(64, 1003, 40, "bf16"), (256, 5003, 48, "bf16"), (96, 4099, 128, "bf16"), (200, 6007, 64, "bf16"),
                (16, 37, 8, "f32"), (64, 999, 32, "f32")]


@pytest.mark.parametrize("d,V,Hs,dtype", TABLE_SHAPES)
def test_input_table_small(d, V, Hs, dtype):
    cfg = small_config(d=d, V=V, Hs=Hs, r=16, P=3, B=2, dtype=dtype)
    say(f"case input table d={d} V={V} Hs={Hs} {dtype}")
    w = synth.make_weights(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    T = head.prepare_input_table().cpu().numpy()
    assert T.shape == (V, 3 * Hs)
    _check_table(T, w["embed"], w["w_ih"], dtype, "table")
    ref = _oracle_table(cfg, w)
    assert row_rel_err(T, ref).max() <= 1e-5
    T2 = head.prepare_input_table().cpu().numpy()
    assert np.array_equal(T, T2)  # fixed summation order


def test_input_table_full_size_rows():
    key = "qwen3_4b_b1"
    cfg = synth.CONFIGS[key]
    say("case input table full size")
    w = weights_for(key)
    head = dh.DraftHead.from_config(cfg, w)
    T = head.prepare_input_table()
    rows = [0, 1, 4097, 77777, cfg.vocab - 2, cfg.vocab - 1]
    g = T[rows].cpu().numpy()
    _check_table(g, w["embed"][rows], w["w_ih"], "bf16", "full-size table")
    assert row_rel_err(g, _oracle_table(cfg, w, rows)).max() <= 1e-5
    del T, head
    torch.cuda.empty_cache()


def _run(head, inp, want_logits=True):
    H, t0 = head.upload(inp["H"]), head.upload(inp["t0"])
    Lb = head.base_logits(H)
    toks, L, ws = head.draft_chain(H, Lb, t0, want_logits=want_logits, check=False)
    torch.cuda.synchronize()
    status = dh.DraftHead.device_status(ws)
    return Lb.cpu().numpy(), toks.cpu().numpy(), None if L is None else L.cpu().numpy(), status


CHAIN_SHAPES = [
    # d, V, Hs, r, P, B, dtype
    (16, 37, 8, 8, 5, 2, "f32"),
    (64, 1003, 40, 24, 7, 5, "bf16"),
    (200, 2051, 64, 64, 16, 17, "bf16"),
    (96, 4099, 128, 256, 16, 32, "bf16"),
    (48, 515, 16, 16, 3, 40, "bf16"),   # two launches of <= 32 sequences
    (32, 64, 8, 8, 1, 1, "bf16"),
    (64, 2053, 32, 256, 5, 24, "bf16"),
]


@pytest.mark.parametrize("d,V,Hs,r,P,B,dtype", CHAIN_SHAPES)
def test_chain_with_table_small(chain_mode, d, V, Hs, r, P, B, dtype):
    cfg = small_config(d=d, V=V, Hs=Hs, r=r, P=P, B=B, dtype=dtype, biases=True)
    say(f"case chain with table mode={chain_mode} d={d} V={V} Hs={Hs} r={r} P={P} B={B} {dtype}")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    head.prepare_input_table()
    _, toks, L, status = _run(head, inp)
    assert status == 0
    m = oracle.Model.from_config(cfg, w)
    info = compare_chain(m, inp["H"], m.base_logits(inp["H"]), inp["t0"], toks, L, "table small")
    say("  ", info)


@pytest.mark.parametrize("B,r", [(20, 32), (9, 32), (1, 256), (8, 256), (32, 64)])
def test_chain_with_table_modes_agree_bitwise(B, r):
    cfg = small_config(d=96, V=1501, Hs=48, r=r, P=12, B=B, dtype="bf16", biases=True)
    say(f"case chain with table modes agree B={B} r={r}")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    head.prepare_input_table()
    out = []
    prev = dh.set_chain_mode(0)
    try:
        for mode in (0, 1, 2, 3):
            dh.set_chain_mode(mode)
            out.append(_run(head, inp))
    finally:
        dh.set_chain_mode(prev)
    for _, t, L, s in out:
        assert s == 0
        assert np.array_equal(t, out[0][1]) and np.array_equal(L, out[0][2])


def test_sampled_chain_with_table_zero_temperature_is_greedy():
    cfg = small_config(d=64, V=2003, Hs=32, r=32, P=8, B=6, dtype="bf16", biases=True)
    say("case sampled chain with table T=0")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    head.prepare_input_table()
    H, t0 = head.upload(inp["H"]), head.upload(inp["t0"])
    Lb = head.base_logits(H)
    prev = dh.set_chain_mode(1)
    try:
        g_t, g_L, _ = head.draft_chain(H, Lb, t0)
    finally:
        dh.set_chain_mode(prev)
    s_t, s_L, _ = head.draft_chain_sampled(H, Lb, t0, 0.0, seed=5)
    assert torch.equal(g_t, s_t) and torch.equal(g_L, s_L)


@functools.lru_cache(maxsize=1)
def _table_head(key):
    cfg = synth.CONFIGS[key]
    head = dh.DraftHead.from_config(cfg, weights_for(key))
    head.prepare_input_table()
    return head


# the bench's launch configurations with the table: batch 1 persistent
# (tokens only, as timed, and with logits), batch 32 and 8B batch 16 three
# launches per step
@pytest.mark.parametrize("key,sample,mode,logits", [
    ("qwen3_4b_b1", [0], 0, False), ("qwen3_4b_b1", [0], 0, True), ("qwen3_4b_b1", [0], 1, True),
    ("qwen3_4b_b32", [0, 13, 31], 0, True), ("qwen3_4b_b32", [5, 30], 0, False),
    ("qwen3_8b_b16", [0, 15], 0, False), ("qwen3_8b_b16", [7], 3, True)])
def test_chain_with_table_full_size_sampled(key, sample, mode, logits):
    cfg = synth.CONFIGS[key]
    say(f"case chain with table full {key} mode={mode} logits={logits} sample={sample}")
    head = _table_head(key)
    inp = synth.make_inputs(cfg)
    prev = dh.set_chain_mode(mode)
    try:
        H, t0 = head.upload(inp["H"]), head.upload(inp["t0"])
        Lb = head.base_logits(H)
        toks, L, _ = head.draft_chain(H, Lb, t0, want_logits=logits)
        torch.cuda.synchronize()
    finally:
        dh.set_chain_mode(prev)
    w = weights_for(key)
    m = oracle.Model.from_config(cfg, w)
    Hs_ = np.ascontiguousarray(inp["H"][sample])
    info = compare_chain(m, Hs_, m.base_logits(Hs_), inp["t0"][sample], toks.cpu().numpy()[sample],
                         L.cpu().numpy()[sample] if logits else None, key)
    say("  ", info)
