"""Pins of the oracle's correction chain.

* a hand-sized worked example whose expected values follow in closed form
  (the GRU reduces to h' = tanh(x0 - 2 x1)/2 + h/2 there);
* the zero-correction case, which must reproduce argmax of the base logits
  (the "without Domino head" arm of the explainer's ablation, section 6);
* a chain assembled from torch float64 library routines;
* invariants: prefix stability, forced prefix, batch independence.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import small_config, widen


def micro_model(P=2):
    w = {
        "lm_head": np.array([[1, 0], [0, 1], [1, 1], [-1, 0]], np.float32),
        "embed": np.array([[0, 0], [1, 0], [0, 1], [1, 1]], np.float32),
        "w_ih": np.array([[0, 0], [0, 0], [1, -2]], np.float32),  # only the n gate reads x
        "w_hh": np.zeros((3, 1), np.float32),
        "w1": np.array([[0, 0, 4]], np.float32),
        "w2": np.array([[0], [1], [-1], [0]], np.float32),
    }
    return oracle.Model(2, 4, 1, 1, P, "f32", w), w


MICRO_H = np.array([[[1, 0], [0, 1]]], np.float32)


def silu(z):
    return z / (1 + math.exp(-z))


def micro_closed_form(t0):
    """Expected (tokens, logits) of the micro example, derived by hand."""
    E = [(0, 0), (1, 0), (0, 1), (1, 1)]
    Lb = [[1, 0, 1, -1], [0, 1, 1, 0]]
    h, prev, toks, logits = 0.0, t0, [], []
    for p in range(2):
        h = math.tanh(E[prev][0] - 2 * E[prev][1]) / 2 + h / 2  # r = z = 1/2, W_hh = 0
        a = silu(4 * h)
        L = [Lb[p][0], Lb[p][1] + a, Lb[p][2] - a, Lb[p][3]]
        t = max(range(4), key=lambda v: (L[v], -v))
        toks.append(t)
        logits.append(L)
        prev = t
    return toks, logits


@pytest.mark.parametrize("t0", [0, 1, 2, 3])
def test_micro_example(t0):
    m, w = micro_model()
    Lb = m.base_logits(MICRO_H)
    np.testing.assert_array_equal(Lb, [[[1, 0, 1, -1], [0, 1, 1, 0]]])
    toks, L, margins = m.chain(MICRO_H, Lb, np.array([t0]))
    ref_t, ref_L = micro_closed_form(t0)
    assert toks[0].tolist() == ref_t
    np.testing.assert_allclose(L[0], ref_L, rtol=0, atol=1e-15)


def test_micro_example_printed_values():
    # decimals of the worked example (t0 = 1 and t0 = 2), ten digits
    m, _ = micro_model()
    Lb = m.base_logits(MICRO_H)
    toks, L, _ = m.chain(np.concatenate([MICRO_H] * 2), np.concatenate([Lb] * 2), np.array([1, 2]))
    assert toks.tolist() == [[1, 1], [2, 2]]
    np.testing.assert_allclose(L[0, 0], [1, 1.2505490219, -0.2505490219, -1], atol=1e-10)
    np.testing.assert_allclose(L[0, 1], [0, 3.0736888186, -1.0736888186, 0], atol=1e-10)
    np.testing.assert_allclose(L[1, 0], [1, -0.2447974530, 1.2447974530, -1], atol=1e-10)
    np.testing.assert_allclose(L[1, 1], [0, 0.8480316599, 1.1519683401, 0], atol=1e-10)


def test_micro_ties_go_to_lowest_index():
    m, _ = micro_model()
    Lb = m.base_logits(MICRO_H)
    toks, _, margins = m.chain(MICRO_H, Lb, np.array([0]))
    assert toks[0].tolist() == [0, 1]  # [1,0,1,-1] -> 0 and [0,1,1,0] -> 1
    assert margins[0].tolist() == [0.0, 0.0]


def _model(cfg, **override):
    w = synth.make_weights(cfg)
    w.update(override)
    return oracle.Model.from_config(cfg, w), w


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_correction_reproduces_base_argmax(dtype):
    cfg = small_config(dtype=dtype, B=3, V=61)
    store = np.float32 if dtype == "f32" else np.uint16
    m, w = _model(cfg, w2=np.zeros((cfg.vocab, cfg.rank), store), b2=None)
    inp = synth.make_inputs(cfg)
    Lb = m.base_logits(inp["H"])
    toks, L, _ = m.chain(inp["H"], Lb, inp["t0"])
    assert np.array_equal(L, Lb.astype(np.float64))
    assert np.array_equal(toks, np.argmax(Lb, axis=-1))


def torch_chain(cfg, w, H, Lb, t0):
    """The chain assembled from torch float64 routines (GRUCell, silu, matmul)."""
    dt = cfg.dtype
    cell = torch.nn.GRUCell(cfg.hidden, cfg.gru_hidden, dtype=torch.float64)
    f = lambda a: torch.from_numpy(widen(a, dt))
    with torch.no_grad():
        cell.weight_ih.copy_(f(w["w_ih"]))
        cell.weight_hh.copy_(f(w["w_hh"]))
        cell.bias_ih.copy_(torch.from_numpy(w["b_ih"].astype(np.float64)))
        cell.bias_hh.copy_(torch.from_numpy(w["b_hh"].astype(np.float64)))
        E, W1, W2 = f(w["embed"]), f(w["w1"]), f(w["w2"])
        b1, b2 = torch.from_numpy(w["b1"].astype(np.float64)), torch.from_numpy(w["b2"].astype(np.float64))
        Hd = f(H)
        B, P = Hd.shape[0], Hd.shape[1]
        toks = np.zeros((B, P), np.int64)
        logits = np.zeros((B, P, cfg.vocab))
        for b in range(B):
            h = torch.zeros(1, cfg.gru_hidden, dtype=torch.float64)
            prev = int(t0[b])
            for p in range(P):
                h = cell(E[prev][None], h)
                a = torch.nn.functional.silu(W1 @ torch.cat([Hd[b, p], h[0]]) + b1)
                L = torch.from_numpy(Lb[b, p].astype(np.float64)) + W2 @ a + b2
                prev = int(torch.argmax(L))
                toks[b, p] = prev
                logits[b, p] = L.numpy()
    return toks, logits


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_matches_torch_assembly(dtype):
    cfg = small_config(dtype=dtype, B=3, P=6, V=71, d=32, Hs=16, r=16)
    m, w = _model(cfg)
    inp = synth.make_inputs(cfg)
    Lb = m.base_logits(inp["H"])
    toks, L, margins = m.chain(inp["H"], Lb, inp["t0"])
    rt, rL = torch_chain(cfg, w, inp["H"], Lb, inp["t0"])
    assert margins.min() > 1e-9
    assert np.array_equal(toks, rt)
    np.testing.assert_allclose(L, rL, rtol=1e-12, atol=1e-12)


def test_feedback_changes_later_positions():
    cfg = small_config(B=1, P=4, V=41)
    m, _ = _model(cfg)
    inp = synth.make_inputs(cfg)
    Lb = m.base_logits(inp["H"])
    toks, L, _ = m.chain(inp["H"], Lb, inp["t0"])
    other = (toks + 1) % cfg.vocab
    _, L2, _ = m.chain(inp["H"], Lb, inp["t0"], forced=other)
    np.testing.assert_array_equal(L2[:, 0], L[:, 0])  # position 0 sees only t0
    assert np.abs(L2[:, 1:] - L[:, 1:]).max() > 1e-3


def test_forced_with_own_tokens_reproduces_chain():
    cfg = small_config(B=2, P=6)
    m, _ = _model(cfg)
    inp = synth.make_inputs(cfg)
    Lb = m.base_logits(inp["H"])
    toks, L, mg = m.chain(inp["H"], Lb, inp["t0"])
    t2, L2, mg2 = m.chain(inp["H"], Lb, inp["t0"], forced=toks)
    assert np.array_equal(toks, t2) and np.array_equal(L, L2) and np.array_equal(mg, mg2)


def test_prefix_and_batch_independence():
    cfg = small_config(B=3, P=6)
    m, _ = _model(cfg)
    inp = synth.make_inputs(cfg)
    H, t0 = inp["H"], inp["t0"]
    Lb = m.base_logits(H)
    toks, L, _ = m.chain(H, Lb, t0)
    # a shorter block on the same rows gives the same leading outputs
    m3 = m.with_block(3)
    t3, L3, _ = m3.chain(np.ascontiguousarray(H[:, :3]), np.ascontiguousarray(Lb[:, :3]), t0)
    assert np.array_equal(t3, toks[:, :3]) and np.array_equal(L3, L[:, :3])
    # each sequence alone gives what it gives inside the batch
    for b in range(3):
        tb, Lb_b, _ = m.chain(H[b:b + 1], Lb[b:b + 1], t0[b:b + 1])
        assert np.array_equal(tb[0], toks[b]) and np.array_equal(Lb_b[0], L[b])
