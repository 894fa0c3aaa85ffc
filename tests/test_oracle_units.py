"""Pins of the oracle's single operations.

Each check ties the oracle to something other than itself: hand values of
the definitions, torch float64 library routines, or exact arithmetic.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import small_config, widen


def _scalar_model(w_ih, w_hh, b_ih=None, b_hh=None):
    """d = Hs = 1 GRU with fp32 storage (r = 1, V = 1 placeholders)."""
    z = np.zeros((1, 1), np.float32)
    w = {"lm_head": z, "embed": z, "w_ih": np.array(w_ih, np.float32).reshape(3, 1),
         "w_hh": np.array(w_hh, np.float32).reshape(3, 1), "w1": np.zeros((1, 2), np.float32), "w2": z,
         "b_ih": None if b_ih is None else np.array(b_ih, np.float32),
         "b_hh": None if b_hh is None else np.array(b_hh, np.float32)}
    return oracle.Model(1, 1, 1, 1, 1, "f32", w)


# ---- SiLU: SiLU(z) = z * sigmoid(z) ---------------------------------------
@pytest.mark.parametrize("z,val", [(0.0, 0.0), (1.0, 0.7310585786300049), (-1.0, -0.2689414213699951),
                                   (2.0, 1.7615941559557646), (-2.0, -0.2384058440442351),
                                   (0.5, 0.3112296656009273)])
def test_silu_hand_values(z, val):
    assert oracle.silu(z) == pytest.approx(val, abs=1e-15)


def test_silu_matches_torch():
    z = np.linspace(-30, 30, 1201)
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    got = np.array([oracle.silu(v) for v in z])
    np.testing.assert_allclose(got, ref, rtol=1e-15, atol=1e-300)


# ---- GRU cell: hand values that also tell the two common GRU forms apart ----
# weights listed as (r, z, n) rows
def test_gru_G0_zero_weights_average_state():
    m = _scalar_model([0, 0, 0], [0, 0, 0])
    assert m.gru_cell([3.0], [0.8])[0] == pytest.approx(0.4, abs=1e-15)


def test_gru_G1_input_only():
    m = _scalar_model([1, 1, 1], [0, 0, 0])
    assert m.gru_cell([1.0], [0.0])[0] == pytest.approx(0.20482421480982513, abs=1e-14)


def test_gru_G2_hidden_n_path():
    # n = tanh(0.5), h' = (1 + tanh 0.5) / 2 = sigmoid(1)
    m = _scalar_model([0, 0, 0], [0, 0, 1])
    assert m.gru_cell([0.0], [1.0])[0] == pytest.approx(0.7310585786300049, abs=1e-14)


def test_gru_G3_reset_gates_hidden_bias():
    # torch form: n = tanh(r * (W_hn h + b_hn)) = tanh(0.5) -> h' = 0.2310585786;
    # the reset-before-matmul form would give 0.5 * tanh(1) = 0.3807970780
    m = _scalar_model([0, 0, 0], [0, 0, 0], b_hh=[0, 0, 1])
    got = m.gru_cell([0.0], [0.0])[0]
    assert got == pytest.approx(0.23105857863000487, abs=1e-14)
    assert abs(got - 0.3807970779778824) > 0.1


def test_gru_G4_mixed():
    m = _scalar_model([0, 0, 0], [1, -1, 2], b_hh=[0, 0, 0.25])
    assert m.gru_cell([0.0], [0.5])[0] == pytest.approx(0.5943647950267916, abs=1e-14)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gru_matches_torch_grucell(dtype):
    cfg = small_config(d=24, Hs=16, dtype=dtype)
    w = synth.make_weights(cfg)
    m = oracle.Model.from_config(cfg, w)
    cell = torch.nn.GRUCell(cfg.hidden, cfg.gru_hidden, dtype=torch.float64)
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(widen(w["w_ih"], dtype)))
        cell.weight_hh.copy_(torch.from_numpy(widen(w["w_hh"], dtype)))
        cell.bias_ih.copy_(torch.from_numpy(w["b_ih"].astype(np.float64)))
        cell.bias_hh.copy_(torch.from_numpy(w["b_hh"].astype(np.float64)))
    rng = np.random.default_rng(0)
    for _ in range(5):
        x = rng.standard_normal(cfg.hidden)
        h = rng.standard_normal(cfg.gru_hidden) * 0.7
        with torch.no_grad():
            ref = cell(torch.from_numpy(x)[None], torch.from_numpy(h)[None])[0].numpy()
        np.testing.assert_allclose(m.gru_cell(x, h), ref, rtol=1e-13, atol=1e-14)


# ---- argmax: first maximum wins, -0 equals +0 -------------------------------
def test_argmax_ties_and_zero_sign():
    assert oracle.argmax([1, 3, 3, 2])[0] == 1
    assert oracle.argmax([5, 5, 5, 5]) == (0, 0.0)
    assert oracle.argmax([-0.0, 0.0])[0] == 0
    assert oracle.argmax([0.0, -0.0])[0] == 0
    t, m = oracle.argmax([0.5, 2.0, -1.0, 1.25])
    assert t == 1 and m == pytest.approx(0.75)


def test_argmax_matches_torch_first_occurrence():
    rng = np.random.default_rng(1)
    for _ in range(50):
        L = np.round(rng.standard_normal(97) * 3) / 2  # many exact ties
        assert oracle.argmax(L)[0] == int(torch.argmax(torch.from_numpy(L)))


# ---- top-M: ordered by (value desc, index asc) ------------------------------
def test_topm_matches_lexsort():
    rng = np.random.default_rng(2)
    for M in (1, 3, 8, 64):
        row = (np.round(rng.standard_normal(500) * 4) / 4).astype(np.float32)  # ties
        idx, val = oracle.topm(row, M)
        ref = np.lexsort((np.arange(row.size), -row.astype(np.float64)))[:M]
        assert np.array_equal(idx, ref)
        assert np.array_equal(val, row[ref])


# ---- base logits: H W_lm^T against a library product in float64 ------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_base_logits_matches_torch_matmul(dtype):
    cfg = small_config(d=72, V=53, dtype=dtype)
    w = synth.make_weights(cfg)
    H = synth.make_inputs(cfg)["H"]
    m = oracle.Model.from_config(cfg, w)
    got = m.base_logits(H)
    ref = torch.from_numpy(widen(H, dtype)) @ torch.from_numpy(widen(w["lm_head"], dtype)).T
    # the oracle rounds a double sum once to fp32: within one fp32 rounding of the exact value
    ref = ref.numpy()
    assert got.dtype == np.float32 and got.shape == (cfg.batch, cfg.block, cfg.vocab)
    np.testing.assert_allclose(got, ref, rtol=2 ** -24 * 1.0001, atol=1e-30)


def test_bottleneck_and_final_logits_match_torch():
    cfg = small_config(d=24, Hs=16, r=8, V=29, dtype="bf16")
    w = synth.make_weights(cfg)
    m = oracle.Model.from_config(cfg, w)
    H = synth.make_inputs(cfg)["H"]
    rng = np.random.default_rng(3)
    S = rng.standard_normal(cfg.gru_hidden)
    a = m.bottleneck(H[0, 1], S)
    cat = np.concatenate([widen(H[0, 1], "bf16"), S])
    ref_a = torch.nn.functional.silu(torch.from_numpy(widen(w["w1"], "bf16") @ cat + w["b1"])).numpy()
    np.testing.assert_allclose(a, ref_a, rtol=1e-13, atol=1e-15)
    Lb = rng.standard_normal(cfg.vocab).astype(np.float32)
    L = m.final_logits(Lb, a)
    ref_L = Lb.astype(np.float64) + widen(w["w2"], "bf16") @ ref_a + w["b2"]
    np.testing.assert_allclose(L, ref_L, rtol=1e-13, atol=1e-14)
