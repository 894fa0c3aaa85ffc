"""Pins of the oracle's sampled chain (temperature T > 0, Gumbel-max).

* Philox4x32-10, the counter-based generator the noise comes from, against
  the published known-answer vectors of its definition (Salmon, Moraes,
  Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011; the
  vectors ship with the authors' Random123 library);
* the noise: its empirical distribution against the standard Gumbel CDF
  exp(-exp(-x)) (Kolmogorov-Smirnov), mean (Euler's constant) and variance
  (pi^2 / 6), and no correlation between neighbouring counters;
* T = 0 is the greedy chain exactly;
* the drawn tokens follow softmax(L / T): many independent sequences on the
  same logits, chi-square against the closed-form probabilities (a sign
  error, a missing temperature or noise applied to the wrong side fails).
"""
import math

import numpy as np
import pytest
from scipy import stats

import oracle
import synth
from helpers import small_config

# (counter, key) -> output, from the known-answer tests published with the generator
PHILOX_KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("ctr,key,expect", PHILOX_KAT)
def test_philox_known_answers(ctr, key, expect):
    assert tuple(int(x) for x in oracle.philox4x32_10(ctr, key)) == expect


def _noise(seed, b, p, n):
    return np.array([oracle.gumbel(seed, b, p, v) for v in range(n)])


def test_gumbel_noise_distribution():
    g = _noise(12345, 3, 5, 100000)
    # the distribution the Gumbel-max trick needs: F(x) = exp(-exp(-x))
    ks = stats.kstest(g, "gumbel_r")
    assert ks.pvalue > 1e-3, ks
    assert abs(g.mean() - np.euler_gamma) < 0.02
    assert abs(g.var() - math.pi ** 2 / 6) < 0.05
    # the u grid (2k+1)/2^24 bounds the tails: g lies within [-log(-log(2^-24)), -log(-log(1-2^-24))]
    assert g.min() >= -math.log(-math.log(2.0 ** -24)) and g.max() <= -math.log(-math.log1p(-2.0 ** -24))


def test_gumbel_noise_streams_independent():
    n = 20000
    base = _noise(7, 0, 0, n)
    for other in (_noise(7, 1, 0, n), _noise(7, 2, 0, n), _noise(7, 0, 1, n), _noise(8, 0, 0, n)):
        assert not np.array_equal(base, other)
        assert abs(np.corrcoef(base, other)[0, 1]) < 0.03


def _model(V=6, P=2, seed=3):
    cfg = small_config(d=8, V=V, Hs=8, r=8, P=P, B=1, dtype="f32", biases=False)
    w = synth.make_weights(cfg)
    return cfg, w


def test_zero_temperature_is_greedy():
    cfg = small_config(d=16, V=37, Hs=8, r=8, P=5, B=3, dtype="f32", biases=True)
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    m = oracle.Model.from_config(cfg, w)
    Lb = m.base_logits(inp["H"])
    t_g, L_g, m_g = m.chain(inp["H"], Lb, inp["t0"])
    t_s, L_s, m_s = m.chain_sampled(inp["H"], Lb, inp["t0"], 0.0, seed=99)
    assert np.array_equal(t_g, t_s) and np.array_equal(L_g, L_s) and np.array_equal(m_g, m_s)


@pytest.mark.parametrize("T", [0.7, 1.0, 2.5])
def test_sampled_tokens_follow_softmax(T):
    """W2 = 0 makes every position's logits the given base row, so sequence b's first token
    is one Gumbel-max draw from softmax(L / T) with noise of its own (b differs)."""
    cfg, w = _model()
    w["w2"] = np.zeros_like(w["w2"])
    m = oracle.Model.from_config(cfg, w)
    L = np.array([1.0, 0.5, 0.0, -0.5, 2.0, 1.2], np.float32)
    B = 4000
    H = np.zeros((B, cfg.block, cfg.hidden), np.float32)
    Lb = np.broadcast_to(L, (B, cfg.block, cfg.vocab)).copy()
    t0 = np.zeros(B, np.int32)
    toks, logits, _ = m.chain_sampled(H, Lb, t0, T, seed=2024, want_logits=False)
    counts = np.bincount(toks[:, 0], minlength=cfg.vocab)
    p = np.exp(L / T - np.max(L / T))
    p /= p.sum()
    chi = stats.chisquare(counts, p * B)
    assert chi.pvalue > 1e-3, (counts, p * B)
    # the second position draws again, independently of the first
    agree = np.mean(toks[:, 0] == toks[:, 1])
    assert abs(agree - np.sum(p * p)) < 0.04


def test_sampled_chain_with_correction_and_forced_prefix():
    """With the correction on, the draw is the argmax of L + T g over the final logits, which
    oracle_chain computes; a forced prefix replays the fed-back tokens."""
    cfg = small_config(d=16, V=37, Hs=8, r=8, P=5, B=3, dtype="f32", biases=True)
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    m = oracle.Model.from_config(cfg, w)
    Lb = m.base_logits(inp["H"])
    T, seed = 0.8, 5
    toks, L, marg = m.chain_sampled(inp["H"], Lb, inp["t0"], T, seed)
    # the same logits come out of the greedy chain when its history is forced to the draws
    _, L_f, _ = m.chain(inp["H"], Lb, inp["t0"], forced=toks)
    assert np.array_equal(L, L_f)
    for b in range(cfg.batch):
        for p in range(cfg.block):
            pert = L[b, p] + T * np.array([oracle.gumbel(seed, b, p, v) for v in range(cfg.vocab)])
            assert toks[b, p] == int(np.argmax(pert))
            s = np.sort(pert)
            assert marg[b, p] == pytest.approx(s[-1] - s[-2], abs=1e-12)
    # forcing the sampled tokens replays them; seq0 shifts the noise streams
    t2, _, _ = m.chain_sampled(inp["H"], Lb, inp["t0"], T, seed, forced=toks)
    assert np.array_equal(t2, toks)
    t3, _, _ = m.chain_sampled(inp["H"][1:], Lb[1:], inp["t0"][1:], T, seed, seq0=1)
    assert np.array_equal(t3, toks[1:])
