"""Pins of the oracle's best-first tree.

The tree is pinned by brute force: every node of the M-ary tree to depth P
is scored independently (its GRU state recomputed from the anchor along its
own path with torch.nn.GRUCell), all nodes are sorted by score, and the top
N must be the oracle's nodes in the same order with the same parents.
Special cases: W2 = 0 makes scores path independent (marginal k-best sums);
M = 1 gives a single chain; a hand-sized example in closed form.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import small_config, widen
from test_oracle_chain import MICRO_H, micro_model


def candidates(Lb_b, M):
    return [np.lexsort((np.arange(Lb_b.shape[1]), -Lb_b[p].astype(np.float64)))[:M] for p in range(Lb_b.shape[0])]


def brute_force_tree(cfg, w, H_b, Lb_b, t0, M, N, P):
    dt = cfg.dtype
    f = lambda a: torch.from_numpy(widen(a, dt))
    cell = torch.nn.GRUCell(cfg.hidden, cfg.gru_hidden, dtype=torch.float64)
    zeros = lambda n: np.zeros(n)
    with torch.no_grad():
        cell.weight_ih.copy_(f(w["w_ih"]))
        cell.weight_hh.copy_(f(w["w_hh"]))
        cell.bias_ih.copy_(torch.from_numpy(w["b_ih"] if w["b_ih"] is not None else zeros(3 * cfg.gru_hidden)))
        cell.bias_hh.copy_(torch.from_numpy(w["b_hh"] if w["b_hh"] is not None else zeros(3 * cfg.gru_hidden)))
    E, W1, W2 = widen(w["embed"], dt), widen(w["w1"], dt), widen(w["w2"], dt)
    b1 = w["b1"].astype(np.float64) if w["b1"] is not None else zeros(cfg.rank)
    b2 = w["b2"].astype(np.float64) if w["b2"] is not None else zeros(cfg.vocab)
    Hd = widen(H_b, dt)
    C = candidates(Lb_b, M)

    def state_after(tokens):
        h = torch.zeros(1, cfg.gru_hidden, dtype=torch.float64)
        with torch.no_grad():
            for t in tokens:
                h = cell(torch.from_numpy(E[t])[None], h)
        return h[0].numpy()

    def logp(depth, prefix_tokens):
        S = state_after([t0] + prefix_tokens)
        a = torch.nn.functional.silu(torch.from_numpy(W1 @ np.concatenate([Hd[depth], S]) + b1)).numpy()
        c = C[depth]
        l = Lb_b[depth][c].astype(np.float64) + W2[c] @ a + b2[c]
        mx = l.max()
        return l - (mx + math.log(np.exp(l - mx).sum()))

    nodes = []  # (score, ranks path)
    for D in range(1, P + 1):
        for ranks in itertools.product(range(M), repeat=D):
            toks = [int(C[i][ranks[i]]) for i in range(D)]
            score = sum(logp(i, toks[:i])[ranks[i]] for i in range(D))
            nodes.append((score, ranks, toks[-1]))
    nodes.sort(key=lambda n: -n[0])
    top = nodes[:N]
    index = {n[1]: k for k, n in enumerate(top)}
    parents = [index[n[1][:-1]] if len(n[1]) > 1 else -1 for n in top]
    return {"parents": parents, "tokens": [n[2] for n in top], "depth": [len(n[1]) for n in top],
            "scores": [n[0] for n in top]}


def _setup(cfg, **override):
    w = synth.make_weights(cfg)
    w.update(override)
    m = oracle.Model.from_config(cfg, w)
    inp = synth.make_inputs(cfg)
    Lb = m.base_logits(inp["H"])
    return m, w, inp, Lb


@pytest.mark.parametrize("M,P,dtype,seed", [(2, 4, "f32", 1), (3, 3, "f32", 2), (3, 4, "bf16", 3),
                                            (2, 5, "bf16", 4)])
def test_tree_matches_brute_force(M, P, dtype, seed):
    cfg = small_config(dtype=dtype, P=P, B=2, V=29, iseed=seed, wseed=seed + 10)
    N = 16
    m, w, inp, Lb = _setup(cfg)
    got = m.tree(inp["H"], Lb, inp["t0"], N, M)
    for b in range(cfg.batch):
        ref = brute_force_tree(cfg, w, inp["H"][b], Lb[b], int(inp["t0"][b]), M, N, P)
        assert got["tokens"][b].tolist() == ref["tokens"]
        assert got["parents"][b].tolist() == ref["parents"]
        assert got["depth"][b].tolist() == ref["depth"]
        np.testing.assert_allclose(got["scores"][b], ref["scores"], rtol=0, atol=1e-12)


def test_tree_invariants():
    cfg = small_config(P=8, B=3, V=97)
    N, M = 40, 6
    m, w, inp, Lb = _setup(cfg)
    t = m.tree(inp["H"], Lb, inp["t0"], N, M)
    for b in range(cfg.batch):
        C = candidates(Lb[b], M)
        s, par, dep, tok = t["scores"][b], t["parents"][b], t["depth"][b], t["tokens"][b]
        assert np.all(np.diff(s) <= 0)
        for k in range(N):
            assert par[k] < k
            assert dep[k] == (1 if par[k] < 0 else dep[par[k]] + 1)
            assert tok[k] in C[dep[k] - 1]
            assert s[k] < (0 if par[k] < 0 else s[par[k]])


def test_tree_zero_correction_is_marginal_kbest():
    cfg = small_config(P=4, B=2, V=31, dtype="f32")
    M, N = 3, 16
    m, w, inp, Lb = _setup(cfg, w2=np.zeros((cfg.vocab, cfg.rank), np.float32), b2=None)
    got = m.tree(inp["H"], Lb, inp["t0"], N, M)
    for b in range(cfg.batch):
        C = candidates(Lb[b], M)
        lp = []
        for p in range(cfg.block):
            l = Lb[b, p][C[p]].astype(np.float64)
            lp.append(l - (l.max() + math.log(np.exp(l - l.max()).sum())))
        nodes = sorted(((sum(lp[i][r] for i, r in enumerate(ranks)), ranks)
                        for D in range(1, cfg.block + 1) for ranks in itertools.product(range(M), repeat=D)),
                       key=lambda n: -n[0])[:N]
        assert got["tokens"][b].tolist() == [int(C[len(r) - 1][r[-1]]) for _, r in nodes]
        np.testing.assert_allclose(got["scores"][b], [s for s, _ in nodes], rtol=0, atol=1e-12)


def test_tree_single_candidate_is_a_chain():
    cfg = small_config(P=5, B=2, V=23)
    m, w, inp, Lb = _setup(cfg)
    t = m.tree(inp["H"], Lb, inp["t0"], 8, 1)
    for b in range(cfg.batch):
        assert t["tokens"][b, :5].tolist() == np.argmax(Lb[b], axis=-1).tolist()
        assert t["parents"][b, :5].tolist() == [-1, 0, 1, 2, 3]
        assert t["depth"][b, :5].tolist() == [1, 2, 3, 4, 5]
        assert np.all(t["scores"][b, :5] == 0)
        assert t["tokens"][b, 5:].tolist() == [-1] * 3 and t["parents"][b, 5:].tolist() == [-1] * 3
        assert np.all(np.isneginf(t["scores"][b, 5:]))


def test_tree_first_node_agrees_with_chain():
    cfg = small_config(P=4, B=4, V=53)
    M = 8
    m, w, inp, Lb = _setup(cfg)
    t = m.tree(inp["H"], Lb, inp["t0"], 6, M)
    toks, _, _ = m.chain(inp["H"], Lb, inp["t0"])
    checked = 0
    for b in range(cfg.batch):
        if toks[b, 0] in candidates(Lb[b], M)[0]:
            assert t["tokens"][b, 0] == toks[b, 0]
            checked += 1
    assert checked >= 2


def test_micro_tree():
    m, w = micro_model()
    Lb = m.base_logits(MICRO_H)
    H2 = np.concatenate([MICRO_H] * 2)
    t = m.tree(H2, np.concatenate([Lb] * 2), np.array([1, 2]), 3, 2)
    # closed form: r = z = 1/2, n = tanh(x0 - 2 x1), a = SiLU(4 h); C_0 = [0, 2], C_1 = [1, 2]
    sig = lambda x: 1 / (1 + math.exp(-x))
    silu = lambda x: x * sig(x)

    def lsm2(l0, l1):
        mx = max(l0, l1)
        lse = mx + math.log(math.exp(l0 - mx) + math.exp(l1 - mx))
        return l0 - lse, l1 - lse

    # anchor 1: h_root = tanh(1)/2
    a = silu(4 * math.tanh(1) / 2)
    p0 = lsm2(1.0, 1.0 - a)                     # children tokens 0, 2 at depth 1
    h1 = 0 / 2 + math.tanh(1) / 4               # node 0 read token 0: n = tanh(0)
    a1 = silu(4 * h1)
    p1 = lsm2(1.0 + a1, 1.0 - a1)               # its children tokens 1, 2
    assert t["tokens"][0].tolist() == [0, 1, 2]
    assert t["parents"][0].tolist() == [-1, 0, -1]
    np.testing.assert_allclose(t["scores"][0], [p0[0], p0[0] + p1[0], p0[1]], atol=1e-15)
    np.testing.assert_allclose(t["scores"][0], [-0.2518068402, -0.5548964967, -1.5023558621], atol=1e-10)
    # anchor 2: h_root = tanh(-2)/2
    a = silu(4 * math.tanh(-2) / 2)
    q0 = lsm2(1.0, 1.0 - a)
    h2 = math.tanh(-2) / 2 / 2 + math.tanh(0 - 2 * 1) / 2  # node 0 = token 2 -> x = (0, 1)
    a2 = silu(4 * h2)
    q1 = lsm2(1.0 + a2, 1.0 - a2)
    assert t["tokens"][1].tolist() == [2, 0, 2]
    assert t["parents"][1].tolist() == [-1, -1, 0]
    np.testing.assert_allclose(t["scores"][1], [q0[1], q0[0], q0[1] + q1[1]], atol=1e-15)
    np.testing.assert_allclose(t["scores"][1], [-0.5782205489, -0.8230180019, -1.1309024036], atol=1e-10)
