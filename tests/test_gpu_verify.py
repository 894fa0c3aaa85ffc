"""GPU parity of the tree verification inputs against the oracle: bit-exact
(integer work) on hand-built, built and degenerate trees."""
import numpy as np
import pytest
import torch

import draft_head_amd as dh
import oracle
import synth
from gpu_common import say, weights_for
from helpers import small_config

pytestmark = pytest.mark.gpu


def _gpu(parents, tokens, t0, start=None):
    d = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    mask, pos, tok = dh.tree_verify_inputs(d(parents), d(tokens), d(t0), d(start))
    torch.cuda.synchronize()
    return mask.cpu().numpy(), pos.cpu().numpy(), tok.cpu().numpy()


def _check(parents, tokens, t0, start=None, label=""):
    g = _gpu(parents, tokens, t0, start)
    o = oracle.tree_verify_inputs(parents, tokens, t0, start)
    for name, a, b in zip(("mask", "positions", "tokens"), g, o):
        assert np.array_equal(a, b), f"{label}: {name} differ"
    return g


def test_micro_and_degenerate_trees():
    say("case verify micro / degenerate")
    _check(np.array([[-1, 0, -1]]), np.array([[0, 1, 2]]), np.array([1]), np.array([10]), "micro")
    for N in (1, 2, 63, 64):  # chains up to the 65-entry mask (bit 64 of a row)
        _check(np.arange(-1, N - 1)[None], np.arange(N)[None] + 5, np.array([3]), np.array([7]), f"chain {N}")
        _check(np.full((1, N), -1), np.arange(N)[None], np.array([3]), None, f"star {N}")
    # padding, malformed parents (ahead of the node, below -1), a negative token
    parents = np.array([[-1, 0, 5, -1, 2, 1, -7, 0]])
    tokens = np.array([[4, 5, 6, -1, 8, 9, 3, -2]])
    _check(parents, tokens, np.array([2]), np.array([1 << 20]), "padding")


def test_random_structures_many_sequences():
    say("case verify random structures")
    rng = np.random.default_rng(3)
    B, N = 300, 64
    parents = np.empty((B, N), np.int64)
    for k in range(N):
        parents[:, k] = rng.integers(-1, k, size=B) if k > 0 else -1
    tokens = rng.integers(-1, 1000, size=(B, N))  # about 0.1% padding slots
    tokens[rng.random((B, N)) < 0.05] = -1
    parents[rng.random((B, N)) < 0.02] += 70   # some malformed parents
    _check(parents, tokens, rng.integers(0, 1000, size=B), rng.integers(0, 4096, size=B), "random")


@pytest.mark.parametrize("N,M", [(16, 4), (40, 3), (64, 8)])
def test_built_trees(N, M):
    cfg = small_config(d=64, V=1003, Hs=32, r=32, P=6, B=5, dtype="bf16", biases=True)
    say(f"case verify built trees N={N} M={M}")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    H, t0 = head.upload(inp["H"]), head.upload(inp["t0"])
    out, _ = head.tree_draft(H, head.base_logits(H), t0, N, M)
    mask, pos, tok = dh.tree_verify_inputs(out["parents"], out["tokens"], t0)
    torch.cuda.synchronize()
    o = oracle.tree_verify_inputs(out["parents"].cpu().numpy(), out["tokens"].cpu().numpy(), inp["t0"])
    assert np.array_equal(mask.cpu().numpy(), o[0]) and np.array_equal(pos.cpu().numpy(), o[1])
    assert np.array_equal(tok.cpu().numpy(), o[2])
    # positions are the tree's depths
    d = out["depth"].cpu().numpy()
    assert np.array_equal(pos.cpu().numpy()[:, 1:][d > 0], d[d > 0])


def test_full_size_tree_then_verification_inputs():
    key = "qwen3_4b_tree"
    cfg = synth.CONFIGS[key]
    say(f"case verify full {key}")
    w = weights_for("qwen3_4b_b1")
    inp = synth.make_inputs(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    H, t0 = head.upload(inp["H"]), head.upload(inp["t0"])
    out, _ = head.tree_draft(H, head.base_logits(H), t0, cfg.nodes, cfg.topm)
    start = torch.arange(cfg.batch, dtype=torch.int32, device="cuda") * 1000
    mask, pos, tok = dh.tree_verify_inputs(out["parents"], out["tokens"], t0, start)
    torch.cuda.synchronize()
    o = oracle.tree_verify_inputs(out["parents"].cpu().numpy(), out["tokens"].cpu().numpy(), inp["t0"],
                                  start.cpu().numpy())
    assert np.array_equal(mask.cpu().numpy(), o[0]) and np.array_equal(pos.cpu().numpy(), o[1])
    assert np.array_equal(tok.cpu().numpy(), o[2])
