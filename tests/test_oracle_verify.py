"""Pins of the oracle's tree verification inputs (ancestor-only mask, position ids).

* the worked micro tree (one anchor, three nodes), written out by hand;
* closed forms: a chain-shaped tree gives the ordinary lower-triangular
  causal mask and consecutive positions; a star gives the anchor column plus
  the diagonal;
* trees from the oracle's own best-first builder: the mask equals the
  reflexive-transitive closure of the parent relation computed by repeated
  boolean matrix products (a different algorithm from the parent walk), and
  positions minus the start equal the builder's depths;
* padding: unfilled slots and malformed parents are marked, never followed.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import small_config


def test_micro_tree_by_hand():
    # anchor t0 = 1; nodes (parent, token): (-1, 0), (0, 1), (-1, 2)
    parents = np.array([[-1, 0, -1]], np.int32)
    tokens = np.array([[0, 1, 2]], np.int32)
    mask, pos, tok = oracle.tree_verify_inputs(parents, tokens, np.array([1], np.int32), np.array([10], np.int32))
    assert mask[0].tolist() == [[1, 0, 0, 0], [1, 1, 0, 0], [1, 1, 1, 0], [1, 0, 0, 1]]
    assert pos[0].tolist() == [10, 11, 12, 11]
    assert tok[0].tolist() == [1, 0, 1, 2]


@pytest.mark.parametrize("N", [1, 5, 16, 64])
def test_chain_tree_is_causal_mask(N):
    parents = np.arange(-1, N - 1, dtype=np.int32)[None]
    tokens = np.arange(100, 100 + N, dtype=np.int32)[None]
    mask, pos, tok = oracle.tree_verify_inputs(parents, tokens, np.array([7], np.int32))
    assert np.array_equal(mask[0], np.tril(np.ones((N + 1, N + 1), np.uint8)))
    assert pos[0].tolist() == list(range(N + 1))
    assert tok[0].tolist() == [7] + list(range(100, 100 + N))


def test_star_tree():
    N = 9
    parents = np.full((1, N), -1, np.int32)
    tokens = np.arange(N, dtype=np.int32)[None]
    mask, pos, _ = oracle.tree_verify_inputs(parents, tokens, np.array([3], np.int32), np.array([4], np.int32))
    expect = np.eye(N + 1, dtype=np.uint8)
    expect[:, 0] = 1
    assert np.array_equal(mask[0], expect)
    assert pos[0].tolist() == [4] + [5] * N


def closure(parents, in_tree):
    """Reflexive-transitive closure of child -> parent over entries (anchor = 0)."""
    E = parents.size + 1
    A = np.eye(E, dtype=np.int64)
    for k, q in enumerate(parents):
        if in_tree[k + 1]:
            A[k + 1, q + 1] = 1
    R = A.copy()
    for _ in range(E):
        R2 = ((R @ A) > 0).astype(np.int64) | R
        if np.array_equal(R2, R):
            break
        R = R2
    return R.astype(np.uint8)


@pytest.mark.parametrize("N,M,P", [(16, 4, 5), (40, 3, 16), (64, 8, 6), (12, 2, 2)])
def test_builder_trees_against_closure(N, M, P):
    cfg = small_config(d=16, V=97, Hs=8, r=8, P=P, B=4, dtype="f32", biases=True)
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    m = oracle.Model.from_config(cfg, w)
    Lb = m.base_logits(inp["H"])
    tr = m.tree(inp["H"], Lb, inp["t0"], N, M)
    start = np.array([0, 3, 100, 2 ** 20], np.int32)
    mask, pos, tok = oracle.tree_verify_inputs(tr["parents"], tr["tokens"], inp["t0"], start)
    for b in range(cfg.batch):
        in_tree = np.concatenate([[True], tr["tokens"][b] >= 0])
        assert np.array_equal(mask[b], closure(tr["parents"][b], in_tree))
        d = np.concatenate([[0], tr["depth"][b]])
        assert np.array_equal(pos[b][in_tree], start[b] + d[in_tree])
        assert np.all(pos[b][~in_tree] == -1)
        # the depth is the number of strict ancestors
        assert np.array_equal((mask[b].sum(axis=1) - 1)[in_tree], d[in_tree])


def test_padding_and_malformed_parents():
    parents = np.array([[-1, 0, 5, -1, 2, 1]], np.int32)   # slot 2 points ahead: malformed
    tokens = np.array([[4, 5, 6, -1, 8, 9]], np.int32)     # slot 3 unfilled
    mask, pos, tok = oracle.tree_verify_inputs(parents, tokens, np.array([2], np.int32))
    in_tree = [True, True, True, False, False, False, True]  # slot 4's parent (slot 2) is not in the tree
    for i in range(7):
        if not in_tree[i]:
            assert mask[0, i].tolist() == [int(j == i) for j in range(7)]
            assert pos[0, i] == -1 and tok[0, i] == -1
    assert mask[0, 6].tolist() == [1, 1, 1, 0, 0, 0, 1]  # node 5 -> node 1 -> node 0 -> anchor
    assert pos[0].tolist() == [0, 1, 2, -1, -1, -1, 3]
