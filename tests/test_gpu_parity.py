"""GPU parity: the HIP path through the C ABI against the oracle.

Element-wise at sizes the oracle finishes in seconds (several tiles and a
ragged tail in every dimension), and on sampled sequences / rows at the full
Qwen3-4B / Qwen3-8B shapes, in the launch configuration the bench times.
"""
import functools

import numpy as np
import pytest
import torch

import draft_head_amd as dh
import oracle
import synth
from gpu_common import LOGIT_TOL, compare_chain, gemm_bound, say, weights_for
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


@functools.lru_cache(maxsize=2)
def device_head(cfg_key):
    cfg = synth.CONFIGS[cfg_key]
    return dh.DraftHead.from_config(cfg, weights_for(cfg_key))


def _run(cfg, w, inp, want_logits=True, head=None):
    head = head or dh.DraftHead.from_config(cfg, w)
    H = head.upload(inp["H"])
    t0 = head.upload(inp["t0"])
    Lb = head.base_logits(H)
    toks, L, ws = head.draft_chain(H, Lb, t0, want_logits=want_logits, check=False)
    torch.cuda.synchronize()
    status = dh.DraftHead.device_status(ws)
    return head, Lb.cpu().numpy(), toks.cpu().numpy(), None if L is None else L.cpu().numpy(), status


def _check_base_rel(g, ref, label):
    """The benchmark spec bar on L^base: row-relative error <= 1e-3 against the oracle."""
    err = row_rel_err(g, ref)
    assert err.max() <= LOGIT_TOL, f"{label}: base-logit error {err.max():.3e}"
    return float(err.max())


# ---- base logits ------------------------------------------------------------------
def _check_gemm(g, H, Wlm, dtype, label):
    Hd = widen(H, dtype).reshape(-1, H.shape[-1])
    Wd = widen(Wlm, dtype)
    exact = Hd @ Wd.T
    bound = gemm_bound(Hd, Wd) + np.abs(exact) * 2.0 ** -24
    err = np.abs(g.reshape(exact.shape).astype(np.float64) - exact)
    assert np.all(err <= bound), f"{label}: worst excess {(err - bound).max():.3e}"


def test_base_logits_tiny_f32():
    cfg = synth.CONFIGS["tiny_f32"]
    say("case tiny_f32 base logits")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    g = head.base_logits(head.upload(inp["H"])).cpu().numpy()
    _check_gemm(g, inp["H"], w["lm_head"], "f32", "tiny_f32")
    ref = oracle.Model.from_config(cfg, w).base_logits(inp["H"])
    assert np.max(np.abs(g - ref) / np.maximum(np.abs(ref), 1)) < 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,V,B,P", [(72, 1003, 3, 5), (136, 2051, 13, 16), (264, 1000, 5, 16), (40, 17, 1, 1),
                                     (72, 5003, 3, 5), (136, 6007, 13, 16), (264, 4099, 5, 16)])
def test_base_logits_ragged(dtype, d, V, B, P):
    cfg = small_config(d=d, V=V, B=B, P=P, dtype=dtype)
    say(f"case base logits ragged dtype={dtype} d={d} V={V} B={B} P={P}")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    g = head.base_logits(head.upload(inp["H"])).cpu().numpy()
    _check_gemm(g, inp["H"], w["lm_head"], dtype, "ragged")
    _check_base_rel(g, oracle.Model.from_config(cfg, w).base_logits(inp["H"]), "ragged")


# one sequence, many columns: the persistent balanced kernels (at least eight
# 16-column tiles per CU), with ragged rows, columns and k tails; k a multiple
# of 256 takes the slab-streaming kernel (the widest k whose A and slabs fit
# the LDS, the fewest tiles it takes, one row; up to 64 tiles per workgroup
# its output goes out as one block per workgroup, beyond that tile by tile),
# any other k the fragment one
@pytest.mark.parametrize("d,V,P", [(264, 33013, 5), (2568, 40009, 16), (40, 70001, 3), (1032, 36871, 1),
                                   (256, 32769, 5), (1024, 40009, 16), (2816, 36001, 7), (2560, 65537, 1),
                                   (256, 270001, 2)])
def test_base_logits_one_sequence_wide(d, V, P):
    cfg = small_config(d=d, V=V, B=1, P=P, dtype="bf16")
    say(f"case base logits one sequence wide d={d} V={V} P={P}")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    g = head.base_logits(head.upload(inp["H"])).cpu().numpy()
    _check_gemm(g, inp["H"], w["lm_head"], "bf16", "one sequence wide")
    g2 = head.base_logits(head.upload(inp["H"])).cpu().numpy()
    assert np.array_equal(g, g2)  # fixed split and summation order


# many rows (several sequences' blocks): the LDS-ring MFMA kernel for k a
# multiple of 64, all three tile shapes (128 x 320 up to 128 rows, 256 x 320 up
# to 256, 256 x 256 above), ragged rows and columns, several tiles per
# workgroup, and the look-ahead loads crossing tile boundaries
@pytest.mark.parametrize("d,V,B,P", [(320, 40009, 19, 16), (576, 9001, 8, 16), (1024, 70001, 3, 11),
                                     (384, 5003, 1, 7), (640, 33331, 40, 13), (2560, 12007, 32, 16),
                                     (1280, 20011, 13, 16), (768, 30011, 16, 16), (128, 4099, 2, 9)])
def test_base_logits_many_rows(d, V, B, P):
    cfg = small_config(d=d, V=V, B=B, P=P, dtype="bf16")
    say(f"case base logits many rows d={d} V={V} B={B} P={P}")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    Hd = head.upload(inp["H"])
    g = head.base_logits(Hd).cpu().numpy()
    _check_gemm(g, inp["H"], w["lm_head"], "bf16", "many rows")
    g2 = head.base_logits(Hd).cpu().numpy()
    assert np.array_equal(g, g2)


@pytest.mark.parametrize("key,rows", [("qwen3_4b_b1", [(0, 0), (0, 15)]), ("qwen3_4b_b32", [(0, 0), (31, 9)]),
                                      ("qwen3_8b_b16", [(0, 3), (15, 15)]), ("qwen3_4b_tree", [(0, 0), (7, 15)])])
def test_base_logits_full_size_sampled(key, rows):
    cfg = synth.CONFIGS[key]
    say(f"case base logits full {key}")
    head = device_head(key)
    inp = synth.make_inputs(cfg)
    g = head.base_logits(head.upload(inp["H"]))
    torch.cuda.synchronize()
    assert torch.isfinite(g).all().item()
    w = weights_for(key)
    m = oracle.Model.from_config(cfg, w)
    for b, p in rows:
        row = g[b, p].cpu().numpy()
        _check_gemm(row[None], inp["H"][b, p][None], w["lm_head"], cfg.dtype, f"{key} row {(b, p)}")
        _check_base_rel(row[None], m.base_logits(inp["H"][b, p][None]), f"{key} row {(b, p)}")


# ---- chain ---------------------------------------------------------------------------
def test_chain_tiny_f32(chain_mode):
    cfg = synth.CONFIGS["tiny_f32"]
    say(f"case chain tiny_f32 mode={chain_mode}")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    _, Lb, toks, L, status = _run(cfg, w, inp)
    assert status == 0
    m = oracle.Model.from_config(cfg, w)
    info = compare_chain(m, inp["H"], m.base_logits(inp["H"]), inp["t0"], toks, L, "tiny_f32")
    say("  ", info)


CHAIN_SHAPES = [
    # d, V, Hs, r, P, B, dtype
    (16, 37, 8, 8, 5, 2, "f32"),
    (64, 1003, 40, 24, 7, 5, "bf16"),
    (200, 2051, 64, 64, 16, 17, "bf16"),
    (96, 4099, 128, 256, 16, 32, "bf16"),
    (48, 515, 16, 16, 3, 40, "bf16"),   # two launches of <= 32 sequences
    (64, 999, 32, 40, 16, 9, "f32"),
    (32, 64, 8, 8, 1, 1, "bf16"),
    (64, 2053, 32, 256, 5, 24, "bf16"),  # rank 256: whole-row phase O, ragged vocabulary and row groups
    (32, 1037, 16, 256, 3, 40, "bf16"),
    # W1[:, :d] H split over k across workgroups (few tiles): 4 splits of 4
    # chunks; 6 splits, the last of 2 chunks and a ragged k tail; fp32, 4 splits
    (512, 1531, 64, 64, 4, 2, "bf16"),
    (1000, 2003, 32, 256, 16, 3, "bf16"),
    (520, 777, 16, 32, 2, 1, "f32"),
]


@pytest.mark.parametrize("d,V,Hs,r,P,B,dtype", CHAIN_SHAPES)
def test_chain_small_shapes(chain_mode, d, V, Hs, r, P, B, dtype):
    cfg = small_config(d=d, V=V, Hs=Hs, r=r, P=P, B=B, dtype=dtype, biases=True)
    say(f"case chain small mode={chain_mode} d={d} V={V} Hs={Hs} r={r} P={P} B={B} {dtype}")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    _, Lb, toks, L, status = _run(cfg, w, inp)
    assert status == 0
    m = oracle.Model.from_config(cfg, w)
    info = compare_chain(m, inp["H"], m.base_logits(inp["H"]), inp["t0"], toks, L, "small")
    say("  ", info)


def test_chain_zero_correction_is_base_argmax(chain_mode):
    cfg = small_config(d=64, V=2003, Hs=32, r=32, P=16, B=6, dtype="bf16", biases=False)
    say(f"case chain zero correction mode={chain_mode}")
    w = synth.make_weights(cfg)
    w["w2"] = np.zeros_like(w["w2"])
    inp = synth.make_inputs(cfg)
    _, Lb, toks, L, status = _run(cfg, w, inp)
    assert status == 0
    assert np.array_equal(L, Lb)
    assert np.array_equal(toks, np.argmax(Lb, axis=-1))


def test_chain_deterministic_and_prefix_stable():
    cfg = small_config(d=128, V=3001, Hs=64, r=64, P=16, B=7, dtype="bf16")
    say("case chain determinism / prefix")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    head, Lb, t1, L1, s1 = _run(cfg, w, inp)
    _, _, t2, L2, s2 = _run(cfg, w, inp, head=head)
    assert s1 == s2 == 0
    assert np.array_equal(t1, t2) and np.array_equal(L1, L2)
    cfg8 = cfg.with_(block=8)
    inp8 = {"H": np.ascontiguousarray(inp["H"][:, :8]), "t0": inp["t0"]}
    _, _, t8, L8, s8 = _run(cfg8, w, inp8)
    assert s8 == 0
    assert np.array_equal(t8, t1[:, :8]) and np.array_equal(L8, L1[:, :8])


# B <= 16 with bf16 weights keeps W2 on chip in mode 0; phase O takes 8
# sequences per MFMA row group (B 1, 8 | 9, 16 | 17 .. 32: 1, 2, 4 groups);
# every mode sums in the same order, so all three agree to the bit
@pytest.mark.parametrize("B,r", [(20, 32), (9, 32), (16, 256), (1, 256), (8, 256), (32, 64)])
def test_chain_modes_agree_bitwise(B, r):
    cfg = small_config(d=96, V=1501, Hs=48, r=r, P=12, B=B, dtype="bf16", biases=True)
    say(f"case chain modes agree B={B} r={r}")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    prev = dh.set_chain_mode(0)
    try:
        head, _, t0_, L0, s0 = _run(cfg, w, inp)
        dh.set_chain_mode(1)
        _, _, t1_, L1, s1 = _run(cfg, w, inp, head=head)
        dh.set_chain_mode(2)
        _, _, t2_, L2, s2 = _run(cfg, w, inp, head=head)
    finally:
        dh.set_chain_mode(prev)
    assert s0 == s1 == s2 == 0
    assert np.array_equal(t0_, t1_) and np.array_equal(L0, L1)
    assert np.array_equal(t0_, t2_) and np.array_equal(L0, L2)


# the H half split over k (B 1: 8 splits, B 3: 6, B 8: 2): the persistent
# schedule adds the splits once per launch, the stepwise one where it reads
# them, in the same order
@pytest.mark.parametrize("B", [1, 3, 8])
def test_chain_h_half_splits_agree_bitwise(B):
    cfg = small_config(d=1000, V=1501, Hs=48, r=256, P=16, B=B, dtype="bf16", biases=True)
    say(f"case chain H-half splits agree B={B}")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    prev = dh.set_chain_mode(0)
    try:
        head, _, t0_, L0, s0 = _run(cfg, w, inp)
        dh.set_chain_mode(1)
        _, _, t1_, L1, s1 = _run(cfg, w, inp, head=head)
        dh.set_chain_mode(2)
        _, _, t2_, L2, s2 = _run(cfg, w, inp, head=head)
    finally:
        dh.set_chain_mode(prev)
    assert s0 == s1 == s2 == 0
    assert np.array_equal(t0_, t1_) and np.array_equal(L0, L1)
    assert np.array_equal(t0_, t2_) and np.array_equal(L0, L2)
    m = oracle.Model.from_config(cfg, w)
    say("  ", compare_chain(m, inp["H"], m.base_logits(inp["H"]), inp["t0"], t0_, L0, "H-half splits"))


def test_chain_bad_first_token_flagged(chain_mode):
    cfg = small_config(d=32, V=101, Hs=16, r=16, P=4, B=3, dtype="bf16")
    say(f"case chain bad first token mode={chain_mode}")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    inp["t0"] = np.array([5, cfg.vocab + 7, -3], np.int32)
    head, _, toks, _, status = _run(cfg, w, inp, want_logits=False)
    assert status == dh.STATUS_BAD_FIRST_TOKEN
    # the flagged sequences were drafted from token 0: tokens as the oracle drafts them from there
    m = oracle.Model.from_config(cfg, w)
    compare_chain(m, inp["H"], m.base_logits(inp["H"]), np.array([5, 0, 0], np.int32), toks, None, "bad t0")
    # the checked binding call raises on the device status
    H, t0 = head.upload(inp["H"]), head.upload(inp["t0"])
    with pytest.raises(dh.DominoError) as ei:
        head.draft_chain(H, head.base_logits(H), t0, want_logits=False)
    assert ei.value.status == dh.ERR_FIRST_TOKEN


def test_chain_in_place_logits_and_guard_bytes():
    cfg = small_config(d=64, V=777, Hs=32, r=32, P=6, B=4, dtype="bf16")
    say("case chain in place + guards")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    H = head.upload(inp["H"])
    t0 = head.upload(inp["t0"])
    B, P, V = cfg.batch, cfg.block, cfg.vocab
    guard = 4096
    lb_buf = torch.full((guard + B * P * V + guard,), 7.5, dtype=torch.float32, device=head.device)
    tok_buf = torch.full((guard + B * P + guard,), -77, dtype=torch.int32, device=head.device)
    Lb = lb_buf[guard:guard + B * P * V].view(B, P, V)
    toks = tok_buf[guard:guard + B * P].view(B, P)
    head.base_logits(H, out=Lb)
    Lb_copy = Lb.clone()
    ws = head.workspace(B)
    toks_ref, L_ref, _ = head.draft_chain(H, Lb_copy, t0)
    head.draft_chain(H, Lb, t0, out_tokens=toks, out_logits=Lb, workspace=ws)  # in place
    torch.cuda.synchronize()
    assert torch.equal(Lb, L_ref) and torch.equal(toks, toks_ref)
    assert torch.all(lb_buf[:guard] == 7.5) and torch.all(lb_buf[-guard:] == 7.5)
    assert torch.all(tok_buf[:guard] == -77) and torch.all(tok_buf[-guard:] == -77)


def test_chain_on_side_stream():
    cfg = small_config(d=64, V=1001, Hs=32, r=32, P=8, B=3, dtype="bf16")
    say("case chain side stream")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    H = head.upload(inp["H"])
    t0 = head.upload(inp["t0"])
    ref_L = head.base_logits(H)
    ref_t, ref_logits, _ = head.draft_chain(H, ref_L, t0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Lb = head.base_logits(H, stream=s)
        toks, L, _ = head.draft_chain(H, Lb, t0, stream=s)
    s.synchronize()
    assert torch.equal(toks, ref_t) and torch.equal(L, ref_logits)


# logits: True writes the final logits (compared within 1e-3); False is the
# tokens-only launch, exactly the call and kernel that bench.py times
@pytest.mark.parametrize("key,sample,mode,logits", [
    ("qwen3_4b_b1", [0], 0, True), ("qwen3_4b_b1", [0], 1, True), ("qwen3_4b_b1", [0], 2, True),
    ("qwen3_4b_b1", [0], 0, False), ("qwen3_4b_b1", [0], 2, False),
    ("qwen3_4b_b32", [0, 13, 31], 0, True), ("qwen3_4b_b32", [0, 20, 31], 0, False),
    ("qwen3_8b_b16", [0, 15], 0, True), ("qwen3_8b_b16", [3, 9], 0, False), ("qwen3_8b_b16", [3], 2, True)])
def test_chain_full_size_sampled(key, sample, mode, logits):
    cfg = synth.CONFIGS[key]
    say(f"case chain full {key} mode={mode} logits={logits} sample={sample}")
    prev = dh.set_chain_mode(mode)
    try:
        head = device_head(key)
        inp = synth.make_inputs(cfg)
        H = head.upload(inp["H"])
        t0 = head.upload(inp["t0"])
        Lb = head.base_logits(H)
        toks, L, ws = head.draft_chain(H, Lb, t0, want_logits=logits)  # raises on a device status
        torch.cuda.synchronize()
    finally:
        dh.set_chain_mode(prev)
    w = weights_for(key)
    m = oracle.Model.from_config(cfg, w)
    Hs_ = np.ascontiguousarray(inp["H"][sample])
    Lb_ref = m.base_logits(Hs_)
    info = compare_chain(m, Hs_, Lb_ref, inp["t0"][sample], toks.cpu().numpy()[sample],
                         L.cpu().numpy()[sample] if logits else None, key)
    say("  ", info)
    t = toks.cpu().numpy()
    assert t.min() >= 0 and t.max() < cfg.vocab


# ---- exact ties and signed zeros across workgroups ----------------------------------
def _tie_case(V, zero_w2):
    """Hand-built base logits (the chain takes them as an input) with exact ties whose
    copies sit in the tile ranges of the first and of the last workgroups, and rows
    whose maximum is a signed zero.  With W2 != 0 the tied entries get identical W2
    rows, so their corrections are identical too."""
    cfg = small_config(d=64, V=V, Hs=32, r=32, P=5, B=4, dtype="bf16", biases=False)
    w = synth.make_weights(cfg)
    if zero_w2:
        w["w2"] = np.zeros_like(w["w2"])
    inp = synth.make_inputs(cfg)
    B, P = cfg.batch, cfg.block
    rng = np.random.default_rng(11)
    Lb = (rng.standard_normal((B, P, V)) * 0.5 - 3.0).astype(np.float32)
    lo, mid, hi = 5, V // 2 + 3, V - 3  # first workgroup's range, the middle, the last one's
    ties = {  # (b, p): entries holding the row's maximum
        (0, 0): [lo, hi], (0, 2): [mid, hi], (1, 1): [lo, mid, hi], (2, 3): [hi - 1, hi],
        (3, 0): [lo, lo + 1], (3, 4): [lo, hi],
    }
    for (b, p), idx in ties.items():
        Lb[b, p, idx] = 40.0
    zeros = {(1, 3): (lo + 2, -0.0, hi, 0.0), (2, 1): (lo + 2, 0.0, hi, -0.0), (3, 2): (mid, -0.0, hi - 2, 0.0)}
    for (b, p), (i, vi, j, vj) in zeros.items():
        Lb[b, p] = -np.abs(Lb[b, p]) - 1.0
        Lb[b, p, i] = vi
        Lb[b, p, j] = vj
    if not zero_w2:
        for idx in ties.values():
            for v in idx[1:]:
                w["w2"][v] = w["w2"][idx[0]]
    return cfg, w, inp, Lb, ties, zeros


@pytest.mark.parametrize("zero_w2", [True, False])
def test_chain_exact_ties_across_workgroups(chain_mode, zero_w2):
    V = 60013
    say(f"case chain ties mode={chain_mode} zero_w2={zero_w2}")
    cfg, w, inp, Lb, ties, zeros = _tie_case(V, zero_w2)
    head = dh.DraftHead.from_config(cfg, w)
    H, t0, Lbd = head.upload(inp["H"]), head.upload(inp["t0"]), head.upload(Lb)
    for logits in (True, False):
        toks, L, _ = head.draft_chain(H, Lbd, t0, want_logits=logits)
        g = toks.cpu().numpy()
        for (b, p), idx in ties.items():
            assert g[b, p] == min(idx), ((b, p), g[b, p], idx)
        if zero_w2:  # zero correction: L = L^base bitwise, both signed zeros count as the maximum
            for (b, p), (i, _, j, _) in zeros.items():
                assert g[b, p] == min(i, j), ((b, p), g[b, p])
            assert np.array_equal(g, np.argmax(Lb + np.float32(0.0), axis=-1))
            if logits:
                assert np.array_equal(L.cpu().numpy(), Lb)
        m = oracle.Model.from_config(cfg, w)
        compare_chain(m, inp["H"], Lb, inp["t0"], g, L.cpu().numpy() if logits else None, "ties")


# ---- the worked micro example, zero padded ---------------------------------------------
# V=4, d=2, Hs=1, r=1, P=2 (written out below); padded to d = Hs = r = 8 with
# zeros, which leaves every value unchanged: padded GRU units keep h = 0
# (h' = h/2 with all their weights zero), padded bottleneck units give SiLU(0) = 0.
MICRO_EXPECT = {  # t0 -> (tokens, logits at p=0, logits at p=1), closed forms of the definitions
    0: ([0, 1], [1, 0, 1, -1], [0, 1, 1, 0]),
    1: ([1, 1], [1, 1.2505490219, -0.2505490219, -1], [0, 3.0736888186, -1.0736888186, 0]),
    2: ([2, 2], [1, -0.2447974530, 1.2447974530, -1], [0, 0.8480316599, 1.1519683401, 0]),
    3: ([2, 2], [1, -0.2726392900, 1.2726392900, -1], [0, 0.8289735483, 1.1710264517, 0]),
}


def _micro_weights(dtype):
    d = Hs = r = 8
    V = 4
    f = np.float32
    lm = np.zeros((V, d), f)
    lm[:, :2] = [[1, 0], [0, 1], [1, 1], [-1, 0]]
    E = np.zeros((V, d), f)
    E[:, :2] = [[0, 0], [1, 0], [0, 1], [1, 1]]
    w_ih = np.zeros((3 * Hs, d), f)
    w_ih[2 * Hs + 0, :2] = [1, -2]          # only the n gate of unit 0 reads x
    w_hh = np.zeros((3 * Hs, Hs), f)
    w1 = np.zeros((r, d + Hs), f)
    w1[0, d + 0] = 4.0                       # bottleneck unit 0 reads state unit 0
    w2 = np.zeros((V, r), f)
    w2[:, 0] = [0, 1, -1, 0]
    w = {"lm_head": lm, "embed": E, "w_ih": w_ih, "w_hh": w_hh, "w1": w1, "w2": w2}
    if dtype == "bf16":  # every value above is exact in bf16
        w = {k: (v.view(np.uint32) >> 16).astype(np.uint16) for k, v in w.items()}
    H = np.zeros((4, 2, d), f)
    H[:, 0, 0] = 1.0
    H[:, 1, 1] = 1.0
    if dtype == "bf16":
        H = (H.view(np.uint32) >> 16).astype(np.uint16)
    return w, H


@pytest.mark.parametrize("dtype,tol", [("f32", 1e-6), ("bf16", 2e-5)])
def test_chain_micro_example(chain_mode, dtype, tol):
    """All four anchors at once (one sequence each).  fp32 weights: logits within 1e-6 of the
    closed forms.  bf16: the fp32 activations meet the weights as bf16 hi + lo, which keeps
    them to 2^-17 relative, so the bound is 2e-5 at these magnitudes."""
    say(f"case chain micro example mode={chain_mode} {dtype}")
    w, H = _micro_weights(dtype)
    head = dh.DraftHead(8, 4, 8, 8, 2, dtype, w)
    Hd = head.upload(H)
    t0 = head.upload(np.arange(4, dtype=np.int32))
    Lb = head.base_logits(Hd)
    assert np.array_equal(Lb.cpu().numpy()[0], np.array([[1, 0, 1, -1], [0, 1, 1, 0]], np.float32))
    for logits in (True, False):
        toks, L, _ = head.draft_chain(Hd, Lb, t0, want_logits=logits)
        g = toks.cpu().numpy()
        for t in range(4):
            exp_tok, l0, l1 = MICRO_EXPECT[t]
            assert g[t].tolist() == exp_tok, (t, g[t])
            if logits:
                Lt = L.cpu().numpy()[t].astype(np.float64)
                assert np.max(np.abs(Lt - np.array([l0, l1]))) <= tol, (t, Lt)


def test_timing_events_bracket_main_launches():
    cfg = small_config(d=64, V=1001, Hs=32, r=32, P=8, B=3, dtype="bf16")
    say("case timing events")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    H = head.upload(inp["H"])
    t0 = head.upload(inp["t0"])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    dh.domino_set_timing_events(*ev)
    try:
        Lb = head.base_logits(H)
        toks, L, ws = head.draft_chain(H, Lb, t0)
        torch.cuda.synchronize()
    finally:
        dh.domino_set_timing_events()
    assert ev[0].elapsed_time(ev[1]) > 0 and ev[2].elapsed_time(ev[3]) > 0
    assert ev[1].elapsed_time(ev[2]) >= 0  # the chain's main launch follows the GEMM
    Lb2 = head.base_logits(H)
    toks2, L2, _ = head.draft_chain(H, Lb2, t0)
    torch.cuda.synchronize()
    assert torch.equal(toks, toks2) and torch.equal(L, L2)
