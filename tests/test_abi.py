"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

import draft_head_amd as dh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "domino.h")
BENCH_HEADER = os.path.join(ROOT, "include", "domino_bench.h")


def declared_functions(path=HEADER):
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(domino_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_contract_calls():
    names = declared_functions()
    # the calls of the boundary: the three operations, workspace sizing,
    # error reporting and cache release
    for n in ("domino_base_logits", "domino_draft_chain", "domino_tree_draft", "domino_workspace_size",
              "domino_last_error", "domino_release_cache", "domino_device_status"):
        assert n in names
    # process-wide hooks stay out of the contract header
    for n in ("domino_set_chain_mode", "domino_set_timing_events"):
        assert n not in names and n in declared_functions(BENCH_HEADER)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(dh.LIB_PATH)
    declared = declared_functions()
    bench = declared_functions(BENCH_HEADER)
    missing = [n for n in declared + bench if not hasattr(lib, n)]
    assert not missing, missing
    assert set(dh.EXPORTS) == set(declared)
    assert set(dh.BENCH_EXPORTS) == set(bench)


def test_status_codes_are_negative():
    src = open(HEADER).read()
    vals = dict((k, int(v)) for k, v in re.findall(r"(DOMINO_(?:OK|ERR_[A-Z_]+))\s*=\s*(-?\d+)", src))
    assert vals["DOMINO_OK"] == 0
    assert all(v < 0 for k, v in vals.items() if k != "DOMINO_OK")
    assert (dh.ERR_INVALID_ARGUMENT, dh.ERR_UNSUPPORTED, dh.ERR_WORKSPACE, dh.ERR_DEVICE, dh.ERR_TIMEOUT,
            dh.ERR_FIRST_TOKEN) == tuple(vals[k] for k in (
                "DOMINO_ERR_INVALID_ARGUMENT", "DOMINO_ERR_UNSUPPORTED", "DOMINO_ERR_WORKSPACE", "DOMINO_ERR_DEVICE",
                "DOMINO_ERR_TIMEOUT", "DOMINO_ERR_FIRST_TOKEN"))


def test_version_and_empty_error():
    assert dh.version().startswith("domino-gfx950")


def _dims(**kw):
    base = dict(hidden=2560, vocab=151936, gru_hidden=1024, rank=256, block=16, dtype="bf16")
    base.update(kw)
    return dh.make_dims(**base)


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation or is a no-op


def _weights(**kw):
    w = {k: FAKE for k in ("lm_head", "embed", "w_ih", "w_hh", "w1", "w2")}
    w.update(kw)
    return dh.Weights(**w)


@pytest.mark.parametrize("kw,msg", [
    (dict(hidden=0), "hidden"), (dict(hidden=12), "hidden"), (dict(gru_hidden=-8), "gru_hidden"),
    (dict(rank=7), "rank"), (dict(vocab=0), "vocab"), (dict(block=0), "block"), (dict(block=65), "block"),
    (dict(dtype=5), "dtype"),
])
def test_bad_dims_rejected(kw, msg):
    L = dh.lib()
    st = L.domino_base_logits(ctypes.byref(_dims(**kw)), ctypes.byref(_weights()), FAKE, 1, FAKE, None)
    assert st == dh.ERR_INVALID_ARGUMENT
    assert msg in dh.last_error()


def test_rank_above_256_unsupported():
    L = dh.lib()
    st = L.domino_base_logits(ctypes.byref(_dims(rank=264)), ctypes.byref(_weights()), FAKE, 1, FAKE, None)
    assert st == dh.ERR_UNSUPPORTED


def test_null_and_misaligned_pointers_rejected():
    L = dh.lib()
    d = _dims()
    assert L.domino_base_logits(ctypes.byref(d), ctypes.byref(_weights()), None, 1, FAKE, None) == \
        dh.ERR_INVALID_ARGUMENT
    assert "H is NULL" in dh.last_error()
    assert L.domino_base_logits(ctypes.byref(d), ctypes.byref(_weights(lm_head=FAKE + 8)), FAKE, 1, FAKE,
                                None) == dh.ERR_INVALID_ARGUMENT
    assert "aligned" in dh.last_error()
    assert L.domino_base_logits(None, ctypes.byref(_weights()), FAKE, 1, FAKE, None) == dh.ERR_INVALID_ARGUMENT
    assert L.domino_base_logits(ctypes.byref(d), None, FAKE, 1, FAKE, None) == dh.ERR_INVALID_ARGUMENT
    ws = dh.domino_workspace_size(d, 4, dh.OP_CHAIN)
    # every call below is short of workspace or has one bad argument, so none reaches a launch
    args = (ctypes.byref(d), ctypes.byref(_weights()), FAKE, FAKE, FAKE, 4, FAKE, None, FAKE, ws - 1, None)
    assert L.domino_draft_chain(*args) == dh.ERR_WORKSPACE
    for i, name in ((2, "H"), (3, "base_logits"), (4, "first_tokens"), (6, "out_tokens"), (8, "workspace")):
        bad = list(args)
        bad[i] = None
        bad[9] = 1 << 40
        assert L.domino_draft_chain(*bad) == dh.ERR_INVALID_ARGUMENT, name
        assert name in dh.last_error()
    bad = list(args)
    bad[7], bad[9] = FAKE + 4, 1 << 40
    assert L.domino_draft_chain(*bad) == dh.ERR_INVALID_ARGUMENT
    assert "out_logits" in dh.last_error()
    for wname in ("embed", "w_ih", "w_hh", "w1", "w2"):
        bad = list(args)
        bad[1] = ctypes.byref(_weights(**{wname: None}))
        bad[9] = 1 << 40
        assert L.domino_draft_chain(*bad) == dh.ERR_INVALID_ARGUMENT
        assert wname in dh.last_error()


def test_workspace_too_small():
    L = dh.lib()
    d = _dims()
    need = dh.domino_workspace_size(d, 8, dh.OP_CHAIN)
    st = L.domino_draft_chain(ctypes.byref(d), ctypes.byref(_weights()), FAKE, FAKE, FAKE, 8, FAKE, None, FAKE,
                              need - 1, None)
    assert st == dh.ERR_WORKSPACE
    assert str(need) in dh.last_error()


def test_negative_and_zero_batch():
    L = dh.lib()
    d = _dims()
    assert L.domino_base_logits(ctypes.byref(d), ctypes.byref(_weights()), FAKE, -1, FAKE, None) == \
        dh.ERR_INVALID_ARGUMENT
    # batch 0 is a no-op: returns OK without touching memory or the device
    assert L.domino_base_logits(ctypes.byref(d), ctypes.byref(_weights()), None, 0, None, None) == dh.OK
    assert L.domino_draft_chain(ctypes.byref(d), ctypes.byref(_weights()), None, None, None, 0, None, None, None, 0,
                                None) == dh.OK


def test_workspace_size_grows_then_saturates():
    d = _dims()
    s = [dh.domino_workspace_size(d, b, dh.OP_CHAIN) for b in (1, 2, 16, 32, 33, 1000)]
    assert s[0] < s[1] < s[2] < s[3]
    assert s[3] == s[4] == s[5]  # sequences run in groups of at most 32
    assert dh.domino_workspace_size(_dims(hidden=3), 1, dh.OP_CHAIN) == 0
    assert "hidden" in dh.last_error()


def test_workspace_size_by_op():
    d = _dims()
    assert dh.domino_workspace_size(d, 8, dh.OP_BASE) == 0
    assert dh.domino_workspace_size(d, 8, dh.OP_TREE, 16, 64) > 0
    assert dh.domino_workspace_size(d, 8, dh.OP_CANDIDATES, 0, 64) > 0
    assert dh.domino_workspace_size(d, 8, 9) == 0
    assert "op" in dh.last_error()
    assert dh.domino_workspace_size(d, -1, dh.OP_CHAIN) == 0
    assert "batch" in dh.last_error()
    # the step clocks sit inside the chain workspace
    off = dh.domino_chain_stamp_offset(d, 8)
    assert 0 < off and off + (d.block + 1) * 8 <= dh.domino_workspace_size(d, 8, dh.OP_CHAIN)


def test_device_status_and_release_without_launch():
    L = dh.lib()
    assert L.domino_device_status(None, None) == dh.ERR_INVALID_ARGUMENT
    assert L.domino_device_status(FAKE + 4, None) == dh.ERR_INVALID_ARGUMENT
    dh.domino_release_cache()  # nothing cached yet: a no-op that needs no device


def test_chain_mode_switch():
    prev = dh.set_chain_mode(1)
    assert dh.set_chain_mode(2) == 1
    assert dh.set_chain_mode(prev) == 2
    for bad in (7, 4, -1):
        with pytest.raises(ValueError):
            dh.set_chain_mode(bad)


def test_tree_arguments_rejected_before_launch():
    L = dh.lib()
    d = _dims()
    ws = dh.domino_workspace_size(d, 8, dh.OP_TREE, 16, 64)
    assert ws > 0
    assert dh.domino_workspace_size(d, 8, dh.OP_TREE, 0, 64) == 0
    assert dh.domino_workspace_size(d, 8, dh.OP_TREE, 65, 64) == 0
    assert dh.domino_workspace_size(d, 8, dh.OP_TREE, 16, 257) == 0
    good = dict(dims=ctypes.byref(d), w=ctypes.byref(_weights()), H=FAKE, Lb=FAKE, t0=FAKE, B=8, N=16, M=64,
                par=FAKE, tok=FAKE, dep=None, sc=None, ws=FAKE, wsb=ws - 1, s=None)

    def call(**kw):
        a = dict(good)
        a.update(kw)
        return L.domino_tree_draft(*a.values())

    assert call() == dh.ERR_WORKSPACE  # one byte short: still no launch
    for kw, msg in ((dict(N=0), "nodes"), (dict(N=65), "nodes"), (dict(M=0), "topm"), (dict(M=300), "topm"),
                    (dict(par=None, wsb=1 << 40), "out_parents"), (dict(tok=None, wsb=1 << 40), "out_tokens"),
                    (dict(sc=FAKE + 8, wsb=1 << 40), "out_scores"), (dict(H=None, wsb=1 << 40), "H")):
        assert call(**kw) == dh.ERR_INVALID_ARGUMENT, kw
        assert msg in dh.last_error()
    small_v = _dims(vocab=50)
    assert call(dims=ctypes.byref(small_v), M=64, wsb=1 << 40) == dh.ERR_INVALID_ARGUMENT
    assert "vocabulary" in dh.last_error()
    cw = dh.domino_workspace_size(d, 2, dh.OP_CANDIDATES, 0, 8)
    assert cw > 0
    assert L.domino_tree_candidates(ctypes.byref(d), FAKE, 2, 0, FAKE, FAKE, FAKE, cw, None) == dh.ERR_INVALID_ARGUMENT
    assert L.domino_tree_candidates(ctypes.byref(d), None, 2, 8, FAKE, FAKE, FAKE, cw, None) == dh.ERR_INVALID_ARGUMENT
    assert L.domino_tree_candidates(ctypes.byref(d), FAKE, 2, 8, FAKE, FAKE, FAKE, cw - 1, None) == dh.ERR_WORKSPACE
    assert L.domino_tree_candidates(ctypes.byref(d), FAKE, 0, 8, None, None, None, 0, None) == dh.OK
    # fp32 weights: the GRU step stages eight states and embedding rows in LDS,
    # which these sizes overflow (the bf16 step stages nothing)
    big = _dims(hidden=8192, gru_hidden=2048, dtype="f32")
    assert call(dims=ctypes.byref(big), wsb=1 << 40) == dh.ERR_UNSUPPORTED


def test_verify_inputs_rejected_before_launch():
    L = dh.lib()
    a = [FAKE, FAKE, FAKE, None, 4, 16, FAKE, FAKE, FAKE, None]
    for i, v, msg in ((5, 0, "nodes"), (5, 65, "nodes"), (4, -1, "batch"), (0, None, "parents"),
                      (6, None, "out_mask"), (3, FAKE + 4, "start_positions")):
        bad = list(a)
        bad[i] = v
        assert L.domino_tree_verify_inputs(*bad) == dh.ERR_INVALID_ARGUMENT, msg
        assert msg in dh.last_error()
    bad = list(a)
    bad[4] = 0
    assert L.domino_tree_verify_inputs(*bad) == dh.OK  # an empty batch launches nothing


def test_input_table_arguments_rejected():
    L = dh.lib()
    d = _dims()
    # the table call: every bad argument is caught before a launch
    assert L.domino_prepare_input_table(ctypes.byref(d), ctypes.byref(_weights()), None, None) == \
        dh.ERR_INVALID_ARGUMENT
    assert "table is NULL" in dh.last_error()
    assert L.domino_prepare_input_table(ctypes.byref(d), ctypes.byref(_weights()), FAKE + 4, None) == \
        dh.ERR_INVALID_ARGUMENT
    assert "aligned" in dh.last_error()
    for wname in ("embed", "w_ih"):
        assert L.domino_prepare_input_table(ctypes.byref(d), ctypes.byref(_weights(**{wname: None})), FAKE,
                                            None) == dh.ERR_INVALID_ARGUMENT
        assert wname in dh.last_error()
    assert L.domino_prepare_input_table(ctypes.byref(_dims(hidden=12)), ctypes.byref(_weights()), FAKE, None) == \
        dh.ERR_INVALID_ARGUMENT
    # a misaligned table passed to the chain is rejected too
    ws = dh.domino_workspace_size(d, 4, dh.OP_CHAIN)
    st = L.domino_draft_chain(ctypes.byref(d), ctypes.byref(_weights(input_table=FAKE + 8)), FAKE, FAKE, FAKE, 4,
                              FAKE, None, FAKE, ws, None)
    assert st == dh.ERR_INVALID_ARGUMENT
    assert "input_table" in dh.last_error()


def test_input_table_f64_arguments_rejected():
    L = dh.lib()
    d = _dims()
    assert L.domino_prepare_input_table_f64(ctypes.byref(d), ctypes.byref(_weights()), None, None) == \
        dh.ERR_INVALID_ARGUMENT
    assert "table is NULL" in dh.last_error()
    for wname in ("embed", "w_ih"):
        assert L.domino_prepare_input_table_f64(ctypes.byref(d), ctypes.byref(_weights(**{wname: None})), FAKE,
                                                None) == dh.ERR_INVALID_ARGUMENT
        assert wname in dh.last_error()
    # a misaligned fp64 table passed to the tree is rejected
    ws = dh.domino_workspace_size(d, 2, dh.OP_TREE, 16, 64)
    st = L.domino_tree_draft(ctypes.byref(d), ctypes.byref(_weights(input_table_f64=FAKE + 8)), FAKE, FAKE, FAKE, 2,
                             16, 64, FAKE, FAKE, None, None, FAKE, ws, None)
    assert st == dh.ERR_INVALID_ARGUMENT
    assert "input_table_f64" in dh.last_error()
