"""The allocation-free chain entry point (domino_draft_chain_noalloc) against
domino_draft_chain: the same kernels on a static workspace, so tokens and
logits must agree to the bit; two calls in a row, the second smaller, so the
static workspace is reused at a different layout."""
import ctypes

import numpy as np
import pytest
import torch

import draft_head_amd as dh
import synth
from gpu_common import say
from helpers import small_config

pytestmark = pytest.mark.gpu


def _reference(head, H, Lb, t0):
    toks, L, _ = head.draft_chain(H, Lb, t0)  # its own fresh workspace
    return toks, L


def _noalloc(head, H, Lb, t0):
    B, P, V = H.shape[0], head.dims.block, head.dims.vocab
    toks = torch.full((B, P), -5, dtype=torch.int32, device=head.device)
    L = torch.full((B, P, V), 7.0, dtype=torch.float32, device=head.device)
    dh.domino_draft_chain_noalloc(head.dims, head.weights, H, Lb, t0, B, toks, L)
    dh.domino_noalloc_device_status()  # raises on a device-side status
    return toks, L


@pytest.mark.parametrize("mode", [0, 1])
def test_noalloc_matches_workspace_call_twice(mode):
    assert torch.cuda.is_available()
    prev = dh.set_chain_mode(mode)
    try:
        for d, V, Hs, r, P, B in ((96, 5003, 64, 64, 8, 6), (96, 5003, 64, 64, 8, 3), (64, 2051, 32, 32, 5, 2)):
            say(f"case no-alloc mode={mode} d={d} V={V} Hs={Hs} r={r} P={P} B={B}")
            cfg = small_config(d=d, V=V, Hs=Hs, r=r, P=P, B=B, dtype="bf16", biases=True)
            w = synth.make_weights(cfg)
            inp = synth.make_inputs(cfg)
            head = dh.DraftHead.from_config(cfg, w)
            H, t0 = head.upload(inp["H"]), head.upload(inp["t0"])
            Lb = head.base_logits(H)
            t_ref, L_ref = _reference(head, H, Lb, t0)
            t_na, L_na = _noalloc(head, H, Lb, t0)
            torch.cuda.synchronize()
            assert torch.equal(t_na, t_ref) and torch.equal(L_na, L_ref)
    finally:
        dh.set_chain_mode(prev)


def test_noalloc_tokens_only_and_bad_first_token():
    cfg = small_config(d=64, V=3001, Hs=32, r=32, P=6, B=4, dtype="bf16", biases=True)
    say("case no-alloc tokens only / bad first token")
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg)
    head = dh.DraftHead.from_config(cfg, w)
    H, t0 = head.upload(inp["H"]), head.upload(inp["t0"])
    Lb = head.base_logits(H)
    t_ref, _, _ = head.draft_chain(H, Lb, t0, want_logits=False)
    toks = torch.empty_like(t_ref)
    dh.domino_draft_chain_noalloc(head.dims, head.weights, H, Lb, t0, 4, toks, None)
    dh.domino_noalloc_device_status()
    assert torch.equal(toks, t_ref)
    bad = t0.clone()
    bad[1] = cfg.vocab + 3
    dh.domino_draft_chain_noalloc(head.dims, head.weights, H, Lb, bad, 4, toks, None)
    with pytest.raises(dh.DominoError) as ei:
        dh.domino_noalloc_device_status()
    assert ei.value.status == dh.ERR_FIRST_TOKEN
    # the next call starts from a clean status word
    dh.domino_draft_chain_noalloc(head.dims, head.weights, H, Lb, t0, 4, toks, None)
    dh.domino_noalloc_device_status()
    assert torch.equal(toks, t_ref)


def test_noalloc_rejects_what_does_not_fit():
    L = dh.lib()
    d = dh.make_dims(4096, 151936, 4096, 256, 64, "bf16")
    assert dh.domino_workspace_size(d, 32, dh.OP_CHAIN) > 32 << 20
    fake = 0x10000
    w = dh.Weights(**{k: fake for k in ("lm_head", "embed", "w_ih", "w_hh", "w1", "w2")})
    st = L.domino_draft_chain_noalloc(ctypes.byref(d), ctypes.byref(w), fake, fake, fake, 32, fake, None, None)
    assert st == dh.ERR_UNSUPPORTED
    assert "32" in dh.last_error() or "bytes" in dh.last_error()
