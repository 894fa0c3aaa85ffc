"""Shared pieces of the GPU tests: device model cache and comparison rules."""
from __future__ import annotations

import functools
import sys

import numpy as np

import oracle
import synth
from helpers import row_rel_err

LOGIT_TOL = 1e-3      # max row-relative error of logits against the oracle
MARGIN_FIRM = 1e-2    # tokens must agree where the oracle's top-2 margin exceeds this


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=2)
def weights_for(cfg_key):
    cfg = synth.CONFIGS[cfg_key] if isinstance(cfg_key, str) else cfg_key
    return synth.make_weights(cfg)


def gemm_bound(Hd, Wd):
    """A-priori bound of an fp32-accumulated dot product: gamma_K * sum |h w| (u = 2^-24).
    Hd [M][K], Wd [N][K] float64 -> [M][N]."""
    K = Hd.shape[-1]
    u = 2.0 ** -24
    gamma = 2 * K * u / (1 - 2 * K * u)  # two roundings per term leave room for fp32 products too
    return gamma * (np.abs(Hd) @ np.abs(Wd).T) + 1e-30


def compare_chain(m: oracle.Model, H, Lb_ref, t0, g_tokens, g_logits, label=""):
    """Check GPU chain outputs against the oracle.

    The oracle is run with the GPU's own drafted tokens as the fed-back prefix
    (forced prefix), so every position is compared under the same history:
    logits within LOGIT_TOL row-relative, and the GPU token must equal the
    oracle argmax wherever that position's margin exceeds MARGIN_FIRM.  The
    free-running oracle must agree with the GPU up to its first near tie.
    Returns a dict of diagnostics.
    """
    g_tokens = np.asarray(g_tokens)
    f_t, f_L, f_m = m.chain(H, Lb_ref, t0, forced=g_tokens, want_logits=g_logits is not None)
    r_t, _, r_m = m.chain(H, Lb_ref, t0, want_logits=False)
    firm = f_m > MARGIN_FIRM
    bad = firm & (g_tokens != f_t)
    assert not bad.any(), f"{label}: token mismatch at firm positions {np.argwhere(bad)[:5].tolist()}"
    for b in range(g_tokens.shape[0]):
        diff = np.nonzero(g_tokens[b] != r_t[b])[0]
        if diff.size:
            p = diff[0]
            assert r_m[b, p] <= MARGIN_FIRM, f"{label}: seq {b} leaves the free oracle run at a firm position {p}"
    err = None
    if g_logits is not None:
        err = row_rel_err(g_logits, f_L)
        assert err.max() <= LOGIT_TOL, f"{label}: logit error {err.max():.3e}"
    return {"max_logit_err": None if err is None else float(err.max()), "near_ties": int((~firm).sum()),
            "diverged": int((g_tokens != r_t).any(axis=1).sum())}
