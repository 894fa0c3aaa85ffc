"""Shared test helpers: small synthetic models and comparison rules."""
from __future__ import annotations

import numpy as np

import synth


def small_config(name="small", d=16, V=37, Hs=8, r=8, P=5, B=2, dtype="f32", biases=True, wseed=7, iseed=9,
                 std_lm=0.5, std_embed=1.0, scale_whh=3.0):
    """A tiny model with enough signal that token feedback changes the logits."""
    return synth.Config(name, d, V, Hs, r, P, B, dtype, wseed, iseed, std_lm=std_lm, std_embed=std_embed,
                        scale_whh=scale_whh, biases=biases)


def widen(a, dtype):
    """Stored array -> float64 values."""
    if dtype == "bf16":
        return synth.bf16_to_f32(np.asarray(a)).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def row_rel_err(gpu, ref):
    """Per-row error max_v |g - o| / max(|o_v|, rms_v(o)); rows along the last axis."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    denom = np.maximum(np.abs(ref), rms)
    denom = np.where(denom == 0, 1.0, denom)
    return np.max(np.abs(gpu - ref) / denom, axis=-1)
