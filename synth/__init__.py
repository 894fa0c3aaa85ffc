"""Seeded synthetic inputs for the Domino draft-head path.

This module draws numbers and nothing else: it holds none of the draft
head's arithmetic.  The oracle tests, the GPU parity tests and the bench
all take their inputs from here, so both sides of a comparison consume
identical bits.  The generator itself (SplitMix64 counters + Box-Muller)
is defined in ``synth.c``.

Shapes follow the Domino head as the pages describe it (Domino paper
summary, "Methodologie: Domino" / "Domino-head"; news explainer section 4):
a 16-position draft block, a GRU causal encoder of width 1024, a rank-256
bottleneck, and the Qwen3-4B / Qwen3-8B hidden and vocabulary sizes.

bf16 tensors are returned as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# tensor ids of the counter-based generator
TID_H, TID_WLM, TID_E, TID_WIH, TID_WHH, TID_W1, TID_W2, TID_T0 = 1, 2, 3, 4, 5, 6, 7, 8
TID_BIH, TID_BHH, TID_B1, TID_B2 = 9, 10, 11, 12


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_LIB_PATH)
        u64, p = ctypes.c_uint64, ctypes.c_void_p
        lib.synth_raw_u64.argtypes = [u64, u64, u64, p]
        lib.synth_normal_f32.argtypes = [u64, u64, u64, ctypes.c_double, p]
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, ctypes.c_double, p]
        lib.synth_uniform_int.argtypes = [u64, u64, u64, u64, p]
        for f in (lib.synth_raw_u64, lib.synth_normal_f32, lib.synth_normal_bf16, lib.synth_uniform_int):
            f.restype = None
        _lib = lib
    return _lib


def raw_u64(n: int, seed: int, tensor_id: int) -> np.ndarray:
    out = np.empty(int(n), dtype=np.uint64)
    _load().synth_raw_u64(seed, tensor_id, out.size, out.ctypes.data)
    return out


def normal(shape, std: float, seed: int, tensor_id: int, dtype: str = "f32") -> np.ndarray:
    """N(0, std^2) draws, fp32 values or bf16 bit patterns (uint16)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    if dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
        _load().synth_normal_f32(seed, tensor_id, n, float(std), out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(shape, dtype=np.uint16)
        _load().synth_normal_bf16(seed, tensor_id, n, float(std), out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out


def uniform_int(n: int, bound: int, seed: int, tensor_id: int) -> np.ndarray:
    out = np.empty(int(n), dtype=np.int32)
    _load().synth_uniform_int(seed, tensor_id, out.size, int(bound), out.ctypes.data)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Config:
    """One synthetic workload: shapes, seeds and the std of every tensor."""
    name: str
    hidden: int          # d
    vocab: int           # V
    gru_hidden: int      # Hs
    rank: int            # r
    block: int           # P, positions per draft block
    batch: int           # B, independent sequences
    dtype: str           # storage type of H and of every weight: "f32" or "bf16"
    weight_seed: int
    input_seed: int
    std_lm: float = 0.02
    std_embed: float = 0.02
    std_h: float = 1.0
    scale_whh: float = 1.0
    biases: bool = False
    nodes: int = 16      # tree budget
    topm: int = 64       # tree candidates per depth
    tree: bool = False   # best-first tree instead of the chain
    extra: dict = field(default_factory=dict)

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)

    # fan-in reading: N(0, 1/fan_in) is a variance, fan_in = stored row length
    @property
    def std_wih(self):
        return 1.0 / math.sqrt(self.hidden)

    @property
    def std_whh(self):
        return self.scale_whh / math.sqrt(self.gru_hidden)

    @property
    def std_w1(self):
        return 1.0 / math.sqrt(self.hidden + self.gru_hidden)

    @property
    def std_w2(self):
        return 1.0 / math.sqrt(self.rank)


CONFIGS = {
    # tiny fp32 chain: every weight N(0, 1/fan_in)
    "tiny_f32": Config("tiny_f32", 256, 4096, 128, 32, 16, 1, "f32", 1, 1,
                       std_lm=1 / 16, std_embed=1 / 16),
    # Qwen3-4B shapes, one sequence
    "qwen3_4b_b1": Config("qwen3_4b_b1", 2560, 151936, 1024, 256, 16, 1, "bf16", 4, 101),
    # Qwen3-4B shapes, 32 concurrent sequences sharing each W2 read
    "qwen3_4b_b32": Config("qwen3_4b_b32", 2560, 151936, 1024, 256, 16, 32, "bf16", 4, 102),
    # Qwen3-8B shapes, 16 sequences
    "qwen3_8b_b16": Config("qwen3_8b_b16", 4096, 151936, 1024, 256, 16, 16, "bf16", 8, 103),
    # best-first tree on Qwen3-4B shapes: 8 sequences, 16 nodes, top-64
    "qwen3_4b_tree": Config("qwen3_4b_tree", 2560, 151936, 1024, 256, 16, 8, "bf16", 4, 104,
                            nodes=16, topm=64, tree=True),
}


def make_weights(cfg: Config) -> dict:
    """All head and LM-head weights of ``cfg`` as host arrays ([out][in] row-major)."""
    d, V, Hs, r, dt, s = cfg.hidden, cfg.vocab, cfg.gru_hidden, cfg.rank, cfg.dtype, cfg.weight_seed
    w = {
        "lm_head": normal((V, d), cfg.std_lm, s, TID_WLM, dt),
        "embed": normal((V, d), cfg.std_embed, s, TID_E, dt),
        "w_ih": normal((3 * Hs, d), cfg.std_wih, s, TID_WIH, dt),
        "w_hh": normal((3 * Hs, Hs), cfg.std_whh, s, TID_WHH, dt),
        "w1": normal((r, d + Hs), cfg.std_w1, s, TID_W1, dt),
        "w2": normal((V, r), cfg.std_w2, s, TID_W2, dt),
        "b_ih": None, "b_hh": None, "b1": None, "b2": None,
    }
    if cfg.biases:
        w["b_ih"] = normal((3 * Hs,), 0.1, s, TID_BIH, "f32")
        w["b_hh"] = normal((3 * Hs,), 0.1, s, TID_BHH, "f32")
        w["b1"] = normal((r,), 0.1, s, TID_B1, "f32")
        w["b2"] = normal((V,), 0.1, s, TID_B2, "f32")
    return w


def make_inputs(cfg: Config, batch: int | None = None) -> dict:
    """Backbone hidden states H[B][P][d] and the anchor tokens t0[B]."""
    B = cfg.batch if batch is None else batch
    return {
        "H": normal((B, cfg.block, cfg.hidden), cfg.std_h, cfg.input_seed, TID_H, cfg.dtype),
        "t0": uniform_int(B, cfg.vocab, cfg.input_seed, TID_T0),
    }
