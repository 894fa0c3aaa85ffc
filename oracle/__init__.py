"""ctypes wrapper of the oracle (``oracle.c``).  TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg
may import this package; the product path never does.  It shares no code
with the GPU path: it marshals numpy arrays into the C oracle and back.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("hidden", "vocab", "gru_hidden", "rank", "block", "dtype")]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("lm_head", "embed", "w_ih", "w_hh", "b_ih", "b_hh", "w1", "b1", "w2", "b2")]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, f64 = ctypes.c_int32, ctypes.c_double
        sig = {
            "oracle_num_threads": ([], ctypes.c_int),
            "oracle_sigmoid": ([f64], f64),
            "oracle_silu": ([f64], f64),
            "oracle_base_logits": ([P, P, P, i32, P], None),
            "oracle_gru_cell": ([P, P, P, P, P], None),
            "oracle_head_bottleneck": ([P, P, P, P, P], None),
            "oracle_final_logits": ([P, P, P, P, P], None),
            "oracle_argmax": ([P, i32, P], i32),
            "oracle_chain": ([P, P, i32, P, P, P, P, P, P, P], None),
            "oracle_topm": ([P, i32, i32, P, P], None),
            "oracle_tree": ([P, P, i32, P, P, P, i32, i32, P, P, P, P], None),
            "oracle_philox4x32_10": ([P, P, P], None),
            "oracle_gumbel": ([ctypes.c_uint64, i32, i32, i32], f64),
            "oracle_chain_sampled": ([P, P, i32, i32, P, P, P, P, f64, ctypes.c_uint64, P, P, P], None),
            "oracle_tree_verify_inputs": ([i32, i32, P, P, P, P, P, P, P], None),
        }
        for name, (args, res) in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_code(dtype: str) -> int:
    return {"f32": F32, "bf16": BF16}[dtype]


class Model:
    """Dims + host weights as the oracle sees them (arrays kept alive here)."""

    def __init__(self, hidden, vocab, gru_hidden, rank, block, dtype, weights: dict):
        self.dims = Dims(hidden, vocab, gru_hidden, rank, block, _dtype_code(dtype))
        self.dtype = dtype
        store = np.float32 if dtype == "f32" else np.uint16
        self._keep = {}
        vals = {}
        for k in ("lm_head", "embed", "w_ih", "w_hh", "w1", "w2"):
            a = np.ascontiguousarray(weights[k], dtype=store)
            self._keep[k] = a
            vals[k] = a.ctypes.data
        for k in ("b_ih", "b_hh", "b1", "b2"):
            a = weights.get(k)
            if a is not None:
                a = np.ascontiguousarray(a, dtype=np.float32)
                self._keep[k] = a
                vals[k] = a.ctypes.data
            else:
                vals[k] = None
        self.weights = Weights(**vals)

    @classmethod
    def from_config(cls, cfg, weights: dict, block: int | None = None):
        return cls(cfg.hidden, cfg.vocab, cfg.gru_hidden, cfg.rank, cfg.block if block is None else block,
                   cfg.dtype, weights)

    def _store(self, a):
        return np.ascontiguousarray(a, dtype=np.float32 if self.dtype == "f32" else np.uint16)

    def with_block(self, block: int) -> "Model":
        m = Model.__new__(Model)
        m.dims = Dims(self.dims.hidden, self.dims.vocab, self.dims.gru_hidden, self.dims.rank, block, self.dims.dtype)
        m.dtype, m._keep, m.weights = self.dtype, self._keep, self.weights
        return m

    # ---- single operations -------------------------------------------------
    def base_logits(self, H) -> np.ndarray:
        """H: [..., d] stored dtype -> fp32 [..., V]."""
        H = self._store(H)
        rows = H.size // self.dims.hidden
        out = np.empty(H.shape[:-1] + (self.dims.vocab,), dtype=np.float32)
        _load().oracle_base_logits(ctypes.byref(self.dims), _ptr(self._keep["lm_head"]), _ptr(H), rows, _ptr(out))
        return out

    def gru_cell(self, x, h) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float64)
        h = np.ascontiguousarray(h, dtype=np.float64)
        out = np.empty(self.dims.gru_hidden, dtype=np.float64)
        _load().oracle_gru_cell(ctypes.byref(self.dims), ctypes.byref(self.weights), _ptr(x), _ptr(h), _ptr(out))
        return out

    def bottleneck(self, Hrow, S) -> np.ndarray:
        Hrow = self._store(Hrow)
        S = np.ascontiguousarray(S, dtype=np.float64)
        out = np.empty(self.dims.rank, dtype=np.float64)
        _load().oracle_head_bottleneck(ctypes.byref(self.dims), ctypes.byref(self.weights), _ptr(Hrow), _ptr(S),
                                       _ptr(out))
        return out

    def final_logits(self, Lbrow, a) -> np.ndarray:
        Lbrow = np.ascontiguousarray(Lbrow, dtype=np.float32)
        a = np.ascontiguousarray(a, dtype=np.float64)
        out = np.empty(self.dims.vocab, dtype=np.float64)
        _load().oracle_final_logits(ctypes.byref(self.dims), ctypes.byref(self.weights), _ptr(Lbrow), _ptr(a),
                                    _ptr(out))
        return out

    # ---- whole path --------------------------------------------------------
    def chain(self, H, Lb, t0, forced=None, want_logits=True):
        """H [B][P][d], Lb [B][P][V] fp32, t0 [B] -> (tokens, logits|None, margins)."""
        H = self._store(H)
        Lb = np.ascontiguousarray(Lb, dtype=np.float32)
        t0 = np.ascontiguousarray(t0, dtype=np.int32)
        B, P, V = t0.size, self.dims.block, self.dims.vocab
        assert H.size == B * P * self.dims.hidden and Lb.size == B * P * V
        if forced is not None:
            forced = np.ascontiguousarray(forced, dtype=np.int32)
            assert forced.size == B * P
        tokens = np.empty((B, P), dtype=np.int32)
        margins = np.empty((B, P), dtype=np.float64)
        logits = np.empty((B, P, V), dtype=np.float64) if want_logits else None
        _load().oracle_chain(ctypes.byref(self.dims), ctypes.byref(self.weights), B, _ptr(H), _ptr(Lb), _ptr(t0),
                             _ptr(forced), _ptr(tokens), _ptr(logits), _ptr(margins))
        return tokens, logits, margins

    def chain_sampled(self, H, Lb, t0, temperature, seed, seq0=0, forced=None, want_logits=True):
        """Gumbel-max chain at `temperature` -> (tokens, logits|None, perturbed margins)."""
        H = self._store(H)
        Lb = np.ascontiguousarray(Lb, dtype=np.float32)
        t0 = np.ascontiguousarray(t0, dtype=np.int32)
        B, P, V = t0.size, self.dims.block, self.dims.vocab
        assert H.size == B * P * self.dims.hidden and Lb.size == B * P * V
        if forced is not None:
            forced = np.ascontiguousarray(forced, dtype=np.int32)
            assert forced.size == B * P
        tokens = np.empty((B, P), dtype=np.int32)
        margins = np.empty((B, P), dtype=np.float64)
        logits = np.empty((B, P, V), dtype=np.float64) if want_logits else None
        _load().oracle_chain_sampled(ctypes.byref(self.dims), ctypes.byref(self.weights), B, int(seq0), _ptr(H),
                                     _ptr(Lb), _ptr(t0), _ptr(forced), float(temperature), int(seed), _ptr(tokens),
                                     _ptr(logits), _ptr(margins))
        return tokens, logits, margins

    def tree(self, H, Lb, t0, nodes, topm):
        """-> dict(parents, tokens, depth, scores), each [B][N]."""
        H = self._store(H)
        Lb = np.ascontiguousarray(Lb, dtype=np.float32)
        t0 = np.ascontiguousarray(t0, dtype=np.int32)
        B = t0.size
        out = {k: np.empty((B, nodes), dtype=np.int32) for k in ("parents", "tokens", "depth")}
        out["scores"] = np.empty((B, nodes), dtype=np.float64)
        _load().oracle_tree(ctypes.byref(self.dims), ctypes.byref(self.weights), B, _ptr(H), _ptr(Lb), _ptr(t0),
                            nodes, topm, _ptr(out["parents"]), _ptr(out["tokens"]), _ptr(out["depth"]),
                            _ptr(out["scores"]))
        return out


def num_threads() -> int:
    return _load().oracle_num_threads()


def silu(z: float) -> float:
    return _load().oracle_silu(float(z))


def sigmoid(z: float) -> float:
    return _load().oracle_sigmoid(float(z))


def argmax(L):
    L = np.ascontiguousarray(L, dtype=np.float64)
    m = ctypes.c_double()
    t = _load().oracle_argmax(_ptr(L), L.size, ctypes.byref(m))
    return int(t), m.value


def topm(row, M):
    row = np.ascontiguousarray(row, dtype=np.float32)
    idx = np.empty(M, dtype=np.int32)
    val = np.empty(M, dtype=np.float32)
    _load().oracle_topm(_ptr(row), row.size, M, _ptr(idx), _ptr(val))
    return idx, val


def philox4x32_10(counter, key):
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, dtype=np.uint32)
    _load().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def gumbel(seed, b, p, v) -> float:
    return _load().oracle_gumbel(int(seed), int(b), int(p), int(v))


def tree_verify_inputs(parents, tokens, first_tokens, start_positions=None):
    """parents, tokens [B][N] -> (mask [B][N+1][N+1] uint8, positions [B][N+1], tokens [B][N+1])."""
    parents = np.ascontiguousarray(parents, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    first_tokens = np.ascontiguousarray(first_tokens, dtype=np.int32)
    B, N = parents.shape
    sp = None if start_positions is None else np.ascontiguousarray(start_positions, dtype=np.int32)
    mask = np.empty((B, N + 1, N + 1), dtype=np.uint8)
    pos = np.empty((B, N + 1), dtype=np.int32)
    tok = np.empty((B, N + 1), dtype=np.int32)
    _load().oracle_tree_verify_inputs(B, N, _ptr(parents), _ptr(tokens), _ptr(first_tokens), _ptr(sp), _ptr(mask),
                                      _ptr(pos), _ptr(tok))
    return mask, pos, tok
