"""Python binding of libdomino.so, the Domino draft-head hot path for gfx950.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors are torch tensors on the GPU (torch supplies device memory
and streams); the functions below pass their raw pointers through the C ABI
declared in include/domino.h, under the same names.

Importing this package does not touch the GPU.  Loading the library fails
loudly when it has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdomino.so")

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_DEVICE = 0, -1, -2, -3, -4
ERR_TIMEOUT, ERR_FIRST_TOKEN = -5, -6
F32, BF16 = 0, 1
OP_BASE, OP_CHAIN, OP_TREE, OP_CANDIDATES = 0, 1, 2, 3
# raw device-side status word at offset 0 of a workspace
STATUS_FINE, STATUS_BAD_FIRST_TOKEN, STATUS_TIMEOUT = 0, 1, 2

# include/domino.h (the contract) and include/domino_bench.h (bench and test hooks)
EXPORTS = ("domino_version", "domino_last_error", "domino_workspace_size", "domino_device_status",
           "domino_release_cache", "domino_base_logits", "domino_prepare_input_table",
           "domino_prepare_input_table_f64", "domino_draft_chain",
           "domino_draft_chain_sampled",
           "domino_draft_chain_noalloc",
           "domino_noalloc_device_status", "domino_tree_candidates", "domino_tree_draft",
           "domino_tree_verify_inputs")
BENCH_EXPORTS = ("domino_set_timing_events", "domino_set_chain_mode", "domino_chain_stamp_offset")


class DominoError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"domino status {status}: {message}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("hidden", "vocab", "gru_hidden", "rank", "block", "dtype")]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("lm_head", "embed", "w_ih", "w_hh", "b_ih", "b_hh", "w1", "b1", "w2", "b2", "input_table",
                 "input_table_f64")]


_lib = None


def lib():
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build(); "
                               "the draft head has no non-HIP path")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.domino_version.restype = ctypes.c_char_p
        L.domino_version.argtypes = []
        L.domino_last_error.restype = ctypes.c_char_p
        L.domino_last_error.argtypes = []
        L.domino_workspace_size.restype = sz
        L.domino_workspace_size.argtypes = [P, i32, i32, i32, i32]
        L.domino_device_status.restype = ctypes.c_int
        L.domino_device_status.argtypes = [P, P]
        L.domino_release_cache.restype = None
        L.domino_release_cache.argtypes = []
        L.domino_base_logits.restype = ctypes.c_int
        L.domino_base_logits.argtypes = [P, P, P, i32, P, P]
        L.domino_prepare_input_table.restype = ctypes.c_int
        L.domino_prepare_input_table.argtypes = [P, P, P, P]
        L.domino_prepare_input_table_f64.restype = ctypes.c_int
        L.domino_prepare_input_table_f64.argtypes = [P, P, P, P]
        L.domino_draft_chain.restype = ctypes.c_int
        L.domino_draft_chain.argtypes = [P, P, P, P, P, i32, P, P, P, sz, P]
        L.domino_draft_chain_sampled.restype = ctypes.c_int
        L.domino_draft_chain_sampled.argtypes = [P, P, P, P, P, i32, ctypes.c_float, ctypes.c_uint64, P, P, P, sz, P]
        L.domino_draft_chain_noalloc.restype = ctypes.c_int
        L.domino_draft_chain_noalloc.argtypes = [P, P, P, P, P, i32, P, P, P]
        L.domino_noalloc_device_status.restype = ctypes.c_int
        L.domino_noalloc_device_status.argtypes = [P]
        L.domino_tree_candidates.restype = ctypes.c_int
        L.domino_tree_candidates.argtypes = [P, P, i32, i32, P, P, P, sz, P]
        L.domino_tree_draft.restype = ctypes.c_int
        L.domino_tree_draft.argtypes = [P, P, P, P, P, i32, i32, i32, P, P, P, P, P, sz, P]
        L.domino_tree_verify_inputs.restype = ctypes.c_int
        L.domino_tree_verify_inputs.argtypes = [P, P, P, P, i32, i32, P, P, P, P]
        L.domino_set_chain_mode.restype = i32
        L.domino_set_chain_mode.argtypes = [i32]
        L.domino_set_timing_events.restype = None
        L.domino_set_timing_events.argtypes = [P, P, P, P]
        L.domino_chain_stamp_offset.restype = sz
        L.domino_chain_stamp_offset.argtypes = [P, i32]
        _lib = L
    return _lib


def _check(status: int):
    if status != OK:
        raise DominoError(status, lib().domino_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr()) if hasattr(t, "data_ptr") else ctypes.c_void_p(t)


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def version() -> str:
    return lib().domino_version().decode()


def last_error() -> str:
    return lib().domino_last_error().decode()


def set_chain_mode(mode: int) -> int:
    prev = lib().domino_set_chain_mode(int(mode))
    if prev < 0:
        raise ValueError(f"chain mode {mode}")
    return prev


def domino_set_timing_events(base_start=None, base_stop=None, chain_start=None, chain_stop=None):
    """torch.cuda.Event objects (or None) recorded around the main launches of the calls."""
    h = lambda e: None if e is None else ctypes.c_void_p(e.cuda_event)
    lib().domino_set_timing_events(h(base_start), h(base_stop), h(chain_start), h(chain_stop))


def make_dims(hidden, vocab, gru_hidden, rank, block, dtype) -> Dims:
    return Dims(hidden, vocab, gru_hidden, rank, block, {"f32": F32, "bf16": BF16}.get(dtype, dtype))


def make_weights(t: dict) -> Weights:
    """Weights struct from a dict of device tensors (missing biases -> NULL)."""
    names = [f for f, _ in Weights._fields_]
    return Weights(**{k: (t[k].data_ptr() if t.get(k) is not None else None) for k in names})


def domino_workspace_size(dims: Dims, batch: int, op: int, nodes: int = 0, topm: int = 0) -> int:
    return int(lib().domino_workspace_size(ctypes.byref(dims), int(batch), int(op), int(nodes), int(topm)))


def domino_device_status(workspace, stream=None):
    """Waits for the stream and raises DominoError if the last call on `workspace` flagged a device status."""
    _check(lib().domino_device_status(_ptr(workspace), _stream(stream)))


def domino_release_cache():
    lib().domino_release_cache()


def domino_chain_stamp_offset(dims: Dims, batch: int) -> int:
    return int(lib().domino_chain_stamp_offset(ctypes.byref(dims), int(batch)))


def domino_base_logits(dims: Dims, weights: Weights, H, batch: int, base_logits, stream=None):
    _check(lib().domino_base_logits(ctypes.byref(dims), ctypes.byref(weights), _ptr(H), int(batch),
                                    _ptr(base_logits), _stream(stream)))


def domino_prepare_input_table(dims: Dims, weights: Weights, table, stream=None):
    _check(lib().domino_prepare_input_table(ctypes.byref(dims), ctypes.byref(weights), _ptr(table), _stream(stream)))


def domino_prepare_input_table_f64(dims: Dims, weights: Weights, table, stream=None):
    _check(lib().domino_prepare_input_table_f64(ctypes.byref(dims), ctypes.byref(weights), _ptr(table),
                                                _stream(stream)))


def domino_draft_chain(dims: Dims, weights: Weights, H, base_logits, first_tokens, batch: int, out_tokens,
                       out_logits, workspace, workspace_bytes: int, stream=None):
    _check(lib().domino_draft_chain(ctypes.byref(dims), ctypes.byref(weights), _ptr(H), _ptr(base_logits),
                                    _ptr(first_tokens), int(batch), _ptr(out_tokens), _ptr(out_logits),
                                    _ptr(workspace), int(workspace_bytes), _stream(stream)))


def domino_draft_chain_sampled(dims: Dims, weights: Weights, H, base_logits, first_tokens, batch: int,
                               temperature: float, seed: int, out_tokens, out_logits, workspace, workspace_bytes: int,
                               stream=None):
    _check(lib().domino_draft_chain_sampled(ctypes.byref(dims), ctypes.byref(weights), _ptr(H), _ptr(base_logits),
                                            _ptr(first_tokens), int(batch), float(temperature), int(seed),
                                            _ptr(out_tokens), _ptr(out_logits), _ptr(workspace),
                                            int(workspace_bytes), _stream(stream)))


def domino_draft_chain_noalloc(dims: Dims, weights: Weights, H, base_logits, first_tokens, batch: int, out_tokens,
                               out_logits, stream=None):
    _check(lib().domino_draft_chain_noalloc(ctypes.byref(dims), ctypes.byref(weights), _ptr(H), _ptr(base_logits),
                                            _ptr(first_tokens), int(batch), _ptr(out_tokens), _ptr(out_logits),
                                            _stream(stream)))


def domino_noalloc_device_status(stream=None):
    _check(lib().domino_noalloc_device_status(_stream(stream)))


def domino_tree_candidates(dims: Dims, base_logits, batch: int, topm: int, out_index, out_value, workspace,
                           workspace_bytes: int, stream=None):
    _check(lib().domino_tree_candidates(ctypes.byref(dims), _ptr(base_logits), int(batch), int(topm), _ptr(out_index),
                                        _ptr(out_value), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def domino_tree_draft(dims: Dims, weights: Weights, H, base_logits, first_tokens, batch: int, nodes: int, topm: int,
                      out_parents, out_tokens, out_depth, out_scores, workspace, workspace_bytes: int, stream=None):
    _check(lib().domino_tree_draft(ctypes.byref(dims), ctypes.byref(weights), _ptr(H), _ptr(base_logits),
                                   _ptr(first_tokens), int(batch), int(nodes), int(topm), _ptr(out_parents),
                                   _ptr(out_tokens), _ptr(out_depth), _ptr(out_scores), _ptr(workspace),
                                   int(workspace_bytes), _stream(stream)))


def domino_tree_verify_inputs(parents, tokens, first_tokens, start_positions, batch: int, nodes: int, out_mask,
                              out_positions, out_tokens, stream=None):
    _check(lib().domino_tree_verify_inputs(_ptr(parents), _ptr(tokens), _ptr(first_tokens), _ptr(start_positions),
                                           int(batch), int(nodes), _ptr(out_mask), _ptr(out_positions),
                                           _ptr(out_tokens), _stream(stream)))


def tree_verify_inputs(parents, tokens, first_tokens, start_positions=None, stream=None):
    """Device tensors parents, tokens [B][N] -> (mask [B][N+1][N+1] uint8, positions, tokens [B][N+1])."""
    import torch
    B, N = parents.shape
    dev = parents.device
    mask = torch.empty((B, N + 1, N + 1), dtype=torch.uint8, device=dev)
    pos = torch.empty((B, N + 1), dtype=torch.int32, device=dev)
    tok = torch.empty((B, N + 1), dtype=torch.int32, device=dev)
    domino_tree_verify_inputs(parents, tokens, first_tokens, start_positions, B, N, mask, pos, tok, stream)
    return mask, pos, tok


class DraftHead:
    """Device-resident weights plus the three calls, for tests and the bench.

    `weights` holds host arrays as produced by synth.make_weights (bf16 as
    uint16 bit patterns).  Uploading them is the only work done here.
    """

    def __init__(self, hidden, vocab, gru_hidden, rank, block, dtype, weights: dict, device="cuda:0"):
        import numpy as np
        import torch
        self.device = torch.device(device)
        self.dtype = dtype
        self.dims = make_dims(hidden, vocab, gru_hidden, rank, block, dtype)
        self.tensors = {}
        for k, a in weights.items():
            if a is None:
                continue
            if a.dtype == np.uint16:
                t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
            else:
                t = torch.from_numpy(np.ascontiguousarray(a))
            self.tensors[k] = t.to(self.device)
        self.weights = make_weights(self.tensors)

    @classmethod
    def from_config(cls, cfg, weights, device="cuda:0", block=None):
        return cls(cfg.hidden, cfg.vocab, cfg.gru_hidden, cfg.rank, cfg.block if block is None else block,
                   cfg.dtype, weights, device)

    def upload(self, a):
        import numpy as np
        import torch
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(self.device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(self.device)

    def base_logits(self, H, out=None, stream=None):
        import torch
        B = H.shape[0]
        if out is None:
            out = torch.empty((B, self.dims.block, self.dims.vocab), dtype=torch.float32, device=self.device)
        domino_base_logits(self.dims, self.weights, H, B, out, stream)
        return out

    def prepare_input_table(self, stream=None):
        """Builds the per-token GRU input table (domino_prepare_input_table) into a new device
        tensor [V][3 Hs] fp32 and passes it to the chain calls from now on; returns it."""
        import torch
        d = self.dims
        table = torch.empty((d.vocab, 3 * d.gru_hidden), dtype=torch.float32, device=self.device)
        domino_prepare_input_table(d, self.weights, table, stream)
        self.tensors["input_table"] = table
        self.weights = make_weights(self.tensors)
        return table

    def prepare_input_table_f64(self, stream=None):
        """The fp64 table for the tree (domino_prepare_input_table_f64), passed to
        domino_tree_draft from now on; returns it."""
        import torch
        d = self.dims
        table = torch.empty((d.vocab, 3 * d.gru_hidden), dtype=torch.float64, device=self.device)
        domino_prepare_input_table_f64(d, self.weights, table, stream)
        self.tensors["input_table_f64"] = table
        self.weights = make_weights(self.tensors)
        return table

    def drop_input_table(self):
        """The chain and tree calls compute W_ih x from the embedding again."""
        self.tensors.pop("input_table", None)
        self.tensors.pop("input_table_f64", None)
        self.weights = make_weights(self.tensors)

    def workspace(self, batch, op=OP_CHAIN, nodes=0, topm=0):
        import torch
        n = domino_workspace_size(self.dims, batch, op, nodes, topm)
        return torch.zeros(max(n, 16), dtype=torch.uint8, device=self.device)

    def draft_chain(self, H, base_logits, first_tokens, want_logits=True, out_tokens=None, out_logits=None,
                    workspace=None, stream=None, check=True):
        """Enqueue the chain; with `check`, wait for it and raise DominoError on a device status
        (a timed-out wait, or a first token outside the vocabulary)."""
        import torch
        B = H.shape[0]
        if out_tokens is None:
            out_tokens = torch.empty((B, self.dims.block), dtype=torch.int32, device=self.device)
        if want_logits and out_logits is None:
            out_logits = torch.empty((B, self.dims.block, self.dims.vocab), dtype=torch.float32, device=self.device)
        if workspace is None:
            workspace = self.workspace(B)
        domino_draft_chain(self.dims, self.weights, H, base_logits, first_tokens, B, out_tokens,
                           out_logits if want_logits else None, workspace, workspace.numel(), stream)
        if check:
            domino_device_status(workspace, stream)
        return out_tokens, (out_logits if want_logits else None), workspace

    def draft_chain_sampled(self, H, base_logits, first_tokens, temperature, seed, want_logits=True,
                            workspace=None, stream=None, check=True):
        import torch
        B = H.shape[0]
        out_tokens = torch.empty((B, self.dims.block), dtype=torch.int32, device=self.device)
        out_logits = (torch.empty((B, self.dims.block, self.dims.vocab), dtype=torch.float32, device=self.device)
                      if want_logits else None)
        if workspace is None:
            workspace = self.workspace(B)
        domino_draft_chain_sampled(self.dims, self.weights, H, base_logits, first_tokens, B, temperature, seed,
                                   out_tokens, out_logits, workspace, workspace.numel(), stream)
        if check:
            domino_device_status(workspace, stream)
        return out_tokens, out_logits, workspace

    def tree_draft(self, H, base_logits, first_tokens, nodes, topm, workspace=None, stream=None, check=True):
        """-> dict of device tensors parents, tokens, depth [B][N] int32 and scores [B][N] fp64, and the workspace."""
        import torch
        B = H.shape[0]
        out = {k: torch.empty((B, nodes), dtype=torch.int32, device=self.device) for k in ("parents", "tokens", "depth")}
        out["scores"] = torch.empty((B, nodes), dtype=torch.float64, device=self.device)
        if workspace is None:
            workspace = self.workspace(B, OP_TREE, nodes, topm)
        domino_tree_draft(self.dims, self.weights, H, base_logits, first_tokens, B, nodes, topm, out["parents"],
                          out["tokens"], out["depth"], out["scores"], workspace, workspace.numel(), stream)
        if check:
            domino_device_status(workspace, stream)
        return out, workspace

    @staticmethod
    def device_status(workspace) -> int:
        """The device-side status word at offset 0 of a chain workspace (synchronises)."""
        return int(workspace[:4].view(__import__("torch").int32).item())
