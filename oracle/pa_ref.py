"""ctypes face of the C oracle (``pa_ref.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may use this module; the product path never does.

The C source is compiled with gcc on first use (or when it is newer than the
built library), so the oracle needs nothing from the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_ref.c")
LIB = os.path.join(HERE, "libpa_ref.so")

F16, BF16 = 0, 1
MASK_NONE, MASK_CAUSAL, MASK_BAND, MASK_TENSOR, MASK_SPARSE = 0, 1, 2, 3, 4
MASK_DIM = 2048   # the shared mask matrix of the tensor mask is MASK_DIM x MASK_DIM fp16
ERRORS = {-1: "bad argument", -2: "block id out of range", -3: "bad lengths", -4: "out of memory"}

_lock = threading.Lock()
_libs = {}


def build(src=SRC, out=LIB, extra_flags=()):
    """Compile an oracle source to a shared library with gcc."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", *extra_flags, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path=None):
    """Load (building first if needed) an oracle library; returns a ctypes CDLL."""
    path = path or LIB
    with _lock:
        if path in _libs:
            return _libs[path]
        if path == LIB and (not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC)):
            build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        common = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, i64, i32, i32, i32, f64, i32, i32, P, P, i32]
        lib.pa_ref_forward.argtypes = common + [P, P, ctypes.c_int]
        lib.pa_ref_forward.restype = ctypes.c_int
        lib.pa_ref_rows.argtypes = common + [i64, P, P, P, P, ctypes.c_int]
        lib.pa_ref_rows.restype = ctypes.c_int
        _libs[path] = lib
        return lib


def default_threads():
    """The host threads to use: the CPUs this process may run on, at most the
    share named by OMP_NUM_THREADS (16 when unset)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "16"))
    except ValueError:
        share = 16
    return max(1, min(n, share if share > 0 else 16))


class Inputs:
    """Host copies of one problem, in the form the oracle reads: fp16/bf16 as
    raw uint16 bit patterns, lengths and tables as int32."""

    def __init__(self, query, key_cache, value_cache, block_tables, context_lens, q_seq_lens,
                 head_num, kv_head_num, dtype, mask, scale, head_size_v=None, window=(0, 0),
                 mask_tensor=None, topk_idx=None):
        self.query = _bits(query)
        self.key_cache = _bits(key_cache)
        # value_cache None: the V row of a token is the first head_size_v
        # elements of its K row (one cache for both)
        self.value_cache = None if value_cache is None else _bits(value_cache)
        self.head_size_v = int(self.value_cache.shape[3] if value_cache is not None else head_size_v)
        self.block_tables = np.ascontiguousarray(block_tables, dtype=np.int32)
        self.context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
        self.q_seq_lens = None if q_seq_lens is None else np.ascontiguousarray(q_seq_lens, dtype=np.int32)
        self.head_num = int(head_num)
        self.kv_head_num = int(kv_head_num)
        self.dtype = {"f16": F16, "bf16": BF16}.get(dtype, dtype)
        self.mask = {"none": MASK_NONE, "causal": MASK_CAUSAL, "band": MASK_BAND,
                     "tensor": MASK_TENSOR, "sparse": MASK_SPARSE}.get(mask, mask)
        # sparse: int32 [num_q_tokens, kv_head_num, topk] lists of token indices
        self.topk_idx = None
        if topk_idx is not None:
            ti = topk_idx.detach().cpu().numpy() if hasattr(topk_idx, "detach") else topk_idx
            self.topk_idx = np.ascontiguousarray(ti, dtype=np.int32)
        # tensor mask: fp16 [MASK_DIM, MASK_DIM] added to the scaled scores
        self.mask_tensor = None if mask_tensor is None else _bits(mask_tensor)
        if self.mask_tensor is not None:
            assert self.mask_tensor.shape == (MASK_DIM, MASK_DIM)
        self.scale = float(scale)
        # band mask: (tokens before the query's position, tokens after it)
        self.win_left, self.win_right = int(window[0]), int(window[1])

    @classmethod
    def from_problem(cls, p):
        """From a ``synth.Problem`` (tensors are copied to the host)."""
        w = p.workload
        return cls(p.query, p.key_cache, p.value_cache, p.block_tables_np, p.context_lens_np,
                   p.q_seq_lens_np, w.head_num, w.kv_head_num, w.dtype, w.mask, w.scale, w.head_size_v,
                   (w.window_left, w.window_right), getattr(p, "mask_tensor", None), getattr(p, "topk_idx", None))

    @property
    def batch(self):
        return int(self.context_lens.shape[0])

    @property
    def num_q_tokens(self):
        return int(self.query.shape[0])

    def _args(self):
        nb, bs, _, dk = self.key_cache.shape
        dv = self.head_size_v
        mb = self.block_tables.shape[1] if self.block_tables.ndim == 2 else 0
        ptr = lambda a: None if a is None else a.ctypes.data
        return [ptr(self.query), ptr(self.key_cache), ptr(self.value_cache), ptr(self.block_tables),
                ptr(self.context_lens), ptr(self.q_seq_lens), self.batch, self.num_q_tokens,
                self.head_num, self.kv_head_num, dk, dv, bs, nb, mb, self.dtype, self.mask, self.scale,
                self.win_left, self.win_right, ptr(self.mask_tensor), ptr(self.topk_idx),
                0 if self.topk_idx is None else int(self.topk_idx.shape[-1])]


def _bits(t):
    """A fp16/bf16 torch tensor or uint16 numpy array -> contiguous uint16 array."""
    if isinstance(t, np.ndarray):
        assert t.dtype == np.uint16
        return np.ascontiguousarray(t)
    import torch
    return np.ascontiguousarray(t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def forward(inp: Inputs, threads=None, lib=None):
    """All rows: returns (out float64 [T, H, Dv], lse float64 [T, H])."""
    lib = lib or load()
    dv = inp.head_size_v
    out = np.zeros((inp.num_q_tokens, inp.head_num, dv), dtype=np.float64)
    lse = np.zeros((inp.num_q_tokens, inp.head_num), dtype=np.float64)
    rc = lib.pa_ref_forward(*inp._args(), out.ctypes.data, lse.ctypes.data, threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle: {ERRORS.get(rc, rc)}")
    return out, lse


def rows(inp: Inputs, tokens, heads, threads=None, lib=None):
    """Selected (packed token, head) rows: returns (out [n, Dv], lse [n])."""
    lib = lib or load()
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    heads = np.ascontiguousarray(heads, dtype=np.int32)
    dv = inp.head_size_v
    out = np.zeros((len(tokens), dv), dtype=np.float64)
    lse = np.zeros(len(tokens), dtype=np.float64)
    rc = lib.pa_ref_rows(*inp._args(), len(tokens), tokens.ctypes.data, heads.ctypes.data,
                         out.ctypes.data, lse.ctypes.data, threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle: {ERRORS.get(rc, rc)}")
    return out, lse
