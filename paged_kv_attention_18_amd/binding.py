"""Python face of the C ABI (include/pa.h), over ctypes.

Argument marshalling only: every step of the forward pass runs in the HIP
library ``libpa.so`` built next to this file.  The functions carry the C
names (``pa_create``, ``pa_forward``, ``pa_destroy``, ...); ``Attention``
wraps them for torch tensors on a ROCm device, using the current torch
stream.  There is no CPU fallback: without the built library or a gfx950
device every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_HIP, PA_ERR_OOM, PA_ERR_SCRATCH = range(6)
PA_NOALLOC_SCRATCH_BYTES = 64 << 20
PA_F16, PA_BF16 = 0, 1
PA_MASK_NONE, PA_MASK_CAUSAL, PA_MASK_BAND, PA_MASK_TENSOR, PA_MASK_SPARSE = 0, 1, 2, 3, 4
PA_FLAG_FORCE_VALU, PA_FLAG_FORCE_MFMA, PA_FLAG_NO_SPLIT, PA_FLAG_SHARED_KV, PA_FLAG_STATIC_PIECES = 1, 2, 4, 8, 16
PA_FLAG_PLAN_KERNEL = 32
PA_DEVERR_BLOCK_ID, PA_DEVERR_TABLE_SHORT, PA_DEVERR_QLEN, PA_DEVERR_TOKENS, PA_DEVERR_CTX = 1, 2, 4, 8, 16

EXPORTS = ("pa_create", "pa_forward", "pa_forward_sparse", "pa_destroy", "pa_status_string",
           "pa_get_device_error", "pa_set_timing", "pa_read_timing", "pa_describe", "pa_read_probe",
           "pa_forward_noalloc")


class pa_config(ctypes.Structure):
    _fields_ = [
        ("head_num", ctypes.c_int32),
        ("kv_head_num", ctypes.c_int32),
        ("head_size_k", ctypes.c_int32),
        ("head_size_v", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("max_batch", ctypes.c_int32),
        ("max_num_blocks_per_seq", ctypes.c_int32),
        ("max_q_seq_len", ctypes.c_int32),
        ("dtype", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("mask", ctypes.c_int),
        ("flags", ctypes.c_uint32),
        ("num_partitions", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("mask_tensor", ctypes.c_void_p),
        ("topk", ctypes.c_int32),
    ]


class PaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {_status_string(status)} ({status})")


_lock = threading.Lock()
_lib = None


def load_library(path=LIB_PATH):
    """Load libpa.so (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"HIP library {path} is not built; run __graft_entry__.build() "
                               "(or python -m paged_kv_attention_18_amd.build)")
        lib = ctypes.CDLL(path)
        P, i32, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32
        lib.pa_create.argtypes = [ctypes.POINTER(pa_config), ctypes.POINTER(P)]
        lib.pa_create.restype = ctypes.c_int
        lib.pa_forward.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, P, P, P]
        lib.pa_forward.restype = ctypes.c_int
        lib.pa_forward_sparse.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, P, P, P]
        lib.pa_forward_sparse.restype = ctypes.c_int
        lib.pa_forward_noalloc.argtypes = [ctypes.POINTER(pa_config), P, P, P, P, P, P, i32, i32, i32, P, P, P]
        lib.pa_forward_noalloc.restype = ctypes.c_int
        lib.pa_destroy.argtypes = [P]
        lib.pa_destroy.restype = ctypes.c_int
        lib.pa_status_string.argtypes = [ctypes.c_int]
        lib.pa_status_string.restype = ctypes.c_char_p
        lib.pa_get_device_error.argtypes = [P, ctypes.POINTER(u32), i32]
        lib.pa_get_device_error.restype = ctypes.c_int
        lib.pa_set_timing.argtypes = [P, i32]
        lib.pa_set_timing.restype = ctypes.c_int
        lib.pa_read_timing.argtypes = [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32), ctypes.POINTER(i32),
                                       ctypes.POINTER(ctypes.c_double), i32]
        lib.pa_read_timing.restype = ctypes.c_int
        lib.pa_read_probe.argtypes = [P, ctypes.c_int64, P, i32, P]
        lib.pa_read_probe.restype = ctypes.c_int
        lib.pa_describe.argtypes = [P, i32, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                    ctypes.POINTER(i32), ctypes.POINTER(i32)]
        lib.pa_describe.restype = ctypes.c_int
        _lib = lib
        return lib


def _status_string(status):
    try:
        return load_library().pa_status_string(status).decode()
    except Exception:
        return "status"


def _check(status, what):
    if status != PA_OK:
        raise PaError(status, what)


# ------------------------------------------------------------- C-named calls
def pa_create(cfg: pa_config) -> int:
    """Returns an opaque handle (int)."""
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.pa_create(ctypes.byref(cfg), ctypes.byref(h)), "pa_create")
    return h.value


def pa_forward(handle, query, key_cache, value_cache, block_tables, context_lens, q_seq_lens,
               batch, num_q_tokens, max_q_seq_len, out, lse, stream):
    """Pointer-level call: every tensor argument is a device address (int) or 0."""
    lib = load_library()
    _check(lib.pa_forward(handle, query, key_cache, value_cache, block_tables, context_lens,
                          q_seq_lens or None, batch, num_q_tokens, max_q_seq_len, out, lse or None,
                          stream or None), "pa_forward")


def pa_forward_sparse(handle, query, key_cache, value_cache, block_tables, context_lens, q_seq_lens,
                      topk_indices, batch, num_q_tokens, max_q_seq_len, out, lse, stream):
    """Pointer-level call of the sparse mode (device addresses or 0)."""
    lib = load_library()
    _check(lib.pa_forward_sparse(handle, query, key_cache, value_cache, block_tables, context_lens,
                                 q_seq_lens or None, topk_indices, batch, num_q_tokens, max_q_seq_len, out,
                                 lse or None, stream or None), "pa_forward_sparse")


def pa_forward_noalloc(cfg: pa_config, query, key_cache, value_cache, block_tables, context_lens, q_seq_lens,
                       batch, num_q_tokens, max_q_seq_len, out, lse, stream):
    """Pointer-level call of the allocation-free pass (no handle; device
    addresses or 0).  Returns the status instead of raising, so callers can
    tell PA_ERR_SCRATCH apart."""
    lib = load_library()
    return lib.pa_forward_noalloc(ctypes.byref(cfg), query, key_cache, value_cache, block_tables, context_lens,
                                  q_seq_lens or None, batch, num_q_tokens, max_q_seq_len, out, lse or None,
                                  stream or None)


def pa_destroy(handle):
    if handle:
        _check(load_library().pa_destroy(handle), "pa_destroy")


def pa_status_string(status) -> str:
    return _status_string(status)


def pa_get_device_error(handle, clear=True) -> int:
    code = ctypes.c_uint32()
    _check(load_library().pa_get_device_error(handle, ctypes.byref(code), int(clear)), "pa_get_device_error")
    return code.value


def pa_set_timing(handle, enable):
    _check(load_library().pa_set_timing(handle, int(enable)), "pa_set_timing")


def pa_read_timing(handle, per_pass_cap=0):
    """Returns ([plan_ms, attention_ms, merge_ms] summed, passes, passes that
    launched the plan kernel, per-pass [plan, attention, merge] ms lists --
    plan -1 where no plan kernel ran -- for the first per_pass_cap passes)."""
    ms = (ctypes.c_double * 3)()
    n, planned = ctypes.c_int32(), ctypes.c_int32()
    cap = max(0, int(per_pass_cap))
    per = (ctypes.c_double * (3 * max(1, cap)))()
    _check(load_library().pa_read_timing(handle, ms, ctypes.byref(n), ctypes.byref(planned), per if cap else None,
                                         cap), "pa_read_timing")
    rows = [[per[3 * k], per[3 * k + 1], per[3 * k + 2]] for k in range(min(cap, n.value))]
    return [ms[0], ms[1], ms[2]], n.value, planned.value, rows


def pa_read_probe(src, nbytes, sink, workgroups, stream):
    """Pointer-level call of the streaming-read probe (device addresses)."""
    _check(load_library().pa_read_probe(src, int(nbytes), sink, int(workgroups), stream or None), "pa_read_probe")


def pa_describe(handle, max_q_seq_len):
    vals = [ctypes.c_int32() for _ in range(4)]
    _check(load_library().pa_describe(handle, max_q_seq_len, *[ctypes.byref(v) for v in vals]), "pa_describe")
    path, rows, chunk, parts = (v.value for v in vals)
    return {"path": {0: "valu", 1: "mfma", 2: "stream"}[path], "rows_per_tile": rows, "tokens_per_chunk": chunk,
            "partitions": parts}


# ------------------------------------------------------------------ wrapper
_TORCH_DT = {torch.float16: PA_F16, torch.bfloat16: PA_BF16}


class Attention:
    """One configured operator (a pa_create handle) for torch tensors."""

    def __init__(self, head_num, kv_head_num, head_size_k, head_size_v, block_size, num_blocks,
                 max_batch, max_num_blocks_per_seq, max_q_seq_len=1, dtype=torch.float16,
                 scale=None, mask="none", flags=0, num_partitions=0, window=(0, 0), mask_tensor=None, topk=0):
        if dtype not in _TORCH_DT:
            raise ValueError("dtype must be torch.float16 or torch.bfloat16")
        if scale is None:
            scale = head_size_k ** -0.5
        self.dtype = dtype
        if mask == "tensor":
            # the shared fp16 [2048, 2048] matrix; kept referenced by the handle
            self._need(mask_tensor, "mask_tensor", torch.float16, (2048, 2048))
        self.mask_tensor = mask_tensor if mask == "tensor" else None
        self.cfg = pa_config(head_num, kv_head_num, head_size_k, head_size_v, block_size, num_blocks,
                             max_batch, max_num_blocks_per_seq, max_q_seq_len, _TORCH_DT[dtype],
                             float(scale),
                             {"none": PA_MASK_NONE, "causal": PA_MASK_CAUSAL, "band": PA_MASK_BAND,
                              "tensor": PA_MASK_TENSOR, "sparse": PA_MASK_SPARSE}[mask],
                             int(flags), int(num_partitions), int(window[0]), int(window[1]),
                             self.mask_tensor.data_ptr() if self.mask_tensor is not None else None, int(topk))
        self.handle = pa_create(self.cfg)

    def close(self):
        if getattr(self, "handle", None):
            pa_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def describe(self, max_q_seq_len=None):
        return pa_describe(self.handle, max_q_seq_len or self.cfg.max_q_seq_len)

    def device_error(self, clear=True):
        return pa_get_device_error(self.handle, clear)

    def _need(self, t, name, dtype, shape=None):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a torch tensor on the GPU")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")

    def forward(self, query, key_cache, value_cache, block_tables, context_lens, q_seq_lens=None,
                max_q_seq_len=None, out=None, lse=None, return_lse=False, stream=None, topk_indices=None):
        c = self.cfg
        T = query.shape[0] if query.dim() == 3 else -1
        B = context_lens.shape[0]
        self._need(query, "query", self.dtype, (T, c.head_num, c.head_size_k))
        self._need(key_cache, "key_cache", self.dtype,
                   (c.num_blocks, c.block_size, c.kv_head_num, c.head_size_k))
        shared = bool(c.flags & PA_FLAG_SHARED_KV)
        if shared:
            # one cache for K and V: pass None (or the key cache itself)
            if value_cache is not None and value_cache is not key_cache:
                raise ValueError("with PA_FLAG_SHARED_KV value_cache must be None or key_cache")
        else:
            self._need(value_cache, "value_cache", self.dtype,
                       (c.num_blocks, c.block_size, c.kv_head_num, c.head_size_v))
        self._need(block_tables, "block_tables", torch.int32, (B, c.max_num_blocks_per_seq))
        self._need(context_lens, "context_lens", torch.int32, (B,))
        if q_seq_lens is not None:
            self._need(q_seq_lens, "q_seq_lens", torch.int32, (B,))
            if max_q_seq_len is None:
                max_q_seq_len = c.max_q_seq_len
        else:
            max_q_seq_len = 1
        if out is None:
            out = torch.empty((T, c.head_num, c.head_size_v), dtype=self.dtype, device=query.device)
        self._need(out, "out", self.dtype, (T, c.head_num, c.head_size_v))
        if return_lse and lse is None:
            lse = torch.empty((T, c.head_num), dtype=torch.float32, device=query.device)
        if lse is not None:
            self._need(lse, "lse", torch.float32, (T, c.head_num))
        if stream is None:
            stream = torch.cuda.current_stream(query.device).cuda_stream
        args = (self.handle, query.data_ptr(), key_cache.data_ptr(), 0 if shared else value_cache.data_ptr(),
                block_tables.data_ptr(), context_lens.data_ptr(),
                q_seq_lens.data_ptr() if q_seq_lens is not None else 0)
        tail = (B, T, int(max_q_seq_len), out.data_ptr(), lse.data_ptr() if lse is not None else 0, stream)
        if c.mask == PA_MASK_SPARSE:
            # per (query token, KV head) lists of selected token indices
            self._need(topk_indices, "topk_indices", torch.int32, (T, c.kv_head_num, c.topk))
            pa_forward_sparse(*args, topk_indices.data_ptr(), *tail)
        else:
            pa_forward(*args, *tail)
        return (out, lse) if (return_lse or lse is not None) else out

    __call__ = forward


def for_problem(p, **kw):
    """An Attention configured for a ``synth.Problem``."""
    w = p.workload
    from .synth import DTYPES
    args = dict(head_num=w.head_num, kv_head_num=w.kv_head_num, head_size_k=w.head_size_k,
                head_size_v=w.head_size_v, block_size=w.block_size, num_blocks=p.num_blocks,
                max_batch=p.batch, max_num_blocks_per_seq=p.max_num_blocks_per_seq,
                max_q_seq_len=max(1, p.max_q_seq_len), dtype=DTYPES[w.dtype], scale=w.scale, mask=w.mask,
                window=(w.window_left, w.window_right), mask_tensor=p.mask_tensor, topk=w.topk)
    args.update(kw)
    if w.shared_kv:
        args["flags"] = args.get("flags", 0) | PA_FLAG_SHARED_KV
    return Attention(**args)


def run_problem(att, p, **kw):
    return att.forward(p.query, p.key_cache, p.value_cache, p.block_tables, p.context_lens,
                       p.q_seq_lens, max_q_seq_len=max(1, p.max_q_seq_len), topk_indices=p.topk_idx, **kw)
