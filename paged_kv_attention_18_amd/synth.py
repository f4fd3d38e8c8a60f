"""Seeded synthetic inputs for the paged-attention forward pass.

This module draws lengths, block tables and query/key/value values.  It holds
none of the attention arithmetic, so the oracle and the HIP path can both be
fed from it.

Recipe (one seed per workload):
  * numpy ``Generator(PCG64(seed))`` draws, in this order, the context lengths
    (and query lengths), then one permutation of the physical block ids;
  * query, key cache and value cache are float32 N(0, 1) from
    ``torch.Generator`` seeded with ``seed * 16 + {1, 2, 3}`` on the target
    device, drawn in chunks and rounded to fp16/bf16 (round to nearest even);
  * every sequence takes the next ceil(kv / block_size) ids of the permutation,
    so no physical block is shared; unused table entries hold block 0, a valid
    id as the pages require of every entry;
  * blocks that no sequence references (the slack) keep their random values.

The named workloads follow the shapes, dtypes, length mixes and mask modes of
the operator's documented use: decode (one query token per sequence), GQA
decode, long skewed decode, parallel decoding / splitfuse with the causal
mask aligned at prefix = kvSeqLen - qSeqLen, single-KV-head decode with
576/512 key/value head sizes (also with one cache for K and V), the band
mask with a 127-token window (decode and splitfuse), and splitfuse with the
shared compressed mask matrix.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, Optional

import numpy as np
import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    head_num: int
    kv_head_num: int
    head_size_k: int
    head_size_v: int
    block_size: int
    dtype: str                 # "f16" | "bf16"
    mask: str                  # "none" | "causal" | "band"
    scale: float
    lengths: Callable          # rng -> (context_lens int32[B], q_seq_lens int32[B] or None)
    num_blocks: Optional[int] = None   # fixed pool size; None -> used blocks + slack
    slack: float = 0.10
    seed: int = 0
    shared_kv: bool = False    # V rows are the first head_size_v elements of the K rows
    window_left: int = 0       # band mask: tokens before the query's position it sees
    window_right: int = 0      # band mask: tokens after it
    mask_fill: float = -10000.0   # tensor mask: the value above the diagonal of the shared matrix
    topk: int = 0              # sparse mask: entries per (query token, KV head) list


def _tiny_lengths(rng):
    return rng.integers(1, 129, size=4).astype(np.int32), None


def _gqa_lengths(rng):
    return rng.integers(512, 4097, size=64).astype(np.int32), None


def _skewed_lengths(rng):
    u = rng.uniform(math.log(256.0), math.log(32768.0), size=256)
    kv = np.clip(np.floor(np.exp(u)), 256, 32768).astype(np.int32)
    kv[rng.choice(256, size=4, replace=False)] = 32768   # "a few sequences at 32768"
    return kv, None


def _splitfuse_lengths(rng):
    qlen = rng.choice(np.array([4, 8, 16], dtype=np.int32), size=32)
    qlen[rng.choice(32, size=16, replace=False)] = 512      # prefill chunks for half the batch
    hist = rng.integers(0, 8193, size=32).astype(np.int32)
    return (qlen + hist).astype(np.int32), qlen.astype(np.int32)


def _mla_lengths(rng):
    return rng.integers(1024, 16385, size=128).astype(np.int32), None


WORKLOADS = {
    1: Workload("tiny_decode", 4, 4, 4, 64, 64, 16, "f16", "none", 1.0 / 8.0,
                _tiny_lengths, num_blocks=64, seed=1001),
    2: Workload("gqa_decode", 64, 32, 8, 128, 128, 128, "bf16", "none", 1.0 / math.sqrt(128),
                _gqa_lengths, seed=1002),
    3: Workload("skewed_long_decode", 256, 64, 8, 128, 128, 128, "f16", "none",
                1.0 / math.sqrt(128), _skewed_lengths, seed=1003),
    4: Workload("splitfuse_causal", 32, 32, 8, 128, 128, 128, "f16", "causal",
                1.0 / math.sqrt(128), _splitfuse_lengths, seed=1004),
    5: Workload("mla_decode", 128, 64, 1, 576, 512, 128, "bf16", "none", 1.0 / math.sqrt(576),
                _mla_lengths, seed=1005),
    # shared-KV form of the MLA decode: V is the first 512 elements of each K row
    6: Workload("mla_shared_kv_decode", 128, 64, 1, 576, 512, 128, "bf16", "none", 1.0 / math.sqrt(576),
                _mla_lengths, seed=1006, shared_kv=True),
    # band (sliding-window) mask with the window the pages fix (127 past
    # tokens, none ahead): the shared-KV decode of 64 query heads on one KV
    # head, and the splitfuse mix on the GQA shape
    7: Workload("band_shared_kv_decode", 128, 64, 1, 576, 512, 128, "bf16", "band", 1.0 / math.sqrt(576),
                _mla_lengths, seed=1007, shared_kv=True, window_left=127, window_right=0),
    8: Workload("splitfuse_band", 32, 32, 8, 128, 128, 128, "f16", "band", 1.0 / math.sqrt(128),
                _splitfuse_lengths, seed=1008, window_left=127, window_right=0),
    # the splitfuse mix with the pages' own mask interface: the shared
    # compressed 2048 x 2048 matrix (-10000 above the diagonal) added to the
    # scores, every context token computed
    9: Workload("splitfuse_tensor_mask", 32, 32, 8, 128, 128, 128, "f16", "tensor", 1.0 / math.sqrt(128),
                _splitfuse_lengths, seed=1009),
    # sparse top-k decode over a compressed cache (compression ratio 4 of the
    # MLA decode's lengths; 512 entries per list, as the pages fix cmp_topk),
    # 64 query heads on one shared K/V head
    10: Workload("sparse_topk_decode", 128, 64, 1, 576, 512, 128, "bf16", "sparse", 1.0 / math.sqrt(576),
                 lambda rng: (_mla_lengths(rng)[0] // 4, None), seed=1010, shared_kv=True, topk=512),
}


def by_name(name: str) -> Workload:
    for w in WORKLOADS.values():
        if w.name == name:
            return w
    raise KeyError(name)


def fixed_lengths(context_lens, q_seq_lens=None):
    """A ``lengths`` callable that ignores the generator (for hand-made cases)."""
    kv = np.asarray(context_lens, dtype=np.int32)
    ql = None if q_seq_lens is None else np.asarray(q_seq_lens, dtype=np.int32)
    return lambda rng: (kv.copy(), None if ql is None else ql.copy())


@dataclasses.dataclass
class Problem:
    """One generated input set.  Tensors live on ``device``; lengths and
    tables are also kept as host numpy arrays."""
    workload: Workload
    context_lens: torch.Tensor       # int32 [B]
    q_seq_lens: Optional[torch.Tensor]  # int32 [B] or None (one query token each)
    block_tables: torch.Tensor       # int32 [B, max_num_blocks_per_seq]
    query: torch.Tensor              # [T, H, Dk]
    key_cache: torch.Tensor          # [num_blocks, block_size, Hkv, Dk]
    value_cache: Optional[torch.Tensor]   # [num_blocks, block_size, Hkv, Dv]; None with shared_kv
    context_lens_np: np.ndarray
    q_seq_lens_np: Optional[np.ndarray]
    block_tables_np: np.ndarray
    num_blocks: int
    max_num_blocks_per_seq: int
    mask_tensor: Optional[torch.Tensor] = None   # tensor mask: fp16 [MASK_DIM, MASK_DIM]
    topk_idx: Optional[torch.Tensor] = None      # sparse mask: int32 [T, Hkv, topk], -1 = unused

    @property
    def batch(self) -> int:
        return int(self.context_lens_np.shape[0])

    @property
    def num_q_tokens(self) -> int:
        return int(self.query.shape[0])

    @property
    def max_q_seq_len(self) -> int:
        if self.q_seq_lens_np is None:
            return 1
        return int(self.q_seq_lens_np.max()) if self.batch else 0

    def kv_tokens(self) -> int:
        return int(self.context_lens_np.astype(np.int64).sum())

    def sparse_entries(self) -> int:
        """Sparse mask: list entries that select a visible token, over every
        (query token, KV head) list."""
        idx = self.topk_idx.detach().cpu().numpy()
        kv = self.context_lens_np.astype(np.int64)
        ql = np.ones_like(kv) if self.q_seq_lens_np is None else self.q_seq_lens_np.astype(np.int64)
        total, t0 = 0, 0
        for b in range(self.batch):
            for i in range(int(ql[b])):
                lim = min(int(kv[b]), max(0, int(kv[b] - ql[b])) + i + 1)
                e = idx[t0 + i]
                total += int(((e >= 0) & (e < lim)).sum())
            t0 += int(ql[b])
        return total

    def read_tokens(self) -> int:
        """Tokens some row of their sequence sees, summed over sequences: all
        of them, except under a band mask, whose rows (at positions
        prefix .. kv - 1) see nothing before prefix - window_left."""
        kv = self.context_lens_np.astype(np.int64)
        w = self.workload
        if w.mask != "band":
            return int(kv.sum())
        ql = np.ones_like(kv) if self.q_seq_lens_np is None else self.q_seq_lens_np.astype(np.int64)
        lo = np.maximum(0, np.maximum(0, kv - ql) - w.window_left)
        return int(np.maximum(0, kv - lo).sum())


MASK_DIM = 2048   # side of the shared mask matrix of the tensor mask


def causal_mask_tensor(fill=-10000.0, device="cpu"):
    """The shared compressed mask as the pages describe it: fp16
    [MASK_DIM, MASK_DIM], ``fill`` above the diagonal, 0 on and below it."""
    m = torch.zeros(MASK_DIM, MASK_DIM, dtype=torch.float16, device=device)
    return m.masked_fill(torch.ones(MASK_DIM, MASK_DIM, dtype=torch.bool, device=device).triu(1), fill)


def random_mask_tensor(seed, device="cpu", scale=2.0, neg_inf_frac=0.05):
    """A mask matrix of seeded N(0, scale^2) values (fp16) with a fraction of
    -inf entries: arbitrary additive values, not only 0 / large negative."""
    m = _normal((MASK_DIM, MASK_DIM), torch.float32, seed, device) * scale
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) + 1)
    holes = torch.rand(MASK_DIM, MASK_DIM, generator=gen, device=device) < neg_inf_frac
    return m.masked_fill(holes, float("-inf")).to(torch.float16)


def topk_lists(kv, ql, kv_heads, topk, rng):
    """Synthetic selector output: for every query token (row i of its
    sequence) and KV head, min(topk, n) distinct indices drawn uniformly from
    the n = min(kv, prefix + i + 1) compressed tokens the row may see, in
    random order, padded with -1."""
    T = int(kv.shape[0]) if ql is None else int(np.asarray(ql, np.int64).sum())
    out = np.full((T, kv_heads, topk), -1, dtype=np.int32)
    qls = np.ones_like(kv) if ql is None else np.asarray(ql, np.int64)
    t = 0
    for b in range(kv.shape[0]):
        prefix = max(0, int(kv[b]) - int(qls[b]))
        for i in range(int(qls[b])):
            n = min(int(kv[b]), prefix + i + 1)
            m = min(topk, n)
            for g in range(kv_heads):
                out[t, g, :m] = rng.choice(n, size=m, replace=False)
            t += 1
    return out


def _normal(shape, dtype, seed, device, chunk_elems=1 << 26):
    """float32 N(0,1) from a seeded torch generator, rounded to ``dtype``."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        flat[s:e] = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32).to(dtype)
    return out


def make_block_tables(context_lens, block_size, rng, num_blocks=None, slack=0.10, max_blocks=None):
    """Distinct physical blocks per sequence, drawn from one permutation."""
    need = (context_lens.astype(np.int64) + block_size - 1) // block_size
    used = int(need.sum())
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil(used * (1.0 + slack))))
    if used > num_blocks:
        raise ValueError(f"{used} blocks needed, pool has {num_blocks}")
    mb = int(need.max()) if need.size else 0
    if max_blocks is not None:
        mb = max(mb, int(max_blocks))
    mb = max(mb, 1)
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.zeros((context_lens.shape[0], mb), dtype=np.int32)
    k = 0
    for b, n in enumerate(need):
        tables[b, :n] = perm[k:k + n]
        k += n
    return tables, num_blocks


def layout(w: Workload, seed: Optional[int] = None, max_blocks=None):
    """The integer part of problem ``w`` without any tensor values:
    (context_lens int32[B], q_seq_lens int32[B] or None, block_tables
    int32[B, max_blocks], num_blocks, sparse lists int32[T, Hkv, topk] or
    None) -- the same draws ``generate`` makes."""
    seed = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    kv, ql = w.lengths(rng)
    kv = np.asarray(kv, dtype=np.int32)
    ql = None if ql is None else np.asarray(ql, dtype=np.int32)
    tables, nb = make_block_tables(kv, w.block_size, rng, w.num_blocks, w.slack, max_blocks)
    lists = (topk_lists(kv, ql, w.kv_head_num, w.topk, np.random.Generator(np.random.PCG64(seed * 16 + 4)))
             if w.mask == "sparse" else None)
    return kv, ql, tables, nb, lists


def generate(w: Workload, device="cpu", seed: Optional[int] = None, values=True,
             max_blocks=None) -> Problem:
    """Draw one problem for workload ``w`` (see the module docstring)."""
    seed = w.seed if seed is None else seed
    kv, ql, tables, nb, lists = layout(w, seed, max_blocks)
    T = int(kv.shape[0]) if ql is None else int(np.asarray(ql, dtype=np.int64).sum())
    dt = DTYPES[w.dtype]
    qshape = (T, w.head_num, w.head_size_k)
    kshape = (nb, w.block_size, w.kv_head_num, w.head_size_k)
    vshape = (nb, w.block_size, w.kv_head_num, w.head_size_v)
    if values:
        q = _normal(qshape, dt, seed * 16 + 1, device)
        kc = _normal(kshape, dt, seed * 16 + 2, device)
        vc = None if w.shared_kv else _normal(vshape, dt, seed * 16 + 3, device)
    else:
        q = torch.zeros(qshape, dtype=dt, device=device)
        kc = torch.zeros(kshape, dtype=dt, device=device)
        vc = None if w.shared_kv else torch.zeros(vshape, dtype=dt, device=device)
    return Problem(
        workload=w,
        context_lens=torch.from_numpy(kv.copy()).to(device),
        q_seq_lens=None if ql is None else torch.from_numpy(np.asarray(ql, np.int32).copy()).to(device),
        block_tables=torch.from_numpy(tables.copy()).to(device),
        query=q, key_cache=kc, value_cache=vc,
        context_lens_np=kv, q_seq_lens_np=None if ql is None else np.asarray(ql, np.int32),
        block_tables_np=tables, num_blocks=nb, max_num_blocks_per_seq=int(tables.shape[1]),
        mask_tensor=causal_mask_tensor(w.mask_fill, device) if w.mask == "tensor" else None,
        topk_idx=torch.from_numpy(lists).to(device) if lists is not None else None,
    )


def custom(batch_lens, head_num, kv_head_num, head_size_k, head_size_v, block_size,
           dtype="f16", mask="none", scale=None, q_seq_lens=None, num_blocks=None,
           slack=0.25, seed=7, name="custom", device="cpu", max_blocks=None, shared_kv=False,
           window=(0, 0), topk=0) -> Problem:
    """A small hand-shaped problem (tests)."""
    if scale is None:
        scale = 1.0 / math.sqrt(head_size_k)
    w = Workload(name, len(batch_lens), head_num, kv_head_num, head_size_k, head_size_v,
                 block_size, dtype, mask, float(scale), fixed_lengths(batch_lens, q_seq_lens),
                 num_blocks=num_blocks, slack=slack, seed=seed, shared_kv=shared_kv,
                 window_left=int(window[0]), window_right=int(window[1]), topk=int(topk))
    return generate(w, device=device, max_blocks=max_blocks)


def kv_bytes(p: Problem) -> int:
    """Key+value bytes the method must read: each (sequence, KV head, token)
    row that some query row sees, once, K and V head sizes at 2 bytes per
    element (only the K row when V lives inside it)."""
    w = p.workload
    per_row = w.head_size_k if w.shared_kv else w.head_size_k + w.head_size_v
    if w.mask == "sparse":   # the rows the lists select, once per list
        return p.sparse_entries() * per_row * 2
    return p.read_tokens() * w.kv_head_num * per_row * 2
