"""The seeded input generators (CPU)."""
import math

import numpy as np
import torch

from paged_kv_attention_18_amd import synth


def lengths(n):
    w = synth.WORKLOADS[n]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    return w.lengths(rng)


def test_deterministic_bytes():
    w = synth.WORKLOADS[1]
    a = synth.generate(w)
    b = synth.generate(w)
    assert torch.equal(a.query.view(torch.int16), b.query.view(torch.int16))
    assert torch.equal(a.key_cache.view(torch.int16), b.key_cache.view(torch.int16))
    assert torch.equal(a.value_cache.view(torch.int16), b.value_cache.view(torch.int16))
    assert np.array_equal(a.block_tables_np, b.block_tables_np)
    c = synth.generate(w, seed=5)
    assert not torch.equal(a.key_cache.view(torch.int16), c.key_cache.view(torch.int16))


def test_tiny_decode_shape():
    p = synth.generate(synth.WORKLOADS[1])
    assert p.num_blocks == 64 and p.key_cache.shape == (64, 16, 4, 64)
    assert p.query.dtype == torch.float16 and p.query.shape == (4, 4, 64)
    assert p.context_lens_np.min() >= 1 and p.context_lens_np.max() <= 128


def test_block_tables_distinct_and_in_range():
    for n in (1, 2):
        p = synth.generate(synth.WORKLOADS[n], values=False)
        bs = p.workload.block_size
        used = []
        for b in range(p.batch):
            nb = (int(p.context_lens_np[b]) + bs - 1) // bs
            used.extend(p.block_tables_np[b, :nb].tolist())
            assert nb <= p.max_num_blocks_per_seq
        assert len(used) == len(set(used))
        assert min(used) >= 0 and max(used) < p.num_blocks
        assert p.block_tables_np.min() >= 0 and p.block_tables_np.max() < p.num_blocks


def test_gqa_decode_recipe():
    kv, ql = lengths(2)
    assert ql is None and kv.shape == (64,) and kv.min() >= 512 and kv.max() <= 4096
    p = synth.generate(synth.WORKLOADS[2], values=False)
    need = sum(math.ceil(k / 128) for k in p.context_lens_np)
    assert p.num_blocks == math.ceil(need * 1.1)
    assert p.query.dtype == torch.bfloat16


def test_skewed_recipe():
    kv, _ = lengths(3)
    assert kv.shape == (256,) and kv.min() >= 256 and kv.max() == 32768
    assert (kv == 32768).sum() >= 4
    assert np.median(kv) < 4096          # log-uniform: most sequences short


def test_splitfuse_recipe():
    kv, ql = lengths(4)
    assert (ql == 512).sum() == 16
    assert set(ql[ql != 512].tolist()) <= {4, 8, 16}
    hist = kv - ql
    assert hist.min() >= 0 and hist.max() <= 8192


def test_mla_recipe():
    kv, _ = lengths(5)
    assert kv.min() >= 1024 and kv.max() <= 16384
    w = synth.WORKLOADS[5]
    assert (w.head_size_k, w.head_size_v, w.kv_head_num, w.head_num) == (576, 512, 1, 64)
    assert abs(w.scale - 1 / 24) < 1e-12
