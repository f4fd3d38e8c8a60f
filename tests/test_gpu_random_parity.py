"""A seeded sweep of small random problems on the GPU, each compared with the
oracle on every output element and lse.

Every case draws a head shape (64/64, 128/128, 256/256, 576/512 with or
without one K/V cache), a mask (none, causal, band, the tensor mask), a dtype,
a group size, a block size (powers of two and others), a batch of ragged
lengths with empty sequences among them, query lengths (one token or several)
and block tables with spare columns; the cases are fixed by their seeds.  They
reach the kernel variants the named workloads and the hand-made cases do
(streaming kernel with and without head pairs, whole units and split pieces,
64- and 128-row tiles, whole-tile mode, the 576/512 kernels) in combinations
no hand-made case lists."""
import math

import numpy as np
import pytest

from paged_kv_attention_18_amd import synth

from gpu_util import assert_close, assert_lse_close, log, oracle_full, run_hip, to_device

pytestmark = pytest.mark.gpu

N_CASES = 96
MAX_WORK = 1.5e9   # row x token x (Dk + Dv) products per case (the oracle stays fast)


def draw(i):
    """Case i: (description, problem)."""
    rng = np.random.default_rng(9000 + i)
    while True:
        dk, dv = [(64, 64), (128, 128), (256, 256), (576, 512)][rng.choice(4, p=[0.25, 0.35, 0.15, 0.25])]
        mask = ["none", "causal", "band", "tensor"][rng.integers(4)]
        dt = ["f16", "bf16"][rng.integers(2)]
        shared = dk == 576 and bool(rng.integers(2))
        if dk == 576:
            hkv, g = 1, int(rng.choice([8, 16, 32, 64]))
        else:
            hkv, g = int(rng.choice([1, 2, 4, 8])), int(rng.choice([1, 2, 4, 8, 16]))
        H = hkv * g
        big = mask in ("causal", "band") or dk > 256
        bs = int(rng.choice([16, 32, 48, 64, 96, 128] + ([] if big else [256])))
        B = int(rng.integers(1, 11))
        kvmax = 800 if dk == 576 else 1500
        kv = rng.integers(0, kvmax + 1, size=B)
        kv[rng.random(B) < 0.15] = 0
        if mask == "none" and rng.random() < 0.6:
            ql = None   # decode: one query token per sequence
        else:
            qcap = 16 if dk == 576 else 96
            ql = np.array([int(rng.integers(0, min(int(k), qcap) + 1)) if mask != "none"
                           else int(rng.integers(1, qcap + 1)) for k in kv], dtype=np.int64)
            if mask != "none":
                ql = np.minimum(ql, kv)
        q_tokens = B if ql is None else int(ql.sum())
        if q_tokens == 0:
            continue
        rows = np.ones(B) if ql is None else ql
        if float((rows * kv).sum()) * H * (dk + dv) > MAX_WORK:
            continue
        max_blocks = int(math.ceil(max(1, int(kv.max())) / bs)) + int(rng.integers(0, 3))
        window = (int(rng.integers(0, 300)), int(rng.integers(0, 24))) if mask == "band" else (0, 0)
        desc = (f"case{i}: D{dk}/{dv}{' shared' if shared else ''} {mask} {dt} H{H}/Hkv{hkv} bs{bs} "
                f"kv={kv.tolist()} ql={None if ql is None else ql.tolist()} mb={max_blocks} win={window}")
        p = synth.custom(kv.tolist(), H, hkv, dk, dv, bs, dt, mask,
                         q_seq_lens=None if ql is None else ql.tolist(), seed=int(rng.integers(1 << 30)),
                         max_blocks=max_blocks, shared_kv=shared, window=window)
        return desc, p


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case_matches_oracle(i):
    desc, p_cpu = draw(i)
    log(desc)
    ref_o, ref_l = oracle_full(p_cpu)
    o, l, att = run_hip(to_device(p_cpu))
    assert_close(o, ref_o, p_cpu.workload.dtype, desc)
    assert_lse_close(l, ref_l, desc)
    assert att.device_error() == 0, desc
