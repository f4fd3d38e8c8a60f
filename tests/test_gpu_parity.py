"""Parity of the HIP path (through the C ABI) with the oracle, on the GPU.

Small problems are compared element by element; they span several chunks,
several row tiles and ragged tails.  The named workloads are compared at
full size on every output row, element by element, with the launch
configuration the benchmark uses.
Probes check gathering, masking and poison handling bit for bit."""
import math

import numpy as np
import pytest
import torch

from oracle import pa_ref
from paged_kv_attention_18_amd import binding, synth

from gpu_util import assert_close, assert_lse_close, log, oracle_full, run_hip, to_device

pytestmark = pytest.mark.gpu

F = binding


def check_full(p_cpu, flags=0, num_partitions=0, what=""):
    ref_o, ref_l = oracle_full(p_cpu)
    p = to_device(p_cpu)
    o, l, att = run_hip(p, flags=flags, num_partitions=num_partitions)
    e = assert_close(o, ref_o, p_cpu.workload.dtype, what)
    assert_lse_close(l, ref_l, what)
    assert att.device_error() == 0
    return e


# ------------------------------------------------------------------ decode
DECODE_CASES = [
    # (lens, H, Hkv, D, bs, dtype)
    ([1, 17, 64, 33, 100, 300], 4, 4, 64, 16, "f16"),       # G = 1, tiny tails
    ([700, 129, 2050, 5], 32, 8, 128, 128, "bf16"),         # G = 4
    ([1000, 64, 65, 3000], 16, 2, 128, 64, "f16"),          # G = 8
    ([513, 2, 1500], 8, 8, 256, 32, "bf16"),                # Dk = 256
    ([90, 400], 12, 1, 64, 48, "f16"),                      # G = 12 (16-row pad), bs not a power of 2
    ([257, 31], 2, 1, 128, 16, "bf16"),                     # G = 2
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"G{c[1]//c[2]}_D{c[3]}_bs{c[4]}_{c[5]}")
def test_decode_parity(case):
    lens, H, Hkv, D, bs, dt = case
    log(f"decode {case}")
    p = synth.custom(lens, H, Hkv, D, D, bs, dt, seed=sum(lens) % 1000)
    check_full(p, what=f"decode {case}")
    if H // Hkv <= 8:   # the VALU kernel (built for up to 8 rows)
        check_full(p, flags=F.PA_FLAG_FORCE_VALU, what=f"decode valu {case}")


# Short decode passes: block tables of at most 128 tokens (8 chunks of 16), so
# the self-planning streaming kernel runs every unit whole (no partials, no
# merge launch); with and without head pairs, an empty sequence included.
SHORT_DECODE_CASES = [
    # (lens, H, Hkv, D, bs, dtype)
    ([116, 79, 105, 3], 4, 4, 64, 16, "f16"),
    ([100, 37, 128, 0, 60, 1], 32, 8, 128, 16, "bf16"),     # head pairs (G = 4)
    ([128, 17, 64], 16, 2, 128, 32, "f16"),                 # G = 8: head pairs of 16 rows
    ([90, 128, 33], 8, 8, 256, 16, "bf16"),                 # Dk = 256
]


@pytest.mark.parametrize("case", SHORT_DECODE_CASES, ids=["G1", "G4_pairs", "G8_pairs", "D256"])
def test_short_decode_runs_whole_units(case):
    lens, H, Hkv, D, bs, dt = case
    log(f"short decode {case}")
    p_cpu = synth.custom(lens, H, Hkv, D, D, bs, dt, seed=41, max_blocks=128 // bs)
    check_full(p_cpu, what=f"short decode {case}")


@pytest.mark.parametrize("case", DECODE_CASES[:3], ids=["G1", "G4", "G8"])
def test_decode_no_split_and_forced_mfma_agree(case):
    lens, H, Hkv, D, bs, dt = case
    log(f"modes {case}")
    p = synth.custom(lens, H, Hkv, D, D, bs, dt, seed=3)
    check_full(p, flags=F.PA_FLAG_NO_SPLIT, what="no-split")
    check_full(p, flags=F.PA_FLAG_FORCE_MFMA, what="mfma")
    check_full(p, num_partitions=7, what="7 partitions")


# ------------------------------------------------------------ causal / MFMA
CAUSAL_CASES = [
    # (kv, qlen, H, Hkv, D, bs, dtype)
    ([300, 37, 520, 16], [40, 5, 300, 16], 8, 2, 128, 128, "f16"),
    ([1100, 90], [130, 90], 8, 8, 64, 32, "bf16"),
    ([700, 260], [64, 20], 4, 1, 256, 64, "f16"),
    ([150, 40, 1], [4, 8, 1], 32, 8, 128, 128, "f16"),      # splitfuse decode half (16-32 rows)
    ([200, 97], [20, 33], 8, 2, 128, 48, "bf16"),           # block size not a power of 2
]


@pytest.mark.parametrize("case", CAUSAL_CASES, ids=lambda c: f"H{c[2]}_{c[3]}_D{c[4]}_{c[6]}")
def test_causal_mfma_parity(case):
    kv, ql, H, Hkv, D, bs, dt = case
    log(f"causal {case}")
    p = synth.custom(kv, H, Hkv, D, D, bs, dt, "causal", q_seq_lens=ql, seed=11)
    check_full(p, what=f"causal {case}")
    check_full(p, flags=F.PA_FLAG_NO_SPLIT, what="causal no-split")


@pytest.mark.parametrize("scale", [-0.09, 0.0, 2.5], ids=["negative", "zero", "large"])
def test_scale_sign_and_degenerate_values(scale):
    # The MFMA path folds the sign of the scale into Q; scale 0 weighs every
    # visible token equally.
    log(f"scale {scale}")
    p = synth.custom([300, 45], 8, 2, 128, 128, 64, "f16", "causal", q_seq_lens=[40, 45], scale=scale, seed=16)
    check_full(p, what=f"mfma scale {scale}")
    p = synth.custom([300, 45, 1000], 8, 2, 128, 128, 64, "bf16", scale=scale, seed=17)
    check_full(p, what=f"decode scale {scale}")
    check_full(p, flags=F.PA_FLAG_FORCE_VALU, what=f"valu scale {scale}")


@pytest.mark.parametrize("flags", [F.PA_FLAG_FORCE_VALU, 0], ids=["valu", "mfma"])
def test_split_units_merged_across_calls(flags):
    # Many small pieces: every unit is split over several parts, written by
    # workgroups that may sit on different XCDs and merged by the last one.
    # One handle alternates between two problems of the same shape, so a
    # merge that read a stale part of the previous call would show.
    log(f"split merge {flags}")
    pa = synth.custom([2000, 1500, 3000, 700], 8, 2, 128, 128, 64, "bf16", seed=40)
    pb = synth.custom([2000, 1500, 3000, 700], 8, 2, 128, 128, 64, "bf16", seed=41)
    refs = [oracle_full(pa), oracle_full(pb)]
    gs = [to_device(pa), to_device(pb)]
    att = binding.for_problem(gs[0], flags=flags, num_partitions=97)
    for rep in range(3):
        for k in (0, 1):
            o, l, _ = run_hip(gs[k], att=att)
            assert_close(o, refs[k][0], "bf16", f"rep {rep} problem {k}")
            assert_lse_close(l, refs[k][1], f"rep {rep} problem {k}")
    assert att.device_error() == 0


def test_causal_small_rows():
    # qlen * G <= 16 in causal mode: one 16-row tile per unit (streaming kernel)
    log("causal small rows")
    p = synth.custom([50, 9, 200], 8, 4, 128, 128, 16, "bf16", "causal", q_seq_lens=[7, 3, 5], seed=12)
    check_full(p, what="causal small rows")
    # The VALU kernel's causal mode is switched off: the handle is refused.
    p = synth.custom([50, 9, 200], 8, 4, 128, 128, 16, "bf16", "causal", q_seq_lens=[4, 3, 1], seed=12)
    with pytest.raises(binding.PaError) as e:
        binding.for_problem(to_device(p), flags=F.PA_FLAG_FORCE_VALU)
    assert e.value.status == binding.PA_ERR_UNSUPPORTED


VALU_CAUSAL_FAULT = ("one GPU run of this case on the VALU kernel's causal mode ended in a GPU memory "
                     "fault; its cause has not been shown, so the mode is refused and the case stays off the GPU")


@pytest.mark.skip(reason=VALU_CAUSAL_FAULT)
def test_causal_small_rows_valu():
    # kv [50, 9, 200], q [4, 3, 1], H 8 / Hkv 4 (G 2, 8 rows), D 128, bs 16, bf16
    log("causal small rows valu")
    p = synth.custom([50, 9, 200], 8, 4, 128, 128, 16, "bf16", "causal", q_seq_lens=[4, 3, 1], seed=12)
    check_full(p, flags=F.PA_FLAG_FORCE_VALU, what="causal valu")


def test_no_mask_multi_token():
    log("no-mask multi token")
    p = synth.custom([80, 300], 8, 2, 64, 64, 16, "f16", "none", q_seq_lens=[3, 9], seed=13)
    check_full(p, what="none multi")


def test_mla_shape_small():
    log("mla small")
    p = synth.custom([1500, 77, 640, 33], 64, 1, 576, 512, 128, "bf16", scale=1 / 24, seed=14)
    check_full(p, what="mla")
    check_full(p, flags=F.PA_FLAG_NO_SPLIT, what="mla no-split")


def test_mla_shape_f16_causal_small():
    log("mla causal")
    p = synth.custom([300, 70], 16, 1, 576, 512, 64, "f16", "causal", q_seq_lens=[5, 2], seed=15)
    check_full(p, what="mla causal")


# ------------------------------------------------------- shared K/V cache
SHARED_CASES = [
    # (lens, H, Hkv, Dk, Dv, bs, dtype, mask, q_seq_lens)
    ([1500, 77, 640, 33], 64, 1, 576, 512, 128, "bf16", "none", None),   # MLA decode: V from the K tile in LDS
    ([300, 70], 16, 1, 576, 512, 64, "f16", "causal", [5, 2]),            # MLA, parallel decoding
    ([700, 129, 2050, 5], 32, 8, 128, 128, 128, "bf16", "none", None),    # streaming kernel, V = K
    ([80, 300], 8, 2, 64, 64, 16, "f16", "causal", [40, 100]),            # 400-row units (two blocks per wave)
    ([90, 33], 8, 4, 64, 64, 32, "f16", "causal", [9, 12]),               # 24-48 row units
]


@pytest.mark.parametrize("case", SHARED_CASES, ids=lambda c: f"D{c[3]}_{c[4]}_H{c[1]}_{c[7]}")
def test_shared_kv_parity(case):
    """One cache for K and V (V = leading Dv elements of each K row): parity
    with the oracle, and bit-identity with the same problem given V as its
    own tensor cut from K when both kernels take the same chunk size (one
    worker per unit, so both runs add in the same order)."""
    lens, H, Hkv, Dk, Dv, bs, dt, mask, ql = case
    log(f"shared kv {case}")
    p = synth.custom(lens, H, Hkv, Dk, Dv, bs, dt, mask, q_seq_lens=ql, seed=40 + Dk, shared_kv=True)
    assert p.value_cache is None
    check_full(p, what=f"shared {case}")
    shared_ns, shared_l, att_s = run_hip(to_device(p), flags=F.PA_FLAG_NO_SPLIT)
    p2 = synth.Problem(**{**p.__dict__})
    p2.workload = synth.Workload(**{**p.workload.__dict__, "shared_kv": False})
    p2.value_cache = p.key_cache[..., :Dv].contiguous()
    sep_ns, sep_l, att_v = run_hip(to_device(p2), flags=F.PA_FLAG_NO_SPLIT)
    if att_s.describe()["tokens_per_chunk"] == att_v.describe()["tokens_per_chunk"]:
        assert np.array_equal(shared_ns, sep_ns) and np.array_equal(shared_l, sep_l)
    else:   # another summation order: both within the tolerance of the oracle's result
        ref_o, ref_l = oracle_full(p)
        assert_close(shared_ns, ref_o, dt, "shared no-split")
        assert_close(sep_ns, ref_o, dt, "separate no-split")
        assert_lse_close(shared_l, ref_l, "shared no-split")
    if Dk == Dv and mask == "none" and H // Hkv <= 8:
        check_full(p, flags=F.PA_FLAG_FORCE_VALU, what=f"shared valu {case}")


def test_shared_kv_poison_and_arguments():
    """Shared K/V: NaN in K rows past each context and in unreferenced blocks
    leaves the output bit-identical; a value_cache other than NULL or the key
    cache is refused before any launch."""
    log("shared kv poison")
    p = synth.custom([70, 200, 129], 16, 1, 576, 512, 64, "bf16", seed=47, max_blocks=8, shared_kv=True)
    pd = to_device(p)
    clean, _, att = run_hip(pd)
    assert att.describe()["path"] == "mfma"
    bs = 64
    used = set()
    for b in range(p.batch):
        n = int(p.context_lens_np[b])
        nb = (n + bs - 1) // bs
        used.update(p.block_tables_np[b, :nb].tolist())
        if n % bs:
            p.key_cache[int(p.block_tables_np[b, nb - 1]), n % bs:] = float("nan")
        p.block_tables_np[b, nb:] = -1
    for blk in range(p.num_blocks):
        if blk not in used:
            p.key_cache[blk] = float("nan")
    dirty, _, _ = run_hip(to_device(p))
    assert np.array_equal(clean, dirty)
    # the same key cache object as value_cache is accepted, another tensor is not
    o1 = att.forward(pd.query, pd.key_cache, pd.key_cache, pd.block_tables, pd.context_lens)
    torch.cuda.synchronize()
    assert np.array_equal(o1.to(torch.float64).cpu().numpy(), clean)
    other = pd.key_cache[..., :512].contiguous()
    with pytest.raises(ValueError):
        att.forward(pd.query, pd.key_cache, other, pd.block_tables, pd.context_lens)
    lib = binding.load_library()
    out = torch.empty((p.batch, 16, 512), dtype=pd.query.dtype, device="cuda")
    st = lib.pa_forward(att.handle, pd.query.data_ptr(), pd.key_cache.data_ptr(), other.data_ptr(),
                        pd.block_tables.data_ptr(), pd.context_lens.data_ptr(), None, p.batch, p.batch, 1,
                        out.data_ptr(), None, None)
    assert st == binding.PA_ERR_INVALID_ARG
    assert att.device_error() == 0


# ------------------------------------------------------------------- band mask
BAND_CASES = [
    # (lens, H, Hkv, Dk, Dv, bs, dtype, q_seq_lens, (left, right), shared)
    ([300, 17, 128, 129, 1000, 2050], 32, 8, 128, 128, 128, "bf16", None, (127, 0), False),   # streaming
    ([90, 47, 33, 400], 8, 2, 64, 64, 16, "f16", None, (5, 0), False),       # window inside one chunk
    ([200, 70, 33], 8, 2, 64, 64, 16, "f16", [40, 5, 33], (20, 3), False),    # rows see ahead too
    ([900, 300], 32, 8, 128, 128, 128, "f16", [512, 8], (127, 0), False),     # long chunk, most blocks skipped
    ([1500, 77, 640], 64, 1, 576, 512, 128, "bf16", None, (127, 0), True),    # the pages' shape: 64 heads, 1 KV head
    ([300, 70], 16, 1, 576, 512, 64, "f16", [5, 2], (40, 2), False),
    ([2500, 900], 16, 2, 128, 128, 64, "f16", [64, 3], (700, 0), False),    # window of many chunks: split units
]


@pytest.mark.parametrize("case", BAND_CASES, ids=lambda c: f"D{c[3]}_H{c[1]}_w{c[8][0]}_{c[8][1]}")
def test_band_parity(case):
    """Band mask: parity with the oracle, balanced and one worker per unit."""
    lens, H, Hkv, Dk, Dv, bs, dt, ql, win, shared = case
    log(f"band {case}")
    p = synth.custom(lens, H, Hkv, Dk, Dv, bs, dt, "band", q_seq_lens=ql, seed=50 + Dk, shared_kv=shared,
                     window=win)
    check_full(p, what=f"band {case}")
    check_full(p, flags=F.PA_FLAG_NO_SPLIT, what=f"band no-split {case}")


def test_band_wide_windows_equal_causal_and_none():
    """A window reaching past every sequence start is the causal mask when it
    reaches nothing ahead, and no mask when it reaches past every end: the
    same plan and arithmetic, so bit for bit."""
    log("band limits")
    for ql in ([7, 30], None):
        p = synth.custom([200, 77], 16, 4, 128, 128, 64, "bf16", "causal" if ql else "none", q_seq_lens=ql,
                         seed=57)
        ref, ref_l, _ = run_hip(to_device(p))
        q = synth.Problem(**{**p.__dict__})
        q.workload = synth.Workload(**{**p.workload.__dict__, "mask": "band", "window_left": 1 << 30,
                                       "window_right": 0 if ql else 1 << 30})
        o, l, att = run_hip(to_device(q))
        assert np.array_equal(ref, o) and np.array_equal(ref_l, l)
        assert att.device_error() == 0


def test_band_skips_blocks_before_the_window():
    """Blocks wholly before every row's window are never read: their table
    entries may be invalid and their contents NaN; NaN in the tokens of a
    window's first block that lie before the window changes nothing either.
    exp(lse) with q = 0 counts each row's window."""
    log("band skips")
    p = synth.custom([700, 129, 1000], 16, 4, 128, 128, 16, "f16", "band", q_seq_lens=[3, 1, 9], seed=58,
                     window=(100, 0))
    clean, clean_l, _ = run_hip(to_device(p))
    bs = 16
    for b in range(p.batch):
        kv, q = int(p.context_lens_np[b]), int(p.q_seq_lens_np[b])
        lo = max(0, kv - q - 100)          # lowest token any row of b sees
        for blk in range(lo // bs):        # blocks wholly before it
            p.key_cache[int(p.block_tables_np[b, blk])] = float("nan")
            p.value_cache[int(p.block_tables_np[b, blk])] = float("nan")
            p.block_tables_np[b, blk] = -7
        first = int(p.block_tables_np[b, lo // bs])
        p.key_cache[first, :lo % bs] = float("nan")
        p.value_cache[first, :lo % bs] = float("nan")
    o, l, att = run_hip(to_device(p))
    assert np.array_equal(clean, o) and np.array_equal(clean_l, l)
    assert att.device_error() == 0
    p.query.zero_()
    _, l, _ = run_hip(to_device(p))
    t0 = 0
    for b in range(p.batch):
        kv, q = int(p.context_lens_np[b]), int(p.q_seq_lens_np[b])
        for i in range(q):
            pos = kv - q + i
            count = min(kv, pos + 1) - max(0, pos - 100)
            assert np.all(np.abs(np.exp(l[t0 + i]) - count) <= 1e-3 * count), (b, i)
        t0 += q


# ------------------------------------------------------------------ tensor mask
TENSOR_CASES = [
    # (lens, H, Hkv, Dk, Dv, bs, dtype, q_seq_lens, shared)
    ([300, 17, 128, 1000], 32, 8, 128, 128, 128, "bf16", None, False),      # decode, streaming
    ([90, 47, 33], 8, 4, 64, 64, 16, "f16", [5, 1, 8], False),              # streaming, several tokens
    ([200, 70, 33], 8, 2, 64, 64, 16, "f16", [40, 5, 33], False),           # 16-row+ units (tile)
    ([900, 300], 16, 8, 256, 256, 64, "bf16", [130, 8], False),             # Dk 256
    ([1500, 77, 640], 64, 1, 576, 512, 128, "bf16", None, True),            # MLA, shared K/V
    ([300, 70], 16, 1, 576, 512, 64, "f16", [5, 2], False),
]


@pytest.mark.parametrize("case", TENSOR_CASES, ids=lambda c: f"D{c[3]}_H{c[1]}_{'dec' if c[7] is None else 'multi'}")
def test_tensor_mask_parity(case):
    """The shared mask matrix with arbitrary values (N(0, 4), some -inf)
    added to the scores: parity with the oracle, balanced and one worker per
    unit; with the pages' matrix (-10000 above the diagonal) the result is
    the causal one."""
    lens, H, Hkv, Dk, Dv, bs, dt, ql, shared = case
    log(f"tensor mask {case}")
    p = synth.custom(lens, H, Hkv, Dk, Dv, bs, dt, "tensor", q_seq_lens=ql, seed=60 + Dk, shared_kv=shared)
    p.mask_tensor = synth.random_mask_tensor(61)
    check_full(p, what=f"tensor {case}")
    check_full(p, flags=F.PA_FLAG_NO_SPLIT, what=f"tensor no-split {case}")
    p.mask_tensor = synth.causal_mask_tensor(-10000.0)
    check_full(p, what=f"pages matrix {case}")


def test_tensor_mask_beyond_the_matrix():
    """Query rows past 2048 and columns past the matrix follow the causal rule."""
    log("tensor mask beyond the matrix")
    p = synth.custom([2150, 40], 2, 1, 64, 64, 16, "f16", "tensor", q_seq_lens=[2100, 3], seed=62)
    p.mask_tensor = synth.random_mask_tensor(63)
    check_full(p, what="tensor beyond")


# ------------------------------------------------------------------ sparse lists
SPARSE_CASES = [
    # (lens, H, Hkv, Dk, Dv, bs, dtype, q_seq_lens, topk, shared)
    ([300, 17, 1000, 70], 64, 1, 128, 128, 16, "bf16", None, 40, False),
    ([200, 70, 33], 128, 2, 64, 64, 16, "f16", [4, 5, 3], 24, False),
    ([1500, 77, 640], 64, 1, 576, 512, 128, "bf16", None, 512, True),     # the pages' shape: cmp_topk 512
    ([300, 70], 64, 1, 576, 512, 64, "f16", [3, 2], 100, False),
]


def _sparse_problem(case, seed):
    lens, H, Hkv, Dk, Dv, bs, dt, ql, topk, shared = case
    p = synth.custom(lens, H, Hkv, Dk, Dv, bs, dt, "sparse", q_seq_lens=ql, seed=seed, shared_kv=shared, topk=topk)
    # the last two entries of every list: one past the row's causal limit
    # (where the sequence has one) and one past the sequence -- both skipped
    idx = p.topk_idx.numpy()
    qls = np.ones(p.batch, np.int64) if p.q_seq_lens_np is None else p.q_seq_lens_np
    t = 0
    for b in range(p.batch):
        kv, q = int(p.context_lens_np[b]), int(qls[b])
        for i in range(q):
            pos = max(0, kv - q) + i
            idx[t, :, -2] = pos + 1 if pos + 1 < kv else -1
            idx[t, :, -1] = kv + 3
            t += 1
    p.topk_idx = torch.from_numpy(idx)
    return p


@pytest.mark.parametrize("case", SPARSE_CASES, ids=lambda c: f"D{c[3]}_H{c[1]}_k{c[8]}")
def test_sparse_parity(case):
    """Sparse lists over a compressed cache: parity with the oracle, balanced
    and one worker per unit."""
    log(f"sparse {case}")
    p = _sparse_problem(case, 70 + case[3])
    check_full(p, what=f"sparse {case}")
    check_full(p, flags=F.PA_FLAG_NO_SPLIT, what=f"sparse no-split {case}")


def test_sparse_reads_only_listed_rows():
    """Cache rows no list selects may hold NaN and blocks holding none of
    them may have invalid table entries: the output does not change, and no
    error is flagged."""
    log("sparse poison")
    p = _sparse_problem(SPARSE_CASES[0], 75)
    clean, _, _ = run_hip(to_device(p))
    bs = p.workload.block_size
    idx = p.topk_idx.numpy()
    for b in range(p.batch):
        kv = int(p.context_lens_np[b])
        sel = set(int(c) for c in idx[b, 0] if 0 <= c < kv)
        for j in range(kv):
            if j not in sel:
                p.key_cache[int(p.block_tables_np[b, j // bs]), j % bs] = float("nan")
                p.value_cache[int(p.block_tables_np[b, j // bs]), j % bs] = float("nan")
        for blk in range((kv + bs - 1) // bs):
            if not any(blk * bs <= c < (blk + 1) * bs for c in sel):
                p.block_tables_np[b, blk] = -9
    dirty, _, att = run_hip(to_device(p))
    assert np.array_equal(clean, dirty)
    assert att.device_error() == 0


# ------------------------------------------------------------------ probes
def test_one_hot_gather_bit_exact():
    """K zero except the row of logical token t*, q one-hot: out is V[t*] bit for bit."""
    log("one-hot")
    for D, bs, dt, H, Hkv in ((128, 128, "bf16", 8, 2), (64, 16, "f16", 4, 4), (576, 128, "bf16", 16, 1)):
        Dv = 512 if D == 576 else D
        p = synth.custom([700, 129, 40], H, Hkv, D, Dv, bs, dt, seed=21)
        rng = np.random.default_rng(1)
        p.key_cache.zero_()
        p.query.zero_()
        p.query[:, :, 0] = 64.0
        stars = []
        for b in range(p.batch):
            n = int(p.context_lens_np[b])
            t = int(rng.choice([0, n - 1, min(bs, n - 1), int(rng.integers(0, n))]))
            stars.append(t)
            blk = int(p.block_tables_np[b, t // bs])
            p.key_cache[blk, t % bs, :, 0] = 64.0
        for flags in (0, F.PA_FLAG_NO_SPLIT):
            o, _, _ = run_hip(to_device(p), flags=flags)
            for b, t in enumerate(stars):
                blk = int(p.block_tables_np[b, t // bs])
                for h in range(H):
                    want = p.value_cache[blk, t % bs, h // (H // Hkv)].to(torch.float64).numpy()
                    assert np.array_equal(o[b, h], want), (D, b, h, t)


def test_lse_counts_visible_tokens():
    """q = 0: every logit is 0, lse = ln(#visible) exactly recoverable per row."""
    log("lse count")
    for mask, ql in (("none", None), ("causal", [5, 40, 1, 17])):
        kv = [5, 300, 1, 1000]
        p = synth.custom(kv, 8, 2, 128, 128, 16 if mask == "none" else 64, "f16", mask, q_seq_lens=ql, seed=22)
        p.query.zero_()
        _, l, _ = run_hip(to_device(p))
        t0 = 0
        qls = ql or [1] * len(kv)
        for b, (n, q) in enumerate(zip(kv, qls)):
            prefix = max(0, n - q)
            for i in range(q):
                vis = n if mask == "none" else min(n, prefix + i + 1)
                got = np.exp(l[t0 + i])
                assert np.all(np.rint(got) == vis), (mask, b, i, got[:2], vis)
            t0 += q


def test_poison_tails_and_slack():
    """NaN in tail slots, unreferenced blocks and padding table entries leaves
    the output bit-identical and finite."""
    log("poison")
    for D, dt, mask, ql in ((128, "bf16", "none", None), (128, "f16", "causal", [20, 3]), (576, "bf16", "none", None)):
        Dv = 512 if D == 576 else D
        H, Hkv = (16, 1) if D == 576 else (8, 2)
        p = synth.custom([70, 200], H, Hkv, D, Dv, 64, dt, mask, q_seq_lens=ql, seed=23, max_blocks=8)
        clean, _, _ = run_hip(to_device(p))
        valu = D != 576 and mask == "none"
        clean_valu = run_hip(to_device(p), flags=F.PA_FLAG_FORCE_VALU)[0] if valu else None
        bs = 64
        used = set()
        for b in range(p.batch):
            n = int(p.context_lens_np[b])
            nb = (n + bs - 1) // bs
            used.update(p.block_tables_np[b, :nb].tolist())
            last = int(p.block_tables_np[b, nb - 1])
            if n % bs:
                p.key_cache[last, n % bs:] = float("nan")
                p.value_cache[last, n % bs:] = float("nan")
            p.block_tables_np[b, nb:] = -1            # never read
        for blk in range(p.num_blocks):
            if blk not in used:
                p.key_cache[blk] = float("nan")
                p.value_cache[blk] = float("nan")
        dirty, _, att = run_hip(to_device(p))
        assert np.array_equal(clean, dirty), (D, mask)
        if valu:
            assert np.array_equal(clean_valu, run_hip(to_device(p), flags=F.PA_FLAG_FORCE_VALU)[0]), (D, "valu")


def test_masked_positions_have_zero_weight():
    """Changing K/V at token j changes no causal row that cannot see j."""
    log("mask weight")
    p = synth.custom([300], 8, 2, 128, 128, 64, "f16", "causal", q_seq_lens=[40], seed=24)
    base, _, _ = run_hip(to_device(p))
    prefix = 260
    j = prefix + 20            # visible from row i >= 20
    blk = int(p.block_tables_np[0, j // 64])
    p.key_cache[blk, j % 64] = 3.0
    p.value_cache[blk, j % 64] = -7.0
    pert, _, _ = run_hip(to_device(p))
    assert np.array_equal(base[:20], pert[:20])
    assert not np.array_equal(base[20:], pert[20:])


def test_block_permutation_bit_exact():
    log("permutation")
    for case in (DECODE_CASES[1], DECODE_CASES[2]):
        lens, H, Hkv, D, bs, dt = case
        p = synth.custom(lens, H, Hkv, D, D, bs, dt, seed=25)
        o1, l1, _ = run_hip(to_device(p))
        v1, w1, _ = run_hip(to_device(p), flags=F.PA_FLAG_FORCE_VALU)
        perm = np.random.default_rng(4).permutation(p.num_blocks)
        inv = torch.from_numpy(np.argsort(perm).astype(np.int64))
        p2 = synth.Problem(**{**p.__dict__})
        p2.key_cache = p.key_cache[inv].clone()
        p2.value_cache = p.value_cache[inv].clone()
        p2.block_tables_np = perm[p.block_tables_np].astype(np.int32)
        o2, l2, _ = run_hip(to_device(p2))
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        v2, w2, _ = run_hip(to_device(p2), flags=F.PA_FLAG_FORCE_VALU)
        assert np.array_equal(v1, v2) and np.array_equal(w1, w2)


def test_hip_graph_replays_match_eager():
    """pa_forward captured in a HIP graph (through torch's graph capture):
    every replay, with other GPU work and synchronisations in between,
    gives the eager result bit for bit (decode with split units, a causal
    splitfuse mix on the matrix cores, the claimed tail, a short decode
    whose units run whole with no merge, and the 576/512 kernel planning for
    itself, split and whole)."""
    log("graph replay")
    tail = synth.custom(np.random.default_rng(29).integers(1000, 4000, size=24).tolist(), 32, 8, 128, 128, 128,
                        "bf16", seed=29)
    short = synth.custom([116, 79, 105, 3], 32, 8, 128, 128, 16, "f16", seed=30, max_blocks=8)
    for p_cpu, parts in ((synth.custom([3000, 100, 2049, 700], 32, 8, 128, 128, 128, "bf16", seed=27), 0),
                         (synth.custom([600, 90], 8, 2, 128, 128, 64, "f16", "causal", q_seq_lens=[130, 6],
                                       seed=28), 0),
                         (tail, 16),    # the streaming kernel's claimed tail (counter reset by the merge)
                         (short, 0),    # whole units: one kernel, no merge
                         # the 576/512 kernel planning for itself, one cache, then band whole units
                         (synth.custom([700, 33, 2050, 5], 16, 1, 576, 512, 64, "bf16", seed=31,
                                       shared_kv=True), 0),
                         (synth.custom([300, 5, 900, 129], 64, 1, 576, 512, 64, "bf16", "band", window=(127, 0),
                                       shared_kv=True, seed=32), 0)):
        p = to_device(p_cpu)
        att = binding.for_problem(p, num_partitions=parts)
        T, H, Dv = p.num_q_tokens, p.workload.head_num, p.workload.head_size_v
        ref_o, ref_l = binding.run_problem(att, p, return_lse=True)
        ref_o, ref_l = ref_o.clone(), ref_l.clone()
        out = torch.empty(T, H, Dv, dtype=p.query.dtype, device="cuda")
        lse = torch.empty(T, H, dtype=torch.float32, device="cuda")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            binding.run_problem(att, p, out=out, lse=lse)   # warm-up on the capture stream
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=side):
                binding.run_problem(att, p, out=out, lse=lse)
        torch.cuda.synchronize()
        for rep in range(3):
            out.fill_(float("nan"))
            lse.zero_()
            junk = torch.randn(1 << 20, device="cuda").sum()   # other work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), rep
            del junk
        assert att.device_error() == 0


def test_deterministic_runs():
    log("determinism")
    p = to_device(synth.custom([3000, 100, 2049], 32, 8, 128, 128, 128, "bf16", seed=26))
    att = binding.for_problem(p)
    a = binding.run_problem(att, p).clone()
    b = binding.run_problem(att, p).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_whole_tile_mode_claims_are_deterministic():
    """Prefill-sized causal units with a handful of workers: the planner runs
    whole row tiles from per-XCD queues, workers claim tasks at run time, and
    with 4 workers the queues of the other 4 XCDs are served only by claims
    from other queues.  Whole tiles are computed in one piece whichever worker
    runs them, so every worker count and every run gives the same bits, and
    those match the oracle."""
    log("whole-tile mode: claims")
    p_cpu = synth.custom([600, 900, 1300, 700], 8, 2, 128, 128, 128, "f16", "causal",
                         q_seq_lens=[256, 128, 256, 64], seed=28)
    ref_o, ref_l = oracle_full(p_cpu)
    p = to_device(p_cpu)
    runs = []
    for parts in (4, 8, 6, 4):
        o, l, att = run_hip(p, num_partitions=parts)
        assert att.device_error() == 0
        runs.append((o, l))
    assert_close(runs[0][0], ref_o, "f16", "whole-tile mode")
    assert_lse_close(runs[0][1], ref_l, "whole-tile mode")
    for o, l in runs[1:]:
        assert np.array_equal(o, runs[0][0]) and np.array_equal(l, runs[0][1])


def test_bad_block_id_is_flagged_not_read():
    log("bad block id")
    p = synth.custom([100, 50], 4, 2, 64, 64, 16, "f16", seed=27)
    p.block_tables_np[0, 2] = p.num_blocks + 5
    p.block_tables_np[1, 0] = -3
    g = to_device(p)
    att = binding.for_problem(g)
    binding.run_problem(att, g)
    torch.cuda.synchronize()
    assert att.device_error() & F.PA_DEVERR_BLOCK_ID
    assert att.device_error() == 0          # cleared by the previous read


# The streaming kernel cuts its own pieces for up to 256 sequences (four per
# lane of its wave) and takes the plan kernel's above; both cuts must give the
# oracle's answer, at the register boundaries too.  The plan kernel spreads
# its pieces over several workgroups while the sequences fit its LDS (2048)
# and places them all in one workgroup past that.
@pytest.mark.parametrize("batch", [63, 64, 65, 128, 256, 257, 400, 2048, 2049, 2300])
def test_decode_batch_sizes_around_self_planning(batch):
    log(f"decode batch {batch}")
    rng = np.random.default_rng(batch)
    lens = rng.integers(1, 300 if batch <= 400 else 80, size=batch).tolist()
    p = synth.custom(lens, 8, 2, 64, 64, 16, "f16", seed=batch)
    check_full(p, what=f"batch {batch}")


# The self-planning streaming kernel's claimed tail: each worker streams a
# static piece of about nine tenths of its share, then claims further, smaller
# pieces from a counter while it computes, so fast workers take more.  Few
# workers make the tail appear at sizes the oracle finishes quickly (it needs
# at least 320 chunks per worker); the map of pieces depends on the
# lengths alone, so results are the same whichever worker ran which piece.
TAIL_CASES = [
    # (batch, length range, H, Hkv, D, bs, dtype, workers)
    (48, (200, 3000), 32, 8, 128, 128, "bf16", 16),
    (100, (1, 1800), 16, 2, 64, 16, "f16", 8),
    (256, (1, 2000), 32, 8, 128, 64, "f16", 48),
    (7, (3000, 9000), 64, 8, 128, 128, "bf16", 8),
]


@pytest.mark.parametrize("case", TAIL_CASES, ids=lambda c: f"B{c[0]}_G{c[2]//c[3]}_D{c[4]}_P{c[7]}")
def test_claimed_tail_parity(case):
    B, (lo, hi), H, Hkv, D, bs, dt, P = case
    log(f"claimed tail {case}")
    lens = np.random.default_rng(B + P).integers(lo, hi, size=B).tolist()
    p = synth.custom(lens, H, Hkv, D, D, bs, dt, seed=40 + P)
    items = sum(-(-k // 16) for k in lens) * Hkv
    assert items >= 20 * 16 * P   # long enough for a tail
    check_full(p, num_partitions=P, what=f"tail {case}")
    check_full(p, num_partitions=P, flags=F.PA_FLAG_STATIC_PIECES, what=f"static pieces {case}")


# The claimed tail in the other modes of the streaming kernel (each mode is
# its own kernel instance): causal rows of a few query tokens, the band
# mask, the shared mask matrix, and one cache for K and V.
TAIL_MODE_CASES = [
    # (name, batch, length range, q range, H, Hkv, Dk, Dv, bs, dtype, mask, window, shared, workers)
    ("causal", 40, (300, 4000), (1, 4), 32, 8, 128, 128, 128, "f16", "causal", (0, 0), False, 16),
    ("band", 96, (500, 6000), None, 16, 8, 64, 64, 16, "bf16", "band", (127, 0), False, 8),
    ("tensor", 32, (300, 3000), (1, 2), 16, 4, 128, 128, 64, "f16", "tensor", (0, 0), False, 8),
    ("shared", 48, (200, 3000), None, 32, 8, 128, 128, 128, "bf16", "none", (0, 0), True, 16),
]


@pytest.mark.parametrize("case", TAIL_MODE_CASES, ids=lambda c: c[0])
def test_claimed_tail_mask_modes(case):
    name, B, (lo, hi), qr, H, Hkv, Dk, Dv, bs, dt, mask, win, shared, P = case
    log(f"claimed tail, {name}")
    rng = np.random.default_rng(B * 7 + P)
    lens = rng.integers(lo, hi, size=B).tolist()
    ql = None if qr is None else rng.integers(qr[0], qr[1] + 1, size=B).tolist()
    p = synth.custom(lens, H, Hkv, Dk, Dv, bs, dt, mask, q_seq_lens=ql, seed=70 + B, shared_kv=shared,
                     window=win)
    if mask == "tensor":
        p.mask_tensor = synth.random_mask_tensor(71)
    assert binding.for_problem(to_device(p), num_partitions=P).describe()["path"] == "stream"
    check_full(p, num_partitions=P, what=f"tail {name}")
    check_full(p, num_partitions=P, flags=F.PA_FLAG_STATIC_PIECES, what=f"static pieces {name}")


def test_claimed_tail_repeatable_and_reset_between_calls():
    """Back-to-back calls on one handle (the piece counter is reset after
    every pass): the same lengths give bit-identical results, a different
    batch in between gives its own oracle answer, and a permutation of the
    physical blocks changes nothing."""
    log("claimed tail: repeats")
    rng = np.random.default_rng(77)
    la, lb = rng.integers(500, 4000, size=40).tolist(), rng.integers(100, 2500, size=64).tolist()
    nb = int(1.25 * max(sum(-(-k // 128) for k in la), sum(-(-k // 128) for k in lb)))
    pa_cpu = synth.custom(la, 32, 8, 128, 128, 128, "bf16", seed=78, num_blocks=nb, max_blocks=32)
    pb_cpu = synth.custom(lb, 32, 8, 128, 128, 128, "bf16", seed=79, num_blocks=nb, max_blocks=32)
    pa, pb = to_device(pa_cpu), to_device(pb_cpu)
    att = binding.for_problem(pb, num_partitions=16)
    first = binding.run_problem(att, pa).clone()
    ob = binding.run_problem(att, pb).clone()
    again = binding.run_problem(att, pa).clone()
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), again.view(torch.int16))
    assert_close(first.double().cpu().numpy(), oracle_full(pa_cpu)[0], "bf16", "tail call 1")
    assert_close(ob.double().cpu().numpy(), oracle_full(pb_cpu)[0], "bf16", "tail call 2")
    perm = np.random.default_rng(5).permutation(pa_cpu.num_blocks)
    inv = torch.from_numpy(np.argsort(perm).astype(np.int64))
    p2 = synth.Problem(**{**pa_cpu.__dict__})
    p2.key_cache = pa_cpu.key_cache[inv].clone()
    p2.value_cache = pa_cpu.value_cache[inv].clone()
    p2.block_tables_np = perm[pa_cpu.block_tables_np].astype(np.int32)
    permuted = binding.run_problem(att, to_device(p2)).clone()
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), permuted.view(torch.int16))
    assert att.device_error() == 0


# Kernels that cut their own pieces (the streaming kernel; the 576/512 tile
# kernel for one row tile per unit) cut them as the plan kernel does.  With
# PA_FLAG_PLAN_KERNEL the plan kernel runs instead, on the same pieces, so the
# two passes give the same bits; the per-kernel events show which one ran.
SELF_PLAN_CASES = [
    # (name, problem, flags)
    ("mla_decode", lambda: synth.custom([700, 0, 33, 2050, 16, 1500, 290], 32, 1, 576, 512, 64, "bf16", seed=41), 0),
    ("mla_decode_fewer_items_than_workers",
     lambda: synth.custom([20, 3, 40], 16, 1, 576, 512, 16, "f16", seed=42), 0),
    ("mla_decode_rows_0", lambda: synth.custom([300, 90, 5, 600], 16, 1, 576, 512, 32, "bf16",
                                               q_seq_lens=[1, 0, 1, 0], seed=43), 0),
    ("band_shared_whole_units", lambda: synth.custom([300, 5, 900, 129], 64, 1, 576, 512, 64, "bf16", "band",
                                                     window=(127, 0), shared_kv=True, seed=44), 0),
    # several query tokens per sequence, still one 64-row tile (G 16, at most 4 tokens): causal rows
    ("mla_causal_four_tokens", lambda: synth.custom(
        np.random.default_rng(48).integers(4, 700, size=60).tolist(), 16, 1, 576, 512, 32, "f16", "causal",
        q_seq_lens=np.random.default_rng(49).integers(0, 5, size=60).tolist(), seed=48), 0),
    ("mla_decode_200_sequences", lambda: synth.custom(
        np.random.default_rng(50).integers(0, 1500, size=200).tolist(), 16, 1, 576, 512, 64, "bf16",
        shared_kv=True, seed=50), 0),
    ("sparse_lists", lambda: _sparse_problem(([1500, 77, 640, 0, 333], 64, 1, 576, 512, 128, "bf16", None, 512,
                                              True), 45), 0),
    ("stream_static_pieces", lambda: synth.custom([700, 129, 2050, 5], 32, 8, 128, 128, 128, "bf16", seed=7),
     F.PA_FLAG_STATIC_PIECES),
    ("stream_whole_units", lambda: synth.custom([116, 79, 105, 3], 32, 8, 128, 128, 16, "f16", seed=9,
                                                max_blocks=8), 0),
]


@pytest.mark.parametrize("case", SELF_PLAN_CASES, ids=[c[0] for c in SELF_PLAN_CASES])
def test_self_planned_pass_matches_plan_kernel(case):
    name, make, flags = case
    log(f"self plan {name}")
    p_cpu = make()
    p = to_device(p_cpu)
    res = []
    for extra, planned in ((0, 0), (F.PA_FLAG_PLAN_KERNEL, 1)):
        att = binding.for_problem(p, flags=flags | extra)
        binding.pa_set_timing(att.handle, 1)
        o, l, _ = run_hip(p, att=att)
        _, passes, n_planned, _ = binding.pa_read_timing(att.handle)
        assert (passes, n_planned) == (1, planned), name
        assert att.device_error() == 0, name
        res.append((o, l))
    assert np.array_equal(res[0][0], res[1][0], equal_nan=True), name
    assert np.array_equal(res[0][1], res[1][1], equal_nan=True), name
    ref_o, ref_l = oracle_full(p_cpu)
    assert_close(res[0][0], ref_o, p_cpu.workload.dtype, name)
    assert_lse_close(res[0][1], ref_l, name)


def test_self_planned_576_flags_bad_lengths():
    """The 576/512 kernel's own plan flags what the plan kernel flags: a query
    token count that disagrees with the lengths, and a context the block table
    cannot hold (clamped)."""
    log("576 self plan: errors")
    p = synth.custom([30, 40], 16, 1, 576, 512, 16, "bf16", q_seq_lens=[1, 1], seed=46)
    g = to_device(p)
    ref_o, _ = oracle_full(p)
    g.query = g.query[:1].contiguous()   # the lengths ask for 2 query tokens
    att = binding.for_problem(g)
    binding.pa_set_timing(att.handle, 1)
    o, _, _ = run_hip(g, att=att)
    assert binding.pa_read_timing(att.handle)[2] == 0   # no plan kernel
    assert att.device_error() & F.PA_DEVERR_TOKENS
    assert_close(o, ref_o[:1], "bf16", "rows that exist")
    g = to_device(synth.custom([100, 50], 16, 1, 576, 512, 16, "bf16", seed=47))
    g.context_lens = torch.tensor([100, 10_000], dtype=torch.int32, device="cuda")   # table too short
    att = binding.for_problem(g)
    binding.run_problem(att, g)
    torch.cuda.synchronize()
    assert att.device_error() & F.PA_DEVERR_TABLE_SHORT


@pytest.mark.parametrize("batch", [255, 256, 257])
def test_576_batch_sizes_around_self_planning(batch):
    """Up to 256 sequences the 576/512 kernel plans for itself, past that the
    plan kernel runs: both agree with the oracle."""
    log(f"576 batch {batch}")
    rng = np.random.default_rng(500 + batch)
    lens = rng.integers(1, 120, size=batch).tolist()
    p = synth.custom(lens, 16, 1, 576, 512, 16, "bf16", seed=batch)
    att = binding.for_problem(to_device(p))
    binding.pa_set_timing(att.handle, 1)
    check_full(p, what=f"576 batch {batch}")
    o, l, _ = run_hip(to_device(p), att=att)
    assert binding.pa_read_timing(att.handle)[2] == (0 if batch <= 256 else 1)


def test_stream_sequences_without_rows():
    log("sequences without query rows")
    p = synth.custom([40, 70, 5, 130, 64, 1, 333], 8, 4, 128, 128, 16, "bf16",
                     q_seq_lens=[1, 0, 2, 0, 4, 0, 3], seed=31)
    assert binding.for_problem(to_device(p)).describe()["path"] == "stream"
    check_full(p, what="rows 0")


def test_token_count_mismatch_is_flagged():
    log("token count mismatch")
    p = synth.custom([30, 40], 8, 2, 64, 64, 16, "f16", q_seq_lens=[2, 3], seed=32)
    g = to_device(p)
    ref_o, _ = oracle_full(p)
    g.query = g.query[:4].contiguous()   # the lengths ask for 5 query tokens
    o, _, att = run_hip(g)
    assert att.device_error() & F.PA_DEVERR_TOKENS
    assert_close(o, ref_o[:4], "f16", "rows that exist")


def test_bad_lengths_are_clamped_and_flagged():
    log("bad lengths")
    p = synth.custom([100, 50], 4, 2, 64, 64, 16, "f16", seed=28)
    g = to_device(p)
    g.context_lens = torch.tensor([100, 10_000], dtype=torch.int32, device="cuda")   # table too short
    att = binding.for_problem(g)
    binding.run_problem(att, g)
    torch.cuda.synchronize()
    assert att.device_error() & F.PA_DEVERR_TABLE_SHORT


def test_empty_context_outputs_zero():
    log("empty context")
    p = synth.custom([0, 33], 4, 2, 64, 64, 16, "f16", seed=29)
    o, l, _ = run_hip(to_device(p))
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
    ref_o, ref_l = oracle_full(p)
    assert_close(o[1:], ref_o[1:], "f16")


def test_describe_paths():
    p = to_device(synth.custom([10], 32, 8, 128, 128, 128, "bf16", seed=30))
    assert binding.for_problem(p).describe()["path"] == "stream"
    assert binding.for_problem(p, flags=F.PA_FLAG_FORCE_VALU).describe()["path"] == "valu"
    p = to_device(synth.custom([10], 64, 1, 576, 512, 128, "bf16", seed=30))
    assert binding.for_problem(p).describe()["path"] == "mfma"


# ----------------------------------------------------- the named workloads
def full_size_all_rows(n):
    """A named workload at full size, in the benchmark's launch configuration,
    compared with the oracle on every output row, element by element."""
    w = synth.WORKLOADS[n]
    log(f"workload {w.name}: generating on the GPU")
    p = synth.generate(w, device="cuda")
    o, l, att = run_hip(p)
    assert att.device_error() == 0
    log(f"workload {w.name}: oracle on all {p.num_q_tokens} x {w.head_num} rows ({att.describe()})")
    ro, rl = pa_ref.forward(pa_ref.Inputs.from_problem(p))
    e = assert_close(o, ro, w.dtype, w.name)
    assert_lse_close(l, rl, w.name)
    # properties that hold at any size: finite everywhere, |o| <= max |V|
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    vsrc = p.key_cache[..., :w.head_size_v] if w.shared_kv else p.value_cache
    vmax = float(vsrc.abs().max())
    assert np.abs(o).max() <= vmax * (1 + 1e-2)
    log(f"workload {w.name}: max err {e:.2e} over {o.size} outputs")
    return p, o, l, ro, rl


def test_workload_tiny_decode_full():
    w = synth.WORKLOADS[1]
    p = synth.generate(w)
    check_full(p, what=w.name)


def test_workload_gqa_decode_full():
    full_size_all_rows(2)


def test_workload_skewed_long_decode_full():
    p, o, l, ro, rl = full_size_all_rows(3)
    # the longest sequences (32768 tokens), every head, once more on their own
    long_b = np.flatnonzero(p.context_lens_np == 32768)
    assert len(long_b) == 4
    assert_close(o[long_b], ro[long_b], "f16", "skewed 32768-token rows")
    assert_lse_close(l[long_b], rl[long_b], "skewed 32768-token rows")


def test_workload_splitfuse_causal_full():
    p, o, l, ro, rl = full_size_all_rows(4)
    # rows at the starts and ends of the prefill chunks (the causal diagonal
    # at the first and last query token), on their own
    cu = np.concatenate([[0], np.cumsum(p.q_seq_lens_np)])
    big = np.flatnonzero(p.q_seq_lens_np == 512)
    toks = np.concatenate([[cu[b], cu[b] + 1, cu[b + 1] - 1] for b in big]).astype(np.int64)
    assert_close(o[toks], ro[toks], "f16", "splitfuse chunk edges")
    assert_lse_close(l[toks], rl[toks], "splitfuse chunk edges")


def test_workload_mla_decode_full():
    full_size_all_rows(5)


def test_workload_mla_shared_kv_decode_full():
    full_size_all_rows(6)


def test_workload_band_shared_kv_decode_full():
    full_size_all_rows(7)


def test_workload_splitfuse_tensor_mask_full():
    full_size_all_rows(9)


def test_workload_sparse_topk_decode_full():
    full_size_all_rows(10)


def test_workload_splitfuse_band_full():
    p, o, l, ro, rl = full_size_all_rows(8)
    # rows at the starts and ends of the prefill chunks, on their own
    cu = np.concatenate([[0], np.cumsum(p.q_seq_lens_np)])
    big = np.flatnonzero(p.q_seq_lens_np == 512)
    toks = np.concatenate([[cu[b], cu[b] + 1, cu[b] + 200, cu[b + 1] - 1] for b in big]).astype(np.int64)
    assert_close(o[toks], ro[toks], "f16", "splitfuse band chunk rows")
