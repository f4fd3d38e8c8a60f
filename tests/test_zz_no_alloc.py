"""pa_forward_noalloc (the allocation-free entry point) against pa_forward on a
handle for the same configuration, through the C ABI, on the GPU.

Each case makes two calls in a row, the second on a smaller input (the first
sequences of the same problem), and compares both with pa_forward: the same
kernels and pieces run, so the outputs agree bit for bit, and both are also
held to the oracle's tolerance.  The cases run one after another on the one
static array, with other configurations in between, so stale contents from
an earlier call would show."""
import ctypes

import numpy as np
import pytest
import torch

from paged_kv_attention_18_amd import binding, synth

from gpu_util import assert_close, assert_lse_close, log, oracle_full, to_device

pytestmark = pytest.mark.gpu


def first_sequences(p, n):
    """The problem restricted to its first n sequences (same caches)."""
    q = synth.Problem(**{**p.__dict__})
    q.context_lens_np = p.context_lens_np[:n].copy()
    q.block_tables_np = p.block_tables_np[:n].copy()
    ql = np.ones(p.batch, np.int64) if p.q_seq_lens_np is None else p.q_seq_lens_np.astype(np.int64)
    rows = int(ql[:n].sum())
    q.query = p.query[:rows].contiguous()
    if p.q_seq_lens_np is not None:
        q.q_seq_lens_np = p.q_seq_lens_np[:n].copy()
    q.context_lens = torch.from_numpy(q.context_lens_np.copy())
    q.block_tables = torch.from_numpy(q.block_tables_np.copy())
    q.q_seq_lens = None if p.q_seq_lens_np is None else torch.from_numpy(q.q_seq_lens_np.copy())
    return q


def noalloc(cfg, g):
    """One pa_forward_noalloc call on the GPU problem g: (status, out, lse)."""
    w = g.workload
    out = torch.full((g.num_q_tokens, w.head_num, w.head_size_v), float("nan"), dtype=g.query.dtype, device="cuda")
    lse = torch.full((g.num_q_tokens, w.head_num), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    st = binding.pa_forward_noalloc(
        cfg, g.query.data_ptr(), g.key_cache.data_ptr(),
        0 if g.value_cache is None else g.value_cache.data_ptr(), g.block_tables.data_ptr(),
        g.context_lens.data_ptr(), 0 if g.q_seq_lens is None else g.q_seq_lens.data_ptr(),
        len(g.context_lens_np), g.num_q_tokens, max(1, int(g.max_q_seq_len)), out.data_ptr(), lse.data_ptr(),
        stream)
    torch.cuda.synchronize()
    return st, out, lse


def with_handle(att, g):
    o, l = binding.run_problem(att, g, return_lse=True)
    torch.cuda.synchronize()
    return o, l


CASES = {
    # decode, GQA 4: the self-planning streaming kernel
    "gqa_decode": dict(lens=None, H=32, Hkv=8, D=(128, 128), bs=128, dt="bf16", mask="none", parts=0, small=20),
    # splitfuse-like causal units of up to 1200 rows: the 128-row tile kernel, plan and merge
    "causal_tiles": dict(lens=([300, 37, 520, 16, 900], [40, 5, 300, 16, 64]), H=8, Hkv=2, D=(128, 128), bs=64,
                         dt="f16", mask="causal", parts=48, small=2),
    # prefill-sized causal units on 8 workers: whole row tiles from per-XCD
    # queues with claimed tasks (the queues and their counters in the array)
    "causal_whole_tiles": dict(lens=([600, 900, 1300, 700], [256, 128, 256, 64]), H=8, Hkv=2, D=(128, 128),
                               bs=128, dt="f16", mask="causal", parts=8, small=2),
    # 576/512 on one KV head
    "mla": dict(lens=[1500, 77, 640, 33, 2100], H=64, Hkv=1, D=(576, 512), bs=128, dt="bf16", mask="none",
                parts=40, small=2),
}


def make_problem(name, seed):
    c = CASES[name]
    if c["lens"] is None:
        rng = np.random.default_rng(seed)
        kv = rng.integers(100, 3000, size=48).tolist()
        ql = None
    elif isinstance(c["lens"], tuple):
        kv, ql = c["lens"]
    else:
        kv, ql = c["lens"], None
    return synth.custom(kv, c["H"], c["Hkv"], c["D"][0], c["D"][1], c["bs"], c["dt"], c["mask"], q_seq_lens=ql,
                        scale=c["D"][0] ** -0.5, seed=seed)


def run_case(name, seed):
    c = CASES[name]
    p = make_problem(name, seed)
    g = to_device(p)
    att = binding.for_problem(g, num_partitions=c["parts"])
    cfg = att.cfg
    for what, pc in (("full", p), ("smaller", first_sequences(p, c["small"]))):
        log(f"noalloc {name} {what}: batch {len(pc.context_lens_np)}, {pc.num_q_tokens} query tokens")
        gc = to_device(pc)
        st, o, l = noalloc(cfg, gc)
        assert st == binding.PA_OK, binding.pa_status_string(st)
        ho, hl = with_handle(att, gc)
        # the same kernels, pieces and merge order: bit for bit
        assert torch.equal(o.view(torch.int16), ho.view(torch.int16)), f"{name} {what}: out differs from pa_forward"
        assert torch.equal(l.view(torch.int32), hl.view(torch.int32)), f"{name} {what}: lse differs from pa_forward"
        ref_o, ref_l = oracle_full(pc)
        assert_close(o.to(torch.float64).cpu().numpy(), ref_o, c["dt"], f"noalloc {name} {what}")
        assert_lse_close(l.to(torch.float64).cpu().numpy(), ref_l, f"noalloc {name} {what}")
    assert att.device_error() == 0


def test_noalloc_matches_pa_forward_two_calls():
    # configurations alternate on the one array: stale words from the
    # previous configuration's layout must not leak into the next pass
    for name, seed in (("gqa_decode", 71), ("causal_tiles", 72), ("causal_whole_tiles", 75), ("mla", 73),
                       ("gqa_decode", 74)):
        run_case(name, seed)


def test_noalloc_refuses_a_pass_larger_than_the_array():
    # the causal tile kernel with its default grid: 2 x 1024 partial slots of
    # 128 rows x 130 floats, well beyond the array; refused before any launch
    p = make_problem("causal_tiles", 75)
    g = to_device(p)
    att = binding.for_problem(g)
    st, o, _ = noalloc(att.cfg, g)
    assert st == binding.PA_ERR_SCRATCH
    assert torch.isnan(o.float()).all()
    # the same configuration with fewer partitions fits
    att.cfg.num_partitions = 48
    st, _, _ = noalloc(att.cfg, g)
    assert st == binding.PA_OK


def test_noalloc_checks_the_configuration_first():
    p = make_problem("gqa_decode", 76)
    g = to_device(p)
    cfg = binding.for_problem(g).cfg
    bad = binding.pa_config.from_buffer_copy(cfg)
    bad.block_size = 24   # not a multiple of 16
    st, _, _ = noalloc(bad, g)
    assert st == binding.PA_ERR_INVALID_ARG
