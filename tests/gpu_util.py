"""Helpers for the GPU parity tests: run the HIP path through the C ABI and the
oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from oracle import pa_ref
from paged_kv_attention_18_amd import binding, synth

# Tolerances on |gpu - oracle| / max(1, |oracle|) for the outputs (max-abs for
# outputs of O(1) magnitude: 2e-3 fp16, 8e-3 bf16) and on the fp32 lse.
TOL = {"f16": 2e-3, "bf16": 8e-3}
LSE_TOL = 2e-4


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(p: synth.Problem, device="cuda"):
    """The same problem with its tensors on the GPU (values copied bit for bit)."""
    q = synth.Problem(**{**p.__dict__})
    for name in ("context_lens", "q_seq_lens", "block_tables", "query", "key_cache", "value_cache", "mask_tensor",
                 "topk_idx"):
        t = getattr(p, name)
        if t is not None:
            setattr(q, name, t.to(device))
    q.block_tables = torch.from_numpy(p.block_tables_np.copy()).to(device)
    q.context_lens = torch.from_numpy(p.context_lens_np.copy()).to(device)
    if p.q_seq_lens_np is not None:
        q.q_seq_lens = torch.from_numpy(p.q_seq_lens_np.copy()).to(device)
    return q


def run_hip(p: synth.Problem, flags=0, num_partitions=0, att=None, lse=True):
    """HIP forward on a GPU problem; returns (out float64 numpy, lse numpy, attention)."""
    own = att is None
    if own:
        att = binding.for_problem(p, flags=flags, num_partitions=num_partitions)
    # NaN-filled outputs: a row the kernels never write cannot pass on
    # whatever the allocator's memory held
    w = p.workload
    out = torch.full((p.num_q_tokens, w.head_num, w.head_size_v), float("nan"), dtype=p.query.dtype,
                     device=p.query.device)
    lse = torch.full((p.num_q_tokens, w.head_num), float("nan"), dtype=torch.float32, device=p.query.device)
    o, l = binding.run_problem(att, p, out=out, lse=lse)
    torch.cuda.synchronize()
    res = (o.to(torch.float64).cpu().numpy(), l.to(torch.float64).cpu().numpy(), att)
    return res


def oracle_full(p: synth.Problem, threads=None):
    return pa_ref.forward(pa_ref.Inputs.from_problem(p), threads=threads)


def assert_close(gpu_o, ref_o, dtype, what=""):
    tol = TOL[dtype]
    d = np.abs(gpu_o - ref_o) / np.maximum(1.0, np.abs(ref_o))
    assert np.all(np.isfinite(gpu_o)), f"{what}: non-finite output"
    worst = float(d.max()) if d.size else 0.0
    assert worst <= tol, f"{what}: max err {worst:.3e} > {tol} at {np.unravel_index(np.argmax(d), d.shape)}"
    return worst


def assert_lse_close(gpu_l, ref_l, what=""):
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(gpu_l), fin), f"{what}: lse finite pattern"
    d = np.abs(gpu_l[fin] - ref_l[fin]) / np.maximum(1.0, np.abs(ref_l[fin]))
    worst = float(d.max()) if d.size else 0.0
    assert worst <= LSE_TOL, f"{what}: lse err {worst:.3e}"
    return worst
