"""Pins for the oracle: checks against facts that do not come from the oracle.

Each ``pin_*`` function takes an oracle library handle (``oracle.pa_ref.load``)
and raises AssertionError when the oracle disagrees with:

  * a library routine on a case the method reduces to (torch's
    scaled_dot_product_attention in float64 on contiguous K/V), including the
    pages' own additive 2048x2048 mask filled with -10000 / -60000;
  * hand-written visibility patterns from the pages (tests/golden);
  * closed forms (one visible token, two tokens, equal scores, q = 0);
  * exact invariants (permuting physical blocks, GQA as repeated MHA, a
    causal row as a shorter decode).

``test_oracle_pins.py`` runs them on the oracle; ``test_oracle_mutants.py``
plants plausible mistakes in the oracle's source and checks that every one
of them trips at least one pin.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from oracle import pa_ref
from paged_kv_attention_18_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers
def to_f64(t):
    return t.detach().cpu().to(torch.float64)


def gather_contiguous(p: synth.Problem, b: int, cache: torch.Tensor):
    """Sequence b's cache rows [kv, Hkv, D], assembled with torch indexing:
    the listed blocks in order, flattened, cut to kv tokens."""
    kv = int(p.context_lens_np[b])
    bs = p.workload.block_size
    nblk = (kv + bs - 1) // bs
    ids = torch.from_numpy(p.block_tables_np[b, :nblk].astype(np.int64))
    blocks = cache.detach().cpu()[ids]                      # [nblk, bs, Hkv, D]
    return blocks.reshape(nblk * bs, blocks.shape[2], blocks.shape[3])[:kv]


def sdpa_reference(p: synth.Problem, attn_mask_fn=None):
    """Per sequence: torch SDPA in float64 over contiguous K/V with GQA.
    attn_mask_fn(qlen, kv) -> additive float mask [qlen, kv] or None; the
    default is the pages' causal rule via ``is_causal`` when history is 0."""
    w = p.workload
    T = p.num_q_tokens
    out = torch.zeros(T, w.head_num, w.head_size_v, dtype=torch.float64)
    lse = torch.zeros(T, w.head_num, dtype=torch.float64)
    ql = np.ones(p.batch, np.int64) if p.q_seq_lens_np is None else p.q_seq_lens_np.astype(np.int64)
    t0 = 0
    G = w.head_num // w.kv_head_num
    for b in range(p.batch):
        qlen, kv = int(ql[b]), int(p.context_lens_np[b])
        if qlen == 0:
            continue
        q = to_f64(p.query[t0:t0 + qlen]).permute(1, 0, 2).unsqueeze(0)           # [1,H,q,Dk]
        k = to_f64(gather_contiguous(p, b, p.key_cache)).permute(1, 0, 2).unsqueeze(0)
        v = to_f64(gather_contiguous(p, b, p.value_cache)).permute(1, 0, 2).unsqueeze(0)
        mask = attn_mask_fn(qlen, kv) if attn_mask_fn else None
        if kv == 0:
            t0 += qlen
            lse[t0 - qlen:t0] = -math.inf
            continue
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=w.scale, enable_gqa=True)
        out[t0:t0 + qlen] = o[0].permute(1, 0, 2)
        logits = torch.matmul(q, k.repeat_interleave(G, dim=1).transpose(-1, -2).contiguous()) * w.scale
        if mask is not None:
            logits = logits + mask
        lse[t0:t0 + qlen] = torch.logsumexp(logits, dim=-1)[0].permute(1, 0)
        t0 += qlen
    return out.numpy(), lse.numpy()


def run(lib, p, threads=2):
    return pa_ref.forward(pa_ref.Inputs.from_problem(p), threads=threads, lib=lib)


def close(a, b, rtol=1e-11, atol=1e-12):
    a, b = np.asarray(a), np.asarray(b)
    finite = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), finite), "finite pattern differs"
    assert np.array_equal(a[~finite], b[~finite]), "non-finite values differ"
    d = np.abs(a[finite] - b[finite])
    lim = atol + rtol * np.abs(b[finite])
    assert np.all(d <= lim), f"max diff {d.max() if d.size else 0:.3e}"


def pages_mask(fill):
    """The pages' shared 2048x2048 causal mask: upper triangle without the
    diagonal holds ``fill``, the rest 0 (stored as fp16 on the device)."""
    m = torch.triu(torch.full((2048, 2048), float(fill), dtype=torch.float16), diagonal=1)
    return m.to(torch.float64)


def load_visibility():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "causal_visibility.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("case"):
                _, q, kv = line.split()
                cur = (int(q), int(kv), [])
                cases.append(cur)
            else:
                cur[2].append([c == "1" for c in line])
    for q, kv, rows in cases:
        assert len(rows) == q and all(len(r) == kv for r in rows)
    return cases


# --------------------------------------------------------- random problems
def decode_cases():
    yield synth.custom([1, 17, 64, 33, 100], 4, 4, 64, 64, 16, "f16", seed=11)
    yield synth.custom([130, 5, 256, 77], 8, 2, 32, 32, 32, "bf16", seed=12)
    yield synth.custom([40, 95, 3], 6, 3, 48, 80, 16, "f16", seed=13)          # Dk != Dv
    yield synth.custom([200, 129], 4, 1, 96, 64, 64, "bf16", scale=0.3, seed=14)


def causal_cases():
    yield synth.custom([9, 20, 37, 16], 4, 2, 32, 32, 16, "f16", "causal",
                       q_seq_lens=[4, 7, 16, 16], seed=21)                        # incl. history 0
    yield synth.custom([70, 33, 128], 8, 2, 64, 48, 32, "bf16", "causal",
                       q_seq_lens=[19, 1, 65], seed=22)
    yield synth.custom([300, 12], 2, 1, 32, 64, 64, "f16", "causal",
                       q_seq_lens=[5, 12], seed=23)


# -------------------------------------------------------------------- pins
def pin_sdpa_decode(lib):
    """Decode (one query token, no mask) equals SDPA on contiguous K/V."""
    for p in decode_cases():
        o, l = run(lib, p)
        ro, rl = sdpa_reference(p)
        close(o, ro)
        close(l, rl)


def pin_sdpa_no_mask_multi_token(lib):
    """Several query tokens with mask 'none': every row sees all kv tokens."""
    p = synth.custom([30, 50], 4, 2, 32, 32, 16, "f16", "none", q_seq_lens=[3, 6], seed=31)
    o, l = run(lib, p)
    ro, rl = sdpa_reference(p)
    close(o, ro)
    close(l, rl)


def pin_sdpa_prefill_is_causal(lib):
    """History 0 (qSeqLen == kvSeqLen): plain causal prefill, torch's is_causal."""
    p = synth.custom([16, 9, 33], 4, 2, 32, 32, 16, "bf16", "causal",
                     q_seq_lens=[16, 9, 33], seed=32)
    o, l = run(lib, p)
    tri = lambda q, kv: torch.zeros(q, kv, dtype=torch.float64).masked_fill(
        torch.ones(q, kv, dtype=torch.bool).triu(1), -math.inf)
    ro, rl = sdpa_reference(p, tri)
    close(o, ro)
    close(l, rl)
    # and with torch's own causal flag on the same data
    w = p.workload
    t0 = 0
    for b in range(p.batch):
        qlen = int(p.q_seq_lens_np[b])
        q = to_f64(p.query[t0:t0 + qlen]).permute(1, 0, 2).unsqueeze(0)
        k = to_f64(gather_contiguous(p, b, p.key_cache)).permute(1, 0, 2).unsqueeze(0)
        v = to_f64(gather_contiguous(p, b, p.value_cache)).permute(1, 0, 2).unsqueeze(0)
        r = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.scale, enable_gqa=True)
        close(o[t0:t0 + qlen], r[0].permute(1, 0, 2).numpy())
        t0 += qlen


def pin_pages_additive_mask(lib):
    """Causal mode equals the pages' additive mask: the shared 2048x2048 mask
    (fill -10000 or -60000), row i of a sequence reading mask row prefix + i."""
    for fill in (-10000.0, -60000.0):
        m = pages_mask(fill)

        def slice_mask(q, kv):
            prefix = max(0, kv - q)
            return m[prefix:prefix + q, :kv].clone()

        for p in causal_cases():
            o, l = run(lib, p)
            ro, rl = sdpa_reference(p, slice_mask)
            close(o, ro)
            close(l, rl)


def pin_visibility_golden(lib):
    """q = 0 makes every logit 0: lse = ln(#visible) and out = mean of the
    visible V rows, row by row, for the hand-written patterns."""
    cases = load_visibility()
    kv = [c[1] for c in cases]
    ql = [c[0] for c in cases]
    p = synth.custom(kv, 2, 1, 16, 16, 16, "f16", "causal", q_seq_lens=ql, seed=41)
    p.query.zero_()
    o, l = run(lib, p)
    t0 = 0
    for b, (q, n, pattern) in enumerate(cases):
        v = to_f64(gather_contiguous(p, b, p.value_cache))[:, 0].numpy()      # [kv, Dv]
        for i in range(q):
            vis = np.array(pattern[i])
            for h in range(2):
                assert abs(l[t0 + i, h] - math.log(vis.sum())) < 1e-12, (q, n, i)
                close(o[t0 + i, h], v[vis].mean(axis=0))
        t0 += q


def pin_one_hot_gather(lib):
    """Cache built by scattering a known logical sequence through the block
    table; a one-hot query picks logical token t* and returns its V row."""
    rng = np.random.default_rng(5)
    for bs, kv in ((16, 70), (32, 32), (64, 129)):
        p = synth.custom([kv, kv // 2 + 1], 2, 1, 16, 8, bs, "f16", seed=50 + bs)
        for b in range(p.batch):
            n = int(p.context_lens_np[b])
            logical_v = torch.randn(n, 8, generator=torch.Generator().manual_seed(b)).to(torch.float16)
            for j in range(n):   # scatter: logical token j -> (table[j // bs], j % bs)
                blk = int(p.block_tables_np[b, j // bs])
                p.value_cache[blk, j % bs, 0] = logical_v[j]
                p.key_cache[blk, j % bs, 0] = 0
            for tstar in sorted({0, n - 1, min(bs, n - 1), int(rng.integers(0, n))}):
                for j in range(n):
                    blk = int(p.block_tables_np[b, j // bs])
                    p.key_cache[blk, j % bs, 0, 0] = 64.0 if j == tstar else 0.0
                p.query.zero_()
                p.query[b, :, 0] = 64.0
                o, _ = run(lib, p)
                assert np.array_equal(o[b, 0], logical_v[tstar].double().numpy()), (bs, b, tstar)
                assert np.array_equal(o[b, 1], logical_v[tstar].double().numpy())


def pin_single_visible_token(lib):
    """kv = 1 (or causal row 0 at history 0): out is that token's V row exactly
    and lse its logit."""
    p = synth.custom([1, 1], 4, 2, 32, 24, 16, "bf16", seed=61)
    o, l = run(lib, p)
    for b in range(2):
        blk = int(p.block_tables_np[b, 0])
        for h in range(4):
            v = to_f64(p.value_cache[blk, 0, h // 2]).numpy()
            assert np.array_equal(o[b, h], v)
            z = p.workload.scale * float(torch.dot(to_f64(p.query[b, h]), to_f64(p.key_cache[blk, 0, h // 2])))
            assert abs(l[b, h] - z) <= 1e-12 * max(1.0, abs(z))
    p = synth.custom([6], 2, 1, 16, 16, 16, "f16", "causal", q_seq_lens=[6], seed=62)
    o, _ = run(lib, p)
    blk = int(p.block_tables_np[0, 0])
    assert np.array_equal(o[0, 0], to_f64(p.value_cache[blk, 0, 0]).numpy())


def pin_two_token_closed_form(lib):
    """Head size 1, scale 1, q = 1: logits are the two K values a, c, so
    out = (e^a v0 + e^c v1) / (e^a + e^c), lse = ln(e^a + e^c)."""
    for a, c, v0, v1 in ((0.0, 1.0, 2.0, -3.0), (-2.5, 0.75, 0.5, 0.25), (3.0, 3.0, 1.0, -1.0)):
        p = synth.custom([2], 1, 1, 1, 1, 16, "f16", scale=1.0, seed=70)
        p.query.fill_(1.0)
        blk = int(p.block_tables_np[0, 0])
        p.key_cache[blk, 0, 0, 0], p.key_cache[blk, 1, 0, 0] = a, c
        p.value_cache[blk, 0, 0, 0], p.value_cache[blk, 1, 0, 0] = v0, v1
        o, l = run(lib, p)
        ea, ec = math.exp(a), math.exp(c)
        assert abs(o[0, 0, 0] - (ea * v0 + ec * v1) / (ea + ec)) < 1e-14
        assert abs(l[0, 0] - math.log(ea + ec)) < 1e-14


def pin_equal_scores_mean(lib):
    """Identical K rows give equal logits: out = mean of the V rows."""
    p = synth.custom([37, 5], 4, 2, 32, 32, 16, "bf16", seed=80)
    for b in range(p.batch):
        n = int(p.context_lens_np[b])
        for j in range(n):
            blk = int(p.block_tables_np[b, j // 16])
            p.key_cache[blk, j % 16] = p.key_cache[int(p.block_tables_np[b, 0]), 0]
    o, l = run(lib, p)
    for b in range(p.batch):
        v = to_f64(gather_contiguous(p, b, p.value_cache)).numpy()     # [kv, Hkv, Dv]
        for h in range(4):
            close(o[b, h], v[:, h // 2].mean(axis=0), rtol=1e-12, atol=1e-13)


def pin_block_permutation(lib):
    """Relabelling physical blocks (moving their contents along) changes no bit."""
    for p in list(decode_cases())[:2] + list(causal_cases())[:1]:
        o, l = run(lib, p)
        nb = p.num_blocks
        perm = np.random.default_rng(90).permutation(nb)
        inv = torch.from_numpy(np.argsort(perm).astype(np.int64))
        # new id perm[i] holds old block i
        p2 = synth.Problem(**{**p.__dict__})
        p2.key_cache = p.key_cache[inv].clone()
        p2.value_cache = p.value_cache[inv].clone()
        p2.block_tables_np = perm[p.block_tables_np].astype(np.int32)
        o2, l2 = run(lib, p2)
        assert np.array_equal(o, o2) and np.array_equal(l, l2)


def pin_gqa_is_repeated_mha(lib):
    """GQA with group G equals MHA whose KV heads repeat each group's head G times."""
    p = synth.custom([50, 21], 6, 2, 32, 40, 16, "f16", seed=100)
    o, l = run(lib, p)
    p2 = synth.Problem(**{**p.__dict__})
    p2.workload = synth.Workload(**{**p.workload.__dict__, "kv_head_num": 6})
    p2.key_cache = p.key_cache.repeat_interleave(3, dim=2).contiguous()
    p2.value_cache = p.value_cache.repeat_interleave(3, dim=2).contiguous()
    o2, l2 = run(lib, p2)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def pin_causal_row_is_short_decode(lib):
    """Causal row i of sequence b equals decode of that row's query over the
    first prefix + i + 1 tokens of the same blocks."""
    for p in causal_cases():
        o, l = run(lib, p)
        w = p.workload
        t0 = 0
        for b in range(p.batch):
            qlen, kv = int(p.q_seq_lens_np[b]), int(p.context_lens_np[b])
            prefix = max(0, kv - qlen)
            for i in range(qlen):
                d = synth.Problem(**{**p.__dict__})
                d.workload = synth.Workload(**{**w.__dict__, "mask": "none"})
                d.context_lens_np = np.array([prefix + i + 1], np.int32)
                d.q_seq_lens_np = None
                d.block_tables_np = p.block_tables_np[b:b + 1].copy()
                d.query = p.query[t0 + i:t0 + i + 1]
                od, ld = run(lib, d)
                assert np.array_equal(od[0], o[t0 + i]) and np.array_equal(ld[0], l[t0 + i])
            t0 += qlen


def pin_rows_equal_forward(lib):
    """The row-subset entry point returns the same bits as the full pass."""
    p = next(causal_cases())
    o, l = run(lib, p)
    inp = pa_ref.Inputs.from_problem(p)
    toks = np.array([0, 3, p.num_q_tokens - 1, 10], np.int32)
    heads = np.array([0, 3, 1, 2], np.int32)
    ro, rl = pa_ref.rows(inp, toks, heads, threads=2, lib=lib)
    assert np.array_equal(ro, o[toks, heads]) and np.array_equal(rl, l[toks, heads])


def pin_empty_rows(lib):
    """kv = 0 with mask 'none': out 0 and lse -inf; qlen = 0 contributes no row."""
    p = synth.custom([0, 5, 3], 2, 1, 16, 16, 16, "f16", "none", q_seq_lens=[1, 0, 2], seed=110)
    o, l = run(lib, p)
    assert o.shape[0] == 3
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
    ro, rl = sdpa_reference(p)
    close(o[1:], ro[1:])
    close(l[1:], rl[1:])


def pin_element_decoding(lib):
    """fp16/bf16 bit patterns decode as numpy/torch decode them (normals,
    subnormals, signed zero, extremes): one visible token returns V exactly."""
    for dt, torch_dt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        p = synth.custom([1], 1, 1, 16, 64, 16, dt, seed=120)
        blk = int(p.block_tables_np[0, 0])
        bits = np.array([0x0001, 0x03FF, 0x0400, 0x3C00, 0xBC00, 0x7BFF, 0x8000, 0x3555,
                         0x0200, 0x4248, 0xC0A0, 0x1234, 0x2E66, 0x5640, 0x8001, 0x6A00] * 4, np.uint16)
        if dt == "bf16":
            bits = np.array([0x0001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x7F7F, 0x8000, 0x3EAB,
                             0x4049, 0xC2F7, 0x3C23, 0x1234, 0x4B00, 0x0040, 0x8081, 0x5F00] * 4, np.uint16)
        p.value_cache[blk, 0, 0] = torch.from_numpy(bits.view(np.int16)).view(torch_dt)
        o, _ = run(lib, p)
        want = torch.from_numpy(bits.view(np.int16)).view(torch_dt).to(torch.float64).numpy()
        assert np.array_equal(o[0, 0], want), dt


def pin_shared_kv_is_sliced_v(lib):
    """Shared K/V (no value cache; V is the first Dv elements of each K row,
    the reading of the SparseAttnSharedkvMetadata page's single K/V cache) equals SDPA
    with V cut from K by torch slicing, and the oracle with that V passed as
    its own tensor, bit for bit.  Dv > Dk without a value cache is refused."""
    for p in (synth.custom([37, 70, 5], 8, 2, 72, 64, 16, "bf16", seed=130, shared_kv=True),
              synth.custom([40, 19], 4, 1, 48, 16, 16, "f16", "causal", q_seq_lens=[9, 19],
                           seed=131, shared_kv=True)):
        assert p.value_cache is None
        o, l = run(lib, p)
        p2 = synth.Problem(**{**p.__dict__})
        p2.workload = synth.Workload(**{**p.workload.__dict__, "shared_kv": False})
        p2.value_cache = p.key_cache[..., :p.workload.head_size_v].contiguous()
        shifted = None
        if p.workload.mask == "causal":     # row i sees tokens up to (kv - qlen) + i
            shifted = lambda q, kv: torch.zeros(q, kv, dtype=torch.float64).masked_fill(
                torch.ones(q, kv, dtype=torch.bool).triu(1 + max(0, kv - q)), -math.inf)
        ro, rl = sdpa_reference(p2, shifted)
        close(o, ro)
        close(l, rl)
        o2, l2 = run(lib, p2)
        assert np.array_equal(o, o2) and np.array_equal(l, l2)
    bad = synth.custom([5], 2, 1, 16, 32, 16, "f16", seed=132, shared_kv=True)
    try:
        run(lib, bad)
    except ValueError:
        pass
    else:
        raise AssertionError("Dv > Dk with V inside K accepted")


def band_cases():
    """Band-mask problems: decode with the pages' window (127 past tokens, 0
    future), and several query tokens with a window reaching forward too."""
    yield synth.custom([300, 17, 128, 129, 1000], 8, 2, 64, 64, 16, "f16", "band", seed=140, window=(127, 0))
    yield synth.custom([200, 70, 33], 4, 1, 32, 48, 16, "bf16", "band", q_seq_lens=[40, 5, 33], seed=141,
                       window=(20, 3))


def _with_mask(p, mask, window=(0, 0)):
    q = synth.Problem(**{**p.__dict__})
    q.workload = synth.Workload(**{**p.workload.__dict__, "mask": mask, "window_left": window[0],
                                   "window_right": window[1]})
    return q


def pin_band_extremes_are_causal_and_none(lib):
    """A band reaching back past every sequence start is the causal mask when
    it reaches no token ahead, and no mask at all when it also reaches past
    every sequence end (bit for bit)."""
    for p in band_cases():
        o_c, l_c = run(lib, _with_mask(p, "causal"))
        o_b, l_b = run(lib, _with_mask(p, "band", (10 ** 6, 0)))
        assert np.array_equal(o_c, o_b) and np.array_equal(l_c, l_b)
        o_n, l_n = run(lib, _with_mask(p, "none"))
        o_b, l_b = run(lib, _with_mask(p, "band", (10 ** 6, 10 ** 6)))
        assert np.array_equal(o_n, o_b) and np.array_equal(l_n, l_b)


def _window_problem(p, b, lo, hi, query):
    """One sequence holding only tokens lo .. hi - 1 of sequence b of p,
    copied into fresh blocks with torch indexing, no mask, one query row."""
    w = p.workload
    n = hi - lo
    bs = w.block_size
    nblk = max(1, (n + bs - 1) // bs)
    kc = gather_contiguous(p, b, p.key_cache)[lo:hi]
    vsrc = p.key_cache[..., :w.head_size_v] if w.shared_kv else p.value_cache
    vc = gather_contiguous(p, b, vsrc)[lo:hi]
    def pack(rows):
        out = torch.zeros(nblk * bs, rows.shape[1], rows.shape[2], dtype=rows.dtype)
        out[:n] = rows
        return out.reshape(nblk, bs, rows.shape[1], rows.shape[2])
    d = synth.Problem(**{**p.__dict__})
    d.workload = synth.Workload(**{**w.__dict__, "mask": "none", "shared_kv": False})
    d.key_cache, d.value_cache = pack(kc), pack(vc)
    d.num_blocks = nblk
    d.block_tables_np = np.arange(nblk, dtype=np.int32)[None, :]
    d.max_num_blocks_per_seq = nblk
    d.context_lens_np = np.array([n], np.int32)
    d.q_seq_lens_np = None
    d.query = query
    return d


def pin_band_row_is_window_attention(lib):
    """Row i of sequence b under the band mask is attention without a mask
    over just the tokens of its window, copied out of the paged cache:
    positions prefix + i - win_left .. prefix + i + win_right, cut to the
    sequence (bit for bit)."""
    for p in band_cases():
        o, l = run(lib, p)
        w = p.workload
        ql = np.ones(p.batch, np.int64) if p.q_seq_lens_np is None else p.q_seq_lens_np.astype(np.int64)
        t0 = 0
        for b in range(p.batch):
            kv = int(p.context_lens_np[b])
            prefix = max(0, kv - int(ql[b]))
            for i in range(int(ql[b])):
                pos = prefix + i
                lo, hi = max(0, pos - w.window_left), min(kv, pos + 1 + w.window_right)
                d = _window_problem(p, b, lo, hi, p.query[t0 + i:t0 + i + 1])
                od, ld = run(lib, d)
                assert np.array_equal(od[0], o[t0 + i]) and np.array_equal(ld[0], l[t0 + i]), (b, i)
            t0 += int(ql[b])


def pin_band_lse_counts_window(lib):
    """q = 0 makes every score 0, so exp(lse) counts the visible tokens: the
    window's size, min(kv, pos + 1 + right) - max(0, pos - left)."""
    for p in band_cases():
        p.query.zero_()
        _, l = run(lib, p)
        w = p.workload
        ql = np.ones(p.batch, np.int64) if p.q_seq_lens_np is None else p.q_seq_lens_np.astype(np.int64)
        t0 = 0
        for b in range(p.batch):
            kv = int(p.context_lens_np[b])
            for i in range(int(ql[b])):
                pos = max(0, kv - int(ql[b])) + i
                count = min(kv, pos + 1 + w.window_right) - max(0, pos - w.window_left)
                assert np.all(np.rint(np.exp(l[t0 + i])) == count), (b, i)
            t0 += int(ql[b])


def _tensor_mask_problem(p, m):
    q = _with_mask(p, "tensor")
    q.mask_tensor = m
    return q


def shifted_mask(m, q, kv):
    """The additive [q, kv] mask a sequence's rows take from the shared
    matrix m, built with torch indexing: 0 over the history (columns below
    prefix), m[i, j - prefix] inside the matrix, and outside it 0 on and
    below the diagonal, -inf above it."""
    prefix = max(0, kv - q)
    D = m.shape[0]
    out = torch.zeros(q, kv, dtype=torch.float64)
    i = torch.arange(q)[:, None]
    c = torch.arange(kv)[None, :] - prefix
    inside = (c >= 0) & (c < D) & (i < D)
    mf = m.to(torch.float64)
    out[inside] = mf[i.expand(q, kv)[inside], c.expand(q, kv)[inside]]
    out[(~inside) & (c > i)] = -math.inf
    return out


def pin_tensor_mask_pages_matrix_is_causal(lib):
    """The pages' shared matrix (-10000 or -60000 above the diagonal) gives
    exactly the causal result: the masked weights underflow to 0."""
    for fill in (-10000.0, -60000.0):
        m = synth.causal_mask_tensor(fill)
        for p in causal_cases():
            o, l = run(lib, p)
            ot, lt = run(lib, _tensor_mask_problem(p, m))
            assert np.array_equal(o, ot) and np.array_equal(l, lt), fill


def pin_tensor_mask_is_additive(lib):
    """Arbitrary matrix values (N(0, 4), some -inf) are added to the scaled
    scores: torch SDPA with the shifted additive mask."""
    m = synth.random_mask_tensor(150)
    for p in list(causal_cases())[:2] + [
            synth.custom([30, 50], 4, 2, 32, 32, 16, "f16", "causal", q_seq_lens=[3, 6], seed=151)]:
        pt = _tensor_mask_problem(p, m)
        o, l = run(lib, pt)
        ro, rl = sdpa_reference(pt, lambda q, kv: shifted_mask(m, q, kv))
        close(o, ro)
        close(l, rl)


def pin_tensor_mask_beyond_the_matrix(lib):
    """Rows past the matrix (query index >= 2048) and columns past it follow
    the causal rule, as the pages say longer sequences are handled."""
    m = synth.random_mask_tensor(152)
    p = synth.custom([2150], 1, 1, 16, 16, 16, "f16", "causal", q_seq_lens=[2100], seed=153)
    pt = _tensor_mask_problem(p, m)
    o, l = run(lib, pt, threads=4)
    ro, rl = sdpa_reference(pt, lambda q, kv: shifted_mask(m, q, kv))
    close(o, ro, rtol=1e-10, atol=1e-11)
    close(l, rl, rtol=1e-10, atol=1e-11)


def sparse_cases():
    """Sparse-list problems: decode and several query tokens, two KV heads.
    The last two entries of every multi-token list are overwritten with
    indices the row must skip: one past its causal limit (when the sequence
    has such a token) and one past the sequence."""
    yield synth.custom([300, 17, 128, 129], 8, 2, 64, 64, 16, "f16", "sparse", seed=160, topk=40)
    p = synth.custom([200, 70, 33], 4, 2, 32, 48, 16, "bf16", "sparse", q_seq_lens=[40, 5, 33], seed=161,
                     topk=24)
    idx = p.topk_idx.numpy()
    t = 0
    for b in range(p.batch):
        kv, q = int(p.context_lens_np[b]), int(p.q_seq_lens_np[b])
        for i in range(q):
            pos = max(0, kv - q) + i
            idx[t, :, -2] = pos + 1 if pos + 1 < kv else -1
            idx[t, :, -1] = kv + 3
            t += 1
    p.topk_idx = torch.from_numpy(idx)
    yield p


def pin_sparse_sorted_full_lists_are_causal(lib):
    """Lists holding every token a row may see, in ascending order, give the
    causal result bit for bit (the compressed-axis rule is the causal rule)."""
    for p in sparse_cases():
        w = p.workload
        kv = p.context_lens_np
        ql = np.ones_like(kv) if p.q_seq_lens_np is None else p.q_seq_lens_np
        K = int(kv.max())
        idx = np.full((p.num_q_tokens, w.kv_head_num, K), -1, np.int32)
        t = 0
        for b in range(p.batch):
            prefix = max(0, int(kv[b]) - int(ql[b]))
            for i in range(int(ql[b])):
                n = min(int(kv[b]), prefix + i + 1)
                idx[t, :, :n] = np.arange(n)
                t += 1
        ps = synth.Problem(**{**p.__dict__})
        ps.workload = synth.Workload(**{**w.__dict__, "topk": K})
        ps.topk_idx = torch.from_numpy(idx)
        o, l = run(lib, ps)
        oc, lc = run(lib, _with_mask(p, "causal"))
        assert np.array_equal(o, oc) and np.array_equal(l, lc)


def pin_sparse_row_is_attention_over_its_list(lib):
    """Each row equals unmasked attention over just the tokens its list
    selects, copied out of the paged cache in list order (bit for bit)."""
    for p in sparse_cases():
        o, l = run(lib, p)
        w = p.workload
        G = w.head_num // w.kv_head_num
        idx = p.topk_idx.numpy()
        ql = np.ones(p.batch, np.int64) if p.q_seq_lens_np is None else p.q_seq_lens_np.astype(np.int64)
        t0 = 0
        for b in range(p.batch):
            kv = int(p.context_lens_np[b])
            prefix = max(0, kv - int(ql[b]))
            for i in range(int(ql[b])):
                for g in range(w.kv_head_num):
                    sel = [int(c) for c in idx[t0 + i, g] if 0 <= c < kv and c <= prefix + i]
                    heads = list(range(g * G, (g + 1) * G))
                    d = _list_problem(p, b, g, sel, p.query[t0 + i:t0 + i + 1, heads[0]:heads[-1] + 1])
                    od, ld = run(lib, d)
                    assert np.array_equal(od[0], o[t0 + i, heads]) and np.array_equal(ld[0], l[t0 + i, heads])
            t0 += int(ql[b])


def _list_problem(p, b, g, sel, query):
    """One sequence of KV head g's rows of tokens `sel` (in that order) of
    sequence b, copied into fresh blocks with torch indexing; one KV head."""
    w = p.workload
    n = len(sel)
    bs = w.block_size
    nblk = max(1, (n + bs - 1) // bs)
    rows_k = gather_contiguous(p, b, p.key_cache)[:, g:g + 1]
    vsrc = p.key_cache[..., :w.head_size_v] if w.shared_kv else p.value_cache
    rows_v = gather_contiguous(p, b, vsrc)[:, g:g + 1]
    ids = torch.tensor(sel, dtype=torch.long)
    def pack(rows):
        out = torch.zeros(nblk * bs, 1, rows.shape[2], dtype=rows.dtype)
        out[:n] = rows[ids] if n else out[:0]
        return out.reshape(nblk, bs, 1, rows.shape[2])
    d = synth.Problem(**{**p.__dict__})
    d.workload = synth.Workload(**{**w.__dict__, "mask": "none", "shared_kv": False,
                                   "head_num": query.shape[1], "kv_head_num": 1, "topk": 0})
    d.key_cache, d.value_cache = pack(rows_k), pack(rows_v)
    d.num_blocks = nblk
    d.block_tables_np = np.arange(nblk, dtype=np.int32)[None, :]
    d.max_num_blocks_per_seq = nblk
    d.context_lens_np = np.array([n], np.int32)
    d.q_seq_lens_np = None
    d.query = query.contiguous()
    d.topk_idx = None
    return d


def pin_sparse_lse_counts_entries(lib):
    """q = 0: exp(lse) counts the list entries that select a visible token."""
    for p in sparse_cases():
        p.query.zero_()
        _, l = run(lib, p)
        w = p.workload
        G = w.head_num // w.kv_head_num
        idx = p.topk_idx.numpy()
        ql = np.ones(p.batch, np.int64) if p.q_seq_lens_np is None else p.q_seq_lens_np.astype(np.int64)
        t0 = 0
        for b in range(p.batch):
            kv = int(p.context_lens_np[b])
            for i in range(int(ql[b])):
                lim = min(kv, max(0, kv - int(ql[b])) + i + 1)
                for h in range(w.head_num):
                    e = idx[t0 + i, h // G]
                    count = int(((e >= 0) & (e < lim)).sum())
                    got = np.exp(l[t0 + i, h])
                    assert (count == 0 and got == 0) or np.rint(got) == count, (b, i, h)
            t0 += int(ql[b])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
