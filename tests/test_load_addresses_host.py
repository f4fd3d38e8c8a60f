"""Every LDS load of the matrix-core kernels, enumerated on the host
(tests/lds_load_addr_host.cpp) for the named workloads at full size, the GPU
parity tests' shapes (the random sweep's included) and caches just under and
just over 4 GiB.

Asserted: every lane's address stays inside its buffer, row and LDS stage;
the K/V and mask-slab loads split into a wave-uniform base (the kernel's own
lane-independent part: the 16-token group's row in the head, or the zero
page) and a per-lane offset below 2^32 at every shape.  Recorded as facts
that any load form with a scalar base register has to respect: the
streaming kernel's Q-tile loads mix two allocations (query rows and the zero
page) within one instruction, offsets from a head's column of the cache pass
2^31 on the long-context workload and 2^32 on caches above 4 GiB, and so do
the sparse loads' per-lane row offsets there."""
import os
import subprocess

import numpy as np
import pytest

from paged_kv_attention_18_amd import binding, synth

import test_gpu_parity as gp
import test_gpu_random_parity as rp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MODES = {"none": 0, "causal": 1, "band": 2, "tensor": 3, "sparse": 4}


def _record(name, H, Hkv, Dk, Dv, bs, mask, window, shared, topk, kv, ql, tables, nb, lists):
    kv = np.asarray(kv, np.int64)
    B = kv.shape[0]
    ql = np.ones(B, np.int64) if ql is None else np.asarray(ql, np.int64)
    tables = np.asarray(tables, np.int64).reshape(B, -1)
    head = [name, B, H, Hkv, Dk, Dv, bs, int(nb), tables.shape[1], MODES[mask], int(window[0]), int(window[1]),
            int(bool(shared)), int(topk)]
    parts = ["case " + " ".join(str(x) for x in head),
             " ".join(map(str, kv.tolist())), " ".join(map(str, ql.tolist())),
             " ".join(map(str, tables.ravel().tolist()))]
    if mask == "sparse":
        parts.append(" ".join(map(str, np.asarray(lists, np.int64).ravel().tolist())))
    return "\n".join(parts) + "\n"


def _from_problem(name, p):
    w = p.workload
    lists = p.topk_idx.numpy() if p.topk_idx is not None else None
    return _record(name, w.head_num, w.kv_head_num, w.head_size_k, w.head_size_v, w.block_size, w.mask,
                   (w.window_left, w.window_right), w.shared_kv, w.topk, p.context_lens_np, p.q_seq_lens_np,
                   p.block_tables_np, p.num_blocks, lists)


def _workloads():
    for w in synth.WORKLOADS.values():
        kv, ql, tables, nb, lists = synth.layout(w)
        yield _record(w.name, w.head_num, w.kv_head_num, w.head_size_k, w.head_size_v, w.block_size, w.mask,
                      (w.window_left, w.window_right), w.shared_kv, w.topk, kv, ql, tables, nb, lists)


def _test_shapes():
    for i, (lens, H, Hkv, D, bs, dt) in enumerate(gp.DECODE_CASES):
        yield _from_problem(f"decode{i}", synth.custom(lens, H, Hkv, D, D, bs, dt, seed=3))
    for i, (kv, ql, H, Hkv, D, bs, dt) in enumerate(gp.CAUSAL_CASES):
        yield _from_problem(f"causal{i}", synth.custom(kv, H, Hkv, D, D, bs, dt, "causal", q_seq_lens=ql, seed=11))
    for i, (lens, H, Hkv, Dk, Dv, bs, dt, mask, ql) in enumerate(gp.SHARED_CASES):
        yield _from_problem(f"shared{i}", synth.custom(lens, H, Hkv, Dk, Dv, bs, dt, mask, q_seq_lens=ql, seed=5,
                                                       shared_kv=True))
    for i, (lens, H, Hkv, Dk, Dv, bs, dt, ql, win, shared) in enumerate(gp.BAND_CASES):
        yield _from_problem(f"band{i}", synth.custom(lens, H, Hkv, Dk, Dv, bs, dt, "band", q_seq_lens=ql, seed=9,
                                                     shared_kv=shared, window=win))
    for i, (lens, H, Hkv, Dk, Dv, bs, dt, ql, shared) in enumerate(gp.TENSOR_CASES):
        yield _from_problem(f"tensor{i}", synth.custom(lens, H, Hkv, Dk, Dv, bs, dt, "tensor", q_seq_lens=ql,
                                                       seed=13, shared_kv=shared))
    for i, case in enumerate(gp.SPARSE_CASES):
        yield _from_problem(f"sparse{i}", gp._sparse_problem(case, 21))
    for i in range(rp.N_CASES):   # the seeded random sweep
        yield _from_problem(f"random{i}", rp.draw(i)[1])
    for name, B, (lo, hi), qr, H, Hkv, Dk, Dv, bs, dt, mask, win, shared, P in gp.TAIL_MODE_CASES:
        rng = np.random.default_rng(B * 7 + P)
        lens = rng.integers(lo, hi, size=B).tolist()
        ql = None if qr is None else rng.integers(qr[0], qr[1] + 1, size=B).tolist()
        yield _from_problem(f"tail_{name}", synth.custom(lens, H, Hkv, Dk, Dv, bs, dt, mask, q_seq_lens=ql, seed=17,
                                                         shared_kv=shared, window=win))


def _near_4gib():
    """Caches just under and just over 4 GiB, the sequences' blocks at the top
    of the pool (arithmetic only: nothing is allocated)."""
    def top_tables(kv, bs, nb):
        need = [(k + bs - 1) // bs for k in kv]
        t = np.zeros((len(kv), max(need)), np.int64)
        nxt = nb - 1
        for b, n in enumerate(need):
            for j in range(n):
                t[b, j] = nxt
                nxt -= 1
        return t

    for label, Hkv, Dk, Dv, H, shared in (("gqa", 8, 128, 128, 64, False), ("mla", 1, 576, 512, 64, False),
                                          ("mla_shared", 1, 576, 512, 64, True)):
        row = 128 * Hkv * Dk * 2   # K bytes per block
        for side, nb in (("under", (1 << 32) // row), ("over", (1 << 32) // row + 2)):
            kv = [32768, 4097, 300, 1]
            yield _record(f"{label}_{side}_4GiB", H, Hkv, Dk, Dv, 128, "none", (0, 0), shared, 0, kv, None,
                          top_tables(kv, 128, nb), nb, None)
    # sparse lists into a cache above 4 GiB (64 query heads on one K/V head)
    row = 128 * 576 * 2
    nb = (1 << 32) // row + 2
    kv = [30000, 2000]
    t = top_tables(kv, 128, nb)
    rng = np.random.default_rng(5)
    lists = np.stack([rng.choice(k, size=512, replace=False) for k in kv]).reshape(2, 1, 512)
    yield _record("sparse_over_4GiB", 64, 1, 576, 512, 128, "sparse", (0, 0), True, 512, kv, None, t, nb, lists)


def _parse(out):
    rows = {}
    for line in out.splitlines():
        if not (line.startswith("case ") or line.startswith("total")):
            continue
        tok = line.split()
        key = (tok[1], tok[3]) if tok[0] == "case" else ("total", "")
        stats, cur, i = {}, None, 4 if tok[0] == "case" else 1
        while i < len(tok):
            if tok[i] in ("kv", "q", "mask"):
                cur = stats.setdefault(tok[i], {})
                i += 1
            else:
                cur[tok[i]] = int(tok[i + 1])
                i += 2
        rows[key] = stats
    return rows


@pytest.fixture(scope="module")
def enumeration(tmp_path_factory):
    hipcc = "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not installed")
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libpa.so is not built (run __graft_entry__.build())")
    d = tmp_path_factory.mktemp("lds_loads")
    cases = d / "cases.txt"
    with open(cases, "w") as f:
        for gen in (_workloads, _test_shapes, _near_4gib):
            for rec in gen():
                f.write(rec)
    exe = str(d / "lds_load_addr_host")
    pkg = os.path.dirname(binding.LIB_PATH)
    csrc = os.path.join(ROOT, "paged_kv_attention_18_amd", "csrc")
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17",
                    "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    os.path.join(ROOT, "tests", "lds_load_addr_host.cpp"), "-o", exe,
                    "-L", pkg, "-lpa", "-Wl,-rpath," + pkg], check=True, capture_output=True, text=True)
    r = subprocess.run([exe, str(cases)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "\nok " in r.stdout, r.stdout[-3000:] + r.stderr[-2000:]
    return _parse(r.stdout)


def test_every_lds_load_in_bounds_and_group_split_fits(enumeration):
    """Bounds hold everywhere (the enumeration fails otherwise); below 4 GiB
    of cache every K/V and mask-slab instruction splits into one base shared
    by its 64 lanes and offsets below 2^32."""
    seen = set()
    for k, s in enumeration.items():
        if k[0] == "total" or k[0].endswith("_over_4GiB"):
            continue
        for kind in ("kv", "mask"):
            assert s[kind]["group_nonuniform"] == 0, (k, kind)
            assert s[kind]["group_off_range"] == 0, (k, kind)
            if s[kind]["instr"]:
                seen.add(kind)
        if not k[0].startswith("sparse"):   # the group's 16 token rows at most
            assert s["kv"]["group_max"] < 16 * 8 * 576 * 2, k
    assert seen == {"kv", "mask"}


def test_scalar_base_facts(enumeration):
    rows = {k: s for k, s in enumeration.items() if k[0] != "total"}
    # Q tiles of the streaming kernel: the rows of a unit past its last row
    # read the zero page, in the same instruction as real rows wherever the
    # unit's rows end inside one instruction's rows (1 KiB: 8 rows of 64
    # elements, 4 of 128, 2 of 256) -- the small decode workload (4 rows of
    # 64) and one-row units of head size 256; never where the rows end on an
    # instruction's boundary (4 rows of 128: the GQA decode workload)
    mixed = {k[0] for k, s in rows.items() if s["q"]["multi_buf"] > 0}
    assert {"tiny_decode", "decode0", "decode3"} <= mixed
    assert "gqa_decode" not in mixed and "skewed_long_decode" not in mixed
    # long-context workload: offsets from the head's column reach 2^31, not 2^32
    skew = [s for k, s in rows.items() if k[0] == "skewed_long_decode"]
    assert skew and all(s["kv"]["head_ge31"] > 0 and s["kv"]["head_ge32"] == 0 for s in skew)
    # caches above 4 GiB: offsets from the head's column pass 2^32 (just under
    # 4 GiB they do not); so do the sparse loads' per-lane row offsets
    over = [k for k in rows if k[0].endswith("_over_4GiB")]
    under = [k for k in rows if k[0].endswith("_under_4GiB")]
    assert over and under
    for k in over:
        assert rows[k]["kv"]["head_ge32"] > 0, k
    for k in under:
        assert rows[k]["kv"]["head_ge32"] == 0, k
    for k in over:
        if k[0] == "sparse_over_4GiB":
            assert rows[k]["kv"]["group_off_range"] > 0, k
        else:
            assert rows[k]["kv"]["group_off_range"] == 0 and rows[k]["kv"]["group_nonuniform"] == 0, k
