"""The C-ABI library on the CPU: it loads, exports what include/pa.h declares,
and rejects bad configurations before touching the GPU."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from paged_kv_attention_18_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libpa.so is not built (run __graft_entry__.build())")
    return binding.load_library()


def good_cfg(**kw):
    c = dict(head_num=8, kv_head_num=2, head_size_k=128, head_size_v=128, block_size=128,
             num_blocks=100, max_batch=4, max_num_blocks_per_seq=8, max_q_seq_len=1,
             dtype=binding.PA_F16, scale=0.125, mask=binding.PA_MASK_NONE, flags=0, num_partitions=0)
    c.update(kw)
    return binding.pa_config(**c)


def create_status(lib, cfg):
    h = ctypes.c_void_p()
    st = lib.pa_create(ctypes.byref(cfg), ctypes.byref(h))
    if st == binding.PA_OK:
        lib.pa_destroy(h)
    return st


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ("pa_create", "pa_forward", "pa_destroy", "pa_status_string"):
        assert n in names


def test_every_declared_function_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (pa_[a-z_]+)\b", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert set(binding.EXPORTS) == set(declared_functions())


def test_config_struct_matches_header():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{(.*?)\} pa_config;", text, re.S).group(1)
    fields = re.findall(r"\b([a-z_]+)\s*;", body.replace(",", ";"))
    assert fields == [f for f, _ in binding.pa_config._fields_]


@pytest.mark.parametrize("bad", [
    dict(head_num=0), dict(kv_head_num=0), dict(head_num=6, kv_head_num=4),
    dict(head_size_k=0), dict(head_size_k=577), dict(head_size_v=600),
    dict(block_size=0), dict(block_size=24), dict(block_size=272),
    dict(block_size=256, mask=binding.PA_MASK_CAUSAL),
    dict(block_size=256, head_size_k=576, head_size_v=512),
    dict(num_blocks=0), dict(max_batch=0), dict(max_num_blocks_per_seq=0), dict(max_q_seq_len=0),
    dict(dtype=7), dict(mask=4), dict(mask=binding.PA_MASK_TENSOR),   # (no matrix given)
    dict(scale=float("inf")), dict(scale=float("nan")),
    dict(num_partitions=-1), dict(flags=binding.PA_FLAG_FORCE_VALU | binding.PA_FLAG_FORCE_MFMA),
    dict(flags=64), dict(flags=128),
    dict(flags=binding.PA_FLAG_SHARED_KV, head_size_k=64, head_size_v=128),
    dict(mask=binding.PA_MASK_BAND, window_left=-1), dict(mask=binding.PA_MASK_BAND, window_right=-5),
    dict(mask=binding.PA_MASK_BAND, window_left=(1 << 30) + 1),
    dict(mask=binding.PA_MASK_SPARSE, topk=0),
])
def test_create_rejects_invalid(lib, bad):
    assert create_status(lib, good_cfg(**bad)) == binding.PA_ERR_INVALID_ARG


@pytest.mark.parametrize("shape", [dict(head_size_k=96, head_size_v=96), dict(head_size_k=128, head_size_v=64),
                                   dict(mask=binding.PA_MASK_BAND, window_left=127,
                                        flags=binding.PA_FLAG_FORCE_VALU),
                                   dict(mask=binding.PA_MASK_CAUSAL, flags=binding.PA_FLAG_FORCE_VALU),
                                   dict(mask=binding.PA_MASK_SPARSE, topk=16)])   # G 4: not a multiple of 64
def test_create_unsupported_shape(lib, shape):
    assert create_status(lib, good_cfg(**shape)) == binding.PA_ERR_UNSUPPORTED


def test_create_null_out(lib):
    cfg = good_cfg()
    assert lib.pa_create(ctypes.byref(cfg), None) == binding.PA_ERR_INVALID_ARG


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU error path")
def test_create_without_gpu_reports_hip_error(lib):
    assert create_status(lib, good_cfg()) in (binding.PA_ERR_HIP, binding.PA_ERR_UNSUPPORTED)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU error path")
@pytest.mark.parametrize("flags", [binding.PA_FLAG_PLAN_KERNEL, binding.PA_FLAG_PLAN_KERNEL | binding.PA_FLAG_STATIC_PIECES,
                                   binding.PA_FLAG_PLAN_KERNEL | binding.PA_FLAG_NO_SPLIT])
def test_create_accepts_every_declared_flag(lib, flags):
    """Declared flags pass the configuration check (which runs before any HIP
    call); without a GPU the call then fails in HIP, not as an invalid argument."""
    assert create_status(lib, good_cfg(flags=flags)) in (binding.PA_ERR_HIP, binding.PA_ERR_UNSUPPORTED)


def test_forward_null_handle(lib):
    st = lib.pa_forward(None, 1, 1, 1, 1, 1, None, 1, 1, 1, 1, None, None)
    assert st == binding.PA_ERR_INVALID_ARG
    st = lib.pa_forward_sparse(None, 1, 1, 1, 1, 1, None, 1, 1, 1, 1, 1, None, None)
    assert st == binding.PA_ERR_INVALID_ARG


def test_other_calls_null_handle(lib):
    code = ctypes.c_uint32()
    assert lib.pa_get_device_error(None, ctypes.byref(code), 0) == binding.PA_ERR_INVALID_ARG
    assert lib.pa_set_timing(None, 1) == binding.PA_ERR_INVALID_ARG
    assert lib.pa_describe(None, 1, None, None, None, None) == binding.PA_ERR_INVALID_ARG
    assert lib.pa_destroy(None) == binding.PA_OK


def test_status_strings(lib):
    for s in range(5):
        assert lib.pa_status_string(s)
    assert binding.pa_status_string(binding.PA_ERR_INVALID_ARG) == "invalid argument"


def test_binding_refuses_missing_library(tmp_path, monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        binding.load_library(str(tmp_path / "nope.so"))


def test_product_path_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "paged_kv_attention_18_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("the oracle and the HIP path", ""), f
                assert "pa_ref" not in text, f


def test_piece_map_host_invariants(tmp_path):
    """The piece map shared by the self-planning streaming kernel and the
    merge kernel, compiled for the host from the library's own header: the
    pieces tile the item range, claimed pieces keep their minimum size and
    the count fits the workspace (tests/piece_map_host.cpp)."""
    hipcc = "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not installed")
    src = os.path.join(ROOT, "tests", "piece_map_host.cpp")
    exe = str(tmp_path / "piece_map_host")
    csrc = os.path.join(ROOT, "paged_kv_attention_18_amd", "csrc")
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17",
                    "-I", os.path.join(ROOT, "include"), "-I", csrc, src, "-o", exe],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr


def test_self_plan_matches_plan_kernel_host(tmp_path):
    """The 576/512 tile kernel's own plan, compiled for the host from the
    library's header: for 3000 seeded passes of one row tile per unit (no
    mask, causal, band, sparse lists; empty and malformed lengths; 1 to 256
    sequences; split and whole units) every worker walks the same segments,
    and every split entry is the same, as with the plan kernel's arrays
    (tests/self_plan_host.cpp)."""
    hipcc = "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not installed")
    src = os.path.join(ROOT, "tests", "self_plan_host.cpp")
    exe = str(tmp_path / "self_plan_host")
    csrc = os.path.join(ROOT, "paged_kv_attention_18_amd", "csrc")
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17",
                    "-I", os.path.join(ROOT, "include"), "-I", csrc, src, "-o", exe],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok 3000 "), r.stdout + r.stderr


def test_valu_decode_addresses_in_bounds_host(tmp_path):
    """The VALU decode kernel's addressing and the planning it runs on,
    compiled for the host from the library's own header: for the causal case
    whose GPU run once faulted and a seeded sweep (causal and unmasked,
    malformed lengths and block ids included), every query, cache, table,
    output, lse and partial access of every lane stays inside its buffer
    (tests/decode_addr_host.cpp)."""
    hipcc = "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not installed")
    src = os.path.join(ROOT, "tests", "decode_addr_host.cpp")
    exe = str(tmp_path / "decode_addr_host")
    csrc = os.path.join(ROOT, "paged_kv_attention_18_amd", "csrc")
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17",
                    "-I", os.path.join(ROOT, "include"), "-I", csrc, src, "-o", exe],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
