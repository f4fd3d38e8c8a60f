"""Per-kernel timing (pa_set_timing / pa_read_timing) on the GPU.

The events on each kernel's launch report every timed pass, which passes
launched the plan and merge kernels, and positive kernel times; a timed pass
gives the same bits as an untimed one."""
import numpy as np
import pytest

from paged_kv_attention_18_amd import binding, synth

from gpu_util import log, run_hip, to_device

pytestmark = pytest.mark.gpu

F = binding

CASES = [
    # (name, problem, flags, plan kernel launched, merge kernel launched)
    ("decode_self_planned",
     lambda: synth.custom([700, 129, 2050, 5], 32, 8, 128, 128, 128, "bf16", seed=7), 0, False, True),
    ("decode_planned_valu",
     lambda: synth.custom([700, 129, 2050, 5], 32, 8, 128, 128, 128, "bf16", seed=7), F.PA_FLAG_FORCE_VALU,
     True, True),
    ("decode_short_whole_units",   # every unit whole: neither a plan nor a merge kernel
     lambda: synth.custom([116, 79, 105, 3], 32, 8, 128, 128, 16, "f16", seed=9, max_blocks=8), 0, False, False),
    ("mla_self_planned",   # the 576/512 kernel cuts its own pieces: no plan kernel
     lambda: synth.custom([700, 129, 2050, 5], 16, 1, 576, 512, 64, "bf16", seed=7), 0, False, True),
    ("causal_planned",
     lambda: synth.custom([300, 24, 900], 8, 2, 128, 128, 64, "f16", "causal", q_seq_lens=[40, 8, 200], seed=8),
     0, True, True),
    ("causal_no_split",
     lambda: synth.custom([300, 24, 900], 8, 2, 128, 128, 64, "f16", "causal", q_seq_lens=[40, 8, 200], seed=8),
     F.PA_FLAG_NO_SPLIT, True, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_timing_reports_each_kernel_and_changes_no_bits(case):
    name, make, flags, plan_expected, merge_expected = case
    log(f"timing {name}")
    p = to_device(make())
    att = binding.for_problem(p, flags=flags)
    o0, l0, _ = run_hip(p, att=att)
    binding.pa_set_timing(att.handle, 1)
    runs = [run_hip(p, att=att)[:2] for _ in range(3)]
    kms, passes, planned, per = binding.pa_read_timing(att.handle, per_pass_cap=3)
    binding.pa_set_timing(att.handle, 0)
    assert att.device_error() == 0
    assert passes == 3
    assert planned == (3 if plan_expected else 0)
    for o, l in runs:
        assert np.array_equal(o, o0, equal_nan=True) and np.array_equal(l, l0, equal_nan=True)
    for plan, attn, merge in per:
        assert 0.0 < attn < 1000.0
        assert (0.0 < plan < 1000.0) if plan_expected else plan == -1.0
        assert (0.0 < merge < 1000.0) if merge_expected else merge == 0.0
    assert kms[1] == pytest.approx(sum(r[1] for r in per), rel=1e-6)
    assert kms[2] == pytest.approx(sum(r[2] for r in per), rel=1e-6)
    # nothing is kept after a read
    kms2, passes2, _, _ = binding.pa_read_timing(att.handle)
    assert passes2 == 0 and kms2 == [0.0, 0.0, 0.0]
