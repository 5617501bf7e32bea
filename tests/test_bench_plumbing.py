"""CPU checks of bench.py's host-side plumbing (no GPU): the step kinds it can profile are defined consistently,
their FLOP and byte accounting matches the closed forms of the workloads, and the counter-derived figures come
out of the formulas the summaries state."""
import math

import pytest

import bench
from workloads import accounting as acc
from workloads.configs import CONFIGS


def test_profile_kinds_are_consistent():
    kinds = set(bench.PROFILE_TARGETS)
    assert kinds == set(bench.PROFILE_SUMMARY) == set(bench.SOURCES)
    for kind in kinds:
        child, kernels, steps, warmup = bench.PROFILE_TARGETS[kind]
        assert child and kernels and steps >= 1 and warmup >= 1
        acct = bench.profile_accounting(kind)
        assert set(acct) == set(kernels), kind
        assert len(bench.source_hash(bench.SOURCES[kind])) == 16


@pytest.mark.parametrize("kind,key", [("fwd", "causal_8k"), ("long", "causal_128k"), ("rows", "tabular_rows_150k")])
def test_forward_accounting(kind, key):
    c = CONFIGS[key]
    (fl, nbytes, _), = bench.profile_accounting(kind).values()
    assert fl == 4 * c.d * acc.config_pairs(c)
    assert nbytes == acc.attn_fwd_bytes(c.B, c.H, c.Nq, c.Nq, c.d, 2, 2)


def test_headline_flop_count():
    # causal self-attention B=4 H=32 N=8192 d=128: 4*d per visible pair, N(N+1)/2 pairs per head
    (fl, _, _), = bench.profile_accounting("fwd").values()
    assert fl == 4 * 128 * 4 * 32 * 8192 * 8193 // 2
    assert math.isclose(fl, 2.1993e12, rel_tol=1e-4)


def test_backward_accounting_is_seven_products():
    a = bench.profile_accounting("bwd")
    (dq_fl, _, _), (kv_fl, _, _) = a["attn_bwd_dq_kernel<128"], a["attn_bwd_dkdv_kernel<128"]
    pairs = 4 * 32 * acc.visible_pairs(8192, 8192, True)
    assert dq_fl == 3 * 2 * 128 * pairs and kv_fl == 4 * 2 * 128 * pairs


def test_derived_counter_figures():
    # one dispatch's counters: 8 XCDs of 1e6 active cycles each, the matrix unit busy half of them on 1024 SIMDs
    c = {"GRBM_GUI_ACTIVE": 8e6, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1024 * 1e6, "SQ_INSTS_VALU": 5e6,
         "SQ_INSTS_MFMA": 1e6, "SQ_INSTS_LDS": 1.5e6, "SQ_WAIT_INST_LDS": 1e5, "SQ_WAVE_CYCLES": 1e7}
    c2 = {"SQ_INSTS_VALU_MFMA_MOPS_BF16": 2e6, "SQ_INSTS_VALU_TRANS_F32": 1e6, "SQ_ACTIVE_INST_VALU": 1.28e8,
          "GRBM_GUI_ACTIVE": 8e6}
    f = bench.derive_sq(c, c2, kernel_ns=5e5)
    assert math.isclose(f["mfma_busy"], 0.5)
    assert math.isclose(f["clock_ghz"], 2.0)                   # 1e6 cycles in 0.5 ms
    assert math.isclose(f["valu_per_mfma"], 5.0) and math.isclose(f["lds_per_mfma"], 1.5)
    assert math.isclose(f["mfma_flop_executed"], 2e6 * 512)
    assert math.isclose(f["valu_busy"], 4 * 1.28e8 / 1024 / 1e6)
