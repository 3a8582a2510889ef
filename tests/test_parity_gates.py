"""The code-parity gate itself, on the CPU: codes decided by an independent fp32
evaluation pass it; a code moved by one step away from a near-tie, or by two
steps anywhere, fails it ("H3 Streamed Blocks" node page, Inputs table,
kv_store row: int8 codes with one fp16 scale per row; the only freedom is the
rounding of values that sit at a half-step)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import assert_quantize_ok, quantize_report
from test_oracle_kvi8r import _fp32_code_variable


def _case(n=2048):
    bits = synth.head_bf16(synth.WORKLOADS["outlier16k"], "k", 0)[:n]
    x = oracle.bf16_to_f64(bits)
    v32, y, s_bits = _fp32_code_variable(x)
    codes = np.clip(np.rint(v32), -127, 127).astype(np.int8)
    return bits, codes, s_bits, y


def test_fp32_evaluated_codes_pass():
    bits, codes, s_bits, _ = _case()
    assert_quantize_ok(quantize_report(bits, codes, s_bits))


def test_one_step_off_a_tie_fails():
    bits, codes, s_bits, y = _case()
    v = y / oracle.f16_to_f64(s_bits)[:, None]
    far = np.argmax(np.abs(v - np.rint(v)) < 0.4)  # a value well away from any half-step
    bad = codes.copy().reshape(-1)
    bad[far] += 1 if bad[far] < 127 else -1
    rep = quantize_report(bits, bad.reshape(codes.shape), s_bits)
    assert rep["code_mismatch_off_tie"] == 1
    with pytest.raises(AssertionError):
        assert_quantize_ok(rep)


def test_two_steps_at_a_tie_fails():
    bits, codes, s_bits, y = _case()
    w = oracle.fp32_decision_width(oracle.bf16_to_f64(bits), s_bits)
    ties = np.argwhere(oracle.near_ties(y, s_bits, w))
    assert len(ties) > 0
    r, c = ties[0]
    bad = codes.copy()
    bad[r, c] = np.clip(int(bad[r, c]) + 2 * (1 if bad[r, c] < 0 else -1), -127, 127)
    with pytest.raises(AssertionError):
        assert_quantize_ok(quantize_report(bits, bad, s_bits))


def test_scale_two_ulps_off_fails():
    bits, codes, s_bits, _ = _case()
    bad = s_bits.copy()
    bad[5] += 2
    with pytest.raises(AssertionError):
        assert_quantize_ok(quantize_report(bits, codes, bad))


def _bf16_bits(a):
    return synth.bf16_bits_from_f32(np.asarray(a, np.float32))


def test_oracle_pool_jobs_and_per_head_gate():
    # Spawned workers regenerate each head's inputs and return error statistics.  The "GPU" rows here are
    # the oracle's own output rounded to bf16, so every head passes; rows of another head fail that head.
    from parity import OraclePool, assert_attention_ok, attention_job, quantize_job, reference_rows

    w = synth.WORKLOADS["tiny"]
    rows = synth.sampled_rows(w, 0, 64)
    good = [_bf16_bits(reference_rows("exact", w, h, rows)) for h in range(w.heads)]
    specs = [{"kind": "exact", "workload": w, "head": h, "rows": rows, "got": good[h]} for h in range(w.heads)]
    pool = OraclePool(2)
    try:
        res = pool.map(attention_job, specs)
        s = assert_attention_ok(res, "exact")
        assert s["rows"] == 64 * w.heads and 0 < s["rel_l2"] < 2e-3
        specs[1]["got"] = good[0]
        with pytest.raises(AssertionError):
            assert_attention_ok(pool.map(attention_job, specs), "exact")
        x = synth.head_bf16(w, "k", 1)
        codes, s_bits, _ = oracle.quantize_rows(oracle.bf16_to_f64(x))
        rep = pool.map(quantize_job, [{"workload": w, "tensor": "k", "head": 1, "codes": codes, "scales": s_bits}])[0]
        assert_quantize_ok(rep)
        assert rep["code_mismatch_same_scale"] == 0 and rep["head"] == 1
    finally:
        pool.close()
