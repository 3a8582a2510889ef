"""GPU parity of the query rotation and output un-rotation kernels (through the
C ABI hooks) against the oracle's explicit Hadamard product ("H3 Streamed
Blocks" node page, Inputs table, kv_store row; "Low VRAM, low RAM", "The K/V
store options", rotation paragraph)."""
import numpy as np
import pytest
import torch

import oracle
import store_kvi8r_quantize_amd as h3a
import synth
from gpu_common import gpu_u16, host_u16, say

pytestmark = pytest.mark.gpu


def _ulp_dist(a_vals, b_vals, ulp_of):
    return np.abs(a_vals - b_vals) / ulp_of(np.maximum(np.abs(a_vals), np.abs(b_vals)))


def _f16_ulp(x):
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def _bf16_ulp(x):
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("n_rows", [1, 63, 4096 * 8 + 5])
def test_rotate_rows(n_rows):
    w = synth.WORKLOADS["outlier16k"]
    x = synth.qkv_bf16(w, ("q",))["q"].reshape(-1, 128)[:n_rows]
    y = torch.empty((n_rows, 128), dtype=torch.float16, device="cuda")
    h3a.h3a_rotate_rows(gpu_u16(x), y)
    got = oracle.f16_to_f64(host_u16(y))
    ref = oracle.rotate_rows(oracle.bf16_to_f64(x))
    ref16 = oracle.f16_to_f64(oracle.f64_to_f16_bits(ref))
    exact = np.mean(got == ref16)
    dist = _ulp_dist(got, ref, _f16_ulp)
    say("rotate", n_rows, "bit-exact frac", exact, "max ulp", dist.max())
    assert dist.max() <= 1.0
    assert exact >= 0.999


@pytest.mark.parametrize("n_rows", [1, 100, 50001])
def test_unrotate_rows(n_rows):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((n_rows, 128)).astype(np.float32)
    y = torch.empty((n_rows, 128), dtype=torch.bfloat16, device="cuda")
    h3a.h3a_unrotate_rows(torch.from_numpy(x).cuda(), y)
    got = oracle.bf16_to_f64(host_u16(y))
    ref = oracle.rotate_rows(x.astype(np.float64))  # H^T = H
    # fp32 butterflies on fp32 inputs: besides the final bf16 rounding (<= 1 ulp with
    # the fp32 error), an absolute error of a few fp32 ulps of the row's magnitude,
    # which dominates for outputs that cancel to nearly zero.
    fp32_abs = 8 * 2.0 ** -24 * np.abs(x).astype(np.float64).sum(axis=1, keepdims=True) / np.sqrt(128)
    excess = np.abs(got - ref) - _bf16_ulp(np.abs(ref))
    say("unrotate", n_rows, "max ulp", _ulp_dist(got, ref, _bf16_ulp).max(), "max excess / fp32 bound",
        (excess / fp32_abs).max())
    assert np.all(excess <= fp32_abs)


def test_rotation_round_trip():
    # un-rotating a rotated row returns it (up to fp16 / bf16 rounding)
    w = synth.WORKLOADS["tiny"]
    x = synth.qkv_bf16(w, ("q",))["q"].reshape(-1, 128)
    y = torch.empty(x.shape, dtype=torch.float16, device="cuda")
    h3a.h3a_rotate_rows(gpu_u16(x), y)
    back = torch.empty(x.shape, dtype=torch.bfloat16, device="cuda")
    h3a.h3a_unrotate_rows(y.float(), back)
    d = oracle.bf16_to_f64(host_u16(back)) - oracle.bf16_to_f64(x)
    assert np.abs(d).max() <= 2e-2 and np.sqrt(np.mean(d ** 2)) < 2e-3


def test_zero_rows():
    y = torch.empty((0, 128), dtype=torch.float16, device="cuda")
    h3a.h3a_rotate_rows(torch.empty((0, 128), dtype=torch.bfloat16, device="cuda"), y)
    z = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda")
    y = torch.ones((64, 128), dtype=torch.float16, device="cuda")
    h3a.h3a_rotate_rows(z, y)
    assert not bool(y.any())
