"""GPU parity of kvi8r_quantize (through the C ABI) against the oracle.

Codes must equal the oracle's with at most 1e-4 of them off by one (rounding
ties), scales within 1 fp16 ulp; closed forms bit-exact; a store built in
kv_chunk pieces equals a one-shot build bitwise ("H3 Streamed Blocks" node
page, Inputs table, kv_chunk and kv_store rows).
"""
import numpy as np
import pytest
import torch

import oracle
import store_kvi8r_quantize_amd as h3a
import synth
from gpu_common import assert_quantize_ok, gpu_inputs, gpu_u16, host_u16, quantize_report, say

pytestmark = pytest.mark.gpu


def _quantize(x_bits_tok_major):
    """x: uint16 [n, H, 128] -> (codes [H, n, 128], scale bits [H, n])."""
    n, nh, _ = x_bits_tok_major.shape
    x = gpu_u16(x_bits_tok_major)
    codes = torch.empty((nh, n, 128), dtype=torch.int8, device="cuda")
    scales = torch.empty((nh, n), dtype=torch.float16, device="cuda")
    h3a.h3a_kv_quantize(x, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), host_u16(scales)


def test_closed_forms_bit_exact():
    h = oracle.sylvester_hadamard()
    rows = []
    for j in (0, 1, 77, 127):
        r = np.zeros(128, np.float32)
        r[j] = 1.0
        rows.append(r)
    for i in (0, 5, 64, 127):
        rows.append(h[i].astype(np.float32))
    rows.append(np.zeros(128, np.float32))
    big = np.zeros(128, np.float32)
    big[0] = 2.0 ** 30
    rows += [big, -big]
    x = synth.bf16_bits_from_f32(np.stack(rows))[:, None, :]
    codes, scales = _quantize(x)
    codes, scales = codes[0], scales[0]
    for n, j in enumerate((0, 1, 77, 127)):
        assert scales[n] == 0x11B4
        assert np.array_equal(codes[n].astype(np.int64), 127 * h[j])
    for n, i in enumerate((0, 5, 64, 127)):
        want = np.zeros(128, np.int8)
        want[i] = 127
        assert scales[4 + n] == 0x2DB4 and np.array_equal(codes[4 + n], want)
    assert scales[8] == 0 and not codes[8].any()
    assert scales[9] == 0x7BFF and np.all(codes[9] == 127)
    assert scales[10] == 0x7BFF and np.all(codes[10] == -127)


@pytest.mark.parametrize("name", ["tiny", "outlier16k"])
@pytest.mark.parametrize("tensor", ["k", "v"])
def test_parity_all_rows(name, tensor):
    w = synth.WORKLOADS[name]
    x = synth.qkv_bf16(w, (tensor,))[tensor]
    codes, scales = _quantize(x)
    for h in range(w.heads):
        rep = quantize_report(x[:, h], codes[h], scales[h])
        say(name, tensor, h, rep)
        assert_quantize_ok(rep)


def test_chunked_build_equals_one_shot_and_leaves_other_rows():
    w = synth.WORKLOADS["outlier16k"]
    x = synth.qkv_bf16(w, ("k",))["k"][:5000]
    xg = gpu_u16(x)
    nh = w.heads
    one_c = torch.empty((nh, 5000, 128), dtype=torch.int8, device="cuda")
    one_s = torch.empty((nh, 5000), dtype=torch.float16, device="cuda")
    h3a.h3a_kv_quantize(xg, one_c, one_s)
    # ragged chunks into a larger store pre-filled with a sentinel
    s_total = 5200
    cc = torch.full((nh, s_total, 128), 0x55, dtype=torch.int8, device="cuda")
    cs = torch.full((nh, s_total), -7.0, dtype=torch.float16, device="cuda")
    for t0 in range(0, 5000, 1000 - 23):
        t1 = min(t0 + 977, 5000)
        h3a.h3a_kv_quantize(xg[t0:t1], cc, cs, token_offset=100 + t0)
    torch.cuda.synchronize()
    assert torch.equal(cc[:, 100:5100], one_c)
    assert np.array_equal(host_u16(cs[:, 100:5100]), host_u16(one_s))
    assert bool((cc[:, :100] == 0x55).all()) and bool((cc[:, 5100:] == 0x55).all())
    assert bool((cs[:, :100] == -7.0).all()) and bool((cs[:, 5100:] == -7.0).all())


def test_strided_input_from_fused_buffer():
    w = synth.WORKLOADS["tiny"]
    x = synth.qkv_bf16(w, ("k",))["k"]
    n, nh, _ = x.shape
    fused = torch.zeros((n, 3, nh, 128), dtype=torch.bfloat16, device="cuda")
    fused[:, 1] = gpu_u16(x)
    codes = torch.empty((nh, n, 128), dtype=torch.int8, device="cuda")
    scales = torch.empty((nh, n), dtype=torch.float16, device="cuda")
    h3a.h3a_kv_quantize(fused[:, 1], codes, scales)
    c_ref, s_ref = _quantize(x)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(host_u16(scales), s_ref)


def test_rejects_buffer_too_small():
    x = torch.zeros((128, 2, 128), dtype=torch.bfloat16, device="cuda")
    codes = torch.empty((2, 100, 128), dtype=torch.int8, device="cuda")
    scales = torch.empty((2, 100), dtype=torch.float16, device="cuda")
    with pytest.raises(h3a.H3AError, match="exceeds"):
        h3a.h3a_kv_quantize(x, codes, scales)
    # a view that claims more rows than its allocation holds is caught by the range check
    lib = h3a.library()
    rc = lib.h3a_kv_quantize(x.data_ptr(), 256, 128, 2, 128, 0, 100000, codes.data_ptr(), scales.data_ptr(),
                             None)
    assert rc == -1 and "allocation" in lib.h3a_last_error().decode()


def test_host_pointer_rejected():
    lib = h3a.library()
    host = torch.zeros((64, 1, 128), dtype=torch.bfloat16)
    codes = torch.empty((1, 64, 128), dtype=torch.int8, device="cuda")
    scales = torch.empty((1, 64), dtype=torch.float16, device="cuda")
    rc = lib.h3a_kv_quantize(host.data_ptr(), 128, 64, 1, 128, 0, 64, codes.data_ptr(), scales.data_ptr(), None)
    assert rc == -1 and "device memory" in lib.h3a_last_error().decode()


@pytest.mark.timeout(900)
def test_long217k_full_store_all_heads(oracle_pool):
    # codes and scales of every row of all 32 heads of K and of V, built kv_chunk by kv_chunk
    from parity import quantize_job

    w = synth.WORKLOADS["long217k"]
    for tensor in ("k", "v"):
        xg = gpu_inputs(w, (tensor,))[tensor]
        codes = torch.empty((w.heads, w.seq, 128), dtype=torch.int8, device="cuda")
        scales = torch.empty((w.heads, w.seq), dtype=torch.float16, device="cuda")
        for t0 in range(0, w.seq, w.q_chunk):  # kv_chunk = 16384, 13 full chunks + a 4096 tail
            h3a.h3a_kv_quantize(xg[t0:t0 + w.q_chunk], codes, scales, token_offset=t0)
        torch.cuda.synchronize()
        del xg
        specs = [{"workload": w, "tensor": tensor, "head": h, "codes": codes[h].cpu().numpy(),
                  "scales": host_u16(scales[h])} for h in range(w.heads)]
        del codes, scales
        worst = {}
        for rep in oracle_pool.ex.map(quantize_job, specs):
            say("long217k", tensor, rep)
            assert_quantize_ok(rep)
            for k in ("scale_rows_differ", "code_mismatch_same_scale", "code_mismatch_off_tie"):
                worst[k] = worst.get(k, 0) + rep[k]
        say("long217k", tensor, "all heads", worst)


@pytest.mark.parametrize("grouped", [False, True])
@pytest.mark.parametrize("n_heads", [3, 5, 12, 20])
def test_head_counts_off_the_block_size(n_heads, grouped):
    # Workgroups cover 8 tokens x 8 heads; head counts that leave a partial head block, written at a token
    # offset into a larger store filled with a sentinel: every row against the oracle, nothing else touched.
    n, off, total = 333, 17, 400
    w = synth.Workload("heads", n, n_heads, 60 + n_heads, 256, 0)
    x = synth.qkv_bf16(w, ("k",))["k"]
    g = 4 if grouped else 1
    codes = torch.full((n_heads, total, 128), 99, dtype=torch.int8, device="cuda")
    scales = torch.full((n_heads, total, g) if grouped else (n_heads, total), 3.0, dtype=torch.float16, device="cuda")
    h3a.h3a_kv_quantize(gpu_u16(x), codes, scales, token_offset=off)
    torch.cuda.synchronize()
    cg, sg = codes.cpu().numpy(), host_u16(scales)
    outside = np.r_[0:off, off + n:total]
    assert np.all(cg[:, outside] == 99) and np.all(sg[:, outside] == 0x4200)  # fp16 3.0
    for h in range(n_heads):
        sh = sg[h, off:off + n].reshape(n, 4) if grouped else sg[h, off:off + n]
        assert_quantize_ok(quantize_report(x[:, h], cg[h, off:off + n], sh, group=32 if grouped else 128))


@pytest.mark.parametrize("n_heads", [32, 5])
def test_pair_equals_two_single_calls(n_heads):
    # K and V of each chunk in one launch: bitwise the codes and scales of one call per tensor, chunk by chunk
    # (ragged chunks, at a token offset, a partial head block for 5 heads), from slices of a fused QKV buffer.
    n, off, total = 3000, 40, 3100
    w = synth.Workload("pair", n, n_heads, 70 + n_heads, 256, 0, k_outliers=True)
    bits = synth.qkv_bf16(w, ("k", "v"))
    fused = torch.zeros((n, 3, n_heads, 128), dtype=torch.bfloat16, device="cuda")
    fused[:, 1], fused[:, 2] = gpu_u16(bits["k"]), gpu_u16(bits["v"])
    kc = torch.full((n_heads, total, 128), 7, dtype=torch.int8, device="cuda")
    vc = torch.full((n_heads, total, 128), 7, dtype=torch.int8, device="cuda")
    sc = torch.full((2, n_heads, total), 5.0, dtype=torch.float16, device="cuda")
    kc1, vc1, sc1 = kc.clone(), vc.clone(), sc.clone()
    for t0 in range(0, n, 1024):
        t1 = min(t0 + 1024, n)
        h3a.h3a_kv_quantize_pair(fused[t0:t1, 1], fused[t0:t1, 2], kc, vc, sc, token_offset=off + t0)
        h3a.h3a_kv_quantize(fused[t0:t1, 1], kc1, sc1[0], token_offset=off + t0)
        h3a.h3a_kv_quantize(fused[t0:t1, 2], vc1, sc1[1], token_offset=off + t0)
    torch.cuda.synchronize()
    assert torch.equal(kc, kc1) and torch.equal(vc, vc1)
    assert torch.equal(sc.view(torch.int16), sc1.view(torch.int16))
    assert bool((kc[:, :off] == 7).all()) and bool((sc[:, :, off + n:] == 5.0).all())
    for h in (0, n_heads - 1):
        assert_quantize_ok(quantize_report(bits["v"][:, h], vc[h, off:off + n].cpu().numpy(),
                                           host_u16(sc[1, h, off:off + n])))


def _mixed_scale_rows(rng) -> np.ndarray:
    """bf16 bits [64, 128]: four waves of 16 rows.  Wave 0: N(0,1) rows (normal scales, no clamp).
    Wave 1: N(0,1) rows and one row whose fp16 scale is subnormal and rounded far down (one-hot
    magnitude 1.4 subnormal steps), so |y/s| reaches ~178 and the code must clamp to 127.  Wave 2:
    rows scaled so that their scales run through the subnormal range and across the smallest normal.
    Wave 3: zero rows, a saturating row of each sign and N(0,1) rows."""
    rows = rng.standard_normal((64, 128)).astype(np.float32)
    unit = 2.0 ** -24 * 127 * np.sqrt(128.0)  # max|y| of a one-hot row of this magnitude puts s at 1 step
    hot = np.zeros(128, np.float32)
    hot[37] = 1.4 * unit
    rows[20] = hot
    rows[32:48] *= (np.float32(2.0) ** -np.linspace(8, 26, 16).astype(np.float32))[:, None]
    rows[48:51] = 0.0
    rows[51] = 0.0
    rows[51, 5] = 2.0 ** 28
    rows[52] = -rows[51]
    return synth.bf16_bits_from_f32(rows)


@pytest.mark.parametrize("grouped", [False, True])
def test_clamp_decision_in_mixed_waves(grouped):
    # Codes skip the clamp only when every row of the wave has a normal fp16 scale below the largest;
    # rows around those limits, mixed in one wave with ordinary rows, must still match the oracle.
    x = _mixed_scale_rows(np.random.default_rng(21))
    xg = gpu_u16(x[:, None, :])
    codes = torch.empty((1, 64, 128), dtype=torch.int8, device="cuda")
    scales = torch.empty((1, 64, 4) if grouped else (1, 64), dtype=torch.float16, device="cuda")
    h3a.h3a_kv_quantize(xg, codes, scales)
    torch.cuda.synchronize()
    got_c, got_s = codes.cpu().numpy()[0], host_u16(scales)[0]
    rep = quantize_report(x, got_c, got_s, group=32 if grouped else 128)
    say("mixed scales", "grouped" if grouped else "per row", rep)
    assert_quantize_ok(rep)
    if not grouped:
        assert got_s[20] == 1 and np.abs(got_c[20].astype(np.int64)).max() == 127  # clamped subnormal-scale row
        assert (got_s[32:48] < 0x0400).any() and (got_s[32:48] >= 0x0400).any()  # both sides of the smallest normal
        assert not got_c[48:51].any() and not got_s[48:51].any()
        assert got_s[51] == 0x7BFF and got_s[52] == 0x7BFF
