"""The C-ABI library loads, exports every function include/h3a.h declares, and
rejects bad arguments on the host before any GPU work (CPU only: no call here
reaches the HIP runtime)."""
import ctypes
import os
import re

import pytest

import store_kvi8r_quantize_amd as h3a

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3a.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(h3a_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(h3a.LIB_PATH):
        pytest.fail("libh3a.so is not built (run __graft_entry__.build())")
    return h3a.library()


def test_header_declares_the_entry_points():
    names = _declared()
    for need in ("h3a_kv_quantize", "h3a_attention", "h3a_attention_routed", "h3a_attention_workspace_bytes",
                 "h3a_abi_version", "h3a_last_error", "h3a_rotate_rows", "h3a_unrotate_rows"):
        assert need in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_abi_version(lib):
    assert lib.h3a_abi_version() == h3a.ABI_VERSION


def _attn(lib, **kw):
    a = dict(q=None, k=None, v=None, scales=None, s_q=1024, s_kv=1024, n_heads=2, head_dim=128, scale=0.088,
             q_chunk=256, kv_block=0, mode=1, mask=None, out=None, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.h3a_attention(a["q"], a["k"], a["v"], a["scales"], a["s_q"], a["s_kv"], a["n_heads"],
                             a["head_dim"], a["scale"], a["q_chunk"], a["kv_block"], a["mode"], a["mask"],
                             a["out"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status,msg", [
    (dict(head_dim=64), -2, "head_dim"),
    (dict(mode=7), -1, "mode"),
    (dict(mode=3), -1, "mode"),
    (dict(mode=2, scales=None), -1, "scales"),
    (dict(n_heads=0), -1, "n_heads"),
    (dict(n_heads=65537), -1, "n_heads"),
    (dict(s_kv=1 << 31), -1, "sequence too long"),
    (dict(s_q=(1 << 31) + 1), -1, "sequence too long"),
    (dict(s_q=-1), -1, "s_q"),
    (dict(q_chunk=0), -1, "q_chunk"),
    (dict(kv_block=100), -1, "kv_block"),
    (dict(kv_block=-64), -1, "kv_block"),
    (dict(scale=0.0), -1, "softmax_scale"),
    (dict(scale=float("nan")), -1, "softmax_scale"),
    (dict(mask=1, q_chunk=100), -1, "multiple of 64"),
    (dict(mode=1, scales=None), -1, "scales"),
    (dict(mode=0, scales=16), -1, "no scales"),
    (dict(mode=0x100 | 1, scales=16), -1, "H3A_SOL needs a tile_mask"),
    (dict(mode=0x100 | 7, mask=1), -1, "mode"),
    (dict(mode=0x400 | 1, mask=1, scales=16), -1, "mode"),
    (dict(mode=0x200 | 0), -1, "H3A_OUT_F16"),
    (dict(mode=0x200 | 0x100 | 0, mask=1), -1, "H3A_OUT_F16"),
    (dict(mode=0x100 | 1, mask=1, scales=16, s_kv=(1 << 30) - 63), -1, "2^30 - 64"),
    (dict(mode=2, scales=16, scale=0.7), -1, "softmax_scale <= ln 2"),
    (dict(mode=0x200 | 2, scales=16, scale=2.0), -1, "softmax_scale <= ln 2"),
])
def test_attention_rejects_bad_arguments(lib, kw, status, msg):
    assert _attn(lib, **kw) == status
    assert msg in lib.h3a_last_error().decode()


def test_attention_empty_query_is_noop(lib):
    assert _attn(lib, s_q=0, scales=16) == 0


def _routed(lib, spans, **kw):
    import ctypes

    a = dict(s_q=1024, s_kv=1024, n_heads=2, head_dim=128, scale=0.088, q_chunk=256, kv_block=0, scales=16)
    a.update(kw)
    flat = [x for sp in (spans or []) for x in sp]
    arr = (ctypes.c_int64 * max(len(flat), 1))(*flat) if spans is not None else None
    n = kw.get("n_spans", len(flat) // 2)
    return lib.h3a_attention_routed(None, None, None, None, None, a["scales"], a["s_q"], a["s_kv"], a["n_heads"],
                                    a["head_dim"], a["scale"], a["q_chunk"], a["kv_block"], arr, n, None, None, 0,
                                    None)


@pytest.mark.parametrize("spans,kw,status,msg", [
    ([(0, 64)], dict(head_dim=64), -2, "head_dim"),
    ([(10, 5)], {}, -1, "exact span 0"),
    ([(0, 100), (50, 200)], {}, -1, "exact span 1"),
    ([(0, 100), (900, 1025)], {}, -1, "exact span 1"),
    ([(-1, 10)], {}, -1, "exact span 0"),
    (None, dict(n_spans=2), -1, "exact_spans"),
    ([(0, 10)], dict(n_spans=-1), -1, "exact_spans"),
    ([(0, 64)], dict(scales=None), -1, "scales"),
    ([(0, 64)], dict(q_chunk=0), -1, "q_chunk"),
])
def test_routed_rejects_bad_arguments(lib, spans, kw, status, msg):
    assert _routed(lib, spans, **kw) == status
    assert msg in lib.h3a_last_error().decode()


def test_routed_empty_query_is_noop(lib):
    assert _routed(lib, [(0, 0)], s_q=0) == 0


@pytest.mark.parametrize("kw,status,msg", [
    (dict(head_dim=96), -2, "head_dim"),
    (dict(n_heads=0), -1, "n_heads"),
    (dict(token_offset=1000, n_tokens=100, s_total=1024), -1, "exceeds"),
    (dict(stride=100), -1, "x_token_stride"),
    (dict(n_tokens=-5), -1, ">= 0"),
])
def test_quantize_rejects_bad_arguments(lib, kw, status, msg):
    a = dict(x=None, stride=256, n_tokens=64, n_heads=2, head_dim=128, token_offset=0, s_total=64, codes=None,
             scales=None, stream=None)
    a.update(kw)
    rc = lib.h3a_kv_quantize(a["x"], a["stride"], a["n_tokens"], a["n_heads"], a["head_dim"], a["token_offset"],
                             a["s_total"], a["codes"], a["scales"], a["stream"])
    assert rc == status
    assert msg in lib.h3a_last_error().decode()


def test_quantize_zero_tokens_is_noop(lib):
    assert lib.h3a_kv_quantize(None, 256, 0, 2, 128, 0, 0, None, None, None) == 0


def test_quantize_g32_rejects_bad_arguments(lib):
    assert lib.h3a_kv_quantize_g32(None, 256, 64, 2, 96, 0, 64, None, None, None) == -2
    assert lib.h3a_kv_quantize_g32(None, 256, 64, 2, 128, 10, 64, None, None, None) == -1
    assert "exceeds" in lib.h3a_last_error().decode()
    assert lib.h3a_kv_quantize_g32(None, 256, 0, 2, 128, 0, 0, None, None, None) == 0


@pytest.mark.parametrize("kw,status,msg", [
    (dict(head_dim=64), -2, "head_dim"),
    (dict(mode=3), -1, "mode"),
    (dict(mode=0x200 | 0, scales=None), -1, "H3A_OUT_F16"),
    (dict(mode=0x100 | 1), -1, "mode"),
    (dict(mode=1, scales=None), -1, "scales"),
    (dict(mode=0, scales=16), -1, "no scales"),
    (dict(kv_block=100), -1, "kv_block"),
    (dict(q_chunk=0), -1, "q_chunk"),
    (dict(mode=2, scale=0.7), -1, "softmax_scale <= ln 2"),
])
def test_host_kv_rejects_bad_arguments(lib, kw, status, msg):
    a = dict(s_q=1024, s_kv=1024, n_heads=2, head_dim=128, scale=0.088, q_chunk=256, kv_block=256, mode=1, scales=16)
    a.update(kw)
    rc = lib.h3a_attention_host_kv(None, None, None, a["scales"], a["s_q"], a["s_kv"], a["n_heads"], a["head_dim"],
                                   a["scale"], a["q_chunk"], a["kv_block"], a["mode"], None, None, 0, None)
    assert rc == status
    assert msg in lib.h3a_last_error().decode()


def test_host_kv_workspace_sizes():
    dense = h3a.h3a_attention_workspace_bytes(1024, 1000, 2, 256, "kvi8r", False)
    staged = h3a.h3a_attention_host_kv_workspace_bytes(1024, 1000, 2, 256, 256, "kvi8r")
    state = 1 * 2 * 512 * 66 * 4                      # one query chunk of 256 rows, 2 heads
    blocks = 2 * (2 * 256 * 2 * 128 + 2 * 256 * 2 * 2)  # two buffers: K, V codes + their scales for 256 tokens
    assert staged >= dense + state + blocks
    assert h3a.h3a_attention_host_kv_workspace_bytes(1024, 1000, 2, 256, 100, "kvi8r") == 0
    # kv_block 0 = 16384, clipped to the store
    assert h3a.h3a_attention_host_kv_workspace_bytes(1024, 1000, 2, 256, 0, "exact") == \
        h3a.h3a_attention_host_kv_workspace_bytes(1024, 1000, 2, 256, 1024, "exact")


def test_workspace_sizes(lib):
    # kvi8r: rotated Q (fp16) + rotated output (fp32) for one chunk of rows
    assert h3a.h3a_attention_workspace_bytes(1024, 1024, 2, 256, "kvi8r", False) == 256 * 2 * 128 * 6
    assert h3a.h3a_attention_workspace_bytes(1024, 1024, 2, 256, "exact", False) == 0
    assert h3a.h3a_attention_workspace_bytes(1024, 1024, 2, 256, "kvi8r32", False) == 256 * 2 * 128 * 6
    assert h3a.h3a_attention_workspace_bytes(100, 1024, 2, 256, "kvi8r", False) == 100 * 2 * 128 * 6
    # sparse adds per-(head, q-tile) counts and kept lists
    dense = h3a.h3a_attention_workspace_bytes(1024, 1024, 2, 256, "exact", True)
    assert dense >= 2 * 4 * 16 * 4 + 2 * 4 * 4
    assert h3a.h3a_attention_workspace_bytes(1024, 1024, 2, 256, "kvi8r", False, head_dim=64) == 0
    # Sol: tile means of the store (K, V: [H, n_kt, 128] 16-bit; K scales: [H, n_kt] fp32) plus dropped lists
    hard = h3a.h3a_attention_workspace_bytes(1024, 1000, 2, 256, "exact", True)
    sol = h3a.h3a_attention_workspace_bytes(1024, 1000, 2, 256, "exact", True, sol=True)
    n_kt = 16
    assert sol >= hard + 2 * (2 * n_kt * 128 * 2) + 2 * n_kt * 4 + 2 * 4 * n_kt * 4
    assert h3a.h3a_attention_workspace_bytes(1024, 1000, 2, 256, "exact", False, sol=True) == 0


def test_noalloc_scratch_size_matches_the_header():
    src = open(HEADER).read()
    m = re.search(r"#define H3A_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == h3a.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("q_chunk,heads,mode,mask", [(65536, 32, 1, None), (16384, 32, 1, None),
                                                     (8192, 64, 2, None), (16384, 32, 0x101, 1)])
def test_noalloc_rejects_requests_above_its_scratch(lib, q_chunk, heads, mode, mask):
    # Checked from the sizes alone, before any pointer or GPU call: nothing is queued.
    need = h3a.h3a_attention_workspace_bytes(65536, 65536, heads, q_chunk, mode, mask is not None)
    assert need > h3a.NOALLOC_SCRATCH_BYTES
    rc = lib.h3a_attention_noalloc(None, None, None, 16 if mode else None, 65536, 65536, heads, 128, 0.088, q_chunk,
                                   0, mode, mask, None, None)
    assert rc == -4
    err = lib.h3a_last_error().decode()
    assert "h3a_attention_noalloc" in err and str(need) in err


def test_noalloc_checks_arguments_like_h3a_attention(lib):
    assert lib.h3a_attention_noalloc(None, None, None, 16, 1024, 1024, 2, 64, 0.088, 256, 0, 1, None, None,
                                     None) == -2
    assert lib.h3a_attention_noalloc(None, None, None, None, 1024, 1024, 2, 128, 0.088, 256, 0, 1, None, None,
                                     None) == -1
    assert "scales" in lib.h3a_last_error().decode()
    assert lib.h3a_attention_noalloc(None, None, None, 16, 0, 1024, 2, 128, 0.088, 256, 0, 1, None, None,
                                     None) == 0


def test_out_f16_flag_does_not_change_workspace_sizes():
    for mode in (1, 2):
        for sparse in (False, True):
            assert h3a.h3a_attention_workspace_bytes(1024, 1000, 2, 256, mode | 0x200, sparse) == \
                h3a.h3a_attention_workspace_bytes(1024, 1000, 2, 256, mode, sparse) > 0
    assert h3a.h3a_attention_host_kv_workspace_bytes(1024, 1000, 2, 256, 256, 1 | 0x200) == \
        h3a.h3a_attention_host_kv_workspace_bytes(1024, 1000, 2, 256, 256, 1)


def test_quantize_pair_rejects_bad_arguments(lib):
    assert lib.h3a_kv_quantize_pair(None, None, 256, 64, 2, 96, 0, 64, None, None, None, None) == -2
    assert lib.h3a_kv_quantize_pair(None, None, 256, 64, 2, 128, 0, 64, None, None, None, None) == -1
    assert "k and v" in lib.h3a_last_error().decode()
    assert lib.h3a_kv_quantize_pair(16, 32, 256, 64, 2, 128, 10, 64, None, None, None, None) == -1
    assert "exceeds" in lib.h3a_last_error().decode()
    assert lib.h3a_kv_quantize_pair(None, None, 256, 0, 2, 128, 0, 0, None, None, None, None) == 0


def test_timing_kinds_match_the_header(lib):
    src = open(HEADER).read()
    kinds = {m.group(1).lower(): int(m.group(2)) for m in re.finditer(r"#define H3A_TIMING_([A-Z_]+) (\d+)", src)}
    assert kinds == h3a.TIMING_KINDS
    ms, n = ctypes.c_double(1.0), ctypes.c_int64(7)
    for kind in kinds.values():  # nothing timed yet: zero launches, no HIP call
        assert lib.h3a_timing_collect_kernel(kind, ctypes.byref(ms), ctypes.byref(n)) == 0
        assert (ms.value, n.value) == (0.0, 0)
    assert lib.h3a_timing_collect_kernel(len(kinds), ctypes.byref(ms), ctypes.byref(n)) == -1
    assert "timing kind" in lib.h3a_last_error().decode()
    assert lib.h3a_timing_collect_kernel(-1, ctypes.byref(ms), ctypes.byref(n)) == -1
