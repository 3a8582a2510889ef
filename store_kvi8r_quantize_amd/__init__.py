"""Python binding of libh3a.so: rotated-int8 ("kvi8r") K/V store and chunked attention on MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/h3a.h.  Tensors are PyTorch
device tensors (PyTorch provides device memory and streams); the functions
pass their device pointers, shapes and the current HIP stream to the library.
There is no CPU fallback: if the library is not built, or its ABI version does
not match, every call raises.

Functions carry the C names: h3a_kv_quantize (+ h3a_kv_quantize_g32, chosen by the
scales' shape), h3a_kv_quantize_pair, h3a_attention, h3a_attention_noalloc, h3a_attention_routed, h3a_attention_host_kv
(+ its workspace query),
h3a_attention_workspace_bytes, h3a_rotate_rows, h3a_unrotate_rows,
h3a_timing_enable, h3a_timing_collect, h3a_abi_version.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

ABI_VERSION = 1
HEAD_DIM = 128
TILE = 64
MODE_EXACT_BF16 = 0
MODE_KVI8R = 1
MODE_KVI8R32 = 2  # kvi8r with one fp16 scale per 32 rotated values
MODES = {"exact": MODE_EXACT_BF16, "bf16": MODE_EXACT_BF16, "kvi8r": MODE_KVI8R, "kvi8r32": MODE_KVI8R32}
SOL = 0x100  # H3A_SOL: dropped tiles of a tile_mask enter as one pseudo-key each
OUT_F16 = 0x200  # H3A_OUT_F16: fp16 output rows for the kvi8r stores (chosen here from out's dtype)
NOALLOC_SCRATCH_BYTES = 256 << 20  # H3A_NOALLOC_SCRATCH_BYTES: the library's own scratch per GPU

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libh3a.so")

_lib = None


class H3AError(RuntimeError):
    """A call into libh3a returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"h3a status {status}: {message}")
        self.status = status


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m store_kvi8r_quantize_amd.build` "
                           "(or __graft_entry__.build()) first")
    # torch is imported above, so its HIP runtime is already mapped and the
    # library binds to that same runtime (one HIP runtime per process).
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    lib.h3a_abi_version.restype = i32
    lib.h3a_abi_version.argtypes = []
    lib.h3a_last_error.restype = ctypes.c_char_p
    lib.h3a_last_error.argtypes = []
    lib.h3a_kv_quantize.restype = i32
    lib.h3a_kv_quantize.argtypes = [vp, i64, i64, i32, i32, i64, i64, vp, vp, vp]
    lib.h3a_kv_quantize_pair.restype = i32
    lib.h3a_kv_quantize_pair.argtypes = [vp, vp, i64, i64, i32, i32, i64, i64, vp, vp, vp, vp]
    lib.h3a_kv_quantize_g32.restype = i32
    lib.h3a_kv_quantize_g32.argtypes = [vp, i64, i64, i32, i32, i64, i64, vp, vp, vp]
    lib.h3a_attention_workspace_bytes.restype = sz
    lib.h3a_attention_workspace_bytes.argtypes = [i64, i64, i32, i32, i64, i32, i32]
    lib.h3a_attention.restype = i32
    lib.h3a_attention.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, f32, i64, i64, i32, vp, vp, vp, sz, vp]
    lib.h3a_attention_noalloc.restype = i32
    lib.h3a_attention_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, f32, i64, i64, i32, vp, vp, vp]
    lib.h3a_attention_routed.restype = i32
    lib.h3a_attention_routed.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, f32, i64, i64,
                                         ctypes.POINTER(ctypes.c_int64), i32, vp, vp, sz, vp]
    lib.h3a_attention_host_kv_workspace_bytes.restype = sz
    lib.h3a_attention_host_kv_workspace_bytes.argtypes = [i64, i64, i32, i32, i64, i64, i32]
    lib.h3a_attention_host_kv.restype = i32
    lib.h3a_attention_host_kv.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, f32, i64, i64, i32, vp, vp, sz, vp]
    lib.h3a_rotate_rows.restype = i32
    lib.h3a_rotate_rows.argtypes = [vp, vp, i64, vp]
    lib.h3a_unrotate_rows.restype = i32
    lib.h3a_unrotate_rows.argtypes = [vp, vp, i64, vp]
    lib.h3a_timing_enable.restype = i32
    lib.h3a_timing_enable.argtypes = [i32]
    lib.h3a_timing_collect.restype = i32
    lib.h3a_timing_collect.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.h3a_timing_collect_kernel.restype = i32
    lib.h3a_timing_collect_kernel.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    if lib.h3a_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libh3a ABI {lib.h3a_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = lib
    return lib


def library():
    """The loaded ctypes library (loads it on first use)."""
    return _load()


def _check(rc: int):
    if rc != 0:
        raise H3AError(rc, _lib.h3a_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream_obj(t, stream):
    """The torch stream the call's work is queued on: the caller's (a torch stream, or a raw hipStream_t
    handle wrapped as an external stream), else the current stream of t's device."""
    if stream is None:
        return torch.cuda.current_stream(t.device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=t.device)


def _stream(t, stream):
    return _stream_obj(t, stream).cuda_stream


def _workspace(need: int, device, stream_obj):
    """A workspace of `need` bytes for work queued on stream_obj.

    It is allocated with stream_obj current, so the caching allocator files the
    block under that stream: when the tensor is freed (on return), the block is
    handed out again only to work ordered after what is already queued on that
    stream, which includes the kernels that use it.
    """
    with torch.cuda.stream(stream_obj):
        return torch.empty(need, dtype=torch.uint8, device=device)


def _out_flag(out, mode) -> int:
    """H3A_OUT_F16 when out is fp16 (kvi8r stores only), 0 when it is bf16."""
    if not isinstance(out, torch.Tensor) or not out.is_cuda:
        raise TypeError("out must be a GPU tensor")
    if out.dtype == torch.float16:
        if mode not in (MODE_KVI8R, MODE_KVI8R32):
            raise TypeError("an fp16 out is for the kvi8r stores; the exact store's output is bf16")
        return OUT_F16
    if out.dtype != torch.bfloat16:
        raise TypeError(f"out must be bfloat16 (or float16 for the kvi8r stores), got {out.dtype}")
    return 0


def _need(t, name, dtype):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")


def h3a_abi_version() -> int:
    return _load().h3a_abi_version()


def h3a_kv_quantize(x, codes, scales, token_offset: int = 0, stream=None):
    """Quantise x (bf16 [n_tokens, n_heads, 128], rows contiguous) into rows
    [token_offset, token_offset + n_tokens) of a kvi8r store: codes int8
    [n_heads, s_total, 128] and scales fp16 [n_heads, s_total] (one per row,
    h3a_kv_quantize) or [n_heads, s_total, 4] (one per 32 values, the kvi8r32
    store, h3a_kv_quantize_g32)."""
    lib = _load()
    _need(x, "x", torch.bfloat16)
    _need(codes, "codes", torch.int8)
    _need(scales, "scales", torch.float16)
    if x.dim() != 3 or x.stride(2) != 1 or (x.shape[1] > 1 and x.stride(1) != x.shape[2]):
        raise ValueError("x must be [n_tokens, n_heads, head_dim] with contiguous (token, head) rows")
    grouped = scales.dim() == 3
    if codes.dim() != 3 or not codes.is_contiguous() or scales.dim() not in (2, 3) or not scales.is_contiguous() \
            or (grouped and scales.shape[2] != 4):
        raise ValueError("codes must be contiguous [n_heads, s_total, 128] and scales contiguous "
                         "[n_heads, s_total] or [n_heads, s_total, 4]")
    stride = x.stride(0) if x.shape[0] > 1 else x.shape[1] * x.shape[2]
    fn = lib.h3a_kv_quantize_g32 if grouped else lib.h3a_kv_quantize
    _check(fn(_ptr(x), stride, x.shape[0], x.shape[1], x.shape[2], int(token_offset), codes.shape[1], _ptr(codes),
              _ptr(scales), _stream(x, stream)))


def h3a_kv_quantize_pair(k, v, k_codes, v_codes, scales, token_offset: int = 0, stream=None):
    """Quantise one kv_chunk of K and of V (bf16 [n_tokens, n_heads, 128] each, same strides) in one launch into
    rows [token_offset, token_offset + n_tokens) of a kvi8r store: codes int8 [n_heads, s_total, 128] each and
    scales fp16 [2, n_heads, s_total] (K, then V).  Same codes and scales as two h3a_kv_quantize calls."""
    lib = _load()
    for name, t in (("k", k), ("v", v)):
        _need(t, name, torch.bfloat16)
        if t.dim() != 3 or t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != t.shape[2]):
            raise ValueError(f"{name} must be [n_tokens, n_heads, head_dim] with contiguous (token, head) rows")
    if k.shape != v.shape or (k.shape[0] > 1 and k.stride(0) != v.stride(0)):
        raise ValueError("k and v must have the same shape and token stride")
    _need(k_codes, "k_codes", torch.int8)
    _need(v_codes, "v_codes", torch.int8)
    _need(scales, "scales", torch.float16)
    if not (k_codes.is_contiguous() and v_codes.is_contiguous() and scales.is_contiguous()) or scales.dim() != 3 \
            or scales.shape[0] != 2 or k_codes.shape != v_codes.shape:
        raise ValueError("k_codes / v_codes must be contiguous [n_heads, s_total, 128] and scales contiguous "
                         "[2, n_heads, s_total]")
    stride = k.stride(0) if k.shape[0] > 1 else k.shape[1] * k.shape[2]
    _check(lib.h3a_kv_quantize_pair(_ptr(k), _ptr(v), stride, k.shape[0], k.shape[1], k.shape[2], int(token_offset),
                                    k_codes.shape[1], _ptr(k_codes), _ptr(v_codes), _ptr(scales), _stream(k, stream)))


def new_kvi8r_store(s_total: int, n_heads: int, device="cuda", per32: bool = False):
    """Allocate an empty kvi8r store: (k_codes, v_codes, scales[2, n_heads, s_total]), or with per32 the
    kvi8r32 store, scales[2, n_heads, s_total, 4]."""
    k = torch.empty((n_heads, s_total, HEAD_DIM), dtype=torch.int8, device=device)
    v = torch.empty((n_heads, s_total, HEAD_DIM), dtype=torch.int8, device=device)
    shape = (2, n_heads, s_total, 4) if per32 else (2, n_heads, s_total)
    s = torch.empty(shape, dtype=torch.float16, device=device)
    return k, v, s


def h3a_attention_workspace_bytes(s_q: int, s_kv: int, n_heads: int, q_chunk: int, mode, sparse: bool,
                                  head_dim: int = HEAD_DIM, sol: bool = False) -> int:
    mode = int(MODES.get(mode, mode)) | (SOL if sol else 0)
    return int(_load().h3a_attention_workspace_bytes(s_q, s_kv, n_heads, head_dim, q_chunk, mode, int(sparse)))


def h3a_attention(q, k_store, v_store, scales, out, *, q_chunk: int, kv_block: int = 0, mode="kvi8r",
                  tile_mask=None, sol: bool = False, softmax_scale: float | None = None, workspace=None,
                  stream=None):
    """Chunked attention of q (bf16 [s_q, H, 128]) against a K/V store, written into out (bf16 [s_q, H, 128]).

    mode "exact": k_store / v_store bf16 [s_kv, H, 128], scales None.
    mode "kvi8r": k_store / v_store int8 [H, s_kv, 128], scales fp16 [2, H, s_kv].
    mode "kvi8r32": k_store / v_store int8 [H, s_kv, 128], scales fp16 [2, H, s_kv, 4].
    tile_mask: None (dense) or uint8 [H, ceil(s_q/64), ceil(s_kv/64)].
    sol: with a tile_mask, each dropped tile enters as one pseudo-key (tile-mean K and V, weight = its key count).
    workspace: a uint8 GPU tensor of at least h3a_attention_workspace_bytes; allocated here when None.
    """
    lib = _load()
    mode = MODES.get(mode, mode)
    flags = (SOL if sol else 0) | _out_flag(out, mode)
    _need(q, "q", torch.bfloat16)
    if not (q.is_contiguous() and out.is_contiguous()) or q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be contiguous [s_q, n_heads, head_dim] tensors of equal shape")
    s_q, n_heads, head_dim = q.shape
    if mode in (MODE_KVI8R, MODE_KVI8R32):
        _need(k_store, "k_store", torch.int8)
        _need(v_store, "v_store", torch.int8)
        _need(scales, "scales", torch.float16)
        if scales.dim() != (4 if mode == MODE_KVI8R32 else 3):
            raise ValueError("scales must be [2, H, s_kv] (kvi8r) or [2, H, s_kv, 4] (kvi8r32)")
        s_kv = k_store.shape[1]
    else:
        _need(k_store, "k_store", torch.bfloat16)
        _need(v_store, "v_store", torch.bfloat16)
        s_kv = k_store.shape[0]
    for name, t in (("k_store", k_store), ("v_store", v_store), ("scales", scales)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if tile_mask is not None:
        _need(tile_mask, "tile_mask", torch.uint8)
        if not tile_mask.is_contiguous():
            raise ValueError("tile_mask must be contiguous")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    need = int(lib.h3a_attention_workspace_bytes(s_q, s_kv, n_heads, head_dim, q_chunk, int(mode) | flags,
                                                 int(tile_mask is not None)))
    st = _stream_obj(q, stream)
    if workspace is None and need > 0:
        workspace = _workspace(need, q.device, st)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.h3a_attention(_ptr(q), _ptr(k_store), _ptr(v_store), _ptr(scales), s_q, s_kv, n_heads, head_dim,
                             float(softmax_scale), int(q_chunk), int(kv_block), int(mode) | flags, _ptr(tile_mask),
                             _ptr(out), _ptr(workspace), ws_bytes, st.cuda_stream))
    return out


def h3a_attention_noalloc(q, k_store, v_store, scales, out, *, q_chunk: int, kv_block: int = 0, mode="kvi8r",
                          tile_mask=None, sol: bool = False, softmax_scale: float | None = None, stream=None):
    """h3a_attention without a workspace: the library's own per-GPU scratch (NOALLOC_SCRATCH_BYTES) is used,
    and nothing is allocated, here or in the library.  A call needing more scratch raises H3AError
    (H3A_EWORKSPACE); a smaller q_chunk needs less and gives the same output.  Calls on one GPU share the
    scratch, so calls on different streams must not overlap."""
    lib = _load()
    mode = MODES.get(mode, mode)
    flags = (SOL if sol else 0) | _out_flag(out, mode)
    _need(q, "q", torch.bfloat16)
    if not (q.is_contiguous() and out.is_contiguous()) or q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be contiguous [s_q, n_heads, head_dim] tensors of equal shape")
    s_q, n_heads, head_dim = q.shape
    if mode in (MODE_KVI8R, MODE_KVI8R32):
        _need(k_store, "k_store", torch.int8)
        _need(v_store, "v_store", torch.int8)
        _need(scales, "scales", torch.float16)
        s_kv = k_store.shape[1]
    else:
        _need(k_store, "k_store", torch.bfloat16)
        _need(v_store, "v_store", torch.bfloat16)
        s_kv = k_store.shape[0]
    for name, t in (("k_store", k_store), ("v_store", v_store), ("scales", scales), ("tile_mask", tile_mask)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if tile_mask is not None:
        _need(tile_mask, "tile_mask", torch.uint8)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    _check(lib.h3a_attention_noalloc(_ptr(q), _ptr(k_store), _ptr(v_store), _ptr(scales), s_q, s_kv, n_heads,
                                     head_dim, float(softmax_scale), int(q_chunk), int(kv_block), int(mode) | flags,
                                     _ptr(tile_mask), _ptr(out), _stream(q, stream)))
    return out


def h3a_attention_routed(q, k_bf16, v_bf16, store, out, *, exact_spans, q_chunk: int, kv_block: int = 0,
                         softmax_scale: float | None = None, workspace=None, stream=None):
    """Attention of q (bf16 [s_q, H, 128]) into out, rows chosen per span between two stores of one K/V.

    Rows inside one of exact_spans (increasing, disjoint [begin, end) pairs) attend k_bf16 / v_bf16
    (bf16 [s_kv, H, 128]) exactly; the other rows attend the kvi8r store = (k_codes, v_codes, scales).
    """
    lib = _load()
    kc, vc, sc = store
    _need(q, "q", torch.bfloat16)
    _need(out, "out", torch.bfloat16)
    _need(k_bf16, "k_bf16", torch.bfloat16)
    _need(v_bf16, "v_bf16", torch.bfloat16)
    _need(kc, "k_codes", torch.int8)
    _need(vc, "v_codes", torch.int8)
    _need(sc, "scales", torch.float16)
    for name, t in (("q", q), ("out", out), ("k_bf16", k_bf16), ("v_bf16", v_bf16), ("k_codes", kc),
                    ("v_codes", vc), ("scales", sc)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be [s_q, n_heads, head_dim] tensors of equal shape")
    s_q, n_heads, head_dim = q.shape
    s_kv = k_bf16.shape[0]
    if kc.shape[1] != s_kv:
        raise ValueError("the bf16 K/V and the kvi8r store must hold the same number of tokens")
    flat = [int(x) for span in exact_spans for x in span]
    spans = (ctypes.c_int64 * max(len(flat), 1))(*flat)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    need = int(lib.h3a_attention_workspace_bytes(s_q, s_kv, n_heads, head_dim, q_chunk, MODE_KVI8R, 0))
    st = _stream_obj(q, stream)
    if workspace is None and need > 0:
        workspace = _workspace(need, q.device, st)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.h3a_attention_routed(_ptr(q), _ptr(k_bf16), _ptr(v_bf16), _ptr(kc), _ptr(vc), _ptr(sc), s_q, s_kv,
                                    n_heads, head_dim, float(softmax_scale), int(q_chunk), int(kv_block), spans,
                                    len(flat) // 2, _ptr(out), _ptr(workspace), ws_bytes, st.cuda_stream))
    return out


def h3a_attention_host_kv_workspace_bytes(s_q: int, s_kv: int, n_heads: int, q_chunk: int, kv_block: int, mode,
                                          head_dim: int = HEAD_DIM) -> int:
    mode = MODES.get(mode, mode)
    return int(_load().h3a_attention_host_kv_workspace_bytes(s_q, s_kv, n_heads, head_dim, q_chunk, kv_block,
                                                             int(mode)))


def h3a_attention_host_kv(q, k_host, v_host, scales_host, out, *, q_chunk: int, kv_block: int = 0, mode="kvi8r",
                          softmax_scale: float | None = None, workspace=None, stream=None):
    """h3a_attention with the K/V store in pinned host memory (CPU tensors with pin_memory), streamed to the GPU
    one kv_block at a time.  Store layouts as for h3a_attention; q and out are GPU tensors."""
    lib = _load()
    mode = MODES.get(mode, mode)
    flags = _out_flag(out, mode)
    _need(q, "q", torch.bfloat16)
    if not (q.is_contiguous() and out.is_contiguous()) or q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be contiguous [s_q, n_heads, head_dim] tensors of equal shape")
    want = torch.bfloat16 if mode == MODE_EXACT_BF16 else torch.int8
    for name, t in (("k_host", k_host), ("v_host", v_host), ("scales_host", scales_host)):
        if t is None:
            continue
        # an empty store has no storage to pin; the library reads nothing from it
        if t.device.type != "cpu" or not t.is_contiguous() or (t.numel() > 0 and not t.is_pinned()):
            raise ValueError(f"{name} must be a contiguous pinned CPU tensor")
    if k_host.dtype != want or v_host.dtype != want:
        raise ValueError(f"k_host / v_host must be {want} for mode {mode}")
    s_q, n_heads, head_dim = q.shape
    s_kv = k_host.shape[0] if mode == MODE_EXACT_BF16 else k_host.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    need = int(lib.h3a_attention_host_kv_workspace_bytes(s_q, s_kv, n_heads, head_dim, q_chunk, kv_block, int(mode)))
    st = _stream_obj(q, stream)
    if workspace is None and need > 0:
        workspace = _workspace(need, q.device, st)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    hp = lambda t: None if t is None else t.data_ptr()
    _check(lib.h3a_attention_host_kv(_ptr(q), hp(k_host), hp(v_host), hp(scales_host), s_q, s_kv, n_heads, head_dim,
                                     float(softmax_scale), int(q_chunk), int(kv_block), int(mode) | flags,
                                     _ptr(out), _ptr(workspace), ws_bytes, st.cuda_stream))
    return out


def h3a_rotate_rows(x, y, stream=None):
    """y (fp16 [..., 128]) = x (bf16 [..., 128]) rotated into the Hadamard basis."""
    lib = _load()
    _need(x, "x", torch.bfloat16)
    _need(y, "y", torch.float16)
    if not (x.is_contiguous() and y.is_contiguous()) or x.numel() != y.numel() or x.shape[-1] != HEAD_DIM:
        raise ValueError("x and y must be contiguous with equal sizes and rows of 128")
    _check(lib.h3a_rotate_rows(_ptr(x), _ptr(y), x.numel() // HEAD_DIM, _stream(x, stream)))
    return y


def h3a_unrotate_rows(x, y, stream=None):
    """y (bf16 [..., 128]) = x (fp32 [..., 128]) rotated back out of the Hadamard basis."""
    lib = _load()
    _need(x, "x", torch.float32)
    _need(y, "y", torch.bfloat16)
    if not (x.is_contiguous() and y.is_contiguous()) or x.numel() != y.numel() or x.shape[-1] != HEAD_DIM:
        raise ValueError("x and y must be contiguous with equal sizes and rows of 128")
    _check(lib.h3a_unrotate_rows(_ptr(x), _ptr(y), x.numel() // HEAD_DIM, _stream(x, stream)))
    return y


def h3a_timing_enable(on: bool):
    _check(_load().h3a_timing_enable(int(bool(on))))


TIMING_KINDS = {"attention": 0, "rotate_q": 1, "unrotate_o": 2, "kv_quantize": 3}


def h3a_timing_collect(kind: str = "attention"):
    """(summed kernel milliseconds, launches) of one timed kernel kind since its last collect."""
    lib = _load()
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(lib.h3a_timing_collect_kernel(TIMING_KINDS[kind], ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
