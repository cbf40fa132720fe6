"""Q4 KV-cache codec and fused-dequant decode attention for MI355X (gfx950).

A thin ctypes binding over ``libkvq.so`` (C ABI in ``include/kvq.h``): it checks tensor dtypes, devices,
shapes and alignment, then passes raw device pointers and torch's current HIP stream. Every step of the
computation runs in the library's HIP kernels; there is no fallback. If ``libkvq.so`` has not been built
(``python -m bit_quantized_kv_quantize_amd._build``), importing this package raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK, KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP = 0, -1, -2, -3, -4
BLOCK_TOKENS = 256


class KvqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (%d)" % (fn, status_string(status), status))
        self.status = status


class Layout(ctypes.Structure):
    """Mirror of ``kvq_layout`` (include/kvq.h)."""

    _fields_ = [(n, ctypes.c_int32) for n in
                ("head_dim", "num_kv_heads", "block_tokens", "k_group", "v_group", "rotate", "mixed",
                 "format", "v_head_dim")]

    def __init__(self, head_dim, num_kv_heads, k_group=64, v_group=64, rotate=0, mixed=0,
                 block_tokens=BLOCK_TOKENS, format=0, v_head_dim=0):
        super().__init__(head_dim, num_kv_heads, block_tokens, k_group, v_group, int(rotate), int(mixed),
                         int(format), int(v_head_dim))

    @property
    def dv(self) -> int:
        """V's head dim (the K head dim unless v_head_dim gives another)."""
        return self.v_head_dim if self.v_head_dim > 0 else self.head_dim

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


if not os.path.exists(LIB_PATH):
    raise ImportError("libkvq.so is not built (%s); run `python -m bit_quantized_kv_quantize_amd._build` "
                      "(or __graft_entry__.build())" % LIB_PATH)

# torch first: it carries its own HIP runtime, and libkvq.so must bind to that same runtime (loaded first,
# it would pull in the system one as well, and the two would not share streams or device memory).
import torch as _torch_runtime  # noqa: E402,F401

_P = ctypes.c_void_p
_I = ctypes.c_int32
_LP = ctypes.POINTER(Layout)


def _load(path):
    L = ctypes.CDLL(path)
    L.kvq_check_layout.argtypes = [_LP]
    L.kvq_check_layout.restype = ctypes.c_int
    L.kvq_tile_bytes.argtypes = [_LP]
    L.kvq_tile_bytes.restype = ctypes.c_size_t
    L.kvq_pool_bytes.argtypes = [_LP, _I]
    L.kvq_pool_bytes.restype = ctypes.c_size_t
    L.kvq_decode_workspace_bytes.argtypes = [_LP, _I, _I, _I]
    L.kvq_decode_workspace_bytes.restype = ctypes.c_size_t
    L.kvq_status_string.argtypes = [ctypes.c_int]
    L.kvq_status_string.restype = ctypes.c_char_p
    L.kvq_quantize_blocks.argtypes = [_LP, _P, _P, _I, _P, _P, _P, _P]
    L.kvq_quantize_blocks.restype = ctypes.c_int
    L.kvq_dequantize_blocks.argtypes = [_LP, _P, _P, _I, _P, _P, _P]
    L.kvq_dequantize_blocks.restype = ctypes.c_int
    L.kvq_copy_blocks.argtypes = [_LP, _P, _P, _P, _P, _I, _P]
    L.kvq_copy_blocks.restype = ctypes.c_int
    L.kvq_append_tokens.argtypes = [_LP, _P, _I, _P, _P, _P, _I, _P, _P, _P]
    L.kvq_append_tokens.restype = ctypes.c_int
    L.kvq_decode_attention.argtypes = [_LP, _P, _P, _I, _I, _P, _I, _P, _I, _P, _I, ctypes.c_float, _P, _P,
                                       ctypes.c_size_t, _P]
    L.kvq_decode_attention.restype = ctypes.c_int
    L.kvq_decode_attention_static.argtypes = [_LP, _P, _P, _I, _I, _P, _I, _P, _I, _P, _I, ctypes.c_float, _P, _P]
    L.kvq_decode_attention_static.restype = ctypes.c_int
    return L


_libs = {"release": _load(LIB_PATH)}
_lib = _libs["release"]
DEBUG_LIB_PATH = os.path.join(_HERE, "libkvq_debug.so")


def use_library(which: str = "release"):
    """Route every call of this module to the release library (default) or to its debug build
    (``libkvq_debug.so``: device-resident ids, lengths and positions are checked on the host before any
    launch, and the KVQ_DECODE_KERNEL environment variable may force a decode kernel - a test hook). Returns
    the ctypes handle now in use."""
    global _lib
    if which not in ("release", "debug"):
        raise ValueError("use_library: 'release' or 'debug'")
    if which not in _libs:
        if not os.path.exists(DEBUG_LIB_PATH):
            raise ImportError("libkvq_debug.so is not built (%s)" % DEBUG_LIB_PATH)
        _libs[which] = _load(DEBUG_LIB_PATH)
    _lib = _libs[which]
    return _lib


EXPORTS = ("kvq_check_layout", "kvq_tile_bytes", "kvq_pool_bytes", "kvq_decode_workspace_bytes",
           "kvq_status_string", "kvq_quantize_blocks", "kvq_dequantize_blocks", "kvq_copy_blocks",
           "kvq_append_tokens", "kvq_decode_attention", "kvq_decode_attention_static")


def lib():
    return _lib


def status_string(status: int) -> str:
    return _lib.kvq_status_string(int(status)).decode()


def check_layout(layout: Layout) -> int:
    return int(_lib.kvq_check_layout(ctypes.byref(layout)))


def tile_bytes(layout: Layout) -> int:
    return int(_lib.kvq_tile_bytes(ctypes.byref(layout)))


def pool_bytes(layout: Layout, num_blocks: int) -> int:
    return int(_lib.kvq_pool_bytes(ctypes.byref(layout), int(num_blocks)))


def decode_workspace_bytes(layout: Layout, n_seqs: int, num_q_heads: int, max_seq_len: int) -> int:
    return int(_lib.kvq_decode_workspace_bytes(ctypes.byref(layout), int(n_seqs), int(num_q_heads),
                                               int(max_seq_len)))


# ----------------------------------------------------------------------------------------- tensors

def _torch():
    import torch

    return torch


def _ptr(t, name, dtypes, align=1, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError("%s is required" % name)
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU torch tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s must have dtype in %s, got %s" % (name, dtypes, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    p = t.data_ptr()
    if p % align:
        raise ValueError("%s must be %d-byte aligned" % (name, align))
    return ctypes.c_void_p(p)


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, st):
    if st != KVQ_OK:
        raise KvqError(fn, st)


def _f16():
    torch = _torch()
    return (torch.float16, torch.int16, torch.uint16) if hasattr(torch, "uint16") else (torch.float16, torch.int16)


def new_pool(layout: Layout, num_blocks: int, device="cuda"):
    """A zero-filled pool tensor (uint8) for ``num_blocks`` blocks."""
    torch = _torch()
    n = pool_bytes(layout, num_blocks)
    if n == 0 and num_blocks:
        raise KvqError("kvq_pool_bytes", check_layout(layout) or KVQ_ERR_ARG)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def new_workspace(layout: Layout, n_seqs: int, num_q_heads: int, max_seq_len: int, device="cuda"):
    """A zero-filled decode workspace for calls of this size or smaller (split-K partials and arrival
    counters; every call leaves the counters at zero, so it can be reused without clearing)."""
    torch = _torch()
    need = decode_workspace_bytes(layout, n_seqs, num_q_heads, max_seq_len)
    return torch.zeros(max(need, 256), dtype=torch.uint8, device=device)


def quantize_blocks(layout: Layout, pool, block_ids, k, v, prec_bits=None, stream=None) -> None:
    """k fp16 [n_blocks*256, H_kv, d], v [.., dv]; block_ids int32 [n_blocks]; prec_bits int32/uint32 [n_blocks, W]:
    the rows' width words, W = 8 (mixed = 1: one bit per row, set = 8-bit) or 16 (mixed = 2: a 2-bit code per
    row, 0..3 = 2, 4, 8, 16 bits), or None (every row 4-bit)."""
    torch = _torch()
    n_blocks = int(block_ids.numel())
    if prec_bits is not None and int(prec_bits.numel()) != n_blocks * (16 if layout.mixed == 2 else 8):
        raise ValueError("prec_bits must hold %d words per block" % (16 if layout.mixed == 2 else 8))
    st = _lib.kvq_quantize_blocks(ctypes.byref(layout), _ptr(pool, "pool", (torch.uint8,), 256),
                                  _ptr(block_ids, "block_ids", (torch.int32,)), n_blocks,
                                  _ptr(k, "k", _f16(), 16), _ptr(v, "v", _f16(), 16),
                                  _ptr(prec_bits, "prec_bits", (torch.int32, torch.uint32), 4, True),
                                  _stream(stream))
    _check("kvq_quantize_blocks", st)


def dequantize_blocks(layout: Layout, pool, block_ids, k_out=None, v_out=None, stream=None):
    """fp16 k [n_blocks*256, H_kv, d], v [.., dv] of the listed blocks (un-rotated for rotated pools);
    allocated here unless given."""
    torch = _torch()
    n_blocks = int(block_ids.numel())
    shape = (n_blocks * 256, layout.num_kv_heads, layout.head_dim)
    vshape = shape[:2] + (layout.dv,)
    if k_out is None:
        k_out = torch.empty(shape, dtype=torch.float16, device=pool.device)
    if v_out is None:
        v_out = torch.empty(vshape, dtype=torch.float16, device=pool.device)
    if tuple(k_out.shape) != shape or tuple(v_out.shape) != vshape:
        raise ValueError("k_out and v_out must have shapes %s and %s" % (shape, vshape))
    st = _lib.kvq_dequantize_blocks(ctypes.byref(layout), _ptr(pool, "pool", (torch.uint8,), 256),
                                    _ptr(block_ids, "block_ids", (torch.int32,)), n_blocks,
                                    _ptr(k_out, "k_out", _f16(), 16), _ptr(v_out, "v_out", _f16(), 16),
                                    _stream(stream))
    _check("kvq_dequantize_blocks", st)
    return k_out, v_out


def copy_blocks(layout: Layout, src_pool, src_ids, dst_pool, dst_ids, stream=None) -> None:
    """Block src_ids[i] of src_pool -> block dst_ids[i] of dst_pool (all KV heads); int32 id tensors."""
    torch = _torch()
    n = int(src_ids.numel())
    if int(dst_ids.numel()) != n:
        raise ValueError("src_ids and dst_ids differ in length")
    st = _lib.kvq_copy_blocks(ctypes.byref(layout), _ptr(src_pool, "src_pool", (torch.uint8,), 16),
                              _ptr(src_ids, "src_ids", (torch.int32,)), _ptr(dst_pool, "dst_pool", (torch.uint8,), 16),
                              _ptr(dst_ids, "dst_ids", (torch.int32,)), n, _stream(stream))
    _check("kvq_copy_blocks", st)


def append_tokens(layout: Layout, pool, k, v, block_table, positions, prec=None, stream=None) -> None:
    """k fp16 [n_seqs, H_kv, d], v [n_seqs, H_kv, dv]; block_table int32 [n_seqs, max_blocks]; positions int32 [n_seqs];
    prec uint8 [n_seqs]: each row's width (4 or 8 in a mixed = 1 pool; 2, 4, 8 or 16 in a mixed = 2 pool)
    or None (all 4-bit)."""
    torch = _torch()
    n = int(positions.numel())
    st = _lib.kvq_append_tokens(ctypes.byref(layout), _ptr(pool, "pool", (torch.uint8,), 256), n,
                                _ptr(k, "k", _f16(), 16), _ptr(v, "v", _f16(), 16),
                                _ptr(block_table, "block_table", (torch.int32,)), int(block_table.shape[1]),
                                _ptr(positions, "positions", (torch.int32,)),
                                _ptr(prec, "prec", (torch.uint8,), 1, True), _stream(stream))
    _check("kvq_append_tokens", st)


def decode_attention(layout: Layout, pool, q, block_table, seq_lens, max_seq_len: int, sentinel_mask=None,
                     softmax_scale: Optional[float] = None, out=None, workspace=None, stream=None):
    """q fp16 [n_seqs, H_q, d] -> fp32 [n_seqs, H_q, dv]. ``max_seq_len`` must bound every seq_lens
    entry (it sizes the split plan); sentinel_mask int32/uint32 [n_seqs, words] or None."""
    torch = _torch()
    n_seqs, hq, d = (int(x) for x in q.shape)
    if d != layout.head_dim:
        raise ValueError("q has head dim %d, the layout %d" % (d, layout.head_dim))
    if softmax_scale is None:
        softmax_scale = d ** -0.5
    if out is None:
        out = torch.empty((n_seqs, hq, layout.dv), dtype=torch.float32, device=q.device)
    if tuple(out.shape) != (n_seqs, hq, layout.dv):
        raise ValueError("out must have shape %s" % ((n_seqs, hq, layout.dv),))
    need = decode_workspace_bytes(layout, n_seqs, hq, max_seq_len)
    if workspace is None:
        workspace = new_workspace(layout, n_seqs, hq, max_seq_len, q.device)
    words = 0 if sentinel_mask is None else int(sentinel_mask.shape[1])
    st = _lib.kvq_decode_attention(ctypes.byref(layout), _ptr(pool, "pool", (torch.uint8,), 256),
                                   _ptr(q, "q", _f16(), 16), n_seqs, hq,
                                   _ptr(block_table, "block_table", (torch.int32,)), int(block_table.shape[1]),
                                   _ptr(seq_lens, "seq_lens", (torch.int32,)), int(max_seq_len),
                                   _ptr(sentinel_mask, "sentinel_mask", (torch.int32, torch.uint32), 4, True),
                                   words, float(softmax_scale), _ptr(out, "out", (torch.float32,), 16),
                                   _ptr(workspace, "workspace", (torch.uint8,), 256), int(workspace.numel()),
                                   _stream(stream))
    _check("kvq_decode_attention", st)
    return out
