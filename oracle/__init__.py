"""TEST INFRASTRUCTURE: the CPU oracle for the Q4 KV-cache codec and decode attention.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import this
package. It wraps ``kvq_oracle.c`` (plain C, built with gcc, no FMA contraction) through ctypes and
offers numpy-friendly calls. It shares no code with the GPU library; see ``kvq_oracle.c`` for the
pages each function follows and the tests that pin it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_kvq.so")

ORC_OK = 0
ORC_ERR_ARG = -1
ORC_ERR_UNSUPPORTED = -2


class OrcLayout(ctypes.Structure):
    """Same field order as the library's layout struct (head_dim, num_kv_heads, block_tokens, k_group,
    v_group, rotate, mixed, format, v_head_dim)."""

    _fields_ = [(n, ctypes.c_int32) for n in
                ("head_dim", "num_kv_heads", "block_tokens", "k_group", "v_group", "rotate", "mixed",
                 "format", "v_head_dim")]


def make_layout(head_dim, num_kv_heads, k_group, v_group, rotate=0, mixed=0, block_tokens=256, format=0,
                v_head_dim=0):
    return OrcLayout(head_dim, num_kv_heads, block_tokens, k_group, v_group, int(rotate), int(mixed),
                     int(format), int(v_head_dim))


def v_dim(layout: OrcLayout) -> int:
    """V's head dim (the K head dim unless the layout gives another)."""
    return layout.v_head_dim if layout.v_head_dim > 0 else layout.head_dim


def build(force: bool = True) -> str:
    """Compile kvq_oracle.c into liboracle_kvq.so (gcc, -O2, no FP contraction, OpenMP)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = build(force=False)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32 = ctypes.c_int32
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_e4m3.argtypes = [ctypes.c_float]
        L.orc_f32_to_e4m3.restype = ctypes.c_uint8
        L.orc_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_to_f32.restype = ctypes.c_float
        L.orc_fwht_f32.argtypes = [P, i32]
        L.orc_fwht_f32.restype = None
        L.orc_rot_scale.argtypes = [i32]
        L.orc_rot_scale.restype = ctypes.c_float
        L.orc_quantize_group.argtypes = [P, i32, i32, i32, P, P, P]
        L.orc_quantize_group.restype = None
        L.orc_check_layout.argtypes = [ctypes.POINTER(OrcLayout)]
        L.orc_check_layout.restype = ctypes.c_int
        L.orc_tile_bytes.argtypes = [ctypes.POINTER(OrcLayout)]
        L.orc_tile_bytes.restype = ctypes.c_size_t
        L.orc_quantize_blocks.argtypes = [ctypes.POINTER(OrcLayout), P, P, i32, P, P, P]
        L.orc_quantize_blocks.restype = ctypes.c_int
        L.orc_append_tokens.argtypes = [ctypes.POINTER(OrcLayout), P, i32, P, P, P, i32, P, P]
        L.orc_append_tokens.restype = ctypes.c_int
        L.orc_dequant_row.argtypes = [ctypes.POINTER(OrcLayout), P, i32, P, P]
        L.orc_dequant_row.restype = i32
        L.orc_dequantize_blocks.argtypes = [ctypes.POINTER(OrcLayout), P, P, i32, P, P]
        L.orc_dequantize_blocks.restype = ctypes.c_int
        L.orc_decode_attention.argtypes = [ctypes.POINTER(OrcLayout), P, P, i32, i32, P, i32, P, P, i32,
                                           ctypes.c_float, P, P, i32, i32]
        L.orc_decode_attention.restype = ctypes.c_int
        L.orc_set_threads.argtypes = [i32]
        L.orc_set_threads.restype = None
        L.orc_max_threads.argtypes = []
        L.orc_max_threads.restype = i32
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def f32_to_f16_bits(x: float) -> int:
    return int(lib().orc_f32_to_f16(float(x)))


def f16_bits_to_f32(h: int) -> float:
    return float(lib().orc_f16_to_f32(int(h)))


def f32_to_e4m3(x: float) -> int:
    return int(lib().orc_f32_to_e4m3(float(x)))


def e4m3_to_f32(b: int) -> float:
    return float(lib().orc_e4m3_to_f32(int(b)))


def fwht_f32(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform of a 1-D fp32 vector (power-of-two length)."""
    y = _c(x, np.float32).copy()
    lib().orc_fwht_f32(_p(y), y.size)
    return y


def rot_scale(n: int) -> float:
    return float(lib().orc_rot_scale(n))


def quantize_group(x: np.ndarray, bits: int = 4):
    """Quantise one group of fp32 values -> (codes uint8[n], scale fp16 bits, zero fp16 bits)."""
    x = _c(x, np.float32)
    codes = np.zeros(x.size, np.uint8)
    sh = np.zeros(1, np.uint16)
    zh = np.zeros(1, np.uint16)
    lib().orc_quantize_group(_p(x), x.size, 1, bits, _p(codes), _p(sh), _p(zh))
    return codes, int(sh[0]), int(zh[0])


def check_layout(layout: OrcLayout) -> int:
    return int(lib().orc_check_layout(ctypes.byref(layout)))


def tile_bytes(layout: OrcLayout) -> int:
    return int(lib().orc_tile_bytes(ctypes.byref(layout)))


def quantize_blocks(layout: OrcLayout, pool: np.ndarray, block_ids, k: np.ndarray, v: np.ndarray,
                    prec_bits: Optional[np.ndarray] = None) -> None:
    """In-place on ``pool`` (uint8, host). k, v: uint16 fp16 bits [n_blocks*256][H_kv][d] and [..][dv]."""
    assert pool.dtype == np.uint8 and pool.flags.c_contiguous
    block_ids = _c(block_ids, np.int32)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    pb = None if prec_bits is None else _c(prec_bits, np.uint32)
    st = lib().orc_quantize_blocks(ctypes.byref(layout), _p(pool), _p(block_ids), block_ids.size, _p(k),
                                   _p(v), _p(pb))
    if st != ORC_OK:
        raise RuntimeError("orc_quantize_blocks failed: %d" % st)


def append_tokens(layout: OrcLayout, pool: np.ndarray, k: np.ndarray, v: np.ndarray, block_table,
                  positions, prec=None) -> int:
    bt = _c(block_table, np.int32)
    pos = _c(positions, np.int32)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    pr = None if prec is None else _c(prec, np.uint8)
    return int(lib().orc_append_tokens(ctypes.byref(layout), _p(pool), pos.size, _p(k), _p(v), _p(bt),
                                       bt.shape[1], _p(pos), _p(pr)))


def dequant_row(layout: OrcLayout, tile: np.ndarray, t: int):
    """Rotated-domain fp64 (k, v) of row t of one tile, plus the row's bit width."""
    k = np.zeros(layout.head_dim, np.float64)
    v = np.zeros(v_dim(layout), np.float64)
    tile = _c(tile, np.uint8)
    bits = lib().orc_dequant_row(ctypes.byref(layout), _p(tile), t, _p(k), _p(v))
    return k, v, int(bits)


def dequantize_blocks(layout: OrcLayout, pool: np.ndarray, block_ids):
    """fp16 bits (uint16) k [n_blocks * 256, H, d], v [.., dv]: the listed blocks restored (and un-rotated),
    one rounding from the exact fp64 values."""
    ids = _c(block_ids, np.int32)
    n, H, d = ids.size, layout.num_kv_heads, layout.head_dim
    k = np.zeros((n * 256, H, d), np.uint16)
    v = np.zeros((n * 256, H, v_dim(layout)), np.uint16)
    pool = _c(pool, np.uint8)
    st = lib().orc_dequantize_blocks(ctypes.byref(layout), _p(pool), _p(ids), n, _p(k), _p(v))
    if st != 0:
        raise ValueError("orc_dequantize_blocks: status %d" % st)
    return k, v


def decode_attention(layout: OrcLayout, pool: np.ndarray, q: np.ndarray, block_table, seq_lens,
                     sentinel_mask=None, softmax_scale: float = None, want_weights: bool = False,
                     n_threads: int = 0):
    """fp64 attention output [n_seqs][H_q][dv] for queries [n_seqs][H_q][d] (and optionally the softmax
    weights)."""
    q = _c(q, np.uint16)
    n_seqs, hq, d = q.shape
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    if softmax_scale is None:
        softmax_scale = float(np.float32(1.0 / np.sqrt(d)))
    mask = None if sentinel_mask is None else _c(sentinel_mask, np.uint32)
    words = 0 if mask is None else mask.shape[1]
    max_len = int(max(1, sl.max() if sl.size else 1))
    out = np.zeros((n_seqs, hq, v_dim(layout)), np.float64)
    w = np.zeros((n_seqs, hq, max_len), np.float64) if want_weights else None
    st = lib().orc_decode_attention(ctypes.byref(layout), _p(pool), _p(q), n_seqs, hq, _p(bt), bt.shape[1],
                                    _p(sl), _p(mask), words, float(softmax_scale), _p(out), _p(w), max_len,
                                    int(n_threads))
    if st != ORC_OK:
        raise RuntimeError("orc_decode_attention failed: %d" % st)
    return (out, w) if want_weights else out


def max_threads() -> int:
    return int(lib().orc_max_threads())


def set_threads(n: int) -> None:
    """Threads of the quantisation loop (and the default of every parallel loop); n <= 0 keeps the default."""
    lib().orc_set_threads(int(n))
