"""TEST INFRASTRUCTURE: dense fp64 brute force for tiny inputs, written independently of kvq_oracle.c.

It reads the tile bytes with numpy (its own parse of the storage layout), builds the whole dequantised
K and V of a sequence as matrices, undoes the rotation with an explicit Hadamard matrix
H[i][j] = (-1)^popcount(i & j) (not with butterflies), and evaluates softmax attention as matrix
products. It follows the same pages as the C oracle (Agent Memory Below the Prompt, technical summary
2.1-2.2; UltraQuant technology section; IntentKV invalidation section) and is used only to pin the C
oracle's decode loops on tiny inputs.
"""
from __future__ import annotations

import numpy as np


def hadamard(n: int) -> np.ndarray:
    i = np.arange(n)
    bits = np.bitwise_and.outer(i, i)
    pop = np.zeros_like(bits)
    b = bits.copy()
    while b.any():
        pop += b & 1
        b >>= 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def e4m3_values() -> np.ndarray:
    """fp64 value of each of the 256 FP8 E4M3 ("fn") bytes: sign bit 7, exponent bits 6..3 (bias 7), mantissa
    bits 2..0; exponent 0 is subnormal (m * 2^-9); 0x7F and 0xFF are NaN."""
    b = np.arange(256)
    e, m = (b >> 3) & 15, (b & 7).astype(np.float64)
    v = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    v = np.where((b & 0x7F) == 0x7F, np.nan, v)
    return np.where(b & 0x80, -v, v)


def _fp8_tile(tile: np.ndarray, d, dv):
    rows = 256
    rec = tile[: rows * (d + dv)].reshape(rows, d + dv)
    vals = e4m3_values()
    return vals[rec[:, :d]], vals[rec[:, d:]]


def _layout_offsets(d, k_group, v_group, mixed, dv=None):
    """Byte geometry of a tile (K head dim d, V head dim dv): row records (K codes then V codes of the row's
    width, rec bytes = K and V at the pool's widest width), the per-channel K parameters (if K is grouped per
    channel), per-row parameter records (K groups then V groups), header."""
    dv = d if dv is None else dv
    rows = 256
    rec = (d + dv) * (16 if mixed == 2 else 8 if mixed else 4) // 8
    off_par = rows * rec
    kpr = d // k_group if k_group > 0 else 0
    prow = (kpr + dv // v_group) * 4
    off_prow = off_par + (0 if k_group > 0 else d * 4)
    off_hdr = off_prow + rows * prow
    end = off_hdr + (64 if mixed == 2 else 32 if mixed else 0)
    tile = (end + 255) // 256 * 256
    return rec, off_par, off_prow, prow, kpr, off_hdr, tile


def _codes(rows_bytes: np.ndarray, d: int, bits: np.ndarray) -> np.ndarray:
    """rows_bytes: uint8 [n][slot]; bits: [n] 2, 4 or 8 -> integer codes [n][d]."""
    n = rows_bytes.shape[0]
    out = np.zeros((n, d), np.int64)
    lo = rows_bytes[:, : d // 2] & 0xF
    hi = rows_bytes[:, : d // 2] >> 4
    four = np.empty((n, d), np.int64)
    four[:, 0::2] = lo
    four[:, 1::2] = hi
    two = np.empty((n, d), np.int64)
    for k in range(4):
        two[:, k::4] = (rows_bytes[:, : d // 4] >> (2 * k)) & 3
    eight = rows_bytes[:, :d].astype(np.int64) if rows_bytes.shape[1] >= d else four
    for b, src in ((4, four), (2, two), (8, eight)):
        sel = bits == b
        if sel.any():
            out[sel] = src[sel]
    return out


def dequant_tile(tile: np.ndarray, d, k_group, v_group, mixed, fmt=0, dv=None):
    """-> (K [256][d], V [256][dv]) fp64 in the stored (rotated) domain. fmt 1: FP8 E4M3 records."""
    dv = d if dv is None else dv
    if fmt == 1:
        return _fp8_tile(tile, d, dv)
    recb, off_par, off_prow, prow, kpr, off_hdr, _ = _layout_offsets(d, k_group, v_group, mixed, dv)
    rows = 256
    t = np.arange(rows)
    if mixed == 2:
        hdr = tile[off_hdr: off_hdr + 64]
        bits = 2 << ((hdr[t // 4] >> (2 * (t % 4))) & 3).astype(np.int64)
    elif mixed:
        hdr = tile[off_hdr: off_hdr + 32]
        bits = np.where((hdr[t // 8] >> (t % 8)) & 1, 8, 4)
    else:
        bits = np.full(rows, 4)
    rec = tile[: rows * recb].reshape(rows, recb)
    kc = _codes(rec[:, :d], d, np.where(bits == 16, 4, bits))
    # V codes follow the row's own K codes: d * bits / 8 bytes in
    vc = np.zeros((rows, dv), np.int64)
    for b in (2, 4, 8):
        sel = bits == b
        if sel.any():
            vc[sel] = _codes(rec[sel, d * b // 8: d * b // 8 + dv], dv, np.full(int(sel.sum()), b))
    par = tile[off_prow: off_prow + rows * prow].reshape(rows, prow)
    if k_group > 0:
        kp = par[:, : kpr * 4].copy().view(np.float16).reshape(rows, kpr, 2)
        ks = np.repeat(kp[:, :, 0].astype(np.float64), k_group, axis=1)
        kz = np.repeat(kp[:, :, 1].astype(np.float64), k_group, axis=1)
    else:
        kp = tile[off_par: off_par + d * 4].view(np.float16).reshape(d, 2)
        ks = np.broadcast_to(kp[:, 0].astype(np.float64), (rows, d))
        kz = np.broadcast_to(kp[:, 1].astype(np.float64), (rows, d))
    vp = par[:, kpr * 4:].copy().view(np.float16).reshape(rows, dv // v_group, 2)
    vs = np.repeat(vp[:, :, 0].astype(np.float64), v_group, axis=1)
    vz = np.repeat(vp[:, :, 1].astype(np.float64), v_group, axis=1)
    K, V = kc * ks + kz, vc * vs + vz
    f16 = bits == 16  # FP16 rows: raw values, K then V
    if f16.any():
        K[f16] = rec[f16, : 2 * d].copy().view(np.float16).astype(np.float64)
        V[f16] = rec[f16, 2 * d: 2 * d + 2 * dv].copy().view(np.float16).astype(np.float64)
    return K, V


def decode_attention(pool: np.ndarray, d, h_kv, k_group, v_group, rotate, mixed, q_bits: np.ndarray,
                     block_table, seq_lens, sentinel_mask=None, softmax_scale=None, fmt=0, dv=None) -> np.ndarray:
    """Dense fp64 attention of every query head over its sequence's dequantised cache (queries of K's head
    dim d, outputs of V's head dim dv)."""
    dv = d if dv is None else dv
    tile_bytes = (_layout_offsets(d, k_group, v_group, mixed, dv)[6] if fmt == 0
                  else (256 * (d + dv) + 255) // 256 * 256)
    q = q_bits.view(np.float16).astype(np.float64)
    n_seqs, hq, _ = q.shape
    g = hq // h_kv
    # the scale crosses the C ABI as fp32
    scale = float(np.float32(1.0 / np.sqrt(d) if softmax_scale is None else softmax_scale))
    if rotate:
        unrot_k = hadamard(d) / (d * float(np.float32(1.0 / np.sqrt(d))))
        unrot_v = hadamard(dv) / (dv * float(np.float32(1.0 / np.sqrt(dv))))
    out = np.zeros((n_seqs, hq, dv))
    for s in range(n_seqs):
        n = int(seq_lens[s])
        if n == 0:
            continue
        t = np.arange(n)
        if sentinel_mask is not None:
            sent = ((sentinel_mask[s][t // 32] >> (t % 32)) & 1).astype(bool)
        else:
            sent = np.zeros(n, bool)
        for h in range(h_kv):
            K = np.zeros((n, d))
            V = np.zeros((n, dv))
            for lb in range((n + 255) // 256):
                blk = int(block_table[s][lb])
                base = (blk * h_kv + h) * tile_bytes
                Kt, Vt = dequant_tile(pool[base: base + tile_bytes], d, k_group, v_group, mixed, fmt, dv)
                m = min(256, n - lb * 256)
                K[lb * 256: lb * 256 + m] = Kt[:m]
                V[lb * 256: lb * 256 + m] = Vt[:m]
            if rotate:
                K = K @ unrot_k.T
                V = V @ unrot_v.T
            V[sent] = 0.0
            Q = q[s, h * g: (h + 1) * g]
            logits = scale * (Q @ K.T)
            logits[:, sent] = -1e4
            logits -= logits.max(axis=1, keepdims=True)
            w = np.exp(logits)
            w /= w.sum(axis=1, keepdims=True)
            out[s, h * g: (h + 1) * g] = w @ V
    return out
