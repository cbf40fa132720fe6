"""Pins of the oracle's restore-to-fp16 function (orc_dequantize_blocks).

Pages: QKVShare methodology section, injection path (the quantised cache is rebuilt as fp16 key/value
tensors before the receiving agent's forward pass); "Agent Memory Below the Prompt" technical summary 2.1
(the stored form: codes plus one 16-bit scale and bias per group); UltraQuant technology section (the
Walsh-Hadamard rotation applied before quantisation, undone on the way back).

The pins: values already on the 4-bit grid come back bit for bit; the restored rows stay within the
per-element error bound of their stored scales, carried through the (orthogonal) rotation; and an
independent dense computation (numpy tile parser, explicit Hadamard matrix, numpy's fp64 -> fp16 cast)
gives the same bits.
"""
import numpy as np
import pytest

from oracle import brute


def _layout(orc, d, kg, vg, rotate, mixed, H=2):
    return orc.make_layout(head_dim=d, num_kv_heads=H, k_group=kg, v_group=vg, rotate=rotate, mixed=mixed)


def _pool(orc, lay, n_blocks):
    return np.zeros(orc.tile_bytes(lay) * n_blocks * lay.num_kv_heads, np.uint8)


@pytest.mark.parametrize("kg", [32, -1])
def test_grid_exact_blocks_come_back_bit_for_bit(orc, kg):
    # Every group holds codes 0 and 15 and values zero + code * scale with zero = -2 and scale = 0.25 (or 0.5,
    # per row or per channel), all exact in fp16: quantising reproduces the scale, zero and codes exactly,
    # and the restored values are the inputs.
    d, H, vg = 64, 2, 16
    lay = _layout(orc, d, kg, vg, 0, 0, H)
    rng = np.random.default_rng(3)
    n = 2
    codes_k = rng.integers(0, 16, (n * 256, H, d))
    codes_v = rng.integers(0, 16, (n * 256, H, d))
    if kg > 0:
        codes_k[:, :, 0::kg] = 0
        codes_k[:, :, 1::kg] = 15
    else:  # per channel over each block's 256 rows
        codes_k[0::256] = 0
        codes_k[1::256] = 15
    codes_v[:, :, 0::vg] = 0
    codes_v[:, :, 1::vg] = 15
    ks = np.where(np.arange(n * 256)[:, None, None] % 2 == 0, 0.25, 0.5) if kg > 0 else \
        np.where(np.arange(d)[None, None, :] % 2 == 0, 0.25, 0.5)
    k = (-2.0 + codes_k * ks).astype(np.float16)
    v = (-1.0 + codes_v * 0.125).astype(np.float16)
    pool = _pool(orc, lay, n)
    ids = np.array([1, 0], np.int32)
    orc.quantize_blocks(lay, pool, ids, k.view(np.uint16), v.view(np.uint16))
    kk, vv = orc.dequantize_blocks(lay, pool, ids)
    assert np.array_equal(kk, k.view(np.uint16))
    assert np.array_equal(vv, v.view(np.uint16))


@pytest.mark.parametrize("rotate,kg,mixed", [(0, 32, 0), (1, 32, 0), (1, -1, 0), (1, 64, 1), (0, 64, 1)])
def test_restored_rows_within_stored_scale_bound(orc, rotate, kg, mixed):
    # In the stored domain every element is within s / 2 of its (rotated) input when the input lies inside
    # [z, z + L s] (up to the fp32 roundings of the quantiser, relative L * 4 * 2^-24 of s), and within its
    # distance to that interval plus s / 2 otherwise. Undoing the rotation with (1 / (d c)) H multiplies the
    # L2 norm of an error by 1 / (c sqrt(d)), so per row
    #   || x - restored ||_2 <= || per-element bound ||_2 / (c sqrt(d)) + || half an fp16 ulp of restored ||_2.
    d, H, vg = 128, 2, 32
    lay = _layout(orc, d, kg, vg, rotate, mixed, H)
    rng = np.random.default_rng(7 + rotate + 2 * mixed)
    n = 2
    x = rng.standard_normal((2, n * 256, H, d)).astype(np.float32)
    x[:, :, :, 5] *= 10.0  # an outlier channel
    xk, xv = x[0].astype(np.float16), x[1].astype(np.float16)
    prec = None
    if mixed:
        prec = rng.integers(0, 2 ** 32, (n, 8), dtype=np.uint64).astype(np.uint32)
    pool = _pool(orc, lay, n)
    ids = np.array([0, 1], np.int32)
    orc.quantize_blocks(lay, pool, ids, xk.view(np.uint16), xv.view(np.uint16), prec)
    kk, vv = orc.dequantize_blocks(lay, pool, ids)
    c = float(orc.rot_scale(d)) if rotate else 1.0
    tb = orc.tile_bytes(lay)
    checked = 0
    for i in range(n):
        for h in range(H):
            tile = pool[(i * H + h) * tb:(i * H + h + 1) * tb]
            _, off_par, off_prow, prow, kpr, off_hdr, _ = brute._layout_offsets(d, kg, vg, mixed)
            bits = np.full(256, 4)
            if mixed:
                hdr = tile[off_hdr:off_hdr + 32]
                bits = np.where((hdr[np.arange(256) // 8] >> (np.arange(256) % 8)) & 1, 8, 4)
            par = tile[off_prow:off_prow + 256 * prow].reshape(256, prow)
            for which, src, got in ((0, xk, kk), (1, xv, vv)):
                rows = src[i * 256:(i + 1) * 256, h].astype(np.float32)
                if rotate:
                    xr = np.stack([orc.fwht_f32(r) for r in rows]) * np.float32(c)
                else:
                    xr = rows
                xr = xr.astype(np.float64)
                if which == 0 and kg < 0:
                    p = tile[off_par:off_par + d * 4].view(np.float16).reshape(d, 2).astype(np.float64)
                    s, z = np.broadcast_to(p[:, 0], (256, d)), np.broadcast_to(p[:, 1], (256, d))
                else:
                    g = kg if which == 0 else vg
                    off = 0 if which == 0 else kpr * 4
                    p = par[:, off:off + (d // g) * 4].copy().view(np.float16).reshape(256, d // g, 2)
                    s = np.repeat(p[:, :, 0].astype(np.float64), g, axis=1)
                    z = np.repeat(p[:, :, 1].astype(np.float64), g, axis=1)
                L = np.where(bits == 8, 255.0, 15.0)[:, None]
                dist = np.maximum(z - xr, 0) + np.maximum(xr - (z + L * s), 0)
                elem = dist + s * (0.5 + L * 4 * 2.0 ** -24) + np.abs(xr) * 2.0 ** -22
                restored = got[i * 256:(i + 1) * 256, h].view(np.float16).astype(np.float64)
                ulp = np.spacing(np.abs(restored).astype(np.float16)).astype(np.float64)
                bound = np.sqrt((elem ** 2).sum(1)) / (c * np.sqrt(d) if rotate else 1.0) + \
                    np.sqrt(((ulp / 2) ** 2).sum(1))
                err = np.sqrt(((restored - src[i * 256:(i + 1) * 256, h].astype(np.float64)) ** 2).sum(1))
                assert np.all(err <= bound * (1 + 1e-9)), (i, h, which, float((err / bound).max()))
                checked += 256
    assert checked == n * H * 2 * 256


@pytest.mark.parametrize("rotate,kg,vg,mixed,d", [(1, 32, 32, 0, 128), (1, -1, 32, 0, 128), (1, 64, 64, 1, 64),
                                                 (0, 16, 64, 0, 64)])
def test_matches_dense_hadamard_and_numpy_rounding(orc, rotate, kg, vg, mixed, d):
    # Independent route: numpy's tile parser, the explicit +-1 Hadamard matrix and numpy's fp64 -> fp16 cast.
    H = 2
    lay = _layout(orc, d, kg, vg, rotate, mixed, H)
    rng = np.random.default_rng(11 + d)
    n = 2
    xk = (rng.standard_normal((n * 256, H, d)) * 2).astype(np.float16)
    xv = rng.standard_normal((n * 256, H, d)).astype(np.float16)
    prec = rng.integers(0, 2 ** 32, (n, 8), dtype=np.uint64).astype(np.uint32) if mixed else None
    pool = _pool(orc, lay, n)
    ids = np.array([1, 0], np.int32)
    orc.quantize_blocks(lay, pool, ids, xk.view(np.uint16), xv.view(np.uint16), prec)
    kk, vv = orc.dequantize_blocks(lay, pool, ids)
    tb = orc.tile_bytes(lay)
    Hm = brute.hadamard(d)
    unrot = 1.0 / (d * float(orc.rot_scale(d)))
    for i, b in enumerate(ids):
        for h in range(H):
            kt, vt = brute.dequant_tile(pool[(b * H + h) * tb:(b * H + h + 1) * tb], d, kg, vg, mixed)
            if rotate:
                kt, vt = (kt @ Hm.T) * unrot, (vt @ Hm.T) * unrot
            assert np.array_equal(kk[i * 256:(i + 1) * 256, h], kt.astype(np.float16).view(np.uint16))
            assert np.array_equal(vv[i * 256:(i + 1) * 256, h], vt.astype(np.float16).view(np.uint16))
