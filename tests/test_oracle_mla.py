"""Pins of the oracle with unequal K and V head dims (MLA models).

Page: "Agent Memory Below the Prompt", technical summary 2.2 (MLA models such as DeepSeek-Coder-V2-Lite have
K and V head dims that differ); the codec is that of technical summary 2.1 applied to each tensor at its own
length. The pins: byte positions of a hand-built grid-exact tile; each tensor's rows equal those of a pool
with equal dims fed the same tensor (K of a 256/128 pool as in a 256/256 pool, V as in a 128/128 pool);
append equals the same row of a whole block; restore and decode against the dense brute force (its own tile
parser, explicit Hadamard matrices of each length).
"""
import numpy as np
import pytest

from oracle import brute


def _lay(orc, d, dv, kg, vg, rotate=0, mixed=0, H=2):
    return orc.make_layout(d, H, kg, vg, rotate, mixed, v_head_dim=dv)


def test_layout_checks(orc):
    assert orc.check_layout(_lay(orc, 192, 128, 64, 64)) == 0
    assert orc.check_layout(_lay(orc, 256, 128, 64, 32, rotate=1)) == 0
    assert orc.check_layout(_lay(orc, 192, 128, 64, 64, rotate=1)) == orc.ORC_ERR_UNSUPPORTED
    assert orc.check_layout(_lay(orc, 192, 128, 64, 256)) == orc.ORC_ERR_ARG   # V group longer than dv
    assert orc.check_layout(_lay(orc, 192, 100, 64, 32)) == orc.ORC_ERR_ARG    # dv not a multiple of 8
    # v_head_dim equal to head_dim is the same layout as 0
    assert orc.tile_bytes(_lay(orc, 128, 128, 64, 64)) == orc.tile_bytes(_lay(orc, 128, 0, 64, 64))


def test_tile_bytes_and_positions_of_a_grid_exact_tile(orc):
    # K: 192 channels in groups of 64, V: 128 channels in groups of 32. Each group holds codes 0 and 15 and
    # values zero + code * scale exact in fp16, so codes and parameters are known in advance.
    d, dv, kg, vg, H = 192, 128, 64, 32, 1
    lay = _lay(orc, d, dv, kg, vg, H=H)
    rec = (d + dv) // 2
    prow = (d // kg + dv // vg) * 4
    assert orc.tile_bytes(lay) == (256 * rec + 256 * prow + 255) // 256 * 256
    rng = np.random.default_rng(1)
    ck = rng.integers(0, 16, (256, d))
    cv = rng.integers(0, 16, (256, dv))
    ck[:, 0::kg], ck[:, 1::kg] = 0, 15
    cv[:, 0::vg], cv[:, 1::vg] = 0, 15
    k = (-3.0 + ck * 0.5).astype(np.float16).reshape(256, 1, d)
    v = (1.0 + cv * 0.25).astype(np.float16).reshape(256, 1, dv)
    pool = np.zeros(orc.tile_bytes(lay), np.uint8)
    orc.quantize_blocks(lay, pool, np.array([0], np.int32), k.view(np.uint16), v.view(np.uint16))
    for t in (0, 1, 100, 255):
        r = pool[t * rec:(t + 1) * rec]
        kb = r[: d // 2]
        vb = r[d // 2:]
        assert np.array_equal(kb & 15, ck[t, 0::2]) and np.array_equal(kb >> 4, ck[t, 1::2])
        assert np.array_equal(vb & 15, cv[t, 0::2]) and np.array_equal(vb >> 4, cv[t, 1::2])
        p = pool[256 * rec + t * prow: 256 * rec + (t + 1) * prow].view(np.float16)
        assert np.array_equal(p[0:2 * (d // kg):2], np.full(d // kg, 0.5, np.float16))
        assert np.array_equal(p[1:2 * (d // kg):2], np.full(d // kg, -3.0, np.float16))
        assert np.array_equal(p[2 * (d // kg)::2], np.full(dv // vg, 0.25, np.float16))
        assert np.array_equal(p[2 * (d // kg) + 1::2], np.full(dv // vg, 1.0, np.float16))


@pytest.mark.parametrize("rotate,mixed", [(0, 0), (1, 0), (1, 1), (0, 2)])
def test_each_tensor_as_in_a_pool_of_equal_dims(orc, rotate, mixed):
    # K of a 256/128 pool dequantises as K of a 256/256 pool; V as V of a 128/128 pool (same inputs, same
    # widths): the record split, the parameter split and the per-tensor rotation length are all pinned.
    H = 2
    rng = np.random.default_rng(3 + rotate + 2 * mixed)
    k = rng.standard_normal((256, H, 256)).astype(np.float16)
    v = rng.standard_normal((256, H, 128)).astype(np.float16)
    v2 = rng.standard_normal((256, H, 256)).astype(np.float16)
    k2 = rng.standard_normal((256, H, 128)).astype(np.float16)
    words = None
    if mixed == 1:
        words = rng.integers(0, 2 ** 32, (1, 8), dtype=np.uint64).astype(np.uint32)
    elif mixed == 2:
        words = rng.integers(0, 2 ** 32, (1, 16), dtype=np.uint64).astype(np.uint32)
    ids = np.array([0], np.int32)

    def build(d, dv, kk, vv):
        lay = _lay(orc, d, dv, 64, 32, rotate, mixed, H)
        pool = np.zeros(orc.tile_bytes(lay) * H, np.uint8)
        orc.quantize_blocks(lay, pool, ids, kk.view(np.uint16), vv.view(np.uint16), words)
        return lay, pool

    mla = build(256, 128, k, v)
    ke = build(256, 256, k, v2)
    ve = build(128, 128, k2, v)
    for h in range(H):
        for t in (0, 7, 128, 255):
            def row(lp):
                lay, pool = lp
                tb = orc.tile_bytes(lay)
                return orc.dequant_row(lay, pool[h * tb:(h + 1) * tb], t)
            a, b, c = row(mla), row(ke), row(ve)
            assert a[2] == b[2] == c[2]
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], c[1])
    kr, vr = orc.dequantize_blocks(mla[0], mla[1], ids)
    kb, _ = orc.dequantize_blocks(ke[0], ke[1], ids)
    _, vc = orc.dequantize_blocks(ve[0], ve[1], ids)
    assert np.array_equal(kr, kb) and np.array_equal(vr, vc)


@pytest.mark.parametrize("d,rotate,mixed", [(192, 0, 0), (256, 1, 0), (192, 0, 2), (256, 1, 1)])
def test_append_equals_row_of_whole_block(orc, d, rotate, mixed):
    dv, H = 128, 2
    lay = _lay(orc, d, dv, 64, 64, rotate, mixed, H)
    rng = np.random.default_rng(5 + d + mixed)
    k = rng.standard_normal((256, H, d)).astype(np.float16)
    v = rng.standard_normal((256, H, dv)).astype(np.float16)
    rows = [0, 31, 32, 200, 255]
    prec = None
    words = None
    if mixed:
        bits = rng.choice([4, 8] if mixed == 1 else [2, 4, 8, 16], 256)
        if mixed == 1:
            words = np.zeros((1, 8), np.uint32)
            for t in range(256):
                if bits[t] == 8:
                    words[0, t // 32] |= np.uint32(1 << (t % 32))
        else:
            code = {2: 0, 4: 1, 8: 2, 16: 3}
            words = np.zeros((1, 16), np.uint64)
            for t in range(256):
                words[0, t // 16] |= np.uint64(code[int(bits[t])] << (2 * (t % 16)))
            words = words.astype(np.uint32)
        prec = bits[rows].astype(np.uint8)
    whole = np.zeros(orc.tile_bytes(lay) * H, np.uint8)
    orc.quantize_blocks(lay, whole, np.array([0], np.int32), k.view(np.uint16), v.view(np.uint16), words)
    built = np.zeros_like(whole)
    table = np.zeros((len(rows), 1), np.int32)
    assert orc.append_tokens(lay, built, k[rows].view(np.uint16), v[rows].view(np.uint16), table,
                             np.array(rows, np.int32), prec) == 0
    tb = orc.tile_bytes(lay)
    for h in range(H):
        for r in rows:
            a = orc.dequant_row(lay, whole[h * tb:(h + 1) * tb], r)
            b = orc.dequant_row(lay, built[h * tb:(h + 1) * tb], r)
            assert a[2] == b[2] and np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("d,rotate,mixed", [(192, 0, 0), (256, 1, 0), (192, 0, 2)])
def test_decode_and_restore_match_dense_brute_force(orc, d, rotate, mixed):
    dv, H, G, kg, vg = 128, 2, 3, 64, 32
    lay = _lay(orc, d, dv, kg, vg, rotate, mixed, H)
    rng = np.random.default_rng(9 + d + mixed)
    nb = 3
    k = (rng.standard_normal((nb * 256, H, d)) * 2).astype(np.float16)
    v = rng.standard_normal((nb * 256, H, dv)).astype(np.float16)
    words = None
    if mixed == 2:
        words = rng.integers(0, 2 ** 32, (nb, 16), dtype=np.uint64).astype(np.uint32)
    pool = np.zeros(orc.tile_bytes(lay) * H * nb, np.uint8)
    ids = np.array([2, 0, 1], np.int32)
    orc.quantize_blocks(lay, pool, ids, k.view(np.uint16), v.view(np.uint16), words)
    q = rng.standard_normal((2, H * G, d)).astype(np.float16).view(np.uint16)
    table = np.array([[2, 0, 1], [1, 2, 0]], np.int32)
    lens = np.array([700, 257], np.int32)
    mask = np.zeros((2, 22), np.uint32)
    mask[0, 5] = 0x0FF00FF0
    out = orc.decode_attention(lay, pool, q, table, lens, mask)
    assert out.shape == (2, H * G, dv)
    ref = brute.decode_attention(pool, d, H, kg, vg, rotate, mixed, q, table, lens, mask, dv=dv)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    # restore: the brute force's own parse, explicit Hadamard matrices of each length, numpy's fp16 cast
    kk, vv = orc.dequantize_blocks(lay, pool, ids)
    tb = orc.tile_bytes(lay)
    for i, b in enumerate(ids):
        for h in range(H):
            kt, vt = brute.dequant_tile(pool[(b * H + h) * tb:(b * H + h + 1) * tb], d, kg, vg, mixed, dv=dv)
            if rotate:
                kt = (kt @ brute.hadamard(d).T) / (d * float(orc.rot_scale(d)))
                vt = (vt @ brute.hadamard(dv).T) / (dv * float(orc.rot_scale(dv)))
            assert np.array_equal(kk[i * 256:(i + 1) * 256, h], kt.astype(np.float16).view(np.uint16))
            assert np.array_equal(vv[i * 256:(i + 1) * 256, h], vt.astype(np.float16).view(np.uint16))
