"""Pins of the oracle's per-token widths {2, 4, 8, FP16} (pools with mixed = 2).

Pages: QKVShare methodology section (per-token bit widths drawn from {2, 4, 8, FP16}); "Agent Memory Below
the Prompt" technical summary 2.1 (the stored form: codes plus a 16-bit scale and bias per group). The pins:
2-bit groups on their grid come back exactly, the stored-scale error bound at 2 bits, FP16 rows equal the
fp16 rounding of their (rotated) input, tile bytes at the documented positions, an appended row of each
width equals the same row inside a whole block, and decode attention against the dense brute force.
"""
import numpy as np
import pytest

from oracle import brute


def _lay(orc, d=64, H=2, kg=32, vg=32, rotate=0):
    return orc.make_layout(d, H, kg, vg, rotate, 2)


def _width_words(codes):
    """codes: [n_blocks][256] width codes 0..3 -> the 16 uint32 width words of each block."""
    n = codes.shape[0]
    w = np.zeros((n, 16), np.uint64)
    for t in range(256):
        w[:, t // 16] |= codes[:, t].astype(np.uint64) << np.uint64(2 * (t % 16))
    return w.astype(np.uint32)


def test_two_bit_grid_groups_and_error_bound(orc):
    # Grid-exact: values z + k s with k in 0..3 (both ends present) come back exactly.
    for s, z in ((0.5, -1.0), (0.25, 3.0), (2.0, -3.0)):
        k = np.array([0, 3, 1, 2, 2, 1, 0, 3] * 4)
        x = (z + k * s).astype(np.float32)
        codes, sh, zh = orc.quantize_group(x, 2)
        assert np.array_equal(codes, k)
        assert float(np.uint16(sh).view(np.float16)) == s and float(np.uint16(zh).view(np.float16)) == z
    # Error bound at L = 3 from the stored parameters (inside [z, z + 3 s]).
    rng = np.random.default_rng(2)
    for i in range(2000):
        x = rng.standard_normal(32).astype(np.float32) * np.float32(rng.choice([0.01, 1.0, 30.0]))
        codes, sh, zh = orc.quantize_group(x, 2)
        s = float(np.uint16(sh).view(np.float16))
        z = float(np.uint16(zh).view(np.float16))
        assert codes.max() <= 3
        xd = x.astype(np.float64)
        inside = (xd >= z) & (xd <= z + 3 * s)
        assert np.all(np.abs(codes * s + z - xd)[inside] <= s * (0.5 + 3 * 4 * 2.0 ** -24)), i


def test_tile_bytes_and_positions(orc):
    d, H, kg, vg = 64, 2, 32, 32
    lay = _lay(orc, d, H, kg, vg)
    rec = 2 * 2 * d                      # K and V slots of FP16 width
    prow = (d // kg + d // vg) * 4
    assert orc.tile_bytes(lay) == (256 * rec + 256 * prow + 64 + 255) // 256 * 256
    rng = np.random.default_rng(3)
    widths = rng.integers(0, 4, (1, 256))
    x = (rng.standard_normal((256, H, d))).astype(np.float16)
    pool = np.zeros(orc.tile_bytes(lay) * H, np.uint8)
    orc.quantize_blocks(lay, pool, np.array([0], np.int32), x.view(np.uint16), x.view(np.uint16),
                        _width_words(widths))
    tile = pool[: orc.tile_bytes(lay)]
    hdr = tile[256 * rec + 256 * prow: 256 * rec + 256 * prow + 64]
    for t in range(256):
        assert (hdr[t // 4] >> (2 * (t % 4))) & 3 == widths[0, t]
        b = 2 << widths[0, t]
        r = tile[t * rec:(t + 1) * rec]
        assert not r[2 * d * b // 8:].any()  # the rest of a narrower row's record is zero
        if b == 16:  # K then V as raw fp16
            assert np.array_equal(r[:2 * d].view(np.uint16), x[t, 0].view(np.uint16))
            assert not tile[256 * rec + t * prow: 256 * rec + (t + 1) * prow].any()


def test_blocks_without_width_words_are_four_bit(orc):
    # No width words: every row is 4-bit, and each row's codes and parameters are those of a pool with a
    # single width (mixed = 0) fed the same input; the header says 4 bits for every row.
    d, H = 64, 2
    lay = _lay(orc, d, H, 32, 32)
    one = orc.make_layout(d, H, 32, 32, 0, 0)
    rng = np.random.default_rng(5)
    k = rng.standard_normal((256, H, d)).astype(np.float16)
    v = rng.standard_normal((256, H, d)).astype(np.float16)
    pool = np.zeros(orc.tile_bytes(lay) * H, np.uint8)
    ref = np.zeros(orc.tile_bytes(one) * H, np.uint8)
    orc.quantize_blocks(lay, pool, np.array([0], np.int32), k.view(np.uint16), v.view(np.uint16))
    orc.quantize_blocks(one, ref, np.array([0], np.int32), k.view(np.uint16), v.view(np.uint16))
    tb, tr = orc.tile_bytes(lay), orc.tile_bytes(one)
    for h in range(H):
        for t in (0, 1, 77, 255):
            a = orc.dequant_row(lay, pool[h * tb:(h + 1) * tb], t)
            b = orc.dequant_row(one, ref[h * tr:(h + 1) * tr], t)
            assert a[2] == b[2] == 4
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("rotate", [0, 1])
def test_append_equals_row_of_whole_block(orc, rotate):
    d, H = 64, 2
    lay = _lay(orc, d, H, 32, 32, rotate)
    rng = np.random.default_rng(4 + rotate)
    widths = rng.integers(0, 4, (1, 256))
    k = rng.standard_normal((256, H, d)).astype(np.float16)
    v = rng.standard_normal((256, H, d)).astype(np.float16)
    whole = np.zeros(orc.tile_bytes(lay) * H, np.uint8)
    orc.quantize_blocks(lay, whole, np.array([0], np.int32), k.view(np.uint16), v.view(np.uint16),
                        _width_words(widths))
    rows = [3, 100, 101, 102, 255]
    built = np.zeros_like(whole)
    # each row is first appended at another width, so the second append has to clear the whole record
    # and rewrite its header field
    table = np.zeros((len(rows), 1), np.int32)
    pos = np.array(rows, np.int32)
    prec = np.array([2 << int(widths[0, r]) for r in rows], np.uint8)
    wrong = np.array([2 << int(3 - widths[0, r]) for r in rows], np.uint8)
    assert orc.append_tokens(lay, built, k[rows].view(np.uint16), v[rows].view(np.uint16), table, pos, wrong) == 0
    assert orc.append_tokens(lay, built, k[rows].view(np.uint16), v[rows].view(np.uint16), table, pos, prec) == 0
    tb = orc.tile_bytes(lay)
    # a width the pool does not hold stores the row at 4 bits, as if 4 had been given
    odd = np.zeros_like(whole)
    four = np.zeros_like(whole)
    for buf, w in ((odd, 5), (four, 4)):
        assert orc.append_tokens(lay, buf, k[rows].view(np.uint16), v[rows].view(np.uint16), table, pos,
                                 np.full(len(rows), w, np.uint8)) == 0
    assert np.array_equal(odd, four)
    for h in range(H):
        for r in rows:
            a = orc.dequant_row(lay, whole[h * tb:(h + 1) * tb], r)
            b = orc.dequant_row(lay, built[h * tb:(h + 1) * tb], r)
            assert a[2] == b[2] == 2 << int(widths[0, r])
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("rotate", [0, 1])
def test_decode_matches_dense_brute_force(orc, rotate):
    d, H, G, kg, vg = 64, 2, 3, 32, 16
    lay = _lay(orc, d, H, kg, vg, rotate)
    rng = np.random.default_rng(9 + rotate)
    n_blocks = 3
    widths = rng.integers(0, 4, (n_blocks, 256))
    k = (rng.standard_normal((n_blocks * 256, H, d)) * 2).astype(np.float16)
    v = rng.standard_normal((n_blocks * 256, H, d)).astype(np.float16)
    pool = np.zeros(orc.tile_bytes(lay) * H * n_blocks, np.uint8)
    orc.quantize_blocks(lay, pool, np.array([1, 2, 0], np.int32), k.view(np.uint16), v.view(np.uint16),
                        _width_words(widths))
    q = rng.standard_normal((2, H * G, d)).astype(np.float16).view(np.uint16)
    table = np.array([[2, 0, 1], [0, 1, 2]], np.int32)
    lens = np.array([700, 300], np.int32)
    mask = np.zeros((2, 22), np.uint32)
    mask[0, 3] = 0xF0F0F0F0
    out = orc.decode_attention(lay, pool, q, table, lens, mask)
    ref = brute.decode_attention(pool, d, H, kg, vg, rotate, 2, q, table, lens, mask)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
