"""Pins of the oracle's FP8 (E4M3) pool format, the KV-cache baseline the UltraQuant article measures the
4-bit cache against (technology section: FP8 as today's practical standard).

The pins: the format's published anchor values, torch's own E4M3 conversion (round to nearest even) inside
the finite range, saturation beyond it, and decode attention against the dense fp64 brute force reading the
bytes through a numpy table built from the format's definition.
"""
import numpy as np
import pytest
import torch

from oracle import brute


def test_anchor_values_of_the_format(orc):
    anchors = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5,
               0x40: 2.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for b, v in anchors.items():
        assert orc.e4m3_to_f32(b) == v and np.signbit(orc.e4m3_to_f32(b)) == np.signbit(v), hex(b)
        assert orc.f32_to_e4m3(v) == b, hex(b)
    assert np.isnan(orc.e4m3_to_f32(0x7F)) and np.isnan(orc.e4m3_to_f32(0xFF))
    assert orc.f32_to_e4m3(float("nan")) == 0x7F


def test_every_code_round_trips_and_matches_torch_and_the_table(orc):
    table = brute.e4m3_values()
    tvals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for b in range(256):
        v = orc.e4m3_to_f32(b)
        if np.isnan(table[b]):
            assert np.isnan(v) and np.isnan(tvals[b])
            continue
        assert v == table[b] == tvals[b]
        if b != 0x80:
            assert orc.f32_to_e4m3(v) == b


def test_rounding_matches_torch_inside_the_range(orc):
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.6, 20000),
        # every midpoint between neighbouring finite codes (ties go to the even code)
        (brute.e4m3_values()[0:126] + brute.e4m3_values()[1:127]) / 2,
        -(brute.e4m3_values()[0:126] + brute.e4m3_values()[1:127]) / 2,
        np.array([463.99, -463.99, 447.9, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -12]),
    ]).astype(np.float32)
    x = x[np.abs(x) < 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.f32_to_e4m3(float(v)) for v in x], np.uint8)
    assert np.array_equal(got, ref)


def test_saturation(orc):
    for v, b in ((464.0, 0x7E), (480.0, 0x7E), (1e9, 0x7E), (-500.0, 0xFE), (float("inf"), 0x7E),
                 (float("-inf"), 0xFE)):
        assert orc.f32_to_e4m3(v) == b, v


@pytest.mark.parametrize("rotate", [0, 1])
def test_fp8_pool_decode_matches_dense_brute_force(orc, rotate):
    d, H, G, n_seqs = 64, 2, 3, 2
    lay = orc.make_layout(d, H, 0, 0, rotate, 0, format=1)
    assert orc.check_layout(lay) == 0 and orc.tile_bytes(lay) == 256 * 2 * d
    rng = np.random.default_rng(5 + rotate)
    n_blocks = 3
    k = (rng.standard_normal((n_blocks * 256, H, d)) * 3).astype(np.float16)
    k[:, :, 7] *= 40  # beyond 448 after the outlier: saturates
    v = rng.standard_normal((n_blocks * 256, H, d)).astype(np.float16)
    pool = np.zeros(orc.tile_bytes(lay) * H * n_blocks, np.uint8)
    ids = np.array([2, 0, 1], np.int32)
    orc.quantize_blocks(lay, pool, ids, k.view(np.uint16), v.view(np.uint16))
    if not rotate:  # stored bytes are the E4M3 rounding of the inputs (torch inside the range, saturation outside)
        tb = orc.tile_bytes(lay)
        rec = pool.reshape(n_blocks, H, 256, 2 * d)
        kf = k.astype(np.float32)
        want = torch.from_numpy(np.clip(kf, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        for i, b in enumerate(ids):
            assert np.array_equal(rec[b, :, :, :d], want[i * 256:(i + 1) * 256].transpose(1, 0, 2))
    q = rng.standard_normal((n_seqs, H * G, d)).astype(np.float16).view(np.uint16)
    table = np.array([[2, 0, 1], [1, 2, 0]], np.int32)
    lens = np.array([700, 513], np.int32)
    out = orc.decode_attention(lay, pool, q, table, lens)
    ref = brute.decode_attention(pool, d, H, 0, 0, rotate, 0, q, table, lens, fmt=1)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_fp8_layout_validation(orc):
    assert orc.check_layout(orc.make_layout(64, 2, 0, 0, 0, 0, format=1)) == 0
    assert orc.check_layout(orc.make_layout(64, 2, 32, 0, 0, 0, format=1)) != 0  # no groups in FP8 pools
    assert orc.check_layout(orc.make_layout(64, 2, 0, 0, 0, 1, format=1)) != 0   # no per-token widths
    assert orc.check_layout(orc.make_layout(64, 2, 64, 64, 0, 0, format=2)) != 0
