"""Pins of the oracle's quantisation and storage layout.

Pages: "Agent Memory Below the Prompt" technical summary 2.1 (256-token blocks; codes packed in uint32
words; one 16-bit scale and one 16-bit bias per group; about 72% less memory than FP16, i.e. 4x
capacity: 3 FP16 agents vs 12 Q4 agents at 8K context in a 10.2 GB budget, section 1 and 4.1);
QKVShare methodology (per-token widths). The pins are closed forms, hand-worked examples, invariants
and library routines (numpy's fp16 conversion), not the oracle's own formulas.
"""
import os

import numpy as np
import pytest

import kvq_workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f16(x):
    return np.float16(x)


# ------------------------------------------------------------------------------------------------ fp16

def test_f16_conversion_matches_numpy(orc):
    # numpy's float32 -> float16 cast is IEEE round-to-nearest-even with subnormals and overflow.
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-9, 6, 20000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -24, 2.0 ** -25,
                  2.0 ** -25 * 1.0000001, 2.0 ** -26, 6.1e-5, 6.103515625e-05, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, np.inf, -np.inf], np.float32),
        # exact halfway points between adjacent fp16 values (ties)
        ((np.arange(0, 65536, 97, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
          + np.nextafter(np.arange(0, 65536, 97, dtype=np.uint32).astype(np.uint16).view(np.float16),
                         np.float16(np.inf)).astype(np.float32)) / np.float32(2)),
    ]).astype(np.float32)
    vals = vals[np.isfinite(vals) | np.isinf(vals)]
    with np.errstate(over="ignore", invalid="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([orc.f32_to_f16_bits(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, ref)


def test_f16_to_f32_exact_all_patterns(orc):
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([orc.f16_bits_to_f32(int(b)) for b in bits], np.float32)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.all(np.isnan(got[np.isnan(ref)]))


# ------------------------------------------------------------------------------------------- one group

def test_tie_break_worked_example(orc):
    # Worked example (ours; the pages print none). min -2, max 1.75: scale = 3.75 / 15 = 0.25 and
    # zero = -2, both exact in fp16, r = 1 / 0.25 = 4 exact. The value -2 + 0.25 k + 0.125 maps to
    # (0.25 k + 0.125) * 4 = k + 0.5 exactly, a tie: round-half-to-even gives k for even k and k + 1 for
    # odd k (so -1.375 -> 2 and -1.125 -> 4). Values -2 + 0.25 k map to k exactly.
    ks_tie = np.arange(0, 14)
    ks_grid = np.arange(0, 16)
    x = np.concatenate([[-2.0, 1.75], -2 + 0.25 * ks_tie + 0.125, -2 + 0.25 * ks_grid])
    x = np.concatenate([x, np.full(64 - x.size, -2 + 0.25 * 7)]).astype(np.float32)
    expect = np.concatenate([[0, 15], np.where(ks_tie % 2 == 0, ks_tie, ks_tie + 1), ks_grid,
                             np.full(64 - 2 - ks_tie.size - ks_grid.size, 7)])
    codes, sh, zh = orc.quantize_group(x, 4)
    assert sh == int(f16(0.25).view(np.uint16)) and zh == int(f16(-2.0).view(np.uint16))
    assert np.array_equal(codes, expect)
    assert codes[2 + 2] == 2 and codes[2 + 3] == 4     # -1.375 -> 2, -1.125 -> 4


@pytest.mark.parametrize("bits", [4, 8])
def test_grid_exact_groups(orc, bits):
    # x = z + k s with z, s exact in fp16 and k spanning 0 .. L: max - min = L s exactly, so the scale is
    # s, every code is k and dequantisation k * s + z reproduces x exactly.
    L = (1 << bits) - 1
    rng = np.random.default_rng(bits)
    for _ in range(200):
        z = float(rng.integers(-400, 400)) * 2.0 ** -6
        s = float(rng.integers(1, 300)) * 2.0 ** -10
        k = rng.integers(0, L + 1, 64)
        k[rng.integers(64)] = 0
        k[(rng.integers(63) + 1 + np.argmin(k)) % 64] = L
        x = (z + k * s).astype(np.float32)
        assert np.array_equal(x.astype(np.float64), z + k * s)
        codes, sh, zh = orc.quantize_group(x, bits)
        assert np.array_equal(codes, k)
        assert sh == int(f16(s).view(np.uint16)) and zh == int(f16(z).view(np.uint16))
        assert np.array_equal(codes * s + z, x.astype(np.float64))


def test_constant_and_signed_zero_groups(orc):
    codes, sh, zh = orc.quantize_group(np.full(64, 0.3, np.float32), 4)
    assert sh == 0 and zh == int(f16(np.float32(0.3)).view(np.uint16)) and not codes.any()
    x = np.zeros(64, np.float32)
    x[::3] = -0.0
    codes, sh, zh = orc.quantize_group(x, 4)
    assert sh == 0 and zh == 0 and not codes.any()      # a zero minimum is stored as +0
    x = np.zeros(32, np.float32)
    x[:] = -0.0
    x[5] = 1.0
    codes, sh, zh = orc.quantize_group(x, 4)
    assert zh == 0 and codes[5] == 15


@pytest.mark.parametrize("bits", [4, 8])
def test_error_bound_from_stored_params(orc, bits):
    # Inside [z, z + L s] the decoded value k s + z is within s / 2 of x, up to the three fp32
    # roundings of (x - z) * (1 / s) (relative 3 * 2^-24 of at most L steps). Outside that interval the
    # code saturates at 0 or L. Codes computed from the unrounded scale would miss this bound by up to
    # L * 2^-11 steps near half-way points, which random groups hit many times.
    L = (1 << bits) - 1
    slack = L * 4 * 2.0 ** -24
    rng = np.random.default_rng(10 + bits)
    hits = 0
    for i in range(3000):
        x = rng.standard_normal(64).astype(np.float32) * np.float32(rng.choice([0.01, 1.0, 10.0, 300.0]))
        codes, sh, zh = orc.quantize_group(x, bits)
        s = float(np.uint16(sh).view(np.float16))
        z = float(np.uint16(zh).view(np.float16))
        assert s > 0
        assert codes.max() <= L
        xd = x.astype(np.float64)
        inside = (xd >= z) & (xd <= z + L * s)
        err = np.abs(codes * s + z - xd)
        assert np.all(err[inside] <= s * (0.5 + slack)), i
        assert np.all(codes[xd < z] == 0) and np.all(codes[xd > z + L * s] == L)
        e = (xd - z) / s
        hits += int(np.sum(inside & (np.abs(np.abs(e - np.floor(e)) - 0.5) < L * 2.0 ** -11)))
    assert hits > 100      # the bound was exercised close to half-way points


# ------------------------------------------------------------------------------------------- layout

@pytest.mark.parametrize("name,expect", [
    ("tiny_1k", 36864), ("gemma3_12b_4k", 73728), ("llama31_8b_pool_8k", 36864),
    ("qwen25_14b_prefix_32k", 37376), ("mixed_sentinel_32k", 69888)])
def test_tile_bytes(orc, name, expect):
    # 256 rows x (codes + params): d=128 g=64: 256 * (64 + 64 + 8 + 8) = 36864; d=256: 256 * 288;
    # per-channel K: 2 * 16384 + 128 * 4 + 256 * 4 * 4 = 37376; mixed d=128: 2 * 32768 + 2 * 2048 + 32
    # = 69664, padded to 69888.
    lay = orc.make_layout(**{k: v for k, v in W.CONFIGS[name].layout().items()})
    assert orc.tile_bytes(lay) == expect and expect % 256 == 0


def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, v = line.split("=")
                vals[k.strip()] = float(v)
    return vals


def test_storage_matches_pages_figures(orc):
    # The pages' capacity figures follow from the stored bytes per token at a Gemma-3-12B-like shape
    # (48 layers, 8 KV heads, head_dim 256) with groups of 64.
    g = read_golden("pages_storage_figures.txt")
    lay = orc.make_layout(256, 8, 64, 64)
    q4_per_token = orc.tile_bytes(lay) / 256 * 8 * 48
    fp16_per_token = 2 * 2 * 256 * 8 * 48
    assert abs(1 - q4_per_token / fp16_per_token - g["q4_memory_reduction"]) < 0.005
    assert round(fp16_per_token / q4_per_token) == g["q4_capacity_factor"]
    budget = g["cache_budget_gb"] * 2 ** 30
    ctx = g["context_tokens"]
    assert int(budget // (fp16_per_token * ctx)) == g["fp16_agents"]
    assert int(budget // (q4_per_token * ctx)) == g["q4_agents"]
    assert g["block_tokens"] == lay.block_tokens


def grid_rows(rng, n_rows, d, g, bits):
    """Rows whose every group is an exact grid with known codes; returns (fp16 bits, codes, s, z)."""
    # s = m 2^-e and z = z' 2^-e with |z' + k m| < 2048, so every z + k s is exact in fp16.
    L = (1 << bits) - 1
    m_max = 7 if bits == 8 else 100
    codes = rng.integers(0, L + 1, (n_rows, d))
    s = np.zeros((n_rows, d // g))
    z = np.zeros((n_rows, d // g))
    for t in range(n_rows):
        for k in range(d // g):
            codes[t, k * g] = 0
            codes[t, k * g + 1] = L
            e = int(rng.integers(8, 13))
            s[t, k] = float(rng.integers(1, m_max + 1)) * 2.0 ** -e
            z[t, k] = float(rng.integers(-200, 201)) * 2.0 ** -e
    x = codes * np.repeat(s, g, axis=1) + np.repeat(z, g, axis=1)
    assert np.array_equal(x.astype(np.float16).astype(np.float64), x)
    return x.astype(np.float16).view(np.uint16), codes, s, z


@pytest.mark.parametrize("mixed", [0, 1])
def test_tile_byte_positions(orc, mixed):
    # Codes, params and header land where the layout says: row record t at t * 2S holds the row's K codes
    # then, right after them, its V codes (d/2 bytes each for a 4-bit row, d for an 8-bit row); parameter
    # record t at 2 * 256 * S + t * P holds K params [group] {scale, zero} then V params; header last;
    # 4-bit codes low nibble first (codes (2, 4) -> byte 0x42); the rest of a record and the tail padding
    # are zero.
    d, H, g = 64, 2, 32
    rng = np.random.default_rng(5)
    lay = orc.make_layout(d, H, g, g, 0, mixed)
    tb = orc.tile_bytes(lay)
    wide = np.zeros(256, bool)
    if mixed:
        wide[rng.choice(256, 60, replace=False)] = True
    k = np.zeros((256, H, d), np.uint16)
    v = np.zeros_like(k)
    ref = {}
    for h in range(H):
        for name, arr in (("k", k), ("v", v)):
            xs, cs, ss, zs = [], [], [], []
            for t in range(256):
                xb, c, s, z = grid_rows(rng, 1, d, g, 8 if wide[t] else 4)
                arr[t, h] = xb[0]
                cs.append(c[0]); ss.append(s[0]); zs.append(z[0])
            ref[(name, h)] = (np.array(cs), np.array(ss), np.array(zs))
    prec = W.bits_words(wide) if mixed else None
    pool = np.zeros(3 * H * tb, np.uint8)
    orc.quantize_blocks(lay, pool, [1], k, v, prec)
    assert not pool[: H * tb].any() and not pool[2 * H * tb:].any()
    S = d * (8 if mixed else 4) // 8
    P = 2 * (d // g) * 4
    for h in range(H):
        tile = pool[(1 * H + h) * tb: (1 * H + h + 1) * tb]
        for name, base_p in (("k", 2 * 256 * S), ("v", 2 * 256 * S + (d // g) * 4)):
            codes, s, z = ref[(name, h)]
            for t in range(256):
                rec = tile[t * 2 * S: (t + 1) * 2 * S]
                n = d if wide[t] else d // 2          # code bytes of this row, for K and for V
                row = rec[:n] if name == "k" else rec[n: 2 * n]
                if wide[t]:
                    assert np.array_equal(row, codes[t].astype(np.uint8))
                else:
                    packed = (codes[t][0::2] | (codes[t][1::2] << 4)).astype(np.uint8)
                    assert np.array_equal(row, packed)
                assert not rec[2 * n:].any()
                par = tile[base_p + t * P: base_p + t * P + (d // g) * 4].view(np.float16)
                assert np.array_equal(par[0::2].astype(np.float64), s[t])
                assert np.array_equal(par[1::2].astype(np.float64), z[t])
        end = 2 * 256 * S + 2 * 256 * (d // g) * 4
        if mixed:
            hdr = tile[end: end + 32].view(np.uint32)
            assert np.array_equal(hdr, W.bits_words(wide)[0])
            end += 32
        assert not tile[end:].any()
    # nibble order on a literal pair: codes 2 then 4 share byte 0x42
    assert (2 | (4 << 4)) == 0x42


def test_per_channel_groups_are_columns(orc):
    # K grouped per channel over the block's 256 rows: a column that is an exact grid gets codes k.
    d, H = 64, 1
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, (256, d))
    codes[0] = 0
    codes[1] = 15
    s = rng.integers(1, 64, d) * 2.0 ** -10
    z = rng.integers(-64, 64, d) * 2.0 ** -7
    xf = codes * s + z
    assert np.array_equal(xf.astype(np.float16).astype(np.float64), xf)
    x = xf.astype(np.float16).view(np.uint16).reshape(256, 1, d)
    lay = orc.make_layout(d, H, -1, 32, 0, 0)
    tb = orc.tile_bytes(lay)
    pool = np.zeros(tb, np.uint8)
    orc.quantize_blocks(lay, pool, [0], x, x)
    S = d // 2
    got = np.zeros((256, d), np.int64)
    kc = pool[: 256 * 2 * S].reshape(256, 2 * S)[:, :S]
    got[:, 0::2] = kc & 0xF
    got[:, 1::2] = kc >> 4
    assert np.array_equal(got, codes)
    par = pool[2 * 256 * S: 2 * 256 * S + d * 4].view(np.float16)
    assert np.array_equal(par[0::2].astype(np.float64), s) and np.array_equal(par[1::2].astype(np.float64), z)


@pytest.mark.parametrize("rotate,mixed", [(0, 0), (1, 0), (0, 1)])
def test_append_equals_row_of_whole_block(orc, rotate, mixed):
    # Appending a token writes the same bytes that quantising it inside a whole block writes.
    d, H, g = 128, 2, 64
    lay = orc.make_layout(d, H, g, 32, rotate, mixed)
    tb = orc.tile_bytes(lay)
    rng = np.random.default_rng(11)
    k = rng.standard_normal((256, H, d)).astype(np.float16).view(np.uint16)
    v = rng.standard_normal((256, H, d)).astype(np.float16).view(np.uint16)
    wide = rng.random(256) < 0.3 if mixed else np.zeros(256, bool)
    whole = np.zeros(H * tb, np.uint8)
    orc.quantize_blocks(lay, whole, [0], k, v, W.bits_words(wide) if mixed else None)
    app = np.zeros(H * tb, np.uint8)
    table = np.zeros((1, 1), np.int32)
    for t in range(256):
        st = orc.append_tokens(lay, app, k[t:t + 1], v[t:t + 1], table, [t],
                               np.array([8 if wide[t] else 4], np.uint8) if mixed else None)
        assert st == 0
    assert np.array_equal(app, whole)


def test_append_rejects_per_channel(orc):
    lay = orc.make_layout(128, 1, -1, 32, 1, 0)
    pool = np.zeros(orc.tile_bytes(lay), np.uint8)
    z = np.zeros((1, 1, 128), np.uint16)
    assert orc.append_tokens(lay, pool, z, z, np.zeros((1, 1), np.int32), [0]) == orc.ORC_ERR_UNSUPPORTED


def test_layout_validation(orc):
    assert orc.check_layout(orc.make_layout(128, 8, 64, 64)) == 0
    assert orc.check_layout(orc.make_layout(128, 8, 48, 64)) == orc.ORC_ERR_ARG     # 48 does not divide 128
    assert orc.check_layout(orc.make_layout(96, 8, 32, 32, 1, 0)) == orc.ORC_ERR_UNSUPPORTED
    assert orc.check_layout(orc.make_layout(128, 8, -1, 32, 0, 1)) == orc.ORC_ERR_UNSUPPORTED
    assert orc.check_layout(orc.make_layout(128, 8, 64, 64, block_tokens=128)) == orc.ORC_ERR_ARG
