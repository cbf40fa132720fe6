"""Pins of the oracle's decode attention over the quantised cache.

Pages: "Agent Memory Below the Prompt" technical summary 2.1 (attention reads the quantised cache
directly; agents batched) and 2.2 (GQA); IntentKV invalidation section (a sentinel slot's key is -1e4
so its softmax weight is zero); UltraQuant technology section (rotation). Pins: an independent dense
numpy brute force (explicit Hadamard matrix, matrix products), closed-form special cases and the
sentinel invariants.
"""
import numpy as np
import pytest

import kvq_workloads as W
from oracle import brute


def small_case(rng, d, h_kv, g, k_group, v_group, rotate, mixed, lens, sentinel_frac=0.0, scale_k=1.0):
    n = len(lens)
    nblk = [(L + 255) // 256 for L in lens]
    num_blocks = sum(nblk) + 1
    perm = rng.permutation(num_blocks)
    table = np.zeros((n, max(1, max(nblk))), np.int32)
    off = 0
    for s in range(n):
        table[s, :nblk[s]] = perm[off: off + nblk[s]]
        off += nblk[s]
    k = (rng.standard_normal((num_blocks * 256, h_kv, d)) * scale_k).astype(np.float16).view(np.uint16)
    v = rng.standard_normal((num_blocks * 256, h_kv, d)).astype(np.float16).view(np.uint16)
    q = rng.standard_normal((n, h_kv * g, d)).astype(np.float16).view(np.uint16)
    prec = W.bits_words(rng.random(num_blocks * 256) < 0.25) if mixed else None
    mask = None
    if sentinel_frac > 0:
        words = (max(lens) + 31) // 32
        mask = np.zeros((n, max(words, 1)), np.uint32)
        for s in range(n):
            dead = rng.random(lens[s]) < sentinel_frac
            idx = np.nonzero(dead)[0]
            np.bitwise_or.at(mask[s], idx // 32, (np.uint32(1) << (idx % 32).astype(np.uint32)))
    return dict(num_blocks=num_blocks, table=table, k=k, v=v, q=q, prec=prec, mask=mask,
                lens=np.array(lens, np.int32))


def build_pool(orc, lay, c):
    pool = np.zeros(orc.tile_bytes(lay) * lay.num_kv_heads * c["num_blocks"], np.uint8)
    orc.quantize_blocks(lay, pool, np.arange(c["num_blocks"], dtype=np.int32), c["k"], c["v"], c["prec"])
    return pool


LAYOUTS = [
    # d, h_kv, G, k_group, v_group, rotate, mixed
    (64, 2, 1, 32, 32, 0, 0),
    (128, 2, 4, 64, 64, 0, 0),
    (128, 1, 5, -1, 32, 1, 0),
    (128, 2, 2, 64, 64, 0, 1),
    (256, 1, 2, 64, 64, 0, 0),
    (64, 1, 3, 32, 64, 1, 1),
]


@pytest.mark.parametrize("spec", LAYOUTS)
@pytest.mark.parametrize("sentinel", [0.0, 0.6])
def test_matches_dense_brute_force(orc, spec, sentinel):
    d, h_kv, g, kg, vg, rot, mixed = spec
    rng = np.random.default_rng(hash((spec, sentinel)) & 0xFFFF)
    c = small_case(rng, d, h_kv, g, kg, vg, rot, mixed, [300, 1, 0, 512, 77], sentinel)
    lay = orc.make_layout(d, h_kv, kg, vg, rot, mixed)
    pool = build_pool(orc, lay, c)
    got = orc.decode_attention(lay, pool, c["q"], c["table"], c["lens"], c["mask"])
    ref = brute.decode_attention(pool, d, h_kv, kg, vg, rot, mixed, c["q"], c["table"], c["lens"], c["mask"])
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
    assert not got[2].any()                                   # seq_len 0 -> zeros


def test_single_slot_returns_its_value_row(orc):
    # seq_len 1: softmax over one logit is 1, so the output is that slot's dequantised V row.
    d, h = 128, 2
    rng = np.random.default_rng(3)
    c = small_case(rng, d, h, 2, 64, 64, 0, 0, [1])
    lay = orc.make_layout(d, h, 64, 64)
    pool = build_pool(orc, lay, c)
    out = orc.decode_attention(lay, pool, c["q"], c["table"], c["lens"])
    tb = orc.tile_bytes(lay)
    for kvh in range(h):
        blk = c["table"][0, 0]
        _, v0, _ = orc.dequant_row(lay, pool[(blk * h + kvh) * tb: (blk * h + kvh + 1) * tb], 0)
        for j in range(2):
            assert np.array_equal(out[0, kvh * 2 + j], v0)


def test_equal_keys_give_mean_of_values(orc):
    # Identical K rows dequantise identically, all logits tie, weights are 1/n: out = mean of V rows.
    d, h, n = 64, 1, 300
    rng = np.random.default_rng(4)
    c = small_case(rng, d, h, 1, 32, 32, 0, 0, [n])
    c["k"][:] = c["k"][0]
    lay = orc.make_layout(d, h, 32, 32)
    pool = build_pool(orc, lay, c)
    out, w = orc.decode_attention(lay, pool, c["q"], c["table"], c["lens"], want_weights=True)
    assert np.allclose(w[0, 0, :n], 1.0 / n, rtol=1e-14, atol=0)
    tb = orc.tile_bytes(lay)
    vs = []
    for t in range(n):
        blk = c["table"][0, t // 256]
        vs.append(orc.dequant_row(lay, pool[blk * tb:(blk + 1) * tb], t % 256)[1])
    assert np.allclose(out[0, 0], np.mean(vs, axis=0), rtol=0, atol=1e-13)


def test_gqa_head_mapping_reduces_to_mha(orc):
    # With G query heads per KV head, head j must read KV head j // G (contiguous groups): the result for
    # head j equals an MHA call (G = 1) with only query head j // G's slice in the right place.
    d, h, g = 64, 3, 4
    rng = np.random.default_rng(5)
    c = small_case(rng, d, h, g, 32, 32, 0, 0, [400, 130])
    lay = orc.make_layout(d, h, 32, 32)
    pool = build_pool(orc, lay, c)
    full = orc.decode_attention(lay, pool, c["q"], c["table"], c["lens"])
    qb = c["q"].reshape(2, h, g, d)
    for jj in range(g):
        mha = orc.decode_attention(lay, pool, np.ascontiguousarray(qb[:, :, jj]), c["table"], c["lens"])
        assert np.array_equal(mha, full.reshape(2, h, g, d)[:, :, jj])


def test_sentinel_weights_and_all_sentinel(orc):
    # A sentinel slot's softmax weight is below 1e-30 (exactly 0: e^-1e4 underflows in fp64); remapping
    # every slot to the sentinel leaves value rows of 0, so the output is 0.
    d, h = 128, 2
    rng = np.random.default_rng(6)
    c = small_case(rng, d, h, 4, 64, 64, 0, 0, [700, 700], sentinel_frac=0.7)
    c["mask"][1, :] = 0xFFFFFFFF
    lay = orc.make_layout(d, h, 64, 64)
    pool = build_pool(orc, lay, c)
    out, w = orc.decode_attention(lay, pool, c["q"], c["table"], c["lens"], c["mask"], want_weights=True)
    t = np.arange(700)
    sent0 = ((c["mask"][0][t // 32] >> (t % 32)) & 1).astype(bool)
    assert sent0.sum() > 300
    assert np.all(w[0][:, sent0] < 1e-30)
    assert np.allclose(w[0].sum(axis=1), 1.0, rtol=1e-13)
    assert not out[1].any()
    # Invalidation without compaction: plain softmax attention over the surviving slots alone (no
    # sentinel in sight) gives the same output, because the sentinel weights are exactly zero.
    keep = np.nonzero(~sent0)[0]
    tb = orc.tile_bytes(lay)
    q = c["q"].view(np.float16).astype(np.float64)
    for kvh in range(h):
        K = np.zeros((700, d))
        V = np.zeros((700, d))
        for lb in range(3):
            blk = c["table"][0, lb]
            Kt, Vt = brute.dequant_tile(pool[(blk * h + kvh) * tb:(blk * h + kvh + 1) * tb], d, 64, 64, 0)
            m = min(256, 700 - lb * 256)
            K[lb * 256: lb * 256 + m] = Kt[:m]
            V[lb * 256: lb * 256 + m] = Vt[:m]
        logits = float(np.float32(1 / np.sqrt(d))) * (q[0, kvh * 4:(kvh + 1) * 4] @ K[keep].T)
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        ref = (p / p.sum(axis=1, keepdims=True)) @ V[keep]
        assert np.allclose(out[0, kvh * 4:(kvh + 1) * 4], ref, rtol=0, atol=1e-12)


def test_rotation_round_trip_bound(orc):
    # Un-rotating the decoded rows of a rotated pool lands within the quantisation error of the original
    # rows: |x_rot - x_hat_rot| <= s/2 per element (plus fp32 slack), and (1/(d c)) H is orthogonal up to
    # the rounding of c, so ||x - unrot(x_hat_rot)||_2 <= sqrt(sum of (s/2)^2) * (1 + 1e-6) + fp32 slack.
    d = 128
    rng = np.random.default_rng(8)
    k = rng.standard_normal((256, 1, d)).astype(np.float16)
    k[:, :, 3] *= 10
    kb = k.view(np.uint16)
    lay = orc.make_layout(d, 1, 32, 32, 1, 0)
    tb = orc.tile_bytes(lay)
    pool = np.zeros(tb, np.uint8)
    orc.quantize_blocks(lay, pool, [0], kb, kb)
    c = orc.rot_scale(d)
    Hm = brute.hadamard(d)
    par = pool[2 * 256 * (d // 2): 2 * 256 * (d // 2) + 256 * 4 * 4].view(np.float16).reshape(256, 4, 2)
    for t in range(0, 256, 17):
        kr, _, _ = orc.dequant_row(lay, pool, t)
        x_t = Hm @ kr / (d * c)
        s = np.repeat(par[t, :, 0].astype(np.float64), 32)
        z = np.repeat(par[t, :, 1].astype(np.float64), 32)
        bound = np.sqrt(np.sum((s / 2) ** 2)) * (1 + 1e-6) + 1e-4 * np.abs(k[t, 0]).max()
        # elements saturated by fp16 rounding of z would add their excess; the bound covers interior ones
        err = np.linalg.norm(x_t - k[t, 0].astype(np.float64))
        assert err <= bound + np.sum(np.abs(z) * 2.0 ** -11), t
