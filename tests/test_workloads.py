"""Host-side checks of the seeded workload generators (shapes, determinism, table structure)."""
import numpy as np

import kvq_workloads as W


def test_deterministic_and_shaped():
    cfg = W.CONFIGS["llama31_8b_pool_8k"]
    k1, v1 = W.block_kv(cfg, 3, 17)
    k2, v2 = W.block_kv(cfg, 3, 17)
    assert k1.shape == (256, 8, 128) and k1.dtype == np.uint16
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    assert not np.array_equal(k1, W.block_kv(cfg, 4, 17)[0])
    kb, _ = W.blocks_kv(cfg, 3, [5, 17], threads=2)
    assert np.array_equal(kb[256:], k1)


def test_outliers_scale_k_channels():
    cfg = W.CONFIGS["gemma3_12b_4k"]
    out = W.outlier_channels(cfg, 0)
    assert out.shape == (8, 5) and all(len(set(r)) == 5 for r in out)
    k, v = W.blocks_kv(cfg, 0, range(4))
    kf = k.view(np.float16).astype(np.float64)
    std = kf.std(axis=0)
    for h in range(8):
        assert np.all(std[h, out[h]] > 6) and np.median(std[h]) < 1.2
    assert 0.45 < v.view(np.float16).astype(np.float64).std() < 0.55


def test_pool_tables():
    case = W.make_case(W.CONFIGS["llama31_8b_pool_8k"])
    assert case.block_table.shape == (12, 33) and case.num_blocks == 396
    assert np.array_equal(np.sort(case.block_table.ravel()), np.arange(396))
    assert case.prefill_blocks.size == 384 and int(case.seq_lens[0]) == 8193
    c4 = W.make_case(W.CONFIGS["qwen25_14b_prefix_32k"])
    assert c4.num_blocks == 256 and c4.block_table.shape == (64, 130)
    assert np.all(c4.block_table[:, :128] == c4.block_table[0, :128])
    assert np.unique(c4.block_table[:, 128:]).size == 128
    assert int(c4.seq_lens[0]) == 33280 and not c4.append


def test_sentinel_mask_exact_count_and_precision_map():
    cfg = W.CONFIGS["mixed_sentinel_32k"]
    case = W.make_case(cfg, n_seqs=3, context=[4096, 1000, 300])
    assert case.mask_words == (4097 + 31) // 32
    for s, n in enumerate([4096, 1000, 300]):
        bits = np.unpackbits(case.sentinel_mask[s].view(np.uint8), bitorder="little")
        assert bits.sum() == int(0.75 * n) and not bits[n:].any()
    norms = np.arange(100, dtype=np.float64)[::-1].copy()
    norms[50] = norms[19]                                 # tie exactly at the cut
    sel = W.precision_map(norms, 0.2)
    assert sel.sum() == 20 and sel[:20].all() and not sel[50]  # ties go to the lower index
    assert W.appended_is_8bit(norms, norms[19], 0.2) and not W.appended_is_8bit(norms, norms[19] - 0.5, 0.2)
    words = W.bits_words(np.arange(512) % 3 == 0)
    assert words.shape == (2, 8) and (words[0, 0] & 1) == 1 and ((words[0, 0] >> 1) & 1) == 0


def test_prefill_chunks_cover_every_block_once():
    for name, kw, widths in [("llama31_8b_pool_8k", dict(n_seqs=3, context=[1000, 513, 0]), False),
                             ("mixed_sentinel_32k", dict(n_seqs=4, context=[1024, 600, 0, 333]), False),
                             ("llama31_8b_pool_8k", dict(n_seqs=4, context=[1000, 513, 0, 300]), True)]:
        cfg = W.widths_variant(W.CONFIGS[name]) if widths else W.CONFIGS[name]
        case = W.make_case(cfg, **kw)
        prec = np.zeros(case.n_seqs, np.uint8)
        ids, ks, bms = [], [], []
        for chunk, k, v, bm in W.prefill_chunks(case, 0, max_blocks=3, threads=2, prec_out=prec):
            assert k.shape == v.shape == (chunk.size * W.BLOCK, 8, 128)
            ids.append(chunk)
            ks.append(k)
            bms.append(bm)
        ids = np.concatenate(ids)
        assert np.array_equal(np.sort(ids), case.prefill_blocks)
        order = np.argsort(ids)
        k_ref, _ = W.blocks_kv(case.cfg, 0, case.prefill_blocks)
        assert np.array_equal(np.concatenate(ks).reshape(ids.size, W.BLOCK, 8, 128)[order].reshape(k_ref.shape), k_ref)
        if case.cfg.mixed:
            bm_ref, prec_ref = W.mixed_precision_inputs(case, 0)
            assert np.array_equal(np.concatenate(bms)[order], bm_ref)
            assert np.array_equal(prec, prec_ref)
        else:
            assert all(b is None for b in bms)


def test_width_codes_and_words():
    norms = np.arange(100, dtype=np.float64)[::-1].copy()   # token i has the (100 - i)-th norm
    codes = W.width_codes(norms, (0.05, 0.15, 0.3))
    assert (codes[:5] == 3).all() and (codes[5:20] == 2).all() and (codes[20:70] == 1).all()
    assert (codes[70:] == 0).all()
    assert W.appended_width(norms, norms[4], (0.05, 0.15, 0.3)) == 16
    assert W.appended_width(norms, norms[10], (0.05, 0.15, 0.3)) == 8
    assert W.appended_width(norms, norms[40], (0.05, 0.15, 0.3)) == 4
    assert W.appended_width(norms, norms[80], (0.05, 0.15, 0.3)) == 2
    assert W.appended_width(norms[:0], 1.0, (0.05, 0.15, 0.3)) == 4
    rows = np.arange(512) % 4
    words = W.width_words(rows.astype(np.uint8))
    assert words.shape == (2, 16)
    for t in (0, 1, 2, 3, 17, 255, 300, 511):
        assert (words[t // 256, (t % 256) // 16] >> (2 * (t % 16))) & 3 == rows[t]
