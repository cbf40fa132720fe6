"""Card files (QKVShare methodology: the CacheCard of quantised groups, per-token widths and metadata;
"Agent Memory Below the Prompt" 2.1: blocks kept on disk as safetensors, as stored): the host-side packing
round trip, with tiles made by the oracle. The device copies are covered by the GPU tests."""
import numpy as np
import pytest
from safetensors import safe_open
from safetensors.numpy import load_file, save_file

import kvq_workloads as W
from bit_quantized_kv_quantize_amd import cachecard
from gpu_cases import host_inputs, oracle_run


def _oracle_case(orc, name, **kw):
    case = W.make_case(W.named_config(name), **kw)
    inp = host_inputs(case)
    pool, out = oracle_run(orc, case, inp)
    return case, inp, pool, out


@pytest.mark.parametrize("name,kw", [
    ("qwen25_14b_prefix_32k", dict(n_seqs=3, shared_prefix=512, context=[768, 612, 1023])),
    ("mixed_sentinel_32k", dict(n_seqs=3, context=[1024, 600, 333])),
    ("mixed_sentinel_32k_widths", dict(n_seqs=3, context=[1024, 600, 333])),
    ("deepseek_v2_lite_mla_8k", dict(n_seqs=2, context=[700, 257])),
])
def test_card_round_trip_reproduces_decode(orc, tmp_path, name, kw):
    case, inp, pool, ref = _oracle_case(orc, name, **kw)
    cfg = case.cfg
    fields = dict(cfg.layout())
    lay = orc.make_layout(**cfg.layout())
    tb = orc.tile_bytes(lay)
    H = cfg.num_kv_heads
    used = cachecard.used_blocks(case.block_table, case.seq_lens)
    tiles = pool.reshape(case.num_blocks, H, tb)[used]
    offs = np.arange(case.n_seqs, dtype=np.int32) * 1000
    tensors, meta = cachecard.pack(fields, tiles, case.block_table, case.seq_lens, "model-x", offs)
    path = str(tmp_path / "card.safetensors")
    save_file(tensors, path, metadata=meta)
    with safe_open(path, framework="numpy") as f:
        meta2 = f.metadata()
    card = cachecard.unpack(load_file(path), meta2, fields)
    assert card["model_id"] == "model-x" and card["layout"] == dict({k: int(v) for k, v in fields.items()}, format=0)
    assert np.array_equal(card["seq_lens"], case.seq_lens) and np.array_equal(card["position_offsets"], offs)
    if cfg.table == "shared_prefix":  # the shared prefix is stored once
        n_pref = kw["shared_prefix"] // 256
        assert card["tiles"].shape[0] == n_pref + sum((int(L) + 255) // 256 - n_pref for L in case.seq_lens)
    # the blocks placed at new ids in a fresh pool give the same attention output, bit for bit
    n = card["tiles"].shape[0]
    new_ids = (np.random.default_rng(1).permutation(n) + 5).astype(np.int32)
    pool2 = np.zeros((n + 5) * H * tb, np.uint8).reshape(n + 5, H, tb)
    pool2[new_ids] = card["tiles"]
    bt = card["block_table"]
    table2 = np.where(bt >= 0, new_ids[np.maximum(bt, 0)], 0).astype(np.int32)
    out2 = orc.decode_attention(lay, pool2.reshape(-1), inp["q"], table2, case.seq_lens, case.sentinel_mask)
    assert np.array_equal(out2, ref)


def test_card_rejects_other_layouts_and_bad_tables(orc):
    fields = dict(head_dim=128, num_kv_heads=2, block_tokens=256, k_group=64, v_group=64, rotate=0, mixed=0)
    tiles = np.zeros((2, 2, 36864), np.uint8)
    tensors, meta = cachecard.pack(fields, tiles, np.array([[7, 9]], np.int32), np.array([300], np.int32))
    assert list(tensors["block_table"][0]) == [0, 1]
    other = dict(fields, rotate=1)
    with pytest.raises(ValueError):
        cachecard.unpack(tensors, meta, other)
    bad = dict(tensors, block_table=np.array([[0, 2]], np.int32))
    with pytest.raises(ValueError):
        cachecard.unpack(bad, meta, fields)
    with pytest.raises(ValueError):
        cachecard.unpack(tensors, dict(meta, card_format="other"), fields)
