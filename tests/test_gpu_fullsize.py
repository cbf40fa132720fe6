"""GPU parity at the workloads' full sizes, in the launch configuration of the full batch, over every sequence.

Each layer is built twice from the same seeded chunks of source rows (the generator module is the only
code the two sides share): on the GPU the way the benchmark builds it - every prefill block quantised in
chunks, one token appended per sequence where the workload appends, then one decode call over all
sequences, so the split plan, grid and workspace are those of the full-size call - and by the oracle
(quantisation parallel over tiles, decode parallel over (sequence, KV head)). Compared:

* the whole pool, bit for bit: codes, fp16 scales/zeros, width headers, padding and the appended rows of
  every block;
* every output row - all sequences, all query heads - within 2e-3 max relative error.

Nothing computed on the GPU feeds the oracle."""
import os

import numpy as np
import pytest

import kvq_workloads as W
from gpu_cases import TOL, rel_err

pytestmark = pytest.mark.gpu

# workload -> layers checked
FULL = {
    "tiny_1k": [0],
    "gemma3_12b_4k": [0, 47],
    "llama31_8b_pool_8k": [0, 31],
    "qwen25_14b_prefix_32k": [0],
    "mixed_sentinel_32k": [0],
    "deepseek_v2_lite_mla_8k": [0, 26],
}
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module")
def env():
    import torch

    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import bit_quantized_kv_quantize_amd as kvq

    return kvq, torch


def build_both(kvq, torch, orc, case, layer):
    """The full-size layer on the GPU and in the oracle from the same chunks: (GPU pool as host bytes, oracle
    pool, GPU decode output, oracle decode output)."""
    cfg = case.cfg
    lay = kvq.Layout(**cfg.layout())
    lay_o = orc.make_layout(**cfg.layout())
    pool = kvq.new_pool(lay, case.num_blocks)
    ref_pool = np.zeros(orc.tile_bytes(lay_o) * cfg.num_kv_heads * case.num_blocks, np.uint8)
    prec = np.full(case.n_seqs, 4, np.uint8) if cfg.mixed else None
    orc.set_threads(THREADS)
    for ids, k, v, bm in W.prefill_chunks(case, layer, max_blocks=2048, threads=THREADS, prec_out=prec):
        kvq.quantize_blocks(lay, pool, torch.from_numpy(ids).cuda(), torch.from_numpy(k).view(torch.float16).cuda(),
                            torch.from_numpy(v).view(torch.float16).cuda(),
                            None if bm is None else torch.from_numpy(bm.view(np.int32)).cuda())
        orc.quantize_blocks(lay_o, ref_pool, ids, k, v, bm)
        torch.cuda.synchronize()
    table = torch.from_numpy(case.block_table).cuda()
    if case.append:
        ak, av = W.append_kv(cfg, layer, case.n_seqs)
        kvq.append_tokens(lay, pool, torch.from_numpy(ak).view(torch.float16).cuda(),
                          torch.from_numpy(av).view(torch.float16).cuda(), table,
                          torch.from_numpy(case.positions).cuda(),
                          None if prec is None else torch.from_numpy(prec).cuda())
        assert orc.append_tokens(lay_o, ref_pool, ak, av, case.block_table, case.positions, prec) == 0
    qh = W.queries(cfg, layer, case.n_seqs)
    q = torch.from_numpy(qh).view(torch.float16).cuda()
    mask = None if case.sentinel_mask is None else torch.from_numpy(case.sentinel_mask.view(np.int32)).cuda()
    out = kvq.decode_attention(lay, pool, q, table, torch.from_numpy(case.seq_lens).cuda(), case.max_seq_len, mask)
    torch.cuda.synchronize()
    got_pool = pool.cpu().numpy()
    out = out.cpu().numpy()
    del pool
    torch.cuda.empty_cache()
    ref_out = orc.decode_attention(lay_o, ref_pool, qh, case.block_table, case.seq_lens, case.sentinel_mask,
                                   n_threads=THREADS)
    return got_pool, ref_pool, out, ref_out


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", W.CONFIG_ORDER + ["llama31_8b_pool_8k_fp8", "llama31_8b_pool_8k_widths",
                                                   "mixed_sentinel_32k_widths", "deepseek_v2_lite_mla_8k",
                                                   "deepseek_v2_lite_mla_8k_sentinel",
                                                   "deepseek_v2_lite_mla_8k_widths"])
def test_full_size_every_sequence(env, orc, name):
    # (the last cases: the 12 x 8K pool stored as FP8 E4M3, the baseline the 4-bit pool is measured against,
    # two workloads stored with per-token widths {2, 4, 8, FP16}, and an MLA model's pool: K head dim 192,
    # V head dim 128, also with half of its cached slots remapped to the sentinel and with per-token widths)
    kvq, torch = env
    base = name
    while base not in FULL:  # strip the variant suffixes (_fp8, _widths, _sentinel)
        base = base.rsplit("_", 1)[0]
    case = W.make_case(W.named_config(name))
    for layer in FULL[base]:
        print("[fullsize] %s layer %d: %d seqs, %d blocks" % (name, layer, case.n_seqs, case.num_blocks), flush=True)
        got_pool, ref_pool, out, ref_out = build_both(kvq, torch, orc, case, layer)
        if not np.array_equal(got_pool, ref_pool):
            tb = got_pool.size // case.num_blocks
            diff = np.nonzero(got_pool != ref_pool)[0]
            raise AssertionError("pool bytes differ: %d bytes, first in blocks %s (offsets %s)"
                                 % (diff.size, np.unique(diff // tb)[:4], diff[:4] % tb))
        err = rel_err(out, ref_out)
        print("[fullsize] %s layer %d: pool bit-exact (%.2f GB), max rel err %.3g over all %d sequences"
              % (name, layer, got_pool.size / 1e9, err, case.n_seqs), flush=True)
        assert np.isfinite(out).all()
        assert err <= TOL
        del got_pool, ref_pool
