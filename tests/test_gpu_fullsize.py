"""GPU parity at the five workloads' full sizes, in the launch configuration of the full batch.

Each layer is built on the GPU the way the benchmark builds it: every prefill block quantised (in chunks
of the seeded source), one token appended per sequence where the workload appends, then one decode call
over all sequences - so the split plan, grid and workspace are those of the full-size call. The oracle
then rebuilds, from the same seeded inputs, what it can compute in seconds:

* every tile of the sampled sequences' blocks (codes, fp16 scales/zeros, bitmaps, padding and the
  appended rows), compared bit for bit with the GPU pool;
* the decode output of the sampled sequences (all their query heads), within 2e-3 max relative error.

The oracle's pool for the sample holds only the sampled sequences' blocks (renumbered); nothing computed
on the GPU feeds it."""
import numpy as np
import pytest

import kvq_workloads as W
from gpu_cases import TOL, rel_err

pytestmark = pytest.mark.gpu

# workload -> (layers checked, sampled sequences)
FULL = {
    "tiny_1k": ([0], [0]),
    "gemma3_12b_4k": ([0, 47], [0]),
    "llama31_8b_pool_8k": ([0, 31], [0, 5, 11]),
    "qwen25_14b_prefix_32k": ([0], [0, 37, 63]),
    "mixed_sentinel_32k": ([0], [0, 77, 127]),
    "deepseek_v2_lite_mla_8k": ([0, 26], [0, 5, 11]),
}


@pytest.fixture(scope="module")
def env():
    import torch

    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import bit_quantized_kv_quantize_amd as kvq

    return kvq, torch


def build_on_gpu(kvq, torch, case, layer):
    """Full-size layer on the GPU: pool, appended tokens, decode output (host copy)."""
    cfg = case.cfg
    lay = kvq.Layout(**cfg.layout())
    pool = kvq.new_pool(lay, case.num_blocks)
    prec = np.full(case.n_seqs, 4, np.uint8) if cfg.mixed else None
    for ids, k, v, bm in W.prefill_chunks(case, layer, max_blocks=2048, threads=16, prec_out=prec):
        kvq.quantize_blocks(lay, pool, torch.from_numpy(ids).cuda(), torch.from_numpy(k).view(torch.float16).cuda(),
                            torch.from_numpy(v).view(torch.float16).cuda(),
                            None if bm is None else torch.from_numpy(bm.view(np.int32)).cuda())
        torch.cuda.synchronize()
    table = torch.from_numpy(case.block_table).cuda()
    if case.append:
        ak, av = W.append_kv(cfg, layer, case.n_seqs)
        kvq.append_tokens(lay, pool, torch.from_numpy(ak).view(torch.float16).cuda(),
                          torch.from_numpy(av).view(torch.float16).cuda(), table,
                          torch.from_numpy(case.positions).cuda(),
                          None if prec is None else torch.from_numpy(prec).cuda())
    q = torch.from_numpy(W.queries(cfg, layer, case.n_seqs)).view(torch.float16).cuda()
    mask = None if case.sentinel_mask is None else torch.from_numpy(case.sentinel_mask.view(np.int32)).cuda()
    out = kvq.decode_attention(lay, pool, q, table, torch.from_numpy(case.seq_lens).cuda(), case.max_seq_len, mask)
    torch.cuda.synchronize()
    return lay, pool, out.cpu().numpy()


def oracle_sample(orc, case, layer, seqs):
    """The oracle on the sampled sequences only: (original block ids, their tiles, decode output)."""
    cfg = case.cfg
    n_used = (case.seq_lens[seqs] + W.BLOCK - 1) // W.BLOCK
    ids = np.unique(np.concatenate([case.block_table[s, :n] for s, n in zip(seqs, n_used)])).astype(np.int32)
    compact = {int(b): i for i, b in enumerate(ids)}
    table = np.zeros((len(seqs), case.max_blocks_per_seq), np.int32)
    for r, (s, n) in enumerate(zip(seqs, n_used)):
        table[r, :n] = [compact[int(b)] for b in case.block_table[s, :n]]
    prefill = np.array([b for b in ids if b in set(case.prefill_blocks.tolist())], np.int32)
    lay = orc.make_layout(**cfg.layout())
    tb = orc.tile_bytes(lay)
    pool = np.zeros(tb * cfg.num_kv_heads * ids.size, np.uint8)
    bitmaps = None
    prec = None
    ak = av = None
    if case.append:
        ak, av = W.append_kv(cfg, layer, case.n_seqs)
        ak, av = ak[seqs], av[seqs]
    if cfg.mixed:
        # per-sequence ranking of cached tokens by K norm, as for the whole batch
        bm = {}
        prec = np.full(len(seqs), 4, np.uint8)
        for r, s in enumerate(seqs):
            blocks = W.sequence_blocks(case, s)
            k, _ = W.blocks_kv(cfg, layer, blocks, threads=16)
            n = int(case.context[s])
            ns = W.k_norms_sq(k[:n])
            for i, words in enumerate(W.block_width_words(cfg, ns, blocks.size)):
                bm[int(blocks[i])] = words
            if case.append and blocks.size:
                prec[r] = W.append_prec(cfg, ns, float(W.k_norms_sq(ak[r:r + 1])[0]))
        bitmaps = np.stack([bm[int(b)] for b in prefill])
    k, v = W.blocks_kv(cfg, layer, prefill, threads=16)
    orc.quantize_blocks(lay, pool, np.array([compact[int(b)] for b in prefill], np.int32), k, v, bitmaps)
    pos = case.positions[seqs]
    if case.append:
        assert orc.append_tokens(lay, pool, ak, av, table, pos, prec) == 0
    q = W.queries(cfg, layer, case.n_seqs)[seqs]
    mask = None if case.sentinel_mask is None else np.ascontiguousarray(case.sentinel_mask[seqs])
    out = orc.decode_attention(lay, pool, q, table, case.seq_lens[seqs], mask, n_threads=16)
    return ids, pool.reshape(ids.size, -1), out


@pytest.mark.parametrize("name", W.CONFIG_ORDER + ["llama31_8b_pool_8k_fp8", "llama31_8b_pool_8k_widths",
                                                   "mixed_sentinel_32k_widths", "deepseek_v2_lite_mla_8k"])
def test_full_size_sampled(env, orc, name):
    # (the last cases: the 12 x 8K pool stored as FP8 E4M3, the baseline the 4-bit pool is measured against,
    # two workloads stored with per-token widths {2, 4, 8, FP16}, and an MLA model's pool: K head dim 192,
    # V head dim 128)
    kvq, torch = env
    base = name.replace("_fp8", "").replace("_widths", "")
    layers, seqs = FULL[base]
    case = W.make_case(W.named_config(name))
    for layer in layers:
        print("[fullsize] %s layer %d: %d seqs, %d blocks" % (name, layer, case.n_seqs, case.num_blocks), flush=True)
        _, pool, out = build_on_gpu(kvq, torch, case, layer)
        ids, ref_tiles, ref_out = oracle_sample(orc, case, layer, seqs)
        got_tiles = pool.view(case.num_blocks, -1)[torch.from_numpy(ids).long().cuda()].cpu().numpy()
        diff = np.nonzero(got_tiles != ref_tiles)
        assert diff[0].size == 0, "tiles differ: block %s byte %s" % (ids[diff[0][:4]], diff[1][:4])
        err = rel_err(out[seqs], ref_out)
        print("[fullsize] %s layer %d: max rel err %.3g over sequences %s" % (name, layer, err, seqs), flush=True)
        assert err <= TOL
        assert np.isfinite(out).all()
        del pool
        torch.cuda.empty_cache()
