"""Helpers for the GPU parity tests: one scenario built twice from the same seeded inputs, once through
the HIP library (device) and once through the CPU oracle (host). Nothing here feeds a GPU result into
the oracle."""
from __future__ import annotations

import numpy as np

import kvq_workloads as W

TOL = 2e-3  # max relative error of decode attention, normwise per (sequence, head) row


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||got - ref||_inf / max(||ref||_inf, 1e-6)."""
    g = got.reshape(-1, got.shape[-1]).astype(np.float64)
    r = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    num = np.abs(g - r).max(axis=1)
    den = np.maximum(np.abs(r).max(axis=1), 1e-6)
    return float((num / den).max()) if num.size else 0.0


def host_inputs(case: W.Case, layer: int = 0):
    cfg = case.cfg
    k, v = W.blocks_kv(cfg, layer, case.prefill_blocks)
    bitmaps, prec = (None, None)
    if cfg.mixed:
        bitmaps, prec = W.mixed_precision_inputs(case, layer)
    ak = av = None
    if case.append:
        ak, av = W.append_kv(cfg, layer, case.n_seqs)
    q = W.queries(cfg, layer, case.n_seqs)
    return dict(k=k, v=v, bitmaps=bitmaps, prec=prec, ak=ak, av=av, q=q)


def oracle_run(orc, case: W.Case, inp, decode=True, n_threads=0):
    cfg = case.cfg
    lay = orc.make_layout(**cfg.layout())
    pool = np.zeros(orc.tile_bytes(lay) * cfg.num_kv_heads * case.num_blocks, np.uint8)
    if case.prefill_blocks.size:
        orc.quantize_blocks(lay, pool, case.prefill_blocks, inp["k"], inp["v"], inp["bitmaps"])
    if case.append:
        st = orc.append_tokens(lay, pool, inp["ak"], inp["av"], case.block_table, case.positions, inp["prec"])
        assert st == 0
    out = None
    if decode:
        out = orc.decode_attention(lay, pool, inp["q"], case.block_table, case.seq_lens, case.sentinel_mask,
                                   n_threads=n_threads)
    return pool, out


def to_dev(a, torch, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def gpu_run(kvq, torch, case: W.Case, inp, decode=True):
    cfg = case.cfg
    lay = kvq.Layout(**cfg.layout())
    pool = kvq.new_pool(lay, case.num_blocks)
    if case.prefill_blocks.size:
        kvq.quantize_blocks(lay, pool, to_dev(case.prefill_blocks, torch), to_dev(inp["k"], torch, torch.float16),
                            to_dev(inp["v"], torch, torch.float16),
                            None if inp["bitmaps"] is None else to_dev(inp["bitmaps"].view(np.int32), torch))
    table = to_dev(case.block_table, torch)
    if case.append:
        kvq.append_tokens(lay, pool, to_dev(inp["ak"], torch, torch.float16), to_dev(inp["av"], torch, torch.float16),
                          table, to_dev(case.positions, torch),
                          None if inp["prec"] is None else to_dev(inp["prec"], torch))
    out = None
    if decode:
        mask = None if case.sentinel_mask is None else to_dev(case.sentinel_mask.view(np.int32), torch)
        out = kvq.decode_attention(lay, pool, to_dev(inp["q"], torch, torch.float16), table,
                                   to_dev(case.seq_lens, torch), max(case.max_seq_len, 1), mask)
        out = out.cpu().numpy()
    torch.cuda.synchronize()
    return pool.cpu().numpy(), out
