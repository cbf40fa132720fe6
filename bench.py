#!/usr/bin/env python3
"""Benchmark: Q4 decode-attention effective HBM GB/s (% of peak) + KV tokens/s quantized, on one MI355X.

Workload (default ``llama31_8b_pool_8k``): 12 agents x 8192 cached tokens, 32 query / 8 KV heads,
head_dim 128, 32 layers, one pool of 256-token Q4 blocks per layer (groups of 64 per token), block tables
a seeded random permutation of the pool. Every input is seeded synthetic data (kvq_workloads), resident
in HBM before any timed region.

  step   one decode step over all layers: per layer, kvq_append_tokens (quantise the new token of each
         agent into its slot 8192) then kvq_decode_attention over 8193 slots. The step is captured once
         as a HIP graph and replayed; ``value`` = algorithmic bytes of the step / step time.
  kernel the decode-attention kernel alone, launched per layer between HIP events on the launch stream;
         ``roofline.achieved`` = its algorithmic bytes per launch / mean launch duration.
  prefill kvq_quantize_blocks over every cached block of every layer -> KV token-layers quantised / s.
  cpu     the CPU oracle on a bounded sample (one layer of decode attention, a few blocks of quantise).

Prints one JSON line on rank 0. Only one GPU is supported.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import kvq_workloads as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama31_8b_pool_8k", choices=W.CONFIG_ORDER)
    ap.add_argument("--kernel-reps", type=int, default=50, help="graph replays of all layers' decode kernels")
    ap.add_argument("--no-graph", action="store_true", help="launch the step eagerly instead of a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (diagnostics only)")
    ap.add_argument("--no-workloads", action="store_true", help="skip the per-workload decode table")
    ap.add_argument("--workload-table", default="",
                    help="comma-separated workloads for the per-workload table (default: every workload)")
    ap.add_argument("--workload-launches", type=int, default=16, help="decode launches per workload graph")
    ap.add_argument("--workload-reps", type=int, default=20, help="timed replays of each workload graph")
    ap.add_argument("--cpu-budget", type=float, default=1.0,
                    help="scale of the CPU oracle samples (1.0: about half a minute of oracle time)")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def pct(xs):
    """median, p10 and p90 of a list of times."""
    a = np.asarray(xs, np.float64)
    return float(np.median(a)), float(np.percentile(a, 10)), float(np.percentile(a, 90))


def live_rows(case: W.Case, width_words=None, appended_prec=None):
    """Live rows of one decode call per sequence and width: int64 [n_seqs, 4], columns 2, 4, 8 and 16 bits.
    A row is live when it lies below seq_len and its sentinel bit is clear; its width comes from its block's
    width words (``width_words``: physical block -> uint32 words in the pool header's encoding) or, for the
    appended slot, from ``appended_prec``; rows of blocks without words are 4-bit."""
    mixed = case.cfg.mixed
    counts = np.zeros((case.n_seqs, 4), np.int64)
    for s in range(case.n_seqs):
        L = int(case.seq_lens[s])
        t = np.arange(L)
        live = np.ones(L, bool)
        if case.sentinel_mask is not None:
            live = ~((case.sentinel_mask[s][t // 32] >> (t % 32).astype(np.uint32)) & 1).astype(bool)
        code = np.ones(L, np.int64)  # width codes 0..3 = 2, 4, 8, 16 bits
        if width_words is not None:
            for bi in range((L + W.BLOCK - 1) // W.BLOCK):
                words = width_words.get(int(case.block_table[s, bi]))
                if words is None:
                    continue
                tt = np.arange(min(W.BLOCK, L - bi * W.BLOCK))
                if mixed == 2:
                    c = (words[tt // 16] >> (2 * (tt % 16)).astype(np.uint32)) & 3
                else:
                    c = np.where((words[tt // 32] >> (tt % 32).astype(np.uint32)) & 1, 2, 1)
                code[bi * W.BLOCK: bi * W.BLOCK + tt.size] = c
            if case.append and appended_prec is not None and L:
                code[L - 1] = {2: 0, 8: 2, 16: 3}.get(int(appended_prec[s]), 1)
        counts[s] = np.bincount(code[live], minlength=4)
    return counts


def decode_bytes(cfg: W.Config, case: W.Case, counts: np.ndarray, unique: bool = True) -> int:
    """Algorithmic bytes of one decode-attention call: every live row's K and V codes and parameters once
    (a block shared by several block tables counted once when ``unique``; an FP16 row has no parameters),
    the per-channel K parameters and width headers of the tiles touched, q, out, block tables, lengths and
    masks. ``counts``: live rows per sequence and width (2, 4, 8, 16 bits), as from live_rows."""
    d, dv, H = cfg.head_dim, cfg.dv, cfg.num_kv_heads
    kpar = (d // cfg.k_group) * 4 if cfg.k_group > 0 else 0
    vpar = (dv // cfg.v_group) * 4 if cfg.v_group > 0 else 0
    row = np.array([(d + dv) * bits // 8 + kpar + vpar for bits in (2, 4, 8)] + [2 * (d + dv)], np.int64)
    if cfg.fmt == 1:  # FP8 E4M3: one byte per K and V element, no parameters
        row[:] = d + dv
    if unique and cfg.table == "shared_prefix":
        # every physical block read once: its live rows are the rows below the longest sequence using it
        rows = 0
        for b in np.unique(case.block_table[case.block_table >= 0]):
            hits = np.argwhere(case.block_table == b)
            rows += max(min(W.BLOCK, int(case.seq_lens[s]) - int(j) * W.BLOCK) for s, j in hits)
        b = rows * H * int(row[1])
        tiles = np.unique(case.block_table).size
    else:
        b = int((counts * row).sum()) * H
        tiles = int(np.ceil(case.seq_lens / W.BLOCK).sum())
    if cfg.k_group < 0 and cfg.fmt == 0:
        b += tiles * H * d * 4
    if cfg.mixed:
        b += tiles * H * (64 if cfg.mixed == 2 else 32)
    b += case.n_seqs * cfg.num_q_heads * (d * 2 + dv * 4)             # q fp16 in, out fp32
    b += case.block_table.size * 4 + case.n_seqs * 4
    if case.sentinel_mask is not None:
        b += case.sentinel_mask.size * 4
    return b


def append_bytes(cfg: W.Config, n_seqs: int) -> int:
    d, dv, H = cfg.head_dim, cfg.dv, cfg.num_kv_heads
    kpar = (d // cfg.k_group) * 4
    row_out = (d + dv) // 2 + kpar + (dv // cfg.v_group) * 4
    return n_seqs * H * ((d + dv) * 2 + row_out) + n_seqs * 4 * 2


def quantize_bytes(cfg: W.Config, n_blocks: int, tile_bytes: int) -> int:
    return n_blocks * W.BLOCK * cfg.num_kv_heads * (cfg.head_dim + cfg.dv) * 2 + n_blocks * cfg.num_kv_heads * tile_bytes


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_quantized_kv_quantize_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if not os.path.isfile(os.path.join(csrc, f)):
            continue  # (the probe library's sources are not libkvq's)
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, digest: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary of this workload, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "decode_attn_%s_counters.md" % workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel sources:\s*([0-9a-f]{16})", text)
    m_b = re.search(r"HBM bytes per launch \(scaled\):\s*([0-9.eE+]+)", text)
    if not (m_src and m_b) or m_src.group(1) != digest:
        return None
    return float(m_b.group(1))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_quantized_kv_quantize_amd as kvq

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.CONFIGS[args.workload]
    if cfg.mixed or cfg.k_group < 0 or not cfg.append:
        raise SystemExit("bench.py times the per-token Q4 append + decode step; workload %s is a parity case"
                         % args.workload)
    layers = args.layers or cfg.layers
    case = W.make_case(cfg)
    lay = kvq.Layout(**cfg.layout())
    tb = kvq.tile_bytes(lay)
    n_prefill = case.prefill_blocks.size
    log("workload %s: %d seqs x %d ctx, %d layers, %d pool blocks, tile %d B" %
        (cfg.name, case.n_seqs, cfg.context, layers, case.num_blocks, tb))

    # ---------------------------------------------------------------- inputs, resident in HBM
    t0 = time.time()
    pools, kin, vin, qs, aks, avs, outs = [], [], [], [], [], [], []
    for l in range(layers):
        k, v = W.blocks_kv(cfg, l, case.prefill_blocks, threads=16)
        kin.append(torch.from_numpy(k).view(torch.float16).to(dev))
        vin.append(torch.from_numpy(v).view(torch.float16).to(dev))
        ak, av = W.append_kv(cfg, l, case.n_seqs)
        aks.append(torch.from_numpy(ak).view(torch.float16).to(dev))
        avs.append(torch.from_numpy(av).view(torch.float16).to(dev))
        qs.append(torch.from_numpy(W.queries(cfg, l, case.n_seqs)).view(torch.float16).to(dev))
        pools.append(kvq.new_pool(lay, case.num_blocks))
        outs.append(torch.empty((case.n_seqs, cfg.num_q_heads, cfg.dv), dtype=torch.float32, device=dev))
        if l % 8 == 7:
            log("generated layer %d/%d (%.1f s)" % (l + 1, layers, time.time() - t0))
    block_ids = torch.from_numpy(case.prefill_blocks).to(dev)
    table = torch.from_numpy(case.block_table).to(dev)
    positions = torch.from_numpy(case.positions).to(dev)
    seq_lens = torch.from_numpy(case.seq_lens).to(dev)
    max_len = case.max_seq_len
    ws = kvq.new_workspace(lay, case.n_seqs, cfg.num_q_heads, max_len)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    # ---------------------------------------------------------------- prefill quantise
    q_tok_s = None
    q_gbps = None
    for l in range(layers):  # untimed pass fills every pool
        kvq.quantize_blocks(lay, pools[l], block_ids, kin[l], vin[l])
    torch.cuda.synchronize()
    if not args.no_prefill:
        reps = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            for l in range(layers):
                kvq.quantize_blocks(lay, pools[l], block_ids, kin[l], vin[l])
        e1.record(stream)
        torch.cuda.synchronize()
        qs_t = e0.elapsed_time(e1) / 1e3 / reps
        q_tok_s = n_prefill * W.BLOCK * layers / qs_t
        q_gbps = quantize_bytes(cfg, n_prefill, tb) * layers / qs_t / 1e9
        log("prefill quantise: %.3f ms for %d token-layers -> %.3g token-layers/s, %.0f GB/s" %
            (qs_t * 1e3, n_prefill * W.BLOCK * layers, q_tok_s, q_gbps))
    del kin, vin

    # ---------------------------------------------------------------- the decode step
    def step():
        for l in range(layers):
            kvq.append_tokens(lay, pools[l], aks[l], avs[l], table, positions)
            kvq.decode_attention(lay, pools[l], qs[l], table, seq_lens, max_len, out=outs[l], workspace=ws)

    step()
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()  # warm the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
    else:
        run = step
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_start = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        run()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t_start) / args.steps
    step_med, step_p10, step_p90 = pct([evs[i].elapsed_time(evs[i + 1]) / 1e3 for i in range(args.steps)])
    dec_b = decode_bytes(cfg, case, live_rows(case))
    app_b = append_bytes(cfg, case.n_seqs)
    step_bytes = (dec_b + app_b) * layers
    value = step_bytes / step_s / 1e9
    log("step: %.3f ms, %.1f GB/s algorithmic (%.1f%% of 8 TB/s)" % (step_s * 1e3, value, value / 80))

    # ---------------------------------------------------------------- the decode kernel alone
    # The decode kernels of all layers, captured back to back in one HIP graph and replayed between two
    # events on the launch stream: the mean per launch is the kernel's duration plus the (small) gap
    # between graph nodes, comparable with a profiler's per-kernel average.
    kg = torch.cuda.CUDAGraph()
    s2 = torch.cuda.Stream()
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s2):
        for l in range(layers):
            kvq.decode_attention(lay, pools[l], qs[l], table, seq_lens, max_len, out=outs[l], workspace=ws)
    torch.cuda.current_stream().wait_stream(s2)
    torch.cuda.synchronize()
    with torch.cuda.graph(kg):
        for l in range(layers):
            kvq.decode_attention(lay, pools[l], qs[l], table, seq_lens, max_len, out=outs[l], workspace=ws)
    kg.replay()
    torch.cuda.synchronize()
    per_rep = []
    for _ in range(args.kernel_reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kg.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        per_rep.append(e0.elapsed_time(e1) / 1e3 / layers)
    kern_s, kern_p10, kern_p90 = pct(per_rep)
    achieved = dec_b / kern_s / 1e9
    log("decode kernel: %.2f us per launch (median of %d graph replays of %d launches; p10 %.2f, p90 %.2f) -> "
        "%.1f GB/s" % (kern_s * 1e6, len(per_rep), layers, kern_p10 * 1e6, kern_p90 * 1e6, achieved))

    # the streaming-read ceiling: the same tiles read with the decode's load pattern and no arithmetic, and a
    # flat 2 GiB read
    ceiling = read_ceiling(torch, cfg, case, pools, table, seq_lens, layers)

    # the prefill quantiser's read-plus-write ceiling: one layer's fp16 K/V in, its tiles out
    q_ceiling = stream_rw_ceiling(torch, n_prefill * W.BLOCK * cfg.num_kv_heads * (cfg.head_dim + cfg.dv) * 2,
                                  n_prefill * cfg.num_kv_heads * tb)

    # plain device copy of 2 GiB for context (read + write bandwidth the box delivers)
    a = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * a.numel() * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del a, b
    log("device copy: %.0f GB/s (read + write)" % copy_gbps)

    digest = kernel_source_digest()
    traffic = recorded_traffic(cfg.name, digest)

    # ---------------------------------------------------------------- every workload's decode kernel
    workloads = None
    if not args.no_workloads:
        del pools, aks, avs, qs, outs
        torch.cuda.empty_cache()
        workloads = {}
        names = W.CONFIG_ORDER + [FP8_BASELINE, WIDTHS_POOL, MLA_POOL] + MLA_VARIANTS
        if args.workload_table:
            names = [n for n in args.workload_table.split(",") if n]
            for n in names:
                workload_config(n)  # unknown names fail here, before any timing
        for name in names:
            if name != cfg.name:
                workloads[name] = measure_workload(kvq, torch, name, launches=args.workload_launches,
                                                   graph=not args.no_graph, reps=args.workload_reps)
        workloads[cfg.name] = {"decode_us": round(kern_s * 1e6, 2),
                               "decode_us_p10_p90": [round(kern_p10 * 1e6, 2), round(kern_p90 * 1e6, 2)],
                               "bytes": dec_b, "GBps": round(achieved, 1),
                               "frac_of_hbm_peak": round(achieved / HBM_PEAK_GBPS, 4), "pool_instances": layers,
                               "append_us": None,
                               "quantize": None if q_tok_s is None else {
                                   "blocks": int(n_prefill) * layers, "us": round(qs_t * 1e6, 2),
                                   "token_layers_per_s": round(q_tok_s, 0), "GBps": round(q_gbps, 1)}}

    # ---------------------------------------------------------------- baselines of the pages' comparisons
    baselines = None
    if workloads is not None and FP8_BASELINE in workloads:
        f8 = workloads[FP8_BASELINE]
        baselines = {
            "fp8_e4m3_cache": {"workload": FP8_BASELINE, "decode_us": f8["decode_us"], "bytes": f8["bytes"],
                               "GBps": f8["GBps"], "q4_speedup": round(f8["decode_us"] / (kern_s * 1e6), 3),
                               "q4_byte_ratio": round(f8["bytes"] / dec_b, 3)},
            "restore_fp16": measure_restore(kvq, torch, cfg.name),
        }

    # ---------------------------------------------------------------- CPU oracle on a bounded sample
    cpu = None
    if not args.no_cpu_baseline:
        dec_bytes = {n: (workloads[n]["bytes"] if workloads and n in workloads else None) for n in CPU_SAMPLES}
        for n in dec_bytes:
            if dec_bytes[n] is None:
                c = W.make_case(W.CONFIGS[n])
                dec_bytes[n] = decode_bytes(c.cfg, c, live_rows(c)) if not c.cfg.mixed else None
        dec_bytes = {n: b for n, b in dec_bytes.items() if b}
        cpu = cpu_baseline(cfg.name, dec_bytes, args.cpu_budget) if cfg.name in dec_bytes else None

    line = {
        "metric": "Q4 decode-attention effective HBM GB/s (% of peak) + KV tokens/s quantized",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "ms_per_step_median_p10_p90": [round(step_med * 1e3, 4), round(step_p10 * 1e3, 4), round(step_p90 * 1e3, 4)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4+f32",
        "data": "synthetic (seeded, kvq_workloads)",
        "config": {"workload": cfg.name, "agents": case.n_seqs, "context": cfg.context, "layers": layers,
                   "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads, "head_dim": cfg.head_dim,
                   "group": cfg.k_group, "block_tokens": W.BLOCK, "graph": graph is not None,
                   "step": "per layer: append 1 token/agent + decode attention over 8193 slots"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "kv_tokens_quantized_per_s": None if q_tok_s is None else round(q_tok_s, 0),
        "quantize_GBps": None if q_gbps is None else round(q_gbps, 1),
        "quantize_roofline": None if q_gbps is None else {
            "bound": "hbm", "achieved": round(q_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(q_gbps / HBM_PEAK_GBPS, 4), "kernel": "quantize_rows16_k<8, false, 0, 2, 2>",
            "bytes_per_layer": quantize_bytes(cfg, n_prefill, tb), "us_per_layer": round(qs_t * 1e6 / layers, 2),
            "ceiling": q_ceiling,
            "frac_of_rw_ceiling": None if not q_ceiling else round(q_gbps / q_ceiling["GBps"], 4)},
        "device_copy_GBps": round(copy_gbps, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "decode_rows_k<4, false, false, 128>", "bytes_per_launch": dec_b,
                     "us_per_launch": round(kern_s * 1e6, 3),
                     "us_per_launch_p10_p90": [round(kern_p10 * 1e6, 3), round(kern_p90 * 1e6, 3)],
                     "launches_timed": len(per_rep) * layers,
                     "ceiling": ceiling,
                     "frac_of_flat_read": None if not ceiling else round(achieved / ceiling["flat_GBps"], 4),
                     "frac_of_tile_read": None if not ceiling else round(achieved / ceiling["tiles_GBps"], 4),
                     "kernel_sources": digest},
        "cpu_baseline": cpu,
        "workloads": workloads,
        "baselines": baselines,
    }
    print(json.dumps(line), flush=True)


# Pool instances cycled through when one workload's decode is timed on its own: enough distinct copies that
# the working set exceeds the 256 MB Infinity Cache (the multi-layer workloads use their layer count).
INSTANCES = {"tiny_1k": 1, "gemma3_12b_4k": 48, "llama31_8b_pool_8k": 32, "qwen25_14b_prefix_32k": 16,
             "mixed_sentinel_32k": 1, "deepseek_v2_lite_mla_8k": 8}
# The 12 x 8K pool stored as FP8 E4M3: the cache the 4-bit one is compared against (UltraQuant, technology section).
FP8_BASELINE = "llama31_8b_pool_8k_fp8"
# The 12 x 8K pool with per-token widths {2, 4, 8, FP16} (QKVShare, methodology section).
WIDTHS_POOL = "llama31_8b_pool_8k_widths"
# 12 agents x 8K of an MLA model: K head dim 192, V 128 ("Agent Memory Below the Prompt", 2.2).
MLA_POOL = "deepseek_v2_lite_mla_8k"
# The MLA pool with half of the cached slots remapped to the sentinel (IntentKV), and with per-token widths
# {2, 4, 8, FP16} (QKVShare, methodology section); both read through the row lists.
MLA_VARIANTS = ["deepseek_v2_lite_mla_8k_sentinel", "deepseek_v2_lite_mla_8k_widths"]


def base_name(name):
    """The workload a variant name derives from."""
    for suffix in ("_fp8", "_widths", "_sentinel"):
        if name.endswith(suffix):
            return base_name(name[:-len(suffix)])
    return name


def workload_config(name):
    return W.named_config(name)


def read_ceiling(torch, cfg, case, pools, table, seq_lens, layers, reps=20):
    """Streaming-read ceilings from libkvq_probe.so: the decode's own tiles of every layer read with its load
    pattern (512 workgroups, 16-byte loads, rows below each sequence's length, no arithmetic), timed like the
    decode kernel (a graph of one launch per layer between events), and a flat 2 GiB read."""
    import ctypes

    path = os.path.join(ROOT, "bit_quantized_kv_quantize_amd", "libkvq_probe.so")
    if not os.path.exists(path):
        log("no libkvq_probe.so: read ceiling not measured")
        return None
    lib = ctypes.CDLL(path)
    P, I, U = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32
    lib.kvq_probe_read_tiles.argtypes = [P, P, P, I, I, I, U, U, U, U, I, P, P]
    lib.kvq_probe_read_linear.argtypes = [P, ctypes.c_size_t, I, P, P]
    d, dv, H = cfg.head_dim, cfg.dv, cfg.num_kv_heads
    rec = (d + dv) // 2
    prow = 4 * (d // cfg.k_group + dv // cfg.v_group)
    import bit_quantized_kv_quantize_amd as kvq
    tb = kvq.tile_bytes(kvq.Layout(**cfg.layout()))
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def tiles(l):
        st = lib.kvq_probe_read_tiles(P(pools[l].data_ptr()), P(table.data_ptr()), P(seq_lens.data_ptr()),
                                      case.n_seqs, H, case.max_blocks_per_seq, tb, rec, 256 * rec, prow, 512,
                                      P(sink.data_ptr()), P(torch.cuda.current_stream().cuda_stream))
        assert st == 0

    def timed(fn, n):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(n):
                fn(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3 / n)
        return pct(ts)

    kv_bytes = int(case.seq_lens.sum()) * H * (rec + prow)
    t_tiles, _, _ = timed(tiles, layers)
    # flat reads of the decode's byte count, cycling through enough buffers to exceed the Infinity Cache
    nbytes = kv_bytes // 16 * 16
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(max(4, (1 << 31) // nbytes + 1))]

    def linear(i):
        st = lib.kvq_probe_read_linear(P(bufs[i % len(bufs)].data_ptr()), nbytes, 2048, P(sink.data_ptr()),
                                       P(torch.cuda.current_stream().cuda_stream))
        assert st == 0

    t_lin, _, _ = timed(linear, len(bufs))
    res = {"tiles_GBps": round(kv_bytes / t_tiles / 1e9, 1), "tiles_us": round(t_tiles * 1e6, 2),
           "flat_GBps": round(nbytes / t_lin / 1e9, 1), "flat_us": round(t_lin * 1e6, 2), "bytes": kv_bytes,
           "kind": "libkvq_probe, per launch in a graph: the decode's tiles read with its load pattern and work "
                   "split and no arithmetic (tiles), and a flat read of the same byte count from 2048 "
                   "workgroups (flat)"}
    del bufs
    torch.cuda.empty_cache()
    log("read ceiling (%.1f MB per launch): decode tiles %.1f us -> %.0f GB/s; flat read %.1f us -> %.0f GB/s" %
        (kv_bytes / 1e6, t_tiles * 1e6, res["tiles_GBps"], t_lin * 1e6, res["flat_GBps"]))
    return res


def stream_rw_ceiling(torch, in_bytes, out_bytes, reps=20):
    """Read-plus-write ceiling for the prefill quantiser (libkvq_probe.so): in_bytes read and out_bytes written
    per launch, interleaved at their ratio, from 2048 workgroups; launches cycle through enough buffers to
    exceed the Infinity Cache and are timed in a graph between events."""
    import ctypes

    path = os.path.join(ROOT, "bit_quantized_kv_quantize_amd", "libkvq_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.kvq_probe_stream_rw.argtypes = [P, ctypes.c_size_t, P, ctypes.c_size_t, ctypes.c_int, P]
    in_bytes, out_bytes = in_bytes // 16 * 16, out_bytes // 16 * 16
    n = max(2, (1 << 30) // (in_bytes + out_bytes) + 1)
    ins = [torch.empty(in_bytes, dtype=torch.uint8, device="cuda") for _ in range(n)]
    outs = [torch.empty(out_bytes, dtype=torch.uint8, device="cuda") for _ in range(n)]

    def launch(i):
        st = lib.kvq_probe_stream_rw(P(ins[i % n].data_ptr()), in_bytes, P(outs[i % n].data_ptr()), out_bytes, 2048,
                                     P(torch.cuda.current_stream().cuda_stream))
        assert st == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(n):
            launch(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            launch(i)
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3 / n)
    t, _, _ = pct(ts)
    del ins, outs
    torch.cuda.empty_cache()
    res = {"GBps": round((in_bytes + out_bytes) / t / 1e9, 1), "us": round(t * 1e6, 2), "read_bytes": in_bytes,
           "write_bytes": out_bytes,
           "kind": "libkvq_probe stream_rw: a flat read of the quantiser's input bytes and a flat write of its "
                   "tile bytes, interleaved at their ratio, 2048 workgroups, per launch in a graph"}
    log("read+write ceiling (%.1f MB in, %.1f MB out): %.1f us -> %.0f GB/s" %
        (in_bytes / 1e6, out_bytes / 1e6, t * 1e6, res["GBps"]))
    return res


def measure_restore(kvq, torch, name, launches=4):
    """The unfused path of QKVShare's injection step: every block of the workload's pool restored to fp16
    K/V rows (kvq_dequantize_blocks), timed in a graph between events."""
    cfg = W.CONFIGS[name]
    case = W.make_case(cfg)
    lay = kvq.Layout(**cfg.layout())
    pool = kvq.new_pool(lay, case.num_blocks)
    for ids, k, v, bm in W.prefill_chunks(case, 0, max_blocks=2048, threads=16):
        kvq.quantize_blocks(lay, pool, torch.from_numpy(ids).cuda(), torch.from_numpy(k).view(torch.float16).cuda(),
                            torch.from_numpy(v).view(torch.float16).cuda())
    ids = torch.arange(case.num_blocks, dtype=torch.int32, device="cuda")
    ko, vo = kvq.dequantize_blocks(lay, pool, ids)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kvq.dequantize_blocks(lay, pool, ids, ko, vo)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for _ in range(launches):
            kvq.dequantize_blocks(lay, pool, ids, ko, vo)
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / launches)
    us = float(np.median(ts))
    moved = pool.numel() + 2 * ko.numel() * 2
    log("restore fp16 %s: %.1f us for %d blocks, %.0f GB/s (read + write)" % (name, us, case.num_blocks,
                                                                             moved / us / 1e3))
    del pool, ko, vo
    torch.cuda.empty_cache()
    return {"workload": name, "blocks": case.num_blocks, "us": round(us, 2), "bytes_moved": moved,
            "GBps": round(moved / us / 1e3, 1)}


def measure_workload(kvq, torch, name, launches=16, graph=True, reps=20):
    """One workload at full size: its layer quantised on the GPU (copied to INSTANCES pools), the append
    where the workload appends, then decode kernels captured back to back in a HIP graph (cycling the
    pools) and timed between events on the launch stream (launched eagerly with graph=False); the prefill
    quantiser timed the same way on the layer's first chunk of blocks (at most 2048, kept resident).
    Returns per-launch times (median, p10, p90) and algorithmic bytes."""
    cfg = workload_config(name)
    case = W.make_case(cfg)
    lay = kvq.Layout(**cfg.layout())
    pool = kvq.new_pool(lay, case.num_blocks)
    prec = np.full(case.n_seqs, 4, np.uint8) if cfg.mixed else None
    wide = {} if cfg.mixed else None
    qchunk = None
    for ids, k, v, bm in W.prefill_chunks(case, 0, max_blocks=2048, threads=16, prec_out=prec):
        dev_in = (torch.from_numpy(ids).cuda(), torch.from_numpy(k).view(torch.float16).cuda(),
                  torch.from_numpy(v).view(torch.float16).cuda(),
                  None if bm is None else torch.from_numpy(bm.view(np.int32)).cuda())
        kvq.quantize_blocks(lay, pool, *dev_in)
        if qchunk is None:
            qchunk = dev_in
        if bm is not None:
            for i, b in enumerate(ids):
                wide[int(b)] = bm[i]
    table = torch.from_numpy(case.block_table).cuda()
    positions = torch.from_numpy(case.positions).cuda()
    seq_lens = torch.from_numpy(case.seq_lens).cuda()
    mask = None if case.sentinel_mask is None else torch.from_numpy(case.sentinel_mask.view(np.int32)).cuda()
    q = torch.from_numpy(W.queries(cfg, 0, case.n_seqs)).view(torch.float16).cuda()
    out = torch.empty((case.n_seqs, cfg.num_q_heads, cfg.dv), dtype=torch.float32, device="cuda")
    ws = kvq.new_workspace(lay, case.n_seqs, cfg.num_q_heads, case.max_seq_len)
    app = None
    if case.append:
        ak, av = W.append_kv(cfg, 0, case.n_seqs)
        app = (torch.from_numpy(ak).view(torch.float16).cuda(), torch.from_numpy(av).view(torch.float16).cuda(),
               None if prec is None else torch.from_numpy(prec).cuda())
        kvq.append_tokens(lay, pool, app[0], app[1], table, positions, app[2])
    pools = [pool] + [pool.clone() for _ in range(INSTANCES.get(base_name(name), 1) - 1)]
    torch.cuda.synchronize()

    def timed(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(launches):
                fn(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        if graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(launches):
                    fn(i)
            run = g.replay
        else:
            def run():
                for i in range(launches):
                    fn(i)
        run()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / launches)
        return pct(ts)

    dec_us, dec_p10, dec_p90 = timed(lambda i: kvq.decode_attention(lay, pools[i % len(pools)], q, table, seq_lens,
                                                                     case.max_seq_len, mask, out=out, workspace=ws))
    app_us = None
    if app is not None:
        app_us = timed(lambda i: kvq.append_tokens(lay, pools[i % len(pools)], app[0], app[1], table, positions,
                                                   app[2]))[0]
    nq = int(qchunk[0].numel())
    quant_us = timed(lambda i: kvq.quantize_blocks(lay, pools[i % len(pools)], *qchunk))[0]
    quant = {"blocks": nq, "us": round(quant_us, 2), "token_layers_per_s": round(nq * W.BLOCK / quant_us * 1e6, 0),
             "GBps": round(quantize_bytes(cfg, nq, kvq.tile_bytes(lay)) / quant_us / 1e3, 1)}
    counts = live_rows(case, wide, prec)
    b = decode_bytes(cfg, case, counts, unique=True)
    res = {"decode_us": round(dec_us, 2), "decode_us_p10_p90": [round(dec_p10, 2), round(dec_p90, 2)], "bytes": b,
           "GBps": round(b / dec_us / 1e3, 1),
           "frac_of_hbm_peak": round(b / dec_us / 1e3 / HBM_PEAK_GBPS, 4), "pool_instances": len(pools),
           "append_us": None if app_us is None else round(app_us, 2), "quantize": quant}
    b_log = decode_bytes(cfg, case, counts, unique=False)
    if b_log != b:
        res["logical_bytes"] = b_log
        res["logical_GBps"] = round(b_log / dec_us / 1e3, 1)
    log("workload %s: decode %.2f us/launch, %.1f GB/s algorithmic (%.1f%% of 8 TB/s)%s; quantise %d blocks "
        "%.1f us -> %.3g token-layers/s, %.0f GB/s" %
        (name, dec_us, b / dec_us / 1e3, b / dec_us / 1e3 / 80, "" if app_us is None else ", append %.2f us" % app_us,
         nq, quant_us, quant["token_layers_per_s"], quant["GBps"]))
    del pools, pool, qchunk
    torch.cuda.empty_cache()
    return res


# CPU oracle samples per workload: (sequences decoded with 1 thread, with all threads; blocks quantised with 1
# thread, with all threads). Each workload's sample is a smaller case of the same shapes and distributions
# (its first sequences); times are scaled to one whole layer of the full workload.
CPU_SAMPLES = {
    "tiny_1k": (1, 1, 4, 4),
    "gemma3_12b_4k": (1, 1, 8, 16),
    "llama31_8b_pool_8k": (1, 12, 8, 96),
    "qwen25_14b_prefix_32k": (1, 8, 8, 96),
    "mixed_sentinel_32k": (1, 16, 8, 96),
}


def cpu_baseline(headline, dec_bytes, budget=1.0):
    """The oracle as it stands, timed on this host's cores: per workload, decode attention and quantisation
    with one thread and with all threads (OpenMP over (sequence, KV head) and over tiles), on bounded samples
    scaled to one layer of the full workload. ``dec_bytes``: the GPU's algorithmic decode bytes per layer of
    each workload (the same bytes for the GB/s figures). ``value`` is the headline workload's decode GB/s
    with all threads."""
    import oracle

    visible = len(os.sched_getaffinity(0))
    threads = max(1, min(visible, 16))   # the host share of one GPU: 16 cores
    per = {}
    for name, (s1, sn, q1, qn) in CPU_SAMPLES.items():
        if name not in dec_bytes:
            continue
        cfg = W.CONFIGS[name]
        full = W.make_case(cfg)
        sn = max(1, int(round(sn * budget)))
        sub = W.make_case(cfg, n_seqs=min(sn, full.n_seqs))
        lay = oracle.make_layout(**cfg.layout())
        tb = oracle.tile_bytes(lay)
        k, v = W.blocks_kv(cfg, 0, sub.prefill_blocks, threads=threads)
        bitmaps, prec = W.mixed_precision_inputs(sub, 0, threads) if cfg.mixed else (None, None)
        pool = np.zeros(tb * cfg.num_kv_heads * sub.num_blocks, np.uint8)
        res = {}
        for nt, nb in ((1, q1), (threads, qn)):
            nb = min(nb, sub.prefill_blocks.size)
            oracle.set_threads(nt)
            t0 = time.perf_counter()
            oracle.quantize_blocks(lay, pool, sub.prefill_blocks[:nb], k[: nb * W.BLOCK], v[: nb * W.BLOCK],
                                   None if bitmaps is None else bitmaps[:nb])
            res["quantize_token_layers_per_s_%dt" % nt] = round(nb * W.BLOCK / (time.perf_counter() - t0), 0)
        oracle.set_threads(threads)
        oracle.quantize_blocks(lay, pool, sub.prefill_blocks, k, v, bitmaps)
        if sub.append:
            ak, av = W.append_kv(cfg, 0, sub.n_seqs)
            oracle.append_tokens(lay, pool, ak, av, sub.block_table, sub.positions, prec)
        q = W.queries(cfg, 0, sub.n_seqs)
        for nt, ns in ((1, s1), (threads, sub.n_seqs)):
            ns = min(ns, sub.n_seqs)
            mask = None if sub.sentinel_mask is None else np.ascontiguousarray(sub.sentinel_mask[:ns])
            t0 = time.perf_counter()
            oracle.decode_attention(lay, pool, q[:ns], sub.block_table[:ns], sub.seq_lens[:ns], mask, n_threads=nt)
            t_layer = (time.perf_counter() - t0) * full.n_seqs / ns
            res["decode_s_per_layer_%dt" % nt] = round(t_layer, 3)
            res["decode_GBps_%dt" % nt] = round(dec_bytes[name] / t_layer / 1e9, 4)
        res["sample"] = "%d of %d sequences decoded (1 thread: %d), %d / %d blocks quantised" % (
            sub.n_seqs, full.n_seqs, min(s1, sub.n_seqs), min(qn, sub.prefill_blocks.size),
            min(q1, sub.prefill_blocks.size))
        per[name] = res
        log("cpu oracle %s: decode %.3g s/layer (1 thread), %.3g s/layer (%d threads); quantise %.3g / %.3g "
            "token-layers/s" % (name, res["decode_s_per_layer_1t"], res["decode_s_per_layer_%dt" % threads], threads,
                                res["quantize_token_layers_per_s_1t"], res["quantize_token_layers_per_s_%dt" % threads]))
    h = per[headline]
    return {"value": h["decode_GBps_%dt" % threads], "unit": "GB/s", "cores": threads, "threads": threads,
            "host_cpus_visible": visible, "kind": "oracle",
            "sample": "one layer of each workload from bounded samples (per_workload[*].sample), scaled to the "
                      "whole layer; value = %s decode attention with %d threads" % (headline, threads),
            "per_workload": per}


if __name__ == "__main__":
    main()
