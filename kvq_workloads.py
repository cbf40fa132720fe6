"""Seeded synthetic workloads shaped like the pages' multi-agent KV-cache scenarios.

This module only draws inputs: fp16 K/V rows, decode queries, block tables, sentinel masks and per-token
precision maps. It holds none of the codec's or the attention's arithmetic, so the GPU library and the
CPU oracle can both consume exactly the same bytes.

Every random draw uses numpy ``Generator(PCG64(SeedSequence([config_index, layer, stream, index])))``.
Values are drawn in fp32, outlier channels are scaled in fp32, and the result is rounded to fp16
(round to nearest even). K and V of one physical block are drawn from that block's own seed, so a block
shared by several block tables (a shared prefix) is one set of rows, and any subset of blocks can be
regenerated on its own.

The five workloads (sizes from the task configuration; the pages give only model names and context
lengths: Gemma 3 12B and Llama 3.1 8B agents at 4K-32K in "Agent Memory Below the Prompt", a long shared
prefix reused by many short agent turns in the UltraQuant article, an 8k live budget with sentinel slots
in the IntentKV article, per-token bit widths in QKVShare):

  tiny_1k              1 seq x 1024 tokens, 8 q heads = 8 KV heads, d 128, K/V groups of 64 per token.
  gemma3_12b_4k        1 agent x 4096 tokens, 16 q / 8 KV heads, d 256, 48 layers, groups of 64.
  llama31_8b_pool_8k   12 agents x 8192 tokens, 32 q / 8 KV heads, d 128, 32 layers, one pool of blocks,
                       block tables a seeded random permutation of the pool, groups of 64.
  qwen25_14b_prefix_32k  64 requests sharing one 32768-token prefix plus 512 private tokens each,
                       40 q / 8 KV heads, d 128, Walsh-Hadamard rotation, K per channel per block,
                       V per token in groups of 32.
  mixed_sentinel_32k   128 seqs x 32768 slots, 32 q / 8 KV heads, d 128, groups of 64, top 20% of tokens
                       by K norm stored 8-bit, 24576 of 32768 slots per sequence remapped to the
                       sentinel (8192 live), then one appended token per sequence.

One more workload for the MLA models "Agent Memory Below the Prompt" lists (technical summary 2.2,
DeepSeek-Coder-V2-Lite: K and V head dims differ):

  deepseek_v2_lite_mla_8k  12 agents x 8192 tokens, 16 q = 16 KV heads, K head dim 192 (128 + 64 rotary),
                       V head dim 128, 27 layers, one pool of blocks (permuted tables), groups of 64, no
                       rotation (192 is not a power of two).
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 256

# Random streams of SeedSequence([config_index, layer, stream, index]).
STREAM_K, STREAM_V, STREAM_Q, STREAM_OUTLIER, STREAM_TABLE, STREAM_SENTINEL, STREAM_APPEND = range(1, 8)


@dataclasses.dataclass(frozen=True)
class Config:
    index: int            # position in the task's list of configurations
    name: str
    head_dim: int
    num_q_heads: int
    num_kv_heads: int
    layers: int
    k_group: int          # > 0 per-token groups; -1 per channel per block
    v_group: int
    rotate: int
    mixed: int
    n_seqs: int
    context: int          # tokens already cached per sequence before the decode step
    table: str            # "identity" | "perm" | "shared_prefix"
    append: bool          # the decode step first appends one token per sequence
    outlier_channels: int  # per (layer, KV head): K channels scaled by outlier_scale
    outlier_scale: float
    v_std: float
    shared_prefix: int = 0  # shared_prefix tables: tokens of the common prefix
    dead_fraction: float = 0.0  # fraction of cached slots remapped to the sentinel
    top_fraction: float = 0.0   # mixed pools: fraction of tokens (largest K norm) stored 8-bit
    fmt: int = 0                # pool format: 0 group-wise codes, 1 FP8 E4M3 per element
    width_fracs: Tuple[float, float, float] = (0.0, 0.0, 0.0)  # mixed = 2 pools: fractions of tokens
    # stored FP16 (largest K norms), 8-bit (the next largest) and 2-bit (the smallest); the rest are 4-bit
    v_head_dim: int = 0         # V's head dim when it differs from K's (MLA); 0 = head_dim

    @property
    def dv(self) -> int:
        return self.v_head_dim or self.head_dim

    def layout(self) -> Dict[str, int]:
        return dict(head_dim=self.head_dim, num_kv_heads=self.num_kv_heads, block_tokens=BLOCK,
                    k_group=self.k_group, v_group=self.v_group, rotate=self.rotate, mixed=self.mixed,
                    format=self.fmt, v_head_dim=self.v_head_dim)


CONFIGS: Dict[str, Config] = {
    c.name: c for c in [
        Config(0, "tiny_1k", 128, 8, 8, 1, 64, 64, 0, 0, 1, 1024, "identity", True, 4, 10.0, 1.0),
        Config(1, "gemma3_12b_4k", 256, 16, 8, 48, 64, 64, 0, 0, 1, 4096, "identity", True, 5, 8.0, 0.5),
        Config(2, "llama31_8b_pool_8k", 128, 32, 8, 32, 64, 64, 0, 0, 12, 8192, "perm", True, 4, 10.0, 1.0),
        Config(3, "qwen25_14b_prefix_32k", 128, 40, 8, 1, -1, 32, 1, 0, 64, 32768 + 512, "shared_prefix",
               False, 4, 10.0, 1.0, shared_prefix=32768),
        Config(4, "mixed_sentinel_32k", 128, 32, 8, 1, 64, 64, 0, 1, 128, 32768, "perm", True, 4, 10.0,
               1.0, dead_fraction=0.75, top_fraction=0.2),
    ]
}
CONFIG_ORDER: List[str] = [n for n, _ in sorted(CONFIGS.items(), key=lambda kv: kv[1].index)]

EXTRA: Dict[str, Config] = {
    c.name: c for c in [
        Config(10, "deepseek_v2_lite_mla_8k", 192, 16, 16, 27, 64, 64, 0, 0, 12, 8192, "perm", True, 4, 10.0,
               1.0, v_head_dim=128),
    ]
}


def fp8_variant(cfg: Config) -> Config:
    """The same workload (same seeds, shapes and tables) stored as an FP8 E4M3 pool, the baseline the
    UltraQuant article compares the 4-bit cache against: no groups, no per-token widths."""
    return dataclasses.replace(cfg, name=cfg.name + "_fp8", k_group=0, v_group=0, mixed=0, fmt=1,
                               top_fraction=0.0)


def widths_variant(cfg: Config, fracs: Tuple[float, float, float] = (0.05, 0.15, 0.30)) -> Config:
    """The same workload with per-token widths {2, 4, 8, FP16} (a mixed = 2 pool): each sequence's tokens
    ranked by K norm, the largest ``fracs[0]`` stored FP16, the next ``fracs[1]`` 8-bit, the smallest
    ``fracs[2]`` 2-bit, the rest 4-bit. Per-token K groups only."""
    return dataclasses.replace(cfg, name=cfg.name + "_widths", mixed=2, top_fraction=0.0, width_fracs=fracs)


def sentinel_variant(cfg: Config, dead: float = 0.5) -> Config:
    """The same workload with a fraction ``dead`` of every sequence's cached slots remapped to the sentinel
    (the IntentKV article's invalidation instead of compaction)."""
    return dataclasses.replace(cfg, name=cfg.name + "_sentinel", dead_fraction=dead)


def named_config(name: str) -> Config:
    """A workload by name; the suffixes _fp8, _widths and _sentinel name its FP8, per-token-width and
    sentinel-slot variants (they compose, innermost first)."""
    for suffix, variant in (("_fp8", fp8_variant), ("_widths", widths_variant), ("_sentinel", sentinel_variant)):
        if name.endswith(suffix):
            return variant(named_config(name[:-len(suffix)]))
    return CONFIGS[name] if name in CONFIGS else EXTRA[name]


def _rng(cfg: Config, layer: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.index, layer, stream, index])))


def outlier_channels(cfg: Config, layer: int) -> np.ndarray:
    """int [H_kv][n_outliers]: K channels scaled by cfg.outlier_scale, fixed across tokens."""
    rng = _rng(cfg, layer, STREAM_OUTLIER)
    return np.stack([rng.choice(cfg.head_dim, cfg.outlier_channels, replace=False)
                     for _ in range(cfg.num_kv_heads)])


def _draw_rows(cfg: Config, layer: int, stream_k: int, stream_v: int, index: int, n_rows: int,
               outliers: np.ndarray):
    shape = (n_rows, cfg.num_kv_heads, cfg.head_dim)
    k = _rng(cfg, layer, stream_k, index).standard_normal(shape, dtype=np.float32)
    for h in range(cfg.num_kv_heads):
        k[:, h, outliers[h]] *= np.float32(cfg.outlier_scale)
    v = _rng(cfg, layer, stream_v, index).standard_normal((n_rows, cfg.num_kv_heads, cfg.dv), dtype=np.float32)
    if cfg.v_std != 1.0:
        v *= np.float32(cfg.v_std)
    return k.astype(np.float16).view(np.uint16), v.astype(np.float16).view(np.uint16)


def block_kv(cfg: Config, layer: int, block_id: int, outliers: Optional[np.ndarray] = None):
    """fp16 bits (K [256][H_kv][d], V [256][H_kv][dv]) of physical block ``block_id`` in ``layer``."""
    if outliers is None:
        outliers = outlier_channels(cfg, layer)
    return _draw_rows(cfg, layer, STREAM_K, STREAM_V, block_id, BLOCK, outliers)


def blocks_kv(cfg: Config, layer: int, block_ids: Sequence[int], threads: int = 8):
    """(K, V) for several physical blocks, concatenated token-major: [len(block_ids) * 256][H_kv][d or dv]."""
    outl = outlier_channels(cfg, layer)
    ids = [int(b) for b in block_ids]
    n = len(ids)
    k = np.empty((n * BLOCK, cfg.num_kv_heads, cfg.head_dim), np.uint16)
    v = np.empty((n * BLOCK, cfg.num_kv_heads, cfg.dv), np.uint16)

    def one(i):
        kb, vb = block_kv(cfg, layer, ids[i], outl)
        k[i * BLOCK:(i + 1) * BLOCK] = kb
        v[i * BLOCK:(i + 1) * BLOCK] = vb

    if threads > 1 and n > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(n)))
    else:
        for i in range(n):
            one(i)
    return k, v


def append_kv(cfg: Config, layer: int, n_seqs: int, step: int = 0):
    """fp16 bits (K [n_seqs][H_kv][d], V [n_seqs][H_kv][dv]) of the token each sequence appends at decode
    step ``step``."""
    k, v = _draw_rows(cfg, layer, STREAM_APPEND, STREAM_APPEND + 100, step, n_seqs,
                      outlier_channels(cfg, layer))
    return k, v


def queries(cfg: Config, layer: int, n_seqs: int, step: int = 0) -> np.ndarray:
    """fp16 bits [n_seqs][H_q][d], N(0, 1)."""
    q = _rng(cfg, layer, STREAM_Q, step).standard_normal((n_seqs, cfg.num_q_heads, cfg.head_dim),
                                                          dtype=np.float32)
    return q.astype(np.float16).view(np.uint16)


@dataclasses.dataclass
class Case:
    """One layer-independent decode scenario: pool geometry, tables, lengths, masks."""
    cfg: Config
    n_seqs: int
    context: np.ndarray          # int32 [n_seqs] tokens cached before the step
    num_blocks: int              # physical blocks in the pool
    block_table: np.ndarray      # int32 [n_seqs][max_blocks_per_seq]; unused entries 0
    prefill_blocks: np.ndarray   # int32 physical ids holding cached tokens (each once)
    append: bool
    sentinel_mask: Optional[np.ndarray]  # uint32 [n_seqs][words] over the post-append length

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def seq_lens(self) -> np.ndarray:
        """Lengths attended by the decode step (after the append, if any)."""
        return (self.context + (1 if self.append else 0)).astype(np.int32)

    @property
    def positions(self) -> np.ndarray:
        return self.context.astype(np.int32)

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.n_seqs else 0

    @property
    def mask_words(self) -> int:
        return 0 if self.sentinel_mask is None else int(self.sentinel_mask.shape[1])


def make_case(cfg: Config, n_seqs: Optional[int] = None, context=None, shared_prefix: Optional[int] = None,
              append: Optional[bool] = None, dead_fraction: Optional[float] = None) -> Case:
    """Build the scenario of ``cfg``; the keyword arguments shrink it (parity cases) or make it ragged
    (``context`` may be a list of per-sequence lengths)."""
    n = cfg.n_seqs if n_seqs is None else int(n_seqs)
    if context is None:
        ctx = np.full(n, cfg.context, np.int64)
    elif np.isscalar(context):
        ctx = np.full(n, int(context), np.int64)
    else:
        ctx = np.asarray(context, np.int64)
        assert ctx.size == n
    app = cfg.append if append is None else bool(append)
    total = ctx + (1 if app else 0)
    nblk = (total + BLOCK - 1) // BLOCK
    maxb = int(max(1, nblk.max() if n else 1))
    table = np.zeros((n, maxb), np.int32)
    rng = _rng(cfg, 0, STREAM_TABLE)
    if cfg.table == "shared_prefix":
        sp = cfg.shared_prefix if shared_prefix is None else int(shared_prefix)
        assert sp % BLOCK == 0 and np.all(ctx >= sp)
        n_pref = sp // BLOCK
        n_priv = nblk - n_pref
        num_blocks = int(n_pref + n_priv.sum())
        perm = rng.permutation(num_blocks).astype(np.int32)
        off = n_pref
        for s in range(n):
            table[s, :n_pref] = perm[:n_pref]
            table[s, n_pref:nblk[s]] = perm[off: off + n_priv[s]]
            off += n_priv[s]
    else:
        num_blocks = int(nblk.sum())
        ids = rng.permutation(num_blocks).astype(np.int32) if cfg.table == "perm" else \
            np.arange(num_blocks, dtype=np.int32)
        off = 0
        for s in range(n):
            table[s, :nblk[s]] = ids[off: off + nblk[s]]
            off += nblk[s]
    # Blocks that hold cached (pre-step) tokens, each physical id once.
    used = []
    for s in range(n):
        used.extend(table[s, : (ctx[s] + BLOCK - 1) // BLOCK].tolist())
    prefill = np.array(sorted(set(used)), np.int32)
    dead = cfg.dead_fraction if dead_fraction is None else float(dead_fraction)
    mask = None
    if dead > 0.0:
        words = (int(total.max()) + 31) // 32
        mask = np.zeros((n, words), np.uint32)
        for s in range(n):
            m = int(np.floor(dead * ctx[s]))
            r = _rng(cfg, 0, STREAM_SENTINEL, s)
            slots = r.choice(int(ctx[s]), m, replace=False)
            np.bitwise_or.at(mask[s], slots // 32, (np.uint32(1) << (slots % 32).astype(np.uint32)))
    return Case(cfg, n, ctx.astype(np.int32), num_blocks, table, prefill, app, mask)


def k_norms_sq(k_rows: np.ndarray) -> np.ndarray:
    """Squared L2 norm (fp64) of each token's K over all heads and channels: [n_tokens]."""
    x = k_rows.view(np.float16).astype(np.float64)
    return (x * x).reshape(x.shape[0], int(np.prod(x.shape[1:]))).sum(axis=1)


def precision_map(norms_sq: np.ndarray, top_fraction: float) -> np.ndarray:
    """bool [n]: the floor(top_fraction * n) tokens with the largest K norm (ties to the lower index)."""
    n = norms_sq.size
    k = int(np.floor(top_fraction * n))
    order = np.argsort(-norms_sq, kind="stable")
    sel = np.zeros(n, bool)
    sel[order[:k]] = True
    return sel


def appended_is_8bit(norms_sq_cached: np.ndarray, norm_sq_new: float, top_fraction: float) -> bool:
    """The appended token is 8-bit iff its norm is at least the smallest norm of the cached top set."""
    k = int(np.floor(top_fraction * norms_sq_cached.size))
    if k == 0:
        return False
    kth = np.sort(norms_sq_cached)[::-1][k - 1]
    return bool(norm_sq_new >= kth)


def width_codes(norms_sq: np.ndarray, fracs) -> np.ndarray:
    """uint8 [n] width codes (0, 1, 2, 3 = 2, 4, 8, 16 bits) of tokens ranked by K norm (ties to the lower
    index): floor(fracs[0] n) largest -> 3, the next floor(fracs[1] n) -> 2, floor(fracs[2] n) smallest
    -> 0 (never one already given 3 or 2), the rest -> 1."""
    n = norms_sq.size
    order = np.argsort(-norms_sq, kind="stable")
    n16, n8 = int(np.floor(fracs[0] * n)), int(np.floor(fracs[1] * n))
    n2 = min(int(np.floor(fracs[2] * n)), n - n16 - n8)
    codes = np.ones(n, np.uint8)
    codes[order[:n16]] = 3
    codes[order[n16:n16 + n8]] = 2
    if n2:
        codes[order[n - n2:]] = 0
    return codes


def appended_width(norms_sq_cached: np.ndarray, norm_sq_new: float, fracs) -> int:
    """Width in bits of an appended token: 16 or 8 if its norm reaches the smallest norm of the cached
    FP16 or FP16 + 8-bit set, 2 if it is below the largest norm of the cached 2-bit set, else 4."""
    codes = width_codes(norms_sq_cached, fracs)
    for c, bits in ((3, 16), (2, 8)):
        if (codes >= c).any() and norm_sq_new >= norms_sq_cached[codes >= c].min():
            return bits
    if (codes == 0).any() and norm_sq_new < norms_sq_cached[codes == 0].max():
        return 2
    return 4


def width_words(codes_rows: np.ndarray) -> np.ndarray:
    """uint8 [n_blocks * 256] width codes -> uint32 [n_blocks][16] (code of row t at bits 2 (t % 16) of
    word t / 16)."""
    nb = codes_rows.size // BLOCK
    c = codes_rows.reshape(nb, 16, 16).astype(np.uint64)
    w = (c << (2 * np.arange(16, dtype=np.uint64))).sum(axis=2)
    return w.astype(np.uint32)


def block_width_words(cfg: Config, ns: np.ndarray, nb: int) -> np.ndarray:
    """Width words of one sequence's nb blocks from the K norms of its ns.size cached tokens; slots past
    the cached tokens get the 4-bit code (mixed = 2) or a clear bit."""
    n = ns.size
    if cfg.mixed == 2:
        codes = np.ones(nb * BLOCK, np.uint8)
        codes[:n] = width_codes(ns, cfg.width_fracs)
        return width_words(codes)
    sel = np.zeros(nb * BLOCK, bool)
    sel[:n] = precision_map(ns, cfg.top_fraction)
    return bits_words(sel)


def append_prec(cfg: Config, ns: np.ndarray, norm_sq_new: float) -> int:
    if cfg.mixed == 2:
        return appended_width(ns, norm_sq_new, cfg.width_fracs)
    return 8 if appended_is_8bit(ns, norm_sq_new, cfg.top_fraction) else 4


def bits_words(sel_rows: np.ndarray) -> np.ndarray:
    """bool [n_blocks * 256] -> uint32 [n_blocks][8] bitmap (bit t % 32 of word t / 32)."""
    nb = sel_rows.size // BLOCK
    b = sel_rows.reshape(nb, 8, 32).astype(np.uint64)
    w = (b << np.arange(32, dtype=np.uint64)).sum(axis=2)
    return w.astype(np.uint32)


def sequence_blocks(case: Case, s: int) -> np.ndarray:
    """Physical ids of the blocks holding sequence s's cached tokens, in logical order."""
    return case.block_table[s, : (int(case.context[s]) + BLOCK - 1) // BLOCK]


def prefill_chunks(case: Case, layer: int, max_blocks: int = 2048, threads: int = 8,
                   prec_out: Optional[np.ndarray] = None):
    """Yield (block_ids, K, V, bitmaps) chunks that together cover every prefill block of ``case`` once,
    each chunk at most ``max_blocks`` blocks (one sequence more for mixed pools), so a full-size pool can
    be filled without holding all of its fp16 source at once.

    For mixed pools ``bitmaps`` is the uint32 [n][W] width words of the chunk's blocks (the same
    per-sequence ranking as ``mixed_precision_inputs``) and, if ``prec_out`` is given, the width of each
    sequence's appended token is written into it; otherwise ``bitmaps`` is None."""
    cfg = case.cfg
    if not cfg.mixed:
        ids = case.prefill_blocks
        for i in range(0, ids.size, max_blocks):
            chunk = ids[i:i + max_blocks]
            k, v = blocks_kv(cfg, layer, chunk, threads)
            yield chunk, k, v, None
        return
    ak = append_kv(cfg, layer, case.n_seqs)[0] if (case.append and prec_out is not None) else None
    outl = outlier_channels(cfg, layer)
    s0 = 0
    while s0 < case.n_seqs:
        seqs, n_blk = [], 0
        while s0 < case.n_seqs and (not seqs or n_blk < max_blocks):
            seqs.append(s0)
            n_blk += sequence_blocks(case, s0).size
            s0 += 1
        if prec_out is not None:
            prec_out[seqs] = 4
        if n_blk == 0:
            continue
        ids = np.concatenate([sequence_blocks(case, s) for s in seqs]).astype(np.int32)
        k = np.empty((n_blk * BLOCK, cfg.num_kv_heads, cfg.head_dim), np.uint16)
        v = np.empty((n_blk * BLOCK, cfg.num_kv_heads, cfg.dv), np.uint16)
        norms = np.empty(n_blk * BLOCK, np.float64)

        def one(i):
            kb, vb = block_kv(cfg, layer, int(ids[i]), outl)
            k[i * BLOCK:(i + 1) * BLOCK] = kb
            v[i * BLOCK:(i + 1) * BLOCK] = vb
            norms[i * BLOCK:(i + 1) * BLOCK] = k_norms_sq(kb)

        if threads > 1:
            with ThreadPoolExecutor(max_workers=threads) as ex:
                list(ex.map(one, range(n_blk)))
        else:
            for i in range(n_blk):
                one(i)
        bitmaps = np.empty((n_blk, 16 if cfg.mixed == 2 else 8), np.uint32)
        off = 0
        for s in seqs:
            nb = sequence_blocks(case, s).size
            n = int(case.context[s])
            ns = norms[off * BLOCK: off * BLOCK + n]
            bitmaps[off: off + nb] = block_width_words(cfg, ns, nb)
            if ak is not None and nb:
                prec_out[s] = append_prec(cfg, ns, float(k_norms_sq(ak[s:s + 1])[0]))
            off += nb
        yield ids, k, v, bitmaps


def mixed_precision_inputs(case: Case, layer: int, threads: int = 8):
    """For a mixed pool: per prefill block the uint32 [W] width words (W = 8 for mixed = 1, 16 for mixed = 2;
    aligned with case.prefill_blocks) and per sequence the width in bits of its appended token.

    Each sequence ranks its own cached tokens by K norm; blocks must not be shared between sequences."""
    cfg = case.cfg
    pos = {int(b): i for i, b in enumerate(case.prefill_blocks)}
    bitmaps = np.zeros((case.prefill_blocks.size, 16 if cfg.mixed == 2 else 8), np.uint32)
    prec = np.full(case.n_seqs, 4, np.uint8)
    ak, _ = append_kv(cfg, layer, case.n_seqs)
    for s in range(case.n_seqs):
        blocks = sequence_blocks(case, s)
        k, _ = blocks_kv(cfg, layer, blocks, threads)
        n = int(case.context[s])
        ns = k_norms_sq(k[:n])
        words = block_width_words(cfg, ns, blocks.size)
        for i, b in enumerate(blocks):
            bitmaps[pos[int(b)]] = words[i]
        if case.append and blocks.size:
            prec[s] = append_prec(cfg, ns, float(k_norms_sq(ak[s:s + 1])[0]))
    return bitmaps, prec
