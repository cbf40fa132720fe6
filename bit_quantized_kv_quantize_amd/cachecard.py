"""Saving and restoring quantised sequences as a card file.

The card follows QKVShare's methodology section (the CacheCard: the quantised groups, the per-token bit
widths, and metadata - sequence length, model identity, position offsets - handed from one agent to the
next) stored the way "Agent Memory Below the Prompt" (technical summary 2.1) keeps its block pool on disk:
safetensors files of the quantised blocks as stored. Here a card is one safetensors file holding

* ``tiles``            uint8 [n_blocks, H_kv, tile_bytes]: the blocks the sequences use, byte for byte as in
                       the pool (codes, fp16 scales and zeros, the width bitmap of mixed pools);
* ``block_table``      int32 [n_seqs, max_blocks]: each sequence's blocks as indices into ``tiles`` (-1 past
                       its end);
* ``seq_lens``         int32 [n_seqs];
* ``position_offsets`` int32 [n_seqs]: position of each sequence's first slot in the sender's numbering;

and, in the file's metadata, the layout fields and the model identity. Moving blocks between the pool and
host memory runs in the library (kvq_copy_blocks); this module only arranges the host-side arrays.
"""
from __future__ import annotations

import json
from typing import Optional

import numpy as np

FORMAT = "kvq-cachecard"
VERSION = "1"
_LAYOUT_FIELDS = ("head_dim", "num_kv_heads", "block_tokens", "k_group", "v_group", "rotate", "mixed", "format",
                  "v_head_dim")


def _host_i32(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


def pack(layout_fields: dict, tiles: np.ndarray, block_table, seq_lens, model_id: str = "",
         position_offsets=None):
    """Host arrays -> (tensors, metadata) of a card. ``tiles`` holds the blocks that ``block_table`` names,
    in the order of ``used`` (returned by :func:`used_blocks`), so the table is rewritten as indices."""
    bt = _host_i32(block_table)
    lens = _host_i32(seq_lens)
    used = used_blocks(bt, lens, int(layout_fields["block_tokens"]))
    if tiles.shape[0] != used.size:
        raise ValueError("tiles holds %d blocks, the tables use %d" % (tiles.shape[0], used.size))
    index = {int(b): i for i, b in enumerate(used)}
    local = np.full(bt.shape, -1, np.int32)
    for s in range(bt.shape[0]):
        nb = _n_blocks(int(lens[s]), int(layout_fields["block_tokens"]))
        local[s, :nb] = [index[int(b)] for b in bt[s, :nb]]
    po = np.zeros(lens.size, np.int32) if position_offsets is None else _host_i32(position_offsets)
    meta = {k: str(int(layout_fields.get(k, 0))) for k in _LAYOUT_FIELDS}
    meta.update(card_format=FORMAT, card_version=VERSION, model_id=str(model_id), tile_bytes=str(tiles.shape[2]))
    tensors = {"tiles": np.ascontiguousarray(tiles, dtype=np.uint8), "block_table": local, "seq_lens": lens,
               "position_offsets": po}
    return tensors, meta


def unpack(tensors: dict, meta: dict, layout_fields: Optional[dict] = None):
    """(tensors, metadata) of a card -> dict with tiles, block_table (card indices), seq_lens,
    position_offsets, model_id and layout. With ``layout_fields`` the card's layout must equal it."""
    if meta.get("card_format") != FORMAT or meta.get("card_version") != VERSION:
        raise ValueError("not a %s v%s file" % (FORMAT, VERSION))
    layout = {k: int(meta.get(k, "0")) for k in _LAYOUT_FIELDS}
    if layout_fields is not None:
        want = {k: int(layout_fields.get(k, 0)) for k in _LAYOUT_FIELDS}
        if want != layout:
            raise ValueError("card layout %s differs from %s" % (json.dumps(layout), json.dumps(want)))
    tiles = tensors["tiles"]
    if tiles.ndim != 3 or tiles.shape[1] != layout["num_kv_heads"] or tiles.shape[2] != int(meta["tile_bytes"]):
        raise ValueError("tiles have shape %s" % (tiles.shape,))
    bt = tensors["block_table"]
    if bt.size and (bt.max() >= tiles.shape[0] or bt.min() < -1):
        raise ValueError("block table names blocks outside the card")
    return dict(tiles=tiles, block_table=bt, seq_lens=tensors["seq_lens"],
                position_offsets=tensors["position_offsets"], model_id=meta.get("model_id", ""), layout=layout)


def _n_blocks(seq_len: int, block_tokens: int) -> int:
    return (seq_len + block_tokens - 1) // block_tokens


def used_blocks(block_table, seq_lens, block_tokens: int = 256) -> np.ndarray:
    """Distinct physical blocks the sequences use (their first ceil(seq_len / 256) table entries), sorted."""
    bt = _host_i32(block_table)
    lens = _host_i32(seq_lens)
    ids = [bt[s, :_n_blocks(int(lens[s]), block_tokens)] for s in range(bt.shape[0])]
    return np.unique(np.concatenate(ids)) if ids else np.zeros(0, np.int32)


def save(path: str, layout, pool, block_table, seq_lens, model_id: str = "", position_offsets=None) -> int:
    """Write the blocks of these sequences from a device pool to a card file; returns the number of blocks.
    A block shared by several sequences (a common prefix) is stored once."""
    import torch
    from safetensors.numpy import save_file

    from . import copy_blocks, new_pool, tile_bytes

    fields = layout.as_dict()
    used = used_blocks(block_table, seq_lens, fields["block_tokens"])
    stage = new_pool(layout, int(used.size), device=pool.device)
    if used.size:
        copy_blocks(layout, pool, torch.from_numpy(used.astype(np.int32)).to(pool.device), stage,
                    torch.arange(used.size, dtype=torch.int32, device=pool.device))
    tiles = stage.cpu().numpy().reshape(used.size, fields["num_kv_heads"], tile_bytes(layout))
    tensors, meta = pack(fields, tiles, block_table, seq_lens, model_id, position_offsets)
    save_file(tensors, path, metadata=meta)
    return int(used.size)


def load(path: str, layout, pool, block_ids):
    """Place a card's blocks into a device pool at ``block_ids`` (one free block per card block, int32 on
    the pool's device) and return the card's contents with ``block_table`` rewritten to those ids (a
    device int32 tensor; -1 past each sequence's end)."""
    import torch
    from safetensors import safe_open
    from safetensors.numpy import load_file

    from . import copy_blocks

    with safe_open(path, framework="numpy") as f:
        meta = f.metadata()
    card = unpack(load_file(path), meta, layout.as_dict())
    n = card["tiles"].shape[0]
    if int(block_ids.numel()) != n:
        raise ValueError("card holds %d blocks, %d ids given" % (n, int(block_ids.numel())))
    if n:
        stage = torch.from_numpy(np.ascontiguousarray(card["tiles"]).reshape(-1)).to(pool.device)
        copy_blocks(layout, stage, torch.arange(n, dtype=torch.int32, device=pool.device), pool, block_ids)
    ids = block_ids.detach().cpu().numpy().astype(np.int32)
    bt = card["block_table"]
    table = np.full(bt.shape, -1, np.int32)
    table[bt >= 0] = ids[bt[bt >= 0]]
    card["block_table"] = torch.from_numpy(table).to(pool.device)
    return card
