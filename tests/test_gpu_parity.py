"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Codes, fp16 scales/zeros, width bitmaps and padding must be bit-exact (whole pool bytes compared);
decode attention must be within 2e-3 max relative error (normwise per sequence and query head).
Sizes span several tiles with ragged tails; the configurations are the five workloads shrunk so the
oracle finishes in seconds (full-size sampled checks live in test_gpu_fullsize.py)."""
import numpy as np
import pytest

import kvq_workloads as W
from gpu_cases import TOL, gpu_run, host_inputs, oracle_run, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import bit_quantized_kv_quantize_amd as kvq

    return kvq, torch


SMALL = {
    "tiny_1k": dict(n_seqs=2, context=[1024, 700]),
    "gemma3_12b_4k": dict(n_seqs=2, context=[1000, 513]),
    "llama31_8b_pool_8k": dict(n_seqs=4, context=[2048, 777, 1, 0]),
    "qwen25_14b_prefix_32k": dict(n_seqs=3, shared_prefix=512, context=[768, 612, 1023]),
    "mixed_sentinel_32k": dict(n_seqs=3, context=[1024, 600, 333]),
}


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_pool_bytes_bit_exact(env, orc, name):
    kvq, torch = env
    case = W.make_case(W.CONFIGS[name], **SMALL[name])
    inp = host_inputs(case)
    ref_pool, _ = oracle_run(orc, case, inp, decode=False)
    got_pool, _ = gpu_run(kvq, torch, case, inp, decode=False)
    diff = np.nonzero(got_pool != ref_pool)[0]
    assert diff.size == 0, "first differing bytes at %s" % diff[:16]


GARBAGE_LAYOUTS = [  # head dim, V head dim, k_group, v_group, rotate, mixed, format
    (128, 0, 64, 64, 0, 0, 0), (128, 0, 64, 64, 1, 1, 0), (128, 0, 32, 64, 0, 2, 0), (128, 0, -1, 32, 1, 0, 0),
    (64, 0, 16, 32, 1, 2, 0), (256, 0, 64, 8, 1, 1, 0), (192, 128, 64, 32, 0, 2, 0), (192, 128, 64, 64, 0, 1, 0),
    (256, 128, 64, 32, 1, 2, 0), (128, 0, 0, 0, 1, 0, 1)]


@pytest.mark.parametrize("layout", GARBAGE_LAYOUTS)
def test_quantize_overwrites_every_byte_of_its_tiles(env, orc, layout):
    # Whole blocks quantised into a pool whose bytes were all 0xFF (a reused pool): every byte of the
    # written tiles - codes, the zeroed rest of narrower records, parameters, headers, padding - equals the
    # oracle's (which clears each tile first); tiles of other blocks keep their bytes.
    kvq, torch = env
    d, dv, kg, vg, rotate, mixed, fmt = layout
    cfg = W.Config(9, "garbage", d, 4, 2, 1, kg, vg, rotate, mixed, 3, 0, "perm", False, 3, 10.0, 1.0,
                   top_fraction=0.3 if mixed == 1 else 0.0, fmt=fmt,
                   width_fracs=(0.1, 0.2, 0.3) if mixed == 2 else (0.0, 0.0, 0.0), v_head_dim=dv)
    case = W.make_case(cfg, context=[700, 257, 1024])
    inp = host_inputs(case)
    lay_o = orc.make_layout(**cfg.layout())
    ref = np.full(orc.tile_bytes(lay_o) * cfg.num_kv_heads * (case.num_blocks + 2), 0xFF, np.uint8)
    orc.quantize_blocks(lay_o, ref, case.prefill_blocks, inp["k"], inp["v"], inp["bitmaps"])
    lay = kvq.Layout(**cfg.layout())
    pool = torch.full((ref.size,), 0xFF, dtype=torch.uint8, device="cuda")
    kvq.quantize_blocks(lay, pool, to_dev(case.prefill_blocks, torch), to_dev(inp["k"], torch, torch.float16),
                        to_dev(inp["v"], torch, torch.float16),
                        None if inp["bitmaps"] is None else to_dev(inp["bitmaps"].view(np.int32), torch))
    got = pool.cpu().numpy()
    diff = np.nonzero(got != ref)[0]
    assert diff.size == 0, "first differing bytes at %s" % diff[:16]


@pytest.fixture(params=["dispatch", "mfma", "generic"])
def decode_path(request, monkeypatch, env):
    """Run decode through the release library's normal dispatch (the row-list matrix-core kernel where
    compiled), and through the block matrix-core kernel and the generic kernel, forced in the debug build
    (libkvq_debug.so) by its test hook KVQ_DECODE_KERNEL; a layout a forced kernel lacks falls through to the
    next."""
    kvq, _ = env
    if request.param == "dispatch":
        monkeypatch.delenv("KVQ_DECODE_KERNEL", raising=False)
        kvq.use_library("release")
    else:
        monkeypatch.setenv("KVQ_DECODE_KERNEL", request.param)
        kvq.use_library("debug")
    yield request.param
    kvq.use_library("release")


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_decode_within_tolerance(env, orc, name, decode_path):
    kvq, torch = env
    case = W.make_case(W.CONFIGS[name], **SMALL[name])
    inp = host_inputs(case)
    _, ref = oracle_run(orc, case, inp)
    _, got = gpu_run(kvq, torch, case, inp)
    err = rel_err(got, ref)
    print("%s [%s]: max rel err %.3g" % (name, decode_path, err))
    assert err <= TOL
    assert np.all(got[case.seq_lens == 0] == 0)


@pytest.mark.parametrize("rotate,mixed,kg,vg,G,d", [
    (0, 0, 64, 64, 1, 128), (0, 0, 32, 32, 3, 64), (1, 0, 64, 32, 8, 128), (0, 1, 64, 64, 16, 128),
    (1, 0, -1, 32, 5, 256), (1, 1, 32, 64, 2, 64), (0, 0, 128, 16, 4, 128), (0, 0, 8, 256, 2, 256),
    (1, 0, 64, 64, 8, 128), (0, 0, 64, 64, 2, 128), (1, 0, 64, 64, 4, 256), (0, 0, 64, 64, 1, 256),
    (1, 0, -1, 32, 5, 128), (0, 0, -1, 64, 8, 128), (1, 0, -1, 32, 3, 128), (0, 0, -1, 32, 1, 128),
    (0, 1, 64, 64, 4, 128), (1, 1, 64, 64, 2, 128), (0, 2, 64, 64, 4, 128), (1, 2, 32, 64, 2, 64),
    (1, 2, 64, 32, 8, 256), (0, 2, 16, 128, 1, 128), (1, 2, 64, 64, 2, 128), (0, 2, 64, 64, 1, 128)])
def test_layout_variants(env, orc, rotate, mixed, kg, vg, G, d, decode_path):
    # Generic layouts beyond the five workloads: group sizes, widths, rotation, G up to 16, ragged
    # lengths (0, 1, 255, 256, 257, long) and sentinel masks (one sequence entirely sentinel).
    kvq, torch = env
    H = 2
    cfg = W.Config(9, "variant", d, H * G, H, 1, kg, vg, rotate, mixed, 6, 0, "perm", kg > 0, 3, 10.0, 1.0,
                   dead_fraction=0.5, top_fraction=0.2 if mixed == 1 else 0.0,
                   width_fracs=(0.1, 0.2, 0.3) if mixed == 2 else (0.0, 0.0, 0.0))
    case = W.make_case(cfg, context=[0, 1, 255, 256, 700, 1500] if kg > 0 else [1, 255, 256, 257, 700, 1500])
    case.sentinel_mask[4] = 0xFFFFFFFF
    if kg > 0:
        case.sentinel_mask[4, (int(case.seq_lens[4]) - 1) // 32:] = 0xFFFFFFFF  # include the appended slot
    inp = host_inputs(case)
    ref_pool, ref = oracle_run(orc, case, inp)
    got_pool, got = gpu_run(kvq, torch, case, inp)
    assert np.array_equal(got_pool, ref_pool)
    err = rel_err(got, ref)
    print("variant rotate=%d mixed=%d kg=%d vg=%d G=%d d=%d [%s]: max rel err %.3g" % (rotate, mixed, kg, vg, G, d,
                                                                                    decode_path, err))
    assert err <= TOL
    assert not got[4].any()                                  # every slot remapped to the sentinel
    if case.seq_lens[0] == 0:
        assert not got[0].any()


def test_decode_is_deterministic(env, decode_path):
    kvq, torch = env
    case = W.make_case(W.CONFIGS["llama31_8b_pool_8k"], n_seqs=3, context=[3000, 2048, 100])
    inp = host_inputs(case)
    _, a = gpu_run(kvq, torch, case, inp)
    _, b = gpu_run(kvq, torch, case, inp)
    assert np.array_equal(a, b)


SENTINEL_LAYOUTS = {
    # name: (d, dv, G, k_group, v_group, rotate, mixed, format, row width of every row (mixed pools))
    "d128_g1": (128, 0, 1, 64, 64, 0, 0, 0, None),       # row-list kernel (gather mode); forced block, generic
    "d128_g4_rot": (128, 0, 4, 64, 64, 1, 0, 0, None),   # row-list kernel, rotated pool
    "d128_g4_8bit": (128, 0, 4, 64, 64, 0, 1, 0, 8),     # row-list kernel, 8-bit chunks
    "d128_g2_2bit": (128, 0, 2, 64, 64, 0, 2, 0, 2),     # row-list kernel, 2-bit chunks
    "d128_g2_fp16": (128, 0, 2, 64, 64, 0, 2, 0, 16),    # row-list kernel, FP16 chunks
    "d128_g8": (128, 0, 8, 64, 64, 0, 0, 0, None),       # block matrix-core kernel
    "d256_g2": (256, 0, 2, 64, 64, 0, 0, 0, None),       # block matrix-core kernel, head dim 256
    "mla_g1": (192, 128, 1, 64, 64, 0, 0, 0, None),      # row-list kernel, K 192 / V 128; forced block, generic
    "mla_g2_8bit": (192, 128, 2, 64, 64, 0, 1, 0, 8),    # row-list kernel, K 192, 8-bit chunks
    "mla_g1_2bit": (192, 128, 1, 64, 64, 0, 2, 0, 2),    # row-list kernel, K 192, 2-bit chunks
    "mla_g4_fp16": (192, 128, 4, 64, 64, 0, 2, 0, 16),   # row-list kernel, K 192, FP16 chunks
    "kchan_g5": (128, 0, 5, -1, 32, 0, 0, 0, None),      # per-channel-K kernel
    "kchan_g5_rot": (128, 0, 5, -1, 32, 1, 0, 0, None),  # per-channel-K kernel, rotated pool
    "fp8_g4": (128, 0, 4, 0, 0, 0, 0, 1, None),          # FP8 pool with a sentinel mask: generic kernel
}
_WIDTH_WORD = {8: 0xFFFFFFFF, 2: 0x00000000, 16: 0xFFFFFFFF}  # mixed = 1: bit set = 8-bit; mixed = 2: codes


@pytest.mark.parametrize("layout", sorted(SENTINEL_LAYOUTS))
def test_sentinel_terms_count_when_live_logits_are_near_minus_1e4(env, orc, layout, decode_path):
    # With every K row identical (and every query head the same), every live logit is scale * c for one
    # constant c; choosing the scale so that this is -1e4 - 1 gives the sentinel slots (logit -1e4, value 0)
    # a weight comparable to the live ones. Skipping sentinel slots alone would then be wrong; the kernels
    # add their exact term in the final merge, and the live logits - of magnitude 1.4e4 in base-2 units -
    # must be accurate to about 1e-3 for the output to stay within tolerance (the matrix-core kernels take
    # their fp64 pass here). Every decode kernel is held to the same 2e-3.
    kvq, torch = env
    d, dv, G, kg, vg, rotate, mixed, fmt, width = SENTINEL_LAYOUTS[layout]
    cfg = W.Config(8, "sentinel_probe", d, G, 1, 1, kg, vg, rotate, mixed, 1, 600, "identity", False, 0, 1.0,
                   1.0, dead_fraction=0.5, fmt=fmt, v_head_dim=dv)
    case = W.make_case(cfg)
    inp = host_inputs(case)
    inp["k"][:] = inp["k"][0]
    inp["q"][0, :] = inp["q"][0, 0]
    if mixed:
        inp["bitmaps"][:] = _WIDTH_WORD[width] if mixed == 1 or width != 8 else 0xAAAAAAAA
    lay_o = orc.make_layout(**cfg.layout())
    tb = orc.tile_bytes(lay_o)
    pool = np.zeros(tb * case.num_blocks, np.uint8)
    orc.quantize_blocks(lay_o, pool, case.prefill_blocks, inp["k"], inp["v"], inp["bitmaps"])
    # the unrotated dequantised K row (fp64) fixes the scale; the oracle and the library both get it
    k0, _, _ = orc.dequant_row(lay_o, pool[:tb], 0)
    if rotate:
        from scipy.linalg import hadamard

        c32 = float(np.float32(1.0 / np.sqrt(d)))
        k0 = hadamard(d).astype(np.float64) @ k0 / (d * c32)
    c = float(inp["q"][0, 0].view(np.float16).astype(np.float64) @ k0)
    scale = float(np.float32(-(1e4 + 1.0) / c))
    ref = orc.decode_attention(lay_o, pool, inp["q"], case.block_table, case.seq_lens, case.sentinel_mask,
                               softmax_scale=scale)
    lay = kvq.Layout(**cfg.layout())
    gp = kvq.new_pool(lay, case.num_blocks)
    kvq.quantize_blocks(lay, gp, to_dev(case.prefill_blocks, torch), to_dev(inp["k"], torch, torch.float16),
                        to_dev(inp["v"], torch, torch.float16),
                        None if inp["bitmaps"] is None else to_dev(inp["bitmaps"].view(np.int32), torch))
    out = kvq.decode_attention(lay, gp, to_dev(inp["q"], torch, torch.float16), to_dev(case.block_table, torch),
                               to_dev(case.seq_lens, torch), case.max_seq_len,
                               to_dev(case.sentinel_mask.view(np.int32), torch), softmax_scale=scale).cpu().numpy()
    assert np.array_equal(gp.cpu().numpy(), pool)
    err = rel_err(out, ref)
    print("sentinel vs live %s [%s]: max rel err %.3g" % (layout, decode_path, err))
    assert err <= TOL
    # the sentinel terms matter here: the live-only average is far from the reference
    t = np.arange(600)
    live = ~((case.sentinel_mask[0][t // 32] >> (t % 32)) & 1).astype(bool)
    vmean = np.mean([orc.dequant_row(lay_o, pool[(case.block_table[0, i // 256]) * tb:][:tb], i % 256)[1]
                     for i in t[live]], axis=0)
    if rotate:
        from scipy.linalg import hadamard

        vmean = hadamard(vmean.size).astype(np.float64) @ vmean / (vmean.size * float(np.float32(1.0 / np.sqrt(
            vmean.size))))
    assert np.abs(ref[0, 0]).max() < 0.5 * np.abs(vmean).max()


def _decode_with(kvq, torch, case, inp, pool, workspace):
    mask = None if case.sentinel_mask is None else to_dev(case.sentinel_mask.view(np.int32), torch)
    out = kvq.decode_attention(kvq.Layout(**case.cfg.layout()), pool, to_dev(inp["q"], torch, torch.float16),
                               to_dev(case.block_table, torch), to_dev(case.seq_lens, torch),
                               max(case.max_seq_len, 1), mask, workspace=workspace)
    return out.cpu().numpy()


REUSE = {  # workload: (large call, small call)
    "llama31_8b_pool_8k": (dict(n_seqs=12, context=[1500 + 211 * i for i in range(12)]),
                           dict(n_seqs=4, context=[3000, 700, 2100, 40])),
    "mixed_sentinel_32k": (dict(n_seqs=10, context=[900 + 150 * i for i in range(10)]),
                           dict(n_seqs=3, context=[2000, 300, 1100])),
    "qwen25_14b_prefix_32k": (dict(n_seqs=9, shared_prefix=512, context=[700 + 90 * i for i in range(9)]),
                              dict(n_seqs=3, shared_prefix=512, context=[1500, 600, 800])),
}


@pytest.mark.parametrize("name", sorted(REUSE))
def test_workspace_reused_across_call_sizes(env, orc, name):
    # One workspace, sized for the large call, serves a large call, a small one, the large one again, and so
    # on: the split-K arrival counters of the large call (at the workspace's end) must not be overwritten by
    # the small call's partials, and every call must leave them at zero.
    kvq, torch = env
    large, small = (W.make_case(W.CONFIGS[name], **kw) for kw in REUSE[name])
    runs = []
    for case in (large, small):
        inp = host_inputs(case)
        _, ref = oracle_run(orc, case, inp)
        pool = to_dev(gpu_run(kvq, torch, case, inp, decode=False)[0], torch)
        runs.append((case, inp, pool, ref))
    lay = kvq.Layout(**large.cfg.layout())
    ws = kvq.new_workspace(lay, large.n_seqs, large.cfg.num_q_heads, large.max_seq_len)
    for step, (case, inp, pool, ref) in enumerate([runs[0], runs[1], runs[0], runs[1], runs[0]]):
        got = _decode_with(kvq, torch, case, inp, pool, ws)
        err = rel_err(got, ref)
        print("workspace reuse %s step %d (%d seqs): max rel err %.3g" % (name, step, case.n_seqs, err))
        assert err <= TOL
    tail = ws[-4 * large.n_seqs * large.cfg.num_kv_heads:].cpu().numpy()
    assert not tail.any()  # the counters are back at zero


def test_debug_build_rejects_bad_device_arguments(env, orc):
    # The debug build copies block ids, lengths and positions back before any launch and returns
    # KVQ_ERR_ARG for out-of-range ones; the outputs stay untouched (nothing ran).
    kvq, torch = env
    case = W.make_case(W.CONFIGS["llama31_8b_pool_8k"], n_seqs=2, context=[600, 300])
    inp = host_inputs(case)
    lay = kvq.Layout(**case.cfg.layout())
    pool = to_dev(gpu_run(kvq, torch, case, inp, decode=False)[0], torch)
    q = to_dev(inp["q"], torch, torch.float16)
    kvq.use_library("debug")
    try:
        table = to_dev(case.block_table, torch)
        lens = to_dev(case.seq_lens, torch)
        out = torch.full((2, case.cfg.num_q_heads, 128), float("nan"), device="cuda")
        kvq.decode_attention(lay, pool, q, table, lens, case.max_seq_len, out=out)  # valid: runs
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()

        def rejects(fn, *args, **kw):
            with pytest.raises(kvq.KvqError) as e:
                fn(*args, **kw)
            assert e.value.status == kvq.KVQ_ERR_ARG

        for bad in (10 ** 6, -1):
            t2 = case.block_table.copy()
            t2[1, 1] = bad
            out.fill_(float("nan"))
            rejects(kvq.decode_attention, lay, pool, q, to_dev(t2, torch), lens, case.max_seq_len, out=out)
            torch.cuda.synchronize()
            assert torch.isnan(out).all()
        rejects(kvq.decode_attention, lay, pool, q, table, to_dev(np.array([600, 5000], np.int32), torch),
                case.max_seq_len)                                              # length above max_seq_len
        before = pool.clone()
        k1, v1 = W.blocks_kv(case.cfg, 0, [0])
        rejects(kvq.quantize_blocks, lay, pool, to_dev(np.array([10 ** 6], np.int32), torch),
                to_dev(k1, torch, torch.float16), to_dev(v1, torch, torch.float16))
        k2, v2 = W.blocks_kv(case.cfg, 0, [0, 1])
        rejects(kvq.quantize_blocks, lay, pool, to_dev(np.array([1, 1], np.int32), torch),
                to_dev(k2, torch, torch.float16), to_dev(v2, torch, torch.float16))   # repeated id
        ak, av = W.append_kv(case.cfg, 0, 2)
        rejects(kvq.append_tokens, lay, pool, to_dev(ak, torch, torch.float16), to_dev(av, torch, torch.float16),
                table, to_dev(np.array([100, case.block_table.shape[1] * 256], np.int32), torch))
        rejects(kvq.dequantize_blocks, lay, pool, to_dev(np.array([0, 10 ** 6], np.int32), torch))
        rejects(kvq.copy_blocks, lay, pool, to_dev(np.array([0, 1], np.int32), torch), pool,
                to_dev(np.array([2, 2], np.int32), torch))
        torch.cuda.synchronize()
        assert torch.equal(pool, before)
    finally:
        kvq.use_library("release")


@pytest.fixture(params=["cascade", "nocascade"])
def cascade_mode(request, monkeypatch, env):
    """Shared blocks through the cascade kernel (the release library's dispatch) or left to the per-sequence
    kernel (the debug build's test hook, KVQ_DECODE_KERNEL=nocascade)."""
    kvq, _ = env
    if request.param == "cascade":
        monkeypatch.delenv("KVQ_DECODE_KERNEL", raising=False)
        kvq.use_library("release")
    else:
        monkeypatch.setenv("KVQ_DECODE_KERNEL", "nocascade")
        kvq.use_library("debug")
    yield request.param
    kvq.use_library("release")


CASCADE_CASES = {
    # 40 sequences x 5 query heads = 200 rows per KV head: two row groups of seven 16-row tiles, the second
    # with a partial tile and idle waves; ragged suffixes
    "rows_40": ({}, dict(n_seqs=40, shared_prefix=1024, context=[1024 + (97 * i) % 1100 for i in range(40)])),
    # more block ranges than shared blocks (empty cascade units); one sequence ends where the prefix ends
    "prefix_8": ({}, dict(n_seqs=4, shared_prefix=2048, context=[2048, 2100, 4000, 2304])),
    # 17 sequences x 8 query heads = 136 rows (two row groups of five tiles), V groups of 64, no rotation
    "g8_vg64": (dict(num_q_heads=64, v_group=64, rotate=0),
                dict(n_seqs=17, shared_prefix=1536, context=[1536 + (131 * i) % 900 for i in range(17)])),
    # one query head per KV head: 3 rows, one partial tile
    "g1": (dict(num_q_heads=8), dict(n_seqs=3, shared_prefix=768, context=[768, 1000, 1300])),
}


@pytest.mark.parametrize("name", sorted(CASCADE_CASES))
def test_cascade_shared_blocks(env, orc, name, cascade_mode):
    # The shared-prefix layout (K per channel, V groups of 32, rotation, G = 5, and the variants above) with
    # the prefix blocks aliased in every sequence's table, against the oracle (which reads each sequence's
    # table as given).
    import dataclasses

    kvq, torch = env
    over, kw = CASCADE_CASES[name]
    cfg = dataclasses.replace(W.CONFIGS["qwen25_14b_prefix_32k"], name="prefix_" + name, **over)
    case = W.make_case(cfg, **kw)
    inp = host_inputs(case)
    _, ref = oracle_run(orc, case, inp)
    _, got = gpu_run(kvq, torch, case, inp)
    err = rel_err(got, ref)
    print("cascade %s [%s]: max rel err %.3g" % (name, cascade_mode, err))
    assert err <= TOL


def _two_prefix_case(n_seqs, prefix_blocks, context):
    """The prefix workload's layout with two shared prompts: sequences below n_seqs // 2 share prefix A (the
    case's own), the others a second copy of it at other physical blocks (prefix B)."""
    case = W.make_case(W.CONFIGS["qwen25_14b_prefix_32k"], n_seqs=n_seqs, shared_prefix=256 * prefix_blocks,
                       context=context)
    b_ids = np.arange(case.num_blocks, case.num_blocks + prefix_blocks, dtype=np.int32)
    case.block_table[n_seqs // 2:, :prefix_blocks] = b_ids
    case.num_blocks += prefix_blocks
    case.prefill_blocks = np.array(sorted(set(case.prefill_blocks.tolist()) | set(b_ids.tolist())), np.int32)
    return case


def _nested_prefix_case(over):
    """Sharing among subsets of the batch, nested as in a prefix tree: blocks 0-3 are shared by sequences 0-10
    (sequence 10 ends inside block 3), blocks 4-7 by sequences 0-4 and, as other blocks, by sequences 5-9,
    blocks 8-9 by sequences 0-1 and by 5-7; sequence 11 shares nothing; the rest of every table is private."""
    import dataclasses

    cfg = dataclasses.replace(W.CONFIGS["qwen25_14b_prefix_32k"], name="prefix_nested", **over)
    ctx = [2560 + (37 * i) % 700 for i in range(10)] + [900, 3000]
    case = W.make_case(cfg, n_seqs=12, shared_prefix=0, context=ctx)
    nb = case.num_blocks
    new = iter(range(nb, nb + 100))
    shared = {}

    def put(seqs, cols, tag):
        for c in cols:
            key = (tag, c)
            if key not in shared:
                shared[key] = next(new)
            for sq in seqs:
                case.block_table[sq, c] = shared[key]

    put(range(11), range(4), "all")
    put(range(5), range(4, 8), "A")
    put(range(5, 10), range(4, 8), "B")
    put(range(2), range(8, 10), "C")
    put(range(5, 8), range(8, 10), "D")
    case.num_blocks = nb + len(shared)
    case.prefill_blocks = np.array(sorted(set(case.prefill_blocks.tolist()) | set(shared.values())), np.int32)
    return case


@pytest.mark.parametrize("over", [{}, dict(num_q_heads=64, v_group=64, rotate=0)], ids=["g5", "g8_vg64"])
def test_cascade_nested_subsets(env, orc, over, cascade_mode):
    # Blocks shared by subsets of the sequences (a prefix tree of four levels, a sequence that ends inside a
    # shared block, one that shares nothing) against the oracle, which reads every table as given.
    kvq, torch = env
    case = _nested_prefix_case(over)
    inp = host_inputs(case)
    _, ref = oracle_run(orc, case, inp)
    _, got = gpu_run(kvq, torch, case, inp)
    err = rel_err(got, ref)
    print("nested subsets %s [%s]: max rel err %.3g" % (over, cascade_mode, err))
    assert err <= TOL


@pytest.mark.parametrize("n_seqs", [8, 13])
def test_cascade_groups_sharing_different_prefixes(env, orc, n_seqs, cascade_mode):
    # Two prompts, each shared by half of the sequences: blocks aliased by several tables but not by all of
    # them. The cascade takes each prompt's blocks for its half; the output must not depend on which kernel
    # took which block.
    kvq, torch = env
    case = _two_prefix_case(n_seqs, 4, [1024 + (211 * i) % 700 for i in range(n_seqs)])
    inp = host_inputs(case)
    _, ref = oracle_run(orc, case, inp)
    _, got = gpu_run(kvq, torch, case, inp)
    err = rel_err(got, ref)
    print("two prefixes n_seqs=%d [%s]: max rel err %.3g" % (n_seqs, cascade_mode, err))
    assert err <= TOL


def _f16_ulps(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in fp16 ulps between bit patterns (order-preserving integer map; +0 and -0 coincide)."""
    def key(x):
        x = x.astype(np.int64)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(key(a_bits) - key(b_bits))


DEQUANT_VARIANTS = [  # rotate, mixed, k_group, v_group, d
    (0, 0, 64, 64, 128), (1, 0, -1, 32, 128), (1, 1, 64, 64, 128), (0, 1, 32, 64, 64), (1, 0, 64, 32, 256),
    (0, 0, -1, 64, 64), (1, 0, 8, 256, 256), (0, 2, 64, 64, 128), (1, 2, 32, 16, 64), (1, 2, 64, 64, 256)]


@pytest.mark.parametrize("variant", DEQUANT_VARIANTS + W.CONFIG_ORDER)
def test_dequantize_blocks_within_one_ulp(env, orc, variant):
    # The restored fp16 rows of every quantised block (and, where the workload appends, the appended rows)
    # against the oracle's exact values rounded once: at most one fp16 ulp apart, and equal almost everywhere.
    kvq, torch = env
    if isinstance(variant, str):
        case = W.make_case(W.CONFIGS[variant], **SMALL[variant])
    else:
        rotate, mixed, kg, vg, d = variant
        cfg = W.Config(9, "variant", d, 2, 2, 1, kg, vg, rotate, mixed, 3, 0, "perm", kg > 0, 3, 10.0, 1.0,
                       top_fraction=0.3 if mixed == 1 else 0.0,
                       width_fracs=(0.1, 0.2, 0.3) if mixed == 2 else (0.0, 0.0, 0.0))
        case = W.make_case(cfg, context=[700, 257, 1024])
    inp = host_inputs(case)
    ref_pool, _ = oracle_run(orc, case, inp, decode=False)
    got_pool, _ = gpu_run(kvq, torch, case, inp, decode=False)
    assert np.array_equal(got_pool, ref_pool)
    ids = np.unique(case.block_table[case.block_table >= 0]).astype(np.int32)
    ids = ids[ids < case.num_blocks][::-1].copy()  # reversed: output order follows the id list
    lay_o = orc.make_layout(**case.cfg.layout())
    kr, vr = orc.dequantize_blocks(lay_o, ref_pool, ids)
    lay = kvq.Layout(**case.cfg.layout())
    kg_, vg_ = kvq.dequantize_blocks(lay, to_dev(got_pool, torch), to_dev(ids, torch))
    torch.cuda.synchronize()
    for got, ref in ((kg_, kr), (vg_, vr)):
        g = got.cpu().numpy().view(np.uint16)
        u = _f16_ulps(g, ref)
        print("dequantize %s: %d values, %d differ by one ulp, max %d" % (variant, u.size, int((u == 1).sum()),
                                                                          int(u.max())))
        assert u.max() <= 1
        assert (u > 0).mean() < 1e-3


@pytest.mark.parametrize("name", ["qwen25_14b_prefix_32k", "mixed_sentinel_32k", "llama31_8b_pool_8k",
                                  "llama31_8b_pool_8k_widths", "deepseek_v2_lite_mla_8k"])
def test_card_save_load_round_trip(env, orc, tmp_path, name):
    # Blocks saved from a GPU pool to a card file (kvq_copy_blocks gathers them) and loaded into another pool
    # at shuffled ids (kvq_copy_blocks scatters them): the card's tiles equal the oracle's bytes, and decode
    # over the reloaded pool equals decode over the original pool bit for bit.
    kvq, torch = env
    from bit_quantized_kv_quantize_amd import cachecard
    from safetensors.numpy import load_file

    size = SMALL.get(name.replace("_widths", ""), dict(n_seqs=3, context=[1000, 300, 513]))
    case = W.make_case(W.named_config(name), **size)
    inp = host_inputs(case)
    ref_pool, _ = oracle_run(orc, case, inp, decode=False)
    cfg = case.cfg
    lay = kvq.Layout(**cfg.layout())
    pool = to_dev(gpu_run(kvq, torch, case, inp, decode=False)[0], torch)
    table = to_dev(case.block_table, torch)
    lens = to_dev(case.seq_lens, torch)
    q = to_dev(inp["q"], torch, torch.float16)
    mask = None if case.sentinel_mask is None else to_dev(case.sentinel_mask.view(np.int32), torch)
    out1 = kvq.decode_attention(lay, pool, q, table, lens, case.max_seq_len, mask)
    path = str(tmp_path / "card.safetensors")
    n = cachecard.save(path, lay, pool, table, lens, model_id=name)
    tb = kvq.tile_bytes(lay)
    used = cachecard.used_blocks(case.block_table, case.seq_lens)
    assert n == used.size
    tiles = load_file(path)["tiles"]
    assert np.array_equal(tiles, ref_pool.reshape(case.num_blocks, cfg.num_kv_heads, tb)[used])
    pool2 = kvq.new_pool(lay, n + 7)
    ids = torch.from_numpy((np.random.default_rng(2).permutation(n) + 7).astype(np.int32)).cuda()
    card = cachecard.load(path, lay, pool2, ids)
    assert card["model_id"] == name
    t2 = card["block_table"].clamp(min=0).contiguous()
    out2 = kvq.decode_attention(lay, pool2, q, t2, lens, case.max_seq_len, mask)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)


def test_fp8_quantize_every_fp16_value_bit_exact(env, orc):
    # Every finite fp16 bit pattern once in K and once (reversed) in V of an FP8 pool: the hardware conversion
    # after the clamp to +-448 gives the oracle's E4M3 rounding (nearest even, saturating) for all of them.
    kvq, torch = env
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    bits = np.where(np.isfinite(vals), bits, np.uint16(0))
    k = bits.reshape(2 * 256, 2, 64)
    v = bits[::-1].copy().reshape(2 * 256, 2, 64)
    for rotate in (0, 1):
        lay_o = orc.make_layout(64, 2, 0, 0, rotate, 0, format=1)
        ref = np.zeros(orc.tile_bytes(lay_o) * 2 * 2, np.uint8)
        ids = np.array([1, 0], np.int32)
        kk, vv = (k, v) if not rotate else (np.clip(vals.reshape(k.shape), -8, 8).astype(np.float16).view(np.uint16),
                                            np.clip(vals[::-1].reshape(k.shape), -8, 8).astype(np.float16).view(np.uint16))
        kk = np.where(np.isfinite(kk.view(np.float16)), kk, np.uint16(0))
        vv = np.where(np.isfinite(vv.view(np.float16)), vv, np.uint16(0))
        orc.quantize_blocks(lay_o, ref, ids, kk, vv)
        lay = kvq.Layout(64, 2, 0, 0, rotate, 0, format=1)
        pool = kvq.new_pool(lay, 2)
        kvq.quantize_blocks(lay, pool, to_dev(ids, torch), to_dev(kk, torch, torch.float16),
                            to_dev(vv, torch, torch.float16))
        got = pool.cpu().numpy()
        diff = np.nonzero(got != ref)[0]
        assert diff.size == 0, (rotate, diff[:8], got[diff[:8]], ref[diff[:8]])


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_fp8_pool_decode_and_restore(env, orc, name):
    # The workloads stored as FP8 pools (same seeded data and tables): pool bytes (quantise and append)
    # bit-exact, decode attention within tolerance, and the restored fp16 rows exact (unrotated pools) or
    # within one fp16 ulp (rotated).
    kvq, torch = env
    cfg = W.fp8_variant(W.CONFIGS[name])
    case = W.make_case(cfg, **SMALL[name])
    inp = host_inputs(case)
    ref_pool, ref = oracle_run(orc, case, inp)
    got_pool, got = gpu_run(kvq, torch, case, inp)
    assert np.array_equal(got_pool, ref_pool)
    err = rel_err(got, ref)
    print("fp8 %s: max rel err %.3g" % (name, err))
    assert err <= TOL
    ids = np.unique(case.prefill_blocks).astype(np.int32)
    kr, vr = orc.dequantize_blocks(orc.make_layout(**cfg.layout()), ref_pool, ids)
    kg_, vg_ = kvq.dequantize_blocks(kvq.Layout(**cfg.layout()), to_dev(got_pool, torch), to_dev(ids, torch))
    for g_, r_ in ((kg_, kr), (vg_, vr)):
        u = _f16_ulps(g_.cpu().numpy().view(np.uint16), r_)
        assert u.max() <= (1 if cfg.rotate else 0)


WIDTH_WORKLOADS = ["tiny_1k", "gemma3_12b_4k", "llama31_8b_pool_8k", "mixed_sentinel_32k"]


@pytest.mark.parametrize("name", WIDTH_WORKLOADS)
def test_widths_pool_decode_and_restore(env, orc, name):
    # The workloads with per-token K groups stored with widths {2, 4, 8, FP16} (same seeded data and tables;
    # widths by K-norm rank): pool bytes (quantise and append) bit-exact, decode attention within
    # tolerance, and the restored fp16 rows within one fp16 ulp of the oracle's.
    kvq, torch = env
    cfg = W.widths_variant(W.CONFIGS[name])
    case = W.make_case(cfg, **SMALL[name])
    inp = host_inputs(case)
    ref_pool, ref = oracle_run(orc, case, inp)
    got_pool, got = gpu_run(kvq, torch, case, inp)
    diff = np.nonzero(got_pool != ref_pool)[0]
    assert diff.size == 0, "first differing bytes at %s" % diff[:16]
    err = rel_err(got, ref)
    print("widths %s: max rel err %.3g" % (name, err))
    assert err <= TOL
    ids = np.unique(case.prefill_blocks).astype(np.int32)
    kr, vr = orc.dequantize_blocks(orc.make_layout(**cfg.layout()), ref_pool, ids)
    kg_, vg_ = kvq.dequantize_blocks(kvq.Layout(**cfg.layout()), to_dev(got_pool, torch), to_dev(ids, torch))
    for g_, r_ in ((kg_, kr), (vg_, vr)):
        u = _f16_ulps(g_.cpu().numpy().view(np.uint16), r_)
        assert u.max() <= 1 and (u > 0).mean() < 1e-3


def test_widths_append_rewrites_record_at_another_width(env, orc):
    # Each slot appended twice, the second time at another width (and once at a width the pool does not
    # hold, stored 4-bit): the record, the parameters and the header field end up as the oracle's.
    kvq, torch = env
    d, H = 128, 4
    rng = np.random.default_rng(21)
    n = 40
    table = np.array([[i % 3] for i in range(n)], np.int32)
    pos = rng.choice(256 * 3, n, replace=False) % 256
    pos = np.unique(pos)[:n].astype(np.int32)
    n = pos.size
    table = table[:n]
    k = rng.standard_normal((2, n, H, d)).astype(np.float16)
    v = rng.standard_normal((2, n, H, d)).astype(np.float16)
    first = rng.choice(np.array([2, 4, 8, 16, 5], np.uint8), n)
    second = rng.choice(np.array([2, 4, 8, 16, 7], np.uint8), n)
    for rotate in (0, 1):
        lay_o = orc.make_layout(d, H, 64, 32, rotate, 2)
        ref = np.zeros(orc.tile_bytes(lay_o) * H * 3, np.uint8)
        lay = kvq.Layout(d, H, 64, 32, rotate, 2)
        pool = kvq.new_pool(lay, 3)
        for step, prec in ((0, first), (1, second)):
            assert orc.append_tokens(lay_o, ref, k[step].view(np.uint16), v[step].view(np.uint16), table, pos,
                                     prec) == 0
            kvq.append_tokens(lay, pool, to_dev(k[step], torch), to_dev(v[step], torch), to_dev(table, torch),
                              to_dev(pos, torch), to_dev(prec, torch))
        got = pool.cpu().numpy()
        diff = np.nonzero(got != ref)[0]
        assert diff.size == 0, (rotate, diff[:16])


@pytest.mark.parametrize("mixed", [1, 2])
def test_row_lists_of_a_sequence_past_256k_slots(env, orc, mixed):
    # One sequence of 270,000 slots (1055 blocks, more than the compaction kernel's 1024 threads scan in one
    # pass) with sentinel slots and per-token widths: row lists of 100K+ entries per width.
    kvq, torch = env
    cfg = W.Config(9, "long", 128, 4, 1, 1, 64, 64, 1, mixed, 1, 270000, "perm", True, 3, 10.0, 1.0,
                   dead_fraction=0.4, top_fraction=0.2 if mixed == 1 else 0.0,
                   width_fracs=(0.05, 0.15, 0.3) if mixed == 2 else (0.0, 0.0, 0.0))
    case = W.make_case(cfg)
    inp = host_inputs(case)
    ref_pool, ref = oracle_run(orc, case, inp, n_threads=8)
    got_pool, got = gpu_run(kvq, torch, case, inp)
    assert np.array_equal(got_pool, ref_pool)
    err = rel_err(got, ref)
    print("long sequence mixed=%d: max rel err %.3g" % (mixed, err))
    assert err <= TOL


MLA_VARIANTS = [  # K head dim, rotate, mixed, k_group, v_group, G (V head dim 128)
    (192, 0, 0, 64, 64, 1), (192, 0, 0, 64, 64, 2), (192, 0, 0, 64, 64, 4), (192, 0, 2, 64, 32, 2),
    (256, 1, 0, 64, 32, 4), (256, 1, 1, 32, 64, 1), (192, 0, 1, 32, 128, 16), (192, 0, 0, 8, 16, 3),
    (192, 0, 2, 64, 64, 1), (192, 0, 1, 64, 64, 4), (192, 0, 2, 64, 64, 2)]


# The same without sentinel slots (pure 4-bit MLA pools stream through the row-list kernel)
MLA_STREAMING = [(192, 0, 0, 64, 64, 1, 0.0), (192, 0, 0, 64, 64, 2, 0.0), (192, 0, 0, 64, 64, 4, 0.0)]


@pytest.mark.parametrize("variant", [v + (0.5,) for v in MLA_VARIANTS] + MLA_STREAMING)
def test_unequal_head_dims(env, orc, variant, decode_path):
    # MLA layouts (K and V head dims differ): pool bytes (quantise and append) bit-exact, decode within
    # tolerance over ragged lengths, with sentinel slots (one sequence all sentinel) or without, restore
    # within one ulp.
    kvq, torch = env
    d, rotate, mixed, kg, vg, G, dead = variant
    H = 2
    cfg = W.Config(9, "mla", d, H * G, H, 1, kg, vg, rotate, mixed, 6, 0, "perm", True, 3, 10.0, 1.0,
                   dead_fraction=dead, top_fraction=0.2 if mixed == 1 else 0.0,
                   width_fracs=(0.1, 0.2, 0.3) if mixed == 2 else (0.0, 0.0, 0.0), v_head_dim=128)
    case = W.make_case(cfg, context=[0, 1, 255, 256, 700, 1500] if dead else [0, 1, 255, 256, 700, 2900])
    if dead:
        case.sentinel_mask[4] = 0xFFFFFFFF
    inp = host_inputs(case)
    ref_pool, ref = oracle_run(orc, case, inp)
    got_pool, got = gpu_run(kvq, torch, case, inp)
    diff = np.nonzero(got_pool != ref_pool)[0]
    assert diff.size == 0, "first differing bytes at %s" % diff[:16]
    assert got.shape == (6, H * G, 128)
    err = rel_err(got, ref)
    print("mla d=%d rotate=%d mixed=%d kg=%d vg=%d G=%d dead=%.1f [%s]: max rel err %.3g" % (
        d, rotate, mixed, kg, vg, G, dead, decode_path, err))
    assert err <= TOL
    if dead:
        assert not got[4].any()                              # every slot remapped to the sentinel
    ids = np.unique(case.prefill_blocks).astype(np.int32)
    kr, vr = orc.dequantize_blocks(orc.make_layout(**cfg.layout()), ref_pool, ids)
    kg_, vg_ = kvq.dequantize_blocks(kvq.Layout(**cfg.layout()), to_dev(got_pool, torch), to_dev(ids, torch))
    for g_, r_ in ((kg_, kr), (vg_, vr)):
        u = _f16_ulps(g_.cpu().numpy().view(np.uint16), r_)
        assert u.max() <= 1 and (u > 0).mean() < 1e-3


@pytest.mark.parametrize("layout", ["rows", "rows_sentinel", "kchan", "generic_d64"])
def test_many_short_sequences(env, orc, layout):
    # 2000 sequences of 1..600 slots in one call (grids of thousands of (sequence, KV head) pairs, row lists
    # of 2000 sequences): every output row against the oracle.
    kvq, torch = env
    n = 2000
    ctx = [1 + (37 * i) % 600 for i in range(n)]
    if layout == "kchan":
        cfg = W.Config(9, "many", 128, 4, 2, 1, -1, 32, 1, 0, n, 0, "perm", False, 3, 10.0, 1.0)
    elif layout == "generic_d64":
        cfg = W.Config(9, "many", 64, 6, 2, 1, 32, 32, 0, 0, n, 0, "perm", True, 3, 10.0, 1.0)
    else:
        cfg = W.Config(9, "many", 128, 8, 2, 1, 64, 64, 0, 0, n, 0, "perm", True, 3, 10.0, 1.0,
                       dead_fraction=0.3 if layout == "rows_sentinel" else 0.0)
    case = W.make_case(cfg, context=ctx)
    inp = host_inputs(case)
    ref_pool, ref = oracle_run(orc, case, inp, n_threads=8)
    got_pool, got = gpu_run(kvq, torch, case, inp)
    assert np.array_equal(got_pool, ref_pool)
    err = rel_err(got, ref)
    print("many sequences [%s]: max rel err %.3g" % (layout, err))
    assert err <= TOL
