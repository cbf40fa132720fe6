"""The C-ABI library builds, loads and exports every entry point declared in include/kvq.h. Only host-side
calls run here (layout/size helpers and argument errors that return before any launch), so no GPU is
needed."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")
LIB = os.path.join(ROOT, "bit_quantized_kv_quantize_amd", "libkvq.so")
DEBUG_LIB = os.path.join(ROOT, "bit_quantized_kv_quantize_amd", "libkvq_debug.so")


@pytest.fixture(scope="module")
def kvq():
    if not (os.path.exists(LIB) and os.path.exists(DEBUG_LIB)):
        import importlib.util

        spec = importlib.util.spec_from_file_location(
            "kvq_build", os.path.join(ROOT, "bit_quantized_kv_quantize_amd", "_build.py"))
        _build = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(_build)
        _build.build_all()
    import bit_quantized_kv_quantize_amd as kvq

    return kvq


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


@pytest.mark.parametrize("path", [LIB, DEBUG_LIB])
def test_every_declared_symbol_is_exported(kvq, path):
    # the release library and its debug build export exactly the header's entry points (internal symbols
    # are hidden)
    names = declared_functions()
    assert len(names) == 11, names
    dyn = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" [TW] (\S+)", dyn))
    assert set(names) <= exported, set(names) - exported
    assert not {e for e in exported if e.startswith("_ZN3kvq")}, "internal symbols exported"
    assert set(kvq.EXPORTS) == set(names)
    lib = ctypes.CDLL(path)
    for n in names:
        assert getattr(lib, n) is not None


def test_layout_helpers_match_oracle(kvq, orc):
    import kvq_workloads as W

    for cfg in list(W.CONFIGS.values()) + list(W.EXTRA.values()):
        lay = kvq.Layout(**cfg.layout())
        assert kvq.check_layout(lay) == 0
        olay = orc.make_layout(**cfg.layout())
        assert kvq.tile_bytes(lay) == orc.tile_bytes(olay)
        assert kvq.pool_bytes(lay, 10) == 10 * cfg.num_kv_heads * orc.tile_bytes(olay)
        ws = kvq.decode_workspace_bytes(lay, cfg.n_seqs, cfg.num_q_heads, cfg.context + 1)
        assert ws > 0 and ws % 256 == 0


def test_layout_validation_and_status(kvq):
    assert kvq.check_layout(kvq.Layout(96, 8)) == kvq.KVQ_ERR_ARG
    assert kvq.check_layout(kvq.Layout(128, 8, 48, 64)) == kvq.KVQ_ERR_ARG
    assert kvq.check_layout(kvq.Layout(128, 8, -1, 32, 0, 1)) == kvq.KVQ_ERR_UNSUPPORTED
    assert kvq.check_layout(kvq.Layout(128, 0)) == kvq.KVQ_ERR_ARG
    assert kvq.check_layout(kvq.Layout(128, 8, block_tokens=128)) == kvq.KVQ_ERR_ARG
    # unequal K and V head dims: K 192 or 256 with V 128, per-token K groups, no rotation at 192
    assert kvq.check_layout(kvq.Layout(192, 16, 64, 64, v_head_dim=128)) == kvq.KVQ_OK
    assert kvq.check_layout(kvq.Layout(256, 8, 64, 32, 1, v_head_dim=128)) == kvq.KVQ_OK
    assert kvq.check_layout(kvq.Layout(192, 16, 64, 64, 1, v_head_dim=128)) == kvq.KVQ_ERR_UNSUPPORTED
    assert kvq.check_layout(kvq.Layout(192, 16, 64, 64)) == kvq.KVQ_ERR_UNSUPPORTED
    assert kvq.check_layout(kvq.Layout(128, 8, 64, 32, v_head_dim=192)) == kvq.KVQ_ERR_UNSUPPORTED
    assert kvq.check_layout(kvq.Layout(192, 16, -1, 32, v_head_dim=128)) == kvq.KVQ_ERR_UNSUPPORTED
    assert kvq.check_layout(kvq.Layout(192, 16, 128, 64, v_head_dim=128)) == kvq.KVQ_ERR_ARG  # 128 does not divide 192
    assert kvq.check_layout(kvq.Layout(192, 16, 0, 0, format=1, v_head_dim=128)) == kvq.KVQ_ERR_UNSUPPORTED
    assert kvq.check_layout(kvq.Layout(128, 8, v_head_dim=-1)) == kvq.KVQ_ERR_ARG
    assert kvq.tile_bytes(kvq.Layout(96, 8)) == 0
    assert kvq.decode_workspace_bytes(kvq.Layout(128, 8), 4, 12, 100) == 0   # 12 % 8 != 0
    for st in (0, -1, -2, -3, -4, -99):
        assert isinstance(kvq.status_string(st), str) and kvq.status_string(st)


def test_host_argument_errors_return_before_launch(kvq):
    lib = kvq.lib()
    lay = kvq.Layout(128, 8)
    P = ctypes.c_void_p
    bad = kvq.Layout(100, 8)
    assert lib.kvq_quantize_blocks(ctypes.byref(bad), None, None, 1, None, None, None, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_quantize_blocks(ctypes.byref(lay), None, None, 0, None, None, None, None) == kvq.KVQ_OK
    assert lib.kvq_quantize_blocks(ctypes.byref(lay), None, None, 2, None, None, None, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_quantize_blocks(ctypes.byref(lay), P(256), P(256), 1, P(256), P(256), P(256),
                                   None) == kvq.KVQ_ERR_ARG                    # prec_bits on a non-mixed pool
    assert lib.kvq_dequantize_blocks(ctypes.byref(bad), P(256), P(256), 1, P(256), P(256), None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_dequantize_blocks(ctypes.byref(lay), None, None, 0, None, None, None) == kvq.KVQ_OK
    assert lib.kvq_dequantize_blocks(ctypes.byref(lay), P(256), P(256), -1, P(256), P(256), None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_dequantize_blocks(ctypes.byref(lay), P(256), P(256), 3, None, P(256), None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_copy_blocks(ctypes.byref(lay), None, None, None, None, 0, None) == kvq.KVQ_OK
    assert lib.kvq_copy_blocks(ctypes.byref(lay), P(256), P(256), P(256), None, 2, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_copy_blocks(ctypes.byref(lay), P(264), P(256), P(256), P(256), 2, None) == kvq.KVQ_ERR_ARG
    chan = kvq.Layout(128, 8, -1, 32, 1, 0)
    assert lib.kvq_append_tokens(ctypes.byref(chan), P(256), 1, P(256), P(256), P(256), 1, P(256), None,
                                 None) == kvq.KVQ_ERR_UNSUPPORTED
    assert lib.kvq_decode_attention(ctypes.byref(lay), P(256), P(256), 2, 12, P(256), 4, P(256), 100, None, 0,
                                    0.1, P(256), P(256), 1 << 20, None) == kvq.KVQ_ERR_ARG   # 12 % 8
    assert lib.kvq_decode_attention(ctypes.byref(lay), P(256), P(256), 2, 16, P(256), 1, P(256), 300, None, 0,
                                    0.1, P(256), P(256), 1 << 20, None) == kvq.KVQ_ERR_ARG   # 300 > 1 block
    assert lib.kvq_decode_attention(ctypes.byref(lay), P(256), P(256), 2, 16, P(256), 4, P(256), 1000, P(256), 3,
                                    0.1, P(256), P(256), 1 << 20, None) == kvq.KVQ_ERR_ARG   # mask too short
    assert lib.kvq_decode_attention(ctypes.byref(lay), P(256), P(256), 2, 16, P(256), 4, P(256), 1000, None, 0,
                                    0.1, P(256), P(256), 16, None) == kvq.KVQ_ERR_WORKSPACE
    assert lib.kvq_decode_attention(ctypes.byref(lay), P(256), P(256), 2, 16, P(256), 4, P(256), 1000, None, 0,
                                    0.1, P(256), P(257), 1 << 20, None) == kvq.KVQ_ERR_WORKSPACE  # misaligned
    assert lib.kvq_decode_attention(ctypes.byref(lay), P(256), P(256), 0, 16, P(256), 4, P(256), 1000, None, 0,
                                    0.1, None, None, 0, None) == kvq.KVQ_OK                 # nothing to do


def test_workspace_bytes_never_shrink_with_size(kvq):
    # A workspace sized for (n_seqs, max_seq_len) serves every call with no more sequences and no longer
    # maximum length (include/kvq.h), across the split plans of every decode kernel.
    layouts = [kvq.Layout(128, 8, 64, 64), kvq.Layout(128, 8, -1, 32, 1, 0), kvq.Layout(256, 8, 64, 64),
               kvq.Layout(128, 8, 64, 64, 0, 1), kvq.Layout(128, 2, -1, 64), kvq.Layout(64, 4, 32, 32),
               kvq.Layout(128, 8, 64, 64, 0, 2), kvq.Layout(192, 16, 64, 64, v_head_dim=128)]
    lens = [0, 1, 255, 256, 1000, 4096, 8193, 32768, 100000, 300000]
    seqs = [1, 2, 3, 5, 12, 40, 64, 128, 300, 1000]
    for lay in layouts:
        for g in (1, 2, 4, 5, 8):
            nqh = lay.num_kv_heads * g
            tab = {(s, n): kvq.decode_workspace_bytes(lay, s, nqh, n) for s in seqs for n in lens}
            for (s, n), b in tab.items():
                for (s2, n2), b2 in tab.items():
                    if s2 <= s and n2 <= n:
                        assert b2 <= b, (lay.as_dict(), nqh, (s, n, b), (s2, n2, b2))
