"""The decode entry point that allocates nothing (kvq_decode_attention_static, its workspace a per-GPU device
array inside the library) against kvq_decode_attention with a caller-supplied workspace, called through the
C ABI: two calls in a row on each workload, the second with a smaller input, must give the same output bit
for bit (the same kernels and split plan run) and stay within tolerance of the oracle."""
import ctypes

import numpy as np
import pytest

import kvq_workloads as W
from gpu_cases import TOL, gpu_run, host_inputs, oracle_run, rel_err, to_dev

pytestmark = pytest.mark.gpu

# workload -> (first call, second, smaller call)
CALLS = {
    "llama31_8b_pool_8k": (dict(n_seqs=12, context=[2048 + 301 * i for i in range(12)]),
                           dict(n_seqs=3, context=[1200, 5000, 7])),
    "mixed_sentinel_32k": (dict(n_seqs=8, context=[3000 + 500 * i for i in range(8)]),
                           dict(n_seqs=2, context=[1500, 640])),
    "qwen25_14b_prefix_32k": (dict(n_seqs=10, shared_prefix=1024, context=[1100 + 70 * i for i in range(10)]),
                              dict(n_seqs=4, shared_prefix=512, context=[600, 900, 512, 700])),
    "gemma3_12b_4k": (dict(n_seqs=3, context=[4096, 3000, 100]), dict(n_seqs=1, context=[1000])),
}


@pytest.fixture(scope="module")
def env():
    import torch

    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import bit_quantized_kv_quantize_amd as kvq

    kvq.use_library("release")
    return kvq, torch


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _decode_static(kvq, torch, lay, pool, q, table, lens, max_len, mask, scale):
    n, hq, _ = q.shape
    out = torch.full((n, hq, lay.dv), float("nan"), dtype=torch.float32, device="cuda")
    st = kvq.lib().kvq_decode_attention_static(
        ctypes.byref(lay), _p(pool), _p(q), n, hq, _p(table), int(table.shape[1]), _p(lens), int(max_len), _p(mask),
        0 if mask is None else int(mask.shape[1]), ctypes.c_float(scale), _p(out),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == kvq.KVQ_OK, kvq.status_string(st)
    return out


@pytest.mark.parametrize("name", sorted(CALLS))
def test_static_entry_matches_workspace_entry(env, orc, name):
    kvq, torch = env
    for step, kw in enumerate(CALLS[name]):
        case = W.make_case(W.CONFIGS[name], **kw)
        inp = host_inputs(case)
        _, ref = oracle_run(orc, case, inp)
        pool = to_dev(gpu_run(kvq, torch, case, inp, decode=False)[0], torch)
        lay = kvq.Layout(**case.cfg.layout())
        q = to_dev(inp["q"], torch, torch.float16)
        table = to_dev(case.block_table, torch)
        lens = to_dev(case.seq_lens, torch)
        mask = None if case.sentinel_mask is None else to_dev(case.sentinel_mask.view(np.int32), torch)
        scale = float(np.float32(1.0 / np.sqrt(case.cfg.head_dim)))
        got = _decode_static(kvq, torch, lay, pool, q, table, lens, case.max_seq_len, mask, scale)
        want = kvq.decode_attention(lay, pool, q, table, lens, case.max_seq_len, mask, softmax_scale=scale)
        torch.cuda.synchronize()
        got, want = got.cpu().numpy(), want.cpu().numpy()
        err = rel_err(got, ref)
        print("static entry %s call %d (%d seqs): max rel err %.3g" % (name, step, case.n_seqs, err))
        assert np.array_equal(got, want)
        assert err <= TOL


def test_static_entry_rejects_calls_beyond_its_array(env):
    # 128 sequences of 200,000 slots with a sentinel mask need about 200 MB of row lists, beyond the array:
    # KVQ_ERR_WORKSPACE before anything is launched on these (never read) buffers.
    kvq, torch = env
    lay = kvq.Layout(128, 8, 64, 64)
    n, hq, max_len = 128, 32, 200000
    assert kvq.decode_workspace_bytes(lay, n, hq, max_len) > (64 << 20)
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(dummy.data_ptr())
    st = kvq.lib().kvq_decode_attention_static(ctypes.byref(lay), p, p, n, hq, p, (max_len + 255) // 256, p, max_len,
                                               p, (max_len + 31) // 32, ctypes.c_float(0.1), p,
                                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == kvq.KVQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert not dummy.any()
