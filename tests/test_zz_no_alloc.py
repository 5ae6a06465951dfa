"""hsa_forward_noalloc (static scratch, no workspace argument) against
hsa_forward (caller workspace) through the C ABI: the same kernels, so the
outputs and the selection must agree bit for bit, on two calls in a row, the
second with a smaller input (the scratch keeps the first call's contents);
also for global HSA, whose scratch holds the normalised keys."""
import ctypes

import numpy as np
import pytest

import workloads as W

from hsa_check import inputs_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hsa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ultra_long_context_amd as h
    h.load_library()
    return h


def _call_both(hsa, cfg):
    import torch
    inp = W.generate(cfg)
    dev = inputs_to_device(inp)
    print("case %s Lq=%d Lkv=%d q_pos0=%d K=%d G=%d" % (cfg.name, cfg.q_len, cfg.kv_len, cfg.q_pos0,
                                                        cfg.top_k, cfg.group), flush=True)
    ref_out, ref_idx, ref_score = hsa.forward(*dev, q_pos0=cfg.q_pos0, top_k=cfg.top_k, return_topk=True)
    shape = hsa.make_shape(batch=cfg.batch, q_len=cfg.q_len, kv_len=cfg.kv_len, q_pos0=cfg.q_pos0,
                           n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim,
                           top_k=cfg.top_k, dtype=hsa.DTYPE_BF16)
    out = torch.empty_like(ref_out)
    idx = torch.empty_like(ref_idx)
    score = torch.empty_like(ref_score)
    lib = hsa.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptrs = [ctypes.c_void_p(t.data_ptr()) for t in (*dev, out, idx, score)]
    st = lib.hsa_forward_noalloc(ctypes.byref(shape), *ptrs, stream)
    assert st == 0, lib.hsa_status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx)
    assert torch.equal(score, ref_score)
    assert torch.equal(out, ref_out)
    # the binding's wrapper (caller-provided outputs) gives the same again
    out2 = torch.empty_like(ref_out)
    hsa.forward_noalloc(*dev, out2, q_pos0=cfg.q_pos0, top_k=cfg.top_k)
    torch.cuda.synchronize()
    assert torch.equal(out2, ref_out)


def test_noalloc_matches_forward_two_calls_second_smaller(hsa):
    big = W.shrink(W.CONFIGS[3], kv_len=1 << 21)                # 16 rows, 32768 chunks, K 32 (split lists)
    small = W.shrink(W.CONFIGS[3], kv_len=3 << 15, top_k=12)    # 16 rows, 1536 chunks
    _call_both(hsa, big)
    _call_both(hsa, small)


def test_noalloc_rejects_a_prefill_beyond_the_scratch(hsa):
    import torch
    cfg = W.shrink(W.CONFIGS[1], q_len=8192, kv_len=8192)
    dev = inputs_to_device(W.generate(cfg))
    out = torch.empty_like(dev[2])
    with pytest.raises(hsa.HsaError, match="SCRATCH_TOO_SMALL"):
        hsa.forward_noalloc(*dev, out, q_pos0=0, top_k=cfg.top_k)


def _global_both(hsa, cfg, K):
    import torch
    inp = W.generate(cfg)
    dev = inputs_to_device(inp)
    print("case global %s Lq=%d Lkv=%d q_pos0=%d K=%d G=%d" % (cfg.name, cfg.q_len, cfg.kv_len, cfg.q_pos0,
                                                               K, cfg.group), flush=True)
    ref_out = hsa.forward(*dev, q_pos0=cfg.q_pos0, top_k=K)
    shape = hsa.make_shape(batch=cfg.batch, q_len=cfg.q_len, kv_len=cfg.kv_len, q_pos0=cfg.q_pos0,
                           n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim,
                           top_k=K, dtype=hsa.DTYPE_BF16)
    out = torch.empty_like(ref_out)
    lib = hsa.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptrs = [ctypes.c_void_p(t.data_ptr()) for t in (*dev, out)]
    st = lib.hsa_forward_noalloc(ctypes.byref(shape), *ptrs, None, None, stream)
    assert st == 0, lib.hsa_status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)


def test_noalloc_global_hsa_two_calls_second_smaller(hsa):
    """Global HSA (top-K covering every eligible chunk) through the static
    scratch: the normalised keys live there too; two calls, the second smaller."""
    big = W.HsaConfig(name="global_noalloc_big", batch=1, q_len=2048, q_pos0=0, kv_len=2048, n_q_heads=8,
                      n_kv_heads=1, head_dim=128, top_k=8, dtype="bf16", noise_std=0.5, n_needles=4, seed=81)
    small = W.HsaConfig(name="global_noalloc_small", batch=1, q_len=300, q_pos0=900, kv_len=1200, n_q_heads=16,
                        n_kv_heads=2, head_dim=64, top_k=8, dtype="bf16", noise_std=0.5, n_needles=2, seed=82)
    _global_both(hsa, big, K=4096)
    _global_both(hsa, small, K=100)
