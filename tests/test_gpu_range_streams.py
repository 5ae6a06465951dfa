"""GPU parity at extreme value magnitudes, and concurrent calls on two streams.

Value range: V scaled to about 1e5 (beyond fp16's range) and to about 1e-6
(fp16's subnormal range) must give the oracle's output within 2e-2 of the
output's largest magnitude on every attend path: the chunk-major path (many
rows; per-pair partials in HBM), the decode path (few rows; fp32 partials) and
the global path (top-K covering every chunk).  The selection does not depend on
V, so it is checked as in the other parity tests.

Streams: each call on its own stream gets its own cached workspace (arrival
counters, partial buffers), so two forwards enqueued on two streams at once
give exactly the outputs they give alone.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import workloads as W
from workloads import HsaConfig

from hsa_check import check_selection, inputs_to_device, out_to_f64, to_device

pytestmark = pytest.mark.gpu

REL_TOL = 2e-2


@pytest.fixture(scope="module")
def hsa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ultra_long_context_amd as h
    h.load_library()
    return h


def scaled_v(inp, factor):
    """The same inputs with V multiplied by `factor` (in fp64, then stored)."""
    v = W.store(W.to_f64(inp.v, inp.cfg.dtype) * factor, inp.cfg.dtype)
    return replace(inp, v=v)


def sample(total, n, seed):
    if total <= n:
        return np.arange(total)
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(total, size=n - 2, replace=False).tolist()) | {0, total - 1}
    return np.array(sorted(rows))


def check_relative(got, ref, what):
    scale = float(np.abs(ref).max())
    err = float(np.abs(got - ref).max())
    assert np.all(np.isfinite(got)), (what, "non-finite output")
    print("  %s: max |out| %.3e, max-abs err %.3e (%.2e of max)" % (what, scale, err, err / scale),
          flush=True)
    assert err <= REL_TOL * scale, (what, err, scale)


CASES = {
    # many rows: B=2, 32 q heads / 4 kv heads, K=16 (the 128K prefill's heads), cut to 2048 tokens
    "chunk_major": lambda: W.shrink(W.CONFIGS[2], q_len=2048, kv_len=2048),
    # few rows over a long history: the decode path (split lists merged by the attend)
    "decode": lambda: W.shrink(W.CONFIGS[3], kv_len=1 << 18),
}


@pytest.mark.parametrize("factor", [1e5, 1e-6])
@pytest.mark.parametrize("case", sorted(CASES))
def test_forward_value_range(hsa, case, factor):
    import torch
    cfg = CASES[case]()
    inp = scaled_v(W.generate(cfg), factor)
    print("case %s V x %g: B=%d Lq=%d Lkv=%d Hq=%d Hkv=%d K=%d" % (
        case, factor, cfg.batch, cfg.q_len, cfg.kv_len, cfg.n_q_heads, cfg.n_kv_heads, cfg.top_k), flush=True)
    dev = inputs_to_device(inp)
    out, idx, score = hsa.forward(*dev, q_pos0=cfg.q_pos0, top_k=cfg.top_k, return_topk=True)
    torch.cuda.synchronize()
    total = cfg.batch * cfg.q_len
    rows = sample(total, 256, seed=int(factor > 1))
    oi, os_, _, oo = oracle.forward(inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v,
                                    q_pos0=cfg.q_pos0, top_k=cfg.top_k, rows=rows)
    gi = idx.cpu().numpy().reshape(total, cfg.n_kv_heads, cfg.top_k)[rows]
    gs = score.cpu().numpy().reshape(total, cfg.n_kv_heads, cfg.top_k)[rows]
    rep = check_selection(inp, rows, gi, gs, oi, os_, ret_scale=oracle.default_scale(cfg.head_dim))
    # the output is compared on the GPU's own selection (identical to the
    # oracle's except for admissible near-tie swaps)
    sel = gi.astype(np.int32)
    _, ref = oracle.attend_blend(inp.q_attn, inp.k, inp.v, sel, gs.astype(np.float64), rows=rows)
    got = out_to_f64(out).reshape(total, cfg.n_q_heads, cfg.head_dim)[rows]
    check_relative(got, ref, "%s forward, %s" % (case, rep))


@pytest.mark.parametrize("factor", [1e5, 1e-6])
def test_chunk_attend_blend_value_range(hsa, factor):
    """hsa_chunk_attend_blend on the chunk-major path with the oracle's selection."""
    import torch
    cfg = W.shrink(W.CONFIGS[2], q_len=2048, kv_len=2048)
    inp = scaled_v(W.generate(cfg), factor)
    oi, os_, _, _ = oracle.forward(inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v,
                                   q_pos0=cfg.q_pos0, top_k=cfg.top_k, with_output=False)
    total = cfg.batch * cfg.q_len
    rows = sample(total, 256, seed=7)
    _, ref = oracle.attend_blend(inp.q_attn, inp.k, inp.v, oi[rows], os_[rows], rows=rows)
    qa, k, v = (to_device(a, cfg.dtype) for a in (inp.q_attn, inp.k, inp.v))
    shp = (cfg.batch, cfg.q_len, cfg.n_kv_heads, cfg.top_k)
    ti = torch.from_numpy(oi.reshape(shp).astype(np.int32)).cuda()
    ts = torch.from_numpy(os_.reshape(shp).astype(np.float32)).cuda()
    out = hsa.chunk_attend_blend(qa, k, v, ti, ts)
    torch.cuda.synchronize()
    got = out_to_f64(out).reshape(total, cfg.n_q_heads, cfg.head_dim)[rows]
    check_relative(got, ref, "chunk_attend_blend V x %g" % factor)


@pytest.mark.parametrize("factor", [1e5, 1e-6])
def test_global_value_range(hsa, factor):
    import torch
    cfg = HsaConfig(name="global_range", batch=1, q_len=1024, q_pos0=0, kv_len=1024, n_q_heads=8,
                    n_kv_heads=1, head_dim=128, top_k=8, dtype="bf16", noise_std=0.5, n_needles=4,
                    seed=51)
    inp = scaled_v(W.generate(cfg), factor)
    dev = inputs_to_device(inp)
    out = hsa.forward(*dev, q_pos0=0, top_k=100)
    torch.cuda.synchronize()
    rows = sample(cfg.q_len, 200, seed=3)
    _, _, _, ref = oracle.forward(inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v, q_pos0=0,
                                  top_k=100, rows=rows)
    got = out_to_f64(out).reshape(cfg.q_len, cfg.n_q_heads, cfg.head_dim)[rows]
    check_relative(got, ref, "global V x %g" % factor)


# ----------------------------------------------------------------------------
# two streams at once
# ----------------------------------------------------------------------------

def _decode_case(seed, kv_len, top_k):
    cfg = replace(W.shrink(W.CONFIGS[3], kv_len=kv_len), top_k=top_k, seed=seed)
    return cfg, inputs_to_device(W.generate(cfg))


def test_two_streams_at_once_match_single_stream(hsa):
    """Two different decode-shaped forwards (arrival-counter hand-offs in the
    attend) and a chunk-major prefill, enqueued alternately on two streams many
    times, give the single-stream outputs bit for bit."""
    import torch
    cases = [_decode_case(1301, 1 << 19, 32), _decode_case(1302, 3 << 17, 20)]
    pcfg = W.shrink(W.CONFIGS[1], q_len=2048, kv_len=2048)
    cases.append((pcfg, inputs_to_device(W.generate(pcfg))))

    def run(i):
        cfg, dev = cases[i]
        return hsa.forward(*dev, q_pos0=cfg.q_pos0, top_k=cfg.top_k)

    refs = [run(i).clone() for i in range(len(cases))]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = []
    for it in range(12):
        for j, s in enumerate(streams):
            i = (it + j) % len(cases)
            with torch.cuda.stream(s):
                got.append((i, run(i)))
    torch.cuda.synchronize()
    for i, o in got:
        assert torch.equal(o, refs[i]), ("stream result differs", i)
    # each stream had its own workspace
    keys = {k for k in hsa._ws_cache if k[1] in {s.cuda_stream for s in streams}}
    assert len(keys) == 2
