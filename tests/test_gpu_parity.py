"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Tolerances: selected chunk sets bit-exact (with the fp32 error-band rule for
continuous scores, exact order and scores in grid mode); output max-abs error
<= 1e-5 for fp32 inputs and <= 2e-2 for bf16 inputs (fp32 accumulation).
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import workloads as W
from workloads import HsaConfig

from hsa_check import check_output, check_selection, inputs_to_device, out_to_f64, to_device

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


@pytest.fixture(scope="module")
def hsa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ultra_long_context_amd as h
    h.load_library()
    return h


def sample_rows(cfg, n, seed=0):
    total = cfg.batch * cfg.q_len
    if total <= n:
        return np.arange(total)
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(total, size=n - 4, replace=False).tolist())
    rows |= {0, total - 1, cfg.q_len - 1, min(total - 1, 64)}
    return np.array(sorted(rows))


def run_forward(hsa, inp, **kw):
    import torch
    cfg = inp.cfg
    dev = inputs_to_device(inp)
    print("case %s B=%d Lq=%d Lkv=%d Hq=%d Hkv=%d d=%d K=%d %s" % (
        cfg.name, cfg.batch, cfg.q_len, cfg.kv_len, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
        cfg.top_k, cfg.dtype), flush=True)
    out, idx, score = hsa.forward(*dev, q_pos0=cfg.q_pos0, top_k=cfg.top_k, qk_norm=cfg.qk_norm,
                                  return_topk=True, **kw)
    torch.cuda.synchronize()
    return out, idx, score


def parity(hsa, inp, rows=None, exact=False, ret_scale=None, attn_scale=None):
    cfg = inp.cfg
    out, idx, score = run_forward(hsa, inp, ret_scale=ret_scale, attn_scale=attn_scale)
    rows = np.arange(cfg.batch * cfg.q_len) if rows is None else np.asarray(rows)
    oi, os_, _, oo = oracle.forward(inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v,
                                    q_pos0=cfg.q_pos0, top_k=cfg.top_k, qk_norm=cfg.qk_norm,
                                    ret_scale=ret_scale, attn_scale=attn_scale, rows=rows)
    B, Lq = cfg.batch, cfg.q_len
    gi = idx.cpu().numpy().reshape(B * Lq, cfg.n_kv_heads, cfg.top_k)[rows]
    gs = score.cpu().numpy().reshape(B * Lq, cfg.n_kv_heads, cfg.top_k)[rows]
    go = out_to_f64(out).reshape(B * Lq, cfg.n_q_heads, cfg.head_dim)[rows]
    rs = oracle.default_scale(cfg.head_dim) if ret_scale is None else ret_scale
    rep = check_selection(inp, rows, gi, gs, oi, os_, ret_scale=rs, exact=exact)
    err = check_output(inp, rows, go, oo, atol=TOL[cfg.dtype], rep=rep, gpu_idx=gi,
                       qk_norm=cfg.qk_norm, attn_scale=attn_scale, ret_scale=ret_scale)
    print("  %s  max-abs err %.3e" % (rep, err), flush=True)
    return rep, err, (out, idx, score)


def small(**kw):
    base = dict(name="small", batch=1, q_len=1024, q_pos0=0, kv_len=1024, n_q_heads=8, n_kv_heads=1,
                head_dim=128, top_k=8, dtype="bf16", noise_std=0.5, n_needles=4, seed=31)
    base.update(kw)
    return HsaConfig(**base)


# ----------------------------------------------------------------------------
# workload-shaped cases at oracle-friendly sizes
# ----------------------------------------------------------------------------

def test_tiny_fp32_full(hsa):
    parity(hsa, W.generate(W.CONFIGS[0]))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_tiny_fp32_seeds(hsa, seed):
    parity(hsa, W.generate(W.CONFIGS[0], seed=seed))


def test_tiny_grid_exact(hsa):
    parity(hsa, W.generate(W.CONFIGS[0], mode="grid"), exact=True, ret_scale=0.125)


def test_prefill_32k_shape_cut_to_4k(hsa):
    cfg = W.shrink(W.CONFIGS[1], q_len=4096, kv_len=4096)
    parity(hsa, W.generate(cfg))


def test_prefill_grid_small_ties_exact(hsa):
    cfg = W.shrink(W.CONFIGS[1], q_len=2048, kv_len=2048, top_k=16)
    parity(hsa, W.generate(cfg, mode="grid_small"), exact=True, ret_scale=0.125)


def test_prefill_128k_shape_cut(hsa):
    cfg = W.shrink(W.CONFIGS[2], q_len=2048, kv_len=2048)
    inp = W.generate(cfg)
    parity(hsa, inp, rows=sample_rows(cfg, 700))


def test_decode_shape_split_merge(hsa):
    """Few rows over a long history: the scan splits the chunks and merges."""
    cfg = W.shrink(W.CONFIGS[3], kv_len=1 << 20)
    parity(hsa, W.generate(cfg))


def test_split_merge_one_list_holds_the_top_k(hsa):
    """All scores tie (q_ret = 0): the first 32 chunks win, all from the first
    split's list, so the merge must read that list past its first entries."""
    cfg = W.shrink(W.CONFIGS[3], kv_len=1 << 20)
    inp = W.generate(cfg)
    inp.q_ret[:] = 0
    _, _, (_, idx, _) = parity(hsa, inp)
    assert np.all(idx.cpu().numpy() == np.arange(cfg.top_k))


def test_split_merge_clustered_winners(hsa):
    """Every row shares one retrieval query and 20 boosted chunks inside one
    1024-chunk split: that split's list contributes 20 of the 32 winners."""
    cfg = W.shrink(W.CONFIGS[3], kv_len=1 << 20)
    inp = W.generate(cfg)
    q = W.to_f64(inp.q_ret[0, 0], cfg.dtype)                     # [Hkv, d]
    inp.q_ret[:] = inp.q_ret[0:1, 0:1]
    lm = W.to_f64(inp.landmarks, cfg.dtype)
    u = q / np.linalg.norm(q, axis=-1, keepdims=True)
    lm[0, :, 2048:2068, :] += 6.0 * cfg.sigma_l * u[:, None, :]
    inp.landmarks[:] = W.store(lm, cfg.dtype)
    _, _, (_, idx, _) = parity(hsa, inp)
    sel = idx.cpu().numpy()
    assert np.all(((sel >= 2048) & (sel < 2068)).sum(-1) == 20)


@pytest.mark.parametrize("K", [3, 4, 5])
def test_split_merge_small_top_k(hsa, K):
    """K at and around the merge's first-entries depth."""
    cfg = W.shrink(W.CONFIGS[3], kv_len=1 << 20, top_k=K)
    parity(hsa, W.generate(cfg))


def test_split_merge_retrieve_entry(hsa):
    """The standalone merge kernel (hsa_retrieve_topk with several splits)."""
    import torch
    cfg = W.shrink(W.CONFIGS[3], kv_len=1 << 20)
    inp = W.generate(cfg)
    inp.q_ret[:, ::2] = 0
    q_ret, lm = (to_device(a, cfg.dtype) for a in (inp.q_ret, inp.landmarks))
    idx, score = hsa.retrieve_topk(q_ret, lm, q_pos0=cfg.q_pos0, top_k=cfg.top_k)
    torch.cuda.synchronize()
    rows = np.arange(cfg.q_len)
    oi, os_, _, _ = oracle.forward(inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v, q_pos0=cfg.q_pos0,
                                   top_k=cfg.top_k, with_output=False)
    gi = idx.cpu().numpy().reshape(cfg.q_len, cfg.n_kv_heads, cfg.top_k)
    gs = score.cpu().numpy().reshape(cfg.q_len, cfg.n_kv_heads, cfg.top_k)
    rs = oracle.default_scale(cfg.head_dim)
    check_selection(inp, rows, gi, gs, oi, os_, ret_scale=rs)
    assert np.all(gi[::2] == np.arange(cfg.top_k))


def test_chunked_prefill_shape_cut(hsa):
    cfg = W.shrink(W.CONFIGS[4], q_len=512, kv_len=65536 + 512)
    inp = W.generate(cfg)
    parity(hsa, inp, rows=sample_rows(cfg, 300))


@pytest.mark.parametrize("Hkv,Nc", [(1, 2047), (1, 2049), (2, 1025)])
def test_bin_scan_tile_edges(hsa, Hkv, Nc):
    """The many-row path's bin offsets and work items come from a scan over
    tiles of 2,048 (batch, kv head, band, chunk) bins: bin counts just below and
    past a tile, and a tile that holds the end of one kv head's bins and the
    start of the next."""
    L = Nc * 64
    cfg = small(q_len=1024, kv_len=L, q_pos0=L - 1024, n_q_heads=8 * Hkv, n_kv_heads=Hkv)
    inp = W.generate(cfg)
    parity(hsa, inp, rows=sample_rows(cfg, 300))


# ----------------------------------------------------------------------------
# edge cases
# ----------------------------------------------------------------------------

def test_softmax_exercised_without_qk_norm(hsa):
    cfg = small(qk_norm=False, q_len=512, kv_len=512)
    parity(hsa, W.generate(cfg), attn_scale=0.2)


def test_sharp_softmax_with_qk_norm(hsa):
    parity(hsa, W.generate(small(q_len=512, kv_len=512)), attn_scale=8.0)


@pytest.mark.parametrize("K", [1, 5, 64])
def test_top_k_extremes(hsa, K):
    parity(hsa, W.generate(small(top_k=K, q_len=1024, kv_len=1024 * 5, q_pos0=1024 * 4)))


@pytest.mark.parametrize("G,Hkv", [(1, 2), (2, 2), (4, 1), (16, 1)])
def test_group_sizes(hsa, G, Hkv):
    parity(hsa, W.generate(small(n_q_heads=G * Hkv, n_kv_heads=Hkv, batch=2, q_len=256, kv_len=256)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_head_dim_64(hsa, dtype):
    parity(hsa, W.generate(small(head_dim=64, dtype=dtype, q_len=512, kv_len=512)))


def test_head_dim_128_fp32(hsa):
    parity(hsa, W.generate(small(dtype="f32", q_len=512, kv_len=512)))


def test_ragged_history_and_rows(hsa):
    """Lkv % 64 != 0 (partial last chunk never eligible), Lq % 16 != 0."""
    cfg = small(q_len=77, kv_len=1000 + 37, q_pos0=1000 + 37 - 77 + 10)
    cfg = replace(cfg, q_pos0=min(cfg.q_pos0, (cfg.kv_len // 64) * 64 + 63 - 76))
    parity(hsa, W.generate(cfg))


def test_rows_without_chunks_output_zero(hsa):
    cfg = small(q_len=100, kv_len=100)
    _, _, (out, idx, _) = parity(hsa, W.generate(cfg))
    o = out_to_f64(out)
    assert np.all(o[0, :64] == 0.0)
    assert np.all(idx.cpu().numpy()[0, :64] == -1)


def test_uniform_scores_select_first_chunks(hsa):
    cfg = small(q_len=256, kv_len=4096, q_pos0=3840, top_k=7)
    inp = W.generate(cfg)
    inp.q_ret[:] = 0
    _, _, (_, idx, _) = parity(hsa, inp, exact=False)
    assert np.all(idx.cpu().numpy()[..., :] == np.arange(7))


def test_negative_zero_ties(hsa):
    cfg = small(q_len=64, kv_len=1024, q_pos0=960, top_k=6, dtype="f32")
    inp = W.generate(cfg)
    inp.q_ret[:] = 0.0
    inp.landmarks[:, :, ::2] = -np.abs(inp.landmarks[:, :, ::2]) - 1
    _, _, (_, idx, score) = parity(hsa, inp)
    assert np.all(idx.cpu().numpy() == np.arange(6))
    assert np.all(score.cpu().numpy() == 0.0)


def test_buffer_compaction_many_candidates(hsa):
    """K = 64 with few groups per lane forces the candidate buffer to be cut back."""
    cfg = small(q_len=64, kv_len=65536, q_pos0=65536 - 64, top_k=64)
    parity(hsa, W.generate(cfg, mode="grid_small"), exact=True, ret_scale=0.125)


def test_deterministic(hsa):
    import torch
    inp = W.generate(W.shrink(W.CONFIGS[3], kv_len=1 << 18))
    a = run_forward(hsa, inp)
    b = run_forward(hsa, inp)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("cfg_i,kw", [(3, dict(kv_len=1 << 18)), (1, dict(q_len=4096, kv_len=8192)),
                                      (2, dict(q_len=2048, kv_len=2048))])
def test_profiled_forward_matches_and_records_stages(hsa, cfg_i, kw):
    """hsa_forward_profiled gives the outputs of hsa_forward bit for bit and
    records an event pair around every stage its plan runs."""
    import torch
    cfg = W.shrink(W.CONFIGS[cfg_i], **kw)
    inp = W.generate(cfg)
    dev = inputs_to_device(inp)
    a = hsa.forward(*dev, q_pos0=cfg.q_pos0, top_k=cfg.top_k, return_topk=True)
    evs = {n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in hsa.STAGES}
    b = hsa.forward(*dev, q_pos0=cfg.q_pos0, top_k=cfg.top_k, return_topk=True, stage_events=evs)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert evs["scan"][0].elapsed_time(evs["scan"][1]) > 0
    assert evs["attend"][0].elapsed_time(evs["attend"][1]) > 0


# ----------------------------------------------------------------------------
# the two halves through their own entry points
# ----------------------------------------------------------------------------

def test_retrieve_topk_entry(hsa):
    cfg = W.shrink(W.CONFIGS[1], q_len=1024, kv_len=1024)
    inp = W.generate(cfg)
    q, lm = (to_device(a, cfg.dtype) for a in (inp.q_ret, inp.landmarks))
    idx, score = hsa.retrieve_topk(q, lm, q_pos0=0, top_k=cfg.top_k)
    oi, os_, _, _ = oracle.forward(inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v, q_pos0=0,
                                   top_k=cfg.top_k, with_output=False)
    rows = np.arange(cfg.q_len)
    check_selection(inp, rows, idx.cpu().numpy().reshape(-1, 1, cfg.top_k),
                    score.cpu().numpy().reshape(-1, 1, cfg.top_k), oi, os_,
                    ret_scale=oracle.default_scale(128))


def test_chunk_attend_blend_entry_with_given_selection(hsa):
    """Oracle indices fed in, unsorted scores, unused (-1) and out-of-range slots."""
    cfg = small(q_len=300, kv_len=2048, q_pos0=1748, top_k=6, n_kv_heads=2, n_q_heads=8)
    inp = W.generate(cfg)
    oi, os_, _, _ = oracle.forward(inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v,
                                   q_pos0=cfg.q_pos0, top_k=cfg.top_k, with_output=False)
    rng = np.random.default_rng(5)
    perm = rng.permutation(cfg.top_k)
    sel = oi[:, :, perm].copy()
    sc = os_[:, :, perm].copy()
    sel[::7, :, 2] = -1
    sel[::11, 1, 0] = 10 ** 6          # outside [0, Nc): skipped
    sel[5] = -1                        # a row with nothing selected -> 0
    w, ref = oracle.attend_blend(inp.q_attn, inp.k, inp.v, sel, sc)
    qa, k, v = (to_device(a, cfg.dtype) for a in (inp.q_attn, inp.k, inp.v))
    import torch
    ti = torch.from_numpy(sel.reshape(1, cfg.q_len, 2, cfg.top_k)).cuda()
    ts = torch.from_numpy(sc.reshape(1, cfg.q_len, 2, cfg.top_k).astype(np.float32)).cuda()
    out = hsa.chunk_attend_blend(qa, k, v, ti, ts)
    got = out_to_f64(out).reshape(cfg.q_len, cfg.n_q_heads, cfg.head_dim)
    assert np.abs(got - ref).max() <= TOL["bf16"]
    assert np.all(got[5] == 0)


def test_many_row_blocks_one_wave_scan(hsa):
    """More than 2048 blocks of 16 rows in fp32: the one-wave-per-16-rows scan path."""
    cfg = small(batch=1, n_kv_heads=4, n_q_heads=8, q_len=8256, kv_len=8256, top_k=8, head_dim=64,
                dtype="f32")
    inp = W.generate(cfg)
    parity(hsa, inp, rows=sample_rows(cfg, 400))


@pytest.mark.parametrize("d,K", [(64, 8), (128, 32), (128, 1)])
def test_block_scan_many_rows(hsa, d, K):
    """More than 2048 blocks of 16 rows in bf16 with K <= 32: the block scan
    (64 rows per workgroup); ragged rows, history and first position, early
    rows with fewer than K (or no) eligible chunks."""
    cfg = small(batch=1, n_kv_heads=4, n_q_heads=8, q_len=8250, kv_len=8300, q_pos0=37, top_k=K,
                head_dim=d)
    inp = W.generate(cfg)
    rows = np.union1d(sample_rows(cfg, 300, seed=d + K), np.arange(0, 200, 7))
    parity(hsa, inp, rows=rows)


def test_block_scan_long_rows(hsa):
    """Block scan over ~2000 chunks per row: many LDS tiles and candidate cuts."""
    cfg = small(batch=1, n_kv_heads=1, n_q_heads=8, q_len=33000, q_pos0=98304, kv_len=131304,
                top_k=16, head_dim=128)
    inp = W.generate(cfg)
    parity(hsa, inp, rows=sample_rows(cfg, 200, seed=5))


def test_block_scan_ties_exact(hsa):
    """Block scan with K = 32 on integer-valued scores full of ties: exact order."""
    cfg = small(batch=2, n_kv_heads=2, n_q_heads=4, q_len=8256, kv_len=8256, top_k=32, head_dim=64)
    inp = W.generate(cfg, mode="grid_small")
    parity(hsa, inp, rows=sample_rows(cfg, 150), exact=True, ret_scale=0.125)


@pytest.mark.parametrize("mode,K", [("grid_small", 32), ("normal", 8)])
def test_block_scan_small_tiles(hsa, mode, K):
    """Block scan with at least 3072 workgroups: 32-chunk landmark tiles, three
    workgroups per CU (the 128K prefill launch).  Ragged rows and history;
    integer-valued scores full of ties compared exactly."""
    cfg = small(batch=1, n_kv_heads=8, n_q_heads=8, q_len=24600, q_pos0=45, kv_len=24700, top_k=K,
                head_dim=64)
    inp = W.generate(cfg, mode=mode)
    rows = np.union1d(sample_rows(cfg, 150, seed=K), np.arange(0, 130, 9))
    if mode == "grid_small":
        parity(hsa, inp, rows=rows, exact=True, ret_scale=0.125)
    else:
        parity(hsa, inp, rows=rows)


def _random_shapes(n, seed):
    """Seeded small shapes across the plan's branches: few rows (decode
    attend) and many (chunk-major), bf16 and fp32, G 1-16, d 64/128, K 1-64,
    ragged histories and first positions, qk_norm on and off."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = int(rng.choice([1, 2])) if G <= 8 else 1
        d = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["bf16", "bf16", "f32"]))
        q_len = int(rng.choice([1, 7, 16, 40, 300, 1100]))
        kv_len = max(int(rng.integers(64, 9000)), q_len)
        q_pos0 = int(rng.integers(0, (kv_len // 64 + 1) * 64 - q_len + 1))   # rows' chunks lie in the history
        K = int(rng.choice([1, 3, 8, 16, 32, 64]))
        out.append(dict(name="rand%d" % i, batch=int(rng.choice([1, 2])), q_len=q_len, q_pos0=q_pos0,
                        kv_len=kv_len, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=d, top_k=K, dtype=dtype,
                        qk_norm=bool(rng.integers(0, 2)), n_needles=2, seed=100 + i))
    return out


@pytest.mark.parametrize("kw", _random_shapes(12, seed=2024), ids=lambda kw: kw["name"])
def test_random_shapes(hsa, kw):
    cfg = small(**kw)
    assert (cfg.q_pos0 + cfg.q_len - 1) // 64 <= cfg.kv_len // 64
    parity(hsa, W.generate(cfg), rows=sample_rows(cfg, 120, seed=cfg.seed))


def _random_long_shapes(n, seed):
    """Seeded few-row shapes over histories of more than 1024 chunks, so the
    wide scan splits the chunks and the per-split lists are merged: bf16
    (decode attend, merge in its prologue) and fp32 (merge kernel, then the
    per-row attend), G 1-16, d 64/128, K 1-64, rows short of their chunk end."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = int(rng.choice([1, 2])) if G <= 4 else 1
        q_len = int(rng.choice([1, 5, 16, 33]))
        kv_len = int(rng.integers(65600, 300000))
        q_pos0 = max(0, kv_len - q_len - int(rng.integers(0, 5000)))
        out.append(dict(name="long%d" % i, batch=int(rng.choice([1, 2])), q_len=q_len, q_pos0=q_pos0,
                        kv_len=kv_len, n_q_heads=G * Hkv, n_kv_heads=Hkv,
                        head_dim=int(rng.choice([64, 128])), top_k=int(rng.choice([1, 7, 32, 64])),
                        dtype=str(rng.choice(["bf16", "f32"])), qk_norm=bool(rng.integers(0, 2)),
                        n_needles=3, seed=200 + i))
    return out


@pytest.mark.parametrize("kw", _random_long_shapes(8, seed=77), ids=lambda kw: kw["name"])
def test_random_long_histories(hsa, kw):
    cfg = small(**kw)
    assert cfg.kv_len // 64 > 1024 and (cfg.q_pos0 + cfg.q_len - 1) // 64 <= cfg.kv_len // 64
    parity(hsa, W.generate(cfg))


# ----------------------------------------------------------------------------
# full workload sizes, in the launch configuration bench.py times; the oracle
# checks sampled rows (all 16 rows for the decode workload)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("i,n_rows", [(1, 300), (2, 120), (3, 16), (4, 120)])
def test_full_size_workloads_sampled(hsa, i, n_rows):
    cfg = W.CONFIGS[i]
    inp = W.generate(cfg)
    parity(hsa, inp, rows=sample_rows(cfg, n_rows, seed=i))


def test_decode_16M_largest_top_k_and_group(hsa):
    """The 16M-token decode history at the largest top-K (64) with 16 query
    heads per kv head: 256 split lists of 64 entries per row, all 16 rows
    checked."""
    cfg = W.config(3, top_k=64, n_q_heads=16)
    parity(hsa, W.generate(cfg))


def test_one_wave_scan_buffer_compaction(hsa):
    """One-wave scan path with K = 64 and heavy ties: the LDS buffer is cut back."""
    cfg = small(batch=2, n_kv_heads=2, n_q_heads=4, q_len=8256, kv_len=8256, top_k=64, head_dim=64)
    inp = W.generate(cfg, mode="grid_small")
    parity(hsa, inp, rows=sample_rows(cfg, 150), exact=True, ret_scale=0.125)


@pytest.mark.parametrize("G,d", [(1, 128), (4, 64), (16, 128)])
def test_chunk_major_attend_group_sizes(hsa, G, d):
    """Many rows in bf16: pairs bucketed by chunk, MFMA tiles of 16/G pairs."""
    cfg = small(n_q_heads=G, n_kv_heads=1, head_dim=d, q_len=1024, kv_len=4096, q_pos0=3072, top_k=8)
    parity(hsa, W.generate(cfg), rows=sample_rows(cfg, 400))


def test_chunk_major_global_histogram_bucketing(hsa):
    """More than 16,384 chunks per kv head (past the LDS histogram): pairs are
    counted into their bins with global atomics whose return values place them,
    and the scatter adds each pair's rank to its bin's first slot.  Ragged
    rows and history, two kv heads, needles for popular bins."""
    cfg = small(batch=1, n_kv_heads=2, n_q_heads=16, q_len=1500, q_pos0=1048700, kv_len=1048700 + 1500 + 37,
                top_k=16, n_needles=32)
    parity(hsa, W.generate(cfg), rows=sample_rows(cfg, 300, seed=11))


def test_chunk_major_given_selection_with_gaps(hsa):
    """hsa_chunk_attend_blend in the chunk-major mode with -1 and out-of-range slots."""
    import torch
    cfg = small(q_len=1100, kv_len=4096, q_pos0=2996, top_k=6, n_kv_heads=2, n_q_heads=16)
    inp = W.generate(cfg)
    oi, os_, _, _ = oracle.forward(inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v,
                                   q_pos0=cfg.q_pos0, top_k=cfg.top_k, with_output=False)
    sel, sc = oi.copy(), os_.copy()
    sel[::5, :, 1] = -1
    sel[::13, 0, 3] = 10 ** 6
    sel[7] = -1
    rows = sample_rows(cfg, 300)
    _, ref = oracle.attend_blend(inp.q_attn, inp.k, inp.v, sel[rows], sc[rows], rows=rows)
    qa, k, v = (to_device(a, cfg.dtype) for a in (inp.q_attn, inp.k, inp.v))
    ti = torch.from_numpy(sel.reshape(1, cfg.q_len, 2, cfg.top_k)).cuda()
    ts = torch.from_numpy(sc.reshape(1, cfg.q_len, 2, cfg.top_k).astype(np.float32)).cuda()
    out = hsa.chunk_attend_blend(qa, k, v, ti, ts)
    got = out_to_f64(out).reshape(cfg.q_len, cfg.n_q_heads, cfg.head_dim)
    assert np.abs(got[rows] - ref).max() <= TOL["bf16"]
    assert np.all(got[7] == 0)


# ----------------------------------------------------------------------------
# chunk-mean landmarks (the Step 1 stand-in; KV-cache maintenance)
# ----------------------------------------------------------------------------

def _landmark_err(got_t, ref64, dtype):
    got = out_to_f64(got_t)
    return np.abs(got - ref64).max() if ref64.size else 0.0


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_chunk_landmarks_parity(hsa, dtype, d):
    """All complete chunks of a ragged history (trailing partial chunk ignored),
    then a sub-range written into an existing buffer (the rest untouched)."""
    import torch
    cfg = small(batch=2, n_kv_heads=3, n_q_heads=3, q_len=64, kv_len=64 * 37 + 21, head_dim=d, dtype=dtype)
    inp = W.generate(cfg)
    k = to_device(inp.k, dtype)
    ref = oracle.chunk_landmarks(inp.k)
    got = hsa.chunk_landmarks(k)
    torch.cuda.synchronize()
    tol = TOL[dtype] if dtype == "f32" else 2.0 ** -8 * max(1.0, np.abs(ref).max())
    assert _landmark_err(got, ref, dtype) <= tol
    sentinel = torch.full_like(got, 7.0)
    hsa.chunk_landmarks(k, chunk_begin=5, chunk_end=19, out=sentinel)
    torch.cuda.synchronize()
    s64 = out_to_f64(sentinel)
    assert np.all(s64[:, :, :5] == 7.0) and np.all(s64[:, :, 19:] == 7.0)
    assert np.abs(s64[:, :, 5:19] - ref[:, :, 5:19]).max() <= tol


def test_chunk_landmarks_decode_history_sampled(hsa):
    """The 16M-token decode history: every landmark rebuilt on the GPU, sampled
    chunks checked against the oracle."""
    import torch
    cfg = W.CONFIGS[3]
    inp = W.generate(cfg)
    k = to_device(inp.k, cfg.dtype)
    got = out_to_f64(hsa.chunk_landmarks(k))
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    cs = np.unique(np.concatenate([rng.choice(cfg.n_chunks, 60, replace=False), [0, cfg.n_chunks - 1]]))
    for c in cs:
        ref = oracle.chunk_landmarks(inp.k[:, :, 64 * c:64 * c + 64])
        assert np.abs(got[:, :, c:c + 1] - ref).max() <= 2.0 ** -8 * max(1.0, np.abs(ref).max())


def test_decode_with_incremental_append(hsa):
    """Decode steps over a growing history: each step appends 16 tokens, the
    chunks the append completes get their landmarks (hsa_chunk_landmarks), and
    the 16 new tokens query the history (hsa_forward).  Checked against the
    oracle on the same landmarks."""
    import torch
    L0, steps, T = 64 * 40 + 24, 5, 16
    cfg = small(batch=1, n_kv_heads=1, n_q_heads=8, q_len=T, kv_len=L0 + steps * T, top_k=8, head_dim=128)
    inp = W.generate(cfg)
    k_all, v_all = to_device(inp.k, "bf16"), to_device(inp.v, "bf16")
    lm = torch.zeros((1, 1, cfg.kv_len // 64, 128), dtype=torch.bfloat16, device="cuda:0")
    hsa.chunk_landmarks(k_all[:, :, :L0], out=lm[:, :, :L0 // 64])
    rng = np.random.default_rng(11)
    for s in range(steps):
        L = L0 + (s + 1) * T                         # history after this step's append
        nc_old, nc = (L - T) // 64, L // 64
        k, v = k_all[:, :, :L].contiguous(), v_all[:, :, :L].contiguous()
        if nc > nc_old:
            view = lm[:, :, :nc].contiguous()
            hsa.chunk_landmarks(k, chunk_begin=nc_old, chunk_end=nc, out=view)
            lm[:, :, :nc] = view
        q_ret = to_device(W.store(rng.standard_normal((1, T, 1, 128)), "bf16"), "bf16")
        q_attn = to_device(W.store(rng.standard_normal((1, T, 8, 128)), "bf16"), "bf16")
        lmk = lm[:, :, :nc].contiguous()
        out, idx, score = hsa.forward(q_ret, lmk, q_attn, k, v, q_pos0=L - T, top_k=8, return_topk=True)
        torch.cuda.synchronize()
        bits = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)
        ref_lm = oracle.chunk_landmarks(inp.k[:, :, :L])
        got_lm = out_to_f64(lmk)
        assert np.abs(got_lm - ref_lm).max() <= 2.0 ** -8 * max(1.0, np.abs(ref_lm).max())
        oi, os_, _, oo = oracle.forward(bits(q_ret), bits(lmk), bits(q_attn), bits(k), bits(v),
                                        q_pos0=L - T, top_k=8)
        sub = replace(cfg, q_len=T, kv_len=L, q_pos0=L - T)
        step_inp = W.HsaInputs(sub, bits(q_ret), bits(lmk), bits(q_attn), bits(k), bits(v), [])
        rows = np.arange(T)
        gi = idx.cpu().numpy().reshape(T, 1, 8)
        gs = score.cpu().numpy().reshape(T, 1, 8)
        rep = check_selection(step_inp, rows, gi, gs, oi, os_, ret_scale=oracle.default_scale(128))
        err = check_output(step_inp, rows, out_to_f64(out).reshape(T, 8, 128), oo, atol=TOL["bf16"],
                           rep=rep, gpu_idx=gi, qk_norm=True, attn_scale=None, ret_scale=None)
        assert err <= TOL["bf16"]


# ----------------------------------------------------------------------------
# global HSA: a top-K that covers every eligible chunk (warm-up stage)
# ----------------------------------------------------------------------------

def global_parity(hsa, inp, K, rows=None):
    import torch
    cfg = inp.cfg
    dev = inputs_to_device(inp)
    print("case global %s B=%d Lq=%d q_pos0=%d Lkv=%d Hq=%d Hkv=%d d=%d K=%d" % (
        cfg.name, cfg.batch, cfg.q_len, cfg.q_pos0, cfg.kv_len, cfg.n_q_heads, cfg.n_kv_heads,
        cfg.head_dim, K), flush=True)
    out = hsa.forward(*dev, q_pos0=cfg.q_pos0, top_k=K, qk_norm=cfg.qk_norm)
    torch.cuda.synchronize()
    total = cfg.batch * cfg.q_len
    rows = np.arange(total) if rows is None else np.asarray(rows)
    _, _, _, oo = oracle.forward(inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v, q_pos0=cfg.q_pos0,
                                 top_k=K, qk_norm=cfg.qk_norm, rows=rows)
    got = out_to_f64(out).reshape(total, cfg.n_q_heads, cfg.head_dim)[rows]
    err = np.abs(got - oo).max()
    print("  max-abs err %.3e" % err, flush=True)
    assert err <= TOL["bf16"]
    return out


@pytest.mark.parametrize("G,d", [(8, 128), (16, 128), (8, 64), (16, 64), (1, 128), (2, 128), (4, 128),
                                 (1, 64), (2, 64), (4, 64)])
def test_global_hsa_prefill(hsa, G, d):
    """Every eligible chunk selected (K > 64): dense in-chunk attention blended
    by the softmax of all retrieval scores; early rows have no chunk (zero)."""
    cfg = small(n_q_heads=G, n_kv_heads=1, head_dim=d, q_len=3000, kv_len=3000, top_k=8, seed=41 + G + d)
    global_parity(hsa, W.generate(cfg), K=4096, rows=sample_rows(cfg, 300, seed=G))


def test_global_hsa_appended_rows_and_batch(hsa):
    """Appended rows (q_pos0 not chunk-aligned), two sequences, two kv heads."""
    cfg = small(batch=2, n_kv_heads=2, n_q_heads=16, head_dim=128, q_len=700, q_pos0=2083, kv_len=2816,
                top_k=8, seed=43)
    global_parity(hsa, W.generate(cfg), K=65, rows=sample_rows(cfg, 300, seed=3))


@pytest.mark.parametrize("G,Hkv", [(1, 4), (2, 2), (4, 2)])
def test_global_hsa_small_groups_appended_rows(hsa, G, Hkv):
    """G = 1, 2, 4 (256, 128, 64 rows per workgroup): appended rows over a longer
    history, several kv heads, two sequences."""
    cfg = small(batch=2, n_kv_heads=Hkv, n_q_heads=G * Hkv, head_dim=128, q_len=600, q_pos0=2500,
                kv_len=3100, top_k=8, seed=60 + G)
    global_parity(hsa, W.generate(cfg), K=100, rows=sample_rows(cfg, 240, seed=G))


@pytest.mark.parametrize("d", [128, 64])
def test_global_hsa_without_qk_norm(hsa, d):
    """Without query-key normalisation the global kernel stages the keys as
    given (no normalisation pass) and subtracts each chunk's maximum logit
    (the logits are then unbounded); appended rows, two kv heads."""
    cfg = small(n_q_heads=8, n_kv_heads=2, head_dim=d, q_len=1500, q_pos0=500, kv_len=2000, top_k=8,
                qk_norm=False, seed=70 + d)
    global_parity(hsa, W.generate(cfg), K=100, rows=sample_rows(cfg, 240, seed=d))


def test_global_hsa_uniform_scores_equal_chunk_mean(hsa):
    """q_ret = 0: every score equal, so the output is the mean of the per-chunk
    attentions (the pages' K >= #chunks invariant), through the dense path."""
    cfg = small(n_q_heads=8, n_kv_heads=1, head_dim=128, q_len=512, kv_len=2048, q_pos0=1536, top_k=8,
                seed=44)
    inp = W.generate(cfg)
    inp = replace(inp, q_ret=np.zeros_like(inp.q_ret))
    global_parity(hsa, inp, K=100)


def test_global_hsa_matches_sparse_path_when_k_covers(hsa):
    """With <= 64 eligible chunks the sparse path at K = 64 selects them all:
    both paths agree (each within the tolerance of the oracle)."""
    import torch
    cfg = small(n_q_heads=8, n_kv_heads=1, head_dim=128, q_len=1024, kv_len=4096, q_pos0=3072, top_k=64,
                seed=45)
    inp = W.generate(cfg)
    dev = inputs_to_device(inp)
    a = out_to_f64(hsa.forward(*dev, q_pos0=cfg.q_pos0, top_k=64))
    b = out_to_f64(global_parity(hsa, inp, K=65))
    assert np.abs(a - b).max() <= TOL["bf16"]
