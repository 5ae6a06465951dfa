"""Pins of the fp64 oracle against facts fixed by the paper's definition and by
mathematics, independent of the oracle's own code.

Definition pinned: "Every Token Counts: Generalizing 16M Ultra-Long Context in
LLMs" (agent-atlas explainer), "How It Works (Technically)" Steps 1-4 and the
hsa_step sketch under "The algorithm, simplified".

Each test names the plausible oracle mistake it would catch.  Library routines
used as independent references: torch scaled_dot_product_attention (fp64, CPU),
Python's stable sorted(), exact integer arithmetic.
"""
import math
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads import HsaConfig

torch.set_default_dtype(torch.float64)


def small_cfg(**kw):
    base = dict(name="t", batch=1, q_len=512, q_pos0=0, kv_len=512, n_q_heads=2, n_kv_heads=1,
                head_dim=64, top_k=3, dtype="f32", seed=7)
    base.update(kw)
    return HsaConfig(**base)


def run(inp, cfg=None, rows=None, **kw):
    cfg = cfg or inp.cfg
    args = dict(q_pos0=cfg.q_pos0, top_k=cfg.top_k, qk_norm=cfg.qk_norm)
    args.update(kw)
    return oracle.forward(inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v, rows=rows, **args)


def f64(a, dtype):
    return W.to_f64(a, dtype)


def sdpa_chunk(q, k, v, scale, qk_norm=True):
    """torch SDPA of one query row over one chunk's keys/values (fp64)."""
    q = torch.tensor(q)[None, None, None, :]
    k = torch.tensor(k)[None, None]
    v = torch.tensor(v)[None, None]
    if qk_norm:
        q = torch.nn.functional.normalize(q, dim=-1, eps=1e-6)
        k = torch.nn.functional.normalize(k, dim=-1, eps=1e-6)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
    return o[0, 0, 0].numpy()


# ----------------------------------------------------------------------------
# Selection (Step 2 + the stable descending sort of the hsa_step sketch)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["normal", "grid_small", "grid"])
def test_topk_equals_bruteforce_stable_sort(mode):
    """Catches: wrong causal bound, wrong tie rule, wrong operand row/head."""
    cfg = replace(W.CONFIGS[0], top_k=5)
    inp = W.generate(cfg, seed=11, mode=mode)
    rows = np.arange(0, cfg.q_len, 7)
    idx, score, _, _ = run(inp, rows=rows, with_output=False)
    q = f64(inp.q_ret, cfg.dtype)
    lm = f64(inp.landmarks, cfg.dtype)
    for i, r in enumerate(rows):
        n = min((cfg.q_pos0 + r) // 64, cfg.n_chunks)          # chunks fully before p's chunk
        s = [float(np.dot(q[0, r, 0], lm[0, 0, c])) for c in range(n)]
        sel = sorted(range(n), key=lambda c: s[c], reverse=True)[:cfg.top_k]   # stable
        k_eff = min(cfg.top_k, n)
        assert list(idx[i, 0, :k_eff]) == sel
        assert all(idx[i, 0, k_eff:] == -1)
        assert all(np.isneginf(score[i, 0, k_eff:]))


def test_grid_scores_exact_integers():
    """Grid entries are k/8: raw*64 is an exact integer sum.  Catches a dropped or
    wrong-index term in the dot product and a wrong ret_scale."""
    cfg = small_cfg(dtype="bf16", head_dim=128, top_k=8, n_kv_heads=2, n_q_heads=4, batch=2)
    inp = W.generate(cfg, seed=3, mode="grid")
    qi = np.rint(f64(inp.q_ret, "bf16") * 8).astype(np.int64)
    li = np.rint(f64(inp.landmarks, "bf16") * 8).astype(np.int64)
    rs = 0.3
    rows = np.array([64 * 3, 200, 511, 512 + 300, 1023])
    idx, score, _, _ = run(inp, rows=rows, ret_scale=rs, with_output=False)
    for i, fr in enumerate(rows):
        b, r = divmod(int(fr), cfg.q_len)
        n = r // 64
        for g in range(2):
            ints = [int(np.dot(qi[b, r, g], li[b, g, c])) for c in range(n)]
            order = sorted(range(n), key=lambda c: (-ints[c], c))[:cfg.top_k]
            assert list(idx[i, g, :len(order)]) == order
            for k, c in enumerate(order):
                assert score[i, g, k] == (ints[c] / 64.0) * rs


def test_ties_go_to_lower_index_and_signed_zero():
    """q_ret = 0: every raw score is +-0 and all tie; a landmark row that is all
    negative yields -0.0.  The first K eligible chunks must win, in index order."""
    cfg = small_cfg(top_k=4)
    inp = W.generate(cfg, seed=5)
    inp.q_ret[:] = 0.0
    inp.landmarks[0, 0, 1] = -np.abs(inp.landmarks[0, 0, 1]) - 1.0
    rows = np.array([64 * 6 + 5, 511])
    idx, score, _, _ = run(inp, rows=rows, with_output=False)
    for i in range(2):
        assert list(idx[i, 0]) == [0, 1, 2, 3]
        assert np.all(score[i, 0] == 0.0)


def test_positive_rescaling_of_query_keeps_sets():
    cfg = small_cfg(top_k=6)
    inp = W.generate(cfg, seed=9)
    idx1, s1, _, _ = run(inp, with_output=False)
    inp2 = replace(inp, q_ret=(inp.q_ret * np.float32(2.0)).astype(np.float32))
    idx2, s2, _, _ = run(inp2, with_output=False)
    assert np.array_equal(idx1, idx2)
    np.testing.assert_array_equal(s2[idx2 >= 0], 2 * s1[idx1 >= 0])


def test_rows_without_eligible_chunk_are_empty():
    """Rows in the first chunk see nothing: all slots -1/-inf and output 0 (empty sum)."""
    cfg = small_cfg()
    inp = W.generate(cfg, seed=1)
    rows = np.array([0, 1, 63])
    idx, score, w, out = run(inp, rows=rows)
    assert np.all(idx == -1) and np.all(np.isneginf(score)) and np.all(w == 0)
    assert np.all(out == 0.0)


def test_partial_trailing_chunk_is_never_selected():
    cfg = small_cfg(kv_len=512 + 40, q_len=8, q_pos0=600, top_k=16)
    inp = W.generate(cfg, seed=2)
    idx, _, _, _ = run(inp, with_output=False)
    assert idx.max() == cfg.n_chunks - 1 == 7
    assert np.all(np.sort(idx[0, 0][idx[0, 0] >= 0]) == np.arange(8))


def test_causality_future_chunks_do_not_matter():
    """Changing landmarks/K/V of the query's own and later chunks changes nothing."""
    cfg = small_cfg(top_k=3)
    inp = W.generate(cfg, seed=4)
    r = 64 * 5 + 17
    idx1, s1, _, o1 = run(inp, rows=[r])
    own = r // 64
    inp.landmarks[0, :, own:] = 100.0
    inp.k[0, :, own * 64:] *= -3
    inp.v[0, :, own * 64:] += 5
    idx2, s2, _, o2 = run(inp, rows=[r])
    assert np.array_equal(idx1, idx2) and np.array_equal(s1, s2) and np.array_equal(o1, o2)


# ----------------------------------------------------------------------------
# Attention inside a chunk (Step 3) and fusion (Step 4)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("qk_norm", [True, False])
def test_k1_equals_dense_sdpa_over_chosen_chunk(qk_norm):
    """Invariant: K = 1 gives dense softmax attention over the chosen
    chunk.  Reference: torch SDPA.  Catches missing/extra normalisation, wrong
    scale, K/V transposed or read from the wrong chunk/head."""
    cfg = small_cfg(top_k=1, n_q_heads=4, n_kv_heads=2, batch=2, qk_norm=qk_norm)
    inp = W.generate(cfg, seed=21)
    inp.k[1, 1, 64 * 2 + 5] = 0.0           # a zero key row (norm clamp)
    rows = np.array([70, 300, 511, 512 + 200, 512 + 450])
    a_s = 0.37
    idx, _, w, out = run(inp, rows=rows, attn_scale=a_s)
    q = f64(inp.q_attn, cfg.dtype)
    k = f64(inp.k, cfg.dtype)
    v = f64(inp.v, cfg.dtype)
    for i, fr in enumerate(rows):
        b, r = divmod(int(fr), cfg.q_len)
        for h in range(cfg.n_q_heads):
            g = h // cfg.group
            c = idx[i, g, 0]
            assert w[i, g, 0] == 1.0
            ref = sdpa_chunk(q[b, r, h], k[b, g, 64 * c:64 * c + 64], v[b, g, 64 * c:64 * c + 64],
                             a_s, qk_norm)
            np.testing.assert_allclose(out[i, h], ref, rtol=0, atol=1e-13)


def test_uniform_scores_give_mean_of_chunk_attentions():
    """Invariant: uniform retrieval scores and K >= #chunks give the mean
    of the per-chunk attentions (reference: torch SDPA per chunk)."""
    cfg = small_cfg(top_k=8, n_q_heads=2)
    inp = W.generate(cfg, seed=8)
    inp.q_ret[:] = 0.0
    rows = np.array([64 * 4 + 3, 64 * 7 + 63])
    idx, _, w, out = run(inp, rows=rows)
    q = f64(inp.q_attn, "f32"); k = f64(inp.k, "f32"); v = f64(inp.v, "f32")
    for i, r in enumerate(rows):
        n = r // 64
        np.testing.assert_allclose(w[i, 0, :n], 1.0 / n, rtol=1e-15)
        for h in range(2):
            ref = np.mean([sdpa_chunk(q[0, r, h], k[0, 0, 64 * c:64 * c + 64],
                                      v[0, 0, 64 * c:64 * c + 64], 1 / 8.0) for c in range(n)], axis=0)
            np.testing.assert_allclose(out[i, h], ref, rtol=0, atol=1e-13)


def test_weights_sum_to_one_and_follow_scores():
    """Invariant: blend weights sum to 1; larger score => larger weight."""
    cfg = W.shrink(W.CONFIGS[1], q_len=2048, kv_len=2048)
    inp = W.generate(cfg)
    rows = np.arange(64, 2048, 97)
    idx, score, w, _ = run(inp, rows=rows, with_output=False)
    valid = idx >= 0
    sums = np.where(valid, w, 0).sum(-1)
    np.testing.assert_allclose(sums, 1.0, rtol=0, atol=1e-14)
    assert np.all(w[~valid] == 0) and np.all(w[valid] > 0)
    assert np.all(np.diff(np.where(valid, w, -1), axis=-1)[valid[..., 1:]] <= 1e-17)


def test_two_chunk_blend_closed_form():
    """Two eligible chunks, K = 2, V constant per chunk (so each chunk attention is
    exactly that constant): out = w0*a + w1*b with w0 = 1/(1+exp(s1-s0)) and
    s = raw * ret_scale.  Catches raw-vs-s, sign of the softmax, weight/chunk swap."""
    cfg = small_cfg(q_len=1, q_pos0=150, kv_len=192, top_k=2, head_dim=64, n_q_heads=1)
    inp = W.generate(cfg, seed=6)
    qv = np.zeros(64, np.float32); qv[0] = 1.0; qv[5] = 2.0
    inp.q_ret[0, 0, 0] = qv
    inp.landmarks[0, 0, 0] = 0; inp.landmarks[0, 0, 0, 0] = 3.0            # raw 3
    inp.landmarks[0, 0, 1] = 0; inp.landmarks[0, 0, 1, 5] = 0.25           # raw 0.5
    inp.landmarks[0, 0, 2] = 50.0                                          # not eligible (p=150)
    a = np.linspace(-1, 1, 64).astype(np.float32)
    bvec = np.cos(np.arange(64)).astype(np.float32)
    inp.v[0, 0, 0:64] = a
    inp.v[0, 0, 64:128] = bvec
    rs = 0.7
    idx, score, w, out = run(inp, ret_scale=rs)
    assert list(idx[0, 0]) == [0, 1]
    w0 = 1.0 / (1.0 + math.exp((0.5 - 3.0) * rs))
    np.testing.assert_allclose(w[0, 0], [w0, 1 - w0], rtol=1e-15)
    np.testing.assert_allclose(out[0, 0], w0 * a.astype(np.float64) + (1 - w0) * bvec, atol=1e-14)


def test_hand_worked_example_d2():
    """A fully hand-derived case with d = 2 (derivation in tests/golden/hand_worked_example.json)."""
    import json, os
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked_example.json")))
    f = lambda x: np.array(x, np.float32)
    q_ret, lm, q_attn, k, v = (f(ex["inputs"][n]) for n in ("q_ret", "landmarks", "q_attn", "k", "v"))
    idx, score, w, out = oracle.forward(q_ret, lm, q_attn, k, v, q_pos0=ex["q_pos0"],
                                        top_k=ex["top_k"], qk_norm=True)
    a = 1 / math.sqrt(2)
    sig = 1 / (1 + math.exp(-a))
    assert list(idx[0, 0]) == ex["expected"]["topk_idx"]
    np.testing.assert_allclose(score[0, 0], [3 * a, 2 * a], rtol=1e-15)
    np.testing.assert_allclose(w[0, 0], [sig, 1 - sig], rtol=1e-15)
    ref = [sig * sig + (1 - sig) * 2.0, sig * (1 - sig) - (1 - sig)]
    np.testing.assert_allclose(out[0, 0], ref, rtol=0, atol=1e-15)


def test_constant_values_give_that_value():
    cfg = small_cfg(top_k=4)
    inp = W.generate(cfg, seed=12)
    const = np.float32(0.625)
    inp.v[:] = const
    idx, _, _, out = run(inp, rows=np.arange(64, 512, 13))
    np.testing.assert_allclose(out, 0.625, rtol=0, atol=1e-14)


def test_zero_keys_give_chunk_mean_of_values():
    """All keys zero => uniform in-chunk softmax => chunk mean of V (K = 1)."""
    cfg = small_cfg(top_k=1)
    inp = W.generate(cfg, seed=13)
    inp.k[:] = 0.0
    rows = np.array([100, 400])
    idx, _, _, out = run(inp, rows=rows)
    v = f64(inp.v, "f32")
    for i, r in enumerate(rows):
        c = idx[i, 0, 0]
        np.testing.assert_allclose(out[i, 0], v[0, 0, 64 * c:64 * c + 64].mean(0), atol=1e-15)


def test_linear_in_values():
    cfg = small_cfg(top_k=3)
    inp = W.generate(cfg, seed=14)
    rows = np.arange(64, 512, 31)
    v2 = W.generate(cfg, seed=15).v
    _, _, _, o1 = run(inp, rows=rows)
    _, _, _, o2 = run(replace(inp, v=v2), rows=rows)
    mix = (inp.v.astype(np.float64) * 0.5 - v2.astype(np.float64) * 2.0).astype(np.float32)
    _, _, _, o3 = run(replace(inp, v=mix), rows=rows)
    ref = 0.5 * o1 - 2.0 * o2
    # mix is rounded to fp32; compare against the exact combination of rounded inputs
    np.testing.assert_allclose(o3, ref, atol=1e-6)


def test_qk_norm_scale_invariance():
    """With query-key normalisation, positive rescaling of q_attn rows or key rows
    leaves the output unchanged; without it, the output changes."""
    cfg = small_cfg(top_k=3)
    inp = W.generate(cfg, seed=16)
    rows = np.arange(64, 512, 29)
    _, _, _, o1 = run(inp, rows=rows)
    scale_rows = np.float32(4.0)
    kscale = (2.0 ** np.random.default_rng(0).integers(-3, 4, size=inp.k.shape[:-1] + (1,))).astype(np.float32)
    inp2 = replace(inp, q_attn=inp.q_attn * scale_rows, k=(inp.k * kscale).astype(np.float32))
    _, _, _, o2 = run(inp2, rows=rows)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
    _, _, _, o3 = run(inp, rows=rows, qk_norm=False)
    _, _, _, o4 = run(inp2, rows=rows, qk_norm=False)
    assert np.abs(o3 - o4).max() > 1e-3


def test_shift_invariance_of_given_scores():
    """Step 4 softmax: adding a constant to all selected scores changes nothing."""
    cfg = small_cfg(top_k=4)
    inp = W.generate(cfg, seed=17)
    rows = np.arange(300, 512, 19)
    idx, score, w, out = run(inp, rows=rows)
    w2, out2 = oracle.attend_blend(inp.q_attn, inp.k, inp.v, idx, score + 3.25, rows=rows)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-14)
    np.testing.assert_allclose(w2, w, rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------
# Whole-forward structural facts
# ----------------------------------------------------------------------------

def test_gqa_shared_selection_equals_replicated_single_head_groups():
    """G q heads sharing one kv head equal G separate G=1 problems with that kv
    head's q_ret/landmarks/K/V replicated.  Catches a wrong h -> g mapping."""
    cfg = small_cfg(n_q_heads=8, n_kv_heads=2, top_k=3, q_len=256, kv_len=256)
    inp = W.generate(cfg, seed=18)
    _, _, _, out = run(inp)
    G = 4
    rep = lambda a, axis: np.repeat(a, G, axis=axis)
    out1 = run(replace(inp, q_ret=rep(inp.q_ret, 2), landmarks=rep(inp.landmarks, 1),
                       k=rep(inp.k, 1), v=rep(inp.v, 1)), cfg=cfg)[3]
    np.testing.assert_array_equal(out, out1)


def test_appended_rows_equal_rows_of_full_prefill():
    """Rows given with q_pos0 > 0 (chunked prefill / decode) equal the same rows of
    a prefill over the whole sequence."""
    cfg = small_cfg(q_len=640, kv_len=640, top_k=4, n_q_heads=2)
    inp = W.generate(cfg, seed=19)
    full = run(inp)
    m = 100
    tail = replace(inp, q_ret=inp.q_ret[:, -m:].copy(), q_attn=inp.q_attn[:, -m:].copy())
    part = oracle.forward(tail.q_ret, tail.landmarks, tail.q_attn, tail.k, tail.v,
                          q_pos0=640 - m, top_k=4)
    for a, b in zip(full, part):
        np.testing.assert_array_equal(a[-m:], b)


def test_batch_independence():
    cfg = small_cfg(batch=3, top_k=3, q_len=256, kv_len=256)
    inp = W.generate(cfg, seed=20)
    full = run(inp)
    one = replace(inp, q_ret=inp.q_ret[1:2], landmarks=inp.landmarks[1:2], q_attn=inp.q_attn[1:2],
                  k=inp.k[1:2], v=inp.v[1:2])
    part = run(one)
    for a, b in zip(full, part):
        np.testing.assert_array_equal(a[256:512], b)


def test_thread_count_does_not_change_results():
    cfg = small_cfg(top_k=4, n_q_heads=2)
    inp = W.generate(cfg, seed=22)
    n0 = oracle.max_threads()
    try:
        oracle.set_threads(1)
        a = run(inp)
        oracle.set_threads(max(2, n0))
        b = run(inp)
    finally:
        oracle.set_threads(n0)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_raw_scores_match_selection():
    cfg = small_cfg(top_k=5)
    inp = W.generate(cfg, seed=23)
    r = 64 * 6 + 2
    raw, n = oracle.raw_scores(inp.q_ret, inp.landmarks, q_pos0=0, kv_len=512, flat_row=r, g=0)
    assert n == 6 and np.all(np.isnan(raw[6:]))
    idx, score, _, _ = run(inp, rows=[r], with_output=False)
    np.testing.assert_array_equal(raw[idx[0, 0]] / 8.0, score[0, 0])


# ----------------------------------------------------------------------------
# landmark stand-in (chunk mean of the keys): Step 1 gives one landmark per
# 64-token chunk; the workloads' stand-in for the learned encoder is the mean
# ----------------------------------------------------------------------------

def test_landmarks_of_constant_chunks_are_the_constant():
    """Catches a wrong divisor, a dropped key or a chunk offset error."""
    rng = np.random.default_rng(3)
    B, Hkv, nc, d = 2, 3, 5, 16
    vals = rng.standard_normal((B, Hkv, nc, d)).astype(np.float32)
    k = np.repeat(vals[:, :, :, None, :], 64, axis=3).reshape(B, Hkv, nc * 64, d)
    out = oracle.chunk_landmarks(k)
    assert np.array_equal(out, vals.astype(np.float64))


def test_landmarks_exact_on_integer_keys():
    """Integer keys: the mean is sum/64, computed here with Python integers."""
    rng = np.random.default_rng(4)
    B, Hkv, L, d = 1, 2, 64 * 7 + 19, 8          # trailing partial chunk has no landmark
    ki = rng.integers(-50, 51, size=(B, Hkv, L, d))
    k = ki.astype(np.float32)
    out = oracle.chunk_landmarks(k)
    assert out.shape == (B, Hkv, 7, d)
    for b in range(B):
        for g in range(Hkv):
            for c in range(7):
                for x in range(d):
                    s = sum(int(v) for v in ki[b, g, 64 * c:64 * c + 64, x])
                    assert out[b, g, c, x] == s / 64          # exact: s / 64 is a dyadic rational


def test_landmarks_range_and_locality():
    """A chunk range equals the same slice of the full result, and changing one
    key changes only its own chunk's landmark."""
    rng = np.random.default_rng(5)
    k = rng.standard_normal((1, 2, 64 * 9, 8)).astype(np.float32)
    full = oracle.chunk_landmarks(k)
    part = oracle.chunk_landmarks(k, chunk_begin=3, chunk_end=7)
    assert np.array_equal(part, full[:, :, 3:7])
    k2 = k.copy()
    k2[0, 1, 64 * 5 + 17, 3] += 1.0
    diff = np.argwhere(oracle.chunk_landmarks(k2) != full)
    assert diff.tolist() == [[0, 1, 5, 3]]
    assert oracle.chunk_landmarks(k, chunk_begin=4, chunk_end=4).shape == (1, 2, 0, 8)
    with pytest.raises(ValueError):
        oracle.chunk_landmarks(k, chunk_begin=2, chunk_end=10)


def test_landmarks_match_the_generators_stand_in():
    """The generator's landmarks without noise or needles are the stored chunk
    means: an independent implementation of the same definition (bf16, RNE)."""
    cfg = small_cfg(dtype="bf16", kv_len=64 * 20, q_len=64, n_kv_heads=2, n_q_heads=2)
    inp = W.generate(cfg)
    ref = W.store(oracle.chunk_landmarks(inp.k), "bf16")
    a = W.bf16_bits_to_f32(ref).astype(np.float64)
    b = W.bf16_bits_to_f32(inp.landmarks).astype(np.float64)
    ulp = np.abs(b) * 2.0 ** -7
    assert np.all(np.abs(a - b) <= ulp)          # at most one bf16 step apart
    assert np.mean(a == b) > 0.99


# ----------------------------------------------------------------------------
# backward (the next step after the forward): gradients of sum(out * dout)
# for a fixed selection
# ----------------------------------------------------------------------------

def _bwd_case(qk_norm=True, seed=21, B=1, Lq=40, Lkv=64 * 6 + 10, Hq=4, Hkv=2, d=16, K=3):
    rng = np.random.default_rng(seed)
    nc = Lkv // 64
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    q_ret, lm, q_attn = f(B, Lq, Hkv, d), f(B, Hkv, nc, d), f(B, Lq, Hq, d)
    k, v, dout = f(B, Hkv, Lkv, d), f(B, Hkv, Lkv, d), f(B, Lq, Hq, d)
    idx = np.full((B, Lq, Hkv, K), -1, np.int32)
    for b in range(B):
        for r in range(Lq):
            for g in range(Hkv):
                m = rng.integers(0, K + 1)           # 0..K used slots, some rows empty
                idx[b, r, g, :m] = rng.choice(nc, size=m, replace=False)
    return q_ret, lm, q_attn, k, v, dout, idx


def _scores(q_ret, lm, idx, rs):
    """s = ret_scale * q_ret . landmark[idx] (numpy fp64); -inf on unused slots."""
    B, Lq, Hkv, K = idx.shape
    s = np.full(idx.shape, -np.inf)
    for b in range(B):
        for g in range(Hkv):
            L = lm[b, g].astype(np.float64)
            for r in range(Lq):
                ok = idx[b, r, g] >= 0
                s[b, r, g, ok] = rs * (L[idx[b, r, g, ok]] @ q_ret[b, r, g].astype(np.float64))
    return s


def _torch_forward(q_ret, lm, q_attn, k, v, idx, qk_norm, rs, as_):
    """The fixed-selection forward of Steps 2-4 in torch (fp64), for autograd."""
    B, Lq, Hkv, K = idx.shape
    Hq, d = q_attn.shape[2], q_attn.shape[3]
    G = Hq // Hkv
    nrm = lambda x: x / torch.clamp(torch.linalg.vector_norm(x, dim=-1, keepdim=True), min=1e-6)
    outs = []
    for b in range(B):
        rows = []
        for r in range(Lq):
            heads = []
            for g in range(Hkv):
                ok = [kk for kk in range(K) if idx[b, r, g, kk] >= 0]
                if not ok:
                    heads.append(torch.zeros(G, d))
                    continue
                cs = [int(idx[b, r, g, kk]) for kk in ok]
                s = torch.stack([rs * torch.dot(q_ret[b, r, g], lm[b, g, c]) for c in cs])
                w = torch.softmax(s, 0)
                q = q_attn[b, r, g * G:(g + 1) * G]
                qh = nrm(q) if qk_norm else q
                o = torch.zeros(G, d)
                for wk, c in zip(w, cs):
                    kc, vc = k[b, g, 64 * c:64 * c + 64], v[b, g, 64 * c:64 * c + 64]
                    kh = nrm(kc) if qk_norm else kc
                    p = torch.softmax(as_ * qh @ kh.T, dim=-1)
                    o = o + wk * (p @ vc)
                heads.append(o)
            rows.append(torch.cat(heads, 0))
        outs.append(torch.stack(rows))
    return torch.stack(outs)


@pytest.mark.parametrize("qk_norm", [True, False])
def test_backward_matches_autograd_of_the_forward(qk_norm):
    """torch autograd of the fixed-selection forward gives every gradient; the
    oracle's hand-derived backward must agree (catches a dropped term of the
    softmax or normalisation gradients, a missing blend weight, a wrong sign,
    a transposed product, a wrong chunk offset in the scatter)."""
    q_ret, lm, q_attn, k, v, dout, idx = _bwd_case(qk_norm=qk_norm)
    d = q_ret.shape[-1]
    rs, as_ = 1.0 / math.sqrt(d), 0.9
    s = _scores(q_ret, lm, idx, rs)
    ts = [torch.tensor(a.astype(np.float64), requires_grad=True) for a in (q_ret, lm, q_attn, k, v)]
    out = _torch_forward(*ts, idx, qk_norm, rs, as_)
    (out * torch.tensor(dout.astype(np.float64))).sum().backward()
    got = oracle.backward(q_ret, lm, q_attn, k, v, dout, idx, s, qk_norm=qk_norm, ret_scale=rs, attn_scale=as_)
    for name, g_or, t in zip(("dq_ret", "dlm", "dq_attn", "dk", "dv"), got, ts):
        ref = t.grad.numpy()
        assert np.abs(g_or - ref).max() <= 1e-9 * max(1.0, np.abs(ref).max()), name


def test_backward_matches_finite_differences_of_the_oracle_forward():
    """Central differences of the oracle's own forward (attend_blend with the
    scores recomputed from q_ret and landmarks) at sampled coordinates."""
    q_ret, lm, q_attn, k, v, dout, idx = _bwd_case(seed=22, Lq=12, Hq=2, Hkv=1, d=8, K=2)
    d = q_ret.shape[-1]
    rs = 1.0 / math.sqrt(d)
    base = [a.copy() for a in (q_ret, lm, q_attn, k, v)]

    def loss(arrs):
        s = _scores(arrs[0], arrs[1], idx, rs)
        B, Lq, Hkv, K = idx.shape
        _, out = oracle.attend_blend(arrs[2], arrs[3], arrs[4], idx.reshape(B * Lq, Hkv, K),
                                     s.reshape(B * Lq, Hkv, K))
        return float((out.reshape(dout.shape) * dout.astype(np.float64)).sum())

    grads = oracle.backward(*base, dout, idx, _scores(q_ret, lm, idx, rs))
    rng = np.random.default_rng(5)
    for which in range(5):
        g = grads[which]
        flat = np.flatnonzero(np.abs(g) > 1e-3)
        for pos in rng.choice(flat, size=min(6, flat.size), replace=False):
            arrs = [a.copy() for a in base]
            x = arrs[which].reshape(-1)
            x0 = np.float64(x[pos])
            h = 1e-2 * max(1.0, abs(x0))
            x[pos] = np.float32(x0 + h)
            up, hp = loss(arrs), np.float64(x[pos]) - x0
            x[pos] = np.float32(x0 - h)
            dn, hm = loss(arrs), x0 - np.float64(x[pos])
            fd = (up - dn) / (hp + hm)
            assert abs(fd - g.reshape(-1)[pos]) <= 2e-3 * max(1.0, abs(fd)), (which, pos)


def test_backward_invariants():
    """Closed forms: with QK-norm the loss does not change under positive
    rescaling of a query or key row, so those gradients are orthogonal to the
    row; P sums to 1, so the V gradients of a (b, kv head) sum to the dout of
    its rows that select something; a common shift of all landmarks leaves every
    blend weight unchanged, so their gradients sum to 0."""
    q_ret, lm, q_attn, k, v, dout, idx = _bwd_case(seed=23)
    rs = 1.0 / math.sqrt(q_ret.shape[-1])
    dq_ret, dlm, dq_attn, dk, dv = oracle.backward(q_ret, lm, q_attn, k, v, dout, idx,
                                                   _scores(q_ret, lm, idx, rs))
    assert np.abs((dq_attn * q_attn).sum(-1)).max() < 1e-10
    nck = (k.shape[2] // 64) * 64
    assert np.abs((dk[:, :, :nck] * k[:, :, :nck]).sum(-1)).max() < 1e-10
    assert np.all(dk[:, :, nck:] == 0) and np.all(dv[:, :, nck:] == 0)   # partial chunk: no landmark
    B, Lq, Hkv, K = idx.shape
    G = q_attn.shape[2] // Hkv
    for b in range(B):
        for g in range(Hkv):
            used = (idx[b, :, g] >= 0).any(-1)
            want = dout[b, used][:, g * G:(g + 1) * G].astype(np.float64).sum((0, 1))
            assert np.allclose(dv[b, g].sum(0), want, atol=1e-10)
            assert np.abs(dlm[b, g].sum(0)).max() < 1e-10
    # rows with no used slot get no gradient
    empty = ~(idx >= 0).any(-1)
    assert np.all(dq_ret[empty] == 0)
