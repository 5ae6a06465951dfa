"""GPU parity of the HSA backward (hsa_backward through its C ABI) against the
fp64 oracle's backward, for a selection the oracle's forward made.

Tolerance: for each gradient tensor, max |gpu - oracle| <= 2e-2 * max |oracle|
and ||gpu - oracle||_2 <= 6e-3 * ||oracle||_2.  The kernels take bf16 inputs,
round the MFMA operands P, w*dout, dz/|q| and dz/|k| and the per-pair query
gradients to bf16 (relative error up to 2^-9 each) and accumulate in fp32, so a
gradient entry carries a relative error of about 1e-3 per rounded factor; a
dropped term or a wrong index moves the result by O(1) of the gradient's scale.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from workloads import HsaConfig

from hsa_check import inputs_to_device, out_to_f64, to_device

pytestmark = pytest.mark.gpu

MAX_TOL, L2_TOL = 2e-2, 6e-3
NAMES = ("dq_ret", "dlandmarks", "dq_attn", "dk", "dv")


@pytest.fixture(scope="module")
def hsa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ultra_long_context_amd as h
    h.load_library()
    return h


def small(**kw):
    base = dict(name="bwd", batch=1, q_len=1024, q_pos0=3072, kv_len=4096, n_q_heads=8, n_kv_heads=1,
                head_dim=128, top_k=8, dtype="bf16", noise_std=0.5, n_needles=4, seed=41)
    base.update(kw)
    return HsaConfig(**base)


def selection(inp):
    """The oracle's own selection; scores rounded to the fp32 both sides take."""
    cfg = inp.cfg
    oi, os_, _, _ = oracle.forward(inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v, q_pos0=cfg.q_pos0,
                                   top_k=cfg.top_k, qk_norm=cfg.qk_norm, with_output=False)
    shp = (cfg.batch, cfg.q_len, cfg.n_kv_heads, cfg.top_k)
    return oi.reshape(shp).copy(), os_.astype(np.float32).reshape(shp).copy()


def gpu_backward(hsa, inp, dout, idx, sc, **kw):
    import torch
    cfg = inp.cfg
    print("case %s B=%d Lq=%d Lkv=%d Hq=%d Hkv=%d d=%d K=%d norm=%d" % (
        cfg.name, cfg.batch, cfg.q_len, cfg.kv_len, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
        cfg.top_k, cfg.qk_norm), flush=True)
    dev = inputs_to_device(inp)
    ti = torch.from_numpy(idx).cuda()
    ts = torch.from_numpy(sc).cuda()
    td = to_device(dout, "bf16")
    grads = hsa.backward(*dev, ti, ts, td, qk_norm=cfg.qk_norm, **kw)
    torch.cuda.synchronize()
    return [out_to_f64(g) for g in grads]


def compare(got, ref, where=""):
    for name, g, r in zip(NAMES, got, ref):
        assert g.shape == r.shape, name
        scale = np.abs(r).max()
        if scale == 0:
            assert np.all(g == 0), name + where
            continue
        mx = np.abs(g - r).max() / scale
        l2 = np.linalg.norm(g - r) / np.linalg.norm(r)
        print("  %-10s max %.2e  l2 %.2e" % (name, mx, l2), flush=True)
        assert mx <= MAX_TOL, "%s%s: max-abs %.3e of scale" % (name, where, mx)
        assert l2 <= L2_TOL, "%s%s: l2 %.3e" % (name, where, l2)


def full_parity(hsa, cfg, idx_edit=None, **kw):
    inp = W.generate(cfg)
    idx, sc = selection(inp)
    if idx_edit is not None:
        idx_edit(idx)
    dout = W.cotangent(cfg)
    got = gpu_backward(hsa, inp, dout, idx, sc, **kw)
    ref = oracle.backward(inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v, dout, idx, sc,
                          qk_norm=cfg.qk_norm, **kw)
    compare(got, ref)
    return got, ref, idx


@pytest.mark.parametrize("G,Hkv,d,qk_norm", [(8, 1, 128, True), (1, 1, 128, True), (4, 2, 64, True),
                                             (16, 1, 128, True), (2, 1, 64, False), (8, 2, 128, False)])
def test_backward_parity(hsa, G, Hkv, d, qk_norm):
    full_parity(hsa, small(n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=d, qk_norm=qk_norm))


def test_backward_given_scales(hsa):
    full_parity(hsa, small(q_len=512, top_k=5), ret_scale=0.3, attn_scale=0.05)


def test_backward_gaps_partial_chunk_and_empty_rows(hsa):
    """Unused (-1) and out-of-range slots, a row with no used slot, a trailing
    partial chunk (its dk, dv stay zero) and unselected chunks."""
    cfg = small(q_len=700, kv_len=4096 + 37, q_pos0=3433, n_q_heads=16, n_kv_heads=2, top_k=6)

    def edit(idx):
        idx[0, ::5, :, 1] = -1
        idx[0, ::13, 0, 3] = 10 ** 6
        idx[0, 7] = -1

    got, ref, idx = full_parity(hsa, cfg, edit)
    dq_ret, dlm, dq_attn, dk, dv = got
    assert np.all(dq_attn[0, 7] == 0) and np.all(dq_ret[0, 7] == 0)
    nc = cfg.kv_len // 64
    assert np.all(dk[:, :, nc * 64:] == 0) and np.all(dv[:, :, nc * 64:] == 0)
    used = np.zeros((cfg.n_kv_heads, nc), bool)
    for g in range(cfg.n_kv_heads):
        c = idx[0, :, g].ravel()
        used[g, c[(c >= 0) & (c < nc)]] = True
    for g in range(cfg.n_kv_heads):
        for c in np.nonzero(~used[g])[0]:
            assert np.all(dk[0, g, c * 64:(c + 1) * 64] == 0) and np.all(dlm[0, g, c] == 0)


def test_backward_batch_and_row_bands(hsa):
    """Two sequences and more than 8192 query rows (pairs of one chunk split over
    row bands, summed in a fixed order)."""
    cfg = small(batch=2, q_len=8704, q_pos0=0, kv_len=8704, n_q_heads=2, n_kv_heads=1, head_dim=64,
                top_k=4, n_needles=8)
    full_parity(hsa, cfg)


def test_backward_k1_and_k64(hsa):
    full_parity(hsa, small(q_len=256, top_k=1, n_q_heads=4))
    full_parity(hsa, small(q_len=256, top_k=64, n_q_heads=4, q_pos0=3840))


def test_backward_deterministic(hsa):
    import torch
    cfg = small(q_len=2048, q_pos0=2048)
    inp = W.generate(cfg)
    idx, sc = selection(inp)
    dout = W.cotangent(cfg)
    a = gpu_backward(hsa, inp, dout, idx, sc)
    b = gpu_backward(hsa, inp, dout, idx, sc)
    for name, x, y in zip(NAMES, a, b):
        assert np.array_equal(x, y), name


def test_backward_training_window_sampled(hsa):
    """The 32K training window (B=1, 32768 rows, GQA-8, d=128, K=8) in the
    launch the benchmark times.  Row gradients (dq_ret, dq_attn) of sampled rows
    come from the oracle run on those rows alone; the key, value and landmark
    gradients of sampled chunks from the oracle run on every row that selected
    the chunk (a chunk's gradient sums over exactly those rows)."""
    cfg = W.config(1)
    inp = W.generate(cfg)
    idx, sc = selection(inp)
    dout = W.cotangent(cfg)
    got = gpu_backward(hsa, inp, dout, idx, sc)

    def sub(rows):
        r = np.asarray(rows)
        return oracle.backward(inp.q_ret[:, r], inp.landmarks, inp.q_attn[:, r], inp.k, inp.v, dout[:, r],
                               idx[:, r], sc[:, r], qk_norm=cfg.qk_norm)

    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 63, 64, 4095, cfg.q_len - 1], rng.choice(cfg.q_len, 59, replace=False)]))
    ref = sub(rows)
    z = np.zeros(1)
    compare([got[0][:, rows], z, got[2][:, rows], z, z], [ref[0], z, ref[2], z, z], " (sampled rows)")
    counts = np.bincount(idx[0, :, 0].ravel()[idx[0, :, 0].ravel() >= 0], minlength=cfg.n_chunks)
    chunks = {0, int(np.argmax(counts)), cfg.n_chunks - 2}
    chunks |= set(rng.choice(cfg.n_chunks - 1, 3, replace=False).tolist())
    for c in sorted(chunks):
        rows_c = np.nonzero((idx[0, :, 0] == c).any(axis=-1))[0]
        if rows_c.size == 0:
            continue
        ref = sub(rows_c)
        sl = slice(c * 64, (c + 1) * 64)
        compare([z, got[1][:, :, c], z, got[3][:, :, sl], got[4][:, :, sl]],
                [z, ref[1][:, :, c], z, ref[3][:, :, sl], ref[4][:, :, sl]],
                " (chunk %d, %d rows)" % (c, rows_c.size))


def test_backward_without_complete_chunks(hsa):
    """A history shorter than one chunk: nothing can be selected, every
    gradient is zero (the partial chunk's keys included)."""
    import torch
    cfg = small(q_len=64, q_pos0=0, kv_len=37, n_needles=0, top_k=4)
    inp = W.generate(cfg)
    idx = np.full((1, cfg.q_len, 1, cfg.top_k), -1, np.int32)
    idx[0, ::3, 0, 0] = 0                       # chunk 0 does not exist (Nc = 0): unused
    sc = np.zeros(idx.shape, np.float32)
    dout = W.cotangent(cfg)
    got = gpu_backward(hsa, inp, dout, idx, sc)
    for name, g in zip(NAMES, got):
        assert np.all(g == 0), name


def test_backward_global_histogram_bucketing(hsa):
    """A history of more than 16,384 chunks: the backward's bucketing counts
    pairs with global atomics whose return values place them in their bins."""
    full_parity(hsa, small(q_len=600, q_pos0=1048700, kv_len=1048700 + 600 + 37, n_q_heads=2, n_kv_heads=1,
                           head_dim=64, top_k=8, n_needles=16))


def test_backward_duplicate_slots(hsa):
    """A given selection may name one chunk in two slots of a row: two pairs,
    as in the oracle."""
    cfg = small(q_len=300, top_k=6)

    def edit(idx):
        idx[0, ::7, 0, 1] = idx[0, ::7, 0, 0]

    full_parity(hsa, cfg, edit)


def test_backward_profiled_matches(hsa):
    """hsa_backward_profiled gives the gradients of hsa_backward bit for bit and
    records its bucket, attend and combine stages."""
    import torch
    cfg = small(q_len=512)
    inp = W.generate(cfg)
    idx, sc = selection(inp)
    dout = W.cotangent(cfg)
    dev = inputs_to_device(inp)
    ti, ts, td = torch.from_numpy(idx).cuda(), torch.from_numpy(sc).cuda(), to_device(dout, "bf16")
    a = hsa.backward(*dev, ti, ts, td)
    evs = {n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in hsa.STAGES}
    b = hsa.backward(*dev, ti, ts, td, stage_events=evs)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    for n in ("bucket", "attend", "combine"):
        assert evs[n][0].elapsed_time(evs[n][1]) > 0, n


# ----------------------------------------------------------------------------
# the warm-up stage's global HSA: a selection of every eligible chunk (K > 64)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("G,Hkv,d,qk_norm,q_len,kv_len,q_pos0", [
    (8, 1, 128, True, 768, 6144, 5376),       # 84..95 eligible chunks per row, K = 96
    (4, 2, 64, True, 4608, 4608, 0),          # prefill: 0..71 eligible chunks, K = 72
    (16, 1, 128, False, 300, 8448, 8148),     # K = 132, no query-key normalisation
])
def test_backward_every_eligible_chunk(hsa, G, Hkv, d, qk_norm, q_len, kv_len, q_pos0):
    """hsa_backward for a selection listing every eligible chunk (the oracle's
    forward with top_k >= the number of eligible chunks): more than 64 slots
    per row, the case global HSA trains with."""
    n_max = min((q_pos0 + q_len - 1) // 64, kv_len // 64)
    K = n_max + 1
    cfg = small(q_len=q_len, kv_len=kv_len, q_pos0=q_pos0, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=d,
                qk_norm=qk_norm, top_k=K, seed=70 + G)
    assert K > 64
    full_parity(hsa, cfg)
