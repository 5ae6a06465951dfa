"""Comparison helpers for GPU-vs-oracle parity (test infrastructure).

Selection parity follows the rule for continuous data: the selected chunk set
must equal the oracle's, except that a swap of two chunks is admissible when
their fp64 raw scores differ by less than the fp32 forward-error bound of the
two dot products (the GPU ranks fp32 dot products, the oracle fp64 ones).  Any
other difference fails.  Rows with an admissible swap have their output checked
against the oracle re-run on the GPU's own selection.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads as W

U32 = 2.0 ** -24


def gamma(n: int) -> float:
    return n * U32 / (1 - n * U32)


def to_device(a: np.ndarray, dtype: str, device="cuda:0"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def inputs_to_device(inp: W.HsaInputs, device="cuda:0"):
    dt = inp.cfg.dtype
    return [to_device(a, dt, device) for a in (inp.q_ret, inp.landmarks, inp.q_attn, inp.k, inp.v)]


def out_to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def dot_bounds(q_ret: np.ndarray, landmarks: np.ndarray, dtype: str, b: int, r: int, g: int):
    """Per-chunk forward-error bound 2*gamma_d*sum|q_x l_x| of the fp32 dot product."""
    q = W.to_f64(q_ret[b, r, g], dtype)
    lm = W.to_f64(landmarks[b, g], dtype)
    d = q.shape[-1]
    return 2.0 * gamma(d) * (np.abs(lm) @ np.abs(q))


class SelectionReport:
    def __init__(self):
        self.rows = 0
        self.swaps = 0
        self.swapped_rows = []   # (flat_row, g)

    def __repr__(self):
        return "SelectionReport(rows=%d, admissible swaps=%d)" % (self.rows, self.swaps)


def check_selection(inp: W.HsaInputs, rows, gpu_idx: np.ndarray, gpu_score: np.ndarray,
                    orc_idx: np.ndarray, orc_score: np.ndarray, *, ret_scale: float,
                    exact: bool = False) -> SelectionReport:
    """gpu_* and orc_* are [n_rows, Hkv, K] for the flat rows `rows`.

    exact=True demands identical indices in identical order and bit-identical
    scores (grid mode, where fp32 scoring is exact)."""
    cfg = inp.cfg
    rep = SelectionReport()
    K = cfg.top_k
    for i, fr in enumerate(rows):
        b, r = divmod(int(fr), cfg.q_len)
        n = min((cfg.q_pos0 + r) // 64, cfg.n_chunks)
        keff = min(K, n)
        for g in range(cfg.n_kv_heads):
            rep.rows += 1
            gi, oi = gpu_idx[i, g], orc_idx[i, g]
            assert np.all(gi[keff:] == -1), (fr, g, gi)
            assert np.all(np.isneginf(gpu_score[i, g, keff:])), (fr, g)
            gset, oset = gi[:keff], oi[:keff]
            assert len(set(gset.tolist())) == keff, ("duplicate chunks", fr, g, gset)
            assert np.all((gset >= 0) & (gset < n)), ("ineligible chunk", fr, g, gset, n)
            if exact:
                assert np.array_equal(gset, oset), (fr, g, gset, oset)
                exp = (orc_score[i, g, :keff] / ret_scale).astype(np.float32) * np.float32(ret_scale)
                assert np.array_equal(gpu_score[i, g, :keff], exp), (fr, g)
                continue
            if keff == 0:
                continue
            raw, _ = oracle.raw_scores(inp.q_ret, inp.landmarks, q_pos0=cfg.q_pos0,
                                       kv_len=cfg.kv_len, flat_row=int(fr), g=g)
            tol = dot_bounds(inp.q_ret, inp.landmarks, cfg.dtype, b, r, g)
            # scores of the GPU's chunks agree with the oracle's fp64 values
            np.testing.assert_allclose(gpu_score[i, g, :keff], raw[gset] * ret_scale,
                                       rtol=2e-6, atol=float(tol[gset].max()) * ret_scale + 1e-30)
            only_g = sorted(set(gset.tolist()) - set(oset.tolist()))
            only_o = sorted(set(oset.tolist()) - set(gset.tolist()))
            if not only_g:
                continue
            for c_o in only_o:
                for c_g in only_g:
                    gap = raw[c_o] - raw[c_g]
                    assert gap <= tol[c_o] + tol[c_g], \
                        ("selection differs beyond the fp32 error band", fr, g, c_o, c_g, gap,
                         tol[c_o] + tol[c_g])
            rep.swaps += len(only_g)
            rep.swapped_rows.append((int(fr), g))
    return rep


def check_output(inp: W.HsaInputs, rows, gpu_out: np.ndarray, orc_out: np.ndarray, *, atol: float,
                 rep: SelectionReport | None = None, gpu_idx=None, qk_norm=True, attn_scale=None,
                 ret_scale=None):
    """Max-abs check of [n_rows, Hq, d] outputs; rows with admissible selection swaps are
    compared with the oracle re-run on the GPU's selection."""
    cfg = inp.cfg
    rows = np.asarray(rows)
    ref = orc_out.copy()
    if rep is not None and rep.swapped_rows:
        pos = {int(fr): i for i, fr in enumerate(rows)}
        rs = oracle.default_scale(cfg.head_dim) if ret_scale is None else ret_scale
        for fr in sorted({fr for fr, _ in rep.swapped_rows}):
            i = pos[fr]
            sel = gpu_idx[i:i + 1].astype(np.int32)
            sc = np.full(sel.shape, -np.inf)
            for g in range(cfg.n_kv_heads):
                raw, _ = oracle.raw_scores(inp.q_ret, inp.landmarks, q_pos0=cfg.q_pos0,
                                           kv_len=cfg.kv_len, flat_row=fr, g=g)
                ok = sel[0, g] >= 0
                sc[0, g, ok] = raw[sel[0, g, ok]] * rs
            _, o = oracle.attend_blend(inp.q_attn, inp.k, inp.v, sel, sc, rows=[fr], qk_norm=qk_norm,
                                       attn_scale=attn_scale)
            ref[i] = o[0]
    err = np.abs(gpu_out - ref)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= atol, ("max-abs error %.3e > %.1e" % (worst, atol),
                           np.unravel_index(int(err.argmax()), err.shape))
    return worst
