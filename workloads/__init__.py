"""Seeded synthetic inputs for the Hierarchical Sparse Attention (HSA) forward.

This module only draws and stores input tensors. It contains none of the
method's arithmetic (no scoring, selection, attention or blending), so both
the fp64 oracle under ``oracle/`` and the HIP library can be fed from it
without sharing any code with each other.

Workloads follow the shapes of the paper's setting ("Every Token Counts:
Generalizing 16M Ultra-Long Context in LLMs", agent-atlas explainer, section
"How It Works", Step 1: 64-token chunks; TL;DR: a 32K training window and
contexts out to 16M tokens).

Recipe (all five workloads):
  * q_ret, q_attn, K, V: i.i.d. N(0,1) drawn in fp32 (numpy's float32 sampler)
    and, for bf16 workloads, rounded to bf16 (RNE).  Stored arrays hold the dtype's bits
    (``float32`` or ``uint16`` for bf16).
  * landmark of chunk i = fp64 mean of the chunk's 64 *stored* keys, plus
    optional N(0, noise_std) noise, plus needle boosts, then rounded like the
    other tensors.  (The paper's landmark comes from a learned encoder; the
    chunk mean is a stand-in with the same role.)
  * a needle boost of b sigma along the owner's retrieval query raises that
    owner's raw score by exactly b times the std of its raw-score distribution:
    l_n += b * sigma_l * q_ret[o] / ||q_ret[o]||, in every kv head with that
    head's q_ret.
  * RNG: numpy Generator(PCG64(SeedSequence([seed, tensor_id, block]))), with
    blocks of 2^23 elements of each flattened tensor, so any block of a
    16M-token history can be drawn on its own.  tensor ids: 0 q_ret, 1 q_attn, 2 K, 3 V, 4 landmark noise,
    5 needles.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

CHUNK = 64
BLOCK_TOKENS = 65536
BLOCK_ELEMS = 1 << 23

T_QRET, T_QATTN, T_K, T_V, T_NOISE, T_NEEDLE, T_DOUT = range(7)


@dataclass(frozen=True)
class HsaConfig:
    name: str
    batch: int
    q_len: int
    q_pos0: int
    kv_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    top_k: int
    dtype: str                      # "f32" or "bf16"
    noise_std: float = 0.0          # landmark noise std
    n_needles: int = 0              # per sequence (prefill style)
    needle_sigma: float = 4.0
    needle_hi: int = -1             # needles drawn in [0, needle_hi]; -1 => all visible chunks
    decode_needles: bool = False    # 32 needles per query row (one +5 sigma, 31 +3 sigma)
    qk_norm: bool = True
    seed: int = 0

    @property
    def n_chunks(self) -> int:
        return self.kv_len // CHUNK

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def sigma_l(self) -> float:
        return math.sqrt(1.0 / CHUNK + self.noise_std ** 2)


# The five workloads.  Index i uses seed 1000 + i.
CONFIGS = [
    HsaConfig("tiny_fp32_L1K", 1, 1024, 0, 1024, 1, 1, 64, 4, "f32",
              n_needles=3, needle_hi=14, seed=1000),
    HsaConfig("prefill_32K_gqa8", 1, 32768, 0, 32768, 8, 1, 128, 8, "bf16",
              noise_std=0.5, n_needles=16, needle_hi=510, seed=1001),
    HsaConfig("prefill_128K_b2_gqa8", 2, 131072, 0, 131072, 32, 4, 128, 16, "bf16",
              noise_std=0.5, n_needles=64, needle_hi=2046, seed=1002),
    HsaConfig("decode_16M_16q", 1, 16, 16777216, 16777216, 8, 1, 128, 32, "bf16",
              decode_needles=True, seed=1003),
    HsaConfig("chunked_prefill_1M_plus_8K", 1, 8192, 1048576, 1048576 + 8192, 32, 4, 128, 32,
              "bf16", noise_std=0.5, n_needles=256, needle_hi=16510, seed=1004),
]


def config(i: int, **overrides) -> HsaConfig:
    return replace(CONFIGS[i], **overrides)


# ----------------------------------------------------------------------------
# storage helpers (bit-level rounding; no arithmetic of the method)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    u += t
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def store(x64: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> fp32 (RNE) -> bf16 (RNE) storage, as the workloads specify."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of stored values."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    return bf16_bits_to_f32(a).astype(np.float64)


def storage_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def _rng(seed: int, tensor_id: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, block])))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_rows(seed: int, tensor_id: int, n_rows: int, row_len: int, dtype: str) -> np.ndarray:
    """[n_rows, row_len] stored N(0,1) values, drawn in blocks of BLOCK_ELEMS elements of the
    flattened array (block b covers elements [b*BLOCK_ELEMS, (b+1)*BLOCK_ELEMS))."""
    out = np.empty(n_rows * row_len, dtype=storage_dtype(dtype))
    n = out.size
    n_blocks = (n + BLOCK_ELEMS - 1) // BLOCK_ELEMS

    def work(blk):
        lo = blk * BLOCK_ELEMS
        hi = min(n, lo + BLOCK_ELEMS)
        x = _rng(seed, tensor_id, blk).standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = x if dtype == "f32" else f32_to_bf16_bits(x)

    if n_blocks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(n_blocks)))
    return out.reshape(n_rows, row_len)


def _grid_rows(seed: int, tensor_id: int, n_rows: int, row_len: int, dtype: str,
               lo: int, hi: int, denom: float) -> np.ndarray:
    """Entries k/denom with k uniform in [lo, hi]; exactly representable in bf16 and fp32."""
    k = _rng(seed, tensor_id, 0).integers(lo, hi + 1, size=(n_rows, row_len))
    return store(k.astype(np.float64) / denom, dtype)


def _chunk_means(k_store: np.ndarray, cfg: HsaConfig) -> np.ndarray:
    """fp64 mean of the 64 stored keys of every complete chunk: [B, Hkv, Nc, d]."""
    B, H, L, d = k_store.shape
    nc = L // CHUNK
    out = np.empty((B, H, nc, d), dtype=np.float64)
    step = BLOCK_TOKENS // CHUNK
    jobs = [(b, h, c0) for b in range(B) for h in range(H) for c0 in range(0, nc, step)]

    def work(job):
        b, h, c0 = job
        c1 = min(nc, c0 + step)
        blk = to_f64(k_store[b, h, c0 * CHUNK:c1 * CHUNK], cfg.dtype)
        out[b, h, c0:c1] = blk.reshape(c1 - c0, CHUNK, d).mean(axis=1)

    if len(jobs) == 1:
        work(jobs[0])
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, jobs))
    return out


@dataclass
class HsaInputs:
    cfg: HsaConfig
    q_ret: np.ndarray       # [B, Lq, Hkv, d]
    landmarks: np.ndarray   # [B, Hkv, Nc, d]
    q_attn: np.ndarray      # [B, Lq, Hq, d]
    k: np.ndarray           # [B, Hkv, Lkv, d]
    v: np.ndarray           # [B, Hkv, Lkv, d]
    needles: list = field(default_factory=list)   # (b, chunk, owner_row, sigma)


def generate(cfg: HsaConfig, seed: int | None = None, mode: str = "normal") -> HsaInputs:
    """Draw one workload.

    mode:
      "normal"     the recipe in the module docstring.
      "grid"       q_ret and landmarks hold k/8 with k uniform in [-32, 32]; every
                   fp32 partial sum of a d<=128 dot product is then a multiple of
                   1/64 below 2^24/64, so fp32 scoring is exact in any order.
      "grid_small" q_ret and landmarks hold integers in [-2, 2] (many exact ties).
    K, V and q_attn are N(0,1) in every mode.
    """
    seed = cfg.seed if seed is None else seed
    B, Lq, Hq, Hkv, d = cfg.batch, cfg.q_len, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    L, nc = cfg.kv_len, cfg.n_chunks

    k = _normal_rows(seed, T_K, B * Hkv * L, d, cfg.dtype).reshape(B, Hkv, L, d)
    v = _normal_rows(seed, T_V, B * Hkv * L, d, cfg.dtype).reshape(B, Hkv, L, d)
    q_attn = _normal_rows(seed, T_QATTN, B * Lq, Hq * d, cfg.dtype).reshape(B, Lq, Hq, d)

    if mode == "normal":
        q_ret = _normal_rows(seed, T_QRET, B * Lq, Hkv * d, cfg.dtype).reshape(B, Lq, Hkv, d)
        lm = _chunk_means(k, cfg)
        if cfg.noise_std > 0:
            noise = _rng(seed, T_NOISE, 0).standard_normal(lm.shape) * cfg.noise_std
            lm += noise
        needles = _plant_needles(cfg, seed, q_ret, lm)
        landmarks = store(lm, cfg.dtype)
    elif mode == "grid":
        q_ret = _grid_rows(seed, T_QRET, B * Lq, Hkv * d, cfg.dtype, -32, 32, 8.0).reshape(B, Lq, Hkv, d)
        landmarks = _grid_rows(seed, T_NOISE, B * Hkv * nc, d, cfg.dtype, -32, 32, 8.0).reshape(B, Hkv, nc, d)
        needles = []
    elif mode == "grid_small":
        q_ret = _grid_rows(seed, T_QRET, B * Lq, Hkv * d, cfg.dtype, -2, 2, 1.0).reshape(B, Lq, Hkv, d)
        landmarks = _grid_rows(seed, T_NOISE, B * Hkv * nc, d, cfg.dtype, -2, 2, 1.0).reshape(B, Hkv, nc, d)
        needles = []
    else:
        raise ValueError(mode)
    return HsaInputs(cfg, q_ret, landmarks, q_attn, k, v, needles)


def cotangent(cfg: HsaConfig, seed: int | None = None) -> np.ndarray:
    """Output cotangent dout [B, Lq, Hq, d] for the backward: stored N(0,1) values
    drawn like q_attn from their own stream."""
    seed = cfg.seed if seed is None else seed
    B, Lq, Hq, d = cfg.batch, cfg.q_len, cfg.n_q_heads, cfg.head_dim
    return _normal_rows(seed, T_DOUT, B * Lq, Hq * d, cfg.dtype).reshape(B, Lq, Hq, d)


def _plant_needles(cfg: HsaConfig, seed: int, q_ret_store: np.ndarray, lm: np.ndarray) -> list:
    rng = _rng(seed, T_NEEDLE, 0)
    B, Lq = cfg.batch, cfg.q_len
    nc = cfg.n_chunks
    sig = cfg.sigma_l
    planted = []

    def boost(b, chunk, row, nsig):
        q = to_f64(q_ret_store[b, row], cfg.dtype)          # [Hkv, d]
        nrm = np.linalg.norm(q, axis=-1, keepdims=True)
        nrm[nrm == 0] = 1.0
        lm[b, :, chunk, :] += nsig * sig * q / nrm
        planted.append((b, int(chunk), int(row), float(nsig)))

    if cfg.decode_needles:
        # every query row owns 32 distinct chunks: one at +5 sigma, 31 at +3 sigma
        per = 32
        for b in range(B):
            chosen = rng.choice(nc, size=min(nc, per * Lq), replace=False)
            for r in range(Lq):
                own = chosen[r * per:(r + 1) * per]
                for j, c in enumerate(own):
                    boost(b, c, r, 5.0 if j == 0 else 3.0)
        return planted

    if cfg.n_needles <= 0:
        return planted
    last_row_pos = cfg.q_pos0 + Lq - 1
    visible = min(last_row_pos // CHUNK, nc)          # chunks 0..visible-1 can be seen
    hi = visible - 1 if cfg.needle_hi < 0 else min(cfg.needle_hi, visible - 1)
    if hi < 0:
        return planted
    for b in range(B):
        chunks = rng.choice(hi + 1, size=min(cfg.n_needles, hi + 1), replace=False)
        for c in chunks:
            r_min = max(0, CHUNK * (int(c) + 1) - cfg.q_pos0)
            row = int(rng.integers(r_min, Lq))
            boost(b, c, row, cfg.needle_sigma)
    return planted


def shrink(cfg: HsaConfig, q_len: int | None = None, kv_len: int | None = None, **kw) -> HsaConfig:
    """Smaller variant of a workload for parity sweeps (needles clipped to what is visible)."""
    q_len = cfg.q_len if q_len is None else q_len
    kv_len = cfg.kv_len if kv_len is None else kv_len
    over = dict(q_len=q_len, kv_len=kv_len)
    if cfg.q_pos0 == cfg.kv_len:            # decode style: rows sit right after the history
        over["q_pos0"] = kv_len
    elif cfg.q_pos0 > 0:                   # appended rows: keep them at the end of the history
        over["q_pos0"] = kv_len - q_len
    if cfg.n_needles:
        over["n_needles"] = max(1, min(cfg.n_needles, kv_len // CHUNK // 8))
        over["needle_hi"] = -1
    over.update(kw)
    return replace(cfg, **over)
