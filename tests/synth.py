"""Seeded synthetic inputs for the verify-and-sample step.

This module is shared by the tests, the smoke check and the benchmark; it
feeds both the HIP library and the oracle and holds none of the verify
step's arithmetic.  It plays the parts of the two models that the pages
treat as given (Phase 1 draft sampling and Phase 2 target scoring of
Algorithm 1 in "Fast Inference from Transformers via Speculative Decoding",
"Speculative Sampling: The Core Algorithm"): it draws logits, forms the
draft distribution q = softmax(z_q / T) in fp64 exactly as a draft model
would, samples the draft tokens x_i ~ q_i, and draws the uniforms.

Uniforms are u = (k + 1) * 2^-24 with k uniform on [0, 2^24 - 1), so every
u is an exact fp32 value in [2^-24, 1 - 2^-24].

Workloads (the five configurations the benchmark and the parity tests use):
  c1  B=1 x trials, gamma=4, V=8, fp32/fp32, z_q ~ N(0,1), z_p = z_q + 0.7 N,
      T=1.0; one fixed pair of distributions per position, fresh drafts and
      uniforms per trial (the chi-square workload).
  c2  B=8, gamma=4, V=32000, fp32/fp32, z_q ~ N(0, 2^2), z_p = z_q + 0.5 N, T=1.
  c3  B=64, gamma=4, V=128256, bf16 logits / fp32 probs, z_q ~ N(0, 3^2),
      z_p = z_q + N, T=0.8; also run in greedy mode on the same inputs.
  c4  B=256, gamma=8, V=152064, bf16/bf16, z_q ~ N(0, 3^2), per-sequence
      eps ~ U(0.2, 2.0), z_p = z_q + eps N, T=1.0.
  c5  B=32, gamma=16, V=256000, bf16/bf16, z_q = 4 Gumbel(0,1),
      z_p = z_q + 1.5 N, T=0.7; each draft row is "disjoint" with
      probability 0.01 (row (0,0) always): z_p's values at q's top-64
      indices are swapped with 64 random indices outside that set.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

FP32 = "fp32"
BF16 = "bf16"


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    gamma: int
    V: int
    logits_dtype: str
    probs_dtype: str
    T: float
    kind: str  # "c1" .. "c5": which construction


CONFIGS = {
    "c1": Config("c1", 100_000, 4, 8, FP32, FP32, 1.0, "c1"),
    "c2": Config("c2", 8, 4, 32_000, FP32, FP32, 1.0, "c2"),
    "c3": Config("c3", 64, 4, 128_256, BF16, FP32, 0.8, "c3"),
    "c4": Config("c4", 256, 8, 152_064, BF16, BF16, 1.0, "c4"),
    "c5": Config("c5", 32, 16, 256_000, BF16, BF16, 0.7, "c5"),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((b >> 16) & 1) + np.uint32(0x7FFF)
    return ((b + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _cast(a64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == FP32:
        return a64.astype(np.float32)
    return f32_to_bf16_bits(a64.astype(np.float32))


def _softmax64(z: np.ndarray, T: float) -> np.ndarray:
    """Draft-model output distribution (stands in for M_q's softmax)."""
    z = z.astype(np.float64) / T
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def _sample_rows(rng: np.random.Generator, q: np.ndarray) -> np.ndarray:
    """x_i ~ q_i for each row of q (the draft model's own sampling)."""
    c = np.cumsum(q, axis=-1)
    r = rng.random(q.shape[0]) * c[:, -1]
    x = np.array([np.searchsorted(c[i], r[i], side="right") for i in range(q.shape[0])])
    return np.minimum(x, q.shape[1] - 1).astype(np.int32)


def draw_uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    k = rng.integers(0, (1 << 24) - 1, size=shape, dtype=np.int64)
    return ((k + 1).astype(np.float64) * 2.0 ** -24).astype(np.float32)


def _one_sequence(cfg: Config, gamma: int, V: int, seq_seed, force_disjoint: bool) -> tuple:
    rng = np.random.default_rng(seq_seed)
    G1 = gamma + 1
    f32n = cfg.logits_dtype == BF16  # float32 normals are plenty for bf16 logits
    def normal(shape):
        return rng.standard_normal(shape, dtype=np.float32 if f32n else np.float64)

    if cfg.kind == "c2":
        zq = 2.0 * normal((G1, V))
        zp = zq + 0.5 * normal((G1, V))
    elif cfg.kind == "c3":
        zq = 3.0 * normal((G1, V))
        zp = zq + 1.0 * normal((G1, V))
    elif cfg.kind == "c4":
        eps = rng.uniform(0.2, 2.0)
        zq = 3.0 * normal((G1, V))
        zp = zq + np.float32(eps) * normal((G1, V))
    elif cfg.kind == "c5":
        # Gumbel(0,1) = -log(E) with E ~ Exp(1)
        e = rng.standard_exponential((G1, V), dtype=np.float32)
        zq = -4.0 * np.log(np.maximum(e, np.float32(1e-30)))
        zp = zq + 1.5 * normal((G1, V))
    else:
        raise ValueError(cfg.kind)

    disjoint = np.zeros(gamma, dtype=bool)
    if cfg.kind == "c5":
        disjoint = rng.random(gamma) < 0.01
        disjoint[0] |= force_disjoint
        k = min(64, V // 2)
        for i in np.nonzero(disjoint)[0]:
            top = np.argpartition(-zq[i], k - 1)[:k]
            mask = np.ones(V, dtype=bool)
            mask[top] = False
            others = rng.choice(np.nonzero(mask)[0], size=k, replace=False)
            a, b = zp[i, top].copy(), zp[i, others].copy()
            zp[i, top], zp[i, others] = b, a

    q = _softmax64(zq[:gamma], cfg.T)
    x = _sample_rows(rng, q)
    u = draw_uniforms(rng, G1)
    return zp, q, x, u, disjoint


def make_inputs(name: str, seed: int, *, B: int | None = None, gamma: int | None = None,
                V: int | None = None, threads: int | None = None) -> dict:
    """Seeded inputs for configuration ``name`` (c2..c5), optionally resized.

    Returns host arrays: target_logits [B, gamma+1, V] (float32, or uint16
    bf16 bits), draft_probs [B, gamma, V] (likewise), draft_tokens [B, gamma]
    int32, uniforms [B, gamma+1] float32, plus temperature and metadata.
    """
    if name == "c1":
        return make_c1(seed, trials=B or CONFIGS["c1"].B)
    cfg = CONFIGS[name]
    B = cfg.B if B is None else B
    gamma = cfg.gamma if gamma is None else gamma
    V = cfg.V if V is None else V
    G1 = gamma + 1
    seeds = np.random.SeedSequence([seed, sum(map(ord, name))]).spawn(B)
    zl = np.empty((B, G1, V), dtype=np.float32 if cfg.logits_dtype == FP32 else np.uint16)
    qp = np.empty((B, gamma, V), dtype=np.float32 if cfg.probs_dtype == FP32 else np.uint16)
    x = np.empty((B, gamma), dtype=np.int32)
    u = np.empty((B, G1), dtype=np.float32)
    disjoint = np.zeros((B, gamma), dtype=bool)

    def work(b):
        # Row (0, 0) of c5 is always disjoint so the near-total-rejection path
        # is exercised in every batch.
        zp_b, q_b, x_b, u_b, d_b = _one_sequence(cfg, gamma, V, seeds[b], b == 0)
        zl[b] = _cast(zp_b, cfg.logits_dtype)
        qp[b] = _cast(q_b, cfg.probs_dtype)
        x[b] = x_b
        u[b] = u_b
        disjoint[b] = d_b

    nthreads = threads or min(16, os.cpu_count() or 1)
    if B * G1 * V < 1 << 20 or nthreads == 1:
        for b in range(B):
            work(b)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, range(B)))
    return {
        "name": name, "B": B, "gamma": gamma, "V": V, "temperature": cfg.T,
        "logits_dtype": cfg.logits_dtype, "probs_dtype": cfg.probs_dtype,
        "target_logits": zl, "draft_probs": qp, "draft_tokens": x, "uniforms": u,
        "disjoint_rows": disjoint,
    }


def make_c1(seed: int, trials: int = 100_000, iid: bool = False) -> dict:
    """c1: one fixed (z_q, z_p) pair per position, ``trials`` fresh draws of
    drafts and uniforms, laid out as a batch of ``trials`` identical sequences.
    With ``iid`` every position uses the same pair of rows (for the
    expected-tokens check under i.i.d. acceptance)."""
    cfg = CONFIGS["c1"]
    gamma, V, T = cfg.gamma, cfg.V, cfg.T
    G1 = gamma + 1
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xC1]))
    if iid:
        zq1 = rng.standard_normal(V)
        zp1 = zq1 + 0.7 * rng.standard_normal(V)
        zq = np.tile(zq1, (G1, 1))
        zp = np.tile(zp1, (G1, 1))
    else:
        zq = rng.standard_normal((G1, V))
        zp = zq + 0.7 * rng.standard_normal((G1, V))
    zp32 = zp.astype(np.float32)
    q64 = _softmax64(zq[:gamma], T)
    q32 = q64.astype(np.float32)
    # draft tokens per trial and position, sampled from the fp64 draft rows
    cq = np.cumsum(q64, axis=-1)
    r = rng.random((trials, gamma)) * cq[None, :, -1]
    x = np.empty((trials, gamma), dtype=np.int32)
    for i in range(gamma):
        x[:, i] = np.minimum(np.searchsorted(cq[i], r[:, i], side="right"), V - 1)
    u = draw_uniforms(rng, (trials, G1))
    return {
        "name": "c1", "B": trials, "gamma": gamma, "V": V, "temperature": T,
        "logits_dtype": FP32, "probs_dtype": FP32,
        "target_logits": np.ascontiguousarray(np.broadcast_to(zp32, (trials, G1, V))),
        "draft_probs": np.ascontiguousarray(np.broadcast_to(q32, (trials, gamma, V))),
        "draft_tokens": x, "uniforms": u,
        "rows_zp": zp32, "rows_q": q32,
        "disjoint_rows": np.zeros((trials, gamma), dtype=bool),
    }


def make_position_models(L: int, V: int, seed: int, dtype: str = FP32, T: float = 1.0,
                         sigma: float = 1.0, shift: float = 0.8, iid: bool = False):
    """Position-only target and draft "models" for the multi-step driver:
    for each absolute position t, z_q[t] ~ N(0, sigma^2), z_p[t] = z_q[t] +
    shift * N(0, 1); q[t] = softmax(z_q[t] / T) in fp64 (the draft's output),
    cast to ``dtype``.  ``iid``: one row pair for every position.  Returns the
    driver's PositionOnlyModels."""
    from exact_rejection_sampling_temp_amd.driver import PositionOnlyModels
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xF4]))
    n = 1 if iid else L
    zq = sigma * rng.standard_normal((n, V))
    zp = zq + shift * rng.standard_normal((n, V))
    if iid:
        zq = np.repeat(zq, L, 0)
        zp = np.repeat(zp, L, 0)
    q64 = _softmax64(zq, T)
    zp_c = _cast(zp, dtype)
    return PositionOnlyModels(target_logits=np.ascontiguousarray(zp_c), draft_probs=_cast(q64, dtype),
                              draft_probs64=q64, temperature=T)


def standardize_draft_topk(d: dict, k: int, seed: int) -> dict:
    """The draft model's own top-k standardisation (its part of "Standardized
    Sampling"): each draft row keeps its k largest probabilities (ties in
    index order), renormalised in fp64 and cast back; the draft tokens are
    redrawn from the standardised rows.  Returns a new input dict."""
    out = dict(d)
    q = d["draft_probs"]
    q64 = (q.astype(np.float64) if q.dtype == np.float32 else bf16_bits_to_f32(q).astype(np.float64))
    B, G, V = q64.shape
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xF2]))
    qs = np.zeros_like(q64)
    x = np.empty((B, G), np.int32)
    for b in range(B):
        for i in range(G):
            keep = np.argsort(-q64[b, i], kind="stable")[:k]
            row = np.zeros(V)
            row[keep] = q64[b, i, keep]
            row /= row.sum()
            qs[b, i] = row
        x[b] = _sample_rows(rng, qs[b])
    out["draft_probs"] = _cast(qs, FP32 if q.dtype == np.float32 else BF16)
    out["draft_tokens"] = x
    return out
