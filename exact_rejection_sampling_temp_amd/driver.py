"""Multi-step speculative decoding over position-only models.

The orchestration loop around the verify step ("Fast Inference from
Transformers via Speculative Decoding", summary page, the system overview's
"Orchestration Loop": each iteration drafts gamma tokens, verifies them with
one parallel target evaluation, and extends the prefix by n + 1 tokens; the
KV-cache rollback of "Speculative Decoding Paper Breakdown: Lossless
Draft-and-Verify Acceleration for Autoregressive Transformers", section 5,
"Production Engineering Takeaways": after a rejection at k the sequence's
length pointer becomes base + k + 1 and nothing else is undone).

The "models" here are position-only: the target's logits and the draft's
probabilities at absolute position t do not depend on the tokens before t.
That keeps the loop exact to check (every emitted token at position t must
follow p_t, whatever happened before) while exercising everything the loop
does: per-stream length pointers, drafting from the current pointer,
gathering the gamma + 1 target rows, the verify call, the rollback, and the
stop at a maximum length.

gamma is chosen with ``optimal_gamma`` ("Choosing gamma: The Optimal Number
of Guesses", Theorem 3.8): the integer maximising
(1 - alpha^(gamma+1)) / ((1 - alpha) (gamma c + 1)).

The verify step is the GPU library (``GpuVerifier``: tables resident on the
device, rows gathered there, then ``spec_verify``); a caller may pass any
function verify(pos, x, u, lenience) -> (n_accepted, out_tokens) (the tests
pass the CPU reference to compare whole streams).  The draft sampling is
the draft model's part and runs on the host, vectorised, from the fp64
draft rows.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


def walltime_improvement(alpha: float, gamma: int, c: float) -> float:
    """Expected tokens per iteration over the iteration's cost in target
    runs, (1 - alpha^(gamma+1)) / ((1 - alpha)(gamma c + 1)) (Theorem 3.8)."""
    tokens = float(gamma + 1) if alpha >= 1.0 else (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)
    return tokens / (gamma * c + 1.0)


def optimal_gamma(alpha: float, c: float, gamma_max: int = 63) -> int:
    """The gamma in 1..gamma_max with the largest walltime improvement,
    found by evaluating every candidate (the page's recipe); ties go to the
    smaller gamma.  alpha in [0, 1], c >= 0."""
    if not (0.0 <= alpha <= 1.0) or not (c >= 0.0) or gamma_max < 1:
        raise ValueError("need 0 <= alpha <= 1, c >= 0, gamma_max >= 1")
    best, best_v = 1, -math.inf
    for g in range(1, gamma_max + 1):
        v = walltime_improvement(alpha, g, c)
        if v > best_v:
            best, best_v = g, v
    return best


@dataclass
class PositionOnlyModels:
    """Target logits z[t] ([L, V], float32 or bf16 bits as uint16) and draft
    probabilities q[t] ([L, V] float32 or bf16 bits, with the fp64 rows the
    draft samples from) for absolute positions t = 0 .. L-1."""
    target_logits: np.ndarray
    draft_probs: np.ndarray
    draft_probs64: np.ndarray
    temperature: float = 1.0

    @property
    def length(self) -> int:
        return self.target_logits.shape[0]

    @property
    def vocab(self) -> int:
        return self.target_logits.shape[1]


def batched_icdf(cq: np.ndarray, rows: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """For each k the smallest j with cq[rows[k], j] > keys[k] (V - 1 if none):
    np.searchsorted(cq[row], key, side="right") for many rows at once, by a
    vectorised binary search over the row."""
    V = cq.shape[1]
    lo = np.zeros(keys.shape, np.int64)
    hi = np.full(keys.shape, V, np.int64)
    for _ in range(int(V).bit_length() + 1):
        open_ = lo < hi
        if not open_.any():
            break
        mid = (lo + hi) // 2
        right = cq[rows, np.minimum(mid, V - 1)] <= keys
        lo = np.where(open_ & right, mid + 1, lo)
        hi = np.where(open_ & ~right, mid, hi)
    return np.minimum(lo, V - 1)


def draft_tokens(cq: np.ndarray, pos: np.ndarray, u: np.ndarray) -> np.ndarray:
    """The draft model's guesses: x_i ~ q_{pos_i} by inverse CDF of the fp64
    draft row (cq its running sums) with the uniform u_i."""
    keys = u * cq[pos, -1]
    return batched_icdf(cq, pos, keys).astype(np.int32)


class GpuVerifier:
    """The library's verify step with the position-only tables resident on the
    GPU: each call gathers the gamma + 1 target rows and gamma draft rows of
    every stream on the device, then runs spec_verify."""

    def __init__(self, models: PositionOnlyModels, device="cuda"):
        import torch
        import exact_rejection_sampling_temp_amd as sv
        self.torch, self.sv, self.device = torch, sv, device

        def dev(a):
            t = torch.from_numpy(np.ascontiguousarray(a))
            if a.dtype == np.uint16:
                t = t.view(torch.bfloat16)
            return t.to(device)
        self.z = dev(models.target_logits)
        self.q = dev(models.draft_probs)
        self.T = models.temperature
        self.aux = None

    def __call__(self, pos: np.ndarray, x: np.ndarray, u: np.ndarray, lenience: float = 1.0):
        torch = self.torch
        p = torch.from_numpy(pos).to(self.device)
        zl = self.z[p]                                    # [B, gamma+1, V]
        qp = self.q[p[:, :-1]]                            # [B, gamma, V]
        n, out = self.sv.spec_verify(zl, qp, torch.from_numpy(x).to(self.device),
                                     torch.from_numpy(u).to(self.device), self.T, "sample",
                                     lenience=lenience, aux=self.aux)
        return n.cpu().numpy(), out.cpu().numpy()


def speculative_decode(models: PositionOnlyModels, streams: int, max_len: int, gamma: int, seed: int,
                       verify=None, lenience: float = 1.0) -> dict:
    """Decode ``streams`` independent sequences of ``max_len`` tokens.

    Every iteration: each unfinished stream drafts gamma tokens at positions
    t .. t+gamma-1 (t its length pointer), the verify step sees the target
    rows t .. t+gamma and the draft rows t .. t+gamma-1, and the stream keeps
    x_0 .. x_{n-1} and the correction / bonus token, so its pointer moves to
    t + n + 1 (tokens past max_len are dropped).  Finished streams leave the
    batch.  Position-only models need L >= max_len + gamma rows.
    Returns the token streams [streams, max_len], the iterations each stream
    took, and the per-iteration accepted counts."""
    verify = verify or GpuVerifier(models)
    if models.length < max_len + gamma:
        raise ValueError("the position-only models need max_len + gamma rows")
    rng = np.random.default_rng(seed)
    cq = np.cumsum(models.draft_probs64, axis=-1)
    # the per-stream bookkeeping below is vectorised; only small arrays
    # ([B, gamma+1]) cross to and from the device each iteration
    tokens = np.full((streams, max_len), -1, np.int32)
    ptr = np.zeros(streams, np.int64)
    iters = np.zeros(streams, np.int64)
    accepted = []
    while True:
        live = np.nonzero(ptr < max_len)[0]
        if live.size == 0:
            break
        B = live.size
        pos = ptr[live, None] + np.arange(gamma + 1)[None, :]                    # [B, gamma+1]
        x = draft_tokens(cq, pos[:, :gamma], rng.random((B, gamma)))
        # verify uniforms as the generator makes them: (k+1) 2^-24
        u = ((rng.integers(0, (1 << 24) - 1, (B, gamma + 1)) + 1) * 2.0 ** -24).astype(np.float32)
        n, out = verify(pos, x, u, lenience)
        if np.any(n < 0):
            raise RuntimeError("a draft token fell outside the vocabulary")
        k = n.astype(np.int64) + 1
        cols = ptr[live, None] + np.arange(gamma + 1)[None, :]
        keep = (np.arange(gamma + 1)[None, :] < k[:, None]) & (cols < max_len)
        rr, cc = np.nonzero(keep)
        tokens[live[rr], cols[rr, cc]] = out[rr, cc]
        ptr[live] += k                                                          # length-pointer rollback
        iters[live] += 1
        accepted.append(n.copy())
    return {"tokens": tokens, "iterations": iters, "accepted": accepted}


def estimate_alpha(models: PositionOnlyModels, positions, device="cuda") -> float:
    """alpha = the mean of beta_t = sum_v min(p_t, q_t) over the given
    positions, measured with the library's acceptance-rate telemetry (one call,
    one "sequence" per position with gamma = 1) -- the pages' way of getting
    alpha from the two models ("Computing alpha from p and q", Corollary 3.6)."""
    import torch
    import exact_rejection_sampling_temp_amd as sv
    pos = np.asarray(positions, np.int64)
    if pos.size == 0 or pos.max() + 1 >= models.length:
        raise ValueError("positions must leave one row after each")
    ver = GpuVerifier(models, device)
    p = torch.from_numpy(np.stack([pos, pos + 1], 1)).to(device)
    zl = ver.z[p]
    qp = ver.q[p[:, :1]]
    B = pos.size
    beta = torch.empty((B, 1), dtype=torch.float64, device=device)
    alpha = torch.empty(1, dtype=torch.float64, device=device)
    sv.spec_verify(zl, qp, torch.zeros((B, 1), dtype=torch.int32, device=device),
                   torch.full((B, 2), 0.5, dtype=torch.float32, device=device), models.temperature, "sample",
                   aux={"beta": beta, "alpha": alpha})
    return float(alpha.cpu()[0])
