"""The multi-step driver over position-only models (CPU: the verify step is
the fp64 oracle).  With position-only models the target's distribution at
absolute position t is p_t whatever came before, so an exact decoding loop
must emit, at every position, a token distributed as p_t ("Fast Inference
from Transformers via Speculative Decoding", summary page, "Why This
Procedure Preserves the Target Distribution"), and, with the same pair of
rows at every position, deliver (1 - alpha^(gamma+1)) / (1 - alpha) tokens
per iteration on average ("Expected Number of Generated Tokens",
Equation 1).  gamma* follows Theorem 3.8 ("Choosing gamma")."""
import math

import numpy as np
import pytest
import scipy.stats

import oracle
from oracle import analysis
import exact_rejection_sampling_temp_amd as sv
from exact_rejection_sampling_temp_amd import driver
from tests import synth
from tests.laws import target_law


class OracleVerifier:
    """The fp64 reference as the driver's verify step (host tables)."""

    def __init__(self, models):
        self.m = models

    def __call__(self, pos, x, u, lenience=1.0):
        zl = self.m.target_logits[pos]
        qp = self.m.draft_probs[pos[:, :-1]]
        r = oracle.spec_verify_ref(zl, qp, x, u, self.m.temperature, aux=False, lenience=lenience)
        return r["n_accepted"], r["out_tokens"]


def _chisq(counts, probs):
    exp = probs * counts.sum()
    keep = exp >= 5
    c = np.append(counts[keep], counts[~keep].sum())
    e = np.append(exp[keep], exp[~keep].sum())
    if e[-1] == 0:
        c, e = c[:-1], e[:-1]
    return scipy.stats.chisquare(c, e * c.sum() / e.sum()).pvalue


def test_batched_icdf_matches_searchsorted():
    rng = np.random.default_rng(9)
    for V in (1, 2, 7, 1000):
        q = rng.random((5, V))
        q[:, ::3] = 0.0
        cq = np.cumsum(q, axis=-1)
        rows = rng.integers(0, 5, 4000)
        keys = rng.random(4000) * cq[rows, -1]
        keys[:50] = cq[rows[:50], rng.integers(0, V, 50)]   # keys on the boundaries
        want = np.array([min(np.searchsorted(cq[r], k, side="right"), V - 1) for r, k in zip(rows, keys)])
        assert np.array_equal(driver.batched_icdf(cq, rows, keys), want)


def test_optimal_gamma_is_the_argmax_of_theorem_3_8():
    """gamma* by the driver equals a brute-force argmax of the oracle-side
    closed form, and moves as the page says: non-decreasing in alpha,
    non-increasing in c."""
    for a in np.linspace(0.05, 0.95, 19):
        prev = None
        for c in (0.0, 0.01, 0.02, 0.05, 0.1, 0.2, 0.5):
            vals = [analysis.walltime_improvement(a, g, c) for g in range(1, sv.SV_MAX_GAMMA + 1)]
            want = int(np.argmax(vals)) + 1
            got = driver.optimal_gamma(a, c)
            assert got == want, (a, c, got, want)
            if prev is not None:
                assert got <= prev
            prev = got
    for c in (0.01, 0.05, 0.1):
        gs = [driver.optimal_gamma(a, c) for a in np.linspace(0.05, 0.95, 19)]
        assert all(g1 <= g2 for g1, g2 in zip(gs, gs[1:]))
    with pytest.raises(ValueError):
        driver.optimal_gamma(1.5, 0.1)


def test_streams_follow_p_at_every_position():
    """20 000 streams of 10 tokens, V = 6, gamma = 3: the token at each
    position is distributed as p_t (chi-square per position, fixed seed)."""
    L, V, gamma = 10, 6, 3
    m = synth.make_position_models(L + gamma, V, seed=3)
    p64 = target_law(m)
    r = driver.speculative_decode(m, 20_000, L, gamma, seed=4, verify=OracleVerifier(m))
    tok = r["tokens"]
    assert np.all(tok >= 0)
    for t in range(L):
        assert _chisq(np.bincount(tok[:, t], minlength=V).astype(float), p64[t]) > 1e-3, t
    # each iteration moves a stream by 1 .. gamma + 1 tokens
    acc = np.concatenate(r["accepted"])
    assert acc.min() >= 0 and acc.max() <= gamma


@pytest.mark.parametrize("gamma", [2, 5])
def test_tokens_per_iteration_match_equation_1(gamma):
    """Same rows at every position: mean tokens per iteration within 4 sigma
    of (1 - alpha^(gamma+1)) / (1 - alpha), alpha = sum min(p, q)."""
    L, V = 40, 8
    m = synth.make_position_models(L + gamma, V, seed=5, iid=True)
    p64 = target_law(m)
    alpha = analysis.acceptance_rate(p64[0], m.draft_probs.astype(np.float64)[0])
    r = driver.speculative_decode(m, 3000, L, gamma, seed=6, verify=OracleVerifier(m))
    k = np.concatenate(r["accepted"]).astype(float) + 1.0
    E = analysis.expected_tokens(alpha, gamma)
    assert abs(k.mean() - E) < 4 * k.std() / math.sqrt(k.size), (k.mean(), E)
    # and the iteration count: each stream needs about L / E iterations
    assert abs(r["iterations"].mean() - L / E) < 0.15 * L / E


def test_lenient_driver_bounds_each_position_by_p_over_l():
    """With lenience l the emitted law at each position stays below p_t / l
    (the page's guarantee) and accepts more per iteration."""
    L, V, gamma, l = 6, 5, 2, 0.5
    m = synth.make_position_models(L + gamma, V, seed=7)
    p64 = target_law(m)
    r = driver.speculative_decode(m, 20_000, L, gamma, seed=8, verify=OracleVerifier(m), lenience=l)
    r1 = driver.speculative_decode(m, 20_000, L, gamma, seed=8, verify=OracleVerifier(m))
    for t in range(L):
        law = np.bincount(r["tokens"][:, t], minlength=V) / 20_000
        assert np.all(law <= p64[t] / l + 4 * np.sqrt(p64[t] / l / 20_000) + 1e-3)
    assert np.concatenate(r["accepted"]).mean() > np.concatenate(r1["accepted"]).mean()
