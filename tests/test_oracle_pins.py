"""Pins for the fp64 oracle: checks against what the pages and the mathematics
fix, independent of the oracle's own code.

Sources (page title, section):
  [FI] "Fast Inference from Transformers via Speculative Decoding" (summary)
  [TM] "Speculative Decoding: Two Models, One Output"
  [PB] "Speculative Decoding Paper Breakdown: Lossless Draft-and-Verify
       Acceleration for Autoregressive Transformers"
  [ST] "The exact decoding shortcut that burns compute when guesses miss"

Every check here is one of: a value printed on the pages (tests/golden), a
library routine the step reduces to (scipy softmax, numpy argmax and
searchsorted), an exact law by exhaustive midpoint grids on tiny
vocabularies, a closed form, an invariant, or a seeded statistical test with
a fixed pass/fail outcome.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from oracle import analysis
from tests import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _tol(digits):
    return 0.5 * 10.0 ** (-digits) + 1e-12


# ---------------------------------------------------------------- printed values

def test_printed_expected_tokens():
    g = _golden("printed_values.json")
    for e in g["expected_tokens"]:
        got = analysis.expected_tokens(e["alpha"], e["gamma"])
        assert abs(got - e["value"]) <= _tol(e["digits"]), (e, got)
    for e in g["expected_tokens_limit"]:
        got = analysis.expected_tokens(e["alpha"], 10_000)
        assert abs(got - e["value"]) <= _tol(e["digits"]) + 1e-6, (e, got)


def test_printed_walltime_and_operations():
    g = _golden("printed_values.json")
    for e in g["walltime_improvement"]:
        got = analysis.walltime_improvement(e["alpha"], e["gamma"], e["c"])
        assert abs(got - e["value"]) <= _tol(e["digits"]), (e, got)
    for e in g["operations_factor"]:
        got = analysis.operations_factor(e["alpha"], e["gamma"], e["c_hat"])
        assert abs(got - e["value"]) <= _tol(e["digits"]), (e, got)


def test_excluded_row_is_really_inconsistent():
    # [PB] section 4 table, third row: 2.53 tokens does not follow from
    # Equation 1 at gamma=4 but does at gamma=3.
    assert abs(analysis.expected_tokens(0.7, 4) - 2.53) > 0.2
    assert abs(analysis.expected_tokens(0.7, 3) - 2.53) < 0.005


# ------------------------------------------------- library routines the steps reduce to

@pytest.mark.parametrize("T", [0.7, 1.0, 1.3])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_softmax_matches_scipy(T, dtype):
    rng = np.random.default_rng(11)
    for V in (1, 2, 7, 1000, 32_000):
        z = (3.0 * rng.standard_normal(V)).astype(np.float32)
        if dtype == "bf16":
            bits = synth.f32_to_bf16_bits(z)
            z64 = synth.bf16_bits_to_f32(bits).astype(np.float64)
            p = oracle.softmax_row(bits, T)
        else:
            z64 = z.astype(np.float64)
            p = oracle.softmax_row(z, T)
        ref = scipy.special.softmax(z64 / np.float64(np.float32(T)))
        np.testing.assert_allclose(p, ref, rtol=1e-12, atol=1e-300)
        assert abs(p.sum() - 1.0) < 1e-12


def test_softmax_neg_inf_entries_are_zero():
    z = np.array([0.0, -np.inf, 1.0, -np.inf], dtype=np.float32)
    p = oracle.softmax_row(z, 1.0)
    assert p[1] == 0.0 and p[3] == 0.0
    np.testing.assert_allclose(p[[0, 2]], scipy.special.softmax([0.0, 1.0]), rtol=1e-14)


def test_argmax_first_occurrence_matches_numpy():
    rng = np.random.default_rng(12)
    for V in (1, 3, 64, 5000):
        for _ in range(20):
            # coarse values -> many ties; bf16 rounding adds more
            z = np.round(rng.standard_normal(V) * 2.0).astype(np.float32)
            assert oracle.argmax_row(z) == int(np.argmax(z))
            bits = synth.f32_to_bf16_bits(z * 3.3)
            assert oracle.argmax_row(bits) == int(np.argmax(synth.bf16_bits_to_f32(bits)))


def test_icdf_matches_searchsorted():
    rng = np.random.default_rng(13)
    for V in (1, 2, 5, 100, 4096):
        for _ in range(50):
            w = rng.random(V)
            w[rng.random(V) < 0.4] = 0.0
            if w.sum() == 0:
                w[rng.integers(V)] = 0.5
            u = float(rng.random())
            k, _ = oracle.icdf(w, u)
            ref = int(np.searchsorted(np.cumsum(w), u * w.sum(), side="right"))
            if ref >= V:  # u * total >= total: largest positive-weight index
                ref = int(np.nonzero(w > 0)[0][-1])
            assert k == ref, (V, u)
            assert w[k] > 0.0  # zero-weight tokens are never drawn


def test_icdf_boundary_flags():
    w = np.array([0.25, 0.25, 0.5])
    k, fl = oracle.icdf(w, 0.5)  # exactly on the C_1 boundary: strict '>' picks k=2
    assert k == 2 and fl
    k, fl = oracle.icdf(w, 0.3)
    assert k == 1 and not fl


# ----------------------------------------------------------------- helpers

def _run(zl, q, x, u, T, mode=oracle.SAMPLE):
    return oracle.spec_verify_ref(zl, q, x, u, T, mode)


def _midpoints(n):
    return ((np.arange(n) + 0.5) / n).astype(np.float64)


def _grid_batch(p_logits, q_rows, gamma, fixed_drafts, grid_axes, N):
    """Build a batch enumerating draft tokens and midpoint-grid uniforms.

    p_logits [gamma+1, V] fp32, q_rows [gamma, V] fp32, fixed_drafts: dict
    position -> token for positions whose draft is fixed, the remaining
    position's draft is enumerated over all V tokens.  grid_axes: list of
    uniform indices swept on an N-point midpoint grid (others set to 0.5)."""
    V = p_logits.shape[1]
    enum_pos = [i for i in range(gamma) if i not in fixed_drafts]
    assert len(enum_pos) == 1
    ep = enum_pos[0]
    g = _midpoints(N)
    mesh = np.stack(np.meshgrid(*([g] * len(grid_axes)), indexing="ij"), -1).reshape(-1, len(grid_axes))
    M = mesh.shape[0]
    B = V * M
    x = np.zeros((B, gamma), np.int32)
    for pos, tok in fixed_drafts.items():
        x[:, pos] = tok
    x[:, ep] = np.repeat(np.arange(V, dtype=np.int32), M)
    u = np.full((B, gamma + 1), 0.5, np.float64)
    for j, ax in enumerate(grid_axes):
        u[:, ax] = np.tile(mesh[:, j], V)
    zl = np.ascontiguousarray(np.broadcast_to(p_logits, (B, gamma + 1, V)))
    qq = np.ascontiguousarray(np.broadcast_to(q_rows, (B, gamma, V)))
    # weight of each batch row = q_ep(y) / M
    wts = np.repeat(q_rows[ep].astype(np.float64), M) / M
    return zl, qq, x, u.astype(np.float32), wts


def _rand_pq(rng, V, gamma, shift=0.8):
    zq = rng.standard_normal((gamma + 1, V))
    zp = (zq + shift * rng.standard_normal((gamma + 1, V))).astype(np.float32)
    q = scipy.special.softmax(zq[:gamma], axis=-1).astype(np.float32)
    p = scipy.special.softmax(zp.astype(np.float64), axis=-1)
    return zp, q, p


# ---------------------------------------------------- exact law by exhaustive grids

def test_exact_law_single_position():
    """[FI] Appendix A.1 / [PB] section 3 proof: the emitted token is
    distributed exactly as p.  Enumerate every draft y (weight q(y)) and an
    N x N midpoint grid of (u_accept, u_draw); the law must equal p within the
    grid's resolution (1/N per uniform)."""
    rng = np.random.default_rng(21)
    N = 400
    for V in (2, 3, 6):
        zp, q, p = _rand_pq(rng, V, 1)
        zl, qq, x, u, wts = _grid_batch(zp, q, 1, {}, [0, 1], N)
        r = _run(zl, qq, x, u, 1.0)
        law = np.bincount(r["out_tokens"][:, 0], weights=wts, minlength=V)
        q_total = float(q[0].astype(np.float64).sum())  # fp32 q sums to 1 +- 1e-7
        assert np.max(np.abs(law - p[0] * q_total)) <= 2.0 / N + 1e-6, (law, p[0])


def test_exact_law_rows_are_not_shifted():
    """Off-by-one check on which position's rows are used: gamma=2, the first
    draft is always accepted (q_0(x_0) <= p_0(x_0)), so the second emitted
    token must follow p_1 and, after a full acceptance, the bonus token
    must follow p_2 ([FI] Algorithm 1 Phase 4)."""
    rng = np.random.default_rng(22)
    N = 300
    V = 5
    zp, q, p = _rand_pq(rng, V, 2, shift=1.5)
    y0 = int(np.argmax(p[0] - q[0]))  # p_0(y0) > q_0(y0) -> accepted for any u
    assert p[0][y0] > q[0][y0]
    zl, qq, x, u, wts = _grid_batch(zp, q, 2, {0: y0}, [1, 2], N)
    r = _run(zl, qq, x, u, 1.0)
    out, n = r["out_tokens"], r["n_accepted"]
    assert np.all(n >= 1) and np.all(out[:, 0] == y0)
    law1 = np.bincount(out[:, 1], weights=wts, minlength=V)
    q1 = float(q[1].astype(np.float64).sum())
    assert np.max(np.abs(law1 - p[1] * q1)) <= 2.0 / N + 1e-6
    full = n == 2
    law2 = np.bincount(out[full, 2], weights=wts[full], minlength=V)
    law2 = law2 / law2.sum()
    assert np.max(np.abs(law2 - p[2])) <= 3.0 / N
    # and it is not p_1's law (the rows differ enough to tell)
    assert np.max(np.abs(p[2] - p[1])) > 0.05


def test_two_token_example():
    """[ST] two-token example: the draft over-proposes B, every rejected B is
    corrected to A, acceptance is 60 %, and the composite law equals p."""
    g = _golden("two_token_example.json")
    p = np.array(g["p"])
    q32 = np.array(g["q"], np.float32)
    zp = np.log(p).astype(np.float32)[None, :].repeat(2, 0)
    p_used = scipy.special.softmax(zp[0].astype(np.float64))
    assert abs(analysis.acceptance_rate(p, q32.astype(np.float64)) - g["printed"]["acceptance_rate"]) < 1e-7
    N = 1000
    zl, qq, x, u, wts = _grid_batch(zp, q32[None, :], 1, {}, [0, 1], 40)
    # finer grid on the acceptance uniform only
    zl, qq, x, u, wts = _grid_batch(zp, q32[None, :], 1, {}, [0], N)
    r = _run(zl, qq, x, u, 1.0)
    acc = (r["n_accepted"] == 1)
    assert abs(float(wts[acc].sum()) - g["printed"]["acceptance_rate"]) <= 1.0 / N + 1e-6
    rejected = ~acc
    assert np.all(x[rejected, 0] == 1)            # only B proposals are ever rejected
    assert np.all(r["out_tokens"][rejected, 0] == 0)  # ... and they are corrected to A
    law = np.bincount(r["out_tokens"][:, 0], weights=wts, minlength=2)
    assert np.max(np.abs(law - p_used)) <= 1.0 / N + 1e-6
    # closed form of the proof with these numbers: min(p,q) + max(0,p-q) = p
    assert np.max(np.abs(np.minimum(p, q32) + np.maximum(0, p - q32) - p)) <= g["printed"]["max_numerical_difference"] * 10


def test_zero_residual_falls_back_to_target():
    """[ST] correction_distribution: if max(0, p - q) has (numerically) no
    mass, the corrected token is drawn from p.  q >= p everywhere here."""
    V = 4
    zp = np.log(np.array([0.1, 0.2, 0.3, 0.4])).astype(np.float32)[None, :].repeat(2, 0)
    p = scipy.special.softmax(zp[0].astype(np.float64))
    q = (p * np.array([1.5, 1.0, 1.0, 1.0]) + 0.01).astype(np.float32)[None, :]
    assert np.all(q[0] >= p)
    N = 400
    zl, qq, x, u, wts = _grid_batch(zp, q, 1, {}, [0, 1], N)
    r = _run(zl, qq, x, u, 1.0)
    rej = r["n_accepted"] == 0
    assert rej.any()
    assert np.all(r["resid_mass"][rej] == 0.0)
    law = np.bincount(r["out_tokens"][rej, 0], weights=wts[rej], minlength=V)
    law /= law.sum()
    assert np.max(np.abs(law - p)) <= 2.0 / N


# ------------------------------------------------------------ closed forms

def test_acceptance_identities_and_residual_mass():
    """[FI] Lemma 3.3 / Theorem 3.5 and [PB] section 3: for normalised p, q,
    sum min(p,q) = 1 - DLK(p,q) = 1 - 0.5 sum|p-q| = 1 - sum max(0, p-q), and
    the oracle's residual mass equals that last sum."""
    rng = np.random.default_rng(31)
    for V in (8, 100, 5000):
        for T in (0.7, 1.0):
            zq = 2.0 * rng.standard_normal(V)
            zp = (zq + rng.standard_normal(V)).astype(np.float32)
            p = oracle.softmax_row(zp, T)
            q = scipy.special.softmax(zq / T)
            beta = analysis.acceptance_rate(p, q)
            assert abs(beta - (1.0 - analysis.dlk(p, q))) < 1e-12
            assert abs(beta - (1.0 - 0.5 * np.abs(p - q).sum())) < 1e-12
            assert abs(beta - (1.0 - np.maximum(0.0, p - q).sum())) < 1e-12
            # residual mass reported by the oracle on a forced rejection
            q32 = q.astype(np.float32)
            y = int(np.argmax(q32.astype(np.float64) - p))  # q > p there -> thr < 1
            zl = np.stack([zp, zp])[None]
            r = oracle.spec_verify_ref(zl, q32[None, None, :], np.array([[y]], np.int32),
                                       np.array([[1.0 - 2 ** -24, 0.5]], np.float32), T)
            assert r["n_accepted"][0] == 0
            ref_mass = np.maximum(0.0, p - q32.astype(np.float64)).sum()
            assert abs(r["resid_mass"][0] - ref_mass) < 1e-14
            assert abs(r["thr"][0, 0] - p[y] / float(q32[y])) < 1e-14


def _chisq_pvalue(counts, probs):
    counts = np.asarray(counts, np.float64)
    exp = np.asarray(probs, np.float64) * counts.sum()
    keep = exp >= 5
    c = np.append(counts[keep], counts[~keep].sum())
    e = np.append(exp[keep], exp[~keep].sum())
    if e[-1] == 0:
        c, e = c[:-1], e[:-1]
    e = e * (c.sum() / e.sum())
    return scipy.stats.chisquare(c, e).pvalue


def test_chi_square_c1():
    """The c1 workload (V=8, gamma=4, 100 000 trials): (i) the first emitted
    token ~ p_0, (ii) token j given n >= j ~ p_j, (iii) tokens drawn after a
    rejection at position 0 ~ norm(max(0, p_0 - q_0)), (iv) P(n >= j) =
    prod_{i<j} beta_i ([FI] 'Expected Number of Generated Tokens', capped
    geometric law).  Fixed seed: the outcome is deterministic."""
    d = synth.make_c1(seed=5, trials=100_000)
    r = oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], d["draft_tokens"],
                               d["uniforms"], d["temperature"])
    out, n = r["out_tokens"], r["n_accepted"]
    gamma, V = d["gamma"], d["V"]
    P = scipy.special.softmax(d["rows_zp"].astype(np.float64), axis=-1)
    Q = d["rows_q"].astype(np.float64)
    assert _chisq_pvalue(np.bincount(out[:, 0], minlength=V), P[0]) > 1e-3
    for j in range(1, gamma + 1):
        sel = n >= j
        assert _chisq_pvalue(np.bincount(out[sel, j], minlength=V), P[j]) > 1e-3
    rej0 = n == 0
    res = np.maximum(0.0, P[0] - Q[0])
    assert _chisq_pvalue(np.bincount(out[rej0, 0], minlength=V), res / res.sum()) > 1e-3
    beta = np.minimum(P[:gamma], Q).sum(-1)
    surv = np.concatenate([[1.0], np.cumprod(beta)])
    pn = surv[:-1] * (1 - beta)
    pn = np.append(pn, surv[-1])
    assert _chisq_pvalue(np.bincount(n, minlength=gamma + 1), pn) > 1e-3


def test_expected_tokens_monte_carlo():
    """[FI] Equation 1 under i.i.d. acceptance: with the same pair of rows at
    every position, mean(n + 1) must be within 4 sigma of
    (1 - alpha^(gamma+1)) / (1 - alpha), alpha = sum min(p, q)."""
    d = synth.make_c1(seed=6, trials=100_000, iid=True)
    r = oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], d["draft_tokens"],
                               d["uniforms"], d["temperature"])
    p = scipy.special.softmax(d["rows_zp"][0].astype(np.float64))
    alpha = analysis.acceptance_rate(p, d["rows_q"][0].astype(np.float64))
    E = analysis.expected_tokens(alpha, d["gamma"])
    tok = r["n_accepted"] + 1.0
    se = tok.std() / math.sqrt(tok.size)
    assert abs(tok.mean() - E) < 4 * se, (tok.mean(), E, se)


# ---------------------------------------------------------- special cases

def test_identical_distributions_accept_everything():
    """q = p -> beta = 1 ([FI] 'DLK(p,q) = 0 iff p = q'): every draft is
    accepted and a bonus token is drawn.  Uniform rows make p exact."""
    B, gamma, V = 2000, 5, 4
    rng = np.random.default_rng(41)
    zl = np.zeros((B, gamma + 1, V), np.float32)
    q = np.full((B, gamma, V), 0.25, np.float32)
    x = rng.integers(0, V, (B, gamma)).astype(np.int32)
    u = synth.draw_uniforms(rng, (B, gamma + 1))
    r = _run(zl, q, x, u, 1.0)
    assert np.all(r["n_accepted"] == gamma)
    assert np.all(r["out_tokens"][:, :gamma] == x)
    assert _chisq_pvalue(np.bincount(r["out_tokens"][:, gamma], minlength=V), np.full(V, 0.25)) > 1e-3


def test_disjoint_supports_reject_at_once():
    """Disjoint supports -> beta = 0 ([FI] 'DLK(p,q) = 1 iff disjoint
    supports'): the first draft is always rejected and the corrected token
    follows p_0."""
    B, gamma, V = 20_000, 3, 6
    rng = np.random.default_rng(42)
    zp = rng.standard_normal((gamma + 1, V)).astype(np.float32)
    zp[:, 3:] = -np.inf  # p lives on {0,1,2}
    qrow = np.zeros(V, np.float32)
    qrow[3:] = [0.2, 0.3, 0.5]  # q lives on {3,4,5}
    zl = np.ascontiguousarray(np.broadcast_to(zp, (B, gamma + 1, V)))
    q = np.ascontiguousarray(np.broadcast_to(qrow, (B, gamma, V)))
    x = rng.choice(np.arange(3, 6), size=(B, gamma), p=[0.2, 0.3, 0.5]).astype(np.int32)
    u = synth.draw_uniforms(rng, (B, gamma + 1))
    r = _run(zl, q, x, u, 1.0)
    assert np.all(r["n_accepted"] == 0)
    p0 = scipy.special.softmax(zp[0, :3].astype(np.float64))
    assert np.all(r["out_tokens"][:, 0] < 3)
    assert _chisq_pvalue(np.bincount(r["out_tokens"][:, 0], minlength=3), p0) > 1e-3


def test_greedy_mode_is_argmax_matching():
    """[FI] 'Standardized Sampling', argmax case: a draft survives iff it is the
    target argmax; the emitted token at the first mismatch is that argmax."""
    rng = np.random.default_rng(43)
    B, gamma, V = 300, 6, 50
    zl = np.round(rng.standard_normal((B, gamma + 1, V)) * 3).astype(np.float32)  # ties
    am = np.argmax(zl, axis=-1)
    k = rng.integers(0, gamma + 1, B)
    x = am[:, :gamma].astype(np.int32).copy()
    for b in range(B):
        if k[b] < gamma:
            x[b, k[b]] = (am[b, k[b]] + 1 + rng.integers(V - 1)) % V
    r = oracle.spec_verify_ref(zl, None, x, None, 1.0, oracle.GREEDY)
    assert np.array_equal(r["n_accepted"], k)
    for b in range(B):
        n = k[b]
        assert np.array_equal(r["out_tokens"][b, :n], x[b, :n])
        assert r["out_tokens"][b, n] == am[b, n]
        assert np.all(r["out_tokens"][b, n + 1:] == -1)


# ------------------------------------------------------------- invariants

@pytest.mark.parametrize("name", ["c2", "c3", "c5"])
def test_block_advance_invariant(name):
    """[PB] section 2: a step advances by at least 1 and at most gamma+1
    tokens; the first n outputs are the accepted drafts."""
    kw = {"c5": dict(B=8, V=20_000), "c3": dict(B=16, V=20_000), "c2": {}}[name]
    d = synth.make_inputs(name, 3, **kw)
    r = oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], d["draft_tokens"],
                               d["uniforms"], d["temperature"])
    n, out, x = r["n_accepted"], r["out_tokens"], d["draft_tokens"]
    g = d["gamma"]
    assert np.all((n >= 0) & (n <= g))
    for b in range(d["B"]):
        assert np.count_nonzero(out[b] != -1) == n[b] + 1
        assert np.array_equal(out[b, :n[b]], x[b, :n[b]])
        assert 0 <= out[b, n[b]] < d["V"]


def test_unused_rows_do_not_matter():
    """[FI] Phase 3: the walk stops at the first rejection, so target rows after
    position n and draft rows after position n are never read.  Poisoning
    them with NaN must leave every output unchanged."""
    d = synth.make_inputs("c2", 4, B=32, V=3000)
    args = (d["draft_tokens"], d["uniforms"], d["temperature"])
    r0 = oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], *args)
    zl = d["target_logits"].copy()
    q = d["draft_probs"].copy()
    for b, n in enumerate(r0["n_accepted"]):
        zl[b, n + 1:] = np.nan
        q[b, n + 1:] = np.nan
    r1 = oracle.spec_verify_ref(zl, q, *args)
    assert np.array_equal(r0["n_accepted"], r1["n_accepted"])
    assert np.array_equal(r0["out_tokens"], r1["out_tokens"])


def test_invalid_draft_token_marks_sequence():
    d = synth.make_inputs("c2", 5, B=4, V=100)
    x = d["draft_tokens"].copy()
    x[1, 2] = 100
    x[3, 0] = -1
    r = oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], x, d["uniforms"], 1.0)
    for b in (1, 3):
        assert r["n_accepted"][b] == -1 and np.all(r["out_tokens"][b] == -1)
    for b in (0, 2):
        assert r["n_accepted"][b] >= 0


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_p_out_is_the_target_probability_of_the_drawn_token(name):
    """p_out[b] is p_n(t) for the token t drawn at position n, the bonus
    token's p_gamma(t) when every draft passed ([FI] "Speculative Sampling:
    The Core Algorithm", Phase 4): pinned to scipy's softmax of row n at the
    temperature, over seeded batches with rejections, full acceptances (q
    equal to p), the residual fallback's rows and invalid drafts."""
    d = synth.make_inputs(name, 21, B=24, V=3000)
    z, q, x, u = d["target_logits"], d["draft_probs"].copy(), d["draft_tokens"].copy(), d["uniforms"]
    T = d["temperature"]
    bf16 = z.dtype == np.uint16
    z64 = (synth.bf16_bits_to_f32(z) if bf16 else z).astype(np.float64)
    B, G1, V = z.shape
    G = G1 - 1
    # sequences 0..3: q = p at every position, so every draft passes (bonus draws)
    for b in range(4):
        for i in range(G):
            pi = scipy.special.softmax(z64[b, i] / np.float64(np.float32(T)))
            qi = pi.astype(np.float32)
            q[b, i] = qi if q.dtype != np.uint16 else synth.f32_to_bf16_bits(qi)
            x[b, i] = int(np.argmax(pi))
    x[5, 1] = V  # an invalid draft
    r = oracle.spec_verify_ref(z, q, x, u, T)
    n, out = r["n_accepted"], r["out_tokens"]
    assert np.any(n == G) and np.any((n >= 0) & (n < G))
    for b in range(B):
        if n[b] < 0:
            assert np.isnan(r["p_out"][b])
            continue
        ref = scipy.special.softmax(z64[b, n[b]] / np.float64(np.float32(T)))
        np.testing.assert_allclose(r["p_out"][b], ref[out[b, n[b]]], rtol=1e-12, atol=1e-300)
    g = oracle.spec_verify_ref(z, None, x, None, 1.0, oracle.GREEDY)
    assert np.all(np.isnan(g["p_out"]))


def test_argument_validation():
    z = np.zeros((1, 2, 4), np.float32)
    q = np.full((1, 1, 4), 0.25, np.float32)
    x = np.zeros((1, 1), np.int32)
    u = np.full((1, 2), 0.5, np.float32)
    with pytest.raises(ValueError):
        oracle.spec_verify_ref(z, q, x, u, 0.0)
    with pytest.raises(ValueError):
        oracle.spec_verify_ref(z, q, x, u, float("nan"))
    # greedy ignores T, q and u
    r = oracle.spec_verify_ref(z, None, x, None, 0.0, oracle.GREEDY)
    assert r["n_accepted"][0] == 1  # all logits tie -> argmax 0 == x


def test_thread_count_does_not_change_results():
    d = synth.make_inputs("c3", 7, B=24, V=5000)
    a = oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], d["draft_tokens"],
                               d["uniforms"], d["temperature"], n_threads=1)
    b = oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], d["draft_tokens"],
                               d["uniforms"], d["temperature"], n_threads=4)
    for k in ("n_accepted", "out_tokens", "p_tok", "resid_mass", "row_sum"):
        np.testing.assert_array_equal(a[k], b[k])


# ------------------------------------------- acceptance-rate telemetry (beta)

def test_beta_is_one_minus_residual_mass():
    """[FI] Theorem 3.5 with [FI] Phase 4: sum min(p, q) + sum max(0, p - q) =
    sum p = 1, so at the rejected position the telemetry beta_n and the
    residual mass the draw used add up to 1 (two separate sums in the oracle)."""
    d = synth.make_inputs("c2", 3)
    r = oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], d["draft_tokens"],
                               d["uniforms"], d["temperature"], telemetry=True)
    rej = np.nonzero(r["n_accepted"] < d["gamma"])[0]
    assert rej.size > 0
    for b in rej:
        n = r["n_accepted"][b]
        assert abs(r["beta"][b, n] + r["resid_mass"][b] - 1.0) < 1e-10


def test_beta_matches_dlk_closed_form():
    """[FI] Definition 3.2 / Lemma 3.3: with M = (p + q)/2, DLK = sum |p - M| =
    sum |p - q| / 2, and sum min(p, q) = (sum p + sum q - sum |p - q|) / 2 =
    (1 + sum q)/2 - DLK for a draft row used as given (not renormalised).
    Every position, reached by the walk or not."""
    d = synth.make_inputs("c3", 2, B=6)
    r = oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], d["draft_tokens"],
                               d["uniforms"], d["temperature"], telemetry=True)
    zl = d["target_logits"]
    q = d["draft_probs"]
    q64 = q.astype(np.float64) if q.dtype == np.float32 else synth.bf16_bits_to_f32(q).astype(np.float64)
    for b in range(zl.shape[0]):
        for i in range(d["gamma"]):
            p = oracle.softmax_row(zl[b, i], d["temperature"])
            want = 0.5 * (1.0 + q64[b, i].sum()) - analysis.dlk(p, q64[b, i])
            assert abs(r["beta"][b, i] - want) < 1e-12
    assert np.allclose(r["alpha"], r["beta"].mean(axis=0), rtol=0, atol=1e-15)


def test_beta_two_token_example():
    """[ST] two-token example: acceptance is 60 %."""
    g = _golden("two_token_example.json")
    zp = np.log(np.array(g["p"])).astype(np.float32)
    zl = np.stack([zp, zp])[None]
    q = np.array(g["q"], np.float32)[None, None, :]
    r = oracle.spec_verify_ref(zl, q, np.array([[1]], np.int32), np.array([[0.5, 0.5]], np.float32),
                               1.0, telemetry=True)
    assert abs(r["beta"][0, 0] - g["printed"]["acceptance_rate"]) < 1e-7
    assert abs(r["alpha"][0] - g["printed"]["acceptance_rate"]) < 1e-7


def test_beta_special_cases():
    """[FI] 'DLK(p,q) = 0 iff p = q' and '= 1 iff disjoint supports': beta is
    exactly 1 for equal uniform rows and exactly 0 for disjoint supports."""
    V, gamma = 6, 2
    zl = np.zeros((2, gamma + 1, V), np.float32)
    q = np.full((2, gamma, V), 1.0 / V, np.float32)
    zl[1, :, 3:] = -np.inf
    q[1] = 0.0
    q[1, :, 3:] = [0.2, 0.3, 0.5]
    x = np.array([[0, 1], [4, 5]], np.int32)
    u = np.full((2, gamma + 1), 0.5, np.float32)
    r = oracle.spec_verify_ref(zl, q, x, u, 1.0, telemetry=True)
    p_uniform = oracle.softmax_row(zl[0, 0], 1.0)
    assert np.all(r["beta"][0] == np.minimum(p_uniform, q[0, 0].astype(np.float64)).sum())
    assert abs(r["beta"][0, 0] - 1.0) < 1e-7
    assert np.all(r["beta"][1] == 0.0)


def test_beta_is_the_acceptance_probability():
    """[FI] Theorem 3.5: beta_0 is the probability that the first draft is
    accepted.  c1 workload (100 000 trials, one fixed row pair per position):
    the fraction with n >= 1 is Binomial(N, beta_0), checked at 4 sigma; the
    run-to-run identical rows give identical beta and alpha = beta."""
    d = synth.make_c1(seed=8, trials=100_000)
    r = oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], d["draft_tokens"],
                               d["uniforms"], d["temperature"], telemetry=True)
    beta = r["beta"]
    assert np.all(beta == beta[0])
    # (alpha sums 100 000 equal terms in order: rounding ~N eps)
    assert np.allclose(r["alpha"], beta[0], rtol=0, atol=1e-10)
    b0 = beta[0, 0]
    N = beta.shape[0]
    f = float((r["n_accepted"] >= 1).mean())
    assert abs(f - b0) < 4 * math.sqrt(b0 * (1 - b0) / N), (f, b0)
    # and position by position: P(n >= j+1 | n >= j) = beta_j
    n = r["n_accepted"]
    for j in range(1, d["gamma"]):
        sel = n >= j
        fj = float((n[sel] >= j + 1).mean())
        bj = beta[0, j]
        assert abs(fj - bj) < 4 * math.sqrt(bj * (1 - bj) / sel.sum()), (j, fj, bj)


# ------------------------------------------------------------- lenience (l)

def _lenient_law(p, q, l):
    """Closed form of the emitted token's law for one position under the
    lenience reading (accept iff u <= min(1, p/(l q)); residual
    norm(max(0, p - l q))): min(q, p/l) + (1 - sum min(q, p/l)) * r."""
    acc = np.minimum(q, p / l) if l > 0 else q.copy()
    res = np.maximum(0.0, p - l * q)
    r = res / res.sum() if res.sum() > 1e-15 else p
    return acc + (1.0 - acc.sum()) * r, float(acc.sum())


@pytest.mark.parametrize("l", [1.0, 0.5, 0.1])
def test_lenient_law_single_position(l):
    """[FI] 'Ablation Studies and Robustness Checks' (Appendix A.5): with a
    lenience l the acceptance rate is sum min(q, p/l) and, under the stated
    residual reading, the emitted law is the closed form above; l = 1 is the
    exact method (law = p).  Exhaustive draft x midpoint-grid enumeration."""
    rng = np.random.default_rng(61)
    N = 400
    for V in (2, 3, 6):
        zp, q, p = _rand_pq(rng, V, 1)
        zl, qq, x, u, wts = _grid_batch(zp, q, 1, {}, [0, 1], N)
        r = oracle.spec_verify_ref(zl, qq, x, u, 1.0, lenience=l)
        q64 = q[0].astype(np.float64)
        want, acc = _lenient_law(p[0], q64, l)
        law = np.bincount(r["out_tokens"][:, 0], weights=wts, minlength=V)
        assert np.max(np.abs(law - want)) <= 2.0 / N + 1e-6, (l, law, want)
        assert abs(float(wts[r["n_accepted"] == 1].sum()) - acc) <= 1.0 / N + 1e-6
        if l == 1.0:
            assert np.max(np.abs(law - p[0] * q64.sum())) <= 2.0 / N + 1e-6


@pytest.mark.parametrize("l", [0.5, 0.2, 0.1])
def test_lenient_guarantee_p_over_l(l):
    """[FI] 'How This Work Changes the Landscape': under lenience no token is
    sampled with probability greater than p(x)/l.  Checked on the oracle's
    exact law (grid enumeration) for random pairs of rows."""
    rng = np.random.default_rng(62)
    N = 300
    for _ in range(6):
        V = int(rng.integers(2, 7))
        zp, q, p = _rand_pq(rng, V, 1)
        zl, qq, x, u, wts = _grid_batch(zp, q, 1, {}, [0, 1], N)
        r = oracle.spec_verify_ref(zl, qq, x, u, 1.0, lenience=l)
        law = np.bincount(r["out_tokens"][:, 0], weights=wts, minlength=V)
        assert np.all(law <= p[0] / l + 2.0 / N + 1e-6), (law, p[0] / l)


def test_lenience_zero_accepts_every_draft_and_one_is_exact():
    """l = 0 makes p/(l q) infinite: every draft is accepted (the bonus is
    drawn); l = 1 reproduces the exact method bit for bit."""
    d = synth.make_inputs("c2", 5, B=6, V=2000)
    r0 = oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], d["draft_tokens"],
                                d["uniforms"], d["temperature"], lenience=0.0)
    assert np.all(r0["n_accepted"] == d["gamma"])
    r1 = oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], d["draft_tokens"],
                                d["uniforms"], d["temperature"], lenience=1.0)
    rs = oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], d["draft_tokens"],
                                d["uniforms"], d["temperature"])
    assert np.array_equal(r1["out_tokens"], rs["out_tokens"])
    with pytest.raises(ValueError):
        oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], d["draft_tokens"],
                               d["uniforms"], d["temperature"], lenience=1.5)


# ------------------------------------- top-k / nucleus standardisation (f2)

def _rows_with_ties(rng, R, V, dtype):
    z = np.round(rng.standard_normal((R, V)) * 2, 1).astype(np.float32)   # many exact ties
    z[:, rng.integers(0, V, 3)] = -np.inf
    if dtype == "bf16":
        zb = synth.f32_to_bf16_bits(z)
        return zb, synth.bf16_bits_to_f32(zb)
    return z, z


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_topk_matches_a_stable_sort(dtype):
    """[FI] 'Standardized Sampling', top-k: the k largest entries survive.
    Reference: numpy's stable argsort of -z (ties in index order), first k."""
    rng = np.random.default_rng(71)
    V = 300
    z, zf = _rows_with_ties(rng, 12, V, dtype)
    for k in (1, 2, 7, 50, V - 1, V, V + 5):
        out, kept, _ = oracle.standardize(z, oracle.TOPK, k=k)
        outf = out if dtype == "fp32" else synth.bf16_bits_to_f32(out)
        for r in range(z.shape[0]):
            keep = np.zeros(V, bool)
            keep[np.argsort(-zf[r], kind="stable")[:min(k, V)]] = True
            want = np.where(keep, zf[r], -np.inf)
            assert np.array_equal(outf[r], want), (k, r)
            assert kept[r] == min(k, V)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_topp_matches_a_sorted_running_sum(dtype):
    """[FI] 'Standardized Sampling', nucleus: sort the probabilities, keep the
    shortest prefix whose running sum reaches top_p.  Reference: scipy's
    softmax, numpy's stable argsort and cumsum; rows the oracle flags as
    within 1e-9 of the boundary are skipped (other summation orders)."""
    rng = np.random.default_rng(72)
    V = 400
    z, zf = _rows_with_ties(rng, 16, V, dtype)
    checked = 0
    for T in (0.7, 1.0):
        for top_p in (0.05, 0.3, 0.9, 0.999, 1.0):
            out, kept, flag = oracle.standardize(z, oracle.TOPP, top_p=top_p, temperature=T)
            outf = out if dtype == "fp32" else synth.bf16_bits_to_f32(out)
            for r in range(z.shape[0]):
                if flag[r]:
                    continue
                # (the temperature reaches the oracle as fp32)
                p = scipy.special.softmax(zf[r].astype(np.float64) / float(np.float32(T)))
                order = np.argsort(-zf[r], kind="stable")
                c = np.cumsum(p[order])
                hit = np.nonzero(c >= float(np.float32(top_p)))[0]  # top_p also arrives as fp32
                nk = int(hit[0]) + 1 if hit.size and top_p < 1.0 else V
                keep = np.zeros(V, bool)
                keep[order[:nk]] = True
                assert np.array_equal(outf[r], np.where(keep, zf[r], -np.inf)), (T, top_p, r)
                assert kept[r] == nk
                checked += 1
    assert checked > 100


def test_topk_one_is_the_argmax_and_full_k_is_identity():
    """k = 1 leaves the point mass at the first maximum ([FI]'s argmax case);
    k = V (and top_p below the largest probability / top_p = 1) as stated."""
    rng = np.random.default_rng(73)
    z, _ = _rows_with_ties(rng, 8, 64, "fp32")
    out, _, _ = oracle.standardize(z, oracle.TOPK, k=1)
    for r in range(8):
        assert np.nonzero(np.isfinite(out[r]))[0].tolist() == [oracle.argmax_row(z[r])]
    out, _, _ = oracle.standardize(z, oracle.TOPK, k=64)
    assert np.array_equal(out, z)
    out, kept, _ = oracle.standardize(z, oracle.TOPP, top_p=1e-6)
    assert np.all(kept == 1)
    out, kept, _ = oracle.standardize(z, oracle.TOPP, top_p=1.0)
    assert np.all(kept == 64) and np.array_equal(out, z)


def test_standardised_verification_is_exact():
    """[FI] 'Standardized Sampling': with p and q both standardised (top-k
    here), the verify step emits the standardised p exactly.  Exhaustive
    draft x midpoint-grid enumeration on tiny rows."""
    rng = np.random.default_rng(74)
    N = 300
    for V, k in ((5, 3), (6, 2)):
        zq = rng.standard_normal(V)
        zp = (zq + 0.8 * rng.standard_normal(V)).astype(np.float32)
        zp_std, _, _ = oracle.standardize(np.stack([zp, zp]), oracle.TOPK, k=k)
        q = scipy.special.softmax(zq)
        q[np.argsort(-q, kind="stable")[k:]] = 0.0
        q = (q / q.sum()).astype(np.float32)
        zl, qq, x, u, wts = _grid_batch(zp_std, q[None, :], 1, {}, [0, 1], N)
        r = oracle.spec_verify_ref(zl, qq, x, u, 1.0)
        law = np.bincount(r["out_tokens"][:, 0], weights=wts, minlength=V)
        p = scipy.special.softmax(zp.astype(np.float64))
        p[np.argsort(-zp, kind="stable")[k:]] = 0.0
        p /= p.sum()
        assert np.max(np.abs(law - p * float(q.astype(np.float64).sum()))) <= 2.0 / N + 1e-6
