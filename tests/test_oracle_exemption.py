"""Pins of the oracle's exemption bookkeeping: which decisions it flags as
near-boundary, where the first flag sits, and how decisions are counted.

These outputs decide which GPU results the parity tests excuse from
bit-exact agreement, so a wrong window, a wrong position or a wrong count
would silently widen the exemption.  Each case is built so that the
quantity the oracle compares (an acceptance threshold, a normalised CDF
boundary, a residual mass) is known here, by repeating the oracle's few
fp64 operations on inputs with exactly known values, and then sits just
inside or just outside its window.

The rules pinned (north-star exemption, "Fast Inference from Transformers
via Speculative Decoding", "Critical Assessment": exactness depends on the
implementation near normalisation and at the boundaries of each decision):
  acceptance test at position i: flagged iff |u_i - thr| <= 1e-6 thr;
  inverse-CDF draw: flagged iff u is within 1e-9 (relative) of either
    normalised boundary of the chosen token;
  residual mass Z: flagged iff |Z - 1e-15| <= 1e-6 * 1e-15 (the fallback of
    "The exact decoding shortcut that burns compute when guesses miss");
  flag_pos = position of the first flagged decision (the draw counts at
    position n), n_flags = flagged decisions, n_decisions = acceptance tests
    run + 1 draw (sample mode); invalid sequences count nothing.
"""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_util import compare

F32 = np.float32


def _softmax_like_oracle(z, T):
    """The oracle's row softmax, operation for operation (max, then
    exp((z - m) / T) summed in index order, then each term / sum)."""
    z = [float(F32(v)) for v in z]
    T = float(F32(T))
    m = max(z)
    e = [math.exp((v - m) / T) for v in z]
    s = 0.0
    for v in e:
        s += v
    return [v / s for v in e]


def _one(z_rows, q_rows, x, u, T=1.0):
    """Oracle on one sequence: z_rows [gamma+1][V], q_rows [gamma][V]."""
    zl = np.asarray(z_rows, F32)[None]
    q = np.asarray(q_rows, F32)[None]
    r = oracle.spec_verify_ref(zl, q, np.asarray([x], np.int32), np.asarray([u], F32), float(T))
    return {k: (v[0] if getattr(v, "ndim", 0) else v) for k, v in r.items()}


def _u_near(b, rel):
    """The fp32 value nearest to b * (1 + rel), and its actual relative
    distance to b in double."""
    u = F32(b * (1.0 + rel))
    return u, abs(float(u) - b) / b


# ------------------------------------------------------------- acceptance window

@pytest.mark.parametrize("rel", [0.5e-6, -0.5e-6, 0.9e-6, -0.9e-6, 2e-6, -2e-6, 5e-6])
def test_acceptance_window_is_1e6_relative(rel):
    # row 0: draft token 1 with q > p there, so thr = p/q < 1
    z0 = [0.3, -0.4, 1.1, 0.0]
    q0 = [0.1, 0.6, 0.2, 0.1]
    p0 = _softmax_like_oracle(z0, 1.0)
    thr = p0[1] / float(F32(q0[1]))
    assert thr < 1.0
    u0, dist = _u_near(thr, rel)
    assert abs(dist - abs(rel)) < 1.5e-7  # fp32 rounding of u moves it by <= 6e-8 relative
    # row 1: clearly rejected (q(x) = 0.9, p(x) tiny, u near 1)
    z = [z0, [5.0, -5.0, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0]]
    q = [q0, [0.05, 0.9, 0.025, 0.025]]
    r = _one(z, q, [1, 1], [u0, 1.0 - 2 ** -24, 0.37])
    assert r["thr"][0] == pytest.approx(thr, rel=1e-15)
    accepted = float(u0) <= thr
    assert r["n_accepted"] == (1 if accepted else 0)
    flagged = dist <= 1e-6
    assert bool(r["n_flags"] >= 1) == flagged
    assert r["flag_pos"] == (0 if flagged else -1)
    # tests run: position 0, and position 1 only if 0 accepted; + the draw
    assert r["n_decisions"] == (3 if accepted else 2)


def test_acceptance_flag_names_its_position():
    # position 0 clearly accepted (q(x) <= p(x): thr = 1, u = 0.5),
    # position 1 exactly on its threshold
    z0 = [2.0, 0.0, 0.0]
    q0 = [0.2, 0.4, 0.4]
    z1 = [0.0, 0.5, -0.5]
    q1 = [0.1, 0.7, 0.2]
    p1 = _softmax_like_oracle(z1, 1.0)
    thr1 = p1[1] / float(F32(q1[1]))
    u1, dist = _u_near(thr1, 0.0)
    assert dist <= 1e-7
    r = _one([z0, z1, [0.0, 0.0, 0.0]], [q0, q1], [0, 1], [0.5, u1, 0.25])
    assert r["thr"][0] == 1.0
    assert r["flag_pos"] == 1
    assert r["n_flags"] >= 1
    # both positions on their thresholds (position 0 accepted: u <= thr):
    # the first flag is the one reported, and both are counted
    z0b = [0.0, 0.5, -0.5]
    q0b = [0.1, 0.7, 0.2]
    p0b = _softmax_like_oracle(z0b, 1.0)
    thr0 = p0b[1] / float(F32(q0b[1]))
    u0 = F32(thr0)
    if float(u0) > thr0:
        u0 = np.nextafter(u0, F32(0), dtype=F32)
    assert abs(float(u0) - thr0) <= 1e-7 * thr0
    r2 = _one([z0b, z1, [0.0, 0.0, 0.0]], [q0b, q1], [1, 1], [u0, u1, 0.25])
    assert r2["n_accepted"] >= 1
    assert r2["flag_pos"] == 0
    assert r2["n_flags"] >= 2


# ------------------------------------------------------------------ draw window

@pytest.mark.parametrize("d,expect_flag", [(1e-9, True), (1.6e-9, True), (2.4e-9, False), (4e-9, False),
                                           (-1e-9, True), (-4e-9, False)])
def test_icdf_window_is_1e9_relative(d, expect_flag):
    # every draft accepted (thr = 1), so the draw is the bonus token from
    # row 1 = softmax(0, -d): its first boundary C_0 / total sits at
    # 1/2 (1 + d/2 + ...) and u = 1/2 exactly
    dz = F32(d)
    z = [[1.0, 0.0], [0.0, -float(dz)]]
    q = [[0.5, 0.5]]
    p1 = _softmax_like_oracle(z[1], 1.0)
    total = p1[0] + p1[1]
    b = p1[0] / total
    rel = abs(0.5 - b) / b
    assert (rel <= 1e-9) == expect_flag  # the case is where it is meant to be
    r = _one(z, q, [0], [0.5, 0.5])
    assert r["n_accepted"] == 1
    assert r["out_tokens"].tolist() == [0, 0 if 0.5 * total < p1[0] else 1]
    assert bool(r["n_flags"]) == expect_flag
    assert r["flag_pos"] == (1 if expect_flag else -1)  # the draw counts at position n = gamma
    assert r["n_decisions"] == 2


def test_icdf_flag_of_a_residual_draw_names_position_n():
    # gamma = 2, rejected at position 0; the residual has two equal
    # positive entries (tokens 0 and 1), so its first boundary is 1/2 exactly
    z0 = [1.0, 1.0, -3.0]
    q0 = [0.05, 0.05, 0.9]
    rows = [z0, [0.0, 0.0, 0.0], [0.0, 0.0, 0.0]]
    qs = [q0, [0.3, 0.3, 0.4]]
    p0 = _softmax_like_oracle(z0, 1.0)
    w = [max(0.0, p0[v] - float(F32(q0[v]))) for v in range(3)]
    assert w[0] == w[1] > 0 and w[2] == 0
    on = _one(rows, qs, [2, 0], [0.9, 0.5, 0.5])
    off = _one(rows, qs, [2, 0], [0.9, 0.5, 0.5 + 2 ** -24])
    for r in (on, off):
        assert r["n_accepted"] == 0
        assert r["n_decisions"] == 2
    assert on["flag_pos"] == 0 and on["n_flags"] == 1
    assert on["out_tokens"].tolist() == [1, -1, -1]  # strict '>': u * total == C_0 moves on
    assert off["flag_pos"] == -1 and off["n_flags"] == 0  # 1.2e-7 relative is outside 1e-9
    assert off["out_tokens"].tolist() == [1, -1, -1]


# -------------------------------------------------------- residual-mass window

def _tiny_mass_case(target_rel):
    """Logit a and temperature T (both fp32) for which the residual mass of
    the case below is 1e-15 (1 + target_rel) to within 2e-8 relative."""
    best = None
    base_a = F32(math.log(1e15 / (1.0 + target_rel)))
    for da in range(-40, 41):
        a = np.nextafter(base_a, F32(np.inf) if da > 0 else F32(0), dtype=F32) if da else base_a
        for _ in range(abs(da) - 1 if da else 0):
            a = np.nextafter(a, F32(np.inf) if da > 0 else F32(0), dtype=F32)
        for dt in range(-40, 41):
            T = F32(1.0)
            for _ in range(abs(dt)):
                T = np.nextafter(T, F32(2.0) if dt > 0 else F32(0.0), dtype=F32)
            p = _softmax_like_oracle([-float(a), 0.0, -100.0], float(T))
            Z = p[0]
            err = abs(Z / 1e-15 - (1.0 + target_rel))
            if best is None or err < best[0]:
                best = (err, float(a), float(T), Z)
    assert best[0] < 2e-8
    return best[1:]


@pytest.mark.parametrize("target_rel,expect_flag", [(0.5e-6, True), (-0.5e-6, True),
                                                    (2e-6, False), (-2e-6, False)])
def test_residual_mass_window(target_rel, expect_flag):
    # position 0 rejects (draft token 2 has q = 0.5, p ~ e^-100); the
    # residual max(0, p - q) is p_0 alone (q_0 = 0, q_1 = 1 >= p_1), so
    # Z = p_0 = e^{-a/T} / (1 + e^{-a/T} + e^{-100/T})
    a, T, Z = _tiny_mass_case(target_rel)
    z = [[-a, 0.0, -100.0], [0.0, 0.0, 0.0]]
    q = [[0.0, 1.0, 0.5]]
    r = _one(z, q, [2], [0.5, 0.5], T=T)
    assert r["n_accepted"] == 0
    assert r["resid_mass"] == Z
    assert bool(r["n_flags"]) == expect_flag
    assert r["flag_pos"] == (0 if expect_flag else -1)
    # Z > 1e-15: the residual (all mass on token 0); else the target row,
    # whose mass is on token 1
    assert r["out_tokens"][0] == (0 if Z > 1e-15 else 1)


# ---------------------------------------------------------------- decision counts

def test_decision_count_and_first_flag():
    rng = np.random.default_rng(5)
    V, gamma = 64, 4
    zq = rng.standard_normal((gamma + 1, V))
    q = np.exp(zq[:gamma]) / np.exp(zq[:gamma]).sum(-1, keepdims=True)
    zp = (zq + 0.3 * rng.standard_normal((gamma + 1, V))).astype(F32)
    x = [int(np.argmax(q[i])) for i in range(gamma)]
    # all accepted: u tiny at every test
    r = _one(zp, q, x, [2 ** -24] * gamma + [0.5])
    assert r["n_accepted"] == gamma and r["n_decisions"] == gamma + 1
    # rejected at 2: u = 1 - 2^-24 there and thr < 1 (checked)
    thr2 = r["thr"][2]
    if thr2 < 1.0 - 1e-5:
        r2 = _one(zp, q, x, [2 ** -24, 2 ** -24, 1.0 - 2 ** -24, 2 ** -24, 0.5])
        assert r2["n_accepted"] == 2 and r2["n_decisions"] == 4
    # two flagged decisions: position 0 on its threshold and the bonus draw
    # on a boundary of a row of equal logits (boundaries at k / V)
    zp2 = zp.copy()
    zp2[gamma] = 0.0
    r3 = _one(zp2, q, x, [2 ** -24] * gamma + [0.5])
    thr0 = r3["thr"][0]
    if thr0 < 1.0:
        u0, _ = _u_near(thr0, 0.0)
        r4 = _one(zp2, q, x, [u0] + [2 ** -24] * (gamma - 1) + [0.5])
        if r4["n_accepted"] == gamma:
            assert r4["n_flags"] == 2 and r4["flag_pos"] == 0


def test_greedy_and_invalid_counts():
    rng = np.random.default_rng(6)
    V, gamma = 32, 3
    z = rng.standard_normal((gamma + 1, V)).astype(F32)
    am = [int(np.argmax(z[i])) for i in range(gamma + 1)]
    zl = z[None]
    # greedy: tests run, no draw decision, never a flag
    r = oracle.spec_verify_ref(zl, None, np.asarray([am[:gamma]], np.int32), None, 1.0, oracle.GREEDY)
    assert r["n_accepted"][0] == gamma and r["n_decisions"][0] == gamma
    assert r["n_flags"][0] == 0 and r["flag_pos"][0] == -1
    x = am[:gamma]
    x[1] = (x[1] + 1) % V
    r = oracle.spec_verify_ref(zl, None, np.asarray([x], np.int32), None, 1.0, oracle.GREEDY)
    assert r["n_accepted"][0] == 1 and r["n_decisions"][0] == 2
    # an invalid draft token: nothing counted
    q = np.full((1, gamma, V), 1.0 / V, F32)
    r = oracle.spec_verify_ref(zl, q, np.asarray([[0, V, 0]], np.int32), np.full((1, gamma + 1), 0.5, F32), 1.0)
    assert r["n_accepted"][0] == -1 and r["n_decisions"][0] == 0 and r["flag_pos"][0] == -1


# ------------------------------------------------------------ the comparison rule

def _ref_with_flags():
    rng = np.random.default_rng(8)
    B, gamma, V = 6, 3, 16
    zq = rng.standard_normal((B, gamma + 1, V))
    q = (np.exp(zq[:, :gamma]) / np.exp(zq[:, :gamma]).sum(-1, keepdims=True)).astype(F32)
    zp = (zq + 0.5 * rng.standard_normal(zq.shape)).astype(F32)
    x = np.argmax(q, -1).astype(np.int32)
    u = rng.random((B, gamma + 1)).astype(F32)
    r = oracle.spec_verify_ref(zp, q, x, u, 1.0)
    # pretend sequence 2's first decision was flagged (the rule, not the case, is tested)
    r["flag_pos"] = r["flag_pos"].copy()
    r["flag_pos"][2] = 0
    return r, x, V


def test_compare_accepts_identical_and_rejects_planted_mistakes():
    ref, x, V = _ref_with_flags()
    gamma = x.shape[1]
    g = {"n_accepted": ref["n_accepted"].copy(), "out_tokens": ref["out_tokens"].copy()}
    compare(g, ref, gamma, draft_tokens=x, vocab=V)

    def bad(mut):
        gg = {"n_accepted": ref["n_accepted"].copy(), "out_tokens": ref["out_tokens"].copy()}
        mut(gg)
        with pytest.raises(AssertionError):
            compare(gg, ref, gamma, draft_tokens=x, vocab=V)

    b = 2  # the flagged sequence: its outputs may differ, but must stay well formed
    def wrong_padding(gg):
        gg["n_accepted"][b] = 0
        gg["out_tokens"][b] = [x[b, 0], 1, -1, -1]
    bad(wrong_padding)

    def token_out_of_range(gg):
        gg["n_accepted"][b] = 0
        gg["out_tokens"][b] = [V, -1, -1, -1]
    bad(token_out_of_range)

    def accepted_prefix_not_drafts(gg):
        gg["n_accepted"][b] = 2
        gg["out_tokens"][b] = [x[b, 0], (x[b, 1] + 1) % V, 3, -1]
    bad(accepted_prefix_not_drafts)

    def n_too_large(gg):
        gg["n_accepted"][b] = gamma + 1
    bad(n_too_large)

    clean = int(np.nonzero(ref["flag_pos"] < 0)[0][0])
    def unflagged_differs(gg):
        gg["out_tokens"][clean, ref["n_accepted"][clean]] ^= 1
    bad(unflagged_differs)

    # a well-formed different outcome of the flagged sequence is allowed
    ok = {"n_accepted": ref["n_accepted"].copy(), "out_tokens": ref["out_tokens"].copy()}
    ok["n_accepted"][b] = 1
    ok["out_tokens"][b] = [x[b, 0], 5, -1, -1]
    compare(ok, ref, gamma, draft_tokens=x, vocab=V)
