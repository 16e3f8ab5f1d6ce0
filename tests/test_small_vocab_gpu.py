"""GPU parity of the small-vocabulary path (V <= 512: one wave per sequence,
one launch) against the fp64 oracle, through the C ABI (via the binding):
outputs bit-exact outside the oracle's near-boundary decisions, row
statistics and the residual mass as for the many-workgroup path, in sample,
lenient and greedy mode, with the edge cases of the method (invalid drafts,
-inf logits, q(x) = 0, identical distributions, no residual mass)."""
import numpy as np
import pytest

from tests import synth
from tests.gpu_util import check_aux, compare, run_gpu, run_ref

pytestmark = pytest.mark.gpu


def _check(d, mode="sample", lenience=1.0):
    print(f"[small] {d['name']} B={d['B']} gamma={d['gamma']} V={d['V']} mode={mode} l={lenience}", flush=True)
    g = run_gpu(d, mode, with_aux=mode == "sample", lenience=lenience)
    if mode == "greedy":
        r = run_ref(d, mode)
    else:
        import oracle
        r = oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], d["draft_tokens"], d["uniforms"],
                                   d["temperature"], oracle.SAMPLE, lenience=lenience)
    compare(g, r, d["gamma"], draft_tokens=d["draft_tokens"], vocab=d["V"])
    if mode == "sample":
        check_aux(g, r, 1e-6)
    return g, r


@pytest.mark.parametrize("V", [1, 2, 7, 63, 64, 65, 300, 511, 512])
def test_fp32_sample(V):
    _check(synth.make_inputs("c2", 900 + V, B=64, V=V))


@pytest.mark.parametrize("gamma", [1, 16, 62, 63])
@pytest.mark.parametrize("V", [8, 100, 512])
def test_bf16_sample(gamma, V):
    _check(synth.make_inputs("c5", 1000 + gamma * 7 + V, B=32, gamma=gamma, V=V))


def test_bf16_logits_fp32_probs():
    _check(synth.make_inputs("c3", 1100, B=48, V=257))


@pytest.mark.parametrize("lenience", [0.0, 0.5])
def test_lenient(lenience):
    _check(synth.make_inputs("c2", 1200, B=64, V=200), lenience=lenience)


@pytest.mark.parametrize("V", [1, 5, 300, 512])
def test_greedy(V):
    d = synth.make_inputs("c3", 1300 + V, B=64, V=V)
    _check(d, "greedy")
    # drafts set to the argmax are all accepted
    z = synth.bf16_bits_to_f32(d["target_logits"])
    d["draft_tokens"] = np.argmax(z[:, :-1, :], axis=2).astype(np.int32)
    g, _ = _check(d, "greedy")
    assert np.all(g["n_accepted"] == d["gamma"])


def test_greedy_ties_pick_lowest_index():
    B, gamma, V = 16, 3, 200
    zl = np.zeros((B, gamma + 1, V), np.float32)
    zl[:, :, 17] = 2.0
    zl[:, :, 130] = 2.0
    zl[:, :, 5] = -0.0
    d = {"name": "ties", "B": B, "gamma": gamma, "V": V, "temperature": 1.0, "target_logits": zl,
         "draft_probs": np.full((B, gamma, V), 1.0 / V, np.float32),
         "draft_tokens": np.full((B, gamma), 17, np.int32),
         "uniforms": np.full((B, gamma + 1), 0.5, np.float32)}
    d["draft_tokens"][3, 1] = 130
    g, _ = _check(d, "greedy")
    assert g["n_accepted"][3] == 1 and g["out_tokens"][3, 1] == 17
    assert np.all(np.delete(g["n_accepted"], 3) == gamma)


def test_invalid_tokens():
    d = synth.make_inputs("c2", 1400, B=8, V=300)
    d["draft_tokens"][1, 3] = 300
    d["draft_tokens"][4, 0] = -1
    d["draft_tokens"][6, 2] = 1 << 30
    for mode in ("sample", "greedy"):
        g, _ = _check(d, mode)
        for b in (1, 4, 6):
            assert g["n_accepted"][b] == -1 and np.all(g["out_tokens"][b] == -1)


def test_neg_inf_logits_and_zero_probs():
    d = synth.make_inputs("c2", 1500, B=32, V=400)
    rng = np.random.default_rng(1500)
    zl = d["target_logits"]
    zl[rng.random(zl.shape) < 0.3] = -np.inf
    zl[:, :, 0] = 0.0  # keep every row's max finite
    q = d["draft_probs"]
    q[rng.random(q.shape) < 0.2] = 0.0
    for b in range(d["B"]):
        for i in range(d["gamma"]):
            if q[b, i, d["draft_tokens"][b, i]] == 0:
                q[b, i, d["draft_tokens"][b, i]] = 1e-3
    q[0, 0, d["draft_tokens"][0, 0]] = 0.0  # q(x) = 0 -> accepted
    _check(d)


def test_identical_distributions_take_bonus():
    B, gamma, V = 32, 5, 100
    rng = np.random.default_rng(1600)
    d = {"name": "same", "B": B, "gamma": gamma, "V": V, "temperature": 1.0,
         "target_logits": np.zeros((B, gamma + 1, V), np.float32),
         "draft_probs": np.full((B, gamma, V), 1.0 / V, np.float32),
         "draft_tokens": rng.integers(0, V, (B, gamma)).astype(np.int32),
         "uniforms": synth.draw_uniforms(rng, (B, gamma + 1))}
    g, _ = _check(d)
    assert np.all(g["n_accepted"] == gamma)


def test_zero_residual_fallback():
    # q >= p everywhere on the draft's support: a rejection leaves no
    # residual mass and the draw falls back to p ([ST])
    B, gamma, V = 32, 4, 64
    rng = np.random.default_rng(1700)
    zl = np.zeros((B, gamma + 1, V), np.float32)
    q = np.zeros((B, gamma, V), np.float32)
    q[:, :, :8] = 1.0 / 8
    zl[:, :, 8:] = -np.inf
    d = {"name": "noresid", "B": B, "gamma": gamma, "V": V, "temperature": 1.0, "target_logits": zl,
         "draft_probs": q, "draft_tokens": rng.integers(0, 8, (B, gamma)).astype(np.int32),
         "uniforms": synth.draw_uniforms(rng, (B, gamma + 1))}
    g, _ = _check(d)
    assert np.all(g["out_tokens"][np.arange(B), np.minimum(g["n_accepted"], gamma)] < 8)


@pytest.mark.parametrize("V,gamma", [(16, 15), (3, 15), (16, 1), (9, 7)])
def test_four_sequences_per_wave(V, gamma):
    """V <= 16 and gamma < 16 run four sequences per wave (one per 16-lane
    DPP row): a ragged batch, invalid drafts in some rows, lenience and greedy."""
    d = synth.make_inputs("c2", 1800 + V * 16 + gamma, B=37, gamma=gamma, V=V)
    d["draft_tokens"][5, gamma - 1] = V
    d["draft_tokens"][18, 0] = -3
    for lenience in (1.0, 0.4):
        g, _ = _check(d, lenience=lenience)
        for b in (5, 18):
            assert g["n_accepted"][b] == -1 and np.all(g["out_tokens"][b] == -1)
    _check(d, "greedy")
    db = synth.make_inputs("c5", 1900 + V + gamma, B=21, gamma=gamma, V=V)
    _check(db)


@pytest.mark.parametrize("V,gamma", [(8, 7), (1, 1), (5, 3), (8, 4), (2, 7)])
def test_eight_sequences_per_wave(V, gamma):
    """V <= 8 and gamma + 1 <= 8 run eight sequences per wave (one per 8-lane
    half row): a ragged batch, invalid drafts, lenience, greedy, bf16."""
    d = synth.make_inputs("c2", 2000 + V * 16 + gamma, B=45, gamma=gamma, V=V)
    d["draft_tokens"][9, gamma - 1] = V
    d["draft_tokens"][30, 0] = -1
    for lenience in (1.0, 0.3):
        g, _ = _check(d, lenience=lenience)
        for b in (9, 30):
            assert g["n_accepted"][b] == -1 and np.all(g["out_tokens"][b] == -1)
    _check(d, "greedy")
    db = synth.make_inputs("c5", 2100 + V + gamma, B=29, gamma=gamma, V=V)
    _check(db)
