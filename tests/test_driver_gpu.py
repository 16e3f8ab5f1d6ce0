"""The multi-step driver with the GPU verify step (through the C ABI via the
binding): whole token streams identical to the same loop driven by the fp64
reference, the per-position law p_t, and gamma* chosen from the library's
own alpha telemetry delivering Equation 1's tokens per iteration."""
import math

import numpy as np
import pytest

from oracle import analysis
from exact_rejection_sampling_temp_amd import driver
from tests import synth
from tests.laws import target_law
from tests.test_driver import OracleVerifier, _chisq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,V", [(synth.FP32, 1000), (synth.BF16, 4096)])
def test_streams_equal_the_reference_loop(dtype, V):
    L, gamma = 24, 4
    m = synth.make_position_models(L + gamma, V, seed=11, dtype=dtype, sigma=2.0)
    print(f"[driver] dtype={dtype} V={V} streams=400 L={L} gamma={gamma}", flush=True)
    g = driver.speculative_decode(m, 400, L, gamma, seed=12)
    r = driver.speculative_decode(m, 400, L, gamma, seed=12, verify=OracleVerifier(m))
    assert np.array_equal(g["tokens"], r["tokens"])
    assert np.array_equal(g["iterations"], r["iterations"])


def test_gpu_loop_emits_p_at_every_position():
    L, V, gamma = 10, 6, 3
    m = synth.make_position_models(L + gamma, V, seed=13)
    p64 = target_law(m)
    r = driver.speculative_decode(m, 20_000, L, gamma, seed=14)
    for t in range(L):
        assert _chisq(np.bincount(r["tokens"][:, t], minlength=V).astype(float), p64[t]) > 1e-3, t


def test_gamma_star_from_telemetry():
    L, V, c = 60, 2000, 0.05
    m = synth.make_position_models(L + 64, V, seed=15, iid=True, sigma=1.5, shift=0.6)
    p64 = target_law(m)
    alpha = driver.estimate_alpha(m, np.arange(8))
    want = analysis.acceptance_rate(p64[0], m.draft_probs[0].astype(np.float64))
    assert abs(alpha - want) < 1e-6
    gamma = driver.optimal_gamma(alpha, c)
    print(f"[driver] alpha={alpha:.4f} c={c} gamma*={gamma}", flush=True)
    r = driver.speculative_decode(m, 2000, L, gamma, seed=16)
    k = np.concatenate(r["accepted"]).astype(float) + 1.0
    E = analysis.expected_tokens(alpha, gamma)
    assert abs(k.mean() - E) < 4 * k.std() / math.sqrt(k.size), (k.mean(), E)
