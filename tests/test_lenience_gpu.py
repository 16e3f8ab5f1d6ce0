"""GPU parity of the lenient variant (spec_verify_lenient): accept iff
u <= min(1, p/(l q)), residual norm(max(0, p - l q)) ("Fast Inference from
Transformers via Speculative Decoding", summary page, Appendix A.5; the
residual is this build's stated reading), against the fp64 oracle with the
same l, through the C ABI (via the binding).  Same bar as the exact method:
bit-exact outputs outside the oracle's near-boundary flags, p(x) within 1e-6
relative, the lenient residual mass within 1e-9 relative."""
import numpy as np
import pytest

from tests import synth
from tests.gpu_util import check_aux, compare, run_gpu, run_ref

pytestmark = pytest.mark.gpu


def _check_len(d, l):
    print(f"[lenience] {d['name']} B={d['B']} gamma={d['gamma']} V={d['V']} l={l}", flush=True)
    g = run_gpu(d, lenience=l)
    r = run_ref(d, lenience=l)
    c = compare(g, r, d["gamma"], draft_tokens=d["draft_tokens"], vocab=d["V"])
    check_aux(g, r, 1e-6)
    assert c["flagged_decisions"] <= max(1, c["decisions"] // 1000)
    return g, r


@pytest.mark.parametrize("l", [0.5, 0.1])
def test_lenient_c4_full_size(l):
    g, r = _check_len(synth.make_inputs("c4", 0), l)
    # a lower l accepts at least as many drafts on the same inputs
    g1 = run_gpu(synth.make_inputs("c4", 0), with_aux=False)
    assert g["n_accepted"].mean() >= g1["n_accepted"].mean()


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("l", [0.8, 0.3])
def test_lenient_c2(seed, l):
    _check_len(synth.make_inputs("c2", 50 + seed), l)


@pytest.mark.parametrize("l", [0.5])
def test_lenient_c3_and_c5(l):
    _check_len(synth.make_inputs("c3", 3, B=16), l)
    _check_len(synth.make_inputs("c5", 3, B=8, V=60_000), l)


def test_lenience_zero_accepts_everything():
    d = synth.make_inputs("c4", 61, B=12, V=20_000)
    g, r = _check_len(d, 0.0)
    assert np.all(g["n_accepted"] == d["gamma"])


def test_lenient_scalar_path_and_repeated_calls():
    for V in (7, 1001):
        _check_len(synth.make_inputs("c2", 70 + V, B=6, V=V), 0.6)
    # exact call after a lenient one on the same workspace
    d = synth.make_inputs("c2", 80, B=6, V=4000)
    g = run_gpu(d)
    r = run_ref(d)
    compare(g, r, d["gamma"], draft_tokens=d["draft_tokens"], vocab=d["V"])
