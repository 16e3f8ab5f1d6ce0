"""Seeded random shapes through the C ABI against the fp64 oracle: batch,
gamma, vocabulary (log-uniform from 1 to 70 000, so both the one-wave path
for V <= 512 and the two-launch path), dtypes, mode and lenience drawn per
case.  Outputs must match outside the oracle's near-boundary decisions, and
every call must leave the shared workspace zero (run_gpu checks it)."""
import numpy as np
import pytest

import oracle
from tests import synth
from tests.gpu_util import check_aux, compare, run_gpu, run_ref

pytestmark = pytest.mark.gpu

KINDS = ["c2", "c3", "c4", "c5"]  # fp32/fp32, bf16/fp32, bf16/bf16, bf16/bf16 (T = 1.0, 0.8, 1.0, 0.7)


@pytest.mark.parametrize("case", range(24))
def test_random_shapes(case):
    rng = np.random.default_rng(7000 + case)
    kind = KINDS[case % 4]
    B = int(rng.integers(1, 41))
    gamma = int(rng.integers(1, 13))
    V = int(np.exp(rng.uniform(0.0, np.log(70_000))))
    mode = "greedy" if rng.random() < 0.25 else "sample"
    lenience = 1.0 if mode == "greedy" or rng.random() < 0.6 else float(rng.choice([0.0, 0.3, 0.9]))
    d = synth.make_inputs(kind, 8000 + case, B=B, gamma=gamma, V=max(V, 1))
    print(f"[fuzz] case={case} {kind} B={B} gamma={gamma} V={d['V']} {mode} l={lenience}", flush=True)
    g = run_gpu(d, mode, with_aux=mode == "sample", lenience=lenience)
    if mode == "greedy":
        r = run_ref(d, mode)
    else:
        r = oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], d["draft_tokens"], d["uniforms"],
                                   d["temperature"], oracle.SAMPLE, lenience=lenience)
    compare(g, r, gamma, draft_tokens=d["draft_tokens"], vocab=d["V"])
    if mode == "sample":
        check_aux(g, r, 1e-6)
