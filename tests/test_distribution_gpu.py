"""The law of the GPU path's outputs over many trials, against its closed form
(no oracle involved): every trial repeats one fixed set of target and draft
rows with fresh draft tokens and uniforms, so the emitted tokens are i.i.d.
draws whose law follows from the rows alone.

With the stored draft row q (its sum S may differ from 1 after rounding to
the storage dtype, and the drafts are drawn from q / S) and the target
distribution p at temperature T, speculative sampling ("Fast Inference from
Transformers via Speculative Decoding", Section 2.3 and Appendix A.1) gives:

- a drafted token v is accepted at position j with probability
  min(q_j(v), p_j(v)) / S_j, so beta_j = sum_v min(q_j, p_j)(v) / S_j;
- P(n >= j) = prod_{i<j} beta_i;
- after a rejection at j the token follows norm(max(0, p_j - q_j));
- the token at position j < gamma, given n >= j, has the law
  min(q_j, p_j) / S_j + (1 - beta_j) norm(max(0, p_j - q_j)), which is p_j
  when S_j = 1; the bonus token (n = gamma) follows p_gamma.

With a lenience l in (0, 1] (same page, Appendix A.5 "Ablation Studies and
Robustness Checks": q(x) is multiplied by l before the comparison; the draw
after a rejection uses the residual of that same comparison, the library's
reading where the page gives only the acceptance side) min(q_j, p_j / l)
replaces min(q_j, p_j) and the residual is norm(max(0, p_j - l q_j)).

Each case takes a different kernel path: four sequences per wave (V <= 16),
one wave per sequence (V <= 512), and the two launches (one and several
chunks per row).  Every tensor stays below 2 GiB.
"""
import numpy as np
import pytest
import scipy.stats

from tests import synth

pytestmark = pytest.mark.gpu


def _chisq_pvalue(counts, probs):
    """Pearson's test, bins with an expected count below 5 pooled into one."""
    counts = np.asarray(counts, np.float64)
    exp = np.asarray(probs, np.float64) * counts.sum()
    keep = exp >= 5
    c = np.append(counts[keep], counts[~keep].sum())
    e = np.append(exp[keep], exp[~keep].sum())
    if e[-1] == 0:
        assert c[-1] == 0, "a token of probability zero was emitted"
        c, e = c[:-1], e[:-1]
    e = e * (c.sum() / e.sum())
    return scipy.stats.chisquare(c, e).pvalue


def _softmax64(z, T):
    z = z.astype(np.float64) / T
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _run_law_case(seed, trials, gamma, V, T, ldt, pdt, lenience=1.0):
    import torch
    import exact_rejection_sampling_temp_amd as sv

    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xD157]))
    zq = 1.5 * rng.standard_normal((gamma + 1, V))
    zp = zq + 0.7 * rng.standard_normal((gamma + 1, V))
    q_store = synth._cast(_softmax64(zq[:gamma], T), pdt)
    zp_store = synth._cast(zp, ldt)
    dec = lambda a: (synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)
    Q, P = dec(q_store), _softmax64(dec(zp_store), T)

    # draft tokens from q / S, fresh per trial; uniforms on the 2^-24 grid
    cq = np.cumsum(Q, axis=-1)
    x = np.empty((trials, gamma), np.int32)
    for j in range(gamma):
        r = rng.random(trials) * cq[j, -1]
        x[:, j] = np.minimum(np.searchsorted(cq[j], r, side="right"), V - 1)
    u = synth.draw_uniforms(rng, (trials, gamma + 1))

    def dev_rows(a, rows):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if a.dtype == np.uint16:
            t = t.view(torch.bfloat16)
        return t.cuda().unsqueeze(0).expand(trials, rows, V).contiguous()

    print(f"[law] seed={seed} trials={trials} gamma={gamma} V={V} T={T} {ldt}/{pdt} l={lenience}", flush=True)
    n, out = sv.spec_verify(dev_rows(zp_store, gamma + 1), dev_rows(q_store, gamma),
                            torch.from_numpy(x).cuda(), torch.from_numpy(u).cuda(), T, "sample",
                            lenience=lenience)
    torch.cuda.synchronize()
    n, out = n.cpu().numpy(), out.cpu().numpy()
    assert n.min() >= 0 and n.max() <= gamma

    m = np.minimum(Q, P[:gamma] / lenience)
    beta = m.sum(-1) / Q.sum(-1)
    resid = np.maximum(0.0, P[:gamma] - lenience * Q)
    resid /= resid.sum(-1, keepdims=True)
    surv = np.concatenate([[1.0], np.cumprod(beta)])
    law_n = np.append(surv[:-1] * (1 - beta), surv[-1])
    assert _chisq_pvalue(np.bincount(n, minlength=gamma + 1), law_n) > 1e-4
    for j in range(gamma + 1):
        sel = n >= j
        law = P[gamma] if j == gamma else m[j] / Q[j].sum() + (1 - beta[j]) * resid[j]
        assert _chisq_pvalue(np.bincount(out[sel, j], minlength=V), law) > 1e-4, f"position {j}"
    rej0 = n == 0
    assert _chisq_pvalue(np.bincount(out[rej0, 0], minlength=V), resid[0]) > 1e-4
    # positions past the emitted ones are -1
    cols = np.arange(gamma + 1)[None, :]
    assert np.all(out[cols > n[:, None]] == -1)


def test_law_four_sequences_per_wave():
    _run_law_case(1, 4_000_000, 4, 8, 1.0, synth.FP32, synth.FP32)


def test_law_one_wave_per_sequence():
    _run_law_case(2, 400_000, 5, 300, 0.8, synth.BF16, synth.BF16)


def test_law_two_launches_one_chunk():
    _run_law_case(3, 60_000, 3, 3000, 0.7, synth.BF16, synth.BF16)


def test_law_two_launches_several_chunks():
    _run_law_case(4, 4_000, 2, 40_000, 1.0, synth.BF16, synth.FP32)


@pytest.mark.parametrize("lenience", [0.4, 0.8])
def test_law_lenient_four_sequences_per_wave(lenience):
    _run_law_case(5, 2_000_000, 4, 8, 1.0, synth.FP32, synth.FP32, lenience)


@pytest.mark.parametrize("lenience", [0.4, 0.8])
def test_law_lenient_two_launches(lenience):
    _run_law_case(6, 60_000, 3, 3000, 0.7, synth.BF16, synth.BF16, lenience)
