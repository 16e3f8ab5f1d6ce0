"""The allocation-free entry point spec_verify_noalloc against spec_verify.

spec_verify_noalloc runs the same kernels on the library's static per-GPU
scratch array instead of a caller's workspace.  Each case makes calls in a
row on that one array, a later one with a smaller input than the one before,
and checks every call bit for bit against spec_verify on the same inputs and
against the oracle under the near-boundary exemption.
"""
import numpy as np
import pytest

from tests import synth
from tests.gpu_util import compare, run_ref, to_device

pytestmark = pytest.mark.gpu

_AUX = (("p_tok", "float64", "BG"), ("q_tok", "float64", "BG"), ("resid_mass", "float64", "B"),
        ("row_max", "float32", "BG1"), ("row_sum", "float64", "BG1"), ("p_out", "float64", "B"))


def _aux(B, gamma, dev):
    import torch
    shape = {"BG": (B, gamma), "B": (B,), "BG1": (B, gamma + 1)}
    return {k: torch.full(shape[s], float("nan"), dtype=getattr(torch, dt), device=dev) for k, dt, s in _AUX}


def _run(fn, d, x, mode, lenience, with_aux):
    import torch
    B, gamma = d["B"], d["gamma"]
    dev = x["target_logits"].device
    n = torch.full((B,), -7, dtype=torch.int32, device=dev)
    out = torch.full((B, gamma + 1), -7, dtype=torch.int32, device=dev)
    aux = _aux(B, gamma, dev) if with_aux else None
    fn(x["target_logits"], x.get("draft_probs") if mode == "sample" else None, x["draft_tokens"],
       x.get("uniforms") if mode == "sample" else None, d.get("temperature", 1.0), mode,
       n_accepted=n, out_tokens=out, aux=aux, lenience=lenience)
    torch.cuda.synchronize()
    res = {"n_accepted": n.cpu().numpy(), "out_tokens": out.cpu().numpy()}
    for k, v in (aux or {}).items():
        res[k] = v.cpu().numpy()
    return res


def _check_one(name, seed, mode="sample", lenience=1.0, with_aux=True, oracle=True, **shape):
    import exact_rejection_sampling_temp_amd as sv
    d = synth.make_inputs(name, seed, **shape)
    print(f"[noalloc] {name} seed={seed} mode={mode} l={lenience} B={d['B']} gamma={d['gamma']} V={d['V']}",
          flush=True)
    x = to_device(d)
    got = _run(sv.spec_verify_noalloc, d, x, mode, lenience, with_aux)
    want = _run(sv.spec_verify, d, x, mode, lenience, with_aux)
    for k in want:
        np.testing.assert_array_equal(got[k], want[k], err_msg=k)
    if oracle:
        r = run_ref(d, mode, lenience=lenience)
        compare(got, r, d["gamma"], draft_tokens=d["draft_tokens"], vocab=d["V"])
    return got


def test_noalloc_sample_calls_in_a_row_shrinking():
    # full-size bf16 rows first, then smaller inputs on the same scratch array
    _check_one("c4", 7001, oracle=False)
    _check_one("c3", 7002)
    _check_one("c2", 7003)
    _check_one("c2", 7004, B=3, gamma=2, V=4_099)


def test_noalloc_greedy_and_lenient_in_a_row():
    _check_one("c3", 7011, mode="greedy")
    _check_one("c2", 7012, mode="greedy", B=5, V=9_000)
    _check_one("c2", 7013, lenience=0.5)
    _check_one("c2", 7014, lenience=0.8, B=2, gamma=3, V=2_000)


def test_noalloc_single_wave_path_needs_no_scratch():
    # rows of at most 512 entries take the one-wave-per-sequence path
    _check_one("c2", 7021, B=40, gamma=4, V=300)
    _check_one("c2", 7022, B=6, gamma=3, V=17)


def test_noalloc_allocates_nothing_and_rejects_too_large():
    import torch
    import exact_rejection_sampling_temp_amd as sv
    d = synth.make_inputs("c2", 7031)
    x = to_device(d)
    B, gamma = d["B"], d["gamma"]
    n = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty((B, gamma + 1), dtype=torch.int32, device="cuda")
    sv.spec_verify_noalloc(x["target_logits"], x["draft_probs"], x["draft_tokens"], x["uniforms"],
                           d["temperature"], n_accepted=n, out_tokens=out)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats()["allocation.all.allocated"]
    sv.spec_verify_noalloc(x["target_logits"], x["draft_probs"], x["draft_tokens"], x["uniforms"],
                           d["temperature"], n_accepted=n, out_tokens=out)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats()["allocation.all.allocated"] == before
    r = run_ref(d)
    compare({"n_accepted": n.cpu().numpy(), "out_tokens": out.cpu().numpy()}, r, gamma,
            draft_tokens=d["draft_tokens"], vocab=d["V"])
    # a batch whose workspace exceeds the array is refused before any launch
    big = torch.empty((4096, 9, 152_064), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sv.SpecVerifyError) as e:
        sv.spec_verify_noalloc(big, None, torch.zeros((4096, 8), dtype=torch.int32, device="cuda"), None,
                               1.0, "greedy")
    assert "scratch" in str(e.value)
    del big
    # and the array is still good for the next call
    _check_one("c2", 7032, with_aux=False)
