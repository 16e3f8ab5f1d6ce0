"""GPU parity of top-k / nucleus standardisation (sv_standardize) against the
fp64 oracle ("Fast Inference from Transformers via Speculative Decoding",
summary page, "Standardized Sampling"), through the C ABI (via the binding):
the standardised rows must be bit-identical (top-k always; nucleus outside
rows the oracle flags as within 1e-9 of the top_p boundary), and the verify
step on standardised target rows with a standardised draft must match the
oracle's verify on its own standardised rows."""
import numpy as np
import pytest

import oracle
from tests import synth
from tests.gpu_util import compare, run_gpu, run_ref

pytestmark = pytest.mark.gpu


def _gpu_std(z, method, k=0, top_p=1.0, T=1.0, inplace=False):
    import torch
    import exact_rejection_sampling_temp_amd as sv
    t = torch.from_numpy(np.ascontiguousarray(z))
    if z.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    t = t.to("cuda")
    out = sv.standardize(t, method, k=k, top_p=top_p, temperature=T, out=t if inplace else None)
    torch.cuda.synchronize()
    o = out.cpu()
    return (o.view(torch.uint16) if z.dtype == np.uint16 else o).numpy()


def _check(z, method, **kw):
    code = oracle.TOPK if method == "topk" else oracle.TOPP
    want, kept, flag = oracle.standardize(z, code, k=kw.get("k", 0), top_p=kw.get("top_p", 1.0),
                                          temperature=kw.get("T", 1.0))
    got = _gpu_std(z, method, **kw)
    ok = flag == 0
    assert ok.sum() >= max(1, len(ok) // 2)
    bad = np.nonzero(ok & np.any(got != want, axis=1))[0]
    assert bad.size == 0, (method, kw, bad[:5], kept[bad[:5]])
    return kept


def _c4_rows(n, seed):
    d = synth.make_inputs("c4", seed, B=max(1, n // 9))
    return np.ascontiguousarray(d["target_logits"].reshape(-1, d["V"])[:n])


@pytest.mark.parametrize("k", [1, 50, 1000, 152_064])
def test_topk_c4_rows(k):
    print(f"[standardize] topk k={k} c4 rows", flush=True)
    kept = _check(_c4_rows(36, 1), "topk", k=k)
    assert np.all(kept == min(k, 152_064))


@pytest.mark.parametrize("top_p", [0.3, 0.9, 0.99, 1.0])
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_topp_c4_rows(top_p, T):
    print(f"[standardize] topp p={top_p} T={T} c4 rows", flush=True)
    z = _c4_rows(36, 2)
    if top_p == 1.0:
        # the whole distribution: every entry stays, on both sides
        assert np.array_equal(_gpu_std(z, "topp", top_p=1.0, T=T), z)
        assert np.array_equal(oracle.standardize(z, oracle.TOPP, top_p=1.0, temperature=T)[0], z)
        return
    _check(z, "topp", top_p=top_p, T=T)


@pytest.mark.parametrize("method,kw", [("topk", dict(k=17)), ("topk", dict(k=999)), ("topp", dict(top_p=0.8)),
                                       ("topp", dict(top_p=0.999, T=1.3))])
def test_fp32_rows_with_ties_inf_and_signed_zero(method, kw):
    rng = np.random.default_rng(5)
    z = np.round(rng.standard_normal((24, 32_000)) * 3, 1).astype(np.float32)   # many ties
    z[:, rng.integers(0, 32_000, 500)] = -np.inf
    z[:, :40] = 0.0
    z[:, 40:80] = -0.0
    _check(z, method, **kw)


@pytest.mark.parametrize("V", [1, 7, 1001, 20_001])
def test_scalar_path_ragged_vocab(V):
    rng = np.random.default_rng(V)
    zb = synth.f32_to_bf16_bits(np.round(rng.standard_normal((9, V)) * 2, 1).astype(np.float32))
    _check(zb, "topk", k=3)
    _check(zb, "topp", top_p=0.7)
    zf = rng.standard_normal((5, V)).astype(np.float32)
    _check(zf, "topk", k=max(1, V // 3))
    _check(zf, "topp", top_p=0.5, T=0.8)


def test_in_place():
    z = _c4_rows(9, 3)
    want, _, _ = oracle.standardize(z, oracle.TOPK, k=64)
    assert np.array_equal(_gpu_std(z, "topk", k=64, inplace=True), want)


@pytest.mark.parametrize("k", [2, 20])
def test_verify_on_standardised_rows(k):
    """Standardised target rows (GPU) and a standardised draft: the verify
    step matches the oracle's verify on the oracle's standardised rows."""
    d = synth.standardize_draft_topk(synth.make_inputs("c4", 40 + k, B=16, V=30_000), k, seed=k)
    z = d["target_logits"]
    B, G1, V = z.shape
    zs = _gpu_std(z.reshape(-1, V), "topk", k=k).reshape(B, G1, V)
    want, _, _ = oracle.standardize(z.reshape(-1, V), oracle.TOPK, k=k)
    assert np.array_equal(zs, want.reshape(B, G1, V))
    ds = dict(d)
    ds["target_logits"] = zs
    g = run_gpu(ds)
    r = run_ref(ds)
    compare(g, r, d["gamma"], draft_tokens=d["draft_tokens"], vocab=d["V"])
    # every emitted token is inside its row's top-k
    for b in range(B):
        n = r["n_accepted"][b]
        t = g["out_tokens"][b, n]
        assert zs[b, n, t] != 0xff80


@pytest.mark.parametrize("method,kw", [("topk", dict(k=9)), ("topk", dict(k=999)), ("topp", dict(top_p=0.6)),
                                       ("topp", dict(top_p=0.95, T=0.8))])
def test_bf16_rows_with_ties_inf_and_signed_zero(method, kw):
    """bf16 rows rounded to few distinct values (long runs of ties), -inf
    entries and both zeros: the 16-bit key histogram, the tie counts per
    wave run and the packed output pass."""
    rng = np.random.default_rng(11)
    z = np.round(rng.standard_normal((16, 50_000)) * 2, 1).astype(np.float32)
    z[:, rng.integers(0, 50_000, 300)] = -np.inf
    z[:, 100:140] = 0.0
    z[:, 140:180] = -0.0
    _check(synth.f32_to_bf16_bits(z), method, **kw)


@pytest.mark.parametrize("method,kw", [("topk", dict(k=5)), ("topk", dict(k=66_500)), ("topp", dict(top_p=0.5)),
                                       ("topp", dict(top_p=0.999))])
def test_bf16_value_repeated_past_16_bit_counts(method, kw):
    """One value occurs 66 000 times in a row of 70 000: its 16-bit counter
    wraps, the total count shows it, and the row takes the radix select."""
    rng = np.random.default_rng(12)
    V = 70_000
    z = (rng.standard_normal((4, V)) * 2).astype(np.float32)
    for r in range(4):
        z[r, rng.permutation(V)[:66_000]] = 0.5 if r % 2 == 0 else -1.25
    _check(synth.f32_to_bf16_bits(z), method, **kw)


@pytest.mark.parametrize("method,kw", [("topk", dict(k=30_000)), ("topk", dict(k=3)), ("topp", dict(top_p=0.5)),
                                       ("topp", dict(top_p=0.97, T=2.0))])
def test_bf16_long_tie_runs(method, kw):
    """bf16 rows of ~7 distinct values over 150 000 entries: the final key
    has tens of thousands of ties, more than a wave's tie list holds, so the
    wave holding the last kept tie ranks its run again."""
    rng = np.random.default_rng(13)
    z = np.round(rng.standard_normal((6, 150_000))).astype(np.float32)
    _check(synth.f32_to_bf16_bits(z), method, **kw)


@pytest.mark.parametrize("method,kw", [("topk", dict(k=50)), ("topk", dict(k=120_000)), ("topp", dict(top_p=0.9)),
                                       ("topp", dict(top_p=0.5, T=0.7))])
@pytest.mark.parametrize("V", [155_648, 155_656, 200_000])
def test_bf16_rows_at_and_past_the_register_path(method, kw, V):
    """bf16 rows whose every wave run just fits in registers (V = 155 648)
    and rows one group longer or much longer (read twice), with ties."""
    rng = np.random.default_rng(15)
    z = (rng.standard_normal((3, V)) * 3).astype(np.float32)
    z[1] = np.round(z[1], 1)
    _check(synth.f32_to_bf16_bits(z), method, **kw)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_degenerate_rows(dt):
    """Rows of -inf only, a single finite entry among -inf, half -inf,
    one-entry rows, and k at 1, 2, V - 1, V and past V."""
    rng = np.random.default_rng(14)
    V = 4096
    z = (rng.standard_normal((6, V)) * 2).astype(np.float32)
    z[0] = -np.inf                      # no finite entry
    z[1] = -np.inf
    z[1, 1234] = 0.75                   # one finite entry
    z[2, :V // 2] = -np.inf
    zz = synth.f32_to_bf16_bits(z) if dt == "bf16" else z
    for k in (1, 2, V - 1):
        _check(zz, "topk", k=k)
    for k in (V, V + 5):                # the whole row
        assert np.array_equal(_gpu_std(zz, "topk", k=k), zz)
    for top_p in (0.5, 0.999):
        _check(zz[1:], "topp", top_p=top_p)
        # no finite entry: no mass to reach top_p, every entry stays
        assert np.array_equal(_gpu_std(zz[:1], "topp", top_p=top_p), zz[:1])
    one = np.ascontiguousarray(zz[1:, :1])
    for k in (1, 3):
        assert np.array_equal(_gpu_std(one, "topk", k=k), one)
    finite = one[np.isfinite(synth.bf16_bits_to_f32(one) if dt == "bf16" else one)[:, 0]]
    _check(finite, "topp", top_p=0.5)
