"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
library through its binding, and compare with the oracle under the
near-boundary exemption."""
from __future__ import annotations

import numpy as np


def to_device(d: dict, device="cuda"):
    import torch

    def t(a, bf16):
        x = torch.from_numpy(np.ascontiguousarray(a))
        if bf16:
            x = x.view(torch.bfloat16)
        return x.to(device)

    out = {
        "target_logits": t(d["target_logits"], d["target_logits"].dtype == np.uint16),
        "draft_tokens": t(d["draft_tokens"], False),
    }
    if d.get("draft_probs") is not None:
        out["draft_probs"] = t(d["draft_probs"], d["draft_probs"].dtype == np.uint16)
    if d.get("uniforms") is not None:
        out["uniforms"] = t(d["uniforms"], False)
    return out


def run_gpu(d: dict, mode: str = "sample", with_aux: bool = True, dev_inputs=None, telemetry: bool = False,
            lenience: float = 1.0):
    import torch
    import exact_rejection_sampling_temp_amd as sv
    x = dev_inputs or to_device(d)
    B, G1, V = d["target_logits"].shape
    G = G1 - 1
    aux = None
    if with_aux:
        dv = x["target_logits"].device
        aux = {
            "p_tok": torch.empty((B, G), dtype=torch.float64, device=dv),
            "q_tok": torch.empty((B, G), dtype=torch.float64, device=dv),
            "resid_mass": torch.empty(B, dtype=torch.float64, device=dv),
            "row_max": torch.empty((B, G1), dtype=torch.float32, device=dv),
            "row_sum": torch.empty((B, G1), dtype=torch.float64, device=dv),
            "p_out": torch.empty(B, dtype=torch.float64, device=dv),
        }
    if telemetry:
        dv = x["target_logits"].device
        aux = aux or {}
        aux["beta"] = torch.full((B, G), float("nan"), dtype=torch.float64, device=dv)
        aux["alpha"] = torch.full((G,), float("nan"), dtype=torch.float64, device=dv)
    n, out = sv.spec_verify(x["target_logits"], x.get("draft_probs") if mode == "sample" else None,
                            x["draft_tokens"], x.get("uniforms") if mode == "sample" else None,
                            d.get("temperature", 1.0), mode, aux=aux, lenience=lenience)
    torch.cuda.synchronize()
    # every call must leave the shared workspace all zero (the next call may
    # have another shape, and so another layout of it)
    for ws in sv._ws_cache.values():
        assert int(ws.count_nonzero()) == 0, "a finished call must leave the workspace zero"
    res = {"n_accepted": n.cpu().numpy(), "out_tokens": out.cpu().numpy()}
    if aux:
        res.update({k: v.cpu().numpy() for k, v in aux.items()})
    return res


def run_ref(d: dict, mode: str = "sample", telemetry: bool = False, lenience: float = 1.0):
    import oracle  # here, not at module level: bench.py takes to_device from this module
    if mode == "greedy":
        return oracle.spec_verify_ref(d["target_logits"], None, d["draft_tokens"], None, 1.0, oracle.GREEDY)
    return oracle.spec_verify_ref(d["target_logits"], d["draft_probs"], d["draft_tokens"],
                                  d["uniforms"], d["temperature"], oracle.SAMPLE, telemetry=telemetry,
                                  lenience=lenience)


def well_formed(n, out, draft_tokens, vocab: int, gamma: int):
    """Indices of sequences whose outputs break the block-advance rule: a
    valid sequence has 0 <= n <= gamma, out[:n] == its drafts, out[n] a token
    in [0, vocab) and -1 after it; an invalid one (n = -1) is all -1."""
    pos = np.arange(gamma + 1)[None, :]
    nn = n[:, None]
    inval = n == -1
    ok_n = (n >= -1) & (n <= gamma)
    prefix = np.where(pos < nn, out == np.pad(draft_tokens, ((0, 0), (0, 1)), constant_values=-2), True)
    at_n = np.where(pos == nn, (out >= 0) & (out < vocab), True)
    after = np.where(pos > nn, out == -1, True)
    valid_ok = prefix.all(1) & at_n.all(1) & after.all(1)
    inval_ok = np.all(out == -1, axis=1)
    good = ok_n & np.where(inval, inval_ok, valid_ok)
    return np.nonzero(~good)[0]


def compare(gpu: dict, ref: dict, gamma: int, draft_tokens=None, vocab: int | None = None) -> dict:
    """Bit-exact agreement except downstream of a near-boundary decision.

    A sequence whose oracle walk has no flagged decision must match exactly.
    For a sequence whose first flagged decision is at position f, the
    outputs before f must match and n must be at least f (every later output
    depends on the flagged decision); given the draft tokens and the
    vocabulary size, every sequence's outputs must also be well formed
    (well_formed), the flagged ones included.  Returns counts for
    reporting."""
    n_g, o_g = gpu["n_accepted"], gpu["out_tokens"]
    n_r, o_r = ref["n_accepted"], ref["out_tokens"]
    fp = ref["flag_pos"]
    clean = fp < 0
    bad = np.nonzero(clean & ((n_g != n_r) | np.any(o_g != o_r, axis=1)))[0]
    if bad.size:
        b = bad[0]
        raise AssertionError(
            f"{bad.size} unflagged sequences differ; first b={b}: gpu n={n_g[b]} out={o_g[b].tolist()} "
            f"ref n={n_r[b]} out={o_r[b].tolist()}")
    flagged = np.nonzero(~clean)[0]
    for b in flagged:
        f = fp[b]
        assert n_r[b] >= 0 and f <= n_r[b], (b, f, n_r[b])
        assert f <= n_g[b] <= gamma, (b, f, n_g[b])
        assert np.array_equal(o_g[b, :f], o_r[b, :f]), b
    if draft_tokens is not None:
        assert vocab is not None
        wf = well_formed(np.asarray(n_g), np.asarray(o_g), np.asarray(draft_tokens), vocab, gamma)
        if wf.size:
            b = wf[0]
            raise AssertionError(f"{wf.size} sequences with malformed outputs; first b={b}: n={n_g[b]} "
                                 f"out={o_g[b].tolist()} drafts={np.asarray(draft_tokens)[b].tolist()}")
    return {"sequences": int(n_r.size), "flagged_sequences": int(flagged.size),
            "decisions": int(ref["n_decisions"].sum()), "flagged_decisions": int(ref["n_flags"].sum())}


def check_aux(gpu: dict, ref: dict, rtol_p: float):
    """Probabilities at the tested positions, row normalisers and the
    residual mass against the oracle (positions both sides reached)."""
    n = np.minimum(gpu["n_accepted"], ref["n_accepted"])
    B, G = ref["p_tok"].shape
    valid = n >= 0
    pos = np.arange(G)[None, :] <= n[:, None]
    sel = pos & valid[:, None]
    np.testing.assert_allclose(gpu["p_tok"][sel], ref["p_tok"][sel], rtol=rtol_p, atol=1e-12)
    np.testing.assert_array_equal(gpu["q_tok"][sel], ref["q_tok"][sel])
    rows = (np.arange(G + 1)[None, :] <= n[:, None]) & valid[:, None]
    np.testing.assert_array_equal(gpu["row_max"][rows].astype(np.float64), ref["row_max"][rows])
    np.testing.assert_allclose(gpu["row_sum"][rows], ref["row_sum"][rows], rtol=rtol_p)
    same = valid & (gpu["n_accepted"] == ref["n_accepted"]) & (ref["n_accepted"] < G)
    # Z = sum over the support A of (p_v - l q_v): each p_v carries the
    # kernel's exp2 error (<= 5.6e-11 relative, twice that after dividing by
    # S), and the subtraction keeps it absolute, so Z is off by up to
    # ~1.1e-10 * P(A) <= 1.1e-10 whatever Z is; relative to Z that grows as
    # P(A) / Z where the draft nearly matches the target on A
    np.testing.assert_allclose(gpu["resid_mass"][same], ref["resid_mass"][same], rtol=1e-9, atol=2e-10)
    # p_n of the drawn token, where both sides drew the same token at the same n
    if "p_out" in gpu:
        nn = np.clip(ref["n_accepted"], 0, G)
        rows_b = np.arange(B)
        drew = valid & (gpu["n_accepted"] == ref["n_accepted"]) & \
            (gpu["out_tokens"][rows_b, nn] == ref["out_tokens"][rows_b, nn])
        np.testing.assert_allclose(gpu["p_out"][drew], ref["p_out"][drew], rtol=1e-9, atol=1e-300)
        assert np.all(np.isnan(gpu["p_out"][gpu["n_accepted"] < 0]))
    # positions past the walk are NaN on the GPU side
    assert np.all(np.isnan(gpu["p_tok"][~sel & valid[:, None]]))
