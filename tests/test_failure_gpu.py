"""The failure path of the row merge's bounded wait, forced from the host.

A row's last workgroup merges the partial (max, sum) of every chunk and waits,
bounded, for each partial to land.  Should that wait ever run out, the
library must not emit a token built from an incomplete normaliser: the
sequence is reported with n_accepted = -2, every token -1, and counted in
the caller's error counter.  The test makes the wait run out on purpose from
the host, with the extras' test hooks (the first chunk of every row at one
position withholds its partial; the wait is bounded to a few polls), so every
kernel still completes normally.  A normal call on the same workspace then
shows that the failed call left it clean.
"""
import numpy as np
import pytest

from tests import synth
from tests.gpu_util import compare, run_ref, to_device

pytestmark = pytest.mark.gpu


def _call(d, x, **kw):
    import torch
    import exact_rejection_sampling_temp_amd as sv
    n, out = sv.spec_verify(x["target_logits"], x["draft_probs"], x["draft_tokens"], x["uniforms"],
                            d["temperature"], "sample", **kw)
    torch.cuda.synchronize()
    return n.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("position", [0, 2])
def test_merge_wait_that_runs_out_withholds_the_outputs(position):
    import torch
    import exact_rejection_sampling_temp_amd as sv
    d = synth.make_inputs("c4", 1300 + position, B=12, gamma=4, V=40_000)
    print(f"[failure] position={position} B={d['B']} V={d['V']}", flush=True)
    x = to_device(d)
    r = run_ref(d)
    errs = torch.zeros(1, dtype=torch.int32, device="cuda")
    n, out = _call(d, x, error_count=errs, _test_withhold_partial=position + 1, _test_wait_polls=2)
    # every sequence whose walk reached the position has a row there whose
    # merge ran out: withheld; the others are untouched and exact
    reached = r["n_accepted"] >= position
    assert np.all(n[reached] == -2) and np.all(out[reached] == -1)
    if (~reached).any():
        assert np.array_equal(n[~reached], r["n_accepted"][~reached])
        assert np.array_equal(out[~reached], r["out_tokens"][~reached])
    assert int(errs.item()) == int(reached.sum())
    for ws in sv._ws_cache.values():
        assert int(ws.count_nonzero()) == 0, "a failed call must still leave the workspace zero"
    # the same workspace, a normal call: exact again
    n2, out2 = _call(d, x)
    compare({"n_accepted": n2, "out_tokens": out2}, r, d["gamma"], draft_tokens=d["draft_tokens"], vocab=d["V"])


@pytest.mark.parametrize("cfg,B,V,polls", [("c4", 12, 40_000, 1), ("c3", 16, 30_001, 1), ("c4", 256, 152_064, 1),
                                           ("c5", 32, 256_000, 1), ("c4", 64, 152_064, 64)])
def test_draw_chunks_the_helpers_leave_to_the_last_launch(cfg, B, V, polls):
    """The first launch's draw helpers wait for their sequence at most
    `polls` polls here, so that most of them give up and the last launch
    computes their chunks (all of them for the small grids, a mix for the
    large ones).  The outputs are the oracle's, and the workspace is left
    zero."""
    import torch
    import exact_rejection_sampling_temp_amd as sv
    d = synth.make_inputs(cfg, 1320 + B, B=B, V=V)
    print(f"[helpers] {cfg} B={d['B']} gamma={d['gamma']} V={d['V']} polls={polls}", flush=True)
    x = to_device(d)
    r = run_ref(d)
    n, out = _call(d, x, _test_help_polls=polls)
    compare({"n_accepted": n, "out_tokens": out}, r, d["gamma"], draft_tokens=d["draft_tokens"], vocab=d["V"])
    for ws in sv._ws_cache.values():
        assert int(ws.count_nonzero()) == 0


def test_calls_on_another_stream():
    import torch
    import exact_rejection_sampling_temp_amd as sv
    d = synth.make_inputs("c4", 1310, B=8, gamma=4, V=30_000)
    x = to_device(d)
    r = run_ref(d)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        n, out = sv.spec_verify(x["target_logits"], x["draft_probs"], x["draft_tokens"], x["uniforms"],
                                d["temperature"], "sample")
    s.synchronize()
    compare({"n_accepted": n.cpu().numpy(), "out_tokens": out.cpu().numpy()}, r, d["gamma"],
            draft_tokens=d["draft_tokens"], vocab=d["V"])
    keys = [k for k in sv._ws_cache if k[2] == int(s.cuda_stream)]
    assert len(keys) == 1, "the call's workspace belongs to its stream"
