"""MI355X-native verify-and-sample step of speculative decoding.

Thin ctypes binding over the C ABI in ``include/spec_verify.h`` (shared
library ``libspecverify.so`` in this directory, built for gfx950 by
``exact_rejection_sampling_temp_amd.build``).  This module only checks
shapes and dtypes and passes device pointers and the current HIP stream;
every step of the computation runs in the library's kernels.  There is no
fallback: if the library is missing or no GPU is visible, calls raise.

PyTorch supplies device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspecverify.so")

# Values of the C ABI's constants (include/spec_verify.h).
SV_FP32 = 0
SV_BF16 = 1
SV_SAMPLE = 0
SV_GREEDY = 1
SV_MAX_GAMMA = 63
SV_OK = 0
SV_TOPK = 0
SV_TOPP = 1

__all__ = [
    "spec_verify", "spec_verify_noalloc", "standardize", "sv_workspace_bytes", "sv_workspace_init", "sv_status_string",
    "SpecVerifyError", "load_library", "EXPORTED_SYMBOLS",
    "SV_FP32", "SV_BF16", "SV_SAMPLE", "SV_GREEDY", "SV_MAX_GAMMA",
]

EXPORTED_SYMBOLS = ("spec_verify", "spec_verify_lenient", "spec_verify_noalloc", "sv_workspace_bytes",
                    "sv_workspace_init", "sv_status_string", "sv_standardize", "sv_extras_bytes")


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, where: str = "spec_verify"):
        super().__init__(f"{where} failed with status {status}: {sv_status_string(status)}")
        self.status = status


class Extras(ctypes.Structure):
    """Mirror of sv_extras_t."""
    _fields_ = [
        ("p_tok", ctypes.c_void_p),
        ("q_tok", ctypes.c_void_p),
        ("resid_mass", ctypes.c_void_p),
        ("row_max", ctypes.c_void_p),
        ("row_sum", ctypes.c_void_p),
        ("p_out", ctypes.c_void_p),
        ("ev_begin", ctypes.c_void_p),
        ("ev_mid", ctypes.c_void_p),
        ("ev_end", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("alpha", ctypes.c_void_p),
        ("ev_tele", ctypes.c_void_p),
        ("error_count", ctypes.c_void_p),
        ("withhold_partial", ctypes.c_int32),
        ("wait_polls", ctypes.c_int32),
        ("help_polls", ctypes.c_int32),
    ]


_lib = None
_lib_lock = threading.Lock()


def load_library(path: str = LIB_PATH):
    """Load the HIP library (no GPU needed to load it).

    torch is imported first so that its HIP runtime is the one in the
    process: the library's libamdhip64.so.7 dependency then binds to it by
    soname instead of loading a second runtime from /opt/rocm."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        import torch  # noqa: F401  (see docstring)
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build it first (python -m exact_rejection_sampling_temp_amd.build)")
        lib = ctypes.CDLL(path)
        lib.sv_extras_bytes.restype = ctypes.c_size_t
        lib.sv_extras_bytes.argtypes = []
        if lib.sv_extras_bytes() != ctypes.sizeof(Extras):
            raise ImportError(f"{path}: sv_extras_t is {lib.sv_extras_bytes()} bytes, the binding's mirror "
                              f"{ctypes.sizeof(Extras)}: rebuild the library or update Extras")
        lib.sv_workspace_bytes.restype = ctypes.c_size_t
        lib.sv_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.sv_workspace_init.restype = ctypes.c_int
        lib.sv_workspace_init.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.sv_status_string.restype = ctypes.c_char_p
        lib.sv_status_string.argtypes = [ctypes.c_int]
        lib.spec_verify.restype = ctypes.c_int
        lib.spec_verify.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
            ctypes.POINTER(Extras), ctypes.c_void_p,
        ]
        lib.sv_standardize.restype = ctypes.c_int
        lib.sv_standardize.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                       ctypes.c_void_p]
        lib.spec_verify_lenient.restype = ctypes.c_int
        lib.spec_verify_lenient.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_float, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
            ctypes.POINTER(Extras), ctypes.c_void_p,
        ]
        lib.spec_verify_noalloc.restype = ctypes.c_int
        lib.spec_verify_noalloc.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_float, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p,
            ctypes.POINTER(Extras), ctypes.c_void_p,
        ]
        _lib = lib
        return lib


def sv_workspace_bytes(batch: int, gamma: int, vocab: int) -> int:
    return int(load_library().sv_workspace_bytes(batch, gamma, vocab))


def sv_status_string(status: int) -> str:
    return load_library().sv_status_string(int(status)).decode()


def sv_workspace_init(workspace, stream=None) -> None:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(workspace.device)
    rc = load_library().sv_workspace_init(ctypes.c_void_p(workspace.data_ptr()),
                                          workspace.numel() * workspace.element_size(),
                                          ctypes.c_void_p(s.cuda_stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "sv_workspace_init")


# One zero-initialised workspace per (device, stream), grown on demand.  It
# is allocated and zero-filled on the stream that uses it, so the fill is
# ordered before that stream's kernels, a replaced (smaller) one is freed
# through the caching allocator on the same stream, and calls on different
# streams never share one.
_ws_cache: dict = {}


def _workspace(device, nbytes: int, stream):
    import torch
    key = (device.type, device.index, int(stream.cuda_stream))
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(stream):
            ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


_AUX_SPEC = {"p_tok": ("float64", "BG"), "q_tok": ("float64", "BG"), "resid_mass": ("float64", "B"),
             "p_out": ("float64", "B"),
             "row_max": ("float32", "BG1"), "row_sum": ("float64", "BG1"),
             "beta": ("float64", "BG"), "alpha": ("float64", "G")}


def _check_out(t, dtype, numel, dev, name):
    if t.dtype != dtype or t.numel() != numel or t.device != dev or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of {numel} elements on {dev}")


def _dtype_tag(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return SV_FP32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"expected float32 or bfloat16, got {t.dtype}")


def spec_verify(target_logits, draft_probs, draft_tokens, uniforms, temperature: float = 1.0,
                mode: str | int = "sample", *, n_accepted=None, out_tokens=None, workspace=None,
                aux: dict | None = None, events=None, stream=None, lenience: float = 1.0,
                error_count=None, _test_withhold_partial: int = 0, _test_wait_polls: int = 0,
                _test_help_polls: int = 0, _noalloc: bool = False):
    """Batched verify-and-sample on the GPU.

    target_logits [B, gamma+1, V] fp32/bf16, draft_probs [B, gamma, V] fp32/bf16
    (None in greedy mode), draft_tokens [B, gamma] int32, uniforms [B, gamma+1]
    fp32 (None in greedy mode), all CUDA/HIP tensors on one device.
    Returns (n_accepted [B] int32, out_tokens [B, gamma+1] int32).

    ``aux``: optional dict of preallocated device tensors with keys among
    p_tok [B,gamma] f64, q_tok [B,gamma] f64, resid_mass [B] f64,
    row_max [B,gamma+1] f32, row_sum [B,gamma+1] f64, p_out [B] f64 (p_n of the
    drawn token), and the acceptance-rate
    telemetry beta [B,gamma] f64 / alpha [gamma] f64 (sample mode; either one
    makes the call stream every row, see include/spec_verify.h).
    ``events``: optional (begin, mid, end) or (begin, mid, end, tele) raw
    hipEvent_t handles (ints); tele is recorded after the telemetry sweep.
    ``lenience``: l in [0, 1] (spec_verify_lenient); 1 calls spec_verify.
    ``error_count``: optional uint32 device counter (one element, zeroed by
    the caller) of sequences whose outputs were withheld because a bounded
    device-side wait ran out (n_accepted = -2).  ``_test_withhold_partial``,
    ``_test_wait_polls``: sv_extras_t's test hooks for that failure path;
    ``_test_help_polls``: its hook bounding the draw helpers' wait.
    """
    import torch
    lib = load_library()
    m = mode if isinstance(mode, int) else {"sample": SV_SAMPLE, "greedy": SV_GREEDY}[mode]
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, gamma+1, V]")
    B, G1, V = target_logits.shape
    gamma = G1 - 1
    dev = target_logits.device
    if dev.type != "cuda":
        raise ValueError("spec_verify runs on the GPU only; tensors must be on a HIP device")
    tensors = [target_logits, draft_tokens]
    if m == SV_SAMPLE:
        if draft_probs is None or uniforms is None:
            raise ValueError("sample mode needs draft_probs and uniforms")
        if tuple(draft_probs.shape) != (B, gamma, V):
            raise ValueError(f"draft_probs must be {(B, gamma, V)}, got {tuple(draft_probs.shape)}")
        if tuple(uniforms.shape) != (B, G1) or uniforms.dtype != torch.float32:
            raise ValueError(f"uniforms must be float32 {(B, G1)}")
        tensors += [draft_probs, uniforms]
    if tuple(draft_tokens.shape) != (B, gamma) or draft_tokens.dtype != torch.int32:
        raise ValueError(f"draft_tokens must be int32 {(B, gamma)}")
    for t in tensors:
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if n_accepted is None:
        n_accepted = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, G1), dtype=torch.int32, device=dev)
    _check_out(n_accepted, torch.int32, B, dev, "n_accepted")
    _check_out(out_tokens, torch.int32, B * G1, dev, "out_tokens")
    for k, t in (aux or {}).items():
        if k not in _AUX_SPEC:
            raise ValueError(f"unknown aux output {k!r}")
        dt, per = _AUX_SPEC[k]
        _check_out(t, getattr(torch, dt), {"B": B, "G": gamma, "BG": B * gamma, "BG1": B * G1}[per], dev, k)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    if workspace is None and not _noalloc:
        workspace = _workspace(dev, lib.sv_workspace_bytes(B, gamma, V), s)
    ex = None
    if error_count is not None:
        _check_out(error_count, torch.int32, 1, dev, "error_count")
    if aux or events or error_count is not None or _test_withhold_partial or _test_wait_polls or _test_help_polls:
        ex = Extras()
        if error_count is not None:
            ex.error_count = error_count.data_ptr()
        ex.withhold_partial = int(_test_withhold_partial)
        ex.wait_polls = int(_test_wait_polls)
        ex.help_polls = int(_test_help_polls)
        for k, t in (aux or {}).items():
            setattr(ex, k, t.data_ptr())
        if events:
            ex.ev_begin, ex.ev_mid, ex.ev_end = events[:3]
            if len(events) > 3:
                ex.ev_tele = events[3]
    head = (B, gamma, V,
            target_logits.data_ptr(), _dtype_tag(target_logits),
            draft_probs.data_ptr() if (m == SV_SAMPLE) else None,
            _dtype_tag(draft_probs) if m == SV_SAMPLE else 0,
            draft_tokens.data_ptr(), uniforms.data_ptr() if m == SV_SAMPLE else None,
            float(temperature))
    if _noalloc:
        rc = lib.spec_verify_noalloc(*head, float(lenience), m, n_accepted.data_ptr(), out_tokens.data_ptr(),
                                     ctypes.byref(ex) if ex is not None else None, s.cuda_stream)
        if rc != SV_OK:
            raise SpecVerifyError(rc, "spec_verify_noalloc")
        return n_accepted, out_tokens
    tail = (m, n_accepted.data_ptr(), out_tokens.data_ptr(),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            ctypes.byref(ex) if ex is not None else None,
            s.cuda_stream)
    if lenience == 1.0:
        rc = lib.spec_verify(*head, *tail)
    else:
        rc = lib.spec_verify_lenient(*head, float(lenience), *tail)
    if rc != SV_OK:
        raise SpecVerifyError(rc)
    return n_accepted, out_tokens


def spec_verify_noalloc(target_logits, draft_probs, draft_tokens, uniforms, temperature: float = 1.0,
                        mode: str | int = "sample", *, n_accepted=None, out_tokens=None, aux: dict | None = None,
                        events=None, stream=None, lenience: float = 1.0, error_count=None):
    """spec_verify through the allocation-free entry point spec_verify_noalloc
    (its workspace is the library's static per-GPU scratch array; calls that
    overlap on one GPU race).  For callers that cannot allocate, pass
    preallocated ``n_accepted`` and ``out_tokens``: then nothing is allocated
    on any path of the call.  Arguments and results as for spec_verify."""
    return spec_verify(target_logits, draft_probs, draft_tokens, uniforms, temperature, mode,
                       n_accepted=n_accepted, out_tokens=out_tokens, aux=aux, events=events, stream=stream,
                       lenience=lenience, error_count=error_count, _noalloc=True)


def standardize(logits, method: str | int, k: int = 0, top_p: float = 1.0, temperature: float = 1.0, *,
                out=None, stream=None):
    """Top-k ("topk", k) or nucleus ("topp", top_p at temperature T)
    standardisation of the rows of ``logits`` (any shape [..., V], fp32 or
    bf16, contiguous, on the GPU): returns ``out`` (new, or the given tensor,
    which may be ``logits`` itself) holding the rows with every dropped entry
    set to -inf (sv_standardize in include/spec_verify.h)."""
    import torch
    lib = load_library()
    m = method if isinstance(method, int) else {"topk": SV_TOPK, "topp": SV_TOPP}[method]
    if logits.device.type != "cuda":
        raise ValueError("standardize runs on the GPU only")
    if not logits.is_contiguous() or logits.dim() < 1:
        raise ValueError("logits must be a contiguous tensor [..., V]")
    V = logits.shape[-1]
    rows = logits.numel() // max(V, 1)
    if out is None:
        out = torch.empty_like(logits)
    elif out.shape != logits.shape or out.dtype != logits.dtype or out.device != logits.device or \
            not out.is_contiguous():
        raise ValueError("out must match logits")
    s = stream if stream is not None else torch.cuda.current_stream(logits.device)
    rc = lib.sv_standardize(rows, V, logits.data_ptr(), _dtype_tag(logits), m, int(k), float(top_p),
                            float(temperature), out.data_ptr(), s.cuda_stream)
    if rc != SV_OK:
        raise SpecVerifyError(rc, "sv_standardize")
    return out
