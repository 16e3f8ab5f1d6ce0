"""fp64 CPU oracle for the speculative-decoding verify-and-sample step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  It shares no code
with the HIP library and the library never calls it.

The arithmetic lives in ``spec_verify_ref.c`` (plain C, double precision,
sequential sums); this module only compiles it with gcc and marshals numpy
arrays through ctypes.  Closed-form helpers used to pin the oracle live in
``oracle.analysis``.

Dtype and mode codes are this module's own: FP32 = 0, BF16 = 1 (bf16 arrays
are passed as their raw uint16 bit patterns); SAMPLE = 0, GREEDY = 1.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

FP32 = 0
BF16 = 1
SAMPLE = 0
GREEDY = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_verify_ref.c")
_LIB = os.path.join(_HERE, "libspecverify_ref.so")

# Strict IEEE double: no fast-math, no FMA contraction, so the oracle's sums
# are the plain sequential sums the source states.
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/libspecverify_ref.so``."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + res.stdout + res.stderr)
    if verbose and res.stderr:
        print(res.stderr)
    os.replace(tmp, _LIB)
    return _LIB


class _Aux(ctypes.Structure):
    _fields_ = [
        ("p_tok", ctypes.c_void_p),
        ("q_tok", ctypes.c_void_p),
        ("thr", ctypes.c_void_p),
        ("resid_mass", ctypes.c_void_p),
        ("row_max", ctypes.c_void_p),
        ("row_sum", ctypes.c_void_p),
        ("flag_pos", ctypes.c_void_p),
        ("n_decisions", ctypes.c_void_p),
        ("n_flags", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("alpha", ctypes.c_void_p),
        ("p_out", ctypes.c_void_p),
    ]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    lib.spec_verify_ref.restype = ctypes.c_int
    lib.spec_verify_ref.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_float, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(_Aux), ctypes.c_int,
    ]
    lib.ref_softmax_row.restype = ctypes.c_int
    lib.ref_softmax_row.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_float, ctypes.c_void_p]
    lib.ref_icdf.restype = ctypes.c_int
    lib.ref_icdf.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_double,
                             ctypes.POINTER(ctypes.c_int)]
    lib.ref_argmax_row.restype = ctypes.c_int
    lib.ref_argmax_row.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
    _lib = lib
    return lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return FP32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle inputs must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def spec_verify_ref(target_logits: np.ndarray, draft_probs: np.ndarray | None,
                    draft_tokens: np.ndarray, uniforms: np.ndarray | None,
                    temperature: float, mode: int = SAMPLE, n_threads: int = 0,
                    aux: bool = True, telemetry: bool = False, lenience: float = 1.0) -> dict:
    """Run the oracle on host arrays.

    target_logits: [B, gamma+1, V] float32 or uint16 (bf16 bits)
    draft_probs:   [B, gamma, V]   float32 or uint16, or None in greedy mode
    draft_tokens:  [B, gamma] int32
    uniforms:      [B, gamma+1] float32, or None in greedy mode
    Returns a dict with n_accepted [B], out_tokens [B, gamma+1] and, when
    ``aux``, the per-decision diagnostics (see spec_verify_ref.c); with
    ``telemetry`` also beta [B, gamma] (sum_v min(p_i, q_i) for every
    position) and alpha [gamma] (its mean over the batch).  ``lenience`` l in
    [0, 1] scales q before the acceptance comparison and in the residual
    (see spec_verify_ref.c); 1 is the exact method.
    """
    lib = _load()
    zl = np.ascontiguousarray(target_logits)
    B, G1, V = zl.shape
    G = G1 - 1
    x = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    assert x.shape == (B, G)
    qp = None if draft_probs is None else np.ascontiguousarray(draft_probs)
    if qp is not None:
        assert qp.shape == (B, G, V)
    u = None if uniforms is None else np.ascontiguousarray(uniforms, dtype=np.float32)
    if u is not None:
        assert u.shape == (B, G1)
    n_acc = np.empty(B, dtype=np.int32)
    out = np.empty((B, G1), dtype=np.int32)
    res = {"n_accepted": n_acc, "out_tokens": out}
    aux_s = None
    if telemetry and not aux:
        raise ValueError("telemetry outputs come with aux=True")
    if aux:
        arrs = {
            "p_tok": np.empty((B, G), np.float64),
            "q_tok": np.empty((B, G), np.float64),
            "thr": np.empty((B, G), np.float64),
            "resid_mass": np.empty(B, np.float64),
            "row_max": np.empty((B, G1), np.float64),
            "row_sum": np.empty((B, G1), np.float64),
            "flag_pos": np.empty(B, np.int32),
            "n_decisions": np.empty(B, np.int32),
            "n_flags": np.empty(B, np.int32),
            "p_out": np.empty(B, np.float64),
        }
        if telemetry:
            arrs["beta"] = np.empty((B, G), np.float64)
            arrs["alpha"] = np.empty(G, np.float64)
        aux_s = _Aux(**{k: v.ctypes.data for k, v in arrs.items()})
        res.update(arrs)
    rc = lib.spec_verify_ref(
        B, G, V, _ptr(zl), _dtype_code(zl),
        _ptr(qp), _dtype_code(qp) if qp is not None else 0,
        _ptr(x), _ptr(u), float(temperature), float(lenience), int(mode),
        _ptr(n_acc), _ptr(out), ctypes.byref(aux_s) if aux_s is not None else None,
        int(n_threads))
    if rc != 0:
        raise ValueError(f"spec_verify_ref rejected its arguments (status {rc})")
    return res


def softmax_row(z: np.ndarray, temperature: float) -> np.ndarray:
    """The oracle's temperature softmax of one row (float32 or bf16 bits)."""
    lib = _load()
    z = np.ascontiguousarray(z)
    p = np.empty(z.shape[0], np.float64)
    rc = lib.ref_softmax_row(_ptr(z), _dtype_code(z), z.shape[0], float(temperature), _ptr(p))
    if rc != 0:
        raise ValueError("bad softmax arguments")
    return p


def icdf(w: np.ndarray, u: float) -> tuple[int, bool]:
    """The oracle's inverse-CDF draw from an unnormalised fp64 weight row."""
    lib = _load()
    w = np.ascontiguousarray(w, dtype=np.float64)
    fl = ctypes.c_int(0)
    k = lib.ref_icdf(_ptr(w), w.shape[0], float(u), ctypes.byref(fl))
    return k, bool(fl.value)


def argmax_row(z: np.ndarray) -> int:
    """The oracle's first-occurrence argmax of one raw row."""
    lib = _load()
    z = np.ascontiguousarray(z)
    return lib.ref_argmax_row(_ptr(z), _dtype_code(z), z.shape[0])


TOPK = 0
TOPP = 1


def standardize(z: np.ndarray, method: int, k: int = 0, top_p: float = 1.0, temperature: float = 1.0):
    """The oracle's top-k / nucleus standardisation of rows of logits
    ([R, V] float32 or bf16 bits): returns (logits with dropped entries set
    to -inf, kept count per row, near-boundary flag per row)."""
    lib = _load()
    if not hasattr(lib, "_std_ready"):
        lib.ref_standardize.restype = ctypes.c_int
        lib.ref_standardize.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]
        lib._std_ready = True
    z = np.ascontiguousarray(z)
    R, V = z.shape
    out = np.empty_like(z)
    kept = np.empty(R, np.int32)
    flag = np.empty(R, np.int32)
    rc = lib.ref_standardize(R, V, _ptr(z), _dtype_code(z), int(method), int(k), float(top_p),
                             float(temperature), _ptr(out), _ptr(kept), _ptr(flag))
    if rc != 0:
        raise ValueError(f"ref_standardize rejected its arguments (status {rc})")
    return out, kept, flag
