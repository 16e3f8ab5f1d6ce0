"""The C-ABI library loads and exports every symbol its header declares, and
its host-side argument checks return the documented status codes without
touching the GPU (no kernel is launched on any of these paths)."""
import ctypes
import os
import re

import pytest

import exact_rejection_sampling_temp_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


def _header_text():
    with open(HEADER) as f:
        return f.read()


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", _header_text(), flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


def _header_defines():
    return {m.group(1): int(m.group(2))
            for m in re.finditer(r"#define\s+(SV_\w+)\s+(-?\d+)", _header_text())}


def test_library_loads_and_exports_declared_symbols():
    lib = sv.load_library()
    declared = _declared_functions()
    assert set(declared) == set(sv.EXPORTED_SYMBOLS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_extras_mirror_matches_the_library():
    # the binding's ctypes copy of sv_extras_t must be exactly the struct the
    # library reads: a shorter mirror leaves the library reading host memory
    # past its end (uninitialised fields, device pointers among them)
    lib = sv.load_library()
    assert lib.sv_extras_bytes() == ctypes.sizeof(sv.Extras)
    fields = re.search(r"typedef struct \{(.*?)\} sv_extras_t;", _header_text(), flags=re.S).group(1)
    fields = re.sub(r"/\*.*?\*/", "", fields, flags=re.S)
    names = re.findall(r"([A-Za-z_]\w*)\s*;", fields)
    assert names == [f[0] for f in sv.Extras._fields_]


def test_binding_constants_match_header():
    d = _header_defines()
    for k in ("SV_FP32", "SV_BF16", "SV_SAMPLE", "SV_GREEDY", "SV_MAX_GAMMA", "SV_OK"):
        assert getattr(sv, k) == d[k], k


def test_status_strings():
    d = _header_defines()
    codes = [v for k, v in d.items() if k.startswith("SV_ERR_") or k == "SV_OK"]
    seen = set()
    for c in codes:
        s = sv.sv_status_string(c)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == len(codes)
    assert sv.sv_status_string(12345) == "unknown status"


def test_workspace_bytes():
    assert sv.sv_workspace_bytes(0, 4, 10) == 0
    assert sv.sv_workspace_bytes(1, 0, 10) == 0
    assert sv.sv_workspace_bytes(1, sv.SV_MAX_GAMMA + 1, 10) == 0
    a = sv.sv_workspace_bytes(256, 8, 152_064)
    assert a > 0 and a % 256 == 0
    assert sv.sv_workspace_bytes(512, 8, 152_064) > a
    assert sv.sv_workspace_bytes(256, 8, 300_000) > a


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _call(**kw):
    lib = sv.load_library()
    args = dict(batch=2, gamma=3, vocab=100, logits=FAKE, ldt=sv.SV_FP32, probs=FAKE, pdt=sv.SV_FP32,
                tokens=FAKE, uniforms=FAKE, T=1.0, mode=sv.SV_SAMPLE, n_acc=FAKE, out=FAKE,
                ws=FAKE * 16, ws_bytes=0)
    args.update(kw)
    return lib.spec_verify(args["batch"], args["gamma"], args["vocab"], args["logits"], args["ldt"],
                           args["probs"], args["pdt"], args["tokens"], args["uniforms"], args["T"],
                           args["mode"], args["n_acc"], args["out"], args["ws"], args["ws_bytes"],
                           None, None)


def test_argument_validation_codes():
    d = _header_defines()
    assert _call(mode=7) == d["SV_ERR_MODE"]
    assert _call(batch=0) == d["SV_ERR_BATCH"]
    assert _call(gamma=0) == d["SV_ERR_GAMMA"]
    assert _call(gamma=sv.SV_MAX_GAMMA + 1) == d["SV_ERR_GAMMA"]
    assert _call(vocab=0) == d["SV_ERR_VOCAB"]
    assert _call(ldt=5) == d["SV_ERR_DTYPE"]
    assert _call(pdt=5) == d["SV_ERR_DTYPE"]
    assert _call(logits=None) == d["SV_ERR_NULL_POINTER"]
    assert _call(tokens=None) == d["SV_ERR_NULL_POINTER"]
    assert _call(probs=None) == d["SV_ERR_NULL_POINTER"]
    assert _call(uniforms=None) == d["SV_ERR_NULL_POINTER"]
    assert _call(n_acc=None) == d["SV_ERR_NULL_POINTER"]
    assert _call(T=0.0) == d["SV_ERR_TEMPERATURE"]
    assert _call(T=-1.0) == d["SV_ERR_TEMPERATURE"]
    assert _call(T=float("inf")) == d["SV_ERR_TEMPERATURE"]
    assert _call(T=float("nan")) == d["SV_ERR_TEMPERATURE"]
    assert _call(logits=FAKE + 2) == d["SV_ERR_ALIGNMENT"]
    assert _call(logits=FAKE + 2, ldt=sv.SV_BF16) == d["SV_ERR_WORKSPACE"]  # 2-byte aligned is fine for bf16
    assert _call(ws_bytes=10) == d["SV_ERR_WORKSPACE"]
    assert _call(ws=None, ws_bytes=1 << 30) == d["SV_ERR_WORKSPACE"]
    assert _call(ws=FAKE + 8, ws_bytes=1 << 30) == d["SV_ERR_ALIGNMENT"]
    # greedy mode needs neither q nor u nor a valid temperature
    assert _call(mode=sv.SV_GREEDY, probs=None, uniforms=None, T=0.0) == d["SV_ERR_WORKSPACE"]


def test_lenient_entry_point_validation():
    d = _header_defines()
    lib = sv.load_library()

    def call(l, **kw):
        a = dict(mode=sv.SV_SAMPLE, T=1.0, ws_bytes=0)
        a.update(kw)
        return lib.spec_verify_lenient(2, 3, 100, FAKE, sv.SV_FP32, FAKE, sv.SV_FP32, FAKE, FAKE, a["T"], l,
                                       a["mode"], FAKE, FAKE, FAKE * 16, a["ws_bytes"], None, None)
    for bad in (-0.1, 1.01, float("nan"), float("inf")):
        assert call(bad) == d["SV_ERR_LENIENCE"]
    for ok in (0.0, 0.5, 1.0):
        assert call(ok) == d["SV_ERR_WORKSPACE"]  # passes the lenience check, stops at the workspace
    assert call(2.0, mode=sv.SV_GREEDY) == d["SV_ERR_WORKSPACE"]  # greedy mode ignores l
    assert call(0.5, T=0.0) == d["SV_ERR_TEMPERATURE"]


def test_noalloc_entry_point_validation():
    """The allocation-free entry point checks its arguments, then that the
    workspace fits its static scratch array, before any HIP call."""
    d = _header_defines()
    lib = sv.load_library()

    def call(B=2, gamma=3, V=100, mode=sv.SV_SAMPLE, T=1.0, l=1.0, logits=FAKE):
        return lib.spec_verify_noalloc(B, gamma, V, logits, sv.SV_BF16, FAKE, sv.SV_FP32, FAKE, FAKE, T, l, mode,
                                       FAKE, FAKE, None, None)
    assert call(mode=7) == d["SV_ERR_MODE"]
    assert call(B=0) == d["SV_ERR_BATCH"]
    assert call(gamma=sv.SV_MAX_GAMMA + 1) == d["SV_ERR_GAMMA"]
    assert call(T=0.0) == d["SV_ERR_TEMPERATURE"]
    assert call(l=1.5) == d["SV_ERR_LENIENCE"]
    assert call(logits=None) == d["SV_ERR_NULL_POINTER"]
    assert call(logits=FAKE + 1) == d["SV_ERR_ALIGNMENT"]
    # 4096 x 9 rows of 152064 need about 27 MiB of workspace: more than the 8 MiB array
    m = re.search(r"#define\s+SV_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", _header_text())
    limit = int(m.group(1)) << int(m.group(2))
    assert limit == 8 << 20
    assert sv.sv_workspace_bytes(4096, 8, 152_064) > limit
    assert call(B=4096, gamma=8, V=152_064) == d["SV_ERR_SCRATCH"]
    assert call(B=4096, gamma=8, V=152_064, mode=sv.SV_GREEDY) == d["SV_ERR_SCRATCH"]
    # every shape the benchmark and the tests use fits
    for B, g, V in ((1, 4, 8), (8, 4, 32_000), (64, 4, 128_256), (256, 8, 152_064), (32, 16, 256_000)):
        assert sv.sv_workspace_bytes(B, g, V) <= limit


def test_standardize_validation():
    d = _header_defines()
    lib = sv.load_library()

    def call(rows=2, V=100, z=FAKE, dt=sv.SV_FP32, m=sv.SV_TOPK, k=5, p=0.9, T=1.0, out=FAKE):
        return lib.sv_standardize(rows, V, z, dt, m, k, p, T, out, None)
    assert call(z=None) == d["SV_ERR_NULL_POINTER"]
    assert call(out=None) == d["SV_ERR_NULL_POINTER"]
    assert call(rows=0) == d["SV_ERR_BATCH"]
    assert call(V=0) == d["SV_ERR_VOCAB"]
    assert call(dt=7) == d["SV_ERR_DTYPE"]
    assert call(m=5) == d["SV_ERR_STANDARDIZE"]
    assert call(k=0) == d["SV_ERR_STANDARDIZE"]
    for bad in (0.0, -0.5, 1.5, float("nan")):
        assert call(m=sv.SV_TOPP, p=bad) == d["SV_ERR_STANDARDIZE"]
    assert call(m=sv.SV_TOPP, T=0.0) == d["SV_ERR_TEMPERATURE"]
    assert call(z=FAKE + 2) == d["SV_ERR_ALIGNMENT"]
    assert d["SV_TOPK"] == sv.SV_TOPK and d["SV_TOPP"] == sv.SV_TOPP


def test_workspace_init_validation():
    lib = sv.load_library()
    d = _header_defines()
    assert lib.sv_workspace_init(None, 16, None) == d["SV_ERR_NULL_POINTER"]
    assert lib.sv_workspace_init(ctypes.c_void_p(FAKE + 8), 16, None) == d["SV_ERR_ALIGNMENT"]
    assert lib.sv_workspace_init(ctypes.c_void_p(FAKE), 0, None) == d["SV_OK"]


def test_python_binding_refuses_cpu_tensors():
    import torch
    z = torch.zeros(1, 2, 4)
    with pytest.raises(ValueError):
        sv.spec_verify(z, torch.zeros(1, 1, 4), torch.zeros(1, 1, dtype=torch.int32),
                       torch.zeros(1, 2), 1.0)


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "exact_rejection_sampling_temp_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                with open(os.path.join(dirpath, fn)) as f:
                    text = f.read()
                assert "oracle" not in text.replace("Oracle", ""), fn
