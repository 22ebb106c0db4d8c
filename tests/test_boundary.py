"""The C ABI boundary on the CPU: libfa.so loads, exports what include/fa.h declares, and
rejects bad arguments with the documented status codes before any HIP call."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import exact_io_aware_70_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fa.library_path()),
                                reason="libfa.so not built (python -m exact_io_aware_70_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_is_plain_c():
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    res = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"fa_fwd", "fa_fwd_fp8", "fa_fwd_dropout", "fa_bwd_dropout", "fa_bwd", "fa_bwd_timed", "fa_bwd_noalloc",
            "fa_std_fwd", "fa_std_bwd", "fa_std_ld", "fa_std_matrix_bytes", "fa_bwd_workspace_size", "fa_softmax_rows", "fa_status_string", "fa_version"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    lib = fa.load_library()
    for n in names:
        assert hasattr(lib, n)


def test_version_and_status_strings():
    assert fa.fa_version() == 100
    seen = set()
    for code in [0, -1, -2, -3, -4, -5, -6, -7]:
        s = fa.fa_status_string(code)
        assert s and s not in seen
        seen.add(s)
    assert fa.fa_status_string(12345) == "unknown fa_status code"


GOOD = dict(B=2, H=3, N=100, d=64, scale=0.125, causal=0, dtype=1)
P = 4096  # a fake, 16-byte aligned, never dereferenced address


def call_fwd(q=P, k=P, v=P, o=P, lse=P, **kw):
    a = dict(GOOD, **kw)
    return fa.load_library().fa_fwd(q, k, v, o, lse, a["B"], a["H"], a["N"], a["d"], a["scale"],
                                    a["causal"], a["dtype"], None)


def call_bwd(ptrs=None, ws=P, ws_bytes=1 << 30, **kw):
    a = dict(GOOD, **kw)
    p = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P)
    p.update(ptrs or {})
    return fa.load_library().fa_bwd(p["q"], p["k"], p["v"], p["o"], p["do"], p["lse"], p["dq"], p["dk"], p["dv"],
                                    a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"],
                                    ws, ws_bytes, None)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_fwd_null(which):
    assert call_fwd(**{which: None}) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -2), (dict(H=0), -2), (dict(N=0), -2), (dict(N=-5), -2),
    (dict(d=32), -3), (dict(d=96), -3), (dict(d=256), -3), (dict(dtype=2), -3), (dict(dtype=-1), -3),
    (dict(scale=0.0), -3), (dict(scale=-0.1), -3), (dict(scale=float("inf")), -3), (dict(scale=float("nan")), -3),
    (dict(B=1 << 20, H=1 << 12, N=1 << 12), -2),
])
def test_fwd_bad_sizes(kw, code):
    assert call_fwd(**kw) == code


@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
def test_fwd_misaligned(which):
    assert call_fwd(**{which: P + 8}) == -4
    assert call_fwd(lse=P + 2) == -4


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"])
def test_bwd_null(which):
    assert call_bwd(ptrs={which: None}) == -1


def test_bwd_workspace():
    need = fa.fa_bwd_workspace_size(2, 3, 100, 64, 1)
    assert need >= 2 * 3 * 100 * 4 and need % 256 == 0
    assert call_bwd(ws=None) == -5
    assert call_bwd(ws_bytes=need - 1) == -5
    assert call_bwd(ws=P + 16) == -5  # not 256-byte aligned
    assert fa.fa_bwd_workspace_size(0, 3, 100, 64, 1) == 0
    assert fa.fa_bwd_workspace_size(2, 3, 100, 48, 1) == 0


@pytest.mark.parametrize("kw,code", [(dict(N=0), -2), (dict(d=80), -3), (dict(dtype=5), -3), (dict(scale=0.0), -3)])
def test_bwd_bad_sizes(kw, code):
    assert call_bwd(**kw) == code


def call_bwd_timed(events, **kw):
    a = dict(GOOD, **kw)
    return fa.load_library().fa_bwd_timed(P, P, P, P, P, P, P, P, P, a["B"], a["H"], a["N"], a["d"], a["scale"],
                                          a["causal"], a["dtype"], P, 1 << 30, None, events)


def test_bwd_timed_rejects_missing_events():
    """fa_bwd_timed needs FA_BWD_LAUNCHES + 1 event handles; NULL array or handle -> FA_ERR_NULL."""
    assert fa.FA_BWD_LAUNCHES == 2  # dQ (with D), then dK/dV
    header = open(os.path.join(os.path.dirname(__file__), "..", "include", "fa.h")).read()
    assert f"#define FA_BWD_LAUNCHES {fa.FA_BWD_LAUNCHES}\n" in header
    assert call_bwd_timed(None) == -1
    handles = (ctypes.c_void_p * (fa.FA_BWD_LAUNCHES + 1))(*([P] * fa.FA_BWD_LAUNCHES + [None]))
    assert call_bwd_timed(handles) == -1
    # With all handles present the ordinary checks still run first (nothing is launched).
    handles = (ctypes.c_void_p * (fa.FA_BWD_LAUNCHES + 1))(*([P] * (fa.FA_BWD_LAUNCHES + 1)))
    assert call_bwd_timed(handles, d=80) == -3
    assert call_bwd_timed(handles, N=0) == -2


def test_bwd_misaligned():
    for which in ["q", "k", "v", "o", "do", "dq", "dk", "dv"]:
        assert call_bwd(ptrs={which: P + 4}) == -4


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    """No CPU fallback: a missing library is an error, not a silent alternative path."""
    monkeypatch.setenv("FA_LIBRARY", str(tmp_path / "missing.so"))
    monkeypatch.setattr(fa, "_LIB", None)
    with pytest.raises(RuntimeError, match="not found"):
        fa.load_library()


def test_product_does_not_import_oracle():
    """The package and its sources never reference the oracle."""
    pkg = os.path.join(ROOT, "exact_io_aware_70_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "oracle/" not in text, f


def call_softmax(x=P, y=P, lse=P, rows=4, cols=100, dtype=1):
    return fa.load_library().fa_softmax_rows(x, y, lse, rows, cols, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), -1), (dict(y=None), -1),
    (dict(rows=0), -2), (dict(cols=0), -2), (dict(rows=-3), -2), (dict(rows=1 << 31), -2),
    (dict(dtype=2), -3), (dict(dtype=-1), -3),
    (dict(x=P + 8), -4), (dict(y=P + 4), -4), (dict(lse=P + 2), -4),
])
def test_softmax_rejects_bad_arguments(kw, code):
    """fa_softmax_rows validates before any HIP call (lse may be NULL; rows < 2^31)."""
    assert call_softmax(**kw) == code


def call_fp8(ptrs=None, **kw):
    a = dict(GOOD, **kw)
    p = dict(q=P, k=P, v=P, qd=P, kd=P, vd=P, o=P, lse=P)
    p.update(ptrs or {})
    return fa.load_library().fa_fwd_fp8(p["q"], p["k"], p["v"], p["qd"], p["kd"], p["vd"], p["o"], p["lse"],
                                        a["B"], a["H"], a["N"], 128 if "d" not in kw else a["d"], a["scale"],
                                        a["causal"], None)


@pytest.mark.parametrize("which", ["q", "k", "v", "qd", "kd", "vd", "o", "lse"])
def test_fp8_null(which):
    assert call_fp8(ptrs={which: None}) == -1


@pytest.mark.parametrize("kw,code", [(dict(N=0), -2), (dict(B=0), -2), (dict(d=64), -3), (dict(d=96), -3),
                                     (dict(scale=0.0), -3)])
def test_fp8_bad_sizes(kw, code):
    assert call_fp8(**kw) == code


@pytest.mark.parametrize("which,off", [("q", 8), ("o", 4), ("lse", 2), ("qd", 2)])
def test_fp8_misaligned(which, off):
    assert call_fp8(ptrs={which: P + off}) == -4


def test_dropout_rejects_bad_arguments():
    lib = fa.load_library()
    a = GOOD
    def fwd(p=0.1, dtype=1, q=P):
        return lib.fa_fwd_dropout(q, P, P, P, P, a["B"], a["H"], a["N"], a["d"], a["scale"], 0, dtype, p, 1, 0, None)
    def bwd(p=0.1, dtype=1, ws=P, events=None):
        return lib.fa_bwd_dropout(P, P, P, P, P, P, P, P, P, a["B"], a["H"], a["N"], a["d"], a["scale"], 0, dtype, p,
                                  1, 0, ws, 1 << 30, None, events)
    assert fwd(q=None) == -1
    assert fwd(p=1.0) == -3 and fwd(p=-0.1) == -3 and fwd(p=float("nan")) == -3 and fwd(dtype=0) == -3
    assert bwd(p=1.5) == -3 and bwd(dtype=0) == -3 and bwd(ws=None) == -5
    events = (ctypes.c_void_p * (fa.FA_BWD_LAUNCHES + 1))(P, None, P)
    assert bwd(events=events) == -1


@pytest.mark.parametrize("kw", [dict(B=1, H=1, N=(1 << 30) + 1), dict(B=1, H=1, N=(1 << 31) - 1),
                                dict(B=1, H=1, N=1 << 30), dict(B=1, H=1 << 24, N=64),
                                dict(B=1 << 12, H=1 << 12, N=1), dict(B=2, H=1 << 10, N=1 << 19)])
def test_sizes_past_the_supported_domain(kw):
    """N <= FA_MAX_N = 2^30 and B*H*ceil(N/64) <= FA_MAX_TILES = 2^24 - 1 (a dispatch holds
    fewer than 2^32 work-items); every entry point returns FA_ERR_SHAPE outside, before any
    launch, and fa_bwd_workspace_size returns 0."""
    assert call_fwd(**kw) == -2
    assert call_bwd(**kw) == -2
    assert call_fp8(**kw) == -2
    a = dict(GOOD, **kw)
    assert fa.fa_bwd_workspace_size(a["B"], a["H"], a["N"], 64, 1) == 0


@pytest.mark.parametrize("B,H,N", [(1, (1 << 24) - 1, 64), (1, 1, (1 << 30) - 64 * 1024), (1, 1023, 1 << 20),
                                   (3, 5, 1 << 20)])
def test_sizes_at_the_edge_of_the_domain(B, H, N):
    """Just inside both limits the sizes are accepted (the workspace size is their check):
    tiles = B*H*ceil(N/64) <= 2^24 - 1 and N <= 2^30."""
    assert B * H * -(-N // 64) <= (1 << 24) - 1
    assert fa.fa_bwd_workspace_size(B, H, N, 128, 1) == 2 * (-(-B * H * N * 4 // 256) * 256)


def test_binding_checks_gradients_and_workspace():
    """The bindings check every caller-supplied tensor before any library call: gradients of
    the wrong shape, dtype or layout, and a workspace that is too small, strided or on
    another device, raise instead of handing the library a bad pointer."""
    import torch
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 8)
    need = fa.fa_bwd_workspace_size(1, 2, 8, 64, fa.FA_BF16)
    for bwd in (lambda **kw: fa.fa_bwd(q, q, q, q, lse, q, **kw),
                lambda **kw: fa.fa_bwd_dropout(q, q, q, q, lse, q, 0.1, 1, **kw)):
        with pytest.raises(ValueError, match="dq"):
            bwd(dq=torch.zeros(1, 2, 8, 32, dtype=torch.bfloat16))
        with pytest.raises(TypeError, match="dk"):
            bwd(dk=torch.zeros(1, 2, 8, 64, dtype=torch.float32))
        with pytest.raises(ValueError, match="dv"):
            bwd(dv=torch.zeros(1, 2, 64, 8, dtype=torch.bfloat16).transpose(2, 3))
        with pytest.raises(ValueError, match="workspace"):
            bwd(workspace=torch.zeros(need - 1, dtype=torch.uint8))
        with pytest.raises(ValueError, match="workspace"):
            bwd(workspace=torch.zeros(2 * need, dtype=torch.uint8)[::2])
        with pytest.raises(ValueError, match="workspace"):
            bwd(workspace=torch.zeros(need, dtype=torch.uint8, device="meta"))


def call_bwd_noalloc(ptrs=None, **kw):
    a = dict(GOOD, **kw)
    p = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P)
    p.update(ptrs or {})
    return fa.load_library().fa_bwd_noalloc(p["q"], p["k"], p["v"], p["o"], p["do"], p["lse"], p["dq"], p["dk"],
                                            p["dv"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"],
                                            a["dtype"], None)


def test_bwd_noalloc_rejects_before_any_hip_call():
    """fa_bwd_noalloc runs fa_bwd's checks, then refuses sizes whose workspace exceeds the
    static scratch (FA_ERR_SCRATCH), all before touching HIP."""
    assert fa.FA_NOALLOC_SCRATCH_BYTES == 16 << 20
    for which in ["q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"]:
        assert call_bwd_noalloc(ptrs={which: None}) == -1
    assert call_bwd_noalloc(N=0) == -2 and call_bwd_noalloc(d=80) == -3
    assert call_bwd_noalloc(ptrs={"dq": P + 4}) == -4
    # 2 * round_up(rows * 4, 256) bytes: 2^21 rows fit 16 MiB exactly, one more row does not.
    assert fa.fa_bwd_workspace_size(1, 512, 4096, 128, 1) == 16 << 20
    assert fa.fa_bwd_workspace_size(1, 512, 4097, 128, 1) > 16 << 20
    assert call_bwd_noalloc(B=1, H=512, N=4097, d=128) == -7
    assert call_bwd_noalloc(B=4, H=32, N=16400, d=128) == -7
    assert "scratch" in fa.fa_status_string(-7)


def test_std_sizes_and_rejections():
    """The standard path's matrix layout ([B, H, N, ld], ld = N rounded up to 128) and its
    argument checks (bf16 only, N <= FA_STD_MAX_N = 65536), before any HIP call."""
    lib = fa.load_library()
    assert [fa.fa_std_ld(n) for n in (1, 127, 128, 129, 4096, 65536)] == [128, 128, 128, 256, 4096, 65536]
    assert fa.fa_std_ld(0) == 0 and fa.fa_std_ld(65537) == 0
    assert lib.fa_std_matrix_bytes(2, 3, 100) == 2 * 3 * 100 * 128 * 2
    assert lib.fa_std_matrix_bytes(1, 1, 65537) == 0
    a = GOOD

    def fwd(dtype=1, N=a["N"], d=a["d"], q=P, p=P):
        return lib.fa_std_fwd(q, P, P, P, P, p, a["B"], a["H"], N, d, a["scale"], 0, dtype, None)

    def bwd(dtype=1, N=a["N"], d=a["d"], dp=P):
        return lib.fa_std_bwd(P, P, P, P, P, P, P, P, dp, a["B"], a["H"], N, d, a["scale"], 1, dtype, None)
    assert fwd(q=None) == -1 and fwd(p=None) == -1 and bwd(dp=None) == -1
    assert fwd(dtype=0) == -3 and bwd(dtype=0) == -3 and fwd(d=96) == -3
    assert fwd(N=65537) == -2 and bwd(N=65537) == -2 and fwd(N=0) == -2
    assert fwd(p=P + 8) == -4 and bwd(dp=P + 2) == -4
