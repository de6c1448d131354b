"""The C-ABI library: loads, exports exactly what include/fa.h declares, and
rejects bad arguments before touching the GPU. CPU only: every call below
fails validation, which runs before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

from io_aware_flashattention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libfa.so not built")


def declared_functions():
    text = open(HEADER).read()
    return set(re.findall(r"FA_API\s+[\w\s\*]+?\b(fa_\w+)\s*\(", text))


def test_exports_match_header():
    decl = declared_functions()
    assert decl == set(_lib.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True, check=True).stdout
    funcs = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert funcs == decl
    lib = _lib.load()
    for name in decl:
        assert hasattr(lib, name)


def test_status_strings():
    lib = _lib.load()
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.fa_status_string(code).decode() == name
    assert lib.fa_status_string(99).decode() == "FA_ERR_UNKNOWN"


FAKE = 0x10000   # 16-byte aligned, never dereferenced: every call below fails validation first


def _fwd(**kw):
    lib = _lib.load()
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000, lse=None, B=1, Hq=2, Hkv=1,
             Nq=64, Nk=64, d=128, qs=(16384, 8192, 128), ks=(8192, 8192, 128), vs=(8192, 8192, 128),
             os_=(16384, 8192, 128), ind=0, outd=0, mask=0, scale=0.125)
    a.update(kw)
    arr = lambda t: (ctypes.c_int64 * 3)(*t) if t is not None else None
    st = lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                    arr(a["qs"]), arr(a["ks"]), arr(a["vs"]), arr(a["os_"]), a["ind"], a["outd"], a["mask"],
                    a["scale"], None)
    return st, lib.fa_last_error_message().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), 1, "non-null"),
    (dict(qs=None), 1, "stride"),
    (dict(B=0), 1, "positive"),
    (dict(Nk=-3), 1, "positive"),
    (dict(scale=float("nan")), 1, "softmax_scale"),
    (dict(scale=0.0), 1, "softmax_scale"),
    (dict(ind=7), 1, "in_dtype"),
    (dict(mask=5), 1, "mask"),
    (dict(d=96), 2, "head_dim"),
    (dict(Hq=3, Hkv=2), 2, "multiple"),
    (dict(mask=1, Nq=64, Nk=80), 2, "causal"),
    (dict(q=FAKE + 8), 2, "aligned"),
    (dict(qs=(16384, 8192, 132)), 2, "multiples"),
    (dict(ind=1, qs=(16384, 8192, 130)), 2, "multiples"),
    (dict(o=FAKE + 0x100), 1, "overlaps"),
    (dict(ks=(8192, 8192, (1 << 24) + 8)), 2, "row strides"),
])
def test_fwd_rejects_before_launch(kw, status, needle):
    st, msg = _fwd(**kw)
    assert st == status, msg
    assert needle in msg


def _varlen(**kw):
    lib = _lib.load()
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000, lse=None, cu=FAKE + 0x400000,
             B=2, Hq=4, Hkv=2, T=100, maxl=64, d=128, qs=(512, 128), ks=(256, 128), vs=(256, 128), os_=(512, 128),
             outd=0, mask=1, win=-1, scale=0.125)
    a.update(kw)
    arr = lambda t: (ctypes.c_int64 * 2)(*t) if t is not None else None
    st = lib.fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["B"], a["Hq"], a["Hkv"], a["T"],
                           a["maxl"], a["d"], arr(a["qs"]), arr(a["ks"]), arr(a["vs"]), arr(a["os_"]), a["outd"],
                           a["mask"], a["win"], a["scale"], None)
    return st, lib.fa_last_error_message().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(cu=None), 1, "non-null"),
    (dict(os_=None), 1, "stride"),
    (dict(T=0), 1, "positive"),
    (dict(maxl=0), 1, "positive"),
    (dict(win=-2), 1, "window"),
    (dict(mask=3), 1, "mask"),
    (dict(scale=-1.0), 1, "softmax_scale"),
    (dict(d=96), 2, "head_dim"),
    (dict(Hq=6, Hkv=4), 2, "multiple"),
    (dict(mask=0, win=16), 2, "causal"),
    (dict(o=FAKE + 0x300008), 2, "aligned"),
    (dict(qs=(516, 128)), 2, "16 bytes"),
    (dict(ks=((1 << 24) + 8, 128)), 2, "token strides"),
    (dict(o=FAKE + 0x10), 1, "overlaps"),
])
def test_fwd_varlen_rejects_before_launch(kw, status, needle):
    st, msg = _varlen(**kw)
    assert st == status, msg
    assert needle in msg


def _bwd(**kw):
    lib = _lib.load()
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000, do=FAKE + 0x400000,
             lse=FAKE + 0x500000, dq=FAKE + 0x600000, dk=FAKE + 0x700000, dv=FAKE + 0x800000, B=1, Hq=4, Hkv=2,
             Nq=64, Nk=64, d=128, qs=(4 * 64 * 128, 64 * 128, 128), ks=(2 * 64 * 128, 64 * 128, 128),
             dqs=(4 * 64 * 128, 64 * 128, 128), dks=(2 * 64 * 128, 64 * 128, 128), od=0, gd=1, mask=1, scale=0.125,
             ws=FAKE + 0x900000, wsb=1 << 20)
    a.update(kw)
    arr = lambda t: (ctypes.c_int64 * 3)(*t) if t is not None else None
    st = lib.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["B"], a["Hq"],
                    a["Hkv"], a["Nq"], a["Nk"], a["d"], arr(a["qs"]), arr(a["ks"]), arr(a["dqs"]), arr(a["dks"]),
                    a["od"], a["gd"], a["mask"], a["scale"], a["ws"], a["wsb"], None)
    return st, lib.fa_last_error_message().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(do=None), 1, "non-null"),
    (dict(dks=None), 1, "stride"),
    (dict(Nk=0), 1, "positive"),
    (dict(gd=5), 1, "grad_dtype"),
    (dict(od=9), 1, "o_dtype"),
    (dict(mask=2), 1, "mask"),
    (dict(scale=float("nan")), 1, "softmax_scale"),
    (dict(d=32), 2, "head_dim"),
    (dict(Hq=6, Hkv=4), 2, "multiple"),
    (dict(Nq=64, Nk=96), 2, "causal"),
    (dict(lse=FAKE + 0x500004), 2, "aligned"),
    (dict(qs=(4 * 64 * 128, 64 * 128, 132)), 2, "input strides"),
    (dict(dqs=(4 * 64 * 128, 64 * 128, 130)), 2, "gradient strides"),
    (dict(wsb=100), 3, "workspace"),
    (dict(dk=FAKE + 0x100000), 1, "overlap"),
    (dict(dv=FAKE + 0x700100), 1, "overlap"),
])
def test_bwd_rejects_before_launch(kw, status, needle):
    st, msg = _bwd(**kw)
    assert st == status, msg
    assert needle in msg


def test_bwd_workspace_size():
    lib = _lib.load()
    assert lib.fa_bwd_workspace_bytes(2, 8, 100) == 2 * 8 * 100 * 4
    assert lib.fa_bwd_workspace_bytes(0, 8, 100) == 0


def _fp8q(**kw):
    lib = _lib.load()
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, s=None, B=1, Hq=4, Hkv=2, N=64, d=128,
             qs=(4 * 64 * 128, 64 * 128, 128), ks=(2 * 64 * 128, 64 * 128, 128), q8=FAKE + 0x300000,
             k8=FAKE + 0x400000, v8=FAKE + 0x500000, sq=FAKE + 0x600000, sk=FAKE + 0x700000, sv=FAKE + 0x800000)
    a.update(kw)
    arr = lambda t: (ctypes.c_int64 * 3)(*t) if t is not None else None
    st = lib.fa_fp8_quantize(a["q"], a["k"], a["v"], a["s"], a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], arr(a["qs"]),
                             arr(a["ks"]), a["q8"], a["k8"], a["v8"], a["sq"], a["sk"], a["sv"], None)
    return st, lib.fa_last_error_message().decode()


def _fp8f(**kw):
    lib = _lib.load()
    a = dict(q8=FAKE, k8=FAKE + 0x100000, v8=FAKE + 0x200000, sq=FAKE + 0x300000, sk=FAKE + 0x400000,
             sv=FAKE + 0x500000, o=FAKE + 0x600000, lse=None, B=1, Hq=4, Hkv=2, N=64, d=128, outd=0, mask=1,
             scale=0.088)
    a.update(kw)
    st = lib.fa_fwd_fp8(a["q8"], a["k8"], a["v8"], a["sq"], a["sk"], a["sv"], a["o"], a["lse"], a["B"], a["Hq"],
                        a["Hkv"], a["N"], a["d"], a["outd"], a["mask"], a["scale"], None)
    return st, lib.fa_last_error_message().decode()


@pytest.mark.parametrize("fn,kw,status,needle", [
    (_fp8q, dict(v8=None), 1, "non-null"),
    (_fp8q, dict(qs=None), 1, "stride"),
    (_fp8q, dict(N=0), 1, "positive"),
    (_fp8q, dict(d=64), 2, "head_dim"),
    (_fp8q, dict(Hq=3, Hkv=2), 2, "multiple"),
    (_fp8q, dict(k8=FAKE + 0x400008), 2, "aligned"),
    (_fp8q, dict(ks=(2 * 64 * 128, 64 * 128, 132)), 2, "multiples"),
    (_fp8f, dict(sv=None), 1, "non-null"),
    (_fp8f, dict(Hkv=0), 1, "positive"),
    (_fp8f, dict(scale=0.0), 1, "softmax_scale"),
    (_fp8f, dict(outd=4), 1, "out_dtype"),
    (_fp8f, dict(mask=9), 1, "mask"),
    (_fp8f, dict(d=256), 2, "head_dim"),
    (_fp8f, dict(o=FAKE + 0x600004), 2, "aligned"),
])
def test_fp8_rejects_before_launch(fn, kw, status, needle):
    st, msg = fn(**kw)
    assert st == status, msg
    assert needle in msg


def _dec(**kw):
    lib = _lib.load()
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, lens=FAKE + 0x300000, o=FAKE + 0x400000, lse=None,
             B=2, Hq=16, Hkv=2, L=4096, d=128, kvs=(2 * 4096 * 128, 4096 * 128, 128), outd=0, scale=0.0884,
             split=0, ws=FAKE + 0x800000, wsb=1 << 30)
    a.update(kw)
    kvs = (ctypes.c_int64 * 3)(*a["kvs"]) if a["kvs"] is not None else None
    st = lib.fa_decode(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["L"],
                       a["d"], kvs, a["outd"], a["scale"], a["split"], a["ws"], a["wsb"], None)
    return st, lib.fa_last_error_message().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(lens=None), 1, "non-null"),
    (dict(kvs=None), 1, "non-null"),
    (dict(L=0), 1, "positive"),
    (dict(scale=float("inf")), 1, "softmax_scale"),
    (dict(d=96), 2, "head_dim"),
    (dict(d=256), 2, "head_dim"),
    (dict(Hq=16, Hkv=3), 2, "multiple"),
    (dict(Hq=66, Hkv=1), 2, "at most 32"),
    (dict(k=FAKE + 4), 2, "aligned"),
    (dict(kvs=(2 * 4096 * 128, 4096 * 128, 132)), 2, "multiples"),
    (dict(wsb=1000), 3, "workspace"),
    (dict(ws=None), 3, "workspace"),
])
def test_decode_rejects_before_launch(kw, status, needle):
    st, msg = _dec(**kw)
    assert st == status, msg
    assert needle in msg


def _paged(**kw):
    lib = _lib.load()
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, bt=FAKE + 0x300000, lens=FAKE + 0x380000,
             o=FAKE + 0x400000, lse=None, B=2, Hq=16, Hkv=2, d=128, P=64, ps=16, mb=32,
             pst=(2 * 16 * 128, 16 * 128, 128), outd=0, scale=0.0884, split=0, ws=FAKE + 0x800000, wsb=1 << 30)
    a.update(kw)
    pst = (ctypes.c_int64 * 3)(*a["pst"]) if a["pst"] is not None else None
    st = lib.fa_decode_paged(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["o"], a["lse"], a["B"], a["Hq"],
                             a["Hkv"], a["d"], a["P"], a["ps"], a["mb"], pst, a["outd"], a["scale"], a["split"],
                             a["ws"], a["wsb"], None)
    return st, lib.fa_last_error_message().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(bt=None), 1, "non-null"),
    (dict(pst=None), 1, "non-null"),
    (dict(P=0), 1, "positive"),
    (dict(mb=0), 1, "positive"),
    (dict(ps=-16), 1, "positive"),
    (dict(pst=(-4096, 2048, 128)), 1, "non-negative"),
    (dict(mb=1 << 27, ps=32), 1, "overflows"),
    (dict(outd=3), 1, "out_dtype"),
    (dict(d=96), 2, "head_dim"),
    (dict(Hq=16, Hkv=3), 2, "multiple"),
    (dict(ps=8), 2, "page_size"),
    (dict(v=FAKE + 0x200004), 2, "aligned"),
    (dict(pst=(4096, 2048, 132)), 2, "multiples"),
    (dict(ps=1024, pst=(1 << 32, 1 << 22, 1 << 21)), 2, "2^31"),
    (dict(wsb=100), 3, "workspace"),
])
def test_decode_paged_rejects_before_launch(kw, status, needle):
    st, msg = _paged(**kw)
    assert st == status, msg
    assert needle in msg


def test_decode_workspace_size():
    lib = _lib.load()
    waves = lib.fa_decode_workspace_bytes(1, 1, 1, 100, 128, 0) // (129 * 4) - 1   # decode grid size
    assert waves > 0
    # (batch * heads_kv + waves) pieces, each heads_q / heads_kv heads of (d + 1) floats,
    # whatever split_tokens is (a larger split leaves waves without a range)
    for split in (0, 1, 256, 4096, 1 << 20):
        assert lib.fa_decode_workspace_bytes(64, 64, 8, 32768, 128, split) == (64 * 8 + waves) * 8 * 129 * 4
        assert lib.fa_decode_workspace_bytes(8, 12, 12, 1024, 64, split) == (8 * 12 + waves) * 65 * 4
    assert lib.fa_decode_workspace_bytes(2, 8, 8, 1000, 128, 0) == (16 + waves) * 129 * 4
    assert lib.fa_decode_workspace_bytes(0, 1, 1, 100, 128, 0) == 0
    assert lib.fa_decode_workspace_bytes(1, 6, 4, 100, 128, 0) == 0


def test_decode_accepts_head_dim_64_up_to_the_workspace_check():
    """d = 64 passes every argument check; with a too-small workspace the call
    then stops at that check, still before any launch."""
    st, msg = _dec(d=64, kvs=(2 * 4096 * 64, 4096 * 64, 64), wsb=16)
    assert st == 3 and "workspace" in msg, msg
    st, msg = _paged(d=64, pst=(2 * 16 * 64, 16 * 64, 64), wsb=16)
    assert st == 3 and "workspace" in msg, msg


def test_binding_refuses_missing_library(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(FileNotFoundError):
        _lib.load()


def _dec_noalloc(**kw):
    lib = _lib.load()
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, lens=FAKE + 0x300000, o=FAKE + 0x400000, lse=None,
             B=2, Hq=16, Hkv=2, L=4096, d=128, kvs=(2 * 4096 * 128, 4096 * 128, 128), outd=0, scale=0.0884,
             split=0)
    a.update(kw)
    kvs = (ctypes.c_int64 * 3)(*a["kvs"]) if a["kvs"] is not None else None
    st = lib.fa_decode_noalloc(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                               a["L"], a["d"], kvs, a["outd"], a["scale"], a["split"], None)
    return st, lib.fa_last_error_message().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(lens=None), 1, "non-null"),
    (dict(B=0), 1, "positive"),
    (dict(d=96), 2, "head_dim"),
    (dict(Hq=66, Hkv=1), 2, "at most 32"),
    (dict(k=FAKE + 4), 2, "aligned"),
    (dict(B=4096, Hq=64, Hkv=8), 2, "static scratch"),      # partials past the 16 MiB scratch
])
def test_decode_noalloc_rejects_before_launch(kw, status, needle):
    st, msg = _dec_noalloc(**kw)
    assert st == status, msg
    assert needle in msg
    assert "fa_decode_noalloc" in msg


def test_decode_noalloc_limit_is_the_scratch_size():
    lib = _lib.load()
    assert lib.fa_decode_workspace_bytes(64, 64, 8, 32768, 128, 0) <= _lib.DECODE_SCRATCH_BYTES
    assert lib.fa_decode_workspace_bytes(4096, 64, 8, 1024, 128, 0) > _lib.DECODE_SCRATCH_BYTES
