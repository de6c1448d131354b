"""The Python binding checks every tensor's shape, dtype and device before it
calls into libfa: the C ABI receives bare pointers and sizes taken from q, so
a short k/v/out or a host tensor would otherwise become an out-of-bounds GPU
access. CPU only: every call below is refused before the library is used."""
import pytest
import torch

import io_aware_flashattention_amd as fa

bf = torch.bfloat16


def t(*shape, dtype=bf):
    return torch.zeros(*shape, dtype=dtype)


@pytest.mark.parametrize("kw,needle", [
    (dict(k=t(2, 2, 64, 128)), "k must have shape"),                 # batch mismatch
    (dict(k=t(1, 2, 64, 64)), "k must have shape"),                  # head_dim mismatch
    (dict(v=t(1, 2, 63, 128)), "v must have shape"),                 # v shorter than k
    (dict(out=t(1, 4, 32, 128)), "out must have shape"),             # short output
    (dict(out=t(1, 4, 64, 128, dtype=torch.float16)), "unsupported dtype"),
    (dict(q=t(4, 64, 128)), "q must have 4 dimensions"),
    (dict(v=t(1, 2, 64, 128, dtype=torch.float32)), "share a dtype"),
    (dict(), "must be on a GPU"),                                     # right shapes, host tensors
])
def test_fwd_refuses(kw, needle):
    a = dict(q=t(1, 4, 64, 128), k=t(1, 2, 64, 128), v=t(1, 2, 64, 128))
    a.update(kw)
    with pytest.raises(ValueError, match=needle):
        fa.fwd(a["q"], a["k"], a["v"], out=a.get("out"))


@pytest.mark.parametrize("kw,needle", [
    (dict(k=t(99, 2, 128)), "k must have shape"),
    (dict(v=t(100, 2, 64)), "v must have shape"),
    (dict(out=t(100, 4, 64)), "out must have shape"),
    (dict(cu=torch.zeros(1, dtype=torch.int32)), "cu_seqlens"),
    (dict(cu=torch.zeros(3, dtype=torch.int64)), "cu_seqlens"),
    (dict(), "must be on a GPU"),
])
def test_fwd_varlen_refuses(kw, needle):
    a = dict(q=t(100, 4, 128), k=t(100, 2, 128), v=t(100, 2, 128), cu=torch.tensor([0, 40, 100], dtype=torch.int32))
    a.update(kw)
    with pytest.raises(ValueError, match=needle):
        fa.fwd_varlen(a["q"], a["k"], a["v"], a["cu"], 60, causal=True, out=a.get("out"))


@pytest.mark.parametrize("kw,needle", [
    (dict(k=t(1, 2, 64, 64)), "k must have shape"),
    (dict(v=t(1, 2, 32, 128)), "v must share k's shape"),
    (dict(o=t(1, 4, 64, 128)[:, :, :32]), "o and dout must share"),
    (dict(lse=torch.zeros(1, 4, 63)), "lse must be"),
    (dict(dq=t(1, 4, 64, 64)), "dq must have shape"),
    (dict(dk=t(1, 2, 60, 128)), "dk must have shape"),
    (dict(), "must be on a GPU"),
])
def test_bwd_refuses(kw, needle):
    a = dict(q=t(1, 4, 64, 128), k=t(1, 2, 64, 128), v=t(1, 2, 64, 128), o=t(1, 4, 64, 128), g=t(1, 4, 64, 128),
             lse=torch.zeros(1, 4, 64))
    a.update(kw)
    with pytest.raises(ValueError, match=needle):
        fa.bwd(a["q"], a["k"], a["v"], a["o"], a["g"], a["lse"], dq=a.get("dq"), dk=a.get("dk"), dv=a.get("dv"))


@pytest.mark.parametrize("kw,needle", [
    (dict(k=t(3, 2, 100, 128)), "k_cache must have shape"),          # batch mismatch
    (dict(k=t(2, 2, 100, 64)), "k_cache must have shape"),           # head_dim mismatch
    (dict(v=t(2, 2, 90, 128)), "share shape"),
    (dict(out=t(2, 16, 64)), "out must have shape"),
    (dict(lens=torch.zeros(3, dtype=torch.int32)), "seqlens"),
    (dict(q=t(2, 16, 128, dtype=torch.float32)), "bfloat16"),
    (dict(), "must be on a GPU"),
])
def test_decode_refuses(kw, needle):
    a = dict(q=t(2, 16, 128), k=t(2, 2, 100, 128), v=t(2, 2, 100, 128), lens=torch.zeros(2, dtype=torch.int32))
    a.update(kw)
    with pytest.raises(ValueError, match=needle):
        fa.decode(a["q"], a["k"], a["v"], a["lens"], out=a.get("out"))
    if "out" not in kw:
        with pytest.raises(ValueError, match=needle):
            fa.decode_noalloc(a["q"], a["k"], a["v"], a["lens"], t(2, 16, 128))


@pytest.mark.parametrize("kw,needle", [
    (dict(kp=t(10, 2, 16, 64)), "k_pages must have shape"),
    (dict(table=torch.zeros(3, 7, dtype=torch.int32)), "block_table"),
    (dict(out=t(2, 16, 100)), "out must have shape"),
    (dict(), "must be on a GPU"),
])
def test_decode_paged_refuses(kw, needle):
    a = dict(q=t(2, 16, 128), kp=t(10, 2, 16, 128), vp=t(10, 2, 16, 128), table=torch.zeros(2, 7, dtype=torch.int32),
             lens=torch.zeros(2, dtype=torch.int32))
    a.update(kw)
    vp = a["kp"] if "kp" in kw else a["vp"]        # a bad k pool comes with a v pool of the same shape
    with pytest.raises(ValueError, match=needle):
        fa.decode_paged(a["q"], a["kp"], vp, a["table"], a["lens"], out=a.get("out"))


def test_fp8_refuses():
    q, k = t(1, 4, 64, 128), t(1, 2, 64, 128)
    with pytest.raises(ValueError, match="k must have shape"):
        fa.fp8_quantize(q, t(1, 2, 64, 64), t(1, 2, 64, 64))
    with pytest.raises(ValueError, match="must be on a GPU"):
        fa.fp8_quantize(q, k, k)
    f8 = torch.float8_e4m3fn
    quant = dict(q8=torch.zeros(1, 4, 64, 128, dtype=f8), k8=torch.zeros(1, 2, 64, 128, dtype=f8),
                 v8t=torch.zeros(1, 2, 128, 64, dtype=f8), q_scale=torch.zeros(1, 4, 1), k_scale=torch.zeros(1, 2, 1),
                 v_scale=torch.zeros(1, 2))
    with pytest.raises(ValueError, match="must be on a GPU"):
        fa.fwd_fp8(quant)
    bad = dict(quant, v8t=torch.zeros(1, 2, 128, 32, dtype=f8))
    with pytest.raises(ValueError, match="v8t must have shape"):
        fa.fwd_fp8(bad)
    bad = dict(quant, k8=torch.zeros(1, 2, 64, 128))
    with pytest.raises(ValueError, match="float8_e4m3fn"):
        fa.fwd_fp8(bad)
