"""ctypes binding of libfa (include/fa.h) over torch tensors.

Argument marshalling only: every step of attention runs in the HIP kernels of
libfa.so. torch supplies device memory and the current stream. If the library
is missing or a call is unsupported, these functions raise; there is no other
code path.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_OK = 0
FA_DTYPE_BF16, FA_DTYPE_FP32 = 0, 1
FA_MASK_NONE, FA_MASK_CAUSAL = 0, 1
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_INVALID_ARGUMENT", 2: "FA_ERR_UNSUPPORTED",
                3: "FA_ERR_WORKSPACE_TOO_SMALL", 4: "FA_ERR_HIP"}
EXPORTED = ("fa_fwd", "fa_fwd_varlen", "fa_bwd_workspace_bytes", "fa_bwd", "fa_fp8_quantize", "fa_fwd_fp8",
            "fa_decode_workspace_bytes", "fa_decode", "fa_decode_noalloc", "fa_decode_paged", "fa_status_string",
            "fa_last_error_message")
DECODE_SCRATCH_BYTES = 16 << 20      # the static workspace behind fa_decode_noalloc

_i32, _i64p, _vp = ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p
_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load():
    """Load libfa.so (built by ``python -m io_aware_flashattention_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(f"{LIB_PATH} is not built; run python -m io_aware_flashattention_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                           _i64p, _i64p, _i64p, _i64p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                           ctypes.c_float, _vp]
    lib.fa_fwd_varlen.restype = ctypes.c_int
    lib.fa_fwd_varlen.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp,             # q, k, v, o, lse, cu_seqlens
                                  _i32, _i32, _i32, _i32, _i32, _i32,       # batch, Hq, Hkv, total, max_seqlen, d
                                  _i64p, _i64p, _i64p, _i64p, ctypes.c_int, ctypes.c_int, _i32,
                                  ctypes.c_float, _vp]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_workspace_bytes.argtypes = [_i32, _i32, _i32]                 # batch, heads_q, seqlen_q
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,     # q k v o dout lse dq dk dv
                           _i32, _i32, _i32, _i32, _i32, _i32,              # batch Hq Hkv Nq Nk d
                           _i64p, _i64p, _i64p, _i64p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                           ctypes.c_float, _vp, ctypes.c_size_t, _vp]
    lib.fa_fp8_quantize.restype = ctypes.c_int
    lib.fa_fp8_quantize.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64p, _i64p,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.fa_fwd_fp8.restype = ctypes.c_int
    lib.fa_fwd_fp8.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                               ctypes.c_int, ctypes.c_int, ctypes.c_float, _vp]
    lib.fa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_decode_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]   # batch, Hq, Hkv, max_seqlen, d, split
    lib.fa_decode.restype = ctypes.c_int
    lib.fa_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64p,
                              ctypes.c_int, ctypes.c_float, _i32, _vp, ctypes.c_size_t, _vp]
    lib.fa_decode_noalloc.restype = ctypes.c_int
    lib.fa_decode_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64p,
                                      ctypes.c_int, ctypes.c_float, _i32, _vp]
    lib.fa_decode_paged.restype = ctypes.c_int
    lib.fa_decode_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp,      # q, k/v pages, table, seqlens, o, lse
                                    _i32, _i32, _i32, _i32,                  # batch, heads_q, heads_kv, head_dim
                                    _i32, _i32, _i32, _i64p,                 # num_pages, page_size, max_blocks, strides
                                    ctypes.c_int, ctypes.c_float, _i32, _vp, ctypes.c_size_t, _vp]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [ctypes.c_int]
    lib.fa_last_error_message.restype = ctypes.c_char_p
    lib.fa_last_error_message.argtypes = []
    _lib = lib
    return lib


def _check(status: int):
    if status != FA_OK:
        raise FaError(status, load().fa_last_error_message().decode())


def _strides3(t: torch.Tensor):
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B, H, N, d] tensor with contiguous last dimension")
    return (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return FA_DTYPE_BF16
    if dt == torch.float32:
        return FA_DTYPE_FP32
    raise ValueError(f"unsupported dtype {dt}")


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _shape(t: torch.Tensor, want: tuple, name: str):
    if tuple(t.shape) != tuple(want):
        raise ValueError(f"{name} must have shape {tuple(want)}, got {tuple(t.shape)}")


def _dims(t: torch.Tensor, n: int, name: str):
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")


def _on_gpu(*named):
    """Every tensor on one GPU (the C ABI takes device pointers and cannot
    tell a host pointer from a device one, so this is checked here)."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU, got device {t.device}")
        if dev is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, other operands on {dev}")
        dev = t.device


def _lse_arg(lse, want: tuple, device):
    if lse is True:
        return torch.empty(want, dtype=torch.float32, device=device)
    if lse is False or lse is None:
        return None
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(want):
        raise ValueError(f"lse must be a contiguous float32 {list(want)} tensor")
    return lse


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
        scale: float | None = None, out_dtype: torch.dtype | None = None,
        out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = True):
    """Prefill attention. q [B,Hq,N,d], k/v [B,Hkv,Nk,d] on the GPU (bf16 or fp32).

    Returns (O, LSE); LSE is float32 [B,Hq,N] (None if ``lse`` is False).
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dims(t, 4, name)
    B, Hq, N, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _shape(k, (B, Hkv, Nk, d), "k")
    _shape(v, (B, Hkv, Nk, d), "v")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share a dtype")
    _dtype_code(q.dtype)
    if out is not None:
        _shape(out, (B, Hq, N, d), "out")
        _dtype_code(out.dtype)
    _on_gpu(("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse if isinstance(lse, torch.Tensor) else None))
    lib = load()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=out_dtype or q.dtype, device=q.device)
    lse = _lse_arg(lse, (B, Hq, N), q.device)
    st = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                    lse.data_ptr() if lse is not None else None,
                    B, Hq, Hkv, N, Nk, d, _strides3(q), _strides3(k), _strides3(v), _strides3(out),
                    _dtype_code(q.dtype), _dtype_code(out.dtype),
                    FA_MASK_CAUSAL if causal else FA_MASK_NONE, float(scale), _stream(q.device))
    _check(st)
    return out, lse


def _strides2(t: torch.Tensor):
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError("expected a [tokens, heads, d] tensor with contiguous last dimension")
    return (ctypes.c_int64 * 2)(t.stride(0), t.stride(1))


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
               causal: bool = False, window: int | None = None, scale: float | None = None,
               out_dtype: torch.dtype | None = None, out: torch.Tensor | None = None,
               lse: torch.Tensor | bool | None = True):
    """Packed prefill. q [total,Hq,d], k/v [total,Hkv,d] bf16 on the GPU; cu_seqlens int32 [B+1]
    on the GPU; ``window`` (causal only): row r sees keys r-window .. r.

    Returns (O [total,Hq,d], LSE float32 [Hq,total] or None).
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dims(t, 3, name)
    total, Hq, d = q.shape
    Hkv = k.shape[1]
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must be bfloat16")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous() \
            or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be a contiguous int32 vector of batch + 1 >= 2 entries")
    _shape(k, (total, Hkv, d), "k")
    _shape(v, (total, Hkv, d), "v")
    if out is not None:
        _shape(out, (total, Hq, d), "out")
        _dtype_code(out.dtype)
    _on_gpu(("q", q), ("k", k), ("v", v), ("cu_seqlens", cu_seqlens), ("out", out),
            ("lse", lse if isinstance(lse, torch.Tensor) else None))
    lib = load()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((total, Hq, d), dtype=out_dtype or q.dtype, device=q.device)
    lse = _lse_arg(lse, (Hq, total), q.device)
    st = lib.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           lse.data_ptr() if lse is not None else None, cu_seqlens.data_ptr(),
                           cu_seqlens.numel() - 1, Hq, Hkv, total, int(max_seqlen), d,
                           _strides2(q), _strides2(k), _strides2(v), _strides2(out), _dtype_code(out.dtype),
                           FA_MASK_CAUSAL if causal else FA_MASK_NONE, -1 if window is None else int(window),
                           float(scale), _stream(q.device))
    _check(st)
    return out, lse


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, dout: torch.Tensor,
        lse: torch.Tensor, causal: bool = False, scale: float | None = None,
        grad_dtype: torch.dtype | None = None, dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
        dv: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Backward of ``fwd``. q, dout [B,Hq,N,d] bf16 and o (bf16 or float32) sharing element strides;
    k, v [B,Hkv,Nk,d] bf16 sharing strides; lse float32 [B,Hq,N] from ``fwd``. Returns (dq, dk, dv)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _dims(t, 4, name)
    B, Hq, N, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _shape(k, (B, Hkv, Nk, d), "k")
    for t in (q, k, v, dout):
        if t.dtype != torch.bfloat16:
            raise ValueError("q, k, v and dout must be bfloat16")
    _dtype_code(o.dtype)
    if o.stride() != q.stride() or dout.stride() != q.stride() or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must share q's shape and strides")
    if v.stride() != k.stride() or v.shape != k.shape:
        raise ValueError("v must share k's shape and strides")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("lse must be a contiguous float32 [B, Hq, N] tensor")
    for name, t, want in (("dq", dq, (B, Hq, N, d)), ("dk", dk, (B, Hkv, Nk, d)), ("dv", dv, (B, Hkv, Nk, d))):
        if t is not None:
            _shape(t, want, name)
            _dtype_code(t.dtype)
    _on_gpu(("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("lse", lse), ("dq", dq), ("dk", dk),
            ("dv", dv), ("workspace", workspace))
    lib = load()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    gdt = grad_dtype or torch.bfloat16
    dq = torch.empty((B, Hq, N, d), dtype=gdt, device=q.device) if dq is None else dq
    dk = torch.empty((B, Hkv, Nk, d), dtype=gdt, device=q.device) if dk is None else dk
    dv = torch.empty((B, Hkv, Nk, d), dtype=gdt, device=q.device) if dv is None else dv
    if dk.stride() != dv.stride() or dk.dtype != dv.dtype or dq.dtype != dk.dtype:
        raise ValueError("dk and dv must share strides, and all gradients one dtype")
    need = int(lib.fa_bwd_workspace_bytes(B, Hq, N))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                    dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, N, Nk, d, _strides3(q), _strides3(k),
                    _strides3(dq), _strides3(dk), _dtype_code(o.dtype), _dtype_code(dq.dtype),
                    FA_MASK_CAUSAL if causal else FA_MASK_NONE, float(scale), workspace.data_ptr(),
                    workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(st)
    return dq, dk, dv


def fp8_quantize(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, signs: torch.Tensor | None = None) -> dict:
    """FP8 quantiser. q [B,Hq,N,128], k/v [B,Hkv,N,128] bf16 (k and v sharing strides); signs a
    float32 [128] tensor of +-1 on the GPU (None: no rotation). Returns the e4m3 tensors and scales."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dims(t, 4, name)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    _shape(k, (B, Hkv, N, d), "k")
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must be bfloat16")
    if k.stride() != v.stride() or k.shape != v.shape:
        raise ValueError("k and v must share shape and strides")
    if signs is not None and (signs.dtype != torch.float32 or signs.numel() != d or not signs.is_contiguous()):
        raise ValueError("signs must be a contiguous float32 vector of head_dim entries")
    _on_gpu(("q", q), ("k", k), ("v", v), ("signs", signs))
    lib = load()
    f8, dev = torch.float8_e4m3fn, q.device
    npad = -(-N // 64) * 64
    out = dict(q8=torch.empty((B, Hq, N, d), dtype=f8, device=dev),
               q_scale=torch.empty((B, Hq, -(-N // 128)), dtype=torch.float32, device=dev),
               k8=torch.empty((B, Hkv, N, d), dtype=f8, device=dev),
               k_scale=torch.empty((B, Hkv, npad // 64), dtype=torch.float32, device=dev),
               v8t=torch.empty((B, Hkv, d, npad), dtype=f8, device=dev),
               v_scale=torch.empty((B, Hkv), dtype=torch.float32, device=dev))
    st = lib.fa_fp8_quantize(q.data_ptr(), k.data_ptr(), v.data_ptr(), signs.data_ptr() if signs is not None else None,
                             B, Hq, Hkv, N, d, _strides3(q), _strides3(k), out["q8"].data_ptr(), out["k8"].data_ptr(),
                             out["v8t"].data_ptr(), out["q_scale"].data_ptr(), out["k_scale"].data_ptr(),
                             out["v_scale"].data_ptr(), _stream(q.device))
    _check(st)
    return out


def fwd_fp8(quant: dict, causal: bool = False, scale: float | None = None, out_dtype: torch.dtype = torch.bfloat16,
            out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = True):
    """FP8 prefill on ``fp8_quantize``'s outputs. Returns (O [B,Hq,N,128], LSE float32 [B,Hq,N])."""
    _dims(quant["q8"], 4, "q8")
    B, Hq, N, d = quant["q8"].shape
    Hkv = quant["k8"].shape[1]
    npad = -(-N // 64) * 64
    for name, want in (("k8", (B, Hkv, N, d)), ("v8t", (B, Hkv, d, npad)), ("q_scale", (B, Hq, -(-N // 128))),
                       ("k_scale", (B, Hkv, npad // 64)), ("v_scale", (B, Hkv))):
        _shape(quant[name], want, name)
    for name in ("q8", "k8", "v8t"):
        if quant[name].dtype != torch.float8_e4m3fn or not quant[name].is_contiguous():
            raise ValueError(f"{name} must be a contiguous float8_e4m3fn tensor")
    for name in ("q_scale", "k_scale", "v_scale"):
        if quant[name].dtype != torch.float32 or not quant[name].is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor")
    if out is not None:
        _shape(out, (B, Hq, N, d), "out")
        _dtype_code(out.dtype)
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
    _on_gpu(*((n, quant[n]) for n in ("q8", "k8", "v8t", "q_scale", "k_scale", "v_scale")), ("out", out),
            ("lse", lse if isinstance(lse, torch.Tensor) else None))
    lib = load()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=out_dtype, device=quant["q8"].device)
    lse = _lse_arg(lse, (B, Hq, N), out.device)
    st = lib.fa_fwd_fp8(quant["q8"].data_ptr(), quant["k8"].data_ptr(), quant["v8t"].data_ptr(),
                        quant["q_scale"].data_ptr(), quant["k_scale"].data_ptr(), quant["v_scale"].data_ptr(),
                        out.data_ptr(), lse.data_ptr() if lse is not None else None, B, Hq, Hkv, N, d,
                        _dtype_code(out.dtype), FA_MASK_CAUSAL if causal else FA_MASK_NONE, float(scale),
                        _stream(out.device))
    _check(st)
    return out, lse


def decode_workspace_bytes(batch: int, heads_q: int, heads_kv: int, max_seqlen: int, head_dim: int,
                           split_tokens: int = 0) -> int:
    return int(load().fa_decode_workspace_bytes(batch, heads_q, heads_kv, max_seqlen, head_dim, split_tokens))


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seqlens: torch.Tensor,
           scale: float | None = None, split_tokens: int = 0, out_dtype: torch.dtype | None = None,
           out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = True,
           workspace: torch.Tensor | None = None):
    """Split-KV decode. q [B,Hq,d] bf16; caches [B,Hkv,Lmax,d] bf16; seqlens int32 [B] on the GPU."""
    _dims(q, 3, "q")
    _dims(k_cache, 4, "k_cache")
    B, Hq, d = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    _shape(k_cache, (B, Hkv, Lmax, d), "k_cache")
    if q.dtype != torch.bfloat16 or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and the caches must be bfloat16")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if seqlens.dtype != torch.int32 or seqlens.numel() != B or not seqlens.is_contiguous():
        raise ValueError("seqlens must be a contiguous int32 tensor of length batch")
    if out is not None:
        _shape(out, (B, Hq, d), "out")
        _dtype_code(out.dtype)
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
    _on_gpu(("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seqlens", seqlens), ("out", out),
            ("lse", lse if isinstance(lse, torch.Tensor) else None), ("workspace", workspace))
    lib = load()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype or torch.bfloat16, device=q.device)
    lse = _lse_arg(lse, (B, Hq), q.device)
    need = decode_workspace_bytes(B, Hq, Hkv, Lmax, d, split_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib.fa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seqlens.data_ptr(),
                       out.data_ptr(), lse.data_ptr() if lse is not None else None,
                       B, Hq, Hkv, Lmax, d, _strides3(k_cache), _dtype_code(out.dtype), float(scale),
                       int(split_tokens), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                       _stream(q.device))
    _check(st)
    return out, lse



def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seqlens: torch.Tensor,
                   out: torch.Tensor, lse: torch.Tensor | None = None, scale: float | None = None,
                   split_tokens: int = 0):
    """``decode`` through fa_decode_noalloc: the partials live in the library's
    static scratch, so the library allocates nothing; the caller passes the
    output (and optionally the LSE) tensors, so this wrapper allocates nothing
    either."""
    _dims(q, 3, "q")
    _dims(k_cache, 4, "k_cache")
    B, Hq, d = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    _shape(k_cache, (B, Hkv, Lmax, d), "k_cache")
    if q.dtype != torch.bfloat16 or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and the caches must be bfloat16")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if seqlens.dtype != torch.int32 or seqlens.numel() != B or not seqlens.is_contiguous():
        raise ValueError("seqlens must be a contiguous int32 tensor of length batch")
    _shape(out, (B, Hq, d), "out")
    _dtype_code(out.dtype)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq)):
        raise ValueError(f"lse must be a contiguous float32 [{B}, {Hq}] tensor")
    _on_gpu(("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seqlens", seqlens), ("out", out), ("lse", lse))
    lib = load()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.fa_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seqlens.data_ptr(),
                               out.data_ptr(), lse.data_ptr() if lse is not None else None,
                               B, Hq, Hkv, Lmax, d, _strides3(k_cache), _dtype_code(out.dtype), float(scale),
                               int(split_tokens), _stream(q.device))
    _check(st)
    return out, lse

def decode_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                 seqlens: torch.Tensor, scale: float | None = None, split_tokens: int = 0,
                 out_dtype: torch.dtype | None = None, out: torch.Tensor | None = None,
                 lse: torch.Tensor | bool | None = True, workspace: torch.Tensor | None = None):
    """Split-KV decode against a paged cache.

    q [B,Hq,d] bf16; k_pages/v_pages indexed [page, kv head, slot, d] bf16 with
    any strides on the first three axes (a token-major pool [P, page_size,
    Hkv, d] is passed as ``pool.transpose(1, 2)``); block_table int32
    [B, max_blocks]; seqlens int32 [B]; all on the GPU.
    """
    _dims(q, 3, "q")
    _dims(k_pages, 4, "k_pages")
    B, Hq, d = q.shape
    P, Hkv, ps = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    _shape(k_pages, (P, Hkv, ps, d), "k_pages")
    if q.dtype != torch.bfloat16 or k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise ValueError("q and the pages must be bfloat16")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if k_pages.stride() != v_pages.stride() or k_pages.shape != v_pages.shape:
        raise ValueError("k_pages and v_pages must share shape and strides")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B \
            or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 [batch, max_blocks] tensor")
    if seqlens.dtype != torch.int32 or seqlens.numel() != B or not seqlens.is_contiguous():
        raise ValueError("seqlens must be a contiguous int32 tensor of length batch")
    max_blocks = block_table.shape[1]
    if out is not None:
        _shape(out, (B, Hq, d), "out")
        _dtype_code(out.dtype)
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
    _on_gpu(("q", q), ("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table),
            ("seqlens", seqlens), ("out", out), ("lse", lse if isinstance(lse, torch.Tensor) else None),
            ("workspace", workspace))
    lib = load()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype or torch.bfloat16, device=q.device)
    lse = _lse_arg(lse, (B, Hq), q.device)
    need = decode_workspace_bytes(B, Hq, Hkv, max_blocks * ps, d, split_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib.fa_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
                             seqlens.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else None,
                             B, Hq, Hkv, d, P, ps, max_blocks, _strides3(k_pages), _dtype_code(out.dtype),
                             float(scale), int(split_tokens), workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(st)
    return out, lse
