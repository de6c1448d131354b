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
            "fa_decode_workspace_bytes", "fa_decode", "fa_decode_paged", "fa_status_string", "fa_last_error_message")

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
    lib.fa_decode_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32]   # batch, heads_q, heads_kv, max_seqlen, head_dim
    lib.fa_decode.restype = ctypes.c_int
    lib.fa_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64p,
                              ctypes.c_int, ctypes.c_float, _i32, _vp, ctypes.c_size_t, _vp]
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


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
        scale: float | None = None, out_dtype: torch.dtype | None = None,
        out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = True):
    """Prefill attention. q [B,Hq,N,d], k/v [B,Hkv,Nk,d] on the GPU (bf16 or fp32).

    Returns (O, LSE); LSE is float32 [B,Hq,N] (None if ``lse`` is False).
    """
    lib = load()
    B, Hq, N, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=out_dtype or q.dtype, device=q.device)
    if lse is True:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, N)):
        raise ValueError("lse must be a contiguous float32 [B, Hq, N] tensor")
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
    lib = load()
    total, Hq, d = q.shape
    Hkv = k.shape[1]
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must be bfloat16")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 vector")
    if k.shape[0] != total or v.shape[0] != total:
        raise ValueError("q, k and v must hold the same packed tokens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((total, Hq, d), dtype=out_dtype or q.dtype, device=q.device)
    if lse is True:
        lse = torch.empty((Hq, total), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (Hq, total)):
        raise ValueError("lse must be a contiguous float32 [Hq, total] tensor")
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
    lib = load()
    B, Hq, N, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    for t in (q, k, v, dout):
        if t.dtype != torch.bfloat16:
            raise ValueError("q, k, v and dout must be bfloat16")
    if o.stride() != q.stride() or dout.stride() != q.stride() or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must share q's shape and strides")
    if v.stride() != k.stride() or v.shape != k.shape:
        raise ValueError("v must share k's shape and strides")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("lse must be a contiguous float32 [B, Hq, N] tensor")
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
    lib = load()
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must be bfloat16")
    if k.stride() != v.stride() or k.shape != v.shape:
        raise ValueError("k and v must share shape and strides")
    if signs is not None and (signs.dtype != torch.float32 or signs.numel() != d or not signs.is_contiguous()):
        raise ValueError("signs must be a contiguous float32 vector of head_dim entries")
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
    lib = load()
    B, Hq, N, d = quant["q8"].shape
    Hkv = quant["k8"].shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=out_dtype, device=quant["q8"].device)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    if lse is True:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=out.device)
    elif lse is False:
        lse = None
    st = lib.fa_fwd_fp8(quant["q8"].data_ptr(), quant["k8"].data_ptr(), quant["v8t"].data_ptr(),
                        quant["q_scale"].data_ptr(), quant["k_scale"].data_ptr(), quant["v_scale"].data_ptr(),
                        out.data_ptr(), lse.data_ptr() if lse is not None else None, B, Hq, Hkv, N, d,
                        _dtype_code(out.dtype), FA_MASK_CAUSAL if causal else FA_MASK_NONE, float(scale),
                        _stream(out.device))
    _check(st)
    return out, lse


def decode_workspace_bytes(batch: int, heads_q: int, heads_kv: int, max_seqlen: int, head_dim: int) -> int:
    return int(load().fa_decode_workspace_bytes(batch, heads_q, heads_kv, max_seqlen, head_dim))


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seqlens: torch.Tensor,
           scale: float | None = None, split_tokens: int = 0, out_dtype: torch.dtype | None = None,
           out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = True,
           workspace: torch.Tensor | None = None):
    """Split-KV decode. q [B,Hq,d] bf16; caches [B,Hkv,Lmax,d] bf16; seqlens int32 [B] on the GPU."""
    lib = load()
    B, Hq, d = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if seqlens.dtype != torch.int32 or seqlens.numel() != B or not seqlens.is_contiguous():
        raise ValueError("seqlens must be a contiguous int32 tensor of length batch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype or torch.bfloat16, device=q.device)
    if lse is True:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    need = decode_workspace_bytes(B, Hq, Hkv, Lmax, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib.fa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seqlens.data_ptr(),
                       out.data_ptr(), lse.data_ptr() if lse is not None else None,
                       B, Hq, Hkv, Lmax, d, _strides3(k_cache), _dtype_code(out.dtype), float(scale),
                       int(split_tokens), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                       _stream(q.device))
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
    lib = load()
    B, Hq, d = q.shape
    P, Hkv, ps = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
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
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype or torch.bfloat16, device=q.device)
    if lse is True:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    need = decode_workspace_bytes(B, Hq, Hkv, max_blocks * ps, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib.fa_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
                             seqlens.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else None,
                             B, Hq, Hkv, d, P, ps, max_blocks, _strides3(k_pages), _dtype_code(out.dtype),
                             float(scale), int(split_tokens), workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(st)
    return out, lse
