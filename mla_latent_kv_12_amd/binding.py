"""Thin ctypes binding of ``libmla.so`` (the C ABI in include/mla.h).

Argument marshalling only: every computation runs in the library's HIP
kernels.  Torch tensors supply device memory and the current stream.  If the
library is missing this module raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = range(5)
MLA_F32, MLA_BF16 = 0, 1
NOALLOC_MAX_BYTES = 80 << 20  # MLA_DECODE_NOALLOC_MAX_BYTES in include/mla.h

EXPORTS = (
    "mla_absorb_q",
    "mla_decode_num_splits",
    "mla_decode_workspace_bytes",
    "mla_decode",
    "mla_decode_profiled",
    "mla_decode_noalloc",
    "mla_decode_latent",
    "mla_prefill_workspace_bytes",
    "mla_prefill_naive",
    "mla_prefill_absorbed_num_splits",
    "mla_prefill_absorbed_workspace_bytes",
    "mla_prefill_absorbed",
    "mla_output_proj_workspace_bytes",
    "mla_output_proj",
    "mla_fold_value_output",
    "mla_cache_append",
    "mla_kv_cache_bytes",
    "mla_status_string",
    "mla_last_error",
    "mla_version",
)


class MLAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


class DecodeParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("d_c", ctypes.c_int64),
        ("d_r", ctypes.c_int64), ("d_n", ctypes.c_int64), ("d_v", ctypes.c_int64),
        ("n_max", ctypes.c_int64),
        ("ckv_stride_b", ctypes.c_int64), ("ckv_stride_n", ctypes.c_int64),
        ("kpe_stride_b", ctypes.c_int64), ("kpe_stride_n", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("num_splits", ctypes.c_int32),
        ("q_rope_base", ctypes.c_double),
    ]


class PrefillParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("tokens", ctypes.c_int64), ("heads", ctypes.c_int64),
        ("d_c", ctypes.c_int64), ("d_r", ctypes.c_int64), ("d_n", ctypes.c_int64),
        ("d_v", ctypes.c_int64), ("n_max", ctypes.c_int64),
        ("ckv_stride_b", ctypes.c_int64), ("ckv_stride_n", ctypes.c_int64),
        ("kpe_stride_b", ctypes.c_int64), ("kpe_stride_n", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("num_splits", ctypes.c_int32),
        ("q_rope_base", ctypes.c_double),
    ]


class ProjParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("in_features", ctypes.c_int64),
        ("out_features", ctypes.c_int64), ("dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("num_splits", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class AppendParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("d_model", ctypes.c_int64), ("d_c", ctypes.c_int64),
        ("d_r", ctypes.c_int64), ("n_max", ctypes.c_int64),
        ("ckv_stride_b", ctypes.c_int64), ("ckv_stride_n", ctypes.c_int64),
        ("kpe_stride_b", ctypes.c_int64), ("kpe_stride_n", ctypes.c_int64),
        ("rope_base", ctypes.c_double), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load ``libmla.so`` (built by ``mla_latent_kv_12_amd.build``); raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MLAError(-1, f"{LIB_PATH} is missing: build it with "
                               "`python -m mla_latent_kv_12_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.mla_absorb_q.argtypes = [ctypes.POINTER(DecodeParams), vp, vp, vp, vp]
        L.mla_absorb_q.restype = ctypes.c_int
        L.mla_decode_num_splits.argtypes = [ctypes.POINTER(DecodeParams)]
        L.mla_decode_num_splits.restype = ctypes.c_int
        L.mla_decode_workspace_bytes.argtypes = [ctypes.POINTER(DecodeParams)]
        L.mla_decode_workspace_bytes.restype = sz
        L.mla_decode.argtypes = [ctypes.POINTER(DecodeParams), vp, vp, vp, vp, vp, vp, vp, vp,
                                 vp, sz, vp]
        L.mla_decode.restype = ctypes.c_int
        L.mla_decode_profiled.argtypes = [ctypes.POINTER(DecodeParams), vp, vp, vp, vp, vp, vp,
                                          vp, vp, vp, sz, vp, vp]
        L.mla_decode_profiled.restype = ctypes.c_int
        L.mla_decode_noalloc.argtypes = [ctypes.POINTER(DecodeParams), vp, vp, vp, vp, vp, vp,
                                         vp, vp, vp]
        L.mla_decode_noalloc.restype = ctypes.c_int
        L.mla_decode_latent.argtypes = [ctypes.POINTER(DecodeParams), vp, vp, vp, vp, vp, vp, vp,
                                        vp, sz, vp]
        L.mla_decode_latent.restype = ctypes.c_int
        L.mla_output_proj_workspace_bytes.argtypes = [ctypes.POINTER(ProjParams)]
        L.mla_output_proj_workspace_bytes.restype = sz
        L.mla_output_proj.argtypes = [ctypes.POINTER(ProjParams), vp, vp, vp, vp, sz, vp]
        L.mla_output_proj.restype = ctypes.c_int
        L.mla_fold_value_output.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int32, vp, vp, vp, vp]
        L.mla_fold_value_output.restype = ctypes.c_int
        L.mla_prefill_workspace_bytes.argtypes = [ctypes.POINTER(PrefillParams)]
        L.mla_prefill_workspace_bytes.restype = sz
        L.mla_prefill_naive.argtypes = [ctypes.POINTER(PrefillParams), vp, vp, vp, vp, vp, vp, vp,
                                        vp, vp, sz, vp]
        L.mla_prefill_naive.restype = ctypes.c_int
        L.mla_prefill_absorbed_num_splits.argtypes = [ctypes.POINTER(PrefillParams)]
        L.mla_prefill_absorbed_num_splits.restype = ctypes.c_int
        L.mla_prefill_absorbed_workspace_bytes.argtypes = [ctypes.POINTER(PrefillParams)]
        L.mla_prefill_absorbed_workspace_bytes.restype = sz
        L.mla_prefill_absorbed.argtypes = [ctypes.POINTER(PrefillParams), vp, vp, vp, vp, vp, vp,
                                           vp, vp, vp, sz, vp]
        L.mla_prefill_absorbed.restype = ctypes.c_int
        L.mla_cache_append.argtypes = [ctypes.POINTER(AppendParams), vp, vp, vp, vp, vp, vp, vp]
        L.mla_cache_append.restype = ctypes.c_int
        L.mla_kv_cache_bytes.argtypes = [ctypes.c_int64] * 6
        L.mla_kv_cache_bytes.restype = ctypes.c_uint64
        L.mla_status_string.argtypes = [ctypes.c_int]
        L.mla_status_string.restype = ctypes.c_char_p
        L.mla_last_error.argtypes = []
        L.mla_last_error.restype = ctypes.c_char_p
        L.mla_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != MLA_OK:
        raise MLAError(status, lib().mla_last_error().decode())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return MLA_F32
    if t == torch.bfloat16:
        return MLA_BF16
    raise MLAError(MLA_ERR_UNSUPPORTED, f"dtype {t} is not supported (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_TORCH_DTYPE = {MLA_F32: torch.float32, MLA_BF16: torch.bfloat16}


def _need(t, what: str, shape, dtype) -> None:
    """The library reads and writes plain pointers: every tensor must be a
    contiguous GPU tensor of exactly the shape and dtype the call implies."""
    if not isinstance(t, torch.Tensor):
        raise MLAError(MLA_ERR_INVALID_ARG, f"{what} must be a tensor")
    if t.device.type != "cuda":
        raise MLAError(MLA_ERR_INVALID_ARG, f"{what} must be on the GPU (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise MLAError(MLA_ERR_INVALID_ARG, f"{what} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(int(d) for d in shape):
        raise MLAError(MLA_ERR_INVALID_ARG,
                       f"{what} must have shape {tuple(int(d) for d in shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise MLAError(MLA_ERR_INVALID_ARG, f"{what} must be contiguous")


def _need_cache(t, what: str, batch: int, n_max: int, width: int, dtype, stride_b: int,
                stride_n: int) -> None:
    """A cache view: [batch, n_max, width] with unit element stride and the
    sequence and row strides the parameters carry."""
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise MLAError(MLA_ERR_INVALID_ARG, f"{what} must be a GPU tensor")
    if t.dtype != dtype:
        raise MLAError(MLA_ERR_INVALID_ARG, f"{what} must be {dtype} (got {t.dtype})")
    if (t.dim() != 3 or tuple(t.shape) != (batch, n_max, width) or t.stride(2) != 1 or
            (batch > 1 and t.stride(0) != stride_b) or t.stride(1) != stride_n):
        raise MLAError(MLA_ERR_INVALID_ARG,
                       f"{what} must be a [{batch}, {n_max}, {width}] view with unit element "
                       f"stride and strides ({stride_b}, {stride_n}) (got shape "
                       f"{tuple(t.shape)}, strides {tuple(t.stride())})")


def _need_workspace(ws) -> None:
    if ws is not None and (not isinstance(ws, torch.Tensor) or ws.device.type != "cuda" or
                           ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous()):
        raise MLAError(MLA_ERR_INVALID_ARG, "workspace must be a contiguous 1-D uint8 GPU tensor")


def _check_attention_tensors(p, q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens, out,
                             workspace, *, rows, out_width) -> None:
    """rows: the leading query dimensions ((B,) for decode, (B, T) for prefill)."""
    dt, odt = _TORCH_DTYPE[p.dtype], _TORCH_DTYPE[p.out_dtype]
    _need(q_nope, "q_nope", rows + (p.heads, p.d_n), dt)
    if p.d_r > 0:
        _need(q_rope, "q_rope", rows + (p.heads, p.d_r), dt)
    _need(w_uk, "w_uk", (p.heads, p.d_n, p.d_c), dt)
    if w_uv is not None:
        _need(w_uv, "w_uv", (p.heads, p.d_v, p.d_c), dt)
    _need_cache(ckv_cache, "ckv_cache", p.batch, p.n_max, p.d_c, dt, p.ckv_stride_b,
                p.ckv_stride_n)
    if p.d_r > 0:
        _need_cache(kpe_cache, "kpe_cache", p.batch, p.n_max, p.d_r, dt, p.kpe_stride_b,
                    p.kpe_stride_n)
    _need(seqlens, "seqlens", (p.batch,), torch.int32)
    _need(out, "out", rows + (p.heads, out_width), odt)
    _need_workspace(workspace)


def _cache_strides(cache: torch.Tensor, width: int, what: str):
    if cache.dim() != 3 or cache.shape[2] != width or cache.stride(2) != 1:
        raise MLAError(MLA_ERR_INVALID_ARG, f"{what} must be a [B, N, {width}] view with unit "
                                            "element stride")
    return cache.stride(0), cache.stride(1)


def decode_params(q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, *, softmax_scale=None,
                  out_dtype=None, num_splits=0, q_rope_base=None) -> DecodeParams:
    B, H, dn = q_nope.shape
    dr = q_rope.shape[-1]
    dc = w_uk.shape[2]
    dv = w_uv.shape[1]
    csb, csn = _cache_strides(ckv_cache, dc, "ckv_cache")
    ksb, ksn = _cache_strides(kpe_cache, dr, "kpe_cache")
    return DecodeParams(
        batch=B, heads=H, d_c=dc, d_r=dr, d_n=dn, d_v=dv, n_max=ckv_cache.shape[1],
        ckv_stride_b=csb, ckv_stride_n=csn, kpe_stride_b=ksb, kpe_stride_n=ksn,
        softmax_scale=0.0 if softmax_scale is None else float(softmax_scale),
        dtype=_dtype_code(q_nope.dtype),
        out_dtype=_dtype_code(out_dtype if out_dtype is not None else q_nope.dtype),
        num_splits=int(num_splits),
        q_rope_base=0.0 if q_rope_base is None else float(q_rope_base))


def decode_num_splits(params: DecodeParams) -> int:
    return int(lib().mla_decode_num_splits(ctypes.byref(params)))


def decode_workspace_bytes(params: DecodeParams) -> int:
    return int(lib().mla_decode_workspace_bytes(ctypes.byref(params)))


def absorb_q(q_nope: torch.Tensor, w_uk: torch.Tensor, out: torch.Tensor | None = None,
             stream=None) -> torch.Tensor:
    """q_abs[b,h,:] = W_UK[h]^T q_nope[b,h,:] in fp32 (``mla_absorb_q``)."""
    B, H, dn = q_nope.shape
    dc = w_uk.shape[2]
    if out is None:
        out = torch.empty((B, H, dc), dtype=torch.float32, device=q_nope.device)
    _need(q_nope, "q_nope", (B, H, dn), q_nope.dtype)
    _need(w_uk, "w_uk", (H, dn, dc), q_nope.dtype)
    _need(out, "out", (B, H, dc), torch.float32)
    p = DecodeParams(batch=B, heads=H, d_c=dc, d_r=0, d_n=dn, d_v=1, n_max=1,
                     dtype=_dtype_code(q_nope.dtype), out_dtype=MLA_F32)
    qn, wk = q_nope.contiguous(), w_uk.contiguous()
    _check(lib().mla_absorb_q(ctypes.byref(p), _ptr(qn), _ptr(wk), _ptr(out), _stream(stream)))
    return out


def decode(q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens, *, out=None,
           workspace=None, softmax_scale=None, out_dtype=None, num_splits=0, q_rope_base=None,
           stream=None, params: DecodeParams | None = None, events=None):
    """Absorbed MLA decode (``mla_decode``).  Shapes as in include/mla.h;
    caches are [B, N_max, width] views (they may share one buffer).
    ``q_rope_base``: None if q_rope arrives rotated, else the rotary base with
    which the library rotates it at position seqlens[b] - 1.
    ``events``: optional ctypes array of 4 hipEvent_t handles, recorded around
    the three kernels (``mla_decode_profiled``)."""
    if params is None:
        params = decode_params(q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache,
                               softmax_scale=softmax_scale, out_dtype=out_dtype,
                               num_splits=num_splits, q_rope_base=q_rope_base)
    if out is None:
        odt = torch.float32 if params.out_dtype == MLA_F32 else torch.bfloat16
        out = torch.empty((params.batch, params.heads, params.d_v), dtype=odt,
                          device=q_nope.device)
    need = decode_workspace_bytes(params)
    if need == 0:
        _check(lib().mla_decode(ctypes.byref(params), None, None, None, None, None, None, None,
                                None, None, 0, None))
    _check_attention_tensors(params, q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens,
                             out, workspace, rows=(params.batch,), out_width=params.d_v)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_nope.device)
    if events is None:
        _check(lib().mla_decode(ctypes.byref(params), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                                _ptr(w_uv), _ptr(ckv_cache), _ptr(kpe_cache), _ptr(seqlens),
                                _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))
    else:
        _check(lib().mla_decode_profiled(ctypes.byref(params), _ptr(q_nope), _ptr(q_rope),
                                         _ptr(w_uk), _ptr(w_uv), _ptr(ckv_cache),
                                         _ptr(kpe_cache), _ptr(seqlens), _ptr(out),
                                         _ptr(workspace), workspace.numel(), _stream(stream),
                                         events))
    return out


def decode_noalloc(q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens, *, out,
                   softmax_scale=None, out_dtype=None, num_splits=0, q_rope_base=None,
                   stream=None, params: DecodeParams | None = None):
    """``mla_decode_noalloc``: mla_decode with the library's own fixed device
    scratch (NOALLOC_MAX_BYTES) instead of a workspace; ``out`` is the
    caller's.  Calls that overlap in time on one GPU race on that scratch."""
    if params is None:
        params = decode_params(q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache,
                               softmax_scale=softmax_scale, out_dtype=out_dtype,
                               num_splits=num_splits, q_rope_base=q_rope_base)
    _check_attention_tensors(params, q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens,
                             out, None, rows=(params.batch,), out_width=params.d_v)
    _check(lib().mla_decode_noalloc(ctypes.byref(params), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                                    _ptr(w_uv), _ptr(ckv_cache), _ptr(kpe_cache), _ptr(seqlens),
                                    _ptr(out), _stream(stream)))
    return out


def decode_latent(q_nope, q_rope, w_uk, ckv_cache, kpe_cache, seqlens, *, out=None,
                  workspace=None, softmax_scale=None, out_dtype=None, num_splits=0,
                  q_rope_base=None, stream=None, params: DecodeParams | None = None):
    """Absorbed decode up to the merged latent (``mla_decode_latent``):
    o_lat [B, H, d_c] = sum_n p_n c[b, n], before any up-projection."""
    B, H, dn = q_nope.shape
    dc = w_uk.shape[2]
    if params is None:
        # d_v plays no part in the latent form; the workspace query checks it
        # against the implemented widths (128 on the bf16 path)
        dv = 128 if w_uk.dtype == torch.bfloat16 else 1
        fake_wuv = torch.empty((H, dv, dc), dtype=w_uk.dtype, device="meta")
        params = decode_params(q_nope, q_rope, w_uk, fake_wuv, ckv_cache, kpe_cache,
                               softmax_scale=softmax_scale, out_dtype=out_dtype,
                               num_splits=num_splits, q_rope_base=q_rope_base)
    if out is None:
        odt = torch.float32 if params.out_dtype == MLA_F32 else torch.bfloat16
        out = torch.empty((B, H, dc), dtype=odt, device=q_nope.device)
    need = decode_workspace_bytes(params)
    if need == 0:
        _check(lib().mla_decode_latent(ctypes.byref(params), None, None, None, None, None, None,
                                       None, None, 0, None))
    _check_attention_tensors(params, q_nope, q_rope, w_uk, None, ckv_cache, kpe_cache, seqlens,
                             out, workspace, rows=(params.batch,), out_width=params.d_c)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_nope.device)
    _check(lib().mla_decode_latent(ctypes.byref(params), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                                   _ptr(ckv_cache), _ptr(kpe_cache), _ptr(seqlens), _ptr(out),
                                   _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def proj_params(x, w, *, out_dtype=None, num_splits=0) -> ProjParams:
    B, K = x.shape
    N = w.shape[0]
    return ProjParams(batch=B, in_features=K, out_features=N, dtype=_dtype_code(x.dtype),
                      out_dtype=_dtype_code(out_dtype if out_dtype is not None else x.dtype),
                      num_splits=int(num_splits), reserved=0)


def output_proj_workspace_bytes(params: ProjParams) -> int:
    return int(lib().mla_output_proj_workspace_bytes(ctypes.byref(params)))


def output_proj(x, w, *, out=None, workspace=None, out_dtype=None, num_splits=0, stream=None,
                params: ProjParams | None = None):
    """Output projection y = x w^T (``mla_output_proj``): x [B, K], w [N, K] -> y [B, N]."""
    if params is None:
        params = proj_params(x, w, out_dtype=out_dtype, num_splits=num_splits)
    if out is None:
        odt = torch.float32 if params.out_dtype == MLA_F32 else torch.bfloat16
        out = torch.empty((params.batch, params.out_features), dtype=odt, device=x.device)
    dt, odt = _TORCH_DTYPE.get(params.dtype), _TORCH_DTYPE.get(params.out_dtype)
    _need(x, "x", (params.batch, params.in_features), dt)
    _need(w, "w", (params.out_features, params.in_features), dt)
    _need(out, "out", (params.batch, params.out_features), odt)
    _need_workspace(workspace)
    # 0 bytes: the direct form needs none, or params are invalid (the call
    # itself then reports why, before any launch)
    need = output_proj_workspace_bytes(params)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(lib().mla_output_proj(ctypes.byref(params), _ptr(x), _ptr(w), _ptr(out),
                                 _ptr(workspace) if ws_bytes else None, ws_bytes, _stream(stream)))
    return out


def fold_value_output(w_o, w_uv, *, out=None, stream=None):
    """W_OV [d_model, H*d_c] = W_O [d_model, H*d_v] folded with W_UV [H, d_v, d_c]
    (``mla_fold_value_output``)."""
    H, dv, dc = w_uv.shape
    d_model = w_o.shape[0]
    if out is None:
        out = torch.empty((d_model, H * dc), dtype=w_o.dtype, device=w_o.device)
    _dtype_code(w_o.dtype)
    _need(w_o, "w_o", (d_model, H * dv), w_o.dtype)
    _need(w_uv, "w_uv", (H, dv, dc), w_o.dtype)
    _need(out, "out", (d_model, H * dc), w_o.dtype)
    _check(lib().mla_fold_value_output(d_model, H, dv, dc, _dtype_code(w_o.dtype), _ptr(w_o),
                                       _ptr(w_uv), _ptr(out), _stream(stream)))
    return out


def prefill_params(q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, *, softmax_scale=None,
                   out_dtype=None, num_splits=0, q_rope_base=None) -> PrefillParams:
    B, T, H, dn = q_nope.shape
    dr = q_rope.shape[-1]
    dc = w_uk.shape[2]
    dv = w_uv.shape[1]
    csb, csn = _cache_strides(ckv_cache, dc, "ckv_cache")
    ksb, ksn = _cache_strides(kpe_cache, dr, "kpe_cache")
    return PrefillParams(
        batch=B, tokens=T, heads=H, d_c=dc, d_r=dr, d_n=dn, d_v=dv, n_max=ckv_cache.shape[1],
        ckv_stride_b=csb, ckv_stride_n=csn, kpe_stride_b=ksb, kpe_stride_n=ksn,
        softmax_scale=0.0 if softmax_scale is None else float(softmax_scale),
        dtype=_dtype_code(q_nope.dtype),
        out_dtype=_dtype_code(out_dtype if out_dtype is not None else q_nope.dtype),
        num_splits=int(num_splits),
        q_rope_base=0.0 if q_rope_base is None else float(q_rope_base))


def prefill_workspace_bytes(params: PrefillParams) -> int:
    return int(lib().mla_prefill_workspace_bytes(ctypes.byref(params)))


def prefill_naive(q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens, *, out=None,
                  workspace=None, softmax_scale=None, out_dtype=None, q_rope_base=None,
                  stream=None, params: PrefillParams | None = None):
    """Naive causal prefill (``mla_prefill_naive``): q [B,T,H,*] -> out [B,T,H,d_v]."""
    if params is None:
        params = prefill_params(q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache,
                                softmax_scale=softmax_scale, out_dtype=out_dtype,
                                q_rope_base=q_rope_base)
    if out is None:
        odt = torch.float32 if params.out_dtype == MLA_F32 else torch.bfloat16
        out = torch.empty((params.batch, params.tokens, params.heads, params.d_v), dtype=odt,
                          device=q_nope.device)
    need = prefill_workspace_bytes(params)
    if need == 0:
        _check(lib().mla_prefill_naive(ctypes.byref(params), None, None, None, None, None, None,
                                       None, None, None, 0, None))
    _check_attention_tensors(params, q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens,
                             out, workspace, rows=(params.batch, params.tokens),
                             out_width=params.d_v)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_nope.device)
    _check(lib().mla_prefill_naive(ctypes.byref(params), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                                   _ptr(w_uv), _ptr(ckv_cache), _ptr(kpe_cache), _ptr(seqlens),
                                   _ptr(out), _ptr(workspace), workspace.numel(),
                                   _stream(stream)))
    return out


def prefill_absorbed_num_splits(params: PrefillParams) -> int:
    return int(lib().mla_prefill_absorbed_num_splits(ctypes.byref(params)))


def prefill_absorbed_workspace_bytes(params: PrefillParams) -> int:
    return int(lib().mla_prefill_absorbed_workspace_bytes(ctypes.byref(params)))


def prefill_absorbed(q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens, *, out=None,
                     workspace=None, softmax_scale=None, out_dtype=None, num_splits=0,
                     q_rope_base=None, stream=None, params: PrefillParams | None = None):
    """Absorbed causal prefill (``mla_prefill_absorbed``): q [B,T,H,*] ->
    out [B,T,H,d_v], each query attending to its causal prefix in latent space."""
    if params is None:
        params = prefill_params(q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache,
                                softmax_scale=softmax_scale, out_dtype=out_dtype,
                                num_splits=num_splits, q_rope_base=q_rope_base)
    if out is None:
        odt = torch.float32 if params.out_dtype == MLA_F32 else torch.bfloat16
        out = torch.empty((params.batch, params.tokens, params.heads, params.d_v), dtype=odt,
                          device=q_nope.device)
    need = prefill_absorbed_workspace_bytes(params)
    if need == 0:
        _check(lib().mla_prefill_absorbed(ctypes.byref(params), None, None, None, None, None,
                                          None, None, None, None, 0, None))
    _check_attention_tensors(params, q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens,
                             out, workspace, rows=(params.batch, params.tokens),
                             out_width=params.d_v)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_nope.device)
    _check(lib().mla_prefill_absorbed(ctypes.byref(params), _ptr(q_nope), _ptr(q_rope),
                                      _ptr(w_uk), _ptr(w_uv), _ptr(ckv_cache), _ptr(kpe_cache),
                                      _ptr(seqlens), _ptr(out), _ptr(workspace),
                                      workspace.numel(), _stream(stream)))
    return out


def cache_append(h, w_dkv, w_kr, positions, ckv_cache, kpe_cache, *, rope_base=None,
                 stream=None):
    """Write the new token's cache rows (``mla_cache_append``): for each sequence b
    with 0 <= positions[b] < n_max, ckv_cache[b, pos] = W_DKV h[b] and
    kpe_cache[b, pos] = RoPE_pos(W_KR h[b]).  h [B, d_model], W_DKV [d_c, d_model],
    W_KR [d_r, d_model]; the caches are [B, n_max, width] views (updated in place)."""
    B, d_model = h.shape
    dc = w_dkv.shape[0]
    dr = w_kr.shape[0] if w_kr is not None else 0
    csb, csn = _cache_strides(ckv_cache, dc, "ckv_cache")
    ksb, ksn = _cache_strides(kpe_cache, dr, "kpe_cache") if dr > 0 else (0, 0)
    p = AppendParams(batch=B, d_model=d_model, d_c=dc, d_r=dr, n_max=ckv_cache.shape[1],
                     ckv_stride_b=csb, ckv_stride_n=csn, kpe_stride_b=ksb, kpe_stride_n=ksn,
                     rope_base=0.0 if rope_base is None else float(rope_base),
                     dtype=_dtype_code(h.dtype), reserved=0)
    dt = h.dtype
    _need(h, "h", (B, d_model), dt)
    _need(w_dkv, "w_dkv", (dc, d_model), dt)
    if dr > 0:
        _need(w_kr, "w_kr", (dr, d_model), dt)
    _need(positions, "positions", (B,), torch.int32)
    _need_cache(ckv_cache, "ckv_cache", B, p.n_max, dc, dt, csb, csn)
    if dr > 0:
        _need_cache(kpe_cache, "kpe_cache", B, p.n_max, dr, dt, ksb, ksn)
    _check(lib().mla_cache_append(ctypes.byref(p), _ptr(h), _ptr(w_dkv), _ptr(w_kr),
                                  _ptr(positions), _ptr(ckv_cache),
                                  _ptr(kpe_cache) if dr > 0 else None, _stream(stream)))


def kv_cache_bytes(n_layers, batch, seq_len, d_c=512, d_r=64, bytes_per_elem=2) -> int:
    return int(lib().mla_kv_cache_bytes(n_layers, batch, seq_len, d_c, d_r, bytes_per_elem))


def status_string(status: int) -> str:
    return lib().mla_status_string(status).decode()


def version() -> int:
    return int(lib().mla_version())


def default_scale(d_n: int, d_r: int) -> float:
    return 1.0 / math.sqrt(d_n + d_r)
