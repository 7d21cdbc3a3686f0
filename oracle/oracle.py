"""ctypes wrapper of the fp64 C oracle (``mla_oracle.c``).

Test infrastructure only (see the package docstring).  Inputs are numpy
arrays holding the exact stored values: float64, float32, or bfloat16 bit
patterns as uint16.  The C code widens them to double itself.

Parity status of each function (the pins live in ``tests/test_oracle_pins.py``):
  decode_naive     pinned: torch fp64 scaled-dot-product attention over
                   explicitly decompressed K/V, closed forms at L=1, uniform
                   scores, softmax mass, cache permutation, padding.
  absorb_q         pinned: the content-score identity q~ . c == q . (W_UK c).
  decode_absorbed  pinned: equals decode_naive on the latent-width x length x
                   RoPE-width grid, plus the same closed forms.
  prefill_naive    pinned: torch fp64 attention with an explicit bottom-right
                   causal mask; T=1 reduces to decode.
  prefill_absorbed pinned: equals prefill_naive over a grid of widths, query
                   counts and lengths (L < T included); each row equals
                   decode_absorbed over its causal prefix.
  kv_cache_bytes   pinned: the cache tables printed on the pages.
  decode_latent    pinned: W_UV times it equals decode_absorbed; L=1 gives the
                   cached latent row exactly.
  output_proj      pinned: a numpy fp64 matrix product.
  fold_value_output pinned: selection-matrix W_UV gives W_O's columns exactly in
                   the selected places; the folded and unfolded projections of
                   the same decode agree (associativity).
  rope             pinned: the relative-position property (scores depend only on
                   the position difference), norm preservation, position 0 is
                   the identity, closed forms for one and two rotation pairs.
  cache_rows       pinned: position 0 equals a plain fp64 matrix product
                   (numpy); the RoPE part is rope() of that product.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "libmla_oracle.so")

OR_F64, OR_F32, OR_BF16 = 0, 1, 2


class OracleError(RuntimeError):
    pass


class _Dims(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("dc", ctypes.c_int64),
        ("dr", ctypes.c_int64), ("dn", ctypes.c_int64), ("dv", ctypes.c_int64),
        ("ckv_sb", ctypes.c_int64), ("ckv_sn", ctypes.c_int64),
        ("kpe_sb", ctypes.c_int64), ("kpe_sn", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("scale", ctypes.c_double),
    ]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP) into ``libmla_oracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _open(path: str) -> ctypes.CDLL:
    """Load a build of ``mla_oracle.c`` and declare its C signatures."""
    lib = ctypes.CDLL(path)
    vp, i64, dp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p
    for name in ("oracle_decode_naive", "oracle_decode_absorbed"):
        f = getattr(lib, name)
        f.argtypes = [ctypes.POINTER(_Dims), vp, vp, vp, vp, vp, vp, vp, vp, i64, dp, dp]
        f.restype = ctypes.c_int
    lib.oracle_absorb_q.argtypes = [ctypes.POINTER(_Dims), vp, vp, dp]
    lib.oracle_absorb_q.restype = ctypes.c_int
    for name in ("oracle_prefill_naive", "oracle_prefill_absorbed"):
        f = getattr(lib, name)
        f.argtypes = [ctypes.POINTER(_Dims), i64, vp, vp, vp, vp, vp, vp, vp, vp, i64, dp]
        f.restype = ctypes.c_int
    lib.oracle_decode_latent.argtypes = [ctypes.POINTER(_Dims), vp, vp, vp, vp, vp, vp, vp, i64,
                                         dp]
    lib.oracle_decode_latent.restype = ctypes.c_int
    lib.oracle_output_proj.argtypes = [i64, i64, i64, ctypes.c_int32, vp, ctypes.c_int32, vp, dp]
    lib.oracle_output_proj.restype = ctypes.c_int
    lib.oracle_fold_value_output.argtypes = [i64, i64, i64, i64, ctypes.c_int32, vp, vp, dp]
    lib.oracle_fold_value_output.restype = ctypes.c_int
    lib.oracle_kv_cache_bytes.argtypes = [i64] * 6
    lib.oracle_rope.argtypes = [i64, dp, ctypes.c_double, ctypes.c_double, dp]
    lib.oracle_rope.restype = None
    lib.oracle_cache_rows.argtypes = [i64, i64, i64, i64, ctypes.c_int32, vp, vp, vp, vp,
                                      ctypes.c_double, dp, dp]
    lib.oracle_cache_rows.restype = ctypes.c_int
    lib.oracle_kv_cache_bytes.restype = ctypes.c_uint64
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _open(_LIB)
    return _lib


def _code(a: np.ndarray) -> int:
    if a.dtype == np.float64:
        return OR_F64
    if a.dtype == np.float32:
        return OR_F32
    if a.dtype == np.uint16:
        return OR_BF16
    raise OracleError(f"unsupported storage dtype {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _cache_view(cache: np.ndarray, dim: int):
    """(base array, stride_b, stride_n) for a [B, N, >=dim] row-major view."""
    if cache.ndim != 3:
        raise OracleError("caches must be [B, N, width] views")
    es = cache.dtype.itemsize
    sb, sn, sc = (s // es for s in cache.strides)
    if sc != 1 or cache.shape[2] != dim:
        raise OracleError("cache rows must be contiguous and exactly the feature width")
    return cache, sb, sn


def _dims(q_nope, q_rope, w_uk, w_uv, ckv, kpe, scale, H_axis):
    dt = _code(q_nope)
    for a in (q_rope, w_uk, w_uv, ckv, kpe):
        if _code(a) != dt:
            raise OracleError("all inputs must share one storage dtype")
    H, dn, dc = w_uk.shape
    dv = w_uv.shape[1]
    dr = q_rope.shape[-1]
    _, csb, csn = _cache_view(ckv, dc)
    _, ksb, ksn = _cache_view(kpe, dr) if dr > 0 else (kpe, 0, 0)
    d = _Dims(B=ckv.shape[0], H=H, dc=dc, dr=dr, dn=dn, dv=dv, ckv_sb=csb, ckv_sn=csn,
              kpe_sb=ksb, kpe_sn=ksn, dtype=dt, reserved=0, scale=float(scale))
    return d


def _base_ptr(a: np.ndarray):
    # pointer to element [0,0,0] of a possibly strided cache view
    return ctypes.c_void_p(a.__array_interface__["data"][0])


def _decode(fname, q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens, scale, pairs):
    q_nope = np.ascontiguousarray(q_nope)
    q_rope = np.ascontiguousarray(q_rope)
    w_uk = np.ascontiguousarray(w_uk)
    w_uv = np.ascontiguousarray(w_uv)
    d = _dims(q_nope, q_rope, w_uk, w_uv, ckv, kpe, scale, 1)
    seq = np.ascontiguousarray(seqlens, dtype=np.int32)
    if pairs is None:
        n = d.B * d.H
        pp = None
    else:
        pp = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
        n = pp.shape[0]
    out = np.zeros((n, d.dv), dtype=np.float64)
    psum = np.zeros(n, dtype=np.float64)
    rc = getattr(_load(), fname)(ctypes.byref(d), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                                 _ptr(w_uv), _base_ptr(ckv), _base_ptr(kpe), _ptr(seq),
                                 _ptr(pp), n, _ptr(out), _ptr(psum))
    if rc != 0:
        raise OracleError(f"{fname} rejected its arguments")
    if pairs is None:
        return out.reshape(d.B, d.H, d.dv), psum.reshape(d.B, d.H)
    return out, psum


def decode_naive(q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens, scale, pairs=None):
    """O1: decompress-then-attend decode.  Returns (out, softmax_mass).

    Shapes: q_nope [B,H,dn], q_rope [B,H,dr], w_uk [H,dn,dc], w_uv [H,dv,dc],
    ckv [B,N,dc] and kpe [B,N,dr] (views into one buffer are fine),
    seqlens [B] (cached length including the current token).
    With ``pairs`` ([(b,h), ...]) only those pairs are computed and out is
    [len(pairs), dv]; otherwise out is [B,H,dv].
    """
    return _decode("oracle_decode_naive", q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens,
                   scale, pairs)


def decode_absorbed(q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens, scale, pairs=None):
    """O2: absorbed decode (q~ = W_UK^T q_nope, latent-space attention, one
    W_UV up-projection).  Same arguments and returns as :func:`decode_naive`."""
    return _decode("oracle_decode_absorbed", q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens,
                   scale, pairs)


def decode_latent(q_nope, q_rope, w_uk, ckv, kpe, seqlens, scale, pairs=None):
    """Merged latent of absorbed decode, o[b,h] = sum_n p_n c[b,n] (before the
    W_UV up-projection).  Returns [B,H,dc], or [len(pairs), dc] for a pair list."""
    q_nope = np.ascontiguousarray(q_nope)
    q_rope = np.ascontiguousarray(q_rope)
    w_uk = np.ascontiguousarray(w_uk)
    H, dn, dc = w_uk.shape
    dr = q_rope.shape[-1]
    dt = _code(q_nope)
    for a in (q_rope, w_uk, ckv, kpe):
        if _code(a) != dt:
            raise OracleError("all inputs must share one storage dtype")
    _, csb, csn = _cache_view(ckv, dc)
    _, ksb, ksn = _cache_view(kpe, dr) if dr > 0 else (kpe, 0, 0)
    d = _Dims(B=ckv.shape[0], H=H, dc=dc, dr=dr, dn=dn, dv=1, ckv_sb=csb, ckv_sn=csn,
              kpe_sb=ksb, kpe_sn=ksn, dtype=dt, reserved=0, scale=float(scale))
    seq = np.ascontiguousarray(seqlens, dtype=np.int32)
    if pairs is None:
        n, pp = d.B * d.H, None
    else:
        pp = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
        n = pp.shape[0]
    out = np.zeros((n, dc), dtype=np.float64)
    rc = _load().oracle_decode_latent(ctypes.byref(d), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                                      _base_ptr(ckv), _base_ptr(kpe), _ptr(seq), _ptr(pp), n,
                                      _ptr(out))
    if rc != 0:
        raise OracleError("oracle_decode_latent rejected its arguments")
    return out.reshape(d.B, d.H, dc) if pairs is None else out


def output_proj(x, w):
    """y = x W^T in fp64: x [B, K], w [N, K] (each fp64, fp32 or bf16 bits)."""
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    B, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise OracleError("x and w disagree on the input width")
    y = np.zeros((B, N), dtype=np.float64)
    if _load().oracle_output_proj(B, K, N, _code(x), _ptr(x), _code(w), _ptr(w), _ptr(y)) != 0:
        raise OracleError("oracle_output_proj rejected its arguments")
    return y


def fold_value_output(w_o, w_uv):
    """W_OV [N, H*dc] with W_OV[:, h*dc:(h+1)*dc] = W_O[:, h*dv:(h+1)*dv] W_UV[h],
    from w_o [N, H*dv] and w_uv [H, dv, dc] (one storage type), in fp64."""
    w_o = np.ascontiguousarray(w_o)
    w_uv = np.ascontiguousarray(w_uv)
    if _code(w_o) != _code(w_uv):
        raise OracleError("all inputs must share one storage dtype")
    H, dv, dc = w_uv.shape
    N = w_o.shape[0]
    if w_o.shape[1] != H * dv:
        raise OracleError("W_O width must be heads * d_v")
    out = np.zeros((N, H * dc), dtype=np.float64)
    if _load().oracle_fold_value_output(N, H, dv, dc, _code(w_o), _ptr(w_o), _ptr(w_uv),
                                        _ptr(out)) != 0:
        raise OracleError("oracle_fold_value_output rejected its arguments")
    return out


def absorb_q(q_nope, w_uk):
    """q~[b,h,:] = W_UK[h]^T q_nope[b,h,:] in fp64.  q_nope [B,H,dn], w_uk [H,dn,dc]."""
    q_nope = np.ascontiguousarray(q_nope)
    w_uk = np.ascontiguousarray(w_uk)
    if _code(q_nope) != _code(w_uk):
        raise OracleError("all inputs must share one storage dtype")
    B, H, dn = q_nope.shape
    dc = w_uk.shape[2]
    d = _Dims(B=B, H=H, dc=dc, dr=0, dn=dn, dv=1, dtype=_code(q_nope), scale=1.0)
    out = np.zeros((B, H, dc), dtype=np.float64)
    if _load().oracle_absorb_q(ctypes.byref(d), _ptr(q_nope), _ptr(w_uk), _ptr(out)) != 0:
        raise OracleError("oracle_absorb_q rejected its arguments")
    return out


def _prefill(fname, q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens, scale, rows):
    q_nope = np.ascontiguousarray(q_nope)
    q_rope = np.ascontiguousarray(q_rope)
    w_uk = np.ascontiguousarray(w_uk)
    w_uv = np.ascontiguousarray(w_uv)
    T = q_nope.shape[1]
    d = _dims(q_nope, q_rope, w_uk, w_uv, ckv, kpe, scale, 2)
    seq = np.ascontiguousarray(seqlens, dtype=np.int32)
    rr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
    out = np.zeros((rr.shape[0], d.H, d.dv), dtype=np.float64)
    rc = getattr(_load(), fname)(ctypes.byref(d), T, _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                                 _ptr(w_uv), _base_ptr(ckv), _base_ptr(kpe), _ptr(seq),
                                 _ptr(rr), rr.shape[0], _ptr(out))
    if rc != 0:
        raise OracleError(f"{fname} rejected its arguments")
    return out


def prefill_naive(q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens, scale, rows):
    """O3: naive causal prefill for selected query rows.

    q_nope [B,T,H,dn], q_rope [B,T,H,dr]; query t of sequence b sits at
    position seqlens[b] - T + t and sees cached rows up to and including it
    (none, giving a zero row, when that position is negative).
    rows = [(b, t), ...]; returns [len(rows), H, dv].
    """
    return _prefill("oracle_prefill_naive", q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens,
                    scale, rows)


def prefill_absorbed(q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens, scale, rows):
    """O5: absorbed causal prefill (each query row through the absorbed decode
    definition over its causal prefix).  Same arguments and result as
    :func:`prefill_naive`."""
    return _prefill("oracle_prefill_absorbed", q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens,
                    scale, rows)


def rope(x, pos, base=10000.0):
    """Rotary embedding at position pos (fp64) of every d_r-vector along the
    last axis of x (x may hold several vectors, e.g. one per head)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    dr = x.shape[-1]
    if dr % 2:
        raise OracleError("rotary width must be even")
    xs, os_ = x.reshape(-1, dr), out.reshape(-1, dr)
    for i in range(xs.shape[0]):
        _load().oracle_rope(dr, _ptr(xs[i]), float(pos), float(base), _ptr(os_[i]))
    return out


def cache_rows(h, w_dkv, w_kr, positions, base=10000.0):
    """New cache rows for one token per sequence: c = W_DKV h and the rotated
    decoupled key k^R = RoPE_pos(W_KR h).  h [B, d_model], W_DKV [d_c, d_model],
    W_KR [d_r, d_model]; returns (c [B, d_c], k^R [B, d_r]) in fp64."""
    h = np.ascontiguousarray(h)
    w_dkv = np.ascontiguousarray(w_dkv)
    w_kr = np.ascontiguousarray(w_kr)
    dt = _code(h)
    if _code(w_dkv) != dt or _code(w_kr) != dt:
        raise OracleError("all inputs must share one storage dtype")
    B, d_model = h.shape
    dc, dr = w_dkv.shape[0], w_kr.shape[0]
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    c = np.zeros((B, dc), dtype=np.float64)
    kr = np.zeros((B, dr), dtype=np.float64)
    rc = _load().oracle_cache_rows(B, d_model, dc, dr, dt, _ptr(h), _ptr(w_dkv), _ptr(w_kr),
                                   _ptr(pos), float(base), _ptr(c), _ptr(kr))
    if rc != 0:
        raise OracleError("oracle_cache_rows rejected its arguments")
    return c, kr


def kv_cache_bytes(n_layers, batch, seq_len, d_c=512, d_r=64, bytes_per_elem=2) -> int:
    """O4: latent KV-cache bytes = layers * batch * seq * (d_c + d_r) * bytes."""
    return int(_load().oracle_kv_cache_bytes(n_layers, batch, seq_len, d_c, d_r, bytes_per_elem))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))
