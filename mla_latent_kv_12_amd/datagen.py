"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and stores them (fp32, or bf16 bit
patterns rounded to nearest-even); it performs none of the attention
arithmetic.  Both the HIP path and the fp64 oracle consume exactly the
arrays made here.

Recipe (all draws from ``numpy.random.default_rng(seed)``, standard normals
in float32, scaled where a standard deviation is given):
  decode:  q_nope [B,H,dn], q_rope [B,H,dr], W_UK [H,dn,dc] (std 1/sqrt(dc)),
           W_UV [H,dv,dc] (std 1/sqrt(dc)), the cache rows [B,Nmax,dc+dr]
           sequence by sequence, then (ragged workloads only) the lengths
           uniform in [1, Nmax].
  prefill: q_nope [B,T,H,dn], q_rope [B,T,H,dr], W_UK, W_UV, then
           x [B,T,d_model] ~ N(0,1) and W_DKV [dc,d_model] (std
           1/sqrt(d_model)); the latent rows c = W_DKV x come from a callable
           the caller supplies (the tests pass the fp64 oracle's cache-row
           producer), then are stored; then the decoupled RoPE keys k^R
           [B,T,dr] ~ N(0,1).  Queries' RoPE channels and k^R are taken as already
           rotated: a rotation maps i.i.d. standard normals to i.i.d. standard
           normals, so the rotated values are drawn directly.
  chunk:   (a chunk of T new queries over a cached context, for the absorbed
           prefill) q_nope [B,T,H,dn], q_rope [B,T,H,dr], W_UK, W_UV as for
           decode, the cache rows [B,Nmax,dc+dr] ~ N(0,1) sequence by
           sequence, then (ragged workloads only) the lengths uniform in
           [T, Nmax].
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

SEED_BASE = 20260000


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bfloat16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class DecodeCase:
    name: str
    dtype: str            # "f32" or "bf16" (storage type of every tensor)
    B: int
    H: int
    dc: int
    dr: int
    dn: int
    dv: int
    n_max: int
    scale: float
    q_nope: np.ndarray    # [B,H,dn]
    q_rope: np.ndarray    # [B,H,dr]
    w_uk: np.ndarray      # [H,dn,dc]
    w_uv: np.ndarray      # [H,dv,dc]
    cache: np.ndarray     # [B,n_max,dc+dr]: latent c then RoPE key
    seqlens: np.ndarray   # int32 [B]

    @property
    def ckv(self) -> np.ndarray:
        return self.cache[:, :, : self.dc]

    @property
    def kpe(self) -> np.ndarray:
        return self.cache[:, :, self.dc:]


@dataclasses.dataclass
class PrefillCase:
    name: str
    dtype: str
    B: int
    T: int
    H: int
    dc: int
    dr: int
    dn: int
    dv: int
    scale: float
    q_nope: np.ndarray    # [B,T,H,dn]
    q_rope: np.ndarray    # [B,T,H,dr]
    w_uk: np.ndarray
    w_uv: np.ndarray
    cache: np.ndarray     # [B,N,dc+dr] (N = T for a whole prompt)
    seqlens: np.ndarray   # int32 [B]; the T queries are the last T of L_b rows

    @property
    def ckv(self) -> np.ndarray:
        return self.cache[:, :, : self.dc]

    @property
    def kpe(self) -> np.ndarray:
        return self.cache[:, :, self.dc:]


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _normal(rng, shape, std=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def make_decode_case(*, B, H, dc, dr, dn, dv, n_max, dtype="bf16", seed=SEED_BASE,
                     seqlens=None, ragged=False, scale=None, w_std=None, name="custom"):
    """Draw one decode workload.  ``seqlens`` None -> every sequence full
    (n_max) unless ``ragged`` (then uniform integers in [1, n_max])."""
    rng = np.random.default_rng(seed)
    w_std = 1.0 / math.sqrt(dc) if w_std is None else w_std
    q_nope = _store(_normal(rng, (B, H, dn)), dtype)
    q_rope = _store(_normal(rng, (B, H, dr)), dtype)
    w_uk = _store(_normal(rng, (H, dn, dc), w_std), dtype)
    w_uv = _store(_normal(rng, (H, dv, dc), w_std), dtype)
    width = dc + dr
    cache = np.empty((B, n_max, width), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for b in range(B):  # sequence by sequence keeps peak host memory low
        cache[b] = _store(_normal(rng, (n_max, width)), dtype)
    if seqlens is None:
        if ragged:
            seqlens = rng.integers(1, n_max + 1, size=B)
        else:
            seqlens = np.full(B, n_max)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(dn + dr)
    return DecodeCase(name, dtype, B, H, dc, dr, dn, dv, n_max, float(scale), q_nope, q_rope,
                      w_uk, w_uv, cache, seqlens)


def make_prefill_case(*, B, T, H, dc, dr, dn, dv, d_model, latents, dtype="bf16",
                      seed=SEED_BASE, scale=None, name="custom"):
    """Draw one causal-prefill workload.  The latent rows c = W_DKV x are the
    caller's to compute (this module only draws random numbers):
    ``latents(x_b, w_dkv)`` returns them in fp64, [T, dc], from sequence b's
    stored hidden states x_b [T, d_model] and the stored W_DKV [dc, d_model];
    they are rounded to the storage type here.  Draw order: q_nope, q_rope,
    W_UK, W_UV, x, W_DKV, then the RoPE keys."""
    rng = np.random.default_rng(seed)
    w_std = 1.0 / math.sqrt(dc)
    q_nope = _store(_normal(rng, (B, T, H, dn)), dtype)
    q_rope = _store(_normal(rng, (B, T, H, dr)), dtype)
    w_uk = _store(_normal(rng, (H, dn, dc), w_std), dtype)
    w_uv = _store(_normal(rng, (H, dv, dc), w_std), dtype)
    x = _store(_normal(rng, (B, T, d_model)), dtype)
    w_dkv = _store(_normal(rng, (dc, d_model), 1.0 / math.sqrt(d_model)), dtype)
    cache = np.empty((B, T, dc + dr), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for b in range(B):
        lat = np.asarray(latents(x[b], w_dkv), dtype=np.float64)
        if lat.shape != (T, dc):
            raise ValueError(f"latents() returned shape {lat.shape}, expected {(T, dc)}")
        cache[b, :, :dc] = _store(lat.astype(np.float32), dtype)
    cache[:, :, dc:] = _store(_normal(rng, (B, T, dr)), dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(dn + dr)
    return PrefillCase(name, dtype, B, T, H, dc, dr, dn, dv, float(scale), q_nope, q_rope,
                       w_uk, w_uv, cache, np.full(B, T, dtype=np.int32))


def make_chunk_case(*, B, T, H, dc, dr, dn, dv, n_max, dtype="bf16", seed=SEED_BASE,
                    seqlens=None, ragged=False, scale=None, name="custom"):
    """T new queries per sequence over a cached context of up to n_max rows
    (the queries are the last T of the L_b cached rows).  ``seqlens`` None ->
    every sequence full (n_max) unless ``ragged`` (uniform in [T, n_max])."""
    rng = np.random.default_rng(seed)
    w_std = 1.0 / math.sqrt(dc)
    q_nope = _store(_normal(rng, (B, T, H, dn)), dtype)
    q_rope = _store(_normal(rng, (B, T, H, dr)), dtype)
    w_uk = _store(_normal(rng, (H, dn, dc), w_std), dtype)
    w_uv = _store(_normal(rng, (H, dv, dc), w_std), dtype)
    width = dc + dr
    cache = np.empty((B, n_max, width), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for b in range(B):
        cache[b] = _store(_normal(rng, (n_max, width)), dtype)
    if seqlens is None:
        seqlens = rng.integers(T, n_max + 1, size=B) if ragged else np.full(B, n_max)
    if scale is None:
        scale = 1.0 / math.sqrt(dn + dr)
    return PrefillCase(name, dtype, B, T, H, dc, dr, dn, dv, float(scale), q_nope, q_rope,
                       w_uk, w_uv, cache, np.asarray(seqlens, dtype=np.int32))


@dataclasses.dataclass
class AppendCase:
    """One new token per sequence: hidden states and the two producer weights."""
    name: str
    dtype: str
    B: int
    d_model: int
    dc: int
    dr: int
    h: np.ndarray       # [B, d_model]
    w_dkv: np.ndarray   # [dc, d_model]
    w_kr: np.ndarray    # [dr, d_model]


def make_append_case(*, B, d_model, dc, dr, dtype="bf16", seed=SEED_BASE, name="custom"):
    """h ~ N(0, 1); W_DKV, W_KR ~ N(0, std 1/sqrt(d_model)), so the new latent
    and key entries are of unit scale.  Draw order: h, W_DKV, W_KR."""
    rng = np.random.default_rng(seed)
    w_std = 1.0 / math.sqrt(d_model)
    h = _store(_normal(rng, (B, d_model)), dtype)
    w_dkv = _store(_normal(rng, (dc, d_model), w_std), dtype)
    w_kr = _store(_normal(rng, (dr, d_model), w_std), dtype)
    return AppendCase(name, dtype, B, d_model, dc, dr, h, w_dkv, w_kr)


# The named workloads: name -> (kind, seed offset, keyword arguments).  The
# seed of a workload is SEED_BASE + its offset.
WORKLOADS = {
    "tiny-f32": ("decode", 0, dict(name="tiny-f32 B1 H4 dc64 dr16 L128", dtype="f32", B=1, H=4,
                                   dc=64, dr=16, dn=32, dv=32, n_max=128)),
    "v3-4k": ("decode", 1, dict(name="V3 bf16 B1 L4096", dtype="bf16", B=1, H=128, dc=512, dr=64,
                                dn=128, dv=128, n_max=4096)),
    "v3-ragged": ("decode", 2, dict(name="V3 bf16 B32 ragged L~U[1,8192]", dtype="bf16", B=32,
                                    H=128, dc=512, dr=64, dn=128, dv=128, n_max=8192,
                                    ragged=True)),
    "v3-128k": ("decode", 3, dict(name="V3 bf16 B8 L131072", dtype="bf16", B=8, H=128, dc=512,
                                  dr=64, dn=128, dv=128, n_max=131072)),
    "v3-append": ("append", 5, dict(name="V3 bf16 cache append B8 d_model 7168", dtype="bf16",
                                    B=8, d_model=7168, dc=512, dr=64)),
    "v3-prefill-4k": ("prefill", 4, dict(name="V3 bf16 causal prefill B1 T4096", dtype="bf16",
                                         B=1, T=4096, H=128, dc=512, dr=64, dn=128, dv=128,
                                         d_model=7168)),
    "v3-chunk-32k": ("chunk", 6, dict(name="V3 bf16 absorbed prefill B4 T64 over L32768",
                                      dtype="bf16", B=4, T=64, H=128, dc=512, dr=64, dn=128,
                                      dv=128, n_max=32768)),
}


def make_workload(name: str, seed: int | None = None, latents=None):
    """The named workload; prefill workloads need ``latents`` (see
    :func:`make_prefill_case`)."""
    kind, offset, kw = WORKLOADS[name]
    seed = SEED_BASE + offset if seed is None else seed
    if kind == "decode":
        return make_decode_case(seed=seed, **kw)
    if kind == "append":
        return make_append_case(seed=seed, **kw)
    if kind == "chunk":
        return make_chunk_case(seed=seed, **kw)
    if latents is None:
        raise ValueError(f"workload {name} needs latents(x, w_dkv) for c = W_DKV x")
    return make_prefill_case(seed=seed, latents=latents, **kw)
