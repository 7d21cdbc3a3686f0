"""GPU parity of the query-side rotary embedding (q_rope_base > 1): decode,
naive prefill and absorbed prefill rotate q_rope at each query's own position
before attending.  The expected values rotate the stored q_rope with the
oracle's RoPE (fp64), round the rotated vector to the storage type as the
library's contract states (it replaces q_rope, an MFMA operand in bf16), and
run the oracle on the widened inputs."""
import numpy as np
import pytest
import torch

import mla_latent_kv_12_amd as mla
import oracle
from gpu_util import assert_close, say, to_device, to_host_f64
from mla_latent_kv_12_amd import datagen
from mla_latent_kv_12_amd.tensors import decode_tensors

pytestmark = pytest.mark.gpu

V3 = dict(dc=512, dr=64, dn=128, dv=128)
TINY = dict(dc=64, dr=16, dn=32, dv=32)
BASE = 10000.0


def wide(a, dtype):
    return (datagen.bf16_to_f32(a) if dtype == "bf16" else a).astype(np.float64)


def rotated_queries(q_rope, positions, base, dtype):
    """q_rope [..., H, dr] (widened to fp64) rotated at positions[...] by the
    oracle and rounded to the storage type; rows with a negative position are
    left as they are (they see no key)."""
    out = q_rope.copy()
    flat = out.reshape(-1, out.shape[-2], out.shape[-1])     # [rows, H, dr]
    pos = np.asarray(positions).reshape(-1)
    for r, p in enumerate(pos):
        if p >= 0:
            flat[r] = oracle.rope(flat[r], float(p), base)
    f32 = out.astype(np.float32)
    if dtype == "bf16":
        return datagen.bf16_to_f32(datagen.bf16_bits(f32)).astype(np.float64)
    return f32.astype(np.float64)


def widened(case):
    w = {k: wide(getattr(case, k), case.dtype) for k in ("q_nope", "q_rope", "w_uk", "w_uv")}
    cache = wide(case.cache, case.dtype)
    return w, cache


@pytest.mark.parametrize("dtype,dims,H,L", [
    ("f32", TINY, 4, [128, 37, 1]),
    ("bf16", V3, 128, [300, 77, 1]),
    ("bf16", V3, 128, [131072 // 16, 4000, 2]),   # positions up to 8191
])
def test_decode_rotates_queries_at_their_position(dtype, dims, H, L):
    say(f"decode with q rotation {dtype} H={H} L={L}")
    case = datagen.make_decode_case(B=len(L), H=H, n_max=max(L), dtype=dtype, seed=3100 + L[0],
                                    seqlens=L, **dims)
    t = decode_tensors(case)
    out = mla.decode(t["q_nope"], t["q_rope"], t["w_uk"], t["w_uv"], t["ckv_cache"],
                     t["kpe_cache"], t["seqlens"], softmax_scale=case.scale,
                     out_dtype=torch.float32, q_rope_base=BASE)
    torch.cuda.synchronize()
    w, cache = widened(case)
    qr = rotated_queries(w["q_rope"], case.seqlens - 1, BASE, dtype)
    ref, _ = oracle.decode_absorbed(w["q_nope"], qr, w["w_uk"], w["w_uv"], cache[:, :, :case.dc],
                                    cache[:, :, case.dc:], case.seqlens, case.scale)
    assert_close(to_host_f64(out), ref, dtype, "rotated at L-1")
    # position 0 (a sequence of length 1) is the identity: same bits as no rotation
    plain = mla.decode(t["q_nope"], t["q_rope"], t["w_uk"], t["w_uv"], t["ckv_cache"],
                       t["kpe_cache"], t["seqlens"], softmax_scale=case.scale,
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    last = len(L) - 1 if L[-1] == 1 else None
    if last is not None:
        assert np.array_equal(to_host_f64(out)[last], to_host_f64(plain)[last])


@pytest.mark.parametrize("path", ["naive", "absorbed"])
def test_prefill_rotates_queries_at_their_position(path):
    say(f"{path} prefill with q rotation (bf16, H=128, T=24, L=[24, 90])")
    case = datagen.make_chunk_case(B=2, T=24, H=128, n_max=90, seqlens=[24, 90], dtype="bf16",
                                   seed=3200, **V3)
    dt = case.dtype
    cache = to_device(case.cache, dt)
    args = (to_device(case.q_nope, dt), to_device(case.q_rope, dt), to_device(case.w_uk, dt),
            to_device(case.w_uv, dt), cache[:, :, :case.dc], cache[:, :, case.dc:],
            torch.from_numpy(case.seqlens).cuda())
    fn = mla.prefill_naive if path == "naive" else mla.prefill_absorbed
    out = to_host_f64(fn(*args, softmax_scale=case.scale, out_dtype=torch.float32,
                         q_rope_base=BASE))
    torch.cuda.synchronize()
    w, wc = widened(case)
    pos = case.seqlens[:, None] - case.T + np.arange(case.T)[None, :]
    qr = rotated_queries(w["q_rope"], pos, BASE, "bf16")
    rows = [(b, q) for b in range(2) for q in range(case.T)]
    ref = oracle.prefill_absorbed(w["q_nope"], qr, w["w_uk"], w["w_uv"], wc[:, :, :case.dc],
                                  wc[:, :, case.dc:], case.seqlens, case.scale, rows)
    assert_close(out.reshape(-1, case.H, case.dv), ref, "bf16", "all rows, rotated at L-T+t")


def test_append_then_decode_with_rotation_matches_oracle():
    """The whole positional path on the GPU: every cache row written by the
    producer (key rotated at its row), then decode rotating the query at
    L - 1; against the oracle's producer and decode on the same stored data."""
    B, H, L, d_model = 2, 128, 96, 256
    say(f"append {L} rows then decode with q rotation (bf16, H={H}, d_model={d_model})")
    dec = datagen.make_decode_case(B=B, H=H, n_max=L, dtype="bf16", seed=3300,
                                   seqlens=[L, 50], **V3)
    app = datagen.make_append_case(B=B * L, d_model=d_model, dc=512, dr=64, dtype="bf16",
                                   seed=3301)
    t = decode_tensors(dec)
    t["cache"].fill_(float("nan"))                       # every row must come from the producer
    h = to_device(app.h, "bf16").view(B, L, d_model)
    w_dkv, w_kr = to_device(app.w_dkv, "bf16"), to_device(app.w_kr, "bf16")
    for n in range(L):
        pos = torch.full((B,), n, dtype=torch.int32, device="cuda")
        mla.cache_append(h[:, n].contiguous(), w_dkv, w_kr, pos, t["ckv_cache"], t["kpe_cache"],
                         rope_base=BASE)
    out = mla.decode(t["q_nope"], t["q_rope"], t["w_uk"], t["w_uv"], t["ckv_cache"],
                     t["kpe_cache"], t["seqlens"], softmax_scale=dec.scale,
                     out_dtype=torch.float32, q_rope_base=BASE)
    torch.cuda.synchronize()
    # oracle: the producer's rows in fp64, rounded to bf16 as the cache stores them
    positions = np.tile(np.arange(L), B)
    c, kr = oracle.cache_rows(app.h, app.w_dkv, app.w_kr, positions, BASE)
    rows = np.concatenate([c, kr], axis=1).reshape(B, L, -1)
    cache = wide(datagen.bf16_bits(rows.astype(np.float32)), "bf16")
    w = {k: wide(getattr(dec, k), "bf16") for k in ("q_nope", "q_rope", "w_uk", "w_uv")}
    qr = rotated_queries(w["q_rope"], dec.seqlens - 1, BASE, "bf16")
    ref, _ = oracle.decode_absorbed(w["q_nope"], qr, w["w_uk"], w["w_uv"], cache[:, :, :512],
                                    cache[:, :, 512:], dec.seqlens, dec.scale)
    assert_close(to_host_f64(out), ref, "bf16", "producer + rotated decode")
