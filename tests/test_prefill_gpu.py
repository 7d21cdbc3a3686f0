"""GPU parity of mla_prefill_naive (naive causal prefill) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import mla_latent_kv_12_amd as mla
import oracle
from gpu_util import (assert_close, oracle_latents, run_decode, run_prefill_naive, say, to_device,
                      to_host_f64)
from mla_latent_kv_12_amd import datagen

pytestmark = pytest.mark.gpu


def prefill_tensors(case):
    dt = case.dtype
    cache = to_device(case.cache, dt)
    return dict(q_nope=to_device(case.q_nope, dt), q_rope=to_device(case.q_rope, dt),
                w_uk=to_device(case.w_uk, dt), w_uv=to_device(case.w_uv, dt), cache=cache,
                ckv=cache[:, :, : case.dc], kpe=cache[:, :, case.dc:],
                seqlens=torch.from_numpy(case.seqlens.astype(np.int32)).cuda())


def run_prefill(case, t=None, out_dtype=None):
    t = t or prefill_tensors(case)
    odt = {None: None, "f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    out = run_prefill_naive(t, case.scale, out_dtype=odt)
    return to_host_f64(out)


def make_case(B, T, L, H, dtype, seed, dims=None):
    """Prefill workload with L_b >= T cached rows (the last T are the queries)."""
    d = dims or dict(dc=512, dr=64, dn=128, dv=128)
    n_max = max(L)
    base = datagen.make_prefill_case(B=B, T=n_max, H=H, d_model=64, dtype=dtype, seed=seed,
                                     latents=oracle_latents, **d)
    # keep the first T query rows; seqlens may exceed T (bottom-right alignment)
    base.q_nope = np.ascontiguousarray(base.q_nope[:, :T])
    base.q_rope = np.ascontiguousarray(base.q_rope[:, :T])
    base.T = T
    base.seqlens = np.asarray(L, dtype=np.int32)
    return base


def oracle_rows(case, rows, heads=None):
    """Naive oracle on (b, t) rows, optionally restricted to a head subset."""
    hs = list(range(case.H)) if heads is None else list(heads)
    out = oracle.prefill_naive(case.q_nope[:, :, hs], case.q_rope[:, :, hs], case.w_uk[hs],
                               case.w_uv[hs], case.ckv, case.kpe, case.seqlens, case.scale, rows)
    return out


def absorbed_rows(case, rows):
    """Prefill row t == absorbed decode over the first pos_t + 1 rows (an identity
    the oracle's own tests pin); much cheaper than the naive form at full size."""
    res = []
    for b, t in rows:
        pos = int(case.seqlens[b]) - case.T + t
        out, _ = oracle.decode_absorbed(case.q_nope[b:b + 1, t], case.q_rope[b:b + 1, t],
                                        case.w_uk, case.w_uv, case.ckv[b:b + 1], case.kpe[b:b + 1],
                                        [pos + 1], case.scale)
        res.append(out[0])
    return np.stack(res)


def test_prefill_f32_small_all_rows():
    say("prefill f32 small")
    case = make_case(2, 9, [9, 13], 3, "f32", 1201, dims=dict(dc=64, dr=16, dn=32, dv=32))
    out = run_prefill(case)
    rows = [(b, t) for b in range(2) for t in range(9)]
    ref = oracle_rows(case, rows)
    got = np.stack([out[b, t] for b, t in rows])
    assert_close(got, ref, "f32", "all rows")


@pytest.mark.parametrize("T,L", [(1, [1, 1]), (37, [37, 50]), (130, [130, 200]), (64, [64, 64])])
def test_prefill_bf16_against_naive(T, L):
    say(f"prefill bf16 T={T} L={L} H=4")
    case = make_case(2, T, L, 4, "bf16", 1300 + T)
    out = run_prefill(case, out_dtype="f32")
    rows = [(b, t) for b in range(2) for t in sorted({0, T // 2, T - 1, min(T - 1, 31), min(T - 1, 33)})]
    ref = oracle_rows(case, rows)
    got = np.stack([out[b, t] for b, t in rows])
    assert_close(got, ref, "bf16", "sampled rows vs naive oracle")
    rows_all = [(b, t) for b in range(2) for t in range(T)]
    got = np.stack([out[b, t] for b, t in rows_all])
    assert_close(got, absorbed_rows(case, rows_all), "bf16", "all rows vs absorbed identity")


@pytest.mark.parametrize("B,T,L,H", [
    (1, 40, [50], 3),               # 3 (sequence, head) pairs: plain block order
    (3, 300, [300, 310, 555], 8),   # two query blocks, a ragged tail, keys beyond T
    (2, 257, [257, 700], 4),        # one query past a 256-query block
    (1, 70, [2200], 24),            # 3 heads per XCD, 9 token blocks: a partial block group
])
def test_prefill_bf16_block_mapping_and_ragged(B, T, L, H):
    say(f"prefill bf16 B={B} T={T} L={L} H={H}")
    case = make_case(B, T, L, H, "bf16", 1500 + T + H)
    out = run_prefill(case, out_dtype="f32")
    rows = [(b, t) for b in range(B) for t in sorted({0, 1, T // 3, T - 2, T - 1, min(T - 1, 255), min(T - 1, 256)})]
    got = np.stack([out[b, t] for b, t in rows])
    assert_close(got, absorbed_rows(case, rows), "bf16", "sampled rows vs absorbed identity")
    ref = oracle_rows(case, rows[:4])
    assert_close(np.stack([out[b, t] for b, t in rows[:4]]), ref, "bf16", "4 rows vs naive oracle")


def test_prefill_single_token_equals_decode():
    say("prefill T=1 vs decode (bf16, 128 heads)")
    case = make_case(3, 1, [200, 33, 1], 128, "bf16", 1401)
    pre = run_prefill(case, out_dtype="f32")[:, 0]
    dcase = datagen.DecodeCase("p11", "bf16", 3, 128, 512, 64, 128, 128, case.cache.shape[1],
                               case.scale, np.ascontiguousarray(case.q_nope[:, 0]),
                               np.ascontiguousarray(case.q_rope[:, 0]), case.w_uk, case.w_uv,
                               case.cache, case.seqlens)
    dec = to_host_f64(run_decode(dcase, out_dtype="f32"))
    assert_close(pre, dec, "bf16", "prefill(T=1) vs decode")


def test_prefill_v3_4k_full():
    case = datagen.make_workload("v3-prefill-4k", latents=oracle_latents)
    say(f"V3 prefill T=4096 H=128 seed={datagen.SEED_BASE + 4}")
    t = prefill_tensors(case)
    out16 = run_prefill(case, t)              # the benchmark's launch: bf16 output
    out = run_prefill(case, t, out_dtype="f32")
    # the bf16 output is the fp32 result rounded to nearest-even, bit for bit
    assert np.array_equal(out16, torch.from_numpy(out).to(torch.bfloat16).double().numpy())
    rows = [(0, t) for t in (0, 1, 31, 32, 2047, 4095)]
    heads = [0, 77, 127]
    ref = oracle_rows(case, rows, heads=heads)
    got = np.stack([out[0, t][heads] for _, t in rows])
    assert_close(got, ref, "bf16", "naive oracle, 6 rows x 3 heads")
    rng = np.random.default_rng(4)
    rows2 = [(0, int(t)) for t in rng.integers(0, 4096, 24)]
    got2 = np.stack([out[b, t] for b, t in rows2])
    assert_close(got2, absorbed_rows(case, rows2), "bf16", "24 rows x 128 heads, absorbed identity")
