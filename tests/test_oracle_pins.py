"""Pins of the fp64 oracle against what the pages and the mathematics fix.

These run on the CPU only.  Each check is chosen so that a plausible mistake
in the oracle (a dropped RoPE term, a transposed W_UK, a wrong scale, an
off-by-one in the cached length or the causal mask, a broken softmax) fails
at least one of them; the "mutation" tests at the end demonstrate that.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_12_amd import datagen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cache_tables.json")


def _rand_case(rng, B, H, dc, dr, dn, dv, N):
    q_nope = rng.standard_normal((B, H, dn))
    q_rope = rng.standard_normal((B, H, dr))
    w_uk = rng.standard_normal((H, dn, dc)) / math.sqrt(dc)
    w_uv = rng.standard_normal((H, dv, dc)) / math.sqrt(dc)
    cache = rng.standard_normal((B, N, dc + dr))
    return q_nope, q_rope, w_uk, w_uv, cache


def _sdpa_decode(q_nope, q_rope, w_uk, w_uv, cache, seqlens, scale):
    """Independent reference: materialise K and V per head (section 2 of the
    distaisys deep-dive), then torch's fp64 scaled-dot-product attention."""
    B, H, dn = q_nope.shape
    dc = w_uk.shape[2]
    out = np.zeros((B, H, w_uv.shape[1]))
    for b in range(B):
        L = int(seqlens[b])
        if L == 0:
            continue
        c = torch.from_numpy(cache[b, :L, :dc])
        kr = torch.from_numpy(cache[b, :L, dc:])
        for h in range(H):
            k = torch.cat([c @ torch.from_numpy(w_uk[h]).T, kr], dim=1)   # [L, dn+dr]
            v = c @ torch.from_numpy(w_uv[h]).T                          # [L, dv]
            q = torch.from_numpy(np.concatenate([q_nope[b, h], q_rope[b, h]]))[None, None]
            o = torch.nn.functional.scaled_dot_product_attention(
                q, k[None], v[None], scale=scale)
            out[b, h] = o[0, 0].numpy()
    return out


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------
# P8: cache arithmetic reproduces every table printed on the pages
# --------------------------------------------------------------------------

def test_cache_bytes_eyestech_telemetry():
    g = json.load(open(GOLDEN))["eyestech_telemetry"]
    for row in g["rows"]:
        width = row["elems_per_token"]
        dc, dr = row.get("d_c", width), row.get("d_r", 0)
        assert dc + dr == width
        for s, gib in zip(g["seq_lens"], row["gib"]):
            nbytes = oracle.kv_cache_bytes(g["n_layers"], g["batch"], s, dc, dr, g["bytes_per_elem"])
            assert round(nbytes / 2**30, 2) == pytest.approx(gib, abs=1e-9), (row["arch"], s)
    mla = oracle.kv_cache_bytes(60, 8, 131072, 512, 64, 2)
    mha32 = oracle.kv_cache_bytes(60, 8, 131072, 8192, 0, 2)
    assert round(100 * (1 - mla / mha32), 2) == g["mla_reduction_vs_mha32_percent"]


def test_cache_bytes_mla_from_scratch_table():
    g = json.load(open(GOLDEN))["mla_from_scratch_table"]
    mha = oracle.kv_cache_bytes(g["n_layers"], g["batch"], g["seq_len"], 8192, 0, 2)
    for row in g["rows"]:
        dc, dr = row.get("d_c", row["elems"]), row.get("d_r", 0)
        nbytes = oracle.kv_cache_bytes(g["n_layers"], g["batch"], g["seq_len"], dc, dr,
                                       g["bytes_per_elem"])
        assert round(nbytes / 2**30, 2) == row["gib"], row["variant"]
        assert round(mha / nbytes, 2) == row["ratio"], row["variant"]
    with_rope = oracle.kv_cache_bytes(60, 1, 131072, 512, 64, 2)
    without = oracle.kv_cache_bytes(60, 1, 131072, 512, 0, 2)
    assert round((with_rope - without) / 2**30, 2) == g["rope_cost_gib"]
    # 576 elements per token per layer
    assert oracle.kv_cache_bytes(1, 1, 1, 512, 64, 1) == 576


def test_cache_elems_songhuiming_99_tokens():
    g = json.load(open(GOLDEN))["songhuiming_99_tokens"]
    mla = oracle.kv_cache_bytes(g["n_layers"], 1, g["seq_len"], g["d_c"], 0, 1)
    mha = oracle.kv_cache_bytes(g["n_layers"], 1, g["seq_len"], g["mha_width"], 0, 1)
    assert mla == g["mla_elems"] and mha == g["mha_elems"]
    assert round(2 * mla / 2**20, 1) == g["mla_mib_approx"]
    assert round(2 * mha / 2**20) == g["mha_mib_approx"]


# --------------------------------------------------------------------------
# O1 (naive) against an independent library attention
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dc,dr,L", [(16, 0, 1), (16, 16, 7), (64, 16, 128), (64, 64, 33),
                                     (512, 64, 7)])
def test_naive_matches_torch_sdpa(dc, dr, L):
    rng = np.random.default_rng(11 + dc + dr + L)
    B, H, dn, dv = 2, 3, 8, 6
    q_nope, q_rope, w_uk, w_uv, cache = _rand_case(rng, B, H, dc, dr, dn, dv, L + 3)
    seqlens = np.array([L, max(L - 1, 0)], dtype=np.int32)
    scale = 1.0 / math.sqrt(dn + dr)
    out, psum = oracle.decode_naive(q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc],
                                    cache[:, :, dc:], seqlens, scale)
    ref = _sdpa_decode(q_nope, q_rope, w_uk, w_uv, cache, seqlens, scale)
    assert np.max(np.abs(out - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


# --------------------------------------------------------------------------
# P1: absorbed == naive over latent widths x lengths (incl. 1) x RoPE widths
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dc", [16, 64, 512])
@pytest.mark.parametrize("L", [1, 7, 128])
@pytest.mark.parametrize("dr", [0, 16, 64])
def test_absorbed_equals_naive(dc, L, dr):
    rng = np.random.default_rng(1000 * dc + 10 * L + dr)
    B, H, dn, dv = 2, 2, 16, 12
    q_nope, q_rope, w_uk, w_uv, cache = _rand_case(rng, B, H, dc, dr, dn, dv, L)
    seqlens = np.array([L, L], dtype=np.int32)
    scale = 1.0 / math.sqrt(dn + dr)
    args = (q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc], cache[:, :, dc:], seqlens, scale)
    naive, _ = oracle.decode_naive(*args)
    absorbed, _ = oracle.decode_absorbed(*args)
    assert _rel(absorbed, naive) <= 1e-12


# --------------------------------------------------------------------------
# P2: a single cached token -> softmax weight exactly 1 -> out = W_UV c_0
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fn", [oracle.decode_naive, oracle.decode_absorbed])
def test_single_token_selection_exact(fn):
    rng = np.random.default_rng(5)
    B, H, dc, dr, dn, dv = 2, 3, 64, 16, 32, 32
    q_nope, q_rope, w_uk, _, cache = _rand_case(rng, B, H, dc, dr, dn, dv, 4)
    # W_UV[h] row i selects latent channel sel[h][i]: out must be c_0[sel] exactly
    sel = np.stack([rng.permutation(dc)[:dv] for _ in range(H)])
    w_uv = np.zeros((H, dv, dc))
    for h in range(H):
        w_uv[h, np.arange(dv), sel[h]] = 1.0
    seqlens = np.array([1, 1], dtype=np.int32)
    out, psum = fn(q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc], cache[:, :, dc:], seqlens, 0.3)
    for b in range(B):
        for h in range(H):
            assert np.array_equal(out[b, h], cache[b, 0, sel[h]])
    assert np.all(psum == 1.0)


@pytest.mark.parametrize("fn", [oracle.decode_naive, oracle.decode_absorbed])
def test_single_token_random_weights(fn):
    rng = np.random.default_rng(6)
    B, H, dc, dr, dn, dv = 1, 4, 64, 16, 32, 32
    q_nope, q_rope, w_uk, w_uv, cache = _rand_case(rng, B, H, dc, dr, dn, dv, 1)
    out, _ = fn(q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc], cache[:, :, dc:],
                np.array([1], np.int32), 0.25)
    ref = np.einsum("hij,j->hi", w_uv, cache[0, 0, :dc])
    assert _rel(out[0], ref) <= 1e-14


# --------------------------------------------------------------------------
# P3: softmax rows sum to one (directly, and through a constant channel)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("L", [1, 2, 77, 500])
def test_softmax_mass_is_one(L):
    rng = np.random.default_rng(L)
    B, H, dc, dr, dn, dv = 1, 2, 16, 8, 8, 4
    q_nope, q_rope, w_uk, w_uv, cache = _rand_case(rng, B, H, dc, dr, dn, dv, L)
    q_nope *= 5.0  # sharpen the distribution
    cache[:, :, 3] = 1.0
    w_uv[:, 0, :] = 0.0
    w_uv[:, 0, 3] = 1.0
    for fn in (oracle.decode_naive, oracle.decode_absorbed):
        out, psum = fn(q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc], cache[:, :, dc:],
                       np.array([L], np.int32), 0.5)
        assert np.all(np.abs(psum - 1.0) <= 1e-14)
        assert np.all(np.abs(out[:, :, 0] - 1.0) <= 1e-14)


# --------------------------------------------------------------------------
# P4: uniform scores -> plain mean of the up-projected latents
# --------------------------------------------------------------------------

def test_uniform_scores_give_mean():
    rng = np.random.default_rng(9)
    B, H, dc, dr, dn, dv, N = 3, 2, 64, 16, 32, 24, 50
    _, _, w_uk, w_uv, cache = _rand_case(rng, B, H, dc, dr, dn, dv, N)
    q_nope = np.zeros((B, H, dn))
    q_rope = np.zeros((B, H, dr))
    seqlens = np.array([50, 13, 1], dtype=np.int32)
    for fn in (oracle.decode_naive, oracle.decode_absorbed):
        out, _ = fn(q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc], cache[:, :, dc:], seqlens, 1.0)
        for b in range(B):
            mean = cache[b, : seqlens[b], :dc].mean(axis=0)
            ref = w_uv @ mean
            assert _rel(out[b], ref) <= 1e-13


# --------------------------------------------------------------------------
# P5: one dominant token (huge logits, no overflow) -> W_UV c_{n*}
# --------------------------------------------------------------------------

@pytest.mark.parametrize("star", [0, 17, 39])   # first, middle and last cached row
def test_dominant_token_no_overflow(star):
    rng = np.random.default_rng(21)
    B, H, dc, dr, dn, dv, N = 1, 2, 64, 16, 32, 32, 40
    _, _, w_uk, w_uv, cache = _rand_case(rng, B, H, dc, dr, dn, dv, N)
    q_nope = np.zeros((B, H, dn))
    q_rope = np.stack([1e3 * cache[0, star, dc:]] * H)[None]
    for fn in (oracle.decode_naive, oracle.decode_absorbed):
        out, psum = fn(q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc], cache[:, :, dc:],
                       np.array([N], np.int32), 1.0)
        assert np.all(np.isfinite(out)) and np.all(np.abs(psum - 1) < 1e-14)
        ref = w_uv @ cache[0, star, :dc]
        assert _rel(out[0], ref) <= 1e-12


# --------------------------------------------------------------------------
# P6/P7: order independence; padding rows beyond the length are never read
# --------------------------------------------------------------------------

def test_permutation_invariance():
    rng = np.random.default_rng(31)
    B, H, dc, dr, dn, dv, N = 1, 3, 64, 16, 32, 32, 61
    q_nope, q_rope, w_uk, w_uv, cache = _rand_case(rng, B, H, dc, dr, dn, dv, N)
    perm = rng.permutation(N)
    c2 = cache[:, perm]
    args = (q_nope, q_rope, w_uk, w_uv)
    a, _ = oracle.decode_absorbed(*args, cache[:, :, :dc], cache[:, :, dc:], [N], 0.2)
    b, _ = oracle.decode_absorbed(*args, c2[:, :, :dc], c2[:, :, dc:], [N], 0.2)
    assert _rel(a, b) <= 1e-13


@pytest.mark.parametrize("fn", [oracle.decode_naive, oracle.decode_absorbed])
def test_nan_padding_ignored(fn):
    rng = np.random.default_rng(41)
    B, H, dc, dr, dn, dv, N = 2, 2, 16, 8, 8, 8, 30
    q_nope, q_rope, w_uk, w_uv, cache = _rand_case(rng, B, H, dc, dr, dn, dv, N)
    seqlens = np.array([11, 30], dtype=np.int32)
    clean, _ = fn(q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc], cache[:, :, dc:], seqlens, 0.3)
    poisoned = cache.copy()
    poisoned[0, 11:] = np.nan
    dirty, _ = fn(q_nope, q_rope, w_uk, w_uv, poisoned[:, :, :dc], poisoned[:, :, dc:],
                  seqlens, 0.3)
    assert np.array_equal(clean, dirty)


def test_zero_length_gives_zero_output():
    rng = np.random.default_rng(42)
    q_nope, q_rope, w_uk, w_uv, cache = _rand_case(rng, 2, 2, 16, 8, 8, 8, 5)
    out, psum = oracle.decode_absorbed(q_nope, q_rope, w_uk, w_uv, cache[:, :, :16],
                                       cache[:, :, 16:], np.array([0, 5], np.int32), 0.3)
    assert np.all(out[0] == 0.0) and np.all(psum[0] == 0.0) and np.all(psum[1] != 0.0)


def test_pairs_subset_and_thread_count_independence():
    rng = np.random.default_rng(43)
    B, H, dc, dr, dn, dv, N = 3, 5, 64, 16, 16, 16, 40
    q_nope, q_rope, w_uk, w_uv, cache = _rand_case(rng, B, H, dc, dr, dn, dv, N)
    args = (q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc], cache[:, :, dc:], [40, 3, 17], 0.4)
    full, _ = oracle.decode_absorbed(*args)
    pairs = [(2, 4), (0, 0), (1, 3)]
    sub, _ = oracle.decode_absorbed(*args, pairs=pairs)
    for k, (b, h) in enumerate(pairs):
        assert np.array_equal(sub[k], full[b, h])
    n = oracle.max_threads()
    oracle.set_threads(1)
    try:
        single, _ = oracle.decode_absorbed(*args)
    finally:
        oracle.set_threads(n)
    assert np.array_equal(single, full)


def test_bf16_and_f32_storage_widen_exactly():
    rng = np.random.default_rng(44)
    B, H, dc, dr, dn, dv, N = 1, 2, 32, 8, 8, 8, 9
    parts = _rand_case(rng, B, H, dc, dr, dn, dv, N)
    bits = [datagen.bf16_bits(p.astype(np.float32)) for p in parts]
    f32 = [datagen.bf16_to_f32(b) for b in bits]
    f64 = [f.astype(np.float64) for f in f32]
    res = []
    for arrs in (bits, f32, f64):
        q_nope, q_rope, w_uk, w_uv, cache = arrs
        out, _ = oracle.decode_absorbed(q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc],
                                        cache[:, :, dc:], [N], 0.3)
        res.append(out)
    assert np.array_equal(res[0], res[2]) and np.array_equal(res[1], res[2])


# --------------------------------------------------------------------------
# O3: naive causal prefill
# --------------------------------------------------------------------------

def _sdpa_prefill(q_nope, q_rope, w_uk, w_uv, cache, seqlens, scale, b, rows):
    T = q_nope.shape[1]
    H = w_uk.shape[0]
    dc = w_uk.shape[2]
    L = int(seqlens[b])
    c = torch.from_numpy(cache[b, :L, :dc])
    kr = torch.from_numpy(cache[b, :L, dc:])
    # bottom-right aligned causal mask: query t sees keys j <= L - T + t
    t_idx = torch.arange(T)[:, None]
    j_idx = torch.arange(L)[None, :]
    mask = j_idx <= (L - T + t_idx)
    out = np.zeros((len(rows), H, w_uv.shape[1]))
    for h in range(H):
        k = torch.cat([c @ torch.from_numpy(w_uk[h]).T, kr], dim=1)
        v = c @ torch.from_numpy(w_uv[h]).T
        q = torch.from_numpy(np.concatenate([q_nope[b, :, h], q_rope[b, :, h]], axis=1))
        o = torch.nn.functional.scaled_dot_product_attention(
            q[None], k[None], v[None], attn_mask=mask[None], scale=scale)[0]
        out[:, h] = o.numpy()[rows]
    return out


@pytest.mark.parametrize("T,L", [(1, 1), (5, 5), (9, 9), (4, 11), (16, 16)])
def test_prefill_matches_masked_sdpa(T, L):
    rng = np.random.default_rng(100 + T * 7 + L)
    B, H, dc, dr, dn, dv = 1, 3, 32, 8, 16, 16
    q_nope = rng.standard_normal((B, T, H, dn))
    q_rope = rng.standard_normal((B, T, H, dr))
    w_uk = rng.standard_normal((H, dn, dc)) / math.sqrt(dc)
    w_uv = rng.standard_normal((H, dv, dc)) / math.sqrt(dc)
    cache = rng.standard_normal((B, L, dc + dr))
    seqlens = np.array([L], np.int32)
    rows = list(range(T))
    out = oracle.prefill_naive(q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc], cache[:, :, dc:],
                               seqlens, 0.3, [(0, t) for t in rows])
    ref = _sdpa_prefill(q_nope, q_rope, w_uk, w_uv, cache, seqlens, 0.3, 0, rows)
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_prefill_row_equals_decode_prefix():
    """P11 on the oracle: query row t equals a decode over the first pos_t+1 keys."""
    rng = np.random.default_rng(7)
    B, T, H, dc, dr, dn, dv, L = 1, 6, 2, 32, 8, 16, 16, 10
    q_nope = rng.standard_normal((B, T, H, dn))
    q_rope = rng.standard_normal((B, T, H, dr))
    w_uk = rng.standard_normal((H, dn, dc)) / math.sqrt(dc)
    w_uv = rng.standard_normal((H, dv, dc)) / math.sqrt(dc)
    cache = rng.standard_normal((B, L, dc + dr))
    pre = oracle.prefill_naive(q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc], cache[:, :, dc:],
                               [L], 0.3, [(0, t) for t in range(T)])
    for t in range(T):
        dec, _ = oracle.decode_naive(q_nope[:, t], q_rope[:, t], w_uk, w_uv, cache[:, :, :dc],
                                     cache[:, :, dc:], [L - T + t + 1], 0.3)
        assert np.array_equal(pre[t], dec[0])


@pytest.mark.parametrize("T,L", [(3, 9), (6, 4)])
def test_prefill_rows_before_the_cache(T, L):
    """Queries whose position L - T + t is negative (L < T) see no row and give
    exact zeros; the remaining rows still match the masked SDPA reference."""
    rng = np.random.default_rng(200 + 10 * T + L)
    B, H, dc, dr, dn, dv = 1, 2, 24, 8, 16, 12
    q_nope = rng.standard_normal((B, T, H, dn))
    q_rope = rng.standard_normal((B, T, H, dr))
    w_uk = rng.standard_normal((H, dn, dc)) / math.sqrt(dc)
    w_uv = rng.standard_normal((H, dv, dc)) / math.sqrt(dc)
    cache = rng.standard_normal((B, max(L, 1), dc + dr))
    rows = [(0, t) for t in range(T)]
    for fn in (oracle.prefill_naive, oracle.prefill_absorbed):
        out = fn(q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc], cache[:, :, dc:], [L], 0.3, rows)
        first = max(T - L, 0)                      # first query with a non-negative position
        assert np.all(out[:first] == 0.0)
        live = list(range(first, T))
        # the live rows are the last L - (T - T') queries of a prefill with T' = T - first
        ref = _sdpa_prefill(q_nope[:, first:], q_rope[:, first:], w_uk, w_uv, cache,
                            np.array([L], np.int32), 0.3, 0, [t - first for t in live])
        assert np.max(np.abs(out[first:] - ref)) <= 1e-12


# --------------------------------------------------------------------------
# O5: absorbed causal prefill == naive causal prefill
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dc,dr", [(16, 0), (64, 16), (512, 64)])
@pytest.mark.parametrize("T,L", [(1, 1), (4, 4), (5, 13), (7, 3)])
def test_prefill_absorbed_equals_naive(dc, dr, T, L):
    """The associativity behind absorbed decode, for T > 1 causal queries that
    share one latent cache (ragged, L < T included)."""
    rng = np.random.default_rng(3000 + dc + 10 * dr + 100 * T + L)
    B, H, dn, dv = 2, 2, 16, 12
    q_nope = rng.standard_normal((B, T, H, dn))
    q_rope = rng.standard_normal((B, T, H, dr))
    w_uk = rng.standard_normal((H, dn, dc)) / math.sqrt(dc)
    w_uv = rng.standard_normal((H, dv, dc)) / math.sqrt(dc)
    N = max(L, T)
    cache = rng.standard_normal((B, N, dc + dr))
    seqlens = np.array([L, N], np.int32)            # second sequence: its own length
    rows = [(b, t) for b in range(B) for t in range(T)]
    args = (q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc], cache[:, :, dc:], seqlens,
            1.0 / math.sqrt(dn + dr), rows)
    naive = oracle.prefill_naive(*args)
    absorbed = oracle.prefill_absorbed(*args)
    assert _rel(absorbed, naive) <= 1e-12


def test_prefill_absorbed_row_equals_decode_prefix():
    """Each absorbed prefill row is bitwise the absorbed decode over the first
    pos_t + 1 cached rows."""
    rng = np.random.default_rng(8)
    B, T, H, dc, dr, dn, dv, L = 1, 5, 2, 32, 8, 16, 16, 9
    q_nope = rng.standard_normal((B, T, H, dn))
    q_rope = rng.standard_normal((B, T, H, dr))
    w_uk = rng.standard_normal((H, dn, dc)) / math.sqrt(dc)
    w_uv = rng.standard_normal((H, dv, dc)) / math.sqrt(dc)
    cache = rng.standard_normal((B, L, dc + dr))
    pre = oracle.prefill_absorbed(q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc],
                                  cache[:, :, dc:], [L], 0.3, [(0, t) for t in range(T)])
    for t in range(T):
        dec, _ = oracle.decode_absorbed(q_nope[:, t], q_rope[:, t], w_uk, w_uv,
                                        cache[:, :, :dc], cache[:, :, dc:], [L - T + t + 1], 0.3)
        assert np.array_equal(pre[t], dec[0])


# --------------------------------------------------------------------------
# Value side: the merged latent, the output projection and W_UV folded into W_O
# --------------------------------------------------------------------------

def test_decode_latent_up_projected_is_decode():
    """W_UV[h] o[b,h] equals the absorbed decode's output, so the latent is the
    attention output before the single up-projection."""
    rng = np.random.default_rng(61)
    B, H, dc, dr, dn, dv, N = 2, 3, 48, 16, 16, 12, 40
    q_nope, q_rope, w_uk, w_uv, cache = _rand_case(rng, B, H, dc, dr, dn, dv, N)
    seq = np.array([N, 17], np.int32)
    o = oracle.decode_latent(q_nope, q_rope, w_uk, cache[:, :, :dc], cache[:, :, dc:], seq, 0.3)
    out, _ = oracle.decode_absorbed(q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc],
                                    cache[:, :, dc:], seq, 0.3)
    up = np.einsum("hvc,bhc->bhv", w_uv, o)
    assert _rel(up, out) <= 1e-13
    # one cached row: the softmax weight is exactly 1 and o is that row
    one = oracle.decode_latent(q_nope, q_rope, w_uk, cache[:, :, :dc], cache[:, :, dc:],
                               np.array([1, 1], np.int32), 0.3)
    assert np.array_equal(one, np.broadcast_to(cache[:, None, 0, :dc], one.shape))


def test_output_proj_is_a_matrix_product():
    rng = np.random.default_rng(62)
    x = rng.standard_normal((5, 96))
    w = datagen.bf16_bits(rng.standard_normal((33, 96)).astype(np.float32))
    y = oracle.output_proj(x, w)
    ref = x @ datagen.bf16_to_f32(w).astype(np.float64).T      # numpy's fp64 product
    assert _rel(y, ref) <= 1e-13


def test_fold_with_selection_weights_places_columns():
    """W_UV[h] row i selecting latent channel sel[h][i] makes W_OV carry W_O's
    column (h, i) at (h, sel[h][i]) and zeros elsewhere, exactly."""
    rng = np.random.default_rng(63)
    N, H, dv, dc = 7, 3, 4, 10
    w_o = rng.standard_normal((N, H * dv))
    sel = np.stack([rng.permutation(dc)[:dv] for _ in range(H)])
    w_uv = np.zeros((H, dv, dc))
    for h in range(H):
        w_uv[h, np.arange(dv), sel[h]] = 1.0
    w_ov = oracle.fold_value_output(w_o, w_uv)
    expect = np.zeros((N, H * dc))
    for h in range(H):
        for i in range(dv):
            expect[:, h * dc + sel[h][i]] = w_o[:, h * dv + i]
    assert np.array_equal(w_ov, expect)


@pytest.mark.parametrize("dtype", ["f64", "bf16"])
def test_folded_projection_equals_unfolded(dtype):
    """Associativity on the value side: W_O concat_h(W_UV[h] o_h) from the
    absorbed decode equals W_OV concat_h(o_h) from the merged latent."""
    rng = np.random.default_rng(64)
    B, H, dc, dr, dn, dv, N, d_model = 2, 3, 32, 8, 16, 12, 25, 20
    q_nope, q_rope, w_uk, w_uv, cache = _rand_case(rng, B, H, dc, dr, dn, dv, N)
    w_o = rng.standard_normal((d_model, H * dv)) / math.sqrt(H * dv)
    if dtype == "bf16":
        q_nope, q_rope, w_uk, w_uv, cache, w_o = (
            datagen.bf16_bits(a.astype(np.float32)) for a in (q_nope, q_rope, w_uk, w_uv, cache, w_o))
    seq = np.array([N, 9], np.int32)
    out, _ = oracle.decode_absorbed(q_nope, q_rope, w_uk, w_uv, cache[:, :, :dc],
                                    cache[:, :, dc:], seq, 0.25)
    y_unfolded = oracle.output_proj(out.reshape(B, H * dv), w_o)
    o = oracle.decode_latent(q_nope, q_rope, w_uk, cache[:, :, :dc], cache[:, :, dc:], seq, 0.25)
    y_folded = oracle.output_proj(o.reshape(B, H * dc), oracle.fold_value_output(w_o, w_uv))
    assert _rel(y_folded, y_unfolded) <= 1e-12


# --------------------------------------------------------------------------
# Mutations: each plausible oracle mistake is caught by the pins above
# --------------------------------------------------------------------------

def test_pins_catch_plausible_mistakes():
    """Simulate mistakes by mutating the inputs the oracle sees and check that
    the independent SDPA reference would flag each of them."""
    rng = np.random.default_rng(77)
    B, H, dc, dr, dn, dv, N = 1, 2, 32, 16, 32, 32, 20
    q_nope, q_rope, w_uk, w_uv, cache = _rand_case(rng, B, H, dc, dr, dn, dv, N)
    scale = 1.0 / math.sqrt(dn + dr)
    seq = np.array([N], np.int32)
    ref = _sdpa_decode(q_nope, q_rope, w_uk, w_uv, cache, seq, scale)

    def run(qn=q_nope, qr=q_rope, wk=w_uk, wv=w_uv, c=cache, L=seq, s=scale):
        return oracle.decode_absorbed(qn, qr, wk, wv, c[:, :, :dc], c[:, :, dc:], L, s)[0]

    assert _rel(run(), ref) <= 1e-12                      # the unmutated oracle passes
    mutations = {
        "transposed W_UK": dict(wk=np.ascontiguousarray(w_uk.transpose(0, 2, 1))),
        "dropped RoPE term": dict(qr=np.zeros_like(q_rope)),
        "scale 1/sqrt(d_n)": dict(s=1.0 / math.sqrt(dn)),
        "length off by one": dict(L=seq - 1),
        "W_UV of another head": dict(wv=w_uv[::-1].copy()),
    }
    for name, kw in mutations.items():
        assert _rel(run(**kw), ref) > 1e-3, name


# --------------------------------------------------------------------------
# absorb_q: the content score through the absorbed query equals the score
# against the decompressed key ("mla-from-scratch" README, absorption)
# --------------------------------------------------------------------------

def test_absorb_content_score_identity():
    rng = np.random.default_rng(55)
    B, H, dn, dc = 2, 3, 16, 40
    q = rng.standard_normal((B, H, dn))
    w = rng.standard_normal((H, dn, dc))
    c = rng.standard_normal(dc)
    qa = oracle.absorb_q(q, w)
    for b in range(B):
        for h in range(H):
            k = w[h] @ c                     # decompressed key W_UK c
            assert abs(qa[b, h] @ c - q[b, h] @ k) <= 1e-12 * max(1.0, abs(q[b, h] @ k))
    # a transposed weight would not even have the right length
    assert qa.shape == (B, H, dc)


# --------------------------------------------------------------------------
# Rotary embedding of the decoupled key (RoFormer, cited by the
# "mla-from-scratch" README for the relative position property) and the
# cache-row producer c = W_DKV h, k^R = RoPE(W_KR h)
# --------------------------------------------------------------------------

def test_rope_relative_position_property():
    """<R_m q, R_n k> depends on n - m only."""
    rng = np.random.default_rng(61)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n in [(0, 5), (3, 8), (1000, 1005), (131066, 131071)]:
        ref = oracle.rope(q, 0) @ oracle.rope(k, n - m)
        got = oracle.rope(q, m) @ oracle.rope(k, n)
        assert abs(got - ref) <= 1e-10 * max(1.0, abs(ref)), (m, n)
    a = oracle.rope(q, 0) @ oracle.rope(k, 5)
    b = oracle.rope(q, 0) @ oracle.rope(k, 6)
    assert abs(a - b) > 1e-3


def test_rope_norm_and_identity():
    rng = np.random.default_rng(62)
    x = rng.standard_normal(64)
    assert np.array_equal(oracle.rope(x, 0), x)
    for p in (1, 77, 4096, 131071):
        assert abs(np.linalg.norm(oracle.rope(x, p)) - np.linalg.norm(x)) <= 1e-12 * np.linalg.norm(x)


@pytest.mark.parametrize("base", [10000.0, 500.0])
def test_rope_closed_forms(base):
    """One pair: rotation by pos radians (theta_0 = 1).  Two pairs: the second
    turns by pos * base^(-1/2)."""
    x = np.array([0.3, -1.7, 2.2, 0.9])
    for p in (1, 2, 13, 1000):
        one = oracle.rope(x[:2], p, base)
        assert np.allclose(one, [x[0] * math.cos(p) - x[1] * math.sin(p),
                                 x[0] * math.sin(p) + x[1] * math.cos(p)], rtol=0, atol=1e-12)
        two = oracle.rope(x, p, base)
        a = p * base ** -0.5
        assert np.allclose(two[:2], one, rtol=0, atol=1e-12)
        assert np.allclose(two[2:], [x[2] * math.cos(a) - x[3] * math.sin(a),
                                     x[2] * math.sin(a) + x[3] * math.cos(a)], rtol=0, atol=1e-12)


def test_rope_rotates_every_vector_of_an_array():
    """A stack of vectors (one per head) is rotated vector by vector."""
    rng = np.random.default_rng(44)
    x = rng.standard_normal((3, 5, 16))
    got = oracle.rope(x, 123, 10000.0)
    for i in range(3):
        for j in range(5):
            assert np.array_equal(got[i, j], oracle.rope(x[i, j], 123, 10000.0))
    assert not np.array_equal(got[2, 4], x[2, 4])


def test_cache_rows_are_projections_then_rotation():
    rng = np.random.default_rng(63)
    B, d_model, dc, dr = 3, 96, 32, 8
    h = rng.standard_normal((B, d_model))
    w_dkv = rng.standard_normal((dc, d_model)) / math.sqrt(d_model)
    w_kr = rng.standard_normal((dr, d_model)) / math.sqrt(d_model)
    pos = [0, 7, 131071]
    c, kr = oracle.cache_rows(h, w_dkv, w_kr, pos)
    assert np.allclose(c, h @ w_dkv.T, rtol=0, atol=1e-12)            # library matmul
    assert np.allclose(kr[0], h[0] @ w_kr.T, rtol=0, atol=1e-12)      # position 0: no rotation
    for b in (1, 2):
        assert np.allclose(kr[b], oracle.rope(h[b] @ w_kr.T, pos[b]), rtol=0, atol=1e-12)
