"""The oracle's pins catch plausible mistakes in the oracle itself.

Each case below plants one mistake in a copy of ``oracle/mla_oracle.c`` (a
textual substitution), compiles that copy on the CPU into a temporary
directory, points the oracle's Python wrapper at it and runs the pin checks
of ``test_oracle_pins.py``.  At least one pin must fail for every planted
mistake, and all of them must pass on an unmodified copy built the same way.
"""
import contextlib
import os
import subprocess

import numpy as np
import pytest

import oracle
import oracle.oracle as oracle_impl
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle_impl.__file__), "mla_oracle.c")

# (name, text in the source, replacement); the text must occur exactly once.
MUTATIONS = [
    ("absorbed: RoPE term dropped",
     "s[n] = d->scale * (content + pos);", "s[n] = d->scale * content; (void)pos;"),
    ("absorbed: scale on the content term only",
     "s[n] = d->scale * (content + pos);", "s[n] = d->scale * content + pos;"),
    ("naive: RoPE term dropped",
     "for (int64_t r = 0; r < dr; ++r) dot += qr[r] * kr[r];", "(void)qr;"),
    ("naive: RoPE term subtracted",
     "for (int64_t r = 0; r < dr; ++r) dot += qr[r] * kr[r];",
     "for (int64_t r = 0; r < dr; ++r) dot -= qr[r] * kr[r];"),
    ("absorbed: W_UK read transposed",
     "acc += widen(w_uk, dt, (h * dn + i) * dc + j) * qn[i];",
     "acc += widen(w_uk, dt, (h * dn + (j % dn)) * dc + (i % dc)) * qn[i];"),
    ("naive: W_UK read transposed",
     "k += widen(w_uk, dt, (h * dn + i) * dc + j) * c[j];",
     "k += widen(w_uk, dt, (h * dn + (j % dn)) * dc + (i % dc)) * c[j];"),
    ("naive: W_UV read transposed",
     "acc += widen(w_uv, dt, (h * dv + i) * dc + j) * c[j];",
     "acc += widen(w_uv, dt, (h * dv + (j % dv)) * dc + (i % dc)) * c[j];"),
    ("absorbed: W_UV of the next head",
     "acc += widen(w_uv, dt, (h * dv + i) * dc + j) * o[j];",
     "acc += widen(w_uv, dt, (((h + 1) % d->H) * dv + i) * dc + j) * o[j];"),
    ("absorbed: latent sum over shifted channels",
     "for (int64_t j = 0; j < dc; ++j) o[j] += p[n] * c[j];",
     "for (int64_t j = 0; j < dc; ++j) o[j] += p[n] * c[(j + 1) % dc];"),
    ("softmax: no max subtraction",
     "p[n] = exp(s[n] - m); z += p[n];", "p[n] = exp(s[n]); z += p[n]; (void)m;"),
    ("softmax: not normalised",
     "p[n] /= z; total += p[n];", "total += p[n]; (void)z;"),
    ("softmax: last weight missing from the normaliser",
     "p[n] = exp(s[n] - m); z += p[n];", "p[n] = exp(s[n] - m); z += (n + 1 < L) ? p[n] : 0.0;"),
    ("softmax: max taken over all but the last score",
     "for (int64_t n = 0; n < L; ++n) if (s[n] > m) m = s[n];",
     "for (int64_t n = 0; n + 1 < L; ++n) if (s[n] > m) m = s[n]; if (L == 1) m = s[0];"),
    ("decode: cached length off by one",
     "(int64_t)seqlens[b], out + k * d->dv);", "(int64_t)seqlens[b] - 1, out + k * d->dv);"),
    ("prefill: diagonal masked out",
     "fn(d, qn, qr, w_uk, w_uv, ckv, kpe, b, h, pos + 1, out + k * d->dv);",
     "fn(d, qn, qr, w_uk, w_uv, ckv, kpe, b, h, pos > 0 ? pos : 1, out + k * d->dv);"),
    ("prefill: queries before the cache see row 0",
     "fn(d, qn, qr, w_uk, w_uv, ckv, kpe, b, h, pos + 1, out + k * d->dv);",
     "fn(d, qn, qr, w_uk, w_uv, ckv, kpe, b, h, pos < 0 ? 1 : pos + 1, out + k * d->dv);"),
    ("absorbed prefill: through the naive definition with W_UK for W_UV",
     "return prefill_common(absorbed_one, d, T, q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens,",
     "return prefill_common(absorbed_one, d, T, q_nope, q_rope, w_uk, w_uk, ckv, kpe, seqlens,"),
    ("prefill: queries aligned top-left",
     "const int64_t pos = (int64_t)seqlens[b] - T + t;", "const int64_t pos = t;"),
    ("absorb_q: W_UK read transposed",
     "acc += widen(w_uk, d->dtype, (h * d->dn + i) * d->dc + j) *",
     "acc += widen(w_uk, d->dtype, (h * d->dn + (j % d->dn)) * d->dc + (i % d->dc)) *"),
    ("cache bytes: RoPE part left out",
     "(uint64_t)(d_c + d_r) * (uint64_t)bytes_per_elem;",
     "(uint64_t)d_c * (uint64_t)bytes_per_elem; (void)d_r;"),
    ("rope: sine of the first component flipped",
     "out[2 * i] = x0 * c - x1 * s;", "out[2 * i] = x0 * c + x1 * s;"),
    ("rope: theta exponent without its factor 2",
     "pow(base, -2.0 * (double)i / (double)dr)", "pow(base, -1.0 * (double)i / (double)dr)"),
    ("rope: rotation angle without the position",
     "const double a = pos * theta;", "const double a = theta; (void)pos;"),
    ("cache rows: RoPE key projected with W_DKV",
     "acc += widen(w_kr, dtype, j * d_model + k) * hb[k];",
     "acc += widen(w_dkv, dtype, j * d_model + k) * hb[k];"),
    ("cache rows: the key left unrotated",
     "if (dr > 0) oracle_rope(dr, raw, (double)pos[b], base, kr + b * dr);",
     "if (dr > 0) oracle_rope(dr, raw, 0.0, base, kr + b * dr);"),
    ("output projection: weight read transposed",
     "acc += widen(w, dtype_w, n * K + k) * widen(x, dtype_x, b * K + k);",
     "acc += widen(w, dtype_w, (k % N) * K + (n % K)) * widen(x, dtype_x, b * K + k);"),
    ("fold: W_UV read transposed",
     "widen(w_uv, dtype, (h * dv + i) * dc + j);",
     "widen(w_uv, dtype, (h * dv + (j % dv)) * dc + (i % dc));"),
    ("fold: W_O column of the wrong head",
     "acc += widen(w_o, dtype, n * H * dv + h * dv + i) *",
     "acc += widen(w_o, dtype, n * H * dv + ((h + 1) % H) * dv + i) *"),
    ("bf16 widening shifted",
     "uint32_t u = ((uint32_t)((const uint16_t *)base)[i]) << 16;",
     "uint32_t u = ((uint32_t)((const uint16_t *)base)[i]) << 15;"),
]

# The pin battery: every check here is one of the pins, at one parameter set.
PINS = {
    "naive vs torch SDPA": lambda: pins.test_naive_matches_torch_sdpa(64, 16, 33),
    "naive vs torch SDPA, L=1": lambda: pins.test_naive_matches_torch_sdpa(16, 0, 1),
    "absorbed == naive": lambda: pins.test_absorbed_equals_naive(64, 7, 16),
    "L=1 selection (naive)": lambda: pins.test_single_token_selection_exact(oracle.decode_naive),
    "L=1 selection (absorbed)":
        lambda: pins.test_single_token_selection_exact(oracle.decode_absorbed),
    "L=1 random W_UV (naive)": lambda: pins.test_single_token_random_weights(oracle.decode_naive),
    "L=1 random W_UV (absorbed)":
        lambda: pins.test_single_token_random_weights(oracle.decode_absorbed),
    "softmax mass": lambda: pins.test_softmax_mass_is_one(77),
    "uniform scores": pins.test_uniform_scores_give_mean,
    "dominant first token": lambda: pins.test_dominant_token_no_overflow(0),
    "dominant last token": lambda: pins.test_dominant_token_no_overflow(39),
    "permutation": pins.test_permutation_invariance,
    "NaN padding (absorbed)": lambda: pins.test_nan_padding_ignored(oracle.decode_absorbed),
    "zero length": pins.test_zero_length_gives_zero_output,
    "storage widening": pins.test_bf16_and_f32_storage_widen_exactly,
    "prefill vs masked SDPA, L>T": lambda: pins.test_prefill_matches_masked_sdpa(4, 11),
    "prefill vs masked SDPA, L=T": lambda: pins.test_prefill_matches_masked_sdpa(9, 9),
    "prefill row == decode prefix": pins.test_prefill_row_equals_decode_prefix,
    "prefill rows before the cache": lambda: pins.test_prefill_rows_before_the_cache(6, 4),
    "absorbed prefill == naive prefill":
        lambda: pins.test_prefill_absorbed_equals_naive(64, 16, 5, 13),
    "absorbed prefill row == decode prefix": pins.test_prefill_absorbed_row_equals_decode_prefix,
    "absorb_q content identity": pins.test_absorb_content_score_identity,
    "eyestech telemetry table": pins.test_cache_bytes_eyestech_telemetry,
    "mla-from-scratch table": pins.test_cache_bytes_mla_from_scratch_table,
    "songhuiming 99 tokens": pins.test_cache_elems_songhuiming_99_tokens,
    "rope relative position": pins.test_rope_relative_position_property,
    "rope norm and identity": pins.test_rope_norm_and_identity,
    "rope closed forms": lambda: pins.test_rope_closed_forms(10000.0),
    "cache rows": pins.test_cache_rows_are_projections_then_rotation,
    "latent up-projected is decode": pins.test_decode_latent_up_projected_is_decode,
    "output projection": pins.test_output_proj_is_a_matrix_product,
    "fold with selection weights": pins.test_fold_with_selection_weights_places_columns,
    "folded == unfolded": lambda: pins.test_folded_projection_equals_unfolded("f64"),
}


def _build(src_text: str, out_dir: str, tag: str) -> str:
    c = os.path.join(out_dir, f"oracle_{tag}.c")
    so = os.path.join(out_dir, f"liboracle_{tag}.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-w", "-o", so, c,
                    "-lm"], check=True)
    return so


@contextlib.contextmanager
def _oracle_build(path):
    saved = oracle_impl._lib
    oracle_impl._lib = oracle_impl._open(path)
    try:
        yield
    finally:
        oracle_impl._lib = saved


def _failing_pins():
    failed = []
    with np.errstate(all="ignore"):
        for name, check in PINS.items():
            try:
                check()
            except Exception:  # an assertion, or an oracle error on bad output
                failed.append(name)
    return failed


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


def test_unmodified_copy_passes_every_pin(source, tmp_path):
    with _oracle_build(_build(source, str(tmp_path), "clean")):
        assert _failing_pins() == []


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(source, tmp_path, name, old, new):
    assert source.count(old) == 1, f"mutation site not unique: {old!r}"
    mutated = source.replace(old, new)
    with _oracle_build(_build(mutated, str(tmp_path), "mut")):
        failed = _failing_pins()
    print(f"{name}: caught by {failed}")
    assert failed, f"no pin catches: {name}"
