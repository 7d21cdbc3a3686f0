/*
 * oracle_sanitize_driver.c -- runs every entry point of the C oracle on small
 * seeded inputs, under AddressSanitizer and UndefinedBehaviorSanitizer
 * (host code only; built and run by tests/test_oracle_sanitizers.py), and
 * checks the identities that tie the entry points together:
 *   absorbed decode = naive decode (the associativity the "mla-from-scratch"
 *   README, "Absorption, and why RoPE breaks it", relies on); a selected pair
 *   list returns the same rows as the whole batch; W_UV applied to the merged
 *   latent is the absorbed output; q~ . c = q_nope . (W_UK c); absorbed
 *   prefill = naive prefill row by row, queries before the cache give zeros;
 *   the rotary embedding preserves the norm and is the identity at position
 *   0; the cache rows and the output projection equal direct sums; the
 *   folded projection equals the unfolded one; the cache-size formula.
 * Inputs cover fp64, fp32 and bf16 storage, strided caches with padding, and
 * lengths 0, 1 and full.  Exit status 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

enum { F64 = 0, F32 = 1, BF16 = 2 };

typedef struct {
    int64_t B, H, dc, dr, dn, dv;
    int64_t ckv_sb, ckv_sn, kpe_sb, kpe_sn;
    int32_t dtype, reserved;
    double scale;
} dims_t;

int oracle_decode_naive(const dims_t *, const void *, const void *, const void *, const void *,
                        const void *, const void *, const int32_t *, const int64_t *, int64_t,
                        double *, double *);
int oracle_decode_absorbed(const dims_t *, const void *, const void *, const void *, const void *,
                           const void *, const void *, const int32_t *, const int64_t *, int64_t,
                           double *, double *);
int oracle_decode_latent(const dims_t *, const void *, const void *, const void *, const void *,
                         const void *, const int32_t *, const int64_t *, int64_t, double *);
int oracle_absorb_q(const dims_t *, const void *, const void *, double *);
int oracle_prefill_naive(const dims_t *, int64_t, const void *, const void *, const void *,
                         const void *, const void *, const void *, const int32_t *,
                         const int64_t *, int64_t, double *);
int oracle_prefill_absorbed(const dims_t *, int64_t, const void *, const void *, const void *,
                            const void *, const void *, const void *, const int32_t *,
                            const int64_t *, int64_t, double *);
void oracle_rope(int64_t, const double *, double, double, double *);
int oracle_cache_rows(int64_t, int64_t, int64_t, int64_t, int32_t, const void *, const void *,
                      const void *, const int64_t *, double, double *, double *);
int oracle_output_proj(int64_t, int64_t, int64_t, int32_t, const void *, int32_t, const void *,
                       double *);
int oracle_fold_value_output(int64_t, int64_t, int64_t, int64_t, int32_t, const void *,
                             const void *, double *);
uint64_t oracle_kv_cache_bytes(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t);

static int failures = 0;

static void expect(int ok, const char *what)
{
    if (!ok) {
        fprintf(stderr, "FAIL: %s\n", what);
        ++failures;
    }
}

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double normal(void)  /* a sum of 12 uniforms minus 6: mean 0, variance 1 */
{
    double s = 0.0;
    for (int i = 0; i < 12; ++i) {
        rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
        s += (double)(rng_state >> 11) / 9007199254740992.0;
    }
    return s - 6.0;
}

/* A buffer of n values in storage type dt, and the same values widened. */
typedef struct { void *p; double *w; } buf_t;

static uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);  /* round to nearest even (finite inputs) */
    return (uint16_t)(u >> 16);
}
static double from_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static buf_t make_buf(int dt, int64_t n, double sd)
{
    buf_t b;
    b.w = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (dt == F64) {
        double *p = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        for (int64_t i = 0; i < n; ++i) b.w[i] = p[i] = sd * normal();
        b.p = p;
    } else if (dt == F32) {
        float *p = malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
        for (int64_t i = 0; i < n; ++i) { p[i] = (float)(sd * normal()); b.w[i] = p[i]; }
        b.p = p;
    } else {
        uint16_t *p = malloc(sizeof(uint16_t) * (size_t)(n > 0 ? n : 1));
        for (int64_t i = 0; i < n; ++i) { p[i] = to_bf16((float)(sd * normal())); b.w[i] = from_bf16(p[i]); }
        b.p = p;
    }
    return b;
}
static void free_buf(buf_t b) { free(b.p); free(b.w); }

static int close_rel(const double *a, const double *b, int64_t n, double tol)
{
    double scale = 0.0, err = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        scale = fmax(scale, fabs(b[i]));
        err = fmax(err, fabs(a[i] - b[i]));
    }
    return err <= tol * (scale > 1.0 ? scale : 1.0);
}

static void run_dtype(int dt)
{
    const int64_t B = 3, H = 2, dc = 16, dr = 8, dn = 8, dv = 12, nmax = 37, T = 4;
    dims_t d = {B, H, dc, dr, dn, dv, 0, 0, 0, 0, dt, 0, 1.0 / sqrt((double)(dn + dr))};
    d.ckv_sn = dc + 3;            /* padded latent rows */
    d.ckv_sb = nmax * d.ckv_sn + 5;
    d.kpe_sn = dr + 1;            /* padded RoPE-key rows */
    d.kpe_sb = nmax * d.kpe_sn + 2;
    buf_t ckv = make_buf(dt, B * d.ckv_sb, 1.0), kpe = make_buf(dt, B * d.kpe_sb, 1.0);
    buf_t wuk = make_buf(dt, H * dn * dc, 1.0 / sqrt((double)dc));
    buf_t wuv = make_buf(dt, H * dv * dc, 1.0 / sqrt((double)dc));
    buf_t qn = make_buf(dt, B * T * H * dn, 1.0), qr = make_buf(dt, B * T * H * dr, 1.0);
    const int32_t seqlens[3] = {(int32_t)nmax, 1, 0};

    /* decode: absorbed = naive, an empty sequence gives zeros */
    double *o_n = calloc((size_t)(B * H * dv), sizeof(double));
    double *o_a = calloc((size_t)(B * H * dv), sizeof(double));
    double psum[6];
    expect(oracle_decode_naive(&d, qn.p, qr.p, wuk.p, wuv.p, ckv.p, kpe.p, seqlens, NULL, 0, o_n, psum) == 0, "decode_naive status");
    expect(oracle_decode_absorbed(&d, qn.p, qr.p, wuk.p, wuv.p, ckv.p, kpe.p, seqlens, NULL, 0, o_a, NULL) == 0, "decode_absorbed status");
    expect(close_rel(o_a, o_n, B * H * dv, 1e-12), "absorbed decode equals naive decode");
    for (int64_t i = 2 * H * dv; i < 3 * H * dv; ++i) expect(o_a[i] == 0.0, "empty sequence gives zeros");
    expect(fabs(psum[0] - 1.0) < 1e-14, "softmax mass is one");

    /* a pair list returns the same rows */
    const int64_t pairs[4] = {1, 1, 0, 0};
    double o_p[2 * 12];
    expect(oracle_decode_absorbed(&d, qn.p, qr.p, wuk.p, wuv.p, ckv.p, kpe.p, seqlens, pairs, 2, o_p, NULL) == 0, "pairs status");
    expect(memcmp(o_p, o_a + (1 * H + 1) * dv, sizeof(double) * dv) == 0 &&
           memcmp(o_p + dv, o_a, sizeof(double) * dv) == 0, "pair list rows equal the batch rows");

    /* W_UV applied to the merged latent is the absorbed output */
    double *lat = calloc((size_t)(B * H * dc), sizeof(double));
    expect(oracle_decode_latent(&d, qn.p, qr.p, wuk.p, ckv.p, kpe.p, seqlens, NULL, 0, lat) == 0, "decode_latent status");
    double *up = calloc((size_t)(B * H * dv), sizeof(double));
    for (int64_t k = 0; k < B * H; ++k)
        for (int64_t i = 0; i < dv; ++i) {
            double a = 0.0;
            for (int64_t j = 0; j < dc; ++j) a += wuv.w[((k % H) * dv + i) * dc + j] * lat[k * dc + j];
            up[k * dv + i] = a;
        }
    expect(close_rel(up, o_a, B * H * dv, 1e-12), "W_UV o equals the absorbed output");

    /* q~ . c = q_nope . (W_UK c) */
    double *qa = calloc((size_t)(B * H * dc), sizeof(double));
    expect(oracle_absorb_q(&d, qn.p, wuk.p, qa) == 0, "absorb_q status");
    {
        const double *c = ckv.w;  /* sequence 0, row 0 */
        double lhs = 0.0, rhs = 0.0;
        for (int64_t j = 0; j < dc; ++j) lhs += qa[j] * c[j];
        for (int64_t i = 0; i < dn; ++i) {
            double k = 0.0;
            for (int64_t j = 0; j < dc; ++j) k += wuk.w[i * dc + j] * c[j];
            rhs += qn.w[i] * k;
        }
        expect(fabs(lhs - rhs) <= 1e-12 * (1.0 + fabs(rhs)), "absorbed query identity");
    }

    /* prefill: absorbed = naive row by row; queries before the cache give zeros */
    const int32_t plens[3] = {(int32_t)nmax, 2, 0};
    int64_t rows[2 * 12];
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < T; ++t) { rows[2 * (b * T + t)] = b; rows[2 * (b * T + t) + 1] = t; }
    double *p_n = calloc((size_t)(B * T * H * dv), sizeof(double));
    double *p_a = calloc((size_t)(B * T * H * dv), sizeof(double));
    expect(oracle_prefill_naive(&d, T, qn.p, qr.p, wuk.p, wuv.p, ckv.p, kpe.p, plens, rows, B * T, p_n) == 0, "prefill_naive status");
    expect(oracle_prefill_absorbed(&d, T, qn.p, qr.p, wuk.p, wuv.p, ckv.p, kpe.p, plens, rows, B * T, p_a) == 0, "prefill_absorbed status");
    expect(close_rel(p_a, p_n, B * T * H * dv, 1e-12), "absorbed prefill equals naive prefill");
    /* sequence 1 has 2 rows for 4 queries: queries 0 and 1 sit before the cache */
    for (int64_t i = (1 * T + 0) * H * dv; i < (1 * T + 2) * H * dv; ++i) expect(p_a[i] == 0.0, "query before the cache gives zeros");
    for (int64_t i = (2 * T) * H * dv; i < (3 * T) * H * dv; ++i) expect(p_n[i] == 0.0, "empty sequence gives zero rows");

    /* cache rows: c = W_DKV h and the unrotated key at position 0 */
    const int64_t dm = 20;
    buf_t hh = make_buf(dt, B * dm, 1.0), wd = make_buf(dt, dc * dm, 0.2), wk = make_buf(dt, dr * dm, 0.2);
    const int64_t pos[3] = {0, 5, 36};
    double *c = calloc((size_t)(B * dc), sizeof(double)), *kr = calloc((size_t)(B * dr), sizeof(double));
    expect(oracle_cache_rows(B, dm, dc, dr, dt, hh.p, wd.p, wk.p, pos, 10000.0, c, kr) == 0, "cache_rows status");
    for (int64_t j = 0; j < dc; ++j) {
        double a = 0.0;
        for (int64_t k = 0; k < dm; ++k) a += wd.w[j * dm + k] * hh.w[k];
        expect(fabs(a - c[j]) <= 1e-12 * (1.0 + fabs(a)), "latent row equals W_DKV h");
    }
    for (int64_t j = 0; j < dr; ++j) {
        double a = 0.0;
        for (int64_t k = 0; k < dm; ++k) a += wk.w[j * dm + k] * hh.w[k];
        expect(fabs(a - kr[j]) <= 1e-12 * (1.0 + fabs(a)), "position 0 leaves the key unrotated");
    }

    /* output projection and the fold: W_O (W_UV o) = W_OV o */
    const int64_t N = 7;
    buf_t wo = make_buf(dt, N * H * dv, 0.3);
    double *wov = calloc((size_t)(N * H * dc), sizeof(double));
    expect(oracle_fold_value_output(N, H, dv, dc, dt, wo.p, wuv.p, wov) == 0, "fold status");
    double *y1 = calloc((size_t)(B * N), sizeof(double)), *y2 = calloc((size_t)(B * N), sizeof(double));
    expect(oracle_output_proj(B, H * dv, N, F64, o_a, dt, wo.p, y1) == 0, "output_proj status");
    expect(oracle_output_proj(B, H * dc, N, F64, lat, F64, wov, y2) == 0, "folded output_proj status");
    expect(close_rel(y2, y1, B * N, 1e-12), "folded projection equals unfolded");
    for (int64_t n = 0; n < N; ++n) {
        double a = 0.0;
        for (int64_t k = 0; k < H * dv; ++k) a += wo.w[n * H * dv + k] * o_a[k];
        expect(fabs(a - y1[n]) <= 1e-12 * (1.0 + fabs(a)), "output projection equals the direct sum");
    }

    free(o_n); free(o_a); free(lat); free(up); free(qa); free(p_n); free(p_a); free(c); free(kr);
    free(wov); free(y1); free(y2);
    free_buf(ckv); free_buf(kpe); free_buf(wuk); free_buf(wuv); free_buf(qn); free_buf(qr);
    free_buf(hh); free_buf(wd); free_buf(wk); free_buf(wo);
}

int main(void)
{
    for (int dt = F64; dt <= BF16; ++dt) run_dtype(dt);

    /* rotary embedding: norm preserved, identity at position 0 */
    double x[8], y[8];
    for (int i = 0; i < 8; ++i) x[i] = normal();
    oracle_rope(8, x, 0.0, 10000.0, y);
    expect(memcmp(x, y, sizeof x) == 0, "position 0 is the identity");
    oracle_rope(8, x, 123.0, 10000.0, y);
    double nx = 0.0, ny = 0.0;
    for (int i = 0; i < 8; ++i) { nx += x[i] * x[i]; ny += y[i] * y[i]; }
    expect(fabs(nx - ny) <= 1e-12 * nx, "rotation preserves the norm");

    /* cache size: layers x batch x tokens x (d_c + d_r) x bytes */
    expect(oracle_kv_cache_bytes(61, 1, 131072, 512, 64, 2) == 61ull * 131072ull * 576ull * 2ull, "cache-size formula");

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: all checks hold\n");
    return 0;
}
