/*
 * mla_oracle.c -- plain fp64 CPU oracle for Multi-Head Latent Attention
 * decode and naive causal prefill.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it is used by the tests, by the smoke check and by the
 * benchmark's CPU-baseline leg, and by nothing else.  It shares no code,
 * header, table or helper with the HIP library.
 *
 * Every stored input (fp64, fp32 or bf16) is widened to double exactly; all
 * arithmetic is double precision with plain sequential loops, in the order
 * the definitions below state them.  Parallelism (OpenMP) is only over
 * independent (sequence, head) pairs or query rows, so results do not depend
 * on the thread count.
 *
 * Notation (the pages' own): c = latent cache row (d_c), k^R = decoupled
 * RoPE key (d_r), W_UK[h] in R^{d_n x d_c} and W_UV[h] in R^{d_v x d_c}
 * (row-major [H][d][d_c]), so k = W_UK[h] c and v = W_UV[h] c.
 *
 * Sources:
 *  - "Deep-Dive: Multi-Head Latent Attention (MLA) and Low-Rank KV Cache
 *    Compression in DeepSeek-V3", section 2 (per-head up-projections
 *    k_{t,i} = W_UK(i) c_t, v_{t,i} = W_UV(i) c_t) and section 3 (scaled
 *    dot-product softmax attention over the decompressed K and V).
 *  - "mla-from-scratch" README, section "Absorption, and why RoPE breaks it"
 *    (the score is an absorbed content term plus a decoupled positional term;
 *    value-side absorption: attend over latents, up-project once).
 *  - "DeepSeek MLA Architecture: How It Cuts KV Cache by 93%", section 2
 *    (absorbed query q~ = W_UK^T q).
 *  - songhuiming "MHA vs MLA" decode walk-through, MLA step 2 (the new
 *    token's latent is appended to the cache before attention, so the cached
 *    length counts the current token).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F64 = 0, OR_F32 = 1, OR_BF16 = 2 };

typedef struct {
    int64_t B, H, dc, dr, dn, dv;
    int64_t ckv_sb, ckv_sn; /* element strides of the latent cache       */
    int64_t kpe_sb, kpe_sn; /* element strides of the RoPE-key cache     */
    int32_t dtype;          /* storage type of every input (OR_*)        */
    int32_t reserved;
    double scale;           /* softmax scale applied to the full score   */
} oracle_dims;

/* Exact widening of one stored element to double. */
static double widen(const void *base, int dt, int64_t i)
{
    if (dt == OR_F64) return ((const double *)base)[i];
    if (dt == OR_F32) return (double)((const float *)base)[i];
    uint32_t u = ((uint32_t)((const uint16_t *)base)[i]) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static void widen_row(const void *base, int dt, int64_t off, int64_t n, double *dst)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = widen(base, dt, off + i);
}

/* Softmax over s[0..L): p_n = exp(s_n - max) / sum_m exp(s_m - max).
 * Returns sum_n p_n computed as its own sum (used by the normalisation pin). */
static double softmax(const double *s, int64_t L, double *p)
{
    double m = -INFINITY;
    for (int64_t n = 0; n < L; ++n) if (s[n] > m) m = s[n];
    double z = 0.0;
    for (int64_t n = 0; n < L; ++n) { p[n] = exp(s[n] - m); z += p[n]; }
    double total = 0.0;
    for (int64_t n = 0; n < L; ++n) { p[n] /= z; total += p[n]; }
    return total;
}

/*
 * O1 -- naive decode for one (b, h) with L cached rows: decompress every
 * cached latent into k_n = [W_UK[h] c_n ; k^R_n] and v_n = W_UV[h] c_n,
 * then out = sum_n softmax_n(scale * q . k_n) v_n with q = [q_nope ; q_rope].
 * q_nope/q_rope are given as already-widened vectors.
 */
static double naive_one(const oracle_dims *d, const double *qn, const double *qr,
                        const void *w_uk, const void *w_uv,
                        const void *ckv, const void *kpe, int64_t b, int64_t h,
                        int64_t L, double *out)
{
    const int dt = d->dtype;
    const int64_t dc = d->dc, dr = d->dr, dn = d->dn, dv = d->dv;
    for (int64_t i = 0; i < dv; ++i) out[i] = 0.0;
    if (L <= 0) return 0.0;

    double *c = malloc(sizeof(double) * (size_t)dc);
    double *kr = malloc(sizeof(double) * (size_t)(dr > 0 ? dr : 1));
    double *s = malloc(sizeof(double) * (size_t)L);
    double *p = malloc(sizeof(double) * (size_t)L);
    double *v = malloc(sizeof(double) * (size_t)dv);

    /* scores against the decompressed keys */
    for (int64_t n = 0; n < L; ++n) {
        widen_row(ckv, dt, b * d->ckv_sb + n * d->ckv_sn, dc, c);
        widen_row(kpe, dt, b * d->kpe_sb + n * d->kpe_sn, dr, kr);
        double dot = 0.0;
        for (int64_t i = 0; i < dn; ++i) {
            double k = 0.0; /* k_nope[i] = sum_j W_UK[h][i][j] c[j] */
            for (int64_t j = 0; j < dc; ++j)
                k += widen(w_uk, dt, (h * dn + i) * dc + j) * c[j];
            dot += qn[i] * k;
        }
        for (int64_t r = 0; r < dr; ++r) dot += qr[r] * kr[r];
        s[n] = d->scale * dot;
    }
    double total = softmax(s, L, p);

    /* weighted sum of the decompressed values */
    for (int64_t n = 0; n < L; ++n) {
        widen_row(ckv, dt, b * d->ckv_sb + n * d->ckv_sn, dc, c);
        for (int64_t i = 0; i < dv; ++i) {
            double acc = 0.0; /* v[i] = sum_j W_UV[h][i][j] c[j] */
            for (int64_t j = 0; j < dc; ++j)
                acc += widen(w_uv, dt, (h * dv + i) * dc + j) * c[j];
            v[i] = acc;
        }
        for (int64_t i = 0; i < dv; ++i) out[i] += p[n] * v[i];
    }
    free(c); free(kr); free(s); free(p); free(v);
    return total;
}

/*
 * O2, latent part -- absorbed attention for one (b, h) up to the merged
 * latent: q~ = W_UK[h]^T q_nope, s_n = scale * (q~ . c_n + q_rope . k^R_n),
 * the same softmax, o = sum_n p_n c_n (attention accumulated in latent
 * space).  o has d_c entries; returns the softmax mass.
 */
static double absorbed_latent(const oracle_dims *d, const double *qn, const double *qr,
                              const void *w_uk, const void *ckv, const void *kpe, int64_t b,
                              int64_t h, int64_t L, double *o)
{
    const int dt = d->dtype;
    const int64_t dc = d->dc, dr = d->dr, dn = d->dn;
    for (int64_t j = 0; j < dc; ++j) o[j] = 0.0;
    if (L <= 0) return 0.0;

    double *qa = malloc(sizeof(double) * (size_t)dc);
    double *c = malloc(sizeof(double) * (size_t)dc);
    double *kr = malloc(sizeof(double) * (size_t)(dr > 0 ? dr : 1));
    double *s = malloc(sizeof(double) * (size_t)L);
    double *p = malloc(sizeof(double) * (size_t)L);

    for (int64_t j = 0; j < dc; ++j) { /* q~[j] = sum_i W_UK[h][i][j] q_nope[i] */
        double acc = 0.0;
        for (int64_t i = 0; i < dn; ++i) acc += widen(w_uk, dt, (h * dn + i) * dc + j) * qn[i];
        qa[j] = acc;
    }
    for (int64_t n = 0; n < L; ++n) {
        widen_row(ckv, dt, b * d->ckv_sb + n * d->ckv_sn, dc, c);
        widen_row(kpe, dt, b * d->kpe_sb + n * d->kpe_sn, dr, kr);
        double content = 0.0, pos = 0.0;
        for (int64_t j = 0; j < dc; ++j) content += qa[j] * c[j];
        for (int64_t r = 0; r < dr; ++r) pos += qr[r] * kr[r];
        s[n] = d->scale * (content + pos);
    }
    double total = softmax(s, L, p);
    for (int64_t n = 0; n < L; ++n) {
        widen_row(ckv, dt, b * d->ckv_sb + n * d->ckv_sn, dc, c);
        for (int64_t j = 0; j < dc; ++j) o[j] += p[n] * c[j];
    }
    free(qa); free(c); free(kr); free(s); free(p);
    return total;
}

/*
 * O2 -- absorbed decode for one (b, h): the merged latent o above, then
 * out = W_UV[h] o (one up-projection at the end).
 */
static double absorbed_one(const oracle_dims *d, const double *qn, const double *qr,
                           const void *w_uk, const void *w_uv,
                           const void *ckv, const void *kpe, int64_t b, int64_t h,
                           int64_t L, double *out)
{
    const int dt = d->dtype;
    const int64_t dc = d->dc, dv = d->dv;
    double *o = malloc(sizeof(double) * (size_t)dc);
    const double total = absorbed_latent(d, qn, qr, w_uk, ckv, kpe, b, h, L, o);
    for (int64_t i = 0; i < dv; ++i) { /* out[i] = sum_j W_UV[h][i][j] o[j] */
        double acc = 0.0;
        for (int64_t j = 0; j < dc; ++j) acc += widen(w_uv, dt, (h * dv + i) * dc + j) * o[j];
        out[i] = L > 0 ? acc : 0.0;
    }
    free(o);
    return total;
}

typedef double (*one_fn)(const oracle_dims *, const double *, const double *,
                         const void *, const void *, const void *, const void *,
                         int64_t, int64_t, int64_t, double *);

static int check_dims(const oracle_dims *d)
{
    if (!d || d->B < 0 || d->H <= 0 || d->dc <= 0 || d->dr < 0 || d->dn <= 0 || d->dv <= 0) return 1;
    if (d->dtype != OR_F64 && d->dtype != OR_F32 && d->dtype != OR_BF16) return 1;
    return 0;
}

/* Decode over a list of (b, h) pairs (npairs entries of two int64), or over
 * every pair in b-major order when pairs == NULL.  q_nope is [B][H][dn],
 * q_rope is [B][H][dr].  out is [npairs][dv]; psum (optional) receives the
 * separately summed softmax mass of each pair. */
static int decode_common(one_fn fn, const oracle_dims *d, const void *q_nope, const void *q_rope,
                         const void *w_uk, const void *w_uv, const void *ckv, const void *kpe,
                         const int32_t *seqlens, const int64_t *pairs, int64_t npairs,
                         double *out, double *psum)
{
    if (check_dims(d) || !out || !seqlens) return 1;
    const int64_t total = pairs ? npairs : d->B * d->H;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t k = 0; k < total; ++k) {
        const int64_t b = pairs ? pairs[2 * k] : k / d->H;
        const int64_t h = pairs ? pairs[2 * k + 1] : k % d->H;
        if (b < 0 || b >= d->B || h < 0 || h >= d->H) { bad = 1; continue; }
        double *qn = malloc(sizeof(double) * (size_t)d->dn);
        double *qr = malloc(sizeof(double) * (size_t)(d->dr > 0 ? d->dr : 1));
        widen_row(q_nope, d->dtype, (b * d->H + h) * d->dn, d->dn, qn);
        widen_row(q_rope, d->dtype, (b * d->H + h) * d->dr, d->dr, qr);
        double t = fn(d, qn, qr, w_uk, w_uv, ckv, kpe, b, h, (int64_t)seqlens[b], out + k * d->dv);
        if (psum) psum[k] = t;
        free(qn); free(qr);
    }
    return bad;
}

int oracle_decode_naive(const oracle_dims *d, const void *q_nope, const void *q_rope,
                        const void *w_uk, const void *w_uv, const void *ckv, const void *kpe,
                        const int32_t *seqlens, const int64_t *pairs, int64_t npairs,
                        double *out, double *psum)
{
    return decode_common(naive_one, d, q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens,
                         pairs, npairs, out, psum);
}

int oracle_decode_absorbed(const oracle_dims *d, const void *q_nope, const void *q_rope,
                           const void *w_uk, const void *w_uv, const void *ckv, const void *kpe,
                           const int32_t *seqlens, const int64_t *pairs, int64_t npairs,
                           double *out, double *psum)
{
    return decode_common(absorbed_one, d, q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens,
                         pairs, npairs, out, psum);
}

/*
 * The merged latent of absorbed decode, o[b][h] = sum_n p_n c[b][n] (before
 * the W_UV up-projection), for a list of (b, h) pairs or every pair
 * (b-major) when pairs == NULL.  out is [npairs][dc].
 */
int oracle_decode_latent(const oracle_dims *d, const void *q_nope, const void *q_rope,
                         const void *w_uk, const void *ckv, const void *kpe,
                         const int32_t *seqlens, const int64_t *pairs, int64_t npairs,
                         double *out)
{
    if (check_dims(d) || !out || !seqlens) return 1;
    const int64_t total = pairs ? npairs : d->B * d->H;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t k = 0; k < total; ++k) {
        const int64_t b = pairs ? pairs[2 * k] : k / d->H;
        const int64_t h = pairs ? pairs[2 * k + 1] : k % d->H;
        if (b < 0 || b >= d->B || h < 0 || h >= d->H) { bad = 1; continue; }
        double *qn = malloc(sizeof(double) * (size_t)d->dn);
        double *qr = malloc(sizeof(double) * (size_t)(d->dr > 0 ? d->dr : 1));
        widen_row(q_nope, d->dtype, (b * d->H + h) * d->dn, d->dn, qn);
        widen_row(q_rope, d->dtype, (b * d->H + h) * d->dr, d->dr, qr);
        absorbed_latent(d, qn, qr, w_uk, ckv, kpe, b, h, (int64_t)seqlens[b], out + k * d->dc);
        free(qn); free(qr);
    }
    return bad;
}

/*
 * The attention block's output projection y = W x for every row of x: the
 * linear map from the concatenated head outputs back to the model width
 * (the "mla-from-scratch" reference model's out_proj; the distaisys
 * deep-dive's W_O).  x [B][K] and w [N][K] (row-major, a linear layer's
 * weight layout), each in its own storage type; y [B][N] fp64.
 */
int oracle_output_proj(int64_t B, int64_t K, int64_t N, int32_t dtype_x, const void *x,
                       int32_t dtype_w, const void *w, double *y)
{
    if (B < 0 || K <= 0 || N <= 0 || !y) return 1;
    if ((dtype_x != OR_F64 && dtype_x != OR_F32 && dtype_x != OR_BF16) ||
        (dtype_w != OR_F64 && dtype_w != OR_F32 && dtype_w != OR_BF16)) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < B; ++b) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += widen(w, dtype_w, n * K + k) * widen(x, dtype_x, b * K + k);
            y[b * N + n] = acc;
        }
    return 0;
}

/*
 * Value-side absorption into the output projection ("mla-from-scratch"
 * README, "Absorption, and why RoPE breaks it": attending over the latents
 * and up-projecting once lets W_UV fold into W_O, by associativity):
 *   W_OV[n][h d_c + j] = sum_i W_O[n][h d_v + i] W_UV[h][i][j],
 * so that W_O concat_h(W_UV[h] o_h) = W_OV concat_h(o_h).
 * w_o [N][H d_v], w_uv [H][d_v][d_c] (one storage type); w_ov [N][H d_c] fp64.
 */
int oracle_fold_value_output(int64_t N, int64_t H, int64_t dv, int64_t dc, int32_t dtype,
                             const void *w_o, const void *w_uv, double *w_ov)
{
    if (N <= 0 || H <= 0 || dv <= 0 || dc <= 0 || !w_ov) return 1;
    if (dtype != OR_F64 && dtype != OR_F32 && dtype != OR_BF16) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t j = 0; j < dc; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < dv; ++i)
                    acc += widen(w_o, dtype, n * H * dv + h * dv + i) *
                           widen(w_uv, dtype, (h * dv + i) * dc + j);
                w_ov[n * H * dc + h * dc + j] = acc;
            }
    return 0;
}

/*
 * Query absorption alone: q~[b][h][j] = sum_i W_UK[h][i][j] q_nope[b][h][i]
 * ("DeepSeek MLA Architecture: How It Cuts KV Cache by 93%", section 2).
 * out is [B][H][dc].
 */
int oracle_absorb_q(const oracle_dims *d, const void *q_nope, const void *w_uk, double *out)
{
    if (check_dims(d) || !out) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < d->B * d->H; ++k) {
        const int64_t h = k % d->H;
        for (int64_t j = 0; j < d->dc; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < d->dn; ++i)
                acc += widen(w_uk, d->dtype, (h * d->dn + i) * d->dc + j) *
                       widen(q_nope, d->dtype, k * d->dn + i);
            out[k * d->dc + j] = acc;
        }
    }
    return 0;
}

/*
 * Causal prefill over selected query rows.  T queries per sequence,
 * q_nope [B][T][H][dn], q_rope [B][T][H][dr].  Query t of sequence b sits at
 * position pos = L_b - T + t (the queries are the last T cached rows) and
 * attends to cached rows 0..pos inclusive through `fn`.  A query with
 * pos < 0 (possible when L_b < T) sees no row and its output is zero, as for
 * an empty decode.  rows lists (b, t) pairs; out is [nrows][H][dv].
 */
static int prefill_common(one_fn fn, const oracle_dims *d, int64_t T, const void *q_nope,
                          const void *q_rope, const void *w_uk, const void *w_uv,
                          const void *ckv, const void *kpe, const int32_t *seqlens,
                          const int64_t *rows, int64_t nrows, double *out)
{
    if (check_dims(d) || T <= 0 || !rows || !out || !seqlens) return 1;
    int bad = 0;
    const int64_t work = nrows * d->H;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t k = 0; k < work; ++k) {
        const int64_t r = k / d->H, h = k % d->H;
        const int64_t b = rows[2 * r], t = rows[2 * r + 1];
        if (b < 0 || b >= d->B || t < 0 || t >= T) { bad = 1; continue; }
        const int64_t pos = (int64_t)seqlens[b] - T + t;
        double *qn = malloc(sizeof(double) * (size_t)d->dn);
        double *qr = malloc(sizeof(double) * (size_t)(d->dr > 0 ? d->dr : 1));
        widen_row(q_nope, d->dtype, ((b * T + t) * d->H + h) * d->dn, d->dn, qn);
        widen_row(q_rope, d->dtype, ((b * T + t) * d->H + h) * d->dr, d->dr, qr);
        fn(d, qn, qr, w_uk, w_uv, ckv, kpe, b, h, pos + 1, out + k * d->dv);
        free(qn); free(qr);
    }
    return bad;
}

/*
 * O3 -- naive causal prefill: every query row through the decompress-then-
 * attend definition O1 ("Deep-Dive ...", section 3, with the causal mask).
 */
int oracle_prefill_naive(const oracle_dims *d, int64_t T, const void *q_nope, const void *q_rope,
                         const void *w_uk, const void *w_uv, const void *ckv, const void *kpe,
                         const int32_t *seqlens, const int64_t *rows, int64_t nrows, double *out)
{
    return prefill_common(naive_one, d, T, q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens, rows,
                          nrows, out);
}

/*
 * O5 -- absorbed causal prefill: every query row through the absorbed
 * definition O2 (the query folded through W_UK, attention over the latent
 * rows, one W_UV up-projection), the same associativity that makes absorbed
 * decode exact ("mla-from-scratch" README, "Absorption, and why RoPE breaks
 * it"), applied to T > 1 queries that share one latent cache.
 */
int oracle_prefill_absorbed(const oracle_dims *d, int64_t T, const void *q_nope,
                            const void *q_rope, const void *w_uk, const void *w_uv,
                            const void *ckv, const void *kpe, const int32_t *seqlens,
                            const int64_t *rows, int64_t nrows, double *out)
{
    return prefill_common(absorbed_one, d, T, q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens,
                          rows, nrows, out);
}

/*
 * Rotary position embedding of one d_r-vector at position pos (RoFormer, the
 * rotary embedding the "mla-from-scratch" README cites for its relative
 * position property): consecutive pairs (x_{2i}, x_{2i+1}) are rotated by the
 * angle pos * theta_i, theta_i = base^(-2 i / d_r).  d_r must be even.
 */
void oracle_rope(int64_t dr, const double *x, double pos, double base, double *out)
{
    for (int64_t i = 0; i < dr / 2; ++i) {
        const double theta = pow(base, -2.0 * (double)i / (double)dr);
        const double a = pos * theta;
        const double c = cos(a), s = sin(a);
        const double x0 = x[2 * i], x1 = x[2 * i + 1];
        out[2 * i] = x0 * c - x1 * s;
        out[2 * i + 1] = x0 * s + x1 * c;
    }
}

/*
 * The cache producer for one new token per sequence: the compressed latent
 * c_t = W_DKV h_t ("Deep-Dive ...", section 2: the down-projection of the
 * hidden state) and the decoupled RoPE key k^R_t = RoPE_t(W_KR h_t) (the
 * extra, uncompressed positional channels of the eyestech-mla description,
 * "Key Architectural Highlights", and the "mla-from-scratch" README).  These
 * are the rows the decode step appends to the cache before attending
 * (songhuiming walk-through, MLA step 2).  h is [B][d_model]; W_DKV is
 * [d_c][d_model]; W_KR is [d_r][d_model]; pos[b] is the row's position.
 * Outputs: c [B][d_c] and kr [B][d_r], both fp64.
 */
int oracle_cache_rows(int64_t B, int64_t d_model, int64_t dc, int64_t dr, int32_t dtype,
                      const void *h, const void *w_dkv, const void *w_kr, const int64_t *pos,
                      double base, double *c, double *kr)
{
    if (B < 0 || d_model <= 0 || dc <= 0 || dr < 0 || (dr & 1) || !c || (dr > 0 && !kr)) return 1;
    if (dtype != OR_F64 && dtype != OR_F32 && dtype != OR_BF16) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        double *hb = malloc(sizeof(double) * (size_t)d_model);
        double *raw = malloc(sizeof(double) * (size_t)(dr > 0 ? dr : 1));
        widen_row(h, dtype, b * d_model, d_model, hb);
        for (int64_t j = 0; j < dc; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < d_model; ++k) acc += widen(w_dkv, dtype, j * d_model + k) * hb[k];
            c[b * dc + j] = acc;
        }
        for (int64_t j = 0; j < dr; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < d_model; ++k) acc += widen(w_kr, dtype, j * d_model + k) * hb[k];
            raw[j] = acc;
        }
        if (dr > 0) oracle_rope(dr, raw, (double)pos[b], base, kr + b * dr);
        free(hb); free(raw);
    }
    return 0;
}

/*
 * O4 -- latent-cache size in bytes: one row of d_c + d_r scalars per token
 * per layer per sequence ("mla-from-scratch" README, cache table: MLA is
 * d_c + d_rope = 512 + 64; eyestech-mla description, memory benchmark API).
 */
uint64_t oracle_kv_cache_bytes(int64_t n_layers, int64_t batch, int64_t seq_len,
                               int64_t d_c, int64_t d_r, int64_t bytes_per_elem)
{
    return (uint64_t)n_layers * (uint64_t)batch * (uint64_t)seq_len *
           (uint64_t)(d_c + d_r) * (uint64_t)bytes_per_elem;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
