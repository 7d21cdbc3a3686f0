/*
 * mla.h -- C ABI of the MI355X (gfx950) Multi-Head Latent Attention library.
 *
 * The library computes MLA decode over a compressed latent KV cache with
 * query absorption, causal prefill both as the naive decompress-then-attend
 * form and in absorbed (latent-space) form, and the cache producer that
 * writes a new token's latent and rotated RoPE key.
 *
 * Notation (the pages' own): each cached token holds a latent row c of d_c
 * scalars and a decoupled-RoPE key k^R of d_r scalars (512 + 64 = 576 for the
 * DeepSeek-V3 shape: "mla-from-scratch" README, cache table, and the
 * eyestech-mla description, "Key Architectural Highlights").  Per head h the
 * up-projections are W_UK[h] in R^{d_n x d_c} and W_UV[h] in R^{d_v x d_c},
 * stored row-major as [H][d_n][d_c] and [H][d_v][d_c], so the decompressed
 * key and value are k = W_UK[h] c and v = W_UV[h] c ("Deep-Dive: Multi-Head
 * Latent Attention (MLA) and Low-Rank KV Cache Compression in DeepSeek-V3",
 * section 2).
 *
 * Conventions shared by every entry point:
 *  - Pointers are DEVICE memory unless a comment says "host".  The caller
 *    owns every buffer; the library never allocates, frees or synchronises.
 *    Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *  - Tensors are row-major and dense unless strides are given.  Cache strides
 *    are in elements.  The latent and RoPE caches may be two views into one
 *    [B][n_max][d_c + d_r] buffer (kpe = ckv + d_c, both row strides d_c+d_r).
 *  - `dtype` is the storage type of q, weights and caches; `out_dtype` that
 *    of the output.  Arithmetic accumulates in fp32.  bf16 values are
 *    produced with round-to-nearest-even.
 *  - `seqlens[b]` (device, int32) is the cached length of sequence b and
 *    counts the current token: the caller appends the new token's latent
 *    and RoPE key before calling (songhuiming "MHA vs MLA" walk-through, MLA
 *    step 2; eyestech-mla quickstart, where the returned cache grows by one
 *    row).  Values are clamped to [0, n_max] on the device; a sequence with
 *    length 0 gets an all-zero output row.  Rows at or beyond the length are
 *    never read, so they may hold anything, NaN included.  With the
 *    environment variable MLA_DEBUG_CHECKS=1 the calls that take seqlens
 *    first copy it to the host (a synchronisation of the stream) and return
 *    MLA_ERR_INVALID_ARG for a value outside [1, n_max] ([tokens, n_max] for
 *    the prefills); without it no call ever waits on the device.
 *  - Functions return an mla_status.  All argument checks run on the host
 *    before any launch; a rejected call enqueues nothing.  MLA_ERR_HIP means
 *    a launch failed to enqueue; faults inside kernels surface at the
 *    caller's next synchronisation.  mla_last_error() gives a per-thread
 *    message for the last failing call.  The library never aborts and no C++
 *    exception crosses this interface.  It may be called from several
 *    threads at once.  Its only mutable global state is the per-device
 *    address table of mla_decode_noalloc's scratch array.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad stride or alignment */
    MLA_ERR_UNSUPPORTED = 2, /* dimensions or dtype outside what the kernels implement   */
    MLA_ERR_WORKSPACE = 3,   /* workspace missing, too small or misaligned                */
    MLA_ERR_HIP = 4          /* the HIP runtime refused a launch                          */
} mla_status;

typedef enum mla_dtype {
    MLA_F32 = 0,
    MLA_BF16 = 1
} mla_dtype;

/*
 * Shape of a decode call.
 *
 * Supported dimensions:
 *  - dtype MLA_F32: any heads >= 1, 1 <= d_c <= 1024, 0 <= d_r <= 256,
 *    1 <= d_n <= 512, 1 <= d_v <= 1024 (scalar fp32 kernels).
 *  - dtype MLA_BF16: d_c = 512, d_r = 64, d_n = 128, d_v = 128 (the
 *    DeepSeek-V2/V3 shape) and heads a multiple of 128 (MFMA kernels; one
 *    workgroup holds 128 heads).  n_max * row stride * 2 bytes of each
 *    cache must stay below 4 GiB per sequence.
 *    Cache pointers must be 16-byte aligned and row strides multiples of 8.
 *  - any dtype: each cache's extent, (batch - 1) * stride_b + n_max *
 *    stride_n elements, stays below 2^60 elements (so that every offset fits
 *    in 64 bits; the same holds for the prefill and cache-append calls).
 * Anything else returns MLA_ERR_UNSUPPORTED: the library refuses a shape it
 * does not implement rather than computing something else (the
 * "mla-from-scratch" README's absorbed model likewise refuses to build from
 * a model it cannot fold correctly).
 */
typedef struct mla_decode_params {
    int64_t batch;        /* B >= 1 sequences                                   */
    int64_t heads;        /* H query heads, all sharing the one latent cache   */
    int64_t d_c;          /* latent width                                      */
    int64_t d_r;          /* decoupled RoPE key width                          */
    int64_t d_n;          /* q_nope / decompressed key width per head          */
    int64_t d_v;          /* value width per head                              */
    int64_t n_max;        /* cache capacity (rows) per sequence                */
    int64_t ckv_stride_b; /* elements between sequences in the latent cache    */
    int64_t ckv_stride_n; /* elements between rows in the latent cache         */
    int64_t kpe_stride_b; /* elements between sequences in the RoPE-key cache  */
    int64_t kpe_stride_n; /* elements between rows in the RoPE-key cache       */
    float softmax_scale;  /* multiplies the full score; 0 -> 1/sqrt(d_n + d_r) */
    int32_t dtype;        /* mla_dtype of q_nope, q_rope, weights and caches   */
    int32_t out_dtype;    /* mla_dtype of out                                   */
    int32_t num_splits;   /* context splits per sequence; 0 -> chosen by the
                             library (bf16: from the actual lengths, below)    */
    double q_rope_base;   /* 0: q_rope arrives rotated for its position; > 1:
                             the library rotates it (see below) with this base */
} mla_decode_params;

/*
 * Query-side rotary embedding (q_rope_base > 1).  The query of sequence b at
 * position p has its q_rope rotated before use: consecutive pairs (2i, 2i+1)
 * turn by p * theta_i, theta_i = q_rope_base^(-2i/d_r) (RoFormer, the rotary
 * embedding the "mla-from-scratch" README cites; the same convention as the
 * key rotation of mla_cache_append).  The position is that of the query's own
 * cache row: p = L_b - 1 for decode and p = L_b - T + t for query t of a
 * prefill (L_b clamped to [0, n_max]).  Angles are formed and the rotation
 * applied in fp64; the rotated vector is rounded to `dtype` and used in
 * place of q_rope.  A query with p < 0 sees no key and gets a zero row.  d_r
 * must be even.  With keys written by mla_cache_append at their row index,
 * the positional score term then depends only on the distance between the
 * query's row and the key's row (RoFormer's relative-position property).
 */

/*
 * Query absorption: q_abs[b][h][:] = W_UK[h]^T q_nope[b][h][:]
 * ("DeepSeek MLA Architecture: How It Cuts KV Cache by 93%", section 2, the
 * absorbed query; "mla-from-scratch" README, "Absorption, and why RoPE
 * breaks it": the content score q . (W_UK c) equals (W_UK^T q) . c).
 *   q_nope [B][H][d_n] (dtype), w_uk [H][d_n][d_c] (dtype),
 *   q_abs  [B][H][d_c] fp32, written.
 * Only batch, heads, d_c, d_n and dtype of `p` are read.
 */
mla_status mla_absorb_q(const mla_decode_params *p, const void *q_nope, const void *w_uk,
                        float *q_abs, void *stream);

/*
 * Context splits (host function; 0 if `p` is invalid).  With p->num_splits
 * set, every sequence is cut into that many equal ranges of 32-row tiles.
 * With num_splits = 0 the fp32 path picks one count for all sequences from
 * the batch, head count and n_max; the bf16 path builds a balanced plan on
 * the device from the seqlens values (its first kernel): every sequence is
 * cut into ranges of at most C tiles, C the smallest width of at least 4
 * tiles that keeps the whole call within 256 / (heads / 128) ranges (one
 * workgroup per compute unit), so long and short sequences share the chip
 * evenly; sequences are never cut into more than 256 ranges, and when there
 * are that many sequences or more each is one range.  For that plan this
 * function returns the ranges a sequence gets when every sequence holds
 * n_max rows.
 */
int mla_decode_num_splits(const mla_decode_params *p);

/*
 * Bytes of device workspace mla_decode needs for `p` (host function; 0 if
 * `p` is invalid).  The size depends on batch, heads, n_max, dims and the
 * split count, never on the seqlens values.
 */
size_t mla_decode_workspace_bytes(const mla_decode_params *p);

/*
 * Absorbed MLA decode, one new query token per sequence:
 *   q~      = W_UK[h]^T q_nope[b][h]
 *   s_n     = scale * (q~ . c[b][n] + q_rope[b][h] . k^R[b][n]),  n < L_b
 *   p_n     = softmax_n(s)
 *   o       = sum_n p_n c[b][n]            (attention in latent space)
 *   out     = W_UV[h] o                    (one up-projection at the end)
 * which equals softmax attention over the decompressed keys
 * [W_UK[h] c_n ; k^R_n] and values W_UV[h] c_n ("mla-from-scratch" README,
 * "Absorption, and why RoPE breaks it"; distaisys deep-dive, section 3).
 *   q_nope    [B][H][d_n]  dtype
 *   q_rope    [B][H][d_r]  dtype (rotated for the query's position, or
 *             rotated here when q_rope_base > 1, see above)
 *   w_uk      [H][d_n][d_c], w_uv [H][d_v][d_c]  dtype
 *   ckv_cache latent rows, element (b, n, j) at b*ckv_stride_b + n*ckv_stride_n + j
 *   kpe_cache RoPE keys, rotated for their rows (as mla_cache_append writes
 *             them), likewise with the kpe strides
 *   seqlens   [B] int32 (see the conventions above)
 *   out       [B][H][d_v]  out_dtype, written
 *   workspace >= mla_decode_workspace_bytes(p) bytes, 256-byte aligned;
 *             scratch owned by the caller, contents not preserved.
 * Results are bitwise reproducible for the same arguments and seqlens
 * values (fixed-order reduction, no floating-point atomics).  Under the bf16
 * balanced plan a sequence's cut points depend on the other sequences'
 * lengths too, so its result can change in the last bits with theirs; a
 * fixed num_splits makes each sequence's result depend on its own data only.
 */
mla_status mla_decode(const mla_decode_params *p, const void *q_nope, const void *q_rope,
                      const void *w_uk, const void *w_uv, const void *ckv_cache,
                      const void *kpe_cache, const int32_t *seqlens, void *out,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * mla_decode with stage timing: identical work and results, and in addition
 * records caller-created HIP events (hipEvent_t, host array of 4 handles, or
 * NULL for none) on `stream`: events[0] before the absorb kernel, events[1]
 * between absorb and the split-KV attention kernel, events[2] between that
 * kernel and the merge/up-projection kernel, events[3] after the last
 * kernel; a NULL entry skips that record.  For benchmarks that time the
 * attention kernel on its own (each record between two kernels idles the
 * GPU for a few microseconds, so a benchmark records only the events it
 * reads).
 */
mla_status mla_decode_profiled(const mla_decode_params *p, const void *q_nope,
                               const void *q_rope, const void *w_uk, const void *w_uv,
                               const void *ckv_cache, const void *kpe_cache,
                               const int32_t *seqlens, void *out, void *workspace,
                               size_t workspace_bytes, void *stream, void *const *events);

/*
 * Largest workspace, in bytes, that mla_decode_noalloc serves (80 MiB: the
 * DeepSeek-V3 shape at batch 8 and 131072 cached tokens per sequence with
 * the library's split count needs 67.4 MiB).
 */
#define MLA_DECODE_NOALLOC_MAX_BYTES ((size_t)80 << 20)

/*
 * mla_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments without `workspace` / `workspace_bytes`, the same
 * kernels and bitwise the same results as mla_decode with the same split
 * count.  The workspace is a device array inside the library, of
 * MLA_DECODE_NOALLOC_MAX_BYTES, that each GPU the library runs on holds
 * until the process ends; its address on the current device is looked up
 * on the first call there (`stream` must belong to the current device).
 * No call allocates, frees or synchronises.
 *   Returns MLA_ERR_WORKSPACE, before any launch, when
 *   mla_decode_workspace_bytes(p) exceeds MLA_DECODE_NOALLOC_MAX_BYTES
 *   (fewer sequences or context splits fit), and MLA_ERR_HIP when the
 *   array's address cannot be looked up.
 *   Every call on one GPU shares that GPU's array, and the kernels need
 *   nothing of its previous contents: calls that overlap in time on one GPU
 *   (on different streams, or from several threads) race on it and must be
 *   ordered by the caller.
 */
mla_status mla_decode_noalloc(const mla_decode_params *p, const void *q_nope,
                              const void *q_rope, const void *w_uk, const void *w_uv,
                              const void *ckv_cache, const void *kpe_cache,
                              const int32_t *seqlens, void *out, void *stream);

/*
 * Shape of a naive causal prefill call: T new query tokens per sequence,
 * which are the last T of the L_b cached rows (L_b >= T).
 * Supported: dtype MLA_BF16 with d_c = 512, d_r = 64, d_n = 128, d_v = 128,
 * heads >= 1, tokens >= 1; dtype MLA_F32 with the fp32 decode limits.
 */
typedef struct mla_prefill_params {
    int64_t batch;
    int64_t tokens;       /* T query tokens per sequence                       */
    int64_t heads;
    int64_t d_c, d_r, d_n, d_v;
    int64_t n_max;        /* cache capacity (rows) per sequence, >= tokens     */
    int64_t ckv_stride_b, ckv_stride_n, kpe_stride_b, kpe_stride_n;
    float softmax_scale;  /* 0 -> 1/sqrt(d_n + d_r)                             */
    int32_t dtype;
    int32_t out_dtype;
    int32_t num_splits;   /* mla_prefill_absorbed: context splits per query row,
                             0 -> chosen by the library (as for decode, each
                             query row a sequence); mla_prefill_naive: 0     */
    double q_rope_base;   /* 0: q_rope arrives rotated; > 1: rotated by the
                             library at each query's position (see above)     */
} mla_prefill_params;

/* Bytes of device workspace mla_prefill_naive needs (host; 0 if invalid). */
size_t mla_prefill_workspace_bytes(const mla_prefill_params *p);

/*
 * Naive causal prefill: decompress every cached latent row into the key and
 * value of every head, K_nope = W_UK[h] c[b][n] and V = W_UV[h] c[b][n] (kept
 * in the workspace, i.e. materialised in HBM on purpose, in a layout private
 * to the library), then for query t at
 * position pos = L_b - T + t attend over rows n <= pos with keys
 * [K_nope ; k^R] and values V (distaisys deep-dive, section 3, with a causal
 * mask that includes the diagonal; songhuiming walk-through, MLA step 2).
 *   q_nope [B][T][H][d_n], q_rope [B][T][H][d_r]   dtype
 *   w_uk, w_uv, ckv_cache, kpe_cache, seqlens        as for mla_decode
 *   out    [B][T][H][d_v]                            out_dtype, written
 * L_b is clamped to [0, n_max] on the device.  If L_b < T the leading
 * queries get pos < 0, see no key, and their output rows are zero.
 */
mla_status mla_prefill_naive(const mla_prefill_params *p, const void *q_nope,
                             const void *q_rope, const void *w_uk, const void *w_uv,
                             const void *ckv_cache, const void *kpe_cache,
                             const int32_t *seqlens, void *out, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Context splits per query row that mla_prefill_absorbed will use (host;
 * 0 if `p` is invalid), as mla_decode_num_splits: for the bf16 plan, those
 * of a query row when every sequence holds n_max rows. */
int mla_prefill_absorbed_num_splits(const mla_prefill_params *p);

/* Bytes of device workspace mla_prefill_absorbed needs (host; 0 if invalid).
 * Depends on batch, tokens, heads, dims and the split count. */
size_t mla_prefill_absorbed_workspace_bytes(const mla_prefill_params *p);

/*
 * Absorbed causal prefill (chunked prefill in latent space): the T new
 * queries of each sequence, the last T of its L_b cached rows, attend to the
 * latent cache directly, each exactly as an absorbed decode over its causal
 * prefix: for query t at position pos = L_b - T + t,
 *   q~  = W_UK[h]^T q_nope[b][t][h]
 *   s_n = scale * (q~ . c[b][n] + q_rope[b][t][h] . k^R[b][n]),  n <= pos
 *   out[b][t][h] = W_UV[h] sum_n softmax_n(s) c[b][n]
 * The associativity that makes absorbed decode exact ("mla-from-scratch"
 * README, "Absorption, and why RoPE breaks it") applied to T > 1 queries
 * sharing one cache; no key or value is decompressed, so the cost grows with
 * T x L_b at 2 (2 d_c + d_r) flop per (query, key, head) and the cache is
 * read as for decode.  It pays when T is small beside L_b (a chunk appended
 * to a long context); for a whole prompt the naive path does fewer flops.
 *   Arguments, layouts and the causal alignment as for mla_prefill_naive;
 *   workspace >= mla_prefill_absorbed_workspace_bytes(p), 256-byte aligned.
 * Supported: the decode limits (dtype MLA_BF16: the V3 widths and heads a
 * multiple of 128; MLA_F32: the fp32 limits), batch * tokens <= 65535.
 * Results are reproducible as for mla_decode; a query with pos < 0 gets a
 * zero row.
 */
mla_status mla_prefill_absorbed(const mla_prefill_params *p, const void *q_nope,
                                const void *q_rope, const void *w_uk, const void *w_uv,
                                const void *ckv_cache, const void *kpe_cache,
                                const int32_t *seqlens, void *out, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * Absorbed decode up to the merged latent: the same call as mla_decode
 * without the final up-projection, writing
 *   o_lat[b][h][:] = sum_n p_n c[b][n]      (d_c values, out_dtype)
 * the attention output in latent space, for a caller that folds W_UV into
 * its output projection ("mla-from-scratch" README, "Absorption, and why
 * RoPE breaks it": attending over the latents and up-projecting once lets
 * W_UV fold into W_O).  W_UV is not an argument; p->d_v is ignored.  The
 * workspace is mla_decode_workspace_bytes(p).  Other arguments, checks and
 * reproducibility as for mla_decode.
 */
mla_status mla_decode_latent(const mla_decode_params *p, const void *q_nope, const void *q_rope,
                             const void *w_uk, const void *ckv_cache, const void *kpe_cache,
                             const int32_t *seqlens, void *o_lat, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * Shape of an output projection y = x W^T: batch rows of in_features
 * values each, against a weight of out_features rows.
 * Supported: dtype MLA_BF16 (x and w; in_features a multiple of 64, x and w
 * 16-byte aligned; MFMA path) or MLA_F32 (any in_features); out_dtype either.
 */
typedef struct mla_proj_params {
    int64_t batch;         /* B rows of x                                        */
    int64_t in_features;   /* K: H * d_v (unfolded) or H * d_c (W_UV folded in)  */
    int64_t out_features;  /* N: the model width                                 */
    int32_t dtype;         /* mla_dtype of x and w                               */
    int32_t out_dtype;     /* mla_dtype of y                                     */
    int32_t num_splits;    /* slices of K summed in a fixed order; 0 -> by size */
                           /* (bf16 with N >= 2048: the direct form, below)    */
    int32_t reserved;      /* must be 0                                          */
} mla_proj_params;

/* Bytes of device workspace mla_output_proj needs (host): the fp32 partial
 * sums of every K slice.  0 when the call needs none (the direct form) or
 * when p is invalid; mla_output_proj validates p itself before any launch. */
size_t mla_output_proj_workspace_bytes(const mla_proj_params *p);

/*
 * The attention block's output projection, the step after decode:
 *   y[b][n] = sum_k x[b][k] w[n][k]
 * with x the concatenated head outputs ([B][H][d_v] from mla_decode is
 * [B][H * d_v]) and w = W_O [d_model][H * d_v] (row-major, a linear layer's
 * weight), or x the merged latents of mla_decode_latent ([B][H * d_c]) and
 * w = W_OV from mla_fold_value_output ("mla-from-scratch" reference model,
 * out_proj; "Absorption, and why RoPE breaks it" for the folded form).
 *   x [B][K], w [N][K] dtype; y [B][N] out_dtype, written.
 * Dot products accumulate in fp32 over slices of K whose partial sums are
 * added in ascending slice order: bitwise reproducible for a fixed split
 * count.  workspace >= mla_output_proj_workspace_bytes(p), 256-byte aligned
 * (may be NULL when that is 0).
 * Direct form (bf16, num_splits = 0, N >= 2048): each workgroup takes R =
 * min(32, ceil(N / 256)) rows over all of K, its 8 waves' eighths of K added
 * in a fixed order: one launch, no workspace, bitwise reproducible.
 */
mla_status mla_output_proj(const mla_proj_params *p, const void *x, const void *w, void *y,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Value-side absorption of the weights (a one-off transform, not per step):
 *   w_ov[n][h * d_c + j] = sum_i w_o[n][h * d_v + i] w_uv[h][i][j]
 * so that W_O concat_h(W_UV[h] o_h) = W_OV concat_h(o_h) by associativity
 * ("mla-from-scratch" README, "Absorption, and why RoPE breaks it").
 *   w_o [d_model][heads * d_v], w_uv [heads][d_v][d_c] (dtype), w_ov
 *   [d_model][heads * d_c] (dtype), written; fp32 accumulation, bf16 results
 *   rounded to nearest even.
 * At the V3 shape W_OV holds 4x the bytes of W_UV and W_O together (d_c =
 * 512 > d_v = 128), so for decode the unfolded pair is the cheaper one; the
 * folded form is offered for callers that want the single product.
 */
mla_status mla_fold_value_output(int64_t d_model, int64_t heads, int64_t d_v, int64_t d_c,
                                 int32_t dtype, const void *w_o, const void *w_uv, void *w_ov,
                                 void *stream);

/*
 * Shape of a cache-append call: one new token per sequence.
 * Supported: dtype MLA_BF16 or MLA_F32 (every tensor the same), d_c >= 2 and
 * even, d_r >= 0 and even, d_model a multiple of 8 (bf16) or 4 (fp32).
 */
typedef struct mla_append_params {
    int64_t batch;
    int64_t d_model;      /* width of the hidden state h                        */
    int64_t d_c, d_r;
    int64_t n_max;        /* cache capacity (rows) per sequence                 */
    int64_t ckv_stride_b, ckv_stride_n, kpe_stride_b, kpe_stride_n;  /* elements */
    double rope_base;     /* rotary base; 0 -> 10000                            */
    int32_t dtype;        /* MLA_BF16 or MLA_F32                                */
    int32_t reserved;     /* must be 0                                          */
} mla_append_params;

/*
 * The cache producer, the step before decode: for every sequence b whose
 * positions[b] lies in [0, n_max), write the new token's cache row
 *   ckv_cache[b][positions[b]] = W_DKV h_b            (d_c values)
 *   kpe_cache[b][positions[b]] = RoPE_pos(W_KR h_b)   (d_r values)
 * ("Deep-Dive: Multi-Head Latent Attention (MLA) and Low-Rank KV Cache
 * Compression in DeepSeek-V3", section 2: c_t = W_DKV h_t; eyestech-mla
 * description, "Key Architectural Highlights": the decoupled RoPE key stored
 * beside the latent; songhuiming walk-through, MLA step 2: the new latent is
 * appended before attending).  RoPE rotates consecutive pairs (2i, 2i+1) by
 * the angle pos * theta_i, theta_i = rope_base^(-2i/d_r) (RoFormer, the
 * rotary embedding the "mla-from-scratch" README cites).
 *   h         [B][d_model]     dtype
 *   w_dkv     [d_c][d_model]   dtype (row-major)
 *   w_kr      [d_r][d_model]   dtype (row-major; may be NULL when d_r == 0)
 *   positions [B] int32, device memory
 *   ckv_cache, kpe_cache: strided as for mla_decode, one row written per
 *             sequence (they may be the two views of one [B][n_max][d_c+d_r]
 *             buffer)
 * No other row is touched; a position outside [0, n_max) writes nothing for
 * its sequence.  Dot products accumulate in fp32, rotation angles are
 * formed in fp64; bf16 results are rounded to nearest even.
 */
mla_status mla_cache_append(const mla_append_params *p, const void *h, const void *w_dkv,
                            const void *w_kr, const int32_t *positions, void *ckv_cache,
                            void *kpe_cache, void *stream);

/*
 * Latent-cache size (host): n_layers * batch * seq_len * (d_c + d_r) *
 * bytes_per_elem; 576 scalars per token per layer at the V3 shape
 * (eyestech-mla description, programmatic memory benchmark API).  Returns 0
 * for negative arguments.
 */
uint64_t mla_kv_cache_bytes(int64_t n_layers, int64_t batch, int64_t seq_len, int64_t d_c,
                            int64_t d_r, int64_t bytes_per_elem);

/* Static text for a status code (host). */
const char *mla_status_string(mla_status s);

/* Per-thread message describing the last failing call on this thread (host);
 * an empty string if none failed.  Valid until the next call on the thread. */
const char *mla_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
