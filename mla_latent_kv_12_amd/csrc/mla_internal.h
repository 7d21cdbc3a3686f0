// mla_internal.h -- declarations shared by the library's own translation units
// (host API <-> kernel launchers).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Token granularity at which a sequence is cut into context splits.  Both the
// fp32 and the bf16 decode kernels use it, so a split boundary never falls
// inside an MFMA token tile.
constexpr int kSplitGranule = 32;
constexpr int kMaxSplits = 256;

// A decode call, or an absorbed prefill of T query tokens per sequence.  The
// kernels see B * T query rows ("virtual sequences" v = b * T + t); row v
// reads the cache of sequence b = v / T and attends to its first
// clamp(L_b) - (T - 1 - t) rows (the causal prefix of query t).  T = 1 is
// plain decode.
struct DecodeShape {
    int B, T, H, dc, dr, dn, dv;
    int64_t n_max;
    int64_t ckv_sb, ckv_sn, kpe_sb, kpe_sn;
    float scale;         // softmax scale (natural-log units)
    // fp32 path: context splits per query row.  bf16 path: the caller's fixed
    // split count, or 0 for the balanced work plan (see items).
    int S;
    // bf16 path: work items the split-KV launch covers (its grid), each a
    // range of one query row's tiles; the partials are stored per item.
    int items;
    int out_bf16;        // output stored as bf16 (else fp32)
    double q_rope_base;  // > 0: rotate q_rope at each query's position first
};

// The bf16 split-KV work plan.  With a fixed split count S every query row is
// cut into S equal tile ranges (items v * S .. v * S + S - 1).  Without one,
// each row is cut into ranges of at most C tiles, C the smallest width (at
// least kPlanMinTiles) for which the whole call needs no more than
// kPlanTargetItems / head groups items (one workgroup per compute unit); a
// row's items are consecutive, in ascending tile order.
// Rows that cannot be held to that budget (as many active rows as items, or
// more) get one item each.  A row never gets more than kMaxSplits items.
constexpr int kPlanTargetItems = 256;
constexpr int kPlanMinTiles = 4;
__host__ __device__ inline int plan_target(int H)
{
    const int groups = H / 128 > 0 ? H / 128 : 1;
    return kPlanTargetItems / groups > 0 ? kPlanTargetItems / groups : 1;
}
// Items the split-KV grid covers: fixed split count, or the plan's bound.
inline int64_t plan_capacity(int64_t rows, int H, int fixed_S)
{
    if (fixed_S > 0) return rows * fixed_S;
    return rows > plan_target(H) ? rows : plan_target(H);
}
// Search interval of the plan's width C (tiles per item) when 0 < active <
// target (tiles = sum of the rows' tile counts nt_v, max_nt their maximum).
// Every C in it keeps a row at kMaxSplits items or fewer, and C = hi meets
// the budget: sum_v ceil(nt_v / C) <= tiles / C + active <= target for
// C >= tiles / (target - active), and the sum is active for C >= max_nt.
// The item count only falls as C grows, so the plan takes the smallest C in
// [lo, hi] that meets the budget by bisection.
__host__ __device__ inline void plan_bounds(int64_t tiles, int active, int max_nt, int target,
                                            int *lo, int *hi)
{
    int64_t l = (tiles + target - 1) / target;
    const int64_t per_row = (static_cast<int64_t>(max_nt) + kMaxSplits - 1) / kMaxSplits;
    if (l < kPlanMinTiles) l = kPlanMinTiles;
    if (l < per_row) l = per_row;
    const int64_t room = target - active;
    int64_t h = (tiles + room - 1) / room;
    if (h > max_nt) h = max_nt;  // C >= max_nt: one item per active row, also within budget
    if (h < l) h = l;
    *lo = static_cast<int>(l);
    *hi = static_cast<int>(h);
}

// Workspace carving, identical for the fp32 and bf16 paths except for the
// query buffer's element type and width.  Rows are the B * T query rows.
struct DecodeWorkspace {
    void *q;          // bf16 path: [rows][H][dc+dr] bf16 pre-absorbed query; fp32: [rows][H][dc] fp32
    float *part_o;    // fp32: [rows][S][H][dc]; bf16: [items][H][dc]  un-normalised latent sums
    float *part_ml;   // fp32: [rows][S][H][2];  bf16: [items][H][2]   reference max (log2) and mass
    void *q_rope;     // fp32 path with q rotation: [rows][H][dr] q_rope rotated at its position
    float *o_lat;     // bf16 path with many query rows: [rows][H][dc] merged latents
    int *plan_items;  // bf16 path: [items][4] query row (-1: unused), first tile, end tile, 0
    int *plan_rows;   // bf16 path: [rows][2] first item, item count
};

// With many (query row, head) pairs (a decode batch of 8 or more at 128
// heads, an absorbed prefill) the bf16 path merges into fp32 latents and
// up-projects them with one batched product per head, instead of re-reading
// W_UV[h] for every query row.
inline bool batched_upproj(const DecodeShape &s, bool bf16)
{
    return bf16 && static_cast<int64_t>(s.B) * s.T * s.H >= 1024;
}

size_t decode_workspace_layout(const DecodeShape &s, bool bf16, DecodeWorkspace *ws_or_null,
                               void *base);

// Rows visible to query t of a sequence with `seqlen` cached rows (clamped to
// [0, n_max]) when its T queries are the last T rows: the causal prefix up to
// and including the query's own row, L - (T - 1 - t), or none.
__device__ __forceinline__ int query_len(int32_t seqlen, int64_t n_max, int T, int t)
{
    const int L = static_cast<int>(min<int64_t>(max(seqlen, 0), n_max));
    return max(L - (T - 1 - t), 0);
}

// fp32 path (any supported small shape)
hipError_t launch_absorb_f32(int B, int H, int dn, int dc, bool in_bf16, const void *q_nope,
                             const void *w_uk, float *q_abs, hipStream_t st);
hipError_t launch_decode_f32(const DecodeShape &s, const float *q_nope, const float *q_rope,
                             const float *w_uk, const float *w_uv, const float *ckv,
                             const float *kpe, const int32_t *seqlens, void *out,
                             const DecodeWorkspace &ws, hipStream_t st,
                             hipEvent_t const *events);

// Fixed-order split merge + W_UV up-projection (scalar; any shape).
hipError_t launch_merge_upproj_generic(const DecodeShape &s, const DecodeWorkspace &ws,
                                       const void *w_uv, bool w_bf16, void *out, hipStream_t st);

// bf16 MFMA path (d_c = 512, d_r = 64, d_n = d_v = 128, H % 128 == 0)
// `events` (may be null): 4 hipEvent_t recorded before, between and after
// the three kernels.
hipError_t launch_decode_bf16(const DecodeShape &s, const void *q_nope, const void *q_rope,
                              const void *w_uk, const void *w_uv, const void *ckv,
                              const void *kpe, const int32_t *seqlens, void *out,
                              const DecodeWorkspace &ws, hipStream_t st,
                              hipEvent_t const *events);
int decode_bf16_heads_per_block(int H);

struct PrefillShape {
    int B, T, H, dc, dr, dn, dv;
    int64_t n_max;
    int64_t ckv_sb, ckv_sn, kpe_sb, kpe_sn;
    float scale;
    int out_bf16;
    double q_rope_base;  // > 0: rotate q_rope at each query's position first
};
// K, V and (when rotating) the rotated q_rope [B][T][H][dr] in the workspace.
size_t prefill_workspace_layout(const PrefillShape &s, bool bf16, void *base, void **k_out,
                                void **v_out, void **qr_out);

// Rotary embedding of the queries: out[v][h] = RoPE_p(q_rope[v][h]) for the
// rows = B * T query rows v = b * T + t at position p = clamp(L_b) - T + t,
// pairs (2i, 2i+1) turned by p * base^(-2i/dr) in fp64 and rounded to the
// storage type; rows with p < 0 are copied unrotated.
hipError_t launch_rope_q(int B, int T, int H, int dr, int64_t n_max, double base, bool bf16,
                         const int32_t *seqlens, const void *q_rope, void *out, hipStream_t st);
hipError_t launch_prefill_f32(const PrefillShape &s, const float *q_nope, const float *q_rope,
                              const float *w_uk, const float *w_uv, const float *ckv,
                              const float *kpe, const int32_t *seqlens, void *out, void *kbuf,
                              void *vbuf, hipStream_t st);
hipError_t launch_prefill_bf16(const PrefillShape &s, const void *q_nope, const void *q_rope,
                               const void *w_uk, const void *w_uv, const void *ckv,
                               const void *kpe, const int32_t *seqlens, void *out, void *kbuf,
                               void *vbuf, hipStream_t st);

// Output projection y[B][N] = x[B][K] w[N][K]^T, K cut into S slices, or
// (R > 0, bf16 only) the direct form: R rows per workgroup over all of K.
struct ProjShape {
    int B, K, N, S;
    int R;          // > 0: direct form with R <= 32 rows per workgroup (S = 1, no partials)
    bool bf16;      // x and w bf16 (MFMA path; K % 64 == 0), else fp32
    int out_bf16;
};
// part: S * B * N fp32 of workspace (none for the direct form).
hipError_t launch_output_proj(const ProjShape &p, const void *x, const void *w, void *y,
                              float *part, hipStream_t st);
hipError_t launch_fold_value_output(int N, int H, int dv, int dc, bool bf16, const void *w_o,
                                    const void *w_uv, void *w_ov, hipStream_t st);

struct AppendShape {
    int B, d_model, dc, dr;
    int64_t n_max;
    int64_t ckv_sb, ckv_sn, kpe_sb, kpe_sn;
    double rope_base;
    bool bf16;
};
hipError_t launch_cache_append(const AppendShape &s, const void *h, const void *w_dkv,
                               const void *w_kr, const int32_t *positions, void *ckv,
                               void *kpe, hipStream_t st);

}  // namespace mla
