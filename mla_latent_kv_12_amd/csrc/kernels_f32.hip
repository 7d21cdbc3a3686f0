// kernels_f32.hip -- scalar fp32 kernels for small MLA shapes (any head count,
// latent width up to 1024).  They implement the same steps as the bf16 MFMA
// path -- absorb, split-context attention in latent space with an online
// softmax, fixed-order split merge fused with the W_UV up-projection -- with
// plain fp32 FMA loops, and the naive decompress-then-attend prefill.
//
// The math follows "mla-from-scratch" README, "Absorption, and why RoPE breaks
// it" (content score against the latent, decoupled positional term, value
// side up-projected once at the end) and the distaisys deep-dive, section 3
// (softmax attention), with the running-max rescaling of a split softmax.
#include <hip/hip_runtime.h>
#include <math.h>

#include "mla_internal.h"

namespace mla {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 256;
constexpr int kMaxCols = 4;  // columns per thread: 4 * 256 = 1024 >= d_c, d_v

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b)
{
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

template <typename T>
__device__ __forceinline__ float load_f(const T *p, int64_t i);
template <>
__device__ __forceinline__ float load_f<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_f<uint16_t>(const uint16_t *p, int64_t i)
{
    return bf16_bits_to_f32(p[i]);
}

__device__ __forceinline__ void store_out(void *out, int64_t i, float v, int out_bf16)
{
    if (out_bf16)
        reinterpret_cast<__bf16 *>(out)[i] = static_cast<__bf16>(v);
    else
        reinterpret_cast<float *>(out)[i] = v;
}

// Block-wide max / sum over kThreads threads (fixed combination order).
__device__ float block_max(float v, float *red)
{
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
    return r;
}

__device__ float block_sum(float v, float *red)
{
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < kThreads / 64; ++i) r += red[i];
    return r;
}

// q_abs[b][h][j] = sum_i W_UK[h][i][j] q_nope[b][h][i]
template <typename T>
__global__ __launch_bounds__(kThreads) void absorb_f32_kernel(int H, int dn, int dc,
                                                              const T *q_nope, const T *w_uk,
                                                              float *q_abs)
{
    const int h = blockIdx.y, b = blockIdx.z;
    const int j = blockIdx.x * kThreads + threadIdx.x;
    extern __shared__ float qs[];
    for (int i = threadIdx.x; i < dn; i += kThreads)
        qs[i] = load_f(q_nope, (static_cast<int64_t>(b) * H + h) * dn + i);
    __syncthreads();
    if (j >= dc) return;
    float acc = 0.f;
    const int64_t wbase = static_cast<int64_t>(h) * dn * dc + j;
    for (int i = 0; i < dn; ++i) acc = fmaf(load_f(w_uk, wbase + static_cast<int64_t>(i) * dc), qs[i], acc);
    q_abs[(static_cast<int64_t>(b) * H + h) * dc + j] = acc;
}

// Token range [start, end) of split `sp` of a sequence with L cached rows.
__device__ __forceinline__ void split_range(int L, int S, int sp, int *start, int *end)
{
    const int ntiles = (L + kSplitGranule - 1) / kSplitGranule;
    const int tps = (ntiles + S - 1) / S;
    const int s0 = sp * tps * kSplitGranule;
    *start = s0;
    *end = min(L, s0 + tps * kSplitGranule);
}

// One block per (split, head, sequence): online softmax over the split's
// cached rows, accumulating the softmax-weighted latent rows.
__global__ __launch_bounds__(kThreads) void decode_split_f32_kernel(
    DecodeShape s, const float *q_abs, const float *q_rope, const float *ckv, const float *kpe,
    const int32_t *seqlens, float *part_o, float *part_ml)
{
    const int sp = blockIdx.x, h = blockIdx.y, v = blockIdx.z;  // v = b * T + t: query row
    const int b = v / s.T;
    const int tid = threadIdx.x;
    extern __shared__ float sm[];
    float *qa = sm;                 // [dc]
    float *qr = qa + s.dc;          // [dr]
    float *pt = qr + s.dr;          // [kThreads] scores / probabilities of a tile
    float *red = pt + kThreads;     // [kThreads / 64]

    const int64_t qoff = static_cast<int64_t>(v) * s.H + h;
    for (int j = tid; j < s.dc; j += kThreads) qa[j] = q_abs[qoff * s.dc + j];
    for (int r = tid; r < s.dr; r += kThreads) qr[r] = q_rope[qoff * s.dr + r];

    const int L = query_len(seqlens[b], s.n_max, s.T, v - b * s.T);
    int start, end;
    split_range(L, s.S, sp, &start, &end);

    const float c2 = s.scale * kLog2e;  // scores are kept in log2 units
    float m = -INFINITY, l = 0.f;
    float o[kMaxCols];
#pragma unroll
    for (int i = 0; i < kMaxCols; ++i) o[i] = 0.f;
    const float *cb = ckv + static_cast<int64_t>(b) * s.ckv_sb;
    const float *kb = kpe + static_cast<int64_t>(b) * s.kpe_sb;
    __syncthreads();

    for (int n0 = start; n0 < end; n0 += kThreads) {
        const int n = n0 + tid;
        float sv = -INFINITY;
        if (n < end) {
            const float *crow = cb + static_cast<int64_t>(n) * s.ckv_sn;
            const float *krow = kb + static_cast<int64_t>(n) * s.kpe_sn;
            float dot = 0.f;
            for (int j = 0; j < s.dc; ++j) dot = fmaf(qa[j], crow[j], dot);
            for (int r = 0; r < s.dr; ++r) dot = fmaf(qr[r], krow[r], dot);
            sv = dot * c2;
        }
        const float mt = block_max(sv, red);
        const float m_new = fmaxf(m, mt);
        const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - m_new);
        const float p = (n < end) ? exp2f(sv - m_new) : 0.f;
        pt[tid] = p;
        const float ps = block_sum(p, red);  // also orders the pt[] writes before the reads
        l = l * alpha + ps;
        m = m_new;
        const int cnt = min(kThreads, end - n0);
#pragma unroll
        for (int i = 0; i < kMaxCols; ++i) {
            const int j = tid + i * kThreads;
            if (j < s.dc) {
                float acc = o[i] * alpha;
                for (int t = 0; t < cnt; ++t)
                    acc = fmaf(pt[t], cb[static_cast<int64_t>(n0 + t) * s.ckv_sn + j], acc);
                o[i] = acc;
            }
        }
        __syncthreads();
    }

    const int64_t prow = (static_cast<int64_t>(v) * s.S + sp) * s.H + h;
#pragma unroll
    for (int i = 0; i < kMaxCols; ++i) {
        const int j = tid + i * kThreads;
        if (j < s.dc) part_o[prow * s.dc + j] = o[i];
    }
    if (tid == 0) {
        part_ml[prow * 2 + 0] = m;
        part_ml[prow * 2 + 1] = l;
    }
}

}  // namespace

// Fixed-order merge of the S split partials of one (head, query row) followed
// by out = W_UV[h] o_lat, or (w_uv == nullptr) the merged latent o_lat itself,
// [rows][H][dc].
template <typename TW>
__global__ __launch_bounds__(kThreads) void merge_upproj_generic_kernel(
    int H, int S, int dc, int dv, const float *part_o, const float *part_ml, const TW *w_uv,
    void *out, int out_bf16)
{
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;  // b: query row
    extern __shared__ float sm[];
    float *ol = sm;            // [dc]
    float *wt = ol + dc;       // [S]
    float *red = wt + S;       // [kThreads/64]

    const int64_t base = static_cast<int64_t>(b) * S * H + h;  // row of split 0
    float mx = -INFINITY;
    for (int sp = tid; sp < S; sp += kThreads) mx = fmaxf(mx, part_ml[(base + static_cast<int64_t>(sp) * H) * 2]);
    mx = block_max(mx, red);
    for (int sp = tid; sp < S; sp += kThreads) {
        const float ms = part_ml[(base + static_cast<int64_t>(sp) * H) * 2];
        wt[sp] = (ms == -INFINITY) ? 0.f : exp2f(ms - mx);
    }
    __syncthreads();
    float lsum = 0.f;  // every thread sums in the same ascending order
    for (int sp = 0; sp < S; ++sp)
        if (wt[sp] != 0.f) lsum = fmaf(wt[sp], part_ml[(base + static_cast<int64_t>(sp) * H) * 2 + 1], lsum);
    const float inv = (lsum > 0.f) ? 1.f / lsum : 0.f;
    for (int j = tid; j < dc; j += kThreads) {
        float acc = 0.f;
        for (int sp = 0; sp < S; ++sp)
            if (wt[sp] != 0.f) acc = fmaf(wt[sp], part_o[(base + static_cast<int64_t>(sp) * H) * dc + j], acc);
        ol[j] = acc * inv;
        if (!w_uv) store_out(out, (static_cast<int64_t>(b) * H + h) * dc + j, acc * inv, out_bf16);
    }
    if (!w_uv) return;
    __syncthreads();
    for (int v = tid; v < dv; v += kThreads) {
        const int64_t wrow = (static_cast<int64_t>(h) * dv + v) * dc;
        float acc = 0.f;
        for (int j = 0; j < dc; ++j) acc = fmaf(load_f(w_uv, wrow + j), ol[j], acc);
        store_out(out, (static_cast<int64_t>(b) * H + h) * dv + v, acc, out_bf16);
    }
}

hipError_t launch_merge_upproj_generic(const DecodeShape &s, const DecodeWorkspace &ws,
                                       const void *w_uv, bool w_bf16, void *out, hipStream_t st)
{
    dim3 grid(s.H, s.B * s.T);
    size_t shm = sizeof(float) * (s.dc + s.S + kThreads / 64);
    if (w_bf16)
        merge_upproj_generic_kernel<uint16_t><<<grid, kThreads, shm, st>>>(
            s.H, s.S, s.dc, s.dv, ws.part_o, ws.part_ml, static_cast<const uint16_t *>(w_uv), out,
            s.out_bf16);
    else
        merge_upproj_generic_kernel<float><<<grid, kThreads, shm, st>>>(
            s.H, s.S, s.dc, s.dv, ws.part_o, ws.part_ml, static_cast<const float *>(w_uv), out,
            s.out_bf16);
    return hipGetLastError();
}

hipError_t launch_absorb_f32(int B, int H, int dn, int dc, bool in_bf16, const void *q_nope,
                             const void *w_uk, float *q_abs, hipStream_t st)
{
    dim3 grid((dc + kThreads - 1) / kThreads, H, B);
    size_t shm = sizeof(float) * dn;
    if (in_bf16)
        absorb_f32_kernel<uint16_t><<<grid, kThreads, shm, st>>>(
            H, dn, dc, static_cast<const uint16_t *>(q_nope), static_cast<const uint16_t *>(w_uk), q_abs);
    else
        absorb_f32_kernel<float><<<grid, kThreads, shm, st>>>(
            H, dn, dc, static_cast<const float *>(q_nope), static_cast<const float *>(w_uk), q_abs);
    return hipGetLastError();
}

hipError_t launch_decode_f32(const DecodeShape &s, const float *q_nope, const float *q_rope,
                             const float *w_uk, const float *w_uv, const float *ckv,
                             const float *kpe, const int32_t *seqlens, void *out,
                             const DecodeWorkspace &ws, hipStream_t st, hipEvent_t const *events)
{
    float *qabs = static_cast<float *>(ws.q);
    const int rows = s.B * s.T;  // query rows
    if (events && events[0]) (void)hipEventRecord(events[0], st);
    hipError_t e;
    if (s.q_rope_base > 0.0 && s.dr > 0) {  // rotate the queries' RoPE channels at their positions
        e = launch_rope_q(s.B, s.T, s.H, s.dr, s.n_max, s.q_rope_base, false, seqlens, q_rope,
                          ws.q_rope, st);
        if (e != hipSuccess) return e;
        q_rope = static_cast<const float *>(ws.q_rope);
    }
    e = launch_absorb_f32(rows, s.H, s.dn, s.dc, false, q_nope, w_uk, qabs, st);
    if (e != hipSuccess) return e;
    if (events && events[1]) (void)hipEventRecord(events[1], st);
    {
        dim3 grid(s.S, s.H, rows);
        size_t shm = sizeof(float) * (s.dc + s.dr + kThreads + kThreads / 64);
        decode_split_f32_kernel<<<grid, kThreads, shm, st>>>(s, qabs, q_rope, ckv, kpe, seqlens,
                                                             ws.part_o, ws.part_ml);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (events && events[2]) (void)hipEventRecord(events[2], st);
    e = launch_merge_upproj_generic(s, ws, w_uv, false, out, st);
    if (events && events[3]) (void)hipEventRecord(events[3], st);
    return e;
}

// ---------------------------------------------------------------------------
// Naive causal prefill, fp32: decompress K_nope and V for every cached row,
// then one block per (query, head) attends over the visible rows.
// ---------------------------------------------------------------------------
namespace {

// K[b][n][h][i] = W_UK[h][i] . c[b][n],  V[b][n][h][i] = W_UV[h][i] . c[b][n]
__global__ __launch_bounds__(kThreads) void decompress_f32_kernel(PrefillShape s, const float *w_uk,
                                                                  const float *w_uv, const float *ckv,
                                                                  const int32_t *seqlens, float *K,
                                                                  float *V)
{
    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int L = static_cast<int>(min<int64_t>(max(seqlens[b], 0), s.n_max));
    if (n >= L) return;
    extern __shared__ float cs[];
    const float *crow = ckv + static_cast<int64_t>(b) * s.ckv_sb + static_cast<int64_t>(n) * s.ckv_sn;
    for (int j = threadIdx.x; j < s.dc; j += kThreads) cs[j] = crow[j];
    __syncthreads();
    const int64_t row = (static_cast<int64_t>(b) * s.n_max + n) * s.H + h;
    for (int i = threadIdx.x; i < s.dn + s.dv; i += kThreads) {
        const bool is_k = i < s.dn;
        const float *w = is_k ? w_uk + (static_cast<int64_t>(h) * s.dn + i) * s.dc
                              : w_uv + (static_cast<int64_t>(h) * s.dv + (i - s.dn)) * s.dc;
        float acc = 0.f;
        for (int j = 0; j < s.dc; ++j) acc = fmaf(w[j], cs[j], acc);
        if (is_k)
            K[row * s.dn + i] = acc;
        else
            V[row * s.dv + (i - s.dn)] = acc;
    }
}

__global__ __launch_bounds__(kThreads) void prefill_attn_f32_kernel(PrefillShape s, const float *q_nope,
                                                                    const float *q_rope, const float *kpe,
                                                                    const int32_t *seqlens, const float *K,
                                                                    const float *V, void *out)
{
    const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    extern __shared__ float sm[];
    float *qn = sm;             // [dn]
    float *qr = qn + s.dn;      // [dr]
    float *pt = qr + s.dr;      // [kThreads]
    float *red = pt + kThreads;
    const int64_t qrow = (static_cast<int64_t>(b) * s.T + t) * s.H + h;
    for (int i = tid; i < s.dn; i += kThreads) qn[i] = q_nope[qrow * s.dn + i];
    for (int i = tid; i < s.dr; i += kThreads) qr[i] = q_rope[qrow * s.dr + i];
    const int L = static_cast<int>(min<int64_t>(max(seqlens[b], 0), s.n_max));
    const int nvis = min(L, L - s.T + t + 1);  // rows 0 .. pos inclusive
    const float c2 = s.scale * kLog2e;
    float m = -INFINITY, l = 0.f, o[kMaxCols];
#pragma unroll
    for (int i = 0; i < kMaxCols; ++i) o[i] = 0.f;
    const float *kb = kpe + static_cast<int64_t>(b) * s.kpe_sb;
    __syncthreads();
    for (int n0 = 0; n0 < nvis; n0 += kThreads) {
        const int n = n0 + tid;
        float sv = -INFINITY;
        if (n < nvis) {
            const int64_t row = (static_cast<int64_t>(b) * s.n_max + n) * s.H + h;
            float dot = 0.f;
            for (int i = 0; i < s.dn; ++i) dot = fmaf(qn[i], K[row * s.dn + i], dot);
            const float *krow = kb + static_cast<int64_t>(n) * s.kpe_sn;
            for (int r = 0; r < s.dr; ++r) dot = fmaf(qr[r], krow[r], dot);
            sv = dot * c2;
        }
        const float mt = block_max(sv, red);
        const float m_new = fmaxf(m, mt);
        const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - m_new);
        const float p = (n < nvis) ? exp2f(sv - m_new) : 0.f;
        pt[tid] = p;
        const float ps = block_sum(p, red);
        l = l * alpha + ps;
        m = m_new;
        const int cnt = min(kThreads, nvis - n0);
#pragma unroll
        for (int i = 0; i < kMaxCols; ++i) {
            const int v = tid + i * kThreads;
            if (v < s.dv) {
                float acc = o[i] * alpha;
                for (int u = 0; u < cnt; ++u)
                    acc = fmaf(pt[u], V[((static_cast<int64_t>(b) * s.n_max + n0 + u) * s.H + h) * s.dv + v], acc);
                o[i] = acc;
            }
        }
        __syncthreads();
    }
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
    for (int i = 0; i < kMaxCols; ++i) {
        const int v = tid + i * kThreads;
        if (v < s.dv) store_out(out, qrow * s.dv + v, o[i] * inv, s.out_bf16);
    }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillShape &s, const float *q_nope, const float *q_rope,
                              const float *w_uk, const float *w_uv, const float *ckv,
                              const float *kpe, const int32_t *seqlens, void *out, void *kbuf,
                              void *vbuf, hipStream_t st)
{
    float *K = static_cast<float *>(kbuf), *V = static_cast<float *>(vbuf);
    {
        dim3 grid(static_cast<unsigned>(s.n_max), s.H, s.B);
        decompress_f32_kernel<<<grid, kThreads, sizeof(float) * s.dc, st>>>(s, w_uk, w_uv, ckv,
                                                                            seqlens, K, V);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    dim3 grid(s.T, s.H, s.B);
    size_t shm = sizeof(float) * (s.dn + s.dr + kThreads + kThreads / 64);
    prefill_attn_f32_kernel<<<grid, kThreads, shm, st>>>(s, q_nope, q_rope, kpe, seqlens, K, V, out);
    return hipGetLastError();
}

}  // namespace mla
