// outproj.hip -- the value side after attention: the output projection
// y = W x of the concatenated head outputs (the linear map from H * d_v back
// to the model width; the "mla-from-scratch" reference model's out_proj), and
// the one-off weight transform that folds W_UV into it (value-side
// absorption, "mla-from-scratch" README, "Absorption, and why RoPE breaks
// it"): W_OV[n][h d_c + j] = sum_i W_O[n][h d_v + i] W_UV[h][i][j], so that
// W_O concat_h(W_UV[h] o_h) = W_OV concat_h(o_h).
//
// The projection for a decode batch is a skinny product: a few query rows
// against a weight of d_model rows, HBM-bound on the weight.  bf16 path:
// v_mfma_f32_32x32x16_bf16 with the weight rows as the A operand straight
// from global memory (each weight byte read once) and the batch rows as the
// B operand (batch padded to the MFMA's 32 columns); the K range is cut into
// slices so that thousands of waves stream the weight, each slice's partial
// sums are written as fp32 and a second kernel adds the slices in ascending
// order (bitwise repeatable).
#include <hip/hip_runtime.h>

#include "cdna4.h"
#include "mla_internal.h"

namespace mla {
namespace {

using namespace cdna4;

constexpr int kPWaves = 4;            // waves per workgroup, splitting the slice's K steps
constexpr int kPRows = 64;            // weight rows per workgroup (two 32-row MFMA tiles)
constexpr int kPUnroll = 4;           // K steps (16 each) of loads in flight per lane
constexpr int kPBatch = 32;           // batch rows per pass (the MFMA's N)

// K range [k0, k1) of slice s when K is cut into S slices of whole 64-element
// units (the workgroup's four waves then take whole 16-element steps).
__device__ __forceinline__ void slice_range(int K, int S, int s, int *k0, int *k1)
{
    const int units = K / 64;
    *k0 = 64 * static_cast<int>((static_cast<int64_t>(units) * s) / S);
    *k1 = 64 * static_cast<int>((static_cast<int64_t>(units) * (s + 1)) / S);
}

// part[s][b][n] = sum_{k in slice s} w[n][k] x[b][k] for the workgroup's 64
// rows n and the batch group's 32 rows b.  Grid (ceil(N / 64), S, ceil(B / 32)).
__global__ __launch_bounds__(64 * kPWaves) void rowproj_bf16_kernel(
    int B, int K, int N, int S, const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
    float *__restrict__ part)
{
    __shared__ f32x4 red[kPWaves][2][4][64];  // per wave: 2 tiles x 16 values per lane
    const int n0 = blockIdx.x * kPRows, s = blockIdx.y, b0 = blockIdx.z * kPBatch;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int half = lane >> 5, l32 = lane & 31;
    int k0, k1;
    slice_range(K, S, s, &k0, &k1);
    // this wave's share of the slice's 16-element steps, as a contiguous range
    const int steps = (k1 - k0) / 16;
    const int st0 = k0 / 16 + (steps * wv) / kPWaves, st1 = k0 / 16 + (steps * (wv + 1)) / kPWaves;

    // A operand: weight row n0 + 32 t + l32 (clamped inside the weight),
    // elements 8 half .. 8 half + 7 of each step.  B operand: batch row
    // b0 + l32 (zeros past the batch), the same elements.
    const u32x4 *wrow[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
        wrow[t] = reinterpret_cast<const u32x4 *>(w + static_cast<int64_t>(min(n0 + 32 * t + l32, N - 1)) * K) + half;
    const bool xv = b0 + l32 < B;
    const u32x4 *xrow = reinterpret_cast<const u32x4 *>(x + static_cast<int64_t>(xv ? b0 + l32 : 0) * K) + half;

    f32x16 acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // full batches of kPUnroll steps: every load of a batch is issued before
    // the first MFMA that uses it (no per-step branch for the compiler to sink
    // the loads under), then the remaining steps one at a time
    int st = st0;
    for (; st + kPUnroll <= st1; st += kPUnroll) {
        u32x4 wa[kPUnroll][2], xb[kPUnroll];
#pragma unroll
        for (int u = 0; u < kPUnroll; ++u) {
#pragma unroll
            for (int t = 0; t < 2; ++t) wa[u][t] = wrow[t][2 * (st + u)];
            xb[u] = xrow[2 * (st + u)];
        }
#pragma unroll
        for (int u = 0; u < kPUnroll; ++u) {
            const u32x4 bx = xv ? xb[u] : zero;
#pragma unroll
            for (int t = 0; t < 2; ++t) acc[t] = mfma32(wa[u][t], bx, acc[t]);
        }
    }
    for (; st < st1; ++st) {
        const u32x4 w0 = wrow[0][2 * st], w1 = wrow[1][2 * st], xq = xrow[2 * st];
        const u32x4 bx = xv ? xq : zero;
        acc[0] = mfma32(w0, bx, acc[0]);
        acc[1] = mfma32(w1, bx, acc[1]);
    }
    // fixed-order sum of the four waves' partials, then one store per value
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            red[wv][t][g][lane] = f32x4{acc[t][4 * g], acc[t][4 * g + 1], acc[t][4 * g + 2], acc[t][4 * g + 3]};
    __syncthreads();
    // thread -> (tile t, group g, lane) of the wave-0 layout: 2 x 4 x 64 = 512 = 2 per thread
    for (int e = tid; e < 2 * 4 * 64; e += 64 * kPWaves) {
        const int t = e >> 8, g = (e >> 6) & 3, ln = e & 63;
        f32x4 v = red[0][t][g][ln];
#pragma unroll
        for (int q = 1; q < kPWaves; ++q) v += red[q][t][g][ln];
        // lane ln holds batch column ln % 32, rows 8 g + 4 (ln / 32) + 0..3 of tile t
        const int b = b0 + (ln & 31), n = n0 + 32 * t + 8 * g + 4 * (ln >> 5);
        if (b < B) {
            float *dst = part + (static_cast<int64_t>(s) * B + b) * N + n;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (n + i < N) dst[i] = v[i];
        }
    }
}

// Direct form for weights with many rows: workgroup g takes rows
// [g R, g R + R) (R <= 32: one MFMA tile, rows past R or N clamped on load
// and not stored) over the whole of K, its 8 waves taking interleaved
// blocks of 4 16-element steps; the waves' sums are added in LDS in wave
// order and stored in the output type.  No slice partials and no second launch;
// R is chosen so that the row groups cover every CU once.
// Grid (ceil(N / R), ceil(B / 32)).
constexpr int kDWaves = 8;   // waves per workgroup, splitting K
constexpr int kDUnroll = 4;  // K steps (16 each) of loads in flight per lane
__global__ __launch_bounds__(64 * kDWaves) void rowproj_direct_bf16_kernel(
    int B, int K, int N, int R, const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
    void *__restrict__ y, int out_bf16)
{
    __shared__ f32x4 red[kDWaves][4][64];  // per wave: 16 values per lane
    const int n0 = blockIdx.x * R, b0 = blockIdx.y * kPBatch;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int half = lane >> 5, l32 = lane & 31;
    const int steps = K / 16;  // a multiple of kDUnroll: K % 64 == 0

    // A operand: weight row n0 + min(l32, R - 1) (inside the weight);
    // B operand: batch row b0 + l32 (zeros past the batch); elements
    // 8 half .. 8 half + 7 of each step.
    const u32x4 *wrow = reinterpret_cast<const u32x4 *>(
                            w + static_cast<int64_t>(min(n0 + min(l32, R - 1), N - 1)) * K) + half;
    const bool xv = b0 + l32 < B;
    const u32x4 *xrow = reinterpret_cast<const u32x4 *>(x + static_cast<int64_t>(xv ? b0 + l32 : 0) * K) + half;

    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // Wave w takes the blocks of kDUnroll steps b = w, w + 8, ...: at any
    // time the workgroup's 8 waves read neighbouring 128-byte blocks of its
    // rows, one 1-KiB span per row, rather than 8 spans 1/8 of the row
    // apart (that form ran 44 or 66 us per call at the V3 width depending on
    // the process, and 187 us folded, against 44 and 177 us for this one).
    for (int blk = wv; blk * kDUnroll < steps; blk += kDWaves) {
        const int st = blk * kDUnroll;
        u32x4 wa[kDUnroll], xb[kDUnroll];
#pragma unroll
        for (int u = 0; u < kDUnroll; ++u) {
            wa[u] = wrow[2 * (st + u)];
            xb[u] = xrow[2 * (st + u)];
        }
#pragma unroll
        for (int u = 0; u < kDUnroll; ++u) acc = mfma32(wa[u], xv ? xb[u] : zero, acc);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
        red[wv][g][lane] = f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
    __syncthreads();
    // thread -> (group g, lane) of the wave-0 layout: 4 x 64 = 256 entries
    if (tid < 4 * 64) {
        const int g = tid >> 6, ln = tid & 63;
        f32x4 v = red[0][g][ln];
#pragma unroll
        for (int q = 1; q < kDWaves; ++q) v += red[q][g][ln];
        // lane ln holds batch column ln % 32, rows 8 g + 4 (ln / 32) + 0..3 of the tile
        const int b = b0 + (ln & 31), r = 8 * g + 4 * (ln >> 5);
        if (b < B) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = n0 + r + i;
                if (r + i >= R || n >= N) continue;
                const int64_t o = static_cast<int64_t>(b) * N + n;
                if (out_bf16)
                    reinterpret_cast<__bf16 *>(y)[o] = static_cast<__bf16>(v[i]);
                else
                    reinterpret_cast<float *>(y)[o] = v[i];
            }
        }
    }
}

// y[b][n] = sum_{s ascending} part[s][b][n], rounded to the output type.
__global__ __launch_bounds__(256) void rowproj_reduce_kernel(int B, int N, int S,
                                                             const float *__restrict__ part,
                                                             void *__restrict__ y, int out_bf16)
{
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= static_cast<int64_t>(B) * N) return;
    float acc = 0.f;
    for (int s = 0; s < S; ++s) acc += part[static_cast<int64_t>(s) * B * N + i];
    if (out_bf16)
        reinterpret_cast<__bf16 *>(y)[i] = static_cast<__bf16>(acc);
    else
        reinterpret_cast<float *>(y)[i] = acc;
}

// fp32 path, any shape: part[s][b][n] over slice s of K with one thread per
// weight row n; x's slice is staged in LDS in chunks.  Grid (ceil(N / 256), S, B).
constexpr int kFChunk = 1024;
__global__ __launch_bounds__(256) void rowproj_f32_kernel(int B, int K, int N, int S,
                                                          const float *__restrict__ x,
                                                          const float *__restrict__ w,
                                                          float *__restrict__ part)
{
    __shared__ float xs[kFChunk];
    const int n = blockIdx.x * 256 + threadIdx.x, s = blockIdx.y, b = blockIdx.z;
    const int k0 = static_cast<int>((static_cast<int64_t>(K) * s) / S);
    const int k1 = static_cast<int>((static_cast<int64_t>(K) * (s + 1)) / S);
    float acc = 0.f;
    for (int kc = k0; kc < k1; kc += kFChunk) {
        const int len = min(kFChunk, k1 - kc);
        __syncthreads();
        for (int k = threadIdx.x; k < len; k += 256) xs[k] = x[static_cast<int64_t>(b) * K + kc + k];
        __syncthreads();
        if (n < N) {
            const float *wr = w + static_cast<int64_t>(n) * K + kc;
            for (int k = 0; k < len; ++k) acc = fmaf(wr[k], xs[k], acc);
        }
    }
    if (n < N) part[(static_cast<int64_t>(s) * B + b) * N + n] = acc;
}

// W_OV[n][h dc + j] = sum_i W_O[n][h dv + i] W_UV[h][i][j]: a 64 x 64 output
// tile of one head per workgroup, 4 x 4 outputs per thread, the i range in
// LDS-staged chunks of 32.  Grid (ceil(N / 64), ceil(dc / 64), H).
template <bool BF16>
__device__ __forceinline__ float ld(const void *p, int64_t i)
{
    if constexpr (BF16) return bf16lo(static_cast<const uint16_t *>(p)[i]);
    else return static_cast<const float *>(p)[i];
}

template <bool BF16>
__global__ __launch_bounds__(256) void fold_value_output_kernel(int N, int H, int dv, int dc,
                                                                const void *__restrict__ w_o,
                                                                const void *__restrict__ w_uv,
                                                                void *__restrict__ w_ov)
{
    constexpr int kT = 64, kI = 32;
    __shared__ float a[kI][kT + 1];  // W_O[n0 + r][h dv + i0 + i], as [i][r]
    __shared__ float bm[kI][kT];     // W_UV[h][i0 + i][j0 + c]
    const int n0 = blockIdx.x * kT, j0 = blockIdx.y * kT, h = blockIdx.z;
    const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;  // 16 x 16 threads, 4 x 4 each
    float acc[4][4] = {};
    for (int i0 = 0; i0 < dv; i0 += kI) {
        __syncthreads();
        for (int e = tid; e < kI * kT; e += 256) {
            {   // consecutive threads: consecutive i of one W_O row
                const int i = e % kI, r = e / kI, n = n0 + r, ii = i0 + i;
                a[i][r] = (n < N && ii < dv)
                              ? ld<BF16>(w_o, static_cast<int64_t>(n) * H * dv + static_cast<int64_t>(h) * dv + ii)
                              : 0.f;
            }
            {   // consecutive threads: consecutive j of one W_UV row
                const int c = e % kT, i = e / kT, j = j0 + c, ii = i0 + i;
                bm[i][c] = (j < dc && ii < dv) ? ld<BF16>(w_uv, (static_cast<int64_t>(h) * dv + ii) * dc + j) : 0.f;
            }
        }
        __syncthreads();
#pragma unroll 8
        for (int i = 0; i < kI; ++i) {
            float av[4], bv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                av[q] = a[i][4 * tr + q];
                bv[q] = bm[i][4 * tc + q];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int p = 0; p < 4; ++p) acc[q][p] = fmaf(av[q], bv[p], acc[q][p]);
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int n = n0 + 4 * tr + q;
        if (n >= N) continue;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int j = j0 + 4 * tc + p;
            if (j >= dc) continue;
            const int64_t o = static_cast<int64_t>(n) * H * dc + static_cast<int64_t>(h) * dc + j;
            if constexpr (BF16) reinterpret_cast<__bf16 *>(w_ov)[o] = static_cast<__bf16>(acc[q][p]);
            else reinterpret_cast<float *>(w_ov)[o] = acc[q][p];
        }
    }
}

// MFMA form of the fold for bf16 with d_v = 128 and d_c a multiple of 128:
// workgroup (head h, column block jb, row part z) computes
// W_OV[n][h dc + 128 jb + j] for the rows n of its part, as
// D^T[j][n] = sum_i W_UV[h][i][128 jb + j] W_O[n][h dv + i].
// A = W_UV[h]'s column block, transposed once into LDS and then held in
// registers (wave w: columns 32 w .. 32 w + 31, all 8 K steps of 16);
// B = W_O rows straight from global memory, 64 rows per pass.  All heads'
// workgroups of one column block share an XCD with h % 8 (blockIdx.x = h),
// so the 4 column blocks of a head find its W_O columns in one L2.
// Grid (H, dc / 128, parts), 256 threads; `rows` (a multiple of 64) per part.
constexpr int kFoldDv = 128;
__global__ __launch_bounds__(256) void fold_value_output_mfma_kernel(int N, int H, int dc, int rows,
                                                                     const uint16_t *__restrict__ w_o,
                                                                     const uint16_t *__restrict__ w_uv,
                                                                     uint16_t *__restrict__ w_ov)
{
    constexpr int kRow = kFoldDv + 8;            // padded LDS row of the transposed block (bf16)
    __shared__ __attribute__((aligned(16))) uint16_t wt[128 * kRow];  // [j][i]
    const int h = blockIdx.x, jb = blockIdx.y;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int half = lane >> 5, l32 = lane & 31;

    // W_UV[h][i][128 jb + 8 c .. + 7] -> wt[8 c + e][i]
    const uint16_t *src = w_uv + static_cast<int64_t>(h) * kFoldDv * dc + 128 * jb;
    for (int e = tid; e < kFoldDv * 16; e += 256) {
        const int i = e >> 4, c = e & 15;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(src + static_cast<int64_t>(i) * dc + 8 * c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            wt[(8 * c + 2 * q) * kRow + i] = static_cast<uint16_t>(v[q] & 0xffffu);
            wt[(8 * c + 2 * q + 1) * kRow + i] = static_cast<uint16_t>(v[q] >> 16);
        }
    }
    __syncthreads();
    u32x4 a[kFoldDv / 16];  // A: column 32 wv + l32, K elements 16 s + 8 half .. + 7
#pragma unroll
    for (int s = 0; s < kFoldDv / 16; ++s)
        a[s] = *reinterpret_cast<const u32x4 *>(&wt[(32 * wv + l32) * kRow + 16 * s + 8 * half]);

    const int64_t ld = static_cast<int64_t>(H) * kFoldDv;       // W_O row length
    const int64_t ldo = static_cast<int64_t>(H) * dc;           // W_OV row length
    const int n_end = min(N, (static_cast<int>(blockIdx.z) + 1) * rows);
    // The transposed block now lives in registers; its LDS holds each pass's
    // 64 x 128 output tile as bf16 rows (stride kRow), written out as whole
    // 256-byte row segments.
    for (int n0 = blockIdx.z * rows; n0 < n_end; n0 += 64) {
        u32x4 b[2][kFoldDv / 16];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int n = min(n0 + 32 * t + l32, N - 1);
            const u32x4 *row = reinterpret_cast<const u32x4 *>(w_o + n * ld + static_cast<int64_t>(h) * kFoldDv) + half;
#pragma unroll
            for (int s = 0; s < kFoldDv / 16; ++s) b[t][s] = row[2 * s];
        }
        __syncthreads();  // the previous pass's tile has been written out
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
            for (int s = 0; s < kFoldDv / 16; ++s) acc = mfma32(a[s], b[t][s], acc);
            // acc[r]: column j = 32 wv + 8 (r / 4) + 4 half + r % 4 of row n0 + 32 t + l32
            uint16_t *trow = &wt[(32 * t + l32) * kRow + 32 * wv + 4 * half];
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<u32x2 *>(trow + 8 * g) =
                    u32x2{pack_bf16(acc[4 * g], acc[4 * g + 1]), pack_bf16(acc[4 * g + 2], acc[4 * g + 3])};
        }
        __syncthreads();
        // 64 rows x 16 pieces of 16 bytes, 4 per thread
#pragma unroll
        for (int e = tid; e < 64 * 16; e += 256) {
            const int r = e >> 4, c = e & 15, n = n0 + r;
            if (n < n_end)
                *reinterpret_cast<u32x4 *>(w_ov + n * ldo + static_cast<int64_t>(h) * dc + 128 * jb + 8 * c) =
                    *reinterpret_cast<const u32x4 *>(&wt[r * kRow + 8 * c]);
        }
    }
}

}  // namespace

hipError_t launch_output_proj(const ProjShape &p, const void *x, const void *w, void *y,
                              float *part, hipStream_t st)
{
    if (p.R > 0) {
        dim3 grid((p.N + p.R - 1) / p.R, (p.B + kPBatch - 1) / kPBatch);
        rowproj_direct_bf16_kernel<<<grid, 64 * kDWaves, 0, st>>>(
            p.B, p.K, p.N, p.R, static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w),
            y, p.out_bf16);
        return hipGetLastError();
    }
    if (p.bf16) {
        dim3 grid((p.N + kPRows - 1) / kPRows, p.S, (p.B + kPBatch - 1) / kPBatch);
        rowproj_bf16_kernel<<<grid, 64 * kPWaves, 0, st>>>(p.B, p.K, p.N, p.S,
                                                          static_cast<const uint16_t *>(x),
                                                          static_cast<const uint16_t *>(w), part);
    } else {
        dim3 grid((p.N + 255) / 256, p.S, p.B);
        rowproj_f32_kernel<<<grid, 256, 0, st>>>(p.B, p.K, p.N, p.S, static_cast<const float *>(x),
                                                 static_cast<const float *>(w), part);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = static_cast<int64_t>(p.B) * p.N;
    rowproj_reduce_kernel<<<static_cast<unsigned>((total + 255) / 256), 256, 0, st>>>(
        p.B, p.N, p.S, part, y, p.out_bf16);
    return hipGetLastError();
}

hipError_t launch_fold_value_output(int N, int H, int dv, int dc, bool bf16, const void *w_o,
                                    const void *w_uv, void *w_ov, hipStream_t st)
{
    const auto al = [](const void *p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; };
    if (bf16 && dv == kFoldDv && dc % 128 == 0 && al(w_o, 16) && al(w_uv, 16) && al(w_ov, 16)) {
        // up to 4 row parts, so that enough waves stream W_O at once
        const int chunks = (N + 63) / 64, parts = chunks < 4 ? chunks : 4;
        const int rows = 64 * ((chunks + parts - 1) / parts);
        fold_value_output_mfma_kernel<<<dim3(H, dc / 128, (N + rows - 1) / rows), 256, 0, st>>>(
            N, H, dc, rows, static_cast<const uint16_t *>(w_o), static_cast<const uint16_t *>(w_uv),
            static_cast<uint16_t *>(w_ov));
        return hipGetLastError();
    }
    dim3 grid((N + 63) / 64, (dc + 63) / 64, H);
    if (bf16)
        fold_value_output_kernel<true><<<grid, 256, 0, st>>>(N, H, dv, dc, w_o, w_uv, w_ov);
    else
        fold_value_output_kernel<false><<<grid, 256, 0, st>>>(N, H, dv, dc, w_o, w_uv, w_ov);
    return hipGetLastError();
}

}  // namespace mla
