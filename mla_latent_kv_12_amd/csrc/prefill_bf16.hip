// prefill_bf16.hip -- naive (decompress-then-attend) causal MLA prefill for
// the DeepSeek-V2/V3 shape on gfx950, bf16 storage, fp32 accumulation.
//
//   1. decompress: K_nope[b][n][h] = W_UK[h] c[b][n] and V[b][n][h] = W_UV[h] c[b][n]
//      for every cached row, written to the workspace (materialised on
//      purpose: this is the naive form the pages contrast with absorption --
//      distaisys deep-dive, section 3; songhuiming walk-through, MLA step 2,
//      "up-project ALL cached latents to K, V").  One MFMA GEMM
//      [rows x 512] . [512 x H*128] per weight.
//   2. causal attention: query t (position L - T + t) attends over rows
//      n <= its position with key [K_nope ; k^R] (k^R shared by all heads)
//      and value V.  Scores and P.V on v_mfma_f32_32x32x16_bf16 with an
//      online softmax; one workgroup per (128 queries, head, sequence).
#include <hip/hip_runtime.h>
#include <math.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int DC = 512, DR = 64, DN = 128, DV = 128, DQK = DN + DR;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// 1. decompress GEMM.  D[feature][token] = W[feature][:] . c[token][:], i.e.
//    out[token][feature] for feature = h*128 + i over all heads.
//    Workgroup tile: 128 features x 128 tokens, 4 waves as 2 x 2 of 64 x 64.
// ---------------------------------------------------------------------------
constexpr int GT = 128;            // tile edge (features and tokens)
constexpr int GK = 32;             // K chunk per LDS stage
constexpr int GRow = GK * 2 + 16;  // 80-byte padded LDS row
constexpr int kGemmThreads = 256;

__global__ __launch_bounds__(kGemmThreads) void decompress_gemm_bf16_kernel(
    int64_t n_max, int n_feat, const uint16_t *__restrict__ w, const uint16_t *__restrict__ ckv,
    int64_t ckv_sb, int64_t ckv_sn, const int32_t *__restrict__ seqlens, uint16_t *__restrict__ dst)
{
    __shared__ __attribute__((aligned(16))) unsigned char sw[GT * GRow];
    __shared__ __attribute__((aligned(16))) unsigned char sc[GT * GRow];

    const int f0 = blockIdx.x * GT;
    const int64_t n0 = static_cast<int64_t>(blockIdx.y) * GT;
    const int b = blockIdx.z;
    const int L = static_cast<int>(min<int64_t>(max(seqlens[b], 0), n_max));
    if (n0 >= L) return;  // rows past the cached length are never attended to

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int half = lane >> 5, l32 = lane & 31;
    const int wf = (wv >> 1) * 64, wt = (wv & 1) * 64;

    const uint16_t *cb = ckv + static_cast<int64_t>(b) * ckv_sb;
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // per K chunk: 128 rows x 64 B of each operand = 512 16-byte pieces, 2 per thread
    u32x4 pw[2], pc[2];
    auto load = [&](int k0) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int c = tid + kGemmThreads * e, row = c >> 2, cc = c & 3;
            pw[e] = *reinterpret_cast<const u32x4 *>(w + static_cast<int64_t>(f0 + row) * DC + k0 + 8 * cc);
            const int64_t n = n0 + row;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (n < L) v = *reinterpret_cast<const u32x4 *>(cb + n * ckv_sn + k0 + 8 * cc);
            pc[e] = v;
        }
    };
    load(0);
    for (int k0 = 0; k0 < DC; k0 += GK) {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int c = tid + kGemmThreads * e, row = c >> 2, cc = c & 3;
            *reinterpret_cast<u32x4 *>(sw + row * GRow + 16 * cc) = pw[e];
            *reinterpret_cast<u32x4 *>(sc + row * GRow + 16 * cc) = pc[e];
        }
        __syncthreads();
        if (k0 + GK < DC) load(k0 + GK);
#pragma unroll
        for (int ks = 0; ks < GK / 16; ++ks) {
            u32x4 a[2], bb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a[i] = *reinterpret_cast<const u32x4 *>(sw + (wf + 32 * i + l32) * GRow + 32 * ks + 16 * half);
                bb[i] = *reinterpret_cast<const u32x4 *>(sc + (wt + 32 * i + l32) * GRow + 32 * ks + 16 * half);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], bb[j], acc[i][j]);
        }
    }

    // D[feature i][token j]: lane holds token j = l32, features 8(r/4)+4half+r%4
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wt + 32 * j + l32;
        if (n >= L) continue;
        uint16_t *drow = dst + (static_cast<int64_t>(b) * n_max + n) * n_feat;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int feat = f0 + wf + 32 * i + 8 * g + 4 * half;
                u32x2 v = {pack_bf16(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]),
                           pack_bf16(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
                *reinterpret_cast<u32x2 *>(drow + feat) = v;
            }
    }
}

// ---------------------------------------------------------------------------
// 2. causal attention over the materialised K/V.
// ---------------------------------------------------------------------------
constexpr int kQB = 128;                   // queries per workgroup (4 waves x 32)
constexpr int kKT = 32;                    // keys per tile
constexpr int kKRow = DQK * 2 + 16;        // 400 B: K tile row (k_nope | k^R) + pad
constexpr int kVRow = DV * 2 + 16;         // 272 B
constexpr int kAttnThreads = 256;
constexpr int kKChunks = DQK * 2 / 16;     // 24 per key row
constexpr int kVChunks = DV * 2 / 16;      // 16 per value row
constexpr int kChunksPerThreadA = kKT * (kKChunks + kVChunks) / kAttnThreads;  // 5
static_assert(kKT * (kKChunks + kVChunks) % kAttnThreads == 0, "tile split");
constexpr float kRescaleThreshold = 8.0f;

__global__ __launch_bounds__(kAttnThreads, 1) void prefill_attn_bf16_kernel(
    int T, int H, int64_t n_max, const uint16_t *__restrict__ q_nope,
    const uint16_t *__restrict__ q_rope, const uint16_t *__restrict__ kpe, int64_t kpe_sb,
    int64_t kpe_sn, const int32_t *__restrict__ seqlens, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, float c2, void *__restrict__ out, int out_bf16)
{
    __shared__ __attribute__((aligned(16))) unsigned char ks_lds[2][kKT * kKRow];
    __shared__ __attribute__((aligned(16))) unsigned char vs_lds[2][kKT * kVRow];

    // heaviest (latest) query blocks first
    const int qb = gridDim.x - 1 - blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int half = lane >> 5, l32 = lane & 31;
    const int L = static_cast<int>(min<int64_t>(max(seqlens[b], 0), n_max));
    const int off = L - T;  // position of query t is off + t
    const int t = qb * kQB + wv * 32 + l32;
    const int pos = off + t;  // keys n <= pos are visible
    const int wave_last = off + qb * kQB + wv * 32 + 31;  // largest position in this wave
    const int blk_last = min(L - 1, off + min(T - 1, qb * kQB + kQB - 1));
    const int nkt = blk_last < 0 ? 0 : blk_last / kKT + 1;

    // query row of this lane's column as the B operand: k = 16 s + 8 half + 0..7
    u32x4 qreg[DQK / 16];
    {
        const bool tv = t < T;
        const int64_t qi = (static_cast<int64_t>(b) * T + (tv ? t : 0)) * H + h;
#pragma unroll
        for (int s = 0; s < DQK / 16; ++s) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (tv) {
                const uint16_t *src = s < DN / 16 ? q_nope + qi * DN + 16 * s + 8 * half
                                                  : q_rope + qi * DR + 16 * (s - DN / 16) + 8 * half;
                v = *reinterpret_cast<const u32x4 *>(src);
            }
            qreg[s] = v;
        }
    }

    f32x16 oacc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[q][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int64_t rowstride = static_cast<int64_t>(H) * DN;  // K and V rows: [b][n][h][128]
    u32x4 stage[kChunksPerThreadA];
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int e = 0; e < kChunksPerThreadA; ++e) {
            const int c = tid + kAttnThreads * e;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (c < kKT * kKChunks) {
                const int row = c / kKChunks, cc = c % kKChunks;
                const int n = k0 + row;
                if (n < L) {
                    const uint16_t *src = cc < DN / 8
                        ? K + (static_cast<int64_t>(b) * n_max + n) * rowstride + static_cast<int64_t>(h) * DN + 8 * cc
                        : kpe + static_cast<int64_t>(b) * kpe_sb + static_cast<int64_t>(n) * kpe_sn + 8 * (cc - DN / 8);
                    v = *reinterpret_cast<const u32x4 *>(src);
                }
            } else {
                const int c2i = c - kKT * kKChunks;
                const int row = c2i / kVChunks, cc = c2i % kVChunks;
                const int n = k0 + row;
                if (n < L)
                    v = *reinterpret_cast<const u32x4 *>(
                        V + (static_cast<int64_t>(b) * n_max + n) * rowstride + static_cast<int64_t>(h) * DV + 8 * cc);
            }
            stage[e] = v;
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int e = 0; e < kChunksPerThreadA; ++e) {
            const int c = tid + kAttnThreads * e;
            if (c < kKT * kKChunks) {
                const int row = c / kKChunks, cc = c % kKChunks;
                *reinterpret_cast<u32x4 *>(ks_lds[buf] + row * kKRow + 16 * cc) = stage[e];
            } else {
                const int c2i = c - kKT * kKChunks;
                const int row = c2i / kVChunks, cc = c2i % kVChunks;
                *reinterpret_cast<u32x4 *>(vs_lds[buf] + row * kVRow + 16 * cc) = stage[e];
            }
        }
    };

    if (nkt > 0) load_tile(0);
    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1, k0 = kt * kKT;
        store_tile(buf);
        __syncthreads();
        if (kt + 1 < nkt) load_tile(k0 + kKT);
        if (k0 > wave_last) continue;  // every key of the tile is in this wave's future

        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
        const unsigned char *krow = ks_lds[buf] + l32 * kKRow + 16 * half;
#pragma unroll
        for (int s = 0; s < DQK / 16; ++s)
            sacc = mfma32(*reinterpret_cast<const u32x4 *>(krow + 32 * s), qreg[s], sacc);

        float sv[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int n = k0 + 8 * (r >> 2) + 4 * half + (r & 3);
            sv[r] = (n <= pos && t < T) ? sacc[r] * c2 : -INFINITY;
            tmax = fmaxf(tmax, sv[r]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const bool need = tmax > m_run + kRescaleThreshold;
        if (__ballot(need) != 0) {
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
            // a column with no visible key yet keeps m = -inf and weights 0
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[q][r] *= alpha;
        }
        u32x4 pk[2];
        float psum = 0.f;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float x0 = sv[8 * kk + 2 * p], x1 = sv[8 * kk + 2 * p + 1];
                const float p0 = x0 == -INFINITY ? 0.f : exp2f(x0 - m_run);
                const float p1 = x1 == -INFINITY ? 0.f : exp2f(x1 - m_run);
                const uint32_t wpk = pack_bf16(p0, p1);
                psum += bf16lo(wpk) + bf16hi(wpk);
                pk[kk][p] = wpk;
            }
        l_run += psum;

        const unsigned char *vt = vs_lds[buf];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            u32x2 R[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int row = 16 * kk + 8 * (e >> 2) + 4 * half + (e & 3);
                R[e] = *reinterpret_cast<const u32x2 *>(vt + row * kVRow + 8 * l32);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint32_t sel = (v & 1) ? 0x07060302u : 0x05040100u;
                u32x4 a;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t x = (v < 2) ? R[2 * p][0] : R[2 * p][1];
                    const uint32_t y = (v < 2) ? R[2 * p + 1][0] : R[2 * p + 1][1];
                    a[p] = __builtin_amdgcn_perm(y, x, sel);
                }
                oacc[v] = mfma32(a, pk[kk], oacc[v]);
            }
        }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (t >= T) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t orow = ((static_cast<int64_t>(b) * T + t) * H + h) * DV;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = 8 * (r >> 2) + 4 * half + (r & 3);  // value columns 4 i .. 4 i + 3
        const float o0 = oacc[0][r] * inv, o1 = oacc[1][r] * inv;
        const float o2 = oacc[2][r] * inv, o3 = oacc[3][r] * inv;
        if (out_bf16) {
            u32x2 v = {pack_bf16(o0, o1), pack_bf16(o2, o3)};
            *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(out) + orow + 4 * i) = v;
        } else {
            float *o = reinterpret_cast<float *>(out) + orow + 4 * i;
            o[0] = o0; o[1] = o1; o[2] = o2; o[3] = o3;
        }
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillShape &s, const void *q_nope, const void *q_rope,
                               const void *w_uk, const void *w_uv, const void *ckv,
                               const void *kpe, const int32_t *seqlens, void *out, void *kbuf,
                               void *vbuf, hipStream_t st)
{
    const int n_feat = s.H * DN;
    dim3 ggrid(n_feat / GT, static_cast<unsigned>((s.n_max + GT - 1) / GT), s.B);
    decompress_gemm_bf16_kernel<<<ggrid, kGemmThreads, 0, st>>>(
        s.n_max, n_feat, static_cast<const uint16_t *>(w_uk), static_cast<const uint16_t *>(ckv),
        s.ckv_sb, s.ckv_sn, seqlens, static_cast<uint16_t *>(kbuf));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    decompress_gemm_bf16_kernel<<<ggrid, kGemmThreads, 0, st>>>(
        s.n_max, n_feat, static_cast<const uint16_t *>(w_uv), static_cast<const uint16_t *>(ckv),
        s.ckv_sb, s.ckv_sn, seqlens, static_cast<uint16_t *>(vbuf));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 agrid((s.T + kQB - 1) / kQB, s.H, s.B);
    prefill_attn_bf16_kernel<<<agrid, kAttnThreads, 0, st>>>(
        s.T, s.H, s.n_max, static_cast<const uint16_t *>(q_nope), static_cast<const uint16_t *>(q_rope),
        static_cast<const uint16_t *>(kpe), s.kpe_sb, s.kpe_sn, seqlens,
        static_cast<const uint16_t *>(kbuf), static_cast<const uint16_t *>(vbuf), s.scale * kLog2e,
        out, s.out_bf16);
    return hipGetLastError();
}

}  // namespace mla
