// append.hip -- the cache producer, the step before decode: for one new
// token per sequence, c = W_DKV h and k^R = RoPE_pos(W_KR h), written into
// row `pos` of that sequence's latent and RoPE-key caches ("Deep-Dive: MLA
// and Low-Rank KV Cache Compression in DeepSeek-V3", section 2; eyestech-mla
// description, "Key Architectural Highlights"; songhuiming walk-through, MLA
// step 2).  The rotation turns consecutive pairs (2i, 2i+1) by pos * theta_i,
// theta_i = base^(-2i/d_r) (RoFormer).
//
// A matrix-vector product per sequence: HBM-bound on the weights (d_c + d_r
// rows of d_model values, 8.3 MB at the V3 shape), in practice bound by the
// stream from L2 into each CU, since every workgroup reads the hidden states
// of its sequences in full.  Workgroup = 4 waves, 6 output rows and 4
// sequences (grid.y runs over the sequence groups): wave w streams the w-th
// quarter of the six rows in 16-byte pieces, lane-strided, so that each
// hidden-state piece it loads serves six rows and each weight piece four
// sequences; then the workgroup's 256 lanes are summed in LDS in a fixed
// order.  At the V3 shape that is 96 x 2 workgroups reading 143 KB each,
// against 144 reading 172 KB with 4 rows and 8 sequences.  Rows d_c + 2i and
// d_c + 2i + 1 (one rotation pair) always fall in the same workgroup (row
// groups start at multiples of 6 and d_c is even), which rotates the pair
// and writes both.
#include <hip/hip_runtime.h>
#include <math.h>

#include "cdna4.h"
#include "mla_internal.h"

namespace mla {
namespace {

using namespace cdna4;

constexpr int kAppendRows = 6;     // output rows per workgroup (even: a RoPE pair never straddles two)
constexpr int kAppendWaves = 4;    // waves per workgroup: contiguous quarters of d_model
constexpr int kAppendGroup = 4;    // sequences per workgroup (grid.y runs over the groups)
constexpr int kAppendUnroll = 2;   // 16-byte pieces per lane and row in flight per pass
constexpr int kAppendVals = kAppendRows * kAppendGroup;  // dot products per workgroup
constexpr int kAppendChunks = 8;   // the lane sum: 8 chunks of 32 lanes, then the chunks
static_assert(kAppendChunks * 32 == 64 * kAppendWaves, "chunks of 32 lanes cover the workgroup");
static_assert(kAppendChunks * kAppendVals <= 64 * kAppendWaves, "one thread per (chunk, value)");
static_assert(kAppendRows % 2 == 0, "rotation pairs stay inside one workgroup");

template <bool BF16>
__device__ __forceinline__ void piece_to_f32(const u32x4 &v, float *f)
{
    if constexpr (BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[2 * e] = bf16lo(v[e]);
            f[2 * e + 1] = bf16hi(v[e]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(v[e]);
    }
}

template <bool BF16>
__global__ __launch_bounds__(64 * kAppendWaves) void cache_append_kernel(
    int B, int d_model, int dc, int dr, int64_t n_max, const u32x4 *__restrict__ h,
    const u32x4 *__restrict__ w_dkv, const u32x4 *__restrict__ w_kr,
    const int32_t *__restrict__ positions, double base, void *__restrict__ ckv, int64_t ckv_sb,
    int64_t ckv_sn, void *__restrict__ kpe, int64_t kpe_sb, int64_t kpe_sn)
{
    constexpr int kVec = BF16 ? 8 : 4;  // elements per 16-byte piece
    __shared__ float part[64 * kAppendWaves][kAppendVals + 1];  // per lane, padded rows
    __shared__ float part2[kAppendChunks][kAppendVals];
    __shared__ float res[kAppendRows][kAppendGroup];

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int row0 = blockIdx.x * kAppendRows;
    const int pieces = d_model / kVec;          // 16-byte pieces per row
    // this wave's quarter of every row, and the workgroup's rows (rows past
    // d_c + d_r read row 0 of W_DKV; their sums are never stored)
    const int p_begin = (pieces * wv) / kAppendWaves, p_end = (pieces * (wv + 1)) / kAppendWaves;
    const u32x4 *wrow[kAppendRows];
#pragma unroll
    for (int r = 0; r < kAppendRows; ++r) {
        const int row = row0 + r;
        wrow[r] = row >= dc + dr ? w_dkv
                : row < dc       ? w_dkv + static_cast<int64_t>(row) * pieces
                                 : w_kr + static_cast<int64_t>(row - dc) * pieces;
    }

    // sequence groups: normally one per workgroup (grid.y = groups), more
    // when the groups outnumber the grid's y range
    for (int b0 = blockIdx.y * kAppendGroup; b0 < B; b0 += gridDim.y * kAppendGroup) {
        const int nb = min(kAppendGroup, B - b0);
        float acc[kAppendRows][kAppendGroup];
#pragma unroll
        for (int r = 0; r < kAppendRows; ++r)
#pragma unroll
            for (int g = 0; g < kAppendGroup; ++g) acc[r][g] = 0.f;
        // kAppendUnroll pieces per lane per pass, every load of a pass issued
        // before any is used (indices past the quarter or the group are
        // clamped to valid ones and their products dropped); each
        // hidden-state piece serves all the workgroup's rows
        for (int p0 = p_begin + lane; p0 < p_end; p0 += 64 * kAppendUnroll) {
            u32x4 wq[kAppendUnroll][kAppendRows], hq[kAppendUnroll][kAppendGroup];
#pragma unroll
            for (int u = 0; u < kAppendUnroll; ++u) {
                const int p = min(p0 + 64 * u, p_end - 1);
#pragma unroll
                for (int r = 0; r < kAppendRows; ++r) wq[u][r] = wrow[r][p];
#pragma unroll
                for (int g = 0; g < kAppendGroup; ++g)
                    hq[u][g] = h[static_cast<int64_t>(b0 + min(g, nb - 1)) * pieces + p];
            }
#pragma unroll
            for (int u = 0; u < kAppendUnroll; ++u) {
                if (p0 + 64 * u >= p_end) break;
                float hf[kAppendGroup][kVec];
#pragma unroll
                for (int g = 0; g < kAppendGroup; ++g) piece_to_f32<BF16>(hq[u][g], hf[g]);
#pragma unroll
                for (int r = 0; r < kAppendRows; ++r) {
                    float wf[kVec];
                    piece_to_f32<BF16>(wq[u][r], wf);
#pragma unroll
                    for (int g = 0; g < kAppendGroup; ++g)
#pragma unroll
                        for (int e = 0; e < kVec; ++e) acc[r][g] = fmaf(wf[e], hf[g][e], acc[r][g]);
                }
            }
        }
        // fixed-order sum over the workgroup's 256 lanes: 8 chunks of 32
        // lanes, each in ascending lane order, then the chunks in order
#pragma unroll
        for (int r = 0; r < kAppendRows; ++r)
#pragma unroll
            for (int g = 0; g < kAppendGroup; ++g) part[tid][r * kAppendGroup + g] = acc[r][g];
        __syncthreads();
        if (tid < kAppendChunks * kAppendVals) {
            const int v = tid % kAppendVals, c = tid / kAppendVals;
            float sum = 0.f;
            for (int l = 32 * c; l < 32 * c + 32; ++l) sum += part[l][v];
            part2[c][v] = sum;
        }
        __syncthreads();
        if (tid < kAppendVals) {
            float sum = 0.f;
#pragma unroll
            for (int c = 0; c < kAppendChunks; ++c) sum += part2[c][tid];
            res[tid / kAppendGroup][tid % kAppendGroup] = sum;
        }
        __syncthreads();
        // one thread per (row, sequence): rotate RoPE pairs, round, store
        if (tid < kAppendVals) {
            const int r = tid / kAppendGroup, g = tid % kAppendGroup;
            const int j = row0 + r, b = b0 + g;
            if (g < nb && j < dc + dr) {
                const int pos = positions[b];
                if (pos >= 0 && pos < n_max) {
                    float v = res[r][g];
                    if (j >= dc) {                 // rotation pair (2i, 2i + 1)
                        const int i = (j - dc) >> 1;
                        const double theta = pow(base, -2.0 * i / dr);
                        double sn, cs;
                        sincos(static_cast<double>(pos) * theta, &sn, &cs);
                        const double x0 = res[r & ~1][g], x1 = res[r | 1][g];
                        v = static_cast<float>(((j - dc) & 1) == 0 ? x0 * cs - x1 * sn
                                                                   : x0 * sn + x1 * cs);
                    }
                    if (j < dc) {
                        const int64_t o = static_cast<int64_t>(b) * ckv_sb + static_cast<int64_t>(pos) * ckv_sn + j;
                        if constexpr (BF16) reinterpret_cast<__bf16 *>(ckv)[o] = static_cast<__bf16>(v);
                        else reinterpret_cast<float *>(ckv)[o] = v;
                    } else {
                        const int64_t o = static_cast<int64_t>(b) * kpe_sb + static_cast<int64_t>(pos) * kpe_sn + (j - dc);
                        if constexpr (BF16) reinterpret_cast<__bf16 *>(kpe)[o] = static_cast<__bf16>(v);
                        else reinterpret_cast<float *>(kpe)[o] = v;
                    }
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_cache_append(const AppendShape &s, const void *h, const void *w_dkv,
                               const void *w_kr, const int32_t *positions, void *ckv, void *kpe,
                               hipStream_t st)
{
    const int rows = s.dc + s.dr;
    const int groups = (s.B + kAppendGroup - 1) / kAppendGroup;
    const dim3 grid(static_cast<unsigned>((rows + kAppendRows - 1) / kAppendRows),
                    static_cast<unsigned>(min(groups, 65535)));
    if (s.bf16)
        cache_append_kernel<true><<<grid, 64 * kAppendWaves, 0, st>>>(
            s.B, s.d_model, s.dc, s.dr, s.n_max, static_cast<const u32x4 *>(h),
            static_cast<const u32x4 *>(w_dkv), static_cast<const u32x4 *>(w_kr), positions,
            s.rope_base, ckv, s.ckv_sb, s.ckv_sn, kpe, s.kpe_sb, s.kpe_sn);
    else
        cache_append_kernel<false><<<grid, 64 * kAppendWaves, 0, st>>>(
            s.B, s.d_model, s.dc, s.dr, s.n_max, static_cast<const u32x4 *>(h),
            static_cast<const u32x4 *>(w_dkv), static_cast<const u32x4 *>(w_kr), positions,
            s.rope_base, ckv, s.ckv_sb, s.ckv_sn, kpe, s.kpe_sb, s.kpe_sn);
    return hipGetLastError();
}

}  // namespace mla
