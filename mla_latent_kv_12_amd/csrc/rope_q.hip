// rope_q.hip -- rotary embedding of the queries' decoupled channels at their
// own positions, the query-side half of RoPE (the key side is rotated when
// the cache row is written, append.hip).  RoFormer's rotation, the one the
// "mla-from-scratch" README cites for the decoupled key ("Absorption, and why
// RoPE breaks it"): consecutive pairs (2i, 2i+1) turn by p * theta_i,
// theta_i = base^(-2i/d_r).  With both sides rotated at their row positions
// the positional score term depends only on the distance between the rows.
//
// One workgroup per query row v = b * T + t at position p = clamp(L_b) - T + t
// (decode: T = 1, p = L_b - 1).  The row's d_r / 2 angles are formed once in
// fp64 and kept in LDS; the H heads' pairs are then rotated in fp64 with
// consecutive threads on consecutive pairs (coalesced), and rounded (through
// fp32) to the storage type.  A row with p < 0 (it sees no key) is copied unrotated.
#include <hip/hip_runtime.h>
#include <math.h>

#include "cdna4.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeMaxPairs = 128;  // d_r <= 256

template <bool BF16>
__global__ __launch_bounds__(kRopeThreads) void rope_q_kernel(int T, int H, int dr, int64_t n_max,
                                                              double base,
                                                              const int32_t *__restrict__ seqlens,
                                                              const void *__restrict__ q_rope,
                                                              void *__restrict__ out)
{
    __shared__ double cs[kRopeMaxPairs][2];
    const int v = blockIdx.x, b = v / T, t = v - b * T;
    const int L = static_cast<int>(min<int64_t>(max(seqlens[b], 0), n_max));
    const int pos = L - T + t;
    const int np = dr / 2;
    for (int i = threadIdx.x; i < np; i += kRopeThreads) {
        double sn = 0.0, c = 1.0;
        if (pos > 0) {
            const double theta = pow(base, -2.0 * i / dr);
            sincos(static_cast<double>(pos) * theta, &sn, &c);
        }
        cs[i][0] = c;
        cs[i][1] = sn;
    }
    __syncthreads();
    const int64_t row0 = static_cast<int64_t>(v) * H * dr;  // element offset of the row
    for (int k = threadIdx.x; k < H * np; k += kRopeThreads) {
        const int i = k % np;                  // pair index within its head
        const int64_t e = row0 + 2 * static_cast<int64_t>(k);
        double x0, x1;
        if constexpr (BF16) {
            const uint32_t two = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(q_rope) + e);
            x0 = cdna4::bf16lo(two);
            x1 = cdna4::bf16hi(two);
        } else {
            x0 = static_cast<const float *>(q_rope)[e];
            x1 = static_cast<const float *>(q_rope)[e + 1];
        }
        const double c = cs[i][0], sn = cs[i][1];
        const float y0 = static_cast<float>(x0 * c - x1 * sn);
        const float y1 = static_cast<float>(x0 * sn + x1 * c);
        if constexpr (BF16) {
            *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(out) + e) = cdna4::pack_bf16(y0, y1);
        } else {
            static_cast<float *>(out)[e] = y0;
            static_cast<float *>(out)[e + 1] = y1;
        }
    }
}

}  // namespace

hipError_t launch_rope_q(int B, int T, int H, int dr, int64_t n_max, double base, bool bf16,
                         const int32_t *seqlens, const void *q_rope, void *out, hipStream_t st)
{
    if (dr <= 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>(B) * static_cast<unsigned>(T);
    if (bf16)
        rope_q_kernel<true><<<grid, kRopeThreads, 0, st>>>(T, H, dr, n_max, base, seqlens, q_rope, out);
    else
        rope_q_kernel<false><<<grid, kRopeThreads, 0, st>>>(T, H, dr, n_max, base, seqlens, q_rope, out);
    return hipGetLastError();
}

}  // namespace mla
