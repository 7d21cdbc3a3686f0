// decode_bf16.hip -- absorbed MLA decode for the DeepSeek-V2/V3 shape on
// gfx950: d_c = 512 latent, d_r = 64 decoupled RoPE key, d_n = d_v = 128,
// heads a multiple of 128, bf16 storage, fp32 accumulation.
//
// Three kernels on the caller's stream:
//   1. absorb:  Qa[b][h] = [ W_UK[h]^T q_nope[b][h] ; q_rope[b][h] ]   (bf16, 576 wide)
//      ("DeepSeek MLA Architecture: How It Cuts KV Cache by 93%", section 2:
//      the up-projection is folded into the query, so keys are never built.)
//   2. split-KV flash-decode: one workgroup per (context split, 128 heads,
//      sequence).  Cache rows (576 bf16 = 1152 B) are streamed into LDS once
//      and shared by all 128 heads -- the absorbed decode is MQA-shaped.
//      Scores S^T[token][head] = C . Qa^T and the latent accumulation
//      O^T[col][head] += C^T . P^T both run on v_mfma_f32_32x32x16_bf16.
//      Online softmax in log2 units with a lazily raised running max.
//      ("mla-from-scratch" README, "Absorption, and why RoPE breaks it":
//      score = absorbed content term + decoupled positional term; attend
//      over the latents and up-project once at the end.)
//   3. merge + up-project: fixed-order (ascending split) combination of the
//      split partials, then out = W_UV[h] o_lat.
#include <hip/hip_runtime.h>
#include <math.h>

#include "cdna4.h"
#include "mla_internal.h"

namespace mla {
namespace {

using namespace cdna4;

constexpr int DC = 512, DR = 64, DQK = DC + DR, DN = 128, DV = 128;

// ---------------------------------------------------------------------------
// 1. absorb: grid (4 column quarters, H, ceil(B/8)), 256 threads, B = query
//    rows.  Wave w reduces rows i in [32w, 32w+32) of W_UK[h]; lane holds 2
//    columns.  The quarter-0 workgroups also place the RoPE query channels
//    beside q~, rotated at the query's position when rope_base > 0 (RoFormer
//    pairs (2i, 2i+1) turned by pos * rope_base^(-2i/d_r), angle and rotation
//    in fp64, rounded through fp32 to bf16).
// ---------------------------------------------------------------------------
constexpr int kAbsorbBatch = 8;

__global__ __launch_bounds__(256) void absorb_bf16_kernel(int B, int H, int T, int64_t n_max,
                                                          const int32_t *seqlens, double rope_base,
                                                          const uint16_t *q_nope,
                                                          const uint16_t *q_rope,
                                                          const uint16_t *w_uk, uint16_t *qa)
{
    const int qtr = blockIdx.x, h = blockIdx.y, b0 = blockIdx.z * kAbsorbBatch;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int nb = min(kAbsorbBatch, B - b0);
    __shared__ float qs[kAbsorbBatch][DN];
    __shared__ float red[4][kAbsorbBatch][128];

    // Every global load is issued before the first wait: this wave's 32
    // weight pieces, then the queries, then (quarter 0) the RoPE channel
    // pair of this thread, so the kernel costs one memory round trip.
    const int col = qtr * 128 + 2 * lane;
    const uint32_t *wrow = reinterpret_cast<const uint32_t *>(w_uk + (static_cast<int64_t>(h) * DN + 32 * w) * DC + col);
    uint32_t wvals[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) wvals[i] = wrow[i * (DC / 2)];
    constexpr int kQPer = kAbsorbBatch * DN / 256;  // query values per thread
    uint16_t qv[kQPer];
#pragma unroll
    for (int k = 0; k < kQPer; ++k) {
        const int e = tid + 256 * k, bb = e / DN, i = e % DN;
        qv[k] = q_nope[(static_cast<int64_t>(b0 + min(bb, nb - 1)) * H + h) * DN + i];
    }
    // one rotation pair per thread: nb * d_r / 2 <= 8 * 32 = 256 threads
    static_assert(kAbsorbBatch * (DR / 2) <= 256, "one RoPE pair per thread");
    const bool rope_lane = qtr == 0 && tid < nb * (DR / 2);
    const int rv = b0 + tid / (DR / 2), ri = tid % (DR / 2);
    const int64_t rrow = static_cast<int64_t>(rv) * H + h;
    uint32_t two = rope_lane ? *reinterpret_cast<const uint32_t *>(q_rope + rrow * DR + 2 * ri) : 0u;
#pragma unroll
    for (int k = 0; k < kQPer; ++k) {
        const int e = tid + 256 * k, bb = e / DN, i = e % DN;
        qs[bb][i] = bb < nb ? bf16lo(qv[k]) : 0.f;
    }
    __syncthreads();

    float acc[kAbsorbBatch][2];
#pragma unroll
    for (int bb = 0; bb < kAbsorbBatch; ++bb) acc[bb][0] = acc[bb][1] = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const uint32_t wv = wvals[i];
        const float w0 = bf16lo(wv), w1 = bf16hi(wv);
#pragma unroll
        for (int bb = 0; bb < kAbsorbBatch; ++bb) {
            const float q = qs[bb][32 * w + i];
            acc[bb][0] = fmaf(w0, q, acc[bb][0]);
            acc[bb][1] = fmaf(w1, q, acc[bb][1]);
        }
    }
#pragma unroll
    for (int bb = 0; bb < kAbsorbBatch; ++bb) {
        red[w][bb][2 * lane] = acc[bb][0];
        red[w][bb][2 * lane + 1] = acc[bb][1];
    }
    __syncthreads();
    // 8 batches x 128 columns = 1024 outputs, 4 per thread, summed in wave order.
    for (int e = tid; e < kAbsorbBatch * 128; e += 256) {
        const int bb = e / 128, c = e % 128;
        if (bb >= nb) continue;
        const float v = ((red[0][bb][c] + red[1][bb][c]) + red[2][bb][c]) + red[3][bb][c];
        reinterpret_cast<__bf16 *>(qa)[(static_cast<int64_t>(b0 + bb) * H + h) * DQK + qtr * 128 + c] =
            static_cast<__bf16>(v);
    }
    if (rope_lane) {  // RoPE query channels beside q~
        if (rope_base > 0.0) {
            const int b = rv / T;
            const int pos = static_cast<int>(min<int64_t>(max(seqlens[b], 0), n_max)) - T + (rv - b * T);
            if (pos > 0) {
                const double theta = pow(rope_base, -2.0 * ri / DR);
                double sn, cs;
                sincos(static_cast<double>(pos) * theta, &sn, &cs);
                const double x0 = bf16lo(two), x1 = bf16hi(two);
                two = pack_bf16(static_cast<float>(x0 * cs - x1 * sn),
                                static_cast<float>(x0 * sn + x1 * cs));
            }
        }
        *reinterpret_cast<uint32_t *>(qa + rrow * DQK + DC + 2 * ri) = two;
    }
}

// ---------------------------------------------------------------------------
// 2. split-KV flash-decode
//
// Workgroup = 4 waves = 128 heads of one sequence over one context split.
// Cache tiles of 32 rows x 576 bf16 (36 KiB) are copied HBM -> LDS with
// direct-to-LDS 16-byte buffer loads (buffer_load_dwordx4 ... lds, with the
// non-temporal policy: a decode call reads each row once) into three LDS
// buffers, so two tiles are in flight while one is consumed.  The buffer
// descriptor's range ends at the split's last row: rows past it arrive as
// zeros (weight zero, and they can never inject NaN/Inf).  The cross-wave
// hand-off is an explicit "wait for my tile loads, then s_barrier".
//
// LDS tile layout: latent row r (one 1-KiB load each, so its placement is
// free) sits at r * 1280 + 16 * f(r), f(r) = 4 (r & 3) + ((r >> 2) & 3) < 16:
// 1280-byte slots keep the staggered rows from overlapping and leave the bank
// phase to f alone.  The stagger keeps both access patterns free of bank
// conflicts: the score MFMA's lanes read 16 consecutive rows at one column
// (f distinct over any 16 consecutive rows), and each 16-lane group of a
// transposing read takes 32 bytes from 4 consecutive rows r = 4m..4m+3
// (f = 4k + const, so their windows start 64 bytes apart).  Then come 32
// RoPE-key rows of 128 bytes, 16-byte chunks XOR-swizzled by (row >> 1) & 7.
// Every read address is a per-lane base plus an immediate.
//
// Score  S^T[token][head] = C . Qa^T  (A = cache rows, B = absorbed query)
// Accum  O^T[col][head] += C^T . P^T  (A = cache columns, read with the
//        transposing ds_read_b64_tr_b16, B = softmax weights from registers)
// both on v_mfma_f32_32x32x16_bf16.  The absorbed query's 512 latent channels
// stay in VGPRs (128 per lane), its 64 RoPE channels in LDS; the 512 x 32 fp32
// accumulator of the wave's heads fills the 256 AGPRs.
//
// Softmax: scores are kept in log2 units (scale * log2(e) folded in).  The
// reference maximum m_ref of each head is fixed by the split's first tile;
// later weights are exp2(s - m_ref) <= 2^64, which bf16 and the fp32
// accumulators hold without overflow, so the accumulators are never
// rescaled.  Should a later score exceed m_ref + 64, the head's partial is
// marked (NaN maximum) and the merge kernel recomputes that (split, head)
// with the split's true maximum; ordinary inputs never take that path.
// ---------------------------------------------------------------------------
constexpr int kTile = 32;                       // tokens per LDS tile (== split granule)
constexpr int kLatRow = DC * 2;                 // 1024 B per latent row
constexpr int kLatSlot = kLatRow + 256;         // 1280 B LDS slot per latent row
constexpr int kRopeRow = DR * 2;                // 128 B
constexpr int kRopeBase = kTile * kLatSlot;     // 40960: RoPE rows follow the latent slots
constexpr int kTileBytes = kRopeBase + kTile * kRopeRow;  // 45056
constexpr int kThreadsDec = 256;                // 4 waves x 32 heads
constexpr int kLoadsPerWave = 9;                // 8 latent rows + 1/4 of the RoPE rows
constexpr int kQRopeStride = kRopeRow + 16;     // 144 B per head row (bank stagger)
constexpr int kQRopeBytes = 32 * kQRopeStride;  // one wave's 32 heads
constexpr int kStageRow = 256 + 4;              // floats per staged partial row (bank stagger)
static_assert(kTile == 4 * 8, "each wave loads 8 latent rows per tile");
static_assert(kTile * kRopeRow == 4 * 64 * 16, "each wave loads one quarter of the RoPE rows");
static_assert(kTile == kSplitGranule, "split boundaries must align to tiles");
static_assert(3 * kTileBytes + 4 * kQRopeBytes <= 160 * 1024, "LDS budget");
static_assert(128 * kStageRow * 4 <= 3 * kTileBytes, "the partial rows are staged in the tile buffers");

// Byte offset of latent row r inside a tile.  Each row starts 16 B times a
// stagger in 0..15 into its slot: 4 (r mod 4) + (r div 4 mod 4).  Rows that
// one score read touches together (consecutive r) then start in distinct
// 16-byte bank groups, and so do the rows of one transposing read.
__host__ __device__ constexpr int lat_slot(int r)
{
    return r * kLatSlot + 16 * (4 * (r & 3) + ((r >> 2) & 3));
}
static_assert(lat_slot(kTile - 1) + kLatRow <= kRopeBase, "staggered rows fit before the RoPE rows");
static_assert(16 * 15 + kLatRow <= kLatSlot, "a staggered row stays inside its slot");
// Rows 16 ks + 8 + j and 16 ks + j differ by 8 * 1280 plus this stagger delta,
// the same for every j in 0..7 and every ks, so the second transposing read
// of a K step is the first one's address plus an immediate.
// The loads address row 8 w + k of a tile through this closed form of lat_slot.
__host__ __device__ constexpr int lat_slot_wk(int w, int k)
{
    return (8 * w + k) * kLatSlot + 16 * (4 * (k & 3) + ((2 * w + (k >> 2)) & 3));
}
static_assert(lat_slot_wk(0, 0) == lat_slot(0) && lat_slot_wk(1, 5) == lat_slot(13) &&
              lat_slot_wk(2, 7) == lat_slot(23) && lat_slot_wk(3, 6) == lat_slot(30) &&
              lat_slot_wk(3, 3) == lat_slot(27), "closed form of the load slots");
constexpr int kTrHiStagger = lat_slot(8) - 8 * kLatSlot;
static_assert(kTrHiStagger == lat_slot(9) - lat_slot(1) - 8 * kLatSlot &&
              kTrHiStagger == lat_slot(15) - lat_slot(7) - 8 * kLatSlot &&
              kTrHiStagger == lat_slot(31) - lat_slot(23) - 8 * kLatSlot,
              "uniform stagger delta between the two halves of a K step");
constexpr float kRefSlack = 64.0f;              // log2 headroom above the reference maximum
// LDS operand reads kept in flight ahead of the MFMA that consumes them: with
// one wave per SIMD, this depth is what covers the LDS latency.
#ifndef MLA_DECODE_LOOKAHEAD
#define MLA_DECODE_LOOKAHEAD 8
#endif
constexpr int kLook = MLA_DECODE_LOOKAHEAD;

__global__ __launch_bounds__(kThreadsDec, 1) void decode_splitkv_bf16_kernel(
    int T, int H, int S, int64_t n_max, const uint16_t *__restrict__ ckv, int64_t ckv_sb, int ckv_rowb,
    const uint16_t *__restrict__ kpe, int64_t kpe_sb, int kpe_rowb,
    const int32_t *__restrict__ seqlens, const uint16_t *__restrict__ qa, float c2,
    float *__restrict__ part_o, float *__restrict__ part_ml)
{
    __shared__ __attribute__((aligned(1024))) unsigned char tiles[3 * kTileBytes];
    __shared__ __attribute__((aligned(16))) unsigned char qrope_lds[4 * kQRopeBytes];

    // Query row v = b * T + t: query t of sequence b (T = 1 for decode)
    // attends to the causal prefix of its sequence's cache.
    const int sp = blockIdx.x, hg = blockIdx.y, v = blockIdx.z;
    const int b = v / T, tq = v - b * T;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int half = lane >> 5, l32 = lane & 31;
    const int hq = hg * 128 + w * 32 + l32;  // this lane's head (score column)

    const int L = query_len(seqlens[b], n_max, T, tq);
    const int ntiles_seq = (L + kTile - 1) / kTile;
    const int tps = (ntiles_seq + S - 1) / S;
    const int start = sp * tps * kTile;
    const int end = min(L, start + tps * kTile);
    const int64_t prow = (static_cast<int64_t>(v) * S + sp) * H + hq;

    if (start >= end) {  // empty split: weight zero in the merge, O never read
        if (half == 0) {
            part_ml[prow * 2 + 0] = -INFINITY;
            part_ml[prow * 2 + 1] = 0.f;
        }
        return;
    }
    const int ntiles = (end - start + kTile - 1) / kTile;

    // Absorbed query of this lane's head as the score MFMA's B operand:
    // B[k][j = head], lane holds k = 16 s + 8 half + 0..7.  Latent channels
    // (s < 32) in registers; RoPE channels (s = 32..35) in this wave's LDS
    // slice (head row l32 at a 144-byte stride).
    const uint16_t *qrow = qa + (static_cast<int64_t>(v) * H + hq) * DQK + 8 * half;
    u32x4 qreg[DC / 16];
#pragma unroll
    for (int s = 0; s < DC / 16; ++s) qreg[s] = *reinterpret_cast<const u32x4 *>(qrow + 16 * s);
    const unsigned char *qr = qrope_lds + w * kQRopeBytes + l32 * kQRopeStride + 16 * half;
#pragma unroll
    for (int s = 0; s < DR / 16; ++s)
        *reinterpret_cast<u32x4 *>(const_cast<unsigned char *>(qr) + 32 * s) =
            *reinterpret_cast<const u32x4 *>(qrow + DC + 16 * s);
    // Let the query loads land here, once: the compiler then knows they are
    // complete and puts no wait on them inside the tile loop (where any
    // vector-memory wait would also wait for the tile loads in flight).
    __builtin_amdgcn_s_waitcnt(0);

    // Buffer descriptors covering rows [0, end) of this sequence.
    const i32x4 rs_lat =
        make_rsrc(ckv + static_cast<int64_t>(b) * ckv_sb, static_cast<uint32_t>(end) * ckv_rowb);
    const i32x4 rs_rope =
        make_rsrc(kpe + static_cast<int64_t>(b) * kpe_sb, static_cast<uint32_t>(end) * kpe_rowb);

    // This wave's nine loads of the tile starting at token n0: latent rows
    // 8 w .. 8 w + 7 (one 1-KiB load each), and RoPE rows 8 w .. 8 w + 7 in
    // one load (lane -> row 8 w + lane / 8, LDS chunk lane % 8 holding source
    // chunk (lane % 8) ^ (row & 7)).
    const unsigned lat_src = static_cast<unsigned>(8 * w * ckv_rowb + 16 * lane);
    const int rr = 8 * w + (lane >> 3);
    const unsigned rope_src = static_cast<unsigned>(rr * kpe_rowb + 16 * ((lane & 7) ^ ((rr >> 1) & 7)));
    // LDS addresses of this wave's rows (wave-uniform, scalar arithmetic).
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const uint32_t tiles_lds = lds_addr(tiles);
    auto issue_tile = [&](int n0, int dst_buf) {
        const unsigned lat_base = static_cast<unsigned>(n0) * static_cast<unsigned>(ckv_rowb);
        const uint32_t dst = tiles_lds + static_cast<uint32_t>(dst_buf) * kTileBytes;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            lds_dma16_stream(rs_lat, dst + lat_slot_wk(wu, k),
                         lat_src + lat_base + static_cast<unsigned>(k * ckv_rowb));
        lds_dma16_stream(rs_rope, dst + kRopeBase + wu * 8 * kRopeRow,
                     rope_src + static_cast<unsigned>(n0) * static_cast<unsigned>(kpe_rowb));
    };

    // Per-lane LDS offsets within a tile (immediates are added per access).
    // Score A operand, latent step s: row l32, byte 32 s + 16 half.
    const int s_lat = lat_slot(l32) + 16 * half;
    // P.C A operand via the transposing read, K step ks, j-block q, read r:
    // source lane 4 k + c of each 16-lane group g addresses token (row)
    // 16 ks + 8 r + 4 (g >> 1) + k, latent columns 32 q + 16 (g & 1) + 4 c.
    // lat_slot of that row = its lane part lat_slot(4 (g >> 1) + k) plus
    // (16 ks + 8 r) * 1280 + r * kTrHiStagger, an immediate.
    const int g16 = lane >> 4, k4 = (lane >> 2) & 3, c4 = lane & 3;
    const int pv_base = lat_slot(4 * (g16 >> 1) + k4) + 2 * (16 * (g16 & 1) + 4 * c4);

    f32x16 oacc[16];
#pragma unroll
    for (int q = 0; q < 16; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[q][r] = 0.f;
    float m_ref = -INFINITY;  // per head (lane column): the first tile's maximum
    float l_run = 0.f;
    bool over = false;        // a later score exceeded m_ref + 64 for this head

    // One tile: wait for it, hand the next-but-one tile's loads to the
    // hardware, then scores, softmax weights and the latent accumulation.
    auto tile_step = [&](int t, const unsigned char *tb, int next_buf) {
        const int n0 = start + t * kTile;
        if (t + 1 < ntiles)
            wait_then_barrier<kLoadsPerWave>();
        else
            wait_then_barrier<0>();
        if (t + 2 < ntiles) issue_tile(n0 + 2 * kTile, next_buf);

        // ---- scores: S^T[token i][head j] = sum_k C[i][k] Qa[j][k] ----
        const unsigned char *sa = tb + s_lat;
        const unsigned char *sr = tb + kRopeBase + l32 * kRopeRow;
        auto a_at = [&](int s) -> u32x4 {
            if (s < DC / 16) return *reinterpret_cast<const u32x4 *>(sa + 32 * s);
            return *reinterpret_cast<const u32x4 *>(sr + 16 * ((2 * (s - DC / 16) + half) ^ ((l32 >> 1) & 7)));
        };
        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
        u32x4 abuf[kLook];
#pragma unroll
        for (int s = 0; s < kLook; ++s) abuf[s] = a_at(s);
#pragma unroll
        for (int s = 0; s < DQK / 16; ++s) {
            const u32x4 bq = s < DC / 16 ? qreg[s]
                                         : *reinterpret_cast<const u32x4 *>(qr + 32 * (s - DC / 16));
            sacc = mfma32(abuf[s % kLook], bq, sacc);
            if (s + kLook < DQK / 16) abuf[s % kLook] = a_at(s + kLook);
            __builtin_amdgcn_sched_barrier(0);
        }
        // sacc[r] is token 8 (r/4) + 4 half + r%4 of the tile, head l32.
        float tmax = -INFINITY;
        if (n0 + kTile <= end) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sacc[r] *= c2;
                tmax = fmaxf(tmax, sacc[r]);
            }
        } else {  // the split's last, partial tile
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tok = n0 + 8 * (r >> 2) + 4 * half + (r & 3);
                sacc[r] = tok < end ? sacc[r] * c2 : -INFINITY;
                tmax = fmaxf(tmax, sacc[r]);
            }
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        if (t == 0) m_ref = tmax;
        over |= tmax > m_ref + kRefSlack;

        u32x4 pk[2];
        float psum = 0.f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float p0 = __builtin_amdgcn_exp2f(sacc[8 * ks + 2 * p] - m_ref);
                const float p1 = __builtin_amdgcn_exp2f(sacc[8 * ks + 2 * p + 1] - m_ref);
                psum += p0 + p1;
                pk[ks][p] = pack_bf16(p0, p1);
            }
        l_run += psum;

        // ---- O^T[col][head] += C^T[col][token] P^T[token][head] ----
        // K step ks covers tokens 16 ks + 8 (e / 4) + 4 half + e % 4 (e = 0..7
        // across the two transposing reads), where the score accumulator left
        // them; j-block q holds latent columns 32 q .. 32 q + 31.
        const unsigned char *pv = tb + pv_base;
        auto a_tr = [&](int ks, int q) -> u32x4 {
            const u32x2 lo = lds_read_tr4(pv + (16 * ks) * kLatSlot + 64 * q);
            const u32x2 hi = lds_read_tr4(pv + (16 * ks + 8) * kLatSlot + kTrHiStagger + 64 * q);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        u32x4 av[kLook];
#pragma unroll
        for (int i = 0; i < kLook; ++i) av[i] = a_tr(0, i);
#pragma unroll
        for (int i = 0; i < 32; ++i) {  // i = 16 ks + q
            const int ks = i >> 4, q = i & 15;
            oacc[q] = mfma32(av[i % kLook], pk[ks], oacc[q]);
            if (i + kLook < 32) av[i % kLook] = a_tr((i + kLook) >> 4, (i + kLook) & 15);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    issue_tile(start, 0);
    if (ntiles > 1) issue_tile(start + kTile, 1);
    int buf = 0;  // tile t lives in buffer t % 3
    for (int t = 0; t < ntiles; ++t) {
        const int nxt = buf == 0 ? 2 : buf - 1;  // (t + 2) % 3
        tile_step(t, tiles + buf * kTileBytes, nxt);
        buf = buf == 2 ? 0 : buf + 1;
    }

    // ---- write the split partial: un-normalised O, reference max, mass ----
    // The workgroup's 128 heads are 128 consecutive 2-KiB rows of part_o.
    // Accumulator q, element r is latent column 32 q + 8 (r/4) + 4 half + r%4
    // of this lane's head; each lane's 16-byte pieces would land in 32
    // different rows per store, so the rows are staged in the (now idle) tile
    // buffers, half of the columns at a time, and written as whole 1-KiB row
    // segments.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    float *stage = reinterpret_cast<float *>(tiles);  // [128 heads][kStageRow]
    float *obase = part_o + ((static_cast<int64_t>(v) * S + sp) * H + hg * 128) * DC;
    __syncthreads();  // every wave is done with the last tile
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int q = 8 * p; q < 8 * p + 8; ++q)
#pragma unroll
            for (int m = 0; m < 4; ++m)
                *reinterpret_cast<f32x4 *>(stage + (32 * w + l32) * kStageRow + 32 * (q - 8 * p) + 8 * m + 4 * half) =
                    f32x4{oacc[q][4 * m], oacc[q][4 * m + 1], oacc[q][4 * m + 2], oacc[q][4 * m + 3]};
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 128 * 64 / kThreadsDec; ++e) {
            const int idx = tid + kThreadsDec * e, head = idx >> 6, piece = idx & 63;
            *reinterpret_cast<f32x4 *>(obase + head * DC + 256 * p + 4 * piece) =
                *reinterpret_cast<const f32x4 *>(stage + head * kStageRow + 4 * piece);
        }
        __syncthreads();
    }
    if (half == 0) {
        // NaN marks a head whose weights could overflow: the merge kernel
        // recomputes that (split, head) with the split's true maximum.
        part_ml[prow * 2 + 0] = over ? __builtin_nanf("") : m_ref;
        part_ml[prow * 2 + 1] = l_tot;
    }
}

// ---------------------------------------------------------------------------
// 3. merge + up-project: grid (H, B * T), 256 threads, one (head, query row)
//    each.
//    M = max_s m_s, w_s = 2^(m_s - M), o_lat = sum_s w_s O_s / sum_s w_s l_s,
//    every sum in a fixed order (bitwise repeatable), then out = W_UV[h] o_lat.
//    A split marked with a NaN maximum (its weights could have overflowed) is
//    first recomputed here for this head with the split's true maximum, in
//    plain fp32.  The workgroups of one head differ in blockIdx by multiples
//    of H, so with H a multiple of 8 they share an XCD and its L2 copy of
//    W_UV[h].
// ---------------------------------------------------------------------------
constexpr int kMergeLoads = 8;  // partial pieces per thread in flight

struct CacheView {
    int T;                   // query tokens per sequence (1 for decode)
    int64_t n_max;
    const uint16_t *ckv;
    int64_t ckv_sb, ckv_sn;  // elements
    const uint16_t *kpe;
    int64_t kpe_sb, kpe_sn;
    const int32_t *seqlens;
    const uint16_t *qa;      // [B * T][H][576] absorbed queries (bf16)
    float c2;                // softmax scale * log2(e)
};

__device__ float block_reduce(float v, float *red, bool is_max)
{
    for (int o = 32; o > 0; o >>= 1) {
        const float u = __shfl_xor(v, o);
        v = is_max ? fmaxf(v, u) : v + u;
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < 4; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
    return r;
}

// Recompute one (query row, split, head) partial: scores against the split's
// rows, their maximum, then weights, mass and the weighted latent sum.
__device__ void recompute_partial(const CacheView &cv, int H, int S, int v, int sp, int h,
                                  float *part_o, float *part_ml)
{
    __shared__ float q[DQK];
    __shared__ float pw[256];
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int b = v / cv.T;
    const int L = query_len(cv.seqlens[b], cv.n_max, cv.T, v - b * cv.T);
    const int ntiles_seq = (L + kSplitGranule - 1) / kSplitGranule;
    const int tps = (ntiles_seq + S - 1) / S;
    const int start = sp * tps * kSplitGranule;
    const int end = min(L, start + tps * kSplitGranule);
    const uint16_t *qrow = cv.qa + (static_cast<int64_t>(v) * H + h) * DQK;
    for (int k = tid; k < DQK; k += 256) q[k] = bf16lo(qrow[k]);
    __syncthreads();
    auto score = [&](int n) {
        const uint16_t *c = cv.ckv + static_cast<int64_t>(b) * cv.ckv_sb + static_cast<int64_t>(n) * cv.ckv_sn;
        const uint16_t *r = cv.kpe + static_cast<int64_t>(b) * cv.kpe_sb + static_cast<int64_t>(n) * cv.kpe_sn;
        float d = 0.f;
        for (int k = 0; k < DC; ++k) d = fmaf(q[k], bf16lo(c[k]), d);
        for (int k = 0; k < DR; ++k) d = fmaf(q[DC + k], bf16lo(r[k]), d);
        return d * cv.c2;
    };
    float m = -INFINITY;
    for (int n = start + tid; n < end; n += 256) m = fmaxf(m, score(n));
    m = block_reduce(m, red, true);
    float l = 0.f, o0 = 0.f, o1 = 0.f;
    for (int n0 = start; n0 < end; n0 += 256) {
        const int n = n0 + tid;
        const float p = n < end ? exp2f(score(n) - m) : 0.f;
        pw[tid] = p;
        l += block_reduce(p, red, false);  // its barriers also publish pw[]
        const int cnt = min(256, end - n0);
        for (int t = 0; t < cnt; ++t) {
            const uint16_t *c = cv.ckv + static_cast<int64_t>(b) * cv.ckv_sb + static_cast<int64_t>(n0 + t) * cv.ckv_sn;
            const uint32_t two = *reinterpret_cast<const uint32_t *>(c + 2 * tid);
            o0 = fmaf(pw[t], bf16lo(two), o0);
            o1 = fmaf(pw[t], bf16hi(two), o1);
        }
        __syncthreads();
    }
    const int64_t prow = (static_cast<int64_t>(v) * S + sp) * H + h;
    part_o[prow * DC + 2 * tid] = o0;
    part_o[prow * DC + 2 * tid + 1] = o1;
    if (tid == 0) {
        part_ml[prow * 2 + 0] = m;
        part_ml[prow * 2 + 1] = l;
    }
    __syncthreads();
}

// kUpProj = false: write the merged latent o_lat [rows][H][512] itself (the
// attention output before the up-projection, for a caller that folds W_UV
// into its output projection) instead of W_UV[h] o_lat.
template <bool kUpProj>
__global__ __launch_bounds__(256) void merge_upproj_bf16_kernel(int H, int S,
                                                                float *__restrict__ part_o,
                                                                float *__restrict__ part_ml,
                                                                const uint16_t *__restrict__ w_uv,
                                                                void *__restrict__ out, int out_bf16,
                                                                CacheView cv)
{
    const int h = blockIdx.x, v = blockIdx.y, tid = threadIdx.x;  // v: query row
    const int lane = tid & 63, wv_id = tid >> 6;
    __shared__ float wt[kMaxSplits];      // split weights 2^(m_s - M), 0 for empty splits
    __shared__ float red[4];
    __shared__ int any_nan;
    __shared__ __attribute__((aligned(16))) f32x4 half_sum[2][DC / 4];
    __shared__ __attribute__((aligned(16))) float ol[DC];

    const int64_t base = static_cast<int64_t>(v) * S * H + h;  // row of split 0
    if constexpr (!kUpProj) {
        if (S == 1) {  // one split: o = O / l, no cross-split weighting
            float m0 = part_ml[base * 2], l0 = part_ml[base * 2 + 1];
            if (__builtin_isnan(m0)) {  // marked: recompute with the split's true maximum
                recompute_partial(cv, H, 1, v, 0, h, part_o, part_ml);
                m0 = part_ml[base * 2];
                l0 = part_ml[base * 2 + 1];
            }
            if (tid < DC / 4) {
                // an empty split (m = -inf) never wrote O: its row is zeros
                const bool live = m0 != -INFINITY && l0 > 0.f;
                const f32x4 o = live ? *reinterpret_cast<const f32x4 *>(part_o + base * DC + 4 * tid) * (1.f / l0)
                                     : f32x4{0.f, 0.f, 0.f, 0.f};
                const int64_t oi = (static_cast<int64_t>(v) * H + h) * DC + 4 * tid;
                if (out_bf16) {
                    const u32x2 pk = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
                    *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(out) + oi) = pk;
                } else {
                    *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + oi) = o;
                }
            }
            return;
        }
    }
    // Every load is issued up front, in the order the data is needed, so the
    // whole merge costs one memory round trip: (m, l) of split tid, then this
    // thread's first 16 partial pieces, then its W_UV pieces.
    // Loads are unconditional (indices past the last split are clamped) so
    // that no branch makes the compiler wait on them early; the surplus values
    // are discarded by selects.
    const float2 ml = *reinterpret_cast<const float2 *>(
        part_ml + (base + static_cast<int64_t>(min(tid, S - 1)) * H) * 2);
    float ms = tid < S ? ml.x : -INFINITY;
    float ls = tid < S ? ml.y : 0.f;
    // partials: thread -> 4 columns (4 (tid % 128)), splits of parity tid / 128,
    // kMergeLoads splits per batch
    const int c4 = tid & (DC / 4 - 1), par = tid >> 7;
    const float *po = part_o + base * DC + 4 * c4;
    f32x4 pv[kMergeLoads];
    auto load_batch = [&](int sp0) {
#pragma unroll
        for (int k = 0; k < kMergeLoads; ++k) {
            const int sp = min(sp0 + 2 * k, S - 1);
            pv[k] = *reinterpret_cast<const f32x4 *>(po + static_cast<int64_t>(sp) * H * DC);
        }
    };
    load_batch(par);
    // W_UV[h]: wave w takes rows 32 w .. 32 w + 31 in 4 groups of 8; lane
    // (row 32 w + 8 j + l / 8, 16-byte piece l % 8 + 8 c) -- 8 rows x 128
    // contiguous bytes per load instruction.
    const int r8 = lane >> 3, p8 = lane & 7;
    const u32x4 *wbase = reinterpret_cast<const u32x4 *>(w_uv + (static_cast<int64_t>(h) * DV + 32 * wv_id + r8) * DC) + p8;
    u32x4 wq[4][8];
    if constexpr (kUpProj) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int c = 0; c < 8; ++c) wq[j][c] = wbase[j * 8 * (DC / 8) + 8 * c];
    }

    // Marked (NaN) splits are recomputed first, in ascending order, and the
    // partials reloaded.
    if (tid == 0) any_nan = 0;
    __syncthreads();
    if (__builtin_isnan(ms)) any_nan = 1;
    __syncthreads();
    if (any_nan) {
        for (int sp = 0; sp < S; ++sp)
            if (__builtin_isnan(part_ml[(base + static_cast<int64_t>(sp) * H) * 2]))
                recompute_partial(cv, H, S, v, sp, h, part_o, part_ml);
        if (tid < S) {
            ms = part_ml[(base + static_cast<int64_t>(tid) * H) * 2];
            ls = part_ml[(base + static_cast<int64_t>(tid) * H) * 2 + 1];
        }
        load_batch(par);
    }
    const float mx = block_reduce(ms, red, true);           // M = max_s m_s
    const float w = (ms == -INFINITY) ? 0.f : exp2f(ms - mx);
    if (tid < S) wt[tid] = w;
    const float l = block_reduce(w != 0.f ? w * ls : 0.f, red, false);  // its barriers publish wt[]
    const float inv_l = l > 0.f ? 1.f / l : 0.f;

    // Weighted sum; empty splits (weight 0, O never written) are selected
    // away, not multiplied.
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int sp0 = par;;) {
#pragma unroll
        for (int k = 0; k < kMergeLoads; ++k) {
            const int sp = sp0 + 2 * k;
            const float wk = sp < S ? wt[sp] : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = fmaf(wk, wk != 0.f ? pv[k][e] : 0.f, acc[e]);
        }
        sp0 += 2 * kMergeLoads;
        if (sp0 >= S) break;
        load_batch(sp0);
    }
    half_sum[par][c4] = acc;
    __syncthreads();
    if (tid < DC / 4) {
        const f32x4 o = (half_sum[0][tid] + half_sum[1][tid]) * inv_l;
        if constexpr (kUpProj) {
            *reinterpret_cast<f32x4 *>(ol + 4 * tid) = o;
        } else {
            const int64_t oi = (static_cast<int64_t>(v) * H + h) * DC + 4 * tid;
            if (out_bf16) {
                const u32x2 pk = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
                *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(out) + oi) = pk;
            } else {
                *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + oi) = o;
            }
        }
    }
    if constexpr (!kUpProj) return;
    __syncthreads();

    // out[b][h][v] = W_UV[h][v] . o_lat: each row's 8 lanes add their 64
    // columns, then a 3-step butterfly over the 8 lanes.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float *o = ol + 8 * (p8 + 8 * c);
            const f32x4 o0 = *reinterpret_cast<const f32x4 *>(o);
            const f32x4 o1 = *reinterpret_cast<const f32x4 *>(o + 4);
            a = fmaf(bf16lo(wq[j][c][0]), o0[0], a);
            a = fmaf(bf16hi(wq[j][c][0]), o0[1], a);
            a = fmaf(bf16lo(wq[j][c][1]), o0[2], a);
            a = fmaf(bf16hi(wq[j][c][1]), o0[3], a);
            a = fmaf(bf16lo(wq[j][c][2]), o1[0], a);
            a = fmaf(bf16hi(wq[j][c][2]), o1[1], a);
            a = fmaf(bf16lo(wq[j][c][3]), o1[2], a);
            a = fmaf(bf16hi(wq[j][c][3]), o1[3], a);
        }
        a += __shfl_xor(a, 1);
        a += __shfl_xor(a, 2);
        a += __shfl_xor(a, 4);
        if (p8 == 0) {
            const int vr = 32 * wv_id + 8 * j + r8;  // output row of W_UV
            const int64_t oi = (static_cast<int64_t>(v) * H + h) * DV + vr;
            if (out_bf16)
                reinterpret_cast<__bf16 *>(out)[oi] = static_cast<__bf16>(a);
            else
                reinterpret_cast<float *>(out)[oi] = a;
        }
    }
}

// Batched up-projection for many query rows: out[v][h][i] = W_UV[h][i] . o[v][h]
// for 32 query rows and 32 output features of head h per workgroup of one
// wave (features 32 w .. 32 w + 31, w = blockIdx.x % 4), on MFMA; four
// workgroups per head spread W_UV over four times as many CUs.  A = W_UV
// rows straight from global memory; B = the fp32 latents, each split into a
// bf16 high part and a bf16 remainder (x = hi + lo to about 2^-17
// relative), two MFMAs per K step, so the product keeps the latent's fp32
// precision.  W_UV[h] is read once per 32 query rows.
// Grid (4 H, ceil(rows / 32)), 64 threads.
__global__ __launch_bounds__(64) void upproj_bf16_kernel(int H, int rows,
                                                         const float *__restrict__ o_lat,
                                                         const uint16_t *__restrict__ w_uv,
                                                         void *__restrict__ out, int out_bf16)
{
    const int h = blockIdx.x >> 2, wv = blockIdx.x & 3, v0 = blockIdx.y * 32;
    const int lane = threadIdx.x;
    const int half = lane >> 5, l32 = lane & 31;
    // A: W_UV[h] row 32 wv + l32, elements 16 s + 8 half .. + 7 of step s
    const u32x4 *wrow = reinterpret_cast<const u32x4 *>(w_uv + (static_cast<int64_t>(h) * DV + 32 * wv + l32) * DC) + half;
    // B: latent of query row v0 + l32 (clamped inside the rows), same elements
    const int vr = min(v0 + l32, rows - 1);
    const f32x4 *orow = reinterpret_cast<const f32x4 *>(o_lat + (static_cast<int64_t>(vr) * H + h) * DC) + 2 * half;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    // The 32 K steps in 4 batches of 8, double-buffered: the loads of batch
    // k + 1 are issued before the MFMAs of batch k, so the call costs about
    // one memory round trip instead of one per batch.
    constexpr int kU = 8, kBatches = DC / 16 / kU;
    u32x4 a[2][kU];
    f32x4 x0[2][kU], x1[2][kU];
    auto load = [&](int buf, int s0) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            a[buf][u] = wrow[2 * (s0 + u)];
            x0[buf][u] = orow[4 * (s0 + u)];
            x1[buf][u] = orow[4 * (s0 + u) + 1];
        }
    };
    // (the scheduling barriers keep the compiler from spreading a batch's
    // loads between the previous batch's MFMAs)
    load(0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kBatches; ++k) {
        const int buf = k & 1;
        if (k + 1 < kBatches) load(buf ^ 1, (k + 1) * kU);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const float x[8] = {x0[buf][u][0], x0[buf][u][1], x0[buf][u][2], x0[buf][u][3],
                                x1[buf][u][0], x1[buf][u][1], x1[buf][u][2], x1[buf][u][3]};
            u32x4 hi, lo;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hi[e] = pack_bf16(x[2 * e], x[2 * e + 1]);
                lo[e] = pack_bf16(x[2 * e] - bf16lo(hi[e]), x[2 * e + 1] - bf16hi(hi[e]));
            }
            acc = mfma32(a[buf][u], hi, acc);
            acc = mfma32(a[buf][u], lo, acc);
        }
    }
    // acc[r] is feature 32 wv + 8 (r / 4) + 4 half + r % 4 of query row v0 + l32
    if (v0 + l32 >= rows) return;
    const int64_t orow_out = (static_cast<int64_t>(v0 + l32) * H + h) * DV + 32 * wv + 4 * half;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const f32x4 v4 = {acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
        if (out_bf16) {
            const u32x2 pk = {pack_bf16(v4[0], v4[1]), pack_bf16(v4[2], v4[3])};
            *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(out) + orow_out + 8 * g) = pk;
        } else {
            *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + orow_out + 8 * g) = v4;
        }
    }
}

}  // namespace

int decode_bf16_heads_per_block(int H) { return H % 128 == 0 ? 128 : 0; }

hipError_t launch_decode_bf16(const DecodeShape &s, const void *q_nope, const void *q_rope,
                              const void *w_uk, const void *w_uv, const void *ckv,
                              const void *kpe, const int32_t *seqlens, void *out,
                              const DecodeWorkspace &ws, hipStream_t st, hipEvent_t const *events)
{
    // w_uv == nullptr: write the merged latent instead of W_UV[h] o_lat.
    uint16_t *qa = static_cast<uint16_t *>(ws.q);
    const int rows = s.B * s.T;  // query rows
    if (events && events[0]) (void)hipEventRecord(events[0], st);
    {
        dim3 grid(4, s.H, (rows + kAbsorbBatch - 1) / kAbsorbBatch);
        absorb_bf16_kernel<<<grid, 256, 0, st>>>(rows, s.H, s.T, s.n_max, seqlens, s.q_rope_base,
                                                 static_cast<const uint16_t *>(q_nope),
                                                 static_cast<const uint16_t *>(q_rope),
                                                 static_cast<const uint16_t *>(w_uk), qa);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (events && events[1]) (void)hipEventRecord(events[1], st);
    {
        dim3 grid(s.S, s.H / 128, rows);
        decode_splitkv_bf16_kernel<<<grid, kThreadsDec, 0, st>>>(
            s.T, s.H, s.S, s.n_max, static_cast<const uint16_t *>(ckv), s.ckv_sb,
            static_cast<int>(s.ckv_sn * 2), static_cast<const uint16_t *>(kpe), s.kpe_sb,
            static_cast<int>(s.kpe_sn * 2), seqlens, qa, s.scale * kLog2e, ws.part_o, ws.part_ml);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (events && events[2]) (void)hipEventRecord(events[2], st);
    dim3 grid(s.H, rows);
    CacheView cv{s.T, s.n_max, static_cast<const uint16_t *>(ckv), s.ckv_sb, s.ckv_sn,
                 static_cast<const uint16_t *>(kpe), s.kpe_sb, s.kpe_sn, seqlens, qa,
                 s.scale * kLog2e};
    hipError_t e;
    if (w_uv && batched_upproj(s, true)) {
        // many query rows: merge into fp32 latents, then one product per head
        merge_upproj_bf16_kernel<false><<<grid, 256, 0, st>>>(s.H, s.S, ws.part_o, ws.part_ml,
                                                              nullptr, ws.o_lat, 0, cv);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        dim3 ugrid(4 * s.H, (rows + 31) / 32);
        upproj_bf16_kernel<<<ugrid, 64, 0, st>>>(s.H, rows, ws.o_lat,
                                                  static_cast<const uint16_t *>(w_uv), out, s.out_bf16);
    } else if (w_uv) {
        merge_upproj_bf16_kernel<true><<<grid, 256, 0, st>>>(
            s.H, s.S, ws.part_o, ws.part_ml, static_cast<const uint16_t *>(w_uv), out, s.out_bf16, cv);
    } else {
        merge_upproj_bf16_kernel<false><<<grid, 256, 0, st>>>(
            s.H, s.S, ws.part_o, ws.part_ml, nullptr, out, s.out_bf16, cv);
    }
    e = hipGetLastError();
    if (events && events[3]) (void)hipEventRecord(events[3], st);
    return e;
}

}  // namespace mla
