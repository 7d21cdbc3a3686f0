// prefill_bf16.hip -- naive (decompress-then-attend) causal MLA prefill for
// the DeepSeek-V2/V3 shape on gfx950, bf16 storage, fp32 accumulation.
//
//   1. decompress: K_nope[b][h][n] = W_UK[h] c[b][n] and V[b][h][n] = W_UV[h] c[b][n]
//      for every cached row, written to the workspace (materialised on
//      purpose: this is the naive form the pages contrast with absorption --
//      distaisys deep-dive, section 3; songhuiming walk-through, MLA step 2,
//      where all cached latents are up-projected to K and V).  One MFMA GEMM
//      workgroup per (head, 256-token block) computes both, head-major output
//      so that each head's keys and values are contiguous.
//   2. causal attention: query t (position L - T + t) attends over rows
//      n <= its position with key [K_nope ; k^R] (k^R shared by all heads)
//      and value V.  One workgroup of 8 waves per (256 queries, head,
//      sequence); key tiles of 64 rows stream HBM -> LDS with direct-to-LDS
//      loads, three tiles deep; scores and P.V on v_mfma_f32_32x32x16_bf16
//      with an online softmax.
#include <hip/hip_runtime.h>
#include <math.h>

#include "cdna4.h"
#include "mla_internal.h"

namespace mla {
namespace {

using namespace cdna4;

constexpr int DC = 512, DR = 64, DN = 128, DV = 128, DQK = DN + DR;

__device__ __forceinline__ int clamp_len(int32_t v, int64_t n_max)
{
    return static_cast<int>(min<int64_t>(max<int64_t>(v, 0), n_max));
}

// ---------------------------------------------------------------------------
// 1. decompress GEMM: D[token][feature] = c[token][:] . W[feature][:] for the
//    128 features of one head, both weights (W_UK -> K_nope, W_UV -> V), and
//    256 tokens.  16 waves: waves 0-7 take W_UK, waves 8-15 W_UV, each group
//    as 2 (features) x 4 (tokens) waves of 64 x 64, so every chunk of c is
//    read from L2 once for both products.  K (the 512 latent channels) in
//    chunks of 32: each chunk is 2 x 128 W rows + 256 c rows of 64 bytes
//    (32 KiB, one W load and one c load per wave), loaded direct-to-LDS
//    into four buffers, three chunks in flight.  Row r's 16-byte pieces are
//    XOR-swizzled by (r / 4) & 3, so the MFMA operand reads (16 consecutive
//    rows at one piece) touch 16 distinct bank groups.  The bf16 results are
//    staged in LDS and written as whole 256-byte rows of the head-major
//    outputs.
// ---------------------------------------------------------------------------
constexpr int kGF = 128;                                // features per weight (one head)
constexpr int kGN = 256;                                // tokens per workgroup
constexpr int kGK = 32;                                 // K chunk
constexpr int kGWaves = 16;                             // 2 weights x 8 waves
constexpr int kGThreads = 64 * kGWaves;
constexpr int kGStages = 4;                             // chunk buffers
constexpr int kGRowB = kGK * 2;                         // 64 B per LDS row of a chunk
constexpr int kGPieces = kGRowB / 16;                   // 16-byte pieces per row
constexpr int kGRowsPerLoad = 1024 / kGRowB;            // 16 rows per 1-KiB load
constexpr int kGWBytes = kGF * kGRowB;                  // 8 KiB per weight
constexpr int kGCOff = 2 * kGWBytes;                    // c rows follow both weights
constexpr int kGStage = kGCOff + kGN * kGRowB;          // 32 KiB
constexpr int kGChunks = DC / kGK;                      // 16
constexpr int kGOutRow = DN * 2 + 16;                   // 272 B epilogue staging row
constexpr int kGOutBytes = kGN * kGOutRow;              // 68 KiB per weight
constexpr int kGLds = kGStages * kGStage > 2 * kGOutBytes ? kGStages * kGStage : 2 * kGOutBytes;
static_assert(kGF == DN && kGF == DV, "one workgroup covers one head's features");
static_assert(kGCOff == 1024 * kGWaves && kGN * kGRowB == 1024 * kGWaves,
              "per chunk: load wv is a W load (W_UK for waves 0-7), load 16 + wv a c load");
static_assert(kGLds <= 160 * 1024, "LDS budget");

// Piece swizzle of chunk row r: the rows of one 16-row group take the 16
// (row phase, piece) combinations of the 16 bank groups.
__host__ __device__ constexpr int gemm_swz(int r) { return (r / (16 / kGPieces)) % kGPieces; }

constexpr int kGHeadGroup = 4;   // heads per item group of one XCD
constexpr int kGBlockGroup = 8;  // token blocks per item group

// (head, token block) of workgroup i = blockIdx.x + H blockIdx.y of one
// sequence.  Workgroups are dispatched round-robin over the 8 XCDs; when H
// divides by 8, XCD x = i % 8 takes the heads x, x + 8, ... and walks its
// items in groups of kGHeadGroup heads x kGBlockGroup token blocks, so the
// weights and latent rows that its resident workgroups read at one time
// stay within its L2.  The map is a bijection for any H and block count.
__device__ __forceinline__ void gemm_item(int H, int nblk, int &h, int &nb)
{
    const int i = blockIdx.x + H * blockIdx.y;
    if (H % 8 != 0) {
        h = blockIdx.x;
        nb = blockIdx.y;
        return;
    }
    const int hpx = H / 8, x = i & 7;
    int j = i >> 3;
    int hg = kGHeadGroup;
    while (hpx % hg) hg >>= 1;                  // a power-of-two divisor of hpx
    const int t = j / (hpx * kGBlockGroup);     // token-block group (the last may be partial)
    j -= t * hpx * kGBlockGroup;
    const int sz = min(kGBlockGroup, nblk - t * kGBlockGroup);
    const int g = j / (hg * sz), r = j % (hg * sz);
    h = x + 8 * (g * hg + r / sz);
    nb = t * kGBlockGroup + r % sz;
}

__global__ __launch_bounds__(kGThreads, 1) void decompress_gemm_bf16_kernel(
    int H, int64_t n_max, const uint16_t *__restrict__ w_uk, const uint16_t *__restrict__ w_uv,
    const uint16_t *__restrict__ ckv, int64_t ckv_sb, int ckv_rowb,
    const int32_t *__restrict__ seqlens, uint16_t *__restrict__ kbuf, uint16_t *__restrict__ vbuf)
{
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kGLds];

    int h, nb;
    gemm_item(H, gridDim.y, h, nb);
    const int n0 = nb * kGN;
    const int b = blockIdx.z;
    const int L = clamp_len(seqlens[b], n_max);
    if (n0 >= L) return;  // rows past the cached length are never attended to

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int which = wv >> 3, g8 = wv & 7;  // weight, wave within its group
    const int half = lane >> 5, l32 = lane & 31;
    const int wf = (g8 & 1) * 64, wt = (g8 >> 1) * 64;

    const uint16_t *w = which ? w_uv : w_uk;
    const i32x4 rs_w = make_rsrc(w + static_cast<int64_t>(h) * DN * DC, DN * DC * 2);
    const i32x4 rs_c = make_rsrc(ckv + static_cast<int64_t>(b) * ckv_sb,
                                 static_cast<uint32_t>(L) * static_cast<uint32_t>(ckv_rowb));

    // The wave's two loads of a chunk: W rows 16 g8 .. + 15 of its weight
    // and c rows 16 wv .. + 15.  Lane -> row (first row) + lane / 4, LDS
    // piece lane % 4 holding source piece (lane % 4) ^ gemm_swz(row).
    const int rw = kGRowsPerLoad * g8 + lane / kGPieces;
    const int rc = kGRowsPerLoad * wv + lane / kGPieces;
    const unsigned voff_w =
        static_cast<unsigned>(rw * DC * 2 + 16 * ((lane % kGPieces) ^ gemm_swz(rw)));
    const unsigned voff_c = static_cast<unsigned>((n0 + rc) * ckv_rowb +
                                                  16 * ((lane % kGPieces) ^ gemm_swz(rc)));
    // LDS address of this wave's 1-KiB W slot (wave-uniform); its c slot
    // is kGCOff further.
    const uint32_t wave_lds = lds_addr(lds) + 1024 * wv;
    auto issue_chunk = [&](int kc) {
        const unsigned k_byte = static_cast<unsigned>(kc * kGK * 2);
        const uint32_t dst = wave_lds + static_cast<uint32_t>(kc & (kGStages - 1)) * kGStage;
        lds_dma16(rs_w, dst, voff_w + k_byte);
        lds_dma16(rs_c, dst + kGCOff, voff_c + k_byte);
    };

    // Operand reads: row base + 32 rows per block (immediate), piece
    // (2 ks + half) ^ gemm_swz(l32) (block bases are multiples of 32 rows).
    int aoff[kGK / 16];
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks)
        aoff[ks] = l32 * kGRowB + 16 * ((2 * ks + half) ^ gemm_swz(l32));
    const int a_base = which * kGWBytes + wf * kGRowB, c_base = kGCOff + wt * kGRowB;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    static_assert(kGStages == 4 && kGChunks >= 3, "three chunks in flight");
    issue_chunk(0);
    issue_chunk(1);
    issue_chunk(2);
    for (int kc = 0; kc < kGChunks; ++kc) {
        // chunk kc has landed once at most the loads of the chunks issued
        // after it (two loads each) are still in flight
        if (kc + 2 < kGChunks)
            wait_then_barrier<4>();
        else if (kc + 1 < kGChunks)
            wait_then_barrier<2>();
        else
            wait_then_barrier<0>();
        // the buffer of chunk kc - 1, which every wave has finished reading
        if (kc + 3 < kGChunks) issue_chunk(kc + 3);
        const unsigned char *st = lds + (kc & (kGStages - 1)) * kGStage;
#pragma unroll
        for (int ks = 0; ks < kGK / 16; ++ks) {
            u32x4 a[2], c[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a[i] = *reinterpret_cast<const u32x4 *>(st + a_base + 32 * i * kGRowB + aoff[ks]);
                c[i] = *reinterpret_cast<const u32x4 *>(st + c_base + 32 * i * kGRowB + aoff[ks]);
            }
            // D^T[feature][token]: A = W rows, B = c rows
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], c[j], acc[i][j]);
        }
    }

    // Epilogue: stage [token][feature] bf16 rows of both weights, then
    // whole-row stores.
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            unsigned char *row = lds + which * kGOutBytes + (wt + 32 * j + l32) * kGOutRow;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int feat = wf + 32 * i + 8 * g + 4 * half;
                const u32x2 v = {pack_bf16(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]),
                                 pack_bf16(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
                *reinterpret_cast<u32x2 *>(row + 2 * feat) = v;
            }
        }
    __syncthreads();
    const int64_t obase = ((static_cast<int64_t>(b) * H + h) * n_max + n0) * DN;
#pragma unroll
    for (int e = 0; e < 2 * kGN * 16 / kGThreads; ++e) {
        const int id = tid + kGThreads * e;
        const int out = id / (kGN * 16), row = (id >> 4) % kGN, piece = id & 15;
        uint16_t *dst = (out ? vbuf : kbuf) + obase;
        if (n0 + row < L)
            *reinterpret_cast<u32x4 *>(dst + static_cast<int64_t>(row) * DN + 8 * piece) =
                *reinterpret_cast<const u32x4 *>(lds + out * kGOutBytes + row * kGOutRow +
                                                 16 * piece);
    }
}

// ---------------------------------------------------------------------------
// 2. causal attention over the materialised K/V.
//
// Workgroup = 8 waves x 32 queries of one (sequence, head).  Key tiles of 64
// rows: K_nope (64 x 256 B), k^R (64 x 128 B) and V (64 x 256 B), 40 KiB,
// loaded direct-to-LDS (5 loads per wave) into three buffers, so two tiles
// are in flight while one is consumed.  Loads past the sequence's length
// read zeros (buffer range), and those keys are masked anyway.
//
// LDS swizzles (16-byte pieces p of a row; every access pattern below
// touches distinct bank groups within 16 lanes):
//   K_nope row r: piece p at p ^ (r & 15)        (score reads: 16 rows, one piece)
//   k^R    row r: piece p at p ^ ((r >> 1) & 7)  (same, with 128-byte rows)
//   V      row r: piece p at p ^ (4 (r & 3))     (transposing reads: 4 rows x 64 B)
//
// Score  S^T[key][query] = K . Q^T   (A = key rows, B = the wave's queries in VGPRs)
// Accum  O^T[dim][query] += V^T . P^T (A = V read with ds_read_b64_tr_b16,
//        B = softmax weights repacked from the score accumulators)
// Softmax in log2 units, running maximum raised lazily: the accumulators
// are rescaled only when a query's maximum grows by more than 2^8.
// ---------------------------------------------------------------------------
constexpr int kAW = 8;                                  // waves per workgroup
constexpr int kAThreads = 64 * kAW;
constexpr int kAQ = 32 * kAW;                           // 256 queries per workgroup
constexpr int kAT = 64;                                 // keys per tile
constexpr int kKnOff = 0;
constexpr int kKrOff = kAT * DN * 2;                    // 16 KiB
constexpr int kVOff = kKrOff + kAT * DR * 2;            // 24 KiB
constexpr int kATile = kVOff + kAT * DV * 2;            // 40 KiB
constexpr int kADmaPerWave = kATile / 1024 / kAW;       // 5
constexpr float kRescaleThreshold = 8.0f;
constexpr int kAOutRow = DV * 2 + 16;                   // 272 B staged bf16 output row
static_assert(kAW * 32 * kAOutRow <= 3 * kATile, "output rows are staged in the tile buffers");

static_assert(kADmaPerWave * 1024 * kAW == kATile, "whole loads per wave");
static_assert(kKrOff / 1024 == 2 * kAW && (kVOff - kKrOff) / 1024 == kAW &&
              (kATile - kVOff) / 1024 == 2 * kAW, "load d = w + 8 e: e 0-1 K, 2 k^R, 3-4 V");
static_assert(3 * kATile <= 160 * 1024, "LDS budget");

__global__ __launch_bounds__(kAThreads, 1) void prefill_attn_bf16_kernel(
    int T, int H, int B, int nqb, int64_t n_max, const uint16_t *__restrict__ q_nope,
    const uint16_t *__restrict__ q_rope, const uint16_t *__restrict__ kpe, int64_t kpe_sb,
    int kpe_rowb, const int32_t *__restrict__ seqlens, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, float c2, void *__restrict__ out, int out_bf16)
{
    __shared__ __attribute__((aligned(1024))) unsigned char tiles[3 * kATile];

    // Work item: (query block, sequence, head).  Workgroups are dispatched
    // round-robin over the 8 XCDs; when the (sequence, head) pairs divide by
    // 8, XCD x serves the pairs x, x + 8, ..., so each pair's keys and values
    // are fetched into one XCD's L2.  Heaviest (latest) query blocks first.
    const int npairs = B * H;
    int qb, pair;
    if ((npairs & 7) == 0) {
        const int i = blockIdx.x, x = i & 7, j = i >> 3, ppx = npairs >> 3;
        qb = nqb - 1 - j / ppx;
        pair = x + 8 * (j % ppx);
    } else {
        qb = nqb - 1 - static_cast<int>(blockIdx.x) / npairs;
        pair = static_cast<int>(blockIdx.x) % npairs;
    }
    const int b = pair / H, h = pair % H;

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int half = lane >> 5, l32 = lane & 31;
    const int L = clamp_len(seqlens[b], n_max);
    const int off = L - T;                   // position of query t is off + t
    const int q0 = qb * kAQ + 32 * w;        // this wave's first query
    const int t = q0 + l32;
    const int pos = t < T ? off + t : -1;    // keys n <= pos are visible
    // smallest visible-key bound in the wave (-1 when it holds padding queries)
    const int wave_min_pos = q0 + 31 < T ? off + q0 : -1;
    const int wave_last = q0 < T ? min(L - 1, off + min(T - 1, q0 + 31)) : -1;
    const int blk_last = min(L - 1, off + min(T - 1, qb * kAQ + kAQ - 1));
    const int ntiles = blk_last < 0 ? 0 : blk_last / kAT + 1;

    // The lane's query row as the score MFMA's B operand: k = 16 s + 8 half + 0..7.
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
    // Let the query loads land here: no vector-memory wait inside the tile loop.
    __builtin_amdgcn_s_waitcnt(0);

    const i32x4 rs_k = make_rsrc(K + static_cast<int64_t>(pair) * n_max * DN,
                                 static_cast<uint32_t>(L) * (DN * 2));
    const i32x4 rs_v = make_rsrc(V + static_cast<int64_t>(pair) * n_max * DV,
                                 static_cast<uint32_t>(L) * (DV * 2));
    const i32x4 rs_r = make_rsrc(kpe + static_cast<int64_t>(b) * kpe_sb,
                                 static_cast<uint32_t>(L) * static_cast<uint32_t>(kpe_rowb));

    // This wave's 5 loads of a tile (load d = w + 8 e):
    //   e = 0, 1: K_nope rows 4 i .. 4 i + 3 (i = d), lane -> row 4 i + lane / 16
    //   e = 2:    k^R rows 8 w .. 8 w + 7,            lane -> row 8 w + lane / 8
    //   e = 3, 4: V rows 4 i .. 4 i + 3 (i = d - 24)
    // each lane fetching the source piece that its LDS piece holds.
    unsigned voff[kADmaPerWave];
    {
        const int rk0 = 4 * w + (lane >> 4), rk1 = 4 * (w + 8) + (lane >> 4);
        voff[0] = static_cast<unsigned>(rk0 * DN * 2 + 16 * ((lane & 15) ^ (rk0 & 15)));
        voff[1] = static_cast<unsigned>(rk1 * DN * 2 + 16 * ((lane & 15) ^ (rk1 & 15)));
        const int rr = 8 * w + (lane >> 3);
        voff[2] = static_cast<unsigned>(rr * kpe_rowb + 16 * ((lane & 7) ^ ((rr >> 1) & 7)));
        voff[3] = static_cast<unsigned>(rk0 * DV * 2 + 16 * ((lane & 15) ^ (4 * (rk0 & 3))));
        voff[4] = static_cast<unsigned>(rk1 * DV * 2 + 16 * ((lane & 15) ^ (4 * (rk1 & 3))));
    }
    // LDS address of this wave's first 1-KiB load slot (wave-uniform).
    const uint32_t wave_lds = lds_addr(tiles) + 1024 * __builtin_amdgcn_readfirstlane(w);
    auto issue_tile = [&](int n0, int dst_buf) {
        const unsigned kb = static_cast<unsigned>(n0) * (DN * 2);
        const unsigned rb = static_cast<unsigned>(n0) * static_cast<unsigned>(kpe_rowb);
        const uint32_t dst = wave_lds + static_cast<uint32_t>(dst_buf) * kATile;
        lds_dma16(rs_k, dst + kKnOff, voff[0] + kb);
        lds_dma16(rs_k, dst + kKnOff + 1024 * 8, voff[1] + kb);
        lds_dma16(rs_r, dst + kKrOff, voff[2] + rb);
        lds_dma16(rs_v, dst + kVOff, voff[3] + kb);
        lds_dma16(rs_v, dst + kVOff + 1024 * 8, voff[4] + kb);
    };

    // Score A operand (key row 32 kb + l32, K elements 16 s + 8 half + 0..7):
    // per-lane offsets for the 8 K_nope and 4 k^R steps; + kb * rows (immediate).
    int sk[DQK / 16];
#pragma unroll
    for (int s = 0; s < DN / 16; ++s)
        sk[s] = kKnOff + l32 * (DN * 2) + 16 * ((2 * s + half) ^ (l32 & 15));
#pragma unroll
    for (int s = DN / 16; s < DQK / 16; ++s)
        sk[s] = kKrOff + l32 * (DR * 2) + 16 * ((2 * (s - DN / 16) + half) ^ ((l32 >> 1) & 7));
    // P.V A operand via the transposing read: source lane 4 k + c of 16-lane
    // group g addresses key 16 ks + 8 r + 4 (g >> 1) + k (r = 0, 1: the two
    // reads of a K step), value dims 32 q + 16 (g & 1) + 4 c .. + 3; with the
    // V swizzle that is byte 64 (q ^ k) + 32 (g & 1) + 8 c of the row.
    const int g16 = lane >> 4, k4 = (lane >> 2) & 3, c4 = lane & 3;
    int pv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        pv[q] = kVOff + (4 * (g16 >> 1) + k4) * (DV * 2) + 64 * (q ^ k4) + 32 * (g16 & 1) + 8 * c4;

    f32x16 oacc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[q][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    auto tile_step = [&](int it, const unsigned char *tb, int next_buf) {
        const int n0 = it * kAT;
        if (it + 1 < ntiles)
            wait_then_barrier<kADmaPerWave>();
        else
            wait_then_barrier<0>();
        if (it + 2 < ntiles) issue_tile(n0 + 2 * kAT, next_buf);
        if (n0 > wave_last) return;  // every key of the tile is in this wave's future

        // ---- scores: two 32-key blocks, interleaved accumulation chains ----
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
        auto a_at = [&](int i) -> u32x4 {  // i = 2 s + kb
            const int s = i >> 1, kb = i & 1;
            const int rowb = s < DN / 16 ? DN * 2 : DR * 2;
            return *reinterpret_cast<const u32x4 *>(tb + sk[s] + 32 * kb * rowb);
        };
        u32x4 abuf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) abuf[i] = a_at(i);
        // Raised wave priority over each MFMA block: of the two waves sharing a
        // SIMD, the one in its MFMA phase issues first, so the other's softmax
        // arithmetic fills the matrix core's busy cycles instead of both
        // waves running the same phase in lockstep after the barrier.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < 2 * (DQK / 16); ++i) {
            sacc[i & 1] = mfma32(abuf[i & 3], qreg[i >> 1], sacc[i & 1]);
            if (i + 4 < 2 * (DQK / 16)) abuf[i & 3] = a_at(i + 4);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);

        // ---- online softmax (lane = query column; sacc[kb][r] is key
        //      n0 + 32 kb + 8 (r / 4) + 4 half + r % 4) ----
        if (n0 + kAT - 1 > wave_min_pos) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int n = n0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
                    if (n > pos) sacc[kb][r] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mt = mx * c2;  // log2 units; -inf stays -inf
        if (__ballot(mt > m_run + kRescaleThreshold) != 0) {
            const float m_new = fmaxf(m_run, mt);
            const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[q][r] *= alpha;
        }
        // a query with no visible key yet keeps m = -inf: its scores are -inf, weights 0
        const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
        u32x4 pk[4];
        float psum = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int kb = ks >> 1, r = 8 * (ks & 1) + 2 * p;
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], c2, neg_m));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r + 1], c2, neg_m));
                psum += p0 + p1;
                pk[ks][p] = pack_bf16(p0, p1);
            }
        l_run += psum;

        // ---- O^T[dim][query] += V^T[dim][key] P^T[key][query] ----
        // K step ks covers keys 16 ks + 8 (e / 4) + 4 half + e % 4 (e = 0..7),
        // as the score accumulators hold them; block q = dims 32 q .. + 31.
        auto a_tr = [&](int ks, int q) -> u32x4 {
            const u32x2 lo = lds_read_tr4(tb + pv[q] + (16 * ks) * (DV * 2));
            const u32x2 hi = lds_read_tr4(tb + pv[q] + (16 * ks + 8) * (DV * 2));
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        u32x4 av[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = a_tr(0, i);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {  // i = 4 ks + q
            oacc[i & 3] = mfma32(av[i & 3], pk[i >> 2], oacc[i & 3]);
            if (i + 4 < 16) av[i & 3] = a_tr((i + 4) >> 2, (i + 4) & 3);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    if (ntiles > 0) issue_tile(0, 0);
    if (ntiles > 1) issue_tile(kAT, 1);
    int buf = 0;  // tile it lives in buffer it % 3
    for (int it = 0; it < ntiles; ++it) {
        const int nxt = buf == 0 ? 2 : buf - 1;  // (it + 2) % 3
        tile_step(it, tiles + buf * kATile, nxt);
        buf = buf == 2 ? 0 : buf + 1;
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    // oacc[q][r] is value dim 32 q + 8 (r / 4) + 4 half + r % 4 of query t.
    if (out_bf16) {
        // The wave's 32 query rows are staged as bf16 in the idle tile
        // buffers and written as whole 256-byte rows (a store straight from
        // the accumulators would touch 32 rows per instruction).
        __syncthreads();  // every wave is done with the last tile
        unsigned char *wstage = tiles + w * (32 * kAOutRow);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * q + 8 * g + 4 * half;
                *reinterpret_cast<u32x2 *>(wstage + l32 * kAOutRow + 2 * d) =
                    u32x2{pack_bf16(oacc[q][4 * g] * inv, oacc[q][4 * g + 1] * inv),
                          pack_bf16(oacc[q][4 * g + 2] * inv, oacc[q][4 * g + 3] * inv)};
            }
        __syncthreads();
        uint16_t *obase = reinterpret_cast<uint16_t *>(out) + ((static_cast<int64_t>(b) * T + q0) * H + h) * DV;
#pragma unroll
        for (int e = 0; e < 32 * 16 / 64; ++e) {
            const int idx = lane + 64 * e, r = idx >> 4, pc = idx & 15;
            if (q0 + r < T)
                *reinterpret_cast<u32x4 *>(obase + static_cast<int64_t>(r) * H * DV + 8 * pc) =
                    *reinterpret_cast<const u32x4 *>(wstage + r * kAOutRow + 16 * pc);
        }
        return;
    }
    if (t >= T) return;
    const int64_t orow = ((static_cast<int64_t>(b) * T + t) * H + h) * DV;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = 32 * q + 8 * g + 4 * half;
            const float o0 = oacc[q][4 * g] * inv, o1 = oacc[q][4 * g + 1] * inv;
            const float o2 = oacc[q][4 * g + 2] * inv, o3 = oacc[q][4 * g + 3] * inv;
            if (out_bf16) {
                const u32x2 v = {pack_bf16(o0, o1), pack_bf16(o2, o3)};
                *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(out) + orow + d) = v;
            } else {
                const f32x4 v = {o0, o1, o2, o3};
                *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + orow + d) = v;
            }
        }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillShape &s, const void *q_nope, const void *q_rope,
                               const void *w_uk, const void *w_uv, const void *ckv,
                               const void *kpe, const int32_t *seqlens, void *out, void *kbuf,
                               void *vbuf, hipStream_t st)
{
    // K and V are [B][H][n_max][128] bf16 in the workspace.
    dim3 ggrid(s.H, static_cast<unsigned>((s.n_max + kGN - 1) / kGN), s.B);
    decompress_gemm_bf16_kernel<<<ggrid, kGThreads, 0, st>>>(
        s.H, s.n_max, static_cast<const uint16_t *>(w_uk), static_cast<const uint16_t *>(w_uv),
        static_cast<const uint16_t *>(ckv), s.ckv_sb, static_cast<int>(s.ckv_sn * 2), seqlens,
        static_cast<uint16_t *>(kbuf), static_cast<uint16_t *>(vbuf));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nqb = (s.T + kAQ - 1) / kAQ;
    const unsigned nblk = static_cast<unsigned>(nqb) * static_cast<unsigned>(s.B * s.H);
    prefill_attn_bf16_kernel<<<nblk, kAThreads, 0, st>>>(
        s.T, s.H, s.B, nqb, s.n_max, static_cast<const uint16_t *>(q_nope),
        static_cast<const uint16_t *>(q_rope), static_cast<const uint16_t *>(kpe), s.kpe_sb,
        static_cast<int>(s.kpe_sn * 2), seqlens, static_cast<const uint16_t *>(kbuf),
        static_cast<const uint16_t *>(vbuf), s.scale * kLog2e, out, s.out_bf16);
    return hipGetLastError();
}

}  // namespace mla
