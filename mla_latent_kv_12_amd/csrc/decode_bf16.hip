// decode_bf16.hip -- absorbed MLA decode for the DeepSeek-V2/V3 shape on
// gfx950: d_c = 512 latent, d_r = 64 decoupled RoPE key, d_n = d_v = 128,
// heads a multiple of 128, bf16 storage, fp32 accumulation.
//
// Three kernels on the caller's stream:
//   1. absorb:  Qa[b][h] = [ W_UK[h]^T q_nope[b][h] ; q_rope[b][h] ]   (bf16, 576 wide)
//      ("DeepSeek MLA Architecture: How It Cuts KV Cache by 93%", section 2:
//      the up-projection is folded into the query, so keys are never built.)
//   2. split-KV flash-decode: one workgroup per (work item, 128 heads), a
//      work item being a range of one query row's context (the absorb
//      launch plans them from the sequence lengths, so long and short
//      sequences spread evenly over the compute units).  Cache rows (576 bf16 = 1152 B) are streamed into LDS once
//      and shared by all 128 heads -- the absorbed decode is MQA-shaped.
//      Scores S^T[token][head] = C . Qa^T and the latent accumulation
//      O^T[col][head] += C^T . P^T both run on v_mfma_f32_32x32x16_bf16.
//      Online softmax in log2 units with a lazily raised running max.
//      ("mla-from-scratch" README, "Absorption, and why RoPE breaks it":
//      score = absorbed content term + decoupled positional term; attend
//      over the latents and up-project once at the end.)
//   3. merge + up-project: fixed-order (ascending range) combination of a
//      row's partials, then out = W_UV[h] o_lat.
#include <hip/hip_runtime.h>
#include <math.h>

#include "cdna4.h"
#include "mla_internal.h"

namespace mla {
namespace {

using namespace cdna4;

constexpr int DC = 512, DR = 64, DQK = DC + DR, DN = 128, DV = 128;

// ---------------------------------------------------------------------------
// 0. work plan, built by one workgroup of the absorb launch: the item table
//    [items] = (query row or -1 for none, first tile, end tile, 0) that the
//    split-KV grid walks, and the row table [rows] = (first item, item
//    count) that the merge walks; a row's items are consecutive and in
//    ascending tile order.  With a fixed split count S, item v S + sp is
//    split sp of row v (equal ranges of ceil(nt / S) tiles).  Otherwise the
//    balanced plan: every active row cut into ranges of C tiles (the last
//    one shorter), C found by bisection over plan_bounds' interval.
// ---------------------------------------------------------------------------
struct PlanArgs {
    int rows, T, fixed_S, capacity, target;
    int64_t n_max;
    int4 *items;
    int2 *row_tab;
};

__device__ __forceinline__ int tiles_of(int L) { return (L + kSplitGranule - 1) / kSplitGranule; }

// Exclusive prefix sum of x over the workgroup's 256 threads in thread
// order; *total gets the sum of all.  tmp: 4 ints of LDS.
__device__ int block_scan256(int x, int *total, int *tmp)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(inc, o);
        if (lane >= o) inc += u;
    }
    __syncthreads();  // the previous call's readers of tmp are done
    if (lane == 63) tmp[w] = inc;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = tmp[i];
        before += i < w ? t : 0;
        all += t;
    }
    *total = all;
    return before + inc - x;
}

// Sum (is_max = false) or maximum over the workgroup's 256 threads, returned
// to all of them.  tmp: 4 values of LDS.
template <typename V>
__device__ V block_all256(V x, V *tmp, bool is_max)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const V u = __shfl_xor(x, o);
        x = is_max ? max(x, u) : x + u;
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = x;
    __syncthreads();
    V r = tmp[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) r = is_max ? max(r, tmp[i]) : r + tmp[i];
    return r;
}

__device__ void build_plan(const PlanArgs &a, const int32_t *seqlens)
{
    __shared__ int s_nt[256], s_row[256], s_off[256];
    __shared__ int s_tmp[4];
    __shared__ long long s_sum[4];
    const int tid = threadIdx.x;
    auto row_tiles = [&](int v) {
        const int b = v / a.T;
        return tiles_of(query_len(seqlens[b], a.n_max, a.T, v - b * a.T));
    };
    if (a.fixed_S > 0) {  // capacity == rows * S
        const int S = a.fixed_S;
        for (int g = tid; g < a.capacity; g += 256) {
            const int v = g / S, sp = g - v * S;
            const int nt = row_tiles(v);
            const int tps = (nt + S - 1) / S;
            const int t0 = min(nt, sp * tps);
            a.items[g] = make_int4(v, t0, min(nt, t0 + tps), 0);
            if (sp == 0) a.row_tab[v] = make_int2(v * S, S);
        }
        return;
    }
    // Tile counts: total, maximum, active rows, and the first 256 active
    // rows (all of them whenever the width is searched) in row order.
    long long tot = 0;
    int mx = 0, active = 0;
    for (int v0 = 0; v0 < a.rows; v0 += 256) {
        const int v = v0 + tid;
        const int nt = v < a.rows ? row_tiles(v) : 0;
        tot += nt;
        mx = max(mx, nt);
        int n_act;
        const int k = active + block_scan256(nt > 0 ? 1 : 0, &n_act, s_tmp);
        if (nt > 0 && k < 256) {
            s_nt[k] = nt;
            s_row[k] = v;
        }
        active += n_act;
    }
    tot = block_all256<long long>(tot, s_sum, false);
    mx = block_all256<int>(mx, s_tmp, true);
    int C = max(mx, 1);  // as many active rows as items or more: one item per row
    if (active > 0 && active < a.target) {
        int lo, hi;
        plan_bounds(tot, active, mx, a.target, &lo, &hi);
        while (lo < hi) {  // the sums reach every thread: the loop is uniform
            const int mid = lo + (hi - lo) / 2;
            const int n = block_all256<int>(tid < active ? (s_nt[tid] + mid - 1) / mid : 0, s_tmp, false);
            if (n <= a.target) hi = mid; else lo = mid + 1;
        }
        C = lo;
    }
    // Rows in chunks of 256: item counts, their offsets, the row table; then
    // the chunk's items, each thread finding its item's row by bisection
    // over the chunk's offsets (rows without items share the next row's
    // offset, so the last entry at or below the item is its row).
    int carry = 0;
    for (int v0 = 0; v0 < a.rows; v0 += 256) {
        const int v = v0 + tid;
        const int nt = v < a.rows ? row_tiles(v) : 0;
        const int cnt = nt > 0 ? (nt + C - 1) / C : 0;
        int n_chunk;
        const int off = carry + block_scan256(cnt, &n_chunk, s_tmp);
        if (v < a.rows) a.row_tab[v] = make_int2(off, cnt);
        s_off[tid] = off;
        s_nt[tid] = nt;
        s_row[tid] = v;
        __syncthreads();
        for (int g = carry + tid; g < carry + n_chunk && g < a.capacity; g += 256) {
            int lo = 0, hi = 255;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_off[mid] <= g) lo = mid; else hi = mid - 1;
            }
            const int k = g - s_off[lo];
            a.items[g] = make_int4(s_row[lo], k * C, min(s_nt[lo], (k + 1) * C), 0);
        }
        carry += n_chunk;
        __syncthreads();  // before the next chunk overwrites the tables
    }
    for (int g = carry + tid; g < a.capacity; g += 256) a.items[g] = make_int4(-1, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// 1. absorb on MFMA: grid (3, H, ceil(rows / 128)), 256 threads.
//    x = 0, 1: columns 256 x .. 256 x + 255 of q~ = W_UK[h]^T q_nope for
//    head y and query rows 128 z .. 128 z + 127.  The workgroup copies its
//    W_UK[h] slice (128 x 256 bf16, 64 KiB) into LDS once, then computes
//    q~^T[col][row] = sum_k W[k][col] q[row][k] on v_mfma_f32_32x32x16_bf16
//    in blocks of 32 rows: A = W columns through the transposing LDS read,
//    B = query rows straight from global memory; wave w takes columns
//    64 w .. 64 w + 63 of the 256.  So W_UK is read from memory once per
//    128 query rows, and the product costs a few MFMAs per wave.  The x = 0
//    workgroups also place the RoPE query channels beside q~, rotated at
//    the query's position when rope_base > 0 (RoFormer pairs (2i, 2i+1)
//    turned by pos * rope_base^(-2i/d_r), angle and rotation in fp64,
//    rounded through fp32 to bf16).
//    x = 2: workgroup (2, 0, 0) builds the work plan; the others exit.
//
//    LDS: W row k (512 bytes) at k * 512, its 16-byte chunk c stored at
//    chunk c ^ 4 (k mod 4).  A transposing read takes 4 consecutive rows x
//    16 columns per group of 16 lanes, and the two groups of a 32-lane pass
//    take neighbouring columns of the same rows: with the swizzle their 16
//    chunks cover the 256-byte bank window once.
// ---------------------------------------------------------------------------
constexpr int kAbsorbRows = 128;   // query rows per workgroup (4 MFMA blocks of 32)
constexpr int kAbsorbCols = 256;   // q~ columns per workgroup
constexpr int kWRowBytes = kAbsorbCols * 2;

__device__ __forceinline__ unsigned w_swz(int k, int chunk) { return static_cast<unsigned>(chunk ^ (4 * (k & 3))); }

__global__ __launch_bounds__(256) void absorb_bf16_kernel(int B, int H, int T, int64_t n_max,
                                                          const int32_t *seqlens, double rope_base,
                                                          const uint16_t *q_nope,
                                                          const uint16_t *q_rope,
                                                          const uint16_t *w_uk, uint16_t *qa,
                                                          PlanArgs plan)
{
    if (blockIdx.x == 2) {
        if (blockIdx.y == 0 && blockIdx.z == 0) build_plan(plan, seqlens);
        return;
    }
    __shared__ __attribute__((aligned(1024))) unsigned char wt[DN * kWRowBytes];
    const int half = blockIdx.x, h = blockIdx.y, row0 = blockIdx.z * kAbsorbRows;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nrows = min(kAbsorbRows, B - row0);

    // W_UK[h][k][256 half .. + 255] -> LDS: wave w copies rows 32 w .. 32 w + 31,
    // two rows (1 KiB) per load; lane i lands at chunk i % 32 of row
    // 2 j + i / 32 and fetches the source chunk that belongs there.
    {
        const i32x4 rs = make_rsrc(w_uk + static_cast<int64_t>(h) * DN * DC, DN * DC * 2);
        const uint32_t base = lds_addr(wt);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int k = 32 * wu + 2 * j + (lane >> 5), p = lane & 31;
            lds_dma16(rs, base + (32 * wu + 2 * j) * kWRowBytes,
                      static_cast<unsigned>(k * DC * 2 + half * kWRowBytes + 16 * w_swz(k, p)));
        }
    }

    // RoPE query channels beside q~ (x = 0 only): one pair per thread, 8
    // rows per pass.
    if (half == 0) {
        for (int e = tid; e < nrows * (DR / 2); e += 256) {
            const int rv = row0 + e / (DR / 2), ri = e % (DR / 2);
            const int64_t rrow = static_cast<int64_t>(rv) * H + h;
            uint32_t two = *reinterpret_cast<const uint32_t *>(q_rope + rrow * DR + 2 * ri);
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
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // A operand (W^T, rows = columns of q~, K = k): lane l takes column
    // 64 w + 32 nb + l % 32 and k = 16 s + 8 (l / 32) .. + 7 as two
    // transposing reads of 4 rows; in its group of 16 lanes, lane a
    // addresses row 4 (a / 4) + (0 | 4) ... + 8 (l / 32) and the 4 columns
    // 16 (l / 16 % 2) + 4 (a % 4) .. + 3 of the block.
    const int a16 = lane & 15, G = lane >> 4;
    const int krow = 8 * (G >> 1) + (a16 >> 2);               // + 16 s, + 4 for the second read
    const int ccol = 64 * wu + 16 * (G & 1) + 4 * (a16 & 3);  // + 32 nb
    auto a_op = [&](int s, int nb) -> u32x4 {
        u32x2 v[2];
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
            const int k = 16 * s + krow + 4 * hlf, c = ccol + 32 * nb;
            v[hlf] = lds_read_tr4(wt + k * kWRowBytes + 16 * w_swz(k, c >> 3) + 8 * ((c >> 2) & 1));
        }
        return u32x4{v[0][0], v[0][1], v[1][0], v[1][1]};
    };
    for (int mb = 0; mb * 32 < nrows; ++mb) {
        // B operand: query row row0 + 32 mb + l % 32 (clamped), k = 16 s + 8 (l / 32) .. + 7
        const int rv = row0 + 32 * mb + (lane & 31);
        const uint16_t *qrow = q_nope + (static_cast<int64_t>(min(rv, B - 1)) * H + h) * DN + 8 * (lane >> 5);
        u32x4 qb[DN / 16];
#pragma unroll
        for (int s = 0; s < DN / 16; ++s) qb[s] = *reinterpret_cast<const u32x4 *>(qrow + 16 * s);
        f32x16 acc[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[nb][r] = 0.f;
#pragma unroll
        for (int s = 0; s < DN / 16; ++s)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) acc[nb] = mfma32(a_op(s, nb), qb[s], acc[nb]);
        // acc[nb][r]: q~ row rv, column 256 half + 64 w + 32 nb + 8 (r / 4) + 4 (l / 32) + r % 4
        if (rv < B) {
            uint16_t *dst = qa + (static_cast<int64_t>(rv) * H + h) * DQK + half * kAbsorbCols + 64 * wu +
                            4 * (lane >> 5);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<u32x2 *>(dst + 32 * nb + 8 * j) =
                        u32x2{pack_bf16(acc[nb][4 * j], acc[nb][4 * j + 1]),
                              pack_bf16(acc[nb][4 * j + 2], acc[nb][4 * j + 3])};
        }
    }
}

// ---------------------------------------------------------------------------
// 2. split-KV flash-decode
//
// Workgroup = 8 waves = 128 heads of one query row over one context split,
// two waves per SIMD.  Cache tiles of 32 rows x 576 bf16 (36 KiB) are copied
// HBM -> LDS with direct-to-LDS 16-byte buffer loads (non-temporal: a decode
// call reads each row once) into four tile buffers; the buffer descriptor's
// range ends at the split's last row, so rows past it arrive as zeros.
//
// The waves come in four pairs; pair p owns heads 32p .. 32p + 31 of the
// workgroup's 128, and the two waves of a pair split the work of those heads:
//   score   S[head][token] = Qa . C^T over the 576-wide row, for the 16 heads
//           of the wave's half of the pair (v_mfma_f32_16x16x32_bf16, A = the
//           absorbed query held in VGPRs, B = cache rows from LDS);
//   softmax weights of those 16 heads, written to LDS as bf16 [token][head];
//   latent  O^T[col][head] += C^T . P^T for all 32 heads of the pair and the
//           wave's half of the 512 latent columns (v_mfma_f32_32x32x16_bf16,
//           A = cache columns, B = the pair's softmax weights, both through
//           the transposing LDS read), 128 accumulator registers.
// A wave therefore needs 128 accumulator + 72 query registers and fits two to
// a SIMD, so one wave's softmax and waits run under the other's MFMAs.  Each
// LDS read of the cache tile serves 16 heads (score) or 32 heads (latent).
//
// Pipeline, one workgroup barrier per tile: iteration i (after the barrier
// that publishes tile i + 1 and the weights P(i)) issues the loads of tile
// i + 3, computes the scores of tile i + 1 and writes their weights P(i + 1),
// then the latent products of tile i.  Tiles i .. i + 3 occupy the four
// buffers; P is double-buffered.  The two waves of a SIMD drift apart within
// an iteration, so one's softmax overlaps the other's MFMAs.
//
// LDS tile layout: latent row r at r * 1024, its 16-byte chunk c stored at
// chunk c ^ phase(r), phase(r) = 4 (r mod 4) + (r div 4 mod 4) (an
// involution).  The 32 RoPE-key rows of 128 bytes follow, chunk c of row r
// at c ^ rphase(r), rphase(r) = (r div 4 mod 4) + 4 (r div 2 mod 2).  The
// loads place the chunks by gathering each lane's source chunk accordingly.
// Bank behaviour measured on gfx950 (LDS bank-conflict counter): a 16-byte
// read is conflict-free when, in each group of four consecutive lanes, the
// lanes hit the four chunks of one 64-byte block of the 256-byte bank
// window; a transposing read when the 32 lanes of each half hit 32 distinct
// 8-byte slots.  The score read therefore takes the 16 tokens of a block in
// the order phase(i) (lane i reads row phase(i), whose chunk 4 s + g then
// sits at (4 s + g) ^ i), and the transposing reads take 4 consecutive rows;
// both are conflict-free on this layout, and so are the weight reads.
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
constexpr int kRopeRow = DR * 2;                // 128 B
constexpr int kRopeOff = kTile * kLatRow;       // 32768: RoPE rows follow the latent rows
constexpr int kTileBytes = kRopeOff + kTile * kRopeRow;  // 36864
constexpr int kTileBufs = 4;
constexpr int kPBytes = 128 * kTile * 2;        // softmax weights, 128 heads x 32 tokens (bf16)
constexpr int kThreadsDec = 512;                // 8 waves, two per SIMD
constexpr int kStageRow = 256 + 4;              // floats per staged partial row (bank stagger)
static_assert(kTile == kSplitGranule, "split boundaries must align to tiles");
static_assert(kTileBufs * kTileBytes + 2 * kPBytes <= 160 * 1024, "LDS budget");
static_assert(128 * kStageRow * 4 <= kTileBufs * kTileBytes, "partial rows are staged in the tile buffers");
constexpr float kRefSlack = 64.0f;              // log2 headroom above the reference maximum
constexpr int kLookS = 4;                       // score operand reads in flight
constexpr int kLookP = 2;                       // latent-product operand reads in flight

// 16-byte chunk phase of latent row r (XOR applied to the chunk index); an
// involution on 0..15: lat_phase(lat_phase(r)) = r for r < 16.
__host__ __device__ constexpr int lat_phase(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }
// 16-byte chunk phase of RoPE row r (0..7).
__host__ __device__ constexpr int rope_phase(int r) { return ((r >> 2) & 3) + 4 * ((r >> 1) & 1); }
static_assert(lat_phase(lat_phase(13)) == 13 && lat_phase(lat_phase(6)) == 6, "phase is an involution");

template <int N>
__device__ __forceinline__ void vm_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__global__ __launch_bounds__(kThreadsDec, 1) void decode_splitkv_bf16_kernel(
    int T, int H, const int4 *__restrict__ plan_items, int64_t n_max,
    const uint16_t *__restrict__ ckv, int64_t ckv_sb, int ckv_rowb,
    const uint16_t *__restrict__ kpe, int64_t kpe_sb, int kpe_rowb,
    const int32_t *__restrict__ seqlens, const uint16_t *__restrict__ qa, float c2,
    float *__restrict__ part_o, float *__restrict__ part_ml)
{
    __shared__ __attribute__((aligned(1024))) unsigned char tiles[kTileBufs * kTileBytes];
    __shared__ __attribute__((aligned(16))) unsigned char pbuf[2 * kPBytes];

    // Work item = a range of tiles of query row v = b * T + t: query t of
    // sequence b (T = 1 for decode) attends to the causal prefix of its
    // sequence's cache.
    const int item = blockIdx.x, hg = blockIdx.y;
    const int4 work = plan_items[item];
    const int v = work.x;
    if (v < 0) return;  // unused item: nothing reads its partials
    const int b = v / T, tq = v - b * T;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index, known uniform
    const int pr = wu & 3, role = wu >> 2;      // pair, and this wave's half of it
    const int l16 = lane & 15, g = lane >> 4;   // 16x16x32 layout: row/column, K slice
    const int l32 = lane & 31, hh = lane >> 5;  // 32x32x16 layout: row/column, K half
    const int hs0 = hg * 128 + 32 * pr + 16 * role;       // first of this wave's 16 score heads
    const int hs = hs0 + l16;                              // query row of this lane (score A operand)

    const int L = query_len(seqlens[b], n_max, T, tq);
    const int start = work.y * kTile;
    const int end = min(L, work.z * kTile);

    if (start >= end) {  // empty split: weight zero in the merge, O never read
        if (g == 0) {
            const int64_t prow = static_cast<int64_t>(item) * H + hs;
            part_ml[prow * 2 + 0] = -INFINITY;
            part_ml[prow * 2 + 1] = 0.f;
        }
        return;
    }
    const int ntiles = (end - start + kTile - 1) / kTile;

    // ---- loads: wave w places latent rows 4w .. 4w + 3 of each tile, and
    // waves 0..3 also RoPE rows 8w .. 8w + 7 (one 1-KiB load).  Each tile's
    // buffer descriptors start at its first row and end at the split's last
    // row, so rows past the end read as zeros and never reach memory. ----
    const unsigned char *lat_seq =
        reinterpret_cast<const unsigned char *>(ckv + static_cast<int64_t>(b) * ckv_sb);
    const unsigned char *rope_seq =
        reinterpret_cast<const unsigned char *>(kpe + static_cast<int64_t>(b) * kpe_sb);
    const uint32_t tiles_lds = lds_addr(tiles);
    auto issue_tile = [&](int t) {
        const int n0 = start + t * kTile;
        const uint32_t dst = tiles_lds + static_cast<uint32_t>(t & 3) * kTileBytes;
        const i32x4 rs_lat = make_rsrc(lat_seq + static_cast<int64_t>(n0) * ckv_rowb,
                                       static_cast<uint32_t>(end - n0) * ckv_rowb);
        // The per-lane source offsets are rebuilt for every tile from a lane
        // index the compiler cannot see through, so that they are not kept
        // live (the loop's registers are all taken).
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int k = 0; k < 4; ++k)   // row 4w + k: LDS chunk ln holds source chunk ln ^ phase
            lds_dma16_stream(rs_lat, dst + (4 * wu + k) * kLatRow,
                             static_cast<unsigned>((4 * wu + k) * ckv_rowb + 16 * (ln ^ lat_phase(4 * wu + k))));
        if (wu < 4) {  // RoPE rows 8w + ln / 8, LDS chunk ln % 8 holding source chunk (ln % 8) ^ rphase
            const i32x4 rs_rope = make_rsrc(rope_seq + static_cast<int64_t>(n0) * kpe_rowb,
                                            static_cast<uint32_t>(end - n0) * kpe_rowb);
            const int rq = 8 * wu + (ln >> 3);
            lds_dma16_stream(rs_rope, dst + kRopeOff + wu * 8 * kRopeRow,
                             static_cast<unsigned>(rq * kpe_rowb + 16 * ((ln & 7) ^ rope_phase(rq))));
        }
    };
    // Wait until this wave's loads of tile t have landed, given whether the
    // next tile's loads were issued after them (5 loads per tile on waves
    // 0..3, 4 on waves 4..7), then meet the other waves.
    auto wait_tile_then_barrier = [&](bool next_in_flight) {
        if (wu < 4) {
            if (next_in_flight) vm_wait<5>(); else vm_wait<0>();
        } else {
            if (next_in_flight) vm_wait<4>(); else vm_wait<0>();
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    issue_tile(0);
    if (ntiles > 1) issue_tile(1);

    // Absorbed query of head l16 of the wave's 16 as the 16x16x32 A operand:
    // K step s holds channels 32 s + 8 g .. + 7 (s < 16 latent, s = 16, 17 RoPE).
    const uint16_t *qrow = qa + (static_cast<int64_t>(v) * H + hs) * DQK + 8 * g;
    u32x4 qreg[DQK / 32];
#pragma unroll
    for (int s = 0; s < DQK / 32; ++s) qreg[s] = *reinterpret_cast<const u32x4 *>(qrow + 32 * s);
    // Let the query loads land here, once (they also retire tiles 0 and 1):
    // the compiler then puts no wait on them inside the tile loop.
    __builtin_amdgcn_s_waitcnt(0);
    if (ntiles > 2) issue_tile(2);
    // From here on this wave's vector-memory operations are tile loads only,
    // issued in tile order, so "tile t landed" is a count of loads in flight.

    // ---- per-lane LDS offsets within a tile (immediates added per access) ----
    // Only one base per access pattern stays live through the loop; the
    // variants that differ from it by an XOR of a few address bits are formed
    // at the start of each phase (from an opaque copy, so that the compiler
    // does not hoist them out of the loop: its registers are all taken).
    //
    // Score B operand, token block tb, K step s < 16: MFMA column l16 is row
    // 16 tb + phase(l16) (its token), logical chunk 4 s + g, stored at chunk
    // (4 s + g) ^ l16: byte (sc0 ^ 64 (s & 3)) + 16384 tb + 256 (s >> 2).
    const unsigned sc0 = lat_phase(l16) * kLatRow + 64 * (l16 >> 2) + 16 * (g ^ (l16 & 3));
    // RoPE steps s = 16 + s2: logical chunk 4 s2 + g of RoPE row 16 tb +
    // phase(l16), at chunk (4 s2 + g) ^ rphase(row): byte (rp0 ^ 64 s2) + 2048 tb.
    const unsigned rp0 = kRopeOff + lat_phase(l16) * kRopeRow + 64 * ((l16 >> 3) & 1) + 16 * (g ^ (l16 & 3));
    // Latent-product A operand through the transposing read: column block q
    // (32 columns of this wave's half), K step ks, read ri.  Source lane
    // 4 k + c of 16-lane group G addresses token 16 ks + 8 (G >> 1) + 4 ri + k,
    // columns 256 role + 32 q + 16 (G & 1) + 4 c; the lane then holds column
    // 32 q + (lane & 31), tokens 16 ks + 8 (lane >> 5) + 4 ri + 0..3.  With
    // ri = 0 the byte offset is (pv0 ^ 64 (q & 3)) + 16384 ks + 256 (q >> 2);
    // ri = 1 (4 rows on, chunk bit 0 flipped) adds 4096 to that with bit 4
    // flipped.
    const unsigned pv0 = [&] {
        const int kk = l16 >> 2, cc = l16 & 3, G = lane >> 4, h2 = G >> 1;
        const int a = 2 * (G & 1) + (cc >> 1);
        return static_cast<unsigned>((8 * h2 + kk) * kLatRow + 512 * role + 64 * kk +
                                     16 * (a ^ ((2 * h2) & 3)) + 8 * (cc & 1));
    }();
    // Softmax weights in LDS: [pair][32 tokens][32 heads] bf16 (64-byte rows),
    // the 16-byte chunk c of token row t at c ^ (t div 4 mod 4).  This lane
    // writes heads 16 role + 4 g .. + 3 of token 16 tb + phase(l16).  The
    // latent product reads them back as its B operand through the
    // transposing read: source lane 4 k + c of group G addresses token
    // 16 ks + 8 (G >> 1) + 4 ri + k, heads 16 (G & 1) + 4 c .. + 3, so the
    // lane holds head lane & 31, tokens 16 ks + 8 hh + 4 ri + 0..3 (the same
    // tokens as its A operand).  ri = 1 is 4 rows on with chunk bit 0 flipped.
    const uint32_t pw_off = pr * 2048 + lat_phase(l16) * 64 + 16 * ((2 * role + (g >> 1)) ^ (l16 & 3)) + 8 * (g & 1);
    const uint32_t pr_off = [&] {
        const int kk = l16 >> 2, cc = l16 & 3, G = lane >> 4;
        return static_cast<uint32_t>(pr * 2048 + (8 * (G >> 1) + kk) * 64 +
                                     16 * ((2 * (G & 1) + (cc >> 1)) ^ ((2 * (G >> 1)) & 3)) + 8 * (cc & 1));
    }();

    f32x16 oacc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[q][r] = 0.f;
    // Softmax state of this lane's 4 score heads 4 g + r (r = 0..3).
    float m_ref[4];           // the split's first tile's maximum, per head
    float l_run[4];           // this lane's share of each head's softmax mass
#pragma unroll
    for (int r = 0; r < 4; ++r) { m_ref[r] = -INFINITY; l_run[r] = 0.f; }
    int over = 0;             // bit r: a later score of head 4 g + r exceeded its m_ref + 64

    // Scores of tile t (buffer t & 3) for this wave's 16 heads: sacc[tb][r] is
    // head 4 g + r, token 16 tb + phase(l16).
    auto scores = [&](int t, f32x4 (&sacc)[2]) {
        const unsigned char *tb = tiles + (t & 3) * kTileBytes;
        unsigned sb = sc0, rb = rp0;
        asm volatile("" : "+v"(sb), "+v"(rb));
        const unsigned sc_base[4] = {sb, sb ^ 64u, sb ^ 128u, sb ^ 192u};
        const unsigned rp_base[2] = {rb, rb ^ 64u};
        auto a_at = [&](int i) -> u32x4 {  // i = 2 s + token block
            const int s = i >> 1, blk = i & 1;
            if (s < DC / 32)
                return *reinterpret_cast<const u32x4 *>(tb + sc_base[s & 3] + 16384 * blk + 256 * (s >> 2));
            return *reinterpret_cast<const u32x4 *>(tb + rp_base[s - DC / 32] + 2048 * blk);
        };
        sacc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        sacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x4 abuf[kLookS];
#pragma unroll
        for (int i = 0; i < kLookS; ++i) abuf[i] = a_at(i);
#pragma unroll
        for (int i = 0; i < 2 * (DQK / 32); ++i) {
            sacc[i & 1] = mfma16(qreg[i >> 1], abuf[i % kLookS], sacc[i & 1]);
            if (i + kLookS < 2 * (DQK / 32)) abuf[i % kLookS] = a_at(i + kLookS);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Softmax weights of tile t from its scores, written to P buffer t & 1.
    auto softmax = [&](int t, f32x4 (&sacc)[2]) {
        const int n0 = start + t * kTile;
        const int tok0 = n0 + lat_phase(l16);  // this lane's token of block 0
        float lmax[4];
        if (n0 + kTile <= end) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sacc[0][r] *= c2;
                sacc[1][r] *= c2;
                lmax[r] = fmaxf(sacc[0][r], sacc[1][r]);
            }
        } else {  // the split's last, partial tile
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sacc[0][r] = tok0 < end ? sacc[0][r] * c2 : -INFINITY;
                sacc[1][r] = tok0 + 16 < end ? sacc[1][r] * c2 : -INFINITY;
                lmax[r] = fmaxf(sacc[0][r], sacc[1][r]);
            }
        }
        if (t == 0) {  // each head's maximum over the first tile: its 16 lanes
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float m = lmax[r];
                m = fmaxf(m, __shfl_xor(m, 1));
                m = fmaxf(m, __shfl_xor(m, 2));
                m = fmaxf(m, __shfl_xor(m, 4));
                m = fmaxf(m, __shfl_xor(m, 8));
                m_ref[r] = m;
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) over |= static_cast<int>(lmax[r] > m_ref[r] + kRefSlack) << r;
        unsigned char *pw = pbuf + (t & 1) * kPBytes + pw_off;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[r] = __builtin_amdgcn_exp2f(sacc[tb][r] - m_ref[r]);
                l_run[r] += p[r];
            }
            *reinterpret_cast<u32x2 *>(pw + 1024 * tb) = u32x2{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
        }
    };
    // Latent products of tile t with the pair's weights from P buffer t & 1.
    auto latent = [&](int t) {
        const unsigned char *tb = tiles + (t & 3) * kTileBytes;
        unsigned pq = (t & 1) * kPBytes + pr_off;
        asm volatile("" : "+v"(pq));
        auto p_tr = [&](int ks) -> u32x4 {
            const u32x2 lo = lds_read_tr4(pbuf + pq + 1024 * ks);
            const u32x2 hi = lds_read_tr4(pbuf + (pq ^ 16u) + 256 + 1024 * ks);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        const u32x4 pk0 = p_tr(0);
        const u32x4 pk1 = p_tr(1);
        unsigned pb = pv0;
        asm volatile("" : "+v"(pb));
        const unsigned pv_base[4][2] = {{pb, (pb ^ 16u) + 4096u},
                                        {pb ^ 64u, (pb ^ 80u) + 4096u},
                                        {pb ^ 128u, (pb ^ 144u) + 4096u},
                                        {pb ^ 192u, (pb ^ 208u) + 4096u}};
        auto a_tr = [&](int i) -> u32x4 {  // i = 8 ks + q
            const int ks = i >> 3, q = i & 7;
            const u32x2 lo = lds_read_tr4(tb + pv_base[q & 3][0] + 16384 * ks + 256 * (q >> 2));
            const u32x2 hi = lds_read_tr4(tb + pv_base[q & 3][1] + 16384 * ks + 256 * (q >> 2));
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        u32x4 av[kLookP];
#pragma unroll
        for (int i = 0; i < kLookP; ++i) av[i] = a_tr(i);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            oacc[i & 7] = mfma32(av[i % kLookP], (i >> 3) ? pk1 : pk0, oacc[i & 7]);
            if (i + kLookP < 16) av[i % kLookP] = a_tr(i + kLookP);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Prologue: tile 0's scores and weights.
    wait_tile_then_barrier(ntiles > 2);   // tiles 0 and 1 landed above; tile 0 visible to all
    {
        f32x4 sacc[2];
        scores(0, sacc);
        softmax(0, sacc);
    }
    for (int i = 0; i < ntiles; ++i) {
        // Tile i + 1 landed (tile i + 2 may still be in flight), P(i)
        // written, and every wave is done with tile i - 1's buffer.
        wait_tile_then_barrier(i + 2 < ntiles);
        if (i + 3 < ntiles) issue_tile(i + 3);
        if (i + 1 < ntiles) {
            f32x4 sacc[2];
            scores(i + 1, sacc);
            softmax(i + 1, sacc);
        }
        latent(i);
    }

    // ---- write the split partial: un-normalised O, reference max, mass ----
    // Pair p's 32 heads are rows 32 p .. 32 p + 31 of the workgroup's 128
    // consecutive 2-KiB rows of part_o.  Accumulator q, element r of this
    // lane is latent column 256 role + 32 q + 8 (r / 4) + 4 hh + r % 4 of
    // pair head l32.  The rows are staged in the (now idle) tile buffers, one
    // half of the columns (one role) at a time, and written as whole 1-KiB
    // row segments.
    // Each score head's mass and overflow mark over its 16 lanes.
    float l_tot[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float l = l_run[r];
        l += __shfl_xor(l, 1);
        l += __shfl_xor(l, 2);
        l += __shfl_xor(l, 4);
        l += __shfl_xor(l, 8);
        l_tot[r] = l;
    }
    int ov = over;
    ov |= __shfl_xor(ov, 1);
    ov |= __shfl_xor(ov, 2);
    ov |= __shfl_xor(ov, 4);
    ov |= __shfl_xor(ov, 8);
    float *stage = reinterpret_cast<float *>(tiles);  // [128 heads][kStageRow]
    float *obase = part_o + (static_cast<int64_t>(item) * H + hg * 128) * DC;
    __syncthreads();  // every wave is done with the last tile
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        if (role == half) {
#pragma unroll
            for (int q = 0; q < 8; ++q)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    *reinterpret_cast<f32x4 *>(stage + (32 * pr + l32) * kStageRow + 32 * q + 8 * m + 4 * hh) =
                        f32x4{oacc[q][4 * m], oacc[q][4 * m + 1], oacc[q][4 * m + 2], oacc[q][4 * m + 3]};
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 128 * 64 / kThreadsDec; ++e) {
            const int idx = tid + kThreadsDec * e, head = idx >> 6, piece = idx & 63;
            *reinterpret_cast<f32x4 *>(obase + head * DC + 256 * half + 4 * piece) =
                *reinterpret_cast<const f32x4 *>(stage + head * kStageRow + 4 * piece);
        }
        __syncthreads();
    }
    if (l16 == 0) {
        // NaN marks a (split, head) whose weights could overflow: the merge
        // kernel recomputes it with the split's true maximum.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = static_cast<int64_t>(item) * H + hs0 + 4 * g + r;
            part_ml[row * 2 + 0] = ((ov >> r) & 1) ? __builtin_nanf("") : m_ref[r];
            part_ml[row * 2 + 1] = l_tot[r];
        }
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
    const int4 *items;       // the work plan's item table
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

// Recompute one (work item, head) partial: scores against the item's rows,
// their maximum, then weights, mass and the weighted latent sum.
__device__ void recompute_partial(const CacheView &cv, int H, int item, int h, float *part_o,
                                  float *part_ml)
{
    __shared__ float q[DQK];
    __shared__ float pw[256];
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int4 work = cv.items[item];
    const int v = work.x, b = v / cv.T;
    const int L = query_len(cv.seqlens[b], cv.n_max, cv.T, v - b * cv.T);
    const int start = work.y * kSplitGranule;
    const int end = min(L, work.z * kSplitGranule);
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
    const int64_t prow = static_cast<int64_t>(item) * H + h;
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
__global__ __launch_bounds__(256) void merge_upproj_bf16_kernel(int H, const int2 *__restrict__ row_tab,
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

    // The row's splits are work items first .. first + S - 1, in ascending
    // order of their context ranges.
    const int2 rt = row_tab[v];
    const int first = rt.x, S = rt.y;
    if (S == 0) {  // no context: a zero row
        if constexpr (kUpProj) {
            const int64_t oi = (static_cast<int64_t>(v) * H + h) * DV + tid;
            if (tid < DV) {
                if (out_bf16) reinterpret_cast<uint16_t *>(out)[oi] = 0;
                else reinterpret_cast<float *>(out)[oi] = 0.f;
            }
        } else {
            const int64_t oi = (static_cast<int64_t>(v) * H + h) * DC + 2 * tid;
            if (out_bf16) *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(out) + oi) = 0u;
            else *reinterpret_cast<float2 *>(reinterpret_cast<float *>(out) + oi) = float2{0.f, 0.f};
        }
        return;
    }
    const int64_t base = static_cast<int64_t>(first) * H + h;  // row of split 0
    if constexpr (!kUpProj) {
        if (S == 1) {  // one split: o = O / l, no cross-split weighting
            float m0 = part_ml[base * 2], l0 = part_ml[base * 2 + 1];
            if (__builtin_isnan(m0)) {  // marked: recompute with the split's true maximum
                recompute_partial(cv, H, first, h, part_o, part_ml);
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
                recompute_partial(cv, H, first + sp, h, part_o, part_ml);
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
    int4 *plan_items = reinterpret_cast<int4 *>(ws.plan_items);
    int2 *plan_rows = reinterpret_cast<int2 *>(ws.plan_rows);
    {
        const PlanArgs plan{rows, s.T, s.S, s.items, plan_target(s.H), s.n_max, plan_items, plan_rows};
        dim3 grid(3, s.H, (rows + kAbsorbRows - 1) / kAbsorbRows);
        absorb_bf16_kernel<<<grid, 256, 0, st>>>(rows, s.H, s.T, s.n_max, seqlens, s.q_rope_base,
                                                 static_cast<const uint16_t *>(q_nope),
                                                 static_cast<const uint16_t *>(q_rope),
                                                 static_cast<const uint16_t *>(w_uk), qa, plan);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (events && events[1]) (void)hipEventRecord(events[1], st);
    {
        dim3 grid(s.items, s.H / 128);
        decode_splitkv_bf16_kernel<<<grid, kThreadsDec, 0, st>>>(
            s.T, s.H, plan_items, s.n_max, static_cast<const uint16_t *>(ckv), s.ckv_sb,
            static_cast<int>(s.ckv_sn * 2), static_cast<const uint16_t *>(kpe), s.kpe_sb,
            static_cast<int>(s.kpe_sn * 2), seqlens, qa, s.scale * kLog2e, ws.part_o, ws.part_ml);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (events && events[2]) (void)hipEventRecord(events[2], st);
    dim3 grid(s.H, rows);
    CacheView cv{s.T, s.n_max, static_cast<const uint16_t *>(ckv), s.ckv_sb, s.ckv_sn,
                 static_cast<const uint16_t *>(kpe), s.kpe_sb, s.kpe_sn, seqlens, qa,
                 s.scale * kLog2e, plan_items};
    hipError_t e;
    if (w_uv && batched_upproj(s, true)) {
        // many query rows: merge into fp32 latents, then one product per head
        merge_upproj_bf16_kernel<false><<<grid, 256, 0, st>>>(s.H, plan_rows, ws.part_o, ws.part_ml,
                                                              nullptr, ws.o_lat, 0, cv);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        dim3 ugrid(4 * s.H, (rows + 31) / 32);
        upproj_bf16_kernel<<<ugrid, 64, 0, st>>>(s.H, rows, ws.o_lat,
                                                  static_cast<const uint16_t *>(w_uv), out, s.out_bf16);
    } else if (w_uv) {
        merge_upproj_bf16_kernel<true><<<grid, 256, 0, st>>>(
            s.H, plan_rows, ws.part_o, ws.part_ml, static_cast<const uint16_t *>(w_uv), out, s.out_bf16, cv);
    } else {
        merge_upproj_bf16_kernel<false><<<grid, 256, 0, st>>>(
            s.H, plan_rows, ws.part_o, ws.part_ml, nullptr, out, s.out_bf16, cv);
    }
    e = hipGetLastError();
    if (events && events[3]) (void)hipEventRecord(events[3], st);
    return e;
}

}  // namespace mla
