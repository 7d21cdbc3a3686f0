// mla_api.hip -- the library's C ABI (declared in include/mla.h): host-side
// validation, workspace carving and kernel dispatch.  Nothing here allocates,
// frees or synchronises (except the opt-in MLA_DEBUG_CHECKS seqlens check).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "mla.h"
#include "mla_internal.h"

namespace {

thread_local char g_err[512] = "";

mla_status fail(mla_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

mla_status ok()
{
    g_err[0] = '\0';
    return MLA_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kAlign = 256;
constexpr int64_t kProjDirectGroups = 256;  // workgroups of the direct projection: one per CU
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// A cache's extent, (batch - 1) * stride_b + n_max * stride_n elements of
// `elt` bytes, stays below 2^62 bytes: every later product of sizes and
// strides (host checks and the kernels' 64-bit offsets) then fits in int64.
bool cache_span_ok(int64_t batch, int64_t n_max, int64_t stride_b, int64_t stride_n, int64_t elt)
{
    const __int128 span = (__int128)(batch - 1) * stride_b + (__int128)n_max * stride_n;
    return span * elt < ((__int128)1 << 62);
}

bool debug_checks()
{
    const char *e = getenv("MLA_DEBUG_CHECKS");
    return e && e[0] && strcmp(e, "0") != 0;
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------

bool f32_dims_ok(int64_t dc, int64_t dr, int64_t dn, int64_t dv)
{
    return dc >= 1 && dc <= 1024 && dr >= 0 && dr <= 256 && dn >= 1 && dn <= 512 && dv >= 1 &&
           dv <= 1024;
}

bool bf16_dims_ok(int64_t H, int64_t dc, int64_t dr, int64_t dn, int64_t dv)
{
    return dc == 512 && dr == 64 && dn == 128 && dv == 128 && H % 128 == 0;
}

// Split count of the fp32 path; rows = query rows (batch for decode, batch *
// tokens for absorbed prefill).
int auto_splits(int64_t rows, int64_t heads, int64_t n_max)
{
    // Enough (query row, head, split) blocks to cover the 256 compute units
    // about once, but at least four 32-token tiles of context per split so
    // the split partials stay small next to the cache rows they summarise.
    const int64_t tiles = (n_max + mla::kSplitGranule - 1) / mla::kSplitGranule;
    const int64_t groups = rows * heads;
    const int64_t target = 256;
    int64_t s = (target + groups - 1) / groups;
    int64_t cap = tiles / 4;
    if (s > cap) s = cap;
    if (s < 1) s = 1;
    if (s > mla::kMaxSplits) s = mla::kMaxSplits;
    return (int)s;
}

// Items the bf16 balanced plan gives one query row holding all n_max rows of
// its sequence (host-side report; the device builds the plan from the actual
// lengths).  B sequences of T queries: query t sees n_max - (T - 1 - t) rows.
int plan_splits_full(int64_t B, int64_t T, int64_t H, int64_t n_max)
{
    const int G = mla::plan_target((int)H);
    auto nt_of = [&](int64_t t) {
        const int64_t L = n_max - (T - 1 - t);
        return L > 0 ? (L + mla::kSplitGranule - 1) / mla::kSplitGranule : (int64_t)0;
    };
    int64_t tiles = 0, active = 0, max_nt = 0;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t nt = nt_of(t);
        tiles += B * nt;
        active += nt > 0 ? B : 0;
        max_nt = nt > max_nt ? nt : max_nt;
    }
    if (active == 0) return 0;
    if (active >= G) return 1;
    int lo, hi;
    mla::plan_bounds(tiles, (int)active, (int)max_nt, G, &lo, &hi);
    while (lo < hi) {
        const int mid = lo + (hi - lo) / 2;
        int64_t n = 0;
        for (int64_t t = 0; t < T; ++t) n += B * ((nt_of(t) + mid - 1) / mid);
        if (n <= G) hi = mid; else lo = mid + 1;
    }
    return (int)((max_nt + lo - 1) / lo);
}

// The bf16 path's plan for B * T query rows: a fixed split count S (> 0) or
// the balanced plan (S = 0).  The parameter checks bound B * T by 65535 and
// S by kMaxSplits, so the item count stays below 2^24.
void set_plan(mla::DecodeShape *s, int64_t B, int64_t T, int S)
{
    s->S = S;
    s->items = (int)mla::plan_capacity(B * T, s->H, S);
}

mla_status check_rope_base(double base, int64_t dr)
{
    if (!(base >= 0.0) || isinf(base) || (base > 0.0 && base <= 1.0))
        return fail(MLA_ERR_INVALID_ARG, "q_rope_base must be 0 (q_rope already rotated) or a finite value > 1");
    if (base > 0.0 && (dr & 1))
        return fail(MLA_ERR_UNSUPPORTED, "rotating q_rope needs an even d_r (rotation pairs)");
    return MLA_OK;
}

// Structural validation shared by the workspace query and the decode call.
mla_status check_decode_params(const mla_decode_params *p)
{
    if (!p) return fail(MLA_ERR_INVALID_ARG, "params is NULL");
    if (p->batch < 1 || p->heads < 1 || p->n_max < 1 || p->d_c < 1 || p->d_n < 1 || p->d_v < 1 ||
        p->d_r < 0)
        return fail(MLA_ERR_INVALID_ARG,
                    "non-positive size (batch=%lld heads=%lld n_max=%lld d_c=%lld d_r=%lld d_n=%lld d_v=%lld)",
                    (long long)p->batch, (long long)p->heads, (long long)p->n_max, (long long)p->d_c,
                    (long long)p->d_r, (long long)p->d_n, (long long)p->d_v);
    if (p->batch > 65535 || p->heads > 65535 || p->n_max > (int64_t)1 << 30)
        return fail(MLA_ERR_UNSUPPORTED, "batch, heads or n_max beyond the supported range");
    if ((p->dtype != MLA_F32 && p->dtype != MLA_BF16) ||
        (p->out_dtype != MLA_F32 && p->out_dtype != MLA_BF16))
        return fail(MLA_ERR_UNSUPPORTED, "unknown dtype %d / out_dtype %d", p->dtype, p->out_dtype);
    if (p->dtype == MLA_F32 && !f32_dims_ok(p->d_c, p->d_r, p->d_n, p->d_v))
        return fail(MLA_ERR_UNSUPPORTED,
                    "fp32 kernels support d_c<=1024, d_r<=256, d_n<=512, d_v<=1024");
    if (p->dtype == MLA_BF16 && !bf16_dims_ok(p->heads, p->d_c, p->d_r, p->d_n, p->d_v))
        return fail(MLA_ERR_UNSUPPORTED,
                    "bf16 kernels support d_c=512, d_r=64, d_n=d_v=128 and heads %% 128 == 0 "
                    "(got d_c=%lld d_r=%lld d_n=%lld d_v=%lld heads=%lld)",
                    (long long)p->d_c, (long long)p->d_r, (long long)p->d_n, (long long)p->d_v,
                    (long long)p->heads);
    if (p->ckv_stride_n < p->d_c || (p->d_r > 0 && p->kpe_stride_n < p->d_r))
        return fail(MLA_ERR_INVALID_ARG, "cache row stride smaller than the row width");
    if (p->ckv_stride_b < 0 || p->kpe_stride_b < 0)
        return fail(MLA_ERR_INVALID_ARG, "negative cache stride");
    if (!cache_span_ok(p->batch, p->n_max, p->ckv_stride_b, p->ckv_stride_n, 4) ||
        !cache_span_ok(p->batch, p->n_max, p->kpe_stride_b, p->kpe_stride_n, 4))
        return fail(MLA_ERR_UNSUPPORTED, "cache strides span beyond the addressable range");
    if (p->dtype == MLA_BF16 && (p->n_max * p->ckv_stride_n * 2 >= ((int64_t)1 << 32) ||
                                 p->n_max * p->kpe_stride_n * 2 >= ((int64_t)1 << 32)))
        return fail(MLA_ERR_UNSUPPORTED, "bf16 decode addresses one sequence's cache with 32-bit offsets");
    if (p->batch > 1 && (p->ckv_stride_b < p->n_max * p->ckv_stride_n ||
                         (p->d_r > 0 && p->kpe_stride_b < p->n_max * p->kpe_stride_n)))
        return fail(MLA_ERR_INVALID_ARG, "cache sequence stride smaller than n_max rows");
    if (p->num_splits < 0 || p->num_splits > mla::kMaxSplits)
        return fail(MLA_ERR_INVALID_ARG, "num_splits must be in [0, %d]", mla::kMaxSplits);
    if (!(p->softmax_scale >= 0.f) || isinf(p->softmax_scale))
        return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
    return check_rope_base(p->q_rope_base, p->d_r);
}

mla::DecodeShape make_shape(const mla_decode_params *p)
{
    mla::DecodeShape s;
    s.B = (int)p->batch;
    s.T = 1;
    s.H = (int)p->heads;
    s.dc = (int)p->d_c;
    s.dr = (int)p->d_r;
    s.dn = (int)p->d_n;
    s.dv = (int)p->d_v;
    s.n_max = p->n_max;
    s.ckv_sb = p->ckv_stride_b;
    s.ckv_sn = p->ckv_stride_n;
    s.kpe_sb = p->kpe_stride_b;
    s.kpe_sn = p->kpe_stride_n;
    s.scale = p->softmax_scale > 0.f ? p->softmax_scale
                                     : (float)(1.0 / sqrt((double)(p->d_n + p->d_r)));
    if (p->dtype == MLA_BF16) {
        set_plan(&s, p->batch, 1, p->num_splits);
    } else {
        s.S = p->num_splits > 0 ? p->num_splits : auto_splits(p->batch, p->heads, p->n_max);
        s.items = s.B * s.S;
    }
    s.out_bf16 = p->out_dtype == MLA_BF16;
    s.q_rope_base = p->q_rope_base;
    return s;
}

mla_status check_seqlens_debug(const int32_t *seqlens, int64_t B, int64_t n_max, hipStream_t st,
                               int64_t min_len)
{
    std::vector<int32_t> h((size_t)B);
    if (hipMemcpyAsync(h.data(), seqlens, sizeof(int32_t) * (size_t)B, hipMemcpyDeviceToHost, st) !=
            hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return fail(MLA_ERR_HIP, "MLA_DEBUG_CHECKS: could not read seqlens");
    for (int64_t b = 0; b < B; ++b)
        if (h[(size_t)b] < min_len || h[(size_t)b] > n_max)
            return fail(MLA_ERR_INVALID_ARG, "MLA_DEBUG_CHECKS: seqlens[%lld]=%d outside [%lld, %lld]",
                        (long long)b, h[(size_t)b], (long long)min_len, (long long)n_max);
    return MLA_OK;
}

}  // namespace

namespace mla {

size_t decode_workspace_layout(const DecodeShape &s, bool bf16, DecodeWorkspace *ws, void *base)
{
    const size_t qrows = (size_t)s.B * (size_t)s.T;  // query rows
    const size_t rows = qrows * (size_t)s.H;           // (query row, head) pairs
    const size_t qbytes = bf16 ? rows * (size_t)(s.dc + s.dr) * 2 : rows * (size_t)s.dc * 4;
    // partial (O, m, l) per (query row, split, head), or per (item, head)
    const size_t units = bf16 ? (size_t)s.items * (size_t)s.H : rows * (size_t)s.S;
    const size_t obytes = units * (size_t)s.dc * 4;
    const size_t mlbytes = units * 2 * 4;
    const size_t ibytes = bf16 ? (size_t)s.items * 4 * sizeof(int) : 0;
    const size_t vbytes = bf16 ? qrows * 2 * sizeof(int) : 0;
    // the fp32 path rotates q_rope into its own buffer; the bf16 absorb kernel
    // rotates while it copies q_rope beside q~
    const size_t rbytes = (s.q_rope_base > 0.0 && !bf16) ? rows * (size_t)s.dr * 4 : 0;
    const size_t lbytes = batched_upproj(s, bf16) ? rows * (size_t)s.dc * 4 : 0;
    const size_t off_o = round_up(qbytes, kAlign);
    const size_t off_ml = off_o + round_up(obytes, kAlign);
    const size_t off_r = off_ml + round_up(mlbytes, kAlign);
    const size_t off_l = off_r + round_up(rbytes, kAlign);
    const size_t off_i = off_l + round_up(lbytes, kAlign);
    const size_t off_v = off_i + round_up(ibytes, kAlign);
    const size_t total = off_v + round_up(vbytes, kAlign);
    if (ws) {
        char *b = static_cast<char *>(base);
        ws->q = b;
        ws->part_o = reinterpret_cast<float *>(b + off_o);
        ws->part_ml = reinterpret_cast<float *>(b + off_ml);
        ws->q_rope = rbytes ? b + off_r : nullptr;
        ws->o_lat = lbytes ? reinterpret_cast<float *>(b + off_l) : nullptr;
        ws->plan_items = ibytes ? reinterpret_cast<int *>(b + off_i) : nullptr;
        ws->plan_rows = vbytes ? reinterpret_cast<int *>(b + off_v) : nullptr;
    }
    return total;
}

}  // namespace mla

extern "C" {

int mla_decode_num_splits(const mla_decode_params *p)
{
    if (check_decode_params(p) != MLA_OK) return 0;
    if (p->dtype == MLA_BF16 && p->num_splits == 0)
        return plan_splits_full(p->batch, 1, p->heads, p->n_max);
    return make_shape(p).S;
}

size_t mla_decode_workspace_bytes(const mla_decode_params *p)
{
    if (check_decode_params(p) != MLA_OK) return 0;
    mla::DecodeShape s = make_shape(p);
    return mla::decode_workspace_layout(s, p->dtype == MLA_BF16, nullptr, nullptr);
}

mla_status mla_absorb_q(const mla_decode_params *p, const void *q_nope, const void *w_uk,
                        float *q_abs, void *stream)
{
    if (!p) return fail(MLA_ERR_INVALID_ARG, "params is NULL");
    if (p->batch < 1 || p->heads < 1 || p->d_c < 1 || p->d_n < 1)
        return fail(MLA_ERR_INVALID_ARG, "non-positive size");
    if (p->batch > 65535 || p->heads > 65535 || p->d_c > 1 << 20 || p->d_n > 512)
        return fail(MLA_ERR_UNSUPPORTED, "absorb supports d_n <= 512 and batch, heads <= 65535");
    if (p->dtype != MLA_F32 && p->dtype != MLA_BF16)
        return fail(MLA_ERR_UNSUPPORTED, "unknown dtype %d", p->dtype);
    if (!q_nope || !w_uk || !q_abs) return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
    hipError_t e = mla::launch_absorb_f32((int)p->batch, (int)p->heads, (int)p->d_n, (int)p->d_c,
                                          p->dtype == MLA_BF16, q_nope, w_uk, q_abs,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "absorb launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

namespace {

// Pointer and alignment checks of a decode call (after check_decode_params).
mla_status check_decode_tensors(const mla_decode_params *p, const void *q_nope,
                                const void *q_rope, const void *w_uk, const void *w_uv,
                                const void *ckv_cache, const void *kpe_cache,
                                const int32_t *seqlens, const void *out)
{
    if (!q_nope || !w_uk || !w_uv || !ckv_cache || !seqlens || !out)
        return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (p->d_r > 0 && (!q_rope || !kpe_cache))
        return fail(MLA_ERR_INVALID_ARG, "NULL q_rope or kpe_cache with d_r > 0");
    if (p->dtype == MLA_BF16) {
        if (!aligned(ckv_cache, 16) || !aligned(kpe_cache, 16) || p->ckv_stride_n % 8 ||
            p->kpe_stride_n % 8 || p->ckv_stride_b % 8 || p->kpe_stride_b % 8)
            return fail(MLA_ERR_INVALID_ARG,
                        "bf16 caches need 16-byte aligned rows (pointers %% 16, strides %% 8 elements)");
        if (!aligned(q_nope, 16) || !aligned(q_rope, 16) || !aligned(w_uk, 16) ||
            !aligned(w_uv, 16) || !aligned(out, 16))
            return fail(MLA_ERR_INVALID_ARG, "bf16 path needs 16-byte aligned q, weights and out");
    } else {
        if (!aligned(q_nope, 4) || (q_rope && !aligned(q_rope, 4)) || !aligned(w_uk, 4) ||
            !aligned(w_uv, 4) || !aligned(ckv_cache, 4) || (kpe_cache && !aligned(kpe_cache, 4)) ||
            !aligned(out, 4))
            return fail(MLA_ERR_INVALID_ARG, "fp32 tensors must be 4-byte aligned");
    }
    return MLA_OK;
}

// The launches of a checked decode call on workspace `ws` (laid out for s).
mla_status launch_decode(const mla_decode_params *p, const mla::DecodeShape &s,
                         const mla::DecodeWorkspace &ws, const void *q_nope, const void *q_rope,
                         const void *w_uk, const void *w_uv, const void *ckv_cache,
                         const void *kpe_cache, const int32_t *seqlens, void *out,
                         hipStream_t hs, hipEvent_t const *ev)
{
    if (debug_checks()) {
        mla_status st = check_seqlens_debug(seqlens, p->batch, p->n_max, hs, 1);
        if (st != MLA_OK) return st;
    }
    hipError_t e;
    if (p->dtype == MLA_BF16)
        e = mla::launch_decode_bf16(s, q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens,
                                    out, ws, hs, ev);
    else
        e = mla::launch_decode_f32(s, static_cast<const float *>(q_nope),
                                   static_cast<const float *>(q_rope), static_cast<const float *>(w_uk),
                                   static_cast<const float *>(w_uv), static_cast<const float *>(ckv_cache),
                                   static_cast<const float *>(kpe_cache), seqlens, out, ws, hs, ev);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
    return ok();
}

// ---------------------------------------------------------------------------
// Decode without a caller workspace: the workspace lives in `scratch`, a
// device array of fixed size that every GPU the library runs on holds once
// (it is part of the library's code object).  In host code the array's name
// is only a stand-in: its device address on the current GPU is looked up
// once per device with hipGetSymbolAddress and kept in scratch_addr[].
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = MLA_DECODE_NOALLOC_MAX_BYTES;
static_assert(kScratchBytes % kAlign == 0, "scratch size is a multiple of the region alignment");
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void *> scratch_addr[kMaxDevices];
std::mutex scratch_mu;

mla_status scratch_on_current_device(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MLA_ERR_UNSUPPORTED, "device %d beyond the %d devices the scratch table holds",
                    dev, kMaxDevices);
    void *ptr = scratch_addr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(scratch_mu);
        ptr = scratch_addr[dev].load(std::memory_order_relaxed);
        if (!ptr) {
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !ptr)
                return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                            hipGetErrorString(e));
            scratch_addr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_decode_profiled(const mla_decode_params *p, const void *q_nope,
                               const void *q_rope, const void *w_uk, const void *w_uv,
                               const void *ckv_cache, const void *kpe_cache,
                               const int32_t *seqlens, void *out, void *workspace,
                               size_t workspace_bytes, void *stream, void *const *events)
{
    mla_status st = check_decode_params(p);
    if (st != MLA_OK) return st;
    st = check_decode_tensors(p, q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens, out);
    if (st != MLA_OK) return st;
    mla::DecodeShape s = make_shape(p);
    mla::DecodeWorkspace ws;
    const size_t need = mla::decode_workspace_layout(s, p->dtype == MLA_BF16, &ws, workspace);
    if (!workspace || workspace_bytes < need || !aligned(workspace, kAlign))
        return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes at 256-byte alignment (got %zu at %p)",
                    need, workspace_bytes, workspace);
    return launch_decode(p, s, ws, q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens, out,
                         static_cast<hipStream_t>(stream),
                         reinterpret_cast<hipEvent_t const *>(events));
}

mla_status mla_decode_noalloc(const mla_decode_params *p, const void *q_nope, const void *q_rope,
                              const void *w_uk, const void *w_uv, const void *ckv_cache,
                              const void *kpe_cache, const int32_t *seqlens, void *out,
                              void *stream)
{
    mla_status st = check_decode_params(p);
    if (st != MLA_OK) return st;
    st = check_decode_tensors(p, q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens, out);
    if (st != MLA_OK) return st;
    mla::DecodeShape s = make_shape(p);
    const size_t need = mla::decode_workspace_layout(s, p->dtype == MLA_BF16, nullptr, nullptr);
    if (need > kScratchBytes)
        return fail(MLA_ERR_WORKSPACE,
                    "mla_decode_noalloc: this call needs %zu bytes of scratch, beyond the library's "
                    "fixed %zu (fewer sequences or splits fit; mla_decode takes a caller workspace)",
                    need, kScratchBytes);
    void *base = nullptr;
    st = scratch_on_current_device(&base);
    if (st != MLA_OK) return st;
    mla::DecodeWorkspace ws;
    mla::decode_workspace_layout(s, p->dtype == MLA_BF16, &ws, base);
    return launch_decode(p, s, ws, q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens, out,
                         static_cast<hipStream_t>(stream), nullptr);
}

mla_status mla_decode_latent(const mla_decode_params *p, const void *q_nope, const void *q_rope,
                             const void *w_uk, const void *ckv_cache, const void *kpe_cache,
                             const int32_t *seqlens, void *o_lat, void *workspace,
                             size_t workspace_bytes, void *stream)
{
    if (!p) return fail(MLA_ERR_INVALID_ARG, "params is NULL");
    mla_decode_params q = *p;  // d_v plays no part: check with the implemented value
    q.d_v = p->dtype == MLA_BF16 ? 128 : 1;
    p = &q;
    mla_status st = check_decode_params(p);
    if (st != MLA_OK) return st;
    if (!q_nope || !w_uk || !ckv_cache || !seqlens || !o_lat)
        return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (p->d_r > 0 && (!q_rope || !kpe_cache))
        return fail(MLA_ERR_INVALID_ARG, "NULL q_rope or kpe_cache with d_r > 0");
    const bool bf16 = p->dtype == MLA_BF16;
    if (bf16) {
        if (!aligned(ckv_cache, 16) || !aligned(kpe_cache, 16) || p->ckv_stride_n % 8 ||
            p->kpe_stride_n % 8 || p->ckv_stride_b % 8 || p->kpe_stride_b % 8)
            return fail(MLA_ERR_INVALID_ARG,
                        "bf16 caches need 16-byte aligned rows (pointers %% 16, strides %% 8 elements)");
        if (!aligned(q_nope, 16) || !aligned(q_rope, 16) || !aligned(w_uk, 16) || !aligned(o_lat, 16))
            return fail(MLA_ERR_INVALID_ARG, "bf16 path needs 16-byte aligned q, weights and output");
    } else {
        if (!aligned(q_nope, 4) || (q_rope && !aligned(q_rope, 4)) || !aligned(w_uk, 4) ||
            !aligned(ckv_cache, 4) || (kpe_cache && !aligned(kpe_cache, 4)) || !aligned(o_lat, 4))
            return fail(MLA_ERR_INVALID_ARG, "fp32 tensors must be 4-byte aligned");
    }
    mla::DecodeShape s = make_shape(p);
    mla::DecodeWorkspace ws;
    const size_t need = mla::decode_workspace_layout(s, bf16, &ws, workspace);
    if (!workspace || workspace_bytes < need || !aligned(workspace, kAlign))
        return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes at 256-byte alignment (got %zu at %p)",
                    need, workspace_bytes, workspace);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (debug_checks()) {
        st = check_seqlens_debug(seqlens, p->batch, p->n_max, hs, 1);
        if (st != MLA_OK) return st;
    }
    hipError_t e;
    if (bf16)
        e = mla::launch_decode_bf16(s, q_nope, q_rope, w_uk, nullptr, ckv_cache, kpe_cache, seqlens,
                                    o_lat, ws, hs, nullptr);
    else
        e = mla::launch_decode_f32(s, static_cast<const float *>(q_nope),
                                   static_cast<const float *>(q_rope), static_cast<const float *>(w_uk),
                                   nullptr, static_cast<const float *>(ckv_cache),
                                   static_cast<const float *>(kpe_cache), seqlens, o_lat, ws, hs, nullptr);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
    return ok();
}

mla_status mla_decode(const mla_decode_params *p, const void *q_nope, const void *q_rope,
                      const void *w_uk, const void *w_uv, const void *ckv_cache,
                      const void *kpe_cache, const int32_t *seqlens, void *out, void *workspace,
                      size_t workspace_bytes, void *stream)
{
    return mla_decode_profiled(p, q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens, out,
                               workspace, workspace_bytes, stream, nullptr);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// prefill
// ---------------------------------------------------------------------------
namespace {

mla_status check_prefill_params(const mla_prefill_params *p)
{
    if (!p) return fail(MLA_ERR_INVALID_ARG, "params is NULL");
    if (p->batch < 1 || p->tokens < 1 || p->heads < 1 || p->n_max < 1 || p->d_c < 1 ||
        p->d_n < 1 || p->d_v < 1 || p->d_r < 0)
        return fail(MLA_ERR_INVALID_ARG, "non-positive size");
    if (p->tokens > p->n_max) return fail(MLA_ERR_INVALID_ARG, "tokens exceeds n_max");
    if (p->batch > 65535 || p->heads > 65535 || p->tokens > (1 << 24) || p->n_max > (1 << 24))
        return fail(MLA_ERR_UNSUPPORTED, "sizes beyond the supported range");
    if ((p->dtype != MLA_F32 && p->dtype != MLA_BF16) ||
        (p->out_dtype != MLA_F32 && p->out_dtype != MLA_BF16))
        return fail(MLA_ERR_UNSUPPORTED, "unknown dtype");
    if (p->dtype == MLA_F32 && !f32_dims_ok(p->d_c, p->d_r, p->d_n, p->d_v))
        return fail(MLA_ERR_UNSUPPORTED, "fp32 kernels support d_c<=1024, d_r<=256, d_n<=512, d_v<=1024");
    if (p->dtype == MLA_BF16 && !(p->d_c == 512 && p->d_r == 64 && p->d_n == 128 && p->d_v == 128))
        return fail(MLA_ERR_UNSUPPORTED, "bf16 prefill supports d_c=512, d_r=64, d_n=d_v=128");
    if (p->ckv_stride_n < p->d_c || (p->d_r > 0 && p->kpe_stride_n < p->d_r))
        return fail(MLA_ERR_INVALID_ARG, "cache row stride smaller than the row width");
    if (p->ckv_stride_b < 0 || p->kpe_stride_b < 0)
        return fail(MLA_ERR_INVALID_ARG, "negative cache stride");
    if (!cache_span_ok(p->batch, p->n_max + 256, p->ckv_stride_b, p->ckv_stride_n, 4) ||
        !cache_span_ok(p->batch, p->n_max, p->kpe_stride_b, p->kpe_stride_n, 4))
        return fail(MLA_ERR_UNSUPPORTED, "cache strides span beyond the addressable range");
    if (p->dtype == MLA_BF16 &&
        ((uint64_t)(p->n_max + 256) * (uint64_t)p->ckv_stride_n * 2 >= (1ull << 32) ||
         (uint64_t)p->n_max * (uint64_t)p->kpe_stride_n * 2 >= (1ull << 32)))
        return fail(MLA_ERR_UNSUPPORTED, "bf16 prefill: one sequence's cache rows must span < 4 GiB");
    if (p->batch > 1 && (p->ckv_stride_b < p->n_max * p->ckv_stride_n ||
                         (p->d_r > 0 && p->kpe_stride_b < p->n_max * p->kpe_stride_n)))
        return fail(MLA_ERR_INVALID_ARG, "cache sequence stride smaller than n_max rows");
    if (!(p->softmax_scale >= 0.f) || isinf(p->softmax_scale))
        return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
    return check_rope_base(p->q_rope_base, p->d_r);
}

mla_status check_prefill_naive_params(const mla_prefill_params *p)
{
    mla_status st = check_prefill_params(p);
    if (st != MLA_OK) return st;
    if (p->num_splits != 0) return fail(MLA_ERR_INVALID_ARG, "num_splits must be 0 for the naive prefill");
    return MLA_OK;
}

// The absorbed prefill runs the decode kernels over batch * tokens query
// rows, so it takes the decode limits on top of the common prefill checks.
mla_status check_prefill_absorbed_params(const mla_prefill_params *p)
{
    mla_status st = check_prefill_params(p);
    if (st != MLA_OK) return st;
    if (p->batch * p->tokens > 65535)
        return fail(MLA_ERR_UNSUPPORTED, "absorbed prefill supports batch * tokens <= 65535");
    if (p->dtype == MLA_BF16 && !bf16_dims_ok(p->heads, p->d_c, p->d_r, p->d_n, p->d_v))
        return fail(MLA_ERR_UNSUPPORTED,
                    "bf16 absorbed prefill supports d_c=512, d_r=64, d_n=d_v=128 and heads %% 128 == 0");
    if (p->dtype == MLA_BF16 && (p->n_max * p->ckv_stride_n * 2 >= ((int64_t)1 << 32) ||
                                 p->n_max * p->kpe_stride_n * 2 >= ((int64_t)1 << 32)))
        return fail(MLA_ERR_UNSUPPORTED, "bf16 absorbed prefill addresses one sequence's cache with 32-bit offsets");
    if (p->num_splits < 0 || p->num_splits > mla::kMaxSplits)
        return fail(MLA_ERR_INVALID_ARG, "num_splits must be in [0, %d]", mla::kMaxSplits);
    return MLA_OK;
}

// Decode shape of an absorbed prefill: T query rows per sequence.
mla::DecodeShape make_absorbed_shape(const mla_prefill_params *p)
{
    mla::DecodeShape s;
    s.B = (int)p->batch;
    s.T = (int)p->tokens;
    s.H = (int)p->heads;
    s.dc = (int)p->d_c;
    s.dr = (int)p->d_r;
    s.dn = (int)p->d_n;
    s.dv = (int)p->d_v;
    s.n_max = p->n_max;
    s.ckv_sb = p->ckv_stride_b;
    s.ckv_sn = p->ckv_stride_n;
    s.kpe_sb = p->kpe_stride_b;
    s.kpe_sn = p->kpe_stride_n;
    s.scale = p->softmax_scale > 0.f ? p->softmax_scale
                                     : (float)(1.0 / sqrt((double)(p->d_n + p->d_r)));
    if (p->dtype == MLA_BF16) {
        set_plan(&s, p->batch, p->tokens, p->num_splits);
    } else {
        s.S = p->num_splits > 0 ? p->num_splits
                                : auto_splits(p->batch * p->tokens, p->heads, p->n_max);
        s.items = s.B * s.T * s.S;
    }
    s.out_bf16 = p->out_dtype == MLA_BF16;
    s.q_rope_base = p->q_rope_base;
    return s;
}

mla::PrefillShape make_pshape(const mla_prefill_params *p)
{
    mla::PrefillShape s;
    s.B = (int)p->batch;
    s.T = (int)p->tokens;
    s.H = (int)p->heads;
    s.dc = (int)p->d_c;
    s.dr = (int)p->d_r;
    s.dn = (int)p->d_n;
    s.dv = (int)p->d_v;
    s.n_max = p->n_max;
    s.ckv_sb = p->ckv_stride_b;
    s.ckv_sn = p->ckv_stride_n;
    s.kpe_sb = p->kpe_stride_b;
    s.kpe_sn = p->kpe_stride_n;
    s.scale = p->softmax_scale > 0.f ? p->softmax_scale
                                     : (float)(1.0 / sqrt((double)(p->d_n + p->d_r)));
    s.out_bf16 = p->out_dtype == MLA_BF16;
    s.q_rope_base = p->q_rope_base;
    return s;
}

}  // namespace

namespace mla {

size_t prefill_workspace_layout(const PrefillShape &s, bool bf16, void *base, void **k_out,
                                void **v_out, void **qr_out)
{
    const size_t elt = bf16 ? 2 : 4;
    const size_t rows = (size_t)s.B * (size_t)s.n_max * (size_t)s.H;
    const size_t kb = round_up(rows * (size_t)s.dn * elt, kAlign);
    const size_t vb = round_up(rows * (size_t)s.dv * elt, kAlign);
    const size_t rb = s.q_rope_base > 0.0
                          ? round_up((size_t)s.B * (size_t)s.T * (size_t)s.H * (size_t)s.dr * elt, kAlign)
                          : 0;
    if (k_out) *k_out = base;
    if (v_out) *v_out = static_cast<char *>(base) + kb;
    if (qr_out) *qr_out = rb ? static_cast<char *>(base) + kb + vb : nullptr;
    return kb + vb + rb;
}

}  // namespace mla

extern "C" {

size_t mla_prefill_workspace_bytes(const mla_prefill_params *p)
{
    if (check_prefill_naive_params(p) != MLA_OK) return 0;
    mla::PrefillShape s = make_pshape(p);
    return mla::prefill_workspace_layout(s, p->dtype == MLA_BF16, nullptr, nullptr, nullptr,
                                         nullptr);
}

mla_status mla_prefill_naive(const mla_prefill_params *p, const void *q_nope, const void *q_rope,
                             const void *w_uk, const void *w_uv, const void *ckv_cache,
                             const void *kpe_cache, const int32_t *seqlens, void *out,
                             void *workspace, size_t workspace_bytes, void *stream)
{
    mla_status st = check_prefill_naive_params(p);
    if (st != MLA_OK) return st;
    if (!q_nope || !w_uk || !w_uv || !ckv_cache || !seqlens || !out)
        return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (p->d_r > 0 && (!q_rope || !kpe_cache))
        return fail(MLA_ERR_INVALID_ARG, "NULL q_rope or kpe_cache with d_r > 0");
    const bool bf16 = p->dtype == MLA_BF16;
    const size_t a = bf16 ? 16 : 4;
    if (!aligned(q_nope, a) || !aligned(q_rope, a) || !aligned(w_uk, a) || !aligned(w_uv, a) ||
        !aligned(ckv_cache, a) || !aligned(kpe_cache, a) || !aligned(out, a))
        return fail(MLA_ERR_INVALID_ARG, "tensors must be %zu-byte aligned", a);
    if (bf16 && (p->ckv_stride_n % 8 || p->kpe_stride_n % 8 || p->ckv_stride_b % 8 ||
                 p->kpe_stride_b % 8))
        return fail(MLA_ERR_INVALID_ARG, "bf16 cache strides must be multiples of 8 elements");
    mla::PrefillShape s = make_pshape(p);
    void *kbuf = nullptr, *vbuf = nullptr, *qrbuf = nullptr;
    const size_t need = mla::prefill_workspace_layout(s, bf16, workspace, &kbuf, &vbuf, &qrbuf);
    if (!workspace || workspace_bytes < need || !aligned(workspace, kAlign))
        return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes at 256-byte alignment (got %zu)",
                    need, workspace_bytes);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (debug_checks()) {
        st = check_seqlens_debug(seqlens, p->batch, p->n_max, hs, p->tokens);
        if (st != MLA_OK) return st;
    }
    hipError_t e;
    if (qrbuf && p->d_r > 0) {  // rotate the queries' RoPE channels at their positions first
        e = mla::launch_rope_q(s.B, s.T, s.H, s.dr, s.n_max, s.q_rope_base, bf16, seqlens, q_rope,
                               qrbuf, hs);
        if (e != hipSuccess) return fail(MLA_ERR_HIP, "rope launch failed: %s", hipGetErrorString(e));
        q_rope = qrbuf;
    }
    if (bf16)
        e = mla::launch_prefill_bf16(s, q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens,
                                     out, kbuf, vbuf, hs);
    else
        e = mla::launch_prefill_f32(s, static_cast<const float *>(q_nope),
                                    static_cast<const float *>(q_rope), static_cast<const float *>(w_uk),
                                    static_cast<const float *>(w_uv), static_cast<const float *>(ckv_cache),
                                    static_cast<const float *>(kpe_cache), seqlens, out, kbuf, vbuf, hs);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
    return ok();
}

int mla_prefill_absorbed_num_splits(const mla_prefill_params *p)
{
    if (check_prefill_absorbed_params(p) != MLA_OK) return 0;
    if (p->dtype == MLA_BF16 && p->num_splits == 0)
        return plan_splits_full(p->batch, p->tokens, p->heads, p->n_max);
    return make_absorbed_shape(p).S;
}

size_t mla_prefill_absorbed_workspace_bytes(const mla_prefill_params *p)
{
    if (check_prefill_absorbed_params(p) != MLA_OK) return 0;
    return mla::decode_workspace_layout(make_absorbed_shape(p), p->dtype == MLA_BF16, nullptr,
                                        nullptr);
}

mla_status mla_prefill_absorbed(const mla_prefill_params *p, const void *q_nope,
                                const void *q_rope, const void *w_uk, const void *w_uv,
                                const void *ckv_cache, const void *kpe_cache,
                                const int32_t *seqlens, void *out, void *workspace,
                                size_t workspace_bytes, void *stream)
{
    mla_status st = check_prefill_absorbed_params(p);
    if (st != MLA_OK) return st;
    if (!q_nope || !w_uk || !w_uv || !ckv_cache || !seqlens || !out)
        return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (p->d_r > 0 && (!q_rope || !kpe_cache))
        return fail(MLA_ERR_INVALID_ARG, "NULL q_rope or kpe_cache with d_r > 0");
    const bool bf16 = p->dtype == MLA_BF16;
    if (bf16) {
        if (!aligned(ckv_cache, 16) || !aligned(kpe_cache, 16) || p->ckv_stride_n % 8 ||
            p->kpe_stride_n % 8 || p->ckv_stride_b % 8 || p->kpe_stride_b % 8)
            return fail(MLA_ERR_INVALID_ARG,
                        "bf16 caches need 16-byte aligned rows (pointers %% 16, strides %% 8 elements)");
        if (!aligned(q_nope, 16) || !aligned(q_rope, 16) || !aligned(w_uk, 16) ||
            !aligned(w_uv, 16) || !aligned(out, 16))
            return fail(MLA_ERR_INVALID_ARG, "bf16 path needs 16-byte aligned q, weights and out");
    } else {
        if (!aligned(q_nope, 4) || (q_rope && !aligned(q_rope, 4)) || !aligned(w_uk, 4) ||
            !aligned(w_uv, 4) || !aligned(ckv_cache, 4) || (kpe_cache && !aligned(kpe_cache, 4)) ||
            !aligned(out, 4))
            return fail(MLA_ERR_INVALID_ARG, "fp32 tensors must be 4-byte aligned");
    }
    mla::DecodeShape s = make_absorbed_shape(p);
    mla::DecodeWorkspace ws;
    const size_t need = mla::decode_workspace_layout(s, bf16, &ws, workspace);
    if (!workspace || workspace_bytes < need || !aligned(workspace, kAlign))
        return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes at 256-byte alignment (got %zu at %p)",
                    need, workspace_bytes, workspace);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (debug_checks()) {
        st = check_seqlens_debug(seqlens, p->batch, p->n_max, hs, p->tokens);
        if (st != MLA_OK) return st;
    }
    hipError_t e;
    if (bf16)
        e = mla::launch_decode_bf16(s, q_nope, q_rope, w_uk, w_uv, ckv_cache, kpe_cache, seqlens,
                                    out, ws, hs, nullptr);
    else
        e = mla::launch_decode_f32(s, static_cast<const float *>(q_nope),
                                   static_cast<const float *>(q_rope), static_cast<const float *>(w_uk),
                                   static_cast<const float *>(w_uv), static_cast<const float *>(ckv_cache),
                                   static_cast<const float *>(kpe_cache), seqlens, out, ws, hs, nullptr);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "absorbed prefill launch failed: %s", hipGetErrorString(e));
    return ok();
}

mla_status mla_cache_append(const mla_append_params *p, const void *h, const void *w_dkv,
                            const void *w_kr, const int32_t *positions, void *ckv_cache,
                            void *kpe_cache, void *stream)
{
    if (!p) return fail(MLA_ERR_INVALID_ARG, "params is NULL");
    if (p->batch < 0 || p->d_model < 1 || p->d_c < 1 || p->d_r < 0 || p->n_max < 1)
        return fail(MLA_ERR_INVALID_ARG, "invalid size");
    if (p->reserved != 0) return fail(MLA_ERR_INVALID_ARG, "reserved field must be 0");
    if (p->dtype != MLA_BF16 && p->dtype != MLA_F32) return fail(MLA_ERR_UNSUPPORTED, "unknown dtype");
    const bool bf16 = p->dtype == MLA_BF16;
    const int64_t vec = bf16 ? 8 : 4;  // elements per 16-byte piece
    if ((p->d_c & 1) || (p->d_r & 1))
        return fail(MLA_ERR_UNSUPPORTED, "d_c and d_r must be even (rotation pairs)");
    if (p->d_model % vec)
        return fail(MLA_ERR_UNSUPPORTED, "d_model must be a multiple of %lld", (long long)vec);
    if (p->batch > (1 << 24) || p->d_model > (1 << 24) || p->d_c + p->d_r > (1 << 20) ||
        p->n_max > (1 << 30))
        return fail(MLA_ERR_UNSUPPORTED, "sizes beyond the supported range");
    if ((uint64_t)p->batch * (uint64_t)p->d_model * (bf16 ? 2u : 4u) >= (1ull << 32))
        return fail(MLA_ERR_UNSUPPORTED, "the hidden states must span < 4 GiB");
    if (p->ckv_stride_n < p->d_c || (p->d_r > 0 && p->kpe_stride_n < p->d_r) ||
        p->ckv_stride_b < 0 || p->kpe_stride_b < 0)
        return fail(MLA_ERR_INVALID_ARG, "cache strides smaller than the row width");
    if (p->batch > 0 && (!cache_span_ok(p->batch, p->n_max, p->ckv_stride_b, p->ckv_stride_n, 4) ||
                         !cache_span_ok(p->batch, p->n_max, p->kpe_stride_b, p->kpe_stride_n, 4)))
        return fail(MLA_ERR_UNSUPPORTED, "cache strides span beyond the addressable range");
    if (p->batch > 1 && (p->ckv_stride_b < p->n_max * p->ckv_stride_n ||
                         (p->d_r > 0 && p->kpe_stride_b < p->n_max * p->kpe_stride_n)))
        return fail(MLA_ERR_INVALID_ARG, "cache sequence stride smaller than n_max rows");
    if (!(p->rope_base >= 0.0) || isinf(p->rope_base) || (p->rope_base > 0.0 && p->rope_base <= 1.0))
        return fail(MLA_ERR_INVALID_ARG, "rope_base must be 0 (default) or a finite value > 1");
    if (p->batch == 0) return ok();
    if (!h || !w_dkv || !positions || !ckv_cache || (p->d_r > 0 && (!w_kr || !kpe_cache)))
        return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
    if (!aligned(h, 16) || !aligned(w_dkv, 16) || (w_kr && !aligned(w_kr, 16)) ||
        !aligned(ckv_cache, bf16 ? 2 : 4) || (kpe_cache && !aligned(kpe_cache, bf16 ? 2 : 4)))
        return fail(MLA_ERR_INVALID_ARG, "h and the weights must be 16-byte aligned");
    mla::AppendShape s;
    s.B = (int)p->batch;
    s.d_model = (int)p->d_model;
    s.dc = (int)p->d_c;
    s.dr = (int)p->d_r;
    s.n_max = p->n_max;
    s.ckv_sb = p->ckv_stride_b;
    s.ckv_sn = p->ckv_stride_n;
    s.kpe_sb = p->kpe_stride_b;
    s.kpe_sn = p->kpe_stride_n;
    s.rope_base = p->rope_base > 0.0 ? p->rope_base : 10000.0;
    s.bf16 = bf16;
    hipError_t e = mla::launch_cache_append(s, h, w_dkv, w_kr, positions, ckv_cache, kpe_cache,
                                            static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "append launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

namespace {

mla_status check_proj_params(const mla_proj_params *p)
{
    if (!p) return fail(MLA_ERR_INVALID_ARG, "params is NULL");
    if (p->batch < 1 || p->in_features < 1 || p->out_features < 1)
        return fail(MLA_ERR_INVALID_ARG, "non-positive size");
    if (p->reserved != 0) return fail(MLA_ERR_INVALID_ARG, "reserved field must be 0");
    if ((p->dtype != MLA_F32 && p->dtype != MLA_BF16) ||
        (p->out_dtype != MLA_F32 && p->out_dtype != MLA_BF16))
        return fail(MLA_ERR_UNSUPPORTED, "unknown dtype");
    if (p->batch > 65535 || p->in_features > (1 << 24) || p->out_features > (1 << 24) ||
        p->batch * p->out_features >= ((int64_t)1 << 31))
        return fail(MLA_ERR_UNSUPPORTED, "sizes beyond the supported range");
    if ((uint64_t)p->out_features * (uint64_t)p->in_features * (p->dtype == MLA_BF16 ? 2u : 4u) >=
        (1ull << 40))
        return fail(MLA_ERR_UNSUPPORTED, "weight beyond the supported size");
    if (p->dtype == MLA_BF16 && p->in_features % 64)
        return fail(MLA_ERR_UNSUPPORTED, "bf16 projection needs in_features %% 64 == 0");
    if (p->num_splits < 0 || p->num_splits > mla::kMaxSplits)
        return fail(MLA_ERR_INVALID_ARG, "num_splits must be in [0, %d]", mla::kMaxSplits);
    return MLA_OK;
}

mla::ProjShape make_proj_shape(const mla_proj_params *p)
{
    mla::ProjShape s;
    s.B = (int)p->batch;
    s.K = (int)p->in_features;
    s.N = (int)p->out_features;
    s.bf16 = p->dtype == MLA_BF16;
    s.out_bf16 = p->out_dtype == MLA_BF16;
    s.R = 0;
    // bf16 weights with at least 8 rows per CU, split count left to the
    // library: the direct form, one group of R <= 32 rows per workgroup over
    // all of K, the groups covering the 256 CUs of an MI355X once
    // (R = 28 for 7168 rows).
    if (s.bf16 && p->num_splits == 0 && p->out_features >= 8 * kProjDirectGroups) {
        s.S = 1;
        s.R = (int)std::min<int64_t>(32, (p->out_features + kProjDirectGroups - 1) / kProjDirectGroups);
        return s;
    }
    // Otherwise slices of about 1024 input features: enough workgroups to
    // stream the weight from every CU.
    int64_t S = p->num_splits > 0 ? p->num_splits : (p->in_features + 1023) / 1024;
    if (S < 1) S = 1;
    if (S > mla::kMaxSplits) S = mla::kMaxSplits;
    s.S = (int)S;
    return s;
}

size_t proj_workspace(const mla::ProjShape &s)
{
    if (s.R > 0) return 0;  // the direct form keeps its partial sums in LDS
    return round_up((size_t)s.S * (size_t)s.B * (size_t)s.N * 4, kAlign);
}

}  // namespace

extern "C" {

size_t mla_output_proj_workspace_bytes(const mla_proj_params *p)
{
    if (check_proj_params(p) != MLA_OK) return 0;
    return proj_workspace(make_proj_shape(p));
}

mla_status mla_output_proj(const mla_proj_params *p, const void *x, const void *w, void *y,
                           void *workspace, size_t workspace_bytes, void *stream)
{
    mla_status st = check_proj_params(p);
    if (st != MLA_OK) return st;
    if (!x || !w || !y) return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
    const bool bf16 = p->dtype == MLA_BF16;
    if (!aligned(x, bf16 ? 16 : 4) || !aligned(w, bf16 ? 16 : 4) ||
        !aligned(y, p->out_dtype == MLA_BF16 ? 2 : 4))
        return fail(MLA_ERR_INVALID_ARG, "x and w must be %d-byte aligned", bf16 ? 16 : 4);
    mla::ProjShape s = make_proj_shape(p);
    const size_t need = proj_workspace(s);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, kAlign)))
        return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes at 256-byte alignment (got %zu)",
                    need, workspace_bytes);
    hipError_t e = mla::launch_output_proj(s, x, w, y, static_cast<float *>(workspace),
                                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "projection launch failed: %s", hipGetErrorString(e));
    return ok();
}

mla_status mla_fold_value_output(int64_t d_model, int64_t heads, int64_t d_v, int64_t d_c,
                                 int32_t dtype, const void *w_o, const void *w_uv, void *w_ov,
                                 void *stream)
{
    if (d_model < 1 || heads < 1 || d_v < 1 || d_c < 1)
        return fail(MLA_ERR_INVALID_ARG, "non-positive size");
    if (dtype != MLA_F32 && dtype != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "unknown dtype");
    if (d_model > (1 << 24) || heads > 65535 || d_v > (1 << 20) || d_c > (1 << 20) ||
        (uint64_t)d_model * (uint64_t)heads * (uint64_t)(d_v > d_c ? d_v : d_c) >= (1ull << 40))
        return fail(MLA_ERR_UNSUPPORTED, "sizes beyond the supported range");
    if (!w_o || !w_uv || !w_ov) return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
    const size_t a = dtype == MLA_BF16 ? 2 : 4;
    if (!aligned(w_o, a) || !aligned(w_uv, a) || !aligned(w_ov, a))
        return fail(MLA_ERR_INVALID_ARG, "tensors must be %zu-byte aligned", a);
    hipError_t e = mla::launch_fold_value_output((int)d_model, (int)heads, (int)d_v, (int)d_c,
                                                 dtype == MLA_BF16, w_o, w_uv, w_ov,
                                                 static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "fold launch failed: %s", hipGetErrorString(e));
    return ok();
}

uint64_t mla_kv_cache_bytes(int64_t n_layers, int64_t batch, int64_t seq_len, int64_t d_c,
                            int64_t d_r, int64_t bytes_per_elem)
{
    if (n_layers < 0 || batch < 0 || seq_len < 0 || d_c < 0 || d_r < 0 || bytes_per_elem < 0)
        return 0;
    return (uint64_t)n_layers * (uint64_t)batch * (uint64_t)seq_len * (uint64_t)(d_c + d_r) *
           (uint64_t)bytes_per_elem;
}

const char *mla_status_string(mla_status s)
{
    switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: invalid argument";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: shape or dtype not implemented";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing, too small or misaligned";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime error";
    }
    return "unknown mla_status";
}

const char *mla_last_error(void) { return g_err; }

int mla_version(void) { return 10200; }

}  // extern "C"
