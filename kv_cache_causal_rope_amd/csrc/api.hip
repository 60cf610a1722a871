// api.hip -- the C ABI of libkvrope: host-side validation, rotary tables and dispatch.
//
// Every status except ATTN_ERR_HIP is decided here, on the host, before any HIP call.
// See include/kvrope.h for the contract of each entry point.
#include "../../include/kvrope.h"

#include "device_common.h"
#include "launch.h"

#include <math.h>

#include <atomic>
#include <mutex>

namespace {

// Device scratch of attn_decode_noalloc: the split-key partials, in a file-scope array
// every GPU the library runs on holds until the process ends.  Host code never uses the
// array's name as an address: it takes each device's own address once, through
// hipGetSymbolAddress, and passes that to the kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// The scratch address on the current device (set up on the first call there), or NULL
// with *err set.
void *device_scratch(hipError_t *err)
{
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess)
        return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess || !p) {
            if (*err == hipSuccess)
                *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

// the library's only state, per thread
thread_local int g_last_hip_error = 0;
thread_local hipEvent_t g_ev_before = nullptr;
thread_local hipEvent_t g_ev_after = nullptr;

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline bool finite_pos(double x) { return isfinite(x) && x > 0.0; }

// the frequency fields of one parameter set (base, YaRN fields, mscale)
int check_freqs(const kvrope_rope_params &r)
{
    if (!isfinite(r.base) || r.base <= 1.0)
        return ATTN_ERR_ROPE;
    if (!finite_pos(r.mscale))
        return ATTN_ERR_ROPE;
    if (r.yarn != 0 && r.yarn != 1)
        return ATTN_ERR_ROPE;
    if (r.yarn) {
        if (!finite_pos(r.freq_scale) || !isfinite(r.ext_factor) || r.ext_factor < 0.0 ||
            r.ext_factor > 1.0 || r.n_ctx_orig <= 0 || !finite_pos(r.beta_fast) ||
            !finite_pos(r.beta_slow))
            return ATTN_ERR_ROPE;
    }
    return ATTN_OK;
}

int check_rope(const kvrope_rope_params *rp, int d)
{
    if (!rp)
        return ATTN_ERR_NULL;
    if (rp->n_rot < 2 || rp->n_rot > d || (rp->n_rot & 1))
        return ATTN_ERR_ROPE;
    if ((rp->pairing != 0 && rp->pairing != 1) || (rp->inverse != 0 && rp->inverse != 1))
        return ATTN_ERR_ROPE;
    if (rp->pairing == 1 && rp->n_rot % 32 != 0)
        return ATTN_ERR_ROPE;
    if ((rp->cos_table == nullptr) != (rp->sin_table == nullptr))
        return ATTN_ERR_ROPE;
    if (rp->n_sets < 0 || rp->n_sets > KVROPE_MAX_ROPE_SETS)
        return ATTN_ERR_ROPE;
    if (rp->n_sets > 0) {
        if (rp->cos_table)
            return ATTN_ERR_ROPE; // sets and tables exclude each other
        if (!rp->sets || !rp->unit_set)
            return ATTN_ERR_NULL;
        if (!aligned4(rp->unit_set))
            return ATTN_ERR_ALIGN;
        for (int s = 0; s < rp->n_sets; ++s)
            if (int st = check_freqs(rp->sets[s]))
                return st;
        return ATTN_OK;
    }
    if (rp->cos_table) {
        if (rp->table_rows < 1)
            return ATTN_ERR_ROPE;
        if (!aligned4(rp->cos_table) || !aligned4(rp->sin_table))
            return ATTN_ERR_ALIGN;
        return ATTN_OK; // the computed-angle fields are not used
    }
    return check_freqs(*rp);
}

// Angle rates of one parameter set in fp64 ("ds4.c study notes", Part 4 sec. 1, Traces
// 1-2), in revolutions per position.  Pair j turns at base^(-2j / n_rot) radians per
// position; under YaRN that rate is blended with the interpolated rate freq_scale times
// it, the weight of the original rate being ext_factor times the ramp: the ramp is 1 for
// pairs below the correction dim of beta_fast, 0 above that of beta_slow and linear
// between (the width of the linear part kept at least 0.001), where the correction dim
// of beta is the pair index that turns beta full circles over n_ctx_orig positions,
// n_rot * ln(n_ctx_orig / (2 pi beta)) / (2 ln base).
void set_rates(const kvrope_rope_params &r, int n_rot, double (&wrev)[kvrope::kMaxPairs])
{
    const double two_pi = 6.283185307179586476925286766559;
    const int n_pairs = n_rot / 2;
    double fast = 0.0, slow = 0.0;
    if (r.yarn) {
        auto corr_dim = [&](double beta) {
            return (double)n_rot * log((double)r.n_ctx_orig / (two_pi * beta)) / (2.0 * log(r.base));
        };
        fast = corr_dim(r.beta_fast);
        slow = corr_dim(r.beta_slow);
    }
    const double ramp_width = fmax(0.001, slow - fast);
    for (int j = 0; j < kvrope::kMaxPairs; ++j) {
        double rate = 0.0;
        if (j < n_pairs) {
            rate = pow(r.base, -2.0 * (double)j / (double)n_rot);
            if (r.yarn) {
                const double t = fmin(fmax(((double)j - fast) / ramp_width, 0.0), 1.0);
                const double keep = r.ext_factor * (1.0 - t); // weight of the original rate
                rate = rate * (r.freq_scale * (1.0 - keep) + keep);
            }
        }
        wrev[j] = rate / two_pi;
    }
}

kvrope::RopeTable rope_table(const kvrope_rope_params &rp, int d)
{
    kvrope::RopeTable tab = {};
    tab.n_pairs = rp.n_rot / 2;
    tab.off = d - rp.n_rot;
    tab.half = rp.pairing;
    tab.sgn = rp.inverse ? -1.0 : 1.0;
    tab.cos_t = rp.cos_table;
    tab.sin_t = rp.sin_table;
    tab.rows = rp.cos_table ? rp.table_rows : 0;
    if (rp.n_sets > 0) {
        tab.nsets = rp.n_sets;
        tab.unit_set = rp.unit_set;
        for (int s = 0; s < rp.n_sets; ++s) {
            set_rates(rp.sets[s], rp.n_rot, tab.wrev[s]);
            tab.mscale[s] = rp.sets[s].mscale;
        }
    } else {
        tab.nsets = 1;
        tab.unit_set = nullptr;
        if (!rp.cos_table)
            set_rates(rp, rp.n_rot, tab.wrev[0]);
        tab.mscale[0] = rp.cos_table ? 1.0 : rp.mscale;
    }
    return tab;
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return ATTN_OK;
    g_last_hip_error = (int)e;
    return ATTN_ERR_HIP;
}

void take_profile_events(hipEvent_t *before, hipEvent_t *after)
{
    *before = g_ev_before;
    *after = g_ev_after;
    g_ev_before = nullptr;
    g_ev_after = nullptr;
}

constexpr int64_t kMaxGrid = 0x7fffffff;

} // namespace

extern "C" {

const char *attn_status_string(int status)
{
    switch (status) {
    case ATTN_OK:
        return "ok";
    case ATTN_ERR_NULL:
        return "a required pointer is NULL";
    case ATTN_ERR_SHAPE:
        return "invalid shape (negative size, d != 128, hq not a multiple of hkv, or grid too large)";
    case ATTN_ERR_ROPE:
        return "invalid rotary parameters (or parameter sets)";
    case ATTN_ERR_CAPACITY:
        return "cache capacity exceeded (max_len + t > s_cap) or negative max_len";
    case ATTN_ERR_ALIGN:
        return "a tensor pointer is not 16-byte aligned (int32 arrays: 4-byte)";
    case ATTN_ERR_WORKSPACE:
        return "workspace missing or smaller than attn_workspace_size()";
    case ATTN_ERR_SCALE:
        return "softmax scale is not finite and positive";
    case ATTN_ERR_HIP:
        return "a HIP launch failed";
    default:
        return "unknown status";
    }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

int attn_set_profile_events(void *before, void *after)
{
    g_ev_before = reinterpret_cast<hipEvent_t>(before);
    g_ev_after = reinterpret_cast<hipEvent_t>(after);
    return ATTN_OK;
}

size_t attn_workspace_size(int op, int n, int t, int hq, int hkv, int d, int max_len)
{
    (void)t;
    (void)d;
    if (op != ATTN_OP_DECODE || n <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || max_len < 0)
        return 0;
    return kvrope::decode_workspace_bytes(n, hq, hkv, max_len);
}

int attn_decode_chunk_keys(int n, int hq, int hkv, int max_len)
{
    if (n <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || max_len < 0)
        return 0;
    return kvrope::decode_chunk_keys(n, hq, hkv, max_len);
}

int attn_rope_apply(void *x, const int32_t *positions, int n, int t, int h, int d,
                    const kvrope_rope_params *rp, void *stream)
{
    if (n < 0 || t < 0 || h < 1 || d != kvrope::kHeadDim)
        return ATTN_ERR_SHAPE;
    int st = check_rope(rp, d);
    if (st)
        return st;
    const int64_t rows = (int64_t)n * t;
    if (rows == 0)
        return ATTN_OK;
    if (!x || !positions)
        return ATTN_ERR_NULL;
    if (!aligned16(x) || !aligned4(positions))
        return ATTN_ERR_ALIGN;
    if (rows * 16 / 256 > kMaxGrid)
        return ATTN_ERR_SHAPE;
    const kvrope::RopeTable tab = rope_table(*rp, d);
    return hip_status(kvrope::launch_rope_inplace(static_cast<uint16_t *>(x), positions, rows, t, h, tab,
                                                  static_cast<hipStream_t>(stream)));
}

int kv_cache_append(void *cache_k, void *cache_v, const void *k, const void *v,
                    const int32_t *lens, int max_len, int n, int t, int hkv, int d, int s_cap,
                    void *stream)
{
    if (n < 0 || t < 0 || hkv < 1 || d != kvrope::kHeadDim || s_cap < 1)
        return ATTN_ERR_SHAPE;
    if (max_len < 0 || (int64_t)max_len + t > s_cap)
        return ATTN_ERR_CAPACITY;
    if ((int64_t)n * t == 0)
        return ATTN_OK;
    if (!cache_k || !cache_v || !k || !v || !lens)
        return ATTN_ERR_NULL;
    if (!aligned16(cache_k) || !aligned16(cache_v) || !aligned16(k) || !aligned16(v) || !aligned4(lens))
        return ATTN_ERR_ALIGN;
    if ((int64_t)n * t * hkv * 16 / 256 > kMaxGrid)
        return ATTN_ERR_SHAPE;
    return hip_status(kvrope::launch_append(static_cast<uint16_t *>(cache_k), static_cast<uint16_t *>(cache_v),
                                            static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v),
                                            lens, max_len, n, t, hkv, s_cap, static_cast<hipStream_t>(stream)));
}

namespace {

// attn_prefill_kv and attn_prefill_kv_varlen (new_lens NULL: t new tokens per unit)
int prefill_kv_impl(const void *q, const void *k, const void *v, const int32_t *positions,
                    void *history_k, void *history_v, const int32_t *hist_lens, int max_hist,
                    const int32_t *new_lens, void *out, int n, int t, int hq, int hkv, int d, int s_cap,
                    double scale, const kvrope_rope_params *rp, void *stream)
{
    if (n < 0 || t < 0 || hq < 1 || hkv < 1 || hq % hkv != 0 || d != kvrope::kHeadDim || s_cap < 1)
        return ATTN_ERR_SHAPE;
    int st = check_rope(rp, d);
    if (st)
        return st;
    if (!(isfinite(scale) && scale > 0.0))
        return ATTN_ERR_SCALE;
    if (max_hist < 0 || (int64_t)max_hist + t > s_cap)
        return ATTN_ERR_CAPACITY;
    if ((int64_t)n * t == 0)
        return ATTN_OK;
    if (!q || !k || !v || !positions || !history_k || !history_v || !out)
        return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(history_k) ||
        !aligned16(history_v) || !aligned16(out) || !aligned4(positions) ||
        (hist_lens && !aligned4(hist_lens)) || (new_lens && !aligned4(new_lens)))
        return ATTN_ERR_ALIGN;
    const int G = hq / hkv;
    if ((int64_t)n * hkv * G * ((t + 31) / 32) > kMaxGrid || (int64_t)n * t * 16 / 256 > kMaxGrid)
        return ATTN_ERR_SHAPE;
    const kvrope::RopeTable tab = rope_table(*rp, d);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t eb, ea;
    take_profile_events(&eb, &ea);
    uint16_t *ck = static_cast<uint16_t *>(history_k);
    uint16_t *cv = static_cast<uint16_t *>(history_v);
    hipError_t e = kvrope::launch_rope_append(ck, cv, static_cast<const uint16_t *>(k),
                                              static_cast<const uint16_t *>(v), positions, hist_lens,
                                              new_lens, max_hist, n, t, hkv, s_cap, tab, s);
    if (e != hipSuccess)
        return hip_status(e);
    kvrope::PrefillShape ps{n, t, hq, hkv, s_cap, max_hist, (float)scale};
    return hip_status(kvrope::launch_prefill_attention(static_cast<const uint16_t *>(q), ck, cv, positions,
                                                       hist_lens, new_lens, static_cast<uint16_t *>(out), ps,
                                                       tab, s, eb, ea));
}

} // namespace

int attn_prefill_kv(const void *q, const void *k, const void *v, const int32_t *positions,
                    void *history_k, void *history_v, const int32_t *hist_lens, int max_hist,
                    void *out, int n, int t, int hq, int hkv, int d, int s_cap, double scale,
                    const kvrope_rope_params *rp, void *stream)
{
    return prefill_kv_impl(q, k, v, positions, history_k, history_v, hist_lens, max_hist, nullptr, out, n, t,
                           hq, hkv, d, s_cap, scale, rp, stream);
}

int attn_prefill_kv_varlen(const void *q, const void *k, const void *v, const int32_t *positions,
                           void *history_k, void *history_v, const int32_t *hist_lens, int max_hist,
                           const int32_t *new_lens, void *out, int n, int t, int hq, int hkv, int d,
                           int s_cap, double scale, const kvrope_rope_params *rp, void *stream)
{
    if (!new_lens && (int64_t)n * t > 0)
        return ATTN_ERR_NULL;
    return prefill_kv_impl(q, k, v, positions, history_k, history_v, hist_lens, max_hist, new_lens, out, n,
                           t, hq, hkv, d, s_cap, scale, rp, stream);
}

int attn_prefill(const void *q, const void *k, const void *v, const int32_t *positions,
                 void *cache_k, void *cache_v, void *out, int n, int t, int hq, int hkv, int d,
                 int s_cap, double scale, const kvrope_rope_params *rp, void *stream)
{
    return attn_prefill_kv(q, k, v, positions, cache_k, cache_v, nullptr, 0, out, n, t, hq, hkv, d,
                           s_cap, scale, rp, stream);
}

int attn_decode(const void *q, const void *k, const void *v, const int32_t *positions,
                void *cache_k, void *cache_v, const int32_t *cache_lens, int max_len,
                void *out, int n, int hq, int hkv, int d, int s_cap, double scale,
                const kvrope_rope_params *rp, void *workspace, size_t ws_bytes, void *stream)
{
    if (n < 0 || hq < 1 || hkv < 1 || hq % hkv != 0 || d != kvrope::kHeadDim || s_cap < 1)
        return ATTN_ERR_SHAPE;
    int st = check_rope(rp, d);
    if (st)
        return st;
    if (!(isfinite(scale) && scale > 0.0))
        return ATTN_ERR_SCALE;
    if (max_len < 0 || (int64_t)max_len + 1 > s_cap)
        return ATTN_ERR_CAPACITY;
    if (n == 0)
        return ATTN_OK;
    if (!q || !k || !v || !positions || !cache_k || !cache_v || !cache_lens || !out)
        return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(cache_k) || !aligned16(cache_v) ||
        !aligned16(out) || !aligned4(positions) || !aligned4(cache_lens))
        return ATTN_ERR_ALIGN;
    const size_t need = kvrope::decode_workspace_bytes(n, hq, hkv, max_len);
    if (need > 0 && (!workspace || ws_bytes < need))
        return ATTN_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace))
        return ATTN_ERR_ALIGN;
    const int64_t nsplit_max = (int64_t)max_len / 128 + 1;
    if ((int64_t)n * hq * nsplit_max > kMaxGrid || (int64_t)n * hq * 64 / 256 > kMaxGrid)
        return ATTN_ERR_SHAPE;
    const kvrope::RopeTable tab = rope_table(*rp, d);
    hipEvent_t eb, ea;
    take_profile_events(&eb, &ea);
    kvrope::DecodeShape ds{n, hq, hkv, s_cap, max_len, (float)scale};
    return hip_status(kvrope::launch_decode(static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                                            static_cast<const uint16_t *>(v), positions,
                                            static_cast<uint16_t *>(cache_k), static_cast<uint16_t *>(cache_v),
                                            cache_lens, static_cast<uint16_t *>(out), ds, tab, workspace,
                                            static_cast<hipStream_t>(stream), eb, ea));
}

int attn_decode_noalloc(const void *q, const void *k, const void *v, const int32_t *positions,
                        void *cache_k, void *cache_v, const int32_t *cache_lens, int max_len,
                        void *out, int n, int hq, int hkv, int d, int s_cap, double scale,
                        const kvrope_rope_params *rp, void *stream)
{
    // the size check needs valid shapes; every other check is attn_decode's
    if (n >= 0 && hq >= 1 && hkv >= 1 && hq % hkv == 0 && max_len >= 0 &&
        kvrope::decode_workspace_bytes(n, hq, hkv, max_len) > kScratchBytes)
        return ATTN_ERR_WORKSPACE;
    hipError_t e = hipSuccess;
    void *ws = nullptr;
    if (n > 0 && hq >= 1 && hkv >= 1 && hq % hkv == 0 && max_len >= 0) {
        ws = device_scratch(&e);
        if (!ws)
            return hip_status(e);
    }
    return attn_decode(q, k, v, positions, cache_k, cache_v, cache_lens, max_len, out, n, hq, hkv, d, s_cap,
                       scale, rp, ws, ws ? kScratchBytes : 0, stream);
}

size_t attn_decode_noalloc_max_workspace(void) { return kScratchBytes; }

int attn_prefill_kv_cached(const void *q, const int32_t *positions, const void *cache_k, const void *cache_v,
                           const int32_t *hist_lens, int max_hist, void *out, int n, int t, int hq, int hkv,
                           int d, int s_cap, double scale, const kvrope_rope_params *rp, void *stream)
{
    if (n < 0 || t < 0 || hq < 1 || hkv < 1 || hq % hkv != 0 || d != kvrope::kHeadDim || s_cap < 1)
        return ATTN_ERR_SHAPE;
    int st = check_rope(rp, d);
    if (st)
        return st;
    if (!(isfinite(scale) && scale > 0.0))
        return ATTN_ERR_SCALE;
    if (max_hist < 0 || (int64_t)max_hist + t > s_cap)
        return ATTN_ERR_CAPACITY;
    if ((int64_t)n * t == 0)
        return ATTN_OK;
    if (!q || !positions || !cache_k || !cache_v || !out)
        return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(cache_k) || !aligned16(cache_v) || !aligned16(out) || !aligned4(positions) ||
        (hist_lens && !aligned4(hist_lens)))
        return ATTN_ERR_ALIGN;
    if ((int64_t)n * hkv * (hq / hkv) * ((t + 31) / 32) > kMaxGrid)
        return ATTN_ERR_SHAPE;
    const kvrope::RopeTable tab = rope_table(*rp, d);
    hipEvent_t eb, ea;
    take_profile_events(&eb, &ea);
    kvrope::PrefillShape ps{n, t, hq, hkv, s_cap, max_hist, (float)scale};
    return hip_status(kvrope::launch_prefill_attention(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(cache_k),
        static_cast<const uint16_t *>(cache_v), positions, hist_lens, nullptr, static_cast<uint16_t *>(out), ps,
        tab, static_cast<hipStream_t>(stream), eb, ea));
}

int attn_qkv_project(const void *x, const void *w_qkv, int w_per_unit, const int32_t *positions, void *q,
                     void *cache_k, void *cache_v, const int32_t *lens, int max_len, int n, int t, int hidden,
                     int hq, int hkv, int d, int s_cap, const kvrope_rope_params *rp, void *stream)
{
    if (n < 0 || t < 0 || hq < 1 || hkv < 1 || hq % hkv != 0 || d != kvrope::kHeadDim || s_cap < 1 ||
        hidden < 64 || hidden % 64 != 0 || (w_per_unit != 0 && w_per_unit != 1))
        return ATTN_ERR_SHAPE;
    int st = check_rope(rp, d);
    if (st)
        return st;
    if (max_len < 0 || (int64_t)max_len + t > s_cap)
        return ATTN_ERR_CAPACITY;
    if ((int64_t)n * t == 0)
        return ATTN_OK;
    if (!x || !w_qkv || !positions || !q || !cache_k || !cache_v)
        return ATTN_ERR_NULL;
    if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(q) || !aligned16(cache_k) || !aligned16(cache_v) ||
        !aligned4(positions) || (lens && !aligned4(lens)))
        return ATTN_ERR_ALIGN;
    const int64_t nout = (int64_t)(hq + 2 * hkv) * d;
    if ((int64_t)n * ((t + 127) / 128) * (nout / 128) > kMaxGrid)
        return ATTN_ERR_SHAPE;
    const kvrope::RopeTable tab = rope_table(*rp, d);
    return hip_status(kvrope::launch_qkv_projection(
        static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w_qkv), w_per_unit ? nout * hidden : 0,
        positions, static_cast<uint16_t *>(q), static_cast<uint16_t *>(cache_k), static_cast<uint16_t *>(cache_v),
        lens, max_len, n, t, hidden, hq, hkv, s_cap, tab, static_cast<hipStream_t>(stream)));
}

int attn_out_project(const void *attn, const void *w_o, int w_per_unit, const void *residual, void *out, int n,
                     int t, int hq, int d, int hidden, void *stream)
{
    if (n < 0 || t < 0 || hq < 1 || d != kvrope::kHeadDim || hidden < 128 || hidden % 128 != 0 ||
        (w_per_unit != 0 && w_per_unit != 1))
        return ATTN_ERR_SHAPE;
    if ((int64_t)n * t == 0)
        return ATTN_OK;
    if (!attn || !w_o || !residual || !out)
        return ATTN_ERR_NULL;
    if (!aligned16(attn) || !aligned16(w_o) || !aligned16(residual) || !aligned16(out))
        return ATTN_ERR_ALIGN;
    const int in_features = hq * d;
    if ((int64_t)n * ((t + 127) / 128) * (hidden / 128) > kMaxGrid)
        return ATTN_ERR_SHAPE;
    return hip_status(kvrope::launch_out_projection(
        static_cast<const uint16_t *>(attn), static_cast<const uint16_t *>(w_o),
        w_per_unit ? (int64_t)hidden * in_features : 0, static_cast<const uint16_t *>(residual),
        static_cast<uint16_t *>(out), n, t, in_features, hidden, static_cast<hipStream_t>(stream)));
}

} // extern "C"
