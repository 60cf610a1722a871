/*
 * kvrope.h -- C ABI of the MI355X (gfx950) attention hot path: rotary embedding of
 * Q/K (plain RoPE or the YaRN-ramped tail rotation), KV-cache append, and causal
 * grouped-query attention in the three phases prefill, prefill_kv and decode.
 *
 * Sources (cited by page and section):
 *   [Sophgo] "An MLIR-based LLM compilation method" (Sophgo TPU-MLIR paper): sec. 2.2
 *            (top.Rope, top.Concat, top.FAttention = scaled dot product + causal mask),
 *            sec. 3.1 Listing 1 (block without history), Listing 2 (block with
 *            history_k / history_v and Concat(history, new)), sec. 4 and 4.1 (the
 *            prefill / prefill_kv / decode split).
 *   [ds4]    "ds4.c study notes", Part 4 sec. 1: Trace 1 (YaRN ramp, correction dims),
 *            Trace 2 (tail rotation of the last n_rot dims, theta schedule, matrix).
 *   [Buddy]  "Buddy-MLIR DeepSeek model import, compilation and inference scheduling"
 *            (juejin): sec. 6.4.3 (per-layer cache [B, kv_heads, max_len, head_dim] f16),
 *            sec. 6.4.5 (prompt rows copied into the decode cache, position = prompt
 *            length), sec. 6.4.6 (decode position grows by one per step), sec. 5.4.2
 *            and 9.2 (results returned through caller-provided memory).
 *   [CGDR]   "02 Prefill integration of CGDR" (MindSpore Qwen3.5 notes): sec. 1-2
 *            (KV heads shared by query-head groups via repeat_interleave; flat
 *            [tokens, heads, head_dim] f16 at the kernel boundary), sec. 6 (a
 *            hard-coded softmax scale as a silent-error hazard: here it is an argument).
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers.  f16 tensors are IEEE binary16 bit patterns
 *     (uint16_t storage), dense, row-major, innermost dimension last:
 *         q, out            [n, t, hq, d]
 *         k, v (new rows)   [n, t, hkv, d]
 *         cache_k, cache_v  [n, hkv, s_cap, d]
 *         positions         [n, t]   int32
 *         lens              [n]      int32   (valid history rows per unit)
 *     n counts independent units (layers x sequences); every unit has its own cache.
 *   - Query head h reads KV head h / (hq / hkv).  hq must be a multiple of hkv.
 *   - d must be 128.  Tensor pointers must be 16-byte aligned.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream) and
 *     never synchronises.  The caller owns every buffer; the library allocates and frees
 *     no device memory and keeps no per-call state.
 *   - Return value: ATTN_OK (0) or a negative status.  Every status except ATTN_ERR_HIP
 *     is decided on the host before any HIP call, so on error nothing has been launched
 *     and no buffer has been touched.  No call clamps silently.
 *   - The library's only state is per thread: the hipError_t of the last failed launch
 *     (attn_last_hip_error) and the profiling hook (attn_set_profile_events).
 *   - Lengths and positions live in device memory and are not read by the host.  The
 *     host checks the capacity with the caller's bound `max_len` (>= every lens[u]).  A
 *     kernel that finds lens[u] < 0 or lens[u] > max_len writes no cache row of unit u
 *     and fills that unit's output with NaN, so a wrong bound never writes out of bounds.
 *   - `out` must not overlap q, k, v or the caches.
 */
#ifndef KVROPE_H
#define KVROPE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_OK 0
#define ATTN_ERR_NULL (-1)      /* a required pointer is NULL */
#define ATTN_ERR_SHAPE (-2)     /* negative size, d != 128, hq % hkv != 0, hkv < 1 */
#define ATTN_ERR_ROPE (-3)      /* n_rot odd / < 2 / > d, base <= 1, bad YaRN field, bad set */
#define ATTN_ERR_CAPACITY (-4)  /* max_len + t > s_cap, or max_len < 0 */
#define ATTN_ERR_ALIGN (-5)     /* a tensor pointer is not 16-byte aligned */
#define ATTN_ERR_WORKSPACE (-6) /* workspace smaller than attn_workspace_size() */
#define ATTN_ERR_SCALE (-7)     /* softmax scale not finite or <= 0 */
#define ATTN_ERR_HIP (-8)       /* a HIP launch failed (see attn_last_hip_error) */

/* Most rotary parameter sets one call can carry (kvrope_rope_params.n_sets). */
#define KVROPE_MAX_ROPE_SETS 4

/* Rotary embedding parameters ([ds4] Traces 1-2).
 * Pair j = 0 .. n_rot/2-1 of a head, with o = d - n_rot, is the dims
 *     (o + 2j, o + 2j + 1)          pairing 0 (adjacent, as the trace prints it)
 *     (o + j, o + j + n_rot/2)      pairing 1 (half-split; requires n_rot % 32 == 0)
 * and turns by theta = pos * w_j with
 *     w_j = base^(-2j / n_rot)                                   (plain)
 *     w_j = base^(-2j / n_rot) * (freq_scale * (1 - g_j) + g_j)   (yarn)
 *     g_j = ext_factor * ramp(c(beta_fast), c(beta_slow), j)
 *     c(beta) = n_rot * ln(n_ctx_orig / (2 pi beta)) / (2 ln base)
 *     ramp(lo, hi, j) = 1 - clamp((j - lo) / max(0.001, hi - lo), 0, 1)
 * The pair (x0, x1) becomes (x0 c - x1 s, x0 s + x1 c) with c = cos(theta) * mscale,
 * s = sgn * sin(theta) * mscale, sgn = -1 for the inverse rotation ([ds4] Trace 2's
 * `inverse` flag), else +1.  Dims [0, o) are left unchanged.  Plain RoPE over a whole
 * head is n_rot = d, yarn = 0, mscale = 1, and the added fields zero.
 * Tables ([Sophgo] Listings 1-2 gather precomputed cos / sin by position_ids): when
 * cos_table and sin_table are set (device, float32 [table_rows, n_rot/2], 4-byte
 * aligned), pair j of a token at position p takes c = cos_table[p][j] and
 * s = sgn * sin_table[p][j] instead (base, yarn fields and mscale are then not used).  A
 * token whose position lies outside [0, table_rows) gets NaN in its rotated dims (the
 * library cannot report it; for k that row of the cache holds NaN). */
typedef struct kvrope_rope_params {
    double base;        /* > 1 (10000 in the workloads) */
    int32_t n_rot;      /* even, 2 .. d */
    int32_t yarn;       /* 0 = plain, 1 = YaRN ramp */
    double freq_scale;  /* yarn: 1 / scale factor, > 0 */
    double ext_factor;  /* yarn: ramp weight, in [0, 1] */
    int32_t n_ctx_orig; /* yarn: > 0 */
    double beta_fast;   /* yarn: > 0 */
    double beta_slow;   /* yarn: > 0 */
    double mscale;      /* finite, > 0 */
    int32_t pairing;    /* 0 = adjacent, 1 = half-split */
    int32_t inverse;    /* 0 = forward, 1 = inverse rotation */
    const float *cos_table; /* NULL, or device float32 [table_rows, n_rot / 2] */
    const float *sin_table; /* NULL exactly when cos_table is */
    int32_t table_rows;     /* >= 1 when the tables are set */
    /* Per-unit parameter sets ([ds4] Part 4 sec. 1, Trace 2: every layer has its own
     * frequency base and scale, and only the compressed layers switch the YaRN ramp on).
     * n_sets = 0: the fields above serve every unit.  1 <= n_sets <= KVROPE_MAX_ROPE_SETS:
     * unit u takes base, yarn, freq_scale, ext_factor, n_ctx_orig, beta_fast, beta_slow
     * and mscale from sets[unit_set[u]] (each set is checked like the fields above;
     * the sets' other fields are not read); n_rot, pairing and inverse stay this
     * struct's.  Sets and tables exclude each other.  A unit whose device index lies
     * outside [0, n_sets) gets NaN in its rotated dims (as for a position outside a
     * table). */
    int32_t n_sets;
    const struct kvrope_rope_params *sets; /* host array [n_sets] (read during the call) */
    const int32_t *unit_set;               /* device int32 [n], 4-byte aligned */
} kvrope_rope_params;

/* attn_rope_apply -- rotate x in place ([Sophgo] Listings 1-2: top.Rope(x, cos, sin) on
 * q and on k at position_ids; [ds4] Trace 2).
 *   x          device, f16 [n, t, h, d], rotated in place
 *   positions  device, int32 [n, t]
 * Each rotated value is computed in fp64 and rounded to f16 (nearest, ties to even). */
int attn_rope_apply(void *x, const int32_t *positions, int n, int t, int h, int d,
                    const kvrope_rope_params *rp, void *stream);

/* kv_cache_append -- copy new rows into the caches ([Sophgo] Listing 2 Concat(history,
 * new); [Buddy] sec. 6.4.5): cache_k[u, g, lens[u] + i, :] = k[u, i, g, :] and the same
 * for v, for i < t.  Bit copy; every other row is untouched.
 *   lens      device, int32 [n], history rows per unit; the host checks
 *             max_len + t <= s_cap with the caller's bound max_len >= every lens[u]. */
int kv_cache_append(void *cache_k, void *cache_v, const void *k, const void *v,
                    const int32_t *lens, int max_len, int n, int t, int hkv, int d, int s_cap,
                    void *stream);

/* attn_prefill -- a block without history ([Sophgo] Listing 1, sec. 4.1 prefill): the
 * same as attn_prefill_kv with every history length 0 (hist_lens may be NULL here). */
int attn_prefill(const void *q, const void *k, const void *v, const int32_t *positions,
                 void *cache_k, void *cache_v, void *out, int n, int t, int hq, int hkv, int d,
                 int s_cap, double scale, const kvrope_rope_params *rp, void *stream);

/* attn_prefill_kv -- chunked prefill over a history ([Sophgo] Listing 2, sec. 4.1).
 *   history_k, history_v  device, f16 [n, hkv, s_cap, d]: the per-unit caches.  Rows
 *             [0, hist_lens[u]) hold already-rotated history and are read only.
 *   hist_lens device, int32 [n]; max_hist >= every hist_lens[u] (host bound).
 * Steps: k is rotated at `positions` (fp64, rounded to f16) and written with v to rows
 * [hist_lens[u], hist_lens[u] + t); then new token i of unit u and query head h attends
 * over rows 0 .. hist_lens[u] + i of KV head h / (hq / hkv):
 *     out = softmax(scale * q_hat K^T) V,
 * where q_hat is q rotated at `positions` and rounded to f16.  The scores and the softmax
 * are fp32; out is rounded to f16.  Requires max_hist + t <= s_cap. */
int attn_prefill_kv(const void *q, const void *k, const void *v, const int32_t *positions,
                    void *history_k, void *history_v, const int32_t *hist_lens, int max_hist,
                    void *out, int n, int t, int hq, int hkv, int d, int s_cap, double scale,
                    const kvrope_rope_params *rp, void *stream);

/* attn_prefill_kv_varlen -- attn_prefill_kv over a batch whose units bring different
 * numbers of new tokens (continuous batching of resumed conversations; the chunked
 * prefill of [Sophgo] Listing 2 per sequence, history lengths already per unit).
 *   new_lens  device, int32 [n]: unit u's new tokens are rows 0 .. new_lens[u] - 1 of its
 *             q, k, v, positions (all padded to t rows); 0 <= new_lens[u] <= t.
 * Unit u computes exactly what attn_prefill_kv computes for that unit alone with
 * t = new_lens[u]: cache rows [hist_lens[u], hist_lens[u] + new_lens[u]) are written and
 * out rows 0 .. new_lens[u] - 1.  Padding rows of out and every other cache row are left
 * as they were; padding rows of q, k, v and positions may hold anything (they are read
 * but never used).  A unit with new_lens[u] outside [0, t] is treated like an invalid
 * history length: no cache row written, NaN in all t of its out rows.  new_lens may not be
 * NULL (ATTN_ERR_NULL) unless n * t == 0; everything else as for attn_prefill_kv. */
int attn_prefill_kv_varlen(const void *q, const void *k, const void *v, const int32_t *positions,
                           void *history_k, void *history_v, const int32_t *hist_lens, int max_hist,
                           const int32_t *new_lens, void *out, int n, int t, int hq, int hkv, int d,
                           int s_cap, double scale, const kvrope_rope_params *rp, void *stream);

/* attn_decode -- one new token per unit ([Sophgo] sec. 4.1 decode; [Buddy] sec.
 * 6.4.5-6.4.6).
 *   q    [n, 1, hq, d] (= [n, hq, d]);  k, v  [n, 1, hkv, d];  positions [n]
 *   cache_lens  device, int32 [n]: rows already in the cache; max_len >= every one.
 *   workspace   device scratch of at least attn_workspace_size(ATTN_OP_DECODE, n, 1,
 *               hq, hkv, d, max_len) bytes (may be NULL when that size is 0).  Its
 *               contents on entry do not matter; calls sharing one workspace must be
 *               ordered on one stream.
 * Steps: q and k are rotated at positions[u] (k in fp64, both rounded to f16); the new
 * k, v are written to row cache_lens[u]; then every query head attends over rows
 * 0 .. cache_lens[u] (cache_lens[u] + 1 keys), split into key chunks whose partial
 * softmax states are merged in a fixed order (deterministic).  The caller advances its
 * lengths; the library never writes them.  Requires max_len + 1 <= s_cap. */
int attn_decode(const void *q, const void *k, const void *v, const int32_t *positions,
                void *cache_k, void *cache_v, const int32_t *cache_lens, int max_len,
                void *out, int n, int hq, int hkv, int d, int s_cap, double scale,
                const kvrope_rope_params *rp, void *workspace, size_t ws_bytes,
                void *stream);

/* attn_decode_noalloc -- attn_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same steps, kernels and results, with the split-key partials kept in a scratch
 * array the library holds on each GPU (attn_decode_noalloc_max_workspace() bytes, 64 MiB,
 * for the life of the process) instead of a caller workspace.  The call allocates and
 * frees nothing.  Shapes whose workspace (attn_workspace_size(ATTN_OP_DECODE, ...))
 * exceeds the scratch size return ATTN_ERR_WORKSPACE before any HIP call; the first call
 * on a device looks up that device's scratch address (hipGetSymbolAddress; a failure is
 * ATTN_ERR_HIP).  Every call on one GPU shares its scratch: calls that overlap on one GPU
 * (on different streams, or from different threads without ordering) race and may
 * return wrong outputs; calls ordered on one stream are safe.  No part of the scratch
 * needs to start at zero.  Everything else as attn_decode. */
int attn_decode_noalloc(const void *q, const void *k, const void *v, const int32_t *positions,
                        void *cache_k, void *cache_v, const int32_t *cache_lens, int max_len,
                        void *out, int n, int hq, int hkv, int d, int s_cap, double scale,
                        const kvrope_rope_params *rp, void *stream);

/* Bytes of device scratch attn_decode_noalloc holds per GPU (its workspace limit). */
size_t attn_decode_noalloc_max_workspace(void);

/* ---- The projections either side of attention ([Sophgo] Listings 1-2: q, k, v =
 * MatMul(x, w_q / w_k / w_v), Rope on q and k, Concat into the cache; h = Add(input,
 * MatMul(attn, w_o))), on f16 MFMA with fp32 accumulation.  Weights are stored one row per
 * output feature ([out_features, in_features], the transpose of the listings' w), so
 * y = x . w^T.  w_per_unit = 0: one weight matrix for all n units; 1: n matrices back to
 * back (e.g. one per layer when the units are layers).
 *
 * attn_qkv_project -- the QKV projection with the rotary embedding of k and the cache
 * append as its epilogue.
 *   x       device, f16 [n, t, hidden]; hidden a multiple of 64
 *   w_qkv   device, f16 [(w_per_unit ? n : 1), (hq + 2 hkv) * d, hidden]: rows 0 .. hq d - 1
 *           project q (head h = rows h d .. h d + d - 1), then hkv * d rows for k, then v
 *   q       device, f16 [n, t, hq, d] out: the projected q, rounded to f16, NOT rotated (the
 *           attention entry points rotate q themselves)
 *   k, v    never written to memory: the projected k (rounded to f16) is rotated at
 *           positions[u][i] exactly as attn_rope_apply rotates (fp64, rounded once) and
 *           written with v (rounded to f16) to cache rows lens[u] + i, i < t
 *   lens, max_len, s_cap, positions, rp: as for attn_prefill_kv (lens may be NULL: all 0)
 * Each projected value is the f16 rounding of an fp32-accumulated dot product, so it may
 * differ by one f16 ulp from the rounding of the exact product where the two straddle a
 * rounding boundary.
 *
 * attn_out_project -- out = attn . w_o^T + residual, rounded once to f16.
 *   attn      device, f16 [n, t, hq * d]  (the attention output, [n, t, hq, d])
 *   w_o       device, f16 [(w_per_unit ? n : 1), hidden, hq * d]; hidden a multiple of 128
 *   residual  device, f16 [n, t, hidden];  out  device, f16 [n, t, hidden] (may alias
 *             residual)
 * Both are asynchronous on `stream` and return ATTN_OK, ATTN_ERR_SHAPE, ATTN_ERR_NULL,
 * ATTN_ERR_ALIGN, ATTN_ERR_CAPACITY / ATTN_ERR_ROPE (qkv) or ATTN_ERR_HIP. */
/* attn_prefill_kv_cached -- attn_prefill_kv whose new k, v rows are already in the caches
 * (written by attn_qkv_project): rows [hist_lens[u], hist_lens[u] + t) of each cache hold
 * the rotated k and the v of the t new tokens; the caches are only read.  q is the
 * unrotated query (rotated here at `positions`); everything else as attn_prefill_kv. */
int attn_prefill_kv_cached(const void *q, const int32_t *positions, const void *cache_k, const void *cache_v,
                           const int32_t *hist_lens, int max_hist, void *out, int n, int t, int hq, int hkv,
                           int d, int s_cap, double scale, const kvrope_rope_params *rp, void *stream);
int attn_qkv_project(const void *x, const void *w_qkv, int w_per_unit, const int32_t *positions, void *q,
                     void *cache_k, void *cache_v, const int32_t *lens, int max_len, int n, int t, int hidden,
                     int hq, int hkv, int d, int s_cap, const kvrope_rope_params *rp, void *stream);
int attn_out_project(const void *attn, const void *w_o, int w_per_unit, const void *residual, void *out, int n,
                     int t, int hq, int d, int hidden, void *stream);

#define ATTN_OP_DECODE 1

/* Bytes of device workspace the operation needs (0 for operations that need none). */
size_t attn_workspace_size(int op, int n, int t, int hq, int hkv, int d, int max_len);

/* How attn_decode splits the work for this shape: a unit's cache_lens[u] + 1 keys are cut
 * into the fewest chunks of at most this many keys (a multiple of 32), of equal size
 * rounded up to 32 keys, one workgroup per chunk (0 for an invalid shape).  For
 * benchmarks that reproduce the same access pattern. */
int attn_decode_chunk_keys(int n, int hq, int hkv, int max_len);

/* Static description of a status code (never NULL). */
const char *attn_status_string(int status);

/* The hipError_t of the most recent ATTN_ERR_HIP on the calling thread (0 if none). */
int attn_last_hip_error(void);

/* Profiling hook of the calling thread.  When `before` / `after` are non-NULL hipEvent_t
 * handles, the next attn_prefill, attn_prefill_kv, attn_prefill_kv_varlen,
 * attn_prefill_kv_cached or attn_decode call made ON THIS THREAD records `before` on its
 * stream just before its attention kernel (the flash kernel of prefill, the split-key
 * kernel of decode) and `after` just after that same kernel, then clears the hook.  Calls
 * on other threads neither see nor clear it.  Returns ATTN_OK. */
int attn_set_profile_events(void *before, void *after);

#ifdef __cplusplus
}
#endif

#endif /* KVROPE_H */
