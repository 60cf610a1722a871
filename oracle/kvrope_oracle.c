/*
 * kvrope_oracle.c -- plain, slow, fp64 CPU reference for the attention hot path
 * (rotary embedding of Q/K, KV-cache append, causal grouped-query attention in the
 * prefill / prefill_kv / decode phases).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  It shares no code, header, table or
 * helper with the GPU library; both sides only read the same seeded inputs.
 *
 * Sources (cited by page title and section):
 *   [Sophgo]  "An MLIR-based LLM compilation method" (Sophgo TPU-MLIR paper):
 *             sec. 2.2 (top.Rope, top.Concat, top.FAttention = scaled dot product + causal
 *             mask), sec. 3.1 Listings 1-2 (block without / with history_k, history_v),
 *             sec. 4.1 (the prefill / prefill_kv / decode split).
 *   [ds4]     "ds4.c study notes", Part 4, section 1, Trace 1 (YaRN ramp and correction
 *             dims) and Trace 2 (tail RoPE rotation, rotation matrix, theta schedule,
 *             per-layer frequency base / scale with the ramp only on compressed layers).
 *   [Buddy]   "Buddy-MLIR DeepSeek model import, compilation and inference scheduling"
 *             (juejin), sec. 6.4.3 (KV cache [B, kv_heads, max_len, head_dim], f16),
 *             sec. 6.4.5-6.4.6 (cache hand-off: position = prompt length, +1 per step),
 *             sec. 6.4.7 (an f16 decode done with a bf16 shift: why the codec here is
 *             hand-written and checked against every bit pattern).
 *   [CGDR]    "02 Prefill integration of CGDR" (MindSpore Qwen3.5 notes), sec. 1-2: the
 *             unfused path expands KV heads with repeat_interleave, so query head h
 *             reads KV head floor(h / G).
 *
 * Where the pages leave a step open, the reading taken is stated next to the code that
 * takes it.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC (see build.py).
 * Every floating-point step is fp64; f16 appears only at tensor boundaries.  The
 * attention loops decode each (unit, KV head) slab of the cache to fp64 once and then
 * sum every dot product and every weighted sum in ascending index order.
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------ */
/* IEEE binary16 codec (fp64 <-> f16, round to nearest, ties to even).                   */
/* Written arithmetically (frexp / ldexp / nearbyint), not by bit surgery.               */
/* ------------------------------------------------------------------------------------ */

double ora_f16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int m = h & 0x3ff;
    double v;
    if (e == 0x1f) {
        v = (m == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    } else {
        v = ldexp((double)(m + 1024), e - 25); /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

uint16_t ora_f64_to_f16(double x)
{
    if (isnan(x))
        return (uint16_t)(signbit(x) ? 0xfe00 : 0x7e00);
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    /* quantum of the f16 grid at the magnitude of a: 2^(max(E,-14)-10), E = floor(log2 a) */
    int e2;
    (void)frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1): E = e2 - 1 */
    int E = e2 - 1;
    if (E < -14)
        E = -14;
    const double quantum = ldexp(1.0, E - 10);
    /* a / quantum is exact (power-of-two scaling); nearbyint rounds half to even */
    const double n = nearbyint(a / quantum);
    const double r = n * quantum; /* exact */
    if (r >= 65536.0)              /* largest finite f16 is 65504; 65520 rounds up to inf */
        return (uint16_t)(sign | 0x7c00);
    /* encode r exactly */
    if (r < ldexp(1.0, -14)) {
        /* subnormal: r = k * 2^-24 */
        const uint16_t k = (uint16_t)ldexp(r, 24);
        return (uint16_t)(sign | k);
    }
    int re;
    const double f = frexp(r, &re); /* r = f * 2^re, f in [0.5,1) */
    const int biased = re - 1 + 15;
    const uint16_t mant = (uint16_t)(ldexp(f, 11) - 1024.0); /* f*2^11 in [1024, 2048) */
    return (uint16_t)(sign | (uint16_t)(biased << 10) | mant);
}

void ora_f16_to_f64_array(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = ora_f16_to_f64(h[i]);
}

void ora_f64_to_f16_array(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = ora_f64_to_f16(x[i]);
}

/* The value of every f16 bit pattern, filled once by ora_f16_to_f64 itself: a lookup in
 * it is that function's result, not a second decoder. */
static double g_f16_value[65536];
static int g_f16_value_ready;

static void ora_fill_f16_values(void)
{
    if (g_f16_value_ready)
        return;
    for (int b = 0; b < 65536; ++b)
        g_f16_value[b] = ora_f16_to_f64((uint16_t)b);
    g_f16_value_ready = 1;
}

/* rows [0, rows) of a [*, d] f16 slab to fp64 */
static void ora_slab_to_f64(const uint16_t *src, int64_t rows, int d, double *dst)
{
    for (int64_t i = 0; i < rows * (int64_t)d; ++i)
        dst[i] = g_f16_value[src[i]];
}

/* the same, transposed: dst[i * rows + j] = row j, dim i (64 rows at a time, so that
 * both sides of the copy stay in cache) */
static void ora_slab_to_f64_t(const uint16_t *src, int64_t rows, int d, double *dst)
{
    for (int64_t j0 = 0; j0 < rows; j0 += 64) {
        const int64_t j1 = j0 + 64 < rows ? j0 + 64 : rows;
        for (int i = 0; i < d; ++i)
            for (int64_t j = j0; j < j1; ++j)
                dst[(int64_t)i * rows + j] = g_f16_value[src[j * d + i]];
    }
}

/* dot[j] = <q, key j> for keys j < nk of a transposed slab kt [d][stride]: the scores of
 * all keys are accumulated one head dim at a time, so each dot product sums its d terms
 * in ascending dim order. */
static void ora_scores(const double *q, const double *kt, int64_t stride, int64_t nk, int d, double *dot)
{
    for (int64_t j = 0; j < nk; ++j)
        dot[j] = 0.0;
    for (int i = 0; i < d; ++i) {
        const double qi = q[i];
        const double *ki = kt + (int64_t)i * stride;
        for (int64_t j = 0; j < nk; ++j)
            dot[j] += qi * ki[j];
    }
}

/* ------------------------------------------------------------------------------------ */
/* Rotary embedding parameters and per-pair frequencies.                                 */
/* ------------------------------------------------------------------------------------ */

typedef struct ora_rope_params {
    double base;        /* theta base (10000 in every workload here) */
    int32_t n_rot;      /* rotated dims per head (even); they are the LAST n_rot dims */
    int32_t yarn;       /* 0: plain RoPE; 1: YaRN ramp between interpolated/extrapolated */
    double freq_scale;  /* YaRN: 1 / scale factor */
    double ext_factor;  /* YaRN: weight of the ramp */
    int32_t n_ctx_orig; /* YaRN: original training context */
    double beta_fast;   /* YaRN: correction-dim boundary (fast) */
    double beta_slow;   /* YaRN: correction-dim boundary (slow) */
    double mscale;      /* magnitude factor applied to both outputs of every rotated pair */
    int32_t pairing;    /* 0: adjacent pairs (o + 2j, o + 2j + 1); 1: half-split pairs
                           (o + j, o + j + n_rot/2) */
    int32_t inverse;    /* 1: rotate by -theta (the sine's sign flipped) */
    const float *cos_table; /* optional [table_rows][n_rot/2] factors gathered by position */
    const float *sin_table; /* (both or neither); they replace cos/sin(theta) * mscale */
    int32_t table_rows;
} ora_rope_params;

/* [ds4] Trace 1: the dimension index at which a pair turns `beta` full circles over the
 * original context.  A pair of frequency base^(-2 x / n_dims) turns
 * n_ctx_orig * base^(-2 x / n_dims) / (2 pi) times over n_ctx_orig positions; setting
 * that count to beta and solving for x gives
 *     x = n_dims * ln(n_ctx_orig / (2 pi beta)) / (2 ln base).
 * Reading: n_dims is the rotated width n_rot; x is used unrounded and unclamped (the page
 * elides the body of the two-boundary helper). */
double ora_yarn_corr_dim(int n_dims, int n_ctx_orig, double beta, double base)
{
    return (double)n_dims * log((double)n_ctx_orig / (2.0 * M_PI * beta)) / (2.0 * log(base));
}

/* [ds4] Trace 1: the ramp over the pair index j (= i0/2) is 1 up to `low` (the pair keeps
 * its original frequency), 0 from low + width on (fully interpolated) and falls linearly
 * in between; width = high - low, floored at 0.001 as on the page. */
double ora_yarn_ramp(double low, double high, int j)
{
    const double width = fmax(0.001, high - low);
    const double along = ((double)j - low) / width; /* 0 at low, 1 at low + width */
    if (along <= 0.0)
        return 1.0;
    if (along >= 1.0)
        return 0.0;
    return 1.0 - along;
}

/* Per-pair effective angular frequency omega_eff[j], j = 0 .. n_rot/2 - 1.
 * [ds4] Trace 2: theta = pos * base^(-2 j / n_rot) for pair j (the exponent uses the
 * rotated width n_rot, so the tail rotation has its own schedule).
 * YaRN reading (the page gives this step only as a comment): the ramp value
 * gamma = ext_factor * ramp(d0, d1, j) mixes the interpolated frequency freq_scale*omega
 * with the original omega: omega_eff = omega * (freq_scale * (1 - gamma) + gamma).
 * Reading: the angle is pos * omega_eff (the position multiplies the effective frequency).
 * gamma_out (optional) receives gamma; dims_out (optional) receives d0, d1. */
void ora_rope_freqs(const ora_rope_params *rp, double *omega_eff, double *gamma_out,
                    double *dims_out)
{
    const int half = rp->n_rot / 2;
    double d0 = 0.0, d1 = 0.0;
    if (rp->yarn) {
        d0 = ora_yarn_corr_dim(rp->n_rot, rp->n_ctx_orig, rp->beta_fast, rp->base);
        d1 = ora_yarn_corr_dim(rp->n_rot, rp->n_ctx_orig, rp->beta_slow, rp->base);
    }
    if (dims_out) {
        dims_out[0] = d0;
        dims_out[1] = d1;
    }
    for (int j = 0; j < half; ++j) {
        const double omega = pow(rp->base, -2.0 * (double)j / (double)rp->n_rot);
        double gamma = 1.0;
        double w = omega;
        if (rp->yarn) {
            gamma = rp->ext_factor * ora_yarn_ramp(d0, d1, j);
            w = omega * (rp->freq_scale * (1.0 - gamma) + gamma);
        }
        omega_eff[j] = w;
        if (gamma_out)
            gamma_out[j] = gamma;
    }
}

/* Rotate rows of x into out.
 * x, out: f16 [rows, h, d] (row-major, d innermost); positions: [rows].
 * [ds4] Trace 2 turns each rotated pair by theta and scales it by mscale: read as a
 * complex number z = x0 + i x1, the pair becomes z * mscale * e^(i theta) (the rotation
 * matrix [[cos, -sin], [sin, cos]] of the page is multiplication by e^(i theta)).
 * Reading: the rotated dims are the last n_rot dims of each head (the page's pointer to
 * the head start contradicts its own "tail" wording and the tail-rotation workload).
 * Pairs: (x[o + 2j], x[o + 2j + 1]) as printed on the page (pairing 0), or
 * (x[o + j], x[o + j + n_rot/2]) (pairing 1, the half-split convention of many
 * checkpoints; the same rotation on a permuted pairing), o = d - n_rot.
 * Direction: [ds4] Trace 2 passes an `inverse` flag and a sign on the sine it does not
 * define.  Reading: the inverse rotation turns by -theta (z * mscale * e^(-i theta)).
 * Tables: [Sophgo] Listings 1-2 gather precomputed cos / sin by position_ids
 * (top.Gather(rotary_cos_w, pos_ids)) and hand them to top.Rope.  Reading: one value per
 * rotated pair, rows indexed by position; the gathered (cos, sin) is the whole factor
 * (cos + i sin, no mscale), conjugated for the inverse rotation.  A position outside
 * [0, table_rows) makes that row's rotated dims NaN.
 * Dims [0, o) are copied bit for bit.  out64 (optional) gets the unrounded fp64 values. */
void ora_rope(const uint16_t *x, const int32_t *positions, int64_t rows, int h, int d,
              const ora_rope_params *rp, uint16_t *out, double *out64)
{
    const int half = rp->n_rot / 2;
    const int o = d - rp->n_rot;
    double *omega = (double *)malloc(sizeof(double) * (size_t)(half > 0 ? half : 1));
    ora_rope_freqs(rp, omega, NULL, NULL);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const int p = positions[r];
        double complex factor[half > 0 ? half : 1];
        /* the factor of each rotated pair at this position (a quiet NaN for a position
           the table does not hold) */
        const int in_table = !rp->cos_table || (p >= 0 && p < rp->table_rows);
        for (int j = 0; j < half && !in_table; ++j)
            factor[j] = CMPLX(NAN, NAN);
        for (int j = 0; j < half && in_table; ++j) {
            double complex f;
            if (rp->cos_table) {
                f = CMPLX((double)rp->cos_table[(int64_t)p * half + j],
                          (double)rp->sin_table[(int64_t)p * half + j]);
            } else {
                const double theta = (double)p * omega[j];
                f = rp->mscale * CMPLX(cos(theta), sin(theta));
            }
            factor[j] = rp->inverse ? conj(f) : f;
        }
        for (int hh = 0; hh < h; ++hh) {
            const int64_t head = (r * h + hh) * (int64_t)d;
            for (int i = 0; i < o; ++i) {
                out[head + i] = x[head + i];
                if (out64)
                    out64[head + i] = ora_f16_to_f64(x[head + i]);
            }
            for (int j = 0; j < half; ++j) {
                const int64_t re_at = head + o + (rp->pairing ? j : 2 * j);
                const int64_t im_at = rp->pairing ? re_at + half : re_at + 1;
                const double complex z = CMPLX(ora_f16_to_f64(x[re_at]), ora_f16_to_f64(x[im_at]));
                const double complex w = z * factor[j];
                out[re_at] = ora_f64_to_f16(creal(w));
                out[im_at] = ora_f64_to_f16(cimag(w));
                if (out64) {
                    out64[re_at] = creal(w);
                    out64[im_at] = cimag(w);
                }
            }
        }
    }
    free(omega);
}

/* The parameter set unit u rotates with: sets[unit_set[u]] ([ds4] Part 4 sec. 1, Trace 2:
 * each layer carries its own frequency base and scale, and only the compressed layers
 * turn the YaRN ramp on), or sets[0] for every unit when unit_set is NULL. */
static const ora_rope_params *ora_unit_params(const ora_rope_params *sets, const int32_t *unit_set, int u)
{
    return unit_set ? &sets[unit_set[u]] : &sets[0];
}

/* [Buddy] sec. 6.4.5 / [Sophgo] Listing 2 (Concat(history, new)):
 * cache_k[n, g, lens[n] + t, :] = k[n, t, g, :], same for v; every other row unchanged.
 * Caches: [n, hkv, s_cap, d]; k, v: [n, t, hkv, d].  Returns -1 (and writes nothing) if
 * any lens[n] + t exceeds s_cap: no silent clamping. */
int ora_append(uint16_t *cache_k, uint16_t *cache_v, const uint16_t *k, const uint16_t *v,
               const int32_t *lens, int n, int t, int hkv, int d, int s_cap)
{
    for (int u = 0; u < n; ++u)
        if (lens[u] < 0 || (int64_t)lens[u] + t > s_cap)
            return -1;
    for (int u = 0; u < n; ++u)
        for (int tt = 0; tt < t; ++tt)
            for (int g = 0; g < hkv; ++g) {
                const int64_t dst = (((int64_t)u * hkv + g) * s_cap + lens[u] + tt) * d;
                const int64_t src = (((int64_t)u * t + tt) * hkv + g) * d;
                memcpy(cache_k + dst, k + src, sizeof(uint16_t) * (size_t)d);
                memcpy(cache_v + dst, v + src, sizeof(uint16_t) * (size_t)d);
            }
    return 0;
}

/* rotate q [n, t, hq, d] and k [n, t, hkv, d] unit by unit, each unit with its own set */
static void ora_rope_units(const uint16_t *q, const uint16_t *k, const int32_t *positions, int n, int t,
                           int hq, int hkv, int d, const ora_rope_params *sets, const int32_t *unit_set,
                           uint16_t *qh, uint16_t *kh, double *k64)
{
    for (int u = 0; u < n; ++u) {
        const ora_rope_params *rp = ora_unit_params(sets, unit_set, u);
        const int64_t qo = (int64_t)u * t * hq * d, ko = (int64_t)u * t * hkv * d;
        ora_rope(q + qo, positions + (int64_t)u * t, t, hq, d, rp, qh + qo, NULL);
        ora_rope(k + ko, positions + (int64_t)u * t, t, hkv, d, rp, kh + ko, k64 ? k64 + ko : NULL);
    }
}

/* ------------------------------------------------------------------------------------ */
/* Attention.                                                                            */
/* ------------------------------------------------------------------------------------ */

/* prefill_kv ([Sophgo] Listing 2 and sec. 4.1; prefill is the case lens == 0, Listing 1):
 *   1. rotate q and k at their positions, each unit with its parameter set; the rotated
 *      q and k are rounded to f16 because the Rope op hands f16 tensors to the attention
 *      op in an f16 model;
 *   2. append rotated k and raw v at rows [lens[n], lens[n] + t) of the cache;
 *   3. for query token tt of unit n and query head hq, with g = hq / (h_q / h_kv)
 *      ([CGDR] repeat_interleave head mapping), attend over cache rows j = 0 .. lens[n]+tt
 *      (the causal mask over the concatenation [history; new]):
 *         s_j = scale * <q_hat, K_j>,  p = softmax(s),  o = sum_j p_j V_j.
 * This implementation builds the full masked score matrix of each (unit, head) and then
 * normalises each row; the decode function below is written as a per-query loop instead.
 * q, out: [n, t, hq, d]; k, v: [n, t, hkv, d]; positions: [n, t]; lens: [n] (host);
 * caches: [n, hkv, s_cap, d] (updated in place); sets / unit_set: see ora_unit_params.
 * out64 (optional): unrounded output.  k64 (optional): unrounded rotated k,
 * [n, t, hkv, d].  Returns 0, or -1 on a capacity or shape error (nothing written). */
int ora_prefill_kv(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   const int32_t *positions, uint16_t *cache_k, uint16_t *cache_v,
                   const int32_t *lens, uint16_t *out, int n, int t, int hq, int hkv, int d,
                   int s_cap, double scale, const ora_rope_params *sets, const int32_t *unit_set,
                   double *out64, double *k64)
{
    if (hkv <= 0 || hq % hkv != 0)
        return -1;
    for (int u = 0; u < n; ++u)
        if (lens[u] < 0 || (int64_t)lens[u] + t > s_cap)
            return -1;
    ora_fill_f16_values();
    const int G = hq / hkv;
    const int64_t qn = (int64_t)n * t * hq * d, kn = (int64_t)n * t * hkv * d;
    uint16_t *qh = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(qn > 0 ? qn : 1));
    uint16_t *kh = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(kn > 0 ? kn : 1));
    ora_rope_units(q, k, positions, n, t, hq, hkv, d, sets, unit_set, qh, kh, k64);
    ora_append(cache_k, cache_v, kh, v, lens, n, t, hkv, d, s_cap);

#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int u = 0; u < n; ++u) {
        for (int h = 0; h < hq; ++h) {
            const int g = h / G;
            const int L = lens[u] + t; /* keys visible to the last query */
            const int64_t Lr = L > 0 ? L : 1;
            double *Kd = (double *)malloc(sizeof(double) * (size_t)(Lr * d));
            double *Vd = (double *)malloc(sizeof(double) * (size_t)(Lr * d));
            double *S = (double *)malloc(sizeof(double) * (size_t)t * (size_t)Lr);
            double *qd = (double *)malloc(sizeof(double) * (size_t)d);
            double *acc = (double *)malloc(sizeof(double) * (size_t)d);
            ora_slab_to_f64_t(cache_k + ((int64_t)u * hkv + g) * s_cap * d, L, d, Kd);
            ora_slab_to_f64(cache_v + ((int64_t)u * hkv + g) * s_cap * d, L, d, Vd);
            /* masked score matrix: keys j <= lens + tt are visible to query tt */
            for (int tt = 0; tt < t; ++tt) {
                double *row = S + (int64_t)tt * L;
                const int nvis = lens[u] + tt + 1;
                ora_slab_to_f64(qh + (((int64_t)u * t + tt) * hq + h) * d, 1, d, qd);
                ora_scores(qd, Kd, L, nvis, d, row);
                for (int j = 0; j < L; ++j)
                    row[j] = (j < nvis) ? scale * row[j] : -INFINITY;
            }
            /* row softmax, then P V (each output dim summed over keys in ascending order) */
            for (int tt = 0; tt < t; ++tt) {
                double *row = S + (int64_t)tt * L;
                double mx = -INFINITY;
                for (int j = 0; j < L; ++j)
                    if (row[j] > mx)
                        mx = row[j];
                double sum = 0.0;
                for (int j = 0; j < L; ++j) {
                    row[j] = (row[j] == -INFINITY) ? 0.0 : exp(row[j] - mx);
                    sum += row[j];
                }
                for (int j = 0; j < L; ++j)
                    row[j] /= sum;
                for (int i = 0; i < d; ++i)
                    acc[i] = 0.0;
                for (int j = 0; j < L; ++j) {
                    const double *vr = Vd + (int64_t)j * d;
                    for (int i = 0; i < d; ++i)
                        acc[i] += row[j] * vr[i];
                }
                uint16_t *orow = out + (((int64_t)u * t + tt) * hq + h) * d;
                for (int i = 0; i < d; ++i) {
                    orow[i] = ora_f64_to_f16(acc[i]);
                    if (out64)
                        out64[(((int64_t)u * t + tt) * hq + h) * d + i] = acc[i];
                }
            }
            free(acc);
            free(qd);
            free(S);
            free(Vd);
            free(Kd);
        }
    }
    free(qh);
    free(kh);
    return 0;
}

/* decode ([Sophgo] sec. 4.1: one query per sequence, attending over every earlier key;
 * [Buddy] sec. 6.4.5-6.4.6: the new token sits at the current cache length, which then
 * grows by one).  For unit n: rotate q[n] and k[n] at positions[n] (with the unit's
 * parameter set), write the rotated k and v at cache row lens[n], then for each query
 * head attend over rows 0 .. lens[n].  Written as a per-query loop over the cache (max,
 * then exp-sum, then weighted sum).
 * q, out: [n, hq, d]; k, v: [n, hkv, d]; positions, lens: [n] (host).
 * Returns 0, or -1 (nothing written) on a capacity / shape error. */
int ora_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v,
               const int32_t *positions, uint16_t *cache_k, uint16_t *cache_v,
               const int32_t *lens, uint16_t *out, int n, int hq, int hkv, int d, int s_cap,
               double scale, const ora_rope_params *sets, const int32_t *unit_set, double *out64,
               double *k64)
{
    if (hkv <= 0 || hq % hkv != 0)
        return -1;
    for (int u = 0; u < n; ++u)
        if (lens[u] < 0 || (int64_t)lens[u] + 1 > s_cap)
            return -1;
    ora_fill_f16_values();
    const int G = hq / hkv;
    uint16_t *qh = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)((int64_t)n * hq * d + 1));
    uint16_t *kh = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)((int64_t)n * hkv * d + 1));
    ora_rope_units(q, k, positions, n, 1, hq, hkv, d, sets, unit_set, qh, kh, k64);
    ora_append(cache_k, cache_v, kh, v, lens, n, 1, hkv, d, s_cap);

#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int u = 0; u < n; ++u) {
        for (int h = 0; h < hq; ++h) {
            const int g = h / G;
            const int nk = lens[u] + 1;
            double *Kd = (double *)malloc(sizeof(double) * (size_t)nk * (size_t)d);
            double *Vd = (double *)malloc(sizeof(double) * (size_t)nk * (size_t)d);
            double *qd = (double *)malloc(sizeof(double) * (size_t)d);
            double *s = (double *)malloc(sizeof(double) * (size_t)nk);
            double *acc = (double *)calloc((size_t)d, sizeof(double));
            ora_slab_to_f64_t(cache_k + ((int64_t)u * hkv + g) * s_cap * d, nk, d, Kd);
            ora_slab_to_f64(cache_v + ((int64_t)u * hkv + g) * s_cap * d, nk, d, Vd);
            ora_slab_to_f64(qh + ((int64_t)u * hq + h) * d, 1, d, qd);
            ora_scores(qd, Kd, nk, nk, d, s);
            double mx = -INFINITY;
            for (int j = 0; j < nk; ++j) {
                s[j] = scale * s[j];
                if (s[j] > mx)
                    mx = s[j];
            }
            double denom = 0.0;
            for (int j = 0; j < nk; ++j) {
                const double e = exp(s[j] - mx);
                const double *vr = Vd + (int64_t)j * d;
                denom += e;
                for (int i = 0; i < d; ++i)
                    acc[i] += e * vr[i];
            }
            uint16_t *orow = out + ((int64_t)u * hq + h) * d;
            for (int i = 0; i < d; ++i) {
                const double val = acc[i] / denom;
                orow[i] = ora_f64_to_f16(val);
                if (out64)
                    out64[((int64_t)u * hq + h) * d + i] = val;
            }
            free(acc);
            free(s);
            free(qd);
            free(Vd);
            free(Kd);
        }
    }
    free(qh);
    free(kh);
    return 0;
}

int ora_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* threads the parallel loops use from now on (timing runs only; no effect on results) */
void ora_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
