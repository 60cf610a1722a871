// rope_device.h -- the fp64 rotation of 16-byte f16 chunks shared by the kernels that
// write rotated K rows (gfx950): the rotary-append kernels and the fused projection's
// epilogue.  See rope_append.hip for the method ("ds4.c study notes", Part 4 sec. 1,
// Trace 2; the Sophgo MLIR-based LLM compilation paper, Listings 1-2 for tables).
#pragma once

#include "device_common.h"

namespace kvrope {

namespace {

// Rotate the rotated-region pairs inside one 8-dim chunk (dims 8c .. 8c+7) in fp64.
// cs/sn hold cos/sin * mscale for the chunk's four candidate pairs (unused where a
// dim pair lies before `off`).
__device__ inline void rotate_chunk_f64(const uint16_t (&in)[8], uint16_t (&out)[8], int c,
                                        const double (&cs)[4], const double (&sn)[4], int off)
{
#pragma clang fp contract(off)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int dim = 8 * c + 2 * m;
        if (dim >= off) {
            const double x0 = h2d(in[2 * m]);
            const double x1 = h2d(in[2 * m + 1]);
            const double y0 = x0 * cs[m] - x1 * sn[m];
            const double y1 = x0 * sn[m] + x1 * cs[m];
            out[2 * m] = f64_to_f16_rne_dev(y0);
            out[2 * m + 1] = f64_to_f16_rne_dev(y1);
        } else {
            out[2 * m] = in[2 * m];
            out[2 * m + 1] = in[2 * m + 1];
        }
    }
}

// sin(2 pi r) and cos(2 pi r) in fp64.  r - rint(r) = f in [-1/2, 1/2] is exact; so is
// g = f - q/4 with q = rint(4 f) the nearest quarter turn, |g| <= 1/8.  For x = 2 pi g
// (|x| <= pi/4) the Taylor series of sin through x^15 and of cos through x^16 leave a
// remainder below 5e-17; the quarter turns q then rotate (sin x, cos x).
__device__ inline void sincos_turns(double r, double &s, double &c)
{
    const double f = r - __builtin_rint(r);
    const double q = __builtin_rint(4.0 * f);
    const double x = (f - 0.25 * q) * 6.283185307179586476925;
    const double x2 = x * x;
    const double sx =
        x * (1.0 + x2 * (-1.0 / 6 + x2 * (1.0 / 120 + x2 * (-1.0 / 5040 + x2 * (1.0 / 362880 +
        x2 * (-1.0 / 39916800 + x2 * (1.0 / 6227020800.0 + x2 * (-1.0 / 1307674368000.0))))))));
    const double cx =
        1.0 + x2 * (-1.0 / 2 + x2 * (1.0 / 24 + x2 * (-1.0 / 720 + x2 * (1.0 / 40320 +
        x2 * (-1.0 / 3628800 + x2 * (1.0 / 479001600.0 + x2 * (-1.0 / 87178291200.0 +
        x2 * (1.0 / 20922789888000.0))))))));
    switch ((int)q & 3) {
    case 0: s = sx; c = cx; break;
    case 1: s = cx; c = -sx; break;
    case 2: s = -sx; c = -cx; break;
    default: s = -cx; c = sx; break;
    }
}

// c and s of rotated pair j at position pos under parameter set `set` (rope_set); NaN
// when a table does not cover pos or the set index was invalid
__device__ inline void pair_factor(int j, int pos, const RopeTable &tab, int set, double &c, double &s)
{
#pragma clang fp contract(off)
    if (set < 0) {
        c = s = __builtin_nan("");
    } else if (tab.cos_t) {
        if (pos >= 0 && pos < tab.rows) {
            c = (double)tab.cos_t[(int64_t)pos * tab.n_pairs + j];
            s = (double)tab.sin_t[(int64_t)pos * tab.n_pairs + j] * tab.sgn;
        } else {
            c = s = __builtin_nan("");
        }
    } else {
        double sv, cv;
        sincos_turns((double)pos * tab.wrev[set][j], sv, cv);
        c = cv * tab.mscale[set];
        s = sv * tab.mscale[set] * tab.sgn;
    }
}

// The table entries the factors of N pairs are computed from, read before any of them is
// used: from clamped indices (a pair before `off`, an invalid set or a position the table
// does not cover reads a valid entry that is then discarded), so that the loads of all N
// go out together instead of one round trip after another.
template <int N> struct TrigIn {
    double w[N];   // revolutions per position (computed angles)
    double ms;     // output scale of the set
    float tc[N];   // caller table entries (tables)
    float ts[N];
};
template <int N>
__device__ inline void trig_load(const int (&j)[N], int pos, const RopeTable &tab, int set, TrigIn<N> &in)
{
    const int sc = set < 0 ? 0 : set;
    if (tab.cos_t) {
        const int64_t rb = (int64_t)((pos >= 0 && pos < tab.rows) ? pos : 0) * tab.n_pairs;
#pragma unroll
        for (int m = 0; m < N; ++m) {
            const int jj = min(max(j[m], 0), tab.n_pairs - 1);
            in.tc[m] = tab.cos_t[rb + jj];
            in.ts[m] = tab.sin_t[rb + jj];
        }
    } else {
#pragma unroll
        for (int m = 0; m < N; ++m)
            in.w[m] = tab.wrev[sc][min(max(j[m], 0), kMaxPairs - 1)];
        in.ms = tab.mscale[sc];
    }
}
// c and s of pair m from its loaded entries, as pair_factor computes them
template <int N>
__device__ inline void trig_eval(int m, int pos, const RopeTable &tab, int set, const TrigIn<N> &in, double &c,
                                 double &s)
{
#pragma clang fp contract(off)
    if (set < 0) {
        c = s = __builtin_nan("");
    } else if (tab.cos_t) {
        if (pos >= 0 && pos < tab.rows) {
            c = (double)in.tc[m];
            s = (double)in.ts[m] * tab.sgn;
        } else {
            c = s = __builtin_nan("");
        }
    } else {
        double sv, cv;
        sincos_turns((double)pos * in.w[m], sv, cv);
        c = cv * in.ms;
        s = sv * in.ms * tab.sgn;
    }
}

// adjacent pairing: the rotated pairs of chunk c (dims 8c .. 8c+7)
__device__ inline void chunk_pairs(int c, const RopeTable &tab, int (&j)[4])
{
#pragma unroll
    for (int m = 0; m < 4; ++m)
        j[m] = (8 * c + 2 * m - tab.off) >> 1; // negative: a pair before `off`
}
// the factors of the four pairs of chunk c (identity before `off`) from loaded entries
__device__ inline void chunk_trig_eval(int c, int pos, const RopeTable &tab, int set, const TrigIn<4> &in,
                                       double (&cs)[4], double (&sn)[4])
{
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        cs[m] = 1.0;
        sn[m] = 0.0;
        if (8 * c + 2 * m >= tab.off)
            trig_eval(m, pos, tab, set, in, cs[m], sn[m]);
    }
}
__device__ inline void chunk_trig(int c, int pos, const RopeTable &tab, int set, double (&cs)[4],
                                  double (&sn)[4])
{
    int j[4];
    chunk_pairs(c, tab, j);
    TrigIn<4> in;
    trig_load(j, pos, tab, set, in);
    chunk_trig_eval(c, pos, tab, set, in, cs, sn);
}

// half-split pairing: chunk c0 of the first rotated half and its partner chunk
// c0 + n_pairs / 8 hold the two dims of pairs 8 (c0 - off / 8) + e, e = 0 .. 7
__device__ inline void rotate_half_chunks(const uint16_t (&a)[8], const uint16_t (&b)[8], uint16_t (&ya)[8],
                                          uint16_t (&yb)[8], int j0, int pos, const RopeTable &tab, int set)
{
#pragma clang fp contract(off)
    int j[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        j[e] = j0 + e;
    TrigIn<8> in;
    trig_load(j, pos, tab, set, in);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        double c, s;
        trig_eval(e, pos, tab, set, in, c, s);
        const double x0 = h2d(a[e]);
        const double x1 = h2d(b[e]);
        ya[e] = f64_to_f16_rne_dev(x0 * c - x1 * s);
        yb[e] = f64_to_f16_rne_dev(x0 * s + x1 * c);
    }
}

union Chunk16 {
    uint4 v;
    uint16_t h[8];
};

} // namespace

} // namespace kvrope
