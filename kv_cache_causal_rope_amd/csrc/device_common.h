// device_common.h -- types and small helpers shared by the gfx950 kernels of libkvrope.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvrope {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
// Native 16-byte vector (HIP's uint4 is a struct with a union inside, which can keep
// values out of registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr int kMaxPairs = kHeadDim / 2;
constexpr int kMaxRopeSets = 4; // KVROPE_MAX_ROPE_SETS

// Per-call rotary table, passed by value as a kernel argument.  Built on the host in
// fp64 (rope_table() in api.hip): pair j of a head rotates dims (off + 2j, off + 2j + 1)
// by 2 pi * pos * wrev[s][j] radians (wrev: revolutions per position) and scales them
// by mscale[s], where s is the unit's parameter set.
struct RopeTable {
    double wrev[kMaxRopeSets][kMaxPairs];
    double mscale[kMaxRopeSets];
    const int32_t *unit_set; // device [n]: set of unit u (NULL: set 0 for every unit)
    int nsets;
    int n_pairs; // n_rot / 2
    int off;     // first rotated dim (d - n_rot)
    int half;    // 1: pair j is dims (off + j, off + j + n_pairs); 0: (off + 2j, off + 2j + 1)
    double sgn;  // sign of the sine: -1 for the inverse rotation
    const float *cos_t; // caller tables [rows][n_pairs] (NULL: cos / sin of the angle)
    const float *sin_t;
    int rows;
};

// The parameter set of unit u, or -1 when the caller's index lies outside [0, nsets)
// (its rotated dims become NaN, like a position a table does not cover).
__device__ inline int rope_set(const RopeTable &tab, int u)
{
    if (!tab.unit_set)
        return 0;
    const int s = tab.unit_set[u];
    return (s >= 0 && s < tab.nsets) ? s : -1;
}

// fp64 -> IEEE binary16, round to nearest, ties to even, by bit manipulation.
// Used for every rotated K value, so the cache holds the correctly rounded f16 of the
// fp64 rotation (no intermediate fp32 rounding).
__host__ __device__ inline uint16_t f64_to_f16_rne(double x)
{
    union {
        double d;
        uint64_t u;
    } cv;
    cv.d = x;
    const uint64_t b = cv.u;
    const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
    const int ex = (int)((b >> 52) & 0x7ff);
    const uint64_t man = b & 0xFFFFFFFFFFFFFull;
    if (ex == 0x7ff)
        return (uint16_t)(sign | (man ? 0x7e00u : 0x7c00u));
    const int e = ex - 1023;
    if (e > 15)
        return (uint16_t)(sign | 0x7c00u);
    if (e >= -14) {
        uint32_t m16 = (uint32_t)(man >> 42) | 0x400u;
        const uint64_t rem = man & ((1ull << 42) - 1);
        const uint64_t half = 1ull << 41;
        if (rem > half || (rem == half && (m16 & 1u)))
            ++m16;
        int eb = e + 15;
        if (m16 == 0x800u) {
            m16 = 0x400u;
            ++eb;
        }
        if (eb >= 31)
            return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | (uint32_t)(eb << 10) | (m16 & 0x3ffu));
    }
    if (ex == 0 || e < -25)
        return sign; // below half of the smallest subnormal (2^-25 itself ties to 0)
    const uint64_t M = man | (1ull << 52);
    const int shift = 28 - e; // 43 .. 53: value in units of 2^-24
    uint64_t qv = M >> shift;
    const uint64_t rem = M & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (qv & 1u)))
        ++qv;
    return (uint16_t)(sign | (uint16_t)qv);
}

// fp64 -> IEEE binary16, round to nearest even, on the conversion units: x is rounded to
// f32 by rounding to odd (the nearest f32, stepped back toward zero when it rounded
// away, with its last bit set when inexact), then f32 -> f16 rounds to nearest even.
// Rounding to odd at 24 bits keeps the second rounding to 11 bits exact, so the result
// equals f64_to_f16_rne bit for bit (NaN: the same quiet NaN).
__device__ inline uint16_t f64_to_f16_rne_dev(double x)
{
    if (x != x)
        return (uint16_t)((__builtin_bit_cast(uint64_t, x) >> 48) & 0x8000u) | 0x7e00u;
    const float f = (float)x;
    const double back = (double)f;
    uint32_t b = __builtin_bit_cast(uint32_t, f);
    if (back != x) {
        if (__builtin_fabs(back) > __builtin_fabs(x))
            b -= 1u;
        b |= 1u;
    }
    return __builtin_bit_cast(uint16_t, (_Float16)__builtin_bit_cast(float, b));
}

__device__ inline float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// Low / high f16 of a 32-bit word, widened to fp32.
__device__ inline float lo2f(uint32_t w) { return h2f((uint16_t)(w & 0xffffu)); }
__device__ inline float hi2f(uint32_t w) { return h2f((uint16_t)(w >> 16)); }

__device__ inline u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ inline void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

__device__ inline double h2d(uint16_t h) { return (double)h2f(h); }

// fp32 -> f16 with the hardware conversion (round to nearest even in the default mode).
__device__ inline uint16_t f2h(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

// Two fp32 -> packed f16 pair (each rounded to nearest even), low half first.
__device__ inline uint32_t pack2h(float a, float b)
{
    return (uint32_t)f2h(a) | ((uint32_t)f2h(b) << 16);
}

__device__ inline uint16_t qnan16() { return 0x7e00u; }

// Combine a lane's value with the one 32 lanes away (lanes l and l ^ 32) without LDS:
// v_permlane32_swap exchanges lanes 32-63 of one register with lanes 0-31 of another, so
// after swapping two copies of x every lane holds {x[l], x[l ^ 32]} in some order.
__device__ inline floatx2 swap_halves(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    return floatx2{__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])};
}
__device__ inline float half_max(float x)
{
    const floatx2 r = swap_halves(x);
    return __builtin_fmaxf(r[0], r[1]);
}
__device__ inline float half_sum(float x)
{
    const floatx2 r = swap_halves(x);
    return r[0] + r[1];
}

} // namespace kvrope
