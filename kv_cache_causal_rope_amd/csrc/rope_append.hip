// rope_append.hip -- rotary embedding and KV-cache append kernels (gfx950).
//
// Rotation ("ds4.c study notes", Part 4 sec. 1, Trace 2): pair j of a head holds dims
// (off + 2j, off + 2j + 1), off = d - n_rot (or, half-split, (off + j, off + j + n_rot/2));
// with theta = pos * w[j], c = cos(theta) * mscale and s = sgn * sin(theta) * mscale
// (sgn = -1 for the inverse rotation) the pair (x0, x1) becomes (x0 c - x1 s, x0 s + x1 c);
// w and mscale are those of the unit's parameter set (Trace 2: a frequency base and
// scale per layer).
// With caller tables (the Sophgo MLIR-based LLM compilation paper, Listings 1-2: cos / sin
// gathered by position_ids) c and s / sgn are the table entries of the token's position.
// These kernels evaluate it in fp64 and round once to f16 (nearest even), so a rotated K
// row in the cache is the correctly rounded f16 of the exact rotation.  The angle is taken in turns (pos * w[j] / 2 pi, reduced exactly to a
// fraction of a turn) and its sine and cosine come from Taylor series on at most an
// eighth of a turn: within a few 1e-16 of fp64 sin / cos of pos * w[j], at a fraction
// of their cost.
//
// Append (Sophgo MLIR-based LLM compilation paper, sec. 3.1 Listing 2: Concat(history,
// new); Buddy-MLIR walkthrough, sec. 6.4.5): new row i of unit u goes to cache row
// lens[u] + i of its KV head.  Every kernel here moves 16-byte chunks so that a wave's
// accesses to one row are contiguous.
#include "device_common.h"
#include "launch.h"
#include "rope_device.h"

namespace kvrope {

namespace {

// 16-byte chunks per row a thread of the rotation kernels starts from: every chunk of
// the rotated region (adjacent pairs), or its first half (half-split pairs, the thread
// also taking the partner chunk)
inline int rope_chunks(const RopeTable &tab)
{
    return tab.half ? tab.n_pairs >> 3 : (kHeadDim >> 3) - (tab.off >> 3);
}

// x[rows, h, 128] rotated in place, rows = units x t; one thread per (row, 16-byte chunk
// of the rotated region), looping over the heads so the trig is shared by all heads of a
// row.  One instance per pairing (own register allocation, as for rope_append_kernel).
template <bool HALF>
__global__ void __launch_bounds__(256) rope_inplace_kernel(uint16_t *__restrict__ x,
                                                           const int32_t *__restrict__ positions,
                                                           int64_t rows, int t, int h, RopeTable tab)
{
    const int first_chunk = tab.off >> 3;
    const int nchunks = HALF ? tab.n_pairs >> 3 : (kHeadDim >> 3) - first_chunk;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * nchunks)
        return;
    const int c = first_chunk + (int)(idx % nchunks);
    const int64_t r = idx / nchunks;
    const int pos = positions[r];
    const int set = rope_set(tab, (int)(r / t));
    if (HALF) {
        const int c2 = c + (tab.n_pairs >> 3);
        for (int hh = 0; hh < h; ++hh) {
            uint4 *p = reinterpret_cast<uint4 *>(x + (r * h + hh) * kHeadDim);
            Chunk16 a, b, ya, yb;
            a.v = p[c];
            b.v = p[c2];
            rotate_half_chunks(a.h, b.h, ya.h, yb.h, 8 * (c - first_chunk), pos, tab, set);
            p[c] = ya.v;
            p[c2] = yb.v;
        }
        return;
    }
    double cs[4], sn[4];
    chunk_trig(c, pos, tab, set, cs, sn);
    for (int hh = 0; hh < h; ++hh) {
        uint4 *p = reinterpret_cast<uint4 *>(x + (r * h + hh) * kHeadDim) + c;
        Chunk16 in, out;
        in.v = *p;
        rotate_chunk_f64(in.h, out.h, c, cs, sn, tab.off);
        *p = out.v;
    }
}

// Pure copy of new rows into the caches: one thread per 16-byte chunk of k (and v).
__global__ void __launch_bounds__(256) append_kernel(uint16_t *__restrict__ cache_k,
                                                     uint16_t *__restrict__ cache_v,
                                                     const uint16_t *__restrict__ k,
                                                     const uint16_t *__restrict__ v,
                                                     const int32_t *__restrict__ lens,
                                                     int max_len, int n, int t, int hkv,
                                                     int s_cap)
{
    const int64_t total = (int64_t)n * t * hkv * 16;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total)
        return;
    const int c = (int)(idx & 15);
    int64_t rest = idx >> 4;
    const int g = (int)(rest % hkv);
    rest /= hkv;
    const int i = (int)(rest % t);
    const int u = (int)(rest / t);
    const int len = lens[u];
    if (len < 0 || len > max_len)
        return; // host bound violated: leave the cache untouched
    const int64_t src = (((int64_t)u * t + i) * hkv + g) * kHeadDim;
    const int64_t dst = (((int64_t)u * hkv + g) * s_cap + len + i) * kHeadDim;
    reinterpret_cast<uint4 *>(cache_k + dst)[c] = reinterpret_cast<const uint4 *>(k + src)[c];
    reinterpret_cast<uint4 *>(cache_v + dst)[c] = reinterpret_cast<const uint4 *>(v + src)[c];
}

// Fused prefill step 1: rotate new k (fp64 -> f16 RNE) and write k, v to cache rows
// [lens[u], lens[u] + t).  One thread per (unit, token, 16-byte chunk), looping over
// the KV heads so the trig of a (token, pair) is computed once.  The loads a thread needs
// before its first store go out together, ahead of any use: the unit's counts, the
// token's position, the rotation inputs and head 0's k and v chunks (from addresses that
// do not depend on the loaded counts); a unit or row that is not appended discards them.
// One instance per pairing, each with its own register allocation: the adjacent pairing's
// uses 66 VGPRs (7 waves a SIMD) instead of the 108 (4) that the half-split path's eight
// factors a thread cost a shared one (T = 1024 28-layer prefill: 17.8 -> 14.5 us).
template <bool HALF>
__global__ void __launch_bounds__(256)
rope_append_kernel(
    uint16_t *__restrict__ cache_k, uint16_t *__restrict__ cache_v,
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ positions, const int32_t *__restrict__ lens,
    const int32_t *__restrict__ new_lens, int max_len, int n, int t, int hkv, int s_cap, RopeTable tab)
{
    const int64_t total = (int64_t)n * t * 16;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total)
        return;
    const int c = (int)(idx & 15);
    const int64_t ti = idx >> 4;
    const int i = (int)(ti % t);
    const int u = (int)(ti / t);
    const int len = lens ? lens[u] : 0;
    const int tu = new_lens ? new_lens[u] : t;
    const int pos = positions[ti];
    const int set = rope_set(tab, u);
    const int64_t src = ((int64_t)u * t + i) * hkv * kHeadDim; // head 0's row of token i
    auto dst_row = [&](int g) { return (((int64_t)u * hkv + g) * s_cap + len + i) * kHeadDim; };
    if (!HALF) {
        int j[4];
        chunk_pairs(c, tab, j);
        TrigIn<4> tin;
        trig_load(j, pos, tab, set, tin);
        // the k and v chunks of head 0 (the other heads' after it is stored)
        const uint4 *ks = reinterpret_cast<const uint4 *>(k + src) + c;
        const uint4 *vs = reinterpret_cast<const uint4 *>(v + src) + c;
        const uint4 k0 = ks[0], v0 = vs[0];
        double cs[4], sn[4];
        chunk_trig_eval(c, pos, tab, set, tin, cs, sn);
        const bool rotated = 8 * c + 7 >= tab.off;
        auto put = [&](int g, uint4 kc, uint4 vc) {
            Chunk16 in, out;
            in.v = kc;
            if (rotated)
                rotate_chunk_f64(in.h, out.h, c, cs, sn, tab.off);
            else
                out.v = in.v;
            const int64_t d = dst_row(g);
            reinterpret_cast<uint4 *>(cache_k + d)[c] = out.v;
            reinterpret_cast<uint4 *>(cache_v + d)[c] = vc;
        };
        // a padding row or an invalid count appends nothing; tested only here, after the
        // loads, so that the compiler keeps them ahead of the wait for the counts
        if (len < 0 || len > max_len || (new_lens && (tu < 0 || tu > t || i >= tu)))
            return;
        put(0, k0, v0);
        for (int g = 1; g < hkv; ++g)
            put(g, ks[g * (kHeadDim / 8)], vs[g * (kHeadDim / 8)]);
        return;
    }
    // chunks before `off` copy K; a first-half chunk rotates with its partner and
    // writes both; a second-half chunk only copies V
    if (len < 0 || len > max_len || (new_lens && (tu < 0 || tu > t || i >= tu)))
        return; // padding row, or an invalid count: nothing appended
    const int first_chunk = tab.off >> 3, h8 = tab.n_pairs >> 3;
    for (int g = 0; g < hkv; ++g) {
        const uint4 *ks = reinterpret_cast<const uint4 *>(k + src + g * kHeadDim);
        uint4 *kd = reinterpret_cast<uint4 *>(cache_k + dst_row(g));
        if (c < first_chunk) {
            kd[c] = ks[c];
        } else if (c < first_chunk + h8) {
            Chunk16 a, b, ya, yb;
            a.v = ks[c];
            b.v = ks[c + h8];
            rotate_half_chunks(a.h, b.h, ya.h, yb.h, 8 * (c - first_chunk), pos, tab, set);
            kd[c] = ya.v;
            kd[c + h8] = yb.v;
        }
        reinterpret_cast<uint4 *>(cache_v + dst_row(g))[c] =
            reinterpret_cast<const uint4 *>(v + src + g * kHeadDim)[c];
    }
}

inline unsigned grid_for(int64_t threads, int block) { return (unsigned)((threads + block - 1) / block); }

} // namespace

hipError_t launch_rope_inplace(uint16_t *x, const int32_t *positions, int64_t rows, int t, int h,
                               const RopeTable &tab, hipStream_t stream)
{
    const int64_t threads = rows * rope_chunks(tab);
    if (threads == 0)
        return hipSuccess;
    hipLaunchKernelGGL(tab.half ? rope_inplace_kernel<true> : rope_inplace_kernel<false>,
                       dim3(grid_for(threads, 256)), dim3(256), 0, stream, x, positions, rows, t, h, tab);
    return hipGetLastError();
}

hipError_t launch_append(uint16_t *cache_k, uint16_t *cache_v, const uint16_t *k,
                         const uint16_t *v, const int32_t *lens, int max_len, int n, int t,
                         int hkv, int s_cap, hipStream_t stream)
{
    const int64_t threads = (int64_t)n * t * hkv * 16;
    if (threads == 0)
        return hipSuccess;
    hipLaunchKernelGGL(append_kernel, dim3(grid_for(threads, 256)), dim3(256), 0, stream,
                       cache_k, cache_v, k, v, lens, max_len, n, t, hkv, s_cap);
    return hipGetLastError();
}

hipError_t launch_rope_append(uint16_t *cache_k, uint16_t *cache_v, const uint16_t *k,
                              const uint16_t *v, const int32_t *positions, const int32_t *lens,
                              const int32_t *new_lens, int max_len, int n, int t, int hkv, int s_cap,
                              const RopeTable &tab, hipStream_t stream)
{
    const int64_t threads = (int64_t)n * t * 16;
    if (threads == 0)
        return hipSuccess;
    hipLaunchKernelGGL(tab.half ? rope_append_kernel<true> : rope_append_kernel<false>, dim3(grid_for(threads, 256)),
                       dim3(256), 0, stream, cache_k, cache_v, k, v, positions, lens, new_lens, max_len, n, t,
                       hkv, s_cap, tab);
    return hipGetLastError();
}

} // namespace kvrope
