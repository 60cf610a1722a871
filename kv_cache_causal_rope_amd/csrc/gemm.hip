// gemm.hip -- the projections either side of attention (gfx950): the fused QKV projection
// whose epilogue writes q, rotates k and appends k and v to the caches, and the output
// projection with the residual add (the Sophgo MLIR-based LLM compilation paper, sec. 3.1
// Listings 1-2: q/k/v = MatMul(x, w_q/w_k/w_v), Rope on q and k, Concat into the cache,
// h = Add(input, MatMul(attn, w_o))).
//
// Both are C = A . W^T on v_mfma_f32_32x32x16_f16 with f16 inputs and fp32 accumulation:
// A [rows, K] row-major (tokens), W [N, K] row-major (one row per output feature, the
// layout linear layers keep their weights in), so both operands of every MFMA are 16-byte
// runs along K.  A workgroup of 4 waves owns a 128 x 128 tile of C (each wave 64 x 64 =
// 2 x 2 MFMA blocks) and walks K in 64-wide steps through a two-stage LDS ring: each step's
// A and W tiles (16 KB each) go from HBM/L2 straight into LDS (global_load_lds_dwordx4)
// while the previous step's MFMAs run.  LDS rows are 128 bytes; the 16-byte chunk c of row
// r sits at chunk c ^ ((r >> 1) & 7), so the 16 lanes of an operand read (16 consecutive
// rows, one chunk) hit 16 distinct bank groups.
//
// Epilogue: the fp32 tile goes to LDS, then each thread takes 16-byte output chunks:
//   QKV: the tile's 128 columns are one head (head_dim 128): q heads are rounded to f16
//        and written to q (unrotated: the attention kernels rotate q); k heads are rounded
//        to f16 (the k a separate projection would produce), rotated in fp64 and rounded
//        again (as the rotary-append kernel does) into cache row lens[u] + i; v heads are
//        rounded into the V cache row.
//   OUT: fp32 result + residual, rounded once to f16.
#include "device_common.h"
#include "launch.h"
#include "rope_device.h"

#include <stdint.h>

namespace kvrope {

namespace {

constexpr int TM = 128, TN = 128, TK = 64;
constexpr int ROW_B = TK * 2;              // bytes per staged row
constexpr int STAGE_B = 2 * TM * ROW_B;    // A tile + W tile: 32 KB
constexpr int NTHR = 256;

enum { EPI_QKV = 0, EPI_OUT = 1 };

struct GemmParams {
    const uint16_t *a;  // [units, rows_u, K]
    const uint16_t *w;  // [w_units, N, K]
    int64_t w_stride;   // elements between units' weights (0: shared)
    int units, rows_u, n, k;
    // QKV epilogue
    uint16_t *q;        // [units, rows_u, hq, 128]
    uint16_t *ck, *cv;  // [units, hkv, s_cap, 128]
    const int32_t *pos; // [units, rows_u]
    const int32_t *lens;
    int max_len, hq, hkv, s_cap;
    // OUT epilogue
    const uint16_t *res; // [units, rows_u, N]
    uint16_t *out;       // [units, rows_u, N]
};

__device__ inline uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)p; }

// DMA of one 128-row x 64-column tile (rows past `rows` clamp to the last row) into LDS at
// `dst`: 16 instructions of 1 KB, four per wave; lane L of instruction g fills LDS row
// 8 g + L / 8, physical chunk L % 8, which holds logical chunk (L % 8) ^ ((row >> 1) & 7).
// (s_nop: the wait state an LDS DMA needs after the scalar write of M0, its destination)
__device__ inline void dma_tile(const uint16_t *base, int ld, int rows, int k0, uint32_t dst, int wave, int lane)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = 4 * wave + i;
        const int row = 8 * g + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        const int src_row = min(row, rows - 1);
        const uint32_t off = (uint32_t)(((int64_t)src_row * ld + k0 + 8 * c) * 2);
        const uint32_t d = __builtin_amdgcn_readfirstlane(dst + (uint32_t)(g * 1024));
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "s"(d), "v"(off), "s"(base)
                     : "memory", "m0");
    }
}

__device__ inline const uint16_t *uniform(const uint16_t *p)
{
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const uint16_t *>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

template <int EPI>
__global__ void __launch_bounds__(NTHR) gemm_kernel(GemmParams p, RopeTable tab)
{
    // the ring (64 KB), then the fp32 tile (128 rows of 516 bytes)
    __shared__ __align__(16) char lds[TM * (TN * 4 + 4)];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int tiles_m = (p.rows_u + TM - 1) / TM;
    const int tiles_n = p.n / TN;
    // Tile order: layer, then row tile, then column tile (QKV: layer, column tile with the
    // k heads' columns first, whose rotating epilogue takes about twice as long, then row
    // tile).  Workgroups are dealt to
    // the 8 XCDs round-robin, so workgroup b runs on XCD b % 8; when the grid is a multiple
    // of 8, XCD x takes the contiguous range of tiles [x B/8, (x+1) B/8) in order, and the
    // ~64 workgroups it runs at a time share a few A row panels and W column panels in its
    // L2 instead of every XCD fetching every layer's operands.
    int b = blockIdx.x, tn;
    const int nblk = (int)gridDim.x;
    if ((nblk & 7) == 0)
        b = (b & 7) * (nblk >> 3) + (b >> 3);
    int tm, u;
    if (EPI == EPI_QKV) {
        // column tile outside the row tile: the layer's fused weight (6 MB at hidden 1536)
        // outgrows an XCD's L2, so its resident workgroups share fewer weight panels
        tm = b % tiles_m;
        b /= tiles_m;
        const int j = b % tiles_n;
        u = b / tiles_n;
        tn = j < p.hkv ? p.hq + j : (j < p.hkv + p.hq ? j - p.hkv : j);
    } else {
        tn = b % tiles_n;
        b /= tiles_n;
        tm = b % tiles_m;
        u = b / tiles_m;
    }
    const int m0 = tm * TM, n0 = tn * TN;
    const int rows = min(TM, p.rows_u - m0);

    const uint16_t *abase = uniform(p.a + ((int64_t)u * p.rows_u + m0) * p.k);
    const uint16_t *wbase = uniform(p.w + (int64_t)u * p.w_stride + (int64_t)n0 * p.k);
    const uint32_t lds0 = lds_addr(lds);

    // wave (wr, wc) owns rows 64 wr .. + 63 and columns 64 wc .. + 63 of the tile
    const int wr = wave >> 1, wc = wave & 1;
    const int c32 = lane & 31, h = lane >> 5;
    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = floatx16{0.f};

    const int nkt = p.k / TK;
    dma_tile(abase, p.k, rows, 0, lds0, wave, lane);
    dma_tile(wbase, p.k, TN, 0, lds0 + TM * ROW_B, wave, lane);
    for (int kt = 0; kt < nkt; ++kt) {
        const uint32_t st = (uint32_t)((kt & 1) * STAGE_B);
        asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (kt + 1 < nkt) {
            const uint32_t nx = lds0 + (uint32_t)(((kt + 1) & 1) * STAGE_B);
            dma_tile(abase, p.k, rows, (kt + 1) * TK, nx, wave, lane);
            dma_tile(wbase, p.k, TN, (kt + 1) * TK, nx + TM * ROW_B, wave, lane);
        }
        // operands: A rows 64 wr + 32 i + c32, W rows 64 wc + 32 j + c32, K chunk 2 ks + h
        half8 av[4][2], wv[4][2];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ra = 64 * wr + 32 * i + c32;
                const int rw = 64 * wc + 32 * i + c32;
                const int c = 2 * ks + h;
                av[ks][i] = *reinterpret_cast<const half8 *>(lds + st + ra * ROW_B + 16 * (c ^ ((ra >> 1) & 7)));
                wv[ks][i] = *reinterpret_cast<const half8 *>(lds + st + TM * ROW_B + rw * ROW_B +
                                                             16 * (c ^ ((rw >> 1) & 7)));
            }
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[ks][i], wv[ks][j], acc[i][j], 0, 0, 0);
    }

    // ---- epilogue: the fp32 tile through LDS ([128 rows][128 columns], 516-byte rows)
    constexpr int CROW = TN * 4 + 4;
    static_assert(TM * CROW >= 2 * STAGE_B, "the LDS array holds both the ring and the tile");
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float *ct = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                // C block layout: lane holds column c32, rows 8 (r / 4) + 4 h + r % 4
                const int row = 64 * wr + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                const int col = 64 * wc + 32 * j + c32;
                ct[row * (CROW / 4) + col] = acc[i][j][r];
            }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    auto chunk_f16 = [&](int row, int ch, uint16_t (&o)[8]) {
        const float *src = ct + row * (CROW / 4) + 8 * ch;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            o[e] = f2h(src[e]);
    };

    if (EPI == EPI_OUT) {
        for (int it = tid; it < TM * (TN / 8); it += NTHR) {
            const int row = it / (TN / 8), ch = it % (TN / 8);
            if (row >= rows)
                continue;
            const int64_t base = ((int64_t)u * p.rows_u + m0 + row) * p.n + n0 + 8 * ch;
            Chunk16 rin, o;
            rin.v = *reinterpret_cast<const uint4 *>(p.res + base);
            const float *src = ct + row * (CROW / 4) + 8 * ch;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o.h[e] = f2h(src[e] + h2f(rin.h[e]));
            *reinterpret_cast<uint4 *>(p.out + base) = o.v;
        }
        return;
    }

    // QKV: the tile is head hn of the fused [q heads | k heads | v heads] columns
    const int hn = n0 / 128;
    const int len = p.lens ? p.lens[u] : 0;
    const bool cache_ok = len >= 0 && len <= p.max_len;
    if (hn < p.hq) {
        for (int it = tid; it < TM * 16; it += NTHR) {
            const int row = it >> 4, ch = it & 15;
            if (row >= rows)
                continue;
            Chunk16 o;
            chunk_f16(row, ch, o.h);
            reinterpret_cast<uint4 *>(p.q + (((int64_t)u * p.rows_u + m0 + row) * p.hq + hn) * 128)[ch] = o.v;
        }
    } else if (hn < p.hq + p.hkv) {
        if (!cache_ok)
            return;
        const int g = hn - p.hq;
        const int first = tab.off >> 3, h8 = tab.n_pairs >> 3;
        const int set = rope_set(tab, u);
        for (int it = tid; it < TM * 16; it += NTHR) {
            const int row = it >> 4, ch = it & 15;
            if (row >= rows)
                continue;
            const int i = m0 + row;
            uint16_t *dst = p.ck + (((int64_t)u * p.hkv + g) * p.s_cap + len + i) * 128;
            const int pos = p.pos[(int64_t)u * p.rows_u + i];
            Chunk16 a, y;
            chunk_f16(row, ch, a.h);
            if (tab.half) {
                if (ch < first) {
                    reinterpret_cast<uint4 *>(dst)[ch] = a.v;
                } else if (ch < first + h8) {
                    Chunk16 bb, yb;
                    chunk_f16(row, ch + h8, bb.h);
                    rotate_half_chunks(a.h, bb.h, y.h, yb.h, 8 * (ch - first), pos, tab, set);
                    reinterpret_cast<uint4 *>(dst)[ch] = y.v;
                    reinterpret_cast<uint4 *>(dst)[ch + h8] = yb.v;
                }
            } else if (8 * ch + 7 >= tab.off) {
                double cs[4], sn[4];
                chunk_trig(ch, pos, tab, set, cs, sn);
                rotate_chunk_f64(a.h, y.h, ch, cs, sn, tab.off);
                reinterpret_cast<uint4 *>(dst)[ch] = y.v;
            } else {
                reinterpret_cast<uint4 *>(dst)[ch] = a.v;
            }
        }
    } else {
        if (!cache_ok)
            return;
        const int g = hn - p.hq - p.hkv;
        for (int it = tid; it < TM * 16; it += NTHR) {
            const int row = it >> 4, ch = it & 15;
            if (row >= rows)
                continue;
            Chunk16 o;
            chunk_f16(row, ch, o.h);
            reinterpret_cast<uint4 *>(p.cv + (((int64_t)u * p.hkv + g) * p.s_cap + len + m0 + row) * 128)[ch] = o.v;
        }
    }
}

} // namespace

hipError_t launch_qkv_projection(const uint16_t *x, const uint16_t *w, int64_t w_stride, const int32_t *positions,
                                 uint16_t *q, uint16_t *cache_k, uint16_t *cache_v, const int32_t *lens,
                                 int max_len, int n, int t, int hidden, int hq, int hkv, int s_cap,
                                 const RopeTable &tab, hipStream_t stream)
{
    GemmParams p{};
    p.a = x;
    p.w = w;
    p.w_stride = w_stride;
    p.units = n;
    p.rows_u = t;
    p.n = (hq + 2 * hkv) * 128;
    p.k = hidden;
    p.q = q;
    p.ck = cache_k;
    p.cv = cache_v;
    p.pos = positions;
    p.lens = lens;
    p.max_len = max_len;
    p.hq = hq;
    p.hkv = hkv;
    p.s_cap = s_cap;
    const int64_t blocks = (int64_t)n * ((t + TM - 1) / TM) * (p.n / TN);
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL(gemm_kernel<EPI_QKV>, dim3((unsigned)blocks), dim3(NTHR), 0, stream, p, tab);
    return hipGetLastError();
}

hipError_t launch_out_projection(const uint16_t *attn, const uint16_t *w, int64_t w_stride, const uint16_t *residual,
                                 uint16_t *out, int n, int t, int in_features, int hidden, hipStream_t stream)
{
    GemmParams p{};
    p.a = attn;
    p.w = w;
    p.w_stride = w_stride;
    p.units = n;
    p.rows_u = t;
    p.n = hidden;
    p.k = in_features;
    p.res = residual;
    p.out = out;
    const int64_t blocks = (int64_t)n * ((t + TM - 1) / TM) * (hidden / TN);
    if (blocks == 0)
        return hipSuccess;
    RopeTable tab{};
    hipLaunchKernelGGL(gemm_kernel<EPI_OUT>, dim3((unsigned)blocks), dim3(NTHR), 0, stream, p, tab);
    return hipGetLastError();
}

} // namespace kvrope
