// decode.hip -- split-key decode attention with fused rotary embedding and cache append
// (gfx950).
//
// One decode step per unit u (Sophgo MLIR-based LLM compilation paper, sec. 4.1: query
// length 1, keys = every earlier token; Buddy-MLIR walkthrough, sec. 6.4.5-6.4.6: the new
// token sits at position = current cache length):
//   1. q[u] and k[u] are rotated at positions[u] (fp64 factors, rounded once to f16 --
//      "ds4.c study notes", Part 4 sec. 1, Trace 2);
//   2. the rotated k and the raw v are written to cache row lens[u];
//   3. each query head h attends over rows 0 .. lens[u] of KV head h / (hq / hkv)
//      ("02 Prefill integration of CGDR", sec. 1-2: repeat_interleave sharing).
//
// Kernel 1 (decode_attn_kernel): the len + 1 keys of a (unit, KV head) are cut into
// chunks of nearly equal size (at most `target` keys, a multiple of 32); a workgroup of
// 4 waves owns (unit, KV head, up to 32 query heads of the group, chunk), so the chunk is
// read from HBM once for every head of the group.  Each wave takes the chunk's 32-key
// tiles w, w + 4, ...; a tile's K and V rows go from HBM straight into the wave's LDS
// stage (global_load_lds_dwordx4: 1 KB contiguous per instruction, no registers), the
// next tile's load in flight while the current one is computed:
//   * S^T (32 keys x 32 heads) = K . Q^T on v_mfma_f32_32x32x16_f16, the heads' rotated
//     q (rounded to f16, exactly the unfused rotation's q) as the B operand, columns past
//     the group zero; scores scaled by scale * log2(e) in fp32;
//   * online softmax in fp32 per head (log2 domain);
//   * O^T (128 dims x 32 heads) += V^T . P^T on the same MFMA, V^T read from LDS with
//     transposing reads (ds_read_b64_tr_b16), P^T straight from the softmax registers.
// The four waves' (max, sum, output) states are merged through LDS into one fp32 partial
// per (unit, head, chunk) in the caller's workspace.
// Kernel 2 (decode_combine_kernel): per (unit, head), merges the chunks in index order
// (M = max m_s, L = sum l_s 2^(m_s - M), O = sum o_s 2^(m_s - M) / L), so results are
// deterministic.  No float atomics anywhere.
#include "device_common.h"
#include "launch.h"
#include "rope_device.h"

#include <math.h>

#include <algorithm>
#include <type_traits>

namespace kvrope {

namespace {

constexpr int KT = 32;              // keys per tile
constexpr int NWAVES = 4;
constexpr int NT = NWAVES * 64;
constexpr int ROWB = kHeadDim * 2;  // bytes per K / V row
constexpr int TILE_B = KT * ROWB;   // 8 KB per tensor per tile
constexpr int STAGE_B = 2 * TILE_B; // K then V
constexpr int PART = kHeadDim + 2;  // floats per partial: m, l, o[128]
constexpr int MAXG = 32;            // query heads per workgroup (the MFMA's columns)
constexpr int kAssumedCUs = 256;    // MI355X compute units (chunk heuristic only)

struct DecodeParams {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    const int32_t *pos;
    const int32_t *lens;
    uint16_t *ck;
    uint16_t *cv;
    float *ws;      // partials [n, hq, nsplit, PART]
    int n, hq, hkv, G, s_cap, max_len;
    int target;  // keys per chunk at most (multiple of 32)
    int nsplit;  // chunk slots per (unit, KV head): chunks of a unit with max_len + 1 keys
    int slices;  // ceil(G / 32)
    float scale_log2;
};

// The chunks of a unit with nk keys: as few as `target` allows, of equal size rounded up
// to whole tiles (the last one shorter).
__host__ __device__ inline void unit_chunks(int nk, int target, int &chunk, int &ns)
{
    const int want = (nk + target - 1) / target;
    chunk = ((nk + want - 1) / want + KT - 1) / KT * KT;
    ns = (nk + chunk - 1) / chunk;
}

// LDS row swizzles (16-byte chunk index xor): K rows so the S^T operand reads (16 B of
// 32 consecutive keys) hit distinct banks; V rows so the four rows one transposing read
// covers per lane half sit on distinct banks.
__device__ inline int kswz(int key) { return key & 15; }
__device__ inline int vswz(int key) { return 4 * (key & 3); }

typedef short short4v __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 at LDS byte offset `off`: within each 16-lane group, lane i receives
// 16-bit element i % 4 of the 8 bytes that lane 4 j + i / 4 addresses, as its element j.
__device__ inline u32x2 lds_read_tr16(const char *lds, uint32_t off)
{
    const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4v *)(lds + off));
    return __builtin_bit_cast(u32x2, v);
}

__device__ inline uint32_t lds_offset(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

__device__ inline const char *uniform_ptr(const char *ptr)
{
    const uint64_t x = (uint64_t)(uintptr_t)ptr;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return (const char *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Rows of one 32-row tile of a cache (starting at the wave-uniform `rows`) into the LDS
// region at `dst`: 8 instructions of 4 rows (1 KB) each; lane L takes row 4 i + L / 16 and
// the global chunk that lands in LDS chunk L % 16 of that row (off: the per-lane byte
// offsets, rows clamped to the last valid one).  Not tracked by the compiler: waited for
// with an explicit vmcnt.  The s_nop: the wait state an LDS DMA needs after the scalar
// write of M0 that gives its destination.
__device__ inline void dma_tile(const char *rows, const uint32_t (&off)[8], uint32_t dst)
{
    const char *t = uniform_ptr(rows);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t d = __builtin_amdgcn_readfirstlane(dst + (uint32_t)(4 * i * ROWB));
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "s"(d), "v"(off[i]), "s"(t)
                     : "memory", "m0");
    }
}

// per-lane source offsets of a tile whose valid rows are 0 .. last (rows past it repeat it)
template <bool V>
__device__ inline void tile_offsets(int lane, int last, uint32_t (&off)[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 4 * i + (lane >> 4);
        const int sw = V ? vswz(row) : kswz(row);
        off[i] = (uint32_t)(min(row, last) * ROWB + (((lane & 15) ^ sw) << 4));
    }
}

// Per-lane base (within a stage's V region) of the V^T operand reads.  For key step x and
// dim block db the lane's two transposing reads (keys 16 x + 4 hh + 0..3, then + 8..11)
// sit at (base ^ 64 db) + 4 KB x (+ 2 KB): in its 16-lane group (gq = lane / 16; gq % 2
// picks which 16 dims of the block), lane 4 j + r addresses key row 16 x + 4 hh + j, dims
// 32 db + 16 (gq % 2) + 4 r .. + 3, i.e. chunk 4 db + 2 (gq % 2) + r / 2 swizzled to
// 4 (db ^ j) + 2 (gq % 2) + r / 2.
__device__ inline uint32_t vt_base(int lane)
{
    const int hh = lane >> 5, j = (lane >> 2) & 3, r = lane & 3;
    return (uint32_t)((4 * hh + j) * ROWB + 64 * j + 32 * ((lane >> 4) & 1) + 8 * r);
}

__device__ inline half8 read_vt(const char *lds, uint32_t vb, uint32_t vstage, int x, int db)
{
    const uint32_t a = (vb ^ (uint32_t)(64 * db)) + vstage + (uint32_t)(x * 16 * ROWB);
    const u32x2 lo = lds_read_tr16(lds, a), hi = lds_read_tr16(lds, a + 8 * ROWB);
    return __builtin_bit_cast(half8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// NS: LDS stages per wave (each a 32-key K and V tile); HALF: half-split pairing of q's
// rotated dims (one kernel per pairing keeps the other's code out of the register
// allocation)
template <int NS, bool HALF>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) decode_attn_kernel(DecodeParams p, RopeTable tab)
{
    constexpr int RING_B = NWAVES * NS * STAGE_B;
    __shared__ __align__(16) char lds[RING_B];
    __shared__ __align__(16) float fct[NWAVES][2][kMaxPairs]; // per wave: cos, sin of pair j
    __shared__ float wm[NWAVES][MAXG];
    __shared__ float wl[NWAVES][MAXG];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane & 31;
    const int hh = lane >> 5;

    // block -> (unit, KV head, slice, split); split is the fastest index
    int b = blockIdx.x;
    const int split = b % p.nsplit;
    b /= p.nsplit;
    const int sl = b % p.slices;
    b /= p.slices;
    const int g = b % p.hkv;
    const int u = b / p.hkv;
    const int h0 = g * p.G + sl * MAXG; // first query head of this slice
    const int nh = min(MAXG, p.G - sl * MAXG);

    // the unit's scalars first, before any store or untracked load (so they stay scalar
    // loads and no wait for them waits for the tiles)
    const int len = p.lens[u];
    const int posi = p.pos[u];
    const int rs = rope_set(tab, u);
    if (len < 0 || len > p.max_len)
        return; // no cache write for this unit; the combine kernel emits NaN
    const int nk = len + 1;
    int chunk, ns;
    unit_chunks(nk, p.target, chunk, ns);
    if (split >= ns)
        return; // no such chunk for this unit's length
    const int k0 = split * chunk;
    const int k1 = min(k0 + chunk, nk);
    const int ntiles = (k1 - k0 + KT - 1) / KT;
    const bool has_new = len >= k0 && len < k1;
    // this lane's rotated pair's rate (revolutions per position), read early
    const double wrev_l = (rs >= 0 && lane < tab.n_pairs && !tab.cos_t) ? tab.wrev[rs][lane] : 0.0;

    // The wave that owns the tile holding key len rotates the new k and appends it (with
    // v) when it reaches that tile: lane `it` takes pair slot it of the head, rotated pair
    // j = it - off/2 when it >= off/2 with dims (off + 2j, off + 2j + 1) or, half-split,
    // (off + j, off + j + n_pairs); below off/2 the dims (2 it, 2 it + 1) are copied.
    const int t_new = has_new ? (len - k0) / KT : -1;
    const bool new_here = has_new && (t_new % NWAVES) == wave;
    int nda = 0, ndb = 0, nj = -1;
    uint16_t ka = 0, kb_ = 0, va = 0, vb_ = 0;

    // ---- the loads the prologue needs, first: the lane's q dims 16 s + 8 hh .. + 7 of head
    // column c (c < nh), and the new k / v of the owning wave
    u32x4 qin[8];
    {
        const uint16_t *qr = p.q + ((int64_t)u * p.hq + h0 + min(c, nh - 1)) * kHeadDim + 8 * hh;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8)
            qin[s8] = ld16(qr + 16 * s8);
    }
    if (new_here) {
        nj = lane - (tab.off >> 1);
        if (nj < 0) {
            nda = 2 * lane;
            ndb = nda + 1;
        } else {
            nda = tab.half ? tab.off + nj : tab.off + 2 * nj;
            ndb = tab.half ? nda + tab.n_pairs : nda + 1;
        }
        const uint16_t *kr = p.k + ((int64_t)u * p.hkv + g) * kHeadDim;
        const uint16_t *vr = p.v + ((int64_t)u * p.hkv + g) * kHeadDim;
        ka = kr[nda];
        kb_ = kr[ndb];
        va = vr[nda];
        vb_ = vr[ndb];
    }

    // ---- then the first tiles, whose latency the rest of the prologue runs under
    const char *kslab = reinterpret_cast<const char *>(p.ck + ((int64_t)u * p.hkv + g) * p.s_cap * kHeadDim);
    const char *vslab = reinterpret_cast<const char *>(p.cv + ((int64_t)u * p.hkv + g) * p.s_cap * kHeadDim);
    const uint32_t lds0 = lds_offset(lds);
    const uint32_t my_stage0 = (uint32_t)(wave * NS * STAGE_B);

    // tile t of the chunk (t = wave + 4 i) into stage i % NS of this wave
    // (K and V separately: with one stage per wave, the next tile's K goes out once the
    // S^T product has read this tile's K, and its V once the PV product has read this V)
    auto issue_t = [&](auto v_c, int i) {
        constexpr bool ISV = decltype(v_c)::value;
        const int t = wave + NWAVES * i;
        const int kb = k0 + KT * t;
        const int last = min(KT, k1 - kb) - 1;
        uint32_t of[8];
        tile_offsets<ISV>(lane, last, of);
        const uint32_t st = lds0 + my_stage0 + (uint32_t)((i % NS) * STAGE_B) + (ISV ? TILE_B : 0u);
        dma_tile((ISV ? vslab : kslab) + (int64_t)kb * ROWB, of, st);
    };
    auto issue = [&](int i) {
        issue_t(std::false_type{}, i);
        issue_t(std::true_type{}, i);
    };
    const int my_tiles = wave < ntiles ? (ntiles - wave + NWAVES - 1) / NWAVES : 0;
#pragma unroll
    for (int i = 0; i < NS; ++i)
        if (i < my_tiles)
            issue(i);

    // ---- the new row (owning wave only; lane = pair slot): k rotated in fp64 and rounded
    // once, written with v to cache row len
    uint32_t kyy = 0;
    if (new_here) {
        uint16_t y0 = ka, y1 = kb_;
        if (nj >= 0) {
#pragma clang fp contract(off)
            double co, sv;
            pair_factor(nj, posi, tab, rs, co, sv);
            const double x0 = h2d(ka), x1 = h2d(kb_);
            y0 = f64_to_f16_rne(x0 * co - x1 * sv);
            y1 = f64_to_f16_rne(x0 * sv + x1 * co);
        }
        kyy = (uint32_t)y0 | ((uint32_t)y1 << 16);
        if (sl == 0) {
            const int64_t row = (((int64_t)u * p.hkv + g) * p.s_cap + len) * kHeadDim;
            p.ck[row + nda] = y0;
            p.ck[row + ndb] = y1;
            p.cv[row + nda] = va;
            p.cv[row + ndb] = vb_;
        }
    }

    // ---- q rotation, per wave (no barrier): lane j computes rotated pair j's factors in
    // fp32 (hardware sin / cos of the angle in turns, reduced in fp64), times mscale, the
    // sine times the rotation's sign; or the caller's table entries (NaN outside the table
    // or for an invalid parameter set).  Every lane then rotates its own q dims in fp32 and
    // rounds them to f16: q_hat up to one f16 ulp where the fp32 value sits next to a
    // rounding boundary.
    if (lane < tab.n_pairs) {
        float fc, fs;
        if (rs < 0) {
            fc = fs = __builtin_nanf("");
        } else if (tab.cos_t) {
            const bool in = posi >= 0 && posi < tab.rows;
            fc = in ? tab.cos_t[(int64_t)posi * tab.n_pairs + lane] : __builtin_nanf("");
            fs = in ? tab.sin_t[(int64_t)posi * tab.n_pairs + lane] * (float)tab.sgn : __builtin_nanf("");
        } else {
            const float rf = (float)__builtin_amdgcn_fract((double)posi * wrev_l);
            const float m = (float)tab.mscale[rs];
            fc = __builtin_amdgcn_cosf(rf) * m;
            fs = __builtin_amdgcn_sinf(rf) * m * (float)tab.sgn;
        }
        fct[wave][0][lane] = fc;
        fct[wave][1][lane] = fs;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    half8 qop[8];
    {
        const float *fcw = fct[wave][0], *fsw = fct[wave][1];
        const int off = tab.off;
        if (!HALF) {
            // adjacent pairs: word m of block s holds dims 16 s + 8 hh + 2 m, + 1
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8) {
                u32x4 hv;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int d0 = 16 * s8 + 8 * hh + 2 * m;
                    const uint32_t w = qin[s8][m];
                    if (d0 >= off) {
                        const int jj = (d0 - off) >> 1;
                        const float x0 = lo2f(w), x1 = hi2f(w), cc = fcw[jj], ss = fsw[jj];
                        hv[m] = pack2h(x0 * cc - x1 * ss, x0 * ss + x1 * cc);
                    } else {
                        hv[m] = w;
                    }
                }
                qop[s8] = __builtin_bit_cast(half8, hv);
            }
        } else {
            // half-split pairs (n_pairs a multiple of 16): dim d of block s pairs with dim
            // d + n_pairs of block s + n_pairs / 16, in the same lane
            const int h16 = tab.n_pairs >> 4;
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8)
                qop[s8] = __builtin_bit_cast(half8, qin[s8]);
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8) {
                const int d0 = 16 * s8 + 8 * hh;
                if (d0 >= off && d0 < off + tab.n_pairs) {
                    u32x4 ya, yb;
                    u32x4 a = qin[s8], bq = qin[s8];
#pragma unroll
                    for (int s2 = 0; s2 < 8; ++s2)
                        if (s2 == s8 + h16)
                            bq = qin[s2];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int jj = d0 + 2 * m - off;
                        const float a0 = lo2f(a[m]), a1 = hi2f(a[m]), b0 = lo2f(bq[m]), b1 = hi2f(bq[m]);
                        const float c0 = fcw[jj], s0 = fsw[jj], c1 = fcw[jj + 1], s1 = fsw[jj + 1];
                        ya[m] = pack2h(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
                        yb[m] = pack2h(a0 * s0 + b0 * c0, a1 * s1 + b1 * c1);
                    }
                    qop[s8] = __builtin_bit_cast(half8, ya);
#pragma unroll
                    for (int s2 = 0; s2 < 8; ++s2)
                        if (s2 == s8 + h16)
                            qop[s2] = __builtin_bit_cast(half8, yb);
                }
            }
        }
        if (c >= nh) {
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8)
                qop[s8] = half8{0};
        }
    }

    const uint32_t kb0 = (uint32_t)(c * ROWB + ((hh ^ kswz(c)) << 4)); // K operand, step 0
    const uint32_t vb0 = vt_base(lane);

    float m_run = -INFINITY, l_run = 0.f; // per query column c (lane halves share m)
    floatx16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
        o[db] = floatx16{0.f};

    for (int i = 0; i < my_tiles; ++i) {
        const int t = wave + NWAVES * i;
        const int kb = k0 + KT * t;
        const uint32_t st = my_stage0 + (uint32_t)((i % NS) * STAGE_B);
        // this tile's K: with more stages, done once at most the next tile's 16 loads are
        // outstanding; with one, once at most this tile's 8 V loads are (loads complete in
        // order, and K went out first)
        if (i + 1 < my_tiles && NS > 1)
            asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else if (NS == 1 && !(new_here && t == t_new))
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (new_here && t == t_new) {
            // The new row goes into this tile, whose copy of that row may predate it.  The
            // rows after it (copies of that stale row, masked) must hold finite V: a masked
            // key's zero probability times a NaN would still be NaN.
            const int r = len - kb;
            const uint16_t y0 = (uint16_t)(kyy & 0xffffu), y1 = (uint16_t)(kyy >> 16);
            // dim d of row r sits at byte 2 (d % 8) of chunk (d / 8) ^ swizzle(r)
            char *krow_l = lds + st + r * ROWB;
            char *vrow_l = lds + st + TILE_B + r * ROWB;
            auto at = [&](char *rowp, int d, int sw) {
                return reinterpret_cast<uint16_t *>(rowp + ((((d >> 3) ^ sw) << 4) | ((d & 7) << 1)));
            };
            *at(krow_l, nda, kswz(r)) = y0;
            *at(krow_l, ndb, kswz(r)) = y1;
            *at(vrow_l, nda, vswz(r)) = va;
            *at(vrow_l, ndb, vswz(r)) = vb_;
            for (int idx = lane; idx < (KT - 1 - r) * 16; idx += 64)
                *reinterpret_cast<u32x4 *>(lds + st + TILE_B + (r + 1) * ROWB + 16 * idx) = u32x4{0u, 0u, 0u, 0u};
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        // S^T = K . Q^T (32 keys x 32 heads)
        floatx16 sacc = floatx16{0.f};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const half8 a = *reinterpret_cast<const half8 *>(lds + st + (kb0 ^ (uint32_t)(s << 5)));
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qop[s], sacc, 0, 0, 0);
        }
        if (NS == 1 && i + 1 < my_tiles) {
            // the K stage is free once the S^T operand reads returned
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            issue_t(std::false_type{}, i + 1);
        }
        // lane holds keys kb + 8 (r / 4) + 4 hh + r % 4 of head column c
        const int lim = k1 - kb - 4 * hh; // keys at or past k1 are masked
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float sv = sacc[r] * p.scale_log2;
            if (8 * (r >> 2) + (r & 3) >= lim)
                sv = -INFINITY;
            sacc[r] = sv;
            mx = fmaxf(mx, sv);
        }
        mx = half_max(mx);
        const float m_new = fmaxf(m_run, mx); // finite: the tile's first key is valid
        if (__builtin_amdgcn_ballot_w64(m_new != m_run) != 0) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
                o[db] *= alpha;
            m_run = m_new;
        }
        u32x4 pw[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 8 * x + 2 * jj;
                const floatx2 pf = {__builtin_amdgcn_exp2f(sacc[r] - m_run), __builtin_amdgcn_exp2f(sacc[r + 1] - m_run)};
                l_run += pf[0] + pf[1];
                pw[x][jj] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pf, half2v));
            }
        }
        // this tile's V: with one stage, at most the next tile's 8 K loads may be outstanding
        if (NS == 1) {
            if (i + 1 < my_tiles)
                asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            else
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        // O^T += V^T . P^T
#pragma unroll
        for (int x = 0; x < 2; ++x) {
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const half8 a = read_vt(lds, vb0, st + TILE_B, x, db);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(half8, pw[x]), o[db], 0, 0, 0);
            }
        }
        // the stage is free once its operand reads returned (the MFMAs above consumed them)
        if (i + NS < my_tiles) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (NS == 1)
                issue_t(std::true_type{}, i + 1);
            else
                issue(i + NS);
        }
    }

    // ---- merge the four waves' states through LDS (the ring is idle now); a wave without
    // keys has m = -inf, l = 0, o = 0
    __syncthreads();
    const float l_tot = half_sum(l_run);
    if (c < nh && hh == 0) {
        wm[wave][c] = m_run;
        wl[wave][c] = l_tot;
    }
    float *wo = reinterpret_cast<float *>(lds); // [wave][head column][dim]
    if (c < nh) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int d = 32 * db + 8 * (r >> 2) + 4 * hh + (r & 3);
                wo[(wave * MAXG + c) * kHeadDim + d] = o[db][r];
            }
        }
    }
    __syncthreads();
    for (int it = tid; it < nh * kHeadDim; it += NT) {
        const int hl = it / kHeadDim, d = it % kHeadDim;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w)
            M = fmaxf(M, wm[w][hl]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) {
            const float f = (wm[w][hl] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(wm[w][hl] - M);
            L += wl[w][hl] * f;
            O += wo[(w * MAXG + hl) * kHeadDim + d] * f;
        }
        float *part = p.ws + (((int64_t)u * p.hq + h0 + hl) * p.nsplit + split) * PART;
        part[2 + d] = O;
        if (d == 0) {
            part[0] = M;
            part[1] = L;
        }
    }
}

// Merge the chunks of each (unit, head) in index order; one wave per (unit, head): lane s
// holds chunk s's max and sum (64 chunks per pass), every lane two output dims.  The
// output slices are read 8 chunks at a time, the first 8 together with the maxima, so a
// unit with at most 8 chunks costs one round trip to memory.
__global__ void __launch_bounds__(256) decode_combine_kernel(const float *__restrict__ ws,
                                                             const int32_t *__restrict__ lens,
                                                             uint16_t *__restrict__ out, int n, int hq,
                                                             int nsplit, int target, int max_len)
{
    constexpr int B = 8;
    const int wid = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
    const int lane = threadIdx.x & 63;
    if (wid >= n * hq)
        return;
    const int u = wid / hq;
    const int len = lens[u];
    uint16_t *orow = out + (int64_t)wid * kHeadDim;
    if (len < 0 || len > max_len) {
        orow[2 * lane] = qnan16();
        orow[2 * lane + 1] = qnan16();
        return;
    }
    int chunk, ns;
    unit_chunks(len + 1, target, chunk, ns);
    const float *part = ws + (int64_t)wid * nsplit * PART;
    floatx2 ob[B];
#pragma unroll
    for (int s = 0; s < B; ++s)
        ob[s] = s < ns ? *reinterpret_cast<const floatx2 *>(part + s * PART + 2 + 2 * lane) : floatx2{0.f, 0.f};
    float M = -INFINITY;
    for (int s0 = 0; s0 < ns; s0 += 64) {
        const float ms = (s0 + lane < ns) ? part[(s0 + lane) * PART] : -INFINITY;
        M = fmaxf(M, ms);
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1)
        M = fmaxf(M, __shfl_xor(M, sh, 64));
    float L = 0.f, O0 = 0.f, O1 = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 64) {
        const int cnt = min(64, ns - s0);
        const float ms = (lane < cnt) ? part[(s0 + lane) * PART] : -INFINITY;
        const float ls = (lane < cnt) ? part[(s0 + lane) * PART + 1] : 0.f;
        const float f = (lane < cnt) ? __builtin_amdgcn_exp2f(ms - M) : 0.f;
        float lf = ls * f;
#pragma unroll
        for (int sh = 32; sh >= 1; sh >>= 1)
            lf += __shfl_xor(lf, sh, 64);
        L += lf;
        for (int sb = 0; sb < cnt; sb += B) {
            // the block's output slices: the preloaded first block, later blocks loaded
            // together before they are used
            if (s0 + sb > 0) {
#pragma unroll
                for (int b = 0; b < B; ++b)
                    ob[b] = sb + b < cnt ? *reinterpret_cast<const floatx2 *>(part + (s0 + sb + b) * PART + 2 + 2 * lane)
                                         : floatx2{0.f, 0.f};
            }
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float fs = __shfl(f, sb + b, 64); // 0 past cnt
                O0 += ob[b][0] * fs;
                O1 += ob[b][1] * fs;
            }
        }
    }
    const float inv = 1.f / L;
    orow[2 * lane] = f2h(O0 * inv);
    orow[2 * lane + 1] = f2h(O1 * inv);
}

// Largest chunk, in keys, a workgroup takes: about two chunks' worth of workgroups per
// compute unit for the longest possible caches, between 256 and 1024 keys (below 256, two
// tiles a wave, the per-workgroup fixed work outweighs the extra parallelism: 28 layers
// of one sequence with rows to 1024, 128-key chunks 15.1 us, 256-key 13.9 us, 384-key
// 14.9 us per launch).
int decode_target(int n, int hkv, int slices, int max_len)
{
    const int64_t keys = (int64_t)n * hkv * slices * (max_len + 1);
    int64_t t = keys / (2 * kAssumedCUs);
    t = (t + KT - 1) / KT * KT;
    return (int)std::min<int64_t>(1024, std::max<int64_t>(256, t));
}

} // namespace

int decode_chunk_keys(int n, int hq, int hkv, int max_len)
{
    const int slices = (hq / hkv + MAXG - 1) / MAXG;
    return decode_target(n, hkv, slices, max_len);
}

size_t decode_workspace_bytes(int n, int hq, int hkv, int max_len)
{
    const int G = hq / hkv;
    const int slices = (G + MAXG - 1) / MAXG;
    const int target = decode_target(n, hkv, slices, max_len);
    const int nsplit = (max_len + 1 + target - 1) / target;
    return (size_t)n * hq * nsplit * PART * sizeof(float);
}

hipError_t launch_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const int32_t *positions, uint16_t *cache_k, uint16_t *cache_v,
                         const int32_t *lens, uint16_t *out, const DecodeShape &s,
                         const RopeTable &tab, void *workspace, hipStream_t stream,
                         hipEvent_t ev_before, hipEvent_t ev_after)
{
    if (s.n == 0)
        return hipSuccess;
    DecodeParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.pos = positions;
    p.lens = lens;
    p.ck = cache_k;
    p.cv = cache_v;
    p.ws = reinterpret_cast<float *>(workspace);
    p.n = s.n;
    p.hq = s.hq;
    p.hkv = s.hkv;
    p.G = s.hq / s.hkv;
    p.s_cap = s.s_cap;
    p.max_len = s.max_len;
    p.slices = (p.G + MAXG - 1) / MAXG;
    p.target = decode_target(s.n, s.hkv, p.slices, s.max_len);
    p.nsplit = (s.max_len + 1 + p.target - 1) / p.target;
    p.scale_log2 = (float)((double)s.scale * 1.4426950408889634);
    const int64_t blocks = (int64_t)s.n * s.hkv * p.slices * p.nsplit;

    if (ev_before)
        (void)hipEventRecord(ev_before, stream);
    if (tab.half)
        hipLaunchKernelGGL((decode_attn_kernel<1, true>), dim3((unsigned)blocks), dim3(NT), 0, stream, p, tab);
    else
        hipLaunchKernelGGL((decode_attn_kernel<1, false>), dim3((unsigned)blocks), dim3(NT), 0, stream, p, tab);
    hipError_t err = hipGetLastError();
    if (ev_after)
        (void)hipEventRecord(ev_after, stream);
    if (err != hipSuccess)
        return err;
    const int64_t waves = (int64_t)s.n * s.hq;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)((waves * 64 + 255) / 256)), dim3(256), 0,
                       stream, p.ws, lens, out, s.n, s.hq, p.nsplit, p.target, s.max_len);
    return hipGetLastError();
}

} // namespace kvrope
