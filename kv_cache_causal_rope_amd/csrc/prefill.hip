// prefill.hip -- causal grouped-query flash attention for prefill / prefill_kv (gfx950).
//
// Computes, for new token i of unit u and query head h (Sophgo MLIR-based LLM
// compilation paper, sec. 2.2 FAttention = scaled dot product + causal mask; sec. 3.1
// Listing 2: keys are the concatenation [history; new]):
//     out[u, i, h] = softmax_j(scale * <q_hat[u, i, h], K[u, g, j]>) V[u, g, j],
//     j = 0 .. hist[u] + i,   g = h / (hq / hkv)
// (KV-head sharing as repeat_interleave: "02 Prefill integration of CGDR", sec. 1-2).
// The caches already hold the new rows (rope_append_kernel ran first).  q is rotated
// in the prologue ("ds4.c study notes", Part 4 sec. 1, Trace 2) and rounded to f16.
//
// Work decomposition.  For one (unit, KV head) the work items are (block of 32 new
// tokens, query head of the group), numbered token-block-major.  A workgroup of 8 waves
// takes a work unit of 8 consecutive items (one per wave), so it spans few adjacent
// token blocks and shares every K/V tile it stages in LDS among 8 x 32 query rows.  Per
// 64-key tile a wave issues 32 MFMAs (v_mfma_f32_32x32x16_f16):
//   S^T (64 keys x 32 queries) = K . Q^T        -- 2 key blocks x 8 head-dim steps
//   O^T (128 dims x 32 queries) += V^T . P^T    -- 2 key blocks x 2 key steps x 4 dim blocks
// Working on S^T puts one query in each lane (lane l: query l % 32, half l / 32), so the
// probabilities come out of the softmax already in the B-operand layout of the PV
// product (the key order inside each 16-key step is permuted consistently on both
// operands, which the reduction allows).
//
// Softmax: fp32, log2 domain.  q is rotated and rounded to f16 unscaled (the f16 tensor a
// rotation hands to attention).  The score accumulators start at -m (m = the row's reference
// max of the plain dot products), so S^T leaves the matrix core as (s - m), and each
// probability is 2^((s - m) * scale * log2(e)): one multiply and one exp2.  m is set exactly
// from a row's first tile and is otherwise left alone: the probabilities are rounded to f16
// for the PV product, so they may grow up to the f16 range (relative precision is the same
// at any magnitude) before anything must move.
// A tile whose probabilities overflow f16 -- seen as an infinite row sum -- takes the
// exact path: m moves to the tile's max, O and the running sum are rescaled and the
// tile's probabilities are recomputed.  So the common tile costs no max reduction.
//
// Two wave groups in ping-pong: waves 0-3 (one per SIMD) and waves 4-7 run the same
// phase sequence, the second one phase behind, so while one wave of a SIMD runs its 32
// MFMAs the other runs its softmax on the vector ALU.  Every phase ends in a workgroup
// barrier.  Per MFMA phase the operand reads (16 bytes per lane, one per MFMA) run eight
// ahead of the MFMAs across the PV -> QK boundary.
//
// LDS: a four-stage ring of (K tile, V tile), 16 KB each.  The K regions of all stages
// sit in the first 64 KB and the V regions in the second, so every operand read uses an
// immediate offset from one per-lane base.
//   K tile: row-major [64 keys][256 B], 16-byte chunk index xor-swizzled by the row
//           (chunk ^ (key & 15)) so the S^T A-operand reads (16 B of 32 consecutive keys)
//           hit distinct banks.  It goes from HBM/L2 straight into LDS
//           (global_load_lds_dwordx4: lane L of a wave's load lands at byte 16 L of a
//           1 KB block; the swizzle picks which global chunk each lane fetches).
//   V tile: row-major like K, loaded the same way (HBM/L2 straight into LDS), chunk
//           index xor-swizzled by 4 (key % 4).  The PV A-operand (8 keys of one dim per
//           lane) comes out of two transposing reads (ds_read_b64_tr_b16, 4 keys each), so
//           V never passes through registers and the softmax phase issues no LDS stores.
// Tile loads use a wave-uniform tile base address plus per-lane 32-bit offsets fixed for
// the whole kernel; only a workgroup's last, partial tile clamps rows to the last key.
// Persistent grid: one workgroup per compute unit loops over the work units (8 items
// each), heavier (later) units first, in a snake order that evens out the rounds and
// keeps every unit of a (unit, KV head) pair on one XCD when the counts allow it.  A
// workgroup's next unit starts while the previous one's output stores drain, with no
// workgroup launch in between.  Outputs leave through LDS so that each global store
// writes whole 256-byte rows.
#include "device_common.h"
#include "launch.h"

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

namespace kvrope {

namespace {

constexpr int KT = 64;                 // keys per tile
constexpr int QB = 32;                 // query tokens per wave
constexpr int ROWB = kHeadDim * 2;     // bytes per K / V row
constexpr int TILE_B = KT * ROWB;      // 16 KB per tensor per stage

// The two workgroup layouts:
//   PP (ping-pong): 8 waves in two groups a phase apart, a 4-stage ring, one workgroup per
//       compute unit -- for long units (history at least as long as the new tokens);
//   !PP: 4 waves in lock-step, a 2-stage ring, two workgroups per compute unit whose waves
//       share the SIMDs -- for short units, whose prologue and epilogue the other
//       workgroup's tile loop then covers.
template <bool PP> struct Lay {
    static constexpr int NW = PP ? 8 : 4;          // waves per workgroup
    static constexpr int NT = NW * 64;             // threads per workgroup
    static constexpr int NSTAGE = PP ? 4 : 2;      // LDS stages, a K and a V tile each
    static constexpr int VREG_B = NSTAGE * TILE_B; // V regions start after the K regions
    static constexpr int ROWS = KT / NW;           // rows of a tile one wave moves
    static constexpr int NDMA = ROWS / 4;          // DMA instructions per wave and tile
};
constexpr int RD = 6;                  // operand reads in flight ahead of the MFMAs

// How q is rotated beyond the per-slot angle rates and scales kept in LDS.  Slot dp of a
// head is the dim pair (2 dp, 2 dp + 1) below off / 2; from off / 2 on it is rotated pair
// j = dp - off / 2, whose dims are (off + 2 j, off + 2 j + 1), or, half-split,
// (off + j, off + j + n_pairs).
struct QRot {
    const float *cos_t; // caller tables [rows][n_pairs] (NULL: computed angles)
    const float *sin_t;
    int rows;
    int n_pairs;
    int off2; // off / 2: the first rotated slot
    int h16;  // half-split: n_pairs / 16 (1 .. 4); 0: adjacent pairs
    float sgn; // sign of the sine (-1: inverse rotation)
};

struct PrefillParams {
    const uint16_t *q;
    const uint16_t *ck;
    const uint16_t *cv;
    const int32_t *pos;
    const int32_t *lens;
    const int32_t *new_lens; // new tokens per unit (NULL: t each); rows past it are padding
    uint16_t *out;
    int n, t, hq, hkv, s_cap, max_hist;
    int G;       // query heads per KV head
    int items;   // tblocks * G work items per (unit, KV head)
    int wpk;     // work units per (unit, KV head) = ceil(items / 8)
    int units;   // work units in all: n * hkv * wpk
    int xcd;     // grid size is a multiple of 8 (XCD-preserving snake order)
    int pairmajor; // XCD-local, pair-major unit order (KV pairs a multiple of 8; see the kernel)
    float scale_log2; // scale * log2(e), applied to the fp32 scores
};

// Workgroup barrier without the release fence of __syncthreads (which would drain every
// outstanding global load, including tiles prefetched for later phases).  LDS reads and
// writes complete before it (lgkmcnt); tile loads into LDS are waited for explicitly
// with vmcnt; the memory clobber keeps the compiler from moving memory ops across it.
__device__ inline void wg_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The barrier that ends a softmax phase: its LDS stores must be complete, but the RD
// operand reads it issued last (for the next MFMA phase) may stay in flight.  LDS
// operations of a wave complete in order, so at most RD outstanding means every store
// (issued before the reads) is done.
template <int N>
__device__ inline void wg_barrier_reads_in_flight()
{
    asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" : : "i"(N) : "memory");
}

__device__ inline int kswz(int key) { return key & 15; }
// V rows: 16-byte chunk index xor 4 (key % 4), so the four rows one transposing read
// covers per lane half sit on distinct banks
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

// Per-lane byte offsets of the K rows a lane moves into LDS: wave w moves rows
// ROWS w .. ROWS (w + 1) - 1, 4 rows per instruction, lane L taking row 4i + L/16 of its
// group and the global chunk that lands in LDS chunk L % 16 of that row.
template <bool PP>
__device__ inline int krow(int wave, int lane, int i) { return Lay<PP>::ROWS * wave + 4 * i + (lane >> 4); }
__device__ inline uint32_t koffset(int row, int lane)
{
    return (uint32_t)(row * ROWB + (((lane & 15) ^ kswz(row)) << 4));
}

// Per-lane base of the V^T operand reads (stage 0).  For key step x and dim block db the
// lane's two transposing reads (keys 16 x + 4 hh + 0..3, then + 8..11) sit at
// (base ^ 64 db) + 4 KB x (+ 2 KB): in its 16-lane group (gq = lane / 16; gq % 2 picks
// which 16 dims of the block), lane 4 j + r addresses key row 16 x + 4 hh + j, dims
// 32 db + 16 (gq % 2) + 4 r .. + 3, i.e. chunk 4 db + 2 (gq % 2) + r / 2 swizzled to
// 4 (db ^ j) + 2 (gq % 2) + r / 2.
template <bool PP>
__device__ inline uint32_t vt_base(int lane)
{
    const int hh = lane >> 5, j = (lane >> 2) & 3, r = lane & 3;
    return (uint32_t)(Lay<PP>::VREG_B + (4 * hh + j) * ROWB + 64 * j + 32 * ((lane >> 4) & 1) + 8 * r);
}

// V^T operand of key step x, dim block db from the stage at byte offset so
__device__ inline half8 read_vt(const char *lds, uint32_t vb, int so, int x, int db)
{
    const uint32_t a = (vb ^ (uint32_t)(64 * db)) + (uint32_t)so + (uint32_t)(x * 16 * ROWB);
    const u32x2 lo = lds_read_tr16(lds, a), hi = lds_read_tr16(lds, a + 8 * ROWB);
    return __builtin_bit_cast(half8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// A wave-uniform pointer held in vector registers (e.g. an argument of a
// non-inlined function), moved to scalar registers for the scalar base of a load.
__device__ inline const char *uniform_ptr(const char *ptr)
{
    const uint64_t x = (uint64_t)(uintptr_t)ptr;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return (const char *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// K rows of one tile straight into an LDS stage.  `tile` is the wave-uniform address of
// the tile's first row; the loads are inline asm so the compiler does not track them;
// they are waited for explicitly (vmcnt) before the barrier that publishes the stage.
// An LDS DMA reads its destination from M0 one wait state after the scalar write of M0
// at the earliest (the s_nop; the compiler puts the same wait after its own M0 writes).
template <bool PP>
__device__ inline void dma_k(const char *tile, const uint32_t (&off)[Lay<PP>::NDMA], uint32_t stage_lds, int wave)
{
    const char *t = uniform_ptr(tile);
#pragma unroll
    for (int i = 0; i < Lay<PP>::NDMA; ++i) {
        const uint32_t dst =
            __builtin_amdgcn_readfirstlane(stage_lds + (uint32_t)((Lay<PP>::ROWS * wave + 4 * i) * ROWB));
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "s"(dst), "v"(off[i]), "s"(t)
                     : "memory", "m0");
    }
}


// Factors (c, s) of slot dp at position qpos, times the slot's output scale sdim[dp]:
// fp32 trig of the fp64-reduced angle (signed revolutions wdim[dp] per position, negative
// for the inverse rotation; 0 for unrotated slots), or, with TAB, the caller's table entry
// of a rotated slot (NaN for a position the table does not cover), the sine times the
// rotation's sign.
template <bool TAB>
__device__ inline void slot_factor(int dp, int qpos, const double *wdim, const float *sdim, const QRot r,
                                   float &cs, float &sn)
{
    const float sc = sdim[dp];
    if (TAB && dp >= r.off2) {
        const int j = dp - r.off2;
        const bool in = qpos >= 0 && qpos < r.rows;
        cs = in ? r.cos_t[(int64_t)qpos * r.n_pairs + j] * sc : __builtin_nanf("");
        sn = in ? r.sin_t[(int64_t)qpos * r.n_pairs + j] * sc * r.sgn : __builtin_nanf("");
    } else {
        const float rf = (float)__builtin_amdgcn_fract((double)qpos * wdim[dp]);
        cs = __builtin_amdgcn_cosf(rf) * sc;
        sn = __builtin_amdgcn_sinf(rf) * sc;
    }
}

__device__ inline uint32_t rot_pack(float x0, float x1, float cs, float sn)
{
    const floatx2 y = {x0 * cs - x1 * sn, x0 * sn + x1 * cs};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(y, half2v));
}

// Half-split rotation of block pair (s, s + H16) (dims 16 s + 8 hh + e and the same plus
// n_pairs, for e = 0 .. 7): cs / sn of the eight pairs given.
__device__ inline void rot_half_blocks(const u32x4 &a, const u32x4 &b, const float (&cs)[8], const float (&sn)[8],
                                       half8 &ya, half8 &yb)
{
    u32x4 ha, hb;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float a0 = lo2f(a[w]), a1 = hi2f(a[w]), b0 = lo2f(b[w]), b1 = hi2f(b[w]);
        const int e = 2 * w;
        const floatx2 y0 = {a0 * cs[e] - b0 * sn[e], a1 * cs[e + 1] - b1 * sn[e + 1]};
        const floatx2 y1 = {a0 * sn[e] + b0 * cs[e], a1 * sn[e + 1] + b1 * cs[e + 1]};
        ha[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(y0, half2v));
        hb[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(y1, half2v));
    }
    ya = __builtin_bit_cast(half8, ha);
    yb = __builtin_bit_cast(half8, hb);
}

// q rotation (times the attention factor mscale) rounded to f16: the B operands of the S^T product.  The lane
// holds dims 16 s + 8 hh .. + 7 of its query in qin[s].  Adjacent pairs: slot
// 8 s + 4 hh + m is the lane's word m of block s.  Half-split (H16 = n_pairs / 16; the
// rotated dims start at block 8 - 2 H16): a block below that is taken per slot as
// above; block s of the first rotated half and block s + H16 hold the two dims of slots
// off / 2 + 16 (s - (8 - 2 H16)) + 8 hh + e.
template <int H16, bool TAB>
__device__ inline void rotate_q_t(half8 (&qop)[8], const u32x4 (&qin)[8], int qpos, int hh, const double *wdim,
                                  const float *sdim, const QRot r)
{
    constexpr int S0 = H16 ? 8 - 2 * H16 : 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        if (s < S0) {
            const int dp0 = 8 * s + 4 * hh;
            const u32x4 in = qin[s];
            u32x4 hv;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                float cs, sn;
                slot_factor<TAB>(dp0 + m, qpos, wdim, sdim, r, cs, sn);
                hv[m] = rot_pack(lo2f(in[m]), hi2f(in[m]), cs, sn);
            }
            qop[s] = __builtin_bit_cast(half8, hv);
        } else if (s < S0 + H16) {
            const int dp0 = 8 * S0 + 16 * (s - S0) + 8 * hh;
            float cs[8], sn[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                slot_factor<TAB>(dp0 + e, qpos, wdim, sdim, r, cs[e], sn[e]);
            rot_half_blocks(qin[s], qin[s + H16], cs, sn, qop[s], qop[s + H16]);
        }
    }
}



// The rotation factors of a workgroup's tokens, shared by the query heads of a group:
// entry (token k, slots 4 g .. 4 g + 3) holds {cos, sin} of each slot as slot_factor
// gives them, 32 bytes at byte (g * ntok + k) * 32 (a row of consecutive tokens per slot
// group, so the lanes of a wave read consecutive entries).
constexpr int TAB_B = 2 * TILE_B; // LDS byte offset: the K regions of stages 2 and 3

// Fill the table for ntok tokens (32 or 64): thread tid computes token k = tid % ntok at
// position tpos (that token's), pair groups (tid / ntok) * (ntok / 32) + 0 .. ntok / 32 - 1.
// The factors are the ones rotate_q computes.
template <bool TAB>
__device__ inline void fill_rot_table(char *lds, int tpos, int ntok, int tid, const double *wdim,
                                      const float *sdim, const QRot r)
{
    const int k = tid % ntok;
    const int per = ntok / QB;
    for (int e = 0; e < per; ++e) {
        const int g = (tid / ntok) * per + e;
        floatx4 f[2];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float cs, sn;
            slot_factor<TAB>(4 * g + m, tpos, wdim, sdim, r, cs, sn);
            f[m >> 1][2 * (m & 1)] = cs;
            f[m >> 1][2 * (m & 1) + 1] = sn;
        }
        floatx4 *dst = reinterpret_cast<floatx4 *>(lds + TAB_B + (g * ntok + k) * 32);
        dst[0] = f[0];
        dst[1] = f[1];
    }
}

// rotate_q with the factors of table token k (slots as in rotate_q_t)
template <int H16>
__device__ inline void rotate_q_tab_t(half8 (&qop)[8], const u32x4 (&qin)[8], const char *lds, int ntok, int k,
                                      int hh)
{
    constexpr int S0 = H16 ? 8 - 2 * H16 : 8;
    auto entry = [&](int g) { return reinterpret_cast<const floatx4 *>(lds + TAB_B + (g * ntok + k) * 32); };
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        if (s < S0) {
            const floatx4 *src = entry(2 * s + hh);
            const floatx4 f0 = src[0], f1 = src[1];
            const float cs[4] = {f0[0], f0[2], f1[0], f1[2]};
            const float sn[4] = {f0[1], f0[3], f1[1], f1[3]};
            const u32x4 in = qin[s];
            u32x4 hv;
#pragma unroll
            for (int m = 0; m < 4; ++m)
                hv[m] = rot_pack(lo2f(in[m]), hi2f(in[m]), cs[m], sn[m]);
            qop[s] = __builtin_bit_cast(half8, hv);
        } else if (s < S0 + H16) {
            const int g0 = (8 * S0 + 16 * (s - S0) + 8 * hh) / 4;
            const floatx4 *p0 = entry(g0), *p1 = entry(g0 + 1);
            const floatx4 f0 = p0[0], f1 = p0[1], f2 = p1[0], f3 = p1[1];
            const float cs[8] = {f0[0], f0[2], f1[0], f1[2], f2[0], f2[2], f3[0], f3[2]};
            const float sn[8] = {f0[1], f0[3], f1[1], f1[3], f2[1], f2[3], f3[1], f3[3]};
            rot_half_blocks(qin[s], qin[s + H16], cs, sn, qop[s], qop[s + H16]);
        }
    }
}


// Rare path.  The fast path keeps each row's reference max from its first tile; when a
// later key scores 2^16 or more above it, an f16 probability overflows and the row sum
// turns infinite.  Then the whole workgroup recomputes the unit here with the running
// max moved on every tile that exceeds it (so no probability exceeds 1): plainly, one
// tile at a time through LDS stage 0, each wave its own item.  Not inlined, so that its
// registers do not weigh on the fast path.
template <int H16, bool TAB, bool PP>
__device__ __attribute__((noinline)) void exact_unit(const PrefillParams p, char *lds, const double *wdim,
                                                     const float *sdim, int u, int g, int wk, int hist,
                                                     int tu, const QRot rot, float sl2)
{
    constexpr int NW = Lay<PP>::NW, NDMA = Lay<PP>::NDMA, VREG_B = Lay<PP>::VREG_B;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane & 31, hh = lane >> 5;
    const int item = wk * NW + wave;
    const bool wave_valid = item < p.items;
    const int last_item = min(wk * NW + NW - 1, p.items - 1);
    const int my_item = wave_valid ? item : last_item;
    const int tb = my_item / p.G;
    const int h = g * p.G + (my_item - tb * p.G);
    const int i0 = tb * QB, i = i0 + c;
    const int kend = hist + min((last_item / p.G + 1) * QB, tu);
    const int klast = kend - 1;
    const int ntiles = (kend + KT - 1) / KT;
    const int qlimit = hist + i;
    const char *kbase = reinterpret_cast<const char *>(p.ck + ((int64_t)u * p.hkv + g) * p.s_cap * kHeadDim);
    const char *vbase = reinterpret_cast<const char *>(p.cv + ((int64_t)u * p.hkv + g) * p.s_cap * kHeadDim);

    const int iq = min(i, p.t - 1);
    const uint16_t *qrow = p.q + (((int64_t)u * p.t + iq) * p.hq + h) * kHeadDim;
    u32x4 qin[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
        qin[s] = ld16(qrow + 16 * s + 8 * hh);
    half8 qop[8];
    rotate_q_t<H16, TAB>(qop, qin, p.pos[(int64_t)u * p.t + iq], hh, wdim, sdim, rot);

    const uint32_t vb = vt_base<PP>(lane);
    floatx16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
        o[db] = floatx16{0.f};
    float m_run = -INFINITY, l_run = 0.f;
    for (int j = 0; j < ntiles; ++j) {
        const int kb = j * KT;
        // K and V rows (clamped past kend) straight into stage 0
        uint32_t ko[NDMA], vo[NDMA];
#pragma unroll
        for (int r = 0; r < NDMA; ++r) {
            const int row = krow<PP>(wave, lane, r);
            ko[r] = (uint32_t)(min(row, klast - kb) * ROWB + (((lane & 15) ^ kswz(row)) << 4));
            vo[r] = (uint32_t)(min(row, klast - kb) * ROWB + (((lane & 15) ^ vswz(row)) << 4));
        }
        const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));
        dma_k<PP>(uniform_ptr(kbase + (int64_t)kb * ROWB), ko, lds0, wave);
        dma_k<PP>(uniform_ptr(vbase + (int64_t)kb * ROWB), vo, lds0 + VREG_B, wave);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        wg_barrier();

        floatx16 sacc[2] = {floatx16{0.f}, floatx16{0.f}};
#pragma unroll
        for (int y = 0; y < 16; ++y) {
            const int sb = y & 1, st = y >> 1;
            const half8 a = *reinterpret_cast<const half8 *>(lds + (32 * sb + c) * ROWB + (((2 * st + hh) ^ kswz(c)) << 4));
            sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qop[st], sacc[sb], 0, 0, 0);
        }
        // running max of the plain dot products; the scale enters each exp2 argument
        const int lim = qlimit - kb - 4 * hh;
        float mx = -INFINITY;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (32 * sb + 8 * (r >> 2) + (r & 3) > lim)
                    sacc[sb][r] = -INFINITY;
                mx = fmaxf(mx, sacc[sb][r]);
            }
        }
        mx = half_max(mx);
        if (mx > m_run) {
            // (the first tile holds key 0, visible to every row, so mx is finite)
            const float alpha = __builtin_amdgcn_exp2f((m_run - mx) * sl2);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
                o[db] *= alpha;
            m_run = mx;
        }
        u32x4 pw[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 8 * (x & 1) + 2 * jj;
                const floatx2 pf = {__builtin_amdgcn_exp2f((sacc[x >> 1][r] - m_run) * sl2),
                                    __builtin_amdgcn_exp2f((sacc[x >> 1][r + 1] - m_run) * sl2)};
                l_run += pf[0] + pf[1];
                pw[x][jj] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pf, half2v));
            }
        }
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int db = x & 3;
            const half8 a = read_vt(lds, vb, 0, x >> 2, db);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(half8, pw[x >> 2]), o[db], 0, 0, 0);
        }
        wg_barrier(); // stage 0 is reloaded next
    }
    const float inv = 1.f / half_sum(l_run);
    if (wave_valid && i < tu) {
        uint16_t *orow = p.out + (((int64_t)u * p.t + i) * p.hq + h) * kHeadDim;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int ig = 0; ig < 4; ++ig) {
                const u32x2 w = {pack2h(o[db][4 * ig + 0] * inv, o[db][4 * ig + 1] * inv),
                                 pack2h(o[db][4 * ig + 2] * inv, o[db][4 * ig + 3] * inv)};
                *reinterpret_cast<u32x2 *>(orow + 32 * db + 8 * ig + 4 * hh) = w;
            }
        }
    }
}

// H16: the pairing of q's rotated dims, as in rotate_q_t; TAB: factors from the caller's
// tables.  One kernel per variant keeps the other variants' code out of the fast path's
// register allocation.
template <int H16, bool TAB, bool PP>
__global__ void __launch_bounds__(Lay<PP>::NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_attn_kernel(PrefillParams p, RopeTable tab, QRot rot)
{
    constexpr int NW = Lay<PP>::NW, NT = Lay<PP>::NT, NSTAGE = Lay<PP>::NSTAGE, VREG_B = Lay<PP>::VREG_B,
                  NDMA = Lay<PP>::NDMA;
    __shared__ __align__(16) char lds[2 * NSTAGE * TILE_B];
    // per parameter set (row kMaxRopeSets: NaN, for an invalid set index): revolutions per
    // position of dim pair dp (0: unrotated) and its output scale
    __shared__ double wdim[kMaxRopeSets + 1][kMaxPairs];
    __shared__ float sdim[kMaxRopeSets + 1][kMaxPairs];
    __shared__ int ovf_unit;           // last unit whose row sums overflowed

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane & 31;  // query within the wave's block (S^T column)
    const int hh = lane >> 5; // lane half
    const int KP = p.n * p.hkv;

    // Persistent workgroups.  Work unit v (0 .. units-1) is (KV pair v % KP, rank v / KP);
    // rank 0 is the heaviest (the last token blocks).  Round r hands unit r * P + w' to
    // workgroup w, with w' = w on even rounds and reversed on odd ones, so the cost of
    // consecutive rounds evens out.  With P a multiple of 8 the reversal keeps w' = w
    // (mod 8): workgroups are dealt to the 8 XCDs round-robin, so when KP is a multiple
    // of 8 too, every unit of a pair runs on the same XCD and its K/V stays in that L2.
    // Pair-major order (when the history dominates, so that the units of a pair cost about
    // the same): XCD x takes the pairs x, x + 8, ... one after another, all units of a pair
    // in the same round, heaviest rank first; so the XCD's workgroups stream one pair's K/V
    // together instead of every pair's at once, and a tile leaves HBM about once.
    const int P = gridDim.x;

    // rotation tables of every parameter set, shared by every unit
    for (int e = tid; e < (kMaxRopeSets + 1) * kMaxPairs; e += NT) {
        const int rs = e / kMaxPairs, dp = e % kMaxPairs;
        const bool rot_t = 2 * dp >= tab.off;
        if (rs < tab.nsets) {
            wdim[rs][dp] = rot_t ? tab.sgn * tab.wrev[rs][dp - (tab.off >> 1)] : 0.0;
            sdim[rs][dp] = rot_t ? (float)tab.mscale[rs] : 1.f;
        } else {
            wdim[rs][dp] = __builtin_nan("");
            sdim[rs][dp] = __builtin_nanf("");
        }
    }
    if (tid == 0)
        ovf_unit = -1;
    wg_barrier();

    for (int round = 0;; ++round) {
        int slot = blockIdx.x;
        if (round & 1)
            slot = p.xcd ? ((P >> 3) - 1 - (slot >> 3)) * 8 + (slot & 7) : P - 1 - slot;
        int v, rank, kp;
        if (p.pairmajor) {
            const int i = round * (P >> 3) + (slot >> 3); // unit index on this XCD
            if (i >= (KP >> 3) * p.wpk)
                break;
            const int pl = i / p.wpk;
            rank = i - pl * p.wpk;
            kp = (slot & 7) + 8 * pl;
            v = rank * KP + kp;
        } else {
            v = round * P + slot;
            if (v >= p.units)
                break;
            rank = v / KP;
            kp = v - rank * KP;
        }
        const int wk = p.wpk - 1 - rank;
        const int u = kp / p.hkv, g = kp - u * p.hkv;
        const int item = wk * NW + wave;
        const bool wave_valid = item < p.items;
        const int last_item = min(wk * NW + NW - 1, p.items - 1);
        const int my_item = wave_valid ? item : last_item;
        const int tb = my_item / p.G;
        const int h = g * p.G + (my_item - tb * p.G);
        const int i0 = tb * QB;
        const int i = i0 + c;
        const int hist = p.lens ? p.lens[u] : 0;
        const int tu = p.new_lens ? p.new_lens[u] : p.t; // this unit's new tokens
        const int rset = rope_set(tab, u);
        const double *wd = wdim[rset < 0 ? kMaxRopeSets : rset];
        const float *sd = sdim[rset < 0 ? kMaxRopeSets : rset];
        if (hist < 0 || hist > p.max_hist || tu < 0 || tu > p.t) {
            // invalid history or new-token count: no cache was written for this unit; report
            // NaN in every row
            const bool row_valid = wave_valid && i < p.t;
            if (row_valid && hh == 0) {
                uint16_t *orow = p.out + (((int64_t)u * p.t + i) * p.hq + h) * kHeadDim;
                for (int d = 0; d < kHeadDim; ++d)
                    orow[d] = qnan16();
            }
            continue; // uniform over the workgroup: hist belongs to the unit
        }
        const int tb_first = (wk * NW) / p.G;
        if (tb_first * QB >= tu)
            continue; // every row of the unit is padding (uniform over the workgroup)
        const bool row_valid = wave_valid && i < tu;
        const int tb_last = last_item / p.G;
        const int kend = hist + min((tb_last + 1) * QB, tu); // keys the workgroup needs
        const int klast = kend - 1;
        const int ntiles = (kend + KT - 1) / KT;
        const int kend_w = hist + min(i0 + QB, tu);         // keys this wave needs
        const int qlimit = hist + i;                         // last visible key of the lane's query

        const char *kbase = reinterpret_cast<const char *>(p.ck + ((int64_t)u * p.hkv + g) * p.s_cap * kHeadDim);
        const char *vbase = reinterpret_cast<const char *>(p.cv + ((int64_t)u * p.hkv + g) * p.s_cap * kHeadDim);

        // per-lane tile offsets (full tiles) and the LDS addresses of this thread
        uint32_t koff[NDMA], voff[NDMA];
#pragma unroll
        for (int r = 0; r < NDMA; ++r) {
            const int row = krow<PP>(wave, lane, r);
            koff[r] = koffset(row, lane);
            voff[r] = (uint32_t)(row * ROWB + (((lane & 15) ^ vswz(row)) << 4));
        }
        const uint32_t lds_base = lds_offset(lds);

        // Tile loads.  Rows at or past kend clamp to the last key (finite values; they are
        // masked or carry probability 0), and only the last tile can hold such rows.
        auto issue_k = [&](int j, uint32_t stage_lds) {
            const int kb = j * KT;
            const char *tile = kbase + (int64_t)kb * ROWB;
            if (kb + KT <= kend) {
                dma_k<PP>(tile, koff, stage_lds, wave);
            } else {
                // the source row clamps; the swizzled chunk stays the destination row's
                uint32_t o[NDMA];
#pragma unroll
                for (int r = 0; r < NDMA; ++r) {
                    const int row = krow<PP>(wave, lane, r);
                    o[r] = (uint32_t)(min(row, klast - kb) * ROWB + (((lane & 15) ^ kswz(row)) << 4));
                }
                dma_k<PP>(tile, o, stage_lds, wave);
            }
        };
        // V rows the same way into the V region of a stage, under their own chunk swizzle
        auto issue_v = [&](int j, uint32_t stage_lds) {
            const int kb = j * KT;
            const char *tile = vbase + (int64_t)kb * ROWB;
            if (kb + KT <= kend) {
                dma_k<PP>(tile, voff, stage_lds, wave);
            } else {
                uint32_t o[NDMA];
#pragma unroll
                for (int r = 0; r < NDMA; ++r) {
                    const int row = krow<PP>(wave, lane, r);
                    o[r] = (uint32_t)(min(row, klast - kb) * ROWB + (((lane & 15) ^ vswz(row)) << 4));
                }
                dma_k<PP>(tile, o, stage_lds, wave);
            }
        };

        // ---- loads in flight: this lane's q row, tiles 0 and 1
        // rows past t read row t-1 (branch-free loads; their outputs are never written)
        const int iq = min(i, p.t - 1);
        const uint16_t *qrow = p.q + (((int64_t)u * p.t + iq) * p.hq + h) * kHeadDim;
        const int qpos = p.pos[(int64_t)u * p.t + iq];
        // position of this thread's token of the unit's rotation table (see below; rows
        // past t take row t - 1's), loaded first so that it arrives first
        const int ntok = (tb_last - tb_first + 1) * QB;
        const int tpos = PP ? p.pos[(int64_t)u * p.t + min(tb_first * QB + tid % ntok, p.t - 1)] : 0;
        u32x4 qin[8];
#pragma unroll
        for (int s = 0; s < 8; ++s)
            qin[s] = ld16(qrow + 16 * s + 8 * hh);
        if (!PP)
            wg_barrier(); // every wave has read its previous unit's output rows back (K region)
        issue_k(0, lds_base);
        issue_v(0, lds_base + VREG_B);
        if (ntiles > 1)
            issue_k(1, lds_base + TILE_B);

        // ---- q prologue: rotate (fp32 trig of the fp64-reduced angle), round to f16.
        // In the ping-pong layout, when the unit's items span at most two token blocks, the
        // workgroup computes each (token, pair) factor once into LDS (the K region of stages
        // 2-3, free at this point) instead of once per query head; the lock-step layout's
        // ring has no room for the table, and the other workgroup covers the trig.
        half8 qop[8];
        if (PP && ntok <= 2 * QB) {
            wg_barrier(); // every wave has read its previous unit's output rows back
            fill_rot_table<TAB>(lds, tpos, ntok, tid, wd, sd, rot);
            wg_barrier();
            rotate_q_tab_t<H16>(qop, qin, lds, ntok, (tb - tb_first) * QB + c, hh);
        } else {
            rotate_q_t<H16, TAB>(qop, qin, qpos, hh, wd, sd, rot);
        }

        // ---- per-lane LDS byte addresses (stage 0; other stages by immediate offsets)
        // K operand of head-dim step s: chunk (2s + hh) ^ (c % 16) of key row c.  The step
        // sits in bits 5-7 of the byte offset, so one per-lane base serves all eight steps
        // through an xor.  V^T operands: vt_base.
        const uint32_t kbase0 = (uint32_t)(c * ROWB + ((hh ^ kswz(c)) << 4));
        const uint32_t vbase0 = vt_base<PP>(lane);

        floatx16 o[4];
        // row sums of the f16 probabilities, accumulated on the matrix core by one
        // v_mfma_f32_16x16x32_f16 per 16-key step (half the cycles of a 32x32x16): B is the
        // step's P^T operand read as 16x16x32 B (lane l: column l % 16, k 8 (l / 16) ..),
        // so column n gathers query n (lane groups 0, 2) and query n + 16 (groups 1, 3);
        // the A operand (row m, k-group l / 16) is 1 where m % 2 == group % 2, so even rows
        // of the result sum query n and odd rows query n + 16.  Lane l finds its query's sum
        // in slot (l / 16) % 2.
        floatx4 lsum;
        float m_run = 0.f; // reference max of the dot products
        const float sl2 = p.scale_log2;
        bool first = true;
        floatx16 sacc[2];  // S^T of the current tile, as (dot product - m_run)
        u32x4 pw[4];       // f16 probabilities of the previous tile (PV B operands)
        const _Float16 sel1 = (lane & 1) == ((lane >> 4) & 1) ? (_Float16)1.f : (_Float16)0.f;
        const half8 sel = {sel1, sel1, sel1, sel1, sel1, sel1, sel1, sel1};

        // A wave's phases alternate
        //   M(j): PV of tile j-1, then S^T of tile j   (32 MFMAs)
        //   S(j): softmax of tile j                     (VALU)
        auto tile_active = [&](int j) { return wave_valid && j * KT < kend_w; };

        // The operand reads of an M phase, x = 0 .. 31: x < 16 the V^T blocks of tile j-1
        // (key group x/4, dim block x%4) from the V region at byte offset vso, x >= 16 the K
        // blocks of tile j (head-dim step (x-16)/2, key block x%2) from the K region at kso.
        // (kb, vb: the per-lane bases, made opaque once per phase so that the compiler
        // keeps two registers instead of hoisting twelve precomputed addresses)
        auto rd = [&](uint32_t kb, uint32_t vb, int kso, int vso, int x) -> half8 {
            if (x < 16)
                return read_vt(lds, vb, vso, x >> 2, x & 3);
            const int y = x - 16;
            return *reinterpret_cast<const half8 *>(lds + ((kb ^ (uint32_t)((y >> 1) << 5)) + kso + (y & 1) * 32 * ROWB));
        };

        // MFMAs x0 .. x1-1 of the sequence above, each operand read RD MFMAs ahead.  With
        // PRE the first RD reads were issued by the preceding softmax phase.
        half8 buf[RD];
        auto prefetch = [&](int vso) {
            uint32_t kb = kbase0, vb = vbase0;
            asm volatile("" : "+v"(kb), "+v"(vb));
#pragma unroll
            for (int k = 0; k < RD; ++k)
                buf[k] = rd(kb, vb, 0, vso, k);
        };
        auto mstream = [&](auto x0_c, auto x1_c, auto pre_c, int kso, int vso) {
            constexpr int X0 = decltype(x0_c)::value, X1 = decltype(x1_c)::value;
            uint32_t kb = kbase0, vb = vbase0;
            asm volatile("" : "+v"(kb), "+v"(vb));
            // the S^T chains start at -m: written into the (dead) S^T registers two slots per
            // PV MFMA, or all at once when the phase has no PV part
            float mr = -m_run;
            asm volatile("" : "+v"(mr));
            if (!decltype(pre_c)::value) {
#pragma unroll
                for (int k = 0; k < RD; ++k)
                    if (X0 + k < X1)
                        buf[k] = rd(kb, vb, kso, vso, X0 + k);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int x = X0; x < X1; ++x) {
                const half8 a = buf[(x - X0) % RD];
                if (x < 16) {
                    o[x & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(half8, pw[x >> 2]),
                                                                      o[x & 3], 0, 0, 0);
                    // after the last dim block of key group x/4: its row sums
                    if ((x & 3) == 3)
                        lsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(sel, __builtin_bit_cast(half8, pw[x >> 2]),
                                                                      lsum, 0, 0, 0);
                    if (X1 > 16) {
                        sacc[x >> 3][2 * (x & 7)] = mr;
                        sacc[x >> 3][2 * (x & 7) + 1] = mr;
                    }
                } else {
                    if (x == 16 && X0 == 16) {
                        sacc[0] = floatx16(mr);
                        sacc[1] = floatx16(mr);
                    }
                    // the two key blocks' chains alternate, so consecutive MFMAs never wait
                    // on each other's results
                    const int y = x - 16, sb = y & 1;
                    sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qop[y >> 1], sacc[sb], 0, 0, 0);
                }
                if (x + RD < X1)
                    buf[(x - X0) % RD] = rd(kb, vb, kso, vso, x + RD);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // probabilities of the tile (f16 pairs, the PV operand) and their sum
        // probabilities of the tile (f16 pairs, the PV operand)
        auto probs = [&]() {
#pragma unroll
            for (int x = 0; x < 4; ++x) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int r = 8 * (x & 1) + 2 * jj;
                    const floatx2 pf = {__builtin_amdgcn_exp2f(sacc[x >> 1][r] * sl2),
                                        __builtin_amdgcn_exp2f(sacc[x >> 1][r + 1] * sl2)};
                    pw[x][jj] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pf, half2v));
                }
            }
        };
        // row max of the tile's (masked) scores, over both lane halves
        auto tile_max = [&]() -> float {
            float mx = -INFINITY;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    mx = fmaxf(mx, sacc[sb][r]);
            }
            return half_max(mx);
        };
        // causal mask of tile j (only tiles reaching past the block's first query)
        auto mask_tile = [&](int j) {
            const int kb = j * KT;
            if (kb + KT - 1 > hist + i0) {
                const int lim = qlimit - kb - 4 * hh;
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        if (32 * sb + 8 * (r >> 2) + (r & 3) > lim)
                            sacc[sb][r] = -INFINITY;
                    }
                }
            }
        };

        // softmax of tile j into pw (zero probabilities for a wave past its last key)
        auto softmax = [&](int j) {
            if (tile_active(j)) {
                mask_tile(j);
                if (first) {
                    // a row's first tile holds key 0, visible to every row
                    const float mx = tile_max();
                    m_run = mx;
#pragma unroll
                    for (int sb = 0; sb < 2; ++sb)
                        sacc[sb] -= mx;
                    first = false;
                }
                probs();
            } else {
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    pw[x] = u32x4{0u};
            }
        };

#pragma unroll
        for (int db = 0; db < 4; ++db)
            o[db] = floatx16{0.f};
        lsum = floatx4{0.f};

        if constexpr (PP) {
            // Ping-pong: waves 0-3 and 4-7 run the same phases, the second group one phase
            // behind, each phase ending in a workgroup barrier.  Tile j sits in LDS stage
            // j % 4 from two tiles before its first use (S^T in M(j)) until its last (PV in
            // M(j+1) of the trailing group).
            const int grp = wave >> 2;
            // Tile staging for M(j) (STG = j % 4): wait for this wave's share of the previous
            // staging's loads (K of tile j+1, V of tile j), which the barrier ending the phase
            // then publishes, and start the next: K of tile j+2 and V of tile j+1, each into its
            // stage.  It runs at the end of the softmax phase before M(j), while the SIMD
            // partner is in its MFMA phase.  A V stage is refilled one phase pair after its K
            // stage: V of tile j-3 is read by the PV part of M(j-2), which the trailing group
            // runs during the leading group's softmax phase S(j-2).
            auto stage_tiles = [&](auto stg_c, int j) {
                constexpr int STG = decltype(stg_c)::value;
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                if (j + 2 < ntiles)
                    issue_k(j + 2, lds_base + (uint32_t)(((STG + 2) % NSTAGE) * TILE_B));
                if (j + 1 < ntiles)
                    issue_v(j + 1, lds_base + (uint32_t)(VREG_B + ((STG + 1) % NSTAGE) * TILE_B));
            };

            // M(j), 1 <= j < ntiles: PV of tile j-1 and S^T of tile j.  A wave whose tile j-1 is
            // past its last key runs it anyway on zero probabilities (its SIMD partner is in
            // its softmax, so the matrix core is free), which keeps one code path.
            auto phase_m = [&](auto stg_c, int j) {
                constexpr int STG = decltype(stg_c)::value;
                // the matrix-core phase outranks the other group's softmax for issue slots
                __builtin_amdgcn_s_setprio(1);
                mstream(std::integral_constant<int, 0>{}, std::integral_constant<int, 32>{}, std::true_type{},
                        STG * TILE_B, ((STG + NSTAGE - 1) % NSTAGE) * TILE_B);
                __builtin_amdgcn_s_setprio(0);
                wg_barrier();
            };

            // S(j) (STG = j % 4): softmax of tile j, then the staging and the first operand
            // reads (V^T of tile j) of M(j+1).
            auto phase_s = [&](auto stg_c, int j) {
                constexpr int STG = decltype(stg_c)::value;
                softmax(j);
                stage_tiles(std::integral_constant<int, (STG + 1) % NSTAGE>{}, j + 1);
                prefetch(STG * TILE_B);
                wg_barrier_reads_in_flight<2 * RD>(); // two transposing reads per V^T operand
            };

            // tile 0 (K and V) in stage 0, K of tile 1 in stage 1
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            wg_barrier();

            if (grp == 1)
                wg_barrier(); // the trailing group starts one phase late
            // M(0): S^T of tile 0 only
            stage_tiles(std::integral_constant<int, 0>{}, 0);
            __builtin_amdgcn_s_setprio(1);
            mstream(std::integral_constant<int, 16>{}, std::integral_constant<int, 32>{}, std::false_type{}, 0, 0);
            __builtin_amdgcn_s_setprio(0);
            wg_barrier();
            phase_s(std::integral_constant<int, 0>{}, 0);
            for (int j0 = 1; j0 < ntiles; j0 += 4) {
                phase_m(std::integral_constant<int, 1>{}, j0);
                phase_s(std::integral_constant<int, 1>{}, j0);
                if (j0 + 1 < ntiles) {
                    phase_m(std::integral_constant<int, 2>{}, j0 + 1);
                    phase_s(std::integral_constant<int, 2>{}, j0 + 1);
                    if (j0 + 2 < ntiles) {
                        phase_m(std::integral_constant<int, 3>{}, j0 + 2);
                        phase_s(std::integral_constant<int, 3>{}, j0 + 2);
                        if (j0 + 3 < ntiles) {
                            phase_m(std::integral_constant<int, 0>{}, j0 + 3);
                            phase_s(std::integral_constant<int, 0>{}, j0 + 3);
                        }
                    }
                }
            }
            // M(ntiles): PV of the last tile only (its first reads were issued by S(ntiles-1))
            __builtin_amdgcn_s_setprio(1);
            mstream(std::integral_constant<int, 0>{}, std::integral_constant<int, 16>{}, std::true_type{}, 0,
                    ((ntiles - 1) % NSTAGE) * TILE_B);
            __builtin_amdgcn_s_setprio(0);
            wg_barrier();
            if (grp == 0)
                wg_barrier(); // same barrier count for both groups
        } else {
            // Lock-step: the four waves run the same phase; the other workgroup on the compute
            // unit supplies the overlap of matrix and vector work.  One barrier per tile, in
            // S(j) after this wave's wait for its share of K(j+1) and V(j): it publishes them,
            // and every wave is then past M(j).  Then K of tile j+2 goes into K stage j % 2
            // (K(j) was last read by M(j)'s S^T part) and V of tile j+1 into V stage
            // (j+1) % 2 (V(j-1) was last read by M(j)'s PV part).
            auto phase_s = [&](auto stg_c, int j) {
                constexpr int STG = decltype(stg_c)::value;
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                wg_barrier();
                if (j + 2 < ntiles)
                    issue_k(j + 2, lds_base + (uint32_t)(STG * TILE_B));
                if (j + 1 < ntiles)
                    issue_v(j + 1, lds_base + (uint32_t)(VREG_B + (STG ^ 1) * TILE_B));
                softmax(j);
                prefetch(STG * TILE_B); // V^T of tile j, for M(j+1)
            };
            // M(j), 1 <= j < ntiles (STG = j % 2): PV of tile j-1 and S^T of tile j
            auto phase_m = [&](auto stg_c, int j) {
                constexpr int STG = decltype(stg_c)::value;
                (void)j;
                __builtin_amdgcn_s_setprio(1);
                mstream(std::integral_constant<int, 0>{}, std::integral_constant<int, 32>{}, std::true_type{},
                        STG * TILE_B, (STG ^ 1) * TILE_B);
                __builtin_amdgcn_s_setprio(0);
            };

            // tile 0 (K and V) in stage 0, K of tile 1 in stage 1
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            wg_barrier();
            // M(0): S^T of tile 0 only
            __builtin_amdgcn_s_setprio(1);
            mstream(std::integral_constant<int, 16>{}, std::integral_constant<int, 32>{}, std::false_type{}, 0, 0);
            __builtin_amdgcn_s_setprio(0);
            phase_s(std::integral_constant<int, 0>{}, 0);
            for (int j0 = 1; j0 < ntiles; j0 += 2) {
                phase_m(std::integral_constant<int, 1>{}, j0);
                phase_s(std::integral_constant<int, 1>{}, j0);
                if (j0 + 1 < ntiles) {
                    phase_m(std::integral_constant<int, 0>{}, j0 + 1);
                    phase_s(std::integral_constant<int, 0>{}, j0 + 1);
                }
            }
            // M(ntiles): PV of the last tile only
            __builtin_amdgcn_s_setprio(1);
            mstream(std::integral_constant<int, 0>{}, std::integral_constant<int, 16>{}, std::true_type{}, 0,
                    ((ntiles - 1) % NSTAGE) * TILE_B);
            __builtin_amdgcn_s_setprio(0);
        }

        // An f16 probability past its range made a row sum infinite (or a NaN input made
        // it NaN): the workgroup recomputes the unit on the exact path.  The flag holds the
        // unit, so it never needs clearing.
        const float lrow = ((lane >> 4) & 1) ? lsum[1] : lsum[0];
        if (__builtin_amdgcn_ballot_w64(row_valid && !(lrow <= 3.0e38f)) != 0 && lane == 0)
            ovf_unit = v;
        wg_barrier();
        if (ovf_unit == v) {
            // (without tables the rotation needs nothing beyond LDS: no live kernel arguments)
            exact_unit<H16, TAB, PP>(p, lds, wd, sd, u, g, wk, hist, tu, TAB ? rot : QRot{}, sl2);
            continue;
        }

        // ---- normalise and write.  The lane holds dims 32db + 8*(r/4) + 4*hh + r%4 of query
        // c; the rows pass through the wave's own 8 KB slice of LDS stages 2-3 (idle from the
        // last barrier until the next unit's first K tile 2 load, two barriers later), so
        // that every global store writes whole 256-byte rows instead of 8-byte pieces of 64
        // rows.  16-byte chunk k of row c sits at chunk k ^ (c % 16).
        const float inv = 1.f / lrow;
        // (ping-pong: stages 2-3, idle from the last barrier until the next unit's first K
        // tile 2 load; lock-step: the K region, last read by M(ntiles-1), refilled only after
        // the next unit's first barrier)
        char *ostage = lds + (!PP ? wave * (QB * ROWB)
                              : wave < 4 ? 2 * TILE_B + wave * (QB * ROWB)
                                         : VREG_B + 2 * TILE_B + (wave - 4) * (QB * ROWB));
        // the per-lane staging addresses below are recomputed per unit from an opaque copy of
        // the lane index, so that they are not hoisted to the kernel's start and kept (or
        // spilled) across the tile loop
        int le = lane;
        asm volatile("" : "+v"(le));
        const int ce = le & 31, he = le >> 5;
        // chunk k of row c: the per-lane base with bits 4-7 flipped by k (opaque, so the
        // sixteen addresses are not hoisted out of the unit loop into spilled registers)
        uint32_t wbase = (uint32_t)((ostage - lds) + ce * ROWB + ((ce & 15) << 4) + he * 8);
        asm volatile("" : "+v"(wbase));
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int ig = 0; ig < 4; ++ig) {
                const u32x2 w = {pack2h(o[db][4 * ig + 0] * inv, o[db][4 * ig + 1] * inv),
                                 pack2h(o[db][4 * ig + 2] * inv, o[db][4 * ig + 3] * inv)};
                *reinterpret_cast<u32x2 *>(lds + (wbase ^ (uint32_t)((4 * db + ig) << 4))) = w;
            }
        }
        // lanes read what other lanes wrote: keep the reads after the writes
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // Read back: lane L takes 16-byte chunk L % 16 of row 4x + L / 16.  With g = L / 16 the
        // physical chunk is (L % 16) ^ g ^ 4 (x % 4), so row 4x's address is a per-lane base
        // with bits 6-7 flipped by x % 4, plus 1 KB x.  All reads are issued before the
        // first store; the asm statements keep the compiler from hoisting per-row values
        // out of the unit loop (into spilled registers) or sinking reads into the stores'
        // branches.
        uint32_t rbase = (uint32_t)((ostage - lds) + (le >> 4) * ROWB + (((le & 15) ^ (le >> 4)) << 4));
        uint32_t olane = (uint32_t)((le >> 4) * p.hq * ROWB + 16 * (le & 15));
        asm volatile("" : "+v"(rbase), "+v"(olane));
        u32x4 orows[QB / 4];
#pragma unroll
        for (int x = 0; x < QB / 4; ++x) {
            const uint32_t a = (rbase ^ (uint32_t)((x & 3) << 6)) + (uint32_t)(x * 4 * ROWB);
            orows[x] = *reinterpret_cast<const u32x4 *>(lds + a);
        }
#pragma unroll
        for (int x = 0; x < QB / 4; ++x)
            asm volatile("" : "+v"(orows[x]));
#pragma unroll
        for (int x = 0; x < QB / 4; ++x) {
            char *rows4 = reinterpret_cast<char *>(p.out + (((int64_t)u * p.t + i0 + 4 * x) * p.hq + h) * kHeadDim);
            if (wave_valid && i0 + 4 * x + (le >> 4) < tu)
                *reinterpret_cast<u32x4 *>(rows4 + olane) = orows[x];
        }
    } // work units
}

} // namespace

hipError_t launch_prefill_attention(const uint16_t *q, const uint16_t *cache_k,
                                    const uint16_t *cache_v, const int32_t *positions,
                                    const int32_t *lens, const int32_t *new_lens, uint16_t *out,
                                    const PrefillShape &s,
                                    const RopeTable &tab, hipStream_t stream,
                                    hipEvent_t ev_before, hipEvent_t ev_after)
{
    if (s.n == 0 || s.t == 0)
        return hipSuccess;
    PrefillParams p;
    p.q = q;
    p.ck = cache_k;
    p.cv = cache_v;
    p.pos = positions;
    p.lens = lens;
    p.new_lens = new_lens;
    p.out = out;
    p.n = s.n;
    p.t = s.t;
    p.hq = s.hq;
    p.hkv = s.hkv;
    p.s_cap = s.s_cap;
    p.max_hist = s.max_hist;
    p.G = s.hq / s.hkv;
    // Layout: ping-pong when the history is at least as long as the new tokens (long
    // units: measured 3 % faster than lock-step on a 32-layer 3840 + 256 prefill_kv),
    // lock-step otherwise (short units: 5-6 % faster on a 28-layer T = 1024 prefill)
    const bool pp = s.max_hist >= s.t;
    const int nw = pp ? Lay<true>::NW : Lay<false>::NW;
    const int tblocks = (s.t + QB - 1) / QB;
    p.items = tblocks * p.G;
    p.wpk = (p.items + nw - 1) / nw;
    const int64_t units = (int64_t)s.n * s.hkv * p.wpk;
    if (units > INT32_MAX)
        return hipErrorInvalidValue;
    p.units = (int)units;
    p.scale_log2 = (float)((double)s.scale * 1.4426950408889634);
    QRot rot;
    rot.cos_t = tab.cos_t;
    rot.sin_t = tab.sin_t;
    rot.rows = tab.rows;
    rot.n_pairs = tab.n_pairs;
    rot.off2 = tab.off >> 1;
    rot.h16 = tab.half ? tab.n_pairs / 16 : 0;
    rot.sgn = (float)tab.sgn;
    // one ping-pong workgroup per compute unit (its ring takes most of a CU's LDS), or two
    // lock-step ones
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return e;
    const int64_t blocks = std::min<int64_t>(units, (int64_t)std::max(ncu, 1) * (pp ? 1 : 2));
    p.xcd = (blocks % 8 == 0) ? 1 : 0;
    // pair-major order when the history bounds the work per unit (the units of a pair then
    // differ by at most t keys of their max_hist + t): measured 2-3 % faster on a 32-layer
    // 3840 + 256 prefill_kv, 1-2 % slower on a T = 1024 prefill
    p.pairmajor = (pp && p.xcd && (s.n * s.hkv) % 8 == 0) ? 1 : 0;

    if (ev_before)
        (void)hipEventRecord(ev_before, stream);
    using Kernel = void (*)(PrefillParams, RopeTable, QRot);
    static const Kernel kernels[2][2][5] = {
        {{prefill_attn_kernel<0, false, false>, prefill_attn_kernel<1, false, false>,
          prefill_attn_kernel<2, false, false>, prefill_attn_kernel<3, false, false>,
          prefill_attn_kernel<4, false, false>},
         {prefill_attn_kernel<0, true, false>, prefill_attn_kernel<1, true, false>,
          prefill_attn_kernel<2, true, false>, prefill_attn_kernel<3, true, false>,
          prefill_attn_kernel<4, true, false>}},
        {{prefill_attn_kernel<0, false, true>, prefill_attn_kernel<1, false, true>,
          prefill_attn_kernel<2, false, true>, prefill_attn_kernel<3, false, true>,
          prefill_attn_kernel<4, false, true>},
         {prefill_attn_kernel<0, true, true>, prefill_attn_kernel<1, true, true>,
          prefill_attn_kernel<2, true, true>, prefill_attn_kernel<3, true, true>,
          prefill_attn_kernel<4, true, true>}}};
    hipLaunchKernelGGL(kernels[pp ? 1 : 0][tab.cos_t ? 1 : 0][rot.h16], dim3((unsigned)blocks),
                       dim3(pp ? Lay<true>::NT : Lay<false>::NT), 0, stream, p, tab, rot);
    hipError_t err = hipGetLastError();
    if (ev_after)
        (void)hipEventRecord(ev_after, stream);
    return err;
}

} // namespace kvrope
