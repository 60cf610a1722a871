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
// takes 8 consecutive items (one per wave), so it spans at most two adjacent token
// blocks and shares every K/V tile it stages in LDS among 8 x 32 query rows; 8 waves
// also keep the 4 SIMDs of a CU evenly loaded for any group size.  Per 64-key tile a
// wave issues 32 MFMAs (v_mfma_f32_32x32x16_f16):
//   S^T (64 keys x 32 queries) = K . Q^T        -- 2 key blocks x 8 head-dim steps
//   O^T (128 dims x 32 queries) += V^T . P^T    -- 2 key blocks x 2 key steps x 4 dim blocks
// Working on S^T puts one query in each lane (lane l: query l % 32, half l / 32), so the
// row max is a per-lane reduction plus one cross-half exchange, and the probabilities
// are already in the B-operand layout of the PV product (the key order inside each
// 16-key step is permuted consistently on both operands, which the reduction allows).
// Softmax runs in fp32 in the log2 domain (exp2 of scale*log2(e)-scaled scores) with the
// running max / running sum rescaling, applied lazily: the accumulators are rescaled only
// when some lane's max grows by more than 2^8, so the probabilities stay <= 256 (exact
// enough in f16) and most tiles skip the 64 multiplies.  The causal mask is applied only
// on tiles that reach past the first query of the block.
//
// LDS (four stages, 32 KB each).
//   K tile: row-major [64 keys][256 B] with the 16-byte chunk index xor-swizzled by the
//           row (chunk ^ (key & 15)), so the S^T A-operand reads (16 B of 32 consecutive
//           keys) hit distinct banks.  It goes from HBM/L2 straight into LDS
//           (global_load_lds_dwordx4: lane L of a wave's load lands at byte 16 L of a
//           1 KB block; the swizzle picks which global chunk each lane fetches).
//   V tile: pre-transposed for the PV A-operand, [4 groups of 16 keys][2 lane halves]
//           [128 dims][8 keys]: the 8 keys of (group, half) are the ones that half's
//           lanes contribute to one 16-key MFMA step, so each A operand is a single
//           16-byte read; the dim index is xor-swizzled inside groups of 8 to spread the
//           transposing writes.  V rows are staged through registers (2 rows x 16 B per
//           thread) one phase pair before they are written.
// A tile's K is issued two tiles ahead of its first use and its V one tile ahead.  All
// per-lane LDS addresses are computed once; the phase loop is unrolled over the four
// stages so they are immediate offsets (and separate objects, so the compiler never
// waits on one stage before reading another), and the operand reads run four ahead of
// the MFMAs that consume them.
// Grid order: heavier (later) work first; when the number of (unit, KV head) pairs is a
// multiple of 8, all workgroups of one pair go to the same XCD (workgroups are dealt to
// the 8 XCDs round-robin) so its K/V stays in that XCD's L2.
#include "device_common.h"
#include "launch.h"

#include <math.h>

#include <type_traits>

namespace kvrope {

namespace {

constexpr int KT = 64;                 // keys per tile
constexpr int QB = 32;                 // query tokens per wave
constexpr int NW = 8;                  // waves per workgroup
constexpr int NT = NW * 64;            // threads per workgroup
constexpr int ROWB = kHeadDim * 2;     // bytes per K / V row
constexpr int TILE_B = KT * ROWB;      // 16 KB per tensor per stage
constexpr int STAGE_B = 2 * TILE_B;    // K tile, then V tile
constexpr float RESCALE_LOG2 = 8.f;    // lazy-rescale threshold (log2 units)


struct PrefillParams {
    const uint16_t *q;
    const uint16_t *ck;
    const uint16_t *cv;
    const int32_t *pos;
    const int32_t *lens;
    uint16_t *out;
    int n, t, hq, hkv, s_cap, max_hist;
    int G;       // query heads per KV head
    int items;   // tblocks * G work items per (unit, KV head)
    int wpk;     // workgroups per (unit, KV head) = ceil(items / 8)
    int xcd;     // XCD-aware block mapping
    float scale_log2;
};

// Workgroup barrier without the release fence of __syncthreads (which would drain every
// outstanding global load, including tiles prefetched for later phases).  LDS reads and
// writes complete before it (lgkmcnt); tile loads into LDS are waited for explicitly
// with vmcnt; the memory clobber keeps the compiler from moving memory ops across it.
__device__ inline void wg_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ inline int kswz(int key) { return key & 15; }

__device__ inline uint32_t lds_offset(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// Issue the K rows of one tile (keys kb .. kb+63, clamped to klast) into an LDS stage:
// wave w moves rows 8w .. 8w+7, 4 rows per instruction.  The loads are inline asm so
// the compiler does not track them; they are waited for explicitly (vmcnt) before the
// barrier that publishes the stage.
__device__ inline void dma_k(const uint16_t *kbase, int kb, int klast, const char *stage, int wave,
                             int lane)
{
    const uint32_t tdst = lds_offset(stage);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r0 = 8 * wave + 4 * i;
        const int row = r0 + (lane >> 4);
        const int gchunk = (lane & 15) ^ kswz(row);
        const int key = min(kb + row, klast);
        const uint16_t *src = kbase + (int64_t)key * kHeadDim + gchunk * 8;
        const uint32_t dst = __builtin_amdgcn_readfirstlane(tdst + (uint32_t)(r0 * ROWB));
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                     :
                     : "s"(dst), "v"(src)
                     : "memory", "m0");
    }
}

// V staging: thread tid owns lane half hh = (tid >> 6) & 1 of key group grp = tid >> 7,
// the 8-dim chunk m = (tid >> 2) & 15 and the key pair kq = tid & 3 of that half's list
// (keys 16 grp + 4 hh + {0, 1, 2, 3, 8, 9, 10, 11}).
struct VRegs {
    u32x4 a, b;
};

__device__ inline int vkey(int tid, int which)
{
    const int kq = tid & 3, hh = (tid >> 6) & 1, grp = tid >> 7;
    const int pos = 2 * kq + which;
    return 16 * grp + 4 * hh + (pos < 4 ? pos : pos + 4);
}

__device__ inline void load_v(VRegs &r, const uint16_t *vbase, int kb, int klast, int tid)
{
    const int m = (tid >> 2) & 15;
    r.a = ld16(vbase + (int64_t)min(kb + vkey(tid, 0), klast) * kHeadDim + 8 * m);
    r.b = ld16(vbase + (int64_t)min(kb + vkey(tid, 1), klast) * kHeadDim + 8 * m);
}

__device__ inline int vpos(int dim) { return dim ^ ((dim >> 3) & 7); }

__device__ inline void store_v(const VRegs &r, char *stage, int tid)
{
    const int kq = tid & 3, m = (tid >> 2) & 15, hh = (tid >> 6) & 1, grp = tid >> 7;
    char *vt = stage + TILE_B + (grp * 2 + hh) * kHeadDim * 16 + 4 * kq;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t x = r.a[e >> 1], y = r.b[e >> 1];
        const uint32_t w = (e & 1) ? __builtin_amdgcn_perm(y, x, 0x07060302u)
                                   : __builtin_amdgcn_perm(y, x, 0x05040100u);
        *reinterpret_cast<uint32_t *>(vt + vpos(8 * m + e) * 16) = w;
    }
}

__global__ void __launch_bounds__(NT) prefill_attn_kernel(PrefillParams p, RopeTable tab)
{
    // two pipeline stages as separate objects, so the compiler can tell that loads into
    // one stage never alias reads of the other (no spurious waits on the in-flight tile)
    __shared__ __align__(16) char lds_st0[STAGE_B];
    __shared__ __align__(16) char lds_st1[STAGE_B];
    __shared__ __align__(16) char lds_st2[STAGE_B];
    __shared__ __align__(16) char lds_st3[STAGE_B];
    __shared__ double wrev[kMaxPairs];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane & 31;  // query within the wave's block (S^T column)
    const int hh = lane >> 5; // lane half

    // ---- block -> (unit, KV head, workgroup rank); heavier workgroups first
    const int KP = p.n * p.hkv;
    int kp, rank;
    const int b = blockIdx.x;
    if (p.xcd) {
        const int x = b & 7, slot = b >> 3;
        const int per_x = KP >> 3;
        rank = slot / per_x;
        kp = x + 8 * (slot - rank * per_x);
    } else {
        rank = b / KP;
        kp = b - rank * KP;
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
    const bool row_valid = wave_valid && i < p.t;

    const int hist = p.lens ? p.lens[u] : 0;
    if (hist < 0 || hist > p.max_hist) {
        // invalid history length: no cache was written for this unit; report NaN
        if (row_valid && hh == 0) {
            uint16_t *orow = p.out + (((int64_t)u * p.t + i) * p.hq + h) * kHeadDim;
            for (int d = 0; d < kHeadDim; ++d)
                orow[d] = qnan16();
        }
        return;
    }
    const int tb_last = last_item / p.G;
    const int kend = hist + min((tb_last + 1) * QB, p.t); // keys the workgroup needs
    const int ntiles = (kend + KT - 1) / KT;
    const int kend_w = hist + min(i0 + QB, p.t);        // keys this wave needs
    const int qlimit = hist + i;                         // last visible key of the lane's query

    const uint16_t *kbase = p.ck + ((int64_t)u * p.hkv + g) * p.s_cap * kHeadDim;
    const uint16_t *vbase = p.cv + ((int64_t)u * p.hkv + g) * p.s_cap * kHeadDim;

    // ---- loads in flight, oldest first: rotation table, this lane's q row, tiles 0 and 1
    const double wr = tab.wrev[tid & (kMaxPairs - 1)];
    // rows past t read row t-1 (branch-free loads; their outputs are never written)
    const int iq = min(i, p.t - 1);
    const uint16_t *qrow = p.q + (((int64_t)u * p.t + iq) * p.hq + h) * kHeadDim;
    const int qpos = p.pos[(int64_t)u * p.t + iq];
    u32x4 qin[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
        qin[s] = ld16(qrow + 16 * s + 8 * hh);
    dma_k(kbase, 0, kend - 1, lds_st0, wave, lane);
    if (ntiles > 1)
        dma_k(kbase, KT, kend - 1, lds_st1, wave, lane);
    VRegs vr;
    load_v(vr, vbase, 0, kend - 1, tid);
    if (tid < kMaxPairs)
        wrev[tid] = wr;
    wg_barrier();

    // ---- q prologue: rotate (fp32 trig with fp64 range reduction), scale, round to f16
    const float sl2 = p.scale_log2;
    half8 qop[8];
    {
        const double posd = (double)qpos;
        const float msc = (float)tab.mscale;
        const int off = tab.off;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const u32x4 in = qin[s];
            u32x4 hv;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int dim = 16 * s + 8 * hh + 2 * m;
                const uint32_t w = in[m];
                float x0 = lo2f(w), x1 = hi2f(w);
                if (dim >= off) {
                    const int j = (dim - off) >> 1;
                    double rev = posd * wrev[j];
                    rev -= floor(rev);
                    const float rf = (float)rev;
                    const float cs = __builtin_amdgcn_cosf(rf) * msc;
                    const float sn = __builtin_amdgcn_sinf(rf) * msc;
                    const float y0 = x0 * cs - x1 * sn;
                    const float y1 = x0 * sn + x1 * cs;
                    x0 = y0;
                    x1 = y1;
                }
                // the softmax scale (log2 units) rides on q: S^T comes out pre-scaled
                hv[m] = pack2h(x0 * sl2, x1 * sl2);
            }
            qop[s] = __builtin_bit_cast(half8, hv);
        }
    }

    // ---- per-lane LDS byte addresses inside a stage
    int kaddr[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
        kaddr[s] = c * ROWB + (((2 * s + hh) ^ kswz(c)) << 4);
    int vaddr[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
        vaddr[db] = TILE_B + (hh * kHeadDim + vpos(32 * db + c)) * 16;

    // tile 0 (K and V) into stage 0; tile 1's V rows stay in registers until M(0)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    store_v(vr, lds_st0, tid);
    if (ntiles > 1)
        load_v(vr, vbase, KT, kend - 1, tid);
    wg_barrier();

    floatx16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
        o[db] = floatx16{0.f};
    // running max (log2 units) and the sum of the f16 probabilities, per query lane
    float m_run = 0.f, l_run = 0.f;
    bool first = true;
    floatx16 sacc[2];  // S^T of the current tile, as (score - running max)
    u32x4 pw[4];       // f16 probabilities of the previous tile (PV B operands)

    // Ping-pong: waves 0-3 (one per SIMD) and waves 4-7 run the same sequence of
    // phases, the second group one phase behind.  A wave's phases alternate
    //   M(j): PV of tile j-1, then S^T of tile j   (32 MFMAs)
    //   S(j): softmax of tile j                     (VALU)
    // so on every SIMD one wave keeps the matrix core busy while the other does its
    // softmax.  Each phase ends with a workgroup barrier.  Tile j sits in LDS stage
    // j % 4 from two tiles before its first use (S^T in M(j)) until its last (PV in
    // M(j+1) of the trailing group).
    const int grp = wave >> 2;
    const bool row_active = wave_valid;

    auto tile_active = [&](int j) { return row_active && j * KT < kend_w; };

    auto phase_m = [&](auto stg_c, int j) {
        constexpr int STG = decltype(stg_c)::value;
        const char *st = STG == 0 ? lds_st0 : (STG == 1 ? lds_st1 : (STG == 2 ? lds_st2 : lds_st3));
        const char *stp = STG == 0 ? lds_st3 : (STG == 1 ? lds_st0 : (STG == 2 ? lds_st1 : lds_st2));
        char *st2 = STG == 0 ? lds_st2 : (STG == 1 ? lds_st3 : (STG == 2 ? lds_st0 : lds_st1));
        char *st1 = STG == 0 ? lds_st1 : (STG == 1 ? lds_st2 : (STG == 2 ? lds_st3 : lds_st0));
        // tile j+1: its V rows (loaded one phase pair ago) into its stage; all of this
        // wave's loads are complete afterwards, including its K share of tile j+1
        if (j + 1 < ntiles) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            store_v(vr, st1, tid);
        }
        // tile j+2: K straight into its stage, V rows into registers
        // (V first: the compiler's own wait before reusing vr must not cover the K loads)
        if (j + 2 < ntiles) {
            load_v(vr, vbase, (j + 2) * KT, kend - 1, tid);
            dma_k(kbase, (j + 2) * KT, kend - 1, st2, wave, lane);
        }
        // the matrix-core phase outranks the other group's softmax for issue slots
        __builtin_amdgcn_s_setprio(1);

        // O^T += V^T . P^T for tile j-1: 16 MFMAs (key step g = 2 sb + s2, dim block db),
        // V^T operands read four ahead
        if (j >= 1 && tile_active(j - 1)) {
            half8 vq[4];
#pragma unroll
            for (int x = 0; x < 4; ++x)
                vq[x] = *reinterpret_cast<const half8 *>(stp + vaddr[x & 3] + (x >> 2) * 2 * kHeadDim * 16);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                const int gi = x >> 2, db = x & 3;
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vq[x & 3], __builtin_bit_cast(half8, pw[gi]),
                                                               o[db], 0, 0, 0);
                if (x + 4 < 16)
                    vq[x & 3] = *reinterpret_cast<const half8 *>(stp + vaddr[(x + 4) & 3] +
                                                                  ((x + 4) >> 2) * 2 * kHeadDim * 16);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // S^T = K . Q^T for tile j: 16 MFMAs, K operands read four ahead; the
        // accumulators start at -m_run so S^T leaves the MFMAs as (score - max)
        if (j < ntiles && tile_active(j)) {
            // the two key blocks' accumulation chains alternate, so consecutive MFMAs
            // never wait on each other's results
            half8 kq[4];
#pragma unroll
            for (int x = 0; x < 4; ++x)
                kq[x] = *reinterpret_cast<const half8 *>(st + kaddr[x >> 1] + (x & 1) * 32 * ROWB);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                const int sb = x & 1, s = x >> 1;
                sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    kq[x & 3], qop[s], s == 0 ? floatx16(-m_run) : sacc[sb], 0, 0, 0);
                if (x + 4 < 16)
                    kq[x & 3] = *reinterpret_cast<const half8 *>(st + kaddr[(x + 4) >> 1] + ((x + 4) & 1) * 32 * ROWB);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        wg_barrier();
    };

    auto phase_s = [&](int j) {
        if (tile_active(j)) {
            const int kb = j * KT;
            // causal mask (only on tiles reaching past the block's first query)
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
            float mx = -INFINITY;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    mx = fmaxf(mx, sacc[sb][r]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32)); // max over the tile of (score - m_run)
            // The first tile sets the max exactly; later tiles move it (and rescale the
            // accumulators) only when some lane's max grows by more than 2^8.
            if (first || __any(mx > RESCALE_LOG2)) {
                const float d = first ? mx : fmaxf(mx, 0.f);
                const float alpha = __builtin_amdgcn_exp2f(-d);
                if (!first) {
                    l_run *= alpha;
#pragma unroll
                    for (int db = 0; db < 4; ++db)
                        o[db] *= alpha;
                }
                m_run += d;
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        sacc[sb][r] -= d;
                }
                first = false;
            }
            // probabilities, packed to f16 pairs (the PV operand) and summed as used
            float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int r = 8 * (x & 1) + 2 * jj;
                    const floatx2 pf = {__builtin_amdgcn_exp2f(sacc[x >> 1][r]),
                                        __builtin_amdgcn_exp2f(sacc[x >> 1][r + 1])};
                    const half2v ph = __builtin_convertvector(pf, half2v);
                    pw[x][jj] = __builtin_bit_cast(uint32_t, ph);
                    if (jj & 1)
                        ls1 = __builtin_amdgcn_fdot2(ph, half2v{(_Float16)1.f, (_Float16)1.f}, ls1, false);
                    else
                        ls0 = __builtin_amdgcn_fdot2(ph, half2v{(_Float16)1.f, (_Float16)1.f}, ls0, false);
                }
            }
            l_run += ls0 + ls1;
        }
        wg_barrier();
    };

    if (grp == 1)
        wg_barrier(); // the trailing group starts one phase late
    for (int j0 = 0; j0 <= ntiles; j0 += 4) {
        phase_m(std::integral_constant<int, 0>{}, j0);
        if (j0 < ntiles) {
            phase_s(j0);
            phase_m(std::integral_constant<int, 1>{}, j0 + 1);
            if (j0 + 1 < ntiles) {
                phase_s(j0 + 1);
                phase_m(std::integral_constant<int, 2>{}, j0 + 2);
                if (j0 + 2 < ntiles) {
                    phase_s(j0 + 2);
                    phase_m(std::integral_constant<int, 3>{}, j0 + 3);
                    if (j0 + 3 < ntiles)
                        phase_s(j0 + 3);
                }
            }
        }
    }
    if (grp == 0)
        wg_barrier(); // same barrier count for both groups

    // ---- normalise and write: lane holds dims 32db + 8*(r/4) + 4*hh + r%4 of query c
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
    if (row_valid) {
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

} // namespace

hipError_t launch_prefill_attention(const uint16_t *q, const uint16_t *cache_k,
                                    const uint16_t *cache_v, const int32_t *positions,
                                    const int32_t *lens, uint16_t *out, const PrefillShape &s,
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
    p.out = out;
    p.n = s.n;
    p.t = s.t;
    p.hq = s.hq;
    p.hkv = s.hkv;
    p.s_cap = s.s_cap;
    p.max_hist = s.max_hist;
    p.G = s.hq / s.hkv;
    const int tblocks = (s.t + QB - 1) / QB;
    p.items = tblocks * p.G;
    p.wpk = (p.items + NW - 1) / NW;
    const int KP = s.n * s.hkv;
    p.xcd = (KP % 8 == 0) ? 1 : 0;
    p.scale_log2 = (float)((double)s.scale * 1.4426950408889634);
    const int64_t blocks = (int64_t)KP * p.wpk;

    if (ev_before)
        (void)hipEventRecord(ev_before, stream);
    hipLaunchKernelGGL(prefill_attn_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, p, tab);
    hipError_t err = hipGetLastError();
    if (ev_after)
        (void)hipEventRecord(ev_after, stream);
    return err;
}

} // namespace kvrope
