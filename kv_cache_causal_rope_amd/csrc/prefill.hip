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
// Work decomposition.  A workgroup owns one (unit, KV head, slice of the head group,
// block of 32 new tokens); each of its W waves owns one query head of that group and
// the 32 tokens.  The W waves share every K/V tile the workgroup stages in LDS, so a
// tile read from L2 feeds W*32 query rows.  Per 64-key tile a wave issues 32 MFMAs
// (v_mfma_f32_32x32x16_f16):
//   S^T (64 keys x 32 queries) = K . Q^T        -- 2 key blocks x 8 head-dim steps
//   O^T (128 dims x 32 queries) += V^T . P^T    -- 2 key blocks x 2 key steps x 4 dim blocks
// Working on S^T puts one query in each lane (lane l: query l % 32, half l / 32), so the
// row max is a per-lane reduction plus one cross-half exchange, and the probabilities
// are already in the B-operand layout of the PV product (the key order inside each
// 16-key step is permuted consistently on both operands, which the reduction allows).
// Softmax runs in fp32 in the log2 domain (exp2 of scale*log2(e)-scaled scores) with the
// usual running max / running sum rescaling.
//
// LDS (double buffered, one barrier per tile):
//   K tile: [64 keys][136 halves] (row padding keeps 16-byte reads of 16 consecutive
//           keys on distinct banks);
//   V tile: [16 key quads][128 dims][4 keys] with the dim index xor-swizzled inside
//           groups of 8, so the transposed A-operand reads (4 consecutive keys of one
//           dim) are contiguous and the transposing writes spread over banks.
// Grid order: heavier (later) token blocks first; when the number of (unit, KV head)
// pairs is a multiple of 8, all blocks of one pair go to the same XCD (blocks are dealt
// to the 8 XCDs round-robin) so its K/V stays in that XCD's L2.
#include "device_common.h"
#include "launch.h"

#include <math.h>

namespace kvrope {

namespace {

constexpr int KT = 64;          // keys per tile
constexpr int QB = 32;          // query tokens per wave
constexpr int KPITCH = 136;     // halves per K row in LDS
constexpr int K_STAGE = KT * KPITCH;
constexpr int V_STAGE = KT * kHeadDim;
constexpr int STAGE = K_STAGE + V_STAGE; // halves per pipeline stage
constexpr int LDS_BYTES = 2 * STAGE * 2;
constexpr int TASKS = KT / 4 * (kHeadDim / 8); // 256 loader tasks: (key quad, 16-byte chunk)

struct PrefillParams {
    const uint16_t *q;
    const uint16_t *ck;
    const uint16_t *cv;
    const int32_t *pos;
    const int32_t *lens;
    uint16_t *out;
    int n, t, hq, hkv, s_cap, max_hist;
    int W;       // waves (= query heads) per workgroup
    int slices;  // (hq / hkv) / W
    int tblocks; // ceil(t / 32)
    int xcd;     // XCD-aware block mapping
    float scale_log2;
};

__device__ inline int vswz(int dim) { return dim ^ ((dim >> 3) & 7); }

union U4H {
    uint4 v;
    uint16_t h[8];
};

template <int TPT>
struct TileRegs {
    uint4 k[TPT][4];
    uint4 v[TPT][4];
};

template <int TPT>
__device__ inline void load_tile(TileRegs<TPT> &r, const uint16_t *kbase, const uint16_t *vbase,
                                 int kb, int kend, int tid, int nthr)
{
#pragma unroll
    for (int tt = 0; tt < TPT; ++tt) {
        const int task = tid + tt * nthr;
        const int qd = task >> 4, mm = task & 15;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int key = kb + 4 * qd + rr;
            if (task < TASKS && key < kend) {
                r.k[tt][rr] = *reinterpret_cast<const uint4 *>(kbase + (int64_t)key * kHeadDim + 8 * mm);
                r.v[tt][rr] = *reinterpret_cast<const uint4 *>(vbase + (int64_t)key * kHeadDim + 8 * mm);
            } else {
                r.k[tt][rr] = make_uint4(0, 0, 0, 0);
                r.v[tt][rr] = make_uint4(0, 0, 0, 0);
            }
        }
    }
}

template <int TPT>
__device__ inline void store_tile(const TileRegs<TPT> &r, uint16_t *stage, int tid, int nthr)
{
    uint16_t *Ks = stage;
    uint16_t *Vs = stage + K_STAGE;
#pragma unroll
    for (int tt = 0; tt < TPT; ++tt) {
        const int task = tid + tt * nthr;
        if (task >= TASKS)
            continue;
        const int qd = task >> 4, mm = task & 15;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            *reinterpret_cast<uint4 *>(Ks + (4 * qd + rr) * KPITCH + 8 * mm) = r.k[tt][rr];
        U4H v0, v1, v2, v3;
        v0.v = r.v[tt][0];
        v1.v = r.v[tt][1];
        v2.v = r.v[tt][2];
        v3.v = r.v[tt][3];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int slot = vswz(8 * mm + e);
            uint2 quad;
            quad.x = (uint32_t)v0.h[e] | ((uint32_t)v1.h[e] << 16);
            quad.y = (uint32_t)v2.h[e] | ((uint32_t)v3.h[e] << 16);
            *reinterpret_cast<uint2 *>(Vs + (qd * kHeadDim + slot) * 4) = quad;
        }
    }
}

template <int TPT>
__global__ void __launch_bounds__(TPT == 1 ? 512 : 256) prefill_attn_kernel(PrefillParams p, RopeTable tab)
{
    extern __shared__ __align__(16) uint16_t lds[];

    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int c = lane & 31;  // query within the wave's block (S^T column)
    const int hh = lane >> 5; // lane half

    // ---- block -> (unit, KV head, head slice, token block)
    const int KP = p.n * p.hkv;
    const int S = p.slices;
    int kp, sl, tbr;
    const int b = blockIdx.x;
    if (p.xcd) {
        const int x = b & 7, slot = b >> 3;
        const int per_rank = (KP >> 3) * S;
        tbr = slot / per_rank;
        const int r = slot - tbr * per_rank;
        kp = x + 8 * (r / S);
        sl = r % S;
    } else {
        const int per_rank = KP * S;
        tbr = b / per_rank;
        const int r = b - tbr * per_rank;
        kp = r / S;
        sl = r % S;
    }
    const int tb = p.tblocks - 1 - tbr;
    const int u = kp / p.hkv, g = kp - (kp / p.hkv) * p.hkv;
    const int G = p.hq / p.hkv;
    const int h = g * G + sl * p.W + wave;
    const int i0 = tb * QB;
    const int i = i0 + c;
    const bool row_valid = i < p.t;

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
    const int kend = hist + min(i0 + QB, p.t);
    const int ntiles = (kend + KT - 1) / KT;
    const int qlimit = hist + i; // last visible key of this lane's query

    const uint16_t *kbase = p.ck + ((int64_t)u * p.hkv + g) * p.s_cap * kHeadDim;
    const uint16_t *vbase = p.cv + ((int64_t)u * p.hkv + g) * p.s_cap * kHeadDim;

    // ---- issue the first tile's loads before the q prologue
    TileRegs<TPT> regs;
    load_tile<TPT>(regs, kbase, vbase, 0, kend, tid, nthr);

    // ---- q prologue: load, rotate (fp32 trig with fp64 range reduction), round to f16
    half8 qop[8];
    {
        const uint16_t *qrow = p.q + (((int64_t)u * p.t + (row_valid ? i : 0)) * p.hq + h) * kHeadDim;
        const double posd = row_valid ? (double)p.pos[(int64_t)u * p.t + i] : 0.0;
        const float msc = (float)tab.mscale;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            U4H in;
            in.v = row_valid ? *reinterpret_cast<const uint4 *>(qrow + 16 * s + 8 * hh)
                             : make_uint4(0, 0, 0, 0);
            half8 hv;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int dim = 16 * s + 8 * hh + 2 * m;
                float x0 = h2f(in.h[2 * m]), x1 = h2f(in.h[2 * m + 1]);
                if (dim >= tab.off) {
                    const int j = (dim - tab.off) >> 1;
                    double rev = posd * tab.wrev[j];
                    rev -= floor(rev);
                    const float rf = (float)rev;
                    const float cs = __builtin_amdgcn_cosf(rf) * msc;
                    const float sn = __builtin_amdgcn_sinf(rf) * msc;
                    const float y0 = x0 * cs - x1 * sn;
                    const float y1 = x0 * sn + x1 * cs;
                    x0 = y0;
                    x1 = y1;
                }
                hv[2 * m] = (_Float16)x0;
                hv[2 * m + 1] = (_Float16)x1;
            }
            qop[s] = hv;
        }
    }

    store_tile<TPT>(regs, lds, tid, nthr);
    __syncthreads();

    floatx16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
        o[db] = floatx16{0.f};
    float m_run = -INFINITY, l_run = 0.f;

    for (int tile = 0; tile < ntiles; ++tile) {
        const int kb = tile * KT;
        const uint16_t *Ks = lds + (tile & 1) * STAGE;
        const uint16_t *Vs = Ks + K_STAGE;
        const bool more = tile + 1 < ntiles;
        if (more)
            load_tile<TPT>(regs, kbase, vbase, kb + KT, kend, tid, nthr);

        // S^T = K . Q^T for the tile's two 32-key blocks
        floatx16 sacc[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            sacc[sb] = floatx16{0.f};
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const half8 a = *reinterpret_cast<const half8 *>(Ks + (32 * sb + c) * KPITCH + 16 * s + 8 * hh);
                sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qop[s], sacc[sb], 0, 0, 0);
            }
        }

        // scale, causal mask, running max
        const bool need_mask = kb + KT - 1 > hist + i0;
        float mx = -INFINITY;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float sv = sacc[sb][r] * p.scale_log2;
                if (need_mask) {
                    const int key = kb + 32 * sb + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (key > qlimit)
                        sv = -INFINITY;
                }
                sacc[sb][r] = sv;
                mx = fmaxf(mx, sv);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float rs = 0.f;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pv = __builtin_amdgcn_exp2f(sacc[sb][r] - m_new);
                sacc[sb][r] = pv;
                rs += pv;
            }
        }
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < 4; ++db)
            o[db] *= alpha;

        // O^T += V^T . P^T
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                half8 pop;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    pop[j] = (_Float16)sacc[sb][8 * s2 + j];
                const int q1 = 8 * sb + 4 * s2 + hh;
                const int q2 = q1 + 2;
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const int slot = vswz(32 * db + c);
                    const half4 lo = *reinterpret_cast<const half4 *>(Vs + (q1 * kHeadDim + slot) * 4);
                    const half4 hi = *reinterpret_cast<const half4 *>(Vs + (q2 * kHeadDim + slot) * 4);
                    const half8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pop, o[db], 0, 0, 0);
                }
            }
        }

        if (more)
            store_tile<TPT>(regs, lds + ((tile + 1) & 1) * STAGE, tid, nthr);
        __syncthreads();
    }

    // ---- normalise and write: lane holds dims 32db + 8*(r/4) + 4*hh + r%4 of query c
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
    if (row_valid) {
        uint16_t *orow = p.out + (((int64_t)u * p.t + i) * p.hq + h) * kHeadDim;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int ig = 0; ig < 4; ++ig) {
                uint2 w;
                w.x = (uint32_t)f2h(o[db][4 * ig + 0] * inv) | ((uint32_t)f2h(o[db][4 * ig + 1] * inv) << 16);
                w.y = (uint32_t)f2h(o[db][4 * ig + 2] * inv) | ((uint32_t)f2h(o[db][4 * ig + 3] * inv) << 16);
                *reinterpret_cast<uint2 *>(orow + 32 * db + 8 * ig + 4 * hh) = w;
            }
        }
    }
}

int largest_divisor_at_most(int g, int cap)
{
    for (int w = cap < g ? cap : g; w >= 1; --w)
        if (g % w == 0)
            return w;
    return 1;
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
    const int G = s.hq / s.hkv;
    p.W = largest_divisor_at_most(G, 8);
    p.slices = G / p.W;
    p.tblocks = (s.t + QB - 1) / QB;
    const int KP = s.n * s.hkv;
    p.xcd = (KP % 8 == 0) ? 1 : 0;
    p.scale_log2 = (float)((double)s.scale * 1.4426950408889634);
    const int64_t blocks = (int64_t)KP * p.slices * p.tblocks;
    const int threads = 64 * p.W;
    const int tpt = (TASKS + threads - 1) / threads;

    if (ev_before)
        (void)hipEventRecord(ev_before, stream);
    if (tpt <= 1) {
        static bool attr = false;
        if (!attr) {
            (void)hipFuncSetAttribute(reinterpret_cast<const void *>(prefill_attn_kernel<1>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
            attr = true;
        }
        hipLaunchKernelGGL(prefill_attn_kernel<1>, dim3((unsigned)blocks), dim3(threads), LDS_BYTES,
                           stream, p, tab);
    } else if (tpt <= 2) {
        static bool attr = false;
        if (!attr) {
            (void)hipFuncSetAttribute(reinterpret_cast<const void *>(prefill_attn_kernel<2>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
            attr = true;
        }
        hipLaunchKernelGGL(prefill_attn_kernel<2>, dim3((unsigned)blocks), dim3(threads), LDS_BYTES,
                           stream, p, tab);
    } else {
        static bool attr = false;
        if (!attr) {
            (void)hipFuncSetAttribute(reinterpret_cast<const void *>(prefill_attn_kernel<4>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
            attr = true;
        }
        hipLaunchKernelGGL(prefill_attn_kernel<4>, dim3((unsigned)blocks), dim3(threads), LDS_BYTES,
                           stream, p, tab);
    }
    hipError_t err = hipGetLastError();
    if (ev_after)
        (void)hipEventRecord(ev_after, stream);
    return err;
}

} // namespace kvrope
