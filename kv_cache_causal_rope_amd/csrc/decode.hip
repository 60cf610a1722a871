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
// Kernel 1 (decode_split_kernel): a workgroup of 4 waves owns (unit, KV head, slice of
// up to GS query heads of the group, chunk of `chunk` keys).  The chunk is streamed from
// HBM once and serves all GS heads:
//   * S^T (32 keys x 32 query columns) = K . Q^T on v_mfma_f32_32x32x16_f16, the K
//     operand loaded straight from the cache (16 bytes per lane per step, each row read
//     as contiguous 32-byte pieces); columns >= GS are zero;
//   * fp32 online softmax per query column (log2 domain);
//   * O += P V on the VALU: lane l owns head dims 2l, 2l+1, reads one 4-byte word of each
//     V row (a wave reads whole 256-byte rows) and takes the probabilities from LDS.
//   The four waves' (max, sum, output) states are merged through LDS and written as one
//   fp32 partial per (unit, head, chunk) to the caller's workspace.
// Kernel 2 (decode_combine_kernel): per (unit, head), merges the chunks in a fixed order
// (M = max m_s, L = sum l_s 2^(m_s - M), O = sum o_s 2^(m_s - M) / L), so results are
// deterministic.  No float atomics anywhere.
#include "device_common.h"
#include "launch.h"
#include "rope_device.h"

#include <math.h>

namespace kvrope {

namespace {

constexpr int KB = 32;          // keys per MFMA block
constexpr int NWAVES = 4;
constexpr int PART = kHeadDim + 2; // floats per partial: m, l, o[128]

struct DecodeParams {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    const int32_t *pos;
    const int32_t *lens;
    uint16_t *ck;
    uint16_t *cv;
    float *ws;
    int n, hq, hkv, s_cap, max_len;
    int chunk;   // keys per workgroup (multiple of 128)
    int nsplit;  // chunks per unit at max_len
    int slices;  // ceil(G / GS)
    float scale_log2;
};

union U4H {
    uint4 v;
    uint16_t h[8];
};

template <int GS>
struct __align__(16) DecodeSmem {
    double cs[kMaxPairs];
    double sn[kMaxPairs];
    uint16_t qh[GS][kHeadDim];
    uint16_t knew[kHeadDim];
    uint16_t vnew[kHeadDim];
    float p[NWAVES][KB][GS];
    float alpha[NWAVES][GS];
    float wm[NWAVES][GS];
    float wl[NWAVES][GS];
    float wo[NWAVES][GS][kHeadDim];
};

template <int GS>
__global__ void __launch_bounds__(256) decode_split_kernel(DecodeParams p, RopeTable tab)
{
    __shared__ DecodeSmem<GS> sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int c = lane & 31;
    const int hh = lane >> 5;

    // block -> (unit, kv head, slice, split); split is the fastest index
    int b = blockIdx.x;
    const int split = b % p.nsplit;
    b /= p.nsplit;
    const int sl = b % p.slices;
    b /= p.slices;
    const int g = b % p.hkv;
    const int u = b / p.hkv;
    const int G = p.hq / p.hkv;
    const int h0 = g * G + sl * GS; // first query head of this slice
    const int nh = min(GS, G - sl * GS);

    const int len = p.lens[u];
    const bool bad = len < 0 || len > p.max_len;
    const int nk = len + 1;
    const int k0 = split * p.chunk;
    if (bad) {
        // no cache write for this unit; the combine kernel emits NaN
        return;
    }
    if (k0 >= nk)
        return; // chunk beyond this unit's keys: the combine kernel ignores it
    const int k1 = min(k0 + p.chunk, nk);
    const bool has_new = (len >= k0 && len < k1);

    // ---- prologue: the factors of each rotated pair once (fp64), shared by the q heads
    // and k, by the routine every kernel that writes K rows uses (or the caller's table
    // entries of the token's position; NaN when the table does not cover it)
    const int posi = p.pos[u];
    if (tid < tab.n_pairs) {
        double co, s;
        pair_factor(tid, posi, tab, rope_set(tab, u), co, s);
        sm.cs[tid] = co;
        sm.sn[tid] = s;
    }
    __syncthreads();
    {
#pragma clang fp contract(off)
        // Pair `it` of a head: rotated pair j = it - off/2 when it >= off/2, with dims
        // (off + 2j, off + 2j + 1) or, half-split, (off + j, off + j + n_pairs); below
        // off/2 the pair (2 it, 2 it + 1) is copied.
        const int half_d = kHeadDim / 2;
        auto dims = [&](int it, int &da, int &db) -> int {
            const int j = it - (tab.off >> 1);
            if (j < 0) {
                da = 2 * it;
                db = da + 1;
            } else {
                da = tab.half ? tab.off + j : tab.off + 2 * j;
                db = tab.half ? da + tab.n_pairs : da + 1;
            }
            return j;
        };
        // rotated q heads of this slice -> LDS (f16, nearest even); one thread per pair
        for (int it = tid; it < GS * half_d; it += 256) {
            const int hl = it / half_d, pr = it % half_d;
            int da, db;
            const int j = dims(pr, da, db);
            uint16_t y0 = 0, y1 = 0;
            if (hl < nh) {
                const uint16_t *qr = p.q + ((int64_t)u * p.hq + h0 + hl) * kHeadDim;
                const uint16_t a0 = qr[da], a1 = qr[db];
                y0 = a0;
                y1 = a1;
                if (j >= 0) {
                    const double x0 = h2d(a0), x1 = h2d(a1);
                    y0 = f64_to_f16_rne(x0 * sm.cs[j] - x1 * sm.sn[j]);
                    y1 = f64_to_f16_rne(x0 * sm.sn[j] + x1 * sm.cs[j]);
                }
            }
            sm.qh[hl][da] = y0;
            sm.qh[hl][db] = y1;
        }
        if (has_new && tid < half_d) {
            int da, db;
            const int j = dims(tid, da, db);
            const uint16_t *kr = p.k + ((int64_t)u * p.hkv + g) * kHeadDim;
            const uint16_t *vr = p.v + ((int64_t)u * p.hkv + g) * kHeadDim;
            uint16_t y0 = kr[da], y1 = kr[db];
            if (j >= 0) {
                const double x0 = h2d(y0), x1 = h2d(y1);
                y0 = f64_to_f16_rne(x0 * sm.cs[j] - x1 * sm.sn[j]);
                y1 = f64_to_f16_rne(x0 * sm.sn[j] + x1 * sm.cs[j]);
            }
            sm.knew[da] = y0;
            sm.knew[db] = y1;
            sm.vnew[da] = vr[da];
            sm.vnew[db] = vr[db];
            if (sl == 0) {
                // append: row len of this unit's KV head g
                const int64_t row = (((int64_t)u * p.hkv + g) * p.s_cap + len) * kHeadDim;
                p.ck[row + da] = y0;
                p.ck[row + db] = y1;
                p.cv[row + da] = vr[da];
                p.cv[row + db] = vr[db];
            }
        }
    }
    __syncthreads();

    // ---- B operands (Q^T): lane (c, hh) holds q_hat[c][16 s + 8 hh .. +7], zero for c >= nh
    half8 qop[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        if (c < nh)
            qop[s] = *reinterpret_cast<const half8 *>(&sm.qh[c < GS ? c : 0][16 * s + 8 * hh]);
        else
            qop[s] = half8{0};
    }

    const uint16_t *kbase = p.ck + ((int64_t)u * p.hkv + g) * p.s_cap * kHeadDim;
    const uint16_t *vbase = p.cv + ((int64_t)u * p.hkv + g) * p.s_cap * kHeadDim;

    float m_run = -INFINITY, l_run = 0.f; // per query column c (lane pair shares m)
    float o0[GS], o1[GS];                 // dims 2*lane, 2*lane+1 for each head
#pragma unroll
    for (int hl = 0; hl < GS; ++hl) {
        o0[hl] = 0.f;
        o1[hl] = 0.f;
    }

    for (int kb = k0 + wave * KB; kb < k1; kb += NWAVES * KB) {
        // K operand: key kb + c, dims 16 s + 8 hh .. +7
        const int kkey = kb + c;
        half8 kop[8];
        if (kkey < k1 && kkey != len) {
            const uint4 *src = reinterpret_cast<const uint4 *>(kbase + (int64_t)kkey * kHeadDim + 8 * hh);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const uint4 w = src[2 * s];
                kop[s] = *reinterpret_cast<const half8 *>(&w);
            }
        } else if (kkey == len) {
#pragma unroll
            for (int s = 0; s < 8; ++s)
                kop[s] = *reinterpret_cast<const half8 *>(&sm.knew[16 * s + 8 * hh]);
        } else {
#pragma unroll
            for (int s = 0; s < 8; ++s)
                kop[s] = half8{0};
        }
        // V words: lane owns dims 2*lane, 2*lane+1 of each of the 32 rows
        uint32_t vw[KB];
#pragma unroll
        for (int r = 0; r < KB; ++r) {
            const int key = kb + r;
            if (key < k1 && key != len)
                vw[r] = *reinterpret_cast<const uint32_t *>(vbase + (int64_t)key * kHeadDim + 2 * lane);
            else if (key == len)
                vw[r] = *reinterpret_cast<const uint32_t *>(&sm.vnew[2 * lane]);
            else
                vw[r] = 0u;
        }

        floatx16 sacc = floatx16{0.f};
#pragma unroll
        for (int s = 0; s < 8; ++s)
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop[s], qop[s], sacc, 0, 0, 0);

        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            float sv = sacc[r] * p.scale_log2;
            if (key >= k1)
                sv = -INFINITY;
            sacc[r] = sv;
            mx = fmaxf(mx, sv);
        }
        mx = half_max(mx);
        const float m_new = fmaxf(m_run, mx); // finite: key kb < k1 is always valid
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float rs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pv = __builtin_amdgcn_exp2f(sacc[r] - m_new);
            rs += pv;
            if (c < GS)
                sm.p[wave][8 * (r >> 2) + 4 * hh + (r & 3)][c] = pv;
        }
        l_run = l_run * alpha + rs;
        m_run = m_new;
        if (c < GS && hh == 0)
            sm.alpha[wave][c] = alpha;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // O = alpha O + P V for this lane's two dims
#pragma unroll
        for (int hl = 0; hl < GS; ++hl) {
            const float a = sm.alpha[wave][hl];
            o0[hl] *= a;
            o1[hl] *= a;
        }
#pragma unroll
        for (int r = 0; r < KB; ++r) {
            const float v0 = h2f((uint16_t)(vw[r] & 0xffffu));
            const float v1 = h2f((uint16_t)(vw[r] >> 16));
#pragma unroll
            for (int hl = 0; hl < GS; ++hl) {
                const float pr = sm.p[wave][r][hl];
                o0[hl] += pr * v0;
                o1[hl] += pr * v1;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- merge the four waves' states (a wave without keys has m = -inf, l = 0, o = 0)
    const float l_tot = half_sum(l_run);
    if (c < GS && hh == 0) {
        sm.wm[wave][c] = m_run;
        sm.wl[wave][c] = l_tot;
    }
#pragma unroll
    for (int hl = 0; hl < GS; ++hl) {
        sm.wo[wave][hl][2 * lane] = o0[hl];
        sm.wo[wave][hl][2 * lane + 1] = o1[hl];
    }
    __syncthreads();
    for (int it = tid; it < nh * kHeadDim; it += 256) {
        const int hl = it / kHeadDim, d = it % kHeadDim;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w)
            M = fmaxf(M, sm.wm[w][hl]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) {
            const float f = (sm.wm[w][hl] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sm.wm[w][hl] - M);
            L += sm.wl[w][hl] * f;
            O += sm.wo[w][hl][d] * f;
        }
        float *part = p.ws + (((int64_t)u * p.hq + h0 + hl) * p.nsplit + split) * PART;
        part[2 + d] = O;
        if (d == 0) {
            part[0] = M;
            part[1] = L;
        }
    }
}

// Merge the chunks of each (unit, head) in index order; one wave per (unit, head).
__global__ void __launch_bounds__(256) decode_combine_kernel(const float *__restrict__ ws,
                                                             const int32_t *__restrict__ lens,
                                                             uint16_t *__restrict__ out, int n,
                                                             int hq, int nsplit, int chunk,
                                                             int max_len)
{
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
    const int ns = (len + 1 + chunk - 1) / chunk;
    const float *part = ws + (int64_t)wid * nsplit * PART;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s)
        M = fmaxf(M, part[s * PART]);
    float L = 0.f, O0 = 0.f, O1 = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float *ps = part + s * PART;
        const float f = __builtin_amdgcn_exp2f(ps[0] - M);
        L += ps[1] * f;
        O0 += ps[2 + 2 * lane] * f;
        O1 += ps[3 + 2 * lane] * f;
    }
    const float inv = 1.f / L;
    orow[2 * lane] = f2h(O0 * inv);
    orow[2 * lane + 1] = f2h(O1 * inv);
}

int decode_chunk(int n, int hkv, int slices, int max_len)
{
    // keys per workgroup: a multiple of 128 (4 waves x 32 keys), the largest in the list
    // that still gives the grid >= 2048 workgroups when the cache allows it.  The list
    // tops out at 1536 rather than 2048: on MI355X, 2048-key chunks streamed the
    // 32k-row caches about 15% slower than 1408..1664-key chunks, which measured best
    // on both the 4k-row and the 32k-row caches.
    static const int kChunks[] = {1536, 1024, 768, 512, 384, 256, 128};
    const int nk = max_len + 1;
    const int64_t pairs = (int64_t)n * hkv * slices;
    for (const int chunk : kChunks)
        if (pairs * ((nk + chunk - 1) / chunk) >= 2048)
            return chunk;
    return 128;
}

// query heads per workgroup: the whole group up to 8 (no idle head slots in the VALU part)
int slice_width(int G) { return G >= 8 ? 8 : G; }

} // namespace

size_t decode_workspace_bytes(int n, int hq, int hkv, int max_len)
{
    const int G = hq / hkv;
    const int gs = slice_width(G);
    const int slices = (G + gs - 1) / gs;
    const int chunk = decode_chunk(n, hkv, slices, max_len);
    const int nsplit = (max_len + 1 + chunk - 1) / chunk;
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
    const int G = s.hq / s.hkv;
    const int gs = slice_width(G);
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
    p.s_cap = s.s_cap;
    p.max_len = s.max_len;
    p.slices = (G + gs - 1) / gs;
    p.chunk = decode_chunk(s.n, s.hkv, p.slices, s.max_len);
    p.nsplit = (s.max_len + 1 + p.chunk - 1) / p.chunk;
    p.scale_log2 = (float)((double)s.scale * 1.4426950408889634);
    const int64_t blocks = (int64_t)s.n * s.hkv * p.slices * p.nsplit;

    if (ev_before)
        (void)hipEventRecord(ev_before, stream);
    using Kernel = void (*)(DecodeParams, RopeTable);
    static const Kernel kernels[8] = {decode_split_kernel<1>, decode_split_kernel<2>, decode_split_kernel<3>,
                                      decode_split_kernel<4>, decode_split_kernel<5>, decode_split_kernel<6>,
                                      decode_split_kernel<7>, decode_split_kernel<8>};
    hipLaunchKernelGGL(kernels[gs - 1], dim3((unsigned)blocks), dim3(256), 0, stream, p, tab);
    hipError_t err = hipGetLastError();
    if (ev_after)
        (void)hipEventRecord(ev_after, stream);
    if (err != hipSuccess)
        return err;
    const int64_t waves = (int64_t)s.n * s.hq;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)((waves * 64 + 255) / 256)), dim3(256), 0,
                       stream, p.ws, lens, out, s.n, s.hq, p.nsplit, p.chunk, s.max_len);
    return hipGetLastError();
}

} // namespace kvrope
