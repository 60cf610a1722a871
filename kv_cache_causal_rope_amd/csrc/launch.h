// launch.h -- internal launchers of libkvrope (host side of each kernel file).
// All sizes were validated by api.cpp before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvrope {

struct RopeTable;

// rows = units x t (row r belongs to unit r / t, whose parameter set it rotates with)
hipError_t launch_rope_inplace(uint16_t *x, const int32_t *positions, int64_t rows, int t, int h,
                               const RopeTable &tab, hipStream_t stream);

hipError_t launch_append(uint16_t *cache_k, uint16_t *cache_v, const uint16_t *k,
                         const uint16_t *v, const int32_t *lens, int max_len, int n, int t,
                         int hkv, int s_cap, hipStream_t stream);

// new_lens may be NULL (t rows per unit); rows i >= new_lens[u] are not appended
hipError_t launch_rope_append(uint16_t *cache_k, uint16_t *cache_v, const uint16_t *k,
                              const uint16_t *v, const int32_t *positions, const int32_t *lens,
                              const int32_t *new_lens, int max_len, int n, int t, int hkv, int s_cap,
                              const RopeTable &tab, hipStream_t stream);

struct PrefillShape {
    int n, t, hq, hkv, s_cap, max_hist;
    float scale;
};

// Causal GQA flash attention over the caches (rows already appended), with q rotated in
// the kernel's prologue.  lens may be NULL (all zero); new_lens may be NULL (t each).
hipError_t launch_prefill_attention(const uint16_t *q, const uint16_t *cache_k,
                                    const uint16_t *cache_v, const int32_t *positions,
                                    const int32_t *lens, const int32_t *new_lens, uint16_t *out,
                                    const PrefillShape &s,
                                    const RopeTable &tab, hipStream_t stream,
                                    hipEvent_t ev_before, hipEvent_t ev_after);

// Fused QKV projection (C = x . w^T, w [(hq + 2 hkv) * 128, hidden] per unit or shared):
// q heads written to q, k heads rotated and v heads copied into cache rows lens[u] + i.
hipError_t launch_qkv_projection(const uint16_t *x, const uint16_t *w, int64_t w_stride, const int32_t *positions,
                                 uint16_t *q, uint16_t *cache_k, uint16_t *cache_v, const int32_t *lens,
                                 int max_len, int n, int t, int hidden, int hq, int hkv, int s_cap,
                                 const RopeTable &tab, hipStream_t stream);

// Output projection: out = attn . w^T + residual, w [hidden, in_features] per unit or shared.
hipError_t launch_out_projection(const uint16_t *attn, const uint16_t *w, int64_t w_stride, const uint16_t *residual,
                                 uint16_t *out, int n, int t, int in_features, int hidden, hipStream_t stream);

struct DecodeShape {
    int n, hq, hkv, s_cap, max_len;
    float scale;
};

// Bytes of fp32 workspace the split-key decode needs for this shape.
size_t decode_workspace_bytes(int n, int hq, int hkv, int max_len);
// Keys per chunk (at most) the split-key decode cuts a unit's keys into for this shape.
int decode_chunk_keys(int n, int hq, int hkv, int max_len);

hipError_t launch_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const int32_t *positions, uint16_t *cache_k, uint16_t *cache_v,
                         const int32_t *lens, uint16_t *out, const DecodeShape &s,
                         const RopeTable &tab, void *workspace, hipStream_t stream,
                         hipEvent_t ev_before, hipEvent_t ev_after);

} // namespace kvrope
