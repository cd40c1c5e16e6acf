// Top-K selection of one router row by one full wave.
#pragma once

#include "common.h"

namespace moe {

// A slot's expert for the other waves of the workgroup: one 64-bit LDS word
// holding a published mark (1) above the expert index, stored at once (an
// aligned 64-bit LDS access is single-copy atomic), so a reader sees either
// the word it was reset to (0, before the workgroup's first barrier) or the
// expert. Nothing is ordered between two different words.
__device__ __forceinline__ void publish_slot(uint64_t *slot, int e) {
    __hip_atomic_store(slot, (1ull << 32) | (uint32_t)e, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Top-K of one router row by one full wave, then the softmax over the K in
// slot order (results to LDS). Lane l holds experts l, l + 64, ...; it sorts
// its NL values once (logit descending, expert ascending), so each of the K
// rounds is one wave max of the lanes' heads, one wave min over the heads
// that equal it (the lowest expert index wins ties), and a shift in the
// winning lane. +0 and -0 compare equal, as floats do.
// COHERENT: the logits were written by other workgroups of the same kernel
// and are read with device-coherent (sc1) loads.
// Selection on values already in registers: lane l holds experts l, l + 64,
// ... (v = -inf, ix = INT_MAX beyond E). Results (slot order) to ids/wts.
// With PUB, slot j's expert is published as soon as its round ends, in
// one 64-bit LDS word slots[j] (see publish_slot; ids is then not written),
// so other waves of the workgroup can start on slot j while the later
// rounds run.
template <int NL, bool PUB = false>
__device__ __forceinline__ void topk_select_n(float (&v)[NL], int (&ix)[NL], int K, int lane,
                                              int32_t *ids, float *wts,
                                              uint64_t *slots = nullptr) {
    // odd-even transposition sort of the lane's NL entries
#pragma unroll
    for (int r = 0; r < NL; ++r)
#pragma unroll
        for (int i = r & 1; i + 1 < NL; i += 2)
            if (v[i + 1] > v[i] || (v[i + 1] == v[i] && ix[i + 1] < ix[i])) {
                const float tv = v[i];
                v[i] = v[i + 1];
                v[i + 1] = tv;
                const int ti = ix[i];
                ix[i] = ix[i + 1];
                ix[i + 1] = ti;
            }
    float my_v = 0.0f, v0 = 0.0f;
    int my_id = 0;
    for (int j = 0; j < K; ++j) {
        const float vmax = wave_allmax(v[0]);
        const int win = wave_allmin_i(v[0] == vmax ? ix[0] : 0x7FFFFFFF);
        if (ix[0] == win) {
#pragma unroll
            for (int i = 0; i + 1 < NL; ++i) {
                v[i] = v[i + 1];
                ix[i] = ix[i + 1];
            }
            v[NL - 1] = -INFINITY;
            ix[NL - 1] = 0x7FFFFFFF;
        }
        if (j == 0) v0 = vmax;
        if (lane == j) {
            my_id = win;
            my_v = vmax;
        }
        if (PUB && lane == 0) publish_slot(slots + j, win);
    }
    const float ex = lane < K ? expf(my_v - v0) : 0.0f;
    float sum = 0.0f;
    for (int j = 0; j < K; ++j) sum += readlane_f(ex, j);
    if (lane < K) {
        if (!PUB) ids[lane] = my_id;
        wts[lane] = ex / sum;
    }
}

template <bool COHERENT, int NL>
__device__ inline void topk_row_n(const float *lr, int E, int K, int lane, int32_t *ids,
                                  float *wts) {
    float v[NL];
    int ix[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int e = lane + WAVE * i;
        if (e < E) {
            v[i] = COHERENT ? __hip_atomic_load(lr + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                            : lr[e];
            ix[i] = e;
        } else {
            v[i] = -INFINITY;
            ix[i] = 0x7FFFFFFF;
        }
    }
    topk_select_n<NL>(v, ix, K, lane, ids, wts);
}

// When every logit is a bf16 value (no bias, bf16 rounding on), a logit
// and its expert index pack into one 32-bit key whose unsigned order is
// (logit descending, expert ascending): each round is then a single wave
// max. +0 and -0 map to the same key.
__device__ __forceinline__ uint32_t bf16_order_key(float v, int e) {
    uint32_t b = __float_as_uint(v) >> 16;
    if (b == 0x8000u) b = 0;                       // -0 ranks as +0
    const uint32_t o = (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
    return (o << 16) | (uint32_t)(0xFFFF - e);
}

__device__ __forceinline__ uint32_t wave_allmax_u32(uint32_t v) {
    v = max(v, (uint32_t)dpp_i<DPP_XOR1>((int)v));
    v = max(v, (uint32_t)dpp_i<DPP_XOR2>((int)v));
    v = max(v, (uint32_t)dpp_i<DPP_HALF_MIRROR>((int)v));
    v = max(v, (uint32_t)dpp_i<DPP_MIRROR>((int)v));
    return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                   (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
               max((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                   (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// Selection on packed keys already in registers (0 beyond E); PUB as for
// topk_select_n.
template <int NL, bool PUB = false>
__device__ __forceinline__ void topk_select_packed(uint32_t (&k)[NL], int K, int lane,
                                                   int32_t *ids, float *wts,
                                                   uint64_t *slots = nullptr) {
#pragma unroll
    for (int r = 0; r < NL; ++r)
#pragma unroll
        for (int i = r & 1; i + 1 < NL; i += 2)
            if (k[i + 1] > k[i]) {
                const uint32_t tk = k[i];
                k[i] = k[i + 1];
                k[i + 1] = tk;
            }
    uint32_t my_k = 0, k0 = 0;
    for (int j = 0; j < K; ++j) {
        const uint32_t best = wave_allmax_u32(k[0]);
        if (k[0] == best) {
#pragma unroll
            for (int i = 0; i + 1 < NL; ++i) k[i] = k[i + 1];
            k[NL - 1] = 0u;
        }
        if (j == 0) k0 = best;
        if (lane == j) my_k = best;
        if (PUB && lane == 0) publish_slot(slots + j, (int)(0xFFFF - (best & 0xFFFFu)));
    }
    // back to the logit values: undo the order map of the top 16 bits
    auto val = [](uint32_t key) {
        const uint32_t o = key >> 16;
        const uint32_t b = (o & 0x8000u) ? (o & 0x7FFFu) : (~o & 0xFFFFu);
        return __uint_as_float(b << 16);
    };
    const float ex = lane < K ? expf(val(my_k) - val(k0)) : 0.0f;
    float sum = 0.0f;
    for (int j = 0; j < K; ++j) sum += readlane_f(ex, j);
    if (lane < K) {
        if (!PUB) ids[lane] = (int)(0xFFFF - (my_k & 0xFFFFu));
        wts[lane] = ex / sum;
    }
}

template <bool COHERENT, int NL>
__device__ inline void topk_row_packed(const float *lr, int E, int K, int lane, int32_t *ids,
                                       float *wts) {
    uint32_t k[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int e = lane + WAVE * i;
        float v = 0.0f;
        if (e < E)
            v = COHERENT ? __hip_atomic_load(lr + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : lr[e];
        k[i] = e < E ? bf16_order_key(v, e) : 0u;  // valid keys are never 0
    }
    topk_select_packed<NL>(k, K, lane, ids, wts);
}

// PACKED: the logits are plain bf16 values (see bf16_order_key).
template <bool COHERENT>
__device__ inline void topk_row(const float *lr, int E, int K, int lane, int32_t *ids,
                                float *wts, bool packed) {
    if (packed) {
        if (E <= 64) return topk_row_packed<COHERENT, 1>(lr, E, K, lane, ids, wts);
        if (E <= 128) return topk_row_packed<COHERENT, 2>(lr, E, K, lane, ids, wts);
        if (E <= 256) return topk_row_packed<COHERENT, 4>(lr, E, K, lane, ids, wts);
        if (E <= 512) return topk_row_packed<COHERENT, 8>(lr, E, K, lane, ids, wts);
        return topk_row_packed<COHERENT, 16>(lr, E, K, lane, ids, wts);
    }
    if (E <= 64) topk_row_n<COHERENT, 1>(lr, E, K, lane, ids, wts);
    else if (E <= 128) topk_row_n<COHERENT, 2>(lr, E, K, lane, ids, wts);
    else if (E <= 256) topk_row_n<COHERENT, 4>(lr, E, K, lane, ids, wts);
    else if (E <= 512) topk_row_n<COHERENT, 8>(lr, E, K, lane, ids, wts);
    else topk_row_n<COHERENT, 16>(lr, E, K, lane, ids, wts);
}

}  // namespace moe
