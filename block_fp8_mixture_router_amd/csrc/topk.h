// Top-K selection of one router row by one full wave.
#pragma once

#include "common.h"

namespace moe {

// Top-K of one row by K rounds of a wave argmax (largest logit, then lowest
// expert index), then the softmax over the K in slot order. Results to LDS.
__device__ inline void topk_row(const float *lr, int E, int K, int lane, int32_t *ids, float *wts) {
    float v[16];
    uint32_t live = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int e = lane + WAVE * i;
        v[i] = e < E ? lr[e] : 0.0f;
        if (e < E) live |= 1u << i;
    }
    float my_v = 0.0f, v0 = 0.0f;
    int my_id = 0;
    for (int j = 0; j < K; ++j) {
        float bv = 0.0f;
        int bi = -1;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if ((live >> i) & 1u)
                if (bi < 0 || v[i] > bv) {
                    bv = v[i];
                    bi = i;
                }
        const float vmax = wave_allmax(bi >= 0 ? bv : -INFINITY);
        const int cand = (bi >= 0 && bv == vmax) ? lane + WAVE * bi : 0x7FFFFFFF;
        const int win = wave_allmin_i(cand);
        if (win == cand) live &= ~(1u << bi);
        if (j == 0) v0 = vmax;
        if (lane == j) {
            my_id = win;
            my_v = vmax;
        }
    }
    const float ex = lane < K ? expf(my_v - v0) : 0.0f;
    float sum = 0.0f;
    for (int j = 0; j < K; ++j) sum += readlane_f(ex, j);
    if (lane < K) {
        ids[lane] = my_id;
        wts[lane] = ex / sum;
    }
}

}  // namespace moe
