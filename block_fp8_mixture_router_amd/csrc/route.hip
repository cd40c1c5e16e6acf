// Router: logits, top-K selection and renormalised softmax.
//
// The pages' router decides on bf16 logits and runs its softmax in fp32
// (PR #939 "drama3: Fish Audio Drama 3 text to speech on one CUDA GPU",
// "Fidelity against the PyTorch oracle" and "How it fits the engine" >
// Precision). bf16 logits tie often, so any change of summation order would
// move picks; each logit here is the exact sum of the exact bf16 x bf16
// products, accumulated in fp64 and rounded once to fp32, then to bf16.
//
// Two logit kernels:
//  - few rows (decode): one wave per (row, expert), 16-byte loads, fp64 FMA,
//    a wave reduction; the 1 MiB router matrix streams once per row.
//  - many rows (prompt chunks): fp64 MFMA 16x16x4 tiles; each lane streams 32
//    contiguous bytes of its row and of its experts per 64 columns and the
//    MFMA sums over the lanes' column slices.
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

__device__ __forceinline__ float finish_logit(double acc, const float *bias, int e,
                                              uint32_t flags) {
    float l = (float)acc;  // the single rounding of the exact sum to fp32
    if (!(flags & K_LOGITS_FP32)) l = __uint_as_float(f32_to_bf16(l) << 16);
    if (bias) l = l + bias[e];
    return l;
}

__global__ __launch_bounds__(256) void route_logits_vec(const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ rw,
                                                        const float *__restrict__ bias, int H,
                                                        int E, uint32_t flags,
                                                        float *__restrict__ logits) {
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.y;
    if (e >= E) return;
    const uint16_t *xr = x + (int64_t)t * H;
    const uint16_t *wr = rw + (int64_t)e * H;
    double acc = 0.0;
    for (int c = lane; c < H / 8; c += WAVE) {
        const uint4 a = ld16(xr + c * 8), b = ld16(wr + c * 8);
        const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = fma((double)bf16_lo(av[i]), (double)bf16_lo(bv[i]), acc);
            acc = fma((double)bf16_hi(av[i]), (double)bf16_hi(bv[i]), acc);
        }
    }
    acc = wave_allsum_d(acc);
    if (lane == 0) logits[(int64_t)t * E + e] = finish_logit(acc, bias, e, flags);
}

// grid: x = ceil(E / 64), y = ceil(T / 16). A workgroup owns 16 rows x 64
// experts; wave w sums the 64-column chunks w, w+4, w+8, ... into four
// independent 16x16 fp64 accumulators (one per 16 experts, so each converted
// x value feeds four MFMAs), and the four quarters are added in LDS in a
// fixed order. fp64 sums of exact products: rounding once to fp32 gives the
// same logit as any other summation order unless the sum lies within ~2^-40
// (relative) of an fp32 rounding boundary.
__global__ __launch_bounds__(256) void route_logits_mfma(const uint16_t *__restrict__ x, int T,
                                                         const uint16_t *__restrict__ rw,
                                                         const float *__restrict__ bias, int H,
                                                         int E, uint32_t flags,
                                                         float *__restrict__ logits) {
    __shared__ double part[4][4][64][4];  // [wave][expert tile][lane][element]
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e0 = blockIdx.x * 64, t0 = blockIdx.y * 16;
    const int r = lane & 15, q = lane >> 4;
    const bool tv = t0 + r < T;
    // lane (r, q) supplies row r / expert r of each tile, columns
    // [k + 16q, k + 16q + 16) of every 64-column chunk k
    const uint16_t *xr = x + (int64_t)(tv ? t0 + r : 0) * H + q * 16;
    const uint16_t *wr[4];
    bool ev[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ev[j] = e0 + 16 * j + r < E;
        wr[j] = rw + (int64_t)(ev[j] ? e0 + 16 * j + r : 0) * H + q * 16;
    }
    v4d acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = (v4d){0.0, 0.0, 0.0, 0.0};
    for (int k = wave * 64; k < H; k += 256) {
        uint4 xa = ld16(xr + k), xb = ld16(xr + k + 8);
        if (!tv) xa = xb = make_uint4(0, 0, 0, 0);
        uint4 wa[4], wb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            wa[j] = ev[j] ? ld16(wr[j] + k) : make_uint4(0, 0, 0, 0);
            wb[j] = ev[j] ? ld16(wr[j] + k + 8) : make_uint4(0, 0, 0, 0);
        }
        const uint32_t xs[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double xl = (double)bf16_lo(xs[i]), xh = (double)bf16_hi(xs[i]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t ws[8] = {wa[j].x, wa[j].y, wa[j].z, wa[j].w,
                                        wb[j].x, wb[j].y, wb[j].z, wb[j].w};
                acc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(xl, (double)bf16_lo(ws[i]), acc[j],
                                                              0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(xh, (double)bf16_hi(ws[i]), acc[j],
                                                              0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[wave][j][lane][i] = acc[j][i];
    __syncthreads();
    // wave w finishes expert tile w: fp64 accumulator layout is
    // element i of lane (r, q) = row q + 4i, column r
    const int j = wave;
    const int e = e0 + 16 * j + r;
    if (e >= E) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double v = ((part[0][j][lane][i] + part[1][j][lane][i]) + part[2][j][lane][i]) +
                         part[3][j][lane][i];
        const int t = t0 + q + 4 * i;
        if (t < T) logits[(int64_t)t * E + e] = finish_logit(v, bias, e, flags);
    }
}

hipError_t launch_route_logits(const uint16_t *x, int T, const uint16_t *router_w,
                               const float *bias, int H, int E, uint32_t flags, float *logits,
                               hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (T <= 16) {
        hipLaunchKernelGGL(route_logits_vec, dim3((E + 3) / 4, T), dim3(256), 0, st, x,
                           router_w, bias, H, E, flags, logits);
    } else {
        hipLaunchKernelGGL(route_logits_mfma, dim3((E + 63) / 64, (T + 15) / 16), dim3(256), 0,
                           st, x, T, router_w, bias, H, E, flags, logits);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ top-K

// One wave per row: the shared top-K routine, then (forward only) the
// shared-expert gate gamma[t] = sigmoid(gate_w . x[t]) and the 1x128
// quantisation of x[t] (the same arithmetic as moe_quant_act), so the
// expert-grouped path needs no separate quantiser launch.
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float *__restrict__ logits, int T, int E, int K, int32_t *__restrict__ ids,
    float *__restrict__ wts, const uint16_t *__restrict__ x,
    const uint16_t *__restrict__ gate_w, int H, float *__restrict__ gamma, bool packed,
    uint8_t *__restrict__ qx, float *__restrict__ sx) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= T) return;  // whole waves leave together
    topk_row<false>(logits + (int64_t)t * E, E, K, lane, ids + (int64_t)t * K,
                    wts + (int64_t)t * K, packed);
    if (gate_w) {
        const uint16_t *xr = x + (int64_t)t * H;
        float z = 0.0f;
        for (int c = lane; c < H / 8; c += WAVE) {
            const uint4 a = ld16(xr + c * 8), b = ld16(gate_w + c * 8);
            const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                z = fmaf(bf16_lo(av[i]), bf16_lo(bv[i]), z);
                z = fmaf(bf16_hi(av[i]), bf16_hi(bv[i]), z);
            }
        }
        z = wave_allsum(z);
        if (lane == 0) gamma[t] = 1.0f / (1.0f + expf(-z));
    }
    if (qx) {
        // 16 lanes per 128-column group, 8 values per lane, 4 groups per pass
        const uint16_t *xr = x + (int64_t)t * H;
        for (int c = lane; c < H / 8; c += WAVE) {
            const uint4 v = ld16(xr + c * 8);
            float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                          bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
            amax = group16_max(amax);
            const float sc = group_scale(amax);
            uint2 out;
            out.x = e4m3x4(f[0] / sc, f[1] / sc, f[2] / sc, f[3] / sc);
            out.y = e4m3x4(f[4] / sc, f[5] / sc, f[6] / sc, f[7] / sc);
            *reinterpret_cast<uint2 *>(qx + (int64_t)t * H + c * 8) = out;
            if ((c & 15) == 0) sx[(int64_t)t * (H / GROUP) + c / 16] = sc;
        }
    }
}

hipError_t launch_route_topk(const float *logits, int T, int E, int K, int32_t *ids,
                             float *weights, const uint16_t *x, const uint16_t *gate_w, int H,
                             float *gamma, bool packed, uint8_t *qx, float *sx,
                             hipStream_t st) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(route_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, E, K,
                       ids, weights, x, gate_w, H, gamma, packed, qx, sx);
    return hipGetLastError();
}

}  // namespace moe
