// Row-at-a-time path (decode): block-FP8 GEMVs that stream only the
// selected experts' weights.
//
// The pages' one-row projection streams each warp's weight chunks through a
// ring and keeps the row tiling's arithmetic (PR #925 "drama: load the
// checkpoint with direct I/O in file order and build the codec on its own
// thread", commit summaries of the single-row projection). On gfx950 the
// one-row problem is purely HBM-bound (1.5 FLOP per weight byte), so the
// kernels here skip matrix cores: every lane streams 16 contiguous weight
// bytes per load, a 64-lane wave covers 1 KiB of a weight row per load, and
// partial dot products meet in wave reductions.
//
// gate/up: one wave owns four output rows n of one (row, slot) pair, reads
// gate and up rows together, quantises its x row on the fly (the 1x128
// rule, same arithmetic as moe_quant_act, one 8-lane max per group) and
// writes h = silu(g) * u in fp32. Shared-expert waves do the bf16 gate/up rows
// and write bf16(silu(gs) * us).
// down + combine: one workgroup owns a block of output columns of one row;
// it re-quantises that row's h (all K slots, 1x128) into LDS, then each wave
// reduces all K slots' down rows plus the shared down row and writes
// y = bf16(sum_j w_j e_j + gamma s), summed in slot order.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int GU_ROWS = 4;  // output rows per wave in the gate/up kernel

// Dot product of 16 decoded e4m3 activation values with 16 e4m3 weights.
__device__ __forceinline__ float dot16_fp8(const float (&a)[16], uint4 w) {
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    float p = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float b0, b1, b2, b3;
        e4m3x4_to_f32(wv[i], b0, b1, b2, b3);
        p = fmaf(a[4 * i + 0], b0, p);
        p = fmaf(a[4 * i + 1], b1, p);
        p = fmaf(a[4 * i + 2], b2, p);
        p = fmaf(a[4 * i + 3], b3, p);
    }
    return p;
}

// NC = 16-byte chunks of an FP8 weight row per lane (H / 1024, rounded up).
template <int NC>
__global__ __launch_bounds__(256) void decode_gateup_kernel(DecodeArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * 4 + wave;
    const int H = a.H, I = a.I, K = a.K;
    const int nchunk = H / 16;  // 16-byte FP8 chunks per weight row
    const int64_t routed_waves = (int64_t)a.T * K * (I / GU_ROWS);
    if (wid < routed_waves) {
        const int64_t p = wid / (I / GU_ROWS);
        const int n0 = (int)(wid % (I / GU_ROWS)) * GU_ROWS;
        const int t = (int)(p / K);
        const int e = a.ids[p];
        const uint16_t *xr = a.x + (int64_t)t * H;
        const uint8_t *wg = a.w_gate + ((int64_t)e * I + n0) * H;
        const uint8_t *wu = a.w_up + ((int64_t)e * I + n0) * H;
        const int KB = H / GROUP;
        const float *sg = a.s_gate + ((int64_t)e * (I / GROUP) + n0 / GROUP) * KB;
        const float *su = a.s_up + ((int64_t)e * (I / GROUP) + n0 / GROUP) * KB;
        // issue every weight load of this wave first
        uint4 wgv[NC][GU_ROWS], wuv[NC][GU_ROWS];
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = lane + WAVE * i;
#pragma unroll
            for (int r = 0; r < GU_ROWS; ++r) {
                if (c < nchunk) {
                    wgv[i][r] = ld16(wg + (int64_t)r * H + c * 16);
                    wuv[i][r] = ld16(wu + (int64_t)r * H + c * 16);
                } else {
                    wgv[i][r] = wuv[i][r] = make_uint4(0, 0, 0, 0);
                }
            }
        }
        float accg[GU_ROWS] = {}, accu[GU_ROWS] = {};
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = lane + WAVE * i;
            if (c >= nchunk) continue;  // whole 8-lane groups skip together
            const uint4 x0 = ld16(xr + c * 16), x1 = ld16(xr + c * 16 + 8);
            float xf[16] = {bf16_lo(x0.x), bf16_hi(x0.x), bf16_lo(x0.y), bf16_hi(x0.y),
                            bf16_lo(x0.z), bf16_hi(x0.z), bf16_lo(x0.w), bf16_hi(x0.w),
                            bf16_lo(x1.x), bf16_hi(x1.x), bf16_lo(x1.y), bf16_hi(x1.y),
                            bf16_lo(x1.z), bf16_hi(x1.z), bf16_lo(x1.w), bf16_hi(x1.w)};
            float amax = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(xf[k]));
            amax = wave_max<8>(amax);  // the 8 lanes of this 128-column group
            const float sx = group_scale(amax);
            float xq[16];
#pragma unroll
            for (int k = 0; k < 16; k += 4) {
                const uint32_t codes =
                    e4m3x4(xf[k] / sx, xf[k + 1] / sx, xf[k + 2] / sx, xf[k + 3] / sx);
                e4m3x4_to_f32(codes, xq[k], xq[k + 1], xq[k + 2], xq[k + 3]);
            }
            const int b = c / 8;
#pragma unroll
            for (int r = 0; r < GU_ROWS; ++r) {
                accg[r] = fmaf(sx * sg[b], dot16_fp8(xq, wgv[i][r]), accg[r]);
                accu[r] = fmaf(sx * su[b], dot16_fp8(xq, wuv[i][r]), accu[r]);
            }
        }
        float hv = 0.0f;
#pragma unroll
        for (int r = 0; r < GU_ROWS; ++r) {
            const float g = wave_sum<64>(accg[r]);
            const float u = wave_sum<64>(accu[r]);
            if (lane == r) hv = silu(g) * u;
        }
        if (lane < GU_ROWS) a.h[p * I + n0 + lane] = hv;
        return;
    }
    // shared expert rows (bf16 weights)
    const int64_t s = wid - routed_waves;
    if (a.Is == 0 || s >= (int64_t)a.T * (a.Is / GU_ROWS)) return;
    const int t = (int)(s / (a.Is / GU_ROWS));
    const int n0 = (int)(s % (a.Is / GU_ROWS)) * GU_ROWS;
    const uint16_t *xr = a.x + (int64_t)t * H;
    const int nc8 = H / 8;  // 16-byte bf16 chunks per row
    float accg[GU_ROWS] = {}, accu[GU_ROWS] = {};
    for (int c = lane; c < nc8; c += WAVE) {
        const uint4 xv = ld16(xr + c * 8);
        const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int r = 0; r < GU_ROWS; ++r) {
            const uint4 gv = ld16(a.sh_gate + (int64_t)(n0 + r) * H + c * 8);
            const uint4 uv = ld16(a.sh_up + (int64_t)(n0 + r) * H + c * 8);
            const uint32_t gs[4] = {gv.x, gv.y, gv.z, gv.w}, us[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                accg[r] = fmaf(bf16_lo(xs[i]), bf16_lo(gs[i]), accg[r]);
                accg[r] = fmaf(bf16_hi(xs[i]), bf16_hi(gs[i]), accg[r]);
                accu[r] = fmaf(bf16_lo(xs[i]), bf16_lo(us[i]), accu[r]);
                accu[r] = fmaf(bf16_hi(xs[i]), bf16_hi(us[i]), accu[r]);
            }
        }
    }
    uint32_t hv = 0;
#pragma unroll
    for (int r = 0; r < GU_ROWS; ++r) {
        const float g = wave_sum<64>(accg[r]);
        const float u = wave_sum<64>(accu[r]);
        if (lane == r) hv = f32_to_bf16(silu(g) * u);
    }
    if (lane < GU_ROWS) a.hs[(int64_t)t * a.Is + n0 + lane] = (uint16_t)hv;
}

hipError_t launch_decode_gateup(const DecodeArgs &a, hipStream_t st) {
    const int64_t waves = (int64_t)a.T * a.K * (a.I / GU_ROWS) + (int64_t)a.T * (a.Is / GU_ROWS);
    const dim3 grid((unsigned)((waves + 3) / 4));
    const int nc = (a.H / 16 + WAVE - 1) / WAVE;
    if (nc <= 1)
        hipLaunchKernelGGL(decode_gateup_kernel<1>, grid, dim3(256), 0, st, a);
    else if (nc <= 2)
        hipLaunchKernelGGL(decode_gateup_kernel<2>, grid, dim3(256), 0, st, a);
    else if (nc <= 4)
        hipLaunchKernelGGL(decode_gateup_kernel<4>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(decode_gateup_kernel<8>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

// ----------------------------------------------------------------- down

constexpr int DOWN_ROWS = 16;  // output columns per workgroup
constexpr int MAX_K = 16;

// CPL = 16-byte chunks per lane of one I-long down row; LPR = lanes per row.
template <int CPL, int LPR>
__global__ __launch_bounds__(256) void decode_down_kernel(DecodeArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int H = a.H, I = a.I, K = a.K, Is = a.Is;
    const int t = blockIdx.y;
    const int m_base = blockIdx.x * DOWN_ROWS;
    uint8_t *qh = lds;                                      // [K][I]
    float *shs = reinterpret_cast<float *>(lds + K * I);    // [K][I/128]
    // 1. re-quantise this row's h, 16 threads per 128-value group
    {
        const int G = K * I / GROUP;
        const float *hr = a.h + (int64_t)t * K * I;
        const int sub = threadIdx.x & 15;
        for (int g = threadIdx.x >> 4; g < G; g += 16) {
            const float4 v0 = *reinterpret_cast<const float4 *>(hr + g * GROUP + sub * 8);
            const float4 v1 = *reinterpret_cast<const float4 *>(hr + g * GROUP + sub * 8 + 4);
            float amax = fmaxf(fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w))),
                               fmaxf(fmaxf(fabsf(v1.x), fabsf(v1.y)), fmaxf(fabsf(v1.z), fabsf(v1.w))));
            amax = wave_max<16>(amax);
            const float sc = group_scale(amax);
            uint2 q;
            q.x = e4m3x4(v0.x / sc, v0.y / sc, v0.z / sc, v0.w / sc);
            q.y = e4m3x4(v1.x / sc, v1.y / sc, v1.z / sc, v1.w / sc);
            *reinterpret_cast<uint2 *>(qh + g * GROUP + sub * 8) = q;
            if (sub == 0) shs[g] = sc;
        }
    }
    __syncthreads();
    // 2. rows of the down matrices
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane % LPR, rsel = lane / LPR;
    constexpr int RPP = WAVE / LPR;  // rows per pass of a wave
    const int IB = I / GROUP;
    const int ncs = Is / 8;          // 16-byte bf16 chunks of a shared down row
    const int32_t *idr = a.ids + (int64_t)t * K;
    const float *wr = a.wts + (int64_t)t * K;
    const float gam = Is > 0 ? a.gamma[t] : 0.0f;
    for (int mr = wave * RPP + rsel; mr < DOWN_ROWS; mr += 4 * RPP) {
        const int m = m_base + mr;
        const bool mv = m < H;
        const int mm = mv ? m : 0;
        // issue the loads of every slot's down row
        uint4 wv[MAX_K][CPL];
#pragma unroll
        for (int j = 0; j < MAX_K; ++j) {
            if (j < K) {
                const uint8_t *row = a.w_down + ((int64_t)idr[j] * H + mm) * I;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const int c = sub + LPR * i;
                    wv[j][i] = c < I / 16 ? ld16(row + c * 16) : make_uint4(0, 0, 0, 0);
                }
            }
        }
        float yacc = 0.0f;
#pragma unroll
        for (int j = 0; j < MAX_K; ++j) {
            if (j < K) {
                const int e = idr[j];
                const float *sd = a.s_down + ((int64_t)e * (H / GROUP) + mm / GROUP) * IB;
                float acc = 0.0f;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const int c = sub + LPR * i;
                    if (c < I / 16) {
                        const uint4 qv = *reinterpret_cast<const uint4 *>(qh + j * I + c * 16);
                        const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
                        float hq[16];
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            e4m3x4_to_f32(qw[k], hq[4 * k], hq[4 * k + 1], hq[4 * k + 2],
                                          hq[4 * k + 3]);
                        const int b = c / 8;
                        acc = fmaf(shs[j * IB + b] * sd[b], dot16_fp8(hq, wv[j][i]), acc);
                    }
                }
                acc = wave_sum<LPR>(acc);
                yacc = fmaf(wr[j], acc, yacc);
            }
        }
        if (Is > 0) {
            float sacc = 0.0f;
            const uint16_t *srow = a.sh_down + (int64_t)mm * Is;
            const uint16_t *hsr = a.hs + (int64_t)t * Is;
            for (int c = sub; c < ncs; c += LPR) {
                const uint4 wv8 = ld16(srow + c * 8), hv8 = ld16(hsr + c * 8);
                const uint32_t ws[4] = {wv8.x, wv8.y, wv8.z, wv8.w};
                const uint32_t hs[4] = {hv8.x, hv8.y, hv8.z, hv8.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sacc = fmaf(bf16_lo(hs[i]), bf16_lo(ws[i]), sacc);
                    sacc = fmaf(bf16_hi(hs[i]), bf16_hi(ws[i]), sacc);
                }
            }
            sacc = wave_sum<LPR>(sacc);
            yacc = fmaf(gam, sacc, yacc);
        }
        if (mv && sub == 0) a.y[(int64_t)t * H + m] = (uint16_t)f32_to_bf16(yacc);
    }
}

hipError_t launch_decode_down(const DecodeArgs &a, hipStream_t st) {
    const dim3 grid((a.H + DOWN_ROWS - 1) / DOWN_ROWS, a.T);
    const size_t lds = (size_t)a.K * a.I + (size_t)a.K * (a.I / GROUP) * sizeof(float);
    const int chunks = a.I / 16;  // 8 .. 256
    if (chunks <= 8)
        hipLaunchKernelGGL((decode_down_kernel<1, 8>), grid, dim3(256), lds, st, a);
    else if (chunks <= 16)
        hipLaunchKernelGGL((decode_down_kernel<1, 16>), grid, dim3(256), lds, st, a);
    else if (chunks <= 32)
        hipLaunchKernelGGL((decode_down_kernel<1, 32>), grid, dim3(256), lds, st, a);
    else if (chunks <= 64)
        hipLaunchKernelGGL((decode_down_kernel<1, 64>), grid, dim3(256), lds, st, a);
    else if (chunks <= 128)
        hipLaunchKernelGGL((decode_down_kernel<2, 64>), grid, dim3(256), lds, st, a);
    else
        hipLaunchKernelGGL((decode_down_kernel<4, 64>), grid, dim3(256), lds, st, a);
    return hipGetLastError();
}

}  // namespace moe
