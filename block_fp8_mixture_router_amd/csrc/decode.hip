// Row-at-a-time path (decode): the whole layer in one persistent kernel.
//
// The pages' one-row projection streams weight chunks through a ring, and
// their frame step chains its kernels with programmatic dependent launch so
// a kernel can stream immutable weights before waiting on its predecessor
// (PR #925 "drama: load the checkpoint with direct I/O in file order and build
// the codec on its own thread", commit summaries of the single-row
// projection; PR #927, "What this changes"). On gfx950 the layer for one row
// is purely HBM-bound (1.5 FLOP per weight byte) and latency-bound by its
// three dependent steps, so it runs as ONE launch of one workgroup per
// compute unit, with two grid-wide handoffs instead of kernel boundaries:
//
//  A. router logits (exact fp64 sums), shared-expert gate/up rows and the
//     shared gate; every workgroup also quantises x (1x128) into LDS;
//     -- handoff 1: logits, hs and gamma visible --
//  B. every workgroup selects the top-K itself (wave argmax, DPP lane moves)
//     and streams its share of the routed gate/up rows: h = silu(g) * u;
//     -- handoff 2: h visible --
//  C. every workgroup re-quantises h (1x128) into LDS and owns whole output
//     rows m: all K down rows plus the shared down row, then writes
//     y = bf16(sum_j w_j e_j + gamma s) in slot order. No third handoff.
//
// Work is spread over waves workgroup-major, so consecutive items land on
// different compute units. Each lane streams 16 contiguous weight bytes per
// load; a wave covers 1 KiB of a weight row per load.
//
// Handoffs: each workgroup publishes a per-call flag value (generation + 1)
// in its own slot and waits until all slots carry it. The generation word
// lives in the workspace and advances by 2 per call, so neither an
// uninitialised workspace nor flags left by an earlier call (or an earlier
// replay of a captured graph) can satisfy a wait. The wait is bounded: if it
// ever spins out (workgroups not co-resident) an error word is set and the
// kernel still finishes.
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

constexpr int GU_ROWS = 4;       // routed gate/up rows per wave item
constexpr int SH_ROWS = 2;       // shared gate/up rows per wave item
constexpr int MAX_K = 16;
constexpr uint32_t SPIN_LIMIT = 1u << 17;  // ~0.2 s of polling, then give up

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

__device__ __forceinline__ void decode16(uint4 q, float (&f)[16]) {
    e4m3x4_to_f32(q.x, f[0], f[1], f[2], f[3]);
    e4m3x4_to_f32(q.y, f[4], f[5], f[6], f[7]);
    e4m3x4_to_f32(q.z, f[8], f[9], f[10], f[11]);
    e4m3x4_to_f32(q.w, f[12], f[13], f[14], f[15]);
}

// ------------------------------------------------------------ handoffs

__device__ __forceinline__ uint32_t ld_acquire_relaxed(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void handoff(const FusedArgs &a, int b, uint32_t target) {
    // every wave releases its own stores at device scope before the flag
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    uint32_t *flags = a.sync + 64 + b * a.nwg;
    if (threadIdx.x == 0)
        __hip_atomic_store(flags + blockIdx.x, target, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x < WAVE) {
        for (uint32_t spin = 0;; ++spin) {
            bool ok = true;
            for (int i = threadIdx.x; i < a.nwg; i += WAVE) ok &= ld_acquire_relaxed(flags + i) == target;
            if (__all(ok)) break;
            if (spin >= SPIN_LIMIT) {
                if (threadIdx.x == 0)
                    __hip_atomic_store(a.sync + 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    __syncthreads();
    // every wave acquires the other workgroups' results
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// ------------------------------------------------------------- phase A

// logit of (row t, expert e): exact fp64 sum of bf16 products, one rounding
__device__ void router_item(const FusedArgs &a, int t, int e, int lane) {
    const uint16_t *xr = a.x + (int64_t)t * a.H;
    const uint16_t *wr = a.router_w + (int64_t)e * a.H;
    double acc = 0.0;
    for (int c = lane; c < a.H / 8; c += WAVE) {
        const uint4 xv = ld16(xr + c * 8), wv = ld16(wr + c * 8);
        const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w}, ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = fma((double)bf16_lo(xs[i]), (double)bf16_lo(ws[i]), acc);
            acc = fma((double)bf16_hi(xs[i]), (double)bf16_hi(ws[i]), acc);
        }
    }
    acc = wave_allsum_d(acc);
    if (lane == 0) {
        float l = (float)acc;
        if (!(a.flags & K_LOGITS_FP32)) l = __uint_as_float(f32_to_bf16(l) << 16);
        if (a.bias) l = l + a.bias[e];
        a.logits[(int64_t)t * a.E + e] = l;
    }
}

// shared-expert rows n0..n0+SH_ROWS-1 of row t: hs = bf16(silu(g) * u)
__device__ void shared_item(const FusedArgs &a, int t, int n0, int lane) {
    const uint16_t *xr = a.x + (int64_t)t * a.H;
    float g[SH_ROWS] = {}, u[SH_ROWS] = {};
    for (int c = lane; c < a.H / 8; c += WAVE) {
        const uint4 xv = ld16(xr + c * 8);
        const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
        uint4 gv[SH_ROWS], uv[SH_ROWS];
#pragma unroll
        for (int r = 0; r < SH_ROWS; ++r) {
            gv[r] = ld16(a.sh_gate + (int64_t)(n0 + r) * a.H + c * 8);
            uv[r] = ld16(a.sh_up + (int64_t)(n0 + r) * a.H + c * 8);
        }
#pragma unroll
        for (int r = 0; r < SH_ROWS; ++r) {
            const uint32_t gs[4] = {gv[r].x, gv[r].y, gv[r].z, gv[r].w};
            const uint32_t us[4] = {uv[r].x, uv[r].y, uv[r].z, uv[r].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                g[r] = fmaf(bf16_lo(xs[i]), bf16_lo(gs[i]), g[r]);
                g[r] = fmaf(bf16_hi(xs[i]), bf16_hi(gs[i]), g[r]);
                u[r] = fmaf(bf16_lo(xs[i]), bf16_lo(us[i]), u[r]);
                u[r] = fmaf(bf16_hi(xs[i]), bf16_hi(us[i]), u[r]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < SH_ROWS; ++r) {
        const float gs = wave_allsum(g[r]), us = wave_allsum(u[r]);
        if (lane == r) a.hs[(int64_t)t * a.Is + n0 + r] = (uint16_t)f32_to_bf16(silu(gs) * us);
    }
}

__device__ void gamma_item(const FusedArgs &a, int t, int lane) {
    const uint16_t *xr = a.x + (int64_t)t * a.H;
    float z = 0.0f;
    for (int c = lane; c < a.H / 8; c += WAVE) {
        const uint4 xv = ld16(xr + c * 8), wv = ld16(a.sh_gate_w + c * 8);
        const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w}, ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z = fmaf(bf16_lo(xs[i]), bf16_lo(ws[i]), z);
            z = fmaf(bf16_hi(xs[i]), bf16_hi(ws[i]), z);
        }
    }
    z = wave_allsum(z);
    if (lane == 0) a.gamma[t] = 1.0f / (1.0f + expf(-z));
}

// ------------------------------------------------------------- phase B

// routed rows n0..n0+GU_ROWS-1 of pair p: h = silu(g) * u (fp32)
template <int NC>
__device__ void gateup_item(const FusedArgs &a, int p, int n0, int e, const uint8_t *qx,
                            const float *sx, int lane) {
    const int H = a.H, I = a.I, nchunk = H / 16, KB = H / GROUP;
    const uint8_t *wg = a.w_gate + ((int64_t)e * I + n0) * H;
    const uint8_t *wu = a.w_up + ((int64_t)e * I + n0) * H;
    const float *sg = a.s_gate + ((int64_t)e * (I / GROUP) + n0 / GROUP) * KB;
    const float *su = a.s_up + ((int64_t)e * (I / GROUP) + n0 / GROUP) * KB;
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
        if (c < nchunk) {
            float xq[16];
            decode16(*reinterpret_cast<const uint4 *>(qx + c * 16), xq);
            const int b = c / 8;
            const float s = sx[b];
#pragma unroll
            for (int r = 0; r < GU_ROWS; ++r) {
                accg[r] = fmaf(s * sg[b], dot16_fp8(xq, wgv[i][r]), accg[r]);
                accu[r] = fmaf(s * su[b], dot16_fp8(xq, wuv[i][r]), accu[r]);
            }
        }
    }
    float hv = 0.0f;
#pragma unroll
    for (int r = 0; r < GU_ROWS; ++r) {
        const float g = wave_allsum(accg[r]), u = wave_allsum(accu[r]);
        if (lane == r) hv = silu(g) * u;
    }
    if (lane < GU_ROWS) a.h[(int64_t)p * I + n0 + lane] = hv;
}

// ------------------------------------------------------------- phase C

template <int WIDTH>
__device__ __forceinline__ float seg_sum(float v) {
    if constexpr (WIDTH == 64) return wave_allsum(v);
    if constexpr (WIDTH == 32) return group32_sum(v);
    if constexpr (WIDTH == 16) return group16_sum(v);
    v += dpp_f<DPP_XOR1>(v);
    v += dpp_f<DPP_XOR2>(v);
    return v + dpp_f<DPP_HALF_MIRROR>(v);
}

// Output rows of row t: RPP = 64 / LPR rows per wave item, LPR lanes per
// row, CPL 16-byte chunks per lane of one I-long down row.
template <int CPL, int LPR>
__device__ void down_item(const FusedArgs &a, int t, int m, int sub, const uint8_t *qh,
                          const float *shs, const int32_t *ids, const float *wts) {
    const int H = a.H, I = a.I, K = a.K, Is = a.Is, IB = I / GROUP;
    uint4 wv[MAX_K][CPL];
#pragma unroll
    for (int j = 0; j < MAX_K; ++j)
        if (j < K) {
            const uint8_t *row = a.w_down + ((int64_t)ids[t * K + j] * H + m) * I;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = sub + LPR * i;
                wv[j][i] = c < I / 16 ? ld16(row + c * 16) : make_uint4(0, 0, 0, 0);
            }
        }
    float sacc = 0.0f;
    if (Is > 0) {
        const uint16_t *srow = a.sh_down + (int64_t)m * Is;
        const uint16_t *hsr = a.hs + (int64_t)t * Is;
        for (int c = sub; c < Is / 8; c += LPR) {
            const uint4 w8 = ld16(srow + c * 8), h8 = ld16(hsr + c * 8);
            const uint32_t ws[4] = {w8.x, w8.y, w8.z, w8.w}, hs[4] = {h8.x, h8.y, h8.z, h8.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sacc = fmaf(bf16_lo(hs[i]), bf16_lo(ws[i]), sacc);
                sacc = fmaf(bf16_hi(hs[i]), bf16_hi(ws[i]), sacc);
            }
        }
    }
    float yacc = 0.0f;
#pragma unroll
    for (int j = 0; j < MAX_K; ++j)
        if (j < K) {
            const int p = t * K + j;
            const float *sd = a.s_down + ((int64_t)ids[p] * (H / GROUP) + m / GROUP) * IB;
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = sub + LPR * i;
                if (c < I / 16) {
                    float hq[16];
                    decode16(*reinterpret_cast<const uint4 *>(qh + (int64_t)p * I + c * 16), hq);
                    const int b = c / 8;
                    acc = fmaf(shs[p * IB + b] * sd[b], dot16_fp8(hq, wv[j][i]), acc);
                }
            }
            yacc = fmaf(wts[p], seg_sum<LPR>(acc), yacc);
        }
    if (Is > 0) yacc = fmaf(a.gamma[t], seg_sum<LPR>(sacc), yacc);
    if (sub == 0) a.y[(int64_t)t * H + m] = (uint16_t)f32_to_bf16(yacc);
}

// ---------------------------------------------------------------- kernel

// LDS carve-up of the fused kernel, every piece 16-byte aligned
struct LdsPlan {
    int qx, sx, qh, shs, ids, wts, total;
};
__host__ __device__ inline int al16i(int b) { return (b + 15) & ~15; }
__host__ __device__ inline LdsPlan lds_plan(int T, int H, int K, int I) {
    LdsPlan L;
    const int P = T * K;
    L.qx = 0;
    L.sx = L.qx + al16i(T * H);
    L.qh = L.sx + al16i(T * (H / GROUP) * 4);
    L.shs = L.qh + al16i(P * I);
    L.ids = L.shs + al16i(P * (I / GROUP) * 4);
    L.wts = L.ids + al16i(P * 4);
    L.total = L.wts + al16i(P * 4);
    return L;
}

bool decode_fits(int T, int H, int K, int I) {
    return T >= 1 && T <= DECODE_MAX_ROWS && lds_plan(T, H, K, I).total <= 150 * 1024;
}

// quantise n_groups 128-groups of fp32 or bf16 values into LDS codes/scales
template <bool BF16>
__device__ void quant_to_lds(const void *src, int n_groups, uint8_t *q, float *s) {
    const int sub = threadIdx.x & 15;
    for (int g = threadIdx.x >> 4; g < n_groups; g += blockDim.x >> 4) {
        float f[8];
        if constexpr (BF16) {
            const uint4 v = ld16(static_cast<const uint16_t *>(src) + (int64_t)g * GROUP + sub * 8);
            f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
            f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
        } else {
            const float *p = static_cast<const float *>(src) + (int64_t)g * GROUP + sub * 8;
            const float4 v0 = *reinterpret_cast<const float4 *>(p);
            const float4 v1 = *reinterpret_cast<const float4 *>(p + 4);
            f[0] = v0.x; f[1] = v0.y; f[2] = v0.z; f[3] = v0.w;
            f[4] = v1.x; f[5] = v1.y; f[6] = v1.z; f[7] = v1.w;
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
        amax = group16_max(amax);
        const float sc = group_scale(amax);
        uint2 out;
        out.x = e4m3x4(f[0] / sc, f[1] / sc, f[2] / sc, f[3] / sc);
        out.y = e4m3x4(f[4] / sc, f[5] / sc, f[6] / sc, f[7] / sc);
        *reinterpret_cast<uint2 *>(q + g * GROUP + sub * 8) = out;
        if (sub == 0) s[g] = sc;
    }
}

template <int NC, int CPL, int LPR>
__global__ __launch_bounds__(256, 1) void decode_fused_kernel(FusedArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int T = a.T, H = a.H, K = a.K, I = a.I, P = T * K;
    const LdsPlan L = lds_plan(T, H, K, I);
    uint8_t *qx = lds + L.qx;                                 // [T][H]
    float *sx = reinterpret_cast<float *>(lds + L.sx);        // [T][H/128]
    uint8_t *qh = lds + L.qh;                                 // [P][I]
    float *shs = reinterpret_cast<float *>(lds + L.shs);      // [P][I/128]
    int32_t *ids = reinterpret_cast<int32_t *>(lds + L.ids);  // [P]
    float *wts = reinterpret_cast<float *>(lds + L.wts);      // [P]
    __shared__ uint32_t s_target;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nw = a.nwg * 4;
    const int gw = wave * a.nwg + blockIdx.x;  // workgroup-major wave index
    if (threadIdx.x == 0) s_target = ld_acquire_relaxed(a.sync) + 1u;
    quant_to_lds<true>(a.x, T * (H / GROUP), qx, sx);

    // A: router logits, shared gate/up, gate
    const int n_router = T * a.E;
    const int n_shared = a.Is > 0 ? T * (a.Is / SH_ROWS) : 0;
    const int n_gamma = a.Is > 0 ? T : 0;
    for (int it = gw; it < n_router + n_shared + n_gamma; it += nw) {
        if (it < n_router) {
            router_item(a, it / a.E, it % a.E, lane);
        } else if (it < n_router + n_shared) {
            const int s = it - n_router, per = a.Is / SH_ROWS;
            shared_item(a, s / per, (s % per) * SH_ROWS, lane);
        } else {
            gamma_item(a, it - n_router - n_shared, lane);
        }
    }
    __syncthreads();
    const uint32_t target = s_target;
    handoff(a, 0, target);
    // every workgroup has read the generation word: advance it for the next call
    if (blockIdx.x == 0 && threadIdx.x == 0)
        __hip_atomic_store(a.sync, target + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // B: top-K per row (one wave per row), then routed gate/up
    for (int t = wave; t < T; t += 4) topk_row(a.logits + (int64_t)t * a.E, a.E, K, lane,
                                               ids + t * K, wts + t * K);
    __syncthreads();
    const int per_pair = I / GU_ROWS;
    for (int it = gw; it < P * per_pair; it += nw) {
        const int p = it / per_pair, n0 = (it % per_pair) * GU_ROWS, t = p / K;
        gateup_item<NC>(a, p, n0, ids[p], qx + t * H, sx + t * (H / GROUP), lane);
    }
    handoff(a, 1, target);

    // C: re-quantise h, then whole output rows with the combine
    quant_to_lds<false>(a.h, P * (I / GROUP), qh, shs);
    __syncthreads();
    constexpr int RPP = WAVE / LPR;
    const int sub = lane % LPR, rsel = lane / LPR;
    const int items = T * (H / RPP);
    for (int it = gw; it < items; it += nw) {
        const int t = it / (H / RPP);
        const int m = (it % (H / RPP)) * RPP + rsel;
        down_item<CPL, LPR>(a, t, m, sub, qh, shs, ids, wts);
    }
}

template <int NC>
static hipError_t launch_nc(const FusedArgs &a, size_t lds, hipStream_t st) {
    const dim3 grid(a.nwg), block(256);
    const int chunks = a.I / 16;
    if (chunks <= 8)
        hipLaunchKernelGGL((decode_fused_kernel<NC, 1, 8>), grid, block, lds, st, a);
    else if (chunks <= 16)
        hipLaunchKernelGGL((decode_fused_kernel<NC, 1, 16>), grid, block, lds, st, a);
    else if (chunks <= 32)
        hipLaunchKernelGGL((decode_fused_kernel<NC, 1, 32>), grid, block, lds, st, a);
    else if (chunks <= 64)
        hipLaunchKernelGGL((decode_fused_kernel<NC, 1, 64>), grid, block, lds, st, a);
    else if (chunks <= 128)
        hipLaunchKernelGGL((decode_fused_kernel<NC, 2, 64>), grid, block, lds, st, a);
    else
        hipLaunchKernelGGL((decode_fused_kernel<NC, 4, 64>), grid, block, lds, st, a);
    return hipGetLastError();
}

template <int NC, int CPL, int LPR>
static hipError_t set_lds_limit() {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&decode_fused_kernel<NC, CPL, LPR>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
}

hipError_t launch_decode_fused(const FusedArgs &a, hipStream_t st) {
    const size_t lds = (size_t)lds_plan(a.T, a.H, a.K, a.I).total;
    if (lds > 64 * 1024) {
        static const bool once = [] {
#define MOE_SET(NC)                                                                       \
    (void)set_lds_limit<NC, 1, 8>(); (void)set_lds_limit<NC, 1, 16>();                       \
    (void)set_lds_limit<NC, 1, 32>(); (void)set_lds_limit<NC, 1, 64>();                      \
    (void)set_lds_limit<NC, 2, 64>(); (void)set_lds_limit<NC, 4, 64>();
            MOE_SET(1) MOE_SET(2) MOE_SET(4) MOE_SET(8)
#undef MOE_SET
            return true;
        }();
        (void)once;
    }
    const int nc = (a.H / 16 + WAVE - 1) / WAVE;
    if (nc <= 1) return launch_nc<1>(a, lds, st);
    if (nc <= 2) return launch_nc<2>(a, lds, st);
    if (nc <= 4) return launch_nc<4>(a, lds, st);
    return launch_nc<8>(a, lds, st);
}

}  // namespace moe
