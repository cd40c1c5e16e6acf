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
//  A. router logits (exact fp64 sums), shared-expert gate/up rows
//     (hs = bf16(silu(gs) * us)) and the shared gate; every load that does not
//     depend on the routing, the phase-C shared down rows included, is issued
//     here; every workgroup also quantises x (1x128) into LDS;
//     -- handoff 1: logits, hs and gamma visible --
//  B. every workgroup selects the top-K itself (wave argmax, DPP lane moves),
//     issues the loads of its phase-C routed down rows, and streams its share
//     of the routed gate/up rows: h = silu(g) * u;
//     -- handoff 2: h visible --
//  C. every workgroup re-quantises h (1x128) into LDS and owns whole output
//     rows m: all K down rows plus the shared down row, then writes
//     y = bf16(sum_j w_j e_j + gamma s) in slot order. No third handoff.
//
// Work is spread over waves workgroup-major, so consecutive items land on
// different compute units. Each lane streams 16 contiguous weight bytes per
// load; a wave covers 1 KiB of a weight row per load.
//
// Handoffs: every value that crosses workgroups (logits, hs, gamma, h, the
// flags) is written and read with device-coherent (sc1) loads and stores,
// which bypass the per-XCD L2 for that access only; a device-scope fence
// would instead write back or invalidate a whole L2, and a thousand of them
// per handoff cost tens of microseconds. A producer drains its own stores
// (s_waitcnt) before its workgroup's arrival flag is stored. Every such value
// is stored in DECODE_REPLICAS copies and each workgroup reads copy
// blockIdx % DECODE_REPLICAS, so no cache line is read by more than 1/8 of
// the workgroups (one copy per XCD when workgroups are dealt round-robin).
// Flag values are the call's generation + 1; the
// generation word lives in the workspace and advances by 2 per call, so
// neither an uninitialised workspace nor flags left by an earlier call (or an
// earlier replay of a captured graph) can satisfy a wait. Waits are bounded:
// a spin-out (workgroups not co-resident) sets an error word and the kernel
// still finishes.
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

constexpr int GU_ROWS = 4;       // routed gate/up rows per wave item
constexpr int REPL = DECODE_REPLICAS;  // copies of every cross-workgroup value
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

template <typename T>
__device__ __forceinline__ T ld_dev(const T *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_dev(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// sync words: [0] generation, [32] error, [SYNC_FLAGS + (b * REPL + r) * nwg + w]
// replica r of workgroup w's arrival flag at handoff b. Each workgroup writes
// its flag into every replica and polls replica blockIdx % REPL.
__device__ __forceinline__ void handoff(const FusedArgs &a, int b, uint32_t target) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's device-coherent stores are done
    __syncthreads();
    uint32_t *flags = a.sync + SYNC_FLAGS + b * REPL * a.nwg;
    if (threadIdx.x < REPL) st_dev(flags + threadIdx.x * a.nwg + blockIdx.x, target);
    if (threadIdx.x < WAVE) {
        const uint32_t *mine = flags + (blockIdx.x % REPL) * a.nwg;
        for (uint32_t spin = 0;; ++spin) {
            bool ok = true;
            for (int i = threadIdx.x; i < a.nwg; i += WAVE) ok &= ld_dev(mine + i) == target;
            if (__all(ok)) break;
            if (spin >= SPIN_LIMIT) {
                if (threadIdx.x == 0) st_dev(a.sync + 32, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    __syncthreads();
}

// ------------------------------------------------------------- phase A

// NB = 16-byte chunks of a bf16 H-row per lane (H / 512, rounded up). All of
// an item's loads are issued before any arithmetic.

// logit of (row t, expert e): exact fp64 sum of bf16 products, one rounding
template <int NB>
__device__ void router_item(const FusedArgs &a, int t, int e, int lane) {
    const uint16_t *xr = a.x + (int64_t)t * a.H;
    const uint16_t *wr = a.router_w + (int64_t)e * a.H;
    const int nc8 = a.H / 8;
    uint4 xv[NB], wv[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int c = lane + WAVE * i;
        xv[i] = c < nc8 ? ld16(xr + c * 8) : make_uint4(0, 0, 0, 0);
        wv[i] = c < nc8 ? ld16(wr + c * 8) : make_uint4(0, 0, 0, 0);
    }
    double acc0 = 0.0, acc1 = 0.0;  // two independent chains
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const uint32_t xs[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
        const uint32_t ws[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc0 = fma((double)bf16_lo(xs[k]), (double)bf16_lo(ws[k]), acc0);
            acc1 = fma((double)bf16_hi(xs[k]), (double)bf16_hi(ws[k]), acc1);
        }
    }
    const double acc = wave_allsum_d(acc0 + acc1);
    if (lane < REPL) {
        float l = (float)acc;
        if (!(a.flags & K_LOGITS_FP32)) l = __uint_as_float(f32_to_bf16(l) << 16);
        if (a.bias) l = l + a.bias[e];
        st_dev(a.logits + (int64_t)(lane * a.T + t) * a.E + e, l);
    }
}

__device__ __forceinline__ float dot8_bf16_regs(uint4 a, uint4 b, float acc) {
    const uint32_t as[4] = {a.x, a.y, a.z, a.w}, bs[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        acc = fmaf(bf16_lo(as[k]), bf16_lo(bs[k]), acc);
        acc = fmaf(bf16_hi(as[k]), bf16_hi(bs[k]), acc);
    }
    return acc;
}

// one shared-expert row n of row t: hs = bf16(silu(g) * u); loads first
template <int NB>
struct SharedRegs {
    uint4 x[NB], g[NB], u[NB];
};

template <int NB>
__device__ __forceinline__ void shared_load(const FusedArgs &a, int t, int n, int lane,
                                            SharedRegs<NB> &r) {
    const uint16_t *xr = a.x + (int64_t)t * a.H;
    const int nc8 = a.H / 8;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int c = lane + WAVE * i;
        const bool ok = c < nc8;
        r.x[i] = ok ? ld16(xr + c * 8) : make_uint4(0, 0, 0, 0);
        r.g[i] = ok ? ld16(a.sh_gate + (int64_t)n * a.H + c * 8) : make_uint4(0, 0, 0, 0);
        r.u[i] = ok ? ld16(a.sh_up + (int64_t)n * a.H + c * 8) : make_uint4(0, 0, 0, 0);
    }
}

template <int NB>
__device__ __forceinline__ void shared_compute(const FusedArgs &a, int t, int n, int lane,
                                               const SharedRegs<NB> &r) {
    float g = 0.0f, u = 0.0f;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        g = dot8_bf16_regs(r.x[i], r.g[i], g);
        u = dot8_bf16_regs(r.x[i], r.u[i], u);
    }
    g = wave_allsum(g);
    u = wave_allsum(u);
    if (lane < REPL)
        st_dev(a.hs + (int64_t)(lane * a.T + t) * a.Is + n, (uint16_t)f32_to_bf16(silu(g) * u));
}

template <int NB>
__device__ void gamma_item(const FusedArgs &a, int t, int lane) {
    const uint16_t *xr = a.x + (int64_t)t * a.H;
    const int nc8 = a.H / 8;
    uint4 xv[NB], wv[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int c = lane + WAVE * i;
        xv[i] = c < nc8 ? ld16(xr + c * 8) : make_uint4(0, 0, 0, 0);
        wv[i] = c < nc8 ? ld16(a.sh_gate_w + c * 8) : make_uint4(0, 0, 0, 0);
    }
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < NB; ++i) z = dot8_bf16_regs(xv[i], wv[i], z);
    z = wave_allsum(z);
    if (lane < REPL) st_dev(a.gamma + lane * a.T + t, 1.0f / (1.0f + expf(-z)));
}

// ------------------------------------------------------------- phase B

// routed rows n0..n0+GU_ROWS-1 of pair p: h = silu(g) * u (fp32); loads first
template <int NC>
struct GateUpRegs {
    uint4 g[NC][GU_ROWS], u[NC][GU_ROWS];
};

template <int NC>
__device__ __forceinline__ void gateup_load(const FusedArgs &a, int n0, int e, int lane,
                                            GateUpRegs<NC> &r) {
    const int H = a.H, I = a.I, nchunk = H / 16;
    const uint8_t *wg = a.w_gate + ((int64_t)e * I + n0) * H;
    const uint8_t *wu = a.w_up + ((int64_t)e * I + n0) * H;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + WAVE * i;
#pragma unroll
        for (int q = 0; q < GU_ROWS; ++q) {
            if (c < nchunk) {
                r.g[i][q] = ld16(wg + (int64_t)q * H + c * 16);
                r.u[i][q] = ld16(wu + (int64_t)q * H + c * 16);
            } else {
                r.g[i][q] = r.u[i][q] = make_uint4(0, 0, 0, 0);
            }
        }
    }
}

template <int NC>
__device__ __forceinline__ void gateup_compute(const FusedArgs &a, int p, int n0, int e,
                                               const uint8_t *qx, const float *sx, int lane,
                                               const GateUpRegs<NC> &r) {
    const int H = a.H, I = a.I, nchunk = H / 16, KB = H / GROUP;
    const float *sg = a.s_gate + ((int64_t)e * (I / GROUP) + n0 / GROUP) * KB;
    const float *su = a.s_up + ((int64_t)e * (I / GROUP) + n0 / GROUP) * KB;
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
            for (int q = 0; q < GU_ROWS; ++q) {
                accg[q] = fmaf(s * sg[b], dot16_fp8(xq, r.g[i][q]), accg[q]);
                accu[q] = fmaf(s * su[b], dot16_fp8(xq, r.u[i][q]), accu[q]);
            }
        }
    }
    float hv = 0.0f;
#pragma unroll
    for (int q = 0; q < GU_ROWS; ++q) {
        const float g = wave_allsum(accg[q]), u = wave_allsum(accu[q]);
        if (lane % GU_ROWS == q) hv = silu(g) * u;
    }
    if (lane < GU_ROWS * REPL)
        st_dev(a.h + ((int64_t)(lane / GU_ROWS) * a.T * a.K + p) * I + n0 + lane % GU_ROWS, hv);
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
// row, CPL 16-byte chunks per lane of one I-long down row. The weight loads
// are split from the arithmetic so a wave can issue its first item's down
// rows before the routed gate/up work and the second handoff.
constexpr int SD_CH = 4;  // shared down-row chunks per lane held in registers

template <int KMAX, int CPL>
struct DownRegs {
    uint4 w[KMAX][CPL];  // routed down rows (known after routing)
    uint4 s[SD_CH];      // shared down row (known at kernel start)
};

template <int KMAX, int CPL, int LPR>
__device__ __forceinline__ void down_load_shared(const FusedArgs &a, int m, int sub,
                                                 DownRegs<KMAX, CPL> &r) {
    const uint16_t *srow = a.sh_down + (int64_t)m * a.Is;
#pragma unroll
    for (int i = 0; i < SD_CH; ++i) {
        const int c = sub + LPR * i;
        r.s[i] = c < a.Is / 8 ? ld16(srow + c * 8) : make_uint4(0, 0, 0, 0);
    }
}

template <int KMAX, int CPL, int LPR>
__device__ __forceinline__ void down_load_routed(const FusedArgs &a, int t, int m, int sub,
                                                 const int32_t *ids, DownRegs<KMAX, CPL> &r) {
    const int H = a.H, I = a.I, K = a.K;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
        if (j < K) {
            const uint8_t *row = a.w_down + ((int64_t)ids[t * K + j] * H + m) * I;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = sub + LPR * i;
                r.w[j][i] = c < I / 16 ? ld16(row + c * 16) : make_uint4(0, 0, 0, 0);
            }
        }
}

// hs chunks and gamma of row t for one shared down row, from this
// workgroup's replica (written by other workgroups: device-coherent loads)
struct HsRegs {
    uint64_t h[SD_CH][2];
    float gamma;
};

template <int LPR>
__device__ __forceinline__ void hs_load(const FusedArgs &a, int t, int sub, HsRegs &r) {
    const int rp = blockIdx.x % REPL;
    const uint64_t *hsr =
        reinterpret_cast<const uint64_t *>(a.hs + (int64_t)(rp * a.T + t) * a.Is);
#pragma unroll
    for (int i = 0; i < SD_CH; ++i) {
        const int c = sub + LPR * i;
        r.h[i][0] = c < a.Is / 8 ? ld_dev(hsr + 2 * c) : 0ull;
        r.h[i][1] = c < a.Is / 8 ? ld_dev(hsr + 2 * c + 1) : 0ull;
    }
    r.gamma = ld_dev(a.gamma + rp * a.T + t);
}

__device__ __forceinline__ float dot8_bf16_pair(uint4 w8, uint64_t h01, uint64_t h23) {
    const uint32_t hs[4] = {(uint32_t)h01, (uint32_t)(h01 >> 32), (uint32_t)h23,
                            (uint32_t)(h23 >> 32)};
    const uint32_t ws[4] = {w8.x, w8.y, w8.z, w8.w};
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc = fmaf(bf16_lo(hs[i]), bf16_lo(ws[i]), acc);
        acc = fmaf(bf16_hi(hs[i]), bf16_hi(ws[i]), acc);
    }
    return acc;
}

// gamma * (shared down row m . hs[t]), reduced over the row's LPR lanes
template <int KMAX, int CPL, int LPR>
__device__ float shared_down(const FusedArgs &a, int t, int m, int sub,
                             const DownRegs<KMAX, CPL> &r, const HsRegs &hr) {
    const int Is = a.Is;
    if (Is == 0) return 0.0f;
    float sacc = 0.0f;
#pragma unroll
    for (int i = 0; i < SD_CH; ++i) {
        const int c = sub + LPR * i;
        if (c < Is / 8) sacc += dot8_bf16_pair(r.s[i], hr.h[i][0], hr.h[i][1]);
    }
    if (Is / 8 > LPR * SD_CH) {  // rows longer than the register copy
        const int rp = blockIdx.x % REPL;
        const uint64_t *hsr =
            reinterpret_cast<const uint64_t *>(a.hs + (int64_t)(rp * a.T + t) * Is);
        const uint16_t *srow = a.sh_down + (int64_t)m * Is;
        for (int c = sub + LPR * SD_CH; c < Is / 8; c += LPR)
            sacc += dot8_bf16_pair(ld16(srow + c * 8), ld_dev(hsr + 2 * c), ld_dev(hsr + 2 * c + 1));
    }
    return hr.gamma * seg_sum<LPR>(sacc);
}

// routed down rows and the combine: y = bf16(sum_j w_j e_j + gs), gs from
// shared_down
template <int KMAX, int CPL, int LPR>
__device__ void down_compute(const FusedArgs &a, int t, int m, int sub, const uint8_t *qh,
                             const float *shs, const int32_t *ids, const float *wts,
                             const DownRegs<KMAX, CPL> &r, float gs) {
    const int H = a.H, I = a.I, K = a.K, IB = I / GROUP;
    // each lane sums its slots' partial products (weight applied per slot,
    // slots in order), then one reduction over the row's lanes
    float yacc = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
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
                    acc = fmaf(shs[p * IB + b] * sd[b], dot16_fp8(hq, r.w[j][i]), acc);
                }
            }
            yacc = fmaf(wts[p], acc, yacc);
        }
    yacc = seg_sum<LPR>(yacc) + gs;
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
            // h was written by other workgroups: device-coherent loads
            const uint64_t *p = reinterpret_cast<const uint64_t *>(
                static_cast<const float *>(src) + (int64_t)g * GROUP + sub * 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint64_t v = ld_dev(p + i);
                f[2 * i] = __uint_as_float((uint32_t)v);
                f[2 * i + 1] = __uint_as_float((uint32_t)(v >> 32));
            }
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

template <int NC, int KMAX, int CPL, int LPR>
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
    constexpr int NB = 2 * NC;  // bf16 H-row chunks per lane
    const int gw = wave * a.nwg + blockIdx.x;  // workgroup-major wave index
    if (threadIdx.x == 0) s_target = ld_dev(a.sync) + 1u;

    constexpr int RPP = WAVE / LPR;
    const int sub = lane % LPR, rsel = lane / LPR;
    const int items = T * (H / RPP);  // phase-C output row blocks
    const int t_first = gw / (H / RPP), m_first = (gw % (H / RPP)) * RPP + rsel;
    DownRegs<KMAX, CPL> dr;

    // A: router logits, shared-expert gate/up rows and the shared gate. Every
    // load that does not depend on the routing is issued here, including
    // this wave's first shared down row (kept in registers until phase C).
    if (gw < items && a.Is > 0) down_load_shared<KMAX, CPL, LPR>(a, m_first, sub, dr);
    const int n_router = T * a.E, n_shrows = T * a.Is, n_gamma = a.Is > 0 ? T : 0;
    for (int it = gw; it < n_router + n_shrows + n_gamma; it += nw) {
        if (it < n_router) {
            router_item<NB>(a, it / a.E, it % a.E, lane);
        } else if (it < n_router + n_shrows) {
            const int sidx = it - n_router;
            SharedRegs<NB> sr;
            shared_load<NB>(a, sidx / a.Is, sidx % a.Is, lane, sr);
            shared_compute<NB>(a, sidx / a.Is, sidx % a.Is, lane, sr);
        } else {
            gamma_item<NB>(a, it - n_router - n_shrows, lane);
        }
    }
    quant_to_lds<true>(a.x, T * (H / GROUP), qx, sx);  // needed from phase B on
    __syncthreads();
    const uint32_t target = s_target;
    handoff(a, 0, target);
    // every workgroup has read the generation word: advance it for the next call
    if (blockIdx.x == 0 && threadIdx.x == 0) st_dev(a.sync, target + 1u);

    // B: top-K per row (one wave per row); issue this wave's first block of
    // routed down rows; then the routed gate/up rows
    for (int t = wave; t < T; t += 4)
        topk_row<true>(a.logits + (int64_t)((blockIdx.x % REPL) * T + t) * a.E, a.E, K, lane,
                       ids + t * K, wts + t * K, !a.bias && !(a.flags & K_LOGITS_FP32));
    __syncthreads();
    HsRegs hr;
    if (gw < items) {
        down_load_routed<KMAX, CPL, LPR>(a, t_first, m_first, sub, ids, dr);
        if (a.Is > 0) hs_load<LPR>(a, t_first, sub, hr);
    }
    const int per_pair = I / GU_ROWS;
    for (int it = gw; it < P * per_pair; it += nw) {
        const int p = it / per_pair, n0 = (it % per_pair) * GU_ROWS, t = p / K;
        GateUpRegs<NC> gr;
        gateup_load<NC>(a, n0, ids[p], lane, gr);
        gateup_compute<NC>(a, p, n0, ids[p], qx + t * H, sx + t * (H / GROUP), lane, gr);
    }
    // the first item's shared-expert term needs only phase-A results
    float gs_first = 0.0f;
    if (gw < items) gs_first = shared_down<KMAX, CPL, LPR>(a, t_first, m_first, sub, dr, hr);
    handoff(a, 1, target);

    // C: re-quantise h, then whole output rows with the combine
    quant_to_lds<false>(a.h + (int64_t)(blockIdx.x % REPL) * P * I, P * (I / GROUP), qh, shs);
    __syncthreads();
    for (int it = gw; it < items; it += nw) {
        const int t = it / (H / RPP);
        const int m = (it % (H / RPP)) * RPP + rsel;
        float gsv = gs_first;
        if (it != gw) {
            if (a.Is > 0) {
                down_load_shared<KMAX, CPL, LPR>(a, m, sub, dr);
                hs_load<LPR>(a, t, sub, hr);
            }
            down_load_routed<KMAX, CPL, LPR>(a, t, m, sub, ids, dr);
            gsv = shared_down<KMAX, CPL, LPR>(a, t, m, sub, dr, hr);
        }
        down_compute<KMAX, CPL, LPR>(a, t, m, sub, qh, shs, ids, wts, dr, gsv);
    }
}

template <int NC, int KMAX>
static hipError_t launch_k(const FusedArgs &a, size_t lds, hipStream_t st) {
    const dim3 grid(a.nwg), block(256);
    const int chunks = a.I / 16;
    if (chunks <= 8)
        hipLaunchKernelGGL((decode_fused_kernel<NC, KMAX, 1, 8>), grid, block, lds, st, a);
    else if (chunks <= 16)
        hipLaunchKernelGGL((decode_fused_kernel<NC, KMAX, 1, 16>), grid, block, lds, st, a);
    else if (chunks <= 32)
        hipLaunchKernelGGL((decode_fused_kernel<NC, KMAX, 1, 32>), grid, block, lds, st, a);
    else if (chunks <= 64)
        hipLaunchKernelGGL((decode_fused_kernel<NC, KMAX, 1, 64>), grid, block, lds, st, a);
    else if (chunks <= 128)
        hipLaunchKernelGGL((decode_fused_kernel<NC, KMAX, 2, 64>), grid, block, lds, st, a);
    else
        hipLaunchKernelGGL((decode_fused_kernel<NC, KMAX, 4, 64>), grid, block, lds, st, a);
    return hipGetLastError();
}

template <int NC>
static hipError_t launch_nc(const FusedArgs &a, size_t lds, hipStream_t st) {
    if (a.K <= 4) return launch_k<NC, 4>(a, lds, st);
    if (a.K <= 8) return launch_k<NC, 8>(a, lds, st);
    return launch_k<NC, 16>(a, lds, st);
}

template <int NC, int KMAX, int CPL, int LPR>
static void set_lds_limit() {
    (void)hipFuncSetAttribute(
        reinterpret_cast<const void *>(&decode_fused_kernel<NC, KMAX, CPL, LPR>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
}

template <int NC, int KMAX>
static void set_lds_limits_k() {
    set_lds_limit<NC, KMAX, 1, 8>();
    set_lds_limit<NC, KMAX, 1, 16>();
    set_lds_limit<NC, KMAX, 1, 32>();
    set_lds_limit<NC, KMAX, 1, 64>();
    set_lds_limit<NC, KMAX, 2, 64>();
    set_lds_limit<NC, KMAX, 4, 64>();
}

template <int NC>
static void set_lds_limits() {
    set_lds_limits_k<NC, 4>();
    set_lds_limits_k<NC, 8>();
    set_lds_limits_k<NC, 16>();
}

hipError_t launch_decode_fused(const FusedArgs &a, hipStream_t st) {
    const size_t lds = (size_t)lds_plan(a.T, a.H, a.K, a.I).total;
    if (lds > 64 * 1024) {
        static const bool once = [] {
            set_lds_limits<1>();
            set_lds_limits<2>();
            set_lds_limits<4>();
            set_lds_limits<8>();
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
