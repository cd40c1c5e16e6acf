// Router: logits, top-K selection and renormalised softmax.
//
// The pages' router decides on bf16 logits and runs its softmax in fp32
// (PR #939 "drama3: Fish Audio Drama 3 text to speech on one CUDA GPU",
// "Fidelity against the PyTorch oracle" and "How it fits the engine" >
// Precision). bf16 logits tie often, so any change of summation order would
// move picks; each logit here is the exact sum of the exact bf16 x bf16
// products, accumulated in fp64 and rounded once to fp32, then to bf16.
//
// Logit kernels:
//  - few rows (decode): one wave per (row, expert), 16-byte loads, fp64 FMA,
//    a wave reduction; the 1 MiB router matrix streams once per row.
//  - many rows, every logit wanted (moe_route with a logits buffer): fp64
//    MFMA 16x16x4 tiles; each lane streams 32 contiguous bytes of its row and
//    of its experts per 64 columns and the MFMA sums over the lanes' column
//    slices.
//  - many rows, only the top-K wanted (the layer): bf16 MFMA scores S (fp32
//    sums of the exact products) and A (the same for |x||w|), which bound
//    the exact sum to S +- delta(A); each row's wave rules out every expert
//    whose upper bound falls below the K-th largest lower bound and computes
//    the exact logits (fp64) of the few that remain. The picks and weights
//    are those of the exact logits.
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

// ------------------------------------------------------ bounded scores

// A workgroup owns 32 rows x 32 experts (two 16-row tiles times two
// 16-expert tiles: 256 KiB of operands per workgroup at H = 2048, the least
// for 256 workgroups over these shapes; the kernel is bound by what each CU
// pulls from L2); wave w sums the 128-column blocks w, w+4, ...; lane
// (l16, kq) supplies columns [32kq, 32kq + 32) of each block of its rows
// (A operands) and of its experts' rows (B operands), split over four
// 16x16x32 MFMAs. Each MFMA starts from zero and its 32-product partial is
// added in fp64, so a score carries the rounding error of one 32-term fp32
// sum per chunk only. A second MFMA on the sign-stripped operands sums
// |x||w| in fp32 (chained), for the bound. The four waves' partials are
// added in LDS in a fixed order.
// 1-D grid: the expert blocks of a row tile sit 8 workgroups apart, so with
// workgroups dealt round-robin over the 8 XCDs they share one L2 and the
// tile's rows come from memory once.
__global__ __launch_bounds__(256) void route_scores_bf16(const uint16_t *__restrict__ x, int T,
                                                         const uint16_t *__restrict__ rw, int H,
                                                         int E, float *__restrict__ S,
                                                         float *__restrict__ A) {
    __shared__ double sp[4][4][64][4];  // [wave][(row tile, expert tile)][lane][element]
    __shared__ float ap[4][4][64][4];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, kq = lane >> 4;
    const int nE = (E + 31) / 32, nT = (T + 31) / 32;
    // linear id L -> (row tile, expert block): L = 8 * (nE * g + eb) + r, tile = 8g + r
    const int L = blockIdx.x, r8 = L % 8, q = L / 8;
    const int eb = q % nE, tt = (q / nE) * 8 + r8;
    if (tt >= nT) return;
    const int e0 = eb * 32, t0 = tt * 32;
    // rows and experts past the end read a valid row; their results are dropped
    const uint16_t *xr[2], *wr[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        xr[u] = x + (int64_t)min(t0 + 16 * u + l16, T - 1) * H + 32 * kq;
        wr[u] = rw + (int64_t)min(e0 + 16 * u + l16, E - 1) * H + 32 * kq;
    }
    double sd[2][2][4] = {};  // [row tile][expert tile][element]
    v4f aa[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int j = 0; j < 2; ++j) aa[rt][j] = (v4f){0.f, 0.f, 0.f, 0.f};
    const int KB = H / GROUP;
    uint4 xv[2][2][4], wv[2][2][4];
    auto load = [&](int kb, uint4 (&xs)[2][4], uint4 (&ws)[2][4]) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xs[u][i] = ld16(xr[u] + kb * GROUP + 8 * i);
                ws[u][i] = ld16(wr[u] + kb * GROUP + 8 * i);
            }
    };
    auto step = [&](const uint4 (&xs)[2][4], const uint4 (&ws)[2][4]) {
        constexpr uint32_t M = 0x7FFF7FFFu;  // clears both bf16 sign bits
        const v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const uint4 xa = xs[rt][i];
                const v8bf af = __builtin_bit_cast(v8bf, xa);
                const v8bf aabs =
                    __builtin_bit_cast(v8bf, make_uint4(xa.x & M, xa.y & M, xa.z & M, xa.w & M));
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const uint4 w = ws[j][i];
                    const v4f p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        af, __builtin_bit_cast(v8bf, w), z, 0, 0, 0);
#pragma unroll
                    for (int k = 0; k < 4; ++k) sd[rt][j][k] += (double)p[k];
                    aa[rt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        aabs,
                        __builtin_bit_cast(v8bf, make_uint4(w.x & M, w.y & M, w.z & M, w.w & M)),
                        aa[rt][j], 0, 0, 0);
                }
            }
    };
    // this wave's blocks kb = wave + 4i, i < nit; two blocks of loads in flight
    const int nit = KB > wave ? (KB - wave + 3) / 4 : 0;
    if (nit > 0) load(wave, xv[0], wv[0]);
    if (nit > 1) load(wave + 4, xv[1], wv[1]);
    for (int it = 0; it < nit; it += 2) {
        step(xv[0], wv[0]);
        if (it + 2 < nit) load(wave + 4 * (it + 2), xv[0], wv[0]);
        if (it + 1 < nit) {
            step(xv[1], wv[1]);
            if (it + 3 < nit) load(wave + 4 * (it + 3), xv[1], wv[1]);
        }
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                sp[wave][2 * rt + j][lane][k] = sd[rt][j][k];
                ap[wave][2 * rt + j][lane][k] = aa[rt][j][k];
            }
    __syncthreads();
    // wave w finishes tile (rt, j) = (w / 2, w % 2); element k of lane
    // (l16, kq) = row 16rt + 4kq + k, expert 16j + l16
    const int tl = wave, rt = wave >> 1, j = wave & 1;
    const int e = e0 + 16 * j + l16;
    if (e >= E) return;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int t = t0 + 16 * rt + 4 * kq + k;
        if (t >= T) continue;
        const double sv = ((sp[0][tl][lane][k] + sp[1][tl][lane][k]) + sp[2][tl][lane][k]) +
                          sp[3][tl][lane][k];
        const float av = ((ap[0][tl][lane][k] + ap[1][tl][lane][k]) + ap[2][tl][lane][k]) +
                         ap[3][tl][lane][k];
        S[(int64_t)t * E + e] = (float)sv;
        A[(int64_t)t * E + e] = av;
    }
}

hipError_t launch_route_scores(const uint16_t *x, int T, const uint16_t *router_w, int H, int E,
                               float *S, float *A, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const int nE = (E + 31) / 32, nT = (T + 31) / 32;
    const int groups = (nT + 7) / 8;  // row tiles come in groups of 8 (one per XCD)
    hipLaunchKernelGGL(route_scores_bf16, dim3(groups * nE * 8), dim3(256), 0, st, x, T,
                       router_w, H, E, S, A);
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

// ------------------------------------------- top-K from bounded scores

// How far the exact sum can lie from the stored score s, given the stored
// |x||w| sum a. Every product is exact in fp32 (bf16 x bf16); each MFMA
// sums 32 of them from zero with at most 31 roundings plus one for its
// output, each of relative size at most u = 2^-23 (truncation allowed), so
// a chunk partial errs by at most 32u/(1 - 32u) times its sum of |p|. The
// fp64 sum of the H/32 partials adds at most (H/32 + 4) 2^-53 of the same,
// and storing the score as fp32 adds half an fp32 ulp of |s|. a itself
// went through at most c = 33 H/32 + 3 roundings and may fall short of
// sum |p| by the factor (1 - c u). Products below 2^-126, which the matrix
// cores may flush, add at most H 2^-126.
__device__ __forceinline__ double score_delta(float s, float a, int H) {
    const double u = 1.0 / 8388608.0;
    const double c = 33.0 * H / 32.0 + 3.0;
    const double chunk = 32.0 * u / (1.0 - 32.0 * u) + (H / 32.0 + 4.0) * 0x1p-53;
    const double sum_abs = (double)a / (1.0 - c * u);
    return chunk * sum_abs * (1.0 + 0x1p-40) + fabs((double)s) * 0x1p-24 + (double)H * 0x1p-126;
}

// Exact logit (fp64 sum of exact products, one rounding to fp32) of expert e
// for the row held in xv (chunk c = lane + 64i of 8 bf16 per lane).
template <int NB>
__device__ __forceinline__ double exact_dot(const uint4 (&xv)[NB], const uint4 (&wv)[NB]) {
    double acc0 = 0.0, acc1 = 0.0;
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
    return wave_allsum_d(acc0 + acc1);
}

constexpr int EXACT_BATCH = 4;  // candidate rows fetched per round trip

// One wave per row t. NL logits per lane (expert e = lane + 64i), NB 16-byte
// chunks of the x row per lane. Writes ids/weights; with gate_w also gamma;
// with qx also the 1x128 quantisation of x[t]. With SPLIT the workgroup has
// eight waves: waves 0-3 pick the experts of rows 4b..4b+3 and waves 4-7
// compute the same rows' gamma and FP8 groups, so neither chain waits for
// the other.
template <int NL, int NB, bool SPLIT>
__global__ __launch_bounds__(SPLIT ? 512 : 256) void route_topk_bounded_kernel(
    const float *__restrict__ S, const float *__restrict__ A, int T, int E, int K,
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ rw,
    const float *__restrict__ bias, uint32_t flags, int H, int32_t *__restrict__ ids,
    float *__restrict__ wts, const uint16_t *__restrict__ gate_w, float *__restrict__ gamma,
    uint8_t *__restrict__ qx, float *__restrict__ sx) {
    const int t = blockIdx.x * 4 + ((threadIdx.x >> 6) & 3);
    const bool side = SPLIT && (threadIdx.x >> 8) != 0;
    const int lane = threadIdx.x & 63;
    if (t >= T) return;  // whole waves leave together
    const int nc8 = H / 8;
    const uint16_t *xr = x + (int64_t)t * H;
    uint4 xv[NB], gv[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int c = lane + WAVE * i;
        xv[i] = c < nc8 ? ld16(xr + c * 8) : make_uint4(0, 0, 0, 0);
        gv[i] = ((!SPLIT || side) && gate_w && c < nc8) ? ld16(gate_w + c * 8)
                                                        : make_uint4(0, 0, 0, 0);
    }
    // gamma[t] and the FP8 groups of x[t]
    auto side_work = [&]() {
        if (gate_w) {
            float z = 0.0f;
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int c = lane + WAVE * i;
                if (c < nc8) {
                    const uint4 b = gv[i];
                    const uint32_t av[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
                    const uint32_t bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        z = fmaf(bf16_lo(av[k]), bf16_lo(bv[k]), z);
                        z = fmaf(bf16_hi(av[k]), bf16_hi(bv[k]), z);
                    }
                }
            }
            z = wave_allsum(z);
            if (lane == 0) gamma[t] = 1.0f / (1.0f + expf(-z));
        }
        if (qx) {
            // 16 lanes per 128-column group: chunk c = lane + 64i is in group c / 16
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int c = lane + WAVE * i;
                if (WAVE * i >= nc8) break;  // wave-uniform
                const uint4 v = xv[i];
                float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                              bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
                float amax = 0.0f;
#pragma unroll
                for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(f[k]));
                amax = group16_max(amax);
                const float sc = group_scale(amax);
                if (c < nc8) {
                    uint2 out;
                    out.x = e4m3x4(f[0] / sc, f[1] / sc, f[2] / sc, f[3] / sc);
                    out.y = e4m3x4(f[4] / sc, f[5] / sc, f[6] / sc, f[7] / sc);
                    *reinterpret_cast<uint2 *>(qx + (int64_t)t * H + c * 8) = out;
                    if ((c & 15) == 0) sx[(int64_t)t * (H / GROUP) + c / 16] = sc;
                }
            }
        }
    };
    if (side) {
        side_work();
        return;
    }

    // intervals [lo, hi] that hold each exact logit
    float lo[NL], hi[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int e = lane + WAVE * i;
        if (e < E) {
            const float sf = S[(int64_t)t * E + e];
            const double sv = sf, d = score_delta(sf, A[(int64_t)t * E + e], H);
            lo[i] = finish_logit(sv - d, bias, e, flags);
            hi[i] = finish_logit(sv + d, bias, e, flags);
        } else {
            lo[i] = hi[i] = -INFINITY;
        }
    }
    // LK = K-th largest lower bound; an expert with hi < LK trails K others
    float LK;
    {
        float v[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) v[i] = lo[i];
#pragma unroll
        for (int r = 0; r < NL; ++r)
#pragma unroll
            for (int i = r & 1; i + 1 < NL; i += 2)
                if (v[i + 1] > v[i]) {
                    const float tv = v[i];
                    v[i] = v[i + 1];
                    v[i + 1] = tv;
                }
        LK = -INFINITY;
        for (int j = 0; j < K; ++j) {
            LK = wave_allmax(v[0]);
            // remove one copy of the maximum (the lowest lane holding it)
            const uint64_t holders = __ballot(v[0] == LK);
            if (lane == (int)__builtin_ctzll(holders)) {
#pragma unroll
                for (int i = 0; i + 1 < NL; ++i) v[i] = v[i + 1];
                v[NL - 1] = -INFINITY;
            }
        }
    }
    // candidates keep their logit once it is exact; the rest drop out
    float val[NL];
    uint64_t pending[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const bool cand = hi[i] >= LK && lane + WAVE * i < E;
        val[i] = cand ? lo[i] : -INFINITY;
        pending[i] = __ballot(cand && lo[i] != hi[i]);
    }
    // exact logits of the undecided candidates, EXACT_BATCH rows per round trip
    for (int i0 = 0; i0 < NL; ++i0) {
        uint64_t m = 0;
#pragma unroll
        for (int i = 0; i < NL; ++i)
            if (i == i0) m = pending[i];
        while (m) {
            int eb[EXACT_BATCH];
            int nb = 0;
#pragma unroll
            for (int b = 0; b < EXACT_BATCH; ++b) {
                eb[b] = -1;
                if (m) {
                    const int l = (int)__builtin_ctzll(m);
                    m &= m - 1;
                    eb[b] = l + WAVE * i0;
                    ++nb;
                }
            }
            uint4 wv[EXACT_BATCH][NB];
#pragma unroll
            for (int b = 0; b < EXACT_BATCH; ++b) {
                const uint16_t *wr = rw + (int64_t)(eb[b] >= 0 ? eb[b] : 0) * H;
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    const int c = lane + WAVE * i;
                    wv[b][i] = (b < nb && c < nc8) ? ld16(wr + c * 8) : make_uint4(0, 0, 0, 0);
                }
            }
#pragma unroll
            for (int b = 0; b < EXACT_BATCH; ++b)
                if (b < nb) {
                    const float l = finish_logit(exact_dot<NB>(xv, wv[b]), bias, eb[b], flags);
                    const int owner = eb[b] - WAVE * i0;
#pragma unroll
                    for (int i = 0; i < NL; ++i)
                        if (i == i0 && lane == owner) val[i] = l;
                }
        }
    }
    {
        int ix[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) ix[i] = lane + WAVE * i < E ? lane + WAVE * i : 0x7FFFFFFF;
        topk_select_n<NL>(val, ix, K, lane, ids + (int64_t)t * K, wts + (int64_t)t * K);
    }
    if (!SPLIT) side_work();
}

template <int NL>
static hipError_t launch_bounded_nl(const float *S, const float *A, int T, int E, int K,
                                    const uint16_t *x, const uint16_t *rw, const float *bias,
                                    uint32_t flags, int H, int32_t *ids, float *wts,
                                    const uint16_t *gate_w, float *gamma, uint8_t *qx,
                                    float *sx, hipStream_t st) {
    const dim3 grid((T + 3) / 4);
    const int nb = (H / 8 + WAVE - 1) / WAVE;
    // side waves for gamma and the FP8 groups when there is such work (and
    // the row fits the 256 registers a wave gets at eight waves per CU)
    const bool split = (gate_w || qx) && nb <= 8;
#define MOE_BOUNDED(NBV, SP)                                                                  \
    hipLaunchKernelGGL((route_topk_bounded_kernel<NL, NBV, SP>), grid, dim3(SP ? 512 : 256), 0, \
                       st, S, A, T, E, K, x, rw, bias, flags, H, ids, wts, gate_w, gamma, qx, sx)
    if (split) {
        if (nb <= 1) MOE_BOUNDED(1, true);
        else if (nb <= 2) MOE_BOUNDED(2, true);
        else if (nb <= 4) MOE_BOUNDED(4, true);
        else MOE_BOUNDED(8, true);
    } else {
        if (nb <= 1) MOE_BOUNDED(1, false);
        else if (nb <= 2) MOE_BOUNDED(2, false);
        else if (nb <= 4) MOE_BOUNDED(4, false);
        else if (nb <= 8) MOE_BOUNDED(8, false);
        else MOE_BOUNDED(16, false);
    }
#undef MOE_BOUNDED
    return hipGetLastError();
}

hipError_t launch_route_topk_bounded(const float *S, const float *A, int T, int E, int K,
                                     const uint16_t *x, const uint16_t *router_w,
                                     const float *bias, uint32_t flags, int H, int32_t *ids,
                                     float *weights, const uint16_t *gate_w, float *gamma,
                                     uint8_t *qx, float *sx, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (E <= 64)
        return launch_bounded_nl<1>(S, A, T, E, K, x, router_w, bias, flags, H, ids, weights,
                                    gate_w, gamma, qx, sx, st);
    if (E <= 128)
        return launch_bounded_nl<2>(S, A, T, E, K, x, router_w, bias, flags, H, ids, weights,
                                    gate_w, gamma, qx, sx, st);
    if (E <= 256)
        return launch_bounded_nl<4>(S, A, T, E, K, x, router_w, bias, flags, H, ids, weights,
                                    gate_w, gamma, qx, sx, st);
    if (E <= 512)
        return launch_bounded_nl<8>(S, A, T, E, K, x, router_w, bias, flags, H, ids, weights,
                                    gate_w, gamma, qx, sx, st);
    return launch_bounded_nl<16>(S, A, T, E, K, x, router_w, bias, flags, H, ids, weights,
                                 gate_w, gamma, qx, sx, st);
}

}  // namespace moe
