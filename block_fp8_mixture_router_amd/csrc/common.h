// Device helpers shared by the gfx950 kernels of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int GROUP = 128;  // activation group width and weight block edge
constexpr int WAVE = 64;    // CDNA wavefront

typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef double v4d __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) {
    return __uint_as_float(pair & 0xFFFF0000u);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// ------------------------------------------------------------------ e4m3
// OCP e4m3 is gfx950's native FP8 format. v_cvt_pk_fp8_f32 rounds to
// nearest even; values are saturated to +-448 first (without saturation an
// out-of-range value would become NaN).

__device__ __forceinline__ float sat448(float v) { return __builtin_amdgcn_fmed3f(v, 448.0f, -448.0f); }

// Four saturated fp32 values -> four e4m3 codes packed little-endian.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), r, true);
    return (uint32_t)r;
}

// Decode the four e4m3 codes of a 32-bit word.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float &a, float &b, float &c, float &d) {
    v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    a = lo.x;
    b = lo.y;
    c = hi.x;
    d = hi.y;
}

// Eight e4m3 codes (a uint2) -> eight bf16 values (exact: every e4m3 value
// is a bf16 value).
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint2 c) {
    float f[8];
    e4m3x4_to_f32(c.x, f[0], f[1], f[2], f[3]);
    e4m3x4_to_f32(c.y, f[4], f[5], f[6], f[7]);
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = f32_to_bf16(f[2 * k]) | (f32_to_bf16(f[2 * k + 1]) << 16);
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Scale of one 128-wide group from its amax: fp32(max(amax, 1e-10) / 448),
// with a correctly rounded division (the library is built with
// -fhip-fp32-correctly-rounded-divide-sqrt).
__device__ __forceinline__ float group_scale(float amax) { return fmaxf(amax, 1e-10f) / 448.0f; }

// ------------------------------------------------------- wave reductions
// DPP lane moves inside rows of 16 lanes, then v_readlane across the four
// rows: no LDS round trips on the dependency chain. Every lane of the wave
// must be active.

constexpr int DPP_XOR1 = 0xB1;         // quad_perm(1,0,3,2)
constexpr int DPP_XOR2 = 0x4E;         // quad_perm(2,3,0,1)
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7-i within 8
constexpr int DPP_MIRROR = 0x140;      // lane i <-> 15-i within 16

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const int lo = dpp_i<CTRL>((int)(uint32_t)u), hi = dpp_i<CTRL>((int)(uint32_t)(u >> 32));
    return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
__device__ __forceinline__ float readlane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double readlane_d(double v, int l) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// all-lanes sum / max / min over the 64-lane wave (fixed order: deterministic)
__device__ __forceinline__ float wave_allsum(float v) {
    v += dpp_f<DPP_XOR1>(v);
    v += dpp_f<DPP_XOR2>(v);
    v += dpp_f<DPP_HALF_MIRROR>(v);
    v += dpp_f<DPP_MIRROR>(v);
    return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
__device__ __forceinline__ double wave_allsum_d(double v) {
    v += dpp_d<DPP_XOR1>(v);
    v += dpp_d<DPP_XOR2>(v);
    v += dpp_d<DPP_HALF_MIRROR>(v);
    v += dpp_d<DPP_MIRROR>(v);
    return (readlane_d(v, 0) + readlane_d(v, 16)) + (readlane_d(v, 32) + readlane_d(v, 48));
}
__device__ __forceinline__ float wave_allmax(float v) {
    v = fmaxf(v, dpp_f<DPP_XOR1>(v));
    v = fmaxf(v, dpp_f<DPP_XOR2>(v));
    v = fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
    v = fmaxf(v, dpp_f<DPP_MIRROR>(v));
    return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)),
                 fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ int wave_allmin_i(int v) {
    v = min(v, dpp_i<DPP_XOR1>(v));
    v = min(v, dpp_i<DPP_XOR2>(v));
    v = min(v, dpp_i<DPP_HALF_MIRROR>(v));
    v = min(v, dpp_i<DPP_MIRROR>(v));
    return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
// max over aligned groups of 8 lanes (result in every lane of the group)
__device__ __forceinline__ float group8_max(float v) {
    v = fmaxf(v, dpp_f<DPP_XOR1>(v));
    v = fmaxf(v, dpp_f<DPP_XOR2>(v));
    return fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
}
// max / sum over aligned groups of 16 lanes
__device__ __forceinline__ float group16_max(float v) {
    v = group8_max(v);
    return fmaxf(v, dpp_f<DPP_MIRROR>(v));
}
__device__ __forceinline__ float group16_sum(float v) {
    v += dpp_f<DPP_XOR1>(v);
    v += dpp_f<DPP_XOR2>(v);
    v += dpp_f<DPP_HALF_MIRROR>(v);
    return v + dpp_f<DPP_MIRROR>(v);
}
// sum over aligned groups of 32 lanes
__device__ __forceinline__ float group32_sum(float v) {
    v = group16_sum(v);
    return v + __shfl_xor(v, 16);
}


template <int WIDTH>
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WIDTH));
    return v;
}

template <int WIDTH>
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WIDTH);
    return v;
}

template <int WIDTH>
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WIDTH);
    return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// fp32 rounded to the nearest bf16 value (kept as fp32)
__device__ __forceinline__ float bf16_round(float f) { return __uint_as_float(f32_to_bf16(f) << 16); }

// ------------------------------------------------------------ matrix cores
// Block products shared by the expert-grouped kernels and the one-row
// kernel. An output element of these MFMAs depends only on its own row of A
// and column of B: on gfx950 it is the same bits at every position in the
// tile, whatever the other rows and columns hold, and with the operands
// swapped. So a row computed alone, in any tile position, gets the bits it
// gets inside a chunk, provided the same operand bytes meet in the same
// instruction sequence.

__device__ __forceinline__ v8i as_v8i(uint4 lo, uint4 hi) {
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

// One 128x128 weight block: v_mfma_scale_f32_16x16x128_f8f6f4 on e4m3
// operands, from zero, E8M0 scales 127 (x1). Lane (l16, kq) supplies A row
// l16 and B column l16, bytes [32 kq, 32 kq + 32) of the block; element i of
// its result is row 4 kq + i, column l16.
__device__ __forceinline__ v4f mfma_fp8_k128(v8i a, v8i b) {
    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ v8bf as_v8bf(uint4 v) { return __builtin_bit_cast(v8bf, v); }

// bf16 16x16x32 MFMA accumulating into c. Lane (l16, kq) supplies A row l16
// and B column l16, eight bf16 elements each.
__device__ __forceinline__ v4f mfma_bf16_k32(v8bf a, v8bf b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Row RMS normalisation between stacked layers, shared by the stand-alone
// kernel and the renormalising prologue of the one-row kernel so both give
// the same bits. A workgroup of 256 threads owns the row; thread tid holds
// the 16-byte chunks tid + 256 i, i < RENORM_CHUNKS (H <= 8192). It adds the
// exact squares of its chunks in element order (fp64), a DPP wave sum and
// the four wave totals in order give the row sum, the scale is
// 1 / sqrt(fp32(sum / H) + eps) in fp32 and x = bf16(fp32(y * scale)).
constexpr int RENORM_CHUNKS = 4;

__device__ __forceinline__ double sumsq8(const float (&v)[8], double acc) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc = fma((double)v[k], (double)v[k], acc);
    return acc;
}
// sum / H correctly rounded: for a power-of-two H the exact scaling by
// 2^-log2(H) (one instruction, rounded only if the result is subnormal, as
// the division would be), else the division
__device__ __forceinline__ float rms_scale(double sum, int H, float eps) {
    const double q = (H & (H - 1)) == 0 ? ldexp(sum, -__builtin_ctz((unsigned)H)) : sum / (double)H;
    const float ms = (float)q;
    return 1.0f / sqrtf(ms + eps);
}

// The row's scale from this thread's chunks (zero past H). part: 4 doubles
// of LDS; every thread of the workgroup calls this (it has a barrier), and
// part may be written again only after a later barrier.
// CH: the thread's chunks (a caller whose rows fit in fewer than
// RENORM_CHUNKS passes fewer: the chunks past H hold zeros, whose squares
// leave the sum unchanged).
template <int CH>
__device__ __forceinline__ float renorm_row_scale(const uint4 (&v)[CH], int H, float eps,
                                                  double *part) {
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const float f[8] = {bf16_lo(v[i].x), bf16_hi(v[i].x), bf16_lo(v[i].y), bf16_hi(v[i].y),
                            bf16_lo(v[i].z), bf16_hi(v[i].z), bf16_lo(v[i].w), bf16_hi(v[i].w)};
        acc = sumsq8(f, acc);
    }
    acc = wave_allsum_d(acc);
    if ((threadIdx.x & (WAVE - 1)) == 0) part[threadIdx.x / WAVE] = acc;
    __syncthreads();
    const double sum = ((part[0] + part[1]) + part[2]) + part[3];
    return rms_scale(sum, H, eps);
}

// eight bf16 values times the row scale, rounded back to bf16
__device__ __forceinline__ uint4 renorm_chunk(uint4 v, float r) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float lo = bf16_lo(w[k]) * r, hi = bf16_hi(w[k]) * r;
        o[k] = f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// 16-byte global load/store helpers.
__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void st16(void *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }

}  // namespace moe
