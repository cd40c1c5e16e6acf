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

// Scale of one 128-wide group from its amax: fp32(max(amax, 1e-10) / 448),
// with a correctly rounded division (the library is built with
// -fhip-fp32-correctly-rounded-divide-sqrt).
__device__ __forceinline__ float group_scale(float amax) { return fmaxf(amax, 1e-10f) / 448.0f; }

// ------------------------------------------------------- wave reductions

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

// 16-byte global load/store helpers.
__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void st16(void *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }

}  // namespace moe
