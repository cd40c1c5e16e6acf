// Dynamic 1x128 e4m3 activation quantisation (PR #925 "drama: load the
// checkpoint with direct I/O in file order and build the codec on its own
// thread", backbone commit summary; PR #939 "drama3: Fish Audio Drama 3 text
// to speech on one CUDA GPU", "How it fits the engine" > Precision).
//
// HBM-bound: reads 256 B and writes 132 B per group. Sixteen lanes own one
// 128-column group, each lane one 16-byte load of 8 bf16 values, so a wave
// covers four groups with fully coalesced loads and 8-byte code stores; the
// group's amax is a 16-lane max reduction.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t *__restrict__ x,
                                                        int64_t n_groups,
                                                        uint8_t *__restrict__ q,
                                                        float *__restrict__ s) {
    const int64_t g = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int sub = threadIdx.x & 15;
    if (g >= n_groups) return;  // whole 16-lane segments leave together
    const uint4 v = ld16(x + g * GROUP + sub * 8);
    float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                  bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = wave_max<16>(amax);
    const float sc = group_scale(amax);
    uint2 out;
    out.x = e4m3x4(f[0] / sc, f[1] / sc, f[2] / sc, f[3] / sc);
    out.y = e4m3x4(f[4] / sc, f[5] / sc, f[6] / sc, f[7] / sc);
    *reinterpret_cast<uint2 *>(q + g * GROUP + sub * 8) = out;
    if (sub == 0) s[g] = sc;
}

// The fp32 -> e4m3 conversion every kernel uses (e4m3x4: saturate to +-448,
// round to nearest even), applied to n values: four per thread, grid-stride.
__global__ __launch_bounds__(256) void e4m3_encode_kernel(const float *__restrict__ x, int64_t n,
                                                          uint8_t *__restrict__ q) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
    for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
        if (i + 4 <= n) {
            const float4 v = *reinterpret_cast<const float4 *>(x + i);
            *reinterpret_cast<uint32_t *>(q + i) = e4m3x4(v.x, v.y, v.z, v.w);
        } else {
            for (int64_t k = i; k < n; ++k) q[k] = (uint8_t)(e4m3x4(x[k], 0.f, 0.f, 0.f) & 0xFFu);
        }
    }
}

hipError_t launch_e4m3_encode(const float *x, int64_t n, uint8_t *q, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int64_t quads = (n + 3) / 4;
    const int64_t blocks = (quads + 255) / 256 < 8192 ? (quads + 255) / 256 : 8192;
    hipLaunchKernelGGL(e4m3_encode_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, n, q);
    return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t *x, int64_t n_groups, uint8_t *q, float *s,
                            hipStream_t st) {
    if (n_groups <= 0) return hipSuccess;
    const int64_t blocks = (n_groups + 15) / 16;
    hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, n_groups,
                       q, s);
    return hipGetLastError();
}

}  // namespace moe
