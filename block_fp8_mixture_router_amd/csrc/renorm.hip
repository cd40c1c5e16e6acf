// RMS renormalisation of rows between the layers of a decode stack. The
// backbone normalises every row before its MoE layer (PR #925 "drama: load
// the checkpoint with direct I/O in file order and build the codec on its own
// thread", backbone commit summaries: residual add and RMSnorm ahead of the
// FP8 quantisation); a chain of independent synthetic layers keeps only the
// normalisation, with no learned gain:
//   ms = fp32(sum of exact squares, in fp64, / H); r = 1 / sqrt(ms + eps);
//   x  = bf16(y * r).
// One workgroup per row: each thread loads up to four 16-byte chunks,
// squares and sums them in fp64, a DPP wave sum and a fixed-order sum of the
// four wave totals give the row sum. Reads and writes 2H bytes per row.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void rms_renorm_kernel(const uint16_t *__restrict__ y, int H,
                                                         float eps, uint16_t *x) {
    __shared__ double part[4];
    const int64_t row = blockIdx.x;
    const uint16_t *yr = y + row * H;
    const int nc = H / 8;
    uint4 v[RENORM_CHUNKS];
#pragma unroll
    for (int i = 0; i < RENORM_CHUNKS; ++i) {
        const int c = threadIdx.x + 256 * i;
        v[i] = c < nc ? ld16(yr + c * 8) : make_uint4(0, 0, 0, 0);
    }
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < RENORM_CHUNKS; ++i) {
        const float f[8] = {bf16_lo(v[i].x), bf16_hi(v[i].x), bf16_lo(v[i].y), bf16_hi(v[i].y),
                            bf16_lo(v[i].z), bf16_hi(v[i].z), bf16_lo(v[i].w), bf16_hi(v[i].w)};
        acc = sumsq8(f, acc);  // chunks past H are zero and add nothing
    }
    acc = wave_allsum_d(acc);
    if ((threadIdx.x & (WAVE - 1)) == 0) part[threadIdx.x / WAVE] = acc;
    __syncthreads();  // every load of this row is done before any store (x may alias y)
    const double sum = ((part[0] + part[1]) + part[2]) + part[3];
    const float r = rms_scale(sum, H, eps);
    uint16_t *xr = x + row * H;
#pragma unroll
    for (int i = 0; i < RENORM_CHUNKS; ++i) {
        const int c = threadIdx.x + 256 * i;
        if (c >= nc) continue;
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float a = bf16_lo(w[k]) * r, b = bf16_hi(w[k]) * r;
            o[k] = f32_to_bf16(a) | (f32_to_bf16(b) << 16);
        }
        st16(xr + c * 8, make_uint4(o[0], o[1], o[2], o[3]));
    }
}

hipError_t launch_rms_renorm(const uint16_t *y, int T, int H, float eps, uint16_t *x,
                             hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (H / 8 > 256 * RENORM_CHUNKS) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rms_renorm_kernel, dim3((unsigned)T), dim3(256), 0, st, y, H, eps, x);
    return hipGetLastError();
}

}  // namespace moe
