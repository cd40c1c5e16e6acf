// RMS renormalisation of rows between the layers of a decode stack. The
// backbone normalises every row before its MoE layer (PR #925 "drama: load
// the checkpoint with direct I/O in file order and build the codec on its own
// thread", backbone commit summaries: residual add and RMSnorm ahead of the
// FP8 quantisation); a chain of independent synthetic layers keeps only the
// normalisation, with no learned gain:
//   ms = fp32(sum of exact squares, in fp64, / H); r = 1 / sqrt(ms + eps);
//   x  = bf16(y * r).
// One workgroup per row, with the arithmetic of renorm_row_scale and
// renorm_chunk (common.h), which the one-row layer kernel's renormalising
// prologue also uses. Reads and writes 2H bytes per row.
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
    // the barrier inside also orders every load of this row before any
    // store (x may alias y)
    const float r = renorm_row_scale(v, H, eps, part);
    uint16_t *xr = x + row * H;
#pragma unroll
    for (int i = 0; i < RENORM_CHUNKS; ++i) {
        const int c = threadIdx.x + 256 * i;
        if (c < nc) st16(xr + c * 8, renorm_chunk(v[i], r));
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
