// Residual add, RMS norm and 1x128 e4m3 quantisation of the normed rows: the
// step in front of the layer. The pages' add-norm before the MoE also writes
// the normed rows' FP8 groups, with the order and rounding of the separate
// quantisation launch it replaces (PR #925 "drama: load the checkpoint with
// direct I/O in file order and build the codec on its own thread", commit
// summaries of the Drama 3 backbone). Per row:
//   r  = bf16(fp32(hidden) + fp32(residual))          (the new residual stream)
//   ms = fp32(sum of exact squares of r, in fp64, / H); rs = 1 / sqrt(ms + eps)
//   x  = bf16(fp32(fp32(r * rs) * norm_w))
//   (q, s) = the 1x128 quantisation of x, as moe_quant_act.
// One workgroup per row, each thread owning up to four 16-byte chunks of 8
// values (chunk c = tid + 256 i), so the 16 lanes of a 128-column group sit
// in one DPP row and the group's amax is a 16-lane reduction. HBM-bound:
// reads 4H + (2H for the gain, shared by the rows) bytes per row and writes
// 4H + H + H/32.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void add_rmsnorm_quant_kernel(
    const uint16_t *__restrict__ hidden, const uint16_t *res_in, const uint16_t *__restrict__ norm_w,
    int H, float eps, uint16_t *res_out, uint16_t *__restrict__ x, uint8_t *__restrict__ q,
    float *__restrict__ s) {
    __shared__ double part[4];
    const int64_t row = blockIdx.x;
    const int nc = H / 8;
    const uint16_t *hr = hidden + row * H, *rr = res_in + row * H;
    uint4 hv[RENORM_CHUNKS], rv[RENORM_CHUNKS], wv[RENORM_CHUNKS];
#pragma unroll
    for (int i = 0; i < RENORM_CHUNKS; ++i) {
        const int c = threadIdx.x + 256 * i;
        const bool ok = c < nc;
        hv[i] = ok ? ld16(hr + c * 8) : make_uint4(0, 0, 0, 0);
        rv[i] = ok ? ld16(rr + c * 8) : make_uint4(0, 0, 0, 0);
        wv[i] = ok ? ld16(norm_w + c * 8) : make_uint4(0, 0, 0, 0);
    }
    // the new residual stream (bf16), and the fp64 sum of its exact squares
    float r[RENORM_CHUNKS][8];
    uint4 ro[RENORM_CHUNKS];
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < RENORM_CHUNKS; ++i) {
        const uint32_t a[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
        const uint32_t b[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t lo = f32_to_bf16(bf16_lo(a[k]) + bf16_lo(b[k]));
            const uint32_t hi = f32_to_bf16(bf16_hi(a[k]) + bf16_hi(b[k]));
            o[k] = lo | (hi << 16);
            r[i][2 * k] = bf16_to_f32((uint16_t)lo);
            r[i][2 * k + 1] = bf16_to_f32((uint16_t)hi);
        }
        ro[i] = make_uint4(o[0], o[1], o[2], o[3]);
        acc = sumsq8(r[i], acc);  // chunks past H are zero and add nothing
    }
    acc = wave_allsum_d(acc);
    if ((threadIdx.x & (WAVE - 1)) == 0) part[threadIdx.x / WAVE] = acc;
    __syncthreads();  // every load of this row is done before any store (res_out may alias res_in)
    const double sum = ((part[0] + part[1]) + part[2]) + part[3];
    const float rs = rms_scale(sum, H, eps);
    uint16_t *ror = res_out + row * H, *xr = x + row * H;
    uint8_t *qr = q + row * H;
    float *sr = s + row * (H / GROUP);
#pragma unroll
    for (int i = 0; i < RENORM_CHUNKS; ++i) {
        const int c = threadIdx.x + 256 * i;
        if (c >= nc) continue;  // whole 16-lane groups (H / 8 is a multiple of 16)
        st16(ror + c * 8, ro[i]);
        const uint32_t w[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
        float f[8];
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t lo = f32_to_bf16((r[i][2 * k] * rs) * bf16_lo(w[k]));
            const uint32_t hi = f32_to_bf16((r[i][2 * k + 1] * rs) * bf16_hi(w[k]));
            o[k] = lo | (hi << 16);
            f[2 * k] = bf16_to_f32((uint16_t)lo);
            f[2 * k + 1] = bf16_to_f32((uint16_t)hi);
        }
        st16(xr + c * 8, make_uint4(o[0], o[1], o[2], o[3]));
        // the group of chunk c is c / 16; its 16 chunks are 16 adjacent lanes
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(f[k]));
        amax = group16_max(amax);
        const float sc = group_scale(amax);
        uint2 out;
        out.x = e4m3x4(f[0] / sc, f[1] / sc, f[2] / sc, f[3] / sc);
        out.y = e4m3x4(f[4] / sc, f[5] / sc, f[6] / sc, f[7] / sc);
        *reinterpret_cast<uint2 *>(qr + c * 8) = out;
        if ((c & 15) == 0) sr[c >> 4] = sc;
    }
}

hipError_t launch_add_rmsnorm_quant(const uint16_t *hidden, const uint16_t *res_in,
                                    const uint16_t *norm_w, int T, int H, float eps,
                                    uint16_t *res_out, uint16_t *x, uint8_t *q, float *s,
                                    hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (H % GROUP || H / 8 > 256 * RENORM_CHUNKS) return hipErrorInvalidValue;
    hipLaunchKernelGGL(add_rmsnorm_quant_kernel, dim3((unsigned)T), dim3(256), 0, st, hidden,
                       res_in, norm_w, H, eps, res_out, x, q, s);
    return hipGetLastError();
}

}  // namespace moe
