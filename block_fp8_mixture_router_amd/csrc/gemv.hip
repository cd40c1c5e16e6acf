// One-row bf16 projection, the backbone's other bf16 projections streamed
// the way the layer's decode path streams its experts (PR #925 "drama: load
// the checkpoint with direct I/O in file order and build the codec on its
// own thread", commit summaries: the backbone's bf16 GEMMs and the
// single-row projection that streams its weights ahead of use):
//   y[t, n] = bf16(fp32(sum_k x[t, k] W[n, k])),   t < T <= 4,
// the sum of exact bf16 products accumulated in fp64 and rounded once to
// fp32, as the router logits are.
//
// Bound by HBM: W is read once, 2 bytes per multiply-add. Each wave owns
// GV_ROWS rows of W; lane l reads the 16-byte chunks c = l + 64i of each
// row, so every load instruction reads 1 KiB of one row contiguously, and
// all of a wave's chunks (GV_ROWS rows x NC chunks) are issued before the
// first is used. x sits in LDS (T x K bf16, loaded once per workgroup).
// Each lane accumulates its chunks' exact products in fp64; a DPP wave sum
// gives the row's total.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int GV_ROWS = 2;   // rows of W per wave
constexpr int GV_WAVES = 4;  // waves per workgroup
constexpr int GV_MAXK = 8192;

template <int NC>
__global__ __launch_bounds__(GV_WAVES * 64) void bf16_gemv_kernel(
    const uint16_t *__restrict__ W, int N, int K, const uint16_t *__restrict__ x, int T,
    uint16_t *__restrict__ y) {
    extern __shared__ __align__(16) uint16_t xs[];  // T x K, sized at launch
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nc8 = K / 8;  // 16-byte chunks per row
    const int n0 = (blockIdx.x * GV_WAVES + wave) * GV_ROWS;
    // this wave's weight chunks first (rows past N read row N - 1, unused)
    uint4 wv[GV_ROWS][NC];
#pragma unroll
    for (int r = 0; r < GV_ROWS; ++r) {
        const uint16_t *wr = W + (int64_t)min(n0 + r, N - 1) * K;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = lane + 64 * i;
            wv[r][i] = c < nc8 ? ld16(wr + c * 8) : make_uint4(0, 0, 0, 0);
        }
    }
    for (int c = tid; c < T * nc8; c += GV_WAVES * 64)
        *reinterpret_cast<uint4 *>(&xs[c * 8]) = ld16(x + (int64_t)c * 8);
    __syncthreads();
    if (n0 >= N) return;  // whole waves; no barrier follows
    double acc[GV_ROWS][4];
#pragma unroll
    for (int r = 0; r < GV_ROWS; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[r][t] = 0.0;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + 64 * i;
        if (c >= nc8) continue;  // past the row (its weights were zeroed; x there is not)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t >= T) break;  // uniform
            const uint4 xv = *reinterpret_cast<const uint4 *>(&xs[t * K + c * 8]);
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
            double xd[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                xd[2 * k] = (double)bf16_lo(xw[k]);
                xd[2 * k + 1] = (double)bf16_hi(xw[k]);
            }
#pragma unroll
            for (int r = 0; r < GV_ROWS; ++r) {
                const uint32_t ww[4] = {wv[r][i].x, wv[r][i].y, wv[r][i].z, wv[r][i].w};
                double a = acc[r][t];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    a = fma(xd[2 * k], (double)bf16_lo(ww[k]), a);
                    a = fma(xd[2 * k + 1], (double)bf16_hi(ww[k]), a);
                }
                acc[r][t] = a;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < GV_ROWS; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t >= T) break;  // uniform
            const double s = wave_allsum_d(acc[r][t]);
            if (lane == 0 && n0 + r < N)
                y[(int64_t)t * N + n0 + r] = (uint16_t)f32_to_bf16((float)s);
        }
}

hipError_t launch_bf16_gemv(const uint16_t *W, int N, int K, const uint16_t *x, int T,
                            uint16_t *y, hipStream_t st) {
    if (N <= 0 || T <= 0) return hipSuccess;
    if (T > 4 || K > GV_MAXK || K % 8) return hipErrorInvalidValue;
    const int rows_per_wg = GV_WAVES * GV_ROWS;
    const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg)), block(GV_WAVES * 64);
    const int nc = (K / 8 + 63) / 64;
    const size_t lds = (size_t)T * K * sizeof(uint16_t);  // x only: many workgroups per CU
#define MOE_GEMV(NCV) \
    hipLaunchKernelGGL(bf16_gemv_kernel<NCV>, grid, block, lds, st, W, N, K, x, T, y)
    if (nc <= 1) MOE_GEMV(1);
    else if (nc <= 2) MOE_GEMV(2);
    else if (nc <= 4) MOE_GEMV(4);
    else if (nc <= 8) MOE_GEMV(8);
    else MOE_GEMV(16);
#undef MOE_GEMV
    return hipGetLastError();
}

}  // namespace moe
