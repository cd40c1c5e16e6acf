// The no-activation-quantisation control on the expert-grouped path: the
// routed experts multiply bf16 x (gate/up) and bf16 h (down) by the decoded
// e4m3 weights, with the weights' 128x128 block scales and no activation
// scale. The pages quantise both activations (PR #939 "drama3: Fish Audio
// Drama 3 text to speech on one CUDA GPU", "What it adds": dynamic 1x128 FP8
// activation groups; PR #925 commit summary of the SwiGLU launch: routed rows
// written as FP8); this variant is the fidelity control that isolates what
// that quantisation costs, as a switch on the same layer.
//
// Every e4m3 value is exact in bf16, so a K block's partial is a sum of
// exact bf16 products: four chained 16x16x32 bf16 MFMAs from zero (fp32),
// then scale x partial added into the fp32 accumulator in block order. h is
// handed to the down product rounded to bf16 (the oracle keeps it in fp32;
// that rounding is inside the layer's output tolerance). Not tuned: one K
// block of loads in flight.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int NQ_GR = GROUP_ROWS;  // 64 rows per tile, as the FP8 kernels
constexpr int NQ_PAD = 16;         // LDS row padding (bytes)

__device__ __forceinline__ v8bf nq_as_v8bf(uint4 v) { return __builtin_bit_cast(v8bf, v); }

// One K block (128 columns) of a weight row for lane (l16, kq): the codes of
// columns 32i + 8kq .. +8 for i = 0..3, as bf16 B operands.
__device__ __forceinline__ void nq_load_w(const uint8_t *row, int kb, int kq, uint2 (&c)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        c[i] = *reinterpret_cast<const uint2 *>(row + kb * GROUP + 32 * i + 8 * kq);
}

// grid.x = max_tiles * (I / 128): tile (expert, sorted rows r0.., nr) x
// column block nb; wave w owns columns nb*128 + 32w .. +32 of gate and up.
// Writes hb (bf16 h, sorted order).
__global__ __launch_bounds__(256) void grouped_gateup_noq_kernel(GroupedArgs a) {
    __shared__ __align__(16) uint8_t As[NQ_GR][GROUP * 2 + NQ_PAD];
    __shared__ int toks[NQ_GR];
    const int nbs = a.I / GROUP;
    const int tile = blockIdx.x / nbs, nb = blockIdx.x % nbs;
    if (tile >= *a.n_tiles) return;
    const int e = a.tiles[4 * tile], r0 = a.tiles[4 * tile + 1], nr = a.tiles[4 * tile + 2];
    const int H = a.H, I = a.I, KB = H / GROUP;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, kq = lane >> 4;
    if (tid < NQ_GR) toks[tid] = tid < nr ? a.perm[r0 + tid] / a.K : -1;
    __syncthreads();
    // staging: thread -> (row, 64-byte slice) of the tile's bf16 x rows
    const int arow = tid >> 2, acol = (tid & 3) * 64;
    const int atok = toks[arow];
    const uint8_t *aptr =
        reinterpret_cast<const uint8_t *>(a.x + (int64_t)(atok >= 0 ? atok : 0) * H) + acol;
    const uint8_t *wg[2], *wu[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int n = nb * GROUP + 32 * wave + 16 * ct + l16;
        wg[ct] = a.w_gate + ((int64_t)e * I + n) * H;
        wu[ct] = a.w_up + ((int64_t)e * I + n) * H;
    }
    const float *sgr = a.s_gate + ((int64_t)e * nbs + nb) * KB;
    const float *sur = a.s_up + ((int64_t)e * nbs + nb) * KB;
    const int nrt = (nr + 15) / 16;
    v4f accg[4][2], accu[4][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) accg[rt][ct] = accu[rt][ct] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < KB; ++kb) {
        uint4 xa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) xa[i] = ld16(aptr + kb * GROUP * 2 + 16 * i);
        uint2 cg[2][4], cu[2][4];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            nq_load_w(wg[ct], kb, kq, cg[ct]);
            nq_load_w(wu[ct], kb, kq, cu[ct]);
        }
        __syncthreads();  // the previous block's reads of As are done
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4 *>(&As[arow][acol + 16 * i]) = xa[i];
        __syncthreads();
        const float sgk = sgr[kb], suk = sur[kb];
        v8bf bg[2][4], bu[2][4];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bg[ct][i] = nq_as_v8bf(e4m3x8_to_bf16(cg[ct][i]));
                bu[ct][i] = nq_as_v8bf(e4m3x8_to_bf16(cu[ct][i]));
            }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            if (rt >= nrt) break;  // uniform
            v8bf af[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = nq_as_v8bf(
                    *reinterpret_cast<const uint4 *>(&As[rt * 16 + l16][64 * i + 16 * kq]));
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                v4f pg = {0.f, 0.f, 0.f, 0.f}, pu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bg[ct][i], pg, 0, 0, 0);
                    pu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bu[ct][i], pu, 0, 0, 0);
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    accg[rt][ct][k] = fmaf(sgk, pg[k], accg[rt][ct][k]);
                    accu[rt][ct][k] = fmaf(suk, pu[k], accu[rt][ct][k]);
                }
            }
        }
    }
    // element k of lane (l16, kq) in row tile rt: row rt*16 + 4kq + k, column l16
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int row = rt * 16 + 4 * kq + k;
            if (row >= nr) continue;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const float h = silu(accg[rt][ct][k]) * accu[rt][ct][k];
                a.hb[(int64_t)(r0 + row) * I + nb * GROUP + 32 * wave + 16 * ct + l16] =
                    (uint16_t)f32_to_bf16(h);
            }
        }
}

// grid.x = max_tiles * (H / 128): tile x output block mb; wave w owns
// outputs mb*128 + 32w .. +32. Writes e_j (bf16) to the pair's stage row.
__global__ __launch_bounds__(256) void grouped_down_noq_kernel(GroupedArgs a) {
    __shared__ __align__(16) uint8_t As[NQ_GR][GROUP * 2 + NQ_PAD];
    __shared__ int pairs[NQ_GR];
    const int mbs = a.H / GROUP;
    const int tile = blockIdx.x / mbs, mb = blockIdx.x % mbs;
    if (tile >= *a.n_tiles) return;
    const int e = a.tiles[4 * tile], r0 = a.tiles[4 * tile + 1], nr = a.tiles[4 * tile + 2];
    const int H = a.H, I = a.I, KB = I / GROUP;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, kq = lane >> 4;
    if (tid < NQ_GR) pairs[tid] = tid < nr ? a.perm[r0 + tid] : -1;
    const int arow = tid >> 2, acol = (tid & 3) * 64;
    // rows past the tile read the tile's first row; their results are dropped
    const uint8_t *aptr =
        reinterpret_cast<const uint8_t *>(a.hb + (int64_t)(r0 + (arow < nr ? arow : 0)) * I) +
        acol;
    const uint8_t *wd[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int m = mb * GROUP + 32 * wave + 16 * ct + l16;
        wd[ct] = a.w_down + ((int64_t)e * H + m) * I;
    }
    const float *sdr = a.s_down + ((int64_t)e * mbs + mb) * KB;
    const int nrt = (nr + 15) / 16;
    v4f acc[4][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < KB; ++kb) {
        uint4 ha[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ha[i] = ld16(aptr + kb * GROUP * 2 + 16 * i);
        uint2 cd[2][4];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) nq_load_w(wd[ct], kb, kq, cd[ct]);
        __syncthreads();  // pairs ready; the previous block's reads of As are done
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4 *>(&As[arow][acol + 16 * i]) = ha[i];
        __syncthreads();
        const float sdk = sdr[kb];
        v8bf bd[2][4];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) bd[ct][i] = nq_as_v8bf(e4m3x8_to_bf16(cd[ct][i]));
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            if (rt >= nrt) break;  // uniform
            v8bf af[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = nq_as_v8bf(
                    *reinterpret_cast<const uint4 *>(&As[rt * 16 + l16][64 * i + 16 * kq]));
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                v4f p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bd[ct][i], p, 0, 0, 0);
#pragma unroll
                for (int k = 0; k < 4; ++k) acc[rt][ct][k] = fmaf(sdk, p[k], acc[rt][ct][k]);
            }
        }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int row = rt * 16 + 4 * kq + k;
            if (row >= nr) continue;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
                a.stage[(int64_t)pairs[row] * H + mb * GROUP + 32 * wave + 16 * ct + l16] =
                    (uint16_t)f32_to_bf16(acc[rt][ct][k]);
        }
}

hipError_t launch_grouped_noq(const GroupedArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(grouped_gateup_noq_kernel, dim3((unsigned)(a.max_tiles * (a.I / GROUP))),
                       dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(grouped_down_noq_kernel, dim3((unsigned)(a.max_tiles * (a.H / GROUP))),
                       dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace moe
