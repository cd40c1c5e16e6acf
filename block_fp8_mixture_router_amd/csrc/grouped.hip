// Expert-grouped path for prompt chunks: rows sorted by expert, block-FP8
// GEMMs on gfx950 FP8 matrix cores, bf16 shared expert on bf16 matrix cores,
// and a combine that reads every slot's output with 16-byte loads.
//
// The pages run the FP8 experts "on FP8 rows with per-row scales", write the
// SwiGLU's routed rows as FP8 and the shared rows as bf16, and combine with
// 8 contiguous outputs per thread from 16-byte loads in a fixed order
// (PR #939 "drama3: Fish Audio Drama 3 text to speech on one CUDA GPU",
// "What it adds"; PR #925 "drama: load the checkpoint with direct I/O in file
// order and build the codec on its own thread", commit summaries of the
// SwiGLU launch and of drama_moe_combine).
//
// MI355X design:
//  - v_mfma_scale_f32_16x16x128_f8f6f4 consumes K = 128 per instruction,
//    exactly one 128x128 weight block and one activation group, so each MFMA
//    starts from zero and the lane folds (activation scale x weight scale) into
//    its fp32 accumulator: the block scaling costs four FMAs per MFMA.
//  - A work tile is up to 64 sorted (row, slot) pairs of one expert times 128
//    output columns; activations are staged through LDS (shared by the four
//    waves), weights stream straight from HBM into registers (each weight
//    byte is used by one wave only) through a ring several K steps deep.
//  - The gate/up epilogue applies SwiGLU and re-quantises each pair's 128
//    columns (one group) to e4m3 before anything leaves the CU.
//  - No floating-point atomics anywhere: every sum has a fixed order, so
//    results are bitwise deterministic.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int GR = GROUP_ROWS;   // 64 rows per tile
constexpr int APAD = 16;         // LDS row padding (bytes) against bank conflicts

// Runs step(kb, slot, refill) for kb = 0 .. KB - 1 over a ring of PD slots.
// The main loop refills every slot it consumes, so each of its iterations
// issues the same loads and the compiler's wait counts stay exact (a load
// issued on one path only makes it wait for every load in flight at the
// loop head); the last PD steps, peeled, issue none. `refill` is a
// compile-time constant. KB is a positive multiple of PD.
template <int PD, typename F>
__device__ __forceinline__ void ring_loop(int KB, F &step) {
    int kb0 = 0;
    for (; kb0 + PD < KB; kb0 += PD)
#pragma unroll
        for (int d = 0; d < PD; ++d) step(kb0 + d, d, std::true_type{});
#pragma unroll
    for (int d = 0; d < PD; ++d) step(kb0 + d, d, std::false_type{});
}

int grouped_max_tiles(int T, int K, int E) {
    const int64_t P = (int64_t)T * K;
    const int64_t used = P < E ? P : E;
    return (int)((P + GR - 1) / GR + used + 1);
}

// ------------------------------------------------------------- group sort
// One workgroup of SORT_THREADS. Stable counting sort of the T*K (row, slot)
// pairs by expert: wave w owns a contiguous segment of pairs; pass A counts
// per (wave, expert); pass B walks the segment in order, 64 pairs at a time,
// and ranks equal experts within the step with ballots over the key bits.
// Both passes load SORT_BATCH steps of ids at once, so a segment costs one
// memory round trip per batch rather than one per step.
constexpr int SORT_THREADS = 1024;
constexpr int SORT_WAVES = SORT_THREADS / 64;
constexpr int SORT_BATCH = 8;
constexpr int SORT_E = 1024;                       // experts supported
constexpr int SORT_EPT = SORT_E / SORT_THREADS;    // experts per thread in the scan

__global__ __launch_bounds__(SORT_THREADS) void group_sort_kernel(GroupedArgs a) {
    __shared__ int wbase[SORT_WAVES][SORT_E];
    __shared__ int offs[SORT_E];
    __shared__ int scan_c[SORT_THREADS];
    __shared__ int scan_t[SORT_THREADS];
    const int P = a.T * a.K, E = a.E;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int i = tid; i < SORT_WAVES * SORT_E; i += SORT_THREADS) (&wbase[0][0])[i] = 0;
    __syncthreads();
    const int seg = (P + SORT_WAVES - 1) / SORT_WAVES;
    const int p_begin = wave * seg;
    const int p_end = min(P, p_begin + seg);
    for (int p0 = p_begin; p0 < p_end; p0 += 64 * SORT_BATCH) {
        int ev[SORT_BATCH];
#pragma unroll
        for (int u = 0; u < SORT_BATCH; ++u) {
            const int p = p0 + 64 * u + lane;
            ev[u] = p < p_end ? a.ids[p] : -1;
        }
#pragma unroll
        for (int u = 0; u < SORT_BATCH; ++u)
            if (ev[u] >= 0) atomicAdd(&wbase[wave][ev[u]], 1);
    }
    __syncthreads();
    // experts [SORT_EPT * tid, +SORT_EPT): per-wave bases, totals and tiles
    int tot[SORT_EPT], nt[SORT_EPT], csum = 0, tsum = 0;
#pragma unroll
    for (int k = 0; k < SORT_EPT; ++k) {
        const int e = SORT_EPT * tid + k;
        int total = 0;
        if (e < E)
            for (int w = 0; w < SORT_WAVES; ++w) {
                const int c = wbase[w][e];
                wbase[w][e] = total;
                total += c;
            }
        tot[k] = total;
        nt[k] = (total + GR - 1) / GR;
        csum += total;
        tsum += nt[k];
    }
    scan_c[tid] = csum;
    scan_t[tid] = tsum;
    __syncthreads();
    // inclusive Hillis-Steele scans over the threads
    for (int o = 1; o < SORT_THREADS; o <<= 1) {
        const int c = tid >= o ? scan_c[tid - o] : 0;
        const int t = tid >= o ? scan_t[tid - o] : 0;
        __syncthreads();
        scan_c[tid] += c;
        scan_t[tid] += t;
        __syncthreads();
    }
    int off = scan_c[tid] - csum, tb = scan_t[tid] - tsum;
#pragma unroll
    for (int k = 0; k < SORT_EPT; ++k) {
        const int e = SORT_EPT * tid + k;
        if (e < E) {
            offs[e] = off;
            a.offsets[e] = off;
            for (int i = 0; i < nt[k]; ++i) {
                int32_t *tl = a.tiles + 4 * (tb + i);
                tl[0] = e;
                tl[1] = off + i * GR;
                tl[2] = min(GR, tot[k] - i * GR);
                tl[3] = 0;
            }
            if (e == E - 1) {
                a.offsets[E] = off + tot[k];
                *a.n_tiles = tb + nt[k];
            }
        }
        off += tot[k];
        tb += nt[k];
    }
    __syncthreads();
    int kbits = 0;
    while ((1 << kbits) < E) ++kbits;
    for (int pb = p_begin; pb < p_end; pb += 64 * SORT_BATCH) {
        int ev[SORT_BATCH];
#pragma unroll
        for (int u = 0; u < SORT_BATCH; ++u) {
            const int p = pb + 64 * u + lane;
            ev[u] = p < p_end ? a.ids[p] : 0;
        }
#pragma unroll
        for (int u = 0; u < SORT_BATCH; ++u) {
            const int p = pb + 64 * u + lane;
            const bool valid = p < p_end;
            const int e = ev[u];
            uint64_t mask = __ballot(valid);
            for (int b = 0; b < kbits; ++b) {
                const bool bit = (e >> b) & 1;
                const uint64_t bal = __ballot(valid && bit);
                mask &= bit ? bal : ~bal;
            }
            const uint64_t below = lane ? (mask & ((1ull << lane) - 1ull)) : 0ull;
            const int rank = __popcll(below);
            const int n = __popcll(mask);
            int base = 0;
            if (valid) base = wbase[wave][e];
            if (valid) a.perm[offs[e] + base + rank] = p;
            if (valid && rank == 0) wbase[wave][e] = base + n;
        }
    }
}

// Counting sort for up to SORT_CAP pairs in one pass over the ids. A pair's
// rank within its expert comes from an LDS atomic add on that expert's
// counter, so the order of equal experts is not fixed. Nothing computed
// depends on it: a pair's row of the gate/up and down products, and the
// requantisation of its h, use that pair's row alone, and the combine reads
// the slots in slot order. (The ballot ranks of group_sort_kernel cost about
// 100 vector instructions per 64 pairs; for 8192 pairs on one CU that was
// 11 us of issue time.) Same kind of output (offsets, perm, tiles) as
// group_sort_kernel.
constexpr int SORT_CAP = 16384;
constexpr int SORT_STEPS = SORT_CAP / SORT_THREADS;  // pairs per thread
static_assert(SORT_E == SORT_THREADS, "one expert counter per thread");

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    return v;
}

__global__ __launch_bounds__(SORT_THREADS) void group_sort_small_kernel(GroupedArgs a) {
    __shared__ int cnt[SORT_E];   // pairs per expert
    __shared__ int offs[SORT_E];  // first sorted position of each expert
    __shared__ int wtot_c[SORT_WAVES], wtot_t[SORT_WAVES];
    const int P = a.T * a.K, E = a.E;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // pair p = tid + SORT_THREADS * u: each load step is one coalesced row
    int ev[SORT_STEPS];
#pragma unroll
    for (int u = 0; u < SORT_STEPS; ++u) {
        const int p = tid + SORT_THREADS * u;
        ev[u] = p < P ? a.ids[p] : -1;
    }
    cnt[tid] = 0;
    __syncthreads();
    int rk[SORT_STEPS];
#pragma unroll
    for (int u = 0; u < SORT_STEPS; ++u) rk[u] = ev[u] >= 0 ? atomicAdd(&cnt[ev[u]], 1) : 0;
    __syncthreads();
    // thread e: expert e's total and tiles; exclusive scans over experts
    const int e = tid;
    const int total = e < E ? cnt[e] : 0;
    const int nt = (total + GR - 1) / GR;
    const int ic = wave_incl_scan(total, lane), it = wave_incl_scan(nt, lane);
    if (lane == 63) {
        wtot_c[wave] = ic;
        wtot_t[wave] = it;
    }
    __syncthreads();
    int bc = 0, bt = 0;
    for (int w = 0; w < wave; ++w) {
        bc += wtot_c[w];
        bt += wtot_t[w];
    }
    const int off = bc + ic - total, tb = bt + it - nt;
    if (e < E) {
        offs[e] = off;
        a.offsets[e] = off;
        for (int i = 0; i < nt; ++i) {
            int32_t *tl = a.tiles + 4 * (tb + i);
            tl[0] = e;
            tl[1] = off + i * GR;
            tl[2] = min(GR, total - i * GR);
            tl[3] = 0;
        }
        if (e == E - 1) {
            a.offsets[E] = off + total;
            *a.n_tiles = tb + nt;
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < SORT_STEPS; ++u)
        if (ev[u] >= 0) a.perm[offs[ev[u]] + rk[u]] = tid + SORT_THREADS * u;
}

hipError_t launch_group_sort(const GroupedArgs &a, hipStream_t st) {
    if (a.T * a.K <= SORT_CAP)
        hipLaunchKernelGGL(group_sort_small_kernel, dim3(1), dim3(SORT_THREADS), 0, st, a);
    else
        hipLaunchKernelGGL(group_sort_kernel, dim3(1), dim3(SORT_THREADS), 0, st, a);
    return hipGetLastError();
}

// The block-FP8 shared expert as one expert holding every row: pair list
// perm[r] = r (read with K = 1, so row r and stage row r) and 64-row tiles.
__global__ __launch_bounds__(256) void shared_tiles_kernel(int T, int32_t *__restrict__ perm,
                                                           int32_t *__restrict__ tiles,
                                                           int32_t *__restrict__ n_tiles) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < T) {
        perm[i] = i;
        if (i % GR == 0) {
            int32_t *tl = tiles + 4 * (i / GR);
            tl[0] = 0;
            tl[1] = i;
            tl[2] = min(GR, T - i);
            tl[3] = 0;
        }
    }
    if (i == 0) *n_tiles = (T + GR - 1) / GR;
}

hipError_t launch_shared_tiles(int T, int32_t *perm, int32_t *tiles, int32_t *n_tiles,
                               hipStream_t st) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(shared_tiles_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, st,
                       T, perm, tiles, n_tiles);
    return hipGetLastError();
}

// ----------------------------------------------------------- gate / up
// grid.x = max_tiles * (I / 128). Wave w owns output columns
// [nb*128 + 32w, +32): two 16-column MFMA tiles for gate and two for up.
// Weights stream through a register ring PD K-steps deep (HBM latency needs
// about 100 KiB in flight per CU); activations for each K-step go through a
// double-buffered LDS tile, so each step needs a single barrier.

// PD = K steps of loads in flight; the host picks PD dividing H / 128.
template <int PD>
__device__ void grouped_gateup_block(const GroupedArgs &a, int blk) {
    __shared__ __align__(16) uint8_t As[2][GR][GROUP + APAD];
    __shared__ float sxs[GR][64];
    __shared__ int toks[GR];
    __shared__ float amax_part[4][GR];
    const int nbs = a.I / GROUP;
    const int tile = blk / nbs, nb = blk % nbs;
    if (tile >= *a.n_tiles) return;
    const int e = a.tiles[4 * tile], r0 = a.tiles[4 * tile + 1], nr = a.tiles[4 * tile + 2];
    const int H = a.H, I = a.I, KB = H / GROUP;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, kq = lane >> 4;
    if (tid < GR) toks[tid] = tid < nr ? a.perm[r0 + tid] / a.K : -1;
    __syncthreads();
    for (int idx = tid; idx < GR * KB; idx += 256) {
        const int row = idx / KB, b = idx % KB;
        const int t = toks[row];
        sxs[row][b] = t >= 0 ? a.sx[(int64_t)t * KB + b] : 0.0f;
    }
    // activation staging: thread -> (row, 32-byte slice)
    const int arow = tid >> 2, acol = (tid & 3) * 32;
    const int atok = toks[arow];
    const uint8_t *aptr = a.qx + (int64_t)(atok >= 0 ? atok : 0) * H + acol;
    // weights: lane (l16, kq) -> column n, bytes [32kq, 32kq + 32) of each K block
    const uint8_t *wgp[2], *wup[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int n = nb * GROUP + 32 * wave + 16 * ct + l16;
        wgp[ct] = a.w_gate + ((int64_t)e * I + n) * H + 32 * kq;
        wup[ct] = a.w_up + ((int64_t)e * I + n) * H + 32 * kq;
    }
    const float *sgr = a.s_gate + ((int64_t)e * nbs + nb) * KB;
    const float *sur = a.s_up + ((int64_t)e * nbs + nb) * KB;
    const int nrt = (nr + 15) / 16;

    v4f accg[4][2], accu[4][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) accg[rt][ct] = accu[rt][ct] = (v4f){0.f, 0.f, 0.f, 0.f};

    uint4 bg[PD][2][2], bu[PD][2][2], av[PD][2];
    // Every load is unconditional and each K step of the main loop issues the
    // same loads (those of step kb + PD), so the compiler's wait counts stay
    // exact across the loop; rows past the tile read a valid row whose
    // results are never stored. The last PD steps issue no loads.
    auto load_a = [&](int kb, uint4 (&dst)[2]) {
        dst[0] = ld16(aptr + kb * GROUP);
        dst[1] = ld16(aptr + kb * GROUP + 16);
    };
    auto load_b = [&](int kb, uint4 (&g)[2][2], uint4 (&u)[2][2]) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            g[ct][0] = ld16(wgp[ct] + kb * GROUP);
            g[ct][1] = ld16(wgp[ct] + kb * GROUP + 16);
            u[ct][0] = ld16(wup[ct] + kb * GROUP);
            u[ct][1] = ld16(wup[ct] + kb * GROUP + 16);
        }
    };
#pragma unroll
    for (int d = 0; d < PD; ++d) {
        load_a(d, av[d]);
        load_b(d, bg[d], bu[d]);
    }
    __syncthreads();  // toks / sxs ready

    // one K step from ring slot d; with `more` it refills the slot with
    // step kb + PD
    auto step = [&](int kb, int d, auto more) {
        uint8_t(*Ab)[GROUP + APAD] = As[kb & 1];
        *reinterpret_cast<uint4 *>(&Ab[arow][acol]) = av[d][0];
        *reinterpret_cast<uint4 *>(&Ab[arow][acol + 16]) = av[d][1];
        if constexpr (decltype(more)::value) load_a(kb + PD, av[d]);
        __syncthreads();
        const float sgk = sgr[kb], suk = sur[kb];
        v8i cg[2], cu[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            cg[ct] = as_v8i(bg[d][ct][0], bg[d][ct][1]);
            cu[ct] = as_v8i(bu[d][ct][0], bu[d][ct][1]);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            if (rt < nrt) {
                const uint8_t *ar = &Ab[rt * 16 + l16][32 * kq];
                const v8i af = as_v8i(*reinterpret_cast<const uint4 *>(ar),
                                      *reinterpret_cast<const uint4 *>(ar + 16));
                float sxr[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) sxr[i] = sxs[rt * 16 + 4 * kq + i][kb];
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const v4f pg = mfma_fp8_k128(af, cg[ct]);
                    const v4f pu = mfma_fp8_k128(af, cu[ct]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        accg[rt][ct][i] = fmaf(sxr[i] * sgk, pg[i], accg[rt][ct][i]);
                        accu[rt][ct][i] = fmaf(sxr[i] * suk, pu[i], accu[rt][ct][i]);
                    }
                }
            }
        }
        if constexpr (decltype(more)::value) load_b(kb + PD, bg[d], bu[d]);
    };
    ring_loop<PD>(KB, step);

    // epilogue: h = silu(g) * u, per-row amax over the 128 columns, e4m3
    float hv[4][2][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        float m4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                hv[rt][ct][i] = silu(accg[rt][ct][i]) * accu[rt][ct][i];
                m4[i] = fmaxf(m4[i], fabsf(hv[rt][ct][i]));
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float m = group16_max(m4[i]);
            if (l16 == 0) amax_part[wave][rt * 16 + 4 * kq + i] = m;
        }
    }
    __syncthreads();
    uint8_t(*Cs)[GROUP + APAD] = As[0];  // reuse the staging buffer for codes
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = rt * 16 + 4 * kq + i;
            const float am = fmaxf(fmaxf(amax_part[0][row], amax_part[1][row]),
                                   fmaxf(amax_part[2][row], amax_part[3][row]));
            const float sc = group_scale(am);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const uint32_t code = e4m3x4(hv[rt][ct][i] / sc, 0.f, 0.f, 0.f) & 0xFFu;
                Cs[row][32 * wave + 16 * ct + l16] = (uint8_t)code;
            }
            if (wave == 0 && l16 == 0 && row < nr)
                a.sh[(int64_t)(r0 + row) * nbs + nb] = sc;
        }
    __syncthreads();
    for (int idx = tid; idx < GR * 8; idx += 256) {
        const int row = idx >> 3, c = idx & 7;
        if (row < nr)
            st16(a.qh + (int64_t)(r0 + row) * I + nb * GROUP + c * 16,
                 *reinterpret_cast<const uint4 *>(&Cs[row][c * 16]));
    }
}


// ----------------------------------------------------------------- down
// grid.x = max_tiles * (H / 128). Outputs e_j in bf16, written to the
// (row, slot) pair's own row of the stage buffer. Up to four K steps
// (the whole K = I = 512 extent) are kept in flight.

struct DownSmem {
    uint8_t As[2][GR][GROUP + APAD];
    float shs[GR][32];
    int pairs[GR];
    uint16_t Ys[GR][GROUP + 8];
};

template <int PD>
__device__ void grouped_down_block(const GroupedArgs &a, int blk, DownSmem &sm) {
    auto &As = sm.As;
    auto &shs = sm.shs;
    auto &pairs = sm.pairs;
    auto &Ys = sm.Ys;
    const int mbs = a.H / GROUP;
    const int tile = blk / mbs, mb = blk % mbs;
    if (tile >= *a.n_tiles) return;
    const int e = a.tiles[4 * tile], r0 = a.tiles[4 * tile + 1], nr = a.tiles[4 * tile + 2];
    const int H = a.H, I = a.I, KB = I / GROUP;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, kq = lane >> 4;
    if (tid < GR) pairs[tid] = tid < nr ? a.perm[r0 + tid] : -1;
    for (int idx = tid; idx < GR * KB; idx += 256) {
        const int row = idx / KB, b = idx % KB;
        shs[row][b] = row < nr ? a.sh[(int64_t)(r0 + row) * KB + b] : 0.0f;
    }
    const int arow = tid >> 2, acol = (tid & 3) * 32;
    const bool arv = arow < nr;
    const uint8_t *aptr = a.qh + (int64_t)(r0 + (arv ? arow : 0)) * I + acol;
    const uint8_t *wdp[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int m = mb * GROUP + 32 * wave + 16 * ct + l16;
        wdp[ct] = a.w_down + ((int64_t)e * H + m) * I + 32 * kq;
    }
    const float *sdr = a.s_down + ((int64_t)e * mbs + mb) * KB;
    const int nrt = (nr + 15) / 16;

    v4f acc[4][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = (v4f){0.f, 0.f, 0.f, 0.f};
    uint4 bd[PD][2][2], av[PD][2];
    // unconditional loads (see the gate/up kernel)
    auto load_a = [&](int kb, uint4 (&dst)[2]) {
        dst[0] = ld16(aptr + kb * GROUP);
        dst[1] = ld16(aptr + kb * GROUP + 16);
    };
    auto load_b = [&](int kb, uint4 (&b)[2][2]) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            b[ct][0] = ld16(wdp[ct] + kb * GROUP);
            b[ct][1] = ld16(wdp[ct] + kb * GROUP + 16);
        }
    };
#pragma unroll
    for (int d = 0; d < PD; ++d) {
        load_a(d, av[d]);
        load_b(d, bd[d]);
    }
    __syncthreads();  // shs and pairs ready

    // one K step from ring slot d; with `more` it refills the slot with
    // step kb + PD
    auto step = [&](int kb, int d, auto more) {
        uint8_t(*Ab)[GROUP + APAD] = As[kb & 1];
        *reinterpret_cast<uint4 *>(&Ab[arow][acol]) = av[d][0];
        *reinterpret_cast<uint4 *>(&Ab[arow][acol + 16]) = av[d][1];
        if constexpr (decltype(more)::value) load_a(kb + PD, av[d]);
        __syncthreads();
        const float sdk = sdr[kb];
        v8i cd[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) cd[ct] = as_v8i(bd[d][ct][0], bd[d][ct][1]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            if (rt < nrt) {
                const uint8_t *ar = &Ab[rt * 16 + l16][32 * kq];
                const v8i af = as_v8i(*reinterpret_cast<const uint4 *>(ar),
                                      *reinterpret_cast<const uint4 *>(ar + 16));
                float shr[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) shr[i] = shs[rt * 16 + 4 * kq + i][kb];
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const v4f p = mfma_fp8_k128(af, cd[ct]);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[rt][ct][i] = fmaf(shr[i] * sdk, p[i], acc[rt][ct][i]);
                }
            }
        }
        if constexpr (decltype(more)::value) load_b(kb + PD, bd[d]);
    };
    ring_loop<PD>(KB, step);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                Ys[rt * 16 + 4 * kq + i][32 * wave + 16 * ct + l16] =
                    (uint16_t)f32_to_bf16(acc[rt][ct][i]);
    __syncthreads();
    for (int idx = tid; idx < GR * 16; idx += 256) {
        const int row = idx >> 4, c = idx & 15;
        if (row < nr)
            st16(a.stage + (int64_t)pairs[row] * H + mb * GROUP + c * 8,
                 *reinterpret_cast<const uint4 *>(&Ys[row][c * 8]));
    }
}

// ------------------------------------------------------ shared down
// Tile: SDR = 64 rows x 128 columns mb of H; wave w owns columns
// mb*128 + 32w .. +32 (two 16-column MFMA tiles) for all rows. Per
// 128-element step of Is, each lane reads 64 contiguous bytes of its weight
// row and splits them over four bf16 MFMAs (MFMA i takes elements
// [32 kq + 8 i, +8) of lane (l16, kq)); the hs rows go through a
// double-buffered LDS tile with the same split. The MFMAs of a tile form
// one chain over Is in ascending order (the one-row kernel runs the same
// chain), and s leaves in fp32 for the combine.
constexpr int SDR = 64;

struct SharedDownSmem {
    uint8_t As[2][SDR][GROUP * 2 + APAD];
};

template <int PD>
__device__ void shared_down_block(const GroupedArgs &a, int blk, SharedDownSmem &sm) {
    constexpr int NRT = SDR / 16, ARR = SDR / 32;
    auto &As = sm.As;
    const int mbs = a.H / GROUP;
    const int t0 = (blk / mbs) * SDR, mb = blk % mbs;
    const int H = a.H, Is = a.Is, KB = Is / GROUP;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, kq = lane >> 4;
    const int arow = tid >> 3, acol = (tid & 7) * 32;  // bytes
    const uint8_t *aptr[ARR];
#pragma unroll
    for (int r = 0; r < ARR; ++r) {
        const int at = min(t0 + arow + 32 * r, a.T - 1);  // rows past T read a valid row
        aptr[r] = reinterpret_cast<const uint8_t *>(a.hs + (int64_t)at * Is) + acol;
    }
    const uint8_t *wp[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int m = mb * GROUP + 32 * wave + 16 * ct + l16;
        wp[ct] = reinterpret_cast<const uint8_t *>(a.sh_down + (int64_t)m * Is) + 64 * kq;
    }
    v4f acc[NRT][2];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = (v4f){0.f, 0.f, 0.f, 0.f};
    uint4 b[PD][2][4], av[PD][ARR][2];
    auto load = [&](int kb, uint4 (&bb)[2][4], uint4 (&x)[ARR][2]) {
        const int off = kb * GROUP * 2;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) bb[ct][i] = ld16(wp[ct] + off + 16 * i);
#pragma unroll
        for (int r = 0; r < ARR; ++r) {
            x[r][0] = ld16(aptr[r] + off);
            x[r][1] = ld16(aptr[r] + off + 16);
        }
    };
#pragma unroll
    for (int d = 0; d < PD; ++d) load(d, b[d], av[d]);
    // one K step from ring slot d; with `more` it refills the slot with
    // step kb + PD
    auto step = [&](int kb, int d, auto more) {
        uint8_t(*Ab)[GROUP * 2 + APAD] = As[kb & 1];
#pragma unroll
        for (int r = 0; r < ARR; ++r) {
            *reinterpret_cast<uint4 *>(&Ab[arow + 32 * r][acol]) = av[d][r][0];
            *reinterpret_cast<uint4 *>(&Ab[arow + 32 * r][acol + 16]) = av[d][r][1];
        }
        __syncthreads();
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const uint8_t *ar = &Ab[rt * 16 + l16][64 * kq];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const v8bf af = as_v8bf(*reinterpret_cast<const uint4 *>(ar + 16 * i));
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
                    acc[rt][ct] = mfma_bf16_k32(af, as_v8bf(b[d][ct][i]), acc[rt][ct]);
            }
        }
        if constexpr (decltype(more)::value) load(kb + PD, b[d], av[d]);
    };
    ring_loop<PD>(KB, step);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + rt * 16 + 4 * kq + i;
            if (t < a.T)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
                    a.ss[(int64_t)t * H + mb * GROUP + 32 * wave + 16 * ct + l16] = acc[rt][ct][i];
        }
}

// One launch for both down products: the bf16 shared expert's tiles first
// (they need only hs and the shared weights), then the routed tiles. The
// two kinds of tile share one LDS buffer.
template <int PD, int SPD>
__global__ __launch_bounds__(256, 2) void expert_down_kernel(GroupedArgs a, int n_shared) {
    __shared__ __align__(16) uint8_t smem[sizeof(DownSmem) > sizeof(SharedDownSmem)
                                             ? sizeof(DownSmem)
                                             : sizeof(SharedDownSmem)];
    if ((int)blockIdx.x < n_shared) {
        shared_down_block<SPD>(a, blockIdx.x, *reinterpret_cast<SharedDownSmem *>(smem));
        return;
    }
    grouped_down_block<PD>(a, blockIdx.x - n_shared, *reinterpret_cast<DownSmem *>(smem));
}

hipError_t launch_grouped_down(const GroupedArgs &a, hipStream_t st) {
    const int n_shared = a.Is > 0 ? ((a.T + SDR - 1) / SDR) * (a.H / GROUP) : 0;
    const dim3 grid((unsigned)(n_shared + a.max_tiles * (a.H / GROUP)));
    if (grid.x == 0) return hipSuccess;
    const int kb = a.I / GROUP, skb = a.Is / GROUP;
    // a ring two blocks deep keeps three workgroups per CU (four deep, two);
    // Is = 0 (no shared tiles) counts as even
    if (kb % 2 == 0 && skb % 2 == 0)
        hipLaunchKernelGGL((expert_down_kernel<2, 2>), grid, dim3(256), 0, st, a, n_shared);
    else if (kb % 2 == 0)
        hipLaunchKernelGGL((expert_down_kernel<2, 1>), grid, dim3(256), 0, st, a, n_shared);
    else if (skb % 2 == 0)
        hipLaunchKernelGGL((expert_down_kernel<1, 2>), grid, dim3(256), 0, st, a, n_shared);
    else
        hipLaunchKernelGGL((expert_down_kernel<1, 1>), grid, dim3(256), 0, st, a, n_shared);
    return hipGetLastError();
}

// ---------------------------------------------------- shared gate / up
// Tile: 64 rows x 64 columns of Is. Wave w owns 16 columns of gate and up.
// Per 128-column K step, four chained bf16 MFMAs from zero give the step's
// partial product Q (an MFMA output element depends only on its own row of
// A and column of B), and the partials are added in fp64 in ascending K
// order, d = ((0 + Q_0) + Q_1) + ...: every row's gs and us are the same
// bits whatever tile it sits in and however many rows come with it, and the
// one-row kernel repeats this sequence exactly. Each lane reads 64
// contiguous bytes of its weight row per 128 columns of H and splits them
// over four MFMAs (MFMA i takes elements [32 kq + 8 i, +8) of lane
// (l16, kq)); the LDS activation fragments follow the same split. Loads run
// two K steps ahead, unconditionally (see the routed kernels).

constexpr int SR = 32;  // rows per combine tile

constexpr int SRG = 64;  // rows per shared gate/up tile (32: +6 us on the skewed chunk, +11 us
                         // on the concentrated one, -1.5 us on the uniform one; 128: +60 us)
template <int PD>
__device__ void shared_gateup_block(const GroupedArgs &a, int blk) {
    constexpr int NRT = SRG / 16, ARR = SRG / 32;
    __shared__ __align__(16) uint8_t Ash[2][SRG][GROUP * 2 + APAD];
    const int H = a.H, Is = a.Is, KB = H / GROUP;
    const int snb = Is / 64;
    const int t0 = (blk / snb) * SRG, nb = blk % snb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, kq = lane >> 4;
    const int arow = tid >> 3, acol = (tid & 7) * 32;  // bytes
    const uint8_t *aptr[ARR];
    for (int r = 0; r < ARR; ++r) {
        const int at = min(t0 + arow + 32 * r, a.T - 1);  // rows past T read a valid row
        aptr[r] = reinterpret_cast<const uint8_t *>(a.x + (int64_t)at * H) + acol;
    }
    const int n = nb * 64 + 16 * wave + l16;
    const uint8_t *gp = reinterpret_cast<const uint8_t *>(a.sh_gate + (int64_t)n * H) + 64 * kq;
    const uint8_t *up = reinterpret_cast<const uint8_t *>(a.sh_up + (int64_t)n * H) + 64 * kq;
    double dg[NRT][4] = {}, du[NRT][4] = {};
    uint4 bg[PD][4], bu[PD][4], av[PD][ARR][2];
    auto load = [&](int kb, uint4 (&g)[4], uint4 (&u)[4], uint4 (&x)[ARR][2]) {
        const int off = kb * GROUP * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            g[i] = ld16(gp + off + 16 * i);
            u[i] = ld16(up + off + 16 * i);
        }
#pragma unroll
        for (int r = 0; r < ARR; ++r) {
            x[r][0] = ld16(aptr[r] + off);
            x[r][1] = ld16(aptr[r] + off + 16);
        }
    };
#pragma unroll
    for (int d = 0; d < PD; ++d) load(d, bg[d], bu[d], av[d]);
    // one K step from ring slot d; with `more` it refills the slot with
    // step kb + PD
    auto step = [&](int kb, int d, auto more) {
        {
            uint8_t(*Ab)[GROUP * 2 + APAD] = Ash[kb & 1];
#pragma unroll
            for (int r = 0; r < ARR; ++r) {
                *reinterpret_cast<uint4 *>(&Ab[arow + 32 * r][acol]) = av[d][r][0];
                *reinterpret_cast<uint4 *>(&Ab[arow + 32 * r][acol + 16]) = av[d][r][1];
            }
            __syncthreads();
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                const uint8_t *ar = &Ab[rt * 16 + l16][64 * kq];
                v4f pg = {0.f, 0.f, 0.f, 0.f}, pu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const v8bf af = as_v8bf(*reinterpret_cast<const uint4 *>(ar + 16 * i));
                    pg = mfma_bf16_k32(af, as_v8bf(bg[d][i]), pg);
                    pu = mfma_bf16_k32(af, as_v8bf(bu[d][i]), pu);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dg[rt][i] += (double)pg[i];
                    du[rt][i] += (double)pu[i];
                }
            }
            if constexpr (decltype(more)::value) load(kb + PD, bg[d], bu[d], av[d]);
        }
    };
    ring_loop<PD>(KB, step);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + rt * 16 + 4 * kq + i;
            if (t < a.T)
                a.hs[(int64_t)t * Is + n] =
                    (uint16_t)f32_to_bf16(silu((float)dg[rt][i]) * (float)du[rt][i]);
        }
}

// One launch for both gate/up products: the shared expert's tiles come
// first (they need only x and start at once; bound by L2), then the routed
// experts' tiles (bound by HBM), so the two overlap. OCC workgroups per CU:
// a launch with fewer workgroups than CUs (a few rows) runs one per CU with
// a ring twice as deep; the arithmetic, K steps in order, is the same.
template <int PD, int OCC>
__global__ __launch_bounds__(256, OCC) void expert_gateup_kernel(GroupedArgs a, int n_shared) {
    if ((int)blockIdx.x < n_shared) {
        shared_gateup_block<PD>(a, blockIdx.x);
        return;
    }
    grouped_gateup_block<PD>(a, blockIdx.x - n_shared);
}

hipError_t launch_expert_gateup(const GroupedArgs &a, hipStream_t st) {
    const int n_shared = a.Is > 0 ? ((a.T + SRG - 1) / SRG) * (a.Is / 64) : 0;
    const dim3 grid((unsigned)(n_shared + a.max_tiles * (a.I / GROUP)));
    if (grid.x == 0) return hipSuccess;
    const int kb = a.H / GROUP;
    if (grid.x <= 256 && kb % 4 == 0)
        hipLaunchKernelGGL((expert_gateup_kernel<4, 1>), grid, dim3(256), 0, st, a, n_shared);
    else if (kb % 2 == 0)
        hipLaunchKernelGGL((expert_gateup_kernel<2, 2>), grid, dim3(256), 0, st, a, n_shared);
    else
        hipLaunchKernelGGL((expert_gateup_kernel<1, 2>), grid, dim3(256), 0, st, a, n_shared);
    return hipGetLastError();
}

// ---------------------------------------------------------- combine
// Tile: 32 rows x 128 columns of H; grid (ceil(T/32), H/128). Each thread
// owns two items (row, 8 contiguous columns): it issues the 16-byte loads
// of the item's staged e_j (K slots) and shared output s (fp32 from the
// bf16 shared expert, bf16 from the block-FP8 one), then produces
// y = bf16(sum_j w_j e_j + gamma s), slots in order.

template <int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(GroupedArgs a) {
    const int H = a.H, K = a.K;
    const int t0 = blockIdx.x * SR, mb = blockIdx.y;
    const int tid = threadIdx.x;
    // every load first (rows past T read row T - 1, slots past K slot K - 1;
    // neither is used), then the arithmetic
    uint4 ev[2][KMAX], sv[2][2];
    float wv[2][KMAX], gv[2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int idx = tid + 256 * it;
        const int t = min(t0 + (idx >> 4), a.T - 1), c = idx & 15;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const int jj = j < K ? j : K - 1;
            ev[it][j] = ld16(a.stage + ((int64_t)t * K + jj) * H + mb * GROUP + c * 8);
            wv[it][j] = a.wts[(int64_t)t * K + jj];
        }
        const float *sp = a.ss ? a.ss + (int64_t)t * H + mb * GROUP + c * 8 : nullptr;
        const uint16_t *ep = a.es ? a.es + (int64_t)t * H + mb * GROUP + c * 8 : nullptr;
        sv[it][0] = sp ? ld16(sp) : ep ? ld16(ep) : make_uint4(0, 0, 0, 0);
        sv[it][1] = sp ? ld16(sp + 4) : make_uint4(0, 0, 0, 0);
        gv[it] = a.gamma[t];
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int idx = tid + 256 * it;
        const int row = idx >> 4, c = idx & 15;
        const int t = t0 + row;
        if (t >= a.T) continue;
        float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (j < K) {
                const float w = wv[it][j];
                const uint32_t vs[4] = {ev[it][j].x, ev[it][j].y, ev[it][j].z, ev[it][j].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc8[2 * i] = fmaf(w, bf16_lo(vs[i]), acc8[2 * i]);
                    acc8[2 * i + 1] = fmaf(w, bf16_hi(vs[i]), acc8[2 * i + 1]);
                }
            }
        if (a.ss) {  // the bf16 shared expert's fp32 output
            const float g = gv[it];
            const uint32_t u[8] = {sv[it][0].x, sv[it][0].y, sv[it][0].z, sv[it][0].w,
                                   sv[it][1].x, sv[it][1].y, sv[it][1].z, sv[it][1].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) acc8[i] = fmaf(g, __uint_as_float(u[i]), acc8[i]);
        } else if (a.es) {  // the block-FP8 shared expert's staged output
            const float g = gv[it];
            const uint4 v = sv[it][0];
            const uint32_t vs[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc8[2 * i] = fmaf(g, bf16_lo(vs[i]), acc8[2 * i]);
                acc8[2 * i + 1] = fmaf(g, bf16_hi(vs[i]), acc8[2 * i + 1]);
            }
        }
        uint4 out;
        out.x = f32_to_bf16(acc8[0]) | (f32_to_bf16(acc8[1]) << 16);
        out.y = f32_to_bf16(acc8[2]) | (f32_to_bf16(acc8[3]) << 16);
        out.z = f32_to_bf16(acc8[4]) | (f32_to_bf16(acc8[5]) << 16);
        out.w = f32_to_bf16(acc8[6]) | (f32_to_bf16(acc8[7]) << 16);
        st16(a.y + (int64_t)t * H + mb * GROUP + c * 8, out);
    }
}

hipError_t launch_combine(const GroupedArgs &a, hipStream_t st) {
    const dim3 grid((a.T + SR - 1) / SR, a.H / GROUP);
    if (a.K <= 4)
        hipLaunchKernelGGL(combine_kernel<4>, grid, dim3(256), 0, st, a);
    else if (a.K <= 8)
        hipLaunchKernelGGL(combine_kernel<8>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(combine_kernel<16>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace moe
