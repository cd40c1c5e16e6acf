// Row-at-a-time path (decode): the whole layer for up to four rows in one
// persistent kernel, computing every value with the arithmetic of the
// expert-grouped kernels, so that a row's output bytes are the ones it gets
// inside any chunk.
//
// The pages' one-row projection issues the same matrix instructions on the
// same fragments in the same K order as the row tiling it replaces, so its
// results are the same bits, and their backbone outputs are hash-identical
// at every chunk size (PR #925 "drama: load the checkpoint with direct I/O in
// file order and build the codec on its own thread", commit summaries of the
// single-row projection; PR #920 "drama: Drama 3 (fishaudio/drama-3)
// text-to-speech on CUDA", Receipt). Their frame step also lets a kernel
// stream immutable weights before waiting on its predecessor (PR #927,
// "What this changes"). On gfx950 the layer for one row is bound by HBM
// (1.5 FLOP per weight byte) and by the latency of its three dependent
// steps, so it runs as ONE launch of one workgroup per compute unit, with no
// grid-wide barrier:
//
//  A. router logits (exact fp64 sums), one per workgroup at a time, and x
//     into LDS (bf16 and its 1x128 e4m3 groups); on waves 1-3 the shared
//     expert's gate/up columns and the shared gate, which need x alone;
//  B. every workgroup waits for the logits of its rows, selects the top-K
//     itself, streams its share of the routed gate/up rows, h = silu(g) * u,
//     and issues the loads of its phase-C down rows, which arrive during the
//     h handoff;
//  C. every workgroup waits for h, hs and gamma, re-quantises h (1x128) into
//     LDS and owns blocks of 8 output rows m: every slot's down rows, the
//     shared down rows and the combine y = bf16(sum_j w_j e_j + gamma s).
//
// The block products are the grouped kernels' MFMA instructions on the same
// operand bytes: an MFMA output element depends only on its own row of A and
// column of B, so a row alone can sit in any row of a tile and the tiles can
// pair blocks along the diagonal (two K halves, four K steps, two slots) to
// use the matrix cores' spare rows, with the same bits.
//
// Cross-workgroup values carry their call's epoch. Every value one workgroup
// hands to others (a logit, an hs or h element, gamma) is one 64-bit word:
// the value's 32 bits and the epoch of the call that wrote it, stored and
// loaded with device-coherent accesses. A consumer polls the words
// themselves until all carry the current epoch, so there is no flag, no
// fence and no barrier: each workgroup moves on as soon as its own inputs
// exist. Each word is stored in DECODE_REPLICAS copies and workgroup b reads
// copy b % DECODE_REPLICAS, so no line is polled by more than 1/8 of the
// workgroups.
//
// Epochs: every workgroup keeps its own call counter in the workspace, reads
// it at the start and writes the next value at the end; all counters advance
// together, so all workgroups of a call agree on its epoch as long as the
// workspace started out filled with one repeated byte. Epochs are odd, below
// 2^30 and differ from the counter they come from, so neither such a fill nor
// words left by an earlier call can satisfy a wait. Waits are bounded: after
// SPIN_LIMIT = 2^17 unsuccessful poll rounds the spin-out word is set and the
// kernel still finishes. A round of a wait on other workgroups is one
// device-coherent load round trip, so such a wait gives up after about
// 0.1-0.3 s (workgroups not all resident); a wave's wait for a top-K slot of
// its own workgroup polls LDS and gives up after about 10 ms.
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

constexpr int REPL = DECODE_REPLICAS;   // copies of every cross-workgroup value
constexpr uint32_t SPIN_LIMIT = 1u << 17;  // poll rounds before a wait gives up
constexpr int ERR_WORD = SYNC_ERR_WORD;
constexpr int MB = 8;  // output rows per phase-C unit

// ------------------------------------------------------ tagged handoffs

template <typename T>
__device__ __forceinline__ T ld_dev(const T *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Handoff words live in the workspace (global memory). Loading them through
// a global-address-space pointer keeps them global loads in functions the
// compiler does not inline: a flat load is also counted as an LDS access,
// and every wait on it becomes a wait for all outstanding memory operations.
typedef __attribute__((address_space(1))) const uint64_t gword;
__device__ __forceinline__ uint64_t ld_word(const uint64_t *p) {
    return __hip_atomic_load((gword *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_dev(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// a value handed to other workgroups: its 32 bits and the call's epoch
__device__ __forceinline__ uint64_t tagged(uint32_t bits, uint32_t epoch) {
    return ((uint64_t)epoch << 32) | bits;
}
__device__ __forceinline__ bool has_epoch(uint64_t w, uint32_t epoch) {
    return (uint32_t)(w >> 32) == epoch;
}

// this call's epoch from a workgroup's call counter c: odd, below 2^30 and
// never equal to c itself, so a workspace filled with one repeated byte
// (zeros included) holds no word tagged with it
__device__ __forceinline__ uint32_t call_epoch(uint32_t c) { return (c & 0x3FFFFFFEu) + 3u; }

// First loads of the tagged words p[idx[i]], i < n (valid entries form a
// prefix; the others read as already carrying `epoch`). Nothing waits for
// them here, so several sets can be in flight before the first is checked.
template <int N>
__device__ __forceinline__ void poll_issue(const uint64_t *p, const int (&idx)[N], int n,
                                           uint32_t epoch, uint64_t (&w)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        // branch-free: entries past n load word 0 and are then marked done
        const uint64_t x = ld_word(p + (i < n ? idx[i] : 0));
        w[i] = i < n ? x : tagged(0u, epoch);
    }
}

template <int N>
__device__ __forceinline__ bool all_have_epoch(const uint64_t (&w)[N], uint32_t epoch) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok &= has_epoch(w[i], epoch);
    return ok;
}

// Polls the words of an earlier poll_issue that do not yet carry `epoch`
// until all do (bounded: past SPIN_LIMIT rounds the error word is set and
// the stale values are returned). The words' value halves go to v.
template <int N>
__device__ __forceinline__ void poll_finish(uint32_t *err, const uint64_t *p,
                                            const int (&idx)[N], int n, uint32_t epoch,
                                            uint64_t (&w)[N], uint32_t (&v)[N]) {
    // the first check stands outside the loop, so the wait for these words
    // does not also wait for loads issued after them
    if (!all_have_epoch<N>(w, epoch)) for (uint32_t spin = 0;; ++spin) {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < N; ++i) ok &= has_epoch(w[i], epoch);
        if (ok) break;
        if (spin >= SPIN_LIMIT) {
            st_dev(err, 1u);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n && !has_epoch(w[i], epoch)) w[i] = ld_word(p + idx[i]);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = (uint32_t)w[i];
}

// Two first loads of the words, a short sleep apart: when the first comes
// back a little too early, the second (already on its way) usually has them,
// instead of a new round trip.
template <int N>
__device__ __forceinline__ void poll_words_staggered(uint32_t *err, const uint64_t *p,
                                                     const int (&idx)[N], int n, uint32_t epoch,
                                                     uint32_t (&v)[N]) {
    uint64_t w0[N], w1[N];
    poll_issue<N>(p, idx, n, epoch, w0);
    __builtin_amdgcn_s_sleep(6);
    poll_issue<N>(p, idx, n, epoch, w1);
    if (all_have_epoch<N>(w0, epoch)) {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = (uint32_t)w0[i];
        return;
    }
#pragma unroll
    for (int i = 0; i < N; ++i)
        if (!has_epoch(w0[i], epoch)) w0[i] = w1[i];
    poll_finish<N>(err, p, idx, n, epoch, w0, v);
}

template <int N>
__device__ __forceinline__ void poll_words(uint32_t *err, const uint64_t *p,
                                           const int (&idx)[N], int n, uint32_t epoch,
                                           uint32_t (&v)[N]) {
    uint64_t w[N];
    poll_issue<N>(p, idx, n, epoch, w);
    poll_finish<N>(err, p, idx, n, epoch, w, v);
}

// Pipelined re-polls. A handoff region as a raw buffer: a load at an offset
// past its end returns zero and touches no memory, so a lane can take part
// in a load instruction without requesting its word. Loads are
// device-coherent (sc1), as the tagged stores are.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr int POLL_OOB = 0x7FFFFFF0;  // past every handoff region

__device__ __forceinline__ __amdgpu_buffer_rsrc_t handoff_region(const uint64_t *base, int words) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint64_t *>(base), 0, words * 8,
                                             0x00020000);
}
__device__ __forceinline__ uint64_t region_word(__amdgpu_buffer_rsrc_t r, int byte_off) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 16 /* sc1 */);
    return ((uint64_t)v.y << 32) | v.x;
}

// Completes a first round w of loads of words idx[i] (i < n) of region r:
// if any lane of the wave still has a stale word, DEPTH re-poll rounds go
// out a short sleep apart, each asking only for the words still stale;
// then each returning round (oldest first) is merged and sent again for
// what is still missing. The wait after the last word lands is one memory
// latency plus part of a round gap, not a full round trip per retry.
// Bounded: past SPIN_LIMIT passes the error word is set and the stale
// values are returned.
// s_sleep units (64 clocks) between re-poll rounds: the lone layer polls at
// the shorter gap, the renormalising (stacked) layer at the longer one (each
// measured the faster for its kernel)
constexpr int POLL_GAP = 3, POLL_GAP_RN = 6;

template <int N, int DEPTH, int GAP = POLL_GAP>
__device__ __forceinline__ void poll_complete(uint32_t *err, __amdgpu_buffer_rsrc_t r,
                                              const int (&idx)[N], int n, uint32_t epoch,
                                              uint64_t (&w)[N], uint32_t (&v)[N]) {
    // valid entries form a prefix; the others count as done
#pragma unroll
    for (int i = 0; i < N; ++i)
        if (i >= n) w[i] = tagged(0u, epoch);
    if (__builtin_amdgcn_ballot_w64(!all_have_epoch<N>(w, epoch)) != 0) {
        uint64_t q[DEPTH][N];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
#pragma unroll
            for (int i = 0; i < N; ++i)
                q[d][i] = region_word(r, has_epoch(w[i], epoch) ? POLL_OOB : 8 * idx[i]);
            if (d + 1 < DEPTH) __builtin_amdgcn_s_sleep(GAP);
        }
        for (uint32_t spin = 0;; ++spin) {
            bool fin = false;  // wave-uniform
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                if (!fin) {
#pragma unroll
                    for (int i = 0; i < N; ++i)
                        if (!has_epoch(w[i], epoch)) w[i] = q[d][i];
                    fin = __builtin_amdgcn_ballot_w64(!all_have_epoch<N>(w, epoch)) == 0;
                    if (!fin)
#pragma unroll
                        for (int i = 0; i < N; ++i)
                            q[d][i] = region_word(r, has_epoch(w[i], epoch) ? POLL_OOB
                                                                            : 8 * idx[i]);
                }
            }
            if (fin) break;
            if (spin >= SPIN_LIMIT) {
                st_dev(err, 1u);
                break;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = (uint32_t)w[i];
}

// the wave's earlier LDS stores are seen by its later LDS loads in other
// lanes: a wave's LDS operations execute in order, and this keeps the
// compiler from moving memory operations across it (a memory fence here
// would also wait for every global load the wave has in flight)
__device__ __forceinline__ void wave_lds_sync() { __builtin_amdgcn_wave_barrier(); }

__device__ __forceinline__ float dot8_bf16_regs(uint4 a, uint4 b, float acc) {
    const uint32_t as[4] = {a.x, a.y, a.z, a.w}, bs[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        acc = fmaf(bf16_lo(as[k]), bf16_lo(bs[k]), acc);
        acc = fmaf(bf16_hi(as[k]), bf16_hi(bs[k]), acc);
    }
    return acc;
}

// ------------------------------------------------------------- phase A

// Router logits come first and alone: each workgroup's four waves share one
// logit at a time (a quarter of the row each), so the 1 MiB of router rows
// is requested before anything else, arrives in about one memory round trip,
// and the routing decision that everything after it waits for is taken as
// early as possible. NQ = 16-byte chunks of a bf16 H-row per lane per wave
// quarter (H / 2048, rounded up).
template <int NQ>
struct RouterRegs {
    uint4 x[NQ], w[NQ];
};

// chunk c = lane + 64 (wave + 4 i) of row e of the router and of row t of x
// (x from global memory, or from the renormalised rows in LDS when RN)
template <int NQ>
__device__ __forceinline__ void router_load_w(const FusedArgs &a, int r, RouterRegs<NQ> &rr) {
    const int e = r % a.E, nc8 = a.H / 8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint16_t *wr = a.router_w + (int64_t)e * a.H;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int c = lane + WAVE * (wave + 4 * i);
        rr.w[i] = c < nc8 ? ld16(wr + c * 8) : make_uint4(0, 0, 0, 0);
    }
}
template <int NQ, bool RN>
__device__ __forceinline__ void router_load_x(const FusedArgs &a, int r, const uint16_t *xs,
                                              RouterRegs<NQ> &rr) {
    const int t = r / a.E, nc8 = a.H / 8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint16_t *xr = (RN ? xs : a.x) + (int64_t)t * a.H;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int c = lane + WAVE * (wave + 4 * i);
        rr.x[i] = c < nc8 ? ld16(xr + c * 8) : make_uint4(0, 0, 0, 0);
    }
}
template <int NQ, bool RN>
__device__ __forceinline__ void router_load(const FusedArgs &a, int r, const uint16_t *xs,
                                            RouterRegs<NQ> &rr) {
    router_load_w<NQ>(a, r, rr);
    router_load_x<NQ, RN>(a, r, xs, rr);
}

// Logit r = (t, e): exact fp64 sum of bf16 products (each wave's partial in
// two chains and a lane tree, the four partials in wave order), rounded once
// to fp32, then to bf16, then the bias; handed off in every copy. Every
// thread of the workgroup calls this (it has a barrier); red is 4 doubles of
// LDS, not reused by the next call before that call's barrier.
template <int NQ>
__device__ __forceinline__ void router_logit(const FusedArgs &a, int r, const RouterRegs<NQ> &rr,
                                             double *red, uint32_t epoch) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double acc0 = 0.0, acc1 = 0.0;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const uint32_t xs[4] = {rr.x[i].x, rr.x[i].y, rr.x[i].z, rr.x[i].w};
        const uint32_t ws[4] = {rr.w[i].x, rr.w[i].y, rr.w[i].z, rr.w[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc0 = fma((double)bf16_lo(xs[k]), (double)bf16_lo(ws[k]), acc0);
            acc1 = fma((double)bf16_hi(xs[k]), (double)bf16_hi(ws[k]), acc1);
        }
    }
    const double part = wave_allsum_d(acc0 + acc1);
    if (lane == 0) red[wave] = part;
    __syncthreads();
    // the last wave stores: wave 0 runs the first top-K, and a store still
    // in flight would hold back the results of its polls (the wave's memory
    // operations complete in order)
    if (wave == 3 && lane < REPL) {
        const int t = r / a.E, e = r % a.E;
        const double acc = ((red[0] + red[1]) + red[2]) + red[3];
        float l = (float)acc;
        if (!(a.flags & K_LOGITS_FP32)) l = bf16_round(l);
        if (a.bias) l = l + a.bias[e];
        st_dev(a.logits + (int64_t)(lane * a.T + t) * a.E + e, tagged(__float_as_uint(l), epoch));
    }
}

// x (bf16) and its 1x128 e4m3 groups into LDS, with the arithmetic of the
// quantiser: chunk c of 8 values, 16 lanes per 128-column group
__device__ __forceinline__ void quant_chunk_to_lds(uint4 v, int c, uint8_t *q, float *s) {
    const float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                        bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = group16_max(amax);
    const float sc = group_scale(amax);
    uint2 out;
    out.x = e4m3x4(f[0] / sc, f[1] / sc, f[2] / sc, f[3] / sc);
    out.y = e4m3x4(f[4] / sc, f[5] / sc, f[6] / sc, f[7] / sc);
    *reinterpret_cast<uint2 *>(q + c * 8) = out;
    if ((c & 15) == 0) s[c >> 4] = sc;
}

// one row: the workgroup's router loads hold all of x (lane chunk
// c = lane + 64 (wave + 4 i), whole 16-lane groups)
template <int NQ>
__device__ __forceinline__ void x_stage_router(const RouterRegs<NQ> &rr, int H, uint16_t *xs,
                                               uint8_t *q, float *s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int c = lane + WAVE * (wave + 4 * i);
        if (c < H / 8) {
            st16(xs + c * 8, rr.x[i]);
            quant_chunk_to_lds(rr.x[i], c, q, s);
        }
    }
}

// every row, thread tid owning chunks tid + 256 k (x from global memory, or
// already in LDS when RN)
template <bool RN>
__device__ __forceinline__ void x_stage_rows(const uint16_t *x, int T, int H, uint16_t *xs,
                                             uint8_t *q, float *s) {
    const int n = T * H / 8;
    for (int c = threadIdx.x; c < n; c += blockDim.x) {
        const uint4 v = RN ? ld16(xs + c * 8) : ld16(x + (int64_t)c * 8);
        if (!RN) st16(xs + c * 8, v);
        quant_chunk_to_lds(v, c, q, s);
    }
}

// Shared expert gate/up. One item: columns n0 = 2s and n0 + 1 of the gate
// and up matrices for every row (T <= 4), all of H, by one wave, with the
// grouped kernel's arithmetic: per 128-column K step, four chained bf16
// MFMAs from zero (MFMA i takes elements [32 kq + 8 i, +8) of lane
// (l16, kq)); the steps' partials added in fp64 in ascending order;
// hs = bf16(silu(gs) * us). One chain covers four K steps: B column l16 is
// weight row (l16 & 3) = gate n0, gate n0 + 1, up n0, up n0 + 1 at step
// 4g + (l16 >> 2); A row l16 is x row (l16 & 3) at the same step; the
// diagonal 4x4 blocks (row block = column block) are kept.
constexpr int SH_GROUPS = 4;  // chains (four K steps each) per batch of loads

__device__ __forceinline__ void s_item(const FusedArgs &a, int s, const uint16_t *xs, float *q,
                                       uint32_t epoch) {
    const int lane = threadIdx.x & 63, l16 = lane & 15, kq = lane >> 4;
    const int H = a.H, KB = H / GROUP, T = a.T, Is = a.Is;
    const int n0 = 2 * s, cid = l16 & 3, qb = l16 >> 2;
    const uint16_t *wrow =
        (cid < 2 ? a.sh_gate : a.sh_up) + (int64_t)(n0 + (cid & 1)) * H + 32 * kq;
    const uint16_t *xrow = xs + min(cid, T - 1) * H + 32 * kq;
    const int NG = (KB + 3) / 4;
    for (int g0 = 0; g0 < NG; g0 += SH_GROUPS) {
        uint4 w[SH_GROUPS][4];
#pragma unroll
        for (int gg = 0; gg < SH_GROUPS; ++gg) {
            const int kb = min(4 * (g0 + gg) + qb, KB - 1);  // steps past H reload the last
#pragma unroll
            for (int i = 0; i < 4; ++i) w[gg][i] = ld16(wrow + kb * GROUP + 8 * i);
        }
#pragma unroll
        for (int gg = 0; gg < SH_GROUPS; ++gg) {
            const int g = g0 + gg;
            if (g < NG) {  // wave-uniform
                const int kb = min(4 * g + qb, KB - 1);
                v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc = mfma_bf16_k32(as_v8bf(ld16(xrow + kb * GROUP + 8 * i)),
                                        as_v8bf(w[gg][i]), acc);
                // element r of lane (l16, kq): row 4 kq + r = x row r at step
                // 4g + kq; column l16 = weight row cid at step 4g + qb
                const int kbv = 4 * g + kq;
                if (kq == qb && kbv < KB)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (r < T) q[kbv * 16 + r * 4 + cid] = acc[r];
            }
        }
    }
    wave_lds_sync();
    uint32_t hv = 0;
    if (lane < 2 * T) {
        const int t = lane >> 1, nl = lane & 1;
        double dg = 0.0, du = 0.0;
        for (int kb = 0; kb < KB; ++kb) {
            dg += (double)q[kb * 16 + t * 4 + nl];
            du += (double)q[kb * 16 + t * 4 + 2 + nl];
        }
        hv = f32_to_bf16(silu((float)dg) * (float)du);
    }
    // copy lane / (2T) of value (t, nl) = lane % (2T)
    const int nv = 2 * T;
    const uint32_t v = (uint32_t)__shfl((int)hv, lane % nv);
    if (lane < REPL * nv) {
        const int r = lane / nv, vi = lane % nv, t = vi >> 1, nl = vi & 1;
        st_dev(a.hs + ((int64_t)r * T + t) * Is + n0 + nl, tagged(v, epoch));
    }
    wave_lds_sync();  // q is rewritten by the wave's next item
}

// shared gate of row t: gamma = 1 / (1 + exp(-(x . wg))), the dot product in
// the top-K kernels' order (lane chunks c = lane + 64 i, fp32 fma chains,
// then the wave sum)
__device__ __forceinline__ void g_item(const FusedArgs &a, int t, const uint16_t *xs,
                                       uint32_t epoch) {
    const int lane = threadIdx.x & 63, nc8 = a.H / 8;
    float z = 0.0f;
    for (int c = lane; c < nc8; c += WAVE)
        z = dot8_bf16_regs(ld16(xs + t * a.H + c * 8), ld16(a.sh_gate_w + c * 8), z);
    z = wave_allsum(z);
    if (lane < REPL)
        st_dev(a.gamma + lane * a.T + t, tagged(__float_as_uint(1.0f / (1.0f + expf(-z))), epoch));
}

// ------------------------------------------------------------- phase B

// top-K of row t from this workgroup's copy of the tagged logits; each
// slot's expert is published in LDS (one 64-bit word per slot, see
// publish_slot) as its round ends
template <int NL, int GAP>
__device__ __forceinline__ void topk_tagged_n(const uint64_t *lr, int E, int K, uint32_t epoch,
                                              uint32_t *err, int lane, uint64_t *slots,
                                              float *wts, bool packed) {
    int idx[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) idx[i] = lane + WAVE * i;
    const int n = min(NL, max(0, (E - lane + WAVE - 1) / WAVE));
    uint32_t bits[NL];
    uint64_t w[NL];
    poll_issue<NL>(lr, idx, n, epoch, w);
    poll_complete<NL, (NL <= 4 ? 3 : 1), GAP>(err, handoff_region(lr, E), idx, n, epoch, w,
                                               bits);
    if (packed) {
        uint32_t k[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) k[i] = i < n ? bf16_order_key(__uint_as_float(bits[i]), idx[i]) : 0u;
        topk_select_packed<NL, true>(k, K, lane, nullptr, wts, slots);
    } else {
        float v[NL];
        int ix[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            v[i] = i < n ? __uint_as_float(bits[i]) : -INFINITY;
            ix[i] = i < n ? idx[i] : 0x7FFFFFFF;
        }
        topk_select_n<NL, true>(v, ix, K, lane, nullptr, wts, slots);
    }
}

// more than 256 experts: 16 per lane, in a function of its own
template <int GAP>
__device__ __noinline__ void topk_tagged_wide(const uint64_t *lr, int E, int K, uint32_t epoch,
                                              uint32_t *err, int lane, uint64_t *slots,
                                              float *wts, bool packed) {
    topk_tagged_n<16, GAP>(lr, E, K, epoch, err, lane, slots, wts, packed);
}

// Up to 256 experts (4 per lane) the top-K is inlined into the kernel, not
// called: a call saves a callee-saved register to scratch memory on entry
// and loads it back on return, one more memory round trip (queued behind
// the wave's other memory operations) on the path every later step waits
// for.
template <int GAP>
__device__ __forceinline__ void topk_tagged(const uint64_t *lr, int E, int K, uint32_t epoch,
                                            uint32_t *err, int lane, uint64_t *slots, float *wts,
                                            bool packed) {
    if (E <= 256) topk_tagged_n<4, GAP>(lr, E, K, epoch, err, lane, slots, wts, packed);
    else topk_tagged_wide<GAP>(lr, E, K, epoch, err, lane, slots, wts, packed);
}

// a slot word's expert (the low half)
__device__ __forceinline__ int slot_expert(uint64_t w) { return (int)(uint32_t)w; }
__device__ __forceinline__ uint64_t ld_slot(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// A slot's expert once the wave selecting its row has published it.
// Bounded like the handoff waits, though the publishing wave depends on
// nothing that can stall for good (on giving up: expert 0).
__device__ __forceinline__ int wait_slot(const uint64_t *slot, uint32_t *err) {
    uint32_t spins = 0;
    uint64_t w;
    while (((w = ld_slot(slot)) >> 32) == 0) {
        if (++spins > SPIN_LIMIT) {
            if ((threadIdx.x & 63) == 0) st_dev(err, 1u);
            return 0;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    return slot_expert(w);
}

// Waits until every slot [0, n) of a row is published (lane l < n polls
// slot l; every word is checked, since different words are not ordered).
__device__ __forceinline__ void wait_row(const uint64_t *slots, int n, uint32_t *err) {
    const int lane = threadIdx.x & 63;
    uint32_t spins = 0;
    while (__builtin_amdgcn_ballot_w64(lane < n && (ld_slot(slots + min(lane, n - 1)) >> 32) == 0)) {
        if (++spins > SPIN_LIMIT) {
            if (lane == 0) st_dev(err, 1u);
            return;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// Routed gate/up. One item: columns n0..n0+3 of the gate and up matrices of
// pair p's expert, all of H, by one wave, with the grouped kernel's
// arithmetic: per 128x128 weight block one FP8 MFMA from zero, folded in
// ascending K order as acc = fmaf(sx * s_w, P, acc), then h = silu(g) * u.
// One MFMA covers two K blocks: B column l16 is weight row (l16 & 7) (gate
// n0..n0+3, then up n0..n0+3) at block j (l16 < 8) or KH + j (l16 >= 8), A
// row l16 is the pair's row of qx at the same block, and the two diagonal
// 8x8 blocks are kept. Lanes 0-7 (D row 0) fold the first KH blocks and hand
// their sums to lanes 40-47 (D row 8, columns 8-15), which fold the rest.
constexpr int GU_STEP = 8;  // MFMAs (block pairs) per batch of loads

struct GateUpRegs {
    uint4 w[GU_STEP][2];
    float sw[GU_STEP];  // weight block scale of each lane's column and block
};

// Expert e's gate or up rows and their block scales; with the block-FP8
// shared expert, e = E is that expert (its matrices have the routed ones'
// shape, Is = I).
// Expert indices come from LDS words the top-K publishes; they are clamped
// to the valid range here (a no-op on published words), so no weight address
// can leave the expert arrays whatever such a word holds.
__device__ __forceinline__ int clamp_expert(int e, int hi) { return min(max(e, 0), hi); }

template <int VAR>
__device__ __forceinline__ void expert_gu(const FusedArgs &a, int e, bool up, const uint8_t *&w,
                                          const float *&s) {
    e = clamp_expert(e, VAR == DV_SFP8 ? a.E : a.E - 1);
    if (VAR == DV_SFP8 && e == a.E) {
        w = up ? a.sh8_up : a.sh8_gate;
        s = up ? a.sh_s_up : a.sh_s_gate;
    } else {
        w = (up ? a.w_up : a.w_gate) + (int64_t)e * a.I * a.H;
        s = (up ? a.s_up : a.s_gate) + (int64_t)e * (a.I / GROUP) * (a.H / GROUP);
    }
}

// The lane's bytes of one K block of its weight row: [32 kq, +32) for the
// FP8 MFMA; with DV_NOQ the four bf16 chain steps' [32 i + 8 kq, +8), i < 4,
// in that order.
template <int VAR>
__device__ __forceinline__ void load_block(const uint8_t *row, int kb, uint4 &w0, uint4 &w1) {
    const int kq = (threadIdx.x & 63) >> 4;
    if constexpr (VAR == DV_NOQ) {
        const uint8_t *b = row + kb * GROUP + 8 * kq;
        const uint2 c0 = *reinterpret_cast<const uint2 *>(b);
        const uint2 c1 = *reinterpret_cast<const uint2 *>(b + 32);
        const uint2 c2 = *reinterpret_cast<const uint2 *>(b + 64);
        const uint2 c3 = *reinterpret_cast<const uint2 *>(b + 96);
        w0 = make_uint4(c0.x, c0.y, c1.x, c1.y);
        w1 = make_uint4(c2.x, c2.y, c3.x, c3.y);
    } else {
        const uint8_t *b = row + kb * GROUP + 32 * kq;
        w0 = ld16(b);
        w1 = ld16(b + 16);
    }
}

template <int VAR>
__device__ __forceinline__ void gateup_load(const FusedArgs &a, int e, int n0, int j0,
                                            GateUpRegs &r) {
    const int lane = threadIdx.x & 63, l16 = lane & 15;
    const int H = a.H, KB = H / GROUP, KH = (KB + 1) / 2;
    const int r8 = l16 & 7, hb = l16 >> 3;
    const uint8_t *wb;
    const float *sb;
    expert_gu<VAR>(a, e, r8 >= 4, wb, sb);
    const uint8_t *row = wb + (int64_t)(n0 + (r8 & 3)) * H;
    const float *srow = sb + (int64_t)(n0 / GROUP) * KB;
    // branch-free: blocks past the end reload the last one (dropped later)
#pragma unroll
    for (int u = 0; u < GU_STEP; ++u) {
        const int kb = min(hb * KH + j0 + u, KB - 1);
        load_block<VAR>(row, kb, r.w[u][0], r.w[u][1]);
        r.sw[u] = srow[kb];
    }
}

// One K block kb of row t against the lane's weight row (its bytes w0, w1):
// the block's product (element 0 of the lane's result) and the scale it is
// folded with. FP8: one MFMA on the e4m3 groups of x, scale sx x s_w. DV_NOQ:
// the control's four chained bf16 MFMAs from zero on bf16 x and the decoded
// codes, scale s_w.
template <int VAR>
__device__ __forceinline__ float2 gu_block(int t, int kb, int H, uint4 w0, uint4 w1, float sw,
                                           const uint8_t *qx, const float *sx,
                                           const uint16_t *xs) {
    const int kq = (threadIdx.x & 63) >> 4;
    if constexpr (VAR == DV_NOQ) {
        const uint16_t *xa = xs + t * H + kb * GROUP + 8 * kq;
        const uint2 c[4] = {make_uint2(w0.x, w0.y), make_uint2(w0.z, w0.w),
                            make_uint2(w1.x, w1.y), make_uint2(w1.z, w1.w)};
        v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            d = mfma_bf16_k32(as_v8bf(ld16(xa + 32 * i)), as_v8bf(e4m3x8_to_bf16(c[i])), d);
        return make_float2(sw, d[0]);
    } else {
        const uint8_t *qa = qx + t * H + kb * GROUP + 32 * kq;
        const v4f d = mfma_fp8_k128(as_v8i(ld16(qa), ld16(qa + 16)), as_v8i(w0, w1));
        return make_float2(sx[t * (H / GROUP) + kb] * sw, d[0]);
    }
}

// the MFMAs of one batch: lanes 0-7 fold their first-half blocks into acc,
// lanes 40-47 keep (scale, product) of the second-half blocks in sp[j][c]
template <int VAR>
__device__ __forceinline__ void gateup_mfma(const FusedArgs &a, int t, int j0,
                                            const GateUpRegs &r, const uint8_t *qx,
                                            const float *sx, const uint16_t *xs, float2 *sp,
                                            float &acc) {
    const int lane = threadIdx.x & 63, l16 = lane & 15;
    const int H = a.H, KB = H / GROUP, KH = (KB + 1) / 2, hb = l16 >> 3;
#pragma unroll
    for (int u = 0; u < GU_STEP; ++u) {
        const int j = j0 + u;
        if (j < KH) {  // wave-uniform
            const int kb = min(hb * KH + j, KB - 1);  // A row l16 and B column l16 share it
            const float2 v = gu_block<VAR>(t, kb, H, r.w[u][0], r.w[u][1], r.sw[u], qx, sx, xs);
            if (lane < 8) acc = fmaf(v.x, v.y, acc);
            else if (lane >= 40 && lane < 48 && KH + j < KB) sp[j * 8 + lane - 40] = v;
        }
    }
}

// The rest of the item once its first batch is in. With one batch
// (H <= 2048) every block's (scale, product) stays in registers: lanes 0-7
// fold the first half, lanes 40-47 take over their sums and fold the second
// half, with no LDS and no wait beyond the item's own loads. Larger H takes
// further batches and keeps the second half's pairs in LDS (sp).
template <int VAR>
__device__ __forceinline__ void gateup_finish(const FusedArgs &a, int p, int n0, int e,
                                              const GateUpRegs &r0, const uint8_t *qx,
                                              const float *sx, const uint16_t *xs, float2 *sp,
                                              uint32_t epoch) {
    const int lane = threadIdx.x & 63, l16 = lane & 15;
    const int H = a.H, KB = H / GROUP, KH = (KB + 1) / 2, t = p / a.KS, hb = l16 >> 3;
    const int src = (lane >= 40 && lane < 48) ? lane - 40 : lane;
    float g;
    if (KH <= GU_STEP) {
        float sc[GU_STEP], pv[GU_STEP];
#pragma unroll
        for (int u = 0; u < GU_STEP; ++u) {
            sc[u] = 0.0f;
            pv[u] = 0.0f;
            if (u < KH) {  // wave-uniform
                const int kb = min(hb * KH + u, KB - 1);  // A row l16 and B column l16 share it
                const float2 v =
                    gu_block<VAR>(t, kb, H, r0.w[u][0], r0.w[u][1], r0.sw[u], qx, sx, xs);
                sc[u] = v.x;
                pv[u] = v.y;
            }
        }
        float acc = 0.0f;  // lanes 0-7: blocks 0..KH-1
#pragma unroll
        for (int u = 0; u < GU_STEP; ++u)
            if (u < KH) acc = fmaf(sc[u], pv[u], acc);
        g = __shfl(acc, src);  // lanes 40-47: blocks KH..KB-1
#pragma unroll
        for (int u = 0; u < GU_STEP; ++u)
            if (KH + u < KB) g = fmaf(sc[u], pv[u], g);
    } else {
        float acc = 0.0f;
        gateup_mfma<VAR>(a, t, 0, r0, qx, sx, xs, sp, acc);
        for (int j0 = GU_STEP; j0 < KH; j0 += GU_STEP) {
            GateUpRegs r;
            gateup_load<VAR>(a, e, n0, j0, r);
            gateup_mfma<VAR>(a, t, j0, r, qx, sx, xs, sp, acc);
        }
        g = __shfl(acc, src);
        wave_lds_sync();
        if (lane >= 40 && lane < 48)
            for (int j = 0; j < KB - KH; ++j) {
                const float2 v = sp[j * 8 + lane - 40];
                g = fmaf(v.x, v.y, g);
            }
        wave_lds_sync();  // sp is rewritten by the wave's next item
    }
    const int F = KB > KH ? 40 : 0;  // lanes F..F+3: gate sums, F+4..F+7: up sums
    const float u = __shfl(g, min(lane + 4, 63));
    const float hv = silu(g) * u;
    const float hl = __shfl(hv, F + (lane & 3));
    // the control hands h over rounded to bf16, as its grouped kernel stages it
    const uint32_t hbits = VAR == DV_NOQ ? f32_to_bf16(hl) : __float_as_uint(hl);
    if (lane < 4 * REPL)
        st_dev(a.h + ((int64_t)(lane >> 2) * a.T * a.KS + p) * a.I + n0 + (lane & 3),
               tagged(hbits, epoch));
}

// ------------------------------------------------------------- phase C

// A phase-C unit is a block of MB output rows m0..m0+MB-1 of one row t of x:
// the routed down rows of all K slots, the shared down rows and the combine.
//
// Routed: a 16x16x128 MFMA takes as A the rows (slot j, row m) of two slots,
// 2 x MB = 16 rows of 128 codes of one K block, and as B the same K block of
// h for all 16 slot columns; only the products of slot j's rows with slot
// j's column are kept (an output element depends only on its own A row and B
// column). The lane folds (h scale x weight block scale) into its fp32 sum
// per K block, in ascending order, as the grouped down kernel does; e_j is
// then rounded to bf16, the grouped path's staging precision.
//
// Shared: the grouped combine kernel's chain of bf16 MFMAs over Is (per
// 128-column block, MFMA i takes elements [32 kq + 8 i, +8)), accumulated in
// the MFMA from zero in ascending order; B column l16 is shared down row
// m0 + (l16 & 7), every A row is hs of row t.
constexpr int SDB = 4;  // 128-column blocks of a shared down row loaded ahead (one per wave)

template <int KBR, int TPW>
struct DownRegs {
    uint4 w[TPW][KBR][2];  // A operands: tile, K block, two 16-byte halves
    float sd[TPW][KBR];    // weight block scale of this lane's D rows
    uint4 s[4];            // shared down operands of block `wave`
};

constexpr int CHAIN_WAVE = 3;  // the wave that runs the shared down chain

// Shared down operands of rows m0..m0+MB-1: wave w loads block w (every
// wave the same loads, so no wave's wait counts depend on a branch; blocks
// past Is reload the last one), staged in LDS for the chain wave.
template <int KBR, int TPW>
__device__ __forceinline__ void down_load_shared(const FusedArgs &a, int m0,
                                                 DownRegs<KBR, TPW> &r) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, kq = lane >> 4;
    const int Is = a.Is, SB = Is / GROUP;
    const uint16_t *row = a.sh_down + (int64_t)(m0 + (l16 & 7)) * Is + 32 * kq;
    const int bc = min(wave, SB - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.s[i] = ld16(row + bc * GROUP + 8 * i);
}

// sdo: LDS [SDB][4][64] uint4
template <int KBR, int TPW>
__device__ __forceinline__ void down_stage_shared(const DownRegs<KBR, TPW> &r, uint4 *sdo) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 4; ++i) sdo[(wave * 4 + i) * 64 + lane] = r.s[i];
}

// Expert e's down rows and block scales (e = E: the block-FP8 shared expert)
template <int VAR>
__device__ __forceinline__ void expert_down(const FusedArgs &a, int e, const uint8_t *&w,
                                            const float *&s) {
    e = clamp_expert(e, VAR == DV_SFP8 ? a.E : a.E - 1);
    if (VAR == DV_SFP8 && e == a.E) {
        w = a.sh8_down;
        s = a.sh_s_down;
    } else {
        w = a.w_down + (int64_t)e * a.H * a.I;
        s = a.s_down + (int64_t)e * (a.H / GROUP) * (a.I / GROUP);
    }
}

// Routed A operands and block scales of unit (t, m0) for this wave's tiles,
// K blocks [0, KBR). Branch-free: slots past KS reload slot KS - 1 and K
// blocks past the row reload the last one (the MFMA loop skips both), so the
// loads form one straight run and a later wait on earlier loads does not
// also wait for these.
template <int KBR, int TPW, int VAR>
__device__ __forceinline__ void down_load_routed(const FusedArgs &a, int t, int m0,
                                                 const uint64_t *slots, DownRegs<KBR, TPW> &r) {
    const int I = a.I, KS = a.KS, IB = I / GROUP;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int tau = wave + 4 * u;
        const uint8_t *wb;
        const float *sb, *sbs;
        const uint8_t *dummy;
        expert_down<VAR>(a, slot_expert(slots[t * KS + min(2 * tau + (l16 >> 3), KS - 1)]), wb, sb);
        expert_down<VAR>(a, slot_expert(slots[t * KS + min(2 * tau + (kq >> 1), KS - 1)]), dummy,
                         sbs);
        const uint8_t *row = wb + (int64_t)(m0 + (l16 & 7)) * I;
        const float *sd = sbs + (int64_t)(m0 / GROUP) * IB;
#pragma unroll
        for (int b = 0; b < KBR; ++b) {
            const int bc = min(b, IB - 1);
            load_block<VAR>(row, bc, r.w[u][b][0], r.w[u][b][1]);
            r.sd[u][b] = sd[bc];
        }
    }
}

// shared down of rows m0 + c, c < 8, in lanes c (D row 0, element 0); the
// first SDB blocks' operands from LDS (sdo), later ones from memory
__device__ __forceinline__ float shared_down_chain(const FusedArgs &a, int t, int m0,
                                                   const uint4 *sdo, const uint16_t *hs_l) {
    const int lane = threadIdx.x & 63, l16 = lane & 15, kq = lane >> 4;
    const int Is = a.Is, SB = Is / GROUP;
    const uint16_t *ha = hs_l + t * Is + 32 * kq;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < SDB; ++b)
        if (b < SB)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc = mfma_bf16_k32(as_v8bf(ld16(ha + b * GROUP + 8 * i)),
                                    as_v8bf(sdo[(b * 4 + i) * 64 + lane]), acc);
    const uint16_t *row = a.sh_down + (int64_t)(m0 + (l16 & 7)) * Is + 32 * kq;
    for (int b = SDB; b < SB; ++b)  // blocks past the ones loaded ahead
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = mfma_bf16_k32(as_v8bf(ld16(ha + b * GROUP + 8 * i)),
                                as_v8bf(ld16(row + b * GROUP + 8 * i)), acc);
    return acc[0];
}

// The unit's output: every routed slot's e_j (MFMA), the gated shared row
// and the combine y = bf16(sum_j w_j e_j + gamma s), slots in order. ej and
// ss are LDS scratch ([KS][MB] and [MB] fp32); hs and gamma were staged in
// LDS; with chain false the shared rows' s is already in ss. With the
// block-FP8 shared expert, s is its slot's e (slot K). qh holds h as 1x128
// e4m3 codes with scales shs, or (DV_NOQ) as bf16 values. Every thread of
// the workgroup calls this (it has barriers).
template <int KBR, int TPW, int VAR>
__device__ __forceinline__ void down_unit(const FusedArgs &a, int t, int m0,
                                          const DownRegs<KBR, TPW> &r, const uint8_t *qh,
                                          const float *shs, const uint64_t *slots,
                                          const float *wts, const uint16_t *hs_l,
                                          const float *gam_l, float *ej, float *ss,
                                          uint4 *sdo, bool chain) {
    const int H = a.H, I = a.I, K = a.K, KS = a.KS, IB = I / GROUP, Is = a.Is;
    const int Isb = VAR == DV_SFP8 ? 0 : Is;  // width of the bf16 shared expert
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, kq = lane >> 4;

    // routed slots: tile tau = wave + 4u holds slots 2 tau, 2 tau + 1
    const int ntiles = (KS + 1) / 2;
    const int jb = min(l16, KS - 1);  // this lane's B column: slot l16
    const uint8_t *qb = qh + (int64_t)(t * KS + jb) * I + 32 * kq;
    const uint16_t *hb = reinterpret_cast<const uint16_t *>(qh) + (int64_t)(t * KS + jb) * I + 8 * kq;
    const uint8_t *wrow[TPW];
    float acc[TPW][4] = {};
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int tau = wave + 4 * u;
        const float *sb;
        expert_down<VAR>(a, slot_expert(slots[t * KS + min(2 * tau + (l16 >> 3), KS - 1)]), wrow[u],
                         sb);
        wrow[u] += (int64_t)(m0 + (l16 & 7)) * I;
    }
    const int js_lane = 2 * wave + (kq >> 1);  // slot of this lane's D rows (tile u adds 8u)
    for (int b = 0; b < IB; ++b) {
        v8i bq;
        v8bf bh[4];
        if constexpr (VAR == DV_NOQ) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                bh[i] = as_v8bf(*reinterpret_cast<const uint4 *>(hb + b * GROUP + 32 * i));
        } else {
            bq = as_v8i(*reinterpret_cast<const uint4 *>(qb + b * GROUP),
                        *reinterpret_cast<const uint4 *>(qb + b * GROUP + 16));
        }
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            if (wave + 4 * u >= ntiles) continue;
            const int js = min(js_lane + 8 * u, KS - 1);
            uint4 w0, w1;
            float sdv;
            if (b < KBR) {
                w0 = r.w[u][b][0];
                w1 = r.w[u][b][1];
                sdv = r.sd[u][b];
            } else {  // K blocks past the register copy
                load_block<VAR>(wrow[u], b, w0, w1);
                const uint8_t *dummy;
                const float *sb;
                expert_down<VAR>(a, slot_expert(slots[t * KS + js]), dummy, sb);
                sdv = sb[(int64_t)(m0 / GROUP) * IB + b];
            }
            v4f d;
            float sc;
            if constexpr (VAR == DV_NOQ) {
                // the control: four chained bf16 MFMAs from zero on the
                // decoded codes and bf16 h, folded with the weight scale
                const uint2 c[4] = {make_uint2(w0.x, w0.y), make_uint2(w0.z, w0.w),
                                    make_uint2(w1.x, w1.y), make_uint2(w1.z, w1.w)};
                d = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    d = mfma_bf16_k32(as_v8bf(e4m3x8_to_bf16(c[i])), bh[i], d);
                sc = sdv;
            } else {
                d = mfma_fp8_k128(as_v8i(w0, w1), bq);
                sc = shs[(t * KS + js) * IB + b] * sdv;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[u][i] = fmaf(sc, d[i], acc[u][i]);
        }
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int js = js_lane + 8 * u;
        // D rows 4 kq + i are slot 2 tau + (kq >> 1), rows m0 + 4 (kq & 1) + i;
        // the lane whose column is that slot holds the product wanted
        if (js < KS && l16 == js)
#pragma unroll
            for (int i = 0; i < 4; ++i) ej[js * MB + 4 * (kq & 1) + i] = bf16_round(acc[u][i]);
    }
    if (Isb > 0 && chain) {  // else computed before the h handoff
        down_stage_shared<KBR, TPW>(r, sdo);
        __syncthreads();
        if (wave == CHAIN_WAVE) {
            const float s = shared_down_chain(a, t, m0, sdo, hs_l);
            if (lane < MB) ss[lane] = s;
        }
    }
    __syncthreads();

    // combine: slots in order, then the shared term
    if (tid < MB) {
        float yacc = 0.0f;
        for (int j = 0; j < K; ++j) yacc = fmaf(wts[t * KS + j], ej[j * MB + tid], yacc);
        if (Is > 0) yacc = fmaf(gam_l[t], VAR == DV_SFP8 ? ej[K * MB + tid] : ss[tid], yacc);
        const uint16_t yb = (uint16_t)f32_to_bf16(yacc);
        a.y[(int64_t)t * H + m0 + tid] = yb;
        if (a.y2) a.y2[(int64_t)t * H + m0 + tid] = yb;
    }
    __syncthreads();  // ej and ss are reused by the next unit
}

// ---------------------------------------------------------------- kernel

// LDS carve-up of the fused kernel, every piece 16-byte aligned
struct LdsPlan {
    int qx, sx, qh, shs, ids, wts, hs, gam, ej, ss, rl, xs, red, sq, sp, sdo, total;
};
__host__ __device__ inline int al16i(int b) { return (b + 15) & ~15; }
// slots per row of variant var: the block-FP8 shared expert is one more
// slot with the routed experts' shape (Is = I) and at most 16 slots fit the
// phase-C tiles; -1 when the kernel cannot run the variant
int decode_slots(int var, int K, int I, int Is) {
    if (var != DV_SFP8) return K;
    if (Is != I || K + 1 > 16) return -1;
    return K + 1;
}

__host__ __device__ inline LdsPlan lds_plan(int T, int H, int K, int I, int Is, int var) {
    LdsPlan L;
    if (var == DV_SFP8) {
        K += 1;  // slots
        Is = 0;  // no bf16 shared expert
    }
    const int P = T * K, KB = H / GROUP, KH = (KB + 1) / 2;
    L.qx = 0;
    L.sx = L.qx + al16i(T * H);
    L.qh = L.sx + al16i(T * KB * 4);
    L.shs = L.qh + al16i(P * I * (var == DV_NOQ ? 2 : 1));  // codes, or bf16 h
    L.ids = L.shs + al16i(P * (I / GROUP) * 4);
    L.wts = L.ids + al16i(P * 8);  // ids: one 64-bit slot word per pair
    L.hs = L.wts + al16i(P * 4);
    L.gam = L.hs + al16i(T * Is * 2);
    L.ej = L.gam + al16i(T * 4);          // phase-C unit: e_j of its rows, every slot
    L.ss = L.ej + al16i(K * MB * 4);      // phase-C unit: shared down of its rows
    L.rl = L.ss + al16i(MB * 4);          // router: 2 x 4 fp64 wave partials
    L.xs = L.rl + 64;                     // x rows, bf16
    L.red = L.xs + al16i(T * H * 2);      // renormalisation: 4 fp64 partial sums
    L.sq = L.red + 32;                    // shared gate/up partials, per wave [KB][16]
    L.sp = L.sq + 4 * al16i(KB * 16 * 4); // routed gate/up second halves, per wave [KH][8]
    L.sdo = L.sp + 4 * al16i(KH * 8 * 8); // shared down operands [SDB][4][64] uint4
    L.total = L.sdo + (Is > 0 ? SDB * 4 * 64 * 16 : 0);
    return L;
}

bool decode_fits(int T, int H, int K, int I, int Is, int var) {
    return T >= 1 && T <= DECODE_MAX_ROWS && decode_slots(var, K, I, Is) > 0 &&
           lds_plan(T, H, K, I, Is, var).total <= 150 * 1024;
}

// h groups each 16-lane team stages per round of loads
constexpr int STAGE_HG = 2;

// 1x128 quantisation of one group held by a 16-lane team, lane `sub` holding
// the values sub + 16 q (q < 8), into LDS codes and the group's scale
__device__ __forceinline__ void quant8_strided_to_lds(const float (&f)[8], int g, int sub,
                                                      uint8_t *q, float *s) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = group16_max(amax);
    const float sc = group_scale(amax);
    const uint32_t c0 = e4m3x4(f[0] / sc, f[1] / sc, f[2] / sc, f[3] / sc);
    const uint32_t c1 = e4m3x4(f[4] / sc, f[5] / sc, f[6] / sc, f[7] / sc);
    uint8_t *row = q + g * GROUP + sub;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        row[16 * i] = (uint8_t)(c0 >> (8 * i));
        row[16 * (i + 4)] = (uint8_t)(c1 >> (8 * i));
    }
    if (sub == 0) s[g] = sc;
}

// Phase C inputs from this workgroup's copy, waiting for each word's epoch:
// h (fp32, re-quantised 1x128 into LDS codes and scales), hs (bf16) and
// gamma into LDS. stage_c_issue sends the first loads of hs, gamma and of the
// first round of h, in that order (a wave's loads return in issue order);
// stage_c_finish_shared waits for hs and gamma alone, stage_c_finish_h for
// h, so the shared down product can run in between.
struct StageC {
    int sidx[8], gidx[1], hidx[8 * STAGE_HG];
    int n_s0, n_g, nk0;
    uint64_t sw[8], gw[1], hw[8 * STAGE_HG];
};

// h: team j of a round stages groups base + team + teams * k, k < STAGE_HG;
// lane `sub` of a team takes the words sub + 16 i of a group, so every load
// instruction of a team reads one whole 128-byte line
__device__ __forceinline__ int stage_h_round(int base, int n_groups, int (&idx)[8 * STAGE_HG]) {
    const int teams = blockDim.x >> 4, team = threadIdx.x >> 4, sub = threadIdx.x & 15;
#pragma unroll
    for (int k = 0; k < STAGE_HG; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) idx[8 * k + i] = (base + team + teams * k) * GROUP + 16 * i + sub;
    return min(STAGE_HG, max(0, (n_groups - base - team + teams - 1) / teams));
}

__device__ __forceinline__ void stage_h_quant(int base, int nk, const uint32_t (&bits)[8 * STAGE_HG],
                                              uint8_t *qh, float *shs) {
    const int teams = blockDim.x >> 4, team = threadIdx.x >> 4, sub = threadIdx.x & 15;
#pragma unroll
    for (int k = 0; k < STAGE_HG; ++k)
        if (k < nk) {
            float f[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = __uint_as_float(bits[8 * k + i]);
            quant8_strided_to_lds(f, base + team + teams * k, sub, qh, shs);
        }
}

// the control's h: bf16 values (the words' low half) into LDS, no scales
__device__ __forceinline__ void stage_h_bf16(int base, int nk, const uint32_t (&bits)[8 * STAGE_HG],
                                             uint8_t *qh) {
    const int teams = blockDim.x >> 4, team = threadIdx.x >> 4, sub = threadIdx.x & 15;
    uint16_t *hb = reinterpret_cast<uint16_t *>(qh);
#pragma unroll
    for (int k = 0; k < STAGE_HG; ++k)
        if (k < nk) {
            uint16_t *row = hb + (base + team + teams * k) * GROUP + sub;
#pragma unroll
            for (int i = 0; i < 8; ++i) row[16 * i] = (uint16_t)bits[8 * k + i];
        }
}

// Isb: width of the bf16 shared expert (hs); gam: whether gamma exists
__device__ __forceinline__ void stage_c_issue(const uint64_t *h, const uint64_t *hs,
                                              const uint64_t *gamma, int T, int P, int I, int Isb,
                                              bool gam, uint32_t epoch, StageC &c) {
    const int rp = blockIdx.x % REPL, tid = threadIdx.x, nth = blockDim.x;
    const int n_hs = T * Isb;
#pragma unroll
    for (int i = 0; i < 8; ++i) c.sidx[i] = tid + nth * i;
    c.n_s0 = min(8, max(0, (n_hs - tid + nth - 1) / nth));
    c.gidx[0] = rp * T + tid;
    c.n_g = gam && tid < T ? 1 : 0;
    c.nk0 = stage_h_round(0, P * (I / GROUP), c.hidx);
    // hs and gamma first: they were written in phase A, and waiting for
    // them must not also wait for the h words behind them
    poll_issue<8>(hs + (int64_t)rp * T * Isb, c.sidx, c.n_s0, epoch, c.sw);
    poll_issue<1>(gamma, c.gidx, c.n_g, epoch, c.gw);
    poll_issue<8 * STAGE_HG>(h + (int64_t)rp * P * I, c.hidx, 8 * c.nk0, epoch, c.hw);
}

__device__ __forceinline__ void stage_c_finish_shared(const uint64_t *hs, const uint64_t *gamma,
                                                      int T, int Is, uint32_t epoch,
                                                      uint32_t *err, StageC &c, uint16_t *hs_l,
                                                      float *gam_l) {
    const int rp = blockIdx.x % REPL, tid = threadIdx.x, nth = blockDim.x;
    const uint64_t *ssrc = hs + (int64_t)rp * T * Is;
    const int n_hs = T * Is;
    {
        uint32_t bits[8];
        poll_finish<8>(err, ssrc, c.sidx, c.n_s0, epoch, c.sw, bits);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < c.n_s0) hs_l[c.sidx[i]] = (uint16_t)bits[i];
    }
    if (c.n_g) {
        uint32_t bits[1];
        poll_finish<1>(err, gamma, c.gidx, 1, epoch, c.gw, bits);
        gam_l[tid] = __uint_as_float(bits[0]);
    }
    for (int b = nth * 8; b < n_hs; b += nth * 8) {  // further rounds of hs (Is > 512 rows)
        int idx[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) idx[i] = b + tid + nth * i;
        const int n = min(8, max(0, (n_hs - b - tid + nth - 1) / nth));
        uint32_t bits[8];
        poll_words<8>(err, ssrc, idx, n, epoch, bits);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < n) hs_l[idx[i]] = (uint16_t)bits[i];
    }
}

template <int VAR, bool RN>
__device__ __forceinline__ void stage_c_finish_h(const uint64_t *h, int T, int P, int I,
                                                 uint32_t epoch, uint32_t *err, StageC &c,
                                                 uint8_t *qh, float *shs) {
    const int rp = blockIdx.x % REPL, teams = blockDim.x >> 4;
    const uint64_t *hsrc = h + (int64_t)rp * P * I;
    const int n_groups = P * (I / GROUP);
    {
        uint32_t bits[8 * STAGE_HG];
        // the lone layer: three re-poll rounds; the renormalising one: two
        poll_complete<8 * STAGE_HG, RN ? 2 : 3, RN ? POLL_GAP_RN : POLL_GAP>(
            err, handoff_region(hsrc, P * I), c.hidx, 8 * c.nk0, epoch, c.hw, bits);
        if constexpr (VAR == DV_NOQ) stage_h_bf16(0, c.nk0, bits, qh);
        else stage_h_quant(0, c.nk0, bits, qh, shs);
    }
    for (int base = STAGE_HG * teams; base < n_groups; base += STAGE_HG * teams) {
        int idx[8 * STAGE_HG];
        const int nk = stage_h_round(base, n_groups, idx);
        uint32_t bits[8 * STAGE_HG];
        poll_words<8 * STAGE_HG>(err, hsrc, idx, 8 * nk, epoch, bits);
        if constexpr (VAR == DV_NOQ) stage_h_bf16(base, nk, bits, qh);
        else stage_h_quant(base, nk, bits, qh, shs);
    }
}

// Renormalising prologue: x_t = bf16(y_prev_t * rms scale) into LDS, every
// workgroup for every row, with the stand-alone renormalisation's arithmetic
// (renorm_row_scale, renorm_chunk). y_prev was written by an earlier launch.
// CH chunks of 8 values per thread cover H (one up to 2048)
template <int CH>
__device__ __forceinline__ void renorm_rows_to_lds(const uint16_t *y, int T, int H, float eps,
                                                   uint16_t *xs, double *red) {
    const int tid = threadIdx.x, nc = H / 8;
    for (int t = 0; t < T; ++t) {
        uint4 v[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + 256 * i;
            v[i] = c < nc ? ld16(y + (int64_t)t * H + c * 8) : make_uint4(0, 0, 0, 0);
        }
        const float r = renorm_row_scale<CH>(v, H, eps, red);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + 256 * i;
            if (c < nc) st16(xs + t * H + c * 8, renorm_chunk(v[i], r));
        }
        __syncthreads();  // red is reused by the next row
    }
}

// RN: the renormalising variant (x from y_prev in the prologue)
template <int NQ, int KBR, int TPW, bool RN, int VAR>
__global__ __launch_bounds__(256, 1) void decode_fused_kernel(FusedArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int T = a.T, H = a.H, K = a.K, KS = a.KS, I = a.I, E = a.E, P = T * KS, Is = a.Is;
    const int Isb = VAR == DV_SFP8 ? 0 : Is;  // width of the bf16 shared expert
    const int KB = H / GROUP, KH = (KB + 1) / 2;
    const LdsPlan L = lds_plan(T, H, K, I, Is, VAR);
    uint8_t *qx = lds + L.qx;                                 // [T][H]
    float *sx = reinterpret_cast<float *>(lds + L.sx);        // [T][H/128]
    uint8_t *qh = lds + L.qh;                                 // [P][I] (bf16 with DV_NOQ)
    float *shs = reinterpret_cast<float *>(lds + L.shs);      // [P][I/128]
    uint64_t *slots = reinterpret_cast<uint64_t *>(lds + L.ids);  // [P] published experts
    float *wts = reinterpret_cast<float *>(lds + L.wts);      // [P]
    uint16_t *hs_l = reinterpret_cast<uint16_t *>(lds + L.hs);  // [T][Isb]
    float *gam_l = reinterpret_cast<float *>(lds + L.gam);      // [T]
    float *ej = reinterpret_cast<float *>(lds + L.ej);          // [KS][MB]
    float *ss = reinterpret_cast<float *>(lds + L.ss);          // [MB]
    double *rl = reinterpret_cast<double *>(lds + L.rl);        // [2][4]
    uint16_t *xs = reinterpret_cast<uint16_t *>(lds + L.xs);    // [T][H]
    uint4 *sdo = reinterpret_cast<uint4 *>(lds + L.sdo);        // [SDB][4][64]

    const int wave = threadIdx.x >> 6;
    const int nw = a.nwg * 4;
    const int gw = wave * a.nwg + blockIdx.x;  // workgroup-major wave index
    float *sq = reinterpret_cast<float *>(lds + L.sq + wave * al16i(KB * 16 * 4));
    float2 *sp = reinterpret_cast<float2 *>(lds + L.sp + wave * al16i(KH * 8 * 8));
    // The counter's load goes out first but is waited for only after the
    // first weight loads have been issued: it is a full device-coherent round
    // trip, and nothing before the first tagged store needs the epoch.
    uint32_t *counter = a.sync + SYNC_FLAGS + blockIdx.x;
    const uint32_t cnt = ld_dev(counter);
    uint32_t *err = a.sync + ERR_WORD;
    if ((int)threadIdx.x < P) slots[threadIdx.x] = 0;  // unpublished, before the barrier below

    // phase-C units (t, MB-row block), workgroup-major; a workgroup past the
    // last unit loads the last unit's rows (unused), so its loads need no
    // branch
    const int units = T * (H / MB);
    const int u_first = min((int)blockIdx.x, units - 1);
    const int t_first = u_first / (H / MB), m_first = (u_first % (H / MB)) * MB;

    // A1: router logits, one per workgroup at a time (four waves each),
    // before any other load; then x into LDS. In a stack's later layer the
    // router rows go out first and the previous layer's output is
    // renormalised into LDS while they are in flight.
    const int n_logits = T * E;
    uint32_t epoch;
    {
        RouterRegs<NQ> rr;
        if constexpr (RN) {
            if ((int)blockIdx.x < n_logits) router_load_w<NQ>(a, blockIdx.x, rr);
            renorm_rows_to_lds<NQ>(a.y_prev, T, H, a.eps, xs,
                                   reinterpret_cast<double *>(lds + L.red));
            if ((int)blockIdx.x < n_logits) router_load_x<NQ, RN>(a, blockIdx.x, xs, rr);
        } else {
            if ((int)blockIdx.x < n_logits) router_load<NQ, RN>(a, blockIdx.x, xs, rr);
        }
        epoch = __builtin_amdgcn_readfirstlane(call_epoch(cnt));
        int round = 0;
        for (int r = blockIdx.x; r < n_logits; r += a.nwg, ++round) {
            if (round > 0) router_load<NQ, RN>(a, r, xs, rr);
            router_logit<NQ>(a, r, rr, rl + 4 * (round & 1), epoch);
        }
        if (!RN && T == 1 && (int)blockIdx.x < n_logits) x_stage_router<NQ>(rr, H, xs, qx, sx);
        else x_stage_rows<RN>(a.x, T, H, xs, qx, sx);
    }
    __syncthreads();  // xs, qx, sx ready

    // A2: the shared expert's gate/up columns and the shared gate, on wave 3
    // (wave 0 runs the top-K next, and a wave with loads in flight would wait
    // for them before its first poll; waves 1 and 2 start their routed
    // gate/up items as soon as the top-K has published their slots). The
    // block-FP8 shared expert is slot K of every row: its gate/up items are
    // the routed items' (expert E), with h handed over among the routed
    // pairs' h.
    if (wave == 3 && Is > 0) {
        if constexpr (VAR == DV_SFP8) {
            const int per_row = Is / 4, n_s = T * per_row, n_items = n_s + T;
            for (int it = blockIdx.x; it < n_items; it += a.nwg) {
                if (it < n_s) {
                    const int t = it / per_row, n0 = (it % per_row) * 4;
                    GateUpRegs gr;
                    gateup_load<VAR>(a, E, n0, 0, gr);
                    gateup_finish<VAR>(a, t * KS + K, n0, E, gr, qx, sx, xs, sp, epoch);
                } else {
                    g_item(a, it - n_s, xs, epoch);
                }
            }
        } else {
            const int n_s = Is / 2, n_items = n_s + T;
            for (int it = blockIdx.x; it < n_items; it += a.nwg) {
                if (it < n_s) s_item(a, it, xs, sq, epoch);
                else g_item(a, it - n_s, xs, epoch);
            }
        }
    }

    // B: top-K per row (one wave per row) once its logits exist, each slot
    // published in LDS as its round ends; then the routed gate/up items, each
    // wave waiting only for the slot of its own item (no barrier: a wave
    // whose slot comes out in an early round starts its loads while the
    // later rounds run)
    for (int t = wave; t < T; t += 4) {
        if (VAR == DV_SFP8 && (threadIdx.x & 63) == 0) {  // slot K: the shared expert
            publish_slot(slots + t * KS + K, E);
            wts[t * KS + K] = 0.0f;
        }
        topk_tagged<RN ? POLL_GAP_RN : POLL_GAP>(
            a.logits + (int64_t)((blockIdx.x % REPL) * T + t) * E, E, K, epoch, err,
            threadIdx.x & 63, slots + t * KS, wts + t * KS, !a.bias && !(a.flags & K_LOGITS_FP32));
    }
    // Routed item it: pair (t, j) of the T * K routed pairs (pair index
    // t * KS + j), columns n0..n0+3. The first unit's routed and shared down
    // rows are issued once this wave's first gate/up rows are in and their h
    // has gone out: they stream in while the h handoff runs, without
    // competing with the gate/up rows (issued alongside them, they held the
    // gate/up phase back by about 0.8 us and the layer by about 0.4 us).
    // Scheduling barriers keep the three steps in this order.
    const int per_pair = I / 4, n_items = T * K * per_pair;
    DownRegs<KBR, TPW> dr;
    {
        const int it = min(gw, n_items - 1);  // waves past the last item load it (unused)
        const int rp = it / per_pair, t = rp / K, j = rp - t * K, p = t * KS + j;
        const int n0 = (it - rp * per_pair) * 4;
        const int e = wait_slot(slots + p, err);
        GateUpRegs gr;
        gateup_load<VAR>(a, e, n0, 0, gr);
        __builtin_amdgcn_sched_barrier(0);
        if (gw < n_items) gateup_finish<VAR>(a, p, n0, e, gr, qx, sx, xs, sp, epoch);
        __builtin_amdgcn_sched_barrier(0);
        wait_row(slots + t_first * KS, KS, err);  // every slot of the unit's row
        down_load_routed<KBR, TPW, VAR>(a, t_first, m_first, slots, dr);
        if (Isb > 0) down_load_shared<KBR, TPW>(a, m_first, dr);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int it = gw + nw; it < n_items; it += nw) {
        const int rp = it / per_pair, t = rp / K, j = rp - t * K, p = t * KS + j;
        const int n0 = (it - rp * per_pair) * 4;
        const int e = wait_slot(slots + p, err);
        GateUpRegs gr;
        gateup_load<VAR>(a, e, n0, 0, gr);
        gateup_finish<VAR>(a, p, n0, e, gr, qx, sx, xs, sp, epoch);
    }

    // C: hs and gamma (ready since phase A) into LDS, the first unit's
    // shared down rows while h is still on its way, then h (re-quantised)
    // into LDS once it exists, and whole output rows with the combine.
    StageC sc;
    stage_c_issue(a.h, a.hs, a.gamma, T, P, I, Isb, Is > 0, epoch, sc);
    __builtin_amdgcn_sched_barrier(0);
    stage_c_finish_shared(a.hs, a.gamma, T, Isb, epoch, err, sc, hs_l, gam_l);
    if (Isb > 0) down_stage_shared<KBR, TPW>(dr, sdo);
    __syncthreads();
    if (Isb > 0 && wave == CHAIN_WAVE && (int)blockIdx.x < units) {
        const float s = shared_down_chain(a, t_first, m_first, sdo, hs_l);
        if ((threadIdx.x & 63) < MB) ss[threadIdx.x & 63] = s;
    }
    stage_c_finish_h<VAR, RN>(a.h, T, P, I, epoch, err, sc, qh, shs);
    __syncthreads();
    for (int u = blockIdx.x; u < units; u += a.nwg) {
        const int t = u / (H / MB), m0 = (u % (H / MB)) * MB;
        const bool first = u == (int)blockIdx.x;
        if (!first) {
            down_load_routed<KBR, TPW, VAR>(a, t, m0, slots, dr);
            if (Isb > 0) down_load_shared<KBR, TPW>(a, m0, dr);
        }
        down_unit<KBR, TPW, VAR>(a, t, m0, dr, qh, shs, slots, wts, hs_l, gam_l, ej, ss, sdo,
                                 !first);
    }
    // every wave has read the counter: advance it for the next call
    if (threadIdx.x == 0) st_dev(counter, call_epoch(cnt) + 1u);
}

// NQ: router chunks per lane (H / 2048, rounded up to 1 or 4); KBR: K blocks
// of a down row held in registers (I / 128 up to 4; more are loaded in the
// loop); TPW: MFMA tiles (slot pairs) per wave (KS up to 8: one, up to 16:
// two); VAR: the layer or one of its switches (the renormalising prologue
// only with the plain layer)
// Every workgroup waits for values other workgroups produce, so all of the
// grid (one workgroup per CU) must be resident at once: the launch is
// refused unless one workgroup with the largest LDS plan the decode path
// takes fits on a CU (checked once per kernel variant).
template <int NQ, int KBR, int TPW, bool RN, int VAR>
static hipError_t launch_v(const FusedArgs &a, size_t lds, hipStream_t st) {
    static const hipError_t fits = [] {
        int n = 0;
        const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void *>(&decode_fused_kernel<NQ, KBR, TPW, RN, VAR>), 256,
            150 * 1024);
        return e != hipSuccess ? e : n >= 1 ? hipSuccess : hipErrorInvalidConfiguration;
    }();
    if (fits != hipSuccess) return fits;
    hipLaunchKernelGGL((decode_fused_kernel<NQ, KBR, TPW, RN, VAR>), dim3(a.nwg), dim3(256), lds,
                       st, a);
    return hipGetLastError();
}

template <int NQ, int TPW, bool RN, int VAR>
static hipError_t launch_t(const FusedArgs &a, size_t lds, hipStream_t st) {
    const int ib = a.I / GROUP;
    if (ib <= 1) return launch_v<NQ, 1, TPW, RN, VAR>(a, lds, st);
    if (ib <= 2) return launch_v<NQ, 2, TPW, RN, VAR>(a, lds, st);
    return launch_v<NQ, 4, TPW, RN, VAR>(a, lds, st);
}

template <int NQ, bool RN, int VAR>
static hipError_t launch_nq(const FusedArgs &a, size_t lds, hipStream_t st) {
    if (a.KS <= 8) return launch_t<NQ, 1, RN, VAR>(a, lds, st);
    return launch_t<NQ, 2, RN, VAR>(a, lds, st);
}

template <int NQ, int KBR, int TPW, bool RN, int VAR>
static void set_lds_limit() {
    (void)hipFuncSetAttribute(
        reinterpret_cast<const void *>(&decode_fused_kernel<NQ, KBR, TPW, RN, VAR>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
}

template <int NQ, bool RN, int VAR>
static void set_lds_limits() {
    set_lds_limit<NQ, 1, 1, RN, VAR>();
    set_lds_limit<NQ, 2, 1, RN, VAR>();
    set_lds_limit<NQ, 4, 1, RN, VAR>();
    set_lds_limit<NQ, 1, 2, RN, VAR>();
    set_lds_limit<NQ, 2, 2, RN, VAR>();
    set_lds_limit<NQ, 4, 2, RN, VAR>();
}

template <int NQ>
static hipError_t launch_var(const FusedArgs &a, size_t lds, hipStream_t st) {
    if (a.y_prev) return a.var == DV_PLAIN ? launch_nq<NQ, true, DV_PLAIN>(a, lds, st)
                                           : hipErrorInvalidValue;
    if (a.var == DV_SFP8) return launch_nq<NQ, false, DV_SFP8>(a, lds, st);
    if (a.var == DV_NOQ) return launch_nq<NQ, false, DV_NOQ>(a, lds, st);
    return launch_nq<NQ, false, DV_PLAIN>(a, lds, st);
}

// copies the spin-out word to *out and, with clear, zeroes it (one thread)
__global__ void decode_status_kernel(uint32_t *sync, uint32_t *out, int clear) {
    out[0] = ld_dev(sync + ERR_WORD);
    if (clear) st_dev(sync + ERR_WORD, 0u);
}

hipError_t launch_decode_status(uint32_t *sync, uint32_t *out, int clear, hipStream_t st) {
    hipLaunchKernelGGL(decode_status_kernel, dim3(1), dim3(1), 0, st, sync, out, clear);
    return hipGetLastError();
}

hipError_t launch_decode_fused(const FusedArgs &a, hipStream_t st) {
    if (a.var < DV_PLAIN || a.var > DV_NOQ || a.KS != decode_slots(a.var, a.K, a.I, a.Is))
        return hipErrorInvalidValue;
    const size_t lds = (size_t)lds_plan(a.T, a.H, a.K, a.I, a.Is, a.var).total;
    if (lds > 64 * 1024) {
        static const bool once = [] {
            set_lds_limits<1, false, DV_PLAIN>();
            set_lds_limits<4, false, DV_PLAIN>();
            set_lds_limits<1, true, DV_PLAIN>();
            set_lds_limits<4, true, DV_PLAIN>();
            set_lds_limits<1, false, DV_SFP8>();
            set_lds_limits<4, false, DV_SFP8>();
            set_lds_limits<1, false, DV_NOQ>();
            set_lds_limits<4, false, DV_NOQ>();
            return true;
        }();
        (void)once;
    }
    if (a.H <= 2048) return launch_var<1>(a, lds, st);
    return launch_var<4>(a, lds, st);
}

}  // namespace moe
