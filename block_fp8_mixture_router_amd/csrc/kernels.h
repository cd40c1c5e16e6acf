// Internal launchers of libmoe's gfx950 kernels. Every launcher enqueues on
// `st` and returns the launch status; shapes were validated by the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// flags understood by the router kernels (same bit as the public flag)
constexpr uint32_t K_LOGITS_FP32 = 1u << 1;

// ---- quant.hip
// the kernels' fp32 -> e4m3 conversion on n values (x 16-byte aligned)
hipError_t launch_e4m3_encode(const float *x, int64_t n, uint8_t *q, hipStream_t st);
hipError_t launch_quant_act(const uint16_t *x, int64_t n_groups, uint8_t *q, float *s,
                            hipStream_t st);

// ---- renorm.hip (row RMS normalisation between stacked layers; H <= 8192)
hipError_t launch_rms_renorm(const uint16_t *y, int T, int H, float eps, uint16_t *x,
                             hipStream_t st);

// ---- addnorm.hip (residual add + RMS norm + 1x128 quantisation, before the layer)
hipError_t launch_add_rmsnorm_quant(const uint16_t *hidden, const uint16_t *res_in,
                                    const uint16_t *norm_w, int T, int H, float eps,
                                    uint16_t *res_out, uint16_t *x, uint8_t *q, float *s,
                                    hipStream_t st);

// ---- route.hip
hipError_t launch_route_logits(const uint16_t *x, int T, const uint16_t *router_w,
                               const float *bias, int H, int E, uint32_t flags, float *logits,
                               hipStream_t st);
// many rows: bf16 MFMA scores S (approximate logits) and A (sums of |x||w|)
hipError_t launch_route_scores(const uint16_t *x, int T, const uint16_t *router_w, int H, int E,
                               float *S, float *A, hipStream_t st);
// top-K + softmax per row from bounded scores, with exact logits for the
// experts the bound leaves undecided; gate_w/gamma and qx/sx as below
hipError_t launch_route_topk_bounded(const float *S, const float *A, int T, int E, int K,
                                     const uint16_t *x, const uint16_t *router_w,
                                     const float *bias, uint32_t flags, int H, int32_t *ids,
                                     float *weights, const uint16_t *gate_w, float *gamma,
                                     uint8_t *qx, float *sx, hipStream_t st);
// top-K + softmax per row; when gate_w != NULL also gamma[t] = sigmoid(gate_w . x[t])
// packed: every logit is a plain bf16 value (no bias, bf16 rounding on);
// qx/sx (or NULL): also write the 1x128 e4m3 quantisation of x
hipError_t launch_route_topk(const float *logits, int T, int E, int K, int32_t *ids,
                             float *weights, const uint16_t *x, const uint16_t *gate_w, int H,
                             float *gamma, bool packed, uint8_t *qx, float *sx,
                             hipStream_t st);

// ---- decode.hip (row-at-a-time path: one persistent kernel per layer)
// what the one-row kernel computes: the layer as the pages define it, or one
// of its two switches (the block-FP8 shared expert, run as one more slot of
// every row; the control without activation quantisation)
constexpr int DV_PLAIN = 0, DV_SFP8 = 1, DV_NOQ = 2;
struct FusedArgs {
    int T, H, E, K, I, Is;
    int KS;   // slots per row: K, or K + 1 when the block-FP8 shared expert is slot K
    int var;  // DV_*
    uint32_t flags;
    const uint16_t *x, *router_w;
    const float *bias;
    const uint8_t *w_gate, *w_up, *w_down;
    const float *s_gate, *s_up, *s_down;
    const uint16_t *sh_gate, *sh_up, *sh_down, *sh_gate_w;
    // DV_SFP8: the shared expert's e4m3 rows and 128x128 block scales
    const uint8_t *sh8_gate, *sh8_up, *sh8_down;
    const float *sh_s_gate, *sh_s_up, *sh_s_down;
    // values that cross workgroups are 64-bit words (32-bit value, call
    // epoch) kept in DECODE_REPLICAS copies, so each copy is read by
    // 1/DECODE_REPLICAS of the workgroups
    uint64_t *logits;  // [R][T, E] fp32 logits
    uint64_t *gamma;   // [R][T] fp32
    uint64_t *hs;      // [R][T, Is] bf16 shared-expert SwiGLU output
    uint64_t *h;       // [R][T*KS, I] fp32 routed SwiGLU output (bf16 bits with DV_NOQ)
    uint32_t *sync;    // [ERR_WORD] spin-out flag, [SYNC_FLAGS + b] workgroup b's call counter
    uint16_t *y;       // [T, H]
    uint16_t *y2;      // [T, H] a second copy of y, or null
    int nwg;           // workgroups = compute units (all co-resident)
    // renormalising variant (the layers of a stack after the first): the
    // layer's input is x = bf16(y_prev * rms scale), computed by every
    // workgroup in the kernel's prologue (x is then unused)
    const uint16_t *y_prev;  // [T, H], or null for the plain layer
    float eps;
};
constexpr int DECODE_MAX_ROWS = 4;
constexpr int DECODE_REPLICAS = 8;
constexpr int SYNC_FLAGS = 64;
constexpr int SYNC_WORDS = SYNC_FLAGS + 1024;  // up to 1024 workgroups
constexpr int SYNC_ERR_WORD = 32;              // the spin-out word
// slots per row of the one-row kernel for variant var (-1: it cannot run it)
int decode_slots(int var, int K, int I, int Is);
bool decode_fits(int T, int H, int K, int I, int Is, int var);
hipError_t launch_decode_fused(const FusedArgs &a, hipStream_t st);
// the decode path's spin-out word (workspace sync word SYNC_ERR_WORD) -> out
hipError_t launch_decode_status(uint32_t *sync, uint32_t *out, int clear, hipStream_t st);

// ---- grouped.hip (expert-grouped MFMA path)
struct GroupedArgs {
    int T, H, E, K, I, Is;
    const uint16_t *x;
    const uint8_t *qx;   // [T, H] e4m3
    const float *sx;     // [T, H/128]
    const int32_t *ids;  // [T, K]
    const float *wts;    // [T, K]
    const float *gamma;  // [T]
    const uint8_t *w_gate, *w_up, *w_down;
    const float *s_gate, *s_up, *s_down;
    const uint16_t *sh_gate, *sh_up, *sh_down;
    int32_t *offsets;    // [E + 1] start of each expert in the sorted pair list
    int32_t *perm;       // [T*K] sorted position -> pair id (t*K + j)
    int32_t *tiles;      // [max_tiles * 4] (expert, first sorted row, rows, 0)
    int32_t *n_tiles;    // [1]
    int max_tiles;
    uint8_t *qh;         // [T*K, I] e4m3, sorted order
    float *sh;           // [T*K, I/128]
    uint16_t *hs;        // [T, Is] bf16
    uint16_t *stage;     // [T*K, H] bf16 expert outputs e_j, pair order
    uint16_t *hb;        // [T*K, I] bf16 h, sorted order (no-quantisation control only)
    const uint16_t *es;  // [T, H] bf16 block-FP8 shared expert output, or null
    float *ss;           // [T, H] fp32 bf16 shared expert's down output, or null
    uint16_t *y;         // [T, H]
};
constexpr int GROUP_ROWS = 64;  // rows (token, slot) per MFMA work tile
int grouped_max_tiles(int T, int K, int E);
hipError_t launch_group_sort(const GroupedArgs &a, hipStream_t st);
// the shared expert's gate/up (when Is > 0) and the routed experts' gate/up,
// one launch
hipError_t launch_expert_gateup(const GroupedArgs &a, hipStream_t st);
// the shared expert's down (when Is > 0, into ss) and the routed experts'
// down (into stage), one launch
hipError_t launch_grouped_down(const GroupedArgs &a, hipStream_t st);
// y = sum_j w_j e_j + gamma s, from stage and ss (or es)
hipError_t launch_combine(const GroupedArgs &a, hipStream_t st);
// the no-activation-quantisation control: routed gate/up and down on bf16
// activations and decoded e4m3 weights (writes hb, then stage)
hipError_t launch_grouped_noq(const GroupedArgs &a, hipStream_t st);
// identity pair list and 64-row tiles over T rows (the block-FP8 shared
// expert run through the routed kernels as one expert holding every row)
hipError_t launch_shared_tiles(int T, int32_t *perm, int32_t *tiles, int32_t *n_tiles,
                               hipStream_t st);

}  // namespace moe
