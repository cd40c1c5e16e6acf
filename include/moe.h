/*
 * libmoe: a block-FP8 mixture-of-experts layer for AMD Instinct MI355X (gfx950).
 *
 * The layer is the backbone MoE of the "Drama 3" speech model described on
 * the pages: 256 routed experts with top-8 routing, block-FP8 (e4m3, one fp32
 * scale per 128x128 block) expert weights, and a gated shared expert (PR #925
 * "drama: load the checkpoint with direct I/O in file order and build the
 * codec on its own thread", commit summary of the Drama 3 backbone).
 * Activations are bf16 and the FP8 experts quantise their input rows to e4m3
 * per row and per 128 columns with scale amax / 448 (PR #939 "drama3: Fish
 * Audio Drama 3 text to speech on one CUDA GPU", "How it fits the engine" >
 * Precision).
 *
 * Conventions shared by every call:
 *  - Pointers named as device pointers are device memory owned by the caller.
 *    bf16 and e4m3 tensors are 16-byte aligned; fp32 scale, bias, weight and
 *    logit arrays and int32 id arrays are 4-byte aligned; the workspace is
 *    256-byte aligned. Config structs are host memory, read during the call
 *    only.
 *  - Matrices are row-major and dense; weight matrices are [out, in].
 *  - bf16 tensors are passed as void* (16-bit storage).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *    work is enqueued on it; no call synchronises, copies to the host or
 *    allocates memory.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    refused call returns a negative moe_status and enqueues nothing.
 *    MOE_E_LAUNCH reports a failed kernel launch. Faults inside kernels
 *    surface at the caller's next synchronisation.
 *  - Results are deterministic: the same inputs give the same bytes on every
 *    call. The only state kept between calls is moe_forward's bookkeeping in
 *    the caller's workspace (see there); calls may run on several streams at
 *    once when their workspaces and outputs are distinct.
 *
 * Supported shapes: hidden H and expert intermediate I are multiples of 128
 * with 128 <= H <= 8192 and 128 <= I <= 4096; the shared intermediate Is is a
 * multiple of 128 up to 4096, or 0 for no shared expert; 1 <= E <= 1024;
 * 1 <= K <= min(E, 16); 0 <= T <= 65536 rows (T = 0 does nothing and
 * returns MOE_OK).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_E_NULL = -1,        /* a required pointer is NULL */
    MOE_E_SHAPE = -2,       /* a size is outside the supported shapes above */
    MOE_E_ALIGN = -3,       /* a pointer is not aligned as required */
    MOE_E_WORKSPACE = -4,   /* workspace smaller than moe_workspace_bytes() */
    MOE_E_UNSUPPORTED = -5, /* the current device is not gfx950, or bad flags */
    MOE_E_LAUNCH = -6       /* a kernel launch failed */
} moe_status;

/* moe_config.flags */
#define MOE_SHARED_FP8    (1u << 0) /* variant: the shared expert stored block-FP8 (codes and
                                       128x128 block scales sh_s_*), run exactly as a routed
                                       expert on the quantised rows, gamma in place of w;
                                       moe_forward only */
#define MOE_LOGITS_FP32   (1u << 1) /* decide on fp32 router logits (no bf16 rounding) */
#define MOE_NO_ACT_QUANT  (1u << 2) /* fidelity control: the routed experts take bf16 x and
                                       bf16 h times the decoded e4m3 weights (no activation
                                       quantisation); moe_forward only */
#define MOE_FORCE_GEMV    (1u << 8) /* run the one-row decode kernel (T <= 4; refused with
                                       MOE_E_UNSUPPORTED beyond, where its LDS plan does not
                                       fit, with MOE_SHARED_FP8 unless Is = I and
                                       top_k <= 15, and for the plain layer (neither
                                       MOE_SHARED_FP8 nor MOE_NO_ACT_QUANT) above
                                       H = 2048, which takes the expert-grouped
                                       kernels at every T) */
#define MOE_FORCE_GROUPED (1u << 9) /* run the expert-grouped path at any T */

typedef struct {
    int32_t hidden;       /* H */
    int32_t n_experts;    /* E */
    int32_t top_k;        /* K */
    int32_t inter;        /* I: routed expert intermediate */
    int32_t shared_inter; /* Is: shared expert intermediate, 0 = none */
    uint32_t flags;       /* MOE_* flags above */
} moe_config;

/* Layer weights, all device pointers, caller-owned, read-only.
 * FP8 matrices hold OCP e4m3 codes; w ~= code * scale of its 128x128 block. */
typedef struct {
    const void *router_w;     /* bf16 [E, H] */
    const float *router_bias; /* fp32 [E], added to the logits; or NULL */
    const uint8_t *w_gate;    /* e4m3 [E][I, H] */
    const float *s_gate;      /* fp32 [E][I/128, H/128] */
    const uint8_t *w_up;      /* e4m3 [E][I, H] */
    const float *s_up;        /* fp32 [E][I/128, H/128] */
    const uint8_t *w_down;    /* e4m3 [E][H, I] */
    const float *s_down;      /* fp32 [E][H/128, I/128] */
    const void *sh_gate;      /* bf16 [Is, H]; unused when Is = 0; e4m3 [Is, H]
                                 with MOE_SHARED_FP8 */
    const void *sh_up;        /* bf16 [Is, H]; e4m3 [Is, H] with MOE_SHARED_FP8 */
    const void *sh_down;      /* bf16 [H, Is]; e4m3 [H, Is] with MOE_SHARED_FP8 */
    const void *sh_gate_w;    /* bf16 [H]: shared-expert gate vector */
    const float *sh_s_gate;   /* fp32 [Is/128, H/128] with MOE_SHARED_FP8, else unused */
    const float *sh_s_up;     /* fp32 [Is/128, H/128] with MOE_SHARED_FP8, else unused */
    const float *sh_s_down;   /* fp32 [H/128, Is/128] with MOE_SHARED_FP8, else unused */
} moe_weights;

/* 1 if `device` is a gfx950 GPU this library was built for; 0 otherwise and
 * on any runtime failure, never an error (the capability convention of PR
 * #925's commit summary on the device-global marker test: a failing driver
 * call is a plain negative). */
int moe_supported(int device);

/* Bytes of device workspace moe_forward and moe_route need for up to
 * `max_rows` rows of this config; 0 if the config is refused. The library
 * allocates nothing (PR #925, commit summary of the allocation cap: device
 * and pinned bytes are bounded by the caller's budget), so the caller sizes
 * and owns this buffer. */
size_t moe_workspace_bytes(const moe_config *cfg, int32_t max_rows);

/*
 * Router (PR #939, "What it adds": the router in the backbone fatbin;
 * "Fidelity against the PyTorch oracle": decisions on bf16 logits; softmax in
 * fp32 per "How it fits the engine" > Precision).
 *   logit[t,e] = bf16(fp32(sum_h x[t,h] * router_w[e,h])) (+ router_bias[e]),
 *                the sum taken exactly (fp64 accumulation of exact products)
 *                and rounded once; MOE_LOGITS_FP32 skips the bf16 rounding;
 *   ids[t,:]   = the K experts with the largest logits, in order of logit
 *                descending, lower expert index first on equal logits;
 *   weights[t,j] = exp(logit_j - logit_0) / sum_i exp(logit_i - logit_0)
 *                over the K selected (softmax renormalised over the top K).
 * x: bf16 [T, H]; ids: int32 [T, K]; weights: fp32 [T, K];
 * logits: fp32 [T, E] (bf16 values held in fp32, bias included) or NULL, in
 * which case `workspace` (>= moe_workspace_bytes(cfg, T)) holds them.
 */
moe_status moe_route(const moe_config *cfg, const void *x, int32_t T,
                     const void *router_w, const float *router_bias,
                     int32_t *ids, float *weights, float *logits,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Dynamic 1x128 activation quantisation (PR #925, backbone commit summary;
 * PR #939, "How it fits the engine" > Precision). For each row t and each
 * group g of 128 columns:
 *   s[t,g]   = fp32(max(amax, 1e-10) / 448), amax = max |x| over the group;
 *   q[t,c]   = e4m3 code nearest fp32(x[t,c] / s[t,g]) after saturation to
 *              +-448, ties to even; a negative value that rounds to 0 gives
 *              0x80.
 * x: bf16 [T, C] with C a multiple of 128 (128 <= C <= 65536);
 * q: uint8 [T, C]; scales: fp32 [T, C/128].
 */
moe_status moe_quant_act(const void *x, int32_t T, int32_t C, uint8_t *q, float *scales,
                         void *stream);

/*
 * The fp32 -> e4m3 conversion every kernel of the library uses (the codes of
 * moe_quant_act, the re-quantised h): saturate to +-448, then round to the
 * nearest e4m3 value, ties to even; a negative value that rounds to 0 gives
 * 0x80 (PR #939, "How it fits the engine" > Precision: e4m3 with amax/448
 * scales). NaN input is outside the contract. Exposed so that the conversion
 * can be checked on every fp32 value.
 * x: fp32 [n], 16-byte aligned; q: uint8 [n], 4-byte aligned; 0 <= n <= 2^40.
 */
moe_status moe_e4m3_encode(const float *x, int64_t n, uint8_t *q, void *stream);

/*
 * The whole layer, without the residual (PR #925 commit summaries: the
 * router, the FP8 experts on FP8 rows with per-row scales, one SwiGLU launch
 * writing routed rows as FP8 and shared rows as bf16, and the combine that
 * keeps every sum in a fixed order). For each row t with routing (ids, w):
 *   (qx, sx)  = the 1x128 quantisation of x[t] (as moe_quant_act);
 *   g_j, u_j  = block-FP8 products of expert ids[t,j]'s gate and up matrices
 *               with (qx, sx), fp32 accumulation;
 *   h_j       = silu(g_j) * u_j, re-quantised 1x128 to e4m3;
 *   e_j       = block-FP8 product of the expert's down matrix with h_j;
 *   s         = Wsd . bf16(silu(Wsg x) * (Wsu x))   (bf16 shared expert);
 *   gamma     = sigmoid(sh_gate_w . x);
 *   y[t]      = bf16(sum_j w_j e_j + gamma s), the sum in slot order.
 * With MOE_SHARED_FP8, s is instead the output of the block-FP8 shared
 * matrices computed as e_j is (quantised x, requantised h, s rounded to
 * bf16); it is refused together with MOE_NO_ACT_QUANT. The one-row kernel
 * runs it as one more slot of every row when Is = I and top_k <= 15 (else
 * the expert-grouped kernels run it, and MOE_FORCE_GEMV is refused).
 * With MOE_NO_ACT_QUANT (a fidelity control, not a fast path): g_j and u_j
 * take bf16 x unquantised, h_j is rounded to bf16 instead of re-quantised,
 * and e_j takes that h; every product is with the decoded e4m3 weights times
 * their block scales.
 * Both switches take the one-row kernel at T <= 4 and the expert-grouped
 * kernels beyond, as the layer does, and a row's output bytes are the same
 * on either.
 * x: bf16 [T, H]; y: bf16 [T, H] (must not alias x);
 * workspace: >= moe_workspace_bytes(cfg, T) bytes, zero-filled once before
 * the first moe_forward call that uses it (any single repeated byte value
 * also works); from then on the library keeps it valid for that config, so
 * later calls need no clearing. The layout depends on the config (flags
 * included): before a call with another config, zero-fill it again
 * (moe_forward_noalloc does so itself). The decode path (T <= 4 by
 * default; the plain layer only up to H = 2048) keeps per-workgroup call
 * counters and epoch-tagged handoff words
 * in it between calls, so two calls that overlap in time must not share a
 * workspace; calls ordered on one stream may. The decode kernel runs one workgroup per CU and every
 * workgroup waits for values the others produce, so all of them must be
 * resident at once: the launch is refused (MOE_E_LAUNCH) on a device where
 * one of its workgroups does not fit on a CU, and concurrent work that holds
 * CUs (another decode call included) can keep some from starting. Its waits
 * are bounded: after 2^17 poll rounds a waiting workgroup gives up (a wait
 * on other workgroups after about 0.1-0.3 s, a round being one
 * device-coherent load round trip; a wait inside a workgroup, for its own
 * top-K, after about 10 ms), the output is undefined, and the workspace's
 * spin-out word is set; moe_decode_status reads (and clears) it.
 * moe_forward still returns MOE_OK, since the outcome is known only on the
 * device.
 */
moe_status moe_forward(const moe_config *cfg, const moe_weights *w, const void *x,
                       int32_t T, void *y, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * The decode path's spin-out word: copies it from `workspace` (as passed to
 * moe_forward, moe_forward_stack) into status[0] on `stream`, after the work
 * already enqueued there, and zeroes it if `clear` is nonzero. 0 means every
 * bounded wait of every decode launch since the last clear was met; nonzero
 * means one gave up and those launches' outputs are undefined. status: a
 * device uint32, 4-byte aligned. The call has no counterpart on the pages;
 * it serves their rule that a failure is observable before success is
 * reported (PR #939 "drama3: Fish Audio Drama 3 text to speech on one CUDA
 * GPU", review thread: the finding on write failures and its fix), which a
 * launch cannot honour from the host for a wait that gives up on the device.
 */
moe_status moe_decode_status(void *workspace, uint32_t *status, int32_t clear, void *stream);

/* Size of the device array moe_forward_noalloc uses as its workspace. */
#define MOE_NOALLOC_WORKSPACE_BYTES ((size_t)32 << 20)

/*
 * moe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, allocation-free serving loops, harnesses that forbid
 * hipMalloc. Same arguments, arithmetic and results as moe_forward, minus
 * the workspace: the library's own device array of
 * MOE_NOALLOC_WORKSPACE_BYTES (32 MiB) per GPU serves instead, held from the
 * library's load until the process ends. The call allocates nothing and
 * calls no allocating routine.
 * Refused with MOE_E_WORKSPACE (nothing enqueued) when
 * moe_workspace_bytes(cfg, T) exceeds that size (with H 2048, 256 experts
 * top-8 and I = Is = 512: beyond 639 rows); every other check and status is
 * moe_forward's.
 * The array starts zero-filled; a call whose config differs from the
 * previous call's on the same GPU first clears it with a kernel on `stream`.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap in time on one GPU race (whatever their
 * streams), so order them, e.g. on one stream. The decode path's error word
 * lives in the array and cannot be read by the caller.
 */
moe_status moe_forward_noalloc(const moe_config *cfg, const moe_weights *w, const void *x,
                               int32_t T, void *y, void *stream);

/*
 * A stack of n_layers layers of one shape, run on the same rows in sequence
 * (the per-frame backbone: PR #925 backbone commit summaries; each of its
 * layers holds this MoE block, and rows are RMS-normalised before each).
 * With x_0 = x:
 *   y_l     = the layer of weights layers[l] applied to x_l (as moe_forward);
 *   x_{l+1} = moe_rms_renorm(y_l, eps).
 * One decode launch per layer: every layer after the first renormalises its
 * predecessor's output in its prologue, with moe_rms_renorm's arithmetic.
 * The result equals, bit for bit, moe_forward and moe_rms_renorm called in
 * turn with the same workspace.
 * layers: HOST array of n_layers moe_weights structs, each checked as
 *   moe_forward checks its weights (shared expert present iff
 *   cfg->shared_inter > 0);
 * x: bf16 [T, H]; y: bf16 [T, H], the last layer's output (must not alias
 * x); ys: bf16 [n_layers][T, H] every layer's output, or NULL (then the
 * layers' outputs alternate between two rows of the workspace);
 * T rows of the decode path only (MOE_E_UNSUPPORTED where it does not take
 * them: beyond 4 rows on the decode-layer shape, and at any T above
 * H = 2048, where the plain layer takes the expert-grouped kernels);
 * cfg->flags may not force a
 * path or set MOE_NO_ACT_QUANT or MOE_SHARED_FP8;
 * 0 <= n_layers <= 4096; 0 <= eps <= 1; workspace as for moe_forward.
 */
moe_status moe_forward_stack(const moe_config *cfg, const moe_weights *layers, int32_t n_layers,
                             const void *x, int32_t T, float eps, void *y, void *ys,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * RMS renormalisation of rows, the step between the layers of a stack of
 * decode layers (the backbone normalises each row before its MoE layer: PR
 * #925 backbone commit summaries; here without a learned gain). Per row:
 *   ms   = fp32(sum_h y[h]^2 / H), the squares exact and summed in fp64;
 *   r    = 1 / sqrt(ms + eps), fp32 with correctly rounded sqrt and division;
 *   x[h] = bf16(fp32(y[h] * r)).
 * y, x: bf16 [T, H], H a multiple of 128 up to 8192; x may equal y (in
 * place); 0 <= eps <= 1.
 */
moe_status moe_rms_renorm(const void *y, int32_t T, int32_t H, float eps, void *x,
                          void *stream);

/*
 * Residual add, RMS norm and 1x128 activation quantisation: the step in front
 * of the layer, whose FP8 groups come out of the norm with the order and
 * rounding of the separate quantisation they replace (PR #925 "drama: load
 * the checkpoint with direct I/O in file order and build the codec on its own
 * thread", commit summaries of the Drama 3 backbone: the add-norm before the
 * MoE writes the normed rows' FP8 groups). For each row t:
 *   r[t,h]   = bf16(fp32(hidden[t,h]) + fp32(residual_in[t,h]))  -> residual_out
 *   ms       = fp32(sum_h r[t,h]^2 / H), the squares exact and summed in fp64;
 *   rs       = 1 / sqrt(ms + eps), fp32 with correctly rounded sqrt and division;
 *   x[t,h]   = bf16(fp32(fp32(r[t,h] * rs) * norm_w[h]));
 *   q, scales = moe_quant_act of x (bit for bit).
 * hidden, residual_in, residual_out, x: bf16 [T, H]; norm_w: bf16 [H];
 * q: uint8 [T, H] e4m3 codes; scales: fp32 [T, H/128]. H is a multiple of 128
 * up to 8192; 0 <= eps <= 1. residual_out may equal residual_in (in place);
 * x must not alias any other row tensor, nor residual_out hidden
 * (MOE_E_UNSUPPORTED).
 */
moe_status moe_add_rmsnorm_quant(const void *hidden, const void *residual_in,
                                 void *residual_out, const void *norm_w, int32_t T, int32_t H,
                                 float eps, void *x, uint8_t *q, float *scales, void *stream);

/*
 * One-row bf16 projection, for the backbone's other bf16 projections around
 * the layer (PR #925 "drama: load the checkpoint with direct I/O in file
 * order and build the codec on its own thread", commit summaries: the
 * backbone's bf16 GEMMs and the single-row projection that streams its
 * weights ahead of use). For t < T and n < N:
 *   y[t,n] = bf16(fp32(sum_k x[t,k] * W[n,k])),
 * the products exact and accumulated in fp64, rounded once to fp32 (the rule
 * of the router logits). W: bf16 [N, K] row-major; x: bf16 [T, K]; y: bf16
 * [T, N]. 0 <= T <= 4 (the one-row decode regime; MOE_E_SHAPE beyond);
 * 0 <= N <= 2^20; K a multiple of 128 up to 8192. W and x 16-byte aligned, y
 * 2-byte aligned; y must not alias x or W (MOE_E_UNSUPPORTED). T = 0 or
 * N = 0 is a no-op.
 */
moe_status moe_bf16_gemv(const void *W, int32_t N, int32_t K, const void *x, int32_t T, void *y,
                         void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
