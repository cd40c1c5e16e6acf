/*
 * Plain CPU oracle of the block-FP8 mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path includes, links or
 * calls this; only the tests, the smoke check and the bench's CPU-baseline
 * leg do. It shares no code, header, table or constant with the HIP library.
 *
 * All pointers are host pointers. Arrays are row-major and dense.
 * bf16 values are passed as their 16-bit patterns (uint16_t).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Variant switches of the oracle. */
#define ORACLE_NO_ACT_QUANT  (1u << 0) /* skip both activation quantisations */
#define ORACLE_LOGITS_FP32   (1u << 1) /* keep router logits in fp32 (no bf16 rounding) */
#define ORACLE_SHARED_FP8    (1u << 2) /* shared expert stored block-FP8, run as the routed experts */

typedef struct {
    int32_t hidden;       /* H */
    int32_t n_experts;    /* E */
    int32_t top_k;        /* K */
    int32_t inter;        /* I, routed expert intermediate */
    int32_t shared_inter; /* Is, 0 = no shared expert */
    uint32_t flags;       /* ORACLE_* */
} oracle_cfg;

typedef struct {
    const uint16_t *router_w;    /* bf16 [E,H] */
    const float *router_bias;    /* fp32 [E] or NULL */
    const uint8_t *w_gate;       /* e4m3 [E][I,H] */
    const float *s_gate;         /* fp32 [E][I/128,H/128] */
    const uint8_t *w_up;         /* e4m3 [E][I,H] */
    const float *s_up;           /* fp32 [E][I/128,H/128] */
    const uint8_t *w_down;       /* e4m3 [E][H,I] */
    const float *s_down;         /* fp32 [E][H/128,I/128] */
    const uint16_t *sh_gate;     /* bf16 [Is,H]; e4m3 bytes with ORACLE_SHARED_FP8 */
    const uint16_t *sh_up;       /* bf16 [Is,H]; e4m3 bytes with ORACLE_SHARED_FP8 */
    const uint16_t *sh_down;     /* bf16 [H,Is]; e4m3 bytes with ORACLE_SHARED_FP8 */
    const uint16_t *sh_gate_w;   /* bf16 [H] */
    const float *sh_s_gate;      /* fp32 [Is/128,H/128], ORACLE_SHARED_FP8 only */
    const float *sh_s_up;        /* fp32 [Is/128,H/128], ORACLE_SHARED_FP8 only */
    const float *sh_s_down;      /* fp32 [H/128,Is/128], ORACLE_SHARED_FP8 only */
} oracle_weights;

float oracle_e4m3_decode(uint8_t code);
uint8_t oracle_e4m3_encode(float r);
void oracle_e4m3_encode_n(const float *r, int64_t n, uint8_t *out);
uint16_t oracle_bf16_round(float f);
void oracle_bf16_round_n(const float *f, int64_t n, uint16_t *out);

void oracle_quant_groups(const float *v, int64_t n_groups, uint8_t *q, float *s);
void oracle_quant_act(const uint16_t *x, int64_t T, int64_t C, uint8_t *q, float *s);

void oracle_route(const oracle_cfg *cfg, const uint16_t *x, int64_t T,
                  const uint16_t *router_w, const float *router_bias,
                  int32_t *ids, float *weights, float *logits);

/* Whole layer. y: bf16 [T,H]; acc (optional): the fp32 value before the
 * final bf16 rounding; ids/weights (optional): the routing it used. */
void oracle_forward(const oracle_cfg *cfg, const oracle_weights *w,
                    const uint16_t *x, int64_t T, uint16_t *y, float *acc,
                    int32_t *ids, float *weights);

/* RMS renormalisation between the layers of a decode stack (the backbone's
 * rows are normalised before each MoE layer; the stack workload keeps only
 * that step, with no learned gain):
 *   ms = fp32(sum_h y[h]^2 / H), the sum of exact squares taken in fp64;
 *   r  = 1 / sqrt(ms + eps) in fp32 (correctly rounded sqrt and division);
 *   x[h] = bf16(fp32(y[h] * r)).
 * y, x: bf16 [T, H]; x may equal y. */
void oracle_rms_renorm(const uint16_t *y, int64_t T, int64_t H, float eps, uint16_t *x);

/* Residual add, RMS norm and 1x128 quantisation, the step before the layer:
 *   r[h]  = bf16(fp32(hidden[h]) + fp32(res_in[h]))     (res_out, new stream);
 *   ms    = fp32(sum_h r[h]^2 / H), the sum of exact squares taken in fp64;
 *   rs    = 1 / sqrt(ms + eps) in fp32;
 *   x[h]  = bf16(fp32(fp32(r[h] * rs) * norm_w[h]));
 *   (q, s) = oracle_quant_act of x.
 * hidden, res_in, res_out, x: bf16 [T, H]; norm_w: bf16 [H]; q: [T, H];
 * s: fp32 [T, H/128]; H a multiple of 128. */
void oracle_add_rmsnorm_quant(const uint16_t *hidden, const uint16_t *res_in,
                              const uint16_t *norm_w, int64_t T, int64_t H, float eps,
                              uint16_t *res_out, uint16_t *x, uint8_t *q, float *s);

/* One-row bf16 projection, the backbone's other bf16 projections (PR #925
 * "drama: load the checkpoint with direct I/O in file order and build the
 * codec on its own thread", commit summaries: the backbone's bf16 GEMMs and
 * the single-row projection that streams its weights):
 *   y[t,n] = bf16(fp32(sum_k x[t,k] * W[n,k])),
 * the sum of exact bf16 products taken in fp64 in ascending k and rounded
 * once to fp32 (the router logits' rule). W: bf16 [N, K] row-major;
 * x: bf16 [T, K]; y: bf16 [T, N]. */
void oracle_bf16_gemv(const uint16_t *W, int64_t N, int64_t K, const uint16_t *x, int64_t T,
                      uint16_t *y);

/* Threads the OpenMP runtime will use (for the baseline record). */
int oracle_num_threads(void);
/* sets the worker threads of later calls (n >= 1); no effect without OpenMP */
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
