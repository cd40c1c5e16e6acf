/*
 * Plain CPU oracle of the block-FP8 mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * bench's CPU-baseline leg. The product path never includes or links it, and
 * it shares nothing with the HIP library.
 *
 * What it computes, and where the pages state it (page titles abbreviated:
 * "PR #925" = "drama: load the checkpoint with direct I/O in file order and
 * build the codec on its own thread"; "PR #939" = "drama3: Fish Audio Drama 3
 * text to speech on one CUDA GPU"):
 *
 *  - The layer: 256 routed experts, top-8, block-FP8 weights, plus a gated
 *    shared expert (PR #925, commit summary of the Drama 3 backbone).
 *  - Activations are bf16; the FP8 experts quantise their inputs to e4m3 per
 *    row and per 128 inputs with scale amax / 448 (PR #939, "How it fits the
 *    engine" > Precision; PR #925, backbone commit: dynamic 1 x 128 FP8
 *    activation quantisation).
 *  - Softmax and norms in fp32 (PR #939, Precision); the router decides on
 *    bf16 logits (PR #939, "Fidelity against the PyTorch oracle", prompt-pass
 *    list, the 8th/9th-expert tie).
 *  - The SwiGLU writes routed rows as their FP8 quantisation and shared rows
 *    as bf16 (PR #925, commit summary "routed rows ... FP8 ... shared ... BF16").
 *  - The combine sums the expert outputs in a fixed order (PR #925, commit
 *    summary of drama_moe_combine).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - logit = bf16(fp32(exact sum)); the exact sum is taken as an fp64
 *    accumulation of the exact bf16 x bf16 products;
 *  - top-K order is (logit descending, expert index ascending); the K
 *    weights are a softmax over the K selected logits (renormalised top-K);
 *  - an optional router bias is added to the bf16 logit in fp32 before both
 *    selection and softmax;
 *  - an all-zero group uses amax = 1e-10 (scale 1e-10/448, codes 0);
 *  - values are saturated to +-448 before the e4m3 rounding (RNE);
 *  - the shared gate is sigmoid(x . wg); the shared expert is a bf16 SwiGLU
 *    MLP whose intermediate is rounded to bf16;
 *  - routing weights are applied in the combine:
 *    y = bf16( sum_j w_j e_j + gamma s ), summed in slot order, then the shared term.
 *
 * Accumulations are fp32 in ascending index order, as a plain loop writes
 * them; the only fp64 sum is the router logit's.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GRP 128

/* ---------------------------------------------------------------- formats */

/* OCP FP8 E4M3 ("e4m3fn"): sign bit 7, exponent bits 6..3 with bias 7,
 * mantissa bits 2..0; exponent 0 encodes subnormals m * 2^-9; S.1111.111 is
 * NaN; no infinities; largest finite value 448 (code 0x7E). The pages' scale
 * amax / 448 is this format's maximum (PR #939, Precision). */
float oracle_e4m3_decode(uint8_t code) {
    int sign = code >> 7;
    int exp = (code >> 3) & 0xF;
    int man = code & 0x7;
    double v;
    if (exp == 0xF && man == 0x7) return NAN;
    if (exp == 0)
        v = ldexp((double)man, -9);
    else
        v = ldexp(1.0 + man / 8.0, exp - 7);
    return (float)(sign ? -v : v);
}

/* The e4m3 value nearest r, ties to the even mantissa; |r| above 448
 * saturates to 448; the sign is kept, so a negative value that rounds to
 * zero gives -0 (0x80). NaN gives 0x7F. */
uint8_t oracle_e4m3_encode(float r) {
    if (isnan(r)) return 0x7F;
    uint8_t sign = signbit(r) ? 0x80 : 0x00;
    double a = fabs((double)r);
    if (a > 448.0) a = 448.0;
    /* grid spacing around a: 2^(e-3) in the binade [2^e, 2^(e+1)) for e >= -6,
     * and 2^-9 below 2^-6 (subnormals) */
    int e;
    if (a < 0x1p-6) {
        e = -6;
    } else {
        (void)frexp(a, &e);
        e -= 1;
    }
    double quantum = ldexp(1.0, e - 3);
    double n = nearbyint(a / quantum); /* exact division; round half to even */
    double v = n * quantum;
    if (v == 0.0) return sign;
    int ev;
    (void)frexp(v, &ev);
    ev -= 1;
    if (ev < -6) return (uint8_t)(sign | (int)(v / 0x1p-9));
    int man = (int)(ldexp(v, -ev) * 8.0) - 8;
    return (uint8_t)(sign | ((ev + 7) << 3) | man);
}

void oracle_e4m3_encode_n(const float *r, int64_t n, uint8_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(r[i]);
}

static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even; NaN stays NaN. */
uint16_t oracle_bf16_round(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

void oracle_bf16_round_n(const float *f, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_round(f[i]);
}

static float g_dec[256];
__attribute__((constructor)) static void build_decode_table(void) {
    for (int c = 0; c < 256; ++c) g_dec[c] = oracle_e4m3_decode((uint8_t)c);
}

/* ----------------------------------------------------------- quantisation */

/* One group of 128 values: s = fp32(max(amax, 1e-10) / 448);
 * q_i = e4m3(clamp(fp32(v_i / s), -448, 448)). */
static void quant_group(const float *v, uint8_t *q, float *s_out) {
    float amax = 0.0f;
    for (int i = 0; i < GRP; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    float s = fmaxf(amax, 1e-10f) / 448.0f;
    for (int i = 0; i < GRP; ++i) {
        float r = v[i] / s;
        if (r > 448.0f) r = 448.0f;
        if (r < -448.0f) r = -448.0f;
        q[i] = oracle_e4m3_encode(r);
    }
    *s_out = s;
}

void oracle_quant_groups(const float *v, int64_t n_groups, uint8_t *q, float *s) {
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < n_groups; ++g) quant_group(v + g * GRP, q + g * GRP, s + g);
}

void oracle_quant_act(const uint16_t *x, int64_t T, int64_t C, uint8_t *q, float *s) {
    int64_t G = C / GRP;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        float v[GRP];
        for (int64_t g = 0; g < G; ++g) {
            for (int i = 0; i < GRP; ++i) v[i] = bf16_to_f32(x[t * C + g * GRP + i]);
            quant_group(v, q + t * C + g * GRP, s + t * G + g);
        }
    }
}

/* ------------------------------------------------ stack renormalisation */

void oracle_rms_renorm(const uint16_t *y, int64_t T, int64_t H, float eps, uint16_t *x) {
    for (int64_t t = 0; t < T; ++t) {
        double sum = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            double v = (double)bf16_to_f32(y[t * H + h]);
            sum += v * v;
        }
        float ms = (float)(sum / (double)H);
        float r = 1.0f / sqrtf(ms + eps);
        for (int64_t h = 0; h < H; ++h) {
            float v = bf16_to_f32(y[t * H + h]) * r;
            x[t * H + h] = oracle_bf16_round(v);
        }
    }
}

/* ------------------------------- residual add, RMS norm and quantisation */

/* The step before the layer (PR #925 commit summaries: the add-norm before the
 * MoE also writes the normed rows' FP8 groups, with the order and rounding of
 * the quantisation launch it replaces). Row by row: the residual stream is
 * updated first and rounded to bf16; the norm reads those bf16 values; the
 * normed row is rounded to bf16; its groups are quantised exactly as
 * oracle_quant_act quantises a bf16 row. */
void oracle_add_rmsnorm_quant(const uint16_t *hidden, const uint16_t *res_in,
                              const uint16_t *norm_w, int64_t T, int64_t H, float eps,
                              uint16_t *res_out, uint16_t *x, uint8_t *q, float *s) {
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *hr = hidden + t * H, *rr = res_in + t * H;
        uint16_t *ro = res_out + t * H, *xr = x + t * H;
        for (int64_t h = 0; h < H; ++h) ro[h] = oracle_bf16_round(bf16_to_f32(hr[h]) + bf16_to_f32(rr[h]));
        double sum = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            double v = (double)bf16_to_f32(ro[h]);
            sum += v * v;
        }
        float ms = (float)(sum / (double)H);
        float r = 1.0f / sqrtf(ms + eps);
        for (int64_t h = 0; h < H; ++h) {
            float v = bf16_to_f32(ro[h]) * r;
            v = v * bf16_to_f32(norm_w[h]);
            xr[h] = oracle_bf16_round(v);
        }
        oracle_quant_act(xr, 1, H, q + t * H, s + t * (H / GRP));
    }
}

/* ----------------------------------------------------------------- router */

static void route_row(const oracle_cfg *cfg, const uint16_t *xr, const uint16_t *rw,
                      const float *bias, int32_t *ids, float *w, float *lg) {
    const int H = cfg->hidden, E = cfg->n_experts, K = cfg->top_k;
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int h = 0; h < H; ++h)
            acc += (double)bf16_to_f32(xr[h]) * (double)bf16_to_f32(rw[(int64_t)e * H + h]);
        float l = (float)acc;
        if (!(cfg->flags & ORACLE_LOGITS_FP32)) l = bf16_to_f32(oracle_bf16_round(l));
        if (bias) l = l + bias[e];
        lg[e] = l;
    }
    /* K rounds of "largest remaining logit, lowest index on ties" */
    unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
    for (int j = 0; j < K; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || lg[e] > lg[best]) best = e;
        }
        taken[best] = 1;
        ids[j] = best;
    }
    free(taken);
    /* softmax over the selected logits, renormalised over the K */
    float m = lg[ids[0]];
    float ex[64];
    float sum = 0.0f;
    for (int j = 0; j < K; ++j) {
        ex[j] = expf(lg[ids[j]] - m);
        sum += ex[j];
    }
    for (int j = 0; j < K; ++j) w[j] = ex[j] / sum;
}

void oracle_route(const oracle_cfg *cfg, const uint16_t *x, int64_t T,
                  const uint16_t *router_w, const float *router_bias,
                  int32_t *ids, float *weights, float *logits) {
    const int H = cfg->hidden, E = cfg->n_experts, K = cfg->top_k;
    float *lg_all = logits ? logits : (float *)malloc(sizeof(float) * (size_t)(T * E));
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t)
        route_row(cfg, x + t * H, router_w, router_bias, ids + t * K, weights + t * K,
                  lg_all + t * E);
    if (!logits) free(lg_all);
}

/* ---------------------------------------------------------------- experts */

static float silu(float z) { return z / (1.0f + expf(-z)); }

/* One block-scaled FP8 matrix-vector product:
 * out[n] = sum_b (sa[b] * S[n/128][b]) * sum_{k in block b} a(k) * dec(W[n][k]),
 * inner sums in ascending k, blocks in ascending b. With a quantised input
 * a(k) = dec(qa[k]); in the no-quantisation variant a(k) = va[k] and sa = 1. */
static void block_fp8_matvec(const uint8_t *W, const float *S, int N, int Kd,
                             const uint8_t *qa, const float *va, const float *sa,
                             float *out) {
    const int KB = Kd / GRP;
    for (int n = 0; n < N; ++n) {
        const uint8_t *wr = W + (int64_t)n * Kd;
        const float *sr = S + (int64_t)(n / GRP) * KB;
        float total = 0.0f;
        for (int b = 0; b < KB; ++b) {
            float p = 0.0f;
            for (int k = b * GRP; k < (b + 1) * GRP; ++k) {
                float a = qa ? g_dec[qa[k]] : va[k];
                p += a * g_dec[wr[k]];
            }
            float scale = (qa ? sa[b] : 1.0f) * sr[b];
            total += scale * p;
        }
        out[n] = total;
    }
}

/* One block-FP8 SwiGLU expert on one row: gate and up [I,H], down [H,I],
 * e4m3 codes with fp32 scales per 128x128 block; x quantised 1x128 (or not,
 * with ORACLE_NO_ACT_QUANT), h = silu(g) * u re-quantised 1x128 (or not). */
static void fp8_expert(const oracle_cfg *cfg, int I, const uint8_t *wg, const float *sg,
                       const uint8_t *wu, const float *su, const uint8_t *wd,
                       const float *sd, const uint8_t *qx, const float *sx,
                       const float *xf, float *out) {
    const int H = cfg->hidden;
    const int noq = (cfg->flags & ORACLE_NO_ACT_QUANT) != 0;
    float *g = (float *)malloc(sizeof(float) * (size_t)I);
    float *u = (float *)malloc(sizeof(float) * (size_t)I);
    float *h = (float *)malloc(sizeof(float) * (size_t)I);
    uint8_t *qh = (uint8_t *)malloc((size_t)I);
    float *sh = (float *)malloc(sizeof(float) * (size_t)(I / GRP));
    block_fp8_matvec(wg, sg, I, H, noq ? NULL : qx, xf, sx, g);
    block_fp8_matvec(wu, su, I, H, noq ? NULL : qx, xf, sx, u);
    for (int n = 0; n < I; ++n) h[n] = silu(g[n]) * u[n];
    if (!noq)
        for (int b = 0; b < I / GRP; ++b) quant_group(h + b * GRP, qh + b * GRP, sh + b);
    block_fp8_matvec(wd, sd, H, I, noq ? NULL : qh, h, sh, out);
    free(g);
    free(u);
    free(h);
    free(qh);
    free(sh);
}

/* Expert output e_j for one (row, slot) pair. */
static void expert_pair(const oracle_cfg *cfg, const oracle_weights *w, int e,
                        const uint8_t *qx, const float *sx, const float *xf, float *out) {
    const int H = cfg->hidden, I = cfg->inter;
    const int64_t gsz = (int64_t)I * H, ssz = (int64_t)(I / GRP) * (H / GRP);
    fp8_expert(cfg, I, w->w_gate + e * gsz, w->s_gate + e * ssz, w->w_up + e * gsz,
               w->s_up + e * ssz, w->w_down + e * gsz, w->s_down + e * ssz, qx, sx, xf, out);
}

/* Shared expert s = Wsd . bf16(silu(Wsg x) * (Wsu x)) and gate
 * gamma = sigmoid(wg . x), fp32 sums of exact bf16 products. With
 * ORACLE_SHARED_FP8 (a variant: the pages keep the shared expert bf16) the
 * shared matrices are block-FP8 and s is computed exactly as a routed
 * expert's output. */
static void shared_row(const oracle_cfg *cfg, const oracle_weights *w, const uint8_t *qx,
                       const float *sx, const float *xf, float *s, float *gamma) {
    const int H = cfg->hidden, Is = cfg->shared_inter;
    float z = 0.0f;
    for (int h = 0; h < H; ++h) z += xf[h] * bf16_to_f32(w->sh_gate_w[h]);
    *gamma = 1.0f / (1.0f + expf(-z));
    if (cfg->flags & ORACLE_SHARED_FP8) {
        /* the shared expert stored block-FP8 runs exactly as a routed expert
         * (same quantised x, same requantised h); gamma takes w's place */
        fp8_expert(cfg, Is, (const uint8_t *)w->sh_gate, w->sh_s_gate,
                   (const uint8_t *)w->sh_up, w->sh_s_up, (const uint8_t *)w->sh_down,
                   w->sh_s_down, qx, sx, xf, s);
        return;
    }
    float *hs = (float *)malloc(sizeof(float) * (size_t)(Is > 0 ? Is : 1));
    for (int n = 0; n < Is; ++n) {
        float gs = 0.0f, us = 0.0f;
        for (int h = 0; h < H; ++h) {
            gs += xf[h] * bf16_to_f32(w->sh_gate[(int64_t)n * H + h]);
            us += xf[h] * bf16_to_f32(w->sh_up[(int64_t)n * H + h]);
        }
        hs[n] = bf16_to_f32(oracle_bf16_round(silu(gs) * us));
    }
    for (int m = 0; m < H; ++m) {
        float acc = 0.0f;
        for (int n = 0; n < Is; ++n) acc += hs[n] * bf16_to_f32(w->sh_down[(int64_t)m * Is + n]);
        s[m] = acc;
    }
    free(hs);
}

void oracle_forward(const oracle_cfg *cfg, const oracle_weights *w,
                    const uint16_t *x, int64_t T, uint16_t *y, float *acc_out,
                    int32_t *ids_out, float *weights_out) {
    const int H = cfg->hidden, E = cfg->n_experts, K = cfg->top_k;
    const int G = H / GRP;
    if (T <= 0) return;
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T * K));
    float *rw = (float *)malloc(sizeof(float) * (size_t)(T * K));
    float *logits = (float *)malloc(sizeof(float) * (size_t)(T * E));
    float *xf = (float *)malloc(sizeof(float) * (size_t)(T * H));
    uint8_t *qx = (uint8_t *)malloc((size_t)(T * H));
    float *sx = (float *)malloc(sizeof(float) * (size_t)(T * G));
    float *ej = (float *)malloc(sizeof(float) * (size_t)(T * K) * (size_t)H);
    float *s = (float *)malloc(sizeof(float) * (size_t)(T * H));
    float *gamma = (float *)malloc(sizeof(float) * (size_t)T);

    oracle_route(cfg, x, T, w->router_w, w->router_bias, ids, rw, logits);
    for (int64_t i = 0; i < T * H; ++i) xf[i] = bf16_to_f32(x[i]);
    oracle_quant_act(x, T, H, qx, sx);

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < T * K; ++p) {
        int64_t t = p / K;
        expert_pair(cfg, w, ids[p], qx + t * H, sx + t * G, xf + t * H, ej + p * H);
    }

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        if (cfg->shared_inter > 0) {
            shared_row(cfg, w, qx + t * H, sx + t * G, xf + t * H, s + t * H, gamma + t);
        } else {
            gamma[t] = 0.0f;
            for (int m = 0; m < H; ++m) s[t * H + m] = 0.0f;
        }
        for (int m = 0; m < H; ++m) {
            float a = 0.0f;
            for (int j = 0; j < K; ++j) a += rw[t * K + j] * ej[(t * K + j) * H + m];
            if (cfg->shared_inter > 0) a += gamma[t] * s[t * H + m];
            if (acc_out) acc_out[t * H + m] = a;
            y[t * H + m] = oracle_bf16_round(a);
        }
    }
    if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)(T * K));
    if (weights_out) memcpy(weights_out, rw, sizeof(float) * (size_t)(T * K));
    free(ids);
    free(rw);
    free(logits);
    free(xf);
    free(qx);
    free(sx);
    free(ej);
    free(s);
    free(gamma);
}

void oracle_bf16_gemv(const uint16_t *W, int64_t N, int64_t K, const uint16_t *x, int64_t T,
                      uint16_t *y) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t t = 0; t < T; ++t) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += (double)bf16_to_f32(x[t * K + k]) * (double)bf16_to_f32(W[n * K + k]);
            y[t * N + n] = oracle_bf16_round((float)acc);
        }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
