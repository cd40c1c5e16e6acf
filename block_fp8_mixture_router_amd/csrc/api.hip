// C ABI of libmoe: validation, workspace layout and dispatch.
//
// Conventions follow the host code the pages describe: shapes the kernels
// cannot honour are refused at the door with a named code, before anything
// is enqueued; buffers are caller-owned and the library allocates nothing
// (PR #925 "drama: load the checkpoint with direct I/O in file order and
// build the codec on its own thread", commit summaries on refusal at open
// and on the allocation cap; PR #939 "drama3: Fish Audio Drama 3 text to
// speech on one CUDA GPU", "What it adds": config.zig refuses other shapes).
#include <atomic>
#include <cstring>

#include "../../include/moe.h"
#include "kernels.h"

namespace moe {
// csrc/gemv.hip (declared here so that the decode kernel's sources stay as
// they are)
hipError_t launch_bf16_gemv(const uint16_t *W, int N, int K, const uint16_t *x, int T,
                            uint16_t *y, hipStream_t st);
}  // namespace moe

using namespace moe;

namespace {

constexpr int MAX_DEVICES = 64;
std::atomic<int> g_dev_state[MAX_DEVICES];  // 0 unknown, 1 gfx950, 2 other

int device_is_gfx950(int dev) {
    if (dev < 0 || dev >= MAX_DEVICES) return 0;
    int s = g_dev_state[dev].load(std::memory_order_acquire);
    if (s == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return 0;
        s = (std::strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_dev_state[dev].store(s, std::memory_order_release);
    }
    return s == 1;
}

std::atomic<int> g_dev_cus[MAX_DEVICES];

// compute units of the current device (the decode kernel's grid)
int device_cus() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return 0;
    int n = g_dev_cus[dev].load(std::memory_order_acquire);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        if (n > 1024) n = 1024;
        g_dev_cus[dev].store(n, std::memory_order_release);
    }
    return n;
}

bool current_device_ok() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    return device_is_gfx950(dev) != 0;
}

bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_cfg(const moe_config *c) {
    if (!c) return MOE_E_NULL;
    const uint32_t known =
        MOE_SHARED_FP8 | MOE_LOGITS_FP32 | MOE_NO_ACT_QUANT | MOE_FORCE_GEMV | MOE_FORCE_GROUPED;
    if (c->flags & ~known) return MOE_E_UNSUPPORTED;
    if ((c->flags & MOE_FORCE_GEMV) && (c->flags & MOE_FORCE_GROUPED)) return MOE_E_UNSUPPORTED;
    // the two variants are separate switches, not combined
    if ((c->flags & MOE_SHARED_FP8) && (c->flags & MOE_NO_ACT_QUANT)) return MOE_E_UNSUPPORTED;
    if (c->hidden < 128 || c->hidden > 8192 || c->hidden % 128) return MOE_E_SHAPE;
    if (c->inter < 128 || c->inter > 4096 || c->inter % 128) return MOE_E_SHAPE;
    if (c->shared_inter < 0 || c->shared_inter > 4096 || c->shared_inter % 128) return MOE_E_SHAPE;
    if (c->n_experts < 1 || c->n_experts > 1024) return MOE_E_SHAPE;
    if (c->top_k < 1 || c->top_k > 16 || c->top_k > c->n_experts) return MOE_E_SHAPE;
    return MOE_OK;
}

constexpr int MAX_ROWS = 65536;
constexpr int MAX_STACK_LAYERS = 4096;
// above this many rows the router ranks bf16 MFMA scores with an error bound
// and computes exact logits only where the bound leaves the pick undecided
constexpr int BOUNDED_MIN_ROWS = 16;

size_t a256(size_t b) { return (b + 255) & ~(size_t)255; }

// what the one-row kernel computes for this config (the block-FP8 shared
// switch means nothing without a shared expert)
int decode_var(const moe_config *c) {
    if ((c->flags & MOE_SHARED_FP8) && c->shared_inter > 0) return DV_SFP8;
    if (c->flags & MOE_NO_ACT_QUANT) return DV_NOQ;
    return DV_PLAIN;
}

// The most rows the one-row path can take for this config (0 if none): it
// alone fixes the size of the decode handoff regions, so that no region of
// the workspace moves with T (a grouped call's plain data can never sit
// where a later decode call polls for tagged words).
int decode_rows_max(const moe_config *c) {
    // The plain layer's one-row kernel with four router chunks per lane
    // (hidden above 2048) made an illegal memory access the first time it
    // ran (hidden 8192, 64 experts, top-8, intermediate 1024, one row), and
    // no cause has been shown; such configs take the expert-grouped kernels
    // until one is.
    if (decode_var(c) == DV_PLAIN && c->hidden > 2048) return 0;
    for (int t = DECODE_MAX_ROWS; t >= 1; --t)
        if (decode_fits(t, c->hidden, c->top_k, c->inter, c->shared_inter, decode_var(c)))
            return t;
    return 0;
}

struct Layout {
    size_t sync, dlogits, dgamma, dhs, dh, ybuf, logits, absums, ids, wts, gamma, hs, qx, sx,
        offsets, perm, tiles, n_tiles, qh, sh, stage, hb, sperm, stiles, sntiles, sqh, ssh, so;
    size_t total;
    int max_tiles;
};

Layout layout_of(const moe_config *c, int T) {
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += a256(bytes);
        return o;
    };
    const size_t t = (size_t)T, E = c->n_experts, K = c->top_k, H = c->hidden, I = c->inter,
                 Is = c->shared_inter;
    L.max_tiles = grouped_max_tiles(T, (int)K, (int)E);
    L.sync = take((size_t)SYNC_WORDS * 4);
    // The decode path hands logits, gamma, hs and h between workgroups as
    // 64-bit tagged words in DECODE_REPLICAS copies (regions d*, used by it
    // alone, so no plain value can ever be read as a tag), sized for the
    // most rows it can take whatever T is; the grouped path keeps one plain
    // copy of logits (fp32), gamma (fp32) and hs (bf16) after them. Every
    // other size is non-decreasing in T, so a workspace sized for max_rows
    // serves every T <= max_rows.
    const size_t R = DECODE_REPLICAS, td = (size_t)decode_rows_max(c);
    const int var = decode_var(c);
    const size_t KS = td ? (size_t)decode_slots(var, (int)K, (int)I, (int)Is) : 0;
    L.dlogits = take(R * td * E * 8);
    L.dgamma = take(R * td * 8);
    L.dhs = take(var == DV_SFP8 ? 0 : R * td * Is * 8);
    L.dh = take(R * td * KS * I * 8);
    L.ybuf = take(2 * td * H * 2);  // a stack's layer outputs, alternating
    L.logits = take(t * E * 4);  // exact logits, or the bounded scores S
    L.absums = take(t * E * 4);  // the bounded scores' sums of |x||w|
    L.ids = take(t * K * 4);
    L.wts = take(t * K * 4);
    L.gamma = take(t * 4);
    L.hs = take(t * Is * 2);
    L.qx = take(t * H);
    L.sx = take(t * (H / 128) * 4);
    L.offsets = take((E + 1) * 4);
    L.perm = take(t * K * 4);
    L.tiles = take((size_t)L.max_tiles * 16);
    L.n_tiles = take(4);
    L.qh = take(t * K * I);
    L.sh = take(t * K * (I / 128) * 4);
    L.stage = take(t * K * H * 2);
    // bf16 h of the no-activation-quantisation control
    L.hb = take((c->flags & MOE_NO_ACT_QUANT) ? t * K * I * 2 : 0);
    // the block-FP8 shared expert as one more grouped expert over all rows:
    // its pair list and tiles, its h codes and scales
    const bool sfp8 = (c->flags & MOE_SHARED_FP8) && Is > 0;
    L.sperm = take(sfp8 ? t * 4 : 0);
    L.stiles = take(sfp8 ? (t + GROUP_ROWS - 1) / GROUP_ROWS * 16 : 0);
    L.sntiles = take(sfp8 ? 4 : 0);
    L.sqh = take(sfp8 ? t * Is : 0);
    L.ssh = take(sfp8 ? t * (Is / 128) * 4 : 0);
    // the shared expert's output s for the combine: fp32 from the bf16
    // expert, bf16 (in the first half) from the block-FP8 one
    L.so = take(Is > 0 ? t * H * 4 : 0);
    L.total = off;
    return L;
}

template <typename T>
T *at(void *ws, size_t off) {
    return reinterpret_cast<T *>(static_cast<unsigned char *>(ws) + off);
}

#define MOE_TRY(expr)                                  \
    do {                                               \
        if ((expr) != hipSuccess) return MOE_E_LAUNCH; \
    } while (0)

}  // namespace

extern "C" {

int moe_supported(int device) {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) return 0;
    return device_is_gfx950(device);
}

size_t moe_workspace_bytes(const moe_config *cfg, int32_t max_rows) {
    if (check_cfg(cfg) != MOE_OK || max_rows < 0 || max_rows > MAX_ROWS) return 0;
    return layout_of(cfg, max_rows < 1 ? 1 : max_rows).total;
}

moe_status moe_quant_act(const void *x, int32_t T, int32_t C, uint8_t *q, float *scales,
                         void *stream) {
    if (T < 0 || T > MAX_ROWS || C < 128 || C > 65536 || C % 128) return MOE_E_SHAPE;
    if (T == 0) return MOE_OK;
    if (!x || !q || !scales) return MOE_E_NULL;
    if (!al16(x) || !al16(q) || (reinterpret_cast<uintptr_t>(scales) & 3u)) return MOE_E_ALIGN;
    if (!current_device_ok()) return MOE_E_UNSUPPORTED;
    MOE_TRY(launch_quant_act(static_cast<const uint16_t *>(x), (int64_t)T * (C / 128), q, scales,
                             static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

moe_status moe_e4m3_encode(const float *x, int64_t n, uint8_t *q, void *stream) {
    if (n < 0 || n > ((int64_t)1 << 40)) return MOE_E_SHAPE;
    if (n == 0) return MOE_OK;
    if (!x || !q) return MOE_E_NULL;
    if ((reinterpret_cast<uintptr_t>(x) & 15u) || (reinterpret_cast<uintptr_t>(q) & 3u))
        return MOE_E_ALIGN;
    if (!current_device_ok()) return MOE_E_UNSUPPORTED;
    MOE_TRY(launch_e4m3_encode(x, n, q, static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

moe_status moe_decode_status(void *workspace, uint32_t *status, int32_t clear, void *stream) {
    if (!workspace || !status) return MOE_E_NULL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) ||
        (reinterpret_cast<uintptr_t>(status) & 3u))
        return MOE_E_ALIGN;
    if (!current_device_ok()) return MOE_E_UNSUPPORTED;
    // the sync region opens every layout, at offset 0
    MOE_TRY(launch_decode_status(static_cast<uint32_t *>(workspace), status, clear != 0,
                                 static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

moe_status moe_rms_renorm(const void *y, int32_t T, int32_t H, float eps, void *x,
                          void *stream) {
    if (T < 0 || T > MAX_ROWS || H < 128 || H > 8192 || H % 128) return MOE_E_SHAPE;
    if (!(eps >= 0.0f) || eps > 1.0f) return MOE_E_SHAPE;
    if (T == 0) return MOE_OK;
    if (!y || !x) return MOE_E_NULL;
    if (!al16(y) || !al16(x)) return MOE_E_ALIGN;
    if (!current_device_ok()) return MOE_E_UNSUPPORTED;
    MOE_TRY(launch_rms_renorm(static_cast<const uint16_t *>(y), T, H, eps,
                              static_cast<uint16_t *>(x), static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

moe_status moe_add_rmsnorm_quant(const void *hidden, const void *residual_in,
                                 void *residual_out, const void *norm_w, int32_t T, int32_t H,
                                 float eps, void *x, uint8_t *q, float *scales, void *stream) {
    if (T < 0 || T > MAX_ROWS || H < 128 || H > 8192 || H % 128) return MOE_E_SHAPE;
    if (!(eps >= 0.0f) || eps > 1.0f) return MOE_E_SHAPE;
    if (T == 0) return MOE_OK;
    if (!hidden || !residual_in || !residual_out || !norm_w || !x || !q || !scales)
        return MOE_E_NULL;
    const void *a16[] = {hidden, residual_in, residual_out, norm_w, x, q};
    for (const void *p : a16)
        if (!al16(p)) return MOE_E_ALIGN;
    if (reinterpret_cast<uintptr_t>(scales) & 3u) return MOE_E_ALIGN;
    if (x == hidden || x == residual_in || x == residual_out || residual_out == hidden)
        return MOE_E_UNSUPPORTED;
    if (!current_device_ok()) return MOE_E_UNSUPPORTED;
    MOE_TRY(launch_add_rmsnorm_quant(
        static_cast<const uint16_t *>(hidden), static_cast<const uint16_t *>(residual_in),
        static_cast<const uint16_t *>(norm_w), T, H, eps, static_cast<uint16_t *>(residual_out),
        static_cast<uint16_t *>(x), q, scales, static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

moe_status moe_bf16_gemv(const void *W, int32_t N, int32_t K, const void *x, int32_t T, void *y,
                         void *stream) {
    if (N < 0 || N > (1 << 20) || T < 0 || T > 4 || K < 128 || K > 8192 || K % 128)
        return MOE_E_SHAPE;
    if (N == 0 || T == 0) return MOE_OK;
    if (!W || !x || !y) return MOE_E_NULL;
    if (!al16(W) || !al16(x) || (reinterpret_cast<uintptr_t>(y) & 1u)) return MOE_E_ALIGN;
    if (y == x || y == W) return MOE_E_UNSUPPORTED;
    if (!current_device_ok()) return MOE_E_UNSUPPORTED;
    MOE_TRY(launch_bf16_gemv(static_cast<const uint16_t *>(W), N, K,
                             static_cast<const uint16_t *>(x), T, static_cast<uint16_t *>(y),
                             static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

moe_status moe_route(const moe_config *cfg, const void *x, int32_t T, const void *router_w,
                     const float *router_bias, int32_t *ids, float *weights, float *logits,
                     void *workspace, size_t workspace_bytes, void *stream) {
    moe_status s = check_cfg(cfg);
    if (s != MOE_OK) return s;
    if (T < 0 || T > MAX_ROWS) return MOE_E_SHAPE;
    if (T == 0) return MOE_OK;
    if (!x || !router_w || !ids || !weights) return MOE_E_NULL;
    if (!logits && !workspace) return MOE_E_NULL;
    if (!al16(x) || !al16(router_w) || (reinterpret_cast<uintptr_t>(ids) & 3u) ||
        (reinterpret_cast<uintptr_t>(weights) & 3u) ||
        (logits && (reinterpret_cast<uintptr_t>(logits) & 3u)) ||
        (router_bias && (reinterpret_cast<uintptr_t>(router_bias) & 3u)))
        return MOE_E_ALIGN;
    if (!logits) {
        if (reinterpret_cast<uintptr_t>(workspace) & 255u) return MOE_E_ALIGN;
        if (workspace_bytes < layout_of(cfg, T).total) return MOE_E_WORKSPACE;
    }
    if (!current_device_ok()) return MOE_E_UNSUPPORTED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    if (!logits && T > BOUNDED_MIN_ROWS) {
        const Layout L = layout_of(cfg, T);
        float *S = at<float>(workspace, L.logits), *A = at<float>(workspace, L.absums);
        MOE_TRY(launch_route_scores(xb, T, static_cast<const uint16_t *>(router_w), cfg->hidden,
                                    cfg->n_experts, S, A, st));
        MOE_TRY(launch_route_topk_bounded(S, A, T, cfg->n_experts, cfg->top_k, xb,
                                          static_cast<const uint16_t *>(router_w), router_bias,
                                          cfg->flags, cfg->hidden, ids, weights, nullptr, nullptr,
                                          nullptr, nullptr, st));
        return MOE_OK;
    }
    float *lg = logits ? logits : at<float>(workspace, layout_of(cfg, T).logits);
    MOE_TRY(launch_route_logits(xb, T, static_cast<const uint16_t *>(router_w), router_bias,
                                cfg->hidden, cfg->n_experts, cfg->flags, lg, st));
    MOE_TRY(launch_route_topk(lg, T, cfg->n_experts, cfg->top_k, ids, weights, nullptr, nullptr,
                              cfg->hidden, nullptr,
                              !router_bias && !(cfg->flags & MOE_LOGITS_FP32), nullptr, nullptr,
                              st));
    return MOE_OK;
}

namespace {
void fill_decode_args(FusedArgs &a, const moe_config *cfg, const moe_weights *w, int T,
                      void *workspace, const Layout &L) {
    a.T = T; a.H = cfg->hidden; a.E = cfg->n_experts; a.K = cfg->top_k; a.I = cfg->inter;
    a.Is = cfg->shared_inter;
    a.flags = cfg->flags;
    a.router_w = static_cast<const uint16_t *>(w->router_w);
    a.bias = w->router_bias;
    a.w_gate = w->w_gate; a.w_up = w->w_up; a.w_down = w->w_down;
    a.s_gate = w->s_gate; a.s_up = w->s_up; a.s_down = w->s_down;
    a.sh_gate = static_cast<const uint16_t *>(w->sh_gate);
    a.sh_up = static_cast<const uint16_t *>(w->sh_up);
    a.sh_down = static_cast<const uint16_t *>(w->sh_down);
    a.sh_gate_w = static_cast<const uint16_t *>(w->sh_gate_w);
    a.var = decode_var(cfg);
    a.KS = decode_slots(a.var, a.K, a.I, a.Is);
    if (a.var == DV_SFP8) {
        a.sh8_gate = static_cast<const uint8_t *>(w->sh_gate);
        a.sh8_up = static_cast<const uint8_t *>(w->sh_up);
        a.sh8_down = static_cast<const uint8_t *>(w->sh_down);
        a.sh_s_gate = w->sh_s_gate;
        a.sh_s_up = w->sh_s_up;
        a.sh_s_down = w->sh_s_down;
    }
    a.logits = at<uint64_t>(workspace, L.dlogits);
    a.gamma = at<uint64_t>(workspace, L.dgamma);
    a.hs = at<uint64_t>(workspace, L.dhs);
    a.h = at<uint64_t>(workspace, L.dh);
    a.sync = at<uint32_t>(workspace, L.sync);
    a.nwg = device_cus();
}

// the checks of moe_forward on one layer's weights
moe_status check_weights(const moe_config *cfg, const moe_weights *w) {
    if (!w->router_w || !w->w_gate || !w->s_gate || !w->w_up || !w->s_up || !w->w_down ||
        !w->s_down)
        return MOE_E_NULL;
    const bool shared = cfg->shared_inter > 0;
    if (shared && (!w->sh_gate || !w->sh_up || !w->sh_down || !w->sh_gate_w)) return MOE_E_NULL;
    const void *ptrs[] = {w->router_w, w->w_gate, w->w_up, w->w_down};
    for (const void *p : ptrs)
        if (!al16(p)) return MOE_E_ALIGN;
    const void *scalars[] = {w->s_gate, w->s_up, w->s_down, w->router_bias};
    for (const void *p : scalars)
        if (reinterpret_cast<uintptr_t>(p) & 3u) return MOE_E_ALIGN;
    if (shared && (!al16(w->sh_gate) || !al16(w->sh_up) || !al16(w->sh_down) ||
                   !al16(w->sh_gate_w)))
        return MOE_E_ALIGN;
    if (shared && (cfg->flags & MOE_SHARED_FP8)) {
        if (!w->sh_s_gate || !w->sh_s_up || !w->sh_s_down) return MOE_E_NULL;
        const void *ss[] = {w->sh_s_gate, w->sh_s_up, w->sh_s_down};
        for (const void *p : ss)
            if (reinterpret_cast<uintptr_t>(p) & 3u) return MOE_E_ALIGN;
    }
    return MOE_OK;
}
}  // namespace

}  // extern "C"

namespace moe {
// moe_forward's host-side checks, in its order; with own_workspace the
// workspace pointer and size are the library's (not checked here)
moe_status forward_checks(const moe_config *cfg, const moe_weights *w, const void *x, int32_t T,
                          const void *y, const void *workspace, size_t workspace_bytes,
                          bool own_workspace) {
    moe_status s = check_cfg(cfg);
    if (s != MOE_OK) return s;
    if (T < 0 || T > MAX_ROWS) return MOE_E_SHAPE;
    if (T == 0) return MOE_OK;
    if (!w || !x || !y || (!own_workspace && !workspace)) return MOE_E_NULL;
    if ((s = check_weights(cfg, w)) != MOE_OK) return s;
    if (!al16(x) || !al16(y)) return MOE_E_ALIGN;
    if (!own_workspace) {
        if (reinterpret_cast<uintptr_t>(workspace) & 255u) return MOE_E_ALIGN;
        if (workspace_bytes < layout_of(cfg, T).total) return MOE_E_WORKSPACE;
    }
    if (x == y) return MOE_E_UNSUPPORTED;
    if (!current_device_ok()) return MOE_E_UNSUPPORTED;
    return MOE_OK;
}
}  // namespace moe

extern "C" {

moe_status moe_forward(const moe_config *cfg, const moe_weights *w, const void *x, int32_t T,
                       void *y, void *workspace, size_t workspace_bytes, void *stream) {
    moe_status s = forward_checks(cfg, w, x, T, y, workspace, workspace_bytes, false);
    if (s != MOE_OK || T == 0) return s;
    const bool shared = cfg->shared_inter > 0;
    const bool sfp8 = shared && (cfg->flags & MOE_SHARED_FP8);
    const Layout L = layout_of(cfg, T);

    hipStream_t st = static_cast<hipStream_t>(stream);
    const int H = cfg->hidden, E = cfg->n_experts, K = cfg->top_k;
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    float *lg = at<float>(workspace, L.logits);
    int32_t *ids = at<int32_t>(workspace, L.ids);
    float *wts = at<float>(workspace, L.wts);
    float *gamma = at<float>(workspace, L.gamma);
    const bool fits = T <= decode_rows_max(cfg);
    const bool noq = (cfg->flags & MOE_NO_ACT_QUANT) != 0;
    if ((cfg->flags & MOE_FORCE_GEMV) && !fits) return MOE_E_UNSUPPORTED;
    const bool gemv =
        (cfg->flags & MOE_FORCE_GEMV) || (!(cfg->flags & MOE_FORCE_GROUPED) && fits);
    if (gemv) {
        FusedArgs a{};
        fill_decode_args(a, cfg, w, T, workspace, L);
        a.x = xb;
        a.y = static_cast<uint16_t *>(y);
        if (a.nwg <= 0 || a.nwg > SYNC_WORDS - SYNC_FLAGS) return MOE_E_UNSUPPORTED;
        MOE_TRY(launch_decode_fused(a, st));
        return MOE_OK;
    }
    GroupedArgs g{};
    g.T = T; g.H = H; g.E = E; g.K = K; g.I = cfg->inter; g.Is = cfg->shared_inter;
    g.x = xb;
    g.qx = at<uint8_t>(workspace, L.qx);
    g.sx = at<float>(workspace, L.sx);
    g.ids = ids; g.wts = wts; g.gamma = gamma;
    g.w_gate = w->w_gate; g.w_up = w->w_up; g.w_down = w->w_down;
    g.s_gate = w->s_gate; g.s_up = w->s_up; g.s_down = w->s_down;
    g.sh_gate = static_cast<const uint16_t *>(w->sh_gate);
    g.sh_up = static_cast<const uint16_t *>(w->sh_up);
    g.sh_down = static_cast<const uint16_t *>(w->sh_down);
    g.offsets = at<int32_t>(workspace, L.offsets);
    g.perm = at<int32_t>(workspace, L.perm);
    g.tiles = at<int32_t>(workspace, L.tiles);
    g.n_tiles = at<int32_t>(workspace, L.n_tiles);
    g.max_tiles = L.max_tiles;
    g.qh = at<uint8_t>(workspace, L.qh);
    g.sh = at<float>(workspace, L.sh);
    g.hs = at<uint16_t>(workspace, L.hs);
    g.stage = at<uint16_t>(workspace, L.stage);
    g.hb = noq ? at<uint16_t>(workspace, L.hb) : nullptr;
    g.ss = (shared && !sfp8) ? at<float>(workspace, L.so) : nullptr;
    g.y = static_cast<uint16_t *>(y);
    const uint16_t *rw = static_cast<const uint16_t *>(w->router_w);
    const uint16_t *gw = shared ? static_cast<const uint16_t *>(w->sh_gate_w) : nullptr;
    if (T > BOUNDED_MIN_ROWS) {
        float *A = at<float>(workspace, L.absums);
        MOE_TRY(launch_route_scores(xb, T, rw, H, E, lg, A, st));
        MOE_TRY(launch_route_topk_bounded(lg, A, T, E, K, xb, rw, w->router_bias, cfg->flags, H,
                                          ids, wts, gw, gamma, at<uint8_t>(workspace, L.qx),
                                          at<float>(workspace, L.sx), st));
    } else {
        MOE_TRY(launch_route_logits(xb, T, rw, w->router_bias, H, E, cfg->flags, lg, st));
        MOE_TRY(launch_route_topk(lg, T, E, K, ids, wts, xb, gw, H, gamma,
                                  !w->router_bias && !(cfg->flags & MOE_LOGITS_FP32),
                                  at<uint8_t>(workspace, L.qx), at<float>(workspace, L.sx), st));
    }
    MOE_TRY(launch_group_sort(g, st));
    // the routed products (with the bf16 shared expert's gate/up tiles in
    // the same launch, unless the shared expert is block-FP8)
    GroupedArgs gr = g;
    if (sfp8) gr.Is = 0;
    if (noq) {
        // the bf16 shared expert's tiles alone (the launches hold no routed
        // tiles when max_tiles is 0) around the control's routed products
        GroupedArgs gs = gr;
        gs.max_tiles = 0;
        MOE_TRY(launch_expert_gateup(gs, st));
        MOE_TRY(launch_grouped_noq(gr, st));
        MOE_TRY(launch_grouped_down(gs, st));
    } else {
        MOE_TRY(launch_expert_gateup(gr, st));
        MOE_TRY(launch_grouped_down(gr, st));
    }
    if (sfp8) {
        // the block-FP8 shared expert: one expert holding every row (K = 1),
        // through the routed kernels, its output staged in es
        GroupedArgs gs = gr;
        gs.K = 1;
        gs.E = 1;
        gs.I = cfg->shared_inter;
        gs.w_gate = static_cast<const uint8_t *>(w->sh_gate);
        gs.w_up = static_cast<const uint8_t *>(w->sh_up);
        gs.w_down = static_cast<const uint8_t *>(w->sh_down);
        gs.s_gate = w->sh_s_gate;
        gs.s_up = w->sh_s_up;
        gs.s_down = w->sh_s_down;
        gs.perm = at<int32_t>(workspace, L.sperm);
        gs.tiles = at<int32_t>(workspace, L.stiles);
        gs.n_tiles = at<int32_t>(workspace, L.sntiles);
        gs.max_tiles = (T + GROUP_ROWS - 1) / GROUP_ROWS;
        gs.qh = at<uint8_t>(workspace, L.sqh);
        gs.sh = at<float>(workspace, L.ssh);
        gs.stage = at<uint16_t>(workspace, L.so);
        MOE_TRY(launch_shared_tiles(T, gs.perm, gs.tiles, gs.n_tiles, st));
        MOE_TRY(launch_expert_gateup(gs, st));
        MOE_TRY(launch_grouped_down(gs, st));
        gr.es = gs.stage;
    }
    MOE_TRY(launch_combine(gr, st));
    return MOE_OK;
}

moe_status moe_forward_stack(const moe_config *cfg, const moe_weights *layers, int32_t n_layers,
                             const void *x, int32_t T, float eps, void *y, void *ys,
                             void *workspace, size_t workspace_bytes, void *stream) {
    moe_status s = check_cfg(cfg);
    if (s != MOE_OK) return s;
    if (cfg->flags & (MOE_FORCE_GEMV | MOE_FORCE_GROUPED | MOE_NO_ACT_QUANT | MOE_SHARED_FP8))
        return MOE_E_UNSUPPORTED;
    if (T < 0 || T > MAX_ROWS || n_layers < 0 || n_layers > MAX_STACK_LAYERS) return MOE_E_SHAPE;
    if (!(eps >= 0.0f) || eps > 1.0f) return MOE_E_SHAPE;
    if (T == 0 || n_layers == 0) return MOE_OK;
    if (!layers || !x || !y || !workspace) return MOE_E_NULL;
    for (int l = 0; l < n_layers; ++l)
        if ((s = check_weights(cfg, &layers[l])) != MOE_OK) return s;
    if (!al16(x) || !al16(y) || (ys && !al16(ys))) return MOE_E_ALIGN;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return MOE_E_ALIGN;
    const Layout L = layout_of(cfg, T);
    if (workspace_bytes < L.total) return MOE_E_WORKSPACE;
    if (x == y) return MOE_E_UNSUPPORTED;
    if (T > decode_rows_max(cfg)) return MOE_E_UNSUPPORTED;
    if (!current_device_ok()) return MOE_E_UNSUPPORTED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t row_elems = (size_t)T * cfg->hidden;
    uint16_t *ybuf = at<uint16_t>(workspace, L.ybuf);
    uint16_t *ysb = static_cast<uint16_t *>(ys);
    const uint16_t *prev = nullptr;
    for (int l = 0; l < n_layers; ++l) {
        FusedArgs a{};
        fill_decode_args(a, cfg, &layers[l], T, workspace, L);
        if (a.nwg <= 0 || a.nwg > SYNC_WORDS - SYNC_FLAGS) return MOE_E_UNSUPPORTED;
        // layer l > 0 renormalises the output of layer l - 1 in its prologue
        if (l == 0) a.x = static_cast<const uint16_t *>(x);
        else {
            a.y_prev = prev;
            a.eps = eps;
        }
        uint16_t *out = ysb ? ysb + (size_t)l * row_elems : ybuf + (size_t)(l & 1) * row_elems;
        if (l == n_layers - 1) {
            a.y = static_cast<uint16_t *>(y);
            a.y2 = ysb ? out : nullptr;
        } else {
            a.y = out;
        }
        MOE_TRY(launch_decode_fused(a, st));
        prev = out;
    }
    return MOE_OK;
}

}  // extern "C"
