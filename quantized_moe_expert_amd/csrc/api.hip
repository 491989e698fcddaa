// C ABI of libmoe_q4: argument checks, workspace layout and launch order.
#include "../../include/moe_q4.h"
#include "moe_internal.h"
#include "shared_dev.h"

#include <mutex>

using namespace moeq4;

// Workspace of moe_q4_forward_noalloc: device memory that the library holds
// for the life of the process, one copy of this array per GPU.  Host code
// never uses the array's name as an address (on the host it is a stand-in
// for the symbol); it uses the device address hipGetSymbolAddress returns
// for the current device (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[MOE_Q4_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t ALIGN = 256;

inline size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

// Workspace carving: regions are appended in a fixed order, each 256-byte
// aligned.  With base == nullptr only the size is computed.
struct Carver {
    char *base;
    size_t used = 0;
    template <typename T>
    T *take(size_t count) {
        T *p = base ? reinterpret_cast<T *>(base + used) : nullptr;
        used += align_up(count * sizeof(T));
        return p;
    }
};

bool pow2_between(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

int check_route_shape(int64_t T, int H, int E, int k) {
    if (T < 0 || E < 1 || k < 1 || k > E) return MOE_Q4_ERR_INVALID_ARG;
    if (E > 1024 || k > 32 || T * (int64_t)k >= (int64_t)1 << 31) return MOE_Q4_ERR_UNSUPPORTED;
    if (H < 0) return MOE_Q4_ERR_INVALID_ARG;
    return MOE_Q4_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// The prefill kernels address activations and weights with 32-bit offsets.
bool prefill_fits(int64_t T, int k, int H, int I) {
    return T * (int64_t)H < ((int64_t)1 << 31) && T * (int64_t)k * I < ((int64_t)1 << 31) &&
           T * (int64_t)k * H < ((int64_t)1 << 31);
}

int check_layer(const moe_q4_layer *w, bool prefill) {
    if (!w || !w->gate_q || !w->up_q || !w->down_q || !w->gate_sm || !w->up_sm || !w->down_sm)
        return MOE_Q4_ERR_INVALID_ARG;
    if (!aligned(w->gate_q, 16) || !aligned(w->up_q, 16) || !aligned(w->down_q, 16) || !aligned(w->gate_sm, 4) ||
        !aligned(w->up_sm, 4) || !aligned(w->down_sm, 4))
        return MOE_Q4_ERR_INVALID_ARG;
    if (w->num_experts < 1 || w->hidden < 1 || w->inter < 1) return MOE_Q4_ERR_INVALID_ARG;
    if (w->format != MOE_Q4_ASYM_G64 && w->format != MOE_Q4_SYM_G128 && w->format != MOE_Q4_FP8_B128 &&
        w->format != MOE_Q4_NVFP4)
        return MOE_Q4_ERR_UNSUPPORTED;
    if (w->format == MOE_Q4_NVFP4 && (!w->global_scale || !aligned(w->global_scale, 4)))
        return MOE_Q4_ERR_INVALID_ARG;
    const int G = w->format == MOE_Q4_ASYM_G64 ? 64 : w->format == MOE_Q4_NVFP4 ? 16 : 128;
    if (w->num_experts > 1024) return MOE_Q4_ERR_UNSUPPORTED;
    if (!pow2_between(w->hidden, 64, 2048) || !pow2_between(w->inter, 64, 2048)) return MOE_Q4_ERR_UNSUPPORTED;
    if (w->hidden % G || w->inter % G) return MOE_Q4_ERR_UNSUPPORTED;
    if (prefill && (w->inter % 128 || w->hidden % 256)) return MOE_Q4_ERR_UNSUPPORTED;
    if (!aligned(w->prefill_pack, 256)) return MOE_Q4_ERR_INVALID_ARG;
    return MOE_Q4_OK;
}

LayerPtrs layer_ptrs(const moe_q4_layer *w) {
    LayerPtrs L;
    L.E = w->num_experts;
    L.H = w->hidden;
    L.I = w->inter;
    L.fmt = w->format;
    L.gq = w->gate_q;
    L.uq = w->up_q;
    L.dq = w->down_q;
    L.gsm = w->gate_sm;
    L.usm = w->up_sm;
    L.dsm = w->down_sm;
    L.glob = w->format == MOE_Q4_NVFP4 ? w->global_scale : nullptr;
    L.pack = static_cast<const uint8_t *>(w->prefill_pack);
    return L;
}

// Grouping regions (shared by group, decode and prefill).
GroupOut carve_group(Carver &c, int64_t T, int E, int k, int rows_per_tile, bool schedule = false) {
    const int64_t P = T * k;
    const int64_t nch = (P + GROUP_CHUNK - 1) / GROUP_CHUNK;
    GroupOut g;
    g.cnt = c.take<int32_t>(E);
    g.off = c.take<int32_t>(E + 1);
    g.perm = c.take<int32_t>(P);
    g.inv = c.take<int32_t>(P);
    g.tiles = c.take<Tile>(max_tiles(P, E, rows_per_tile));
    g.ntiles = c.take<int32_t>(1);
    g.rows_per_tile = rows_per_tile;
    const bool multi = P > GROUP_SINGLE_MAX;
    g.chunk_cnt = c.take<int32_t>(multi ? nch * E : 0);
    g.chunk_base = c.take<int32_t>(multi ? nch * E : 0);
    g.order = schedule ? c.take<int32_t>(max_tiles(P, E, rows_per_tile)) : nullptr;
    g.order2 = schedule ? c.take<int32_t>(max_tiles(P, E, rows_per_tile)) : nullptr;
    return g;
}

struct DecodeWs {
    GroupOut g;
    float *h;  // SwiGLU output per sorted row, fp32 [T*k][I]
};
DecodeWs carve_decode(Carver &c, int64_t T, int E, int k, int H, int I) {
    (void)H;
    DecodeWs d;
    d.g = carve_group(c, T, E, k, DECODE_TT);
    d.h = c.take<float>(T * k * (int64_t)I);
    return d;
}

// moe_q4_forward: a control block (zeroed by moe_q4_workspace_init) followed by
// the decode or prefill regions.
constexpr size_t CONTROL_BYTES = ROUTE_CONTROL_BYTES;
bool forward_uses_decode(int64_t T, int k) { return T <= 64 && T * k <= GROUP_SINGLE_MAX; }
// One-launch routing also needs the T x E logits to fit the last workgroup's LDS.
bool forward_fused_route(int64_t T, int E) { return T * E <= ROUTE_LDS_LOGITS; }

struct PrefillWs {
    GroupOut g;
    uint16_t *x16;   // x as f16 after the per-row power-of-two scale [T][H]
    int32_t *xexp;   // that scale's exponent per token
    uint16_t *h;     // SwiGLU output per sorted row, f16 [T*k][I] (scaled per 128-column block)
    uint16_t *z;     // gate-weighted down output per sorted row, f16 [T*k][H] (scaled per 128 columns)
    int8_t *hx;      // h's power-of-two exponents [T*k][I/128]
    int8_t *zx;      // z's [T*k][H/64]
};
PrefillWs carve_prefill(Carver &c, int64_t T, int E, int k, int H, int I) {
    PrefillWs p;
    p.g = carve_group(c, T, E, k, PREFILL_BM, true);
    p.x16 = c.take<uint16_t>(T * (int64_t)H);
    p.xexp = c.take<int32_t>(T);
    p.h = c.take<uint16_t>(T * k * (int64_t)I);
    p.z = c.take<uint16_t>(T * k * (int64_t)H);
    p.hx = c.take<int8_t>(T * k * (int64_t)(I / 128 > 0 ? I / 128 : 1));
    p.zx = c.take<int8_t>(T * k * (int64_t)(H / 64 > 0 ? H / 64 : 1));
    return p;
}

int check_shared(const moe_q4_shared_expert *sx) {
    if (!sx || !sx->gate_q || !sx->up_q || !sx->down_q || !sx->gate_s || !sx->up_s || !sx->down_s)
        return MOE_Q4_ERR_INVALID_ARG;
    if (!aligned(sx->gate_q, 16) || !aligned(sx->up_q, 16) || !aligned(sx->down_q, 16) || !aligned(sx->gate_s, 2) ||
        !aligned(sx->up_s, 2) || !aligned(sx->down_s, 2))
        return MOE_Q4_ERR_INVALID_ARG;
    if (sx->hidden < 1 || sx->inter < 1) return MOE_Q4_ERR_INVALID_ARG;
    if (!pow2_between(sx->hidden, 128, 2048) || !pow2_between(sx->inter, 128, 2048)) return MOE_Q4_ERR_UNSUPPORTED;
    return MOE_Q4_OK;
}

// Shared expert workspace: h, plus the GEMM path's f16 activations and
// exponents when it runs.
bool shared_uses_gemm(int64_t T, int H) { return T >= SHARED_GEMM_MIN_T && H % 256 == 0; }
struct SharedWs {
    float *h;  // fp32 [T][I] (GEMV path); the GEMM path keeps f16 h in its first half
    uint16_t *x16;
    int32_t *xexp;
    int8_t *hx;  // GEMM path: h's exponents [T][I / 128]
};
SharedWs carve_shared(Carver &c, int64_t T, int H, int I) {
    SharedWs w;
    w.h = c.take<float>(T * (int64_t)I);
    const bool gemm = shared_uses_gemm(T, H);
    w.x16 = c.take<uint16_t>(gemm ? T * (int64_t)H : 0);
    w.xexp = c.take<int32_t>(gemm ? T : 0);
    w.hx = c.take<int8_t>(gemm ? T * (int64_t)(I / 128) : 0);
    return w;
}
hipError_t launch_shared_any(const uint16_t *x, int64_t T, const SharedPtrs &S, const SharedWs &w, float *y,
                             bool accumulate, hipStream_t s, hipEvent_t const *ev) {
    hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr, e2 = ev ? ev[2] : nullptr,
               e3 = ev ? ev[3] : nullptr;
    if (shared_uses_gemm(T, S.H))
        return launch_shared_gemm(x, T, S, w.x16, w.xexp, reinterpret_cast<uint16_t *>(w.h), w.hx, y, accumulate, s,
                                  e0, e1, e2, e3);
    return launch_shared(x, T, S, w.h, y, accumulate, s, e0, e1, e2, e3);
}

SharedPtrs shared_ptrs(const moe_q4_shared_expert *sx) {
    SharedPtrs S;
    S.H = sx->hidden;
    S.I = sx->inter;
    S.gq = sx->gate_q;
    S.uq = sx->up_q;
    S.dq = sx->down_q;
    S.gs = sx->gate_s;
    S.us = sx->up_s;
    S.ds = sx->down_s;
    return S;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_Q4_OK : MOE_Q4_ERR_HIP; }

}  // namespace

extern "C" {

size_t moe_q4_workspace_size(int which, int64_t T, int32_t E, int32_t k, int32_t H, int32_t I) {
    if (T <= 0 || E < 1 || k < 1 || H < 1 || I < 1) return 0;
    Carver c{nullptr};
    switch (which) {
        case MOE_Q4_WS_ROUTE: return 0;
        case MOE_Q4_WS_GROUP: carve_group(c, T, E, k, DECODE_TT); break;
        case MOE_Q4_WS_DECODE: carve_decode(c, T, E, k, H, I); break;
        case MOE_Q4_WS_PREFILL: carve_prefill(c, T, E, k, H, I); break;
        case MOE_Q4_WS_FORWARD:
        case MOE_Q4_WS_FORWARD_DET:
            c.take<char>(CONTROL_BYTES);
            c.take<unsigned int>(T * (int64_t)E);  // logit hand-off of the one-launch routing
            if (forward_uses_decode(T, k)) {
                carve_decode(c, T, E, k, H, I);
                if (which == MOE_Q4_WS_FORWARD_DET) c.take<float>(T * k * (int64_t)H);  // routed rows
            } else {
                carve_prefill(c, T, E, k, H, I);
            }
            break;
        case MOE_Q4_WS_SHARED: carve_shared(c, T, H, I); break;
        default: return 0;
    }
    return c.used;
}

int moe_q4_route(const void *x, const void *router_w, const float *bias, void *logits, int64_t T, int32_t H,
                 int32_t E, int32_t k, int32_t *topk_idx, float *topk_gate, void *ws, size_t ws_bytes,
                 moe_q4_stream stream) {
    (void)ws;
    (void)ws_bytes;
    int st = check_route_shape(T, x ? H : 0, E, k);
    if (st) return st;
    if (!logits || !topk_idx || !topk_gate) return MOE_Q4_ERR_INVALID_ARG;
    if (x && !router_w) return MOE_Q4_ERR_INVALID_ARG;
    if (x && (H < 8 || H % 8 || H > 2048)) return H < 1 ? MOE_Q4_ERR_INVALID_ARG : MOE_Q4_ERR_UNSUPPORTED;
    if (T == 0) return MOE_Q4_OK;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (x) {
        st = hip_status(launch_router_logits(static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(router_w),
                                             bias, T, H, E, static_cast<uint16_t *>(logits), s));
        if (st) return st;
    }
    return hip_status(launch_topk(static_cast<const uint16_t *>(logits), T, E, k, topk_idx, topk_gate, s));
}

int moe_q4_group(const int32_t *topk_idx, int64_t T, int32_t k, int32_t E, int32_t *cnt, int32_t *off,
                 int32_t *perm, int32_t *inv, void *ws, size_t ws_bytes, moe_q4_stream stream) {
    int st = check_route_shape(T, 0, E, k);
    if (st) return st;
    if (!topk_idx || !cnt || !off || !perm || !inv) return MOE_Q4_ERR_INVALID_ARG;
    if (T == 0) return MOE_Q4_OK;
    const size_t need = moe_q4_workspace_size(MOE_Q4_WS_GROUP, T, E, k, 64, 64);
    if (!ws || ws_bytes < need) return MOE_Q4_ERR_WORKSPACE;
    Carver c{static_cast<char *>(ws)};
    GroupOut g = carve_group(c, T, E, k, DECODE_TT);
    g.cnt = cnt;
    g.off = off;
    g.perm = perm;
    g.inv = inv;
    return hip_status(launch_group(topk_idx, T, k, E, g, reinterpret_cast<hipStream_t>(stream)));
}

static int run_experts(bool prefill, const void *x, const int32_t *topk_idx, const float *topk_gate, int64_t T,
                       int32_t k, const moe_q4_layer *w, float *y, void *ws, size_t ws_bytes,
                       moe_q4_stream stream, void *const *events) {
    int st = check_layer(w, prefill);
    if (st) return st;
    st = check_route_shape(T, w->hidden, w->num_experts, k);
    if (st) return st;
    if (!x || !topk_idx || !topk_gate || !y) return MOE_Q4_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(y, 16)) return MOE_Q4_ERR_INVALID_ARG;
    if (prefill && !prefill_fits(T, k, w->hidden, w->inter)) return MOE_Q4_ERR_UNSUPPORTED;
    if (events)
        for (int i = 0; i < MOE_Q4_STAGE_EVENTS; ++i)
            if (!events[i]) return MOE_Q4_ERR_INVALID_ARG;
    if (T == 0) return MOE_Q4_OK;
    const int E = w->num_experts, H = w->hidden, I = w->inter;
    const size_t need = moe_q4_workspace_size(prefill ? MOE_Q4_WS_PREFILL : MOE_Q4_WS_DECODE, T, E, k, H, I);
    if (!ws || ws_bytes < need) return MOE_Q4_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const LayerPtrs L = layer_ptrs(w);
    Carver c{static_cast<char *>(ws)};
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    hipEvent_t const *ev = reinterpret_cast<hipEvent_t const *>(events);
    if (!prefill) {
        DecodeWs d = carve_decode(c, T, E, k, H, I);
        if (T * k <= GROUP_SINGLE_MAX) {
            st = hip_status(launch_group(topk_idx, T, k, E, d.g, s, y, T * (int64_t)H, ev ? ev[2] : nullptr,
                                         ev ? ev[3] : nullptr));
        } else {
            st = hip_status(launch_group(topk_idx, T, k, E, d.g, s, nullptr, 0, ev ? ev[2] : nullptr,
                                         ev ? ev[3] : nullptr));
            if (!st) st = hip_status(launch_fill_zero(y, T * (int64_t)H, s));
        }
        if (st) return st;
        return hip_status(launch_decode_experts(xb, topk_gate, T, k, L, d.g, d.h, y, s, ev ? ev[0] : nullptr,
                                                ev ? ev[1] : nullptr));
    }
    PrefillWs p = carve_prefill(c, T, E, k, H, I);
    st = hip_status(launch_group(topk_idx, T, k, E, p.g, s));
    if (st) return st;
    return hip_status(launch_prefill_experts(xb, topk_gate, T, k, L, p.g, p.x16, p.xexp, p.h, p.z, p.hx, p.zx, y, s, ev));
}

int moe_q4_decode(const void *x, const int32_t *topk_idx, const float *topk_gate, int64_t T, int32_t k,
                  const moe_q4_layer *w, float *y, void *ws, size_t ws_bytes, moe_q4_stream stream) {
    return run_experts(false, x, topk_idx, topk_gate, T, k, w, y, ws, ws_bytes, stream, nullptr);
}

int moe_q4_decode_timed(const void *x, const int32_t *topk_idx, const float *topk_gate, int64_t T, int32_t k,
                        const moe_q4_layer *w, float *y, void *ws, size_t ws_bytes, moe_q4_stream stream,
                        void *const *events) {
    if (!events) return MOE_Q4_ERR_INVALID_ARG;
    return run_experts(false, x, topk_idx, topk_gate, T, k, w, y, ws, ws_bytes, stream, events);
}

int moe_q4_prefill(const void *x, const int32_t *topk_idx, const float *topk_gate, int64_t T, int32_t k,
                   const moe_q4_layer *w, float *y, void *ws, size_t ws_bytes, moe_q4_stream stream) {
    return run_experts(true, x, topk_idx, topk_gate, T, k, w, y, ws, ws_bytes, stream, nullptr);
}

int moe_q4_prefill_timed(const void *x, const int32_t *topk_idx, const float *topk_gate, int64_t T, int32_t k,
                         const moe_q4_layer *w, float *y, void *ws, size_t ws_bytes, moe_q4_stream stream,
                         void *const *events) {
    if (!events) return MOE_Q4_ERR_INVALID_ARG;
    return run_experts(true, x, topk_idx, topk_gate, T, k, w, y, ws, ws_bytes, stream, events);
}

int moe_q4_workspace_init(void *ws, size_t ws_bytes, moe_q4_stream stream) {
    if (!ws || ws_bytes < CONTROL_BYTES) return MOE_Q4_ERR_WORKSPACE;
    return hip_status(launch_fill_zero_u32(static_cast<uint32_t *>(ws), CONTROL_BYTES / 4,
                                           reinterpret_cast<hipStream_t>(stream)));
}

// Every argument check of the layer forward, before anything is launched
// (T = 0 passes with no further checks).
static int forward_checks(const void *x, const float *residual_y, void *x_out, const void *logits, int64_t T,
                          int32_t k, const moe_q4_layer *w, const moe_q4_shared_expert *sx, const int32_t *topk_idx,
                          const float *topk_gate, const float *y, void *const *events) {
    int st = check_layer(w, false);
    if (st) return st;
    if (sx) {
        st = check_shared(sx);
        if (st) return st;
        if (sx->hidden != w->hidden) return MOE_Q4_ERR_INVALID_ARG;
        if (T * (int64_t)sx->inter >= ((int64_t)1 << 31)) return MOE_Q4_ERR_UNSUPPORTED;
    }
    st = check_route_shape(T, w->hidden, w->num_experts, k);
    if (st) return st;
    if (!x || !logits || !topk_idx || !topk_gate || !y) return MOE_Q4_ERR_INVALID_ARG;
    if (residual_y && !x_out) return MOE_Q4_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(x_out, 16) || !aligned(residual_y, 16))
        return MOE_Q4_ERR_INVALID_ARG;
    if (events)
        for (int i = 0; i < MOE_Q4_STAGE_EVENTS; ++i)
            if (!events[i]) return MOE_Q4_ERR_INVALID_ARG;
    if (T == 0) return MOE_Q4_OK;
    if (!forward_uses_decode(T, k) && (check_layer(w, true) || !prefill_fits(T, k, w->hidden, w->inter)))
        return MOE_Q4_ERR_UNSUPPORTED;
    return MOE_Q4_OK;
}

static int run_forward(const void *x, const float *residual_y, void *x_out, const void *router_w, const float *bias,
                       void *logits, int64_t T, int32_t k, const moe_q4_layer *w, const moe_q4_shared_expert *sx,
                       int32_t *topk_idx, float *topk_gate, float *y, void *ws, size_t ws_bytes,
                       moe_q4_stream stream, void *const *events, bool det = false, int grid_div = 1) {
    int st = forward_checks(x, residual_y, x_out, logits, T, k, w, sx, topk_idx, topk_gate, y, events);
    if (st || T == 0) return st;
    const int E = w->num_experts, H = w->hidden, I = w->inter;
    const bool dec = forward_uses_decode(T, k);
    hipEvent_t const *ev = reinterpret_cast<hipEvent_t const *>(events);
    hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
    hipEvent_t e2 = ev ? ev[2] : nullptr, e3 = ev ? ev[3] : nullptr;
    const size_t need_fwd = moe_q4_workspace_size(det ? MOE_Q4_WS_FORWARD_DET : MOE_Q4_WS_FORWARD, T, E, k, H, I);
    const size_t need = need_fwd + (sx ? moe_q4_workspace_size(MOE_Q4_WS_SHARED, T, 1, 1, H, sx->inter) : 0);
    if (!ws || ws_bytes < need) return MOE_Q4_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const LayerPtrs L = layer_ptrs(w);
    // the shared expert's h follows the forward regions
    SharedPtrs S{};
    SharedWs sws{};
    float *hs = nullptr;
    if (sx) {
        S = shared_ptrs(sx);
        Carver cs{static_cast<char *>(ws) + need_fwd};
        sws = carve_shared(cs, T, H, sx->inter);
        hs = sws.h;
    }
    // the deterministic decode keeps the shared expert out of the routed
    // launches (its rows would be added with atomics)
    const bool fuse = sx && dec && !det && decode_fuses_shared(L, &S);
    const SharedPtrs *Sf = fuse ? &S : nullptr;
    // the shared expert on its own, after the routed experts: y += its output
    auto shared_after = [&](const uint16_t *xin_) {
        return sx && !fuse ? hip_status(launch_shared_any(xin_, T, S, sws, y, true, s, nullptr)) : MOE_Q4_OK;
    };
    Carver c{static_cast<char *>(ws)};
    unsigned int *counter = c.take<unsigned int>(CONTROL_BYTES / sizeof(unsigned int));
    unsigned int *handoff = c.take<unsigned int>(T * (int64_t)E);
    const uint16_t *xin = static_cast<const uint16_t *>(residual_y ? x_out : x);
    const uint16_t *wr = static_cast<const uint16_t *>(router_w);
    uint16_t *lg = static_cast<uint16_t *>(logits);
    if (dec) {
        DecodeWs d = carve_decode(c, T, E, k, H, I);
        float *zrows = det ? c.take<float>(T * k * (int64_t)H) : nullptr;
        if ((forward_fused_route(T, E) || !wr) && decode_routes_in_block(T, k, E)) {
            // router GEMV (+ residual, y clear) in one launch; the expert GEMV
            // launches route the tokens in every workgroup
            st = hip_status(launch_decode_route_group(static_cast<const uint16_t *>(x), residual_y,
                                                      static_cast<uint16_t *>(x_out), wr, bias, (int)T, H, E, k, lg,
                                                      topk_idx, topk_gate, d.g, y, counter, handoff, s, false, e2,
                                                      e3));
            if (st) return st;
            st = hip_status(
                launch_decode_experts_routed(xin, lg, T, k, L, d.g, topk_idx, topk_gate, d.h, y, s, e0, e1, Sf, hs,
                                             zrows, grid_div));
            return st ? st : shared_after(xin);
        }
        if (forward_fused_route(T, E) || !wr) {
            st = hip_status(launch_decode_route_group(static_cast<const uint16_t *>(x), residual_y,
                                                      static_cast<uint16_t *>(x_out), wr, bias, (int)T, H, E, k, lg,
                                                      topk_idx, topk_gate, d.g, y, counter, handoff, s, true, e2,
                                                      e3));
        } else {  // separate router, top-k and grouping launches
            if (residual_y)
                st = hip_status(launch_residual(static_cast<const uint16_t *>(x), residual_y, T * (int64_t)H,
                                                static_cast<uint16_t *>(x_out), s));
            if (!st) st = hip_status(launch_router_logits(xin, wr, bias, T, H, E, lg, s));
            if (!st) st = hip_status(launch_topk(lg, T, E, k, topk_idx, topk_gate, s));
            if (!st) st = hip_status(launch_group(topk_idx, T, k, E, d.g, s, y, T * (int64_t)H, e2, e3));
        }
        if (st) return st;
        st = hip_status(
            launch_decode_experts(xin, topk_gate, T, k, L, d.g, d.h, y, s, e0, e1, Sf, hs, zrows, grid_div));
        return st ? st : shared_after(xin);
    }
    if (residual_y) {
        st = hip_status(launch_residual(static_cast<const uint16_t *>(x), residual_y, T * (int64_t)H,
                                        static_cast<uint16_t *>(x_out), s));
        if (st) return st;
    }
    if (wr) {
        st = hip_status(launch_router_logits(xin, wr, bias, T, H, E, lg, s));
        if (st) return st;
    }
    PrefillWs p = carve_prefill(c, T, E, k, H, I);
    const bool prep = T * (int64_t)k > GROUP_SINGLE_MAX;
    if (prep) {  // top-k, the grouping's count and the f16 rows of x in one launch
        st = hip_status(launch_prefill_prep(lg, T, E, k, topk_idx, topk_gate, p.g, xin, H, p.x16, p.xexp, L.fmt, s));
        if (!st) st = hip_status(launch_group_after_count(topk_idx, T, k, E, p.g, s));
    } else {
        st = hip_status(launch_topk(lg, T, E, k, topk_idx, topk_gate, s));
        if (!st) st = hip_status(launch_group(topk_idx, T, k, E, p.g, s));
    }
    if (st) return st;
    st = hip_status(launch_prefill_experts(xin, topk_gate, T, k, L, p.g, p.x16, p.xexp, p.h, p.z, p.hx, p.zx, y, s, ev,
                                           prep));
    return st ? st : shared_after(xin);
}

int moe_q4_forward(const void *x, const float *residual_y, void *x_out, const void *router_w, const float *bias,
                   void *logits, int64_t T, int32_t k, const moe_q4_layer *w, int32_t *topk_idx, float *topk_gate,
                   float *y, void *ws, size_t ws_bytes, moe_q4_stream stream) {
    return run_forward(x, residual_y, x_out, router_w, bias, logits, T, k, w, nullptr, topk_idx, topk_gate, y, ws,
                       ws_bytes, stream, nullptr);
}

int moe_q4_forward_timed(const void *x, const float *residual_y, void *x_out, const void *router_w,
                         const float *bias, void *logits, int64_t T, int32_t k, const moe_q4_layer *w,
                         int32_t *topk_idx, float *topk_gate, float *y, void *ws, size_t ws_bytes,
                         moe_q4_stream stream, void *const *events) {
    if (!events) return MOE_Q4_ERR_INVALID_ARG;
    return run_forward(x, residual_y, x_out, router_w, bias, logits, T, k, w, nullptr, topk_idx, topk_gate, y, ws,
                       ws_bytes, stream, events);
}

int moe_q4_forward_ex(const void *x, const float *residual_y, void *x_out, const void *router_w, const float *bias,
                      void *logits, int64_t T, int32_t k, const moe_q4_layer *w, const moe_q4_shared_expert *shared,
                      int32_t *topk_idx, float *topk_gate, float *y, void *ws, size_t ws_bytes, moe_q4_stream stream,
                      void *const *events) {
    return run_forward(x, residual_y, x_out, router_w, bias, logits, T, k, w, shared, topk_idx, topk_gate, y, ws,
                       ws_bytes, stream, events);
}

int moe_q4_forward_det(const void *x, const float *residual_y, void *x_out, const void *router_w,
                       const float *bias, void *logits, int64_t T, int32_t k, const moe_q4_layer *w,
                       const moe_q4_shared_expert *shared, int32_t *topk_idx, float *topk_gate, float *y, void *ws,
                       size_t ws_bytes, moe_q4_stream stream, void *const *events) {
    return run_forward(x, residual_y, x_out, router_w, bias, logits, T, k, w, shared, topk_idx, topk_gate, y, ws,
                       ws_bytes, stream, events, true);
}

// ------------------------------------------------------------ frame in token lanes

// One lane's workspace: the layer forward's (with the shared expert's after
// it), for the lane's tokens.
static size_t frame_lane_bytes(int64_t TL, int32_t E, int32_t k, int32_t H, int32_t I, int32_t shared_inter) {
    size_t b = moe_q4_workspace_size(MOE_Q4_WS_FORWARD, TL, E, k, H, I);
    if (shared_inter > 0) b += moe_q4_workspace_size(MOE_Q4_WS_SHARED, TL, 1, 1, H, shared_inter);
    return align_up(b);
}

// Token rows [r0, r1) of lane i of `lanes` over T tokens.
static void frame_lane_rows(int64_t T, int i, int lanes, int64_t *r0, int64_t *r1) {
    *r0 = T * i / lanes;
    *r1 = T * (i + 1) / lanes;
}

size_t moe_q4_frame_workspace_size(int64_t T, int32_t E, int32_t k, int32_t H, int32_t I, int32_t shared_inter,
                                   int32_t lanes) {
    if (T <= 0 || lanes < 1 || lanes > MOE_Q4_FRAME_MAX_LANES || lanes > T || shared_inter < 0) return 0;
    const int64_t TL = (T + lanes - 1) / lanes;  // the largest lane
    const size_t b = frame_lane_bytes(TL, E, k, H, I, shared_inter);
    return b ? b * (size_t)lanes : 0;
}

int moe_q4_frame(const void *x, int64_t T, int32_t k, int32_t n_layers, const moe_q4_layer *layers,
                 const void *const *router_w, const moe_q4_shared_expert *shared, void *x_chain, float *y_chain,
                 void *logits, int32_t *topk_idx, float *topk_gate, int32_t lanes, const moe_q4_stream *streams,
                 void *ws, size_t ws_bytes, void *const *events) {
    if (T < 0 || n_layers < 1 || !layers || !router_w || !streams) return MOE_Q4_ERR_INVALID_ARG;
    if (lanes < 1 || lanes > MOE_Q4_FRAME_MAX_LANES || (T > 0 && lanes > T)) return MOE_Q4_ERR_INVALID_ARG;
    if (!x || !y_chain || !logits || !topk_idx || !topk_gate || (n_layers > 1 && !x_chain))
        return MOE_Q4_ERR_INVALID_ARG;
    const int E = layers[0].num_experts, H = layers[0].hidden, I = layers[0].inter;
    const int32_t sinter = shared ? shared[0].inter : 0;
    for (int j = 0; j < n_layers; ++j) {
        if (!router_w[j]) return MOE_Q4_ERR_INVALID_ARG;
        if (layers[j].num_experts != E || layers[j].hidden != H || layers[j].inter != I)
            return MOE_Q4_ERR_INVALID_ARG;
        if (shared && shared[j].inter != sinter) return MOE_Q4_ERR_INVALID_ARG;
    }
    if (events)
        for (int64_t i = 0; i < (int64_t)n_layers * lanes * MOE_Q4_STAGE_EVENTS; ++i)
            if (!events[i]) return MOE_Q4_ERR_INVALID_ARG;
    int st = check_layer(&layers[0], false);
    if (st) return st;
    if (T == 0) return MOE_Q4_OK;
    const size_t lane_b = frame_lane_bytes((T + lanes - 1) / lanes, E, k, H, I, sinter);
    if (!lane_b) return MOE_Q4_ERR_INVALID_ARG;
    if (!ws || ws_bytes < lane_b * (size_t)lanes) return MOE_Q4_ERR_WORKSPACE;

    // the pointers of layer j, lane i
    struct LanePtrs {
        const void *x;
        const float *yres;
        void *xout, *lg;
        int32_t *idx;
        float *gate, *y;
        void *const *ev;
    };
    auto lane_ptrs = [&](int j, int i) {
        int64_t r0, r1;
        frame_lane_rows(T, i, lanes, &r0, &r1);
        const int64_t TH = T * (int64_t)H;
        LanePtrs p;
        // layer j > 0: the residual step bf16(x_{j-1} + y_{j-1}) is its
        // input x_j, written to x_chain[j - 1]
        uint16_t *xc = static_cast<uint16_t *>(x_chain);
        const uint16_t *xprev = j <= 1 ? static_cast<const uint16_t *>(x) : xc + (j - 2) * TH;
        p.x = xprev + r0 * H;
        p.yres = j == 0 ? nullptr : y_chain + (j - 1) * TH + r0 * H;
        p.xout = j == 0 ? nullptr : static_cast<void *>(xc + (j - 1) * TH + r0 * H);
        p.lg = static_cast<uint16_t *>(logits) + (j * T + r0) * (int64_t)E;
        p.idx = topk_idx + (j * T + r0) * (int64_t)k;
        p.gate = topk_gate + (j * T + r0) * (int64_t)k;
        p.y = y_chain + j * TH + r0 * H;
        p.ev = events ? events + ((int64_t)j * lanes + i) * MOE_Q4_STAGE_EVENTS : nullptr;
        return p;
    };
    // every check before the first launch
    for (int j = 0; j < n_layers; ++j)
        for (int i = 0; i < lanes; ++i) {
            int64_t r0, r1;
            frame_lane_rows(T, i, lanes, &r0, &r1);
            const LanePtrs p = lane_ptrs(j, i);
            st = forward_checks(p.x, p.yres, p.xout, p.lg, r1 - r0, k, &layers[j], shared ? &shared[j] : nullptr,
                                p.idx, p.gate, p.y, p.ev);
            if (st) return st;
        }
    char *wsb = static_cast<char *>(ws);
    for (int i = 0; i < lanes; ++i) {  // each lane's routing counters start at zero
        st = hip_status(launch_fill_zero_u32(reinterpret_cast<uint32_t *>(wsb + lane_b * i), CONTROL_BYTES / 4,
                                             reinterpret_cast<hipStream_t>(streams[i])));
        if (st) return st;
    }
    for (int j = 0; j < n_layers; ++j)
        for (int i = 0; i < lanes; ++i) {
            int64_t r0, r1;
            frame_lane_rows(T, i, lanes, &r0, &r1);
            const LanePtrs p = lane_ptrs(j, i);
            st = run_forward(p.x, p.yres, p.xout, router_w[j], nullptr, p.lg, r1 - r0, k, &layers[j],
                             shared ? &shared[j] : nullptr, p.idx, p.gate, p.y, wsb + lane_b * i, lane_b,
                             streams[i], p.ev, false, lanes);
            if (st) return st;
        }
    return MOE_Q4_OK;
}

}  // extern "C"

namespace {

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex noalloc_mutex;
void *noalloc_ptr[NOALLOC_MAX_DEVICES];

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int noalloc_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_Q4_ERR_HIP;
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return MOE_Q4_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(noalloc_mutex);
    if (!noalloc_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_Q4_ERR_HIP;
        noalloc_ptr[dev] = p;
    }
    *out = noalloc_ptr[dev];
    return MOE_Q4_OK;
}

}  // namespace

extern "C" {

int moe_q4_forward_noalloc(const void *x, const float *residual_y, void *x_out, const void *router_w,
                           const float *bias, void *logits, int64_t T, int32_t k, const moe_q4_layer *w,
                           int32_t *topk_idx, float *topk_gate, float *y, moe_q4_stream stream) {
    int st = forward_checks(x, residual_y, x_out, logits, T, k, w, nullptr, topk_idx, topk_gate, y, nullptr);
    if (st || T == 0) return st;
    const size_t need = moe_q4_workspace_size(MOE_Q4_WS_FORWARD, T, w->num_experts, k, w->hidden, w->inter);
    if (need > MOE_Q4_NOALLOC_SCRATCH_BYTES) return MOE_Q4_ERR_WORKSPACE;
    void *ws = nullptr;
    st = noalloc_scratch(&ws);
    if (st) return st;
    // the routing counters must start at zero; a fill kernel (not a memset
    // node) clears them on the caller's stream before the layer's launches
    st = hip_status(launch_fill_zero_u32(static_cast<uint32_t *>(ws), CONTROL_BYTES / 4,
                                         reinterpret_cast<hipStream_t>(stream)));
    if (st) return st;
    return run_forward(x, residual_y, x_out, router_w, bias, logits, T, k, w, nullptr, topk_idx, topk_gate, y, ws,
                       MOE_Q4_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int moe_q4_dequant(const moe_q4_layer *w, int32_t expert, int32_t proj, float *out, moe_q4_stream stream) {
    int st = check_layer(w, false);
    if (st) return st;
    if (!out || expert < 0 || expert >= w->num_experts || proj < 0 || proj > 2) return MOE_Q4_ERR_INVALID_ARG;
    return hip_status(launch_dequant(layer_ptrs(w), expert, proj, out, reinterpret_cast<hipStream_t>(stream)));
}

// The prefill copy is made from the canonical arrays; the field that would
// point to a copy is not read here.
static int check_pack_source(const moe_q4_layer *w, moe_q4_layer *plain) {
    if (!w) return MOE_Q4_ERR_INVALID_ARG;
    *plain = *w;
    plain->prefill_pack = nullptr;
    return check_layer(plain, true);
}

size_t moe_q4_prefill_pack_size(const moe_q4_layer *w) {
    moe_q4_layer plain;
    if (check_pack_source(w, &plain)) return 0;
    return pack_layout(plain.num_experts, plain.hidden, plain.inter, plain.format).total;
}

int moe_q4_prefill_pack(const moe_q4_layer *w, void *dst, size_t dst_bytes, moe_q4_stream stream) {
    moe_q4_layer plain;
    int st = check_pack_source(w, &plain);
    if (st) return st;
    if (!dst || !aligned(dst, 256) ||
        dst_bytes < pack_layout(plain.num_experts, plain.hidden, plain.inter, plain.format).total)
        return MOE_Q4_ERR_INVALID_ARG;
    return hip_status(
        launch_prefill_pack(layer_ptrs(&plain), static_cast<uint8_t *>(dst), reinterpret_cast<hipStream_t>(stream)));
}

static int run_shared(const void *x, int64_t T, const moe_q4_shared_expert *sx, float *y, int32_t accumulate,
                      void *ws, size_t ws_bytes, moe_q4_stream stream, void *const *events) {
    int st = check_shared(sx);
    if (st) return st;
    if (T < 0 || !x || !y) return MOE_Q4_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(y, 16)) return MOE_Q4_ERR_INVALID_ARG;
    const int H = sx->hidden, I = sx->inter;
    if (T * (int64_t)H >= ((int64_t)1 << 31) || T * (int64_t)I >= ((int64_t)1 << 31)) return MOE_Q4_ERR_UNSUPPORTED;
    if (T == 0) return MOE_Q4_OK;
    const size_t need = moe_q4_workspace_size(MOE_Q4_WS_SHARED, T, 1, 1, H, I);
    if (!ws || ws_bytes < need) return MOE_Q4_ERR_WORKSPACE;
    Carver c{static_cast<char *>(ws)};
    const SharedWs w = carve_shared(c, T, H, I);
    return hip_status(launch_shared_any(static_cast<const uint16_t *>(x), T, shared_ptrs(sx), w, y, accumulate != 0,
                                        reinterpret_cast<hipStream_t>(stream),
                                        reinterpret_cast<hipEvent_t const *>(events)));
}

int moe_q4_shared(const void *x, int64_t T, const moe_q4_shared_expert *sx, float *y, int32_t accumulate, void *ws,
                  size_t ws_bytes, moe_q4_stream stream) {
    return run_shared(x, T, sx, y, accumulate, ws, ws_bytes, stream, nullptr);
}

int moe_q4_shared_timed(const void *x, int64_t T, const moe_q4_shared_expert *sx, float *y, int32_t accumulate,
                        void *ws, size_t ws_bytes, moe_q4_stream stream, void *const *events) {
    if (!events) return MOE_Q4_ERR_INVALID_ARG;
    for (int i = 0; i < MOE_Q4_STAGE_EVENTS; ++i)
        if (!events[i]) return MOE_Q4_ERR_INVALID_ARG;
    return run_shared(x, T, sx, y, accumulate, ws, ws_bytes, stream, events);
}

int moe_q4_dequant_int8(const moe_q4_shared_expert *sx, int32_t proj, float *out, moe_q4_stream stream) {
    int st = check_shared(sx);
    if (st) return st;
    if (!out || proj < 0 || proj > 2) return MOE_Q4_ERR_INVALID_ARG;
    return hip_status(launch_dequant_int8(shared_ptrs(sx), proj, out, reinterpret_cast<hipStream_t>(stream)));
}

int moe_q4_residual_bf16(const void *x, const float *y, int64_t n, void *out, moe_q4_stream stream) {
    if (n < 0 || (n > 0 && (!x || !y || !out))) return MOE_Q4_ERR_INVALID_ARG;
    if (n == 0) return MOE_Q4_OK;
    return hip_status(launch_residual(static_cast<const uint16_t *>(x), y, n, static_cast<uint16_t *>(out),
                                      reinterpret_cast<hipStream_t>(stream)));
}

const char *moe_q4_error_string(int status) {
    switch (status) {
        case MOE_Q4_OK: return "ok";
        case MOE_Q4_ERR_INVALID_ARG: return "invalid argument";
        case MOE_Q4_ERR_UNSUPPORTED: return "unsupported shape or format";
        case MOE_Q4_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_Q4_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

}  // extern "C"
