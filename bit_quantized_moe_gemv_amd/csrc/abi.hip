// abi.hip -- the exported C entry points of libbqmoe.so: argument validation,
// workspace carving and the launch sequence of one forward pass.
#include <mutex>
#include <new>
#include <vector>

#include "bqmoe.h"
#include "moe_internal.h"

using namespace bqmoe;

struct moe_layer {
    moe_layer_desc desc;
    Shape shape;
    void *ws_base;
    size_t ws_bytes;
    Workspace ws;
    int last_T;
    int last_path;
    // per-stage timing (moe_layer_set_profiling)
    int prof_slots;
    int prof_next;
    std::vector<hipEvent_t> prof_ev;  // [slots][MOE_N_STAGES][2]
    std::vector<char> prof_ran;       // [slots][MOE_N_STAGES]
};

static void prof_release(moe_layer *L) {
    for (hipEvent_t e : L->prof_ev)
        if (e) (void)hipEventDestroy(e);
    L->prof_ev.clear();
    L->prof_ran.clear();
    L->prof_slots = 0;
    L->prof_next = 0;
}

// Runs one launcher, bracketed by the slot's event pair when profiling.
template <class F>
static hipError_t staged(moe_layer *L, int slot, int stage, hipStream_t st, F &&launch) {
    if (!L || slot < 0) return launch();
    hipEvent_t *ev = &L->prof_ev[((size_t)slot * MOE_N_STAGES + stage) * 2];
    hipError_t e = hipEventRecord(ev[0], st);
    if (e == hipSuccess) e = launch();
    if (e == hipSuccess) e = hipEventRecord(ev[1], st);
    if (e == hipSuccess) L->prof_ran[(size_t)slot * MOE_N_STAGES + stage] = 1;
    return e;
}

namespace bqmoe {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t workspace_bytes(const Shape &s, int tmax) {
    const size_t R = (size_t)tmax * s.K;
    size_t b = 0;
    b += align256((size_t)tmax * s.E * 4);  // logits
    b += align256(R * 4);                   // idx
    b += align256(R * 4);                   // w
    b += align256((size_t)s.E * 4);         // counts
    b += align256((size_t)(s.E + 1) * 4);   // offsets
    b += align256((size_t)(s.E + 1) * 4);   // active
    b += align256(R * 4);                   // perm
    b += align256(R * 4);                   // inv
    b += align256(R * s.I * 4);             // h
    b += align256(R * s.H * 2 + R * (s.H / 4));  // y16, yexp
    b += align256(R * s.I * 2);             // h16
    b += align256(R * 4);                   // hexp
    if (is_vq_format(s.fmt)) {
        b += align256((size_t)tmax * s.H * 2);  // x16
        b += align256((size_t)tmax * 4);        // xexp
        b += align256(R * (s.I / 64) * 4);      // hpmax
    }
    return b;
}

void carve_workspace(const Shape &s, int tmax, void *base, Workspace *ws) {
    const size_t R = (size_t)tmax * s.K;
    char *p = static_cast<char *>(base);
    auto take = [&](size_t bytes) {
        char *r = p;
        p += align256(bytes);
        return r;
    };
    ws->logits = reinterpret_cast<float *>(take((size_t)tmax * s.E * 4));
    ws->idx = reinterpret_cast<int32_t *>(take(R * 4));
    ws->w = reinterpret_cast<float *>(take(R * 4));
    ws->counts = reinterpret_cast<int32_t *>(take((size_t)s.E * 4));
    ws->offsets = reinterpret_cast<int32_t *>(take((size_t)(s.E + 1) * 4));
    ws->active = reinterpret_cast<int32_t *>(take((size_t)(s.E + 1) * 4));
    ws->perm = reinterpret_cast<int32_t *>(take(R * 4));
    ws->inv = reinterpret_cast<int32_t *>(take(R * 4));
    ws->h = take(R * s.I * 4);
    ws->y16 = reinterpret_cast<uint16_t *>(take(R * s.H * 2 + R * (s.H / 4)));
    ws->yexp = reinterpret_cast<int8_t *>(ws->y16 + R * s.H);
    ws->h16 = reinterpret_cast<uint16_t *>(take(R * s.I * 2));
    ws->hexp = reinterpret_cast<int32_t *>(take(R * 4));
    ws->x16 = nullptr;
    ws->xexp = nullptr;
    ws->hpmax = nullptr;
    if (is_vq_format(s.fmt)) {
        ws->x16 = reinterpret_cast<uint16_t *>(take((size_t)tmax * s.H * 2));
        ws->xexp = reinterpret_cast<int32_t *>(take((size_t)tmax * 4));
        ws->hpmax = reinterpret_cast<float *>(take(R * (s.I / 64) * 4));
    }
}

}  // namespace bqmoe

static int check_desc(const moe_layer_desc *d, Shape *s) {
    if (!d) return MOE_EINVAL;
    // hidden <= 8192: the small-batch router holds a token's row in registers
    // (at most 32 groups of 256 columns per wave)
    if (d->hidden < 256 || d->hidden > kMaxHidden || d->hidden % 256) return MOE_EINVAL;
    if (d->inter < 128 || d->inter > 16384) return MOE_EINVAL;
    if (d->n_experts < 1 || d->n_experts > kMaxExperts) return MOE_EINVAL;
    if (d->top_k < 1 || d->top_k > kMaxTopK || d->top_k > d->n_experts) return MOE_EINVAL;
    if (d->max_tokens < 1 || d->max_tokens > 65536) return MOE_EINVAL;
    if (d->force_path < MOE_PATH_AUTO || d->force_path > MOE_PATH_PREFILL) return MOE_EINVAL;
    if (d->routing != MOE_ROUTE_SOFTMAX && d->routing != MOE_ROUTE_SIGMOID) return MOE_EINVAL;
    if (d->format == MOE_FMT_MXFP4) {
        if (d->inter % 128) return MOE_EINVAL;
    } else if (is_vq_format(d->format)) {
        if (d->inter % 256) return MOE_EINVAL;
    } else {
        return MOE_EINVAL;
    }
    if (s) {
        s->H = d->hidden;
        s->I = d->inter;
        s->E = d->n_experts;
        s->K = d->top_k;
        s->fmt = d->format;
        s->routing = d->routing;
        const size_t H = (size_t)d->hidden, I = (size_t)d->inter;
        if (d->format == MOE_FMT_MXFP4) {
            s->expert_bytes = 3 * I * H * 17 / 32;
            s->books_bytes = 0;
        } else if (d->format == MOE_FMT_VQ13R8) {
            s->expert_bytes = 3 * I * H * 21 / 64 + 2 * (2 * I + H);
            s->books_bytes = kVqBooksBytes;
        } else {
            s->expert_bytes = 3 * I * H * 13 / 64 + 2 * (2 * I + H);
            s->books_bytes = kVq13BooksBytes;
        }
    }
    // the decode kernels are instantiated for power-of-two widths
    if (d->force_path == MOE_PATH_DECODE && s && !decode_supported(*s)) return MOE_EUNSUPPORTED;
    return MOE_OK;
}

static bool aligned16(const void *p) { return p && ((uintptr_t)p & 15u) == 0; }

// The path a forward of T tokens takes (MOE_PATH_DECODE or MOE_PATH_PREFILL),
// or MOE_EINVAL when a forced decode path cannot take T tokens.
static int choose_path(const Shape &s, int force_path, int T) {
    int path = force_path;
    if (path == MOE_PATH_AUTO)
        path = (T <= decode_max_tokens(s) && decode_supported(s)) ? MOE_PATH_DECODE
                                                                 : MOE_PATH_PREFILL;
    if (path == MOE_PATH_DECODE && T > decode_max_tokens(s)) return MOE_EINVAL;
    return path;
}

// The kernel sequence of one forward pass on stream st.  L (may be null) and
// slot (-1: none) select the profiling events around each stage.
static hipError_t enqueue_forward(moe_layer *L, int slot, const Shape &s, const Workspace &ws,
                                  int path, const uint16_t *x, int T, const float *router_w,
                                  const uint8_t *packed, float *out, hipStream_t st) {
    hipError_t err = hipSuccess;
    if (path == MOE_PATH_DECODE) {
        err = staged(L, slot, MOE_STAGE_ROUTER, st, [&] {
            return launch_router_route_small(s, x, router_w, T, ws, st, false);
        });
        if (err == hipSuccess)
            err = staged(L, slot, MOE_STAGE_GATEUP, st,
                         [&] { return launch_decode_gateup(s, T, x, packed, ws, st); });
        if (err == hipSuccess)
            err = staged(L, slot, MOE_STAGE_DOWN, st,
                         [&] { return launch_decode_down(s, T, packed, ws, out, st); });
        return err;
    }
    if (T <= kDecodeMaxTokens) {  // small batch (a VQ layer, or a forced path)
        err = staged(L, slot, MOE_STAGE_ROUTER, st, [&] {
            return launch_router_route_small(s, x, router_w, T, ws, st, true);
        });
    } else {
        err = staged(L, slot, MOE_STAGE_ROUTER, st,
                     [&] { return launch_router(s, x, router_w, T, ws.logits, st); });
        if (err == hipSuccess)
            err = staged(L, slot, MOE_STAGE_SELECT, st, [&] { return launch_topk(s, T, ws, st); });
        if (err == hipSuccess)
            err = staged(L, slot, MOE_STAGE_PERMUTE, st,
                         [&] { return launch_permute(s, T, ws, st); });
    }
    const bool vq = is_vq_format(s.fmt);
    if (err == hipSuccess)
        err = staged(L, slot, MOE_STAGE_GATEUP, st, [&] {
            return vq ? launch_vq_prefill_gateup(s, T, x, packed, ws, st)
                      : launch_prefill_gateup(s, T, x, packed, ws, st);
        });
    if (err == hipSuccess)
        err = staged(L, slot, MOE_STAGE_DOWN, st, [&] {
            return vq ? launch_vq_prefill_down(s, T, packed, ws, st)
                      : launch_prefill_down(s, T, packed, ws, st);
        });
    if (err == hipSuccess)
        err = staged(L, slot, MOE_STAGE_COMBINE, st,
                     [&] { return launch_combine(s, T, ws, out, st); });
    return err;
}

extern "C" {

int moe_packed_size(const moe_layer_desc *desc, size_t *bytes) {
    Shape s;
    const int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!bytes) return MOE_EINVAL;
    *bytes = s.books_bytes + s.expert_bytes * (size_t)s.E;
    return MOE_OK;
}

int moe_workspace_size(const moe_layer_desc *desc, size_t *bytes) {
    Shape s;
    const int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!bytes) return MOE_EINVAL;
    *bytes = workspace_bytes(s, desc->max_tokens);
    return MOE_OK;
}

int moe_layer_create(const moe_layer_desc *desc, void *workspace, size_t ws_bytes,
                     moe_layer **out) {
    if (!out) return MOE_EINVAL;
    *out = nullptr;
    Shape s;
    const int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (!workspace || ((uintptr_t)workspace & 255u)) return MOE_EWORKSPACE;
    if (ws_bytes < workspace_bytes(s, desc->max_tokens)) return MOE_EWORKSPACE;
    moe_layer *L = new (std::nothrow) moe_layer;
    if (!L) return MOE_EINVAL;
    L->desc = *desc;
    L->shape = s;
    L->ws_base = workspace;
    L->ws_bytes = ws_bytes;
    carve_workspace(s, desc->max_tokens, workspace, &L->ws);
    L->last_T = 0;
    L->last_path = MOE_EINVAL;
    L->prof_slots = 0;
    L->prof_next = 0;
    *out = L;
    return MOE_OK;
}

int moe_layer_forward(moe_layer *L, const void *x_bf16, int32_t T, const float *router_w,
                      const void *packed_experts, float *out, void *hip_stream) {
    if (!L) return MOE_EINVAL;
    if (T < 1 || T > L->desc.max_tokens) return MOE_EINVAL;
    if (!aligned16(x_bf16) || !aligned16(router_w) || !aligned16(packed_experts) ||
        !aligned16(out))
        return MOE_EINVAL;
    const int path = choose_path(L->shape, L->desc.force_path, T);
    if (path < 0) return path;
    int slot = -1;
    if (L->prof_slots > 0) {
        slot = L->prof_next;
        L->prof_next = (L->prof_next + 1) % L->prof_slots;
        for (int i = 0; i < MOE_N_STAGES; ++i) L->prof_ran[(size_t)slot * MOE_N_STAGES + i] = 0;
    }
    const hipError_t err = enqueue_forward(L, slot, L->shape, L->ws, path,
                                           static_cast<const uint16_t *>(x_bf16), T, router_w,
                                           static_cast<const uint8_t *>(packed_experts), out,
                                           static_cast<hipStream_t>(hip_stream));
    if (err != hipSuccess) return MOE_EHIP;
    L->last_T = T;
    L->last_path = path;
    return MOE_OK;
}

// ---- moe_forward_noalloc: the workspace in a library-owned device array ----
// One copy per GPU, allocated by the runtime when the code object is loaded
// on that GPU and held until the process ends.  Host code never uses the
// array's name as an address: each device's address comes from
// hipGetSymbolAddress, looked up on the first call on that device.
static_assert(MOE_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices];  // per device id; null until looked up

// The current device's scratch address, or null if the lookup fails.
static void *scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

int moe_forward_noalloc(const moe_layer_desc *desc, const void *x_bf16, int32_t T,
                        const float *router_w, const void *packed_experts, float *out,
                        void *hip_stream) {
    Shape s;
    const int rc = check_desc(desc, &s);
    if (rc != MOE_OK) return rc;
    if (T < 1 || T > desc->max_tokens) return MOE_EINVAL;
    if (!aligned16(x_bf16) || !aligned16(router_w) || !aligned16(packed_experts) ||
        !aligned16(out))
        return MOE_EINVAL;
    const int path = choose_path(s, desc->force_path, T);
    if (path < 0) return path;
    // the workspace layout of a handle with max_tokens = T
    if (workspace_bytes(s, T) > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_EWORKSPACE;
    void *base = scratch_for_current_device();
    if (!base) return MOE_EHIP;
    Workspace ws;
    carve_workspace(s, T, base, &ws);
    const hipError_t err = enqueue_forward(nullptr, -1, s, ws, path,
                                           static_cast<const uint16_t *>(x_bf16), T, router_w,
                                           static_cast<const uint8_t *>(packed_experts), out,
                                           static_cast<hipStream_t>(hip_stream));
    return err == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_layer_routing(moe_layer *L, int32_t *topk_idx, float *topk_w, int32_t *counts,
                      int32_t *offsets, int32_t *perm, float *logits, void *hip_stream) {
    if (!L || L->last_T < 1) return MOE_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const Shape &s = L->shape;
    const size_t T = (size_t)L->last_T, R = T * s.K;
    struct { void *dst; const void *src; size_t bytes; } cp[] = {
        {topk_idx, L->ws.idx, R * 4},       {topk_w, L->ws.w, R * 4},
        {counts, L->ws.counts, (size_t)s.E * 4}, {offsets, L->ws.offsets, (size_t)(s.E + 1) * 4},
        {perm, L->ws.perm, R * 4},          {logits, L->ws.logits, T * s.E * 4},
    };
    for (auto &c : cp) {
        if (!c.dst) continue;
        if (hipMemcpyAsync(c.dst, c.src, c.bytes, hipMemcpyDeviceToDevice, st) != hipSuccess)
            return MOE_EHIP;
    }
    return MOE_OK;
}

int moe_layer_replay_stage(moe_layer *L, int32_t stage, int32_t reps, const void *x_bf16,
                           const float *router_w, const void *packed_experts, size_t copy_stride,
                           int32_t n_copies, float *out, void *hip_stream) {
    if (!L || L->last_T < 1) return MOE_EINVAL;
    if (stage < 0 || stage >= MOE_N_STAGES) return MOE_EINVAL;
    const bool decode = L->last_path == MOE_PATH_DECODE;
    if (decode && (stage == MOE_STAGE_SELECT || stage == MOE_STAGE_PERMUTE ||
                   stage == MOE_STAGE_COMBINE))
        return MOE_EINVAL;
    if (reps < 1 || n_copies < 1 || (copy_stride & 15u)) return MOE_EINVAL;
    if (!aligned16(x_bf16) || !aligned16(router_w) || !aligned16(packed_experts) ||
        !aligned16(out))
        return MOE_EINVAL;
    const Shape &s = L->shape;
    const Workspace &ws = L->ws;
    const int T = L->last_T;
    const bool vq = is_vq_format(s.fmt);
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const uint16_t *x = static_cast<const uint16_t *>(x_bf16);
    for (int i = 0; i < reps; ++i) {
        const uint8_t *packed =
            static_cast<const uint8_t *>(packed_experts) + (size_t)(i % n_copies) * copy_stride;
        hipError_t e = hipSuccess;
        switch (stage) {
            case MOE_STAGE_ROUTER:
                e = decode                  ? launch_router_route_small(s, x, router_w, T, ws, st, false)
                    : T <= kDecodeMaxTokens ? launch_router_route_small(s, x, router_w, T, ws, st, true)
                                            : launch_router(s, x, router_w, T, ws.logits, st);
                break;
            case MOE_STAGE_SELECT: e = launch_topk(s, T, ws, st); break;
            case MOE_STAGE_PERMUTE: e = launch_permute(s, T, ws, st); break;
            case MOE_STAGE_GATEUP:
                e = decode ? launch_decode_gateup(s, T, x, packed, ws, st)
                    : vq   ? launch_vq_prefill_gateup(s, T, x, packed, ws, st)
                           : launch_prefill_gateup(s, T, x, packed, ws, st);
                break;
            case MOE_STAGE_DOWN:
                e = decode ? launch_decode_down(s, T, packed, ws, out, st)
                    : vq   ? launch_vq_prefill_down(s, T, packed, ws, st)
                           : launch_prefill_down(s, T, packed, ws, st);
                break;
            default: e = launch_combine(s, T, ws, out, st); break;
        }
        if (e != hipSuccess) return MOE_EHIP;
    }
    return MOE_OK;
}

int moe_read_probe(const void *buf, size_t bytes, size_t copy_stride, int32_t n_copies,
                   int32_t reps, uint32_t *sink, void *hip_stream) {
    if (!aligned16(buf) || bytes < 16 || (bytes & 15u) || (copy_stride & 15u)) return MOE_EINVAL;
    if (n_copies < 1 || reps < 1 || !sink || ((uintptr_t)sink & 3u)) return MOE_EINVAL;
    if (n_copies > 1 && copy_stride < bytes) return MOE_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    for (int i = 0; i < reps; ++i) {
        const uint8_t *p = static_cast<const uint8_t *>(buf) + (size_t)(i % n_copies) * copy_stride;
        if (launch_read_probe(p, bytes, sink, st) != hipSuccess) return MOE_EHIP;
    }
    return MOE_OK;
}

int moe_layer_last_path(const moe_layer *L) { return L && L->last_T > 0 ? L->last_path : MOE_EINVAL; }

int moe_layer_set_profiling(moe_layer *L, int32_t slots) {
    if (!L || slots < 0 || slots > 65536) return MOE_EINVAL;
    prof_release(L);
    if (slots == 0) return MOE_OK;
    L->prof_ev.assign((size_t)slots * MOE_N_STAGES * 2, nullptr);
    L->prof_ran.assign((size_t)slots * MOE_N_STAGES, 0);
    for (hipEvent_t &e : L->prof_ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            e = nullptr;
            prof_release(L);
            return MOE_EHIP;
        }
    }
    L->prof_slots = slots;
    L->prof_next = 0;
    return MOE_OK;
}

int moe_layer_profile_read(moe_layer *L, float *ms, int32_t slots) {
    if (!L || !ms || slots != L->prof_slots || slots <= 0) return MOE_EINVAL;
    for (int sl = 0; sl < slots; ++sl)
        for (int st = 0; st < MOE_N_STAGES; ++st) {
            const size_t i = (size_t)sl * MOE_N_STAGES + st;
            ms[i] = -1.0f;
            if (!L->prof_ran[i]) continue;
            hipEvent_t *ev = &L->prof_ev[i * 2];
            if (hipEventSynchronize(ev[1]) != hipSuccess) return MOE_EHIP;
            float t = 0.0f;
            if (hipEventElapsedTime(&t, ev[0], ev[1]) != hipSuccess) return MOE_EHIP;
            ms[i] = t;
        }
    return MOE_OK;
}

void moe_layer_destroy(moe_layer *L) {
    if (!L) return;
    prof_release(L);
    delete L;
}

const char *moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument";
        case MOE_EUNSUPPORTED: return "unsupported shape or format";
        case MOE_EWORKSPACE: return "workspace missing or too small";
        case MOE_EHIP: return "HIP launch or runtime error";
        default: return "unknown status";
    }
}

}  // extern "C"
