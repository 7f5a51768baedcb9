// api.hip -- the extern "C" entry points declared in include/strata_moe.h:
// host-side argument validation, workspace carving and kernel launches.
// Nothing here synchronises, allocates or reads device memory.
#include "common.hpp"
#include "quant.hpp"
#include "workspace.hpp"
#include <atomic>
#include <mutex>

namespace strata {
hipError_t launch_prep(const float *x, int T, int rmsnorm, uint16_t *xsplit, __half *xperm,
                       int32_t *xexp, hipStream_t st);
hipError_t launch_logits(const uint16_t *xsplit, int T, const uint16_t *R, const float *bias,
                         float *logits, hipStream_t st);
hipError_t launch_topk(const float *logits, int T, int32_t *ids, float *w, hipStream_t st);
hipError_t launch_group(const int32_t *ids, int T, int32_t *offsets, int32_t *slots,
                        int32_t *active, int32_t *gcount, int max_items, int32_t *mlist,
                        int32_t *nitems, hipStream_t st);
hipError_t launch_plan(const int32_t *offsets, const int32_t *active, int max_items, int T,
                       int32_t *mlist, int32_t *nitems, hipStream_t st);
hipError_t launch_route_decode(const float *x, int T, const uint16_t *R, const float *bias,
                               int rmsnorm, float *lraw, XQ xq, bool prep, int32_t *ids,
                               float *w, int group, int32_t *slots, int4 *erec, int32_t *cdone,
                               int32_t *esync, const uint16_t *R2, const float *bias2,
                               float *lraw2, int32_t *pred, hipStream_t st);
hipError_t launch_router_gemv(const float *x, int T, const uint16_t *R, int rmsnorm, float *lraw,
                              XQ xq, const uint16_t *R2, float *lraw2, hipStream_t st);
hipError_t launch_decode_routed(const uint8_t *blobs, const float *lraw, int T, const float *bias,
                                XQ xq, HQ hq, int32_t *ids, float *w, float *y, float *res,
                                const int32_t *hint, const float *lraw2, const float *bias2,
                                int32_t *pred, const uint8_t *blobs_next, hipEvent_t ev0,
                                hipEvent_t ev1, hipStream_t st);
hipError_t launch_prep_decode(const float *x, int T, int rmsnorm, XQ xq, const int32_t *offsets,
                              const int32_t *slots, const int32_t *active, int4 *erec,
                              int32_t *esync, hipStream_t st);
hipError_t launch_decode_experts(const uint8_t *blobs, const int4 *erec, const int32_t *slots,
                                 XQ xq, HQ hq, float *out, int T, int32_t *sync, int32_t *cdone,
                                 const float *w, float *y, float *res, const int32_t *pred,
                                 const uint8_t *blobs_next, int32_t *status, int wait_limit,
                                 hipEvent_t ev0, hipEvent_t ev1, hipStream_t st);
hipError_t launch_prefill_experts(const uint8_t *blobs, const int32_t *offsets,
                                  const int32_t *slots, const int32_t *active,
                                  const int32_t *mlist, const int32_t *nitems, int max_items,
                                  const __half *xperm, const int32_t *xexp, __half *hperm,
                                  int32_t *hexp, float *out, int T, hipEvent_t ev0, hipEvent_t ev1,
                                  hipStream_t st);
hipError_t launch_combine(const float *out, const float *w, int T, float *y, float *res,
                          int accumulate_y, hipStream_t st);
hipError_t launch_prep_i8(const float *x, int T, int rmsnorm, int8_t *x8, float *xs, int32_t *xn,
                          hipStream_t st);
hipError_t launch_prefill_experts_i8(const uint8_t *blobs, const int32_t *offsets,
                                     const int32_t *slots, const int32_t *active,
                                     const int32_t *mlist, const int32_t *nitems, int max_items,
                                     const int8_t *x8, const float *xs8, const int32_t *xn8,
                                     int8_t *h8, float *hs8, int32_t *hn8, float *out, int T,
                                     hipEvent_t ev0, hipEvent_t ev1, hipStream_t st);

constexpr int ALL_FLAGS = STRATA_RMSNORM | STRATA_RESIDUAL | STRATA_INT8;

// The workspace of strata_moe_layer_static: one array per GPU, in the code
// object's device memory (zero at load), shared by every call on that GPU.
// Host code never uses `scratch` itself (on the host it is only a stand-in
// for the symbol): the device address comes from hipGetSymbolAddress, once
// per device, and only that address is handed to kernels.
constexpr size_t STATIC_WS_BYTES = 10u << 20;   // 10 MiB: ws_layout(T) for any T <= 64
static_assert(strata::ws_max_bytes(STRATA_STATIC_T_MAX) <= STATIC_WS_BYTES,
              "the static workspace holds every T up to STRATA_STATIC_T_MAX");
static __device__ __align__(256) uint8_t scratch[STATIC_WS_BYTES];

// Sets a workspace's status word to zero (graph-capturable, unlike a memset).
__global__ void status_clear_kernel(int32_t *status)
{
    if (threadIdx.x == 0)
        *status = 0;
}

namespace {

// Bound on the decode experts kernel's wait, in polls (about 0.3 s by default).
constexpr int WAIT_LIMIT_DEFAULT = 1 << 18;
std::atomic<int> g_wait_limit{WAIT_LIMIT_DEFAULT};

// The measurement hook's events (per host thread, used by one call).
thread_local hipEvent_t t_ev0 = nullptr, t_ev1 = nullptr;

// Take the armed hook events (or two NULLs) and disarm the hook.
void take_events(hipEvent_t &e0, hipEvent_t &e1)
{
    e0 = t_ev0;
    e1 = t_ev1;
    t_ev0 = t_ev1 = nullptr;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_T(int T) { return (T >= 1 && T <= T_MAX) ? STRATA_OK : STRATA_E_SHAPE; }

int check_ws(void *ws, size_t ws_bytes, int T)
{
    if (!ws || ws_bytes < ws_layout(T).total)
        return STRATA_E_WORKSPACE;
    if (!aligned(ws, 256))
        return STRATA_E_ALIGN;
    return STRATA_OK;
}

template <class P> P *at(void *ws, size_t off) { return reinterpret_cast<P *>((uint8_t *)ws + off); }

struct Carve {
    Ws L;
    uint16_t *xsplit;
    float *logits, *w, *out;
    __half *xperm, *hperm;
    XQ xq;
    HQ hq;
    int32_t *offsets, *slots, *active, *ids, *mlist, *nitems;
    int4 *erec;
    int32_t *cdone, *esync;
    float *lraw2;
    int32_t *pred, *gcount;
    int32_t *status, *xexp, *hexp;
    int8_t *x8, *h8;
    float *xs8, *hs8;
    int32_t *xn8, *hn8;
};

Carve carve(void *ws, int T)
{
    Carve c;
    c.L = ws_layout(T);
    const Ws &L = c.L;
    c.xsplit = at<uint16_t>(ws, L.xsplit);
    c.xperm = at<__half>(ws, L.xperm);
    c.logits = at<float>(ws, L.logits);
    c.xq = XQ{at<uint32_t>(ws, L.xq_dig), at<float>(ws, L.xq_scale), at<int32_t>(ws, L.xq_sum),
              at<float>(ws, L.inv_rms)};
    c.hq = HQ{at<uint32_t>(ws, L.hq_dig), at<float>(ws, L.hq_scale), at<int32_t>(ws, L.hq_sum)};
    c.hperm = at<__half>(ws, L.hperm);
    c.offsets = at<int32_t>(ws, L.offsets);
    c.slots = at<int32_t>(ws, L.slots);
    c.active = at<int32_t>(ws, L.active);
    c.erec = at<int4>(ws, L.erec);
    c.cdone = at<int32_t>(ws, L.cdone);
    c.esync = at<int32_t>(ws, L.esync);
    c.lraw2 = at<float>(ws, L.lraw2);
    c.pred = at<int32_t>(ws, L.pred);
    c.gcount = at<int32_t>(ws, L.gcount);
    c.status = at<int32_t>(ws, L.status);
    c.xexp = at<int32_t>(ws, L.xexp);
    c.hexp = at<int32_t>(ws, L.hexp);
    c.x8 = at<int8_t>(ws, L.x8);
    c.h8 = at<int8_t>(ws, L.h8);
    c.xs8 = at<float>(ws, L.xs8);
    c.hs8 = at<float>(ws, L.hs8);
    c.xn8 = at<int32_t>(ws, L.xn8);
    c.hn8 = at<int32_t>(ws, L.hn8);
    c.ids = at<int32_t>(ws, L.ids);
    c.w = at<float>(ws, L.w);
    c.mlist = at<int32_t>(ws, L.mlist);
    c.nitems = at<int32_t>(ws, L.nitems);
    c.out = at<float>(ws, L.out);
    return c;
}

#define STRATA_TRY(expr)                                                                           \
    do {                                                                                           \
        hipError_t e_ = (expr);                                                                    \
        if (e_ != hipSuccess)                                                                      \
            return STRATA_E_HIP;                                                                   \
    } while (0)

// The experts for T tokens of a grouped layer (activation prep already done).
// planned: the prefill work list is already in c.mlist / c.nitems (written
// by the grouping of the layer call).
int run_experts(const Carve &c, const uint8_t *blobs, const int32_t *offsets,
                const int32_t *slots, const int32_t *active, float *out, int T, hipStream_t st,
                bool planned = false, bool int8 = false)
{
    hipEvent_t e0, e1;
    take_events(e0, e1);
    if (is_decode(T)) {
        STRATA_TRY(launch_decode_experts(blobs, c.erec, slots, c.xq, c.hq, out, T, c.esync, nullptr,
                                         nullptr, nullptr, nullptr, nullptr, nullptr, c.status,
                                         g_wait_limit.load(), e0, e1, st));
    } else {
        if (!planned)
            STRATA_TRY(launch_plan(offsets, active, c.L.max_items, T, c.mlist, c.nitems, st));
        if (int8) {
            STRATA_TRY(launch_prefill_experts_i8(blobs, offsets, slots, active, c.mlist, c.nitems,
                                                 c.L.max_items, c.x8, c.xs8, c.xn8, c.h8, c.hs8,
                                                 c.hn8, out, T, e0, e1, st));
            return STRATA_OK;
        }
        STRATA_TRY(launch_prefill_experts(blobs, offsets, slots, active, c.mlist, c.nitems,
                                          c.L.max_items, c.xperm, c.xexp, c.hperm, c.hexp, out, T,
                                          e0, e1, st));
    }
    return STRATA_OK;
}

// Activation prep for the experts (decode: inverse RMS, 16-bit blocks and the
// work records of the caller's grouping; prefill: normalised fp32 and
// K-ordered fp16 copies).
int run_prep(const Carve &c, const float *x, int T, int rms, const int32_t *offsets,
             const int32_t *slots, const int32_t *active, hipStream_t st, bool int8 = false)
{
    if (!is_decode(T) && int8)
        STRATA_TRY(launch_prep_i8(x, T, rms, c.x8, c.xs8, c.xn8, st));
    else if (is_decode(T))
        STRATA_TRY(launch_prep_decode(x, T, rms, c.xq, offsets, slots, active, c.erec, c.esync, st));
    else
        STRATA_TRY(launch_prep(x, T, rms, nullptr, c.xperm, c.xexp, st));
    return STRATA_OK;
}

// The layer, with an optional lookahead (decode T <= 8): the next layer's
// router on the same input predicts its experts (pred) and the experts kernel
// reads their blobs (blobs2) into the memory-side cache.
int layer_impl(float *x, int T, const uint16_t *router, const float *bias, const uint8_t *blobs,
               int flags, float *y, int32_t *ids, float *w, const uint16_t *router2,
               const float *bias2, const uint8_t *blobs2, int32_t *pred, const int32_t *hint,
               void *ws, size_t ws_bytes, void *stream)
{
    int rc = check_T(T);
    if (rc)
        return rc;
    if (!x || !router || !blobs || (flags & ~ALL_FLAGS))
        return STRATA_E_ARG;
    if (!y && !(flags & STRATA_RESIDUAL))
        return STRATA_E_ARG;
    if ((rc = check_ws(ws, ws_bytes, T)))
        return rc;
    if (!aligned(x, 16) || !aligned(router, 16) || !aligned(blobs, 256) || !aligned(y, 16) ||
        !aligned(ids, 4) || !aligned(w, 4) || !aligned(bias, 4) || !aligned(hint, 4))
        return STRATA_E_ALIGN;
    if (router2 && (!aligned(router2, 16) || !aligned(blobs2, 256) || !aligned(bias2, 4) ||
                    !aligned(pred, 4)))
        return STRATA_E_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    Carve c = carve(ws, T);
    int32_t *ids_o = ids ? ids : c.ids;
    float *w_o = w ? w : c.w;
    int32_t *pred_o = pred ? pred : c.pred;
    const int rms = flags & STRATA_RMSNORM;
    if (T <= ROUTED_T_MAX) {   // the gate/up launch routes each token
        STRATA_TRY(launch_router_gemv(x, T, router, rms, c.logits, c.xq, router2, c.lraw2, st));
        hipEvent_t e0, e1;
        take_events(e0, e1);
        STRATA_TRY(launch_decode_routed(blobs, c.logits, T, bias, c.xq, c.hq, ids_o, w_o, y,
                                        (flags & STRATA_RESIDUAL) ? x : nullptr, hint,
                                        router2 ? c.lraw2 : nullptr, bias2,
                                        router2 ? pred_o : nullptr, router2 ? blobs2 : nullptr,
                                        e0, e1, st));
        return STRATA_OK;
    }
    if (is_decode(T)) {
        STRATA_TRY(launch_route_decode(x, T, router, bias, rms, c.logits, c.xq, true, ids_o, w_o, 1,
                                       c.slots, c.erec, c.cdone, c.esync, router2, bias2, c.lraw2,
                                       pred_o, st));
    } else {
        const bool int8 = flags & STRATA_INT8;
        STRATA_TRY(launch_prep(x, T, rms, c.xsplit, int8 ? nullptr : c.xperm, c.xexp, st));
        STRATA_TRY(launch_logits(c.xsplit, T, router, bias, c.logits, st));
        STRATA_TRY(launch_topk(c.logits, T, ids_o, w_o, st));
        STRATA_TRY(launch_group(ids_o, T, c.offsets, c.slots, c.active, c.gcount, c.L.max_items,
                                c.mlist, c.nitems, st));
        if (int8)
            STRATA_TRY(launch_prep_i8(x, T, rms, c.x8, c.xs8, c.xn8, st));
    }
    const bool res = flags & STRATA_RESIDUAL;
    if (is_decode(T)) {   // the experts kernel finishes the combine
        hipEvent_t e0, e1;
        take_events(e0, e1);
        STRATA_TRY(launch_decode_experts(blobs, c.erec, c.slots, c.xq, c.hq, c.out, T, c.esync,
                                         c.cdone, w_o, y, res ? x : nullptr,
                                         router2 ? pred_o : nullptr, router2 ? blobs2 : nullptr,
                                         c.status, g_wait_limit.load(), e0, e1, st));
        return STRATA_OK;
    }
    if ((rc = run_experts(c, blobs, c.offsets, c.slots, c.active, c.out, T, st, true,
                          flags & STRATA_INT8)))
        return rc;
    STRATA_TRY(launch_combine(c.out, w_o, T, y, res ? x : nullptr, 0, st));
    return STRATA_OK;
}
} // namespace
} // namespace strata

namespace strata {
namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch[MAX_DEVICES] = {};

// The device address of `scratch` on the current device (looked up once per
// device, with that device current), or NULL on failure.
void *static_scratch()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return nullptr;
        g_scratch[dev] = ptr;
    }
    return g_scratch[dev];
}
} // namespace
} // namespace strata

using namespace strata;

extern "C" {

size_t strata_moe_blob_bytes(void) { return BLOB; }

size_t strata_moe_workspace_bytes(int T)
{
    if (check_T(T) != STRATA_OK)
        return 0;
    return ws_layout(T).total;
}

int strata_moe_route(const float *x, int T, const uint16_t *router, const float *bias,
                     int flags, int32_t *ids, float *w, void *ws, size_t ws_bytes, void *stream)
{
    int rc = check_T(T);
    if (rc)
        return rc;
    if (!x || !router || !ids || !w || (flags & ~(STRATA_RMSNORM | STRATA_RESIDUAL)))
        return STRATA_E_ARG;
    if ((rc = check_ws(ws, ws_bytes, T)))
        return rc;
    if (!aligned(x, 16) || !aligned(router, 16) || !aligned(ids, 4) || !aligned(w, 4) ||
        !aligned(bias, 4))
        return STRATA_E_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    Carve c = carve(ws, T);
    const int rms = flags & STRATA_RMSNORM;
    if (is_decode(T)) {
        STRATA_TRY(launch_route_decode(x, T, router, bias, rms, c.logits, c.xq, false, ids, w, 0,
                                       nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                       nullptr, st));
    } else {
        STRATA_TRY(launch_prep(x, T, rms, c.xsplit, nullptr, nullptr, st));
        STRATA_TRY(launch_logits(c.xsplit, T, router, bias, c.logits, st));
        STRATA_TRY(launch_topk(c.logits, T, ids, w, st));
    }
    return STRATA_OK;
}

int strata_moe_group(const int32_t *ids, int T, int32_t *offsets, int32_t *slots,
                     int32_t *active, void *ws, size_t ws_bytes, void *stream)
{
    int rc = check_T(T);
    if (rc)
        return rc;
    if (!ids || !offsets || !slots || !active)
        return STRATA_E_ARG;
    if ((rc = check_ws(ws, ws_bytes, T)))
        return rc;
    if (!aligned(ids, 4) || !aligned(offsets, 4) || !aligned(slots, 4) || !aligned(active, 4))
        return STRATA_E_ALIGN;
    STRATA_TRY(launch_group(ids, T, offsets, slots, active, carve(ws, T).gcount, 0, nullptr,
                            nullptr, (hipStream_t)stream));
    return STRATA_OK;
}

int strata_moe_experts(const float *x, int T, const uint8_t *blobs, const int32_t *offsets,
                       const int32_t *slots, const int32_t *active, int flags, float *out,
                       void *ws, size_t ws_bytes, void *stream)
{
    int rc = check_T(T);
    if (rc)
        return rc;
    if (!x || !blobs || !offsets || !slots || !active || !out || (flags & ~ALL_FLAGS))
        return STRATA_E_ARG;
    if ((rc = check_ws(ws, ws_bytes, T)))
        return rc;
    if (!aligned(x, 16) || !aligned(blobs, 256) || !aligned(out, 16) || !aligned(offsets, 4) ||
        !aligned(slots, 4) || !aligned(active, 4))
        return STRATA_E_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    Carve c = carve(ws, T);
    const bool int8 = flags & STRATA_INT8;
    if ((rc = run_prep(c, x, T, flags & STRATA_RMSNORM, offsets, slots, active, st, int8)))
        return rc;
    return run_experts(c, blobs, offsets, slots, active, out, T, st, false, int8);
}

int strata_moe_combine(const float *out, const float *w, int T, int flags, float *y,
                       void *stream)
{
    int rc = check_T(T);
    if (rc)
        return rc;
    if (!out || !w || !y || (flags & ~(STRATA_RMSNORM | STRATA_RESIDUAL)))
        return STRATA_E_ARG;
    if (!aligned(out, 16) || !aligned(y, 16) || !aligned(w, 4))
        return STRATA_E_ALIGN;
    STRATA_TRY(launch_combine(out, w, T, y, nullptr, (flags & STRATA_RESIDUAL) ? 1 : 0,
                              (hipStream_t)stream));
    return STRATA_OK;
}

int strata_moe_layer(float *x, int T, const uint16_t *router, const float *bias,
                     const uint8_t *blobs, int flags, float *y, int32_t *ids, float *w,
                     void *ws, size_t ws_bytes, void *stream)
{
    return strata::layer_impl(x, T, router, bias, blobs, flags, y, ids, w, nullptr, nullptr,
                              nullptr, nullptr, nullptr, ws, ws_bytes, stream);
}

static_assert(2 * STRATA_LOOKAHEAD_T_MAX <= strata::DECODE_T_MAX,
              "the routing workgroup has a wave per token for each of the two routers");

int strata_moe_layer_lookahead(float *x, int T, const uint16_t *router, const float *bias,
                               const uint8_t *blobs, int flags, float *y, int32_t *ids, float *w,
                               const uint16_t *router_next, const float *bias_next,
                               const uint8_t *blobs_next, int32_t *pred_ids,
                               const int32_t *hint_ids, void *ws, size_t ws_bytes, void *stream)
{
    if (T < 1 || T > STRATA_LOOKAHEAD_T_MAX)
        return STRATA_E_SHAPE;
    if (!router_next || !blobs_next)
        return STRATA_E_ARG;
    return strata::layer_impl(x, T, router, bias, blobs, flags, y, ids, w, router_next, bias_next,
                              blobs_next, pred_ids, T == 1 ? hint_ids : nullptr, ws, ws_bytes,
                              stream);
}

int strata_moe_time_next_kernel(void *start, void *stop)
{
    if ((start == nullptr) != (stop == nullptr))
        return STRATA_E_ARG;
    t_ev0 = (hipEvent_t)start;
    t_ev1 = (hipEvent_t)stop;
    return STRATA_OK;
}

int strata_moe_read_status(const void *ws, size_t ws_bytes, int32_t *bits, void *stream)
{
    if (!ws || !bits)
        return STRATA_E_ARG;
    if (ws_bytes < WS_STATUS_BYTES)
        return STRATA_E_WORKSPACE;
    if (!aligned(ws, 256))
        return STRATA_E_ALIGN;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
        return STRATA_E_HIP;
    int32_t v = 0;
    if (hipMemcpy(&v, ws, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess)
        return STRATA_E_HIP;
    *bits = v;
    return STRATA_OK;
}

int strata_moe_clear_status(void *ws, size_t ws_bytes, void *stream)
{
    if (!ws)
        return STRATA_E_ARG;
    if (ws_bytes < WS_STATUS_BYTES)
        return STRATA_E_WORKSPACE;
    if (!aligned(ws, 256))
        return STRATA_E_ALIGN;
    hipLaunchKernelGGL(status_clear_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream,
                       static_cast<int32_t *>(ws));
    return hipGetLastError() == hipSuccess ? STRATA_OK : STRATA_E_HIP;
}

int strata_moe_set_wait_limit(int polls)
{
    if (polls < 0)
        return STRATA_E_ARG;
    g_wait_limit.store(polls == 0 ? WAIT_LIMIT_DEFAULT : polls);
    return STRATA_OK;
}


int strata_moe_layer_static(float *x, int T, const uint16_t *router, const float *bias,
                            const uint8_t *blobs, int flags, float *y, int32_t *ids, float *w,
                            void *stream)
{
    if (T < 1 || T > STRATA_STATIC_T_MAX)
        return STRATA_E_SHAPE;
    const size_t need = strata::ws_layout(T).total;
    if (need > STATIC_WS_BYTES)   // cannot happen for T <= STRATA_STATIC_T_MAX
        return STRATA_E_WORKSPACE;
    void *ws = strata::static_scratch();
    if (!ws)
        return STRATA_E_HIP;
    return strata::layer_impl(x, T, router, bias, blobs, flags, y, ids, w, nullptr, nullptr,
                              nullptr, nullptr, nullptr, ws, STATIC_WS_BYTES, stream);
}

const char *strata_moe_status_string(int status)
{
    switch (status) {
    case STRATA_OK:
        return "ok";
    case STRATA_E_ARG:
        return "invalid argument (NULL pointer or unknown flag)";
    case STRATA_E_SHAPE:
        return "T outside 1..8192";
    case STRATA_E_WORKSPACE:
        return "workspace missing or too small";
    case STRATA_E_HIP:
        return "HIP launch error";
    case STRATA_E_ALIGN:
        return "pointer alignment violated";
    case STRATA_E_CORRUPT:
        return "a blob differs from its expected checksum";
    default:
        return "unknown status";
    }
}

} // extern "C"
