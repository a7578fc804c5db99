// Context, error reporting, allocation and tiled-matrix lifecycle of libgpex.
#include <cstring>
#include <mutex>

#include "common.h"

namespace gpex {

// Scratch memory of the allocation-free entry points: one fixed array per GPU, held from the
// library's load until the process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: its device address is looked up once per device (gpex_ctx_create, with the
// device current) and only that address is handed to kernels.  Every call on a GPU shares that
// GPU's array, so such calls that overlap on one GPU race.
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];
constexpr int MAX_DEVICES = 64;
static void* g_scratch[MAX_DEVICES] = {};
static std::mutex g_scratch_mu;

static int scratch_lookup(int device) {
    if (device >= MAX_DEVICES) return GPEX_OK;   // such a device simply has no scratch
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch[device]) return GPEX_OK;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return GPEX_ERR_HIP;
    }
    g_scratch[device] = p;
    return GPEX_OK;
}

void* scratch_ptr(int device) {
    if (device < 0 || device >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    return g_scratch[device];
}

int set_err(gpex_ctx_t ctx, int code, const std::string& msg) {
    if (ctx) ctx->err = msg;
    return code;
}

static void* raw_alloc(void* (*alloc)(size_t, void*), void* user, size_t bytes) {
    if (alloc) return alloc(bytes, user);
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    return p;
}

static void raw_free(void (*dealloc)(void*, void*), void* user, void* p) {
    if (!p) return;
    if (dealloc) dealloc(p, user);
    else (void)hipFree(p);
}

static int nomem(gpex_ctx_t ctx, const char* what, size_t bytes) {
    return set_err(ctx, GPEX_ERR_NOMEM,
                   std::string("device allocation failed (") + what + ", " + std::to_string(bytes) + " bytes)");
}

int dev_alloc(gpex_ctx_t ctx, void** p, size_t bytes, const char* what) {
    if (bytes == 0) bytes = 256;
    *p = raw_alloc(ctx->alloc, ctx->user, bytes);
    return *p ? GPEX_OK : nomem(ctx, what, bytes);
}

void dev_free(gpex_ctx_t ctx, void* p) { raw_free(ctx->dealloc, ctx->user, p); }

int tiled_alloc(gpex_ctx_t ctx, gpex_tiled_t t, void** p, size_t bytes, const char* what) {
    if (bytes == 0) bytes = 256;
    *p = raw_alloc(t->alloc, t->user, bytes);
    return *p ? GPEX_OK : nomem(ctx, what, bytes);
}

void tiled_free(gpex_tiled_t t, void* p) { raw_free(t->dealloc, t->user, p); }

int ws_get(gpex_ctx_t ctx, int slot, size_t bytes, void** out, const char* what) {
    auto& w = ctx->ws[slot];
    if (w.bytes < bytes) {
        // the old buffer's last users are ordered before this point on the context stream: a
        // stream-ordered allocator may hand it out again, hipFree waits for the device
        dev_free(ctx, w.p);
        w.p = nullptr;
        w.bytes = 0;
        const size_t grown = (bytes + (2u << 20) - 1) / (2u << 20) * (2u << 20);   // 2 MiB granules
        GPEX_TRY(dev_alloc(ctx, &w.p, grown, what));
        w.bytes = grown;
    }
    *out = w.p;
    return GPEX_OK;
}

int ctx_event(gpex_ctx_t ctx, size_t i, hipEvent_t* out) {
    while (ctx->events.size() <= i) {
        hipEvent_t e;
        GPEX_HIP(ctx, hipEventCreateWithFlags(&e, hipEventDisableTiming));
        ctx->events.push_back(e);
    }
    *out = ctx->events[i];
    return GPEX_OK;
}

int ctx_timing_event(gpex_ctx_t ctx, size_t i, hipEvent_t* out) {
    while (ctx->tevents.size() <= i) {
        hipEvent_t e;
        GPEX_HIP(ctx, hipEventCreate(&e));
        ctx->tevents.push_back(e);
    }
    *out = ctx->tevents[i];
    return GPEX_OK;
}

}  // namespace gpex

using namespace gpex;

extern "C" const char* gpex_version(void) { return "gpex 0.1 (gfx950)"; }

extern "C" int gpex_ctx_create(int device, void* hip_stream, void* (*alloc)(size_t, void*),
                               void (*dealloc)(void*, void*), void* user, gpex_ctx_t* out) {
    if (!out) return GPEX_ERR_ARG;
    *out = nullptr;
    if ((alloc == nullptr) != (dealloc == nullptr)) return GPEX_ERR_ARG;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) return GPEX_ERR_ARG;
    if (hipSetDevice(device) != hipSuccess) return GPEX_ERR_HIP;
    if (scratch_lookup(device) != GPEX_OK) return GPEX_ERR_HIP;
    auto* c = new gpex_ctx_s();
    c->device = device;
    c->stream = static_cast<hipStream_t>(hip_stream);
    c->alloc = alloc;
    c->dealloc = dealloc;
    c->user = user;
    if (dev_alloc(c, (void**)&c->d_flags, sizeof(long long) * FLAG_COUNT, "flags") != GPEX_OK) {
        delete c;
        return GPEX_ERR_NOMEM;
    }
    if (hipMemsetAsync(c->d_flags, 0, sizeof(long long) * FLAG_COUNT, c->stream) != hipSuccess ||
        hipStreamSynchronize(c->stream) != hipSuccess ||
        hipHostMalloc((void**)&c->h_ret, sizeof(long long) * (FLAG_COUNT + 1), hipHostMallocDefault) != hipSuccess) {
        dev_free(c, c->d_flags);
        delete c;
        return GPEX_ERR_HIP;
    }
    *out = c;
    return GPEX_OK;
}

static void release_workspace(gpex_ctx_t ctx) {
    for (auto& w : ctx->ws) {
        dev_free(ctx, w.p);
        w.p = nullptr;
        w.bytes = 0;
    }
}

extern "C" int gpex_ctx_release_workspace(gpex_ctx_t ctx) {
    if (!ctx) return GPEX_ERR_ARG;
    GPEX_HIP(ctx, hipSetDevice(ctx->device));
    GPEX_HIP(ctx, hipStreamSynchronize(ctx->stream));
    release_workspace(ctx);
    return GPEX_OK;
}

extern "C" int gpex_ctx_destroy(gpex_ctx_t ctx) {
    if (!ctx) return GPEX_ERR_ARG;
    (void)hipSetDevice(ctx->device);
    (void)hipStreamSynchronize(ctx->stream);
    if (ctx->side) (void)hipStreamSynchronize(ctx->side);
    if (ctx->ahead) (void)hipStreamSynchronize(ctx->ahead);
    release_workspace(ctx);
    dev_free(ctx, ctx->d_flags);
    if (ctx->side) (void)hipStreamDestroy(ctx->side);
    if (ctx->ahead) (void)hipStreamDestroy(ctx->ahead);
    if (ctx->side_fork) (void)hipEventDestroy(ctx->side_fork);
    if (ctx->side_join) (void)hipEventDestroy(ctx->side_join);
    for (auto e : ctx->events) (void)hipEventDestroy(e);
    for (auto e : ctx->tevents) (void)hipEventDestroy(e);
    if (ctx->h_ret) (void)hipHostFree(ctx->h_ret);
    delete ctx;
    return GPEX_OK;
}

extern "C" int gpex_ctx_set_serial(gpex_ctx_t ctx, int on) {
    if (!ctx) return GPEX_ERR_ARG;
    ctx->serial = on != 0;
    return GPEX_OK;
}

extern "C" const char* gpex_last_error(gpex_ctx_t ctx) { return ctx ? ctx->err.c_str() : "null context"; }

extern "C" int gpex_ctx_set_timing(gpex_ctx_t ctx, int on) {
    if (!ctx) return GPEX_ERR_ARG;
    ctx->timing = on != 0;
    return GPEX_OK;
}

extern "C" int gpex_ctx_timings(gpex_ctx_t ctx, double* out) {
    if (!ctx || !out) return GPEX_ERR_ARG;
    for (int i = 0; i < 32; ++i) out[i] = ctx->timings[i];
    return GPEX_OK;
}

extern "C" int gpex_plan(const double* h_stats, int64_t nt, const gpex_prec_opts* opts, uint8_t* h_map,
                         gpex_diag* diag) {
    if (!h_stats || nt < 1 || !opts || !h_map) return GPEX_ERR_ARG;
    std::vector<double> st(h_stats, h_stats + 3 * nt * (nt + 1) / 2);
    std::vector<uint8_t> map;
    gpex_diag d{};
    plan_precision(st, nt, *opts, map, d);
    std::memcpy(h_map, map.data(), map.size());
    if (diag) *diag = d;
    return GPEX_OK;
}

extern "C" int gpex_tiled_info(gpex_tiled_t t, int64_t* n, int* nb, int64_t* nt, uint8_t* h_map, double* s) {
    if (!t) return GPEX_ERR_ARG;
    if (n) *n = t->n;
    if (nb) *nb = t->nb;
    if (nt) *nt = t->nt;
    if (h_map) std::memcpy(h_map, t->map.data(), t->map.size());
    if (s) *s = t->s;
    return GPEX_OK;
}

extern "C" int gpex_tiled_stats(gpex_tiled_t t, double* h_stats) {
    if (!t || !h_stats) return GPEX_ERR_ARG;
    std::memcpy(h_stats, t->stats.data(), sizeof(double) * t->stats.size());
    return GPEX_OK;
}

extern "C" int gpex_tiled_destroy(gpex_tiled_t t) {
    if (!t) return GPEX_ERR_ARG;
    (void)hipSetDevice(t->device);
    // a stream-ordered allocator orders the reuse after the queued work on the context stream;
    // hipFree waits for the device by itself
    tiled_free(t, t->base);
    tiled_free(t, t->tinv);
    tiled_free(t, t->l16);
    delete t;
    return GPEX_OK;
}
