// Context, error reporting, allocation and tiled-matrix lifecycle of libgpex.
#include <cstring>

#include "common.h"

namespace gpex {

int set_err(gpex_ctx_t ctx, int code, const std::string& msg) {
    if (ctx) ctx->err = msg;
    return code;
}

int dev_alloc(gpex_ctx_t ctx, void** p, size_t bytes, const char* what) {
    *p = nullptr;
    if (bytes == 0) bytes = 256;
    hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        *p = nullptr;
        return set_err(ctx, GPEX_ERR_NOMEM,
                       std::string("device allocation failed (") + what + ", " + std::to_string(bytes) + " bytes)");
    }
    return GPEX_OK;
}

void dev_free(void* p) {
    if (p) (void)hipFree(p);
}

}  // namespace gpex

using namespace gpex;

extern "C" const char* gpex_version(void) { return "gpex 0.1 (gfx950)"; }

extern "C" int gpex_ctx_create(int device, void* hip_stream, gpex_ctx_t* out) {
    if (!out) return GPEX_ERR_ARG;
    *out = nullptr;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) return GPEX_ERR_ARG;
    if (hipSetDevice(device) != hipSuccess) return GPEX_ERR_HIP;
    auto* c = new gpex_ctx_s();
    c->device = device;
    c->stream = static_cast<hipStream_t>(hip_stream);
    if (hipMalloc(&c->d_flags, sizeof(long long) * FLAG_COUNT) != hipSuccess) {
        delete c;
        return GPEX_ERR_NOMEM;
    }
    if (hipMemset(c->d_flags, 0, sizeof(long long) * FLAG_COUNT) != hipSuccess) {
        (void)hipFree(c->d_flags);
        delete c;
        return GPEX_ERR_HIP;
    }
    *out = c;
    return GPEX_OK;
}

extern "C" int gpex_ctx_destroy(gpex_ctx_t ctx) {
    if (!ctx) return GPEX_ERR_ARG;
    (void)hipSetDevice(ctx->device);
    if (ctx->stream) (void)hipStreamSynchronize(ctx->stream);
    else (void)hipDeviceSynchronize();
    dev_free(ctx->d_flags);
    dev_free(ctx->sim_ws);
    if (ctx->side) {
        (void)hipStreamSynchronize(ctx->side);
        (void)hipStreamDestroy(ctx->side);
    }
    if (ctx->side_fork) (void)hipEventDestroy(ctx->side_fork);
    if (ctx->side_join) (void)hipEventDestroy(ctx->side_join);
    delete ctx;
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
    for (int i = 0; i < 16; ++i) out[i] = ctx->timings[i];
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
    (void)hipDeviceSynchronize();
    dev_free(t->base);
    dev_free(t->tinv);
    dev_free(t->l16);
    delete t;
    return GPEX_OK;
}
