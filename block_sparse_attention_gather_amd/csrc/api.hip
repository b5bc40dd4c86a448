// C ABI of libbsa: argument validation, workspace sizing, per-device cache, error strings.
// Every entry point validates on the host before enqueuing anything; no entry point
// allocates device memory or synchronizes the stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "bsa_internal.h"

#define BSA_VERSION_STRING "libbsa 0.1.0 (gfx950)"

namespace bsa {

static thread_local char g_err[512] = "";

bsa_status fail(bsa_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

bsa_status check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(BSA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return BSA_OK;
}

// per-device properties, filled once per device ordinal
static std::mutex g_dev_mu;
static DeviceInfo g_dev[64];
static bool g_dev_ok[64];

bsa_status device_info(DeviceInfo* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(BSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(BSA_ERR_HIP, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (!g_dev_ok[dev]) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess || cus <= 0)
            return fail(BSA_ERR_HIP, "device %d CU count: %s", dev, hipGetErrorString(e));
        g_dev[dev].device = dev;
        g_dev[dev].cu_count = cus;
        g_dev_ok[dev] = true;
    }
    *out = g_dev[dev];
    return BSA_OK;
}

// ---- shared validation ------------------------------------------------------------------
static bsa_status geometry(const bsa_grid* grid, Geometry* g) {
    if (!grid) return fail(BSA_ERR_INVALID_ARG, "grid is NULL");
    if (grid->T < 1 || grid->H < 1 || grid->W < 1)
        return fail(BSA_ERR_INVALID_ARG, "grid T, H, W must be >= 1 (got %d, %d, %d)", grid->T,
                    grid->H, grid->W);
    if (grid->tile_t < 1 || grid->tile_h < 1 || grid->tile_w < 1)
        return fail(BSA_ERR_INVALID_ARG, "tile extents must be >= 1");
    if (grid->block < 1) return fail(BSA_ERR_INVALID_ARG, "block must be >= 1");
    g->T = grid->T; g->H = grid->H; g->W = grid->W;
    g->tt = grid->tile_t; g->th = grid->tile_h; g->tw = grid->tile_w;
    g->B = grid->block;
    g->order = grid->order;
    if ((uintptr_t)grid->order & 3) return fail(BSA_ERR_INVALID_ARG, "grid order must be 4-byte aligned");
    g->N = (int64_t)grid->T * grid->H * grid->W;
    if (g->N > ((int64_t)1 << 31) - 1) return fail(BSA_ERR_INVALID_ARG, "N = T*H*W exceeds int32");
    const int64_t nb = (g->N + g->B - 1) / g->B;
    g->n_blk = (int32_t)nb;
    g->Npad = nb * g->B;
    return BSA_OK;
}

static bsa_status check_shape(const bsa_shape* s) {
    if (!s) return fail(BSA_ERR_INVALID_ARG, "shape is NULL");
    if (s->batch < 1 || s->heads < 1 || s->head_dim < 1)
        return fail(BSA_ERR_INVALID_ARG, "batch, heads, head_dim must be >= 1");
    return BSA_OK;
}

static bsa_status check_kernel_dims(const bsa_shape* s, const Geometry& g) {
    if (s->head_dim != 64 && s->head_dim != 128)
        return fail(BSA_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", s->head_dim);
    if (g.B != 64 && g.B != 128)
        return fail(BSA_ERR_UNSUPPORTED, "block %d unsupported (64 or 128)", g.B);
    if ((int64_t)s->batch * s->heads > attn_max_heads())
        return fail(BSA_ERR_UNSUPPORTED, "batch*heads %lld exceeds %d",
                    (long long)s->batch * s->heads, attn_max_heads());
    if (g.n_blk > attn_max_blocks())
        return fail(BSA_ERR_UNSUPPORTED, "n_blk %d exceeds %d", g.n_blk, attn_max_blocks());
    const int64_t rows = (int64_t)s->batch * s->heads * g.n_blk;
    if (rows * g.n_blk > ((int64_t)1 << 31) - 1)
        return fail(BSA_ERR_UNSUPPORTED, "rows*n_blk exceeds int32 CSR capacity");
    if ((int64_t)s->batch * s->heads * g.Npad * s->head_dim > ((int64_t)1 << 40))
        return fail(BSA_ERR_UNSUPPORTED, "tensor too large");
    return BSA_OK;
}

}  // namespace bsa

using namespace bsa;

extern "C" {

int32_t bsa_num_blocks(const bsa_grid* grid) {
    Geometry g;
    if (geometry(grid, &g) != BSA_OK) return 0;
    return g.n_blk;
}

int32_t bsa_padded_len(const bsa_grid* grid) {
    Geometry g;
    if (geometry(grid, &g) != BSA_OK) return 0;
    return g.Npad > INT32_MAX ? 0 : (int32_t)g.Npad;
}

bsa_status bsa_reorder(const void* src, void* dst, const bsa_shape* shape, const bsa_grid* grid,
                       int32_t inverse, void* stream) {
    Geometry g;
    bsa_status st = geometry(grid, &g);
    if (st != BSA_OK) return st;
    if ((st = check_shape(shape)) != BSA_OK) return st;
    if (!src || !dst) return fail(BSA_ERR_INVALID_ARG, "src/dst is NULL");
    if (shape->head_dim % 8 != 0 || shape->head_dim > 1024)
        return fail(BSA_ERR_UNSUPPORTED, "reorder head_dim must be a multiple of 8 in [8, 1024]");
    if (((uintptr_t)src | (uintptr_t)dst) & 15)
        return fail(BSA_ERR_INVALID_ARG, "src/dst must be 16-byte aligned");
    const int64_t elems_src = (int64_t)shape->batch * shape->heads * (inverse ? g.Npad : g.N) *
                              shape->head_dim * 2;
    const int64_t elems_dst = (int64_t)shape->batch * shape->heads * (inverse ? g.N : g.Npad) *
                              shape->head_dim * 2;
    const char* s0 = (const char*)src;
    const char* d0 = (const char*)dst;
    if (s0 < d0 + elems_dst && d0 < s0 + elems_src)
        return fail(BSA_ERR_INVALID_ARG, "src and dst overlap");
    return launch_reorder(src, dst, shape->batch, shape->heads, shape->head_dim, g, inverse,
                          (hipStream_t)stream);
}

static bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    if (!a || !b) return false;
    const char* x = (const char*)a;
    const char* y = (const char*)b;
    return x < y + nb && y < x + na;
}

bsa_status bsa_reorder_pool(const void* src, void* dst, double* pooled, void* x8,
                            float* x8_scales, const bsa_shape* shape, const bsa_grid* grid,
                            void* stream) {
    Geometry g;
    bsa_status st = geometry(grid, &g);
    if (st != BSA_OK) return st;
    if ((st = check_shape(shape)) != BSA_OK) return st;
    if (!src) return fail(BSA_ERR_INVALID_ARG, "src is NULL");
    if ((x8 == nullptr) != (x8_scales == nullptr))
        return fail(BSA_ERR_INVALID_ARG, "x8 and x8_scales must be both NULL or both set");
    if (!dst && !pooled && !x8) return fail(BSA_ERR_INVALID_ARG, "no output requested");
    if ((st = check_kernel_dims(shape, g)) != BSA_OK) return st;
    if (x8 && (shape->head_dim != 128 || g.B != 128))
        return fail(BSA_ERR_UNSUPPORTED, "the FP8 path is built for head_dim 128 and block 128");
    if (((uintptr_t)src | (uintptr_t)dst | (uintptr_t)x8) & 15)
        return fail(BSA_ERR_INVALID_ARG, "src/dst/x8 must be 16-byte aligned");
    if (((uintptr_t)pooled & 7) || ((uintptr_t)x8_scales & 3))
        return fail(BSA_ERR_INVALID_ARG, "pooled must be 8-byte and x8_scales 4-byte aligned");
    const int64_t bh = (int64_t)shape->batch * shape->heads;
    const int64_t n_src = bh * g.N * shape->head_dim * 2;
    const int64_t n_dst = bh * g.Npad * shape->head_dim * 2;
    const int64_t n_pool = bh * g.n_blk * shape->head_dim * 8;
    const int64_t n_x8 = n_dst / 2, n_sc = bh * g.n_blk * 4;
    const void* bufs[5] = {src, dst, pooled, x8, x8_scales};
    const int64_t lens[5] = {n_src, n_dst, n_pool, n_x8, n_sc};
    for (int i = 0; i < 5; ++i)
        for (int k = i + 1; k < 5; ++k)
            if (overlap(bufs[i], lens[i], bufs[k], lens[k]))
                return fail(BSA_ERR_INVALID_ARG, "src, dst, pooled, x8 and x8_scales must not overlap");
    return launch_reorder_pool(src, dst, pooled, x8, x8_scales, shape->batch, shape->heads,
                               shape->head_dim, g, (hipStream_t)stream);
}

bsa_status bsa_reorder_quantize_v(const void* src, void* dst, void* v8, float* v_scales,
                                  const bsa_shape* shape, const bsa_grid* grid, void* stream) {
    Geometry g;
    bsa_status st = geometry(grid, &g);
    if (st != BSA_OK) return st;
    if ((st = check_shape(shape)) != BSA_OK) return st;
    if (!src || !v8 || !v_scales) return fail(BSA_ERR_INVALID_ARG, "src/v8/v_scales is NULL");
    if ((st = check_kernel_dims(shape, g)) != BSA_OK) return st;
    if (shape->head_dim != 128 || g.B != 128)
        return fail(BSA_ERR_UNSUPPORTED, "the FP8 path is built for head_dim 128 and block 128");
    if (((uintptr_t)src | (uintptr_t)dst | (uintptr_t)v8) & 15)
        return fail(BSA_ERR_INVALID_ARG, "src/dst/v8 must be 16-byte aligned");
    if ((uintptr_t)v_scales & 3) return fail(BSA_ERR_INVALID_ARG, "v_scales must be 4-byte aligned");
    const int64_t bh = (int64_t)shape->batch * shape->heads;
    const int64_t n_src = bh * g.N * 256, n_dst = bh * g.Npad * 256;
    const void* bufs[4] = {src, dst, v8, v_scales};
    const int64_t lens[4] = {n_src, n_dst, n_dst / 2, bh * 4};
    for (int i = 0; i < 4; ++i)
        for (int k = i + 1; k < 4; ++k)
            if (overlap(bufs[i], lens[i], bufs[k], lens[k]))
                return fail(BSA_ERR_INVALID_ARG, "src, dst, v8 and v_scales must not overlap");
    return launch_reorder_quant_v(src, dst, v8, v_scales, shape->batch, shape->heads, g,
                                  (hipStream_t)stream);
}

size_t bsa_route_workspace_bytes(const bsa_shape* shape, const bsa_grid* grid) {
    Geometry g;
    if (geometry(grid, &g) != BSA_OK || check_shape(shape) != BSA_OK) return 0;
    return route_ws_bytes(shape->batch, shape->heads, shape->head_dim, g);
}

bsa_status bsa_score_and_route(const void* q_t, const void* k_t, const bsa_shape* shape,
                               const bsa_grid* grid, double top_p, int32_t k_floor,
                               double scale, int32_t* row_ptr, int32_t* col_idx, int32_t* nnz,
                               double* block_scores, void* ws, size_t ws_bytes, void* stream) {
    Geometry g;
    bsa_status st = geometry(grid, &g);
    if (st != BSA_OK) return st;
    if ((st = check_shape(shape)) != BSA_OK) return st;
    if (!q_t || !k_t || !row_ptr || !col_idx || !nnz)
        return fail(BSA_ERR_INVALID_ARG, "q_t, k_t, row_ptr, col_idx and nnz must be non-NULL");
    if (!(top_p >= 0.0 && top_p <= 1.0))
        return fail(BSA_ERR_INVALID_ARG, "top_p must lie in [0, 1] (got %g)", top_p);
    if (k_floor < 1) return fail(BSA_ERR_INVALID_ARG, "k_floor must be >= 1 (got %d)", k_floor);
    if (!isfinite(scale)) return fail(BSA_ERR_INVALID_ARG, "scale must be finite");
    if ((st = check_kernel_dims(shape, g)) != BSA_OK) return st;
    if ((((uintptr_t)q_t | (uintptr_t)k_t) & 15))
        return fail(BSA_ERR_INVALID_ARG, "q_t/k_t must be 16-byte aligned");
    const size_t need = route_ws_bytes(shape->batch, shape->heads, shape->head_dim, g);
    if (!ws || ws_bytes < need || ((uintptr_t)ws & 255))
        return fail(BSA_ERR_WORKSPACE, "route workspace: need %zu bytes, 256-byte aligned", need);
    return launch_route(q_t, k_t, shape->batch, shape->heads, shape->head_dim, g, top_p, k_floor,
                        scale, row_ptr, col_idx, nnz, block_scores, ws, (hipStream_t)stream);
}

bsa_status bsa_route_pooled(const double* qbar, const double* kbar, const bsa_shape* shape,
                            const bsa_grid* grid, double top_p, int32_t k_floor, double scale,
                            int32_t* row_ptr, int32_t* col_idx, int32_t* nnz,
                            double* block_scores, void* ws, size_t ws_bytes, void* stream) {
    Geometry g;
    bsa_status st = geometry(grid, &g);
    if (st != BSA_OK) return st;
    if ((st = check_shape(shape)) != BSA_OK) return st;
    if (!qbar || !kbar || !row_ptr || !col_idx || !nnz)
        return fail(BSA_ERR_INVALID_ARG, "qbar, kbar, row_ptr, col_idx and nnz must be non-NULL");
    if (!(top_p >= 0.0 && top_p <= 1.0))
        return fail(BSA_ERR_INVALID_ARG, "top_p must lie in [0, 1] (got %g)", top_p);
    if (k_floor < 1) return fail(BSA_ERR_INVALID_ARG, "k_floor must be >= 1 (got %d)", k_floor);
    if (!isfinite(scale)) return fail(BSA_ERR_INVALID_ARG, "scale must be finite");
    if ((st = check_kernel_dims(shape, g)) != BSA_OK) return st;
    if ((((uintptr_t)qbar | (uintptr_t)kbar) & 15))
        return fail(BSA_ERR_INVALID_ARG, "qbar/kbar must be 16-byte aligned");
    const size_t need = route_ws_bytes(shape->batch, shape->heads, shape->head_dim, g);
    if (!ws || ws_bytes < need || ((uintptr_t)ws & 255))
        return fail(BSA_ERR_WORKSPACE, "route workspace: need %zu bytes, 256-byte aligned", need);
    return launch_route_pooled(qbar, kbar, shape->batch, shape->heads, shape->head_dim, g, top_p,
                               k_floor, scale, row_ptr, col_idx, nnz, block_scores, ws,
                               (hipStream_t)stream);
}

size_t bsa_stripe_workspace_bytes(const bsa_shape* shape, const bsa_grid* grid) {
    Geometry g;
    if (geometry(grid, &g) != BSA_OK || check_shape(shape) != BSA_OK) return 0;
    return stripe_ws_bytes(shape->batch, shape->heads, g);
}

bsa_status bsa_stripe_mask(const bsa_stripe* params, const bsa_shape* shape,
                           const bsa_grid* grid, int32_t* row_ptr, int32_t* col_idx,
                           int32_t* nnz, void* ws, size_t ws_bytes, void* stream) {
    Geometry g;
    bsa_status st = geometry(grid, &g);
    if (st != BSA_OK) return st;
    if ((st = check_shape(shape)) != BSA_OK) return st;
    if (!params || !row_ptr || !col_idx || !nnz)
        return fail(BSA_ERR_INVALID_ARG, "params, row_ptr, col_idx and nnz must be non-NULL");
    for (int32_t h = 0; h < shape->heads; ++h) {
        const bsa_stripe& m = params[h];
        if (!(m.Tw >= 1 && m.Tw <= m.Ts && m.Sw >= 1 && m.Sw <= m.Ss))
            return fail(BSA_ERR_INVALID_ARG,
                        "stripe parameters of head %d need 1 <= Tw <= Ts and 1 <= Sw <= Ss", h);
    }
    if ((st = check_kernel_dims(shape, g)) != BSA_OK) return st;
    const size_t need = stripe_ws_bytes(shape->batch, shape->heads, g);
    if (!ws || ws_bytes < need || ((uintptr_t)ws & 255))
        return fail(BSA_ERR_WORKSPACE, "stripe workspace: need %zu bytes, 256-byte aligned", need);
    return launch_stripe((const int32_t*)params, shape->batch, shape->heads, g, row_ptr, col_idx,
                         nnz, ws, (hipStream_t)stream);
}

static bsa_status check_fp8_dims(const bsa_shape* shape, const Geometry& g) {
    bsa_status st = check_kernel_dims(shape, g);
    if (st != BSA_OK) return st;
    if (shape->head_dim != 128 || g.B != 128)
        return fail(BSA_ERR_UNSUPPORTED, "the FP8 path is built for head_dim 128 and block 128");
    return BSA_OK;
}

bsa_status bsa_quantize_fp8(const void* x_t, void* x8, float* scales, int32_t v_layout,
                            const bsa_shape* shape, const bsa_grid* grid, void* stream) {
    Geometry g;
    bsa_status st = geometry(grid, &g);
    if (st != BSA_OK) return st;
    if ((st = check_shape(shape)) != BSA_OK) return st;
    if (!x_t || !x8 || !scales) return fail(BSA_ERR_INVALID_ARG, "x_t/x8/scales is NULL");
    if (v_layout != 0 && v_layout != 1)
        return fail(BSA_ERR_INVALID_ARG, "v_layout must be 0 (Q, K) or 1 (V)");
    if ((st = check_fp8_dims(shape, g)) != BSA_OK) return st;
    if (((uintptr_t)x_t | (uintptr_t)x8) & 15)
        return fail(BSA_ERR_INVALID_ARG, "x_t/x8 must be 16-byte aligned");
    if ((uintptr_t)scales & 3) return fail(BSA_ERR_INVALID_ARG, "scales must be 4-byte aligned");
    const int64_t n_src = (int64_t)shape->batch * shape->heads * g.Npad * shape->head_dim * 2;
    const int64_t n_dst = n_src / 2;
    const char* s0 = (const char*)x_t;
    const char* d0 = (const char*)x8;
    if (s0 < d0 + n_dst && d0 < s0 + n_src) return fail(BSA_ERR_INVALID_ARG, "x_t and x8 overlap");
    return launch_quant_fp8(x_t, x8, scales, v_layout, shape->batch, shape->heads, g,
                            (hipStream_t)stream);
}

size_t bsa_attn_fp8_workspace_bytes(const bsa_shape* shape, const bsa_grid* grid) {
    Geometry g;
    if (geometry(grid, &g) != BSA_OK || check_shape(shape) != BSA_OK) return 0;
    if (check_fp8_dims(shape, g) != BSA_OK) return 0;
    DeviceInfo dev;
    if (device_info(&dev) != BSA_OK) return 0;
    return attn_ws_bytes(shape->batch, shape->heads, shape->head_dim, g, attn_fp8_slots(dev));
}

bsa_status bsa_sparse_attn_fwd_fp8(const void* q8, const float* q_scale, const void* k8,
                                   const float* k_scale, const void* v8, const float* v_scale,
                                   const int32_t* row_ptr, const int32_t* col_idx,
                                   const bsa_shape* shape, const bsa_grid* grid, float scale,
                                   int32_t expcast, void* out_t, float* lse, void* ws,
                                   size_t ws_bytes, void* stream) {
    Geometry g;
    bsa_status st = geometry(grid, &g);
    if (st != BSA_OK) return st;
    if ((st = check_shape(shape)) != BSA_OK) return st;
    if (expcast != 0 && expcast != 1) return fail(BSA_ERR_INVALID_ARG, "expcast must be 0 or 1");
    if (!q8 || !q_scale || !k8 || !k_scale || !v8 || !v_scale || !row_ptr || !col_idx || !out_t)
        return fail(BSA_ERR_INVALID_ARG, "every pointer except lse must be non-NULL");
    if (!(scale > 0.f) || !isfinite(scale))
        return fail(BSA_ERR_INVALID_ARG, "scale must be finite and positive");
    if ((st = check_fp8_dims(shape, g)) != BSA_OK) return st;
    if (((uintptr_t)q8 | (uintptr_t)k8 | (uintptr_t)v8 | (uintptr_t)out_t) & 15)
        return fail(BSA_ERR_INVALID_ARG, "q8/k8/v8/out_t must be 16-byte aligned");
    DeviceInfo dev;
    if ((st = device_info(&dev)) != BSA_OK) return st;
    const size_t need =
        attn_ws_bytes(shape->batch, shape->heads, shape->head_dim, g, attn_fp8_slots(dev));
    if (!ws || ws_bytes < need || ((uintptr_t)ws & 255))
        return fail(BSA_ERR_WORKSPACE, "fp8 attention workspace: need %zu bytes, 256-byte aligned",
                    need);
    return launch_attn_fp8(q8, q_scale, k8, k_scale, v8, v_scale, row_ptr, col_idx,
                           shape->batch, shape->heads, g, scale, expcast, out_t, lse, ws,
                           dev, (hipStream_t)stream);
}

size_t bsa_hilbert_order_workspace_bytes(const bsa_grid* grid) {
    Geometry g;
    if (geometry(grid, &g) != BSA_OK) return 0;
    return hilbert_ws_bytes(g);
}

bsa_status bsa_hilbert_order(const bsa_grid* grid, int32_t* order, void* ws, size_t ws_bytes,
                             void* stream) {
    Geometry g;
    bsa_status st = geometry(grid, &g);
    if (st != BSA_OK) return st;
    if (!order) return fail(BSA_ERR_INVALID_ARG, "order is NULL");
    if ((uintptr_t)order & 3) return fail(BSA_ERR_INVALID_ARG, "order must be 4-byte aligned");
    if (g.order && (const int32_t*)order == g.order)
        return fail(BSA_ERR_INVALID_ARG, "order must not be the grid's own order table");
    int32_t side = 1;
    while (side < g.T || side < g.H || side < g.W) side <<= 1;
    if (side > 256) return fail(BSA_ERR_UNSUPPORTED, "the Hilbert order supports axes up to 256");
    const size_t need = hilbert_ws_bytes(g);
    if (!ws || ws_bytes < need || ((uintptr_t)ws & 255))
        return fail(BSA_ERR_WORKSPACE, "hilbert workspace: need %zu bytes, 256-byte aligned", need);
    return launch_hilbert_order(g, order, ws, (hipStream_t)stream);
}

size_t bsa_attn_workspace_bytes(const bsa_shape* shape, const bsa_grid* grid) {
    Geometry g;
    if (geometry(grid, &g) != BSA_OK || check_shape(shape) != BSA_OK) return 0;
    if (check_kernel_dims(shape, g) != BSA_OK) return 0;
    DeviceInfo dev;
    if (device_info(&dev) != BSA_OK) return 0;
    return attn_ws_bytes(shape->batch, shape->heads, shape->head_dim, g,
                         attn_slots(shape->head_dim, g.B, dev));
}

bsa_status bsa_sparse_attn_fwd(const void* q_t, const void* k_t, const void* v_t,
                               const int32_t* row_ptr, const int32_t* col_idx,
                               const bsa_shape* shape, const bsa_grid* grid, float scale,
                               void* out_t, float* lse, void* ws, size_t ws_bytes,
                               void* stream) {
    Geometry g;
    bsa_status st = geometry(grid, &g);
    if (st != BSA_OK) return st;
    if ((st = check_shape(shape)) != BSA_OK) return st;
    if (!q_t || !k_t || !v_t || !row_ptr || !col_idx || !out_t)
        return fail(BSA_ERR_INVALID_ARG, "q_t, k_t, v_t, row_ptr, col_idx, out_t must be non-NULL");
    if (!(scale > 0.f) || !isfinite(scale))
        return fail(BSA_ERR_INVALID_ARG, "scale must be finite and positive");
    if ((st = check_kernel_dims(shape, g)) != BSA_OK) return st;
    if ((((uintptr_t)q_t | (uintptr_t)k_t | (uintptr_t)v_t | (uintptr_t)out_t) & 15))
        return fail(BSA_ERR_INVALID_ARG, "q_t/k_t/v_t/out_t must be 16-byte aligned");
    DeviceInfo dev;
    if ((st = device_info(&dev)) != BSA_OK) return st;
    const size_t need = attn_ws_bytes(shape->batch, shape->heads, shape->head_dim, g,
                                      attn_slots(shape->head_dim, g.B, dev));
    if (!ws || ws_bytes < need || ((uintptr_t)ws & 255))
        return fail(BSA_ERR_WORKSPACE, "attention workspace: need %zu bytes, 256-byte aligned",
                    need);
    return launch_attn(q_t, k_t, v_t, row_ptr, col_idx, shape->batch, shape->heads,
                       shape->head_dim, g, scale, out_t, lse, ws, dev, (hipStream_t)stream);
}

bsa_status bsa_sparse_attn_fwd_noalloc(const void* q_t, const void* k_t, const void* v_t,
                                       const int32_t* row_ptr, const int32_t* col_idx,
                                       const bsa_shape* shape, const bsa_grid* grid,
                                       float scale, void* out_t, float* lse, void* stream) {
    Geometry g;
    bsa_status st = geometry(grid, &g);
    if (st != BSA_OK) return st;
    if ((st = check_shape(shape)) != BSA_OK) return st;
    if (!q_t || !k_t || !v_t || !row_ptr || !col_idx || !out_t)
        return fail(BSA_ERR_INVALID_ARG, "q_t, k_t, v_t, row_ptr, col_idx, out_t must be non-NULL");
    if (!(scale > 0.f) || !isfinite(scale))
        return fail(BSA_ERR_INVALID_ARG, "scale must be finite and positive");
    if ((st = check_kernel_dims(shape, g)) != BSA_OK) return st;
    if ((((uintptr_t)q_t | (uintptr_t)k_t | (uintptr_t)v_t | (uintptr_t)out_t) & 15))
        return fail(BSA_ERR_INVALID_ARG, "q_t/k_t/v_t/out_t must be 16-byte aligned");
    DeviceInfo dev;
    if ((st = device_info(&dev)) != BSA_OK) return st;
    const size_t need = attn_ws_bytes(shape->batch, shape->heads, shape->head_dim, g,
                                      attn_slots(shape->head_dim, g.B, dev));
    if (need > kStaticScratchBytes)
        return fail(BSA_ERR_WORKSPACE,
                    "this call needs %zu bytes of attention workspace, more than the %zu-byte "
                    "static scratch of bsa_sparse_attn_fwd_noalloc (use bsa_sparse_attn_fwd)",
                    need, kStaticScratchBytes);
    void* ws = nullptr;
    if ((st = static_scratch(dev.device, &ws)) != BSA_OK) return st;
    return launch_attn(q_t, k_t, v_t, row_ptr, col_idx, shape->batch, shape->heads,
                       shape->head_dim, g, scale, out_t, lse, ws, dev, (hipStream_t)stream);
}

const char* bsa_last_error(void) { return g_err; }

const char* bsa_version(void) { return BSA_VERSION_STRING; }

}  // extern "C"
