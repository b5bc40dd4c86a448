// Internal declarations shared by the libbsa translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bsa.h"

namespace bsa {

// ---- geometry ----------------------------------------------------------------------
struct Geometry {
    int32_t T, H, W, tt, th, tw, B;
    int64_t N;        // real tokens
    int32_t n_blk;    // ceil(N / B)
    int64_t Npad;     // n_blk * B
    const int32_t* order;   // device table: raster token at each position (NULL: 3D tiles)
};

// 3D-tile grid as kernel arguments, and the tile-order position -> raster token map that
// the reorder and the stripe-mask kernels share.
struct GridArgs {
    int32_t T, H, W, tt, th, tw;
    const int32_t* order;   // raster token at each position, or NULL for the 3D-tile order
};

// Tile-order position p -> raster token n, in 32-bit arithmetic (N < 2^31 is checked on the
// host, so every intermediate fits).
static __device__ __forceinline__ uint32_t tile_pos_to_raster(uint32_t p, const GridArgs& g) {
    if (g.order) return (uint32_t)g.order[p];          // a caller-built order (Hilbert)
    const uint32_t T = g.T, H = g.H, W = g.W, tt = g.tt, th = g.th, tw = g.tw;
    const uint32_t slab = tt * H * W;
    const uint32_t it = p / slab;
    uint32_t r = p - it * slab;
    const uint32_t et = min(tt, T - it * tt);
    const uint32_t row = et * th * W;
    const uint32_t ih = r / row;
    r -= ih * row;
    const uint32_t eh = min(th, H - ih * th);
    const uint32_t tile = et * eh * tw;
    const uint32_t iw = r / tile;
    r -= iw * tile;
    const uint32_t ew = min(tw, W - iw * tw);
    const uint32_t plane = eh * ew;
    const uint32_t rt = r / plane;
    r -= rt * plane;
    const uint32_t rh = r / ew;
    const uint32_t rw = r - rh * ew;
    const uint32_t t = it * tt + rt, h = ih * th + rh, w = iw * tw + rw;
    return (t * H + h) * W + w;
}

// bf16 words -> fp32, and eight bf16 -> eight E4M3 codes (hardware round to nearest even)
static __device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
static __device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// eight bf16 -> eight E4M3 codes
static __device__ __forceinline__ uint2 codes8(const uint4& x, float inv) {
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(bf_lo(x.x) * inv, bf_hi(x.x) * inv, 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(bf_lo(x.y) * inv, bf_hi(x.y) * inv, lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(bf_lo(x.z) * inv, bf_hi(x.z) * inv, 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(bf_lo(x.w) * inv, bf_hi(x.w) * inv, hi, true);
    return make_uint2((uint32_t)lo, (uint32_t)hi);
}

static __device__ __forceinline__ float amax8(const uint4& x) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    float m = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) m = fmaxf(m, fmaxf(fabsf(bf_lo(w[q])), fabsf(bf_hi(w[q]))));
    return m;
}

// ---- error reporting (thread-local message, see bsa_last_error) ---------------------
bsa_status fail(bsa_status st, const char* fmt, ...);
bsa_status check_launch(const char* what);

// ---- per-device properties (read once per device, then cached) ---------------------
struct DeviceInfo {
    int device;           // HIP device ordinal
    int cu_count;         // compute units
};
bsa_status device_info(DeviceInfo* out);
// persistent attention workgroups for one device: CUs x resident workgroups per CU
int attn_slots(int32_t D, int32_t B, const DeviceInfo& dev);
int attn_fp8_slots(const DeviceInfo& dev);
int attn_max_heads();
int attn_max_blocks();

// ---- launchers (defined next to their kernels) -------------------------------------
bsa_status launch_reorder(const void* src, void* dst, int32_t batch, int32_t heads,
                          int32_t D, const Geometry& g, int inverse, hipStream_t s);

bsa_status launch_reorder_pool(const void* src, void* dst, double* pooled, void* x8,
                               float* x8_scales, int32_t batch, int32_t heads, int32_t D,
                               const Geometry& g, hipStream_t s);
bsa_status launch_reorder_quant_v(const void* src, void* dst, void* v8, float* v_scales,
                                  int32_t batch, int32_t heads, const Geometry& g,
                                  hipStream_t s);

size_t route_ws_bytes(int32_t batch, int32_t heads, int32_t D, const Geometry& g);
bsa_status launch_route_pooled(const double* qbar, const double* kbar, int32_t batch,
                               int32_t heads, int32_t D, const Geometry& g, double top_p,
                               int32_t k_floor, double scale, int32_t* row_ptr,
                               int32_t* col_idx, int32_t* nnz, double* block_scores, void* ws,
                               hipStream_t s);
bsa_status launch_route(const void* q_t, const void* k_t, int32_t batch, int32_t heads,
                        int32_t D, const Geometry& g, double top_p, int32_t k_floor,
                        double scale, int32_t* row_ptr, int32_t* col_idx, int32_t* nnz,
                        double* block_scores, void* ws, hipStream_t s);

size_t stripe_ws_bytes(int32_t batch, int32_t heads, const Geometry& g);
bsa_status launch_stripe(const int32_t* params_host, int32_t batch, int32_t heads,
                         const Geometry& g, int32_t* row_ptr, int32_t* col_idx, int32_t* nnz,
                         void* ws, hipStream_t s);

size_t hilbert_ws_bytes(const Geometry& g);
bsa_status launch_hilbert_order(const Geometry& g, int32_t* order, void* ws, hipStream_t s);
bsa_status launch_scan(const int32_t* counts, int32_t* excl, int32_t* total, int64_t n,
                       hipStream_t s);

size_t attn_ws_bytes(int32_t batch, int32_t heads, int32_t D, const Geometry& g, int slots);
// Static scratch of bsa_sparse_attn_fwd_noalloc: kStaticScratchBytes of device memory per
// device (a file-scope __device__ array), its address on `device` (the current device) looked
// up once with hipGetSymbolAddress and cached.
constexpr size_t kStaticScratchBytes = (size_t)136 << 20;
constexpr int kMaxDevices = 64;
bsa_status static_scratch(int device, void** ptr);
bsa_status launch_attn(const void* q_t, const void* k_t, const void* v_t,
                       const int32_t* row_ptr, const int32_t* col_idx, int32_t batch,
                       int32_t heads, int32_t D, const Geometry& g, float scale, void* out_t,
                       float* lse, void* ws, const DeviceInfo& dev, hipStream_t s);

bsa_status launch_attn_fp8(const void* q8, const float* qs, const void* k8, const float* ks,
                           const void* v8, const float* vs, const int32_t* row_ptr,
                           const int32_t* col_idx, int32_t batch, int32_t heads,
                           const Geometry& g, float scale, int32_t expcast, void* out_t,
                           float* lse, void* ws, const DeviceInfo& dev, hipStream_t s);
bsa_status launch_quant_fp8(const void* x_t, void* x8, float* scales, int32_t v_layout,
                            int32_t batch, int32_t heads, const Geometry& g, hipStream_t s);

// ---- small helpers -------------------------------------------------------------------
static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace bsa
