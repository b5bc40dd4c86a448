// 3D-tile token permutation (video-aware block organization, FVAttn page, abstract).
//
// Tokens of the T x H x W latent grid are regrouped into 3D tiles: tiles in (it, ih, iw)
// order, the last tile along each axis truncated to what is left of the grid, row-major
// (t, h, w) inside a tile.  The kernel walks tile-order positions p and maps each back to its
// raster token n with the closed form below (peel complete tile-slabs, then tile rows, then
// tiles, then the in-tile offset), so every destination row is written exactly once and the
// forward direction also zero-fills the padding rows.
//
// HBM-bound gather: one wavefront per position moves the heads*D contiguous raster bytes of
// that token to `heads` contiguous D-element rows of the tiled layout (or back), 16 bytes
// per lane, so both sides are read and written in full cache lines.
#include "bsa_internal.h"

namespace bsa {
namespace {

struct GridArgs {
    int32_t T, H, W, tt, th, tw;
};

__device__ __forceinline__ int64_t tile_pos_to_raster(int64_t p, const GridArgs& g) {
    const int64_t slab = (int64_t)g.tt * g.H * g.W;
    const int64_t it = p / slab;
    int64_t r = p - it * slab;
    const int64_t et = min((int64_t)g.tt, (int64_t)g.T - it * g.tt);
    const int64_t row = et * g.th * g.W;
    const int64_t ih = r / row;
    r -= ih * row;
    const int64_t eh = min((int64_t)g.th, (int64_t)g.H - ih * g.th);
    const int64_t tile = et * eh * g.tw;
    const int64_t iw = r / tile;
    r -= iw * tile;
    const int64_t ew = min((int64_t)g.tw, (int64_t)g.W - iw * g.tw);
    const int64_t rt = r / (eh * ew);
    r -= rt * eh * ew;
    const int64_t rh = r / ew;
    const int64_t rw = r - rh * ew;
    const int64_t t = it * g.tt + rt, h = ih * g.th + rh, w = iw * g.tw + rw;
    return (t * g.H + h) * g.W + w;
}

constexpr int kReorderThreads = 256;
constexpr int kUnroll = 4;

// One wavefront per (batch, tile position).  chunks = heads * D / 8 (16-byte chunks).
__global__ __launch_bounds__(kReorderThreads) void reorder_kernel(
    const uint4* __restrict__ src, uint4* __restrict__ dst, GridArgs g, int32_t batch,
    int32_t heads, int32_t dch, int64_t N, int64_t Npad, int inverse) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * kReorderThreads + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * kReorderThreads) >> 6;
    const int64_t npos = inverse ? N : Npad;
    const int32_t chunks = heads * dch;
    for (int64_t w = wave; w < (int64_t)batch * npos; w += nwaves) {
        const int64_t b = w / npos;
        const int64_t p = w - b * npos;
        const bool real = p < N;
        const int64_t n = real ? tile_pos_to_raster(p, g) : 0;
        const int64_t raster_base = (b * N + n) * (int64_t)chunks;      // in chunks
        const int64_t tiled_head0 = (b * heads * Npad + p) * (int64_t)dch;
        const int64_t head_stride = Npad * (int64_t)dch;
        for (int32_t c0 = lane; c0 < chunks; c0 += 64 * kUnroll) {
            uint4 v[kUnroll];
            int64_t toff[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int32_t c = c0 + 64 * u;
                const int32_t h = c / dch;
                const int32_t dc = c - h * dch;
                toff[u] = tiled_head0 + h * head_stride + dc;
                if (c < chunks) {
                    if (!inverse)
                        v[u] = real ? src[raster_base + c] : make_uint4(0, 0, 0, 0);
                    else
                        v[u] = src[toff[u]];
                }
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int32_t c = c0 + 64 * u;
                if (c < chunks) {
                    if (!inverse)
                        dst[toff[u]] = v[u];
                    else
                        dst[raster_base + c] = v[u];
                }
            }
        }
    }
}

}  // namespace

bsa_status launch_reorder(const void* src, void* dst, int32_t batch, int32_t heads, int32_t D,
                          const Geometry& g, int inverse, hipStream_t s) {
    GridArgs ga{g.T, g.H, g.W, g.tt, g.th, g.tw};
    const int64_t npos = (int64_t)batch * (inverse ? g.N : g.Npad);
    if (npos == 0) return BSA_OK;
    const int64_t waves_per_block = kReorderThreads / 64;
    int64_t blocks = (npos + waves_per_block - 1) / waves_per_block;
    blocks = blocks > 65536 ? 65536 : blocks;
    hipLaunchKernelGGL(reorder_kernel, dim3((unsigned)blocks), dim3(kReorderThreads), 0, s,
                       (const uint4*)src, (uint4*)dst, ga, batch, heads, D / 8, g.N, g.Npad,
                       inverse);
    return check_launch("reorder");
}

}  // namespace bsa
