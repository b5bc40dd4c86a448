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

// Tile-order position p -> raster token n, in 32-bit arithmetic (N < 2^31 is checked on the
// host, so every intermediate fits).
__device__ __forceinline__ uint32_t tile_pos_to_raster(uint32_t p, const GridArgs& g) {
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

constexpr int kReorderThreads = 256;

// One wavefront per tile position p of batch blockIdx.y moves one token: the heads * D
// contiguous raster elements <-> `heads` rows of D elements in the tiled layout, as 16-byte
// chunks (chunk c = head c / DCH, column chunk c % DCH).  DCH = D / 8 is a compile-time
// constant for D = 64 and 128 (0 = runtime dch for other head sizes).  Forward (INV = false)
// writes zeros to the pad positions p >= N; inverse reads only real positions.  Each lane
// keeps up to U chunks in flight before it stores them.  All index math is 32-bit except the
// element offsets, and the batch index is blockIdx.y, so no 64-bit division is left.
template <int DCH, int U, bool INV>
__global__ __launch_bounds__(kReorderThreads) void reorder_kernel(
    const uint4* __restrict__ src, uint4* __restrict__ dst, GridArgs g, int32_t heads,
    int32_t dch_rt, uint32_t N, uint32_t Npad) {
    const int dch = DCH ? DCH : dch_rt;
    const int lane = threadIdx.x & 63;
    const uint32_t wave = (blockIdx.x * kReorderThreads + threadIdx.x) >> 6;
    const uint32_t nwaves = (gridDim.x * kReorderThreads) >> 6;
    const uint32_t npos = INV ? N : Npad;
    const int32_t chunks = heads * dch;
    const int64_t b = blockIdx.y;
    const int64_t head_stride = (int64_t)Npad * dch;
    for (uint32_t p = wave; p < npos; p += nwaves) {
        const bool real = INV || p < N;
        const uint32_t n = real ? tile_pos_to_raster(p, g) : 0u;
        const uint4* rs = (INV ? dst : src) + (b * N + n) * (int64_t)chunks;   // raster row
        const int64_t tiled0 = (b * heads * (int64_t)Npad + p) * (int64_t)dch;
        for (int32_t c0 = lane; c0 < chunks; c0 += 64 * U) {
            uint4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int32_t c = c0 + 64 * u;
                if (c < chunks) {
                    const int32_t h = c / dch;
                    const int64_t toff = tiled0 + h * head_stride + (c - h * dch);
                    if (INV)
                        v[u] = src[toff];
                    else
                        v[u] = real ? rs[c] : make_uint4(0, 0, 0, 0);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int32_t c = c0 + 64 * u;
                if (c < chunks) {
                    const int32_t h = c / dch;
                    const int64_t toff = tiled0 + h * head_stride + (c - h * dch);
                    if (INV)
                        dst[(b * N + n) * (int64_t)chunks + c] = v[u];
                    else
                        dst[toff] = v[u];
                }
            }
        }
    }
}

// Chunks in flight per lane: 4 forward, 2 inverse (inverse reads 256-byte rows of `heads`
// different tiled rows; more than two per lane measured slower).
template <int DCH>
void launch_dir(const uint4* sp, uint4* dp, const GridArgs& ga, dim3 grid, int32_t heads,
                int32_t dch, uint32_t N, uint32_t Npad, int inverse, hipStream_t s) {
    if (inverse)
        hipLaunchKernelGGL((reorder_kernel<DCH, 2, true>), grid, dim3(kReorderThreads), 0, s, sp,
                           dp, ga, heads, dch, N, Npad);
    else
        hipLaunchKernelGGL((reorder_kernel<DCH, 4, false>), grid, dim3(kReorderThreads), 0, s,
                           sp, dp, ga, heads, dch, N, Npad);
}

}  // namespace

bsa_status launch_reorder(const void* src, void* dst, int32_t batch, int32_t heads, int32_t D,
                          const Geometry& g, int inverse, hipStream_t s) {
    GridArgs ga{g.T, g.H, g.W, g.tt, g.th, g.tw};
    const int64_t npos = inverse ? g.N : g.Npad;
    if (npos == 0 || batch == 0) return BSA_OK;
    const int64_t waves_per_block = kReorderThreads / 64;
    int64_t blocks = (npos + waves_per_block - 1) / waves_per_block;
    blocks = blocks > 65536 ? 65536 : blocks;
    const dim3 grid((unsigned)blocks, (unsigned)batch);
    const uint4* sp = (const uint4*)src;
    uint4* dp = (uint4*)dst;
    const uint32_t N = (uint32_t)g.N, Npad = (uint32_t)g.Npad;
    if (D == 128)
        launch_dir<16>(sp, dp, ga, grid, heads, 16, N, Npad, inverse, s);
    else if (D == 64)
        launch_dir<8>(sp, dp, ga, grid, heads, 8, N, Npad, inverse, s);
    else
        launch_dir<0>(sp, dp, ga, grid, heads, D / 8, N, Npad, inverse, s);
    return check_launch("reorder");
}

}  // namespace bsa
