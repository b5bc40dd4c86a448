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
// per lane, so both sides are read and written in full cache lines.  Every byte is read once
// and written once, so the loads and stores are non-temporal (streamed past the caches): a
// plain 1 GiB device copy moves 6.2 TB/s that way against 5.7 TB/s with ordinary accesses,
// and the reorders got 11-22 % faster (the same bytes written).
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kReorderThreads = 256;

// 16-byte non-temporal load and store
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
    const nt_u32x4 v = __builtin_nontemporal_load((const nt_u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(uint4* p, const uint4& v) {
    const nt_u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (nt_u32x4*)p);
}
typedef unsigned int nt_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_nt8(uint2* p, const uint2& v) {
    const nt_u32x2 w = {v.x, v.y};
    __builtin_nontemporal_store(w, (nt_u32x2*)p);
}

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
                        v[u] = ld_nt(src + toff);
                    else
                        v[u] = real ? ld_nt(rs + c) : make_uint4(0, 0, 0, 0);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int32_t c = c0 + 64 * u;
                if (c < chunks) {
                    const int32_t h = c / dch;
                    const int64_t toff = tiled0 + h * head_stride + (c - h * dch);
                    if (INV)
                        st_nt(dst + (b * N + n) * (int64_t)chunks + c, v[u]);
                    else
                        st_nt(dst + toff, v[u]);
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

// Forward reorder fused with routing's block pooling: a workgroup gathers the B raster rows of
// block j of (batch b, head h) (head_dim D contiguous elements each; blockIdx.x = j * heads + h,
// heads fastest, so the workgroups in flight together read whole raster token rows of all
// heads rather than one piece of each; blockIdx.y = b) and, each output
// optional, writes them as the contiguous tiled block (pad rows zero), sums every column over
// the block's real rows in fp64 (pooled[bh][j] = column sums / real rows; a sum of at most
// 128 bf16 values whose nonzero magnitudes lie within a factor 2^38 of each other is exact in
// fp64 in any order, so for such columns the means equal a separate pooling pass bit for
// bit), and with FP8 writes the block's E4M3 codes and scale exactly as
// the per-block quantization of the tiled tensor does (amax over the block, pad rows zero).
template <int D, int B, bool FP8>
__global__ __launch_bounds__(kReorderThreads) void reorder_pool_kernel(
    const uint4* __restrict__ src, uint4* __restrict__ dst, double* __restrict__ pooled,
    uint2* __restrict__ x8, float* __restrict__ x8_scales, GridArgs g, int32_t heads,
    uint32_t N, uint32_t Npad) {
    constexpr int DCH = D / 8;                    // 16-byte chunks per row
    constexpr int RPP = kReorderThreads / DCH;    // rows per pass
    constexpr int NP = B / RPP;                   // passes (rows per thread)
    static_assert(B <= kReorderThreads, "one thread per block row computes its raster row");
    __shared__ double red[RPP][D + 1];
    __shared__ float amax_red[kReorderThreads / 64];
    __shared__ uint32_t rows[B];
    const int t = threadIdx.x;
    const int dc = t % DCH, rp = t / DCH;
    const uint32_t n_blk = Npad / B;
    const uint32_t j = blockIdx.x / (uint32_t)heads, h = blockIdx.x - j * (uint32_t)heads;
    const uint32_t b = blockIdx.y;
    const uint32_t bh = b * (uint32_t)heads + h;
    const uint32_t lo = j * B;
    const uint32_t hi = min(lo + (uint32_t)B, N);
    // The block's raster rows, one per thread of the first B (an explicit order reads its table
    // here), shared through LDS; then the loads, unconditionally (a row past the last token
    // reads row 0 and is zeroed afterwards), so that all of them are in flight together.
    if (t < B) rows[t] = lo + t < N ? tile_pos_to_raster(lo + t, g) : ~0u;
    __syncthreads();
    uint32_t n[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) n[k] = rows[rp + RPP * k];
    uint4 v[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k)
        v[k] = ld_nt(src + (((size_t)b * N + (n[k] != ~0u ? n[k] : 0u)) * heads + h) * DCH + dc);
#pragma unroll
    for (int k = 0; k < NP; ++k)
        if (n[k] == ~0u) v[k] = make_uint4(0, 0, 0, 0);
    if (dst) {
#pragma unroll
        for (int k = 0; k < NP; ++k) st_nt(dst + ((size_t)bh * Npad + lo + rp + RPP * k) * DCH + dc, v[k]);
    }
    if (FP8) {
        float am = 0.f;
#pragma unroll
        for (int k = 0; k < NP; ++k) am = fmaxf(am, amax8(v[k]));
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off, 64));
        if ((t & 63) == 0) amax_red[t >> 6] = am;
        __syncthreads();
        float amax = amax_red[0];
#pragma unroll
        for (int i = 1; i < kReorderThreads / 64; ++i) amax = fmaxf(amax, amax_red[i]);
        const float inv = amax > 0.f ? 448.0f / amax : 0.f;
#pragma unroll
        for (int k = 0; k < NP; ++k)
            st_nt8(x8 + ((size_t)bh * Npad + lo + rp + RPP * k) * DCH + dc,
                   amax > 0.f ? codes8(v[k], inv) : make_uint2(0, 0));
        if (t == 0) x8_scales[(size_t)bh * n_blk + j] = amax / 448.0f;
    }
    if (pooled) {
        double acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                acc[2 * u] += (double)bf_lo(w[u]);
                acc[2 * u + 1] += (double)bf_hi(w[u]);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) red[rp][dc * 8 + e] = acc[e];
        __syncthreads();
        for (int d = t; d < D; d += kReorderThreads) {
            double sum = 0.0;
            for (int r = 0; r < RPP; ++r) sum += red[r][d];
            pooled[((size_t)bh * n_blk + j) * D + d] = sum / (double)(hi - lo);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Hilbert-curve token order (DFSAttn page, abstract: tokens reordered along a Hilbert curve so
// that blocks of consecutive tokens are compact).  Tokens are ordered by their index on the 3D
// Hilbert curve of the smallest 2^bits cube holding the grid, axes (t, h, w), computed with
// J. Skilling's transform ("Programming the Hilbert curve", 2004): per level from the top,
// undo the excess work (invert the low bits of axis 0, or exchange them with axis i), then a
// Gray code across the axes and a final correction give the transposed index, whose bits are
// interleaved from the top level down.  The order table is built by marking the cube cells the
// grid occupies, an exclusive scan over the cube in curve order, and placing every token at
// the scan value of its cell.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t hilbert_index3(uint32_t t, uint32_t h, uint32_t w,
                                                   int bits) {
    uint32_t X[3] = {t, h, w};
    const uint32_t M = 1u << (bits - 1);
    for (uint32_t Q = M; Q > 1; Q >>= 1) {
        const uint32_t P = Q - 1;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            if (X[i] & Q) {
                X[0] ^= P;
            } else {
                const uint32_t x = (X[0] ^ X[i]) & P;
                X[0] ^= x;
                X[i] ^= x;
            }
        }
    }
    X[1] ^= X[0];
    X[2] ^= X[1];
    uint32_t tc = 0;
    for (uint32_t Q = M; Q > 1; Q >>= 1)
        if (X[2] & Q) tc ^= Q - 1;
    X[0] ^= tc;
    X[1] ^= tc;
    X[2] ^= tc;
    uint32_t idx = 0;
    for (int b = bits - 1; b >= 0; --b)
#pragma unroll
        for (int i = 0; i < 3; ++i) idx = (idx << 1) | ((X[i] >> b) & 1u);
    return idx;
}

__device__ __forceinline__ uint32_t token_hilbert(uint32_t n, const GridArgs& g, int bits) {
    const uint32_t HW = (uint32_t)g.H * (uint32_t)g.W;
    const uint32_t t = n / HW, r = n - t * HW;
    const uint32_t h = r / (uint32_t)g.W, w = r - h * (uint32_t)g.W;
    return hilbert_index3(t, h, w, bits);
}

__global__ void fill_zero_kernel(int32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

__global__ void hilbert_mark_kernel(int32_t* cells, GridArgs g, uint32_t N, int bits) {
    const uint32_t n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n < N) cells[token_hilbert(n, g, bits)] = 1;
}

__global__ void hilbert_place_kernel(const int32_t* excl, int32_t* order, GridArgs g, uint32_t N,
                                     int bits) {
    const uint32_t n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n < N) order[excl[token_hilbert(n, g, bits)]] = (int32_t)n;
}

static int hilbert_bits(const Geometry& g) {
    int bits = 1;
    while ((1 << bits) < g.T || (1 << bits) < g.H || (1 << bits) < g.W) ++bits;
    return bits;
}

}  // namespace

bsa_status launch_reorder(const void* src, void* dst, int32_t batch, int32_t heads, int32_t D,
                          const Geometry& g, int inverse, hipStream_t s) {
    GridArgs ga{g.T, g.H, g.W, g.tt, g.th, g.tw, g.order};
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

bsa_status launch_reorder_pool(const void* src, void* dst, double* pooled, void* x8,
                               float* x8_scales, int32_t batch, int32_t heads, int32_t D,
                               const Geometry& g, hipStream_t s) {
    GridArgs ga{g.T, g.H, g.W, g.tt, g.th, g.tw, g.order};
    if ((uint64_t)g.n_blk * (uint64_t)heads * kReorderThreads > 0xffffffffull)
        return fail(BSA_ERR_UNSUPPORTED, "reorder_pool: %d blocks x %d heads exceed one grid axis",
                    g.n_blk, heads);
    const dim3 grid((unsigned)g.n_blk * (unsigned)heads, (unsigned)batch);
    const uint4* sp = (const uint4*)src;
    uint4* dp = (uint4*)dst;
    uint2* qp = (uint2*)x8;
    const uint32_t N = (uint32_t)g.N, Npad = (uint32_t)g.Npad;
    const dim3 blk(kReorderThreads);
#define BSA_RP(DD, BB, F8)                                                                       \
    hipLaunchKernelGGL((reorder_pool_kernel<DD, BB, F8>), grid, blk, 0, s, sp, dp, pooled, qp, \
                       x8_scales, ga, heads, N, Npad)
    if (x8) BSA_RP(128, 128, true);                  // the FP8 path: D = B = 128 (checked)
    else if (D == 128 && g.B == 128) BSA_RP(128, 128, false);
    else if (D == 128) BSA_RP(128, 64, false);
    else if (g.B == 128) BSA_RP(64, 128, false);
    else BSA_RP(64, 64, false);
#undef BSA_RP
    return check_launch("reorder_pool");
}

size_t hilbert_ws_bytes(const Geometry& g) {
    const size_t cells = (size_t)1 << (3 * hilbert_bits(g));
    return align_up(cells * 4, 256) + align_up((cells + 1) * 4, 256) + 256;
}

bsa_status launch_hilbert_order(const Geometry& g, int32_t* order, void* ws, hipStream_t s) {
    const int bits = hilbert_bits(g);
    const int64_t cells = (int64_t)1 << (3 * bits);
    unsigned char* w = (unsigned char*)ws;
    int32_t* mark = (int32_t*)w;
    int32_t* excl = (int32_t*)(w + align_up((size_t)cells * 4, 256));
    int32_t* total = (int32_t*)(w + align_up((size_t)cells * 4, 256) +
                                align_up((size_t)(cells + 1) * 4, 256));
    const GridArgs ga{g.T, g.H, g.W, g.tt, g.th, g.tw, nullptr};   // raster coordinates only
    const uint32_t N = (uint32_t)g.N;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0, s, mark, cells);
    bsa_status st = check_launch("hilbert (clear)");
    if (st != BSA_OK) return st;
    const dim3 tg((N + 255) / 256);
    hipLaunchKernelGGL(hilbert_mark_kernel, tg, dim3(256), 0, s, mark, ga, N, bits);
    if ((st = check_launch("hilbert (mark)")) != BSA_OK) return st;
    if ((st = launch_scan(mark, excl, total, cells, s)) != BSA_OK) return st;
    hipLaunchKernelGGL(hilbert_place_kernel, tg, dim3(256), 0, s, excl, order, ga, N, bits);
    return check_launch("hilbert (place)");
}

}  // namespace bsa
