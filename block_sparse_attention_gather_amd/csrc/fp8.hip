// E4M3 quantization for the FP8 attention (VC-Attention page, abstract: low-bit attention
// quantized per hardware block, the scale set by the block's largest entry).
//
//   rows (Q, K): one workgroup per (block j, batch*head bh): amax over the block's B x D
//                values, codes e4m3(x * (448 / amax)) (fp32 product, hardware round to
//                nearest even), scale amax / 448; layout unchanged ([bh][Npad][D] bytes).
//   V:           one scale per (batch, head): per-block amax folded into the head's maximum
//                with an integer atomic max on the fp32 bits (non-negative, so the bit order
//                is the value order), then every block is quantized with it and stored
//                transposed, [bh][n_blk][D][B] bytes, each row's keys in the order one lane of
//                the FP8 attention kernel holds its probabilities.
// A block whose values are all zero gets scale 0 and codes 0.
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kQThreads = 256;
constexpr int kQB = 128;            // block (tokens) and head dim of the FP8 path
constexpr int kQD = 128;

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < kQThreads / 64; ++i) r = fmaxf(r, red[i]);
    return r;
}

constexpr int kChunks = kQB * kQD / 8;            // 16-byte bf16 chunks per block
constexpr int kPer = kChunks / kQThreads;         // per thread

__global__ __launch_bounds__(kQThreads) void quant_rows_kernel(const uint4* __restrict__ x,
                                                               uint2* __restrict__ out,
                                                               float* __restrict__ scales,
                                                               int64_t Npad) {
    __shared__ float red[kQThreads / 64];
    const int t = threadIdx.x;
    const int64_t j = blockIdx.x, bh = blockIdx.y;
    const int64_t base = (bh * Npad + j * kQB) * (kQD / 8);   // first chunk of the block
    uint4 v[kPer];
    float am = 0.f;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        v[u] = x[base + t + u * kQThreads];
        am = fmaxf(am, amax8(v[u]));
    }
    const float amax = block_max(am, red);
    const float inv = amax > 0.f ? 448.0f / amax : 0.f;
#pragma unroll
    for (int u = 0; u < kPer; ++u)
        out[base + t + u * kQThreads] = amax > 0.f ? codes8(v[u], inv) : make_uint2(0, 0);
    if (t == 0) scales[bh * gridDim.x + j] = amax / 448.0f;
}

__global__ void zero_kernel(uint32_t* p, int32_t n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Chunk u of thread t of block (j, bh): tile-order row j*128 + t/16 + 16u, 16-byte chunk
// t mod 16 of that row, read from the tiled tensor or gathered from the raster one.
struct Gather {
    GridArgs g;
    int32_t heads;
    uint32_t N, Npad;
};

template <bool RASTER>
__device__ __forceinline__ uint4 load_chunk(const uint4* __restrict__ x, const Gather& ga,
                                            int64_t bh, int64_t j, int t, int u) {
    const uint32_t p = (uint32_t)j * kQB + (t >> 4) + 16 * u;
    const int dc = t & 15;
    if (!RASTER) return x[((size_t)bh * ga.Npad + p) * (kQD / 8) + dc];
    if (p >= ga.N) return make_uint4(0, 0, 0, 0);
    const uint32_t n = tile_pos_to_raster(p, ga.g);
    const uint32_t b = (uint32_t)bh / (uint32_t)ga.heads, h = (uint32_t)bh - b * ga.heads;
    return x[(((size_t)b * ga.N + n) * ga.heads + h) * (kQD / 8) + dc];
}

// per-block amax folded into the head maximum; from raster input, optionally also writes the
// tiled bf16 block
template <bool RASTER>
__global__ __launch_bounds__(kQThreads) void vmax_kernel(const uint4* __restrict__ x,
                                                         uint32_t* __restrict__ head_max,
                                                         uint4* __restrict__ tiled, Gather ga) {
    __shared__ float red[kQThreads / 64];
    const int t = threadIdx.x;
    const int64_t j = blockIdx.x, bh = blockIdx.y;
    float am = 0.f;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const uint4 c = load_chunk<RASTER>(x, ga, bh, j, t, u);
        if (tiled) tiled[((size_t)bh * ga.Npad + j * kQB + (t >> 4) + 16 * u) * (kQD / 8) + (t & 15)] = c;
        am = fmaxf(am, amax8(c));
    }
    const float amax = block_max(am, red);
    if (t == 0) atomicMax(&head_max[bh], __float_as_uint(amax));
}

// key held at byte position p of a transposed row (64-key chunk c, half h, byte b)
__device__ __forceinline__ int v_key(int p) {
    const int c = p >> 6, h = (p >> 5) & 1, b = p & 31;
    return 64 * c + 32 * (b >> 4) + 8 * ((b & 15) >> 2) + 4 * h + (b & 3);
}

template <bool RASTER>
__global__ __launch_bounds__(kQThreads) void quant_v_kernel(const uint4* __restrict__ x,
                                                            uint4* __restrict__ out,
                                                            const uint32_t* __restrict__ head_max,
                                                            Gather ga) {
    __shared__ uint8_t codes[kQB][kQD + 4];       // [key][d]; row stride 132 B
    const int t = threadIdx.x;
    const int64_t j = blockIdx.x, bh = blockIdx.y;
    const float amax = __uint_as_float(head_max[bh]);
    const float inv = amax > 0.f ? 448.0f / amax : 0.f;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int ch = t + u * kQThreads;
        const int key = ch / (kQD / 8), d0 = (ch % (kQD / 8)) * 8;
        const uint2 c = amax > 0.f ? codes8(load_chunk<RASTER>(x, ga, bh, j, t, u), inv)
                                   : make_uint2(0, 0);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            codes[key][d0 + b] = (uint8_t)(c.x >> (8 * b));
            codes[key][d0 + 4 + b] = (uint8_t)(c.y >> (8 * b));
        }
    }
    __syncthreads();
    // output block: kQD rows of kQB bytes, 16-byte chunks
    uint4* ob = out + ((bh * gridDim.x + j) * kQD * kQB) / 16;
    for (int ch = t; ch < kQD * kQB / 16; ch += kQThreads) {
        const int d = ch / (kQB / 16), p0 = (ch % (kQB / 16)) * 16;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t acc = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) acc |= (uint32_t)codes[v_key(p0 + 4 * q + b)][d] << (8 * b);
            w[q] = acc;
        }
        ob[ch] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

__global__ void vscale_kernel(uint32_t* head_max, int32_t n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) head_max[i] = __float_as_uint(__uint_as_float(head_max[i]) / 448.0f);
}

}  // namespace

bsa_status launch_quant_fp8(const void* x_t, void* x8, float* scales, int32_t v_layout,
                            int32_t batch, int32_t heads, const Geometry& g, hipStream_t s) {
    const int32_t bh = batch * heads;
    const dim3 grid((unsigned)g.n_blk, (unsigned)bh);
    const uint4* x = (const uint4*)x_t;
    if (!v_layout) {
        hipLaunchKernelGGL(quant_rows_kernel, grid, dim3(kQThreads), 0, s, x, (uint2*)x8, scales,
                           (int64_t)g.Npad);
        return check_launch("quantize rows");
    }
    const Gather ga{GridArgs{g.T, g.H, g.W, g.tt, g.th, g.tw, g.order}, heads, (uint32_t)g.N,
                    (uint32_t)g.Npad};
    uint32_t* hm = (uint32_t*)scales;             // head maxima, then scales, in place
    hipLaunchKernelGGL(zero_kernel, dim3((bh + 255) / 256), dim3(256), 0, s, hm, bh);
    bsa_status st = check_launch("quantize v (clear)");
    if (st != BSA_OK) return st;
    hipLaunchKernelGGL(vmax_kernel<false>, grid, dim3(kQThreads), 0, s, x, hm, (uint4*)nullptr,
                       ga);
    if ((st = check_launch("quantize v (max)")) != BSA_OK) return st;
    hipLaunchKernelGGL(quant_v_kernel<false>, grid, dim3(kQThreads), 0, s, x, (uint4*)x8,
                       (const uint32_t*)hm, ga);
    if ((st = check_launch("quantize v")) != BSA_OK) return st;
    hipLaunchKernelGGL(vscale_kernel, dim3((bh + 255) / 256), dim3(256), 0, s, hm, bh);
    return check_launch("quantize v (scale)");
}

// Raster V [batch, N, heads, 128] -> E4M3 V in the transposed block layout (and, when dst is
// not NULL, the tiled bf16 V): the first pass gathers every block for the head maxima (and
// writes dst), the second gathers again and quantizes.
bsa_status launch_reorder_quant_v(const void* src, void* dst, void* v8, float* v_scales,
                                  int32_t batch, int32_t heads, const Geometry& g,
                                  hipStream_t s) {
    const int32_t bh = batch * heads;
    const dim3 grid((unsigned)g.n_blk, (unsigned)bh);
    const uint4* x = (const uint4*)src;
    const Gather ga{GridArgs{g.T, g.H, g.W, g.tt, g.th, g.tw, g.order}, heads, (uint32_t)g.N,
                    (uint32_t)g.Npad};
    uint32_t* hm = (uint32_t*)v_scales;
    hipLaunchKernelGGL(zero_kernel, dim3((bh + 255) / 256), dim3(256), 0, s, hm, bh);
    bsa_status st = check_launch("reorder_quantize_v (clear)");
    if (st != BSA_OK) return st;
    hipLaunchKernelGGL(vmax_kernel<true>, grid, dim3(kQThreads), 0, s, x, hm, (uint4*)dst, ga);
    if ((st = check_launch("reorder_quantize_v (max)")) != BSA_OK) return st;
    hipLaunchKernelGGL(quant_v_kernel<true>, grid, dim3(kQThreads), 0, s, x, (uint4*)v8,
                       (const uint32_t*)hm, ga);
    if ((st = check_launch("reorder_quantize_v")) != BSA_OK) return st;
    hipLaunchKernelGGL(vscale_kernel, dim3((bh + 255) / 256), dim3(256), 0, s, hm, bh);
    return check_launch("reorder_quantize_v (scale)");
}

}  // namespace bsa
