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

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// eight bf16 -> eight E4M3 codes
__device__ __forceinline__ uint2 codes8(const uint4& x, float inv) {
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(bf_lo(x.x) * inv, bf_hi(x.x) * inv, 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(bf_lo(x.y) * inv, bf_hi(x.y) * inv, lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(bf_lo(x.z) * inv, bf_hi(x.z) * inv, 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(bf_lo(x.w) * inv, bf_hi(x.w) * inv, hi, true);
    return make_uint2((uint32_t)lo, (uint32_t)hi);
}

__device__ __forceinline__ float amax8(const uint4& x) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    float m = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) m = fmaxf(m, fmaxf(fabsf(bf_lo(w[q])), fabsf(bf_hi(w[q]))));
    return m;
}

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

__global__ __launch_bounds__(kQThreads) void vmax_kernel(const uint4* __restrict__ x,
                                                         uint32_t* __restrict__ head_max,
                                                         int64_t Npad) {
    __shared__ float red[kQThreads / 64];
    const int t = threadIdx.x;
    const int64_t j = blockIdx.x, bh = blockIdx.y;
    const int64_t base = (bh * Npad + j * kQB) * (kQD / 8);
    float am = 0.f;
#pragma unroll
    for (int u = 0; u < kPer; ++u) am = fmaxf(am, amax8(x[base + t + u * kQThreads]));
    const float amax = block_max(am, red);
    if (t == 0) atomicMax(&head_max[bh], __float_as_uint(amax));
}

// key held at byte position p of a transposed row (64-key chunk c, half h, byte b)
__device__ __forceinline__ int v_key(int p) {
    const int c = p >> 6, h = (p >> 5) & 1, b = p & 31;
    return 64 * c + 32 * (b >> 4) + 8 * ((b & 15) >> 2) + 4 * h + (b & 3);
}

__global__ __launch_bounds__(kQThreads) void quant_v_kernel(const uint4* __restrict__ x,
                                                            uint4* __restrict__ out,
                                                            const uint32_t* __restrict__ head_max,
                                                            int64_t Npad) {
    __shared__ uint8_t codes[kQB][kQD + 4];       // [key][d]; row stride 132 B
    const int t = threadIdx.x;
    const int64_t j = blockIdx.x, bh = blockIdx.y;
    const float amax = __uint_as_float(head_max[bh]);
    const float inv = amax > 0.f ? 448.0f / amax : 0.f;
    const int64_t base = (bh * Npad + j * kQB) * (kQD / 8);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int ch = t + u * kQThreads;
        const int key = ch / (kQD / 8), d0 = (ch % (kQD / 8)) * 8;
        const uint2 c = amax > 0.f ? codes8(x[base + ch], inv) : make_uint2(0, 0);
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
    uint32_t* hm = (uint32_t*)scales;             // head maxima, then scales, in place
    hipLaunchKernelGGL(zero_kernel, dim3((bh + 255) / 256), dim3(256), 0, s, hm, bh);
    bsa_status st = check_launch("quantize v (clear)");
    if (st != BSA_OK) return st;
    hipLaunchKernelGGL(vmax_kernel, grid, dim3(kQThreads), 0, s, x, hm, (int64_t)g.Npad);
    if ((st = check_launch("quantize v (max)")) != BSA_OK) return st;
    hipLaunchKernelGGL(quant_v_kernel, grid, dim3(kQThreads), 0, s, x, (uint4*)x8,
                       (const uint32_t*)hm, (int64_t)g.Npad);
    if ((st = check_launch("quantize v")) != BSA_OK) return st;
    hipLaunchKernelGGL(vscale_kernel, dim3((bh + 255) / 256), dim3(256), 0, s, hm, bh);
    return check_launch("quantize v (scale)");
}

}  // namespace bsa
