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
static_assert(kPer == 8 && kQB <= kQThreads && kQD == 128, "V gather mapping assumes these sizes");

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

// Row (key) of a block held in chunk u of thread t: each thread holds the four consecutive
// keys 4g..4g+3 of key groups g = t/16 and t/16 + 16, all at 16-byte chunk t mod 16.
__device__ __forceinline__ int blk_row(int t, int u) { return 4 * ((t >> 4) + 16 * (u >> 2)) + (u & 3); }

// What a V pass reads: the grid geometry (for the raster gather), heads per batch entry, and
// the real and padded token counts.
struct Gather {
    GridArgs g;
    int32_t heads;
    uint32_t N, Npad;
};

// Block of a workgroup.  A tiled input walks the blocks of one (batch, head) slab (grid
// n_blk x batch*heads); a raster gather walks the heads fastest (grid heads*n_blk x batch), so
// the workgroups in flight together read whole token rows of the raster tensor (heads x 256
// bytes) rather than one 256-byte piece of each.
struct Blk {
    int64_t j, bh;
    uint32_t b, h;
};

template <bool RASTER>
__device__ __forceinline__ Blk blk_of(const Gather& ga) {
    if (!RASTER) return Blk{(int64_t)blockIdx.x, (int64_t)blockIdx.y, 0u, 0u};
    const uint32_t heads = (uint32_t)ga.heads, j = blockIdx.x / heads, h = blockIdx.x - j * heads;
    return Blk{(int64_t)j, (int64_t)blockIdx.y * heads + h, blockIdx.y, h};
}

// Chunks u = 0..kPer-1 of thread t of block (j, bh): tile-order row j*128 + blk_row(t, u),
// 16-byte chunk t mod 16 of that row, read from the tiled tensor or gathered from the raster
// one (zero past the last real token).  rows: kQB words of LDS for the block's raster rows
// (written and read here, around a workgroup barrier; RASTER only).
// 16-byte non-temporal load (raster V is read by the two passes and nothing else: streaming
// both of them past the caches measured 5-14 % faster than ordinary loads, while streaming only
// the first, so that the second could find V in the caches, was 4 % slower).  The codes are
// stored non-temporally too (with the Q and K codes of the fused reorder: the FP8 layer's
// preparation 4-5 % faster, the attention that reads them next not slowed).
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
    const nt_u32x4 v = __builtin_nontemporal_load((const nt_u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool RASTER>
__device__ __forceinline__ void load_block(uint4 (&c)[kPer], const uint4* __restrict__ x,
                                           const Gather& ga, const Blk& k, int t,
                                           uint32_t* rows) {
    const int64_t bh = k.bh, j = k.j;
    const uint32_t p0 = (uint32_t)j * kQB;
    const int dc = t & 15;
    if (!RASTER) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) c[u] = x[((size_t)bh * ga.Npad + p0 + blk_row(t, u)) * (kQD / 8) + dc];
        return;
    }
    const uint32_t b = k.b, h = k.h;
    // The block's raster rows, one per thread of the first kQB (an explicit order reads its
    // table here), shared through LDS: the sixteen threads of a row need the same one.  Then
    // the data loads, unconditionally (a row past the last token reads row 0 and is zeroed
    // afterwards), so all of them are in flight together.
    if (t < kQB) {
        const uint32_t p = p0 + t;
        rows[t] = p < ga.N ? tile_pos_to_raster(p, ga.g) : ~0u;
    }
    __syncthreads();
    uint32_t n[kPer];
#pragma unroll
    for (int v = 0; v < kPer / 4; ++v) {
        const uint4 r = *(const uint4*)&rows[blk_row(t, 4 * v)];
        n[4 * v] = r.x, n[4 * v + 1] = r.y, n[4 * v + 2] = r.z, n[4 * v + 3] = r.w;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const uint32_t r = n[u] != ~0u ? n[u] : 0u;
        c[u] = ld_nt(x + (((size_t)b * ga.N + r) * ga.heads + h) * (kQD / 8) + dc);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u)
        if (n[u] == ~0u) c[u] = make_uint4(0, 0, 0, 0);
}

// per-block amax folded into the head maximum; from raster input, optionally also writes the
// tiled bf16 block
template <bool RASTER>
__global__ __launch_bounds__(kQThreads) void vmax_kernel(const uint4* __restrict__ x,
                                                         uint32_t* __restrict__ head_max,
                                                         uint4* __restrict__ tiled, Gather ga) {
    __shared__ float red[kQThreads / 64];
    const int t = threadIdx.x;
    __shared__ __align__(16) uint32_t rows[kQB];
    const Blk k = blk_of<RASTER>(ga);
    const int64_t j = k.j, bh = k.bh;
    uint4 c[kPer];
    load_block<RASTER>(c, x, ga, k, t, rows);
    float am = 0.f;
#pragma unroll
    for (int u = 0; u < kPer; ++u) am = fmaxf(am, amax8(c[u]));
    if (tiled)
#pragma unroll
        for (int u = 0; u < kPer; ++u)
            tiled[((size_t)bh * ga.Npad + j * kQB + blk_row(t, u)) * (kQD / 8) + (t & 15)] = c[u];
    const float amax = block_max(am, red);
    if (t == 0) atomicMax(&head_max[bh], __float_as_uint(amax));
}

// Word position, within a transposed row, of the four keys 4g..4g+3 (one 4-byte word, key
// 4g+i in byte i).  A row lists its 128 keys in 64-key chunks c, each as two halves h of 32
// bytes, byte b of a half holding key 64c + 32(b/16) + 8((b mod 16)/4) + 4h + (b mod 4) (the
// order in which one lane of the FP8 attention holds its probabilities).  Inverting that map per 4-key group gives
// word 16c + 8h + 4(b/16) + (b mod 16)/4 for g = 16c + 8(b/16) + 2((b mod 16)/4) + h.
__device__ __forceinline__ int v_group_pos(int g) {
    return 16 * (g >> 4) + 8 * (g & 1) + 4 * ((g >> 3) & 1) + ((g >> 1) & 3);
}

// LDS word column of word w of transposed row d (128-byte rows, two per sweep of the 64
// banks).  The XOR keeps the eight rows x eight words of a read instruction on 64 distinct
// banks and the sixteen d-chunks x four key groups of a write instruction on 32 (rows of one
// parity only reach 32 banks).
__device__ __forceinline__ int vt_col(int d, int w) {
    const int dc = d >> 3;
    return w ^ ((d >> 1) & 3) ^ ((dc & 3) << 1) ^ ((dc & 4) << 2);
}

template <bool RASTER>
__global__ __launch_bounds__(kQThreads) void quant_v_kernel(const uint4* __restrict__ x,
                                                            uint4* __restrict__ out,
                                                            const uint32_t* __restrict__ head_max,
                                                            Gather ga) {
    __shared__ uint32_t vt[kQD][kQB / 4];          // [d][word], words in output order
    __shared__ __align__(16) uint32_t rows[kQB];
    const int t = threadIdx.x;
    const Blk kb = blk_of<RASTER>(ga);
    const int64_t j = kb.j, bh = kb.bh;
    const float amax = __uint_as_float(head_max[bh]);
    const float inv = amax > 0.f ? 448.0f / amax : 0.f;
    uint4 raw[kPer];
    load_block<RASTER>(raw, x, ga, kb, t, rows);
    // per key group: four keys x eight d codes, transposed in registers into eight words
    // (one per d, keys in byte order)
#pragma unroll
    for (int v = 0; v < kPer / 4; ++v) {
        uint2 k[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) k[i] = amax > 0.f ? codes8(raw[4 * v + i], inv) : make_uint2(0, 0);
        const int pos = v_group_pos((t >> 4) + 16 * v);
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t src = dd < 4 ? k[i].x : k[i].y;
                w |= ((src >> (8 * (dd & 3))) & 0xffu) << (8 * i);
            }
            const int d = 8 * (t & 15) + dd;
            vt[d][vt_col(d, pos)] = w;
        }
    }
    __syncthreads();
    // output block: kQD rows of kQB bytes, 16-byte chunks
    uint4* ob = out + ((bh * (int64_t)(ga.Npad / kQB) + j) * kQD * kQB) / 16;
    for (int ch = t; ch < kQD * kQB / 16; ch += kQThreads) {
        const int d = ch / (kQB / 16), w0 = (ch % (kQB / 16)) * 4;
        const nt_u32x4 w = {vt[d][vt_col(d, w0)], vt[d][vt_col(d, w0 + 1)],
                            vt[d][vt_col(d, w0 + 2)], vt[d][vt_col(d, w0 + 3)]};
        __builtin_nontemporal_store(w, (nt_u32x4*)(ob + ch));       // streamed, like the loads
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
    if ((uint64_t)g.n_blk * (uint64_t)heads * kQThreads > 0xffffffffull)
        return fail(BSA_ERR_UNSUPPORTED, "reorder_quantize_v: %d blocks x %d heads exceed one grid axis",
                    g.n_blk, heads);
    const dim3 grid((unsigned)g.n_blk * (unsigned)heads, (unsigned)batch);
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
