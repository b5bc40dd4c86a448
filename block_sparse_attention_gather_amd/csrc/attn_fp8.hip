// FP8 (E4M3) block-sparse attention for head_dim 128 and block 128.
#include "attn_common.h"

namespace bsa {
namespace {

// ---------------------------------------------------------------------------------------
// FP8 attention (VC-Attention page, abstract: both products on low-bit matrix cores, the
// probabilities cast to E4M3 between the exponential and the second product), D = B = 128.
//
// Q and K are E4M3 per 128-token block with fp32 scales (folded into the softmax multiplier
// of each key block); V is E4M3 with one scale per (batch, head), stored per block transposed
// ([D][B] bytes) with its keys in the order one lane holds its probabilities, so both MFMA
// operands that come from LDS are plain 32-byte row reads.  v_mfma_scale_f32_32x32x64_f8f6f4
// with unit scales: A lane l = row l mod 32, B lane l = column l mod 32, and the 32 bytes of
// a lane fill the k-slots of its half-wave; the accumulator has the layout of the 32x32 bf16
// product (element e of lane L: row 8(e/4) + 4(L/32) + e mod 4, column L mod 32), so
// S^T = K Q^T leaves each lane one query and 16 keys per 32-key tile exactly as in the bf16
// kernel.  Probabilities are 2^8 exp(l - m) with m a running maximum that may lag the exact
// one by up to kF8Lag = 0.75 (log2 units; it is raised, and O rescaled, only when a block's
// maximum passes m + 0.75), so every cast value lies in (0, 2^8.75] and stays below E4M3's
// largest finite value 448 (ExpCast code 126 at most).  Two casts:
//   XC = false: exp2 in fp32, then E4M3 with round to nearest even; the row sum is the fp32
//               sum of the uncast values;
//   XC = true:  ExpCast (VC-Attention page, abstract: log-domain scores mapped to E4M3 codes
//               by one fused multiply-add): the code of 2^y is about 8y + 56 (exponent field
//               above the 3 mantissa bits, linear mantissa), so the code is t = 8(s c - m + 8)
//               + 56 rounded to an integer and clamped to [0, 255], with no exponential; the
//               row sum is taken on the matrix cores from the cast values themselves (two
//               16x16x128 MFMAs a block against a 0/1 selector, below).  The FMA yields (t - 2^-8) / 65535 and
//               v_cvt_pknorm_u16_f32 (clamp to [0, 1], x 65535, round to nearest) turns two
//               such values into two 16-bit codes; a byte permute packs four.  The 2^-8 keeps
//               t - code in [-1/2, 1) despite the rounding of the scaled coefficients, which
//               moves t by less than 2^-8 for |m| up to 1000.
// ---------------------------------------------------------------------------------------
struct AttnF8Args {
    const uint8_t* q;       // [bh][Npad][128] e4m3
    const float* qs;        // [bh][n_blk]
    const uint8_t* k;       // [bh][Npad][128] e4m3
    const float* ks;        // [bh][n_blk]
    const uint8_t* v;       // [bh][n_blk][128][128] e4m3, transposed blocks
    const float* vs;        // [bh]
    const int32_t* row_ptr;
    const int32_t* col_idx;
    uint16_t* out;
    float* lse;
    const int32_t* hdr;
    int32_t* ctr;
    const int4* items;
    int32_t* done;
    float* part_o;
    float* part_ml;
    int64_t N, Npad;
    int32_t n_blk;
    float scale_log2;
};

typedef int v8i32 __attribute__((ext_vector_type(8)));
constexpr int kF8Row = 128;                 // bytes per LDS row (D or B fp8 values)
constexpr int kF8TI = 4;                    // DMA instructions per wave per 16 KiB tile
constexpr float kF8Lag = 0.75f;             // allowed lag of the running maximum (log2 units)

// 16-byte chunk c of LDS row r is stored at chunk c ^ ((r / 2) mod 8).  The LDS serves the 16
// lanes of a ds_read_b128 from 256 bytes of banks, i.e. two 128-byte rows: the operand reads
// take 16 consecutive rows at one chunk, and this swizzle puts them on 16 distinct 16-byte bank
// groups (row parity picks the half, the XOR the chunk); c ^ (r mod 8) left rows r and r + 8 on
// the same group (measured: half of all LDS cycles were bank-conflict stalls).
__device__ __forceinline__ int f8_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ uint32_t f8_off(int r, int c) {
    return (uint32_t)(r * kF8Row + ((c ^ f8_swz(r)) << 4));
}

// Instruction u (of kF8TI) of wave wv of the DMA of one 16 KiB fp8 tile: 8 rows, lane i
// writes LDS chunk i mod 8 of row i / 8, fetching the global chunk the swizzle maps there.
__device__ __forceinline__ void dma8_part(const uint8_t* sbase, uint32_t lds_addr, int wv,
                                          int lane, int u) {
    const int lr = lane >> 3, pc = lane & 7;
    const int r0 = (wv * kF8TI + u) * 8;
    const int r = r0 + lr;
    const uint32_t voff = (uint32_t)(lr * kF8Row + ((pc ^ f8_swz(r)) << 4));
    const uint8_t* rowbase = sbase + r0 * kF8Row;
    const uint32_t m0 = lds_addr + (uint32_t)((wv * kF8TI + u) * 1024);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(m0), "v"(voff), "s"(rowbase)
                 : "m0");
}

__device__ __forceinline__ const uint8_t* uniform_ptr8(const uint8_t* p) {
    const uint64_t sp = (uint64_t)(size_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)sp);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(sp >> 32));
    return (const uint8_t*)(size_t)(((uint64_t)hi << 32) | lo);
}

typedef __attribute__((address_space(3))) const char lds_cchar;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x4 lds_cu4;
typedef __attribute__((address_space(4))) const float cfloat;

// 32 bytes of LDS row r, logical chunks 2q and 2q + 1 (q = 2c + h): one MFMA operand
__device__ __forceinline__ v8i32 f8_frag(lds_cchar* base, int r, int q) {
    const u32x4 a = *(lds_cu4*)(base + f8_off(r, 2 * q));
    const u32x4 b = *(lds_cu4*)(base + f8_off(r, 2 * q + 1));
    v8i32 f;
    f[0] = (int)a.x; f[1] = (int)a.y; f[2] = (int)a.z; f[3] = (int)a.w;
    f[4] = (int)b.x; f[5] = (int)b.y; f[6] = (int)b.z; f[7] = (int)b.w;
    return f;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma_f8(const v8i32& a, const v8i32& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Scheduling pin for NM MFMAs that each consume R LDS reads: the reads of the first P MFMAs go
// first, then each MFMA is followed by the reads of the MFMA P places later.
template <int NM, int R, int P>
__device__ __forceinline__ void pin_f8() {
    __builtin_amdgcn_sched_group_barrier(0x100, R * P, 0);          // DS reads
#pragma unroll
    for (int i = 0; i < NM - P; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    }
#pragma unroll
    for (int i = 0; i < P; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

template <bool XC>
__global__ __launch_bounds__(256, 2) void attn_fp8_kernel(AttnF8Args a) {
    constexpr int D = 128, B = 128;
    __shared__ __align__(1024) uint8_t Ks[B * kF8Row];
    __shared__ __align__(1024) uint8_t Vs[D * kF8Row];
    __shared__ int s_pop;
    typedef __attribute__((address_space(3))) char lds_char;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int q0 = (xcc_id() % kNQ) & ~(ld_const(a.hdr, kHdrGroup) - 1);  // first queue
    const int32_t Kc = ld_const(a.hdr, kHdrKc);
    lds_cchar* ks_lds = (lds_cchar*)Ks;
    lds_cchar* vs_lds = (lds_cchar*)Vs;
    const uint32_t ks_addr = (uint32_t)(size_t)(lds_char*)Ks;
    const uint32_t vs_addr = (uint32_t)(size_t)(lds_char*)Vs;

    for (int qo = 0; qo < kNQ; ++qo) {
        const int qi = (q0 + qo) % kNQ;
        const int32_t qlen = ld_const(a.hdr, kHdrQLen + qi);
        const int32_t qstart = ld_const(a.hdr, kHdrQStart + qi);
        while (true) {
            if (t == 0) s_pop = atomicAdd(&a.ctr[32 * qi], 1);
            __syncthreads();
            const int32_t pop = __builtin_amdgcn_readfirstlane(s_pop);
            __syncthreads();
            if (pop >= qlen) break;
            int4 it = ld_const4(a.items, qstart + pop);
            it.x = __builtin_amdgcn_readfirstlane(it.x);
            it.y = __builtin_amdgcn_readfirstlane(it.y);
            it.z = __builtin_amdgcn_readfirstlane(it.z);
            it.w = __builtin_amdgcn_readfirstlane(it.w);
            const int64_t row = it.x;
            const int64_t bh = row / a.n_blk;
            const int32_t iblk = (int32_t)(row - bh * a.n_blk);
            const int64_t qrow0 = (int64_t)iblk * B + wv * 32;
            const uint8_t* kbase = a.k + bh * a.Npad * D;
            const uint8_t* vbase = a.v + bh * a.Npad * D;      // n_blk blocks of D x B bytes
            const float qscale = ((cfloat*)a.qs)[bh * a.n_blk + iblk] * a.scale_log2;
            const float vscale = ((cfloat*)a.vs)[bh];

            // Q^T operand: lane holds query l32, bytes 64c + 32 half .. +32
            v8i32 qf[2];
            {
                const int64_t qpos = qrow0 + l32;
                const uint8_t* qp = a.q + (bh * a.Npad + qpos) * D + 32 * half;
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const uint4 x = qpos < a.N ? *(const uint4*)(qp + 64 * c) : make_uint4(0, 0, 0, 0);
                    const uint4 y = qpos < a.N ? *(const uint4*)(qp + 64 * c + 16) : make_uint4(0, 0, 0, 0);
                    qf[c][0] = (int)x.x; qf[c][1] = (int)x.y; qf[c][2] = (int)x.z; qf[c][3] = (int)x.w;
                    qf[c][4] = (int)y.x; qf[c][5] = (int)y.y; qf[c][6] = (int)y.z; qf[c][7] = (int)y.w;
                }
            }
            wait_vmcnt(0);
            if (it.y < it.z) {              // (a row without blocks is written as zeros)
                const uint8_t* k0 = uniform_ptr8(kbase + (int64_t)ld_const(a.col_idx, it.y) * B * D);
#pragma unroll
                for (int u = 0; u < kF8TI; ++u) dma8_part(k0, ks_addr, wv, lane, u);
            }

            f32x16 o[4];
            f32x4 ol;                       // ExpCast row sum (16x16 MFMA accumulator)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) ol[r] = 0.f;
            float m = -INFINITY, l = 0.f;

            for (int32_t e = it.y; e < it.z; ++e) {
                const int32_t blk = ld_const(a.col_idx, e);
                const bool more = e + 1 < it.z;
                const uint8_t* vsrc = uniform_ptr8(vbase + (int64_t)blk * B * D);
                const uint8_t* ksrc =
                    uniform_ptr8(kbase + (int64_t)(more ? ld_const(a.col_idx, e + 1) : blk) * B * D);
                // (a block of zeros has scale 0: its raw logits are all 0, and the floor keeps
                // the masked pad keys at -inf instead of -inf * 0)
                const float c_blk = fmaxf(qscale * ((cfloat*)a.ks)[bh * a.n_blk + blk], 1.17549435e-38f);
                wait_vm<0>();                            // K_e landed
                barrier_lds();                           // every wave done with V_{e-1}
                // The S MFMAs at issue priority 1, the probabilities and PV (below) at 3: a
                // wavefront in its softmax or PV goes first, one in its S phase before one at
                // the top of its loop (measured 0.5-1.5 % faster than the softmax/PV window
                // alone with ExpCast, the same with the exact cast)
                __builtin_amdgcn_s_setprio(1);
                // S^T = K Q^T: 4 key tiles x 2 chunks of 64 features
                f32x16 s[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[tt][r] = 0.f;
                {
                    v8i32 kf[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int tt = i >> 1, c = i & 1;
                        kf[i] = f8_frag(ks_lds, 32 * tt + l32, 2 * c + half);
                        if (c == 1 && tt < 2) {
#pragma unroll
                            for (int u = 2 * tt; u < 2 * tt + 2; ++u)
                                dma8_part(vsrc, vs_addr, wv, lane, u);
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i) s[i >> 1] = mfma_f8(kf[i], qf[i & 1], s[i >> 1]);
                }
                // every S^T MFMA is issued before the V wait: without this use the compiler sank
                // all eight below the wait and the barrier, so the V tile's arrival was not
                // covered by matrix work (measured 3.4-4.3 % slower)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) keep_issued(s[tt]);
                wait_vm<0>();                            // V_e landed
                barrier_lds();                           // V_e visible; every wave done with K_e
                if (more)
#pragma unroll
                    for (int u = 0; u < kF8TI; ++u) dma8_part(ksrc, ks_addr, wv, lane, u);
                // pad keys of a short last block
                if (a.N - (int64_t)blk * B < B) {
                    const int lim = (int)(a.N - (int64_t)blk * B) - 4 * half;
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            if (32 * tt + 8 * (r >> 2) + (r & 3) >= lim) s[tt][r] = -INFINITY;
                }
                float mx = -INFINITY;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[tt][r]);
                mx = fmaxf(mx, other_half(mx));
                const float mnew = mx * c_blk;
                // (a lagging maximum rescales O rarely; measured 1-3 % faster than raising it
                // with every larger block maximum)
                if (__any(mnew > m + kF8Lag)) {
                    const float mn = fmaxf(m, mnew);
                    const float alpha = __builtin_amdgcn_exp2f(m - mn);
                    l *= alpha;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
                    if (XC)
#pragma unroll
                        for (int r = 0; r < 4; ++r) ol[r] *= alpha;
                    m = mn;
                }
                // issue priority over the other wavefront of the SIMD from the probabilities to the
                // end of the PV MFMAs, as in the bf16 kernel (without any window 7 % slower, same
                // results)
                __builtin_amdgcn_s_setprio(3);
                // probabilities 2^8 exp2(s c - m), cast to E4M3; bytes 16t + e of chunk kc are
                // element e of key tile 2 kc + t
                v8i32 pf[2];
                const float off = 8.0f - m;
                // (floored like c_blk, so that the masked pad keys stay at -inf whatever the
                // denormal mode)
                const float c8 = XC ? fmaxf(8.0f * c_blk * (1.0f / 65535.0f), 1.17549435e-38f) : 0.f;
                const float k8 = XC ? (8.0f * off + 56.0f - 0.00390625f) * (1.0f / 65535.0f) : 0.f;
#pragma unroll
                for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                    for (int w = 0; w < 8; ++w) {
                        const int tt = 2 * kc + (w >> 2);
                        const int r0 = 4 * (w & 3);
                        if (XC) {
                            // 7 vector instructions for four codes (8 with one byte
                            // conversion each: measured 2-3 % slower)
                            const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_u16(
                                fmaf(s[tt][r0 + 0], c8, k8), fmaf(s[tt][r0 + 1], c8, k8)));
                            const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_u16(
                                fmaf(s[tt][r0 + 2], c8, k8), fmaf(s[tt][r0 + 3], c8, k8)));
                            pf[kc][w] = (int)__builtin_amdgcn_perm(lo, hi, 0x02000604u);   // bytes 0, 2 of each
                        } else {
                            float p4[4];
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                p4[j] = __builtin_amdgcn_exp2f(fmaf(s[tt][r0 + j], c_blk, off));
                                l += p4[j];
                            }
                            int pk = __builtin_amdgcn_cvt_pk_fp8_f32(p4[0], p4[1], 0, false);
                            pk = __builtin_amdgcn_cvt_pk_fp8_f32(p4[2], p4[3], pk, true);
                            pf[kc][w] = pk;
                        }
                    }
                // O^T += V^T P^T: 4 feature tiles x 2 chunks of 64 keys
                {
                    v8i32 vf[8];
                    // MFMA i: feature tile dt, key chunk kc.  The exact cast takes the chunks in
                    // turn (its first four MFMAs need only the first chunk's probabilities:
                    // measured 2.6 % faster), ExpCast alternates them (2 % faster with its pinned
                    // V reads)
                    auto dt_of = [](int i) { return XC ? i >> 1 : i & 3; };
                    auto kc_of = [](int i) { return XC ? i & 1 : i >> 2; };
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        vf[i] = f8_frag(vs_lds, 32 * dt_of(i) + l32, 2 * kc_of(i) + half);
#pragma unroll
                    for (int i = 0; i < 8; ++i) o[dt_of(i)] = mfma_f8(vf[i], pf[kc_of(i)], o[dt_of(i)]);
                    // ExpCast: V operands read four MFMAs ahead (left to the compiler, the last
                    // four were read only after the other MFMAs had issued); measured 0.7-1.0 %
                    // faster, while the exact cast ran 1-3 % slower with the same pin
                    if (XC) pin_f8<8, 2, 4>();
                    if (XC) {
                        // Row sum D = A P^T on v_mfma_scale_f32_16x16x128_f8f6f4, with P^T's
                        // registers as they are.  In the 16x16 layout lane j stands for column
                        // j % 16 and key group j / 16 (A's row j % 16), and holds D's rows
                        // 4 (j / 16) .. + 3: lanes j and j + 32 carry query j % 16's keys,
                        // j + 16 and j + 48 those of query j % 16 + 16.  A is 1 (E4M3 0x38)
                        // where the row's quartet parity equals the key group's parity, else
                        // 0, so D's row quartets 0 and 2 sum query n, 1 and 3 query n + 16:
                        // every lane receives its own query's sum, and each block costs two
                        // MFMAs of 8 passes instead of two 32x32x64 ones of 16 (measured
                        // 2.4 % faster on HunyuanVideo, 3-7 % on Wan-480p, same output)
                        const int sel = ((lane >> 2) ^ (lane >> 4)) & 1;
                        v8i32 ones;
#pragma unroll
                        for (int w = 0; w < 8; ++w) ones[w] = sel ? 0 : 0x38383838;
                        ol = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pf[0], ol, 0, 0, 0,
                                                                           127, 0, 127);
                        ol = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pf[1], ol, 0, 0, 0,
                                                                           127, 0, 127);
                    }
                }
                __builtin_amdgcn_s_setprio(0);
            }

            // (ExpCast: each of the lane's four row-sum values is its query's sum)
            const float lt = XC ? ol[0] : l + other_half(l);
            const int64_t qpos = qrow0 + l32;
            if (it.w < 0) {
                const float inv = lt > 0.f ? vscale / lt : 0.f;
                const bool real = qpos < a.N;
                uint16_t* op = a.out + (bh * a.Npad + qpos) * D;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int d = 32 * dt + 8 * g4 + 4 * half;
                        ushort4 pk;
                        pk.x = real ? f2bf(o[dt][4 * g4 + 0] * inv) : 0;
                        pk.y = real ? f2bf(o[dt][4 * g4 + 1] * inv) : 0;
                        pk.z = real ? f2bf(o[dt][4 * g4 + 2] * inv) : 0;
                        pk.w = real ? f2bf(o[dt][4 * g4 + 3] * inv) : 0;
                        *(ushort4*)(op + d) = pk;
                    }
                if (a.lse && half == 0)
                    a.lse[bh * a.Npad + qpos] =
                        (real && lt > 0.f) ? (m - 8.0f + __log2f(lt)) * 0.69314718055994531f : 0.f;
            } else {
                // split row: partial O (V scale applied) and (m - 8, l) in the bf16 kernel's
                // format, merged by combine_split
                const int32_t rbeg = a.row_ptr[row];
                const int32_t cnt = a.row_ptr[row + 1] - rbeg;
                const int32_t chunk = (it.y - rbeg) / Kc;
                const int32_t nchunk = (cnt + Kc - 1) / Kc;
                const int64_t slot = it.w + chunk;
                float* po = a.part_o + (slot * B + wv * 32 + l32) * D;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int d = 32 * dt + 8 * g4 + 4 * half;
                        *(float4*)(po + d) = make_float4(vscale * o[dt][4 * g4], vscale * o[dt][4 * g4 + 1],
                                                         vscale * o[dt][4 * g4 + 2], vscale * o[dt][4 * g4 + 3]);
                    }
                if (half == 0) {
                    a.part_ml[(slot * B + wv * 32 + l32) * 2 + 0] = m - 8.0f;
                    a.part_ml[(slot * B + wv * 32 + l32) * 2 + 1] = lt;
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                __syncthreads();
                if (t == 0) s_pop = atomicAdd(&a.done[it.w], 1);
                __syncthreads();
                const int32_t prev = s_pop;
                __syncthreads();
                if (prev == nchunk - 1) {
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    combine_split<D, B>(a.part_o, a.part_ml, a.out, a.lse, a.N, a.Npad, bh, iblk,
                                        it.w, nchunk);
                }
            }
        }
    }
}

int occupancy_fp8() {
    int nb = 0, nx = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, attn_fp8_kernel<false>, 256, 0) !=
            hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&nx, attn_fp8_kernel<true>, 256, 0) !=
            hipSuccess)
        return 1;
    nb = nb < nx ? nb : nx;                      // one workspace size serves both casts
    return nb < 1 ? 1 : nb;
}


}  // namespace

int attn_fp8_slots(const DeviceInfo& dev) { return dev.cu_count * occupancy_fp8(); }

bsa_status launch_attn_fp8(const void* q8, const float* qs, const void* k8, const float* ks,
                           const void* v8, const float* vs, const int32_t* row_ptr,
                           const int32_t* col_idx, int32_t batch, int32_t heads,
                           const Geometry& g, float scale, int32_t expcast, void* out_t,
                           float* lse, void* ws, const DeviceInfo& dev, hipStream_t s) {
    const int slots = attn_fp8_slots(dev);
    const AttnLayout L = attn_layout(batch, heads, 128, g, slots);
    unsigned char* w = (unsigned char*)ws;
    int32_t* hdr = (int32_t*)(w + L.hdr);
    int4* items = (int4*)(w + L.items);
    int32_t* done = (int32_t*)(w + L.done);
    // K and V of a head, E4M3
    bsa_status st = launch_plan(row_ptr, batch, heads, 128, g, slots, 2 * g.Npad * 128, ws, s);
    if (st != BSA_OK) return st;
    AttnF8Args a;
    a.q = (const uint8_t*)q8;
    a.qs = qs;
    a.k = (const uint8_t*)k8;
    a.ks = ks;
    a.v = (const uint8_t*)v8;
    a.vs = vs;
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.out = (uint16_t*)out_t;
    a.lse = lse;
    a.hdr = hdr;
    a.ctr = hdr + kHdrCtr;
    a.items = items;
    a.done = done;
    a.part_o = (float*)(w + L.part_o);
    a.part_ml = (float*)(w + L.part_ml);
    a.N = g.N;
    a.Npad = g.Npad;
    a.n_blk = g.n_blk;
    a.scale_log2 = scale * 1.4426950408889634f;
    if (expcast)
        hipLaunchKernelGGL(attn_fp8_kernel<true>, dim3(slots), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(attn_fp8_kernel<false>, dim3(slots), dim3(256), 0, s, a);
    return check_launch("sparse_attn_fp8");
}

}  // namespace bsa
