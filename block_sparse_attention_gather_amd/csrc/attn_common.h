// Pieces shared by the bf16 and FP8 attention kernels (internal, not part of the C ABI):
// the persistent scheduler's queue header and workspace layout, the wave-level helpers (XCD
// id, scalar loads of scheduler data, vector-memory waits, the LDS barrier, the cross-half
// exchange) and the fixed-order merge of split rows.
#pragma once

#include "bsa_internal.h"
#include "plan.h"

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

using plan::kNQ;
using plan::kMaxHeads;
using plan::kMaxBlocks;
using plan::kKcMin;
constexpr int kPlanThreads = 1024;
static_assert(kMaxBlocks <= 4096, "the planner packs a row index into 12 bits");
constexpr float kRescaleThresh = 8.0f;   // log2 units the running max may lag

using AttnLayout = plan::Layout;

// header ints: [0] Kc, [1] XCDs per queue, [8 .. 8 + kNQ) queue starts, [32 + 32 q] queue
// counters (128 B apart), [32 + 32 kNQ ..) queue lengths
constexpr int kHdrKc = 0;
constexpr int kHdrGroup = 1;
constexpr int kHdrQStart = 8;
constexpr int kHdrCtr = 32;         // + 32*q
constexpr int kHdrQLen = 32 + 32 * kNQ;
static_assert(plan::kHdrInts == kHdrQLen + kNQ, "header size");

inline AttnLayout attn_layout(int32_t batch, int32_t heads, int32_t D, const Geometry& g,
                              int slots) {
    return plan::workspace_layout((int64_t)batch * heads, g.n_blk, g.B, D, slots);
}

__device__ __forceinline__ int xcc_id() {
    // HW_REG_XCC_ID (hwreg 20), bits [3:0]
    return (int)(__builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & 0xf);
}

__device__ __forceinline__ uint16_t f2bf(float x) {
    const __bf16 b = (__bf16)x;
    return __builtin_bit_cast(uint16_t, b);
}

// Read-only int32 data of the scheduler (CSR columns, work items, header) read through the
// constant address space: uniform indices then compile to scalar loads, which do not share
// the vector-memory counter with the LDS DMA.
typedef __attribute__((address_space(4))) const int32_t cint32;
__device__ __forceinline__ int32_t ld_const(const int32_t* p, int64_t i) {
    return ((cint32*)p)[i];
}
__device__ __forceinline__ int4 ld_const4(const int4* p, int64_t i) {
    const int32_t* q = (const int32_t*)p + 4 * i;
    return make_int4(ld_const(q, 0), ld_const(q, 1), ld_const(q, 2), ld_const(q, 3));
}

template <int D, int B>
struct Tile {
    static constexpr int NW = B / 32;          // wavefronts per workgroup
    static constexpr int NT = NW * 64;         // threads
    static constexpr int KCH = D / 8;          // 16-byte chunks in a K or V row
    static constexpr int NKT = B / 32;         // key tiles of S^T
    static constexpr int NKK = D / 16;         // MFMA k-steps of S^T
    static constexpr int NDT = D / 32;         // d tiles of O^T
    static constexpr int NPK = B / 16;         // MFMA k-steps of O^T
    static constexpr int TI = B * KCH / (NW * 64);   // LDS-DMA instructions per wave per tile
};

// 16-byte-chunk swizzles of the row-major K and V tiles in LDS (row r, logical chunk c is
// stored at chunk c ^ swz(r) of row r):
//  K: the 32 lanes of a half-wave read rows r..r+31 at one chunk (ds_read_b128), so
//     swz(r) = r mod chunks puts any 16 consecutive rows on 16 distinct bank groups;
//  V: ds_read_b64_tr_b16 is served 32 lanes at a time from 64 banks; one half-wave reads 4
//     consecutive rows x 4 adjacent chunks, and swz(r) = 4r mod chunks places those 16
//     chunks on 16 distinct bank groups (measured: no bank-conflict cycles on gfx950).
template <int KCH> __device__ __forceinline__ int swz_k(int r) { return r & (KCH - 1); }
template <int KCH> __device__ __forceinline__ int swz_v(int r) { return (4 * r) & (KCH - 1); }

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt left unconstrained (gfx9 encoding: vmcnt bits
// [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}
__device__ __forceinline__ void wait_vmcnt(int n) {
    if (n == 0) wait_vm<0>();
    else if (n == 4) wait_vm<4>();
    else if (n == 8) wait_vm<8>();
    else wait_vm<0>();
}

// Workgroup barrier that also orders this wave's LDS reads (ds_read results consumed) before
// it; vector-memory traffic (the LDS DMA) is waited for separately with wait_vmcnt.
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
}

// An empty statement that takes an MFMA result, placed before a wait for a tile: the MFMAs that
// produce it are then issued ahead of the wait.  Without such a use the compiler may sink them
// (they touch no memory) below the wait and the barrier after it, and the tile's latency is no
// longer covered by matrix work.
__device__ __forceinline__ void keep_issued(const f32x16& x) { asm volatile("" ::"v"(x)); }

// Value held by lane l ^ 32 (the other half of the wavefront), via v_permlane32_swap.
__device__ __forceinline__ float other_half(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

// A wave-uniform pointer kept in an SGPR pair (the saddr operand of the DMA).
__device__ __forceinline__ const uint16_t* uniform_ptr(const uint16_t* p) {
    const uint64_t sp = (uint64_t)(size_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)sp);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(sp >> 32));
    return (const uint16_t*)(size_t)(((uint64_t)hi << 32) | lo);
}

// Merge the unnormalised partials (O_s, m_s, l_s) of a split row in chunk order:
// O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s.
template <int D, int B>
__device__ __noinline__ void combine_split(const float* __restrict__ part_o,
                                           const float* __restrict__ part_ml,
                                           uint16_t* __restrict__ out, float* __restrict__ lse,
                                           int64_t N, int64_t Npad, int64_t bh, int32_t iblk,
                                           int32_t slot0, int32_t nchunk) {
    constexpr int NT = Tile<D, B>::NT;
    for (int idx = threadIdx.x; idx < B * D; idx += NT) {
        const int qq = idx / D, d = idx % D;
        const int64_t qp = (int64_t)iblk * B + qq;
        float M = -INFINITY;
        for (int c = 0; c < nchunk; ++c)
            M = fmaxf(M, part_ml[((int64_t)(slot0 + c) * B + qq) * 2]);
        float num = 0.f, den = 0.f;
        for (int c = 0; c < nchunk; ++c) {
            const int64_t sl = slot0 + c;
            const float w = __builtin_amdgcn_exp2f(part_ml[(sl * B + qq) * 2] - M);
            num = fmaf(w, part_o[(sl * B + qq) * D + d], num);
            den = fmaf(w, part_ml[(sl * B + qq) * 2 + 1], den);
        }
        const bool real = qp < N;
        out[(bh * Npad + qp) * D + d] = (real && den > 0.f) ? f2bf(num / den) : (uint16_t)0;
        if (d == 0 && lse)
            lse[bh * Npad + qp] =
                (real && den > 0.f) ? (M + __log2f(den)) * 0.69314718055994531f : 0.f;
    }
}

}  // namespace

// Build the persistent schedule of bsa_sparse_attn_fwd for `slots` resident workgroups in the
// workspace laid out by attn_layout(batch, heads, D, g, slots) (defined with the planner);
// head_kv_bytes (K and V of one head as the kernel reads them) sets the queue groups.
bsa_status launch_plan(const int32_t* row_ptr, int32_t batch, int32_t heads, int32_t D,
                       const Geometry& g, int slots, int64_t head_kv_bytes, void* ws,
                       hipStream_t s);

}  // namespace bsa
