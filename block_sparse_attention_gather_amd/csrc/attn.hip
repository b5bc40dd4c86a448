// Exact block-sparse attention forward over CSR key-block lists, bf16 MFMA on gfx950.
//
// What is computed (FVAttn page, abstract: attention over the materialized block mask; PSA
// page, "Approach": one block-sparse kernel; VC-Attention abstract: the running row maximum
// and row sum of an online softmax): for each real query of block i, softmax attention over
// the real keys of the blocks listed for row (b, h, i), evaluated block by block with an
// online softmax (running max m, running sum l, rescaled accumulator).
//
// Scheduling (FVAttn page, abstract: adaptive Top-p gives uneven per-head work; its runtime
// load balancing moves heavy heads between GPUs - here the same problem is solved between the
// compute units of one GPU):
//   plan_global  one workgroup: chunk size Kc from nnz, per-head work, heads assigned to the
//                8 XCD queues longest-first (each head's K/V then stays in one XCD's L2),
//                queue offsets, counters reset.
//   plan_rows    one workgroup per head: rows ordered by cost descending (ties: row order),
//                rows longer than Kc split into chunks, work items written in queue order.
//   attn         persistent: each workgroup reads its XCD id, pops items from its own queue
//                with an atomic counter, then steals from the other queues; every queue is
//                visited once after it runs dry, so every workgroup exits.  A split row's
//                chunks store unnormalised partials; the chunk that finishes last merges them
//                in chunk order, so results do not depend on timing.
//
// Data layout of one work item (B = 128, D = 128; B = D = 64 analogous): 4 wavefronts, each
// owning 32 query rows.  S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T in
// registers) leaves each lane one query and 16 keys per 32x32 tile, so the row max is one
// cross-half exchange and the row sum stays per lane until the end.  P^T is already the B
// operand layout of O^T = V^T P^T.  K and V tiles are copied row-major into LDS by LDS-DMA
// (global_load_lds); K operands are plain 16-byte reads, V^T operands are transposing reads
// (ds_read_b64_tr_b16), and the 16-byte chunks of each tile row are XOR-swizzled by the row
// index (K: c ^ (r mod C), V: c ^ (4r mod C), C = D/8 chunks a row) so neither read pattern
// has bank conflicts.
#include "bsa_internal.h"

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kNQ = 8;             // XCD queues (MI355X: 8 XCDs)
constexpr int kPlanThreads = 1024;
constexpr int kMaxHeads = 2048;    // batch * heads supported by the planner
constexpr int kMaxBlocks = 4096;   // n_blk supported by the planner
static_assert(kMaxBlocks <= 4096, "the planner packs a row index into 12 bits");
constexpr int kKcMin = 8;          // smallest chunk (blocks) a row is split into
constexpr float kRescaleThresh = 8.0f;   // log2 units the running max may lag

struct AttnLayout {
    size_t hdr, head_item_off, head_slot_base, items, done, part_o, part_ml, total;
    int64_t max_items, max_slots;
};

// header ints: [0] Kc, [16 + 32 q] queue counters (128 B apart), [8 .. 8+kNQ) qstart,
// [272 ..) qlen
constexpr int kHdrKc = 0;
constexpr int kHdrQStart = 8;
constexpr int kHdrCtr = 32;         // + 32*q
constexpr int kHdrQLen = 32 + 32 * kNQ;
constexpr int kHdrInts = kHdrQLen + kNQ;

AttnLayout attn_layout(int32_t batch, int32_t heads, int32_t D, const Geometry& g,
                       int slots) {
    AttnLayout L;
    const int64_t bh = (int64_t)batch * heads;
    const int64_t rows = bh * g.n_blk;
    const int64_t target = 2 * (int64_t)slots;
    L.max_items = rows + target;
    L.max_slots = 2 * target;
    size_t off = 0;
    L.hdr = off;            off = align_up(off + kHdrInts * 4, 256);
    L.head_item_off = off;  off = align_up(off + bh * 4, 256);
    L.head_slot_base = off; off = align_up(off + bh * 4, 256);
    L.items = off;          off = align_up(off + L.max_items * 16, 256);
    L.done = off;           off = align_up(off + L.max_slots * 4, 256);
    L.part_o = off;         off = align_up(off + (size_t)L.max_slots * g.B * D * 4, 256);
    L.part_ml = off;        off = align_up(off + (size_t)L.max_slots * g.B * 2 * 4, 256);
    L.total = off;
    return L;
}

// ---------------------------------------------------------------------------------------
// planner
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(kPlanThreads) void plan_global_kernel(
    const int32_t* __restrict__ row_ptr, int32_t n_blk, int32_t nbh, int32_t target,
    int32_t* __restrict__ hdr, int32_t* __restrict__ head_item_off,
    int32_t* __restrict__ head_slot_base) {
    __shared__ int32_t hitems[kMaxHeads], hslots[kMaxHeads], hcost[kMaxHeads];
    __shared__ int32_t horder[kMaxHeads], hqueue[kMaxHeads];
    __shared__ int64_t qload[kNQ];
    __shared__ int32_t qlen[kNQ], qstart[kNQ], qrun[kNQ];
    const int t = threadIdx.x;
    const int64_t rows = (int64_t)nbh * n_blk;
    const int64_t total = row_ptr[rows];
    int64_t kc64 = (total + target - 1) / target;
    const int32_t Kc = (int32_t)(kc64 < kKcMin ? kKcMin : kc64);
    for (int h = t; h < nbh; h += kPlanThreads)
        hcost[h] = row_ptr[(int64_t)(h + 1) * n_blk] - row_ptr[(int64_t)h * n_blk];
    // work items and partial slots per head: one wavefront sums one head's rows
    {
        const int lane = t & 63, w = t >> 6;
        for (int h = w; h < nbh; h += kPlanThreads / 64) {
            int32_t ni_sum = 0, ns_sum = 0;
#pragma unroll 8
            for (int i = lane; i < n_blk; i += 64) {
                const int64_t r = (int64_t)h * n_blk + i;
                const int32_t c = row_ptr[r + 1] - row_ptr[r];
                int32_t ni = (c + Kc - 1) / Kc;
                ni = ni < 1 ? 1 : ni;
                ni_sum += ni;
                ns_sum += ni > 1 ? ni : 0;
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                ni_sum += __shfl_xor(ni_sum, off, 64);
                ns_sum += __shfl_xor(ns_sum, off, 64);
            }
            if (lane == 0) {
                hitems[h] = ni_sum;
                hslots[h] = ns_sum;
            }
        }
    }
    __syncthreads();
    // heads ranked by cost (kept blocks) descending, ties by index
    for (int h = t; h < nbh; h += kPlanThreads) {
        const int32_t ch = hcost[h];
        int rk = 0;
        for (int h2 = 0; h2 < nbh; ++h2) {
            const int32_t c2 = hcost[h2];
            rk += (c2 > ch) || (c2 == ch && h2 < h);
        }
        horder[rk] = h;
    }
    __syncthreads();
    if (t == 0) {
        for (int q = 0; q < kNQ; ++q) { qload[q] = 0; qlen[q] = 0; qrun[q] = 0; }
        // longest-processing-time-first: each head to the least-loaded queue
        for (int k = 0; k < nbh; ++k) {
            const int h = horder[k];
            int best = 0;
            for (int q = 1; q < kNQ; ++q)
                if (qload[q] < qload[best]) best = q;
            qload[best] += hcost[h];
            qlen[best] += hitems[h];
            hqueue[h] = best;
        }
        int32_t acc = 0;
        for (int q = 0; q < kNQ; ++q) { qstart[q] = acc; acc += qlen[q]; }
        for (int k = 0; k < nbh; ++k) {
            const int h = horder[k];
            const int q = hqueue[h];
            head_item_off[h] = qstart[q] + qrun[q];
            qrun[q] += hitems[h];
        }
        int32_t sacc = 0;
        for (int h = 0; h < nbh; ++h) { head_slot_base[h] = sacc; sacc += hslots[h]; }
        hdr[kHdrKc] = Kc;
        for (int q = 0; q < kNQ; ++q) {
            hdr[kHdrQStart + q] = qstart[q];
            hdr[kHdrQLen + q] = qlen[q];
            hdr[kHdrCtr + 32 * q] = 0;
        }
    }
}

__global__ __launch_bounds__(kPlanThreads) void plan_rows_kernel(
    const int32_t* __restrict__ row_ptr, int32_t n_blk, const int32_t* __restrict__ hdr,
    const int32_t* __restrict__ head_item_off, const int32_t* __restrict__ head_slot_base,
    int4* __restrict__ items, int32_t* __restrict__ done) {
    __shared__ int32_t cost[kMaxBlocks], ord[kMaxBlocks], ipos[kMaxBlocks], spos[kMaxBlocks];
    __shared__ int32_t part_i[kPlanThreads], part_s[kPlanThreads];
    const int t = threadIdx.x;
    const int h = blockIdx.x;
    const int64_t base = (int64_t)h * n_blk;
    const int32_t Kc = hdr[kHdrKc];
    for (int i = t; i < n_blk; i += kPlanThreads) cost[i] = row_ptr[base + i + 1] - row_ptr[base + i];
    __syncthreads();
    // rows by cost descending, ties by row index: bitonic sort of one 32-bit word per row,
    // (kMaxBlocks - cost) above the 12-bit row index, padding words last
    int P2 = 2;
    while (P2 < n_blk) P2 <<= 1;
    uint32_t* key = (uint32_t*)ord;
    for (int i = t; i < P2; i += kPlanThreads)
        key[i] = i < n_blk ? ((uint32_t)(kMaxBlocks - cost[i]) << 12) | (uint32_t)i : 0xffffffffu;
    __syncthreads();
    for (int kk = 2; kk <= P2; kk <<= 1)
        for (int jj = kk >> 1; jj > 0; jj >>= 1) {
            for (int i = t; i < P2; i += kPlanThreads) {
                const int l = i ^ jj;
                if (l > i) {
                    const uint32_t x = key[i], y = key[l];
                    if ((x > y) == ((i & kk) == 0)) {
                        key[i] = y;
                        key[l] = x;
                    }
                }
            }
            __syncthreads();
        }
    for (int k = t; k < n_blk; k += kPlanThreads) ord[k] = (int32_t)(key[k] & 0xfffu);
    __syncthreads();
    // exclusive scans (in rank order) of items per row and of partial slots per split row
    const int seg = (n_blk + kPlanThreads - 1) / kPlanThreads;
    const int lo = min(n_blk, t * seg), hi = min(n_blk, lo + seg);
    int32_t li = 0, ls = 0;
    for (int k = lo; k < hi; ++k) {
        int32_t ni = (cost[ord[k]] + Kc - 1) / Kc;
        ni = ni < 1 ? 1 : ni;
        li += ni;
        ls += ni > 1 ? ni : 0;
    }
    part_i[t] = li;
    part_s[t] = ls;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        const int32_t ai = t >= off ? part_i[t - off] : 0;
        const int32_t as = t >= off ? part_s[t - off] : 0;
        __syncthreads();
        part_i[t] += ai;
        part_s[t] += as;
        __syncthreads();
    }
    int32_t ri = part_i[t] - li, rs = part_s[t] - ls;
    for (int k = lo; k < hi; ++k) {
        int32_t ni = (cost[ord[k]] + Kc - 1) / Kc;
        ni = ni < 1 ? 1 : ni;
        ipos[k] = ri;
        spos[k] = rs;
        ri += ni;
        rs += ni > 1 ? ni : 0;
    }
    __syncthreads();
    const int32_t ioff = head_item_off[h];
    const int32_t sbase = head_slot_base[h];
    for (int k = t; k < n_blk; k += kPlanThreads) {
        const int i = ord[k];
        const int32_t c = cost[i];
        const int32_t beg = row_ptr[base + i];
        int32_t ni = (c + Kc - 1) / Kc;
        ni = ni < 1 ? 1 : ni;
        const int32_t slot = ni > 1 ? sbase + spos[k] : -1;
        for (int s = 0; s < ni; ++s) {
            const int32_t b0 = beg + s * Kc;
            const int32_t b1 = min(beg + (s + 1) * Kc, beg + c);
            items[ioff + ipos[k] + s] = make_int4((int32_t)(base + i), b0, b1, slot);
        }
        if (slot >= 0) done[slot] = 0;
    }
}

// ---------------------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------------------
#ifdef BSA_TRACE
// Debug build only (libbsa_trace.so): one record per workgroup of the latest attention launch,
// s_memrealtime (100 MHz) stamps at kernel entry, after the workgroup's last work item and at
// exit, s_memtime (shader clock) stamps at entry and exit, the hardware placement and the work
// done.  Read with bsa_trace_read().
constexpr int kTraceMax = 8192;
struct TraceRec {
    unsigned long long t0, t_last, t_end, c0, c_end;
    uint32_t hw_id, xcc;
    int32_t items, blocks;
};
__device__ TraceRec g_trace_rec[kTraceMax];
#endif

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    uint16_t* out;
    float* lse;
    const int32_t* hdr;
    int32_t* ctr;           // queue counters (hdr + kHdrCtr), 32 ints apart
    const int4* items;
    int32_t* done;
    float* part_o;
    float* part_ml;
    int64_t N, Npad;
    int32_t n_blk;
    float scale_log2;       // softmax scale * log2(e)
};

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

// Enqueue the B x D bf16 tile at `src` (row-major) into LDS at byte address `lds_addr` by
// LDS DMA (global_load_lds_dwordx4: each lane's 16 bytes land at M0 + 16*lane).  Wave w
// writes chunks [w*TI*64, (w+1)*TI*64) of the tile, i.e. 64/KCH whole rows per instruction,
// fetching for each LDS chunk the global chunk the swizzle maps there.  Rows past N of the
// last block are read too (they lie inside the Npad-row tensor; the caller masks them).
// Issued as inline assembly so that the compiler does not serialise every later LDS read
// behind it; completion is awaited explicitly with wait_vmcnt (vector-memory operations
// retire in order).
template <int D, int B, bool IS_V>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ src, uint32_t lds_addr,
                                         int wv, int lane) {
    using Tl = Tile<D, B>;
    constexpr int RPI = 64 / Tl::KCH;                        // rows per instruction
    const uint64_t sp = (uint64_t)(size_t)src;               // wave-uniform: SGPR pair
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)sp);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(sp >> 32));
    const uint16_t* sbase = (const uint16_t*)(size_t)(((uint64_t)hi << 32) | lo);
    const int lr = lane / Tl::KCH;                           // row inside the instruction
    const int pc = lane % Tl::KCH;                           // LDS chunk inside the row
#pragma unroll
    for (int u = 0; u < Tl::TI; ++u) {
        const int r0 = (wv * Tl::TI + u) * RPI;              // first row (uniform)
        const int r = r0 + lr;
        const int lc = pc ^ (IS_V ? swz_v<Tl::KCH>(r) : swz_k<Tl::KCH>(r));
        const uint32_t voff = (uint32_t)((lr * D + lc * 8) * 2);
        const uint16_t* rowbase = sbase + r0 * D;
        const uint32_t m0 = lds_addr + (uint32_t)((wv * Tl::TI + u) * 64 * 16);
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "s"(m0), "v"(voff), "s"(rowbase)
                     : "memory", "m0");
    }
}

// One instruction (u) of dma_tile, for spreading a tile's DMA between compute instructions.
// No memory clobber: LDS reads of the other buffer may be scheduled across it, while the
// volatile statement keeps its place relative to barriers and waits.
template <int D, int B, bool IS_V>
__device__ __forceinline__ void dma_part(const uint16_t* sbase, uint32_t lds_addr, int wv,
                                         int lane, int u) {
    using Tl = Tile<D, B>;
    constexpr int RPI = 64 / Tl::KCH;
    const int lr = lane / Tl::KCH;
    const int pc = lane % Tl::KCH;
    const int r0 = (wv * Tl::TI + u) * RPI;
    const int r = r0 + lr;
    const int lc = pc ^ (IS_V ? swz_v<Tl::KCH>(r) : swz_k<Tl::KCH>(r));
    const uint32_t voff = (uint32_t)((lr * D + lc * 8) * 2);
    const uint16_t* rowbase = sbase + r0 * D;
    const uint32_t m0 = lds_addr + (uint32_t)((wv * Tl::TI + u) * 64 * 16);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(m0), "v"(voff), "s"(rowbase)
                 : "m0");
}

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

// Scheduling pin for an operand pipeline of NM MFMAs that each consume R LDS reads: the reads
// of the first kPrefetch MFMAs go first, then every MFMA is followed by the reads of the MFMA
// kPrefetch places later, so each MFMA's operands were requested about kPrefetch MFMAs (~130
// cycles of matrix-core work) before it issues instead of immediately before it.
constexpr int kPrefetch = 4;
template <int NM, int R>
__device__ __forceinline__ void pin_pipeline() {
    __builtin_amdgcn_sched_group_barrier(0x100, R * kPrefetch, 0);     // DS reads
#pragma unroll
    for (int i = 0; i < NM - kPrefetch; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    }
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

template <int D, int B>
__global__ __launch_bounds__(2 * B, 2) void attn_kernel(AttnArgs a) {
    using Tl = Tile<D, B>;
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    __shared__ __align__(1024) uint16_t Ks[B * D];
    __shared__ __align__(1024) uint16_t Vs[B * D];
    __shared__ int s_pop;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform, kept in an SGPR
    const int half = lane >> 5;      // 0 / 1
    const int l32 = lane & 31;
    const int q0 = xcc_id() % kNQ;
    const int32_t Kc = ld_const(a.hdr, kHdrKc);
#ifdef BSA_TRACE
    const unsigned long long tr_t0 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long tr_c0 = __builtin_amdgcn_s_memtime();
    unsigned long long tr_last = tr_t0;
    int32_t tr_items = 0, tr_blocks = 0;
#endif

    // per-lane LDS byte offsets of the MFMA operand reads (constant over the whole kernel)
    //  K (A of S^T): row 32 tt + l32, logical chunk 2 kk + half
    //  V (A of O^T, transposed read): 16-lane group g = lane / 16 reads rows
    //    32 t + 16 m + 8 s + 4 half + j / 4 (j = lane % 16) at columns 32 dt + 16 (g % 2) + 4 (j % 4)
    const int j16 = lane & 15;
    const int g16 = lane >> 4;
    const int vrow0 = 4 * half + (j16 >> 2);               // row inside a 16-row step, s = 0
    const int vsw = swz_v<Tl::KCH>(vrow0);                 // same for every step (2r mod KCH)
    typedef __attribute__((address_space(3))) char lds_char;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    lds_char* const vs_lds = (lds_char*)Vs;
    const uint32_t ks_addr = (uint32_t)(size_t)(lds_char*)Ks;
    const uint32_t vs_addr = (uint32_t)(size_t)vs_lds;

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
            it.x = __builtin_amdgcn_readfirstlane(it.x);        // the item is workgroup-uniform
            it.y = __builtin_amdgcn_readfirstlane(it.y);
            it.z = __builtin_amdgcn_readfirstlane(it.z);
            it.w = __builtin_amdgcn_readfirstlane(it.w);
            const int64_t row = it.x;
            const int64_t bh = row / a.n_blk;
            const int32_t iblk = (int32_t)(row - bh * a.n_blk);
            const int64_t qrow0 = (int64_t)iblk * B + wv * 32;   // first query row of wave
            const uint16_t* kbase = a.k + bh * a.Npad * D;
            const uint16_t* vbase = a.v + bh * a.Npad * D;

            // Q^T operand: lane holds query l32, d = 16 kk + 8 half .. +8
            bf16x8 qf[Tl::NKK];
            {
                const int64_t qpos = qrow0 + l32;
                const uint16_t* qp = a.q + (bh * a.Npad + qpos) * D + 8 * half;
#pragma unroll
                for (int kk = 0; kk < Tl::NKK; ++kk) {
                    uint4 raw = qpos < a.N ? *(const uint4*)(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
                    qf[kk] = __builtin_bit_cast(bf16x8, raw);
                }
            }
            // Q is in registers before the first LDS DMA of the item is issued, so the only
            // vector-memory operations in flight inside the block loop are the DMA tiles
            wait_vmcnt(0);
            // first key block of the item into LDS
            dma_tile<D, B, false>(kbase + (int64_t)ld_const(a.col_idx, it.y) * B * D, ks_addr, wv,
                                  lane);

            f32x16 o[Tl::NDT];
#pragma unroll
            for (int dt = 0; dt < Tl::NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
            float m = -INFINITY, l = 0.f;

            for (int32_t e = it.y; e < it.z; ++e) {
                const int32_t blk = ld_const(a.col_idx, e);
                const bool more = e + 1 < it.z;
                const uint16_t* vsrc = uniform_ptr(vbase + (int64_t)blk * B * D);
                const uint16_t* ksrc =
                    uniform_ptr(kbase + (int64_t)(more ? ld_const(a.col_idx, e + 1) : blk) * B * D);
                // K_e landed (the only DMA in flight); after the barrier every wave is done
                // with V_{e-1}, so V_e streams into the V buffer during the first half of S_e
                wait_vm<0>();
                barrier_lds();
                // S^T = K Q^T
                f32x16 s[Tl::NKT];
#pragma unroll
                for (int tt = 0; tt < Tl::NKT; ++tt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[tt][r] = 0.f;
                {
                    // K operands are read kPrefetch MFMAs ahead of their use (order pinned
                    // below); the V DMA parts go out during the first half of the reads
                    constexpr int NM = Tl::NKK * Tl::NKT;
                    bf16x8 kf[NM];
#pragma unroll
                    for (int i = 0; i < NM; ++i) {
                        const int kk = i / Tl::NKT, tt = i % Tl::NKT;
                        const int pch = (2 * kk + half) ^ swz_k<Tl::KCH>(l32);
                        kf[i] = *(const bf16x8*)(Ks + (32 * tt + l32) * D + pch * 8);
                        if (tt == Tl::NKT - 1) {
#pragma unroll
                            for (int u = kk * 2 * Tl::TI / Tl::NKK;
                                 u < (kk + 1) * 2 * Tl::TI / Tl::NKK; ++u)
                                if (u < Tl::TI) dma_part<D, B, true>(vsrc, vs_addr, wv, lane, u);
                        }
                    }
#pragma unroll
                    for (int i = 0; i < NM; ++i) {
                        const int kk = i / Tl::NKT, tt = i % Tl::NKT;
                        s[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[kk], s[tt], 0, 0, 0);
                    }
                    pin_pipeline<NM, 1>();
                }
                wait_vm<0>();                            // V_e landed
                barrier_lds();                           // V_e visible; every wave done with K_e
                // pad keys of a short last block
                if (a.N - (int64_t)blk * B < B) {
                    const int lim = (int)(a.N - (int64_t)blk * B) - 4 * half;
#pragma unroll
                    for (int tt = 0; tt < Tl::NKT; ++tt)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            if (32 * tt + 8 * (r >> 2) + (r & 3) >= lim) s[tt][r] = -INFINITY;
                }
                // online softmax (log2 domain, lazy rescale)
                float mx = -INFINITY;
#pragma unroll
                for (int tt = 0; tt < Tl::NKT; ++tt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[tt][r]);
                mx = fmaxf(mx, other_half(mx));
                const float mnew = mx * a.scale_log2;
                if (__any(mnew > m + kRescaleThresh)) {
                    const float mn = fmaxf(m, mnew);
                    const float alpha = __builtin_amdgcn_exp2f(m - mn);
                    l *= alpha;
#pragma unroll
                    for (int dt = 0; dt < Tl::NDT; ++dt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
                    m = mn;
                }
                // softmax of the block (VALU), then O^T += V^T P^T (MFMA) with the V^T operands
                // read from row-major V by transposed LDS reads, kPrefetch MFMAs ahead
                bf16x8 pf[Tl::NPK];
                auto softmax_tile = [&](int tt) {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                        for (int e8 = 0; e8 < 8; ++e8) {
                            const float p = __builtin_amdgcn_exp2f(
                                fmaf(s[tt][8 * hh + e8], a.scale_log2, -m));
                            l += p;
                            pf[2 * tt + hh][e8] = (__bf16)p;
                        }
                };
                // K_{e+1} streams into the K buffer (every wave finished S_e before the last
                // barrier) while the softmax and PV run
                constexpr int KPT = Tl::TI / Tl::NKT;    // K DMA instructions per key tile
#pragma unroll
                for (int tt = 0; tt < Tl::NKT; ++tt) {
                    softmax_tile(tt);
                    if (more)
#pragma unroll
                        for (int u = tt * KPT; u < (tt + 1) * KPT; ++u)
                            dma_part<D, B, false>(ksrc, ks_addr, wv, lane, u);
                }
                {
                    constexpr int NM = Tl::NPK * Tl::NDT;
                    bf16x8 vfr[NM];
#pragma unroll
                    for (int i = 0; i < NM; ++i) {
                        const int ks = i / Tl::NDT, dt = i % Tl::NDT;
                        const int lc = 4 * dt + 2 * (g16 & 1) + ((j16 & 3) >> 1);
                        const uint32_t col_off = (uint32_t)(((lc ^ vsw) * 16) + (j16 & 1) * 8);
                        lds_char* p0 = vs_lds + (16 * ks + vrow0) * D * 2 + col_off;
                        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
                        const s16x4 hi =
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 8 * D * 2));
                        vfr[i] = __builtin_bit_cast(
                            bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    }
#pragma unroll
                    for (int i = 0; i < NM; ++i) {
                        const int ks = i / Tl::NDT, dt = i % Tl::NDT;
                        o[dt] =
                            __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[i], pf[ks], o[dt], 0, 0, 0);
                    }
                    pin_pipeline<NM, 2>();
                }
            }

            const float lt = l + other_half(l);
            const int64_t qpos = qrow0 + l32;
            if (it.w < 0) {
                // whole row in this item: normalise and store
                const float inv = lt > 0.f ? 1.f / lt : 0.f;
                const bool real = qpos < a.N;
                uint16_t* op = a.out + (bh * a.Npad + qpos) * D;
#pragma unroll
                for (int dt = 0; dt < Tl::NDT; ++dt)
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
                        (real && lt > 0.f) ? (m + __log2f(lt)) * 0.69314718055994531f : 0.f;
            } else {
                // one chunk of a split row: store the unnormalised partial
                const int32_t rbeg = a.row_ptr[row];
                const int32_t cnt = a.row_ptr[row + 1] - rbeg;
                const int32_t chunk = (it.y - rbeg) / Kc;
                const int32_t nchunk = (cnt + Kc - 1) / Kc;
                const int64_t slot = it.w + chunk;
                float* po = a.part_o + (slot * B + wv * 32 + l32) * D;
#pragma unroll
                for (int dt = 0; dt < Tl::NDT; ++dt)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int d = 32 * dt + 8 * g4 + 4 * half;
                        *(float4*)(po + d) = make_float4(o[dt][4 * g4], o[dt][4 * g4 + 1],
                                                         o[dt][4 * g4 + 2], o[dt][4 * g4 + 3]);
                    }
                if (half == 0) {
                    a.part_ml[(slot * B + wv * 32 + l32) * 2 + 0] = m;
                    a.part_ml[(slot * B + wv * 32 + l32) * 2 + 1] = lt;
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                __syncthreads();
                if (t == 0) s_pop = atomicAdd(&a.done[it.w], 1);
                __syncthreads();
                const int32_t prev = s_pop;
                __syncthreads();
                if (prev == nchunk - 1) {
                    // last chunk to finish: merge all partials in chunk order
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    combine_split<D, B>(a.part_o, a.part_ml, a.out, a.lse, a.N, a.Npad, bh, iblk,
                                        it.w, nchunk);
                }
            }
#ifdef BSA_TRACE
            tr_last = __builtin_amdgcn_s_memrealtime();
            ++tr_items;
            tr_blocks += it.z - it.y;
#endif
        }
    }
#ifdef BSA_TRACE
    if (t == 0 && blockIdx.x < kTraceMax) {
        TraceRec r;
        r.t0 = tr_t0;
        r.t_last = tr_last;
        r.t_end = __builtin_amdgcn_s_memrealtime();
        r.c0 = tr_c0;
        r.c_end = __builtin_amdgcn_s_memtime();
        r.hw_id = __builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));   // HW_REG_HW_ID
        r.xcc = (uint32_t)xcc_id();
        r.items = tr_items;
        r.blocks = tr_blocks;
        g_trace_rec[blockIdx.x] = r;
    }
#endif
}

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
// kernel.  Probabilities are 2^8 exp(l - m) with m the exact running maximum (rescaled as soon
// as it grows), so every cast value lies in (0, 256].  Two casts:
//   XC = false: exp2 in fp32, then E4M3 with round to nearest even; the row sum is the fp32
//               sum of the uncast values;
//   XC = true:  ExpCast (VC-Attention page, abstract: log-domain scores mapped to E4M3 codes
//               by one fused multiply-add): the code of 2^y is about 8y + 56 (exponent field
//               above the 3 mantissa bits, linear mantissa), so code = u8(8(s c - m + 8) + 56)
//               with no exponential; the row sum is taken by two more MFMAs against an
//               all-ones V tile, so it sums exactly the cast values.
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

// 16-byte chunk c of LDS row r is stored at chunk c ^ (r mod 8).
__device__ __forceinline__ uint32_t f8_off(int r, int c) {
    return (uint32_t)(r * kF8Row + ((c ^ (r & 7)) << 4));
}

// Instruction u (of kF8TI) of wave wv of the DMA of one 16 KiB fp8 tile: 8 rows, lane i
// writes LDS chunk i mod 8 of row i / 8, fetching the global chunk the swizzle maps there.
__device__ __forceinline__ void dma8_part(const uint8_t* sbase, uint32_t lds_addr, int wv,
                                          int lane, int u) {
    const int lr = lane >> 3, pc = lane & 7;
    const int r0 = (wv * kF8TI + u) * 8;
    const int r = r0 + lr;
    const uint32_t voff = (uint32_t)(lr * kF8Row + ((pc ^ (r & 7)) << 4));
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

__device__ __forceinline__ f32x16 mfma_f8(const v8i32& a, const v8i32& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
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
    const int q0 = xcc_id() % kNQ;
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
            {
                const uint8_t* k0 = uniform_ptr8(kbase + (int64_t)ld_const(a.col_idx, it.y) * B * D);
#pragma unroll
                for (int u = 0; u < kF8TI; ++u) dma8_part(k0, ks_addr, wv, lane, u);
            }

            f32x16 o[4], ol;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) ol[r] = 0.f;
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
                if (__any(mnew > m)) {
                    const float mn = fmaxf(m, mnew);
                    const float alpha = __builtin_amdgcn_exp2f(m - mn);
                    l *= alpha;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
                    if (XC)
#pragma unroll
                        for (int r = 0; r < 16; ++r) ol[r] *= alpha;
                    m = mn;
                }
                // probabilities 2^8 exp2(s c - m), cast to E4M3; bytes 16t + e of chunk kc are
                // element e of key tile 2 kc + t
                v8i32 pf[2];
                const float off = 8.0f - m;
                const float c8 = 8.0f * c_blk, k8 = 8.0f * off + 56.0f;
#pragma unroll
                for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                    for (int w = 0; w < 8; ++w) {
                        const int tt = 2 * kc + (w >> 2);
                        const int r0 = 4 * (w & 3);
                        if (XC) {
                            uint32_t pk = 0;
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                pk = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(s[tt][r0 + j], c8, k8), j, pk);
                            pf[kc][w] = (int)pk;
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
#pragma unroll
                    for (int i = 0; i < 8; ++i) vf[i] = f8_frag(vs_lds, 32 * (i >> 1) + l32, 2 * (i & 1) + half);
#pragma unroll
                    for (int i = 0; i < 8; ++i) o[i >> 1] = mfma_f8(vf[i], pf[i & 1], o[i >> 1]);
                    if (XC) {
                        v8i32 ones;
#pragma unroll
                        for (int w = 0; w < 8; ++w) ones[w] = 0x38383838;     // E4M3 1.0
                        ol = mfma_f8(ones, pf[0], ol);
                        ol = mfma_f8(ones, pf[1], ol);
                    }
                }
            }

            // (ExpCast: every row of the all-ones product holds the lane's query's sum)
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

template <int D, int B>
bsa_status run(const AttnArgs& a, int slots, hipStream_t s) {
    hipLaunchKernelGGL((attn_kernel<D, B>), dim3(slots), dim3(Tile<D, B>::NT), 0, s, a);
    return check_launch("sparse_attn");
}

template <int D, int B>
int occupancy() {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, attn_kernel<D, B>, Tile<D, B>::NT, 0) !=
        hipSuccess)
        return 1;
    return nb < 1 ? 1 : nb;
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

int attn_slots(int32_t D, int32_t B, const DeviceInfo& dev) {
    int occ;
    if (D == 128 && B == 128) occ = occupancy<128, 128>();
    else if (D == 64 && B == 64) occ = occupancy<64, 64>();
    else if (D == 128 && B == 64) occ = occupancy<128, 64>();
    else occ = occupancy<64, 128>();
    return dev.cu_count * occ;
}

size_t attn_ws_bytes(int32_t batch, int32_t heads, int32_t D, const Geometry& g, int slots) {
    return attn_layout(batch, heads, D, g, slots).total;
}

bsa_status launch_attn(const void* q_t, const void* k_t, const void* v_t,
                       const int32_t* row_ptr, const int32_t* col_idx, int32_t batch,
                       int32_t heads, int32_t D, const Geometry& g, float scale, void* out_t,
                       float* lse, void* ws, const DeviceInfo& dev, hipStream_t s) {
    const int slots = attn_slots(D, g.B, dev);
    const AttnLayout L = attn_layout(batch, heads, D, g, slots);
    unsigned char* w = (unsigned char*)ws;
    int32_t* hdr = (int32_t*)(w + L.hdr);
    int32_t* head_item_off = (int32_t*)(w + L.head_item_off);
    int32_t* head_slot_base = (int32_t*)(w + L.head_slot_base);
    int4* items = (int4*)(w + L.items);
    int32_t* done = (int32_t*)(w + L.done);
    const int32_t nbh = batch * heads;

    hipLaunchKernelGGL(plan_global_kernel, dim3(1), dim3(kPlanThreads), 0, s, row_ptr, g.n_blk,
                       nbh, 2 * slots, hdr, head_item_off, head_slot_base);
    bsa_status st = check_launch("plan_global");
    if (st != BSA_OK) return st;
    hipLaunchKernelGGL(plan_rows_kernel, dim3(nbh), dim3(kPlanThreads), 0, s, row_ptr, g.n_blk,
                       hdr, head_item_off, head_slot_base, items, done);
    st = check_launch("plan_rows");
    if (st != BSA_OK) return st;

    AttnArgs a;
    a.q = (const uint16_t*)q_t;
    a.k = (const uint16_t*)k_t;
    a.v = (const uint16_t*)v_t;
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
    if (D == 128 && g.B == 128) return run<128, 128>(a, slots, s);
    if (D == 64 && g.B == 64) return run<64, 64>(a, slots, s);
    if (D == 128 && g.B == 64) return run<128, 64>(a, slots, s);
    return run<64, 128>(a, slots, s);
}

bsa_status launch_attn_fp8(const void* q8, const float* qs, const void* k8, const float* ks,
                           const void* v8, const float* vs, const int32_t* row_ptr,
                           const int32_t* col_idx, int32_t batch, int32_t heads,
                           const Geometry& g, float scale, int32_t expcast, void* out_t,
                           float* lse, void* ws, const DeviceInfo& dev, hipStream_t s) {
    const int slots = attn_fp8_slots(dev);
    const AttnLayout L = attn_layout(batch, heads, 128, g, slots);
    unsigned char* w = (unsigned char*)ws;
    int32_t* hdr = (int32_t*)(w + L.hdr);
    int32_t* head_item_off = (int32_t*)(w + L.head_item_off);
    int32_t* head_slot_base = (int32_t*)(w + L.head_slot_base);
    int4* items = (int4*)(w + L.items);
    int32_t* done = (int32_t*)(w + L.done);
    const int32_t nbh = batch * heads;
    hipLaunchKernelGGL(plan_global_kernel, dim3(1), dim3(kPlanThreads), 0, s, row_ptr, g.n_blk,
                       nbh, 2 * slots, hdr, head_item_off, head_slot_base);
    bsa_status st = check_launch("plan_global");
    if (st != BSA_OK) return st;
    hipLaunchKernelGGL(plan_rows_kernel, dim3(nbh), dim3(kPlanThreads), 0, s, row_ptr, g.n_blk,
                       hdr, head_item_off, head_slot_base, items, done);
    st = check_launch("plan_rows");
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

int attn_max_heads() { return kMaxHeads; }
int attn_max_blocks() { return kMaxBlocks; }

}  // namespace bsa

#ifdef BSA_TRACE
// Copy the first `count` workgroup records of the latest attention launch (56 bytes each:
// t0, t_last, t_end as uint64 s_memrealtime ticks, c0, c_end as uint64 s_memtime ticks, hw_id,
// xcc as uint32, items, blocks as int32) to host memory.  Synchronous; debug builds only.
extern "C" BSA_API int bsa_trace_read(void* host, int32_t count) {
    if (!host || count < 0 || count > bsa::kTraceMax) return -1;
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(bsa::g_trace_rec),
                                    (size_t)count * sizeof(bsa::TraceRec), 0,
                                    hipMemcpyDeviceToHost);
}
#endif
