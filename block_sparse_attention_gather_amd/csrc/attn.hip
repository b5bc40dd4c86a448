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
//                8 XCD queues longest-first (each head's K/V then stays in one XCD's L2, or
//                in a pair's when eight heads' K/V exceed the MALL and pairs share a queue),
//                queue offsets, counters reset.
//   plan_rows    one workgroup per head: rows ordered by cost descending (ties: row order),
//                rows longer than Kc split into chunks, work items written in queue order.
//   attn         persistent: each workgroup reads its XCD id, pops items from its own queue
//                (its pair's: the even XCD's) with an atomic counter, then steals from the other queues; every queue is
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
#include <mutex>

#include "attn_common.h"

namespace bsa {
namespace {

// ---------------------------------------------------------------------------------------
// planner
// ---------------------------------------------------------------------------------------
// Head mode (plan.h).  One workgroup: Kc; per head its kept blocks, work items and partial
// slots (a wavefront per head); heads ranked by cost (bitonic sort of plan::head_key in LDS)
// and given longest-first to the least-loaded queue of those in use (every `group`-th);
// queue starts and lengths; every head's first item (head_off) and first partial slot; queue
// counters reset.
__global__ __launch_bounds__(kPlanThreads) void plan_global_kernel(
    const int32_t* __restrict__ row_ptr, int32_t n_blk, int32_t nbh, int32_t target,
    int32_t group, int32_t* __restrict__ hdr, int32_t* __restrict__ head_off,
    int32_t* __restrict__ head_slot_base) {
    __shared__ int32_t hitems[kMaxHeads], hslots[kMaxHeads], horder[kMaxHeads];
    __shared__ uint64_t hkey[kMaxHeads];
    __shared__ int64_t hcost[kMaxHeads];
    __shared__ uint8_t hq[kMaxHeads];          // queue of the head of each rank
    const int t = threadIdx.x;
    const int64_t rows = (int64_t)nbh * n_blk;
    const int32_t Kc = plan::chunk_size(row_ptr[rows], target);
    {
        const int lane = t & 63, w = t >> 6;
        for (int h = w; h < nbh; h += kPlanThreads / 64) {
            int32_t ni = 0, ns = 0;
            int64_t hc = 0;
#pragma unroll 8
            for (int i = lane; i < n_blk; i += 64) {     // (unrolled: 8 loads in flight)
                const int64_t r = (int64_t)h * n_blk + i;
                const int32_t c = row_ptr[r + 1] - row_ptr[r];
                ni += plan::row_items(c, Kc);
                ns += plan::row_slots(c, Kc);
                hc += c;
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                ni += __shfl_xor(ni, off, 64);
                ns += __shfl_xor(ns, off, 64);
                hc += __shfl_xor(hc, off, 64);
            }
            if (lane == 0) {
                hitems[h] = ni;
                hslots[h] = ns;
                hcost[h] = hc;
                hkey[h] = plan::head_key(hc, h);
            }
        }
    }
    // heads ranked by cost descending (ties by index): bitonic sort of the head keys
    int P2 = 1;
    while (P2 < nbh) P2 <<= 1;
    for (int h = nbh + t; h < P2; h += kPlanThreads) hkey[h] = ~(uint64_t)0;
    __syncthreads();
    for (int kk = 2; kk <= P2; kk <<= 1)
        for (int jj = kk >> 1; jj > 0; jj >>= 1) {
            for (int i = t; i < P2; i += kPlanThreads) {
                const int l = i ^ jj;
                if (l > i) {
                    const uint64_t x = hkey[i], y = hkey[l];
                    if ((x > y) == ((i & kk) == 0)) {
                        hkey[i] = y;
                        hkey[l] = x;
                    }
                }
            }
            __syncthreads();
        }
    for (int r = t; r < nbh; r += kPlanThreads) horder[r] = plan::key_head(hkey[r]);
    __syncthreads();
    if (t == 0) {
        // longest processing time first: each head to the least-loaded queue in use (ties:
        // lowest); one thread, so every value it reads back is in registers or LDS
        int64_t qload[kNQ];
        int32_t qlen[kNQ], qstart[kNQ], qrun[kNQ];
        for (int q = 0; q < kNQ; ++q) { qload[q] = 0; qlen[q] = 0; qrun[q] = 0; }
        for (int r = 0; r < nbh; ++r) {
            const int h = horder[r];
            int best = 0;
#pragma unroll
            for (int q = 1; q < kNQ; ++q)       // (unrolled: the loads stay in registers)
                if (q % group == 0 && qload[q] < qload[best]) best = q;
            qload[best] += hcost[h];
            qlen[best] += hitems[h];
            hq[r] = (uint8_t)best;
        }
        int32_t acc = 0;
        for (int q = 0; q < kNQ; ++q) { qstart[q] = acc; acc += qlen[q]; }
        for (int r = 0; r < nbh; ++r) {
            const int h = horder[r];
            const int q = hq[r];
            head_off[h] = qstart[q] + qrun[q];
            qrun[q] += hitems[h];
        }
        int32_t sacc = 0;
        for (int h = 0; h < nbh; ++h) { head_slot_base[h] = sacc; sacc += hslots[h]; }
        hdr[kHdrKc] = Kc;
        hdr[kHdrGroup] = group;
        for (int q = 0; q < kNQ; ++q) {
            hdr[kHdrQStart + q] = qstart[q];
            hdr[kHdrQLen + q] = qlen[q];
            hdr[kHdrCtr + 32 * q] = 0;
        }
    }
}

// Head mode.  One workgroup per head: rows by cost descending (ties by row; bitonic sort of
// plan::row_key), exclusive scans of items and partial slots in that order, items written from
// the head's first item on.
__global__ __launch_bounds__(kPlanThreads) void plan_rows_kernel(
    const int32_t* __restrict__ row_ptr, int32_t n_blk, const int32_t* __restrict__ hdr,
    const int32_t* __restrict__ head_off, const int32_t* __restrict__ head_slot_base,
    int4* __restrict__ items, int32_t* __restrict__ done) {
    __shared__ int32_t cost[kMaxBlocks], ord[kMaxBlocks], ipos[kMaxBlocks], spos[kMaxBlocks];
    __shared__ int32_t part_i[kPlanThreads], part_s[kPlanThreads];
    const int t = threadIdx.x;
    const int h = blockIdx.x;
    const int64_t base = (int64_t)h * n_blk;
    const int32_t Kc = hdr[kHdrKc];
    for (int i = t; i < n_blk; i += kPlanThreads) cost[i] = row_ptr[base + i + 1] - row_ptr[base + i];
    __syncthreads();
    int P2 = 2;
    while (P2 < n_blk) P2 <<= 1;
    uint32_t* key = (uint32_t*)ord;
    for (int i = t; i < P2; i += kPlanThreads)
        key[i] = i < n_blk ? plan::row_key(cost[i], i) : 0xffffffffu;
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
    for (int k = t; k < n_blk; k += kPlanThreads) ord[k] = plan::key_row(key[k]);
    __syncthreads();
    // exclusive scans (in rank order) of items per row and of partial slots per split row
    const int seg = (n_blk + kPlanThreads - 1) / kPlanThreads;
    const int lo = min(n_blk, t * seg), hi = min(n_blk, lo + seg);
    int32_t li = 0, ls = 0;
    for (int k = lo; k < hi; ++k) {
        li += plan::row_items(cost[ord[k]], Kc);
        ls += plan::row_slots(cost[ord[k]], Kc);
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
        ipos[k] = ri;
        spos[k] = rs;
        ri += plan::row_items(cost[ord[k]], Kc);
        rs += plan::row_slots(cost[ord[k]], Kc);
    }
    __syncthreads();
    const int32_t ioff = head_off[h];
    const int32_t sbase = head_slot_base[h];
    for (int k = t; k < n_blk; k += kPlanThreads) {
        const int i = ord[k];
        const int32_t c = cost[i];
        const int32_t beg = row_ptr[base + i];
        const int32_t ni = plan::row_items(c, Kc);
        const int32_t slot = ni > 1 ? sbase + spos[k] : -1;
        for (int s = 0; s < ni; ++s) {
            const int32_t b0 = beg + s * Kc;
            const int32_t b1 = min(beg + (s + 1) * Kc, beg + c);
            items[ioff + ipos[k] + s] = make_int4((int32_t)(base + i), b0, b1, slot);
        }
        if (slot >= 0) done[slot] = 0;               // chunk counter of the split row
    }
}

// Few-heads mode (plan.h).  One workgroup: every row of the layer (at most plan::kFewRows)
// sorted by cost descending (ties by row; bitonic sort of plan::few_key in LDS), exclusive scans
// of items and partial slots in that order, all items in queue 0, the other queues empty.
__global__ __launch_bounds__(kPlanThreads) void plan_few_kernel(
    const int32_t* __restrict__ row_ptr, int32_t rows, int32_t target,
    int32_t* __restrict__ hdr, int4* __restrict__ items, int32_t* __restrict__ done) {
    __shared__ uint32_t key[plan::kFewRows];
    __shared__ int32_t part_i[kPlanThreads], part_s[kPlanThreads];
    const int t = threadIdx.x;
    const int32_t Kc = plan::chunk_size(row_ptr[rows], target);
    int P2 = 2;
    while (P2 < rows) P2 <<= 1;
    for (int r = t; r < P2; r += kPlanThreads)
        key[r] = r < rows ? plan::few_key(row_ptr[r + 1] - row_ptr[r], r) : 0xffffffffu;
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
    const int seg = (rows + kPlanThreads - 1) / kPlanThreads;
    const int lo = min(rows, t * seg), hi = min(rows, lo + seg);
    auto cost_at = [&](int k) {
        const int r = plan::few_key_row(key[k]);
        return row_ptr[r + 1] - row_ptr[r];
    };
    int32_t li = 0, ls = 0;
    for (int k = lo; k < hi; ++k) {
        li += plan::row_items(cost_at(k), Kc);
        ls += plan::row_slots(cost_at(k), Kc);
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
        const int r = plan::few_key_row(key[k]);
        const int32_t c = row_ptr[r + 1] - row_ptr[r], beg = row_ptr[r];
        const int32_t ni = plan::row_items(c, Kc);
        const int32_t slot = ni > 1 ? rs : -1;
        for (int s = 0; s < ni; ++s) {
            const int32_t b0 = beg + s * Kc;
            const int32_t b1 = min(beg + (s + 1) * Kc, beg + c);
            items[ri + s] = make_int4(r, b0, b1, slot);
        }
        if (slot >= 0) done[slot] = 0;
        ri += ni;
        rs += plan::row_slots(c, Kc);
    }
    if (t == kPlanThreads - 1) {
        hdr[kHdrKc] = Kc;
        hdr[kHdrGroup] = 1;
        for (int q = 0; q < kNQ; ++q) {
            hdr[kHdrQStart + q] = q == 0 ? 0 : ri;       // the last thread ends at the total
            hdr[kHdrQLen + q] = q == 0 ? ri : 0;
            hdr[kHdrCtr + 32 * q] = 0;
        }
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
    const int q0 = (xcc_id() % kNQ) & ~(ld_const(a.hdr, kHdrGroup) - 1);  // first queue
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
            // first key block of the item into LDS (a row without blocks reads none and is
            // written as zeros below, like a pad row)
            if (it.y < it.z)
                dma_tile<D, B, false>(kbase + (int64_t)ld_const(a.col_idx, it.y) * B * D,
                                      ks_addr, wv, lane);

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
                // every S^T MFMA is issued before the V wait (the last ones would otherwise be
                // sunk below it)
#pragma unroll
                for (int tt = 0; tt < Tl::NKT; ++tt) keep_issued(s[tt]);
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
                // From here to the end of O^T += V^T P^T this wavefront wins issue arbitration
                // over the other wavefront of its SIMD while that one is elsewhere in its loop:
                // the softmax is the long VALU stretch, and pushing it through keeps the matrix
                // core fed (measured 2.5-3 % faster, identical results)
                __builtin_amdgcn_s_setprio(1);
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
                __builtin_amdgcn_s_setprio(0);
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

}  // namespace

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
    int4* items = (int4*)(w + L.items);
    int32_t* done = (int32_t*)(w + L.done);
    // K and V of a head, bf16
    bsa_status st = launch_plan(row_ptr, batch, heads, D, g, slots, 4 * g.Npad * D, ws, s);
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

bsa_status launch_plan(const int32_t* row_ptr, int32_t batch, int32_t heads, int32_t D,
                       const Geometry& g, int slots, int64_t head_kv_bytes, void* ws,
                       hipStream_t s) {
    const AttnLayout L = attn_layout(batch, heads, D, g, slots);
    unsigned char* w = (unsigned char*)ws;
    int32_t* hdr = (int32_t*)(w + L.hdr);
    int32_t* head_off = (int32_t*)(w + L.head_seg);
    int32_t* head_slot_base = (int32_t*)(w + L.head_slot_base);
    int4* items = (int4*)(w + L.items);
    int32_t* done = (int32_t*)(w + L.done);
    const int32_t nbh = batch * heads;
    if (plan::few_heads(nbh, g.n_blk)) {
        hipLaunchKernelGGL(plan_few_kernel, dim3(1), dim3(kPlanThreads), 0, s, row_ptr,
                           nbh * g.n_blk, 2 * slots, hdr, items, done);
        return check_launch("plan_few");
    }
    hipLaunchKernelGGL(plan_global_kernel, dim3(1), dim3(kPlanThreads), 0, s, row_ptr, g.n_blk,
                       nbh, 2 * slots, plan::queue_group(head_kv_bytes), hdr, head_off,
                       head_slot_base);
    bsa_status st = check_launch("plan_global");
    if (st != BSA_OK) return st;
    hipLaunchKernelGGL(plan_rows_kernel, dim3(nbh), dim3(kPlanThreads), 0, s, row_ptr, g.n_blk,
                       hdr, head_off, head_slot_base, items, done);
    return check_launch("plan_rows");
}

// ---------------------------------------------------------------------------------------
// static scratch of bsa_sparse_attn_fwd_noalloc
// ---------------------------------------------------------------------------------------
// The attention workspace (schedule header, work items, split-row counters and fp32
// partials) for callers that cannot allocate: one array per device, alive until the process
// ends.  Host code never passes `scratch` itself to a kernel (in host code the name is only a
// stand-in for the device symbol); it passes the device address that hipGetSymbolAddress
// returns for the current device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

bsa_status static_scratch(int device, void** ptr) {
    if (device < 0 || device >= kMaxDevices)
        return fail(BSA_ERR_HIP, "device ordinal %d out of range", device);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(BSA_ERR_HIP, "static scratch of device %d: hipGetSymbolAddress: %s",
                        device, hipGetErrorString(e));
        g_scratch_ptr[device] = p;
    }
    *ptr = g_scratch_ptr[device];
    return BSA_OK;
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
