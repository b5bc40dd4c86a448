// Arithmetic of the persistent attention schedule, shared by the planner kernels and by the
// sequential host planner (plan_host.h).  Plain C++: no HIP types, so a host compiler can
// build it on its own.
//
// The schedule (FVAttn page, abstract: per-head work differs under adaptive Top-p, so equal
// head counts give unequal work; here the work is spread over the compute units of one GPU):
//  * work items are rows (batch, head, query block), or chunks of at most Kc key blocks of a
//    row, Kc = max(kKcMin, ceil(nnz / target)) with target = twice the resident workgroups;
//  * head mode (the usual case): one queue per XCD (kNQ); heads are ranked by cost (kept
//    blocks, descending, ties by index) and given longest-first to the least-loaded queue, so
//    a head's K and V stay in one XCD's L2; inside a queue the heads follow in rank order and
//    each head's rows by cost descending (ties by row), the chunks of a split row consecutive;
//  * queue groups (head mode): while eight heads' K and V (one head per XCD queue) fit the
//    memory-side cache in front of HBM (MALL, 256 MiB on MI355X), every XCD has a queue of its
//    own; past that, pairs of XCDs share one queue (0, 2, 4, 6; the odd ones stay empty), so
//    four heads are swept at once and the tiles the L2s miss are found in that cache more
//    often than in HBM;
//  * few-heads mode (batch * heads < kFewHeads and at most kFewRows rows): whole heads are too
//    coarse to balance eight queues, so all rows go to queue 0 in one global order, cost
//    descending (ties by row), and every workgroup takes from it: the last items are the
//    smallest rows of the layer.
#pragma once

#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define BSA_PLAN_FN __host__ __device__ __forceinline__
#else
#define BSA_PLAN_FN inline
#endif

namespace bsa {
namespace plan {

constexpr int kNQ = 8;               // XCD queues (MI355X: 8 XCDs)
constexpr int kMaxHeads = 2048;      // batch * heads supported by the planner
constexpr int kMaxBlocks = 4096;     // n_blk supported by the planner (12-bit row index)
constexpr int kKcMin = 8;            // smallest chunk (blocks) a row is split into

// XCDs per queue for heads of `head_kv_bytes` of K and V each (head mode)
constexpr int64_t kMallBytes = (int64_t)256 << 20;
BSA_PLAN_FN int32_t queue_group(int64_t head_kv_bytes) {
    return (int64_t)kNQ * head_kv_bytes > kMallBytes ? 2 : 1;
}

// chunk size Kc for `total` kept blocks and `target` work items
BSA_PLAN_FN int32_t chunk_size(int64_t total, int64_t target) {
    const int64_t kc = (total + target - 1) / target;
    return kc < kKcMin ? kKcMin : (int32_t)kc;
}

// work items of a row of c kept blocks (a row without blocks is still one item)
BSA_PLAN_FN int32_t row_items(int32_t c, int32_t Kc) {
    const int32_t n = (c + Kc - 1) / Kc;
    return n < 1 ? 1 : n;
}

// partial-result slots of a row: one per chunk if the row is split, none otherwise
BSA_PLAN_FN int32_t row_slots(int32_t c, int32_t Kc) {
    const int32_t n = row_items(c, Kc);
    return n > 1 ? n : 0;
}

// sort key of a row inside its head: cost descending, row index ascending (12 bits)
BSA_PLAN_FN uint32_t row_key(int32_t c, int32_t i) {
    return ((uint32_t)(kMaxBlocks - c) << 12) | (uint32_t)i;
}
BSA_PLAN_FN int32_t key_row(uint32_t k) { return (int32_t)(k & 0xfffu); }

// few-heads mode: rows of the whole layer (< kFewRows) in one order, cost descending, global
// row index ascending (14 bits)
constexpr int kFewHeads = 2 * kNQ;
constexpr int kFewRows = 16384;
BSA_PLAN_FN bool few_heads(int32_t nbh, int32_t n_blk) {
    return nbh < kFewHeads && (int64_t)nbh * n_blk <= kFewRows;
}
BSA_PLAN_FN uint32_t few_key(int32_t c, int32_t r) {
    return ((uint32_t)(kMaxBlocks - c) << 14) | (uint32_t)r;
}
BSA_PLAN_FN int32_t few_key_row(uint32_t k) { return (int32_t)(k & 0x3fffu); }

// sort key of a head: cost (kept blocks, < 2^40) descending, head index ascending
BSA_PLAN_FN uint64_t head_key(int64_t cost, int32_t h) {
    return ((uint64_t)((int64_t)1 << 40) - (uint64_t)cost) << 11 | (uint64_t)h;
}
BSA_PLAN_FN int32_t key_head(uint64_t k) { return (int32_t)(k & 0x7ffu); }

// Byte offsets of the attention workspace (device memory the caller owns): schedule header,
// per-head item offsets, per-head partial-slot bases, work items (int4: row, first
// and end CSR position, first partial slot), split-row chunk counters, fp32 partial outputs
// and (max, sum) pairs.  Items <= rows + target and partial slots <= 2 target (Kc >=
// nnz / target, so the split rows, each longer than Kc, hold fewer than 2 nnz / Kc chunks).
struct Layout {
    size_t hdr, head_seg, head_slot_base, items, done, part_o, part_ml, total;
    int64_t max_items, max_slots;
};
constexpr int kHdrInts = 32 + 32 * kNQ + kNQ;    // Kc, group, queue starts, counters, lengths
BSA_PLAN_FN size_t align256(size_t x) { return (x + 255) / 256 * 256; }
BSA_PLAN_FN Layout workspace_layout(int64_t bh, int32_t n_blk, int32_t B, int32_t D,
                                    int slots) {
    Layout L;
    const int64_t rows = bh * n_blk;
    const int64_t target = 2 * (int64_t)slots;
    L.max_items = rows + target;
    L.max_slots = 2 * target;
    size_t off = 0;
    L.hdr = off;            off = align256(off + kHdrInts * 4);
    L.head_seg = off;       off = align256(off + (size_t)bh * 4);
    L.head_slot_base = off; off = align256(off + (size_t)bh * 4);
    L.items = off;          off = align256(off + (size_t)L.max_items * 16);
    L.done = off;           off = align256(off + (size_t)L.max_slots * 4);
    L.part_o = off;         off = align256(off + (size_t)L.max_slots * B * D * 4);
    L.part_ml = off;        off = align256(off + (size_t)L.max_slots * B * 2 * 4);
    L.total = off;
    return L;
}

}  // namespace plan
}  // namespace bsa
