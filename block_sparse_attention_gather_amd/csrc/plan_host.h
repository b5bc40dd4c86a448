// Sequential host version of the attention schedule the planner kernels build on the device
// (plan_global_kernel, plan_rows_kernel): the same arithmetic (plan.h), one loop at a time.
// Host-only (standard library containers); used to check the device planner and to test the
// schedule on the CPU.
#pragma once

#include <algorithm>
#include <vector>

#include "plan.h"

namespace bsa {
namespace plan {

struct Item {
    int32_t row, b0, b1, slot;    // row r, key blocks col_idx[b0 .. b1), first partial slot or -1
};

struct HostPlan {
    int32_t Kc = 0;
    int32_t qstart[kNQ] = {}, qlen[kNQ] = {};
    std::vector<int32_t> head_rank;         // [nbh] cost rank of each head
    std::vector<int32_t> head_slot_base;    // [nbh] first partial slot of each head
    std::vector<Item> items;                // in queue order: queue 0, then queue 1, ...
};

// Build the schedule of `nbh` heads of n_blk rows each from the CSR row pointers
// (row_ptr[nbh * n_blk + 1]) for `target` work items (twice the resident workgroups), with
// `group` XCDs sharing a queue in head mode (queue_group of the head's K and V bytes).
inline HostPlan plan_host(const int32_t* row_ptr, int32_t n_blk, int32_t nbh, int64_t target,
                          int32_t group) {
    HostPlan P;
    const int64_t rows = (int64_t)nbh * n_blk;
    P.Kc = chunk_size(row_ptr[rows], target);
    auto cost = [&](int64_t r) { return row_ptr[r + 1] - row_ptr[r]; };
    // heads by cost descending (ties by index)
    std::vector<uint64_t> hk(nbh);
    std::vector<int64_t> hcost(nbh, 0);
    for (int32_t h = 0; h < nbh; ++h) {
        for (int32_t i = 0; i < n_blk; ++i) hcost[h] += cost((int64_t)h * n_blk + i);
        hk[h] = head_key(hcost[h], h);
    }
    std::sort(hk.begin(), hk.end());
    std::vector<int32_t> order(nbh);
    P.head_rank.assign(nbh, 0);
    for (int32_t r = 0; r < nbh; ++r) {
        order[r] = key_head(hk[r]);
        P.head_rank[order[r]] = r;
    }
    auto push_row = [&](int64_t r, int32_t slot) {
        const int32_t c = cost(r), beg = row_ptr[r];
        const int32_t ni = row_items(c, P.Kc);
        for (int32_t s = 0; s < ni; ++s) {
            const int32_t b0 = beg + s * P.Kc;
            const int32_t b1 = std::min(beg + (s + 1) * P.Kc, beg + c);
            P.items.push_back(Item{(int32_t)r, b0, b1, slot});
        }
    };
    P.head_slot_base.assign(nbh, 0);
    if (few_heads(nbh, n_blk)) {
        // one queue, every row of the layer by cost descending; partial slots in that order
        std::vector<uint32_t> keys(rows);
        for (int64_t r = 0; r < rows; ++r) keys[r] = few_key(cost(r), (int32_t)r);
        std::sort(keys.begin(), keys.end());
        int32_t sacc = 0;
        for (uint32_t k : keys) {
            const int64_t r = few_key_row(k);
            const int32_t ns = row_slots(cost(r), P.Kc);
            push_row(r, ns ? sacc : -1);
            sacc += ns;
        }
        P.qlen[0] = (int32_t)P.items.size();
        for (int q = 1; q < kNQ; ++q) P.qstart[q] = P.qlen[0];
        return P;
    }
    // head mode: heads longest first to the least-loaded queue in use, every group-th (ties:
    // lowest queue)
    int64_t qload[kNQ] = {};
    std::vector<int32_t> hqueue(nbh);
    for (int32_t r = 0; r < nbh; ++r) {
        int best = 0;
        for (int q = group; q < kNQ; q += group)
            if (qload[q] < qload[best]) best = q;
        qload[best] += hcost[order[r]];
        hqueue[order[r]] = best;
    }
    // rows of every head by cost descending; partial slots per head (heads in index order)
    std::vector<std::vector<int32_t>> hrows(nbh);
    std::vector<std::vector<int32_t>> rslot(nbh);
    int32_t sacc = 0;
    for (int32_t h = 0; h < nbh; ++h) {
        std::vector<uint32_t> keys(n_blk);
        for (int32_t i = 0; i < n_blk; ++i) keys[i] = row_key(cost((int64_t)h * n_blk + i), i);
        std::sort(keys.begin(), keys.end());
        P.head_slot_base[h] = sacc;
        for (uint32_t k : keys) {
            const int32_t i = key_row(k);
            const int32_t ns = row_slots(cost((int64_t)h * n_blk + i), P.Kc);
            hrows[h].push_back(i);
            rslot[h].push_back(ns ? sacc : -1);
            sacc += ns;
        }
    }
    for (int q = 0; q < kNQ; ++q) {
        P.qstart[q] = (int32_t)P.items.size();
        for (int32_t r = 0; r < nbh; ++r) {
            const int32_t h = order[r];
            if (hqueue[h] != q) continue;
            for (size_t k = 0; k < hrows[h].size(); ++k)
                push_row((int64_t)h * n_blk + hrows[h][k], rslot[h][k]);
        }
        P.qlen[q] = (int32_t)P.items.size() - P.qstart[q];
    }
    return P;
}

}  // namespace plan
}  // namespace bsa
