// C entry points around the library's sequential host planner (plan_host.h), compiled by the
// CPU tests with the host compiler so that Python can call it through ctypes.
#include <string.h>

#include "plan_host.h"

extern "C" {

// Schedule of nbh heads x n_blk rows for `target` work items, `group` XCDs a queue.  hdr: Kc,
// qstart[8], qlen[8]; head_rank[nbh]; slot_base[nbh]; items[cap][4].  Returns the item count,
// or -1 if cap is short.
long long plan_ref(const int* row_ptr, int n_blk, int nbh, long long target, int group, int* hdr,
                   int* head_rank, int* slot_base, int* items, long long cap) {
    const bsa::plan::HostPlan P = bsa::plan::plan_host(row_ptr, n_blk, nbh, target, group);
    hdr[0] = P.Kc;
    for (int q = 0; q < bsa::plan::kNQ; ++q) {
        hdr[1 + q] = P.qstart[q];
        hdr[1 + bsa::plan::kNQ + q] = P.qlen[q];
    }
    memcpy(head_rank, P.head_rank.data(), sizeof(int) * nbh);
    memcpy(slot_base, P.head_slot_base.data(), sizeof(int) * nbh);
    if ((long long)P.items.size() > cap) return -1;
    for (size_t k = 0; k < P.items.size(); ++k) {
        items[4 * k + 0] = P.items[k].row;
        items[4 * k + 1] = P.items[k].b0;
        items[4 * k + 2] = P.items[k].b1;
        items[4 * k + 3] = P.items[k].slot;
    }
    return (long long)P.items.size();
}

// XCDs per queue for heads of head_kv_bytes of K and V.
int queue_group_ref(long long head_kv_bytes) { return bsa::plan::queue_group(head_kv_bytes); }

// Workspace offsets: hdr, head_seg, head_slot_base, items, done, part_o, part_ml, total,
// max_items, max_slots.
void layout_ref(long long bh, int n_blk, int B, int D, int slots, long long* out) {
    const bsa::plan::Layout L = bsa::plan::workspace_layout(bh, n_blk, B, D, slots);
    const long long v[10] = {(long long)L.hdr, (long long)L.head_seg, (long long)L.head_slot_base,
                             (long long)L.items, (long long)L.done, (long long)L.part_o,
                             (long long)L.part_ml, (long long)L.total, (long long)L.max_items,
                             (long long)L.max_slots};
    memcpy(out, v, sizeof(v));
}

}  // extern "C"
