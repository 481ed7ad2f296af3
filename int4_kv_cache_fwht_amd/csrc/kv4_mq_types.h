// kv4_mq_types.h -- plain data shared by the host planner and the multi-query attention kernels.
#pragma once

#include <stdint.h>

namespace kv4 {

constexpr int kMqRows = 16;         // query rows per wave: (query, head) pairs of one kv head
constexpr int kMqStepSlots = 32;    // one step: two 16-slot pages (or INT8 tiles)

// One call entry of kv4_multi_query_attention.  Its work is hkv * nch * nrt wave tasks laid out
// (kv head, chunk, row tile) with the row tile fastest, from task0 on; its (kv head, row tile)
// groups, merged one row per wave, start at grp0.
struct MqEntry {
    int32_t seq;
    int32_t len;   // sequence length L
    int32_t nq;    // query rows: positions L - nq .. L - 1
    int32_t qrow0; // first row of q / out
    int32_t task0;
    int32_t grp0;
    int32_t steps; // steps of one (entry, kv head): INT8 steps first, then INT4 page pairs
    int32_t nch;   // chunks of at most `spc` steps
};

} // namespace kv4
