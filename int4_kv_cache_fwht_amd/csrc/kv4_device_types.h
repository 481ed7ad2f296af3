// kv4_device_types.h -- plain data shared by the host planner and the HIP kernels of libkv4.
#pragma once

#include <stdint.h>

namespace kv4 {

constexpr int kPageSize = 16;       // positions per page (one 16-slot tile per kv head)
constexpr int kInt4StepPages = 4;   // decode INT4 step: 4 pages = 64 positions, one per lane
constexpr int kInt8StepSlots = 32;  // decode INT8 step over protection slots: 2 tiles = 32 slots
constexpr int kInt8StepPages = 2;   // decode step of the INT8 format: 2 pages = 32 positions
constexpr int kWavesPerBlock = 8;   // decode split kernel: waves per workgroup (two per SIMD)
constexpr int kArgEntries = 256;    // calls with up to this many sequences pass their plan as kernel arguments
// Device scratch of the allocation-free decode entry point (one array per GPU): the largest decode
// workspace it serves.
constexpr unsigned long long kDecodeScratchBytes = 16ull << 20;
// Decode split: every unit's step range opens with this many accounting steps that hold no work.
// A wave whose slice starts a unit pays its query prologue, its epilogue and a refill of the load
// pipeline; charging that as steps evens out the waves' finishing times (3 measured best on MI355X
// for contexts of 1K to 32K positions).
constexpr int kUnitStartSteps = 3;

enum { kTaskNewPage = 1 };

// One append work item: the positions [t0, t0 + n) of sequence `seq` that fall in one page.
struct AppendTask {
    int32_t seq;
    int32_t page;     // page id holding positions 16*(t0/16) .. +15
    int32_t t0;       // first position written by this task
    int32_t n;        // number of positions (1..16)
    int32_t row0;     // row of k_new / v_new holding position t0
    int32_t len_new;  // sequence length after the call (decides INT8 protection)
    int32_t bt_index; // seq * max_pages_per_seq + t0 / 16
    int32_t flags;    // kTaskNewPage: the page was allocated by this call
};

// One decode unit: (call entry, kv head).  Units are laid out entry-major, and a unit's steps
// occupy [step_begin, next unit's step_begin) of the global step range.
struct DecodeUnit {
    int32_t seq;
    int32_t len;
    int32_t entry;
    int32_t head;
    int64_t step_begin;
};

} // namespace kv4
