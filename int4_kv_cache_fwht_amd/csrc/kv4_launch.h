// kv4_launch.h -- launch interface between the host library and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kv4_device_types.h"
#include "kv4_mq_types.h"

namespace kv4 {

// Optional timing events of one launch. When set, the launch stamps them from its own dispatch
// (hipExtLaunchKernel), so their interval is the kernel's execution alone; unset, the launch is a
// plain one.
struct KernelTimer {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

struct AppendArgs {
    const AppendTask* tasks; // device copy of the call's tasks
    const uint16_t* k;       // bf16 [rows][hkv][D]
    const uint16_t* v;
    uint8_t* pool;
    uint8_t* int8_pool;
    int32_t* bt;
    int64_t page_block;
    int64_t int8_tile;
    int hkv, block, sinks, recent, int8_tiles;
    float cb; // fl32(1/sqrt(block))
    int max_pps;
    int requant; // INT4 codes from the INT8 round trip (eviction by re-quantization)
    // fused RoPE of the key rows (nullptr: keys are taken as given): float [position][D/2]
    const float* rope_cos;
    const float* rope_sin;
    // single-position appends of up to kArgEntries sequences: task e writes position arg_t0[e] of
    // sequence arg_seq[e] from row e into page arg_page[e] & 0x7fffffff (bit 31: allocated by
    // this call).  n_arg == 0: the tasks come from `tasks`.
    int n_arg;
    int32_t arg_seq[kArgEntries];
    int32_t arg_t0[kArgEntries];
    int32_t arg_page[kArgEntries];
};

struct DecodeArgs {
    const uint8_t* pool;
    const uint8_t* int8_pool;
    const int32_t* bt;
    const uint16_t* q;        // bf16 [entries][hq][D]
    const DecodeUnit* units;  // device copy of the plan
    float* part_ml;           // [(W + n_units)][G][2] : (reference max in log2 units, sum)
    float* part_o;            // [(W + n_units)][G][D]
    int32_t* unit_waves;      // [n_units][2]: first and last wave holding work steps of the unit
    float* out;               // fp32 [entries][hq][D]
    int64_t total_steps;
    // two rounds of waves: waves [0, n_waves1) share the first steps1 global steps, waves
    // [n_waves1, n_waves) the rest (one round: n_waves1 = n_waves, steps1 = total_steps)
    int64_t steps1;
    int64_t page_block;
    int64_t int8_tile;
    int n_units, n_waves, n_waves1;
    int hkv, max_pps, sinks, recent, block, int8_tiles;
    float cb;         // fl32(1/sqrt(block))
    float scale_log2; // softmax scale * log2(e)
    // n_arg > 0: the plan is this list of call entries: sequence id, length and the first global
    // step of the entry's units; unit u is entry u / hkv, kv head u % hkv, and its steps follow
    // from the length.  n_arg == 0: `units`.
    int n_arg;
    int32_t arg_seq[kArgEntries];
    int32_t arg_len[kArgEntries];
    int32_t arg_step[kArgEntries];
};

struct MqArgs {
    const uint8_t* pool;
    const uint8_t* int8_pool;
    const int32_t* bt;
    const uint16_t* q;        // bf16 [rows][hq][D]
    const MqEntry* entries;   // device copy of the plan
    float* part_ml;           // [tasks][16][2]: (reference, sum of p) per query row, log2 units
    float* part_o;            // [tasks][16][D]: unnormalised rotated output per query row
    float* out;               // fp32 [rows][hq][D]
    int64_t page_block;
    int64_t int8_tile;
    int n_entries, tasks, groups, spc;
    // INT4_PROT: the four waves of a workgroup share their INT4 steps (every entry's row-tile
    // count is a multiple of 4)
    int share;
    int hq, hkv, max_pps, sinks, recent, block, int8_tiles, n8;
    float cb;         // fl32(1/sqrt(block))
    float scale_log2; // softmax scale * log2(e)
};

hipError_t launch_append(int d, int format, int n_tasks, const AppendArgs& a, hipStream_t stream,
                         const KernelTimer& tm = KernelTimer{});
// INT4_PROT append where every task writes exactly one position.
hipError_t launch_append_token(int d, int n_tasks, const AppendArgs& a, hipStream_t stream,
                               const KernelTimer& tm = KernelTimer{});
hipError_t launch_decode_split(int d, int g, int format, const DecodeArgs& a, hipStream_t stream,
                               const KernelTimer& tm = KernelTimer{});
hipError_t launch_decode_merge(int d, int g, int format, const DecodeArgs& a, hipStream_t stream,
                               const KernelTimer& tm = KernelTimer{});
// The same merge writing bf16 output rows (a.out then points at bf16 [entries][hq][D]).
hipError_t launch_decode_merge_bf16(int d, int g, int format, const DecodeArgs& a, hipStream_t stream,
                                    const KernelTimer& tm = KernelTimer{});
// Address of the current device's decode scratch (kDecodeScratchBytes, 256-byte aligned), looked
// up once per device; later calls return the kept pointer.
hipError_t decode_scratch(void** ptr);
// Workgroups of the split kernel (kWavesPerBlock waves each) that fit on one compute unit at once.
hipError_t decode_split_residency(int d, int g, int format, int* blocks_per_cu);
// Multi-query attention (INT4_PROT and INT8 formats): split kernel over the call's wave tasks,
// then the merge that also applies the inverse rotation.
hipError_t launch_mq_split(int d, int g, int format, const MqArgs& a, hipStream_t stream,
                           const KernelTimer& tm = KernelTimer{});
hipError_t launch_mq_merge(int d, int g, const MqArgs& a, hipStream_t stream, const KernelTimer& tm = KernelTimer{});
hipError_t mq_split_residency(int d, int g, int format, int* blocks_per_cu);
// HBM probes (measurement only): mode 0 streams `bytes` from src and writes one word per lane of
// the grid to dst (blocks * 256 words); mode 1 copies src to dst.  bytes is a multiple of 16.
hipError_t launch_probe(int mode, const void* src, void* dst, uint64_t bytes, int blocks, hipStream_t stream,
                        const KernelTimer& tm = KernelTimer{});

} // namespace kv4
