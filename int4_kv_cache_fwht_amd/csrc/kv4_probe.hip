// kv4_probe.hip -- HBM ceiling probes: a streaming read and a streaming copy of a plain buffer,
// the practical bandwidth ceiling that the cache kernels' achieved bytes per second are set
// against (beside the published 8 TB/s of MI355X HBM3E).  They compute nothing of the method.
//
// Each lane moves 16 bytes per load; a workgroup of 256 lanes keeps kUnroll loads per lane in
// flight and walks the buffer in blocks of 256 * kUnroll * 16 bytes, block b + k * gridDim.x for
// k = 0, 1, ... (grid stride), so consecutive workgroups read consecutive blocks.
#include "kv4_common.h"

namespace kv4 {

constexpr int kProbeLanes = 256;
constexpr int kProbeUnroll = 8;

// Reads n16 16-byte words.  Each lane folds what it read into one word and stores it to
// sink[global lane] (grid * 256 words, about 0.05% of the bytes read for a 4 GiB buffer), so that
// no load can be dropped.
__global__ __launch_bounds__(kProbeLanes) void probe_read_kernel(const u32x4* __restrict__ src, uint64_t n16,
                                                                 uint32_t* __restrict__ sink)
{
    const uint64_t per_block = (uint64_t)kProbeLanes * kProbeUnroll;
    uint32_t acc = 0;
    for (uint64_t b = blockIdx.x; b * per_block < n16; b += gridDim.x) {
        const uint64_t base = b * per_block + threadIdx.x;
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; u++) {
            const uint64_t i = base + (uint64_t)u * kProbeLanes;
            v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; u++) acc ^= (v[u].x ^ v[u].y) ^ (v[u].z ^ v[u].w);
    }
    sink[(uint64_t)blockIdx.x * kProbeLanes + threadIdx.x] = acc;
}

// Copies n16 16-byte words from src to dst.
__global__ __launch_bounds__(kProbeLanes) void probe_copy_kernel(const u32x4* __restrict__ src, uint64_t n16,
                                                                 u32x4* __restrict__ dst)
{
    const uint64_t per_block = (uint64_t)kProbeLanes * kProbeUnroll;
    for (uint64_t b = blockIdx.x; b * per_block < n16; b += gridDim.x) {
        const uint64_t base = b * per_block + threadIdx.x;
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; u++) {
            const uint64_t i = base + (uint64_t)u * kProbeLanes;
            v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; u++) {
            const uint64_t i = base + (uint64_t)u * kProbeLanes;
            if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
        }
    }
}


hipError_t launch_probe(int mode, const void* src, void* dst, uint64_t bytes, int blocks, hipStream_t stream,
                        const KernelTimer& tm)
{
    const uint64_t n16 = bytes / 16;
    dim3 grid((unsigned)blocks), block(kProbeLanes);
    if (mode == 0) {
        if (tm.start || tm.stop)
            hipExtLaunchKernelGGL(probe_read_kernel, grid, block, 0, stream, tm.start, tm.stop, 0,
                                  (const u32x4*)src, n16, (uint32_t*)dst);
        else
            hipLaunchKernelGGL(probe_read_kernel, grid, block, 0, stream, (const u32x4*)src, n16, (uint32_t*)dst);
    } else {
        if (tm.start || tm.stop)
            hipExtLaunchKernelGGL(probe_copy_kernel, grid, block, 0, stream, tm.start, tm.stop, 0,
                                  (const u32x4*)src, n16, (u32x4*)dst);
        else
            hipLaunchKernelGGL(probe_copy_kernel, grid, block, 0, stream, (const u32x4*)src, n16, (u32x4*)dst);
    }
    return hipGetLastError();
}

} // namespace kv4
