// kv4_host.cpp -- C ABI of libkv4 (see include/kv4.h): argument validation, host state, staging of
// the per-call plans to the device and kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kv4.h"
#include "kv4_launch.h"
#include "kv4_plan.hpp"

namespace {

thread_local std::string g_last_error;

// Pinned host staging for the plans that each call copies to the device.  A slot is reused only
// after the copy that read it has completed (its event).
struct Staging {
    struct Slot {
        void* host = nullptr;
        size_t cap = 0;
        hipEvent_t ev = nullptr;
        bool pending = false;
    };
    std::vector<Slot> slots;
    int next = 0;

    hipError_t init(int n)
    {
        slots.resize((size_t)n);
        for (auto& s : slots) {
            hipError_t e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    void release()
    {
        for (auto& s : slots) {
            if (s.pending) hipEventSynchronize(s.ev);
            if (s.host) hipHostFree(s.host);
            if (s.ev) hipEventDestroy(s.ev);
            s = Slot();
        }
    }
    hipError_t acquire(size_t bytes, void** host, int* idx)
    {
        Slot& s = slots[(size_t)next];
        hipError_t e = hipSuccess;
        if (s.pending) {
            e = hipEventSynchronize(s.ev);
            if (e != hipSuccess) return e;
            s.pending = false;
        }
        if (s.cap < bytes) {
            if (s.host) hipHostFree(s.host);
            s.host = nullptr;
            s.cap = 0;
            size_t cap = bytes < 4096 ? 4096 : bytes;
            e = hipHostMalloc(&s.host, cap, hipHostMallocDefault);
            if (e != hipSuccess) return e;
            s.cap = cap;
        }
        *host = s.host;
        *idx = next;
        next = (next + 1) % (int)slots.size();
        return hipSuccess;
    }
    hipError_t commit(int idx, hipStream_t stream)
    {
        Slot& s = slots[(size_t)idx];
        hipError_t e = hipEventRecord(s.ev, stream);
        if (e == hipSuccess) s.pending = true;
        return e;
    }
};

// Event pairs / triples recorded around kernel launches while profiling is on.
struct Profiler {
    bool on = false;
    std::vector<std::vector<hipEvent_t>> append_ev; // {kernel start, kernel stop}
    std::vector<std::vector<hipEvent_t>> decode_ev; // {split start, split stop, merge start, merge stop}
    std::vector<std::vector<hipEvent_t>> mq_ev;     // the same for multi-query calls
    kv4_profile totals{};
    std::vector<float> durations[5]; // per launch, in launch order: append, split, merge, mq split, mq merge

    // Timing-only events (no system-scope fence). Each launch stamps its own start/stop pair from
    // its dispatch, so an interval is one kernel's execution, as a kernel trace reports it.
    static hipError_t make(int n, std::vector<hipEvent_t>* out)
    {
        out->assign((size_t)n, nullptr);
        for (auto& e : *out) {
            hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
            if (r != hipSuccess) return r;
        }
        return hipSuccess;
    }
    void reset()
    {
        for (auto& v : append_ev)
            for (auto e : v)
                if (e) hipEventDestroy(e);
        for (auto& v : decode_ev)
            for (auto e : v)
                if (e) hipEventDestroy(e);
        for (auto& v : mq_ev)
            for (auto e : v)
                if (e) hipEventDestroy(e);
        append_ev.clear();
        decode_ev.clear();
        mq_ev.clear();
        totals = kv4_profile{};
        for (auto& d : durations) d.clear();
    }
    hipError_t collect()
    {
        for (auto& v : append_ev) {
            hipError_t r = hipEventSynchronize(v[1]);
            if (r != hipSuccess) return r;
            float ms = 0.f;
            hipEventElapsedTime(&ms, v[0], v[1]);
            totals.append_launches += 1;
            totals.append_ms += ms;
            durations[0].push_back(ms);
            for (auto e : v) hipEventDestroy(e);
        }
        append_ev.clear();
        for (auto& v : decode_ev) {
            hipError_t r = hipEventSynchronize(v[3]);
            if (r != hipSuccess) return r;
            float a = 0.f, b = 0.f;
            hipEventElapsedTime(&a, v[0], v[1]);
            hipEventElapsedTime(&b, v[2], v[3]);
            totals.decode_launches += 1;
            totals.split_ms += a;
            totals.merge_ms += b;
            durations[1].push_back(a);
            durations[2].push_back(b);
            for (auto e : v) hipEventDestroy(e);
        }
        decode_ev.clear();
        for (auto& v : mq_ev) {
            hipError_t r = hipEventSynchronize(v[3]);
            if (r != hipSuccess) return r;
            float a = 0.f, b = 0.f;
            hipEventElapsedTime(&a, v[0], v[1]);
            hipEventElapsedTime(&b, v[2], v[3]);
            totals.mq_launches += 1;
            totals.mq_split_ms += a;
            totals.mq_merge_ms += b;
            durations[3].push_back(a);
            durations[4].push_back(b);
            for (auto e : v) hipEventDestroy(e);
        }
        mq_ev.clear();
        return hipSuccess;
    }
};

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

} // namespace

struct kv4_cache {
    kv4::State st;
    kv4::Sizes sizes;
    kv4_buffers bufs{};
    int device = 0;
    int num_cus = 256;
    int resident_waves = 2048; // decode split waves resident at once on the device
    int mq_resident_waves = 2048; // multi-query split waves resident at once
    int decode_waves = 0; // 0: automatic
    int round2_waves = 0; // decode split: waves of a second round (0: one round)
    int mq_share = 1;     // multi-query split: workgroup-shared INT4 steps where the row tiles allow
    int round1_permille = 1000; // share of the steps in the first round when there is a second
    float cb = 1.0f;
    void* scratch = nullptr;                // this device's decode scratch (kDecodeScratchBytes)
    std::vector<kv4::DecodeUnit> units_buf; // decode plan, reused (capacity for kArgEntries entries)
    Staging staging;
    Profiler prof;
    std::string err;
};

namespace {

kv4_status fail(kv4_cache* h, kv4_status s, const std::string& msg)
{
    if (h)
        h->err = msg;
    else
        g_last_error = msg;
    return s;
}

kv4_status hip_fail(kv4_cache* h, hipError_t e, const char* where)
{
    std::string m = std::string(where) + ": " + hipGetErrorString(e);
    return fail(h, KV4_ERR_HIP, m);
}

kv4::Config to_config(const kv4_config* c)
{
    kv4::Config k;
    k.hq = c->num_q_heads;
    k.hkv = c->num_kv_heads;
    k.d = c->head_dim;
    k.page = c->page_size;
    k.num_pages = c->num_pages;
    k.max_seqs = c->max_seqs;
    k.max_pps = c->max_pages_per_seq;
    k.sinks = c->num_sinks;
    k.recent = c->num_recent;
    k.block = c->hadamard_block;
    k.format = c->format;
    k.eviction = c->eviction;
    return k;
}

// RAII: make the cache's device current for the duration of a call.
struct DeviceGuard {
    int prev = -1;
    bool changed = false;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev)
    {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) {
            err = hipSetDevice(dev);
            changed = (err == hipSuccess);
        }
    }
    ~DeviceGuard()
    {
        if (changed) hipSetDevice(prev);
    }
};

// Decode split waves: one full round of resident waves.  With the issue-priority feedback between
// the two waves of a SIMD, a second round no longer pays: on MI355X the 8 x 128K-token call takes
// 205 + 6 us (split + merge) in one round against 210 + 11 us in two, the 256-sequence rollout
// call 356 + 9 against 359 + 8 us, and the 64-sequence Qwen3-8B layer 71 against 76 us.
int64_t auto_waves(const kv4_cache* h, int64_t /*total_steps*/) { return h->resident_waves; }


int64_t max_waves(const kv4_cache* h)
{
    int64_t w = 2 * (int64_t)h->resident_waves;
    if (h->decode_waves > w) w = h->decode_waves;
    return w;
}

size_t decode_ws_bytes(const kv4_cache* h, int64_t n_units, int64_t waves)
{
    const int G = h->st.cfg.hq / h->st.cfg.hkv;
    const int D = h->st.cfg.d;
    const int64_t parts = waves + n_units;
    return align_up((size_t)n_units * sizeof(kv4::DecodeUnit)) + align_up((size_t)parts * G * 2 * sizeof(float)) +
           align_up((size_t)parts * G * D * sizeof(float)) + align_up((size_t)n_units * 2 * sizeof(int32_t));
}

// Multi-query split tasks, in rounds of resident waves by the most row tiles (of kMqRows query rows)
// any (sequence, kv head) has: one round at one tile, three at two to four, two above.  Smaller
// chunks balance the waves of the few-tile calls, but each adds a partial per row tile.  With one
// tile, one round of chunks (the planner keeps the count within it) balances the waves and keeps
// the merge short: on the Qwen3-8B layer (MI355X) 4 rows per sequence take 86-94 + 6.6 us (split +
// merge) in one round against 100-104 + 10.4 us in two.  With many tiles per chunk, extra rounds
// only add partials and re-reads.  n_q is read only where it is positive; the call validates it.
int64_t mq_target_tasks(const kv4_cache* h, int32_t n_seqs, const int32_t* n_q)
{
    const int G = h->st.cfg.hq / h->st.cfg.hkv;
    int64_t tiles = 0;
    if (n_q)
        for (int32_t i = 0; i < n_seqs; i++)
            if (n_q[i] > 0) tiles = std::max<int64_t>(tiles, ((int64_t)n_q[i] * G + kv4::kMqRows - 1) / kv4::kMqRows);
    return (tiles <= 1 ? 1 : tiles <= 4 ? 3 : 2) * (int64_t)h->mq_resident_waves;
}

size_t mq_ws_bytes(const kv4_cache* h, const kv4::MqPlan& p)
{
    const int D = h->st.cfg.d;
    return align_up(p.entries.size() * sizeof(kv4::MqEntry)) +
           align_up((size_t)p.tasks * kv4::kMqRows * 2 * sizeof(float)) +
           align_up((size_t)p.tasks * kv4::kMqRows * D * sizeof(float));
}

size_t append_task_bound(int32_t n_seqs, const int32_t* n_new)
{
    size_t tasks = 0;
    for (int i = 0; i < n_seqs; i++)
        if (n_new[i] > 0) tasks += (size_t)n_new[i] / kv4::kPageSize + 2;
    return tasks;
}

} // namespace

extern "C" {

const char* kv4_status_string(kv4_status s)
{
    switch (s) {
    case KV4_OK: return "KV4_OK";
    case KV4_ERR_INVALID_ARGUMENT: return "KV4_ERR_INVALID_ARGUMENT";
    case KV4_ERR_OUT_OF_PAGES: return "KV4_ERR_OUT_OF_PAGES";
    case KV4_ERR_SEQ_STATE: return "KV4_ERR_SEQ_STATE";
    case KV4_ERR_WORKSPACE_TOO_SMALL: return "KV4_ERR_WORKSPACE_TOO_SMALL";
    case KV4_ERR_UNSUPPORTED: return "KV4_ERR_UNSUPPORTED";
    case KV4_ERR_HIP: return "KV4_ERR_HIP";
    }
    return "KV4_UNKNOWN_STATUS";
}

const char* kv4_last_error(kv4_cache_t h) { return h ? h->err.c_str() : g_last_error.c_str(); }

kv4_status kv4_buffer_sizes_query(const kv4_config* cfg, kv4_buffer_sizes* out)
{
    if (!cfg || !out) return fail(nullptr, KV4_ERR_INVALID_ARGUMENT, "null argument");
    kv4::Config c = to_config(cfg);
    std::string msg;
    kv4::Status s = kv4::check_config(c, &msg);
    if (s != kv4::OK) return fail(nullptr, (kv4_status)s, msg);
    kv4::Sizes z = kv4::buffer_sizes(c);
    out->page_pool = z.page_pool;
    out->int8_pool = z.int8_pool;
    out->block_table = z.block_table;
    out->page_block_bytes = z.page_block;
    out->int8_tile_bytes = z.int8_tile;
    out->int8_tiles = z.int8_tiles;
    return KV4_OK;
}

kv4_status kv4_cache_create(const kv4_config* cfg, const kv4_buffers* bufs, kv4_cache_t* out)
{
    if (!cfg || !bufs || !out) return fail(nullptr, KV4_ERR_INVALID_ARGUMENT, "null argument");
    kv4::Config c = to_config(cfg);
    std::string msg;
    kv4::Status s = kv4::check_config(c, &msg);
    if (s != kv4::OK) return fail(nullptr, (kv4_status)s, msg);
    kv4::Sizes z = kv4::buffer_sizes(c);
    if ((z.page_pool && !bufs->page_pool) || (z.int8_pool && !bufs->int8_pool) || !bufs->block_table)
        return fail(nullptr, KV4_ERR_INVALID_ARGUMENT, "missing device buffer");
    if (((uintptr_t)bufs->page_pool % kAlign) || ((uintptr_t)bufs->int8_pool % kAlign) ||
        ((uintptr_t)bufs->block_table % 4))
        return fail(nullptr, KV4_ERR_INVALID_ARGUMENT, "device buffers must be 256-byte aligned");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(nullptr, e, "hipGetDevice");
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(nullptr, e, "hipDeviceGetAttribute");
    kv4_cache* h = new (std::nothrow) kv4_cache();
    if (!h) return fail(nullptr, KV4_ERR_INVALID_ARGUMENT, "out of host memory");
    h->st.init(c);
    h->sizes = z;
    h->bufs = *bufs;
    h->device = dev;
    h->num_cus = cus > 0 ? cus : 256;
    {
        int bpc = 0;
        e = kv4::decode_split_residency(c.d, c.hq / c.hkv, c.format, &bpc);
        if (e != hipSuccess) {
            delete h;
            return hip_fail(nullptr, e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
        }
        h->resident_waves = (bpc > 0 ? bpc : 1) * kv4::kWavesPerBlock * h->num_cus;
        bpc = 0;
        if (c.format != kv4::FMT_BF16) {
            e = kv4::mq_split_residency(c.d, c.hq / c.hkv, c.format, &bpc);
            if (e != hipSuccess) {
                delete h;
                return hip_fail(nullptr, e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
            }
        }
        h->mq_resident_waves = (bpc > 0 ? bpc : 1) * 4 * h->num_cus;
    }
    // the allocation-free decode's scratch: looked up once per device, here where the device is
    // current and the library's kernels are being loaded anyway
    e = kv4::decode_scratch(&h->scratch);
    if (e != hipSuccess) {
        delete h;
        return hip_fail(nullptr, e, "hipGetSymbolAddress(decode scratch)");
    }
    h->units_buf.reserve((size_t)kv4::kArgEntries * c.hkv);
    h->cb = (float)(1.0 / std::sqrt((double)c.block));
    e = h->staging.init(8);
    if (e != hipSuccess) {
        h->staging.release();
        delete h;
        return hip_fail(nullptr, e, "hipEventCreate");
    }
    *out = h;
    return KV4_OK;
}

kv4_status kv4_cache_destroy(kv4_cache_t h)
{
    if (!h) return fail(nullptr, KV4_ERR_INVALID_ARGUMENT, "null handle");
    {
        DeviceGuard g(h->device);
        h->staging.release();
        h->prof.reset();
    }
    delete h;
    return KV4_OK;
}

kv4_status kv4_append_workspace_size(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new,
                                     size_t* bytes)
{
    (void)seq_ids;
    if (!h || !bytes || n_seqs < 0 || (n_seqs > 0 && !n_new)) return fail(h, KV4_ERR_INVALID_ARGUMENT, "bad argument");
    for (int i = 0; i < n_seqs; i++)
        if (n_new[i] < 0) return fail(h, KV4_ERR_INVALID_ARGUMENT, "n_new < 0");
    *bytes = align_up(append_task_bound(n_seqs, n_new) * sizeof(kv4::AppendTask));
    return KV4_OK;
}

} // extern "C"

namespace {

// kv4_append and kv4_append_rope: rope_cos == nullptr is the plain append.
kv4_status append_impl(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new, const void* k_new,
                       const void* v_new, void* workspace, size_t ws_bytes, void* stream, const float* rope_cos,
                       const float* rope_sin, int32_t rope_positions)
{
    if (!h) return fail(nullptr, KV4_ERR_INVALID_ARGUMENT, "null handle");
    if (n_seqs < 0 || (n_seqs > 0 && (!seq_ids || !n_new))) return fail(h, KV4_ERR_INVALID_ARGUMENT, "bad argument list");
    int64_t rows = 0;
    for (int i = 0; i < n_seqs; i++) {
        if (n_new[i] < 0) return fail(h, KV4_ERR_INVALID_ARGUMENT, "n_new < 0");
        rows += n_new[i];
    }
    if (rope_cos) {
        if (h->st.cfg.format == kv4::FMT_BF16)
            return fail(h, KV4_ERR_UNSUPPORTED, "the fused RoPE append needs a quantized format");
        if (!rope_sin || rope_positions < 0) return fail(h, KV4_ERR_INVALID_ARGUMENT, "bad RoPE tables");
        for (int i = 0; i < n_seqs; i++) {
            if (seq_ids[i] < 0 || seq_ids[i] >= h->st.cfg.max_seqs) continue; // the planner rejects it
            if ((int64_t)h->st.len[(size_t)seq_ids[i]] + n_new[i] > rope_positions)
                return fail(h, KV4_ERR_INVALID_ARGUMENT, "a new position is beyond the RoPE tables");
        }
    }
    if (rows > 0 && (!k_new || !v_new)) return fail(h, KV4_ERR_INVALID_ARGUMENT, "null k_new / v_new");
    const size_t need = align_up(append_task_bound(n_seqs, n_new) * sizeof(kv4::AppendTask));
    if (rows > 0 && (!workspace || ws_bytes < need))
        return fail(h, KV4_ERR_WORKSPACE_TOO_SMALL, "append workspace too small");
    std::vector<kv4::AppendTask> tasks;
    std::string msg;
    kv4::Status s = h->st.plan_append(n_seqs, seq_ids, n_new, &tasks, &msg);
    if (s != kv4::OK) return fail(h, (kv4_status)s, msg);
    if (tasks.empty()) return KV4_OK;

    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return hip_fail(h, g.err, "hipSetDevice");
    hipStream_t strm = (hipStream_t)stream;
    // calls whose tasks all write one position take the per-position kernel.  Up to kArgEntries
    // of them travel in the kernel arguments instead of an uploaded task list, but only when no
    // sequence has two tasks (n_new = 2 across a page boundary gives two): the argument plan does
    // not carry the length after the call, and the kernel takes it as t0 + 1.
    bool single = h->st.cfg.format == kv4::FMT_INT4_PROT;
    bool one_per_seq = true;
    for (size_t i = 0; i < tasks.size(); i++) {
        single = single && tasks[i].n == 1;
        one_per_seq = one_per_seq && (i == 0 || tasks[i].seq != tasks[i - 1].seq);
    }
    const bool argplan = single && one_per_seq && tasks.size() <= (size_t)kv4::kArgEntries;
    hipError_t e = hipSuccess;
    if (!argplan) {
        const size_t bytes = tasks.size() * sizeof(kv4::AppendTask);
        void* host = nullptr;
        int slot = 0;
        e = h->staging.acquire(bytes, &host, &slot);
        if (e != hipSuccess) return hip_fail(h, e, "staging");
        std::memcpy(host, tasks.data(), bytes);
        e = hipMemcpyAsync(workspace, host, bytes, hipMemcpyHostToDevice, strm);
        if (e != hipSuccess) return hip_fail(h, e, "hipMemcpyAsync");
        e = h->staging.commit(slot, strm);
        if (e != hipSuccess) return hip_fail(h, e, "hipEventRecord");
    }

    kv4::AppendArgs a;
    a.tasks = (const kv4::AppendTask*)workspace;
    a.max_pps = h->st.cfg.max_pps;
    a.n_arg = 0;
    if (argplan) {
        a.n_arg = (int)tasks.size();
        for (size_t i = 0; i < tasks.size(); i++) {
            a.arg_seq[i] = tasks[i].seq;
            a.arg_t0[i] = tasks[i].t0;
            a.arg_page[i] = (int32_t)((uint32_t)tasks[i].page | ((tasks[i].flags & kv4::kTaskNewPage) ? 0x80000000u : 0u));
        }
    }
    a.k = (const uint16_t*)k_new;
    a.v = (const uint16_t*)v_new;
    a.pool = (uint8_t*)h->bufs.page_pool;
    a.int8_pool = (uint8_t*)h->bufs.int8_pool;
    a.bt = h->bufs.block_table;
    a.page_block = (int64_t)h->sizes.page_block;
    a.int8_tile = (int64_t)h->sizes.int8_tile;
    a.hkv = h->st.cfg.hkv;
    a.block = h->st.cfg.block;
    a.sinks = h->st.cfg.sinks;
    a.recent = h->st.cfg.recent;
    a.int8_tiles = h->sizes.int8_tiles;
    a.cb = h->cb;
    a.requant = h->st.cfg.eviction;
    a.rope_cos = rope_cos;
    a.rope_sin = rope_sin;
    std::vector<hipEvent_t> ev;
    kv4::KernelTimer tm;
    if (h->prof.on) {
        e = Profiler::make(2, &ev);
        if (e != hipSuccess) return hip_fail(h, e, "profiling event");
        tm = kv4::KernelTimer{ev[0], ev[1]};
    }
    if (single)
        e = kv4::launch_append_token(h->st.cfg.d, (int)tasks.size(), a, strm, tm);
    else
        e = kv4::launch_append(h->st.cfg.d, h->st.cfg.format, (int)tasks.size(), a, strm, tm);
    if (e != hipSuccess) return hip_fail(h, e, "append launch");
    if (h->prof.on) h->prof.append_ev.push_back(ev);
    return KV4_OK;
}

} // namespace

extern "C" {

kv4_status kv4_append(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new, const void* k_new,
                      const void* v_new, void* workspace, size_t ws_bytes, void* stream)
{
    return append_impl(h, n_seqs, seq_ids, n_new, k_new, v_new, workspace, ws_bytes, stream, nullptr, nullptr, 0);
}

kv4_status kv4_append_rope(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new,
                           const void* k_new, const void* v_new, const float* rope_cos, const float* rope_sin,
                           int32_t rope_positions, void* workspace, size_t ws_bytes, void* stream)
{
    if (!h) return fail(nullptr, KV4_ERR_INVALID_ARGUMENT, "null handle");
    if (!rope_cos || !rope_sin) return fail(h, KV4_ERR_INVALID_ARGUMENT, "null RoPE tables");
    return append_impl(h, n_seqs, seq_ids, n_new, k_new, v_new, workspace, ws_bytes, stream, rope_cos, rope_sin,
                       rope_positions);
}

kv4_status kv4_seq_free(kv4_cache_t h, int32_t seq_id)
{
    if (!h) return fail(nullptr, KV4_ERR_INVALID_ARGUMENT, "null handle");
    std::string msg;
    kv4::Status s = h->st.seq_free(seq_id, &msg);
    if (s != kv4::OK) return fail(h, (kv4_status)s, msg);
    return KV4_OK;
}

kv4_status kv4_decode_workspace_size(kv4_cache_t h, int32_t n_seqs, size_t* bytes)
{
    if (!h || !bytes || n_seqs < 0) return fail(h, KV4_ERR_INVALID_ARGUMENT, "bad argument");
    *bytes = decode_ws_bytes(h, (int64_t)n_seqs * h->st.cfg.hkv, max_waves(h));
    return KV4_OK;
}

} // extern "C"

namespace {

// noalloc: the workspace is the device's decode scratch (workspace / ws_bytes ignored); the call
// then allocates nothing, host or device: the plan goes in the kernel arguments (at most
// kArgEntries sequences), the unit list reuses the handle's buffer, and no timing events are made.
kv4_status decode_impl(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const void* q, float scale, void* out_ptr,
                       bool out16, void* workspace, size_t ws_bytes, void* stream, bool noalloc = false)
{
    float* out = (float*)out_ptr;
    if (!h) return fail(nullptr, KV4_ERR_INVALID_ARGUMENT, "null handle");
    if (n_seqs < 0 || (n_seqs > 0 && (!seq_ids || !q || !out))) return fail(h, KV4_ERR_INVALID_ARGUMENT, "bad argument list");
    if (!std::isfinite(scale)) return fail(h, KV4_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (noalloc && n_seqs > kv4::kArgEntries)
        return fail(h, KV4_ERR_UNSUPPORTED, "the allocation-free decode takes at most 256 sequences per call");
    std::vector<kv4::DecodeUnit>& units = h->units_buf;
    int64_t total = 0;
    std::string msg;
    kv4::Status s = h->st.plan_decode(n_seqs, seq_ids, &units, &total, &msg);
    if (s != kv4::OK) return fail(h, (kv4_status)s, msg);
    if (units.empty()) return KV4_OK;
    const int64_t wmax = max_waves(h);
    int64_t W = h->decode_waves > 0 ? h->decode_waves : auto_waves(h, total);
    if (W > total) W = total;
    if (W < 1) W = 1;
    // optional second round: W2 more waves share the last (1000 - round1_permille) / 1000 of the
    // steps, when both rounds hold at least one step per wave
    const int64_t W1 = W;
    int64_t T1 = total;
    if (h->round2_waves > 0 && h->round1_permille < 1000) {
        const int64_t W2 = std::min<int64_t>(h->round2_waves, wmax - W1);
        const int64_t t1 = total * h->round1_permille / 1000;
        if (W2 > 0 && t1 >= W1 && total - t1 >= W2) {
            T1 = t1;
            W = W1 + W2;
        }
    }
    const int64_t n_units = (int64_t)units.size();
    if (noalloc) {
        workspace = h->scratch;
        ws_bytes = (size_t)kv4::kDecodeScratchBytes;
        if (decode_ws_bytes(h, n_units, W) > ws_bytes)
            return fail(h, KV4_ERR_WORKSPACE_TOO_SMALL,
                        "the call needs more than the 16 MiB of device scratch of the allocation-free decode");
    }
    if (!workspace || ws_bytes < decode_ws_bytes(h, n_units, W) || W > wmax)
        return fail(h, KV4_ERR_WORKSPACE_TOO_SMALL, "decode workspace too small");

    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return hip_fail(h, g.err, "hipSetDevice");
    hipStream_t strm = (hipStream_t)stream;
    const size_t ubytes = (size_t)n_units * sizeof(kv4::DecodeUnit);
    // up to kArgEntries sequences: the plan is the entry list in the kernel arguments (no upload)
    const bool argplan = n_seqs <= kv4::kArgEntries && total < ((int64_t)1 << 31);
    if (noalloc && !argplan) return fail(h, KV4_ERR_UNSUPPORTED, "the allocation-free decode needs an argument plan");
    hipError_t e = hipSuccess;
    if (!argplan) {
        void* host = nullptr;
        int slot = 0;
        e = h->staging.acquire(ubytes, &host, &slot);
        if (e != hipSuccess) return hip_fail(h, e, "staging");
        std::memcpy(host, units.data(), ubytes);
        e = hipMemcpyAsync(workspace, host, ubytes, hipMemcpyHostToDevice, strm);
        if (e != hipSuccess) return hip_fail(h, e, "hipMemcpyAsync");
        e = h->staging.commit(slot, strm);
        if (e != hipSuccess) return hip_fail(h, e, "hipEventRecord");
    }

    const int G = h->st.cfg.hq / h->st.cfg.hkv;
    const int D = h->st.cfg.d;
    const int64_t parts = W + n_units;
    uint8_t* ws = (uint8_t*)workspace;
    kv4::DecodeArgs a;
    a.pool = (const uint8_t*)h->bufs.page_pool;
    a.int8_pool = (const uint8_t*)h->bufs.int8_pool;
    a.bt = h->bufs.block_table;
    a.q = (const uint16_t*)q;
    a.units = (const kv4::DecodeUnit*)ws;
    a.part_ml = (float*)(ws + align_up(ubytes));
    a.part_o = (float*)(ws + align_up(ubytes) + align_up((size_t)parts * G * 2 * sizeof(float)));
    a.unit_waves = (int32_t*)((uint8_t*)a.part_o + align_up((size_t)parts * G * D * sizeof(float)));
    a.out = out;
    a.total_steps = total;
    a.steps1 = T1;
    a.n_waves1 = (int)W1;
    a.page_block = (int64_t)h->sizes.page_block;
    a.int8_tile = (int64_t)h->sizes.int8_tile;
    a.n_units = (int)n_units;
    a.n_waves = (int)W;
    a.hkv = h->st.cfg.hkv;
    a.max_pps = h->st.cfg.max_pps;
    a.sinks = h->st.cfg.sinks;
    a.recent = h->st.cfg.recent;
    a.block = h->st.cfg.block;
    a.int8_tiles = h->sizes.int8_tiles;
    a.cb = h->cb;
    const double sc = scale > 0.f ? (double)scale : 1.0 / std::sqrt((double)D);
    a.scale_log2 = (float)(sc * 1.4426950408889634);
    a.n_arg = 0;
    if (argplan) {
        a.n_arg = n_seqs;
        for (int i = 0; i < n_seqs; i++) {
            a.arg_seq[i] = seq_ids[i];
            a.arg_len[i] = h->st.len[(size_t)seq_ids[i]];
            a.arg_step[i] = (int32_t)units[(size_t)i * h->st.cfg.hkv].step_begin;
        }
    }
    std::vector<hipEvent_t> ev;
    kv4::KernelTimer t_split, t_merge;
    const bool timed = h->prof.on && !noalloc;
    if (timed) {
        e = Profiler::make(4, &ev);
        if (e != hipSuccess) return hip_fail(h, e, "profiling event");
        t_split = kv4::KernelTimer{ev[0], ev[1]};
        t_merge = kv4::KernelTimer{ev[2], ev[3]};
    }
    e = kv4::launch_decode_split(D, G, h->st.cfg.format, a, strm, t_split);
    if (e != hipSuccess) return hip_fail(h, e, "decode split launch");
    e = out16 ? kv4::launch_decode_merge_bf16(D, G, h->st.cfg.format, a, strm, t_merge)
              : kv4::launch_decode_merge(D, G, h->st.cfg.format, a, strm, t_merge);
    if (e != hipSuccess) return hip_fail(h, e, "decode merge launch");
    if (timed) h->prof.decode_ev.push_back(ev);
    return KV4_OK;
}

} // namespace

extern "C" {

kv4_status kv4_decode_attention(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const void* q, float scale,
                                float* out, void* workspace, size_t ws_bytes, void* stream)
{
    return decode_impl(h, n_seqs, seq_ids, q, scale, out, false, workspace, ws_bytes, stream);
}

kv4_status kv4_decode_attention_bf16(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const void* q,
                                     float scale, void* out, void* workspace, size_t ws_bytes, void* stream)
{
    return decode_impl(h, n_seqs, seq_ids, q, scale, out, true, workspace, ws_bytes, stream);
}

kv4_status kv4_decode_attention_noalloc(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const void* q,
                                        float scale, float* out, void* stream)
{
    return decode_impl(h, n_seqs, seq_ids, q, scale, out, false, nullptr, 0, stream, true);
}

kv4_status kv4_multi_query_workspace_size(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_q,
                                          size_t* bytes)
{
    if (!h || !bytes) return fail(h, KV4_ERR_INVALID_ARGUMENT, "null argument");
    kv4::MqPlan plan;
    std::string msg;
    kv4::Status s = h->st.plan_multi(n_seqs, seq_ids, n_q, mq_target_tasks(h, n_seqs, n_q), &plan, &msg);
    if (s != kv4::OK) return fail(h, (kv4_status)s, msg);
    *bytes = mq_ws_bytes(h, plan);
    return KV4_OK;
}

kv4_status kv4_multi_query_attention(kv4_cache_t h, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_q,
                                     const void* q, float scale, float* out, void* workspace, size_t ws_bytes,
                                     void* stream)
{
    if (!h) return fail(nullptr, KV4_ERR_INVALID_ARGUMENT, "null handle");
    if (n_seqs < 0 || (n_seqs > 0 && (!seq_ids || !n_q || !q || !out)))
        return fail(h, KV4_ERR_INVALID_ARGUMENT, "bad argument list");
    if (!std::isfinite(scale)) return fail(h, KV4_ERR_INVALID_ARGUMENT, "scale must be finite");
    kv4::MqPlan plan;
    std::string msg;
    kv4::Status s = h->st.plan_multi(n_seqs, seq_ids, n_q, mq_target_tasks(h, n_seqs, n_q), &plan, &msg);
    if (s != kv4::OK) return fail(h, (kv4_status)s, msg);
    if (plan.entries.empty()) return KV4_OK;
    if (!workspace || ws_bytes < mq_ws_bytes(h, plan))
        return fail(h, KV4_ERR_WORKSPACE_TOO_SMALL, "multi-query workspace too small");

    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return hip_fail(h, g.err, "hipSetDevice");
    hipStream_t strm = (hipStream_t)stream;
    const size_t ebytes = plan.entries.size() * sizeof(kv4::MqEntry);
    void* host = nullptr;
    int slot = 0;
    hipError_t e = h->staging.acquire(ebytes, &host, &slot);
    if (e != hipSuccess) return hip_fail(h, e, "staging");
    std::memcpy(host, plan.entries.data(), ebytes);
    e = hipMemcpyAsync(workspace, host, ebytes, hipMemcpyHostToDevice, strm);
    if (e != hipSuccess) return hip_fail(h, e, "hipMemcpyAsync");
    e = h->staging.commit(slot, strm);
    if (e != hipSuccess) return hip_fail(h, e, "hipEventRecord");

    const int G = h->st.cfg.hq / h->st.cfg.hkv;
    const int D = h->st.cfg.d;
    uint8_t* ws = (uint8_t*)workspace;
    kv4::MqArgs a;
    a.pool = (const uint8_t*)h->bufs.page_pool;
    a.int8_pool = (const uint8_t*)h->bufs.int8_pool;
    a.bt = h->bufs.block_table;
    a.q = (const uint16_t*)q;
    a.entries = (const kv4::MqEntry*)ws;
    a.part_ml = (float*)(ws + align_up(ebytes));
    a.part_o = (float*)(ws + align_up(ebytes) + align_up((size_t)plan.tasks * kv4::kMqRows * 2 * sizeof(float)));
    a.out = out;
    a.page_block = (int64_t)h->sizes.page_block;
    a.int8_tile = (int64_t)h->sizes.int8_tile;
    a.n_entries = (int)plan.entries.size();
    a.tasks = (int)plan.tasks;
    a.groups = (int)plan.groups;
    a.spc = plan.spc;
    a.hq = h->st.cfg.hq;
    a.hkv = h->st.cfg.hkv;
    a.max_pps = h->st.cfg.max_pps;
    a.sinks = h->st.cfg.sinks;
    a.recent = h->st.cfg.recent;
    a.block = h->st.cfg.block;
    a.int8_tiles = h->sizes.int8_tiles;
    a.n8 = kv4::mq_int8_steps(h->st.cfg);
    // the shared kernel takes row tiles 4k .. 4k + 3 of one chunk per workgroup
    a.share = 0;
    if (h->mq_share && h->st.cfg.format == kv4::FMT_INT4_PROT) {
        a.share = 1;
        for (const kv4::MqEntry& en : plan.entries)
            if ((((int64_t)en.nq * G + kv4::kMqRows - 1) / kv4::kMqRows) % 4 != 0) a.share = 0;
    }
    a.cb = h->cb;
    const double sc = scale > 0.f ? (double)scale : 1.0 / std::sqrt((double)D);
    a.scale_log2 = (float)(sc * 1.4426950408889634);
    std::vector<hipEvent_t> ev;
    kv4::KernelTimer t_split, t_merge;
    if (h->prof.on) {
        e = Profiler::make(4, &ev);
        if (e != hipSuccess) return hip_fail(h, e, "profiling event");
        t_split = kv4::KernelTimer{ev[0], ev[1]};
        t_merge = kv4::KernelTimer{ev[2], ev[3]};
    }
    e = kv4::launch_mq_split(D, G, h->st.cfg.format, a, strm, t_split);
    if (e != hipSuccess) return hip_fail(h, e, "multi-query split launch");
    // row tiles of a single chunk are written by the split kernel; the merge runs for the others
    bool merge = false;
    for (const kv4::MqEntry& en : plan.entries) merge = merge || en.nch > 1;
    if (merge) {
        e = kv4::launch_mq_merge(D, G, a, strm, t_merge);
        if (e != hipSuccess) return hip_fail(h, e, "multi-query merge launch");
    } else if (h->prof.on) {
        // no merge: its event pair brackets nothing
        e = hipEventRecord(ev[2], strm);
        if (e == hipSuccess) e = hipEventRecord(ev[3], strm);
        if (e != hipSuccess) return hip_fail(h, e, "hipEventRecord");
    }
    if (h->prof.on) h->prof.mq_ev.push_back(ev);
    return KV4_OK;
}

kv4_status kv4_seq_length(kv4_cache_t h, int32_t seq_id, int32_t* len)
{
    if (!h || !len) return fail(h, KV4_ERR_INVALID_ARGUMENT, "null argument");
    if (seq_id < 0 || seq_id >= h->st.cfg.max_seqs) return fail(h, KV4_ERR_INVALID_ARGUMENT, "sequence id out of range");
    *len = h->st.len[(size_t)seq_id];
    return KV4_OK;
}

kv4_status kv4_block_table(kv4_cache_t h, int32_t seq_id, int32_t* pages, int32_t cap, int32_t* n)
{
    if (!h || !n || cap < 0 || (cap > 0 && !pages)) return fail(h, KV4_ERR_INVALID_ARGUMENT, "bad argument");
    if (seq_id < 0 || seq_id >= h->st.cfg.max_seqs) return fail(h, KV4_ERR_INVALID_ARGUMENT, "sequence id out of range");
    const int np = (h->st.len[(size_t)seq_id] + kv4::kPageSize - 1) / kv4::kPageSize;
    for (int j = 0; j < np && j < cap; j++) pages[j] = h->st.bt[(size_t)seq_id * h->st.cfg.max_pps + j];
    *n = np;
    return KV4_OK;
}

kv4_status kv4_free_pages(kv4_cache_t h, int32_t* n)
{
    if (!h || !n) return fail(h, KV4_ERR_INVALID_ARGUMENT, "null argument");
    *n = (int32_t)h->st.free_list.size();
    return KV4_OK;
}

kv4_status kv4_set_decode_waves(kv4_cache_t h, int32_t waves)
{
    if (!h || waves < 0) return fail(h, KV4_ERR_INVALID_ARGUMENT, "bad argument");
    h->decode_waves = waves;
    return KV4_OK;
}

kv4_status kv4_set_decode_rounds(kv4_cache_t h, int32_t round2_waves, int32_t round1_permille)
{
    if (!h || round2_waves < 0 || round1_permille < 1 || round1_permille > 1000)
        return fail(h, KV4_ERR_INVALID_ARGUMENT, "bad argument");
    h->round2_waves = round2_waves;
    h->round1_permille = round1_permille;
    return KV4_OK;
}

kv4_status kv4_set_mq_share(kv4_cache_t h, int32_t enable)
{
    if (!h) return fail(nullptr, KV4_ERR_INVALID_ARGUMENT, "null handle");
    h->mq_share = enable != 0;
    return KV4_OK;
}

kv4_status kv4_profile_enable(kv4_cache_t h, int32_t enable)
{
    if (!h) return fail(nullptr, KV4_ERR_INVALID_ARGUMENT, "null handle");
    DeviceGuard g(h->device);
    h->prof.reset();
    h->prof.on = enable != 0;
    return KV4_OK;
}

kv4_status kv4_profile_read(kv4_cache_t h, kv4_profile* out)
{
    if (!h || !out) return fail(h, KV4_ERR_INVALID_ARGUMENT, "null argument");
    DeviceGuard g(h->device);
    hipError_t e = h->prof.collect();
    if (e != hipSuccess) return hip_fail(h, e, "profiling events");
    *out = h->prof.totals;
    return KV4_OK;
}

kv4_status kv4_profile_durations(kv4_cache_t h, int32_t kind, float* ms, int32_t cap, int32_t* n)
{
    if (!h || !n || kind < 0 || kind > 4 || cap < 0 || (cap > 0 && !ms))
        return fail(h, KV4_ERR_INVALID_ARGUMENT, "bad argument");
    DeviceGuard g(h->device);
    hipError_t e = h->prof.collect();
    if (e != hipSuccess) return hip_fail(h, e, "profiling events");
    const std::vector<float>& d = h->prof.durations[kind];
    for (size_t i = 0; i < d.size() && i < (size_t)cap; i++) ms[i] = d[i];
    *n = (int32_t)d.size();
    return KV4_OK;
}

kv4_status kv4_hbm_probe(int32_t mode, const void* src, void* dst, size_t bytes, int32_t blocks, int32_t reps,
                         float* ms, void* stream)
{
    if ((mode != 0 && mode != 1) || !src || !dst || bytes == 0 || bytes % 16 || ((uintptr_t)src % 16) ||
        ((uintptr_t)dst % 16) || reps < 1 || !ms || blocks < 0)
        return fail(nullptr, KV4_ERR_INVALID_ARGUMENT, "bad probe argument");
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(nullptr, e, "device query");
    if (blocks == 0) blocks = 8 * (cus > 0 ? cus : 256);
    hipStream_t strm = (hipStream_t)stream;
    std::vector<hipEvent_t> ev;
    e = Profiler::make(2 * reps, &ev);
    kv4_status st = KV4_OK;
    for (int r = 0; r < reps && e == hipSuccess; r++)
        e = kv4::launch_probe(mode, src, dst, (uint64_t)bytes, blocks, strm, kv4::KernelTimer{ev[2 * r], ev[2 * r + 1]});
    if (e == hipSuccess) e = hipEventSynchronize(ev[2 * reps - 1]);
    for (int r = 0; r < reps && e == hipSuccess; r++) e = hipEventElapsedTime(&ms[r], ev[2 * r], ev[2 * r + 1]);
    if (e != hipSuccess) st = hip_fail(nullptr, e, "probe");
    for (auto x : ev)
        if (x) hipEventDestroy(x);
    return st;
}

} // extern "C"
