// kv4_plan.hpp -- host-side state of a kv4 cache: configuration checks, the FIFO page allocator,
// the host mirror of lengths and block tables, and the plans that the append and decode kernels
// consume.  Pure C++17 (no HIP), so the same code is exercised by a host-only test program.
//
// The paged layout and the per-call page allocation realise the paged KV-cache constraint of
// "SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for Real-World LLM Serving" (Abstract); the
// protected set follows "KV4-RL: Unlocking Faster Asynchronous Rollouts for RLVR with INT4 KV
// Cache Quantization" (Abstract: sinks and recent context, a bounded number of positions).
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <deque>
#include <string>
#include <vector>

#include "kv4_device_types.h"
#include "kv4_mq_types.h"

namespace kv4 {

enum Status : int {
    OK = 0,
    INVALID_ARGUMENT = 1,
    OUT_OF_PAGES = 2,
    SEQ_STATE = 3,
    WORKSPACE_TOO_SMALL = 4,
    UNSUPPORTED = 5,
    HIP_ERROR = 6
};

enum Format : int { FMT_INT4_PROT = 0, FMT_INT8 = 1, FMT_BF16 = 2 };

struct Config {
    int hq = 0, hkv = 0, d = 0, page = 0, num_pages = 0, max_seqs = 0, max_pps = 0;
    int sinks = 0, recent = 0, block = 1, format = 0;
    int eviction = 0; // 0: dual write, 1: INT4 re-quantized from the INT8 round trip
};

struct Sizes {
    size_t page_pool = 0, int8_pool = 0, block_table = 0, page_block = 0, int8_tile = 0;
    int int8_tiles = 0;
};

inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// Validates a configuration; returns OK, INVALID_ARGUMENT or UNSUPPORTED with a message.
inline Status check_config(const Config& c, std::string* msg)
{
    auto bad = [&](Status s, const char* m) {
        if (msg) *msg = m;
        return s;
    };
    if (c.hq <= 0 || c.hkv <= 0) return bad(INVALID_ARGUMENT, "head counts must be positive");
    if (c.hq % c.hkv) return bad(INVALID_ARGUMENT, "num_q_heads must be a multiple of num_kv_heads");
    if (c.d <= 0 || c.page <= 0 || c.num_pages < 0 || c.max_seqs <= 0 || c.max_pps <= 0)
        return bad(INVALID_ARGUMENT, "sizes must be positive (num_pages >= 0)");
    if (c.sinks < 0 || c.recent < 0) return bad(INVALID_ARGUMENT, "num_sinks / num_recent must be >= 0");
    if (!is_pow2(c.block)) return bad(INVALID_ARGUMENT, "hadamard_block must be a power of two");
    if (c.d % c.block) return bad(INVALID_ARGUMENT, "hadamard_block must divide head_dim");
    if (c.format < 0 || c.format > 2) return bad(INVALID_ARGUMENT, "unknown format");
    if (c.eviction < 0 || c.eviction > 1) return bad(INVALID_ARGUMENT, "unknown eviction rule");
    if (c.eviction == 1 && c.format != FMT_INT4_PROT)
        return bad(INVALID_ARGUMENT, "re-quantizing eviction needs the INT4_PROT format");
    if (c.page != kPageSize) return bad(UNSUPPORTED, "page_size must be 16");
    if (c.d != 64 && c.d != 128) return bad(UNSUPPORTED, "head_dim must be 64 or 128");
    int g = c.hq / c.hkv;
    if (g != 1 && g != 2 && g != 4) return bad(UNSUPPORTED, "GQA group size must be 1, 2 or 4");
    if ((long long)c.max_seqs * c.max_pps > (1LL << 30)) return bad(UNSUPPORTED, "block table too large");
    return OK;
}

inline Sizes buffer_sizes(const Config& c)
{
    Sizes s;
    size_t D = (size_t)c.d;
    s.int8_tile = 2 * (16 * D + 128); // two blocks shaped like an INT4 page block
    if (c.format == FMT_INT4_PROT)
        s.page_block = 16 * D + 128;
    else if (c.format == FMT_INT8)
        s.page_block = s.int8_tile;
    else
        s.page_block = 64 * D;
    s.page_pool = (size_t)c.num_pages * c.hkv * s.page_block;
    if (c.format == FMT_INT4_PROT && c.sinks + c.recent > 0) {
        s.int8_tiles = (c.sinks + c.recent + kPageSize - 1) / kPageSize;
        s.int8_pool = (size_t)c.max_seqs * c.hkv * s.int8_tiles * s.int8_tile;
    }
    s.block_table = (size_t)c.max_seqs * c.max_pps * sizeof(int32_t);
    return s;
}

// Number of decode steps of one (sequence, kv head) unit at length L (see kv4_device_types.h for
// what one step covers in each format).
inline int unit_int8_steps(const Config& c, int L)
{
    if (c.format != FMT_INT4_PROT || c.sinks + c.recent == 0 || L <= 0) return 0;
    return (c.sinks + c.recent + kInt8StepSlots - 1) / kInt8StepSlots;
}

// First and one-past-last page index of the INT4-read positions [S, L - R) (empty when L <= S + R).
inline void unit_int4_pages(const Config& c, int L, int* p0, int* p1)
{
    int lo = c.sinks, hi = L - c.recent;
    if (hi <= lo) {
        *p0 = *p1 = 0;
        return;
    }
    *p0 = lo / kPageSize;
    *p1 = (hi - 1) / kPageSize + 1;
}

// Decode steps of one (entry, kv head) unit that read the cache.
inline int unit_work_steps(const Config& c, int L)
{
    if (c.format == FMT_INT4_PROT) {
        int p0, p1;
        unit_int4_pages(c, L, &p0, &p1);
        return unit_int8_steps(c, L) + (p1 - p0 + kInt4StepPages - 1) / kInt4StepPages;
    }
    int pages = (L + kPageSize - 1) / kPageSize;
    if (c.format == FMT_INT8) return (pages + kInt8StepPages - 1) / kInt8StepPages;
    return pages; // bf16: one page per step
}

// The unit's share of the global step range: its start charge, then its work steps.
inline int unit_steps(const Config& c, int L) { return kUnitStartSteps + unit_work_steps(c, L); }

// Multi-query attention steps of one (sequence, kv head): INT4_PROT reads its INT8 protection
// tiles two at a time, then the INT4 pages of [S, L - R) two at a time; the INT8 format reads its
// pages two at a time.  (The BF16 format has no multi-query kernel.)
inline int mq_int8_steps(const Config& c)
{
    if (c.format != FMT_INT4_PROT || c.sinks + c.recent == 0) return 0;
    const int tiles = (c.sinks + c.recent + kPageSize - 1) / kPageSize;
    return (tiles + 1) / 2;
}

inline int mq_unit_steps(const Config& c, int L)
{
    if (c.format == FMT_INT4_PROT) {
        int p0, p1;
        unit_int4_pages(c, L, &p0, &p1);
        return mq_int8_steps(c) + (p1 - p0 + 1) / 2;
    }
    return ((L + kPageSize - 1) / kPageSize + 1) / 2;
}

struct MqPlan {
    std::vector<MqEntry> entries;
    int64_t tasks = 0;  // wave tasks of the split kernel
    int64_t groups = 0; // (entry, kv head, row tile) groups; the merge runs 16 waves per group
    int spc = 1;        // steps per chunk
    int64_t rows = 0;   // query rows of the call (sum of n_q)
};

struct State {
    Config cfg;
    std::deque<int32_t> free_list;
    std::vector<int32_t> len;       // [max_seqs]
    std::vector<int32_t> bt;        // [max_seqs * max_pps]
    std::vector<uint8_t> mark;      // [max_seqs], all 0 between calls: duplicate-id test of plan_decode

    void init(const Config& c)
    {
        cfg = c;
        free_list.clear();
        for (int i = 0; i < c.num_pages; i++) free_list.push_back(i);
        len.assign((size_t)c.max_seqs, 0);
        bt.assign((size_t)c.max_seqs * c.max_pps, -1);
        mark.assign((size_t)c.max_seqs, 0);
    }

    // Validates an append and, on success, builds its page tasks and commits the host state.
    // Returns a status; on any error nothing changes.
    Status plan_append(int n_seqs, const int32_t* ids, const int32_t* n_new, std::vector<AppendTask>* tasks,
                       std::string* msg)
    {
        auto bad = [&](Status s, const std::string& m) {
            if (msg) *msg = m;
            return s;
        };
        if (n_seqs < 0) return bad(INVALID_ARGUMENT, "n_seqs < 0");
        if (n_seqs > 0 && (!ids || !n_new)) return bad(INVALID_ARGUMENT, "null seq_ids / n_new");
        std::vector<uint8_t> seen((size_t)cfg.max_seqs, 0);
        long long needed = 0;
        for (int i = 0; i < n_seqs; i++) {
            int s = ids[i];
            if (s < 0 || s >= cfg.max_seqs) return bad(INVALID_ARGUMENT, "sequence id out of range");
            if (seen[(size_t)s]) return bad(INVALID_ARGUMENT, "duplicate sequence id in one call");
            seen[(size_t)s] = 1;
            if (n_new[i] < 0) return bad(INVALID_ARGUMENT, "n_new < 0");
            long long L0 = len[(size_t)s], L1 = L0 + n_new[i];
            if (L1 > (long long)cfg.max_pps * cfg.page) return bad(SEQ_STATE, "sequence would exceed max_pages_per_seq");
            needed += (L1 + cfg.page - 1) / cfg.page - (L0 + cfg.page - 1) / cfg.page;
        }
        if (needed > (long long)free_list.size()) return bad(OUT_OF_PAGES, "not enough free pages for the call");
        // commit: pages popped from the front, sequences in call order, positions ascending
        tasks->clear();
        int64_t row = 0;
        for (int i = 0; i < n_seqs; i++) {
            int s = ids[i];
            int L0 = len[(size_t)s], L1 = L0 + n_new[i];
            int t = L0;
            while (t < L1) {
                int pidx = t / cfg.page;
                int32_t* slot = &bt[(size_t)s * cfg.max_pps + pidx];
                int flags = 0;
                if (t % cfg.page == 0) {
                    *slot = free_list.front();
                    free_list.pop_front();
                    flags |= kTaskNewPage;
                }
                int end = (pidx + 1) * cfg.page;
                if (end > L1) end = L1;
                AppendTask tk;
                tk.seq = s;
                tk.page = *slot;
                tk.t0 = t;
                tk.n = end - t;
                tk.row0 = (int32_t)row;
                tk.len_new = L1;
                tk.bt_index = s * cfg.max_pps + pidx;
                tk.flags = flags;
                tasks->push_back(tk);
                row += end - t;
                t = end;
            }
            len[(size_t)s] = L1;
        }
        return OK;
    }

    Status seq_free(int s, std::string* msg)
    {
        if (s < 0 || s >= cfg.max_seqs) {
            if (msg) *msg = "sequence id out of range";
            return INVALID_ARGUMENT;
        }
        int n = (len[(size_t)s] + cfg.page - 1) / cfg.page;
        for (int j = 0; j < n; j++) {
            free_list.push_back(bt[(size_t)s * cfg.max_pps + j]);
            bt[(size_t)s * cfg.max_pps + j] = -1;
        }
        len[(size_t)s] = 0;
        return OK;
    }

    // Decode plan: one unit per (call entry, kv head), with its step prefix.  Returns the total
    // step count in *total.  Allocates nothing once `units` has the capacity for the call (the
    // duplicate-id test uses the state's own marks and clears them again).
    Status plan_decode(int n_seqs, const int32_t* ids, std::vector<DecodeUnit>* units, int64_t* total,
                       std::string* msg)
    {
        auto bad = [&](Status s, const char* m) {
            if (msg) *msg = m;
            return s;
        };
        if (n_seqs < 0) return bad(INVALID_ARGUMENT, "n_seqs < 0");
        if (n_seqs > 0 && !ids) return bad(INVALID_ARGUMENT, "null seq_ids");
        Status st = OK;
        const char* why = nullptr;
        int marked = 0;
        for (; marked < n_seqs; marked++) {
            int s = ids[marked];
            if (s < 0 || s >= cfg.max_seqs) {
                st = INVALID_ARGUMENT;
                why = "sequence id out of range";
                break;
            }
            if (mark[(size_t)s]) {
                st = INVALID_ARGUMENT;
                why = "duplicate sequence id in one call";
                break;
            }
            mark[(size_t)s] = 1;
            if (len[(size_t)s] < 1) {
                st = SEQ_STATE;
                why = "decode of an empty sequence";
                marked++;
                break;
            }
        }
        for (int i = 0; i < marked; i++) mark[(size_t)ids[i]] = 0;
        if (st != OK) return bad(st, why);
        units->clear();
        int64_t acc = 0;
        for (int i = 0; i < n_seqs; i++) {
            int s = ids[i];
            int L = len[(size_t)s];
            int st = unit_steps(cfg, L);
            for (int h = 0; h < cfg.hkv; h++) {
                DecodeUnit u;
                u.seq = s;
                u.len = L;
                u.entry = i;
                u.head = h;
                u.step_begin = acc;
                acc += st;
                units->push_back(u);
            }
        }
        *total = acc;
        return OK;
    }

    // Multi-query plan: validates the call (ids distinct, 1 <= n_q[i] <= L) and splits every
    // (entry, kv head, row tile) into chunks of `spc` steps, spc chosen so that the call has about
    // `target_tasks` wave tasks.
    Status plan_multi(int n_seqs, const int32_t* ids, const int32_t* n_q, int64_t target_tasks, MqPlan* plan,
                      std::string* msg)
    {
        auto bad = [&](Status s, const char* m) {
            if (msg) *msg = m;
            return s;
        };
        if (cfg.format == FMT_BF16) return bad(UNSUPPORTED, "multi-query attention needs a quantized format");
        if (n_seqs < 0) return bad(INVALID_ARGUMENT, "n_seqs < 0");
        if (n_seqs > 0 && (!ids || !n_q)) return bad(INVALID_ARGUMENT, "null seq_ids / n_q");
        std::vector<uint8_t> seen((size_t)cfg.max_seqs, 0);
        for (int i = 0; i < n_seqs; i++) {
            int s = ids[i];
            if (s < 0 || s >= cfg.max_seqs) return bad(INVALID_ARGUMENT, "sequence id out of range");
            if (seen[(size_t)s]) return bad(INVALID_ARGUMENT, "duplicate sequence id in one call");
            seen[(size_t)s] = 1;
            if (n_q[i] < 1) return bad(INVALID_ARGUMENT, "n_q < 1");
            if (len[(size_t)s] < 1) return bad(SEQ_STATE, "attention over an empty sequence");
            if (n_q[i] > len[(size_t)s]) return bad(SEQ_STATE, "n_q exceeds the sequence length");
        }
        const int G = cfg.hq / cfg.hkv;
        int64_t work = 0, rows = 0;
        for (int i = 0; i < n_seqs; i++) {
            const int64_t nrt = ((int64_t)n_q[i] * G + kMqRows - 1) / kMqRows;
            work += (int64_t)cfg.hkv * nrt * mq_unit_steps(cfg, len[(size_t)ids[i]]);
            rows += n_q[i];
        }
        if (target_tasks < 1) target_tasks = 1;
        int64_t spc = (work + target_tasks - 1) / target_tasks;
        if (spc < 1) spc = 1;
        // Each (sequence, kv head, row tile) rounds its chunk count up, so the count can pass the
        // target, and the tasks past a whole number of resident rounds then run nearly alone at
        // the end.  The chunk grows until the count fits, or until it covers the longest unit
        // (one task per row tile, the smallest count there is).
        int64_t max_steps = 1;
        for (int i = 0; i < n_seqs; i++) max_steps = std::max<int64_t>(max_steps, mq_unit_steps(cfg, len[(size_t)ids[i]]));
        auto count = [&](int64_t c) {
            int64_t t = 0;
            for (int i = 0; i < n_seqs; i++) {
                const int64_t nrt = ((int64_t)n_q[i] * G + kMqRows - 1) / kMqRows;
                t += (int64_t)cfg.hkv * nrt * ((mq_unit_steps(cfg, len[(size_t)ids[i]]) + c - 1) / c);
            }
            return t;
        };
        if (spc < max_steps && count(spc) > target_tasks) {
            // the count does not grow with the chunk: the smallest chunk that fits, by bisection
            // (count(lo) > target >= count(hi) throughout)
            int64_t lo = spc, hi = max_steps;
            if (count(hi) <= target_tasks) {
                while (hi - lo > 1) {
                    const int64_t mid = lo + (hi - lo) / 2;
                    if (count(mid) > target_tasks)
                        lo = mid;
                    else
                        hi = mid;
                }
            }
            spc = hi;
        }
        plan->entries.clear();
        int64_t qrow = 0;
        for (int i = 0; i < n_seqs; i++) {
            const int L = len[(size_t)ids[i]];
            MqEntry e;
            e.seq = ids[i];
            e.len = L;
            e.nq = n_q[i];
            e.qrow0 = (int32_t)qrow; // rows of the caller's q and out, in call order
            e.steps = mq_unit_steps(cfg, L);
            e.nch = (int32_t)((e.steps + spc - 1) / spc);
            plan->entries.push_back(e);
            qrow += n_q[i];
            if (qrow >= ((int64_t)1 << 30)) return bad(UNSUPPORTED, "multi-query call too large");
        }
        // Tasks are numbered longest entry first.  Workgroups start in task order, so the longest
        // tasks start first and the short ones fill in at the end.  (The kernels find an entry by
        // its first task or merge group, which still increase along the list.)
        std::stable_sort(plan->entries.begin(), plan->entries.end(),
                         [](const MqEntry& x, const MqEntry& y) { return x.steps > y.steps; });
        int64_t tasks = 0, groups = 0;
        for (MqEntry& e : plan->entries) {
            const int64_t nrt = ((int64_t)e.nq * G + kMqRows - 1) / kMqRows;
            e.task0 = (int32_t)tasks;
            e.grp0 = (int32_t)groups;
            tasks += (int64_t)cfg.hkv * e.nch * nrt;
            groups += (int64_t)cfg.hkv * nrt;
            if (tasks >= ((int64_t)1 << 27)) return bad(UNSUPPORTED, "multi-query call too large");
        }
        plan->tasks = tasks;
        plan->groups = groups;
        plan->spc = (int)spc;
        plan->rows = rows;
        return OK;
    }
};

} // namespace kv4
