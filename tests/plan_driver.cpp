// plan_driver.cpp -- host-only test program for the library's planner (kv4_plan.hpp): reads
// commands on stdin, applies them to one planner state and prints what the planner decided, so
// a test can compare the allocator, the block tables and the work lists with the CPU oracle.
//
// Commands (one per line), and what they print:
//   init hq hkv d page num_pages max_seqs max_pps sinks recent block format
//                                -> "status S"
//   append n id0 n0 id1 n1 ...   -> "status S", then one "task seq page t0 n row0 len_new bt_index flags"
//                                   line per append task, then "end"
//   free id                      -> "status S"
//   bt id                        -> "bt LEN p0 p1 ..." (the sequence's pages, in order)
//   freepages                    -> "free N"
//   decode n id0 id1 ...         -> "status S total T start C" (C = the start charge of every unit's
//                                   step range), then one "unit seq len entry head step_begin" line
//                                   per unit, then "end"
//   sizes                        -> "sizes page_pool int8_pool block_table page_block int8_tile int8_tiles"
//   multi target n id0 nq0 ...   -> "status S tasks T groups G spc C n8 N8", then one
//                                   "entry seq len nq qrow0 task0 grp0 steps nch" line per entry, "end"
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "kv4_plan.hpp"

int main()
{
    kv4::State st;
    bool ready = false;
    std::string line;
    while (std::getline(std::cin, line)) {
        std::istringstream in(line);
        std::string cmd;
        if (!(in >> cmd)) continue;
        if (cmd == "init") {
            kv4::Config c;
            in >> c.hq >> c.hkv >> c.d >> c.page >> c.num_pages >> c.max_seqs >> c.max_pps >> c.sinks >> c.recent >>
                c.block >> c.format;
            kv4::Status s = kv4::check_config(c, nullptr);
            if (s == kv4::OK) {
                st.init(c);
                ready = true;
            }
            std::printf("status %d\n", (int)s);
        } else if (!ready) {
            std::printf("status -1\n");
        } else if (cmd == "append") {
            int n = 0;
            in >> n;
            std::vector<int32_t> ids(n > 0 ? n : 0), nn(n > 0 ? n : 0);
            for (int i = 0; i < n; i++) in >> ids[i] >> nn[i];
            std::vector<kv4::AppendTask> tasks;
            kv4::Status s = st.plan_append(n, ids.data(), nn.data(), &tasks, nullptr);
            std::printf("status %d\n", (int)s);
            if (s == kv4::OK)
                for (const auto& t : tasks)
                    std::printf("task %d %d %d %d %d %d %d %d\n", t.seq, t.page, t.t0, t.n, t.row0, t.len_new,
                                t.bt_index, t.flags);
            std::printf("end\n");
        } else if (cmd == "free") {
            int id = 0;
            in >> id;
            std::printf("status %d\n", (int)st.seq_free(id, nullptr));
        } else if (cmd == "bt") {
            int id = 0;
            in >> id;
            int L = st.len[(size_t)id];
            int np = (L + st.cfg.page - 1) / st.cfg.page;
            std::printf("bt %d", L);
            for (int j = 0; j < np; j++) std::printf(" %d", st.bt[(size_t)id * st.cfg.max_pps + j]);
            std::printf("\n");
        } else if (cmd == "freepages") {
            std::printf("free %d\n", (int)st.free_list.size());
        } else if (cmd == "multi") {
            long long target = 0;
            int n = 0;
            in >> target >> n;
            std::vector<int32_t> ids(n > 0 ? n : 0), nq(n > 0 ? n : 0);
            for (int i = 0; i < n; i++) in >> ids[i] >> nq[i];
            kv4::MqPlan plan;
            kv4::Status s = st.plan_multi(n, ids.data(), nq.data(), target, &plan, nullptr);
            std::printf("status %d tasks %lld groups %lld spc %d n8 %d\n", (int)s, (long long)plan.tasks,
                        (long long)plan.groups, plan.spc, kv4::mq_int8_steps(st.cfg));
            if (s == kv4::OK)
                for (const auto& e : plan.entries)
                    std::printf("entry %d %d %d %d %d %d %d %d\n", e.seq, e.len, e.nq, e.qrow0, e.task0, e.grp0, e.steps,
                                e.nch);
            std::printf("end\n");
        } else if (cmd == "decode") {
            int n = 0;
            in >> n;
            std::vector<int32_t> ids(n > 0 ? n : 0);
            for (int i = 0; i < n; i++) in >> ids[i];
            std::vector<kv4::DecodeUnit> units;
            int64_t total = 0;
            kv4::Status s = st.plan_decode(n, ids.data(), &units, &total, nullptr);
            std::printf("status %d total %lld start %d\n", (int)s, (long long)total, kv4::kUnitStartSteps);
            if (s == kv4::OK)
                for (const auto& u : units)
                    std::printf("unit %d %d %d %d %lld\n", u.seq, u.len, u.entry, u.head, (long long)u.step_begin);
            std::printf("end\n");
        } else if (cmd == "sizes") {
            kv4::Sizes z = kv4::buffer_sizes(st.cfg);
            std::printf("sizes %zu %zu %zu %zu %zu %d\n", z.page_pool, z.int8_pool, z.block_table, z.page_block,
                        z.int8_tile, z.int8_tiles);
        } else {
            std::printf("status -2\n");
        }
        std::fflush(stdout);
    }
    return 0;
}
