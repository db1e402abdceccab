// epoch_model.hip -- host model of the call-epoch protocol of
// linear_recurrence_scan_linrec_amd/csrc/call_epoch.hpp.  Test infrastructure:
// built for the host only (no device code runs) by tests/test_epoch_model.py.
//
// Simulated workgroups run the header's own functions on host memory.  Every
// atomic step (load, add, store) waits for a scheduler that grants one step
// at a time, to a workgroup drawn at random among those waiting, so each run
// is one random interleaving of the steps of all resident workgroups.  A
// workgroup has `waves` waves that read the epoch; wave 0 also counts.
//
//   ordered    the kernels' order: the other waves' reads may come before or
//              after wave 0's count, but all before its count_done (a barrier)
//   unordered  count_done straight after the count, the other waves' reads
//              drawn anywhere after the count: an order the kernels must not
//              use, run to show that the model catches a workgroup reading
//              the next call's epoch
//
// For each call it checks that every read returned the call's epoch, and that
// after the call every count and `finished` are zero and every line holds the
// next epoch.  It also checks the slot arithmetic for every grid size from 1
// to 20000: each workgroup lies in its line's contiguous range, the members
// add up to the grid, and the lines with members number slot_lines.
//
// usage: epoch_model <ordered|unordered> <seed> <waves> <resident> <calls> <start_epoch> <grid>...
// Prints one line per call and "ok", or the first violation; exits 0 if every
// check held, 1 otherwise.
#include "call_epoch.hpp"

#include <algorithm>
#include <condition_variable>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <random>
#include <thread>
#include <vector>

using namespace linrec;

namespace {

std::mutex g_m;
std::condition_variable g_cv;                       // the scheduler's
std::vector<std::condition_variable>* g_worker_cv;  // one per worker
std::vector<int> g_waiting;   // workers waiting for a grant
int g_granted = -1;           // worker allowed to take its next step
int g_live = 0;               // workers not finished
thread_local int t_worker = -1;

// One atomic step: wait for the grant, perform it, hand the baton back.
template <class F>
auto step(F f) {
    std::unique_lock<std::mutex> lock(g_m);
    g_waiting.push_back(t_worker);
    g_cv.notify_one();
    (*g_worker_cv)[t_worker].wait(lock, [] { return g_granted == t_worker; });
    auto r = f();
    g_granted = -1;
    g_cv.notify_one();
    return r;
}

struct HostAtomics {
    static uint32_t load(uint32_t* p) {
        return step([p] { return __atomic_load_n(p, __ATOMIC_SEQ_CST); });
    }
    static uint32_t add(uint32_t* p, uint32_t v) {
        return step([p, v] { return __atomic_fetch_add(p, v, __ATOMIC_SEQ_CST); });
    }
    static void store(uint32_t* p, uint32_t v) {
        step([p, v] {
            __atomic_store_n(p, v, __ATOMIC_SEQ_CST);
            return 0;
        });
    }
};

// A read of the epoch that is not part of the header's protocol (the other
// waves' reads use epoch_of_call too; this wrapper only names them).
uint32_t wave_read(const EpochWords& w, int64_t group, int64_t groups) {
    return epoch_of_call<HostAtomics>(w, group, groups);
}

struct Call {
    EpochWords words;
    int64_t groups;
    int waves;
    bool ordered;
    uint64_t seed;                   // workgroup k draws from seed and k
    int64_t next_group = 0;          // dispatch in workgroup order (under g_m)
    std::vector<uint32_t> reads;     // every epoch read of the call (under g_m)
};

void run_workgroup(Call& c, int64_t k) {
    std::mt19937_64 rng(c.seed ^ (static_cast<uint64_t>(k) * 0x9e3779b97f4a7c15ull));
    std::vector<uint32_t> got;
    const uint32_t e = epoch_of_call<HostAtomics>(c.words, k, c.groups);
    got.push_back(e);
    // the other waves' reads: some before wave 0's count, the rest after
    const int others = c.waves - 1;
    const int early = others > 0 ? static_cast<int>(rng() % (others + 1)) : 0;
    for (int i = 0; i < early; ++i) got.push_back(wave_read(c.words, k, c.groups));
    const uint32_t before = epoch_count_in<HostAtomics>(c.words, k, c.groups, e);
    bool last = false;
    if (c.ordered) {
        for (int i = early; i < others; ++i) got.push_back(wave_read(c.words, k, c.groups));
        last = epoch_count_done<HostAtomics>(c.words, k, c.groups, before);   // after the barrier
        if (last) epoch_advance<HostAtomics>(c.words, e, 0, 1);
    } else {
        last = epoch_count_done<HostAtomics>(c.words, k, c.groups, before);
        // the late waves' reads land anywhere among wave 0's remaining steps
        const int steps = last ? kDoneSlots : 0;
        std::vector<int> at(others - early);
        for (int& a : at) a = steps > 0 ? static_cast<int>(rng() % (steps + 1)) : 0;
        for (int s = 0; s <= steps; ++s) {
            for (int a : at)
                if (a == s) got.push_back(wave_read(c.words, k, c.groups));
            if (s < steps) HostAtomics::store(c.words.lines + s * kLineWords + 1, next_epoch(e));
        }
    }
    std::lock_guard<std::mutex> lock(g_m);
    c.reads.insert(c.reads.end(), got.begin(), got.end());
}

// Worker `id` starts with workgroup id, then takes the next one in order.
// Only the worker holding the grant runs between two steps, so with the
// waiting list sorted before each draw a run depends on the seed alone.
void worker(int id, Call& c) {
    t_worker = id;
    int64_t k = id;
    for (;;) {
        run_workgroup(c, k);
        std::lock_guard<std::mutex> lock(g_m);
        k = c.next_group < c.groups ? c.next_group++ : -1;
        if (k < 0) {
            --g_live;
            g_cv.notify_one();
            return;
        }
    }
}

// Runs one call with `resident` workers and a random order of steps.
void run_call(Call& c, int resident, std::mt19937_64& rng) {
    const int workers = static_cast<int>(std::min<int64_t>(resident, c.groups));
    std::vector<std::condition_variable> cvs(static_cast<size_t>(workers));
    g_worker_cv = &cvs;
    g_live = workers;
    g_granted = -1;
    g_waiting.clear();
    c.seed = rng();
    c.next_group = workers;
    std::vector<std::thread> threads;
    for (int i = 0; i < workers; ++i) threads.emplace_back(worker, i, std::ref(c));
    std::unique_lock<std::mutex> lock(g_m);
    for (;;) {
        // quiescent: every live worker waits for a grant (or none is live)
        g_cv.wait(lock, [] { return g_granted == -1 && static_cast<int>(g_waiting.size()) == g_live; });
        if (g_live == 0) break;
        std::sort(g_waiting.begin(), g_waiting.end());
        const size_t pick = rng() % g_waiting.size();
        g_granted = g_waiting[pick];
        g_waiting.erase(g_waiting.begin() + static_cast<std::ptrdiff_t>(pick));
        (*g_worker_cv)[g_granted].notify_one();
    }
    lock.unlock();
    for (std::thread& t : threads) t.join();
}

bool check_arithmetic() {
    for (int64_t groups = 1; groups <= 20000; ++groups) {
        // lines with members: exactly slot_lines of them (count_done counts
        // filled lines up to that number), with every workgroup counted once
        uint32_t used = 0;
        int64_t total = 0;
        for (int64_t s = 0; s < kDoneSlots; ++s) {
            const uint32_t m = slot_members(s, groups);
            used += m > 0 ? 1u : 0u;
            total += m;
        }
        if (used != slot_lines(groups) || total != groups) {
            std::printf("grid %lld: %u lines with members (want %u), %lld members\n", (long long)groups, used,
                        slot_lines(groups), (long long)total);
            return false;
        }
        for (int64_t k = 0; k < groups; ++k) {
            const int64_t s = slot_of(k, groups);
            if (s < 0 || s >= kDoneSlots || k < slot_begin(s, groups) || k >= slot_begin(s + 1, groups)) {
                std::printf("grid %lld: workgroup %lld outside its line %lld\n", (long long)groups, (long long)k,
                            (long long)s);
                return false;
            }
        }
    }
    return true;
}

}  // namespace

int main(int argc, char** argv) {
    if (argc < 8) {
        std::fprintf(stderr, "usage: %s <ordered|unordered> <seed> <waves> <resident> <calls> <start_epoch> <grid>...\n",
                     argv[0]);
        return 2;
    }
    const bool ordered = std::strcmp(argv[1], "ordered") == 0;
    std::mt19937_64 rng(std::strtoull(argv[2], nullptr, 10));
    const int waves = std::atoi(argv[3]);
    const int resident = std::atoi(argv[4]);
    const int calls = std::atoi(argv[5]);
    const uint32_t start = static_cast<uint32_t>(std::strtoul(argv[6], nullptr, 10)) & kEpochMask;
    if (!check_arithmetic()) return 1;

    std::vector<uint32_t> mem(kDoneSlots * kLineWords + kLineWords, 0u);
    EpochWords words{mem.data(), mem.data() + kDoneSlots * kLineWords};
    for (int s = 0; s < kDoneSlots; ++s) mem[s * kLineWords + 1] = start;
    uint32_t epoch = start;
    for (int a = 7; a < argc; ++a) {
        const int64_t groups = std::atoll(argv[a]);
        for (int n = 0; n < calls; ++n) {
            Call c{words, groups, waves, ordered, 0};
            run_call(c, resident, rng);
            for (uint32_t r : c.reads)
                if (r != epoch) {
                    std::printf("grid %lld call %d: a wave read epoch %u during the call of epoch %u\n",
                                (long long)groups, n, r, epoch);
                    return 1;
                }
            const uint32_t called = epoch;
            epoch = next_epoch(epoch);
            for (int s = 0; s < kDoneSlots; ++s)
                if (mem[s * kLineWords] != 0u || mem[s * kLineWords + 1] != epoch) {
                    std::printf("grid %lld call %d: line %d holds count %u epoch %u after the call (want 0, %u)\n",
                                (long long)groups, n, s, mem[s * kLineWords], mem[s * kLineWords + 1], epoch);
                    return 1;
                }
            if (*words.finished != 0u) {
                std::printf("grid %lld call %d: finished = %u after the call\n", (long long)groups, n, *words.finished);
                return 1;
            }
            std::printf("grid %lld call %d: %zu reads of epoch %u\n", (long long)groups, n, c.reads.size(), called);
        }
    }
    std::printf("ok\n");
    return 0;
}
