// Host-side checks of the library's CPU code under AddressSanitizer and
// UndefinedBehaviorSanitizer: the planner, the content validators and the block
// allocator.  The six HIP calls the allocator makes (events and capture status) are
// replaced here by a fake device on which recorded work completes only when the test
// says so, so that the allocator's deferred-release bookkeeping runs deterministically.
// Built with g++ by tests/test_host_sanitizers.py; no GPU and no HIP runtime involved.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "pa.h"

struct ihipEvent_t {
    bool done;
};
static std::vector<ihipEvent_t*> g_recorded;   // events whose work has not completed yet

extern "C" hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned)
{
    *e = new ihipEvent_t{true};
    return hipSuccess;
}
extern "C" hipError_t hipEventRecord(hipEvent_t e, hipStream_t)
{
    e->done = false;
    g_recorded.push_back(e);
    return hipSuccess;
}
extern "C" hipError_t hipEventQuery(hipEvent_t e) { return e->done ? hipSuccess : hipErrorNotReady; }
extern "C" hipError_t hipEventSynchronize(hipEvent_t e)
{
    e->done = true;
    return hipSuccess;
}
extern "C" hipError_t hipEventDestroy(hipEvent_t e)
{
    for (auto& r : g_recorded)
        if (r == e)
            r = nullptr;
    delete e;
    return hipSuccess;
}
extern "C" hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* s)
{
    *s = hipStreamCaptureStatusNone;
    return hipSuccess;
}
static void device_completes_all()
{
    for (auto* e : g_recorded)
        if (e)
            e->done = true;
    g_recorded.clear();
}

#define CHECK(c)                                                                      \
    do {                                                                              \
        if (!(c)) {                                                                   \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);      \
            std::exit(1);                                                             \
        }                                                                             \
    } while (0)

// Random operations against a model of the counts: a block is free, held (count > 0) or
// waiting for recorded device work; waiting blocks become free once that work completes.
static void allocator_walk(uint32_t seed)
{
    std::mt19937 rng(seed);
    const int32_t nb = 1 + (int32_t)(rng() % 64);
    pa_block_allocator* a = nullptr;
    CHECK(pa_allocator_create(nb, &a) == PA_OK);
    std::vector<int32_t> count(nb, 0);
    std::vector<std::vector<int32_t>> waiting_groups;   // blocks released behind one event each
    auto model_free = [&]() {
        int32_t f = 0;
        for (int32_t b = 0; b < nb; ++b) {
            bool waiting = false;
            for (auto& g : waiting_groups)
                for (int32_t x : g)
                    waiting |= x == b;
            f += count[b] == 0 && !waiting;
        }
        return f;
    };
    for (int step = 0; step < 400; ++step) {
        const uint32_t op = rng() % 7;
        if (op == 0) {                                    // alloc
            const int32_t n = (int32_t)(rng() % 5);
            std::vector<int32_t> out((size_t)n + 1, -1);
            const pa_status st = pa_allocator_alloc(a, n, out.data());
            if (n > model_free()) {              // blocks still waiting for device work are not reused
                CHECK(st == PA_ERR_NO_BLOCKS);
                continue;
            }
            CHECK(st == PA_OK);
            for (int32_t i = 0; i < n; ++i) {
                CHECK(out[i] >= 0 && out[i] < nb && count[out[i]] == 0);
                count[out[i]] = 1;
                for (auto& g : waiting_groups)
                    for (int32_t x : g)
                        CHECK(x != out[i]);
            }
        } else if (op == 1 || op == 2) {                  // release (deferred or not), maybe invalid
            std::vector<int32_t> ids;
            const int32_t n = 1 + (int32_t)(rng() % 3);
            for (int32_t i = 0; i < n; ++i)
                ids.push_back((int32_t)(rng() % (nb + 2)) - 1);
            std::map<int32_t, int32_t> drop;
            bool valid = true;
            for (int32_t x : ids) {
                valid &= x >= 0 && x < nb;
                if (x >= 0 && x < nb)
                    drop[x]++;
            }
            for (auto& kv : drop)
                valid &= kv.second <= count[kv.first];
            const bool deferred = op == 2;
            const pa_status st = pa_allocator_release(a, ids.data(), n, nullptr, deferred ? 1 : 0);
            CHECK(valid ? st == PA_OK : st == PA_ERR_RANGE);
            if (valid) {
                std::vector<int32_t> freed;
                for (auto& kv : drop)
                    if ((count[kv.first] -= kv.second) == 0)
                        freed.push_back(kv.first);
                if (deferred && !freed.empty())
                    waiting_groups.push_back(freed);
            }
        } else if (op == 3) {                             // retain
            const int32_t x = (int32_t)(rng() % (nb + 1)) - 1;
            const pa_status st = pa_allocator_retain(a, &x, 1);
            CHECK((x >= 0 && x < nb && count[x] > 0) ? st == PA_OK : st == PA_ERR_RANGE);
            if (st == PA_OK)
                count[x]++;
        } else if (op == 4) {                             // copy-on-write
            const int32_t x = (int32_t)(rng() % nb);
            int32_t out = -1;
            const pa_status st = pa_allocator_cow(a, x, &out);
            if (count[x] == 0) {
                CHECK(st == PA_ERR_RANGE);
            } else if (count[x] == 1) {
                CHECK(st == PA_OK && out == x);
            } else if (st == PA_OK) {
                CHECK(out != x && out >= 0 && out < nb && count[out] == 0);
                count[x]--;
                count[out] = 1;
            } else {
                CHECK(st == PA_ERR_NO_BLOCKS);
            }
        } else if (op == 5) {                             // the device finishes its work
            device_completes_all();
            waiting_groups.clear();
        } else {                                          // counts and free list agree with the model
            int32_t f = -1, w = -1;
            CHECK(pa_allocator_num_free(a, &f, &w) == PA_OK);
            int32_t model_w = 0;
            for (auto& g : waiting_groups)
                model_w += (int32_t)g.size();
            CHECK(f == model_free() && w == model_w);
            for (int32_t b = 0; b < nb; ++b) {
                int32_t c = -1;
                CHECK(pa_allocator_refcount(a, b, &c) == PA_OK && c == count[b]);
            }
        }
    }
    CHECK(pa_allocator_sync(a) == PA_OK);
    g_recorded.clear();
    pa_allocator_destroy(a);
}

// Random batches through the planner and the validators: every call returns a status, a
// successful plan describes the batch, and out-of-range content is reported.
static void planner_walk(uint32_t seed)
{
    std::mt19937 rng(seed);
    const int32_t hkv = 1 + (int32_t)(rng() % 8);
    const pa_geometry g{4 * hkv, hkv, 128, 16, 1 + (int32_t)(rng() % 4000), 0.0883883f};
    const int32_t R = (int32_t)(rng() % 200);
    std::vector<int32_t> qo(R), kv(R);
    int32_t mb = 1;
    for (int32_t r = 0; r < R; ++r) {
        qo[r] = rng() % 3 ? 1 : 1 + (int32_t)(rng() % 600);
        kv[r] = qo[r] + (int32_t)(rng() % 20000);
        mb = std::max(mb, (kv[r] + 15) / 16);
    }
    const int32_t shared = rng() % 2 ? (int32_t)(rng() % 100) : 0;
    std::vector<int32_t> bt((size_t)R * mb, -1);
    for (int32_t r = 0; r < R; ++r)
        for (int32_t b = 0; b < (kv[r] + 15) / 16; ++b)
            bt[(size_t)r * mb + b] = b < shared ? b : (int32_t)(rng() % (uint32_t)g.num_blocks);
    pa_plan_t plan;
    const int32_t split = rng() % 3 ? 0 : 1 + (int32_t)(rng() % 600);
    const int32_t psplit = rng() % 3 ? 0 : (int32_t)(rng() % 70);
    const pa_status st = pa_plan(&g, R, qo.data(), kv.data(), 1 + (int32_t)(rng() % 512), split, psplit, &plan);
    if (psplit > 64) {
        CHECK(st == PA_ERR_SHAPE);
        return;
    }
    if (st != PA_OK) {
        CHECK(st == PA_ERR_UNSUPPORTED);               // too many chunk rows or counters
        return;
    }
    int32_t nd = 0, np = 0;
    for (int32_t r = 0; r < R; ++r)
        (qo[r] == 1 ? nd : np)++;
    CHECK(plan.num_decode_rows == nd && plan.num_prefill_rows == np && plan.num_reqs == R);
    for (int32_t q8 = 0; q8 < 2; ++q8) {
        pa_plan_t p2 = plan;
        const pa_status s2 = (q8 ? pa_plan_shared_prefix_q8 : pa_plan_shared_prefix)(
            &g, qo.data(), kv.data(), bt.data(), mb, 256, 0, (int32_t)(rng() % 8), 0, &p2);
        CHECK(s2 == PA_OK || s2 == PA_ERR_UNSUPPORTED);
        if (s2 == PA_OK)
            for (int32_t i = 0; i < p2.num_prefix_groups; ++i)
                CHECK(p2.prefix_num_reqs[i] >= 2 && p2.prefix_num_reqs[i] <= PA_MAX_PREFIX_GROUP_REQS);
    }
    int32_t bad = -2;
    const pa_status v = pa_validate_batch(&g, R, qo.data(), kv.data(), bt.data(), mb, &bad);
    CHECK(v == PA_OK || v == PA_ERR_RANGE);
    std::vector<int32_t> slots(R);
    std::set<int32_t> seen;
    bool dup = false;
    for (int32_t r = 0; r < R; ++r) {
        slots[r] = (int32_t)(rng() % (uint32_t)(g.num_blocks * 16 + 8)) - 4;
        if (slots[r] >= 0 && slots[r] < g.num_blocks * 16)
            dup |= !seen.insert(slots[r]).second;
    }
    const pa_status va = pa_validate_append(&g, slots.data(), R, &bad);
    CHECK(va == PA_OK || va == PA_ERR_RANGE);
    if (va == PA_OK)
        CHECK(!dup);
}

int main()
{
    // null and negative arguments are reported, not dereferenced
    CHECK(pa_plan(nullptr, 0, nullptr, nullptr, 256, 0, 0, nullptr) == PA_ERR_NULL);
    CHECK(pa_allocator_create(0, nullptr) != PA_OK);
    CHECK(pa_validate_append(nullptr, nullptr, 1, nullptr) == PA_ERR_NULL);
    for (int s = 0; s < 300; ++s)
        allocator_walk(1000 + s);
    for (int s = 0; s < 300; ++s)
        planner_walk(5000 + s);
    std::printf("host checks ok\n");
    return 0;
}
