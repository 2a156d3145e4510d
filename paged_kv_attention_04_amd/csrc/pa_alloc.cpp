// Reference-counted block allocator with stream-deferred release (host side).
//
// The pages give the rules this follows (AI-infra book ch. 8 "Inference optimisation",
// section 8.3.2 and figs. 8-14 / 8-15): a physical block carries a reference count, one
// per block table that points at it; a shared prefix is one set of blocks whose counts
// exceed one; a request about to write into a block it shares first gets a private copy
// (copy-on-write); and a block goes back to the free pool only when its last reference
// is gone *and* the device has finished the work that reads it.  The last condition is
// met here with a HIP event recorded on the caller's stream at release time: the blocks
// wait in a pending list until that event has completed.
//
// Host memory only; not thread-safe (one allocator per host thread, or an outside lock).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <deque>
#include <new>
#include <vector>

#include "pa.h"

namespace {

enum BlockState : uint8_t { kFree = 0, kInUse = 1, kPending = 2 };

struct Pending {
    hipEvent_t event;
    std::vector<int32_t> blocks;
};

}  // namespace

struct pa_block_allocator {
    int32_t num_blocks = 0;
    std::vector<int32_t> refcount;
    std::vector<uint8_t> state;
    std::vector<int32_t> free_list;   // a stack: the most recently freed block is reused first
    std::deque<Pending> pending;      // deferred releases, oldest first
    std::vector<hipEvent_t> spare;    // completed events, kept for reuse

    // Move the blocks of every completed deferred release to the free list.
    void reclaim()
    {
        for (auto it = pending.begin(); it != pending.end();) {
            if (hipEventQuery(it->event) != hipSuccess) {   // not complete yet (or an error: keep waiting)
                ++it;
                continue;
            }
            for (const int32_t b : it->blocks) {
                state[b] = kFree;
                free_list.push_back(b);
            }
            spare.push_back(it->event);
            it = pending.erase(it);
        }
    }
};

namespace {

bool in_use(const pa_block_allocator* a, int32_t b)
{
    return b >= 0 && b < a->num_blocks && a->state[b] == kInUse;
}

}  // namespace

extern "C" pa_status pa_allocator_create(int32_t num_blocks, pa_block_allocator** out)
{
    if (!out)
        return PA_ERR_NULL;
    *out = nullptr;
    if (num_blocks < 1)
        return PA_ERR_SHAPE;
    pa_block_allocator* a = new (std::nothrow) pa_block_allocator;
    if (!a)
        return PA_ERR_NO_BLOCKS;
    a->num_blocks = num_blocks;
    a->refcount.assign(num_blocks, 0);
    a->state.assign(num_blocks, kFree);
    a->free_list.reserve(num_blocks);
    for (int32_t b = num_blocks - 1; b >= 0; --b)   // block 0 is handed out first
        a->free_list.push_back(b);
    *out = a;
    return PA_OK;
}

extern "C" void pa_allocator_destroy(pa_block_allocator* a)
{
    if (!a)
        return;
    for (Pending& p : a->pending)
        (void)hipEventDestroy(p.event);
    for (hipEvent_t e : a->spare)
        (void)hipEventDestroy(e);
    delete a;
}

extern "C" pa_status pa_allocator_alloc(pa_block_allocator* a, int32_t n, int32_t* blocks_out)
{
    if (!a || (n > 0 && !blocks_out))
        return PA_ERR_NULL;
    if (n < 0)
        return PA_ERR_SHAPE;
    if ((int64_t)a->free_list.size() < n)
        a->reclaim();
    if ((int64_t)a->free_list.size() < n)
        return PA_ERR_NO_BLOCKS;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t b = a->free_list.back();
        a->free_list.pop_back();
        a->state[b] = kInUse;
        a->refcount[b] = 1;
        blocks_out[i] = b;
    }
    return PA_OK;
}

extern "C" pa_status pa_allocator_retain(pa_block_allocator* a, const int32_t* blocks, int32_t n)
{
    if (!a || (n > 0 && !blocks))
        return PA_ERR_NULL;
    if (n < 0)
        return PA_ERR_SHAPE;
    for (int32_t i = 0; i < n; ++i)
        if (!in_use(a, blocks[i]))
            return PA_ERR_RANGE;
    for (int32_t i = 0; i < n; ++i)
        ++a->refcount[blocks[i]];
    return PA_OK;
}

extern "C" pa_status pa_allocator_release(pa_block_allocator* a, const int32_t* blocks, int32_t n, void* stream,
                                          int32_t deferred)
{
    if (!a || (n > 0 && !blocks))
        return PA_ERR_NULL;
    if (n < 0)
        return PA_ERR_SHAPE;
    // every block must hold at least as many references as the list drops
    std::vector<int32_t> drop;
    drop.reserve(n);
    for (int32_t i = 0; i < n; ++i) {
        if (!in_use(a, blocks[i]))
            return PA_ERR_RANGE;
        drop.push_back(blocks[i]);
    }
    std::sort(drop.begin(), drop.end());
    for (size_t i = 0; i < drop.size();) {
        size_t j = i;
        while (j < drop.size() && drop[j] == drop[i])
            ++j;
        if ((int64_t)(j - i) > a->refcount[drop[i]])
            return PA_ERR_RANGE;
        i = j;
    }
    hipEvent_t ev = nullptr;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (deferred) {
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cap) != hipSuccess)
            return PA_ERR_HIP;
        if (cap != hipStreamCaptureStatusNone)
            return PA_ERR_UNSUPPORTED;      // an event recorded during capture completes only on replay
        if (!a->spare.empty()) {
            ev = a->spare.back();
            a->spare.pop_back();
        } else if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
            return PA_ERR_HIP;
        }
        if (hipEventRecord(ev, st) != hipSuccess) {
            a->spare.push_back(ev);
            return PA_ERR_HIP;
        }
    }
    Pending p;
    p.event = ev;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t b = blocks[i];
        if (--a->refcount[b] > 0)
            continue;
        if (deferred) {
            a->state[b] = kPending;
            p.blocks.push_back(b);
        } else {
            a->state[b] = kFree;
            a->free_list.push_back(b);
        }
    }
    if (deferred) {
        if (p.blocks.empty())
            a->spare.push_back(ev);
        else
            a->pending.push_back(std::move(p));
    }
    return PA_OK;
}

extern "C" pa_status pa_allocator_cow(pa_block_allocator* a, int32_t block, int32_t* block_out)
{
    if (!a || !block_out)
        return PA_ERR_NULL;
    if (!in_use(a, block))
        return PA_ERR_RANGE;
    if (a->refcount[block] == 1) {
        *block_out = block;          // not shared: write in place
        return PA_OK;
    }
    int32_t fresh = -1;
    const pa_status st = pa_allocator_alloc(a, 1, &fresh);
    if (st != PA_OK)
        return st;
    --a->refcount[block];            // still referenced by the others
    *block_out = fresh;
    return PA_OK;
}

extern "C" pa_status pa_allocator_refcount(const pa_block_allocator* a, int32_t block, int32_t* count)
{
    if (!a || !count)
        return PA_ERR_NULL;
    if (block < 0 || block >= a->num_blocks)
        return PA_ERR_RANGE;
    *count = a->refcount[block];
    return PA_OK;
}

extern "C" pa_status pa_allocator_num_free(pa_block_allocator* a, int32_t* free_blocks, int32_t* pending_blocks)
{
    if (!a)
        return PA_ERR_NULL;
    a->reclaim();
    if (free_blocks)
        *free_blocks = (int32_t)a->free_list.size();
    if (pending_blocks) {
        int64_t n = 0;
        for (const Pending& p : a->pending)
            n += (int64_t)p.blocks.size();
        *pending_blocks = (int32_t)n;
    }
    return PA_OK;
}

extern "C" pa_status pa_allocator_sync(pa_block_allocator* a)
{
    if (!a)
        return PA_ERR_NULL;
    for (Pending& p : a->pending)
        if (hipEventSynchronize(p.event) != hipSuccess)
            return PA_ERR_HIP;
    a->reclaim();
    return PA_OK;
}
