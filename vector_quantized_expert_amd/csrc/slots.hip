// slots.hip -- the HBM expert-slot cache for code banks kept in pinned host
// memory.
//
// [FR] "Architecture de streaming depuis le disque": an expert's gate, up and
// down are one contiguous record, so loading an expert is one read.  [FR]
// "Lecture anticipée et prédiction du routeur": reads are issued as soon as
// the router has decided, and consumed as they land; overlapping them does not
// change any result.  [FR] "Budget RAM et fenêtre de performance étroite":
// a bounded cache of experts, refusing a budget below one token's working set.
// Here the "disk" is a pinned host bank (in the library's internal layout,
// written once at open) and the cache is `S` HBM slots of one record each:
//   - a call's experts are made resident by hipMemcpyAsync on the library's
//     copy stream, one record per copy, into least-recently-used slots;
//   - per slot, `filled` (copy done; the compute stream waits on it) and
//     `released` (the last kernel reading the slot is done; the next copy
//     into the slot waits on it) events order the two streams;
//   - a device table [E] of record pointers tells the kernels where each
//     expert's codes are.  It is written on the compute stream by a small
//     kernel whose arguments carry the call's (expert, slot) pairs: launch
//     arguments are captured at enqueue time, so the host may run ahead.
// All bookkeeping is on the host: the caller's call synchronises once to read
// the expert ids, then everything else is enqueued.
//
// Prefetch ([FR] "Lecture anticipée et prédiction du routeur": the next
// layer's router, run early, predicts its experts and their reads start
// before they are needed) fills slots the same way without a kernel waiting;
// a later acquire that finds such a slot waits on its `filled` event.
#include <string.h>

#include "internal.hpp"
#include "slots.hpp"

namespace rvq {

constexpr int kSetPairs = 128;
struct SlotPairs {
    uint8_t *base;
    int64_t rec;
    int n;
    int expert[kSetPairs];
    int slot[kSetPairs];
};

__global__ __launch_bounds__(kSetPairs) void k_set_slots(const uint8_t **tab, SlotPairs p) {
    if ((int)threadIdx.x < p.n) tab[p.expert[threadIdx.x]] = p.base + (int64_t)p.slot[threadIdx.x] * p.rec;
}

hipError_t slots_open(SlotCache &c, const Geometry &g, int S, int max_pairs, const uint8_t *canon_host,
                      hipStream_t s) {
    c.S = S;
    c.E = g.E;
    c.rec = g.rec_int;
    hipError_t e;
    if ((e = hipMalloc(&c.slots, (size_t)(S * c.rec))) != hipSuccess) return e;
    if ((e = hipHostMalloc(reinterpret_cast<void **>(&c.bank), (size_t)(g.E * c.rec), hipHostMallocDefault)) !=
        hipSuccess)
        return e;
    if ((e = hipHostMalloc(reinterpret_cast<void **>(&c.ids_host), sizeof(int32_t) * (size_t)max_pairs,
                           hipHostMallocDefault)) != hipSuccess)
        return e;
    if ((e = hipMalloc(&c.tab_dev, sizeof(uint8_t *) * (size_t)g.E)) != hipSuccess) return e;
    if ((e = hipMemsetAsync(c.tab_dev, 0, sizeof(uint8_t *) * (size_t)g.E, s)) != hipSuccess) return e;
    if ((e = hipStreamCreateWithFlags(&c.copy, hipStreamNonBlocking)) != hipSuccess) return e;
    c.filled.assign(S, nullptr);
    c.released.assign(S, nullptr);
    for (int i = 0; i < S; i++) {
        if ((e = hipEventCreateWithFlags(&c.filled[i], hipEventDisableTiming)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&c.released[i], hipEventDisableTiming)) != hipSuccess) return e;
    }
    c.slot_of.assign(g.E, -1);
    c.expert_in.assign(S, -1);
    c.last_use.assign(S, 0);
    c.prefetched.assign(S, 0);
    c.mark.assign(g.E, 0);
    c.clock = 0;
    // the bank in the internal layout: canonical records go through the GPU
    // (upload, repack, download) a few experts at a time
    const int B = g.E < 8 ? g.E : 8;
    uint8_t *canon = nullptr, *internal = nullptr;
    if ((e = hipMalloc(&canon, (size_t)(B * g.rec_canon))) != hipSuccess) return e;
    if ((e = hipMalloc(&internal, (size_t)(B * c.rec))) != hipSuccess) {
        (void)hipFree(canon);
        return e;
    }
    for (int e0 = 0; e0 < g.E && e == hipSuccess; e0 += B) {
        const int n = g.E - e0 < B ? g.E - e0 : B;
        e = hipMemcpyAsync(canon, canon_host + (int64_t)e0 * g.rec_canon, (size_t)(n * g.rec_canon),
                           hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = launch_repack(g, canon, internal, n, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync(c.bank + (int64_t)e0 * c.rec, internal, (size_t)(n * c.rec), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);  // the staging buffers are reused
    }
    (void)hipFree(canon);
    (void)hipFree(internal);
    return e;
}

void slots_close(SlotCache &c) {
    if (c.copy) (void)hipStreamSynchronize(c.copy);
    for (hipEvent_t ev : c.filled)
        if (ev) (void)hipEventDestroy(ev);
    for (hipEvent_t ev : c.released)
        if (ev) (void)hipEventDestroy(ev);
    if (c.copy) (void)hipStreamDestroy(c.copy);
    (void)hipFree(c.slots);
    (void)hipFree(c.tab_dev);
    if (c.bank) (void)hipHostFree(c.bank);
    if (c.ids_host) (void)hipHostFree(c.ids_host);
    c = SlotCache{};
}

hipError_t slots_acquire(SlotCache &c, const int *experts, int n, hipStream_t compute, std::vector<int> &used) {
    used.clear();
    if (n > c.S) return hipErrorInvalidValue;
    const uint64_t now = ++c.clock;
    // hits first, so that their slots are protected from this call's misses
    for (int i = 0; i < n; i++) {
        const int e = experts[i];
        const int sl = c.slot_of[e];
        if (sl >= 0 && c.last_use[sl] != now) {
            c.last_use[sl] = now;
            used.push_back(sl);
            c.hits++;
            if (c.prefetched[sl]) {  // its copy may still be in flight
                c.prefetched[sl] = 0;
                c.prefetch_hits++;
            }
            const hipError_t err = hipStreamWaitEvent(compute, c.filled[sl], 0);
            if (err != hipSuccess) return err;
        }
    }
    for (int i = 0; i < n; i++) {
        const int e = experts[i];
        if (c.slot_of[e] >= 0) continue;
        int victim = -1;
        for (int sl = 0; sl < c.S; sl++)
            if (c.last_use[sl] != now && (victim < 0 || c.last_use[sl] < c.last_use[victim])) victim = sl;
        if (victim < 0) return hipErrorInvalidValue;  // n <= S makes this unreachable
        if (c.expert_in[victim] >= 0) c.slot_of[c.expert_in[victim]] = -1;
        c.expert_in[victim] = e;
        c.slot_of[e] = victim;
        c.last_use[victim] = now;
        c.prefetched[victim] = 0;
        used.push_back(victim);
        c.misses++;
        c.h2d_bytes += (uint64_t)c.rec;
        hipError_t err = hipStreamWaitEvent(c.copy, c.released[victim], 0);
        if (err == hipSuccess)
            err = hipMemcpyAsync(c.slots + (int64_t)victim * c.rec, c.bank + (int64_t)e * c.rec, (size_t)c.rec,
                                 hipMemcpyHostToDevice, c.copy);
        if (err == hipSuccess) err = hipEventRecord(c.filled[victim], c.copy);
        if (err == hipSuccess) err = hipStreamWaitEvent(compute, c.filled[victim], 0);
        if (err != hipSuccess) return err;
    }
    for (int i0 = 0; i0 < n; i0 += kSetPairs) {
        SlotPairs p;
        p.base = c.slots;
        p.rec = c.rec;
        p.n = n - i0 < kSetPairs ? n - i0 : kSetPairs;
        for (int i = 0; i < p.n; i++) {
            p.expert[i] = experts[i0 + i];
            p.slot[i] = c.slot_of[experts[i0 + i]];
        }
        hipLaunchKernelGGL(k_set_slots, dim3(1), dim3(kSetPairs), 0, compute, c.tab_dev, p);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

hipError_t slots_prefetch(SlotCache &c, const int *experts, int n) {
    const uint64_t now = ++c.clock;
    for (int i = 0; i < n; i++) {
        const int sl = c.slot_of[experts[i]];
        if (sl >= 0) c.last_use[sl] = now;
    }
    for (int i = 0; i < n; i++) {
        const int e = experts[i];
        if (c.slot_of[e] >= 0) continue;
        int victim = -1;
        for (int sl = 0; sl < c.S; sl++)
            if (c.last_use[sl] != now && (victim < 0 || c.last_use[sl] < c.last_use[victim])) victim = sl;
        if (victim < 0) break;  // every slot already holds one of this prefetch's experts
        if (c.expert_in[victim] >= 0) c.slot_of[c.expert_in[victim]] = -1;
        c.expert_in[victim] = e;
        c.slot_of[e] = victim;
        c.last_use[victim] = now;
        c.prefetched[victim] = 1;
        c.prefetch_fills++;
        c.h2d_bytes += (uint64_t)c.rec;
        hipError_t err = hipStreamWaitEvent(c.copy, c.released[victim], 0);
        if (err == hipSuccess)
            err = hipMemcpyAsync(c.slots + (int64_t)victim * c.rec, c.bank + (int64_t)e * c.rec, (size_t)c.rec,
                                 hipMemcpyHostToDevice, c.copy);
        if (err == hipSuccess) err = hipEventRecord(c.filled[victim], c.copy);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

hipError_t slots_release(SlotCache &c, const std::vector<int> &used, hipStream_t compute) {
    for (int sl : used) {
        const hipError_t e = hipEventRecord(c.released[sl], compute);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace rvq
