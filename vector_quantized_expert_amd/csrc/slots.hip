// slots.hip -- the HBM expert-slot cache for code banks kept in pinned host
// memory.
//
// [FR] "Architecture de streaming depuis le disque": an expert's gate, up and
// down are one contiguous record, so loading an expert is one read.  [FR]
// "Lecture anticipée et prédiction du routeur": reads are issued as soon as
// the router has decided, and consumed as they land; overlapping them does not
// change any result.  [FR] "Budget RAM et fenêtre de performance étroite":
// a bounded cache of experts, refusing a budget below one token's working set.
// Here the "disk" is a pinned host record bank (payloads in the library's
// internal layout, each followed by its trailer: written at open from
// canonical codes, or written earlier by rvq_moe_write_bank and borrowed) and
// the cache is `S` HBM slots of one record each:
//   - a call's experts are made resident by hipMemcpyAsync on the library's
//     copy stream, one record per copy, into least-recently-used slots;
//   - [FR] "Architecture de streaming depuis le disque": every record read is
//     checked.  After its copy (`copied` event) the check stream verifies the
//     slot's trailer (magic, expert id, offset range) and, on request, the
//     payload's CRC-32 as it landed in HBM, then records `filled`; a failure
//     is flagged on the device and reported by the next sync;
//   - per slot, `filled` (copy and checks done; the compute stream waits on
//     it) and `released` (the last kernel reading the slot is done; the next
//     copy into the slot waits on it) events order the streams;
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
                      const uint8_t *bank, bool verify, hipStream_t s) {
    c.S = S;
    c.E = g.E;
    c.ex = record_expect(g);
    c.rec = c.ex.stride;
    c.verify = verify;
    hipError_t e;
    if ((e = hipMalloc(&c.slots, (size_t)(S * c.rec))) != hipSuccess) return e;
    if ((e = hipMalloc(&c.rec_err, 2 * sizeof(int))) != hipSuccess) return e;
    if ((e = hipMemsetAsync(c.rec_err, 0, 2 * sizeof(int), s)) != hipSuccess) return e;
    if (verify) {
        if ((e = crc_plan_init(c.plan, c.ex.payload)) != hipSuccess) return e;
        if ((e = hipMalloc(&c.part, sizeof(uint32_t) * kCrcMaxSpans)) != hipSuccess) return e;
    }
    if ((e = hipHostMalloc(reinterpret_cast<void **>(&c.ids_host), sizeof(int32_t) * (size_t)max_pairs,
                           hipHostMallocDefault)) != hipSuccess)
        return e;
    if ((e = hipMalloc(&c.tab_dev, sizeof(uint8_t *) * (size_t)g.E)) != hipSuccess) return e;
    if ((e = hipMemsetAsync(c.tab_dev, 0, sizeof(uint8_t *) * (size_t)g.E, s)) != hipSuccess) return e;
    if ((e = hipStreamCreateWithFlags(&c.copy, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipStreamCreateWithFlags(&c.check, hipStreamNonBlocking)) != hipSuccess) return e;
    c.copied.assign(S, nullptr);
    c.filled.assign(S, nullptr);
    c.released.assign(S, nullptr);
    for (int i = 0; i < S; i++) {
        if ((e = hipEventCreateWithFlags(&c.copied[i], hipEventDisableTiming)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&c.filled[i], hipEventDisableTiming)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&c.released[i], hipEventDisableTiming)) != hipSuccess) return e;
    }
    c.slot_of.assign(g.E, -1);
    c.expert_in.assign(S, -1);
    c.last_use.assign(S, 0);
    c.prefetched.assign(S, 0);
    c.mark.assign(g.E, 0);
    c.clock = 0;
    if (bank) {
        c.bank = bank;
        return hipStreamSynchronize(s);
    }
    if ((e = hipHostMalloc(reinterpret_cast<void **>(&c.own_bank), (size_t)(g.E * c.rec), hipHostMallocDefault)) !=
        hipSuccess) {
        c.own_bank = nullptr;
        return e;
    }
    c.bank = c.own_bank;
    return write_bank(g, canon_host, true, c.own_bank, s);
}

void slots_close(SlotCache &c) {
    if (c.copy) (void)hipStreamSynchronize(c.copy);
    if (c.check) (void)hipStreamSynchronize(c.check);
    for (hipEvent_t ev : c.copied)
        if (ev) (void)hipEventDestroy(ev);
    for (hipEvent_t ev : c.filled)
        if (ev) (void)hipEventDestroy(ev);
    for (hipEvent_t ev : c.released)
        if (ev) (void)hipEventDestroy(ev);
    if (c.copy) (void)hipStreamDestroy(c.copy);
    if (c.check) (void)hipStreamDestroy(c.check);
    (void)hipFree(c.slots);
    (void)hipFree(c.tab_dev);
    (void)hipFree(c.rec_err);
    (void)hipFree(c.part);
    crc_plan_free(c.plan);
    if (c.own_bank) (void)hipHostFree(c.own_bank);
    if (c.ids_host) (void)hipHostFree(c.ids_host);
    c = SlotCache{};
}

// Copy expert e's record into `slot` and check it there; `filled[slot]` is
// recorded once the checks are done.
static hipError_t fill_slot(SlotCache &c, int slot, int e) {
    uint8_t *dst = c.slots + (int64_t)slot * c.rec;
    c.h2d_bytes += (uint64_t)c.rec;
    hipError_t err = hipStreamWaitEvent(c.copy, c.released[slot], 0);
    if (err == hipSuccess) err = hipStreamWaitEvent(c.copy, c.filled[slot], 0);  // the last checks stopped reading
    if (err == hipSuccess)
        err = hipMemcpyAsync(dst, c.bank + (int64_t)e * c.rec, (size_t)c.rec, hipMemcpyHostToDevice, c.copy);
    if (err == hipSuccess) err = hipEventRecord(c.copied[slot], c.copy);
    if (err == hipSuccess) err = hipStreamWaitEvent(c.check, c.copied[slot], 0);
    if (err == hipSuccess && c.verify) err = launch_crc_spans(c.plan, dst, c.part, c.check);
    if (err == hipSuccess)
        err = launch_check_record(c.verify ? &c.plan : nullptr, dst, c.ex, e, c.verify ? c.part : nullptr, c.rec_err,
                                  c.check);
    if (err == hipSuccess) err = hipEventRecord(c.filled[slot], c.check);
    if (err == hipSuccess) {
        c.records_checked++;
        if (c.verify) c.records_verified++;
    }
    return err;
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
        hipError_t err = fill_slot(c, victim, e);
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
        const hipError_t err = fill_slot(c, victim, e);
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
