// slots.hpp -- HBM expert-slot cache state (host side); see slots.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "integrity.hpp"
#include "internal.hpp"

namespace rvq {

struct SlotCache {
    int S = 0;                         // slots
    int E = 0;
    int64_t rec = 0;                   // bank record stride (one slot): payload, fill, trailer page
    uint8_t *slots = nullptr;          // device [S][rec]
    const uint8_t *bank = nullptr;     // pinned host [E][rec] record bank (own_bank, or the caller's)
    uint8_t *own_bank = nullptr;       // the bank written at open from canonical codes, or null
    RecordExpect ex{};                 // what every record's trailer must say
    bool verify = false;               // also check each landed payload's CRC-32
    CrcPlan plan;                      // its device plan (verify only)
    uint32_t *part = nullptr;          // device [kCrcMaxSpans] CRC partials (check stream order)
    int *rec_err = nullptr;            // device [2]: failed-check flags, highest failing expert + 1
    const uint8_t **tab_dev = nullptr; // device [E]: record pointer of each resident expert
    int32_t *ids_host = nullptr;       // pinned [max_tokens * k]: the call's ids, read back once per call
    hipStream_t copy = nullptr;        // the library's copy stream (default priority)
    hipStream_t check = nullptr;       // the record checks' stream (default priority)
    std::vector<hipEvent_t> copied;    // [S] copy into the slot done (the checks wait on it)
    std::vector<hipEvent_t> filled;    // [S] copy and checks done
    std::vector<hipEvent_t> released;  // [S] last kernel reading the slot done
    std::vector<int> slot_of;          // [E] slot of a resident expert, or -1
    std::vector<int> expert_in;        // [S] expert in a slot, or -1
    std::vector<uint64_t> last_use;    // [S] acquire clock of the last use
    std::vector<uint8_t> prefetched;   // [S] filled by a prefetch and not yet used by a call
    std::vector<uint32_t> mark;        // [E] scratch for set building
    uint64_t clock = 0;
    uint64_t hits = 0, misses = 0, h2d_bytes = 0, syncs = 0;
    uint64_t prefetch_fills = 0, prefetch_hits = 0;
    uint64_t records_checked = 0, records_verified = 0;
};

// Allocate the slots; borrow the caller's record bank (`bank`, already
// checked), or write the handle's own from pinned canonical codes
// (`canon_host`).  Synchronises `s`.
hipError_t slots_open(SlotCache &c, const Geometry &g, int S, int max_pairs, const uint8_t *canon_host,
                      const uint8_t *bank, bool verify, hipStream_t s);
void slots_close(SlotCache &c);
// Make experts[0 .. n) (distinct, n <= S) resident for kernels enqueued next on
// `compute`, and point their table entries at their slots; `used` gets the
// slots to release after those kernels.
hipError_t slots_acquire(SlotCache &c, const int *experts, int n, hipStream_t compute, std::vector<int> &used);
hipError_t slots_release(SlotCache &c, const std::vector<int> &used, hipStream_t compute);
// Start copies that make experts[0 .. n) (distinct) resident ahead of a later
// acquire: resident ones are refreshed, the others take least-recently-used
// slots (at most S experts in all).  Nothing waits for the copies until an
// acquire uses their slots.
hipError_t slots_prefetch(SlotCache &c, const int *experts, int n);

}  // namespace rvq
