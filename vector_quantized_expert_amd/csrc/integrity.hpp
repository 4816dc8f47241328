// integrity.hpp -- expert-record trailers and the CRC-32 of record payloads
// on the device (see integrity.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"
#include "rvq_moe.h"

namespace rvq {

constexpr int64_t kPage = 4096;
constexpr int kCrcMaxSpans = 1024;  // most workgroups one payload's CRC-32 takes

// Bank layout: record e occupies [e * stride, (e + 1) * stride).  Its payload
// (the internal record, rec_int bytes) comes first, then zero fill up to a
// 4 KiB boundary, then one 4 KiB trailer page that starts with an
// rvq_moe_record_trailer and is zero after it.  A slot holds one whole record.
inline int64_t bank_trailer_off(const Geometry &g) { return (g.rec_int + kPage - 1) / kPage * kPage; }
inline int64_t bank_stride(const Geometry &g) { return bank_trailer_off(g) + kPage; }

// What a record's trailer must say for expert e of a bank of this geometry.
struct RecordExpect {
    int64_t payload, stride, trailer_off;
    int32_t d, ffn, n_experts;
};
RecordExpect record_expect(const Geometry &g);

// CRC-32 of an n-byte payload (n a multiple of 16) on the device.  The payload
// is cut into G spans of `iters` 4 KiB rows, after virtually prepending
// `pad` = G * span - n zero bytes (leading zeros leave a zero-initialised CRC
// register unchanged); one workgroup per span.
struct CrcPlan {
    int64_t n = 0, pad = 0;
    int iters = 0, G = 0;
    uint32_t fin = 0;            // xor turning the raw remainder into the CRC-32
    uint32_t *tables = nullptr;  // device: the constant tables (kCrcTableWords + G words)
};
hipError_t crc_plan_init(CrcPlan &p, int64_t n);
void crc_plan_free(CrcPlan &p);
// part: device [kCrcMaxSpans] partial remainders (one plan's launches in
// stream order may share it).
hipError_t launch_crc_spans(const CrcPlan &p, const uint8_t *data, uint32_t *part, hipStream_t s);
// out[0] = the CRC-32 of the payload whose partials are in part.
hipError_t launch_crc_finish(const CrcPlan &p, const uint32_t *part, uint32_t *out, hipStream_t s);
// Checks the trailer of the record at `rec` against expert e (magic, version,
// id, offset, sizes); with `part` non-null also the payload's CRC-32.  A
// failure ORs its flags (RVQ_MOE_RECORD_BAD_*) into rec_err[0] and raises
// rec_err[1] to at least e + 1.
hipError_t launch_check_record(const CrcPlan *p, const uint8_t *rec, const RecordExpect &ex, int e,
                               const uint32_t *part, int *rec_err, hipStream_t s);

// Host side: fill a trailer, and check one (0, or RVQ_MOE_RECORD_BAD_* flags).
void fill_trailer(rvq_moe_record_trailer *t, const RecordExpect &ex, int e, uint32_t crc);
int check_trailer(const rvq_moe_record_trailer *t, const RecordExpect &ex, int e);

// Write the bank of E records (payloads in the internal layout, CRC-32 in each
// trailer) into pinned host memory `bank` (E * stride bytes) from canonical
// records `canon` (host: pinned host memory; else device memory).
// Synchronises `s`.
hipError_t write_bank(const Geometry &g, const uint8_t *canon, bool canon_on_host, uint8_t *bank, hipStream_t s);

}  // namespace rvq
