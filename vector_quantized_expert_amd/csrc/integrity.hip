// integrity.hip -- expert-record trailers, their checks on every slot fill,
// and the CRC-32 of record payloads computed on the device.
//
// [FR] "Architecture de streaming depuis le disque": each expert record read
// from the bank is checked for its magic, its expert id and its offset range,
// so that a truncated or wrongly assembled bank cannot hand out another
// expert's weights; a crc32 of the payload is checked only on request; the
// codebooks have no checksum.  Here the bank is pinned host memory and a read
// is one copy into an HBM slot, so the checks run on the device, on the slot,
// after the copy and before any kernel reads it.
//
// CRC-32 (reflected polynomial 0xEDB88320, initial value and final xor
// 0xFFFFFFFF) is computed from its algebra.  Words are polynomials over GF(2)
// in reflected bit order (bit 31 is x^0, bit 0 is x^31).  With a zero initial
// register, the remainder R(M) of a message is linear in M and
//   R(A || B) = R(A) * x^(8|B|) ⊕ R(B)   (mod P),
// so leading zero bytes change nothing and pieces of a message can be reduced
// independently and combined by multiplications with powers of x.  The
// CRC-32 itself is R(M) ⊕ (0xFFFFFFFF * x^(8n)) ⊕ 0xFFFFFFFF.
//
// Device plan for n bytes (n a multiple of 16): prepend `pad` zero bytes so
// that the message is G spans of `iters` 4 KiB rows.  Workgroup g (256
// threads) reduces span g: thread t takes the 16-byte word at 16 t of every
// row (one coalesced 4 KiB row per iteration), reduces it with 16
// slice tables (one per byte position) and folds it into a running remainder
// that is multiplied by x^(8*4096) per row (4 table lookups).  The threads'
// remainders are then weighted by x^(128 (255 - t)) and xor-ed, and the
// span's remainder weighted by x^(8 span (G - 1 - g)); the G partials xor
// to R(M).
#include <string.h>

#include <vector>

#include "integrity.hpp"

namespace rvq {

namespace {

constexpr uint32_t kPoly = 0xEDB88320u;  // x^32 + x^26 + ... + 1 without x^32, reflected
constexpr uint32_t kOne = 0x80000000u;   // the polynomial 1
constexpr int kRow = 4096;               // bytes per row: 256 threads x 16
constexpr int kSliceWords = 16 * 256;
constexpr int kStepWords = 4 * 256;
constexpr int kLaneWords = 256;
constexpr int kCrcTableWords = kSliceWords + kStepWords + kLaneWords;

__host__ __device__ inline uint32_t mul_x(uint32_t a) { return (a >> 1) ^ ((a & 1u) ? kPoly : 0u); }

// a * b mod P
__host__ __device__ inline uint32_t mul_mod(uint32_t a, uint32_t b) {
    uint32_t r = 0;
    for (int i = 0; i < 32; i++) {
        if (a & (kOne >> i)) r ^= b;
        b = mul_x(b);
    }
    return r;
}

// x^e mod P
uint32_t x_pow(uint64_t e) {
    uint32_t r = kOne, base = kOne >> 1;  // x^1
    while (e) {
        if (e & 1) r = mul_mod(r, base);
        base = mul_mod(base, base);
        e >>= 1;
    }
    return r;
}

__global__ __launch_bounds__(256) void k_crc_spans(const uint8_t *__restrict__ data, int64_t pad, int iters,
                                                   const uint32_t *__restrict__ tab, uint32_t *__restrict__ part) {
    // rows 0..15: S[k][v] = R(byte v followed by k zero bytes); rows 16..19:
    // U[k][v] = (v << 8k) * x^(8*4096); one array, loaded as the table is laid out
    __shared__ uint32_t tl[16 + 4][256];
    __shared__ uint32_t red[4];
    uint32_t(*S)[256] = tl;
    uint32_t(*U)[256] = tl + 16;
    const int t = threadIdx.x, g = blockIdx.x;
    for (int i = t; i < kSliceWords + kStepWords; i += 256) tl[i >> 8][i & 255] = tab[i];
    __syncthreads();
    const int64_t base = (int64_t)g * iters * kRow + 16 * t - pad;  // offset of this thread's word in row 0
    uint32_t acc = 0;
#pragma unroll 4
    for (int i = 0; i < iters; i++) {
        const int64_t o = base + (int64_t)i * kRow;
        uint4 w = make_uint4(0u, 0u, 0u, 0u);
        if (o >= 0) w = *reinterpret_cast<const uint4 *>(data + o);  // words wholly inside the payload
        uint32_t r = U[0][acc & 0xff] ^ U[1][(acc >> 8) & 0xff] ^ U[2][(acc >> 16) & 0xff] ^ U[3][acc >> 24];
        r ^= S[15][w.x & 0xff] ^ S[14][(w.x >> 8) & 0xff] ^ S[13][(w.x >> 16) & 0xff] ^ S[12][w.x >> 24];
        r ^= S[11][w.y & 0xff] ^ S[10][(w.y >> 8) & 0xff] ^ S[9][(w.y >> 16) & 0xff] ^ S[8][w.y >> 24];
        r ^= S[7][w.z & 0xff] ^ S[6][(w.z >> 8) & 0xff] ^ S[5][(w.z >> 16) & 0xff] ^ S[4][w.z >> 24];
        r ^= S[3][w.w & 0xff] ^ S[2][(w.w >> 8) & 0xff] ^ S[1][(w.w >> 16) & 0xff] ^ S[0][w.w >> 24];
        acc = r;
    }
    acc = mul_mod(acc, tab[kSliceWords + kStepWords + t]);
    for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m, 64);
    if ((t & 63) == 0) red[t >> 6] = acc;
    __syncthreads();
    if (t == 0) part[g] = mul_mod(red[0] ^ red[1] ^ red[2] ^ red[3], tab[kCrcTableWords + g]);
}

__device__ inline uint32_t xor_partials(const uint32_t *part, int G) {
    __shared__ uint32_t red[4];
    const int t = threadIdx.x;
    uint32_t x = 0;
    for (int i = t; i < G; i += 256) x ^= part[i];
    for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m, 64);
    if ((t & 63) == 0) red[t >> 6] = x;
    __syncthreads();
    return red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(256) void k_crc_finish(const uint32_t *part, int G, uint32_t fin, uint32_t *out) {
    const uint32_t r = xor_partials(part, G);
    if (threadIdx.x == 0) out[0] = r ^ fin;
}

__global__ __launch_bounds__(256) void k_check_record(const uint8_t *rec, RecordExpect ex, int e,
                                                      const uint32_t *part, int G, uint32_t fin, int *rec_err) {
    const uint32_t r = part ? xor_partials(part, G) : 0u;
    if (threadIdx.x != 0) return;
    const rvq_moe_record_trailer *t = reinterpret_cast<const rvq_moe_record_trailer *>(rec + ex.trailer_off);
    int flags = 0;
    if (t->magic != RVQ_MOE_RECORD_MAGIC || t->version != RVQ_MOE_RECORD_VERSION) flags |= RVQ_MOE_RECORD_BAD_MAGIC;
    if (t->expert != (uint32_t)e || t->n_experts != (uint32_t)ex.n_experts) flags |= RVQ_MOE_RECORD_BAD_ID;
    if (t->offset != (uint64_t)e * (uint64_t)ex.stride || t->payload_bytes != (uint64_t)ex.payload || t->d != ex.d ||
        t->ffn != ex.ffn)
        flags |= RVQ_MOE_RECORD_BAD_RANGE;
    if (part && (r ^ fin) != t->crc32) flags |= RVQ_MOE_RECORD_BAD_CRC;
    if (flags) {
        atomicOr(&rec_err[0], flags);
        atomicMax(&rec_err[1], e + 1);
    }
}

}  // namespace

RecordExpect record_expect(const Geometry &g) {
    RecordExpect ex;
    ex.payload = g.rec_int;
    ex.stride = bank_stride(g);
    ex.trailer_off = bank_trailer_off(g);
    ex.d = g.d;
    ex.ffn = g.ffn;
    ex.n_experts = g.E;
    return ex;
}

hipError_t crc_plan_init(CrcPlan &p, int64_t n) {
    p = CrcPlan{};
    if (n <= 0 || n % 16) return hipErrorInvalidValue;
    const int64_t rows = (n + kRow - 1) / kRow;
    p.n = n;
    p.iters = (int)((rows + kCrcMaxSpans - 1) / kCrcMaxSpans);
    p.G = (int)((rows + p.iters - 1) / p.iters);
    const int64_t span = (int64_t)p.iters * kRow;
    p.pad = (int64_t)p.G * span - n;
    p.fin = mul_mod(0xFFFFFFFFu, x_pow(8 * (uint64_t)n)) ^ 0xFFFFFFFFu;
    std::vector<uint32_t> h(kCrcTableWords + p.G);
    uint32_t *S = h.data(), *U = S + kSliceWords, *L = U + kStepWords, *D = L + kLaneWords;
    for (uint32_t v = 0; v < 256; v++) {
        uint32_t c = v;
        for (int b = 0; b < 8; b++) c = mul_x(c);
        S[v] = c;  // R(v) = v * x^8 with v in the low bits (the x^24 .. x^31 terms)
    }
    const uint32_t x8 = x_pow(8);
    for (int k = 1; k < 16; k++)
        for (int v = 0; v < 256; v++) S[k * 256 + v] = mul_mod(S[(k - 1) * 256 + v], x8);
    const uint32_t step = x_pow(8 * (uint64_t)kRow);
    for (int k = 0; k < 4; k++)
        for (uint32_t v = 0; v < 256; v++) U[k * 256 + v] = mul_mod(v << (8 * k), step);
    for (int t = 0; t < 256; t++) L[t] = x_pow(128 * (uint64_t)(255 - t));
    const uint32_t span_pow = x_pow(8 * (uint64_t)span);
    D[p.G - 1] = kOne;
    for (int g = p.G - 2; g >= 0; g--) D[g] = mul_mod(D[g + 1], span_pow);
    hipError_t e = hipMalloc(&p.tables, sizeof(uint32_t) * h.size());
    if (e != hipSuccess) {
        p.tables = nullptr;
        return e;
    }
    e = hipMemcpy(p.tables, h.data(), sizeof(uint32_t) * h.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) crc_plan_free(p);
    return e;
}

void crc_plan_free(CrcPlan &p) {
    if (p.tables) (void)hipFree(p.tables);
    p = CrcPlan{};
}

hipError_t launch_crc_spans(const CrcPlan &p, const uint8_t *data, uint32_t *part, hipStream_t s) {
    hipLaunchKernelGGL(k_crc_spans, dim3(p.G), dim3(256), 0, s, data, p.pad, p.iters, p.tables, part);
    return hipGetLastError();
}

hipError_t launch_crc_finish(const CrcPlan &p, const uint32_t *part, uint32_t *out, hipStream_t s) {
    hipLaunchKernelGGL(k_crc_finish, dim3(1), dim3(256), 0, s, part, p.G, p.fin, out);
    return hipGetLastError();
}

hipError_t launch_check_record(const CrcPlan *p, const uint8_t *rec, const RecordExpect &ex, int e,
                               const uint32_t *part, int *rec_err, hipStream_t s) {
    hipLaunchKernelGGL(k_check_record, dim3(1), dim3(256), 0, s, rec, ex, e, part, p ? p->G : 0, p ? p->fin : 0u,
                       rec_err);
    return hipGetLastError();
}

void fill_trailer(rvq_moe_record_trailer *t, const RecordExpect &ex, int e, uint32_t crc) {
    memset(t, 0, sizeof *t);
    t->magic = RVQ_MOE_RECORD_MAGIC;
    t->version = RVQ_MOE_RECORD_VERSION;
    t->expert = (uint32_t)e;
    t->n_experts = (uint32_t)ex.n_experts;
    t->offset = (uint64_t)e * (uint64_t)ex.stride;
    t->payload_bytes = (uint64_t)ex.payload;
    t->d = ex.d;
    t->ffn = ex.ffn;
    t->crc32 = crc;
}

int check_trailer(const rvq_moe_record_trailer *t, const RecordExpect &ex, int e) {
    int flags = 0;
    if (t->magic != RVQ_MOE_RECORD_MAGIC || t->version != RVQ_MOE_RECORD_VERSION) flags |= RVQ_MOE_RECORD_BAD_MAGIC;
    if (t->expert != (uint32_t)e || t->n_experts != (uint32_t)ex.n_experts) flags |= RVQ_MOE_RECORD_BAD_ID;
    if (t->offset != (uint64_t)e * (uint64_t)ex.stride || t->payload_bytes != (uint64_t)ex.payload || t->d != ex.d ||
        t->ffn != ex.ffn)
        flags |= RVQ_MOE_RECORD_BAD_RANGE;
    return flags;
}

hipError_t write_bank(const Geometry &g, const uint8_t *canon, bool canon_on_host, uint8_t *bank, hipStream_t s) {
    const RecordExpect ex = record_expect(g);
    const int B = g.E < 8 ? g.E : 8;
    CrcPlan plan;
    uint8_t *staged = nullptr, *internal = nullptr;
    uint32_t *part = nullptr, *crc_dev = nullptr;
    uint32_t crc_host[8];
    hipError_t e = crc_plan_init(plan, g.rec_int);
    if (e == hipSuccess && canon_on_host) e = hipMalloc(&staged, (size_t)(B * g.rec_canon));
    if (e == hipSuccess) e = hipMalloc(&internal, (size_t)(B * g.rec_int));
    if (e == hipSuccess) e = hipMalloc(&part, sizeof(uint32_t) * kCrcMaxSpans);
    if (e == hipSuccess) e = hipMalloc(&crc_dev, sizeof(uint32_t) * B);
    for (int e0 = 0; e0 < g.E && e == hipSuccess; e0 += B) {
        const int n = g.E - e0 < B ? g.E - e0 : B;
        const uint8_t *src = canon + (int64_t)e0 * g.rec_canon;
        if (canon_on_host) {
            e = hipMemcpyAsync(staged, src, (size_t)(n * g.rec_canon), hipMemcpyHostToDevice, s);
            src = staged;
        }
        if (e == hipSuccess) e = launch_repack(g, src, internal, n, s);
        for (int i = 0; i < n && e == hipSuccess; i++) {
            const uint8_t *rec = internal + (int64_t)i * g.rec_int;
            e = launch_crc_spans(plan, rec, part, s);
            if (e == hipSuccess) e = launch_crc_finish(plan, part, crc_dev + i, s);
            if (e == hipSuccess)
                e = hipMemcpyAsync(bank + (int64_t)(e0 + i) * ex.stride, rec, (size_t)g.rec_int,
                                   hipMemcpyDeviceToHost, s);
        }
        if (e == hipSuccess) e = hipMemcpyAsync(crc_host, crc_dev, sizeof(uint32_t) * n, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);  // the staging buffers are reused
        for (int i = 0; i < n && e == hipSuccess; i++) {
            uint8_t *r = bank + (int64_t)(e0 + i) * ex.stride;
            memset(r + g.rec_int, 0, (size_t)(ex.stride - g.rec_int));
            fill_trailer(reinterpret_cast<rvq_moe_record_trailer *>(r + ex.trailer_off), ex, e0 + i, crc_host[i]);
        }
    }
    (void)hipFree(staged);
    (void)hipFree(internal);
    (void)hipFree(part);
    (void)hipFree(crc_dev);
    crc_plan_free(plan);
    return e;
}

}  // namespace rvq
