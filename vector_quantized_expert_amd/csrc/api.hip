// api.hip -- the C ABI declared in include/rvq_moe.h.
//
// [FR] "Objectif et forme d'implémentation de WASTE": the engine exposes a small
// C API (open, set a memory limit, run, close) that Python calls through
// ctypes; [FR] "Budget RAM et fenêtre de performance étroite": it refuses to
// start below the minimum budget instead of degrading.  Here: open validates
// everything and owns all device memory; route_topk and layer_forward only
// enqueue kernels on the caller's stream (no host synchronisation, no
// allocation); close frees everything.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "rvq_moe.h"

#include "integrity.hpp"
#include "internal.hpp"
#include "slots.hpp"

using namespace rvq;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

struct EventPair {
    hipEvent_t a, b;
    int kind;
};

}  // namespace

struct rvq_moe {
    int device;
    Geometry g;
    int pre_rmsnorm, residual, max_tokens;
    bool det;            // deterministic combine (desc.deterministic)
    int chunk_min;       // layer_forward calls with T >= chunk_min take the chunk path
    int lut_tokens;      // in such a call, experts with fewer tokens take the table path
    ChunkWork cw;        // its workspace (all null when max_tokens < chunk_min)
    double eps;
    uint8_t *codes;      // [E][rec_int] internal layout (resident codes), or null when streaming
    bool streaming;      // codes in pinned host memory, cached in HBM slots
    SlotCache cache;     // the slot cache (streaming only)
    std::vector<int> call_experts;  // scratch: a call's distinct experts
    std::vector<int> call_used;     // scratch: slots a launch reads
    void *cbs;           // [E][3][3][256][8]
    float *router_wt;    // [E][d] (transposed copy)
    Workspace ws;
    rvq_moe_stats stats;
    int prof_every;
    uint64_t prof_calls;
    uint64_t prof_route_calls;
    std::vector<EventPair> prof_events;
    std::vector<hipEvent_t> prof_pool;
};

namespace rvq {

Geometry make_geometry(int d, int ffn, int E, int k, int cb_dtype) {
    Geometry g{};
    g.d = d;
    g.ffn = ffn;
    g.E = E;
    g.k = k;
    g.cb_dtype = cb_dtype;
    const int rows[3] = {ffn, ffn, d};
    const int slices[3] = {d / kVec, d / kVec, ffn / kVec};
    int64_t off = 0;
    for (int m = 0; m < 3; m++) {
        MatGeom &mg = g.m[m];
        mg.rows = rows[m];
        mg.slices = slices[m];
        mg.n_tiles = (slices[m] + kTileSlices - 1) / kTileSlices;
        mg.n_chunks = (rows[m] + kChunkRows - 1) / kChunkRows;
        mg.off = off;
        mg.bytes = (int64_t)mg.n_tiles * mg.n_chunks * kChunkBytes;
        off += mg.bytes;
    }
    g.rec_int = off;
    g.rec_canon = (int64_t)9 * d * ffn / 8;
    g.cb_bytes = (int64_t)3 * kStages * kCodes * kVec * (cb_dtype == 0 ? 4 : 2);
    g.ffn_pad = g.m[0].n_chunks * kChunkRows;
    g.d_pad = g.m[2].n_chunks * kChunkRows;
    g.d_tpad = g.m[0].n_tiles * kTileSlices * kVec;
    g.ffn_tpad = g.m[2].n_tiles * kTileSlices * kVec;
    return g;
}

}  // namespace rvq

static void free_handle(rvq_moe *h) {
    if (!h) return;
    (void)hipFree(h->codes);
    (void)hipFree(h->cbs);
    (void)hipFree(h->router_wt);
    (void)hipFree(h->ws.logits);
    (void)hipFree(h->ws.sel);
    (void)hipFree(h->ws.route_logits);
    (void)hipFree(h->ws.fused_logits);
    (void)hipFree(h->ws.part_gu);
    (void)hipFree(h->ws.cnt);
    (void)hipFree(h->ws.err);
    (void)hipFree(h->ws.cb_exp);
    (void)hipFree(h->ws.part_y);
    (void)hipFree(h->cw.X);
    (void)hipFree(h->cw.H);
    (void)hipFree(h->cw.perm);
    (void)hipFree(h->cw.grp_off);
    (void)hipFree(h->cw.act);
    (void)hipFree(h->cw.list);
    if (h->cw.fork) (void)hipEventDestroy(h->cw.fork);
    if (h->cw.join) (void)hipEventDestroy(h->cw.join);
    if (h->cw.side) (void)hipStreamDestroy(h->cw.side);
    for (hipEvent_t e : h->prof_pool) (void)hipEventDestroy(e);
    slots_close(h->cache);
    delete h;
}

#define HIP_TRY(call)                                                                     \
    do {                                                                                  \
        hipError_t _e = (call);                                                           \
        if (_e != hipSuccess) {                                                           \
            int _code = (_e == hipErrorOutOfMemory) ? RVQ_MOE_ENOMEM : RVQ_MOE_EHIP;      \
            fail(_code, "%s failed: %s", #call, hipGetErrorString(_e));                   \
            return _code;                                                                 \
        }                                                                                 \
    } while (0)

static int open_impl(const rvq_moe_desc *desc, rvq_moe *h) {
    const rvq_moe_desc &D = *desc;
    hipStream_t s = static_cast<hipStream_t>(D.stream);
    HIP_TRY(hipGetDevice(&h->device));
    h->g = make_geometry(D.d, D.ffn, D.n_experts, D.top_k, D.codebook_dtype);
    h->pre_rmsnorm = D.pre_rmsnorm != 0;
    h->residual = D.residual != 0;
    h->eps = D.eps;
    h->max_tokens = D.max_tokens;
    h->chunk_min = D.chunk_min_tokens > 0 ? D.chunk_min_tokens : RVQ_MOE_CHUNK_MIN_TOKENS;
    h->lut_tokens = D.lut_expert_tokens > 0 ? D.lut_expert_tokens : RVQ_MOE_LUT_EXPERT_TOKENS;
    h->det = D.deterministic != 0;
    if (D.codes_location != RVQ_MOE_CODES_DEVICE || h->det) h->lut_tokens = 1;
    const Geometry &g = h->g;
    const int64_t E = D.n_experts;
    h->streaming = D.codes_location != RVQ_MOE_CODES_DEVICE;
    if (!h->streaming) HIP_TRY(hipMalloc(&h->codes, (size_t)(E * g.rec_int)));
    HIP_TRY(hipMalloc(&h->cbs, (size_t)(E * g.cb_bytes)));
    HIP_TRY(hipMalloc(&h->router_wt, sizeof(float) * (size_t)D.d * E));
    const int64_t T = D.max_tokens, P = T * D.top_k;
    HIP_TRY(hipMalloc(&h->ws.logits, sizeof(double) * (size_t)(T * E)));
    HIP_TRY(hipMalloc(&h->ws.sel, sizeof(double) * (size_t)(T * D.top_k)));
    HIP_TRY(hipMalloc(&h->ws.route_logits, sizeof(double) * (size_t)route_logit_slots(T, D.n_experts)));
    HIP_TRY(hipMalloc(&h->ws.fused_logits, sizeof(double) * (size_t)fused_route_slots(T, D.n_experts)));
    HIP_TRY(hipMalloc(&h->ws.part_gu, sizeof(float) * (size_t)(P * 2 * g.m[0].n_tiles * g.ffn_pad)));
    h->ws.cnt_per_set = (int)(P + 1);
    h->ws.cnt_phase = 0;
    HIP_TRY(hipMalloc(&h->ws.cnt, sizeof(int) * (size_t)kCntSets * (P + 1) * kCntStride));
    HIP_TRY(hipMalloc(&h->ws.err, sizeof(int)));
    HIP_TRY(hipMalloc(&h->ws.cb_exp, sizeof(int) * 3 * (size_t)E));
    h->ws.det = h->cw.det = h->det;
    if (h->det) {  // pair output rows per down tile (table path) or whole (chunk path: the first d_pad of each)
        HIP_TRY(hipMalloc(&h->ws.part_y, sizeof(float) * (size_t)(P * g.m[2].n_tiles * g.d_pad)));
        h->cw.part_y = h->ws.part_y;
    }
    if (h->max_tokens >= h->chunk_min) {
        HIP_TRY(hipMalloc(&h->cw.X, 2 * (size_t)(T * g.d_tpad)));
        HIP_TRY(hipMalloc(&h->cw.H, 2 * (size_t)(P * g.ffn_tpad)));
        HIP_TRY(hipMemsetAsync(h->cw.X, 0, 2 * (size_t)(T * g.d_tpad), s));  // the pad columns stay zero
        HIP_TRY(hipMemsetAsync(h->cw.H, 0, 2 * (size_t)(P * g.ffn_tpad), s));
        HIP_TRY(hipMalloc(&h->cw.perm, sizeof(int) * (size_t)P));
        HIP_TRY(hipMalloc(&h->cw.grp_off, sizeof(int) * (size_t)(E + 2)));
        HIP_TRY(hipMalloc(&h->cw.act, sizeof(int) * (size_t)(E + 1)));
        HIP_TRY(hipMalloc(&h->cw.list, sizeof(int) * (size_t)kPairListInts));
        if (!h->streaming) {  // (default priority, like every stream here)
            HIP_TRY(hipStreamCreateWithFlags(&h->cw.side, hipStreamNonBlocking));
            HIP_TRY(hipEventCreateWithFlags(&h->cw.fork, hipEventDisableTiming));
            HIP_TRY(hipEventCreateWithFlags(&h->cw.join, hipEventDisableTiming));
        }
    }
    int n_cu = 0;
    HIP_TRY(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, h->device));
    int per_cu = 0;
    HIP_TRY(layer_blocks_per_cu(D.codebook_dtype, &per_cu));
    if (n_cu < 1 || per_cu < 1) return fail(RVQ_MOE_EHIP, "occupancy query gave %d CUs x %d blocks", n_cu, per_cu);
    HIP_TRY(static_scratch_setup(h->device));  // once per device: rvq_moe_layer_forward_noalloc's scratch
    HIP_TRY(init_route(h->ws, D.n_experts, D.top_k, T, n_cu, s));
    // a streaming handle's router may run on a side stream next to layer
    // kernels (router lookahead): it takes the kernels that need no co-resident grid
    if (h->streaming) h->ws.route_one = false;
    h->ws.n_wg = n_cu * per_cu;
    if (h->ws.n_wg > 1024) h->ws.n_wg = 1024;  // a bound on the persistent grid
    HIP_TRY(hipMemsetAsync(h->ws.cnt, 0, sizeof(int) * (size_t)kCntSets * (P + 1) * kCntStride, s));
    HIP_TRY(hipMemsetAsync(h->ws.err, 0, sizeof(int), s));
    HIP_TRY(hipMemcpyAsync(h->cbs, D.codebooks, (size_t)(E * g.cb_bytes), hipMemcpyDeviceToDevice, s));
    HIP_TRY(launch_cb_exponents(h->cbs, D.codebook_dtype, D.n_experts, h->ws.cb_exp, s));
    HIP_TRY(launch_transpose(D.router_w, h->router_wt, D.d, D.n_experts, s));
    if (h->streaming) {
        const int S = D.cache_slots < D.n_experts ? D.cache_slots : D.n_experts;
        const bool borrowed = D.codes_location == RVQ_MOE_CODES_PINNED_BANK;
        HIP_TRY(slots_open(h->cache, g, S, (int)P, borrowed ? nullptr : D.codes, borrowed ? D.codes : nullptr,
                           D.verify_records != 0, s));
    } else {
        HIP_TRY(launch_repack(g, D.codes, h->codes, D.n_experts, s));
    }
    HIP_TRY(hipStreamSynchronize(s));
    h->stats.code_bytes_resident = h->streaming ? (uint64_t)(h->cache.S * h->cache.rec) : (uint64_t)(E * g.rec_int);
    h->stats.record_bytes = (uint64_t)g.rec_canon;
    h->stats.codebook_bytes = (uint64_t)g.cb_bytes;
    return RVQ_MOE_OK;
}

// The layer shape and format fields shared by open, bank_layout and write_bank.
static int check_shape(const rvq_moe_desc *desc) {
    if (!desc) return fail(RVQ_MOE_EINVAL, "desc is NULL");
    const rvq_moe_desc &D = *desc;
    if (D.struct_size != sizeof(rvq_moe_desc))
        return fail(RVQ_MOE_EINVAL, "struct_size %u != %zu", D.struct_size, sizeof(rvq_moe_desc));
    if (D.n_stages != kStages || D.n_codes != kCodes || D.vec_dim != kVec)
        return fail(RVQ_MOE_ENOTSUP, "only 3 stages x 256 codes x 8-wide vectors are supported");
    if (D.d <= 0 || D.ffn <= 0 || D.d % kVec || D.ffn % kVec || D.d > 65536 || D.ffn > 65536)
        return fail(RVQ_MOE_EINVAL, "d=%d ffn=%d must be positive multiples of 8, <= 65536", D.d, D.ffn);
    if (D.n_experts < 1 || D.n_experts > kMaxExperts)
        return fail(RVQ_MOE_EINVAL, "n_experts=%d outside [1, %d]", D.n_experts, kMaxExperts);
    if (D.top_k < 1 || D.top_k > D.n_experts || D.top_k > kMaxTopK)
        return fail(RVQ_MOE_EINVAL, "top_k=%d outside [1, min(E, %d)]", D.top_k, kMaxTopK);
    if (D.codebook_dtype != RVQ_MOE_CB_F32 && D.codebook_dtype != RVQ_MOE_CB_F16)
        return fail(RVQ_MOE_EINVAL, "codebook_dtype=%d", D.codebook_dtype);
    return RVQ_MOE_OK;
}

static bool is_pinned_host(const void *p) {
    hipPointerAttribute_t attr;
    const hipError_t pe = hipPointerGetAttributes(&attr, p);
    (void)hipGetLastError();  // clear the error a plain host pointer leaves
    return pe == hipSuccess && attr.type == hipMemoryTypeHost;
}

extern "C" int rvq_moe_open(const rvq_moe_desc *desc, rvq_moe **out) {
    g_err[0] = 0;
    if (!out) return fail(RVQ_MOE_EINVAL, "out is NULL");
    *out = nullptr;
    if (const int rc = check_shape(desc)) return rc;
    const rvq_moe_desc &D = *desc;
    if (D.max_tokens < 1) return fail(RVQ_MOE_EINVAL, "max_tokens=%d < 1", D.max_tokens);
    {
        // the layer kernel numbers its work units (one 32-row chunk of one
        // 32-slice tile of one pair's matrix) in 32 bits
        const int64_t n_ti = (D.d / kVec + kTileSlices - 1) / kTileSlices, n_cf = (D.ffn + kChunkRows - 1) / kChunkRows;
        const int64_t n_tf = (D.ffn / kVec + kTileSlices - 1) / kTileSlices, n_cd = (D.d + kChunkRows - 1) / kChunkRows;
        const int64_t per_pair = std::max(2 * n_ti * n_cf, n_tf * n_cd);
        if ((int64_t)D.max_tokens * D.top_k * per_pair >= ((int64_t)1 << 31))
            return fail(RVQ_MOE_EINVAL, "max_tokens=%d: one call would exceed 2^31 work units", D.max_tokens);
    }
    if (D.cache_slots < 0) return fail(RVQ_MOE_EINVAL, "cache_slots=%d < 0", D.cache_slots);
    if (D.chunk_min_tokens < 0) return fail(RVQ_MOE_EINVAL, "chunk_min_tokens=%d < 0", D.chunk_min_tokens);
    if (D.lut_expert_tokens < 0) return fail(RVQ_MOE_EINVAL, "lut_expert_tokens=%d < 0", D.lut_expert_tokens);
    if (D.cache_slots > 0 && D.cache_slots < D.top_k)
        return fail(RVQ_MOE_EBUDGET, "cache_slots=%d below one token's working set (top_k=%d)", D.cache_slots,
                    D.top_k);
    if (D.codes_location != RVQ_MOE_CODES_DEVICE && D.codes_location != RVQ_MOE_CODES_PINNED_HOST &&
        D.codes_location != RVQ_MOE_CODES_PINNED_BANK)
        return fail(RVQ_MOE_EINVAL, "codes_location=%d", D.codes_location);
    if (D.codes_location == RVQ_MOE_CODES_DEVICE && D.cache_slots != 0)
        return fail(RVQ_MOE_EINVAL, "cache_slots=%d: the slot cache streams PINNED_HOST or PINNED_BANK codes only",
                    D.cache_slots);
    if (D.deterministic != 0 && D.deterministic != 1)
        return fail(RVQ_MOE_EINVAL, "deterministic=%d must be 0 or 1", D.deterministic);
    if (!D.router_w || !D.codebooks || !D.codes) return fail(RVQ_MOE_EINVAL, "null router_w/codebooks/codes");
    if (D.codes_location != RVQ_MOE_CODES_DEVICE) {
        if (D.cache_slots == 0) return fail(RVQ_MOE_EINVAL, "streamed codes need cache_slots >= top_k");
        if (!is_pinned_host(D.codes))
            return fail(RVQ_MOE_EINVAL, "PINNED_HOST / PINNED_BANK codes must be pinned host memory (hipHostMalloc)");
    }
    if (D.codes_location == RVQ_MOE_CODES_PINNED_BANK) {
        // every trailer, on the host, before anything is allocated
        const Geometry g = make_geometry(D.d, D.ffn, D.n_experts, D.top_k, D.codebook_dtype);
        const RecordExpect ex = record_expect(g);
        for (int e = 0; e < D.n_experts; e++) {
            const auto *t = reinterpret_cast<const rvq_moe_record_trailer *>(D.codes + (int64_t)e * ex.stride +
                                                                              ex.trailer_off);
            if (const int flags = check_trailer(t, ex, e))
                return fail(RVQ_MOE_ECORRUPT, "bank record %d fails its trailer check (flags 0x%x:%s%s%s)", e, flags,
                            (flags & RVQ_MOE_RECORD_BAD_MAGIC) ? " magic/version" : "",
                            (flags & RVQ_MOE_RECORD_BAD_ID) ? " expert id" : "",
                            (flags & RVQ_MOE_RECORD_BAD_RANGE) ? " offset/size/shape" : "");
        }
    }
    if (!(D.eps >= 0.0)) return fail(RVQ_MOE_EINVAL, "eps must be >= 0");
    rvq_moe *h = new (std::nothrow) rvq_moe();
    if (!h) return fail(RVQ_MOE_ENOMEM, "host allocation failed");
    const int rc = open_impl(desc, h);
    if (rc != RVQ_MOE_OK) {
        free_handle(h);
        return rc;
    }
    *out = h;
    return RVQ_MOE_OK;
}

static int check_call(rvq_moe *h, const void *x, int32_t T) {
    if (!h) return fail(RVQ_MOE_EINVAL, "handle is NULL");
    if (!x) return fail(RVQ_MOE_EINVAL, "x is NULL");
    if (T < 1 || T > h->max_tokens) return fail(RVQ_MOE_EINVAL, "n_tokens=%d outside [1, %d]", T, h->max_tokens);
    return RVQ_MOE_OK;
}

// Brackets one kernel launch with profiling events when this call is sampled.
struct ProfScope {
    rvq_moe *h;
    hipStream_t s;
    bool on;
    int kind;
    hipEvent_t a = nullptr, b = nullptr;
    ProfScope(rvq_moe *h_, hipStream_t s_, bool on_, int kind_) : h(h_), s(s_), on(on_), kind(kind_) {
        if (!on) return;
        if (h->prof_pool.size() < 2) {
            on = false;
            return;
        }
        b = h->prof_pool.back();
        h->prof_pool.pop_back();
        a = h->prof_pool.back();
        h->prof_pool.pop_back();
        (void)hipEventRecord(a, s);
    }
    ~ProfScope() {
        if (!on) return;
        (void)hipEventRecord(b, s);
        h->prof_events.push_back({a, b, kind});
    }
};

extern "C" int rvq_moe_route_topk(rvq_moe *h, const float *x, int32_t T, int32_t *ids, float *gates,
                                  void *stream) {
    int rc = check_call(h, x, T);
    if (rc) return rc;
    if (!ids || !gates) return fail(RVQ_MOE_EINVAL, "ids/gates is NULL");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool prof = h->prof_every > 0 && (h->prof_route_calls++ % (uint64_t)h->prof_every) == 0;
    {
        ProfScope p(h, s, prof, 0);
        HIP_TRY(launch_route(h->g, h->ws, x, h->router_wt, T, h->pre_rmsnorm, h->eps, ids, gates, s));
    }
    h->stats.route_calls++;
    h->stats.tokens_routed += (uint64_t)T;
    return RVQ_MOE_OK;
}

// The deterministic combine after the layer kernels of a call (tokens [0, T)
// of x, ids, y): slots = the down projection's tiles on the table path, 1 on
// the chunk path.
static hipError_t combine(rvq_moe *h, const Workspace &w, int slots, const float *x, const int32_t *ids, float *y,
                          int T, hipStream_t s) {
    const Geometry &g = h->g;
    return launch_combine(w.part_y, slots, x, ids, y, T, g.k, g.E, g.d, g.d_pad, h->residual, s);
}

// layer_forward with the codes streaming through the slot cache.  Reads the
// call's ids back (the one host synchronisation), then enqueues everything:
//  - table path: tokens in runs whose distinct experts fit the slots; per run,
//    the copies of its missing experts, then one layer launch on the run;
//  - chunk path: grouping and staging once, then the active experts in rounds
//    of S / 2, so that the copies of one round overlap the kernels of the
//    previous one (least-recently-used slots are the round before's).
static int stream_forward(rvq_moe *h, const float *x, int T, const int32_t *ids, const float *gates, float *y,
                          hipStream_t s) {
    SlotCache &c = h->cache;
    const Geometry &g = h->g;
    const int k = g.k;
    HIP_TRY(hipMemcpyAsync(c.ids_host, ids, sizeof(int32_t) * (size_t)T * k, hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
    c.syncs++;
    std::vector<int> &U = h->call_experts;
    U.clear();
    if (T >= h->chunk_min) {
        for (int p = 0; p < T * k; p++) {
            const int e = c.ids_host[p];
            if (e >= 0 && e < g.E && c.mark[e] != c.clock + 1) {
                c.mark[e] = (uint32_t)(c.clock + 1);
                U.push_back(e);
            }
        }
        std::sort(U.begin(), U.end());  // the device's order of active experts
        HIP_TRY(launch_chunk_prep(g, h->cw, x, ids, y, T, h->pre_rmsnorm, h->residual, h->eps, 1, h->ws.err, s));
        const int R = c.S >= 2 ? c.S / 2 : 1;
        for (int a0 = 0; a0 < (int)U.size(); a0 += R) {
            const int a1 = a0 + R < (int)U.size() ? a0 + R : (int)U.size();
            HIP_TRY(slots_acquire(c, U.data() + a0, a1 - a0, s, h->call_used));
            HIP_TRY(launch_chunk_experts(g, h->cw, nullptr, c.tab_dev, h->cbs, gates, y, a0, a1, T * k, s));
            HIP_TRY(slots_release(c, h->call_used, s));
        }
        if (h->det) HIP_TRY(combine(h, h->ws, 1, x, ids, y, T, s));
        return RVQ_MOE_OK;
    }
    int t0 = 0;
    uint32_t stamp = (uint32_t)(c.clock + 1);
    auto flush = [&](int t1) -> int {
        HIP_TRY(slots_acquire(c, U.data(), (int)U.size(), s, h->call_used));
        HIP_TRY(launch_layer(g, h->ws, nullptr, c.tab_dev, h->cbs, h->router_wt, x + (size_t)t0 * g.d,
                             ids + (size_t)t0 * k, gates + (size_t)t0 * k, y + (size_t)t0 * g.d, t1 - t0,
                             h->pre_rmsnorm, h->residual, h->eps, false, s));
        HIP_TRY(slots_release(c, h->call_used, s));
        if (h->det)
            HIP_TRY(combine(h, h->ws, g.m[2].n_tiles, x + (size_t)t0 * g.d, ids + (size_t)t0 * k,
                            y + (size_t)t0 * g.d, t1 - t0, s));
        return RVQ_MOE_OK;
    };
    for (int t = 0; t < T; t++) {
        int fresh = 0;  // this token's experts not yet in the run's set
        for (int j = 0; j < k; j++) {
            const int e = c.ids_host[t * k + j];
            if (e < 0 || e >= g.E || c.mark[e] == stamp) continue;
            bool dup = false;
            for (int i = 0; i < j; i++) dup |= c.ids_host[t * k + i] == e;
            fresh += !dup;
        }
        if ((int)U.size() + fresh > c.S) {
            const int rc = flush(t);
            if (rc) return rc;
            t0 = t;
            U.clear();
            stamp = (uint32_t)(c.clock + 1);  // flush advanced the clock: a fresh stamp
        }
        for (int j = 0; j < k; j++) {
            const int e = c.ids_host[t * k + j];
            if (e < 0 || e >= g.E || c.mark[e] == stamp) continue;
            c.mark[e] = stamp;
            U.push_back(e);
        }
    }
    return flush(T);
}

extern "C" int rvq_moe_layer_forward(rvq_moe *h, const float *x, int32_t T, const int32_t *ids,
                                     const float *gates, float *y, void *stream) {
    int rc = check_call(h, x, T);
    if (rc) return rc;
    if (!ids || !gates || !y) return fail(RVQ_MOE_EINVAL, "ids/gates/y is NULL");
    if ((const void *)y == (const void *)x) return fail(RVQ_MOE_EINVAL, "y aliases x");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool prof = h->prof_every > 0 && (h->prof_calls++ % (uint64_t)h->prof_every) == 0;
    if (h->streaming) {
        ProfScope p(h, s, prof, T >= h->chunk_min ? 3 : 1);
        rc = stream_forward(h, x, T, ids, gates, y, s);
        if (rc) return rc;
    } else if (T >= h->chunk_min) {
        ProfScope p(h, s, prof, 3);
        HIP_TRY(launch_chunk(h->g, h->cw, h->codes, h->cbs, x, ids, gates, y, T, h->pre_rmsnorm, h->residual,
                             h->eps, h->lut_tokens, h->ws.err, s));
        if (h->lut_tokens > 1)  // the experts with few tokens, listed by the chunk prep, on the table path
            HIP_TRY(launch_layer(h->g, h->ws, h->codes, nullptr, h->cbs, h->router_wt, x, ids, gates, y, T,
                                 h->pre_rmsnorm, h->residual, h->eps, false, s, h->cw.list));
        if (h->det) HIP_TRY(combine(h, h->ws, 1, x, ids, y, T, s));
    } else {
        ProfScope p(h, s, prof, 1);
        HIP_TRY(launch_layer(h->g, h->ws, h->codes, nullptr, h->cbs, h->router_wt, x, ids, gates, y, T,
                             h->pre_rmsnorm, h->residual, h->eps, false, s));
        if (h->det) HIP_TRY(combine(h, h->ws, h->g.m[2].n_tiles, x, ids, y, T, s));
    }
    h->stats.forward_calls++;
    h->stats.tokens_forwarded += (uint64_t)T;
    h->stats.expert_evals += (uint64_t)T * (uint64_t)h->g.k;
    return RVQ_MOE_OK;
}

extern "C" int rvq_moe_layer_forward_noalloc(rvq_moe *h, const float *x, int32_t T, const int32_t *ids,
                                             const float *gates, float *y, void *stream) {
    int rc = check_call(h, x, T);
    if (rc) return rc;
    if (!ids || !gates || !y) return fail(RVQ_MOE_EINVAL, "ids/gates/y is NULL");
    if ((const void *)y == (const void *)x) return fail(RVQ_MOE_EINVAL, "y aliases x");
    if (h->streaming)
        return fail(RVQ_MOE_ENOTSUP, "layer_forward_noalloc needs resident codes (streaming reads the ids on the host)");
    // the static scratch: both completion counter sets, then the gate/up partial sums
    const Geometry &g = h->g;
    const int64_t P = (int64_t)T * g.k;
    const size_t cnt_ints = (size_t)kCntSets * (size_t)(P + 1) * kCntStride;
    const size_t part_off = (cnt_ints * sizeof(int) + 255) / 256 * 256;
    const size_t party_off = (part_off + sizeof(float) * (size_t)P * 2 * g.m[0].n_tiles * g.ffn_pad + 255) / 256 * 256;
    const size_t need = h->det ? party_off + sizeof(float) * (size_t)P * g.m[2].n_tiles * g.d_pad
                               : part_off + sizeof(float) * (size_t)P * 2 * g.m[0].n_tiles * g.ffn_pad;
    if (need > kStaticScratchBytes)
        return fail(RVQ_MOE_EINVAL,
                    "layer_forward_noalloc: %d tokens need %zu bytes of scratch, above the static %zu (fewer tokens "
                    "per call)",
                    T, need, kStaticScratchBytes);
    char *base = static_scratch(h->device);
    if (!base) return fail(RVQ_MOE_EHIP, "static scratch not set up on device %d", h->device);
    hipStream_t s = static_cast<hipStream_t>(stream);
    Workspace w = h->ws;  // the handle's own workspace is not touched
    w.cnt = reinterpret_cast<int *>(base);
    w.cnt_per_set = (int)(P + 1);
    w.cnt_phase = 0;
    w.part_gu = reinterpret_cast<float *>(base + part_off);
    if (h->det) w.part_y = reinterpret_cast<float *>(base + party_off);
    const bool prof = h->prof_every > 0 && (h->prof_calls++ % (uint64_t)h->prof_every) == 0;
    {
        ProfScope p(h, s, prof, 1);
        // the counters start at zero in every call (the array keeps the last
        // call's contents, possibly another handle's), by a kernel, not a memset
        HIP_TRY(launch_zero_ints(w.cnt, (int)cnt_ints, s));
        HIP_TRY(launch_layer(g, w, h->codes, nullptr, h->cbs, h->router_wt, x, ids, gates, y, T, h->pre_rmsnorm,
                             h->residual, h->eps, false, s));
        if (h->det) HIP_TRY(combine(h, w, g.m[2].n_tiles, x, ids, y, T, s));
    }
    h->stats.forward_calls++;
    h->stats.tokens_forwarded += (uint64_t)T;
    h->stats.expert_evals += (uint64_t)T * (uint64_t)g.k;
    return RVQ_MOE_OK;
}

extern "C" int rvq_moe_route_forward(rvq_moe *h, const float *x, int32_t T, int32_t *ids, float *gates, float *y,
                                     void *stream) {
    int rc = check_call(h, x, T);
    if (rc) return rc;
    if (!ids || !gates || !y) return fail(RVQ_MOE_EINVAL, "ids/gates/y is NULL");
    if ((const void *)y == (const void *)x) return fail(RVQ_MOE_EINVAL, "y aliases x");
    if (T * h->g.k > kRouteMaxPairs)
        return fail(RVQ_MOE_EINVAL, "n_tokens * top_k = %d above %d for one routed call", T * h->g.k, kRouteMaxPairs);
    if (h->streaming)
        return fail(RVQ_MOE_ENOTSUP, "route_forward needs resident codes (streaming reads the ids on the host)");
    if (h->g.E > kRouteExperts * h->ws.n_wg)
        return fail(RVQ_MOE_ENOTSUP, "route_forward: %d experts above %d per workgroup of the %d-workgroup grid",
                    h->g.E, kRouteExperts, h->ws.n_wg);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool prof = h->prof_every > 0 && (h->prof_calls++ % (uint64_t)h->prof_every) == 0;
    {
        ProfScope p(h, s, prof, 2);
        HIP_TRY(launch_layer(h->g, h->ws, h->codes, nullptr, h->cbs, h->router_wt, x, ids, gates, y, T,
                             h->pre_rmsnorm, h->residual, h->eps, true, s));
        if (h->det) HIP_TRY(combine(h, h->ws, h->g.m[2].n_tiles, x, ids, y, T, s));
    }
    h->stats.route_calls++;
    h->stats.tokens_routed += (uint64_t)T;
    h->stats.forward_calls++;
    h->stats.tokens_forwarded += (uint64_t)T;
    h->stats.expert_evals += (uint64_t)T * (uint64_t)h->g.k;
    return RVQ_MOE_OK;
}

static int take_device_error(rvq_moe *h) {
    if (h->streaming) {
        int rec[2] = {0, 0};  // never cleared: the bank is damaged
        HIP_TRY(hipMemcpy(rec, h->cache.rec_err, sizeof rec, hipMemcpyDeviceToHost));
        if (rec[0])
            return fail(RVQ_MOE_ECORRUPT, "expert record check failed (flags 0x%x:%s%s%s%s; expert %d%s)", rec[0],
                        (rec[0] & RVQ_MOE_RECORD_BAD_MAGIC) ? " magic/version" : "",
                        (rec[0] & RVQ_MOE_RECORD_BAD_ID) ? " expert id" : "",
                        (rec[0] & RVQ_MOE_RECORD_BAD_RANGE) ? " offset/size/shape" : "",
                        (rec[0] & RVQ_MOE_RECORD_BAD_CRC) ? " payload crc32" : "", rec[1] - 1,
                        "; the highest failing one");
    }
    int flag = 0;
    HIP_TRY(hipMemcpy(&flag, h->ws.err, sizeof(int), hipMemcpyDeviceToHost));
    if (flag) {
        HIP_TRY(hipMemset(h->ws.err, 0, sizeof(int)));
        return fail(RVQ_MOE_EDEVICE, "device error flags 0x%x:%s%s", flag,
                    (flag & 1) ? " an expert id outside [0, E)" : "",
                    (flag & 2) ? " an inter-workgroup wait timed out" : "");
    }
    return RVQ_MOE_OK;
}

extern "C" int rvq_moe_prefetch(rvq_moe *h, const int32_t *ids, int32_t T, int32_t per_token, void *stream) {
    if (!h) return fail(RVQ_MOE_EINVAL, "handle is NULL");
    if (!ids) return fail(RVQ_MOE_EINVAL, "ids is NULL");
    if (T < 1 || T > h->max_tokens) return fail(RVQ_MOE_EINVAL, "n_tokens=%d outside [1, %d]", T, h->max_tokens);
    if (per_token < 1 || per_token > h->g.k)
        return fail(RVQ_MOE_EINVAL, "per_token=%d outside [1, %d]", per_token, h->g.k);
    if (!h->streaming) return fail(RVQ_MOE_ENOTSUP, "prefetch needs codes streaming from pinned host memory");
    hipStream_t s = static_cast<hipStream_t>(stream);
    SlotCache &c = h->cache;
    const int k = h->g.k;
    HIP_TRY(hipMemcpyAsync(c.ids_host, ids, sizeof(int32_t) * (size_t)T * k, hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
    c.syncs++;
    // distinct experts in token-major order, at most one per slot
    std::vector<int> &U = h->call_experts;
    U.clear();
    const uint32_t stamp = (uint32_t)(c.clock + 1);
    for (int t = 0; t < T && (int)U.size() < c.S; t++)
        for (int j = 0; j < per_token && (int)U.size() < c.S; j++) {
            const int e = c.ids_host[t * k + j];
            if (e < 0 || e >= h->g.E || c.mark[e] == stamp) continue;
            c.mark[e] = stamp;
            U.push_back(e);
        }
    HIP_TRY(slots_prefetch(c, U.data(), (int)U.size()));
    return RVQ_MOE_OK;
}

extern "C" int rvq_moe_sync(rvq_moe *h, void *stream) {
    if (!h) return fail(RVQ_MOE_EINVAL, "handle is NULL");
    HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
    return take_device_error(h);
}

extern "C" int rvq_moe_close(rvq_moe *h) {
    if (!h) return RVQ_MOE_OK;
    int rc = RVQ_MOE_OK;
    if (hipDeviceSynchronize() != hipSuccess) rc = fail(RVQ_MOE_EHIP, "hipDeviceSynchronize failed at close");
    if (rc == RVQ_MOE_OK) rc = take_device_error(h);
    free_handle(h);
    return rc;
}

extern "C" int rvq_moe_bank_layout(const rvq_moe_desc *desc, int64_t *record_stride, int64_t *payload_bytes) {
    g_err[0] = 0;
    if (!record_stride || !payload_bytes) return fail(RVQ_MOE_EINVAL, "null output pointer");
    if (const int rc = check_shape(desc)) return rc;
    const Geometry g = make_geometry(desc->d, desc->ffn, desc->n_experts, desc->top_k, desc->codebook_dtype);
    *record_stride = bank_stride(g);
    *payload_bytes = g.rec_int;
    return RVQ_MOE_OK;
}

extern "C" int rvq_moe_write_bank(const rvq_moe_desc *desc, uint8_t *bank) {
    g_err[0] = 0;
    if (const int rc = check_shape(desc)) return rc;
    const rvq_moe_desc &D = *desc;
    if (!D.codes || !bank) return fail(RVQ_MOE_EINVAL, "null codes or bank");
    if (D.codes_location != RVQ_MOE_CODES_DEVICE && D.codes_location != RVQ_MOE_CODES_PINNED_HOST)
        return fail(RVQ_MOE_EINVAL, "codes_location=%d: canonical codes are DEVICE or PINNED_HOST", D.codes_location);
    if (D.codes_location == RVQ_MOE_CODES_PINNED_HOST && !is_pinned_host(D.codes))
        return fail(RVQ_MOE_EINVAL, "PINNED_HOST codes must be pinned host memory (hipHostMalloc)");
    if (!is_pinned_host(bank)) return fail(RVQ_MOE_EINVAL, "bank must be pinned host memory (hipHostMalloc)");
    const Geometry g = make_geometry(D.d, D.ffn, D.n_experts, D.top_k, D.codebook_dtype);
    const hipError_t e = write_bank(g, D.codes, D.codes_location == RVQ_MOE_CODES_PINNED_HOST, bank,
                                    static_cast<hipStream_t>(D.stream));
    if (e != hipSuccess)
        return fail(e == hipErrorOutOfMemory ? RVQ_MOE_ENOMEM : RVQ_MOE_EHIP, "write_bank: %s", hipGetErrorString(e));
    return RVQ_MOE_OK;
}

extern "C" const char *rvq_moe_last_error(void) { return g_err; }

extern "C" int rvq_moe_abi_version(void) { return RVQ_MOE_ABI_VERSION; }

extern "C" int rvq_moe_get_stats(const rvq_moe *h, rvq_moe_stats *out) {
    if (!h || !out) return fail(RVQ_MOE_EINVAL, "null handle or out");
    *out = h->stats;
    out->h2d_bytes = h->cache.h2d_bytes;
    out->slot_hits = h->cache.hits;
    out->slot_misses = h->cache.misses;
    out->host_syncs = h->cache.syncs;
    out->prefetch_fills = h->cache.prefetch_fills;
    out->prefetch_hits = h->cache.prefetch_hits;
    out->records_checked = h->cache.records_checked;
    out->records_verified = h->cache.records_verified;
    return RVQ_MOE_OK;
}

static const char *kKindNames[RVQ_MOE_N_KERNEL_KINDS] = {"route_topk", "layer_lut", "route_layer_lut", "chunk"};

extern "C" int rvq_moe_set_profiling(rvq_moe *h, int every) {
    if (!h || every < 0) return fail(RVQ_MOE_EINVAL, "bad handle or every");
    h->prof_every = every;
    h->prof_calls = 0;
    h->prof_route_calls = 0;
    if (every > 0 && h->prof_pool.empty() && h->prof_events.empty()) {
        for (int i = 0; i < 8192; i++) {
            hipEvent_t e;
            HIP_TRY(hipEventCreate(&e));
            h->prof_pool.push_back(e);
        }
    }
    return RVQ_MOE_OK;
}

extern "C" int rvq_moe_kernel_times(rvq_moe *h, const char **names, uint64_t *launches, double *total_ms,
                                    int max_kinds) {
    if (!h || max_kinds < 0) return fail(RVQ_MOE_EINVAL, "bad handle");
    HIP_TRY(hipDeviceSynchronize());
    const int n = max_kinds < RVQ_MOE_N_KERNEL_KINDS ? max_kinds : RVQ_MOE_N_KERNEL_KINDS;
    for (int i = 0; i < n; i++) {
        if (names) names[i] = kKindNames[i];
        if (launches) launches[i] = 0;
        if (total_ms) total_ms[i] = 0.0;
    }
    for (const EventPair &p : h->prof_events) {
        float ms = 0.f;
        HIP_TRY(hipEventElapsedTime(&ms, p.a, p.b));
        if (p.kind < n) {
            if (launches) launches[p.kind]++;
            if (total_ms) total_ms[p.kind] += ms;
        }
        h->prof_pool.push_back(p.a);
        h->prof_pool.push_back(p.b);
    }
    h->prof_events.clear();
    return n;
}
