// internal.hpp -- layouts and kernel launchers shared by the library's own
// sources (api.hip, router.hip, lut.hip).  Nothing here is part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rvq {

// RVQ format ([FR] "Quantification et exactitude"): 3 stages, 256 entries, 8-wide vectors.
constexpr int kStages = 3;
constexpr int kCodes = 256;
constexpr int kVec = 8;

// Internal code layout of one RVQ matrix [rows][slices][3].
//
// The matrix is cut into tiles of kTileSlices input slices (one table lane
// per slice) and chunks of kChunkRows output rows.  A (tile, chunk) block is
// kChunkBytes contiguous bytes ordered [stage][half][lane][16]: byte i of lane
// (half h, lane l) of stage s is the stage-s code of row (chunk*32 + h*16 + i)
// and slice (tile*32 + l).  One wave64 load of 16 bytes per lane therefore
// reads 1 KB contiguous (one stage of one block).  Blocks are ordered
// tile-major: (tile * n_chunks + chunk).  Rows and slices beyond the matrix
// are zero codes whose table entries are zero (padded slices) or whose sums
// are never read (padded rows).
constexpr int kTileSlices = 32;
constexpr int kChunkRows = 32;
constexpr int kChunkBytes = kStages * kChunkRows * kTileSlices;  // 3072

struct MatGeom {
    int rows;       // output rows
    int slices;     // input slices (cols / 8)
    int n_tiles;    // ceil(slices / 32)
    int n_chunks;   // ceil(rows / 32)
    int64_t off;    // byte offset of the matrix inside an internal record
    int64_t bytes;  // n_tiles * n_chunks * 3072
};

struct Geometry {
    int d, ffn, E, k;
    MatGeom m[3];          // gate, up, down
    int64_t rec_int;       // internal record bytes
    int64_t rec_canon;     // canonical record bytes (9 d ffn / 8)
    int cb_dtype;          // 0 f32, 1 f16
    int64_t cb_bytes;      // one expert's codebooks: 3 * 3 * 256 * 8 * elem
    int ffn_pad;           // gate chunks * 32
    int d_pad;             // down chunks * 32
    int d_tpad, ffn_tpad;  // d, ffn rounded up to whole input tiles (256): row strides of the chunk
                           // path's bf16 X and H, whose pad columns are zero (cleared once, never written)
};

Geometry make_geometry(int d, int ffn, int E, int k, int cb_dtype);

// Data handed between workgroups of one launch (partial sums, logits) is
// written and read with agent-scope relaxed atomics: on gfx950 these are plain
// loads/stores with the sc1 bit, coherent across the XCDs' L2 caches per
// access, so no cache-wide writeback or invalidate (what a fence costs) is
// needed.  A producer waits for its stores to complete (vmcnt 0) before a
// counter increment publishes them.
__device__ inline void store_coherent(float *p, float v) {
    __hip_atomic_store(reinterpret_cast<uint32_t *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float load_coherent(const float *p) {
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t *>(p), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
}
__device__ inline void store_coherent(double *p, double v) {
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), __double_as_longlong(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline double load_coherent(const double *p) {
    return __longlong_as_double(
        (long long)__hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ inline int load_counter(const int *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void store_counter(int *p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's vector memory operations (including sc1 stores) completed.
__device__ inline void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Global-memory (address space 1) view of a device pointer.  Loads through a
// generic pointer that the compiler cannot place (one read from a table, such
// as a slot-cache record pointer) become flat loads, which count against the
// LDS wait counter too: every wait for an LDS result would then also wait for
// the code loads in flight.  Through this view they are global loads, waited
// for by the vector-memory counter only.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T *global_view(const T *p) {
    return (const __attribute__((address_space(1))) T *)p;
}

// Wave-wide sums without LDS round trips: DPP quad and row moves inside each
// 16-lane row, then 16- and 32-lane permlane swaps.
#define RVQ_DPP_U(v, ctrl) __builtin_amdgcn_update_dpp(0u, (v), (ctrl), 0xF, 0xF, true)
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRor4 = 0x124, kDppRor8 = 0x128;

__device__ inline double dpp_d(double v, int step) {
    const uint64_t b = __double_as_longlong(v);
    uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
    switch (step) {
        case 0: lo = RVQ_DPP_U(lo, kDppXor1); hi = RVQ_DPP_U(hi, kDppXor1); break;
        case 1: lo = RVQ_DPP_U(lo, kDppXor2); hi = RVQ_DPP_U(hi, kDppXor2); break;
        case 2: lo = RVQ_DPP_U(lo, kDppRor4); hi = RVQ_DPP_U(hi, kDppRor4); break;
        default: lo = RVQ_DPP_U(lo, kDppRor8); hi = RVQ_DPP_U(hi, kDppRor8); break;
    }
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// The other row's value after a 16-lane (rows 0<->1, 2<->3) or 32-lane swap.
__device__ inline uint32_t swap_other(uint32_t v, bool wide, bool odd) {
    if (wide) {
        auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return odd ? r[0] : r[1];
    }
    auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return odd ? r[0] : r[1];
}

__device__ inline double wave_sum(double v) {
#pragma unroll
    for (int st = 0; st < 4; st++) v += dpp_d(v, st);  // every lane: sum of its row of 16
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int w = 0; w < 2; w++) {
        const bool odd = w ? (lane & 32) : (lane & 16);
        const uint64_t b = __double_as_longlong(v);
        const uint32_t lo = swap_other((uint32_t)b, w, odd), hi = swap_other((uint32_t)(b >> 32), w, odd);
        v += __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
    }
    return v;  // identical in every lane
}


// Logit slots hold this NaN until written.  It is a signalling NaN, which no
// arithmetic result is (results are quiet NaNs at most), so a slot holds it
// exactly while its logit is not yet published.
constexpr uint64_t kUnpublished = 0x7FF4DEAD7FF4DEADull;
constexpr uint32_t kUnpublishedHalf = 0x7FF4DEADu;

// Workspace of one handle (device memory, sized for max_tokens at open).
struct Workspace {
    double *logits;     // [T][E] fp64 router logits
    double *sel;        // [T][k] fp64 logits of the selected experts, by rank
    double *route_logits;  // router logit slots (route_logit_slots()); unpublished slots hold a marker NaN:
                           // route_cap values for several tokens ([S][T][E] parts), then [2][E] logits
                           // and [2][kMaxTopK] selected logits for one token (alternating buffers)
    int64_t route_cap;     // max(max_tokens, 256) * E
    int64_t fused_cap;     // max_tokens * E: one of the two fused_logits buffers
    int route_parity;      // buffer of the next one-token call
    double *fused_logits;  // in-launch routing slots, fused_route_slots() doubles (marker NaN when unpublished)
    int fused_parity;      // buffer of the next in-launch routing
    int fused_prev_T;      // tokens of the last in-launch routing (its slots to reset)
    bool route_one;        // the one-token kernel fits (all E workgroups resident)
    float *part_gu;     // [T*k][2][n_tiles_in][ffn_pad] partial gate/up sums
    int *cnt;           // kCntSets sets of cnt_per_set counters kCntStride apart: per pair the
                        // finished gate/up chunks, then the workgroups whose initial y is out
    int cnt_per_set;    // T*k + 1
    int cnt_phase;      // set of the next layer launch (each launch zeroes the other one)
    int *err;           // device error flag: bit 0 bad id, bit 1 wait timeout
    int n_wg;           // persistent workgroups (all resident at once: blocks per CU x CUs)
    int *cb_exp;        // [E][3] scale exponents of fp32 codebook matrices (0 for fp16), set at open
    bool det;           // deterministic combine: pair outputs go to part_y, combined by k_combine
    float *part_y;      // det: [P][n_tiles of down][d_pad] output rows of each pair and down tile
};

// Chunk-path workspace (device), sized for max_tokens * k pairs.
struct ChunkWork {
    __bf16 *X;     // [T][d_tpad] tokens (normalised), bf16
    __bf16 *H;     // [P][ffn_tpad] SwiGLU outputs in expert-grouped order, bf16
    int *perm;     // [P] position -> pair
    int *grp_off;  // [E + 2] group offsets (group E: invalid ids)
    int *act;      // [E + 1] experts on the matrix cores, then their count at [E]
    int *list;     // [kPairListInts] pairs handed to the table path (see below)
    bool det;      // deterministic combine: pair outputs go to part_y [P][d_pad], combined by k_combine
    float *part_y;
    // resident codes: the kernels for experts with more than 32 tokens (few
    // workgroups, long-running) run on this stream, beside the others
    hipStream_t side;
    hipEvent_t fork, join;
};

// The table path's order table holds up to kOrderMax (token, expert) pairs.
// A pair list handed from the chunk path to it is [1 + 3 * kOrderMax] ints:
// n, then per position (pairs grouped by expert): group start | group size
// << 16, pair index, expert id.
constexpr int kOrderMax = 512;
constexpr int kPairListInts = 1 + 3 * kOrderMax;

// Per-pair completion counters sit kCntStride ints (256 B) apart: counters
// that share a cache line slow each other's atomics and polls down.
constexpr int kCntStride = 64;

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 64;
constexpr int kRouteMaxPairs = 1024;
// Routing inside the layer launch: each persistent workgroup computes the
// logits of at most this many experts (so it needs E <= kRouteExperts * grid).
constexpr int kRouteExperts = 4;
// Layer launches alternate between kCntSets counter sets.  Launch n counts in
// set n % 2 and, as each of its workgroups ends, zeroes its share of the other
// set: the set launch n - 1 used (it has completed, since launches of one
// handle are ordered on one stream) and launch n + 1 will use (it starts after
// launch n completes).  No workgroup has to count out at the end of a launch
// to find who resets the counters.  (Zeroing at the start of a launch instead
// measured 14 us slower per call on the two-call path.)
constexpr int kCntSets = 2;

// Launchers (all asynchronous on `s`; return hipError_t of the launch).
hipError_t launch_repack(const Geometry &g, const uint8_t *canon, uint8_t *internal, int n_experts,
                         hipStream_t s);
hipError_t launch_transpose(const float *W, float *Wt, int d, int E, hipStream_t s);
int64_t route_logit_slots(int64_t max_tokens, int E);
// In-launch routing slots (rvq_moe_route_forward), all doubles: logits
// [2][max_tokens][E], holding the marker until written.
inline int64_t fused_route_slots(int64_t max_tokens, int E) { return 2 * max_tokens * E; }
hipError_t init_route(Workspace &w, int E, int k, int64_t max_tokens, int n_cu, hipStream_t s);
hipError_t launch_route(const Geometry &g, Workspace &w, const float *x, const float *Wt, int T, int pre,
                        double eps, int32_t *ids, float *gates, hipStream_t s);
hipError_t layer_blocks_per_cu(int cb_dtype, int *out);
// Deterministic combine: y[t] = (x[t] when residual) + the k * slots rows
// part[(t k + j) slots + s][0 .. d) added in the order (j, s); NaN for a
// token with an id outside [0, E).  One launch after the layer's kernels.
hipError_t launch_combine(const float *part, int slots, const float *x, const int32_t *ids, float *y, int T, int k,
                          int E, int d, int d_pad, int residual, hipStream_t s);
// Static device scratch of rvq_moe_layer_forward_noalloc (noalloc.hip):
// kStaticScratchBytes per device, its address looked up once per device.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t static_scratch_setup(int device);  // the device must be current
char *static_scratch(int device);             // null before setup
hipError_t launch_zero_ints(int *p, int n, hipStream_t s);
// The table build's per-matrix scale exponents of fp32 codebooks (zeros for fp16).
hipError_t launch_cb_exponents(const void *cbs, int cb_dtype, int n_experts, int *out, hipStream_t s);
// Chunk path: prep + stage (grouping, bf16 tokens, y init), then the
// contractions for the active experts act[a0 .. a1) (a1 clipped to the number
// of active experts on the device); launch_chunk does both for all experts.
// lut_tokens: experts with fewer tokens (while their pairs fit cw.list) are
// left out of the matrix-core kernels and listed for the table path (1: none).
hipError_t launch_chunk_prep(const Geometry &g, const ChunkWork &cw, const float *x, const int32_t *ids, float *y,
                             int T, int pre, int residual, double eps, int lut_tokens, int *err, hipStream_t s);
// pairs: the call's (token, expert) pairs (chooses between the kernel families)
hipError_t launch_chunk_experts(const Geometry &g, const ChunkWork &cw, const uint8_t *codes,
                                const uint8_t *const *slot_tab, const void *cbs, const float *gates, float *y, int a0,
                                int a1, int pairs, hipStream_t s);
hipError_t launch_chunk(const Geometry &g, const ChunkWork &cw, const uint8_t *codes, const void *cbs, const float *x,
                        const int32_t *ids, const float *gates, float *y, int T, int pre, int residual, double eps,
                        int lut_tokens, int *err, hipStream_t s);
// slot_tab: null (resident codes: expert e's record at codes + e * rec_int) or
// a device table [E] of record pointers (the HBM slot cache).
// list: null, or a pair list written by the chunk path's prep (the layer then
// evaluates exactly those pairs and leaves y's initial value to that prep).
hipError_t launch_layer(const Geometry &g, Workspace &w, const uint8_t *codes, const uint8_t *const *slot_tab,
                        const void *cbs, const float *Wt, const float *x, const int32_t *ids, const float *gates,
                        float *y, int T, int pre, int residual, double eps, bool route, hipStream_t s,
                        const int *list = nullptr);

}  // namespace rvq
