// lut.hip -- expert evaluation from RVQ codes through tables of partial dot
// products held in LDS, as one persistent kernel per layer call.
//
// [FR] "Quantification et exactitude": expert weights are 3-stage residual VQ
// (256-entry codebooks, 8-dim vectors, 3.00 bits per weight); the matrix is not
// rebuilt -- a table of partial dot products is built and every row costs 3
// table lookups and 2 additions per 8-wide slice.  [RU] "Расчёт строится на
// устройстве MoE": gate, up and down of an expert lie back to back and the
// matrix is never unfolded.
//
// For an input vector v and one RVQ matrix, the table of slice j is
//     T_s[j][c] = sum_{i<8} C_s[c][i] * v[8j + i]      (s = stage, c = code)
// and row r is  sum_j T_0[j][c0(r,j)] + T_1[j][c1(r,j)] + T_2[j][c2(r,j)].
//
// MI355X mapping
// --------------
// * One workgroup (16 waves) per CU, as many as can be resident at once (LDS
//   use allows one per CU).  The call's work is two phases of 32-row chunks:
//     A  gate and up: (pair, matrix, 32-slice tile) segments x row chunks,
//     B  down:        (pair, 32-slice tile of h) segments x row chunks, each
//        row total times the routing gate added into y with fp32 atomics.
//   Each phase's chunks are split into equal contiguous ranges, one per
//   workgroup, so every CU streams the same number of code bytes.  A segment
//   whose range is cut between two workgroups is built twice (its table) but
//   read once (its codes).  Per-pair counters order A before B; launches
//   alternate between two counter sets, each zeroing the other one as it ends.
// * Table layout in LDS (128 KB), byte address for stage s, code c, lane l:
//     s = 0: c*256 + 4l;   s = 1: c*256 + 128 + 4l;   s = 2: 65536 + c*256 + 4l.
//   Lane l of each half-wave always serves slice l, so a half-wave's 32 random
//   lookups hit 32 distinct banks whatever the codes (bank-conflict free), and
//   one v_perm_b32 turns a packed code byte plus the lane base into the
//   address.  The other half of each stage-2 row holds the staged codebook.
// * Codes are read as 16-byte loads: lane (h, l) of a wave loads 16 rows of
//   slice l for one stage; a wave load is 1 KB contiguous (internal layout
//   of internal.hpp); the next chunk is prefetched while one is summed.
// * The 16 per-lane row values are summed over the 32 slice lanes by a
//   transposed butterfly: permlane16_swap for lane bit 4 (no selects), DPP
//   row rotations for bits 3 and 2, quad permutes for bits 1 and 0.
// * The SwiGLU finish h = silu(a) * b (the FFN reading of the layer) and the
//   routing gate are applied while building the down table:
//   table(g * h) = g * table(h), so phase C is a plain sum.
#include <math.h>

#include "internal.hpp"

namespace rvq {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 1024;              // threads per workgroup (16 waves)
constexpr int kWaves = kBlock / 64;
constexpr int kLutWords = 32768;          // 128 KB
constexpr int kStage2Word = 16384;        // byte 65536
constexpr int kCbHalfWord = 32;           // codebook staging: words 32..63 of each stage-2 row

// ---------------------------------------------------------------------------
// Repack: canonical [rows][slices][3] per matrix -> tiled internal layout.
// One thread writes one 16-byte unit (one lane's stage bytes of a block).
__global__ __launch_bounds__(256) void k_repack(const uint8_t *__restrict__ canon, uint8_t *__restrict__ out,
                                                Geometry g, int64_t units_per_expert, int64_t total_units) {
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= total_units) return;
    const int64_t e = u / units_per_expert;
    int64_t lu = u % units_per_expert;
    int m = 0;
    int64_t canon_off = 0;
    for (; m < 2; m++) {
        const int64_t mu = g.m[m].bytes / 16;
        if (lu < mu) break;
        lu -= mu;
        canon_off += (int64_t)g.m[m].rows * g.m[m].slices * kStages;
    }
    const MatGeom mg = g.m[m];
    const int64_t blk = lu / (kChunkBytes / 16);
    const int within = (int)(lu % (kChunkBytes / 16));
    const int tile = (int)(blk / mg.n_chunks);
    const int chunk = (int)(blk % mg.n_chunks);
    const int s = within / 64;
    const int h = (within / 32) & 1;
    const int l = within & 31;
    const int slice = tile * kTileSlices + l;
    const uint8_t *src = canon + e * g.rec_canon + canon_off;
    uint32_t wv[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
        uint32_t acc = 0;
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const int row = chunk * kChunkRows + h * 16 + q * 4 + b;
            uint32_t c = 0;
            if (row < mg.rows && slice < mg.slices) c = src[((int64_t)row * mg.slices + slice) * kStages + s];
            acc |= c << (8 * b);
        }
        wv[q] = acc;
    }
    uint4 *dst = reinterpret_cast<uint4 *>(out + e * g.rec_int + mg.off + blk * kChunkBytes) + within;
    *dst = make_uint4(wv[0], wv[1], wv[2], wv[3]);
}

hipError_t launch_repack(const Geometry &g, const uint8_t *canon, uint8_t *internal, int n_experts,
                         hipStream_t s) {
    const int64_t upe = g.rec_int / 16;
    const int64_t total = upe * n_experts;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(k_repack, dim3((unsigned)blocks), dim3(256), 0, s, canon, internal, g, upe, total);
    return hipGetLastError();
}

// The wave's index in the workgroup as a wave-uniform value (scalar register),
// so that loops and branches on it are scalar.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------------------
// LDS helpers
__device__ inline float lds_at(const float *lut, uint32_t byte_addr) {
    return *reinterpret_cast<const float *>(reinterpret_cast<const char *>(lut) + byte_addr);
}

__device__ inline int lut_word(int s, int c, int l) {
    return (s == 2 ? kStage2Word : 0) + c * 64 + (s == 1 ? 32 : 0) + l;
}

// Stage one matrix's codebook ([3][256][8] entries) into the free halves of the
// stage-2 rows: entry idx (0..767) goes to row idx / R, slot idx % R, where a
// 128-byte half row holds R = 128 / entry_bytes entries.  Split into a global
// load into registers (issued one segment ahead) and an LDS store.
template <int CB>
struct CbRegs {
    static constexpr int kEntryBytes = CB == 0 ? 32 : 16;
    static constexpr int kUnits = kStages * kCodes * kEntryBytes / 16;  // 16-byte units
    static constexpr int kRegs = (kUnits + kBlock - 1) / kBlock;
    uint4 r[kRegs];
    int ec;  // fp32 codebooks: the matrix's scale exponent (see build_lut)
};

template <int CB>
__device__ inline void cb_load(CbRegs<CB> &cr, const void *cbs, const int *cb_exp, int64_t e, int m) {
    using C = CbRegs<CB>;
    cr.ec = CB == 0 ? cb_exp[e * 3 + m] : 0;
    const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const char *>(cbs) +
                                                       (e * 3 + m) * (int64_t)kStages * kCodes * C::kEntryBytes);
#pragma unroll
    for (int k = 0; k < C::kRegs; k++) {
        const int u = threadIdx.x + k * kBlock;
        if (u < C::kUnits) cr.r[k] = src[u];
    }
}

template <int CB>
__device__ inline void cb_store(float *lut, const CbRegs<CB> &cr) {
    using C = CbRegs<CB>;
    constexpr int kPerRow = 128 / C::kEntryBytes;
#pragma unroll
    for (int k = 0; k < C::kRegs; k++) {
        const int u = threadIdx.x + k * kBlock;
        if (u < C::kUnits) {
            const int entry = u / (C::kEntryBytes / 16), part = u % (C::kEntryBytes / 16);
            const int row = entry / kPerRow, slot = entry % kPerRow;
            uint4 *dst = reinterpret_cast<uint4 *>(lut + kStage2Word + row * 64 + kCbHalfWord) +
                         slot * (C::kEntryBytes / 16) + part;
            *dst = cr.r[k];
        }
    }
}

// Build the table of one 32-slice tile on the matrix cores.  The table is the
// product of the staged codebook C [768 codes x 8] with the slice inputs
// vs [8][32 slices] (element-major, so each lane's reads are bank-conflict free) -- an exact dense contraction -- done as
// 24 blocks of 32 codes x 32 slices with v_mfma_f32_32x32x16_f16 (fp32
// accumulation).  The fp32 inputs are split v = v_hi + v_lo into two fp16
// parts fed as the two K halves (lanes 0-31 carry v_hi, lanes 32-63 v_lo,
// against the same codebook entry), so one instruction forms C.v_hi + C.v_lo,
// within ~2^-22 of C.v; fp16 codebooks are exact, fp32 codebooks get a second
// pass with their own low part.  The inputs are first scaled by 2^-e2 so the
// largest is near 2^14 (no fp16 overflow, negligible underflow) and the table
// is scaled back by 2^e2, both exact.  Operand layout (wave64, verified):
// element j of lane l pairs A[l % 32] with B column l % 32 within the lane
// half l / 32; accumulator v of lane l is D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

//
// fp32 codebooks are first scaled by 2^-ec, ec being the exponent of their
// matrix's largest finite entry (cb_exponent(), computed once at open), so that
// entry lies in [2^13, 2^14) as well: the hi + lo split then keeps ~22 bits of
// every entry whatever the codebook's scale (no fp16 overflow above 65504, no
// loss to fp16 subnormals for small codebooks); the table is scaled back by
// 2^(e2 + ec).  All scalings are v_ldexp (exact, no overflow of a scale factor).
template <int CB>
__device__ inline void build_lut(float *lut, const float (*vs)[kTileSlices], int e2, int ec) {
    constexpr int kEntryBytes = CB == 0 ? 32 : 16;
    constexpr int kPerRow = 128 / kEntryBytes;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int j = lane & 31, kh = lane >> 5;
    const int back = e2 + (CB == 0 ? ec : 0);
    // all eight reads go out before any conversion (one LDS wait, not four)
    float vin[kVec];
#pragma unroll
    for (int i = 0; i < kVec; i++) vin[i] = vs[i][j];
    __builtin_amdgcn_sched_barrier(0);
    half8 bop;
#pragma unroll
    for (int i = 0; i < kVec; i++) {
        const float v = __builtin_amdgcn_ldexpf(vin[i], -e2);
        const _Float16 hi = (_Float16)v;
        bop[i] = kh ? (_Float16)(v - (float)hi) : hi;
    }
    // 24 blocks over 16 waves: waves 0-7 take two, whose operand reads and
    // products are issued before either block's table writes
    constexpr int kBlocks = kStages * kCodes / 32;
    static_assert(kBlocks <= 2 * kWaves, "at most two blocks per wave");
    auto block = [&](int mb) {
        const int s = mb >> 3, c0 = (mb & 7) * 32;
        const int idx = s * kCodes + c0 + j;
        const char *p = reinterpret_cast<const char *>(lut + kStage2Word + (idx / kPerRow) * 64 + kCbHalfWord) +
                        (idx % kPerRow) * kEntryBytes;
        f32x16 acc = {};
        if (CB == 1) {
            const half8 aop = *reinterpret_cast<const half8 *>(p);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop, bop, acc, 0, 0, 0);
        } else {
            const float4 w0 = reinterpret_cast<const float4 *>(p)[0], w1 = reinterpret_cast<const float4 *>(p)[1];
            const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
            half8 ahi, alo;
#pragma unroll
            for (int i = 0; i < kVec; i++) {
                const float ws = __builtin_amdgcn_ldexpf(w[i], -ec);
                ahi[i] = (_Float16)ws;
                alo[i] = (_Float16)(ws - (float)ahi[i]);
            }
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, bop, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo, bop, acc, 0, 0, 0);
        }
        return acc;
    };
    auto store = [&](int mb, const f32x16 &acc) {
        const int s = mb >> 3, c0 = (mb & 7) * 32;
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int c = c0 + 8 * (v >> 2) + 4 * kh + (v & 3);
            lut[lut_word(s, c, j)] = __builtin_amdgcn_ldexpf(acc[v], back);
        }
    };
    const int mb0 = wave, mb1 = wave + kWaves;  // wave-uniform
    if (mb0 < kBlocks) {
        const f32x16 acc0 = block(mb0);
        if (mb1 < kBlocks) {
            const f32x16 acc1 = block(mb1);
            store(mb0, acc0);
            store(mb1, acc1);
        } else {
            store(mb0, acc0);
        }
    }
}

// Exponent e2 with max|v| * 2^-e2 in [2^13, 2^14) over the tile's 256 inputs
// (0 when all are zero or not finite).  The four waves that hold the inputs
// (threads 0..255) each publish their maximum with tile_max_publish() before
// the barrier that follows the vs stores; tile_exponent() reads the four
// maxima after it, so the exponent costs no barrier of its own.
__device__ __forceinline__ void tile_max_publish(float v, float *red2);

__device__ __forceinline__ int tile_exponent(const float *red2) {
    const float m = fmaxf(fmaxf(red2[0], red2[1]), fmaxf(red2[2], red2[3]));
    if (!(m > 0.f) || !isfinite(m)) return 0;
    int ex;
    frexpf(m, &ex);  // m = f * 2^ex, f in [0.5, 1)
    return ex - 14;
}

// Exponent ec of each fp32 codebook matrix (all three stages of one expert's
// gate, up or down): max|entry| * 2^-ec in [2^13, 2^14) over its finite
// entries (0 when all are zero or not finite).  One workgroup per matrix.
__global__ __launch_bounds__(256) void k_cb_exponent(const float *__restrict__ cbs, int n_mats,
                                                     int *__restrict__ out) {
    const float *c = cbs + (size_t)blockIdx.x * kStages * kCodes * kVec;
    float m = 0.f;
    for (int i = threadIdx.x; i < kStages * kCodes * kVec; i += 256) {
        const float v = fabsf(c[i]);
        if (isfinite(v)) m = fmaxf(m, v);
    }
    __shared__ float red[256];
    red[threadIdx.x] = m;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        int ex = 0;
        if (red[0] > 0.f) {
            frexpf(red[0], &ex);
            ex -= 14;
        }
        out[blockIdx.x] = ex;
    }
}

hipError_t launch_cb_exponents(const void *cbs, int cb_dtype, int n_experts, int *out, hipStream_t s) {
    if (cb_dtype != 0) return hipMemsetAsync(out, 0, sizeof(int) * 3 * (size_t)n_experts, s);
    hipLaunchKernelGGL(k_cb_exponent, dim3(3 * n_experts), dim3(256), 0, s, static_cast<const float *>(cbs),
                       3 * n_experts, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Cross-lane helpers (wave64, DPP rows of 16 lanes).
#define RVQ_DPP(v, ctrl) __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), (ctrl), 0xF, 0xF, true))
constexpr int kRor4 = 0x124, kRor8 = 0x128, kRor12 = 0x12C;
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]

// Maximum of |v| over the wave: quad and row rotations give every lane its
// 16-lane row's maximum, then the four rows are read as scalars.
__device__ __forceinline__ void tile_max_publish(float v, float *red2) {
    float m = fabsf(v);
    m = fmaxf(m, RVQ_DPP(m, kQuadXor1));
    m = fmaxf(m, RVQ_DPP(m, kQuadXor2));
    m = fmaxf(m, RVQ_DPP(m, kRor4));
    m = fmaxf(m, RVQ_DPP(m, kRor8));
    const int mi = __float_as_int(m);
    const float r = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(mi, 0)),
                                __int_as_float(__builtin_amdgcn_readlane(mi, 16))),
                          fmaxf(__int_as_float(__builtin_amdgcn_readlane(mi, 32)),
                                __int_as_float(__builtin_amdgcn_readlane(mi, 48))));
    if ((threadIdx.x & 63) == 0) red2[threadIdx.x >> 6] = r;
}

// Sum 16 row values over the 32 slice lanes of each half-wave.  On return the
// lane pair (2r, 2r+1) of a half holds the total of that half's row r.
__device__ __forceinline__ float reduce16(float (&v)[16], int l) {
    // lane bit 4: swap odd DPP rows of v[i] with even rows of v[i+8]
#pragma unroll
    for (int i = 0; i < 8; i++) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 8]), false, false);
        v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    // lane bit 3: partner l ^ 8 (row rotate by 8)
    const bool b3 = l & 8, b2 = l & 4, b1 = l & 2;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float lo = v[i] + RVQ_DPP(v[i], kRor8);
        const float hi = v[i + 4] + RVQ_DPP(v[i + 4], kRor8);
        v[i] = b3 ? hi : lo;
    }
    // lane bit 2: partner l ^ 4 (rotate by 12 for bit2 = 0 lanes, by 4 otherwise)
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const float lo = v[i] + RVQ_DPP(v[i], kRor12);
        const float hi = v[i + 2] + RVQ_DPP(v[i + 2], kRor4);
        v[i] = b2 ? hi : lo;
    }
    // lane bit 1
    {
        const float lo = v[0] + RVQ_DPP(v[0], kQuadXor2);
        const float hi = v[1] + RVQ_DPP(v[1], kQuadXor2);
        v[0] = b1 ? hi : lo;
    }
    // lane bit 0
    return v[0] + RVQ_DPP(v[0], kQuadXor1);
}

// Sum one 32-row chunk whose stage words are q0, q1, q2 (this lane's 16 rows).
// The 48 table reads go out in batches of 12 (4 rows), each batch issued
// before the previous one is summed, so a wave waits for LDS a few times per
// chunk instead of once or twice per row (scheduling groups: mask 2 = VALU,
// 0x100 = LDS read).
__device__ __forceinline__ float sum_chunk(const float *lut, const u32x4 &q0, const u32x4 &q1, const u32x4 &q2, int l) {
    const uint32_t lb0 = 4u * l, lb1 = 128u + 4u * l, lb2 = 0x10000u + 4u * l;
    float t[48];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const uint32_t sel = 0x0C060004u | ((uint32_t)(i & 3) << 8);
        const int w = i >> 2;
        t[3 * i] = lds_at(lut, __builtin_amdgcn_perm(lb0, q0[w], sel));
        t[3 * i + 1] = lds_at(lut, __builtin_amdgcn_perm(lb1, q1[w], sel));
        t[3 * i + 2] = lds_at(lut, __builtin_amdgcn_perm(lb2, q2[w], sel));
    }
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; i++) v[i] = t[3 * i] + t[3 * i + 1] + t[3 * i + 2];
    __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
    return reduce16(v, l);
}

// nt: streaming (non-temporal) loads, for codes no later segment of the call
// re-reads; otherwise ordinary loads, so that the next token of an expert group
// finds the tile in L2 or the Infinity Cache.
__device__ __forceinline__ void load_chunk(const uint8_t *blk, int lane, u32x4 &q0, u32x4 &q1, u32x4 &q2, bool nt) {
    const auto *p = global_view(reinterpret_cast<const u32x4 *>(blk)) + lane;
    if (nt) {  // uniform branch
        q0 = __builtin_nontemporal_load(p);
        q1 = __builtin_nontemporal_load(p + 64);
        q2 = __builtin_nontemporal_load(p + 128);
    } else {
        q0 = p[0];
        q1 = p[64];
        q2 = p[128];
    }
}

// Row totals of the chunks being gathered are staged in LDS: chunk i of a
// sub-range owns piece i, 32 floats, at base + i * stride.  Keeping global
// stores out of the gather loop keeps their completion off its critical path;
// flush_rows() writes a whole sub-range with coalesced coherent stores.  Two
// areas serve: the free halves of the stage-2 rows (the codebook staging area,
// idle once the table is built; 256 pieces), and a separate 64-piece area,
// which lets a segment's flush wait until the next segment's table build
// (the codebook of that segment is staged meanwhile).
struct Stage {
    float *base;
    int stride, cap;  // floats from one piece to the next; pieces held
    bool acc = false;  // add into the staged totals instead of replacing them
    __device__ float *piece(int i) const { return base + i * stride; }
};
constexpr int kStagePieces = 256;
__device__ __forceinline__ Stage cb_area_stage(float *lut) { return {lut + kStage2Word + kCbHalfWord, 64, kStagePieces}; }

// Gather chunks [c0, c1) (c1 - c0 <= st.cap) of one tile, waves
// round-robin.  The first chunk of this wave was already loaded into s0 by the
// caller.  Two register sets alternate (no copies between them): the next
// chunk's loads are issued before the current chunk is summed.  The loads are
// unconditional -- past this wave's last chunk they re-read that chunk (a cache
// hit) -- so every wait is a fixed count of the in-order vector-memory counter.
// A scheduling barrier keeps each load ahead of the sum that follows it.
__device__ __forceinline__ void gather_range(float *lut, const Stage &st, const uint8_t *tile_base, int c0, int c1,
                                             const u32x4 (&s0)[3], bool nt) {
    const int lane = threadIdx.x & 63, wave = wave_id(), l = lane & 31;
    const int row_in = (lane >> 5) * 16 + (l >> 1);
    int q = c0 + wave;
    if (q >= c1) return;
    const int last = c1 - 1 - (c1 - 1 - q) % kWaves;  // this wave's last chunk
    auto at = [&](int qq) { return tile_base + (int64_t)min(qq, last) * kChunkBytes; };
    auto emit = [&](int qq, const u32x4 (&r)[3]) {
        const float sum = sum_chunk(lut, r[0], r[1], r[2], l);
        if (!(lane & 1)) {
            float *q = st.piece(qq - c0) + row_in;
            *q = st.acc ? *q + sum : sum;  // wave-uniform choice
        }
    };
    u32x4 a[3] = {s0[0], s0[1], s0[2]}, b[3];
    while (true) {
        load_chunk(at(q + kWaves), lane, b[0], b[1], b[2], nt);
        __builtin_amdgcn_sched_barrier(0);
        emit(q, a);
        if ((q += kWaves) > last) return;
        load_chunk(at(q + kWaves), lane, a[0], a[1], a[2], nt);
        __builtin_amdgcn_sched_barrier(0);
        emit(q, b);
        if ((q += kWaves) > last) return;
    }
}

// Write the staged row totals of chunks [c0, c1) to out[c0*32 ..): all threads,
// after a barrier; coherent stores, completed before the segment is signalled.
__device__ __forceinline__ void flush_rows(const Stage &st, float *out, int c0, int c1) {
    const int n = (c1 - c0) * kChunkRows;
    for (int i = threadIdx.x; i < n; i += kBlock)
        store_coherent(out + c0 * kChunkRows + i, st.piece(i / kChunkRows)[i % kChunkRows]);
}

// flush_rows for accumulated totals staged at absolute chunk positions
// (base + chunk * 32): writes chunks [c0, c1) to out and puts zeros back in
// their place (each element is read and cleared by the same thread).
__device__ __forceinline__ void flush_rows_clear(float *base, float *out, int c0, int c1) {
    for (int i = c0 * kChunkRows + threadIdx.x; i < c1 * kChunkRows; i += kBlock) {
        const float v = base[i];
        base[i] = 0.f;
        store_coherent(out + i, v);
    }
}

// Add the staged row totals of chunks [c0, c1) into out[row] (rows < n_rows)
// with device-scope fp32 atomics (the hardware global_atomic_add_f32).
__device__ __forceinline__ void flush_rows_add(const Stage &st, float *out, int c0, int c1, int n_rows) {
    const int n = (c1 - c0) * kChunkRows;
    for (int i = threadIdx.x; i < n; i += kBlock) {
        const int row = c0 * kChunkRows + i;
        if (row < n_rows) unsafeAtomicAdd(out + row, st.piece(i / kChunkRows)[i % kChunkRows]);
    }
}

// Whole segment: gather [c0, c1) in sub-ranges of at most st.cap chunks,
// flushing each -- except, with kDeferLast, the last one, whose first chunk is
// returned: its totals stay staged for the caller to flush after a barrier.
// p holds this wave's first chunk of the segment.
template <bool kAdd, bool kDeferLast>
__device__ __forceinline__ int gather_segment(float *lut, const Stage &st, const uint8_t *tile_base, int c0, int c1,
                                              float *out, int n_rows, u32x4 (&p)[3], bool nt) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    for (int s0 = c0;; s0 += st.cap) {
        const int s1 = min(c1, s0 + st.cap);
        if (s0 != c0 && s0 + wave < s1)
            load_chunk(tile_base + (int64_t)(s0 + wave) * kChunkBytes, lane, p[0], p[1], p[2], nt);
        gather_range(lut, st, tile_base, s0, s1, p, nt);
        if (kDeferLast && s1 == c1) return s0;
        __syncthreads();
        if (kAdd)
            flush_rows_add(st, out, s0, s1, n_rows);
        else
            flush_rows(st, out, s0, s1);
        __syncthreads();
        if (s1 == c1) return c1;
    }
}

// ---------------------------------------------------------------------------
// Inter-workgroup ordering (all workgroups are resident together).  A producer
// waits for its stores to complete (vmcnt 0), then a barrier, then one thread
// adds to a counter; consumers wait on the counter.
//
// Poll until *cnt >= target (one lane), one load at a time with a short sleep
// (more polls in flight slow the counter's own atomics down).  Bounded: after
// ~0.5 s the error flag gets bit 2 and the poll gives up, so every wave
// reaches the end of the kernel.
__device__ inline void poll_count(const int *cnt, int target, int *err) {
    const uint64_t t0 = wall_clock64();
    while (load_counter(cnt) < target) {
        __builtin_amdgcn_s_sleep(2);
        if (wall_clock64() - t0 > 50000000ull) {
            atomicOr(err, 2);
            return;
        }
    }
}

// Wait until *cnt >= target.  Consumers read the published data with coherent
// loads after the barrier.
__device__ inline void wait_count(const int *cnt, int target, int *err) {
    if (threadIdx.x == 0) poll_count(cnt, target, err);
    __syncthreads();
}

// ---------------------------------------------------------------------------
struct LayerArgs {
    // routing inside the launch (rvq_moe_route_forward); unused otherwise
    const float *Wt;    // [E][d] transposed router
    double *logits;     // [T][E]
    double *sel;        // [T][k] selected logits by rank
    int *ycnt;          // workgroups whose initial y stores are out (this launch's counter set)
    int *cnt_clear;     // the other counter set, zeroed as this launch ends: n_clear counters kCntStride apart
    int n_clear;
    double *rl_cur, *rl_next;  // [T][E] logit slots of this launch and of the next (in-launch routing)
    int T_reset;               // tokens of the previous routed launch (its slots in the `next` buffer)
    const int *list;    // pairs handed over by the chunk path (n, then the order table), or null
    const uint8_t *codes;
    const uint8_t *const *slot_tab;  // [E] record of each expert (HBM slot cache), or null: codes + e * rec
    const void *cbs;
    const int *cb_exp;  // [E][3] scale exponents of fp32 codebooks (see build_lut)
    const float *x;
    const int32_t *ids;
    const float *gates;
    float *y;
    float *part_gu;  // [P][2][n_ti][ffn_pad]
    int *cntA;       // this launch's set: finished gate/up chunks of pair p at p * kCntStride
    float *part_y;   // deterministic combine: [P][n_tf][d_pad] output rows per pair and down tile, else null
    int *err;
    Geometry g;
    int T;
    int pre;
    int residual;
    double eps;
};

// Internal code record of expert e (its slot when the codes stream through
// the HBM slot cache).
__device__ inline const uint8_t *expert_record(const LayerArgs &a, int e) {
    return a.slot_tab ? a.slot_tab[e] : a.codes + (int64_t)e * a.g.rec_int;
}

// x_hat scale of token t: r = sqrt(mean(x^2) + eps) in fp64 (1 without
// normalisation); cached per workgroup for the last token asked.
__device__ inline double token_r(const LayerArgs &a, int t, int &r_tok, double &r_val, double *red) {
    if (!a.pre) return 1.0;
    if (r_tok == t) return r_val;
    const float *xt = a.x + (size_t)t * a.g.d;
    double ss = 0.0;
    for (int i = threadIdx.x; i < a.g.d; i += kBlock) ss = fma((double)xt[i], (double)xt[i], ss);
    ss = wave_sum(ss);  // DPP and lane swaps: no LDS round trips
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; w++) tot += red[w];
    __syncthreads();
    r_tok = t;
    r_val = sqrt(tot / (double)a.g.d + a.eps);
    return r_val;
}

// Merged gate/up partial sums.  In the one-token (pair) order, a workgroup
// whose range holds consecutive whole tiles of one (pair, matrix) adds their
// row totals up in LDS and writes the sum once, into the slot of the run's
// last tile; a tile cut by a range boundary keeps its own slot, each side
// writing its rows.  Tile t's slot is then empty exactly when t and t + 1 lie
// whole in one workgroup's range: with u0 the first unit of tile t, that is
// when the range holding u0 (the largest r with floor(nA r / G) <= u0) ends
// at or after u0 + 2 n_cf.  Both phases decide this the same way.
__device__ inline bool merged_away(int64_t nA, int G, int64_t u0, int n_cf, bool last_tile) {
    if (last_tile) return false;
    const int64_t r0 = ((u0 + 1) * G + nA - 1) / nA - 1;
    return nA * (r0 + 1) / G >= u0 + 2 * (int64_t)n_cf;
}

// Input tiles of a gate/up matrix are at most 65536 / 8 / 32 = 256 (d <=
// 65536): the valid-slot masks take kMaskWords 64-bit words per matrix.
constexpr int kMaskWords = 4;

// h' = gate * silu(a) * b for the 256 FFN entries of down tile ft of pair p,
// where a and b are the gate and up row sums (sum over the input tiles' partial
// sums; only the slots vmask marks hold one, see merged_away).
__device__ inline void finish_h(const LayerArgs &a, const float *gate_src, int p, int ft, float (*vs)[kTileSlices],
                                float *red2, const uint64_t (*vmask)[kMaskWords]) {
    // threads 0..255, one entry each: the valid slots in batches of 16 per
    // matrix, every load of a batch in flight together
    const Geometry &g = a.g;
    const int n_ti = g.m[0].n_tiles;
    if (threadIdx.x >= 256) return;
    const int fi = threadIdx.x;
    const int f = ft * kTileSlices * kVec + fi;
    float sa = 0.f, sb = 0.f;
    if (f < g.ffn) {
        const float *pa = a.part_gu + ((int64_t)p * 2) * n_ti * g.ffn_pad + f;
        const float *pb = pa + (int64_t)n_ti * g.ffn_pad;
        // vmask[m][w] bit t: tile 64 w + t's partial slot holds a sum (not
        // merged into a later tile's slot by the workgroup that covered both)
        const int n_words = (n_ti + 63) / 64;
        for (int w = 0; w < n_words; w++) {  // uniform
            uint64_t ma = vmask[0][w], mb = vmask[1][w];
            while (ma | mb) {  // uniform
                float va[16], vb[16];
#pragma unroll
                for (int j = 0; j < 16; j++) {
                    const int ta = ma ? 64 * w + __builtin_ctzll(ma) : -1, tb = mb ? 64 * w + __builtin_ctzll(mb) : -1;
                    ma &= ma - 1;
                    mb &= mb - 1;
                    va[j] = ta >= 0 ? load_coherent(pa + (int64_t)ta * g.ffn_pad) : 0.f;
                    vb[j] = tb >= 0 ? load_coherent(pb + (int64_t)tb * g.ffn_pad) : 0.f;
                }
#pragma unroll
                for (int j = 0; j < 16; j++) {
                    sa += va[j];
                    sb += vb[j];
                }
            }
        }
    }
    float hv = 0.f;
    if (f < g.ffn) hv = gate_src[p] * (sa / (1.f + expf(-sa)) * sb);
    vs[fi % kVec][fi / kVec] = hv;
    tile_max_publish(hv, red2);
}

// A phase-A segment: chunks [c0, c1) of one (pair, matrix, tile); e = expert id;
// (gs, gn, j): its group's first position and size, and its position in it.
struct SegA {
    int p, m, tile, c0, c1, e, gs, gn, j;
};
// A phase-B segment: chunks [c0, c1) of one (pair, ffn tile).
struct SegB {
    int p, ft, c0, c1, e, gs, gn, j;
};

// Order of the (token, expert) pairs inside a call (the token x expert
// permutation).  The phases walk groups of positions.  With the order table
// (T > 1 and P <= kOrderMax), positions are pairs sorted by (expert, pair)
// and a group is every pair routed to one expert, so a group's tokens stream
// the same code tile one after another (re-reads hit L2 / the Infinity Cache:
// each expert's codes come from HBM about once per call).  Without it (one
// token, or large P), every pair is its own group in pair order.  Every
// workgroup derives the same table, deterministically, in LDS.
constexpr int kIdCache = 128;
struct Order {
    bool tab;
    const int *info;      // [P] position -> group start | group size << 16
    const int *pair;      // [P] position -> pair
    const short *expert;  // [P] position -> expert id (may be out of range)
    // without the table: expert ids of the positions a workgroup touches
    int a_base, a_n, b_base, b_n;
    const int *lds;  // [2][kIdCache]
    const int *all;  // [P] ids of every pair in LDS (routed in this launch), or null
    const int32_t *ids;
    // (LDS reads give per-lane registers; the values are uniform, so they are
    // moved to scalar registers and the segment arithmetic stays scalar)
    __device__ void group(int q, int &gs, int &gn) const {
        if (tab) {
            const int v = __builtin_amdgcn_readfirstlane(info[q]);
            gs = v & 0xffff;
            gn = v >> 16;
        } else {
            gs = q;
            gn = 1;
        }
    }
    __device__ int pair_at(int pos) const { return tab ? __builtin_amdgcn_readfirstlane(pair[pos]) : pos; }
    __device__ int expert_a(int pos) const {
        return __builtin_amdgcn_readfirstlane(
            tab ? expert[pos] : (all ? all[pos] : ((pos - a_base) < a_n ? lds[pos - a_base] : ids[pos])));
    }
    __device__ int expert_b(int pos) const {
        return __builtin_amdgcn_readfirstlane(
            tab ? expert[pos]
                : (all ? all[pos] : ((pos - b_base) < b_n ? lds[kIdCache + pos - b_base] : ids[pos])));
    }
};

// Build the order table in LDS (all threads).  tmp: scratch of at least
// (E + 1) * (kOrderMax / 64) * 8 + 2 * (E + 1) * 4 bytes (the table area, idle
// here).  Ids outside [0, E) form a last group of their own.
__device__ void build_order(const int32_t *ids, const int *lds_ids, int P, int E, char *tmp, int *info, int *pair,
                            short *expert) {
    constexpr int kW = kOrderMax / 64;
    const int NE = E + 1;
    uint64_t *mask = reinterpret_cast<uint64_t *>(tmp);  // [NE][kW] pair bitmask per expert
    int *cnt = reinterpret_cast<int *>(mask + (size_t)NE * kW);
    int *off = cnt + NE;
    for (int i = threadIdx.x; i < NE * kW; i += kBlock) mask[i] = 0;
    for (int i = threadIdx.x; i < NE; i += kBlock) cnt[i] = 0;
    __syncthreads();
    for (int p = threadIdx.x; p < P; p += kBlock) {
        int e = lds_ids ? lds_ids[p] : load_counter(ids + p);
        if (e < 0 || e >= E) e = E;
        atomicOr(reinterpret_cast<unsigned long long *>(mask + (size_t)e * kW + (p >> 6)), 1ull << (p & 63));
        atomicAdd(cnt + e, 1);
        expert[p] = (short)e;  // temporarily indexed by pair
    }
    __syncthreads();
    if (threadIdx.x < 64) {  // exclusive scan of cnt[0..NE) by one wave
        const int lane = threadIdx.x, per = (NE + 63) / 64;
        int sum = 0;
        for (int i = lane * per; i < min(NE, (lane + 1) * per); i++) sum += cnt[i];
        int incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o);
            if (lane >= o) incl += v;
        }
        int run = incl - sum;
        for (int i = lane * per; i < min(NE, (lane + 1) * per); i++) {
            off[i] = run;
            run += cnt[i];
        }
    }
    __syncthreads();
    int my_e[(kOrderMax + kBlock - 1) / kBlock];
    int my_pos[(kOrderMax + kBlock - 1) / kBlock];
#pragma unroll
    for (int r = 0; r < (kOrderMax + kBlock - 1) / kBlock; r++) {
        const int p = threadIdx.x + r * kBlock;
        my_e[r] = my_pos[r] = -1;
        if (p < P) {
            const int e = expert[p];
            const uint64_t *m = mask + (size_t)e * kW;
            int rank = __popcll(m[p >> 6] & ((1ull << (p & 63)) - 1));
            for (int w = 0; w < (p >> 6); w++) rank += __popcll(m[w]);
            my_e[r] = e;
            my_pos[r] = off[e] + rank;
        }
    }
    __syncthreads();  // all reads of expert[] by pair done before it is rewritten by position
#pragma unroll
    for (int r = 0; r < (kOrderMax + kBlock - 1) / kBlock; r++) {
        const int p = threadIdx.x + r * kBlock;
        if (p < P) {
            const int e = my_e[r], pos = my_pos[r];
            pair[pos] = p;
            expert[pos] = (short)e;
            info[pos] = off[e] | (cnt[e] << 16);
        }
    }
    __syncthreads();
}

// First unit of range r when n units are split over G workgroups.
__device__ inline int range_lo(int n, int r, int G) { return (int)((int64_t)n * r / G); }

// How a phase's units reach the workgroups.  Contiguous: one range each (range
// index rw, consecutive ranges on one XCD).  Strided, for the grouped orders:
// the units form blocks -- all chunks of one (pair, matrix tile), one table
// each -- and each XCD takes a contiguous eighth of the blocks and deals them
// round-robin to its workgroups.  The blocks of an expert group's tokens are
// consecutive, so those tokens stream the same code tile at the same time on
// one XCD and the re-reads hit its L2 (with contiguous ranges each workgroup
// re-reads a 192-672 KB tile after its XCD has streamed ~32 such tiles, more
// than the L2 holds).  Taken when every workgroup gets at least 4 blocks.
struct Deal {
    bool strided = false;
    int blk = 0, blk1 = 0, step = 1, n_c = 1;
    // the first span [u, u1) of this workgroup
    __device__ void start(bool grouped, int n_blocks, int n_chunks, int rw, int &u, int &u1) {
        const int G = gridDim.x, wg = blockIdx.x;
        strided = grouped && G % 8 == 0 && n_blocks >= 4 * G;
        if (strided) {
            n_c = n_chunks;
            step = G / 8;
            blk = range_lo(n_blocks, wg % 8, 8) + wg / 8;
            blk1 = range_lo(n_blocks, wg % 8 + 1, 8);
            u = blk * n_c;
            u1 = blk < blk1 ? u + n_c : u;
        } else {
            const int n = n_blocks * n_chunks;
            u = range_lo(n, rw, G);
            u1 = range_lo(n, rw + 1, G);
        }
    }
    // after the span ended: the next one (strided), or false
    __device__ bool next(int &u, int &u1) {
        if (!strided || (blk += step) >= blk1) return false;
        u = blk * n_c;
        u1 = u + n_c;
        return true;
    }
};

// Work units (one chunk of one pair's matrix tile) are numbered in 32 bits:
// a call has fewer than 2^31 of them (checked when the handle is opened).
__device__ inline SegA seg_a(int u, int u1, int n_ti, int n_cf, const Order &o) {
    SegA s;
    const int per = 2 * n_ti * n_cf;
    int gs, gn;
    o.group(u / per, gs, gn);
    int w = u - gs * per;
    s.c0 = w % n_cf;
    w /= n_cf;
    const int j = w % gn;
    w /= gn;
    s.tile = w % n_ti;
    s.m = w / n_ti;
    s.c1 = min(n_cf, s.c0 + (u1 - u));
    s.gs = gs;
    s.gn = gn;
    s.j = j;
    s.p = o.pair_at(gs + j);
    s.e = o.expert_a(gs + j);
    return s;
}

// The segment after c, which ended at its tile's last chunk, starting at unit un
// (< u1): the same decomposition as seg_a, stepped (chunk, then position in
// the group, then tile, then matrix, then group) without divisions.
__device__ inline SegA next_a(const SegA &c, int un, int u1, int n_ti, int n_cf, const Order &o) {
    SegA s = c;
    s.c0 = 0;
    s.c1 = min(n_cf, u1 - un);
    if (++s.j == s.gn) {
        s.j = 0;
        if (++s.tile == n_ti) {
            s.tile = 0;
            if (++s.m == 2) {
                s.m = 0;
                o.group(c.gs + c.gn, s.gs, s.gn);
            }
        }
    }
    s.p = o.pair_at(s.gs + s.j);
    s.e = o.expert_a(s.gs + s.j);
    return s;
}

__device__ inline SegB seg_b(int u, int u1, int n_tf, int n_cd, const Order &o) {
    SegB s;
    const int per = n_tf * n_cd;
    int gs, gn;
    o.group(u / per, gs, gn);
    int w = u - gs * per;
    s.c0 = w % n_cd;
    w /= n_cd;
    const int j = w % gn;
    s.ft = w / gn;
    s.c1 = min(n_cd, s.c0 + (u1 - u));
    s.gs = gs;
    s.gn = gn;
    s.j = j;
    s.p = o.pair_at(gs + j);
    s.e = o.expert_b(gs + j);
    return s;
}

// The phase-B segment after c (which ended at its tile's last chunk): chunk,
// then position in the group, then ffn tile, then group.
__device__ inline SegB next_b(const SegB &c, int un, int u1, int n_tf, int n_cd, const Order &o) {
    SegB s = c;
    s.c0 = 0;
    s.c1 = min(n_cd, u1 - un);
    if (++s.j == s.gn) {
        s.j = 0;
        if (++s.ft == n_tf) {
            s.ft = 0;
            o.group(c.gs + c.gn, s.gs, s.gn);
        }
    }
    s.p = o.pair_at(s.gs + s.j);
    s.e = o.expert_b(s.gs + s.j);
    return s;
}

// y starts as 0 (or x with the residual); phase B adds into it.  Each
// workgroup writes its share; the stores are published with its first count.
__device__ inline void init_y(const LayerArgs &a) {
    const int G = gridDim.x, wg = blockIdx.x;
    const int64_t n = (int64_t)a.T * a.g.d;
    for (int64_t i = n * wg / G + threadIdx.x; i < n * (wg + 1) / G; i += kBlock)
        store_coherent(a.y + i, a.residual ? a.x[i] : 0.f);
}

// Exact top k of one token's E logits (in LDS, NaN already mapped to -inf),
// ties to the lower id, by the whole workgroup without comparing every pair.
// The maxima of the groups of 16 consecutive experts are distinct logits, so
// theta, the k-th largest of them, is at most the k-th largest logit: the top k
// all lie at or above theta and are ranked against those candidates only
// (about k to 2k of them for spread logits; all E when fewer than k groups or
// many equal logits, still exact).  Writes the k logits and ids by rank.
constexpr int kSelGroup = 16;
__device__ inline int row_sum_u(int v) {  // every lane: the sum over its DPP row of 16 lanes
    uint32_t u = (uint32_t)v;
    u += RVQ_DPP_U(u, kDppXor1);
    u += RVQ_DPP_U(u, kDppXor2);
    u += RVQ_DPP_U(u, kDppRor4);
    u += RVQ_DPP_U(u, kDppRor8);
    return (int)u;
}
__device__ void select_top_local(const double *lg, int E, int k, double *sel_out, int *id_out, double *scr) {
    double *gm = scr;                                         // [E / 16] group maxima
    double *theta = gm + kMaxExperts / kSelGroup;             // [1]
    double *cv = theta + 1;                                   // [E] candidate logits
    int *ci = reinterpret_cast<int *>(cv + kMaxExperts);      // [E] candidate ids
    int *n_cand = ci + 2 * kMaxExperts;                       // [1] candidate count
    const int i = threadIdx.x;
    const int n_grp = (E + kSelGroup - 1) / kSelGroup;
    const double v = i < E ? lg[i] : -INFINITY;
    static_assert(kSelGroup == 16, "a group is one DPP row");
    double m = v;  // max over the group's DPP row (lanes beyond E add -inf)
#pragma unroll
    for (int st = 0; st < 4; st++) m = fmax(m, dpp_d(m, st));
    if (i % kSelGroup == 0 && i / kSelGroup < n_grp) gm[i / kSelGroup] = m;
    if (i == 0) {
        *theta = -INFINITY;
        *n_cand = 0;
    }
    __syncthreads();
    if (n_grp >= k) {  // 16 threads per group maximum count those above it and those at or above it
        const int gi = i / 16, sub = i % 16;
        int cnt = 0;  // (count greater) + (count greater or equal) << 16
        if (gi < n_grp) {
            const double me = gm[gi];
            for (int h = sub; h < n_grp; h += 16) cnt += (gm[h] > me) + ((gm[h] >= me) << 16);
        }
        cnt = row_sum_u(cnt);
        if (sub == 0 && gi < n_grp && (cnt & 0xffff) < k && (cnt >> 16) >= k) *theta = gm[gi];  // all the same value
        __syncthreads();
    }
    if (i < E && v >= *theta) {  // candidates in any order (ranked by value, then id)
        const int pos = atomicAdd(n_cand, 1);
        cv[pos] = v;
        ci[pos] = i;
    }
    __syncthreads();
    const int n_c = *n_cand;
    // rank of each candidate among the candidates: 16 threads per candidate
    // when there are at most 64 of them, else one thread per candidate
    const int q = n_c <= kBlock / 16 ? 16 : 1;
    const int c = i / q, sub = i % q;
    int r = 0;
    if (c < n_c) {
        const double me = cv[c];
        const int id = ci[c];
        for (int j = sub; j < n_c; j += q) r += cv[j] > me || (cv[j] == me && ci[j] < id);
    }
    if (q == 16) r = row_sum_u(r);
    if (c < n_c && sub == 0 && r < k) {
        sel_out[r] = cv[c];
        id_out[r] = ci[c];
    }
    __syncthreads();
}

// Routing inside the launch (rvq_moe_route_forward).  [FR] "Lecture anticipée
// et prédiction du routeur": the router decides the token's experts; reading
// as in the separate route kernels: top-k of fp64 logits, ties to the lower
// id, softmax over the k.  No grid barrier and no counter; workgroup wg owns
// experts wg, wg + G, ... (at most kRouteExp):
//  R1  the logits of its experts for every token (fp64 sums of exact fp32
//      products, wave sums by DPP, divided by the fp64 RMS divisor when
//      normalising), each stored into its slot of buffer `cur`, which holds the
//      marker NaN until then; its slots of the other buffer get the marker back
//      for the next call;
//  R2  per token, it polls the E logit slots until none holds the marker (the
//      poll reads the logits themselves) and selects the token's top k from
//      them itself (select_top_local): every workgroup reaches the same ids,
//      with no further exchange.  The gates follow in route_gates (one exp
//      each, summed in rank order); workgroup 0 writes ids and gates out.
constexpr int kRouteExp = kRouteExperts;  // experts per workgroup (E <= 4 G)
// `idle` runs once R1 is published, before the wait for the other logits.
// With normalisation, r_tok / r_val receive the last token's RMS divisor (the
// one its logits were divided by), so that the experts' token_r() reuses it.
template <class Idle>
__device__ void route_phase(const LayerArgs &a, double *scratch, float *gate_lds, int *pair_ids, int &r_tok,
                            double &r_val, Idle &&idle) {
    const Geometry &g = a.g;
    const int G = gridDim.x, wg = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int n4 = g.d / 4;
    const double unpub = __longlong_as_double((long long)kUnpublished);
    double *lg = scratch;                 // [E] logits of the token being ranked
    double *sel = scratch + kMaxExperts;  // [P] selected logits by rank
    double *ex = sel + kRouteMaxPairs;    // [P] exps
    double *red = ex + kRouteMaxPairs;    // [kWaves][kRouteExp + 1], then the selection scratch
    const int P = a.T * g.k;
    // ---- R1
    // own experts of this workgroup (wave-uniform): loads only for those
    const int n_own = min(kRouteExp, (g.E - wg + G - 1) / G);
    __shared__ double r_share;  // the token's divisor, for the experts
    for (int t = 0; t < a.T; t++) {
        const float4 *x4 = reinterpret_cast<const float4 *>(a.x + (size_t)t * g.d);
        double acc[kRouteExp], ss = 0.0;
#pragma unroll
        for (int j = 0; j < kRouteExp; j++) acc[j] = 0.0;
        // two input blocks per step, every load of both issued before any sum
        // (clamped indices, masked at use), so one round trip serves 2 kBlock
        // float4 columns
        for (int i0 = threadIdx.x; i0 < n4; i0 += 2 * kBlock) {
            float4 xv[2], wv[2][kRouteExp];
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int i = min(i0 + h * kBlock, n4 - 1);
                xv[h] = x4[i];
#pragma unroll
                for (int j = 0; j < kRouteExp; j++)
                    if (j < n_own) wv[h][j] = reinterpret_cast<const float4 *>(a.Wt + (size_t)(wg + j * G) * g.d)[i];
            }
#pragma unroll
            for (int h = 0; h < 2; h++) {
                if (i0 + h * kBlock >= n4) break;
                if (a.pre) {
                    ss = fma((double)xv[h].x, (double)xv[h].x, ss);
                    ss = fma((double)xv[h].y, (double)xv[h].y, ss);
                    ss = fma((double)xv[h].z, (double)xv[h].z, ss);
                    ss = fma((double)xv[h].w, (double)xv[h].w, ss);
                }
#pragma unroll
                for (int j = 0; j < kRouteExp; j++) {
                    if (j >= n_own) break;
                    acc[j] = fma((double)xv[h].x, (double)wv[h][j].x, acc[j]);
                    acc[j] = fma((double)xv[h].y, (double)wv[h][j].y, acc[j]);
                    acc[j] = fma((double)xv[h].z, (double)wv[h][j].z, acc[j]);
                    acc[j] = fma((double)xv[h].w, (double)wv[h][j].w, acc[j]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kRouteExp; j++)
            if (j < n_own) acc[j] = wave_sum(acc[j]);  // uniform: only the owned experts' sums
        if (a.pre) ss = wave_sum(ss);
        if (lane == 0) {
#pragma unroll
            for (int j = 0; j < kRouteExp; j++) red[wave * (kRouteExp + 1) + j] = acc[j];
            red[wave * (kRouteExp + 1) + kRouteExp] = ss;
        }
        __syncthreads();
        if (threadIdx.x < n_own) {
            const int j = threadIdx.x, e = wg + j * G;
            double sa = 0.0, sq = 0.0;
            for (int w = 0; w < kWaves; w++) {
                sa += red[w * (kRouteExp + 1) + j];
                sq += red[w * (kRouteExp + 1) + kRouteExp];
            }
            const double r = a.pre ? sqrt(sq / (double)g.d + a.eps) : 1.0;
            store_coherent(a.rl_cur + (size_t)t * g.E + e, sa / r);
        }
        if (a.pre && threadIdx.x == 0) {  // (also where this workgroup owns no expert)
            double sq = 0.0;
            for (int w = 0; w < kWaves; w++) sq += red[w * (kRouteExp + 1) + kRouteExp];
            r_share = sqrt(sq / (double)g.d + a.eps);
        }
        __syncthreads();
        if (a.pre) {
            r_tok = t;
            r_val = r_share;
        }
    }
    // The other buffer goes back to the marker for the next routed call: the
    // logit slots of this workgroup's experts that the previous routed call
    // wrote there (its T_reset tokens; it has completed, and the next call
    // starts after this one).
    if (threadIdx.x < n_own)
        for (int t = 0; t < a.T_reset; t++)
            store_coherent(a.rl_next + (size_t)t * g.E + wg + threadIdx.x * G, unpub);
    if (!a.part_y) init_y(a);  // independent of the routing: done while the logits land
    idle();
    // ---- R2
    const uint64_t t_start = wall_clock64();
    auto timed_out = [&]() {
        if (wall_clock64() - t_start > 50000000ull) {  // 0.5 s at the 100 MHz constant clock
            if (threadIdx.x == 0) atomicOr(a.err, 2);
            return true;
        }
        __builtin_amdgcn_s_sleep(1);
        return false;
    };
    for (int t = 0; t < a.T; t++) {
        while (true) {
            int ready = 1;
            for (int i = threadIdx.x; i < g.E; i += kBlock) {
                const double v = load_coherent(a.rl_cur + (size_t)t * g.E + i);
                ready &= (uint64_t)__double_as_longlong(v) != kUnpublished;
                lg[i] = isnan(v) ? -INFINITY : v;
            }
            if (__syncthreads_and(ready) || timed_out()) break;
        }
        select_top_local(lg, g.E, g.k, sel + t * g.k, pair_ids + t * g.k, red + kWaves * (kRouteExp + 1));
    }
}

// The gates of the routed pairs from the selected logits route_phase left in
// the scratch (softmax over each token's k, summed in rank order); workgroup
// 0 also writes ids and gates out.  Separate from route_phase so that the
// first codebook and input loads of phase A go out before it.
__device__ void route_gates(const LayerArgs &a, double *scratch, float *gate_lds, const int *pair_ids) {
    const Geometry &g = a.g;
    const int wg = blockIdx.x;
    const double *sel = scratch + kMaxExperts;
    double *ex = scratch + kMaxExperts + kRouteMaxPairs;
    const int P = a.T * g.k;
    for (int i = threadIdx.x; i < P; i += kBlock) ex[i] = exp(sel[i] - sel[(i / g.k) * g.k]);
    __syncthreads();
    for (int i = threadIdx.x; i < P; i += kBlock) {
        const int t = i / g.k;
        double sum = 0.0;
        for (int j = 0; j < g.k; j++) sum += ex[t * g.k + j];
        const float gt = (float)(ex[i] / sum);
        gate_lds[i] = gt;
        if (wg == 0) {
            const_cast<float *>(a.gates)[i] = gt;
            const_cast<int32_t *>(a.ids)[i] = pair_ids[i];
        }
    }
    __syncthreads();
}

// Where a launch's pairs come from: the caller's ids, the launch's own routing
// (rvq_moe_route_forward), or a pair list handed over by the chunk path.
enum LayerMode { kFromIds = 0, kRouted = 1, kListed = 2 };

// kDet: the deterministic combine (output rows to a.part_y; see launch_combine).
// A template parameter, not a runtime flag, so that the other instances keep
// their register allocation.
template <int CB, int kMode, bool kNT, bool kDet>
__global__ __launch_bounds__(kBlock) void k_layer(LayerArgs a) {
    constexpr bool kRoute = kMode == kRouted, kList = kMode == kListed;
    __shared__ __align__(16) float lut[kLutWords];  // also 8-byte staging (logits, order masks)
    __shared__ float vs[kVec][kTileSlices];  // [element][slice]
    __shared__ double red[kWaves];
    static_assert((kMaxExperts + 2 * kRouteMaxPairs + kWaves * (kRouteExp + 1) + kMaxExperts / kSelGroup + 1 +
                   2 * kMaxExperts + kWaves) * sizeof(double) <= kLutWords * sizeof(float),
                  "routing scratch must fit the table area");
    static_assert(kMaxExperts <= kBlock, "one rank comparison per thread");
    __shared__ float hred[4][256][2];
    __shared__ float red2[kWaves];
    const Geometry &g = a.g;
    const int G = gridDim.x, wg = blockIdx.x;
    // range index: consecutive ranges go to workgroups on the same XCD (workgroups
    // are dealt round-robin over the 8 XCDs), so a code tile split between two
    // neighbouring ranges, or re-read by the next token of its group, stays in
    // one XCD's L2
    const int rw = (G % 8 == 0) ? (wg % 8) * (G / 8) + wg / 8 : wg;
    const int lane = threadIdx.x & 63, wave = wave_id();
    // with a handed-over pair list: exactly its pairs (its count read here)
    const int P = kList ? __builtin_amdgcn_readfirstlane(load_counter(a.list)) : a.T * g.k;
    const int n_ti = g.m[0].n_tiles, n_cf = g.m[0].n_chunks;
    const int n_tf = g.m[2].n_tiles, n_cd = g.m[2].n_chunks;
    int r_tok = -1;
    double r_val = 1.0;
    CbRegs<CB> cb;
    __shared__ float gate_lds[kRouteMaxPairs];
    __shared__ int pair_ids[kRouteMaxPairs];
    const float *gate_src = a.gates;
    // Phase A's unit range and, when the pairs keep their order (no order
    // table), its first segment's position: integer divisions that the routed
    // launch does while it waits for the logits.  The segment's expert is read
    // once the ids are known.
    const bool tab_order = kList || (a.T > 1 && P <= kOrderMax);
    int uA = 0, uA1 = 0;
    Deal dealA;
    SegA firstA{};
    bool firstA_placed = false;
    auto place_a = [&]() {
        // (the streaming-load instances serve the pair order only: no strided code there)
        dealA.start(!kNT && tab_order, P * 2 * n_ti, n_cf, rw, uA, uA1);
        if (kRoute && !tab_order && uA < uA1) {
            Order pos_only{};  // no table; its expert lookups read the (not yet routed) LDS ids
            pos_only.tab = false;
            pos_only.all = pair_ids;
            firstA = seg_a(uA, uA1, n_ti, n_cf, pos_only);
            firstA_placed = true;
        }
    };
    if (kRoute) {
        // the routing scratch reuses the table area, which is idle until phase A
        route_phase(a, reinterpret_cast<double *>(lut), gate_lds, pair_ids, r_tok, r_val, place_a);
        gate_src = gate_lds;
    } else {
        place_a();
    }
    bool gates_due = kRoute;  // route_gates not run yet
    // ---------------- pair order (the token x expert permutation)
    __shared__ int id_lds[2 * kIdCache];
    __shared__ int o_info[kOrderMax];
    __shared__ int o_pair[kOrderMax];
    __shared__ short o_expert[kOrderMax];
    Order ord;
    ord.tab = tab_order;
    ord.info = o_info;
    ord.pair = o_pair;
    ord.expert = o_expert;
    ord.ids = a.ids;
    ord.lds = id_lds;
    ord.all = kRoute ? pair_ids : nullptr;
    ord.a_n = ord.b_n = 0;
    ord.a_base = ord.b_base = 0;
    if (kList) {
        for (int i = threadIdx.x; i < P; i += kBlock) {
            o_info[i] = a.list[1 + i];
            o_pair[i] = a.list[1 + kOrderMax + i];
            o_expert[i] = (short)a.list[1 + 2 * kOrderMax + i];
        }
        __syncthreads();
    } else if (ord.tab) {
        if (gates_due) {  // the order table reuses the scratch that holds the selected logits
            route_gates(a, reinterpret_cast<double *>(lut), gate_lds, pair_ids);
            gates_due = false;
        }
        build_order(a.ids, kRoute ? pair_ids : nullptr, P, g.E, reinterpret_cast<char *>(lut), o_info, o_pair,
                    o_expert);
    } else if (!kRoute) {
        // pair order: cache the expert ids of the pairs this workgroup's ranges touch
        const int a0 = range_lo(P * 2 * n_ti * n_cf, rw, G), a1 = range_lo(P * 2 * n_ti * n_cf, rw + 1, G);
        const int b0 = range_lo(P * n_tf * n_cd, rw, G), b1 = range_lo(P * n_tf * n_cd, rw + 1, G);
        ord.a_base = a0 / (2 * n_ti * n_cf);
        ord.a_n = a1 > a0 ? min(kIdCache, (a1 - 1) / (2 * n_ti * n_cf) - ord.a_base + 1) : 0;
        ord.b_base = b0 / (n_tf * n_cd);
        ord.b_n = b1 > b0 ? min(kIdCache, (b1 - 1) / (n_tf * n_cd) - ord.b_base + 1) : 0;
        if (threadIdx.x < ord.a_n) id_lds[threadIdx.x] = load_counter(a.ids + ord.a_base + threadIdx.x);
        if (threadIdx.x < ord.b_n) id_lds[kIdCache + threadIdx.x] = load_counter(a.ids + ord.b_base + threadIdx.x);
        __syncthreads();
    }

    // ---------------- y starts as 0 (or x with the residual); the routed kernel
    // did this while routing, and with a handed-over pair list the chunk path
    // has set it already
    if (!kList && !kRoute && !kDet) init_y(a);
    bool y_ready = kDet;  // the deterministic combine writes y after the launch
    // Phase-A chunk counts are published per pair, once the workgroup moves on
    // to another pair or ends phase A (phase B waits for a pair's total), so
    // only those transitions wait for the stores to complete.  The y stores
    // are published with the first publication, at the latest at the second
    // segment's transition.
    bool y_signalled = false;
    int acc_p = -1, acc_n = 0;  // flushed chunks of pair acc_p not yet published
    auto publish = [&]() {      // all threads
        wait_stores();
        __syncthreads();
        if (threadIdx.x == 0) {
            if (acc_p >= 0) atomicAdd(a.cntA + acc_p * kCntStride, acc_n);
            if (!y_signalled) atomicAdd(a.ycnt, 1);
        }
        y_signalled = true;
        acc_p = -1;
        acc_n = 0;
    };
    auto count = [&](int pp, int n) {  // n chunks of pair pp flushed (stores issued); all threads
        if (acc_p >= 0 && acc_p != pp) publish();
        acc_p = pp;
        acc_n += n;
    };

    // merged gate/up partial sums in the pair order (see merged_away)
    // (not with the deterministic combine: every order then sums each row's
    // tiles one by one, in tile order)
    const bool merge = !ord.tab && n_cf <= 64 && !kDet;
    const int64_t nA = (int64_t)P * 2 * n_ti * n_cf;
    __shared__ uint64_t vmask[2][kMaskWords];
    // ---------------- phase A: gate and up
    {
        int u = uA;
        int u1 = uA1;
        float xv = 0.f;  // this thread's raw input element of the segment's tile
        auto prefetch = [&](const SegA &sg) {
            if (sg.e >= 0 && sg.e < g.E) cb_load<CB>(cb, a.cbs, a.cb_exp, sg.e, sg.m);
            const int col = sg.tile * kTileSlices * kVec + threadIdx.x;
            xv = (threadIdx.x < kTileSlices * kVec && col < g.d) ? a.x[(size_t)(sg.p / g.k) * g.d + col] : 0.f;
        };
        // row totals of phase A go to their own staging area (the finish area of
        // phase B, idle here); the last sub-range of a segment is flushed, and the
        // segment counted, during the next segment's table build
        const Stage ast{&hred[0][0][0], kChunkRows, (int)(sizeof(hred) / sizeof(float)) / kChunkRows};
        // merged partial sums (see merged_away): totals staged at their chunk
        // position and accumulated over a run of whole tiles
        float *const hst = &hred[0][0][0];
        if (merge)
            for (int i = threadIdx.x; i < ast.cap * kChunkRows; i += kBlock) hst[i] = 0.f;  // before the first barrier
        float *pend_out = nullptr;  // pending flush: out, chunks [pend_c0, pend_c1), count pend_n for pair pend_p
        int pend_c0 = 0, pend_c1 = 0, pend_p = 0, pend_n = 0, pend_m = 0, pend_tile = 0;
        bool pend_full = false;
        auto flush_pend = [&]() {  // all threads, after a barrier
            if (merge)
                flush_rows_clear(hst, pend_out, pend_c0, pend_c1);
            else
                flush_rows(ast, pend_out, pend_c0, pend_c1);
        };
        SegA cur{};
        if (u < u1) {
            if (firstA_placed) {
                cur = firstA;
                cur.p = ord.pair_at(cur.gs + cur.j);
                cur.e = ord.expert_a(cur.gs + cur.j);
            } else {
                cur = seg_a(u, u1, n_ti, n_cf, ord);
            }
            prefetch(cur);
        }
        if (gates_due) {  // while the first codebook and inputs are in flight
            route_gates(a, reinterpret_cast<double *>(lut), gate_lds, pair_ids);
            gates_due = false;
        }
        while (u < u1) {
            const int un = u + (cur.c1 - cur.c0);
            int nu = un, nu1 = u1;  // the next segment's span
            if constexpr (!kNT)
                if (un >= u1) dealA.next(nu, nu1);
            SegA nxt{};
            if (nu < nu1) nxt = nu == un ? next_a(cur, un, u1, n_ti, n_cf, ord) : seg_a(nu, nu1, n_ti, n_cf, ord);
            if (cur.e >= 0 && cur.e < g.E) {
                const uint8_t *base = expert_record(a, cur.e) + g.m[cur.m].off +
                                      (int64_t)cur.tile * n_cf * kChunkBytes;
                // consume the prefetched codebook and inputs first, so that waiting
                // for them does not also wait for the code loads issued below
                const double r = token_r(a, cur.p / g.k, r_tok, r_val, red);
                cb_store<CB>(lut, cb);
                if (threadIdx.x < kTileSlices * kVec) {
                    const float v = a.pre ? (float)((double)xv / r) : xv;
                    vs[threadIdx.x % kVec][threadIdx.x / kVec] = v;
                    tile_max_publish(v, red2);
                }
                u32x4 p[3];
                if (cur.c0 + wave < cur.c1)
                    load_chunk(base + (int64_t)(cur.c0 + wave) * kChunkBytes, lane, p[0], p[1], p[2], kNT);
                // a whole tile right after a whole tile of the same (pair, matrix):
                // its totals add to the staged ones, nothing is flushed here
                const bool full = cur.c0 == 0 && cur.c1 == n_cf;
                const bool extend = merge && pend_out && pend_full && full && cur.p == pend_p && cur.m == pend_m &&
                                    cur.tile == pend_tile + 1;
                const bool flush = pend_out && !extend;
                __syncthreads();
                if (flush) flush_pend();
                build_lut<CB>(lut, vs, tile_exponent(red2), cb.ec);
                if (flush) count(pend_p, pend_n);
                if (pend_out && !y_signalled) publish();
                __syncthreads();
                if (nu < nu1) prefetch(nxt);
                float *out = a.part_gu + (((int64_t)cur.p * 2 + cur.m) * n_ti + cur.tile) * g.ffn_pad;
                Stage st = ast;
                if (merge) st = Stage{hst + cur.c0 * kChunkRows, kChunkRows, ast.cap - cur.c0, true};
                const int c0s = gather_segment<false, true>(lut, st, base, cur.c0, cur.c1, out, 0, p, kNT);
                if (extend) {  // the run now ends at this tile: its slot takes the sum
                    pend_out = out;
                    pend_tile = cur.tile;
                    pend_n += cur.c1 - cur.c0;
                } else {
                    pend_c0 = c0s;
                    pend_c1 = cur.c1;
                    pend_out = out;
                    pend_p = cur.p;
                    pend_m = cur.m;
                    pend_tile = cur.tile;
                    pend_n = cur.c1 - cur.c0;
                    pend_full = full;
                }
            } else {
                if (threadIdx.x == 0) atomicOr(a.err, 1);
                if (pend_out) {
                    __syncthreads();
                    flush_pend();
                    count(pend_p, pend_n);
                    pend_out = nullptr;
                }
                count(cur.p, cur.c1 - cur.c0);
                if (nu < nu1) prefetch(nxt);
            }
            cur = nxt;
            u = nu;
            u1 = nu1;
        }
        if (pend_out) {
            __syncthreads();
            flush_pend();
            count(pend_p, pend_n);
        }
    }
    if (acc_p >= 0 || !y_signalled) publish();  // the last pair's count (and y, if not yet)

    // ---------------- phase B: SwiGLU finish, gate, down
    {
        int u, u1;
        Deal dealB;
        dealB.start(!kNT && ord.tab, P * n_tf, n_cd, rw, u, u1);
        const int needA = 2 * n_ti * n_cf;
        SegB cur{};
        if (u < u1) {
            cur = seg_b(u, u1, n_tf, n_cd, ord);
            if (cur.e >= 0 && cur.e < g.E) cb_load<CB>(cb, a.cbs, a.cb_exp, cur.e, 2);
        }
        while (u < u1) {
            const int un = u + (cur.c1 - cur.c0);
            int nu = un, nu1 = u1;  // the next segment's span
            if constexpr (!kNT)
                if (un >= u1) dealB.next(nu, nu1);
            SegB nxt{};
            if (nu < nu1) nxt = nu == un ? next_b(cur, un, u1, n_tf, n_cd, ord) : seg_b(nu, nu1, n_tf, n_cd, ord);
            if (cur.e >= 0 && cur.e < g.E) {
                const uint8_t *base = expert_record(a, cur.e) + g.m[2].off +
                                      (int64_t)cur.ft * n_cd * kChunkBytes;
                cb_store<CB>(lut, cb);
                u32x4 p[3];
                if (cur.c0 + wave < cur.c1)
                    load_chunk(base + (int64_t)(cur.c0 + wave) * kChunkBytes, lane, p[0], p[1], p[2], kNT);
                // which gate/up partial slots of this pair hold sums (before the
                // wait, whose barrier publishes it)
                if (threadIdx.x < 2 * 64 * kMaskWords) {  // one wave per mask word
                    const int m = threadIdx.x / (64 * kMaskWords), t = threadIdx.x % (64 * kMaskWords);
                    const int64_t u0 = (((int64_t)cur.p * 2 + m) * n_ti + t) * n_cf;
                    const bool has = t < n_ti && !(merge && merged_away(nA, G, u0, n_cf, t + 1 == n_ti));
                    const uint64_t bits = __ballot(has);
                    if ((threadIdx.x & 63) == 0) vmask[m][t / 64] = bits;
                }
                wait_count(a.cntA + cur.p * kCntStride, needA, a.err);
                finish_h(a, gate_src, cur.p, cur.ft, vs, red2, vmask);
                __syncthreads();
                build_lut<CB>(lut, vs, tile_exponent(red2), cb.ec);
                __syncthreads();
                if (nu < nu1 && nxt.e >= 0 && nxt.e < g.E) cb_load<CB>(cb, a.cbs, a.cb_exp, nxt.e, 2);
                if (!y_ready) {
                    wait_count(a.ycnt, G, a.err);
                    y_ready = true;
                }
                if (kDet) {  // this pair's rows of down tile ft, combined after the launch
                    float *pt = a.part_y + ((int64_t)cur.p * n_tf + cur.ft) * g.d_pad;
                    gather_segment<false, false>(lut, cb_area_stage(lut), base, cur.c0, cur.c1, pt, g.d, p, kNT);
                } else {
                    float *yt = a.y + (size_t)(cur.p / g.k) * g.d;
                    gather_segment<true, false>(lut, cb_area_stage(lut), base, cur.c0, cur.c1, yt, g.d, p, kNT);
                }
            } else {
                // an invalid id poisons its token's output (the error flag is already set)
                if (!y_ready) {
                    wait_count(a.ycnt, G, a.err);
                    y_ready = true;
                }
                if (cur.ft == 0 && !kDet)  // (the deterministic combine poisons the token itself)
                    for (int r = cur.c0 * kChunkRows + threadIdx.x; r < min(g.d, cur.c1 * kChunkRows); r += kBlock)
                        unsafeAtomicAdd(a.y + (size_t)(cur.p / g.k) * g.d + r, __int_as_float(0x7fc00000));
                if (nu < nu1 && nxt.e >= 0 && nxt.e < g.E) cb_load<CB>(cb, a.cbs, a.cb_exp, nxt.e, 2);
            }
            __syncthreads();
            cur = nxt;
            u = nu;
            u1 = nu1;
        }
    }
    // the other counter set starts the next launch at zero (see kCntSets)
    for (int i = range_lo(a.n_clear, wg, G) + threadIdx.x; i < range_lo(a.n_clear, wg + 1, G); i += kBlock)
        store_counter(a.cnt_clear + (size_t)i * kCntStride, 0);
}

// Deterministic combine (see launch_combine).  A workgroup takes 32 output
// elements of one token; lane q (of kCombLanes) sums the token's partial rows
// q, q + kCombLanes, ... in that order (all of its loads in flight together),
// then the lanes' sums are added in lane order after x.  The order depends on
// k, slots and the element only, never on timing or on how tokens were
// grouped into calls.
constexpr int kCombLanes = 8, kCombRows = 32, kCombInFlight = 16;
__global__ __launch_bounds__(kCombLanes * kCombRows) void k_combine(const float *__restrict__ part, int slots,
                                                                    const float *__restrict__ x,
                                                                    const int32_t *__restrict__ ids,
                                                                    float *__restrict__ y, int k, int E, int d,
                                                                    int d_pad, int residual) {
    const int t = blockIdx.y;
    const int q = threadIdx.x / kCombRows, rr = threadIdx.x % kCombRows;
    const int r = blockIdx.x * kCombRows + rr;
    __shared__ float lane_sum[kCombLanes][kCombRows];
    const int n = k * slots;
    float acc = 0.f;
    if (r < d) {
        const float *p = part + (size_t)t * n * d_pad + r;
        for (int i0 = q; i0 < n; i0 += kCombLanes * kCombInFlight) {
            float v[kCombInFlight];
#pragma unroll
            for (int u = 0; u < kCombInFlight; u++) {
                const int i = i0 + u * kCombLanes;
                v[u] = i < n ? p[(size_t)i * d_pad] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < kCombInFlight; u++)
                if (i0 + u * kCombLanes < n) acc += v[u];
        }
    }
    lane_sum[q][rr] = acc;
    __syncthreads();
    if (q != 0 || r >= d) return;
    bool bad = false;
    for (int j = 0; j < k; j++) {
        const int e = ids[(size_t)t * k + j];
        bad |= e < 0 || e >= E;
    }
    float out = residual ? x[(size_t)t * d + r] : 0.f;
    float sum = lane_sum[0][rr];
#pragma unroll
    for (int l = 1; l < kCombLanes; l++) sum += lane_sum[l][rr];
    out += sum;
    y[(size_t)t * d + r] = bad ? __int_as_float(0x7fc00000) : out;
}

hipError_t launch_combine(const float *part, int slots, const float *x, const int32_t *ids, float *y, int T, int k,
                          int E, int d, int d_pad, int residual, hipStream_t s) {
    hipLaunchKernelGGL(k_combine, dim3((d + kCombRows - 1) / kCombRows, T), dim3(kCombLanes * kCombRows), 0, s, part,
                       slots, x, ids, y, k, E, d, d_pad, residual);
    return hipGetLastError();
}

typedef void (*LayerKernel)(LayerArgs);
template <int CB>
static LayerKernel layer_kernel_cb(int mode, bool nt, bool det) {
    if (mode == kListed) return k_layer<CB, kListed, false, false>;  // (never with the deterministic combine)
    if (det) {
        if (mode == kRouted) return nt ? k_layer<CB, kRouted, true, true> : k_layer<CB, kRouted, false, true>;
        return nt ? k_layer<CB, kFromIds, true, true> : k_layer<CB, kFromIds, false, true>;
    }
    if (mode == kRouted) return nt ? k_layer<CB, kRouted, true, false> : k_layer<CB, kRouted, false, false>;
    return nt ? k_layer<CB, kFromIds, true, false> : k_layer<CB, kFromIds, false, false>;
}
static LayerKernel layer_kernel(int cb_dtype, int mode, bool nt, bool det) {
    return cb_dtype == 0 ? layer_kernel_cb<0>(mode, nt, det) : layer_kernel_cb<1>(mode, nt, det);
}

hipError_t launch_layer(const Geometry &g, Workspace &w, const uint8_t *codes, const uint8_t *const *slot_tab,
                        const void *cbs, const float *Wt, const float *x, const int32_t *ids, const float *gates,
                        float *y, int T, int pre, int residual, double eps, bool route, hipStream_t s,
                        const int *list) {
    double *rl_cur = nullptr, *rl_next = nullptr;
    int T_reset = 0;
    if (route) {  // the slot buffers (see fused_route_slots) alternate between calls
        const int64_t cap = w.fused_cap;  // fused_route_slots() = 2 buffers of this many
        const int par = w.fused_parity;
        rl_cur = w.fused_logits + (par ? cap : 0);
        rl_next = w.fused_logits + (par ? 0 : cap);
        T_reset = w.fused_prev_T;
    }
    // counter sets rotate over launches (see kCntSets)
    const size_t set_ints = (size_t)w.cnt_per_set * kCntStride;
    int *cnt_cur = w.cnt + w.cnt_phase * set_ints;
    int *cnt_clear = w.cnt + ((w.cnt_phase + 1) % kCntSets) * set_ints;
    LayerArgs a{Wt, w.logits, w.sel, cnt_cur + (size_t)(w.cnt_per_set - 1) * kCntStride, cnt_clear, w.cnt_per_set,
                rl_cur, rl_next, T_reset, list, codes, slot_tab, cbs, w.cb_exp, x, ids, gates, y, w.part_gu,
                cnt_cur, w.det ? w.part_y : nullptr, w.err, g, T, pre, residual, eps};
    // A plain launch of exactly as many workgroups as can be resident at once
    // (sized at open from the occupancy query); the inter-workgroup waits are
    // bounded, so a launch that somehow did not get all of them resident ends
    // with an error flag instead of hanging.
    const bool group = list || (T > 1 && T * g.k <= kOrderMax);  // the kernel takes the same decision
    hipLaunchKernelGGL(layer_kernel(g.cb_dtype, list ? kListed : route ? kRouted : kFromIds, !group, w.det && !list),
                       dim3(w.n_wg), dim3(kBlock), 0, s, a);
    const hipError_t e = hipGetLastError();
    // the alternating buffers and counter sets advance only with a launch that
    // was enqueued: a failed launch leaves them as the last launch left them
    if (e != hipSuccess) return e;
    if (route) {
        w.fused_parity ^= 1;
        w.fused_prev_T = T;
    }
    w.cnt_phase = (w.cnt_phase + 1) % kCntSets;
    return hipSuccess;
}

hipError_t layer_blocks_per_cu(int cb_dtype, int *out) {
    // the grid must be resident under every variant: take the smallest occupancy
    int best = 1 << 30;
    for (int v = 0; v < 12; v++) {
        int n = 0;
        const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, layer_kernel(cb_dtype, (v >> 1) % 3, v & 1, v >= 6), kBlock, 0);
        if (e != hipSuccess) return e;
        best = n < best ? n : best;
    }
    *out = best;
    return hipSuccess;
}

}  // namespace rvq
