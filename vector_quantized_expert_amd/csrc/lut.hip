// lut.hip -- expert evaluation from RVQ codes through tables of partial dot
// products held in LDS.
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
// MI355X mapping.  A workgroup owns one tile of 32 slices of one matrix and
// streams all (or a block of) its rows.  Its 3 x 256 x 32 fp32 table (96 KB)
// sits in LDS laid out [stage][code][lane]: lane l of a half-wave always
// serves slice l, so its lookups hit LDS bank l whatever the code value and a
// half-wave's 32 random lookups are bank-conflict free.  Each lane loads 16
// code bytes per stage (16 rows of its slice) with one 16-byte load; a wave's
// load is 1 KB contiguous.  The 16 per-lane row values are then summed across
// the 32 slice lanes with a transposed butterfly (each step halves the values
// held per lane), leaving one row total per lane pair.
#include <math.h>

#include "internal.hpp"

namespace rvq {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 1024;  // threads per gather workgroup (16 waves)
constexpr int kLutFloats = kStages * kCodes * kTileSlices;  // 24576 (96 KB)

// ---------------------------------------------------------------------------
// Repack: canonical [rows][slices][3] per matrix -> tiled internal layout.
// One thread writes one 16-byte unit (one lane's stage bytes of a block).
__global__ __launch_bounds__(256) void k_repack(const uint8_t *__restrict__ canon, uint8_t *__restrict__ out,
                                                Geometry g, int64_t units_per_expert, int64_t total_units) {
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= total_units) return;
    const int64_t e = u / units_per_expert;
    int64_t lu = u % units_per_expert;  // unit inside the internal record
    int m = 0;
    int64_t canon_off = 0;
    for (; m < 3; m++) {
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

// ---------------------------------------------------------------------------
// Codebook access: entry (stage s, code c) of matrix m of expert e, 8 values.
template <int CB>
__device__ inline void load_entry(const void *cbs, int64_t e, int m, int s, int c, float (&w)[8]) {
    const int64_t idx = ((((e * 3 + m) * kStages + s) * kCodes) + c) * kVec;
    if (CB == 0) {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(cbs) + idx);
        const float4 a = p[0], b = p[1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else {
        const uint4 q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(cbs) + idx);
        const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            w[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[i] & 0xffff));
            w[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[i] >> 16));
        }
    }
}

// Build the [stage][code][lane] table of one 32-slice tile in LDS.
// vs[l][i] holds the 8 input values of slice (tile*32 + l) (zero past the end).
template <int CB>
__device__ inline void build_lut(float *lut, const float (*vs)[kVec], const void *cbs, int64_t e, int m) {
    const int l = threadIdx.x & 31;
    float xv[kVec];
#pragma unroll
    for (int i = 0; i < kVec; i++) xv[i] = vs[l][i];
    for (int idx = threadIdx.x >> 5; idx < kStages * kCodes; idx += kBlock / 32) {
        const int s = idx >> 8, c = idx & 255;
        float w[8];
        load_entry<CB>(cbs, e, m, s, c, w);
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < kVec; i++) acc = fmaf(w[i], xv[i], acc);
        lut[idx * kTileSlices + l] = acc;
    }
}

__device__ inline uint32_t byte_of(const u32x4 &q, int i) {
    const uint32_t w = (i < 4) ? q.x : (i < 8) ? q.y : (i < 12) ? q.z : q.w;
    return (w >> (8 * (i & 3))) & 0xffu;
}

// Gather one 32-row chunk: returns the row total held by this lane (valid on
// even lanes of each half; row = chunk*32 + half*16 + (lane&31)/2).
__device__ inline float gather_chunk(const float *lut, const uint8_t *blk, int lane) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(blk) + lane;
    const u32x4 q0 = __builtin_nontemporal_load(p);
    const u32x4 q1 = __builtin_nontemporal_load(p + 64);
    const u32x4 q2 = __builtin_nontemporal_load(p + 128);
    const int l = lane & 31;
    const float *t0 = lut + l;
    const float *t1 = lut + kCodes * kTileSlices + l;
    const float *t2 = lut + 2 * kCodes * kTileSlices + l;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        v[i] = t0[byte_of(q0, i) * kTileSlices] + t1[byte_of(q1, i) * kTileSlices] +
               t2[byte_of(q2, i) * kTileSlices];
    }
    // transposed butterfly over the 32 slice lanes of the half-wave
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const bool hi = l & 16;
        const float send = hi ? v[i] : v[i + 8];
        const float keep = hi ? v[i + 8] : v[i];
        v[i] = keep + __shfl_xor(send, 16);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const bool hi = l & 8;
        const float send = hi ? v[i] : v[i + 4];
        const float keep = hi ? v[i + 4] : v[i];
        v[i] = keep + __shfl_xor(send, 8);
    }
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const bool hi = l & 4;
        const float send = hi ? v[i] : v[i + 2];
        const float keep = hi ? v[i + 2] : v[i];
        v[i] = keep + __shfl_xor(send, 4);
    }
    {
        const bool hi = l & 2;
        const float send = hi ? v[0] : v[1];
        const float keep = hi ? v[1] : v[0];
        v[0] = keep + __shfl_xor(send, 2);
    }
    return v[0] + __shfl_xor(v[0], 1);
}

// ---------------------------------------------------------------------------
// Gate and up: grid (tile, matrix, pair).  Writes the tile's partial sums of
// every row: part_gu[pair][m][tile][row].
template <int CB>
__global__ __launch_bounds__(kBlock) void k_gateup(const uint8_t *__restrict__ codes, const void *__restrict__ cbs,
                                                   const float *__restrict__ x, const double *__restrict__ r,
                                                   const int32_t *__restrict__ ids, Geometry g,
                                                   float *__restrict__ part, int *__restrict__ err) {
    __shared__ float lut[kLutFloats];
    __shared__ float vs[kTileSlices][kVec];
    const int tile = blockIdx.x, m = blockIdx.y, pair = blockIdx.z;
    const int tok = pair / g.k;
    const int e = ids[pair];
    if (e < 0 || e >= g.E) {
        if (threadIdx.x == 0) atomicOr(err, 1);
        return;
    }
    const MatGeom mg = g.m[m];
    if (threadIdx.x < kTileSlices * kVec) {
        const int col = tile * kTileSlices * kVec + threadIdx.x;
        float v = 0.f;
        if (col < g.d) v = (float)((double)x[(size_t)tok * g.d + col] / r[tok]);
        vs[threadIdx.x / kVec][threadIdx.x % kVec] = v;
    }
    __syncthreads();
    build_lut<CB>(lut, vs, cbs, e, m);
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint8_t *base = codes + (int64_t)e * g.rec_int + mg.off + (int64_t)tile * mg.n_chunks * kChunkBytes;
    float *out = part + (((int64_t)pair * 2 + m) * g.m[0].n_tiles + tile) * g.ffn_pad;
    for (int q = wave; q < mg.n_chunks; q += kBlock / 64) {
        const float sum = gather_chunk(lut, base + (int64_t)q * kChunkBytes, lane);
        if (!(lane & 1)) out[q * kChunkRows + (lane >> 5) * 16 + ((lane & 31) >> 1)] = sum;
    }
}

hipError_t launch_gateup(const Geometry &g, const Workspace &w, const uint8_t *codes, const void *cbs,
                         const float *x, const int32_t *ids, int T, hipStream_t s) {
    dim3 grid(g.m[0].n_tiles, 2, T * g.k);
    if (g.cb_dtype == 0)
        hipLaunchKernelGGL(k_gateup<0>, grid, dim3(kBlock), 0, s, codes, cbs, x, w.tok_r, ids, g, w.part_gu, w.err);
    else
        hipLaunchKernelGGL(k_gateup<1>, grid, dim3(kBlock), 0, s, codes, cbs, x, w.tok_r, ids, g, w.part_gu, w.err);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Down: grid (ffn tile, row block, pair).  First finishes h for the tile's
// 256 FFN entries, h = silu(a) * b with a, b the summed gate/up partials (the
// SwiGLU reading of the expert FFN), then builds the table over h and gathers
// the row block: part_dn[pair][tile][row].
template <int CB>
__global__ __launch_bounds__(kBlock) void k_down(const uint8_t *__restrict__ codes, const void *__restrict__ cbs,
                                                 const int32_t *__restrict__ ids, Geometry g,
                                                 const float *__restrict__ part_gu, float *__restrict__ part,
                                                 int *__restrict__ err) {
    __shared__ float lut[kLutFloats];
    __shared__ float vs[kTileSlices][kVec];
    const int tile = blockIdx.x, rb = blockIdx.y, pair = blockIdx.z;
    const int e = ids[pair];
    if (e < 0 || e >= g.E) {
        if (threadIdx.x == 0) atomicOr(err, 1);
        return;
    }
    const MatGeom mg = g.m[2];
    const int nti = g.m[0].n_tiles;
    if (threadIdx.x < kTileSlices * kVec) {
        const int f = tile * kTileSlices * kVec + threadIdx.x;
        float hv = 0.f;
        if (f < g.ffn) {
            const float *pa = part_gu + ((int64_t)pair * 2 + 0) * nti * g.ffn_pad + f;
            const float *pb = part_gu + ((int64_t)pair * 2 + 1) * nti * g.ffn_pad + f;
            float a = 0.f, b = 0.f;
            for (int t = 0; t < nti; t++) {
                a += pa[(int64_t)t * g.ffn_pad];
                b += pb[(int64_t)t * g.ffn_pad];
            }
            hv = a / (1.f + expf(-a)) * b;
        }
        vs[threadIdx.x / kVec][threadIdx.x % kVec] = hv;
    }
    __syncthreads();
    build_lut<CB>(lut, vs, cbs, e, 2);
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint8_t *base = codes + (int64_t)e * g.rec_int + mg.off + (int64_t)tile * mg.n_chunks * kChunkBytes;
    float *out = part + ((int64_t)pair * mg.n_tiles + tile) * g.d_pad;
    const int q0 = rb * g.down_row_block;
    const int q1 = min(mg.n_chunks, q0 + g.down_row_block);
    for (int q = q0 + wave; q < q1; q += kBlock / 64) {
        const float sum = gather_chunk(lut, base + (int64_t)q * kChunkBytes, lane);
        if (!(lane & 1)) out[q * kChunkRows + (lane >> 5) * 16 + ((lane & 31) >> 1)] = sum;
    }
}

hipError_t launch_down(const Geometry &g, const Workspace &w, const uint8_t *codes, const void *cbs,
                       const int32_t *ids, int T, hipStream_t s) {
    dim3 grid(g.m[2].n_tiles, g.n_down_rb, T * g.k);
    if (g.cb_dtype == 0)
        hipLaunchKernelGGL(k_down<0>, grid, dim3(kBlock), 0, s, codes, cbs, ids, g, w.part_gu, w.part_dn, w.err);
    else
        hipLaunchKernelGGL(k_down<1>, grid, dim3(kBlock), 0, s, codes, cbs, ids, g, w.part_gu, w.part_dn, w.err);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine: y[t][q] = sum_j gates[t][j] * y_j[q] (+ x[t][q]), y_j the summed
// down partials of pair (t, j), j ascending.
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ part, const float *__restrict__ x,
                                                 const int32_t *__restrict__ ids, const float *__restrict__ gates,
                                                 Geometry g, int residual, float *__restrict__ y) {
    const int q = blockIdx.x * 256 + threadIdx.x;
    const int t = blockIdx.y;
    if (q >= g.d) return;
    const int ntf = g.m[2].n_tiles;
    float acc = 0.f;
    bool bad = false;
    for (int j = 0; j < g.k; j++) {
        const int pair = t * g.k + j;
        const int e = ids[pair];
        bad |= (e < 0 || e >= g.E);
        const float *p = part + (int64_t)pair * ntf * g.d_pad + q;
        float yj = 0.f;
        for (int tt = 0; tt < ntf; tt++) yj += p[(int64_t)tt * g.d_pad];
        acc = fmaf(gates[pair], yj, acc);
    }
    if (residual) acc += x[(size_t)t * g.d + q];
    y[(size_t)t * g.d + q] = bad ? __int_as_float(0x7fc00000) : acc;
}

hipError_t launch_combine(const Geometry &g, const Workspace &w, const float *x, const int32_t *ids,
                          const float *gates, float *y, int T, int residual, hipStream_t s) {
    dim3 grid((g.d + 255) / 256, T);
    hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, s, w.part_dn, x, ids, gates, g, residual, y);
    return hipGetLastError();
}

}  // namespace rvq
