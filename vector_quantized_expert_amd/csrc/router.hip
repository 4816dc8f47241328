// router.hip -- router GEMV and top-k gates in one launch.
//
// [FR] "Lecture anticipée et prédiction du routeur": a layer's router decides
// the token's expert ids (16 for K3) and the expert reads start from them.  The
// score function is not given on the pages; the reading taken is top-k of the
// raw logits (descending, ties to the lower id) and a softmax over the k
// selected logits.
//
// Precision: logits accumulate exact fp32 x fp32 products in fp64, so the only
// difference from any other summation order is fp64 rounding of the sum
// (~1e-16 relative), which keeps the selected ids reproducible against an
// independent fp64 reference.  With RMS normalisation the logit is
// (sum_i x_i W[i][e]) / r with r = sqrt(mean(x^2) + eps) computed in fp64,
// equal in exact arithmetic to sum_i (x_i / r) W[i][e].
//
// MI355X mapping: the router matrix is stored transposed ([E][d]) so that a
// workgroup streams one expert's column as contiguous 1 KB wave loads (its 4
// waves take a quarter each) for up to TT tokens.  Selection avoids a serial
// chain of k argmax rounds: a second launch ranks every expert in parallel (one
// wave counts the experts ahead of it) and the k with rank < k write their id
// and logit to that slot; a third gives each token one wave for the softmax.
// Wave reductions use DPP row moves and permlane swaps (no LDS round trips).
#include <math.h>

#include "internal.hpp"

namespace rvq {

// ---------------------------------------------------------------------------
// W [d][E] -> Wt [E][d] (once, at open).
__global__ __launch_bounds__(256) void k_transpose(const float *__restrict__ W, float *__restrict__ Wt, int d, int E) {
    __shared__ float tile[32][33];
    const int e0 = blockIdx.x * 32, i0 = blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int r = ty; r < 32; r += 8) {
        const int i = i0 + r, e = e0 + tx;
        tile[r][tx] = (i < d && e < E) ? W[(size_t)i * E + e] : 0.f;
    }
    __syncthreads();
    for (int r = ty; r < 32; r += 8) {
        const int e = e0 + r, i = i0 + tx;
        if (e < E && i < d) Wt[(size_t)e * d + i] = tile[tx][r];
    }
}

hipError_t launch_transpose(const float *W, float *Wt, int d, int E, hipStream_t s) {
    dim3 grid((E + 31) / 32, (d + 31) / 32);
    hipLaunchKernelGGL(k_transpose, grid, dim3(256), 0, s, W, Wt, d, E);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Wave64 cross-lane moves without LDS: DPP within rows of 16 lanes,
// permlane16/32 swaps across rows.
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

// NaN logits rank below every number (and among themselves by id).
__device__ inline double rank_value(double v) { return isnan(v) ? -INFINITY : v; }

// grid (E, ceil(T / TT)), 256 threads: the 4 waves of a workgroup each take a
// quarter of expert e's column (float4 granules) for TT tokens.
template <int TT>
__global__ __launch_bounds__(256) void k_route(const float *__restrict__ x, const float *__restrict__ Wt, int d, int E,
                                               int T, int pre, double eps, double *__restrict__ logits) {
    const int e = blockIdx.x;
    const int t0 = blockIdx.y * TT;
    const int nt = min(TT, T - t0);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n4 = d / 4;
    const int g0 = n4 * wave / 4, g1 = n4 * (wave + 1) / 4;
    const float4 *w4 = reinterpret_cast<const float4 *>(Wt + (size_t)e * d);
    double acc[TT], ss[TT];
#pragma unroll
    for (int t = 0; t < TT; t++) acc[t] = ss[t] = 0.0;
    for (int i = g0 + lane; i < g1; i += 64 * 4) {
        float4 wv[4];
#pragma unroll
        for (int u = 0; u < 4; u++) wv[u] = (i + 64 * u < g1) ? w4[i + 64 * u] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int t = 0; t < TT; t++) {
            if (t >= nt) break;
            const float4 *x4 = reinterpret_cast<const float4 *>(x + (size_t)(t0 + t) * d);
#pragma unroll
            for (int u = 0; u < 4; u++) {
                if (i + 64 * u < g1) {
                    const float4 xv = x4[i + 64 * u];
                    acc[t] = fma((double)xv.x, (double)wv[u].x, acc[t]);
                    acc[t] = fma((double)xv.y, (double)wv[u].y, acc[t]);
                    acc[t] = fma((double)xv.z, (double)wv[u].z, acc[t]);
                    acc[t] = fma((double)xv.w, (double)wv[u].w, acc[t]);
                    if (pre) {
                        ss[t] = fma((double)xv.x, (double)xv.x, ss[t]);
                        ss[t] = fma((double)xv.y, (double)xv.y, ss[t]);
                        ss[t] = fma((double)xv.z, (double)xv.z, ss[t]);
                        ss[t] = fma((double)xv.w, (double)xv.w, ss[t]);
                    }
                }
            }
        }
    }
    __shared__ double red[4][TT][2];
#pragma unroll
    for (int t = 0; t < TT; t++) {
        if (t >= nt) break;
        const double sa = wave_sum(acc[t]);
        const double sq = pre ? wave_sum(ss[t]) : 0.0;
        if (lane == 0) {
            red[wave][t][0] = sa;
            red[wave][t][1] = sq;
        }
    }
    __syncthreads();
    if (threadIdx.x < nt) {
        const int t = threadIdx.x;
        const double sa = red[0][t][0] + red[1][t][0] + red[2][t][0] + red[3][t][0];
        const double sq = red[0][t][1] + red[1][t][1] + red[2][t][1] + red[3][t][1];
        const double r = pre ? sqrt(sq / (double)d + eps) : 1.0;
        logits[(size_t)(t0 + t) * E + e] = sa / r;
    }
}

// Rank of every expert in the strict order (logit descending, id ascending):
// one wave per (expert, token) counts the experts that precede it (E / 64
// comparisons per lane, then a wave sum).  Exactly k experts get a rank < k;
// each writes its id and logit into slot `rank` of the token's selection.
// grid (ceil(E / 4), T), 256 threads.
__global__ __launch_bounds__(256) void k_rank(const double *__restrict__ logits, int E, int k,
                                              int32_t *__restrict__ ids, double *__restrict__ sel) {
    const int t = blockIdx.y;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (e >= E) return;
    const double *lg = logits + (size_t)t * E;
    const double me = rank_value(lg[e]);
    double cnt = 0.0;
    for (int o = lane; o < E; o += 64) {
        const double v = rank_value(lg[o]);
        cnt += (v > me || (v == me && o < e)) ? 1.0 : 0.0;
    }
    const int rank = (int)wave_sum(cnt);
    if (lane == 0 && rank < k) {
        ids[(size_t)t * k + rank] = e;
        sel[(size_t)t * k + rank] = me;
    }
}

// One wave per token: softmax over the k selected logits (slot 0 is the largest).
__global__ __launch_bounds__(64) void k_gates(const double *__restrict__ sel, int k, float *__restrict__ gates) {
    const int t = blockIdx.x, lane = threadIdx.x;
    const double top = sel[(size_t)t * k];
    double ex = 0.0;
    for (int j = lane; j < k; j += 64) ex += exp(sel[(size_t)t * k + j] - top);
    const double sum = wave_sum(ex);
    for (int j = lane; j < k; j += 64) gates[(size_t)t * k + j] = (float)(exp(sel[(size_t)t * k + j] - top) / sum);
}

hipError_t launch_route(const Geometry &g, const Workspace &w, const float *x, const float *Wt, int T, int pre,
                        double eps, int32_t *ids, float *gates, hipStream_t s) {
    if (T == 1) {
        hipLaunchKernelGGL(k_route<1>, dim3(g.E, 1), dim3(256), 0, s, x, Wt, g.d, g.E, T, pre, eps, w.logits);
    } else {
        hipLaunchKernelGGL(k_route<kRouteTok>, dim3(g.E, (T + kRouteTok - 1) / kRouteTok), dim3(256), 0, s, x, Wt,
                           g.d, g.E, T, pre, eps, w.logits);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_rank, dim3((g.E + 3) / 4, T), dim3(256), 0, s, w.logits, g.E, g.k, ids, w.sel);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_gates, dim3(T), dim3(64), 0, s, w.sel, g.k, gates);
    return hipGetLastError();
}

}  // namespace rvq
