// router.hip -- RMS normalisation prologue, router GEMV and top-k gates.
//
// [FR] "Lecture anticipée et prédiction du routeur": a layer's router decides
// the token's expert ids (16 for K3), and expert reads start from them.  The
// score function is not given on the pages; the reading taken is top-k of the
// raw logits (descending, ties to the lower id) and a softmax over the k
// selected logits.  Logits accumulate fp32 x fp32 products in fp64: each
// product is exact in fp64, so the only difference from any other summation
// order is fp64 rounding of the sum (~1e-16 relative), which keeps the
// selected ids reproducible.
#include <math.h>

#include "internal.hpp"

namespace rvq {

// ---------------------------------------------------------------------------
// r[t] = sqrt(sum_i x_i^2 / d + eps) in fp64 (1.0 without normalisation).
__global__ __launch_bounds__(256) void k_prep(const float *__restrict__ x, int d, int pre, double eps,
                                              double *__restrict__ r) {
    const int t = blockIdx.x;
    __shared__ double red[256];
    double ss = 0.0;
    if (pre) {
        const float *xt = x + (size_t)t * d;
        for (int i = threadIdx.x; i < d; i += 256) {
            double v = (double)xt[i];
            ss += v * v;
        }
    }
    red[threadIdx.x] = ss;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) r[t] = pre ? sqrt(red[0] / (double)d + eps) : 1.0;
}

hipError_t launch_prep(const Geometry &g, const Workspace &w, const float *x, int T, int pre,
                       double eps, hipStream_t s) {
    hipLaunchKernelGGL(k_prep, dim3(T), dim3(256), 0, s, x, g.d, pre, eps, w.tok_r);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Partial logits of kRouterRows rows of W_r for up to kRouterTok tokens:
// part[t][blk][e] = sum_{i in blk} x_hat[t][i] * W[i][e], fp64.
// x_hat = x / r (fp64 division, as the normalisation defines it).
template <int NC>
__global__ __launch_bounds__(256) void k_router(const float *__restrict__ x, const double *__restrict__ r,
                                                const float *__restrict__ W, int d, int E, int T,
                                                int n_rblk, double *__restrict__ part) {
    const int blk = blockIdx.x;
    const int t0 = blockIdx.y * kRouterTok;
    const int i0 = blk * kRouterRows;
    const int nrows = min(kRouterRows, d - i0);
    const int ntok = min(kRouterTok, T - t0);
    __shared__ double xs[kRouterTok][kRouterRows];
    for (int idx = threadIdx.x; idx < kRouterTok * kRouterRows; idx += 256) {
        const int tt = idx / kRouterRows, ii = idx % kRouterRows;
        double v = 0.0;
        if (tt < ntok && ii < nrows) v = (double)x[(size_t)(t0 + tt) * d + i0 + ii] / r[t0 + tt];
        xs[tt][ii] = v;
    }
    __syncthreads();
    double acc[kRouterTok][NC];
#pragma unroll
    for (int tt = 0; tt < kRouterTok; tt++)
#pragma unroll
        for (int c = 0; c < NC; c++) acc[tt][c] = 0.0;
    for (int ii = 0; ii < nrows; ii++) {
        const float *wr = W + (size_t)(i0 + ii) * E;
#pragma unroll
        for (int c = 0; c < NC; c++) {
            const int e = threadIdx.x + 256 * c;
            const double wv = e < E ? (double)wr[e] : 0.0;
#pragma unroll
            for (int tt = 0; tt < kRouterTok; tt++) acc[tt][c] = fma(xs[tt][ii], wv, acc[tt][c]);
        }
    }
#pragma unroll
    for (int tt = 0; tt < kRouterTok; tt++) {
        if (tt >= ntok) break;
#pragma unroll
        for (int c = 0; c < NC; c++) {
            const int e = threadIdx.x + 256 * c;
            if (e < E) part[((size_t)(t0 + tt) * n_rblk + blk) * E + e] = acc[tt][c];
        }
    }
}

hipError_t launch_router(const Geometry &g, const Workspace &w, const float *x, const float *router_w,
                         int T, hipStream_t s) {
    dim3 grid(w.n_rblk, (T + kRouterTok - 1) / kRouterTok);
    const int nc = (g.E + 255) / 256;
    switch (nc) {
        case 1: hipLaunchKernelGGL(k_router<1>, grid, dim3(256), 0, s, x, w.tok_r, router_w, g.d, g.E, T, w.n_rblk, w.route_part); break;
        case 2: hipLaunchKernelGGL(k_router<2>, grid, dim3(256), 0, s, x, w.tok_r, router_w, g.d, g.E, T, w.n_rblk, w.route_part); break;
        case 3: hipLaunchKernelGGL(k_router<3>, grid, dim3(256), 0, s, x, w.tok_r, router_w, g.d, g.E, T, w.n_rblk, w.route_part); break;
        default: hipLaunchKernelGGL(k_router<4>, grid, dim3(256), 0, s, x, w.tok_r, router_w, g.d, g.E, T, w.n_rblk, w.route_part); break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// One workgroup per token: sum the partial logits over row blocks (ascending),
// select the top k (value descending, id ascending; NaN ranks lowest) with
// wave64 argmax rounds, and write softmax gates over the selected logits.
__device__ inline bool better(double va, int ia, double vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(256) void k_topk(const double *__restrict__ part, int E, int k, int n_rblk,
                                              int32_t *__restrict__ ids, float *__restrict__ gates) {
    const int t = blockIdx.x;
    __shared__ double lg[kMaxExperts];
    __shared__ int taken[kMaxExperts];
    __shared__ double sel[kMaxTopK];
    for (int e = threadIdx.x; e < E; e += 256) {
        const double *p = part + (size_t)t * n_rblk * E + e;
        double acc = 0.0;
        for (int b = 0; b < n_rblk; b++) acc += p[(size_t)b * E];
        lg[e] = isnan(acc) ? -INFINITY : acc;
        taken[e] = 0;
    }
    __syncthreads();
    const int lane = threadIdx.x;
    for (int j = 0; j < k; j++) {
        if (lane < 64) {
            double bv = -INFINITY;
            int bi = 0x7fffffff;
            for (int e = lane; e < E; e += 64) {
                if (!taken[e] && (bi == 0x7fffffff || better(lg[e], e, bv, bi))) {
                    bv = lg[e];
                    bi = e;
                }
            }
            for (int o = 32; o > 0; o >>= 1) {
                const double ov = __shfl_xor(bv, o);
                const int oi = __shfl_xor(bi, o);
                if (oi != 0x7fffffff && (bi == 0x7fffffff || better(ov, oi, bv, bi))) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (lane == 0) {
                taken[bi] = 1;
                ids[(size_t)t * k + j] = bi;
                sel[j] = bv;
            }
        }
        __syncthreads();
    }
    if (lane >= 64) return;
    // softmax over the k selected logits, relative to the largest
    double ex = 0.0;
    for (int j = lane; j < k; j += 64) ex += exp(sel[j] - sel[0]);
    double sum = ex;
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    for (int j = lane; j < k; j += 64) gates[(size_t)t * k + j] = (float)(exp(sel[j] - sel[0]) / sum);
}

hipError_t launch_topk(const Geometry &g, const Workspace &w, int T, int32_t *ids, float *gates,
                       hipStream_t s) {
    hipLaunchKernelGGL(k_topk, dim3(T), dim3(256), 0, s, w.route_part, g.E, g.k, w.n_rblk, ids, gates);
    return hipGetLastError();
}

}  // namespace rvq
