// router.hip -- router logits, top-k and softmax gates.
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
// MI355X mapping.  The router matrix is stored transposed ([E][d]).
//   One token (decode): one launch of E workgroups, each streaming one
//   expert's row as contiguous wave loads; every workgroup publishes its
//   logit into a slot that holds a marker value, polls the E slots, and ranks
//   its own expert (the experts ahead of it in the order); the k with rank < k
//   publish their logit by rank, poll those k, and write id and gate.
//   Several tokens: the logits are a dense [T][d] x [d][E] contraction, done
//   in fp64 on the matrix cores (16 x 16 tiles); then one workgroup per token
//   selects its k (radix select over order-preserving 64-bit keys) and forms
//   the gates.
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
// NaN logits rank below every number (and among themselves by id).
__device__ inline double rank_value(double v) { return isnan(v) ? -INFINITY : v; }

// (va, expert ia) comes before (vb, ib) in the strict order: logit descending, id ascending.
__device__ inline bool before(double va, int ia, double vb, int ib) { return va > vb || (va == vb && ia < ib); }

// Top-k selection in one 256-thread workgroup by radix select.  Logits become
// order-preserving 64-bit keys (NaN ranks as -inf, -0 as +0, so equal keys are
// exactly the ties of the fp64 order).  The leading bits every key shares are
// fixed first (a block-wide AND / OR).  Then four bits at a time, a 16-bin
// histogram of the candidates' next digit fixes the digit of the k-th largest
// key, until the candidates sharing the fixed prefix are exactly the ones still
// needed (or all 64 bits are fixed: then equal keys go by lower id).  Each wave
// counts its digits with ballots (no contended LDS atomics), every thread reads
// the 16 bins and finds the digit itself, and the histograms rotate over three
// buffers, so a pass costs one barrier.
constexpr int kSelPer = kMaxExperts / 256;  // experts per thread

__device__ inline uint64_t order_key(double v) {
    v = rank_value(v);
    if (v == 0.0) v = 0.0;
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// Sum over each row of 16 lanes (every lane of the row gets it).
__device__ inline int row16_sum(int v) {
    v += (int)RVQ_DPP_U((uint32_t)v, kDppXor1);
    v += (int)RVQ_DPP_U((uint32_t)v, kDppXor2);
    v += (int)RVQ_DPP_U((uint32_t)v, kDppRor4);
    v += (int)RVQ_DPP_U((uint32_t)v, kDppRor8);
    return v;
}

// Bitwise AND (and OR) over the wave, every lane gets it.
__device__ inline uint32_t wave_and(uint32_t v) {
    v &= RVQ_DPP_U(v, kDppXor1);
    v &= RVQ_DPP_U(v, kDppXor2);
    v &= RVQ_DPP_U(v, kDppRor4);
    v &= RVQ_DPP_U(v, kDppRor8);
    const bool o16 = threadIdx.x & 16, o32 = threadIdx.x & 32;
    v &= swap_other(v, false, o16);
    v &= swap_other(v, true, o32);
    return v;
}

struct SelectLds {
    uint64_t key[kMaxExperts];
    int hist[3][16];
    uint32_t red[4][4];  // per wave: AND lo, AND hi, ~OR lo, ~OR hi
    int n_cand;
    uint64_t cand_key[kMaxTopK];
    double cand_v[kMaxTopK];
    int cand_id[kMaxTopK];
};

// Expert i = threadIdx.x + 256 r (i < E) has value v[r] (its rank value) and
// key[r].  Writes the k selected ids in the strict order (logit descending, id
// ascending) to ids_out and their values to v_out (LDS).
__device__ void select_topk(const uint64_t (&key)[kSelPer], const double (&v)[kSelPer], int E, int k, SelectLds &L,
                            int32_t *ids_out, double *v_out) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // ---- bits shared by every key
    uint64_t all_and = ~0ull, all_nor = ~0ull;  // AND of keys, AND of complemented keys
#pragma unroll
    for (int r = 0; r < kSelPer; r++) {
        if (tid + 256 * r < E) {
            L.key[tid + 256 * r] = key[r];
            all_and &= key[r];
            all_nor &= ~key[r];
        }
    }
    {
        const uint32_t a0 = wave_and((uint32_t)all_and), a1 = wave_and((uint32_t)(all_and >> 32));
        const uint32_t n0 = wave_and((uint32_t)all_nor), n1 = wave_and((uint32_t)(all_nor >> 32));
        if (lane == 0) {
            L.red[wave][0] = a0;
            L.red[wave][1] = a1;
            L.red[wave][2] = n0;
            L.red[wave][3] = n1;
        }
    }
    if (tid < 32) L.hist[tid >> 4][tid & 15] = 0;
    if (tid == 0) L.n_cand = 0;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < 4; w++) {
        all_and &= ((uint64_t)L.red[w][1] << 32) | L.red[w][0];
        all_nor &= ((uint64_t)L.red[w][3] << 32) | L.red[w][2];
    }
    const uint64_t differ = ~(all_and | all_nor);  // bits where two keys differ
    int used = differ ? (__clzll((long long)differ) & ~3) : 64;
    uint64_t prefix = used == 0 ? 0 : (used == 64 ? all_and : all_and >> (64 - used));
    int need = k, buf = 0;
    bool all_in = false;
    // ---- four bits per pass
    while (used < 64) {
        int *h = L.hist[buf];
        int cnt = 0;  // lane j < 16: this wave's count of digit j
#pragma unroll
        for (int r = 0; r < kSelPer; r++) {
            const bool live = tid + 256 * r < E && (used == 0 || (key[r] >> (64 - used)) == prefix);
            if (__ballot(live) == 0) continue;
            const int dg = (int)((key[r] >> (60 - used)) & 15);
#pragma unroll
            for (int j = 0; j < 16; j++) {
                const int c = __popcll(__ballot(live && dg == j));
                cnt += lane == j ? c : 0;
            }
        }
        if (lane < 16 && cnt) atomicAdd(&h[lane], cnt);
        __syncthreads();
        if (tid < 16) L.hist[buf == 0 ? 2 : buf - 1][tid] = 0;  // the buffer two passes ahead
        int c[16];
#pragma unroll
        for (int j = 0; j < 16; j++) c[j] = h[j];
        int dgt = 0, gt = 0, eq = 0, above = 0;
#pragma unroll
        for (int j = 15; j >= 0; j--) {
            if (above < need && need <= above + c[j]) {
                dgt = j;
                gt = above;
                eq = c[j];
            }
            above += c[j];
        }
        prefix = (prefix << 4) | (uint64_t)dgt;
        used += 4;
        need -= gt;
        buf = buf == 2 ? 0 : buf + 1;
        if (eq == need) {
            all_in = true;
            break;
        }
    }
    // ---- the selected experts: prefix above the threshold's, or equal to it
    // and (all of those are needed, or among the `need` lowest ids of equal keys)
#pragma unroll
    for (int r = 0; r < kSelPer; r++) {
        const int i = tid + 256 * r;
        if (i >= E) continue;
        const uint64_t top = used == 64 ? key[r] : key[r] >> (64 - used);
        bool in = top > prefix;
        if (top == prefix) {
            if (all_in) {
                in = true;
            } else {
                int lower = 0;
                for (int j = 0; j < i; j++) lower += L.key[j] == key[r];
                in = lower < need;
            }
        }
        if (in) {
            const int slot = atomicAdd(&L.n_cand, 1);
            L.cand_key[slot] = key[r];
            L.cand_v[slot] = v[r];
            L.cand_id[slot] = i;
        }
    }
    __syncthreads();
    // ---- order the k: a row of 16 lanes per candidate, each lane comparing a
    // sixteenth of the others, summed across the row
    for (int j = tid >> 4; j < k; j += 16) {
        const uint64_t mk = L.cand_key[j];
        const int mi = L.cand_id[j];
        int ahead = 0;
        for (int q = tid & 15; q < k; q += 16) {
            const uint64_t ok = L.cand_key[q];
            ahead += ok > mk || (ok == mk && L.cand_id[q] < mi);
        }
        const int rank = row16_sum(ahead);
        if ((tid & 15) == 0) {
            ids_out[rank] = mi;
            v_out[rank] = L.cand_v[j];
        }
    }
    __syncthreads();
}


// Router dot products of expert e (= blockIdx.x) for tokens [t0, t0 + nt):
// 256 threads; the 4 waves each take a quarter of the expert's column (float4
// granules), all of a lane's loads of a pass in flight together.  out[t] (LDS)
// gets the logit, sum / r, for every thread after the internal barrier.
template <int TT>
__device__ void router_dot(const float *__restrict__ x, const float *__restrict__ Wt, int d, int t0, int nt, int pre,
                           double eps, double *out) {
    const int e = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n4 = d / 4;
    const int g0 = n4 * wave / 4, g1 = n4 * (wave + 1) / 4;
    const float4 *w4 = reinterpret_cast<const float4 *>(Wt + (size_t)e * d);
    constexpr int kU = TT == 1 ? 8 : 2;  // float4 loads per lane per pass
    double acc[TT], ss[TT];
#pragma unroll
    for (int t = 0; t < TT; t++) acc[t] = ss[t] = 0.0;
    for (int base = g0 + lane; base < g1; base += 64 * kU) {
        // loads are unconditional (clamped index) so that all of them are in
        // flight together; granules past the end are dropped where they are used
        float4 wv[kU];
        bool ok[kU];
#pragma unroll
        for (int u = 0; u < kU; u++) {
            ok[u] = base + 64 * u < g1;
            wv[u] = w4[min(base + 64 * u, g1 - 1)];
        }
#pragma unroll
        for (int t = 0; t < TT; t++) {
            if (t >= nt) break;
            const float4 *x4 = reinterpret_cast<const float4 *>(x + (size_t)(t0 + t) * d);
            float4 xv[kU];
#pragma unroll
            for (int u = 0; u < kU; u++) xv[u] = x4[min(base + 64 * u, g1 - 1)];
#pragma unroll
            for (int u = 0; u < kU; u++) {
                const double x0 = ok[u] ? (double)xv[u].x : 0.0, x1 = ok[u] ? (double)xv[u].y : 0.0;
                const double x2 = ok[u] ? (double)xv[u].z : 0.0, x3 = ok[u] ? (double)xv[u].w : 0.0;
                acc[t] = fma(x0, (double)wv[u].x, acc[t]);
                acc[t] = fma(x1, (double)wv[u].y, acc[t]);
                acc[t] = fma(x2, (double)wv[u].z, acc[t]);
                acc[t] = fma(x3, (double)wv[u].w, acc[t]);
                if (pre) {
                    ss[t] = fma(x0, x0, ss[t]);
                    ss[t] = fma(x1, x1, ss[t]);
                    ss[t] = fma(x2, x2, ss[t]);
                    ss[t] = fma(x3, x3, ss[t]);
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
        out[t] = sa / r;
    }
    __syncthreads();
}

// Several tokens, step 1: the logits as a dense fp64 contraction on the
// matrix cores, L[t][e] = sum_i x[t][i] Wt[e][i] with v_mfma_f64_16x16x4_f64
// (fp32 inputs widened exactly, so every product is exact; fp64 sums).  Grid
// (ceil(E / 16), ceil(T / 16), S), 256 threads: the input dimension is split
// into S parts (so that few tokens still fill the GPU) and each part into four,
// one per wave of one 16 token x 16 expert tile; the four partial tiles are
// summed in wave order and written to part s of logits ([S][T][E]), which the
// selection sums in part order.  Operands: lane l = 16 q + r loads 4
// consecutive inputs 16 b + 4 q .. + 3 of token row r and of expert row r;
// MFMA step j pairs the j-th of them (A[r][q] = x, B[q][r] = w), so the four
// steps of a block cover its 16 inputs once.  The accumulator v of lane l is
// D[q + 4 v][r] (token q + 4 v, expert r; measured on gfx950).  Rows past T or
// E are clamped on load and dropped on store.
typedef double f64x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void k_route_mm(const float *__restrict__ x, const float *__restrict__ Wt, int d,
                                                  int E, int T, double *__restrict__ logits) {
    const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
    const float *xr = x + (size_t)min(t0 + r, T - 1) * d;
    const float *wr = Wt + (size_t)min(e0 + r, E - 1) * d;
    const int nq = 4 * gridDim.z, qi = 4 * blockIdx.z + wave;  // this wave's quarter of part blockIdx.z
    const int nb = (d + 15) / 16, b0 = (int)((int64_t)nb * qi / nq), b1 = (int)((int64_t)nb * (qi + 1) / nq);
    logits += (size_t)blockIdx.z * T * E;
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
    // kU blocks per pass with all their loads in flight together; the next
    // pass's loads are issued before this pass's products (two register sets)
    constexpr int kU = 4;
    float4 xv[2][kU], wv[2][kU];
    auto load = [&](int set, int b) {
#pragma unroll
        for (int u = 0; u < kU; u++) {
            const int i = (b + u) * 16 + 4 * q;
            const bool ok = b + u < b1 && i < d;  // d % 8 == 0: a 4-aligned start below d has all 4 below d
            xv[set][u] = ok ? *reinterpret_cast<const float4 *>(xr + i) : make_float4(0.f, 0.f, 0.f, 0.f);
            wv[set][u] = ok ? *reinterpret_cast<const float4 *>(wr + i) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto products = [&](int set) {
#pragma unroll
        for (int u = 0; u < kU; u++) {
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[set][u].x, (double)wv[set][u].x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[set][u].y, (double)wv[set][u].y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[set][u].z, (double)wv[set][u].z, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[set][u].w, (double)wv[set][u].w, acc, 0, 0, 0);
        }
    };
    if (b0 < b1) load(0, b0);
    for (int b = b0; b < b1; b += 2 * kU) {  // the sets alternate with no copies between them
        if (b + kU < b1) load(1, b + kU);
        products(0);
        if (b + kU >= b1) break;
        if (b + 2 * kU < b1) load(0, b + 2 * kU);
        products(1);
    }
    __shared__ double part[4][16][17];  // [wave][token][expert], padded
#pragma unroll
    for (int v = 0; v < 4; v++) part[wave][q + 4 * v][r] = acc[v];
    __syncthreads();
    const int tt = threadIdx.x >> 4, ee = threadIdx.x & 15;  // 256 threads = the 16 x 16 tile
    if (t0 + tt < T && e0 + ee < E)
        logits[(size_t)(t0 + tt) * E + e0 + ee] = ((part[0][tt][ee] + part[1][tt][ee]) + part[2][tt][ee]) +
                                                  part[3][tt][ee];
}

// Several tokens, step 2: grid (T), 256 threads, one token each.  Divides the
// token's logits by its RMS divisor (fp64, when normalising), selects the k
// largest (ties to the lower id) and forms the softmax gates over them (one exp
// per selected logit, summed in slot order).
__global__ __launch_bounds__(256) void k_route_sel(const float *__restrict__ x, int d, int E, int k, int pre,
                                                   double eps, const double *__restrict__ logits, int S, int T,
                                                   int32_t *__restrict__ ids, float *__restrict__ gates) {
    const int t = blockIdx.x;
    __shared__ SelectLds L;
    __shared__ double sel[kMaxTopK];
    __shared__ double ex[kMaxTopK];
    __shared__ double red[4];
    double rdiv = 1.0;
    if (pre) {
        const float *xt = x + (size_t)t * d;
        double ss = 0.0;
        for (int i = threadIdx.x; i < d; i += 256) ss = fma((double)xt[i], (double)xt[i], ss);
        ss = wave_sum(ss);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
        __syncthreads();
        rdiv = sqrt((red[0] + red[1] + red[2] + red[3]) / (double)d + eps);
    }
    double v[kSelPer];
    uint64_t key[kSelPer];
#pragma unroll
    for (int r = 0; r < kSelPer; r++) {
        const int i = threadIdx.x + 256 * r;
        double l = 0.0;  // the S parts, in part order
        if (i < E)
            for (int s = 0; s < S; s++) l += logits[((size_t)s * T + t) * E + i];
        v[r] = rank_value(i < E ? l / rdiv : -INFINITY);
        key[r] = order_key(v[r]);
    }
    select_topk(key, v, E, k, L, ids + (size_t)t * k, sel);
    if (threadIdx.x < k) ex[threadIdx.x] = exp(sel[threadIdx.x] - sel[0]);
    __syncthreads();
    if (threadIdx.x < k) {
        double sum = 0.0;
        for (int j = 0; j < k; j++) sum += ex[j];
        gates[(size_t)t * k + threadIdx.x] = (float)(ex[threadIdx.x] / sum);
    }
}

// One token: grid (E), 256 threads, every workgroup resident at once (checked
// when the handle is opened).  No workgroup selects for the others: each
// publishes its logit, polls until all E are in, and counts the experts ahead
// of its own in the strict order (logit descending, id ascending).  The k with
// rank < k publish their logit into slot `rank`, poll the k slots, and write
// their id and gate.  Buffers alternate between calls (parity), and each
// workgroup puts kUnpublished into the other buffer's slots it owns, for the
// next call: nobody can still be reading those.  Waits are bounded (~0.5 s,
// then err bit 2).
__global__ __launch_bounds__(256) void k_route_one(const float *__restrict__ x, const float *__restrict__ Wt, int d,
                                                   int E, int k, int pre, double eps, double *__restrict__ lg_cur,
                                                   double *__restrict__ lg_next, double *__restrict__ sel_cur,
                                                   double *__restrict__ sel_next, int *__restrict__ err,
                                                   int32_t *__restrict__ ids, float *__restrict__ gates) {
    const int e = blockIdx.x, tid = threadIdx.x;
    const double unpub = __longlong_as_double((long long)kUnpublished);
    __shared__ double lgt[1];
    router_dot<1>(x, Wt, d, 0, 1, pre, eps, lgt);
    const double mine = lgt[0];
    if (tid == 0) {
        store_coherent(lg_cur + e, mine);
        store_coherent(lg_next + e, unpub);
    }
    const uint64_t t_start = wall_clock64();
    auto timed_out = [&]() {
        if (wall_clock64() - t_start > 50000000ull) {  // 0.5 s at the 100 MHz constant clock
            if (tid == 0) atomicOr(err, 2);
            return true;
        }
        __builtin_amdgcn_s_sleep(1);
        return false;
    };
    double v[kSelPer];
    while (true) {
        int ready = 1;
#pragma unroll
        for (int r = 0; r < kSelPer; r++) {
            const int i = tid + 256 * r;
            v[r] = i < E ? load_coherent(lg_cur + i) : 0.0;
            ready &= (uint64_t)__double_as_longlong(v[r]) != kUnpublished;
        }
        if (__syncthreads_and(ready) || timed_out()) break;
    }
    // rank of e
    const double me = rank_value(mine);
    int ahead = 0;
#pragma unroll
    for (int r = 0; r < kSelPer; r++) {
        const int i = tid + 256 * r;
        if (i < E) ahead += before(rank_value(v[r]), i, me, e);
    }
    __shared__ int part[4];
    ahead = row16_sum(ahead);
    ahead += (int)swap_other((uint32_t)ahead, false, tid & 16);
    ahead += (int)swap_other((uint32_t)ahead, true, tid & 32);
    if ((tid & 63) == 0) part[tid >> 6] = ahead;
    __syncthreads();
    const int rank = part[0] + part[1] + part[2] + part[3];
    if (rank >= k) return;
    if (tid == 0) {
        store_coherent(sel_cur + rank, me);
        store_coherent(sel_next + rank, unpub);
        ids[rank] = e;
    }
    // gates: softmax over the k selected logits (slot 0 is the largest), one
    // exp per slot, summed in slot order
    __shared__ double ex[kMaxTopK];
    while (true) {
        double sv = 0.0;
        if (tid < k) sv = load_coherent(sel_cur + tid);
        const int ready = tid >= k || (uint64_t)__double_as_longlong(sv) != kUnpublished;
        if (__syncthreads_and(ready) || timed_out()) {
            if (tid < k) ex[tid] = sv;
            break;
        }
    }
    __syncthreads();
    if (tid < k) ex[tid] = exp(ex[tid] - ex[0]);
    __syncthreads();
    if (tid == 0) {
        double sum = 0.0;
        for (int j = 0; j < k; j++) sum += ex[j];
        gates[rank] = (float)(ex[rank] / sum);
    }
}

hipError_t launch_route(const Geometry &g, Workspace &w, const float *x, const float *Wt, int T, int pre, double eps,
                        int32_t *ids, float *gates, hipStream_t s) {
    if (T == 1 && w.route_one) {
        double *lg[2] = {w.route_logits + w.route_cap, w.route_logits + w.route_cap + g.E};
        double *sl[2] = {w.route_logits + w.route_cap + 2 * g.E, w.route_logits + w.route_cap + 2 * g.E + kMaxTopK};
        const int p = w.route_parity;
        hipLaunchKernelGGL(k_route_one, dim3(g.E), dim3(256), 0, s, x, Wt, g.d, g.E, g.k, pre, eps, lg[p], lg[p ^ 1],
                           sl[p], sl[p ^ 1], w.err, ids, gates);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;  // the buffers alternate only with an enqueued launch
        w.route_parity ^= 1;
        return hipSuccess;
    } else {
        // the logits area of the several-token path: plain values, handed from
        // the contraction to the selection across the launch boundary
        double *lg = w.route_logits;  // [S][T][E]
        // parts of the input dimension: enough workgroups for the GPU (~768),
        // at most 16, within the area (route_cap slots)
        const int tiles = ((g.E + 15) / 16) * ((T + 15) / 16);
        int S = 1;
        while (S < 16 && tiles * 2 * S <= 768 && (int64_t)2 * S * T * g.E <= w.route_cap && 2 * S * 4 <= g.d / 16)
            S *= 2;
        hipLaunchKernelGGL(k_route_mm, dim3((g.E + 15) / 16, (T + 15) / 16, S), dim3(256), 0, s, x, Wt, g.d, g.E, T,
                           lg);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_route_sel, dim3(T), dim3(256), 0, s, x, g.d, g.E, g.k, pre, eps, lg, S, T, ids, gates);
    }
    return hipGetLastError();
}

// The several-token area holds max(max_tokens, 256) x E values (parts of the
// input dimension for calls of up to 128 tokens), then the one-token path's
// alternating slots.
static int64_t route_cap(int64_t max_tokens, int E) { return (max_tokens > 256 ? max_tokens : 256) * E; }
int64_t route_logit_slots(int64_t max_tokens, int E) { return route_cap(max_tokens, E) + 2 * E + 2 * kMaxTopK; }

hipError_t init_route(Workspace &w, int E, int k, int64_t max_tokens, int n_cu, hipStream_t s) {
    w.route_cap = route_cap(max_tokens, E);
    w.fused_cap = max_tokens * E;
    w.route_parity = 0;
    // the one-token kernel needs all E workgroups resident together
    int per_cu = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_route_one, 256, 0);
    if (e != hipSuccess) return e;
    w.route_one = (int64_t)per_cu * n_cu >= E;
    w.fused_parity = 0;
    w.fused_prev_T = 0;
    const hipError_t e2 = hipMemsetD32Async(reinterpret_cast<hipDeviceptr_t>(w.fused_logits), kUnpublishedHalf,
                                            (size_t)(2 * fused_route_slots(max_tokens, E)), s);
    if (e2 != hipSuccess) return e2;
    return hipMemsetD32Async(reinterpret_cast<hipDeviceptr_t>(w.route_logits), kUnpublishedHalf,
                             (size_t)(2 * route_logit_slots(max_tokens, E)), s);
}

}  // namespace rvq
