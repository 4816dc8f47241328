// ceilings.hip -- measured ceilings of the machine the layer runs on, for the
// benchmark's report (not part of the layer library).
//
//  - HBM streaming read: every byte of a large buffer read once with 16-byte
//    non-temporal loads, four in flight per thread, XOR-folded so that the
//    loads cannot be dropped; the achievable read rate that the table path's
//    code streaming is compared with.
//  - LDS random gather: the table path's inner operation -- a 4-byte read from
//    a 128 KB table at an address formed from a random code byte, lane l of
//    each half-wave always in bank l -- issued back to back by 16 waves per
//    CU; reported as lookups per second (one lookup per code byte).
//  - Kernel-to-kernel gap: a chain of launches on one stream of a grid shaped
//    like the persistent layer kernel (one 1024-thread workgroup per CU with
//    most of the LDS), each doing nothing; the time per launch is the fixed
//    cost every layer call pays.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_read(const u32x4 *__restrict__ p, uint64_t n16, uint32_t *__restrict__ out) {
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        const u32x4 b = __builtin_nontemporal_load(p + i + stride);
        const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < n16; i += stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u) out[blockIdx.x] = acc;  // practically never: keeps the loads live
}

// 1024 threads; the table is 32768 words of LDS.  Each iteration every lane
// makes 48 lookups (one 32-row chunk's worth) at word c * 64 + 32 * (s == 1)
// + 16384 * (s == 2) + l for pseudo-random codes c.
__global__ __launch_bounds__(1024) void k_lds_gather(int iters, float *__restrict__ out) {
    __shared__ float lut[32768];
    for (int i = threadIdx.x; i < 32768; i += 1024) lut[i] = (float)(i & 255);
    __syncthreads();
    const int l = threadIdx.x & 31;
    uint32_t h = 0x9E3779B9u * (threadIdx.x + 1) + blockIdx.x;
    float acc = 0.f;
    for (int it = 0; it < iters; it++) {
        float t[48];
#pragma unroll
        for (int q = 0; q < 16; q++) {
            h = h * 1664525u + 1013904223u;
            const uint32_t c0 = h >> 24, c1 = (h >> 16) & 255, c2 = (h >> 8) & 255;
            t[3 * q] = lut[c0 * 64 + l];
            t[3 * q + 1] = lut[c1 * 64 + 32 + l];
            t[3 * q + 2] = lut[16384 + c2 * 64 + l];
        }
#pragma unroll
        for (int q = 0; q < 48; q++) acc += t[q];
    }
    if (acc == -1.f) out[blockIdx.x] = acc;
}

__global__ __launch_bounds__(1024) void k_empty(int *__restrict__ out) {
    __shared__ int big[32768];  // 128 KB of LDS: one workgroup per CU, like the layer kernel
    if (threadIdx.x == 0x7fffffff) out[0] = big[0];
}

extern "C" {

// Each returns 0 or a hipError_t; *ms gets the elapsed time of the timed part.
int vqe_ceiling_read(const void *buf, uint64_t bytes, int reps, void *stream, float *ms) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    int n_cu = 0, dev = 0;
    hipGetDevice(&dev);
    hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    const int blocks = n_cu * 8;
    uint32_t *out = nullptr;
    hipError_t e = hipMalloc(&out, sizeof(uint32_t) * blocks);
    if (e != hipSuccess) return (int)e;
    hipEvent_t a, b;
    hipEventCreate(&a);
    hipEventCreate(&b);
    const uint64_t n16 = bytes / 16;
    hipLaunchKernelGGL(k_read, dim3(blocks), dim3(256), 0, s, static_cast<const u32x4 *>(buf), n16, out);  // warm
    hipEventRecord(a, s);
    for (int r = 0; r < reps; r++)
        hipLaunchKernelGGL(k_read, dim3(blocks), dim3(256), 0, s, static_cast<const u32x4 *>(buf), n16, out);
    hipEventRecord(b, s);
    e = hipEventSynchronize(b);
    if (e == hipSuccess) e = hipEventElapsedTime(ms, a, b);
    hipEventDestroy(a);
    hipEventDestroy(b);
    hipFree(out);
    return (int)e;
}

int vqe_ceiling_lds_gather(int iters, void *stream, float *ms, int *blocks_out) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    int n_cu = 0, dev = 0;
    hipGetDevice(&dev);
    hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    float *out = nullptr;
    hipError_t e = hipMalloc(&out, sizeof(float) * n_cu);
    if (e != hipSuccess) return (int)e;
    hipEvent_t a, b;
    hipEventCreate(&a);
    hipEventCreate(&b);
    hipLaunchKernelGGL(k_lds_gather, dim3(n_cu), dim3(1024), 0, s, 8, out);
    hipEventRecord(a, s);
    hipLaunchKernelGGL(k_lds_gather, dim3(n_cu), dim3(1024), 0, s, iters, out);
    hipEventRecord(b, s);
    e = hipEventSynchronize(b);
    if (e == hipSuccess) e = hipEventElapsedTime(ms, a, b);
    *blocks_out = n_cu;
    hipEventDestroy(a);
    hipEventDestroy(b);
    hipFree(out);
    return (int)e;
}

int vqe_ceiling_launch_gap(int launches, void *stream, float *ms) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    int n_cu = 0, dev = 0;
    hipGetDevice(&dev);
    hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    int *out = nullptr;
    hipError_t e = hipMalloc(&out, sizeof(int));
    if (e != hipSuccess) return (int)e;
    hipEvent_t a, b;
    hipEventCreate(&a);
    hipEventCreate(&b);
    for (int i = 0; i < 8; i++) hipLaunchKernelGGL(k_empty, dim3(n_cu), dim3(1024), 0, s, out);
    hipEventRecord(a, s);
    for (int i = 0; i < launches; i++) hipLaunchKernelGGL(k_empty, dim3(n_cu), dim3(1024), 0, s, out);
    hipEventRecord(b, s);
    e = hipEventSynchronize(b);
    if (e == hipSuccess) e = hipEventElapsedTime(ms, a, b);
    hipEventDestroy(a);
    hipEventDestroy(b);
    hipFree(out);
    return (int)e;
}

}  // extern "C"
