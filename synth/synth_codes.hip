// synth_codes.hip -- on-device generation of the seeded canonical code bytes.
//
// Input-generation infrastructure (no arithmetic of the layer).  Produces the
// same bytes as synth.py's expert_record(): word w of expert e's record is
// mix64(key(seed, layer, e) + (w + 1) * GAMMA), stored little-endian, where
// mix64 is the SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014,
// Stafford "Mix13" constants).  Generating on the device avoids moving
// gigabytes of codes across PCIe for the large shapes.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kM1 = 0xBF58476D1CE4E5B9ull;
constexpr uint64_t kM2 = 0x94D049BB133111EBull;
constexpr uint64_t kSalt = 0x5851F42D4C957F2Dull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * kM1;
    z = (z ^ (z >> 27)) * kM2;
    return z ^ (z >> 31);
}

uint64_t expert_key(uint64_t seed, int layer, int expert) {
    uint64_t k = mix64(seed ^ kSalt);
    k = mix64(k + (uint64_t)(layer + 1) * kGamma);
    return mix64(k + (uint64_t)(expert + 1) * kGamma);
}

__global__ __launch_bounds__(256) void k_codes(uint64_t *__restrict__ dst, uint64_t key, uint64_t n_words) {
    const uint64_t w = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    if (w < n_words) dst[w] = mix64(key + (w + 1) * kGamma);
}

}  // namespace

// Writes the records of experts [expert0, expert0 + n_experts) back to back at
// dst (device, record_bytes each, record_bytes % 8 == 0).  Returns 0 or -1.
extern "C" int vqe_synth_codes(uint8_t *dst, uint64_t seed, int layer, int expert0, int n_experts,
                               uint64_t record_bytes, void *stream) {
    if (!dst || n_experts < 0 || record_bytes % 8) return -1;
    const uint64_t n_words = record_bytes / 8;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int i = 0; i < n_experts; i++) {
        const uint64_t key = expert_key(seed, layer, expert0 + i);
        const uint64_t blocks = (n_words + 255) / 256;
        hipLaunchKernelGGL(k_codes, dim3((unsigned)blocks), dim3(256), 0, s,
                           reinterpret_cast<uint64_t *>(dst + (uint64_t)i * record_bytes), key, n_words);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    return 0;
}
