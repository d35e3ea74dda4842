// Microbenchmarks of the two ceilings the BitLinear kernels are measured
// against, so that bench.py can report every fraction against the measured
// peak as well as the published one (MI355X: 8 TB/s HBM3E, 5.0 POP/s dense
// int8 MFMA):
//   peaks_read     streams a device buffer once (16-byte non-temporal loads,
//                  grid-strided) and folds it into one word per thread, which
//                  is stored only if it matches a value it cannot take, so
//                  the loads are not optimised away;
//   peaks_mfma_i8  runs v_mfma_i32_32x32x32_i8 back to back from registers
//                  (eight independent accumulators per wave, no memory
//                  traffic in the loop): 65536 int8 ops per instruction.
// Built by bitlinear_absmean_ternarise_amd/build.py into libbench_peaks.so;
// not part of the library.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void peak_read_kernel(const v4u *__restrict__ src, int64_t n16,
                                                        uint32_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t a = 0;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const v4u v0 = __builtin_nontemporal_load(src + i);
        const v4u v1 = __builtin_nontemporal_load(src + i + stride);
        const v4u v2 = __builtin_nontemporal_load(src + i + 2 * stride);
        const v4u v3 = __builtin_nontemporal_load(src + i + 3 * stride);
        a ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
        a ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
    }
    for (; i < n16; i += stride) {
        const v4u v = __builtin_nontemporal_load(src + i);
        a ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (a == 0x9E3779B9u) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = a;
}

__global__ __launch_bounds__(256) void peak_mfma_i8_kernel(int iters, int *__restrict__ sink) {
    const int t = threadIdx.x;
    const v4i a = {t, t + 1, t + 2, t + 3};
    const v4i b = {t ^ 5, t ^ 7, t ^ 9, t ^ 11};
    v16i c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = v16i{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += c[j][e];
    if (s == 0x1234567) sink[blockIdx.x * blockDim.x + t] = s;
}

extern "C" {

// Reads `bytes` (a multiple of 16) of device memory at `src` once.  `sink`:
// device buffer of blocks * 256 words (written only in the impossible case).
int peaks_read(const void *src, int64_t bytes, void *sink, int blocks, void *stream) {
    if (!src || !sink || bytes <= 0 || (bytes & 15) || blocks <= 0) return -1;
    hipLaunchKernelGGL(peak_read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const v4u *>(src), bytes / 16, static_cast<uint32_t *>(sink));
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// blocks x 256 threads (4 waves) each run iters x 8 MFMAs of 65536 int8 ops.
int peaks_mfma_i8(int iters, int blocks, void *sink, void *stream) {
    if (!sink || iters <= 0 || blocks <= 0) return -1;
    hipLaunchKernelGGL(peak_mfma_i8_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                       static_cast<int *>(sink));
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
