// Per-token absmax int8 activation quantisation, no zero point ("1-bit &
// Ternary LLMs (BitNet b1.58)", BitNet activation equation and the b1.58
// paragraph that drops the zero point; "What 1.58 Bits Actually Changes",
// low-bit linear path: each token scaled into int8 on its own).
//
//   s_m = 127 / max(max_k |x[m][k]|, eps)   (correctly rounded fp32 divide)
//   q   = clip(rint(x * s_m), -127, 127)    (fp32 multiply, ties to even)
//
// The row is read once from HBM into registers, reduced with a wave (and
// for long rows a block) max, then quantised from the same registers:
// 2 B read + 1 B written per element.
#include "device.h"
#include "internal.h"

namespace bl {

namespace {

__device__ __forceinline__ int8_t quant1(float x, float s) {
    float r = rintf(x * s);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int8_t)(int)r;
}

__device__ __forceinline__ uint32_t quant2(uint32_t two_bf16, float s) {
    const uint32_t lo = (uint8_t)quant1(__uint_as_float(two_bf16 << 16), s);
    const uint32_t hi = (uint8_t)quant1(__uint_as_float(two_bf16 & 0xFFFF0000u), s);
    return lo | (hi << 8);
}

// One wave per row; row length K <= 64 * 8 * kIters, K % 8 == 0 (16-byte
// loads of 8 bf16 per lane).  Rows are 16-byte aligned because K % 8 == 0.
template <int kIters>
__global__ __launch_bounds__(256) void quant_rows_wave(const uint16_t *__restrict__ x, int64_t M,
                                                       int64_t K, float eps,
                                                       int8_t *__restrict__ xq,
                                                       float *__restrict__ xs) {
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    const uint4 *row = reinterpret_cast<const uint4 *>(x + m * K);
    const int64_t nvec = K / 8;
    uint4 v[kIters];
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        const int64_t idx = lane + 64 * i;
        if (idx < nvec) {
            v[i] = row[idx];
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                a = fmaxf(a, fabsf(__uint_as_float(w[j] << 16)));
                a = fmaxf(a, fabsf(__uint_as_float(w[j] & 0xFFFF0000u)));
            }
        }
    }
    a = wave_max(a);
    const float s = 127.0f / fmaxf(a, eps);
    if (lane == 0) xs[m] = s;
    uint2 *out = reinterpret_cast<uint2 *>(xq + m * K);
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        const int64_t idx = lane + 64 * i;
        if (idx < nvec) {
            uint2 o;
            o.x = quant2(v[i].x, s) | (quant2(v[i].y, s) << 16);
            o.y = quant2(v[i].z, s) | (quant2(v[i].w, s) << 16);
            out[idx] = o;
        }
    }
}

// One block of 1024 threads per row, for long rows (K % 8 == 0,
// K <= 1024 * 8 * kIters).
template <int kIters>
__global__ __launch_bounds__(1024) void quant_rows_block(const uint16_t *__restrict__ x,
                                                         int64_t K, float eps,
                                                         int8_t *__restrict__ xq,
                                                         float *__restrict__ xs) {
    const int64_t m = blockIdx.x;
    const uint4 *row = reinterpret_cast<const uint4 *>(x + m * K);
    const int64_t nvec = K / 8;
    uint4 v[kIters];
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        const int64_t idx = threadIdx.x + 1024 * i;
        if (idx < nvec) {
            v[i] = row[idx];
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                a = fmaxf(a, fabsf(__uint_as_float(w[j] << 16)));
                a = fmaxf(a, fabsf(__uint_as_float(w[j] & 0xFFFF0000u)));
            }
        }
    }
    a = wave_max(a);
    __shared__ float red[16];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    a = red[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) a = fmaxf(a, red[i]);
    const float s = 127.0f / fmaxf(a, eps);
    if (threadIdx.x == 0) xs[m] = s;
    uint2 *out = reinterpret_cast<uint2 *>(xq + m * K);
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        const int64_t idx = threadIdx.x + 1024 * i;
        if (idx < nvec) {
            uint2 o;
            o.x = quant2(v[i].x, s) | (quant2(v[i].y, s) << 16);
            o.y = quant2(v[i].z, s) | (quant2(v[i].w, s) << 16);
            out[idx] = o;
        }
    }
}

// Any K (unaligned rows): one block of 256 threads per row, scalar loads,
// two passes over the row (the second hits in cache).
__global__ __launch_bounds__(256) void quant_rows_scalar(const uint16_t *__restrict__ x, int64_t K,
                                                         float eps, int8_t *__restrict__ xq,
                                                         float *__restrict__ xs) {
    const int64_t m = blockIdx.x;
    const uint16_t *row = x + m * K;
    float a = 0.0f;
    for (int64_t k = threadIdx.x; k < K; k += 256) a = fmaxf(a, fabsf(bf16_to_f32(row[k])));
    a = wave_max(a);
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = 127.0f / fmaxf(a, eps);
    if (threadIdx.x == 0) xs[m] = s;
    for (int64_t k = threadIdx.x; k < K; k += 256) xq[m * K + k] = quant1(bf16_to_f32(row[k]), s);
}

}  // namespace

hipError_t launch_quant(const uint16_t *x, int64_t M, int64_t K, float eps, int8_t *xq, float *xs,
                        hipStream_t s) {
    if (K % 8 == 0 && K <= 64 * 8 * 8) {
        const unsigned grid = (unsigned)((M + 3) / 4);
        if (K <= 64 * 8 * 1)
            hipLaunchKernelGGL(quant_rows_wave<1>, dim3(grid), dim3(256), 0, s, x, M, K, eps, xq, xs);
        else if (K <= 64 * 8 * 2)
            hipLaunchKernelGGL(quant_rows_wave<2>, dim3(grid), dim3(256), 0, s, x, M, K, eps, xq, xs);
        else if (K <= 64 * 8 * 4)
            hipLaunchKernelGGL(quant_rows_wave<4>, dim3(grid), dim3(256), 0, s, x, M, K, eps, xq, xs);
        else
            hipLaunchKernelGGL(quant_rows_wave<8>, dim3(grid), dim3(256), 0, s, x, M, K, eps, xq, xs);
    } else if (K % 8 == 0 && K <= 1024 * 8 * 4) {
        if (K <= 1024 * 8 * 1)
            hipLaunchKernelGGL(quant_rows_block<1>, dim3((unsigned)M), dim3(1024), 0, s, x, K, eps, xq, xs);
        else if (K <= 1024 * 8 * 2)
            hipLaunchKernelGGL(quant_rows_block<2>, dim3((unsigned)M), dim3(1024), 0, s, x, K, eps, xq, xs);
        else
            hipLaunchKernelGGL(quant_rows_block<4>, dim3((unsigned)M), dim3(1024), 0, s, x, K, eps, xq, xs);
    } else {
        hipLaunchKernelGGL(quant_rows_scalar, dim3((unsigned)M), dim3(256), 0, s, x, K, eps, xq, xs);
    }
    return hipGetLastError();
}

}  // namespace bl
