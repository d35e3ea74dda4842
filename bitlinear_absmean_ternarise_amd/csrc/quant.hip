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

// Fast path of the same arithmetic.  t = x * s is the fp32 product; adding
// 1.5 * 2^23 rounds it to an integer, ties to even (the fp32 spacing there is
// 1), and leaves that integer in the low bits of the sum as two's complement,
// so its low byte is the int8 code.  The clip to +-127 of quant1 never
// applies: |x| <= absmax and s = RN(127 / max(absmax, eps)) give
// |t| <= 127 * (1 + 2^-24), which rounds to at most 127.  (The build keeps
// a * b + c unfused, so t is the rounded product.)
__device__ __forceinline__ uint32_t qbits(float x, float s) {
    const float t = x * s;
    return __float_as_uint(t + 12582912.0f);
}

// four bf16 (two dwords, element order lo, hi, lo, hi) -> four int8 codes
__device__ __forceinline__ uint32_t quant4(uint32_t w01, uint32_t w23, float s) {
    const uint32_t a = qbits(__uint_as_float(w01 << 16), s);
    const uint32_t b = qbits(__uint_as_float(w01 & 0xFFFF0000u), s);
    const uint32_t c = qbits(__uint_as_float(w23 << 16), s);
    const uint32_t d = qbits(__uint_as_float(w23 & 0xFFFF0000u), s);
    const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);  // a -> byte 0, b -> byte 1
    const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x04000C0Cu);  // c -> byte 2, d -> byte 3
    return lo | hi;
}

// Running absmax over bf16 pairs as integers: for values >= 0 the fp32 bit
// patterns order like the values.  The high element with its sign bit
// cleared is already an fp32 pattern; the low element shifted left by 17
// loses its sign bit and is twice its fp32 pattern (same order).
struct AbsMax {
    uint32_t hi = 0, lo2 = 0;
    __device__ __forceinline__ void add(uint32_t w) {
        hi = max(hi, w & 0x7FFF0000u);
        lo2 = max(lo2, w << 17);
    }
    __device__ __forceinline__ float value() const { return __uint_as_float(max(hi, lo2 >> 1)); }
};

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
    const v4u *row = reinterpret_cast<const v4u *>(x + m * K);
    const int64_t nvec = K / 8;
    v4u v[kIters];
    AbsMax am;
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        const int64_t idx = lane + 64 * i;
        if (idx < nvec) {
            v[i] = __builtin_nontemporal_load(row + idx);  // read once
#pragma unroll
            for (int j = 0; j < 4; ++j) am.add(v[i][j]);
        }
    }
    const float a = wave_max_nonneg(am.value());
    const float s = 127.0f / fmaxf(a, eps);
    if (lane == 0) xs[m] = s;
    uint2 *out = reinterpret_cast<uint2 *>(xq + m * K);
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        const int64_t idx = lane + 64 * i;
        if (idx < nvec) out[idx] = make_uint2(quant4(v[i].x, v[i].y, s), quant4(v[i].z, v[i].w, s));
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
    const v4u *row = reinterpret_cast<const v4u *>(x + m * K);
    const int64_t nvec = K / 8;
    v4u v[kIters];
    AbsMax am;
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        const int64_t idx = threadIdx.x + 1024 * i;
        if (idx < nvec) {
            v[i] = __builtin_nontemporal_load(row + idx);  // read once
#pragma unroll
            for (int j = 0; j < 4; ++j) am.add(v[i][j]);
        }
    }
    float a = wave_max_nonneg(am.value());
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
        if (idx < nvec) out[idx] = make_uint2(quant4(v[i].x, v[i].y, s), quant4(v[i].z, v[i].w, s));
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
    a = wave_max_nonneg(a);
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
