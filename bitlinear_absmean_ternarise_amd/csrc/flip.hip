// Sign-flip tracker update ("Which 1-Bit Weights Can You Trust?",
// Methodology): compare the sign of every latent weight with its sign at the
// previous step; where it changed, bump the INT16 flip count (saturating at
// 32767) and record the step in the INT16 last-flip counter.
//
// Elementwise and HBM-bound: 4 weights per thread, so every load instruction
// of a wave covers contiguous memory (16 bytes of each snapshot and 8 bytes of
// each counter array per lane).  Counters are written back only where a sign
// changed (most lanes write nothing: 12 B read per weight, plus 4 B per
// weight of the 4-weight groups that hold a flip).
#include "device.h"
#include "internal.h"

namespace bl {

namespace {

__device__ __forceinline__ int sgn(float v) { return (v > 0.0f) - (v < 0.0f); }

__device__ __forceinline__ void update1(float p, float c, int16_t step, int16_t &fc, int16_t &lf) {
    if (sgn(p) != sgn(c)) {
        fc = (int16_t)(fc == 32767 ? 32767 : fc + 1);
        lf = step;
    }
}

__global__ __launch_bounds__(256) void flip_update_vec(const float *__restrict__ prev,
                                                       const float *__restrict__ curr, int64_t n4,
                                                       int16_t step, int16_t *__restrict__ fc,
                                                       int16_t *__restrict__ lf) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    typedef float v4f __attribute__((ext_vector_type(4)));
    typedef short v4s __attribute__((ext_vector_type(4)));
    const v4f p = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(prev) + i);
    const v4f c = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(curr) + i);
    v4s f = reinterpret_cast<const v4s *>(fc)[i];
    v4s l = reinterpret_cast<const v4s *>(lf)[i];
    bool any = false;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        if (sgn(p[t]) != sgn(c[t])) {
            f[t] = (short)(f[t] == 32767 ? 32767 : f[t] + 1);
            l[t] = step;
            any = true;
        }
    }
    if (any) {
        reinterpret_cast<v4s *>(fc)[i] = f;
        reinterpret_cast<v4s *>(lf)[i] = l;
    }
}

__global__ __launch_bounds__(64) void flip_update_tail(const float *__restrict__ prev,
                                                       const float *__restrict__ curr, int64_t start,
                                                       int64_t n, int16_t step,
                                                       int16_t *__restrict__ fc,
                                                       int16_t *__restrict__ lf) {
    const int64_t i = start + threadIdx.x;
    if (i >= n) return;
    int16_t f = fc[i], l = lf[i];
    update1(prev[i], curr[i], step, f, l);
    fc[i] = f;
    lf[i] = l;
}

// Read-out ("Which 1-Bit Weights Can You Trust?", Methodology): sign age
// (T - last_flip) / T and flip rate flip_count / T, each an fp64 quotient
// rounded once to fp32.  4 weights per thread.
__global__ __launch_bounds__(256) void flip_stats_kernel(const int16_t *__restrict__ fc,
                                                         const int16_t *__restrict__ lf, int64_t n,
                                                         int32_t T, float *__restrict__ age,
                                                         float *__restrict__ rate) {
    const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    const double t = (double)T;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t i = i0 + j;
        if (i < n) {
            age[i] = (float)((t - (double)lf[i]) / t);
            rate[i] = (float)((double)fc[i] / t);
        }
    }
}

}  // namespace

hipError_t launch_flip_stats(const int16_t *fc, const int16_t *lf, int64_t n, int32_t T, float *age,
                             float *rate, hipStream_t s) {
    const int64_t threads = (n + 3) / 4;
    hipLaunchKernelGGL(flip_stats_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, fc, lf, n, T,
                       age, rate);
    return hipGetLastError();
}

hipError_t launch_flip(const float *prev, const float *curr, int64_t n, int32_t step, int16_t *fc,
                       int16_t *lf, hipStream_t s) {
    const int64_t n4 = n / 4;
    if (n4 > 0)
        hipLaunchKernelGGL(flip_update_vec, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                           prev, curr, n4, (int16_t)step, fc, lf);
    if (n4 * 4 < n)
        hipLaunchKernelGGL(flip_update_tail, dim3(1), dim3(64), 0, s, prev, curr, n4 * 4, n,
                           (int16_t)step, fc, lf);
    return hipGetLastError();
}

}  // namespace bl
