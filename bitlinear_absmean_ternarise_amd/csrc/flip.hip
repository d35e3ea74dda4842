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
#include <cmath>

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
// rounded once to fp32.  The kernel divides in fp32, which gives the same
// bits: the numerators (|T - last_flip| < 2^17, |flip_count| <= 2^15) and T
// (1..32767, checked by the entry point) are exact in fp32, fp32 division is
// correctly rounded, and for fp32 operands the fp64 quotient rounded to fp32
// is the correctly rounded fp32 quotient (double rounding is innocuous for
// division when the wider format has at least 2p + 2 bits, 53 >= 2 * 24 + 2:
// S. A. Figueroa, "When is double rounding innocuous?", 1995).  The fp64
// divisions cost more than the memory traffic.  4 weights per thread: 8-byte
// loads and 16-byte stores (the entry point requires 16-byte aligned arrays).
__global__ __launch_bounds__(256) void flip_stats_kernel(const int16_t *__restrict__ fc,
                                                         const int16_t *__restrict__ lf, int64_t n,
                                                         int32_t T, float *__restrict__ age,
                                                         float *__restrict__ rate) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef float v4f __attribute__((ext_vector_type(4)));
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t i0 = q * 4;
    if (i0 >= n) return;
    const float t = (float)T;
    if (i0 + 4 <= n) {
        const v4s f = __builtin_nontemporal_load(reinterpret_cast<const v4s *>(fc) + q);
        const v4s l = __builtin_nontemporal_load(reinterpret_cast<const v4s *>(lf) + q);
        v4f a, r;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[j] = (float)(T - (int32_t)l[j]) / t;
            r[j] = (float)f[j] / t;
        }
        __builtin_nontemporal_store(a, reinterpret_cast<v4f *>(age) + q);
        __builtin_nontemporal_store(r, reinterpret_cast<v4f *>(rate) + q);
    } else {
        for (int64_t i = i0; i < n; ++i) {
            age[i] = (float)(T - (int32_t)lf[i]) / t;
            rate[i] = (float)fc[i] / t;
        }
    }
}

// AdamW step on the shadow weights with the tracker fused ("1-bit & Ternary
// LLMs (BitNet b1.58)", Training: the optimiser steps the full-precision
// weights; "Which 1-Bit Weights Can You Trust?", Methodology: compare each
// weight's sign before and after the step).  The published AdamW update
// (decoupled weight decay), per weight in fp32 with the scalar coefficients
// prepared on the host:
//   w = W * decay;  m = b1*m + a1*g;  v = b2*v + a2*(g*g)
//   W = w - step * (m / (sqrt(v) / rc2 + eps))
// The old weight is still in a register when the new one is known, so the
// tracker needs no snapshot: 16 B read + 12 B written per weight, plus the
// counters where a sign changed.  4 weights per thread.
struct AdamCoef {
    float decay, b1, b2, a1, a2, step, rc2, eps;
};

template <bool kTrack>
__global__ __launch_bounds__(256) void adamw_flip_kernel(float *__restrict__ W, const float *__restrict__ g,
                                                         float *__restrict__ m, float *__restrict__ v, int64_t n4,
                                                         AdamCoef c, int16_t t, int16_t *__restrict__ fc,
                                                         int16_t *__restrict__ lf) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    typedef float v4f __attribute__((ext_vector_type(4)));
    typedef short v4s __attribute__((ext_vector_type(4)));
    // every stream is touched once: non-temporal loads and stores (measured on
    // a 235M-weight matrix: 75% of HBM peak, as fast as the same traffic with
    // no arithmetic; 67% with cached loads and stores)
    const v4f w0 = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(W) + i);
    const v4f gg = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(g) + i);
    v4f mm = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(m) + i);
    v4f vv = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(v) + i);
    v4f w1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float w = w0[j] * c.decay;
        const float mi = c.b1 * mm[j] + c.a1 * gg[j];
        const float vi = c.b2 * vv[j] + c.a2 * (gg[j] * gg[j]);
        const float den = sqrtf(vi) / c.rc2 + c.eps;
        w1[j] = w - c.step * (mi / den);
        mm[j] = mi;
        vv[j] = vi;
    }
    __builtin_nontemporal_store(w1, reinterpret_cast<v4f *>(W) + i);
    __builtin_nontemporal_store(mm, reinterpret_cast<v4f *>(m) + i);
    __builtin_nontemporal_store(vv, reinterpret_cast<v4f *>(v) + i);
    if (kTrack) {
        bool any = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) any |= sgn(w0[j]) != sgn(w1[j]);
        if (any) {
            v4s f = reinterpret_cast<const v4s *>(fc)[i];
            v4s l = reinterpret_cast<const v4s *>(lf)[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (sgn(w0[j]) != sgn(w1[j])) {
                    f[j] = (short)(f[j] == 32767 ? 32767 : f[j] + 1);
                    l[j] = t;
                }
            }
            reinterpret_cast<v4s *>(fc)[i] = f;
            reinterpret_cast<v4s *>(lf)[i] = l;
        }
    }
}

// the n % 4 weights at the end, one per thread
template <bool kTrack>
__global__ __launch_bounds__(64) void adamw_flip_tail(float *__restrict__ W, const float *__restrict__ g,
                                                      float *__restrict__ m, float *__restrict__ v, int64_t start,
                                                      int64_t n, AdamCoef c, int16_t t, int16_t *__restrict__ fc,
                                                      int16_t *__restrict__ lf) {
    const int64_t i = start + threadIdx.x;
    if (i >= n) return;
    const float w0 = W[i];
    const float w = w0 * c.decay;
    const float mi = c.b1 * m[i] + c.a1 * g[i];
    const float vi = c.b2 * v[i] + c.a2 * (g[i] * g[i]);
    const float den = sqrtf(vi) / c.rc2 + c.eps;
    const float w1 = w - c.step * (mi / den);
    W[i] = w1;
    m[i] = mi;
    v[i] = vi;
    if (kTrack && sgn(w0) != sgn(w1)) {
        fc[i] = (int16_t)(fc[i] == 32767 ? 32767 : fc[i] + 1);
        lf[i] = t;
    }
}

}  // namespace

hipError_t launch_adamw_flip(float *W, const float *g, float *m, float *v, int64_t n, int32_t t, double lr,
                             double b1, double b2, double eps, double wd, int16_t *fc, int16_t *lf, hipStream_t s) {
    // scalar coefficients in fp64, each rounded once to fp32
    AdamCoef c;
    c.decay = (float)(1.0 - lr * wd);
    c.b1 = (float)b1;
    c.b2 = (float)b2;
    c.a1 = (float)(1.0 - b1);
    c.a2 = (float)(1.0 - b2);
    c.step = (float)(lr / (1.0 - std::pow(b1, (double)t)));
    c.rc2 = (float)std::sqrt(1.0 - std::pow(b2, (double)t));
    c.eps = (float)eps;
    const bool track = fc != nullptr;
    const int64_t n4 = n / 4;
    const int16_t ts = (int16_t)(t > 32767 ? 32767 : t);
    if (n4 > 0) {
        const dim3 grid((unsigned)((n4 + 255) / 256));
        if (track)
            hipLaunchKernelGGL(adamw_flip_kernel<true>, grid, dim3(256), 0, s, W, g, m, v, n4, c, ts, fc, lf);
        else
            hipLaunchKernelGGL(adamw_flip_kernel<false>, grid, dim3(256), 0, s, W, g, m, v, n4, c, ts, fc, lf);
    }
    if (n4 * 4 < n) {
        if (track)
            hipLaunchKernelGGL(adamw_flip_tail<true>, dim3(1), dim3(64), 0, s, W, g, m, v, n4 * 4, n, c, ts, fc, lf);
        else
            hipLaunchKernelGGL(adamw_flip_tail<false>, dim3(1), dim3(64), 0, s, W, g, m, v, n4 * 4, n, c, ts, fc, lf);
    }
    return hipGetLastError();
}

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
