// Sign-flip tracker update ("Which 1-Bit Weights Can You Trust?",
// Methodology): compare the sign of every latent weight with its sign at the
// previous step; where it changed, bump the INT16 flip count (saturating at
// 32767) and record the step in the INT16 last-flip counter.
//
// Elementwise and HBM-bound: 8 weights per thread, 16-byte loads of both
// snapshots and both counter arrays, 16-byte stores of the counters
// (16 B moved per weight).
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
                                                       const float *__restrict__ curr, int64_t n8,
                                                       int16_t step, int16_t *__restrict__ fc,
                                                       int16_t *__restrict__ lf) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const float4 *p4 = reinterpret_cast<const float4 *>(prev) + 2 * i;
    const float4 *c4 = reinterpret_cast<const float4 *>(curr) + 2 * i;
    const float4 pa = p4[0], pb = p4[1], ca = c4[0], cb = c4[1];
    union U {
        uint4 v;
        int16_t h[8];
    } f, l;
    f.v = reinterpret_cast<const uint4 *>(fc)[i];
    l.v = reinterpret_cast<const uint4 *>(lf)[i];
    const float pv[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
    const float cv[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
#pragma unroll
    for (int t = 0; t < 8; ++t) update1(pv[t], cv[t], step, f.h[t], l.h[t]);
    reinterpret_cast<uint4 *>(fc)[i] = f.v;
    reinterpret_cast<uint4 *>(lf)[i] = l.v;
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

}  // namespace

hipError_t launch_flip(const float *prev, const float *curr, int64_t n, int32_t step, int16_t *fc,
                       int16_t *lf, hipStream_t s) {
    const int64_t n8 = n / 8;
    if (n8 > 0)
        hipLaunchKernelGGL(flip_update_vec, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                           prev, curr, n8, (int16_t)step, fc, lf);
    if (n8 * 8 < n)
        hipLaunchKernelGGL(flip_update_tail, dim3(1), dim3(64), 0, s, prev, curr, n8 * 8, n,
                           (int16_t)step, fc, lf);
    return hipGetLastError();
}

}  // namespace bl
