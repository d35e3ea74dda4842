// Weight ternarisation and packing.
//
// gamma = mean |W| ("1-bit & Ternary LLMs (BitNet b1.58)", BitNet b1.58
// equations; "What 1.58 Bits Actually Changes", Three values), summed in fp64
// in an order fixed by the shape alone (per-block partials over contiguous
// chunks, then one block summing the partials), rounded once to fp32.
// codes = clip(rint(W / fp32(gamma + eps)), -1, 1), one correctly rounded
// fp32 division per weight, written straight into packed layout v1.
//
// All three kernels stream W from HBM: 4 B read per weight for gamma, 4 B
// read + 0.25 B written per weight for the codes.
#include "device.h"
#include "internal.h"

namespace bl {

namespace {

constexpr int kSumThreads = 256;
constexpr int64_t kMaxPartials = 2048;
constexpr int64_t kMinPerPartial = 16384;

// Each block sums |W| (kAbs) or W over one contiguous chunk in fp64.
// Thread t adds elements start + 4t + 1024 i (float4 when aligned) in
// increasing i; the block then folds its 256 thread sums in a fixed tree.
template <bool kAbs>
__device__ __forceinline__ double term(float w) { return kAbs ? fabs((double)w) : (double)w; }

template <bool kAbs>
__device__ __forceinline__ void sum_chunk(const float *__restrict__ W, int64_t count, int64_t chunk, int64_t blk,
                                          double *__restrict__ partials) {
    const int64_t start = blk * chunk;
    int64_t end = start + chunk;
    if (end > count) end = count;
    double s = 0.0;
    // chunk is a multiple of 4 and W is 16-byte aligned, so start is too.
    const int64_t nvec = (end - start) / 4;
    const float4 *W4 = reinterpret_cast<const float4 *>(W + start);
    for (int64_t i = threadIdx.x; i < nvec; i += kSumThreads) {
        float4 v = W4[i];
        s += term<kAbs>(v.x);
        s += term<kAbs>(v.y);
        s += term<kAbs>(v.z);
        s += term<kAbs>(v.w);
    }
    for (int64_t i = start + nvec * 4 + threadIdx.x; i < end; i += kSumThreads) s += term<kAbs>(W[i]);

    __shared__ double red[kSumThreads];
    red[threadIdx.x] = s;
    __syncthreads();
#pragma unroll
    for (int w = kSumThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) partials[blk] = red[0];
}

template <bool kAbs>
__global__ __launch_bounds__(kSumThreads) void abs_sum_partial(const float *__restrict__ W,
                                                               int64_t count, int64_t chunk,
                                                               double *__restrict__ partials) {
    sum_chunk<kAbs>(W, count, chunk, blockIdx.x, partials);
}

__device__ __forceinline__ void mean_of_partials(const double *__restrict__ partials, int64_t np, double count,
                                                 float *__restrict__ gamma) {
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < np; i += kSumThreads) s += partials[i];
    __shared__ double red[kSumThreads];
    red[threadIdx.x] = s;
    __syncthreads();
#pragma unroll
    for (int w = kSumThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) gamma[0] = (float)(red[0] / count);
}

__global__ __launch_bounds__(kSumThreads) void gamma_final(const double *__restrict__ partials,
                                                           int64_t np, double count,
                                                           float *__restrict__ gamma) {
    mean_of_partials(partials, np, count, gamma);
}

__device__ __forceinline__ uint32_t code_bits(float w, float d) {
    // correctly rounded fp32 division, then round half to even
    const float r = rintf(w / d);
    return r > 0.0f ? 1u : (r < 0.0f ? 3u : 0u);
}

// Binary BitNet rule: +1 (01) where W >= alpha, -1 (11) elsewhere.
__device__ __forceinline__ uint32_t binary_bits(float w, float alpha) { return w >= alpha ? 1u : 3u; }

// One thread per packed dword.  The thread's position in the packed buffer
// fixes (row block, group, lane, fragment) and so the 16 weights it reads.
// kBinary: scale[0] is alpha and the binary rule applies; otherwise scale[0]
// is gamma and the ternary rule with divisor gamma + eps.  Padding positions
// keep the zero code either way.
template <bool kAligned, bool kBinary>
__device__ __forceinline__ void pack_dword(const float *__restrict__ W, int64_t N, int64_t K, int64_t KF, int64_t D,
                                           float eps, const float *__restrict__ scale,
                                           uint32_t *__restrict__ packed) {
    const int64_t per_block = KF * 64;
    const int64_t nb = D / per_block;
    const int64_t rem = D - nb * per_block;
    const int64_t g = rem >> 8;
    const int pos = (int)(rem & 255);
    int64_t G = KF - 4 * g;
    if (G > 4) G = 4;
    const int lam = (int)(pos / G);
    const int f = (int)(pos - lam * G);
    const int64_t n = nb * 16 + (lam & 15);
    const int64_t k0 = (4 * g + f) * 64 + 16 * (lam >> 4);

    const float sc = scale[0];
    const float d = kBinary ? sc : sc + eps;  // alpha, or the ternary divisor
    auto bits = [&](float w) { return kBinary ? binary_bits(w, d) : code_bits(w, d); };
    uint32_t word = 0;
    if (n < N && (kBinary || d != 0.0f)) {
        const float *row = W + n * K;
        if (kAligned && k0 + 16 <= K) {
            const float4 *p = reinterpret_cast<const float4 *>(row + k0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = p[q];
                const int t = 4 * q;  // columns t..t+3 of this dword
                word |= bits(v.x) << (8 * ((t + 0) & 3) + 2 * ((t + 0) >> 2));
                word |= bits(v.y) << (8 * ((t + 1) & 3) + 2 * ((t + 1) >> 2));
                word |= bits(v.z) << (8 * ((t + 2) & 3) + 2 * ((t + 2) >> 2));
                word |= bits(v.w) << (8 * ((t + 3) & 3) + 2 * ((t + 3) >> 2));
            }
        } else {
            for (int t = 0; t < 16; ++t) {
                const int64_t k = k0 + t;
                if (k < K) word |= bits(row[k]) << (8 * (t & 3) + 2 * (t >> 2));
            }
        }
    }
    packed[D] = word;
}

// One thread per packed dword.  The thread's position in the packed buffer
// fixes (row block, group, lane, fragment) and so the 16 weights it reads.
// kBinary: scale[0] is alpha and the binary rule applies; otherwise scale[0]
// is gamma and the ternary rule with divisor gamma + eps.  Padding positions
// keep the zero code either way.
template <bool kAligned, bool kBinary>
__global__ __launch_bounds__(256) void ternarise_pack(const float *__restrict__ W, int64_t N,
                                                      int64_t K, int64_t KF, int64_t total_dwords,
                                                      float eps, const float *__restrict__ scale,
                                                      uint32_t *__restrict__ packed) {
    const int64_t D = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (D >= total_dwords) return;
    pack_dword<kAligned, kBinary>(W, N, K, KF, D, eps, scale, packed);
}

// Layout b1 (one bit per binary code, bit 1 = -1): one thread per packed
// dword, which holds row n of pair P of its group: columns 128P + 64h +
// 16*(lam/16) + t of half h = 0, 1, code t at bit 8*(t%4) + 7 - (4h + t/4).
// K % 64 == 0, so a half is either whole or padding (bits 0).
__global__ __launch_bounds__(256) void binary_pack_b1(const float *__restrict__ W, int64_t N, int64_t K, int64_t KP,
                                                      int64_t total_dwords, const float *__restrict__ alpha,
                                                      uint32_t *__restrict__ packed) {
    const int64_t D = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (D >= total_dwords) return;
    const int64_t per_block = KP * 64;
    const int64_t nb = D / per_block;
    const int64_t rem = D - nb * per_block;
    const int64_t g = rem >> 8;
    const int pos = (int)(rem & 255);
    int64_t G = KP - 4 * g;
    if (G > 4) G = 4;
    const int lam = (int)(pos / G);
    const int f = (int)(pos - lam * G);
    const int64_t n = nb * 16 + (lam & 15);
    const float a = alpha[0];
    uint32_t word = 0;
    if (n < N) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t k0 = (4 * g + f) * 128 + 64 * h + 16 * (lam >> 4);
            if (k0 >= K) continue;
            const float4 *p = reinterpret_cast<const float4 *>(W + n * K + k0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = p[q];
                const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 4 * q + i;
                    if (!(e[i] >= a)) word |= 1u << (8 * (t & 3) + 7 - (4 * h + (t >> 2)));
                }
            }
        }
    }
    packed[D] = word;
}

// ---- several tensors per launch: the same three phases, each workgroup
// finding its tensor in the segment table (a tensor's partial sums, and so
// its gamma, are those of a call of its own)
__device__ __forceinline__ int find_seg(const PackSegs &ps, int64_t w, int which) {
    int sidx = 0;
#pragma unroll
    for (int i = 1; i < kPackGroup; ++i) {
        const int64_t b = which == 0 ? ps.s[i].wg_begin : ps.s[i].dw_begin;
        if (i < ps.count && w >= b) sidx = i;
    }
    return sidx;
}

__global__ __launch_bounds__(kSumThreads) void abs_sum_partial_grouped(PackSegs ps) {
    const int sidx = find_seg(ps, blockIdx.x, 0);
    const PackSeg &sg = ps.s[sidx];
    sum_chunk<true>(sg.W, sg.count, sg.chunk, (int64_t)blockIdx.x - sg.wg_begin, sg.partials);
}

__global__ __launch_bounds__(kSumThreads) void gamma_final_grouped(PackSegs ps) {
    const PackSeg &sg = ps.s[blockIdx.x];
    mean_of_partials(sg.partials, sg.nblocks, (double)sg.count, sg.gamma);
}

__global__ __launch_bounds__(256) void ternarise_pack_grouped(PackSegs ps, int64_t total_dwords) {
    const int64_t D = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (D >= total_dwords) return;
    // a block may straddle two tensors: find this thread's
    int sidx = 0;
#pragma unroll
    for (int i = 1; i < kPackGroup; ++i)
        if (i < ps.count && D >= ps.s[i].dw_begin) sidx = i;
    const PackSeg &sg = ps.s[sidx];
    const int64_t d = D - sg.dw_begin;
    if (sg.aligned)
        pack_dword<true, false>(sg.W, sg.N, sg.K, sg.KF, d, sg.eps, sg.gamma, sg.packed);
    else
        pack_dword<false, false>(sg.W, sg.N, sg.K, sg.KF, d, sg.eps, sg.gamma, sg.packed);
}

}  // namespace

int64_t pack_partials(int64_t count) {
    int64_t np = (count + kMinPerPartial - 1) / kMinPerPartial;
    if (np > kMaxPartials) np = kMaxPartials;
    if (np < 1) np = 1;
    return np;
}

namespace {

// fp64 partial sums of |W| (kAbs) or W, then their mean rounded to fp32 into *out
template <bool kAbs>
void launch_mean(const float *W, int64_t count, double *partials, float *out, hipStream_t s) {
    const int64_t np = pack_partials(count);
    int64_t chunk = (count + np - 1) / np;
    chunk = (chunk + 3) & ~int64_t(3);
    const int64_t nblocks = (count + chunk - 1) / chunk;  // <= np
    hipLaunchKernelGGL(abs_sum_partial<kAbs>, dim3((unsigned)nblocks), dim3(kSumThreads), 0, s, W, count, chunk,
                       partials);
    hipLaunchKernelGGL(gamma_final, dim3(1), dim3(kSumThreads), 0, s, partials, nblocks, (double)count, out);
}

template <bool kBinary>
void launch_codes(const float *W, const Layout &L, float eps, const float *scale, uint32_t *packed, hipStream_t s) {
    const int64_t total = L.bytes / 4;
    const unsigned grid = (unsigned)((total + 255) / 256);
    if (L.K % 4 == 0)
        hipLaunchKernelGGL((ternarise_pack<true, kBinary>), dim3(grid), dim3(256), 0, s, W, L.N, L.K, L.KF, total,
                           eps, scale, packed);
    else
        hipLaunchKernelGGL((ternarise_pack<false, kBinary>), dim3(grid), dim3(256), 0, s, W, L.N, L.K, L.KF, total,
                           eps, scale, packed);
}

}  // namespace

hipError_t launch_pack(const float *W, const Layout &L, float eps, double *partials,
                       uint32_t *packed, float *gamma, hipStream_t s) {
    launch_mean<true>(W, L.N * L.K, partials, gamma, s);
    launch_codes<false>(W, L, eps, gamma, packed, s);
    return hipGetLastError();
}

hipError_t launch_pack_grouped(PackSegs &ps, hipStream_t s) {
    int64_t wg = 0, dw = 0;
    for (int i = 0; i < ps.count; ++i) {
        PackSeg &g = ps.s[i];
        const int64_t np = pack_partials(g.count);
        int64_t chunk = (g.count + np - 1) / np;
        chunk = (chunk + 3) & ~int64_t(3);
        g.chunk = chunk;
        g.nblocks = (g.count + chunk - 1) / chunk;
        g.wg_begin = wg;
        wg += g.nblocks;
        g.dw_begin = dw;
        dw += g.dwords;
    }
    hipLaunchKernelGGL(abs_sum_partial_grouped, dim3((unsigned)wg), dim3(kSumThreads), 0, s, ps);
    hipLaunchKernelGGL(gamma_final_grouped, dim3((unsigned)ps.count), dim3(kSumThreads), 0, s, ps);
    hipLaunchKernelGGL(ternarise_pack_grouped, dim3((unsigned)((dw + 255) / 256)), dim3(256), 0, s, ps, dw);
    return hipGetLastError();
}

hipError_t launch_pack_binary(const float *W, const Layout &L, double *partials, uint32_t *packed, float *beta,
                              float *alpha, hipStream_t s) {
    launch_mean<true>(W, L.N * L.K, partials, beta, s);
    launch_mean<false>(W, L.N * L.K, partials, alpha, s);  // same partials buffer, stream-ordered
    launch_codes<true>(W, L, 0.0f, alpha, packed, s);
    return hipGetLastError();
}

hipError_t launch_pack_binary_b1(const float *W, int64_t N, int64_t K, double *partials, uint32_t *packed,
                                 float *beta, float *alpha, hipStream_t s) {
    launch_mean<true>(W, N * K, partials, beta, s);
    launch_mean<false>(W, N * K, partials, alpha, s);
    const int64_t KP = (K + 127) / 128;
    const int64_t total = b1_bytes(N, K) / 4;
    hipLaunchKernelGGL(binary_pack_b1, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, W, N, K, KP, total,
                       alpha, packed);
    return hipGetLastError();
}

}  // namespace bl
