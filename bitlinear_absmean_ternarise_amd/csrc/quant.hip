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

// W waves per row (K % 8 == 0, K <= 64 * W * 8 * kIters): each lane holds
// kIters 16-byte chunks, the wave maxima meet in LDS.  Several waves per row
// keep a 2048-token prefill at 8 waves per SIMD instead of 2 (the kernel is
// latency-bound: each wave issues its loads once, then waits).
template <int W, int kIters>
__global__ __launch_bounds__(W * 64) void quant_rows_block(const uint16_t *__restrict__ x,
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
        const int64_t idx = threadIdx.x + W * 64 * i;
        if (idx < nvec) {
            v[i] = __builtin_nontemporal_load(row + idx);  // read once
#pragma unroll
            for (int j = 0; j < 4; ++j) am.add(v[i][j]);
        }
    }
    float a = wave_max_nonneg(am.value());
    __shared__ float red[W];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    a = red[0];
#pragma unroll
    for (int i = 1; i < W; ++i) a = fmaxf(a, red[i]);
    const float s = 127.0f / fmaxf(a, eps);
    if (threadIdx.x == 0) xs[m] = s;
    uint2 *out = reinterpret_cast<uint2 *>(xq + m * K);
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        const int64_t idx = threadIdx.x + W * 64 * i;
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

// ---------------------------------------------------------------------------
// RMSNorm fused into the activation quant ("1-bit & Ternary LLMs (BitNet
// b1.58)", How it works: the forward quantises the normalised input; b1.58
// takes the LLaMA-style RMSNorm): y = x * r * g, r = 1/sqrt(mean x^2 + eps_n).
//
// r is a positive factor per token and the absmax quant does not see such a
// factor: clip(rint(y * 127/max|y|)) = clip(rint(u * 127/max|u|)) for u = x*g.
// So the codes are decided from u exactly as the plain quant decides them
// (fp32, no reduction order involved; with no gain, u = x and the codes are
// the plain quant's bit for bit), and r, from a sum of squares in fp64, only
// enters the scale: s = 127 / max(max|u| * r, eps) for the epilogue.  When
// the eps floor binds (max|y| < eps) the codes use s_u = s * r instead of
// 127 / max|u|.  One pass over x: 2 B read + 1 B written per element.
// eight gain values (16-byte aligned: 8 * idx floats from an aligned base)
__device__ __forceinline__ void load_gain8(const float *g, float (&out)[8]) {
    const float4 a = reinterpret_cast<const float4 *>(g)[0], b = reinterpret_cast<const float4 *>(g)[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

struct NormRow {
    double ss = 0.0;  // sum of x^2 (each square exact; fp64 sum)
    float a = 0.0f;   // max |u|
};

template <bool kGain>
__device__ __forceinline__ void norm_accum(NormRow &nr, const v4u &v, const float *g) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float x0 = __uint_as_float(v[j] << 16), x1 = __uint_as_float(v[j] & 0xFFFF0000u);
        nr.ss += (double)x0 * (double)x0;
        nr.ss += (double)x1 * (double)x1;
        const float u0 = kGain ? x0 * g[2 * j] : x0, u1 = kGain ? x1 * g[2 * j + 1] : x1;
        nr.a = fmaxf(nr.a, fmaxf(fabsf(u0), fabsf(u1)));
    }
}

// v + (v moved by a DPP pattern), each half of the double moved alike;
// lanes with no source (or masked rows) add 0
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_add_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROW_MASK, 0xf, false);
    return v + __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the wave, uniform: an inclusive scan within each 16-lane row
// (row_shr 1, 2, 4, 8), then the row totals carried by row broadcasts; lane
// 63 ends with the total.  No LDS crossbar (a shuffle tree of doubles takes
// 12 of them).
__device__ __forceinline__ double wave_sum_f64(double v) {
    v = dpp_add_f64<0x111, 0xf>(v);  // row_shr:1
    v = dpp_add_f64<0x112, 0xf>(v);  // row_shr:2
    v = dpp_add_f64<0x114, 0xf>(v);  // row_shr:4
    v = dpp_add_f64<0x118, 0xf>(v);  // row_shr:8
    v = dpp_add_f64<0x142, 0xa>(v);  // row_bcast:15
    v = dpp_add_f64<0x143, 0xc>(v);  // row_bcast:31
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// codes of 8 inputs (one 16-byte vector) from u = x * g and s_u
template <bool kGain>
__device__ __forceinline__ uint2 norm_codes(const v4u &v, const float *g, float su) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (kGain) {
            const float u0 = __uint_as_float(v[j] << 16) * g[2 * j];
            const float u1 = __uint_as_float(v[j] & 0xFFFF0000u) * g[2 * j + 1];
            w[j] = (qbits(u0, su) & 0xFFu) | ((qbits(u1, su) & 0xFFu) << 8);
        } else {
            w[j] = (qbits(__uint_as_float(v[j] << 16), su) & 0xFFu) |
                   ((qbits(__uint_as_float(v[j] & 0xFFFF0000u), su) & 0xFFu) << 8);
        }
    }
    return make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
}

// per-token scales from the reduced row: (s for the epilogue, s_u for the codes)
__device__ __forceinline__ void norm_scales(double ss, float a, int64_t K, float eps_n, float eps, float &s_out,
                                            float &su) {
    const double den = ss / (double)K + (double)eps_n;
    const double r = den > 0.0 ? 1.0 / sqrt(den) : 0.0;
    const double ay = (double)a * r;
    const double sy = 127.0 / (ay > (double)eps ? ay : (double)eps);
    s_out = (float)sy;
    su = ay > (double)eps ? 127.0f / a : (float)(sy * r);
}

// One wave per row (K % 8 == 0, K <= 64 * 8 * kIters).
template <int kIters, bool kGain>
__global__ __launch_bounds__(256) void norm_quant_rows_wave(const uint16_t *__restrict__ x,
                                                           const float *__restrict__ gain, int64_t M,
                                                           int64_t K, float eps_n, float eps,
                                                           int8_t *__restrict__ xq, float *__restrict__ xs) {
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    const v4u *row = reinterpret_cast<const v4u *>(x + m * K);
    const int64_t nvec = K / 8;
    v4u v[kIters];
    float gv[kIters][kGain ? 8 : 1];  // the gain is read once, with the row
    NormRow nr;
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        const int64_t idx = lane + 64 * i;
        if (idx < nvec) {
            v[i] = __builtin_nontemporal_load(row + idx);
            if constexpr (kGain) load_gain8(gain + 8 * idx, gv[i]);
            norm_accum<kGain>(nr, v[i], gv[i]);
        }
    }
    const double ss = wave_sum_f64(nr.ss);
    const float a = wave_max_nonneg(nr.a);
    float s, su;
    norm_scales(ss, a, K, eps_n, eps, s, su);
    if (lane == 0) xs[m] = s;
    uint2 *out = reinterpret_cast<uint2 *>(xq + m * K);
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        const int64_t idx = lane + 64 * i;
        if (idx < nvec) out[idx] = norm_codes<kGain>(v[i], gv[i], su);
    }
}

// One block of W waves per row (K % 8 == 0, K <= W * 64 * 8 * kIters).
template <int W, int kIters, bool kGain>
__global__ __launch_bounds__(W * 64) void norm_quant_rows_block(const uint16_t *__restrict__ x,
                                                               const float *__restrict__ gain, int64_t K,
                                                               float eps_n, float eps, int8_t *__restrict__ xq,
                                                               float *__restrict__ xs) {
    const int64_t m = blockIdx.x;
    const v4u *row = reinterpret_cast<const v4u *>(x + m * K);
    const int64_t nvec = K / 8;
    v4u v[kIters];
    float gv[kIters][kGain ? 8 : 1];  // the gain is read once, with the row
    NormRow nr;
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        const int64_t idx = threadIdx.x + W * 64 * i;
        if (idx < nvec) {
            v[i] = __builtin_nontemporal_load(row + idx);
            if constexpr (kGain) load_gain8(gain + 8 * idx, gv[i]);
            norm_accum<kGain>(nr, v[i], gv[i]);
        }
    }
    __shared__ double red_ss[W];
    __shared__ float red_a[W];
    const double ssw = wave_sum_f64(nr.ss);
    const float aw = wave_max_nonneg(nr.a);
    if ((threadIdx.x & 63) == 0) {
        red_ss[threadIdx.x >> 6] = ssw;
        red_a[threadIdx.x >> 6] = aw;
    }
    __shared__ float su_shared;
    __syncthreads();
    // One wave forms the scales: their fp64 division and square root cost a
    // wave's worth of slow instructions whatever the lane count, so all W
    // waves forming them (the same values) cost W times that (measured:
    // 2048 x 1536 with gain 5.4 -> 4.7 us, 2048 x 4096 8.4 -> 7.8 us).
    if (threadIdx.x < 64) {
        double ss = 0.0;
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < W; ++i) {  // fixed order
            ss += red_ss[i];
            a = fmaxf(a, red_a[i]);
        }
        float s, su0;
        norm_scales(ss, a, K, eps_n, eps, s, su0);
        if (threadIdx.x == 0) {
            xs[m] = s;
            su_shared = su0;
        }
    }
    __syncthreads();
    const float su = su_shared;
    uint2 *out = reinterpret_cast<uint2 *>(xq + m * K);
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
        const int64_t idx = threadIdx.x + W * 64 * i;
        if (idx < nvec) out[idx] = norm_codes<kGain>(v[i], gv[i], su);
    }
}

// Any K: one block of 256 threads per row, two passes over the row.
__global__ __launch_bounds__(256) void norm_quant_rows_scalar(const uint16_t *__restrict__ x,
                                                             const float *__restrict__ gain, int64_t K,
                                                             float eps_n, float eps, int8_t *__restrict__ xq,
                                                             float *__restrict__ xs) {
    const int64_t m = blockIdx.x;
    const uint16_t *row = x + m * K;
    double ssl = 0.0;
    float al = 0.0f;
    for (int64_t k = threadIdx.x; k < K; k += 256) {
        const float xv = bf16_to_f32(row[k]);
        ssl += (double)xv * (double)xv;
        al = fmaxf(al, fabsf(gain ? xv * gain[k] : xv));
    }
    __shared__ double red_ss[4];
    __shared__ float red_a[4];
    const double ssw = wave_sum_f64(ssl);
    const float aw = wave_max_nonneg(al);
    if ((threadIdx.x & 63) == 0) {
        red_ss[threadIdx.x >> 6] = ssw;
        red_a[threadIdx.x >> 6] = aw;
    }
    __syncthreads();
    const double ss = ((red_ss[0] + red_ss[1]) + red_ss[2]) + red_ss[3];
    const float a = fmaxf(fmaxf(red_a[0], red_a[1]), fmaxf(red_a[2], red_a[3]));
    float s, su;
    norm_scales(ss, a, K, eps_n, eps, s, su);
    if (threadIdx.x == 0) xs[m] = s;
    for (int64_t k = threadIdx.x; k < K; k += 256) {
        const float xv = bf16_to_f32(row[k]);
        xq[m * K + k] = (int8_t)(qbits(gain ? xv * gain[k] : xv, su) & 0xFFu);
    }
}

}  // namespace

hipError_t launch_quant(const uint16_t *x, int64_t M, int64_t K, float eps, int8_t *xq, float *xs,
                        hipStream_t s) {
    // up to 512 columns: one wave per row, four rows per block; longer rows:
    // a block of W waves per row with at most two 16-byte chunks per lane
    // (four for rows past 16384 columns)
    const dim3 grid((unsigned)M);
    if (M <= 256 && K % 8 == 0 && K > 64 * 8 && K <= 1024 * 8) {
        // few rows (decode): one 16-byte chunk per lane and as many waves as
        // the row needs, so a row's loads are all in flight at once (K =
        // 8192: 1 row 2.72 -> 2.38 us, 16 rows 3.11 -> 2.72 us, 64 rows 3.26
        // -> 2.85 us; 3B decode step at 8 tokens 33.8 -> 32.4 us)
        const int64_t w = (K / 8 + 63) / 64;
        if (w <= 2) hipLaunchKernelGGL((quant_rows_block<2, 1>), grid, dim3(128), 0, s, x, K, eps, xq, xs);
        else if (w <= 4) hipLaunchKernelGGL((quant_rows_block<4, 1>), grid, dim3(256), 0, s, x, K, eps, xq, xs);
        else if (w <= 8) hipLaunchKernelGGL((quant_rows_block<8, 1>), grid, dim3(512), 0, s, x, K, eps, xq, xs);
        else hipLaunchKernelGGL((quant_rows_block<16, 1>), grid, dim3(1024), 0, s, x, K, eps, xq, xs);
        return hipGetLastError();
    }
    if (K % 8 == 0 && K <= 64 * 8) {
        hipLaunchKernelGGL(quant_rows_wave<1>, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, x, M, K, eps, xq, xs);
    } else if (K % 8 == 0 && K <= 256 * 8) {
        hipLaunchKernelGGL((quant_rows_block<4, 1>), grid, dim3(256), 0, s, x, K, eps, xq, xs);
    } else if (K % 8 == 0 && K <= 256 * 8 * 2) {
        hipLaunchKernelGGL((quant_rows_block<4, 2>), grid, dim3(256), 0, s, x, K, eps, xq, xs);
    } else if (K % 8 == 0 && K <= 512 * 8 * 2) {
        hipLaunchKernelGGL((quant_rows_block<8, 2>), grid, dim3(512), 0, s, x, K, eps, xq, xs);
    } else if (K % 8 == 0 && K <= 1024 * 8 * 2) {
        hipLaunchKernelGGL((quant_rows_block<16, 2>), grid, dim3(1024), 0, s, x, K, eps, xq, xs);
    } else if (K % 8 == 0 && K <= 1024 * 8 * 4) {
        hipLaunchKernelGGL((quant_rows_block<16, 4>), grid, dim3(1024), 0, s, x, K, eps, xq, xs);
    } else {
        hipLaunchKernelGGL(quant_rows_scalar, grid, dim3(256), 0, s, x, K, eps, xq, xs);
    }
    return hipGetLastError();
}

}  // namespace bl

namespace bl {

namespace {

template <int I, bool G>
void norm_wave(unsigned grid, const uint16_t *x, const float *gain, int64_t M, int64_t K, float eps_n, float eps,
               int8_t *xq, float *xs, hipStream_t s) {
    hipLaunchKernelGGL((norm_quant_rows_wave<I, G>), dim3(grid), dim3(256), 0, s, x, gain, M, K, eps_n, eps, xq, xs);
}

template <int W, int I, bool G>
void norm_block(const uint16_t *x, const float *gain, int64_t M, int64_t K, float eps_n, float eps, int8_t *xq,
                float *xs, hipStream_t s) {
    hipLaunchKernelGGL((norm_quant_rows_block<W, I, G>), dim3((unsigned)M), dim3(W * 64), 0, s, x, gain, K, eps_n,
                       eps, xq, xs);
}

template <bool G>
void launch_norm_g(const uint16_t *x, const float *gain, int64_t M, int64_t K, float eps_n, float eps, int8_t *xq,
                   float *xs, hipStream_t s) {
    // the shapes of the plain quant: up to 512 columns one wave per row (four
    // rows per block); longer rows a block of W waves per row with at most two
    // 16-byte chunks per lane (four past 16384 columns).  One wave per row for
    // rows up to 4096 columns left a 2048-row call at two waves per SIMD
    // (6.0 us at K = 1536, against 4.0 us for the plain quant).
    if (M <= 256 && K % 8 == 0 && K > 64 * 8 && K <= 1024 * 8) {
        // few rows (decode), as for the plain quant: one chunk per lane, as
        // many waves as the row needs (1 x 8192 3.18 -> 2.95 us, 8 x 3200
        // 3.33 -> 2.85 us)
        const int64_t w = (K / 8 + 63) / 64;
        if (w <= 2) norm_block<2, 1, G>(x, gain, M, K, eps_n, eps, xq, xs, s);
        else if (w <= 4) norm_block<4, 1, G>(x, gain, M, K, eps_n, eps, xq, xs, s);
        else if (w <= 8) norm_block<8, 1, G>(x, gain, M, K, eps_n, eps, xq, xs, s);
        else norm_block<16, 1, G>(x, gain, M, K, eps_n, eps, xq, xs, s);
        return;
    }
    if (K % 8 == 0 && K <= 64 * 8) {
        norm_wave<1, G>((unsigned)((M + 3) / 4), x, gain, M, K, eps_n, eps, xq, xs, s);
    } else if (K % 8 == 0 && K <= 1024 * 8 * 4) {
        if (K <= 256 * 8) norm_block<4, 1, G>(x, gain, M, K, eps_n, eps, xq, xs, s);
        else if (K <= 256 * 8 * 2) norm_block<4, 2, G>(x, gain, M, K, eps_n, eps, xq, xs, s);
        else if (K <= 512 * 8 * 2) norm_block<8, 2, G>(x, gain, M, K, eps_n, eps, xq, xs, s);
        else if (K <= 1024 * 8 * 2) norm_block<16, 2, G>(x, gain, M, K, eps_n, eps, xq, xs, s);
        else norm_block<16, 4, G>(x, gain, M, K, eps_n, eps, xq, xs, s);
    } else {
        hipLaunchKernelGGL(norm_quant_rows_scalar, dim3((unsigned)M), dim3(256), 0, s, x, gain, K, eps_n, eps, xq,
                           xs);
    }
}

}  // namespace

hipError_t launch_norm_quant(const uint16_t *x, const float *gain, int64_t M, int64_t K, float eps_n, float eps,
                             int8_t *xq, float *xs, hipStream_t s) {
    if (gain)
        launch_norm_g<true>(x, gain, M, K, eps_n, eps, xq, xs, s);
    else
        launch_norm_g<false>(x, gain, M, K, eps_n, eps, xq, xs, s);
    return hipGetLastError();
}

}  // namespace bl
