// BitLinear forward: y[m][n] = bf16( acc[m][n] * gamma / s_m ),
// acc[m][n] = sum_k xq[m][k] * code[n][k]   (exact int32)
//
// "1-bit & Ternary LLMs (BitNet b1.58)", BitLinear forward equation: the inner
// product of ternary weights and int8 activations is integer work and one
// float rescale per output is all that is left; "What one bit actually buys
// you": +1 adds the input, -1 subtracts it, 0 skips it.
//
// Two kernels:
//  * gemv_dot4  - M <= 2 tokens.  Streams the packed weights once from HBM;
//                 each lane unpacks its code dword to four int8 dwords and
//                 applies v_dot4_i32_i8 against the token's bytes (the
//                 add/subtract/skip rule as a 4-wide signed dot product).
//  * gemm_mfma  - M >= 3.  Activations staged in LDS, code dwords loaded
//                 straight from the packed layout into the A operand of
//                 v_mfma_i32_16x16x64_i8 (one dword per lane unpacks to the
//                 16 int8 values the lane contributes), int32 accumulation
//                 in the MFMA, dequant epilogue fused.
#include "device.h"
#include "internal.h"

namespace bl {

namespace {

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// 16 activation bytes starting at column k0 of row `row` (zero past K; never
// reads past the row).
template <bool kAlignedK>
__device__ __forceinline__ uint4 load_x16(const int8_t *__restrict__ row, int64_t k0, int64_t K) {
    if (kAlignedK) {
        // K % 16 == 0: a chunk is either wholly inside the row or wholly past it
        if (k0 < K) return *reinterpret_cast<const uint4 *>(row + k0);
        return make_uint4(0u, 0u, 0u, 0u);
    } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < 16; ++t)
            if (k0 + t < K) w[t >> 2] |= ((uint32_t)(uint8_t)row[k0 + t]) << (8 * (t & 3));
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
}

__device__ __forceinline__ void store_out(uint16_t *__restrict__ y, int32_t *__restrict__ acc_out,
                                          int64_t m, int64_t n, int64_t N, int a, float scale) {
    y[m * N + n] = f32_to_bf16((float)a * scale);
    if (acc_out) acc_out[m * N + n] = a;
}

// --------------------------------------------------------------- gemv_dot4
// One workgroup (4 waves) per 16-row block.  Wave w takes groups w, w+4, ...
// Lane l owns row l%16 of the block and the 16 columns 16*(l/16) of each
// fragment: exactly the dword the layout puts at lane l.
template <int MM, bool kAlignedK>
__global__ __launch_bounds__(256) void gemv_dot4(const uint32_t *__restrict__ packed,
                                                 const float *__restrict__ gamma, int64_t N,
                                                 int64_t K, int64_t KF, int64_t NG,
                                                 const int8_t *__restrict__ xq,
                                                 const float *__restrict__ xs,
                                                 uint16_t *__restrict__ y,
                                                 int32_t *__restrict__ acc_out) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t rb = blockIdx.x;
    const uint32_t *blk = packed + rb * KF * 64;
    const int64_t kl = 16 * (lane >> 4);

    int acc[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) acc[m] = 0;

    for (int64_t g = wave; g < NG; g += 4) {
        int64_t G = KF - 4 * g;
        uint32_t c[4] = {0u, 0u, 0u, 0u};
        if (G >= 4) {
            const uint4 v = *reinterpret_cast<const uint4 *>(blk + g * 256 + lane * 4);
            c[0] = v.x;
            c[1] = v.y;
            c[2] = v.z;
            c[3] = v.w;
            G = 4;
        } else {
            for (int f = 0; f < G; ++f) c[f] = blk[g * 256 + lane * G + f];
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            if (f < G) {
                const int64_t k0 = (4 * g + f) * 64 + kl;
                const uint32_t u0 = unpack4(c[f], 0), u1 = unpack4(c[f], 1);
                const uint32_t u2 = unpack4(c[f], 2), u3 = unpack4(c[f], 3);
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    const uint4 xv = load_x16<kAlignedK>(xq + m * K, k0, K);
                    int a = acc[m];
                    a = dot4(u0, xv.x, a);
                    a = dot4(u1, xv.y, a);
                    a = dot4(u2, xv.z, a);
                    a = dot4(u3, xv.w, a);
                    acc[m] = a;
                }
            }
        }
    }
    // fold the four 16-column slices of each row, then the four waves
    __shared__ int red[4][16][MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) {
        int a = acc[m];
        a += __shfl_xor(a, 16, 64);
        a += __shfl_xor(a, 32, 64);
        if (lane < 16) red[wave][lane][m] = a;
    }
    __syncthreads();
    if (wave == 0 && lane < 16) {
        const int64_t n = rb * 16 + lane;
        if (n < N) {
            const float gm = gamma[0];
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                const int a = red[0][lane][m] + red[1][lane][m] + red[2][lane][m] + red[3][lane][m];
                store_out(y, acc_out, m, n, N, a, gm / xs[m]);
            }
        }
    }
}

// ------------------------------------------------------------ gemv_dot4_nt
// The add / subtract / skip contraction on the vector ALUs for 1..4 tokens,
// with the memory structure of the MFMA decode kernel (gemv.hip): W waves per
// workgroup, RB 16-row blocks per workgroup, wave w takes the 1 KB groups
// w, w + W, ... (U per sweep) through non-temporal 16-byte buffer loads.
// Lane l owns row l % 16 of each row block and the 16 columns 16*(l/16) of
// every fragment: its code dword unpacks to four int8 dwords holding 64 * code
// (7 VALU) and v_dot4_i32_i8 applies them to the token's 16 bytes (16 bytes
// per lane per fragment per token, read from L2 through a descriptor whose
// range ends at M*K).  The four lanes of a row meet by cross-lane adds, the
// waves through LDS; the sums are 64 * acc exactly (K <= kScaledMaxK).
struct Dot4Seg {
    const uint32_t *packed;
    const float *gamma;
    const int8_t *xq;
    const float *xs;
    uint16_t *y;
    int32_t *acc;
    int64_t N, K, KF, NB, M;
    int64_t wg_begin;
};
struct Dot4Segs {
    Dot4Seg s[kMaxSeg];
    int count;
};

template <int W, int RB, int U, int MM>
__global__ __launch_bounds__(W * 64) void gemv_dot4_nt(Dot4Segs segs) {
    __shared__ int red[W][RB][16][MM];
    const int64_t wg = blockIdx.x;
    int sidx = 0;
#pragma unroll
    for (int i = 1; i < kMaxSeg; ++i)
        if (i < segs.count && wg >= segs.s[i].wg_begin) sidx = i;
    const Dot4Seg &sg = segs.s[sidx];
    const int64_t N = sg.N, K = sg.K, KF = sg.KF, NB = sg.NB, M = sg.M;
    const int64_t rb0 = (wg - sg.wg_begin) * RB;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t NGfull = KF / 4;
    const int Gtail = (int)(KF - 4 * NGfull);

    const uint32_t xrange = (uint32_t)(M * K);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void *)sg.xq, 0, (int)xrange, 0x00020000);
    uint32_t x_off[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) x_off[m] = m < M ? (uint32_t)(m * K + 16 * (lane >> 4)) : xrange;
    const uint32_t wrange = (uint32_t)(NB * KF * 256);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc((void *)sg.packed, 0, (int)wrange, 0x00020000);
    uint32_t w_off[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int64_t rb = rb0 + r;
        w_off[r] = (uint32_t)(rb < NB ? rb * KF * 256 + 16 * lane : wrange);
    }

    int acc[RB][MM];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int m = 0; m < MM; ++m) acc[r][m] = 0;
    auto dot16 = [](const v4i &a, const v4i &x, int c) {
        c = __builtin_amdgcn_sdot4(a.x, x.x, c, false);
        c = __builtin_amdgcn_sdot4(a.y, x.y, c, false);
        c = __builtin_amdgcn_sdot4(a.z, x.z, c, false);
        return __builtin_amdgcn_sdot4(a.w, x.w, c, false);
    };

    for (int64_t g0 = wave; g0 < NGfull; g0 += (int64_t)W * U) {
        v4u c[U][RB];
        v4i xv[U][4][MM];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = g0 + (int64_t)u * W;
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const uint32_t off = g < NGfull ? w_off[r] + (uint32_t)g * 1024u : wrange;
                c[u][r] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 2));
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = g0 + (int64_t)u * W;
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    const uint32_t off = g < NGfull ? x_off[m] + (uint32_t)(g * 256 + 64 * f) : xrange;
                    xv[u][f][m] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
                }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    const v4i a = unpack16_x64(c[u][r][f]);
#pragma unroll
                    for (int m = 0; m < MM; ++m) acc[r][m] = dot16(a, xv[u][f][m], acc[r][m]);
                }
    }
    // the partial last group (Gtail fragments: dword (lam, f) at lam*Gtail + f)
    if (Gtail && wave == (int)(NGfull % W)) {
        const int64_t g = NGfull;
        for (int f = 0; f < Gtail; ++f) {
            v4i xv[MM];
#pragma unroll
            for (int m = 0; m < MM; ++m)
                xv[m] = __builtin_amdgcn_raw_buffer_load_b128(xr, x_off[m] + (uint32_t)(g * 256 + 64 * f), 0, 0);
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const uint32_t base = w_off[r] - 16 * lane + (uint32_t)g * 1024u;
                const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(wr, base + 4u * (uint32_t)(lane * Gtail + f), 0, 0);
                const v4i a = unpack16_x64(w);
#pragma unroll
                for (int m = 0; m < MM; ++m) acc[r][m] = dot16(a, xv[m], acc[r][m]);
            }
        }
    }

    // lanes l, l^16, l^32, l^48 hold the four 16-column slices of row l % 16
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            int a = acc[r][m];
            a += __shfl_xor(a, 16, 64);
            a += __shfl_xor(a, 32, 64);
            if (lane < 16) red[wave][r][lane][m] = a;
        }
    __syncthreads();
    const float gm = sg.gamma[0];
    for (int t = threadIdx.x; t < RB * 16 * MM; t += W * 64) {
        const int m = t % MM, row = (t / MM) & 15, r = t / (16 * MM);
        if (m >= M) continue;
        int sum = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) sum += red[w][r][row][m];
        sum >>= 6;  // exact: every partial is a multiple of 64
        const int64_t n = (rb0 + r) * 16 + row;
        if (n < N) store_out(sg.y, sg.acc, m, n, N, sum, gm / sg.xs[m]);
    }
}

template <int W, int RB, int U, int MM>
hipError_t launch_dot4_shape(Dot4Segs &ds, hipStream_t s) {
    int64_t wg = 0;
    for (int i = 0; i < ds.count; ++i) {
        ds.s[i].wg_begin = wg;
        wg += (ds.s[i].NB + RB - 1) / RB;
    }
    hipLaunchKernelGGL((gemv_dot4_nt<W, RB, U, MM>), dim3((unsigned)wg), dim3(W * 64), 0, s, ds);
    return hipGetLastError();
}

// Launch shapes measured on the 70B layer: at one token, 16-wave workgroups
// of 2 row blocks where the launch has under 1024 of them (QKV 7.7 -> 7.2,
// O 6.3 -> 5.6, down 14.6 -> 12.5 us) and 8-wave ones otherwise; at 2..4
// tokens 8 waves x 2 row blocks (4 row blocks, 2 groups per sweep, 4- or
// 16-wave workgroups were no faster overall).
template <int MM>
hipError_t launch_dot4_mm(Dot4Segs &ds, int64_t wg2, hipStream_t s) {
    if (MM == 1 && wg2 < 1024) return launch_dot4_shape<16, 2, 1, MM>(ds, s);
    return launch_dot4_shape<8, 2, 1, MM>(ds, s);
}

// --------------------------------------------------------------- gemm_mfma
// Workgroup tile BM x BN (tokens x output rows) with WM x WN waves, each wave
// MF x NF fragments of 16 x 16.  The activation tile for KG groups (256
// columns each) is staged in LDS; code dwords come straight from the packed
// layout (lane l's dword is its A operand after unpacking).  MFMA operands:
// A = codes (rows = output rows n), B = activations (columns = tokens m);
// result lane l holds n = 4*(l/16) + r, m = l%16.
template <int WM, int WN, int MF, int NF, int KG, bool kAlignedK>
__global__ __launch_bounds__(WM *WN * 64) void gemm_mfma(
    const uint32_t *__restrict__ packed, const float *__restrict__ gamma, int64_t N, int64_t K,
    int64_t KF, int64_t NG, int64_t NB, const int8_t *__restrict__ xq,
    const float *__restrict__ xs, int64_t M, uint16_t *__restrict__ y,
    int32_t *__restrict__ acc_out) {
    constexpr int BM = WM * MF * 16;
    constexpr int BN = WN * NF * 16;
    constexpr int NT = WM * WN * 64;
    constexpr int KT = KG * 256;
    constexpr int LDS_STRIDE = KT + 16;
    __shared__ __attribute__((aligned(16))) int8_t xt[BM * LDS_STRIDE];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;

    v4i accv[NF][MF];
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
        for (int i = 0; i < MF; ++i) accv[j][i] = v4i{0, 0, 0, 0};

    const int64_t nstages = (NG + KG - 1) / KG;
    for (int64_t st = 0; st < nstages; ++st) {
        __syncthreads();
        // stage activations [BM][KT] (zero outside M x K)
        constexpr int CPR = KT / 16;  // 16-byte chunks per row
        for (int c = threadIdx.x; c < BM * CPR; c += NT) {
            const int r = c / CPR;
            const int col = (c - r * CPR) * 16;
            const int64_t gm = m0 + r;
            const int64_t gk = st * KT + col;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (gm < M && gk < K) v = load_x16<kAlignedK>(xq + gm * K, gk, K);
            *reinterpret_cast<uint4 *>(&xt[r * LDS_STRIDE + col]) = v;
        }
        __syncthreads();
        for (int gg = 0; gg < KG; ++gg) {
            const int64_t g = st * KG + gg;
            if (g >= NG) break;
            int64_t G = KF - 4 * g;
            if (G > 4) G = 4;
            uint32_t c[NF][4];
#pragma unroll
            for (int j = 0; j < NF; ++j) {
                const int64_t rb = n0 / 16 + wn * NF + j;
                c[j][0] = c[j][1] = c[j][2] = c[j][3] = 0u;
                if (rb < NB) {
                    const uint32_t *p = packed + rb * KF * 64 + g * 256;
                    if (G == 4) {
                        const uint4 v = *reinterpret_cast<const uint4 *>(p + lane * 4);
                        c[j][0] = v.x;
                        c[j][1] = v.y;
                        c[j][2] = v.z;
                        c[j][3] = v.w;
                    } else {
                        for (int f = 0; f < G; ++f) c[j][f] = p[lane * G + f];
                    }
                }
            }
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                if (f < G) {
                    v4i a[NF];
#pragma unroll
                    for (int j = 0; j < NF; ++j) a[j] = unpack16(c[j][f]);
#pragma unroll
                    for (int i = 0; i < MF; ++i) {
                        const int row = wm * MF * 16 + i * 16 + (lane & 15);
                        const v4i b = *reinterpret_cast<const v4i *>(
                            &xt[row * LDS_STRIDE + gg * 256 + f * 64 + 16 * (lane >> 4)]);
#pragma unroll
                        for (int j = 0; j < NF; ++j)
                            accv[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j], b, accv[j][i], 0, 0, 0);
                    }
                }
            }
        }
    }

    const float gm = gamma[0];
#pragma unroll
    for (int i = 0; i < MF; ++i) {
        const int64_t m = m0 + wm * MF * 16 + i * 16 + (lane & 15);
        if (m >= M) continue;
        const float scale = gm / xs[m];
#pragma unroll
        for (int j = 0; j < NF; ++j) {
            const int64_t nb = n0 + (wn * NF + j) * 16 + 4 * (lane >> 4);
            if ((N & 3) == 0 && nb + 3 < N) {
                uint2 o;
                o.x = (uint32_t)f32_to_bf16((float)accv[j][i][0] * scale) |
                      ((uint32_t)f32_to_bf16((float)accv[j][i][1] * scale) << 16);
                o.y = (uint32_t)f32_to_bf16((float)accv[j][i][2] * scale) |
                      ((uint32_t)f32_to_bf16((float)accv[j][i][3] * scale) << 16);
                *reinterpret_cast<uint2 *>(y + m * N + nb) = o;
                if (acc_out) *reinterpret_cast<v4i *>(acc_out + m * N + nb) = accv[j][i];
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (nb + r < N) store_out(y, acc_out, m, nb + r, N, accv[j][i][r], scale);
            }
        }
    }
}

template <int WM, int WN, int MF, int NF, int KG>
hipError_t launch_mfma(const uint32_t *packed, const float *gamma, const Layout &L,
                       const int8_t *xq, const float *xs, int64_t M, uint16_t *y, int32_t *acc,
                       hipStream_t s) {
    constexpr int BM = WM * MF * 16, BN = WN * NF * 16;
    const dim3 grid((unsigned)((L.N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    if (L.K % 16 == 0)
        hipLaunchKernelGGL((gemm_mfma<WM, WN, MF, NF, KG, true>), grid, dim3(WM * WN * 64), 0, s,
                           packed, gamma, L.N, L.K, L.KF, L.NG, L.NB, xq, xs, M, y, acc);
    else
        hipLaunchKernelGGL((gemm_mfma<WM, WN, MF, NF, KG, false>), grid, dim3(WM * WN * 64), 0, s,
                           packed, gamma, L.N, L.K, L.KF, L.NG, L.NB, xq, xs, M, y, acc);
    return hipGetLastError();
}

template <int MM>
hipError_t launch_dot4(const uint32_t *packed, const float *gamma, const Layout &L,
                       const int8_t *xq, const float *xs, uint16_t *y, int32_t *acc,
                       hipStream_t s) {
    const dim3 grid((unsigned)L.NB);
    if (L.K % 16 == 0)
        hipLaunchKernelGGL((gemv_dot4<MM, true>), grid, dim3(256), 0, s, packed, gamma, L.N, L.K,
                           L.KF, L.NG, xq, xs, y, acc);
    else
        hipLaunchKernelGGL((gemv_dot4<MM, false>), grid, dim3(256), 0, s, packed, gamma, L.N, L.K,
                           L.KF, L.NG, xq, xs, y, acc);
    return hipGetLastError();
}

}  // namespace

bool dot4_ok(const Layout &L, int64_t M) {
    constexpr int64_t kBufMax = ((int64_t)1 << 31) - ((int64_t)1 << 20);
    return M >= 1 && M <= kDot4MaxM && L.K % 16 == 0 && L.K <= kScaledMaxK && M * L.K < kBufMax &&
           L.bytes < kBufMax;
}

hipError_t launch_gemv_dot4_multi(const FwdSeg *segs, int count, hipStream_t s) {
    Dot4Segs ds{};
    ds.count = count;
    int64_t max_m = 0, wg2 = 0;
    for (int i = 0; i < count; ++i) {
        const FwdSeg &f = segs[i];
        ds.s[i] = Dot4Seg{f.packed, f.gamma, f.xq, f.xs, f.y, f.acc, f.L.N, f.L.K, f.L.KF, f.L.NB, f.M, 0};
        if (f.M > max_m) max_m = f.M;
        wg2 += (f.L.NB + 1) / 2;
    }
    if (max_m == 1) return launch_dot4_mm<1>(ds, wg2, s);
    if (max_m == 2) return launch_dot4_mm<2>(ds, wg2, s);
    return launch_dot4_mm<4>(ds, wg2, s);
}

hipError_t launch_forward(const uint32_t *packed, const float *gamma, const Layout &L,
                          const int8_t *xq, const float *xs, int64_t M, uint16_t *y, int32_t *acc,
                          hipStream_t s) {
    constexpr int64_t kBufMax = ((int64_t)1 << 31) - ((int64_t)1 << 20);
    const bool buf_ok = L.K % 16 == 0 && M * L.K < kBufMax && L.bytes < kBufMax;
    if (gemv_ok(L, M)) return launch_gemv(packed, gamma, L, xq, xs, M, y, acc, s);
    if (M == 1) return launch_dot4<1>(packed, gamma, L, xq, xs, y, acc, s);
    if (M == 2) return launch_dot4<2>(packed, gamma, L, xq, xs, y, acc, s);
    if (M <= 16) return launch_mfma<1, 4, 1, 1, 4>(packed, gamma, L, xq, xs, M, y, acc, s);
    if (M <= 32) return launch_mfma<1, 4, 2, 1, 4>(packed, gamma, L, xq, xs, M, y, acc, s);
    if (M <= 64) return launch_mfma<1, 4, 4, 1, 2>(packed, gamma, L, xq, xs, M, y, acc, s);
    if (buf_ok) return launch_gemm_pipe(packed, gamma, L, xq, xs, M, y, acc, s);
    return launch_mfma<2, 2, 4, 4, 1>(packed, gamma, L, xq, xs, M, y, acc, s);
}

}  // namespace bl
