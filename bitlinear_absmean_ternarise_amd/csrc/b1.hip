// Forward over binary weights stored one bit per code (packed layout b1).
//
// Binary BitNet ("1-bit & Ternary LLMs (BitNet b1.58)", How it works, BitNet
// equations): the codes are Sign(W - alpha) in {-1, +1} and the output scale
// is beta = mean |W|, so acc[m][n] = sum_k xq[m][k] * code[n][k] and
// y = bf16(acc * beta / s_m), the ternary forward with beta for gamma.  Two
// values need one bit, so a decode step streams half the bytes of the
// two-bit layout v1.
//
// The kernel keeps the structure of the two-bit decode kernel:
//  * A workgroup of W waves owns RB 16-row blocks and the whole K; wave w
//    takes the 1 KB groups w, w + W, ... of every row block (non-temporal
//    16-byte loads).  A b1 group is four 128-column pairs, so one lane's 16
//    bytes are its A operands for eight 64-column fragments.
//  * Half h of a lane dword becomes the 16 operand bytes as 64 * code: for
//    output dword j, ((w << (4h + j)) & 0x80808080) | 0x40404040 puts the
//    code bits of columns 4j..4j+3 in the byte signs, which read as +64 or
//    -64 (two VALU per four codes), and v_mfma_i32_16x16x64_i8 contracts them
//    against a 16-token x 64-column block of activations read through a
//    buffer descriptor whose range ends at the tile's last token, so token
//    rows past M read as zero.  The sums are 64 * acc exactly (64 * 127 * K <
//    2^31) and an arithmetic shift recovers acc.
//  * Tokens go 16 at a time: the workgroups of token tile t read tokens
//    16t..16t+15, one launch for any M (weights are re-read per tile: this
//    is a decode kernel; prefill reads the two-bit layout).
//  * The waves' partial sums meet in LDS, then the rescale and bf16 stores.
// Requires K % 64 == 0, K <= kScaledMaxK and packed buffers below 2 GB.
#include "../../include/bitlinear.h"
#include "device.h"
#include "internal.h"

namespace bl {

static_assert(BITLINEAR_B1_MAX_K == kScaledMaxK, "the b1 kernel sums 64 * code");

namespace {

struct B1Seg {
    const uint32_t *packed;
    const float *beta;
    const int8_t *xq;
    const float *xs;
    uint16_t *y;
    int32_t *acc;
    int64_t N, K, KP, NB, M;
    int64_t nsets;     // workgroups per token tile
    int64_t wg_begin;  // first workgroup of this segment
};
struct B1Segs {
    B1Seg s[kMaxSeg];
    int count;
};

constexpr int kStream = 2;  // non-temporal weight loads

template <int W, int RB, int U>
__global__ __launch_bounds__(W * 64) void gemv_b1(B1Segs segs) {
    __shared__ v4i red[W][RB][64];
    const int64_t wg = blockIdx.x;
    int sidx = 0;
#pragma unroll
    for (int i = 1; i < kMaxSeg; ++i)
        if (i < segs.count && wg >= segs.s[i].wg_begin) sidx = i;
    const B1Seg &sg = segs.s[sidx];
    const int64_t N = sg.N, K = sg.K, KP = sg.KP, NB = sg.NB, M = sg.M;
    const int64_t local = wg - sg.wg_begin;
    const int64_t tile = local / sg.nsets;
    const int64_t rb0 = (local - tile * sg.nsets) * RB;
    const int64_t m0 = tile * 16;
    const int64_t Mt = M - m0 < 16 ? M - m0 : 16;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // groups whose eight fragments are all real; the rest (up to seven
    // fragments: a partial group, or a whole group whose last half is
    // padding when K / 64 is odd) take the tail path
    const int64_t NGfull = K / 512;
    const int Gtail = (int)(KP - 4 * NGfull < 4 ? KP - 4 * NGfull : 4);  // pairs in that layout group
    const int Ftail = (int)(K / 64 - 8 * NGfull);                          // real fragments in it

    // token operand: lane l supplies token m0 + l % 16, columns 16*(l/16)..+15 of a fragment
    const uint32_t x_off = (uint32_t)((lane & 15) * K + 16 * (lane >> 4));
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void *)(sg.xq + m0 * K), 0, (int)(Mt * K), 0x00020000);
    const uint32_t wrange = (uint32_t)(NB * KP * 256);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc((void *)sg.packed, 0, (int)wrange, 0x00020000);
    uint32_t w_off[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int64_t rb = rb0 + r;
        w_off[r] = (uint32_t)(rb < NB ? rb * KP * 256 + 16 * lane : wrange);
    }

    v4i acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = v4i{0, 0, 0, 0};

    for (int64_t g0 = wave; g0 < NGfull; g0 += (int64_t)W * U) {
        v4u c[U][RB];
        v4i b[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = g0 + (int64_t)u * W;
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const uint32_t off = g < NGfull ? w_off[r] + (uint32_t)g * 1024u : wrange;
                c[u][r] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, kStream));
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = g0 + (int64_t)u * W;
            const bool in = g < NGfull;
#pragma unroll
            for (int f = 0; f < 8; ++f)
                b[u][f] = in ? __builtin_amdgcn_raw_buffer_load_b128(xr, x_off + (uint32_t)(g * 512 + 64 * f), 0, 0)
                             : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int f = 0; f < 8; ++f)
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    const uint32_t w = c[u][r][f >> 1];
                    acc[r] = __builtin_amdgcn_mfma_i32_16x16x64_i8((f & 1) ? unpack_b1<1>(w) : unpack_b1<0>(w),
                                                                   b[u][f], acc[r], 0, 0, 0);
                }
    }
    // the last group: Gtail pairs, dword (lam, p) at lam*Gtail + p, Ftail
    // real fragments (the last pair's second half is padding when Ftail is odd)
    if (Ftail && wave == (int)(NGfull % W)) {
        const int64_t g = NGfull;
        for (int f = 0; f < Ftail; ++f) {
            const v4i b = __builtin_amdgcn_raw_buffer_load_b128(xr, x_off + (uint32_t)(g * 512 + 64 * f), 0, 0);
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const uint32_t base = w_off[r] - 16 * lane + (uint32_t)g * 1024u;
                const uint32_t w =
                    __builtin_amdgcn_raw_buffer_load_b32(wr, base + 4u * (uint32_t)(lane * Gtail + (f >> 1)), 0, 0);
                acc[r] = __builtin_amdgcn_mfma_i32_16x16x64_i8((f & 1) ? unpack_b1<1>(w) : unpack_b1<0>(w), b, acc[r],
                                                               0, 0, 0);
            }
        }
    }

    // sum the waves' partials: lane l holds rows 4*(l/16)+q, token l%16
#pragma unroll
    for (int r = 0; r < RB; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    const float bt = sg.beta[0];
    for (int t = threadIdx.x; t < RB * 64; t += W * 64) {
        const int r = t >> 6, l = t & 63;
        v4i s = red[0][r][l];
#pragma unroll
        for (int w = 1; w < W; ++w) s += red[w][r][l];
        s >>= 6;  // exact: every partial is a multiple of 64
        const int64_t m = m0 + (l & 15);
        if (m >= M) continue;
        const float scale = bt / sg.xs[m];
        const int64_t n0 = (rb0 + r) * 16 + 4 * (l >> 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t n = n0 + q;
            if (n < N) {
                sg.y[m * N + n] = (uint16_t)pack_bf16x2((float)s[q] * scale, 0.0f);
                if (sg.acc) sg.acc[m * N + n] = s[q];
            }
        }
    }
}

template <int W, int RB, int U>
hipError_t launch_shape_b1(B1Segs &segs, hipStream_t s) {
    int64_t wg = 0;
    for (int i = 0; i < segs.count; ++i) {
        B1Seg &g = segs.s[i];
        g.wg_begin = wg;
        g.nsets = (g.NB + RB - 1) / RB;
        wg += g.nsets * ((g.M + 15) / 16);
    }
    hipLaunchKernelGGL((gemv_b1<W, RB, U>), dim3((unsigned)wg), dim3(W * 64), 0, s, segs);
    return hipGetLastError();
}

}  // namespace

bool b1_ok(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0 || K % 64 != 0 || K > kScaledMaxK) return false;
    return b1_bytes(N, K) < ((int64_t)1 << 31);
}

// Launch shape (measured on the 70B layer): 8 waves per workgroup and one
// 1 KB group per wave per sweep; launches with few workgroups take one row
// block per workgroup, long rows two groups per wave per sweep.  Above 8
// tokens each workgroup takes 4 row blocks, which reuses every token operand
// 4 times (16 tokens: 70B layer 69.9 -> 62.0 us; at 1 token it was slower,
// 42.7 -> 50.5 us).  Fewer waves per workgroup (2 or 4), 4 groups per sweep,
// or issuing the next sweep's weight loads before the current sweep's
// multiplies were all slower or no faster.  Up to 2 tokens a launch of
// 257..511 two-block workgroups takes three row blocks per workgroup, which
// evens out the workgroups per CU (70B QKV at one token: 7.61 -> 6.83 us;
// for 512..767, the 3B gate+up, three were slower: 5.69 -> 5.88 us).
hipError_t launch_forward_b1(const FwdSeg *segs, int count, hipStream_t s) {
    B1Segs bs{};
    bs.count = count;
    int64_t max_m = 0, max_k = 0, wg2 = 0;
    for (int i = 0; i < count; ++i) {
        const FwdSeg &f = segs[i];
        B1Seg &g = bs.s[i];
        g.packed = f.packed;
        g.beta = f.gamma;
        g.xq = f.xq;
        g.xs = f.xs;
        g.y = f.y;
        g.acc = f.acc;
        g.N = f.L.N;
        g.K = f.L.K;
        g.KP = (f.L.K + 127) / 128;
        g.NB = (f.L.N + 15) / 16;
        g.M = f.M;
        if (f.M > max_m) max_m = f.M;
        if (f.L.K > max_k) max_k = f.L.K;
        wg2 += (g.NB + 1) / 2 * ((f.M + 15) / 16);
    }
    if (max_m <= 8 && wg2 < 256)
        return max_k > 8192 ? launch_shape_b1<8, 1, 2>(bs, s) : launch_shape_b1<8, 1, 1>(bs, s);
    if (max_m > 8) return launch_shape_b1<8, 4, 1>(bs, s);
    if (max_k > 8192 && wg2 < 1024) return launch_shape_b1<8, 2, 2>(bs, s);
    if (max_m <= 2 && wg2 > 256 && wg2 < 512) return launch_shape_b1<8, 3, 1>(bs, s);
    return launch_shape_b1<8, 2, 1>(bs, s);
}

}  // namespace bl
