// Decode contraction for 1..16 tokens: stream the packed weights once.
//
// acc[m][n] = sum_k xq[m][k] * code[n][k] ("building a 1-bit llm, part 1",
// What one bit actually buys you: +1 adds, -1 subtracts, 0 skips), y = bf16(acc * gamma / s_m) ("1-bit &
// Ternary LLMs (BitNet b1.58)", BitLinear forward equation).
//
// Decode is bound by the weight bytes (two bits per weight), so the design
// is about keeping enough of them in flight:
//  * One workgroup of 8 waves owns RB (2 or 4) 16-row blocks (the rows of
//    its output) and the whole K; wave w takes the 1 KB groups w, w+8, ... of
//    every row block, so the workgroup's reads sweep contiguous memory.
//    Weight loads are non-temporal.
//  * Each lane's 16-byte load of a group is exactly its A operand for the
//    four 64-column fragments of the group (packed layout v1), unpacked in
//    registers (as 64 * code, 7 VALU per 16 codes, when K allows) and fed to
//    v_mfma_i32_16x16x64_i8; the B operand is the
//    16 x 64 block of tokens, read through a bounds-checked buffer
//    descriptor whose range ends at M*K, so token rows past M read as zero.
//    The matrix cores are otherwise idle here, so the contraction costs no
//    VALU beyond the unpacking.
//  * A lane keeps one group per row block in flight per sweep; the many
//    resident waves (6-8 per SIMD at 59-80 VGPRs) supply the parallelism.
//  * The waves' partial accumulators are summed through LDS, then rescaled.
// Requires K % 16 == 0 and buffers below 2 GB.
#include "device.h"
#include "internal.h"

namespace bl {

namespace {

struct GemvSeg {
    const uint32_t *packed;
    const float *gamma;
    const int8_t *xq;
    const float *xs;
    uint16_t *y;
    int32_t *acc;
    int64_t N, K, KF, NB, M;
    int64_t wg_begin;  // first workgroup of this segment
};
struct GemvSegs {
    GemvSeg s[kMaxSeg];
    int count;
};

// Cache policy of the weight loads: non-temporal (each weight byte is read
// once per forward; keep it from displacing the tokens in the caches).
constexpr int kStream = 2;

// W waves per workgroup, RB 16-row blocks per workgroup, U groups per wave
// per sweep; X64: codes unpacked as 64*code (needs K <= kScaledMaxK).
template <int W, int RB, int U, bool X64>
__device__ __forceinline__ void gemv_body(const GemvSeg &sg, int64_t blk, v4i (&red)[W][RB][64]) {
    const uint32_t *__restrict__ packed = sg.packed;
    const int64_t N = sg.N, K = sg.K, KF = sg.KF, NB = sg.NB, M = sg.M;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t rb0 = blk * RB;

    const int64_t NGfull = KF / 4;
    const int Gtail = (int)(KF - 4 * NGfull);

    // token operand: lane l supplies token l % 16, columns 16*(l/16)..+15 of a fragment
    const uint32_t x_off = (uint32_t)((lane & 15) * K + 16 * (lane >> 4));
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void *)sg.xq, 0, (int)(M * K), 0x00020000);
    // weights: lane l's 16 bytes of group g of row block rb
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc((void *)packed, 0, (int)(NB * KF * 256), 0x00020000);
    uint32_t w_off[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int64_t rb = rb0 + r;
        w_off[r] = (uint32_t)(rb < NB ? rb * KF * 256 + 16 * lane : NB * KF * 256);
    }

    v4i acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = v4i{0, 0, 0, 0};

    // full groups: sweeps of U groups per wave; every load of a sweep
    // (weights and token operands) is issued before the first MFMA
    for (int64_t g0 = wave; g0 < NGfull; g0 += (int64_t)W * U) {
        v4u c[U][RB];
        v4i b[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = g0 + (int64_t)u * W;
            const bool in = g < NGfull;
#pragma unroll
            for (int r = 0; r < RB; ++r)
                c[u][r] = in ? __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(wr, w_off[r] + (uint32_t)g * 1024u, 0, kStream))
                             : v4u{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = g0 + (int64_t)u * W;
            const bool in = g < NGfull;
#pragma unroll
            for (int f = 0; f < 4; ++f)
                b[u][f] = in ? __builtin_amdgcn_raw_buffer_load_b128(xr, x_off + (uint32_t)(g * 256 + 64 * f), 0, 0)
                             : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
                for (int r = 0; r < RB; ++r)
                    acc[r] = __builtin_amdgcn_mfma_i32_16x16x64_i8(X64 ? unpack16_x64(c[u][r][f]) : unpack16(c[u][r][f]),
                                                                   b[u][f], acc[r], 0, 0, 0);
        }
    }
    // the partial last group (Gtail fragments: dword (lam, f) at lam*Gtail + f)
    if (Gtail && wave == (int)(NGfull % W)) {
        const int64_t g = NGfull;
        for (int f = 0; f < Gtail; ++f) {
            const v4i b = __builtin_amdgcn_raw_buffer_load_b128(xr, x_off + (uint32_t)(g * 256 + 64 * f), 0, 0);
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const uint32_t base = w_off[r] - 16 * lane + (uint32_t)g * 1024u;
                const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(wr, base + 4u * (uint32_t)(lane * Gtail + f), 0, 0);
                acc[r] = __builtin_amdgcn_mfma_i32_16x16x64_i8(X64 ? unpack16_x64(w) : unpack16(w), b, acc[r], 0, 0, 0);
            }
        }
    }

    // sum the waves' partials: lane l holds rows 4*(l/16)+q, token l%16
#pragma unroll
    for (int r = 0; r < RB; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    // thread t: row block t / 64 (of RB), lane t % 64
    const float gm = sg.gamma[0];
    for (int t = threadIdx.x; t < RB * 64; t += W * 64) {
        const int r = t >> 6, l = t & 63;
        v4i s = red[0][r][l];
#pragma unroll
        for (int w = 1; w < W; ++w) s += red[w][r][l];
        if (X64) s >>= 6;  // exact: every partial is a multiple of 64
        const int64_t m = l & 15;
        if (m >= M) continue;
        const float scale = gm / sg.xs[m];
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

// One launch over up to kMaxSeg independent forwards: workgroup w belongs to
// the last segment whose first workgroup is <= w.
template <int W, int RB, int U, bool X64>
__global__ __launch_bounds__(W * 64) void gemv_mfma16(GemvSegs segs) {
    __shared__ v4i red[W][RB][64];
    const int64_t w = blockIdx.x;
    int sidx = 0;
#pragma unroll
    for (int i = 1; i < kMaxSeg; ++i)
        if (i < segs.count && w >= segs.s[i].wg_begin) sidx = i;
    const GemvSeg &sg = segs.s[sidx];
    gemv_body<W, RB, U, X64>(sg, w - sg.wg_begin, red);
}

template <int W, int RB, int U, bool X64>
hipError_t launch_shape(GemvSegs &segs, hipStream_t s) {
    int64_t wg = 0;
    for (int i = 0; i < segs.count; ++i) {
        segs.s[i].wg_begin = wg;
        wg += (segs.s[i].NB + RB - 1) / RB;
    }
    hipLaunchKernelGGL((gemv_mfma16<W, RB, U, X64>), dim3((unsigned)wg), dim3(W * 64), 0, s, segs);
    return hipGetLastError();
}

// Launch shape: 8 waves per workgroup and one 1 KB group per wave per sweep
// keep a lane at 59-80 VGPRs, so 6-8 waves share each SIMD and the wave
// count, not per-wave unrolling, keeps the weight bytes in flight (measured
// on the 70B layer: fewer, fatter waves or 16-wave workgroups were slower).
// Above 8 tokens the token operands are a larger share of the loads, so each
// workgroup takes 4 row blocks to reuse them.
//
// Long rows in a launch of few workgroups (the down projection: K = 8640 at
// 3B, 28672 at 70B, under 1024 workgroups of 2 row blocks) take two groups
// per wave per sweep, which halves the sweeps each wave waits through
// (measured on the 70B layer: down 15.3 -> 12.7 us at M = 1, 23.2 -> 20.4 us
// at M = 16; shorter rows got slower with it).
//
// Up to 8 tokens, a launch with fewer two-row-block workgroups than CUs (the
// 3B O and down projections: 100) takes one row block per workgroup, which
// spreads it over twice the CUs (3B at M = 1: O 4.2 -> 3.8 us, down 5.6 ->
// 5.0 us).  Launches with more workgroups got slower with one row block.
template <bool X64>
hipError_t launch_x(GemvSegs &segs, int64_t max_m, int64_t max_k, hipStream_t s) {
    int64_t wg2 = 0;
    for (int i = 0; i < segs.count; ++i) wg2 += (segs.s[i].NB + 1) / 2;
    if (max_m <= 8 && wg2 < 256)
        return max_k > 8192 ? launch_shape<8, 1, 2, X64>(segs, s) : launch_shape<8, 1, 1, X64>(segs, s);
    if (max_k > 8192 && wg2 < 1024) return launch_shape<8, 2, 2, X64>(segs, s);
    if (max_m <= 8) return launch_shape<8, 2, 1, X64>(segs, s);
    return launch_shape<8, 4, 1, X64>(segs, s);
}

// ---------------------------------------------------------------------------
// 17..64 tokens: the same streaming structure on v_mfma_i32_32x32x32_i8 (full
// int8 rate; the 16x16x64 form would make 64 tokens MFMA-bound).  A workgroup
// owns RP pairs of row blocks (32 rows each); wave w takes groups w, w+W, ...
// A lane's A operand for 32-column step s = 2f + h of a group is dword f of
// the 16 bytes at lane position lam + 32h of its row block, lam = (l%32)%16 +
// 16*(l/32): two 16-byte loads per pair per group.  The B operand is token
// tb*32 + l%32, 16 bytes at column 32s + 16*(l/32), read from L2 through a
// descriptor whose range ends at M*K (tokens past M read as zero).  Lane l's
// result r belongs to token tb*32 + l%32 and row 8*(r/4) + 4*(l/32) + r%4 of
// the pair.  Partial sums of the waves meet in LDS through integer atomics.
typedef int v16i __attribute__((ext_vector_type(16)));

template <int W, int RP, int TB, bool X64>
__device__ __forceinline__ void gemv32_body(const GemvSeg &sg, int64_t blk, int32_t *red, uint8_t *tok) {
    const int64_t N = sg.N, K = sg.K, KF = sg.KF, NB = sg.NB, M = sg.M;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 31, lh = lane >> 5;
    const int64_t NGfull = KF / 4;
    const int Gtail = (int)(KF - 4 * NGfull);
    const int64_t rp0 = blk * RP;

    constexpr int RED = RP * TB * 16 * 64;  // int32 slots (may alias the token tiles)

    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc((void *)sg.packed, 0, (int)(NB * KF * 256), 0x00020000);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void *)sg.xq, 0, (int)(M * K), 0x00020000);
    const int clam = (lr & 15) + 16 * lh;
    uint32_t c_off[RP];
#pragma unroll
    for (int p = 0; p < RP; ++p) {
        const int64_t rb = 2 * (rp0 + p) + (lr >> 4);
        c_off[p] = (uint32_t)(rb < NB ? rb * KF * 256 + 16 * clam : NB * KF * 256);
    }
    uint32_t x_off[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const int64_t t = tb * 32 + lr;
        x_off[tb] = (uint32_t)((t < M ? t * K : M * K) + 16 * lh);
    }

    v16i acc[RP][TB];
#pragma unroll
    for (int p = 0; p < RP; ++p)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[p][tb] = v16i{};

    auto mma = [&](uint32_t code, const v4i (&bs)[TB], v16i (&ap)[TB]) {
        const v4i a = X64 ? unpack16_x64(code) : unpack16(code);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) ap[tb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bs[tb], ap[tb], 0, 0, 0);
    };

    // Token tiles (32 tokens x 256 bytes of the group) go through this wave's
    // own 8 KB of LDS: row r, 16-byte chunk c at r*256 + ((c ^ (r & 15)) << 4).
    // Global loads read whole rows (16 lanes per 256-byte row); the operand
    // reads (32 rows, one chunk) hit distinct banks.  Read straight from L2 in
    // operand order, each 16-byte load would touch 32 rows (32 bytes of each
    // 128-byte line) and the line traffic, not HBM, would set the pace.
    uint8_t *wtok = tok + wave * 8192;
    const int ld_r = lane >> 4, ld_c = lane & 15;
    for (int64_t g = wave; g < NGfull; g += W) {
        v4u cl[RP][2];
#pragma unroll
        for (int p = 0; p < RP; ++p)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                cl[p][h] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(
                                                       wr, c_off[p] + 512u * h + (uint32_t)g * 1024u, 0, kStream));
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            v4i t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t row = tb * 32 + 4 * j + ld_r;
                const uint32_t off = (uint32_t)((row < M ? row * K : M * K) + g * 256 + 16 * ld_c);
                t[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 4 * j + ld_r;
                *reinterpret_cast<v4i *>(wtok + r * 256 + ((ld_c ^ (r & 15)) << 4)) = t[j];
            }
            v4i bs[8][1];
#pragma unroll
            for (int st = 0; st < 8; ++st)
                bs[st][0] = *reinterpret_cast<const v4i *>(wtok + lr * 256 + (((2 * st + lh) ^ (lr & 15)) << 4));
#pragma unroll
            for (int st = 0; st < 8; ++st)
#pragma unroll
                for (int p = 0; p < RP; ++p) {
                    const uint32_t code = cl[p][st & 1][st >> 1];
                    const v4i a = X64 ? unpack16_x64(code) : unpack16(code);
                    acc[p][tb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bs[st][0], acc[p][tb], 0, 0, 0);
                }
        }
    }
    // partial last group: Gtail fragments, dword (lam, f) at lam*Gtail + f
    if (Gtail && wave == (int)(NGfull % W)) {
        const int64_t g = NGfull;
        for (int st = 0; st < 2 * Gtail; ++st) {
            const int f = st >> 1, h = st & 1;
            v4i b[TB];
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
                b[tb] = __builtin_amdgcn_raw_buffer_load_b128(xr, x_off[tb] + (uint32_t)(g * 256 + 32 * st), 0, 0);
#pragma unroll
            for (int p = 0; p < RP; ++p) {
                const uint32_t base = c_off[p] - 16 * clam + (uint32_t)g * 1024u;
                const uint32_t code = __builtin_amdgcn_raw_buffer_load_b32(
                    wr, base + 4u * (uint32_t)((clam + 32 * h) * Gtail + f), 0, 0);
                mma(code, b, acc[p]);
            }
        }
    }

    __syncthreads();  // every wave is done with its token tile
    for (int i = threadIdx.x; i < RED; i += W * 64) red[i] = 0;
    __syncthreads();
#pragma unroll
    for (int p = 0; p < RP; ++p)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (acc[p][tb][r]) atomicAdd(&red[((p * TB + tb) * 16 + r) * 64 + lane], acc[p][tb][r]);
    __syncthreads();

    // thread t: 4 consecutive rows n (chunk c = t%8 of the pair's 32 rows) of
    // one token; 8 threads cover 64 contiguous bytes of a y row
    const float gm = sg.gamma[0];
    for (int t = threadIdx.x; t < RP * TB * 32 * 8; t += W * 64) {
        const int c = t & 7, ml = (t >> 3) & 31, pt = t >> 8;  // pt = p * TB + tb
        const int p = pt / TB, tb = pt - p * TB;
        const int64_t m = tb * 32 + ml;
        const int64_t n0 = (rp0 + p) * 32 + 4 * c;
        if (m >= M || n0 >= N) continue;
        const int j = c >> 1, h = c & 1;
        const int32_t *src = red + (pt * 16 + 4 * j) * 64 + 32 * h + ml;
        int v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = X64 ? (src[64 * q] >> 6) : src[64 * q];  // exact
        const float scale = gm / sg.xs[m];
        const uint32_t h01 = pack_bf16x2((float)v[0] * scale, (float)v[1] * scale);
        const uint32_t h23 = pack_bf16x2((float)v[2] * scale, (float)v[3] * scale);
        if (n0 + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<uint2 *>(sg.y + m * N + n0) = make_uint2(h01, h23);
            if (sg.acc) *reinterpret_cast<v4i *>(sg.acc + m * N + n0) = v4i{v[0], v[1], v[2], v[3]};
        } else {
            const uint16_t hv[4] = {(uint16_t)h01, (uint16_t)(h01 >> 16), (uint16_t)h23, (uint16_t)(h23 >> 16)};
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (n0 + q < N) {
                    sg.y[m * N + n0 + q] = hv[q];
                    if (sg.acc) sg.acc[m * N + n0 + q] = v[q];
                }
        }
    }
}

template <int W, int RP, int TB, bool X64>
__global__ __launch_bounds__(W * 64) void gemv_mfma32(GemvSegs segs) {
    constexpr int RED_BYTES = RP * TB * 16 * 64 * 4, TOK_BYTES = W * 8192;
    __shared__ __attribute__((aligned(16))) uint8_t lds[RED_BYTES > TOK_BYTES ? RED_BYTES : TOK_BYTES];
    const int64_t w = blockIdx.x;
    int sidx = 0;
#pragma unroll
    for (int i = 1; i < kMaxSeg; ++i)
        if (i < segs.count && w >= segs.s[i].wg_begin) sidx = i;
    const GemvSeg &sg = segs.s[sidx];
    gemv32_body<W, RP, TB, X64>(sg, w - sg.wg_begin, reinterpret_cast<int32_t *>(lds), lds);
}

template <int W, int RP, int TB, bool X64>
hipError_t launch_shape32(GemvSegs &segs, hipStream_t s) {
    int64_t wg = 0;
    for (int i = 0; i < segs.count; ++i) {
        segs.s[i].wg_begin = wg;
        const int64_t pairs = (segs.s[i].NB + 1) / 2;
        wg += (pairs + RP - 1) / RP;
    }
    hipLaunchKernelGGL((gemv_mfma32<W, RP, TB, X64>), dim3((unsigned)wg), dim3(W * 64), 0, s, segs);
    return hipGetLastError();
}

// Measured on the 70B layer: 8 waves x 2 pairs for one token block; for two
// blocks the accumulators double and 4-wave workgroups keep more of them
// resident.
template <bool X64>
hipError_t launch_x32(GemvSegs &segs, int64_t max_m, hipStream_t s) {
    if (max_m <= 32) return launch_shape32<8, 2, 1, X64>(segs, s);
    return launch_shape32<4, 2, 2, X64>(segs, s);
}

}  // namespace

bool gemv_ok(const Layout &L, int64_t M) {
    constexpr int64_t kBufMax = ((int64_t)1 << 31) - ((int64_t)1 << 20);
    return M >= 1 && M <= kGemvMaxM && L.K % 16 == 0 && M * L.K < kBufMax && L.bytes < kBufMax;
}

hipError_t launch_gemv_multi(const FwdSeg *fs, int count, hipStream_t s) {
    GemvSegs segs{};
    int64_t max_m = 0, max_k = 0;
    for (int i = 0; i < count; ++i) {
        GemvSeg &g = segs.s[i];
        const Layout &L = fs[i].L;
        g.packed = fs[i].packed;
        g.gamma = fs[i].gamma;
        g.xq = fs[i].xq;
        g.xs = fs[i].xs;
        g.y = fs[i].y;
        g.acc = fs[i].acc;
        g.N = L.N;
        g.K = L.K;
        g.KF = L.KF;
        g.NB = L.NB;
        g.M = fs[i].M;
        max_m = fs[i].M > max_m ? fs[i].M : max_m;
        max_k = L.K > max_k ? L.K : max_k;
    }
    segs.count = count;
    const bool x64 = max_k <= kScaledMaxK;
    if (max_m <= 16) return x64 ? launch_x<true>(segs, max_m, max_k, s) : launch_x<false>(segs, max_m, max_k, s);
    return x64 ? launch_x32<true>(segs, max_m, s) : launch_x32<false>(segs, max_m, s);
}

hipError_t launch_gemv(const uint32_t *packed, const float *gamma, const Layout &L, const int8_t *xq,
                       const float *xs, int64_t M, uint16_t *y, int32_t *acc, hipStream_t s) {
    FwdSeg f{packed, gamma, L, xq, xs, M, y, acc};
    return launch_gemv_multi(&f, 1, s);
}

}  // namespace bl
