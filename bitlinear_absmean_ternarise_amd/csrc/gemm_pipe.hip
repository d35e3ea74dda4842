// Prefill GEMM for the BitLinear contraction on gfx950.
//
// acc[m][n] = sum_k xq[m][k] * code[n][k] ("What one bit actually buys you":
// +1 adds, -1 subtracts, 0 skips; done 32 columns at a time by
// v_mfma_i32_32x32x32_i8 on int8 codes unpacked in registers), then
// y = bf16(acc * gamma / s_m) ("1-bit & Ternary LLMs (BitNet b1.58)",
// BitLinear forward equation: one float rescale per output).
//
// gfx950 issues one 32x32x32 int8 MFMA per 32 cycles per SIMD (65536 ops,
// the full int8 rate); the 16x16x64 form runs at half that rate, so this
// kernel is built on 32 x 32 fragments.
//
// Design (one workgroup of WM x WN waves per BM x BN output tile):
//  * The K loop runs over groups of 256 columns.  The activation tile
//    (BM x 256 int8) and the code tile (BN rows x 64 B) of a group are loaded
//    global -> VGPRs two groups ahead, written to one of two LDS slots, and
//    read back as MFMA operands (one barrier per group).
//  * Activations sit in LDS row-major (256 B per row) with the 16-byte chunk
//    index XOR-ed by (row & 15): global loads read whole 256 B rows, and both
//    the stores and the operand loads (32 rows x one chunk) are free of bank
//    conflicts.
//  * The code tile is a verbatim copy of the packed layout: for a 32-row
//    fragment, lane l's operand for a 32-column step is the dword of row
//    l % 32 and 16-column chunk l / 32 of that step, two 16-byte LDS reads
//    per group.  Each dword unpacks (shift, mask, byte permute) to the 16
//    int8 values of the A operand.
//  * A = unpacked codes (rows n), B = activations (columns m); each wave owns
//    MF x NF accumulator fragments of 32 x 32.
//  * Loads are issued uniformly (clamped addresses) so the compiler's vmcnt
//    waits stay exact; sched_barrier keeps the prefetch above the MFMAs; the
//    group barrier is s_waitcnt lgkmcnt(0) + a bare s_barrier (a
//    __syncthreads fence would also drain the prefetch).
//  * Tiles are assigned so the tiles of one XCD share activation rows.
// Requires K % 16 == 0 (16-byte aligned activation rows) and both buffers
// below 2 GB (32-bit buffer offsets); other shapes use the generic kernel.
#include "device.h"
#include "internal.h"

namespace bl {

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

template <int WM, int WN, int MF, int NF>
struct Cfg {
    static constexpr int W = WM * WN;
    static constexpr int NT = W * 64;
    static constexpr int BM = WM * MF * 32;
    static constexpr int BN = WN * NF * 32;
    static constexpr int ACT_BYTES = BM * 256;              // LDS per group
    static constexpr int ACT_LOADS = ACT_BYTES / 16 / NT;   // 16-byte loads per thread per group
    static constexpr int CODE_LOADS = 2 * NF;               // per lane per group, straight to VGPRs
    static constexpr int NR = ACT_LOADS + CODE_LOADS;
    static constexpr int STAGE_BYTES = ACT_BYTES;
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
    static_assert(ACT_BYTES % (16 * NT) == 0, "loads must split evenly");
};

__device__ __forceinline__ void lds_fence_barrier() {
    // own LDS stores done, then the hardware barrier; the empty asm blocks keep
    // the compiler from moving LDS accesses across it
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14));  // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int WM, int WN, int MF, int NF>
__global__ __launch_bounds__(WM *WN * 64) void gemm_pipe(
    const uint32_t *__restrict__ packed, const float *__restrict__ gamma, int64_t N, int64_t K,
    int64_t KF, int64_t NB, const int8_t *__restrict__ xq, const float *__restrict__ xs,
    int64_t M, int tiles_m, int tiles_n, uint16_t *__restrict__ y, int32_t *__restrict__ acc_out) {
    using C = Cfg<WM, WN, MF, NF>;
    constexpr int NR = C::NR;
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // XCD-aware tile order: workgroup w runs on XCD w % 8; give each XCD a
    // contiguous run of tiles in m-major order so its L2 keeps activation rows.
    const int T = tiles_m * tiles_n;
    int t = blockIdx.x;
    if ((T & 7) == 0) t = (blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3);
    const int tm = t / tiles_n, tn = t - tm * tiles_n;
    const int64_t m0 = (int64_t)tm * C::BM;
    const int64_t n0 = (int64_t)tn * C::BN;

    const int64_t NGfull = KF / 4;
    const int Gtail = (int)(KF - 4 * NGfull);  // fragments in the last, partial group (0 = none)
    const int64_t NG = NGfull + (Gtail ? 1 : 0);

    // ---- global loads through bounds-checked buffer descriptors: reads past
    // the end of either buffer return zeros, so rows past M, row blocks past
    // N and the bytes of a partial last group need no clamping.  (Bytes past
    // K inside a row belong to the next row; they only ever meet zero codes.)
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)xq, 0, (int)(M * K), 0x00020000);
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)packed, 0, (int)(NB * KF * 256), 0x00020000);
    uint32_t act_off[C::ACT_LOADS];
    int act_dst[C::ACT_LOADS];
#pragma unroll
    for (int i = 0; i < C::ACT_LOADS; ++i) {
        const int q = threadIdx.x + C::NT * i;  // 16-byte chunk of the tile
        const int r = q >> 4, c = q & 15;
        const int64_t m = m0 + r;
        act_off[i] = (uint32_t)(m < M ? m * K + 16 * c : M * K);
        act_dst[i] = r * 256 + ((c ^ (r & 15)) << 4);
    }
    // codes go straight to VGPRs: for fragment j (rows 32*(wn*NF+j) + l%32)
    // lane l needs, per group, the 16 bytes at lane position lam and lam + 32
    // of row block 2*(wn*NF+j) + (l%32)/16, lam = (l%32)%16 + 16*(l/32)
    const int lr = lane & 31, lh = lane >> 5;
    const int clam = (lr & 15) + 16 * lh;
    uint32_t code_off[C::CODE_LOADS];
#pragma unroll
    for (int j = 0; j < NF; ++j) {
        const int64_t rb = n0 / 16 + 2 * (wn * NF + j) + (lr >> 4);
        const uint32_t base = (uint32_t)(rb < NB ? rb * KF * 256 + 16 * clam : NB * KF * 256);
        code_off[2 * j] = base;
        code_off[2 * j + 1] = base + 512;
    }
    // the scale factors of this wave's rows, fetched early
    float xsv[MF];
#pragma unroll
    for (int i = 0; i < MF; ++i) {
        const int64_t m = m0 + (wm * MF + i) * 32 + lr;
        xsv[i] = xs[m < M ? m : M - 1];
    }
    const float gmv = gamma[0];

    auto load = [&](int64_t g, v4u(&r)[NR]) {
        const uint32_t kg = (uint32_t)g * 256u, cg = (uint32_t)g * 1024u;
#pragma unroll
        for (int i = 0; i < C::ACT_LOADS; ++i)
            r[i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(xrs, act_off[i] + kg, 0, 0));
#pragma unroll
        for (int i = 0; i < C::CODE_LOADS; ++i)
            r[C::ACT_LOADS + i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(crs, code_off[i] + cg, 0, 0));
    };
    auto store = [&](int stage, const v4u(&r)[NR]) {
        uint8_t *st = lds + stage * C::STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < C::ACT_LOADS; ++i) *reinterpret_cast<v4u *>(st + act_dst[i]) = r[i];
    };

    v16i acc[NF][MF];
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
        for (int i = 0; i < MF; ++i) acc[j][i] = v16i{};

    // ---- operand addressing inside a stage (all per-lane constants)
    // activation row of fragment i = (wm*MF + i)*32 + lr, swizzle key lr & 15;
    // chunk 2s + lh of that row sits at ((2s ^ key2) << 4) with key2 = lh ^ (lr & 15)
    const int key2 = lh ^ (lr & 15);
    const int arow0 = (wm * MF) * 32 * 256 + lr * 256;

    // B operands of step s: rows arow0 + i*8192, chunk (2s ^ key2)
    auto read_b = [&](const uint8_t *st, int s, v4i(&b)[MF]) {
        const uint8_t *p = st + arow0 + (((2 * s) ^ key2) << 4);
#pragma unroll
        for (int i = 0; i < MF; ++i) b[i] = *reinterpret_cast<const v4i *>(p + i * 32 * 256);
    };
    auto mma_step = [&](int s, const uint32_t(&cw)[NF][8], const v4i(&b)[MF]) {
        v4i a[NF];
#pragma unroll
        for (int j = 0; j < NF; ++j) a[j] = unpack16(cw[j][s]);
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
            for (int j = 0; j < NF; ++j)
                acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[j], b[i], acc[j][i], 0, 0, 0);
    };
    // a full group: the code dword of step s = 2f + h is dword f of lam + 32h
    auto codes_of = [&](const v4u(&r)[NR], uint32_t(&cw)[NF][8]) {
#pragma unroll
        for (int j = 0; j < NF; ++j) {
            const v4u lo = r[C::ACT_LOADS + 2 * j], hi = r[C::ACT_LOADS + 2 * j + 1];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                cw[j][2 * f] = lo[f];
                cw[j][2 * f + 1] = hi[f];
            }
        }
    };
    auto compute_full = [&](int stage, const v4u(&r)[NR]) {
        const uint8_t *st = lds + stage * C::STAGE_BYTES;
        uint32_t cw[NF][8];
        codes_of(r, cw);
        // operands of step s+1 are read while step s multiplies
        v4i b0[MF], b1[MF];
        read_b(st, 0, b0);
#pragma unroll
        for (int s = 0; s < 8; s += 2) {
            read_b(st, s + 1, b1);
            mma_step(s, cw, b0);
            if (s + 2 < 8) read_b(st, s + 2, b0);
            mma_step(s + 1, cw, b1);
        }
    };
    // the partial last group (Gtail fragments) was loaded from a group of
    // 64*Gtail dwords where dword (lam, f) sits at lam*Gtail + f; reload it
    // per dword (rare path)
    auto compute_tail = [&](int stage, int64_t g) {
        const uint8_t *st = lds + stage * C::STAGE_BYTES;
        uint32_t cw[NF][8];
#pragma unroll
        for (int j = 0; j < NF; ++j) {
            const uint32_t blk = code_off[2 * j] - 16 * clam + (uint32_t)g * 1024u;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int f = s >> 1, h = s & 1;
                cw[j][s] = (f < Gtail)
                    ? __builtin_amdgcn_raw_buffer_load_b32(crs, blk + 4u * (uint32_t)((clam + 32 * h) * Gtail + f), 0, 0)
                    : 0u;
            }
        }
        for (int s = 0; s < 2 * Gtail; ++s) {
            v4i b[MF];
            read_b(st, s, b);
            mma_step(s, cw, b);
        }
    };
    auto compute_any = [&](int64_t g, const v4u(&r)[NR]) {
        const int stage = (int)(g & 1);
        if (g < NGfull) {
            if (stage) compute_full(1, r);
            else compute_full(0, r);
        } else {
            compute_tail(stage, g);
        }
    };

    // ---- pipeline: LDS slot g&1 holds the activations of group g and a VGPR
    // set holds its codes; the other set is being filled for group g+1 / g+2.
    // rc keeps the codes of the group in LDS while its set is refilled.
    v4u r0[NR], r1[NR];
    load(0, r0);
    store(0, r0);
    if (NG > 1) load(1, r1);
    lds_fence_barrier();
    int64_t g = 0;
    // steady state: groups g, g+1 are full and g+2, g+3 exist
    // (sched_barrier keeps the scheduler from sinking the prefetch below the MFMAs)
    for (; g + 3 < NG; g += 2) {
        v4u rc[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) rc[i] = r0[i];
        load(g + 2, r0);
        __builtin_amdgcn_sched_barrier(0);
        compute_full(0, rc);
        store(1, r1);
        lds_fence_barrier();
#pragma unroll
        for (int i = 0; i < NR; ++i) rc[i] = r1[i];
        load(g + 3, r1);
        __builtin_amdgcn_sched_barrier(0);
        compute_full(1, rc);
        store(0, r0);
        lds_fence_barrier();
    }
    // tail: 1 to 3 groups left; slot g&1 holds g (codes in r0), r1 holds g+1
    {
        v4u rc[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) rc[i] = r0[i];
        if (g + 2 < NG) load(g + 2, r0);
        compute_any(g, rc);
    }
    if (g + 1 < NG) {
        store((int)((g + 1) & 1), r1);
        lds_fence_barrier();
        compute_any(g + 1, r1);
        if (g + 2 < NG) {
            store((int)(g & 1), r0);
            lds_fence_barrier();
            compute_any(g + 2, r0);
        }
    }

    // ---- epilogue: y[m][n] = bf16(acc * gamma / s_m).  Fragment lane l holds
    // m = l % 32 and n = 8*(r/4) + 4*(l/32) + r%4 for its 16 values r.
    float scale[MF];
#pragma unroll
    for (int i = 0; i < MF; ++i) scale[i] = gmv / xsv[i];
    if (acc_out == nullptr && (N & 7) == 0) {
        // Stage the bf16 tile in LDS (row-major, 16-byte chunks XOR-swizzled
        // by row) and write it out in whole rows: 16 lanes cover 256
        // contiguous bytes of y.
        constexpr int ROWB = C::BN * 2;   // bytes per tile row
        constexpr int CPR = C::BN / 8;    // 16-byte chunks per row
        lds_fence_barrier();              // every wave is done with the last stage
#pragma unroll
        for (int i = 0; i < MF; ++i) {
            const int r = (wm * MF + i) * 32 + lr;
#pragma unroll
            for (int j = 0; j < NF; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = (wn * NF + j) * 4 + q;
                    v2f f01 = {(float)acc[j][i][4 * q] * scale[i], (float)acc[j][i][4 * q + 1] * scale[i]};
                    v2f f23 = {(float)acc[j][i][4 * q + 2] * scale[i], (float)acc[j][i][4 * q + 3] * scale[i]};
                    uint2 o;
                    o.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(f01, v2bf));
                    o.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(f23, v2bf));
                    *reinterpret_cast<uint2 *>(lds + r * ROWB + ((c ^ (r & (CPR - 1))) << 4) + 8 * lh) = o;
                }
            }
        }
        lds_fence_barrier();
        constexpr int ROWS_PER_PASS = C::NT / CPR;
#pragma unroll
        for (int r0 = 0; r0 < C::BM; r0 += ROWS_PER_PASS) {
            const int r = r0 + (int)threadIdx.x / CPR, c = (int)threadIdx.x % CPR;
            const int64_t m = m0 + r, n = n0 + 8 * c;
            const v4u v = *reinterpret_cast<const v4u *>(lds + r * ROWB + ((c ^ (r & (CPR - 1))) << 4));
            if (m < M && n < N) *reinterpret_cast<v4u *>(y + m * N + n) = v;
        }
        return;
    }
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < MF; ++i) {
        const int64_t m = m0 + (wm * MF + i) * 32 + lr;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < NF; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t nb = n0 + (wn * NF + j) * 32 + 8 * q + 4 * lh;
                const int a0 = acc[j][i][4 * q], a1 = acc[j][i][4 * q + 1];
                const int a2 = acc[j][i][4 * q + 2], a3 = acc[j][i][4 * q + 3];
                v2f f01 = {(float)a0 * scale[i], (float)a1 * scale[i]};
                v2f f23 = {(float)a2 * scale[i], (float)a3 * scale[i]};
                const uint32_t h01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f01, v2bf));
                const uint32_t h23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f23, v2bf));
                if (vec && nb + 3 < N) {
                    *reinterpret_cast<uint2 *>(y + m * N + nb) = make_uint2(h01, h23);
                    if (acc_out) *reinterpret_cast<v4i *>(acc_out + m * N + nb) = v4i{a0, a1, a2, a3};
                } else {
                    const int av[4] = {a0, a1, a2, a3};
                    const uint16_t hv[4] = {(uint16_t)h01, (uint16_t)(h01 >> 16), (uint16_t)h23, (uint16_t)(h23 >> 16)};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (nb + r < N) {
                            y[m * N + nb + r] = hv[r];
                            if (acc_out) acc_out[m * N + nb + r] = av[r];
                        }
                    }
                }
            }
        }
    }
}

template <int WM, int WN, int MF, int NF>
hipError_t launch_cfg(const uint32_t *packed, const float *gamma, const Layout &L, const int8_t *xq,
                      const float *xs, int64_t M, uint16_t *y, int32_t *acc, hipStream_t s) {
    using C = Cfg<WM, WN, MF, NF>;
    const int tm = (int)((M + C::BM - 1) / C::BM);
    const int tn = (int)((L.N + C::BN - 1) / C::BN);
    auto kern = gemm_pipe<WM, WN, MF, NF>;
    static bool attr_set = false;  // LDS above 64 KB must be opted into
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           C::LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(tm * tn)), dim3(C::NT), C::LDS_BYTES, s, packed, gamma,
                       L.N, L.K, L.KF, L.NB, xq, xs, M, tm, tn, y, acc);
    return hipGetLastError();
}

// Workgroup shapes (WM, WN, MF, NF) of the three candidate tiles
#ifndef GEMM_CFG_A
#define GEMM_CFG_A 2, 2, 2, 2   /* 128 x 128, waves of 64 x 64 */
#endif
#ifndef GEMM_CFG_B
#define GEMM_CFG_B 4, 1, 2, 2   /* 256 x 64 */
#endif
#ifndef GEMM_CFG_C
#define GEMM_CFG_C 1, 2, 2, 2   /* 64 x 128 */
#endif

struct Choice {
    int id;
    int bm, bn, waves;
};

}  // namespace

// Tile choice: each wave owns a 128 x 32 output block (four activation
// fragments per unpacked code operand), so the work is a fixed number of
// wave tiles; pick the workgroup shape whose tiles waste the least of M x N
// to padding and of the 1024 SIMDs (256 CUs x 4) in the last round of waves;
// earlier (4-wave) candidates win ties.
hipError_t launch_gemm_pipe(const uint32_t *packed, const float *gamma, const Layout &L,
                            const int8_t *xq, const float *xs, int64_t M, uint16_t *y,
                            int32_t *acc, hipStream_t s) {
    // candidates: (id, BM, BN, waves)
    static const Choice cands[] = {{0, 128, 128, 4}, {1, 256, 64, 4}, {2, 64, 128, 2}};
    int best = 0;
    double best_eff = -1.0;
    for (const Choice &c : cands) {
        const int64_t tm = (M + c.bm - 1) / c.bm, tn = (L.N + c.bn - 1) / c.bn;
        const int64_t waves = tm * tn * c.waves;
        const int64_t rounds = (waves + 1023) / 1024;
        const double pad = (double)(M * L.N) / (double)(tm * c.bm * tn * c.bn);
        const double eff = pad * (double)waves / (double)(rounds * 1024);
        if (eff > best_eff + 1e-9) {
            best_eff = eff;
            best = c.id;
        }
    }
    switch (best) {
        case 0: return launch_cfg<GEMM_CFG_A>(packed, gamma, L, xq, xs, M, y, acc, s);
        case 1: return launch_cfg<GEMM_CFG_B>(packed, gamma, L, xq, xs, M, y, acc, s);
        default: return launch_cfg<GEMM_CFG_C>(packed, gamma, L, xq, xs, M, y, acc, s);
    }
}

}  // namespace bl
