// The int8 MFMA GEMM for the BitLinear contraction on gfx950 (prefill, and
// decode batches of 14..64 tokens).
//
// acc[m][n] = sum_k xq[m][k] * code[n][k] ("building a 1-bit llm, part 1",
// What one bit actually buys you: +1 adds, -1 subtracts, 0 skips; done 32 columns at a time by
// v_mfma_i32_32x32x32_i8 on int8 codes unpacked in registers), then
// y = bf16(acc * gamma / s_m) ("1-bit & Ternary LLMs (BitNet b1.58)",
// BitLinear forward equation: one float rescale per output).
//
// gfx950 issues one 32x32x32 int8 MFMA per 32 cycles per SIMD (65536 ops,
// the full int8 rate); the 16x16x64 form runs at half that rate, so this
// kernel is built on 32 x 32 fragments.
//
// Design (one workgroup of WM x WN waves per BM x BN output tile):
//  * The K loop runs over groups of 256 columns.  Each group's activation
//    tile (BM x 256 int8) and each wave's code dwords are loaded global ->
//    VGPRs through bounds-checked buffer descriptors into a ring of D
//    register sets, D - 1 groups ahead of the group being multiplied; the
//    activations are then written to one of two LDS slots (one barrier per
//    group) and read back as MFMA B operands.
//  * Activations sit in LDS row-major (256 B per row) with the 16-byte chunk
//    index XOR-ed by (row & 15): global loads read whole 256 B rows, and both
//    the stores and the operand loads (32 rows x one chunk) are free of bank
//    conflicts.
//  * Codes never touch LDS: for a 32-row fragment, lane l's operand for a
//    32-column step is the dword of row l % 32 and 16-column chunk l / 32 of
//    that step, i.e. two 16-byte loads per group straight from the packed
//    layout.  Each dword unpacks (shift, mask, byte permute) to the 16 int8
//    values of the A operand; the next step is unpacked while the current
//    one multiplies.
//  * A = unpacked codes (rows n), B = activations (columns m); each wave owns
//    MF x NF accumulator fragments of 32 x 32.
//  * Loads are issued uniformly with loop-invariant per-lane offsets (the
//    group offset lives in the descriptor) so the compiler's vmcnt waits stay
//    exact; sched_barrier keeps the prefetch above the MFMAs; the group
//    barrier is s_waitcnt lgkmcnt(0) + a bare s_barrier (a __syncthreads
//    fence would also drain the prefetch).
//  * Tiles are assigned so the tiles of one XCD share activation rows.
//  * Epilogue: the bf16 tile (v_cvt_pk_bf16_f32) is staged in LDS and
//    written out in whole 256-byte rows.
//  * The same kernel takes decode batches of 14..64 tokens (its 64 x 128 and
//    32 x 256 tiles), where K may be cut into runs: a run's workgroup writes
//    its int32 sums to a workspace and splitk_reduce adds the runs and
//    applies the epilogue (the plan at the end of this file).
// Requires K % 16 == 0 (16-byte aligned activation rows) and both buffers
// below 2 GB (32-bit buffer offsets); other shapes use the generic kernel.
#include <cstdint>
#include <type_traits>

#include "../../include/bitlinear.h"
#include "device.h"
#include "internal.h"

namespace bl {

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

// One GEMM of a (possibly grouped) launch: its tiles are workgroups
// tile_begin .. tile_begin + splits * tiles_m * tiles_n - 1 of the launch.
// With splits > 1 the K groups are cut into `splits` runs of `gps` groups
// (the last run may be shorter and holds the partial last group); the
// workgroup of run r writes its int32 sums to part + r * M * N ([M][N]) and
// splitk_reduce adds the runs and applies the epilogue.
struct GemmSeg {
    const uint32_t *packed;
    const float *gamma;
    const int8_t *xq;
    const float *xs;
    uint16_t *y;
    int32_t *acc;
    int32_t *part;  // NULL: one run, the epilogue writes y (and acc)
    int64_t N, K, KF, NB, M;
    int64_t gps;    // groups per run
    int tiles_m, tiles_n, tile_begin, splits;
};
struct GemmSegs {
    GemmSeg s[kMaxSeg];
    int count, total_tiles;
};

// WM x WN waves per K slice, each owning MF x NF fragments of 32 x 32; KS
// slices per workgroup split the K groups between them (slice k takes groups
// k, k + KS, ...) and add their accumulators at the end.
template <int WM, int WN, int MF, int NF, int KS>
struct Cfg {
    static constexpr int W = WM * WN;                        // waves per slice
    static constexpr int NT = W * 64;                        // threads per slice
    static constexpr int NTT = NT * KS;                      // threads per workgroup
    static constexpr int BM = WM * MF * 32;
    static constexpr int BN = WN * NF * 32;
    static constexpr int ACT_BYTES = BM * 256;              // LDS per group
    static constexpr int ACT_LOADS = ACT_BYTES / 16 / NT;   // 16-byte loads per thread per group
    static constexpr int CODE_LOADS = 2 * NF;               // per lane per group, straight to VGPRs
    static constexpr int NR = ACT_LOADS + CODE_LOADS;
    static constexpr int STAGE_BYTES = ACT_BYTES;
    static constexpr int SLICE_BYTES = 2 * STAGE_BYTES;     // two stages per slice
    static constexpr int RED_BYTES = KS > 1 ? W * MF * NF * 16 * 64 * 4 : 0;  // one slice's accumulators
    static constexpr int EPI_BYTES = BM * BN * 2;           // the bf16 tile
    static constexpr int LDS_BYTES = (KS * SLICE_BYTES > RED_BYTES ? KS * SLICE_BYTES : RED_BYTES) > EPI_BYTES
                                         ? (KS * SLICE_BYTES > RED_BYTES ? KS * SLICE_BYTES : RED_BYTES)
                                         : EPI_BYTES;
    static_assert(ACT_BYTES % (16 * NT) == 0, "loads must split evenly");
    static_assert(KS == 1 || KS == 2, "K slices");
};

__device__ __forceinline__ void lds_fence_barrier() {
    // own LDS stores done, then the hardware barrier; the empty asm blocks keep
    // the compiler from moving LDS accesses across it
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14));  // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// X64: codes unpacked as 64 * code (7 VALU per dword instead of 11), the
// accumulators shifted back by 6 before the epilogue; needs K <= kScaledMaxK.
// D: depth of the register ring (2, or 4 where the VGPR budget allows);
// WPE: waves per SIMD the register budget is sized for.
template <int WM, int WN, int MF, int NF, int KS, bool X64, int D = 2, int WPE = 2>
__global__ __launch_bounds__(WM *WN * 64 * KS) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void gemm_pipe(GemmSegs segs) {
    using C = Cfg<WM, WN, MF, NF, KS>;
    constexpr int NR = C::NR;
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds_all[];

    const int lane = threadIdx.x & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = wave_all / C::W;             // K slice of this wave
    const int wave = wave_all - ks * C::W;      // wave within the slice
    const int tid = (int)threadIdx.x - ks * C::NT;  // thread within the slice
    const int wm = wave / WN, wn = wave % WN;
    uint8_t *lds = lds_all + ks * C::SLICE_BYTES;   // this slice's two stages

    // XCD-aware tile order: workgroup w runs on XCD w % 8; give each XCD a
    // contiguous run of tiles in m-major order so its L2 keeps activation rows
    // (and, in a grouped launch, mostly one GEMM's weights).
    const int T = segs.total_tiles;
    int t = blockIdx.x;
    if ((T & 7) == 0) t = (blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3);
    int sidx = 0;
#pragma unroll
    for (int i = 1; i < kMaxSeg; ++i)
        if (i < segs.count && t >= segs.s[i].tile_begin) sidx = i;
    const GemmSeg &sg = segs.s[sidx];
    const uint32_t *__restrict__ packed = sg.packed;
    const float *__restrict__ gamma = sg.gamma;
    const int8_t *__restrict__ xq = sg.xq;
    const float *__restrict__ xs = sg.xs;
    uint16_t *__restrict__ y = sg.y;
    int32_t *__restrict__ acc_out = sg.acc;
    const int64_t N = sg.N, K = sg.K, KF = sg.KF, NB = sg.NB, M = sg.M;
    const int tiles_n = sg.tiles_n;
    t -= sg.tile_begin;
    // run outermost: the tiles of one run (one range of K) sit next to each
    // other, so an XCD's tiles mostly share the run's activation columns
    const int tmn = sg.tiles_m * tiles_n;
    const int run = t / tmn;
    t -= run * tmn;
    const int tm = t / tiles_n, tn = t - tm * tiles_n;
    const int64_t m0 = (int64_t)tm * C::BM;
    const int64_t n0 = (int64_t)tn * C::BN;

    const int64_t NGfull = KF / 4;
    const int Gtail = (int)(KF - 4 * NGfull);  // fragments in the last, partial group (0 = none)
    const int64_t NG = NGfull + (Gtail ? 1 : 0);
    // this workgroup's groups: gb .. ge - 1, of which NGf full ones first and
    // then, in the last run, the partial group
    const int64_t gb = (int64_t)run * sg.gps;
    const int64_t ge = gb + sg.gps < NG ? gb + sg.gps : NG;
    const int64_t NGf = (ge < NGfull ? ge : NGfull) - gb;
    const bool tail = Gtail && ge == NG;
    const int64_t NGl = NGf + (tail ? 1 : 0);

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
        const int q = tid + C::NT * i;  // 16-byte chunk of the tile
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

    // The group offset goes into the descriptors (base advanced, range shrunk
    // by the same amount, so the bounds check stays exact) and the per-lane
    // offsets stay loop-invariant: no address registers are rewritten between
    // loads, which keeps the compiler's vmcnt waits exact.
    auto load = [&](int64_t g, v4u(&r)[NR]) {
        const int64_t kg = g * 256, cg = g * 1024;
        const __amdgpu_buffer_rsrc_t xg = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(xq + kg), 0, (int)(M * K - kg), 0x00020000);
        const __amdgpu_buffer_rsrc_t cgr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(packed + cg / 4), 0, (int)(NB * KF * 256 - cg), 0x00020000);
#pragma unroll
        for (int i = 0; i < C::ACT_LOADS; ++i)
            r[i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(xg, act_off[i], 0, 0));
#pragma unroll
        for (int i = 0; i < C::CODE_LOADS; ++i)
            r[C::ACT_LOADS + i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(cgr, code_off[i], 0, 0));
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
        for (int j = 0; j < NF; ++j) a[j] = X64 ? unpack16_x64(cw[j][s]) : unpack16(cw[j][s]);
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
    // Eight 32-column steps.  B operands are read two steps ahead and the A
    // operands of step s+1 are unpacked while step s multiplies.  A scheduling
    // fence after every step keeps that order (left alone, the compiler
    // clusters the MFMAs of one accumulator and moves each LDS read next to
    // its use, exposing the LDS latency on every MFMA); inside a step the
    // independent MFMAs alternate with the unpacking.
    auto compute_full = [&](int stage, const v4u(&r)[NR]) {
        const uint8_t *st = lds + stage * C::STAGE_BYTES;
        uint32_t cw[NF][8];
        codes_of(r, cw);
        v4i bq[3][MF];
        v4i a_cur[NF], a_nxt[NF];
        read_b(st, 0, bq[0]);
        read_b(st, 1, bq[1]);
#pragma unroll
        for (int j = 0; j < NF; ++j) a_cur[j] = X64 ? unpack16_x64(cw[j][0]) : unpack16(cw[j][0]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            if (s + 2 < 8) read_b(st, s + 2, bq[(s + 2) % 3]);
            if (s + 1 < 8) {
#pragma unroll
                for (int j = 0; j < NF; ++j) a_nxt[j] = X64 ? unpack16_x64(cw[j][s + 1]) : unpack16(cw[j][s + 1]);
            }
#pragma unroll
            for (int i = 0; i < MF; ++i)
#pragma unroll
                for (int j = 0; j < NF; ++j)
                    acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_cur[j], bq[s % 3][i], acc[j][i], 0, 0, 0);
            if (s + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, MF, 0);  // the LDS reads first
#pragma unroll
            for (int k = 0; k < MF * NF; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (s + 1 < 8)
                    __builtin_amdgcn_sched_group_barrier(0x002, ((X64 ? 7 : 11) * NF + MF * NF - 1) / (MF * NF), 0);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NF; ++j) a_cur[j] = a_nxt[j];
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
    // ---- pipeline.  A ring of D VGPR sets: set g % D holds the codes (and,
    // until they are stored, the activations) of group g; the loads of
    // group g + D - 1 are issued while group g multiplies, so each group's
    // loads have D - 1 group times to land.  LDS slot g % 2 holds the
    // activations of group g.  Loads past the last group repeat it (uniform
    // load count, exact vmcnt bookkeeping).
    static_assert(D == 2 || D == 4, "ring depth");
    // This slice's full groups: g(j) = gb + ks + KS * j for j < J, the same J
    // in every slice so every wave meets the same barriers (a slice past the
    // last full group loads a repeat and skips the multiply).
    const int64_t J = (NGf + KS - 1) / KS;
    auto grp = [&](int64_t j) -> int64_t {
        const int64_t g = ks + (int64_t)KS * j;
        return gb + (g < NGl ? g : NGl - 1);
    };
    v4u rs[D][NR];
#pragma unroll
    for (int k = 0; k < D - 1; ++k) load(grp(k), rs[k]);
    store(0, rs[0]);
    lds_fence_barrier();
    // One step of the pipeline: prefetch step j + D - 1 into ring set
    // (k + D - 1) % D, multiply step j (ring set k, LDS slot k & 1), then
    // store step j + 1's activations into the other slot.  The main loop runs
    // whole ring cycles with no early exit (an exit inside the unrolled body
    // makes the compiler drain every load at the loop latch); the remaining
    // steps follow it.
    auto step = [&](int64_t j, auto kc) {
        constexpr int k = decltype(kc)::value;
        load(grp(j + D - 1), rs[(k + D - 1) % D]);
        // keeps the scheduler from sinking the prefetch below the MFMAs
        __builtin_amdgcn_sched_barrier(0);
        if (ks + (int64_t)KS * j < NGf) compute_full(k & 1, rs[k]);
        store((k + 1) & 1, rs[(k + 1) % D]);  // past the last step: a harmless repeat
        lds_fence_barrier();
    };
    const int64_t cycles = J / D;
    for (int64_t c = 0; c < cycles; ++c) {
        const int64_t j0 = c * D;
        step(j0, std::integral_constant<int, 0>{});
        step(j0 + 1, std::integral_constant<int, 1>{});
        if constexpr (D > 2) {
            step(j0 + 2, std::integral_constant<int, 2>{});
            step(j0 + 3, std::integral_constant<int, 3>{});
        }
    }
    const int64_t j0 = cycles * D;
    const int rem = (int)(J - j0);
    if (rem > 0) step(j0, std::integral_constant<int, 0>{});
    if constexpr (D > 2) {
        if (rem > 1) step(j0 + 1, std::integral_constant<int, 1>{});
        if (rem > 2) step(j0 + 2, std::integral_constant<int, 2>{});
    }
    // The partial last group (Gtail fragments) is step NGf / KS of slice
    // NGf % KS; its activations are in that step's LDS slot (the steps after
    // it stored repeats into the other slot).
    if (tail && ks == (int)(NGf % KS)) compute_tail((int)((NGf / KS) & 1), NGfull);

    // ---- K slices: slice 1 hands its accumulators to slice 0 through LDS,
    // over the stages once no wave reads them any more (the partial group's
    // multiply runs after the last step's barrier)
    if constexpr (KS > 1) {
        int32_t *red = reinterpret_cast<int32_t *>(lds_all) + wave * (MF * NF * 16 * 64) + lane;
        lds_fence_barrier();
        if (ks == 1) {
#pragma unroll
            for (int j = 0; j < NF; ++j)
#pragma unroll
                for (int i = 0; i < MF; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e) red[((j * MF + i) * 16 + e) * 64] = acc[j][i][e];
        }
        lds_fence_barrier();
        if (ks == 0) {
#pragma unroll
            for (int j = 0; j < NF; ++j)
#pragma unroll
                for (int i = 0; i < MF; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[j][i][e] += red[((j * MF + i) * 16 + e) * 64];
        }
    }

    if (X64) {
#pragma unroll
        for (int j = 0; j < NF; ++j)
#pragma unroll
            for (int i = 0; i < MF; ++i) acc[j][i] >>= 6;  // exact: every term is a multiple of 64
    }

    // ---- one run of several: the exact int32 sums of this run go to its
    // [M][N] slice of the workspace (4 consecutive n per store), to be added
    // up by splitk_reduce.  Fragment lane l holds m = l % 32 and
    // n = 8*(r/4) + 4*(l/32) + r%4 for its 16 values r.
    if (sg.part != nullptr) {
        if (ks != 0) return;  // slice 0 holds the sums
        int32_t *__restrict__ part = sg.part + (int64_t)run * M * N;
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
                    const v4i v = {acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2], acc[j][i][4 * q + 3]};
                    if (vec && nb + 3 < N) {
                        *reinterpret_cast<v4i *>(part + m * N + nb) = v;
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (nb + r < N) part[m * N + nb + r] = v[r];
                    }
                }
            }
        }
        return;
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
        // XOR key of a row's chunks: the low bits of the row, within the chunk
        // count (a power of two), or 4 bits when the count is a multiple of 16
        constexpr int SWZ = (CPR & (CPR - 1)) == 0 ? CPR - 1 : 15;
        static_assert((CPR & (CPR - 1)) == 0 || CPR % 16 == 0, "chunk swizzle stays in the row");
        lds_fence_barrier();              // every wave is done with the last stage
#pragma unroll
        for (int i = 0; i < MF; ++i) {
            if (ks != 0) break;           // slice 0 holds the sums
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
                    *reinterpret_cast<uint2 *>(lds_all + r * ROWB + ((c ^ (r & SWZ)) << 4) + 8 * lh) = o;
                }
            }
        }
        lds_fence_barrier();
        static_assert((C::BM * CPR) % C::NTT == 0, "epilogue passes");
#pragma unroll
        for (int q0 = 0; q0 < C::BM * CPR; q0 += C::NTT) {
            const int q = q0 + (int)threadIdx.x;
            const int r = q / CPR, c = q - r * CPR;
            const int64_t m = m0 + r, n = n0 + 8 * c;
            const v4u v = *reinterpret_cast<const v4u *>(lds_all + r * ROWB + ((c ^ (r & SWZ)) << 4));
            // non-temporal: the output is not read again by this launch, and
            // streaming it out keeps dirty lines from piling up in L2 for the
            // flush at the end of the kernel (measured: the 700M layer's four
            // launches 84.9 -> 76.6 us)
            if (m < M && n < N) __builtin_nontemporal_store(v, reinterpret_cast<v4u *>(y + m * N + n));
        }
        return;
    }
    if (ks != 0) return;  // slice 0 holds the sums (no barrier follows)
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

template <int WM, int WN, int MF, int NF, int KS, bool X64, int D = 2, int WPE = 2>
hipError_t launch_cfg(GemmSegs &segs, hipStream_t s) {
    using C = Cfg<WM, WN, MF, NF, KS>;
    int tiles = 0;
    for (int i = 0; i < segs.count; ++i) {
        GemmSeg &g = segs.s[i];
        g.tiles_m = (int)((g.M + C::BM - 1) / C::BM);
        g.tiles_n = (int)((g.N + C::BN - 1) / C::BN);
        g.tile_begin = tiles;
        tiles += g.splits * g.tiles_m * g.tiles_n;
    }
    segs.total_tiles = tiles;
    auto kern = gemm_pipe<WM, WN, MF, NF, KS, X64, D, WPE>;
    static_assert(C::LDS_BYTES <= 65536, "no LDS opt-in needed up to 64 KB");
    hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(C::NTT), C::LDS_BYTES, s, segs);
    return hipGetLastError();
}

// Workgroup shapes (WM, WN, MF, NF) of the three candidate tiles
#define GEMM_CFG_A 1, 4, 2, 2   /* 64 x 256, waves of 64 x 64 */
#define GEMM_CFG_B 2, 2, 2, 2   /* 128 x 128 */
#define GEMM_CFG_C 1, 2, 2, 2   /* 64 x 128 */
#define GEMM_CFG_D 1, 4, 2, 3   /* 64 x 384, waves of 64 x 96 */
#define GEMM_CFG_E 1, 4, 1, 3   /* 32 x 384, waves of 32 x 96 (with two K slices) */
#define GEMM_CFG_F 1, 4, 1, 2   /* 32 x 256, waves of 32 x 64 (decode, <= 32 tokens) */
#define GEMM_CFG_G 1, 4, 2, 1   /* 64 x 128, waves of 64 x 32 (decode, 33..64 tokens, two K slices) */

// ---- split K: the runs' int32 sums added up, then the epilogue
// y = bf16(acc * (gamma / s_m)), evaluated exactly as in gemm_pipe.
struct RedSeg {
    const int32_t *part;  // runs x [M][N]
    const float *gamma;
    const float *xs;
    uint16_t *y;
    int32_t *acc;
    int64_t M, N, NQ;     // NQ = ceil(N / 4): 4-column quads per row
    int64_t q_begin;      // first quad of this segment in the launch (a multiple of 256)
    int runs;
};
struct RedSegs {
    RedSeg s[kMaxSeg];
    int count;
};

__global__ __launch_bounds__(256) void splitk_reduce(RedSegs rs) {
    // segments start on workgroup boundaries, so the segment is the same for
    // the whole workgroup and its fields come through scalar loads
    const int64_t q0 = (int64_t)blockIdx.x * 256;
    const int64_t q = q0 + threadIdx.x;
    int sidx = 0;
#pragma unroll
    for (int i = 1; i < kMaxSeg; ++i)
        if (i < rs.count && q0 >= rs.s[i].q_begin) sidx = i;
    sidx = __builtin_amdgcn_readfirstlane(sidx);
    const RedSeg &sg = rs.s[sidx];
    const int64_t ql = q - sg.q_begin;
    const int64_t M = sg.M, N = sg.N;
    if (ql >= M * sg.NQ) return;
    const int64_t m = ql / sg.NQ, n = 4 * (ql - m * sg.NQ);
    const int64_t MN = M * N;
    const int32_t *p = sg.part + m * N + n;
    if ((N & 3) == 0) {
        // The runs' loads go out 8 at a time, with the token's scale, before
        // the first wait (a loop of one load per iteration waited out a
        // memory latency per run).  Loads past the last run repeat it, so no
        // branch separates the loads, and are not added.  int32 sums are
        // exact in any order.
        const int runs = sg.runs;
        auto load8 = [&](int r0, v4i(&v)[8]) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = r0 + u < runs ? r0 + u : runs - 1;
                v[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p + r * MN));
            }
        };
        auto sum8 = [&](int r0, const v4i(&v)[8]) __attribute__((always_inline)) {
            v4i t = v[0];
#pragma unroll
            for (int u = 1; u < 8; ++u) t += r0 + u < runs ? v[u] : v4i{0, 0, 0, 0};
            return t;
        };
        const float xsm = sg.xs[m];
        v4i v[8];
        load8(0, v);
        v4i a = sum8(0, v);
        for (int r0 = 8; r0 < runs; r0 += 8) {
            load8(r0, v);
            a += sum8(r0, v);
        }
        const float scale = sg.gamma[0] / xsm;
        const uint2 h = make_uint2(pack_bf16x2((float)a.x * scale, (float)a.y * scale),
                                   pack_bf16x2((float)a.z * scale, (float)a.w * scale));
        *reinterpret_cast<uint2 *>(sg.y + m * N + n) = h;
        if (sg.acc) *reinterpret_cast<v4i *>(sg.acc + m * N + n) = a;
        return;
    }
    const float scale = sg.gamma[0] / sg.xs[m];
    for (int e = 0; e < 4 && n + e < N; ++e) {
        int a = p[e];
        for (int r = 1; r < sg.runs; ++r) a += p[r * MN + e];
        sg.y[m * N + n + e] = (uint16_t)pack_bf16x2((float)a * scale, 0.0f);
        if (sg.acc) sg.acc[m * N + n + e] = a;
    }
}

struct Choice {
    int id;
    int bm, bn, waves;
};

}  // namespace

// Tile choice: pick the workgroup shape whose tiles waste the least of M x N
// to padding and of the 2048 wave slots (256 CUs x 4 SIMDs x 2 waves) in the
// last round of waves; earlier candidates (64 x 256, the fewest bytes loaded
// per MFMA) win ties.  The 64 x 384 tile (waves of 64 x 96) is chosen when
// 64 x 256 tiles would spill into a nearly empty second round.
bool gemm_ok(const Layout &L, int64_t M) {
    constexpr int64_t kBufMax = ((int64_t)1 << 31) - ((int64_t)1 << 20);
    return M >= 1 && L.K % 16 == 0 && M * L.K < kBufMax && L.bytes < kBufMax;
}

hipError_t launch_gemm_multi(const FwdSeg *fs, int count, hipStream_t s) {
    // candidates: (id, BM, BN, waves)
    static const Choice cands[] = {{0, 64, 256, 4}, {1, 128, 128, 4}, {2, 64, 128, 2}, {3, 64, 384, 4}};
    int best = 0;
    double best_eff = -1.0;
    int64_t tiles_a = 0;
    for (int i = 0; i < count; ++i) tiles_a += ((fs[i].M + 63) / 64) * ((fs[i].L.N + 255) / 256);
    for (const Choice &c : cands) {
        int64_t waves = 0;
        double useful = 0.0, padded = 0.0;
        for (int i = 0; i < count; ++i) {
            const int64_t tm = (fs[i].M + c.bm - 1) / c.bm, tn = (fs[i].L.N + c.bn - 1) / c.bn;
            waves += tm * tn * c.waves;
            useful += (double)fs[i].M * (double)fs[i].L.N;
            padded += (double)(tm * c.bm) * (double)(tn * c.bn);
        }
        const int64_t rounds = (waves + 2047) / 2048;
        const double eff = useful / padded * (double)waves / (double)(rounds * 2048);
        if (eff > best_eff + 1e-9) {
            best_eff = eff;
            best = c.id;
        }
    }
    GemmSegs segs{};
    int64_t max_k = 0;
    for (int i = 0; i < count; ++i) {
        GemmSeg &g = segs.s[i];
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
        g.part = nullptr;
        g.gps = L.NG;
        g.splits = 1;
        max_k = L.K > max_k ? L.K : max_k;
    }
    segs.count = count;
    const bool x64 = max_k <= kScaledMaxK;
    // Fewer 64 x 256 tiles than CUs: each CU would run a single 4-wave
    // workgroup (one wave per SIMD); split K over two 4-wave slices instead
    // so two waves share each SIMD.  If 32 x 384 tiles still fit one per CU,
    // they spread the same work over more CUs: 3 fragments per wave instead
    // of 4 on the busiest SIMD.  A launch whose rows are one group of 256
    // columns or less has nothing to split: it takes 32 x 256 tiles of one
    // slice (the 16.4M model's O projection, 8192 x 256 x 256: 5.8 -> 4.5 us;
    // the same tiles for every one-group launch were slower on the others).
    // Where 384-column tiles would pad a 256-multiple N (the 16.4M model's
    // down projection, 8192 x 256 x 512), 32 x 256 tiles with two K slices
    // cover it exactly: 6.2 -> 5.5 us.
    int64_t min_ng = INT64_MAX;
    for (int i = 0; i < count; ++i) min_ng = fs[i].L.NG < min_ng ? fs[i].L.NG : min_ng;
    if (best == 0 && tiles_a <= 256 && min_ng < 2)
        return x64 ? launch_cfg<GEMM_CFG_F, 1, true>(segs, s) : launch_cfg<GEMM_CFG_F, 1, false>(segs, s);
    if (best == 0 && tiles_a <= 256) {
        int64_t tiles_e = 0;
        for (int i = 0; i < count; ++i) tiles_e += ((fs[i].M + 31) / 32) * ((fs[i].L.N + 383) / 384);
        bool pad384 = false;
        int64_t tiles_f = 0;
        for (int i = 0; i < count; ++i) {
            pad384 = pad384 || (fs[i].L.N % 384 != 0 && fs[i].L.N % 256 == 0);
            tiles_f += ((fs[i].M + 31) / 32) * ((fs[i].L.N + 255) / 256);
        }
        if (tiles_e <= 256 && pad384 && tiles_f <= 256)
            return x64 ? launch_cfg<GEMM_CFG_F, 2, true>(segs, s) : launch_cfg<GEMM_CFG_F, 2, false>(segs, s);
        if (tiles_e <= 256)
            return x64 ? launch_cfg<GEMM_CFG_E, 2, true>(segs, s) : launch_cfg<GEMM_CFG_E, 2, false>(segs, s);
        return x64 ? launch_cfg<GEMM_CFG_A, 2, true>(segs, s) : launch_cfg<GEMM_CFG_A, 2, false>(segs, s);
    }
    switch (best) {
        case 0: return x64 ? launch_cfg<GEMM_CFG_A, 1, true>(segs, s) : launch_cfg<GEMM_CFG_A, 1, false>(segs, s);
        case 1: return x64 ? launch_cfg<GEMM_CFG_B, 1, true>(segs, s) : launch_cfg<GEMM_CFG_B, 1, false>(segs, s);
        case 3: return x64 ? launch_cfg<GEMM_CFG_D, 1, true>(segs, s) : launch_cfg<GEMM_CFG_D, 1, false>(segs, s);
        default: return x64 ? launch_cfg<GEMM_CFG_C, 1, true>(segs, s) : launch_cfg<GEMM_CFG_C, 1, false>(segs, s);
    }
}

// ---- decode batches of 14..64 tokens.  Such a launch has few output tiles
// (the 70B down projection at 64 tokens: 64 tiles of 64 x 128), and a
// workgroup that owns a tile for the whole K streams every token column
// through its CU.  Two remedies, chosen by measurement on the 70B and 3B
// layers (the workspace-free decode kernel stays where neither pays):
//  * 33..64 tokens: 64 x 128 tiles, 4 waves (one fragment column each) in
//    each of two K slices: 8 waves per workgroup, sized for 4 per SIMD (124
//    VGPRs; against one slice, 70B at 64 tokens: gate+up 46.3 -> 44.0 us,
//    down 28.3 -> 26.3 us, QKV and O unchanged).  With >= kSmallTarget tiles
//    the launch needs nothing more (the 70B gate+up launch: 448 tiles); with
//    fewer, K is cut into runs so that tiles x runs ~ kSmallTarget, each
//    run's int32 sums go to the workspace and splitk_reduce adds them (70B
//    down 44 -> 27 us, O 17 -> 16; half or twice as many runs were slower).
//    A launch with no runs whose 64 x 256 tiles number kWideMin..256 takes
//    those instead, with two K slices (the prefill few-tile configuration).
//  * 14..32 tokens: 32 x 256 tiles with two K slices, cut into runs the same
//    way, but only for rows of >= kSmallLongGroups groups of 256 columns (the
//    70B down projection, 27 -> 19 us at 32 tokens, 19.0 -> 18.1 us at 14);
//    shorter rows, and fewer tokens, run faster on the decode kernels (at 12
//    tokens: 17.7 us there, 18.2 us cut into runs).
// Every run is at least kSplitMinGroups groups long.
namespace {
constexpr int64_t kWideMin = 193;  // 64 x 256 tiles: three quarters of the CUs and more
struct SmallPlan {
    int cfg;  // 0: not for this path, 1: 32 x 256, 2: 64 x 128 (both with two K slices;
              // a cfg 2 launch with no runs may take 64 x 256 tiles, see kWideMin)
    int64_t runs[kMaxSeg], gps[kMaxSeg];
    size_t off[kMaxSeg];
    size_t bytes;  // workspace for the runs' partial sums (0: no entry is cut)
};

void small_plan(const FwdSeg *fs, int count, SmallPlan &p) {
    p.cfg = 0;
    p.bytes = 0;
    int64_t max_m = 0, min_ng = INT64_MAX;
    for (int i = 0; i < count; ++i) {
        max_m = fs[i].M > max_m ? fs[i].M : max_m;
        min_ng = fs[i].L.NG < min_ng ? fs[i].L.NG : min_ng;
    }
    if (max_m < kSplitMinM || max_m > kGemvMaxM) return;
    const int bm = max_m <= 32 ? 32 : 64, bn = max_m <= 32 ? 256 : 128;
    int64_t tiles = 0;
    for (int i = 0; i < count; ++i) tiles += ((fs[i].M + bm - 1) / bm) * ((fs[i].L.N + bn - 1) / bn);
    const int64_t S = kSmallTarget / tiles;
    if (bm == 32 && (S < 2 || min_ng < kSmallLongGroups)) return;
    p.cfg = bm == 32 ? 1 : 2;
    for (int i = 0; i < count; ++i) {
        const int64_t NG = fs[i].L.NG;
        const int64_t cap = NG / kSplitMinGroups > 1 ? NG / kSplitMinGroups : 1;
        const int64_t si = S < 1 ? 1 : (S < cap ? S : cap);
        p.gps[i] = (NG + si - 1) / si;
        p.runs[i] = (NG + p.gps[i] - 1) / p.gps[i];
        p.off[i] = p.bytes;
        if (p.runs[i] > 1)
            p.bytes += ((size_t)p.runs[i] * (size_t)fs[i].M * (size_t)fs[i].L.N * 4 + 255) & ~(size_t)255;
    }
}
}  // namespace

// ---- the fixed scratch of bitlinear_forward_grouped_noalloc: the runs'
// int32 partial sums of a cut launch, for callers that cannot allocate.  One
// copy per device, held until the process ends; every no-allocation call on a
// device shares it (calls that overlap on one device race).  Host code never
// uses the array's name as an address: scratch_ptr() looks up each device's
// copy once, with that device current, and the kernels receive that pointer.
static_assert(kSmallMaxBytes <= BITLINEAR_SCRATCH_BYTES, "the scratch holds any plan's partial sums");
static __device__ __align__(256) uint8_t scratch[BITLINEAR_SCRATCH_BYTES];

hipError_t scratch_ptr(void **out) {
    static std::atomic<void *> per_device[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void *p = per_device[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        per_device[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

size_t gemm_small_bytes(const FwdSeg *fs, int count) {
    SmallPlan p;
    small_plan(fs, count, p);
    return p.bytes;
}

bool gemm_small_ok(const FwdSeg *fs, int count, bool have_workspace) {
    SmallPlan p;
    small_plan(fs, count, p);
    return p.cfg != 0 && (p.bytes == 0 || have_workspace);
}

hipError_t launch_gemm_small(const FwdSeg *fs, int count, void *workspace, hipStream_t s) {
    SmallPlan p;
    small_plan(fs, count, p);
    if (p.cfg == 0 || (p.bytes > 0 && workspace == nullptr)) return hipErrorInvalidValue;
    GemmSegs segs{};
    RedSegs rs{};
    int64_t max_k = 0, quads = 0;
    for (int i = 0; i < count; ++i) {
        GemmSeg &g = segs.s[i];
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
        g.gps = p.gps[i];
        g.splits = (int)p.runs[i];
        g.part = p.runs[i] > 1 ? reinterpret_cast<int32_t *>(static_cast<uint8_t *>(workspace) + p.off[i]) : nullptr;
        max_k = L.K > max_k ? L.K : max_k;
        if (g.part) {
            RedSeg &r = rs.s[rs.count++];
            r.part = g.part;
            r.gamma = g.gamma;
            r.xs = g.xs;
            r.y = g.y;
            r.acc = g.acc;
            r.M = g.M;
            r.N = g.N;
            r.NQ = (g.N + 3) / 4;
            r.q_begin = quads;
            r.runs = g.splits;
            quads += (r.M * r.NQ + 255) / 256 * 256;  // whole workgroups per segment
        }
    }
    segs.count = count;
    const bool x64 = max_k <= kScaledMaxK;
    // 33..64 tokens, no K runs: a launch whose 64 x 256 tiles number
    // kWideMin..256 takes them with two K slices, one 8-wave workgroup per
    // CU (each wave 64 x 64: half the B-operand LDS reads per MFMA of the
    // 64 x 128 tile's 64 x 32 waves).  The 70B gate+up launch at 64 tokens,
    // 448 -> 224 workgroups: 70B step 123.5 -> 119.3 us; a single 70B gate
    // projection (112 such tiles) was slower on them, 21.7 -> 28.0 us.
    if (p.cfg == 2 && p.bytes == 0) {
        int64_t ta = 0;
        for (int i = 0; i < count; ++i) ta += ((fs[i].M + 63) / 64) * ((fs[i].L.N + 255) / 256);
        if (ta >= kWideMin && ta <= 256)
            return x64 ? launch_cfg<GEMM_CFG_A, 2, true>(segs, s) : launch_cfg<GEMM_CFG_A, 2, false>(segs, s);
    }
    hipError_t e = p.cfg == 1 ? (x64 ? launch_cfg<GEMM_CFG_F, 2, true>(segs, s) : launch_cfg<GEMM_CFG_F, 2, false>(segs, s))
                              : (x64 ? launch_cfg<GEMM_CFG_G, 2, true, 2, 4>(segs, s) : launch_cfg<GEMM_CFG_G, 2, false, 2, 4>(segs, s));
    if (e != hipSuccess || rs.count == 0) return e;
    hipLaunchKernelGGL(splitk_reduce, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s, rs);
    return hipGetLastError();
}

hipError_t launch_gemm_pipe(const uint32_t *packed, const float *gamma, const Layout &L,
                            const int8_t *xq, const float *xs, int64_t M, uint16_t *y,
                            int32_t *acc, hipStream_t s) {
    FwdSeg f{packed, gamma, L, xq, xs, M, y, acc};
    return launch_gemm_multi(&f, 1, s);
}

}  // namespace bl
