// STE backward to the layer input on gfx950 ("1-bit & Ternary LLMs (BitNet
// b1.58)", Training: the forward runs on the ternary weights, the
// straight-through estimator treats both quantisers as identities, so the
// gradient of y = x (gamma W~)^T with respect to x is dx = dy (gamma W~)).
//
//   dx[m][k] = bf16(gamma * sum_n dy[m][n] * code[n][k]  (+ dx[m][k]))
//
// The contraction runs over the output features n, the dimension along which
// layout v1 does not keep a lane's codes together, so the codes are first
// rearranged into layout t1 (v1's geometry over the transposed K x N code
// matrix, with an in-dword order made for bf16 operands).
//
// Design of dgrad_pipe (one workgroup of WM x WN waves per BM x BN tile of dx):
//  * MFMA v_mfma_f32_32x32x16_bf16: A = dy (rows m) from LDS, B = codes
//    (columns k) unpacked in registers; each wave owns MF x NF fragments of
//    32 x 32 fp32 accumulators.
//  * Codes to bf16 at 15 VALU per 16 codes: layout t1 puts columns 2p, 2p+1
//    of a dword at bits 14-2p and 30-2p, so (w << 2p) & 0xC000C000 is the
//    bf16 pair (2 c_2p, 2 c_2p+1): the 2-bit two's complement code becomes
//    the sign and the exponent LSB of +-2.0 (0x4000 / 0xC000).  Products with
//    +-2 are exact, so the accumulators hold 2 * sum exactly as far as fp32
//    sums go, and the epilogue multiplies by gamma / 2 (exact halving).
//  * The contraction runs over groups of 256 n: the group's dy tile (BM x 512
//    B) and each wave's code dwords are loaded global -> VGPRs through
//    bounds-checked buffer descriptors one group ahead; dy then goes to one
//    of two LDS slots (one barrier per group).  A lane's 16-byte code load
//    brings its dwords of the group's four fragments, exactly as the forward
//    kernel reads layout v1.
//  * dy rows in LDS are 512 B with the 16-byte chunk index XOR-ed by
//    (row & 31), so the operand loads of 32 rows x one chunk spread over the
//    banks.
//  * Tiles are handed out XCD by XCD in m-major runs so one XCD's L2 keeps
//    the dy rows its tiles share.
// Requires N % 8 == 0 (16-byte dy rows) and dy and the codes below 2 GB.
#include <atomic>
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace bl {

namespace {

// Kernels whose LDS exceeds 64 KB are opted into once per device (the
// attribute is per kernel and per device).  The template argument is the
// kernel itself, so every instantiation keeps its own bits: one per device,
// set once the opt-in succeeded.  Two threads racing the first launch both
// make the (idempotent) call; devices past 63 make it on every launch.
template <auto Kern>
hipError_t lds_optin(int bytes) {
    static std::atomic<uint64_t> done{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- v1 -> t1
// One workgroup per 64 rows (four 16-row blocks) of the N x K code matrix and
// one 64-column fragment: decode the 64 x 64 codes into LDS as bytes, then
// write them back as the 64 x 64 block of the transposed matrix.  Reads and
// writes 0.25 B per weight.
__device__ __forceinline__ void t1_block(const uint32_t *__restrict__ in, uint32_t *__restrict__ out, int64_t NB,
                                         int64_t KF, int64_t KBo, int64_t KFo, int64_t b, int64_t f) {
    __shared__ uint8_t tile[64][68];  // [k][n] inside the block
    const int i = threadIdx.x;
    const int rbl = i >> 6, lam = i & 63;
    // b: 64-row block of n = fragment b of the transposed matrix;
    // f: 64-column fragment of k = row blocks 4f..4f+3 of the transposed matrix
    {
        const int64_t rb = 4 * b + rbl;
        uint32_t w = 0;
        if (rb < NB) {
            const int64_t g = f >> 2;
            const int64_t G = KF - 4 * g < 4 ? KF - 4 * g : 4;
            w = in[rb * KF * 64 + g * 256 + lam * G + (f & 3)];
        }
        const int nl = 16 * rbl + (lam & 15);
        const int kl0 = 16 * (lam >> 4);
#pragma unroll
        for (int t = 0; t < 16; ++t) tile[kl0 + t][nl] = (uint8_t)((w >> (8 * (t & 3) + 2 * (t >> 2))) & 3u);
    }
    __syncthreads();
    const int64_t rbo = 4 * f + rbl;
    if (rbo >= KBo) return;
    const int kl = 16 * rbl + (lam & 15);
    const int nl0 = 16 * (lam >> 4);
    uint32_t w = 0;
#pragma unroll
    for (int t = 0; t < 16; ++t) w |= (uint32_t)tile[kl][nl0 + t] << ((t & 1) ? 31 - t : 14 - t);
    const int64_t g = b >> 2;
    const int64_t G = KFo - 4 * g < 4 ? KFo - 4 * g : 4;
    out[rbo * KFo * 64 + g * 256 + lam * G + (b & 3)] = w;
}

__global__ __launch_bounds__(256) void codes_to_t1(const uint32_t *__restrict__ in, uint32_t *__restrict__ out,
                                                   int64_t NB, int64_t KF, int64_t KBo, int64_t KFo) {
    t1_block(in, out, NB, KF, KBo, KFo, blockIdx.x, blockIdx.y);
}

// the same for the tensors of a grouped pack that asked for layout t1
__global__ __launch_bounds__(256) void codes_to_t1_grouped(PackSegs ps) {
    const int64_t w = blockIdx.x;
    int sidx = 0;
#pragma unroll
    for (int i = 1; i < kPackGroup; ++i)
        if (i < ps.count && w >= ps.s[i].t1_begin) sidx = i;
    const PackSeg &sg = ps.s[sidx];
    const int64_t NB = (sg.N + 15) / 16, KF = (sg.K + 63) / 64;     // layout v1 of N x K
    const int64_t KBo = (sg.K + 15) / 16, KFo = (sg.N + 63) / 64;   // layout t1 (v1 of K x N)
    const int64_t local = w - sg.t1_begin;
    t1_block(sg.packed, sg.packed_t, NB, KF, KBo, KFo, local / KF, local % KF);
}

// ------------------------------------------------------------------ dgrad

// WM x WN waves per slice own MF x NF fragments each; KS slices split the
// contraction groups between them (slice k takes groups k, k + KS, ...) and
// add their accumulators through LDS at the end.
template <int WM, int WN, int MF, int NF, int KS>
struct DgCfg {
    static constexpr int W = WM * WN;       // waves per slice
    static constexpr int NT = W * 64;       // threads per slice
    static constexpr int NTT = NT * KS;     // threads per workgroup
    static constexpr int BM = WM * MF * 32;
    static constexpr int BN = WN * NF * 32;
    static constexpr int ROW = 512;  // bytes of one dy row per group (256 bf16)
    static constexpr int STAGE = BM * ROW;
    static constexpr int DY_LOADS = STAGE / 16 / NT;
    static constexpr int CODE_LOADS = 2 * NF;
    static constexpr int NR = DY_LOADS + CODE_LOADS;
    static constexpr int SLICE_BYTES = 2 * STAGE;
    static constexpr int LDS_BYTES = KS * SLICE_BYTES;
    static_assert(STAGE % (16 * NT) == 0, "dy loads must split evenly");
    static_assert(KS == 1 || KS == 2, "K slices");
    static_assert(BM * BN * 4 <= LDS_BYTES, "one slice's accumulators and the fp32 tile fit");
};

__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14));  // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// B operand of MFMA u (0: columns 0..7 of the dword's 16, 1: columns 8..15)
__device__ __forceinline__ v8bf codes_bf16(uint32_t w, int u) {
    const uint32_t M2 = 0xC000C000u;
    v4u r;
    if (u == 0) {
        r.x = w & M2;
        r.y = (w << 2) & M2;
        r.z = (w << 4) & M2;
        r.w = (w << 6) & M2;
    } else {
        r.x = (w << 8) & M2;
        r.y = (w << 10) & M2;
        r.z = (w << 12) & M2;
        r.w = (w << 14) & M2;
    }
    return __builtin_bit_cast(v8bf, r);
}

template <int WM, int WN, int MF, int NF, int KS>
__global__ __launch_bounds__(WM *WN * 64 * KS) __attribute__((amdgpu_waves_per_eu(2, 2))) void dgrad_pipe(DgradArgs a) {
    using C = DgCfg<WM, WN, MF, NF, KS>;
    constexpr int NR = C::NR;
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds_all[];

    const int lane = threadIdx.x & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = wave_all / C::W;                 // contraction slice of this wave
    const int wave = wave_all - ks * C::W;          // wave within the slice
    const int tid = (int)threadIdx.x - ks * C::NT;  // thread within the slice
    uint8_t *lds = lds_all + ks * C::SLICE_BYTES;   // this slice's two stages
    const int wm = wave / WN, wn = wave % WN;
    const int lr = lane & 31, lh = lane >> 5;

    const int T = a.tiles_m * a.tiles_n;
    int t = blockIdx.x;
    if ((T & 7) == 0) t = (blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3);
    const int tm = t / a.tiles_n, tn = t - tm * a.tiles_n;
    const int64_t m0 = (int64_t)tm * C::BM;
    const int64_t k0 = (int64_t)tn * C::BN;
    const int64_t M = a.M, N = a.N, K = a.K, KB = a.KB, KFt = a.KFt;
    const uint16_t *__restrict__ dy = a.dy;
    const uint32_t *__restrict__ packed = a.packed_t;

    const int64_t NGfull = KFt / 4;
    const int Gtail = (int)(KFt - 4 * NGfull);
    const int64_t NG = NGfull + (Gtail ? 1 : 0);

    // ---- per-lane load offsets (loop invariant; the group offset goes into
    // the descriptor).  Reads past either buffer return zeros: rows past M
    // and row blocks past K.  Bytes past N inside a row belong to the next
    // row and only ever meet zero codes.
    const uint32_t dy_bytes = (uint32_t)(M * N * 2);
    const uint32_t code_bytes = (uint32_t)(KB * KFt * 256);
    uint32_t dy_off[C::DY_LOADS];
    int dy_dst[C::DY_LOADS];
#pragma unroll
    for (int i = 0; i < C::DY_LOADS; ++i) {
        const int q = tid + C::NT * i;  // 16-byte chunk of the tile
        const int r = q >> 5, c = q & 31;
        const int64_t m = m0 + r;
        dy_off[i] = m < M ? (uint32_t)(m * N * 2 + 16 * c) : dy_bytes;
        dy_dst[i] = r * C::ROW + ((c ^ (r & 31)) << 4);
    }
    // fragment j (columns 32*(wn*NF + j) + lr of the tile): the lane's dwords
    // sit at lane positions lam and lam + 32 of row block 2*(wn*NF+j) + lr/16,
    // lam = lr % 16 + 16 * lh
    const int clam = (lr & 15) + 16 * lh;
    uint32_t code_off[C::CODE_LOADS];
    uint32_t code_blk[NF];  // start of the lane's row block, code_bytes past the last
#pragma unroll
    for (int j = 0; j < NF; ++j) {
        const int64_t rb = k0 / 16 + 2 * (wn * NF + j) + (lr >> 4);
        code_blk[j] = rb < KB ? (uint32_t)(rb * KFt * 256) : code_bytes;
        const uint32_t base = rb < KB ? code_blk[j] + 16u * (uint32_t)clam : code_bytes;
        code_off[2 * j] = base;
        code_off[2 * j + 1] = base + 512;
    }
    const float ghalf = a.gamma[0] * 0.5f;  // codes enter the MFMA as +-2

    auto load = [&](int64_t g, v4u(&r)[NR]) {
        const __amdgpu_buffer_rsrc_t dg = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(dy + g * 256), 0, (int)(dy_bytes - (uint32_t)(g * 512)), 0x00020000);
        const __amdgpu_buffer_rsrc_t cg = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(packed + g * 256), 0, (int)(code_bytes - (uint32_t)(g * 1024)), 0x00020000);
#pragma unroll
        for (int i = 0; i < C::DY_LOADS; ++i)
            r[i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(dg, dy_off[i], 0, 0));
#pragma unroll
        for (int i = 0; i < C::CODE_LOADS; ++i)
            r[C::DY_LOADS + i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(cg, code_off[i], 0, 0));
    };
    auto store = [&](int stage, const v4u(&r)[NR]) {
        uint8_t *st = lds + stage * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::DY_LOADS; ++i) *reinterpret_cast<v4u *>(st + dy_dst[i]) = r[i];
    };

    v16f acc[MF][NF];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) acc[i][j] = v16f{};

    // A operand of step s, MFMA u, fragment i: row (wm*MF + i)*32 + lr, chunk
    // 4s + 2*lh + u (n = 32s + 16*lh + 8u .. +7), swizzled by lr
    const uint8_t *arow = lds + (wm * MF * 32 + lr) * C::ROW;
    auto read_a = [&](const uint8_t *st, int s, v8bf(&x)[MF][2]) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int ch = ((4 * s + 2 * lh + u) ^ lr) << 4;
#pragma unroll
            for (int i = 0; i < MF; ++i) x[i][u] = *reinterpret_cast<const v8bf *>(st + (arow - lds) + i * 32 * C::ROW + ch);
        }
    };
    auto mma = [&](const v8bf(&x)[MF][2], const uint32_t(&w)[NF]) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            v8bf bq[NF];
#pragma unroll
            for (int j = 0; j < NF; ++j) bq[j] = codes_bf16(w[j], u);
#pragma unroll
            for (int i = 0; i < MF; ++i)
#pragma unroll
                for (int j = 0; j < NF; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[i][u], bq[j], acc[i][j], 0, 0, 0);
        }
    };
    // a full group: the code dword of step s = 2f + e is dword f of the load at lam + 32e
    auto compute_full = [&](int stage, const v4u(&r)[NR]) {
        const uint8_t *st = lds + stage * C::STAGE;
        v8bf xa[2][MF][2];
        read_a(st, 0, xa[0]);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            if (s + 1 < 8) read_a(st, s + 1, xa[(s + 1) & 1]);
            uint32_t w[NF];
#pragma unroll
            for (int j = 0; j < NF; ++j) w[j] = r[C::DY_LOADS + 2 * j + (s & 1)][s >> 1];
            mma(xa[s & 1], w);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // the partial last group of Gtail fragments: dword lam of fragment f at
    // lam*Gtail + f; reloaded per dword (at most one group per tile)
    auto compute_tail = [&](int stage, int64_t g) {
        const uint8_t *st = lds + stage * C::STAGE;
        const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc((void *)packed, 0, (int)code_bytes,
                                                                             0x00020000);
        for (int s = 0; s < 2 * Gtail; ++s) {
            const int f = s >> 1, e = s & 1;
            uint32_t w[NF];
#pragma unroll
            for (int j = 0; j < NF; ++j)
                w[j] = code_blk[j] >= code_bytes
                           ? 0u
                           : __builtin_amdgcn_raw_buffer_load_b32(
                                 crs, code_blk[j] + (uint32_t)(g * 1024) + 4u * (uint32_t)((clam + 32 * e) * Gtail + f), 0, 0);
            v8bf x[MF][2];
            read_a(st, s, x);
            mma(x, w);
        }
    };

    // ---- pipeline: ring of two VGPR sets, LDS slot j & 1 of the slice holds
    // the dy of its step j, group ks + KS*j.  Every slice runs the same J
    // steps so all waves meet the same barriers; a step past the slice's
    // last full group loads a repeat and multiplies nothing.
    const int64_t J = (NGfull + KS - 1) / KS;
    auto grp = [&](int64_t j) -> int64_t {
        const int64_t g = ks + (int64_t)KS * j;
        return g < NG ? g : NG - 1;
    };
    v4u rs[2][NR];
    load(grp(0), rs[0]);
    store(0, rs[0]);
    lds_barrier();
    auto step = [&](int64_t j, auto kc) {
        constexpr int k = decltype(kc)::value;
        load(grp(j + 1), rs[k ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
        if (ks + (int64_t)KS * j < NGfull) compute_full(k, rs[k]);
        store(k ^ 1, rs[k ^ 1]);  // past the last full group: the tail group, or a harmless repeat
        lds_barrier();
    };
    const int64_t pairs = J / 2;
    for (int64_t c = 0; c < pairs; ++c) {
        step(2 * c, std::integral_constant<int, 0>{});
        step(2 * c + 1, std::integral_constant<int, 1>{});
    }
    if (J & 1) step(J - 1, std::integral_constant<int, 0>{});
    // the partial last group is step NGfull / KS of slice NGfull % KS; the
    // steps after it stored repeats of it into the other slot
    if (Gtail && ks == (int)(NGfull % KS)) compute_tail((int)((NGfull / KS) & 1), NGfull);

    // ---- K slices: slice 1 hands its accumulators to slice 0 through LDS
    if constexpr (KS > 1) {
        float *red = reinterpret_cast<float *>(lds_all) + wave * (MF * NF * 16 * 64) + lane;
        lds_barrier();  // every wave is done with the stages
        if (ks == 1) {
#pragma unroll
            for (int i = 0; i < MF; ++i)
#pragma unroll
                for (int j = 0; j < NF; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) red[((i * NF + j) * 16 + e) * 64] = acc[i][j][e];
        }
        lds_barrier();
        if (ks == 0) {
#pragma unroll
            for (int i = 0; i < MF; ++i)
#pragma unroll
                for (int j = 0; j < NF; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[i][j][e] += red[((i * NF + j) * 16 + e) * 64];
        }
    }

    // ---- epilogue.  Lane l of fragment (i, j) holds row 8*(r/4) + 4*lh + r%4
    // and column lr of its 16 values r.
    uint16_t *__restrict__ dx = a.dx;
    if ((K & 7) == 0) {
        // Slice 0 stages the scaled fp32 tile in LDS (over the stages), then
        // each thread of the workgroup finishes 8 contiguous columns of a
        // row: one 16-byte read of dx when accumulating, one 16-byte write.
        float *tile = reinterpret_cast<float *>(lds_all);
        lds_barrier();  // every wave is done with the stages (and the slice sums)
        if (ks == 0) {
#pragma unroll
            for (int i = 0; i < MF; ++i)
#pragma unroll
                for (int j = 0; j < NF; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = (wm * MF + i) * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                        tile[row * C::BN + (wn * NF + j) * 32 + lr] = acc[i][j][r] * ghalf;
                    }
        }
        lds_barrier();
        constexpr int CPR = C::BN / 8;  // 8-column chunks per tile row
        for (int q = threadIdx.x; q < C::BM * CPR; q += C::NTT) {
            const int row = q / CPR, c8 = q - row * CPR;
            const int64_t m = m0 + row, k = k0 + 8 * c8;
            if (m >= M || k >= K) continue;  // K % 8 == 0: a chunk is all in or all out
            const v4u lo = *reinterpret_cast<const v4u *>(tile + row * C::BN + 8 * c8);
            const v4u hi = *reinterpret_cast<const v4u *>(tile + row * C::BN + 8 * c8 + 4);
            float v[8] = {__uint_as_float(lo.x), __uint_as_float(lo.y), __uint_as_float(lo.z), __uint_as_float(lo.w),
                          __uint_as_float(hi.x), __uint_as_float(hi.y), __uint_as_float(hi.z), __uint_as_float(hi.w)};
            v4u *dst = reinterpret_cast<v4u *>(dx + m * K + k);
            if (a.accumulate) {
                const v4u p = *dst;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[2 * e] += __uint_as_float(p[e] << 16);
                    v[2 * e + 1] += __uint_as_float(p[e] & 0xFFFF0000u);
                }
            }
            __builtin_nontemporal_store(v4u{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                            pack_bf16x2(v[6], v[7])},
                                        dst);
        }
        return;
    }
    if (ks != 0) return;  // slice 0 holds the sums (no barrier follows)
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) {
            const int64_t k = k0 + (wn * NF + j) * 32 + lr;
            if (k >= K) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + (wm * MF + i) * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (m >= M) continue;
                float v = acc[i][j][r] * ghalf;
                if (a.accumulate) v += bf16_to_f32(dx[m * K + k]);
                dx[m * K + k] = f32_to_bf16(v);
            }
        }
}

// ------------------------------------------------- several entries, one dx
// The straight-through input gradient ("1-bit & Ternary LLMs (BitNet
// b1.58)", Training) of the layers that read one input (Q, K and V, or gate
// and up), summed in one launch.  Each tile runs the contraction groups of
// every entry in turn (a partial last group's codes gathered into the places
// of a full group's, zeros past its fragments) and, at the end of an entry,
// folds the entry's fp32 sum into a running total rounded to bf16 exactly as
// a separate call with accumulate rounds its dx: total = bf16(acc * gamma/2
// + total).  With two K slices, each entry's groups are dealt to the slices
// in turn (an entry's steps padded to whole pairs); at the end of an entry
// slice 1 hands its sums to slice 0 through the LDS slots that the step just
// consumed.  Slice 0 keeps the total in LDS past the stages (bf16 pairs),
// which leaves the registers to the accumulators and the load ring.
template <int WM, int WN, int MF, int NF, int KS>
__global__ __launch_bounds__(WM *WN * 64 * KS) __attribute__((amdgpu_waves_per_eu(2, 2))) void dgrad_grouped(
    DgradGroupArgs a) {
    using C = DgCfg<WM, WN, MF, NF, KS>;
    constexpr int NR = C::NR;
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds_all[];

    const int lane = threadIdx.x & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = wave_all / C::W;                 // contraction slice of this wave
    const int wave = wave_all - ks * C::W;          // wave within the slice
    const int tid = (int)threadIdx.x - ks * C::NT;  // thread within the slice
    uint8_t *lds = lds_all + ks * C::SLICE_BYTES;   // this slice's two stages
    const int wm = wave / WN, wn = wave % WN;
    const int lr = lane & 31, lh = lane >> 5;

    const int T = a.tiles_m * a.tiles_n;
    int t = blockIdx.x;
    if ((T & 7) == 0) t = (blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3);
    const int tm = t / a.tiles_n, tn = t - tm * a.tiles_n;
    const int64_t m0 = (int64_t)tm * C::BM;
    const int64_t k0 = (int64_t)tn * C::BN;
    const int64_t M = a.M, K = a.K;

    // per-lane geometry that does not depend on the entry: 16-byte dy chunk
    // tid + NT*i of the stage is row r0 + RSTEP*i, chunk c0 of the row
    constexpr int RSTEP = C::NT / 32;
    const int r0 = tid >> 5, c0 = tid & 31;
    const int rows_left = (int)min(M - m0, (int64_t)C::BM);
    const int clam = (lr & 15) + 16 * lh;
    int rbj[NF];  // the lane's 16-row block of the layout t1 codes
#pragma unroll
    for (int j = 0; j < NF; ++j) rbj[j] = (int)(k0 / 16) + 2 * (wn * NF + j) + (lr >> 4);

    // the entry of a step, and its fields, read with constant indices only:
    // indexing the argument array with a computed index would copy the whole
    // argument to private memory
    static_assert(kDgradMaxEntries == 4, "the selections below list four entries");
    auto entry_of = [&](int step) __attribute__((always_inline)) -> int {
        return (a.count > 3 && step >= a.e[3].step_begin)   ? 3
               : (a.count > 2 && step >= a.e[2].step_begin) ? 2
               : (a.count > 1 && step >= a.e[1].step_begin) ? 1
                                                            : 0;
    };
    auto pick = [&](int e, auto f) __attribute__((always_inline)) {
        return e == 0 ? f(a.e[0]) : e == 1 ? f(a.e[1]) : e == 2 ? f(a.e[2]) : f(a.e[3]);
    };
    auto entry = [&](int e) __attribute__((always_inline)) -> DgradEntry {
        DgradEntry r;
        r.packed_t = pick(e, [](const DgradEntry &x) { return x.packed_t; });
        r.gamma = pick(e, [](const DgradEntry &x) { return x.gamma; });
        r.dy = pick(e, [](const DgradEntry &x) { return x.dy; });
        r.N = pick(e, [](const DgradEntry &x) { return x.N; });
        r.KB = pick(e, [](const DgradEntry &x) { return x.KB; });
        r.KFt = pick(e, [](const DgradEntry &x) { return x.KFt; });
        r.groups = pick(e, [](const DgradEntry &x) { return x.groups; });
        r.step_begin = pick(e, [](const DgradEntry &x) { return x.step_begin; });
        return r;
    };
    // step j of this slice: contraction group (j - step_begin) * KS + ks of
    // its entry, past the entry's last group on padding steps
    auto group_of = [&](const DgradEntry &en, int j) __attribute__((always_inline)) -> int {
        return (j - en.step_begin) * KS + ks;
    };

    // group g of entry en into a register set (reads past either buffer
    // return zeros, as in dgrad_pipe)
    auto load = [&](int j, v4u(&r)[NR]) __attribute__((always_inline)) {
        const DgradEntry en = entry(entry_of(j));
        const int64_t g = min(group_of(en, j), en.groups - 1);  // padding: a harmless repeat
        const uint32_t dy_bytes = (uint32_t)(M * en.N * 2), code_bytes = (uint32_t)(en.KB * en.KFt * 256);
        const __amdgpu_buffer_rsrc_t dg = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(en.dy + g * 256), 0, (int)(dy_bytes - (uint32_t)(g * 512)), 0x00020000);
        const __amdgpu_buffer_rsrc_t cg = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(en.packed_t + g * 256), 0, (int)(code_bytes - (uint32_t)(g * 1024)), 0x00020000);
        const uint32_t row_bytes = (uint32_t)en.N * 2;
        const uint32_t off0 = (uint32_t)(m0 + r0) * row_bytes + 16u * (uint32_t)c0;  // used only for rows of the tile
#pragma unroll
        for (int i = 0; i < C::DY_LOADS; ++i) {
            const uint32_t off = r0 + RSTEP * i < rows_left ? off0 + (uint32_t)(RSTEP * i) * row_bytes : dy_bytes;
            r[i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(dg, off, 0, 0));
        }
        const int ngfull = (int)(en.KFt / 4);
        if (g < ngfull) {
#pragma unroll
            for (int j2 = 0; j2 < NF; ++j2) {
                const uint32_t base = rbj[j2] < en.KB
                                          ? (uint32_t)rbj[j2] * (uint32_t)en.KFt * 256u + 16u * (uint32_t)clam
                                          : code_bytes;
                r[C::DY_LOADS + 2 * j2] =
                    __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(cg, base, 0, 0));
                r[C::DY_LOADS + 2 * j2 + 1] =
                    __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(cg, base + 512, 0, 0));
            }
        } else {
            // the partial last group (Gt fragments; dword lam of fragment f
            // at lam*Gt + f) gathered into the places a full group's dwords
            // take, zero codes past its fragments: the full-group compute
            // then runs it unchanged
            const int Gt = (int)(en.KFt - 4 * ngfull);
#pragma unroll
            for (int j2 = 0; j2 < NF; ++j2) {
                const uint32_t blk = rbj[j2] < en.KB ? (uint32_t)rbj[j2] * (uint32_t)en.KFt * 256u : code_bytes;
#pragma unroll
                for (int e2 = 0; e2 < 2; ++e2)
#pragma unroll
                    for (int f = 0; f < 4; ++f) {
                        const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(
                            cg, blk + 4u * (uint32_t)((clam + 32 * e2) * Gt + f), 0, 0);
                        r[C::DY_LOADS + 2 * j2 + e2][f] = f < Gt ? w : 0u;
                    }
            }
        }
    };
    auto store = [&](int stage, const v4u(&r)[NR]) __attribute__((always_inline)) {
        uint8_t *st = lds + stage * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::DY_LOADS; ++i) {
            const int row = r0 + RSTEP * i;
            *reinterpret_cast<v4u *>(st + row * C::ROW + ((c0 ^ (row & 31)) << 4)) = r[i];
        }
    };

    v16f acc[MF][NF];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) acc[i][j] = v16f{};
    // slice 0's running total in LDS past the stages, bf16 pairs (values q
    // and q + 1 of a fragment) in lane order; it starts at dx when
    // accumulating, else at 0
    uint32_t *tot = reinterpret_cast<uint32_t *>(lds_all + KS * C::SLICE_BYTES) + wave * (MF * NF * 8 * 64) + lane;
    if (ks == 0) {
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
            for (int j = 0; j < NF; ++j) {
                const int64_t k = k0 + (wn * NF + j) * 32 + lr;
#pragma unroll
                for (int q = 0; q < 16; q += 2) {
                    const int64_t m = m0 + (wm * MF + i) * 32 + 8 * (q >> 2) + 4 * lh + (q & 3);
                    uint32_t lo = 0, hi = 0;
                    if (a.accumulate && k < K) {
                        if (m < M) lo = a.dx[m * K + k];
                        if (m + 1 < M) hi = a.dx[(m + 1) * K + k];
                    }
                    tot[((i * NF + j) * 8 + (q >> 1)) * 64] = lo | (hi << 16);
                }
            }
    }

    const uint8_t *arow = lds + (wm * MF * 32 + lr) * C::ROW;
    auto read_a = [&](const uint8_t *st, int s, v8bf(&x)[MF][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int ch = ((4 * s + 2 * lh + u) ^ lr) << 4;
#pragma unroll
            for (int i = 0; i < MF; ++i) x[i][u] = *reinterpret_cast<const v8bf *>(st + (arow - lds) + i * 32 * C::ROW + ch);
        }
    };
    auto mma = [&](const v8bf(&x)[MF][2], const uint32_t(&w)[NF]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            v8bf bq[NF];
#pragma unroll
            for (int j = 0; j < NF; ++j) bq[j] = codes_bf16(w[j], u);
#pragma unroll
            for (int i = 0; i < MF; ++i)
#pragma unroll
                for (int j = 0; j < NF; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[i][u], bq[j], acc[i][j], 0, 0, 0);
        }
    };
    auto compute_full = [&](int stage, const v4u(&r)[NR]) __attribute__((always_inline)) {
        const uint8_t *st = lds + stage * C::STAGE;
        v8bf xa[2][MF][2];
        read_a(st, 0, xa[0]);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            if (s + 1 < 8) read_a(st, s + 1, xa[(s + 1) & 1]);
            uint32_t w[NF];
#pragma unroll
            for (int j = 0; j < NF; ++j) w[j] = r[C::DY_LOADS + 2 * j + (s & 1)][s >> 1];
            mma(xa[s & 1], w);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // slice 0 folds the entry's sums into the total; slice 1's sums come
    // through the two slots (of both slices) that hold no live stage now
    auto fold = [&](const DgradEntry &en, int stage) __attribute__((always_inline)) {
        if constexpr (KS > 1) {
            constexpr int PER_WAVE = MF * NF * 16 * 64 * 4;  // bytes
            static_assert(C::W * PER_WAVE <= 2 * C::STAGE, "slice 1's sums fit the two free slots");
            constexpr int WAVES_PER_SLOT = C::STAGE / PER_WAVE;
            const int w_slot = wave / WAVES_PER_SLOT, w_in = wave - w_slot * WAVES_PER_SLOT;
            float *red = reinterpret_cast<float *>(lds_all + w_slot * C::SLICE_BYTES + stage * C::STAGE +
                                                   w_in * PER_WAVE) + lane;
            if (ks == 1) {
#pragma unroll
                for (int i = 0; i < MF; ++i)
#pragma unroll
                    for (int j = 0; j < NF; ++j)
#pragma unroll
                        for (int q = 0; q < 16; ++q) red[((i * NF + j) * 16 + q) * 64] = acc[i][j][q];
            }
            lds_barrier();
            if (ks == 0) {
#pragma unroll
                for (int i = 0; i < MF; ++i)
#pragma unroll
                    for (int j = 0; j < NF; ++j)
#pragma unroll
                        for (int q = 0; q < 16; ++q) acc[i][j][q] += red[((i * NF + j) * 16 + q) * 64];
            }
        }
        if (ks == 0) {
            const float ghalf = en.gamma[0] * 0.5f;  // codes enter the MFMA as +-2
#pragma unroll
            for (int i = 0; i < MF; ++i)
#pragma unroll
                for (int j = 0; j < NF; ++j)
#pragma unroll
                    for (int q = 0; q < 16; q += 2) {
                        uint32_t &tp = tot[((i * NF + j) * 8 + (q >> 1)) * 64];
                        const uint32_t t0 = tp;
                        const float v0 = acc[i][j][q] * ghalf + __uint_as_float(t0 << 16);
                        const float v1 = acc[i][j][q + 1] * ghalf + __uint_as_float(t0 & 0xFFFF0000u);
                        tp = pack_bf16x2(v0, v1);
                    }
        }
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
            for (int j = 0; j < NF; ++j) acc[i][j] = v16f{};
        if constexpr (KS > 1) lds_barrier();  // slice 0 is done reading before the slots are refilled
    };

    // ---- pipeline: ring of two VGPR sets, LDS slot j & 1 of each slice holds
    // the dy of its step j; both slices run the same a.steps steps
    const int J = a.steps;
    v4u rs[2][NR];
    load(0, rs[0]);
    store(0, rs[0]);
    lds_barrier();
    auto step = [&](int j, auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        load(j + 1 < J ? j + 1 : J - 1, rs[k ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
        const int e = entry_of(j);
        const DgradEntry en = entry(e);
        if (group_of(en, j) < en.groups) compute_full(k, rs[k]);  // else a padding step
        store(k ^ 1, rs[k ^ 1]);  // past the last step: a harmless repeat
        lds_barrier();
        const int next = e + 1 < a.count ? entry(e + 1).step_begin : J;
        if (j + 1 == next) fold(en, k);
    };
    for (int c = 0; c < J / 2; ++c) {
        step(2 * c, std::integral_constant<int, 0>{});
        step(2 * c + 1, std::integral_constant<int, 1>{});
    }
    if (J & 1) step(J - 1, std::integral_constant<int, 0>{});

    // ---- epilogue: slice 0's totals are bf16 already; stage the tile in
    // LDS, then every thread writes 16-byte chunks of rows
    uint16_t *__restrict__ dx = a.dx;
    if ((K & 7) == 0) {
        uint16_t *tile = reinterpret_cast<uint16_t *>(lds_all);
        if constexpr (KS == 1) lds_barrier();  // every wave is done with the stages
        if (ks == 0) {
#pragma unroll
            for (int i = 0; i < MF; ++i)
#pragma unroll
                for (int j = 0; j < NF; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = (wm * MF + i) * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                        const uint32_t tp = tot[((i * NF + j) * 8 + (r >> 1)) * 64];
                        tile[row * C::BN + (wn * NF + j) * 32 + lr] = (uint16_t)((r & 1) ? tp >> 16 : tp);
                    }
        }
        lds_barrier();
        constexpr int CPR = C::BN / 8;
        for (int q = threadIdx.x; q < C::BM * CPR; q += C::NTT) {
            const int row = q / CPR, c8 = q - row * CPR;
            const int64_t m = m0 + row, k = k0 + 8 * c8;
            if (m >= M || k >= K) continue;  // K % 8 == 0: a chunk is all in or all out
            __builtin_nontemporal_store(*reinterpret_cast<const v4u *>(tile + row * C::BN + 8 * c8),
                                        reinterpret_cast<v4u *>(dx + m * K + k));
        }
        return;
    }
    if (ks != 0) return;
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) {
            const int64_t k = k0 + (wn * NF + j) * 32 + lr;
            if (k >= K) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + (wm * MF + i) * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                const uint32_t tp = tot[((i * NF + j) * 8 + (r >> 1)) * 64];
                if (m < M) dx[m * K + k] = (uint16_t)((r & 1) ? tp >> 16 : tp);
            }
        }
}

template <int WM, int WN, int MF, int NF, int KS>
hipError_t launch_dgrad_cfg(DgradArgs &a, hipStream_t s) {
    using C = DgCfg<WM, WN, MF, NF, KS>;
    a.tiles_m = (int)((a.M + C::BM - 1) / C::BM);
    a.tiles_n = (int)((a.K + C::BN - 1) / C::BN);
    auto kern = dgrad_pipe<WM, WN, MF, NF, KS>;
    if (C::LDS_BYTES > 65536) {
        hipError_t e = lds_optin<dgrad_pipe<WM, WN, MF, NF, KS>>(C::LDS_BYTES);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.tiles_m * a.tiles_n)), dim3(C::NTT), C::LDS_BYTES, s, a);
    return hipGetLastError();
}

}  // namespace

template <int WM, int WN, int MF, int NF, int KS>
hipError_t launch_dgrad_grouped_cfg(DgradGroupArgs &a, hipStream_t s) {
    using C = DgCfg<WM, WN, MF, NF, KS>;
    a.tiles_m = (int)((a.M + C::BM - 1) / C::BM);
    a.tiles_n = (int)((a.K + C::BN - 1) / C::BN);
    int steps = 0;  // each entry's groups dealt to the slices in turn, padded to whole rounds
    for (int e = 0; e < a.count; ++e) {
        a.e[e].step_begin = steps;
        steps += (a.e[e].groups + KS - 1) / KS;
    }
    a.steps = steps;
    constexpr int LDS = C::LDS_BYTES + C::BM * C::BN * 2;  // the stages, then the bf16 totals
    static_assert(LDS <= 160 * 1024, "a CU's LDS");
    auto kern = dgrad_grouped<WM, WN, MF, NF, KS>;
    if (LDS > 65536) {
        hipError_t e = lds_optin<dgrad_grouped<WM, WN, MF, NF, KS>>(LDS);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.tiles_m * a.tiles_n)), dim3(C::NTT), LDS, s, a);
    return hipGetLastError();
}

// 64 x 256 tiles with two K slices when 32-row tiles would take more than
// one round of the 256 CUs but 64-row ones do not, and the entries have four
// or more groups between them (each slice then has work between folds);
// otherwise 32 x 256 tiles, two workgroups per CU.
hipError_t launch_dgrad_grouped(DgradGroupArgs &a, hipStream_t s) {
    const int64_t tiles64 = ((a.M + 63) / 64) * ((a.K + 255) / 256);
    int64_t groups = 0;
    for (int e = 0; e < a.count; ++e) groups += a.e[e].groups;
    if (2 * tiles64 > 256 && tiles64 <= 256 && groups >= 4) return launch_dgrad_grouped_cfg<1, 4, 2, 2, 2>(a, s);
    return launch_dgrad_grouped_cfg<1, 4, 1, 2, 1>(a, s);
}

bool dgrad_ok(int64_t M, int64_t N, int64_t K) {
    const Layout Lt = Layout::of(K, N);
    return N % 8 == 0 && M * N * 2 < ((int64_t)1 << 31) && Lt.bytes < ((int64_t)1 << 31) &&
           (M + 31) / 32 * ((K + 255) / 256) < ((int64_t)1 << 31);
}

hipError_t launch_pack_t1_grouped(PackSegs &ps, hipStream_t s) {
    int64_t wg = 0;
    for (int i = 0; i < ps.count; ++i) {
        PackSeg &g = ps.s[i];
        const Layout L = Layout::of(g.N, g.K);
        g.t1_begin = wg;
        if (g.packed_t) wg += (L.NB + 3) / 4 * L.KF;
    }
    if (wg == 0) return hipSuccess;
    hipLaunchKernelGGL(codes_to_t1_grouped, dim3((unsigned)wg), dim3(256), 0, s, ps);
    return hipGetLastError();
}

hipError_t launch_pack_t1(const uint32_t *packed, int64_t N, int64_t K, uint32_t *packed_t, hipStream_t s) {
    const Layout L = Layout::of(N, K), Lt = Layout::of(K, N);
    const dim3 grid((unsigned)((L.NB + 3) / 4), (unsigned)L.KF);
    hipLaunchKernelGGL(codes_to_t1, grid, dim3(256), 0, s, packed, packed_t, L.NB, L.KF, Lt.NB, Lt.KF);
    return hipGetLastError();
}

hipError_t launch_dgrad(const uint32_t *packed_t, const float *gamma, int64_t N, int64_t K, const uint16_t *dy,
                        int64_t M, uint16_t *dx, int accumulate, hipStream_t s) {
    const Layout Lt = Layout::of(K, N);
    DgradArgs a;
    a.packed_t = packed_t;
    a.gamma = gamma;
    a.dy = dy;
    a.dx = dx;
    a.M = M;
    a.N = N;
    a.K = K;
    a.KB = Lt.NB;
    a.KFt = Lt.KF;
    a.accumulate = accumulate ? 1 : 0;
    // 64 x 256 tiles when they fill the chip's 512 four-wave slots; when
    // they number a CU's worth or less and the contraction has at least four
    // groups, the same tiles with the contraction split over two slices (two
    // waves per SIMD); otherwise 32 x 256 tiles
    const int64_t tiles64 = ((M + 63) / 64) * ((K + 255) / 256);
    if (tiles64 >= 512) return launch_dgrad_cfg<1, 4, 2, 2, 1>(a, s);
    if (tiles64 <= 256 && Lt.KF / 4 >= 4) return launch_dgrad_cfg<1, 4, 2, 2, 2>(a, s);
    return launch_dgrad_cfg<1, 4, 1, 2, 1>(a, s);
}

}  // namespace bl
