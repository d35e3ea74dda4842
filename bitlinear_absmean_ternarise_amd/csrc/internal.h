// Internal declarations shared by the host entry points and the kernel files.
// Device pointers only; shapes already validated by the entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace bl {

// ---- packed layout v1 geometry (see include/bitlinear.h)
struct Layout {
    int64_t N, K;
    int64_t NB;   // 16-row blocks
    int64_t KF;   // 64-column fragments
    int64_t NG;   // groups of up to four fragments
    int64_t bytes;
    static Layout of(int64_t N, int64_t K) {
        Layout L;
        L.N = N;
        L.K = K;
        L.NB = (N + 15) / 16;
        L.KF = (K + 63) / 64;
        L.NG = (L.KF + 3) / 4;
        L.bytes = L.NB * L.KF * 256;
        return L;
    }
};

// ---- pack
int64_t pack_partials(int64_t count);  // number of fp64 partial sums used for gamma
hipError_t launch_pack(const float *W, const Layout &L, float eps, double *partials,
                       uint32_t *packed, float *gamma, hipStream_t s);

// Up to kPackGroup tensors per launch, each packed exactly as by launch_pack
// (the host fills W, partials, gamma, packed, count, N, K, KF, dwords, eps,
// aligned; the launcher fills the rest)
constexpr int kPackGroup = 16;
struct PackSeg {
    const float *W;
    double *partials;
    float *gamma;
    uint32_t *packed;
    uint32_t *packed_t;  // layout t1 of the same codes, or NULL
    int64_t count, chunk, nblocks, wg_begin, N, K, KF, dwords, dw_begin, t1_begin;
    float eps;
    int aligned;
};
struct PackSegs {
    PackSeg s[kPackGroup];
    int count;
};
hipError_t launch_pack_grouped(PackSegs &ps, hipStream_t s);
// layout t1 of the codes of the segments whose packed_t is set (after launch_pack_grouped)
hipError_t launch_pack_t1_grouped(PackSegs &ps, hipStream_t s);

// Binary BitNet weights in the same layout: codes +1 where W >= alpha, -1
// elsewhere; beta = mean |W|, alpha = mean W (device scalars).
hipError_t launch_pack_binary(const float *W, const Layout &L, double *partials, uint32_t *packed,
                              float *beta, float *alpha, hipStream_t s);

// ---- one-bit layout b1 of binary weights (see include/bitlinear.h):
// 16-row x 128-column pairs of 64 dwords, groups of up to four pairs
inline int64_t b1_bytes(int64_t N, int64_t K) { return (N + 15) / 16 * ((K + 127) / 128) * 256; }
// shapes the b1 kernels take: K % 64 == 0, K <= kScaledMaxK, buffer below 2 GB
bool b1_ok(int64_t N, int64_t K);
hipError_t launch_pack_binary_b1(const float *W, int64_t N, int64_t K, double *partials, uint32_t *packed,
                                 float *beta, float *alpha, hipStream_t s);

// ---- STE backward to the input: codes rearranged into layout t1, then
// dx = bf16(gamma * dy @ codes (+ dx))
struct DgradArgs {
    const uint32_t *packed_t;
    const float *gamma;
    const uint16_t *dy;
    uint16_t *dx;
    int64_t M, N, K;
    int64_t KB;   // 16-row blocks of the transposed matrix (along K)
    int64_t KFt;  // 64-column fragments of the transposed matrix (along N)
    int tiles_m, tiles_n, accumulate;
};
// Several layers that read one input (Q, K and V; gate and up) in one
// launch: dx = bf16(g_E/2 acc_E + ... bf16(g_1/2 acc_1 (+ dx))), the rounding
// sequence of one call per entry with accumulate on from the second entry.
constexpr int kDgradMaxEntries = 4;
struct DgradEntry {
    const uint32_t *packed_t;
    const float *gamma;
    const uint16_t *dy;
    int64_t N, KB, KFt;
    int groups;      // contraction groups (of 256 dy columns, the last one partial)
    int step_begin;  // first pipeline step of the entry (set by the launcher)
};
struct DgradGroupArgs {
    DgradEntry e[kDgradMaxEntries];
    uint16_t *dx;
    int64_t M, K;
    int count, steps, tiles_m, tiles_n, accumulate;
};
hipError_t launch_dgrad_grouped(DgradGroupArgs &a, hipStream_t s);
bool dgrad_ok(int64_t M, int64_t N, int64_t K);
hipError_t launch_pack_t1(const uint32_t *packed, int64_t N, int64_t K, uint32_t *packed_t, hipStream_t s);
hipError_t launch_dgrad(const uint32_t *packed_t, const float *gamma, int64_t N, int64_t K, const uint16_t *dy,
                        int64_t M, uint16_t *dx, int accumulate, hipStream_t s);

// ---- AdamW step with the tracker fused (counters NULL: no tracking)
hipError_t launch_adamw_flip(float *W, const float *g, float *m, float *v, int64_t n, int32_t t, double lr,
                             double b1, double b2, double eps, double wd, int16_t *fc, int16_t *lf,
                             hipStream_t s);

// ---- tracker read-out: sign age and flip rate after T steps
hipError_t launch_flip_stats(const int16_t *fc, const int16_t *lf, int64_t n, int32_t T, float *age,
                             float *rate, hipStream_t s);

// ---- activation quant
hipError_t launch_quant(const uint16_t *x, int64_t M, int64_t K, float eps, int8_t *xq,
                        float *xs, hipStream_t s);
hipError_t launch_norm_quant(const uint16_t *x, const float *gain, int64_t M, int64_t K, float eps_n,
                             float eps, int8_t *xq, float *xs, hipStream_t s);

// ---- forward
hipError_t launch_forward(const uint32_t *packed, const float *gamma, const Layout &L,
                          const int8_t *xq, const float *xs, int64_t M, uint16_t *y,
                          int32_t *acc, hipStream_t s);

hipError_t launch_gemm_pipe(const uint32_t *packed, const float *gamma, const Layout &L,
                            const int8_t *xq, const float *xs, int64_t M, uint16_t *y,
                            int32_t *acc, hipStream_t s);

hipError_t launch_gemv(const uint32_t *packed, const float *gamma, const Layout &L,
                       const int8_t *xq, const float *xs, int64_t M, uint16_t *y,
                       int32_t *acc, hipStream_t s);

// ---- grouped forward: several independent forwards in one launch
constexpr int kMaxSeg = 8;
struct FwdSeg {
    const uint32_t *packed;
    const float *gamma;
    Layout L;
    const int8_t *xq;
    const float *xs;
    int64_t M;
    uint16_t *y;
    int32_t *acc;
    int8_t *xq_out = nullptr;  // quant + forward: where the activation codes go
    float *xs_out = nullptr;
};
// Decode kernels take 1..kGemvMaxM tokens (K % 16 == 0, buffers below 2 GB).
constexpr int64_t kGemvMaxM = 64;
bool gemv_ok(const Layout &L, int64_t M);
hipError_t launch_gemv_multi(const FwdSeg *segs, int count, hipStream_t s);
// Decode with the activation quant in the same launch (each workgroup
// quantises the tokens into LDS): one token with K <= kFusedMaxMK, or 2..16
// tokens with M*K <= kFusedMaxMK / 2 (past that, measured on the 3B layer,
// the repeated quant costs more than a quant launch).  The segment's
// xq / xs (FwdSeg::xq_out / xs_out) are written when write_q is set (one
// segment per distinct input).
constexpr int64_t kFusedMaxMK = 32768;
struct QFwdSeg {
    FwdSeg f;           // f.xq / f.xs unused; f.xq_out / f.xs_out receive the codes and scales
    const uint16_t *x;  // [M][K] bf16 bits
    bool write_q;
};
bool gemv_quant_ok(const Layout &L, int64_t M);
// The decode contraction on the vector ALUs (v_dot4_i32_i8) for 1..kDot4MaxM
// tokens: K % 16 == 0, K <= kScaledMaxK, buffers below 2 GB.
constexpr int64_t kDot4MaxM = 4;
bool dot4_ok(const Layout &L, int64_t M);
hipError_t launch_gemv_dot4_multi(const FwdSeg *segs, int count, hipStream_t s);
// Forward over layout b1 (FwdSeg::gamma holds beta; FwdSeg::L only its N
// and K): any M >= 1, tokens in tiles of 16, one launch for all segments.
hipError_t launch_forward_b1(const FwdSeg *segs, int count, hipStream_t s);
// b1: the one-launch decode over layout b1 (f.gamma holds beta);
// gemv_quant_b1_ok: its token limits (as gemv_quant_ok) over shapes b1 takes
bool gemv_quant_b1_ok(int64_t N, int64_t K, int64_t M);
hipError_t launch_gemv_quant_multi(const QFwdSeg *segs, int count, float eps, hipStream_t s, bool b1 = false);
// Prefill GEMM: K % 16 == 0 and buffers below 2 GB; any M.
bool gemm_ok(const Layout &L, int64_t M);
hipError_t launch_gemm_multi(const FwdSeg *segs, int count, hipStream_t s);
// Decode batches of kSplitMinM..kGemvMaxM tokens on the GEMM, with K cut
// into runs whose int32 sums meet in a caller workspace where a launch has
// too few output tiles.  gemm_small_bytes: the workspace a launch needs (0:
// none); gemm_small_ok: whether the path takes the launch (with or without a
// workspace at hand); launch_gemm_small also launches the reduce.
constexpr int64_t kSplitMinM = 14;
constexpr int64_t kSmallTarget = 256;      // tiles x runs: one workgroup per CU
constexpr int64_t kSplitMinGroups = 4;     // groups of 256 columns per run, at least
constexpr int64_t kSmallLongGroups = 64;   // 14..32 tokens: only rows this long are cut
size_t gemm_small_bytes(const FwdSeg *segs, int count);
// Largest workspace the plan can ask for: runs x tiles <= kSmallTarget, and
// a run's partial sums cover at most one 64 x 128 (or 32 x 256) int32 tile,
// plus 256-byte alignment per entry.
constexpr size_t kSmallMaxBytes = (size_t)kSmallTarget * 64 * 128 * 4 + (size_t)kMaxSeg * 256;
// Device address, on the current device, of the library's fixed scratch for
// the no-allocation forward (kScratchBytes bytes; looked up once per device).
hipError_t scratch_ptr(void **ptr);
bool gemm_small_ok(const FwdSeg *segs, int count, bool have_workspace);
hipError_t launch_gemm_small(const FwdSeg *segs, int count, void *workspace, hipStream_t s);

// ---- tracker
hipError_t launch_flip(const float *prev, const float *curr, int64_t n, int32_t step,
                       int16_t *fc, int16_t *lf, hipStream_t s);

}  // namespace bl
