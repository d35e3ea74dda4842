// C-ABI entry points: validate on the host, then enqueue the gfx950 kernels on
// the caller's stream.  No allocation, no synchronisation, no exceptions.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>

#include "../../include/bitlinear.h"
#include "internal.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // rows / tokens per call

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-device cache of "is this gfx950?" (0 unknown, 1 yes, -1 no).
std::atomic<int> g_arch_ok[64];

int check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return BL_ERR_DEVICE;
    if (dev < 0 || dev >= 64) return BL_ERR_DEVICE;
    int state = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BL_ERR_DEVICE;
        state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
        g_arch_ok[dev].store(state, std::memory_order_relaxed);
    }
    return state == 1 ? BL_OK : BL_ERR_ARCH;
}

int shape_ok(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0) return BL_ERR_SHAPE;
    if (N > kMaxDim || K > BITLINEAR_MAX_K) return BL_ERR_SHAPE;
    return BL_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? BL_OK : BL_ERR_DEVICE; }

}  // namespace

extern "C" {

int bitlinear_packed_bytes(int64_t N, int64_t K, size_t *bytes) {
    if (!bytes) return BL_ERR_NULL;
    int st = shape_ok(N, K);
    if (st) return st;
    *bytes = (size_t)bl::Layout::of(N, K).bytes;
    return BL_OK;
}

int bitlinear_pack_workspace_bytes(int64_t N, int64_t K, size_t *bytes) {
    if (!bytes) return BL_ERR_NULL;
    int st = shape_ok(N, K);
    if (st) return st;
    *bytes = (size_t)bl::pack_partials(N * K) * sizeof(double);
    return BL_OK;
}

int bitlinear_pack_weights(const float *W, int64_t N, int64_t K, float eps, void *workspace,
                           size_t workspace_bytes, uint8_t *packed, float *gamma, void *stream) {
    if (!W || !packed || !gamma) return BL_ERR_NULL;
    int st = shape_ok(N, K);
    if (st) return st;
    if (!std::isfinite(eps) || eps < 0.0f) return BL_ERR_VALUE;
    if (!workspace) return BL_ERR_WORKSPACE;
    if (workspace_bytes < (size_t)bl::pack_partials(N * K) * sizeof(double)) return BL_ERR_WORKSPACE;
    if (!aligned16(W) || !aligned16(packed) || !aligned16(gamma) || !aligned16(workspace))
        return BL_ERR_ALIGN;
    if ((st = check_device())) return st;
    const bl::Layout L = bl::Layout::of(N, K);
    return launched(bl::launch_pack(W, L, eps, static_cast<double *>(workspace),
                                    reinterpret_cast<uint32_t *>(packed), gamma,
                                    static_cast<hipStream_t>(stream)));
}

int bitlinear_pack_weights_grouped(const bitlinear_pack_args *args, int count, void *stream) {
    if (!args) return BL_ERR_NULL;
    if (count < 1 || count > BITLINEAR_MAX_PACK_GROUP) return BL_ERR_SHAPE;
    for (int i = 0; i < count; ++i) {
        const bitlinear_pack_args &a = args[i];
        if (!a.W || !a.packed || !a.gamma) return BL_ERR_NULL;
        int st = shape_ok(a.N, a.K);
        if (st) return st;
        if (!std::isfinite(a.eps) || a.eps < 0.0f) return BL_ERR_VALUE;
        if (!a.workspace) return BL_ERR_WORKSPACE;
        if (a.workspace_bytes < (size_t)bl::pack_partials(a.N * a.K) * sizeof(double)) return BL_ERR_WORKSPACE;
        if (!aligned16(a.W) || !aligned16(a.packed) || !aligned16(a.gamma) || !aligned16(a.workspace) ||
            (a.packed_t && !aligned16(a.packed_t)))
            return BL_ERR_ALIGN;
    }
    int st = check_device();
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int i0 = 0; i0 < count; i0 += bl::kPackGroup) {
        bl::PackSegs ps{};
        ps.count = count - i0 < bl::kPackGroup ? count - i0 : bl::kPackGroup;
        for (int j = 0; j < ps.count; ++j) {
            const bitlinear_pack_args &a = args[i0 + j];
            const bl::Layout L = bl::Layout::of(a.N, a.K);
            bl::PackSeg &g = ps.s[j];
            g.W = a.W;
            g.partials = static_cast<double *>(a.workspace);
            g.gamma = a.gamma;
            g.packed = reinterpret_cast<uint32_t *>(a.packed);
            g.count = a.N * a.K;
            g.N = a.N;
            g.K = a.K;
            g.KF = L.KF;
            g.dwords = L.bytes / 4;
            g.eps = a.eps;
            g.aligned = a.K % 4 == 0 ? 1 : 0;
            g.packed_t = reinterpret_cast<uint32_t *>(a.packed_t);
        }
        st = launched(bl::launch_pack_grouped(ps, s));
        if (st) return st;
        st = launched(bl::launch_pack_t1_grouped(ps, s));
        if (st) return st;
    }
    return BL_OK;
}

int bitlinear_pack_binary(const float *W, int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                          uint8_t *packed, float *beta, float *alpha, void *stream) {
    if (!W || !packed || !beta || !alpha) return BL_ERR_NULL;
    int st = shape_ok(N, K);
    if (st) return st;
    if (!workspace) return BL_ERR_WORKSPACE;
    if (workspace_bytes < (size_t)bl::pack_partials(N * K) * sizeof(double)) return BL_ERR_WORKSPACE;
    if (!aligned16(W) || !aligned16(packed) || !aligned16(beta) || !aligned16(alpha) || !aligned16(workspace))
        return BL_ERR_ALIGN;
    if ((st = check_device())) return st;
    const bl::Layout L = bl::Layout::of(N, K);
    return launched(bl::launch_pack_binary(W, L, static_cast<double *>(workspace), reinterpret_cast<uint32_t *>(packed),
                                           beta, alpha, static_cast<hipStream_t>(stream)));
}

int bitlinear_quant_act(const uint16_t *x, int64_t M, int64_t K, float eps, int8_t *xq,
                        float *x_scale, void *stream) {
    if (M < 0 || K <= 0 || M > kMaxDim || K > BITLINEAR_MAX_K) return BL_ERR_SHAPE;
    if (!std::isfinite(eps) || !(eps > 0.0f)) return BL_ERR_VALUE;
    if (M == 0) return BL_OK;
    if (!x || !xq || !x_scale) return BL_ERR_NULL;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(x_scale)) return BL_ERR_ALIGN;
    int st = check_device();
    if (st) return st;
    return launched(bl::launch_quant(x, M, K, eps, xq, x_scale, static_cast<hipStream_t>(stream)));
}

int bitlinear_rmsnorm_quant_act(const uint16_t *x, const float *gain, int64_t M, int64_t K, float eps_norm,
                                float eps, int8_t *xq, float *x_scale, void *stream) {
    if (M < 0 || K <= 0 || M > kMaxDim || K > BITLINEAR_MAX_K) return BL_ERR_SHAPE;
    if (!std::isfinite(eps) || !(eps > 0.0f)) return BL_ERR_VALUE;
    if (!std::isfinite(eps_norm) || eps_norm < 0.0f) return BL_ERR_VALUE;
    if (M == 0) return BL_OK;
    if (!x || !xq || !x_scale) return BL_ERR_NULL;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(x_scale) || (gain && !aligned16(gain))) return BL_ERR_ALIGN;
    int st = check_device();
    if (st) return st;
    return launched(bl::launch_norm_quant(x, gain, M, K, eps_norm, eps, xq, x_scale, static_cast<hipStream_t>(stream)));
}

int bitlinear_forward(const uint8_t *packed, const float *gamma, int64_t N, int64_t K,
                      const int8_t *xq, const float *x_scale, int64_t M, uint16_t *y,
                      int32_t *acc, void *stream) {
    int st = shape_ok(N, K);
    if (st) return st;
    if (M < 0 || M > kMaxDim) return BL_ERR_SHAPE;
    if (M == 0) return BL_OK;
    if (!packed || !gamma || !xq || !x_scale || !y) return BL_ERR_NULL;
    if (!aligned16(packed) || !aligned16(gamma) || !aligned16(xq) || !aligned16(x_scale) ||
        !aligned16(y) || (acc && !aligned16(acc)))
        return BL_ERR_ALIGN;
    if ((st = check_device())) return st;
    const bl::Layout L = bl::Layout::of(N, K);
    return launched(bl::launch_forward(reinterpret_cast<const uint32_t *>(packed), gamma, L, xq,
                                       x_scale, M, y, acc, static_cast<hipStream_t>(stream)));
}

namespace {
static int forward_args_ok(const bitlinear_forward_args &a) {
    int st = shape_ok(a.N, a.K);
    if (st) return st;
    if (a.M < 0 || a.M > kMaxDim) return BL_ERR_SHAPE;
    if (a.M == 0) return BL_OK;
    if (!a.packed || !a.gamma || !a.xq || !a.x_scale || !a.y) return BL_ERR_NULL;
    if (!aligned16(a.packed) || !aligned16(a.gamma) || !aligned16(a.xq) || !aligned16(a.x_scale) ||
        !aligned16(a.y) || (a.acc && !aligned16(a.acc)))
        return BL_ERR_ALIGN;
    return BL_OK;
}
}  // namespace

namespace {
// Validates the entries and gathers the non-empty ones into segs; *all_gemv /
// *all_gemm tell whether one decode or one prefill launch can take them all.
static int gather_forward(const bitlinear_forward_args *args, int count, bl::FwdSeg *segs, int *n_out,
                          bool *all_gemv, bool *all_gemm, bool *all_split) {
    if (!args) return BL_ERR_NULL;
    if (count < 1 || count > BITLINEAR_MAX_GROUP) return BL_ERR_SHAPE;
    for (int i = 0; i < count; ++i) {
        int st = forward_args_ok(args[i]);
        if (st) return st;
    }
    int n = 0;
    *all_gemv = *all_gemm = *all_split = true;
    for (int i = 0; i < count; ++i) {
        const bitlinear_forward_args &a = args[i];
        if (a.M == 0) continue;
        segs[n] = bl::FwdSeg{reinterpret_cast<const uint32_t *>(a.packed), a.gamma, bl::Layout::of(a.N, a.K),
                             a.xq, a.x_scale, a.M, a.y, a.acc};
        *all_gemv = *all_gemv && bl::gemv_ok(segs[n].L, a.M);
        *all_gemm = *all_gemm && a.M > bl::kGemvMaxM && bl::gemm_ok(segs[n].L, a.M);
        *all_split = *all_split && a.M <= bl::kGemvMaxM && bl::gemm_ok(segs[n].L, a.M);
        ++n;
    }
    *n_out = n;
    return BL_OK;
}

// The launches of validated, non-empty forward entries.  One launch when
// every entry takes the same kind of kernel: the GEMM for 14..64 tokens where
// it beats the decode kernel (cut into runs only with a workspace), else the
// decode kernels (1..64 tokens) or the prefill GEMM (more tokens).
static int dispatch_forward(const bl::FwdSeg *segs, int n, bool all_gemv, bool all_gemm, bool all_split,
                            void *workspace, hipStream_t s) {
    if (all_split && bl::gemm_small_ok(segs, n, workspace != nullptr))
        return launched(bl::launch_gemm_small(segs, n, workspace, s));
    if (all_gemv) return launched(bl::launch_gemv_multi(segs, n, s));
    if (all_gemm) return launched(bl::launch_gemm_multi(segs, n, s));
    for (int i = 0; i < n; ++i) {
        const bl::FwdSeg &f = segs[i];
        hipError_t e = bl::launch_forward(f.packed, f.gamma, f.L, f.xq, f.xs, f.M, f.y, f.acc, s);
        if (e != hipSuccess) return BL_ERR_DEVICE;
    }
    return BL_OK;
}

// use_scratch: the no-allocation variant, whose workspace is the library's
// fixed scratch (looked up after the device check).
static int forward_grouped_impl(const bitlinear_forward_args *args, int count, void *workspace, size_t workspace_bytes,
                                void *stream, bool use_scratch = false) {
    bl::FwdSeg segs[BITLINEAR_MAX_GROUP];
    int n = 0;
    bool all_gemv, all_gemm, all_split;
    int st = gather_forward(args, count, segs, &n, &all_gemv, &all_gemm, &all_split);
    if (st) return st;
    if (workspace && !aligned16(workspace)) return BL_ERR_ALIGN;
    const size_t need = ((workspace || use_scratch) && n > 0 && all_split) ? bl::gemm_small_bytes(segs, n) : 0;
    if (use_scratch && need > BITLINEAR_SCRATCH_BYTES) return BL_ERR_SCRATCH;
    if (!use_scratch && need > workspace_bytes) return BL_ERR_WORKSPACE;
    if ((st = check_device())) return st;
    if (n == 0) return BL_OK;
    if (use_scratch && need > 0 && bl::scratch_ptr(&workspace) != hipSuccess) return BL_ERR_DEVICE;
    return dispatch_forward(segs, n, all_gemv, all_gemm, all_split, workspace, static_cast<hipStream_t>(stream));
}
}  // namespace

int bitlinear_forward_grouped(const bitlinear_forward_args *args, int count, void *stream) {
    return forward_grouped_impl(args, count, nullptr, 0, stream);
}

int bitlinear_forward_workspace_bytes(const bitlinear_forward_args *args, int count, size_t *bytes) {
    if (!bytes) return BL_ERR_NULL;
    bl::FwdSeg segs[BITLINEAR_MAX_GROUP];
    int n = 0;
    bool all_gemv, all_gemm, all_split;
    int st = gather_forward(args, count, segs, &n, &all_gemv, &all_gemm, &all_split);
    if (st) return st;
    *bytes = (n > 0 && all_split) ? bl::gemm_small_bytes(segs, n) : 0;
    return BL_OK;
}

int bitlinear_forward_grouped_ws(const bitlinear_forward_args *args, int count, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    return forward_grouped_impl(args, count, workspace, workspace_bytes, stream);
}

int bitlinear_forward_grouped_noalloc(const bitlinear_forward_args *args, int count, void *stream) {
    return forward_grouped_impl(args, count, nullptr, 0, stream, true);
}

namespace {
// Validates quant + forward entries and gathers the non-empty ones (fused:
// whether one decode launch takes them all; the other flags as for the
// grouped forward).
// b1: the packed buffers are layout b1 (binary codes, one bit each).
static int gather_quant_forward(const bitlinear_quant_forward_args *args, int count, bl::QFwdSeg *q, bl::FwdSeg *f,
                                int *n_out, bool *fused, bool *all_gemv, bool *all_gemm, bool *all_split,
                                bool b1 = false) {
    if (!args) return BL_ERR_NULL;
    if (count < 1 || count > BITLINEAR_MAX_GROUP) return BL_ERR_SHAPE;
    for (int i = 0; i < count; ++i) {
        const bitlinear_quant_forward_args &a = args[i];
        int st = shape_ok(a.N, a.K);
        if (st) return st;
        if (b1 && !bl::b1_ok(a.N, a.K)) return BL_ERR_SHAPE;
        if (a.M < 0 || a.M > kMaxDim) return BL_ERR_SHAPE;
        if (a.M == 0) continue;
        if (!a.packed || !a.gamma || !a.x || !a.xq || !a.x_scale || !a.y) return BL_ERR_NULL;
        if (!aligned16(a.packed) || !aligned16(a.gamma) || !aligned16(a.x) || !aligned16(a.xq) ||
            !aligned16(a.x_scale) || !aligned16(a.y) || (a.acc && !aligned16(a.acc)))
            return BL_ERR_ALIGN;
    }
    int n = 0;
    *fused = *all_gemv = *all_gemm = *all_split = true;
    for (int i = 0; i < count; ++i) {
        const bitlinear_quant_forward_args &a = args[i];
        if (a.M == 0) continue;
        f[n] = bl::FwdSeg{reinterpret_cast<const uint32_t *>(a.packed), a.gamma, bl::Layout::of(a.N, a.K), a.xq,
                          a.x_scale, a.M, a.y, a.acc, a.xq, a.x_scale};
        // entries that read one input into one pair of buffers quantise it once
        bool first = true;
        for (int j = 0; j < n; ++j)
            if (q[j].x == a.x && q[j].f.xq_out == a.xq && q[j].f.xs_out == a.x_scale && q[j].f.M == a.M &&
                q[j].f.L.K == a.K)
                first = false;
        q[n] = bl::QFwdSeg{f[n], a.x, first};
        *fused = *fused && (b1 ? bl::gemv_quant_b1_ok(a.N, a.K, a.M) : bl::gemv_quant_ok(f[n].L, a.M));
        *all_gemv = *all_gemv && bl::gemv_ok(f[n].L, a.M);
        *all_gemm = *all_gemm && a.M > bl::kGemvMaxM && bl::gemm_ok(f[n].L, a.M);
        *all_split = *all_split && a.M <= bl::kGemvMaxM && bl::gemm_ok(f[n].L, a.M);
        ++n;
    }
    *n_out = n;
    return BL_OK;
}
}  // namespace

namespace {
// A call the one-launch path does not take because an entry has more than
// 16 tokens, whose weights are small: the same kernel on 16-token slices of
// each entry, up to kMaxSeg slices.  The quant and the contraction are both
// per token, so each slice's xq, x_scale, y and acc rows are exactly those
// of the whole entry; every slice reads the entry's codes again, which the
// byte bound keeps negligible (a single BitLinear 256 -> 512 at 32 tokens:
// 6.2 -> 3.9 us, one launch instead of two).  Every slice offset is a
// multiple of 16 rows, so the slices keep the entries' 16-byte alignment.
constexpr int64_t kSliceM = 16;
constexpr int64_t kSliceMaxBytes = 1 << 20;  // codes read, summed over the slices
bool slice_quant_forward(const bl::QFwdSeg *q, int n, bl::QFwdSeg *out, int *n_out) {
    int m = 0;
    int64_t bytes = 0;
    for (int i = 0; i < n; ++i) {
        const bl::FwdSeg &f = q[i].f;
        if (f.M <= kSliceM) return false;
        const int64_t slices = (f.M + kSliceM - 1) / kSliceM;
        if (m + slices > bl::kMaxSeg) return false;
        bytes += slices * f.L.bytes;
        if (bytes > kSliceMaxBytes) return false;
        for (int64_t c = 0; c < slices; ++c) {
            const int64_t m0 = c * kSliceM, mc = f.M - m0 < kSliceM ? f.M - m0 : kSliceM;
            if (!bl::gemv_quant_ok(f.L, mc)) return false;
            bl::FwdSeg g = f;
            g.M = mc;
            g.y = f.y + m0 * f.L.N;
            g.acc = f.acc ? f.acc + m0 * f.L.N : nullptr;
            g.xq_out = f.xq_out + m0 * f.L.K;
            g.xs_out = f.xs_out + m0;
            g.xq = g.xq_out;
            g.xs = g.xs_out;
            out[m++] = bl::QFwdSeg{g, q[i].x + m0 * f.L.K, q[i].write_q};
        }
    }
    *n_out = m;
    return m > 0;
}
}  // namespace

int bitlinear_quant_forward_workspace_bytes(const bitlinear_quant_forward_args *args, int count, size_t *bytes) {
    if (!bytes) return BL_ERR_NULL;
    bl::QFwdSeg q[BITLINEAR_MAX_GROUP];
    bl::FwdSeg f[BITLINEAR_MAX_GROUP];
    int n = 0;
    bool fused, all_gemv, all_gemm, all_split;
    int st = gather_quant_forward(args, count, q, f, &n, &fused, &all_gemv, &all_gemm, &all_split);
    if (st) return st;
    bl::QFwdSeg qs[bl::kMaxSeg];
    int ns = 0;
    const bool sliced = n > 0 && !fused && slice_quant_forward(q, n, qs, &ns);
    *bytes = (n > 0 && !fused && !sliced && all_split) ? bl::gemm_small_bytes(f, n) : 0;
    return BL_OK;
}

int bitlinear_quant_forward_grouped(const bitlinear_quant_forward_args *args, int count, float eps, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    if (!std::isfinite(eps) || !(eps > 0.0f)) {
        if (!args) return BL_ERR_NULL;
        return BL_ERR_VALUE;
    }
    bl::QFwdSeg q[BITLINEAR_MAX_GROUP];
    bl::FwdSeg f[BITLINEAR_MAX_GROUP];
    int n = 0;
    bool fused, all_gemv, all_gemm, all_split;
    int st = gather_quant_forward(args, count, q, f, &n, &fused, &all_gemv, &all_gemm, &all_split);
    if (st) return st;
    if (workspace && !aligned16(workspace)) return BL_ERR_ALIGN;
    bl::QFwdSeg qs[bl::kMaxSeg];
    int ns = 0;
    const bool sliced = n > 0 && !fused && slice_quant_forward(q, n, qs, &ns);
    const size_t need = (workspace && n > 0 && !fused && !sliced && all_split) ? bl::gemm_small_bytes(f, n) : 0;
    if (need > workspace_bytes) return BL_ERR_WORKSPACE;
    if (n == 0) return BL_OK;
    if ((st = check_device())) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fused) return launched(bl::launch_gemv_quant_multi(q, n, eps, s));
    if (sliced) return launched(bl::launch_gemv_quant_multi(qs, ns, eps, s));
    // otherwise: one quant launch per distinct input, then the forwards
    for (int i = 0; i < n; ++i) {
        if (!q[i].write_q) continue;
        st = launched(bl::launch_quant(q[i].x, f[i].M, f[i].L.K, eps, f[i].xq_out, f[i].xs_out, s));
        if (st) return st;
    }
    return dispatch_forward(f, n, all_gemv, all_gemm, all_split, workspace, s);
}

namespace {
int b1_shape_ok(int64_t N, int64_t K) {
    int st = shape_ok(N, K);
    if (st) return st;
    return bl::b1_ok(N, K) ? BL_OK : BL_ERR_SHAPE;
}

int forward_b1_impl(const bitlinear_forward_args *args, int count, void *stream) {
    if (!args) return BL_ERR_NULL;
    if (count < 1 || count > BITLINEAR_MAX_GROUP) return BL_ERR_SHAPE;
    int64_t wgs = 0;  // the launch's workgroups at one row block each: its grid must fit
    for (int i = 0; i < count; ++i) {
        int st = b1_shape_ok(args[i].N, args[i].K);
        if (st) return st;
        if ((st = forward_args_ok(args[i]))) return st;
        wgs += (args[i].N + 15) / 16 * ((args[i].M + 15) / 16);
    }
    if (wgs > kMaxDim - 1) return BL_ERR_SHAPE;
    int st = check_device();
    if (st) return st;
    bl::FwdSeg segs[BITLINEAR_MAX_GROUP];
    int n = 0;
    for (int i = 0; i < count; ++i) {
        const bitlinear_forward_args &a = args[i];
        if (a.M == 0) continue;
        segs[n++] = bl::FwdSeg{reinterpret_cast<const uint32_t *>(a.packed), a.gamma, bl::Layout::of(a.N, a.K), a.xq,
                               a.x_scale, a.M, a.y, a.acc};
    }
    if (n == 0) return BL_OK;
    return launched(bl::launch_forward_b1(segs, n, static_cast<hipStream_t>(stream)));
}
}  // namespace

int bitlinear_forward_grouped_dot4(const bitlinear_forward_args *args, int count, void *stream) {
    if (!args) return BL_ERR_NULL;
    if (count < 1 || count > BITLINEAR_MAX_GROUP) return BL_ERR_SHAPE;
    for (int i = 0; i < count; ++i) {
        int st = forward_args_ok(args[i]);
        if (st) return st;
        if (args[i].M > 0 && !bl::dot4_ok(bl::Layout::of(args[i].N, args[i].K), args[i].M)) return BL_ERR_SHAPE;
    }
    int st = check_device();
    if (st) return st;
    bl::FwdSeg segs[BITLINEAR_MAX_GROUP];
    int n = 0;
    for (int i = 0; i < count; ++i) {
        const bitlinear_forward_args &a = args[i];
        if (a.M == 0) continue;
        segs[n++] = bl::FwdSeg{reinterpret_cast<const uint32_t *>(a.packed), a.gamma, bl::Layout::of(a.N, a.K), a.xq,
                               a.x_scale, a.M, a.y, a.acc};
    }
    if (n == 0) return BL_OK;
    return launched(bl::launch_gemv_dot4_multi(segs, n, static_cast<hipStream_t>(stream)));
}

int bitlinear_quant_forward_b1_grouped(const bitlinear_quant_forward_args *args, int count, float eps, void *stream) {
    if (!std::isfinite(eps) || !(eps > 0.0f)) {
        if (!args) return BL_ERR_NULL;
        return BL_ERR_VALUE;
    }
    bl::QFwdSeg q[BITLINEAR_MAX_GROUP];
    bl::FwdSeg f[BITLINEAR_MAX_GROUP];
    int n = 0;
    bool fused, all_gemv, all_gemm, all_split;
    int st = gather_quant_forward(args, count, q, f, &n, &fused, &all_gemv, &all_gemm, &all_split, true);
    if (st) return st;
    if (n == 0) return BL_OK;
    if ((st = check_device())) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fused) return launched(bl::launch_gemv_quant_multi(q, n, eps, s, true));
    for (int i = 0; i < n; ++i) {
        if (!q[i].write_q) continue;
        st = launched(bl::launch_quant(q[i].x, f[i].M, f[i].L.K, eps, f[i].xq_out, f[i].xs_out, s));
        if (st) return st;
    }
    return launched(bl::launch_forward_b1(f, n, s));
}

int bitlinear_packed_bytes_b1(int64_t N, int64_t K, size_t *bytes) {
    if (!bytes) return BL_ERR_NULL;
    int st = b1_shape_ok(N, K);
    if (st) return st;
    *bytes = (size_t)bl::b1_bytes(N, K);
    return BL_OK;
}

int bitlinear_pack_binary_b1(const float *W, int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                             uint8_t *packed_b1, float *beta, float *alpha, void *stream) {
    if (!W || !packed_b1 || !beta || !alpha) return BL_ERR_NULL;
    int st = b1_shape_ok(N, K);
    if (st) return st;
    if (!workspace) return BL_ERR_WORKSPACE;
    if (workspace_bytes < (size_t)bl::pack_partials(N * K) * sizeof(double)) return BL_ERR_WORKSPACE;
    if (!aligned16(W) || !aligned16(packed_b1) || !aligned16(beta) || !aligned16(alpha) || !aligned16(workspace))
        return BL_ERR_ALIGN;
    if ((st = check_device())) return st;
    return launched(bl::launch_pack_binary_b1(W, N, K, static_cast<double *>(workspace),
                                              reinterpret_cast<uint32_t *>(packed_b1), beta, alpha,
                                              static_cast<hipStream_t>(stream)));
}

int bitlinear_forward_b1(const uint8_t *packed_b1, const float *beta, int64_t N, int64_t K, const int8_t *xq,
                         const float *x_scale, int64_t M, uint16_t *y, int32_t *acc, void *stream) {
    int st = b1_shape_ok(N, K);
    if (st) return st;
    if (M < 0 || M > kMaxDim) return BL_ERR_SHAPE;
    if (M == 0) return BL_OK;
    const bitlinear_forward_args a{packed_b1, beta, N, K, xq, x_scale, M, y, acc};
    return forward_b1_impl(&a, 1, stream);
}

int bitlinear_forward_b1_grouped(const bitlinear_forward_args *args, int count, void *stream) {
    return forward_b1_impl(args, count, stream);
}

int bitlinear_flip_update(const float *w_prev, const float *w_curr, int64_t n, int32_t step,
                          int16_t *flip_count, int16_t *last_flip, void *stream) {
    if (n < 0) return BL_ERR_SHAPE;
    if (step < 1 || step > 32767) return BL_ERR_VALUE;
    if (n == 0) return BL_OK;
    if (!w_prev || !w_curr || !flip_count || !last_flip) return BL_ERR_NULL;
    if (!aligned16(w_prev) || !aligned16(w_curr) || !aligned16(flip_count) || !aligned16(last_flip))
        return BL_ERR_ALIGN;
    int st = check_device();
    if (st) return st;
    return launched(bl::launch_flip(w_prev, w_curr, n, step, flip_count, last_flip,
                                    static_cast<hipStream_t>(stream)));
}

int bitlinear_pack_transposed(const uint8_t *packed, int64_t N, int64_t K, uint8_t *packed_t, void *stream) {
    int st = shape_ok(N, K);
    if (st) return st;
    if (!packed || !packed_t) return BL_ERR_NULL;
    if (!aligned16(packed) || !aligned16(packed_t)) return BL_ERR_ALIGN;
    if ((st = check_device())) return st;
    return launched(bl::launch_pack_t1(reinterpret_cast<const uint32_t *>(packed), N, K,
                                       reinterpret_cast<uint32_t *>(packed_t), static_cast<hipStream_t>(stream)));
}

int bitlinear_backward_input(const uint8_t *packed_t, const float *gamma, int64_t N, int64_t K, const uint16_t *dy,
                             int64_t M, uint16_t *dx, int accumulate, void *stream) {
    int st = shape_ok(N, K);
    if (st) return st;
    if (M < 0 || M > kMaxDim) return BL_ERR_SHAPE;
    if (N % 8 != 0) return BL_ERR_SHAPE;
    if (M == 0) return BL_OK;
    if (!bl::dgrad_ok(M, N, K)) return BL_ERR_SHAPE;
    if (!packed_t || !gamma || !dy || !dx) return BL_ERR_NULL;
    if (!aligned16(packed_t) || !aligned16(gamma) || !aligned16(dy) || !aligned16(dx)) return BL_ERR_ALIGN;
    if ((st = check_device())) return st;
    return launched(bl::launch_dgrad(reinterpret_cast<const uint32_t *>(packed_t), gamma, N, K, dy, M, dx,
                                     accumulate, static_cast<hipStream_t>(stream)));
}

static_assert(BITLINEAR_MAX_BACKWARD_GROUP == bl::kDgradMaxEntries, "one kernel argument slot per entry");

int bitlinear_backward_input_grouped(const bitlinear_backward_args *args, int count, int64_t K, int64_t M,
                                     uint16_t *dx, int accumulate, void *stream) {
    if (!args) return BL_ERR_NULL;
    if (count < 1 || count > BITLINEAR_MAX_BACKWARD_GROUP) return BL_ERR_SHAPE;
    if (K <= 0 || K > BITLINEAR_MAX_K || M < 0 || M > kMaxDim) return BL_ERR_SHAPE;
    for (int e = 0; e < count; ++e) {
        const bitlinear_backward_args &g = args[e];
        int st = shape_ok(g.N, K);
        if (st) return st;
        if (g.N % 8 != 0 || !bl::dgrad_ok(M, g.N, K)) return BL_ERR_SHAPE;
    }
    if (M == 0) return BL_OK;
    if (!dx) return BL_ERR_NULL;
    if (!aligned16(dx)) return BL_ERR_ALIGN;
    for (int e = 0; e < count; ++e) {
        const bitlinear_backward_args &g = args[e];
        if (!g.packed_t || !g.gamma || !g.dy) return BL_ERR_NULL;
        if (!aligned16(g.packed_t) || !aligned16(g.gamma) || !aligned16(g.dy)) return BL_ERR_ALIGN;
    }
    int st = check_device();
    if (st) return st;
    bl::DgradGroupArgs a{};
    int64_t items = 0;
    for (int e = 0; e < count; ++e) {
        const bl::Layout Lt = bl::Layout::of(K, args[e].N);
        bl::DgradEntry &d = a.e[e];
        d.packed_t = reinterpret_cast<const uint32_t *>(args[e].packed_t);
        d.gamma = args[e].gamma;
        d.dy = args[e].dy;
        d.N = args[e].N;
        d.KB = Lt.NB;
        d.KFt = Lt.KF;
        d.groups = (int)Lt.NG;
        items += Lt.NG;
    }
    if (items >= ((int64_t)1 << 31)) return BL_ERR_SHAPE;
    a.dx = dx;
    a.M = M;
    a.K = K;
    a.count = count;
    a.accumulate = accumulate ? 1 : 0;
    return launched(bl::launch_dgrad_grouped(a, static_cast<hipStream_t>(stream)));
}

int bitlinear_adamw_step(float *W, const float *grad, float *exp_avg, float *exp_avg_sq, int64_t n, int32_t t,
                         double lr, double beta1, double beta2, double eps, double weight_decay, int16_t *flip_count,
                         int16_t *last_flip, void *stream) {
    if (n < 0) return BL_ERR_SHAPE;
    if (t < 1) return BL_ERR_VALUE;
    if (!std::isfinite(lr) || lr < 0.0 || !std::isfinite(weight_decay) || weight_decay < 0.0) return BL_ERR_VALUE;
    if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0)) return BL_ERR_VALUE;
    if (!std::isfinite(eps) || eps < 0.0) return BL_ERR_VALUE;
    if ((flip_count == nullptr) != (last_flip == nullptr)) return BL_ERR_NULL;
    if (flip_count && t > 32767) return BL_ERR_VALUE;
    if (n == 0) return BL_OK;
    if (!W || !grad || !exp_avg || !exp_avg_sq) return BL_ERR_NULL;
    if (!aligned16(W) || !aligned16(grad) || !aligned16(exp_avg) || !aligned16(exp_avg_sq) ||
        (flip_count && (!aligned16(flip_count) || !aligned16(last_flip))))
        return BL_ERR_ALIGN;
    int st = check_device();
    if (st) return st;
    return launched(bl::launch_adamw_flip(W, grad, exp_avg, exp_avg_sq, n, t, lr, beta1, beta2, eps, weight_decay,
                                          flip_count, last_flip, static_cast<hipStream_t>(stream)));
}

int bitlinear_flip_stats(const int16_t *flip_count, const int16_t *last_flip, int64_t n, int32_t T,
                         float *sign_age, float *flip_rate, void *stream) {
    if (n < 0) return BL_ERR_SHAPE;
    if (T < 1 || T > 32767) return BL_ERR_VALUE;
    if (n == 0) return BL_OK;
    if (!flip_count || !last_flip || !sign_age || !flip_rate) return BL_ERR_NULL;
    if (!aligned16(flip_count) || !aligned16(last_flip) || !aligned16(sign_age) || !aligned16(flip_rate))
        return BL_ERR_ALIGN;
    int st = check_device();
    if (st) return st;
    return launched(bl::launch_flip_stats(flip_count, last_flip, n, T, sign_age, flip_rate,
                                          static_cast<hipStream_t>(stream)));
}

const char *bitlinear_strerror(int status) {
    switch (status) {
        case BL_OK: return "ok";
        case BL_ERR_NULL: return "a required pointer is NULL";
        case BL_ERR_SHAPE: return "a size is out of range or inconsistent";
        case BL_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
        case BL_ERR_VALUE: return "eps or step out of range";
        case BL_ERR_DEVICE: return "the HIP runtime reported an error";
        case BL_ERR_ARCH: return "the current device is not gfx950";
        case BL_ERR_WORKSPACE: return "workspace missing or too small";
        case BL_ERR_SCRATCH: return "the call needs more than the library's fixed scratch (BITLINEAR_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int bitlinear_layout_version(void) { return BITLINEAR_LAYOUT_VERSION; }

}  // extern "C"
