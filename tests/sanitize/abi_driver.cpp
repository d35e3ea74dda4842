// Drives the host-side validation of every C-ABI entry point
// (include/bitlinear.h) for a build of the library whose host code carries
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitize.py
// builds it with the sanitizers on the host pass only and runs this).
// Every call here is rejected on the host before any device work, except the
// calls of valid_calls(), which run only when argv[1] == "nodevice" (the
// caller has established that the HIP runtime sees no device): they pass
// validation and must stop at the device check.  No pointer below is ever
// dereferenced on the host; they are fake device addresses.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/bitlinear.h"

static int failures = 0;
#define EXPECT(call, want)                                                                      \
    do {                                                                                        \
        int got_ = (call);                                                                      \
        if (got_ != (want)) {                                                                   \
            std::fprintf(stderr, "line %d: %s returned %d, want %d\n", __LINE__, #call, got_, (int)(want)); \
            ++failures;                                                                         \
        }                                                                                       \
    } while (0)

static void *const A = reinterpret_cast<void *>(uintptr_t(1) << 20);   // aligned fake address
static void *const A2 = reinterpret_cast<void *>(uintptr_t(3) << 20);
static void *const U = reinterpret_cast<void *>((uintptr_t(1) << 20) + 4);  // misaligned

template <typename T>
static T *p(void *v) { return static_cast<T *>(v); }

static void size_queries() {
    size_t b = 0;
    EXPECT(bitlinear_packed_bytes(17, 65, &b), BL_OK);
    if (b != 2 * 2 * 256) ++failures;
    EXPECT(bitlinear_packed_bytes(0, 65, &b), BL_ERR_SHAPE);
    EXPECT(bitlinear_packed_bytes(1, BITLINEAR_MAX_K + 1, &b), BL_ERR_SHAPE);
    EXPECT(bitlinear_packed_bytes(INT64_MAX, INT64_MAX, &b), BL_ERR_SHAPE);
    EXPECT(bitlinear_packed_bytes(1, 1, nullptr), BL_ERR_NULL);
    EXPECT(bitlinear_pack_workspace_bytes(3, 5, &b), BL_OK);
    EXPECT(bitlinear_pack_workspace_bytes(-3, 5, &b), BL_ERR_SHAPE);
    EXPECT(bitlinear_pack_workspace_bytes(3, 5, nullptr), BL_ERR_NULL);
    EXPECT(bitlinear_packed_bytes_b1(17, 192, &b), BL_OK);
    if (b != 2 * 2 * 256) ++failures;
    EXPECT(bitlinear_packed_bytes_b1(17, 96, &b), BL_ERR_SHAPE);
    EXPECT(bitlinear_packed_bytes_b1(1, BITLINEAR_B1_MAX_K + 64, &b), BL_ERR_SHAPE);
    EXPECT(bitlinear_packed_bytes_b1(INT64_MAX / 2, 64, &b), BL_ERR_SHAPE);
    EXPECT(bitlinear_packed_bytes_b1(1, 64, nullptr), BL_ERR_NULL);
    for (int s = -8; s <= 1; ++s)
        if (!bitlinear_strerror(s) || !std::strlen(bitlinear_strerror(s))) ++failures;
    if (bitlinear_layout_version() != BITLINEAR_LAYOUT_VERSION) ++failures;
}

static void invalid_calls() {
    const float *W = p<const float>(A);
    // pack
    EXPECT(bitlinear_pack_weights(nullptr, 4, 4, 1e-5f, A, 1 << 20, p<uint8_t>(A), p<float>(A), nullptr), BL_ERR_NULL);
    EXPECT(bitlinear_pack_weights(W, 0, 4, 1e-5f, A, 1 << 20, p<uint8_t>(A), p<float>(A), nullptr), BL_ERR_SHAPE);
    EXPECT(bitlinear_pack_weights(W, 4, 4, -1.0f, A, 1 << 20, p<uint8_t>(A), p<float>(A), nullptr), BL_ERR_VALUE);
    EXPECT(bitlinear_pack_weights(W, 4, 4, 1e-5f, nullptr, 1 << 20, p<uint8_t>(A), p<float>(A), nullptr), BL_ERR_WORKSPACE);
    EXPECT(bitlinear_pack_weights(W, 4, 4, 1e-5f, A, 0, p<uint8_t>(A), p<float>(A), nullptr), BL_ERR_WORKSPACE);
    EXPECT(bitlinear_pack_weights(W, 4, 4, 1e-5f, A, 1 << 20, p<uint8_t>(U), p<float>(A), nullptr), BL_ERR_ALIGN);
    EXPECT(bitlinear_pack_binary(W, 4, 4, A, 1 << 20, p<uint8_t>(A), p<float>(A), nullptr, nullptr), BL_ERR_NULL);
    EXPECT(bitlinear_pack_binary(W, 4, -4, A, 1 << 20, p<uint8_t>(A), p<float>(A), p<float>(A2), nullptr), BL_ERR_SHAPE);
    EXPECT(bitlinear_pack_binary_b1(W, 4, 96, A, 1 << 20, p<uint8_t>(A), p<float>(A), p<float>(A2), nullptr),
           BL_ERR_SHAPE);
    EXPECT(bitlinear_pack_binary_b1(W, 4, 64, A, 0, p<uint8_t>(A), p<float>(A), p<float>(A2), nullptr),
           BL_ERR_WORKSPACE);
    EXPECT(bitlinear_forward_b1(p<uint8_t>(A), W, 8, 80, p<int8_t>(A), W, 2, p<uint16_t>(A2), nullptr, nullptr),
           BL_ERR_SHAPE);
    EXPECT(bitlinear_forward_b1(p<uint8_t>(A), W, 8, 64, p<int8_t>(U), W, 2, p<uint16_t>(A2), nullptr, nullptr),
           BL_ERR_ALIGN);
    EXPECT(bitlinear_forward_b1_grouped(nullptr, 1, nullptr), BL_ERR_NULL);
    bitlinear_forward_args d5 = {p<uint8_t>(A), W, 16, 64, p<int8_t>(A), W, 5, p<uint16_t>(A2), nullptr};
    EXPECT(bitlinear_forward_grouped_dot4(&d5, 1, nullptr), BL_ERR_SHAPE);
    EXPECT(bitlinear_forward_grouped_dot4(nullptr, 1, nullptr), BL_ERR_NULL);
    bitlinear_quant_forward_args qb = {p<uint8_t>(A), W, 64, 96, p<uint16_t>(A), 4, p<int8_t>(A2), p<float>(A2),
                                       p<uint16_t>(A2), nullptr};
    EXPECT(bitlinear_quant_forward_b1_grouped(&qb, 1, 1e-5f, nullptr), BL_ERR_SHAPE);
    EXPECT(bitlinear_quant_forward_b1_grouped(nullptr, 1, 1e-5f, nullptr), BL_ERR_NULL);
    bitlinear_pack_args pa[2];
    std::memset(pa, 0, sizeof pa);
    pa[0] = bitlinear_pack_args{W, 4, 4, 1e-5f, A, 1 << 20, p<uint8_t>(A), p<float>(A), nullptr};
    pa[1] = pa[0];
    pa[1].K = 0;
    EXPECT(bitlinear_pack_weights_grouped(pa, 2, nullptr), BL_ERR_SHAPE);
    EXPECT(bitlinear_pack_weights_grouped(pa, 0, nullptr), BL_ERR_SHAPE);
    EXPECT(bitlinear_pack_weights_grouped(pa, BITLINEAR_MAX_PACK_GROUP + 1, nullptr), BL_ERR_SHAPE);
    EXPECT(bitlinear_pack_weights_grouped(nullptr, 1, nullptr), BL_ERR_NULL);
    pa[1] = pa[0];
    pa[1].packed_t = p<uint8_t>(U);
    EXPECT(bitlinear_pack_weights_grouped(pa, 2, nullptr), BL_ERR_ALIGN);
    EXPECT(bitlinear_pack_transposed(nullptr, 4, 4, p<uint8_t>(A), nullptr), BL_ERR_NULL);
    // quant
    const uint16_t *x = p<const uint16_t>(A);
    EXPECT(bitlinear_quant_act(x, -1, 4, 1e-5f, p<int8_t>(A), p<float>(A2), nullptr), BL_ERR_SHAPE);
    EXPECT(bitlinear_quant_act(x, 2, 4, 0.0f, p<int8_t>(A), p<float>(A2), nullptr), BL_ERR_VALUE);
    EXPECT(bitlinear_quant_act(x, 2, 4, 1e-5f, nullptr, p<float>(A2), nullptr), BL_ERR_NULL);
    EXPECT(bitlinear_quant_act(x, 2, 4, 1e-5f, p<int8_t>(U), p<float>(A2), nullptr), BL_ERR_ALIGN);
    EXPECT(bitlinear_quant_act(nullptr, 0, 4, 1e-5f, nullptr, nullptr, nullptr), BL_OK);
    EXPECT(bitlinear_rmsnorm_quant_act(x, p<float>(U), 2, 4, 1e-6f, 1e-5f, p<int8_t>(A), p<float>(A2), nullptr),
           BL_ERR_ALIGN);
    EXPECT(bitlinear_rmsnorm_quant_act(x, nullptr, 2, 4, -1.0f, 1e-5f, p<int8_t>(A), p<float>(A2), nullptr),
           BL_ERR_VALUE);
    // forward
    const uint8_t *pk = p<const uint8_t>(A);
    const float *g = p<const float>(A);
    EXPECT(bitlinear_forward(pk, g, 8, 0, p<int8_t>(A), g, 2, p<uint16_t>(A2), nullptr, nullptr), BL_ERR_SHAPE);
    EXPECT(bitlinear_forward(pk, g, 8, 8, p<int8_t>(A), g, -2, p<uint16_t>(A2), nullptr, nullptr), BL_ERR_SHAPE);
    EXPECT(bitlinear_forward(pk, g, 8, 8, p<int8_t>(A), g, 2, nullptr, nullptr, nullptr), BL_ERR_NULL);
    EXPECT(bitlinear_forward(pk, g, 8, 8, p<int8_t>(A), g, 2, p<uint16_t>(A2), p<int32_t>(U), nullptr), BL_ERR_ALIGN);
    EXPECT(bitlinear_forward(nullptr, nullptr, 8, 8, nullptr, nullptr, 0, nullptr, nullptr, nullptr), BL_OK);
    bitlinear_forward_args fa[BITLINEAR_MAX_GROUP + 1];
    for (auto &a : fa) a = bitlinear_forward_args{pk, g, 64, 64, p<int8_t>(A), g, 4, p<uint16_t>(A2), nullptr};
    EXPECT(bitlinear_forward_grouped(fa, BITLINEAR_MAX_GROUP + 1, nullptr), BL_ERR_SHAPE);
    EXPECT(bitlinear_forward_grouped(fa, 0, nullptr), BL_ERR_SHAPE);
    EXPECT(bitlinear_forward_grouped(nullptr, 1, nullptr), BL_ERR_NULL);
    fa[1].K = BITLINEAR_MAX_K + 1;
    EXPECT(bitlinear_forward_grouped(fa, 2, nullptr), BL_ERR_SHAPE);
    fa[1].K = 64;
    size_t ws = 0;
    EXPECT(bitlinear_forward_workspace_bytes(fa, 2, nullptr), BL_ERR_NULL);
    EXPECT(bitlinear_forward_workspace_bytes(fa, 2, &ws), BL_OK);
    // a decode batch whose cut launch needs a workspace
    bitlinear_forward_args big = {pk, g, 8192, 28672, p<int8_t>(A), g, 32, p<uint16_t>(A2), nullptr};
    EXPECT(bitlinear_forward_workspace_bytes(&big, 1, &ws), BL_OK);
    if (ws == 0) ++failures;
    EXPECT(bitlinear_forward_grouped_ws(&big, 1, A, ws - 1, nullptr), BL_ERR_WORKSPACE);
    EXPECT(bitlinear_forward_grouped_ws(&big, 1, U, ws, nullptr), BL_ERR_ALIGN);
    // no-allocation forward, quant + forward
    EXPECT(bitlinear_forward_grouped_noalloc(nullptr, 1, nullptr), BL_ERR_NULL);
    EXPECT(bitlinear_forward_grouped_noalloc(fa, 0, nullptr), BL_ERR_SHAPE);
    bitlinear_quant_forward_args qa[2];
    qa[0] = bitlinear_quant_forward_args{pk, g, 64, 64, p<const uint16_t>(A), 4, p<int8_t>(A2), p<float>(A2),
                                        p<uint16_t>(A2), nullptr};
    qa[1] = qa[0];
    qa[1].x = p<const uint16_t>(U);
    EXPECT(bitlinear_quant_forward_grouped(qa, 2, 1e-5f, nullptr, 0, nullptr), BL_ERR_ALIGN);
    EXPECT(bitlinear_quant_forward_grouped(qa, 1, 0.0f, nullptr, 0, nullptr), BL_ERR_VALUE);
    EXPECT(bitlinear_quant_forward_grouped(qa, 0, 1e-5f, nullptr, 0, nullptr), BL_ERR_SHAPE);
    qa[1] = qa[0];
    qa[1].xq = nullptr;
    EXPECT(bitlinear_quant_forward_grouped(qa, 2, 1e-5f, nullptr, 0, nullptr), BL_ERR_NULL);
    // backward
    EXPECT(bitlinear_backward_input(pk, g, 60, 32, x, 4, p<uint16_t>(A2), 0, nullptr), BL_ERR_SHAPE);
    EXPECT(bitlinear_backward_input(pk, g, 64, 32, x, 4, nullptr, 0, nullptr), BL_ERR_NULL);
    bitlinear_backward_args ba[BITLINEAR_MAX_BACKWARD_GROUP + 1];
    for (auto &b : ba) b = bitlinear_backward_args{pk, g, 64, x};
    EXPECT(bitlinear_backward_input_grouped(ba, BITLINEAR_MAX_BACKWARD_GROUP + 1, 32, 4, p<uint16_t>(A2), 0, nullptr),
           BL_ERR_SHAPE);
    ba[1].dy = p<const uint16_t>(U);
    EXPECT(bitlinear_backward_input_grouped(ba, 2, 32, 4, p<uint16_t>(A2), 0, nullptr), BL_ERR_ALIGN);
    // tracker and optimiser
    EXPECT(bitlinear_flip_update(W, W, 8, 0, p<int16_t>(A), p<int16_t>(A2), nullptr), BL_ERR_VALUE);
    EXPECT(bitlinear_flip_update(W, W, -8, 5, p<int16_t>(A), p<int16_t>(A2), nullptr), BL_ERR_SHAPE);
    EXPECT(bitlinear_flip_update(W, nullptr, 8, 5, p<int16_t>(A), p<int16_t>(A2), nullptr), BL_ERR_NULL);
    float *Wm = p<float>(A);
    EXPECT(bitlinear_adamw_step(Wm, W, Wm, Wm, 8, 0, 1e-3, 0.9, 0.999, 1e-8, 0.1, nullptr, nullptr, nullptr),
           BL_ERR_VALUE);
    EXPECT(bitlinear_adamw_step(Wm, W, Wm, Wm, 8, 1, 1e-3, 1.0, 0.999, 1e-8, 0.1, nullptr, nullptr, nullptr),
           BL_ERR_VALUE);
    EXPECT(bitlinear_adamw_step(Wm, W, Wm, Wm, 8, 1, 1e-3, 0.9, 0.999, 1e-8, 0.1, p<int16_t>(A), nullptr, nullptr),
           BL_ERR_NULL);
    EXPECT(bitlinear_flip_stats(p<int16_t>(A), p<int16_t>(A2), 8, 0, Wm, Wm, nullptr), BL_ERR_VALUE);
}

// Calls that pass validation; with no device they must end at the device
// check, before any launch.
static void valid_calls() {
    const float *W = p<const float>(A);
    const int want = BL_ERR_DEVICE;
    EXPECT(bitlinear_pack_weights(W, 4, 4, 1e-5f, A2, 1 << 20, p<uint8_t>(A), p<float>(A2), nullptr), want);
    EXPECT(bitlinear_quant_act(p<uint16_t>(A), 2, 4, 1e-5f, p<int8_t>(A2), p<float>(A), nullptr), want);
    EXPECT(bitlinear_forward(p<uint8_t>(A), W, 8, 8, p<int8_t>(A), W, 2, p<uint16_t>(A2), nullptr, nullptr), want);
    EXPECT(bitlinear_flip_update(W, W, 8, 5, p<int16_t>(A), p<int16_t>(A2), nullptr), want);
    bitlinear_quant_forward_args qa = {p<uint8_t>(A), W, 64, 64, p<uint16_t>(A), 4, p<int8_t>(A2), p<float>(A2),
                                       p<uint16_t>(A2), nullptr};
    EXPECT(bitlinear_quant_forward_grouped(&qa, 1, 1e-5f, nullptr, 0, nullptr), want);
    bitlinear_forward_args fa = {p<uint8_t>(A), W, 8192, 28672, p<int8_t>(A), W, 64, p<uint16_t>(A2), nullptr};
    EXPECT(bitlinear_forward_grouped_noalloc(&fa, 1, nullptr), want);
    EXPECT(bitlinear_pack_binary_b1(W, 4, 64, A2, 1 << 20, p<uint8_t>(A), p<float>(A2), p<float>(A2), nullptr), want);
    EXPECT(bitlinear_forward_b1(p<uint8_t>(A), W, 8, 64, p<int8_t>(A), W, 2, p<uint16_t>(A2), nullptr, nullptr), want);
    EXPECT(bitlinear_forward_b1_grouped(&fa, 1, nullptr), want);
    bitlinear_forward_args f1 = {p<uint8_t>(A), W, 8192, 28672, p<int8_t>(A), W, 1, p<uint16_t>(A2), nullptr};
    EXPECT(bitlinear_forward_grouped_dot4(&f1, 1, nullptr), want);
    bitlinear_quant_forward_args qb = {p<uint8_t>(A), W, 64, 64, p<uint16_t>(A), 1, p<int8_t>(A2), p<float>(A2),
                                       p<uint16_t>(A2), nullptr};
    EXPECT(bitlinear_quant_forward_b1_grouped(&qb, 1, 1e-5f, nullptr), want);
}

int main(int argc, char **argv) {
    size_queries();
    invalid_calls();
    if (argc > 1 && std::strcmp(argv[1], "nodevice") == 0) valid_calls();
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("abi sanitizer driver: clean\n");
    return 0;
}
