/*
 * CPU oracle for the BitNet b1.58 BitLinear forward path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the path computes.  Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg may load it; the product library never
 * does, and it shares no code, header or table with the GPU kernels.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -fPIC -shared
 * (no fast-math: every floating-point step below is one IEEE operation,
 * rounded to nearest even, in the precision written).
 *
 * Sources (all BitNet pages; cited by page title and section):
 *  [P1] "Which 1-Bit Weights Can You Trust?", Methodology
 *  [P2] "1-bit & Ternary LLMs (BitNet b1.58)", How it works (BitNet and
 *       BitNet b1.58 equations), Training pseudocode
 *  [P3] "What 1.58 Bits Actually Changes", Three values / low-bit linear path
 *  [P4] "building a 1-bit llm, part 1", What one bit actually buys you
 *       (add / subtract / skip rule)
 *  [P5] "1.58 bits: what BitNet promised and what it required", Three values
 *
 * Readings where the pages leave a step open (each listed in the design
 * notes): eps is an argument; rounding is half-to-even; gamma is summed in
 * fp64 and rounded once to fp32; W/(gamma+eps) is one correctly rounded fp32
 * division; activations use s = 127 / max(absmax, eps) and clip to
 * [-127, 127]; the rescale is acc * gamma / s; the tracker compares
 * sgn() in {-1, 0, +1} of the latent weights and saturates at 32767.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_RANGE -1   /* accumulator out of int32, or bad argument   */
#define ORACLE_ERR_CODE -2    /* packed buffer holds a code that is never written */
#define ORACLE_ERR_NONFINITE -3

/* Threads used by the contraction loops (each output is computed by one
 * thread, in the order written; threads only split the list of outputs). */
int oracle_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* ------------------------------------------------------------------ gamma
 * [P2] BitNet b1.58 equation: gamma is the mean absolute value over all
 * n*m entries of the weight matrix; [P3] and [P5] (Three values) restate it
 * as the one per-matrix average of |W| that the weights are divided by.
 * One scale per tensor.  Summed in row-major order in fp64, divided in fp64,
 * rounded once to fp32. */
double oracle_abs_sum(const float *W, int64_t count)
{
    double s = 0.0;
    for (int64_t i = 0; i < count; ++i)
        s += fabs((double)W[i]);
    return s;
}

float oracle_gamma(const float *W, int64_t N, int64_t K)
{
    double s = oracle_abs_sum(W, N * K);
    return (float)(s / ((double)N * (double)K));
}

/* ------------------------------------------------- binary BitNet weights
 * [P2] How it works, BitNet (binary) equations: alpha = mean of W over the
 * whole matrix, W~ = Sign(W - alpha) in {-1, +1}, beta = mean |W| (the
 * per-tensor scale, ||W||_1 / nm).  The forward is the same contraction with
 * beta in place of gamma.  Sign(0) is not given; since the set is {-1, +1},
 * W = alpha is read as +1: the code is +1 exactly when W >= alpha (compared
 * directly, no rounded difference).  alpha and beta: fp64 sums in row-major
 * order, fp64 divide, one rounding to fp32. */
int oracle_binarise(const float *W, int64_t N, int64_t K, int8_t *codes, float *alpha, float *beta)
{
    double s = 0.0;
    for (int64_t i = 0; i < N * K; ++i) {
        if (!isfinite(W[i]))
            return ORACLE_ERR_NONFINITE;
        s += (double)W[i];
    }
    float a = (float)(s / ((double)N * (double)K));
    *alpha = a;
    *beta = oracle_gamma(W, N, K);
    for (int64_t i = 0; i < N * K; ++i)
        codes[i] = W[i] >= a ? 1 : -1;
    return ORACLE_OK;
}

/* ------------------------------------------------------------- ternarise
 * [P2] BitNet b1.58 equation: W~ = RoundClip(W / (gamma + eps), -1, 1),
 * RoundClip(x, a, b) = max(a, min(b, round(x))).  [P3] says the same in
 * words: nearest integer, then clamp into [-1, +1].
 * round(): nearest, ties to even (nearbyintf under the default mode). */
int oracle_ternarise(const float *W, int64_t N, int64_t K, float gamma, float eps, int8_t *codes)
{
    float d = gamma + eps;
    for (int64_t i = 0; i < N * K; ++i) {
        if (!isfinite(W[i]))
            return ORACLE_ERR_NONFINITE;
        if (d == 0.0f) {            /* only when gamma == 0 and eps == 0: W is all zeros */
            codes[i] = 0;
            continue;
        }
        float r = W[i] / d;
        float q = nearbyintf(r);
        if (q > 1.0f) q = 1.0f;
        if (q < -1.0f) q = -1.0f;
        codes[i] = (int8_t)q;
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------- layout
 * Packed layout, version 1 (the library owns it; [P3] notes that the
 * matrices and the computation that consumes them must agree on it).
 *   2-bit codes: 0 -> 00, +1 -> 01, -1 -> 11; 10 is never written.
 *   N padded to a multiple of 16, K to a multiple of 64, padding code 00.
 *   Fragment = 16 rows x 64 columns = 64 dwords.  Dword lam (0..63) of a
 *   fragment holds row (lam mod 16) and columns 16*(lam div 16) + t,
 *   t = 0..15, code t at bit 8*(t mod 4) + 2*(t div 4).
 *   Along K, fragments form groups of up to four; in a group of G fragments
 *   dword lam of fragment f sits at position lam*G + f.  Groups follow each
 *   other along K; 16-row blocks follow each other along N.
 * This is written from that description alone. */
static void layout_dims(int64_t N, int64_t K, int64_t *NB, int64_t *KF)
{
    *NB = (N + 15) / 16;
    *KF = (K + 63) / 64;
}

int64_t oracle_packed_bytes(int64_t N, int64_t K)
{
    int64_t NB, KF;
    layout_dims(N, K, &NB, &KF);
    return NB * KF * 256;
}

/* byte offset and bit shift of code (n, k) */
static void layout_locate(int64_t KF, int64_t n, int64_t k, int64_t *byte, int *shift)
{
    int64_t nb = n / 16, r = n % 16;
    int64_t kf = k / 64, kk = k % 64;
    int64_t chunk = kk / 16, t = kk % 16;
    int64_t lam = r + 16 * chunk;
    int64_t g = kf / 4, f = kf % 4;
    int64_t G = KF - 4 * g;
    if (G > 4) G = 4;
    int64_t dword = nb * KF * 64 + g * 256 + lam * G + f;
    int bit = (int)(8 * (t % 4) + 2 * (t / 4));
    *byte = dword * 4 + bit / 8;
    *shift = bit % 8;
}

int oracle_encode(const int8_t *codes, int64_t N, int64_t K, uint8_t *packed)
{
    int64_t NB, KF;
    layout_dims(N, K, &NB, &KF);
    memset(packed, 0, (size_t)oracle_packed_bytes(N, K));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int8_t c = codes[n * K + k];
            unsigned bits;
            if (c == 0) bits = 0u;
            else if (c == 1) bits = 1u;
            else if (c == -1) bits = 3u;
            else return ORACLE_ERR_CODE;
            int64_t byte;
            int shift;
            layout_locate(KF, n, k, &byte, &shift);
            packed[byte] |= (uint8_t)(bits << shift);
        }
    return ORACLE_OK;
}

/* Decode the real N x K codes; any 10 code, or any nonzero padding bit,
 * is an error. */
int oracle_decode(const uint8_t *packed, int64_t N, int64_t K, int8_t *codes)
{
    int64_t NB, KF;
    layout_dims(N, K, &NB, &KF);
    int64_t Np = NB * 16, Kp = KF * 64;
    for (int64_t n = 0; n < Np; ++n)
        for (int64_t k = 0; k < Kp; ++k) {
            int64_t byte;
            int shift;
            layout_locate(KF, n, k, &byte, &shift);
            unsigned bits = (packed[byte] >> shift) & 3u;
            if (n >= N || k >= K) {
                if (bits != 0u) return ORACLE_ERR_CODE;
                continue;
            }
            if (bits == 2u) return ORACLE_ERR_CODE;
            codes[n * K + k] = (int8_t)(bits == 0u ? 0 : (bits == 1u ? 1 : -1));
        }
    return ORACLE_OK;
}

/* ---------------------------------------------- transposed layout t1
 * The backward pass contracts over the output features n, so it reads the
 * codes as the K x N matrix c^T (row k, column n).  Layout t1 is layout v1's
 * geometry applied to that K x N matrix (16-row blocks along K, 64-column
 * fragments along N, groups of up to four fragments, dword lam of fragment
 * f at lam*G + f; lane lam holds row lam % 16 and the 16 columns starting at
 * 16*(lam/16)), with its own order inside a dword: column t of the 16 sits at
 * bit 14 - t for even t and at bit 31 - t for odd t, so columns 2p and 2p+1
 * occupy bits 14-2p and 30-2p.  Codes as in v1: 0 -> 00, +1 -> 01, -1 -> 11.
 * Written from that description alone. */
static void layout_t1_locate(int64_t KFt, int64_t k, int64_t n, int64_t *byte, int *shift)
{
    int64_t kb = k / 16, r = k % 16;
    int64_t nf = n / 64, nn = n % 64;
    int64_t chunk = nn / 16, t = nn % 16;
    int64_t lam = r + 16 * chunk;
    int64_t g = nf / 4, f = nf % 4;
    int64_t G = KFt - 4 * g;
    if (G > 4) G = 4;
    int64_t dword = kb * KFt * 64 + g * 256 + lam * G + f;
    int bit = (int)((t % 2 == 0) ? 14 - t : 31 - t);
    *byte = dword * 4 + bit / 8;
    *shift = bit % 8;
}

/* codes [N][K] -> layout t1 of c^T; the buffer has oracle_packed_bytes(K, N) bytes */
int oracle_encode_t1(const int8_t *codes, int64_t N, int64_t K, uint8_t *packed_t)
{
    int64_t KB, KFt;
    layout_dims(K, N, &KB, &KFt);
    memset(packed_t, 0, (size_t)oracle_packed_bytes(K, N));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int8_t c = codes[n * K + k];
            unsigned bits;
            if (c == 0) bits = 0u;
            else if (c == 1) bits = 1u;
            else if (c == -1) bits = 3u;
            else return ORACLE_ERR_CODE;
            int64_t byte;
            int shift;
            layout_t1_locate(KFt, k, n, &byte, &shift);
            packed_t[byte] |= (uint8_t)(bits << shift);
        }
    return ORACLE_OK;
}

/* layout t1 -> codes [N][K]; code 10 or a nonzero padding code is an error */
int oracle_decode_t1(const uint8_t *packed_t, int64_t N, int64_t K, int8_t *codes)
{
    int64_t KB, KFt;
    layout_dims(K, N, &KB, &KFt);
    int64_t Kp = KB * 16, Np = KFt * 64;
    for (int64_t k = 0; k < Kp; ++k)
        for (int64_t n = 0; n < Np; ++n) {
            int64_t byte;
            int shift;
            layout_t1_locate(KFt, k, n, &byte, &shift);
            unsigned bits = (packed_t[byte] >> shift) & 3u;
            if (n >= N || k >= K) {
                if (bits != 0u) return ORACLE_ERR_CODE;
                continue;
            }
            if (bits == 2u) return ORACLE_ERR_CODE;
            codes[n * K + k] = (int8_t)(bits == 0u ? 0 : (bits == 1u ? 1 : -1));
        }
    return ORACLE_OK;
}

/* ------------------------------------------- one-bit layout b1 (binary)
 * Binary weights ([P2] How it works, BitNet equations: W~ = Sign(W - alpha))
 * take only -1 and +1, so one bit each carries them: bit 0 is +1, bit 1 is
 * -1.  Layout b1 (library-owned, like v1):
 *   K must be a multiple of 64 (there is no zero code to pad a fragment);
 *   N is padded to a multiple of 16 and K to a multiple of 128, padding
 *   bits 0.
 *   Pair = 16 rows x 128 columns = 64 dwords.  Dword lam (0..63) of pair P
 *   holds row (lam mod 16) and, for h = 0 and 1, the 16 columns
 *   128*P + 64*h + 16*(lam div 16) + t, t = 0..15, code t of half h at bit
 *   8*(t mod 4) + 7 - (4*h + t div 4).
 *   Along K, pairs form groups of up to four; in a group of G pairs dword
 *   lam of pair f sits at position lam*G + f.  Groups follow each other
 *   along K; 16-row blocks follow each other along N.
 * Written from that description alone. */
static int b1_dims(int64_t N, int64_t K, int64_t *NB, int64_t *KP)
{
    if (K % 64 != 0) return ORACLE_ERR_RANGE;
    *NB = (N + 15) / 16;
    *KP = (K + 127) / 128;
    return ORACLE_OK;
}

/* bytes of layout b1, or -1 when K is not a multiple of 64 */
int64_t oracle_packed_bytes_b1(int64_t N, int64_t K)
{
    int64_t NB, KP;
    if (b1_dims(N, K, &NB, &KP) != ORACLE_OK) return -1;
    return NB * KP * 256;
}

static void b1_locate(int64_t KP, int64_t n, int64_t k, int64_t *byte, int *shift)
{
    int64_t nb = n / 16, r = n % 16;
    int64_t P = k / 128, kk = k % 128;
    int64_t h = kk / 64, c = kk % 64;
    int64_t chunk = c / 16, t = c % 16;
    int64_t lam = r + 16 * chunk;
    int64_t g = P / 4, f = P % 4;
    int64_t G = KP - 4 * g;
    if (G > 4) G = 4;
    int64_t dword = nb * KP * 64 + g * 256 + lam * G + f;
    int bit = (int)(8 * (t % 4) + 7 - (4 * h + t / 4));
    *byte = dword * 4 + bit / 8;
    *shift = bit % 8;
}

/* codes [N][K] in {-1, +1} -> layout b1 */
int oracle_encode_b1(const int8_t *codes, int64_t N, int64_t K, uint8_t *packed)
{
    int64_t NB, KP;
    if (b1_dims(N, K, &NB, &KP) != ORACLE_OK) return ORACLE_ERR_RANGE;
    memset(packed, 0, (size_t)oracle_packed_bytes_b1(N, K));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int8_t c = codes[n * K + k];
            if (c != 1 && c != -1) return ORACLE_ERR_CODE;
            if (c == 1) continue;
            int64_t byte;
            int shift;
            b1_locate(KP, n, k, &byte, &shift);
            packed[byte] |= (uint8_t)(1u << shift);
        }
    return ORACLE_OK;
}

/* layout b1 -> codes [N][K]; a set padding bit is an error */
int oracle_decode_b1(const uint8_t *packed, int64_t N, int64_t K, int8_t *codes)
{
    int64_t NB, KP;
    if (b1_dims(N, K, &NB, &KP) != ORACLE_OK) return ORACLE_ERR_RANGE;
    int64_t Np = NB * 16, Kp = KP * 128;
    for (int64_t n = 0; n < Np; ++n)
        for (int64_t k = 0; k < Kp; ++k) {
            int64_t byte;
            int shift;
            b1_locate(KP, n, k, &byte, &shift);
            unsigned bit = (packed[byte] >> shift) & 1u;
            if (n >= N || k >= K) {
                if (bit) return ORACLE_ERR_CODE;
                continue;
            }
            codes[n * K + k] = (int8_t)(bit ? -1 : 1);
        }
    return ORACLE_OK;
}

/* ------------------------------------ base-3 layout t3 (decode prototype)
 * Ternary codes five to a byte ([P2] What it is: about 1.6 bits per weight
 * in practice).  Layout t3, the operand arrangement of the decode
 * prototype that was measured against layout v1 (the library does not
 * write or read it):
 *   K must be a multiple of 320, N is padded to a multiple of 16 (padding
 *   rows hold code 0).  A group is 16 rows x 320 columns = five 64-column
 *   fragments, 1024 bytes; byte 16*lam + t (lam 0..63, t 0..15) of a group
 *   holds row lam % 16 and, for f = 0..4, column 64*f + 16*(lam / 16) + t
 *   of the group as the base-3 digit (code + 1) of weight 3^f.
 *   Groups follow each other along K, 16-row blocks along N:
 *   ceil(N/16) * (K/320) * 1024 bytes. */
int64_t oracle_packed_bytes_t3(int64_t N, int64_t K)
{
    if (K % 320 != 0) return -1;
    return (N + 15) / 16 * (K / 320) * 1024;
}

static void t3_locate(int64_t K, int64_t n, int64_t k, int64_t *byte, int *power)
{
    int64_t nb = n / 16, r = n % 16;
    int64_t g = k / 320, kk = k % 320;
    int64_t f = kk / 64, c = kk % 64;
    int64_t lam = r + 16 * (c / 16), t = c % 16;
    *byte = (nb * (K / 320) + g) * 1024 + 16 * lam + t;
    *power = (int)f;
}

int oracle_encode_t3(const int8_t *codes, int64_t N, int64_t K, uint8_t *packed)
{
    if (K % 320 != 0) return ORACLE_ERR_RANGE;
    static const int pw[5] = {1, 3, 9, 27, 81};
    int64_t bytes = oracle_packed_bytes_t3(N, K);
    /* every padding row digit is 1 (code 0): 1+3+9+27+81 = 121 */
    memset(packed, 121, (size_t)bytes);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int8_t c = codes[n * K + k];
            if (c < -1 || c > 1) return ORACLE_ERR_CODE;
            int64_t byte;
            int p;
            t3_locate(K, n, k, &byte, &p);
            /* the byte holds digit 1 for this weight so far: replace it */
            packed[byte] = (uint8_t)(packed[byte] + (c + 1 - 1) * pw[p]);
        }
    return ORACLE_OK;
}

/* layout t3 -> codes [N][K]; a byte above 242 or a padding row with a
 * nonzero code is an error */
int oracle_decode_t3(const uint8_t *packed, int64_t N, int64_t K, int8_t *codes)
{
    if (K % 320 != 0) return ORACLE_ERR_RANGE;
    int64_t Np = (N + 15) / 16 * 16;
    for (int64_t n = 0; n < Np; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t byte;
            int p;
            t3_locate(K, n, k, &byte, &p);
            unsigned v = packed[byte];
            if (v > 242) return ORACLE_ERR_CODE;
            for (int i = 0; i < p; ++i) v /= 3;
            int c = (int)(v % 3) - 1;
            if (n >= N) {
                if (c != 0) return ORACLE_ERR_CODE;
                continue;
            }
            codes[n * K + k] = (int8_t)c;
        }
    return ORACLE_OK;
}

/* ------------------------------------------------------ activation quant
 * [P2] BitNet equation: activations are scaled per token by Q_b / gamma_x
 * with gamma_x the absmax of the token, then clipped; b1.58 drops the zero
 * point and scales to the symmetric 8-bit range ([P2] b1.58 paragraph;
 * [P3] low-bit linear path: per-token scaling into int8, no zero point; [P5]).
 * s = 127 / max(absmax, eps), q = clip(round(x * s), -127, 127), round half
 * to even.  x arrives as bf16 bit patterns; bf16 -> fp32 is exact. */
static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

int oracle_quant_act(const uint16_t *x, int64_t M, int64_t K, float eps, int8_t *q, float *s)
{
    for (int64_t m = 0; m < M; ++m) {
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = bf16_to_f32(x[m * K + k]);
            if (!isfinite(v))
                return ORACLE_ERR_NONFINITE;
            float av = fabsf(v);
            if (av > a) a = av;
        }
        float sm = 127.0f / fmaxf(a, eps);
        s[m] = sm;
        for (int64_t k = 0; k < K; ++k) {
            float v = bf16_to_f32(x[m * K + k]) * sm;
            float r = nearbyintf(v);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[m * K + k] = (int8_t)r;
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------- RMSNorm before the quant
 * [P2] How it works: the BitLinear forward quantises the normalised input
 * (LayerNorm in BitNet; b1.58 takes the LLaMA-style RMSNorm), and the QAT
 * pseudocode quantises layernorm(x).  The pages give no RMSNorm formula; the
 * plain one is used: r = 1 / sqrt(mean_k x_k^2 + eps_norm), y_k = x_k * r * g_k
 * with a per-channel gain g (1 when absent).  Then the activation quant above
 * applied to y.  Everything in fp64 (this is the definition, not the GPU's
 * arithmetic): s = 127 / max(max_k |y_k|, eps), v_k = y_k * s,
 * q_k = clip(round(v_k), -127, 127), ties to even.  Outputs q, s rounded once
 * to fp32, and (if v is not NULL) the fp64 v for rounding-window checks. */
int oracle_rmsnorm_quant_act(const uint16_t *x, const float *gain, int64_t M, int64_t K, float eps_norm,
                             float eps, int8_t *q, float *s, double *v)
{
    if (K <= 0)
        return ORACLE_ERR_RANGE;
    for (int64_t m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double xv = (double)bf16_to_f32(x[m * K + k]);
            if (!isfinite(xv))
                return ORACLE_ERR_NONFINITE;
            ss += xv * xv;
        }
        double den = ss / (double)K + (double)eps_norm;
        double r = den > 0.0 ? 1.0 / sqrt(den) : 0.0;   /* an all-zero row with eps_norm = 0 stays 0 */
        double a = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double g = gain ? (double)gain[k] : 1.0;
            double y = (double)bf16_to_f32(x[m * K + k]) * r * g;
            if (fabs(y) > a) a = fabs(y);
        }
        double sm = 127.0 / (a > (double)eps ? a : (double)eps);
        s[m] = (float)sm;
        for (int64_t k = 0; k < K; ++k) {
            double g = gain ? (double)gain[k] : 1.0;
            double vv = (double)bf16_to_f32(x[m * K + k]) * r * g * sm;
            if (v) v[m * K + k] = vv;
            double rr = nearbyint(vv);
            if (rr > 127.0) rr = 127.0;
            if (rr < -127.0) rr = -127.0;
            q[m * K + k] = (int8_t)rr;
        }
    }
    return ORACLE_OK;
}

/* ----------------------------------------------------------- contraction
 * [P4] w = +1 adds the input, w = -1 subtracts it, w = 0 skips it; [P3] the
 * same add / subtract / skip rule; [P2] the inner product of the ternary
 * weights and the int8 activations is integer work.
 * acc[m][n] = sum over k of the branch rule applied to q[m][k]; y = x W^T
 * ([P2] BitLinear is a drop-in nn.Linear).  Accumulated in int64 and checked
 * to fit int32. */
int oracle_contract(const int8_t *q, const int8_t *codes, int64_t M, int64_t N, int64_t K,
                    int32_t *acc)
{
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t mn = 0; mn < M * N; ++mn) {
        int64_t m = mn / N, n = mn % N;
        const int8_t *qr = q + m * K;
        const int8_t *cr = codes + n * K;
        int64_t a = 0;
        for (int64_t k = 0; k < K; ++k) {
            if (cr[k] == 1)
                a += qr[k];
            else if (cr[k] == -1)
                a -= qr[k];
        }
        if (a > INT32_MAX || a < INT32_MIN)
            bad = 1;
        acc[mn] = (int32_t)a;
    }
    return bad ? ORACLE_ERR_RANGE : ORACLE_OK;
}

/* Same rule for a list of (m, n) pairs, for sampled checks at full size. */
int oracle_contract_pairs(const int8_t *q, const int8_t *codes, int64_t K, const int64_t *m_idx,
                          const int64_t *n_idx, int64_t P, int32_t *acc)
{
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t p = 0; p < P; ++p) {
        const int8_t *qr = q + m_idx[p] * K;
        const int8_t *cr = codes + n_idx[p] * K;
        int64_t a = 0;
        for (int64_t k = 0; k < K; ++k) {
            if (cr[k] == 1)
                a += qr[k];
            else if (cr[k] == -1)
                a -= qr[k];
        }
        if (a > INT32_MAX || a < INT32_MIN)
            bad = 1;
        acc[p] = (int32_t)a;
    }
    return bad ? ORACLE_ERR_RANGE : ORACLE_OK;
}

/* -------------------------------------------------------------- epilogue
 * [P2] the only floating-point work left is one rescale per output; for
 * b1.58 the rescale multiplies by the weight scale gamma and undoes the
 * activation scale s.  y = acc * gamma / s, computed in fp64 and rounded
 * once to fp32 (the fp32 reference a bf16 result is compared against). */
void oracle_epilogue(const int32_t *acc, int64_t M, int64_t N, float gamma, const float *s,
                     float *y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = (float)((double)acc[m * N + n] * (double)gamma / (double)s[m]);
}

/* ------------------------------------------- STE backward to the input
 * [P2] Training (shadow weights and the straight-through estimator): the
 * forward uses the ternary weights, the backward treats both quantisers as
 * the identity, so the layer is y = x W_eff^T with W_eff = gamma * W~ and the
 * gradient with respect to its input is dx = dy W_eff, i.e.
 *   dx[m][k] = gamma * sum over n of dy[m][n] * code[n][k]
 * (the add / subtract / skip rule again, now over the output features).
 * dy arrives as bf16 bit patterns (exact in fp64).  ref is that value in
 * fp64 (the sum over n in order; exact whenever the terms' exponents span
 * fewer than 53 - 8 bits), plus dx_prev when given (the gradients of layers
 * that share an input add up); mag = gamma * sum |dy * code| bounds the
 * cancellation.  dx is the bf16 result under the reading that the fp64 sum
 * is rounded to fp32, multiplied by gamma in fp32, dx_prev added in fp32,
 * and the total rounded to bf16 (nearest even); when every partial sum is
 * exact in fp32 (small integer dy) any fp32 implementation must give these
 * bits.  Any output pointer may be NULL. */
static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

int oracle_backward_input(const uint16_t *dy, const int8_t *codes, int64_t M, int64_t N, int64_t K, float gamma,
                          const uint16_t *dx_prev, double *ref, double *mag, uint16_t *dx)
{
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t mk = 0; mk < M * K; ++mk) {
        int64_t m = mk / K, k = mk % K;
        double s = 0.0, a = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            int8_t c = codes[n * K + k];
            double d = (double)bf16_to_f32(dy[m * N + n]);
            if (c == 1) {
                s += d;
                a += fabs(d);
            } else if (c == -1) {
                s -= d;
                a += fabs(d);
            } else if (c != 0) {
                bad = 1;
            }
        }
        double prev = dx_prev ? (double)bf16_to_f32(dx_prev[mk]) : 0.0;
        if (ref) ref[mk] = (double)gamma * s + prev;
        if (mag) mag[mk] = (double)gamma * a;
        if (dx) {
            float v = (float)s * gamma;
            if (dx_prev) v = v + bf16_to_f32(dx_prev[mk]);
            dx[mk] = f32_to_bf16_rne(v);
        }
    }
    return bad ? ORACLE_ERR_CODE : ORACLE_OK;
}

/* -------------------------------------- optimiser step + tracker (QAT)
 * [P2] Training: the optimiser steps the full-precision shadow weights (the
 * STE passes the gradient of the ternary weights straight to them); [P1]
 * Experimental Setup: AdamW with decoupled weight decay; [P1] Methodology:
 * the tracker compares each weight's sign before and after the step.  AdamW
 * is the published algorithm (Loshchilov & Hutter).  The hyperparameters
 * are doubles; every scalar coefficient is formed in fp64 and rounded once
 * to fp32: decay = 1 - lr*wd, a1 = 1 - b1, a2 = 1 - b2,
 * step = lr / (1 - b1^t), rc2 = sqrt(1 - b2^t).  Per weight, in fp32:
 *   w = W * decay
 *   m = b1*m + a1*g;   v = b2*v + a2*(g*g)
 *   W = w - step * (m / (sqrt(v) / rc2 + eps))
 * and, if counters are given, where sgn(W_before) != sgn(W_after) the flip
 * count goes up (saturating) and last_flip = t. */
static int sgn_step(float v) { return (v > 0.0f) - (v < 0.0f); }

int oracle_adamw_flip(float *W, const float *g, float *m, float *v, int64_t n, int32_t t, double lr, double b1,
                      double b2, double eps, double wd, int16_t *flip_count, int16_t *last_flip)
{
    if (t < 1)
        return ORACLE_ERR_RANGE;
    const float decay = (float)(1.0 - lr * wd);
    const float fb1 = (float)b1, fb2 = (float)b2, a1 = (float)(1.0 - b1), a2 = (float)(1.0 - b2);
    const float step = (float)(lr / (1.0 - pow(b1, (double)t)));
    const float rc2 = (float)sqrt(1.0 - pow(b2, (double)t));
    const float feps = (float)eps;
    for (int64_t i = 0; i < n; ++i) {
        float w0 = W[i];
        float w = w0 * decay;
        float mi = fb1 * m[i] + a1 * g[i];
        float vi = fb2 * v[i] + a2 * (g[i] * g[i]);
        float den = sqrtf(vi) / rc2 + feps;
        w = w - step * (mi / den);
        W[i] = w;
        m[i] = mi;
        v[i] = vi;
        if (flip_count && last_flip && sgn_step(w0) != sgn_step(w)) {
            flip_count[i] = (int16_t)(flip_count[i] == 32767 ? 32767 : flip_count[i] + 1);
            last_flip[i] = (int16_t)t;
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------- tracker read-out
 * [P1] Methodology: after T steps two values per weight come from the two
 * counters, sign age and flip rate.  The formulas did not survive on the
 * page; its special cases did (a weight that never flipped has sign age 1, a
 * weight that never moved has flip rate 0).  Read as
 *   sign_age = (T - last_flip) / T,   flip_rate = flip_count / T,
 * each an fp64 quotient rounded once to fp32.  [P1] Results call a weight
 * that never flipped after warm-up "locked" (flip_count == 0).  The
 * reliability score and the other three classes have no formula or
 * threshold on the page and are not computed. */
int oracle_flip_stats(const int16_t *flip_count, const int16_t *last_flip, int64_t n, int32_t T,
                      float *sign_age, float *flip_rate)
{
    if (T < 1)
        return ORACLE_ERR_RANGE;
    for (int64_t i = 0; i < n; ++i) {
        sign_age[i] = (float)(((double)T - (double)last_flip[i]) / (double)T);
        flip_rate[i] = (float)((double)flip_count[i] / (double)T);
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------ sign-flip tracker
 * [P1] Methodology: two INT16 counters per weight, both starting at zero;
 * after each step the sign of every weight is compared with its sign at the
 * previous step, and wherever it changed the flip count goes up by one and
 * the last-flip counter takes the current step number.
 * sgn() in {-1, 0, +1}; the count saturates at 32767. */
static int sgn(float v) { return (v > 0.0f) - (v < 0.0f); }

int oracle_flip_update(const float *prev, const float *curr, int64_t n, int32_t step,
                       int16_t *flip_count, int16_t *last_flip)
{
    if (step < 1 || step > 32767)
        return ORACLE_ERR_RANGE;
    for (int64_t i = 0; i < n; ++i) {
        if (sgn(prev[i]) != sgn(curr[i])) {
            int32_t c = (int32_t)flip_count[i] + 1;
            flip_count[i] = (int16_t)(c > 32767 ? 32767 : c);
            last_flip[i] = (int16_t)step;
        }
    }
    return ORACLE_OK;
}
