/*
 * bitlinear.h - C ABI of the MI355X (gfx950) BitNet b1.58 BitLinear library.
 *
 * The library computes the BitLinear forward path of BitNet b1.58:
 *   gamma = mean |W| over the whole weight matrix, codes = RoundClip(W /
 *   (gamma + eps), -1, 1)   ("1-bit & Ternary LLMs (BitNet b1.58)", How it
 *   works, BitNet b1.58 equations; "What 1.58 Bits Actually Changes", Three
 *   values);
 *   per-token absmax int8 activations with no zero point (same page, BitNet
 *   activation equation and the b1.58 paragraph that drops the zero point;
 *   "What 1.58 Bits Actually Changes", low-bit linear path);
 *   an integer contraction in which +1 adds, -1 subtracts and 0 skips
 *   ("building a 1-bit llm, part 1", What one bit actually buys you),
 *   accumulated in int32;
 *   one float rescale per output back to bf16 ("1-bit & Ternary LLMs",
 *   BitLinear forward equation).
 * plus the optional sign-flip tracker update ("Which 1-Bit Weights Can You
 * Trust?", Methodology).
 *
 * Conventions for every entry point
 *  - Pointers are DEVICE pointers (memory the caller allocated on the current
 *    HIP device) unless stated otherwise; scalars and sizes are host values.
 *  - The caller owns every buffer.  The library allocates nothing and is
 *    reentrant; the only state it keeps between calls is per device and
 *    written once: whether the device is gfx950, one-time kernel attributes,
 *    and the address of the fixed device scratch of
 *    bitlinear_forward_grouped_noalloc (all thread-safe, idempotent).  That
 *    scratch's contents are shared by that entry point's calls on a device
 *    (see there); no other entry point touches it.
 *  - All device work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream).  Nothing synchronises; results are ready when the stream is.
 *  - Every argument is validated on the host before any device work; on
 *    error nothing is enqueued and a negative bl_status is returned.  A launch
 *    failure is BL_ERR_DEVICE.  Non-finite inputs are a precondition the
 *    kernels do not check.
 *  - Device pointers must be 16-byte aligned (BL_ERR_ALIGN otherwise).
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BL_OK = 0,
    BL_ERR_NULL = -1,      /* a required pointer is NULL                        */
    BL_ERR_SHAPE = -2,     /* a size is <= 0, too large, or inconsistent         */
    BL_ERR_ALIGN = -3,     /* a device pointer is not 16-byte aligned            */
    BL_ERR_VALUE = -4,     /* eps negative or not finite, step out of [1, 32767] */
    BL_ERR_DEVICE = -5,    /* the HIP runtime reported an error                  */
    BL_ERR_ARCH = -6,      /* the current device is not gfx950                   */
    BL_ERR_WORKSPACE = -7, /* workspace missing or smaller than required         */
    BL_ERR_SCRATCH = -8    /* needs more than the fixed scratch of a no-allocation call */
} bl_status;

/* Largest K accepted: |acc| <= 127 * K must fit in int32. */
#define BITLINEAR_MAX_K 16909320
/* Version of the packed weight layout described below. */
#define BITLINEAR_LAYOUT_VERSION 1

/*
 * Packed ternary weight layout, version 1.  Owned by the library ("What 1.58
 * Bits Actually Changes", low-bit linear path: the stored matrices and the
 * computation that consumes them have to agree on the representation).
 *  - 2-bit codes: 0 -> 00, +1 -> 01, -1 -> 11.  10 is never written.
 *  - N is padded to a multiple of 16 and K to a multiple of 64; padding
 *    holds code 00.  Size in bytes: ceil(N/16) * ceil(K/64) * 256.
 *  - A fragment is 16 rows x 64 columns (64 dwords).  Dword `lam` (0..63)
 *    of a fragment holds row lam % 16 and the 16 columns starting at
 *    16 * (lam / 16); column t of those 16 sits at bit 8*(t%4) + 2*(t/4).
 *    (One dword per lane of a 64-wide wave: the operand shape of
 *    v_mfma_i32_16x16x64_i8, and four int8 dwords after unpacking.)
 *  - Along K the fragments of a 16-row block form groups of up to four; in a
 *    group of G fragments, dword lam of fragment f is at position lam*G + f
 *    (one 16-byte load per lane for a full group).  Groups follow each other
 *    along K, and 16-row blocks follow each other along N.
 */

/*
 * Layout t1: the codes of an N x K weight arranged for the backward pass,
 * which contracts over the output features n.  It is layout v1's geometry
 * applied to the transposed K x N code matrix (row k, column n): K padded to
 * a multiple of 16 and N to a multiple of 64 with code 00, fragments of 16
 * rows x 64 columns, groups of up to four fragments, dword lam of fragment f
 * at lam*G + f.  Only the order inside a dword differs: column t (0..15) of
 * the dword's 16 columns sits at bit 14 - t for even t and at bit 31 - t for
 * odd t, so columns 2p and 2p+1 sit at bits 14-2p and 30-2p, and a left
 * shift by 2p and a mask leave the bf16 pair (2*code, 2*code) of an MFMA
 * operand.  Codes as in v1.  Size: ceil(K/16) * ceil(N/64) * 256 bytes,
 * i.e. bitlinear_packed_bytes(K, N).
 */

/* Host-only.  Size of the packed buffer for an N x K weight. */
int bitlinear_packed_bytes(int64_t N, int64_t K, size_t *bytes);

/* Host-only.  Size of the workspace bitlinear_pack_weights needs (fp64
 * partial sums of |W|). */
int bitlinear_pack_workspace_bytes(int64_t N, int64_t K, size_t *bytes);

/*
 * Ternarise and pack one weight tensor ("1-bit & Ternary LLMs (BitNet
 * b1.58)", BitNet b1.58 equations; "What 1.58 Bits Actually Changes", Three
 * values; "1.58 bits: what BitNet promised and what it required", Three values
 * per weight).
 *   W        [N][K] fp32, row-major (nn.Linear: out x in).  Read only.
 *   eps      >= 0, finite; added to gamma in the divisor (typically 1e-5).
 *   workspace, workspace_bytes  device scratch of at least
 *            bitlinear_pack_workspace_bytes(N, K) bytes.
 *   packed   bitlinear_packed_bytes(N, K) bytes, written in layout v1.
 *   gamma    [1] fp32, written: mean |W| summed in fp64 in a fixed order and
 *            rounded once to fp32 (gamma excludes eps).
 * Codes: clip(rint(W / fp32(gamma + eps)), -1, 1) with a correctly rounded
 * fp32 division and ties to even; gamma + eps == 0 gives code 0.
 */
int bitlinear_pack_weights(const float *W, int64_t N, int64_t K, float eps, void *workspace,
                           size_t workspace_bytes, uint8_t *packed, float *gamma, void *stream);

/*
 * Several weight tensors packed in one call (all the BitLinear weights of a
 * model, re-packed after every optimiser step in quantisation-aware training;
 * "1-bit & Ternary LLMs (BitNet b1.58)", Training: the ternary projection is
 * recomputed from the shadow weights each step).  Each entry means exactly
 * what the same arguments mean to bitlinear_pack_weights and gets the same
 * bytes and gamma; the tensors share three launches per 16 entries instead
 * of three each, and one more for the entries that also ask for layout t1
 * (the codes for bitlinear_backward_input).
 *   args   HOST array of `count` entries, 1 <= count <= BITLINEAR_MAX_PACK_GROUP;
 *          read during the call only.  Every entry is validated before anything
 *          is enqueued; entries must not share a workspace, packed or gamma buffer.
 */
#define BITLINEAR_MAX_PACK_GROUP 64

typedef struct {
    const float *W;          /* [N][K] fp32 */
    int64_t N, K;
    float eps;
    void *workspace;         /* bitlinear_pack_workspace_bytes(N, K) bytes */
    size_t workspace_bytes;
    uint8_t *packed;         /* bitlinear_packed_bytes(N, K) bytes, written */
    float *gamma;            /* [1], written */
    uint8_t *packed_t;       /* optional: bitlinear_packed_bytes(K, N) bytes, written in
                                layout t1 (as bitlinear_pack_transposed) when non-NULL */
} bitlinear_pack_args;

int bitlinear_pack_weights_grouped(const bitlinear_pack_args *args, int count, void *stream);

/*
 * Binary BitNet weights ("1-bit & Ternary LLMs (BitNet b1.58)", How it
 * works, BitNet equations: W~ = Sign(W - alpha) with alpha = mean W, scale
 * beta = mean |W|), stored in packed layout v1 as the codes +1 / -1 so that
 * bitlinear_forward (with beta in place of gamma) and the grouped forward
 * run them unchanged.
 *   W, N, K, workspace, workspace_bytes  as for bitlinear_pack_weights.
 *   packed   bitlinear_packed_bytes(N, K) bytes, written.
 *   beta     [1] fp32, written: mean |W| (fp64 sum, one rounding).
 *   alpha    [1] fp32, written: mean W (fp64 sum, one rounding).
 * Code +1 exactly where W >= alpha (Sign(0) read as +1: the set is {-1, +1}),
 * -1 elsewhere; padding holds code 0.
 */
int bitlinear_pack_binary(const float *W, int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                          uint8_t *packed, float *beta, float *alpha, void *stream);

/*
 * Per-token absmax int8 activation quantisation, no zero point ("1-bit &
 * Ternary LLMs", BitNet activation equation and the b1.58 paragraph; "What
 * 1.58 Bits Actually Changes", low-bit linear path).
 *   x        [M][K] bf16 bit patterns, row-major.  Read only.
 *   eps      > 0 floor on the absmax (typically 1e-5); finite.
 *   xq       [M][K] int8, written: clip(rint(x * s_m), -127, 127).
 *   x_scale  [M] fp32, written: s_m = 127 / max(max_k |x[m][k]|, eps), a
 *            correctly rounded fp32 division.
 */
int bitlinear_quant_act(const uint16_t *x, int64_t M, int64_t K, float eps, int8_t *xq,
                        float *x_scale, void *stream);

/*
 * RMSNorm fused into the activation quant: the step right before the
 * BitLinear contraction ("1-bit & Ternary LLMs (BitNet b1.58)", How it works:
 * the forward quantises the normalised input, LayerNorm in BitNet, the
 * LLaMA-style RMSNorm in b1.58; the QAT pseudocode quantises layernorm(x)).
 *   x        [M][K] bf16 bit patterns, row-major.  Read only.
 *   gain     [K] fp32 per-channel gain g, or NULL for g = 1.  Read only.
 *   eps_norm >= 0, finite: y = x * g / sqrt(mean_k x_k^2 + eps_norm)
 *            (a row of zeros with eps_norm = 0 gives y = 0).
 *   eps      > 0, finite: floor on max|y| as in bitlinear_quant_act.
 *   xq       [M][K] int8, written: clip(rint(y * s_m), -127, 127).
 *   x_scale  [M] fp32, written: s_m = 127 / max(max_k |y_k|, eps), to be
 *            passed to bitlinear_forward with xq.
 * The codes do not depend on the per-token norm factor (absmax quantisation
 * ignores a positive per-token scale), so they are computed from x * g in
 * fp32; the norm factor, from an fp64 sum of squares, enters x_scale only.
 * Without a gain the codes equal bitlinear_quant_act's bit for bit.
 */
int bitlinear_rmsnorm_quant_act(const uint16_t *x, const float *gain, int64_t M, int64_t K, float eps_norm,
                                float eps, int8_t *xq, float *x_scale, void *stream);

/*
 * BitLinear forward: y = x W^T with ternary weights and int8 activations
 * ("1-bit & Ternary LLMs", BitLinear forward equation: integer inner product,
 * then one float rescale per output; "building a 1-bit llm, part 1", What
 * one bit actually buys you: +1 adds, -1 subtracts, 0 skips).
 *   packed, gamma  output of bitlinear_pack_weights for an N x K weight.
 *   xq, x_scale    output of bitlinear_quant_act for [M][K] activations.
 *   y        [M][N] bf16 bit patterns, written: round-to-nearest-even of
 *            acc[m][n] * (gamma / x_scale[m]) evaluated in fp32.
 *   acc      optional [M][N] int32, written when non-NULL with the exact
 *            integer accumulators sum_k xq[m][k] * code[n][k].
 * K <= BITLINEAR_MAX_K.  M, N >= 1.
 */
int bitlinear_forward(const uint8_t *packed, const float *gamma, int64_t N, int64_t K,
                      const int8_t *xq, const float *x_scale, int64_t M, uint16_t *y,
                      int32_t *acc, void *stream);

/*
 * Several independent BitLinear forwards in one call, e.g. the Q, K and V
 * projections of a transformer layer (which read the same tokens), or the
 * gate and up projections of its SwiGLU block ("1-bit & Ternary LLMs",
 * b1.58 adopts LLaMA-style blocks whose linear layers are all BitLinear).
 * Each entry means exactly what the same arguments mean to
 * bitlinear_forward; the results are identical to `count` separate calls.
 * The entries share one launch when every entry has K % 16 == 0 and either
 * every entry has 1 <= M <= 64 (decode: one stream of weight bytes instead
 * of `count` short ones) or every entry has M > 64 (prefill: one grid of
 * output tiles large enough to fill the GPU); otherwise they are launched
 * one after another on `stream`.
 *   args   HOST array of `count` entries, 1 <= count <= BITLINEAR_MAX_GROUP;
 *          read during the call only.
 * No entry's y or acc may overlap any buffer of another entry.  Every entry
 * is validated before anything is enqueued.
 */
#define BITLINEAR_MAX_GROUP 8

typedef struct {
    const uint8_t *packed;  /* bitlinear_pack_weights output for an N x K weight */
    const float *gamma;     /* [1] */
    int64_t N, K;
    const int8_t *xq;       /* [M][K] */
    const float *x_scale;   /* [M] */
    int64_t M;
    uint16_t *y;            /* [M][N] bf16 bits, written */
    int32_t *acc;           /* optional [M][N] int32, written when non-NULL */
} bitlinear_forward_args;

int bitlinear_forward_grouped(const bitlinear_forward_args *args, int count, void *stream);

/*
 * The grouped forward with a caller workspace for batches of a few tokens
 * (decode with 14..64 tokens per call).  Same arguments, checks and results
 * as bitlinear_forward_grouped (bit for bit: the int32 sums are exact in any
 * order); the workspace lets the contraction over K (the integer inner
 * product of "1-bit & Ternary LLMs", BitLinear forward equation) be cut into
 * runs that different workgroups compute and a second launch adds up, so
 * that a call with few output rows still spreads over the whole GPU.
 *   workspace        device scratch of workspace_bytes bytes, 16-byte
 *                    aligned, overlapping no argument of the call; its
 *                    contents on entry do not matter and are undefined
 *                    afterwards.  NULL: exactly bitlinear_forward_grouped.
 *   workspace_bytes  at least bitlinear_forward_workspace_bytes for the same
 *                    entries, else BL_ERR_WORKSPACE (nothing enqueued).
 * The library uses the workspace only while the call's work runs on `stream`;
 * calls that may run at the same time need workspaces of their own.
 * bitlinear_forward_workspace_bytes is host-only: it validates the entries as
 * the forward does and writes the size the call needs, 0 when it takes no
 * workspace: outside 14..64 tokens, K % 16 != 0, output tiles enough to fill
 * the GPU without a cut, or, at 14..32 tokens, rows shorter than 64 groups of
 * 256 columns (the decode kernel is faster there).
 */
int bitlinear_forward_workspace_bytes(const bitlinear_forward_args *args, int count, size_t *bytes);
int bitlinear_forward_grouped_ws(const bitlinear_forward_args *args, int count, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * The activation quant and the forward in one call: for each entry, exactly
 * bitlinear_quant_act(x, M, K, eps, xq, x_scale) followed by
 * bitlinear_forward(packed, gamma, N, K, xq, x_scale, M, y, acc), with the
 * same xq, x_scale, y and acc bit for bit ("1-bit & Ternary LLMs (BitNet
 * b1.58)", BitLinear forward equation: the layer quantises its input per
 * token, contracts with the ternary weights, rescales; "building a 1-bit
 * llm, part 1", What one bit actually buys you: the activation quant, not the
 * contraction, is what a ternary layer pays for).  For decode (every entry
 * one token with K <= 32768, or 2..16 tokens with M * K <= 16384; K % 16 ==
 * 0) the whole call is one launch in which every workgroup quantises the
 * tokens itself.  So is a call whose entries have more than 16 tokens, cut
 * into at most 8 slices of 16 tokens that each meet those limits, when the
 * codes read over all slices stay within 1 MB (each slice reads its
 * entry's codes).  Otherwise it is one quant launch per distinct input
 * followed by the grouped forward.
 *   args   HOST array of `count` entries, 1 <= count <= BITLINEAR_MAX_GROUP,
 *          read during the call only.
 *   eps    > 0, finite: the floor on the per-token absmax (as for
 *          bitlinear_quant_act).
 * Entries may read the same x (Q, K and V): those that also give the same
 * xq and x_scale share them (written once).  Otherwise no output of an entry
 * may overlap a buffer of another entry.  Every entry is validated before
 * anything is enqueued; M = 0 entries are skipped.
 */
typedef struct {
    const uint8_t *packed;  /* bitlinear_pack_weights output for an N x K weight */
    const float *gamma;     /* [1] */
    int64_t N, K;
    const uint16_t *x;      /* [M][K] bf16 bits: the layer input before quantisation */
    int64_t M;
    int8_t *xq;             /* [M][K] int8, written (the activation codes) */
    float *x_scale;         /* [M] fp32, written */
    uint16_t *y;            /* [M][N] bf16 bits, written */
    int32_t *acc;           /* optional [M][N] int32, written when non-NULL */
} bitlinear_quant_forward_args;

/*
 * workspace, workspace_bytes: as for bitlinear_forward_grouped_ws, for the
 * calls that fall back to separate launches with 14..64 tokens (NULL: the
 * forward is never cut into runs).  bitlinear_quant_forward_workspace_bytes
 * (host-only) validates the entries as the call does and writes the size it
 * needs (0: none).
 */
int bitlinear_quant_forward_workspace_bytes(const bitlinear_quant_forward_args *args, int count, size_t *bytes);
int bitlinear_quant_forward_grouped(const bitlinear_quant_forward_args *args, int count, float eps, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * The grouped forward with the contraction on the vector ALUs instead of the
 * matrix cores: each code adds, subtracts or skips its activation ("building
 * a 1-bit llm, part 1", What one bit actually buys you), four at a time with
 * v_dot4_i32_i8, for decode with 1..4 tokens.  Same arguments, checks and
 * results as bitlinear_forward_grouped (bit for bit), plus BL_ERR_SHAPE
 * unless every non-empty entry has 1 <= M <= 4, K % 16 == 0, K <=
 * BITLINEAR_B1_MAX_K and packed and token buffers below 2 GB.  One launch for
 * all entries.  It leaves the matrix cores free for work that runs beside
 * it.  On its own it matches the matrix-core path at one token (both are
 * bound by the weight stream) and is slower from two tokens, where the
 * vector ALUs do 4 dot products per token per 16 codes.
 */
int bitlinear_forward_grouped_dot4(const bitlinear_forward_args *args, int count, void *stream);

/*
 * Binary weights one bit per code: packed layout b1.  Binary BitNet codes
 * ("1-bit & Ternary LLMs (BitNet b1.58)", How it works, BitNet equations:
 * W~ = Sign(W - alpha), scale beta) take only -1 and +1, so a bit holds one:
 * half the bytes of layout v1 for a decode step, whose time is the weight
 * bytes.  Owned by the library like v1:
 *  - bit 0 is +1, bit 1 is -1.  K must be a multiple of 64 (no code is
 *    neutral, so a fragment cannot be padded); N is padded to a multiple of
 *    16 and K to a multiple of 128 with bits 0.  Size in bytes:
 *    ceil(N/16) * ceil(K/128) * 256.
 *  - A pair is 16 rows x 128 columns (64 dwords).  Dword `lam` (0..63) of
 *    pair P holds row lam % 16 and, for h = 0 and 1, the 16 columns
 *    128*P + 64*h + 16*(lam / 16) + t, t = 0..15, with code t of half h at
 *    bit 8*(t % 4) + 7 - (4*h + t / 4).
 *  - Along K, pairs form groups of up to four; in a group of G pairs, dword
 *    lam of pair f is dword lam*G + f of the group.  Groups follow each
 *    other along K; 16-row blocks follow each other along N.
 * bitlinear_packed_bytes_b1 (host-only) writes that size; BL_ERR_SHAPE when
 * K % 64 != 0, K > BITLINEAR_B1_MAX_K (the kernel sums 64 * code: 64 * 127 * K
 * must fit in int32) or the size reaches 2^31 bytes.
 *
 * bitlinear_pack_binary_b1: the codes, beta and alpha of bitlinear_pack_binary
 * (same rule, same scalars, bit for bit), written in layout b1.
 *   W, N, K, workspace, workspace_bytes  as for bitlinear_pack_binary.
 *   packed_b1  bitlinear_packed_bytes_b1(N, K) bytes, written.
 *   beta, alpha  [1] fp32 each, written.
 *
 * bitlinear_forward_b1: bitlinear_forward over layout b1 with beta in place
 * of gamma: acc[m][n] = sum_k xq[m][k] * code[n][k], y = bf16(acc[m][n] *
 * (beta / x_scale[m])) evaluated in fp32; the same arguments otherwise (any
 * M >= 0, M = 0 is a no-op).  Tokens go through the weights 16 at a time,
 * so it is meant for decode (a few tokens per call); BL_ERR_SHAPE when the
 * call's ceil(N/16) * ceil(M/16), summed over its entries, reaches 2^31.
 * bitlinear_forward_b1_grouped: up to BITLINEAR_MAX_GROUP such forwards in
 * one launch; each bitlinear_forward_args entry's packed / gamma are a
 * layout b1 buffer and its beta.  Results identical to separate calls.
 */
#define BITLINEAR_B1_MAX_K 262080
int bitlinear_packed_bytes_b1(int64_t N, int64_t K, size_t *bytes);
int bitlinear_pack_binary_b1(const float *W, int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                             uint8_t *packed_b1, float *beta, float *alpha, void *stream);
int bitlinear_forward_b1(const uint8_t *packed_b1, const float *beta, int64_t N, int64_t K, const int8_t *xq,
                         const float *x_scale, int64_t M, uint16_t *y, int32_t *acc, void *stream);
int bitlinear_forward_b1_grouped(const bitlinear_forward_args *args, int count, void *stream);

/*
 * bitlinear_quant_forward_grouped over layout b1 (each entry's packed /
 * gamma are a layout b1 buffer and its beta): for each entry exactly
 * bitlinear_quant_act then bitlinear_forward_b1, bit for bit, with the same
 * sharing of inputs and the same checks (plus the b1 shape rules).  One
 * launch for decode (every entry one token with K <= 32768, or 2..16 tokens
 * with M * K <= 16384); otherwise one quant launch per distinct input, then
 * the grouped b1 forward.  No workspace.
 */
int bitlinear_quant_forward_b1_grouped(const bitlinear_quant_forward_args *args, int count, float eps, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * grouped forward with a workspace, where the workspace is a fixed scratch
 * array inside the library instead of a caller buffer.  Same arguments,
 * checks and results as bitlinear_forward_grouped_ws given a large enough
 * workspace (bit for bit).  Allocates nothing and calls no allocating
 * routine.
 *  - The scratch holds BITLINEAR_SCRATCH_BYTES bytes per device, from the
 *    library's load until the process ends.  A call whose plan needs more
 *    (bitlinear_forward_workspace_bytes) returns BL_ERR_SCRATCH with nothing
 *    enqueued; the plan never needs more than 8 MiB + 2 KiB.
 *  - Every no-allocation call on a device shares that device's scratch, and
 *    it keeps the last call's contents (no call relies on them).  Calls that
 *    may overlap on one device (other streams, concurrent graph replays) race
 *    on it: serialise them, or give them bitlinear_forward_grouped_ws with
 *    workspaces of their own.
 */
#define BITLINEAR_SCRATCH_BYTES 9437184
int bitlinear_forward_grouped_noalloc(const bitlinear_forward_args *args, int count, void *stream);

/*
 * The codes of a packed weight rearranged into layout t1 for the backward
 * pass (the codes are unchanged; gamma is shared with the forward).
 *   packed    layout v1 codes of an N x K weight (bitlinear_pack_weights or
 *             bitlinear_pack_binary).
 *   packed_t  bitlinear_packed_bytes(K, N) bytes, written in layout t1.
 */
int bitlinear_pack_transposed(const uint8_t *packed, int64_t N, int64_t K, uint8_t *packed_t, void *stream);

/*
 * STE backward to the layer input ("1-bit & Ternary LLMs (BitNet b1.58)",
 * Training: the forward runs on the ternary weights and the straight-through
 * estimator treats both quantisers as identities, so the gradient of
 * y = x (gamma W~)^T with respect to x is dy (gamma W~)):
 *   dx[m][k] = bf16( gamma * sum_n dy[m][n] * code[n][k]  (+ dx[m][k]) )
 * The products are exact, the sum is accumulated in fp32 (bf16 matrix
 * cores), the scale and the optional addition are fp32, and the result is
 * rounded to nearest even.  The weight gradient needs no ternary work: the
 * estimator hands dy^T x^ (x^ the dequantised activations) straight to the
 * shadow weights, a plain bf16 GEMM.
 *   packed_t   layout t1 codes of the N x K weight (bitlinear_pack_transposed).
 *   gamma      [1] fp32, the weight scale from packing.
 *   dy         [M][N] bf16 bit patterns, the gradient of the layer output.
 *   dx         [M][K] bf16 bit patterns: written, or, when accumulate != 0,
 *              read and replaced by the sum (layers that share an input,
 *              such as Q, K and V, add their input gradients).
 * N % 8 == 0, M * N * 2 bytes and the layout t1 buffer below 2 GB
 * (BL_ERR_SHAPE otherwise).  M = 0 is a no-op.
 */
int bitlinear_backward_input(const uint8_t *packed_t, const float *gamma, int64_t N, int64_t K, const uint16_t *dy,
                             int64_t M, uint16_t *dx, int accumulate, void *stream);

/*
 * The input gradient of several layers that read the same input (Q, K and
 * V; gate and up) in one launch.  With x_0 = dx (accumulate != 0) or 0, and
 * for e = 1..count in order,
 *   x_e[m][k] = bf16( gamma_e * sum_n dy_e[m][n] * code_e[n][k] + x_{e-1}[m][k] )
 * and dx receives x_count: exactly the values of bitlinear_backward_input
 * called once per entry in order with accumulate on from the second call,
 * up to the order of the fp32 sums inside each entry.  Fewer launches, one
 * pass over dx, and one grid whose tiles each run every entry's contraction
 * (the straight-through input gradient of "1-bit & Ternary LLMs (BitNet
 * b1.58)", Training, summed over the layers fed by one input).
 *   args        HOST array of `count` entries, 1 <= count <=
 *               BITLINEAR_MAX_BACKWARD_GROUP (BL_ERR_SHAPE otherwise); read
 *               during the call only.
 *               Each entry: packed_t (layout t1 codes of an N x K weight),
 *               gamma ([1] fp32), N, and dy ([M][N] bf16 bit patterns).
 *   K, M        input width and rows, shared by every entry.
 *   dx          [M][K] bf16 bit patterns: written, or, when accumulate != 0,
 *               read and replaced by the sum; must not overlap any dy.
 * Each entry obeys the limits of bitlinear_backward_input (BL_ERR_SHAPE
 * otherwise); every entry is validated before anything is enqueued.  M = 0
 * is a no-op.
 */
#define BITLINEAR_MAX_BACKWARD_GROUP 4

typedef struct {
    const uint8_t *packed_t;  /* bitlinear_pack_transposed output for an N x K weight */
    const float *gamma;       /* [1] */
    int64_t N;
    const uint16_t *dy;       /* [M][N] bf16 bits */
} bitlinear_backward_args;

int bitlinear_backward_input_grouped(const bitlinear_backward_args *args, int count, int64_t K, int64_t M,
                                     uint16_t *dx, int accumulate, void *stream);

/*
 * Sign-flip tracker update, run once after an optimiser step ("Which 1-Bit
 * Weights Can You Trust?", Methodology: two INT16 counters per weight, both
 * starting at zero; where the sign differs from the previous step the flip
 * count goes up by one and the last-flip counter takes the step number).
 *   w_prev, w_curr  [n] fp32 latent weights at the previous and current step.
 *   step     current step, 1..32767.
 *   flip_count, last_flip  [n] int16, read and updated in place: where
 *            sgn(w_prev) != sgn(w_curr), with sgn in {-1, 0, +1} (so +0 and
 *            -0 are equal), flip_count = min(flip_count + 1, 32767) and
 *            last_flip = step; elsewhere both are left as they were.
 */
int bitlinear_flip_update(const float *w_prev, const float *w_curr, int64_t n, int32_t step,
                          int16_t *flip_count, int16_t *last_flip, void *stream);

/*
 * One AdamW step on the full-precision shadow weights with the sign-flip
 * tracker fused ("1-bit & Ternary LLMs (BitNet b1.58)", Training: the
 * straight-through estimator hands the gradient of the ternary weights to
 * the shadow weights, which the optimiser steps; "Which 1-Bit Weights Can You
 * Trust?", Experimental Setup: AdamW; Methodology: compare each weight's sign
 * before and after the step).  The published AdamW with decoupled weight
 * decay; the scalar coefficients are formed in fp64 and rounded once to
 * fp32, the per-weight arithmetic is fp32 in this order:
 *   w = W * (1 - lr*wd);  m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*g*g
 *   W = w - lr/(1-b1^t) * (m / (sqrt(v) / sqrt(1-b2^t) + eps))
 *   W, exp_avg, exp_avg_sq  [n] fp32, updated in place.
 *   grad     [n] fp32, read only.
 *   t        step number, >= 1 (<= 32767 when tracking).
 *   lr, weight_decay >= 0; 0 <= beta1, beta2 < 1; eps >= 0; all finite.
 *   flip_count, last_flip  [n] int16 or both NULL (no tracking, e.g. during
 *            warm-up): where the sign of W changes, flip_count =
 *            min(flip_count + 1, 32767) and last_flip = t, as
 *            bitlinear_flip_update does with two snapshots.
 */
int bitlinear_adamw_step(float *W, const float *grad, float *exp_avg, float *exp_avg_sq, int64_t n, int32_t t,
                         double lr, double beta1, double beta2, double eps, double weight_decay, int16_t *flip_count,
                         int16_t *last_flip, void *stream);

/*
 * Tracker read-out after T steps ("Which 1-Bit Weights Can You Trust?",
 * Methodology: two values per weight from the two counters; a weight that
 * never flipped has sign age 1, one that never moved has flip rate 0).
 *   flip_count, last_flip  [n] int16, read only (bitlinear_flip_update's).
 *   T        1..32767, the number of steps the counters cover.
 *   sign_age [n] fp32, written: (T - last_flip) / T.
 *   flip_rate [n] fp32, written: flip_count / T.
 * Each is an fp64 quotient rounded once to fp32.  (The page's reliability
 * score and its four classes have no surviving formula; a weight with
 * flip_count == 0 is the page's "locked" class.)
 */
int bitlinear_flip_stats(const int16_t *flip_count, const int16_t *last_flip, int64_t n, int32_t T,
                         float *sign_age, float *flip_rate, void *stream);

/* Host-only.  Static description of a status code. */
const char *bitlinear_strerror(int status);

/* Host-only.  BITLINEAR_LAYOUT_VERSION of the library that was loaded. */
int bitlinear_layout_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
