// Device helpers for the gfx950 kernels: code unpacking, bf16 rounding,
// wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));
// plain clang vector (HIP's uint4 struct copies lower to memcpy, which can
// keep register arrays in scratch)
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// two fp32 -> two bf16 (round to nearest even; one v_cvt_pk_bf16_f32), low half first
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}

// One packed dword holds 16 two-bit codes (00 -> 0, 01 -> +1, 11 -> -1).
// Code t of the dword sits at bit 8*(t%4) + 2*(t/4), so shifting by 2*j and
// masking each byte to its low two bits leaves codes 4j..4j+3 in bytes 0..3;
// a byte permute against the table {0x00, 0x01, 0x00, 0xFF} turns the 2-bit
// values into int8 {0, +1, -1}.  Output dword j holds the int8 codes of
// columns 4j..4j+3 in byte order, the order of the activations in memory.
__device__ __forceinline__ uint32_t unpack4(uint32_t w, int j) {
    const uint32_t sel = (w >> (2 * j)) & 0x03030303u;
    return __builtin_amdgcn_perm(0u, 0xFF000100u, sel);
}

__device__ __forceinline__ v4i unpack16(uint32_t w) {
    v4i r;
    r.x = (int)unpack4(w, 0);
    r.y = (int)unpack4(w, 1);
    r.z = (int)unpack4(w, 2);
    r.w = (int)unpack4(w, 3);
    return r;
}

// The same 16 codes as int8 values 64*code: the 2-bit field of each byte is
// shifted into bits 6..7 and everything else masked off, which reads as the
// signed byte 0, 64 or -64 (01 -> 0x40, 11 -> 0xC0) because the layout's code
// is a two-bit two's complement number.  7 VALU instead of 11; a contraction
// over these bytes yields 64 * acc exactly while 64 * 127 * K < 2^31, and an
// arithmetic shift by 6 recovers acc.
constexpr int64_t kScaledMaxK = 262080;  // 64 * 127 * K < 2^31, K a multiple of 64

__device__ __forceinline__ v4i unpack16_x64(uint32_t w) {
    v4i r;
    r.x = (int)((w << 6) & 0xC0C0C0C0u);
    r.y = (int)((w << 4) & 0xC0C0C0C0u);
    r.z = (int)((w << 2) & 0xC0C0C0C0u);
    r.w = (int)(w & 0xC0C0C0C0u);
    return r;
}

// Half H of a layout b1 dword (one bit per binary code, bit 1 = -1; code t
// of half h at bit 8*(t%4) + 7 - (4h + t/4)) -> the 16 int8 operand bytes
// 64 * code: shifting by 4H + j puts the code bits of columns 4j..4j+3 in
// the byte signs, and the mask and or leave 0x40 (+64) or 0xC0 (-64).
template <int H>
__device__ __forceinline__ v4i unpack_b1(uint32_t w) {
    v4i r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = (int)(((w << (4 * H + j)) & 0x80808080u) | 0x40404040u);
    return r;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Max over the 64 lanes of a wave of values >= 0 (absolute values), with DPP
// lane moves instead of LDS-crossbar shuffles: shifts by 1, 2, 4, 8 within
// each 16-lane row leave the row max in its lane 15, two row broadcasts carry
// it to lane 63.  Lanes a move has no source for keep 0, which is neutral for
// values >= 0.  The result is read from lane 63 and is uniform.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max(float v) {
    return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false)));
}

__device__ __forceinline__ float wave_max_nonneg(float v) {
    v = dpp_max<0x111, 0xf>(v);  // row_shr:1
    v = dpp_max<0x112, 0xf>(v);  // row_shr:2
    v = dpp_max<0x114, 0xf>(v);  // row_shr:4
    v = dpp_max<0x118, 0xf>(v);  // row_shr:8
    v = dpp_max<0x142, 0xa>(v);  // row_bcast:15
    v = dpp_max<0x143, 0xc>(v);  // row_bcast:31
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Workgroup barrier that waits only for this wave's LDS operations
// (lgkmcnt), not for its global loads in flight (__syncthreads also drains
// vmcnt); the empty asm blocks keep the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void lds_barrier_only() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14));  // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---- activation quant arithmetic (shared by the quant kernels and the
// decode kernel that quantises its tokens itself): s = 127 / max(absmax,
// eps) as a correctly rounded fp32 divide, q = rint(x * s), ties to even.

// Fast path of the same arithmetic.  t = x * s is the fp32 product; adding
// 1.5 * 2^23 rounds it to an integer, ties to even (the fp32 spacing there is
// 1), and leaves that integer in the low bits of the sum as two's complement,
// so its low byte is the int8 code.  The clip to +-127 of quant1 never
// applies: |x| <= absmax and s = RN(127 / max(absmax, eps)) give
// |t| <= 127 * (1 + 2^-24), which rounds to at most 127.  (The build keeps
// a * b + c unfused, so t is the rounded product.)
__device__ __forceinline__ uint32_t qbits(float x, float s) {
    const float t = x * s;
    return __float_as_uint(t + 12582912.0f);
}

// four bf16 (two dwords, element order lo, hi, lo, hi) -> four int8 codes
__device__ __forceinline__ uint32_t quant4(uint32_t w01, uint32_t w23, float s) {
    const uint32_t a = qbits(__uint_as_float(w01 << 16), s);
    const uint32_t b = qbits(__uint_as_float(w01 & 0xFFFF0000u), s);
    const uint32_t c = qbits(__uint_as_float(w23 << 16), s);
    const uint32_t d = qbits(__uint_as_float(w23 & 0xFFFF0000u), s);
    const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);  // a -> byte 0, b -> byte 1
    const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x04000C0Cu);  // c -> byte 2, d -> byte 3
    return lo | hi;
}

// Running absmax over bf16 pairs as integers: for values >= 0 the fp32 bit
// patterns order like the values.  The high element with its sign bit
// cleared is already an fp32 pattern; the low element shifted left by 17
// loses its sign bit and is twice its fp32 pattern (same order).
struct AbsMax {
    uint32_t hi = 0, lo2 = 0;
    __device__ __forceinline__ void add(uint32_t w) {
        hi = max(hi, w & 0x7FFF0000u);
        lo2 = max(lo2, w << 17);
    }
    __device__ __forceinline__ float value() const { return __uint_as_float(max(hi, lo2 >> 1)); }
};

}  // namespace bl
