"""CPU oracle for the BitNet b1.58 BitLinear forward path (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product library never loads it, and the
two share no code: the arithmetic lives in ``bitlinear_oracle.c`` (plain C,
one IEEE operation per step, no fast-math, no FP contraction), this module
only marshals numpy arrays through ctypes.

Every function names the passage of the BitNet pages it follows in the C
source.  Parity status: every function is pinned by the ``-m "not gpu"``
tests in ``tests/test_oracle_pins.py`` (closed forms, invariants, brute
force, library routines); none is "parity unpinned".
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitlinear_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, ERR_RANGE, ERR_CODE, ERR_NONFINITE = 0, -1, -2, -3


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = C.CDLL(_LIB)
        i64, p = C.c_int64, C.c_void_p
        L.oracle_abs_sum.restype = C.c_double
        L.oracle_abs_sum.argtypes = [p, i64]
        L.oracle_gamma.restype = C.c_float
        L.oracle_gamma.argtypes = [p, i64, i64]
        L.oracle_ternarise.argtypes = [p, i64, i64, C.c_float, C.c_float, p]
        L.oracle_packed_bytes.restype = i64
        L.oracle_packed_bytes.argtypes = [i64, i64]
        L.oracle_encode.argtypes = [p, i64, i64, p]
        L.oracle_decode.argtypes = [p, i64, i64, p]
        L.oracle_encode_t1.argtypes = [p, i64, i64, p]
        L.oracle_decode_t1.argtypes = [p, i64, i64, p]
        L.oracle_packed_bytes_b1.restype = i64
        L.oracle_packed_bytes_b1.argtypes = [i64, i64]
        L.oracle_encode_b1.argtypes = [p, i64, i64, p]
        L.oracle_packed_bytes_t3.restype = i64
        L.oracle_packed_bytes_t3.argtypes = [i64, i64]
        L.oracle_encode_t3.argtypes = [p, i64, i64, p]
        L.oracle_decode_t3.argtypes = [p, i64, i64, p]
        L.oracle_decode_b1.argtypes = [p, i64, i64, p]
        L.oracle_backward_input.argtypes = [p, p, i64, i64, i64, C.c_float, p, p, p, p]
        L.oracle_quant_act.argtypes = [p, i64, i64, C.c_float, p, p]
        L.oracle_rmsnorm_quant_act.argtypes = [p, p, i64, i64, C.c_float, C.c_float, p, p, p]
        L.oracle_contract.argtypes = [p, p, i64, i64, i64, p]
        L.oracle_contract_pairs.argtypes = [p, p, i64, p, p, i64, p]
        L.oracle_epilogue.restype = None
        L.oracle_epilogue.argtypes = [p, i64, i64, C.c_float, p, p]
        L.oracle_flip_update.argtypes = [p, p, i64, C.c_int32, p, p]
        L.oracle_binarise.argtypes = [p, i64, i64, p, p, p]
        L.oracle_flip_stats.argtypes = [p, p, i64, C.c_int32, p, p]
        d = C.c_double
        L.oracle_adamw_flip.argtypes = [p, p, p, p, i64, C.c_int32, d, d, d, d, d, p, p]
        L.oracle_threads.restype = C.c_int
        L.oracle_set_threads.restype = None
        L.oracle_set_threads.argtypes = [C.c_int]
        _lib = L
    return _lib


def threads() -> int:
    return int(lib().oracle_threads())


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != OK:
        raise ValueError(f"oracle {what} failed with status {rc}")


# ------------------------------------------------------------------ weights

def abs_sum(W) -> float:
    W = _c(W, np.float32)
    return lib().oracle_abs_sum(_ptr(W), W.size)


def gamma(W) -> np.float32:
    W = _c(W, np.float32)
    N, K = W.shape
    return np.float32(lib().oracle_gamma(_ptr(W), N, K))


def ternarise(W, g, eps: float = 1e-5) -> np.ndarray:
    W = _c(W, np.float32)
    N, K = W.shape
    out = np.empty((N, K), np.int8)
    _check(lib().oracle_ternarise(_ptr(W), N, K, C.c_float(float(g)), C.c_float(eps), _ptr(out)), "ternarise")
    return out


def packed_bytes(N: int, K: int) -> int:
    return int(lib().oracle_packed_bytes(N, K))


def encode(codes) -> np.ndarray:
    codes = _c(codes, np.int8)
    N, K = codes.shape
    out = np.empty(packed_bytes(N, K), np.uint8)
    _check(lib().oracle_encode(_ptr(codes), N, K, _ptr(out)), "encode")
    return out


def decode(packed, N: int, K: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    if packed.size != packed_bytes(N, K):
        raise ValueError("packed buffer has the wrong size")
    out = np.empty((N, K), np.int8)
    _check(lib().oracle_decode(_ptr(packed), N, K, _ptr(out)), "decode")
    return out


def encode_t1(codes) -> np.ndarray:
    """codes int8 [N][K] -> layout t1 bytes of the transposed K x N code matrix."""
    codes = _c(codes, np.int8)
    N, K = codes.shape
    out = np.empty(packed_bytes(K, N), np.uint8)
    _check(lib().oracle_encode_t1(_ptr(codes), N, K, _ptr(out)), "encode_t1")
    return out


def decode_t1(packed_t, N: int, K: int) -> np.ndarray:
    """layout t1 bytes -> codes int8 [N][K]."""
    packed_t = _c(packed_t, np.uint8)
    if packed_t.size != packed_bytes(K, N):
        raise ValueError("packed buffer has the wrong size")
    out = np.empty((N, K), np.int8)
    _check(lib().oracle_decode_t1(_ptr(packed_t), N, K, _ptr(out)), "decode_t1")
    return out


def pack(W, eps: float = 1e-5):
    """(packed bytes, gamma, codes) for one weight tensor."""
    g = gamma(W)
    codes = ternarise(W, g, eps)
    return encode(codes), g, codes


# -------------------------------------------------------------- activations

def binarise(W):
    """Binary BitNet weights: (codes int8 [N][K] in {-1, +1}, alpha, beta)."""
    W = _c(W, np.float32)
    N, K = W.shape
    codes = np.empty((N, K), np.int8)
    a = C.c_float()
    b = C.c_float()
    _check(lib().oracle_binarise(_ptr(W), N, K, _ptr(codes), C.byref(a), C.byref(b)), "binarise")
    return codes, np.float32(a.value), np.float32(b.value)


def pack_binary(W):
    """(packed bytes in layout v1, beta, alpha, codes) for binary weights."""
    codes, a, b = binarise(W)
    return encode(codes), b, a, codes


def packed_bytes_b1(N: int, K: int) -> int:
    """Bytes of the one-bit layout b1 (K must be a multiple of 64)."""
    n = int(lib().oracle_packed_bytes_b1(N, K))
    if n < 0:
        raise ValueError("layout b1 needs K % 64 == 0")
    return n


def encode_b1(codes) -> np.ndarray:
    """codes int8 [N][K] in {-1, +1} -> layout b1 bytes."""
    codes = _c(codes, np.int8)
    N, K = codes.shape
    out = np.empty(packed_bytes_b1(N, K), np.uint8)
    _check(lib().oracle_encode_b1(_ptr(codes), N, K, _ptr(out)), "encode_b1")
    return out


def decode_b1(packed, N: int, K: int) -> np.ndarray:
    """layout b1 bytes -> codes int8 [N][K]."""
    packed = _c(packed, np.uint8)
    if packed.size != packed_bytes_b1(N, K):
        raise ValueError("packed buffer has the wrong size")
    out = np.empty((N, K), np.int8)
    _check(lib().oracle_decode_b1(_ptr(packed), N, K, _ptr(out)), "decode_b1")
    return out


def packed_bytes_t3(N: int, K: int) -> int:
    """Bytes of the base-3 layout t3 (five codes per byte; K % 320 == 0)."""
    n = int(lib().oracle_packed_bytes_t3(N, K))
    if n < 0:
        raise ValueError("layout t3 needs K % 320 == 0")
    return n


def encode_t3(codes) -> np.ndarray:
    """codes int8 [N][K] in {-1, 0, +1} -> layout t3 bytes (base-3 digits)."""
    codes = _c(codes, np.int8)
    N, K = codes.shape
    out = np.empty(packed_bytes_t3(N, K), np.uint8)
    _check(lib().oracle_encode_t3(_ptr(codes), N, K, _ptr(out)), "encode_t3")
    return out


def decode_t3(packed, N: int, K: int) -> np.ndarray:
    """layout t3 bytes -> codes int8 [N][K]."""
    packed = _c(packed, np.uint8)
    if packed.size != packed_bytes_t3(N, K):
        raise ValueError("packed buffer has the wrong size")
    out = np.empty((N, K), np.int8)
    _check(lib().oracle_decode_t3(_ptr(packed), N, K, _ptr(out)), "decode_t3")
    return out


def pack_binary_b1(W):
    """(packed bytes in layout b1, beta, alpha, codes) for binary weights."""
    codes, a, b = binarise(W)
    return encode_b1(codes), b, a, codes


def quant_act(x_bits, eps: float = 1e-5):
    """x as bf16 bit patterns [M][K] -> (q int8 [M][K], s fp32 [M])."""
    x_bits = _c(x_bits, np.uint16)
    M, K = x_bits.shape
    q = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    _check(lib().oracle_quant_act(_ptr(x_bits), M, K, C.c_float(eps), _ptr(q), _ptr(s)), "quant_act")
    return q, s


def rmsnorm_quant_act(x_bits, gain=None, eps_norm: float = 1e-6, eps: float = 1e-5):
    """RMSNorm (optional per-channel fp32 gain [K]) then the activation quant,
    in fp64.  Returns (q int8 [M][K], s fp32 [M], v fp64 [M][K]) with v the
    value that was rounded to q."""
    x_bits = _c(x_bits, np.uint16)
    M, K = x_bits.shape
    g = None if gain is None else _c(gain, np.float32)
    if g is not None and g.shape != (K,):
        raise ValueError("gain must have K entries")
    q = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    v = np.empty((M, K), np.float64)
    _check(lib().oracle_rmsnorm_quant_act(_ptr(x_bits), None if g is None else _ptr(g), M, K, C.c_float(eps_norm),
                                          C.c_float(eps), _ptr(q), _ptr(s), _ptr(v)), "rmsnorm_quant_act")
    return q, s, v


def half_window_mask(v, rel: float = 1e-6):
    """Positions where |v| lies within rel*b of a half-integer b (the values
    whose rounding to a code the acceptance rule leaves open)."""
    a = np.abs(np.asarray(v, np.float64))
    b = np.floor(a) + 0.5
    return np.abs(a - b) <= rel * b


# -------------------------------------------------------------- contraction

def contract(q, codes) -> np.ndarray:
    q = _c(q, np.int8)
    codes = _c(codes, np.int8)
    M, K = q.shape
    N, K2 = codes.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    _check(lib().oracle_contract(_ptr(q), _ptr(codes), M, N, K, _ptr(acc)), "contract")
    return acc


def contract_pairs(q, codes, m_idx, n_idx) -> np.ndarray:
    q = _c(q, np.int8)
    codes = _c(codes, np.int8)
    K = q.shape[1]
    assert codes.shape[1] == K
    m_idx = _c(m_idx, np.int64)
    n_idx = _c(n_idx, np.int64)
    acc = np.empty(m_idx.size, np.int32)
    _check(lib().oracle_contract_pairs(_ptr(q), _ptr(codes), K, _ptr(m_idx), _ptr(n_idx),
                                       m_idx.size, _ptr(acc)), "contract_pairs")
    return acc


def epilogue(acc, g, s) -> np.ndarray:
    acc = _c(acc, np.int32)
    s = _c(s, np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.float32)
    lib().oracle_epilogue(_ptr(acc), M, N, C.c_float(float(g)), _ptr(s), _ptr(y))
    return y


def forward(x_bits, W, eps_w: float = 1e-5, eps_x: float = 1e-5):
    """The whole path on one tensor: returns dict of every intermediate."""
    packed, g, codes = pack(W, eps_w)
    q, s = quant_act(x_bits, eps_x)
    acc = contract(q, codes)
    y = epilogue(acc, g, s)
    return dict(packed=packed, gamma=g, codes=codes, q=q, s=s, acc=acc, y=y)


# ---------------------------------------------------------------- tracker

def flip_update(prev, curr, step: int, flip_count, last_flip):
    """Returns updated copies of (flip_count, last_flip)."""
    prev = _c(prev, np.float32).reshape(-1)
    curr = _c(curr, np.float32).reshape(-1)
    fc = np.array(flip_count, dtype=np.int16, copy=True).reshape(-1)
    lf = np.array(last_flip, dtype=np.int16, copy=True).reshape(-1)
    assert prev.size == curr.size == fc.size == lf.size
    _check(lib().oracle_flip_update(_ptr(prev), _ptr(curr), prev.size, int(step), _ptr(fc), _ptr(lf)),
           "flip_update")
    return fc, lf


# ------------------------------------------------------------- tolerances

def flip_stats(flip_count, last_flip, T: int):
    """(sign_age fp32 [n], flip_rate fp32 [n]) after T steps."""
    fc = _c(flip_count, np.int16).reshape(-1)
    lf = _c(last_flip, np.int16).reshape(-1)
    age = np.empty(fc.size, np.float32)
    rate = np.empty(fc.size, np.float32)
    _check(lib().oracle_flip_stats(_ptr(fc), _ptr(lf), fc.size, int(T), _ptr(age), _ptr(rate)), "flip_stats")
    return age, rate


def adamw_flip(W, g, m, v, t: int, lr: float, b1: float = 0.9, b2: float = 0.999, eps: float = 1e-8,
               wd: float = 0.0, flip_count=None, last_flip=None):
    """One AdamW step (fp32) with the sign-flip tracker fused; returns updated
    copies (W, m, v, flip_count, last_flip) (counters None when not given)."""
    W = _c(W, np.float32).copy()
    g = _c(g, np.float32)
    m = _c(m, np.float32).copy()
    v = _c(v, np.float32).copy()
    fc = None if flip_count is None else _c(flip_count, np.int16).copy()
    lf = None if last_flip is None else _c(last_flip, np.int16).copy()
    _check(lib().oracle_adamw_flip(_ptr(W), _ptr(g), _ptr(m), _ptr(v), W.size, int(t), float(lr), float(b1),
                                   float(b2), float(eps), float(wd), None if fc is None else _ptr(fc),
                                   None if lf is None else _ptr(lf)), "adamw_flip")
    return W, m, v, fc, lf


# ---------------------------------------------------------------- backward

def backward_input(dy_bits, codes, g, dx_prev=None):
    """STE gradient to the layer input: dx = gamma * dy @ codes.

    Returns (ref fp64 [M][K], mag fp64 [M][K] = gamma * |dy| @ |codes|,
    dx bf16 bits [M][K] under the fp32-then-bf16 reading)."""
    dy_bits = _c(dy_bits, np.uint16)
    codes = _c(codes, np.int8)
    M, N = dy_bits.shape
    N2, K = codes.shape
    if N2 != N:
        raise ValueError("dy and codes disagree on N")
    prev = None if dx_prev is None else _c(dx_prev, np.uint16)
    if prev is not None and prev.shape != (M, K):
        raise ValueError("dx_prev has the wrong shape")
    ref = np.empty((M, K), np.float64)
    mag = np.empty((M, K), np.float64)
    dx = np.empty((M, K), np.uint16)
    _check(lib().oracle_backward_input(_ptr(dy_bits), _ptr(codes), M, N, K, C.c_float(float(g)),
                                       None if prev is None else _ptr(prev), _ptr(ref), _ptr(mag), _ptr(dx)),
           "backward_input")
    return ref, mag, dx


def dx_close(dx_gpu_f32, ref, mag, N: int):
    """Element mask of the backward tolerance: the bf16 rounding of the
    result (2^-8 |ref|, twice its half-ulp) plus the error any fp32 summation
    of N terms can make, in any order and with faithful (not necessarily
    nearest) rounding: N + 1 roundings of at most 2^-23 of a running
    magnitude bounded by mag; plus the smallest normal fp32."""
    dx_gpu_f32 = np.asarray(dx_gpu_f32, np.float64)
    tol = 2.0 ** -8 * np.abs(ref) + (N + 1) * 2.0 ** -23 * mag + 2.0 ** -126
    return np.abs(dx_gpu_f32 - ref) <= tol


def dx_rel_rms(dx_gpu_f32, ref) -> float:
    """RMS of the relative error over the outputs with |ref| >= 10% of the
    largest: bf16 rounding alone keeps it near 2^-10; one lost term of a
    Gaussian sum moves it to about 1/sqrt(N)."""
    ref = np.asarray(ref, np.float64)
    big = np.abs(ref) >= 0.1 * np.abs(ref).max()
    r = (np.asarray(dx_gpu_f32, np.float64)[big] - ref[big]) / ref[big]
    return float(np.sqrt(np.mean(r * r)))


def y_close(y_gpu_f32, y_ref, atol: float = 1e-3, rtol: float = 1e-2):
    """Element mask of |y - y_ref| <= atol + rtol*|y_ref| (bf16 output vs fp32 reference)."""
    y_gpu_f32 = np.asarray(y_gpu_f32, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    return np.abs(y_gpu_f32 - y_ref) <= atol + rtol * np.abs(y_ref)


def weight_boundary_mask(W, g, eps: float = 1e-5, rel: float = 1e-6):
    """Positions where |W|/(gamma+eps), evaluated in fp64, lies within rel*0.5 of 0.5
    (the only rounding boundary that can change a clipped ternary code)."""
    r = np.abs(np.asarray(W, np.float64)) / (float(g) + float(eps))
    return np.abs(r - 0.5) <= rel * 0.5
