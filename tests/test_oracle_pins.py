"""Pins for the CPU oracle: each check rests on something other than the oracle
itself (a hand-worked value, a closed form, an invariant, brute force, or an
independent library routine), so that a dropped term, a wrong sign, a wrong
index or a transposed operand in the oracle fails at least one of them.

The BitNet pages print no worked example for any step of the path, so no value
here comes from the pages except the tracker census (page "Which 1-Bit Weights
Can You Trust?", Methodology), which lives in tests/golden/census.json.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ===================================================================== gamma
# BitNet b1.58 equation (gamma = mean absolute weight over the whole matrix)

def test_gamma_hand_value():
    # sum |W| = 1 + 1 + 0.5 + 1.5 = 4 over 4 entries -> exactly 1.0.
    # A dropped abs() gives 0.5; dividing by N or K alone gives 2.0.
    W = np.array([[1.0, -1.0], [0.5, 1.5]], np.float32)
    assert oracle.gamma(W) == np.float32(1.0)
    W2 = np.array([[3.0, 0.0, -3.0]], np.float32)  # 6/3 = 2, non-square
    assert oracle.gamma(W2) == np.float32(2.0)
    assert oracle.gamma(W2.T.copy()) == np.float32(2.0)


def test_gamma_matches_numpy_pairwise_mean():
    for seed in range(3):
        W = wl.gaussian_weight(37, 301, key=(900, seed))
        ref = np.float32(np.abs(W.astype(np.float64)).mean())
        assert oracle.gamma(W) == ref


def test_gamma_closed_form_gaussian():
    sigma = 0.02
    W = wl.gaussian_weight(1024, 1024, key=(901,), sigma=sigma)
    n = W.size
    mean = sigma * math.sqrt(2 / math.pi)
    se = sigma * math.sqrt(1 - 2 / math.pi) / math.sqrt(n)
    assert abs(float(oracle.gamma(W)) - mean) < 5 * se


def test_gamma_power_of_two_scaling_is_exact():
    W = wl.gaussian_weight(64, 128, key=(902,))
    assert oracle.gamma(W * np.float32(4.0)) == oracle.gamma(W) * np.float32(4.0)
    assert oracle.gamma(W * np.float32(0.125)) == oracle.gamma(W) * np.float32(0.125)


# ================================================================= ternarise
# BitNet b1.58 equation: RoundClip(W / (gamma + eps), -1, 1)

def test_ternarise_hand_values_round_half_even_and_clip():
    # mean |W| = 8 / 8 = 1, so with eps = 0 the ratio is W itself.
    W = np.array([[1.0, -1.0, 0.5, -0.5, 1.5, -1.5, 0.75, 1.25]], np.float32)
    g = oracle.gamma(W)
    assert g == 1.0
    c = oracle.ternarise(W, g, eps=0.0)
    # 0.5 and -0.5 round to 0 (ties to even); 1.5 rounds to 2 then clips to 1;
    # 0.75 and 1.25 round to 1.
    assert c.tolist() == [[1, -1, 0, 0, 1, -1, 1, 1]]


def test_ternarise_eps_sits_in_the_denominator():
    # mean |W| = (1 + 1 + 0.5078125 + 1.4921875) / 4 = 1
    W = np.array([[1.0, -1.0, 0.5078125, 1.4921875]], np.float32)
    g = oracle.gamma(W)
    assert g == 1.0
    assert oracle.ternarise(W, g, eps=0.0).tolist() == [[1, -1, 1, 1]]
    # 0.5078125 / 1.02 = 0.4978... -> 0
    assert oracle.ternarise(W, g, eps=0.02).tolist() == [[1, -1, 0, 1]]


def test_ternarise_invariants():
    W = wl.gaussian_weight(48, 200, key=(903,))
    g = oracle.gamma(W)
    c = oracle.ternarise(W, g, 1e-5)
    assert set(np.unique(c).tolist()) <= {-1, 0, 1}
    # sign symmetry: gamma(-W) = gamma(W) and ties-to-even is symmetric
    assert np.array_equal(oracle.ternarise(-W, oracle.gamma(-W), 1e-5), -c)
    # positive power-of-two scaling with eps = 0 changes nothing
    c0 = oracle.ternarise(W, g, 0.0)
    for f in (0.25, 2.0, 1024.0):
        Ws = W * np.float32(f)
        assert np.array_equal(oracle.ternarise(Ws, oracle.gamma(Ws), 0.0), c0)


def test_ternarise_special_cases():
    rng = wl.rng(904)
    signs = rng.choice([-1.0, 1.0], size=(16, 40)).astype(np.float32)
    W = signs * np.float32(0.037)
    assert np.array_equal(oracle.ternarise(W, oracle.gamma(W), 0.0), signs.astype(np.int8))
    # one nonzero entry: gamma = |w| / (N K), ratio = +-N K -> clipped sign
    W1 = np.zeros((8, 9), np.float32)
    W1[3, 5] = -0.3
    c1 = oracle.ternarise(W1, oracle.gamma(W1), 0.0)
    assert c1[3, 5] == -1 and np.count_nonzero(c1) == 1
    # all zeros, with and without eps
    Z = np.zeros((4, 4), np.float32)
    assert np.all(oracle.ternarise(Z, oracle.gamma(Z), 1e-5) == 0)
    assert np.all(oracle.ternarise(Z, oracle.gamma(Z), 0.0) == 0)


def test_ternarise_zero_fraction_closed_form():
    # For W ~ N(0, s^2), gamma -> s sqrt(2/pi); a code is 0 when |W| < gamma(1+eps/gamma)/2
    # (up to ties), so P(0) = 2 Phi(0.5 sqrt(2/pi) (1 + eps/gamma)) - 1 ~ 0.3102.
    W = wl.gaussian_weight(2048, 2048, key=(905,))
    g = float(oracle.gamma(W))
    eps = 1e-5
    z = 0.5 * (g + eps) / 0.02
    p0 = math.erf(z / math.sqrt(2))
    frac = float(np.mean(oracle.ternarise(W, np.float32(g), eps) == 0))
    se = math.sqrt(p0 * (1 - p0) / W.size)
    assert abs(frac - p0) < 6 * se
    assert abs(frac - 0.3102) < 0.003


def test_ternarise_matches_numpy_fp32_routine():
    W = wl.gaussian_weight(70, 333, key=(906,))
    g = oracle.gamma(W)
    eps = np.float32(1e-5)
    ref = np.clip(np.rint(W / (np.float32(g) + eps)), -1, 1).astype(np.int8)
    assert np.array_equal(oracle.ternarise(W, g, 1e-5), ref)


# ==================================================================== layout
# Library-owned packed layout (the pages say weights and the kernel that reads
# them must agree on the representation).  Byte positions below were worked by
# hand from the layout description in include/bitlinear.h.

def _single(N, K, n, k, code):
    c = np.zeros((N, K), np.int8)
    c[n, k] = code
    return oracle.encode(c)


def test_layout_hand_worked_positions():
    # N=16, K=64: one fragment, group of 1.  (3, 37): lane 35, t = 5 -> bit 10.
    p = _single(16, 64, 3, 37, 1)
    assert p.size == 256
    assert np.flatnonzero(p).tolist() == [141] and p[141] == 0x04
    # N=16, K=256: one group of 4.  (0, 255): fragment 3, lane 48, t = 15 -> bit 30;
    # dword 48*4 + 3 = 195 -> byte 783, code 11 at shift 6.
    p = _single(16, 256, 0, 255, -1)
    assert p.size == 1024
    assert np.flatnonzero(p).tolist() == [783] and p[783] == 0xC0
    # N=20, K=320: two row blocks, five fragments (groups of 4 and 1).
    # (17, 300): block 1, fragment 4 (group 1, size 1), lane 33, t = 12 -> bit 6;
    # dword 1*5*64 + 256 + 33 = 609 -> byte 2436, shift 6.
    p = _single(20, 320, 17, 300, 1)
    assert p.size == 2560
    assert np.flatnonzero(p).tolist() == [2436] and p[2436] == 0x40
    # (5, 70) in the same shape: fragment 1 of group 0 (size 4), lane 5, t = 6 ->
    # bit 8*2 + 2*1 = 18; dword 5*4 + 1 = 21 -> byte 86, code 11 at shift 2.
    p = _single(20, 320, 5, 70, -1)
    assert np.flatnonzero(p).tolist() == [86] and p[86] == 0x0C


def test_layout_round_trip_and_padding():
    for (N, K) in [(16, 64), (17, 65), (33, 300), (5, 1000), (64, 1024)]:
        W = wl.gaussian_weight(N, K, key=(907, N, K))
        c = oracle.ternarise(W, oracle.gamma(W), 1e-5)
        p = oracle.encode(c)
        assert p.size == ((N + 15) // 16) * ((K + 63) // 64) * 256
        assert np.array_equal(oracle.decode(p, N, K), c)
        # the never-written code and nonzero padding are both rejected
        if K % 64:
            bad = p.copy()
            # last code column of row 0 is padding: find its byte by encoding a probe
            probe = np.zeros((N, ((K + 63) // 64) * 64), np.int8)
            probe[0, -1] = 1
            pos = np.flatnonzero(oracle.encode(probe))[0]
            bad[pos] |= oracle.encode(probe)[pos]
            with pytest.raises(ValueError):
                oracle.decode(bad, N, K)
    c = np.zeros((16, 64), np.int8)
    c[0, 0] = 1
    p = oracle.encode(c)
    p[np.flatnonzero(p)[0]] = 0x02  # code 10
    with pytest.raises(ValueError):
        oracle.decode(p, 16, 64)


# ========================================================= activation quant
# Absmax per token, no zero point, symmetric 8-bit range.

def _bits(v):
    return wl.f32_to_bf16_bits(np.asarray(v, np.float32))


def test_quant_hand_values():
    x = _bits([[127.0, 2.5, -3.5, 0.5, 1.5, -126.5],
               [1.0, -0.5, 0.25, 2.0, 0.0, 0.0]])
    q, s = oracle.quant_act(x, 1e-5)
    # row 0: absmax 127 -> s = 1, ties to even: 2.5 -> 2, -3.5 -> -4, 0.5 -> 0, 1.5 -> 2, -126.5 -> -126
    assert s[0] == np.float32(1.0)
    assert q[0].tolist() == [127, 2, -4, 0, 2, -126]
    # row 1: absmax 2 -> s = 63.5: 63.5 -> 64, -31.75 -> -32, 15.875 -> 16, 127
    assert s[1] == np.float32(63.5)
    assert q[1].tolist() == [64, -32, 16, 127, 0, 0]


def test_quant_eps_floor():
    x = _bits([[0.0] * 8, [1e-6] * 8])
    q, s = oracle.quant_act(x, 1e-5)
    assert np.all(q[0] == 0) and s[0] == np.float32(127.0) / np.float32(1e-5)
    xv = wl.bf16_bits_to_f32(x[1])[0]
    assert np.all(q[1] == np.rint(np.float32(xv) * s[1]))
    assert q[1, 0] == 13  # ~1e-6 * 1.27e7 = 12.7 -> 13


def test_quant_invariants():
    x = wl.activation(40, 515, key=(908,), recipe="channels")
    q, s = oracle.quant_act(x)
    assert q.min() >= -127 and q.max() <= 127
    assert np.all(np.abs(q).max(axis=1) == 127)  # the absmax element lands on 127
    qn, sn = oracle.quant_act(x ^ np.uint16(0x8000))  # exact negation of bf16
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    x2 = _bits(wl.bf16_bits_to_f32(x) * np.float32(2.0))
    q2, s2 = oracle.quant_act(x2)
    assert np.array_equal(q2, q) and np.array_equal(s2 * np.float32(2.0), s)


def test_quant_matches_numpy_fp32_routine():
    x = wl.activation(33, 700, key=(909,), recipe="bernoulli")
    xf = wl.bf16_bits_to_f32(x)
    a = np.abs(xf).max(axis=1)
    s = np.float32(127.0) / np.maximum(a, np.float32(1e-5))
    qref = np.clip(np.rint(xf * s[:, None]), -127, 127).astype(np.int8)
    q, so = oracle.quant_act(x, 1e-5)
    assert np.array_equal(so, s) and np.array_equal(q, qref)


# ========================================================= RMSNorm + quant
# The normalisation before the quant ("1-bit & Ternary LLMs", How it works:
# the forward quantises LN(x); b1.58 takes the LLaMA-style RMSNorm).

def test_rmsnorm_quant_hand_values():
    # [3, 4, 0, 0]: mean square 25/4, r = 1/2.5 = 0.4, y = [1.2, 1.6, 0, 0],
    # s = 127 / 1.6 = 79.375, y*s = [95.25, 127, 0, 0]
    x = _bits([[3.0, 4.0, 0.0, 0.0]])
    q, s, v = oracle.rmsnorm_quant_act(x, eps_norm=0.0)
    assert q[0].tolist() == [95, 127, 0, 0]
    assert s[0] == np.float32(79.375)
    # gain [2, 1, 1, 1]: y = [2.4, 1.6, 0, 0], s = 127 / 2.4, y*s = [127, 84.67, 0, 0]
    q, s, v = oracle.rmsnorm_quant_act(x, gain=np.array([2, 1, 1, 1], np.float32), eps_norm=0.0)
    assert q[0].tolist() == [127, 85, 0, 0]
    assert s[0] == np.float32(127.0 / 2.4)


def test_rmsnorm_quant_constant_rows_closed_form():
    for c in (3.0, -0.375, 1e-3, 200.0):
        x = _bits(np.full((1, 96), c))
        cb = float(wl.bf16_bits_to_f32(x)[0, 0])
        q, s, v = oracle.rmsnorm_quant_act(x, eps_norm=0.0)
        assert np.all(q == (127 if c > 0 else -127)) and s[0] == np.float32(127.0)  # y = +-1 exactly
        q, s, v = oracle.rmsnorm_quant_act(x, eps_norm=1e-6)
        ref = 127.0 * math.sqrt(cb * cb + float(np.float32(1e-6))) / abs(cb)  # 127 / |c / sqrt(c^2 + eps)|
        assert abs(float(s[0]) - ref) <= 1e-6 * ref
        assert np.all(np.abs(q) == 127)


def test_rmsnorm_quant_unit_mean_square_and_zero_row():
    x = wl.activation(7, 333, key=(910,), recipe="channels")
    q, s, v = oracle.rmsnorm_quant_act(x, eps_norm=0.0)
    y = v / s.astype(np.float64)[:, None]
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=0, atol=1e-6)  # s is fp32: y carries its rounding
    z = np.zeros((2, 64), np.uint16)
    q, s, v = oracle.rmsnorm_quant_act(z, eps_norm=1e-6)
    assert np.all(q == 0) and np.all(s == np.float32(127.0 / np.float32(1e-5)))


def test_rmsnorm_quant_codes_are_scale_invariant():
    """RMSNorm is a positive per-token scaling, and the absmax quant does not
    see such a scaling: without a gain the codes equal the plain quant's,
    with a gain g they equal the plain quant of x*g (here g are powers of two,
    so x*g is still exact bf16).  Either side may differ only inside the
    rounding window."""
    x = wl.activation(24, 1000, key=(911,), recipe="bernoulli")
    q, s, v = oracle.rmsnorm_quant_act(x, eps_norm=1e-6)
    qp, sp = oracle.quant_act(x)
    xp = wl.bf16_bits_to_f32(x).astype(np.float64) * sp.astype(np.float64)[:, None]
    bad = (q != qp) & ~oracle.half_window_mask(v) & ~oracle.half_window_mask(xp)
    assert not bad.any()
    g = np.float32(2.0) ** wl.rng(912).integers(-3, 4, size=1000).astype(np.float32)
    xg = _bits(wl.bf16_bits_to_f32(x) * g)
    q, s, v = oracle.rmsnorm_quant_act(x, gain=g, eps_norm=1e-6)
    qp, sp = oracle.quant_act(xg)
    xp = wl.bf16_bits_to_f32(xg).astype(np.float64) * sp.astype(np.float64)[:, None]
    bad = (q != qp) & ~oracle.half_window_mask(v) & ~oracle.half_window_mask(xp)
    assert not bad.any()
    # exact power-of-two scaling of the input leaves codes and scale unchanged when eps_norm = 0
    q1, s1, _ = oracle.rmsnorm_quant_act(x, eps_norm=0.0)
    q2, s2, _ = oracle.rmsnorm_quant_act(_bits(wl.bf16_bits_to_f32(x) * np.float32(8.0)), eps_norm=0.0)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


# =============================================================== contraction
# +1 adds, -1 subtracts, 0 skips.

def test_contract_brute_force_all_code_rows():
    K = 5
    rows = np.array(np.meshgrid(*[[-1, 0, 1]] * K, indexing="ij")).reshape(K, -1).T.astype(np.int8)
    assert rows.shape == (3 ** K, K)
    q = wl.rng(910).integers(-127, 128, size=(7, K), dtype=np.int8)
    acc = oracle.contract(q, rows)
    ref = q.astype(np.int64) @ rows.astype(np.int64).T
    assert np.array_equal(acc, ref)


def test_contract_matches_int64_matmul_and_extremes():
    g = wl.rng(911)
    q = g.integers(-127, 128, size=(9, 517), dtype=np.int8)
    c = g.integers(-1, 2, size=(13, 517), dtype=np.int8)
    assert np.array_equal(oracle.contract(q, c), q.astype(np.int64) @ c.astype(np.int64).T)
    K = 4000
    qm = np.full((2, K), 127, np.int8)
    qm[1] = -127
    cm = np.stack([np.ones(K, np.int8), -np.ones(K, np.int8), np.zeros(K, np.int8)])
    assert oracle.contract(qm, cm).tolist() == [[127 * K, -127 * K, 0], [-127 * K, 127 * K, 0]]


def test_contract_linearity_and_pairs():
    g = wl.rng(912)
    q1 = g.integers(-60, 61, size=(5, 300), dtype=np.int8)
    q2 = g.integers(-60, 61, size=(5, 300), dtype=np.int8)
    c = g.integers(-1, 2, size=(11, 300), dtype=np.int8)
    a1, a2 = oracle.contract(q1, c), oracle.contract(q2, c)
    assert np.array_equal(oracle.contract(q1 + q2, c), a1 + a2)
    assert np.array_equal(oracle.contract(-q1, c), -a1)
    mi = np.array([0, 4, 2, 2])
    ni = np.array([10, 0, 3, 7])
    assert np.array_equal(oracle.contract_pairs(q1, c, mi, ni), a1[mi, ni])


# ================================================================== epilogue
# One float rescale per output: y = acc * gamma / s.

def test_epilogue_hand_values():
    acc = np.array([[127, -3], [0, 254]], np.int32)
    y = oracle.epilogue(acc, np.float32(0.5), np.array([127.0, 0.5], np.float32))
    # row 0: 127*0.5/127 = 0.5 and -3*0.5/127 = -1.5/127; row 1 (s = 0.5): 0 and 254*0.5/0.5
    assert y.tolist() == [[0.5, float(np.float32(-1.5 / 127))], [0.0, 254.0]]


def test_epilogue_algebraic_identity():
    # acc * gamma / s  ==  sum_k (q/s) (gamma c), both in fp64, independent of the integer path
    x = wl.activation(6, 257, key=(913,), recipe="channels")
    W = wl.gaussian_weight(19, 257, key=(914,))
    r = oracle.forward(x, W)
    lhs = r["y"].astype(np.float64)
    deq_x = r["q"].astype(np.float64) / r["s"].astype(np.float64)[:, None]
    deq_w = float(r["gamma"]) * r["codes"].astype(np.float64)
    rhs = deq_x @ deq_w.T
    assert np.allclose(lhs, rhs, rtol=2 ** -23, atol=1e-30)


def test_forward_tracks_float_linear():
    # The quantised path approximates the float layer x W^T: error bounded by
    # the quantisation of x (<= 0.5/s per element) and W (codes vs W/gamma).
    x = wl.activation(4, 512, key=(915,), recipe="plain")
    W = wl.gaussian_weight(32, 512, key=(916,))
    r = oracle.forward(x, W)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    y_tern = xf @ (float(r["gamma"]) * r["codes"].astype(np.float64)).T
    err = np.abs(r["y"] - y_tern)
    bound = (0.5 / r["s"].astype(np.float64))[:, None] * float(r["gamma"]) * np.abs(r["codes"]).sum(1)[None, :]
    assert np.all(err <= bound * 1.0001 + 1e-6)


# =================================================================== tracker
# Two INT16 counters per weight, compare signs step to step.

def _py_flip(prev, curr, step, fc, lf):
    fc, lf = fc.copy(), lf.copy()
    for i in range(prev.size):
        p, c = float(prev[i]), float(curr[i])
        sp = (p > 0) - (p < 0)
        sc = (c > 0) - (c < 0)
        if sp != sc:
            fc[i] = min(int(fc[i]) + 1, 32767)
            lf[i] = step
    return fc, lf


def test_flip_brute_force_with_zeros():
    g = wl.rng(917)
    n = 3000
    prev = g.choice([-1.0, -0.5, 0.0, -0.0, 0.25, 1.0], size=n).astype(np.float32)
    curr = g.choice([-1.0, 0.0, 0.5, 2.0], size=n).astype(np.float32)
    fc = g.integers(0, 32768, size=n, dtype=np.int16)
    lf = g.integers(0, 1000, size=n, dtype=np.int16)
    ref = _py_flip(prev, curr, 777, fc, lf)
    out = oracle.flip_update(prev, curr, 777, fc, lf)
    assert np.array_equal(out[0], ref[0]) and np.array_equal(out[1], ref[1])


def test_flip_semantics_special_values():
    prev = np.array([1.0, 1.0, 0.0, -0.0, -2.0, 3.0], np.float32)
    curr = np.array([0.0, 2.0, -0.0, 0.0, 1.0, -3.0], np.float32)
    fc = np.array([0, 5, 7, 0, 32767, 32766], np.int16)
    lf = np.zeros(6, np.int16)
    fc2, lf2 = oracle.flip_update(prev, curr, 50, fc, lf)
    # + -> 0 is a flip; +0 vs -0 is not; saturation at 32767
    assert fc2.tolist() == [1, 5, 7, 0, 32767, 32767]
    assert lf2.tolist() == [50, 0, 0, 0, 50, 50]
    with pytest.raises(ValueError):
        oracle.flip_update(prev, curr, 0, fc, lf)
    with pytest.raises(ValueError):
        oracle.flip_update(prev, curr, 32768, fc, lf)


def test_flip_model16m_counts_and_census():
    prev, curr, mask = wl.flip_snapshots("model_16m")
    with open(os.path.join(GOLDEN, "census.json")) as f:
        census = json.load(f)
    # 42 tensors and 3,538,944 tracked weights; one INT16 array is ~7 MB
    assert len(wl.workload_tensors("model_16m")) == census["tensors"]
    assert abs(prev.size / 1e6 - census["tracked_weights_millions"]) < 0.05
    assert prev.size == 3_538_944  # 6 x (2*65536 + 2*32768 + 3*131072)
    assert abs(prev.size * 2 / 1e6 - census["mb_per_int16_array"]) < 0.1
    for scen in (1, 2):
        fc, lf, step = wl.flip_counters(prev.size, scen)
        fc2, lf2 = oracle.flip_update(prev, curr, step, fc, lf)
        assert int((fc2.astype(np.int64) - fc).sum()) == int(mask.sum())
        assert np.all(lf2[mask] == step) and np.array_equal(lf2[~mask], lf[~mask])
        # comparing a snapshot with itself changes nothing
        fc3, lf3 = oracle.flip_update(prev, prev, step, fc, lf)
        assert np.array_equal(fc3, fc) and np.array_equal(lf3, lf)


# ==================================================== binary BitNet weights
# "1-bit & Ternary LLMs (BitNet b1.58)", How it works, BitNet (binary) equations.

def test_binarise_hand_values_and_ties():
    W = np.array([[1.0, 2.0], [3.0, -6.0]], np.float32)
    codes, a, b = oracle.binarise(W)
    assert a == np.float32(0.0) and b == np.float32(3.0)  # mean 0, mean |W| = 12 / 4
    assert codes.tolist() == [[1, 1], [1, -1]]
    codes, a, b = oracle.binarise(np.array([[1.0, 2.0, 3.0]], np.float32))
    assert a == np.float32(2.0) and codes.tolist() == [[-1, 1, 1]]  # W = alpha reads as +1


def test_binarise_invariants_and_library_routine():
    W = wl.gaussian_weight(37, 301, key=(913,)) + np.float32(0.003)  # off-centre: alpha != 0
    codes, a, b = oracle.binarise(W)
    assert set(np.unique(codes).tolist()) <= {-1, 1}
    assert a == np.float32(np.mean(W.astype(np.float64)))
    assert b == np.float32(np.mean(np.abs(W.astype(np.float64))))
    assert np.array_equal(codes, np.where(W >= a, 1, -1))
    cn, an, bn = oracle.binarise(-W)  # exact negation: alpha negates, beta stays
    assert an == -a and bn == b
    ties = W == a
    assert np.array_equal(cn[~ties], -codes[~ties])
    # the codes of W and W - alpha agree with the sign of the centred matrix
    frac = float((codes == 1).mean())
    assert abs(frac - 0.5) < 5 * math.sqrt(0.25 / codes.size)


# ========================================================= tracker read-out
# "Which 1-Bit Weights Can You Trust?", Methodology: sign age is 1 for a
# weight that never flipped, flip rate is 0 for a weight that never moved.

def test_flip_stats_page_special_cases_and_closed_forms():
    T = 1000
    fc = np.array([0, 0, 1000, 3, 250], np.int16)
    lf = np.array([0, 1000, 1000, 500, 999], np.int16)
    age, rate = oracle.flip_stats(fc, lf, T)
    assert age[0] == 1.0 and rate[0] == 0.0     # never flipped: age 1, rate 0 (the page's two cases)
    assert age[1] == 0.0                         # flipped at the last step
    assert rate[2] == 1.0                        # flipped every step
    assert age[3] == np.float32(0.5) and rate[3] == np.float32(0.003)
    assert age[4] == np.float32(0.001) and rate[4] == np.float32(0.25)


# ===================================== optimiser step with the tracker fused
# "1-bit & Ternary LLMs", Training (the optimiser steps the shadow weights);
# "Which 1-Bit Weights Can You Trust?", Experimental Setup (AdamW) and
# Methodology (the tracker compares signs before and after each step).

def test_adamw_matches_torch_cpu_adamw():
    torch = pytest.importorskip("torch")
    g0 = wl.rng(914)
    n, lr = 5000, 3e-4
    W = (g0.standard_normal(n) * 0.02).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    p = torch.nn.Parameter(torch.from_numpy(W.copy()))
    opt = torch.optim.AdamW([p], lr=lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.1, foreach=False)
    for t in range(1, 8):
        g = (g0.standard_normal(n) * 0.01).astype(np.float32)
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        W, m, v, _, _ = oracle.adamw_flip(W, g, m, v, t, lr, 0.9, 0.999, 1e-8, 0.1)
        st = opt.state[p]
        assert np.abs(p.detach().numpy() - W).max() <= 1e-4 * lr  # 1-2 ulp of the weights
        assert np.abs(st["exp_avg"].numpy() - m).max() <= 1e-6 * np.abs(m).max()
        assert np.all(np.abs(st["exp_avg_sq"].numpy() - v) <= 1e-6 * v + 1e-30)


def test_adamw_closed_forms():
    W = np.array([0.5, -0.25, 1e-3, -2.0], np.float32)
    z = np.zeros(4, np.float32)
    # zero gradient: only the decoupled decay acts, exactly
    W1, m1, v1, _, _ = oracle.adamw_flip(W, z, z, z, 1, 1e-2, wd=0.1)
    assert np.array_equal(W1, W * np.float32(1.0 - 1e-2 * 0.1)) and not m1.any() and not v1.any()
    # first step, no decay, eps -> 0: the update is lr * sign(g) whatever |g|
    g = np.array([3.0, -1e-3, 0.5, -7.0], np.float32)
    W1, _, _, _, _ = oracle.adamw_flip(W, g, z, z, 1, 1e-2, eps=1e-30, wd=0.0)
    assert np.allclose(W1, W - np.float32(1e-2) * np.sign(g), rtol=0, atol=1e-8)


def test_adamw_tracker_counts_the_sign_changes():
    W = np.array([1e-7, -1e-7, 0.3, -0.3, 0.0, 1e-7], np.float32)
    g = np.array([1.0, -1.0, 1.0, -1.0, 1.0, -1.0], np.float32)  # first two and the zero cross, the rest stay
    z = np.zeros(6, np.float32)
    fc = np.array([0, 5, 0, 32767, 0, 0], np.int16)
    lf = np.array([0, 3, 9, 9, 0, 0], np.int16)
    W1, _, _, fc1, lf1 = oracle.adamw_flip(W, g, z, z, 12, 1e-3, flip_count=fc, last_flip=lf)
    assert (np.sign(W1) == np.array([-1, 1, 1, -1, -1, 1])).all()
    assert fc1.tolist() == [1, 6, 0, 32767, 1, 0] and lf1.tolist() == [12, 12, 9, 9, 12, 0]


def test_adamw_fused_tracker_equals_snapshot_tracker():
    """The fused counters after several steps equal those of the
    two-snapshot tracker run on the weights before and after each step."""
    n = 20000
    W = (wl.rng(915).standard_normal(n, dtype=np.float32) * np.float32(0.02))
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    fc = np.zeros(n, np.int16)
    lf = np.zeros(n, np.int16)
    fs, ls = fc.copy(), lf.copy()
    for t in range(1, 6):
        W0 = W
        W, m, v, fc, lf = oracle.adamw_flip(W, wl.adam_grad(n, t), m, v, t, 2e-3, wd=0.1, flip_count=fc,
                                            last_flip=lf)
        fs, ls = oracle.flip_update(W0, W, t, fs, ls)
    assert (fc > 0).sum() > 100
    assert np.array_equal(fc, fs) and np.array_equal(lf, ls)


# ====================================================== transposed layout t1
# Byte positions worked by hand from the layout t1 description in
# include/bitlinear.h (layout v1's geometry over the K x N matrix c^T; column
# t of a dword's 16 at bit 14 - t for even t, 31 - t for odd t).

def _single_t1(N, K, n, k, code):
    c = np.zeros((N, K), np.int8)
    c[n, k] = code
    return oracle.encode_t1(c)


def test_layout_t1_hand_worked_positions():
    # N=1, K=2: c^T is 2 x 1.  (k=0, n=0): lane 0, t = 0 -> bit 14 of dword 0;
    # (k=1, n=0): lane 1 -> dword 1, bit 14.
    c = np.array([[1, -1]], np.int8)
    p = oracle.encode_t1(c)
    assert p.size == 256
    assert np.flatnonzero(p).tolist() == [1, 5] and p[1] == 0x40 and p[5] == 0xC0
    # N=2, K=1: (n=1, k=0) is column t = 1 -> bit 30 -> byte 3, shift 6
    p = _single_t1(2, 1, 1, 0, -1)
    assert np.flatnonzero(p).tolist() == [3] and p[3] == 0xC0
    # N=300, K=20: c^T has two 16-row blocks and five 64-column fragments
    # (groups of 4 and 1).  (n=290, k=17): block 1, fragment 4, lane 1 + 16*2 =
    # 33, t = 2 -> bit 12; dword 1*5*64 + 256 + 33 = 609 -> byte 2437, shift 4.
    p = _single_t1(300, 20, 290, 17, 1)
    assert p.size == 2560
    assert np.flatnonzero(p).tolist() == [2437] and p[2437] == 0x10
    # (n=70, k=5): fragment 1 of group 0 (size 4), lane 5, t = 6 -> bit 8;
    # dword 5*4 + 1 = 21 -> byte 85, shift 0.  (n=79, k=5): t = 15 -> bit 16,
    # byte 86, shift 0.
    p = _single_t1(300, 20, 70, 5, -1)
    assert np.flatnonzero(p).tolist() == [85] and p[85] == 0x03
    p = _single_t1(300, 20, 79, 5, -1)
    assert np.flatnonzero(p).tolist() == [86] and p[86] == 0x03


def test_layout_t1_round_trip_and_same_dwords_as_v1_of_transpose():
    for (N, K) in [(1, 1), (16, 64), (17, 65), (300, 20), (64, 1024), (130, 33)]:
        W = wl.gaussian_weight(N, K, key=(916, N, K))
        c = oracle.ternarise(W, oracle.gamma(W), 1e-5)
        p = oracle.encode_t1(c)
        assert p.size == oracle.packed_bytes(K, N)
        assert np.array_equal(oracle.decode_t1(p, N, K), c)
        # each dword holds the same 16 codes as layout v1 of c^T, reordered:
        # same count of nonzero codes and of -1 codes per dword
        v = oracle.encode(np.ascontiguousarray(c.T)).view(np.uint32)
        t = p.view(np.uint32)

        def counts(words):
            f = (words[:, None] >> (2 * np.arange(16, dtype=np.uint32))[None, :]) & 3
            return (f != 0).sum(1), (f == 3).sum(1)

        assert all(np.array_equal(a, b) for a, b in zip(counts(v), counts(t)))
    bad = oracle.encode_t1(np.zeros((16, 64), np.int8))
    bad[1] = 0x80  # code 10 at bit 14
    with pytest.raises(ValueError):
        oracle.decode_t1(bad, 16, 64)
    pad = oracle.encode_t1(np.zeros((5, 3), np.int8))
    pad[3 * 4 + 1] = 0x40  # row k = 3 is padding of K = 3
    with pytest.raises(ValueError):
        oracle.decode_t1(pad, 5, 3)


# ===================================================== one-bit layout b1
# Byte positions worked by hand from the layout b1 description in
# include/bitlinear.h (16-row x 128-column pairs, groups of up to four pairs,
# dword lam of pair f at lam*G + f; code t of half h at bit
# 8*(t % 4) + 7 - (4h + t // 4); bit 1 is -1).

def _single_b1(N, K, n, k):
    c = np.ones((N, K), np.int8)
    c[n, k] = -1
    return oracle.encode_b1(c)


def test_layout_b1_hand_worked_positions():
    # N=16, K=128: one pair.  (0, 0): lane 0, half 0, t = 0 -> bit 7 of dword 0.
    p = _single_b1(16, 128, 0, 0)
    assert p.size == 256
    assert np.flatnonzero(p).tolist() == [0] and p[0] == 0x80
    # (3, 85): half 1, column 21 -> lane 3 + 16 = 19, t = 5 -> bit 8 + 7 - 5 = 10;
    # byte 19*4 + 1 = 77, shift 2.
    p = _single_b1(16, 128, 3, 85)
    assert np.flatnonzero(p).tolist() == [77] and p[77] == 0x04
    # N=16, K=64: half a pair.  (0, 63): lane 48, t = 15 -> bit 24 + 7 - 3 = 28;
    # byte 195, shift 4.
    p = _single_b1(16, 64, 0, 63)
    assert p.size == 256
    assert np.flatnonzero(p).tolist() == [195] and p[195] == 0x10
    # N=16, K=384: one group of three pairs.  (5, 286): pair 2, half 0, column 30
    # -> lane 21, t = 14 -> bit 16 + 7 - 3 = 20; dword 21*3 + 2 = 65 -> byte 262,
    # shift 4.
    p = _single_b1(16, 384, 5, 286)
    assert p.size == 768
    assert np.flatnonzero(p).tolist() == [262] and p[262] == 0x10
    # N=20, K=640: two row blocks, five pairs (groups of 4 and 1).  (17, 600):
    # block 1, pair 4 (group 1, size 1), half 1, column 24 -> lane 17, t = 8 ->
    # bit 0 + 7 - 6 = 1; dword 1*5*64 + 256 + 17 = 593 -> byte 2372, shift 1.
    p = _single_b1(20, 640, 17, 600)
    assert p.size == 2560
    assert np.flatnonzero(p).tolist() == [2372] and p[2372] == 0x02


def test_layout_b1_round_trip_padding_and_counts():
    for (N, K) in [(16, 64), (17, 64), (33, 320), (5, 1024), (64, 1088), (130, 640)]:
        W = wl.gaussian_weight(N, K, key=(931, N, K))
        c, _, _ = oracle.binarise(W)
        p = oracle.encode_b1(c)
        assert p.size == ((N + 15) // 16) * ((K + 127) // 128) * 256 == oracle.packed_bytes_b1(N, K)
        assert np.array_equal(oracle.decode_b1(p, N, K), c)
        # one set bit per -1 code, none elsewhere
        assert int(np.unpackbits(p).sum()) == int((c == -1).sum())
    # a set padding bit: row 17 of N = 17, and the missing half pair of K = 64
    p = oracle.encode_b1(np.ones((17, 64), np.int8))
    probe = np.ones((32, 64), np.int8)
    probe[17, 0] = -1
    bad = p | oracle.encode_b1(probe)
    with pytest.raises(ValueError):
        oracle.decode_b1(bad, 17, 64)
    probe = np.ones((16, 128), np.int8)
    probe[0, 64] = -1
    bad = oracle.encode_b1(np.ones((16, 64), np.int8)) | oracle.encode_b1(probe)
    with pytest.raises(ValueError):
        oracle.decode_b1(bad, 16, 64)
    # no zero code, and K must be a multiple of 64
    with pytest.raises(ValueError):
        oracle.encode_b1(np.zeros((16, 64), np.int8))
    with pytest.raises(ValueError):
        oracle.packed_bytes_b1(16, 96)


# ================================================ base-3 layout t3
# Byte values worked by hand from the layout t3 text in oracle/bitlinear_oracle.c
# (five codes per byte as base-3 digits code + 1 of weights 1, 3, 9, 27, 81;
# byte 16*lam + t of a 1024-byte group holds row lam % 16, column
# 64 f + 16 (lam / 16) + t of fragment f).

def test_layout_t3_hand_worked_bytes():
    # all-zero codes: every digit 1 -> 1 + 3 + 9 + 27 + 81 = 121
    p = oracle.encode_t3(np.zeros((16, 320), np.int8))
    assert p.size == 1024 and (p == 121).all()
    # (0, 0) = +1: byte 0, digit 2 at weight 1 -> 122
    c = np.zeros((16, 320), np.int8)
    c[0, 0] = 1
    p = oracle.encode_t3(c)
    assert np.flatnonzero(p != 121).tolist() == [0] and p[0] == 122
    # (3, 64*4 + 16 + 5) = (3, 277) = -1: fragment 4, lane 3 + 16 = 19, t = 5 ->
    # byte 16*19 + 5 = 309, digit 0 at weight 81 -> 121 - 81 = 40
    c = np.zeros((16, 320), np.int8)
    c[3, 277] = -1
    p = oracle.encode_t3(c)
    assert np.flatnonzero(p != 121).tolist() == [309] and p[309] == 40
    # five codes sharing one byte: row 5, t = 2 of lane 5 in fragments 0..4 =
    # columns 2, 66, 130, 194, 258 with codes -1, 0, 1, 1, -1 -> digits 0, 1, 2, 2, 0
    # -> 0 + 3 + 18 + 54 + 0 = 75 at byte 16*5 + 2 = 82; second group (K = 640),
    # second row block (N = 20): row 17 -> block 1, group 1 -> byte (2 + 1) * 1024 + 16*1 + 2
    c = np.zeros((20, 640), np.int8)
    for col, v in zip((2, 66, 130, 194, 258), (-1, 0, 1, 1, -1)):
        c[5, col] = v
        c[17, 320 + col] = v
    p = oracle.encode_t3(c)
    assert p.size == 4096
    assert np.flatnonzero(p != 121).tolist() == [82, 3 * 1024 + 18] and p[82] == 75 and p[3 * 1024 + 18] == 75


def test_layout_t3_round_trip_and_size():
    for (N, K) in [(16, 320), (17, 640), (33, 960), (5, 3200)]:
        W = wl.gaussian_weight(N, K, key=(941, N, K))
        c = oracle.ternarise(W, oracle.gamma(W), 1e-5)
        p = oracle.encode_t3(c)
        assert p.size == ((N + 15) // 16) * (K // 320) * 1024 == oracle.packed_bytes_t3(N, K)
        assert p.max() <= 242
        assert np.array_equal(oracle.decode_t3(p, N, K), c)
    # 0.8 of the bytes of layout v1 at the same shape
    assert oracle.packed_bytes_t3(16, 3200) * 5 == oracle.packed_bytes(16, 3200) * 4
    with pytest.raises(ValueError):
        oracle.packed_bytes_t3(16, 64)
    bad = oracle.encode_t3(np.zeros((16, 320), np.int8))
    bad[7] = 243
    with pytest.raises(ValueError):
        oracle.decode_t3(bad, 16, 320)


# ============================================== STE backward to the input
# "1-bit & Ternary LLMs (BitNet b1.58)", Training: the forward uses the
# ternary weights, the straight-through estimator makes the quantisers
# identities for the gradient.

def _bwd_case(M, N, K, key):
    W = wl.gaussian_weight(N, K, key=(917, N, K) + key)
    _, g, codes = oracle.pack(W)
    dy = wl.activation(M, N, key=(918, M, N) + key)
    return W, g, codes, dy


def test_backward_matches_autograd_through_the_ste():
    torch = pytest.importorskip("torch")
    M, N, K = 7, 40, 24
    W, g, codes, dy = _bwd_case(M, N, K, (0,))
    x = wl.activation(M, K, key=(919,))
    q, s = oracle.quant_act(x)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    xt = torch.tensor(wl.bf16_bits_to_f32(x), dtype=torch.float64, requires_grad=True)
    w_eff = Wt + (float(g) * torch.tensor(codes, dtype=torch.float64) - Wt).detach()
    xq = xt + (torch.tensor(q, dtype=torch.float64) / torch.tensor(s, dtype=torch.float64)[:, None] - xt).detach()
    y = xq @ w_eff.T
    dyt = torch.tensor(wl.bf16_bits_to_f32(dy), dtype=torch.float64)
    y.backward(dyt)
    ref, mag, _ = oracle.backward_input(dy, codes, g)
    assert np.allclose(xt.grad.numpy(), ref, rtol=1e-12, atol=1e-300)
    assert np.all(mag >= np.abs(ref) - 1e-12 * mag)
    # the weight gradient is passed straight through: dy^T times the
    # dequantised activations, no BitNet-specific work
    xhat = q.astype(np.float64) / s.astype(np.float64)[:, None]
    assert np.allclose(Wt.grad.numpy(), dyt.numpy().T @ xhat, rtol=1e-12)


def test_backward_one_hot_closed_form():
    M, N, K = 3, 20, 70
    _, g, codes, _ = _bwd_case(M, N, K, (1,))
    dy = np.zeros((M, N), np.uint16)
    dy[1, 13] = wl.f32_to_bf16_bits(np.float32([1.0]))[0]
    dy[2, 0] = wl.f32_to_bf16_bits(np.float32([-1.0]))[0]
    ref, _, dx = oracle.backward_input(dy, codes, g)
    assert not ref[0].any()
    assert np.array_equal(ref[1], float(g) * codes[13])
    assert np.array_equal(ref[2], -float(g) * codes[0])
    gb = wl.f32_to_bf16_bits(np.float32([g]))[0]
    assert np.array_equal(dx[1], np.where(codes[13] == 0, 0, np.where(codes[13] > 0, gb, gb | 0x8000)))


def test_backward_integer_dy_is_exact_in_bf16():
    torch = pytest.importorskip("torch")
    M, N, K = 6, 96, 50
    _, g, codes, _ = _bwd_case(M, N, K, (2,))
    ints = wl.rng(920).integers(-8, 9, size=(M, N)).astype(np.float32)
    dy = wl.f32_to_bf16_bits(ints)
    S = ints.astype(np.int64) @ codes.astype(np.int64)
    prev = wl.f32_to_bf16_bits(wl.rng(921).standard_normal((M, K), dtype=np.float32))
    for p in (None, prev):
        _, _, dx = oracle.backward_input(dy, codes, g, dx_prev=p)
        v = torch.tensor(S.astype(np.float32)) * torch.tensor(np.float32(g))
        if p is not None:
            v = v + torch.tensor(wl.bf16_bits_to_f32(p))
        want = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(dx, want)


def test_backward_tolerance_catches_a_lost_term():
    """A plausible bug (one output feature's term lost) fails the checks that
    the exact answer passes."""
    M, N, K = 64, 512, 96
    _, g, codes, dy = _bwd_case(M, N, K, (3,))
    ref, mag, dx = oracle.backward_input(dy, codes, g)
    good = wl.bf16_bits_to_f32(dx)
    assert oracle.dx_close(good, ref, mag, N).all()
    assert oracle.dx_rel_rms(good, ref) <= 2.0 ** -9
    broken = codes.copy()
    broken[17] = 0
    _, _, dxb = oracle.backward_input(dy, broken, g)
    assert oracle.dx_rel_rms(wl.bf16_bits_to_f32(dxb), ref) > 2.0 ** -8


def test_chained_backward_tolerance():
    """The bound the grouped input gradient is held to: the oracle applied
    entry by entry (each step rounded to bf16) passes it, and the same chain
    with one entry's term lost, or with an entry left out, fails it."""
    from gpu_util import compare_dx_chain
    M, K = 64, 96
    Ns = [512, 136, 264]
    cases = [_bwd_case(M, N, K, (4, e)) for e, N in enumerate(Ns)]
    prev = wl.activation(M, K, key=(1690, M, K))
    for start in (None, prev):
        parts, chain = [], start
        for _, g, codes, dy in cases:
            ref, mag, _ = oracle.backward_input(dy, codes, g)
            _, _, chain = oracle.backward_input(dy, codes, g, dx_prev=chain)
            parts.append((ref, mag))
        addend = None if start is None else wl.bf16_bits_to_f32(start)
        compare_dx_chain(wl.bf16_bits_to_f32(chain), parts, Ns, addend)
        # an entry left out
        _, _, short = oracle.backward_input(cases[1][3], cases[1][2], cases[1][1], dx_prev=start)
        with pytest.raises(AssertionError):
            compare_dx_chain(wl.bf16_bits_to_f32(short), parts, Ns, addend)
        # one feature of the middle entry lost
        broken = cases[1][2].copy()
        broken[5] = 0
        chain = start
        for e, (_, g, codes, dy) in enumerate(cases):
            _, _, chain = oracle.backward_input(dy, broken if e == 1 else codes, g, dx_prev=chain)
        with pytest.raises(AssertionError):
            compare_dx_chain(wl.bf16_bits_to_f32(chain), parts, Ns, addend)


# ====================================================== acceptance predicates
# The rule every GPU parity verdict goes through: bf16 y within 1e-3 absolute
# + 1e-2 relative of the fp32 reference; a code mismatch tolerated only where
# the rounded quantity sits within 1e-6 relative of a .5 rounding boundary
# (the RoundClip of "1-bit & Ternary LLMs (BitNet b1.58)", How it works, b1.58
# equations, and the rounding of the int8 activation quantiser).  Each pin
# puts hand-chosen points just inside and just outside each boundary.

def test_y_close_hand_values_on_both_sides_of_the_bound():
    # y_ref = 100: bound 1e-3 + 1.0 = 1.001
    ref = np.array([100.0, 100.0, 100.0, 100.0])
    y = np.array([100.9, 101.0009, 101.0011, 98.998])
    assert oracle.y_close(y, ref).tolist() == [True, True, False, False]
    # y_ref = 0: only the absolute 1e-3 remains
    ref0 = np.zeros(4)
    assert oracle.y_close(np.array([0.0009, -0.0009, 0.0011, -0.0011]), ref0).tolist() == [True, True, False, False]
    # negative reference: the relative term uses |y_ref|: -50 -> bound 0.501
    refn = np.full(4, -50.0)
    assert oracle.y_close(np.array([-50.5, -49.5, -50.502, -49.498]), refn).tolist() == [True, True, False, False]
    # one ulp of fp64 either side of the exact bound at y_ref = 2 (bound 0.021)
    b = 1e-3 + 1e-2 * 2.0
    inside = np.nextafter(2.0 + b, 0.0)
    outside = np.nextafter(np.nextafter(2.0 + b, 10.0), 10.0)
    assert oracle.y_close(np.array([inside, outside]), np.array([2.0, 2.0])).tolist() == [True, False]


def test_y_close_planted_tolerance_swap_is_caught():
    # the same points judged with atol and rtol swapped give other verdicts,
    # so a swap inside y_close cannot pass the hand values above
    ref = np.array([100.0, 0.0])
    y = np.array([100.9, 0.005])
    assert oracle.y_close(y, ref).tolist() == [True, False]
    assert oracle.y_close(y, ref, atol=1e-2, rtol=1e-3).tolist() == [False, True]


def test_weight_boundary_mask_hand_values():
    # gamma = 0.02, eps = 0: the window is |W| in 0.01 * (1 +- 1e-6)
    g = np.float32(0.02)
    W = np.array([0.01, 0.01 * (1 + 0.9e-6), 0.01 * (1 - 0.9e-6), -0.01 * (1 + 0.9e-6),
                  0.01 * (1 + 1.1e-6), 0.01 * (1 - 1.1e-6), -0.01 * (1 - 1.1e-6),
                  0.03, 0.0, 0.02])
    want = [True, True, True, True, False, False, False, False, False, False]
    # compare in fp64 against the fp64 ratio: g is the fp32 value 0.02 exactly as stored
    ratio_center = 0.5 * float(g)
    W = W / 0.01 * ratio_center
    assert oracle.weight_boundary_mask(W, g, eps=0.0).tolist() == want
    # eps sits in the denominator: with eps = 1e-5 the centre moves to
    # 0.5 * (gamma + eps), so the old centre falls out and the new one is in
    c2 = 0.5 * (float(g) + 1e-5)
    m = oracle.weight_boundary_mask(np.array([ratio_center, c2, -c2]), g, eps=1e-5)
    assert m.tolist() == [False, True, True]
    # 1.5 (the +-1 / clip boundary) never counts: both sides clip to +-1
    assert not oracle.weight_boundary_mask(np.array([3 * ratio_center]), g, eps=0.0).any()


def test_half_window_mask_hand_values():
    v = np.array([2.5, 2.5 * (1 + 0.9e-6), 2.5 * (1 - 0.9e-6), -3.5 * (1 + 0.9e-6), 0.5 * (1 + 0.9e-6), 126.5,
                  2.5 * (1 + 1.1e-6), 2.5 * (1 - 1.1e-6), -3.5 * (1 - 1.1e-6), 3.0, 0.0, 2.4999])
    want = [True] * 6 + [False] * 6
    assert oracle.half_window_mask(v).tolist() == want
    # the window widens with the boundary: rel * b, not a fixed 1e-6
    assert oracle.half_window_mask(np.array([100.5 + 9e-5, 100.5 + 1.1e-4])).tolist() == [True, False]
