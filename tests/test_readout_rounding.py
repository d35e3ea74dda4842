"""The tracker read-out divides in fp32 where the definition ("Which 1-Bit
Weights Can You Trust?", Methodology: sign age (T - last_flip) / T, flip rate
flip_count / T) is read as an fp64 quotient rounded once to fp32.  The two
agree for every input the entry point accepts (T in 1..32767, int16
counters): both numerators and T are exact in fp32, fp32 division is
correctly rounded, and an fp64 quotient of fp32 operands rounds to the
correctly rounded fp32 quotient (53 >= 2 * 24 + 2 bits; Figueroa, "When is
double rounding innocuous?").  Checked here with numpy's IEEE divisions:
every numerator the counters can produce, for every T up to 1024 and for 600
seeded T up to 32767."""
import numpy as np

A_ALL = np.arange(-32768, 32767 + 32768 + 1, dtype=np.int64)  # T - last_flip and flip_count


def _ref(T, a):
    return (a.astype(np.float64) / np.float64(T)).astype(np.float32)


def _ts():
    rng = np.random.default_rng(20260)
    return list(range(1, 1025)) + sorted(set(int(t) for t in rng.integers(1025, 32768, 600))) + [32767]


def test_fp32_division_matches_rounded_fp64_quotient():
    for T in _ts():
        f32 = A_ALL.astype(np.float32) / np.float32(T)
        assert np.array_equal(_ref(T, A_ALL).view(np.uint32), f32.view(np.uint32)), T


def test_reciprocal_multiply_would_be_caught():
    # a cheaper reading (multiply by an fp32 reciprocal) differs on some
    # inputs, so the comparison above is not vacuous
    bad = 0
    for T in _ts()[::20]:
        rec = A_ALL.astype(np.float32) * (np.float32(1.0) / np.float32(T))
        bad += int(np.count_nonzero(_ref(T, A_ALL).view(np.uint32) != rec.view(np.uint32)))
    assert bad > 0
