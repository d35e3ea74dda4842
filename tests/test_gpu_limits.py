"""GPU parity at the largest sizes the library accepts.

* The reduction length: K up to BITLINEAR_MAX_K = 16909320, the largest K for
  which 127 * K still fits an int32 accumulator.  Every code +-1 against
  q = +-127 drives |acc| to 127 * K (2147483640 at the limit) on each kernel
  family that takes such a K: the decode kernels (1 and 3 tokens), the decode
  batch cut into K runs (16 tokens), and the generic kernels for a K that is
  not a multiple of 16.
* The activation buffer: the fast kernels address the int8 tokens with 32-bit
  offsets and take M * K below 2^31 - 2^20; at K = 8192 that is M = 262015
  (the prefill GEMM) and M = 262017 is the first past it (the generic GEMM
  with 64-bit offsets).  Random codes and tokens, accumulators and outputs
  compared on sampled rows (the first, the last and random ones).
* Packing at K = BITLINEAR_MAX_K: gamma over 338M weights and the layout's
  partial last fragment.
"""

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import compare_codes, compare_y, dev, host, host_bf16_f32, say

pytestmark = pytest.mark.gpu

MAX_K = 16909320  # BITLINEAR_MAX_K (include/bitlinear.h)


@pytest.fixture(scope="module")
def bl():
    import torch
    assert torch.cuda.is_available(), "no GPU"
    import bitlinear_absmean_ternarise_amd as m
    return m


def _extreme_codes(N, K):
    codes = np.ones((N, K), np.int8)
    codes[1::2] = -1
    codes[3, ::7] = 0
    return codes


@pytest.mark.parametrize("K", [MAX_K - 8, MAX_K])
@pytest.mark.parametrize("M", [1, 3, 16])
def test_forward_max_k_extreme_sums(bl, M, K):
    """|acc| = 127 K at the largest K: K = MAX_K - 8 (a multiple of 16: the
    decode kernels, and the K-run GEMM at 16 tokens) and K = MAX_K (a
    multiple of 8 only: the generic kernels)."""
    say("forward max K", M, K)
    N = 20
    codes = _extreme_codes(N, K)
    packed = oracle.encode(codes)
    q = np.full((M, K), 127, np.int8)
    q[M // 2] = -127
    q[-1, ::3] = -127
    s = np.full(M, 1.0, np.float32)
    s[0] = np.float32(250.0)
    g = np.float32(0.015)
    acc_ref = oracle.contract(q, codes)
    assert abs(int(acc_ref[0, 0])) == 127 * K
    y, acc = bl.forward(dev(packed), dev(np.array([g], np.float32)), N, K, dev(q), dev(s), acc=True)
    assert np.array_equal(host(acc), acc_ref)
    compare_y(host_bf16_f32(y), oracle.epilogue(acc_ref, g, s), f"max K M={M} K={K}")


@pytest.mark.parametrize("M", [262015, 262017])
def test_forward_largest_activation_buffer(bl, M):
    """M * K just below the fast kernels' 2^31 - 2^20 bound (the prefill GEMM)
    and just past it (the generic GEMM), K = 8192; sampled rows."""
    import torch
    K, N = 8192, 40
    say("forward largest activation buffer", M, N, K)
    W = wl.gaussian_weight(N, K, key=(1500, N, K))
    packed, g, codes = oracle.pack(W, 1e-5)
    r = wl.rng(1501, M, K)
    q = r.integers(-127, 128, size=(M, K), dtype=np.int8)
    s = r.uniform(0.5, 200.0, size=M).astype(np.float32)
    acc_d = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = bl.forward(dev(packed), dev(np.array([g], np.float32)), N, K, dev(q), dev(s), acc=acc_d)[0]
    rows = np.unique(np.concatenate([np.arange(64), np.arange(M - 200, M), r.integers(0, M, 256)]))
    acc_ref = oracle.contract(q[rows], codes)
    acc_g = host(acc_d[torch.from_numpy(rows).cuda()])
    assert np.array_equal(acc_g, acc_ref)
    y_g = host_bf16_f32(y[torch.from_numpy(rows).cuda()].contiguous())
    compare_y(y_g, oracle.epilogue(acc_ref, g, s[rows]), f"largest buffer M={M}")


def test_pack_max_k(bl):
    """gamma and the codes of a 20 x BITLINEAR_MAX_K tensor (K % 64 = 8: the
    last fragment of every row block is partial)."""
    N, K = 20, MAX_K
    say("pack max K", N, K)
    W = wl.gaussian_weight(N, K, key=(1502, N, K))
    ref_packed, ref_g, _ = oracle.pack(W, 1e-5)
    packed, g = bl.pack_weights(dev(W), 1e-5)
    g = host(g)[0]
    assert g == ref_g, f"gamma {g!r} vs oracle {ref_g!r}"
    assert compare_codes(host(packed), ref_packed, N, K, W, ref_g, 1e-5) == 0
