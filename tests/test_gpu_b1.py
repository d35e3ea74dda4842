"""GPU parity of binary weights stored one bit per code (layout b1) against
the CPU oracle: packed bytes, beta and alpha bit-exact (the rule W >= alpha
compares without rounding, so there is no window), int32 accumulators
bit-exact, bf16 outputs within 1e-3 + 1e-2 |y| of the oracle's fp32 result
and bit-identical to the two-bit forward over the same codes.

Shapes cover one pair (K = 64, the second half padding), K with an odd
number of fragments (in a partial last group, or in a last group of four
pairs whose final half is padding: K = 448 mod 512), full groups with a
partial last group of 1..3 pairs,
ragged N, token tiles of 16 with a partial last tile (M = 17, 33, 100), the
longest row of the 70B layer, grouped calls with an empty entry, and the 70B
layer at full size on sampled outputs, grouped as a decode step groups it.
"""

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import compare_y, dev, host, host_bf16_bits, host_bf16_f32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    import torch
    assert torch.cuda.is_available(), "no GPU"
    import bitlinear_absmean_ternarise_amd as m
    return m


PACK = [(16, 64), (17, 64), (1, 128), (33, 320), (512, 256), (130, 4160), (1100, 4096), (40, 1088)]


@pytest.mark.parametrize("N,K", PACK)
def test_pack_b1_parity(bl, N, K):
    say("pack b1", N, K)
    W = wl.gaussian_weight(N, K, key=(1800, N, K)) + np.float32(0.004)
    ref_packed, ref_b, ref_a, _ = oracle.pack_binary_b1(W)
    packed, b, a = bl.pack_binary_b1(dev(W))
    assert host(b)[0] == ref_b and host(a)[0] == ref_a
    assert np.array_equal(host(packed), ref_packed)


def test_pack_b1_ties_and_scalars_of_the_two_bit_pack(bl):
    say("pack b1 ties")
    W = np.tile(np.array([1.0, 2.0, 3.0, 2.0], np.float32), (16, 32))  # alpha = 2 exactly: W = alpha -> +1
    ref_packed, ref_b, ref_a, codes = oracle.pack_binary_b1(W)
    packed, b, a = bl.pack_binary_b1(dev(W))
    assert ref_a == np.float32(2.0) and host(a)[0] == ref_a
    assert np.array_equal(host(packed), ref_packed)
    assert np.array_equal(oracle.decode_b1(host(packed), 16, 128), codes)
    _, b2, a2 = bl.pack_binary(dev(W))
    assert host(b2)[0] == host(b)[0] and host(a2)[0] == host(a)[0]


def _case(M, N, K, key):
    W = wl.gaussian_weight(N, K, key=(key, N, K))
    x = wl.activation(M, K, key=(key + 1, M, K), recipe="channels")
    _, b, _, codes = oracle.pack_binary_b1(W)
    q, s = oracle.quant_act(x, 1e-5)
    acc = oracle.contract(q, codes)
    return W, b, codes, q, s, acc


FWD = [(1, 512, 256), (1, 300, 64), (1, 17, 192), (2, 100, 1088), (5, 1030, 3200), (8, 64, 4096), (16, 200, 8192),
       (17, 130, 640), (33, 77, 2048), (64, 256, 576), (100, 48, 1024), (1, 40, 28672), (3, 24, 1536), (9, 16, 1344),
       (1, 64, 448), (3, 40, 960), (20, 33, 4032), (1, 9000, 1024), (2, 10000, 640),
       (1, 20000, 512)]


@pytest.mark.parametrize("M,N,K", FWD)
def test_forward_b1_parity(bl, M, N, K):
    say("forward b1", M, N, K)
    W, b, codes, q, s, acc_ref = _case(M, N, K, 1810)
    pk, bd, _ = bl.pack_binary_b1(dev(W))
    dq, ds = dev(q), dev(s)
    y, acc = bl.forward_b1(pk, bd, N, K, dq, ds, acc=True)
    assert np.array_equal(host(acc), acc_ref), f"M={M} N={N} K={K}: accumulators differ"
    compare_y(host_bf16_f32(y), oracle.epilogue(acc_ref, b, s), f"b1 M={M} N={N} K={K}")
    y_only = bl.forward_b1(pk, bd, N, K, dq, ds)
    assert np.array_equal(host_bf16_bits(y_only), host_bf16_bits(y))
    # the two-bit layout of the same codes gives the same bits
    pk2, bd2, _ = bl.pack_binary(dev(W))
    y2 = bl.forward(pk2, bd2, N, K, dq, ds)
    assert np.array_equal(host_bf16_bits(y2), host_bf16_bits(y)), "b1 and v1 forwards differ"


def test_forward_b1_extreme_accumulators(bl):
    """Every token at +-127 against all-(-1) / all-(+1) rows at the longest K
    the layout takes: |acc| = 127 K, the most the 64 * code sums can hold."""
    say("forward b1 extremes")
    M, N, K = 4, 32, 262080
    W = np.ones((N, K), np.float32)
    W[::2] = -1.0
    q = np.full((M, K), 127, np.int8)
    q[1] = -127
    q[2, ::2] = -127
    s = np.full(M, 1.0, np.float32)
    _, b, _, codes = oracle.pack_binary_b1(W)
    acc_ref = oracle.contract(q, codes)
    assert np.abs(acc_ref).max() == 127 * K
    pk, bd, _ = bl.pack_binary_b1(dev(W))
    y, acc = bl.forward_b1(pk, bd, N, K, dev(q), dev(s), acc=True)
    assert np.array_equal(host(acc), acc_ref)
    compare_y(host_bf16_f32(y), oracle.epilogue(acc_ref, b, s), "b1 extremes")


@pytest.mark.parametrize("M", [1, 8, 20])
def test_forward_b1_grouped_shared_tokens_and_empty_entry(bl, M):
    import torch
    say("forward b1 grouped", M)
    K = 1024
    x = wl.activation(M, K, key=(1821, M, K), recipe="channels")
    q, s = oracle.quant_act(x, 1e-5)
    dq, ds = dev(q), dev(s)
    ents, refs = [], []
    for i, N in enumerate((1024, 128, 144, 80)):
        W = wl.gaussian_weight(N, K, key=(1822 + i, N, K))
        _, b, _, codes = oracle.pack_binary_b1(W)
        pk, bd, _ = bl.pack_binary_b1(dev(W))
        ents.append(dict(packed=pk, gamma=bd, N=N, K=K, xq=dq, x_scale=ds,
                         y=torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda"),
                         acc=torch.full((M, N), -7, dtype=torch.int32, device="cuda")))
        refs.append((b, oracle.contract(q, codes)))
    # an empty entry (no tokens) is skipped
    W0 = wl.gaussian_weight(64, K, key=(1830, 64, K))
    pk0, bd0, _ = bl.pack_binary_b1(dev(W0))
    ents.insert(2, dict(packed=pk0, gamma=bd0, N=64, K=K, xq=dq[:0], x_scale=ds[:0],
                        y=torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")))
    bl.forward_b1_grouped(ents)
    ents.pop(2)
    for (b, acc_ref), e in zip(refs, ents):
        assert np.array_equal(host(e["acc"]), acc_ref), f"grouped N={e['N']}: accumulators differ"
        compare_y(host_bf16_f32(e["y"]), oracle.epilogue(acc_ref, b, s), f"grouped b1 N={e['N']}")


# the activation quant and the b1 forward in one call: one launch for decode
# (one token with K <= 32768, or 2..16 tokens with M * K <= 16384), else a
# quant launch per distinct input and the grouped b1 forward
QF_FUSED = [(1, 512, 256), (1, 300, 64), (1, 17, 192), (1, 100, 8640), (1, 64, 28672), (1, 40, 32768),
            (2, 100, 1088), (4, 1030, 3200), (16, 200, 1024), (3, 33, 448), (9, 64, 960), (1, 9000, 1024),
            (2, 10000, 640), (1, 20000, 512)]
QF_FALLBACK = [(1, 40, 32832), (17, 130, 640), (8, 64, 4096), (40, 100, 1536)]


@pytest.mark.parametrize("M,N,K", QF_FUSED + QF_FALLBACK)
def test_quant_forward_b1(bl, M, N, K):
    import torch
    say("quant_forward b1", M, N, K)
    W = wl.gaussian_weight(N, K, key=(1850, N, K))
    x = wl.activation(M, K, key=(1851, M, K), recipe="channels")
    _, b, _, codes = oracle.pack_binary_b1(W)
    q, s = oracle.quant_act(x, 1e-5)
    acc_ref = oracle.contract(q, codes)
    pk, bd, _ = bl.pack_binary_b1(dev(W))
    from gpu_util import dev_bf16
    xd = dev_bf16(x)
    e = dict(packed=pk, gamma=bd, N=N, K=K, x=xd,
             y=torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda"),
             acc=torch.full((M, N), -7, dtype=torch.int32, device="cuda"),
             xq=torch.full((M, K), 99, dtype=torch.int8, device="cuda"),
             x_scale=torch.full((M,), -1.0, dtype=torch.float32, device="cuda"))
    y, xq, xs = bl.quant_forward_b1_grouped([e])[0]
    assert np.array_equal(host(xq), q) and np.array_equal(host(xs), s), "activation codes / scales differ"
    assert np.array_equal(host(e["acc"]), acc_ref), f"M={M} N={N} K={K}: accumulators differ"
    compare_y(host_bf16_f32(y), oracle.epilogue(acc_ref, b, s), f"quant_forward b1 M={M} N={N} K={K}")
    y2 = bl.forward_b1(pk, bd, N, K, xq, xs)
    assert np.array_equal(host_bf16_bits(y2), host_bf16_bits(y)), "differs from quant + b1 forward"


@pytest.mark.parametrize("M", [1, 4])
def test_quant_forward_b1_shared_input_and_empty_entry(bl, M):
    import torch
    from gpu_util import dev_bf16
    say("quant_forward b1 shared", M)
    K = 2048
    x = wl.activation(M, K, key=(1860, M, K), recipe="channels")
    q, s = oracle.quant_act(x, 1e-5)
    xd = dev_bf16(x)
    ents, refs = [], []
    for i, N in enumerate((2048, 256, 256)):
        W = wl.gaussian_weight(N, K, key=(1861 + i, N, K))
        _, b, _, codes = oracle.pack_binary_b1(W)
        pk, bd, _ = bl.pack_binary_b1(dev(W))
        ents.append(dict(packed=pk, gamma=bd, N=N, K=K, x=xd,
                         y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
                         acc=torch.empty((M, N), dtype=torch.int32, device="cuda")))
        refs.append((b, oracle.contract(q, codes)))
    empty = dict(ents[0], x=xd[:0], y=torch.empty((0, 2048), dtype=torch.bfloat16, device="cuda"))
    del empty["acc"]
    out = bl.quant_forward_b1_grouped(ents + [empty])
    assert out[0][1].data_ptr() == out[1][1].data_ptr() == out[2][1].data_ptr()
    for (b, acc_ref), e, o in zip(refs, ents, out):
        assert np.array_equal(host(e["acc"]), acc_ref)
        compare_y(host_bf16_f32(o[0]), oracle.epilogue(acc_ref, b, s), f"quant_forward b1 shared N={e['N']}")


# ---------------------------------------- the 70B layer at full size, sampled

def _sampled(y, acc, codes, b, q, s, key, what):
    M, N = y.shape
    g = wl.rng(1840, *key)
    rows = np.unique(np.r_[np.arange(min(N, 32)), np.arange(N - 32, N), g.integers(0, N, 384)]).astype(np.int64)
    m_idx = np.repeat(np.arange(M, dtype=np.int64), rows.size)
    n_idx = np.tile(rows, M)
    acc_ref = oracle.contract_pairs(q, codes, m_idx, n_idx)
    y_ref = oracle.epilogue(acc_ref.reshape(-1, 1), b, s[m_idx]).reshape(-1)
    ok = oracle.y_close(host_bf16_f32(y)[m_idx, n_idx], y_ref)
    assert ok.all(), f"{what}: {int((~ok).sum())} of {ok.size} sampled outputs out of tolerance"
    ah = host(acc)[m_idx, n_idx]
    assert np.array_equal(ah, acc_ref), f"{what}: {int((ah != acc_ref).sum())} accumulators differ"


def test_layer70b_decode_b1(bl):
    """Q, K, V grouped on one input, O alone, gate and up grouped, down alone,
    at 1, 16 and 64 tokens; every tensor's packed bytes compared in full."""
    import torch
    name = "layer_70b"
    shapes = wl.WORKLOADS[name]["tensors"]
    ts = {}
    for p in ("q", "k", "v", "o", "gate", "up", "down"):
        say(name, p, shapes[p], "pack b1")
        W = wl.workload_weight(name, p)
        ref_packed, b, a, codes = oracle.pack_binary_b1(W)
        pk, bd, ad = bl.pack_binary_b1(dev(W))
        assert host(bd)[0] == b and host(ad)[0] == a, f"{p}: beta / alpha differ"
        assert np.array_equal(host(pk), ref_packed), f"{p}: packed bytes differ"
        del W, ref_packed
        ts[p] = (pk, bd, b, codes, shapes[p])
    for M in (1, 16, 64):
        qs = {}
        for p in ts:
            inp = wl.INPUT_OF[p]
            if inp not in qs:
                x = wl.workload_activation(name, p, M)
                q, s = oracle.quant_act(x, 1e-5)
                qs[inp] = (dev(q), dev(s), q, s)
        for group in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
            say(name, "b1 M =", M, group)
            dq, ds, q, s = qs[wl.INPUT_OF[group[0]]]
            ents = []
            for p in group:
                pk, bd, b, codes, (N, K) = ts[p]
                ents.append(dict(packed=pk, gamma=bd, N=N, K=K, xq=dq, x_scale=ds,
                                 y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
                                 acc=torch.empty((M, N), dtype=torch.int32, device="cuda")))
            bl.forward_b1_grouped(ents)
            for p, e in zip(group, ents):
                _, _, b, codes, _ = ts[p]
                _sampled(e["y"], e["acc"], codes, b, q, s, (M, wl.PROJ_IDS[p]), f"70B b1 {p} M={M}")
