"""GPU parity of the decode contraction on the vector ALUs
(bitlinear_forward_grouped_dot4, v_dot4_i32_i8) against the CPU oracle:
int32 accumulators bit-exact, bf16 within 1e-3 + 1e-2 |y| and bit-identical
to the matrix-core forward on the same inputs.  Shapes: 1..4 tokens, ragged
N, K with a partial last fragment and partial last groups of 1..3
fragments, grouped entries (shared tokens, an empty entry), the largest
accumulators, and the 70B layer at full size on sampled outputs."""

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


def _entry(bl, c, dq, ds, M, with_acc=True):
    import torch
    e = dict(packed=c["pk"], gamma=c["gd"], N=c["N"], K=c["K"], xq=dq, x_scale=ds,
             y=torch.full((M, c["N"]), float("nan"), dtype=torch.bfloat16, device="cuda"))
    if with_acc:
        e["acc"] = torch.full((M, c["N"]), -7, dtype=torch.int32, device="cuda")
    return e


def _weights(bl, N, K, key):
    W = wl.gaussian_weight(N, K, key=(key, N, K))
    packed, g, codes = oracle.pack(W, 1e-5)
    return dict(N=N, K=K, g=g, codes=codes, pk=dev(packed), gd=dev(np.array([g], np.float32)))


SHAPES = [(1, 512, 256), (1, 600, 2000), (2, 100, 1088), (3, 1030, 3200), (4, 64, 4096), (1, 40, 28672),
          (2, 17, 16), (4, 33, 80), (1, 3200, 8640), (3, 300, 4160), (1, 16, 48)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_forward_dot4_parity(bl, M, N, K):
    say("forward dot4", M, N, K)
    c = _weights(bl, N, K, 1900)
    x = wl.activation(M, K, key=(1901, M, K), recipe="channels")
    q, s = oracle.quant_act(x, 1e-5)
    acc_ref = oracle.contract(q, c["codes"])
    dq, ds = dev(q), dev(s)
    e = _entry(bl, c, dq, ds, M)
    bl.forward_grouped_dot4([e])
    assert np.array_equal(host(e["acc"]), acc_ref), f"M={M} N={N} K={K}: accumulators differ"
    compare_y(host_bf16_f32(e["y"]), oracle.epilogue(acc_ref, c["g"], s), f"dot4 M={M} N={N} K={K}")
    y2 = bl.forward(c["pk"], c["gd"], N, K, dq, ds)
    assert np.array_equal(host_bf16_bits(y2), host_bf16_bits(e["y"])), "dot4 and MFMA forwards differ"


def test_forward_dot4_extreme_accumulators(bl):
    say("forward dot4 extremes")
    M, N, K = 4, 48, 262080
    codes = np.ones((N, K), np.int8)
    codes[1::3] = -1
    codes[2::3, ::2] = 0
    packed = oracle.encode(codes)
    q = np.full((M, K), 127, np.int8)
    q[1] = -127
    q[3, 1::2] = -127
    s = np.ones(M, np.float32)
    acc_ref = oracle.contract(q, codes)
    assert np.abs(acc_ref).max() == 127 * K
    c = dict(N=N, K=K, pk=dev(packed), gd=dev(np.array([1.0], np.float32)))
    e = _entry(bl, c, dev(q), dev(s), M)
    bl.forward_grouped_dot4([e])
    assert np.array_equal(host(e["acc"]), acc_ref)


@pytest.mark.parametrize("M", [1, 2, 4])
def test_forward_dot4_grouped_shared_tokens_and_empty_entry(bl, M):
    import torch
    say("forward dot4 grouped", M)
    K = 1536
    x = wl.activation(M, K, key=(1910, M, K), recipe="channels")
    q, s = oracle.quant_act(x, 1e-5)
    dq, ds = dev(q), dev(s)
    cs = [_weights(bl, N, K, 1911 + i) for i, N in enumerate((1536, 256, 256, 100))]
    ents = [_entry(bl, c, dq, ds, M) for c in cs]
    empty = _entry(bl, cs[0], dq[:0], ds[:0], 0, with_acc=False)
    bl.forward_grouped_dot4(ents[:2] + [empty] + ents[2:])
    for c, e in zip(cs, ents):
        acc_ref = oracle.contract(q, c["codes"])
        assert np.array_equal(host(e["acc"]), acc_ref), f"grouped N={c['N']}"
        compare_y(host_bf16_f32(e["y"]), oracle.epilogue(acc_ref, c["g"], s), f"dot4 grouped N={c['N']}")


def test_forward_dot4_rejects_more_tokens(bl):
    import torch
    c = _weights(bl, 64, 256, 1920)
    q = torch.zeros((5, 256), dtype=torch.int8, device="cuda")
    s = torch.ones(5, device="cuda")
    with pytest.raises(bl.BitLinearError):
        bl.forward_grouped_dot4([_entry(bl, c, q, s, 5)])


def test_layer70b_dot4_sampled(bl):
    """The 70B layer at one token, grouped as a decode step groups it (QKV,
    O, gate+up, down), against the oracle on sampled outputs."""
    import torch
    name = "layer_70b"
    shapes = wl.WORKLOADS[name]["tensors"]
    for group in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
        say(name, "dot4", group)
        x = wl.workload_activation(name, group[0], 1)
        q, s = oracle.quant_act(x, 1e-5)
        dq, ds = dev(q), dev(s)
        cs, ents = [], []
        for p in group:
            N, K = shapes[p]
            W = wl.workload_weight(name, p)
            packed, g, codes = oracle.pack(W, 1e-5)
            del W
            c = dict(N=N, K=K, g=g, codes=codes, pk=dev(packed), gd=dev(np.array([g], np.float32)))
            cs.append(c)
            ents.append(_entry(bl, c, dq, ds, 1))
        bl.forward_grouped_dot4(ents)
        for p, c, e in zip(group, cs, ents):
            rows = np.unique(np.r_[np.arange(32), np.arange(c["N"] - 32, c["N"]),
                                   wl.rng(1930, wl.PROJ_IDS[p]).integers(0, c["N"], 512)]).astype(np.int64)
            m_idx = np.zeros(rows.size, np.int64)
            acc_ref = oracle.contract_pairs(q, c["codes"], m_idx, rows)
            assert np.array_equal(host(e["acc"])[0, rows], acc_ref), f"70B dot4 {p}: accumulators differ"
            y_ref = oracle.epilogue(acc_ref.reshape(-1, 1), c["g"], s[m_idx]).reshape(-1)
            ok = oracle.y_close(host_bf16_f32(e["y"])[0, rows], y_ref)
            assert ok.all(), f"70B dot4 {p}: {int((~ok).sum())} outputs out of tolerance"
