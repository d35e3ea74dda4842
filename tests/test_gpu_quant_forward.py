"""GPU parity of the activation quant + forward call (bitlinear_quant_forward_grouped)
against the CPU oracle: int8 codes, per-token scales and int32 accumulators
bit-exact, bf16 outputs within 1e-3 + 1e-2 |y| of the oracle's fp32 result,
and bit-identical to a quant launch followed by the forward.

The one-launch decode path (one token with K <= 32768, or 2..16 tokens with
M*K <= 16384: every workgroup quantises the tokens into LDS) is covered at
one token up to the longest row it takes (K = 32768), at 2..16 tokens up to
M*K = 16384 (rows shorter than 512 columns take the per-chunk atomic max),
with ragged N (not a multiple of 16),
K not a multiple of 64 (partial last fragment) and partial last groups of
1..3 fragments, rows of one group or less, outlier channels, an all-zero
token (the eps floor) and huge tokens; grouped entries that share an input
(written once) or not; and the calls that fall back to separate quant and
forward launches (more tokens, longer rows, a mixed group).
"""

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import compare_y, dev, dev_bf16, host, host_bf16_bits, host_bf16_f32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    import torch
    assert torch.cuda.is_available(), "no GPU"
    import bitlinear_absmean_ternarise_amd as m
    return m


def _case(M, N, K, key, recipe="channels", x=None):
    W = wl.gaussian_weight(N, K, key=(key, N, K))
    if x is None:
        x = wl.activation(M, K, key=(key + 1, M, K), recipe=recipe)
    packed, g, codes = oracle.pack(W, 1e-5)
    q, s = oracle.quant_act(x, 1e-5)
    acc = oracle.contract(q, codes)
    return dict(x=x, packed=packed, g=g, q=q, s=s, acc=acc, y=oracle.epilogue(acc, g, s), N=N, K=K, M=M)


def _entry(c, x_dev=None, with_acc=True, own_q=True):
    import torch
    M, N, K = c["M"], c["N"], c["K"]
    e = dict(packed=dev(c["packed"]), gamma=dev(np.array([c["g"]], np.float32)), N=N, K=K,
             x=x_dev if x_dev is not None else dev_bf16(c["x"]),
             y=torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda"))
    if with_acc:
        e["acc"] = torch.full((M, N), -7, dtype=torch.int32, device="cuda")
    if own_q:
        e["xq"] = torch.full((M, K), 99, dtype=torch.int8, device="cuda")
        e["x_scale"] = torch.full((M,), -1.0, dtype=torch.float32, device="cuda")
    return e


def _check(bl, c, e, yq, what):
    y, xq, xs = yq
    assert np.array_equal(host(xq), c["q"]), f"{what}: activation codes differ"
    assert np.array_equal(host(xs), c["s"]), f"{what}: scales differ"
    if "acc" in e:
        assert np.array_equal(host(e["acc"]), c["acc"]), f"{what}: int32 accumulators differ"
    compare_y(host_bf16_f32(y), c["y"], what)
    # the same bits as a quant launch followed by the forward
    y2, _ = bl.forward(e["packed"], e["gamma"], c["N"], c["K"], *bl.quant_act(e["x"], 1e-5), acc=True)
    assert np.array_equal(host_bf16_bits(y2), host_bf16_bits(y)), f"{what}: bf16 differs from quant + forward"


# (M, N, K): one-launch path (one token with K <= 32768; 2..16 tokens with M*K <= 16384),
# incl. launches of 257..767 two-block workgroups (3 row blocks per workgroup, a partial last one)
FUSED = [(1, 512, 256), (1, 600, 2000), (1, 3200, 3200), (1, 100, 8640), (1, 64, 28672), (1, 17, 32768),
         (1, 40, 48), (1, 33, 16), (2, 300, 4160), (3, 1030, 4672), (5, 1000, 1600), (4, 1030, 3200),
         (8, 130, 2048), (16, 200, 1024), (16, 16, 16), (7, 77, 2336), (2, 20, 8192), (4, 100, 480),
         (9, 64, 496), (16, 48, 1008), (1, 9000, 1024), (2, 10000, 640),
         (1, 20000, 768)]


@pytest.mark.parametrize("M,N,K", FUSED)
def test_quant_forward_one_launch(bl, M, N, K):
    say("quant_forward fused", M, N, K)
    c = _case(M, N, K, 1400)
    e = _entry(c)
    out = bl.quant_forward_grouped([e])
    _check(bl, c, e, out[0], f"fused M={M} N={N} K={K}")


# more than 16 tokens, small weights: the one-launch kernel on 16-token slices
# (a single last token, a partial last slice, 8 slices)
SLICED = [(32, 512, 256), (17, 100, 448), (40, 300, 320), (128, 64, 128), (100, 260, 512), (64, 130, 1024)]


@pytest.mark.parametrize("M,N,K", SLICED)
def test_quant_forward_token_slices(bl, M, N, K):
    import ctypes as C
    say("quant_forward sliced", M, N, K)
    c = _case(M, N, K, 1405)
    e = _entry(c)
    arr = (bl.QuantForwardArgs * 1)(bl.QuantForwardArgs(e["packed"].data_ptr(), e["gamma"].data_ptr(), N, K,
                                                         e["x"].data_ptr(), M, e["xq"].data_ptr(),
                                                         e["x_scale"].data_ptr(), e["y"].data_ptr(), None))
    need = C.c_size_t(7)
    assert bl.lib.bitlinear_quant_forward_workspace_bytes(arr, 1, C.byref(need)) == 0 and need.value == 0
    out = bl.quant_forward_grouped([e])
    _check(bl, c, e, out[0], f"sliced M={M} N={N} K={K}")


# fall back to separate launches: more tokens, longer rows, more than 8
# slices, or codes past the slices' byte bound
FALLBACK = [(32, 300, 2048), (17, 100, 2048), (16, 64, 4096), (1, 50, 32784), (2, 50, 8208), (8, 3200, 3200),
            (129, 64, 128), (40, 4100, 512)]


@pytest.mark.parametrize("M,N,K", FALLBACK)
def test_quant_forward_fallback(bl, M, N, K):
    say("quant_forward fallback", M, N, K)
    c = _case(M, N, K, 1410)
    e = _entry(c)
    out = bl.quant_forward_grouped([e])
    _check(bl, c, e, out[0], f"fallback M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [1, 8])
def test_quant_forward_shared_input(bl, M):
    """Q, K, V read one input: one pair of code / scale buffers, written once;
    a fourth entry reads its own input."""
    say("quant_forward shared", M)
    K = 512
    x = wl.activation(M, K, key=(1421, M, K), recipe="channels")
    cases = [_case(M, N, K, 1420 + i, x=x) for i, N in enumerate((512, 128, 144))]
    other = _case(M, 700, 1024, 1430)
    xd = dev_bf16(x)
    ents = [_entry(c, x_dev=xd, own_q=False) for c in cases] + [_entry(other)]
    out = bl.quant_forward_grouped(ents)
    assert out[0][1].data_ptr() == out[1][1].data_ptr() == out[2][1].data_ptr()
    for c, e, o in zip(cases + [other], ents, out):
        _check(bl, c, e, o, f"shared M={M} N={c['N']}")


@pytest.mark.parametrize("M,N,K", [(40, 1000, 4160), (20, 260, 20544)])
def test_quant_forward_fallback_cut_into_runs(bl, M, N, K):
    """A decode batch that falls back to separate launches and whose forward
    is cut into K runs (14..64 tokens, few output tiles): with the workspace
    the same bits as without."""
    import ctypes as C
    say("quant_forward cut fallback", M, N, K)
    c = _case(M, N, K, 1470)
    e = _entry(c)
    arr = (bl.QuantForwardArgs * 1)(bl.QuantForwardArgs(e["packed"].data_ptr(), e["gamma"].data_ptr(), N, K,
                                                         e["x"].data_ptr(), M, e["xq"].data_ptr(),
                                                         e["x_scale"].data_ptr(), e["y"].data_ptr(), None))
    need = C.c_size_t(0)
    assert bl.lib.bitlinear_quant_forward_workspace_bytes(arr, 1, C.byref(need)) == 0 and need.value > 0
    out = bl.quant_forward_grouped([e], workspace="auto")
    _check(bl, c, e, out[0], f"cut fallback M={M} N={N} K={K}")
    e2 = _entry(c)
    out2 = bl.quant_forward_grouped([e2], workspace=None)
    assert np.array_equal(host_bf16_bits(out2[0][0]), host_bf16_bits(out[0][0]))


def test_quant_forward_mixed_group_falls_back(bl):
    say("quant_forward mixed group")
    c1 = _case(1, 256, 1024, 1440)
    c2 = _case(1, 128, 40000, 1441)  # M*K above the one-launch limit
    ents = [_entry(c1), _entry(c2)]
    out = bl.quant_forward_grouped(ents)
    for c, e, o in zip((c1, c2), ents, out):
        _check(bl, c, e, o, f"mixed N={c['N']} K={c['K']}")


def test_quant_forward_special_tokens(bl):
    say("quant_forward special tokens")
    M, K, N = 6, 64, 48
    rows = np.zeros((M, K), np.float32)
    rows[1, :] = 1e-6                          # below the absmax floor
    rows[2, :6] = [127.0, 2.5, -3.5, 0.5, 1.5, -126.5]  # ties at s = 1
    rows[3, :] = np.linspace(-1.0, 1.0, K)
    rows[4, :] = -3.0e38                       # huge, near fp32 max
    rows[5, 7] = -1.0                          # single nonzero
    x = wl.f32_to_bf16_bits(rows)
    c = _case(M, N, K, 1450, x=x)
    e = _entry(c)
    out = bl.quant_forward_grouped([e])
    _check(bl, c, e, out[0], "special tokens")


def test_quant_forward_empty_entries(bl):
    import torch
    say("quant_forward empty entries")
    c = _case(1, 64, 256, 1460)
    e = _entry(c)
    empty = dict(_entry(_case(1, 64, 256, 1461)), x=torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"),
                 y=torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"),
                 xq=torch.empty((0, 256), dtype=torch.int8, device="cuda"),
                 x_scale=torch.empty((0,), dtype=torch.float32, device="cuda"))
    del empty["acc"]
    out = bl.quant_forward_grouped([empty, e])
    _check(bl, c, e, out[1], "with an empty entry")
