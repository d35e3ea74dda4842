"""The no-allocation forward (bitlinear_forward_grouped_noalloc) against the
grouped forward with a caller workspace (bitlinear_forward_grouped_ws), whose
kernels it shares: int32 accumulators and bf16 outputs bit-identical, and the
accumulators equal to the oracle's.  Two calls in a row on the shared scratch,
the second smaller (so it runs over the first call's leftovers), then a call
that needs no scratch at all."""

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


def _entries(M, shapes, key):
    import torch
    ents, refs = [], []
    for i, (N, K) in enumerate(shapes):
        W = wl.gaussian_weight(N, K, key=(key, i, N, K))
        x = wl.activation(M, K, key=(key + 1, i, M, K), recipe="channels")
        packed, g, codes = oracle.pack(W, 1e-5)
        q, s = oracle.quant_act(x, 1e-5)
        ents.append(dict(packed=dev(packed), gamma=dev(np.array([g], np.float32)), N=N, K=K, xq=dev(q),
                         x_scale=dev(s), y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
                         acc=torch.empty((M, N), dtype=torch.int32, device="cuda")))
        refs.append((q, s, codes, g))
    return ents, refs


def _fresh_outputs(ents):
    import torch
    return [dict(e, y=torch.full_like(e["y"], float("nan")), acc=torch.full_like(e["acc"], -7)) for e in ents]


def _check_against_ws(bl, ents, refs_full, what):
    import torch
    need = bl.forward_workspace_bytes(ents)
    a = _fresh_outputs(ents)
    bl.forward_grouped_noalloc(a)
    b = _fresh_outputs(ents)
    ws = torch.randint(0, 256, (max(need, 16),), dtype=torch.uint8, device="cuda")
    bl.forward_grouped(b, workspace=ws)
    torch.cuda.synchronize()
    for i, (ea, eb) in enumerate(zip(a, b)):
        assert np.array_equal(host(ea["acc"]), host(eb["acc"])), f"{what} entry {i}: int32 differs from the _ws call"
        assert np.array_equal(host_bf16_bits(ea["y"]), host_bf16_bits(eb["y"])), f"{what} entry {i}: bf16 differs"
        acc_ref = refs_full[i]
        if acc_ref is not None:
            assert np.array_equal(host(ea["acc"]), acc_ref[0]), f"{what} entry {i}: int32 differs from the oracle"
            compare_y(host_bf16_f32(ea["y"]), acc_ref[1], f"{what} entry {i}")
    return need


def test_noalloc_matches_workspace_call_twice_then_no_cut(bl):
    # 1) the largest plan: 32 tokens, one 8192 x 16384 weight, cut into 8 runs
    #    of 8 groups: 8 x 32 x 8192 int32 partials = the whole 8 MiB
    M, N, K = 32, 8192, 16384
    say("noalloc 1", M, N, K)
    ents, ((q, s, codes, g),) = _entries(M, [(N, K)], 1300)
    need = _check_against_ws(bl, ents, [None], "noalloc 1")
    assert need == 8 * 32 * 8192 * 4
    rows = wl.rng(1302).choice(N, 512, replace=False)
    mi = np.repeat(np.arange(M), rows.size)
    ni = np.tile(rows, M)
    import torch
    a = _fresh_outputs(ents)
    bl.forward_grouped_noalloc(a)
    torch.cuda.synchronize()
    acc_gpu = host(a[0]["acc"])
    assert np.array_equal(acc_gpu[mi, ni], oracle.contract_pairs(q, codes, mi, ni))

    # 2) smaller, two entries, over the first call's leftovers in the scratch
    M2 = 20
    shapes = [(2100, 16448), (1030, 16640)]
    say("noalloc 2", M2, shapes)
    ents2, r2 = _entries(M2, shapes, 1310)
    refs2 = []
    for q2, s2, c2, g2 in r2:
        acc2 = oracle.contract(q2, c2)
        refs2.append((acc2, oracle.epilogue(acc2, g2, s2)))
    need2 = _check_against_ws(bl, ents2, refs2, "noalloc 2")
    assert 0 < need2 < need

    # 3) a call that needs no scratch (one decode token)
    say("noalloc 3")
    ents3, ((q3, s3, c3, g3),) = _entries(1, [(600, 2000)], 1320)
    acc3 = oracle.contract(q3, c3)
    assert _check_against_ws(bl, ents3, [(acc3, oracle.epilogue(acc3, g3, s3))], "noalloc 3") == 0
