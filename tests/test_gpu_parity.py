"""GPU parity of every kernel against the CPU oracle, on seeded inputs at sizes
the oracle finishes in seconds, spanning several tiles and ragged tails.

Bar: packed codes, int8 activations, per-token scales and int32 accumulators
bit-exact (a code may differ only inside the 1e-6 rounding window, counted);
bf16 outputs within 1e-3 + 1e-2 |y| of the oracle's fp32 result.
"""

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import (compare_codes, compare_dx, compare_dx_chain, compare_y, dev, dev_bf16, host, host_bf16_bits,
                      host_bf16_f32, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    import torch
    assert torch.cuda.is_available(), "no GPU"
    import bitlinear_absmean_ternarise_amd as m
    return m


# ----------------------------------------------------------------------- pack

PACK_SHAPES = [(1, 1), (16, 64), (17, 65), (33, 300), (7, 1000), (64, 1024), (100, 63), (5, 129),
               (512, 256), (130, 4100), (48, 28672), (1100, 4096)]


@pytest.mark.parametrize("N,K", PACK_SHAPES)
def test_pack_parity(bl, N, K):
    say("pack", N, K)
    W = wl.gaussian_weight(N, K, key=(1000, N, K))
    ref_packed, ref_g, _ = oracle.pack(W, 1e-5)
    packed, g = bl.pack_weights(dev(W), 1e-5)
    g = host(g)[0]
    assert g == ref_g, f"gamma {g!r} vs oracle {ref_g!r}"
    assert compare_codes(host(packed), ref_packed, N, K, W, ref_g, 1e-5) == 0


def test_pack_special_weights(bl):
    say("pack special")
    cases = []
    Z = np.zeros((20, 70), np.float32)
    cases += [(Z, 1e-5), (Z, 0.0)]
    T = np.array([[1.0, -1.0, 0.5, -0.5, 1.5, -1.5, 0.75, 1.25]] * 3, np.float32)  # ties at +-0.5
    cases += [(T, 0.0), (T, 0.02)]
    S = wl.rng(1001).choice([-1.0, 1.0], size=(33, 100)).astype(np.float32) * np.float32(0.037)
    cases += [(S, 0.0)]
    one = np.zeros((16, 64), np.float32)
    one[3, 5] = -0.3
    cases += [(one, 0.0), (one, 1e-5)]
    for W, eps in cases:
        N, K = W.shape
        ref_packed, ref_g, _ = oracle.pack(W, eps)
        packed, g = bl.pack_weights(dev(W), eps)
        assert host(g)[0] == ref_g
        assert np.array_equal(host(packed), ref_packed), (N, K, eps)


def test_pack_many_partials_and_repeatable(bl):
    # more elements than 2048 x 16384 so every partial sum covers a long chunk
    N, K = 4100, 8200
    say("pack large", N, K)
    W = wl.gaussian_weight(N, K, key=(1002,))
    ref_packed, ref_g, _ = oracle.pack(W, 1e-5)
    Wd = dev(W)
    p1, g1 = bl.pack_weights(Wd, 1e-5)
    p2, g2 = bl.pack_weights(Wd, 1e-5)
    assert host(g1)[0] == ref_g and host(g2)[0] == ref_g
    assert np.array_equal(host(p1), host(p2))
    assert compare_codes(host(p1), ref_packed, N, K, W, ref_g, 1e-5) == 0


# ---------------------------------------------------------------------- quant

QUANT_SHAPES = [(1, 1), (1, 8), (3, 7), (5, 100), (32, 256), (8192, 256), (4, 4096), (2, 4104), (3, 4097),
                (1, 28672), (16, 28672), (2, 33000), (64, 8192), (300, 512), (2048, 1536), (7, 2048), (5, 2056),
                (9, 3200), (3, 8200), (2, 16384), (2, 16392), (1, 1024), (200, 6000), (256, 8192), (257, 1024)]


@pytest.mark.parametrize("M,K", QUANT_SHAPES)
@pytest.mark.parametrize("recipe", ["channels", "bernoulli"])
def test_quant_parity(bl, M, K, recipe):
    say("quant", M, K, recipe)
    x = wl.activation(M, K, key=(1100, M, K), recipe=recipe)
    q_ref, s_ref = oracle.quant_act(x, 1e-5)
    q, s = bl.quant_act(dev_bf16(x), 1e-5)
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(q), q_ref)


def test_quant_special_rows(bl):
    say("quant special")
    rows = np.zeros((6, 24), np.float32)
    rows[1, :] = 1e-6                       # below the absmax floor
    rows[2, :6] = [127.0, 2.5, -3.5, 0.5, 1.5, -126.5]  # ties at s = 1
    rows[3, :4] = [1.0, -0.5, 0.25, 2.0]
    rows[4, :] = -3.0e38                     # huge, near fp32 max
    rows[5, 7] = -1.0                        # single nonzero, negative
    x = wl.f32_to_bf16_bits(rows)
    q_ref, s_ref = oracle.quant_act(x, 1e-5)
    q, s = bl.quant_act(dev_bf16(x), 1e-5)
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(q), q_ref)


# --------------------------------------------------------- RMSNorm + quant
# Codes: bit-exact against the oracle's fp64 definition except where its
# value y*s lies within 1e-6 of a rounding midpoint (counted, reported).
# Scales: the kernel's fp32 scale within 1e-6 relative of the fp64 one.

NORM_SHAPES = [(1, 8), (3, 64), (5, 100), (33, 512), (64, 1536), (7, 4096), (3, 4104), (2, 8192), (2, 28672),
               (4, 33000), (300, 256), (9, 2048), (6, 2056), (5, 16384), (2048, 1536), (1, 1024), (200, 6000)]


def _norm_compare(q, s, q_ref, s_ref, v_ref, what):
    qh, sh = host(q), host(s)
    assert np.allclose(sh, s_ref, rtol=1e-6, atol=0), f"{what}: scales differ beyond 1e-6"
    bad = qh != q_ref
    window = oracle.half_window_mask(v_ref)
    assert not (bad & ~window).any(), f"{what}: {int((bad & ~window).sum())} codes differ outside the window"
    if bad.any():
        say(what, "codes differing inside the rounding window:", int(bad.sum()))


@pytest.mark.parametrize("M,K", NORM_SHAPES)
@pytest.mark.parametrize("with_gain", [False, True])
def test_rmsnorm_quant_parity(bl, M, K, with_gain):
    say("rmsnorm quant", M, K, with_gain)
    x = wl.activation(M, K, key=(1150, M, K), recipe="channels")
    g = (np.float32(1.0) + np.float32(0.25) * wl.rng(1151, K).standard_normal(K, dtype=np.float32)) if with_gain else None
    q_ref, s_ref, v_ref = oracle.rmsnorm_quant_act(x, gain=g, eps_norm=1e-6, eps=1e-5)
    q, s = bl.rmsnorm_quant_act(dev_bf16(x), gain=None if g is None else dev(g), eps_norm=1e-6, eps=1e-5)
    _norm_compare(q, s, q_ref, s_ref, v_ref, f"rmsnorm quant M={M} K={K} gain={with_gain}")
    if not with_gain:  # the norm factor never reaches the codes
        qp, _ = bl.quant_act(dev_bf16(x), 1e-5)
        assert np.array_equal(host(q), host(qp))


def test_rmsnorm_quant_special_rows(bl):
    say("rmsnorm quant special")
    K = 64
    rows = np.zeros((5, K), np.float32)
    rows[1, :] = 3.0                      # constant: y = +-1 (eps_norm = 0)
    rows[2, :] = -1e-7                    # tiny: the eps floor binds on max|y|
    rows[3, :4] = [3.0, 4.0, 0.0, 0.0]
    rows[4, ::2] = 1e-30                  # tiny but nonzero
    x = wl.f32_to_bf16_bits(rows)
    for eps_norm in (0.0, 1e-6):
        q_ref, s_ref, v_ref = oracle.rmsnorm_quant_act(x, eps_norm=eps_norm, eps=1e-5)
        q, s = bl.rmsnorm_quant_act(dev_bf16(x), eps_norm=eps_norm, eps=1e-5)
        _norm_compare(q, s, q_ref, s_ref, v_ref, f"special rows eps_norm={eps_norm}")


@pytest.mark.parametrize("M,N,K", [(5, 300, 1536), (130, 100, 448)])
def test_rmsnorm_quant_then_forward(bl, M, N, K):
    """The chain a layer runs: RMSNorm fused into the quant, then the forward."""
    say("rmsnorm -> forward", M, N, K)
    x = wl.activation(M, K, key=(1152, M, K), recipe="bernoulli")
    g = np.float32(0.5) + wl.rng(1153, K).random(K, dtype=np.float32)
    W = wl.gaussian_weight(N, K, key=(1154, N, K))
    packed, gm, codes = oracle.pack(W, 1e-5)
    q_ref, s_ref, v_ref = oracle.rmsnorm_quant_act(x, gain=g)
    q, s = bl.rmsnorm_quant_act(dev_bf16(x), gain=dev(g))
    _norm_compare(q, s, q_ref, s_ref, v_ref, "chain quant")
    y = bl.forward(dev(packed), dev(np.array([gm], np.float32)), N, K, q, s)
    acc_ref = oracle.contract(host(q), codes)  # the GPU's own codes (identical outside the window)
    compare_y(host_bf16_f32(y), oracle.epilogue(acc_ref, gm, s_ref), f"rmsnorm chain M={M}")


# -------------------------------------------------------------------- forward
# The forward kernels are fed the oracle's packed bytes, gamma, q and s, so
# the int32 accumulators must match the oracle's contraction exactly.

FWD_M = [1, 2, 3, 8, 16, 17, 31, 33, 64, 65, 130]
FWD_NK = [(16, 64), (17, 65), (100, 300), (64, 1024), (48, 1000), (512, 256), (40, 4100), (300, 1536),
          (100, 448), (33, 640), (40, 4096), (48, 3200), (24, 8192)]


@pytest.mark.parametrize("N,K", FWD_NK)
@pytest.mark.parametrize("M", FWD_M)
def test_forward_parity(bl, M, N, K):
    say("forward", M, N, K)
    W = wl.gaussian_weight(N, K, key=(1200, N, K))
    x = wl.activation(M, K, key=(1201, M, K), recipe="channels")
    packed, g, codes = oracle.pack(W, 1e-5)
    q, s = oracle.quant_act(x, 1e-5)
    acc_ref = oracle.contract(q, codes)
    y_ref = oracle.epilogue(acc_ref, g, s)
    y, acc = bl.forward(dev(packed), dev(np.array([g], np.float32)), N, K, dev(q), dev(s), acc=True)
    assert np.array_equal(host(acc), acc_ref)
    compare_y(host_bf16_f32(y), y_ref, f"forward M={M} N={N} K={K}")
    # the same call without the accumulator dump writes the same y
    y2 = bl.forward(dev(packed), dev(np.array([g], np.float32)), N, K, dev(q), dev(s))
    assert np.array_equal(host_bf16_f32(y2), host_bf16_f32(y))
    # and so does the path that takes no workspace (for 14..64 tokens the
    # default may cut K into runs; without a workspace it never does)
    y3, acc3 = bl.forward(dev(packed), dev(np.array([g], np.float32)), N, K, dev(q), dev(s), acc=True,
                          workspace=None)
    assert np.array_equal(host(acc3), acc_ref)
    assert np.array_equal(host_bf16_f32(y3), host_bf16_f32(y))


# Decode batches on the GEMM with K cut into runs of >= 4 groups of 256
# columns, one int32 partial per run in the workspace, then the reduce launch
# (64 x 128 tiles for 33..64 tokens; 32 x 256 tiles with two K slices for
# 14..32 tokens, there only for rows of >= 64 groups).  Shapes with several
# runs, a partial last group (K not a multiple of 256, or of 64), a last run
# holding only that partial group (K = 5184: 20 full groups and one fragment,
# runs of 5; K = 20544: 80 and one, runs of 5), ragged N and M, N not a
# multiple of 4 (the reduce kernel's scalar path), and one-tile calls cut into
# many runs.
SPLIT_CASES = [(64, 1000, 4160), (33, 600, 2000), (17, 2100, 16448), (64, 300, 8256), (40, 90, 3008),
               (64, 257, 2048), (31, 1030, 16640), (50, 40, 8192), (64, 1536, 4096), (64, 500, 5184),
               (20, 260, 20544), (14, 2100, 16448), (16, 300, 28672), (15, 1030, 16640)]


@pytest.mark.parametrize("M,N,K", SPLIT_CASES)
def test_forward_split_k(bl, M, N, K):
    import torch
    say("forward split", M, N, K)
    W = wl.gaussian_weight(N, K, key=(1220, N, K))
    x = wl.activation(M, K, key=(1221, M, K), recipe="channels")
    packed, g, codes = oracle.pack(W, 1e-5)
    q, s = oracle.quant_act(x, 1e-5)
    acc_ref = oracle.contract(q, codes)
    y_ref = oracle.epilogue(acc_ref, g, s)
    ent = dict(packed=dev(packed), gamma=dev(np.array([g], np.float32)), N=N, K=K, xq=dev(q), x_scale=dev(s),
               y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
               acc=torch.empty((M, N), dtype=torch.int32, device="cuda"))
    need = bl.forward_workspace_bytes([ent])
    assert need > 0, "this shape is meant to take the split path"
    # the workspace's contents on entry do not matter: fill it with junk
    ws = torch.randint(0, 256, (need + 4096,), dtype=torch.uint8, device="cuda")
    bl.forward_grouped([ent], workspace=ws)
    assert np.array_equal(host(ent["acc"]), acc_ref)
    compare_y(host_bf16_f32(ent["y"]), y_ref, f"split M={M} N={N} K={K}")
    # without the accumulator dump, and on the path that takes no workspace:
    # the same bf16 bits
    y_split = host_bf16_f32(ent["y"])
    ent2 = dict(ent, y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"), acc=None)
    del ent2["acc"]
    bl.forward_grouped([ent2], workspace=ws)
    assert np.array_equal(host_bf16_f32(ent2["y"]), y_split)
    bl.forward_grouped([ent2], workspace=None)
    assert np.array_equal(host_bf16_f32(ent2["y"]), y_split)
    with pytest.raises(RuntimeError):
        bl.forward_grouped([ent2], workspace=ws[: need - 1])


@pytest.mark.parametrize("M,K", [(40, 320), (64, 1536)])
def test_forward_small_gemm_without_runs(bl, M, K):
    """33..64 tokens with >= 256 output tiles of 64 x 128: the GEMM takes the
    call whole (no workspace), with or without one offered."""
    import torch
    say("forward small gemm", M, K)
    x = wl.activation(M, K, key=(1225, M, K), recipe="channels")
    ents = [_entry(N, K, M, (1226, N, K), x=x) for N in (16384, 16300)]
    args = [dict(packed=dev(e["packed"]), gamma=dev(np.array([e["gamma"]], np.float32)), N=e["N"], K=K,
                 xq=dev(e["q"]), x_scale=dev(e["s"]), y=torch.empty((M, e["N"]), dtype=torch.bfloat16, device="cuda"),
                 acc=torch.empty((M, e["N"]), dtype=torch.int32, device="cuda")) for e in ents]
    assert bl.forward_workspace_bytes(args) == 0
    for ws in ("auto", None):
        bl.forward_grouped(args, workspace=ws)
        for a, e in zip(args, ents):
            assert np.array_equal(host(a["acc"]), e["acc"])
            compare_y(host_bf16_f32(a["y"]), e["y"], f"small gemm N={e['N']} K={K}")


def test_forward_split_k_grouped(bl):
    """Q, K, V-like entries on shared tokens plus one of another K, cut into
    runs in one launch (entries too short to cut write y directly)."""
    import torch
    say("forward split grouped")
    M, K = 48, 4096
    x = wl.activation(M, K, key=(1222, M), recipe="bernoulli")
    ents = [_entry(N, K, M, (1223, N), x=x) for N in (512, 128, 100)]
    ents.append(_entry(200, 1024, M, (1224, 200)))  # 4 groups: never cut
    q, s = dev(ents[0]["q"]), dev(ents[0]["s"])
    args = []
    for i, e in enumerate(ents):
        a = dict(packed=dev(e["packed"]), gamma=dev(np.array([e["gamma"]], np.float32)), N=e["N"], K=e["K"],
                 xq=q if e["K"] == K else dev(e["q"]), x_scale=s if e["K"] == K else dev(e["s"]),
                 y=torch.empty((M, e["N"]), dtype=torch.bfloat16, device="cuda"))
        if i != 1:
            a["acc"] = torch.empty((M, e["N"]), dtype=torch.int32, device="cuda")
        args.append(a)
    assert bl.forward_workspace_bytes(args) > 0
    for _ in range(2):  # a second call reuses the workspace left by the first
        bl.forward_grouped(args)
        for a, e in zip(args, ents):
            if "acc" in a:
                assert np.array_equal(host(a["acc"]), e["acc"])
            compare_y(host_bf16_f32(a["y"]), e["y"], f"split grouped N={e['N']} K={e['K']}")


# 9..16 tokens: the decode kernel takes 1, 2, 3, 4 or 8 row blocks per
# workgroup by the launch's total row blocks (<= 256, <= 512, <= 768,
# <= 2048, more), 7..8 tokens take 8 where a launch has >= 1024 two-block
# workgroups, and 1..2 tokens take 3 where it has 257..767; with a partial
# last workgroup, a ragged N and partial last groups.
@pytest.mark.parametrize("M,Ns,K", [(9, (4100,), 1024), (16, (8192,), 512), (12, (10240,), 320),
                                    (16, (12300,), 256), (10, (8192, 1024, 1000), 448), (16, (3000, 3000, 3000), 192),
                                    (9, (16400, 16400), 256), (16, (33000,), 64), (7, (32770,), 2112),
                                    (8, (20000, 13000), 96), (1, (9000,), 1024), (2, (8192, 1024, 1000), 640),
                                    (1, (10000, 10000), 512)])
def test_forward_decode_row_block_counts(bl, M, Ns, K):
    import torch
    say("forward row-block counts", M, Ns, K)
    x = wl.activation(M, K, key=(1215, M, K), recipe="channels")
    q, s = oracle.quant_act(x, 1e-5)
    dq, ds = dev(q), dev(s)
    ents, refs = [], []
    for i, N in enumerate(Ns):
        W = wl.gaussian_weight(N, K, key=(1216, N, K, i))
        packed, g, codes = oracle.pack(W, 1e-5)
        ents.append(dict(packed=dev(packed), gamma=dev(np.array([g], np.float32)), N=N, K=K, xq=dq, x_scale=ds,
                         y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
                         acc=torch.empty((M, N), dtype=torch.int32, device="cuda")))
        refs.append((g, oracle.contract(q, codes)))
    bl.forward_grouped(ents, workspace=None)
    for (g, acc_ref), e in zip(refs, ents):
        assert np.array_equal(host(e["acc"]), acc_ref), f"M={M} N={e['N']} K={K}"
        compare_y(host_bf16_f32(e["y"]), oracle.epilogue(acc_ref, g, s), f"row blocks M={M} N={e['N']} K={K}")


# 33..64 tokens with no K runs: launches of 193..256 tiles of 64 x 256 take
# those tiles with two K slices (the 70B gate+up launch at 64 tokens: 224);
# 192 and 257 tiles stay on the 64 x 128 tiles.  Ragged M, partial last
# groups (K = 576, 320), and the bounds on both sides.
@pytest.mark.parametrize("M,Ns,K", [(64, (25600, 25600), 576), (33, (28672, 28672), 320), (40, (49152,), 256),
                                    (64, (65536,), 256), (64, (65792,), 128), (50, (30000, 20000, 1000), 448)])
def test_forward_decode_batch_wide_tiles(bl, M, Ns, K):
    import torch
    say("forward decode batch wide tiles", M, Ns, K)
    x = wl.activation(M, K, key=(1217, M, K), recipe="channels")
    q, s = oracle.quant_act(x, 1e-5)
    dq, ds = dev(q), dev(s)
    ents, refs = [], []
    for i, N in enumerate(Ns):
        W = wl.gaussian_weight(N, K, key=(1218, N, K, i))
        packed, g, codes = oracle.pack(W, 1e-5)
        ents.append(dict(packed=dev(packed), gamma=dev(np.array([g], np.float32)), N=N, K=K, xq=dq, x_scale=ds,
                         y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
                         acc=torch.empty((M, N), dtype=torch.int32, device="cuda")))
        refs.append((g, oracle.contract(q, codes)))
    assert bl.forward_workspace_bytes(ents) == 0
    bl.forward_grouped(ents)
    for (g, acc_ref), e in zip(refs, ents):
        assert np.array_equal(host(e["acc"]), acc_ref), f"M={M} N={e['N']} K={K}"
        compare_y(host_bf16_f32(e["y"]), oracle.epilogue(acc_ref, g, s), f"wide tiles M={M} N={e['N']} K={K}")
    # without the int32 dump the epilogue stages the tile in LDS: the same y bits
    ents2 = [dict(e, y=torch.empty_like(e["y"]), acc=None) for e in ents]
    bl.forward_grouped(ents2)
    for e, e2 in zip(ents, ents2):
        assert np.array_equal(host_bf16_f32(e2["y"]), host_bf16_f32(e["y"])), f"staged epilogue N={e['N']}"


# Shapes that steer the prefill GEMM to each of its tile configurations:
# 64 x 256 (one round), 64 x 256 with two K slices, 64 x 384, 32 x 384 with
# two K slices, 32 x 256 for few tiles of one group, 32 x 256 with two K
# slices where 384-column tiles would pad N (the chooser's rules in
# gemm_pipe.hip).
@pytest.mark.parametrize("M,N,K", [(2048, 4096, 256), (2048, 1792, 512), (2048, 4608, 256), (2048, 1536, 320),
                                   (130, 1100, 448), (8192, 256, 256), (4000, 200, 192), (8192, 256, 512),
                                   (4001, 512, 600)])
def test_forward_tile_configs(bl, M, N, K):
    say("forward tiles", M, N, K)
    W = wl.gaussian_weight(N, K, key=(1210, N, K))
    x = wl.activation(M, K, key=(1211, M, K), recipe="bernoulli")
    packed, g, codes = oracle.pack(W, 1e-5)
    q, s = oracle.quant_act(x, 1e-5)
    acc_ref = oracle.contract(q, codes)
    y, acc = bl.forward(dev(packed), dev(np.array([g], np.float32)), N, K, dev(q), dev(s), acc=True)
    assert np.array_equal(host(acc), acc_ref)
    compare_y(host_bf16_f32(y), oracle.epilogue(acc_ref, g, s), f"forward M={M} N={N} K={K}")
    y2 = bl.forward(dev(packed), dev(np.array([g], np.float32)), N, K, dev(q), dev(s))
    assert np.array_equal(host_bf16_f32(y2), host_bf16_f32(y))


def test_forward_extreme_accumulators(bl):
    # all codes +1 / -1 against q = +-127: |acc| = 127 K
    say("forward extremes")
    K, N, M = 8200, 32, 5
    codes = np.ones((N, K), np.int8)
    codes[1::2] = -1
    codes[5] = 0
    packed = oracle.encode(codes)
    q = np.full((M, K), 127, np.int8)
    q[1] = -127
    q[2, ::3] = -127
    s = np.full(M, 1.0, np.float32)
    g = np.float32(0.02)
    acc_ref = oracle.contract(q, codes)
    y, acc = bl.forward(dev(packed), dev(np.array([g], np.float32)), N, K, dev(q), dev(s), acc=True)
    assert np.array_equal(host(acc), acc_ref)
    assert acc_ref[0, 0] == 127 * K
    compare_y(host_bf16_f32(y), oracle.epilogue(acc_ref, g, s))


@pytest.mark.parametrize("K", [262080, 262144])
@pytest.mark.parametrize("M", [1, 5, 100])
def test_forward_scaled_unpack_boundary(bl, M, K):
    """The kernels accumulate 64 * code while 64 * 127 * K fits int32 (K up to
    262080) and switch to the plain unpack above; both sides of the switch
    with every product at its extreme (|acc| = 127 K)."""
    say("forward scaled-unpack boundary", M, K)
    N = 20
    codes = np.ones((N, K), np.int8)
    codes[1::2] = -1
    codes[7, ::5] = 0
    packed = oracle.encode(codes)
    q = np.full((M, K), 127, np.int8)
    q[1 % M] = -127
    q[-1, ::3] = -127
    s = np.full(M, 1.0, np.float32)
    g = np.float32(0.03)
    acc_ref = oracle.contract(q, codes)
    y, acc = bl.forward(dev(packed), dev(np.array([g], np.float32)), N, K, dev(q), dev(s), acc=True)
    assert np.array_equal(host(acc), acc_ref)
    assert abs(int(acc_ref[0, 0])) == 127 * K
    compare_y(host_bf16_f32(y), oracle.epilogue(acc_ref, g, s))


# ----------------------------------------------------------------- end to end

@pytest.mark.parametrize("M", [1, 8, 32, 100])
def test_pipeline_linear_256x512(bl, M):
    """Config 1 shapes (K=256 -> N=512), every step on the GPU, vs the oracle."""
    say("pipeline 256->512 linear", M)
    W = wl.workload_weight("linear_256x512", "w")
    x = wl.activation(M, 256, key=(1, 0, 20, 1, M), recipe="channels")
    r = oracle.forward(x, W)
    packed, g = bl.pack_weights(dev(W))
    q, s = bl.quant_act(dev_bf16(x))
    y, acc = bl.forward(packed, g, 512, 256, q, s, acc=True)
    assert host(g)[0] == r["gamma"]
    assert compare_codes(host(packed), r["packed"], 512, 256, W, r["gamma"], 1e-5) == 0
    assert np.array_equal(host(q), r["q"]) and np.array_equal(host(s), r["s"])
    assert np.array_equal(host(acc), r["acc"])
    compare_y(host_bf16_f32(y), r["y"], "256->512 linear")


# ------------------------------------------------------------------- tracker

@pytest.mark.parametrize("n", [1, 7, 8, 9, 1000, 4099, 65536 + 5])
def test_flip_parity_random(bl, n):
    say("flip", n)
    g = wl.rng(1300, n)
    prev = g.choice([-1.0, -0.5, 0.0, -0.0, 0.25, 1.0], size=n).astype(np.float32)
    curr = g.choice([-1.0, 0.0, 0.5, 2.0, -0.0], size=n).astype(np.float32)
    fc = g.integers(32760, 32768, size=n, dtype=np.int16)
    fc[::2] = g.integers(0, 1000, size=fc[::2].size, dtype=np.int16)
    lf = g.integers(0, 1000, size=n, dtype=np.int16)
    fc_ref, lf_ref = oracle.flip_update(prev, curr, 321, fc, lf)
    fcd, lfd = dev(fc), dev(lf)
    bl.flip_update(dev(prev), dev(curr), 321, fcd, lfd)
    assert np.array_equal(host(fcd), fc_ref)
    assert np.array_equal(host(lfd), lf_ref)


@pytest.mark.parametrize("scenario", [1, 2])
def test_flip_model16m(bl, scenario):
    say("flip 16.4M model", scenario)
    prev, curr, mask = wl.flip_snapshots("model_16m")
    fc, lf, step = wl.flip_counters(prev.size, scenario)
    fc_ref, lf_ref = oracle.flip_update(prev, curr, step, fc, lf)
    fcd, lfd = dev(fc), dev(lf)
    bl.flip_update(dev(prev), dev(curr), step, fcd, lfd)
    assert np.array_equal(host(fcd), fc_ref)
    assert np.array_equal(host(lfd), lf_ref)
    assert int((host(fcd).astype(np.int64) - fc).sum()) == int(mask.sum())


# ---------------------------------------------------------------- API errors

def test_device_errors_through_binding(bl):
    import torch
    W = torch.zeros((16, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(bl.BitLinearError):
        bl.pack_weights(W, eps=-1.0)
    x = torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bl.BitLinearError):
        bl.quant_act(x, eps=0.0)
    # misaligned view
    W2 = torch.zeros(16 * 64 + 1, dtype=torch.float32, device="cuda")[1:].view(16, 64)
    with pytest.raises(bl.BitLinearError) as e:
        bl.pack_weights(W2)
    assert e.value.status == -3


# ------------------------------------------------------------ grouped forward

def _entry(N, K, M, key, x=None):
    W = wl.gaussian_weight(N, K, key=key)
    packed, g, codes = oracle.pack(W, 1e-5)
    if x is None:
        x = wl.activation(M, K, key=key + (1,), recipe="plain")
    q, s = oracle.quant_act(x, 1e-5)
    acc = oracle.contract(q, codes)
    return dict(packed=packed, gamma=g, q=q, s=s, acc=acc, y=oracle.epilogue(acc, g, s), N=N, K=K, M=M)


@pytest.mark.parametrize("M", [1, 5, 16])
def test_forward_grouped_qkv_shared_tokens(bl, M):
    """Q, K, V-like entries reading the same tokens, one launch."""
    import torch
    say("grouped qkv", M)
    K = 512
    x = wl.activation(M, K, key=(1400, M), recipe="channels")
    ents = [_entry(N, K, M, (1401, N, M), x=x) for N in (256, 64, 80)]
    q = dev(ents[0]["q"])
    s = dev(ents[0]["s"])
    args = [dict(packed=dev(e["packed"]), gamma=dev(np.array([e["gamma"]], np.float32)), N=e["N"], K=K, xq=q,
                 x_scale=s, y=torch.empty((M, e["N"]), dtype=torch.bfloat16, device="cuda"),
                 acc=torch.empty((M, e["N"]), dtype=torch.int32, device="cuda")) for e in ents]
    bl.forward_grouped(args)
    for a, e in zip(args, ents):
        assert np.array_equal(host(a["acc"]), e["acc"])
        compare_y(host_bf16_f32(a["y"]), e["y"], f"grouped N={e['N']}")


def test_forward_grouped_mixed_shapes_and_fallback(bl):
    """Entries with their own N, K and M.  Up to 64 tokens and K % 16 == 0 the
    entries share one launch (the 16-token kernel while every M <= 16, the
    32x32 kernel once one entry has more); an entry with K % 16 != 0 or more
    than 64 tokens makes the call run the entries one by one."""
    import torch
    say("grouped mixed")
    base = [(48, 1024, 1), (300, 1536, 16), (17, 320, 3), (16, 64, 2), (100, 448, 7)]
    cases = [base, base + [(64, 256, 40)], base + [(33, 640, 64)], base + [(48, 1000, 1)], base + [(20, 256, 80)]]
    for use in cases:
        ents = [_entry(N, K, M, (1402, N, K, M)) for (N, K, M) in use]
        args = [dict(packed=dev(e["packed"]), gamma=dev(np.array([e["gamma"]], np.float32)), N=e["N"], K=e["K"],
                     xq=dev(e["q"]), x_scale=dev(e["s"]),
                     y=torch.empty((e["M"], e["N"]), dtype=torch.bfloat16, device="cuda"),
                     acc=torch.empty((e["M"], e["N"]), dtype=torch.int32, device="cuda")) for e in ents]
        bl.forward_grouped(args)
        for a, e in zip(args, ents):
            assert np.array_equal(host(a["acc"]), e["acc"]), (e["N"], e["K"], e["M"])
            compare_y(host_bf16_f32(a["y"]), e["y"], f"grouped {e['N']}x{e['K']} M={e['M']}")


@pytest.mark.parametrize("M,K", [(65, 256), (130, 448), (300, 1536)])
def test_forward_grouped_prefill(bl, M, K):
    """Prefill-sized entries (M > 64) that read the same tokens share one
    grouped GEMM launch; ragged N, a partial last K group, acc on and off."""
    import torch
    say("grouped prefill", M, K)
    x = wl.activation(M, K, key=(1403, M, K), recipe="bernoulli")
    ents = [_entry(N, K, M, (1404, N, K, M), x=x) for N in (256, 100, 33, 512)]
    q = dev(ents[0]["q"])
    s = dev(ents[0]["s"])
    args = []
    for i, e in enumerate(ents):
        a = dict(packed=dev(e["packed"]), gamma=dev(np.array([e["gamma"]], np.float32)), N=e["N"], K=K, xq=q,
                 x_scale=s, y=torch.empty((M, e["N"]), dtype=torch.bfloat16, device="cuda"))
        if i % 2 == 0:
            a["acc"] = torch.empty((M, e["N"]), dtype=torch.int32, device="cuda")
        args.append(a)
    bl.forward_grouped(args)
    for a, e in zip(args, ents):
        if "acc" in a:
            assert np.array_equal(host(a["acc"]), e["acc"])
        compare_y(host_bf16_f32(a["y"]), e["y"], f"grouped prefill N={e['N']}")


# --------------------------------------------------- binary BitNet weights

@pytest.mark.parametrize("N,K", [(1, 1), (16, 64), (17, 65), (33, 300), (512, 256), (130, 4100), (1100, 4096)])
def test_pack_binary_parity(bl, N, K):
    say("pack binary", N, K)
    W = wl.gaussian_weight(N, K, key=(1700, N, K)) + np.float32(0.004)
    ref_packed, ref_b, ref_a, _ = oracle.pack_binary(W)
    packed, b, a = bl.pack_binary(dev(W))
    assert host(b)[0] == ref_b and host(a)[0] == ref_a
    assert np.array_equal(host(packed), ref_packed)  # the rule W >= alpha has no rounding window


def test_pack_binary_ties(bl):
    say("pack binary ties")
    W = np.tile(np.array([1.0, 2.0, 3.0, 2.0], np.float32), (16, 16))  # alpha = 2 exactly: W = alpha -> +1
    ref_packed, ref_b, ref_a, codes = oracle.pack_binary(W)
    packed, b, a = bl.pack_binary(dev(W))
    assert ref_a == np.float32(2.0) and host(a)[0] == ref_a
    assert np.array_equal(host(packed), ref_packed)


@pytest.mark.parametrize("M", [1, 5, 40, 130])
def test_forward_binary_weights(bl, M):
    """Binary weights run through the same forward (beta in place of gamma)."""
    say("forward binary", M)
    N, K = 300, 1536
    W = wl.gaussian_weight(N, K, key=(1701, N, K))
    x = wl.activation(M, K, key=(1702, M, K), recipe="channels")
    packed, b, a, codes = oracle.pack_binary(W)
    q, s = oracle.quant_act(x, 1e-5)
    acc_ref = oracle.contract(q, codes)
    pk, bd, ad = bl.pack_binary(dev(W))
    y, acc = bl.forward(pk, bd, N, K, dev(q), dev(s), acc=True)
    assert np.array_equal(host(acc), acc_ref)
    compare_y(host_bf16_f32(y), oracle.epilogue(acc_ref, b, s), f"binary M={M}")


# ------------------------------------------------------- tracker read-out

@pytest.mark.parametrize("n", [1, 5, 4096, 65536 + 3])
def test_flip_stats_parity(bl, n):
    say("flip stats", n)
    g = wl.rng(1703, n)
    T = 1000
    fc = g.integers(0, 1001, size=n, dtype=np.int16)
    lf = g.integers(0, 1001, size=n, dtype=np.int16)
    fc[::5] = 0
    lf[::5] = 0
    age_ref, rate_ref = oracle.flip_stats(fc, lf, T)
    age, rate = bl.flip_stats(dev(fc), dev(lf), T)
    assert np.array_equal(host(age), age_ref) and np.array_equal(host(rate), rate_ref)
    assert np.all(host(age)[::5] == 1.0) and np.all(host(rate)[::5] == 0.0)


# ----------------------------------------------- AdamW step + fused tracker

def _adam_state(n, key):
    g = wl.rng(1800, n, key)
    W = (g.standard_normal(n, dtype=np.float32) * np.float32(0.02))
    W[::97] = 0.0                                     # sign 0 counts as its own sign
    W[1::89] = np.float32(1e-30)                      # tiny: any step crosses zero
    grad = (g.standard_normal(n, dtype=np.float32) * np.float32(1e-3))
    grad[::13] = 0.0
    m = (g.standard_normal(n, dtype=np.float32) * np.float32(1e-3))
    v = np.abs(g.standard_normal(n, dtype=np.float32) * np.float32(1e-6)) ** 2
    v[::7] = 0.0
    fc = g.integers(0, 1001, size=n, dtype=np.int16)
    fc[::11] = 32767                                  # saturated counters stay saturated
    lf = g.integers(0, 1001, size=n, dtype=np.int16)
    return W, grad, m, v.astype(np.float32), fc, lf


def _adam_check(bl, W, grad, m, v, fc, lf, t, lr, wd, what):
    ref = oracle.adamw_flip(W, grad, m, v, t, lr, 0.9, 0.999, 1e-8, wd, fc, lf)
    Wd, gd, md, vd = dev(W), dev(grad), dev(m), dev(v)
    fcd = None if fc is None else dev(fc)
    lfd = None if lf is None else dev(lf)
    bl.adamw_step(Wd, gd, md, vd, t, lr, 0.9, 0.999, 1e-8, wd, fcd, lfd)
    got = (host(Wd), host(md), host(vd), None if fc is None else host(fcd), None if lf is None else host(lfd))
    for name, a, b in zip(("W", "exp_avg", "exp_avg_sq", "flip_count", "last_flip"), got, ref):
        if b is None:
            continue
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), \
            f"{what}: {name} differs at {int((a.view(np.uint8) != b.view(np.uint8)).sum())} bytes"
    assert np.array_equal(host(gd), grad), f"{what}: gradient was written"
    return ref


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1000, 4099, 65536 + 5, (1 << 20) + 7])
@pytest.mark.parametrize("track", [False, True])
def test_adamw_parity_random(bl, n, track):
    say("adamw", n, track)
    W, grad, m, v, fc, lf = _adam_state(n, 0)
    ref = _adam_check(bl, W, grad, m, v, fc if track else None, lf if track else None, 7, 1e-2, 0.1,
                      f"adamw n={n} track={track}")
    if track and n >= 1000:
        assert (ref[3] != fc).any(), "no sign crossed: the case tests nothing"


def test_adamw_model16m_training_steps(bl):
    """All 42 tensors of the 16.4M model as one flat buffer: six steps from
    zero optimiser state, the first two untracked (warm-up), the rest with the
    tracker; the fused counters must also equal the two-snapshot tracker."""
    prev, _, _ = wl.flip_snapshots("model_16m")
    n = prev.size
    W = prev.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    fc = np.zeros(n, np.int16)
    lf = np.zeros(n, np.int16)
    Wd, md, vd, fcd, lfd = dev(W), dev(m), dev(v), dev(fc), dev(lf)
    fc_snap, lf_snap = fc.copy(), lf.copy()
    for t in range(1, 7):
        say("adamw 16.4M model step", t)
        g = wl.adam_grad(n, t)
        lr = wl.lr_schedule(t, peak=3e-2)         # steep so that signs cross within a few steps
        track = t > 2
        W0 = W
        W, m, v, fc_r, lf_r = oracle.adamw_flip(W, g, m, v, t, lr, 0.9, 0.999, 1e-8, 0.1,
                                                fc if track else None, lf if track else None)
        bl.adamw_step(Wd, dev(g), md, vd, t, lr, 0.9, 0.999, 1e-8, 0.1, fcd if track else None,
                      lfd if track else None)
        assert np.array_equal(host(Wd).view(np.int32), W.view(np.int32)), f"step {t}: W differs"
        assert np.array_equal(host(md).view(np.int32), m.view(np.int32)), f"step {t}: exp_avg differs"
        assert np.array_equal(host(vd).view(np.int32), v.view(np.int32)), f"step {t}: exp_avg_sq differs"
        if track:
            fc, lf = fc_r, lf_r
            assert np.array_equal(host(fcd), fc) and np.array_equal(host(lfd), lf), f"step {t}: counters differ"
            fc_snap, lf_snap = oracle.flip_update(W0, W, t, fc_snap, lf_snap)
            assert np.array_equal(fc_snap, fc) and np.array_equal(lf_snap, lf)
    assert (fc > 0).any()


# ------------------------------------------------ STE backward to the input

T1_SHAPES = [(1, 1), (16, 64), (17, 65), (300, 20), (5, 129), (64, 1024), (130, 4100), (1100, 4096),
             (4096, 1536), (1536, 4096)]


@pytest.mark.parametrize("N,K", T1_SHAPES)
def test_pack_transposed_parity(bl, N, K):
    say("pack_transposed", N, K)
    W = wl.gaussian_weight(N, K, key=(1900, N, K))
    packed, g = bl.pack_weights(dev(W), 1e-5)
    codes = oracle.decode(host(packed), N, K)
    pt = bl.pack_transposed(packed, N, K)
    assert np.array_equal(host(pt), oracle.encode_t1(codes))


def _bwd_weights(bl, N, K, key):
    W = wl.gaussian_weight(N, K, key=(1901, N, K) + key)
    packed, g = bl.pack_weights(dev(W), 1e-5)
    codes = oracle.decode(host(packed), N, K)
    return bl.pack_transposed(packed, N, K), g, codes, float(host(g)[0])


BWD_NK = [(8, 1), (64, 32), (136, 300), (256, 256), (264, 100), (520, 77), (1024, 130), (1032, 512), (1288, 100),
          (1536, 96)]
BWD_M = [1, 31, 65, 200]


@pytest.mark.parametrize("N,K", BWD_NK)
@pytest.mark.parametrize("M", BWD_M)
def test_backward_input_parity(bl, M, N, K):
    say("backward_input", M, N, K)
    pt, g, codes, gh = _bwd_weights(bl, N, K, (0,))
    dy = wl.activation(M, N, key=(1902, M, N, K))
    prev = wl.activation(M, K, key=(1903, M, N, K))
    ref, mag, _ = oracle.backward_input(dy, codes, gh)
    dx = bl.backward_input(pt, g, N, K, dev_bf16(dy))
    compare_dx(host_bf16_f32(dx), ref, mag, N, f"dx M={M} N={N} K={K}")
    # accumulate into an existing gradient
    ref2, mag2, _ = oracle.backward_input(dy, codes, gh, dx_prev=prev)
    dx2 = dev_bf16(prev)
    bl.backward_input(pt, g, N, K, dev_bf16(dy), dx=dx2, accumulate=True)
    compare_dx(host_bf16_f32(dx2), ref2, mag2 + np.abs(wl.bf16_bits_to_f32(prev)), N, f"dx+= M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(1, 8, 1), (33, 264, 100), (130, 1000, 70), (64, 2056, 256), (97, 520, 300)])
def test_backward_input_integer_dy_bit_exact(bl, M, N, K):
    """Small-integer gradients keep every fp32 partial sum exact, so the
    bf16 result is fixed bit for bit (one fp32 multiply, one fp32 add, one
    rounding to bf16)."""
    say("backward_input exact", M, N, K)
    pt, g, codes, gh = _bwd_weights(bl, N, K, (1,))
    ints = wl.rng(1904, M, N, K).integers(-8, 9, size=(M, N)).astype(np.float32)
    dy = wl.f32_to_bf16_bits(ints)
    prev = wl.activation(M, K, key=(1905, M, N, K))
    _, _, want = oracle.backward_input(dy, codes, gh)
    dx = bl.backward_input(pt, g, N, K, dev_bf16(dy))
    assert np.array_equal(host_bf16_bits(dx), want)
    _, _, want2 = oracle.backward_input(dy, codes, gh, dx_prev=prev)
    dx2 = dev_bf16(prev)
    bl.backward_input(pt, g, N, K, dev_bf16(dy), dx=dx2, accumulate=True)
    assert np.array_equal(host_bf16_bits(dx2), want2)


def test_backward_input_extreme_sums(bl):
    """All codes +1 (or -1) and dy of one sign: the largest sums the
    accumulators see, exact for integer dy."""
    import torch
    M, N, K = 40, 2048, 96
    for sign in (1.0, -1.0):
        W = np.full((N, K), sign * 0.02, np.float32)
        packed, g = bl.pack_weights(dev(W), 1e-5)
        codes = oracle.decode(host(packed), N, K)
        assert np.all(codes == int(sign))
        pt = bl.pack_transposed(packed, N, K)
        dy = wl.f32_to_bf16_bits(np.full((M, N), 127.0, np.float32))
        _, _, want = oracle.backward_input(dy, codes, float(host(g)[0]))
        dx = bl.backward_input(pt, g, N, K, dev_bf16(dy))
        assert np.array_equal(host_bf16_bits(dx), want)
        assert torch.isfinite(dx.float()).all()


def test_backward_input_empty_and_binary(bl):
    import torch
    pt, g, codes, gh = _bwd_weights(bl, 64, 32, (2,))
    dy = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    assert bl.backward_input(pt, g, 64, 32, dy).shape == (0, 32)
    # binary weights: same layouts, codes +-1, scale beta
    N, K, M = 136, 200, 50
    W = wl.gaussian_weight(N, K, key=(1906,))
    pk, beta, _alpha = bl.pack_binary(dev(W))
    codes = oracle.decode(host(pk), N, K)
    assert np.all(np.abs(codes) == 1)
    dy = wl.activation(M, N, key=(1907,))
    ref, mag, _ = oracle.backward_input(dy, codes, float(host(beta)[0]))
    dx = bl.backward_input(bl.pack_transposed(pk, N, K), beta, N, K, dev_bf16(dy))
    compare_dx(host_bf16_f32(dx), ref, mag, N, "binary dx")


# Several layers reading one input (Q, K, V; gate, up): (M, K, [N of each]).
# N not a multiple of 256 leaves a partial last contraction group; K not a
# multiple of 8 takes the element-wise store; M spans partial row tiles.  The
# last two have 129..256 tiles of 64 x 256 and take the two-slice kernel (odd
# group counts leave padding steps in a slice).
BWD_GROUPS = [(1, 64, [64]), (31, 100, [136, 8, 264]), (65, 300, [256, 520, 1032, 64]), (200, 77, [1024, 1288]),
              (130, 1536, [1536, 1536, 1536]), (97, 520, [4096, 4096]), (33, 2056, [72, 2048]),
              (64, 256, [8, 8, 8, 8]), (130, 11999, [264, 520]), (200, 9000, [8, 520, 72, 256])]


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("M,K,Ns", BWD_GROUPS)
def test_backward_input_grouped_parity(bl, M, K, Ns, accumulate):
    say("backward_input_grouped", M, K, Ns, accumulate)
    entries, parts = [], []
    for e, N in enumerate(Ns):
        pt, g, codes, gh = _bwd_weights(bl, N, K, (3, e))
        dy = wl.activation(M, N, key=(1908, M, N, K, e))
        ref, mag, _ = oracle.backward_input(dy, codes, gh)
        entries.append((pt, g, N, dev_bf16(dy)))
        parts.append((ref, mag))
    prev = wl.activation(M, K, key=(1909, M, K)) if accumulate else None
    dx = dev_bf16(prev) if accumulate else None
    dx = bl.backward_input_grouped(entries, K, dx=dx, accumulate=accumulate)
    compare_dx_chain(host_bf16_f32(dx), parts, Ns, None if prev is None else wl.bf16_bits_to_f32(prev),
                     f"grouped dx M={M} K={K} N={Ns}")


@pytest.mark.parametrize("M,K,Ns", [(33, 100, [264, 136, 8]), (130, 520, [1024, 1032]), (64, 96, [8, 2048, 520, 72]),
                                    (130, 12008, [520, 264])])
def test_backward_input_grouped_integer_dy_bit_exact(bl, M, K, Ns):
    """Small-integer gradients keep every fp32 sum exact, so each step of the
    chain (one fp32 multiply, one fp32 add, one rounding to bf16) is fixed bit
    for bit, and the grouped call equals the oracle applied entry by entry."""
    say("backward_input_grouped exact", M, K, Ns)
    entries, host_side = [], []
    for e, N in enumerate(Ns):
        pt, g, codes, gh = _bwd_weights(bl, N, K, (4, e))
        ints = wl.rng(1910, M, N, K, e).integers(-8, 9, size=(M, N)).astype(np.float32)
        dy = wl.f32_to_bf16_bits(ints)
        entries.append((pt, g, N, dev_bf16(dy)))
        host_side.append((dy, codes, gh))
    prev = wl.activation(M, K, key=(1911, M, K))
    for start in (prev, None):  # with an addend, then from zero
        want = start
        for dy, codes, gh in host_side:
            _, _, want = oracle.backward_input(dy, codes, gh, dx_prev=want)
        dx = bl.backward_input_grouped(entries, K, dx=None if start is None else dev_bf16(start),
                                       accumulate=start is not None)
        assert np.array_equal(host_bf16_bits(dx), want), f"addend {start is not None}"


def test_backward_input_grouped_empty(bl):
    import torch
    pt, g, codes, gh = _bwd_weights(bl, 64, 32, (5,))
    dy = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    assert bl.backward_input_grouped([(pt, g, 64, dy), (pt, g, 64, dy)], 32).shape == (0, 32)


# ------------------------------------------------------ grouped packing

@pytest.mark.parametrize("n_tensors", [1, 5, 16, 17, 42])
def test_pack_grouped_matches_single(bl, n_tensors):
    """Every tensor of a grouped call gets the bytes and gamma of a call of
    its own (and of the oracle), across chunk boundaries of 16 tensors."""
    say("pack grouped", n_tensors)
    if n_tensors == 42:
        tl = wl.workload_tensors("model_16m")
        Ws = [wl.workload_weight("model_16m", p, l) for (l, p, N, K) in tl]
    else:
        g = wl.rng(1950, n_tensors)
        shapes = [(int(g.integers(1, 300)), int(g.integers(1, 700))) for _ in range(n_tensors)]
        Ws = [wl.gaussian_weight(N, K, key=(1951, i, N, K)) for i, (N, K) in enumerate(shapes)]
    outs = bl.pack_weights_grouped([dev(W) for W in Ws], 1e-5, transposed=True)
    for i, (W, (pk, gm, pt)) in enumerate(zip(Ws, outs)):
        N, K = W.shape
        ref_packed, ref_g, _ = oracle.pack(W, 1e-5)
        single_pk, single_g = bl.pack_weights(dev(W), 1e-5)
        assert host(gm)[0] == host(single_g)[0] == ref_g, f"tensor {i} {N}x{K}: gamma"
        assert np.array_equal(host(pk), host(single_pk)), f"tensor {i} {N}x{K}: grouped bytes differ from a single call"
        compare_codes(host(pk), ref_packed, N, K, W, ref_g, 1e-5)  # bit-exact, or only inside the 1e-6 window
        assert np.array_equal(host(pt), oracle.encode_t1(oracle.decode(host(pk), N, K))), f"tensor {i}: layout t1"
