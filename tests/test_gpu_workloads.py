"""GPU parity at the full sizes of the five workloads, called the way the
benchmark calls the library (the same entry points, shapes and grouping).

Packed codes, gamma, int8 activations and per-token scales are compared in
full.  Outputs are compared on a sample of (token, row) pairs that the oracle
computes one by one: every token against a fixed set of rows that covers the
first and last row tiles plus random rows, and one whole row block.  Integer
accumulators are bit-exact; bf16 outputs within 1e-3 + 1e-2 |y|.
"""

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import (compare_codes, compare_dx, compare_dx_chain, dev, dev_bf16, host, host_bf16_bits, host_bf16_f32,
                      say)

pytestmark = pytest.mark.gpu

PROJ = ["q", "k", "v", "o", "gate", "up", "down"]


@pytest.fixture(scope="module")
def bl():
    import torch
    assert torch.cuda.is_available(), "no GPU"
    import bitlinear_absmean_ternarise_amd as m
    return m


def _sample_rows(N, key, n_rand=512):
    g = wl.rng(1500, *key)
    fixed = np.r_[np.arange(min(N, 32)), np.arange(max(0, N - 32), N)]
    return np.unique(np.r_[fixed, g.integers(0, N, size=n_rand)]).astype(np.int64)


def _sample_tokens(M, key, n_rand=128):
    if M <= 64:
        return np.arange(M, dtype=np.int64)
    g = wl.rng(1501, *key)
    fixed = np.r_[np.arange(32), np.arange(M - 32, M)]
    return np.unique(np.r_[fixed, g.integers(0, M, size=n_rand)]).astype(np.int64)


def _pairs(M, N, key):
    rows = _sample_rows(N, key)
    toks = _sample_tokens(M, key)
    m_idx = np.repeat(toks, rows.size)
    n_idx = np.tile(rows, toks.size)
    # one whole block: tokens 0..min(M,64)-1 x rows 0..min(N,64)-1 is already
    # covered by the fixed rows; add a block from the middle of the matrix
    mb = np.arange(min(M, 64), dtype=np.int64)
    nb = np.arange(N // 2, min(N, N // 2 + 64), dtype=np.int64)
    m_idx = np.r_[m_idx, np.repeat(mb, nb.size)]
    n_idx = np.r_[n_idx, np.tile(nb, mb.size)]
    return m_idx, n_idx


def _check_sampled(y, acc, codes, g, q, s, key, what):
    """y (bf16 tensor [M][N]) and optional acc (int32 tensor) vs the oracle
    on sampled pairs."""
    M, N = y.shape
    m_idx, n_idx = _pairs(M, N, key)
    acc_ref = oracle.contract_pairs(q, codes, m_idx, n_idx)
    y_ref = oracle.epilogue(acc_ref.reshape(-1, 1), g, s[m_idx]).reshape(-1)
    yh = host_bf16_f32(y)[m_idx, n_idx]
    ok = oracle.y_close(yh, y_ref)
    assert ok.all(), f"{what}: {int((~ok).sum())} of {ok.size} sampled bf16 outputs out of tolerance"
    if acc is not None:
        ah = host(acc)[m_idx, n_idx]
        assert np.array_equal(ah, acc_ref), f"{what}: {int((ah != acc_ref).sum())} accumulators differ"
    assert np.isfinite(host_bf16_f32(y)).all()


class _Tensor:
    """One projection packed on the GPU and by the oracle, codes compared."""

    def __init__(self, bl, W, what):
        N, K = W.shape
        ref_packed, ref_g, codes = oracle.pack(W, 1e-5)
        packed, g = bl.pack_weights(dev(W), 1e-5)
        gh = host(g)[0]
        assert gh == ref_g, f"{what}: gamma {gh!r} vs oracle {ref_g!r}"
        ph = host(packed)
        n_window = compare_codes(ph, ref_packed, N, K, W, ref_g, 1e-5)
        if n_window:  # a code inside the rounding window differs: contract what the GPU packed
            say(what, "codes differing inside the rounding window:", n_window)
            codes = oracle.decode(ph, N, K)
        self.N, self.K, self.packed, self.g, self.codes, self.gamma = N, K, packed, g, codes, ref_g


def _quant(bl, x, what):
    q_ref, s_ref = oracle.quant_act(x, 1e-5)
    q, s = bl.quant_act(dev_bf16(x), 1e-5)
    assert np.array_equal(host(s), s_ref), f"{what}: per-token scales differ"
    assert np.array_equal(host(q), q_ref), f"{what}: int8 activations differ"
    return q, s, q_ref, s_ref


def _forward_both(bl, t, q, s, qh, sh, key, what):
    """y-only call (the benchmark's) and the call that also dumps int32."""
    y = bl.forward(t.packed, t.g, t.N, t.K, q, s)
    _check_sampled(y, None, t.codes, t.gamma, qh, sh, key, what + " (y only)")
    y2, acc = bl.forward(t.packed, t.g, t.N, t.K, q, s, acc=True)
    _check_sampled(y2, acc, t.codes, t.gamma, qh, sh, key, what + " (with acc)")


# ------------------------------------------------ the 16.4M model: 42 tensors

def test_model16m_all_tensors(bl):
    """Six layers, 42 tensors, M = 8192 tokens per forward."""
    tl = wl.workload_tensors("model_16m")
    assert len(tl) == 42
    M = 8192
    xs = {}
    for (layer, p, N, K) in tl:
        what = f"16.4M model layer {layer} {p} {N}x{K}"
        say(what)
        t = _Tensor(bl, wl.workload_weight("model_16m", p, layer), what)
        inp = (layer, wl.INPUT_OF[p])
        if inp not in xs:
            xs[inp] = _quant(bl, wl.workload_activation("model_16m", p, M, layer), what + " quant")
        q, s, qh, sh = xs[inp]
        _forward_both(bl, t, q, s, qh, sh, (wl.stream_id("model_16m"), layer, wl.PROJ_IDS[p]), what)


# ----------------------------------------------------- 700M layer: prefill

@pytest.mark.parametrize("proj", PROJ)
def test_layer700m_prefill(bl, proj):
    M = 2048
    N, K = wl.WORKLOADS["layer_700m"]["tensors"][proj]
    what = f"700M {proj} {N}x{K} M={M}"
    say(what)
    t = _Tensor(bl, wl.workload_weight("layer_700m", proj), what)
    q, s, qh, sh = _quant(bl, wl.workload_activation("layer_700m", proj, M), what + " quant")
    _forward_both(bl, t, q, s, qh, sh, (wl.stream_id("layer_700m"), wl.PROJ_IDS[proj]), what)


def test_layer700m_prefill_grouped(bl):
    """The layer as the benchmark runs it: Q, K, V in one grouped call, O,
    gate and up in one grouped call, down."""
    import torch
    M = 2048
    shapes = wl.WORKLOADS["layer_700m"]["tensors"]
    ts = {p: _Tensor(bl, wl.workload_weight("layer_700m", p), f"700M {p}") for p in PROJ}
    qs = {}
    for p in PROJ:
        inp = wl.INPUT_OF[p]
        if inp not in qs:
            qs[inp] = _quant(bl, wl.workload_activation("layer_700m", p, M), f"700M {inp} quant")
    for group in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
        say("700M grouped", group)
        q, s, qh, sh = qs[wl.INPUT_OF[group[0]]]
        ents = [dict(packed=ts[p].packed, gamma=ts[p].g, N=shapes[p][0], K=shapes[p][1], xq=q, x_scale=s,
                     y=torch.empty((M, shapes[p][0]), dtype=torch.bfloat16, device="cuda")) for p in group]
        bl.forward_grouped(ents)
        for p, e in zip(group, ents):
            t = ts[p]
            _check_sampled(e["y"], None, t.codes, t.gamma, qh, sh, (wl.stream_id("layer_700m"), 7, wl.PROJ_IDS[p]), f"700M grouped {p}")


# --------------------------------------- 3B and 70B layers: decode, grouped

def _decode_layer(bl, name, Ms):
    """For each M run the layer the way a decode step does: Q, K, V grouped
    on one input, O alone, gate and up grouped on one input, down alone."""
    import torch
    ts = _packed_layer(bl, name)
    for M in Ms:
        qs = {}
        for p in PROJ:
            inp = wl.INPUT_OF[p]
            if inp not in qs:
                qs[inp] = _quant(bl, wl.workload_activation(name, p, M), f"{name} {inp} M={M} quant")
        for group in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
            say(f"{name} M={M} group {group}")
            q, s, qh, sh = qs[wl.INPUT_OF[group[0]]]
            for with_acc in (False, True):
                ents = []
                for p in group:
                    t = ts[p]
                    e = dict(packed=t.packed, gamma=t.g, N=t.N, K=t.K, xq=q, x_scale=s,
                             y=torch.empty((M, t.N), dtype=torch.bfloat16, device="cuda"))
                    if with_acc:
                        e["acc"] = torch.empty((M, t.N), dtype=torch.int32, device="cuda")
                    ents.append(e)
                if len(group) > 1:
                    bl.forward_grouped(ents)
                else:
                    e = ents[0]
                    bl.forward(e["packed"], e["gamma"], e["N"], e["K"], q, s, y=e["y"], acc=e.get("acc"))
                for p, e in zip(group, ents):
                    t = ts[p]
                    _check_sampled(e["y"], e.get("acc"), t.codes, t.gamma, qh, sh, (wl.stream_id(name), M, wl.PROJ_IDS[p]),
                                   f"{name} {p} M={M} acc={with_acc}")


_LAYERS = {}


def _packed_layer(bl, name):
    """The seven tensors of a layer, packed once per test module."""
    if name not in _LAYERS:
        _LAYERS.clear()
        shapes = wl.WORKLOADS[name]["tensors"]
        ts = {}
        for p in PROJ:
            what = f"{name} {p} {shapes[p][0]}x{shapes[p][1]}"
            say(what, "pack")
            ts[p] = _Tensor(bl, wl.workload_weight(name, p), what)
        _LAYERS[name] = ts
    return _LAYERS[name]


def test_layer3b_decode(bl):
    _decode_layer(bl, "layer_3b", (1, 8))


@pytest.mark.parametrize("M", [1, 16, 64])
def test_layer70b_decode(bl, M):
    _decode_layer(bl, "layer_70b", (M,))


# ---------------------------------------------- STE backward at full sizes

def _sample_bwd_rows(M, key, n_rand=96):
    g = wl.rng(1510, *key)
    fixed = np.r_[np.arange(min(M, 32)), np.arange(max(0, M - 32), M)]
    return np.unique(np.r_[fixed, g.integers(0, M, size=n_rand)]).astype(np.int64)


def _backward_layer(bl, name, M):
    """The layer's seven input gradients the way a training step takes
    them: Q, K, V accumulate into one buffer, gate and up into another, O
    and down write their own.  Each call is checked on sampled rows against
    the oracle, with the GPU's own previous buffer as the addend."""
    import torch
    shapes = wl.WORKLOADS[name]["tensors"]
    for group in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
        K = shapes[group[0]][1]
        dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
        for i, p in enumerate(group):
            N, K = shapes[p]
            what = f"{name} backward {p} {N}x{K} M={M}"
            say(what)
            packed, g = bl.pack_weights(dev(wl.workload_weight(name, p)), 1e-5)
            codes = oracle.decode(host(packed), N, K)
            pt = bl.pack_transposed(packed, N, K)
            assert np.array_equal(host(pt), oracle.encode_t1(codes)), what + ": layout t1 bytes differ"
            dy = wl.activation(M, N, key=(1511, wl.stream_id(name), wl.PROJ_IDS[p]))
            rows = _sample_bwd_rows(M, (wl.stream_id(name), wl.PROJ_IDS[p]))
            prev = host_bf16_bits(dx)[rows] if i else None
            bl.backward_input(pt, g, N, K, dev_bf16(dy), dx=dx, accumulate=i > 0)
            ref, mag, _ = oracle.backward_input(dy[rows], codes, float(host(g)[0]), dx_prev=prev)
            if prev is not None:
                mag = mag + np.abs(wl.bf16_bits_to_f32(prev))
            compare_dx(host_bf16_f32(dx)[rows], ref, mag, N, what, rms=i == 0)


def _backward_layer_grouped(bl, name, M):
    """The same input gradients with Q, K, V in one grouped call and gate, up
    in another (the sums of one input's layers), checked on sampled rows
    against the oracle's layers summed in sequence."""
    shapes = wl.WORKLOADS[name]["tensors"]
    for group in (("q", "k", "v"), ("gate", "up")):
        K = shapes[group[0]][1]
        entries, parts, Ns = [], [], []
        rows = _sample_bwd_rows(M, (wl.stream_id(name), 20 + len(group)))
        for p in group:
            N, K = shapes[p]
            say(f"{name} grouped backward {p} {N}x{K} M={M}")
            packed, g = bl.pack_weights(dev(wl.workload_weight(name, p)), 1e-5)
            codes = oracle.decode(host(packed), N, K)
            dy = wl.activation(M, N, key=(1511, wl.stream_id(name), wl.PROJ_IDS[p]))
            entries.append((bl.pack_transposed(packed, N, K), g, N, dev_bf16(dy)))
            parts.append(oracle.backward_input(dy[rows], codes, float(host(g)[0]))[:2])
            Ns.append(N)
        what = f"{name} grouped backward {'+'.join(group)} M={M}"
        say(what)
        dx = bl.backward_input_grouped(entries, K)
        compare_dx_chain(host_bf16_f32(dx)[rows], parts, Ns, None, what)


def test_model16m_backward_grouped(bl):
    _backward_layer_grouped(bl, "model_16m", 8192)


def test_layer700m_backward_grouped(bl):
    _backward_layer_grouped(bl, "layer_700m", 2048)


def test_model16m_backward_layer(bl):
    _backward_layer(bl, "model_16m", 8192)


def test_layer700m_backward_layer(bl):
    _backward_layer(bl, "layer_700m", 2048)


def test_model16m_qat_steps(bl):
    """Three training steps of one 16.4M-model projection (gate, 512 x 256,
    8192 tokens) through the library: pack, quantise, forward, input
    gradient, then AdamW with the tracker on the shadow weights, each stage
    checked against the oracle.  The weight gradient (a plain GEMM, passed
    straight through by the estimator) is formed on the host and handed to
    both sides."""
    import torch
    N, K = wl.WORKLOADS["model_16m"]["tensors"]["gate"]
    M = 8192
    W = wl.workload_weight("model_16m", "gate").copy()
    Wd = dev(W)
    m = np.zeros_like(W)
    v = np.zeros_like(W)
    md, vd = dev(m), dev(v)
    fc = np.zeros(W.shape, np.int16)
    lf = np.zeros(W.shape, np.int16)
    fcd, lfd = dev(fc), dev(lf)
    x = wl.workload_activation("model_16m", "gate", M)
    for t in range(1, 4):
        say("qat step", t)
        ref_packed, ref_g, codes = oracle.pack(W, 1e-5)
        packed, g = bl.pack_weights(Wd, 1e-5)
        assert host(g)[0] == ref_g
        if compare_codes(host(packed), ref_packed, N, K, W, ref_g, 1e-5):
            codes = oracle.decode(host(packed), N, K)  # a code inside the rounding window: use the GPU's
        q, s = bl.quant_act(dev_bf16(x), 1e-5)
        q_ref, s_ref = oracle.quant_act(x, 1e-5)
        assert np.array_equal(host(q), q_ref) and np.array_equal(host(s), s_ref)
        y, acc = bl.forward(packed, g, N, K, q, s, acc=True)
        assert np.array_equal(host(acc), oracle.contract(q_ref, codes))
        # a loss whose output gradient is the output itself, rounded to bf16
        dy = host_bf16_bits(y)
        dx = bl.backward_input(bl.pack_transposed(packed, N, K), g, N, K, y)
        rows = _sample_bwd_rows(M, (wl.stream_id("model_16m"), 9, t))
        ref, mag, _ = oracle.backward_input(dy[rows], codes, float(ref_g))
        compare_dx(host_bf16_f32(dx)[rows], ref, mag, N, f"qat step {t} dx")
        xhat = q_ref.astype(np.float64) / s_ref.astype(np.float64)[:, None]
        gW = (wl.bf16_bits_to_f32(dy).astype(np.float64).T @ xhat).astype(np.float32)
        lr = 1e-3
        W, m, v, fc, lf = oracle.adamw_flip(W, gW, m, v, t, lr, 0.9, 0.999, 1e-8, 0.1, fc, lf)
        bl.adamw_step(Wd, dev(gW), md, vd, t, lr, 0.9, 0.999, 1e-8, 0.1, fcd, lfd)
        for name, a, b in (("W", host(Wd), W), ("exp_avg", host(md), m), ("exp_avg_sq", host(vd), v),
                           ("flip_count", host(fcd), fc), ("last_flip", host(lfd), lf)):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"qat step {t}: {name} differs"
    assert (fc > 0).any()
