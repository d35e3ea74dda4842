"""HIP-graph replays of the library's calls (the benchmark times its steps
from graphs, as a serving loop or training step launches them).  Each graph
is captured once and replayed several times, with the program's own eager
work (refilling the outputs, resetting the state a call reads) and a
synchronisation between replays; every replay must equal the eager result
bit for bit.  The parity of the eager results with the oracle is covered by
the other GPU tests."""

import numpy as np
import pytest

import workloads as wl
from gpu_util import dev, dev_bf16, say

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def bl():
    import torch
    assert torch.cuda.is_available(), "no GPU"
    import bitlinear_absmean_ternarise_amd as m
    return m


def _capture(torch, fn):
    """Capture fn() on a side stream (warmed up eagerly first, as torch's
    graph capture expects)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(torch, g, outs, want, reset=None, what=""):
    for r in range(REPLAYS):
        for o in outs:
            o.fill_(-1 if o.dtype.is_floating_point else 0x55)  # eager work that the replay must overwrite
        if reset is not None:
            reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o, w), f"{what}: replay {r} differs from the eager result"


def test_graph_quant_forward_and_split_k(bl):
    """Activation quant, the grouped prefill and decode forwards, and a decode
    batch whose K is cut into runs (workspace partial sums + reduce launch)."""
    import torch
    say("graph: quant + forwards")
    cases = [("prefill", 300, [(512, 256), (384, 256)]),  # M > 64: the prefill GEMM
             ("decode", 3, [(1024, 512), (256, 512)]),    # M <= 16: the decode GEMV
             ("split", 40, [(1536, 4096)])]              # 33..64 tokens, few tiles: K cut into runs
    for name, M, shapes in cases:
        K = shapes[0][1]
        x = dev_bf16(wl.activation(M, K, key=(2300, M, K)))
        ents = []
        for i, (N, K_) in enumerate(shapes):
            packed, g = bl.pack_weights(dev(wl.gaussian_weight(N, K_, key=(2301, N, K_, i))))
            ents.append(dict(packed=packed, gamma=g, N=N, K=K_))
        xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
        xs = torch.empty(M, dtype=torch.float32, device="cuda")
        for e in ents:
            e.update(xq=xq, x_scale=xs, y=torch.empty((M, e["N"]), dtype=torch.bfloat16, device="cuda"),
                     acc=torch.empty((M, e["N"]), dtype=torch.int32, device="cuda"))
        need = bl.forward_workspace_bytes(ents)
        if name == "split":
            assert need > 0, "the case must take the cut path"
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

        def step():
            bl.quant_act(x, xq=xq, x_scale=xs)
            bl.forward_grouped(ents, workspace=ws if need else None)

        step()
        torch.cuda.synchronize()
        outs = [xq, xs] + [e["y"] for e in ents] + [e["acc"] for e in ents]
        want = [o.clone() for o in outs]
        g = _capture(torch, step)
        _replay_and_check(torch, g, outs, want, what=f"quant + forward ({name}, M={M})")


@pytest.mark.parametrize("M,K", [(1, 8192), (1, 28672), (4, 3200)])
def test_graph_quant_forward_one_launch(bl, M, K):
    """The activation quant and the decode forward in one call (one launch
    per input: every workgroup quantises the tokens), Q/K/V-like entries that
    share the input, replayed."""
    import torch
    say("graph: quant_forward one launch", M, K)
    x = dev_bf16(wl.activation(M, K, key=(2310, M, K), recipe="channels"))
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    xs = torch.empty(M, dtype=torch.float32, device="cuda")
    ents = []
    for i, N in enumerate((1024, 256, 272)):
        packed, g = bl.pack_weights(dev(wl.gaussian_weight(N, K, key=(2311, N, K, i))))
        ents.append(dict(packed=packed, gamma=g, N=N, K=K, x=x, xq=xq, x_scale=xs,
                         y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
                         acc=torch.empty((M, N), dtype=torch.int32, device="cuda")))

    def step():
        bl.quant_forward_grouped(ents)

    step()
    torch.cuda.synchronize()
    outs = [xq, xs] + [e["y"] for e in ents] + [e["acc"] for e in ents]
    want = [o.clone() for o in outs]
    g = _capture(torch, step)
    _replay_and_check(torch, g, outs, want, what=f"quant_forward one launch (M={M}, K={K})")


@pytest.mark.parametrize("M", [1, 4, 20])
def test_graph_binary_b1_and_dot4_forwards(bl, M):
    """Binary weights in the one-bit layout (pack and grouped forward) and,
    for up to 4 tokens, the grouped forward on the vector ALUs, replayed."""
    import torch
    say("graph: b1 + dot4 forwards", M)
    K = 1536
    xq = dev(np.clip(wl.activation(M, K, key=(2320, M, K)).view(np.int16).astype(np.int8), -127, 127))
    xs = torch.rand(M, device="cuda") + 0.5
    Ws = [dev(wl.gaussian_weight(N, K, key=(2321, N, K, i))) for i, N in enumerate((1024, 256, 272))]
    b1 = [bl.pack_binary_b1(W) for W in Ws]
    v1 = [bl.pack_weights(W) for W in Ws]

    def ents(packs):
        return [dict(packed=p[0], gamma=p[1], N=W.shape[0], K=K, xq=xq, x_scale=xs,
                     y=torch.empty((M, W.shape[0]), dtype=torch.bfloat16, device="cuda"),
                     acc=torch.empty((M, W.shape[0]), dtype=torch.int32, device="cuda")) for p, W in zip(packs, Ws)]
    eb, ed = ents(b1), ents(v1)

    def step():
        for W, p in zip(Ws, b1):
            bl.pack_binary_b1(W, packed=p[0], beta=p[1], alpha=p[2])
        bl.forward_b1_grouped(eb)
        if M <= 4:
            bl.forward_grouped_dot4(ed)

    step()
    torch.cuda.synchronize()
    outs = [p[0] for p in b1] + [p[1] for p in b1] + [e["y"] for e in eb] + [e["acc"] for e in eb]
    if M <= 4:
        outs += [e["y"] for e in ed] + [e["acc"] for e in ed]
    want = [o.clone() for o in outs]
    g = _capture(torch, step)
    _replay_and_check(torch, g, outs, want, what=f"b1 / dot4 forwards (M={M})")


def test_graph_pack_and_transpose(bl):
    """Weight packing (partial sums of |W| in the workspace, then gamma) and
    the layout t1 copy, replayed."""
    import torch
    say("graph: pack")
    N, K = 700, 1000
    W = dev(wl.gaussian_weight(N, K, key=(2302,)))
    packed = torch.empty(bl.packed_bytes(N, K), dtype=torch.uint8, device="cuda")
    gamma = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(bl.pack_workspace_bytes(N, K), dtype=torch.uint8, device="cuda")
    pt = torch.empty(bl.packed_bytes(K, N), dtype=torch.uint8, device="cuda")

    def step():
        bl.pack_weights(W, packed=packed, gamma=gamma, workspace=ws)
        bl.pack_transposed(packed, N, K, packed_t=pt)

    step()
    torch.cuda.synchronize()
    outs = [packed, gamma, pt]
    want = [o.clone() for o in outs]
    g = _capture(torch, step)
    _replay_and_check(torch, g, outs, want, what="pack")


def test_graph_backward_input(bl):
    """The input gradient: a grouped call that writes dx, then a single call
    accumulating into it (the eager fill of dx between replays must not
    show)."""
    import torch
    say("graph: backward")
    M, K = 130, 520
    Ns = [1032, 264, 8]
    ents = []
    for i, N in enumerate(Ns):
        packed, g = bl.pack_weights(dev(wl.gaussian_weight(N, K, key=(2303, N, i))))
        ents.append((bl.pack_transposed(packed, N, K), g, N, dev_bf16(wl.activation(M, N, key=(2304, N, i)))))
    pk_o, g_o = bl.pack_weights(dev(wl.gaussian_weight(512, K, key=(2305,))))
    pt_o = bl.pack_transposed(pk_o, 512, K)
    dy_o = dev_bf16(wl.activation(M, 512, key=(2306,)))
    dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")

    def step():
        bl.backward_input_grouped(ents, K, dx=dx)
        bl.backward_input(pt_o, g_o, 512, K, dy_o, dx=dx, accumulate=True)

    step()
    torch.cuda.synchronize()
    want = [dx.clone()]
    g = _capture(torch, step)
    _replay_and_check(torch, g, [dx], want, what="backward")


def test_graph_adamw_tracker_steps(bl):
    """AdamW with the fused tracker, then the tracker read-out: the state is
    updated in place, so replay r must equal eager step r + 1 (the step
    number is fixed at capture, here and in the eager sequence)."""
    import torch
    say("graph: adamw + tracker")
    n = 100_003
    rng = wl.rng(2307)
    W0 = (0.02 * rng.standard_normal(n)).astype(np.float32)
    grads = [(1e-2 * rng.standard_normal(n)).astype(np.float32) for _ in range(REPLAYS + 1)]

    def fresh():
        return (dev(W0), torch.zeros(n, dtype=torch.float32, device="cuda"),
                torch.zeros(n, dtype=torch.float32, device="cuda"),
                torch.zeros(n, dtype=torch.int16, device="cuda"), torch.zeros(n, dtype=torch.int16, device="cuda"))

    t, lr = 7, 3e-3
    # eager: REPLAYS + 1 steps (the warm-up step of the capture, then one per replay)
    Wd, m, v, fc, lf = fresh()
    eager = []
    for k in range(REPLAYS + 1):
        bl.adamw_step(Wd, dev(grads[k]), m, v, t, lr, weight_decay=0.1, flip_count=fc, last_flip=lf)
        age, rate = bl.flip_stats(fc, lf, t)
        torch.cuda.synchronize()
        eager.append([x.clone() for x in (Wd, m, v, fc, lf, age, rate)])
    # graph: the gradient buffer is refilled eagerly before each replay
    Wg, mg, vg, fcg, lfg = fresh()
    grad = dev(grads[0])
    age_g = torch.empty(n, dtype=torch.float32, device="cuda")
    rate_g = torch.empty(n, dtype=torch.float32, device="cuda")

    def step():
        bl.adamw_step(Wg, grad, mg, vg, t, lr, weight_decay=0.1, flip_count=fcg, last_flip=lfg)
        bl.flip_stats(fcg, lfg, t, sign_age=age_g, flip_rate=rate_g)

    g = _capture(torch, step)  # the warm-up inside ran step 1 eagerly
    torch.cuda.synchronize()
    for x, w in zip((Wg, mg, vg, fcg, lfg, age_g, rate_g), eager[0]):
        assert torch.equal(x, w), "eager warm-up step differs"
    for r in range(REPLAYS):
        grad.copy_(dev(grads[r + 1]))
        age_g.fill_(-1)
        rate_g.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, w in zip((Wg, mg, vg, fcg, lfg, age_g, rate_g), eager[r + 1]):
            assert torch.equal(x, w), f"replay {r}: state differs from eager step {r + 2}"
    assert int((fcg > 0).sum()) > 0
