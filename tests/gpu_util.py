"""Shared helpers of the GPU parity tests: host<->device marshalling and the
comparison rules (bit-exact integers, boundary-window accounting for
quantisation codes, allclose for bf16 outputs)."""

import sys

import numpy as np

import oracle
import workloads as wl


def say(*a):
    print("[gpu-step]", *a, file=sys.stderr, flush=True)


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host(t):
    return t.detach().cpu().numpy()


def host_bf16_f32(t):
    import torch
    return wl.bf16_bits_to_f32(t.detach().view(torch.int16).cpu().numpy().view(np.uint16))


def compare_codes(gpu_packed, ref_packed, N, K, W, g, eps):
    """Packed bytes bit-exact, except codes whose ratio sits within 1e-6 of the
    0.5 rounding boundary (counted).  Returns the number of such mismatches."""
    if np.array_equal(gpu_packed, ref_packed):
        return 0
    gc = oracle.decode(gpu_packed, N, K)
    rc = oracle.decode(ref_packed, N, K)
    bad = gc != rc
    window = oracle.weight_boundary_mask(W, g, eps)
    assert not np.any(bad & ~window), f"{int(np.sum(bad & ~window))} code mismatches outside the rounding window"
    return int(bad.sum())


def compare_y(y_gpu_f32, y_ref, what=""):
    ok = oracle.y_close(y_gpu_f32, y_ref)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        raise AssertionError(f"{what}: {int((~ok).sum())} bf16 outputs outside 1e-3 + 1e-2|y|; first {idx.tolist()} "
                             f"gpu {[float(y_gpu_f32[tuple(i)]) for i in idx]} ref {[float(y_ref[tuple(i)]) for i in idx]}")


def host_bf16_bits(t):
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def compare_dx(dx_gpu_f32, ref, mag, N, what="", rms=True):
    """STE backward: every output within the fp32-summation bound around the
    fp64 reference, and (for Gaussian data) the relative RMS error at the
    bf16 level."""
    ok = oracle.dx_close(dx_gpu_f32, ref, mag, N)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} dx outside the bound; first {idx.tolist()} "
                             f"gpu {[float(dx_gpu_f32[tuple(i)]) for i in idx]} ref {[float(ref[tuple(i)]) for i in idx]}")
    assert np.isfinite(dx_gpu_f32).all(), what
    if rms and ref.size >= 64:
        e = oracle.dx_rel_rms(dx_gpu_f32, ref)
        assert e <= 2.0 ** -9, f"{what}: relative RMS error {e:.3g} above the bf16 level"


def compare_dx_chain(dx_gpu_f32, parts, Ns, prev_f32=None, what=""):
    """Input gradient of several layers summed in sequence: x_e = bf16(part_e
    + x_{e-1}), x_0 = prev (or 0), with parts[e] = (ref, mag) of each layer as
    the oracle gives them.  Each step may round once to bf16 (2^-8 of its
    exact value, as for one call) and make the fp32 summation error of its N
    terms and of the addend; the bounds of the steps add up."""
    rsum = np.zeros_like(parts[0][0]) if prev_f32 is None else np.asarray(prev_f32, np.float64).copy()
    tol = np.zeros_like(rsum)
    for (ref, mag), N in zip(parts, Ns):
        tol += (N + 1) * 2.0 ** -23 * (mag + np.abs(rsum))
        rsum = rsum + ref
        tol += 2.0 ** -8 * np.abs(rsum) + 2.0 ** -126
    x = np.asarray(dx_gpu_f32, np.float64)
    ok = np.abs(x - rsum) <= tol
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} dx outside the chained bound; first "
                             f"{idx.tolist()} gpu {[float(x[tuple(i)]) for i in idx]} "
                             f"ref {[float(rsum[tuple(i)]) for i in idx]}")
    assert np.isfinite(x).all(), what
    if rsum.size >= 64 and np.abs(rsum).max() > 0:
        # one bf16 rounding per step: the relative RMS error grows at most as
        # the square root of the number of steps
        e = oracle.dx_rel_rms(x, rsum)
        assert e <= 2.0 ** -9 * np.sqrt(len(parts)), f"{what}: relative RMS error {e:.3g} above the bf16 level"
    return rsum
