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
