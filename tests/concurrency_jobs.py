"""Jobs for the concurrency tests: four kinds of library calls, each launched
on the caller's current stream into outputs allocated per call.

Weights are packed by the oracle (the same bytes the library's packer
writes), so setting the jobs up makes no library call: in a fresh process the
jobs' first launches are the process's first calls into the library.
"""

import threading

import numpy as np

import oracle
import workloads as wl


def make_jobs(bl, torch):
    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def dev_bf16(bits):
        return dev(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)

    def weight(N, K, key):
        packed, g, codes = oracle.pack(wl.gaussian_weight(N, K, key=key), 1e-5)
        return dev(packed), dev(np.array([g], np.float32)), codes

    jobs = {}

    # 1. a prefill forward (the MFMA GEMM): 300 tokens, 1000 x 1536
    p1, g1, _ = weight(1000, 1536, (1600,))
    r = wl.rng(1601)
    q1 = dev(r.integers(-127, 128, size=(300, 1536), dtype=np.int8))
    s1 = dev(r.uniform(0.5, 100.0, size=300).astype(np.float32))

    def prefill():
        y, acc = bl.forward(p1, g1, 1000, 1536, q1, s1, acc=True)
        return [y.view(torch.int16), acc]
    jobs["prefill"] = prefill

    # 2. decode quant + forward in one launch: Q, K, V of a 2048-wide layer, one token
    qkv = [weight(N, 2048, (1602, N)) for N in (512, 128, 128)]
    x2 = dev_bf16(wl.activation(1, 2048, key=(1603,), recipe="channels"))

    def decode():
        ents = [dict(packed=p, gamma=g, N=p_n, K=2048, x=x2,
                     y=torch.empty((1, p_n), dtype=torch.bfloat16, device="cuda"))
                for (p, g, _), p_n in zip(qkv, (512, 128, 128))]
        outs = bl.quant_forward_grouped(ents)
        res = []
        for o in outs:
            y, xq, xs = o
            res += [y.view(torch.int16), xq, xs]
        return res
    jobs["decode"] = decode

    # 3. a decode batch with K cut into runs (caller workspace): 40 tokens, 600 x 8192
    p3, g3, _ = weight(600, 8192, (1604,))
    r = wl.rng(1605)
    q3 = dev(r.integers(-127, 128, size=(40, 8192), dtype=np.int8))
    s3 = dev(r.uniform(0.5, 100.0, size=40).astype(np.float32))

    def batch():
        y, acc = bl.forward(p3, g3, 600, 8192, q3, s3, acc=True)
        return [y.view(torch.int16), acc]
    jobs["batch"] = batch

    # 4. the grouped input gradient of Q, K, V (a kernel above 64 KB of LDS):
    #    700M layer shape, 2048 tokens
    ents4 = []
    for i in range(3):
        _, g, codes = weight(1536, 1536, (1606, i))
        dy = dev_bf16(wl.activation(2048, 1536, key=(1607, i)))
        ents4.append((dev(oracle.encode_t1(codes)), g, 1536, dy))

    def backward():
        return [bl.backward_input_grouped(ents4, 1536).view(torch.int16)]
    jobs["backward"] = backward
    torch.cuda.synchronize()
    return jobs


def run_threads(bl, torch, threads=4, rounds=6, jobs=None, barrier=None, first=None):
    """Each thread runs every job `rounds` times on a stream of its own, in an
    order that differs by thread and round (or, with `first`, starting with
    that job in every thread), after `barrier` if given, and keeps its last
    outputs (on the host).  Returns ({thread: {job: [tensors]}}, [errors])."""
    jobs = jobs if jobs is not None else make_jobs(bl, torch)
    names = sorted(jobs)
    results, errors = {}, []

    def work(tid):
        try:
            s = torch.cuda.Stream()
            last = {}
            if barrier is not None:
                barrier.wait()
            with torch.cuda.stream(s):
                for rnd in range(rounds):
                    k = (tid + rnd) % len(names)
                    order = names[k:] + names[:k]
                    if first is not None:
                        order = [first] + [n for n in order if n != first]
                    for name in order:
                        last[name] = jobs[name]()
            s.synchronize()
            results[tid] = {n: [t.cpu() for t in outs] for n, outs in last.items()}
        except Exception as e:  # reported by the caller
            errors.append(f"thread {tid}: {e!r}")

    ts = [threading.Thread(target=work, args=(i,)) for i in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return results, errors
