"""Started in a fresh process by tests/test_gpu_concurrency.py: four threads
make the process's first calls into the library at the same moment (every
thread starts with the grouped input gradient, whose kernel needs the LDS
opt-in), then the same jobs run once more, one after another; every thread's
outputs must equal those.  Prints OK on success."""

import os
import sys
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path[:0] = [HERE, os.path.dirname(HERE)]

import torch  # noqa: E402

import bitlinear_absmean_ternarise_amd as bl  # noqa: E402
from concurrency_jobs import make_jobs, run_threads  # noqa: E402


def main() -> int:
    jobs = make_jobs(bl, torch)  # the oracle packs the weights: no library call yet
    results, errors = run_threads(bl, torch, threads=4, rounds=1, jobs=jobs, barrier=threading.Barrier(4),
                                  first="backward")
    if errors or sorted(results) != [0, 1, 2, 3]:
        print("errors:", errors, "threads done:", sorted(results))
        return 1
    ref = {name: [t.cpu() for t in run()] for name, run in jobs.items()}
    torch.cuda.synchronize()
    for tid, res in results.items():
        for name, outs in res.items():
            for a, b in zip(outs, ref[name]):
                if not torch.equal(a, b):
                    print(f"mismatch: thread {tid}, job {name}")
                    return 1
    print("OK")
    return 0


if __name__ == "__main__":
    sys.exit(main())
