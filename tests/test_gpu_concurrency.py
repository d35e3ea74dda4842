"""Calls from several host threads, each on a stream of its own.

The library keeps no state between calls except, per device, three values
that the first call sets once through atomics: the architecture check, the
LDS opt-in of the kernels above 64 KB (the grouped input gradient here) and
the no-allocation scratch address.  So concurrent calls on different streams
must give exactly the results of the same calls made one after another:
  * in this process, four threads each run the four jobs below repeatedly,
    in different orders, into buffers of their own;
  * in a fresh process (tests/concurrency_first_calls.py), four threads make
    their very first calls into the library at the same moment.
"""

import os
import subprocess
import sys

import pytest

from concurrency_jobs import make_jobs, run_threads
from gpu_util import say

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def bl():
    import torch
    assert torch.cuda.is_available(), "no GPU"
    import bitlinear_absmean_ternarise_amd as m
    return m


def test_threads_on_own_streams_match_serial_calls(bl):
    import torch
    say("concurrency: 4 threads x 4 jobs x 6 rounds")
    jobs = make_jobs(bl, torch)
    ref = {name: [t.cpu() for t in run()] for name, run in jobs.items()}
    torch.cuda.synchronize()
    results, errors = run_threads(bl, torch, threads=4, rounds=6, jobs=jobs)
    assert not errors, errors
    assert sorted(results) == [0, 1, 2, 3]
    for tid, res in results.items():
        for name, outs in res.items():
            for a, b in zip(outs, ref[name]):
                assert torch.equal(a, b), f"thread {tid}, job {name}"


def test_first_calls_race_in_a_fresh_process():
    say("concurrency: first calls from 4 threads in a fresh process")
    r = subprocess.run([sys.executable, os.path.join(HERE, "concurrency_first_calls.py")], capture_output=True,
                       text=True, timeout=240, cwd=os.path.dirname(HERE))
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout[-2000:] + r.stderr[-2000:]
