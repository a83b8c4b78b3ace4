"""Calls from several host threads at once, each on a stream of its own.

The binding releases the interpreter lock inside every library call, so the
threads really overlap in the library: the per-thread plan cache, the
device-property cache and launches on different streams.  Each thread runs its
own mix of shapes (edge strips, K-split 32 x 32 tiles, large tiles) several
times; every result is compared with the CPU reference, and repeated results
of one shape must agree bit for bit."""
import threading

import numpy as np
import pytest

import fp32_gemm_sgemm_amd as sg
from fp32_gemm_sgemm_amd import inputs

from gpu_cases import check_full, note, to_device

torch = pytest.importorskip("torch")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

SHAPES = [(300, 200, 100), (517, 389, 261), (96, 130, 3000), (1027, 515, 77), (4, 700, 900),
          (640, 3, 500), (512, 512, 512), (33, 65, 2049)]


def test_threads_on_their_own_streams():
    n_threads, reps = 4, 3
    cases = {}
    for t in range(n_threads):
        mine = [SHAPES[(t + i) % len(SHAPES)] for i in range(4)]
        cases[t] = [(M, N, K, inputs.make_operands(M, N, K, seed=900 + 10 * t + i))
                    for i, (M, N, K) in enumerate(mine)]
    results = {t: [] for t in range(n_threads)}
    errors = []
    start = threading.Barrier(n_threads)

    def work(t):
        try:
            stream = torch.cuda.Stream()
            dev = [(to_device(A), to_device(B)) for (_, _, _, (A, B)) in cases[t]]
            torch.cuda.synchronize()
            start.wait()
            outs = []
            with torch.cuda.stream(stream):
                for _ in range(reps):
                    for (dA, dB) in dev:
                        C = torch.empty((dA.shape[0], dB.shape[1]), dtype=torch.float32, device="cuda")
                        sg.sgemm(dA, dB, out=C, stream=stream)
                        outs.append(C)
            stream.synchronize()
            results[t] = [C.cpu().numpy() for C in outs]
        except Exception as e:  # reported below, after every thread ends
            errors.append((t, repr(e)))

    note(f"{n_threads} threads x {reps} repeats x 4 shapes")
    threads = [threading.Thread(target=work, args=(t,)) for t in range(n_threads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors
    for t in range(n_threads):
        outs = results[t]
        k = len(cases[t])
        assert len(outs) == reps * k
        for i, (M, N, K, (A, B)) in enumerate(cases[t]):
            first = outs[i]
            check_full(first, A, B)
            for r in range(1, reps):
                assert np.array_equal(outs[r * k + i], first), (t, M, N, K, r)
