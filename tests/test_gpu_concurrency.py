"""Entry points are reentrant: host threads drive different layers on their
own HIP streams and workspaces at the same time, and every output equals the
single-threaded one bit for bit (the kernels sum in a fixed order).  A
thread whose calls fail reads its own error text (thread-local), while the
others keep succeeding."""
import ctypes
import threading

import numpy as np
import pytest
import torch

import synth
from tests.conftest import announce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    import w4a4_rank_corrected_smooth_amd as lib
    lib.device_check()
    return lib


def test_threads_on_their_own_streams(S):
    dev = torch.device("cuda")
    shapes = [(300, 512, 640, 16), (129, 768, 1024, 8), (64, 256, 4096, 32)]   # the last one is K-split
    jobs = []
    for i, (M, N, K, r) in enumerate(shapes):
        c = synth.linear_case(f"thr{i}", 900 + i, M, N, K, r, x_outlier_n=2, x_outlier_scale=30.0)
        layer = S.Linear(S.prepare_weights(c.W, c.calib_absmax(), c.bias, r))
        X = torch.from_numpy(np.ascontiguousarray(c.X).view(np.int16)).view(torch.bfloat16).to(dev)
        jobs.append((layer, X, M, N))
    announce("concurrency: single-threaded references")
    refs = [S.linear_forward(L, X, out_dtype=torch.float32) for L, X, _, _ in jobs]
    torch.cuda.synchronize()
    results, errors = {}, []

    def work(i):
        try:
            L, X, M, N = jobs[i]
            st = torch.cuda.Stream()
            ws = L.new_workspace(M)
            outs = [torch.empty((M, N), dtype=torch.float32, device=dev) for _ in range(12)]
            with torch.cuda.stream(st):
                for o in outs:
                    S.linear_forward(L, X, out=o, workspace=ws)
            st.synchronize()
            results[i] = outs
        except Exception as e:                       # reported below
            errors.append(f"thread {i}: {e!r}")

    def failing():
        try:
            L = jobs[0][0]
            for _ in range(200):
                rc = S._lib.svdq_linear_forward(ctypes.byref(L._w), 1 << 20, 0, 1 << 20, S.BF16, 0,
                                                1 << 20, 1 << 30, None)
                msg = S._lib.svdq_last_error().decode()
                if rc != 2 or "M=0" not in msg:
                    errors.append(f"failing thread saw rc={rc} msg={msg!r}")
                    return
        except Exception as e:
            errors.append(f"failing thread: {e!r}")

    announce("concurrency: 3 working threads + 1 failing thread")
    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(jobs))]
    threads.append(threading.Thread(target=failing))
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for i, ref in enumerate(refs):
        for o in results[i]:
            assert torch.equal(o, ref), f"job {i}: a concurrent output differs from the single-threaded one"
