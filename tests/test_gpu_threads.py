"""Calls from several host threads at once, each on a stream of its own.

The header promises that the library's global state (per-device caches, per-(device,
stream) workspaces, kernel attributes) is safe to use from several threads. Here four
threads start together, each on a new stream, so that the first use of every stream
(workspace allocation for split-tile GEMVs and split-k GEMM plans) happens concurrently,
and each repeats a mix of launches. Every result must equal, bit for bit, the same call
made alone on the default stream: the kernels, plans and summation orders depend only on
the shapes."""

import threading

import pytest
import torch

import gemm_rfp4_block_amd as R
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def make_cases():
    cases = []
    # down-projection shape at batch 8: matrix-core tiles with split k (stream workspace)
    w = synth.weights_device(1, 5120, 17408, 8100, DEV)
    x = synth.activations_device(8, 17408, "bf16", 8101, DEV)
    cases.append(("gemv_split", lambda y, w=w, x=x: R.rfp4_gemv(w, 1, 5120, 17408, x, y),
                  lambda: torch.empty((8, 5120), dtype=torch.float32, device=DEV)))
    # up-projection shape at batch 1: the dot-product kernel
    w1 = synth.weights_device(0, 17408, 5120, 8102, DEV)
    x1 = synth.activations_device(1, 5120, "f16", 8103, DEV)
    cases.append(("gemv_dot", lambda y, w=w1, x=x1: R.rfp4_gemv(w, 0, 17408, 5120, x, y),
                  lambda: torch.empty((1, 17408), dtype=torch.float32, device=DEV)))
    # a tall batch-1 launch (matrix-core batch-1 kernel)
    w2 = synth.weights_device(0, 8192, 5120, 8104, DEV)
    cases.append(("gemv_tall", lambda y, w=w2, x=x1: R.rfp4_gemv(w, 0, 8192, 5120, x, y),
                  lambda: torch.empty((1, 8192), dtype=torch.float32, device=DEV)))
    # a GEMM whose plan splits k (stream workspace, reduction kernel)
    w3 = synth.weights_device(0, 1024, 5120, 8105, DEV)
    a3 = synth.activations_device(512, 5120, "bf16", 8106, DEV)
    f3 = R.make_force(gemm_plan="tail2")
    cases.append(("gemm_split", lambda c, w=w3, a=a3: R.rfp4_gemm(w, 0, 1024, 5120, a, c, force=f3),
                  lambda: torch.empty((512, 1024), dtype=torch.bfloat16, device=DEV)))
    return cases


def test_concurrent_threads_on_own_streams_match_single_thread():
    cases = make_cases()
    refs = {}
    for name, call, alloc in cases:
        out = alloc()
        call(out)
        refs[name] = out
    torch.cuda.synchronize()

    n_threads, reps = 4, 5
    results = [dict() for _ in range(n_threads)]
    errors = []
    start = threading.Barrier(n_threads)

    def worker(t):
        try:
            s = torch.cuda.Stream(device=DEV)
            outs = {name: [alloc() for _ in range(reps)] for name, _, alloc in cases}
            start.wait()
            with torch.cuda.stream(s):
                for r in range(reps):
                    for name, call, _ in cases[t % len(cases):] + cases[:t % len(cases)]:
                        call(outs[name][r])
            s.synchronize()
            results[t] = outs
        except Exception as e:  # reported below, in the main thread
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(n_threads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for t in range(n_threads):
        for name, outs in results[t].items():
            for r, out in enumerate(outs):
                assert torch.equal(out, refs[name]), f"thread {t} rep {r} {name} differs"
