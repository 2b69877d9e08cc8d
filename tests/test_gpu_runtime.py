"""GPU tests of the library's runtime contract (include/sgemm.h, conventions):
calls are stream-ordered launches that allocate nothing, so they can be
captured into a HIP graph and replayed; and calls from several host threads
at once, each on its own stream, are independent.

Graph replays are each checked against an eager call on the inputs as they
stand at that replay, with eager work between replays that changes the
inputs (a captured call must read the buffers' current contents).
"""
import threading

import numpy as np
import pytest

import oracle
from register_lds_tiled_amd import binding as b
from register_lds_tiled_amd import workloads as W
from tests.test_gpu_parity import DEV, assert_parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def eager(fn, *args):
    out = fn(*args)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("shape", [(2048, 2048, 256), (1000, 1500, 777), (4096, 4096, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_graph_capture_and_replay(shape):
    M, N, K = shape
    A, B = W.random_inputs(M, N, K, seed=M + 2 * K)
    dA = torch.from_numpy(A).to(DEV)
    dB = torch.from_numpy(B).to(DEV)
    dC = torch.full((M, N), float("nan"), device=DEV)
    bias = torch.linspace(-1.0, 1.0, N, device=DEV)
    dE = torch.full((M, N), float("nan"), device=DEV)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        # warm the side stream once outside capture
        b.sgemm_f32(M, N, K, dA, K, dB, N, dC, N, s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            b.sgemm_f32(M, N, K, dA, K, dB, N, dC, N)
            b.sgemm_f32_ex(M, N, K, dA, K, dB, N, dE, N, 0.5, 0.0, bias, b.ACT_RELU)
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: new inputs
        A2, B2 = W.random_inputs(M, N, K, seed=100 * rep + M)
        dA.copy_(torch.from_numpy(A2))
        dB.copy_(torch.from_numpy(B2))
        dC.fill_(float("nan"))
        dE.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = torch.full((M, N), float("nan"), device=DEV)
        b.sgemm_f32(M, N, K, dA, K, dB, N, want, N)
        torch.cuda.synchronize()
        assert torch.equal(dC, want), f"replay {rep}: captured product differs from eager"
        R = oracle.sgemm_ex_ref_f64(A2, B2, None, 0.5, 0.0, bias.cpu().numpy(), 1)
        assert_parity(dE.cpu().numpy(), R, f"replay {rep} fused epilogue")


def test_graph_capture_16bit():
    M, N, K = 2048, 2048, 512
    A16, B16 = W.lowp_inputs(M, N, K, seed=3, fmt="bf16")
    dA = torch.from_numpy(A16.view(np.int16)).to(DEV)
    dB = torch.from_numpy(B16.view(np.int16)).to(DEV)
    dC = torch.full((M, N), float("nan"), device=DEV)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b.gemm_bf16_f32(M, N, K, dA, K, dB, N, dC, N, s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            b.gemm_bf16_f32(M, N, K, dA, K, dB, N, dC, N)
    for rep in range(3):
        A2, B2 = W.lowp_inputs(M, N, K, seed=50 + rep, fmt="bf16")
        dA.copy_(torch.from_numpy(A2.view(np.int16)))
        dB.copy_(torch.from_numpy(B2.view(np.int16)))
        dC.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_parity(dC.cpu().numpy(), oracle.gemm_lowp_ref_f64(A2, B2, "bf16"), f"replay {rep}")


def test_concurrent_host_threads():
    """Four host threads, each with its own stream and inputs, calling the
    library repeatedly at the same time; every result is checked."""
    shapes = [(1024, 1024, 300), (700, 900, 256), (2048, 512, 128), (512, 2048, 640)]
    inputs = [W.random_inputs(M, N, K, seed=7 + i) for i, (M, N, K) in enumerate(shapes)]
    refs = [oracle.sgemm_ref_f64(A, B) for A, B in inputs]
    errors = []

    def worker(i):
        try:
            M, N, K = shapes[i]
            A, B = inputs[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                dA = torch.from_numpy(A).to(DEV, non_blocking=False)
                dB = torch.from_numpy(B).to(DEV, non_blocking=False)
                for rep in range(20):
                    dC = torch.full((M, N), float("nan"), device=DEV)
                    b.sgemm_f32(M, N, K, dA, K, dB, N, dC, N, s)
                    if rep % 5 == 4:
                        s.synchronize()
                        ok, err, ref, tol = oracle.parity(dC.cpu().numpy(), refs[i])
                        if not ok:
                            errors.append(f"thread {i} rep {rep}: err {err} > {tol}")
                s.synchronize()
        except Exception as e:  # noqa: BLE001 -- reported below
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
