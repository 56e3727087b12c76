"""Concurrent host threads: each thread calls the library on its own stream
and buffers (forward with rstd, the backward, LayerNorm) many times; every
result must equal a single-threaded run bit for bit, and no thread may see a
HIP error. (The per-device facts the calls cache are already queried by the
single-threaded reference run; their first-use path is atomic stores of
values every thread computes alike.)"""

import threading

import pytest
import torch

import gen as G
import oracle as O
import row_wise_normalization_fwd_amd as R
from gpu_util import to_device

pytestmark = pytest.mark.gpu

BF = O.BF16
M, N = 96, 8192
THREADS, ITERS = 4, 25


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    R.load_library()
    torch.cuda.set_device(0)


def _work(x, dy, g, stream):
    """Forward (y, rstd), backward (dx, dgamma) and LayerNorm (y, mean, rstd)
    on `stream`; returns the outputs after synchronising that stream."""
    with torch.cuda.stream(stream):
        y, rs = torch.empty_like(x), torch.empty(M, device="cuda")
        assert R.rmsnorm_fwd(x, g, y, rs, M, N, 1e-5, BF, BF, stream) == 0
        dx, dg = torch.empty_like(x), torch.empty(N, device="cuda")
        wsb = R.rmsnorm_bwd_workspace_size(M, N)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        assert R.rmsnorm_bwd(dy, x, rs, g, dx, dg, ws, wsb, M, N, BF, BF, stream) == 0
        ly, lm, lr = torch.empty_like(x), torch.empty(M, device="cuda"), torch.empty(M, device="cuda")
        assert R.layernorm_fwd(x, g, None, ly, lm, lr, M, N, 1e-5, BF, BF, stream) == 0
    stream.synchronize()
    return [t.clone() for t in (y, rs, dx, dg, ly, lm, lr)]


def test_concurrent_threads_match_a_single_thread():
    print(f"threads: {THREADS} x {ITERS} calls of fwd/bwd/layernorm, M={M} N={N}", flush=True)
    x = to_device(G.normal(81, G.STREAM_X, M, N, BF).reshape(-1), BF)
    dy = to_device(G.normal(81, G.STREAM_DY, M, N, BF).reshape(-1), BF)
    g = to_device(G.uniform(81, G.STREAM_GAMMA, N, 0.5, 1.5, BF), BF)
    want = _work(x, dy, g, torch.cuda.Stream())
    errors = []

    def run():
        try:
            torch.cuda.set_device(0)
            s = torch.cuda.Stream()
            for _ in range(ITERS):
                got = _work(x, dy, g, s)
                for a, b in zip(got, want):
                    if not torch.equal(a.view(torch.uint8), b.view(torch.uint8)):
                        errors.append("result differs from the single-threaded run")
                        return
            if R.rmsnorm_last_hip_error() != 0:
                errors.append(f"last HIP error {R.rmsnorm_last_hip_error()}")
        except Exception as e:  # reported below, on the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=run) for _ in range(THREADS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors[0]
