"""The allocation-free backward (rmsnorm_bwd_noalloc) against rmsnorm_bwd with
a caller workspace, bit for bit, and both against the oracle, over calls in a
row on the one fixed scratch array: each pair's second call is smaller than
its first, so it runs over what the first left behind."""

import numpy as np
import pytest
import torch

import gen as G
import oracle as O
import row_wise_normalization_fwd_amd as R
from gpu_util import TORCH_DTYPES, check_dgamma, check_dx, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    R.load_library()
    torch.cuda.set_device(0)
    # The first call on a device looks up its copy of the scratch array, when
    # the runtime may load the library's code for the device and reserve the
    # array; every later call must leave device memory as it finds it.
    t = torch.zeros(64, device="cuda")
    assert R.rmsnorm_bwd_noalloc(t, t, torch.ones(1, device="cuda"), t, torch.empty(64, device="cuda"),
                                 torch.empty(64, device="cuda"), 1, 64, O.F32, O.F32,
                                 torch.cuda.current_stream()) == 0
    torch.cuda.synchronize()


def _put(a, dt):
    return to_device(a.reshape(-1), dt)


def _case(M, N, dt, seed):
    print(f"noalloc bwd M={M} N={N} x={dt} seed={seed}", flush=True)
    x = G.normal(seed, G.STREAM_X, M, N, dt)
    dy = G.normal(seed, G.STREAM_DY, M, N, dt)
    g = G.uniform(seed, G.STREAM_GAMMA, N, 0.5, 1.5, dt)
    rho = O.rmsnorm_fwd(x, g, M, N, 1e-5, dt, dt, want_exact=False)["rstd"]
    xt, dyt, gt = _put(x, dt), _put(dy, dt), _put(g, dt)
    rt = torch.from_numpy(rho.copy()).cuda()
    stream = torch.cuda.current_stream()

    # The existing entry point, with its own workspace.
    wsb = R.rmsnorm_bwd_workspace_size(M, N)
    assert 0 < wsb <= R.RMSN_NOALLOC_SCRATCH_BYTES
    ws = torch.full((wsb // 4,), float("nan"), device="cuda")
    dx_ref = torch.empty(M * N, dtype=TORCH_DTYPES[dt], device="cuda")
    dg_ref = torch.full((N,), float("nan"), device="cuda")
    assert R.rmsnorm_bwd(dyt, xt, rt, gt, dx_ref, dg_ref, ws, wsb, M, N, dt, dt, stream) == 0

    # The allocation-free one: device free memory is the same before and after.
    dx = torch.full((M * N,), float("nan"), dtype=TORCH_DTYPES[dt], device="cuda")
    dg = torch.full((N,), float("nan"), device="cuda")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    st = R.rmsnorm_bwd_noalloc(dyt, xt, rt, gt, dx, dg, M, N, dt, dt, stream)
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0

    got_dx, got_dg = to_host(dx), to_host(dg)
    want_dx, want_dg = to_host(dx_ref), to_host(dg_ref)
    bits = (lambda a: a.view(np.uint32)) if dt == O.F32 else (lambda a: a)
    assert np.array_equal(bits(got_dx), bits(want_dx)), "dx differs from rmsnorm_bwd"
    assert np.array_equal(got_dg.view(np.uint32), want_dg.view(np.uint32)), "dgamma differs"
    if M * N <= 1 << 26:  # larger: equal bit for bit to rmsnorm_bwd, checked above
        ref = O.rmsnorm_bwd(dy, x, rho, g, M, N, dt, dt)
        check_dx(got_dx.reshape(M, N), ref, x, dy, g, rho, dt)
        check_dgamma(got_dg, ref)


@pytest.mark.parametrize("calls", [
    [(700, 12288, O.F32), (300, 4096, O.BF16)],     # two-pass tier (row records), then one-pass
    [(8192, 8192, O.BF16), (1000, 2048, O.BF16)],   # the 8192 x 8192 training shape, then smaller
    [(65536, 8192, O.BF16), (64, 1024, O.F16)],     # the whole buffer, then a few rows
], ids=["f32_long_then_bf16", "bf16_8k_then_2k", "full_buffer_then_small"])
def test_noalloc_backward_matches_rmsnorm_bwd(calls):
    for i, (M, N, dt) in enumerate(calls):
        _case(M, N, dt, seed=900 + 10 * i + N % 7)


def test_noalloc_backward_rejects_oversize_shapes():
    stream = torch.cuda.current_stream()
    x = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    st = R.rmsnorm_bwd_noalloc(x, x, x, x, x, x, 65537, 8192, O.BF16, O.BF16, stream)
    assert st == -9 and "fixed buffer" in R.rmsnorm_status_string(st)
