"""The torch conveniences (fwd, fused_add_fwd, quant_fwd, mx_quant_fwd,
qk_fwd, layernorm, bwd, fused_add_bwd, layernorm_backward) on the GPU: each
must give bit for bit what the same-name C-ABI calls give on separate
buffers, for a [3, 5, N] input (leading dimensions flatten to rows)."""

import numpy as np
import pytest
import torch

import gen as G
import oracle as O
import row_wise_normalization_fwd_amd as R
from gpu_util import check_output, to_device, to_host

pytestmark = pytest.mark.gpu

BF = O.BF16
N = 1024
SHAPE = (3, 5, N)
M = 15


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    R.load_library()
    torch.cuda.set_device(0)


def _t(a):
    return to_device(a.reshape(-1), BF).view(*a.shape) if a.ndim > 1 else to_device(a, BF)


def _inputs(seed):
    x = G.normal(seed, G.STREAM_X, M, N, BF)
    r = G.normal(seed, G.STREAM_R, M, N, BF)
    dy = G.normal(seed, G.STREAM_DY, M, N, BF)
    g = G.uniform(seed, G.STREAM_GAMMA, N, 0.5, 1.5, BF)
    return x, r, dy, g


def _same(a: torch.Tensor, b: torch.Tensor, what: str):
    torch.cuda.synchronize()
    assert a.shape == b.shape, what
    assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                       b.view(torch.uint8) if b.dtype != torch.uint8 else b), what


def _stream():
    return torch.cuda.current_stream()


def test_forward_conveniences():
    print("conveniences: fwd / fused_add_fwd", flush=True)
    x, r, _, g = _inputs(71)
    xt, gt = _t(x).view(SHAPE), _t(g)
    y, rstd = R.fwd(xt, gt, 1e-5, want_rstd=True)
    assert y.shape == SHAPE and rstd.shape == SHAPE[:-1]
    y2, r2 = torch.empty_like(xt), torch.empty(M, device="cuda")
    assert R.rmsnorm_fwd(xt, gt, y2, r2, M, N, 1e-5, BF, BF, _stream()) == 0
    _same(y, y2, "fwd y")
    _same(rstd.reshape(-1), r2, "fwd rstd")
    ref = O.rmsnorm_fwd(x, g, M, N, 1e-5, BF, BF)
    check_output(to_host(y).reshape(M, N), ref["y_exact"], ref["y"], BF, "fwd y")

    res_a, res_b = _t(r).view(SHAPE), _t(r).view(SHAPE)
    y, _ = R.fused_add_fwd(xt, res_a, gt, 1e-5)
    y2 = torch.empty_like(xt)
    assert R.rmsnorm_fused_add_fwd(xt, res_b, gt, y2, None, M, N, 1e-5, BF, BF, _stream()) == 0
    _same(y, y2, "fused y")
    _same(res_a, res_b, "fused h")


def test_quantised_conveniences():
    print("conveniences: quant_fwd / mx_quant_fwd", flush=True)
    x, _, _, g = _inputs(73)
    xt, gt = _t(x).view(SHAPE), _t(g)
    q, sc, rs = R.quant_fwd(xt, gt, want_rstd=True)
    q2, sc2 = torch.empty(M * N, dtype=torch.uint8, device="cuda"), torch.empty(M, device="cuda")
    assert R.rmsnorm_quant_fwd(xt, None, gt, q2, sc2, R.RMSN_QUANT_FP8_ROW, None, M, N, 1e-5, BF,
                               BF, _stream()) == 0
    _same(q.reshape(-1), q2, "fp8 row codes")
    _same(sc.reshape(-1), sc2, "fp8 row scales")
    one = torch.tensor([0.0625], device="cuda")
    q, sc, _ = R.quant_fwd(xt, gt, scale=one)
    assert R.rmsnorm_quant_fwd(xt, None, gt, q2, one, R.RMSN_QUANT_FP8_TENSOR, None, M, N, 1e-5,
                               BF, BF, _stream()) == 0
    _same(q.reshape(-1), q2, "fp8 tensor codes")
    for fp4, mode in ((False, R.RMSN_QUANT_MXFP8), (True, R.RMSN_QUANT_MXFP4)):
        q, sc, _ = R.mx_quant_fwd(xt, gt, fp4=fp4)
        assert q.shape == SHAPE[:-1] + ((N // 2,) if fp4 else (N,))
        assert sc.shape == SHAPE[:-1] + (N // 32,)
        qb = torch.empty(M * N // (2 if fp4 else 1), dtype=torch.uint8, device="cuda")
        sb = torch.empty(M * N // 32, dtype=torch.uint8, device="cuda")
        assert R.rmsnorm_quant_fwd(xt, None, gt, qb, sb, mode, None, M, N, 1e-5, BF, BF,
                                   _stream()) == 0
        _same(q.reshape(-1), qb, f"mx codes fp4={fp4}")
        _same(sc.reshape(-1), sb, f"mx scales fp4={fp4}")


def test_qk_convenience_on_fused_buffer_views():
    print("conveniences: qk_fwd", flush=True)
    T, Hq, Hk, D = 7, 4, 2, 128
    S = (Hq + 2 * Hk) * D
    buf = G.normal(75, G.STREAM_X, T, S, BF)
    gq = G.uniform(75, G.STREAM_GAMMA, D, 0.5, 1.5, BF)
    gk = G.uniform(76, G.STREAM_GAMMA, D, 0.5, 1.5, BF)
    a, b = _t(buf).view(T, Hq + 2 * Hk, D), _t(buf).view(T, Hq + 2 * Hk, D)
    R.qk_fwd(a[:, :Hq], a[:, Hq:Hq + Hk], _t(gq), _t(gk), 1e-6)
    assert R.rmsnorm_qk_fwd(b, b.data_ptr() + Hq * D * 2, _t(gq), _t(gk), T, Hq, Hk, D, S, S,
                            1e-6, BF, BF, _stream()) == 0
    _same(a, b, "qk buffer")


def test_layernorm_conveniences():
    print("conveniences: layernorm / layernorm_backward", flush=True)
    x, _, dy, g = _inputs(77)
    beta = G.uniform(77, G.STREAM_DRES, N, -1.0, 1.0, BF)
    xt, gt, bt, dyt = _t(x).view(SHAPE), _t(g), _t(beta), _t(dy).view(SHAPE)
    y, mean, rstd = R.layernorm(xt, gt, bt, 1e-5, want_stats=True)
    y2, m2, r2 = torch.empty_like(xt), torch.empty(M, device="cuda"), torch.empty(M, device="cuda")
    assert R.layernorm_fwd(xt, gt, bt, y2, m2, r2, M, N, 1e-5, BF, BF, _stream()) == 0
    _same(y, y2, "layernorm y")
    _same(mean.reshape(-1), m2, "layernorm mean")
    _same(rstd.reshape(-1), r2, "layernorm rstd")
    dx, dg, db = R.layernorm_backward(dyt, xt, mean, rstd, gt)
    dx2, dg2, db2 = torch.empty_like(xt), torch.empty(N, device="cuda"), torch.empty(N, device="cuda")
    wsb = R.layernorm_bwd_workspace_size(M, N)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    assert R.layernorm_bwd(dyt, xt, m2, r2, gt, dx2, dg2, db2, ws, wsb, M, N, BF, BF,
                           _stream()) == 0
    _same(dx, dx2, "layernorm dx")
    _same(dg, dg2, "layernorm dgamma")
    _same(db, db2, "layernorm dbeta")


def test_backward_conveniences():
    print("conveniences: bwd / fused_add_bwd", flush=True)
    x, r, dy, g = _inputs(79)
    xt, gt, dyt = _t(x).view(SHAPE), _t(g), _t(dy).view(SHAPE)
    _, rstd = R.fwd(xt, gt, 1e-5, want_rstd=True)
    # A float32 workspace: its size in bytes, not elements, must reach the library.
    wsb = R.rmsnorm_bwd_workspace_size(M, N)
    ws32 = torch.empty(-(-wsb // 4), dtype=torch.float32, device="cuda")
    dx, dg = R.bwd(dyt, xt, rstd, gt, workspace=ws32)
    dx2, dg2 = torch.empty_like(xt), torch.empty(N, device="cuda")
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    assert R.rmsnorm_bwd(dyt, xt, rstd, gt, dx2, dg2, ws, wsb, M, N, BF, BF, _stream()) == 0
    _same(dx, dx2, "bwd dx")
    _same(dg, dg2, "bwd dgamma")
    dres = _t(G.normal(79, G.STREAM_DRES, M, N, BF)).view(SHAPE)
    dh, dg = R.fused_add_bwd(dyt, xt, rstd, gt, dres)
    assert R.rmsnorm_fused_add_bwd(dyt, xt, rstd, gt, dres, dx2, dg2, ws, wsb, M, N, BF, BF,
                                   _stream()) == 0
    _same(dh, dx2, "fused bwd dh")
    _same(dg, dg2, "fused bwd dgamma")
    assert np.isfinite(to_host(dg)).all()
