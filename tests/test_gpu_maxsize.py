"""GPU parity at sizes past 32-bit indexing. Every large operand spans more
than 2^32 bytes (and, for 16-bit types, more than 2^31 elements), so a 32-bit
element or byte offset anywhere in a kernel or its launch would wrap.

Inputs are a period of P seeded rows repeated down the tensor on the device.
P = 1021 is prime, so an offset that wraps at a power of two lands on a
different row and changes the result. Outputs are checked against the oracle
on sampled rows: the first and last rows, both sides of the period seam, the
rows around the 2^31-element and 2^32-byte boundaries, and seeded random rows.
Column reductions (dgamma, dbeta) are checked over the whole tensor through
the period: a sum over M rows is (M // P) times the sum over one period plus
the sum over the first M % P rows, both computed by the oracle."""

import numpy as np
import pytest
import torch

import gen as G
import oracle as O
import row_wise_normalization_fwd_amd as R
from gpu_util import (check_column_sum, check_dgamma, check_dx, check_fp8, check_layernorm,
                      check_layernorm_bwd, check_mx, check_output, check_rstd, partition_blocks,
                      to_device, to_host, unpack_fp4)

pytestmark = pytest.mark.gpu

P = 1021
BIG = 1 << 32       # bytes
BIG_ELEMS = 1 << 31


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    R.load_library()
    torch.cuda.set_device(0)
    yield
    torch.cuda.empty_cache()


def _log(msg):
    print(msg, flush=True)


def _stream():
    return torch.cuda.current_stream()


def _rows_for(N, esize, extra):
    """A row count whose tensor passes 2^32 bytes by `extra` rows."""
    return -(-BIG // (N * esize)) + extra


def _tiled(period: np.ndarray, M: int, N: int, dt: int) -> torch.Tensor:
    """[M, N] device tensor whose row i is row i % P of `period` ([P, N])."""
    t = to_device(period.reshape(-1), dt).view(P, N)
    out = torch.empty((M, N), dtype=t.dtype, device="cuda")
    q, rem = divmod(M, P)
    out[:q * P].view(q, P, N).copy_(t.unsqueeze(0).expand(q, P, N))
    out[q * P:].copy_(t[:rem])
    return out


def _tiled_f32(period: np.ndarray, M: int) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(period, dtype=np.float32)).cuda()
    q, rem = divmod(M, P)
    return torch.cat([t.repeat(q), t[:rem]]).contiguous()


def _sample(M, N, esize, seed):
    b = -(-BIG // (N * esize))        # first row starting at or past 2^32 bytes
    e = -(-BIG_ELEMS // N)            # first row starting at or past 2^31 elements
    rng = np.random.default_rng(seed)
    rows = {0, 1, P - 1, P, b - 1, b, b + 1, e - 1, e, M - 2, M - 1}
    rows |= set(int(v) for v in rng.integers(0, M, 8))
    return np.array(sorted(r for r in rows if 0 <= r < M), dtype=np.int64)


def _gather(t: torch.Tensor, rows: np.ndarray, width: int) -> np.ndarray:
    idx = torch.from_numpy(rows).cuda()
    return to_host(t.reshape(-1, width).index_select(0, idx).contiguous())


def _bytes_cols(t: torch.Tensor, rows: np.ndarray, width: int) -> np.ndarray:
    idx = torch.from_numpy(rows).cuda()
    return t.reshape(-1, width).index_select(0, idx).cpu().numpy()


def _period_sum(fn, M):
    """Column sums over M tiled rows from the oracle over one period and the
    remainder: fn(k) returns the oracle's dict for the first k period rows."""
    q, rem = divmod(M, P)
    full = fn(P)
    part = fn(rem) if rem else None
    return lambda key: q * full[key] + (part[key] if part is not None else 0.0)


# ------------------------------------------------------------------ forward

@pytest.mark.parametrize("kind", ["wide", "register", "persistent"])
def test_maxsize_forward(kind):
    """bf16 rows over the forward kernels at over 2^32 bytes: 8192 (this many
    rows take the register kernel, one 256-lane row of four units per
    block), 4096 with an fp32 gamma and the fused residual add (register,
    two units), 16384 (the persistent kernel, 512-lane row groups)."""
    xdt = O.BF16
    N, gdt, fused = {"wide": (8192, O.BF16, False), "register": (4096, O.F32, True),
                     "persistent": (16384, O.BF16, False)}[kind]
    M = _rows_for(N, 2, 7919 if kind != "persistent" else 613)
    _log(f"maxsize fwd {kind} M={M} N={N} fused={fused}")
    x = G.normal(41, G.STREAM_X, P, N, xdt)
    r = G.normal(41, G.STREAM_R, P, N, xdt) if fused else None
    g = G.uniform(41, G.STREAM_GAMMA, N, 0.5, 1.5, gdt)
    xt, gt = _tiled(x, M, N, xdt), to_device(g, gdt)
    rt = _tiled(r, M, N, xdt) if fused else None
    yt = torch.empty_like(xt)
    rs = torch.full((M,), -1.0, device="cuda")
    if fused:
        st = R.rmsnorm_fused_add_fwd(xt, rt, gt, yt, rs, M, N, 1e-5, xdt, gdt, _stream())
    else:
        st = R.rmsnorm_fwd(xt, gt, yt, rs, M, N, 1e-5, xdt, gdt, _stream())
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    rows = _sample(M, N, 2, 5)
    src = rows % P
    S = rows.size
    if fused:
        ref = O.rmsnorm_fused_add_fwd(x[src], r[src], g, S, N, 1e-5, xdt, gdt)
        assert np.array_equal(_gather(rt, rows, N), ref["h"]), "h not bit-exact"
    else:
        ref = O.rmsnorm_fwd(x[src], g, S, N, 1e-5, xdt, gdt)
    check_output(_gather(yt, rows, N), ref["y_exact"], ref["y"], xdt, "y")
    check_rstd(to_host(rs)[rows], ref["rstd_exact"])
    # The whole rstd vector: every row equals its period row's value.
    rs_all = to_host(rs)
    assert np.array_equal(rs_all, np.tile(rs_all[:P], -(-M // P))[:M]), "rstd not periodic"


@pytest.mark.parametrize("mode", ["fp8_row", "mxfp4"])
def test_maxsize_quantised(mode):
    xdt = gdt = O.BF16
    N = 8192
    M = _rows_for(N, 2, 7919)
    _log(f"maxsize quant {mode} M={M} N={N}")
    x = G.normal(43, G.STREAM_X, P, N, xdt)
    g = G.uniform(43, G.STREAM_GAMMA, N, 0.5, 1.5, gdt)
    xt, gt = _tiled(x, M, N, xdt), to_device(g, gdt)
    rows = _sample(M, N, 2, 6)
    src = rows % P
    S = rows.size
    if mode == "fp8_row":
        qt = torch.empty(M * N, dtype=torch.uint8, device="cuda")
        sc = torch.empty(M, device="cuda")
        st = R.rmsnorm_quant_fwd(xt, None, gt, qt, sc, R.RMSN_QUANT_FP8_ROW, None, M, N, 1e-5,
                                 xdt, gdt, _stream())
        assert st == 0, R.rmsnorm_status_string(st)
        torch.cuda.synchronize()
        ref = O.rmsnorm_quant_fwd(x[src], g, S, N, 1e-5, xdt, gdt, O.QUANT_ROW)
        check_fp8(_bytes_cols(qt, rows, N), ref, True, to_host(sc)[rows])
    else:
        qt = torch.empty(M * N // 2, dtype=torch.uint8, device="cuda")
        sc = torch.empty(M * N // 32, dtype=torch.uint8, device="cuda")
        st = R.rmsnorm_quant_fwd(xt, None, gt, qt, sc, R.RMSN_QUANT_MXFP4, None, M, N, 1e-5,
                                 xdt, gdt, _stream())
        assert st == 0, R.rmsnorm_status_string(st)
        torch.cuda.synchronize()
        ref = O.rmsnorm_mx_fwd(x[src], g, S, N, 1e-5, xdt, gdt, O.E2M1)
        check_mx(unpack_fp4(_bytes_cols(qt, rows, N // 2), S, N), _bytes_cols(sc, rows, N // 32),
                 ref, O.E2M1)


def test_maxsize_layernorm_forward():
    xdt = gdt = O.BF16
    N = 8192
    M = _rows_for(N, 2, 7919)
    _log(f"maxsize layernorm fwd M={M} N={N}")
    x = G.normal(47, G.STREAM_X, P, N, xdt)
    g = G.uniform(47, G.STREAM_GAMMA, N, 0.5, 1.5, gdt)
    beta = G.uniform(47, G.STREAM_DY, N, -1.0, 1.0, gdt)
    xt, gt, bt = _tiled(x, M, N, xdt), to_device(g, gdt), to_device(beta, gdt)
    yt = torch.empty_like(xt)
    mt, rt = torch.empty(M, device="cuda"), torch.empty(M, device="cuda")
    st = R.layernorm_fwd(xt, gt, bt, yt, mt, rt, M, N, 1e-5, xdt, gdt, _stream())
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    rows = _sample(M, N, 2, 7)
    src = rows % P
    ref = O.layernorm_fwd(x[src], g, beta, rows.size, N, 1e-5, xdt, gdt)
    check_layernorm(_gather(yt, rows, N), ref, x[src], g, beta, xdt, to_host(mt)[rows],
                    to_host(rt)[rows])


# ------------------------------------------------------------------ backward

@pytest.mark.parametrize("res", [False, True], ids=["plain", "fused_add"])
def test_maxsize_backward(res):
    xdt = gdt = O.BF16
    N = 8192
    M = _rows_for(N, 2, 7919)
    _log(f"maxsize bwd M={M} N={N} fused_add={res}")
    x = G.normal(53, G.STREAM_X, P, N, xdt)
    dy = G.normal(53, G.STREAM_DY, P, N, xdt)
    dres = G.normal(53, G.STREAM_DRES, P, N, xdt) if res else None
    g = G.uniform(53, G.STREAM_GAMMA, N, 0.5, 1.5, gdt)
    rho = O.rmsnorm_fwd(x, g, P, N, 1e-5, xdt, gdt, want_exact=False)["rstd"]
    xt, dyt, gt = _tiled(x, M, N, xdt), _tiled(dy, M, N, xdt), to_device(g, gdt)
    rt = _tiled_f32(rho, M)
    dxt = torch.empty_like(xt)
    dgt = torch.full((N,), float("nan"), device="cuda")
    wsb = R.rmsnorm_bwd_workspace_size(M, N)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    if res:
        drt = _tiled(dres, M, N, xdt)
        st = R.rmsnorm_fused_add_bwd(dyt, xt, rt, gt, drt, dxt, dgt, ws, wsb, M, N, xdt, gdt,
                                     _stream())
    else:
        st = R.rmsnorm_bwd(dyt, xt, rt, gt, dxt, dgt, ws, wsb, M, N, xdt, gdt, _stream())
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    rows = _sample(M, N, 2, 8)
    src = rows % P
    S = rows.size
    if res:
        ref = O.rmsnorm_fused_add_bwd(dy[src], x[src], rho[src], g, dres[src], S, N, xdt, gdt)
    else:
        ref = O.rmsnorm_bwd(dy[src], x[src], rho[src], g, S, N, xdt, gdt)
    check_dx(_gather(dxt, rows, N), ref, x[src], dy[src], g, rho[src], xdt,
             dres=dres[src] if res else None)
    col = _period_sum(lambda k: O.rmsnorm_bwd(dy[:k], x[:k], rho[:k], g, k, N, xdt, gdt,
                                              want_exact=False), M)
    # At most 64 rows per stage-1 partial: the unwidened bound holds.
    assert -(-M // partition_blocks(M, N)) <= 64
    check_dgamma(to_host(dgt), {"dgamma": col("dgamma"), "s": col("s")})


def test_maxsize_layernorm_backward():
    xdt = gdt = O.BF16
    N = 8192
    M = _rows_for(N, 2, 7919)
    _log(f"maxsize layernorm bwd M={M} N={N}")
    x = G.normal(59, G.STREAM_X, P, N, xdt)
    dy = G.normal(59, G.STREAM_DY, P, N, xdt)
    g = G.uniform(59, G.STREAM_GAMMA, N, 0.5, 1.5, gdt)
    f = O.layernorm_fwd(x, g, None, P, N, 1e-5, xdt, gdt, want_exact=False)
    mean, rstd = f["mean"], f["rstd"]
    xt, dyt, gt = _tiled(x, M, N, xdt), _tiled(dy, M, N, xdt), to_device(g, gdt)
    mt, rt = _tiled_f32(mean, M), _tiled_f32(rstd, M)
    dxt = torch.empty_like(xt)
    dgt = torch.full((N,), float("nan"), device="cuda")
    dbt = torch.full((N,), float("nan"), device="cuda")
    wsb = R.layernorm_bwd_workspace_size(M, N)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    st = R.layernorm_bwd(dyt, xt, mt, rt, gt, dxt, dgt, dbt, ws, wsb, M, N, xdt, gdt, _stream())
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    rows = _sample(M, N, 2, 9)
    src = rows % P
    ref = O.layernorm_bwd(dy[src], x[src], mean[src], rstd[src], g, rows.size, N, xdt, gdt)
    check_layernorm_bwd(_gather(dxt, rows, N), None, None, ref, x[src], dy[src], g, mean[src],
                        rstd[src], xdt)
    col = _period_sum(lambda k: O.layernorm_bwd(dy[:k], x[:k], mean[:k], rstd[:k], g, k, N, xdt,
                                                gdt, want_exact=False), M)
    Rp = -(-M // partition_blocks(M, N))
    check_column_sum("layernorm dgamma", to_host(dgt), col("dgamma"), col("sg"), 3 + Rp)
    check_column_sum("layernorm dbeta", to_host(dbt), col("dbeta"), col("sb"), 1 + Rp)


# ------------------------------------------------------------------ QK-norm

def test_maxsize_qk_fused_buffer():
    """A fused q/k/v buffer of 32 + 8 + 8 heads of 128 bf16 per token, past
    2^32 bytes; the v heads must come back untouched."""
    xdt = gdt = O.BF16
    Hq, Hk, D = 32, 8, 128
    S = (Hq + 2 * Hk) * D
    T = _rows_for(S, 2, 4099)
    _log(f"maxsize qk T={T} Hq={Hq} Hk={Hk} D={D}")
    buf = G.normal(61, G.STREAM_X, P, S, xdt)
    gq = G.uniform(61, G.STREAM_GAMMA, D, 0.5, 1.5, gdt)
    gk = G.uniform(62, G.STREAM_GAMMA, D, -1.0, 1.0, gdt)
    bt = _tiled(buf, T, S, xdt)
    st = R.rmsnorm_qk_fwd(bt, bt.data_ptr() + Hq * D * 2, to_device(gq, gdt), to_device(gk, gdt),
                          T, Hq, Hk, D, S, S, 1e-6, xdt, gdt, _stream())
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    rows = _sample(T, S, 2, 10)
    src = buf[rows % P].reshape(-1)
    want, _ = O.rmsnorm_heads_fwd(src, gq, rows.size, Hq, D, S, 1e-6, xdt, gdt)
    want, _ = O.rmsnorm_heads_fwd(want, gk, rows.size, Hk, D, S, 1e-6, xdt, gdt, offset=Hq * D)
    got = _gather(bt, rows, S).reshape(rows.size, S)
    want = want.reshape(rows.size, S)
    v = slice((Hq + Hk) * D, S)
    assert np.array_equal(got[:, v], src.reshape(rows.size, S)[:, v]), "v heads modified"
    qk = slice(0, (Hq + Hk) * D)
    check_output(np.ascontiguousarray(got[:, qk]), O.decode(np.ascontiguousarray(want[:, qk]), xdt),
                 np.ascontiguousarray(want[:, qk]), xdt, "qk")
