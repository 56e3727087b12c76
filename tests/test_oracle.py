"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: hand-derived
exact rows (tests/golden/exact_rows.txt), closed forms of special inputs,
independent library rounding (numpy's float64->float16, torch's
float32->bfloat16, C's double->float), exact decimal arithmetic, and central
finite differences of the forward for the backward. Together they are chosen so
that a plausible slip in the oracle (a dropped eps, N-1 for N, a wrong sign, a
transposed operand, a misplaced gamma index, a wrong rounding tie) fails one.
"""

import decimal
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "exact_rows.txt")


def _f16_all_finite():
    p = np.arange(0, 0x7c00, dtype=np.uint16)
    return p, p.view(np.float16).astype(np.float64)


# ----------------------------------------------------------------- rounding

def test_round_f16_matches_numpy_everywhere():
    pats, vals = _f16_all_finite()
    mids = (vals[:-1] + vals[1:]) / 2            # every tie between neighbours
    rng = np.random.default_rng(1)
    rand = rng.standard_normal(50000) * 10.0 ** rng.integers(-9, 6, 50000)
    special = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 1e6, -1e6,
                        2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14 - 2.0 ** -25,
                        1 + 2.0 ** -11 + 2.0 ** -40])
    v = np.concatenate([vals, -vals, mids, -mids, rand, special])
    got = O.round_to(v, O.F16)
    with np.errstate(over="ignore"):
        want = v.astype(np.float16)
    assert np.array_equal(got, want.view(np.uint16))


def test_round_bf16_matches_torch_on_f32_values():
    # All bf16 neighbours' midpoints are fp32 values, where torch's float32 ->
    # bfloat16 conversion is round-to-nearest-even.
    hi = np.arange(0, 0x7f80, dtype=np.uint32)
    vals = (hi << 16).view(np.float32)
    mids = ((hi[:-1] << 16) | 0x8000).view(np.float32)
    rng = np.random.default_rng(2)
    rand = (rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000)).astype(np.float32)
    near_max = np.array([3.3895314e38, 3.3961776e38, 3.40e38, -3.40e38], np.float32)
    v32 = np.concatenate([vals, -vals, mids, -mids, rand, near_max])
    got = O.round_to(v32.astype(np.float64), O.BF16)
    want = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_round_f32_matches_c_conversion():
    rng = np.random.default_rng(3)
    rand = rng.standard_normal(100000) * 10.0 ** rng.integers(-40, 38, 100000)
    f = rng.standard_normal(20000).astype(np.float32)
    nxt = np.nextafter(f, np.float32(np.inf))
    mids = (f.astype(np.float64) + nxt.astype(np.float64)) / 2    # exact ties
    sub = np.array([1e-45, 7e-46, 2.0 ** -150, 3 * 2.0 ** -151, 1.2e-38, 3.5e38])
    v = np.concatenate([rand, mids, -mids, sub])
    with np.errstate(over="ignore"):
        want = v.astype(np.float32)
    assert np.array_equal(O.round_to(v, O.F32).view(np.uint32), want.view(np.uint32))


def test_decode_all_16bit_patterns():
    p = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f16 = O.decode(p, O.F16)
    assert np.array_equal(f16, p.view(np.float16).astype(np.float64), equal_nan=True)
    bf = O.decode(p, O.BF16)
    want = torch.from_numpy(p.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(bf, want, equal_nan=True)


# ------------------------------------------------------------------ forward

def _golden_cases():
    cases = []
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            eps, x, g, y, rstd = [part.strip() for part in line.split("|")]
            cases.append((float(eps), [float(t) for t in x.split()],
                          [float(t) for t in g.split()], [float(t) for t in y.split()],
                          float(rstd)))
    return cases


@pytest.mark.parametrize("dt", [O.F32, O.F16, O.BF16, O.F64])
def test_forward_exact_rows(dt):
    cases = _golden_cases()
    assert len(cases) >= 8
    for eps, x, g, y, rstd in cases:
        N = len(x)
        xs, gs = O.round_to(np.array(x), dt), O.round_to(np.array(g), dt)
        assert np.array_equal(O.decode(xs, dt), x) and np.array_equal(O.decode(gs, dt), g)
        out = O.rmsnorm_fwd(xs, gs, 1, N, eps, dt, dt)
        assert np.array_equal(out["y_exact"][0], np.array(y)), (eps, x)
        assert np.array_equal(O.decode(out["y"], dt)[0], np.array(y)), (eps, x)
        assert out["rstd_exact"][0] == pytest.approx(rstd, rel=1e-15)
        assert out["rstd"][0] == np.float32(rstd)


@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.25])
def test_forward_constant_row_closed_form(eps):
    # Row of constant c: y_j = c / sqrt(c^2 + eps) * gamma_j.
    # eps crosses the boundary as an fp32 value; both sides use that value.
    N = 24
    g = np.linspace(0.5, 1.5, N)
    eps = float(np.float32(eps))
    for c in [1e-3, 0.5, 3.0, -7.0, 2.0 ** -10, 123.25]:
        out = O.rmsnorm_fwd(np.full(N, c), g, 1, N, eps, O.F64, O.F64)
        want = c / math.sqrt(c * c + eps) * g
        np.testing.assert_allclose(out["y_exact"][0], want, rtol=1e-14, atol=0)
        assert out["rstd_exact"][0] == pytest.approx(1 / math.sqrt(c * c + eps), rel=1e-14)


def test_forward_rms_is_one(gen_mod):
    # gamma = 1: mean(y^2) = ms / (ms + eps), which is 1 at eps = 0.
    M, N = 16, 1000
    x = gen_mod.normal(7, 1, M, N, gen_mod.F64)
    g = np.ones(N)
    out0 = O.rmsnorm_fwd(x, g, M, N, 0.0, O.F64, O.F64)
    np.testing.assert_allclose((out0["y_exact"] ** 2).mean(axis=1), 1.0, rtol=1e-13)
    out1 = O.rmsnorm_fwd(x, g, M, N, 0.5, O.F64, O.F64)   # 0.5 is exact in fp32
    ms = out0["ms"]
    np.testing.assert_allclose((out1["y_exact"] ** 2).mean(axis=1), ms / (ms + 0.5), rtol=1e-13)
    np.testing.assert_allclose(ms, (x ** 2).mean(axis=1), rtol=1e-13)


def test_forward_scale_invariance(gen_mod):
    M, N = 8, 257
    x = gen_mod.normal(8, 1, M, N, gen_mod.F64)
    g = gen_mod.uniform(8, 4, N, 0.5, 1.5, gen_mod.F64)
    base = O.rmsnorm_fwd(x, g, M, N, 0.0, O.F64, O.F64)["y_exact"]
    # Powers of two scale every intermediate exactly: results are identical.
    for a in [2.0 ** -20, 0.25, 8.0, 2.0 ** 30]:
        assert np.array_equal(O.rmsnorm_fwd(x * a, g, M, N, 0.0, O.F64, O.F64)["y_exact"], base)
    for a in [3.0, 1e-3, 777.7]:
        np.testing.assert_allclose(O.rmsnorm_fwd(x * a, g, M, N, 0.0, O.F64, O.F64)["y_exact"],
                                   base, rtol=1e-13, atol=1e-300)
    # With eps > 0: y(a x)_j = a x_j gamma_j / sqrt(a^2 ms + eps).
    eps, a = float(np.float32(0.3)), 0.05
    ms = (x ** 2).mean(axis=1, keepdims=True)
    want = a * x * g / np.sqrt(a * a * ms + eps)
    np.testing.assert_allclose(O.rmsnorm_fwd(x * a, g, M, N, eps, O.F64, O.F64)["y_exact"],
                               want, rtol=1e-13)


def test_forward_domain_edges(gen_mod):
    """The oracle over the whole input domain, against exact power-of-two
    scaling and the definition: fp32 rows at 2^100 (squares far beyond fp32)
    and on the fp32 subnormal grid give the same y as the rows at scale 1;
    rstd scales by the inverse power and rounds to +inf in fp32 once it
    exceeds FLT_MAX; a zero row gives 0/0 = NaN at eps = 0 and 0 at eps > 0;
    eps near FLT_MAX is added in double."""
    M, N = 4, 64
    z = O.round_to(gen_mod.normal(21, 1, M, N, gen_mod.F64), O.BF16)   # 8-bit mantissas
    zd = O.decode(z, O.BF16).reshape(M, N)
    zd[np.abs(zd) < 2.0 ** -8] = 2.0 ** -8           # keep every value on the subnormal grid below
    g = O.round_to(gen_mod.uniform(21, 4, N, 0.5, 1.5, gen_mod.F64), O.F32)
    base = O.rmsnorm_fwd(O.round_to(zd, O.F32), g, M, N, 0.0, O.F32, O.F32)
    for k in (100, -130):                            # 2^-130 * 2^-8 * 2^-7: subnormal, exact
        x = O.round_to(zd * 2.0 ** k, O.F32)
        assert np.array_equal(O.decode(x, O.F32).reshape(M, N), zd * 2.0 ** k)
        out = O.rmsnorm_fwd(x, g, M, N, 0.0, O.F32, O.F32)
        assert np.array_equal(out["y_exact"], base["y_exact"]), k
        assert np.array_equal(out["rstd_exact"], base["rstd_exact"] * 2.0 ** -k), k
        if k < 0:  # rstd around 2^130 / rms: beyond FLT_MAX (2^128), so +inf in fp32
            big = out["rstd_exact"] > float(np.finfo(np.float32).max)
            assert big.any() and np.all(np.isposinf(out["rstd"][big]))
    # Zero rows.
    x0 = np.zeros((2, N), np.float32)
    nan = O.rmsnorm_fwd(x0, g, 2, N, 0.0, O.F32, O.F32)
    assert np.all(np.isnan(nan["y_exact"])) and np.all(np.isposinf(nan["rstd_exact"]))
    eps = float(np.float32(1e-35))
    zero = O.rmsnorm_fwd(x0, g, 2, N, eps, O.F32, O.F32)
    assert np.all(zero["y_exact"] == 0.0)
    assert np.all(zero["rstd_exact"] == 1.0 / math.sqrt(eps))
    # eps near the fp32 maximum: mean(x^2) + eps exceeds FLT_MAX, in double.
    eps = float(np.float32(3e38))
    x = O.round_to(zd * 2.0 ** 64, O.F32)
    out = O.rmsnorm_fwd(x, g, M, N, eps, O.F32, O.F32)
    xd = O.decode(x, O.F32).reshape(M, N)
    q = (xd ** 2).mean(axis=1) + eps
    assert np.all(q > float(np.finfo(np.float32).max))
    np.testing.assert_allclose(out["rstd_exact"], 1.0 / np.sqrt(q), rtol=1e-15)


def test_backward_domain_scaling(gen_mod):
    """The backward at magnitudes whose products overflow fp32, against its
    exact scaling laws: dx is linear in dy, so dy * 2^100 gives dx * 2^100;
    x * 2^k with rstd * 2^-k gives dx * 2^-k and the same dgamma."""
    M, N = 3, 96
    x = O.round_to(gen_mod.normal(22, 1, M, N, gen_mod.F64), O.BF16)
    dy = O.round_to(gen_mod.normal(22, 3, M, N, gen_mod.F64), O.BF16)
    g = O.round_to(gen_mod.uniform(22, 4, N, 0.5, 1.5, gen_mod.F64), O.F32)
    rho = np.array([0.75, 1.25, 2.0])                # powers of two times short mantissas
    base = O.rmsnorm_bwd(dy, x, rho, g, M, N, O.BF16, O.F32)
    dyd = O.decode(dy, O.BF16)
    big = O.rmsnorm_bwd(O.round_to(dyd * 2.0 ** 100, O.BF16), x, rho, g, M, N, O.BF16, O.F32)
    assert np.array_equal(big["dx_exact"], base["dx_exact"] * 2.0 ** 100)
    assert np.array_equal(big["dgamma"], base["dgamma"] * 2.0 ** 100)
    xd = O.decode(x, O.BF16)
    for k in (60, -60):
        sc = O.rmsnorm_bwd(dy, O.round_to(xd * 2.0 ** k, O.BF16), rho * 2.0 ** -k, g, M, N,
                           O.BF16, O.F32)
        assert np.array_equal(sc["dx_exact"], base["dx_exact"] * 2.0 ** -k), k
        assert np.array_equal(sc["dgamma"], base["dgamma"]), k


def test_forward_brute_force_decimal(gen_mod):
    # 4 x 8 bf16 input, recomputed in 60-digit decimal arithmetic.
    M, N, eps = 4, 8, 1e-5
    x = gen_mod.normal(9, 1, M, N, gen_mod.BF16)
    g = gen_mod.uniform(9, 4, N, 0.5, 1.5, gen_mod.BF16)
    xd, gd = O.decode(x, O.BF16).reshape(M, N), O.decode(g, O.BF16)
    out = O.rmsnorm_fwd(x, g, M, N, eps, O.BF16, O.BF16)
    ctx = decimal.Context(prec=60)
    D = decimal.Decimal
    for i in range(M):
        ss = D(0)
        for j in range(N):
            ss = ctx.add(ss, ctx.multiply(D(xd[i, j]), D(xd[i, j])))
        denom = ctx.sqrt(ctx.add(ctx.divide(ss, D(N)), D(float(np.float32(eps)))))
        for j in range(N):
            want = ctx.multiply(ctx.divide(D(xd[i, j]), denom), D(gd[j]))
            assert abs(out["y_exact"][i, j] - float(want)) <= 1e-15 * abs(float(want))
        assert abs(out["rstd_exact"][i] - float(ctx.divide(D(1), denom))) <= 1e-15


@pytest.mark.parametrize("dt", [O.F16, O.BF16])
def test_fused_add_rounds_h_once_and_normalises_h(dt, gen_mod):
    M, N = 32, 300
    x = gen_mod.normal(10, 1, M, N, dt)
    r = gen_mod.normal(10, 2, M, N, dt, row_scale=1e-3, scale_every=3)  # mixed magnitudes
    g = gen_mod.uniform(10, 4, N, 0.5, 1.5, O.F32)
    out = O.rmsnorm_fused_add_fwd(x, r, g, M, N, 1e-5, dt, O.F32)
    s = O.decode(x, dt) + O.decode(r, dt)        # exact in double
    if dt == O.F16:
        want_h = s.astype(np.float16).view(np.uint16)
    else:
        want_h = torch.from_numpy(s.astype(np.float32)).to(torch.bfloat16).view(
            torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out["h"], want_h)
    plain = O.rmsnorm_fwd(out["h"], g, M, N, 1e-5, dt, O.F32)
    assert np.array_equal(out["y_exact"], plain["y_exact"])
    assert np.array_equal(out["y"], plain["y"])
    assert np.array_equal(out["rstd"], plain["rstd"])


def test_forward_gamma_dtype_is_independent(gen_mod):
    # fp32 gamma with bf16 activations uses the full fp32 gamma value.
    M, N = 4, 64
    x = gen_mod.normal(11, 1, M, N, O.BF16)
    g32 = gen_mod.uniform(11, 4, N, 0.5, 1.5, O.F32)
    out = O.rmsnorm_fwd(x, g32, M, N, 1e-5, O.BF16, O.F32)
    xd = O.decode(x, O.BF16)
    want = xd * out["rstd_exact"][:, None] * g32.astype(np.float64)[None, :]
    np.testing.assert_allclose(out["y_exact"], want, rtol=1e-15)


# ----------------------------------------------------------------- backward

def _loss(x, g, dy, M, N, eps):
    return float((dy * O.rmsnorm_fwd(x, g, M, N, eps, O.F64, O.F64)["y_exact"]).sum())


@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.3])
def test_backward_matches_finite_differences(eps, gen_mod):
    M, N = 4, 8
    x = gen_mod.normal(12, 1, M, N, O.F64)
    x[2, :] = 0.75                           # a constant row
    x[3, :] *= 40.0                          # a large-scale row
    dy = gen_mod.normal(12, 3, M, N, O.F64)
    g = gen_mod.uniform(12, 4, N, 0.5, 1.5, O.F64)
    fwd = O.rmsnorm_fwd(x, g, M, N, eps, O.F64, O.F64)
    b = O.rmsnorm_bwd(dy, x, fwd["rstd_exact"], g, M, N, O.F64, O.F64)
    fd_x = np.zeros((M, N))
    for i in range(M):
        for j in range(N):
            h = 1e-5 * max(1.0, abs(x[i, j]))
            xp, xm = x.copy(), x.copy()
            xp[i, j] += h
            xm[i, j] -= h
            fd_x[i, j] = (_loss(xp, g, dy, M, N, eps) - _loss(xm, g, dy, M, N, eps)) / (2 * h)
    fd_g = np.zeros(N)
    for j in range(N):
        h = 1e-5
        gp, gm = g.copy(), g.copy()
        gp[j] += h
        gm[j] -= h
        fd_g[j] = (_loss(x, gp, dy, M, N, eps) - _loss(x, gm, dy, M, N, eps)) / (2 * h)
    for i in range(M):
        scale = np.abs(fd_x[i]).max() + np.abs(dy[i] * g).max() / max(1.0, abs(x[i]).max())
        assert np.abs(b["dx_exact"][i] - fd_x[i]).max() <= 1e-7 * scale, i
    np.testing.assert_allclose(b["dgamma"], fd_g, rtol=1e-7, atol=1e-9)
    # dx_bits is the exact value in fp64 storage
    assert np.array_equal(b["dx"], b["dx_exact"])


def test_backward_euler_invariant_with_saved_fp32_rstd(gen_mod):
    # With the rho actually used: sum_j x_ij dx_ij = N c_i rho_i (1 - rho_i^2 ms_i).
    M, N = 16, 512
    x = gen_mod.normal(13, 1, M, N, O.BF16)
    dy = gen_mod.normal(13, 3, M, N, O.BF16)
    g = gen_mod.uniform(13, 4, N, 0.5, 1.5, O.BF16)
    fwd = O.rmsnorm_fwd(x, g, M, N, 1e-5, O.BF16, O.BF16)
    rho = fwd["rstd"].astype(np.float64)
    b = O.rmsnorm_bwd(dy, x, rho, g, M, N, O.BF16, O.BF16)
    xd = O.decode(x, O.BF16)
    lhs = (xd * b["dx_exact"]).sum(axis=1)
    rhs = N * b["c"] * rho * (1 - rho ** 2 * fwd["ms"])
    mag = np.abs(xd * b["dx_exact"]).sum(axis=1)
    assert np.all(np.abs(lhs - rhs) <= 1e-12 * mag)


def test_backward_radial_direction(gen_mod):
    # gamma = 1, dy = a x  =>  dx = a rho (1 - rho^2 ms) x; zero at eps = 0.
    M, N, a = 6, 96, 2.0
    x = gen_mod.normal(14, 1, M, N, O.F64)
    g = np.ones(N)
    for eps in [0.0, 0.2]:
        fwd = O.rmsnorm_fwd(x, g, M, N, eps, O.F64, O.F64)
        rho = fwd["rstd_exact"]
        b = O.rmsnorm_bwd(a * x, x, rho, g, M, N, O.F64, O.F64)
        want = a * rho[:, None] * (1 - rho[:, None] ** 2 * fwd["ms"][:, None]) * x
        tol = 1e-13 * a * rho[:, None] * np.abs(x)
        assert np.all(np.abs(b["dx_exact"] - want) <= tol + 1e-300)
        if eps == 0.0:
            assert np.abs(b["dx_exact"]).max() <= 1e-13 * a * rho.max() * np.abs(x).max()


def test_dgamma_with_unit_dy_and_constant_rows():
    # dy = 1 and row i constant c_i: dgamma_j = sum_i c_i / sqrt(c_i^2 + eps).
    cs = np.array([0.5, -2.0, 3.0, 1e-3, 7.25])
    M, N, eps = len(cs), 10, float(np.float32(1e-5))
    x = np.repeat(cs[:, None], N, axis=1)
    g = np.linspace(0.5, 1.5, N)
    fwd = O.rmsnorm_fwd(x, g, M, N, eps, O.F64, O.F64)
    b = O.rmsnorm_bwd(np.ones((M, N)), x, fwd["rstd_exact"], g, M, N, O.F64, O.F64)
    want = float(sum(c / math.sqrt(c * c + eps) for c in cs))
    np.testing.assert_allclose(b["dgamma"], want, rtol=1e-14)


def test_backward_tolerance_magnitudes(gen_mod):
    M, N = 3, 40
    x = gen_mod.normal(15, 1, M, N, O.F64)
    dy = gen_mod.normal(15, 3, M, N, O.F64)
    g = gen_mod.uniform(15, 4, N, 0.5, 1.5, O.F64)
    rho = np.array([0.9, 1.1, 2.0])
    b = O.rmsnorm_bwd(dy, x, rho, g, M, N, O.F64, O.F64)
    np.testing.assert_allclose(b["a"], np.abs(dy * g * x).mean(axis=1), rtol=1e-14)
    np.testing.assert_allclose(b["s"], np.abs(dy * x * rho[:, None]).sum(axis=0), rtol=1e-14)
    np.testing.assert_allclose(b["c"], (dy * g * x).mean(axis=1), rtol=1e-12, atol=1e-15)


# ------------------------------------------------------ fused-add backward

def _fused_loss(x, r, g, dy, dres, M, N, eps):
    h = x + r                                   # fp64 storage: exact sum
    y = O.rmsnorm_fwd(h, g, M, N, eps, O.F64, O.F64)["y_exact"]
    return float((dy * y).sum() + (dres * h).sum())


def test_fused_add_backward_matches_finite_differences(gen_mod):
    # L = sum dy * RMSNorm(x + r) + sum dres * (x + r): dL/dx = dL/dr = dh.
    M, N, eps = 3, 8, float(np.float32(1e-3))
    x = gen_mod.normal(16, 1, M, N, O.F64)
    r = gen_mod.normal(16, 2, M, N, O.F64)
    dy = gen_mod.normal(16, 3, M, N, O.F64)
    dres = gen_mod.normal(16, 5, M, N, O.F64)
    g = gen_mod.uniform(16, 4, N, 0.5, 1.5, O.F64)
    h = x + r
    rho = O.rmsnorm_fwd(h, g, M, N, eps, O.F64, O.F64)["rstd_exact"]
    out = O.rmsnorm_fused_add_bwd(dy, h, rho, g, dres, M, N, O.F64, O.F64)
    for which in ("x", "r"):
        fd = np.zeros((M, N))
        for i in range(M):
            for j in range(N):
                step = 1e-5 * max(1.0, abs(h[i, j]))
                p, m = x.copy(), x.copy()
                q, n = r.copy(), r.copy()
                if which == "x":
                    p[i, j] += step
                    m[i, j] -= step
                else:
                    q[i, j] += step
                    n[i, j] -= step
                fd[i, j] = (_fused_loss(p, q, g, dy, dres, M, N, eps) -
                            _fused_loss(m, n, g, dy, dres, M, N, eps)) / (2 * step)
        scale = np.abs(fd).max(axis=1, keepdims=True)
        assert np.all(np.abs(out["dx_exact"] - fd) <= 1e-7 * scale), which


def test_fused_add_backward_reduces_to_plain_and_to_dres(gen_mod):
    M, N = 5, 96
    h = gen_mod.normal(17, 1, M, N, O.BF16)
    dy = gen_mod.normal(17, 3, M, N, O.BF16)
    dres = gen_mod.normal(17, 5, M, N, O.BF16)
    g = gen_mod.uniform(17, 4, N, 0.5, 1.5, O.BF16)
    rho = O.rmsnorm_fwd(h, g, M, N, 1e-5, O.BF16, O.BF16)["rstd"]
    plain = O.rmsnorm_bwd(dy, h, rho, g, M, N, O.BF16, O.BF16)
    none = O.rmsnorm_fused_add_bwd(dy, h, rho, g, None, M, N, O.BF16, O.BF16)
    assert np.array_equal(none["dx"], plain["dx"]) and np.array_equal(none["dgamma"], plain["dgamma"])
    both = O.rmsnorm_fused_add_bwd(dy, h, rho, g, dres, M, N, O.BF16, O.BF16)
    np.testing.assert_allclose(both["dx_exact"], plain["dx_exact"] + O.decode(dres, O.BF16).reshape(M, N),
                               rtol=0, atol=1e-12)
    zero_dy = np.zeros_like(dy)
    only = O.rmsnorm_fused_add_bwd(zero_dy, h, rho, g, dres, M, N, O.BF16, O.BF16)
    assert np.array_equal(only["dx"], dres.reshape(M, N))    # RNE(dres) == dres
    assert np.all(only["dgamma"] == 0)


# ------------------------------------------------------ fp8 e4m3 quantised output

def _e4m3_torch(v32: np.ndarray) -> np.ndarray:
    """torch's float32 -> float8_e4m3fn conversion (nearest, ties to even; it
    gives NaN instead of saturating beyond 464)."""
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e4m3_saturating(v: np.ndarray) -> np.ndarray:
    """torch's conversion where it is defined (|v| <= 464), +-448 beyond."""
    v = np.asarray(v, np.float64)
    big = np.abs(v) > 464.0
    out = _e4m3_torch(np.where(big, 0.0, v))
    out[big] = np.where(v[big] < 0, 0xfe, 0x7e)
    return out


def _e4m3_all_finite():
    codes = np.arange(0, 0x7f, dtype=np.uint8)          # 0x7f is NaN
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    return codes, vals


def test_decode_all_e4m3_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = O.decode(codes, O.E4M3)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2   # 0x7f, 0xff
    assert np.array_equal(got[~nan], want[~nan])
    assert got[0x7e] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_round_e4m3_matches_torch_and_saturates():
    _, vals = _e4m3_all_finite()
    mids = (vals[:-1] + vals[1:]) / 2                   # every tie between neighbours
    q1 = vals[:-1] + (vals[1:] - vals[:-1]) / 4
    q3 = vals[:-1] + 3 * (vals[1:] - vals[:-1]) / 4
    rng = np.random.default_rng(4)
    rand = rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000)
    edge = np.array([448.0, 456.0, 460.0, 463.99, 464.0, 2.0 ** -10, 3 * 2.0 ** -11,
                     2.0 ** -6 - 2.0 ** -10, 2.0 ** -6 - 2.0 ** -11])
    v = np.concatenate([vals, -vals, mids, -mids, q1, q3, rand, edge, -edge])
    v = v[np.abs(v) <= 464.0].astype(np.float32).astype(np.float64)   # torch's range
    assert np.array_equal(O.round_to(v, O.E4M3), _e4m3_torch(v))
    # Beyond 464 torch gives NaN; the quantiser saturates at +-448 instead.
    big = np.array([464.5, 500.0, 1e6, 1e300, np.inf])
    assert np.all(O.round_to(big, O.E4M3) == 0x7e)
    assert np.all(O.round_to(-big, O.E4M3) == 0xfe)
    assert O.round_to(np.array([np.nan]), O.E4M3)[0] & 0x7f == 0x7f


def test_quant_tensor_scale_on_exact_rows():
    # A constant row c = 2^k with eps = 0 has rstd = 1/|c| exactly, so y_j is
    # sign(c) * gamma_j exactly; with a power-of-two scale s the code must be
    # the e4m3 rounding of sign(c) * gamma_j / s. gamma (fp32) holds every
    # e4m3 value, tie and quarter point.
    _, vals = _e4m3_all_finite()
    mids = (vals[:-1] + vals[1:]) / 2
    q1 = vals[:-1] + (vals[1:] - vals[:-1]) / 4
    g = np.concatenate([vals, mids, q1, [456.0, 463.0, 464.0]]).astype(np.float32)
    N = g.size
    for c, s in ((1.0, 1.0), (-4.0, 1.0), (0.5, 0.125), (2.0, 4.0)):
        x = O.round_to(np.full((2, N), c), O.BF16)
        out = O.rmsnorm_quant_fwd(x, g, 2, N, 0.0, O.BF16, O.F32, O.QUANT_TENSOR, scale=s)
        want = _e4m3_saturating(np.sign(c) * g.astype(np.float64) / s)
        assert np.array_equal(out["q"][0], want) and np.array_equal(out["q"][1], want), (c, s)
        assert np.all(out["scale"] == np.float32(s))


def test_quant_row_scale_maps_each_row_max_to_448(gen_mod):
    M, N = 40, 300
    x = gen_mod.normal(31, 1, M, N, O.BF16, 50.0, 7)
    xs = O.decode(x, O.BF16).reshape(M, N)
    xs[3] = -np.abs(xs[3])                              # a row whose extreme is negative
    x = O.round_to(xs, O.BF16)
    g = gen_mod.uniform(31, 4, N, -1.5, 1.5, O.BF16)    # signed weights
    fwd = O.rmsnorm_fwd(x, g, M, N, 1e-5, O.BF16, O.BF16)
    out = O.rmsnorm_quant_fwd(x, g, M, N, 1e-5, O.BF16, O.BF16, O.QUANT_ROW)
    y = fwd["y_exact"]
    s = np.abs(y).max(axis=1) / 448.0
    np.testing.assert_allclose(out["scale_exact"], s, rtol=1e-15, atol=0)
    assert np.array_equal(out["scale"], s.astype(np.float32))
    assert np.array_equal(out["rstd"], fwd["rstd"])
    deq = O.decode(out["q"], O.E4M3).reshape(M, N)
    assert np.all(np.abs(deq).max(axis=1) == 448.0)
    # Each code is the nearest e4m3 value of y/s: within half a step.
    t = y / s[:, None]
    step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(np.abs(t), 2.0 ** -30))), -6) - 3)
    assert np.all(np.abs(deq - t) <= step / 2 + 1e-12)
    assert np.all(np.sign(deq[deq != 0]) == np.sign(t[deq != 0]))


def test_quant_fused_and_zero_rows(gen_mod):
    M, N = 6, 64
    x = gen_mod.normal(32, 1, M, N, O.F16)
    r = gen_mod.normal(32, 2, M, N, O.F16)
    g = gen_mod.uniform(32, 4, N, 0.5, 1.5, O.F32)
    ref = O.rmsnorm_fused_add_fwd(x, r, g, M, N, 1e-6, O.F16, O.F32)
    out = O.rmsnorm_quant_fwd(x, g, M, N, 1e-6, O.F16, O.F32, O.QUANT_ROW, r=r)
    assert np.array_equal(out["h"], ref["h"])
    np.testing.assert_allclose(out["q_exact"] * out["scale_exact"][:, None], ref["y_exact"],
                               rtol=1e-14, atol=0)
    tq = O.rmsnorm_quant_fwd(x, g, M, N, 1e-6, O.F16, O.F32, O.QUANT_TENSOR, scale=0.01, r=r)
    np.testing.assert_allclose(tq["q_exact"], ref["y_exact"] / np.float64(np.float32(0.01)),
                               rtol=1e-14, atol=0)
    # Zero weights give zero rows: scale 0 and zero codes in the per-row mode.
    z = O.rmsnorm_quant_fwd(x, np.zeros(N, np.float32), M, N, 1e-6, O.F16, O.F32, O.QUANT_ROW)
    assert np.all(z["scale"] == 0) and np.all(z["q"] & 0x7f == 0)


# ------------------------------------------------------- per-head QK-RMSNorm

def test_heads_forward_on_a_fused_qkv_buffer(gen_mod):
    # q, k, v of T tokens interleaved in one buffer (token stride S, with two
    # padding elements); normalising q and k must equal the plain forward of
    # the gathered head vectors, in (token, head) order, and leave v and the
    # padding untouched.
    T, Hq, Hk, D = 5, 4, 2, 24
    S = (Hq + 2 * Hk) * D + 2
    for dt, gdt in ((O.BF16, O.BF16), (O.F16, O.F32), (O.F32, O.F32)):
        buf = gen_mod.normal(41, 1, 1, T * S, dt).reshape(-1)
        gq = gen_mod.uniform(41, 4, D, 0.5, 1.5, gdt)
        gk = gen_mod.uniform(42, 4, D, -1.0, 1.0, gdt)
        out, rq = O.rmsnorm_heads_fwd(buf, gq, T, Hq, D, S, 1e-6, dt, gdt, offset=0)
        out, rk = O.rmsnorm_heads_fwd(out, gk, T, Hk, D, S, 1e-6, dt, gdt, offset=Hq * D)
        b2, o2 = buf.reshape(T, S), out.reshape(T, S)
        for off, H, g, rs in ((0, Hq, gq, rq), (Hq * D, Hk, gk, rk)):
            rows = np.ascontiguousarray(b2[:, off:off + H * D]).reshape(T * H, D)
            ref = O.rmsnorm_fwd(rows, g, T * H, D, 1e-6, dt, gdt)
            got = np.ascontiguousarray(o2[:, off:off + H * D]).reshape(T * H, D)
            assert np.array_equal(got.view(np.uint8), ref["y"].view(np.uint8))
            assert np.array_equal(rs, ref["rstd"])
        rest = (Hq + Hk) * D
        assert np.array_equal(o2[:, rest:].view(np.uint8), b2[:, rest:].view(np.uint8))


def test_heads_forward_contiguous_is_the_plain_forward(gen_mod):
    T, H, D = 7, 3, 64
    x = gen_mod.normal(43, 1, T * H, D, O.BF16)
    g = gen_mod.uniform(43, 4, D, 0.5, 1.5, O.BF16)
    out, rs = O.rmsnorm_heads_fwd(x.reshape(-1), g, T, H, D, H * D, 1e-5, O.BF16, O.BF16)
    ref = O.rmsnorm_fwd(x, g, T * H, D, 1e-5, O.BF16, O.BF16)
    assert np.array_equal(out.reshape(T * H, D), ref["y"]) and np.array_equal(rs, ref["rstd"])
    # Heads of one token differ: scaling head 1 of every token by 4 changes
    # only those rstds, by exactly 1/4.
    xs = O.decode(x, O.BF16).reshape(T, H, D)
    xs[:, 1, :] *= 4.0
    out2, rs2 = O.rmsnorm_heads_fwd(O.round_to(xs, O.BF16).reshape(-1), g, T, H, D, H * D,
                                    0.0, O.BF16, O.BF16)
    _, rs0 = O.rmsnorm_heads_fwd(x.reshape(-1), g, T, H, D, H * D, 0.0, O.BF16, O.BF16)
    r0, r2 = rs0.reshape(T, H), rs2.reshape(T, H)
    assert np.array_equal(r2[:, 0], r0[:, 0]) and np.array_equal(r2[:, 2], r0[:, 2])
    assert np.array_equal(r2[:, 1], r0[:, 1] / 4)


# ------------------------------------------------------------------ LayerNorm

def test_layernorm_alternating_row_closed_form():
    # A row alternating +a, -a has mean 0 and variance a^2, so
    # y_j = +-a / sqrt(a^2 + eps) * gamma_j + beta_j.
    N, eps = 64, 1e-5
    for a in (0.25, 3.0, 1000.0):
        x = np.tile([a, -a], N // 2).reshape(1, N)
        g = np.linspace(0.5, 1.5, N)
        b = np.linspace(-2.0, 2.0, N)
        out = O.layernorm_fwd(x, g, b, 1, N, eps, O.F64, O.F64)
        sign = np.tile([1.0, -1.0], N // 2)
        want = sign * a / np.sqrt(a * a + np.float64(np.float32(eps))) * g + b
        np.testing.assert_allclose(out["y_exact"][0], want, rtol=1e-14, atol=1e-14)
        assert out["mean_exact"][0] == 0.0


def test_layernorm_output_statistics_and_invariances(gen_mod):
    M, N = 6, 257
    x = gen_mod.normal(51, 1, M, N, O.F64) * 3.0 + 7.0       # large mean
    g, b = np.ones(N), np.zeros(N)
    out = O.layernorm_fwd(x, g, b, M, N, 0.0, O.F64, O.F64)
    y = out["y_exact"]
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose((y ** 2).mean(axis=1), 1.0, rtol=1e-13)
    # Shift and (eps = 0) scale invariance.
    gg = gen_mod.uniform(51, 4, N, 0.5, 1.5, O.F64)
    bb = gen_mod.uniform(52, 4, N, -1.0, 1.0, O.F64)
    y0 = O.layernorm_fwd(x, gg, bb, M, N, 0.0, O.F64, O.F64)["y_exact"]
    y1 = O.layernorm_fwd(x + 1024.0, gg, bb, M, N, 0.0, O.F64, O.F64)["y_exact"]
    y2 = O.layernorm_fwd(x * 0.125, gg, bb, M, N, 0.0, O.F64, O.F64)["y_exact"]
    np.testing.assert_allclose(y1, y0, rtol=0, atol=1e-10)
    np.testing.assert_allclose(y2, y0, rtol=0, atol=1e-13)
    # Without beta it is the RMSNorm of the centred row (same eps).
    xc = x - x.mean(axis=1, keepdims=True)
    ln = O.layernorm_fwd(x, gg, None, M, N, 1e-3, O.F64, O.F64)
    rms = O.rmsnorm_fwd(xc, gg, M, N, 1e-3, O.F64, O.F64)
    np.testing.assert_allclose(ln["y_exact"], rms["y_exact"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ln["rstd_exact"], rms["rstd_exact"], rtol=1e-13)


def test_layernorm_brute_force_decimal(gen_mod):
    M, N, eps = 3, 8, 1e-5
    x = gen_mod.normal(53, 1, M, N, O.BF16)
    g = gen_mod.uniform(53, 4, N, 0.5, 1.5, O.BF16)
    b = gen_mod.uniform(54, 4, N, -1.0, 1.0, O.BF16)
    xd, gd, bd = O.decode(x, O.BF16).reshape(M, N), O.decode(g, O.BF16), O.decode(b, O.BF16)
    out = O.layernorm_fwd(x, g, b, M, N, eps, O.BF16, O.BF16)
    ctx = decimal.Context(prec=60)
    D = decimal.Decimal
    for i in range(M):
        s = sum((D(v) for v in xd[i]), D(0))
        mean = ctx.divide(s, D(N))
        sq = sum((ctx.multiply(D(v) - mean, D(v) - mean) for v in xd[i]), D(0))
        denom = ctx.sqrt(ctx.add(ctx.divide(sq, D(N)), D(float(np.float32(eps)))))
        assert abs(out["mean_exact"][i] - float(mean)) <= 1e-15 * max(1.0, abs(float(mean)))
        for j in range(N):
            want = ctx.add(ctx.multiply(ctx.divide(D(xd[i, j]) - mean, denom), D(gd[j])), D(bd[j]))
            assert abs(out["y_exact"][i, j] - float(want)) <= 1e-14 * (1 + abs(float(want)))
        assert np.float32(float(ctx.divide(D(1), denom))) == out["rstd"][i]


def _ln_loss(x, g, b, dy, M, N, eps):
    return float((dy * O.layernorm_fwd(x, g, b, M, N, eps, O.F64, O.F64)["y_exact"]).sum())


@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.3])
def test_layernorm_backward_matches_finite_differences(eps, gen_mod):
    M, N = 4, 8
    x = gen_mod.normal(55, 1, M, N, O.F64)
    x[2, :] += 30.0                           # a row with a large mean
    x[3, :] *= 40.0
    dy = gen_mod.normal(55, 3, M, N, O.F64)
    g = gen_mod.uniform(55, 4, N, 0.5, 1.5, O.F64)
    b = gen_mod.uniform(56, 4, N, -1.0, 1.0, O.F64)
    f = O.layernorm_fwd(x, g, b, M, N, eps, O.F64, O.F64)
    out = O.layernorm_bwd(dy, x, f["mean_exact"], f["rstd_exact"], g, M, N, O.F64, O.F64)

    def fd(arr, idx, fn):
        h = 1e-5 * max(1.0, abs(arr[idx]))
        p, m = arr.copy(), arr.copy()
        p[idx] += h
        m[idx] -= h
        return (fn(p) - fn(m)) / (2 * h)

    fd_x = np.array([[fd(x, (i, j), lambda a: _ln_loss(a, g, b, dy, M, N, eps))
                      for j in range(N)] for i in range(M)])
    fd_g = np.array([fd(g, j, lambda a: _ln_loss(x, a, b, dy, M, N, eps)) for j in range(N)])
    fd_b = np.array([fd(b, j, lambda a: _ln_loss(x, g, a, dy, M, N, eps)) for j in range(N)])
    scale = np.abs(fd_x).max(axis=1, keepdims=True) + 1e-3
    assert np.all(np.abs(out["dx_exact"] - fd_x) <= 1e-6 * scale)
    np.testing.assert_allclose(out["dgamma"], fd_g, rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(out["dbeta"], fd_b, rtol=1e-7, atol=1e-9)


def test_layernorm_backward_invariants(gen_mod):
    # Shift invariance: sum_j dx_ij = 0. With eps = 0, scale invariance:
    # sum_j dx_ij (x_ij - mean_i) = 0.
    M, N = 8, 300
    x = gen_mod.normal(57, 1, M, N, O.BF16)
    dy = gen_mod.normal(57, 3, M, N, O.BF16)
    g = gen_mod.uniform(57, 4, N, 0.5, 1.5, O.BF16)
    f = O.layernorm_fwd(x, g, None, M, N, 0.0, O.BF16, O.BF16)
    out = O.layernorm_bwd(dy, x, f["mean_exact"], f["rstd_exact"], g, M, N, O.BF16, O.BF16)
    dx = out["dx_exact"]
    xc = O.decode(x, O.BF16).reshape(M, N) - f["mean_exact"][:, None]
    mag = np.abs(dx).sum(axis=1)
    assert np.all(np.abs(dx.sum(axis=1)) <= 1e-13 * mag)
    assert np.all(np.abs((dx * xc).sum(axis=1)) <= 1e-12 * (np.abs(dx * xc).sum(axis=1)))
    np.testing.assert_allclose(out["dbeta"], O.decode(dy, O.BF16).reshape(M, N).sum(axis=0),
                               rtol=1e-15)


# ------------------------------------------------- MX block-scaled output

# e2m1 magnitudes by code (sign bit 3): exponent field 0 is subnormal (0, 0.5),
# then 1, 1.5, 2, 3, 4, 6 (bias 1, one fraction bit).
E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_and_rounding_table():
    codes = np.arange(16, dtype=np.uint8)
    want = np.array(E2M1_VALUES + [-v for v in E2M1_VALUES])
    got = O.decode(codes, O.E2M1)
    assert np.array_equal(got, want) and np.signbit(got[8])
    # Every value round-trips; every midpoint goes to the even code; quarter
    # points go to the nearer value; beyond 6 saturates.
    vals = np.array(E2M1_VALUES)
    assert np.array_equal(O.round_to(vals, O.E2M1), np.arange(8))
    mids = (vals[:-1] + vals[1:]) / 2           # 0.25 .. 5: ties
    assert O.round_to(mids, O.E2M1).tolist() == [0, 2, 2, 4, 4, 6, 6]
    q1 = vals[:-1] + (vals[1:] - vals[:-1]) / 4
    q3 = vals[:-1] + 3 * (vals[1:] - vals[:-1]) / 4
    assert O.round_to(q1, O.E2M1).tolist() == list(range(7))
    assert O.round_to(q3, O.E2M1).tolist() == list(range(1, 8))
    assert O.round_to(np.array([6.5, 7.0, 1e9, np.inf]), O.E2M1).tolist() == [7, 7, 7, 7]
    assert O.round_to(np.array([-0.75, -7.0]), O.E2M1).tolist() == [10, 15]


def test_e8m0_decode_matches_torch():
    codes = np.arange(255, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e8m0fnu).float().numpy().astype(np.float64)
    got = O.decode(codes, O.E8M0)
    assert np.array_equal(got[1:], want[1:])        # code 0 is 2^-127 (fp32 keeps it)
    assert got[0] == 2.0 ** -127 and np.isnan(O.decode(np.array([255], np.uint8), O.E8M0)[0])


@pytest.mark.parametrize("elem,emax,top", [(O.E4M3, 8, 448.0), (O.E2M1, 2, 6.0)])
def test_mx_block_scale_and_reconstruction(elem, emax, top, gen_mod):
    M, N = 12, 256
    x = gen_mod.normal(61, 1, M, N, O.BF16, 1e-3, 5)       # rows 0, 5, 10 scaled down
    g = gen_mod.uniform(61, 4, N, -1.5, 1.5, O.BF16)
    xs = O.decode(x, O.BF16).reshape(M, N)
    xs[4, 64:96] = 0.0                                      # one all-zero block
    x = O.round_to(xs, O.BF16)
    out = O.rmsnorm_mx_fwd(x, g, M, N, 1e-5, O.BF16, O.BF16, elem)
    y = O.rmsnorm_fwd(x, g, M, N, 1e-5, O.BF16, O.BF16)["y_exact"]
    yb = y.reshape(M, N // 32, 32)
    amax = np.abs(yb).max(axis=2)
    assert np.array_equal(out["amax"], amax)
    X = O.decode(out["scale"], O.E8M0).reshape(M, N // 32)
    nz = amax > 0
    # The scale is the power of two that puts the block max in [2^emax, 2^(emax+1)).
    r = amax[nz] / X[nz]
    assert np.all((r >= 2.0 ** emax) & (r < 2.0 ** (emax + 1)))
    assert np.all(out["scale"][~nz] == 0) and np.all(out["q"].reshape(M, N // 32, 32)[~nz] & 0x7f == 0)
    # Elements: nearest representable value of y / X (or the saturated top).
    t = yb / X[:, :, None]
    deq = O.decode(out["q"], elem).reshape(M, N // 32, 32)
    sat = np.abs(t) > top
    assert np.all(np.abs(deq[sat]) == top) and np.all(np.sign(deq[sat]) == np.sign(t[sat]))
    lead = np.floor(np.log2(np.maximum(np.abs(t), 1e-300)))
    frac_bits, min_exp = (3, -6) if elem == O.E4M3 else (1, 0)
    step = np.exp2(np.maximum(lead, min_exp) - frac_bits)
    assert np.all(np.abs(deq - t)[~sat] <= step[~sat] / 2 + 1e-12)
    np.testing.assert_allclose(out["q_exact"].reshape(M, N // 32, 32), t, rtol=1e-15, atol=0)


def test_mx_fused_and_worked_block():
    # One hand-worked block: gamma 1, eps 0, a row of 32 values whose RMS is
    # known exactly: x = [4, 4, ..., 4 (16 times), -2 (16 times)] -> ms = 10,
    # y = x / sqrt(10). amax = 4 / sqrt(10) = 1.2649.. -> floor(log2) = 0.
    N = 32
    x = O.round_to(np.array([[4.0] * 16 + [-2.0] * 16]), O.BF16)
    g = O.round_to(np.ones(N), O.BF16)
    out4 = O.rmsnorm_mx_fwd(x, g, 1, N, 0.0, O.BF16, O.BF16, O.E2M1)
    assert out4["scale"][0, 0] == 127 - 2            # X = 2^(0 - 2) = 0.25
    # 1.2649 / 0.25 = 5.06 -> 6;  0.6325 / 0.25 = 2.53 -> 3 (negative: code 8 + 5)
    assert out4["q"][0].tolist() == [7] * 16 + [13] * 16
    out8 = O.rmsnorm_mx_fwd(x, g, 1, N, 0.0, O.BF16, O.BF16, O.E4M3)
    assert out8["scale"][0, 0] == 127 - 8            # X = 2^-8
    # 1.2649 * 256 = 323.8 -> 320 (step 32 above 256); 0.6325 * 256 = 161.9 -> 160
    assert np.array_equal(O.decode(out8["q"][0], O.E4M3), np.array([320.0] * 16 + [-160.0] * 16))
    # The fused variant quantises the forward of the rounded sum.
    xr = O.round_to(np.array([[1.0] * 32]), O.BF16)
    fused = O.rmsnorm_mx_fwd(xr, g, 1, N, 0.0, O.BF16, O.BF16, O.E2M1, r=O.round_to(
        O.decode(x, O.BF16).reshape(1, N) - 1.0, O.BF16))
    assert np.array_equal(fused["h"], x) and np.array_equal(fused["q"], out4["q"])
