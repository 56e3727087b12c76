"""GPU parity on seeded random cases: shapes, dtype pairs, alignment and
variants drawn from a fixed generator, each run through the same checks as
the hand-picked cases in test_gpu_parity.py. Case ids name every parameter."""

import numpy as np
import pytest

import oracle as O
from test_gpu_parity import (PAIRS, QR, QT, _gpu, run_bwd, run_fused, run_fused_bwd, run_fwd,  # noqa: F401
                             run_ln, run_ln_bwd, run_mx, run_qk, run_quant)

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20261202)
_MAX_ELEMS = 1 << 22


def _shape(n_lo=1, n_hi=20000, mult=1):
    N = int(np.exp(_rng.uniform(np.log(n_lo), np.log(n_hi))))
    N = max(mult, (N // mult) * mult)
    M = int(np.exp(_rng.uniform(0, np.log(max(2, min(3000, _MAX_ELEMS // N))))))
    return max(M, 1), N


def _pair():
    return PAIRS[int(_rng.integers(len(PAIRS)))]


def _cases(n, make):
    out = []
    for i in range(n):
        c = make()
        out.append(pytest.param(c, id="-".join(f"{k}{v}" for k, v in c.items())))
    return out


FWD = _cases(40, lambda: dict(zip(("M", "N"), _shape())) | dict(
    pair=_pair(), mis=int(_rng.integers(2)), fused=bool(_rng.integers(2)),
    rstd=bool(_rng.integers(2)), seed=int(_rng.integers(1 << 30))))
BWD = _cases(25, lambda: dict(zip(("M", "N"), _shape())) | dict(
    pair=_pair(), mis=int(_rng.integers(2)), res=bool(_rng.integers(2)),
    seed=int(_rng.integers(1 << 30))))
QUANT = _cases(25, lambda: dict(zip(("M", "N"), _shape())) | dict(
    pair=_pair(), mode=[QT, QR][int(_rng.integers(2))], fused=bool(_rng.integers(2)),
    mis=int(_rng.integers(2)), seed=int(_rng.integers(1 << 30))))
MX = _cases(20, lambda: dict(zip(("M", "N"), _shape(32, 20000, 32))) | dict(
    pair=_pair(), elem=[O.E4M3, O.E2M1][int(_rng.integers(2))], fused=bool(_rng.integers(2)),
    seed=int(_rng.integers(1 << 30))))
QK = _cases(15, lambda: dict(
    T=int(_rng.integers(1, 300)), Hq=int(_rng.integers(1, 33)), Hk=int(_rng.integers(0, 9)),
    D=[64, 80, 96, 128, 160, 256][int(_rng.integers(6))], pad=int(_rng.integers(0, 3)) * 8,
    pair=_pair(), mis=int(_rng.integers(2)), seed=int(_rng.integers(1 << 30))))
LN = _cases(15, lambda: dict(zip(("M", "N"), _shape())) | dict(
    pair=_pair(), mis=int(_rng.integers(2)), beta=bool(_rng.integers(2)),
    seed=int(_rng.integers(1 << 30))))
LNB = _cases(12, lambda: dict(zip(("M", "N"), _shape())) | dict(
    pair=_pair(), mis=int(_rng.integers(2)), seed=int(_rng.integers(1 << 30))))


@pytest.mark.parametrize("c", FWD)
def test_random_forward(c):
    if c["fused"]:
        run_fused(c["M"], c["N"], *c["pair"], seed=c["seed"], want_rstd=c["rstd"],
                  misalign=c["mis"])
    else:
        run_fwd(c["M"], c["N"], *c["pair"], seed=c["seed"], want_rstd=c["rstd"],
                misalign=c["mis"])


@pytest.mark.parametrize("c", BWD)
def test_random_backward(c):
    if c["res"]:
        run_fused_bwd(c["M"], c["N"], *c["pair"], seed=c["seed"], misalign=c["mis"])
    else:
        run_bwd(c["M"], c["N"], *c["pair"], seed=c["seed"], misalign=c["mis"])


@pytest.mark.parametrize("c", QUANT)
def test_random_fp8(c):
    run_quant(c["M"], c["N"], *c["pair"], c["mode"], seed=c["seed"], fused=c["fused"],
              misalign=c["mis"])


@pytest.mark.parametrize("c", MX)
def test_random_mx(c):
    run_mx(c["M"], c["N"], *c["pair"], c["elem"], seed=c["seed"], fused=c["fused"])


@pytest.mark.parametrize("c", QK)
def test_random_qk(c):
    layout = "q_only" if c["Hk"] == 0 else "fused"
    run_qk(c["T"], c["Hq"], c["Hk"], c["D"], *c["pair"], layout=layout, pad=c["pad"],
           misalign=c["mis"], seed=c["seed"])


@pytest.mark.parametrize("c", LN)
def test_random_layernorm(c):
    run_ln(c["M"], c["N"], *c["pair"], seed=c["seed"], with_beta=c["beta"], misalign=c["mis"])


@pytest.mark.parametrize("c", LNB)
def test_random_layernorm_bwd(c):
    run_ln_bwd(c["M"], c["N"], *c["pair"], seed=c["seed"], misalign=c["mis"])
