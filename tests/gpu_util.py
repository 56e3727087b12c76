"""Helpers for the GPU parity tests: host <-> device transfer of storage arrays
and the comparators that define the tolerances.

Tolerances (fixed here, used by every GPU test):
  * 16-bit outputs (y, h, dx): ordinal-ulp distance <= 1 from the oracle value
    rounded to the same type (both neighbours of an exact value are correct
    results); h must match bit for bit.
  * fp32 outputs (y, rstd): relative error <= 1e-5 against the oracle's double
    value (0/0 counts as 0), or, for y, an absolute error <= 2^-144 (32 units
    of the smallest subnormal): no fp32 evaluation resolves a subnormal
    result to 1e-5 of itself. rstd beyond the fp32 range must be +inf (the
    oracle's fp32 rounding of it).
  * dx: within 1 ulp, or, where gamma*dy and x*rho^2*c cancel, absolute error
    <= 2^-18 * rho * (|gamma dy| + |x| rho^2 A) with A = mean_j |dy gamma x|
    (an fp32 evaluation cannot resolve a cancelled result below that scale).
  * dh of the fused-add backward: as dx, with 2^-22 |dresidual| added to the
    floor for the fp32 addition of the residual gradient.
  * dgamma: |g - o| <= max(1e-3 |o|, 2^-24 S_j) with S_j = sum_i |dy x rho|.
  * LayerNorm y: within 1 ulp (fp32: relative 1e-5), or, where the centring
    or beta cancel, |y - y_exact| <= 2^-18 rstd |gamma| (|x - mean| + A) +
    2^-22 |beta| with A = mean_j |x_ij| (the fp32 mean carries an error of a
    few 2^-24 A); mean: |m - mean| <= 2^-18 A + 2^-149 (the fp32 spacing of
    subnormals); rstd: relative 1e-5.
  * LayerNorm dx: within 1 ulp, or |dx - exact| <= 2^-18 rstd (|gamma dy| +
    A1 + |xhat| A2) with A1 = mean_j |gamma dy|, A2 = mean_j |gamma dy xhat|;
    dgamma: |g - o| <= max(1e-3 |o|, (3 + R) 2^-24 S_j), S_j = sum_i |dy xhat|,
    R = rows per partition block (xhat = (x - mean) rstd costs two fp32
    roundings and the FMA a third, then R fp32 additions per block); dbeta
    likewise with (1 + R) and S_j = sum_i |dy| (additions only).
  * MX codes: E8M0 scale codes equal to the oracle's, except where the
    block's amax lies within 2^-18 (relative) of a power of two, where the
    neighbouring code is accepted; elements within one step of the oracle's
    rounding of y under the kernel's scale.
  * fp8 e4m3 codes: ordinal distance <= 1 from the oracle's code (the kernel
    scales in fp32, so y / s can land on the other side of a tie); per-row
    scales: relative error <= 1e-5; every nonzero row's largest code is
    +-448 exactly.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle as O

TORCH_DTYPES = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}

F32_FLOOR = 2.0 ** -144
# Smallest double that rounds to +inf in fp32: the largest fp32 value plus
# half its ulp.
F32_MAX_ROUND = float(np.finfo(np.float32).max) * (1.0 + 2.0 ** -25)


def to_device(a: np.ndarray, dt: int, device="cuda") -> torch.Tensor:
    if dt == O.F32:
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.view(TORCH_DTYPES[dt]).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy().copy()
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def ordinal16(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_distance16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(ordinal16(a) - ordinal16(b))


def rel_error(got: np.ndarray, exact: np.ndarray) -> np.ndarray:
    got = got.astype(np.float64)
    diff = np.abs(got - exact)
    den = np.abs(exact)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(den > 0, diff / den, np.where(diff == 0, 0.0, np.inf))
    return r


def check_output(got: np.ndarray, exact: np.ndarray, rounded: np.ndarray, dt: int, what: str):
    """Forward-style check of an output against the oracle."""
    assert got.shape == rounded.shape, (what, got.shape, rounded.shape)
    if dt == O.F32:
        r = rel_error(got, exact)
        r = np.where(np.abs(got.astype(np.float64) - exact) <= F32_FLOOR, 0.0, r)
        worst = float(r.max()) if r.size else 0.0
        assert worst <= 1e-5, f"{what}: max relative error {worst:.3e} > 1e-5"
        return worst
    d = ulp_distance16(got, rounded)
    worst = int(d.max()) if d.size else 0
    if worst > 1:
        idx = np.unravel_index(int(d.argmax()), d.shape)
        raise AssertionError(f"{what}: {int((d > 1).sum())} elements beyond 1 ulp; worst {worst} "
                             f"at {idx}: got {got[idx]:#06x}, oracle {rounded[idx]:#06x}")
    return worst


def check_rstd(got: np.ndarray, exact: np.ndarray):
    big = exact > F32_MAX_ROUND  # rounds to +inf in fp32
    assert np.all(np.isposinf(got[big])), "rstd beyond the fp32 range must be +inf"
    r = rel_error(got[~big], exact[~big])
    worst = float(r.max()) if r.size else 0.0
    assert worst <= 1e-5, f"rstd: max relative error {worst:.3e}"
    return worst


def check_dx(got: np.ndarray, ref: dict, x: np.ndarray, dy: np.ndarray, gamma: np.ndarray,
             rho: np.ndarray, dt: int, dres: np.ndarray | None = None):
    """Returns the number of elements that passed only through the floor.

    With ``dres`` (fused-add backward) the kernel adds it to the fp32 norm
    gradient before the one rounding; that addition can cancel, so the floor
    also covers one fp32 rounding of each addend (2^-22 |dres| is generous)."""
    M, N = got.shape
    xd = O.decode(x, dt).reshape(M, N)
    dyd = O.decode(dy, dt).reshape(M, N)
    gd = O.decode(gamma, O.F32 if gamma.dtype == np.float32 else dt)
    exact = ref["dx_exact"]
    if dt == O.F32:
        ok_ulp = rel_error(got, exact) <= 1e-5
        gotv = got.astype(np.float64)
    else:
        ok_ulp = ulp_distance16(got, ref["dx"]) <= 1
        gotv = O.decode(got, dt).reshape(M, N)
    rho2 = rho[:, None].astype(np.float64)
    floor = 2.0 ** -18 * rho2 * (np.abs(gd[None, :] * dyd) + np.abs(xd) * rho2 ** 2 * ref["a"][:, None])
    if dres is not None:
        floor = floor + 2.0 ** -22 * np.abs(O.decode(dres, dt).reshape(M, N))
    ok_floor = np.abs(gotv - exact) <= floor
    bad = ~(ok_ulp | ok_floor)
    if bad.any():
        idx = np.unravel_index(int(np.argmax(bad)), bad.shape)
        raise AssertionError(f"dx: {int(bad.sum())} elements out of tolerance; first at {idx}: "
                             f"got {gotv[idx]!r}, exact {exact[idx]!r}, floor {floor[idx]!r}")
    return int((~ok_ulp & ok_floor).sum())


def check_column_sum(name: str, got: np.ndarray, o: np.ndarray, mag: np.ndarray, k: float):
    """A column reduction over the rows (dgamma, dbeta) against the oracle's
    fp64 sum o: within 1e-3 relative, or k * 2^-24 * mag, mag being the sum of
    the terms' magnitudes. Each stage-1 partial is an fp32 sum over R rows,
    whose error is at most about (R + 1) * 2^-24 * mag counting the
    roundings of the products; k = R + 3 leaves room for the fp32 result."""
    tol = np.maximum(1e-3 * np.abs(o), k * 2.0 ** -24 * mag)
    err = np.abs(got.astype(np.float64) - o)
    bad = err > tol
    assert not bad.any(), (f"{name}: {int(bad.sum())} columns out of tolerance; worst ratio "
                           f"{float((err / tol).max()):.3f}")
    return float(np.linalg.norm(got - o) / max(np.linalg.norm(o), 1e-300))


def partition_blocks(M: int, N: int) -> int:
    """Backward partition blocks G for M rows of N: min(M, T) with T = 256,
    or ceil(2^22 / N) for rows longer than 32768 (the long-row tier's tiles),
    more when a block would own over 64 rows (the library's rule, restated)."""
    target = 256 if N <= 32768 else -(-(1 << 22) // N)
    return max(min(M, target), -(-M // 64))


def check_dgamma(got: np.ndarray, ref: dict):
    """dgamma within 1e-3 relative or 2^-24 * sum |terms|. The library's
    partition keeps every stage-1 partial to at most 64 rows, so the bound is
    not widened for the number of rows."""
    return check_column_sum("dgamma", got, ref["dgamma"], ref["s"], 1.0)


def e4m3_ordinal(codes: np.ndarray) -> np.ndarray:
    """Monotone integer image of e4m3 codes (sign-magnitude; +-0 both 0)."""
    c = codes.astype(np.int32)
    mag = c & 0x7f
    return np.where(c & 0x80, -mag, mag)


def check_fp8(got: np.ndarray, ref: dict, per_row: bool, got_scale: np.ndarray | None = None):
    """Codes within one step of the oracle's; per-row scales and row maxima."""
    got = got.reshape(ref["q"].shape)
    assert not np.any((got & 0x7f) == 0x7f), "NaN code in the output"
    d = np.abs(e4m3_ordinal(got) - e4m3_ordinal(ref["q"]))
    if (d > 1).any():
        idx = np.unravel_index(int(np.argmax(d)), d.shape)
        raise AssertionError(f"fp8: {int((d > 1).sum())} codes more than one step off; worst at "
                             f"{idx}: got {got[idx]:#04x}, oracle {ref['q'][idx]:#04x}, "
                             f"y/s {ref['q_exact'][idx]!r}")
    if per_row:
        assert got_scale is not None
        se = ref["scale_exact"]
        err = np.abs(got_scale.astype(np.float64) - se)
        assert np.all(err <= 1e-5 * np.abs(se)), f"scale: worst rel {float((err / np.maximum(se, 1e-300)).max())}"
        nz = se > 0
        top = (got & 0x7f).max(axis=1)
        assert np.all(top[nz] == 0x7e), "a row's largest code is not 448"
        assert np.all((got[~nz] & 0x7f) == 0)
    return int((d == 1).sum())


def check_layernorm(got_y, ref, x, gamma, beta, dt, got_mean=None, got_rstd=None):
    """LayerNorm forward against the oracle (see the module docstring)."""
    M, N = ref["y"].shape
    got_y = got_y.reshape(M, N)
    exact = ref["y_exact"]
    if dt == O.F32:
        ok_ulp = rel_error(got_y, exact) <= 1e-5
        gotv = got_y.astype(np.float64)
    else:
        ok_ulp = ulp_distance16(got_y, ref["y"]) <= 1
        gotv = O.decode(got_y, dt).reshape(M, N)
    gdt = O.F32 if gamma.dtype == np.float32 else dt
    gd = O.decode(gamma, gdt)
    bd = O.decode(beta, gdt) if beta is not None else np.zeros(N)
    xd = O.decode(x, dt).reshape(M, N)
    rs = ref["rstd_exact"][:, None]
    floor = (2.0 ** -18 * rs * np.abs(gd)[None, :] *
             (np.abs(xd - ref["mean_exact"][:, None]) + ref["amag"][:, None]) +
             2.0 ** -22 * np.abs(bd)[None, :])
    ok_floor = np.abs(gotv - exact) <= floor
    bad = ~(ok_ulp | ok_floor)
    if bad.any():
        idx = np.unravel_index(int(np.argmax(bad)), bad.shape)
        raise AssertionError(f"layernorm y: {int(bad.sum())} elements out of tolerance; first at "
                             f"{idx}: got {gotv[idx]!r}, exact {exact[idx]!r}, floor {floor[idx]!r}")
    if got_mean is not None:
        err = np.abs(got_mean.astype(np.float64) - ref["mean_exact"])
        # 2^-149: the fp32 spacing at the bottom of the range, which no fp32
        # mean of subnormal values can beat.
        assert np.all(err <= 2.0 ** -18 * ref["amag"] + 2.0 ** -149), f"mean: worst {float(err.max())}"
    if got_rstd is not None:
        check_rstd(got_rstd, ref["rstd_exact"])
    return int((~ok_ulp & ok_floor).sum())


def check_layernorm_bwd(got_dx, got_dg, got_db, ref, x, dy, gamma, mean, rstd, dt):
    """LayerNorm backward against the oracle run on the same fp32 mean/rstd."""
    M, N = ref["dx"].shape
    got_dx = got_dx.reshape(M, N)
    exact = ref["dx_exact"]
    if dt == O.F32:
        ok_ulp = rel_error(got_dx, exact) <= 1e-5
        gotv = got_dx.astype(np.float64)
    else:
        ok_ulp = ulp_distance16(got_dx, ref["dx"]) <= 1
        gotv = O.decode(got_dx, dt).reshape(M, N)
    gdt = O.F32 if gamma.dtype == np.float32 else dt
    gd = O.decode(gamma, gdt)
    xd = O.decode(x, dt).reshape(M, N)
    dyd = O.decode(dy, dt).reshape(M, N)
    rs = rstd.astype(np.float64)[:, None]
    xh = (xd - mean.astype(np.float64)[:, None]) * rs
    floor = 2.0 ** -18 * rs * (np.abs(gd[None, :] * dyd) + ref["a1"][:, None] +
                               np.abs(xh) * ref["a2"][:, None])
    ok_floor = np.abs(gotv - exact) <= floor
    bad = ~(ok_ulp | ok_floor)
    if bad.any():
        idx = np.unravel_index(int(np.argmax(bad)), bad.shape)
        raise AssertionError(f"layernorm dx: {int(bad.sum())} out of tolerance; first at {idx}: "
                             f"got {gotv[idx]!r}, exact {exact[idx]!r}, floor {floor[idx]!r}")
    R = -(-M // partition_blocks(M, N))  # rows per partition block
    for name, got, o, mag, k in (("dgamma", got_dg, ref["dgamma"], ref["sg"], 3 + R),
                                 ("dbeta", got_db, ref["dbeta"], ref["sb"], 1 + R)):
        if got is not None:
            check_column_sum("layernorm " + name, got, o, mag, k)
    return int((~ok_ulp & ok_floor).sum())


def unpack_fp4(packed: np.ndarray, M: int, N: int) -> np.ndarray:
    """[M, N/2] bytes -> [M, N] codes (element 2k in the low nibble)."""
    p = packed.reshape(M, N // 2)
    out = np.empty((M, N), np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def mx_ordinal(codes: np.ndarray, elem: int) -> np.ndarray:
    c = codes.astype(np.int32)
    if elem == O.E2M1:
        mag, neg = c & 0x7, c & 0x8
    else:
        mag, neg = c & 0x7F, c & 0x80
    return np.where(neg, -mag, mag)


def check_mx(got_q: np.ndarray, got_scale: np.ndarray, ref: dict, elem: int):
    """MX output against the oracle (see the module docstring). Returns the
    number of blocks that took the neighbouring scale code."""
    M, N = ref["q"].shape
    nb = N // 32
    got_q = got_q.reshape(M, N)
    got_scale = got_scale.reshape(M, nb).astype(np.int32)
    ref_scale = ref["scale"].astype(np.int32)
    if elem == O.E4M3:
        assert not np.any((got_q & 0x7F) == 0x7F), "NaN code in the output"
    amax = ref["amax"]
    with np.errstate(divide="ignore"):
        l2 = np.log2(np.where(amax > 0, amax, 1.0))
    near_pow2 = np.abs(l2 - np.round(l2)) < 2.0 ** -18
    diff = got_scale - ref_scale
    bad = (diff != 0) & ~(near_pow2 & (np.abs(diff) == 1))
    if bad.any():
        i, b = np.argwhere(bad)[0]
        raise AssertionError(f"mx scale: {int(bad.sum())} blocks differ; first ({i}, {b}): got "
                             f"{got_scale[i, b]}, oracle {ref_scale[i, b]}, amax {amax[i, b]!r}")
    # Elements: re-quantise the oracle's y under the kernel's scale where it differs.
    y = ref["q_exact"].reshape(M, nb, 32) * np.exp2(ref_scale - 127.0)[:, :, None]
    want = ref["q"].reshape(M, nb, 32).copy()
    moved = diff != 0
    if moved.any():
        t = y * np.exp2(127.0 - got_scale)[:, :, None]
        want[moved] = O.round_to(t[moved], elem)
    d = np.abs(mx_ordinal(got_q.reshape(M, nb, 32), elem) - mx_ordinal(want, elem))
    if (d > 1).any():
        i, b, j = np.argwhere(d > 1)[0]
        raise AssertionError(f"mx elements: {int((d > 1).sum())} codes more than one step off; "
                             f"first ({i}, {b}, {j}): got {got_q.reshape(M, nb, 32)[i, b, j]:#x}, "
                             f"want {want[i, b, j]:#x}, y {y[i, b, j]!r}")
    return int(moved.sum())
