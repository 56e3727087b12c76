"""GPU parity over the whole accepted input domain: rows whose fp32 statistics
overflow or underflow (huge and tiny magnitudes, subnormal inputs, eps = 0,
eps near the fp32 maximum), all-zero rows, and the same for the backward's
row dot, for every forward kernel family and both backward tiers. Each batch
mixes such rows with ordinary ones, and the ordinary rows must come out bit
for bit as in a batch without the extreme rows (the fp64 redo of a rare row
leaves every other row alone). Tolerances are those of tests/gpu_util.py.

Which rows reach the fp64 path: those whose q = mean(x^2) + eps falls outside
[2^-100, FLT_MAX] in fp32. For bf16 and fp32 inputs that is |x| beyond about
1e19 or below about 1e-15 at eps = 0, and all-zero rows at eps below 2^-100;
fp16 inputs can neither overflow nor underflow fp32 squares, so for them only
all-zero rows at eps < 2^-100 do. Their other extremes (subnormals, values
near 65504) are checked on the fp32 path."""

import numpy as np
import pytest
import torch

import gen as G
import oracle as O
import row_wise_normalization_fwd_amd as R
from gpu_util import (TORCH_DTYPES, check_dgamma, check_dx, check_fp8, check_layernorm,
                      check_mx, check_output, check_rstd, partition_blocks, to_device, to_host,
                      unpack_fp4)

pytestmark = pytest.mark.gpu

PAIRS = [(O.F32, O.F32), (O.F16, O.F16), (O.BF16, O.BF16), (O.BF16, O.F32)]
PAIR_IDS = ["f32", "f16", "bf16", "bf16_gf32"]

# Row scales per input type: "huge" rows overflow fp32 squares (fp16: the
# largest safe scale), "tiny" rows underflow them at eps = 0, the last of
# them subnormal in the input type.
HUGE = {O.F32: [1e20, 1e30, 1e37], O.BF16: [1e20, 1e30, 1e37], O.F16: [3e3]}
TINY = {O.F32: [1e-25, 1e-40], O.BF16: [1e-25, 1e-39], O.F16: [1e-5]}
TINY_EPS = 1e-35  # below 2^-100: all-zero rows take the fp64 path with a finite rstd
MX_MODES = {O.E4M3: R.RMSN_QUANT_MXFP8, O.E2M1: R.RMSN_QUANT_MXFP4}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    R.load_library()
    torch.cuda.set_device(0)


def _stream():
    return torch.cuda.current_stream()


def _log(msg):
    print(msg, flush=True)


def _empty(n, dt, misalign=0):
    buf = torch.empty(n + 16, dtype=TORCH_DTYPES[dt], device="cuda")
    return buf[misalign:misalign + n]


def _put(a, dt, misalign=0):
    t = _empty(a.size, dt, misalign)
    t.copy_(to_device(a.reshape(-1), dt))
    return t


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def scaled_rows(seed, stream, M, N, dt, scales):
    """Seeded N(0,1) rows, row i multiplied by scales[i % len(scales)] (0
    gives an all-zero row), rounded to dt."""
    z = G.normal(seed, stream, M, N, G.F64)
    s = np.array([scales[i % len(scales)] for i in range(M)], np.float64)[:, None]
    return O.round_to(z * s, dt)


def _ordinary(M, scales):
    return np.array([scales[i % len(scales)] == 1.0 for i in range(M)])


def _fwd(x, g, M, N, eps, xdt, gdt, misalign=0, inplace=False):
    xt = _put(x, xdt, misalign)
    yt = xt if inplace else _empty(M * N, xdt, misalign)
    rt = torch.full((M,), -1.0, device="cuda")
    st = R.rmsnorm_fwd(xt, _put(g, gdt), yt, rt, M, N, eps, xdt, gdt, _stream())
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    return to_host(yt).reshape(M, N), to_host(rt)


def run_domain_fwd(M, N, xdt, gdt, scales, eps, seed, misalign=0, inplace=False):
    """The forward on a batch mixing rows of the given scales (1.0 among
    them): parity with the oracle on every row, and the 1.0-scaled rows bit
    for bit as in an all-ordinary batch."""
    _log(f"domain fwd M={M} N={N} x={xdt} g={gdt} scales={scales} eps={eps} "
         f"misalign={misalign} inplace={inplace}")
    x = scaled_rows(seed, G.STREAM_X, M, N, xdt, scales)
    g = G.uniform(seed, G.STREAM_GAMMA, N, 0.5, 1.5, gdt)
    ref = O.rmsnorm_fwd(x, g, M, N, eps, xdt, gdt)
    y, rs = _fwd(x, g, M, N, eps, xdt, gdt, misalign, inplace)
    check_output(y, ref["y_exact"], ref["y"], xdt, "y")
    check_rstd(rs, ref["rstd_exact"])
    x2 = scaled_rows(seed, G.STREAM_X, M, N, xdt, [1.0])
    y2, rs2 = _fwd(x2, g, M, N, eps, xdt, gdt, misalign, inplace)
    same = _ordinary(M, scales)
    assert np.array_equal(_bits(y[same]), _bits(y2[same])), "ordinary rows changed"
    assert np.array_equal(rs[same].view(np.uint32), rs2[same].view(np.uint32))


def domain_cases(xdt, kind):
    """(scales, eps) pairs for one kind of extreme row."""
    if kind == "huge":
        return [([1.0] + HUGE[xdt] + [1.0], 1e-5)]
    if kind == "tiny":
        return [([1.0] + TINY[xdt], 0.0), ([1.0] + TINY[xdt], 1e-5)]
    return [([1.0, 0.0], 1e-5), ([1.0, 0.0, 1.0], TINY_EPS)]


# Shapes per kernel family (16-bit units): register rows, several rows per
# block (64, 1000), two 128-lane groups per block, whose rare rows are each
# redone by one wave (2048 16-bit / 1024 fp32), one 512-lane group (4096),
# the persistent kernel over several iterations per row group (8192 up to
# 4096 rows, beyond that one 256-lane row per block; 16384 and 32768 16-bit
# / fp32 16384 with 512- and 1024-lane groups), and
# LDS-cached and re-read long rows.
FWD_SHAPES = [(37, 64), (20000, 64), (37, 1000), (45, 1024), (45, 2048), (45, 4096), (29, 5000),
              (2600, 8192), (5000, 8192), (1030, 16384), (520, 32768), (3, 20000), (3, 45000)]


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("shape", FWD_SHAPES, ids=[f"{m}x{n}" for m, n in FWD_SHAPES])
@pytest.mark.parametrize("kind", ["huge", "tiny", "zero"])
def test_fwd_domain(kind, shape, pair):
    M, N = shape
    for i, (scales, eps) in enumerate(domain_cases(pair[0], kind)):
        run_domain_fwd(M, N, *pair, scales, eps, seed=N + i)


def test_fwd_rare_rows_outnumber_group_waves():
    """Four rows in five overflow the fp32 sum of squares, over six loop
    iterations per row group of the persistent kernel at 16384 elements (two
    512-lane groups per block): a group's waves take its rare rows in turn,
    so most groups have more rare rows than waves."""
    run_domain_fwd(6144, 16384, O.BF16, O.BF16, [1.0, 1e20, 1e30, 1e37, 1e30], 1e-5, seed=77)


def test_fwd_rare_rows_in_late_iterations():
    """Rare rows in loop iterations 0 to 39 of the persistent kernel at 16384
    elements: 40960 rows give every row group 40 iterations (512 blocks of
    two 512-lane groups on 256 CUs: row r is in iteration r // 1024), so the
    rare-row mask's bit 31 and its high word are used. The batch is 1024
    seeded rows repeated; the rare rows and a sample of the others are
    checked against the oracle, and every other row bit for bit against a
    batch without rare rows."""
    M, N, dt = 40960, 16384, O.BF16
    _log(f"late-iteration rare rows M={M} N={N}")
    base = G.normal(101, G.STREAM_X, 1024, N, dt)
    g = G.uniform(101, G.STREAM_GAMMA, N, 0.5, 1.5, dt)
    gt = _put(g, dt)
    rare = np.array(sorted({1024 * t + k for t in (0, 1, 30, 31, 32, 33, 39)
                            for k in (0, 1, 517, 700, 1023)}))
    scale = np.where(np.arange(rare.size) % 2 == 0, 1e30, 1e37)[:, None]
    xr = O.round_to(O.decode(base[rare % 1024], dt) * scale, dt)

    def run(xt):
        yt = torch.empty_like(xt)
        rt = torch.full((M,), -1.0, device="cuda")
        st = R.rmsnorm_fwd(xt, gt, yt, rt, M, N, 1e-5, dt, dt, _stream())
        assert st == 0, R.rmsnorm_status_string(st)
        torch.cuda.synchronize()
        return yt, rt

    xt = to_device(base, dt).repeat(M // 1024, 1)
    y0, r0 = run(xt)
    xt[torch.from_numpy(rare).cuda()] = to_device(xr, dt)
    y1, r1 = run(xt)
    ref = O.rmsnorm_fwd(xr, g, rare.size, N, 1e-5, dt, dt)
    idx = torch.from_numpy(rare).cuda()
    check_output(to_host(y1[idx]), ref["y_exact"], ref["y"], dt, "rare y")
    check_rstd(to_host(r1[idx]), ref["rstd_exact"])
    keep = torch.ones(M, dtype=torch.bool, device="cuda")
    keep[idx] = False
    assert torch.equal(y1[keep].view(torch.int16), y0[keep].view(torch.int16)), "ordinary rows changed"
    assert torch.equal(r1[keep].view(torch.int32), r0[keep].view(torch.int32))
    sample = np.setdiff1d(np.random.default_rng(5).choice(M, 64, replace=False), rare)
    sref = O.rmsnorm_fwd(base[sample % 1024], g, sample.size, N, 1e-5, dt, dt)
    sidx = torch.from_numpy(sample).cuda()
    check_output(to_host(y1[sidx]), sref["y_exact"], sref["y"], dt, "ordinary y")
    check_rstd(to_host(r1[sidx]), sref["rstd_exact"])


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_fwd_domain_misaligned_inplace(pair):
    xdt, gdt = pair
    for scales, eps in domain_cases(xdt, "tiny") + domain_cases(xdt, "huge"):
        run_domain_fwd(23, 4099, xdt, gdt, scales, eps, seed=81, misalign=1)
        run_domain_fwd(2100, 8192, xdt, gdt, scales, eps, seed=82, inplace=True)
        run_domain_fwd(3, 20001, xdt, gdt, scales, eps, seed=83, misalign=1)


def test_fwd_split_domain():
    """Few very long rows (the split path) with huge, tiny and zero rows."""
    N = 262144
    for xdt in (O.BF16, O.F32):
        run_domain_fwd(4, N, xdt, xdt, [1.0, 1e30, TINY[xdt][-1], 1.0], 0.0, seed=91)
        run_domain_fwd(3, N, xdt, xdt, [1.0, 1e37, 0.0], TINY_EPS, seed=92)
    run_domain_fwd(3, N, O.F16, O.F16, [1.0, 0.0, 1.0], TINY_EPS, seed=93)


def test_fwd_zero_row_eps0_is_nan():
    """eps = 0 with an all-zero row: the definition's 0/0, so rstd = +inf and
    y = NaN, as in the oracle; the other rows are unaffected."""
    for xdt in (O.F32, O.BF16, O.F16):
        for N in (64, 2048, 4096, 8192, 20000, 262144):
            M = 6 if N < 262144 else 2
            _log(f"zero rows eps=0 x={xdt} N={N}")
            x = scaled_rows(3, G.STREAM_X, M, N, xdt, [1.0, 0.0])
            g = G.uniform(3, G.STREAM_GAMMA, N, 0.5, 1.5, xdt)
            ref = O.rmsnorm_fwd(x, g, M, N, 0.0, xdt, xdt)
            assert np.all(np.isnan(ref["y_exact"][1::2]))
            y, rs = _fwd(x, g, M, N, 0.0, xdt, xdt)
            yd = O.decode(y, xdt).reshape(M, N)
            assert np.all(np.isnan(yd[1::2])) and np.all(np.isposinf(rs[1::2])), (xdt, N)
            check_output(y[0::2], ref["y_exact"][0::2], ref["y"][0::2], xdt, "y")
            check_rstd(rs[0::2], ref["rstd_exact"][0::2])


def test_fwd_huge_eps():
    """eps near the fp32 maximum: mean(x^2) + eps overflows fp32 for rows
    around 1e19."""
    for xdt in (O.F32, O.BF16):
        for N in (1024, 4096, 8192, 20000):
            run_domain_fwd(40, N, xdt, xdt, [1.0, 1e19], 3e38, seed=95)


# ------------------------------------------------------------- fused add

def run_domain_fused(M, N, xdt, gdt, seed):
    """x + r of huge magnitude, rows where r = -x (h all zero, at a tiny eps
    so they take the fp64 path), ordinary rows: h bit for bit, y and rstd
    within tolerance."""
    _log(f"domain fused M={M} N={N} x={xdt} g={gdt}")
    big = HUGE[xdt][1 if xdt != O.F16 else 0]
    x = scaled_rows(seed, G.STREAM_X, M, N, xdt, [1.0, big, 1.0])
    r = scaled_rows(seed, G.STREAM_R, M, N, xdt, [1.0, big, 1.0])
    rd = O.decode(r, xdt).reshape(M, N)
    rd[2::3] = -O.decode(x, xdt).reshape(M, N)[2::3]
    r = O.round_to(rd, xdt)
    g = G.uniform(seed, G.STREAM_GAMMA, N, 0.5, 1.5, gdt)
    eps = TINY_EPS
    ref = O.rmsnorm_fused_add_fwd(x, r, g, M, N, eps, xdt, gdt)
    rt, xt, gt = _put(r, xdt), _put(x, xdt), _put(g, gdt)
    yt, st = _empty(M * N, xdt), torch.empty(M, device="cuda")
    assert R.rmsnorm_fused_add_fwd(xt, rt, gt, yt, st, M, N, eps, xdt, gdt, _stream()) == 0
    torch.cuda.synchronize()
    h = to_host(rt).reshape(M, N)
    assert np.array_equal(_bits(h), _bits(ref["h"])), "h not bit-exact"
    assert not O.decode(h, xdt).reshape(M, N)[2::3].any()
    y = to_host(yt).reshape(M, N)
    check_output(y, ref["y_exact"], ref["y"], xdt, "y")
    check_rstd(to_host(st), ref["rstd_exact"])


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("N", [1000, 2048, 4096, 8192, 10240, 20000, 32768, 262144])
def test_fused_domain(N, pair):
    M = {8192: 3001, 262144: 3}.get(N, 31)
    run_domain_fused(M, N, *pair, seed=N + 3)


# ------------------------------------------------------- quantised outputs

@pytest.mark.parametrize("N", [1000, 2048, 3072, 4096, 8192, 10240, 16384, 20000, 28672, 32768])
@pytest.mark.parametrize("mode", [O.QUANT_TENSOR, O.QUANT_ROW], ids=["tensor", "row"])
def test_fp8_domain(mode, N):
    M, xdt, gdt = (2100 if N == 8192 else 70), O.BF16, O.BF16
    for scales, eps in (([1.0, 1e30, 1e-39, 1.0], 0.0), ([1.0, 0.0, 1e37], TINY_EPS)):
        _log(f"domain fp8 mode={mode} M={M} N={N} scales={scales} eps={eps}")
        x = scaled_rows(N + 11, G.STREAM_X, M, N, xdt, scales)
        g = G.uniform(11, G.STREAM_GAMMA, N, 0.5, 1.5, gdt)
        scale = 0.0125
        ref = O.rmsnorm_quant_fwd(x, g, M, N, eps, xdt, gdt, mode,
                                  scale=scale if mode == O.QUANT_TENSOR else None)
        qt = torch.empty(M * N, dtype=torch.uint8, device="cuda")
        if mode == O.QUANT_TENSOR:
            st = torch.full((1,), scale, device="cuda")
        else:
            st = torch.full((M,), float("nan"), device="cuda")
        rt = torch.empty(M, device="cuda")
        assert R.rmsnorm_quant_fwd(_put(x, xdt), None, _put(g, gdt), qt, st, mode, rt, M, N, eps,
                                   xdt, gdt, _stream()) == 0
        torch.cuda.synchronize()
        check_fp8(qt.cpu().numpy().reshape(M, N), ref, mode == O.QUANT_ROW,
                  to_host(st) if mode == O.QUANT_ROW else None)
        check_rstd(to_host(rt), ref["rstd"].astype(np.float64))


@pytest.mark.parametrize("N", [1024, 1536, 2048, 4096, 6144, 8192, 10240, 16384, 20000, 32768])
@pytest.mark.parametrize("elem", [O.E4M3, O.E2M1], ids=["mxfp8", "mxfp4"])
def test_mx_domain(elem, N):
    M, xdt, gdt = (2100 if N == 8192 else 70), O.BF16, O.BF16
    for scales, eps in (([1.0, 1e37, 1e-25, 1.0], 0.0), ([1.0, 0.0, 1e30], TINY_EPS)):
        _log(f"domain mx elem={elem} M={M} N={N} scales={scales} eps={eps}")
        x = scaled_rows(N + 13, G.STREAM_X, M, N, xdt, scales)
        g = G.uniform(13, G.STREAM_GAMMA, N, 0.5, 1.5, gdt)
        ref = O.rmsnorm_mx_fwd(x, g, M, N, eps, xdt, gdt, elem)
        fp4 = elem == O.E2M1
        qt = torch.empty(M * N // (2 if fp4 else 1), dtype=torch.uint8, device="cuda")
        st = torch.empty(M * N // 32, dtype=torch.uint8, device="cuda")
        assert R.rmsnorm_quant_fwd(_put(x, xdt), None, _put(g, gdt), qt, st, MX_MODES[elem], None,
                                   M, N, eps, xdt, gdt, _stream()) == 0
        torch.cuda.synchronize()
        q = qt.cpu().numpy()
        q = unpack_fp4(q, M, N) if fp4 else q.reshape(M, N)
        check_mx(q, st.cpu().numpy(), ref, elem)


# ------------------------------------------------------------- LayerNorm

@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("N", [768, 1000, 2048, 5120, 8192, 12288, 16384, 20000, 28672, 32768])
def test_layernorm_domain(N, pair):
    """Rows whose centred squares overflow, tiny rows at eps = 0, zero rows
    at a tiny eps; with and without beta."""
    xdt, gdt = pair
    M = 2100 if N == 8192 else 37
    big = [3e3] if xdt == O.F16 else [1e20, 1e36]
    for k, (scales, eps) in enumerate((([1.0] + big, 1e-5), ([1.0] + TINY[xdt], 0.0),
                                       ([1.0, 0.0], TINY_EPS))):
        _log(f"domain layernorm M={M} N={N} x={xdt} g={gdt} scales={scales} eps={eps}")
        x = scaled_rows(N + k, G.STREAM_X, M, N, xdt, scales)
        g = G.uniform(N, G.STREAM_GAMMA, N, 0.5, 1.5, gdt)
        b = G.uniform(N, G.STREAM_DY, N, -1.0, 1.0, gdt) if k != 1 else None
        ref = O.layernorm_fwd(x, g, b, M, N, eps, xdt, gdt)
        yt, mt, rt = _empty(M * N, xdt), torch.empty(M, device="cuda"), torch.empty(M, device="cuda")
        assert R.layernorm_fwd(_put(x, xdt), _put(g, gdt), _put(b, gdt) if b is not None else None,
                               yt, mt, rt, M, N, eps, xdt, gdt, _stream()) == 0
        torch.cuda.synchronize()
        check_layernorm(to_host(yt), ref, x, g, b, xdt, to_host(mt), to_host(rt))


@pytest.mark.parametrize("N", [2048, 4096, 20000])
def test_layernorm_huge_offset_rows(N):
    """fp32 values around 1e36 with a small spread: the fp32 row sum
    overflows, the centred values are ordinary."""
    M, xdt = 9, O.F32
    _log(f"domain layernorm offset rows N={N}")
    z = G.normal(17, G.STREAM_X, M, N, G.F64)
    odd = (np.arange(M) % 2 == 1)[:, None]
    x = O.round_to(np.where(odd, 1e36 * (1.0 + 1e-3 * z), z), xdt)
    g = G.uniform(17, G.STREAM_GAMMA, N, 0.5, 1.5, xdt)
    ref = O.layernorm_fwd(x, g, None, M, N, 1e-5, xdt, xdt)
    yt, mt, rt = _empty(M * N, xdt), torch.empty(M, device="cuda"), torch.empty(M, device="cuda")
    assert R.layernorm_fwd(_put(x, xdt), _put(g, xdt), None, yt, mt, rt, M, N, 1e-5, xdt, xdt,
                           _stream()) == 0
    torch.cuda.synchronize()
    check_layernorm(to_host(yt), ref, x, g, None, xdt, to_host(mt), to_host(rt))


# ------------------------------------------------------------- QK-norm

@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("D", [64, 128, 2048])
def test_qk_domain(D, pair):
    """Every third token's q, k and v huge; at eps = 0, tiny tokens; at a tiny
    eps, all-zero q heads."""
    xdt, gdt = pair
    T, Hq, Hk = (300 if D < 2048 else 9), 8, 2
    S = (Hq + 2 * Hk) * D
    es = 4 if xdt == O.F32 else 2
    for eps in (1e-6, 0.0, TINY_EPS):
        _log(f"domain qk T={T} D={D} x={xdt} g={gdt} eps={eps}")
        bufd = G.normal(D, G.STREAM_X, T, S, G.F64)
        bufd[1::3] *= HUGE[xdt][1 if xdt != O.F16 else 0]
        if eps == 0.0:
            bufd[2::5] *= TINY[xdt][0]
        if eps == TINY_EPS:
            bufd[2::5, :Hq * D] = 0.0
        buf = O.round_to(bufd, xdt).reshape(-1)
        gq = G.uniform(D, G.STREAM_GAMMA, D, 0.5, 1.5, gdt)
        gk = G.uniform(D + 1, G.STREAM_GAMMA, D, -1.0, 1.0, gdt)
        want, _ = O.rmsnorm_heads_fwd(buf, gq, T, Hq, D, S, eps, xdt, gdt, offset=0)
        want, _ = O.rmsnorm_heads_fwd(want, gk, T, Hk, D, S, eps, xdt, gdt, offset=Hq * D)
        bt = _put(buf, xdt)
        assert R.rmsnorm_qk_fwd(bt.data_ptr(), bt.data_ptr() + Hq * D * es, _put(gq, gdt),
                                _put(gk, gdt), T, Hq, Hk, D, S, S, eps, xdt, gdt, _stream()) == 0
        torch.cuda.synchronize()
        got = to_host(bt).reshape(T, S)
        moved = np.zeros((T, S), bool)
        moved[:, :(Hq + Hk) * D] = True
        assert np.array_equal(_bits(got[~moved]), _bits(buf.reshape(T, S)[~moved]))
        check_output(got[moved], O.decode(want, xdt).reshape(T, S)[moved],
                     want.reshape(T, S)[moved], xdt, "qk")


# ------------------------------------------------------------- backward

def run_domain_bwd(M, N, xdt, gdt, xscales, dyscales, seed, res=False, gpu_rstd=False):
    """The backward on rows whose products dy x overflow fp32, whose row dot
    overflows, all-zero rows and ordinary rows; rstd from the oracle forward
    (or the library's own forward)."""
    _log(f"domain bwd M={M} N={N} x={xdt} g={gdt} xs={xscales} dys={dyscales} res={res} "
         f"gpu_rstd={gpu_rstd}")
    x = scaled_rows(seed, G.STREAM_X, M, N, xdt, xscales)
    dy = scaled_rows(seed, G.STREAM_DY, M, N, xdt, dyscales)
    g = G.uniform(seed, G.STREAM_GAMMA, N, 0.5, 1.5, gdt)
    dres = G.normal(seed, G.STREAM_DRES, M, N, xdt) if res else None
    xt, gt, dyt = _put(x, xdt), _put(g, gdt), _put(dy, xdt)
    if gpu_rstd:
        rt = torch.empty(M, device="cuda")
        assert R.rmsnorm_fwd(xt, gt, _empty(M * N, xdt), rt, M, N, 1e-5, xdt, gdt, _stream()) == 0
        torch.cuda.synchronize()
        rho = to_host(rt)
    else:
        rho = O.rmsnorm_fwd(x, g, M, N, 1e-5, xdt, gdt, want_exact=False)["rstd"]
        rt = torch.from_numpy(rho.copy()).cuda()
    ref = (O.rmsnorm_fused_add_bwd(dy, x, rho, g, dres, M, N, xdt, gdt) if res
           else O.rmsnorm_bwd(dy, x, rho, g, M, N, xdt, gdt))
    dxt, dgt = _empty(M * N, xdt), torch.full((N,), float("nan"), device="cuda")
    wsb = R.rmsnorm_bwd_workspace_size(M, N)
    ws = torch.full((max(wsb, 16) // 4,), float("nan"), device="cuda")
    drt = _put(dres, xdt) if res else None

    def call():
        if res:
            return R.rmsnorm_fused_add_bwd(dyt, xt, rt, gt, drt, dxt, dgt, ws, wsb, M, N, xdt, gdt,
                                           _stream())
        return R.rmsnorm_bwd(dyt, xt, rt, gt, dxt, dgt, ws, wsb, M, N, xdt, gdt, _stream())

    st = call()
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    dx1, dg1 = to_host(dxt), to_host(dgt)
    check_dx(dx1.reshape(M, N), ref, x, dy, g, rho, xdt, dres=dres)
    check_dgamma(dg1, ref)
    assert call() == 0  # a repeated call is bit for bit the same
    torch.cuda.synchronize()
    assert np.array_equal(_bits(to_host(dxt)), _bits(dx1))
    assert np.array_equal(to_host(dgt).view(np.uint32), dg1.view(np.uint32))


# Short rows, one partition block per row and several, the stage-1 kernel's
# wide rows (1024 lanes of three units with prefetch, four without: 20000,
# 24584, 32768 16-bit; the fused add of 16-bit rows takes three units only),
# and the long-row tier (fp32 beyond 16384, 16-bit beyond 32768).
BWD_SHAPES = [(37, 64), (45, 1024), (700, 1536), (500, 3072), (700, 4096), (700, 8192), (9, 12288),
              (5, 20000), (300, 24584), (300, 32768), (130, 40000)]


@pytest.mark.parametrize("pair", [(O.F32, O.F32), (O.BF16, O.BF16), (O.BF16, O.F32)],
                         ids=["f32", "bf16", "bf16_gf32"])
@pytest.mark.parametrize("shape", BWD_SHAPES, ids=[f"{m}x{n}" for m, n in BWD_SHAPES])
def test_bwd_domain(shape, pair):
    M, N = shape
    # Huge x (the row dot overflows at 1e37), dy 1e25 against x 1e20 (every
    # product dy x beyond fp32), all-zero rows, ordinary rows.
    run_domain_bwd(M, N, *pair, [1.0, 1e20, 1e30, 1e37, 0.0, 1e20],
                   [1.0, 1.0, 1.0, 10.0, 1.0, 1e25], seed=N + 1)
    run_domain_bwd(M, N, *pair, [1.0, 1e37], [1.0, 1e3], seed=N + 2, res=True)


def test_bwd_domain_gpu_forward_rstd():
    """End to end: the library's forward rstd of extreme rows feeds its
    backward (tiny rows: rstd 1e25 from the fp64 forward path)."""
    for N in (4096, 20000):
        run_domain_bwd(300 if N == 4096 else 9, N, O.BF16, O.BF16, [1.0, 1e30, 1e-25],
                       [1.0, 1.0, 1.0], seed=5, gpu_rstd=True)


@pytest.mark.parametrize("N", [4096, 20000])
def test_bwd_fp16_extremes(N):
    """fp16: zero rows and rows near the top of the fp16 range."""
    M = 45 if N == 4096 else 7
    run_domain_bwd(M, N, O.F16, O.F16, [1.0, 0.0, 3e3], [1.0, 1.0, 20.0], seed=6)
    run_domain_bwd(M, N, O.F16, O.F16, [1.0, 0.0, 3e3], [1.0, 1.0, 20.0], seed=6, res=True)


# ----------------------------------------------------- dgamma at long M

def test_dgamma_long_m_strict_bound():
    """131072 x 1024 bf16: with at most 64 rows per stage-1 partial, every
    column of dgamma meets max(1e-3 |o|, 2^-24 sum_i |dy x rho|) with no
    widening for the number of rows."""
    M, N, xdt = 131072, 1024, O.BF16
    assert -(-M // partition_blocks(M, N)) == 64
    _log(f"dgamma long M={M} N={N}")
    x = G.normal(21, G.STREAM_X, M, N, xdt)
    dy = G.normal(21, G.STREAM_DY, M, N, xdt)
    g = G.uniform(21, G.STREAM_GAMMA, N, 0.5, 1.5, xdt)
    rho = O.rmsnorm_fwd(x, g, M, N, 1e-5, xdt, xdt, want_exact=False)["rstd"]
    ref = O.rmsnorm_bwd(dy, x, rho, g, M, N, xdt, xdt, want_exact=False)
    dxt, dgt = _empty(M * N, xdt), torch.empty(N, device="cuda")
    wsb = R.rmsnorm_bwd_workspace_size(M, N)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    assert R.rmsnorm_bwd(_put(dy, xdt), _put(x, xdt), torch.from_numpy(rho.copy()).cuda(),
                         _put(g, xdt), dxt, dgt, ws, wsb, M, N, xdt, xdt, _stream()) == 0
    torch.cuda.synchronize()
    rel = check_dgamma(to_host(dgt), ref)
    _log(f"dgamma normwise relative error {rel:.3e}")
