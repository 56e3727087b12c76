"""GPU parity: the HIP kernels, called through the C ABI, against the fp64
oracle, element by element, on seeded inputs. Tolerances are defined in
tests/gpu_util.py. Every case name carries its shape, dtypes and variant."""

import os

import numpy as np
import pytest
import torch

import gen as G
import oracle as O
import row_wise_normalization_fwd_amd as R
from gpu_util import (check_dgamma, check_dx, check_fp8, check_layernorm, check_layernorm_bwd,
                      check_mx, check_output, check_rstd, to_device, to_host, unpack_fp4,
                      TORCH_DTYPES)

pytestmark = pytest.mark.gpu

PAIRS = [(O.F32, O.F32), (O.F16, O.F16), (O.F16, O.F32), (O.BF16, O.BF16), (O.BF16, O.F32)]
PAIR_IDS = ["f32", "f16", "f16_gf32", "bf16", "bf16_gf32"]
# 96 ... 6144: rows that fit half the lanes with three units each (every
# group size from 8 to 512 lanes at 16-bit).
N_SWEEP = [1, 7, 8, 63, 64, 96, 192, 384, 768, 1000, 1024, 1536, 2047, 2048, 3072, 4096, 4999, 5000,
           5001, 5632, 6144, 6152, 7000, 8191, 8192, 8193,
           8196, 12288, 12296, 16384, 20000, 24576, 28000, 32760, 32768]
N_LDS = {O.F32: 20000, O.F16: 40000, O.BF16: 40000}      # 80 KB rows: LDS-cached, 1024 threads
N_REREAD = {O.F32: 45000, O.F16: 90000, O.BF16: 90000}   # 180 KB rows: beyond 160 KiB of LDS
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "exact_rows.txt")


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
    """Device buffer of n elements, optionally starting `misalign` elements past
    a 256-byte boundary (breaks 16-byte row alignment)."""
    buf = torch.empty(n + 16, dtype=TORCH_DTYPES[dt], device="cuda")
    return buf[misalign:misalign + n]


def _put(a, dt, misalign=0):
    t = _empty(a.size, dt, misalign)
    t.copy_(to_device(a.reshape(-1), dt))
    return t


def _inputs(M, N, xdt, gdt, seed, outlier_every=0, outlier_scale=1.0, with_r=False, with_dy=False):
    x = G.normal(seed, G.STREAM_X, M, N, xdt, outlier_scale, outlier_every)
    g = G.uniform(seed, G.STREAM_GAMMA, N, 0.5, 1.5, gdt)
    r = G.normal(seed, G.STREAM_R, M, N, xdt) if with_r else None
    dy = G.normal(seed, G.STREAM_DY, M, N, xdt) if with_dy else None
    return x, g, r, dy


# ------------------------------------------------------------------ forward

def run_fwd(M, N, xdt, gdt, eps=1e-5, seed=7, want_rstd=True, misalign=0, inplace=False,
            outlier_every=0, outlier_scale=1.0):
    _log(f"fwd M={M} N={N} x={xdt} g={gdt} eps={eps} misalign={misalign} inplace={inplace}")
    x, g, _, _ = _inputs(M, N, xdt, gdt, seed, outlier_every, outlier_scale)
    ref = O.rmsnorm_fwd(x, g, M, N, eps, xdt, gdt)
    xt = _put(x, xdt, misalign)
    gt = _put(g, gdt)
    yt = xt if inplace else _empty(M * N, xdt, misalign)
    rt = torch.full((M,), -1.0, device="cuda") if want_rstd else None
    st = R.rmsnorm_fwd(xt, gt, yt, rt, M, N, eps, xdt, gdt, _stream())
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    y = to_host(yt).reshape(M, N)
    check_output(y, ref["y_exact"], ref["y"], xdt, "y")
    if want_rstd:
        check_rstd(to_host(rt), ref["rstd_exact"])
    return x, g, ref, y


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("N", N_SWEEP)
def test_fwd_sweep(N, pair):
    run_fwd(3, N, *pair, seed=100 + N)
    run_fwd(67, N, *pair, seed=200 + N, want_rstd=False)


# Rows of 1537..4096 16-byte units take the persistent kernel with 512 or
# 1024 lanes per row (16-bit N in (12288, 32768], fp32 N in (8192, 16384]):
# enough rows that groups run several loop iterations, the last one ragged.
PP_LONG = {O.F32: [(1500, 8196), (1100, 12288), (1030, 16384)],
           O.F16: [(2100, 16384), (1100, 20000), (1030, 32760)],
           O.BF16: [(2100, 14000), (1100, 24576), (1030, 32768)]}


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_fwd_persistent_long_rows(pair):
    for i, (M, N) in enumerate(PP_LONG[pair[0]]):
        run_fwd(M, N, *pair, seed=40 + i, want_rstd=(i % 2 == 0))
    M, N = PP_LONG[pair[0]][-1]
    run_fwd(M, N, *pair, seed=44, inplace=True)


@pytest.mark.parametrize("pair", [p for p in PAIRS if p[0] != O.F32],
                         ids=[i for p, i in zip(PAIRS, PAIR_IDS) if p[0] != O.F32])
def test_other_outputs_persistent_long_rows(pair):
    """The 16-bit fused add (1024 lanes x 4 units), LayerNorm (512 x 4 and
    1024 x 3), fp8 (512 x 4, 1024 x 3) and MX outputs (also 1024 x 4) of
    long rows on the persistent kernel, over several loop iterations."""
    run_fused(1030, 32768, *pair, seed=45, want_rstd=True)
    run_ln(1100, 12288, *pair, seed=52)
    run_quant(1100, 10240, *pair, QR, seed=53)
    run_mx(1100, 10240, *pair, O.E2M1, seed=54)
    run_ln(1100, 16384, *pair, seed=46)
    run_ln(1030, 20000, *pair, seed=47, with_beta=False)
    run_quant(1100, 16384, *pair, QR, seed=48, want_rstd=True)
    run_quant(1030, 24576, *pair, QT, seed=49)
    run_mx(1030, 20000, *pair, O.E4M3, seed=50)
    run_mx(1030, 32768, *pair, O.E2M1, seed=51, want_rstd=True)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_fwd_long_rows(pair):
    run_fwd(5, N_LDS[pair[0]], *pair, seed=30)
    run_fwd(5, N_REREAD[pair[0]], *pair, seed=31)
    run_fwd(3, N_LDS[pair[0]] + 1, *pair, seed=32, misalign=1)     # scalar units, LDS
    run_fwd(3, N_REREAD[pair[0]] + 3, *pair, seed=33, misalign=1)  # scalar units, re-read


# Few rows too long for the LDS cache take the split path (tiles of 256 lanes x
# 4 units: 8192 16-bit or 4096 fp32 elements; at most half the CU count of
# rows). Lengths give full tiles, a one-unit last tile and a partial one.
SPLIT_N = {O.F32: [45000, 4096 * 24 + 4, 262144], O.F16: [90000, 8192 * 12 + 8, 262144],
           O.BF16: [90000, 8192 * 12 + 8, 262144]}


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_fwd_split_rows(pair):
    for i, N in enumerate(SPLIT_N[pair[0]]):
        run_fwd(1, N, *pair, seed=300 + i, want_rstd=True)
        run_fwd(9, N, *pair, seed=310 + i, want_rstd=(i % 2 == 0))
        run_fused(2, N, *pair, seed=320 + i, want_rstd=(i % 2 == 1))


def test_fwd_split_boundaries():
    """Either side of the row-count switch, the in-place fallback, outlier rows."""
    N = 90000
    run_fwd(128, N, O.BF16, O.BF16, seed=330, want_rstd=True)   # split (256 CUs)
    run_fwd(129, N, O.BF16, O.BF16, seed=331, want_rstd=True)   # one block per row
    run_fwd(4, N, O.BF16, O.BF16, seed=332, inplace=True)       # y == x: one block per row
    run_fwd(3, N, O.F16, O.F16, seed=333, outlier_every=2, outlier_scale=200.0)
    # Fused: y may be x (the partial pass parks its sums over x, which the
    # apply pass no longer reads), and the residual may be x.
    run_fused(2, N, O.BF16, O.BF16, seed=334, want_rstd=True, y_is_x=True)
    run_fused(2, N, O.BF16, O.F32, seed=335, x_is_r=True)


def test_fwd_split_many_tiles():
    """Rows of more than 256 tiles, whose factor adds its partials in several
    batches of four per lane: two launches where the last tile holds a slot
    for every tile of the row, three (the finalize pass) where it does not."""
    run_fwd(2, 8192 * 300 + 4096, O.BF16, O.BF16, seed=336, want_rstd=True)  # 301 tiles, two
    run_fwd(2, 8192 * 300 + 8, O.BF16, O.BF16, seed=337, want_rstd=True)     # 301 tiles, three
    run_fwd(1, 4096 * 700 + 4, O.F32, O.F32, seed=338, want_rstd=True)       # 701 tiles, three
    run_fused(2, 8192 * 520 + 4096, O.BF16, O.BF16, seed=339, want_rstd=True)  # 521 tiles


def test_fwd_split_graph_replay():
    """The split path's three launches captured in a graph: every replay,
    with eager work and other outputs' clearing between replays, equals the
    eager run bit for bit."""
    M, N = 3, 8192 * 12 + 8
    x, g, r, _ = _inputs(M, N, O.BF16, O.BF16, 340, with_r=True)
    xt, gt, r0 = _put(x, O.BF16), _put(g, O.BF16), _put(r, O.BF16)
    rt = r0.clone()
    y, rs = _empty(M * N, O.BF16), torch.empty(M, device="cuda")
    y2 = _empty(M * N, O.BF16)

    def run(stream):
        assert R.rmsnorm_fwd(xt, gt, y, rs, M, N, 1e-5, O.BF16, O.BF16, stream) == 0
        assert R.rmsnorm_fused_add_fwd(xt, rt, gt, y2, None, M, N, 1e-5, O.BF16, O.BF16,
                                       stream) == 0

    run(_stream())
    torch.cuda.synchronize()
    want = [t.cpu().clone() for t in (y, rs, y2, rt)]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rt.copy_(r0)
        with torch.cuda.graph(graph, stream=side):
            run(side)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        rt.copy_(r0)
        for t in (y, rs, y2):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, w in zip((y, rs, y2, rt), want):
            assert torch.equal(t.cpu().view(torch.uint8), w.view(torch.uint8)), rep


@pytest.mark.parametrize("M", [1, 2, 3, 64, 255, 4097])
@pytest.mark.parametrize("N", [16, 64, 1000, 8192])
def test_fwd_row_counts(M, N):
    run_fwd(M, N, O.BF16, O.BF16, seed=M * 31 + N)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("N", [64, 1000, 4096, 8192, 12288])
def test_fwd_misaligned_rows(N, pair):
    # Base pointers one element past a 16-byte boundary take the scalar path.
    run_fwd(9, N, *pair, seed=N + 5, misalign=1)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("N", [1000, 8192, 12288])
def test_fwd_in_place(N, pair):
    run_fwd(6, N, *pair, seed=N + 9, inplace=True)


def test_fwd_empty_is_noop():
    assert R.rmsnorm_fwd(None, None, None, None, 0, 128, 1e-5, O.BF16, O.BF16, _stream()) == 0


def _golden_cases():
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                eps, x, g, y, rstd = [p.strip() for p in line.split("|")]
                yield (float(eps), np.array(x.split(), float), np.array(g.split(), float),
                       np.array(y.split(), float), float(rstd))


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_fwd_exact_rows(pair):
    # Hand-derived rows whose outputs are exact in every type: the GPU must
    # reproduce them exactly (the normalised values need no rounding).
    xdt, gdt = pair
    for eps, x, g, y, rstd in _golden_cases():
        N = x.size
        xt = _put(O.round_to(x, xdt), xdt)
        gt = _put(O.round_to(g, gdt), gdt)
        yt = _empty(N, xdt)
        rt = torch.empty(1, device="cuda")
        assert R.rmsnorm_fwd(xt, gt, yt, rt, 1, N, eps, xdt, gdt, _stream()) == 0
        torch.cuda.synchronize()
        got = O.decode(to_host(yt), xdt)
        assert np.array_equal(got, y), (eps, x, got, y)
        assert abs(float(to_host(rt)[0]) - rstd) <= 2e-7 * rstd


@pytest.mark.parametrize("c", [1e-3, 0.5, 3.0, -7.0])
def test_fwd_constant_row_closed_form(c):
    N, eps = 4096, 1e-5
    x = O.round_to(np.full(N, c), O.BF16)
    cb = float(O.decode(x[:1], O.BF16)[0])
    g = G.uniform(3, G.STREAM_GAMMA, N, 0.5, 1.5, O.BF16)
    gd = O.decode(g, O.BF16)
    want = O.round_to(cb / np.sqrt(cb * cb + float(np.float32(eps))) * gd, O.BF16)
    yt = _empty(N, O.BF16)
    assert R.rmsnorm_fwd(_put(x, O.BF16), _put(g, O.BF16), yt, None, 1, N, eps, O.BF16, O.BF16,
                         _stream()) == 0
    torch.cuda.synchronize()
    from gpu_util import ulp_distance16
    assert ulp_distance16(to_host(yt), want).max() <= 1


def test_fwd_deterministic():
    M, N = 512, 8192
    x, g, _, _ = _inputs(M, N, O.BF16, O.BF16, 77)
    xt, gt = _put(x, O.BF16), _put(g, O.BF16)
    outs = []
    for _ in range(3):
        yt, rt = _empty(M * N, O.BF16), torch.empty(M, device="cuda")
        assert R.rmsnorm_fwd(xt, gt, yt, rt, M, N, 1e-5, O.BF16, O.BF16, _stream()) == 0
        torch.cuda.synchronize()
        outs.append((to_host(yt), to_host(rt)))
    for y, r in outs[1:]:
        assert np.array_equal(y, outs[0][0]) and np.array_equal(r.view(np.uint32),
                                                                outs[0][1].view(np.uint32))


# --------------------------------------------------------------- fused add

def run_fused(M, N, xdt, gdt, eps=1e-5, seed=11, want_rstd=False, misalign=0, x_is_r=False,
              y_is_x=False):
    _log(f"fused M={M} N={N} x={xdt} g={gdt} misalign={misalign} x_is_r={x_is_r} "
         f"y_is_x={y_is_x}")
    x, g, r, _ = _inputs(M, N, xdt, gdt, seed, with_r=True)
    if x_is_r:
        r = x.copy()
    ref = O.rmsnorm_fused_add_fwd(x, r, g, M, N, eps, xdt, gdt)
    rt = _put(r, xdt, misalign)
    xt = rt if x_is_r else _put(x, xdt, misalign)
    gt = _put(g, gdt)
    yt = xt if y_is_x else _empty(M * N, xdt, misalign)
    st_t = torch.empty(M, device="cuda") if want_rstd else None
    st = R.rmsnorm_fused_add_fwd(xt, rt, gt, yt, st_t, M, N, eps, xdt, gdt, _stream())
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    h = to_host(rt).reshape(M, N)
    if xdt == O.F32:
        assert np.array_equal(h.view(np.uint32), ref["h"].view(np.uint32)), "h not bit-exact"
    else:
        assert np.array_equal(h, ref["h"]), f"h not bit-exact: {int((h != ref['h']).sum())} differ"
    y = to_host(yt).reshape(M, N)
    check_output(y, ref["y_exact"], ref["y"], xdt, "y")
    if want_rstd:
        check_rstd(to_host(st_t), ref["rstd_exact"])
    # The fused result is the plain forward of the rounded h, bit for bit.
    y2 = _empty(M * N, xdt, misalign)
    assert R.rmsnorm_fwd(rt, gt, y2, None, M, N, eps, xdt, gdt, _stream()) == 0
    torch.cuda.synchronize()
    assert np.array_equal(to_host(y2).reshape(M, N).view(np.uint8), y.view(np.uint8))
    return ref


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("N", [1, 7, 64, 1000, 2048, 4096, 5000, 8191, 8192, 8193, 8200, 10240,
                               12288, 16384, 24576, 28000, 32768])
def test_fused_sweep(N, pair):
    run_fused(5, N, *pair, seed=300 + N, want_rstd=(N % 2 == 0))


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_fused_long_rows(pair):
    run_fused(3, N_LDS[pair[0]], *pair, seed=40, want_rstd=True)
    run_fused(3, N_REREAD[pair[0]], *pair, seed=41, want_rstd=True)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_fused_misaligned_and_aliased(pair):
    run_fused(7, 4096, *pair, seed=51, misalign=1)
    run_fused(7, 4096, *pair, seed=52, x_is_r=True)
    run_fused(7, 4096, *pair, seed=53, y_is_x=True)


# ------------------------------------------------- quantised (fp8) forward

QT, QR = O.QUANT_TENSOR, O.QUANT_ROW
TENSOR_SCALE = 0.0125   # |y| above 5.6 saturates: a few elements per row do


def run_quant(M, N, xdt, gdt, mode, seed=19, fused=False, eps=1e-5, misalign=0, q_off=0,
              want_rstd=True, outlier_every=0, outlier_scale=1.0, tensor_scale=TENSOR_SCALE):
    _log(f"quant M={M} N={N} x={xdt} g={gdt} mode={mode} fused={fused} misalign={misalign} "
         f"q_off={q_off} rstd={want_rstd}")
    x, g, r, _ = _inputs(M, N, xdt, gdt, seed, outlier_every, outlier_scale, with_r=fused)
    ref = O.rmsnorm_quant_fwd(x, g, M, N, eps, xdt, gdt, mode,
                              scale=tensor_scale if mode == QT else None, r=r)
    xt, gt = _put(x, xdt, misalign), _put(g, gdt)
    rt = _put(r, xdt, misalign) if fused else None
    qbuf = torch.full((M * N + 64,), 0x7f, dtype=torch.uint8, device="cuda")
    qt = qbuf[q_off:q_off + M * N]
    if mode == QT:
        sc = torch.tensor([tensor_scale], dtype=torch.float32, device="cuda")
    else:
        sc = torch.full((M,), float("nan"), device="cuda")
    rs = torch.full((M,), float("nan"), device="cuda") if want_rstd else None
    st = R.rmsnorm_quant_fwd(xt, rt, gt, qt, sc, mode, rs, M, N, eps, xdt, gdt, _stream())
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    q = qt.cpu().numpy().reshape(M, N)
    steps = check_fp8(q, ref, mode == QR, to_host(sc) if mode == QR else None)
    assert np.all(qbuf[:q_off].cpu().numpy() == 0x7f), "write before q"
    assert np.all(qbuf[q_off + M * N:].cpu().numpy() == 0x7f), "write past q"
    if want_rstd:
        check_rstd(to_host(rs), ref["rstd"].astype(np.float64))
    if fused:
        h = to_host(rt).reshape(M, N)
        assert np.array_equal(h.view(np.uint8), ref["h"].view(np.uint8)), "h not bit-exact"
    return steps


@pytest.mark.parametrize("mode", [QT, QR], ids=["tensor", "row"])
@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("N", [1, 7, 64, 768, 1000, 1536, 2048, 3072, 4096, 5000, 6144, 6152, 8191,
                               8192, 8193, 8200, 10240, 12288, 12296, 16384, 20000, 24576, 28672,
                               32768])
def test_quant_sweep(N, pair, mode):
    run_quant(5, N, *pair, mode, seed=1100 + N, want_rstd=(N % 2 == 0))
    run_quant(300, N, *pair, mode, seed=1200 + N, fused=True, want_rstd=(N % 2 == 1))


@pytest.mark.parametrize("mode", [QT, QR], ids=["tensor", "row"])
@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_quant_long_rows_misaligned(pair, mode):
    run_quant(3, N_LDS[pair[0]], *pair, mode, seed=1301)
    run_quant(3, N_REREAD[pair[0]], *pair, mode, seed=1302, fused=True)
    run_quant(7, 4096, *pair, mode, seed=1303, misalign=1)            # scalar units
    run_quant(7, 4096, *pair, mode, seed=1304, q_off=1)               # q not unit-aligned
    run_quant(7, 9000, *pair, mode, seed=1305, q_off=3, fused=True)   # long rows, scalar
    run_quant(1000, 8192, *pair, mode, seed=1306, outlier_every=13, outlier_scale=300.0)


def _e4m3_grid_gamma(max448: bool):
    """fp32 gamma holding every finite e4m3 magnitude, every tie between
    neighbours and a quarter point in each gap, with alternating signs."""
    codes = np.arange(0, 0x7f, dtype=np.uint8)
    vals = O.decode(codes, O.E4M3)
    mids = (vals[:-1] + vals[1:]) / 2
    q1 = vals[:-1] + (vals[1:] - vals[:-1]) / 4
    g = np.concatenate([vals, mids, q1] + ([] if max448 else [[456.0, 463.0, 464.0, 600.0]]))
    g = g * np.where(np.arange(g.size) % 2 == 0, 1.0, -1.0)
    return g.astype(np.float32)


@pytest.mark.parametrize("xdt", [O.F32, O.F16, O.BF16], ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("layout", ["vec", "ragged"])
def test_quant_rounding_is_nearest_even_at_every_tie(xdt, layout):
    # A constant row 2^k with eps = 0 has rstd = 2^-k exactly, so the kernel's
    # y is exactly +-gamma_j; with power-of-two scales y / s is exact too and
    # every code must equal the oracle's bit for bit, ties included. The
    # per-row case uses a gamma whose largest magnitude is 448 (scale 1).
    for mode, max448, scales in ((QT, False, (1.0, 0.125, 4.0)), (QR, True, (None,))):
        g = _e4m3_grid_gamma(max448)
        n8 = -(-g.size // 8) * 8                 # 16-byte rows for every dtype
        pad = n8 - g.size + (3 if layout == "ragged" else 0)
        g = np.concatenate([g, np.zeros(pad, np.float32)])
        N = g.size
        for c in (1.0, -0.25, 8.0):
            M = 3
            x = O.round_to(np.full((M, N), c), xdt)
            for s in scales:
                ref = O.rmsnorm_quant_fwd(x, g, M, N, 0.0, xdt, O.F32, mode, scale=s)
                qt = torch.empty(M * N, dtype=torch.uint8, device="cuda")
                sc = (torch.tensor([s], dtype=torch.float32, device="cuda") if mode == QT
                      else torch.empty(M, device="cuda"))
                assert R.rmsnorm_quant_fwd(_put(x, xdt), None, _put(g, O.F32), qt, sc, mode,
                                           None, M, N, 0.0, xdt, O.F32, _stream()) == 0
                torch.cuda.synchronize()
                got = qt.cpu().numpy().reshape(M, N)
                bad = got != ref["q"]
                assert not bad.any(), (f"c={c} s={s} mode={mode}: {int(bad.sum())} codes differ; "
                                       f"first gamma {g[np.argmax(bad.any(axis=0))]!r}")
                if mode == QR:
                    assert np.all(to_host(sc) == 1.0)


def test_quant_zero_rows_and_tensor_saturation():
    M, N = 8, 4096
    x, g, _, _ = _inputs(M, N, O.BF16, O.BF16, 1401)
    xs = O.decode(x, O.BF16).reshape(M, N)
    xs[2] = 0.0                                       # rstd = 1/sqrt(eps), y = 0
    x = O.round_to(xs, O.BF16)
    ref = O.rmsnorm_quant_fwd(x, g, M, N, 1e-5, O.BF16, O.BF16, QR)
    qt, sc = torch.empty(M * N, dtype=torch.uint8, device="cuda"), torch.empty(M, device="cuda")
    assert R.rmsnorm_quant_fwd(_put(x, O.BF16), None, _put(g, O.BF16), qt, sc, QR, None, M, N,
                               1e-5, O.BF16, O.BF16, _stream()) == 0
    torch.cuda.synchronize()
    check_fp8(qt.cpu().numpy(), ref, True, to_host(sc))
    assert to_host(sc)[2] == 0.0
    # A tiny tensor scale saturates almost everything at +-448.
    ref = O.rmsnorm_quant_fwd(x, g, M, N, 1e-5, O.BF16, O.BF16, QT, scale=1e-6)
    st = torch.tensor([1e-6], dtype=torch.float32, device="cuda")
    assert R.rmsnorm_quant_fwd(_put(x, O.BF16), None, _put(g, O.BF16), qt, st, QT, None, M, N,
                               1e-5, O.BF16, O.BF16, _stream()) == 0
    torch.cuda.synchronize()
    got = qt.cpu().numpy().reshape(M, N)
    assert np.array_equal(got, ref["q"])


def test_quant_matches_plain_forward_values():
    # Dequantised codes track the plain forward's y within one e4m3 step.
    M, N = 256, 8192
    x, g, _, _ = _inputs(M, N, O.BF16, O.BF16, 1402)
    xt, gt = _put(x, O.BF16), _put(g, O.BF16)
    y = _empty(M * N, O.BF16)
    assert R.rmsnorm_fwd(xt, gt, y, None, M, N, 1e-5, O.BF16, O.BF16, _stream()) == 0
    q, sc, _ = R.quant_fwd(xt.view(M, N), gt)
    torch.cuda.synchronize()
    yv = O.decode(to_host(y), O.BF16).reshape(M, N)
    deq = O.decode(q.cpu().numpy(), O.E4M3).reshape(M, N) * to_host(sc)[:, None]
    assert np.all(np.abs(deq - yv) <= np.abs(yv) / 8 + to_host(sc)[:, None] * 2.0 ** -9 + 1e-6)


# --------------------------------------------- MX block-scaled output

MX_MODES = {O.E4M3: R.RMSN_QUANT_MXFP8, O.E2M1: R.RMSN_QUANT_MXFP4}


def run_mx(M, N, xdt, gdt, elem, seed=37, fused=False, want_rstd=False, q_off=0,
           outlier_every=0, outlier_scale=1.0):
    _log(f"mx M={M} N={N} x={xdt} g={gdt} elem={elem} fused={fused} q_off={q_off}")
    x, g, r, _ = _inputs(M, N, xdt, gdt, seed, outlier_every, outlier_scale, with_r=fused)
    ref = O.rmsnorm_mx_fwd(x, g, M, N, 1e-5, xdt, gdt, elem, r=r)
    qbytes = M * N // 2 if elem == O.E2M1 else M * N
    qbuf = torch.full((qbytes + 64,), 0xAB, dtype=torch.uint8, device="cuda")
    qt = qbuf[q_off:q_off + qbytes]
    sbuf = torch.full((M * N // 32 + 64,), 0xAB, dtype=torch.uint8, device="cuda")
    st_ = sbuf[:M * N // 32]
    xt, gt = _put(x, xdt), _put(g, gdt)
    rt = _put(r, xdt) if fused else None
    rs = torch.full((M,), float("nan"), device="cuda") if want_rstd else None
    st = R.rmsnorm_quant_fwd(xt, rt, gt, qt, st_, MX_MODES[elem], rs, M, N, 1e-5, xdt, gdt,
                             _stream())
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    q = qt.cpu().numpy()
    if elem == O.E2M1:
        q = unpack_fp4(q, M, N)
    moved = check_mx(q, st_.cpu().numpy(), ref, elem)
    assert np.all(qbuf[:q_off].cpu().numpy() == 0xAB) and np.all(qbuf[q_off + qbytes:].cpu().numpy() == 0xAB)
    assert np.all(sbuf[M * N // 32:].cpu().numpy() == 0xAB), "write past the scale codes"
    if fused:
        assert np.array_equal(to_host(rt).reshape(M, N).view(np.uint8), ref["h"].view(np.uint8))
    if want_rstd:
        f = O.rmsnorm_fwd(ref["h"] if fused else x, g, M, N, 1e-5, xdt, gdt, want_exact=False)
        check_rstd(to_host(rs), f["rstd"].astype(np.float64))
    return moved


@pytest.mark.parametrize("elem", [O.E4M3, O.E2M1], ids=["mxfp8", "mxfp4"])
@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("N", [32, 64, 96, 768, 800, 1024, 1536, 3072, 4096, 5024, 6144, 8192, 8224,
                               10240, 12288, 12320, 16384, 20000, 24576, 28000, 32768])
def test_mx_sweep(N, pair, elem):
    run_mx(5, N, *pair, elem, seed=2500 + N, want_rstd=True)
    run_mx(300, N, *pair, elem, seed=2600 + N, fused=True)


@pytest.mark.parametrize("elem", [O.E4M3, O.E2M1], ids=["mxfp8", "mxfp4"])
@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_mx_long_rows_and_outliers(pair, elem):
    run_mx(3, 40000, *pair, elem, seed=2701)
    run_mx(3, 90016, *pair, elem, seed=2702, fused=True)
    run_mx(1000, 8192, *pair, elem, seed=2703, outlier_every=13, outlier_scale=300.0, q_off=8)


def _mx_exact_block_gamma(elem):
    """fp32 gamma of 4 blocks of 32 whose block max puts the scale at 1: every
    representable magnitude of the element format that fits, the ties between
    neighbours and quarter points, with alternating signs."""
    if elem == O.E2M1:
        vals = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
        top = 6.5                       # saturates to 6, keeps floor(log2) = 2
    else:
        vals = O.decode(np.arange(0x60, 0x7F, dtype=np.uint8), O.E4M3)  # 32 .. 448
        top = 460.0
    mids = (vals[:-1] + vals[1:]) / 2
    q1 = vals[:-1] + (vals[1:] - vals[:-1]) / 4
    pool = np.concatenate([vals, mids, q1])
    blocks = []
    for b in range(4):
        chunk = np.resize(np.roll(pool, 7 * b), 31)
        blk = np.concatenate([[top], chunk]) * np.where(np.arange(32) % 2 == 0, 1.0, -1.0)
        blocks.append(np.roll(blk, 5 * b))
    return np.concatenate(blocks).astype(np.float32)


@pytest.mark.parametrize("elem", [O.E4M3, O.E2M1], ids=["mxfp8", "mxfp4"])
@pytest.mark.parametrize("xdt", [O.F32, O.F16, O.BF16], ids=["f32", "f16", "bf16"])
def test_mx_rounding_is_nearest_even_at_every_tie(xdt, elem):
    # Constant rows 2^k with eps = 0 give y = +-gamma exactly; every block's
    # max is in [2^emax, 2^(emax+1)), so the scale is 1 and each element code
    # is the exact rounding of gamma: bit-exact, ties included.
    g = _mx_exact_block_gamma(elem)
    N, M = g.size, 3
    for c in (1.0, -0.5, 4.0):
        x = O.round_to(np.full((M, N), c), xdt)
        ref = O.rmsnorm_mx_fwd(x, g, M, N, 0.0, xdt, O.F32, elem)
        assert np.all(ref["scale"] == 127)
        qb = M * N // 2 if elem == O.E2M1 else M * N
        qt = torch.empty(qb, dtype=torch.uint8, device="cuda")
        sc = torch.empty(M * N // 32, dtype=torch.uint8, device="cuda")
        assert R.rmsnorm_quant_fwd(_put(x, xdt), None, _put(g, O.F32), qt, sc, MX_MODES[elem], None,
                                   M, N, 0.0, xdt, O.F32, _stream()) == 0
        torch.cuda.synchronize()
        q = qt.cpu().numpy()
        q = unpack_fp4(q, M, N) if elem == O.E2M1 else q.reshape(M, N)
        assert np.all(sc.cpu().numpy() == 127)
        bad = q != ref["q"]
        assert not bad.any(), f"c={c}: {int(bad.sum())} codes differ"


def test_mx_zero_blocks():
    M, N = 4, 256
    x, g, _, _ = _inputs(M, N, O.BF16, O.BF16, 2801)
    g = O.decode(g, O.BF16)
    g[64:128] = 0.0                                  # blocks 2 and 3 of every row are zero
    g = O.round_to(g, O.BF16)
    for elem in (O.E4M3, O.E2M1):
        ref = O.rmsnorm_mx_fwd(x, g, M, N, 1e-5, O.BF16, O.BF16, elem)
        qb = M * N // 2 if elem == O.E2M1 else M * N
        qt = torch.empty(qb, dtype=torch.uint8, device="cuda")
        sc = torch.empty(M * N // 32, dtype=torch.uint8, device="cuda")
        assert R.rmsnorm_quant_fwd(_put(x, O.BF16), None, _put(g, O.BF16), qt, sc, MX_MODES[elem],
                                   None, M, N, 1e-5, O.BF16, O.BF16, _stream()) == 0
        torch.cuda.synchronize()
        s_ = sc.cpu().numpy().reshape(M, N // 32)
        assert np.all(s_[:, 2:4] == 0)
        q = qt.cpu().numpy()
        q = unpack_fp4(q, M, N) if elem == O.E2M1 else q.reshape(M, N)
        check_mx(q, s_, ref, elem)


# ------------------------------------------------------ per-head QK-RMSNorm

def run_qk(T, Hq, Hk, D, xdt, gdt, layout="fused", pad=0, misalign=0, seed=23, eps=1e-6):
    """layout "fused": q, k, v of each token interleaved in one buffer (token
    stride (Hq + 2 Hk) D + pad); "separate": contiguous q and k buffers;
    "q_only": no k. Every element outside the head windows must survive."""
    _log(f"qk T={T} Hq={Hq} Hk={Hk} D={D} x={xdt} g={gdt} layout={layout} pad={pad} "
         f"misalign={misalign}")
    es = 4 if xdt == O.F32 else 2
    gq = G.uniform(seed, G.STREAM_GAMMA, D, 0.5, 1.5, gdt)
    gk = G.uniform(seed + 1, G.STREAM_GAMMA, D, -1.0, 1.0, gdt)
    if layout == "fused":
        S = (Hq + 2 * Hk) * D + pad
        buf = G.normal(seed, G.STREAM_X, 1, T * S, xdt).reshape(-1)
        want, _ = O.rmsnorm_heads_fwd(buf, gq, T, Hq, D, S, eps, xdt, gdt, offset=0)
        want, _ = O.rmsnorm_heads_fwd(want, gk, T, Hk, D, S, eps, xdt, gdt, offset=Hq * D)
        bt = _put(buf, xdt, misalign)
        args = (bt.data_ptr(), bt.data_ptr() + Hq * D * es, T, Hq, Hk, D, S, S)
        mask = np.zeros((T, S), bool)
        mask[:, :(Hq + Hk) * D] = True
        outs = [(bt, buf, want, mask.reshape(-1))]
    else:
        sq, sk = Hq * D + pad, Hk * D + pad
        qb = G.normal(seed, G.STREAM_X, 1, T * sq, xdt).reshape(-1)
        wq, _ = O.rmsnorm_heads_fwd(qb, gq, T, Hq, D, sq, eps, xdt, gdt)
        qt = _put(qb, xdt, misalign)
        mq = np.zeros((T, sq), bool)
        mq[:, :Hq * D] = True
        outs = [(qt, qb, wq, mq.reshape(-1))]
        if layout == "separate":
            kb = G.normal(seed, G.STREAM_R, 1, T * sk, xdt).reshape(-1)
            wk, _ = O.rmsnorm_heads_fwd(kb, gk, T, Hk, D, sk, eps, xdt, gdt)
            kt = _put(kb, xdt, misalign)
            mk = np.zeros((T, sk), bool)
            mk[:, :Hk * D] = True
            outs.append((kt, kb, wk, mk.reshape(-1)))
            args = (qt.data_ptr(), kt.data_ptr(), T, Hq, Hk, D, sq, sk)
        else:
            args = (qt.data_ptr(), None, T, Hq, 0, D, sq, 0)
    q, k, T_, Hq_, Hk_, D_, sq_, sk_ = args
    st = R.rmsnorm_qk_fwd(q, k, _put(gq, gdt), _put(gk, gdt) if k else None, T_, Hq_, Hk_, D_,
                          sq_, sk_, eps, xdt, gdt, _stream())
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    for t, before, want, moved in outs:
        got = to_host(t)
        # Untouched elements bit for bit; normalised ones within the forward's tolerance.
        if xdt == O.F32:
            assert np.array_equal(got.view(np.uint32)[~moved], before.view(np.uint32)[~moved])
        else:
            assert np.array_equal(got[~moved], before[~moved])
        exact = O.decode(want, xdt)
        check_output(got[moved], exact[moved], want[moved], xdt, "qk")


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("D", [64, 96, 128, 256, 512])
def test_qk_fused_buffer(D, pair):
    run_qk(3, 32, 8, D, *pair, seed=1500 + D)
    run_qk(257, 16, 16, D, *pair, seed=1600 + D, pad=8)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_qk_layouts_and_edges(pair):
    run_qk(100, 8, 2, 128, *pair, layout="separate", seed=1701)
    run_qk(100, 8, 0, 128, *pair, layout="q_only", seed=1702)
    run_qk(9, 4, 2, 128, *pair, seed=1703, misalign=1)            # 1-element units
    run_qk(9, 4, 2, 100, *pair, seed=1704, pad=3)                 # ragged head_dim and stride
    run_qk(1, 1, 1, 8, *pair, seed=1705)
    run_qk(5, 2, 1, 8192, *pair, layout="separate", seed=1706)    # longest head vector
    run_qk(2000, 1, 1, 2, *pair, seed=1707)


# ------------------------------------------------------------ LayerNorm

def run_ln(M, N, xdt, gdt, seed=29, eps=1e-5, with_beta=True, stats=True, misalign=0,
           inplace=False, shift=0.0, outlier_every=0, outlier_scale=1.0):
    _log(f"layernorm M={M} N={N} x={xdt} g={gdt} beta={with_beta} stats={stats} "
         f"misalign={misalign} inplace={inplace} shift={shift}")
    x, g, _, _ = _inputs(M, N, xdt, gdt, seed, outlier_every, outlier_scale)
    if shift:
        x = O.round_to(O.decode(x, xdt).reshape(M, N) + shift, xdt)
    b = G.uniform(seed, G.STREAM_DY, N, -1.0, 1.0, gdt) if with_beta else None
    ref = O.layernorm_fwd(x, g, b, M, N, eps, xdt, gdt)
    xt = _put(x, xdt, misalign)
    yt = xt if inplace else _empty(M * N, xdt, misalign)
    mt = torch.full((M,), float("nan"), device="cuda") if stats else None
    rt = torch.full((M,), float("nan"), device="cuda") if stats else None
    st = R.layernorm_fwd(xt, _put(g, gdt), _put(b, gdt) if with_beta else None, yt, mt, rt, M, N,
                         eps, xdt, gdt, _stream())
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    return check_layernorm(to_host(yt), ref, x, g, b, xdt,
                           to_host(mt) if stats else None, to_host(rt) if stats else None)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("N", [1, 7, 8, 64, 264, 384, 520, 640, 768, 1000, 1536, 2048, 3072, 4096,
                               5000, 6144, 6152, 8191, 8192, 8193, 8200, 10240, 12288, 12296, 16384,
                               20000, 24576, 26000, 28672, 32768])
def test_layernorm_sweep(N, pair):
    run_ln(5, N, *pair, seed=1800 + N, with_beta=(N % 2 == 0), stats=(N % 3 != 0))
    run_ln(300, N, *pair, seed=1900 + N)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_layernorm_long_misaligned_inplace_shifted(pair):
    run_ln(3, N_LDS[pair[0]], *pair, seed=2001)
    run_ln(3, N_REREAD[pair[0]], *pair, seed=2002)
    run_ln(7, 4096, *pair, seed=2003, misalign=1)
    run_ln(7, 9000, *pair, seed=2004, misalign=1)
    run_ln(64, 8192, *pair, seed=2005, inplace=True)
    run_ln(300, 32768, *pair, seed=2008, inplace=True)
    run_ln(64, 4096, *pair, seed=2006, shift=30.0)          # mean far from zero
    run_ln(1000, 8192, *pair, seed=2007, outlier_every=13, outlier_scale=300.0)


def test_layernorm_constant_rows_give_beta():
    # var = 0: y = beta exactly up to the tiny centring error, rstd = 1/sqrt(eps).
    M, N = 4, 4096
    x = O.round_to(np.full((M, N), 0.375), O.BF16)
    g = G.uniform(3, G.STREAM_GAMMA, N, 0.5, 1.5, O.BF16)
    b = G.uniform(3, G.STREAM_DY, N, -1.0, 1.0, O.BF16)
    ref = O.layernorm_fwd(x, g, b, M, N, 1e-5, O.BF16, O.BF16)
    yt, mt, rt = _empty(M * N, O.BF16), torch.empty(M, device="cuda"), torch.empty(M, device="cuda")
    assert R.layernorm_fwd(_put(x, O.BF16), _put(g, O.BF16), _put(b, O.BF16), yt, mt, rt, M, N,
                           1e-5, O.BF16, O.BF16, _stream()) == 0
    torch.cuda.synchronize()
    assert np.array_equal(to_host(yt).reshape(M, N), np.broadcast_to(b, (M, N)))
    assert np.all(to_host(mt) == 0.375)
    check_rstd(to_host(rt), ref["rstd_exact"])


def run_ln_bwd(M, N, xdt, gdt, seed=31, misalign=0, alias=None, gpu_stats=False, dbeta=True,
               shift=0.0):
    _log(f"layernorm_bwd M={M} N={N} x={xdt} g={gdt} misalign={misalign} alias={alias} "
         f"gpu_stats={gpu_stats} dbeta={dbeta} shift={shift}")
    x, g, _, dy = _inputs(M, N, xdt, gdt, seed, with_dy=True)
    if shift:
        x = O.round_to(O.decode(x, xdt).reshape(M, N) + shift, xdt)
    xt, gt, dyt = _put(x, xdt, misalign), _put(g, gdt), _put(dy, xdt, misalign)
    if gpu_stats:
        mt, rt = torch.empty(M, device="cuda"), torch.empty(M, device="cuda")
        assert R.layernorm_fwd(xt, gt, None, _empty(M * N, xdt), mt, rt, M, N, 1e-5, xdt, gdt,
                               _stream()) == 0
        torch.cuda.synchronize()
        mean, rstd = to_host(mt), to_host(rt)
    else:
        f = O.layernorm_fwd(x, g, None, M, N, 1e-5, xdt, gdt, want_exact=False)
        mean, rstd = f["mean"], f["rstd"]
        mt, rt = torch.from_numpy(mean.copy()).cuda(), torch.from_numpy(rstd.copy()).cuda()
    ref = O.layernorm_bwd(dy, x, mean, rstd, g, M, N, xdt, gdt)
    dxt = {"dy": dyt, "x": xt}.get(alias) if alias else _empty(M * N, xdt, misalign)
    dgt = torch.full((N,), float("nan"), device="cuda")
    dbt = torch.full((N,), float("nan"), device="cuda") if dbeta else None
    wsb = R.layernorm_bwd_workspace_size(M, N)
    ws = torch.full((max(wsb, 16) // 4,), float("nan"), device="cuda")
    st = R.layernorm_bwd(dyt, xt, mt, rt, gt, dxt, dgt, dbt, ws, wsb, M, N, xdt, gdt, _stream())
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    return check_layernorm_bwd(to_host(dxt), to_host(dgt), to_host(dbt) if dbeta else None, ref,
                               x, dy, g, mean, rstd, xdt)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("N", [1, 7, 8, 64, 344, 360, 384, 680, 720, 768, 1000, 1032, 1280, 1536, 2047, 4096,
                               5000, 8192, 8193, 12288, 16384, 20000, 24576, 24584, 32768])
def test_layernorm_bwd_sweep(N, pair):
    run_ln_bwd(3, N, *pair, seed=2100 + N, dbeta=(N % 2 == 0))
    run_ln_bwd(300, N, *pair, seed=2200 + N)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_layernorm_bwd_edges(pair):
    run_ln_bwd(600, 20000, *pair, seed=2301)                 # two-pass tier, many rows
    run_ln_bwd(5, 9000, *pair, seed=2302, misalign=1)        # scalar two-pass tier
    run_ln_bwd(9, 4096, *pair, seed=2303, misalign=1)
    run_ln_bwd(9, 4096, *pair, seed=2304, alias="dy")
    run_ln_bwd(9, 20000, *pair, seed=2305, alias="x")
    run_ln_bwd(257, 4096, *pair, seed=2306, shift=30.0)
    run_ln_bwd(300, 8192, *pair, seed=2307, gpu_stats=True)


def test_layernorm_bwd_bit_reproducible():
    M, N = 2048, 8192
    x, g, _, dy = _inputs(M, N, O.BF16, O.BF16, 2401, with_dy=True)
    f = O.layernorm_fwd(x, g, None, M, N, 1e-5, O.BF16, O.BF16, want_exact=False)
    xt, gt, dyt = _put(x, O.BF16), _put(g, O.BF16), _put(dy, O.BF16)
    mt, rt = torch.from_numpy(f["mean"]).cuda(), torch.from_numpy(f["rstd"]).cuda()
    wsb = R.layernorm_bwd_workspace_size(M, N)
    outs = []
    for k in range(3):
        dxt, dgt, dbt = _empty(M * N, O.BF16), torch.empty(N, device="cuda"), torch.empty(N, device="cuda")
        ws = torch.full((wsb // 4,), float(k), device="cuda")
        assert R.layernorm_bwd(dyt, xt, mt, rt, gt, dxt, dgt, dbt, ws, wsb, M, N, O.BF16, O.BF16,
                               _stream()) == 0
        torch.cuda.synchronize()
        outs.append([to_host(t) for t in (dxt, dgt, dbt)])
    for o in outs[1:]:
        for a_, b_ in zip(o, outs[0]):
            assert np.array_equal(a_.view(np.uint8), b_.view(np.uint8))


# ----------------------------------------------------------------- backward

def run_bwd(M, N, xdt, gdt, seed=13, misalign=0, alias=None, gpu_rstd=False, eps=1e-5):
    _log(f"bwd M={M} N={N} x={xdt} g={gdt} misalign={misalign} alias={alias} gpu_rstd={gpu_rstd}")
    x, g, _, dy = _inputs(M, N, xdt, gdt, seed, with_dy=True)
    xt, gt, dyt = _put(x, xdt, misalign), _put(g, gdt), _put(dy, xdt, misalign)
    if gpu_rstd:
        rt = torch.empty(M, device="cuda")
        assert R.rmsnorm_fwd(xt, gt, _empty(M * N, xdt), rt, M, N, eps, xdt, gdt, _stream()) == 0
        torch.cuda.synchronize()
        rho = to_host(rt)
    else:
        rho = O.rmsnorm_fwd(x, g, M, N, eps, xdt, gdt, want_exact=False)["rstd"]
        rt = torch.from_numpy(rho.copy()).cuda()
    ref = O.rmsnorm_bwd(dy, x, rho, g, M, N, xdt, gdt)
    dxt = {"dy": dyt, "x": xt}.get(alias) if alias else _empty(M * N, xdt, misalign)
    dgt = torch.full((N,), float("nan"), device="cuda")
    wsb = R.rmsnorm_bwd_workspace_size(M, N)
    ws = torch.full((max(wsb, 16) // 4,), float("nan"), device="cuda")  # contents must not matter
    st = R.rmsnorm_bwd(dyt, xt, rt, gt, dxt, dgt, ws, wsb, M, N, xdt, gdt, _stream())
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    floor_only = check_dx(to_host(dxt).reshape(M, N), ref, x, dy, g, rho, xdt)
    check_dgamma(to_host(dgt), ref)
    return floor_only


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("N", [1, 7, 8, 64, 768, 1000, 1536, 2047, 2560, 3072, 4096, 5000, 8192,
                               8193, 8196, 12288, 16384, 16392, 24576, 24584, 32768, 40000])
def test_bwd_sweep(N, pair):
    # One pass up to 4096 16-byte units (1024 lanes of two, three with
    # prefetch, or four without: 32768 16-bit / 16384 fp32 elements), the
    # two-pass long-row tier beyond.
    run_bwd(3, N, *pair, seed=400 + N)
    run_bwd(70, N, *pair, seed=500 + N)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_bwd_long_rows_misaligned_and_many_rows(pair):
    run_bwd(5, 9000, *pair, seed=601, misalign=1)   # scalar long-row tier
    run_bwd(600, 20000, *pair, seed=602)            # several rows per partition block
    run_bwd(4, 100000, *pair, seed=603, alias="dy")


@pytest.mark.parametrize("M", [1, 31, 33, 100, 255, 256, 257, 1000, 5000])
def test_bwd_row_partitions(M):
    run_bwd(M, 512, O.BF16, O.BF16, seed=M)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("M,N", [(5000, 136), (3000, 192), (2000, 256), (1000, 384), (1200, 512),
                                 (20000, 256), (17000, 1000)])
def test_bwd_narrow_rows_many_per_block(M, N, pair):
    """Narrow rows with M >= 2G: several row groups per stage-1 block, each
    taking several rows of its partial; M > 16384 gives over 256 partial rows
    (stage 2's 64-slice form)."""
    run_bwd(M, N, *pair, seed=M + N)
    run_fused_bwd(M, N, *pair, seed=M + N + 1)
    run_ln_bwd(M, N, *pair, seed=M + N + 2)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_bwd_misaligned_and_aliased(pair):
    run_bwd(9, 4096, *pair, seed=61, misalign=1)
    run_bwd(9, 4096, *pair, seed=62, alias="dy")
    run_bwd(9, 4096, *pair, seed=63, alias="x")


def test_bwd_with_gpu_forward_rstd():
    run_bwd(300, 8192, O.BF16, O.BF16, seed=71, gpu_rstd=True)


def test_bwd_radial_direction():
    # gamma = 1 and dy = 2x: dx = 2 rho (1 - rho^2 ms) x, tiny; checked by the
    # general tolerance (the floor covers the cancellation).
    M, N = 16, 2048
    x = G.normal(5, G.STREAM_X, M, N, O.BF16)
    xd = O.decode(x, O.BF16)
    dy = O.round_to(2.0 * xd, O.BF16)
    g = O.round_to(np.ones(N), O.BF16)
    rho = O.rmsnorm_fwd(x, g, M, N, 1e-5, O.BF16, O.BF16, want_exact=False)["rstd"]
    ref = O.rmsnorm_bwd(dy, x, rho, g, M, N, O.BF16, O.BF16)
    dxt, dgt = _empty(M * N, O.BF16), torch.empty(N, device="cuda")
    wsb = R.rmsnorm_bwd_workspace_size(M, N)
    ws = torch.empty(wsb // 4, device="cuda")
    assert R.rmsnorm_bwd(_put(dy, O.BF16), _put(x, O.BF16), torch.from_numpy(rho).cuda(),
                         _put(g, O.BF16), dxt, dgt, ws, wsb, M, N, O.BF16, O.BF16, _stream()) == 0
    torch.cuda.synchronize()
    check_dx(to_host(dxt).reshape(M, N), ref, x, dy, g, rho, O.BF16)
    check_dgamma(to_host(dgt), ref)


def test_bwd_bit_reproducible():
    M, N = 2048, 8192
    x, g, _, dy = _inputs(M, N, O.BF16, O.BF16, 81, with_dy=True)
    rho = O.rmsnorm_fwd(x, g, M, N, 1e-5, O.BF16, O.BF16, want_exact=False)["rstd"]
    xt, gt, dyt, rt = _put(x, O.BF16), _put(g, O.BF16), _put(dy, O.BF16), torch.from_numpy(rho).cuda()
    wsb = R.rmsnorm_bwd_workspace_size(M, N)
    outs = []
    for k in range(3):
        dxt, dgt = _empty(M * N, O.BF16), torch.empty(N, device="cuda")
        ws = torch.full((wsb // 4,), float(k), device="cuda")
        assert R.rmsnorm_bwd(dyt, xt, rt, gt, dxt, dgt, ws, wsb, M, N, O.BF16, O.BF16,
                             _stream()) == 0
        torch.cuda.synchronize()
        outs.append((to_host(dxt), to_host(dgt)))
    for dx, dg in outs[1:]:
        assert np.array_equal(dx, outs[0][0])
        assert np.array_equal(dg.view(np.uint32), outs[0][1].view(np.uint32))


def test_bwd_empty_is_noop():
    assert R.rmsnorm_bwd(None, None, None, None, None, None, None, 0, 0, 64, O.BF16, O.BF16,
                         _stream()) == 0


# ------------------------------------------------ fused-add backward

def run_fused_bwd(M, N, xdt, gdt, seed=17, misalign=0, alias=None, with_dres=True):
    """h is the fused forward's sum (any array works: the backward only sees h
    and its rstd); dresidual comes from its own generator stream."""
    _log(f"fused_bwd M={M} N={N} x={xdt} g={gdt} misalign={misalign} alias={alias} "
         f"dres={with_dres}")
    h, g, _, dy = _inputs(M, N, xdt, gdt, seed, with_dy=True)
    dres = G.normal(seed, G.STREAM_DRES, M, N, xdt) if with_dres else None
    rho = O.rmsnorm_fwd(h, g, M, N, 1e-5, xdt, gdt, want_exact=False)["rstd"]
    ref = O.rmsnorm_fused_add_bwd(dy, h, rho, g, dres, M, N, xdt, gdt)
    ht, gt, dyt = _put(h, xdt, misalign), _put(g, gdt), _put(dy, xdt, misalign)
    drt = _put(dres, xdt, misalign) if with_dres else None
    rt = torch.from_numpy(rho.copy()).cuda()
    dht = {"dy": dyt, "h": ht, "dres": drt}.get(alias) if alias else _empty(M * N, xdt, misalign)
    dgt = torch.full((N,), float("nan"), device="cuda")
    wsb = R.rmsnorm_bwd_workspace_size(M, N)
    ws = torch.full((max(wsb, 16) // 4,), float("nan"), device="cuda")
    st = R.rmsnorm_fused_add_bwd(dyt, ht, rt, gt, drt, dht, dgt, ws, wsb, M, N, xdt, gdt,
                                 _stream())
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    check_dx(to_host(dht).reshape(M, N), ref, h, dy, g, rho, xdt, dres=dres)
    check_dgamma(to_host(dgt), ref)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("N", [1, 7, 64, 1000, 4096, 5000, 8192, 8193, 12288, 16384, 20000, 24576,
                               32768])
def test_fused_bwd_sweep(N, pair):
    run_fused_bwd(3, N, *pair, seed=700 + N)
    run_fused_bwd(300, N, *pair, seed=800 + N)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_fused_bwd_long_misaligned_aliased(pair):
    run_fused_bwd(600, 20000, *pair, seed=901)                  # two-pass tier, many rows
    run_fused_bwd(5, 9000, *pair, seed=902, misalign=1)         # scalar two-pass tier
    run_fused_bwd(9, 4096, *pair, seed=903, misalign=1)         # scalar on-chip tier
    run_fused_bwd(9, 4096, *pair, seed=904, alias="dres")
    run_fused_bwd(9, 4096, *pair, seed=905, alias="dy")
    run_fused_bwd(9, 20000, *pair, seed=906, alias="h")
    run_fused_bwd(4, 100000, *pair, seed=907, alias="dres")


def test_fused_bwd_without_dresidual_is_plain_backward():
    M, N = 257, 4096
    run_fused_bwd(M, N, O.BF16, O.BF16, seed=911, with_dres=False)
    h, g, _, dy = _inputs(M, N, O.BF16, O.BF16, 912, with_dy=True)
    rho = O.rmsnorm_fwd(h, g, M, N, 1e-5, O.BF16, O.BF16, want_exact=False)["rstd"]
    ht, gt, dyt, rt = _put(h, O.BF16), _put(g, O.BF16), _put(dy, O.BF16), torch.from_numpy(rho).cuda()
    wsb = R.rmsnorm_bwd_workspace_size(M, N)
    ws = torch.empty(wsb // 4, device="cuda")
    outs = []
    for fused in (False, True):
        dxt, dgt = _empty(M * N, O.BF16), torch.empty(N, device="cuda")
        if fused:
            st = R.rmsnorm_fused_add_bwd(dyt, ht, rt, gt, None, dxt, dgt, ws, wsb, M, N, O.BF16,
                                         O.BF16, _stream())
        else:
            st = R.rmsnorm_bwd(dyt, ht, rt, gt, dxt, dgt, ws, wsb, M, N, O.BF16, O.BF16,
                               _stream())
        assert st == 0
        torch.cuda.synchronize()
        outs.append((to_host(dxt), to_host(dgt)))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))


def test_fused_bwd_zero_upstream_passes_dresidual_through():
    # dy = 0: the norm contributes exactly 0, so dh == dresidual bit for bit.
    M, N = 64, 8192
    h, g, _, _ = _inputs(M, N, O.BF16, O.BF16, 921)
    dy = O.round_to(np.zeros((M, N)), O.BF16)
    dres = G.normal(921, G.STREAM_DRES, M, N, O.BF16)
    rho = O.rmsnorm_fwd(h, g, M, N, 1e-5, O.BF16, O.BF16, want_exact=False)["rstd"]
    dht, dgt = _empty(M * N, O.BF16), torch.empty(N, device="cuda")
    wsb = R.rmsnorm_bwd_workspace_size(M, N)
    ws = torch.empty(wsb // 4, device="cuda")
    assert R.rmsnorm_fused_add_bwd(_put(dy, O.BF16), _put(h, O.BF16), torch.from_numpy(rho).cuda(),
                                   _put(g, O.BF16), _put(dres, O.BF16), dht, dgt, ws, wsb, M, N,
                                   O.BF16, O.BF16, _stream()) == 0
    torch.cuda.synchronize()
    assert np.array_equal(to_host(dht).reshape(-1), dres.reshape(-1))
    assert not to_host(dgt).any()


# ------------------------------------------------- the full-size workloads

@pytest.mark.parametrize("w", G.WORKLOADS + G.EXTRA_WORKLOADS,
                         ids=[w.name for w in G.WORKLOADS + G.EXTRA_WORKLOADS])
def test_workload_full_size(w):
    """Each workload at full size, in the launch configuration the benchmark
    times, checked element by element against the oracle."""
    if w.kind == "fwd":
        run_fwd(w.M, w.N, w.x_dt, w.g_dt, eps=w.eps, seed=w.seed, want_rstd=w.store_rstd,
                outlier_every=w.outlier_every, outlier_scale=w.outlier_scale)
    elif w.kind == "fused_add":
        run_fused(w.M, w.N, w.x_dt, w.g_dt, eps=w.eps, seed=w.seed, want_rstd=w.store_rstd)
    elif w.kind == "fused_add_bwd":
        run_fused_bwd(w.M, w.N, w.x_dt, w.g_dt, seed=w.seed)
    elif w.kind == "ln":
        run_ln(w.M, w.N, w.x_dt, w.g_dt, seed=w.seed, eps=w.eps)
    elif w.kind == "ln_bwd":
        run_ln_bwd(w.M, w.N, w.x_dt, w.g_dt, seed=w.seed)
    elif w.kind == "qk":
        run_qk(w.M, w.heads_q, w.heads_k, w.N, w.x_dt, w.g_dt, seed=w.seed, eps=w.eps)
    elif w.kind == "quant" and w.quant_mode >= 3:
        moved = run_mx(w.M, w.N, w.x_dt, w.g_dt, O.E4M3 if w.quant_mode == 3 else O.E2M1,
                       seed=w.seed, fused=w.fused_quant)
        _log(f"blocks on the neighbouring scale code: {moved}")
    elif w.kind == "quant":
        steps = run_quant(w.M, w.N, w.x_dt, w.g_dt, w.quant_mode, seed=w.seed, eps=w.eps,
                          fused=w.fused_quant, want_rstd=w.store_rstd,
                          tensor_scale=w.tensor_scale)
        _log(f"codes one step from the oracle's: {steps}")
    else:
        floor_only = run_bwd(w.M, w.N, w.x_dt, w.g_dt, seed=w.seed, eps=w.eps)
        _log(f"dx elements passing only by the cancellation floor: {floor_only}")


# ------------------------------------------- streams and graph capture

def test_non_default_stream_matches_default():
    M, N = 257, 8192
    x, g, _, _ = _inputs(M, N, O.BF16, O.BF16, 91)
    xt, gt = _put(x, O.BF16), _put(g, O.BF16)
    y0, y1 = _empty(M * N, O.BF16), _empty(M * N, O.BF16)
    assert R.rmsnorm_fwd(xt, gt, y0, None, M, N, 1e-5, O.BF16, O.BF16, _stream()) == 0
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert R.rmsnorm_fwd(xt, gt, y1, None, M, N, 1e-5, O.BF16, O.BF16, side) == 0
    side.synchronize()
    assert np.array_equal(to_host(y0), to_host(y1))


def test_graph_capture_and_replay():
    # The library allocates nothing and issues no memsets, so its launches can
    # be captured. Replays, with eager work in between, must match eager runs.
    M, N = 512, 8192
    x, g, r, dy = _inputs(M, N, O.BF16, O.BF16, 93, with_r=True, with_dy=True)
    xt, gt, dyt = _put(x, O.BF16), _put(g, O.BF16), _put(dy, O.BF16)
    r0 = _put(r, O.BF16)
    rt = r0.clone()
    y, rs, y2 = _empty(M * N, O.BF16), torch.empty(M, device="cuda"), _empty(M * N, O.BF16)
    dx, dg = _empty(M * N, O.BF16), torch.empty(N, device="cuda")
    wsb = R.rmsnorm_bwd_workspace_size(M, N)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")

    def run(stream):
        assert R.rmsnorm_fwd(xt, gt, y, rs, M, N, 1e-5, O.BF16, O.BF16, stream) == 0
        assert R.rmsnorm_fused_add_fwd(xt, rt, gt, y2, None, M, N, 1e-5, O.BF16, O.BF16,
                                       stream) == 0
        assert R.rmsnorm_bwd(dyt, xt, rs, gt, dx, dg, ws, wsb, M, N, O.BF16, O.BF16, stream) == 0

    rt.copy_(r0)
    run(_stream())
    torch.cuda.synchronize()
    want = [to_host(t) for t in (y, rs, rt, y2, dx, dg)]

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run(side)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        rt.copy_(r0)                      # eager work between replays
        for t in (y, rs, y2, dx, dg):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [to_host(t) for t in (y, rs, rt, y2, dx, dg)]
        for a, b in zip(got, want):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), rep


def test_graph_capture_and_replay_of_every_variant():
    # Fused-add backward, fp8 / MX outputs, QK-norm (in place) and LayerNorm
    # forward and backward captured together; every replay must match the
    # eager run bit for bit.
    M, N = 256, 4096
    x, g, r, dy = _inputs(M, N, O.BF16, O.BF16, 95, with_r=True, with_dy=True)
    xt, gt, dyt, rt0 = _put(x, O.BF16), _put(g, O.BF16), _put(dy, O.BF16), _put(r, O.BF16)
    rs = torch.empty(M, device="cuda")
    assert R.rmsnorm_fwd(xt, gt, _empty(M * N, O.BF16), rs, M, N, 1e-5, O.BF16, O.BF16,
                         _stream()) == 0
    dres = _put(G.normal(95, G.STREAM_DRES, M, N, O.BF16), O.BF16)
    dh, dg = _empty(M * N, O.BF16), torch.empty(N, device="cuda")
    ws = torch.empty(R.rmsnorm_bwd_workspace_size(M, N), dtype=torch.uint8, device="cuda")
    q8, s8 = torch.empty(M * N, dtype=torch.uint8, device="cuda"), torch.empty(M, device="cuda")
    q4 = torch.empty(M * N // 2, dtype=torch.uint8, device="cuda")
    s4 = torch.empty(M * N // 32, dtype=torch.uint8, device="cuda")
    qkv0 = _put(G.normal(96, G.STREAM_X, 1, 64 * 48 * 128, O.BF16).reshape(-1), O.BF16)
    qkv = qkv0.clone()
    g128 = _put(G.uniform(96, G.STREAM_GAMMA, 128, 0.5, 1.5, O.BF16), O.BF16)
    beta = _put(G.uniform(95, G.STREAM_DY, N, -1.0, 1.0, O.BF16), O.BF16)
    ly, lm, lr = _empty(M * N, O.BF16), torch.empty(M, device="cuda"), torch.empty(M, device="cuda")
    ldx, ldg, ldb = _empty(M * N, O.BF16), torch.empty(N, device="cuda"), torch.empty(N, device="cuda")
    lws = torch.empty(R.layernorm_bwd_workspace_size(M, N), dtype=torch.uint8,
                      device="cuda")
    outs = (dh, dg, q8, s8, q4, s4, qkv, ly, lm, lr, ldx, ldg, ldb)

    def run(stream):
        assert R.rmsnorm_fused_add_bwd(dyt, xt, rs, gt, dres, dh, dg, ws, ws.numel(), M, N,
                                       O.BF16, O.BF16, stream) == 0
        assert R.rmsnorm_quant_fwd(xt, None, gt, q8, s8, R.RMSN_QUANT_FP8_ROW, None, M, N, 1e-5,
                                   O.BF16, O.BF16, stream) == 0
        assert R.rmsnorm_quant_fwd(xt, None, gt, q4, s4, R.RMSN_QUANT_MXFP4, None, M, N, 1e-5,
                                   O.BF16, O.BF16, stream) == 0
        assert R.rmsnorm_qk_fwd(qkv, qkv.data_ptr() + 32 * 128 * 2, g128, g128, 64, 32, 8, 128,
                                48 * 128, 48 * 128, 1e-6, O.BF16, O.BF16, stream) == 0
        assert R.layernorm_fwd(xt, gt, beta, ly, lm, lr, M, N, 1e-5, O.BF16, O.BF16, stream) == 0
        assert R.layernorm_bwd(dyt, xt, lm, lr, gt, ldx, ldg, ldb, lws, lws.numel(), M, N,
                               O.BF16, O.BF16, stream) == 0

    run(_stream())
    torch.cuda.synchronize()
    want = [t.cpu().clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        qkv.copy_(qkv0)
        with torch.cuda.graph(graph, stream=side):
            run(side)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        qkv.copy_(qkv0)                   # eager work between replays
        for t in outs:
            if t is not qkv:
                t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, w in zip(outs, want):
            assert torch.equal(t.cpu().view(torch.uint8), w.view(torch.uint8)), rep


def test_stale_hip_error_is_not_reported():
    """A failed HIP runtime call made by someone else on this thread (here an
    invalid hipSetDevice) leaves its error behind; the library's next call must
    still return RMSN_OK, with the right output, not that stale error."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    hip.hipSetDevice.restype = ctypes.c_int
    hip.hipGetLastError.restype = ctypes.c_int
    M, N = 33, 4096
    x, g, _, _ = _inputs(M, N, O.BF16, O.BF16, 1901)
    ref = O.rmsnorm_fwd(x, g, M, N, 1e-5, O.BF16, O.BF16)
    xt, gt, yt = _put(x, O.BF16), _put(g, O.BF16), _empty(M * N, O.BF16)
    torch.cuda.synchronize()
    assert hip.hipSetDevice(999) != 0          # fails on the host, launches nothing
    st = R.rmsnorm_fwd(xt, gt, yt, None, M, N, 1e-5, O.BF16, O.BF16, _stream())
    assert st == 0, R.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    check_output(to_host(yt).reshape(M, N), ref["y_exact"], ref["y"], O.BF16, "y")
    assert torch.cuda.current_device() == 0
    hip.hipGetLastError()                       # leave nothing behind for later tests
