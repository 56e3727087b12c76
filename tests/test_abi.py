"""C-ABI checks that need no GPU: the library loads, exports every function
include/rmsnorm_mi355x.h declares, and rejects bad arguments on the host before
any HIP call (the addresses used here are never dereferenced)."""

import os
import re

import pytest

import row_wise_normalization_fwd_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")

OK, NULL, SHAPE, DTYPE, WORKSPACE, OVERLAP, ALIGN, EPS = 0, -1, -2, -3, -4, -5, -6, -7
SCRATCH = -9
F32, F16, BF16 = 0, 1, 2

# Fake, well-separated, 256-byte-aligned "device" addresses.
A, B, C, D, E, F, G = (0x10000000 * k for k in range(1, 8))


def _declared_functions():
    names = []
    for fn in sorted(os.listdir(HEADER_DIR)):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(HEADER_DIR, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b((?:rmsnorm|layernorm)_\w+)\s*\(",
                            text, re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return R.load_library()


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted(R.ENTRY_POINTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert callable(getattr(R, name)), name


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        R.load_library(str(tmp_path / "nope.so"))


def test_status_strings(lib):
    for code in (OK, NULL, SHAPE, DTYPE, WORKSPACE, OVERLAP, ALIGN, EPS, -8, SCRATCH, -100):
        s = R.rmsnorm_status_string(code)
        assert s and s != "unknown status"
    assert R.rmsnorm_status_string(12345) == "unknown status"
    assert R.rmsnorm_last_hip_error() == 0


def fwd(x=A, g=B, y=C, rstd=None, M=4, N=64, eps=1e-5, xd=BF16, gd=BF16):
    return R.rmsnorm_fwd(x, g, y, rstd, M, N, eps, xd, gd, None)


def fused(x=A, r=D, g=B, y=C, rstd=None, M=4, N=64, eps=1e-5, xd=BF16, gd=BF16):
    return R.rmsnorm_fused_add_fwd(x, r, g, y, rstd, M, N, eps, xd, gd, None)


def test_forward_validation(lib):
    assert fwd(xd=3) == DTYPE
    assert fwd(xd=BF16, gd=F16) == DTYPE          # gamma must be x dtype or fp32
    assert fwd(xd=F32, gd=BF16) == DTYPE
    assert fwd(M=-1) == SHAPE
    assert fwd(N=0) == SHAPE
    assert fwd(N=2 ** 31) == SHAPE
    assert fwd(eps=-1e-6) == EPS
    assert fwd(eps=float("nan")) == EPS
    assert fwd(eps=float("inf")) == EPS
    assert fwd(M=0, x=None, g=None, y=None) == OK   # empty: no-op
    assert fwd(x=None) == NULL
    assert fwd(g=None) == NULL
    assert fwd(y=None) == NULL
    assert fwd(x=A + 1) == ALIGN
    assert fwd(y=C + 1, xd=F32, gd=F32) == ALIGN
    assert fwd(g=B + 2, xd=F16, gd=F32) == ALIGN
    assert fwd(rstd=E + 2) == ALIGN
    # y may equal x exactly, but not overlap it partially, gamma or rstd.
    assert fwd(y=A + 128) == OVERLAP
    assert fwd(y=B) == OVERLAP
    assert fwd(rstd=A + 16) == OVERLAP
    assert fwd(rstd=C) == OVERLAP
    assert fwd(rstd=B) == OVERLAP


def test_fused_validation(lib):
    assert fused(r=None) == NULL
    assert fused(M=0, r=None) == OK
    assert fused(r=D + 2, xd=F32, gd=F32) == ALIGN
    assert fused(r=A + 128) == OVERLAP        # partial overlap of x and residual
    assert fused(r=C) == OVERLAP              # y must not overlap the residual (h)
    assert fused(r=B) == OVERLAP              # residual written over gamma
    assert fused(rstd=D) == OVERLAP


def bwd(dy=A, x=B, rstd=C, g=D, dx=E, dg=F, ws=G, wsb=None, M=64, N=256, xd=BF16, gd=BF16):
    if wsb is None:
        wsb = R.rmsnorm_bwd_workspace_size(M, N)
    return R.rmsnorm_bwd(dy, x, rstd, g, dx, dg, ws, wsb, M, N, xd, gd, None)


def test_workspace_size():
    # One fp32 partial row per partition block, G = max(min(M, 256),
    # ceil(M / 64)) blocks (every block owns at most 64 rows), rounded up to
    # 256 bytes. The size depends on (M, N) only.
    assert R.rmsnorm_bwd_workspace_size(8192, 8192) == 256 * 8192 * 4
    assert R.rmsnorm_bwd_workspace_size(3, 10) == 256          # 3*10*4 = 120 -> 256
    assert R.rmsnorm_bwd_workspace_size(1000, 64) == 256 * 64 * 4
    assert R.rmsnorm_bwd_workspace_size(200, 64) == 200 * 64 * 4
    assert R.rmsnorm_bwd_workspace_size(16384, 4096) == 256 * 4096 * 4     # 64 rows per block
    assert R.rmsnorm_bwd_workspace_size(16385, 4096) == 257 * 4096 * 4     # one block more
    assert R.rmsnorm_bwd_workspace_size(131072, 1024) == 2048 * 1024 * 4
    assert R.rmsnorm_bwd_workspace_size(0, 64) == 0
    assert R.rmsnorm_bwd_workspace_size(10, 0) == 0
    assert R.rmsnorm_bwd_workspace_size(10, 2**31 - 1) == 0    # beyond RMSN_MAX_N
    # Rows longer than 8192 also hold a 16-byte record per row (the two-pass
    # tier's row dots), each region rounded up to 256 bytes.
    assert R.rmsnorm_bwd_workspace_size(1000, 10000) == 256 * 10000 * 4 + 16128
    assert R.rmsnorm_bwd_workspace_size(3, 8193) == 98_560 + 256   # 98,316 -> 98,560
    assert R.rmsnorm_bwd_workspace_size(3, 8192) == 98_304         # no records at 8192
    # Rows longer than 32768 (always the two-pass tier, column tiles x G
    # workgroups): G = max(min(M, ceil(2^22 / N)), ceil(M / 64)).
    assert R.rmsnorm_bwd_workspace_size(4096, 16384) == 256 * 16384 * 4 + 4096 * 16
    assert R.rmsnorm_bwd_workspace_size(2048, 32768) == 256 * 32768 * 4 + 2048 * 16
    assert R.rmsnorm_bwd_workspace_size(2048, 32769) == 128 * 32769 * 4 + 2048 * 16
    assert R.rmsnorm_bwd_workspace_size(2048, 40000) == 105 * 40000 * 4 + 2048 * 16
    assert R.rmsnorm_bwd_workspace_size(512, 131072) == 32 * 131072 * 4 + 512 * 16
    assert R.rmsnorm_bwd_workspace_size(64, 1 << 20) == 4 * (1 << 20) * 4 + 1024
    assert R.rmsnorm_bwd_workspace_size(3, 1 << 21) == 2 * (1 << 21) * 4 + 256
    assert R.rmsnorm_bwd_workspace_size(100000, 20000) == 125_040_128 + 1_600_000  # 64 rows; 1563 * 20000 * 4 rounded up
    assert R.layernorm_bwd_workspace_size(512, 131072) == 2 * 32 * 131072 * 4 + 512 * 16


def test_max_n():
    # N up to RMSN_MAX_N (2^31 - 2^20) is accepted: the argument checks pass
    # and the call reaches the NULL check; one more is a shape error.
    n_max = 2**31 - 2**20
    assert R.rmsnorm_fwd(None, None, None, None, 1, n_max + 1, 1e-5, BF16, BF16, None) == SHAPE
    assert R.rmsnorm_fwd(None, None, None, None, 1, n_max, 1e-5, BF16, BF16, None) == NULL
    assert R.layernorm_fwd(None, None, None, None, None, None, 1, n_max + 1, 1e-5, BF16, BF16,
                           None) == SHAPE


def test_backward_validation(lib):
    assert bwd(xd=5) == DTYPE
    assert bwd(xd=F32, gd=F16) == DTYPE
    assert bwd(M=-3) == SHAPE
    assert bwd(N=0) == SHAPE
    assert bwd(N=2 ** 31) == SHAPE
    assert bwd(M=0, dy=None, x=None, rstd=None, g=None, dx=None, dg=None, ws=None) == OK
    for k in ("dy", "x", "rstd", "g", "dx", "dg"):
        assert bwd(**{k: None}) == NULL, k
    assert bwd(ws=None) == WORKSPACE
    assert bwd(wsb=R.rmsnorm_bwd_workspace_size(64, 256) - 4) == WORKSPACE
    assert bwd(dy=A + 1) == ALIGN
    assert bwd(ws=G + 8) == ALIGN
    assert bwd(dg=F + 2) == ALIGN
    assert bwd(dx=A + 64) == OVERLAP          # partial overlap with dy
    assert bwd(dx=C) == OVERLAP               # dx over rstd
    assert bwd(dg=A + 4) == OVERLAP
    assert bwd(ws=B + 16) == OVERLAP
    assert bwd(ws=F) == OVERLAP               # workspace over dgamma


def nbwd(dy=A, x=B, rstd=C, g=D, dx=E, dg=F, M=64, N=256, xd=BF16, gd=BF16):
    return R.rmsnorm_bwd_noalloc(dy, x, rstd, g, dx, dg, M, N, xd, gd, None)


def test_noalloc_backward_host_checks(lib):
    """The allocation-free backward rejects bad calls, and shapes whose
    workspace exceeds its fixed buffer, before any HIP call."""
    cap = R.RMSN_NOALLOC_SCRATCH_BYTES
    assert cap == 32 * 1024 * 1024
    assert nbwd(xd=5) == DTYPE
    assert nbwd(xd=F32, gd=F16) == DTYPE
    assert nbwd(M=-1) == SHAPE
    assert nbwd(N=0) == SHAPE
    assert nbwd(M=0, dy=None, x=None, rstd=None, g=None, dx=None, dg=None) == OK
    for k in ("dy", "x", "rstd", "g", "dx", "dg"):
        assert nbwd(**{k: None}) == NULL, k
    # The limit is the workspace rmsnorm_bwd would need: 8192 columns fit up
    # to 65536 rows (1024 partial rows of 32 KiB), one row more does not.
    assert R.rmsnorm_bwd_workspace_size(65536, 8192) == cap
    assert R.rmsnorm_bwd_workspace_size(65537, 8192) > cap
    assert nbwd(M=65537, N=8192) == SCRATCH
    assert nbwd(M=65537, N=8192, dy=None) == SCRATCH   # the size check comes first
    assert nbwd(M=8192, N=65536) == SCRATCH            # 128 x 65536 x 4 B of partials + records
    assert nbwd(M=1, N=2 ** 23) == SCRATCH             # one 32 MiB partial row + a record
    assert R.rmsnorm_last_hip_error() == 0


H = 0x80000000  # an eighth well-separated address, for dresidual


def fbwd(dy=A, h=B, rstd=C, g=D, dres=H, dh=E, dg=F, ws=G, wsb=None, M=64, N=256, xd=BF16,
         gd=BF16):
    if wsb is None:
        wsb = R.rmsnorm_bwd_workspace_size(M, N)
    return R.rmsnorm_fused_add_bwd(dy, h, rstd, g, dres, dh, dg, ws, wsb, M, N, xd, gd, None)


def test_fused_backward_validation(lib):
    assert fbwd(xd=5) == DTYPE
    assert fbwd(M=-1) == SHAPE
    assert fbwd(M=0, dy=None, h=None, rstd=None, g=None, dres=None, dh=None, dg=None,
                ws=None) == OK
    for k in ("dy", "h", "rstd", "g", "dh", "dg"):
        assert fbwd(**{k: None}) == NULL, k
    assert fbwd(ws=None) == WORKSPACE
    assert fbwd(dres=H + 1) == ALIGN
    assert fbwd(dres=H + 2, xd=F32, gd=F32) == ALIGN
    # dh may equal dresidual, dy or h exactly, but not overlap any of them
    # partially, nor the outputs and workspace.
    assert fbwd(dh=H + 64) == OVERLAP
    assert fbwd(dres=F) == OVERLAP             # dresidual over dgamma
    assert fbwd(dres=G + 256) == OVERLAP       # dresidual over the workspace


MODE = -8
QT, QR = 1, 2


def quant(x=A, r=None, g=B, q=C, sc=D, mode=QR, rstd=E, M=64, N=256, eps=1e-5, xd=BF16, gd=BF16):
    return R.rmsnorm_quant_fwd(x, r, g, q, sc, mode, rstd, M, N, eps, xd, gd, None)


def test_quant_validation(lib):
    assert quant(mode=0) == MODE
    assert quant(mode=5) == MODE
    assert quant(xd=F32, gd=F16) == DTYPE
    assert quant(N=0) == SHAPE
    assert quant(eps=float("nan")) == EPS
    assert quant(M=0, x=None, g=None, q=None, sc=None, rstd=None) == OK
    for k in ("x", "g", "q", "sc"):
        assert quant(**{k: None}) == NULL, k
    assert quant(sc=D + 2) == ALIGN
    assert quant(x=A + 1) == ALIGN
    assert quant(r=F + 1) == ALIGN
    assert quant(q=A) == OVERLAP                    # q over x, even exactly
    assert quant(q=A + 64 * 256 * 2 - 1) == OVERLAP
    assert quant(q=B) == OVERLAP                    # q over gamma
    assert quant(sc=C + 16) == OVERLAP              # scale inside q
    assert quant(sc=A + 8) == OVERLAP               # per-row scale written over x
    assert quant(rstd=C + 8) == OVERLAP             # rstd inside q
    assert quant(rstd=D) == OVERLAP                 # rstd over the scale
    assert quant(r=C) == OVERLAP                    # residual over q
    assert quant(r=A + 2) == OVERLAP                # residual partially over x
    assert R.rmsnorm_status_string(MODE) == "unknown quantisation mode"


def qk(q=A, k=A + 4096 * 2, gq=E, gk=F, T=16, Hq=32, Hk=8, D=128, sq=6144, sk=6144, eps=1e-6,
       xd=BF16, gd=BF16):
    # Default layout: a fused QKV buffer at A, q at offset 0 and k right after
    # q's 32 heads, token stride (32 + 8 + 8) * 128 elements.
    return R.rmsnorm_qk_fwd(q, k, gq, gk, T, Hq, Hk, D, sq, sk, eps, xd, gd, None)


def test_qk_validation(lib):
    assert qk(xd=9) == DTYPE
    assert qk(Hq=0) == SHAPE
    assert qk(Hk=-1) == SHAPE
    assert qk(D=0) == SHAPE
    assert qk(D=8193, sq=10 ** 6, sk=10 ** 6) == SHAPE
    assert qk(sq=32 * 128 - 1) == SHAPE
    assert qk(sk=8 * 128 - 1) == SHAPE
    assert qk(T=2 ** 26, Hq=32) == SHAPE                 # tokens * heads >= 2^31
    assert qk(T=2 ** 31 // 40 + 1) == SHAPE             # each tensor fits; q + k rows do not
    assert qk(eps=-1.0) == EPS
    assert qk(T=0, q=None, k=None, gq=None, gk=None) == OK
    assert qk(q=None) == NULL
    assert qk(gq=None) == NULL
    assert qk(k=None) == NULL                            # k_heads > 0 needs k
    assert qk(gk=None) == NULL
    assert qk(q=A + 1) == ALIGN
    assert qk(k=A + 8193) == ALIGN
    assert qk(gq=E + 1) == ALIGN
    assert qk(k=A + 4096 * 2 - 2) == OVERLAP             # k's window starts inside q's
    assert qk(k=A + 6144 * 2 - 8 * 128 * 2 + 2) == OVERLAP   # k's window wraps into the next q
    assert qk(sk=6144 + 8) == OVERLAP                    # strides differ, spans meet
    assert qk(gq=A + 100) == OVERLAP                     # gamma inside the q span
    assert qk(gk=A + 4096 * 2 + 64) == OVERLAP           # k gamma inside the k span


def ln(x=A, g=B, b=C, y=D, mean=E, rstd=F, M=64, N=256, eps=1e-5, xd=BF16, gd=BF16):
    return R.layernorm_fwd(x, g, b, y, mean, rstd, M, N, eps, xd, gd, None)


def test_layernorm_validation(lib):
    assert ln(xd=F32, gd=BF16) == DTYPE
    assert ln(N=0) == SHAPE
    assert ln(eps=float("inf")) == EPS
    assert ln(M=0, x=None, g=None, b=None, y=None, mean=None, rstd=None) == OK
    for k in ("x", "g", "y"):
        assert ln(**{k: None}) == NULL, k
    assert ln(b=C + 1) == ALIGN
    assert ln(mean=E + 2) == ALIGN
    assert ln(y=A + 2) == OVERLAP                   # partial overlap with x
    assert ln(y=C) == OVERLAP                       # y over beta
    assert ln(mean=A) == OVERLAP                    # mean over x
    assert ln(rstd=E + 8) == OVERLAP                # rstd over mean
    assert ln(mean=C + 4) == OVERLAP                # mean over beta


def lnb(dy=A, x=B, mean=C, rstd=C + 4096, g=D, dx=E, dg=F, db=F + 65536, ws=G, wsb=None, M=64,
        N=256, xd=BF16, gd=BF16):
    if wsb is None:
        wsb = R.layernorm_bwd_workspace_size(M, N)
    return R.layernorm_bwd(dy, x, mean, rstd, g, dx, dg, db, ws, wsb, M, N, xd, gd, None)


def test_layernorm_workspace_size():
    # Two fp32 partial arrays of G rows (as for RMSNorm); rows longer than
    # 8192 add a 16-byte record per row.
    assert R.layernorm_bwd_workspace_size(8192, 8192) == 2 * 256 * 8192 * 4
    assert R.layernorm_bwd_workspace_size(3, 10) == 2 * 256
    assert R.layernorm_bwd_workspace_size(1000, 10000) == 2 * 256 * 10000 * 4 + 16128
    assert R.layernorm_bwd_workspace_size(131072, 1024) == 2 * 2048 * 1024 * 4
    # LayerNorm partitions as RMSNorm does: 256 partial rows up to 32768
    # elements, ceil(2^22 / N) beyond (128 at 32776).
    assert R.layernorm_bwd_workspace_size(1024, 24584) == 2 * 256 * 24584 * 4 + 1024 * 16
    assert R.layernorm_bwd_workspace_size(1024, 32768) == 2 * 256 * 32768 * 4 + 1024 * 16
    assert R.layernorm_bwd_workspace_size(1024, 32776) == 2 * (128 * 32776 * 4) + 1024 * 16
    assert R.rmsnorm_bwd_workspace_size(1024, 32768) == 256 * 32768 * 4 + 1024 * 16
    assert R.layernorm_bwd_workspace_size(0, 10) == 0


def test_layernorm_backward_validation(lib):
    assert lnb(xd=4) == DTYPE
    assert lnb(M=-1) == SHAPE
    assert lnb(M=0, dy=None, x=None, mean=None, rstd=None, g=None, dx=None, dg=None, db=None,
               ws=None) == OK
    for k in ("dy", "x", "mean", "rstd", "g", "dx", "dg"):
        assert lnb(**{k: None}) == NULL, k
    assert lnb(ws=None) == WORKSPACE
    assert lnb(wsb=R.layernorm_bwd_workspace_size(64, 256) - 1) == WORKSPACE
    assert lnb(mean=C + 2) == ALIGN
    assert lnb(db=F + 65536 + 2) == ALIGN
    assert lnb(dx=A + 64) == OVERLAP
    assert lnb(dx=C) == OVERLAP                      # dx over mean
    assert lnb(db=F + 8) == OVERLAP                  # dbeta over dgamma
    assert lnb(db=G + 16) == OVERLAP                 # dbeta in the workspace
    assert lnb(ws=C) == OVERLAP                      # workspace over the statistics


MX8, MX4 = 3, 4


def test_mx_quant_validation(lib):
    assert quant(mode=MX8, N=100) == SHAPE            # N % 32 != 0
    assert quant(mode=MX4, N=33) == SHAPE
    assert quant(mode=MX8, x=A + 2) == ALIGN          # rows must be 16-byte aligned
    assert quant(mode=MX4, g=B + 8) == ALIGN
    assert quant(mode=MX8, r=F + 4) == ALIGN
    assert quant(mode=MX8, q=C + 4) == ALIGN          # 8-byte fp8 units (bf16 input)
    assert quant(mode=MX4, q=C + 2) == ALIGN          # 4-byte fp4 units
    assert quant(mode=MX4, sc=C + 64 * 128 - 1) == OVERLAP   # scale codes over q's last byte
    assert quant(mode=MX8, sc=A + 8) == OVERLAP       # codes written over x


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError, match="host tensor"):
        R._p(torch.zeros(2))
    x, g = torch.zeros(4, 8), torch.ones(8)
    with pytest.raises(ValueError, match="same GPU"):
        R.fwd(x, g)
    with pytest.raises(ValueError, match="same GPU"):
        R.layernorm(x, g)
    with pytest.raises(ValueError, match="same GPU"):
        R.bwd(torch.zeros(4, 8), x, torch.zeros(4), g)


def test_conveniences_check_sizes_dtypes_and_layout_before_any_call():
    """Every tensor a convenience passes on is checked for its element count,
    dtype and contiguity first (a short out, rstd or dgamma would be written
    past its end by the kernels; a strided one would be read wrongly)."""
    torch = pytest.importorskip("torch")
    x, g = torch.zeros(4, 8), torch.ones(8)
    with pytest.raises(ValueError, match="out: 24 elements, expected 32"):
        R.fwd(x, g, out=torch.zeros(3, 8))
    with pytest.raises(ValueError, match="rstd: 3 elements, expected 4"):
        R.fwd(x, g, want_rstd=True, rstd=torch.zeros(3))
    with pytest.raises(TypeError, match="rstd: dtype"):
        R.fwd(x, g, want_rstd=True, rstd=torch.zeros(4, dtype=torch.float64))
    with pytest.raises(ValueError, match="gamma: must be contiguous"):
        R.fwd(x, torch.ones(16)[::2])
    with pytest.raises(ValueError, match="dgamma: 7 elements"):
        R.bwd(torch.zeros(4, 8), x, torch.zeros(4), g, dgamma=torch.zeros(7))
    with pytest.raises(ValueError, match="dy: must be contiguous"):
        R.bwd(torch.zeros(8, 4).t(), x, torch.zeros(4), g)
    with pytest.raises(ValueError, match="mean: 5 elements"):
        R.layernorm_backward(torch.zeros(4, 8), x, torch.zeros(5), torch.zeros(4), g)
    with pytest.raises(ValueError, match="beta: 9 elements"):
        R.layernorm(x, g, torch.zeros(9))
    with pytest.raises(ValueError, match="residual: must be contiguous"):
        R.fused_add_fwd(x, torch.zeros(8, 4).t(), g)
    with pytest.raises(ValueError, match="scale: 2 elements"):
        R.quant_fwd(x, g, scale=torch.ones(2))
    q = torch.zeros(2, 3, 8)
    with pytest.raises(ValueError, match="k_gamma is required"):
        R.qk_fwd(q, torch.zeros(2, 1, 8), torch.ones(8))
    with pytest.raises(ValueError, match="same GPU"):
        R.qk_fwd(q, None, torch.ones(8))


def test_workspace_bytes_count_the_element_size():
    torch = pytest.importorskip("torch")
    assert R._nbytes(torch.empty(10, dtype=torch.float32)) == 40
    assert R._nbytes(torch.empty(10, dtype=torch.uint8)) == 10


def test_copy16_calibration_library_checks_arguments_on_the_host():
    """The benchmark's copy kernel library (not part of the normalisation ABI)
    loads and rejects bad arguments before any HIP call."""
    import ctypes
    path = os.path.join(ROOT, "row_wise_normalization_fwd_amd", "librmsn_copy16.so")
    if not os.path.exists(path):
        pytest.skip("librmsn_copy16.so not built")
    lib = ctypes.CDLL(path)
    f = lib.rmsn_calib_copy16
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(A, B, 0, None) == 0              # nothing to copy: no launch
    assert f(A, B, 15, None) == -1            # not a multiple of 16
    assert f(A + 8, B, 16, None) == -1        # misaligned source
    assert f(A, A + 16, 64, None) == -1       # overlapping
    assert f(None, B, 16, None) == -1


def test_stream_calibration_checks_arguments_on_the_host():
    """The benchmark's backward-ceiling stream (dst = a ^ b (^ c)) rejects bad
    arguments before any HIP call."""
    import ctypes
    path = os.path.join(ROOT, "row_wise_normalization_fwd_amd", "librmsn_copy16.so")
    if not os.path.exists(path):
        pytest.skip("librmsn_copy16.so not built")
    lib = ctypes.CDLL(path)
    f = lib.rmsn_calib_stream
    vp = ctypes.c_void_p
    f.argtypes = [vp, vp, vp, vp, ctypes.c_int64, vp]
    f.restype = ctypes.c_int
    assert f(A, B, None, F, 0, None) == 0        # nothing to do: no launch
    assert f(A, B, E, F, 0, None) == 0
    assert f(A, B, None, F, 24, None) == -1      # not a multiple of 16
    assert f(A + 8, B, None, F, 16, None) == -1  # misaligned input
    assert f(A, B, E + 4, F, 16, None) == -1     # misaligned third input
    assert f(A, B, None, F + 8, 16, None) == -1  # misaligned output
    assert f(A, B, None, A + 16, 64, None) == -1  # output overlaps an input
    assert f(A, B, F, F, 64, None) == -1         # output is the third input
    assert f(None, B, None, F, 16, None) == -1
    assert f(A, None, None, F, 16, None) == -1
    assert f(A, B, None, None, 16, None) == -1


def test_mix_calibration_checks_arguments_on_the_host():
    """The benchmark's read/write mix stream (A reads to B writes of 16 bytes
    per unit) rejects bad arguments before any HIP call."""
    import ctypes
    path = os.path.join(ROOT, "row_wise_normalization_fwd_amd", "librmsn_copy16.so")
    if not os.path.exists(path):
        pytest.skip("librmsn_copy16.so not built")
    lib = ctypes.CDLL(path)
    f = lib.rmsn_calib_mix
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    f.argtypes = [vp, i32, vp, i32, ctypes.c_int64, vp, vp]
    f.restype = ctypes.c_int
    assert f(A, 2, B, 1, 0, G, None) == 0        # nothing to do: no launch
    assert f(None, 0, B, 1, 0, G, None) == 0     # write-only, empty
    assert f(A, 1, None, 0, 0, G, None) == 0     # read-only, empty
    assert f(A, 0, B, 0, 16, G, None) == -1      # neither reads nor writes
    assert f(A, 5, B, 1, 16, G, None) == -1      # too many planes
    assert f(A, 1, B, -1, 16, G, None) == -1
    assert f(A, 1, B, 1, -1, G, None) == -1
    assert f(None, 1, B, 1, 16, G, None) == -1   # reads need a source
    assert f(A, 1, None, 1, 16, G, None) == -1   # writes need a destination
    assert f(A + 8, 1, B, 1, 16, G, None) == -1  # misaligned
    assert f(A, 1, B + 4, 1, 16, G, None) == -1
    assert f(A, 1, B, 1, 16, None, None) == -1   # no sink
    assert f(A, 1, B, 1, 16, G + 8, None) == -1
    assert f(A, 2, A + 16, 1, 64, G, None) == -1  # output overlaps the source
    assert f(A, 1, B, 1, 64, B + 512, None) == -1  # sink inside the output
    assert f(A, 1, B, 1, 1 << 40, G, None) == -1  # absurd size


def test_bench_mix_ratio_and_byte_split():
    """bench.py's ceiling streams take the offered read:write ratio nearest
    each workload's, and the workloads' read / write split adds up to their
    algorithmic bytes."""
    import sys
    sys.path.insert(0, ROOT)
    import bench
    import gen
    assert bench.mix_ratio(100, 0) == (1, 0)
    assert bench.mix_ratio(0, 100) == (0, 1)
    want = {"fwd_bf16_m4096_n8192_rstd": (1, 1), "bwd_bf16_m8192_n8192": (2, 1),
            "fusedadd_bwd_bf16_m8192_n8192": (3, 1), "fwd_fp8row_bf16_m4096_n8192": (2, 1),
            "fwd_mxfp8_bf16_m4096_n8192": (2, 1), "fwd_mxfp4_bf16_m4096_n8192": (4, 1),
            "fusedadd_fp8tensor_bf16_m16384_n4096_gf32": (4, 3),
            "layernorm_bwd_bf16_m8192_n8192": (2, 1), "fusedadd_bf16_m16384_n4096_gf32": (1, 1)}
    for w in gen.WORKLOADS + gen.EXTRA_WORKLOADS:
        r, wr = w.read_write_bytes()
        assert r + wr == w.algorithmic_bytes() == w._algorithmic_bytes_sum(), w.name
        if w.name in want:
            assert bench.mix_ratio(r, wr) == want[w.name], w.name


def test_bench_busy_monitor(tmp_path):
    """bench.py's idle check: readings above the threshold mark a sample busy,
    an unreadable or missing counter never does, and the log keeps the
    readings."""
    import sys
    sys.path.insert(0, ROOT)
    import bench
    f = tmp_path / "gpu_busy_percent"
    synced = []
    m = bench.BusyMonitor(threshold_pct=10, path=str(f), sync=lambda: synced.append(1))
    f.write_text("3\n")
    assert m.idle("quiet", settle_s=0.0)
    f.write_text("55\n")
    assert not m.idle("busy", settle_s=0.0)
    f.write_text("10\n")
    assert m.idle("at the threshold", settle_s=0.0)
    assert len(synced) == 3
    s = m.summary()
    assert s["samples"] == 3 and s["busy_samples"] == 1 and s["threshold_pct"] == 10
    assert s["log"][1] == {"at": "busy", "busy_pct": [55] * 5, "busy": True}
    f.write_text("not a number")
    assert m.sample() == [] and m.idle("garbled", settle_s=0.0)
    none = bench.BusyMonitor(path=str(tmp_path / "missing"), sync=None)
    assert none.sample() == [] and none.idle("no counter", settle_s=0.0)


def test_bench_parity_check_plumbing():
    """bench.py's sampled parity check accepts outputs equal to the oracle's
    and rejects one corrupted element, for a forward, a quantised forward
    and a backward workload shape (small sizes, CPU only)."""
    import dataclasses
    import sys
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    import gen
    import oracle as O
    base = gen.WORKLOADS_BY_NAME["fwd_bf16_m4096_n8192_rstd"]
    w = dataclasses.replace(base, M=100, N=256)
    h = gen.make_inputs(w)
    ref = O.rmsnorm_fwd(h["x"], h["gamma"], w.M, w.N, w.eps, w.x_dt, w.g_dt)
    outs = {"y": ref["y"].copy(), "rstd": ref["rstd"].copy()}
    p = bench.parity_check(w, outs, h)
    assert p["ok"] and p["rows_checked"] == 64 and p["of"] == 100, p
    outs["y"].reshape(100, 256)[99, 7] ^= 0x0100       # a few ulp off in the last row
    assert not bench.parity_check(w, outs, h)["ok"]
    wq = dataclasses.replace(gen.WORKLOADS_BY_NAME["fwd_mxfp4_bf16_m4096_n8192"], M=20, N=256)
    hq = gen.make_inputs(wq)
    rq = O.rmsnorm_mx_fwd(hq["x"], hq["gamma"], 20, 256, wq.eps, wq.x_dt, wq.g_dt, O.E2M1)
    packed = (rq["q"][:, 0::2] | (rq["q"][:, 1::2] << 4)).astype(np.uint8)
    assert bench.parity_check(wq, {"q": packed.reshape(-1), "scale": rq["scale"].reshape(-1)},
                              hq)["ok"]
    wb = dataclasses.replace(gen.WORKLOADS_BY_NAME["bwd_bf16_m8192_n8192"], M=70, N=128)
    hb = gen.make_inputs(wb)
    rho = O.rmsnorm_fwd(hb["x"], hb["gamma"], 70, 128, wb.eps, wb.x_dt, wb.g_dt)["rstd"]
    rb = O.rmsnorm_bwd(hb["dy"], hb["x"], rho, hb["gamma"], 70, 128, wb.x_dt, wb.g_dt)
    ob = {"dx": rb["dx"].copy(), "rstd": rho}
    assert bench.parity_check(wb, ob, hb)["ok"]
    ob["dx"].reshape(70, 128)[0, 0] ^= 0x4000         # a wildly wrong element
    assert not bench.parity_check(wb, ob, hb)["ok"]


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU; asking for more exits with a message before
    touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_kernel_hash_ignores_comments_and_layout_only():
    """The bench keys stored traffic figures to the kernel sources' code:
    comments and whitespace do not change the key, code and literals do."""
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    base = 'int f(int a) {\n  return a + 1;  // add\n}\nconst char* s = "x // y";\n'
    same = '/* doc */ int f(int a)\n{ return a + 1; }\n// end\nconst char* s = "x // y";'
    assert bench._code_tokens(base) == bench._code_tokens(same)
    for changed in (base.replace("+ 1", "+ 2"), base.replace('"x // y"', '"x / y"')):
        assert bench._code_tokens(base) != bench._code_tokens(changed)
    assert re.fullmatch(r"[0-9a-f]{16}", bench.kernel_source_hash())
