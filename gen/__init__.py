"""Seeded synthetic inputs and the workload table.

Shared by the GPU tests, the benchmark and the oracle's tests. Holds no part of
the normalisation's arithmetic: ``gen.c`` draws counter-based SplitMix64 /
Box-Muller numbers and encodes them in a storage format; this module wraps it
and lists the workloads (shapes, dtypes, eps, distributions).

Storage arrays are numpy ``float32`` for fp32 and ``uint16`` bit patterns for
fp16 / bf16. Type codes: 0 = fp32, 1 = fp16, 2 = bf16, 3 = float64 (tests only).
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

F32, F16, BF16, F64 = 0, 1, 2, 3
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}
ESIZE = {F32: 4, F16: 2, BF16: 2}

# Stream ids per operand.
STREAM_X, STREAM_R, STREAM_DY, STREAM_GAMMA, STREAM_DRES = 1, 2, 3, 4, 5

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgen.so")
SRC_PATH = os.path.join(_HERE, "gen.c")
_lib = None


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC",
                    "-shared", "-o", tmp, SRC_PATH, "-lm"], check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    u64, u32, i64, i32, d, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                 ctypes.c_int, ctypes.c_double, ctypes.c_void_p)
    lib.gen_normal.argtypes = [u64, u32, i64, i64, i32, d, i64, vp, i32]
    lib.gen_uniform.argtypes = [u64, u32, i64, d, d, i32, vp, i32]
    lib.gen_bits.argtypes = [u64, u32, i64, vp]
    for fn in (lib.gen_normal, lib.gen_uniform, lib.gen_bits):
        fn.restype = None
    lib.gen_splitmix64.argtypes = [u64]
    lib.gen_splitmix64.restype = u64
    _lib = lib
    return lib


def default_threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


def storage_dtype(dt: int):
    return {F32: np.float32, F64: np.float64}.get(dt, np.uint16)


def normal(seed: int, stream: int, rows: int, cols: int, dt: int, row_scale: float = 1.0,
           scale_every: int = 0, out: np.ndarray | None = None,
           nthreads: int | None = None) -> np.ndarray:
    """[rows, cols] standard normals in storage format dt. Rows whose index is
    a multiple of ``scale_every`` (if > 0) are scaled by ``row_scale``."""
    if out is None:
        out = np.empty((rows, cols), storage_dtype(dt))
    assert out.dtype == storage_dtype(dt) and out.size == rows * cols and out.flags.c_contiguous
    _load().gen_normal(seed, stream, rows, cols, dt, row_scale, scale_every,
                       out.ctypes.data, nthreads or default_threads())
    return out


def uniform(seed: int, stream: int, n: int, lo: float, hi: float, dt: int,
            out: np.ndarray | None = None, nthreads: int | None = None) -> np.ndarray:
    if out is None:
        out = np.empty(n, storage_dtype(dt))
    assert out.dtype == storage_dtype(dt) and out.size == n and out.flags.c_contiguous
    _load().gen_uniform(seed, stream, n, lo, hi, dt, out.ctypes.data, nthreads or default_threads())
    return out


def splitmix64(z: int) -> int:
    return int(_load().gen_splitmix64(z))


def raw_bits(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint64)
    _load().gen_bits(seed, stream, n, out.ctypes.data)
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark / parity workload."""
    name: str
    kind: str            # "fwd", "fused_add", "bwd", "fused_add_bwd", "quant", "qk", "ln",
                         # "ln_bwd"
    M: int
    N: int
    x_dt: int
    g_dt: int
    eps: float
    seed: int
    store_rstd: bool = False
    outlier_every: int = 0      # rows i with i % outlier_every == 0 are scaled
    outlier_scale: float = 1.0
    quant_mode: int = 0         # "quant": 1 = one tensor scale, 2 = per-row scales,
                                #   3 = MXFP8, 4 = MXFP4 (E8M0 per 32 elements)
    fused_quant: bool = False   # "quant": fused residual add first
    tensor_scale: float = 0.0125  # "quant", one tensor scale: |y| > 5.6 saturates
    heads_q: int = 0            # "qk": M tokens of heads_q + heads_k vectors of N = head_dim,
    heads_k: int = 0            #   in a fused q/k/v buffer of (heads_q + 2 heads_k) N per token

    @property
    def esize(self) -> int:
        return ESIZE[self.x_dt]

    @property
    def gsize(self) -> int:
        return ESIZE[self.g_dt]

    def algorithmic_bytes(self) -> int:
        """Each big operand read or written once, plus gamma, rstd, dgamma."""
        r, w = self.read_write_bytes()
        return r + w

    def read_write_bytes(self) -> tuple[int, int]:
        """algorithmic_bytes() split into the bytes read and the bytes written."""
        big = self.M * self.N * self.esize
        g = self.N * self.gsize
        rstd = 4 * self.M if self.store_rstd else 0
        if self.kind == "fwd":
            return big + g, big + rstd
        if self.kind == "fused_add":
            return 2 * big + g, 2 * big + rstd
        if self.kind == "ln_bwd":
            return 2 * big + 8 * self.M + g, big + 8 * self.N
        if self.kind == "ln":
            return big + 2 * g, big + 8 * self.M
        if self.kind == "qk":
            half = self.M * (self.heads_q + self.heads_k) * self.N * self.esize
            return half + 2 * g, half
        if self.kind == "quant":
            n = self.M * self.N
            qbytes = n // 2 if self.quant_mode == 4 else n
            scale_r = 4 if self.quant_mode == 1 else 0
            scale_w = {1: 0, 2: 4 * self.M}.get(self.quant_mode, n // 32)
            fused = big if self.fused_quant else 0
            return big + fused + g + scale_r, fused + qbytes + scale_w + rstd
        if self.kind == "fused_add_bwd":
            return 3 * big + 4 * self.M + g, big + 4 * self.N
        return 2 * big + 4 * self.M + g, big + 4 * self.N

    def _algorithmic_bytes_sum(self) -> int:
        """The same total written out operand by operand (kept to pin the split)."""
        big = self.M * self.N * self.esize
        g = self.N * self.gsize
        if self.kind == "fwd":
            return 2 * big + g + (4 * self.M if self.store_rstd else 0)
        if self.kind == "fused_add":
            return 4 * big + g + (4 * self.M if self.store_rstd else 0)
        if self.kind == "ln_bwd":
            # read x, dy, mean, rstd, gamma; write dx, dgamma, dbeta (fp32)
            return 3 * big + 8 * self.M + g + 8 * self.N
        if self.kind == "ln":
            # read x, gamma, beta; write y, mean, rstd
            return 2 * big + 2 * g + 8 * self.M
        if self.kind == "qk":
            # read and write every q and k head vector (v is never touched)
            return 2 * self.M * (self.heads_q + self.heads_k) * self.N * self.esize + 2 * g
        if self.kind == "quant":
            # read x (and r, writing h), write the fp8 codes (1 byte each),
            # per-row scales (read one scale per tensor).
            n = self.M * self.N
            # q: one byte per element, half for MXFP4; scales: per tensor 4 B
            # read, per row 4 B, MX one E8M0 byte per 32 elements
            qbytes = n // 2 if self.quant_mode == 4 else n
            extra = {1: 4, 2: 4 * self.M}.get(self.quant_mode, n // 32)
            io = big + (2 * big if self.fused_quant else 0) + qbytes
            return io + g + extra + (4 * self.M if self.store_rstd else 0)
        if self.kind == "fused_add_bwd":
            # read h, dy, dresidual, rstd, gamma; write dh, dgamma (fp32)
            return 4 * big + 4 * self.M + g + 4 * self.N
        # backward: read x, dy, rstd, gamma; write dx, dgamma (fp32)
        return 3 * big + 4 * self.M + g + 4 * self.N


# The five workloads: row-wise RMSNorm forward fp32 (short rows), forward bf16
# with rstd (register-resident rows), fused residual add with fp32 gamma,
# backward bf16, and forward fp16 with a row length that is not a multiple of
# the 2048-element tile and with outlier rows.
WORKLOADS = [
    Workload("fwd_f32_m64_n1024", "fwd", 64, 1024, F32, F32, 1e-5, 1001),
    Workload("fwd_bf16_m4096_n8192_rstd", "fwd", 4096, 8192, BF16, BF16, 1e-5, 1002,
             store_rstd=True),
    Workload("fusedadd_bf16_m16384_n4096_gf32", "fused_add", 16384, 4096, BF16, F32, 1e-5, 1003),
    Workload("bwd_bf16_m8192_n8192", "bwd", 8192, 8192, BF16, BF16, 1e-5, 1004),
    Workload("fwd_f16_m32768_n5000_outliers", "fwd", 32768, 5000, F16, F16, 1e-6, 1005,
             outlier_every=97, outlier_scale=200.0),
]
# Workloads of the operations beyond the five: the fused-add backward at the
# backward's shape (h in place of x, plus the residual stream's gradient).
# The quantised forward (fp8 e4m3 output) at the headline shape with per-row
# scales, and after the fused add at the fused workload's shape with one scale.
EXTRA_WORKLOADS = [
    Workload("fusedadd_bwd_bf16_m8192_n8192", "fused_add_bwd", 8192, 8192, BF16, BF16, 1e-5, 1006),
    Workload("fwd_fp8row_bf16_m4096_n8192", "quant", 4096, 8192, BF16, BF16, 1e-5, 1007,
             quant_mode=2),
    Workload("fusedadd_fp8tensor_bf16_m16384_n4096_gf32", "quant", 16384, 4096, BF16, F32, 1e-5,
             1008, quant_mode=1, fused_quant=True),
    Workload("fwd_mxfp8_bf16_m4096_n8192", "quant", 4096, 8192, BF16, BF16, 1e-5, 1012,
             quant_mode=3),
    Workload("fwd_mxfp4_bf16_m4096_n8192", "quant", 4096, 8192, BF16, BF16, 1e-5, 1013,
             quant_mode=4),
    Workload("qknorm_bf16_t16384_hq32_hk8_d128", "qk", 16384, 128, BF16, BF16, 1e-6, 1009,
             heads_q=32, heads_k=8),
    Workload("layernorm_bf16_m4096_n8192", "ln", 4096, 8192, BF16, BF16, 1e-5, 1010),
    Workload("layernorm_bwd_bf16_m8192_n8192", "ln_bwd", 8192, 8192, BF16, BF16, 1e-5, 1011),
    # A few very long rows (the forward's split path: 128 tiles per row).
    Workload("fwd_bf16_m4_n1048576_rstd", "fwd", 4, 1 << 20, BF16, BF16, 1e-5, 1014,
             store_rstd=True),
]
WORKLOADS_BY_NAME = {w.name: w for w in WORKLOADS + EXTRA_WORKLOADS}


def make_inputs(w: Workload, nthreads: int | None = None) -> dict:
    """Host inputs for workload w: x (h for the fused-add backward), gamma, and
    r (fused add), dy (backward) or dy and dres (fused-add backward).
    The backward's saved rstd comes from the oracle forward and is not made here."""
    out = {"x": normal(w.seed, STREAM_X, w.M, w.N, w.x_dt, w.outlier_scale, w.outlier_every,
                       nthreads=nthreads),
           "gamma": uniform(w.seed, STREAM_GAMMA, w.N, 0.5, 1.5, w.g_dt, nthreads=nthreads)}
    if w.kind == "fused_add" or (w.kind == "quant" and w.fused_quant):
        out["r"] = normal(w.seed, STREAM_R, w.M, w.N, w.x_dt, nthreads=nthreads)
    if w.kind == "qk":
        # the whole fused q/k/v buffer; q's gamma is "gamma", k's "gamma_k"
        out["x"] = normal(w.seed, STREAM_X, w.M, (w.heads_q + 2 * w.heads_k) * w.N, w.x_dt,
                          nthreads=nthreads)
        out["gamma_k"] = uniform(w.seed + 1, STREAM_GAMMA, w.N, -1.0, 1.0, w.g_dt,
                                 nthreads=nthreads)
    if w.kind == "ln":
        out["beta"] = uniform(w.seed, STREAM_DY, w.N, -1.0, 1.0, w.g_dt, nthreads=nthreads)
    if w.kind in ("bwd", "fused_add_bwd", "ln_bwd"):
        out["dy"] = normal(w.seed, STREAM_DY, w.M, w.N, w.x_dt, nthreads=nthreads)
    if w.kind == "fused_add_bwd":
        out["dres"] = normal(w.seed, STREAM_DRES, w.M, w.N, w.x_dt, nthreads=nthreads)
    return out
