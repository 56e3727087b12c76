#!/usr/bin/env python3
"""Benchmark of the row-wise RMSNorm library on one MI355X.

A step is one call of the hot path on one batch: by default the bf16 forward
over a [4096, 8192] batch that also writes the fp32 per-row rstd. Inputs are
seeded synthetic data resident in HBM before timing starts. To measure HBM
rather than the 256 MB Infinity Cache, consecutive steps rotate over R replicas
of every operand (R * footprint >= --rotate-bytes, 1 GiB by default); the R
replicas of an operand are the rows of one [R, numel] allocation.

Timing: W untimed warm-up steps, then exactly K steps between two HIP events
recorded on the stream the kernels run on (torch's current stream), with a
device synchronisation on both sides. value = algorithmic bytes per step
(each big operand read or written once, plus gamma and rstd) / time per step.

Also reported, in the same JSON line:
  roofline      HBM-bound roofline of the step's kernel: achieved GB/s vs the
                8 TB/s peak, and the measured HBM traffic per launch from the
                committed rocprofv3 counter summary when it matches the
                current kernel sources (else null);
  cpu_baseline  the fp64 oracle, single-threaded, on the host, over repeated
                full passes of the same batch for about --cpu-seconds;
  workloads     the other four workloads (fp32 short rows, fused residual add,
                backward, fp16 ragged rows) and the fused-add backward, timed
                the same way, the fp8-output forward (per-row scales at the
                headline shape; one scale after the fused add), MXFP8 and
                MXFP4 outputs at the headline shape, the per-head
                QK-norm on a fused q/k/v buffer, LayerNorm at the headline
                shape and the LayerNorm backward at the backward's shape,
                and 4 rows of 2^20 bf16 elements (the split path); each
                backward also carries stream_gbps, a reduction-free stream
                with its reads and writes (2 or 3 inputs per output), and
                value_over_stream; the launch-bound fp32 64 x 1024 case
                also carries `graph`, the same call replayed 100 at a time
                from a captured HIP graph (no host launch per call);
  hot_cache_gbps  the same step without rotation (inputs in the Infinity
                Cache): context, never the value;
  graph         the same step, 100 calls over the rotation replicas captured in
                one HIP graph and replayed: the step without host launch gaps;
  rounds        five more timing rounds of the step (>= 20 ms each after a
                50 ms warm-up, 1 s cool-down): median / min / mean us, spread,
                and how many rounds were timed again because the device was
                busy before or after them (idle_check);
  ceiling       the matching stream: a 16-byte non-temporal kernel moving the
                step's read and write bytes in (nearly) its read:write ratio
                (librmsn_copy16.so rmsn_calib_mix), rotated the same way, and
                frac_of_ceiling = value / its GB/s; every large workload in
                `workloads` carries its own ceiling and frac_of_ceiling, and
                its own cpu_baseline (one oracle pass; best of three for the
                64 x 1024 case);
  calibration   plain copies of the step's byte count: torch's device-to-device
                copy, and a 16-byte non-temporal copy kernel
                (librmsn_copy16.so, the practical ceiling for equal read and
                write bytes), with value / copy16; read-only and write-only
                16-byte streams of the step's read and write bytes;
  parity        (with the CPU leg) the timed configuration's outputs, recomputed
                from pristine inputs on replica 0, against the fp64 oracle on
                64 rows spread over the batch, with the GPU tests'
                tolerances; every workload carries its own;
  idle_check    gpu_busy_percent of this device (sysfs, matched by PCI
                address) sampled while this process has nothing in flight:
                before and after the main timed region, each round and each
                other workload.

Modes that do not time anything: --collect-profiles DIR runs the rocprofv3
passes behind profiles/ as child processes, --reduce-profiles DIR writes
profiles/ from their output.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0
HEADLINE = "fwd_bf16_m4096_n8192_rstd"
# The kernel that dominates each workload's step, as the dispatcher picks it.
DOMINANT_KERNEL = {
    "fwd_f32_m64_n1024": "fwd_reg_kernel",
    "fwd_bf16_m4096_n8192_rstd": "fwd_pp_kernel",
    "fusedadd_bf16_m16384_n4096_gf32": "fwd_reg_kernel",
    "bwd_bf16_m8192_n8192": "bwd_stage1_kernel",
    "fwd_f16_m32768_n5000_outliers": "fwd_reg_kernel",
    "fusedadd_bwd_bf16_m8192_n8192": "bwd_stage1_kernel",
    "fwd_fp8row_bf16_m4096_n8192": "fwd_pp_kernel",
    "fusedadd_fp8tensor_bf16_m16384_n4096_gf32": "fwd_reg_kernel",
    "fwd_mxfp8_bf16_m4096_n8192": "fwd_pp_kernel",
    "fwd_mxfp4_bf16_m4096_n8192": "fwd_pp_kernel",
    "qknorm_bf16_t16384_hq32_hk8_d128": "qk_norm_kernel",
    "layernorm_bf16_m4096_n8192": "fwd_pp_kernel",
    "layernorm_bwd_bf16_m8192_n8192": "bwd_stage1_kernel",
    "fwd_bf16_m4_n1048576_rstd": "fwd_split_apply_kernel",
}
DT_NAMES = {0: "f32", 1: "f16", 2: "bf16"}


def rows_of(w) -> int:
    """Normalised rows per step (head vectors for the QK-norm)."""
    return w.M * (w.heads_q + w.heads_k) if w.kind == "qk" else w.M


def _code_tokens(text: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed, so that
    editing a comment does not void traffic figures taken on the same code.
    String and character literals are kept verbatim."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the kernel and ABI sources' code (comments and layout ignored)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "row_wise_normalization_fwd_amd", "csrc")
    for p in sorted(glob.glob(os.path.join(csrc, "*"))):
        with open(p, encoding="utf-8") as fh:
            code = _code_tokens(fh.read())
        h.update(os.path.basename(p).encode() + b"\0" + code.encode())
    return h.hexdigest()[:16]


class Runner:
    """Device replicas of one workload's operands and a launcher for step i."""

    def __init__(self, w, rotate_bytes: float, host_inputs: dict):
        import torch

        import row_wise_normalization_fwd_amd as R

        self.w = w
        self.R = R
        dev = torch.device("cuda:0")
        tdt = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}
        M, N = w.M, w.N

        def dev_copy(a, dt):
            import numpy as np
            if dt == 0:
                t = torch.from_numpy(a.reshape(-1))
            else:
                t = torch.from_numpy(a.reshape(-1).view(np.int16)).view(tdt[dt])
            return t.to(dev)

        big = M * N * w.esize
        per_replica = {"fwd": 2 * big, "fused_add": 3 * big, "bwd": 3 * big,
                       "fused_add_bwd": 4 * big,
                       "quant": (2 if w.fused_quant else 1) * big + M * N,  # q <= M N bytes
                       "qk": M * (w.heads_q + 2 * w.heads_k) * N * w.esize,
                       "ln": 2 * big, "ln_bwd": 3 * big}[w.kind]
        self.replicas = max(1, int(-(-rotate_bytes // per_replica))) if rotate_bytes > 0 else 1
        x0 = dev_copy(host_inputs["x"], w.x_dt)
        g = dev_copy(host_inputs["gamma"], w.g_dt)
        self.gamma = g
        self.sets = []
        stream = torch.cuda.current_stream(dev)
        self.stream_handle = stream.cuda_stream
        rstd_bwd = mean_bwd = None
        backward = w.kind in ("bwd", "fused_add_bwd", "ln_bwd")
        if backward:
            # The saved statistics come from this library's own forward pass.
            rstd_bwd = torch.empty(M, dtype=torch.float32, device=dev)
            tmp = torch.empty_like(x0)
            if w.kind == "ln_bwd":
                mean_bwd = torch.empty(M, dtype=torch.float32, device=dev)
                st = R.layernorm_fwd(x0, g, None, tmp, mean_bwd, rstd_bwd, M, N, w.eps, w.x_dt,
                                     w.g_dt, stream)
                self.ws_bytes = R.layernorm_bwd_workspace_size(M, N)
            else:
                st = R.rmsnorm_fwd(x0, g, tmp, rstd_bwd, M, N, w.eps, w.x_dt, w.g_dt, stream)
                self.ws_bytes = R.rmsnorm_bwd_workspace_size(M, N)
            assert st == 0, R.rmsnorm_status_string(st)
            del tmp
            dy0 = dev_copy(host_inputs["dy"], w.x_dt)
        if w.kind == "fused_add_bwd":
            dres0 = dev_copy(host_inputs["dres"], w.x_dt)
        if w.kind == "fused_add" or (w.kind == "quant" and w.fused_quant):
            r0 = dev_copy(host_inputs["r"], w.x_dt)
        if w.kind == "ln":
            self.beta = dev_copy(host_inputs["beta"], w.g_dt)
        if w.kind == "qk":
            self.gamma_k = dev_copy(host_inputs["gamma_k"], w.g_dt)
            self.qkv_stride = (w.heads_q + 2 * w.heads_k) * N
        if w.kind == "quant" and w.quant_mode == 1:
            self.tensor_scale = torch.tensor([w.tensor_scale], dtype=torch.float32, device=dev)
        # Each operand's R replicas are rows of one [R, numel] allocation, the
        # layout of a batched tensor, so every stream is one contiguous range.
        nrep = self.replicas

        def rep_copy(src):
            block = torch.empty((nrep, src.numel()), dtype=src.dtype, device=dev)
            block.copy_(src.reshape(1, -1).expand(nrep, -1))
            return list(block.unbind(0))

        def rep_empty(numel, dtype):
            return list(torch.empty((nrep, numel), dtype=dtype, device=dev).unbind(0))

        def rep_opt(flag, numel, dtype):
            return rep_empty(numel, dtype) if flag else [None] * nrep

        f32, u8 = torch.float32, torch.uint8
        cols = {"x": rep_copy(x0)}
        if w.kind in ("fwd", "fused_add"):
            cols["y"] = rep_empty(M * N, x0.dtype)
            cols["rstd"] = rep_opt(w.store_rstd, M, f32)
            if w.kind == "fused_add":
                cols["r"] = rep_copy(r0)
        elif w.kind == "qk":
            pass  # in place on the fused q/k/v buffer "x"
        elif w.kind == "ln":
            cols["y"] = rep_empty(M * N, x0.dtype)
            cols["mean"] = rep_empty(M, f32)
            cols["rstd"] = rep_empty(M, f32)
        elif w.kind == "quant":
            cols["r"] = rep_copy(r0) if w.fused_quant else [None] * nrep
            cols["q"] = rep_empty(M * N // 2 if w.quant_mode == 4 else M * N, u8)
            if w.quant_mode == 1:
                cols["scale"] = [self.tensor_scale] * nrep
            elif w.quant_mode == 2:
                cols["scale"] = rep_empty(M, f32)
            else:  # MX: E8M0 codes per 32 elements
                cols["scale"] = rep_empty(M * N // 32, u8)
            cols["rstd"] = rep_opt(w.store_rstd, M, f32)
        else:
            cols["dy"] = rep_copy(dy0)
            cols["rstd"] = [rstd_bwd] * nrep
            cols["dx"] = rep_empty(M * N, x0.dtype)
            cols["dgamma"] = rep_empty(N, f32)
            cols["ws"] = rep_empty(max(self.ws_bytes, 16), u8)
            if w.kind == "fused_add_bwd":
                cols["dres"] = rep_copy(dres0)
            if w.kind == "ln_bwd":
                cols["mean"] = [mean_bwd] * nrep
                cols["dbeta"] = rep_empty(N, f32)
        for i in range(nrep):
            self.sets.append({k: v[i] for k, v in cols.items()})
        torch.cuda.synchronize()
        # Pre-marshalled integer arguments keep the host launch path short.
        self.calls = []
        lib = R.load_library()
        for s in self.sets:
            p = {k: (v.data_ptr() if v is not None else None) for k, v in s.items()}
            if w.kind == "fwd":
                args = (p["x"], g.data_ptr(), p["y"], p["rstd"], M, N, w.eps, w.x_dt, w.g_dt,
                        self.stream_handle)
                self.calls.append((lib.rmsnorm_fwd, args))
            elif w.kind == "fused_add":
                args = (p["x"], p["r"], g.data_ptr(), p["y"], p["rstd"], M, N, w.eps, w.x_dt,
                        w.g_dt, self.stream_handle)
                self.calls.append((lib.rmsnorm_fused_add_fwd, args))
            elif w.kind == "ln":
                args = (p["x"], g.data_ptr(), self.beta.data_ptr(), p["y"], p["mean"], p["rstd"],
                        M, N, w.eps, w.x_dt, w.g_dt, self.stream_handle)
                self.calls.append((lib.layernorm_fwd, args))
            elif w.kind == "qk":
                args = (p["x"], p["x"] + w.heads_q * N * w.esize, g.data_ptr(),
                        self.gamma_k.data_ptr(), M, w.heads_q, w.heads_k, N, self.qkv_stride,
                        self.qkv_stride, w.eps, w.x_dt, w.g_dt, self.stream_handle)
                self.calls.append((lib.rmsnorm_qk_fwd, args))
            elif w.kind == "quant":
                args = (p["x"], p["r"], g.data_ptr(), p["q"], p["scale"], w.quant_mode, p["rstd"],
                        M, N, w.eps, w.x_dt, w.g_dt, self.stream_handle)
                self.calls.append((lib.rmsnorm_quant_fwd, args))
            elif w.kind == "ln_bwd":
                args = (p["dy"], p["x"], p["mean"], p["rstd"], g.data_ptr(), p["dx"], p["dgamma"],
                        p["dbeta"], p["ws"], self.ws_bytes, M, N, w.x_dt, w.g_dt,
                        self.stream_handle)
                self.calls.append((lib.layernorm_bwd, args))
            elif w.kind == "bwd":
                args = (p["dy"], p["x"], p["rstd"], g.data_ptr(), p["dx"], p["dgamma"], p["ws"],
                        self.ws_bytes, M, N, w.x_dt, w.g_dt, self.stream_handle)
                self.calls.append((lib.rmsnorm_bwd, args))
            else:
                args = (p["dy"], p["x"], p["rstd"], g.data_ptr(), p["dres"], p["dx"],
                        p["dgamma"], p["ws"], self.ws_bytes, M, N, w.x_dt, w.g_dt,
                        self.stream_handle)
                self.calls.append((lib.rmsnorm_fused_add_bwd, args))

    def step(self, i: int) -> None:
        fn, args = self.calls[i % len(self.calls)]
        st = fn(*args)
        if st != 0:
            raise RuntimeError(f"{self.w.name}: {self.R.rmsnorm_status_string(st)}")

    def pristine_outputs(self, host_inputs: dict) -> dict:
        """Replica 0 recomputed from the workload's original inputs (the
        timed loop overwrites the residual of a fused add and QK-norm's
        buffer in place), outputs copied to the host as storage arrays."""
        import numpy as np
        import torch
        w, s0 = self.w, self.sets[0]

        def put(t, a):
            src = torch.from_numpy(a.reshape(-1) if w.x_dt == 0 or a.dtype != np.uint16
                                   else a.reshape(-1).view(np.int16))
            t.copy_(src.view(t.dtype) if src.dtype != t.dtype else src)

        def host(t):
            t = t.detach().cpu()
            if t.dtype in (torch.bfloat16, torch.float16):
                return t.view(torch.int16).numpy().view(np.uint16).copy()
            return t.numpy().copy()

        if w.kind == "qk":
            put(s0["x"], host_inputs["x"])
        if s0.get("r") is not None:
            put(s0["r"], host_inputs["r"])
        torch.cuda.synchronize()
        self.step(0)
        torch.cuda.synchronize()
        keep = {"y", "rstd", "r", "q", "scale", "dx", "dgamma", "dbeta"}
        keep |= {"x"} if w.kind == "qk" else set()
        keep |= {"mean"} if w.kind in ("ln", "ln_bwd") else set()
        return {k: host(v) for k, v in s0.items() if k in keep and v is not None}


def time_steps(step, steps: int, warmup: int) -> float:
    """Milliseconds per step over exactly `steps` back-to-back steps."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        step(warmup + i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def copy_calibration(nbytes: int, rotate_bytes: float, steps: int = 200) -> float:
    """GB/s of a plain device-to-device tensor copy moving nbytes (read + write)
    per step, over rotated buffers."""
    import torch
    half = nbytes // 2
    reps = max(1, int(-(-rotate_bytes // nbytes)))
    src = list(torch.ones((reps, half), dtype=torch.uint8, device="cuda").unbind(0))
    dst = list(torch.empty((reps, half), dtype=torch.uint8, device="cuda").unbind(0))
    ms = time_steps(lambda i: dst[i % reps].copy_(src[i % reps]), steps, 20)
    del src, dst
    return 2 * half / (ms * 1e-3) / 1e9


_CALIB = None


def _calib_lib():
    """librmsn_copy16.so (the measurement kernels), or None if not built."""
    global _CALIB
    if _CALIB is None:
        import ctypes
        path = os.path.join(ROOT, "row_wise_normalization_fwd_amd", "librmsn_copy16.so")
        if not os.path.exists(path):
            return None
        lib = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.rmsn_calib_copy16.argtypes = [vp, vp, i64, vp]
        lib.rmsn_calib_copy16.restype = i32
        lib.rmsn_calib_stream.argtypes = [vp, vp, vp, vp, i64, vp]
        lib.rmsn_calib_stream.restype = i32
        lib.rmsn_calib_mix.argtypes = [vp, i32, vp, i32, i64, vp, vp]
        lib.rmsn_calib_mix.restype = i32
        _CALIB = lib
    return _CALIB


def copy16_calibration(nbytes: int, rotate_bytes: float, steps: int = 200):
    """GB/s of the 16-byte non-temporal copy kernel (librmsn_copy16.so) moving
    nbytes (read + write) per step over rotated buffers laid out like the
    workloads' (one [R, bytes] allocation per operand); None if not built."""
    import torch
    lib = _calib_lib()
    if lib is None:
        return None
    half = (nbytes // 2) // 16 * 16
    reps = max(1, int(-(-rotate_bytes // (2 * half))))
    src = torch.ones((reps, half), dtype=torch.uint8, device="cuda")
    dst = torch.empty((reps, half), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    ptrs = [(src[i].data_ptr(), dst[i].data_ptr()) for i in range(reps)]

    def step(i):
        s_, d_ = ptrs[i % reps]
        if lib.rmsn_calib_copy16(s_, d_, half, stream) != 0:
            raise RuntimeError("copy16 calibration launch failed")
    ms = time_steps(step, steps, 20)
    ok = torch.equal(dst[0][:4096], src[0][:4096])
    del src, dst
    if not ok:
        raise RuntimeError("copy16 calibration copied wrong bytes")
    return 2 * half / (ms * 1e-3) / 1e9


def stream_calibration(each: int, inputs: int, rotate_bytes: float, steps: int = 200):
    """GB/s of librmsn_copy16.so's stream kernel reading `inputs` (2 or 3)
    arrays of `each` bytes and writing one, per step, over rotated buffers laid
    out like the workloads' (one [R, bytes] allocation per operand); the
    practical ceiling for the backward's mix of reads and writes. None if the
    library is not built."""
    import torch
    lib = _calib_lib()
    if lib is None:
        return None
    each = each // 16 * 16
    reps = max(1, int(-(-rotate_bytes // ((inputs + 1) * each))))
    ins = [torch.randint(0, 256, (reps, each), dtype=torch.uint8, device="cuda")
           for _ in range(inputs)]
    dst = torch.empty((reps, each), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    ptrs = [([t[i].data_ptr() for t in ins] + [None] * (3 - inputs), dst[i].data_ptr())
            for i in range(reps)]

    def step(i):
        (a, b, c), d = ptrs[i % reps]
        if lib.rmsn_calib_stream(a, b, c, d, each, stream) != 0:
            raise RuntimeError("stream calibration launch failed")
    ms = time_steps(step, steps, 20)
    want = ins[0][0][:4096] ^ ins[1][0][:4096]
    if inputs == 3:
        want = want ^ ins[2][0][:4096]
    ok = torch.equal(dst[0][:4096], want)
    del ins, dst
    if not ok:
        raise RuntimeError("stream calibration wrote wrong bytes")
    return (inputs + 1) * each / (ms * 1e-3) / 1e9


# Read:write plane counts the mix stream offers (librmsn_copy16.so,
# rmsn_calib_mix: A 16-byte reads and B 16-byte writes per unit).
MIX_RATIOS = [(1, 0), (0, 1), (1, 1), (2, 1), (3, 1), (4, 1), (4, 3), (3, 2)]


def mix_ratio(read_bytes: int, write_bytes: int) -> tuple[int, int]:
    """The offered (A, B) closest to read_bytes : write_bytes (in log ratio)."""
    import math
    if write_bytes <= 0:
        return (1, 0)
    if read_bytes <= 0:
        return (0, 1)
    want = math.log(read_bytes / write_bytes)
    both = [r for r in MIX_RATIOS if r[0] and r[1]]
    return min(both, key=lambda r: abs(math.log(r[0] / r[1]) - want))


def mix_calibration(read_bytes: int, write_bytes: int, rotate_bytes: float, steps: int = 200,
                    ratio=None):
    """The mix stream (16-byte non-temporal, A reads to B writes per unit with
    (A, B) = mix_ratio(read_bytes, write_bytes) unless given) moving about
    read_bytes in and write_bytes out per step over rotated buffers: dict with
    gbps (its own bytes over its time), the ratio and the bytes per step; None
    if the library is not built."""
    import torch
    lib = _calib_lib()
    if lib is None:
        return None
    A, B = ratio or mix_ratio(read_bytes, write_bytes)
    per_plane = read_bytes / A if A else write_bytes / B
    n = max(64, int(per_plane // 16))
    plane = 16 * n
    step_bytes = (A + B) * plane
    reps = max(1, int(-(-rotate_bytes // step_bytes)))
    src = (torch.randint(-2 ** 31, 2 ** 31 - 1, (reps, A * n * 4), dtype=torch.int32, device="cuda")
           if A else None)
    dst = torch.empty((reps, B * n * 4), dtype=torch.int32, device="cuda") if B else None
    sink = torch.empty(1024, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    ptrs = [(src[i].data_ptr() if A else None, dst[i].data_ptr() if B else None)
            for i in range(reps)]

    def step(i):
        sp, dp = ptrs[i % reps]
        if lib.rmsn_calib_mix(sp, A, dp, B, n, sink.data_ptr(), stream) != 0:
            raise RuntimeError("mix calibration launch failed")
    ms = time_steps(step, steps, 20)
    if B:
        # unit u writes [u, u >> 32, 0, 0] ^ (its A source chunks) to every plane
        k = 64
        idx = torch.zeros((k, 4), dtype=torch.int32, device="cuda")
        idx[:, 0] = torch.arange(k, dtype=torch.int32, device="cuda")
        want = idx
        for a in range(A):
            want = want ^ src[0].view(A, n, 4)[a, :k]
        got = dst[0].view(B, n, 4)[:, :k]
        if not all(torch.equal(got[b], want) for b in range(B)):
            raise RuntimeError("mix calibration wrote wrong bytes")
    del src, dst, sink
    return {"gbps": round(step_bytes / (ms * 1e-3) / 1e9, 2), "reads_per_write":
            f"{A}:{B}", "bytes_per_step": step_bytes, "rotation_replicas": reps}


class BusyMonitor:
    """Samples the device's own sysfs gpu_busy_percent (matched to device 0's
    PCI address) while this process has nothing in flight: a sample above the
    threshold means another process is using the GPU."""

    def __init__(self, threshold_pct: int = 10, path: str | None = None, sync=None):
        """path: the counter file (found from device 0's PCI address when
        None); sync: called before sampling (torch.cuda.synchronize when
        None)."""
        self.threshold = threshold_pct
        self.log = []
        self.path = path
        self.sync = sync
        if path is not None:
            return
        import torch
        self.sync = sync or torch.cuda.synchronize
        p = torch.cuda.get_device_properties(0)
        bus, dev = getattr(p, "pci_bus_id", None), getattr(p, "pci_device_id", None)
        dom = getattr(p, "pci_domain_id", 0) or 0
        if bus is not None and dev is not None:
            cand = f"/sys/bus/pci/devices/{dom:04x}:{bus:02x}:{dev:02x}.0/gpu_busy_percent"
            if os.access(cand, os.R_OK):
                self.path = cand
        if self.path is None:
            cands = {os.path.realpath(c) for c in glob.glob("/sys/class/drm/card*/device/gpu_busy_percent")
                     if os.access(c, os.R_OK)}
            if len(cands) == 1:
                self.path = cands.pop()

    def sample(self, n: int = 5, gap_s: float = 0.02):
        """n readings (percent), or [] when no source is readable."""
        if self.path is None:
            return []
        out = []
        for i in range(n):
            try:
                with open(self.path) as fh:
                    out.append(int(fh.read().strip()))
            except (OSError, ValueError):
                return out
            if i + 1 < n:
                time.sleep(gap_s)
        return out

    def idle(self, tag: str, settle_s: float = 0.5) -> bool:
        """Sample and record; True when every reading is at or below the
        threshold or there is no source. The counter is a running average
        that decays by about a fifth every 20 ms, so it still shows this
        process's own last kernels for a while: wait settle_s after they end
        (half a second takes a full load below 1%) before sampling."""
        if self.sync is not None:
            self.sync()
        if self.path is not None and settle_s > 0:
            time.sleep(settle_s)
        vals = self.sample()
        busy = bool(vals) and max(vals) > self.threshold
        self.log.append({"at": tag, "busy_pct": vals, "busy": busy})
        return not busy

    def summary(self) -> dict:
        return {"source": self.path, "threshold_pct": self.threshold,
                "samples": len(self.log), "busy_samples": sum(r["busy"] for r in self.log),
                "log": self.log[-12:]}


def graph_replay_ms(run, calls: int = 100, replays: int = 40) -> float:
    """Milliseconds per step when `calls` steps are captured in one HIP graph
    (torch.cuda.CUDAGraph) and the graph is replayed: the GPU's own rate for a
    step, without a host launch per call. The captured calls cycle through the
    runner's rotation replicas as the timed steps do."""
    import torch
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(calls):
                fn, args = run.calls[i % len(run.calls)]
                if fn(*(args[:-1] + (side.cuda_stream,))) != 0:
                    raise RuntimeError("graph capture: launch failed")
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    del graph
    return start.elapsed_time(end) / (replays * calls)


def rounds(step, ms_per_step: float, n: int = 5, cooldown_s: float = 1.0, start: int = 0,
           monitor=None, retries: int = 2):
    """n further timing rounds of the same step, each >= 20 ms of back-to-back
    launches after a >= 50 ms warm-up, with a cool-down before each round:
    median, min and mean microseconds per step and the spread. With a
    BusyMonitor, the device is sampled before and after each round; a round
    with a busy sample is timed again (up to `retries` times) and, if still
    busy, kept and counted as interfered."""
    import statistics
    k = max(50, int(0.020 / (ms_per_step * 1e-3)) + 1)
    warm = max(10, int(0.050 / (ms_per_step * 1e-3)) + 1)
    us = []
    requeued = interfered = 0
    i = start
    for r in range(n):
        for attempt in range(retries + 1):
            time.sleep(cooldown_s)
            idle_before = monitor.idle(f"round {r} before", settle_s=0.0) if monitor else True
            t = 1e3 * time_steps(lambda j: step(i + j), k, warm if r == 0 else 10)
            i += k + warm
            idle_after = monitor.idle(f"round {r} after") if monitor else True
            if idle_before and idle_after:
                break
            if attempt < retries:
                requeued += 1
            else:
                interfered += 1
        us.append(t)
    med = statistics.median(us)
    return {"rounds": n, "steps_per_round": k, "cooldown_s": cooldown_s,
            "us_median": round(med, 3), "us_min": round(min(us), 3),
            "us_mean": round(statistics.fmean(us), 3),
            "spread_pct": round(100 * (max(us) - min(us)) / med, 2),
            "requeued_busy": requeued, "interfered": interfered}


def load_traffic(workload: str, src_hash: str):
    """Measured HBM bytes per launch from the committed counter summary, if it
    was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_src_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, host_inputs: dict, seconds: float, best_of: int = 1) -> dict:
    """The fp64 oracle, as it stands, timed on one host core: passes over the
    whole batch until `seconds` have gone by (at least one), or the best of
    `best_of` passes (for batches too small to time one pass reliably)."""
    import oracle as O
    O._load()
    M, N = w.M, w.N
    x, g = host_inputs["x"], host_inputs["gamma"]
    if w.kind == "fwd":
        def one_pass():
            O.rmsnorm_fwd(x, g, M, N, w.eps, w.x_dt, w.g_dt, want_exact=False)
    elif w.kind == "fused_add":
        def one_pass():
            O.rmsnorm_fused_add_fwd(x, host_inputs["r"], g, M, N, w.eps, w.x_dt, w.g_dt,
                                    want_exact=False)
    elif w.kind == "ln":
        def one_pass():
            O.layernorm_fwd(x, g, host_inputs["beta"], M, N, w.eps, w.x_dt, w.g_dt,
                            want_exact=False)
    elif w.kind == "qk":
        S = (w.heads_q + 2 * w.heads_k) * N

        def one_pass():
            buf, _ = O.rmsnorm_heads_fwd(x.reshape(-1), g, M, w.heads_q, N, S, w.eps, w.x_dt,
                                         w.g_dt)
            O.rmsnorm_heads_fwd(buf, host_inputs["gamma_k"], M, w.heads_k, N, S, w.eps, w.x_dt,
                                w.g_dt, offset=w.heads_q * N)
    elif w.kind == "quant" and w.quant_mode >= 3:
        def one_pass():
            O.rmsnorm_mx_fwd(x, g, M, N, w.eps, w.x_dt, w.g_dt,
                             O.E4M3 if w.quant_mode == 3 else O.E2M1, r=host_inputs.get("r"),
                             want_exact=False)
    elif w.kind == "quant":
        def one_pass():
            O.rmsnorm_quant_fwd(x, g, M, N, w.eps, w.x_dt, w.g_dt, w.quant_mode,
                                scale=w.tensor_scale, r=host_inputs.get("r"), want_exact=False)
    elif w.kind == "ln_bwd":
        f = O.layernorm_fwd(x, g, None, M, N, w.eps, w.x_dt, w.g_dt, want_exact=False)

        def one_pass():
            O.layernorm_bwd(host_inputs["dy"], x, f["mean"], f["rstd"], g, M, N, w.x_dt, w.g_dt,
                            want_exact=False)
    else:
        # The saved rstd is an input of the backward, made outside the timing.
        rho = O.rmsnorm_fwd(x, g, M, N, w.eps, w.x_dt, w.g_dt, want_exact=False)["rstd"]
        dres = host_inputs.get("dres")

        def one_pass():
            O.rmsnorm_fused_add_bwd(host_inputs["dy"], x, rho, g, dres, M, N, w.x_dt, w.g_dt,
                                    want_exact=False)
    if best_of > 1:
        times = []
        for _ in range(best_of):
            t0 = time.perf_counter()
            one_pass()
            times.append(time.perf_counter() - t0)
        el, passes = min(times), 1
        sample = (f"best of {best_of} full passes over the {M}x{N} batch (single thread, host "
                  f"has {os.cpu_count()} logical CPUs)")
    else:
        passes, t0 = 0, time.perf_counter()
        while True:
            one_pass()
            passes += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        sample = (f"{passes} full pass{'es' if passes > 1 else ''} over the {M}x{N} batch "
                  f"({el:.1f} s, single thread, host has {os.cpu_count()} logical CPUs)")
    return {"value": round(w.algorithmic_bytes() * passes / el / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle", "sample": sample,
            "rows_per_s": round(rows_of(w) * passes / el, 1),
            "ms_per_pass": round(1e3 * el / passes, 3),
            "host_cpu": _cpu_model()}


def parity_check(w, outs: dict, host_inputs: dict, rows: int = 64) -> dict:
    """Part of the CPU leg: the pristine step's outputs (Runner.pristine_outputs)
    against the fp64 oracle on `rows` rows spread over the batch (every row of
    a smaller one), with the GPU tests' tolerances (tests/gpu_util.py). The
    backwards are checked on dx with the rstd (and mean) their timed step
    used; dgamma and dbeta sum over every row and are left to the tests."""
    import numpy as np

    import oracle as O
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import gpu_util as U
    M, N, xdt, gdt = w.M, w.N, w.x_dt, w.g_dt
    idx = np.unique(np.linspace(0, M - 1, min(rows, M)).round().astype(np.int64))
    S = int(idx.size)
    g = host_inputs["gamma"]

    def pick(a, n=N):
        return np.ascontiguousarray(a.reshape(M, n)[idx])

    try:
        if w.kind == "fwd":
            x = pick(host_inputs["x"])
            ref = O.rmsnorm_fwd(x, g, S, N, w.eps, xdt, gdt)
            U.check_output(pick(outs["y"]), ref["y_exact"], ref["y"], xdt, "y")
            if "rstd" in outs:
                U.check_rstd(outs["rstd"][idx], ref["rstd_exact"])
        elif w.kind == "fused_add":
            x, r = pick(host_inputs["x"]), pick(host_inputs["r"])
            ref = O.rmsnorm_fused_add_fwd(x, r, g, S, N, w.eps, xdt, gdt)
            assert np.array_equal(pick(outs["r"]), ref["h"]), "h not bit for bit"
            U.check_output(pick(outs["y"]), ref["y_exact"], ref["y"], xdt, "y")
        elif w.kind == "quant":
            x = pick(host_inputs["x"])
            r = pick(host_inputs["r"]) if w.fused_quant else None
            if w.quant_mode >= 3:
                elem = O.E4M3 if w.quant_mode == 3 else O.E2M1
                ref = O.rmsnorm_mx_fwd(x, g, S, N, w.eps, xdt, gdt, elem, r=r)
                q = pick(outs["q"], N // 2 if elem == O.E2M1 else N)
                q = U.unpack_fp4(q, S, N) if elem == O.E2M1 else q
                U.check_mx(q, pick(outs["scale"], N // 32), ref, elem)
            else:
                ref = O.rmsnorm_quant_fwd(x, g, S, N, w.eps, xdt, gdt, w.quant_mode,
                                          scale=w.tensor_scale if w.quant_mode == 1 else None, r=r)
                U.check_fp8(pick(outs["q"]), ref, w.quant_mode == 2,
                            outs["scale"][idx] if w.quant_mode == 2 else None)
            if r is not None:
                assert np.array_equal(pick(outs["r"]), ref["h"]), "h not bit for bit"
        elif w.kind == "qk":
            H, Hk = w.heads_q, w.heads_k
            sd = (H + 2 * Hk) * N
            buf = pick(host_inputs["x"], sd)
            want, _ = O.rmsnorm_heads_fwd(buf.reshape(-1), g, S, H, N, sd, w.eps, xdt, gdt)
            want, _ = O.rmsnorm_heads_fwd(want, host_inputs["gamma_k"], S, Hk, N, sd, w.eps, xdt,
                                          gdt, offset=H * N)
            want = want.reshape(S, sd)
            got = pick(outs["x"], sd)
            moved = np.zeros((S, sd), bool)
            moved[:, :(H + Hk) * N] = True
            assert np.array_equal(got[~moved], buf[~moved]), "v heads changed"
            U.check_output(got[moved], O.decode(want, xdt)[moved], want[moved], xdt, "qk")
        elif w.kind == "ln":
            x, b = pick(host_inputs["x"]), host_inputs["beta"]
            ref = O.layernorm_fwd(x, g, b, S, N, w.eps, xdt, gdt)
            U.check_layernorm(pick(outs["y"]), ref, x, g, b, xdt, outs["mean"][idx],
                              outs["rstd"][idx])
        elif w.kind in ("bwd", "fused_add_bwd"):
            x, dy = pick(host_inputs["x"]), pick(host_inputs["dy"])
            rho = outs["rstd"][idx].astype(np.float64)
            dres = pick(host_inputs["dres"]) if w.kind == "fused_add_bwd" else None
            ref = (O.rmsnorm_fused_add_bwd(dy, x, rho, g, dres, S, N, xdt, gdt)
                   if dres is not None else O.rmsnorm_bwd(dy, x, rho, g, S, N, xdt, gdt))
            U.check_dx(pick(outs["dx"]), ref, x, dy, g, rho, xdt, dres=dres)
        elif w.kind == "ln_bwd":
            x, dy = pick(host_inputs["x"]), pick(host_inputs["dy"])
            mean, rstd = outs["mean"][idx], outs["rstd"][idx]
            ref = O.layernorm_bwd(dy, x, mean, rstd, g, S, N, xdt, gdt)
            U.check_layernorm_bwd(pick(outs["dx"]), None, None, ref, x, dy, g, mean, rstd, xdt)
        return {"ok": True, "rows_checked": S, "of": M}
    except AssertionError as e:
        return {"ok": False, "rows_checked": S, "of": M, "error": str(e)[:300]}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------- profiling
#
# --collect-profiles DIR runs rocprofv3 over single-workload bench runs as
# child processes (this process never touches the GPU): a kernel trace, then
# one counter pass per group (FETCH_SIZE, WRITE_SIZE, LDS, occupancy, VALU).
# --reduce-profiles DIR turns their CSV output into profiles/*.md and
# profiles/traffic_*.json. Counter passes time --steps 16 after --warmup 4
# (their dispatches 4..19 of the workload's own kernels), the trace --steps
# 200 after --warmup 500 (dispatches 500..699).

TRACE_W, TRACE_S, PMC_W, PMC_S = 500, 200, 4, 16
PROFILE_PASSES = {
    "fetch": "FETCH_SIZE",
    "write": "WRITE_SIZE",
    "lds": "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAVE_CYCLES SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE",
    "occ": "MeanOccupancyPerActiveCU",
    "valu": "VALUBusy MemUnitStalled",
}


def profile_command(w, kind: str, prof_dir: str) -> str:
    """The rocprofv3 command of one pass over workload w (repository root)."""
    b = f"python3 bench.py --workload {w.name} --no-others --no-cpu --no-graph --rounds 0"
    if w.M * w.N < (1 << 20):
        b += " --rotate-bytes 0"
    d = f"{prof_dir}/{w.name}/{kind}"
    if kind == "trace":
        return (f"rocprofv3 --kernel-trace --stats --output-format csv -d {d} -o trace -- {b} "
                f"--steps {TRACE_S} --warmup {TRACE_W}")
    return (f"rocprofv3 --pmc {PROFILE_PASSES[kind]} --output-format csv -d {d} -o {kind} -- {b} "
            f"--steps {PMC_S} --warmup {PMC_W}")


def collect_profiles(prof_dir: str, names, kinds, timeout_s: int = 150) -> int:
    """Run the passes, each in its own process group under a time limit;
    stop at the first failure. Returns 0 or the failing pass's status."""
    import shlex
    import signal
    import subprocess

    import gen as G
    env = dict(os.environ, TMPDIR="/tmp")
    for name in names:
        w = G.WORKLOADS_BY_NAME[name]
        for kind in kinds:
            cmd = profile_command(w, kind, prof_dir)
            log = os.path.join(ROOT, prof_dir, f"{name}.{kind}.log")
            os.makedirs(os.path.dirname(log), exist_ok=True)
            print(f"[{time.strftime('%H:%M:%S')}] {name} {kind}", flush=True)
            with open(log, "w") as fh:
                proc = subprocess.Popen(shlex.split(cmd), cwd=ROOT, env=env, stdout=fh,
                                        stderr=subprocess.STDOUT, start_new_session=True)
                try:
                    rc = proc.wait(timeout=timeout_s)
                except subprocess.TimeoutExpired:
                    os.killpg(proc.pid, signal.SIGKILL)
                    proc.wait()
                    rc = 124
            if rc != 0:
                # rocprofv3 itself may end with a segmentation fault after a
                # complete run; accept that only when the results are there.
                done = glob.glob(os.path.join(ROOT, prof_dir, name, kind, "*.csv"))
                if rc == -11 or rc == 139:
                    if done:
                        print(f"  rocprofv3 exited {rc} after writing {len(done)} files; kept",
                              flush=True)
                        continue
                print(f"  failed rc={rc}; see {log}", flush=True)
                return rc if rc > 0 else 128 - rc
    print(f"[{time.strftime('%H:%M:%S')}] done", flush=True)
    return 0


def _short_kernel(name: str) -> str:
    s = name[5:] if name.startswith("void ") else name
    s = s.replace("rmsn::", "")
    depth = 0
    for i, c in enumerate(s):
        if c == "<":
            depth += 1
        elif c == ">":
            depth -= 1
        elif c == "(" and depth == 0:
            return s[:i]
    return s


def _csv_rows(path: str):
    import csv
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _one(pattern: str):
    fs = glob.glob(pattern)
    if len(fs) != 1:
        raise RuntimeError(f"expected one file for {pattern}, found {fs}")
    return fs[0]


def _trace_kernels(prof: str, name: str) -> dict:
    """{kernel: trace rows of its timed dispatches}, in launch order."""
    rs = _csv_rows(_one(f"{prof}/{name}/trace/*_kernel_trace.csv"))
    rs.sort(key=lambda r: int(r["Dispatch_Id"]))
    by = {}
    for r in rs:
        if "rmsn::" in r["Kernel_Name"]:
            by.setdefault(_short_kernel(r["Kernel_Name"]), []).append(r)
    out = {k: v[TRACE_W:TRACE_W + TRACE_S] for k, v in by.items() if len(v) >= TRACE_W + TRACE_S}
    return dict(sorted(out.items(), key=lambda kv: int(kv[1][0]["Dispatch_Id"])))


def _counters(prof: str, name: str, kind: str, kernels) -> dict:
    """{kernel: {counter: [values over the timed dispatches]}} ({} if absent)."""
    fs = glob.glob(f"{prof}/{name}/{kind}/*_counter_collection.csv")
    if len(fs) != 1:
        return {}
    disp = {}
    for r in _csv_rows(fs[0]):
        k = _short_kernel(r["Kernel_Name"])
        if k not in kernels:
            continue
        d = disp.setdefault(k, {}).setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["_wg"] = int(r["Workgroup_Size"])
    out = {}
    for k, dd in disp.items():
        vals = {}
        for i in sorted(dd)[PMC_W:PMC_W + PMC_S]:
            for c, v in dd[i].items():
                vals.setdefault(c, []).append(v)
        out[k] = vals
    return out


def _traffic_scale(prof: str):
    """FETCH_SIZE / WRITE_SIZE scale factors from the plain copies in the
    headline workload's counter runs: (read scale, write scale, text)."""
    import statistics

    import gen as G
    res = {}
    for kind, ctr in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        rs = _csv_rows(_one(f"{prof}/{HEADLINE}/{kind}/*_counter_collection.csv"))
        grids = {}
        for r in rs:
            if r["Kernel_Name"] == "__amd_rocclr_copyBuffer" and r["Counter_Name"] == ctr:
                grids.setdefault(int(r["Grid_Size"]), []).append(float(r["Counter_Value"]))
        _, v = max(grids.items(), key=lambda kv: len(kv[1]))
        c16 = [float(r["Counter_Value"]) for r in rs
               if "copy16_kernel" in r["Kernel_Name"] and r["Counter_Name"] == ctr]
        res[kind] = (statistics.median(v), len(v), statistics.median(c16) if c16 else float("nan"))
    w = G.WORKLOADS_BY_NAME[HEADLINE]
    true_kib = w.M * w.N * w.esize / 1024.0
    rsc, wsc = round(true_kib / res["fetch"][0], 4), round(true_kib / res["write"][0], 4)
    text = (f"Calibration: the headline workload's counter runs (`{profile_command(w, 'fetch', prof)}` "
            f"and its WRITE_SIZE twin) copy {true_kib:.0f} KiB each way with torch's device copy "
            f"(`__amd_rocclr_copyBuffer`): FETCH_SIZE {res['fetch'][0]:.1f} KiB and WRITE_SIZE "
            f"{res['write'][0]:.1f} KiB per dispatch (median of {res['fetch'][1]} / {res['write'][1]}), "
            f"so reads are scaled by {rsc:.4f} and writes by {wsc:.4f}. The bench's 16-byte "
            f"non-temporal copy kernel in the same runs reads {res['fetch'][2]:.1f} KiB of "
            f"FETCH_SIZE and {res['write'][2]:.1f} KiB of WRITE_SIZE for the same bytes.")
    return rsc, wsc, text


def reduce_profiles(prof: str) -> int:
    """profiles/<kernel>__<workload>.md, profiles/traffic_<workload>.json and
    the all-workload LDS / occupancy and VALU tables from collect_profiles'
    output under prof (relative to the repository root)."""
    import statistics

    import gen as G
    absprof = os.path.join(ROOT, prof)
    outd = os.path.join(ROOT, "profiles")
    h = kernel_source_hash()
    rscale, wscale, cal_text = _traffic_scale(absprof)
    lds_rows, valu_rows = [], []
    for w in G.WORKLOADS + G.EXTRA_WORKLOADS:
        if not os.path.isdir(f"{absprof}/{w.name}/trace"):
            print("no profile for", w.name)
            continue
        ks = _trace_kernels(absprof, w.name)
        fe = _counters(absprof, w.name, "fetch", ks)
        wr = _counters(absprof, w.name, "write", ks)
        ld = _counters(absprof, w.name, "lds", ks)
        oc = _counters(absprof, w.name, "occ", ks)
        va = _counters(absprof, w.name, "valu", ks)
        small = w.M * w.N < (1 << 20)
        lines = [f"# {w.name}: {' + '.join(ks)}", "",
                 f"Workload: {w.kind}, M={w.M}, N={w.N}, x {DT_NAMES[w.x_dt]}, gamma "
                 f"{DT_NAMES[w.g_dt]}, eps={w.eps}, rstd written: {w.store_rstd}. "
                 + ("Inputs are not rotated (the launch-bound 64 x 1024 case, as in the bench)."
                    if small else "Inputs rotate over >= 1 GiB of replicas (HBM, not Infinity Cache)."),
                 "", f"Kernel sources hash (bench.py `kernel_source_hash`): `{h}`", "",
                 "Made by `python3 bench.py --collect-profiles " + prof + " --profile-workloads "
                 + w.name + "` then `python3 bench.py --reduce-profiles " + prof + "`, which run "
                 "(repository root, one MI355X; each selects the workload's own dispatches inside "
                 f"the timed loop, dispatches {TRACE_W}..{TRACE_W + TRACE_S - 1} of the trace run "
                 f"and {PMC_W}..{PMC_W + PMC_S - 1} of the counter runs):", "",
                 f"    {profile_command(w, 'trace', prof)}", f"    {profile_command(w, 'fetch', prof)}",
                 f"    {profile_command(w, 'write', prof)}", "",
                 "| kernel | timed dispatches | avg us | median us | min us | max us | VGPR_Count | "
                 "SGPR | static LDS B | scratch B/lane |",
                 "|---|---|---|---|---|---|---|---|---|---|"]
        tot_us, tot_bytes, kj = 0.0, 0.0, []
        for k, rs in ks.items():
            d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0 for r in rs]
            r0 = rs[0]
            avg = statistics.mean(d)
            tot_us += avg
            lines.append(f"| `{k}` | {len(d)} | {avg:.2f} | {statistics.median(d):.2f} | "
                         f"{min(d):.2f} | {max(d):.2f} | {r0['VGPR_Count']} | {r0['SGPR_Count']} | "
                         f"{r0['LDS_Block_Size']} | {r0['Scratch_Size']} |")
            rec = {"kernel": k, "avg_us": round(avg, 3)}
            if k in fe and k in wr:
                f = statistics.median(fe[k]["FETCH_SIZE"])
                wv = statistics.median(wr[k]["WRITE_SIZE"])
                tot_bytes += (f * rscale + wv * wscale) * 1024
                rec.update({"fetch_kib_raw": round(f, 1), "write_kib_raw": round(wv, 1)})
            kj.append(rec)
            lv = ld.get(k, {})
            if lv:
                conf = statistics.median(lv["SQ_LDS_BANK_CONFLICT"])
                act = statistics.median(lv["SQ_LDS_IDX_ACTIVE"])
                gui = statistics.median(lv["GRBM_GUI_ACTIVE"])
                occ = statistics.median(oc[k]["MeanOccupancyPerActiveCU"]) if k in oc else float("nan")
                lds_rows.append(f"| {w.name} | `{k}` | {lv['_wg'][0]} | "
                                f"{conf / act if act else 0.0:.4f} | {100.0 * conf / gui / 256:.3f} | "
                                f"{occ:.2f} |")
            if k in va:
                valu_rows.append(f"| {w.name} | `{k}` | {statistics.median(va[k]['VALUBusy']):.1f} | "
                                 f"{statistics.median(va[k]['MemUnitStalled']):.1f} |")
        alg = w.algorithmic_bytes()
        lines += ["", "Register and LDS columns are rocprofv3's kernel-trace fields. On this device "
                  "its VGPR_Count reads the compiler's VGPR allocation halved and rounded up to a "
                  "multiple of 4 (e.g. 52 for 97, 64 for 126), and LDS_Block_Size is the static "
                  "allocation only (512-byte granules): dynamic LDS requested at launch is not "
                  "included.", ""]
        have_traffic = all("fetch_kib_raw" in j for j in kj)
        if have_traffic:
            lines += ["HBM traffic per step (rocprofv3 counters, median KiB per dispatch):", ""]
            for j in kj:
                lines.append(f"- `{j['kernel']}`: FETCH_SIZE {j['fetch_kib_raw']:.1f} KiB raw (x "
                             f"{rscale:.4f} = {j['fetch_kib_raw'] * rscale:.1f} KiB), WRITE_SIZE "
                             f"{j['write_kib_raw']:.1f} KiB raw (x {wscale:.4f})")
            lines += ["", cal_text, "",
                      f"- measured HBM bytes per step: {int(round(tot_bytes)):,} "
                      f"({tot_bytes / alg:.4f} x algorithmic)"]
        lines += [f"- algorithmic bytes per step: {alg:,}",
                  f"- kernel time per step (profiled): {tot_us:.2f} us",
                  f"- achieved (algorithmic / kernel time): {alg / (tot_us * 1e-6) / 1e9:.1f} GB/s = "
                  f"{100 * alg / (tot_us * 1e-6) / 1e9 / PEAK_GBPS:.1f}% of {PEAK_GBPS:.0f} GB/s", ""]
        dom = DOMINANT_KERNEL.get(w.name) or max(kj, key=lambda j: j["avg_us"])["kernel"].split("<")[0]
        for old in glob.glob(f"{outd}/*__{w.name}.md"):
            os.remove(old)
        with open(f"{outd}/{dom}__{w.name}.md", "w") as fh:
            fh.write("\n".join(lines))
        if have_traffic:
            rec = {"workload": w.name, "kernel_src_hash": h, "bytes_per_launch": int(round(tot_bytes)),
                   "algorithmic_bytes": alg, "read_scale": rscale, "write_scale": wscale,
                   "kernels": kj, "commands": [profile_command(w, "fetch", prof),
                                               profile_command(w, "write", prof)]}
            with open(f"{outd}/traffic_{w.name}.json", "w") as fh:
                json.dump(rec, fh, indent=1)
        print(f"{w.name}: {tot_us:.2f} us"
              + (f", traffic {tot_bytes / alg:.4f}x" if have_traffic else ""))
    w0 = G.WORKLOADS_BY_NAME[HEADLINE]
    if lds_rows:
        hdr = ["# LDS bank conflicts and occupancy, every workload's kernels", "",
               f"Kernel sources hash (bench.py `kernel_source_hash`): `{h}`", "",
               "Commands (repository root, one MI355X), for each workload W (`--rotate-bytes 0` "
               "for the 64 x 1024 case, as the bench runs it):", "",
               "    " + profile_command(w0, "lds", prof).replace(HEADLINE, "W"),
               "    " + profile_command(w0, "occ", prof).replace(HEADLINE, "W"), "",
               f"Per kernel: medians over the workload's own dispatches {PMC_W}..{PMC_W + PMC_S - 1}. "
               "`conflict/active` = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; `conflict % GPU time` "
               "= 100 * SQ_LDS_BANK_CONFLICT / GRBM_GUI_ACTIVE / 256 CUs; `occupancy` = "
               "rocprofv3's MeanOccupancyPerActiveCU (resident waves per SIMD, of 8).", "",
               "| workload | kernel | workgroup | LDS conflict/active | conflict % GPU time | "
               "occupancy (waves / SIMD) |", "|---|---|---|---|---|---|"]
        with open(f"{outd}/lds_occupancy__all_workloads.md", "w") as fh:
            fh.write("\n".join(hdr + lds_rows) + "\n")
    if valu_rows:
        hdr = ["# VALU and memory-unit load, every workload's kernels", "",
               f"Kernel sources hash (bench.py `kernel_source_hash`): `{h}`", "",
               "Command (repository root, one MI355X), for each workload W:", "",
               "    " + profile_command(w0, "valu", prof).replace(HEADLINE, "W"), "",
               f"Medians over the workload's own dispatches {PMC_W}..{PMC_W + PMC_S - 1}. `VALUBusy` "
               "is rocprofv3's derived share of GPU time the vector ALUs issue, `MemUnitStalled` "
               "the share of time the vector memory unit is stalled.", "",
               "| workload | kernel | VALUBusy % | MemUnitStalled % |", "|---|---|---|---|"]
        with open(f"{outd}/valu_memunit__all_workloads.md", "w") as fh:
            fh.write("\n".join(hdr + valu_rows) + "\n")
    return 0


# Widths and operations of the --scan mode (bf16 activations and gamma).
SCAN_WIDTHS = [256, 512, 768, 1024, 1536, 2048, 2560, 3072, 3584, 4096, 5120, 6144, 7168, 8192,
               10240, 12288, 14336, 16384, 20480, 24576, 28672, 32768]
SCAN_OPS = {"fwd": {"kind": "fwd"}, "fused_add": {"kind": "fused_add"}, "ln": {"kind": "ln"},
            "fp8row": {"kind": "quant", "quant_mode": 2}, "mxfp4": {"kind": "quant", "quant_mode": 4},
            "bwd": {"kind": "bwd"}, "fused_add_bwd": {"kind": "fused_add_bwd"},
            "ln_bwd": {"kind": "ln_bwd"}}


def scan(mib: int, rotate_bytes: float, steps: int, warmup: int, ops=None,
         widths=None) -> int:
    """Every operation of SCAN_OPS over SCAN_WIDTHS, bf16, with M = mib MiB /
    (2 N) rows: one line per (operation, width) as it is timed, then a table
    of % of the 8 TB/s peak (algorithmic bytes / event-timed step)."""
    import torch

    import gen as G

    ops = ops or list(SCAN_OPS)
    widths = widths or SCAN_WIDTHS
    table = {}
    for op in ops:
        extra = SCAN_OPS[op]
        for n in widths:
            m = max(1, (mib << 20) // (2 * n))
            w = G.Workload(f"scan_{op}_m{m}_n{n}", extra["kind"], m, n, G.BF16, G.BF16, 1e-5,
                           9000 + n, quant_mode=extra.get("quant_mode", 0))
            run = Runner(w, rotate_bytes, G.make_inputs(w))
            ms = time_steps(run.step, steps, warmup)
            pct = w.algorithmic_bytes() / (ms * 1e-3) / 1e9 / (PEAK_GBPS / 100.0)
            table[(op, n)] = pct
            print(f"scan {op} M={m} N={n}: {ms * 1e3:.2f} us {pct:.1f}%", flush=True)
            del run
            torch.cuda.empty_cache()
    print("\n| N | " + " | ".join(ops) + " |")
    print("|---|" + "---|" * len(ops))
    for n in widths:
        print(f"| {n} | " + " | ".join(f"{table[(op, n)]:.1f}" for op in ops) + " |")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--rotate-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-others", action="store_true", help="time only the headline workload")
    ap.add_argument("--other-steps", type=int, default=0,
                    help="steps per other workload (default: enough for ~50 ms each)")
    ap.add_argument("--rounds", type=int, default=5,
                    help="extra timing rounds of the headline step (>= 20 ms each, 1 s "
                         "cool-down) for median / min / mean / spread; 0 skips them")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay timing (profiled runs)")
    ap.add_argument("--collect-profiles", metavar="DIR",
                    help="run the rocprofv3 passes into DIR (relative to the repository root) "
                         "as child processes, then exit")
    ap.add_argument("--profile-workloads", default="",
                    help="comma-separated workloads for --collect-profiles (default: all)")
    ap.add_argument("--profile-passes", default="trace,fetch,write,lds,occ,valu",
                    help="comma-separated passes for --collect-profiles")
    ap.add_argument("--scan", action="store_true",
                    help="time every operation over a ladder of row widths (bf16, --scan-mib "
                         "MiB per operand) and print a table of %% of peak, then exit")
    ap.add_argument("--scan-mib", type=int, default=64)
    ap.add_argument("--scan-ops", default="", help="comma-separated subset of the scan's operations")
    ap.add_argument("--scan-widths", default="", help="comma-separated row widths for --scan")
    ap.add_argument("--reduce-profiles", metavar="DIR",
                    help="write profiles/ from the rocprofv3 output under DIR, then exit")
    args = ap.parse_args()

    if args.collect_profiles or args.reduce_profiles:
        # Neither mode touches the GPU in this process.
        import gen as G
        if args.reduce_profiles:
            return reduce_profiles(args.reduce_profiles)
        names = ([n for n in args.profile_workloads.split(",") if n] or
                 [x.name for x in G.WORKLOADS + G.EXTRA_WORKLOADS])
        kinds = [k for k in args.profile_passes.split(",") if k]
        bad = [n for n in names if n not in G.WORKLOADS_BY_NAME] + \
              [k for k in kinds if k != "trace" and k not in PROFILE_PASSES]
        if bad:
            print(f"unknown workloads or passes: {bad}", file=sys.stderr)
            return 2
        return collect_profiles(args.collect_profiles, names, kinds)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world})", file=sys.stderr)
        return 2

    import torch

    import gen as G

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.scan:
        ops = [o for o in args.scan_ops.split(",") if o]
        if any(o not in SCAN_OPS for o in ops):
            print(f"unknown scan operations: {ops}; choose from {list(SCAN_OPS)}", file=sys.stderr)
            return 2
        widths = [int(v) for v in args.scan_widths.split(",") if v]
        return scan(args.scan_mib, args.rotate_bytes, max(1, args.steps // 20), args.warmup // 10,
                    ops, widths)
    src_hash = kernel_source_hash()

    w = G.WORKLOADS_BY_NAME[args.workload]
    host = G.make_inputs(w)
    run = Runner(w, args.rotate_bytes, host)
    monitor = BusyMonitor()
    # The main timed region: wait (up to 3 s) for an idle device first, and
    # record whether it stayed idle.
    for _ in range(3):
        if monitor.idle("main before"):
            break
        time.sleep(1.0)
    ms = time_steps(run.step, args.steps, args.warmup)
    monitor.idle("main after")
    nbytes = w.algorithmic_bytes()
    rbytes, wbytes = w.read_write_bytes()
    gbps = nbytes / (ms * 1e-3) / 1e9
    round_stats = (rounds(run.step, ms, n=args.rounds, start=args.steps + args.warmup,
                          monitor=monitor) if args.rounds > 0 else None)
    graph_ms = (None if args.no_graph else
                graph_replay_ms(run, calls=100, replays=max(5, int(0.1 / (ms * 1e-3) / 100))))
    hot = Runner(w, 0, host)
    hot_ms = time_steps(hot.step, max(args.steps // 2, 10), max(args.warmup // 2, 5))
    del hot
    calib = copy_calibration(2 * w.M * w.N * w.esize, args.rotate_bytes)
    calib16 = copy16_calibration(2 * w.M * w.N * w.esize, args.rotate_bytes)
    read16 = mix_calibration(rbytes, 0, args.rotate_bytes)
    write16 = mix_calibration(0, wbytes, args.rotate_bytes)
    ceiling = mix_calibration(rbytes, wbytes, args.rotate_bytes)

    result = {
        "metric": "achieved HBM GB/s (% of MI355X peak) and rows/s, RMSNorm fwd/bwd",
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded SplitMix64/Box-Muller, inputs resident in HBM)",
        "config": {"workload": w.name, "kind": w.kind, "M": w.M, "N": w.N,
                   "io_dtype": DT_NAMES[w.x_dt], "gamma_dtype": DT_NAMES[w.g_dt], "eps": w.eps,
                   "rstd_out": w.store_rstd, "rotation_replicas": run.replicas,
                   "algorithmic_bytes_per_step": nbytes, "read_bytes": rbytes,
                   "write_bytes": wbytes},
        "rows_per_s": round(rows_of(w) / (ms * 1e-3), 1),
        "pct_of_peak": round(100 * gbps / PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / PEAK_GBPS, 4),
                     "traffic": load_traffic(w.name, src_hash),
                     "kernel": DOMINANT_KERNEL.get(w.name, w.kind),
                     "kernel_src_hash": src_hash},
        "ceiling": ceiling,
        "frac_of_ceiling": round(gbps / ceiling["gbps"], 4) if ceiling else None,
        "graph": None if graph_ms is None else {
            "calls_per_graph": 100, "ms_per_step": round(graph_ms, 6),
            "gbps": round(nbytes / (graph_ms * 1e-3) / 1e9, 2),
            "pct_of_peak": round(100 * nbytes / (graph_ms * 1e-3) / 1e9 / PEAK_GBPS, 2),
            "what": "the same step, 100 calls over the rotation replicas captured in one HIP "
                    "graph and replayed (no host launch per call)"},
        "hot_cache_gbps": round(nbytes / (hot_ms * 1e-3) / 1e9, 2),
        "rounds": round_stats,
        "calibration": {
            "copy_gbps": round(calib, 2),
            "what": "torch device-to-device copy, same read+write bytes, rotated",
            "copy16_gbps": round(calib16, 2) if calib16 else None,
            "copy16_what": "16-byte non-temporal copy kernel (librmsn_copy16.so), same read+"
                           "write bytes, rotated, one allocation per operand",
            "value_over_copy16": round(gbps / calib16, 4) if calib16 else None,
            "read16_gbps": read16["gbps"] if read16 else None,
            "write16_gbps": write16["gbps"] if write16 else None,
            "read_write_what": "16-byte non-temporal read-only and write-only streams of the "
                               "step's read and write bytes, rotated (librmsn_copy16.so "
                               "rmsn_calib_mix 1:0 and 0:1)",
            "read_then_write_us": (round(1e6 * (rbytes / (read16["gbps"] * 1e9) +
                                               wbytes / (write16["gbps"] * 1e9)), 3)
                                   if read16 and write16 else None)},
    }
    outs = None if args.no_cpu else run.pristine_outputs(host)
    del run
    torch.cuda.empty_cache()

    if not args.no_others:
        others = {}
        for ow in G.WORKLOADS + G.EXTRA_WORKLOADS:
            if ow.name == w.name:
                continue
            oh = G.make_inputs(ow)
            small = ow.M * ow.N < (1 << 20)
            orun = Runner(ow, 0 if small else args.rotate_bytes, oh)
            est = max(ow.algorithmic_bytes() / 6e12, 3e-6)
            k = args.other_steps or int(min(2000, max(50, 0.05 / est)))
            monitor.idle(f"{ow.name} before")
            oms = time_steps(orun.step, k, max(k // 10, 5))
            monitor.idle(f"{ow.name} after")
            ob = ow.algorithmic_bytes()
            ogbps = ob / (oms * 1e-3) / 1e9
            others[ow.name] = {"ms_per_step": round(oms, 6), "gbps": round(ogbps, 2),
                               "pct_of_peak": round(100 * ogbps / PEAK_GBPS, 2),
                               "rows_per_s": round(rows_of(ow) / (oms * 1e-3), 1),
                               "steps": k, "rotation_replicas": orun.replicas}
            if ow.kind in ("bwd", "fused_add_bwd", "ln_bwd"):
                others[ow.name]["workspace_bytes"] = orun.ws_bytes
            if small:
                # Launch-bound: the same call replayed from a captured graph.
                gms = graph_replay_ms(orun)
                others[ow.name]["graph"] = {
                    "calls_per_graph": 100, "ms_per_step": round(gms, 6),
                    "gbps": round(ob / (gms * 1e-3) / 1e9, 2),
                    "pct_of_peak": round(100 * ob / (gms * 1e-3) / 1e9 / PEAK_GBPS, 2),
                    "rows_per_s": round(rows_of(ow) / (gms * 1e-3), 1)}
            oouts = None if args.no_cpu else orun.pristine_outputs(oh)
            del orun
            torch.cuda.empty_cache()
            o = others[ow.name]
            if not small:
                # The matching stream: the workload's read and write bytes in
                # (about) its ratio, 16-byte non-temporal, rotated.
                ocr, ocw = ow.read_write_bytes()
                c = mix_calibration(ocr, ocw, args.rotate_bytes)
                if c is not None:
                    o["ceiling"] = c
                    o["frac_of_ceiling"] = round(ogbps / c["gbps"], 4)
                torch.cuda.empty_cache()
            if ow.kind in ("bwd", "fused_add_bwd", "ln_bwd"):
                # The same read and write streams with no arithmetic: two
                # inputs per output (x, dy -> dx), three for the fused add's.
                nin = 3 if ow.kind == "fused_add_bwd" else 2
                sg = stream_calibration(ow.M * ow.N * ow.esize, nin, args.rotate_bytes)
                if sg is not None:
                    o["stream_gbps"] = round(sg, 2)
                    o["stream_what"] = (f"{nin} reads + 1 write of {ow.M}x{ow.N} {DT_NAMES[ow.x_dt]}, "
                                        "16-byte non-temporal, rotated (librmsn_copy16.so)")
                    o["value_over_stream"] = round(o["gbps"] / sg, 4)
                torch.cuda.empty_cache()
            if not args.no_cpu:
                o["cpu_baseline"] = cpu_baseline(ow, oh, 0.0, best_of=3 if small else 1)
                o["parity"] = parity_check(ow, oouts, oh)
            del oh, oouts
        result["workloads"] = others

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, host, args.cpu_seconds)
        result["parity"] = parity_check(w, outs, host)
    result["idle_check"] = monitor.summary()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
