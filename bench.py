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
  rounds        five more timing rounds of the step (>= 20 ms each after a
                50 ms warm-up, 1 s cool-down): median / min / mean us, spread;
  calibration   plain copies of the step's byte count: torch's device-to-device
                copy, and a 16-byte non-temporal copy kernel
                (librmsn_copy16.so, the practical ceiling for equal read and
                write bytes), with value / copy16.
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


def copy16_calibration(nbytes: int, rotate_bytes: float, steps: int = 200):
    """GB/s of the 16-byte non-temporal copy kernel (librmsn_copy16.so) moving
    nbytes (read + write) per step over rotated buffers laid out like the
    workloads' (one [R, bytes] allocation per operand); None if not built."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "row_wise_normalization_fwd_amd", "librmsn_copy16.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.rmsn_calib_copy16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_void_p]
    lib.rmsn_calib_copy16.restype = ctypes.c_int
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
    import ctypes

    import torch
    path = os.path.join(ROOT, "row_wise_normalization_fwd_amd", "librmsn_copy16.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.rmsn_calib_stream.argtypes = [vp, vp, vp, vp, ctypes.c_int64, vp]
    lib.rmsn_calib_stream.restype = ctypes.c_int
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


def graph_replay_ms(run, calls: int = 100, replays: int = 40) -> float:
    """Milliseconds per step when `calls` steps are captured in one HIP graph
    (torch.cuda.CUDAGraph) and the graph is replayed: the GPU's own rate for a
    launch-bound step, without a host launch per call."""
    import torch
    fn, args = run.calls[0]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        cargs = args[:-1] + (side.cuda_stream,)
        with torch.cuda.graph(graph, stream=side):
            for _ in range(calls):
                if fn(*cargs) != 0:
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
    return start.elapsed_time(end) / (replays * calls)


def rounds(step, ms_per_step: float, n: int = 5, cooldown_s: float = 1.0, start: int = 0):
    """n further timing rounds of the same step, each >= 20 ms of back-to-back
    launches after a >= 50 ms warm-up, with a cool-down before each round:
    median, min and mean microseconds per step and the spread."""
    import statistics
    k = max(50, int(0.020 / (ms_per_step * 1e-3)) + 1)
    warm = max(10, int(0.050 / (ms_per_step * 1e-3)) + 1)
    us = []
    i = start
    for r in range(n):
        time.sleep(cooldown_s)
        us.append(1e3 * time_steps(lambda j: step(i + j), k, warm if r == 0 else 10))
        i += k + warm
    med = statistics.median(us)
    return {"rounds": n, "steps_per_round": k, "cooldown_s": cooldown_s,
            "us_median": round(med, 3), "us_min": round(min(us), 3),
            "us_mean": round(statistics.fmean(us), 3),
            "spread_pct": round(100 * (max(us) - min(us)) / med, 2)}


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


def cpu_baseline(w, host_inputs: dict, seconds: float) -> dict:
    """The fp64 oracle, as it stands, timed on one host core."""
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
    passes, t0 = 0, time.perf_counter()
    while True:
        one_pass()
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(w.algorithmic_bytes() * passes / el / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{passes} full passes over the {M}x{N} batch ({el:.1f} s, single thread,"
                      f" host has {os.cpu_count()} logical CPUs)",
            "rows_per_s": round(M * passes / el, 1),
            "ms_per_pass": round(1e3 * el / passes, 3),
            "host_cpu": _cpu_model()}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
    args = ap.parse_args()

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
    src_hash = kernel_source_hash()

    w = G.WORKLOADS_BY_NAME[args.workload]
    host = G.make_inputs(w)
    run = Runner(w, args.rotate_bytes, host)
    ms = time_steps(run.step, args.steps, args.warmup)
    nbytes = w.algorithmic_bytes()
    gbps = nbytes / (ms * 1e-3) / 1e9
    round_stats = (rounds(run.step, ms, n=args.rounds, start=args.steps + args.warmup)
                   if args.rounds > 0 else None)
    hot = Runner(w, 0, host)
    hot_ms = time_steps(hot.step, max(args.steps // 2, 10), max(args.warmup // 2, 5))
    del hot
    calib = copy_calibration(2 * w.M * w.N * w.esize, args.rotate_bytes)
    calib16 = copy16_calibration(2 * w.M * w.N * w.esize, args.rotate_bytes)

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
                   "algorithmic_bytes_per_step": nbytes},
        "rows_per_s": round(rows_of(w) / (ms * 1e-3), 1),
        "pct_of_peak": round(100 * gbps / PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / PEAK_GBPS, 4),
                     "traffic": load_traffic(w.name, src_hash),
                     "kernel": DOMINANT_KERNEL.get(w.name, w.kind),
                     "kernel_src_hash": src_hash},
        "hot_cache_gbps": round(nbytes / (hot_ms * 1e-3) / 1e9, 2),
        "rounds": round_stats,
        "calibration": {
            "copy_gbps": round(calib, 2),
            "what": "torch device-to-device copy, same read+write bytes, rotated",
            "copy16_gbps": round(calib16, 2) if calib16 else None,
            "copy16_what": "16-byte non-temporal copy kernel (librmsn_copy16.so), same read+"
                           "write bytes, rotated, one allocation per operand",
            "value_over_copy16": round(gbps / calib16, 4) if calib16 else None},
    }
    del run
    torch.cuda.empty_cache()

    if not args.no_others:
        others = {}
        for ow in G.WORKLOADS + G.EXTRA_WORKLOADS:
            if ow.name == w.name:
                continue
            oh = G.make_inputs(ow)
            orun = Runner(ow, 0 if ow.M * ow.N < (1 << 20) else args.rotate_bytes, oh)
            est = max(ow.algorithmic_bytes() / 6e12, 3e-6)
            k = args.other_steps or int(min(2000, max(50, 0.05 / est)))
            oms = time_steps(orun.step, k, max(k // 10, 5))
            ob = ow.algorithmic_bytes()
            others[ow.name] = {"ms_per_step": round(oms, 6), "gbps": round(ob / (oms * 1e-3) / 1e9, 2),
                               "pct_of_peak": round(100 * ob / (oms * 1e-3) / 1e9 / PEAK_GBPS, 2),
                               "rows_per_s": round(rows_of(ow) / (oms * 1e-3), 1),
                               "steps": k, "rotation_replicas": orun.replicas}
            if ow.kind in ("bwd", "fused_add_bwd", "ln_bwd"):
                others[ow.name]["workspace_bytes"] = orun.ws_bytes
            if ow.M * ow.N < (1 << 20):
                # Launch-bound: the same call replayed from a captured graph.
                gms = graph_replay_ms(orun)
                others[ow.name]["graph"] = {
                    "calls_per_graph": 100, "ms_per_step": round(gms, 6),
                    "gbps": round(ob / (gms * 1e-3) / 1e9, 2),
                    "pct_of_peak": round(100 * ob / (gms * 1e-3) / 1e9 / PEAK_GBPS, 2),
                    "rows_per_s": round(rows_of(ow) / (gms * 1e-3), 1)}
            del orun, oh
            torch.cuda.empty_cache()
            if ow.kind in ("bwd", "fused_add_bwd", "ln_bwd"):
                # The same read and write streams with no arithmetic: two
                # inputs per output (x, dy -> dx), three for the fused add's.
                nin = 3 if ow.kind == "fused_add_bwd" else 2
                sg = stream_calibration(ow.M * ow.N * ow.esize, nin, args.rotate_bytes)
                if sg is not None:
                    o = others[ow.name]
                    o["stream_gbps"] = round(sg, 2)
                    o["stream_what"] = (f"{nin} reads + 1 write of {ow.M}x{ow.N} {DT_NAMES[ow.x_dt]}, "
                                        "16-byte non-temporal, rotated (librmsn_copy16.so)")
                    o["value_over_stream"] = round(o["gbps"] / sg, 4)
                torch.cuda.empty_cache()
        result["workloads"] = others

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, host, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
