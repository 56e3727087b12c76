// Forward kernel choice and launch for one activation type. Included by one
// translation unit per activation type so the instantiations compile in
// parallel.
//
// Register path (N <= 8192): a group of TPR lanes per row with UPT units per
// lane. TPR = next power of two of ceil(units / 2), so each lane moves two
// 16-byte units per operand (measured best at 4096 x 8192 bf16 among 1, 2, 4
// and 8 units per lane, with or without a prefetching persistent loop), and
// rows of up to 1024 units use up to 512 lanes; longer register rows (fp32,
// N <= 8192) use 4 units on 512 lanes. Whenever the row fits half the lanes
// with 3 units each, that is used instead, leaving fewer lanes idle (at
// 32768 x 5000 fp16, 625 units: 256 x 3 measured 7% faster than 512 x 2;
// bf16 16384 x 5632 61.1-61.4 us vs 77.4-78.1, 16384 x 6144 66.4-67.1 vs
// 77.9-78.7, 32768 x 2816 +5.5%, 65536 x 1408 +6%, 1536 +2.6%, fp32 2816
// +1.4%, against 2 units on the full lanes; LayerNorm, fp8 and MX outputs
// 10-40% at 2816, 5632 and 6144 bf16; not the fused add, see below). Short
// rows pack BLOCK / TPR rows per block. Rows that are not 16-byte aligned use 1-element units (up to 8 per
// lane). Non-fused 16-bit rows of 769 to 1024 units (N in (6144, 8192]) use
// the persistent fwd_pp_kernel instead (4096 x 8192 bf16: 22.0-22.6 us vs
// 23.7-24.0 us; it did not help the fused add or 625-unit rows), and so do
// plain rows of 1537..4096 units (N in (12288, 32768] 16-bit, (8192, 16384]
// fp32) with 512 or 1024 lanes per row. Other longer rows:
// one block per row, parked in LDS when the row fits the
// device's per-workgroup LDS (160 KiB on gfx950), else re-read; 512 threads
// for rows up to 32 KiB, 1024 above (measured at 128 MiB of bf16: 16384-
// element rows 46 us with 512 threads vs 48 us with 256; 32768 and 65536
// elements 48-50 us with 1024 threads and 64 / 128 KiB of LDS vs 61-63 us
// re-reading). At most CUs / 2 rows too long for LDS take the split path
// instead (a block per tile of the row, three launches; fwd_split.hpp).
#pragma once

#include "fwd_kernels.hpp"
#include "fwd_split.hpp"
#include "rare_row.hpp"
#include "launch.hpp"

namespace rmsn {

template <class T, class G, bool VEC, int TPR, int UPT, int BLOCK, bool FUSED, int OUT, bool LN>
hipError_t run_fwd_reg(const FwdArgs<T, G>& a, hipStream_t s) {
  constexpr int RPB = BLOCK / TPR;
  int64_t blocks = ceil_div(a.M, RPB);
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  // At most kMaxRowIters loop iterations per row group (one bit each in the
  // kernel's rare-row mask).
  const int64_t min_blocks = ceil_div(a.M, RPB * kMaxRowIters);
  if (blocks < min_blocks) blocks = min_blocks;
  fwd_reg_kernel<T, G, VEC, TPR, UPT, BLOCK, FUSED, OUT, LN>
      <<<dim3(static_cast<unsigned>(blocks)), dim3(BLOCK), 0, s>>>(a);
  return hipGetLastError();
}

template <class T, class G, int TPR, int UPT, int BLOCK, bool FUSED, int OUT, bool LN>
hipError_t run_fwd_pp(const FwdArgs<T, G>& a, hipStream_t s) {
  // Two blocks per CU's worth of grid: at 4096 x 8192 bf16 every block then
  // runs exactly two iterations (one prefetch), measured best among 256-1024
  // blocks. 1024-thread blocks (one resident per CU) with at most three row
  // groups per CU take one block per CU instead, so all of them run at once
  // and each still prefetches (bf16 x 8192: 1536 rows 10.0 vs 12.2 us, 2048
  // 11.0 vs 14.1, 3072 17.2 vs 19.3; 1024 x 16384 10.9 vs 13.4; 512 x 32768
  // 11.8 vs 13.3; from 3584 rows of 8192 two per CU are ahead again).
  constexpr int RG = BLOCK / TPR;
  const int64_t groups = ceil_div(a.M, RG);
  const int64_t cus = device_cus();
  int64_t blocks = BLOCK == 1024 && groups <= 3 * cus ? cus : 2 * cus;
  if (blocks > groups) blocks = groups;
  // At most kMaxRowIters iterations per row group (the rare-row mask).
  if (blocks < ceil_div(groups, kMaxRowIters)) blocks = ceil_div(groups, kMaxRowIters);
  constexpr size_t lds = pp_param_lds_bytes<T, G, TPR, UPT, BLOCK, LN>();
  constexpr auto kernel = fwd_pp_kernel<T, G, TPR, UPT, BLOCK, FUSED, OUT, LN>;
  if constexpr (lds > 0) {
    const hipError_t attr = ensure_dynamic_lds<kernel>(lds);
    if (attr != hipSuccess) return attr;
  }
  kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(BLOCK), lds, s>>>(a);
  return hipGetLastError();
}

template <class T, class G, bool VEC, int BLOCK, int UNROLL, bool FUSED, bool CACHE, int OUT,
          bool LN>
hipError_t run_fwd_long(const FwdArgs<T, G>& a, hipStream_t s) {
  int64_t blocks = a.M < kMaxGrid ? a.M : kMaxGrid;
  const size_t lds = CACHE ? static_cast<size_t>(a.N) * T::kSize : 0;
  constexpr auto kernel = fwd_long_kernel<T, G, VEC, BLOCK, UNROLL, FUSED, CACHE, OUT, LN>;
  if constexpr (CACHE) {
    // Allow the largest row cache once; per-launch sizes stay below it.
    const hipError_t attr =
        ensure_dynamic_lds<kernel>(static_cast<size_t>(lds_row_budget()));
    if (attr != hipSuccess) return attr;
  }
  kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(BLOCK), lds, s>>>(a);
  return hipGetLastError();
}

// Few rows too long for the LDS row cache: partials, finalize, apply (see
// fwd_split.hpp). Three launches against one block per row at bf16 (one
// process):
// 256K-element rows 2.0-2.4x faster up to 16 rows, even at 128; 1M-element
// rows 3-11x up to 32 rows, 1.5x at 128; 16M-element rows 8-51x. Rows that
// fit the cache stay with one block per row (the split path's three launches
// cost ~10 us there against 7-8).
template <class T, class G, bool FUSED, bool SPREAD, bool CACHE>
hipError_t run_fwd_split_as(const SplitArgs<T, G>& a, hipStream_t s) {
  const int64_t blocks = a.tiles < kMaxGrid ? a.tiles : kMaxGrid;
  fwd_split_partial_kernel<T, G, FUSED, SPREAD, CACHE>
      <<<dim3(static_cast<unsigned>(blocks)), dim3(kSplitBlock), 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (!SPREAD) {
    int64_t fblocks = ceil_div(a.M, kSplitBlock / kWave);
    if (fblocks > kMaxGrid) fblocks = kMaxGrid;
    fwd_split_finalize_kernel<T, G, FUSED>
        <<<dim3(static_cast<unsigned>(fblocks)), dim3(kSplitBlock), 0, s>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  fwd_split_apply_kernel<T, G, FUSED, SPREAD>
      <<<dim3(static_cast<unsigned>(blocks)), dim3(kSplitBlock), 0, s>>>(a);
  return hipGetLastError();
}

// Two launches (the partials spread to every tile of the row, each apply
// block forming the row's factor itself) when every tile region, the last
// included, holds a float per tile of the row and the partial pass writes
// nothing that it or another block still reads (y is not x); else three.
// x is loaded cacheable in the partial pass when the batch is at most 16 MiB,
// so that the apply pass's second read can come from the Infinity Cache
// (3-11% faster there, 10% slower at 32 MiB, in one process).
template <class T, class G, bool FUSED>
hipError_t run_fwd_split(const FwdArgs<T, G>& f, hipStream_t s) {
  SplitArgs<T, G> a{f.x, f.residual, f.gamma, f.y, f.rstd, f.M, f.N, f.eps, 0, 0};
  a.chunks = static_cast<int>(ceil_div(f.N, split_chunk<T>()));
  a.tiles = f.M * a.chunks;
  const int64_t last = f.N - static_cast<int64_t>(a.chunks - 1) * split_chunk<T>();
  const bool spread = last * T::kSize >= 4 * static_cast<int64_t>(a.chunks) &&
                      static_cast<const void*>(f.y) != static_cast<const void*>(f.x);
  const bool cache = !FUSED && f.M * static_cast<int64_t>(f.N) * T::kSize <= (int64_t(16) << 20);
  if (spread) {
    return cache ? run_fwd_split_as<T, G, FUSED, true, !FUSED>(a, s)
                 : run_fwd_split_as<T, G, FUSED, true, false>(a, s);
  }
  return cache ? run_fwd_split_as<T, G, FUSED, false, !FUSED>(a, s)
               : run_fwd_split_as<T, G, FUSED, false, false>(a, s);
}

template <class T, class G, bool FUSED, int OUT, bool LN = false>
hipError_t fwd_typed(const FwdCall& c) {
  FwdArgs<T, G> a;
  a.x = static_cast<const typename T::S*>(c.x);
  a.residual = static_cast<typename T::S*>(c.residual);
  a.gamma = static_cast<const typename G::S*>(c.gamma);
  a.y = static_cast<typename T::S*>(c.y);
  a.rstd = c.rstd;
  a.M = c.M;
  a.N = static_cast<int>(c.N);
  a.eps = c.eps;
  a.q = static_cast<uint8_t*>(c.q);
  a.scale = c.scale;
  a.beta = static_cast<const typename G::S*>(c.beta);
  a.mean = c.mean;
  a.mx = c.mx;
  hipStream_t s = c.stream;

  // fp8 output units are 16 / sizeof(T) bytes (8 or 4), fp4 half that, each
  // stored with one instruction, so q must be aligned to that.
  constexpr int kE = 16 / T::kSize;
  const bool out_ok = OUT == kOutAct ? aligned16(c.y)
                                     : aligned_to(c.q, OUT == kOutMxFp4 ? kE / 2 : kE);
  const bool vec = (c.N * T::kSize) % 16 == 0 && aligned16(c.x) && out_ok &&
                   aligned16(c.gamma) && (!FUSED || aligned16(c.residual)) &&
                   (!LN || c.beta == nullptr || aligned16(c.beta));
  // MX outputs need the 16-byte unit path (the host checks the alignment).
  if constexpr (kIsMx<OUT>) {
    if (!vec) return hipErrorInvalidValue;
  }
  if (c.N <= kRegMaxN) {
    if (vec) {
      constexpr int E = 16 / T::kSize;
      const int64_t units = c.N / E;
      if (units > 1024) return run_fwd_reg<T, G, true, 512, 4, 512, FUSED, OUT, LN>(a, s);
      if constexpr (T::kSize == 2 && !FUSED) {
        // 16-bit rows of 769..1024 units: persistent kernel with next-row
        // prefetch; four 256-lane row groups per block for 16-bit outputs,
        // one per block for fp8 outputs (4096 x 8192 bf16, fp8 per-row
        // scales: 18.1 us vs 21.4 us with four; one scale: 17.7 vs 20.4 us;
        // bf16 output: 22.9 vs 23.5 us the other way).
        // LayerNorm keeps beta and the mean live too and spills with four
        // row groups, so it also takes the one-group shape.
        if (units > 768) {
          if constexpr (OUT == kOutAct && !LN) {
            // Beyond 16 rows per CU the persistent grid needs several rounds
            // of blocks, and one 256-lane row per block of the register
            // kernel is faster (bf16 x 8192: 6144 rows 34.6 vs 35.6 us,
            // 12288 65.8 vs 68.6, 16384 86.6-87.4 vs 91.9-92.6; x 7168, 12288
            // rows 58.6 vs 64.2), while at 4096 rows it is 7-8% slower.
            if (a.M > 16 * device_cus()) return run_fwd_reg<T, G, true, 256, 4, 256, FUSED, OUT, LN>(a, s);
            return run_fwd_pp<T, G, 256, 4, 1024, FUSED, OUT, LN>(a, s);
          }
          else return run_fwd_pp<T, G, 256, 4, 256, FUSED, OUT, LN>(a, s);
        }
      }
      if constexpr (T::kSize == 2 && !FUSED && (LN || OUT != kOutAct)) {
        // LayerNorm, fp8 and MX outputs of shorter rows (64..256 lanes of the
        // register kernel's shape): the persistent kernel, one row group per
        // 256-thread block (or several for narrower groups), measured against the register kernel at 64 MiB
        // of bf16 per operand, alternating in one process: LayerNorm 3-30%
        // faster from 1024 to 6144 elements (2560: 26.7 vs 33.4 us, 5120:
        // 25.7 vs 33.4), so it takes every such shape; MX 10-18% faster on
        // the three-unit shapes (1536, 2560, 3072, 5120, 6144) but 3-4%
        // slower on the two-unit ones, fp8 2-6% faster on three units and
        // 7-11% slower on two, so those take only the three-unit shapes.
        const int64_t t2 = next_pow2(ceil_div(units, 2));
        const bool th = t2 >= 8 && units <= 3 * (t2 / 2);
        const int64_t tp = th ? t2 / 2 : t2;
        if constexpr (!LN) {
          // fp8 / MX rows of a two-unit shape on 64, 128 or 256 lanes: four
          // units on half the lanes of the persistent kernel (MXFP4 2048 /
          // 3584 / 4096 elements 10-13% faster, fp8 0.4 / 3 / 8%; the
          // register kernel with four units lost 4-11%; at 1024 elements and
          // 64 MiB per operand fp8 per-row 7.8%, MXFP4 10.9%, MXFP8 6.9%,
          // within 1% or better at 16 MiB). 16 and 32 lanes (256, 512
          // elements) lost 2-29% that way.
          if (!th && (tp == 64 || tp == 128 || tp == 256)) {
            if (tp == 64) return run_fwd_pp<T, G, 32, 4, 256, FUSED, OUT, LN>(a, s);
            if (tp == 128) return run_fwd_pp<T, G, 64, 4, 256, FUSED, OUT, LN>(a, s);
            return run_fwd_pp<T, G, 128, 4, 256, FUSED, OUT, LN>(a, s);
          }
        }
        // LayerNorm's three-unit shapes of 16 and 32 lanes too (384 elements
        // 27.4 vs 28.9 us, 640 26.1 vs 31.5, 768 25.4 vs 27.8); its two-unit
        // shapes there lost 5-7% (256, 512) and stay on the register kernel.
        if (tp >= (LN && th ? 16 : 64) && tp <= 256 && (LN || th)) {
          if (th) {
            switch (tp) {
              case 16: return run_fwd_pp<T, G, 16, 3, 256, FUSED, OUT, LN>(a, s);
              case 32: return run_fwd_pp<T, G, 32, 3, 256, FUSED, OUT, LN>(a, s);
              case 64: return run_fwd_pp<T, G, 64, 3, 256, FUSED, OUT, LN>(a, s);
              case 128: return run_fwd_pp<T, G, 128, 3, 256, FUSED, OUT, LN>(a, s);
              default: return run_fwd_pp<T, G, 256, 3, 256, FUSED, OUT, LN>(a, s);
            }
          }
          if constexpr (LN) {
            switch (tp) {
              case 64: return run_fwd_pp<T, G, 64, 2, 256, FUSED, OUT, LN>(a, s);
              case 128: return run_fwd_pp<T, G, 128, 2, 256, FUSED, OUT, LN>(a, s);
              default: return run_fwd_pp<T, G, 256, 2, 256, FUSED, OUT, LN>(a, s);
            }
          }
        }
      }
      // MX blocks span 32 / E lanes of one unit slot: at least that many lanes.
      constexpr int64_t kMinTpr = kIsMx<OUT> ? 32 / E : 1;
      int64_t tpr2 = next_pow2(ceil_div(units, 2));
      if (tpr2 < kMinTpr) tpr2 = kMinTpr;
      // Three units on half the lanes whenever the row fits them; the fused
      // add only where two units would idle over a third of the lanes (three
      // measured 1-4.5% slower for it at 2816, 5632 and 6144 bf16).
      const bool three = units <= 3 * (tpr2 / 2) && (!FUSED || 3 * units < 4 * tpr2);
      if (tpr2 / 2 >= kMinTpr && tpr2 >= 8 && three) {
        switch (tpr2 / 2) {  // 3 units on half the lanes
          case 4: return run_fwd_reg<T, G, true, 4, 3, 256, FUSED, OUT, LN>(a, s);
          case 8: return run_fwd_reg<T, G, true, 8, 3, 256, FUSED, OUT, LN>(a, s);
          case 16: return run_fwd_reg<T, G, true, 16, 3, 256, FUSED, OUT, LN>(a, s);
          case 32: return run_fwd_reg<T, G, true, 32, 3, 256, FUSED, OUT, LN>(a, s);
          case 64: return run_fwd_reg<T, G, true, 64, 3, 256, FUSED, OUT, LN>(a, s);
          case 128: return run_fwd_reg<T, G, true, 128, 3, 256, FUSED, OUT, LN>(a, s);
          default: return run_fwd_reg<T, G, true, 256, 3, 256, FUSED, OUT, LN>(a, s);
        }
      }
      switch (tpr2) {
        case 1: return run_fwd_reg<T, G, true, 1, 2, 256, FUSED, OUT, LN>(a, s);
        case 2: return run_fwd_reg<T, G, true, 2, 2, 256, FUSED, OUT, LN>(a, s);
        case 4: return run_fwd_reg<T, G, true, 4, 2, 256, FUSED, OUT, LN>(a, s);
        case 8: return run_fwd_reg<T, G, true, 8, 2, 256, FUSED, OUT, LN>(a, s);
        case 16: return run_fwd_reg<T, G, true, 16, 2, 256, FUSED, OUT, LN>(a, s);
        case 32: return run_fwd_reg<T, G, true, 32, 2, 256, FUSED, OUT, LN>(a, s);
        case 64: return run_fwd_reg<T, G, true, 64, 2, 256, FUSED, OUT, LN>(a, s);
        case 128: return run_fwd_reg<T, G, true, 128, 2, 256, FUSED, OUT, LN>(a, s);
        case 256: return run_fwd_reg<T, G, true, 256, 2, 256, FUSED, OUT, LN>(a, s);
        default: return run_fwd_reg<T, G, true, 512, 2, 512, FUSED, OUT, LN>(a, s);
      }
    }
    if constexpr (!kIsMx<OUT>) {
      const int64_t tpr = next_pow2(ceil_div(c.N, 8));
      if (tpr <= 16) return run_fwd_reg<T, G, false, 16, 8, 256, FUSED, OUT, LN>(a, s);
      if (tpr <= 64) return run_fwd_reg<T, G, false, 64, 8, 256, FUSED, OUT, LN>(a, s);
      if (tpr <= 256) return run_fwd_reg<T, G, false, 256, 8, 256, FUSED, OUT, LN>(a, s);
      return run_fwd_reg<T, G, false, 1024, 8, 1024, FUSED, OUT, LN>(a, s);
    }
  }
  if constexpr (T::kSize == 2) {
    // 16-bit rows of 1025..1536 units (N in (8192, 12288]): the fused add on
    // 512 lanes of three units (bf16 8192 x 10240 108.0 vs 112.5-112.9 us
    // on the LDS-row kernel, 4096 x 12288 66.9 vs 68.9); LayerNorm, fp8 and
    // MX outputs on the persistent kernel, one 512-lane group of three units
    // per block (LayerNorm 10240 59.1 vs 73.7-74.3 us, 8200 49.8-50.2 vs
    // 64.2-67.2; per-row fp8 10240 49.1-49.4 vs 61.3-62.8, 12288 28.0-28.4
    // vs 37.0-37.3; MXFP4 10240 42.8-43.9 vs 55.3-56.6, 8224 38.8-38.9 vs
    // 50.9-51.5). The plain forward stays on the LDS-row kernel, which both
    // of those shapes lost to (3-9% at 8200 and 10240).
    if (vec) {
      const int64_t units = c.N / 8;
      if (units > 1024 && units <= 1536) {
        if constexpr (FUSED && OUT == kOutAct) {
          return run_fwd_reg<T, G, true, 512, 3, 512, FUSED, OUT, LN>(a, s);
        } else if constexpr (!FUSED && (LN || OUT != kOutAct)) {
          return run_fwd_pp<T, G, 512, 3, 512, FUSED, OUT, LN>(a, s);
        }
      }
    }
  }
  if constexpr (!FUSED && OUT == kOutAct && !LN) {
    // Rows of 1537..4096 16-byte units: the persistent kernel with 512 or
    // 1024 lanes per row and three or four units per lane, chosen to leave
    // few lanes idle. Against the LDS-row kernel, alternating in one process
    // (rows rotated over >= 1 GiB): bf16 2048 x 16384 22.0-22.2 us vs
    // 24.7-24.9, 2048 x 24576 35.8-36.0 vs 37.3-37.5, 1024 x 32768 23.3-23.5
    // vs 25.4-25.6, 20480 and 14000 +1-2%; fp32 4096 x 8196 47.7-47.9 vs
    // 52.1-52.9, 2048 x 12288 +4%, 16384 +0.6%. Shorter rows stay with the
    // LDS-row kernel: 512 lanes of three units lost 5-7% at 8200 and 10000
    // bf16 elements and gained 1.7% only at a full 12288.
    if (vec) {
      const int64_t units = c.N / (16 / T::kSize);
      if (units > 1536 && units <= 2048) return run_fwd_pp<T, G, 512, 4, 1024, FUSED, OUT, LN>(a, s);
      if (units > 2048 && units <= 3072) return run_fwd_pp<T, G, 1024, 3, 1024, FUSED, OUT, LN>(a, s);
      if (units > 3072 && units <= 4096) return run_fwd_pp<T, G, 1024, 4, 1024, FUSED, OUT, LN>(a, s);
    }
  } else if constexpr (T::kSize == 2) {
    // The other 16-bit outputs of rows of 1537..4096 units, where measured
    // faster than the LDS-row kernel (bf16, 2048 x 16384 / 2048 x 24576 /
    // 1024 x 32768, alternating in one process): the fused add with 1024
    // lanes of four units (32768: 48.7-49.3 us vs 50.8-50.9; three units
    // gained 1% at 24576 and lost 3.5% at 16384, so shorter rows stay);
    // LayerNorm with one 512-lane group of four units per block or 1024
    // lanes of three (26.6 vs 29.2 us, 38.7-39.1 vs 44.9-46.2; four units
    // spill); fp8 (18.7 vs 25.7 us, 31.3 vs 46.1-46.7) and MX outputs (MXFP4
    // 17.3-17.5 vs 21.6, 28.1-28.3 vs 37.9-38.7, 22.0-22.2 vs 25.7-25.9) with
    // the same shapes, and both with 1024 lanes of four (per-row fp8 1170 x
    // 28672 26.3 vs 31.6 us, 1232 x 26624 26.7 vs 30.6; per-tensor 6% faster).
    // LayerNorm with 16-bit gamma takes 1024 lanes of four (gamma and beta in
    // LDS) when at least 7/8 of the lanes' units hold the row: 1024 x 32768
    // 28.8-29.3 vs 32.7-33.9 us, 1170 x 28672 29.5-30.1 vs 31.0-31.2, but
    // 1290 x 26000 (3250 units) 34.7-36.4 vs 33.0-34.7. Not the fused add
    // into fp8 / MX.
    if (vec) {
      const int64_t units = c.N / 8;
      if constexpr (FUSED && OUT == kOutAct) {
        if (units > 3072 && units <= 4096) return run_fwd_pp<T, G, 1024, 4, 1024, FUSED, OUT, LN>(a, s);
      } else if constexpr (!FUSED) {
        if (units > 1536 && units <= 2048) return run_fwd_pp<T, G, 512, 4, 512, FUSED, OUT, LN>(a, s);
        if (units > 2048 && units <= 3072) return run_fwd_pp<T, G, 1024, 3, 1024, FUSED, OUT, LN>(a, s);
        if constexpr (OUT != kOutAct) {
          if (units > 3072 && units <= 4096) return run_fwd_pp<T, G, 1024, 4, 1024, FUSED, OUT, LN>(a, s);
        } else if constexpr (LN && G::kSize == 2) {
          if (units >= 3584 && units <= 4096) return run_fwd_pp<T, G, 1024, 4, 1024, FUSED, OUT, LN>(a, s);
        }
      }
    }
  }
  const int64_t row_bytes = c.N * T::kSize;
  const bool cache = row_bytes <= lds_row_budget();
  if constexpr (OUT == kOutAct && !LN) {
    // y holds the split path's partials, so it must not be x itself.
    if (vec && !cache && (FUSED || c.y != c.x) && c.M <= device_cus() / 2)
      return run_fwd_split<T, G, FUSED>(a, s);
  }
  if (vec) {
    if (!cache) return run_fwd_long<T, G, true, 1024, 4, FUSED, false, OUT, LN>(a, s);
    if (row_bytes <= 32 * 1024) return run_fwd_long<T, G, true, 512, 4, FUSED, true, OUT, LN>(a, s);
    return run_fwd_long<T, G, true, 1024, 4, FUSED, true, OUT, LN>(a, s);
  }
  if constexpr (!kIsMx<OUT>) {
    if (!cache) return run_fwd_long<T, G, false, 1024, 8, FUSED, false, OUT, LN>(a, s);
    return run_fwd_long<T, G, false, 1024, 8, FUSED, true, OUT, LN>(a, s);
  }
  return hipErrorInvalidValue;
}

template <class T, class G, int OUT>
hipError_t fwd_gamma_typed(const FwdCall& c) {
  return c.residual ? fwd_typed<T, G, true, OUT>(c) : fwd_typed<T, G, false, OUT>(c);
}

// LayerNorm (plain output, no fused add).
template <class T, class G>
hipError_t ln_fwd_typed(const FwdCall& c) {
  return fwd_typed<T, G, false, kOutAct, true>(c);
}

// Quantised outputs: per-tensor or per-row scale, or MX block scales.
template <class T, class G>
hipError_t fwd_quant_typed(const FwdCall& c) {
  switch (c.out) {
    case kOutFp8Row: return fwd_gamma_typed<T, G, kOutFp8Row>(c);
    case kOutMxFp8: return fwd_gamma_typed<T, G, kOutMxFp8>(c);
    case kOutMxFp4: return fwd_gamma_typed<T, G, kOutMxFp4>(c);
    default: return fwd_gamma_typed<T, G, kOutFp8Tensor>(c);
  }
}

}  // namespace rmsn
