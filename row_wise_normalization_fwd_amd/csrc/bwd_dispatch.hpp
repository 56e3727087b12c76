// Backward kernel choice and launch (stage 1 then stage 2, same stream) for
// RMSNorm, its fused-add variant (RES) and LayerNorm (LN). Included by one
// translation unit per operation so the instantiations compile in parallel.
//
// Stage 1 uses a group of TPR lanes per row with two 16-byte units per lane
// (TPR = next power of two of ceil(units / 2), up to 1024 lanes, i.e. 16384
// bf16 / 8192 fp32 elements; unaligned rows up to 8192 elements), then 1024
// lanes of three or four units (up to 4096 units: 32768 16-bit / 16384 fp32
// elements; see stage1_typed). Longer rows take the two-pass long-row tier
// (row dots, then 2-D tiles). When a block owns at least two rows,
// it runs 1024 threads, i.e. 1024 / TPR row groups whose dgamma partials are
// combined through LDS: at 8192 x 8192 bf16 this (two 512-lane groups per
// block, one block per CU, next-row prefetch) measured fastest among 1, 2 and
// 4 groups, 256 to 1024 lanes per row and 256 / 384 / 512 blocks. Rows that are not 16-byte aligned use 1-element units.
#pragma once

#include "bwd_kernels.hpp"
#include "launch.hpp"

namespace rmsn {

template <class T, class G, bool RES, bool LN, bool VEC, int TPR, int UPT, int BLOCK, bool PF = true>
hipError_t run_stage1(const BwdArgs<T, G>& a, int64_t blocks, hipStream_t s) {
  constexpr int RG = BLOCK / TPR;
  constexpr int E = Unit<T, VEC>::E;
  // Row-group combine buffer, and LayerNorm's gamma copy (or its dbeta sums)
  // aliased with it.
  constexpr size_t kComb = RG > 1 ? static_cast<size_t>(BLOCK) * UPT * E * sizeof(float) : 0;
  constexpr size_t kGam =
      stage1_gamma_in_lds<T, G, VEC, TPR, UPT, BLOCK, LN>() ||
              stage1_dbeta_in_lds<T, G, VEC, TPR, UPT, BLOCK, LN>()
          ? stage1_gamma_lds_bytes<TPR, UPT, E>()
          : 0;
  constexpr size_t kLds = kComb > kGam ? kComb : kGam;
  constexpr auto kernel = bwd_stage1_kernel<T, G, VEC, TPR, UPT, BLOCK, RES, LN, PF>;
  if constexpr (kLds > 48 * 1024) {
    // Raise the dynamic LDS limit (gfx950 has 160 KiB per workgroup).
    const hipError_t attr = ensure_dynamic_lds<kernel>(kLds);
    if (attr != hipSuccess) return attr;
  }
  kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(BLOCK), kLds, s>>>(a);
  return hipGetLastError();
}

// Lanes per row TPR with UPT units each; a full 1024-thread block of row
// groups when each block owns at least two rows. (LayerNorm, which keeps a
// dbeta sum per column too, fits 1024-thread blocks because it reads gamma
// from LDS: at 8192 x 8192 bf16 stage 1 ran 70.5 us there against 74-77 us
// with 512-thread blocks and gamma in registers.)
template <class T, class G, bool RES, bool LN, bool VEC, int TPR, int UPT, bool PF = true>
hipError_t run_stage1_rows(const BwdArgs<T, G>& a, int64_t blocks, hipStream_t s) {
  // Small groups use 256-thread blocks: with at most 64 rows per partial, a
  // 1024-thread block of 8..64 groups runs each group about once, with no
  // prefetch; 256 threads give each group several rows and several blocks per
  // CU. Measured on bf16 at 64 MiB per operand: groups of up to 64 lanes
  // (256..1024 elements) RMSNorm 4-13% faster, fused add 2-11%, LayerNorm
  // 4-31%; 128-lane groups (1536..3072) RMSNorm and fused add up to 9%, while
  // LayerNorm there loses 5-12% and keeps 1024 threads. 16-bit groups of 16
  // or 32 lanes take 128-thread blocks, eight or sixteen rows per group
  // (256 elements: 48.2 vs 51.9 us, fused add 60.5 vs 67.4, LayerNorm 50.3
  // vs 53.8; 512: 1-3.5% faster); 8- and 64-lane groups lost 5-31% there.
  constexpr int kFull = T::kSize == 2 && (TPR == 16 || TPR == 32)  ? 128
                        : TPR <= 64 || (TPR == 128 && !LN)         ? 256
                                                                   : 1024;
  if constexpr (TPR < kFull) {
    if (a.M >= 2 * a.nblk) return run_stage1<T, G, RES, LN, VEC, TPR, UPT, kFull, PF>(a, blocks, s);
  }
  return run_stage1<T, G, RES, LN, VEC, TPR, UPT, (TPR > 256 ? TPR : 256), PF>(a, blocks, s);
}

// One-pass path: returns hipErrorNotSupported when the row does not fit.
template <class T, class G, bool RES, bool LN>
hipError_t stage1_typed(const BwdArgs<T, G>& a, bool vec, int64_t blocks, hipStream_t s) {
  const int64_t N = a.N;
  if (vec) {
    constexpr int E = 16 / T::kSize;
    const int64_t units = N / E;
    if (units > 2048) {
      // 1024 lanes of three units with next-row prefetch, or of four units
      // without it (two register sets of four would not fit 128 VGPRs), gamma
      // read from LDS. The 16-bit fused add (dresidual is a third operand)
      // fits only three units without prefetch. The 16-bit LayerNorm kernel
      // spills 16-17 VGPRs even then, yet runs 14-21% faster than the
      // two-pass tier (bf16 2048 x 20480 78.5 vs 90.3 us, 2048 x 24576 85.2
      // vs 99.4), so it takes three units too; with four it spilled 84-93 and
      // was 35% slower than that tier. With 16-bit gamma it keeps its dbeta
      // sums in LDS instead (stage1_dbeta_in_lds), spilling 8 VGPRs with
      // three units and 15-17 with four, which beats the two-pass tier (bf16
      // 1024 x 32768 66.3 vs 71.5 us, 1170 x 28672 68.6 vs 75.1) and the
      // spilling three-unit shape (2048 x 16392 65.7 vs 73.1, 1365 x 24576
      // 63.9 vs 68.4). The fused add with four units spills 12-14 and is
      // 27-32% faster than that tier (2048 x 28672 101 vs 128 us, 2048 x
      // 32768 110 vs 145.6).
      if constexpr (T::kSize == 4 || (!RES && !LN)) {
        if (units <= 3072) return run_stage1<T, G, RES, LN, true, 1024, 3, 1024, true>(a, blocks, s);
        if (units <= 4096) return run_stage1<T, G, RES, LN, true, 1024, 4, 1024, false>(a, blocks, s);
      } else {
        if (units <= 3072) return run_stage1<T, G, RES, LN, true, 1024, 3, 1024, false>(a, blocks, s);
        if constexpr (RES || (LN && G::kSize == 2)) {
          if (units <= 4096) return run_stage1<T, G, RES, LN, true, 1024, 4, 1024, false>(a, blocks, s);
        }
      }
      return hipErrorNotSupported;
    }
    if constexpr (!LN && !RES) {
      // Rows that fit 64 or 128 lanes of three units (gamma from LDS) take
      // them instead of twice the lanes of two: at 128 MiB of bf16 per
      // operand, 1536 elements 78.1 vs 81.1 us, 2560 77.9 vs 81.9, 3072
      // 81.5 vs 87.1; fp32 1536 77.9 vs 81.7. With 256 or 512 lanes the
      // two-unit shape is as fast or faster (bf16 6144 and 12288, fp32 3072
      // and 6144), and LayerNorm and the 16-bit fused add spill with three.
      const int64_t t2 = next_pow2(ceil_div(units, 2));
      if ((t2 == 128 || t2 == 256) && units <= 3 * (t2 / 2)) {
        if (t2 == 128) return run_stage1_rows<T, G, RES, LN, true, 64, 3>(a, blocks, s);
        return run_stage1_rows<T, G, RES, LN, true, 128, 3>(a, blocks, s);
      }
    }
    if constexpr (LN && T::kSize == 2) {
      // 16-bit LayerNorm rows of 129..192 units (1032..1536 elements): 64
      // lanes of three units without prefetch (256-thread blocks), which fits
      // the registers, instead of 128 lanes of two (bf16 1536 at 64 MiB per
      // operand 50.4-51.1 vs 59.9-60.8 us). Wider groups of three lost 8-16%
      // (2560..12288 elements), spilling in 1024-thread blocks. Groups of 16
      // or 32 lanes of three take rows that fill at least 15/16 of their
      // units (384 elements 47.8-48.2 vs 50.5-51.0 us, 768 41.9 vs 46.4-46.5);
      // rows that fill fewer were as fast or slower (344: 65.3-65.7 either
      // way, 680: 60.2 vs 58.0-59.4, 264: 79.9 vs 74.2, 520: 60.4 vs 57.5), and 128
      // lanes of three lost 22-26% even in 256-thread blocks.
      if (units > 128 && units <= 192) return run_stage1_rows<T, G, RES, LN, true, 64, 3, false>(a, blocks, s);
      if (units >= 45 && units <= 48) return run_stage1_rows<T, G, RES, LN, true, 16, 3, false>(a, blocks, s);
      if (units >= 90 && units <= 96) return run_stage1_rows<T, G, RES, LN, true, 32, 3, false>(a, blocks, s);
    }
    if (units > 1024) return run_stage1_rows<T, G, RES, LN, true, 1024, 2>(a, blocks, s);
    switch (next_pow2(ceil_div(units, 2))) {
      case 1: return run_stage1_rows<T, G, RES, LN, true, 1, 2>(a, blocks, s);
      case 2: return run_stage1_rows<T, G, RES, LN, true, 2, 2>(a, blocks, s);
      case 4: return run_stage1_rows<T, G, RES, LN, true, 4, 2>(a, blocks, s);
      case 8: return run_stage1_rows<T, G, RES, LN, true, 8, 2>(a, blocks, s);
      case 16: return run_stage1_rows<T, G, RES, LN, true, 16, 2>(a, blocks, s);
      case 32: return run_stage1_rows<T, G, RES, LN, true, 32, 2>(a, blocks, s);
      case 64: return run_stage1_rows<T, G, RES, LN, true, 64, 2>(a, blocks, s);
      case 128: return run_stage1_rows<T, G, RES, LN, true, 128, 2>(a, blocks, s);
      case 256: return run_stage1_rows<T, G, RES, LN, true, 256, 2>(a, blocks, s);
      default: return run_stage1_rows<T, G, RES, LN, true, 512, 2>(a, blocks, s);
    }
  }
  if (N > kBwdOnChipN) return hipErrorNotSupported;
  if (N <= 512) return run_stage1<T, G, RES, LN, false, 64, 8, 256>(a, blocks, s);
  if (N <= 2048) return run_stage1<T, G, RES, LN, false, 256, 8, 256>(a, blocks, s);
  return run_stage1<T, G, RES, LN, false, 1024, 8, 1024>(a, blocks, s);
}

// Long-row tier: pass A (row dots), pass B (tiles). Same partition and
// partial layout as the one-pass path.
template <class T, class G, bool RES, bool LN, bool VEC>
hipError_t long_rows_typed(const BwdArgs<T, G>& a, double* cdot, int64_t blocks, hipStream_t s) {
  constexpr int kUnroll = VEC ? 4 : 8;
  constexpr int kTileBlock = 256;
  constexpr int kTileUpt = VEC ? 2 : 8;
  constexpr int E = Unit<T, VEC>::E;
  static_assert(kTileBlock * kTileUpt * E <= kBwdTileCols, "the partition assumes narrower tiles");
  const int64_t rows = a.M < kMaxGrid ? a.M : kMaxGrid;
  bwd_rowdot_kernel<T, G, VEC, 1024, kUnroll, LN>
      <<<dim3(static_cast<unsigned>(rows)), dim3(1024), 0, s>>>(a, cdot);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t units = a.N / E;
  const int64_t chunks = ceil_div(units, kTileBlock * kTileUpt);
  bwd_tile_kernel<T, G, VEC, kTileBlock, kTileUpt, RES, LN>
      <<<dim3(static_cast<unsigned>(chunks), static_cast<unsigned>(blocks)), dim3(kTileBlock), 0,
         s>>>(a, cdot);
  return hipGetLastError();
}

// Stage 2 over one partial array, or two in one launch (partial2 / out2 not
// null). Partial rows are 16-byte aligned when N % 4 == 0 (the workspace and
// partial_bytes are).
inline hipError_t run_stage2(const float* partial, float* out, const float* partial2,
                             float* out2, const BwdCall& c) {
  // 16 slices of partial rows, 64 columns per block, each thread's 16 loads
  // issued together (8192 x 8192 bf16, stage 2 after stage 1 in one process:
  // the RMSNorm, fused-add and LayerNorm backwards 0.5-0.7% faster than 32
  // slices of 8 loads, 3.5-5% faster than 64 slices; 8 slices no better than
  // 32; 4 columns per thread beat 1 and 2; 256-thread blocks tie 128 and beat
  // 512 by 1.3-1.9%).
  constexpr int kSlices = 16;
  constexpr int kGroups = kS2Threads / kSlices;
  const unsigned ny = out2 != nullptr ? 2u : 1u;
  if (c.N % 4 == 0) {
    const int64_t blocks = ceil_div(c.N, 4 * kGroups);
    bwd_stage2_kernel<4, kSlices>
        <<<dim3(static_cast<unsigned>(blocks), ny), dim3(kS2Threads), 0, c.stream>>>(
            partial, out, partial2, out2, static_cast<int>(c.plan.blocks),
            static_cast<int>(c.N));
  } else {
    const int64_t blocks = ceil_div(c.N, kGroups);
    bwd_stage2_kernel<1, kSlices>
        <<<dim3(static_cast<unsigned>(blocks), ny), dim3(kS2Threads), 0, c.stream>>>(
            partial, out, partial2, out2, static_cast<int>(c.plan.blocks),
            static_cast<int>(c.N));
  }
  return hipGetLastError();
}

template <class T, class G, bool RES, bool LN>
hipError_t bwd_typed(const BwdCall& c) {
  BwdArgs<T, G> a;
  a.dy = static_cast<const typename T::S*>(c.dy);
  a.x = static_cast<const typename T::S*>(c.x);
  a.rstd = c.rstd;
  a.gamma = static_cast<const typename G::S*>(c.gamma);
  a.dx = static_cast<typename T::S*>(c.dx);
  a.dres = static_cast<const typename T::S*>(c.dres);
  a.partial = static_cast<float*>(c.workspace);
  a.mean = c.mean;
  a.partial_b = LN ? reinterpret_cast<float*>(static_cast<char*>(c.workspace) +
                                              c.plan.partial_bytes)
                   : nullptr;
  a.M = c.M;
  a.N = static_cast<int>(c.N);
  a.nblk = c.plan.blocks;
  const bool vec = (c.N * T::kSize) % 16 == 0 && aligned16(c.dy) && aligned16(c.x) &&
                   aligned16(c.dx) && aligned16(c.gamma);
  const bool vec_all = vec && (!RES || aligned16(c.dres));
  hipError_t e = stage1_typed<T, G, RES, LN>(a, vec_all, c.plan.blocks, c.stream);
  if (e == hipErrorNotSupported) {
    // Row dots after the partial rows (one array, two with LN).
    double* cdot = reinterpret_cast<double*>(static_cast<char*>(c.workspace) +
                                             (LN ? 2 : 1) * c.plan.partial_bytes);
    e = vec_all ? long_rows_typed<T, G, RES, LN, true>(a, cdot, c.plan.blocks, c.stream)
                : long_rows_typed<T, G, RES, LN, false>(a, cdot, c.plan.blocks, c.stream);
  }
  if (e != hipSuccess) return e;
  if (LN && c.dbeta != nullptr) return run_stage2(a.partial, c.dgamma, a.partial_b, c.dbeta, c);
  return run_stage2(a.partial, c.dgamma, nullptr, nullptr, c);
}

}  // namespace rmsn
