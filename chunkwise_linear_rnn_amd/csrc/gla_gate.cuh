// The chunk-local gate log-cumsum as the chunk kernels form it in LDS (page "Gated Linear
// Attention Transformers with Hardware-Efficient Training", atlas.scime.ai summary,
// section Approach: the per-chunk cumulative log-gates).  Every kernel that needs g for a
// (chunk, 64-column block) builds it with these two pieces, so the values are the same
// bits wherever they are formed.
#pragma once
#include "gla_common.cuh"
#include "gla_internal.h"

namespace gla {

// A C x DB block of g (fp32) or log_alpha (SrcT) in registers as 16-byte units, written to
// LDS as fp32 times log2 e (through the gate front-end).  Rows at and past `rows`: the last
// valid row repeated (clamp) or zero (after the front-end too, so padded rows never
// decay the chunk).
template <typename SrcT, int C, int DB>
struct GBlock {
  static constexpr int kPer = 16 / (int)sizeof(SrcT), kUnitsRow = DB / kPer;
  static constexpr int kUnits = C * kUnitsRow, kPerThread = kUnits / kThreads;
  static_assert(kUnits % kThreads == 0, "whole units per thread");
  u32x4 u[kPerThread];
  int zero_from;   // first row stored as zero
  __device__ __forceinline__ void load(const SrcT* __restrict__ src, long ld, int rows, bool clamp) {
    zero_from = clamp ? 1 << 30 : rows;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int idx = threadIdx.x + j * kThreads, rr = idx / kUnitsRow, c = (idx % kUnitsRow) * kPer;
      // always a load (of the last valid row past `rows`): no branch around it, and the
      // rows past `rows` are zeroed at store time when not clamped
      u[j] = *reinterpret_cast<const u32x4*>(src + (long)min(rr, rows - 1) * ld + c);
    }
  }
  // one gate per row, src[row] (rows past `rows` zero), the same for every column
  __device__ __forceinline__ void load_scalar(const SrcT* __restrict__ src, int rows) {
    zero_from = rows;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int idx = threadIdx.x + j * kThreads, rr = idx / kUnitsRow;
      const SrcT x = src[min(rr, rows - 1)];
      uint32_t wd;
      if constexpr (sizeof(SrcT) == 2) {
        const uint32_t b = __builtin_bit_cast(uint16_t, x);
        wd = b | (b << 16);
      } else {
        wd = __builtin_bit_cast(uint32_t, x);
      }
      u[j] = u32x4{wd, wd, wd, wd};
    }
  }
  // The loaded units are unpacked first, in straight-line code, and rows are zeroed with
  // selects: a branch around the first use of a load makes the compiler wait for every
  // memory operation in flight (the previous block's output stores included).  `scale`:
  // log2 e (the chunk kernels' base-2 exponentials), or 1 for natural-log units.
  __device__ __forceinline__ void store(float* gs, int gld, GateFn gf,
                                        float scale = kLog2e) const {
    constexpr int kF = sizeof(SrcT) == 2 ? 8 : 4;   // floats per unit
    float x[kPerThread][kF];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      if constexpr (sizeof(SrcT) == 2) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, u[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[j][e] = (float)b[e];
      } else {
        const f32x4 f = __builtin_bit_cast(f32x4, u[j]);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[j][e] = f[e];
      }
    }
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
#pragma unroll
      for (int e = 0; e < kF; ++e) x[j][e] = gf(x[j][e]) * scale;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int idx = threadIdx.x + j * kThreads, rr = idx / kUnitsRow, c = (idx % kUnitsRow) * kPer;
      const bool keep = rr < zero_from;
#pragma unroll
      for (int h = 0; h < kF / 4; ++h) {
        f32x4 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = keep ? x[j][4 * h + e] : 0.f;
        *reinterpret_cast<f32x4*>(gs + rr * gld + c + 4 * h) = f;
      }
    }
  }
};

// Chunk-local inclusive cumsum down each of the DB columns of gs ([C][gld] fp32, already
// staged; the caller synchronizes before and after): thread t takes column t % DB and
// the t / DB-th quarter of the rows, sums it in registers, then adds the totals of the
// quarters above it (in order).  segtot: 4 x DB floats of LDS scratch.  Returns the
// largest |g_t - g_rho| over the thread's rows, rho the first row of each 16-row
// sub-chunk (the spread that decides how a diagonal sub-block can be summed).
// TRANS: the sums go to gs transposed, gs[col * OLD + row] (in place: every read of the
// staged rows happens before the internal barrier), as 16-byte pieces of 4 rows.
// OLD: the row stride of the transposed output (0: gld).
template <int C, int DB, bool TRANS = false, int OLD = 0>
__device__ __forceinline__ float chunk_cumsum_cols(float* gs, int gld, float* segtot) {
  static_assert(kThreads == 4 * DB, "four row quarters per column");
  constexpr int L = C / 4;
  static_assert(L % 16 == 0, "row quarters hold whole sub-chunks");
  const int col = threadIdx.x % DB, seg = threadIdx.x / DB;
  float run[L];
#pragma unroll
  for (int rr = 0; rr < L; ++rr) run[rr] = gs[(seg * L + rr) * gld + col];
#pragma unroll
  for (int rr = 1; rr < L; ++rr) run[rr] += run[rr - 1];
  segtot[seg * DB + col] = run[L - 1];
  __syncthreads();
  float off = 0.f;
  for (int s2 = 0; s2 < seg; ++s2) off += segtot[s2 * DB + col];
  float spread = 0.f, first = 0.f;
#pragma unroll
  for (int rr = 0; rr < L; ++rr) {
    run[rr] += off;
    if (rr % 16 == 0) first = run[rr];
    else spread = fmaxf(spread, fabsf(run[rr] - first));
  }
  if constexpr (TRANS) {
    constexpr int kOld = OLD;
    const int old = kOld ? kOld : gld;
#pragma unroll
    for (int rr = 0; rr < L; rr += 4)
      *reinterpret_cast<f32x4*>(gs + col * old + seg * L + rr) =
          f32x4{run[rr], run[rr + 1], run[rr + 2], run[rr + 3]};
  } else {
#pragma unroll
    for (int rr = 0; rr < L; ++rr) gs[(seg * L + rr) * gld + col] = run[rr];
  }
  return spread;
}

}  // namespace gla
