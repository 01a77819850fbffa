// Gate kernels of the chunkwise GLA path (page "Gated Linear Attention Transformers with
// Hardware-Efficient Training", atlas.scime.ai summary, section Approach):
//   k_gate_cumsum     chunk-local inclusive cumsum of log_alpha (the first step of the
//                     chunkwise form) and the chunk totals gamma.
//   k_state_dot       c_T[d] = sum_v dS_T[d,v] * S_T[d,v], the final-state term of the
//                     closed-form gate gradient.
//   k_gate_tot,       the closed-form gate gradient: a reverse cumulative sum over the
//   k_gate_grad       whole sequence of D = q*dq - k*dk plus c_T, taken in two levels:
//                     chunk-local suffix sums come from the backward chunk kernel, the
//                     suffix over later chunks from the chunk totals the state scans form.
// All three are HBM-bound: coalesced along the contiguous d dimension, no MFMA.
#include "gla_common.cuh"
#include "gla_internal.h"
#include "gla_gate.cuh"

namespace gla {

// One workgroup per (chunk, 64 key columns): the block of gates staged into LDS as fp32
// (16-byte loads; rows past T zero, so the sum continues flat), the chunk-local inclusive
// cumsum down each column in four row quarters (chunk_cumsum_cols, the same sums the
// intra-chunk kernels form), then written out as 16-byte rows; gamma is the last row.
template <typename Tin, int C>
__global__ __launch_bounds__(kThreads) void k_gate_cumsum(const Tin* __restrict__ la,
                                                          GateFn gf, int gscalar,
                                                          float* __restrict__ g,
                                                          float* __restrict__ gamma, int T,
                                                          int dk, int N) {
  constexpr int DB = 64, GLD = DB + 4;
  __shared__ __attribute__((aligned(16))) float gs[C * GLD];
  __shared__ float segtot[4 * DB];
  const int d0 = DB * blockIdx.x, i = blockIdx.y, bh = blockIdx.z;
  const int t0 = i * C, rows = min(C, T - t0);
  GBlock<Tin, C, DB> pg;
  if (gscalar) pg.load_scalar(la + (long)bh * T + t0, rows);
  else pg.load(la + ((long)bh * T + t0) * dk + d0, dk, rows, false);
  pg.store(gs, GLD, gf, 1.f);
  __syncthreads();
  chunk_cumsum_cols<C, DB>(gs, GLD, segtot);
  __syncthreads();
  if (g) {
    constexpr int kUnits = C * DB / 4;
#pragma unroll
    for (int u_ = 0; u_ < kUnits / kThreads; ++u_) {   // fixed trip count
      const int idx = threadIdx.x + u_ * kThreads, r = idx / (DB / 4), c = (idx % (DB / 4)) * 4;
      if (r < rows)
        *reinterpret_cast<f32x4*>(g + ((long)bh * T + t0 + r) * dk + d0 + c) =
            *reinterpret_cast<const f32x4*>(gs + r * GLD + c);
    }
  }
  if (gamma && threadIdx.x < DB)
    gamma[((long)bh * N + i) * dk + d0 + threadIdx.x] = gs[(C - 1) * GLD + threadIdx.x];
}

// One wave per state row d; lanes stride over v.
__global__ __launch_bounds__(kThreads) void k_state_dot(const float* __restrict__ dST,
                                                        const float* __restrict__ ST,
                                                        float* __restrict__ cT, int dk,
                                                        int dv) {
  const int bh = blockIdx.x, w = wave_id(), l = lane_id();
  for (int d = w; d < dk; d += kThreads / kWave) {
    const long row = ((long)bh * dk + d) * dv;
    float s = 0.f;
    for (int v = l; v < dv; v += kWave) s += dST[row + v] * ST[row + v];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (l == 0) cT[(long)bh * dk + d] = s;
  }
}

// tot[j][d] = chunk total of D for chunk j: the sum over the 64-column tiles of
// (forward cross term - reverse cross term).
__global__ __launch_bounds__(kThreads) void k_gate_tot(const float* __restrict__ crossF,
                                                       const float* __restrict__ crossR,
                                                       float* __restrict__ tot, int dk,
                                                       int ntile, int N) {
  const int j = blockIdx.x, bh = blockIdx.y;
  for (int d = threadIdx.x; d < dk; d += kThreads) {
    const long base = ((long)bh * N + j) * ntile * dk + d;
    float t = 0.f;
    for (int u = 0; u < ntile; ++u) t += crossF[base + (long)u * dk] - crossR[base + (long)u * dk];
    tot[((long)bh * N + j) * dk + d] = t;
  }
}

// dlog_alpha[t] = (chunk-local suffix sum of D at t) + c_T + sum of chunk totals of the
// later chunks (times the gate front-end's slope when the gates come as logits).
template <typename Tin>
__global__ __launch_bounds__(kThreads) void k_gate_grad(const float* Dloc,   // may alias part
                                                        const float* __restrict__ tot,
                                                        const float* __restrict__ cT,
                                                        const Tin* __restrict__ la, GateFn gf,
                                                        Tin* __restrict__ dla,
                                                        float* part, int T,
                                                        int dk, int C, int N) {
  constexpr int U = 16;
  const int i = blockIdx.x, bh = blockIdx.y;
  const int t0 = i * C, t1 = min(T, t0 + C);
  const long base = (long)bh * T * dk;
  for (int d = threadIdx.x; d < dk; d += kThreads) {
    float cr = cT ? cT[(long)bh * dk + d] : 0.f;
    for (int j = i + 1; j < N; ++j) cr += tot[((long)bh * N + j) * dk + d];
    for (int tb = t0; tb < t1; tb += U) {
      float x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = tb + u < t1 ? Dloc[base + (long)(tb + u) * dk + d] : 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (tb + u < t1) {
          const long at = base + (long)(tb + u) * dk + d;
          if (part) {   // scalar gates: reduced over d afterwards (x[u] was read first)
            part[at] = x[u] + cr;
          } else {
            const float sl = gf.on ? gf.slope(to_f32(la[at])) : 1.f;
            dla[at] = from_f32<Tin>((x[u] + cr) * sl);
          }
        }
    }
  }
}

// Scalar gates (one per token): the gradient of log_alpha_t is the sum over the key
// dimension of the per-key gradient, times the front-end slope of its logit.  One thread
// per row; nparts partial sums per row (64-wide d blocks, or every d).
template <typename Tin>
__global__ __launch_bounds__(kThreads) void k_gate_reduce(const float* __restrict__ part,
                                                          int nparts,
                                                          const Tin* __restrict__ la,
                                                          GateFn gf, Tin* __restrict__ dla,
                                                          long nrows) {
  const long row = (long)blockIdx.x * kThreads + threadIdx.x;
  if (row >= nrows) return;
  const float* p = part + row * nparts;
  float s = 0.f;
  if (nparts % 4 == 0) {
    for (int j = 0; j < nparts; j += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(p + j);
      s += (x[0] + x[1]) + (x[2] + x[3]);
    }
  } else {
    for (int j = 0; j < nparts; ++j) s += p[j];
  }
  if (gf.on) s *= gf.slope(to_f32(la[row]));
  dla[row] = from_f32<Tin>(s);
}

// ---------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------
hipError_t launch_gate_cumsum(int dtype, const void* la, GateFn gate, int gscalar, float* g,
                              float* gamma, int BH, int T, int dk, int C, hipStream_t s) {
  const int N = (T + C - 1) / C;
  if (BH == 0 || N == 0) return hipSuccess;
  if (dk % 64 != 0 || (C != 64 && C != 128)) return hipErrorInvalidValue;
  const dim3 grid(dk / 64, N, BH);
  auto go = [&](auto kern, const auto* x) {
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, x, gate, gscalar, g, gamma, T, dk, N);
  };
  if (dtype == 0) {
    if (C == 64) go(k_gate_cumsum<float, 64>, (const float*)la);
    else go(k_gate_cumsum<float, 128>, (const float*)la);
  } else {
    if (C == 64) go(k_gate_cumsum<bf16, 64>, (const bf16*)la);
    else go(k_gate_cumsum<bf16, 128>, (const bf16*)la);
  }
  return hipGetLastError();
}

hipError_t launch_gate_reduce(int dtype, const float* part, int nparts, const void* la,
                              GateFn gate, void* dla, long nrows, hipStream_t s) {
  if (nrows == 0) return hipSuccess;
  const dim3 grid((unsigned)((nrows + kThreads - 1) / kThreads));
  if (dtype == 0)
    hipLaunchKernelGGL(k_gate_reduce<float>, grid, dim3(kThreads), 0, s, part, nparts,
                       (const float*)la, gate, (float*)dla, nrows);
  else
    hipLaunchKernelGGL(k_gate_reduce<bf16>, grid, dim3(kThreads), 0, s, part, nparts,
                       (const bf16*)la, gate, (bf16*)dla, nrows);
  return hipGetLastError();
}

hipError_t launch_state_dot(const float* dST, const float* ST, float* cT, int BH, int dk, int dv,
                            hipStream_t s) {
  if (BH == 0) return hipSuccess;
  hipLaunchKernelGGL(k_state_dot, dim3(BH), dim3(kThreads), 0, s, dST, ST, cT, dk, dv);
  return hipGetLastError();
}

hipError_t launch_gate_tot(const float* crossF, const float* crossR, const float* cT,
                             float* tot, int BH, int T, int dk, int ntile, int C, hipStream_t s) {
  (void)cT;
  const int N = (T + C - 1) / C;
  if (BH == 0 || N == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gate_tot, dim3(N, BH), dim3(kThreads), 0, s, crossF, crossR, tot, dk,
                     ntile, N);
  return hipGetLastError();
}

hipError_t launch_gate_grad(int dtype, const float* Dloc, const float* tot, const float* cT,
                            const void* la, GateFn gate, void* dla, float* part, int BH,
                            int T, int dk, int C, hipStream_t s) {
  const int N = (T + C - 1) / C;
  if (BH == 0 || N == 0) return hipSuccess;
  dim3 grid(N, BH);
  if (dtype == 0)
    hipLaunchKernelGGL(k_gate_grad<float>, grid, dim3(kThreads), 0, s, Dloc, tot, cT,
                       (const float*)la, gate, (float*)dla, part, T, dk, C, N);
  else
    hipLaunchKernelGGL(k_gate_grad<bf16>, grid, dim3(kThreads), 0, s, Dloc, tot, cT,
                       (const bf16*)la, gate, (bf16*)dla, part, T, dk, C, N);
  return hipGetLastError();
}

// Precondition check of the gate operand (the layer reads log_alpha as finite and <= 0, and
// gate logits as finite): the number of elements that break it, as an exact integer count
// (per-thread counts, summed over the wave, one integer atomic per wave).
__global__ __launch_bounds__(kThreads) void k_zero_count(unsigned long long* cnt) { *cnt = 0ull; }

template <typename T>
__global__ __launch_bounds__(kThreads) void k_count_bad_gates(const T* __restrict__ x, long n,
                                                              int logits,
                                                              unsigned long long* cnt) {
  unsigned long long c = 0;
  for (long i = blockIdx.x * (long)kThreads + threadIdx.x; i < n; i += (long)gridDim.x * kThreads) {
    const float v = (float)x[i];
    c += (!__builtin_isfinite(v) || (!logits && v > 0.f)) ? 1ull : 0ull;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  if (lane_id() == 0 && c) atomicAdd(cnt, c);
}

hipError_t launch_count_bad_gates(int dtype, const void* x, long n, int logits,
                                  unsigned long long* cnt, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_count, dim3(1), dim3(1), 0, s, cnt);
  if (n > 0) {
    const long b = (n + kThreads - 1) / kThreads;
    const dim3 grid((unsigned)(b < 4096 ? b : 4096));
    if (dtype == 0)
      hipLaunchKernelGGL(k_count_bad_gates<float>, grid, dim3(kThreads), 0, s, (const float*)x, n,
                         logits, cnt);
    else
      hipLaunchKernelGGL(k_count_bad_gates<bf16>, grid, dim3(kThreads), 0, s, (const bf16*)x, n,
                         logits, cnt);
  }
  return hipGetLastError();
}

}  // namespace gla
