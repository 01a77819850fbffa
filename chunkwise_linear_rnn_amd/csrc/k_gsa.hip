// Gated Slot Attention (page "Gated Slot Attention for Efficient Linear-Time Sequence
// Modeling", mlsanity.com summary, Abstract: two GLA passes joined by a softmax, m memory
// slots forgotten by a GLA-style gate).  Per batch and head, with per-slot gates alpha_t
// and write strength w_t = 1 - alpha_t:
//
//   first pass   s_t[j] = sum_{u<=t} (q_t . k_u) w_u[j] exp(L_t[j] - L_u[j])
//                (key slots Kt_t = diag(alpha_t) Kt_{t-1} + w_t^T k_t read by q_t; the gate
//                acts on the output, slot, dimension)
//   softmax      p_t = softmax(s_t) over the slots
//   second pass  o_t = p_t Vt_t, Vt_t = diag(alpha_t) Vt_{t-1} + w_t^T v_t: the main layer
//                with queries p, keys w, values v
//
// The second pass and the chunk states of the first reuse the main layer's kernels; this
// file holds what is new: w = 1 - alpha, the chunk output and the chunk backward of the
// first pass, the row softmax and its backward, and the gate-gradient combination.
// fp32 throughout; the chunk kernels run 64 x 64 x 64 products on the vector ALUs from LDS
// (one workgroup per chunk; each thread owns a 4 x 4 output tile).
#include "gla_common.cuh"
#include "gla_internal.h"

namespace gla {

namespace {

constexpr int kC = 64, kLD = 65;   // chunk rows; LDS row stride of a 64 x 64 fp32 tile

// 64 x 64 block of a row-major fp32 matrix (row stride ld) into LDS, rows >= `rows`
// zero; `trans` stores element (r, c) at lds[c * kLD + r].
__device__ __forceinline__ void load_blk(float* lds, const float* __restrict__ g, long ld,
                                         int rows, bool trans) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = threadIdx.x + kThreads * u, r = idx >> 4, c = (idx & 15) * 4;
    const f32x4 x = *reinterpret_cast<const f32x4*>(g + (long)min(r, rows - 1) * ld + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = r < rows ? x[e] : 0.f;
      if (trans) lds[(c + e) * kLD + r] = v;
      else lds[r * kLD + c + e] = v;
    }
  }
}

// acc[a][b] += sum_{k < kn} X(r0 + a, k) * Y(c0 + b, k), with X(r, k) = X[r * xr + k * xk]
// and Y likewise (strides give either orientation of an LDS tile).
__device__ __forceinline__ void mm64(float (&acc)[4][4], const float* X, int xr, int xk,
                                     const float* Y, int yr, int yk, int r0, int c0,
                                     int kn = kC) {
  for (int kk = 0; kk < kn; ++kk) {
    float xa[4], yb[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) xa[a] = X[(r0 + a) * xr + kk * xk];
#pragma unroll
    for (int b = 0; b < 4; ++b) yb[b] = Y[(c0 + b) * yr + kk * yk];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] += xa[a] * yb[b];
  }
}

__device__ __forceinline__ void zero44(float (&x)[4][4]) {
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) x[a][b] = 0.f;
}

__device__ __forceinline__ void store_rows(float* __restrict__ g, long ld, const float (&x)[4][4],
                                           int r0, int c0, int rows) {
#pragma unroll
  for (int a = 0; a < 4; ++a)
    if (r0 + a < rows)
      *reinterpret_cast<f32x4*>(g + (long)(r0 + a) * ld + c0) = f32x4{x[a][0], x[a][1], x[a][2], x[a][3]};
}

}  // namespace

// w = 1 - exp(log_alpha), via expm1 (w is small when the gate is near 1).
__global__ __launch_bounds__(kThreads) void k_gsa_w(const float* __restrict__ la,
                                                    float* __restrict__ w, long n) {
  for (long i = blockIdx.x * (long)kThreads + threadIdx.x; i < n; i += (long)gridDim.x * kThreads)
    w[i] = -expm1f(la[i]);
}

// First pass, chunk i of head bh: s_t = e^{g_t} * (q_t S1_[i]^T) + sum_{u<=t} A_tu w_u e^{g_t - g_u}
// with A = Q K^T (causal), g the chunk-local cumsum (given times log2 e), S1_[i] the key
// slots before the chunk ([m][dk] fp32).
__global__ __launch_bounds__(kThreads) void k_vg_out(const float* __restrict__ q,
                                                     const float* __restrict__ k,
                                                     const float* __restrict__ w,
                                                     const float* __restrict__ g2,
                                                     const float* __restrict__ S1,
                                                     float* __restrict__ s_out, int T, int dk,
                                                     int m, int N) {
  __shared__ float L0[kC * kLD], L1[kC * kLD], LA[kC * kLD], LW[kC * kLD], LG[kC * kLD];
  const int i = blockIdx.x, bh = blockIdx.y, t0 = i * kC, rows = min(kC, T - t0);
  const int r0 = 4 * (threadIdx.x >> 4), c0 = 4 * (threadIdx.x & 15);
  const float* qb = q + ((long)bh * T + t0) * dk;
  const float* kb = k + ((long)bh * T + t0) * dk;
  const float* wb = w + ((long)bh * T + t0) * m;
  const float* gb = g2 + ((long)bh * T + t0) * m;
  const float* Sb = S1 + ((long)bh * N + i) * m * dk;

  float acc[4][4];
  zero44(acc);
  for (int d0 = 0; d0 < dk; d0 += kC) {
    load_blk(L0, qb + d0, dk, rows, false);
    load_blk(L1, kb + d0, dk, rows, false);
    __syncthreads();
    mm64(acc, L0, kLD, 1, L1, kLD, 1, r0, c0);
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) LA[(r0 + a) * kLD + c0 + b] = c0 + b <= r0 + a ? acc[a][b] : 0.f;

  for (int j0 = 0; j0 < m; j0 += kC) {
    float o[4][4];
    zero44(o);
    for (int d0 = 0; d0 < dk; d0 += kC) {
      load_blk(L0, qb + d0, dk, rows, false);
      load_blk(L1, Sb + (long)j0 * dk + d0, dk, kC, false);
      __syncthreads();
      mm64(o, L0, kLD, 1, L1, kLD, 1, r0, c0);
      __syncthreads();
    }
    load_blk(LW, wb + j0, m, rows, false);
    load_blk(LG, gb + j0, m, rows, false);
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) o[a][b] *= __builtin_amdgcn_exp2f(LG[(r0 + a) * kLD + c0 + b]);
    for (int u = 0; u <= r0 + 3; ++u) {
      float wu[4], gu[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        wu[b] = LW[u * kLD + c0 + b];
        gu[b] = LG[u * kLD + c0 + b];
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int t = r0 + a;
        if (u <= t) {
          const float at = LA[t * kLD + u];
#pragma unroll
          for (int b = 0; b < 4; ++b)
            o[a][b] += at * wu[b] * __builtin_amdgcn_exp2f(LG[t * kLD + c0 + b] - gu[b]);
        }
      }
    }
    store_rows(s_out + ((long)bh * T + t0) * m + j0, m, o, r0, c0, rows);
    __syncthreads();
  }
}

// First pass backward, chunk i: given ds (the gradient of s), the key slots S1_[i] and
// their gradient dS1_[i+1] from the reverse scan,
//   dA_tu = sum_j ds_tj w_uj e^{g_tj - g_uj}                      (u <= t)
//   dq_t  = sum_j ds_tj e^{g_tj} S1_[i][j,:] + sum_{u<=t} dA_tu k_u
//   dk_u  = sum_j w_uj e^{gamma_j - g_uj} dS1_[i+1][j,:] + sum_{t>=u} dA_tu q_t
//   dw_uj = e^{gamma_j - g_uj} (dS1_[i+1] k_u)_j + sum_{t>=u} ds_tj A_tu e^{g_tj - g_uj}
// and the closed-form gate gradient's terms D = s*ds - w*dw (its dependence on the
// cumulative log-gate), as chunk-local suffix sums Dloc and chunk totals tot.
__global__ __launch_bounds__(kThreads) void k_vg_bwd(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ w,
    const float* __restrict__ g2, const float* __restrict__ ds, const float* __restrict__ s,
    const float* __restrict__ S1, const float* __restrict__ dS1, float* __restrict__ dq,
    float* __restrict__ dk_out, float* __restrict__ dw, float* __restrict__ Dloc,
    float* __restrict__ tot, int T, int dk, int m, int N) {
  __shared__ float L0[kC * kLD], L1[kC * kLD], L2[kC * kLD], L3[kC * kLD], L4[kC * kLD],
      LA[kC * kLD], LdA[kC * kLD];
  const int i = blockIdx.x, bh = blockIdx.y, t0 = i * kC, rows = min(kC, T - t0);
  const int r0 = 4 * (threadIdx.x >> 4), c0 = 4 * (threadIdx.x & 15);
  const long rowbase = (long)bh * T + t0;
  const float* qb = q + rowbase * dk;
  const float* kb = k + rowbase * dk;
  const float* Sb = S1 + ((long)bh * N + i) * m * dk;
  const float* dSb = dS1 + ((long)bh * N + i) * m * dk;

  // A = Q K^T (causal)
  float acc[4][4];
  zero44(acc);
  for (int d0 = 0; d0 < dk; d0 += kC) {
    load_blk(L0, qb + d0, dk, rows, false);
    load_blk(L1, kb + d0, dk, rows, false);
    __syncthreads();
    mm64(acc, L0, kLD, 1, L1, kLD, 1, r0, c0);
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) LA[(r0 + a) * kLD + c0 + b] = c0 + b <= r0 + a ? acc[a][b] : 0.f;

  float adA[4][4];   // dA, thread tile (t = r0 + a, u = c0 + b)
  zero44(adA);
  for (int j0 = 0; j0 < m; j0 += kC) {
    load_blk(L2, ds + rowbase * m + j0, m, rows, false);   // ds [t][j]
    load_blk(L3, w + rowbase * m + j0, m, rows, false);    // w  [u][j]
    load_blk(L4, g2 + rowbase * m + j0, m, rows, false);   // g  [t][j] (times log2 e)
    __syncthreads();
    for (int j = 0; j < kC; ++j) {
      float dt[4], gt[4], wu[4], gu[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        dt[a] = L2[(r0 + a) * kLD + j];
        gt[a] = L4[(r0 + a) * kLD + j];
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        wu[b] = L3[(c0 + b) * kLD + j];
        gu[b] = L4[(c0 + b) * kLD + j];
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (c0 + b <= r0 + a) adA[a][b] += dt[a] * wu[b] * __builtin_amdgcn_exp2f(gt[a] - gu[b]);
    }
    // (K dS1^T)[u][j] over dk
    float kds[4][4];
    zero44(kds);
    for (int d0 = 0; d0 < dk; d0 += kC) {
      load_blk(L0, kb + d0, dk, rows, false);
      load_blk(L1, dSb + (long)j0 * dk + d0, dk, kC, false);
      __syncthreads();
      mm64(kds, L0, kLD, 1, L1, kLD, 1, r0, c0);
      __syncthreads();
    }
    // dw for (u = r0 + a, j = c0 + b); gamma = g at the chunk's last valid row
    float dwv[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        dwv[a][b] = __builtin_amdgcn_exp2f(L4[(rows - 1) * kLD + c0 + b] - L4[(r0 + a) * kLD + c0 + b]) *
                    kds[a][b];
    for (int t = r0; t < kC; ++t) {
      float dt[4], gt[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        dt[b] = L2[t * kLD + c0 + b];
        gt[b] = L4[t * kLD + c0 + b];
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int u = r0 + a;
        if (t >= u) {
          const float at = LA[t * kLD + u];
#pragma unroll
          for (int b = 0; b < 4; ++b)
            dwv[a][b] += dt[b] * at * __builtin_amdgcn_exp2f(gt[b] - L4[u * kLD + c0 + b]);
        }
      }
    }
    store_rows(dw + rowbase * m + j0, m, dwv, r0, c0, rows);
    // D = s*ds - w*dw into L1, then suffix sums down each column
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int t = r0 + a;
      const f32x4 sv = *reinterpret_cast<const f32x4*>(s + (rowbase + min(t, rows - 1)) * m + j0 + c0);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        L1[t * kLD + c0 + b] = t < rows ? sv[b] * L2[t * kLD + c0 + b] - L3[t * kLD + c0 + b] * dwv[a][b] : 0.f;
    }
    __syncthreads();
    if (threadIdx.x < kC) {
      const int j = threadIdx.x;
      float run = 0.f;
      for (int t = kC - 1; t >= 0; --t) {
        run += L1[t * kLD + j];
        if (t < rows) Dloc[(rowbase + t) * m + j0 + j] = run;
      }
      tot[((long)bh * N + i) * m + j0 + j] = run;
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) LdA[(r0 + a) * kLD + c0 + b] = c0 + b <= r0 + a ? adA[a][b] : 0.f;
  __syncthreads();

  for (int d0 = 0; d0 < dk; d0 += kC) {
    float aq[4][4], ak[4][4];   // (t, d) and (u, d)
    zero44(aq);
    zero44(ak);
    for (int j0 = 0; j0 < m; j0 += kC) {
      load_blk(L2, ds + rowbase * m + j0, m, rows, false);
      load_blk(L3, w + rowbase * m + j0, m, rows, false);
      load_blk(L4, g2 + rowbase * m + j0, m, rows, false);
      load_blk(L0, Sb + (long)j0 * dk + d0, dk, kC, false);    // S1   [j][d]
      load_blk(L1, dSb + (long)j0 * dk + d0, dk, kC, false);   // dS1  [j][d]
      __syncthreads();
      // ds * e^g and w * e^(gamma - g), in place (each thread its own entries)
#pragma unroll
      for (int uu = 0; uu < 16; ++uu) {
        const int idx = threadIdx.x + kThreads * uu, r = idx >> 6, c = idx & 63;
        const float gv = L4[r * kLD + c];
        L2[r * kLD + c] *= __builtin_amdgcn_exp2f(gv);
        L3[r * kLD + c] *= __builtin_amdgcn_exp2f(L4[(rows - 1) * kLD + c] - gv);
      }
      __syncthreads();
      mm64(aq, L2, kLD, 1, L0, 1, kLD, r0, c0);
      mm64(ak, L3, kLD, 1, L1, 1, kLD, r0, c0);
      __syncthreads();
    }
    load_blk(L0, qb + d0, dk, rows, false);   // q [t][d]
    load_blk(L1, kb + d0, dk, rows, false);   // k [u][d]
    __syncthreads();
    mm64(aq, LdA, kLD, 1, L1, 1, kLD, r0, c0);   // sum_u dA[t][u] k[u][d]
    mm64(ak, LdA, 1, kLD, L0, 1, kLD, r0, c0);   // sum_t dA[t][u] q[t][d]
    store_rows(dq + rowbase * dk + d0, dk, aq, r0, c0, rows);
    store_rows(dk_out + rowbase * dk + d0, dk, ak, r0, c0, rows);
    __syncthreads();
  }
}

// Row softmax over m entries (one wave per row).
__global__ __launch_bounds__(kThreads) void k_softmax_rows(const float* __restrict__ s,
                                                           float* __restrict__ p, long nrows,
                                                           int m) {
  const long row = (long)blockIdx.x * (kThreads / kWave) + wave_id();
  if (row >= nrows) return;
  const float* x = s + row * m;
  const int l = lane_id();
  float mx = -3.0e38f;
  for (int j = l; j < m; j += kWave) mx = fmaxf(mx, x[j]);
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  float sum = 0.f;
  for (int j = l; j < m; j += kWave) sum += __expf(x[j] - mx);
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  const float inv = 1.f / sum;
  for (int j = l; j < m; j += kWave) p[row * m + j] = __expf(x[j] - mx) * inv;
}

// ds = p * (dp - sum_j p_j dp_j), one wave per row.
__global__ __launch_bounds__(kThreads) void k_softmax_bwd(const float* __restrict__ p,
                                                          const float* __restrict__ dp,
                                                          float* __restrict__ ds, long nrows,
                                                          int m) {
  const long row = (long)blockIdx.x * (kThreads / kWave) + wave_id();
  if (row >= nrows) return;
  const int l = lane_id();
  float dot = 0.f;
  for (int j = l; j < m; j += kWave) dot += p[row * m + j] * dp[row * m + j];
  for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
  for (int j = l; j < m; j += kWave) ds[row * m + j] = p[row * m + j] * (dp[row * m + j] - dot);
}

// dlog_alpha = dla1 + dla2 - (dw1 + dw2) * exp(log_alpha)   (w = 1 - exp(log_alpha))
__global__ __launch_bounds__(kThreads) void k_gsa_combine(const float* __restrict__ la,
                                                          const float* __restrict__ dla1,
                                                          const float* __restrict__ dla2,
                                                          const float* __restrict__ dw1,
                                                          const float* __restrict__ dw2,
                                                          float* __restrict__ dla, long n) {
  for (long i = blockIdx.x * (long)kThreads + threadIdx.x; i < n; i += (long)gridDim.x * kThreads)
    dla[i] = dla1[i] + dla2[i] - (dw1[i] + dw2[i]) * __expf(la[i]);
}

// ---------------------------------------------------------------------------------
static unsigned grid1d(long n) {
  const long b = (n + kThreads - 1) / kThreads;
  return (unsigned)(b < 16384 ? (b > 0 ? b : 1) : 16384);
}

hipError_t launch_gsa_w(const float* la, float* w, long n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gsa_w, dim3(grid1d(n)), dim3(kThreads), 0, s, la, w, n);
  return hipGetLastError();
}

hipError_t launch_vg_out(const float* q, const float* k, const float* w, const float* g2,
                         const float* S1, float* s_out, int BH, int T, int dk, int m,
                         hipStream_t s) {
  const int N = (T + kC - 1) / kC;
  if (BH == 0 || N == 0) return hipSuccess;
  hipLaunchKernelGGL(k_vg_out, dim3(N, BH), dim3(kThreads), 0, s, q, k, w, g2, S1, s_out, T, dk,
                     m, N);
  return hipGetLastError();
}

hipError_t launch_vg_bwd(const float* q, const float* k, const float* w, const float* g2,
                         const float* ds, const float* s_in, const float* S1, const float* dS1,
                         float* dq, float* dk, float* dw, float* Dloc, float* tot, int BH, int T,
                         int dkh, int m, hipStream_t s) {
  const int N = (T + kC - 1) / kC;
  if (BH == 0 || N == 0) return hipSuccess;
  hipLaunchKernelGGL(k_vg_bwd, dim3(N, BH), dim3(kThreads), 0, s, q, k, w, g2, ds, s_in, S1, dS1,
                     dq, dk, dw, Dloc, tot, T, dkh, m, N);
  return hipGetLastError();
}

hipError_t launch_softmax_rows(const float* x, float* p, long nrows, int m, hipStream_t s) {
  if (nrows == 0) return hipSuccess;
  const long per = kThreads / kWave;
  hipLaunchKernelGGL(k_softmax_rows, dim3((unsigned)((nrows + per - 1) / per)), dim3(kThreads), 0,
                     s, x, p, nrows, m);
  return hipGetLastError();
}

hipError_t launch_softmax_bwd(const float* p, const float* dp, float* ds, long nrows, int m,
                              hipStream_t s) {
  if (nrows == 0) return hipSuccess;
  const long per = kThreads / kWave;
  hipLaunchKernelGGL(k_softmax_bwd, dim3((unsigned)((nrows + per - 1) / per)), dim3(kThreads), 0,
                     s, p, dp, ds, nrows, m);
  return hipGetLastError();
}

hipError_t launch_gsa_combine(const float* la, const float* dla1, const float* dla2,
                              const float* dw1, const float* dw2, float* dla, long n,
                              hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gsa_combine, dim3(grid1d(n)), dim3(kThreads), 0, s, la, dla1, dla2, dw1,
                     dw2, dla, n);
  return hipGetLastError();
}

}  // namespace gla
