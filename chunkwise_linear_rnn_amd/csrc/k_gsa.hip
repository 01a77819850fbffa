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

// 64-row fp32 tiles in LDS with rows of kFL floats: the 16-byte halves of an MFMA
// fragment read (16 consecutive rows, one 32-float k block) then fall on distinct banks.
constexpr int kC = 64, kFL = 68;

// 64 x 64 block of a row-major fp32 matrix (row stride ld) into LDS rows; rows >= `rows`
// (>= 1) zero, or with `clamp` the last valid row repeated (a gate cumsum continuing flat,
// so that every decay factor between two rows stays at most 1).
__device__ __forceinline__ void stage_rows(float* lds, const float* __restrict__ g, long ld,
                                           int rows, bool clamp = false) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = threadIdx.x + kThreads * u, r = idx >> 4, c = (idx & 15) * 4;
    f32x4 x = *reinterpret_cast<const f32x4*>(g + (long)min(r, rows - 1) * ld + c);
    if (r >= rows && !clamp) x = f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(lds + r * kFL + c) = x;
  }
}
// The same block stored transposed, lds[c * kFL + r] (lanes run down the source rows, so
// the 4-byte LDS writes of a wave are consecutive).
__device__ __forceinline__ void stage_cols(float* lds, const float* __restrict__ g, long ld,
                                           int rows) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = threadIdx.x + kThreads * u, r = idx & 63, c = (idx >> 6) * 4;
    f32x4 x = *reinterpret_cast<const f32x4*>(g + (long)min(r, rows - 1) * ld + c);
    if (r >= rows) x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) lds[(c + e) * kFL + r] = x[e];
  }
}

// Wave w's 16 output rows of a 64 x 64 product over k = 64:
//     acc[j][e] += sum_k X[16 w + 4 q + e][k] * Y[16 j + r][k]
// (lane: r = lane % 16, q = lane / 16), both operands row-major in k in LDS: fp32 MFMA
// 16x16x4 in k32 steps.
__device__ __forceinline__ void mm_rows(f32x4 (&acc)[4], const float* X, const float* Y, int w) {
  const int r = lane_id() & 15;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    Frag<float> a;
    load_frag_c(a, X + (16 * w + r) * kFL + 32 * kb);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Frag<float> b;
      load_frag_c(b, Y + (16 * j + r) * kFL + 32 * kb);
      mma(acc[j], a, b);
    }
  }
}

__device__ __forceinline__ void zero4(f32x4 (&x)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// A = tril(Q K^T) of one chunk (rows of q and k past `rows` zero) into lds_a [t][u],
// through the staging tiles x0, x1.  Ends with the staging tiles free.
__device__ __forceinline__ void chunk_qk(float* lds_a, float* x0, float* x1,
                                        const float* __restrict__ qb,
                                        const float* __restrict__ kb, int dk, int rows) {
  const int w = wave_id(), l = lane_id(), r = l & 15, qd = l >> 4;
  f32x4 acc[4];
  zero4(acc);
  for (int d0 = 0; d0 < dk; d0 += kC) {
    stage_rows(x0, qb + d0, dk, rows);
    stage_rows(x1, kb + d0, dk, rows);
    __syncthreads();
    mm_rows(acc, x0, x1, w);
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * w + 4 * qd + e, u = 16 * j + r;
      lds_a[t * kFL + u] = u <= t ? acc[j][e] : 0.f;
    }
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
//
// Wave w owns output rows 16 w .. 16 w + 15 (sub-chunk I = w) for 64 slots at a time.  The
// dense products (Q K^T, Q S1^T) are fp32 MFMAs.  The gate acts on the slot index j, so
// the intra-chunk sum is rebased per sub-chunk as in the main layer: for sources u in
// earlier sub-chunks, with rho = 16 I,
//     sum_u A_tu w_uj e^{g_tj - g_uj} = e^{g_tj - g_rho,j} sum_u A_tu (w_uj e^{g_rho,j - g_uj})
// (both factors at most 1), an MFMA with the rebased w as B operand; the diagonal
// sub-block (u, t in I) is summed directly.
__global__ __launch_bounds__(kThreads, 3) void k_vg_out(const float* __restrict__ q,
                                                        const float* __restrict__ k,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ g2,
                                                        const float* __restrict__ S1,
                                                        float* __restrict__ s_out, int T, int dk,
                                                        int m, int N) {
  __shared__ __attribute__((aligned(16))) float X0[kC * kFL], X1[kC * kFL], XA[kC * kFL];
  const int i = blockIdx.x, bh = blockIdx.y, t0 = i * kC, rows = min(kC, T - t0);
  const int wv = wave_id(), l = lane_id(), r = l & 15, qd = l >> 4, rho = 16 * wv;
  const long rowbase = (long)bh * T + t0;
  const float* qb = q + rowbase * dk;
  const float* kb = k + rowbase * dk;
  const float* Sb = S1 + ((long)bh * N + i) * m * dk;

  // A = tril(Q K^T) and the first 64 slots' Q S1^T in one pass over dk (each q block
  // staged once; XA holds the S1 block until A is written to it)
  f32x4 o0[4];
  zero4(o0);
  {
    f32x4 acc[4];
    zero4(acc);
    for (int d0 = 0; d0 < dk; d0 += kC) {
      stage_rows(X0, qb + d0, dk, rows);
      stage_rows(X1, kb + d0, dk, rows);
      stage_rows(XA, Sb + d0, dk, kC);
      __syncthreads();
      mm_rows(acc, X0, X1, wv);
      mm_rows(o0, X0, XA, wv);
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = rho + 4 * qd + e, u = 16 * j + r;
        XA[t * kFL + u] = u <= t ? acc[j][e] : 0.f;
      }
  }

  for (int j0 = 0; j0 < m; j0 += kC) {
    // inter-chunk part: Q S1^T for 64 slots
    f32x4 o[4];
    if (j0 == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = o0[j];
    } else {
      zero4(o);
      for (int d0 = 0; d0 < dk; d0 += kC) {
        stage_rows(X0, qb + d0, dk, rows);
        stage_rows(X1, Sb + (long)j0 * dk + d0, dk, kC);
        __syncthreads();
        mm_rows(o, X0, X1, wv);
        __syncthreads();
      }
    }
    // w [u][j] (zero past `rows`) and g [t][j] (flat past `rows`) of the block
    stage_rows(X0, w + rowbase * m + j0, m, rows);
    stage_rows(X1, g2 + rowbase * m + j0, m, rows, true);
    __syncthreads();
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[jt][e] *= __builtin_amdgcn_exp2f(X1[(rho + 4 * qd + e) * kFL + 16 * jt + r]);
    // earlier sub-chunks (u < rho), rebased on rho
    if (wv > 0) {
      f32x4 tmp[4];
      zero4(tmp);
      for (int kb2 = 0; kb2 < (rho + 31) / 32; ++kb2) {
        Frag<float> fa;   // A[rho + r][u], u = 32 kb2 + 8 qd + e < rho
        load_frag_c(fa, XA + (rho + r) * kFL + 32 * kb2);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (32 * kb2 + 8 * qd + e >= rho) fa.v[e] = 0.f;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const int j = 16 * jt + r;
          const float grho = X1[rho * kFL + j];
          Frag<float> fb;   // w[u][j] exp(g[rho][j] - g[u][j])
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int u = 32 * kb2 + 8 * qd + e;
            fb.v[e] = u < rho ? X0[u * kFL + j] * __builtin_amdgcn_exp2f(grho - X1[u * kFL + j]) : 0.f;
          }
          mma(tmp[jt], fa, fb);
        }
      }
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int j = 16 * jt + r;
        const float grho = X1[rho * kFL + j];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[jt][e] += tmp[jt][e] * __builtin_amdgcn_exp2f(X1[(rho + 4 * qd + e) * kFL + j] - grho);
      }
    }
    // the diagonal sub-block: sources u in [rho, t]
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = rho + 4 * qd + e;
      float gt[4], sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) gt[jt] = X1[t * kFL + 16 * jt + r];
      for (int u = rho; u <= t; ++u) {
        const float at = XA[t * kFL + u];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const int j = 16 * jt + r;
          sum[jt] += at * X0[u * kFL + j] * __builtin_amdgcn_exp2f(gt[jt] - X1[u * kFL + j]);
        }
      }
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) o[jt][e] += sum[jt];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = rho + 4 * qd + e;
      if (t < rows) {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) s_out[(rowbase + t) * m + j0 + 16 * jt + r] = o[jt][e];
      }
    }
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
//
// Wave w owns rows 16 w .. 16 w + 15 (sub-chunk I = w) of every output tile.  The dense
// products are fp32 MFMAs; the two gated sums over pairs of rows are rebased per
// sub-chunk (dA on rho = 16 I for earlier sources, dw on rho' = 16 I + 15 for later
// targets; every factor at most 1) with their diagonal sub-blocks summed directly.  Four
// 64 x 64 fp32 tiles of LDS, reused phase by phase, keep two workgroups per CU.
// dq, dk are written as OutT (fp32, or bf16 rounded to nearest even).
template <typename OutT>
__global__ __launch_bounds__(kThreads, 2) void k_vg_bwd(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ w,
    const float* __restrict__ g2, const float* __restrict__ ds, const float* __restrict__ s,
    const float* __restrict__ S1, const float* __restrict__ dS1, OutT* __restrict__ dq,
    OutT* __restrict__ dk_out, float* __restrict__ dw, float* __restrict__ Dloc,
    float* __restrict__ tot, int T, int dk, int m, int N) {
  __shared__ __attribute__((aligned(16))) float T0[kC * kFL], T1[kC * kFL], T2[kC * kFL],
      T3[kC * kFL];
  const int i = blockIdx.x, bh = blockIdx.y, t0 = i * kC, rows = min(kC, T - t0);
  const int wv = wave_id(), l = lane_id(), r = l & 15, qd = l >> 4, rho = 16 * wv;
  const long rowbase = (long)bh * T + t0;
  const float* qb = q + rowbase * dk;
  const float* kb = k + rowbase * dk;
  const float* Sb = S1 + ((long)bh * N + i) * m * dk;
  const float* dSb = dS1 + ((long)bh * N + i) * m * dk;

  // A = tril(Q K^T) in T0
  chunk_qk(T0, T1, T2, qb, kb, dk, rows);

  f32x4 adA[4];   // dA tile (row tile wv, column tile J): lane t = rho + 4 qd + e, u = 16 J + r
  zero4(adA);
  for (int j0 = 0; j0 < m; j0 += kC) {
    // (dS1 k_u)_j for this wave's rows u and 64 slots
    f32x4 kds[4];
    zero4(kds);
    for (int d0 = 0; d0 < dk; d0 += kC) {
      stage_rows(T1, kb + d0, dk, rows);
      stage_rows(T2, dSb + (long)j0 * dk + d0, dk, kC);
      __syncthreads();
      mm_rows(kds, T1, T2, wv);
      __syncthreads();
    }
    // ds [t][j], w [u][j] (zero past `rows`), g [t][j] (flat past `rows`)
    stage_rows(T1, ds + rowbase * m + j0, m, rows);
    stage_rows(T2, w + rowbase * m + j0, m, rows);
    stage_rows(T3, g2 + rowbase * m + j0, m, rows, true);
    __syncthreads();

    // dA, earlier sub-chunks J < I: (ds_tj e^{g_tj - g_rho,j}) (w_uj e^{g_rho,j - g_uj})
    if (wv > 0) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        Frag<float> fds, fgt, fgr, fa;
        load_frag_c(fds, T1 + (rho + r) * kFL + 32 * kb2);
        load_frag_c(fgt, T3 + (rho + r) * kFL + 32 * kb2);
        load_frag_c(fgr, T3 + rho * kFL + 32 * kb2);
#pragma unroll
        for (int e = 0; e < 8; ++e) fa.v[e] = fds.v[e] * __builtin_amdgcn_exp2f(fgt.v[e] - fgr.v[e]);
#pragma unroll
        for (int J = 0; J < 3; ++J) {
          if (J < wv) {
            Frag<float> fw, fgu, fb;
            load_frag_c(fw, T2 + (16 * J + r) * kFL + 32 * kb2);
            load_frag_c(fgu, T3 + (16 * J + r) * kFL + 32 * kb2);
#pragma unroll
            for (int e = 0; e < 8; ++e) fb.v[e] = fw.v[e] * __builtin_amdgcn_exp2f(fgr.v[e] - fgu.v[e]);
            mma(adA[J], fa, fb);
          }
        }
      }
    }
    // dA, the diagonal sub-block: (t = rho + 4 qd + e, u = rho + r), u <= t
    {
      const int u = rho + r;
      float sum[4] = {0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < kC; ++j) {
        const float wu = T2[u * kFL + j], gu = T3[u * kFL + j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = rho + 4 * qd + e;
          sum[e] += T1[t * kFL + j] * wu * __builtin_amdgcn_exp2f(T3[t * kFL + j] - gu);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (u <= rho + 4 * qd + e) adA[wv][e] += sum[e];
    }

    // dw for this wave's rows u = rho + 4 qd + e and slots j = 16 jt + r
    float dwv[4][4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const int j = 16 * jt + r;
      const float gam = T3[(kC - 1) * kFL + j];   // g at the last valid row (flat past it)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dwv[jt][e] = __builtin_amdgcn_exp2f(gam - T3[(rho + 4 * qd + e) * kFL + j]) * kds[jt][e];
    }
    // later sub-chunks (t > rho' = rho + 15), rebased on rho'
    if (wv < 3) {
      const int rp = rho + 15;
      f32x4 tmp[4];
      zero4(tmp);
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        if (32 * kb2 + 31 > rp) {
          Frag<float> fa;   // A[t][u], u = rho + r, t = 32 kb2 + 8 qd + e > rp
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = 32 * kb2 + 8 * qd + e;
            fa.v[e] = t > rp ? T0[t * kFL + rho + r] : 0.f;
          }
#pragma unroll
          for (int jt = 0; jt < 4; ++jt) {
            const int j = 16 * jt + r;
            const float grp = T3[rp * kFL + j];
            Frag<float> fb;   // ds[t][j] e^{g_tj - g_rp,j}
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int t = 32 * kb2 + 8 * qd + e;
              fb.v[e] = t > rp ? T1[t * kFL + j] * __builtin_amdgcn_exp2f(T3[t * kFL + j] - grp) : 0.f;
            }
            mma(tmp[jt], fa, fb);
          }
        }
      }
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int j = 16 * jt + r;
        const float grp = T3[rp * kFL + j];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dwv[jt][e] += tmp[jt][e] * __builtin_amdgcn_exp2f(grp - T3[(rho + 4 * qd + e) * kFL + j]);
      }
    }
    // the diagonal sub-block: targets t in [u, rho + 15]
    {
      float gu[4][4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) gu[e][jt] = T3[(rho + 4 * qd + e) * kFL + 16 * jt + r];
      for (int t = rho; t < rho + 16; ++t) {
        float dt[4], gt[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          dt[jt] = T1[t * kFL + 16 * jt + r];
          gt[jt] = T3[t * kFL + 16 * jt + r];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int u = rho + 4 * qd + e;
          if (t >= u) {
            const float at = T0[t * kFL + u];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
              dwv[jt][e] += dt[jt] * at * __builtin_amdgcn_exp2f(gt[jt] - gu[e][jt]);
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int u = rho + 4 * qd + e;
      if (u < rows) {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) dw[(rowbase + u) * m + j0 + 16 * jt + r] = dwv[jt][e];
      }
    }
    // D = s*ds - w*dw in place of w (each lane its own entries, after every read of w),
    // then suffix sums down each slot column
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = rho + 4 * qd + e;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int j = 16 * jt + r;
        const float sv = s[(rowbase + min(t, rows - 1)) * m + j0 + j];
        T2[t * kFL + j] = t < rows ? sv * T1[t * kFL + j] - T2[t * kFL + j] * dwv[jt][e] : 0.f;
      }
    }
    __syncthreads();
    if (threadIdx.x < kC) {
      const int j = threadIdx.x;
      float run = 0.f;
      for (int t = kC - 1; t >= 0; --t) {
        run += T2[t * kFL + j];
        if (t < rows) Dloc[(rowbase + t) * m + j0 + j] = run;
      }
      tot[((long)bh * N + i) * m + j0 + j] = run;
    }
    __syncthreads();
  }

  // dA (masked) into T3 as [t][u] and into T0 (A is dead) as [u][t]
#pragma unroll
  for (int J = 0; J < 4; ++J)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = rho + 4 * qd + e, u = 16 * J + r;
      const float x = (J <= wv && u <= t) ? adA[J][e] : 0.f;
      T3[t * kFL + u] = x;
      T0[u * kFL + t] = x;
    }
  __syncthreads();

  for (int d0 = 0; d0 < dk; d0 += kC) {
    f32x4 aq[4], ak[4];   // dq (rows t), dk (rows u) of this wave, columns d0 + 16 jt + r
    zero4(aq);
    zero4(ak);
    for (int j0 = 0; j0 < m; j0 += kC) {
      // ds e^{g} [t][j] and S1^T [d][j]
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
        const int idx = threadIdx.x + kThreads * uu, rr = idx >> 4, c = (idx & 15) * 4;
        const long off = (rowbase + min(rr, rows - 1)) * m + j0 + c;
        const f32x4 dv4 = *reinterpret_cast<const f32x4*>(ds + off);
        const f32x4 gv4 = *reinterpret_cast<const f32x4*>(g2 + off);
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = rr < rows ? dv4[e] * __builtin_amdgcn_exp2f(gv4[e]) : 0.f;
        *reinterpret_cast<f32x4*>(T1 + rr * kFL + c) = x;
      }
      stage_cols(T2, Sb + (long)j0 * dk + d0, dk, kC);
      __syncthreads();
      mm_rows(aq, T1, T2, wv);
      __syncthreads();
      // w e^{gamma - g} [u][j] and dS1^T [d][j]
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
        const int idx = threadIdx.x + kThreads * uu, rr = idx >> 4, c = (idx & 15) * 4;
        const long off = (rowbase + min(rr, rows - 1)) * m + j0 + c;
        const f32x4 wv4 = *reinterpret_cast<const f32x4*>(w + off);
        const f32x4 gv4 = *reinterpret_cast<const f32x4*>(g2 + off);
        const f32x4 ga4 = *reinterpret_cast<const f32x4*>(g2 + (rowbase + rows - 1) * m + j0 + c);
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[e] = rr < rows ? wv4[e] * __builtin_amdgcn_exp2f(ga4[e] - gv4[e]) : 0.f;
        *reinterpret_cast<f32x4*>(T1 + rr * kFL + c) = x;
      }
      stage_cols(T2, dSb + (long)j0 * dk + d0, dk, kC);
      __syncthreads();
      mm_rows(ak, T1, T2, wv);
      __syncthreads();
    }
    // + dA k and dA^T q: k^T, q^T [d][row]
    stage_cols(T1, kb + d0, dk, rows);
    stage_cols(T2, qb + d0, dk, rows);
    __syncthreads();
    mm_rows(aq, T3, T1, wv);
    mm_rows(ak, T0, T2, wv);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = rho + 4 * qd + e;
      if (t < rows) {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          dq[(rowbase + t) * dk + d0 + 16 * jt + r] = (OutT)aq[jt][e];
          dk_out[(rowbase + t) * dk + d0 + 16 * jt + r] = (OutT)ak[jt][e];
        }
      }
    }
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

// bf16 Gated Slot Attention: the combination above with the second pass's gradients for
// w and log_alpha in bf16 (the layer's bf16 outputs) and dlog_alpha written in bf16.
__global__ __launch_bounds__(kThreads) void k_gsa_combine_bf16(const float* __restrict__ la,
                                                               const float* __restrict__ dla1,
                                                               const bf16* __restrict__ dla2,
                                                               const float* __restrict__ dw1,
                                                               const bf16* __restrict__ dw2,
                                                               bf16* __restrict__ dla, long n) {
  for (long i = blockIdx.x * (long)kThreads + threadIdx.x; i < n; i += (long)gridDim.x * kThreads)
    dla[i] = (bf16)(dla1[i] + (float)dla2[i] - (dw1[i] + (float)dw2[i]) * __expf(la[i]));
}

// Element conversions between bf16 and fp32 (round to nearest even towards bf16): eight
// elements per thread step (one 16-byte bf16 vector, two 16-byte fp32 vectors; both
// buffers 16-byte aligned), then the tail one by one.
template <typename S, typename D>
__global__ __launch_bounds__(kThreads) void k_cast(const S* __restrict__ x, D* __restrict__ y,
                                                   long n) {
  const long stride = (long)gridDim.x * kThreads, n8 = n / 8;
  for (long i = blockIdx.x * (long)kThreads + threadIdx.x; i < n8; i += stride) {
    float f[8];
    if constexpr (sizeof(S) == 2) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(x + 8 * i);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = (float)b[e];
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4*>(x + 8 * i);
      const f32x4 b = *reinterpret_cast<const f32x4*>(x + 8 * i + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { f[e] = a[e]; f[4 + e] = b[e]; }
    }
    if constexpr (sizeof(D) == 2) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (bf16)f[e];
      *reinterpret_cast<bf16x8*>(y + 8 * i) = o;
    } else {
      *reinterpret_cast<f32x4*>(y + 8 * i) = f32x4{f[0], f[1], f[2], f[3]};
      *reinterpret_cast<f32x4*>(y + 8 * i + 4) = f32x4{f[4], f[5], f[6], f[7]};
    }
  }
  for (long i = 8 * n8 + blockIdx.x * (long)kThreads + threadIdx.x; i < n; i += stride)
    y[i] = (D)x[i];
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
                         void* dq, void* dk, int out_bf16, float* dw, float* Dloc, float* tot,
                         int BH, int T, int dkh, int m, hipStream_t s) {
  const int N = (T + kC - 1) / kC;
  if (BH == 0 || N == 0) return hipSuccess;
  if (out_bf16)
    hipLaunchKernelGGL(k_vg_bwd<bf16>, dim3(N, BH), dim3(kThreads), 0, s, q, k, w, g2, ds, s_in,
                       S1, dS1, (bf16*)dq, (bf16*)dk, dw, Dloc, tot, T, dkh, m, N);
  else
    hipLaunchKernelGGL(k_vg_bwd<float>, dim3(N, BH), dim3(kThreads), 0, s, q, k, w, g2, ds, s_in,
                       S1, dS1, (float*)dq, (float*)dk, dw, Dloc, tot, T, dkh, m, N);
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

hipError_t launch_gsa_combine_bf16(const float* la, const float* dla1, const void* dla2,
                                   const float* dw1, const void* dw2, void* dla, long n,
                                   hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gsa_combine_bf16, dim3(grid1d(n)), dim3(kThreads), 0, s, la, dla1,
                     (const bf16*)dla2, dw1, (const bf16*)dw2, (bf16*)dla, n);
  return hipGetLastError();
}

hipError_t launch_cast_bf16_f32(const void* x, float* y, long n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((k_cast<bf16, float>), dim3(grid1d((n + 7) / 8)), dim3(kThreads), 0, s,
                     (const bf16*)x, y, n);
  return hipGetLastError();
}

hipError_t launch_cast_f32_bf16(const float* x, void* y, long n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((k_cast<float, bf16>), dim3(grid1d((n + 7) / 8)), dim3(kThreads), 0, s, x,
                     (bf16*)y, n);
  return hipGetLastError();
}

}  // namespace gla
