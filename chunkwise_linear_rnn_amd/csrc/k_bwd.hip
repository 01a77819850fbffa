// Backward chunk kernel of the chunkwise GLA path (page "Gated Linear Attention
// Transformers with Hardware-Efficient Training", atlas.scime.ai summary, section
// Approach: two-level chunking and a closed-form gate gradient).  One workgroup per
// (batch*head, chunk) computes, from the chunk-start state S_[i] and the state gradient
// dS_[i+1] produced by the two state scans:
//
//   dA = tril(dO V^T)
//   dQ = (dO S_[i]^T) * exp(g)           + sum_{s<=t} dA_ts k_s * exp(g_t - g_s)
//   dK = (V dS_[i+1]^T) * exp(gamma - g) + sum_{t>=s} dA_ts q_t * exp(g_t - g_s)
//   dV = Kh dS_[i+1] + A^T dO,   Kh = k*exp(gamma - g)
//   D  = q*dQ - k*dK  (fp32), written as chunk-local suffix sums (the closed-form gate
//        gradient within the chunk).
//
// Intra-chunk terms use the same sub-chunking as the forward: for sub-chunks I > J the
// dQ part is exp(g_I - g_rho) * (dA_IJ (K_J * exp(g_rho - g_J))) with rho the first row
// of I, and the dK part is exp(g_rho' - g_J) * (dA_IJ^T (Q_I * exp(g_I - g_rho'))) with
// rho' the last row of J (all exponents <= 0).  Those MFMA products take dA and the
// rebased operand each as a bf16 high part plus a bf16 remainder (three MFMAs), since the
// gate gradient sums q*dq - k*dk with heavy cancellation.  Diagonal sub-blocks are summed
// in fp32 from log-space differences, each exp(g_t - g_s) shared by its dQ and dK terms.
// The chunk-local suffix sums of D are completed by the gate-gradient kernel with the
// chunk totals that the two state scans form from their fp32 states.
#include "gla_common.cuh"
#include "gla_internal.h"

namespace gla {

template <typename OpT, typename Tin>
__device__ __forceinline__ void load_frag_gc(Frag<OpT>& f, const Tin* p, bool valid) {
  float x[8];
  if (valid) load8(x, p + 8 * (lane_id() >> 4)); else zero8(x);
#pragma unroll
  for (int e = 0; e < 8; ++e) f.set(e, x[e]);
}

// An operand as high part + remainder in the MFMA type (bf16), or as is (fp32).
template <typename OpT>
struct SFrag {
  Frag<OpT> hi, lo;
  __device__ __forceinline__ void set(int e, float x) {
    hi.set(e, x);
    if constexpr (sizeof(OpT) == 2) lo.set(e, x - hi.get(e));
  }
};
template <typename OpT>
__device__ __forceinline__ void mma_split(f32x4& acc, const SFrag<OpT>& a, const SFrag<OpT>& b) {
  mma(acc, a.hi, b.hi);
  if constexpr (sizeof(OpT) == 2) {
    mma(acc, a.hi, b.lo);
    mma(acc, a.lo, b.hi);
  }
}

template <int C, int DK, typename Tin, typename OpT>
struct BwdLds {
  static constexpr int NS = C / 16;
  static constexpr int DB = (C == 64) ? 64 : 32;
  static constexpr int ALD = C + 8, FLD = C + 4, GLD = DB + 4, XLD = DB + 8;
  // phase 1-2 (dA in fp32)
  static constexpr int o_dA = 0;
  static constexpr int o_g = o_dA + C * FLD * 4;
  static constexpr int o_q = o_g + C * GLD * 4;
  static constexpr int o_k = o_q + C * XLD * (int)sizeof(Tin);
  static constexpr int o_dqd = o_k + C * XLD * (int)sizeof(Tin);
  static constexpr int o_dkd = o_dqd + C * GLD * 4;
  static constexpr int end12 = o_dkd + C * GLD * 4;
  // phase 3
  static constexpr int o_AT = 0;
  static constexpr int o_dOT = o_AT + C * ALD * (int)sizeof(OpT);
  static constexpr int o_dST = o_dOT + 64 * ALD * (int)sizeof(OpT);
  static constexpr int end3 = o_dST + 64 * (DK + 8) * (int)sizeof(OpT);
  static constexpr int bytes = end12 > end3 ? end12 : end3;
};

template <typename Tin, typename OpT, int C, int DK>
__global__ __launch_bounds__(kThreads) void k_bwd_chunk(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ dO, const float* __restrict__ g, const OpT* __restrict__ A,
    const OpT* __restrict__ Kh, const OpT* __restrict__ S, const OpT* __restrict__ dS,
    Tin* __restrict__ dq, Tin* __restrict__ dk_out, Tin* __restrict__ dv_out,
    float* __restrict__ Dloc, int T, int dv, int N) {
  using L = BwdLds<C, DK, Tin, OpT>;
  constexpr int NS = L::NS, NM = C / 16, DB = L::DB, ALD = L::ALD, FLD = L::FLD, GLD = L::GLD,
                XLD = L::XLD;
  constexpr int CT = DB / 16, MG = 4 / CT, NMW = NM / MG;
  __shared__ __attribute__((aligned(16))) char arena[L::bytes];
  float* dAs = (float*)(arena + L::o_dA);
  float* gs = (float*)(arena + L::o_g);
  Tin* qs = (Tin*)(arena + L::o_q);
  Tin* ks = (Tin*)(arena + L::o_k);
  float* dqd = (float*)(arena + L::o_dqd);
  float* dkd = (float*)(arena + L::o_dkd);

  const int i = blockIdx.x, bh = blockIdx.y;
  const int t0 = i * C, rows = min(C, T - t0);
  const int w = wave_id(), l = lane_id(), r = l & 15, qd = l >> 4;
  const long tok0 = (long)bh * T + t0;   // row index of the chunk's first token

  // ---------------- phase 1: dA = tril(dO V^T) -------------------------------------
  {
    constexpr int NT = NM * (NM + 1) / 2;
    for (int p = w; p < NT; p += 4) {
      int m = 0;
      while ((m + 1) * (m + 2) / 2 <= p) ++m;
      const int n = p - m * (m + 1) / 2;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const bool va = 16 * m + r < rows, vb = 16 * n + r < rows;
      const Tin* ap = dO + (tok0 + 16 * m + r) * dv;
      const Tin* bp = v + (tok0 + 16 * n + r) * dv;
      for (int kb = 0; kb < dv / 32; ++kb) {
        Frag<OpT> fa, fb;
        load_frag_gc(fa, ap + kb * 32, va);
        load_frag_gc(fb, bp + kb * 32, vb);
        mma(acc, fa, fb);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tl = 4 * qd + e;
        dAs[(16 * m + tl) * FLD + 16 * n + r] = (m == n && r > tl) ? 0.f : acc[e];
      }
    }
  }

  const int ct = w % CT, mg = w / CT;
  const OpT* Si = S + ((long)bh * N + i) * DK * dv;
  const OpT* dSi = dS + ((long)bh * N + i) * DK * dv;

  // ---------------- phase 2: dq, dk, D per dk block --------------------------------
  for (int d0 = 0; d0 < DK; d0 += DB) {
    for (int idx = threadIdx.x; idx < C * (DB / 8); idx += kThreads) {
      const int rr = idx / (DB / 8), c = (idx % (DB / 8)) * 8;
      float x[8];
      load8(x, g + (tok0 + min(rr, rows - 1)) * DK + d0 + c);
#pragma unroll
      for (int e = 0; e < 8; ++e) gs[rr * GLD + c + e] = x[e] * kLog2e;
    }
    stage_rows<Tin, Tin, C, DB>(qs, XLD, q + tok0 * DK + d0, DK, rows);
    stage_rows<Tin, Tin, C, DB>(ks, XLD, k + tok0 * DK + d0, DK, rows);
    __syncthreads();

    const int c = 16 * ct + r;   // column of this lane within the block
    f32x4 adq[NMW], adk[NMW];
#pragma unroll
    for (int jj = 0; jj < NMW; ++jj) {
      adq[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
      adk[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // inter-chunk parts: dO S^T and V dS^T (contract over dv)
    {
      const OpT* sp = Si + (long)(d0 + c) * dv;
      const OpT* dsp = dSi + (long)(d0 + c) * dv;
      for (int kb = 0; kb < dv / 32; ++kb) {
        Frag<OpT> fS, fdS;
        load_frag_c(fS, sp + kb * 32);
        load_frag_c(fdS, dsp + kb * 32);
#pragma unroll
        for (int jj = 0; jj < NMW; ++jj) {
          const int m = mg + MG * jj;
          const bool valid = 16 * m + r < rows;
          Frag<OpT> fa;
          load_frag_gc(fa, dO + (tok0 + 16 * m + r) * dv + kb * 32, valid);
          mma(adq[jj], fa, fS);
          load_frag_gc(fa, v + (tok0 + 16 * m + r) * dv + kb * 32, valid);
          mma(adk[jj], fa, fdS);
        }
      }
    }
    const float gl = gs[(C - 1) * GLD + c];   // gamma * log2 e
#pragma unroll
    for (int jj = 0; jj < NMW; ++jj) {
      const int m = mg + MG * jj;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float gt = gs[(16 * m + 4 * qd + e) * GLD + c];
        adq[jj][e] *= __builtin_amdgcn_exp2f(gt);
        adk[jj][e] *= __builtin_amdgcn_exp2f(gl - gt);
      }
    }
    // intra-chunk, off-diagonal sub-blocks
#pragma unroll
    for (int jj = 0; jj < NMW; ++jj) {
      const int m = mg + MG * jj;
      if (m > 0) {   // dq rows of sub-chunk I = m, sources J < I
        const int rho = 16 * m;
        const float gr = gs[rho * GLD + c];
        f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
        for (int kb = 0; kb < (16 * m + 31) / 32; ++kb) {
          SFrag<OpT> fa, fb;
          float xa[8];
          load8(xa, dAs + (16 * m + r) * FLD + kb * 32 + 8 * qd);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int s = kb * 32 + 8 * qd + e;
            fa.set(e, xa[e]);
            fb.set(e, s < rho ? to_f32(ks[s * XLD + c]) *
                                    __builtin_amdgcn_exp2f(gr - gs[s * GLD + c])
                              : 0.f);
          }
          mma_split(tmp, fa, fb);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          adq[jj][e] += tmp[e] * __builtin_amdgcn_exp2f(gs[(rho + 4 * qd + e) * GLD + c] - gr);
      }
      if (m < NS - 1) {   // dk rows of sub-chunk J = m, sources I > J
        const int rho = 16 * m + 15;
        const float gr = gs[rho * GLD + c];
        f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
        for (int kb = (16 * m + 16) / 32; kb < C / 32; ++kb) {
          SFrag<OpT> fa, fb;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = kb * 32 + 8 * qd + e;
            const bool on = t > rho;
            fa.set(e, on ? dAs[t * FLD + 16 * m + r] : 0.f);
            fb.set(e, on ? to_f32(qs[t * XLD + c]) * __builtin_amdgcn_exp2f(gs[t * GLD + c] - gr)
                         : 0.f);
          }
          mma_split(tmp, fa, fb);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          adk[jj][e] += tmp[e] * __builtin_amdgcn_exp2f(gr - gs[(16 * m + 4 * qd + e) * GLD + c]);
      }
    }
    // intra-chunk, diagonal sub-blocks: one thread per (sub-chunk, column)
    {
      const int m = threadIdx.x / DB, cc = threadIdx.x % DB, base = 16 * m;
      float gt[16], qv[16], kv[16], aq[16], ak[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        gt[j] = gs[(base + j) * GLD + cc];
        qv[j] = to_f32(qs[(base + j) * XLD + cc]);
        kv[j] = to_f32(ks[(base + j) * XLD + cc]);
        aq[j] = 0.f;
        ak[j] = 0.f;
      }
      const float* dAm = dAs + base * FLD + base;
#pragma unroll
      for (int t = 0; t < 16; ++t)
#pragma unroll
        for (int s = 0; s <= t; ++s) {
          const float ex = __builtin_amdgcn_exp2f(gt[t] - gt[s]) * dAm[t * FLD + s];
          aq[t] += ex * kv[s];
          ak[s] += ex * qv[t];
        }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        dqd[(base + j) * GLD + cc] = aq[j];
        dkd[(base + j) * GLD + cc] = ak[j];
      }
    }
    __syncthreads();
    // finish dq, dk; D = q*dq - k*dk into dqd
#pragma unroll
    for (int jj = 0; jj < NMW; ++jj) {
      const int m = mg + MG * jj;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * m + 4 * qd + e;
        adq[jj][e] += dqd[t * GLD + c];
        adk[jj][e] += dkd[t * GLD + c];
      }
    }
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < NMW; ++jj) {
      const int m = mg + MG * jj;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * m + 4 * qd + e;
        if (t < rows) {
          dq[(tok0 + t) * DK + d0 + c] = from_f32<Tin>(adq[jj][e]);
          dk_out[(tok0 + t) * DK + d0 + c] = from_f32<Tin>(adk[jj][e]);
        }
        dqd[t * GLD + c] = to_f32(qs[t * XLD + c]) * adq[jj][e] - to_f32(ks[t * XLD + c]) * adk[jj][e];
      }
    }
    __syncthreads();
    // chunk-local suffix sums of D, column by column (segmented)
    {
      constexpr int NSEG = kThreads / DB, SL = C / NSEG;
      const int col = threadIdx.x % DB, seg = threadIdx.x / DB;
      float run = 0.f;
      for (int rr = seg * SL + SL - 1; rr >= seg * SL; --rr) {
        run += dqd[rr * GLD + col];
        dqd[rr * GLD + col] = run;
      }
      dkd[seg * DB + col] = run;
      __syncthreads();
      float off = 0.f;
      for (int s2 = seg + 1; s2 < NSEG; ++s2) off += dkd[s2 * DB + col];
      for (int rr = seg * SL; rr < seg * SL + SL; ++rr)
        if (rr < rows) Dloc[(tok0 + rr) * DK + d0 + col] = dqd[rr * GLD + col] + off;
    }
    __syncthreads();
  }

  // ---------------- phase 3: dv = Kh dS_[i+1] + A^T dO ------------------------------
  {
    OpT* ATs = (OpT*)(arena + L::o_AT);
    OpT* dOT = (OpT*)(arena + L::o_dOT);
    OpT* dST = (OpT*)(arena + L::o_dST);
    constexpr int SLD = DK + 8;
    stage_cols<OpT, OpT, C, C>(ATs, ALD, A + ((long)bh * N + i) * C * C, C, C);
    const OpT* khp = Kh + ((long)bh * N * C + t0) * DK;
    for (int vb0 = 0; vb0 < dv; vb0 += 64) {
      stage_cols<OpT, Tin, C, 64>(dOT, ALD, dO + tok0 * dv + vb0, dv, rows);
      stage_cols<OpT, OpT, DK, 64>(dST, SLD, dSi + vb0, dv, DK);
      __syncthreads();
      f32x4 adv[NM];
#pragma unroll
      for (int m = 0; m < NM; ++m) adv[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
      for (int kb = 0; kb < DK / 32; ++kb) {
        Frag<OpT> fb;
        load_frag_c(fb, dST + (16 * w + r) * SLD + kb * 32);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          Frag<OpT> fa;
          load_frag_c(fa, khp + (long)(16 * m + r) * DK + kb * 32);
          mma(adv[m], fa, fb);
        }
      }
#pragma unroll
      for (int kb = 0; kb < C / 32; ++kb) {
        Frag<OpT> fb;
        load_frag_c(fb, dOT + (16 * w + r) * ALD + kb * 32);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          if (32 * kb + 31 >= 16 * m) {
            Frag<OpT> fa;
            load_frag_c(fa, ATs + (16 * m + r) * ALD + kb * 32);
            mma(adv[m], fa, fb);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * m + 4 * qd + e;
          if (t < rows) dv_out[(tok0 + t) * dv + vb0 + 16 * w + r] = from_f32<Tin>(adv[m][e]);
        }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------------
template <typename Tin, typename OpT, int C, int DK>
static hipError_t launch_bwd_t2(const BwdArgs& a, hipStream_t s) {
  dim3 grid(a.N, a.BH);
  hipLaunchKernelGGL((k_bwd_chunk<Tin, OpT, C, DK>), grid, dim3(kThreads), 0, s,
                     (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.v, (const Tin*)a.dO, a.g,
                     (const OpT*)a.A, (const OpT*)a.Kh, (const OpT*)a.S, (const OpT*)a.dS,
                     (Tin*)a.dq, (Tin*)a.dk_out, (Tin*)a.dv_out, a.Dloc, a.T, a.dv, a.N);
  return hipGetLastError();
}
template <typename Tin, typename OpT, int C>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  switch (a.dk) {
    case 64: return launch_bwd_t2<Tin, OpT, C, 64>(a, s);
    case 128: return launch_bwd_t2<Tin, OpT, C, 128>(a, s);
    case 192: return launch_bwd_t2<Tin, OpT, C, 192>(a, s);
    default: return launch_bwd_t2<Tin, OpT, C, 256>(a, s);
  }
}

hipError_t launch_bwd_chunk(const BwdArgs& a, hipStream_t s) {
  if (a.BH == 0 || a.N == 0) return hipSuccess;
  if (a.dtype == 0) return launch_bwd_t<float, float, 64>(a, s);
  if (a.C == 64) return launch_bwd_t<bf16, bf16, 64>(a, s);
  return launch_bwd_t<bf16, bf16, 128>(a, s);
}

}  // namespace gla
