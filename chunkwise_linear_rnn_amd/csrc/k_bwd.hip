// Backward chunk kernels of the chunkwise GLA path (page "Gated Linear Attention
// Transformers with Hardware-Efficient Training", atlas.scime.ai summary, section
// Approach: two-level chunking and a closed-form gate gradient).  Per (batch*head,
// chunk), from the chunk-start state S_[i] and the state gradient dS_[i+1] written by the
// two state scans:
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
// in fp32, each exp(g_t - g_s) (a product of per-row decays, all at most 1) shared by its
// dQ and dK terms.
// The chunk-local suffix sums of D are completed by the gate-gradient kernel with the
// chunk totals that the two state scans form from their fp32 states.
//
// Kernels
//   k_bwd_dqk_dv (chunk 64) one launch holding two kinds of workgroup, interleaved:
//   dq/dk part  dq, dk and dlog_alpha per (chunk, 64-wide dk block): D as
//              chunk-local suffix sums plus the carry from the later chunks' totals
//              (formed by the gate-total kernel from the scans).  One pass over
//              64-wide dv blocks accumulates dA, dO S^T and V dS^T together: dO and V
//              tiles go through LDS (shared by the 4 waves), each wave's S / dS fragments
//              are prefetched straight into registers (double-buffered); then the
//              intra-chunk part of the block.
//   dv part     dv = A^T dO + Kh dS per (chunk, 64 values), looping over 64-wide dk
//              blocks.
//   k_bwd_chunk (chunk 128, and fp32 operands) all of the above in one workgroup per
//              chunk, operands read straight from memory.
#include "gla_common.cuh"
#include "gla_gate.cuh"
#include "gla_internal.h"

namespace gla {

// Diagonal 16 x 16 sub-block of the intra-chunk terms for one column, in fp32: with
// a_ts = exp(g_t - g_s) dA_ts (t >= s, g already times log2 e),
//   aq_t += sum_{s <= t} a_ts k_s,   ak_s += sum_{t >= s} a_ts q_t.
// exp(g_t - g_s) is the running product of the per-row decays exp(g_u - g_{u-1}),
// u = s + 1 .. t: 15 exponentials instead of 136, every factor at most 1 (nothing
// overflows), and each a_ts shared by its two sums.
__device__ __forceinline__ void diag_block16(const float (&gt)[16], const float (&qv)[16],
                                             const float (&kv)[16], const float* dAm, int ld,
                                             float (&aq)[16], float (&ak)[16]) {
  float dec[16];
#pragma unroll
  for (int u = 1; u < 16; ++u) dec[u] = __builtin_amdgcn_exp2f(gt[u] - gt[u - 1]);
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    float ex = 1.f;
#pragma unroll
    for (int s = t; s >= 0; --s) {
      if (s < t) ex *= dec[s + 1];
      const float a = ex * dAm[t * ld + s];
      aq[t] += a * kv[s];
      ak[s] += a * qv[t];
    }
  }
}

// LDS of the intra-chunk / D phase for one dk block of DB columns.
template <int C, int DB, typename Tin>
struct IntraLds {
  static constexpr int FLD = C + 4, GLD = DB + 4, XLD = DB + 8;
  float* dAs;   // [C][FLD] dA in fp32 (written before the first block)
  float* gs;    // [C][GLD] g * log2 e
  Tin* qs;      // [C][XLD]
  Tin* ks;
  float* dqd;   // [C][GLD]
  float* dkd;
  static constexpr int bytes_blk = C * GLD * 4 * 3 + C * XLD * (int)sizeof(Tin) * 2;
};

// Stage g (already times log2 e; rows past T continue the last valid row), q, k for dk
// columns [d0, d0 + DB) of the chunk.  Ends with a barrier.
template <int C, int DB, int DK, typename Tin>
__device__ __forceinline__ void bwd_stage_block(const IntraLds<C, DB, Tin>& L, const Tin* q,
                                                const Tin* k, const float* g, long tok0,
                                                int rows, int d0) {
  constexpr int GLD = IntraLds<C, DB, Tin>::GLD, XLD = IntraLds<C, DB, Tin>::XLD;
  for (int idx = threadIdx.x; idx < C * (DB / 8); idx += kThreads) {
    const int rr = idx / (DB / 8), c = (idx % (DB / 8)) * 8;
    float x[8];
    load8(x, g + (tok0 + min(rr, rows - 1)) * DK + d0 + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) L.gs[rr * GLD + c + e] = x[e];
  }
  stage_rows<Tin, Tin, C, DB>(L.qs, XLD, q + tok0 * DK + d0, DK, rows);
  stage_rows<Tin, Tin, C, DB>(L.ks, XLD, k + tok0 * DK + d0, DK, rows);
  __syncthreads();
}

// Given the inter-chunk products dO S^T (adq) and V dS^T (adk) of this block, unscaled,
// in accumulator layout (wave column tile ct, M-tiles mg + MG*jj), finish dq, dk: decay
// scaling, intra-chunk terms, output, D suffix sums.  Ends with a barrier.
template <int C, int DB, int DK, int NMW, int MG, typename Tin, typename OpT>
__device__ __forceinline__ void bwd_finish_block(const IntraLds<C, DB, Tin>& L,
                                                 f32x4 (&adq)[NMW], f32x4 (&adk)[NMW],
                                                 Tin* dq, Tin* dk_out, float* Dloc, long tok0,
                                                 int rows, int d0, int ct, int mg) {
  constexpr int NS = C / 16;
  constexpr int FLD = IntraLds<C, DB, Tin>::FLD, GLD = IntraLds<C, DB, Tin>::GLD,
                XLD = IntraLds<C, DB, Tin>::XLD;
  const int l = lane_id(), r = l & 15, qd = l >> 4;
  const int c = 16 * ct + r;   // column of this lane within the block
  const float gl = L.gs[(C - 1) * GLD + c];   // gamma * log2 e
#pragma unroll
  for (int jj = 0; jj < NMW; ++jj) {
    const int m = mg + MG * jj;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gt = L.gs[(16 * m + 4 * qd + e) * GLD + c];
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
      const float gr = L.gs[rho * GLD + c];
      f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
      for (int kb = 0; kb < (16 * m + 31) / 32; ++kb) {
        SFrag<OpT> fa, fb;
        float xa[8];
        load8(xa, L.dAs + (16 * m + r) * FLD + kb * 32 + 8 * qd);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int s = kb * 32 + 8 * qd + e;
          fa.set(e, xa[e]);
          fb.set(e, s < rho ? to_f32(L.ks[s * XLD + c]) *
                                  __builtin_amdgcn_exp2f(gr - L.gs[s * GLD + c])
                            : 0.f);
        }
        mma_split(tmp, fa, fb);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        adq[jj][e] += tmp[e] * __builtin_amdgcn_exp2f(L.gs[(rho + 4 * qd + e) * GLD + c] - gr);
    }
    if (m < NS - 1) {   // dk rows of sub-chunk J = m, sources I > J
      const int rho = 16 * m + 15;
      const float gr = L.gs[rho * GLD + c];
      f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
      for (int kb = (16 * m + 16) / 32; kb < C / 32; ++kb) {
        SFrag<OpT> fa, fb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = kb * 32 + 8 * qd + e;
          const bool on = t > rho;
          fa.set(e, on ? L.dAs[t * FLD + 16 * m + r] : 0.f);
          fb.set(e, on ? to_f32(L.qs[t * XLD + c]) * __builtin_amdgcn_exp2f(L.gs[t * GLD + c] - gr)
                       : 0.f);
        }
        mma_split(tmp, fa, fb);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        adk[jj][e] += tmp[e] * __builtin_amdgcn_exp2f(gr - L.gs[(16 * m + 4 * qd + e) * GLD + c]);
    }
  }
  // intra-chunk, diagonal sub-blocks: one thread per (sub-chunk, column)
  {
    const int m = threadIdx.x / DB, cc = threadIdx.x % DB, base = 16 * m;
    float gt[16], qv[16], kv[16], aq[16], ak[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      gt[j] = L.gs[(base + j) * GLD + cc];
      qv[j] = to_f32(L.qs[(base + j) * XLD + cc]);
      kv[j] = to_f32(L.ks[(base + j) * XLD + cc]);
      aq[j] = 0.f;
      ak[j] = 0.f;
    }
    diag_block16(gt, qv, kv, L.dAs + base * FLD + base, FLD, aq, ak);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      L.dqd[(base + j) * GLD + cc] = aq[j];
      L.dkd[(base + j) * GLD + cc] = ak[j];
    }
  }
  __syncthreads();
#pragma unroll
  for (int jj = 0; jj < NMW; ++jj) {
    const int m = mg + MG * jj;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * m + 4 * qd + e;
      adq[jj][e] += L.dqd[t * GLD + c];
      adk[jj][e] += L.dkd[t * GLD + c];
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
      if (t < rows) {
        dq[(tok0 + t) * DK + d0 + c] = from_f32<Tin>(adq[jj][e]);
        dk_out[(tok0 + t) * DK + d0 + c] = from_f32<Tin>(adk[jj][e]);
      }
      L.dqd[t * GLD + c] =
          to_f32(L.qs[t * XLD + c]) * adq[jj][e] - to_f32(L.ks[t * XLD + c]) * adk[jj][e];
    }
  }
  __syncthreads();
  // chunk-local suffix sums of D, column by column (segmented)
  {
    constexpr int NSEG = kThreads / DB, SL = C / NSEG;
    const int col = threadIdx.x % DB, seg = threadIdx.x / DB;
    float run = 0.f;
    for (int rr = seg * SL + SL - 1; rr >= seg * SL; --rr) {
      run += L.dqd[rr * GLD + col];
      L.dqd[rr * GLD + col] = run;
    }
    L.dkd[seg * DB + col] = run;
    __syncthreads();
    float off = 0.f;
    for (int s2 = seg + 1; s2 < NSEG; ++s2) off += L.dkd[s2 * DB + col];
    for (int rr = seg * SL; rr < seg * SL + SL; ++rr)
      if (rr < rows) Dloc[(tok0 + rr) * DK + d0 + col] = L.dqd[rr * GLD + col] + off;
  }
  __syncthreads();
}

// =====================================================================================
// chunk 64, dq/dk part: one workgroup per (batch*head, chunk, 64-wide dk block)
// =====================================================================================
// Wave w owns columns 16w .. 16w+15 of the block for all 64 rows of the chunk (four
// accumulator tiles each for dq and dk).  dA = tril(dO V^T) is formed by every dk block of
// the chunk (it is cheap next to the dO S^T and V dS^T products, and keeps the blocks
// independent).  Three workgroups fit on a CU, so one's loads overlap another's math.
// LDS of a dq/dk workgroup for chunk C: dA [C][C + 4] fp32, the region of the staged g
// block [C][68] and of g^T [64][C + 4] fp32, q and k [C][72]
constexpr int dqk_lds_bytes(int C) {
  return C * (C + 4) * 4 + (C * 68 > 64 * (C + 4) ? C * 68 : 64 * (C + 4)) * 4 + 2 * C * 72 * 2;
}
constexpr int kDqkLds = dqk_lds_bytes(64);
// SFRAG: S and dS in MFMA fragment order (fragment (16-row block, 32-column block) of a
// chunk's [dk][dv] state: lane 16 q + r holds row r, columns 8 q .. 8 q + 7), as the scans
// write them for 128-column tiles; otherwise row-major.
template <typename Tin, typename OpT, bool SFRAG, bool SG, int C>
__device__ __forceinline__ void bwd_dqk_body(
    char* __restrict__ arena, int lt, const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ dO, int gscalar, const OpT* __restrict__ S,
    const OpT* __restrict__ dS, Tin* __restrict__ dq, Tin* __restrict__ dk_out,
    const float* __restrict__ tot, const float* __restrict__ cT, const Tin* __restrict__ la,
    GateFn gf, Tin* __restrict__ dla, float* __restrict__ dla_part, int T, int dk, int dv,
    int N) {
  static_assert(sizeof(Tin) == sizeof(OpT), "input and operand types match");
  // dO / V rows padded to 80: their 16-byte fragment reads (16 consecutive rows) then fall
  // on distinct banks
  constexpr int NM = C / 16, NS = C / 16, YLD = 64 + 16;
  constexpr int NRT = NM / 4;   // dA row tiles per wave: w, w + 4, ...
  constexpr int FLD = C + 4, GLD = 64 + 4, XLD = 64 + 8;
  constexpr int GTLD = C + 4;   // g^T rows (a column's C rows)
  // LDS: dA [C][FLD] fp32, then a region that holds the dO / V tiles during the dv loop,
  // then the staged g block [C][GLD] and in its place g^T [64 columns][GTLD] fp32 (a
  // column's rows contiguous: the post-loop phases read 4 to 16 consecutive rows of one
  // column), q, k [C][XLD] afterwards.  Chunk 64: 53248 bytes, three workgroups per CU;
  // chunk 128: 139264 bytes, one.
  constexpr int GBYTES = (C * GLD > 64 * GTLD ? C * GLD : 64 * GTLD) * 4;
  constexpr int o_u = C * FLD * 4, o_q = o_u + GBYTES, o_k = o_q + C * XLD * 2;
  constexpr int bytes = o_k + C * XLD * 2;
  static_assert(2 * C * YLD * 2 <= bytes - o_u, "dO / V tiles fit the shared region");
  static_assert(bytes == dqk_lds_bytes(C), "arena size");
  // the first-pass diagonal terms of dk go to dA's columns 64 .. (chunk 128) or to g's
  // region (chunk 64)
  constexpr int DKLD = C == 64 ? GLD : FLD;
  float* dAs = (float*)arena;
  OpT* dOs = (OpT*)(arena + o_u);
  OpT* Vs = dOs + C * YLD;
  float* gs = (float*)(arena + o_u);
  Tin* qs = (Tin*)(arena + o_q);
  Tin* ks = (Tin*)(arena + o_k);

  // XCD-aware: the dk blocks of one chunk (same dO and V tiles) are consecutive
  const int NJ = dk / 64;
  const int jb = lt % NJ, i = (lt / NJ) % N, bh = lt / (NJ * N);
  const int d0 = 64 * jb, t0 = i * C, rows = min(C, T - t0);
  const int w = wave_id(), l = lane_id(), r = l & 15, qd = l >> 4;
  const int c = 16 * w + r;   // this lane's column in the block
  const long tok0 = (long)bh * T + t0;
  const OpT* Si = S + ((long)bh * N + i) * dk * dv;
  const OpT* dSi = dS + ((long)bh * N + i) * dk * dv;
  const int NV = dv / 64;

  f32x4 adq[NM], adk[NM], adA[NRT][NM];   // adA[j][n] = dA tile (w + 4 j, n), n <= w + 4 j
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    adq[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    adk[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NRT; ++j) adA[j][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  RowTile<OpT, C, 64, YLD> tdO, tV;
  Frag<OpT> sA[2], dsA[2], sB[2], dsB[2];
  auto fetch = [&](int vb, Frag<OpT> (&fs)[2], Frag<OpT> (&fds)[2]) {
    tdO.load((const OpT*)dO + tok0 * dv + vb * 64, dv, rows);
    tV.load((const OpT*)v + tok0 * dv + vb * 64, dv, rows);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const long off = (long)(d0 + c) * dv + vb * 64 + kb * 32;
      if constexpr (SFRAG) {
        const long fo = (((long)(d0 / 16 + w) * (dv / 32) + (vb * 2 + kb)) * 64 + l) * 8;
        fs[kb].v = *reinterpret_cast<const bf16x8*>(Si + fo);
        fds[kb].v = *reinterpret_cast<const bf16x8*>(dSi + fo);
      } else {
        load_frag_c(fs[kb], Si + off);
        load_frag_c(fds[kb], dSi + off);
      }
    }
  };
  auto body = [&](int vb, Frag<OpT> (&fs)[2], Frag<OpT> (&fds)[2], Frag<OpT> (&ns)[2],
                  Frag<OpT> (&nds)[2]) {
    tdO.store(dOs);
    tV.store(Vs);
    __syncthreads();
    // unconditional (the last block refetches itself): exact wait counts for the compiler
    fetch(min(vb + 1, NV - 1), ns, nds);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      Frag<OpT> fO[NM], fV[NM];
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        load_frag_c(fO[m], dOs + (16 * m + r) * YLD + kb * 32);
        load_frag_c(fV[m], Vs + (16 * m + r) * YLD + kb * 32);
      }
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        mma(adq[m], fO[m], fs[kb]);
        mma(adk[m], fV[m], fds[kb]);
      }
#pragma unroll
      for (int j = 0; j < NRT; ++j) {
        Frag<OpT> fOw;
        load_frag_c(fOw, dOs + (16 * (w + 4 * j) + r) * YLD + kb * 32);
#pragma unroll
        for (int n = 0; n < NM; ++n)
          if (n <= w + 4 * j) mma(adA[j][n], fOw, fV[n]);
      }
    }
    __syncthreads();
  };
  fetch(0, sA, dsA);
  // gate gradient carried into this chunk for column c: the chunk totals of D over the
  // later chunks (lane group qd takes every fourth chunk), plus c_T (eight chunk totals
  // per lane in flight at once; out-of-range ones read a valid entry and are dropped).
  // Loaded after the first block's operands, so that both round trips overlap.
  float carry = 0.f;
  for (int j0 = i + 1 + qd; j0 < N; j0 += 32) {
    float tv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) tv[u] = tot[((long)bh * N + min(j0 + 4 * u, N - 1)) * dk + d0 + c];
#pragma unroll
    for (int u = 0; u < 8; ++u) carry += j0 + 4 * u < N ? tv[u] : 0.f;
  }
  int vb = 0;
  for (; vb + 1 < NV; vb += 2) {
    body(vb, sA, dsA, sB, dsB);
    body(vb + 1, sB, dsB, sA, dsA);
  }
  if (vb < NV) body(vb, sA, dsA, sB, dsB);

  // g * log2 e of the block (rows past T continue the last valid row), rebuilt from the
  // gate operand with the intra-chunk kernel's staging and column cumsum (the same bits),
  // then q, k of the block, into the region the dO / V tiles used; the k tile's space
  // holds the cumsum's segment totals first.  Their loads are issued before the dA tiles
  // (w, n <= w; the diagonal tile masked above the diagonal) go to LDS.
  {
    GBlock<Tin, C, 64> pg;
    if (gscalar) pg.load_scalar(la + tok0, rows);
    else pg.load(la + tok0 * dk + d0, dk, rows, false);
    RowTile<Tin, C, 64, XLD> tq, tk;
    tq.load(q + tok0 * dk + d0, dk, rows);
    tk.load(k + tok0 * dk + d0, dk, rows);
#pragma unroll
    for (int j = 0; j < NRT; ++j) {
      const int wr = w + 4 * j;
#pragma unroll
      for (int n = 0; n < NM; ++n)
        if (n <= wr) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tl = 4 * qd + e;
            dAs[(16 * wr + tl) * FLD + 16 * n + r] = (n == wr && r > tl) ? 0.f : adA[j][n][e];
          }
        }
    }
    pg.store(gs, GLD, gf);
    __syncthreads();
    chunk_cumsum_cols<C, 64, true, GTLD>(gs, GLD, reinterpret_cast<float*>(ks));   // g^T
    __syncthreads();
    tq.store(qs);
    tk.store(ks);
  }
  __syncthreads();

  // inter-chunk parts: dq *= exp(g_t), dk *= exp(gamma - g_t)
  const float* gc = gs + c * GTLD;   // g of this lane's column, by row
  const float gl = gc[C - 1];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const f32x4 gt = *reinterpret_cast<const f32x4*>(gc + 16 * m + 4 * qd);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      adq[m][e] *= __builtin_amdgcn_exp2f(gt[e]);
      adk[m][e] *= __builtin_amdgcn_exp2f(gl - gt[e]);
    }
  }
  if constexpr (SG) {
    // Scalar gates: exp(g_t - g_s) is the same for every column (g of column 0 stands for
    // all), so the intra-chunk terms are two MFMA products with the C x C matrix
    // P = dA * D, D[t][s] = exp(g_t - g_s) (s <= t), formed in fp32 in place of dA:
    //     dq[t] += sum_{s <= t} P[t][s] k_s,     dk[s] += sum_{t >= s} P[t][s] q_t,
    // P entering as three bf16 parts (high, middle, low: fp32-exact) against the exact
    // bf16 q and k.  Tiles above the diagonal tile row are never read.
    for (int idx = threadIdx.x; idx < C * C; idx += kThreads) {
      const int t = idx / C, s2 = idx % C;
      if (s2 <= t) dAs[t * FLD + s2] *= __builtin_amdgcn_exp2f(gs[t] - gs[s2]);
    }
    __syncthreads();
    auto split3 = [](float x, Frag<OpT>& h, Frag<OpT>& md, Frag<OpT>& lo, int e) {
      h.set(e, x);
      const float r1 = x - h.get(e);
      md.set(e, r1);
      lo.set(e, r1 - md.get(e));
    };
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      f32x4 tq = {0.f, 0.f, 0.f, 0.f}, tk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < C / 32; ++kb) {
        if (32 * kb < 16 * (m + 1)) {   // dq rows of tile m: sources s < 16 (m + 1)
          Frag<OpT> h, md, lo, fb;
          float xa[8];
          load8(xa, dAs + (16 * m + r) * FLD + kb * 32 + 8 * qd);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int s2 = kb * 32 + 8 * qd + e;
            const bool on = s2 < 16 * (m + 1);
            split3(on ? xa[e] : 0.f, h, md, lo, e);
            fb.set(e, on ? to_f32(ks[s2 * XLD + c]) : 0.f);
          }
          mma(tq, h, fb);
          mma(tq, md, fb);
          mma(tq, lo, fb);
        }
        if (32 * kb + 31 >= 16 * m) {   // dk rows of tile m: sources t >= 16 m
          Frag<OpT> h, md, lo, fb;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = kb * 32 + 8 * qd + e;
            const bool on = t >= 16 * m;
            split3(on ? dAs[t * FLD + 16 * m + r] : 0.f, h, md, lo, e);
            fb.set(e, on ? to_f32(qs[t * XLD + c]) : 0.f);
          }
          mma(tk, h, fb);
          mma(tk, md, fb);
          mma(tk, lo, fb);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        adq[m][e] += tq[e];
        adk[m][e] += tk[e];
      }
    }
  } else {
  // intra-chunk, off-diagonal sub-blocks (split bf16 operands, three MFMAs each)
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    if (m > 0) {   // dq rows of sub-chunk I = m, sources J < I, rebased on rho = 16 m
      const int rho = 16 * m;
      const float gr = gc[rho];
      f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < (16 * m + 31) / 32; ++kb) {
        SFrag<OpT> fa, fb;
        float xa[8], gv[8];
        load8(xa, dAs + (16 * m + r) * FLD + kb * 32 + 8 * qd);
        load8(gv, gc + kb * 32 + 8 * qd);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int s = kb * 32 + 8 * qd + e;
          // dA is only written below its diagonal: mask the rest on both operands
          fa.set(e, s < rho ? xa[e] : 0.f);
          fb.set(e, s < rho ? to_f32(ks[s * XLD + c]) * __builtin_amdgcn_exp2f(gr - gv[e])
                            : 0.f);
        }
        mma_split(tmp, fa, fb);
      }
      const f32x4 gt = *reinterpret_cast<const f32x4*>(gc + rho + 4 * qd);
#pragma unroll
      for (int e = 0; e < 4; ++e) adq[m][e] += tmp[e] * __builtin_amdgcn_exp2f(gt[e] - gr);
    }
    if (m < NS - 1) {   // dk rows of sub-chunk J = m, sources I > J, rebased on rho' = 16 m + 15
      const int rho = 16 * m + 15;
      const float gr = gc[rho];
      f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = (16 * m + 16) / 32; kb < C / 32; ++kb) {
        SFrag<OpT> fa, fb;
        float gv[8];
        load8(gv, gc + kb * 32 + 8 * qd);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = kb * 32 + 8 * qd + e;
          const bool on = t > rho;
          fa.set(e, on ? dAs[t * FLD + 16 * m + r] : 0.f);
          fb.set(e, on ? to_f32(qs[t * XLD + c]) * __builtin_amdgcn_exp2f(gv[e] - gr) : 0.f);
        }
        mma_split(tmp, fa, fb);
      }
      const f32x4 gt = *reinterpret_cast<const f32x4*>(gc + 16 * m + 4 * qd);
#pragma unroll
      for (int e = 0; e < 4; ++e) adk[m][e] += tmp[e] * __builtin_amdgcn_exp2f(gr - gt[e]);
    }
  }
  // intra-chunk, diagonal sub-blocks in fp32: thread (sub-chunk md, column cd), four
  // sub-chunks per pass
  constexpr int NPD = NS / 4;
  float aq[NPD][16], ak[NPD][16];
  const int cd = threadIdx.x % 64;
#pragma unroll
  for (int pd = 0; pd < NPD; ++pd) {
    const int base = 16 * (threadIdx.x / 64 + 4 * pd);
    float gt[16], qv[16], kv[16];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(gs + cd * GTLD + base + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) gt[4 * h + e] = x[e];
    }
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      qv[jj] = to_f32(qs[(base + jj) * XLD + cd]);
      kv[jj] = to_f32(ks[(base + jj) * XLD + cd]);
      aq[pd][jj] = 0.f;
      ak[pd][jj] = 0.f;
    }
    diag_block16(gt, qv, kv, dAs + base * FLD + base, FLD, aq[pd], ak[pd]);
  }
  __syncthreads();   // dA and g are dead from here: their regions carry the diagonal terms
  float* dqd = dAs;                          // [C][FLD], columns 0 .. 63
  float* dkd = C == 64 ? gs : dAs + 64;      // [C][DKLD]
#pragma unroll
  for (int pd = 0; pd < NPD; ++pd) {
    const int base = 16 * (threadIdx.x / 64 + 4 * pd);
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      dqd[(base + jj) * FLD + cd] = aq[pd][jj];
      dkd[(base + jj) * DKLD + cd] = ak[pd][jj];
    }
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * m + 4 * qd + e;
      adq[m][e] += dqd[t * FLD + c];
      adk[m][e] += dkd[t * DKLD + c];
    }
  }
  // finish dq, dk; D = q*dq - k*dk and its chunk-local suffix sums, in registers
  float Dv[NM][4];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * m + 4 * qd + e;
      Dv[m][e] = to_f32(qs[t * XLD + c]) * adq[m][e] - to_f32(ks[t * XLD + c]) * adk[m][e];
    }
  // dq, dk, dlog_alpha of the block leave as 16-byte rows through LDS (the dA and g
  // regions are dead once every wave has read the diagonal terms)
  constexpr int SLD = 64 + 8;
  Tin* st = (Tin*)arena;   // three [C][SLD] tiles: dq, dk, dlog_alpha
  __syncthreads();
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * m + 4 * qd + e;
      st[t * SLD + c] = from_f32<Tin>(adq[m][e]);
      st[C * SLD + t * SLD + c] = from_f32<Tin>(adk[m][e]);
    }
  // rows of this lane: 16 m + 4 qd + e.  Suffix sums within the lane, then across the
  // four lane groups of the column (lanes r + 16 q') and the later sub-chunks, on top of
  // the carry from the later chunks: the closed-form gate gradient.
  carry += __shfl_xor(carry, 16);
  carry += __shfl_xor(carry, 32);
  if (cT) carry += cT[(long)bh * dk + d0 + c];
  float ptot[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    Dv[m][2] += Dv[m][3];
    Dv[m][1] += Dv[m][2];
    Dv[m][0] += Dv[m][1];
    ptot[m] = Dv[m][0];
  }
  float later = carry;   // carry plus the sum over sub-chunks after m, all lane groups
  // scalar gates: the row sums over this block's 64 columns, per wave (its 16 columns),
  // in the region of the third staging tile
  float* wsum = (float*)(st + 2 * C * SLD);   // [4 waves][C]
#pragma unroll
  for (int m = NM - 1; m >= 0; --m) {
    float after = later, all = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < 4; ++g2) {
      const float x = __shfl(ptot[m], r + 16 * g2);
      all += x;
      if (g2 > qd) after += x;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * m + 4 * qd + e;
      if (dla_part) {
        const float rs = row16_sum(Dv[m][e] + after);
        if (r == 0) wsum[w * C + t] = rs;
      } else {
        // gates given as logits: chain rule to the logit (rows past T hold no logit)
        const float sl = gf.on && t < rows ? gf.slope(to_f32(la[(tok0 + t) * dk + d0 + c])) : 1.f;
        st[2 * C * SLD + t * SLD + c] = from_f32<Tin>((Dv[m][e] + after) * sl);
      }
    }
    later += all;
  }
  __syncthreads();
  constexpr int kPer = 16 / (int)sizeof(Tin), kRowUnits = 64 / kPer, kUnits = 3 * C * kRowUnits;
  static_assert(3 * C * SLD * (int)sizeof(Tin) <= o_q, "staging stays clear of q / k");
  static_assert(4 * C * 4 <= C * SLD * (int)sizeof(Tin), "row sums fit the third tile");
  const int ntile_out = dla_part ? 2 : 3;
  for (int idx = threadIdx.x; idx < kUnits; idx += kThreads) {
    const int tile = idx / (C * kRowUnits), u = idx % (C * kRowUnits);
    const int rr = u / kRowUnits, cc = (u % kRowUnits) * kPer;
    Tin* dst = tile == 0 ? dq : (tile == 1 ? dk_out : dla);
    if (tile < ntile_out && rr < rows)
      stream16(dst + (tok0 + rr) * dk + d0 + cc,
               *reinterpret_cast<const u32x4*>(st + (tile * C + rr) * SLD + cc));
  }
  if (dla_part && threadIdx.x < rows) {
    const int t = threadIdx.x;
    dla_part[(tok0 + t) * NJ + jb] = (wsum[t] + wsum[C + t]) + (wsum[2 * C + t] + wsum[3 * C + t]);
  }
}

// =====================================================================================
// chunk 64, dv part: one workgroup per (batch*head, chunk, 64 values)
// =====================================================================================
// dv = A^T dO + sum over 64-wide dk blocks of Kh_blk dS_blk; the next block's Kh and
// dS^T tiles are loaded into registers while the current one multiplies.
template <typename Tin, typename OpT, bool SFRAG, int C>
__device__ __forceinline__ void bwd_dv_body(char* __restrict__ arena, int lt,
                                            const OpT* __restrict__ Kh,
                                            const OpT* __restrict__ A,
                                            const OpT* __restrict__ dS,
                                            const Tin* __restrict__ dO,
                                            Tin* __restrict__ dv_out, int T, int dk, int dv,
                                            int N) {
  // the Kh block is read row-major (rows padded to 80 for conflict-free fragment reads),
  // the transposed tiles through the swizzle of ColTile (rows of 72)
  // LD: rows of 64 (the dS^T tile, the output staging); TLD: rows of C tokens (A^T, dO^T)
  constexpr int NM = C / 16, LD = 64 + 8, TLD = C + 8, KLD = 64 + 16;
  static_assert(C * KLD * 2 + 64 * LD * 2 + (C + 64) * TLD * 2 <= dqk_lds_bytes(C),
                "the dv tiles fit the shared arena");
  static_assert(C * LD <= C * KLD, "the output staging fits the Kh block's space");
  OpT* ksh = (OpT*)arena;        // Kh block [t][k]
  OpT* dsT = ksh + C * KLD;      // dS block transposed [v][k]
  OpT* aT = dsT + 64 * LD;       // A^T [s][t]
  OpT* doT = aT + C * TLD;       // dO^T [v][t]
  // the dv tiles of one chunk share Kh and A (consecutive logical ids)
  const int nvt = dv / 64, NJ = dk / 64;
  const int vt = lt % nvt, i = (lt / nvt) % N, bh = lt / (nvt * N);
  const int v0 = vt * 64, t0 = i * C, rows = min(C, T - t0);
  const int w = wave_id(), l = lane_id(), r = l & 15;
  const OpT* Khc = Kh + ((long)bh * N * C + t0) * dk;
  const OpT* dSb = dS + ((long)bh * N + i) * dk * dv;   // the chunk's dS (SFRAG: fragment order)
  const OpT* dSc = dSb + v0;
  // The dk blocks' Kh and dS^T tiles (dk <= 256: at most four) are loaded into registers
  // two blocks ahead of their use, so that a block's round trip overlaps two blocks of
  // products rather than one (all four at once cost more L2 hits than it saved).  Block
  // indices past the last are clamped (loaded, staged, never used): no branch around a
  // load or its first use, so the compiler's wait counts stay exact.
  constexpr int MJ = 4;
  RowTile<OpT, C, 64, KLD> tk[MJ];
  // transposed tiles are staged chunk-swizzled (conflict-free stores)
  ColTile<OpT, OpT, 64, LD, kThreads, true> ts[MJ];
  auto load_blk = [&](int jb) {
    const int jc = min(jb, NJ - 1);
    tk[jb].load(Khc + 64 * jc, dk, C);
    if constexpr (SFRAG) ts[jb].load_frag(dSb, dv, 64 * jc, v0);
    else ts[jb].load(dSc + (long)64 * jc * dv, dv, 64);
  };
  {
    // A^T in 64-column slices of A (its s index), dO^T
    ColTile<OpT, OpT, C, TLD, kThreads, true> ta[C / 64];
    ColTile<OpT, Tin, C, TLD, kThreads, true> to;
#pragma unroll
    for (int h = 0; h < C / 64; ++h) ta[h].load(A + ((long)bh * N + i) * C * C + 64 * h, C, C);
    to.load(dO + ((long)bh * T + t0) * dv + v0, dv, rows);
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) load_blk(jb);
#pragma unroll
    for (int h = 0; h < C / 64; ++h) ta[h].store(aT + 64 * h * TLD);
    to.store(doT);
    tk[0].store(ksh);
    ts[0].store(dsT);
  }
  __syncthreads();
  f32x4 acc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < C / 32; ++kb) {
    Frag<OpT> fb;
    load_frag_cs(fb, doT, TLD, 16 * w + r, kb);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (32 * kb + 31 >= 16 * m) {
        Frag<OpT> fa;
        load_frag_cs(fa, aT, TLD, 16 * m + r, kb);
        mma(acc[m], fa, fb);
      }
    }
  }
#pragma unroll
  for (int jb = 0; jb < MJ; ++jb) {
    if (jb + 2 < MJ) load_blk(jb + 2);
    if (jb < NJ) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Frag<OpT> fb;
        load_frag_cs(fb, dsT, LD, 16 * w + r, kb);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          Frag<OpT> fa;
          load_frag_c(fa, ksh + (16 * m + r) * KLD + kb * 32);
          mma(acc[m], fa, fb);
        }
      }
    }
    __syncthreads();
    if (jb + 1 < MJ) {
      tk[jb + 1].store(ksh);
      ts[jb + 1].store(dsT);
      __syncthreads();
    }
  }
  Tin* outs = (Tin*)ksh;   // [C][LD], inside the Kh block's space
  const int qd = l >> 4;
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      outs[(16 * m + 4 * qd + e) * LD + 16 * w + r] = from_f32<Tin>(acc[m][e]);
  __syncthreads();
  constexpr int kPer = 16 / (int)sizeof(Tin), kUnits = C * 64 / kPer;
  for (int idx = threadIdx.x; idx < kUnits; idx += kThreads) {
    const int e0 = idx * kPer, rr = e0 / 64, cc = e0 % 64;
    if (rr < rows)
      stream16(dv_out + ((long)bh * T + t0 + rr) * dv + v0 + cc,
               *reinterpret_cast<const u32x4*>(outs + rr * LD + cc));
  }
}

// =====================================================================================
// chunk 128: k_bwd_chunk (everything in one workgroup per chunk)
// =====================================================================================
template <int C, int DK, typename Tin, typename OpT>
struct BwdLds {
  static constexpr int DB = (C == 64) ? 64 : 32;
  using IL = IntraLds<C, DB, Tin>;
  static constexpr int ALD = C + 8;
  static constexpr int o_dA = 0;
  static constexpr int o_blk = o_dA + C * IL::FLD * 4;
  static constexpr int end12 = o_blk + IL::bytes_blk;
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
  using BL = BwdLds<C, DK, Tin, OpT>;
  using IL = typename BL::IL;
  constexpr int NM = C / 16, DB = BL::DB, ALD = BL::ALD, FLD = IL::FLD;
  constexpr int CT = DB / 16, MG = 4 / CT, NMW = NM / MG;
  __shared__ __attribute__((aligned(16))) char arena[BL::bytes];
  IL L;
  L.dAs = (float*)(arena + BL::o_dA);
  L.gs = (float*)(arena + BL::o_blk);
  L.qs = (Tin*)(arena + BL::o_blk + C * IL::GLD * 4);
  L.ks = L.qs + C * IL::XLD;
  L.dqd = (float*)(L.ks + C * IL::XLD);
  L.dkd = L.dqd + C * IL::GLD;

  const int i = blockIdx.x, bh = blockIdx.y;
  const int t0 = i * C, rows = min(C, T - t0);
  const int w = wave_id(), l = lane_id(), r = l & 15, qd = l >> 4;
  const long tok0 = (long)bh * T + t0;

  // phase 1: dA = tril(dO V^T)
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
        L.dAs[(16 * m + tl) * FLD + 16 * n + r] = (m == n && r > tl) ? 0.f : acc[e];
      }
    }
  }

  const int ct = w % CT, mg = w / CT;
  const OpT* Si = S + ((long)bh * N + i) * DK * dv;
  const OpT* dSi = dS + ((long)bh * N + i) * DK * dv;

  // phase 2: dq, dk, D per dk block
  for (int d0 = 0; d0 < DK; d0 += DB) {
    bwd_stage_block<C, DB, DK, Tin>(L, q, k, g, tok0, rows, d0);
    const int c = 16 * ct + r;
    f32x4 adq[NMW], adk[NMW];
#pragma unroll
    for (int jj = 0; jj < NMW; ++jj) {
      adq[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
      adk[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
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
    bwd_finish_block<C, DB, DK, NMW, MG, Tin, OpT>(L, adq, adk, dq, dk_out, Dloc, tok0, rows, d0,
                                                   ct, mg);
  }

  // phase 3: dv = Kh dS_[i+1] + A^T dO
  {
    OpT* ATs = (OpT*)(arena + BL::o_AT);
    OpT* dOT = (OpT*)(arena + BL::o_dOT);
    OpT* dST = (OpT*)(arena + BL::o_dST);
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

// The two chunk-64 backward kernels as one launch: dq / dk / dlog_alpha workgroups and dv
// workgroups interleaved in proportion (a dv workgroup needs neither the chunk totals nor
// anything the dq / dk workgroups write), so that their memory phases overlap on each CU.
template <typename Tin, typename OpT, bool SFRAG, bool SG, int C>
__global__ __launch_bounds__(kThreads, C == 64 ? 3 : 1) void k_bwd_dqk_dv(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ dO, int gscalar, const OpT* __restrict__ S,
    const OpT* __restrict__ dS, Tin* __restrict__ dq, Tin* __restrict__ dk_out,
    const float* __restrict__ tot, const float* __restrict__ cT, const Tin* __restrict__ la,
    GateFn gf, Tin* __restrict__ dla, float* __restrict__ dla_part, const OpT* __restrict__ Kh,
    const OpT* __restrict__ A, Tin* __restrict__ dv_out, int T, int dk, int dv, int N,
    int n_dqk) {
  __shared__ __attribute__((aligned(16))) char arena[dqk_lds_bytes(C)];
  const int L = xcd_logical(blockIdx.x, gridDim.x);
  const long total = gridDim.x;
  // Bresenham split: logical id L is a dq/dk workgroup when the count of them up to L grows
  const int before = (int)(((long)L * n_dqk) / total), upto = (int)(((long)(L + 1) * n_dqk) / total);
  if (upto > before)
    bwd_dqk_body<Tin, OpT, SFRAG, SG, C>(arena, before, q, k, v, dO, gscalar, S, dS, dq, dk_out, tot, cT, la, gf,
                           dla, dla_part, T, dk, dv, N);
  else
    bwd_dv_body<Tin, OpT, SFRAG, C>(arena, L - before, Kh, A, dS, dO, dv_out, T, dk, dv, N);
}

// ---------------------------------------------------------------------------------
template <typename Tin, typename OpT, int C, int DK>
static hipError_t launch_bwd_t2(const BwdArgs& a, hipStream_t s) {
  if constexpr (sizeof(OpT) == 2) {
    const int n_dqk = (a.dk / 64) * a.N * a.BH, n_dv = (a.dv / 64) * a.N * a.BH;
    // scalar gates: the C x C decay-matrix form of the intra-chunk terms; fragment-order
    // states come with chunk 64 only (the scans' 128-column tiles)
    auto kern = a.gscalar ? (a.s_frag ? k_bwd_dqk_dv<Tin, OpT, C == 64, true, C> : k_bwd_dqk_dv<Tin, OpT, false, true, C>)
                          : (a.s_frag ? k_bwd_dqk_dv<Tin, OpT, C == 64, false, C> : k_bwd_dqk_dv<Tin, OpT, false, false, C>);
    hipLaunchKernelGGL(kern, dim3(n_dqk + n_dv), dim3(kThreads), 0, s,
                       (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.v, (const Tin*)a.dO,
                       a.gscalar ? 1 : 0, (const OpT*)a.S, (const OpT*)a.dS, (Tin*)a.dq,
                       (Tin*)a.dk_out, a.tot, a.cT,
                       (const Tin*)a.la, a.gate, (Tin*)a.dla, a.dla_part, (const OpT*)a.Kh,
                       (const OpT*)a.A, (Tin*)a.dv_out, a.T, a.dk, a.dv, a.N, n_dqk);
  } else {
    hipLaunchKernelGGL((k_bwd_chunk<Tin, OpT, C, DK>), dim3(a.N, a.BH), dim3(kThreads), 0, s,
                       (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.v, (const Tin*)a.dO, a.g,
                       (const OpT*)a.A, (const OpT*)a.Kh, (const OpT*)a.S, (const OpT*)a.dS,
                       (Tin*)a.dq, (Tin*)a.dk_out, (Tin*)a.dv_out, a.Dloc, a.T, a.dv, a.N);
  }
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

bool bwd_split(int dtype, int C) { return dtype != 0 && (C == 64 || C == 128); }

hipError_t launch_bwd_chunk(const BwdArgs& a, hipStream_t s) {
  if (a.BH == 0 || a.N == 0) return hipSuccess;
  if (a.dtype == 0) return launch_bwd_t<float, float, 64>(a, s);
  if (a.C == 64) return launch_bwd_t<bf16, bf16, 64>(a, s);
  return launch_bwd_t<bf16, bf16, 128>(a, s);
}


}  // namespace gla
