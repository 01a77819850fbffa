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
// The dq/dk workgroups finish the gate gradient themselves: the chunk-local suffix sums
// of D plus the carry of the later chunks' totals, which the two state scans form from
// their fp32 states (summed by the gate-total kernel before this launch).
//
// Kernel
//   k_bwd_dqk_dv (bf16 with chunk 64 or 128, fp32 with chunk 64) two kinds of workgroup,
//   interleaved in one launch (chunk 64), or in a launch each (chunk 128, where the dq/dk
//   workgroups' LDS would otherwise hold the dv workgroups to one per CU as well):
//   dq/dk part  dq, dk and dlog_alpha per (chunk, 64-wide dk block): D as
//              chunk-local suffix sums plus the carry from the later chunks' totals
//              (formed by the gate-total kernel from the scans).  One pass over
//              64-wide dv blocks accumulates dA, dO S^T and V dS^T together: dO and V
//              tiles go through LDS (shared by the 4 waves), each wave's S / dS fragments
//              are prefetched straight into registers (double-buffered); then the
//              intra-chunk part of the block.
//   dv part     dv = A^T dO + Kh dS per (chunk, 64 values), looping over 64-wide dk
//              blocks.
//   fp32 operands take tiles with rows padded for 4-byte elements, unswizzled
//   transposed staging and the off-diagonal products as plain fp32 MFMAs (two
//   workgroups per CU); chunk 128 keeps two dA row tiles per wave (dq/dk workgroups one
//   per CU, dv workgroups two).
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

// =====================================================================================
// chunk 64, dq/dk part: one workgroup per (batch*head, chunk, 64-wide dk block)
// =====================================================================================
// Wave w owns columns 16w .. 16w+15 of the block for all 64 rows of the chunk (four
// accumulator tiles each for dq and dk).  dA = tril(dO V^T) is formed by every dk block of
// the chunk (it is cheap next to the dO S^T and V dS^T products, and keeps the blocks
// independent).  Three workgroups fit on a CU, so one's loads overlap another's math.
// LDS of a dq/dk workgroup for chunk C and ES-byte elements: dA [C][C + 4] fp32, the
// region of the staged g block [C][68] and of g^T [64][C + 4] fp32, q and k [C][72]
constexpr int dqk_lds_bytes(int C, int ES = 2) {
  return C * (C + 4) * 4 + (C * 68 > 64 * (C + 4) ? C * 68 : 64 * (C + 4)) * 4 + 2 * C * 72 * ES;
}
constexpr int kDqkLds = dqk_lds_bytes(64);
// LDS of a dv workgroup: the Kh block [C][row pad], the dS^T tile [64][64 + pad], A^T and
// dO^T [C + 64][C + pad] (see bwd_dv_body)
constexpr int dv_lds_bytes(int C, int ES = 2) {
  return C * (ES == 2 ? 80 : 68) * ES + 64 * (ES == 2 ? 72 : 68) * ES +
         (C + 64) * (ES == 2 ? C + 8 : C + 4) * ES;
}
// Row pad of a row-major 64-wide fragment-source tile in LDS: bf16 rows of 80 elements,
// fp32 rows of 68 (16-byte fragment reads of 16 consecutive rows on distinct banks)
template <typename T> constexpr int frag_row_ld() { return sizeof(T) == 2 ? 64 + 16 : 64 + 4; }
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
  constexpr int ES = sizeof(Tin), NM = C / 16, NS = C / 16, YLD = frag_row_ld<OpT>();
  constexpr int NRT = NM / 4;   // dA row tiles per wave: w, w + 4, ...
  constexpr int FLD = C + 4, GLD = 64 + 4, XLD = 64 + 8;
  constexpr int GTLD = C + 4;   // g^T rows (a column's C rows)
  // LDS: dA [C][FLD] fp32, then a region that holds the dO / V tiles during the dv loop,
  // then the staged g block [C][GLD] and in its place g^T [64 columns][GTLD] fp32 (a
  // column's rows contiguous: the post-loop phases read 4 to 16 consecutive rows of one
  // column), q, k [C][XLD] afterwards.  Chunk 64: 53248 bytes (bf16), three workgroups per
  // CU, or 71680 (fp32), two; chunk 128: 139264 bytes, one.
  constexpr int GBYTES = (C * GLD > 64 * GTLD ? C * GLD : 64 * GTLD) * 4;
  constexpr int o_u = C * FLD * 4, o_q = o_u + GBYTES, o_k = o_q + C * XLD * ES;
  constexpr int bytes = o_k + C * XLD * ES;
  static_assert(2 * C * YLD * ES <= bytes - o_u, "dO / V tiles fit the shared region");
  static_assert(bytes == dqk_lds_bytes(C, ES), "arena size");
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
    // (fp32 operands: one exact part)
    constexpr bool P3 = sizeof(OpT) == 2;
    auto split3 = [](float x, Frag<OpT>& h, Frag<OpT>& md, Frag<OpT>& lo, int e) {
      h.set(e, x);
      if constexpr (P3) {
        const float r1 = x - h.get(e);
        md.set(e, r1);
        lo.set(e, r1 - md.get(e));
      }
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
          if constexpr (P3) {
            mma(tq, md, fb);
            mma(tq, lo, fb);
          }
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
          if constexpr (P3) {
            mma(tk, md, fb);
            mma(tk, lo, fb);
          }
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
  static_assert(3 * C * SLD * (int)sizeof(Tin) <= bytes, "staging fits the arena (q, k dead)");
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
// Fragment read from a transposed tile staged by ColTile: row c, elements 32 kb + 8 q ..
// (bf16: the chunk swizzle; fp32: plain rows)
__device__ __forceinline__ void frag_t(Frag<bf16>& f, const bf16* t, int ld, int c, int kb) {
  load_frag_cs(f, t, ld, c, kb);
}
__device__ __forceinline__ void frag_t(Frag<float>& f, const float* t, int ld, int c, int kb) {
  load_frag_c(f, t + c * ld + kb * 32);
}

template <typename Tin, typename OpT, bool SFRAG, int C>
__device__ __forceinline__ void bwd_dv_body(char* __restrict__ arena, int lt,
                                            const OpT* __restrict__ Kh,
                                            const OpT* __restrict__ A,
                                            const OpT* __restrict__ dS,
                                            const Tin* __restrict__ dO,
                                            Tin* __restrict__ dv_out, int T, int dk, int dv,
                                            int N) {
  // the Kh block is read row-major (rows padded for conflict-free fragment reads); bf16
  // transposed tiles through the swizzle of ColTile (rows of 72), fp32 ones unswizzled in
  // rows of 68
  // LD: rows of 64 (the dS^T tile, the output staging); TLD: rows of C tokens (A^T, dO^T)
  constexpr bool SW = sizeof(OpT) == 2;
  constexpr int ES = sizeof(OpT), NM = C / 16, LD = SW ? 64 + 8 : 64 + 4, TLD = SW ? C + 8 : C + 4;
  constexpr int KLD = frag_row_ld<OpT>();
  static_assert(C * KLD * ES + 64 * LD * ES + (C + 64) * TLD * ES <= dqk_lds_bytes(C, ES),
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
  ColTile<OpT, OpT, 64, LD, kThreads, SW> ts[MJ];
  auto load_blk = [&](int jb) {
    const int jc = min(jb, NJ - 1);
    tk[jb].load(Khc + 64 * jc, dk, C);
    if constexpr (SFRAG) ts[jb].load_frag(dSb, dv, 64 * jc, v0);
    else ts[jb].load(dSc + (long)64 * jc * dv, dv, 64);
  };
  {
    // A^T in 64-column slices of A (its s index), dO^T
    ColTile<OpT, OpT, C, TLD, kThreads, SW> ta[C / 64];
    ColTile<OpT, Tin, C, TLD, kThreads, SW> to;
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
    frag_t(fb, doT, TLD, 16 * w + r, kb);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (32 * kb + 31 >= 16 * m) {
        Frag<OpT> fa;
        frag_t(fa, aT, TLD, 16 * m + r, kb);
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
        frag_t(fb, dsT, LD, 16 * w + r, kb);
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

// The two backward chunk kernels as one launch (MODE 0): dq / dk / dlog_alpha workgroups
// and dv workgroups interleaved in proportion (a dv workgroup needs neither the chunk
// totals nor anything the dq / dk workgroups write), so that their memory phases overlap
// on each CU.  MODE 1 / 2: one kind only, in a launch of its own, with its own LDS size.
template <typename Tin, typename OpT, bool SFRAG, bool SG, int C, int MODE = 0>
__global__ __launch_bounds__(kThreads, MODE == 2 ? 2 : C == 128 ? 1 : sizeof(OpT) == 2 ? 3 : 2) void k_bwd_dqk_dv(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ dO, int gscalar, const OpT* __restrict__ S,
    const OpT* __restrict__ dS, Tin* __restrict__ dq, Tin* __restrict__ dk_out,
    const float* __restrict__ tot, const float* __restrict__ cT, const Tin* __restrict__ la,
    GateFn gf, Tin* __restrict__ dla, float* __restrict__ dla_part, const OpT* __restrict__ Kh,
    const OpT* __restrict__ A, Tin* __restrict__ dv_out, int T, int dk, int dv, int N,
    int n_dqk) {
  __shared__ __attribute__((aligned(16)))
  char arena[MODE == 2 ? dv_lds_bytes(C, sizeof(OpT)) : dqk_lds_bytes(C, sizeof(OpT))];
  const int L = xcd_logical(blockIdx.x, gridDim.x);
  if constexpr (MODE == 1) {
    bwd_dqk_body<Tin, OpT, SFRAG, SG, C>(arena, L, q, k, v, dO, gscalar, S, dS, dq, dk_out, tot,
                                         cT, la, gf, dla, dla_part, T, dk, dv, N);
  } else if constexpr (MODE == 2) {
    bwd_dv_body<Tin, OpT, SFRAG, C>(arena, L, Kh, A, dS, dO, dv_out, T, dk, dv, N);
  } else {
    const long total = gridDim.x;
    // Bresenham split: logical id L is a dq/dk workgroup when the count of them up to L grows
    const int before = (int)(((long)L * n_dqk) / total), upto = (int)(((long)(L + 1) * n_dqk) / total);
    if (upto > before)
      bwd_dqk_body<Tin, OpT, SFRAG, SG, C>(arena, before, q, k, v, dO, gscalar, S, dS, dq, dk_out, tot, cT, la, gf,
                             dla, dla_part, T, dk, dv, N);
    else
      bwd_dv_body<Tin, OpT, SFRAG, C>(arena, L - before, Kh, A, dS, dO, dv_out, T, dk, dv, N);
  }
}

// ---------------------------------------------------------------------------------
template <typename Tin, typename OpT, int C>
static hipError_t launch_bwd_t2(const BwdArgs& a, hipStream_t s) {
  {
    const int n_dqk = (a.dk / 64) * a.N * a.BH, n_dv = (a.dv / 64) * a.N * a.BH;
    // scalar gates: the C x C decay-matrix form of the intra-chunk terms; fragment-order
    // states come with bf16 and chunk 64 only (the scans' 128-column tiles)
    constexpr bool kSF = sizeof(OpT) == 2 && C == 64;
    auto go = [&](auto kern, int nwg) {
      hipLaunchKernelGGL(kern, dim3(nwg), dim3(kThreads), 0, s,
                         (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.v, (const Tin*)a.dO,
                         a.gscalar ? 1 : 0, (const OpT*)a.S, (const OpT*)a.dS, (Tin*)a.dq,
                         (Tin*)a.dk_out, a.tot, a.cT,
                         (const Tin*)a.la, a.gate, (Tin*)a.dla, a.dla_part, (const OpT*)a.Kh,
                         (const OpT*)a.A, (Tin*)a.dv_out, a.T, a.dk, a.dv, a.N, n_dqk);
    };
    if constexpr (C == 128) {
      // one dq/dk workgroup per CU (139 KB of LDS): the dv workgroups run in a launch of
      // their own at two per CU
      if (a.gscalar) go(k_bwd_dqk_dv<Tin, OpT, false, true, C, 1>, n_dqk);
      else go(k_bwd_dqk_dv<Tin, OpT, false, false, C, 1>, n_dqk);
      go(k_bwd_dqk_dv<Tin, OpT, false, false, C, 2>, n_dv);
    } else {
      auto kern = a.gscalar ? (a.s_frag ? k_bwd_dqk_dv<Tin, OpT, kSF, true, C> : k_bwd_dqk_dv<Tin, OpT, false, true, C>)
                            : (a.s_frag ? k_bwd_dqk_dv<Tin, OpT, kSF, false, C> : k_bwd_dqk_dv<Tin, OpT, false, false, C>);
      go(kern, n_dqk + n_dv);
    }
  }
  return hipGetLastError();
}

hipError_t launch_bwd_chunk(const BwdArgs& a, hipStream_t s) {
  if (a.BH == 0 || a.N == 0) return hipSuccess;
  if (a.dtype == 0) return a.C == 64 ? launch_bwd_t2<float, float, 64>(a, s) : hipErrorInvalidValue;
  if (a.C == 64) return launch_bwd_t2<bf16, bf16, 64>(a, s);
  return launch_bwd_t2<bf16, bf16, 128>(a, s);
}


}  // namespace gla
