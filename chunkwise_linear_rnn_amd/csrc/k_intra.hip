// Intra-chunk kernel of the chunkwise GLA path (page "Gated Linear Attention Transformers
// with Hardware-Efficient Training", atlas.scime.ai summary, section Approach: two-level
// (secondary) chunking so that most intra-chunk products run on half-precision matrix
// units).  One workgroup per (batch*head, chunk).
//
// It forms the chunk's decayed causal attention matrix
//     A[t][s] = sum_d q_td k_sd exp(g_td - g_sd),  s <= t  (zero above the diagonal)
// with g the chunk-local cumsum of log_alpha, split into 16-row sub-chunks:
//   - a sub-block with t in sub-chunk I and s in an earlier sub-chunk J is the MFMA
//     product (Q_I * exp(g_I - g_rho)) (K_J * exp(g_rho - g_J))^T, rho = first row of I;
//     both exponents are <= 0, so the rounded (bf16) operands stay in [0, |x|];
//   - a diagonal sub-block stays in fp32 (most, not all, intra-chunk products run on
//     the half-precision units).  When the spread of g inside the sub-block is moderate
//     (at most kDiagRange in log2 units, in every column) it is the same product on q and
//     k rebased at the sub-block's first row, with fp32 operands and fp32 MFMA: the key
//     factor exp(g_rho - g_s) is at most 2^96 and the query factor at least 2^-96, both
//     normal fp32 numbers, so each term carries fp32 rounding only.  Otherwise it is
//     summed element by element in fp32 from log-space differences exp(g_t - g_s), which
//     is in [0,1] for any finite gates.  DIAG_BF16 (opt-in) takes the rebased product
//     with bf16 operands instead, at the off-diagonal sub-blocks' operand rounding.
// Alongside it emits, for the chunk, the decayed operands the inter-chunk kernels
// consume (each nullable): Qh = q*exp(g) token-major, its transpose QhT, Kh =
// k*exp(gamma - g) token-major, its transpose KhT, and exp(gamma).  The transposed
// operands feed the state scans; they are written either in the MFMA operand type or
// (XT = float with bf16 operands) as a bf16 high part plus bf16 remainder per row, which
// the backward's scans feed to two MFMAs so the states carry no operand rounding.
//
// g is computed here from log_alpha (through the gate front-end) by a segmented column
// scan, the same one the gate-cumsum kernel runs.  Internally g is held multiplied by
// log2(e) so every decay is one v_exp_f32; g2_out (nullable) receives it for the
// backward chunk kernel.
#include <type_traits>

#include "gla_common.cuh"
#include "gla_gate.cuh"
#include "gla_internal.h"

namespace gla {

// (t, s) of the p-th entry, row-major, of a 16x16 lower triangle with its diagonal.
__device__ __forceinline__ void tri_decode(int p, int& t, int& s) {
  int tt = (int)((sqrtf(8.f * (float)p + 1.f) - 1.f) * 0.5f);
  if ((tt + 1) * (tt + 2) / 2 <= p) ++tt;
  if (tt * (tt + 1) / 2 > p) --tt;
  t = tt;
  s = p - tt * (tt + 1) / 2;
}
// (I, J), J < I, of the p-th strictly-lower sub-chunk pair, ordered by I then J.
__device__ __forceinline__ void pair_decode(int p, int& I, int& J) {
  int ii = (int)((sqrtf(8.f * (float)p + 1.f) + 1.f) * 0.5f);
  if (ii * (ii - 1) / 2 > p) --ii;
  if ((ii + 1) * ii / 2 <= p) ++ii;
  I = ii;
  J = p - ii * (ii - 1) / 2;
}

// One 8-token piece x[0..8) (tokens r8 .. r8 + 7 of the chunk, key dimension d) of a
// chunk's transposed decayed operand, in the layout the inter-chunk kernels read:
//  - XT = float with bf16 operands (the backward's scans): MFMA fragment order, for 16-row
//    block d / 16 and 32-token block kb of the chunk the 64 lanes' 16-byte pieces of the
//    bf16 high part, then of the bf16 remainder; this piece belongs to lane 16 q + d % 16;
//  - XT = bf16: the same fragment order, one plane;
//  - XT = float with fp32 operands: rows [dk][C], token-contiguous.
// bhi = batch*head * N + chunk.
template <typename OpT, typename XT, int C>
__device__ __forceinline__ void store_xt(XT* __restrict__ dst, long bhi, int dk, int d, int r8,
                                         const float (&x)[8]) {
  constexpr bool kSplit = sizeof(XT) == 4 && sizeof(OpT) == 2;
  if constexpr (kSplit || sizeof(XT) == 2) {
    const int j = r8 / 8, kb = j / 4, qd = j % 4;
    const long f = (bhi * (dk / 16) + d / 16) * (C / 32) + kb;
    if constexpr (kSplit) {
      bf16* b = reinterpret_cast<bf16*>(dst) + ((f * 2) * 64 + 16 * qd + d % 16) * 8;
      float lo[8];
      bf16x8 hv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hv[e] = (bf16)x[e];
        lo[e] = x[e] - (float)hv[e];
      }
      *reinterpret_cast<bf16x8*>(b) = hv;
      store8(b + 64 * 8, lo);
    } else {
      store8(dst + (f * 64 + 16 * qd + d % 16) * 8, x);
    }
  } else {
    store8(dst + (bhi * dk + d) * C + r8, x);
  }
}

template <typename Tin, typename OpT, typename XT, int C, bool WANT_A, bool DIAG_BF16>
__global__ __launch_bounds__(kThreads) void k_intra(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ la,
    OpT* __restrict__ A_out, OpT* __restrict__ Qh_out,
    XT* __restrict__ QhT_out, OpT* __restrict__ Kh_out, XT* __restrict__ KhT_out,
    float* __restrict__ eg_out, float* __restrict__ g2_out, GateFn gf, int T, int dk, int N) {
  constexpr int DB = 64;                    // dk columns per pass
  constexpr int NS = C / 16;                // sub-chunks
  constexpr int NPAIR = NS * (NS - 1) / 2;  // off-diagonal sub-block pairs
  constexpr int PPW = (NPAIR + 3) / 4;      // pairs per wave
  constexpr int NITEM = NS * 136 * 4;       // diagonal (pair, 16-column quarter) items
  constexpr int NDW = (NS + 3) / 4;         // diagonal sub-blocks per wave (MFMA path)
  // largest spread of g * log2 e inside a 16-row sub-block for which the diagonal
  // sub-blocks take the rebased MFMA path (factors within 2^+-kDiagRange of the inputs)
  constexpr float kDiagRange = 96.f;
  // operands of the rebased diagonal product: fp32 (fp32 MFMA), or bf16 when opted in
  using DFrag = typename std::conditional<DIAG_BF16, Frag<OpT>, Frag<float>>::type;
  constexpr int IPT = (NITEM + kThreads - 1) / kThreads;
  constexpr int GLD = DB + 4;
  constexpr int XLD = DB + 8;

  __shared__ __attribute__((aligned(16))) float gs[C * GLD];
  __shared__ __attribute__((aligned(16))) Tin qs[C * XLD];
  __shared__ __attribute__((aligned(16))) Tin ks[C * XLD];
  __shared__ float segtot[4 * DB];
  __shared__ float dacc[WANT_A ? NITEM : 1];

  const int i = blockIdx.x, bh = blockIdx.y;
  const int t0 = i * C, rows = min(C, T - t0);
  const int w = wave_id(), l = lane_id(), r = l & 15, qd = l >> 4;
  const long in_base = ((long)bh * T + t0) * dk;

  // off-diagonal sub-blocks accumulate in registers, the diagonal items (each owned by
  // one thread across the dk blocks) in LDS
  f32x4 accp[PPW > 0 ? PPW : 1], accd[NDW];
#pragma unroll
  for (int p = 0; p < (PPW > 0 ? PPW : 1); ++p) accp[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < NDW; ++p) accd[p] = f32x4{0.f, 0.f, 0.f, 0.f};
  // some pass took the log-space diagonal sums (their partials are in dacc, which the
  // first such pass initializes: each item is only ever touched by its own thread there)
  bool anywide = false;

  // The next dk block's log_alpha (or gate logits), q and k are loaded into registers
  // while the current block computes.
  GBlock<Tin, C, DB> pg;
  RowTile<Tin, C, DB, XLD> tq, tk;
  auto fetch = [&](int d0) {
    // rows past T zero (after the gate front-end too): they never decay the chunk
    pg.load(la + in_base + d0, dk, rows, false);
    tq.load(q + in_base + d0, dk, rows);
    tk.load(k + in_base + d0, dk, rows);
  };
  fetch(0);

  for (int d0 = 0; d0 < dk; d0 += DB) {
    // ---- g block (times log2 e), q, k -------------------------------------------------
    // log_alpha (or logits, through the gate front-end gf)
    pg.store(gs, GLD, gf);
    tq.store(qs);
    tk.store(ks);
    fetch(min(d0 + DB, dk - DB));   // unconditional (exact wait counts); the last refetches
    // wide: some 16-row sub-block of this block has a spread of g beyond kDiagRange
    // chunk-local cumsum down each column; its spread decides at the barrier after it
    __syncthreads();
    const bool wide =
        __syncthreads_or(!(chunk_cumsum_cols<C, DB>(gs, GLD, segtot) <= kDiagRange));
    if (g2_out) {   // g * log2 e for the backward chunk kernel
#pragma unroll
      for (int u_ = 0; u_ < (C * (DB / 8) + kThreads - 1) / kThreads; ++u_) {   // fixed trip count
        const int idx = threadIdx.x + u_ * kThreads;
        if ((C * (DB / 8)) % kThreads != 0 && idx >= C * (DB / 8)) continue;
        const int rr = idx / (DB / 8), c = (idx % (DB / 8)) * 8;
        if (rr < rows) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = gs[rr * GLD + c + e];
          stream8(g2_out + in_base + (long)rr * dk + d0 + c, x);
        }
      }
    }

    // ---- decayed operands for the inter-chunk kernels ---------------------------------
    const float* glast = gs + (C - 1) * GLD;   // gamma * log2 e
    if (eg_out && threadIdx.x < DB)
      eg_out[((long)bh * N + i) * dk + d0 + threadIdx.x] = __builtin_amdgcn_exp2f(glast[threadIdx.x]);
    if (Qh_out || Kh_out) {
#pragma unroll
      for (int u_ = 0; u_ < (C * (DB / 8) + kThreads - 1) / kThreads; ++u_) {   // fixed trip count
        const int idx = threadIdx.x + u_ * kThreads;
        if ((C * (DB / 8)) % kThreads != 0 && idx >= C * (DB / 8)) continue;
        const int rr = idx / (DB / 8), c = (idx % (DB / 8)) * 8;
        const long o = ((long)bh * N * C + t0 + rr) * dk + d0 + c;
        float x[8];
        if (Qh_out) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            x[e] = to_f32(qs[rr * XLD + c + e]) * __builtin_amdgcn_exp2f(gs[rr * GLD + c + e]);
          store8(Qh_out + o, x);   // re-read at once by the fused forward: kept cacheable
        }
        if (Kh_out) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            x[e] = to_f32(ks[rr * XLD + c + e]) *
                   __builtin_amdgcn_exp2f(glast[c + e] - gs[rr * GLD + c + e]);
          stream8(Kh_out + o, x);
        }
      }
    }
    if (QhT_out || KhT_out) {
#pragma unroll
      for (int u_ = 0; u_ < (DB * (C / 8) + kThreads - 1) / kThreads; ++u_) {   // fixed trip count
        const int idx = threadIdx.x + u_ * kThreads;
        if ((DB * (C / 8)) % kThreads != 0 && idx >= DB * (C / 8)) continue;
        // a wave takes 32 columns x two 8-row groups of opposite parity, so that its
        // column reads of the g, q, k tiles fall on distinct LDS banks
        const int lw = idx & 63, wv = idx >> 6;
        const int c = 32 * (wv & 1) + (lw & 31), r8 = 8 * (2 * (wv >> 1) + (lw >> 5));
        float x[8];
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
          XT* dst = pass == 0 ? QhT_out : KhT_out;
          if (!dst) continue;
          if (pass == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              x[e] = to_f32(qs[(r8 + e) * XLD + c]) * __builtin_amdgcn_exp2f(gs[(r8 + e) * GLD + c]);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              x[e] = to_f32(ks[(r8 + e) * XLD + c]) *
                     __builtin_amdgcn_exp2f(glast[c] - gs[(r8 + e) * GLD + c]);
          }
          store_xt<OpT, XT, C>(dst, (long)bh * N + i, dk, d0 + c, r8, x);
        }
      }
    }

    if constexpr (WANT_A) {
      // ---- off-diagonal sub-blocks: MFMA on rebased operands ----------------------------
#pragma unroll
      for (int pi = 0; pi < PPW; ++pi) {
        const int p = w + 4 * pi;
        if (p < NPAIR) {
          int I, J;
          pair_decode(p, I, J);
          const int rho = 16 * I, tr = 16 * I + r, sk = 16 * J + r;
#pragma unroll 1
          for (int kb = 0; kb < DB / 32; ++kb) {
            const int c0 = kb * 32 + 8 * qd;
            Frag<OpT> fa, fb;
            float gr[8], gq[8], gk[8], xq[8], xk[8];
            load8(gr, gs + rho * GLD + c0);
            load8(gq, gs + tr * GLD + c0);
            load8(gk, gs + sk * GLD + c0);
            load8(xq, qs + tr * XLD + c0);
            load8(xk, ks + sk * XLD + c0);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              fa.set(e, xq[e] * __builtin_amdgcn_exp2f(gq[e] - gr[e]));
              fb.set(e, xk[e] * __builtin_amdgcn_exp2f(gr[e] - gk[e]));
            }
            mma(accp[pi], fa, fb);
          }
        }
      }
      // ---- diagonal sub-blocks ------------------------------------------------------
      // When the gates' spread inside every 16-row sub-block is moderate (the usual
      // case), an MFMA on operands rebased at the sub-block's first row, fp32 unless
      // opted into bf16 (entries above the diagonal are dropped when the block is
      // written); otherwise the exact fp32 log-space sum per (t, s, column).
      if (!wide) {
#pragma unroll
        for (int dI = 0; dI < NDW; ++dI) {
          const int I = w + 4 * dI;
          if (I < NS) {
            const int rho = 16 * I, tr = 16 * I + r;
#pragma unroll 1
            for (int kb = 0; kb < DB / 32; ++kb) {
              const int c0 = kb * 32 + 8 * qd;
              DFrag fa, fb;
              float gr[8], gq[8], xq[8], xk[8];
              load8(gr, gs + rho * GLD + c0);
              load8(gq, gs + tr * GLD + c0);
              load8(xq, qs + tr * XLD + c0);
              load8(xk, ks + tr * XLD + c0);
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                fa.set(e, xq[e] * __builtin_amdgcn_exp2f(gq[e] - gr[e]));
                fb.set(e, xk[e] * __builtin_amdgcn_exp2f(gr[e] - gq[e]));
              }
              mma(accd[dI], fa, fb);
            }
          }
        }
      } else {
#pragma unroll 1
      for (int item = threadIdx.x; item < NITEM; item += kThreads) {
        {
          const int quarter = item & 3, pr = item >> 2;
          const int I = pr / 136;
          int tt, ss;
          tri_decode(pr % 136, tt, ss);
          const int t = 16 * I + tt, s = 16 * I + ss, cb = quarter * 16;
          float acc = 0.f;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float xq[8], xk[8], gt[8], gsr[8];
            load8(xq, qs + t * XLD + cb + 8 * h);
            load8(xk, ks + s * XLD + cb + 8 * h);
            load8(gt, gs + t * GLD + cb + 8 * h);
            load8(gsr, gs + s * GLD + cb + 8 * h);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += xq[e] * xk[e] * __builtin_amdgcn_exp2f(gt[e] - gsr[e]);
          }
          dacc[item] = (anywide ? dacc[item] : 0.f) + acc;
        }
      }
      anywide = true;
      }
    }
    __syncthreads();
  }

  if constexpr (WANT_A) {
    // The block is assembled in LDS (in the g tile, dead after the last pass) when it fits
    // there, and leaves as 16-byte rows with the entries above the diagonal zeroed on the
    // way; otherwise it is written entry by entry, zeros included.
    OpT* Ab = A_out + ((long)bh * N + i) * C * C;
    constexpr int ALD = C + 8;
    constexpr bool kStageA = C * ALD * (int)sizeof(OpT) <= C * GLD * 4;
    OpT* At = kStageA ? reinterpret_cast<OpT*>(gs) : Ab;
    const int ald = kStageA ? ALD : C;
    if (anywide) {
      // the MFMA part of the diagonal entries (t = 4 qd + e, s = r in sub-block I) joins
      // the log-space part on the first column-quarter item of the entry
#pragma unroll
      for (int dI = 0; dI < NDW; ++dI) {
        const int I = w + 4 * dI;
        if (I < NS) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tt = 4 * qd + e;
            if (r <= tt) dacc[(I * 136 + tt * (tt + 1) / 2 + r) << 2] += accd[dI][e];
          }
        }
      }
    } else {
      // every pass summed the diagonal sub-blocks on the matrix units: they are complete
#pragma unroll
      for (int dI = 0; dI < NDW; ++dI) {
        const int I = w + 4 * dI;
        if (I < NS) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tt = 4 * qd + e;
            At[(16 * I + tt) * ald + 16 * I + r] = from_f32<OpT>(r <= tt ? accd[dI][e] : 0.f);
          }
        }
      }
    }
    if constexpr (!kStageA) {
      for (int idx = threadIdx.x; idx < C * C; idx += kThreads) {   // zero above the diagonal
        const int t = idx / C, s = idx % C;
        if (s / 16 > t / 16) At[t * ald + s] = from_f32<OpT>(0.f);
      }
    }
#pragma unroll
    for (int pi = 0; pi < PPW; ++pi) {
      const int p = w + 4 * pi;
      if (p < NPAIR) {
        int I, J;
        pair_decode(p, I, J);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          At[(16 * I + 4 * qd + e) * ald + 16 * J + r] = from_f32<OpT>(accp[pi][e]);
      }
    }
    if (anywide) {
      __syncthreads();
      // four column-quarter partials of each diagonal entry sit in adjacent lanes
#pragma unroll
      for (int j = 0; j < IPT; ++j) {
        const int item = threadIdx.x + kThreads * j;
        float v = item < NITEM ? dacc[item] : 0.f;
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        if (item < NITEM && (item & 3) == 0) {
          const int pr = item >> 2, I = pr / 136;
          int tt, ss;
          tri_decode(pr % 136, tt, ss);
          At[(16 * I + tt) * ald + 16 * I + ss] = from_f32<OpT>(v);
          if (ss < tt) At[(16 * I + ss) * ald + 16 * I + tt] = from_f32<OpT>(0.f);
        }
      }
    }
    if constexpr (kStageA) {
      constexpr int kPer = 16 / (int)sizeof(OpT), kRowUnits = C / kPer;
      static_assert(C * kRowUnits % kThreads == 0, "whole 16-byte units per thread");
      __syncthreads();
#pragma unroll
      for (int u_ = 0; u_ < C * kRowUnits / kThreads; ++u_) {
        const int idx = threadIdx.x + u_ * kThreads, rr = idx / kRowUnits, cc = (idx % kRowUnits) * kPer;
        union { u32x4 u; OpT x[kPer]; } row;
        row.u = *reinterpret_cast<const u32x4*>(At + rr * ALD + cc);
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          if (cc + j > rr) row.x[j] = from_f32<OpT>(0.f);
        *reinterpret_cast<u32x4*>(Ab + rr * C + cc) = row.u;
      }
    }
  }
}


// Scalar gates: one gate per token and head, shared by every key dimension (the
// data-dependent scalar gate and the data-independent scalar decay that the same summary
// compares with the fine-grained gate, Measured effects and Surprising findings).  The
// decay exp(g_t - g_s) then no longer depends on d and leaves the sum over it:
//     A = tril((Q K^T) * D),   D[t][s] = exp(g_t - g_s),
// one MFMA product of the chunk's q and k over every key dimension (exact products of the
// bf16 inputs, fp32 accumulation; the diagonal sub-blocks included) times the C x C decay
// matrix in fp32: no sub-chunk rebasing and no exponential per element.  The decayed
// operands scale whole rows: Qh = q * exp(g_t), Kh = k * exp(gamma - g_t); exp(gamma) is
// the same for every key dimension.  Same outputs and layouts as k_intra.
template <typename Tin, typename OpT, typename XT, int C, bool WANT_A>
__global__ __launch_bounds__(kThreads) void k_intra_scalar(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ la,
    OpT* __restrict__ A_out, OpT* __restrict__ Qh_out, XT* __restrict__ QhT_out,
    OpT* __restrict__ Kh_out, XT* __restrict__ KhT_out, float* __restrict__ eg_out,
    float* __restrict__ g2_out, GateFn gf, int T, int dk, int N) {
  static_assert(sizeof(Tin) == sizeof(OpT), "operands in the input type");
  constexpr int DB = 64, NS = C / 16, XLD = DB + 8;
  constexpr int NIW = (NS + 3) / 4;   // row tiles of A per wave: I = w + 4 ii
  __shared__ __attribute__((aligned(16))) Tin qs[C * XLD];
  __shared__ __attribute__((aligned(16))) Tin ks[C * XLD];
  __shared__ float gsc[C], pq[C], pk[C], wtot[4];
  const int i = blockIdx.x, bh = blockIdx.y;
  const int t0 = i * C, rows = min(C, T - t0);
  const int w = wave_id(), l = lane_id(), r = l & 15, qd = l >> 4;
  const long in_base = ((long)bh * T + t0) * dk;

  RowTile<Tin, C, DB, XLD> tq, tk;
  auto fetch = [&](int d0) {
    tq.load(q + in_base + d0, dk, rows);
    tk.load(k + in_base + d0, dk, rows);
  };
  fetch(0);

  // g * log2 e per row: the gate front-end (zero past T, so padded rows never decay the
  // chunk), then an inclusive scan over the chunk's rows: shuffles within each wave, then
  // the totals of the waves before
  float x = 0.f;
  if (threadIdx.x < C) {
    const int t = threadIdx.x;
    x = t < rows ? gf(to_f32(la[(long)bh * T + t0 + min(t, rows - 1)])) * kLog2e : 0.f;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float y = __shfl_up(x, off);
      if (l >= off) x += y;
    }
    if (l == kWave - 1) wtot[w] = x;
  }
  __syncthreads();
  if (threadIdx.x < C) {
    for (int u = 0; u < w; ++u) x += wtot[u];
    gsc[threadIdx.x] = x;
  }
  __syncthreads();
  const float gam = gsc[C - 1];
  if (threadIdx.x < C) {
    pq[threadIdx.x] = __builtin_amdgcn_exp2f(gsc[threadIdx.x]);
    pk[threadIdx.x] = __builtin_amdgcn_exp2f(gam - gsc[threadIdx.x]);
  }
  if (eg_out) {
    const float eg = __builtin_amdgcn_exp2f(gam);
    for (int d = threadIdx.x; d < dk; d += kThreads) eg_out[((long)bh * N + i) * dk + d] = eg;
  }

  f32x4 acc[NIW][NS];
#pragma unroll
  for (int ii = 0; ii < NIW; ++ii)
#pragma unroll
    for (int J = 0; J < NS; ++J) acc[ii][J] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int d0 = 0; d0 < dk; d0 += DB) {
    tq.store(qs);
    tk.store(ks);
    fetch(min(d0 + DB, dk - DB));   // unconditional (exact wait counts); the last refetches
    __syncthreads();
    if constexpr (WANT_A) {
      // (Q K^T) over this block's key dimensions, the row tiles of this wave, J <= I
#pragma unroll
      for (int ii = 0; ii < NIW; ++ii) {
        const int I = w + 4 * ii;
        if (I < NS) {
#pragma unroll
          for (int kb = 0; kb < DB / 32; ++kb) {
            Frag<OpT> fa;
            load_frag_c(fa, qs + (16 * I + r) * XLD + kb * 32);
#pragma unroll
            for (int J = 0; J < NS; ++J) {
              if (J <= I) {
                Frag<OpT> fb;
                load_frag_c(fb, ks + (16 * J + r) * XLD + kb * 32);
                mma(acc[ii][J], fa, fb);
              }
            }
          }
        }
      }
    }
    if (g2_out) {   // g * log2 e, the same for every key dimension
#pragma unroll
      for (int u_ = 0; u_ < (C * (DB / 8) + kThreads - 1) / kThreads; ++u_) {   // fixed trip count
        const int idx = threadIdx.x + u_ * kThreads;
        if ((C * (DB / 8)) % kThreads != 0 && idx >= C * (DB / 8)) continue;
        const int rr = idx / (DB / 8), c = (idx % (DB / 8)) * 8;
        if (rr < rows) {
          float y[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = gsc[rr];
          stream8(g2_out + in_base + (long)rr * dk + d0 + c, y);
        }
      }
    }
    if (Qh_out || Kh_out) {
#pragma unroll
      for (int u_ = 0; u_ < (C * (DB / 8) + kThreads - 1) / kThreads; ++u_) {   // fixed trip count
        const int idx = threadIdx.x + u_ * kThreads;
        if ((C * (DB / 8)) % kThreads != 0 && idx >= C * (DB / 8)) continue;
        const int rr = idx / (DB / 8), c = (idx % (DB / 8)) * 8;
        const long o = ((long)bh * N * C + t0 + rr) * dk + d0 + c;
        float y[8];
        if (Qh_out) {
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = to_f32(qs[rr * XLD + c + e]) * pq[rr];
          store8(Qh_out + o, y);
        }
        if (Kh_out) {
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = to_f32(ks[rr * XLD + c + e]) * pk[rr];
          stream8(Kh_out + o, y);
        }
      }
    }
    if (QhT_out || KhT_out) {
#pragma unroll
      for (int u_ = 0; u_ < (DB * (C / 8) + kThreads - 1) / kThreads; ++u_) {   // fixed trip count
        const int idx = threadIdx.x + u_ * kThreads;
        if ((DB * (C / 8)) % kThreads != 0 && idx >= DB * (C / 8)) continue;
        const int lw = idx & 63, wv = idx >> 6;
        const int c = 32 * (wv & 1) + (lw & 31), r8 = 8 * (2 * (wv >> 1) + (lw >> 5));
        float y[8];
        if (QhT_out) {
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = to_f32(qs[(r8 + e) * XLD + c]) * pq[r8 + e];
          store_xt<OpT, XT, C>(QhT_out, (long)bh * N + i, dk, d0 + c, r8, y);
        }
        if (KhT_out) {
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = to_f32(ks[(r8 + e) * XLD + c]) * pk[r8 + e];
          store_xt<OpT, XT, C>(KhT_out, (long)bh * N + i, dk, d0 + c, r8, y);
        }
      }
    }
    __syncthreads();
  }

  if constexpr (WANT_A) {
    // A[t][s] = (Q K^T)[t][s] * exp(g_t - g_s) for s <= t, zero above the diagonal
    OpT* Ab = A_out + ((long)bh * N + i) * C * C;
    for (int idx = threadIdx.x; idx < C * C; idx += kThreads) {
      const int t = idx / C, s2 = idx % C;
      if (s2 > t) Ab[idx] = from_f32<OpT>(0.f);
    }
#pragma unroll
    for (int ii = 0; ii < NIW; ++ii) {
      const int I = w + 4 * ii;
      if (I < NS) {
#pragma unroll
        for (int J = 0; J < NS; ++J) {
          if (J <= I) {
            const int s2 = 16 * J + r;
            const float gs2 = gsc[s2];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int t = 16 * I + 4 * qd + e;
              if (s2 <= t)
                Ab[t * C + s2] = from_f32<OpT>(acc[ii][J][e] * __builtin_amdgcn_exp2f(gsc[t] - gs2));
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
template <typename Tin, typename OpT, typename XT, int C, bool WA, bool DB16 = false>
static void launch_intra_k(const IntraArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_intra<Tin, OpT, XT, C, WA, DB16>), dim3(a.N, a.BH), dim3(kThreads), 0, s,
                     (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.la, (OpT*)a.A, (OpT*)a.Qh,
                     (XT*)a.QhT, (OpT*)a.Kh, (XT*)a.KhT, a.eg, a.g2_out, a.gate, a.T, a.dk, a.N);
}
template <typename Tin, typename OpT, typename XT, int C>
static hipError_t launch_intra_t(const IntraArgs& a, hipStream_t s) {
  if (a.gscalar) {   // scalar gates: the C x C decay-matrix kernel (g formed from the gates)
    auto kern = a.want_A ? k_intra_scalar<Tin, OpT, XT, C, true> : k_intra_scalar<Tin, OpT, XT, C, false>;
    hipLaunchKernelGGL(kern, dim3(a.N, a.BH), dim3(kThreads), 0, s, (const Tin*)a.q,
                       (const Tin*)a.k, (const Tin*)a.la, (OpT*)a.A, (OpT*)a.Qh, (XT*)a.QhT,
                       (OpT*)a.Kh, (XT*)a.KhT, a.eg, a.g2_out, a.gate, a.T, a.dk, a.N);
    return hipGetLastError();
  }
  if (a.want_A) {
    // the bf16 diagonal is an option of bf16 operands only
    if (a.diag_bf16 && sizeof(OpT) == 2) launch_intra_k<Tin, OpT, XT, C, true, true>(a, s);
    else launch_intra_k<Tin, OpT, XT, C, true>(a, s);
  } else {
    launch_intra_k<Tin, OpT, XT, C, false>(a, s);
  }
  return hipGetLastError();
}

hipError_t launch_intra(const IntraArgs& a, hipStream_t s) {
  if (a.BH == 0 || a.N == 0) return hipSuccess;
  if (a.dtype == 0) return launch_intra_t<float, float, float, 64>(a, s);
  if (a.xt_f32) {
    if (a.C == 64) return launch_intra_t<bf16, bf16, float, 64>(a, s);
    return launch_intra_t<bf16, bf16, float, 128>(a, s);
  }
  if (a.C == 64) return launch_intra_t<bf16, bf16, bf16, 64>(a, s);
  return launch_intra_t<bf16, bf16, bf16, 128>(a, s);
}

}  // namespace gla
