// Output kernels of the chunkwise GLA forward (page "Gated Linear Attention Transformers
// with Hardware-Efficient Training", atlas.scime.ai summary, section Approach).
//
//   k_output     materialized states: one workgroup per (batch*head, chunk, 64 values)
//                computes O_i = Qh_i S_[i] + A_i V_i from the chunk-start state written by
//                the state scan ([dv][dk] layout, so both MFMA operands are
//                dk-contiguous) and the intra-chunk matrix A.
//   k_fwd_fused  non-materialized states: one workgroup per (batch*head, 64 values,
//                sequence segment) keeps its dk x 64 slice of the state in fp32
//                accumulators and walks the segment's chunks from the state at its start
//                (S0, or one formed beforehand by a state scan without stores):
//                O_i = Qh_i S + A_i V_i, then S <- diag(exp(gamma_i)) S + Kh_i^T V_i.  No
//                per-chunk state ever reaches memory.  The state accumulators feed the
//                Qh S product directly as the MFMA B operand (acc-order fragments).
//                Chunk 64: eight waves, wave w holding the 16 value columns w % 4 of the
//                state rows of dk half w / 4; O is the sum of the two halves' partial
//                products (added through LDS).  Each chunk's Qh, Kh^T, A and V^T tiles are
//                staged into LDS with cooperative 16-byte loads, the next chunk's tiles
//                are loaded into registers while the current one computes, and O leaves
//                through LDS as 16-byte row stores.  Chunk 128 and fp32 operands (tiles too large for
//                LDS) read the operand fragments straight from memory.
#include "gla_common.cuh"
#include "gla_internal.h"

namespace gla {

constexpr int kFusedThreads = 512;   // eight waves: two per SIMD on the one CU a tile gets

template <typename Tin, typename OpT, int C>
__global__ __launch_bounds__(kThreads) void k_output(const OpT* __restrict__ Qh,
                                                     const OpT* __restrict__ A,
                                                     const OpT* __restrict__ STt,
                                                     const Tin* __restrict__ V,
                                                     Tin* __restrict__ O, int T, int dk, int dv,
                                                     int N) {
  constexpr int TV = 64, VLD = C + 8, NM = C / 16, DB = 64;
  // Qh and the state tile move through LDS in 64-column blocks of the key dimension, as
  // 16-byte row pieces (the state tile of a workgroup is one contiguous block of memory,
  // streamed in order; Qh is read once per workgroup instead of once per wave); rows
  // padded so that the fragment reads of 16 consecutive rows fall on distinct banks
  constexpr int LD = sizeof(OpT) == 2 ? DB + 16 : DB + 4;
  __shared__ __attribute__((aligned(16))) OpT vs[TV * VLD];
  __shared__ __attribute__((aligned(16))) OpT qs[C * LD];
  __shared__ __attribute__((aligned(16))) OpT ss[TV * LD];
  // 1-D grid, XCD-aware: the dv tiles of one chunk share Qh and A
  const int nvt = dv / TV;
  const int lt = xcd_logical(blockIdx.x, gridDim.x);
  const int v0 = (lt % nvt) * TV, i = (lt / nvt) % N, bh = lt / (nvt * N);
  const int w = wave_id(), l = lane_id(), r = l & 15, qd = l >> 4;
  const int t0 = i * C, rows = min(C, T - t0);

  const OpT* qp = Qh + ((long)bh * N * C + t0) * dk;
  const OpT* sp = STt + (((long)bh * N + i) * dv + v0) * dk;
  RowTile<OpT, C, DB, LD> tq;
  RowTile<OpT, TV, DB, LD> ts;
  tq.load(qp, dk, C);
  ts.load(sp, dk, TV);
  stage_cols<OpT, Tin, C, TV>(vs, VLD, V + ((long)bh * T + t0) * dv + v0, dv, rows);

  f32x4 acc[NM];   // acc[m][e] = O[16m + 4qd + e][v0 + 16w + r]
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int d0 = 0; d0 < dk; d0 += DB) {
    __syncthreads();   // the previous block's fragment reads are done
    tq.store(qs);
    ts.store(ss);
    __syncthreads();
    // the next block (the last one refetches itself: no branch around a load)
    const int dn = min(d0 + DB, dk - DB);
    tq.load(qp + dn, dk, C);
    ts.load(sp + dn, dk, TV);
#pragma unroll
    for (int kb = 0; kb < DB / 32; ++kb) {
      Frag<OpT> fb;
      load_frag_c(fb, ss + (16 * w + r) * LD + kb * 32);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        Frag<OpT> fa;
        load_frag_c(fa, qs + (16 * m + r) * LD + kb * 32);
        mma(acc[m], fa, fb);
      }
    }
  }
  const OpT* ap = A + ((long)bh * N + i) * C * C;
#pragma unroll
  for (int kb = 0; kb < C / 32; ++kb) {
    Frag<OpT> fb;
    load_frag_c(fb, vs + (16 * w + r) * VLD + kb * 32);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (32 * kb <= 16 * m + 15) {
        Frag<OpT> fa;
        load_frag_c(fa, ap + (16 * m + r) * C + kb * 32);
        mma(acc[m], fa, fb);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * m + 4 * qd + e;
      if (t < rows) O[((long)bh * T + t0 + t) * dv + v0 + 16 * w + r] = from_f32<Tin>(acc[m][e]);
    }
}

// A chunk's Kh^T as bf16 MFMA fragments (1 KB each), copied to LDS as they are.  kst = 1:
// the forward's layout, fragments back to back; kst = 2: the backward's, each fragment
// followed by its bf16 remainder, which is skipped (the forward's operand is the rounded
// value, the fragment itself).
template <int UNITS, int NT>
struct KhtTile {
  static constexpr int kPerThread = (UNITS + NT - 1) / NT;
  u32x4 u[kPerThread];
  __device__ __forceinline__ void load(const bf16* __restrict__ g, int kst) {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int idx = threadIdx.x + j * NT;
      if (UNITS % NT == 0 || idx < UNITS)
        u[j] = *reinterpret_cast<const u32x4*>(g + ((long)idx + (long)(kst - 1) * (idx & ~63)) * 8);
    }
  }
  __device__ __forceinline__ void store(bf16* lds) const {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int idx = threadIdx.x + j * NT;
      if (UNITS % NT == 0 || idx < UNITS) *reinterpret_cast<u32x4*>(lds + idx * 8) = u[j];
    }
  }
};

template <typename Tin, typename OpT, int C, int DK>
__global__ __launch_bounds__(kFusedThreads) void k_fwd_fused_staged(
    const OpT* __restrict__ Qh, const OpT* __restrict__ KhT, const OpT* __restrict__ A,
    const float* __restrict__ eg, const Tin* __restrict__ V, const float* __restrict__ S0,
    Tin* __restrict__ O, float* __restrict__ S_T, int T, int dv, int N, int nseg,
    const float* __restrict__ S_mid, int kst) {
  static_assert(sizeof(OpT) == 2, "bf16 operands");
  constexpr int NT = kFusedThreads, TV = 64, NM = C / 16, KH = DK / 2, NP = KH / 16;
  // Kh^T arrives in MFMA fragment order (lane 16 q + r of fragment (16-row block, 32-token
  // block) holds row r, tokens 8 q ..) and is copied to LDS as is: each fragment read is 1 KB
  // of consecutive lanes.  A rows padded to 80 elements: 16-byte fragment reads of 16
  // consecutive rows then fall on distinct banks (a stride of 72 pairs rows up on gfx950's
  // 64 banks); the Qh rows are read as 8-byte halves, conflict-free at DK + 8.
  constexpr int QLD = DK + 8, KLD = C, ALD = C + 16, VLD = C + 8, OLD = TV + 8, RLD = TV + 4;
  __shared__ __attribute__((aligned(16))) OpT qs[C * QLD];
  __shared__ __attribute__((aligned(16))) OpT ks[DK * KLD];
  __shared__ __attribute__((aligned(16))) OpT as_[C * ALD];
  __shared__ __attribute__((aligned(16))) OpT vs[TV * VLD];
  __shared__ __attribute__((aligned(16))) Tin os_[2][C * OLD];   // O tile, double-buffered
  __shared__ __attribute__((aligned(16))) float red[C * RLD];     // partial O of the upper dk half
  __shared__ float egs[DK];
  // 1-D grid, XCD-aware: the dv tiles of one bh share every Qh / Kh^T / A tile.  With a
  // sequence split into nseg segments, the s-th part of the logical ids walks chunks
  // [s N / nseg, (s + 1) N / nseg) from the state at its first chunk (S0, or slot s - 1 of
  // S_mid).
  const int nvt = dv / TV, per_seg = (int)gridDim.x / nseg;
  const int lg = xcd_logical(blockIdx.x, gridDim.x);
  const int seg = lg / per_seg, lt = lg % per_seg;
  const int v0 = (lt % nvt) * TV, bh = lt / nvt;
  const int ib = seg * N / nseg, ie = (seg + 1) * N / nseg;
  const float* __restrict__ Sinit =
      seg == 0 ? S0 : S_mid + (long)(seg - 1) * (per_seg / nvt) * DK * dv;
  // wave w: value columns 16 (w % 4) .. +15, state rows kh*KH .. kh*KH + KH-1 (kh = w / 4)
  const int w = threadIdx.x >> 6, vc = w & 3, kh = w >> 2;
  const int l = lane_id(), r = l & 15, qd = l >> 4;
  const int c16 = 16 * vc + r, col = v0 + c16, k0 = kh * KH;

  f32x4 S[NP];   // S[p][e] = state[k0 + 16p + 4qd + e][col]
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S[p][e] = Sinit ? Sinit[((long)bh * DK + k0 + 16 * p + 4 * qd + e) * dv + col] : 0.f;

  FlatTile<OpT, C, DK, QLD, NT> tq;
  static_assert(KLD == C, "the Kh^T tile is copied as is");
  KhtTile<DK * C / 8, NT> tk;
  FlatTile<OpT, C, C, ALD, NT> ta;
  ColTile<OpT, Tin, C, VLD, NT, true> tv;   // chunk-swizzled (conflict-free stores)
  float egr = 0.f;
  auto fetch = [&](int i) {
    const int t0 = i * C;
    tq.load(Qh + ((long)bh * N * C + t0) * DK);
    tk.load(KhT + ((long)bh * N + i) * DK * C * kst, kst);
    ta.load(A + ((long)bh * N + i) * C * C);
    tv.load(V + ((long)bh * T + t0) * dv + v0, dv, min(C, T - t0));
    if (threadIdx.x < DK) egr = eg[((long)bh * N + i) * DK + threadIdx.x];
  };
  if (ie > ib) fetch(ib);

  // O tile of the previous chunk leaves right after the first barrier of the next chunk,
  // before that chunk's prefetch (vector memory operations complete in order).
  constexpr int kPer = 16 / (int)sizeof(Tin), kUnits = C * TV / kPer;
  auto store_o = [&](int ip) {
    const int tp = ip * C, rp = min(C, T - tp);
    const Tin* ob = os_[ip & 1];
#pragma unroll
    for (int u_ = 0; u_ < (kUnits + NT - 1) / NT; ++u_) {   // fixed trip count
      const int idx = threadIdx.x + u_ * NT;
      if ((kUnits) % NT != 0 && idx >= kUnits) continue;
      const int e0 = idx * kPer, rr = e0 / TV, cc = e0 % TV;
      if (rr < rp)
        *reinterpret_cast<u32x4*>(O + ((long)bh * T + tp + rr) * dv + v0 + cc) =
            *reinterpret_cast<const u32x4*>(ob + rr * OLD + cc);
    }
  };
  for (int i = ib; i < ie; ++i) {
    tq.store(qs);
    tk.store(ks);
    ta.store(as_);
    tv.store(vs);
    if (threadIdx.x < DK) egs[threadIdx.x] = egr;
    __syncthreads();
    if (i > ib) store_o(i - 1);
    if (i + 1 < ie) fetch(i + 1);

    // O_i = Qh_i S + A_i V_i as two partial sums, one per dk half; the A V rows are split
    // between the halves
    f32x4 acc[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KH / 32; ++kb) {
      Frag<OpT> fb;
      frag_from_acc(fb, S[2 * kb], S[2 * kb + 1]);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        Frag<OpT> fa;
        load_frag_a(fa, qs + (16 * m + r) * QLD + k0 + kb * 32);
        mma(acc[m], fa, fb);
      }
    }
#pragma unroll
    for (int kb = 0; kb < C / 32; ++kb) {
      Frag<OpT> fb;
      load_frag_cs(fb, vs, VLD, c16, kb);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if ((m < NM / 2) == (kh == 0) && 32 * kb <= 16 * m + 15) {
          Frag<OpT> fa;
          load_frag_c(fa, as_ + (16 * m + r) * ALD + kb * 32);
          mma(acc[m], fa, fb);
        }
      }
    }
    if (kh == 1) {
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[(16 * m + 4 * qd + e) * RLD + c16] = acc[m][e];
    }
    __syncthreads();
    if (kh == 0) {
      Tin* ob = os_[i & 1];
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * m + 4 * qd + e;
          ob[t * OLD + c16] = from_f32<Tin>(acc[m][e] + red[t * RLD + c16]);
        }
    }

    // S <- diag(exp(gamma_i)) S + Kh_i^T V_i, this wave's dk half
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const f32x4 dec = *reinterpret_cast<const f32x4*>(egs + k0 + 16 * p + 4 * qd);
#pragma unroll
      for (int e = 0; e < 4; ++e) S[p][e] *= dec[e];
    }
#pragma unroll
    for (int kb = 0; kb < C / 32; ++kb) {
      Frag<OpT> fb;
      load_frag_cs(fb, vs, VLD, c16, kb);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        Frag<OpT> fa;
        fa.v = *reinterpret_cast<const bf16x8*>(ks + (((k0 / 16 + p) * (C / 32) + kb) * 64 + l) * 8);
        mma(S[p], fa, fb);
      }
    }
    __syncthreads();
  }
  if (ie > ib) store_o(ie - 1);
  if (S_T && seg == nseg - 1) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int e = 0; e < 4; ++e) S_T[((long)bh * DK + k0 + 16 * p + 4 * qd + e) * dv + col] = S[p][e];
  }
}


// Chunk 128, bf16: the same walk in half-chunk steps of 64 rows, so that every staged tile
// stays the size of the chunk-64 kernel's (a whole chunk-128 tile set would need ~260 KB
// of LDS).  Within chunk i the state stays S_[i] for both halves:
//     O_0 = Qh_0 S + A_00 V_0,    O_1 = Qh_1 S + A_10 V_0 + A_11 V_1
// (Qh rows and A taken against the chunk-128 cumulative gate), and the update
//     S <- diag(exp(gamma_i)) S + Kh_0^T V_0 + Kh_1^T V_1
// is formed in two parts: the first half's product goes to a side accumulator while the
// first half runs, and joins the decayed state in the second.  The first half's V^T tile
// stays in LDS for the second half's A_10 V_0.  Eight waves as in the chunk-64 kernel.
template <typename Tin, int DK>
__global__ __launch_bounds__(kFusedThreads) void k_fwd_fused_c128(
    const bf16* __restrict__ Qh, const bf16* __restrict__ KhT, const bf16* __restrict__ A,
    const float* __restrict__ eg, const Tin* __restrict__ V, const float* __restrict__ S0,
    Tin* __restrict__ O, float* __restrict__ S_T, int T, int dv, int N, int nseg,
    const float* __restrict__ S_mid, int kst) {
  using OpT = bf16;
  constexpr int C = 128, H = 64;   // chunk, half-step rows
  constexpr int NT = kFusedThreads, TV = 64, NM = H / 16, KH = DK / 2, NP = KH / 16;
  constexpr int QLD = DK + 8, KLD = H, ALD = C + 16, VLD = H + 8, OLD = TV + 8, RLD = TV + 4;
  __shared__ __attribute__((aligned(16))) OpT qs[H * QLD];
  __shared__ __attribute__((aligned(16))) OpT ks[DK * KLD];       // Kh^T of the half, fragment order
  __shared__ __attribute__((aligned(16))) OpT as_[H * ALD];       // A rows of the half, all columns
  __shared__ __attribute__((aligned(16))) OpT vs[2][TV * VLD];    // V^T of both halves
  __shared__ __attribute__((aligned(16))) Tin os_[2][H * OLD];    // O of a half, double-buffered
  __shared__ __attribute__((aligned(16))) float red[H * RLD];
  __shared__ float egs[DK];
  const int nvt = dv / TV, per_seg = (int)gridDim.x / nseg;
  const int lg = xcd_logical(blockIdx.x, gridDim.x);
  const int seg = lg / per_seg, lt = lg % per_seg;
  const int v0 = (lt % nvt) * TV, bh = lt / nvt;
  const int ib = seg * N / nseg, ie = (seg + 1) * N / nseg;
  const float* __restrict__ Sinit =
      seg == 0 ? S0 : S_mid + (long)(seg - 1) * (per_seg / nvt) * DK * dv;
  const int w = threadIdx.x >> 6, vc = w & 3, kh = w >> 2;
  const int l = lane_id(), r = l & 15, qd = l >> 4;
  const int c16 = 16 * vc + r, col = v0 + c16, k0 = kh * KH;

  f32x4 S[NP], Dl[NP];   // state rows k0 + 16 p + 4 qd + e of column col; Dl: Kh_0^T V_0
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S[p][e] = Sinit ? Sinit[((long)bh * DK + k0 + 16 * p + 4 * qd + e) * dv + col] : 0.f;

  FlatTile<OpT, H, DK, QLD, NT> tq;
  FlatTile<OpT, H, C, ALD, NT> ta;
  ColTile<OpT, Tin, H, VLD, NT, true> tv;
  // Kh^T of one half: for each 16-row block, its two 32-token fragments of that half
  // (2 KB of every 4 KB), copied to LDS as fragments (p, kb local)
  constexpr int kKUnits = DK * H / 8, kKPer = (kKUnits + NT - 1) / NT;
  u32x4 ku[kKPer];
  float egr = 0.f;
  auto fetch = [&](int i, int h) {
    // the second half of a ragged last chunk may lie past T: its V rows are all zero
    const int t0 = i * C + h * H, rows = min(H, T - t0);
    tq.load(Qh + ((long)bh * N * C + t0) * DK);
    ta.load(A + (((long)bh * N + i) * C + h * H) * C);
    tv.load(V + ((long)bh * T + min(t0, T - 1)) * dv + v0, dv, max(rows, 1));
    tv.nrows = max(rows, 0);
    // (kst = 2: the backward's layout, each fragment followed by its remainder, skipped)
    const bf16* kb0 = KhT + ((long)bh * N + i) * DK * C * kst;
#pragma unroll
    for (int j = 0; j < kKPer; ++j) {
      const int u = threadIdx.x + j * NT;   // unit: (row block p, local fragment f, lane piece)
      const int pb = u / 128, f = (u / 64) % 2, pc = u % 64;
      if (kKUnits % NT == 0 || u < kKUnits)
        ku[j] = *reinterpret_cast<const u32x4*>(kb0 + ((pb * 4 + 2 * h + f) * kst * 64 + pc) * 8);
    }
    egr = eg[((long)bh * N + i) * DK + min((int)threadIdx.x, DK - 1)];
  };
  auto store_k = [&]() {
#pragma unroll
    for (int j = 0; j < kKPer; ++j) {
      const int u = threadIdx.x + j * NT;
      if (kKUnits % NT == 0 || u < kKUnits) *reinterpret_cast<u32x4*>(ks + u * 8) = ku[j];
    }
  };
  if (ie > ib) fetch(ib, 0);

  constexpr int kPer = 16 / (int)sizeof(Tin), kUnits = H * TV / kPer;
  auto store_o = [&](int ip, int hp, int buf) {
    const int tp = ip * C + hp * H, rp = min(H, T - tp);
    const Tin* ob = os_[buf];
#pragma unroll
    for (int u_ = 0; u_ < (kUnits + NT - 1) / NT; ++u_) {   // fixed trip count
      const int idx = threadIdx.x + u_ * NT;
      if ((kUnits) % NT != 0 && idx >= kUnits) continue;
      const int e0 = idx * kPer, rr = e0 / TV, cc = e0 % TV;
      if (rr < rp)
        *reinterpret_cast<u32x4*>(O + ((long)bh * T + tp + rr) * dv + v0 + cc) =
            *reinterpret_cast<const u32x4*>(ob + rr * OLD + cc);
    }
  };
  int step = 0;
  for (int i = ib; i < ie; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h, ++step) {
      tq.store(qs);
      store_k();
      ta.store(as_);
      tv.store(vs[h]);
      if (h == 1 && threadIdx.x < DK) egs[threadIdx.x] = egr;
      __syncthreads();
      if (step > 0) store_o(h == 0 ? i - 1 : i, h ^ 1, (step - 1) & 1);
      // next half-step (unconditional: past the end the last one is refetched, unused)
      const int ni = h == 0 ? i : min(i + 1, ie - 1), nh = h == 0 ? 1 : (i + 1 < ie ? 0 : 1);
      fetch(ni, nh);

      // O_h = Qh_h S + (A V) of the half, as two partial sums (dk halves)
      f32x4 acc[NM];
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KH / 32; ++kb) {
        Frag<OpT> fb;
        frag_from_acc(fb, S[2 * kb], S[2 * kb + 1]);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          Frag<OpT> fa;
          load_frag_a(fa, qs + (16 * m + r) * QLD + k0 + kb * 32);
          mma(acc[m], fa, fb);
        }
      }
      // A columns of the first half (all of them for the second half's rows, causal for
      // the first half's), then for the second half its own causal block
#pragma unroll
      for (int kb = 0; kb < H / 32; ++kb) {
        Frag<OpT> fb;
        load_frag_cs(fb, vs[0], VLD, c16, kb);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          if ((m < NM / 2) == (kh == 0) && (h == 1 || 32 * kb <= 16 * m + 15)) {
            Frag<OpT> fa;
            load_frag_c(fa, as_ + (16 * m + r) * ALD + kb * 32);
            mma(acc[m], fa, fb);
          }
        }
      }
      if (h == 1) {
#pragma unroll
        for (int kb = 0; kb < H / 32; ++kb) {
          Frag<OpT> fb;
          load_frag_cs(fb, vs[1], VLD, c16, kb);
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            if ((m < NM / 2) == (kh == 0) && 32 * kb <= 16 * m + 15) {
              Frag<OpT> fa;
              load_frag_c(fa, as_ + (16 * m + r) * ALD + H + kb * 32);
              mma(acc[m], fa, fb);
            }
          }
        }
      }
      if (kh == 1) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int e = 0; e < 4; ++e) red[(16 * m + 4 * qd + e) * RLD + c16] = acc[m][e];
      }
      __syncthreads();
      if (kh == 0) {
        Tin* ob = os_[step & 1];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 16 * m + 4 * qd + e;
            ob[t * OLD + c16] = from_f32<Tin>(acc[m][e] + red[t * RLD + c16]);
          }
      }

      // state: Kh_0^T V_0 aside in the first half; decay, add it, and Kh_1^T V_1 in the second
      if (h == 0) {
#pragma unroll
        for (int p = 0; p < NP; ++p) Dl[p] = f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const f32x4 dec = *reinterpret_cast<const f32x4*>(egs + k0 + 16 * p + 4 * qd);
#pragma unroll
          for (int e = 0; e < 4; ++e) S[p][e] = S[p][e] * dec[e] + Dl[p][e];
        }
      }
#pragma unroll
      for (int kb = 0; kb < H / 32; ++kb) {
        Frag<OpT> fb;
        load_frag_cs(fb, vs[h], VLD, c16, kb);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          Frag<OpT> fa;
          fa.v = *reinterpret_cast<const bf16x8*>(ks + (((k0 / 16 + p) * 2 + kb) * 64 + l) * 8);
          if (h == 0) mma(Dl[p], fa, fb);
          else mma(S[p], fa, fb);
        }
      }
      __syncthreads();
    }
  }
  if (ie > ib) store_o(ie - 1, 1, (step - 1) & 1);
  if (S_T && seg == nseg - 1) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int e = 0; e < 4; ++e) S_T[((long)bh * DK + k0 + 16 * p + 4 * qd + e) * dv + col] = S[p][e];
  }
}

template <typename Tin, typename OpT, int C, int DK>
__global__ __launch_bounds__(kThreads) void k_fwd_fused(
    const OpT* __restrict__ Qh, const OpT* __restrict__ KhT, const OpT* __restrict__ A,
    const float* __restrict__ eg, const Tin* __restrict__ V, const float* __restrict__ S0,
    Tin* __restrict__ O, float* __restrict__ S_T, int T, int dv, int N) {
  constexpr int TV = 64, VLD = C + 8, NM = C / 16, NP = DK / 16;
  __shared__ __attribute__((aligned(16))) OpT vs[TV * VLD];
  const int nvt = dv / TV;
  const int lt = xcd_logical(blockIdx.x, gridDim.x);
  const int v0 = (lt % nvt) * TV, bh = lt / nvt;
  const int w = wave_id(), l = lane_id(), r = l & 15, qd = l >> 4;
  const int col = v0 + 16 * w + r;

  f32x4 S[NP];   // S[p][e] = state[16p + 4qd + e][col]
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S[p][e] = S0 ? S0[((long)bh * DK + 16 * p + 4 * qd + e) * dv + col] : 0.f;

  for (int i = 0; i < N; ++i) {
    const int t0 = i * C, rows = min(C, T - t0);
    stage_cols<OpT, Tin, C, TV>(vs, VLD, V + ((long)bh * T + t0) * dv + v0, dv, rows);
    __syncthreads();

    // O_i = Qh_i S + A_i V_i
    f32x4 acc[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    const OpT* qp = Qh + ((long)bh * N * C + t0) * DK;
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
      Frag<OpT> fb;
      frag_from_acc(fb, S[2 * kb], S[2 * kb + 1]);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        Frag<OpT> fa;
        load_frag_a(fa, qp + (16 * m + r) * DK + kb * 32);
        mma(acc[m], fa, fb);
      }
    }
    const OpT* ap = A + ((long)bh * N + i) * C * C;
#pragma unroll
    for (int kb = 0; kb < C / 32; ++kb) {
      Frag<OpT> fb;
      load_frag_c(fb, vs + (16 * w + r) * VLD + kb * 32);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if (32 * kb <= 16 * m + 15) {
          Frag<OpT> fa;
          load_frag_c(fa, ap + (16 * m + r) * C + kb * 32);
          mma(acc[m], fa, fb);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * m + 4 * qd + e;
        if (t < rows) O[((long)bh * T + t0 + t) * dv + col] = from_f32<Tin>(acc[m][e]);
      }

    // S <- diag(exp(gamma_i)) S + Kh_i^T V_i
    const float* egp = eg + ((long)bh * N + i) * DK + 4 * qd;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const f32x4 dec = *reinterpret_cast<const f32x4*>(egp + 16 * p);
#pragma unroll
      for (int e = 0; e < 4; ++e) S[p][e] *= dec[e];
    }
    const OpT* kp = KhT + ((long)bh * N + i) * DK * C;
#pragma unroll
    for (int kb = 0; kb < C / 32; ++kb) {
      Frag<OpT> fb;
      load_frag_c(fb, vs + (16 * w + r) * VLD + kb * 32);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        Frag<OpT> fa;
        if constexpr (sizeof(OpT) == 2)   // bf16 Kh^T in fragment order
          fa.v = *reinterpret_cast<const bf16x8*>(kp + ((p * (C / 32) + kb) * 64 + l) * 8);
        else
          load_frag_c(fa, kp + (16 * p + r) * C + kb * 32);
        mma(S[p], fa, fb);
      }
    }
    __syncthreads();
  }
  if (S_T) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int e = 0; e < 4; ++e) S_T[((long)bh * DK + 16 * p + 4 * qd + e) * dv + col] = S[p][e];
  }
}

// ---------------------------------------------------------------------------------
template <typename Tin, typename OpT, int C>
static hipError_t launch_output_t(const OutArgs& a, hipStream_t s) {
  dim3 grid((a.dv / 64) * a.N * a.BH);
  hipLaunchKernelGGL((k_output<Tin, OpT, C>), grid, dim3(kThreads), 0, s, (const OpT*)a.Qh,
                     (const OpT*)a.A, (const OpT*)a.STt, (const Tin*)a.v, (Tin*)a.o, a.T, a.dk,
                     a.dv, a.N);
  return hipGetLastError();
}

hipError_t launch_output(const OutArgs& a, hipStream_t s) {
  if (a.BH == 0 || a.N == 0) return hipSuccess;
  if (a.dtype == 0)   // fp32 operands come with chunk 64 only
    return a.C == 64 ? launch_output_t<float, float, 64>(a, s) : hipErrorInvalidValue;
  if (a.C == 64) return launch_output_t<bf16, bf16, 64>(a, s);
  return launch_output_t<bf16, bf16, 128>(a, s);
}

int fused_segments(int dtype, int C, int N, int BH, int dv) {
  if (dtype == 0 || N < 4) return 1;
  const long tiles = (long)BH * (dv / 64);   // workgroups per segment
  int P = tiles >= 128 ? 2 : (int)(256 / tiles);
  P = P > 8 ? 8 : P;
  P = P > N / 2 ? N / 2 : P;
  return P < 2 ? 2 : P;
}

template <typename Tin, typename OpT, int C, int DK>
static hipError_t launch_fused_t2(const FusedArgs& a, hipStream_t s) {
  if constexpr (C == 128 && sizeof(OpT) == 2) {
    const int nseg = a.S_mid && a.nseg > 1 ? a.nseg : 1;
    dim3 grid((a.dv / 64) * a.BH * nseg);
    hipLaunchKernelGGL((k_fwd_fused_c128<Tin, DK>), grid, dim3(kFusedThreads), 0, s,
                       (const bf16*)a.Qh, (const bf16*)a.KhT, (const bf16*)a.A, a.eg,
                       (const Tin*)a.v, a.S0, (Tin*)a.o, a.S_T, a.T, a.dv, a.N, nseg, a.S_mid,
                       a.kht_split ? 2 : 1);
  } else if constexpr (C == 64 && sizeof(OpT) == 2) {
    const int nseg = a.S_mid && a.nseg > 1 ? a.nseg : 1;
    dim3 grid((a.dv / 64) * a.BH * nseg);
    hipLaunchKernelGGL((k_fwd_fused_staged<Tin, OpT, C, DK>), grid, dim3(kFusedThreads), 0, s,
                       (const OpT*)a.Qh, (const OpT*)a.KhT, (const OpT*)a.A, a.eg,
                       (const Tin*)a.v, a.S0, (Tin*)a.o, a.S_T, a.T, a.dv, a.N, nseg, a.S_mid,
                       a.kht_split ? 2 : 1);
  } else {   // fp32, chunk 64: operand fragments read straight from memory
    // (fp32 Kh^T has the same [dk][C] rows in the forward and the backward: no split)
    static_assert(C == 64, "fp32 operands come with chunk 64 only");
    dim3 grid((a.dv / 64) * a.BH);
    hipLaunchKernelGGL((k_fwd_fused<Tin, OpT, C, DK>), grid, dim3(kThreads), 0, s,
                       (const OpT*)a.Qh, (const OpT*)a.KhT, (const OpT*)a.A, a.eg,
                       (const Tin*)a.v, a.S0, (Tin*)a.o, a.S_T, a.T, a.dv, a.N);
  }
  return hipGetLastError();
}
template <typename Tin, typename OpT, int C>
static hipError_t launch_fused_t(const FusedArgs& a, hipStream_t s) {
  switch (a.dk) {
    case 64: return launch_fused_t2<Tin, OpT, C, 64>(a, s);
    case 128: return launch_fused_t2<Tin, OpT, C, 128>(a, s);
    case 192: return launch_fused_t2<Tin, OpT, C, 192>(a, s);
    default: return launch_fused_t2<Tin, OpT, C, 256>(a, s);
  }
}

hipError_t launch_fwd_fused(const FusedArgs& a, hipStream_t s) {
  if (a.BH == 0 || a.N == 0) return hipSuccess;
  if (a.dtype == 0)
    return a.C == 64 ? launch_fused_t<float, float, 64>(a, s) : hipErrorInvalidValue;
  if (a.C == 64) return launch_fused_t<bf16, bf16, 64>(a, s);
  return launch_fused_t<bf16, bf16, 128>(a, s);
}

}  // namespace gla
