// Inter-chunk state scan of the chunkwise GLA path with materialized states (page "Gated
// Linear Attention Transformers with Hardware-Efficient Training", atlas.scime.ai
// summary, section Approach: materialized inter-chunk states).
//
// One workgroup owns a 64 x 64 fp32 tile (dk rows x dv columns) of one (batch, head)
// state and walks the chunks in order (forward) or in reverse (the state gradient):
//     forward:  S_[i+1]  = diag(exp(gamma_i)) S_[i]    + Kh_i^T V_i,   Kh = k*exp(gamma-g)
//     reverse:  dS_[i]   = diag(exp(gamma_i)) dS_[i+1] + Qh_i^T dO_i,  Qh = q*exp(g)
// Before each chunk the tile is written out (the chunk-start state S_[i], or dS_[i+1]).
// The product is a k32 MFMA over the chunk's tokens: the transposed decayed operand
// comes ready-made from the intra-chunk kernel, the value-side tile is staged into LDS
// transposed so both operands are token-contiguous.  The tile stays in fp32 accumulators
// across the whole sequence.  In the backward the transposed operand arrives as a bf16
// high part plus bf16 remainder (two MFMAs), so the state carries no operand rounding;
// the kernel is bound by the state writes, not by the matrix units.
//
// Chunk totals of the closed-form gate gradient (optional cross term): summed over one
// chunk, the intra-chunk parts of q*dq - k*dk cancel pairwise, so the chunk total is
//     sum_t (q*dq_inter - k*dk_inter) = rowsum(S_[i] * (Qh_i^T dO_i))
//                                     - rowsum(dS_[i+1] * (Kh_i^T V_i)).
// The forward scan forms the first term and the reverse scan the second, each from the
// fp32 state it holds, for its 64 columns; the gate-gradient kernel adds the tiles.
#include <type_traits>

#include "gla_common.cuh"
#include "gla_internal.h"

namespace gla {

// Transposed decayed operand in LDS: rows of C tokens in the operand type, or (SPLIT) a
// bf16 high part in [0, C) and its bf16 remainder in [C, 2C) of each row.
template <typename OpT, bool SPLIT>
struct XFrag {
  Frag<OpT> hi, lo;
  __device__ __forceinline__ void load(const OpT* row, int kb, int C) {
    load_frag_c(hi, row + kb * 32);
    if constexpr (SPLIT) load_frag_c(lo, row + C + kb * 32);
  }
  __device__ __forceinline__ void apply(f32x4& acc, const Frag<OpT>& b) const {
    mma(acc, hi, b);
    if constexpr (SPLIT) mma(acc, lo, b);
  }
};

template <typename Tin, typename OpT, bool SPLIT, int C, int STORE, bool CROSS>
__global__ __launch_bounds__(kThreads) void k_state_scan(
    const OpT* __restrict__ XT, const Tin* __restrict__ Y, const OpT* __restrict__ X2T,
    const Tin* __restrict__ Y2, float* __restrict__ cross, const float* __restrict__ eg,
    const float* __restrict__ S_in, void* __restrict__ states, float* __restrict__ S_out,
    int T, int dk, int dv, int N, int reverse) {
  constexpr int TV = 64, TK = 64, YLD = C + 8, XW = SPLIT ? 2 * C : C, XLD = XW + 8;
  constexpr int SLD = 64 + 8;   // state tile staging for 16-byte row stores
  using StT = typename std::conditional<STORE == 3, float, OpT>::type;
  __shared__ __attribute__((aligned(16))) OpT ys[TV * YLD];
  __shared__ __attribute__((aligned(16))) OpT y2s[CROSS ? TV * YLD : 8];
  __shared__ __attribute__((aligned(16))) OpT xs[TK * XLD];
  __shared__ __attribute__((aligned(16))) OpT x2s[CROSS ? TK * XLD : 8];
  __shared__ __attribute__((aligned(16))) StT ss[STORE != 0 ? 64 * SLD : 8];
  __shared__ float egs[TK];
  // 1-D grid, XCD-aware: the dv tiles of one (bh, dk tile) share the Kh^T / Qh^T tiles
  // and the dk tiles of one bh share the value-side tiles, so they run on one XCD.
  const int nvt = dv / TV, nkt = dk / TK;
  const int lt = xcd_logical(blockIdx.x, gridDim.x);
  const int vt = lt % nvt, kt = (lt / nvt) % nkt, bh = lt / (nvt * nkt);
  const int v0 = vt * TV, k0 = kt * TK;
  const int w = wave_id(), l = lane_id(), r = l & 15, qd = l >> 4;
  const int rl = 16 * w + 4 * qd;          // tile-local accumulator rows rl .. rl+3
  const int row0 = k0 + rl;

  f32x4 acc[4];   // acc[j][e] = S[row0 + e][v0 + 16 j + r]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc[j][e] = S_in ? S_in[((long)bh * dk + row0 + e) * dv + v0 + 16 * j + r] : 0.f;

  // next chunk's tiles, loaded into registers while the current chunk computes
  FlatTileRows<OpT, TK, XW, XLD> tx, tx2;
  ColTile<OpT, Tin, C, YLD> ty, ty2;
  float egr = 0.f;
  auto fetch = [&](int i) {
    const int t0 = i * C, rows = min(C, T - t0);
    const long xo = (((long)bh * N + i) * dk + k0) * XW;
    tx.load(XT + xo);
    ty.load(Y + ((long)bh * T + t0) * dv + v0, dv, rows);
    if constexpr (CROSS) {
      tx2.load(X2T + xo);
      ty2.load(Y2 + ((long)bh * T + t0) * dv + v0, dv, rows);
    }
    if (threadIdx.x < TK) egr = eg[((long)bh * N + i) * dk + k0 + threadIdx.x];
  };
  if (N > 0) fetch(reverse ? N - 1 : 0);

  // Stores are issued right after the step's first barrier and before the next chunk's
  // loads: vector memory operations complete in order, so a store issued after the
  // prefetch would make the next step wait for the write round trip.
  float part_prev[4] = {0.f, 0.f, 0.f, 0.f};   // cross term of the previous chunk
  int i_prev = -1;
  for (int step = 0; step < N; ++step) {
    const int i = reverse ? N - 1 - step : step;
    tx.store(xs);
    ty.store(ys);
    if constexpr (CROSS) {
      tx2.store(x2s);
      ty2.store(y2s);
    }
    if (threadIdx.x < TK) egs[threadIdx.x] = egr;
    if constexpr (STORE != 0) {
      // the state before this chunk, through LDS
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (STORE == 2)
            ss[(16 * j + r) * SLD + rl + e] = (StT)acc[j][e];    // [v][k]
          else
            ss[(rl + e) * SLD + 16 * j + r] = (StT)acc[j][e];    // [k][v]
        }
    }
    __syncthreads();
    if constexpr (STORE != 0) {
      constexpr int kPer = 16 / (int)sizeof(StT), kUnits = 64 * 64 / kPer;
      const long sb = ((long)bh * N + i) * dk * dv;
      for (int idx = threadIdx.x; idx < kUnits; idx += kThreads) {
        const int e0 = idx * kPer, a = e0 / 64, b = e0 % 64;
        long off;
        if constexpr (STORE == 2) off = sb + (long)(v0 + a) * dk + k0 + b;
        else off = sb + (long)(k0 + a) * dv + v0 + b;
        *reinterpret_cast<u32x4*>((StT*)states + off) =
            *reinterpret_cast<const u32x4*>(ss + a * SLD + b);
      }
    }
    if constexpr (CROSS) {
      if (i_prev >= 0 && r == 0) {
        f32x4 o = {part_prev[0], part_prev[1], part_prev[2], part_prev[3]};
        *reinterpret_cast<f32x4*>(cross + (((long)bh * N + i_prev) * nvt + vt) * dk + row0) = o;
      }
    }
    if (step + 1 < N) fetch(reverse ? i - 1 : i + 1);

    if constexpr (CROSS) {
      f32x4 P[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) P[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < C / 32; ++kb) {
        XFrag<OpT, SPLIT> fa;
        fa.load(x2s + (16 * w + r) * XLD, kb, C);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          Frag<OpT> fb;
          load_frag_c(fb, y2s + (16 * j + r) * YLD + kb * 32);
          fa.apply(P[j], fb);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) sum += acc[j][e] * P[j][e];
        sum += __shfl_xor(sum, 1);
        sum += __shfl_xor(sum, 2);
        sum += __shfl_xor(sum, 4);
        sum += __shfl_xor(sum, 8);
        part_prev[e] = sum;
      }
      i_prev = i;
    }

#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float dec = egs[rl + e];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j][e] *= dec;
    }
#pragma unroll
    for (int kb = 0; kb < C / 32; ++kb) {
      XFrag<OpT, SPLIT> fa;
      fa.load(xs + (16 * w + r) * XLD, kb, C);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Frag<OpT> fb;
        load_frag_c(fb, ys + (16 * j + r) * YLD + kb * 32);
        fa.apply(acc[j], fb);
      }
    }
    __syncthreads();
  }
  if constexpr (CROSS) {
    if (i_prev >= 0 && r == 0) {
      f32x4 o = {part_prev[0], part_prev[1], part_prev[2], part_prev[3]};
      *reinterpret_cast<f32x4*>(cross + (((long)bh * N + i_prev) * nvt + vt) * dk + row0) = o;
    }
  }
  if (S_out) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S_out[((long)bh * dk + row0 + e) * dv + v0 + 16 * j + r] = acc[j][e];
  }
}

template <typename Tin, typename OpT, bool SPLIT, int C, int STORE, bool CROSS>
static void launch_scan_k(const ScanArgs& a, hipStream_t s) {
  dim3 grid((a.dv / 64) * (a.dk / 64) * a.BH);
  hipLaunchKernelGGL((k_state_scan<Tin, OpT, SPLIT, C, STORE, CROSS>), grid, dim3(kThreads), 0, s,
                     (const OpT*)a.XT, (const Tin*)a.Y, (const OpT*)a.X2T, (const Tin*)a.Y2,
                     a.cross, a.eg, a.S_in, a.states, a.S_out, a.T, a.dk, a.dv, a.N,
                     a.reverse ? 1 : 0);
}

template <typename Tin, typename OpT, bool SPLIT, int C>
static hipError_t launch_scan_t(const ScanArgs& a, hipStream_t s) {
  if (a.cross) {
    // the backward: operand-type states, [dk][dv]
    launch_scan_k<Tin, OpT, SPLIT, C, 1, true>(a, s);
  } else {
    switch (a.store) {
      case 0: launch_scan_k<Tin, OpT, SPLIT, C, 0, false>(a, s); break;
      case 1: launch_scan_k<Tin, OpT, SPLIT, C, 1, false>(a, s); break;
      case 2: launch_scan_k<Tin, OpT, SPLIT, C, 2, false>(a, s); break;
      default: launch_scan_k<Tin, OpT, SPLIT, C, 3, false>(a, s); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_state_scan(const ScanArgs& a, hipStream_t s) {
  if (a.BH == 0 || a.N == 0) return hipSuccess;
  if (a.cross && a.store != 1) return hipErrorInvalidValue;
  if (a.dtype == 0) return launch_scan_t<float, float, false, 64>(a, s);
  if (a.xt_f32) {
    if (a.C == 64) return launch_scan_t<bf16, bf16, true, 64>(a, s);
    return launch_scan_t<bf16, bf16, true, 128>(a, s);
  }
  if (a.C == 64) return launch_scan_t<bf16, bf16, false, 64>(a, s);
  return launch_scan_t<bf16, bf16, false, 128>(a, s);
}

}  // namespace gla
