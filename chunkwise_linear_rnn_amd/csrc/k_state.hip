// Inter-chunk state scan of the chunkwise GLA path with materialized states (page "Gated
// Linear Attention Transformers with Hardware-Efficient Training", atlas.scime.ai
// summary, section Approach: materialized inter-chunk states).
//
// One workgroup owns a 64 x TV fp32 tile (dk rows x dv columns, TV = 64, or 128 in the
// backward at chunk 64) of one (batch, head) state and walks the chunks in order
// (forward) or in reverse (the state gradient):
//     forward:  S_[i+1]  = diag(exp(gamma_i)) S_[i]    + Kh_i^T V_i,   Kh = k*exp(gamma-g)
//     reverse:  dS_[i]   = diag(exp(gamma_i)) dS_[i+1] + Qh_i^T dO_i,  Qh = q*exp(g)
// Before each chunk the tile is written out (the chunk-start state S_[i], or dS_[i+1]).
// The product is a k32 MFMA over the chunk's tokens: the transposed decayed operand
// comes ready-made from the intra-chunk kernel and each wave loads its own rows of it
// straight into MFMA fragments; the value-side tile, shared by the four waves, is staged
// into LDS transposed so both operands are token-contiguous.  The tile stays in fp32
// accumulators across the whole sequence; the per-row decays of 32 steps at a time wait
// in LDS.  In the backward the transposed operand arrives as a bf16 high part plus bf16
// remainder (two MFMAs), so the state carries no operand rounding.  The states leave
// through LDS as 16-byte streaming stores (they are read only by a later kernel); the
// kernel is bound by memory traffic and LDS staging, not by the matrix units.
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

// This wave's 16 rows of a per-chunk transposed operand, as MFMA A fragments held in
// registers.  fp32: rows of C tokens ([rows][C]), `at` = the lane's row.  bf16: fragment
// order, as the intra-chunk kernel writes it: for each 16-row block and 32-token block kb,
// the 64 lanes' 16-byte pieces (lane 16 q + r: row r, tokens 32 kb + 8 q ..), and with
// SPLIT the high-part fragment followed by the remainder's; `at` = the row block's first
// piece plus the lane's, so that every load reads 1 KB of whole cache lines.  Without
// SPLIT, `kst` = 2 reads the high parts of a split operand alone (every other fragment).
template <typename OpT, bool SPLIT, int C>
struct XRegs {
  static constexpr int KB = C / 32;
  Frag<OpT> hi[KB], lo[SPLIT ? KB : 1];
  __device__ __forceinline__ void load(const OpT* __restrict__ at, int kst) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if constexpr (SPLIT) {
        hi[kb].v = *reinterpret_cast<const bf16x8*>(at + (2 * kb) * 64 * 8);
        lo[kb].v = *reinterpret_cast<const bf16x8*>(at + (2 * kb + 1) * 64 * 8);
      } else if constexpr (sizeof(OpT) == 2) {
        hi[kb].v = *reinterpret_cast<const bf16x8*>(at + kb * kst * 64 * 8);
      } else {
        load_frag_c(hi[kb], at + kb * 32);
      }
    }
  }
  // acc += (the value-side fragment b as the A operand) x (these rows as the B operand):
  // the product lands with this wave's rows as output columns, i.e. each lane holds one
  // state row (its r) and four consecutive value columns (4 qd .. 4 qd + 3)
  __device__ __forceinline__ void apply_t(f32x4& acc, int kb, const Frag<OpT>& b) const {
    mma(acc, b, hi[kb]);
    if constexpr (SPLIT) mma(acc, b, lo[kb]);
  }
};

template <typename Tin, typename OpT, bool SPLIT, int C, int STORE, bool CROSS, int TV>
__global__ __launch_bounds__(kThreads, 256 / TV) void k_state_scan(ScanDir d0, ScanDir d1, int ndir,
                                                            const float* __restrict__ eg, int T,
                                                            int dk, int dv, int N, int nsteps,
                                                            int nseg, int segp, int kst) {
  // TV value columns per workgroup: NJ accumulator tiles per wave, NY 64-column
  // value-side tiles per operand
  constexpr int NJ = TV / 16, NY = TV / 64;
  static_assert(TV == 64 || (TV == 128 && STORE != 2), "[v][k] staging is 64 columns wide");
  // WT: bf16, chunk 64 and four 64-column value-side tiles per chunk (two operands of 128
  // columns): wave w stages tile w alone into unpadded swizzled tiles (conflict-free
  // 16-byte writes and fragment reads); otherwise all threads stage every tile
  constexpr bool WT = sizeof(OpT) == 2 && C == 64 && NY * (CROSS ? 2 : 1) == 4;
  constexpr int YLD = WT ? 64 : C + 8;
  using StT = typename std::conditional<STORE == 3, float, OpT>::type;
  // state tile staging for 16-byte row stores: [v][k] (STORE 2) or [k][v].  bf16 rows of
  // 128 columns take a stride of 132: the 8-byte writes of 16 consecutive rows, and the
  // 8-byte reads of two rows by 32 lanes, then fall on distinct banks.
  constexpr bool SPAD4 = STORE == 1 && sizeof(StT) == 2 && TV == 128;
  constexpr int SLD = STORE == 2 ? 64 + 8 : SPAD4 ? TV + 4 : TV + 8;
  constexpr int SROWS = STORE == 2 ? TV : 64;
  using XR = XRegs<OpT, SPLIT, C>;
  __shared__ __attribute__((aligned(16))) OpT ys[TV * YLD];
  __shared__ __attribute__((aligned(16))) OpT y2s[CROSS ? TV * YLD : 8];
  __shared__ __attribute__((aligned(16))) StT ss[STORE != 0 ? SROWS * SLD : 8];
  // per-row decays exp(gamma) of EB consecutive steps, [step][row]
  constexpr int EB = 32;
  __shared__ float egs[EB * 64];
  // 1-D grid, XCD-aware: the dv tiles of one (bh, dk tile) share the transposed operand
  // tiles and the dk tiles of one bh share the value-side tiles, so they run on one XCD.
  // With two scans in the launch, the first half of the logical ids runs the first.
  const int nvt = dv / TV, nkt = dk / 64, tiles = (int)gridDim.x / ndir;
  int lt = xcd_logical(blockIdx.x, gridDim.x);
  const bool second = lt >= tiles;
  if (second) lt -= tiles;
  // segp > 1: the sg-th of nseg segments in walk order of the sequence split into segp
  // parts (forward: chunks [sg N / segp, (sg + 1) N / segp); reverse: the
  // (segp - 1 - sg)-th part, walked downwards), from S_in for the first and, for the
  // others, from slot sg - 1 of seg_in (the states at the segment starts) or from zero;
  // without stores its end state goes to S_out + sg * BH * dk * dv
  const int base = tiles / nseg, sg = lt / base;
  lt -= sg * base;
  const bool segm = segp > 1;
  const int rev0 = second ? d1.reverse : d0.reverse;
  const int part = rev0 ? segp - 1 - sg : sg;
  const int i0 = segm ? part * N / segp : 0;
  const int nst = segm ? (part + 1) * N / segp - i0 : nsteps;
  const float* __restrict__ seg_in = second ? d1.seg_in : d0.seg_in;
  float* __restrict__ segdec = second ? d1.seg_dec : d0.seg_dec;
  const OpT* __restrict__ XT = (const OpT*)(second ? d1.XT : d0.XT);
  const Tin* __restrict__ Y = (const Tin*)(second ? d1.Y : d0.Y);
  const OpT* __restrict__ X2T = (const OpT*)(second ? d1.X2T : d0.X2T);
  const Tin* __restrict__ Y2 = (const Tin*)(second ? d1.Y2 : d0.Y2);
  float* __restrict__ cross = second ? d1.cross : d0.cross;
  const float* __restrict__ S_in =
      sg > 0 ? (seg_in ? seg_in + (long)(sg - 1) * (base / (nvt * nkt)) * dk * dv : nullptr)
             : second ? d1.S_in : d0.S_in;
  void* __restrict__ states = second ? d1.states : d0.states;
  float* __restrict__ S_out = second ? d1.S_out : d0.S_out;
  // segment end states (no stores) go to slot sg; in the storing pass only the last segment
  // forms the final state
  if (S_out && segm) {
    if (segp == nseg) S_out = sg == nseg - 1 ? S_out : nullptr;
    else S_out += (long)sg * (base / (nvt * nkt)) * dk * dv;
  }
  const int reverse = second ? d1.reverse : d0.reverse;
  const int frag_states = second ? d1.frag_states : d0.frag_states;
  const int vt = lt % nvt, kt = (lt / nvt) % nkt, bh = lt / (nvt * nkt);
  const int v0 = vt * TV, k0 = kt * 64;
  const int w = wave_id(), l = lane_id(), r = l & 15, qd = l >> 4;
  const int krow = k0 + 16 * w + r;        // this lane's state row

  f32x4 acc[NJ];   // acc[j][e] = S[krow][v0 + 16 j + 4 qd + e]
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    acc[j] = S_in ? *reinterpret_cast<const f32x4*>(S_in + ((long)bh * dk + krow) * dv + v0 + 16 * j + 4 * qd)
                  : f32x4{0.f, 0.f, 0.f, 0.f};
  // Settle the initial-state loads before the loop: otherwise the compiler, merging the
  // loop's entry with its back edge, treats the state registers as possibly still being
  // loaded and waits for nearly every prefetch in flight at each step.
  // chunk of a step; steps past the end map to the last one (refetched, never used), so
  // that every prefetch is unconditional and the compiler's wait counts stay exact
  auto chunk_of = [&](int step) {
    const int sc = min(step, nst - 1);
    return reverse ? (segm ? i0 + nst - 1 - sc : N - 1 - sc) : i0 + sc;
  };
  // the decays of steps [sb, sb + EB) into LDS: read there at each step, they put no
  // global-memory round trip on the chain of dependent steps
  auto stage_eg = [&](int sb) {
#pragma unroll
    for (int u_ = 0; u_ < EB * 64 / kThreads; ++u_) {
      const int idx = threadIdx.x + u_ * kThreads;
      egs[idx] = eg[((long)bh * N + chunk_of(sb + (idx >> 6))) * dk + k0 + (idx & 63)];
    }
  };
  if (nst > 0) stage_eg(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();

  // The operands of later chunks are loaded into registers while the current chunk
  // computes: the value-side tiles (then LDS, transposed) and this wave's rows of the
  // transposed operands (straight into MFMA fragments), each set reloaded as soon as the
  // current chunk has consumed it.  DEPTH sets of registers keep DEPTH chunks in flight
  // (one set where the register budget of four workgroups per CU leaves no room, and on
  // the WT path, where the registers freed let the compiler keep several fragment reads
  // in flight: measured faster than two chunks ahead).
  constexpr int DEPTH = WT ? 1 : (TV == 128 || (!CROSS && C == 64)) ? 2 : 1;
  // bf16 value-side tiles are staged chunk-swizzled (conflict-free transposing stores)
  constexpr bool SWZ = sizeof(OpT) == 2;
  using YT = ColTile<OpT, Tin, C, YLD, kThreads, SWZ>;
  struct SetAll {
    YT ty[NY], ty2[NY];
    XR cx, cx2;
  };
  struct SetWave {   // the value-side tile is held once (below), one chunk ahead
    XR cx, cx2;
  };
  using Set = typename std::conditional<WT, SetWave, SetAll>::type;
  Set sets[DEPTH];
  WaveColTile ywt;
  auto yfrag = [&](Frag<OpT>& fb, const OpT* tile, int c, int kb) {
    if constexpr (WT) load_frag_x64(fb, tile, c, kb);
    else if constexpr (SWZ) load_frag_cs(fb, tile, YLD, c, kb);
    else load_frag_c(fb, tile + c * YLD + kb * 32);
  };
  // WT: wave w stages 64 columns at 64 (w % 2) of the first (w < 2) or second operand
  const int wu = __builtin_amdgcn_readfirstlane(w), wh = wu & 1, wsec = wu >> 1;
  // where this lane's rows of a chunk's transposed operand start (see XRegs)
  auto xrow = [&](int i) {
    if constexpr (sizeof(OpT) == 2)
      return ((((long)bh * N + i) * (dk / 16) + (k0 / 16 + w)) * ((SPLIT ? 2 : kst) * (C / 32)) * 64 + l) * 8;
    else
      return (((long)bh * N + i) * dk + k0 + 16 * w + r) * (long)C;
  };
  auto fetch_y = [&](Set& st, int i) {
    const int t0 = i * C, rows = min(C, T - t0);
    if constexpr (WT) {
      ywt.load((wsec ? Y2 : Y) + ((long)bh * T + t0) * dv + v0 + 64 * wh, dv, rows);
    } else {
#pragma unroll
      for (int h = 0; h < NY; ++h) {
        st.ty[h].load(Y + ((long)bh * T + t0) * dv + v0 + 64 * h, dv, rows);
        if constexpr (CROSS) st.ty2[h].load(Y2 + ((long)bh * T + t0) * dv + v0 + 64 * h, dv, rows);
      }
    }
  };
  if (nst > 0) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int i0 = chunk_of(d);
      if (!WT || d == 0) fetch_y(sets[d], i0);
      sets[d].cx.load(XT + xrow(i0), kst);
      if constexpr (CROSS) sets[d].cx2.load(X2T + xrow(i0), kst);
    }
  }

  // Stores are issued right after the step's first barrier and before the next chunk's
  // loads: vector memory operations complete in order, so a store issued after the
  // prefetch would make the next step wait for the write round trip.
  float part_prev = 0.f;   // cross term of the previous chunk for row krow
  int i_prev = -1;
  float dprod = 1.f;   // product of the walked chunks' decays of row krow (segmented scan)
  auto body = [&](int step, Set& st) {
    const int i = chunk_of(step), ipre = chunk_of(step + DEPTH);
    const float egr = egs[(step % EB) * 64 + 16 * w + r];   // exp(gamma) of row krow
    dprod *= egr;
    if constexpr (WT) {
      ywt.store((wsec ? y2s : ys) + 64 * wh * YLD);
    } else {
#pragma unroll
      for (int h = 0; h < NY; ++h) {
        st.ty[h].store(ys + 64 * h * YLD);
        if constexpr (CROSS) st.ty2[h].store(y2s + 64 * h * YLD);
      }
    }
    if constexpr (STORE == 2) {
      // the state before this chunk, [v][k], through LDS
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss[(16 * j + 4 * qd + e) * SLD + 16 * w + r] = (StT)acc[j][e];
    } else if constexpr (STORE != 0) {
      // the state before this chunk, [k][v], through LDS: this lane's four consecutive
      // values of row krow in each column tile as one 8- or 16-byte write
      StT* srow = ss + (16 * w + r) * SLD + 4 * qd;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if constexpr (sizeof(StT) == 2) {
          bf16x4 b;
#pragma unroll
          for (int e = 0; e < 4; ++e) b[e] = (bf16)acc[j][e];
          *reinterpret_cast<bf16x4*>(srow + 16 * j) = b;
        } else {
          *reinterpret_cast<f32x4*>(srow + 16 * j) = acc[j];
        }
      }
    }
    __syncthreads();
    if constexpr (STORE != 0) {
      constexpr int kPer = 16 / (int)sizeof(StT), kCols = STORE == 2 ? 64 : TV;
      constexpr int kUnits = 64 * TV / kPer;
      const long sb = ((long)bh * N + i) * dk * dv;
#pragma unroll
      for (int u_ = 0; u_ < (kUnits + kThreads - 1) / kThreads; ++u_) {   // fixed trip count
        const int idx = threadIdx.x + u_ * kThreads;
        if ((kUnits) % kThreads != 0 && idx >= kUnits) continue;
        const int e0 = idx * kPer;
        int a = e0 / kCols, b = e0 % kCols;
        long off;
        if constexpr (STORE == 2) off = sb + (long)(v0 + a) * dk + k0 + b;
        else off = sb + (long)(k0 + a) * dv + v0 + b;
        if constexpr (SPAD4) {
          if (frag_states) {
            // MFMA fragment order of the chunk's [dk][dv] state, as B operands of
            // products over dv: fragment (16-row block, 32-column block) holds, for lane
            // 16 q + r, row r and columns 8 q .. 8 q + 7 (16 bytes); units run through
            // this tile's 4 x 4 fragments lane by lane, so the stores stay contiguous
            const int fi = idx / 64, ln = idx % 64;
            a = 16 * (fi / 4) + ln % 16;
            b = 32 * (fi % 4) + 8 * (ln / 16);
            off = sb + (((long)(k0 / 16 + fi / 4) * (dv / 32) + (v0 / 32 + fi % 4)) * 64 + ln) * 8;
          }
        }
        u32x4 v;
        if constexpr (SPAD4) {   // rows are 8-byte aligned only
          const uint2* p = reinterpret_cast<const uint2*>(ss + a * SLD + b);
          const uint2 p0 = p[0], p1 = p[1];
          v = u32x4{p0.x, p0.y, p1.x, p1.y};
        } else {
          v = *reinterpret_cast<const u32x4*>(ss + a * SLD + b);
        }
        // written once, read by a later kernel: a streaming store, so that the tiles
        // the neighbouring workgroups share stay in L2
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>((StT*)states + off));
      }
    }
    if constexpr (CROSS) {
      if (i_prev >= 0 && qd == 0)
        cross[(((long)bh * N + i_prev) * nvt + vt) * dk + krow] = part_prev;
    }
    fetch_y(st, WT ? chunk_of(step + 1) : ipre);

    if constexpr (CROSS) {
      // P_j = X2^T Y2 for column tile j (same layout as the state), folded into the row
      // sum one tile at a time; the four lanes of a row (qd) then add their partial sums
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < C / 32; ++kb) {
          Frag<OpT> fb;
          yfrag(fb, y2s, 16 * j + r, kb);
          st.cx2.apply_t(P, kb, fb);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sum += acc[j][e] * P[e];
      }
      st.cx2.load(X2T + xrow(ipre), kst);
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      part_prev = sum;
      i_prev = i;
    }

#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[j][e] *= egr;
#pragma unroll
    for (int kb = 0; kb < C / 32; ++kb)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        Frag<OpT> fb;
        yfrag(fb, ys, 16 * j + r, kb);
        st.cx.apply_t(acc[j], kb, fb);
      }
    st.cx.load(XT + xrow(ipre), kst);
    __syncthreads();
  };
  // blocks of EB steps (EB even: step s runs on set s % DEPTH throughout); each step ends
  // with a barrier, so the previous block's decays are no longer read when restaged
  static_assert(EB % 2 == 0 && EB * 64 % kThreads == 0, "decay staging");
  int step = 0;
  for (int sb = 0; sb < nst; sb += EB) {
    if (sb > 0) {
      stage_eg(sb);
      __syncthreads();
    }
    const int se = min(sb + EB, nst);
    if constexpr (DEPTH == 2) {
      for (; step + 1 < se; step += 2) {
        body(step, sets[0]);
        body(step + 1, sets[DEPTH - 1]);
      }
    }
    for (; step < se; ++step) body(step, sets[0]);
  }
  if constexpr (CROSS) {
    if (i_prev >= 0 && qd == 0) cross[(((long)bh * N + i_prev) * nvt + vt) * dk + krow] = part_prev;
  }
  if (S_out) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      *reinterpret_cast<f32x4*>(S_out + ((long)bh * dk + krow) * dv + v0 + 16 * j + 4 * qd) = acc[j];
  }
  // segmented scan: the segment's total decay per row, [nseg][BH][dk]
  if (segdec && vt == 0 && qd == 0)
    segdec[((long)sg * (base / (nvt * nkt)) + bh) * dk + krow] = dprod;
}

template <typename Tin, typename OpT, bool SPLIT, int C, int STORE, bool CROSS, int TV>
static void launch_scan_k(const ScanArgs& a, const ScanArgs* b, hipStream_t s) {
  auto dir = [](const ScanArgs& x) {
    ScanDir d;
    d.XT = x.XT; d.Y = x.Y; d.X2T = x.X2T; d.Y2 = x.Y2; d.cross = x.cross; d.S_in = x.S_in;
    d.states = x.states; d.S_out = x.S_out; d.reverse = x.reverse ? 1 : 0;
    d.frag_states = x.frag_states ? 1 : 0;
    const bool segm = x.seg_p > 1;
    d.seg_in = segm ? x.seg_in : nullptr;
    d.seg_dec = segm ? x.seg_decay : nullptr;
    return d;
  };
  const bool segm = a.seg_p > 1;
  const int ndir = b ? 2 : 1, nseg = segm ? a.nseg : 1;
  dim3 grid(ndir * nseg * (a.dv / TV) * (a.dk / 64) * a.BH);
  hipLaunchKernelGGL((k_state_scan<Tin, OpT, SPLIT, C, STORE, CROSS, TV>), grid, dim3(kThreads), 0,
                     s, dir(a), dir(b ? *b : a), ndir, a.eg, a.T, a.dk, a.dv, a.N,
                     a.nsteps > 0 && a.nsteps < a.N ? a.nsteps : a.N, nseg, segm ? a.seg_p : 1,
                     a.xt_hi ? 2 : 1);
}

int scan_tile_v(const ScanArgs& a) {
  return (a.cross && a.dtype != 0 && a.C == 64 && a.dv % 128 == 0) ? 128 : 64;
}

template <typename Tin, typename OpT, bool SPLIT, int C>
static hipError_t launch_scan_t(const ScanArgs& a, const ScanArgs* b, hipStream_t s) {
  if (a.cross) {
    // the backward: operand-type states, [dk][dv]
    if constexpr (C == 64 && sizeof(OpT) == 2) {
      if (scan_tile_v(a) == 128) {
        launch_scan_k<Tin, OpT, SPLIT, C, 1, true, 128>(a, b, s);
        return hipGetLastError();
      }
    }
    launch_scan_k<Tin, OpT, SPLIT, C, 1, true, 64>(a, b, s);
  } else if constexpr (SPLIT) {
    // split operands come with the backward's scans: the cross-term scans above, and the
    // segment end states before them (no stores)
    if (a.store != 0) return hipErrorInvalidValue;
    launch_scan_k<Tin, OpT, SPLIT, C, 0, false, 64>(a, b, s);
  } else {
    switch (a.store) {
      case 0: launch_scan_k<Tin, OpT, SPLIT, C, 0, false, 64>(a, b, s); break;
      case 1: launch_scan_k<Tin, OpT, SPLIT, C, 1, false, 64>(a, b, s); break;
      case 2: launch_scan_k<Tin, OpT, SPLIT, C, 2, false, 64>(a, b, s); break;
      default: launch_scan_k<Tin, OpT, SPLIT, C, 3, false, 64>(a, b, s); break;
    }
  }
  return hipGetLastError();
}

static hipError_t launch_scans(const ScanArgs& a, const ScanArgs* b, hipStream_t s) {
  if (a.BH == 0 || a.N == 0) return hipSuccess;
  if (a.cross && a.store != 1) return hipErrorInvalidValue;
  // fragment-ordered states: bf16, chunk 64, 128-column tiles (the backward's scans)
  auto frag_ok = [](const ScanArgs& x) {
    return !x.frag_states || (x.dtype != 0 && x.C == 64 && x.store == 1 && x.cross &&
                              scan_tile_v(x) == 128);
  };
  if (!frag_ok(a) || (b && !frag_ok(*b))) return hipErrorInvalidValue;
  // sequence segments (seg_p > 1): without stores, the end states of segments
  // 0 .. nseg - 1 (0 < nseg < seg_p <= N; decay products wherever the segments are
  // chained, nseg > 1); with stores, every segment from its start state
  // (nseg == seg_p <= N); the same segments in both scans of a launch
  auto seg_ok = [](const ScanArgs& x) {
    if (x.seg_p <= 1) return x.nseg <= 1;
    if (x.seg_p > x.N || x.nseg < 1) return false;
    if (x.store == 0) return x.nseg < x.seg_p && x.S_out && (x.nseg == 1 || x.seg_decay);
    return x.nseg == x.seg_p && x.seg_in != nullptr;
  };
  if (!seg_ok(a) || (b && (!seg_ok(*b) || b->seg_p != a.seg_p || b->nseg != a.nseg)))
    return hipErrorInvalidValue;
  if (b && (b->dtype != a.dtype || b->C != a.C || b->BH != a.BH || b->T != a.T ||
            b->dk != a.dk || b->dv != a.dv || b->N != a.N || b->xt_f32 != a.xt_f32 ||
            b->xt_hi != a.xt_hi ||
            b->store != a.store || (b->cross != nullptr) != (a.cross != nullptr) || b->eg != a.eg ||
            b->nsteps != a.nsteps))
    return hipErrorInvalidValue;
  // the high parts alone: bf16 operands in the split layout, read as unsplit ones
  if (a.xt_hi && (a.dtype == 0 || a.xt_f32)) return hipErrorInvalidValue;
  if (a.dtype == 0) return launch_scan_t<float, float, false, 64>(a, b, s);
  if (a.xt_f32) {
    if (a.C == 64) return launch_scan_t<bf16, bf16, true, 64>(a, b, s);
    return launch_scan_t<bf16, bf16, true, 128>(a, b, s);
  }
  if (a.C == 64) return launch_scan_t<bf16, bf16, false, 64>(a, b, s);
  return launch_scan_t<bf16, bf16, false, 128>(a, b, s);
}

hipError_t launch_state_scan(const ScanArgs& a, hipStream_t s) { return launch_scans(a, nullptr, s); }

int scan_segments(const ScanArgs& a) {
  // at least 8 chunks per segment: each pass has a fixed start-up cost (initial state,
  // decay staging) that a shorter walk does not repay
  if (a.cross || a.store == 0 || a.N < 16 || (a.nsteps > 0 && a.nsteps < a.N)) return 1;
  const long tiles = (long)a.BH * (a.dk / 64) * (a.dv / scan_tile_v(a));
  if (tiles >= 256) return 1;
  int P = (int)(512 / tiles);   // these scans hold two or more workgroups per CU
  P = P > 8 ? 8 : P;
  P = P > a.N / 8 ? a.N / 8 : P;
  return P < 2 ? 2 : P;
}

hipError_t launch_state_scan_seg(const ScanArgs& a, float* slots, float* dec, hipStream_t s) {
  const int P = scan_segments(a);
  if (P <= 1) return launch_scans(a, nullptr, s);
  if (!slots || (P > 2 && !dec)) return hipErrorInvalidValue;
  // the states at the segment starts: segment end states from zero (the first from S_in),
  // then chained
  ScanArgs pre = a;
  pre.store = 0; pre.states = nullptr; pre.S_out = slots; pre.seg_in = nullptr;
  if (P == 2) {   // the first half in walk order (reverse: chunks [N / 2, N))
    pre.nseg = 0; pre.nsteps = a.reverse ? a.N - a.N / 2 : a.N / 2; pre.seg_decay = nullptr;
  } else {
    pre.nseg = P - 1; pre.seg_p = P; pre.seg_decay = dec;
  }
  hipError_t e = launch_scans(pre, nullptr, s);
  if (e != hipSuccess) return e;
  if ((e = launch_seg_combine(slots, dec, a.BH, a.dk, a.dv, P, s)) != hipSuccess) return e;
  // every segment from its start state, writing its chunks' states
  ScanArgs run = a;
  run.nseg = P; run.seg_p = P; run.seg_in = slots; run.seg_decay = nullptr;
  return launch_scans(run, nullptr, s);
}

int scan2_segments(int dtype, int C, int BH, int dk, int dv, int N) {
  // the value columns of a cross-term scan workgroup (as scan_tile_v)
  const int TV = (dtype != 0 && C == 64 && dv % 128 == 0) ? 128 : 64;
  const long wgs = 2L * BH * (dk / 64) * (dv / TV);   // both scans
  // at one workgroup per CU and more the scans stream near the copy rate (bf16) or near
  // the fp32 matrix-unit rate (fp32), and a pass for the segment end states costs more
  // than the parallelism gains; so does it for walks shorter than 32 chunks per segment
  // (measured: 32 chunks of 128 workgroups ran fastest as one walk)
  if (N < 64 || wgs >= 256) return 1;
  int P = (int)(512 / wgs);   // these scans hold two workgroups per CU
  P = P > 8 ? 8 : P;
  P = P > N / 32 ? N / 32 : P;
  return P < 2 ? 2 : P;
}

hipError_t launch_state_scan2_seg(const ScanArgs& a, const ScanArgs& b, float* slots, float* dec,
                                  hipStream_t s) {
  const int P = scan2_segments(a.dtype, a.C, a.BH, a.dk, a.dv, a.N);
  if (P <= 1 || (a.nsteps > 0 && a.nsteps < a.N)) return launch_scans(a, &b, s);
  if (!slots || (P > 2 && !dec)) return hipErrorInvalidValue;
  const long slot = (long)(P - 1) * a.BH * a.dk * a.dv, dslot = (long)(P - 1) * a.BH * a.dk;
  // segment end states of both scans, from zero (each first segment from its S_in), no
  // stores and no cross terms
  auto pre = [&](const ScanArgs& x, int k) {
    ScanArgs y = x;
    y.store = 0; y.states = nullptr; y.frag_states = false; y.cross = nullptr;
    y.X2T = nullptr; y.Y2 = nullptr; y.S_out = slots + k * slot; y.seg_in = nullptr;
    y.nseg = P - 1; y.seg_p = P; y.seg_decay = P > 2 ? dec + k * dslot : nullptr;
    return y;
  };
  const ScanArgs pa = pre(a, 0), pb = pre(b, 1);
  hipError_t e = launch_scans(pa, &pb, s);
  if (e != hipSuccess) return e;
  if ((e = launch_seg_combine(slots, dec, a.BH, a.dk, a.dv, P, s)) != hipSuccess) return e;
  if ((e = launch_seg_combine(slots + slot, P > 2 ? dec + dslot : nullptr, a.BH, a.dk, a.dv, P,
                              s)) != hipSuccess)
    return e;
  // every segment of both scans from its start state, with stores and cross terms
  auto run = [&](const ScanArgs& x, int k) {
    ScanArgs y = x;
    y.nseg = P; y.seg_p = P; y.seg_in = slots + k * slot; y.seg_decay = nullptr;
    return y;
  };
  const ScanArgs ra = run(a, 0), rb = run(b, 1);
  return launch_scans(ra, &rb, s);
}

// Segment end states -> states at the segment starts (see launch_seg_combine): one
// workgroup per (16 state rows, 64 columns, bh), 512 and more for the shapes that take
// segments; each thread loads all segment slots of its four elements at once and chains
// them with the segments' decay products.
__global__ __launch_bounds__(kThreads) void k_seg_combine(float* __restrict__ S,
                                                          const float* __restrict__ dec, int BH,
                                                          int dk, int dv, int P) {
  const int c0 = 64 * blockIdx.x, k0 = 16 * blockIdx.y, bh = blockIdx.z;
  const long slot = (long)BH * dk * dv;
  const int kr = threadIdx.x >> 4, c = (threadIdx.x & 15) * 4;
  const long off = ((long)bh * dk + k0 + kr) * dv + c0 + c;
  f32x4 x[8];
  float g[8];
#pragma unroll
  for (int sg = 0; sg < 8; ++sg) {
    if (sg < P - 1) {
      x[sg] = *reinterpret_cast<const f32x4*>(S + sg * slot + off);
      g[sg] = dec[((long)sg * BH + bh) * dk + k0 + kr];
    }
  }
#pragma unroll
  for (int sg = 1; sg < 8; ++sg) {
    if (sg < P - 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[sg][e] = g[sg] * x[sg - 1][e] + x[sg][e];
      *reinterpret_cast<f32x4*>(S + sg * slot + off) = x[sg];
    }
  }
}

hipError_t launch_seg_combine(float* S, const float* dec, int BH, int dk, int dv, int P,
                              hipStream_t s) {
  if (P <= 2 || BH == 0) return hipSuccess;
  if (P > 9 || dk % 64 != 0 || dv % 64 != 0) return hipErrorInvalidValue;
  static_assert(kThreads == 256, "16 rows of 16 four-column units per workgroup");
  hipLaunchKernelGGL(k_seg_combine, dim3(dv / 64, dk / 16, BH), dim3(kThreads), 0, s, S, dec, BH,
                     dk, dv, P);
  return hipGetLastError();
}
hipError_t launch_state_scan2(const ScanArgs& a, const ScanArgs& b, hipStream_t s) {
  return launch_scans(a, &b, s);
}

}  // namespace gla
