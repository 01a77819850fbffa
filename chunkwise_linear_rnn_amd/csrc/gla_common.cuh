// Device-side building blocks shared by the gfx950 GLA kernels: element types, the
// MFMA 16x16 tile step, operand-fragment loads, and global<->LDS tile staging.
//
// MFMA conventions (CDNA4 v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x4_f32, checked
// on the device): in a wave of 64 lanes, lane l has r = l % 16 and q = l / 16.
//   accumulator (16x16 fp32 tile D):  lane holds D[4q + i][r], i = 0..3   (f32x4)
//   one "k32 step" D += A(16x32) * B(32x16): lane supplies 8 values of row r of A and
//   the same 8 k-indices of column r of B.  Which 8 of the 32 k-indices lane group q
//   carries is a free choice as long as A and B agree; two choices are used:
//     contiguous   k = 8q + e                       (one 16-byte bf16 load)
//     acc-order    k = 4q + e (e<4), 16 + 4q + e-4   (matches two stacked accumulator
//                  tiles, so an fp32 accumulator can feed the next product as B)
// For fp32 operands the k32 step is 8 v_mfma_f32_16x16x4_f32, the e-th taking element
// e from every lane group.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kThreads = 256;   // 4 waves per workgroup everywhere
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// MI355X places workgroup L of a launch (linear id) on XCD L % 8, and each XCD has its
// own L2.  This maps the linear id to a logical tile id such that logical ids
// [x*per + min(x, rem), ...) all run on XCD x: tiles that are consecutive in logical order
// (and share operands) share one L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_logical(int L, int total) {
  const int x = L % kXcds, slot = L / kXcds, per = total / kXcds, rem = total % kXcds;
  return x * per + (x < rem ? x : rem) + slot;
}
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// e^x with the hardware base-2 exponential.  Arguments here are differences of
// cumulative log-gates (<= 0 in every use), so no overflow handling is needed.

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// ---------------------------------------------------------------------------------
// Operand fragments and the k32 MFMA step
// ---------------------------------------------------------------------------------
template <typename OpT> struct Frag;
template <> struct Frag<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void set(int e, float x) { v[e] = (bf16)x; }
  __device__ __forceinline__ float get(int e) const { return (float)v[e]; }
};
template <> struct Frag<float> {
  float v[8];
  __device__ __forceinline__ void set(int e, float x) { v[e] = x; }
  __device__ __forceinline__ float get(int e) const { return v[e]; }
};

__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// Contiguous-order fragment: p points at (row, k0) of a k-contiguous tile; reads
// p[8q .. 8q+7].  p + 8q must be 16-byte aligned.
__device__ __forceinline__ void load_frag_c(Frag<bf16>& f, const bf16* p) {
  f.v = *reinterpret_cast<const bf16x8*>(p + 8 * (lane_id() >> 4));
}
__device__ __forceinline__ void load_frag_c(Frag<float>& f, const float* p) {
  const f32x4* s = reinterpret_cast<const f32x4*>(p + 8 * (lane_id() >> 4));
  f32x4 a = s[0], b = s[1];
#pragma unroll
  for (int e = 0; e < 4; ++e) { f.v[e] = a[e]; f.v[4 + e] = b[e]; }
}
// Acc-order fragment: reads p[4q .. 4q+3] and p[16+4q .. 16+4q+3].
__device__ __forceinline__ void load_frag_a(Frag<bf16>& f, const bf16* p) {
  const int q = lane_id() >> 4;
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p + 4 * q);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 16 + 4 * q);
#pragma unroll
  for (int e = 0; e < 4; ++e) { f.v[e] = a[e]; f.v[4 + e] = b[e]; }
}
__device__ __forceinline__ void load_frag_a(Frag<float>& f, const float* p) {
  const int q = lane_id() >> 4;
  f32x4 a = *reinterpret_cast<const f32x4*>(p + 4 * q);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 16 + 4 * q);
#pragma unroll
  for (int e = 0; e < 4; ++e) { f.v[e] = a[e]; f.v[4 + e] = b[e]; }
}
// B fragment (acc order) from two stacked fp32 accumulator tiles (rows 0-15, 16-31).
template <typename OpT>
__device__ __forceinline__ void frag_from_acc(Frag<OpT>& f, const f32x4& lo, const f32x4& hi) {
#pragma unroll
  for (int e = 0; e < 4; ++e) { f.set(e, lo[e]); f.set(4 + e, hi[e]); }
}

// ---------------------------------------------------------------------------------
// Vector loads of 8 consecutive input elements, widened to fp32
// ---------------------------------------------------------------------------------
__device__ __forceinline__ void load8(float (&x)[8], const bf16* p) {
  bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}
__device__ __forceinline__ void load8(float (&x)[8], const float* p) {
  f32x4 a = reinterpret_cast<const f32x4*>(p)[0], b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
  for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
}
__device__ __forceinline__ void store8(bf16* p, const float (&x)[8]) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
  *reinterpret_cast<bf16x8*>(p) = v;
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  f32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) { a[e] = x[e]; b[e] = x[4 + e]; }
  reinterpret_cast<f32x4*>(p)[0] = a;
  reinterpret_cast<f32x4*>(p)[1] = b;
}
// Streaming (nontemporal) 16-byte stores, for outputs written once and read only by a
// later kernel: they do not hold L2 lines that the workgroups still share.
template <typename T>
__device__ __forceinline__ void stream16(T* p, const u32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void stream8(bf16* p, const float (&x)[8]) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
  stream16(p, __builtin_bit_cast(u32x4, v));
}
__device__ __forceinline__ void stream8(float* p, const float (&x)[8]) {
  f32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) { a[e] = x[e]; b[e] = x[4 + e]; }
  stream16(p, __builtin_bit_cast(u32x4, a));
  stream16(p + 4, __builtin_bit_cast(u32x4, b));
}
__device__ __forceinline__ void zero8(float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = 0.f;
}

// ---------------------------------------------------------------------------------
// Tile staging, global (row-major, `rows` valid rows, zero beyond) -> LDS.
// All threads of the workgroup take part; the caller places the barriers.
// ---------------------------------------------------------------------------------
// Same orientation: lds[r * lld + c] = src[r * gld + c], c in [0, COLS).
template <typename OpT, typename Tin, int ROWS, int COLS>
__device__ __forceinline__ void stage_rows(OpT* lds, int lld, const Tin* src, long gld, int rows) {
  constexpr int kVec = COLS / 8;
  for (int idx = threadIdx.x; idx < ROWS * kVec; idx += kThreads) {
    const int r = idx / kVec, c = (idx % kVec) * 8;
    float x[8];
    if (r < rows) load8(x, src + r * gld + c); else zero8(x);
    store8(lds + r * lld + c, x);
  }
}
// Transposed: lds[c * lld + r] = src[r * gld + c] for r in [0, ROWS), c in [0, COLS).
// Each thread moves a 2-row x 8-column block so that bf16 pairs go out as 32-bit words.
template <typename OpT, typename Tin, int ROWS, int COLS>
__device__ __forceinline__ void stage_cols(OpT* lds, int lld, const Tin* src, long gld, int rows) {
  constexpr int kVec = COLS / 8;
  for (int idx = threadIdx.x; idx < (ROWS / 2) * kVec; idx += kThreads) {
    const int r = (idx / kVec) * 2, c = (idx % kVec) * 8;
    float x0[8], x1[8];
    if (r < rows) load8(x0, src + r * gld + c); else zero8(x0);
    if (r + 1 < rows) load8(x1, src + (r + 1) * gld + c); else zero8(x1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (sizeof(OpT) == 2) {
        bf16x2 w;
        w[0] = (bf16)x0[e];
        w[1] = (bf16)x1[e];
        *reinterpret_cast<bf16x2*>(lds + (c + e) * lld + r) = w;
      } else {
        f32x2 w;
        w[0] = x0[e];
        w[1] = x1[e];
        *reinterpret_cast<f32x2*>(lds + (c + e) * lld + r) = w;
      }
    }
  }
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

// ---------------------------------------------------------------------------------
// Register-staged tile copies (global -> registers now, registers -> LDS later), so
// the next chunk's loads are in flight while the current chunk computes.  NT is the
// workgroup size (all of its threads take part).
// ---------------------------------------------------------------------------------

// A contiguous global tile of ROWS x COLS elements (row-major, COLS contiguous) moved as
// 16-byte units into an LDS tile with row stride LD (elements).
template <typename T, int ROWS, int COLS, int LD, int NT = kThreads>
struct FlatTile {
  static constexpr int kPer = 16 / (int)sizeof(T);            // elements per unit
  static constexpr int kUnits = ROWS * COLS / kPer;
  static constexpr int kPerThread = (kUnits + NT - 1) / NT;
  u32x4 u[kPerThread];
  __device__ __forceinline__ void load(const T* __restrict__ g) {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int idx = threadIdx.x + j * NT;
      if (kUnits % NT == 0 || idx < kUnits)
        u[j] = *reinterpret_cast<const u32x4*>(g + (long)idx * kPer);
    }
  }
  __device__ __forceinline__ void store(T* lds) const {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int idx = threadIdx.x + j * NT;
      if (kUnits % NT == 0 || idx < kUnits) {
        const int e = idx * kPer, r = e / COLS, c = e % COLS;
        *reinterpret_cast<u32x4*>(lds + r * LD + c) = u[j];
      }
    }
  }
};

// Sum over the 16 lanes of a DPP row (lanes with the same l / 16), result in every lane.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_f<0x124>(x);   // row_ror 4
  x += dpp_f<0x128>(x);   // row_ror 8
  return x;
}

// Row-bounded tile loads: every lane issues its 16-byte load (rows at or beyond `rows`,
// which must be >= 1, read the last valid row instead), and the words of rows beyond are
// zeroed only when the tile is stored to LDS.  With no branch around the loads and no use
// of their data before the store, the compiler's counts of loads in flight stay exact and
// the loads of a prefetched tile stay in flight until then.
template <typename T>
__device__ __forceinline__ u32x4 load16_clamped(const T* __restrict__ g, long gld, int r, int c,
                                                int rows) {
  return *reinterpret_cast<const u32x4*>(g + (long)min(r, rows - 1) * gld + c);
}
__device__ __forceinline__ u32x4 keep_if(const u32x4& v, bool ok) {
  return u32x4{ok ? v[0] : 0u, ok ? v[1] : 0u, ok ? v[2] : 0u, ok ? v[3] : 0u};
}

// ROWS x COLS tile of a row-major [*, gld] matrix (rows beyond `rows` zero, rows >= 1) moved as
// 16-byte units into an LDS tile with row stride LD, same orientation.
template <typename T, int ROWS, int COLS, int LD, int NT = kThreads>
struct RowTile {
  static constexpr int kPer = 16 / (int)sizeof(T);
  static constexpr int kUnitsRow = COLS / kPer;
  static constexpr int kUnits = ROWS * kUnitsRow;
  static constexpr int kPerThread = (kUnits + NT - 1) / NT;
  u32x4 u[kPerThread];
  int nrows;
  __device__ __forceinline__ void load(const T* __restrict__ g, long gld, int rows) {
    nrows = rows;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int idx = threadIdx.x + j * NT;
      const int r = idx / kUnitsRow, c = (idx % kUnitsRow) * kPer;
      if (kUnits % NT == 0 || idx < kUnits)
        u[j] = load16_clamped(g, gld, r, c, rows);
    }
  }
  __device__ __forceinline__ void store(T* lds) const {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int idx = threadIdx.x + j * NT;
      const int r = idx / kUnitsRow, c = (idx % kUnitsRow) * kPer;
      if (kUnits % NT == 0 || idx < kUnits)
        *reinterpret_cast<u32x4*>(lds + r * LD + c) = keep_if(u[j], r < nrows);
    }
  }
};

// Same as FlatTile, for a tile whose rows are contiguous in global memory and COLS
// elements long (alias kept for readability at call sites).
template <typename T, int ROWS, int COLS, int LD>
using FlatTileRows = FlatTile<T, ROWS, COLS, LD>;

// Position of element (column c, row r) of a transposed tile kept with the swizzle of
// ColTile<..., SWZ = true>: each LDS row (one column c of the source) is made of 8-element
// chunks, and chunk r / 8 sits at chunk (r / 8) ^ ((c / 8) % 8) ^ ((c / 4) % 2).  Banks as
// measured on gfx950: 4-byte writes serve 32 lanes per cycle from 32 banks; 16-byte reads
// serve 16 lanes per cycle from 64 banks (each half wave split by the parity of lane bits
// 2..4).  With row strides of 72 (chunk 64) or 136 (chunk 128) bf16 elements, the
// transposing 4-byte stores of ColTile (eight column blocks of a 2-row unit per 32 lanes)
// and the 16-byte fragment reads of 16 consecutive rows both touch distinct banks.
__device__ __forceinline__ int swz_chunk(int c, int chunk) {
  return chunk ^ ((c >> 3) & 7) ^ ((c >> 2) & 1);
}
// Fragment read from such a tile: row `c`, elements 32 kb + 8 (lane / 16) .. + 7.
__device__ __forceinline__ void load_frag_cs(Frag<bf16>& f, const bf16* tile, int LD, int c,
                                             int kb) {
  const int ch = swz_chunk(c, 4 * kb + (lane_id() >> 4));
  f.v = *reinterpret_cast<const bf16x8*>(tile + c * LD + 8 * ch);
}

// ROWS x 64 slice of a row-major [*, gld] matrix, rows beyond `rows` (>= 1) zero, staged
// transposed (lds[c * LD + r]) through 2-row x 8-column units.  The loads keep the raw
// 16-byte words (no use of the data until store), so they stay in flight.  Input and
// LDS element types are the same (bf16 or fp32).  SWZ (bf16 only): rows of the staged
// tile are chunk-swizzled as described at swz_chunk.
template <typename OpT, typename Tin, int ROWS, int LD, int NT = kThreads, bool SWZ = false>
struct ColTile {
  static_assert(!SWZ || sizeof(OpT) == 2, "swizzled staging is for 16-bit elements");
  static_assert(sizeof(OpT) == sizeof(Tin), "same element type in and out");
  static constexpr int kWords = sizeof(Tin) == 2 ? 1 : 2;   // 16-byte words per 8 elements
  static constexpr int kUnits = (ROWS / 2) * 8;
  static constexpr int kPerThread = (kUnits + NT - 1) / NT;
  u32x4 x0[kPerThread][kWords], x1[kPerThread][kWords];
  int nrows;
  __device__ __forceinline__ void load(const Tin* __restrict__ g, long gld, int rows) {
    nrows = rows;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int idx = threadIdx.x + j * NT;
      const int r = (idx / 8) * 2, c = (idx % 8) * 8;
      if (kUnits % NT == 0 || idx < kUnits) {
#pragma unroll
        for (int h = 0; h < kWords; ++h) {
          const int ce = c + h * (8 / kWords);
          x0[j][h] = load16_clamped(g, gld, r, ce, rows);
          x1[j][h] = load16_clamped(g, gld, r + 1, ce, rows);
        }
      }
    }
  }
  // The same units from a [*][ncols] matrix kept in MFMA fragment order (16-row x
  // 32-column fragments of 1 KB, row-block major; lane 16 q + r of a fragment holds row r,
  // columns 8 q .. 8 q + 7): rows r0 + [0, ROWS), columns c0 + [0, 64), all valid.  The
  // two rows of a unit are adjacent 16-byte pieces; a wave reads two whole fragments.
  __device__ __forceinline__ void load_frag(const Tin* __restrict__ g, int ncols, int r0,
                                            int c0) {
    static_assert(sizeof(Tin) == 2, "fragment order is kept for 16-bit states");
    nrows = ROWS;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int idx = threadIdx.x + j * NT;
      const int r = (idx / 8) * 2, c = (idx % 8) * 8;
      if (kUnits % NT == 0 || idx < kUnits) {
        const int d = r0 + r, v = c0 + c;
        const Tin* p = g + (((long)(d >> 4) * (ncols >> 5) + (v >> 5)) * 64 +
                            16 * ((v & 31) >> 3) + (d & 15)) * 8;
        x0[j][0] = *reinterpret_cast<const u32x4*>(p);
        x1[j][0] = *reinterpret_cast<const u32x4*>(p + 8);
      }
    }
  }
  __device__ __forceinline__ void store(OpT* lds) const {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int idx = threadIdx.x + j * NT;
      const int r = (idx / 8) * 2, c = (idx % 8) * 8;
      if (kUnits % NT == 0 || idx < kUnits) {
        const bool ok0 = r < nrows, ok1 = r + 1 < nrows;
        if constexpr (sizeof(OpT) == 2) {
          // word w of a row holds elements 2w (low half) and 2w+1 (high half)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t a = ok0 ? x0[j][0][w] : 0u, b = ok1 ? x1[j][0][w] : 0u;
            const int c0 = c + 2 * w, c1 = c0 + 1;
            // r is even: the word holding rows r, r + 1 stays inside one 8-row chunk
            const int r0 = SWZ ? 8 * swz_chunk(c0, r >> 3) + (r & 7) : r;
            const int r1 = SWZ ? 8 * swz_chunk(c1, r >> 3) + (r & 7) : r;
            *reinterpret_cast<uint32_t*>(lds + c0 * LD + r0) = (a & 0xFFFFu) | (b << 16);
            *reinterpret_cast<uint32_t*>(lds + c1 * LD + r1) = (a >> 16) | (b & 0xFFFF0000u);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            u32x4 const& A = x0[j][e / 4];
            u32x4 const& B = x1[j][e / 4];
            uint32_t pr[2] = {ok0 ? A[e % 4] : 0u, ok1 ? B[e % 4] : 0u};
            *reinterpret_cast<uint2*>(lds + (c + e) * LD + r) = *reinterpret_cast<uint2*>(pr);
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------------
// Transposed 64 x 64 bf16 tiles without padding (row stride 64 elements = 8 chunks of 8),
// chunk k of row c kept at chunk k ^ g(c), g(c) = 2 ((c / 8) % 4) ^ 4 ((c / 2) % 2).
// Banks of the LDS as measured on gfx950: 16-byte reads serve 16 lanes per cycle from 64
// banks (the lanes of each half wave split by the parity of lane bits 2..4); 16-byte
// writes serve 8 consecutive lanes per cycle from 32 banks.  With this swizzle the
// fragment reads below (16 consecutive rows, one chunk column per 16 lanes) and the block
// writes of WaveColTile (eight lanes: two chunk rows x four column blocks) both touch
// distinct banks in every cycle.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ int swz64(int c, int chunk) {
  return chunk ^ ((c >> 2) & 6) ^ ((c << 1) & 4);
}
// Fragment read: row `c`, elements 32 kb + 8 (lane / 16) .. + 7.
__device__ __forceinline__ void load_frag_x64(Frag<bf16>& f, const bf16* tile, int c, int kb) {
  f.v = *reinterpret_cast<const bf16x8*>(tile + c * 64 + 8 * swz64(c, 4 * kb + (lane_id() >> 4)));
}
// A 64 x 64 slice of a row-major bf16 [*, gld] matrix (rows beyond `rows` >= 1 zero),
// staged by ONE wave into a transposed swizzled tile as above: lane l holds the 8 x 8 block
// at rows 8 rb .., columns 8 cb .. with rb = (l / 4) % 8, cb = l % 4 + 4 (l / 32) (eight
// 16-byte loads; the four lanes of a quad read 64 contiguous bytes of one row), transposes
// it in registers and writes its eight columns as 16-byte words.
struct WaveColTile {
  u32x4 x[8];
  int nrows;
  __device__ __forceinline__ void load(const bf16* __restrict__ g, long gld, int rows) {
    nrows = rows;
    const int l = lane_id(), rb = (l >> 2) & 7, cb = (l & 3) + 4 * (l >> 5);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = load16_clamped(g, gld, 8 * rb + i, 8 * cb, rows);
  }
  __device__ __forceinline__ void store(bf16* lds) const {
    const int l = lane_id(), rb = (l >> 2) & 7, cb = (l & 3) + 4 * (l >> 5);
    // rows at or beyond nrows are zeroed after the transposition: word w of every column
    // holds rows 2w and 2w + 1 of the block
    uint32_t m[4];
#pragma unroll
    for (int w = 0; w < 4; ++w)
      m[w] = (8 * rb + 2 * w < nrows ? 0x0000FFFFu : 0u) | (8 * rb + 2 * w + 1 < nrows ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // column 8 cb + e: word w holds rows 2w (low half) and 2w + 1 (high half), taken from
      // the low (even e) or high (odd e) half of word e / 2 of those rows (v_perm_b32 byte
      // selectors: 0-3 pick bytes of the second source, 4-7 of the first)
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = __builtin_amdgcn_perm(x[2 * w + 1][e / 2], x[2 * w][e / 2], sel) & m[w];
      const int c = 8 * cb + e;
      *reinterpret_cast<u32x4*>(lds + c * 64 + 8 * swz64(c, rb)) = o;
    }
  }
};

}  // namespace gla
