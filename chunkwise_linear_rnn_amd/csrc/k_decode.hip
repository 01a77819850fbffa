// Recurrent (token by token) evaluation of the gated linear-attention state, for decoding
// (page "Gated Slot Attention for Efficient Linear-Time Sequence Modeling", mlsanity.com
// summary, Abstract: linear attention and its gated variants infer recurrently; here the
// layer's own recurrence).  For each (batch, head) and each of the call's T tokens in order:
//     S <- diag(exp(log_alpha_t)) S + k_t^T v_t,     o_t = q_t S
// with S the caller's float32 state, updated in place.
//
// One workgroup per (batch*head, 32 value columns).  Thread (row group rg, column group
// cg) keeps rows rg + 32 j (j < dk / 32) x columns 4 cg .. 4 cg + 3 of the state in
// registers for the whole call, so the state is read and written once however many
// tokens the call has; every step is an fp32 multiply-add per element, as in the
// recurrence.  Each token's output reduces over dk across the 32 row groups through LDS
// (double-buffered, one barrier per token).  The kernel is bound by the state traffic,
// 2 * dk * dv * 4 bytes per head and call.
#include "gla_common.cuh"
#include "gla_internal.h"

namespace gla {

template <typename Tin>
__device__ __forceinline__ f32x4 load4(const Tin* p);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <>
__device__ __forceinline__ f32x4 load4<bf16>(const bf16* p) {
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}

template <typename Tin, int NR>
__global__ __launch_bounds__(kThreads) void k_decode(const Tin* __restrict__ q,
                                                     const Tin* __restrict__ k,
                                                     const Tin* __restrict__ v,
                                                     const Tin* __restrict__ la,
                                                     float* __restrict__ S, Tin* __restrict__ o,
                                                     GateFn gf, int gscalar, int T, int dv) {
  constexpr int DK = 32 * NR, TV = 32;
  __shared__ float red[2][32][TV + 1];
  const int nvt = dv / TV;
  const int vt = blockIdx.x % nvt, bh = blockIdx.x / nvt;
  const int cg = threadIdx.x & 7, rg = threadIdx.x >> 3;
  const int c0 = vt * TV + 4 * cg;
  float* Sb = S + (long)bh * DK * dv + c0;

  f32x4 s[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) s[j] = *reinterpret_cast<const f32x4*>(Sb + (long)(rg + 32 * j) * dv);

  for (int t = 0; t < T; ++t) {
    const long tk = ((long)bh * T + t) * DK;
    const f32x4 vv = load4<Tin>(v + ((long)bh * T + t) * dv + c0);
    // scalar gates: one decay for every row of the state
    const float as = gscalar ? __builtin_amdgcn_exp2f(gf(to_f32(la[(long)bh * T + t])) * kLog2e) : 0.f;
    f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int row = rg + 32 * j;
      const float a = gscalar ? as : __builtin_amdgcn_exp2f(gf(to_f32(la[tk + row])) * kLog2e);
      const float kk = to_f32(k[tk + row]), qq = to_f32(q[tk + row]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[j][e] = a * s[j][e] + kk * vv[e];
        part[e] += qq * s[j][e];
      }
    }
    float (*rb)[TV + 1] = red[t & 1];
#pragma unroll
    for (int e = 0; e < 4; ++e) rb[rg][4 * cg + e] = part[e];
    __syncthreads();
    if (threadIdx.x < TV) {
      float sum = 0.f;
#pragma unroll 8
      for (int g = 0; g < 32; ++g) sum += rb[g][threadIdx.x];
      o[((long)bh * T + t) * dv + vt * TV + threadIdx.x] = from_f32<Tin>(sum);
    }
  }
#pragma unroll
  for (int j = 0; j < NR; ++j) *reinterpret_cast<f32x4*>(Sb + (long)(rg + 32 * j) * dv) = s[j];
}

template <typename Tin>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((long)a.BH * (a.dv / 32)));
  switch (a.dk / 32) {
    case 1: hipLaunchKernelGGL((k_decode<Tin, 1>), grid, dim3(kThreads), 0, s, (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.v, (const Tin*)a.la, a.S, (Tin*)a.o, a.gate, a.gscalar, a.T, a.dv); break;
    case 2: hipLaunchKernelGGL((k_decode<Tin, 2>), grid, dim3(kThreads), 0, s, (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.v, (const Tin*)a.la, a.S, (Tin*)a.o, a.gate, a.gscalar, a.T, a.dv); break;
    case 3: hipLaunchKernelGGL((k_decode<Tin, 3>), grid, dim3(kThreads), 0, s, (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.v, (const Tin*)a.la, a.S, (Tin*)a.o, a.gate, a.gscalar, a.T, a.dv); break;
    case 4: hipLaunchKernelGGL((k_decode<Tin, 4>), grid, dim3(kThreads), 0, s, (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.v, (const Tin*)a.la, a.S, (Tin*)a.o, a.gate, a.gscalar, a.T, a.dv); break;
    case 5: hipLaunchKernelGGL((k_decode<Tin, 5>), grid, dim3(kThreads), 0, s, (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.v, (const Tin*)a.la, a.S, (Tin*)a.o, a.gate, a.gscalar, a.T, a.dv); break;
    case 6: hipLaunchKernelGGL((k_decode<Tin, 6>), grid, dim3(kThreads), 0, s, (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.v, (const Tin*)a.la, a.S, (Tin*)a.o, a.gate, a.gscalar, a.T, a.dv); break;
    case 7: hipLaunchKernelGGL((k_decode<Tin, 7>), grid, dim3(kThreads), 0, s, (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.v, (const Tin*)a.la, a.S, (Tin*)a.o, a.gate, a.gscalar, a.T, a.dv); break;
    case 8: hipLaunchKernelGGL((k_decode<Tin, 8>), grid, dim3(kThreads), 0, s, (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.v, (const Tin*)a.la, a.S, (Tin*)a.o, a.gate, a.gscalar, a.T, a.dv); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.BH == 0 || a.T == 0) return hipSuccess;
  if (a.dtype == 0) return launch_decode_t<float>(a, s);
  return launch_decode_t<bf16>(a, s);
}

}  // namespace gla
