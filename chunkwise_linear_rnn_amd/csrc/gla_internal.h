// Host-side launchers of the gfx950 GLA kernels (internal to libgla_mi355x.so).
// dtype: 0 = fp32 inputs / fp32 operands, 1 = bf16 inputs / bf16 MFMA operands.
#pragma once
#include <hip/hip_runtime.h>

namespace gla {

// Gate front-end (page "Gated Linear Attention Transformers with Hardware-Efficient
// Training", atlas.scime.ai summary, section Approach: a data-dependent gate).  With `on`
// the log_alpha operand holds gate logits x and the layer uses logsigmoid(x) * inv_tau;
// otherwise the operand is log_alpha itself.
struct GateFn {
  int on;
  float inv_tau;
  // logsigmoid(x) = min(x, 0) - log(1 + exp(-|x|)), with the hardware base-2 exp and log
  // (1 + exp(-|x|) is in (1, 2], so its log has no cancellation; for x beyond ~17 the
  // exp term drops below fp32 resolution next to 1 and the gate rounds to exactly 1)
  __device__ __forceinline__ float operator()(float x) const {
    if (!on) return x;
    const float e = __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f);
    return (fminf(x, 0.f) - 0.6931471805599453f * __builtin_amdgcn_logf(1.f + e)) * inv_tau;
  }
  // d log_alpha / dx: sigmoid(-x) * inv_tau, or 1 for log_alpha given directly
  __device__ __forceinline__ float slope(float x) const {
    if (!on) return 1.f;
    const float e = __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f);
    return (x >= 0.f ? e : 1.f) * __builtin_amdgcn_rcpf(1.f + e) * inv_tau;
  }
};

struct IntraArgs {
  int dtype, C, BH, T, dk, N;
  bool want_A;
  bool xt_f32;           // write QhT / KhT as bf16 high part + remainder (bf16 inputs only)
  const void *q, *k, *la;
  const float* g;        // chunk-local cumsum from the gate kernel, or NULL (computed)
  void* A;               // [BH][N][C][C]       operand type
  void *Qh, *QhT, *Kh, *KhT;
  float* eg;             // [BH][N][dk]
  float* g2_out;         // [BH][T][dk] g * log2(e), or NULL
  GateFn gate;           // applied to la (not to g, which is already a cumsum)
  bool gscalar;          // la holds one gate per token: [BH][T], broadcast over dk
};
hipError_t launch_intra(const IntraArgs& a, hipStream_t s);

hipError_t launch_gate_cumsum(int dtype, const void* la, GateFn gate, int gscalar, float* g,
                              float* gamma, int BH, int T, int dk, int C, hipStream_t s);
hipError_t launch_state_dot(const float* dST, const float* ST, float* cT, int BH, int dk, int dv,
                            hipStream_t s);
// chunk totals of D from the scans' cross terms -> tot [BH][N][dk]
hipError_t launch_gate_tot(const float* crossF, const float* crossR, const float* cT,
                             float* tot, int BH, int T, int dk, int ntile, int C, hipStream_t s);
// part != NULL (scalar gates): the per-(t, d) gradient goes to part [BH][T][dk] in fp32,
// without the front-end slope (it may alias Dloc), and dla is not written.
hipError_t launch_gate_grad(int dtype, const float* Dloc, const float* tot, const float* cT,
                            const void* la, GateFn gate, void* dla, float* part, int BH,
                            int T, int dk, int C, hipStream_t s);
// Scalar gates: dla[row] = slope(la[row]) * sum of part[row][0 .. nparts) for the rows
// row < nrows = BH * T (dla and la [BH][T] in the input type).
hipError_t launch_gate_reduce(int dtype, const float* part, int nparts, const void* la,
                              GateFn gate, void* dla, long nrows, hipStream_t s);

// Inter-chunk state scan.  store: 0 = none, 1 = operand type [dk][dv], 2 = operand type
// [dv][dk], 3 = fp32 [dk][dv].  With X2T/Y2/cross set, every step also forms the
// product P_i = X2_i^T Y2_i for the tile and writes the row sums of (held state * P_i)
// to cross [BH][N][dv/64][dk] (fp32).
struct ScanArgs {
  int dtype, C, BH, T, dk, dv, N;
  bool reverse;
  bool xt_f32;           // XT / X2T rows hold a bf16 high part then its remainder
  int store;
  const void* XT;        // [BH][N][dk][C] (Kh^T forward, Qh^T reverse)
  const void* Y;         // [BH][T][dv]    input type (v forward, dO reverse)
  const void* X2T;       // optional second pair for the chunk-total cross term
  const void* Y2;
  float* cross;
  const float* eg;       // [BH][N][dk]
  const float* S_in;     // [BH][dk][dv] or NULL
  void* states;          // see store
  bool frag_states;      // store 1, bf16, 128-column tiles only: states in MFMA fragment
                         // order (see the scan kernel), for the backward chunk kernel
  float* S_out;          // [BH][dk][dv] or NULL
  int nsteps;            // chunks to walk (0: all N); the layout strides still use N
};
hipError_t launch_state_scan(const ScanArgs& a, hipStream_t s);
// Two scans of the same shape and kind (the backward's forward and reverse scans) in one
// launch, so that their workgroups share the machine.
hipError_t launch_state_scan2(const ScanArgs& a, const ScanArgs& b, hipStream_t s);
// Value columns per scan workgroup (the cross-term tiles come in dv / this many).
int scan_tile_v(const ScanArgs& a);
// Per-direction kernel arguments of the scan kernel.
struct ScanDir {
  const void *XT, *Y, *X2T, *Y2;
  float* cross;
  const float* S_in;
  void* states;
  float* S_out;
  int reverse;
  int frag_states;
};

struct OutArgs {
  int dtype, C, BH, T, dk, dv, N;
  const void *Qh, *A, *STt, *v;
  void* o;
};
hipError_t launch_output(const OutArgs& a, hipStream_t s);

struct FusedArgs {
  int dtype, C, BH, T, dk, dv, N;
  const void *Qh, *KhT, *A, *v;
  const float* eg;
  const float* S0;
  void* o;
  float* S_T;
  // sequence split: chunks [0, split) and [split, N) walk in parallel, the second from
  // S_mid = the state before chunk `split` (0: one walk over all chunks)
  int split;
  const float* S_mid;
};
// The split point of the fused forward for a shape (0: no split).  With a split, the
// state before that chunk must be formed first (a state scan over chunks [0, split)).
int fused_split(int dtype, int C, int N);
hipError_t launch_fwd_fused(const FusedArgs& a, hipStream_t s);

struct BwdArgs {
  int dtype, C, BH, T, dk, dv, N;
  const void *q, *k, *v, *dO;
  const float *g, *gamma;   // g: g * log2(e) [BH][T][dk] (from the intra-chunk kernel; the
                            // split path rebuilds it from la and does not read it)
  const void *A, *Kh, *S, *dS;
  void *dq, *dk_out, *dv_out;
  float* Dloc;             // chunk-local suffix sums of D (single-kernel path)
  const float *tot, *cT;   // chunk totals of D, rowsum(dS_T * S_T) or NULL (split path)
  void* dla;               // dlog_alpha, written directly (split path)
  const void* la;          // the gate operand, for the gate front-end's chain rule
  GateFn gate;
  float* dla_part;         // scalar gates (split path): fp32 sums of the per-(t, d) gradient
                           // over each 64-wide d block, [BH][T][dk/64], instead of dla
  bool gscalar;            // la holds one gate per token: [BH][T]
  bool s_frag;             // S and dS (split path) in MFMA fragment order, as the scans wrote them
};
// The backward chunk work (launch_bwd_chunk): with bf16 operands and chunk 64 one launch of
// dq / dk / dlog_alpha workgroups (after the chunk totals are formed) interleaved with dv
// workgroups; otherwise one workgroup per chunk, followed by the gate-gradient kernel.
bool bwd_split(int dtype, int C);
hipError_t launch_bwd_chunk(const BwdArgs& a, hipStream_t s);

// Recurrent evaluation (decoding): T tokens in order, state updated in place.
struct DecodeArgs {
  int dtype, BH, T, dk, dv;
  const void *q, *k, *v, *la;
  float* S;   // [BH][dk][dv]
  void* o;    // [BH][T][dv]
  GateFn gate;
  int gscalar;   // la is [BH][T] (one gate per token), else [BH][T][dk]
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

// Gated Slot Attention (fp32): w = 1 - exp(log_alpha); the first (slot-gated) pass's chunk
// output and chunk backward; row softmax and its backward; the gate-gradient combination.
// Layouts: q, k [BH][T][dk]; w, g2 (chunk-local cumsum * log2 e), s, ds, dw, Dloc [BH][T][m];
// S1, dS1 [BH][N][m][dk] (dS1 of chunk i = the gradient flowing in from chunk i + 1);
// tot [BH][N][m].
hipError_t launch_gsa_w(const float* la, float* w, long n, hipStream_t s);
hipError_t launch_vg_out(const float* q, const float* k, const float* w, const float* g2,
                         const float* S1, float* s_out, int BH, int T, int dk, int m,
                         hipStream_t s);
hipError_t launch_vg_bwd(const float* q, const float* k, const float* w, const float* g2,
                         const float* ds, const float* s_in, const float* S1, const float* dS1,
                         float* dq, float* dk, float* dw, float* Dloc, float* tot, int BH, int T,
                         int dkh, int m, hipStream_t s);
hipError_t launch_softmax_rows(const float* x, float* p, long nrows, int m, hipStream_t s);
hipError_t launch_softmax_bwd(const float* p, const float* dp, float* ds, long nrows, int m,
                              hipStream_t s);
hipError_t launch_gsa_combine(const float* la, const float* dla1, const float* dla2,
                              const float* dw1, const float* dw2, float* dla, long n,
                              hipStream_t s);

}  // namespace gla
