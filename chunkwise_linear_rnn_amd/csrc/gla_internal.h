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
  void* A;               // [BH][N][C][C]       operand type
  void *Qh, *QhT, *Kh, *KhT;
  float* eg;             // [BH][N][dk]
  float* g2_out;         // [BH][T][dk] g * log2(e), or NULL
  GateFn gate;           // applied to la
  bool gscalar;          // la holds one gate per token: [BH][T], broadcast over dk
  bool diag_bf16;        // rebased diagonal sub-blocks with bf16 operands (else fp32)
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
  bool xt_hi;            // bf16 XT / X2T in that split layout, read by the high part alone
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
  // sequence segments (seg_p > 1): the sequence split into seg_p parts (chunks
  // [s N / seg_p, (s + 1) N / seg_p)), indexed in walk order (a reverse scan's segment 0
  // is the last part).  Without stores (0 < nseg < seg_p): segments 0 .. nseg - 1 in one
  // launch, each from zero except the first (from S_in), each end state to
  // S_out + s * BH * dk * dv, and each segment's total decay (product of its chunks'
  // exp(gamma)) per row to seg_decay [nseg][BH][dk] (may be NULL).  With stores
  // (nseg == seg_p, cross terms allowed): every segment writes its chunks' states (and
  // cross terms), segment s > 0 from seg_in + (s - 1) * BH * dk * dv; the last one forms
  // S_out.
  int nseg, seg_p;
  float* seg_decay;
  const float* seg_in;
};
hipError_t launch_state_scan(const ScanArgs& a, hipStream_t s);
// Two scans of the same shape and kind (the backward's forward and reverse scans) in one
// launch, so that their workgroups share the machine.
hipError_t launch_state_scan2(const ScanArgs& a, const ScanArgs& b, hipStream_t s);
// Value columns per scan workgroup (the cross-term tiles come in dv / this many).
int scan_tile_v(const ScanArgs& a);
// Chains the segment end states of a segmented scan into the states at the segment
// starts: S[s] <- diag(dec[s]) S[s - 1] + S[s], s = 1 .. P - 2, in place on
// S [P - 1][BH][dk][dv] (slot 0 already the state at the first boundary), dec the
// segments' decay products [P - 1][BH][dk] from the same scan.
hipError_t launch_seg_combine(float* S, const float* dec, int BH, int dk, int dv, int P,
                              hipStream_t s);
// Segments for a scan that writes every chunk's state (1: one walk): about 512
// workgroups when B*H*(dk/64)*(dv/TV) is below 256, at most 8, at least 8 chunks each.
int scan_segments(const ScanArgs& a);
// A forward scan with stores run as scan_segments(a) segments in parallel: the segments'
// end states from zero (one launch), chained into the states at the segment starts
// (workspace slots: (P - 1) * BH * dk * dv floats at `slots`, (P - 1) * BH * dk at `dec`),
// then every segment walked from its start state.  S_out (the final state) is formed by
// the last segment.  One plain launch when scan_segments(a) == 1.
hipError_t launch_state_scan_seg(const ScanArgs& a, float* slots, float* dec, hipStream_t s);
// Segments for the backward's two scans with cross terms (1: one walk each): only where
// the walk bounds them, below 256 workgroups for both scans; then about 512 workgroups,
// at most 8 segments, at least 32 chunks per segment.
int scan2_segments(int dtype, int C, int BH, int dk, int dv, int N);
// launch_state_scan2 in scan2_segments segments: both scans' segment end states (one
// launch, no stores), chained, then every segment of both scans walked from its start
// state with stores and cross terms.  slots: 2 (P - 1) BH dk dv floats (a's slots, then
// b's); dec: 2 (P - 1) BH dk floats (P > 2 only).
hipError_t launch_state_scan2_seg(const ScanArgs& a, const ScanArgs& b, float* slots, float* dec,
                                  hipStream_t s);
// Per-direction kernel arguments of the scan kernel.
struct ScanDir {
  const void *XT, *Y, *X2T, *Y2;
  float* cross;
  const float* S_in;
  void* states;
  float* S_out;
  const float* seg_in;   // segment start states (see ScanArgs)
  float* seg_dec;        // segment decay products (see ScanArgs)
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
  // sequence split: nseg segments, chunks [s N / nseg, (s + 1) N / nseg), walked in
  // parallel, segment s > 0 from S_mid + (s - 1) * BH * dk * dv (the state at its first
  // chunk); nseg = 1: one walk over all chunks
  int nseg;
  const float* S_mid;
  // bf16: Kh^T in the backward's layout (each fragment followed by its bf16 remainder,
  // as the backward's intra-chunk kernel writes it for the scans); only the fragments are
  // read
  bool kht_split;
};
// The number of sequence segments of the fused forward for a shape (1: no split): enough
// for about 256 workgroups (one per CU) when B*H*dv/64 is small, at most 8, and at least
// two chunks per segment.  With a split, the states at the segment starts are formed first
// (a segmented state scan and, for more than two segments, launch_seg_combine).
int fused_segments(int dtype, int C, int N, int BH, int dv);
hipError_t launch_fwd_fused(const FusedArgs& a, hipStream_t s);

struct BwdArgs {
  int dtype, C, BH, T, dk, dv, N;
  const void *q, *k, *v, *dO;
  const void *A, *Kh, *S, *dS;
  void *dq, *dk_out, *dv_out;
  const float *tot, *cT;   // chunk totals of D, rowsum(dS_T * S_T) or NULL
  void* dla;               // dlog_alpha, written directly
  const void* la;          // the gate operand: g is rebuilt from it, and the gate
                           // front-end's chain rule applied
  GateFn gate;
  float* dla_part;         // scalar gates: fp32 sums of the per-(t, d) gradient over each
                           // 64-wide d block, [BH][T][dk/64], instead of dla
  bool gscalar;            // la holds one gate per token: [BH][T]
  bool s_frag;             // S and dS in MFMA fragment order, as the scans wrote them
};
// The backward chunk work (launch_bwd_chunk, after the chunk totals are formed): dq / dk /
// dlog_alpha workgroups and dv workgroups (bf16 with chunk 64 or 128, fp32 with chunk 64),
// interleaved in one launch at chunk 64, a launch each at chunk 128.
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

// The number of gate elements (n of them, fp32 or bf16) that break the layer's
// precondition (log_alpha finite and <= 0; with `logits`, finite) into *cnt (device).
hipError_t launch_count_bad_gates(int dtype, const void* x, long n, int logits,
                                  unsigned long long* cnt, hipStream_t s);

// Gated Slot Attention (fp32): w = 1 - exp(log_alpha); the first (slot-gated) pass's chunk
// output and chunk backward; row softmax and its backward; the gate-gradient combination.
// Layouts: q, k [BH][T][dk]; w, g2 (chunk-local cumsum * log2 e), s, ds, dw, Dloc [BH][T][m];
// S1, dS1 [BH][N][m][dk] (dS1 of chunk i = the gradient flowing in from chunk i + 1);
// tot [BH][N][m].
hipError_t launch_gsa_w(const float* la, float* w, long n, hipStream_t s);
hipError_t launch_vg_out(const float* q, const float* k, const float* w, const float* g2,
                         const float* S1, float* s_out, int BH, int T, int dk, int m,
                         hipStream_t s);
// (dq, dk: fp32, or bf16 with out_bf16)
hipError_t launch_vg_bwd(const float* q, const float* k, const float* w, const float* g2,
                         const float* ds, const float* s_in, const float* S1, const float* dS1,
                         void* dq, void* dk, int out_bf16, float* dw, float* Dloc, float* tot,
                         int BH, int T, int dkh, int m, hipStream_t s);
hipError_t launch_softmax_rows(const float* x, float* p, long nrows, int m, hipStream_t s);
hipError_t launch_softmax_bwd(const float* p, const float* dp, float* ds, long nrows, int m,
                              hipStream_t s);
hipError_t launch_gsa_combine(const float* la, const float* dla1, const float* dla2,
                              const float* dw1, const float* dw2, float* dla, long n,
                              hipStream_t s);
// bf16 Gated Slot Attention (bf16 pointers as void*): the combination with the second
// pass's bf16 gradients dla2, dw2 and a bf16 dla; element conversions bf16 <-> fp32.
hipError_t launch_gsa_combine_bf16(const float* la, const float* dla1, const void* dla2,
                                   const float* dw1, const void* dw2, void* dla, long n,
                                   hipStream_t s);
hipError_t launch_cast_bf16_f32(const void* x, float* y, long n, hipStream_t s);
hipError_t launch_cast_f32_bf16(const float* x, void* y, long n, hipStream_t s);

}  // namespace gla
