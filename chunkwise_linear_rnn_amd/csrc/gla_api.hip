// C ABI of libgla_mi355x.so: argument validation, workspace planning and launch
// sequencing on the caller's stream.  See include/gla.h for the contract.
//
// Pipelines (page "Gated Linear Attention Transformers with Hardware-Efficient
// Training", atlas.scime.ai summary, section Approach):
//   forward, materialized states:  gate cumsum -> intra-chunk (A, Qh, Kh^T, e^gamma)
//                                  -> state scan (writes every S_[i]) -> output
//   forward, recomputed states:    intra-chunk (cumsum fused) -> fused state+output
//   backward:                      intra-chunk (cumsum fused, writes g) -> state scan (S_[i]) ->
//                                  reverse state scan (dS_[i+1], dS0); both scans also
//                                  form the chunk totals of q*dq - k*dk from their fp32
//                                  states -> chunk backward (dq, dk, dv, chunk-local D
//                                  suffix sums) -> closed-form gate gradient scan
#include <cstdlib>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <initializer_list>

#include "gla.h"
#include "gla_internal.h"

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Dims {
  long B, H, T, dk, dv, C, N, BH;
  int dtype;
  size_t esz;   // bytes per element of the [B,H,T,*] tensors and of MFMA operands
};

Dims dims_of(const gla_desc_t* d) {
  Dims x;
  x.B = d->B; x.H = d->H; x.T = d->T; x.dk = d->dk; x.dv = d->dv; x.C = d->chunk;
  x.N = x.T > 0 ? (x.T + x.C - 1) / x.C : 0;
  x.BH = x.B * x.H;
  x.dtype = d->dtype;
  x.esz = d->dtype == GLA_F32 ? 4 : 2;
  return x;
}

// Workspace carving.  Every region is 256-byte aligned.
struct Plan {
  size_t A = 0, Qh = 0, QhT = 0, Kh = 0, KhT = 0, eg = 0, st = 0, dst = 0, ST = 0,
         cT = 0, crossF = 0, crossR = 0, carry = 0, smid = 0, segdec = 0, dpart = 0,
         sslots = 0, sdec = 0, dbg = 0, total = 0;
};

// The materialized forward's state scan (every chunk state written, [v][k]) for a shape.
gla::ScanArgs mat_scan_shape(const Dims& x) {
  gla::ScanArgs a{};
  a.dtype = x.dtype; a.C = (int)x.C; a.BH = (int)x.BH; a.T = (int)x.T; a.dk = (int)x.dk;
  a.dv = (int)x.dv; a.N = (int)x.N; a.reverse = false; a.store = 2;
  return a;
}

// Passes 3 (forward that saves the intra-chunk operands for the backward) and 4 (backward
// that reads them): the forward / backward plan without those regions, which live in the
// caller's saved buffer (saved_plan).
Plan plan_of(const gla_desc_t* d, int pass) {
  const Dims x = dims_of(d);
  Plan p;
  const bool saved = pass == GLA_PASS_FWD_SAVE || pass == GLA_PASS_BWD_SAVED;
  if (pass == GLA_PASS_FWD_SAVE) pass = GLA_PASS_FWD;
  if (pass == GLA_PASS_BWD_SAVED) pass = GLA_PASS_BWD;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  const size_t rowsP = (size_t)x.BH * x.N * x.C;          // padded token rows
  const size_t AB = (size_t)x.BH * x.N * x.C * x.C * x.esz;
  const size_t opB = rowsP * x.dk * x.esz;
  const size_t egB = (size_t)x.BH * x.N * x.dk * 4;
  const size_t stB = (size_t)x.BH * x.N * x.dk * x.dv * x.esz;
  const bool mat = d->state_mode == GLA_STATES_MATERIALIZED;
  if (pass == GLA_PASS_FWD) {
    // a segmented materialized scan: the states at the segment starts and decay products
    const int P = mat ? gla::scan_segments(mat_scan_shape(x)) : 1;
    if (P > 1) p.sslots = take((size_t)(P - 1) * x.BH * x.dk * x.dv * 4);
    if (P > 2) p.sdec = take((size_t)(P - 1) * x.BH * x.dk * 4);
    if (!saved) {
      p.A = take(AB);
      p.Qh = take(opB);
      p.KhT = take(opB);
      p.eg = take(egB);
    }
    if (mat) p.st = take(stB);
    const int nseg = mat ? 1 : gla::fused_segments(x.dtype, (int)x.C, (int)x.N, (int)x.BH, (int)x.dv);
    if (nseg > 1) p.smid = take((size_t)(nseg - 1) * x.BH * x.dk * x.dv * 4);
    if (nseg > 2) p.segdec = take((size_t)(nseg - 1) * x.BH * x.dk * 4);
  } else if (pass == GLA_PASS_BWD) {
    // the scans' transposed operands are kept in fp32 (split into two bf16 halves)
    const size_t op32 = rowsP * x.dk * 4;
    const size_t crossB = (size_t)x.BH * x.N * (x.dv / 64) * x.dk * 4;
    // (the chunk kernel rebuilds g from the gates: no g in the workspace)
    if (!saved) {
      p.A = take(AB);
      p.QhT = take(op32);
      p.Kh = take(opB);
      p.KhT = take(op32);
      p.eg = take(egB);
    }
    p.st = take(stB);
    p.dst = take(stB);
    p.ST = take((size_t)x.BH * x.dk * x.dv * 4);
    p.cT = take((size_t)x.BH * x.dk * 4);
    p.crossF = take(crossB);
    p.crossR = take(crossB);
    p.carry = take(egB);
    if (d->gate_shape == GLA_GATE_SCALAR)
      p.dpart = take((size_t)x.BH * x.T * (x.dk / 64) * 4);
    // the two scans in segments (few workgroups): both scans' segment start states and
    // decay products
    const int P = gla::scan2_segments(x.dtype, (int)x.C, (int)x.BH, (int)x.dk, (int)x.dv,
                                      (int)x.N);
    if (P > 1) p.sslots = take((size_t)2 * (P - 1) * x.BH * x.dk * x.dv * 4);
    if (P > 2) p.sdec = take((size_t)2 * (P - 1) * x.BH * x.dk * 4);
  } else {
    p.KhT = take(opB);
    p.eg = take(egB);
  }
  // the gate check's counter (GLA_DEBUG_CHECKS)
  if ((pass == GLA_PASS_FWD || pass == GLA_PASS_BWD) && x.BH * x.T > 0) p.dbg = take(256);
  p.total = off;
  return p;
}

// The saved buffer of a forward that keeps its intra-chunk operands for the backward: the
// outputs of the backward's intra-chunk kernel (A, Qh^T and Kh^T as the scans read them,
// Kh, e^gamma) plus the token-major Qh the fused forward reads.  Every region 256-byte
// aligned.
Plan saved_plan(const gla_desc_t* d) {
  const Dims x = dims_of(d);
  Plan p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  const size_t rowsP = (size_t)x.BH * x.N * x.C;
  const size_t opB = rowsP * x.dk * x.esz, op32 = rowsP * x.dk * 4;
  p.A = take((size_t)x.BH * x.N * x.C * x.C * x.esz);
  p.Qh = take(opB);
  p.QhT = take(op32);
  p.Kh = take(opB);
  p.KhT = take(op32);
  p.eg = take((size_t)x.BH * x.N * x.dk * 4);
  p.total = off;
  return p;
}

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

gla_status_t dev(hipError_t e) { return e == hipSuccess ? GLA_OK : GLA_ERR_DEVICE; }

// GLA_DEBUG_CHECKS=1 in the environment (read once, at the first call): the layer's
// forward and backward first count the gate elements that break its precondition and
// refuse the call (GLA_ERR_INVALID_ARG) if there are any, before touching an output.
bool debug_checks() {
  static const bool on = [] {
    const char* e = std::getenv("GLA_DEBUG_CHECKS");
    return e != nullptr && e[0] == '1' && e[1] == 0;
  }();
  return on;
}

// Elements of the gate operand of `d` that break the precondition (synchronizes `s`).
gla_status_t count_bad_gates(const gla_desc_t* d, const void* la, void* counter, hipStream_t s,
                             long long* n_bad) {
  const long n = (long)d->B * d->H * d->T * (d->gate_shape == GLA_GATE_SCALAR ? 1 : d->dk);
  unsigned long long* cnt = (unsigned long long*)counter;
  gla_status_t rs = dev(gla::launch_count_bad_gates(d->dtype, la, n, d->gate == GLA_GATE_LOGITS,
                                                     cnt, s));
  if (rs != GLA_OK) return rs;
  unsigned long long h = 0;
  if ((rs = dev(hipMemcpyAsync(&h, cnt, sizeof(h), hipMemcpyDeviceToHost, s))) != GLA_OK) return rs;
  if ((rs = dev(hipStreamSynchronize(s))) != GLA_OK) return rs;
  *n_bad = (long long)h;
  return GLA_OK;
}

bool gate_ok(const gla_desc_t* d) {
  if (d->gate_shape != GLA_GATE_PER_KEY && d->gate_shape != GLA_GATE_SCALAR) return false;
  if (d->gate == GLA_GATE_LOG_ALPHA) return true;
  return d->gate == GLA_GATE_LOGITS && d->gate_tau > 0.f && d->gate_tau <= 3.0e38f;
}
bool scalar_gate(const gla_desc_t* d) { return d->gate_shape == GLA_GATE_SCALAR; }
gla::GateFn gate_of(const gla_desc_t* d) {
  gla::GateFn g;
  g.on = d->gate == GLA_GATE_LOGITS ? 1 : 0;
  g.inv_tau = g.on ? 1.f / d->gate_tau : 1.f;
  return g;
}

// Zero or copy a [BH,dk,dv] fp32 state with a kernel (safe under stream capture).
__global__ void k_state_copy(const float* __restrict__ src, float* __restrict__ dst, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    dst[i] = src ? src[i] : 0.f;
}
gla_status_t state_copy(const float* src, float* dst, long n, hipStream_t s) {
  if (!dst || n == 0) return GLA_OK;
  const long blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(k_state_copy, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n);
  return dev(hipGetLastError());
}

// Records caller-provided events between kernel launches (profiling); inert when the
// caller passes none, and a NULL entry skips its boundary.
struct Tracer {
  void** ev;
  int n;
  hipStream_t s;
  int k = 0;
  gla_status_t mark() {
    if (!ev) return GLA_OK;
    if (k >= n) return GLA_ERR_INVALID_ARG;
    void* e = ev[k++];
    return e ? dev(hipEventRecord((hipEvent_t)e, s)) : GLA_OK;
  }
};

// Stage names of each pipeline, in launch order.
const char* const kFwdMat[] = {"intra", "state_scan", "output"};
const char* const kFwdRec[] = {"intra", "seg_state", "fwd_fused"};
const char* const kBwd[] = {"intra", "state_scans", "state_dot", "gate_tot", "bwd_dqk_dv"};
const char* const kBwdSaved[] = {"state_scans", "state_dot", "gate_tot", "bwd_dqk_dv"};

int stage_list(const gla_desc_t* d, int pass, int with_dST, const char** out, int max) {
  const char* const* src;
  int n;
  const bool bwd = pass == GLA_PASS_BWD || pass == GLA_PASS_BWD_SAVED;
  int dot = 2;   // position of state_dot
  if (pass == GLA_PASS_FWD || pass == GLA_PASS_FWD_SAVE) {
    if (d->state_mode == GLA_STATES_MATERIALIZED) { src = kFwdMat; n = 3; }
    else { src = kFwdRec; n = 3; }
  } else if (pass == GLA_PASS_BWD_SAVED) {
    src = kBwdSaved; n = 4; dot = 1;
  } else {
    src = kBwd; n = 5;
  }
  int m = 0;
  for (int j = 0; j < n; ++j) {
    if (bwd && j == dot && !with_dST) continue;
    if (out && m < max) out[m] = src[j];
    ++m;
  }
  if (bwd && d->gate_shape == GLA_GATE_SCALAR) {   // the sum over d
    if (out && m < max) out[m] = "gate_reduce";
    ++m;
  }
  return m;
}

}  // namespace

extern "C" {

int32_t gla_trace_stages(const gla_desc_t* d, int32_t pass, int32_t with_dS_T, const char** names,
                         int32_t max_names) {
  if (!d || (pass != GLA_PASS_FWD && pass != GLA_PASS_BWD && pass != GLA_PASS_FWD_SAVE &&
             pass != GLA_PASS_BWD_SAVED))
    return -1;
  return stage_list(d, pass, with_dS_T, names, max_names);
}

const char* gla_status_string(gla_status_t s) {
  switch (s) {
    case GLA_OK: return "GLA_OK";
    case GLA_ERR_INVALID_ARG: return "GLA_ERR_INVALID_ARG";
    case GLA_ERR_UNSUPPORTED: return "GLA_ERR_UNSUPPORTED";
    case GLA_ERR_WORKSPACE: return "GLA_ERR_WORKSPACE";
    case GLA_ERR_DEVICE: return "GLA_ERR_DEVICE";
  }
  return "GLA_ERR_UNKNOWN";
}

int32_t gla_version(void) { return 10000 * 0 + 100 * 2 + 0; }

gla_status_t gla_validate(const gla_desc_t* d, int32_t pass) {
  if (!d) return GLA_ERR_INVALID_ARG;
  if (pass < 0 || pass > GLA_PASS_BWD_SAVED) return GLA_ERR_INVALID_ARG;
  if (d->B < 0 || d->H < 0 || d->T < 0 || d->dk < 0 || d->dv < 0) return GLA_ERR_INVALID_ARG;
  if (d->chunk < 1 || d->subchunk < 1 || d->chunk % d->subchunk != 0) return GLA_ERR_INVALID_ARG;
  if (d->dtype != GLA_F32 && d->dtype != GLA_BF16) return GLA_ERR_INVALID_ARG;
  if (d->state_mode != GLA_STATES_MATERIALIZED && d->state_mode != GLA_STATES_RECOMPUTE)
    return GLA_ERR_INVALID_ARG;
  if (!gate_ok(d)) return GLA_ERR_INVALID_ARG;
  if (d->diag != GLA_DIAG_F32 && d->diag != GLA_DIAG_BF16) return GLA_ERR_INVALID_ARG;
  if (d->chunk != 64 && d->chunk != 128) return GLA_ERR_UNSUPPORTED;
  if (d->subchunk != 16) return GLA_ERR_UNSUPPORTED;
  if (d->dtype == GLA_F32 && d->chunk != 64) return GLA_ERR_UNSUPPORTED;
  if (d->dk < 64 || d->dk > 256 || d->dk % 64 != 0) return GLA_ERR_UNSUPPORTED;
  if (d->dv < 64 || d->dv > 1024 || d->dv % 64 != 0) return GLA_ERR_UNSUPPORTED;
  const long long bh = (long long)d->B * d->H;
  if (bh > 65535) return GLA_ERR_UNSUPPORTED;
  if (bh * (long long)d->T > (1LL << 31) - 1) return GLA_ERR_UNSUPPORTED;
  if (((long long)d->T + d->chunk - 1) / d->chunk > 65535) return GLA_ERR_UNSUPPORTED;
  // the forward that saves for the backward walks the recomputed states
  if (pass == GLA_PASS_FWD_SAVE && d->state_mode != GLA_STATES_RECOMPUTE) return GLA_ERR_UNSUPPORTED;
  return GLA_OK;
}

gla_status_t gla_saved_bytes(const gla_desc_t* d, size_t* bytes) {
  if (!bytes) return GLA_ERR_INVALID_ARG;
  const gla_status_t st = gla_validate(d, GLA_PASS_FWD_SAVE);
  if (st != GLA_OK) return st;
  *bytes = saved_plan(d).total;
  return GLA_OK;
}

gla_status_t gla_workspace_bytes(const gla_desc_t* d, int32_t pass, size_t* bytes) {
  if (!bytes) return GLA_ERR_INVALID_ARG;
  const gla_status_t st = gla_validate(d, pass);
  if (st != GLA_OK) return st;
  *bytes = plan_of(d, pass).total;
  return GLA_OK;
}

gla_status_t gla_check_gates(const gla_desc_t* d, const void* log_alpha, void* ws,
                             size_t ws_bytes, int64_t* n_bad, void* stream) {
  const gla_status_t st = gla_validate(d, GLA_PASS_FWD);
  if (st != GLA_OK) return st;
  if (!n_bad) return GLA_ERR_INVALID_ARG;
  *n_bad = 0;
  if ((long long)d->B * d->H * d->T == 0) return GLA_OK;
  if (!log_alpha || !aligned16(log_alpha) || !aligned16(ws)) return GLA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < 8) return GLA_ERR_WORKSPACE;
  long long bad = 0;
  const gla_status_t rs = count_bad_gates(d, log_alpha, ws, (hipStream_t)stream, &bad);
  if (rs == GLA_OK) *n_bad = bad;
  return rs;
}

gla_status_t gla_gate_cumsum(const gla_desc_t* d, const void* log_alpha, float* g, float* gamma,
                             void* stream) {
  const gla_status_t st = gla_validate(d, GLA_PASS_FWD);
  if (st != GLA_OK) return st;
  const Dims x = dims_of(d);
  if (x.BH * x.T == 0) return GLA_OK;
  if (!log_alpha || (!g && !gamma)) return GLA_ERR_INVALID_ARG;
  if (!aligned16(log_alpha) || !aligned16(g) || !aligned16(gamma)) return GLA_ERR_INVALID_ARG;
  return dev(gla::launch_gate_cumsum(x.dtype, log_alpha, gate_of(d), scalar_gate(d), g, gamma,
                                     (int)x.BH, (int)x.T, (int)x.dk, (int)x.C,
                                     (hipStream_t)stream));
}

gla_status_t gla_chunk_states(const gla_desc_t* d, const void* k, const void* v,
                              const void* log_alpha, const float* S0, float* states, float* S_T,
                              void* ws, size_t ws_bytes, void* stream) {
  const gla_status_t st = gla_validate(d, 2);
  if (st != GLA_OK) return st;
  const Dims x = dims_of(d);
  hipStream_t s = (hipStream_t)stream;
  if (x.BH == 0) return GLA_OK;
  if (x.T == 0) return state_copy(S0, S_T, x.BH * x.dk * x.dv, s);
  if (!k || !v || !log_alpha || !states) return GLA_ERR_INVALID_ARG;
  for (const void* p : std::initializer_list<const void*>{k, v, log_alpha, S0, states, S_T, ws})
    if (!aligned16(p)) return GLA_ERR_INVALID_ARG;
  const Plan p = plan_of(d, 2);
  if (!ws || ws_bytes < p.total) return GLA_ERR_WORKSPACE;
  char* w = (char*)ws;
  gla::IntraArgs ia{};
  ia.dtype = x.dtype; ia.C = (int)x.C; ia.BH = (int)x.BH; ia.T = (int)x.T; ia.dk = (int)x.dk;
  ia.N = (int)x.N; ia.want_A = false; ia.q = k; ia.k = k; ia.la = log_alpha; ia.gate = gate_of(d);
  ia.gscalar = scalar_gate(d);
  ia.KhT = w + p.KhT; ia.eg = (float*)(w + p.eg);
  gla_status_t rs = dev(gla::launch_intra(ia, s));
  if (rs != GLA_OK) return rs;
  gla::ScanArgs sa{};
  sa.dtype = x.dtype; sa.C = (int)x.C; sa.BH = (int)x.BH; sa.T = (int)x.T; sa.dk = (int)x.dk;
  sa.dv = (int)x.dv; sa.N = (int)x.N; sa.reverse = false; sa.store = 3;
  sa.XT = w + p.KhT; sa.Y = v; sa.eg = (const float*)(w + p.eg); sa.S_in = S0;
  sa.states = states; sa.S_out = S_T;
  return dev(gla::launch_state_scan(sa, s));
}

// The layer forward; save: the intra-chunk operands go to `saved` in the backward's layout
// (saved_plan) for a later backward from them, and the rest of the forward reads them there.
static gla_status_t fwd_run(const gla_desc_t* d, const void* q, const void* k, const void* v,
                            const void* log_alpha, const float* S0, void* o, float* S_T,
                            bool save, void* saved, size_t saved_bytes, void* ws,
                            size_t ws_bytes, void* stream, void** events, int32_t n_events) {
  const int pass = save ? GLA_PASS_FWD_SAVE : GLA_PASS_FWD;
  const gla_status_t st = gla_validate(d, pass);
  if (st != GLA_OK) return st;
  if (events && n_events < stage_list(d, pass, 0, nullptr, 0) + 1)
    return GLA_ERR_INVALID_ARG;
  Tracer tr{events, n_events, (hipStream_t)stream};
  const Dims x = dims_of(d);
  hipStream_t s = (hipStream_t)stream;
  if (x.BH == 0) return GLA_OK;
  if (x.T == 0) return state_copy(S0, S_T, x.BH * x.dk * x.dv, s);
  if (!q || !k || !v || !log_alpha || !o) return GLA_ERR_INVALID_ARG;
  for (const void* p : std::initializer_list<const void*>{q, k, v, log_alpha, S0, o, S_T, ws,
                                                          saved})
    if (!aligned16(p)) return GLA_ERR_INVALID_ARG;
  const Plan p = plan_of(d, pass);
  if (!ws || ws_bytes < p.total) return GLA_ERR_WORKSPACE;
  const Plan sp = save ? saved_plan(d) : Plan{};
  if (save && (!saved || saved_bytes < sp.total)) return GLA_ERR_WORKSPACE;
  char* w = (char*)ws;
  // where the intra-chunk operands live: the workspace, or the saved buffer
  char* ob = save ? (char*)saved : w;
  const Plan& op = save ? sp : p;
  const bool split = save && x.dtype == GLA_BF16;   // bf16 Kh^T with its remainder
  const bool mat = d->state_mode == GLA_STATES_MATERIALIZED;
  gla_status_t rs = GLA_OK;
  if (debug_checks()) {
    long long bad = 0;
    if ((rs = count_bad_gates(d, log_alpha, w + p.dbg, s, &bad)) != GLA_OK) return rs;
    if (bad) return GLA_ERR_INVALID_ARG;
  }
  gla::IntraArgs ia{};
  ia.dtype = x.dtype; ia.C = (int)x.C; ia.BH = (int)x.BH; ia.T = (int)x.T; ia.dk = (int)x.dk;
  ia.N = (int)x.N; ia.want_A = true; ia.q = q; ia.k = k; ia.la = log_alpha; ia.gate = gate_of(d);
  ia.gscalar = scalar_gate(d); ia.diag_bf16 = d->diag == GLA_DIAG_BF16;
  ia.A = ob + op.A; ia.Qh = ob + op.Qh; ia.KhT = ob + op.KhT; ia.eg = (float*)(ob + op.eg);
  if (save) {   // also the backward's operands, the transposed ones as its scans read them
    ia.xt_f32 = x.dtype == GLA_BF16;
    ia.QhT = ob + op.QhT; ia.Kh = ob + op.Kh;
  }
  if ((rs = tr.mark()) != GLA_OK) return rs;
  rs = dev(gla::launch_intra(ia, s));
  if (rs != GLA_OK) return rs;
  if (mat) {
    gla::ScanArgs sa = mat_scan_shape(x);
    sa.XT = w + p.KhT; sa.Y = v; sa.eg = (const float*)(w + p.eg); sa.S_in = S0;
    sa.states = w + p.st; sa.S_out = S_T;
    if ((rs = tr.mark()) != GLA_OK) return rs;
    // long sequences with few heads: the scan in parallel segments from their start states
    const int P = gla::scan_segments(sa);
    rs = dev(gla::launch_state_scan_seg(sa, P > 1 ? (float*)(w + p.sslots) : nullptr,
                                        P > 2 ? (float*)(w + p.sdec) : nullptr, s));
    if (rs != GLA_OK) return rs;
    gla::OutArgs oa{};
    oa.dtype = x.dtype; oa.C = (int)x.C; oa.BH = (int)x.BH; oa.T = (int)x.T; oa.dk = (int)x.dk;
    oa.dv = (int)x.dv; oa.N = (int)x.N; oa.Qh = w + p.Qh; oa.A = w + p.A; oa.STt = w + p.st;
    oa.v = v; oa.o = o;
    if ((rs = tr.mark()) != GLA_OK) return rs;
    if ((rs = dev(gla::launch_output(oa, s))) != GLA_OK) return rs;
    return tr.mark();
  }
  gla::FusedArgs fa{};
  fa.dtype = x.dtype; fa.C = (int)x.C; fa.BH = (int)x.BH; fa.T = (int)x.T; fa.dk = (int)x.dk;
  fa.dv = (int)x.dv; fa.N = (int)x.N; fa.Qh = ob + op.Qh; fa.KhT = ob + op.KhT;
  fa.A = ob + op.A; fa.kht_split = split;
  fa.v = v; fa.eg = (const float*)(ob + op.eg); fa.S0 = S0; fa.o = o; fa.S_T = S_T;
  fa.nseg = gla::fused_segments(x.dtype, (int)x.C, (int)x.N, (int)x.BH, (int)x.dv);
  // with a split, the states at the segment starts come first (no per-chunk states
  // written): two segments, a state scan over the first half; more, every segment but the
  // last scanned from zero in one launch (the first from S0), then chained
  if ((rs = tr.mark()) != GLA_OK) return rs;
  if (fa.nseg > 1) {
    gla::ScanArgs sa{};
    sa.dtype = x.dtype; sa.C = (int)x.C; sa.BH = (int)x.BH; sa.T = (int)x.T; sa.dk = (int)x.dk;
    sa.dv = (int)x.dv; sa.N = (int)x.N; sa.reverse = false; sa.store = 0;
    if (fa.nseg == 2) {
      sa.nsteps = (int)x.N / 2;
    } else {
      sa.nseg = fa.nseg - 1; sa.seg_p = fa.nseg; sa.seg_decay = (float*)(w + p.segdec);
    }
    sa.XT = ob + op.KhT; sa.Y = v; sa.eg = (const float*)(ob + op.eg); sa.S_in = S0;
    // the split operand's high part alone: the bf16 rounding the plain forward stores, so
    // that the segment start states, and o, are those of gla_chunk_fwd
    sa.xt_hi = split;
    sa.S_out = (float*)(w + p.smid);
    if ((rs = dev(gla::launch_state_scan(sa, s))) != GLA_OK) return rs;
    if ((rs = dev(gla::launch_seg_combine((float*)(w + p.smid), (const float*)(w + p.segdec),
                                          (int)x.BH, (int)x.dk, (int)x.dv, fa.nseg, s))) != GLA_OK)
      return rs;
    fa.S_mid = (const float*)(w + p.smid);
  }
  if ((rs = tr.mark()) != GLA_OK) return rs;
  if ((rs = dev(gla::launch_fwd_fused(fa, s))) != GLA_OK) return rs;
  return tr.mark();
}

gla_status_t gla_chunk_fwd_traced(const gla_desc_t* d, const void* q, const void* k,
                                  const void* v, const void* log_alpha, const float* S0, void* o,
                                  float* S_T, void* ws, size_t ws_bytes, void* stream,
                                  void** events, int32_t n_events) {
  return fwd_run(d, q, k, v, log_alpha, S0, o, S_T, false, nullptr, 0, ws, ws_bytes, stream,
                 events, n_events);
}

gla_status_t gla_chunk_fwd(const gla_desc_t* d, const void* q, const void* k, const void* v,
                           const void* log_alpha, const float* S0, void* o, float* S_T, void* ws,
                           size_t ws_bytes, void* stream) {
  return fwd_run(d, q, k, v, log_alpha, S0, o, S_T, false, nullptr, 0, ws, ws_bytes, stream,
                 nullptr, 0);
}

gla_status_t gla_chunk_fwd_save_traced(const gla_desc_t* d, const void* q, const void* k,
                                       const void* v, const void* log_alpha, const float* S0,
                                       void* o, float* S_T, void* saved, size_t saved_bytes,
                                       void* ws, size_t ws_bytes, void* stream, void** events,
                                       int32_t n_events) {
  return fwd_run(d, q, k, v, log_alpha, S0, o, S_T, true, saved, saved_bytes, ws, ws_bytes,
                 stream, events, n_events);
}

gla_status_t gla_chunk_fwd_save(const gla_desc_t* d, const void* q, const void* k, const void* v,
                                const void* log_alpha, const float* S0, void* o, float* S_T,
                                void* saved, size_t saved_bytes, void* ws, size_t ws_bytes,
                                void* stream) {
  return fwd_run(d, q, k, v, log_alpha, S0, o, S_T, true, saved, saved_bytes, ws, ws_bytes,
                 stream, nullptr, 0);
}

// The layer backward; from_saved: the intra-chunk operands come from `saved` (written by a
// forward that saved them for the same inputs) and the intra-chunk kernel does not run.
static gla_status_t bwd_run(const gla_desc_t* d, const void* q, const void* k, const void* v,
                            const void* log_alpha, const float* S0, const void* dO,
                            const float* dS_T, void* dq, void* dk, void* dv, void* dlog_alpha,
                            float* dS0, bool from_saved, const void* saved, size_t saved_bytes,
                            void* ws, size_t ws_bytes, void* stream, void** events,
                            int32_t n_events) {
  const int pass = from_saved ? GLA_PASS_BWD_SAVED : GLA_PASS_BWD;
  const gla_status_t st = gla_validate(d, pass);
  if (st != GLA_OK) return st;
  if (events && n_events < stage_list(d, pass, dS_T != nullptr, nullptr, 0) + 1)
    return GLA_ERR_INVALID_ARG;
  Tracer tr{events, n_events, (hipStream_t)stream};
  const Dims x = dims_of(d);
  hipStream_t s = (hipStream_t)stream;
  if (x.BH == 0) return GLA_OK;
  if (x.T == 0) return state_copy(dS_T, dS0, x.BH * x.dk * x.dv, s);
  if (!q || !k || !v || !log_alpha || !dO || !dq || !dk || !dv || !dlog_alpha)
    return GLA_ERR_INVALID_ARG;
  for (const void* p : std::initializer_list<const void*>{q, k, v, log_alpha, S0, dO, dS_T, dq,
                                                          dk, dv, dlog_alpha, dS0, ws, saved})
    if (!aligned16(p)) return GLA_ERR_INVALID_ARG;
  const Plan p = plan_of(d, pass);
  if (!ws || ws_bytes < p.total) return GLA_ERR_WORKSPACE;
  const Plan sp = from_saved ? saved_plan(d) : Plan{};
  if (from_saved && (!saved || saved_bytes < sp.total)) return GLA_ERR_WORKSPACE;
  char* w = (char*)ws;
  // where the intra-chunk operands live: the workspace, or the saved buffer
  char* ob = from_saved ? (char*)saved : w;
  const Plan& op = from_saved ? sp : p;
  const int C = (int)x.C, BH = (int)x.BH, T = (int)x.T, DK = (int)x.dk, DV = (int)x.dv,
            N = (int)x.N;
  gla_status_t rs = GLA_OK;
  if (debug_checks()) {
    long long bad = 0;
    if ((rs = count_bad_gates(d, log_alpha, w + p.dbg, s, &bad)) != GLA_OK) return rs;
    if (bad) return GLA_ERR_INVALID_ARG;
  }
  gla::IntraArgs ia{};
  ia.dtype = x.dtype; ia.C = C; ia.BH = BH; ia.T = T; ia.dk = DK; ia.N = N; ia.want_A = true;
  ia.xt_f32 = x.dtype == GLA_BF16;
  ia.q = q; ia.k = k; ia.la = log_alpha;
  ia.g2_out = nullptr;
  ia.gate = gate_of(d); ia.gscalar = scalar_gate(d); ia.diag_bf16 = d->diag == GLA_DIAG_BF16;
  ia.A = ob + op.A; ia.QhT = ob + op.QhT; ia.Kh = ob + op.Kh; ia.KhT = ob + op.KhT;
  ia.eg = (float*)(ob + op.eg);
  if (!from_saved) {
    if ((rs = tr.mark()) != GLA_OK) return rs;
    rs = dev(gla::launch_intra(ia, s));
    if (rs != GLA_OK) return rs;
  }
  // forward scan: chunk-start states S_[i]; cross term rowsum(S_[i] * Qh_i^T dO_i)
  gla::ScanArgs sa{};
  sa.dtype = x.dtype; sa.C = C; sa.BH = BH; sa.T = T; sa.dk = DK; sa.dv = DV; sa.N = N;
  sa.reverse = false; sa.xt_f32 = ia.xt_f32; sa.store = 1;
  sa.XT = ob + op.KhT; sa.Y = v; sa.X2T = ob + op.QhT; sa.Y2 = dO; sa.cross = (float*)(w + p.crossF);
  sa.eg = (const float*)(ob + op.eg); sa.S_in = S0; sa.states = w + p.st;
  sa.S_out = dS_T ? (float*)(w + p.ST) : nullptr;
  // reverse scan: dS_[i+1]; cross term rowsum(dS_[i+1] * Kh_i^T V_i)
  gla::ScanArgs ra = sa;
  ra.reverse = true; ra.XT = ob + op.QhT; ra.Y = dO; ra.X2T = ob + op.KhT; ra.Y2 = v;
  ra.cross = (float*)(w + p.crossR); ra.S_in = dS_T; ra.states = w + p.dst; ra.S_out = dS0;
  // S and dS go to the backward chunk kernel in MFMA fragment order when the scans run
  // 128-column tiles (bf16, chunk 64): its dq / dk workgroups load whole fragments, its dv
  // workgroups stage dS transposed from them
  sa.frag_states = gla::scan_tile_v(sa) == 128;
  ra.frag_states = sa.frag_states;
  // both scans in one launch (in sequence segments when few workgroups would walk the
  // whole sequence)
  if ((rs = tr.mark()) != GLA_OK) return rs;
  const int P2 = gla::scan2_segments(x.dtype, C, BH, DK, DV, N);
  rs = dev(gla::launch_state_scan2_seg(sa, ra, P2 > 1 ? (float*)(w + p.sslots) : nullptr,
                                       P2 > 2 ? (float*)(w + p.sdec) : nullptr, s));
  if (rs != GLA_OK) return rs;
  if (dS_T) {
    if ((rs = tr.mark()) != GLA_OK) return rs;
    rs = dev(gla::launch_state_dot(dS_T, (const float*)(w + p.ST), (float*)(w + p.cT), BH, DK,
                                   DV, s));
    if (rs != GLA_OK) return rs;
  }
  gla::BwdArgs ba{};
  ba.dtype = x.dtype; ba.C = C; ba.BH = BH; ba.T = T; ba.dk = DK; ba.dv = DV; ba.N = N;
  ba.q = q; ba.k = k; ba.v = v; ba.dO = dO;
  ba.gscalar = scalar_gate(d);
  ba.s_frag = sa.frag_states;
  ba.A = ob + op.A; ba.Kh = ob + op.Kh; ba.S = w + p.st; ba.dS = w + p.dst;
  ba.dq = dq; ba.dk_out = dk; ba.dv_out = dv;
  ba.tot = (const float*)(w + p.carry); ba.cT = dS_T ? (const float*)(w + p.cT) : nullptr;
  ba.dla = dlog_alpha; ba.la = log_alpha; ba.gate = gate_of(d);
  // scalar gates: the per-key gradient is summed over the key dimension afterwards, and
  // the front-end slope (one per token) applied there (the chunk kernel writes partial
  // sums without it; it still takes the gate function, to rebuild g from the gates)
  const bool sg = scalar_gate(d);
  if (sg) ba.dla_part = p.dpart ? (float*)(w + p.dpart) : nullptr;
  auto reduce = [&](const float* part, int nparts) {
    return dev(gla::launch_gate_reduce(x.dtype, part, nparts, log_alpha, gate_of(d), dlog_alpha,
                                       (long)BH * T, s));
  };
  // chunk totals of D from the scans' cross terms
  auto totals = [&]() {
    return dev(gla::launch_gate_tot((const float*)(w + p.crossF), (const float*)(w + p.crossR),
                                    dS_T ? (const float*)(w + p.cT) : nullptr,
                                    (float*)(w + p.carry), BH, T, DK,
                                    DV / gla::scan_tile_v(sa), C, s));
  };
  // totals first: the chunk kernel's dq / dk workgroups finish the gate gradient
  if ((rs = tr.mark()) != GLA_OK) return rs;
  if ((rs = totals()) != GLA_OK) return rs;
  if ((rs = tr.mark()) != GLA_OK) return rs;
  if ((rs = dev(gla::launch_bwd_chunk(ba, s))) != GLA_OK) return rs;
  if (sg) {
    if ((rs = tr.mark()) != GLA_OK) return rs;
    if ((rs = reduce((const float*)(w + p.dpart), DK / 64)) != GLA_OK) return rs;
  }
  return tr.mark();
}

gla_status_t gla_chunk_bwd_traced(const gla_desc_t* d, const void* q, const void* k,
                                  const void* v, const void* log_alpha, const float* S0,
                                  const void* dO, const float* dS_T, void* dq, void* dk, void* dv,
                                  void* dlog_alpha, float* dS0, void* ws, size_t ws_bytes,
                                  void* stream, void** events, int32_t n_events) {
  return bwd_run(d, q, k, v, log_alpha, S0, dO, dS_T, dq, dk, dv, dlog_alpha, dS0, false,
                 nullptr, 0, ws, ws_bytes, stream, events, n_events);
}

gla_status_t gla_chunk_bwd(const gla_desc_t* d, const void* q, const void* k, const void* v,
                           const void* log_alpha, const float* S0, const void* dO,
                           const float* dS_T, void* dq, void* dk, void* dv, void* dlog_alpha,
                           float* dS0, void* ws, size_t ws_bytes, void* stream) {
  return bwd_run(d, q, k, v, log_alpha, S0, dO, dS_T, dq, dk, dv, dlog_alpha, dS0, false,
                 nullptr, 0, ws, ws_bytes, stream, nullptr, 0);
}

gla_status_t gla_chunk_bwd_saved_traced(const gla_desc_t* d, const void* q, const void* k,
                                        const void* v, const void* log_alpha, const float* S0,
                                        const void* dO, const float* dS_T, void* dq, void* dk,
                                        void* dv, void* dlog_alpha, float* dS0,
                                        const void* saved, size_t saved_bytes, void* ws,
                                        size_t ws_bytes, void* stream, void** events,
                                        int32_t n_events) {
  return bwd_run(d, q, k, v, log_alpha, S0, dO, dS_T, dq, dk, dv, dlog_alpha, dS0, true, saved,
                 saved_bytes, ws, ws_bytes, stream, events, n_events);
}

gla_status_t gla_chunk_bwd_saved(const gla_desc_t* d, const void* q, const void* k,
                                 const void* v, const void* log_alpha, const float* S0,
                                 const void* dO, const float* dS_T, void* dq, void* dk, void* dv,
                                 void* dlog_alpha, float* dS0, const void* saved,
                                 size_t saved_bytes, void* ws, size_t ws_bytes, void* stream) {
  return bwd_run(d, q, k, v, log_alpha, S0, dO, dS_T, dq, dk, dv, dlog_alpha, dS0, true, saved,
                 saved_bytes, ws, ws_bytes, stream, nullptr, 0);
}

gla_status_t gla_decode(const gla_desc_t* d, const void* q, const void* k, const void* v,
                        const void* log_alpha, float* S, void* o, void* stream) {
  if (!d) return GLA_ERR_INVALID_ARG;
  if (d->B < 0 || d->H < 0 || d->T < 0 || d->dk < 0 || d->dv < 0) return GLA_ERR_INVALID_ARG;
  if (d->dtype != GLA_F32 && d->dtype != GLA_BF16) return GLA_ERR_INVALID_ARG;
  if (!gate_ok(d)) return GLA_ERR_INVALID_ARG;
  if (d->dk < 32 || d->dk > 256 || d->dk % 32 != 0) return GLA_ERR_UNSUPPORTED;
  if (d->dv < 32 || d->dv > 1024 || d->dv % 32 != 0) return GLA_ERR_UNSUPPORTED;
  const long long bh = (long long)d->B * d->H;
  if (bh * (d->dv / 32) > (1LL << 31) - 1) return GLA_ERR_UNSUPPORTED;
  if (bh * (long long)d->T > (1LL << 31) - 1) return GLA_ERR_UNSUPPORTED;
  if (bh == 0 || d->T == 0) return GLA_OK;   // nothing to do; S is left as it is
  if (!q || !k || !v || !log_alpha || !S || !o) return GLA_ERR_INVALID_ARG;
  for (const void* p : std::initializer_list<const void*>{q, k, v, log_alpha, S, o})
    if (!aligned16(p)) return GLA_ERR_INVALID_ARG;
  gla::DecodeArgs a{};
  a.dtype = d->dtype; a.BH = (int)bh; a.T = d->T; a.dk = d->dk; a.dv = d->dv;
  a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.S = S; a.o = o; a.gate = gate_of(d);
  a.gscalar = scalar_gate(d) ? 1 : 0;
  return dev(gla::launch_decode(a, (hipStream_t)stream));
}

}  // extern "C"

// =====================================================================================
// Gated Slot Attention (page "Gated Slot Attention for Efficient Linear-Time Sequence
// Modeling", Abstract): two GLA passes joined by a softmax.  Pipeline (fp32, chunk 64):
//   w = 1 - exp(log_alpha)
//   first pass  : intra-chunk kernel on (w, log_alpha) -> (w * e^(gamma - g))^T, e^gamma, g;
//                 state scan with values k -> key slots S1_[i] [m][dk]; k_vg_out -> s
//   p = softmax(s)
//   second pass : gla_chunk_fwd with queries p, keys w, values v, gates log_alpha -> o
// backward: the forward again up to p, gla_chunk_bwd of the second pass (dp, dw2, dv,
// dlog_alpha2), ds = softmax backward, the intra-chunk kernel on (ds, log_alpha) ->
// (ds * e^g)^T, the reverse scan with values q -> dS1, k_vg_bwd -> dq, dk, dw1 and the
// gate terms, the closed-form gate scan, and dlog_alpha = dla1 + dla2 - (dw1 + dw2) e^la.
// bf16: the first pass runs on fp32 copies of q, k and log_alpha; p and w go to the
// second pass (the layer's bf16 path, recompute forward) rounded to bf16, its gradients
// come back in bf16; the softmax backward, the first pass's backward and the gate
// combination stay fp32; dq, dk, dlog_alpha are rounded to bf16 at the end.
// =====================================================================================
namespace {

struct GsaPlan {
  size_t w = 0, g2 = 0, KhT = 0, eg = 0, S1 = 0, s = 0, p = 0, ws2 = 0, dp = 0, dw2 = 0,
         dla2 = 0, ds = 0, QhT = 0, dS1 = 0, dw1 = 0, Dloc = 0, tot = 0, dla1 = 0, sslots = 0,
         sdec = 0, total = 0;
  // bf16 only: fp32 copies of q, k, log_alpha; bf16 copies of p and w; the second pass's
  // bf16 gradients for p, w and log_alpha
  size_t q32 = 0, k32 = 0, la32 = 0, p16 = 0, w16 = 0, dp16 = 0, dw2h = 0, dla2h = 0;
  size_t ws2_bytes = 0;
};

gla_desc_t gsa_layer2(const gla_gsa_desc_t* d) {
  gla_desc_t x{};
  x.B = d->B; x.H = d->H; x.T = d->T; x.dk = d->slots; x.dv = d->dv; x.chunk = 64;
  x.subchunk = 16; x.dtype = d->dtype;
  // fp32: the materialized forward (the fused kernel reads fp32 operands from memory);
  // bf16: the layer's fused recompute forward
  x.state_mode = d->dtype == GLA_BF16 ? GLA_STATES_RECOMPUTE : GLA_STATES_MATERIALIZED;
  x.gate = GLA_GATE_LOG_ALPHA; x.gate_tau = 1.f; x.gate_shape = GLA_GATE_PER_KEY;
  return x;
}

// The first pass's key-slot scan (state [slots][dk], every chunk state written, fp32).
gla::ScanArgs gsa_slot_scan(const gla_gsa_desc_t* d) {
  gla::ScanArgs sa{};
  sa.dtype = 0; sa.C = 64; sa.BH = d->B * d->H; sa.T = d->T; sa.dk = d->slots; sa.dv = d->dk;
  sa.N = (d->T + 63) / 64; sa.reverse = false; sa.store = 3;
  return sa;
}

GsaPlan gsa_plan(const gla_gsa_desc_t* d, int pass) {
  GsaPlan p;
  const size_t BH = (size_t)d->B * d->H, T = d->T, m = d->slots, dk = d->dk;
  const size_t N = (T + 63) / 64;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  const size_t TM = BH * T * m * 4, TK = BH * T * dk * 4;
  const bool h = d->dtype == GLA_BF16;
  p.w = take(TM); p.g2 = take(TM); p.KhT = take(BH * N * m * 64 * 4); p.eg = take(BH * N * m * 4);
  p.S1 = take(BH * N * m * dk * 4); p.s = take(TM); p.p = take(TM);
  if (h) {
    p.q32 = take(TK); p.k32 = take(TK); p.la32 = take(TM); p.p16 = take(TM / 2);
    p.w16 = take(TM / 2);
  }
  // the key-slot scan in segments (few heads): states at the segment starts, decay products
  const int P = gla::scan_segments(gsa_slot_scan(d));
  if (P > 1) p.sslots = take((size_t)(P - 1) * BH * m * dk * 4);
  if (P > 2) p.sdec = take((size_t)(P - 1) * BH * m * 4);
  const gla_desc_t l2 = gsa_layer2(d);
  const size_t b2 = plan_of(&l2, pass == GLA_PASS_BWD ? GLA_PASS_BWD : GLA_PASS_FWD).total;
  p.ws2 = take(b2); p.ws2_bytes = b2;
  if (pass == GLA_PASS_BWD) {
    p.dp = take(TM); p.ds = take(TM);
    if (h) {
      p.dp16 = take(TM / 2); p.dw2h = take(TM / 2); p.dla2h = take(TM / 2);
    } else {
      p.dw2 = take(TM); p.dla2 = take(TM);
    }
    p.QhT = take(BH * N * m * 64 * 4); p.dS1 = take(BH * N * m * dk * 4); p.dw1 = take(TM);
    p.Dloc = take(TM); p.tot = take(BH * N * m * 4); p.dla1 = take(TM);
  }
  p.total = off;
  return p;
}

struct GsaFwd {   // the forward up to p (bf16: and its bf16 copies), and o when asked
  gla_status_t run(const gla_gsa_desc_t* d, const void* q_in, const void* k_in, const void* v,
                   const void* la_in, void* o, char* w, const GsaPlan& p, hipStream_t s) {
    const int BH = d->B * d->H, T = d->T, m = d->slots, DK = d->dk, N = (T + 63) / 64;
    const bool h = d->dtype == GLA_BF16;
    const long TK = (long)BH * T * DK, TM = (long)BH * T * m;
    gla_status_t rs;
    const float *q = (const float*)q_in, *k = (const float*)k_in, *la = (const float*)la_in;
    if (h) {   // the first pass in fp32
      if ((rs = dev(gla::launch_cast_bf16_f32(q_in, (float*)(w + p.q32), TK, s))) != GLA_OK) return rs;
      if ((rs = dev(gla::launch_cast_bf16_f32(k_in, (float*)(w + p.k32), TK, s))) != GLA_OK) return rs;
      if ((rs = dev(gla::launch_cast_bf16_f32(la_in, (float*)(w + p.la32), TM, s))) != GLA_OK)
        return rs;
      q = (const float*)(w + p.q32); k = (const float*)(w + p.k32); la = (const float*)(w + p.la32);
    }
    if ((rs = dev(gla::launch_gsa_w(la, (float*)(w + p.w), TM, s))) != GLA_OK) return rs;
    gla::IntraArgs ia{};
    ia.dtype = 0; ia.C = 64; ia.BH = BH; ia.T = T; ia.dk = m; ia.N = N; ia.want_A = false;
    ia.q = w + p.w; ia.k = w + p.w; ia.la = la;
    ia.KhT = w + p.KhT; ia.eg = (float*)(w + p.eg); ia.g2_out = (float*)(w + p.g2);
    ia.gate = gla::GateFn{0, 1.f};
    if ((rs = dev(gla::launch_intra(ia, s))) != GLA_OK) return rs;
    gla::ScanArgs sa = gsa_slot_scan(d);
    sa.XT = w + p.KhT; sa.Y = k; sa.eg = (const float*)(w + p.eg); sa.states = w + p.S1;
    const int P = gla::scan_segments(sa);
    if ((rs = dev(gla::launch_state_scan_seg(sa, P > 1 ? (float*)(w + p.sslots) : nullptr,
                                             P > 2 ? (float*)(w + p.sdec) : nullptr, s))) !=
        GLA_OK)
      return rs;
    if ((rs = dev(gla::launch_vg_out(q, k, (const float*)(w + p.w), (const float*)(w + p.g2),
                                     (const float*)(w + p.S1), (float*)(w + p.s), BH, T, DK, m,
                                     s))) != GLA_OK)
      return rs;
    if ((rs = dev(gla::launch_softmax_rows((const float*)(w + p.s), (float*)(w + p.p),
                                           (long)BH * T, m, s))) != GLA_OK)
      return rs;
    if (h) {   // the second pass's queries and keys in bf16
      if ((rs = dev(gla::launch_cast_f32_bf16((const float*)(w + p.p), w + p.p16, TM, s))) != GLA_OK)
        return rs;
      if ((rs = dev(gla::launch_cast_f32_bf16((const float*)(w + p.w), w + p.w16, TM, s))) != GLA_OK)
        return rs;
    }
    if (!o) return GLA_OK;
    const gla_desc_t l2 = gsa_layer2(d);
    return gla_chunk_fwd(&l2, w + (h ? p.p16 : p.p), w + (h ? p.w16 : p.w), v, la_in, nullptr, o,
                         nullptr, w + p.ws2, p.ws2_bytes, s);
  }
};

gla_status_t gsa_common_checks(const gla_gsa_desc_t* d, int pass) {
  const gla_status_t st = gla_gsa_validate(d);
  if (st != GLA_OK) return st;
  if (pass != GLA_PASS_FWD && pass != GLA_PASS_BWD) return GLA_ERR_INVALID_ARG;
  return GLA_OK;
}

}  // namespace

extern "C" {

gla_status_t gla_gsa_validate(const gla_gsa_desc_t* d) {
  if (!d) return GLA_ERR_INVALID_ARG;
  if (d->B < 0 || d->H < 0 || d->T < 0 || d->dk < 0 || d->dv < 0 || d->slots < 0)
    return GLA_ERR_INVALID_ARG;
  if (d->dtype != GLA_F32 && d->dtype != GLA_BF16) return GLA_ERR_INVALID_ARG;
  if (d->dk < 64 || d->dk > 256 || d->dk % 64 != 0) return GLA_ERR_UNSUPPORTED;
  if (d->slots < 64 || d->slots > 256 || d->slots % 64 != 0) return GLA_ERR_UNSUPPORTED;
  if (d->dv < 64 || d->dv > 1024 || d->dv % 64 != 0) return GLA_ERR_UNSUPPORTED;
  const long long bh = (long long)d->B * d->H;
  if (bh > 65535) return GLA_ERR_UNSUPPORTED;
  if (bh * (long long)d->T > (1LL << 31) - 1) return GLA_ERR_UNSUPPORTED;
  if (((long long)d->T + 63) / 64 > 65535) return GLA_ERR_UNSUPPORTED;
  return GLA_OK;
}

gla_status_t gla_gsa_workspace_bytes(const gla_gsa_desc_t* d, int32_t pass, size_t* bytes) {
  if (!bytes) return GLA_ERR_INVALID_ARG;
  const gla_status_t st = gsa_common_checks(d, pass);
  if (st != GLA_OK) return st;
  *bytes = (size_t)d->B * d->H * d->T == 0 ? 0 : gsa_plan(d, pass).total;
  return GLA_OK;
}

gla_status_t gla_gsa_fwd(const gla_gsa_desc_t* d, const void* q, const void* k, const void* v,
                         const void* log_alpha, void* o, void* ws, size_t ws_bytes,
                         void* stream) {
  const gla_status_t st = gsa_common_checks(d, GLA_PASS_FWD);
  if (st != GLA_OK) return st;
  if ((long long)d->B * d->H * d->T == 0) return GLA_OK;
  if (!q || !k || !v || !log_alpha || !o) return GLA_ERR_INVALID_ARG;
  for (const void* ptr : std::initializer_list<const void*>{q, k, v, log_alpha, o, ws})
    if (!aligned16(ptr)) return GLA_ERR_INVALID_ARG;
  const GsaPlan p = gsa_plan(d, GLA_PASS_FWD);
  if (!ws || ws_bytes < p.total) return GLA_ERR_WORKSPACE;
  GsaFwd f;
  return f.run(d, q, k, v, log_alpha, o, (char*)ws, p, (hipStream_t)stream);
}

gla_status_t gla_gsa_bwd(const gla_gsa_desc_t* d, const void* q, const void* k, const void* v,
                         const void* log_alpha, const void* dO, void* dq, void* dk, void* dv,
                         void* dlog_alpha, void* ws, size_t ws_bytes, void* stream) {
  const gla_status_t st = gsa_common_checks(d, GLA_PASS_BWD);
  if (st != GLA_OK) return st;
  if ((long long)d->B * d->H * d->T == 0) return GLA_OK;
  if (!q || !k || !v || !log_alpha || !dO || !dq || !dk || !dv || !dlog_alpha)
    return GLA_ERR_INVALID_ARG;
  for (const void* ptr : std::initializer_list<const void*>{q, k, v, log_alpha, dO, dq, dk, dv,
                                                            dlog_alpha, ws})
    if (!aligned16(ptr)) return GLA_ERR_INVALID_ARG;
  const GsaPlan p = gsa_plan(d, GLA_PASS_BWD);
  if (!ws || ws_bytes < p.total) return GLA_ERR_WORKSPACE;
  char* w = (char*)ws;
  hipStream_t s = (hipStream_t)stream;
  const bool h = d->dtype == GLA_BF16;
  const int BH = d->B * d->H, T = d->T, m = d->slots, DK = d->dk, N = (T + 63) / 64;
  const long TM = (long)BH * T * m;
  GsaFwd f;
  gla_status_t rs = f.run(d, q, k, v, log_alpha, nullptr, w, p, s);
  if (rs != GLA_OK) return rs;
  // the first pass's operands in fp32 (bf16: the copies the forward made)
  const float* la = h ? (const float*)(w + p.la32) : (const float*)log_alpha;
  const float* q32 = h ? (const float*)(w + p.q32) : (const float*)q;
  const float* k32 = h ? (const float*)(w + p.k32) : (const float*)k;
  // second pass backward: gradients for p, w (as keys), v and log_alpha
  const gla_desc_t l2 = gsa_layer2(d);
  rs = gla_chunk_bwd(&l2, w + (h ? p.p16 : p.p), w + (h ? p.w16 : p.w), v, log_alpha, nullptr, dO,
                     nullptr, w + (h ? p.dp16 : p.dp), w + (h ? p.dw2h : p.dw2), dv,
                     w + (h ? p.dla2h : p.dla2), nullptr, w + p.ws2, p.ws2_bytes, s);
  if (rs != GLA_OK) return rs;
  if (h && (rs = dev(gla::launch_cast_bf16_f32(w + p.dp16, (float*)(w + p.dp), TM, s))) != GLA_OK)
    return rs;
  if ((rs = dev(gla::launch_softmax_bwd((const float*)(w + p.p), (const float*)(w + p.dp),
                                        (float*)(w + p.ds), (long)BH * T, m, s))) != GLA_OK)
    return rs;
  // first pass backward: (ds * e^g)^T per chunk, the reverse scan of the key slots
  gla::IntraArgs ia{};
  ia.dtype = 0; ia.C = 64; ia.BH = BH; ia.T = T; ia.dk = m; ia.N = N; ia.want_A = false;
  ia.q = w + p.ds; ia.k = w + p.w; ia.la = la; ia.QhT = w + p.QhT;
  ia.eg = (float*)(w + p.eg); ia.gate = gla::GateFn{0, 1.f};
  if ((rs = dev(gla::launch_intra(ia, s))) != GLA_OK) return rs;
  gla::ScanArgs ra = gsa_slot_scan(d);
  ra.reverse = true; ra.XT = w + p.QhT; ra.Y = q32; ra.eg = (const float*)(w + p.eg);
  ra.states = w + p.dS1;
  // in segments like the forward key-slot scan (same shape: the same workspace slots)
  const int P = gla::scan_segments(ra);
  if ((rs = dev(gla::launch_state_scan_seg(ra, P > 1 ? (float*)(w + p.sslots) : nullptr,
                                           P > 2 ? (float*)(w + p.sdec) : nullptr, s))) !=
      GLA_OK)
    return rs;
  if ((rs = dev(gla::launch_vg_bwd(q32, k32, (const float*)(w + p.w),
                                   (const float*)(w + p.g2), (const float*)(w + p.ds),
                                   (const float*)(w + p.s), (const float*)(w + p.S1),
                                   (const float*)(w + p.dS1), dq, dk, h ? 1 : 0,
                                   (float*)(w + p.dw1), (float*)(w + p.Dloc), (float*)(w + p.tot),
                                   BH, T, DK, m, s))) != GLA_OK)
    return rs;
  if ((rs = dev(gla::launch_gate_grad(0, (const float*)(w + p.Dloc), (const float*)(w + p.tot),
                                      nullptr, la, gla::GateFn{0, 1.f}, w + p.dla1, nullptr, BH, T,
                                      m, 64, s))) != GLA_OK)
    return rs;
  if (!h)
    return dev(gla::launch_gsa_combine(la, (const float*)(w + p.dla1), (const float*)(w + p.dla2),
                                       (const float*)(w + p.dw1), (const float*)(w + p.dw2),
                                       (float*)dlog_alpha, TM, s));
  return dev(gla::launch_gsa_combine_bf16(la, (const float*)(w + p.dla1), w + p.dla2h,
                                          (const float*)(w + p.dw1), w + p.dw2h, dlog_alpha, TM,
                                          s));
}

}  // extern "C"
