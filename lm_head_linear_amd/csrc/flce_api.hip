// C-ABI entry points: argument checks, workspace carving, launch sequence,
// optional per-kernel timing.
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <cstdint>
#include <mutex>
#include <vector>

#include "../../include/flce.h"
#include "flce_internal.h"
#include "flce_plan.h"
#include "gemm_index.h"

namespace {

// ---- ROCTX ranges -------------------------------------------------------------
// A named range around each entry point's call and each pass it enqueues
// (forward, merge, one per backward chunk or token chunk), for a profiler's
// marker trace (rocprofv3 --marker-trace). They span the host-side enqueue of
// the pass; the kernel trace gives the device times.
struct Range {
  explicit Range(const char* name) { roctxRangePushA(name); }
  ~Range() { roctxRangePop(); }
  Range(const Range&) = delete;
  Range& operator=(const Range&) = delete;
};

// ---- per-kernel timing ------------------------------------------------------
struct Rec {
  int kind;
  hipEvent_t a, b;
};
struct Prof {
  bool on = false;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<Rec> recs;
  int pending_kind = -1;
  hipEvent_t pending = nullptr;
  bool failed = false;
};
Prof g_prof;

hipEvent_t take_event() {
  if (g_prof.used == g_prof.pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) { g_prof.failed = true; return nullptr; }
    g_prof.pool.push_back(e);
  }
  return g_prof.pool[g_prof.used++];
}

void prof_before(int kind, hipStream_t s) {
  hipEvent_t e = take_event();
  if (!e) return;
  if (hipEventRecord(e, s) != hipSuccess) { g_prof.failed = true; return; }
  g_prof.pending = e;
  g_prof.pending_kind = kind;
}

void prof_after(int kind, hipStream_t s) {
  if (!g_prof.pending || g_prof.pending_kind != kind) return;
  hipEvent_t e = take_event();
  if (!e) return;
  if (hipEventRecord(e, s) != hipSuccess) { g_prof.failed = true; g_prof.pending = nullptr; return; }
  g_prof.recs.push_back(Rec{kind, g_prof.pending, e});
  g_prof.pending = nullptr;
}

const char* kKindNames[flce::kNumKinds] = {"label_scan", "lse_fwd_gemm", "lse_merge",
                                           "loss_final", "grad_logits_gemm", "dW_gemm",
                                           "dH_gemm", "fill", "probs_to_grad", "dH_reduce",
                                           "gather", "dH_dW_gemm", "pad_copy"};

// ---- scratch of flce_forward_noalloc ---------------------------------------
// One copy on every GPU the library runs on, held until the process ends. In
// host code `scratch` is only a host-side stand-in for the symbol, never an
// address: the device address of each GPU's copy comes from
// hipGetSymbolAddress, looked up once per device with that device current,
// and only that address is handed to kernels.
static __device__ __align__(256) char scratch[FLCE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch copy of the GPU `stream` runs on (set up on
// the first call on that GPU).
hipError_t scratch_address(hipStream_t stream, void** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream) {
    hipDevice_t sd;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return e;
    dev = int(sd);
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// A call whose bf16 rows are padded (Plan::pad_h) runs at the padded width on
// the workspace's copies: W padded, dW padded from the caller's when it is
// added to, dH and dW written there and copied out at the end. The gather
// pads the hidden rows it copies; a call without it reads a padded copy of h.
hipError_t pad_inputs(const flce::Plan& p, flce::Args& a, char* ws, bool backward,
                      const flce::Launcher& L) {
  if (!p.pad_h) return hipSuccess;
  void* wp = ws + p.off_wp;
  hipError_t e = flce::launch_copy_rows(a.W, p.h_in, wp, p.H, p.V, p.h_in, p.H, p.elem, L);
  a.W = wp;
  a.H = p.H;
  if (e == hipSuccess && !p.compact) {
    void* hp = ws + p.off_hp;
    e = flce::launch_copy_rows(a.h, p.h_in, hp, p.H, p.N, p.h_in, p.H, p.elem, L);
    a.h = hp;
  }
  if (!backward) return e;
  void* dwp = ws + p.off_dwp;
  if (e == hipSuccess && a.accumulate_dW)
    e = flce::launch_copy_rows(a.dW, p.h_in, dwp, p.H, p.V, p.h_in, p.H, p.grad_elem, L);
  a.dW = dwp;
  a.dH = ws + p.off_dhp;
  return e;
}

hipError_t crop_outputs(const flce::Plan& p, const char* ws, void* dH, void* dW,
                        const flce::Launcher& L) {
  if (!p.pad_h) return hipSuccess;
  hipError_t e = flce::launch_copy_rows(ws + p.off_dwp, p.H, dW, p.h_in, p.V, p.h_in, p.h_in,
                                        p.grad_elem, L);
  if (e == hipSuccess)
    e = flce::launch_copy_rows(ws + p.off_dhp, p.H, dH, p.h_in, p.N, p.h_in, p.h_in,
                               p.grad_elem, L);
  return e;
}

// The no-recompute variant (arguments already checked): token chunk by chunk,
// the forward keeps the probabilities, the chunk's merge gives its lse, G is
// formed in place, then dW (added over the chunks) and the chunk's dH.
int run_nr(const void* h, const void* W, const int64_t* labels, int64_t N, int64_t H, int64_t V,
           int64_t ignore_index, float softcap, int reduction, int64_t num_label_tokens,
           float* loss, int64_t* num_tokens, void* dH, void* dW, void* stream, int dtype,
           float mb_scale, int accumulate_dW, void* workspace, int32_t* status, float* lse_out,
           int64_t token_chunk) {
  flce::Plan p;
  if (!flce::make_plan_nr(N, H, V, dtype, token_chunk, &p)) return FLCE_ERR_UNSUPPORTED;
  flce::Launcher L{static_cast<hipStream_t>(stream), nullptr, nullptr};
  if (g_prof.on) { L.before = prof_before; L.after = prof_after; }
  char* ws = static_cast<char*>(workspace);
  flce::Args a{};
  a.h = h; a.W = W; a.labels = labels;
  a.N = N; a.H = H; a.V = V;
  a.ignore_index = ignore_index; a.softcap = softcap; a.reduction = reduction;
  a.num_label_tokens = num_label_tokens;
  a.loss = loss; a.num_tokens = num_tokens; a.dH = dH; a.dW = dW;
  a.mb_scale = mb_scale; a.accumulate_dW = accumulate_dW ? 1 : 0;
  a.status = status; a.lse_out = lse_out;
  a.sc = reinterpret_cast<flce::Scalars*>(ws + p.off_scalars);
  hipError_t e;
  if (N == 0) {
    e = flce::launch_empty(p, a, L);
    if (e == hipSuccess && !a.accumulate_dW)
      e = flce::launch_zero_bytes(dW, size_t(V) * H * p.elem, L);
    return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
  }
  a.part = reinterpret_cast<float2*>(ws + p.off_part);
  a.zt = reinterpret_cast<float*>(ws + p.off_zt);
  a.lse = reinterpret_cast<float*>(ws + p.off_lse);
  a.tok_loss = reinterpret_cast<double*>(ws + p.off_tokloss);
  a.g = ws + p.off_g;
  a.dh_acc = nullptr;
  a.dh_part = p.dh_kseg ? reinterpret_cast<float*>(ws + p.off_dhpart) : nullptr;
  a.dw_acc = p.need_dw_acc ? reinterpret_cast<float*>(ws + p.off_dwacc) : nullptr;
  a.idx = reinterpret_cast<int32_t*>(ws + p.off_idx);
  a.yc = reinterpret_cast<int64_t*>(ws + p.off_yc);
  a.bcnt = reinterpret_cast<int32_t*>(ws + p.off_bcnt);
  a.ccnt = reinterpret_cast<int64_t*>(ws + p.off_ccnt);
  a.hc = ws + p.off_hc;
  {
    Range r("flce.setup");
    e = pad_inputs(p, a, ws, true, L);
    // the labels scanned and the tokens gathered, the kept ones first; the
    // chunks run over that order (the ignored tokens only for their lse, when
    // it is asked for)
    const bool all_rows = lse_out != nullptr;
    if (e == hipSuccess) e = flce::launch_scan_gather(p, a, all_rows, L);
    if (e == hipSuccess) e = flce::launch_chunk_counts(p, a, all_rows, L);
  }
  for (int64_t c = 0; e == hipSuccess && c < p.n_tok_chunks; ++c) {
    Range r("flce.token_chunk");
    const int64_t t0 = c * p.nc, nt = flce::gemm::nr_chunk_tokens(p, c);
    e = flce::bf16_nr_forward_chunk(p, a, c, L);
    if (e == hipSuccess) e = flce::launch_merge_gathered(p, a, t0, nt, a.ccnt + c, L);
    if (e == hipSuccess) e = flce::bf16_nr_backward_chunk(p, a, c, L);
  }
  Range r("flce.finish");
  if (e == hipSuccess) e = flce::launch_loss_final(p, a, L);
  if (e == hipSuccess) e = crop_outputs(p, ws, dH, dW, L);
  return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

// The launch sequence of both entry points; arguments already checked.
// Forward: label scan, forward GEMM with the log-sum-exp partials, merge and
// loss. With backward, then every vocabulary chunk's gradient GEMMs.
int run(const void* h, const void* W, const int64_t* labels, int64_t N, int64_t H, int64_t V,
        int64_t ignore_index, float softcap, int reduction, int64_t num_label_tokens,
        float* loss, int64_t* num_tokens, void* dH, void* dW, void* stream, int dtype,
        float mb_scale, int accumulate_dW, void* workspace, int32_t* status, float* lse_out,
        bool backward, int grad_dtype, void* logits = nullptr, int64_t ld_logits = 0,
        int logits_dtype = FLCE_F32, int gather = -1) {
  flce::Plan p;
  if (!flce::make_plan(N, H, V, dtype, &p, backward, grad_dtype, gather)) return FLCE_ERR_ARG;

  flce::Launcher L{static_cast<hipStream_t>(stream), nullptr, nullptr};
  if (g_prof.on) { L.before = prof_before; L.after = prof_after; }

  char* ws = static_cast<char*>(workspace);
  flce::Args a{};
  a.h = h; a.W = W; a.labels = labels;
  a.N = N; a.H = H; a.V = V;
  a.ignore_index = ignore_index; a.softcap = softcap; a.reduction = reduction;
  a.num_label_tokens = num_label_tokens;
  a.loss = loss; a.num_tokens = num_tokens; a.dH = dH; a.dW = dW;
  a.mb_scale = mb_scale; a.accumulate_dW = accumulate_dW ? 1 : 0;
  a.status = status; a.lse_out = lse_out;
  a.logits = logits; a.ld_logits = ld_logits; a.logits_dtype = logits_dtype;
  a.sc = reinterpret_cast<flce::Scalars*>(ws + p.off_scalars);

  hipError_t e;
  if (N == 0) {
    e = flce::launch_empty(p, a, L);
    if (e == hipSuccess && backward && !a.accumulate_dW)
      e = flce::launch_zero_bytes(dW, size_t(V) * H * p.grad_elem, L);
    return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
  }
  a.part = reinterpret_cast<float2*>(ws + p.off_part);
  a.zt = reinterpret_cast<float*>(ws + p.off_zt);
  a.lse = reinterpret_cast<float*>(ws + p.off_lse);
  a.tok_loss = reinterpret_cast<double*>(ws + p.off_tokloss);
  a.g = backward ? ws + p.off_g : nullptr;
  a.dh_acc = p.need_dh_acc ? reinterpret_cast<float*>(ws + p.off_dhacc) : nullptr;
  a.dh_part = p.dh_kseg ? reinterpret_cast<float*>(ws + p.off_dhpart) : nullptr;
  if (p.compact) {
    a.idx = reinterpret_cast<int32_t*>(ws + p.off_idx);
    a.yc = reinterpret_cast<int64_t*>(ws + p.off_yc);
    a.bcnt = reinterpret_cast<int32_t*>(ws + p.off_bcnt);
    a.hc = ws + p.off_hc;
  }

  const bool bf16 = dtype == FLCE_BF16;
  {
    Range r("flce.setup");
    e = pad_inputs(p, a, ws, backward, L);
    // a compact plan gathers the tokens with the label scan, the kept ones in
    // front; the forward then skips the ignored ones unless their lse is asked
    // for
    if (e == hipSuccess)
      e = p.compact ? flce::launch_scan_gather(p, a, lse_out != nullptr, L)
                    : flce::launch_label_scan(p, a, L);
  }
  {
    Range r("flce.forward");
    if (e == hipSuccess) e = bf16 ? flce::bf16_forward(p, a, L) : flce::f32_forward(p, a, L);
    if (e == hipSuccess) e = flce::launch_merge_and_loss(p, a, L);
  }
  for (int64_t c = 0; backward && e == hipSuccess && c < p.n_chunks; ++c) {
    Range r("flce.backward_chunk");
    e = bf16 ? flce::bf16_backward_chunk(p, a, c, L) : flce::f32_backward_chunk(p, a, c, L);
  }
  if (e == hipSuccess && backward && p.pad_h) {
    Range r("flce.copy_out");
    e = crop_outputs(p, ws, dH, dW, L);
  }
  return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

}  // namespace

extern "C" {

int flce_forward_backward(const void* h, const void* W, const int64_t* labels, int64_t N,
                          int64_t H, int64_t V, int64_t ignore_index, float softcap,
                          int reduction, int64_t num_label_tokens, float* loss,
                          int64_t* num_tokens, void* dH, void* dW, void* stream, int dtype,
                          float mb_scale, int accumulate_dW, void* workspace,
                          size_t workspace_bytes, int32_t* status, float* lse_out) {
  return flce_forward_backward_ex(h, W, labels, N, H, V, ignore_index, softcap, reduction,
                                  num_label_tokens, loss, num_tokens, dH, dW, stream, dtype,
                                  mb_scale, accumulate_dW, workspace, workspace_bytes, status,
                                  lse_out, dtype);
}

int flce_forward_backward_ex(const void* h, const void* W, const int64_t* labels, int64_t N,
                             int64_t H, int64_t V, int64_t ignore_index, float softcap,
                             int reduction, int64_t num_label_tokens, float* loss,
                             int64_t* num_tokens, void* dH, void* dW, void* stream, int dtype,
                             float mb_scale, int accumulate_dW, void* workspace,
                             size_t workspace_bytes, int32_t* status, float* lse_out,
                             int grad_dtype) {
  int st = flce_check_args_ex(h, W, labels, N, H, V, ignore_index, softcap, reduction,
                              num_label_tokens, loss, num_tokens, dH, dW, stream, dtype,
                              mb_scale, accumulate_dW, workspace, workspace_bytes, status,
                              lse_out, grad_dtype);
  if (st != FLCE_OK) return st;
  Range r("flce_forward_backward");
  return run(h, W, labels, N, H, V, ignore_index, softcap, reduction, num_label_tokens, loss,
             num_tokens, dH, dW, stream, dtype, mb_scale, accumulate_dW, workspace, status,
             lse_out, true, grad_dtype);
}

size_t flce_workspace_size_nr(int64_t N, int64_t H, int64_t V, int dtype, int64_t token_chunk) {
  flce::Plan p;
  if (!flce::make_plan_nr(N, H, V, dtype, token_chunk, &p)) return 0;
  return p.total;
}

int64_t flce_token_chunk_nr(int64_t N, int64_t H, int64_t V, int dtype, int64_t token_chunk) {
  flce::Plan p;
  if (!flce::make_plan_nr(N, H, V, dtype, token_chunk, &p)) return 0;
  return p.nc;
}

int flce_check_args_nr(const void* h, const void* W, const int64_t* labels, int64_t N,
                       int64_t H, int64_t V, int64_t ignore_index, float softcap,
                       int reduction, int64_t num_label_tokens, float* loss,
                       int64_t* num_tokens, void* dH, void* dW, void* stream, int dtype,
                       float mb_scale, int accumulate_dW, void* workspace,
                       size_t workspace_bytes, int32_t* status, float* lse_out,
                       int64_t token_chunk) {
  // the common rules, with the workspace checked against this variant's plan
  (void)ignore_index; (void)stream; (void)accumulate_dW;
  const size_t need = flce_workspace_size_nr(N, H, V, dtype, token_chunk);
  int st = flce::check_grad_args(h, W, labels, N, H, V, softcap, reduction, num_label_tokens,
                                 loss, num_tokens, dH, dW, dtype, mb_scale, workspace,
                                 workspace_bytes, status, lse_out, need ? need : 1);
  if (st != FLCE_OK && st != FLCE_ERR_WORKSPACE) return st;
  if (dtype != FLCE_BF16 || token_chunk < 0) return FLCE_ERR_UNSUPPORTED;
  if (need == 0) return FLCE_ERR_UNSUPPORTED;   // shapes beyond the kernels' index range
  return st;
}

int flce_forward_backward_nr(const void* h, const void* W, const int64_t* labels, int64_t N,
                             int64_t H, int64_t V, int64_t ignore_index, float softcap,
                             int reduction, int64_t num_label_tokens, float* loss,
                             int64_t* num_tokens, void* dH, void* dW, void* stream, int dtype,
                             float mb_scale, int accumulate_dW, void* workspace,
                             size_t workspace_bytes, int32_t* status, float* lse_out,
                             int64_t token_chunk) {
  int st = flce_check_args_nr(h, W, labels, N, H, V, ignore_index, softcap, reduction,
                              num_label_tokens, loss, num_tokens, dH, dW, stream, dtype,
                              mb_scale, accumulate_dW, workspace, workspace_bytes, status,
                              lse_out, token_chunk);
  if (st != FLCE_OK) return st;
  Range r("flce_forward_backward_nr");
  return run_nr(h, W, labels, N, H, V, ignore_index, softcap, reduction, num_label_tokens, loss,
                num_tokens, dH, dW, stream, dtype, mb_scale, accumulate_dW, workspace, status,
                lse_out, token_chunk);
}

int flce_forward(const void* h, const void* W, const int64_t* labels, int64_t N, int64_t H,
                 int64_t V, int64_t ignore_index, float softcap, int reduction,
                 int64_t num_label_tokens, float* loss, int64_t* num_tokens, void* stream,
                 int dtype, float mb_scale, void* workspace, size_t workspace_bytes,
                 int32_t* status, float* lse_out) {
  int st = flce_forward_check_args(h, W, labels, N, H, V, ignore_index, softcap, reduction,
                                   num_label_tokens, loss, num_tokens, stream, dtype, mb_scale,
                                   workspace, workspace_bytes, status, lse_out);
  if (st != FLCE_OK) return st;
  Range r("flce_forward");
  return run(h, W, labels, N, H, V, ignore_index, softcap, reduction, num_label_tokens, loss,
             num_tokens, nullptr, nullptr, stream, dtype, mb_scale, 0, workspace, status,
             lse_out, false, dtype);
}

int flce_forward_noalloc(const void* h, const void* W, const int64_t* labels, int64_t N,
                         int64_t H, int64_t V, int64_t ignore_index, float softcap,
                         int reduction, int64_t num_label_tokens, float* loss,
                         int64_t* num_tokens, void* stream, int dtype, float mb_scale,
                         int32_t* status, float* lse_out) {
  // the argument checks first, against a stand-in aligned address: only the
  // workspace rules depend on it, and the scratch is always large enough
  // once the size check below has passed
  int st = flce_forward_check_args(h, W, labels, N, H, V, ignore_index, softcap, reduction,
                                   num_label_tokens, loss, num_tokens, stream, dtype, mb_scale,
                                   reinterpret_cast<void*>(uintptr_t(256)), size_t(-1), status,
                                   lse_out);
  if (st != FLCE_OK) return st;
  // the forward without the token gather (its scratch is the partials and
  // per-token arrays alone, and padded copies of h and W for a bf16 hidden
  // size that is not a multiple of 8), bit-identical to flce_forward's results
  flce::Plan p;
  if (!flce::make_plan(N, H, V, dtype, &p, false, -1, 0)) return FLCE_ERR_ARG;
  if (p.total > FLCE_NOALLOC_SCRATCH_BYTES) return FLCE_ERR_SCRATCH;
  void* ws = nullptr;
  if (scratch_address(static_cast<hipStream_t>(stream), &ws) != hipSuccess) return FLCE_ERR_HIP;
  Range r("flce_forward_noalloc");
  return run(h, W, labels, N, H, V, ignore_index, softcap, reduction, num_label_tokens, loss,
             num_tokens, nullptr, nullptr, stream, dtype, mb_scale, 0, ws, status, lse_out,
             false, dtype, nullptr, 0, FLCE_F32, 0);
}

int flce_forward_logits(const void* h, const void* W, const int64_t* labels, int64_t N,
                        int64_t H, int64_t V, int64_t ignore_index, float softcap,
                        int reduction, int64_t num_label_tokens, float* loss,
                        int64_t* num_tokens, void* stream, int dtype, float mb_scale,
                        void* workspace, size_t workspace_bytes, int32_t* status,
                        float* lse_out, void* logits, int64_t ld_logits, int logits_dtype) {
  int st = flce_forward_logits_check_args(h, W, labels, N, H, V, ignore_index, softcap,
                                          reduction, num_label_tokens, loss, num_tokens, stream,
                                          dtype, mb_scale, workspace, workspace_bytes, status,
                                          lse_out, logits, ld_logits, logits_dtype);
  if (st != FLCE_OK) return st;
  Range r("flce_forward_logits");
  return run(h, W, labels, N, H, V, ignore_index, softcap, reduction, num_label_tokens, loss,
             num_tokens, nullptr, nullptr, stream, dtype, mb_scale, 0, workspace, status,
             lse_out, false, dtype, N > 0 ? logits : nullptr, ld_logits, logits_dtype, 0);
}

int flce_profile_begin(void) {
  g_prof.on = true;
  g_prof.used = 0;
  g_prof.recs.clear();
  g_prof.pending = nullptr;
  g_prof.failed = false;
  return FLCE_OK;
}

int flce_profile_end(void) {
  g_prof.on = false;
  return g_prof.failed ? FLCE_ERR_HIP : FLCE_OK;
}

int flce_profile_kinds(void) { return flce::kNumKinds; }

const char* flce_kernel_kind_name(int kind) {
  return (kind >= 0 && kind < flce::kNumKinds) ? kKindNames[kind] : "unknown";
}

int flce_profile_query(int kind, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind >= flce::kNumKinds || !total_ms || !launches) return FLCE_ERR_ARG;
  double sum = 0.0;
  int64_t n = 0;
  for (const Rec& r : g_prof.recs) {
    if (r.kind != kind) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return FLCE_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return FLCE_ERR_HIP;
    sum += ms;
    ++n;
  }
  *total_ms = sum;
  *launches = n;
  return FLCE_OK;
}

}  // extern "C"
