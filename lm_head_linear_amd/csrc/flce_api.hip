// C-ABI entry points: argument checks, workspace carving, launch sequence,
// optional per-kernel timing.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "../../include/flce.h"
#include "flce_internal.h"
#include "flce_plan.h"
#include "gemm_index.h"

namespace {

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
                                           "dH_gemm", "fill", "probs_to_grad", "dH_reduce"};

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
  a.lsum = reinterpret_cast<double*>(ws + p.off_lsum);
  a.g = ws + p.off_g;
  a.dh_acc = nullptr;
  a.dh_part = p.dh_kseg ? reinterpret_cast<float*>(ws + p.off_dhpart) : nullptr;
  e = flce::launch_label_scan(p, a, L);
  for (int64_t c = 0; e == hipSuccess && c < p.n_tok_chunks; ++c) {
    e = flce::bf16_nr_forward_chunk(p, a, c, L);
    if (e == hipSuccess) e = flce::launch_merge(p, a, c * p.nc, flce::gemm::nr_chunk_tokens(p, c), L);
    if (e == hipSuccess) e = flce::bf16_nr_backward_chunk(p, a, c, L);
  }
  if (e == hipSuccess) e = flce::launch_loss_final(p, a, L);
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
        int logits_dtype = FLCE_F32) {
  flce::Plan p;
  if (!flce::make_plan(N, H, V, dtype, &p, backward, grad_dtype)) return FLCE_ERR_ARG;

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
  a.lsum = reinterpret_cast<double*>(ws + p.off_lsum);
  a.g = backward ? ws + p.off_g : nullptr;
  a.dh_acc = p.need_dh_acc ? reinterpret_cast<float*>(ws + p.off_dhacc) : nullptr;
  a.dh_part = p.dh_kseg ? reinterpret_cast<float*>(ws + p.off_dhpart) : nullptr;

  const bool bf16 = dtype == FLCE_BF16;
  e = flce::launch_label_scan(p, a, L);
  if (e == hipSuccess) e = bf16 ? flce::bf16_forward(p, a, L) : flce::f32_forward(p, a, L);
  if (e == hipSuccess) e = flce::launch_merge_and_loss(p, a, L);
  for (int64_t c = 0; backward && e == hipSuccess && c < p.n_chunks; ++c)
    e = bf16 ? flce::bf16_backward_chunk(p, a, c, L) : flce::f32_backward_chunk(p, a, c, L);
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
  int st = flce_check_args_ex(h, W, labels, N, H, V, ignore_index, softcap, reduction,
                              num_label_tokens, loss, num_tokens, dH, dW, stream, dtype,
                              mb_scale, accumulate_dW, workspace, size_t(-1), status, lse_out,
                              dtype);
  if (st != FLCE_OK) return st;
  if (dtype != FLCE_BF16 || token_chunk < 0) return FLCE_ERR_UNSUPPORTED;
  const size_t need = flce_workspace_size_nr(N, H, V, dtype, token_chunk);
  if (need == 0) return FLCE_ERR_UNSUPPORTED;   // shapes beyond the kernels' index range
  if (workspace_bytes < need) return FLCE_ERR_WORKSPACE;
  return FLCE_OK;
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
  return run(h, W, labels, N, H, V, ignore_index, softcap, reduction, num_label_tokens, loss,
             num_tokens, nullptr, nullptr, stream, dtype, mb_scale, 0, workspace, status,
             lse_out, false, dtype);
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
  return run(h, W, labels, N, H, V, ignore_index, softcap, reduction, num_label_tokens, loss,
             num_tokens, nullptr, nullptr, stream, dtype, mb_scale, 0, workspace, status,
             lse_out, false, dtype, N > 0 ? logits : nullptr, ld_logits, logits_dtype);
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
