// Synchronous argument checks and workspace planning (no HIP calls).
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <utility>

#include "../../include/flce.h"
#include "flce_plan.h"
#include "gemm_index.h"

namespace flce {
namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The padded buffers of a Plan::pad_h call at the padded width: W, h when the
// call does not gather (the gather pads the rows it copies), and with
// gradients dW and dH.
size_t carve_pad(Plan& q, size_t off, bool backward) {
  if (!q.pad_h) return off;
  q.off_wp = off;  off = align256(off + size_t(q.V) * q.H * q.elem);
  if (!q.compact) { q.off_hp = off; off = align256(off + size_t(q.N) * q.H * q.elem); }
  if (backward) {
    q.off_dwp = off; off = align256(off + size_t(q.V) * q.H * q.grad_elem);
    q.off_dhp = off; off = align256(off + size_t(q.N) * q.H * q.grad_elem);
  }
  return off;
}

// Optional override of the backward vocabulary chunk (rows of W), for tuning
// and for tests of the multi-chunk path; 0 = automatic. Read on every plan,
// so flce_workspace_size and flce_forward_backward must see the same value
// (a mismatch is caught as FLCE_ERR_WORKSPACE).
int64_t env_vchunk() {
  const char* s = std::getenv("FLCE_VCHUNK");
  if (!s || !*s) return 0;
  const long long x = std::atoll(s);
  return x > 0 ? int64_t(x) : int64_t(0);
}

}  // namespace

bool make_plan(int64_t N, int64_t H, int64_t V, int dtype, Plan* p, bool backward,
               int grad_dtype, int gather) {
  if (N < 0 || H <= 0 || V <= 0) return false;
  if (dtype != FLCE_F32 && dtype != FLCE_BF16) return false;
  if (grad_dtype < 0) grad_dtype = dtype;
  if (grad_dtype != FLCE_F32 && grad_dtype != FLCE_BF16) return false;
  if (dtype == FLCE_F32 && grad_dtype != FLCE_F32) return false;
  // Keep every size product far from int64 overflow.
  if (N > (int64_t(1) << 31) || H > (int64_t(1) << 24) || V > (int64_t(1) << 31)) return false;
  Plan q;
  q.h_in = H;
  if (dtype == FLCE_BF16 && H % 8 != 0) {      // see Plan::pad_h
    q.pad_h = true;
    H = round_up(H, 8);
  }
  q.N = N; q.H = H; q.V = V; q.dtype = dtype; q.grad_dtype = grad_dtype;
  q.tile = dtype == FLCE_BF16 ? kTileBF16 : kTileF32;
  q.elem = dtype == FLCE_BF16 ? 2 : 4;
  q.grad_elem = grad_dtype == FLCE_BF16 ? 2 : 4;
  q.g_parts = (dtype == FLCE_BF16 && grad_dtype == FLCE_F32) ? 2 : 1;
  q.n_tok_tiles = ceil_div(N, q.tile);
  q.n_voc_tiles = ceil_div(V, q.tile);
  q.ld_part = round_up(N > 0 ? N : 1, q.tile);
  q.ldg = round_up(N > 0 ? N : 1, 8);
  // Backward chunk: a multiple of the tile, at least one tile, at most the
  // (tile-rounded) vocabulary, with G^T's elements (both parts) within the
  // budget; the vocabulary is then split into chunks of equal size (the last
  // one shorter by less than a tile per chunk).
  int64_t vmax = round_up(V, q.tile);
  int64_t vc = env_vchunk();
  if (vc <= 0) {
    int64_t budget = N / 4 * V / q.elem;       // N V 4 / 16 bytes
    if (budget < kChunkElems) budget = kChunkElems;
    if (budget > kMaxChunkElems) budget = kMaxChunkElems;
    vc = (budget / q.g_parts / (N > 0 ? q.ldg : 1)) / q.tile * q.tile;
    if (vc >= q.tile && vc < vmax) vc = round_up(ceil_div(V, ceil_div(V, vc)), q.tile);
  } else {
    vc = round_up(vc, q.tile);
  }
  if (vc < q.tile) vc = q.tile;
  if (vc > vmax) vc = vmax;
  q.vchunk = vc;
  q.n_chunks = ceil_div(V, vc);
  q.n_loss_blocks = ceil_div(N > 0 ? N : 1, 32);   // tokens per block of the loss sum
  q.backward = backward;
  q.need_dh_acc = backward && (dtype == FLCE_BF16) && q.g_parts == 1 && q.n_chunks > 1 && N > 0;
  if (backward && dtype == FLCE_BF16 && q.g_parts == 1 && N > 0)
    q.dh_kseg = dh_split(N, H, q.vchunk, &q.dh_segs);

  size_t off = 0;
  q.off_scalars = off; off = align256(off + sizeof(Scalars));
  if (N > 0) {
    q.off_part = off;  off = align256(off + size_t(q.n_voc_tiles) * q.ld_part * 2 * sizeof(float));
    q.off_zt = off;    off = align256(off + size_t(q.ld_part) * sizeof(float));
    q.off_lse = off;   off = align256(off + size_t(q.ld_part) * sizeof(float));
    q.off_tokloss = off;
    off = align256(off + size_t(q.n_loss_blocks) * 32 * sizeof(double));
    if (backward) {
      q.off_g = off;
      off = align256(off + size_t(q.g_parts) * size_t(q.vchunk) * q.ldg * q.elem);
    }
    if (q.need_dh_acc) { q.off_dhacc = off; off = align256(off + size_t(N) * H * sizeof(float)); }
    if (q.dh_kseg) {
      q.off_dhpart = off;
      off = align256(off + size_t(q.dh_segs) * size_t(N) * H * sizeof(float));
    }
    // the tokens gathered, the non-ignored ones first (see Plan::compact)
    q.compact = dtype == FLCE_BF16 && gather != 0;
    if (q.compact) {
      q.n_gather_blocks = ceil_div(N, kGatherBlock);
      q.off_idx = off;  off = align256(off + size_t(N) * sizeof(int32_t));
      q.off_yc = off;   off = align256(off + size_t(N) * sizeof(int64_t));
      q.off_bcnt = off; off = align256(off + size_t(q.n_gather_blocks) * sizeof(int32_t));
      q.off_hc = off;   off = align256(off + size_t(N) * H * q.elem);
    }
    off = carve_pad(q, off, backward);
  }
  q.total = off;
  *p = q;
  return true;
}

bool make_plan_nr(int64_t N, int64_t H, int64_t V, int dtype, int64_t token_chunk, Plan* p) {
  if (dtype != FLCE_BF16) return false;
  if (token_chunk < 0) token_chunk = 0;
  if (token_chunk > (int64_t(1) << 31)) return false;
  if (H <= 0) return false;
  const int64_t h_in = H;
  H = round_up(H, 8);                           // see Plan::pad_h
  Plan q;
  if (!make_plan(N, H, V, dtype, &q, false, -1, 0)) return false;
  q.h_in = h_in;
  q.pad_h = H != h_in;
  q.nr = true;
  q.backward = true;
  q.grad_dtype = dtype;
  q.grad_elem = q.elem;
  const int64_t nmax = round_up(N > 0 ? N : 1, q.tile);
  constexpr int64_t kDefaultChunk = 8192;
  int64_t nc = token_chunk > 0 ? round_up(token_chunk, q.tile)
                               : round_up(N < kDefaultChunk ? (N > 0 ? N : 1) : kDefaultChunk, q.tile);
  if (nc > nmax) nc = nmax;
  q.nc = nc;
  q.n_tok_chunks = ceil_div(N, nc);
  q.vp = round_up(V, q.tile);
  if (q.vp > kMaxLdBF16) return false;        // G row length: 32-bit tile offsets
  // per chunk: partials and per-token arrays for nc tokens; block sums for all N
  q.ld_part = nc;
  q.vchunk = q.vp;          // G row length
  q.n_chunks = 1;
  size_t off = 0;
  q.off_scalars = off; off = align256(off + sizeof(Scalars));
  if (N > 0) {
    q.off_part = off;  off = align256(off + size_t(q.n_voc_tiles) * q.ld_part * 2 * sizeof(float));
    q.off_zt = off;    off = align256(off + size_t(q.ld_part) * sizeof(float));
    q.off_lse = off;   off = align256(off + size_t(q.ld_part) * sizeof(float));
    q.off_tokloss = off;
    off = align256(off + size_t(q.n_loss_blocks) * 32 * sizeof(double));
    q.off_g = off;     off = align256(off + size_t(nc) * size_t(q.vp) * q.elem);
    // dH of a token chunk: M = its tokens, K = the whole vocabulary
    q.dh_kseg = dh_split(nc, H, V, &q.dh_segs);
    if (q.dh_kseg) {
      q.off_dhpart = off;
      off = align256(off + size_t(q.dh_segs) * size_t(nc) * H * sizeof(float));
    }
    // dW summed over several token chunks in float32, rounded to bf16 once
    // (the chunked path of Modalities PR 464, "What the reference
    // implementations do", keeps a float32 gradient accumulator)
    if (q.n_tok_chunks > 1) {
      q.need_dw_acc = true;
      q.off_dwacc = off;
      off = align256(off + size_t(V) * size_t(H) * sizeof(float));
    }
    // the tokens gathered, the non-ignored ones first; the token chunks run
    // over the gathered order, each with its live token counts (forward,
    // backward) computed on the device
    q.compact = true;
    q.n_gather_blocks = ceil_div(N, kGatherBlock);
    q.off_idx = off;  off = align256(off + size_t(N) * sizeof(int32_t));
    q.off_yc = off;   off = align256(off + size_t(N) * sizeof(int64_t));
    q.off_bcnt = off; off = align256(off + size_t(q.n_gather_blocks) * sizeof(int32_t));
    q.off_ccnt = off; off = align256(off + size_t(2 * q.n_tok_chunks) * sizeof(int64_t));
    q.off_hc = off;   off = align256(off + size_t(N) * H * q.elem);
    off = carve_pad(q, off, true);
  }
  q.off_dhacc = 0;
  q.need_dh_acc = false;
  q.total = off;
  *p = q;
  return true;
}

}  // namespace flce

extern "C" {

size_t flce_workspace_size(int64_t N, int64_t H, int64_t V, int dtype) {
  return flce_workspace_size_ex(N, H, V, dtype, dtype);
}

size_t flce_workspace_size_ex(int64_t N, int64_t H, int64_t V, int dtype, int grad_dtype) {
  flce::Plan p;
  if (!flce::make_plan(N, H, V, dtype, &p, true, grad_dtype)) return 0;
  return p.total;
}

int64_t flce_vocab_chunk(int64_t N, int64_t H, int64_t V, int dtype) {
  return flce_vocab_chunk_ex(N, H, V, dtype, dtype);
}

int64_t flce_vocab_chunk_ex(int64_t N, int64_t H, int64_t V, int dtype, int grad_dtype) {
  flce::Plan p;
  if (!flce::make_plan(N, H, V, dtype, &p, true, grad_dtype)) return 0;
  return p.vchunk;
}

int64_t flce_kept_chunks(int64_t N, int64_t H, int64_t V, int dtype, int accumulate_dW) {
  flce::Plan p;
  if (dtype != FLCE_BF16 || N <= 0 || !flce::make_plan(N, H, V, dtype, &p, true, dtype))
    return 0;
  return flce::gemm::kept_chunks(p, accumulate_dW == 0).n;
}

static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t flce_forward_workspace_size(int64_t N, int64_t H, int64_t V, int dtype) {
  flce::Plan p;
  if (!flce::make_plan(N, H, V, dtype, &p, false)) return 0;
  return p.total;
}

}  // extern "C"

namespace {

bool misaligned(const void* q, uintptr_t mask) { return (reinterpret_cast<uintptr_t>(q) & mask) != 0; }

// Checks shared by both entry points, in the order they are reported:
// argument errors, then unsupported layouts, then the workspace. dH and dW
// are NULL for the forward-only entry, which has no gradient outputs.
int check_common(const void* h, const void* W, const int64_t* labels, int64_t N, int64_t H,
                 int64_t V, float softcap, int reduction, int64_t num_label_tokens,
                 const float* loss, const int64_t* num_tokens, const void* dH, const void* dW,
                 int dtype, int grad_dtype, float mb_scale, const void* workspace,
                 size_t workspace_bytes, bool backward, int gather = -1,
                 const void* status = nullptr, const void* lse_out = nullptr,
                 size_t workspace_need = 0) {
  if (N < 0 || H <= 0 || V <= 0) return FLCE_ERR_ARG;
  if (dtype != FLCE_F32 && dtype != FLCE_BF16) return FLCE_ERR_ARG;
  if (grad_dtype != FLCE_F32 && grad_dtype != FLCE_BF16) return FLCE_ERR_ARG;
  if (dtype == FLCE_F32 && grad_dtype == FLCE_BF16) return FLCE_ERR_UNSUPPORTED;
  if (reduction != FLCE_SUM && reduction != FLCE_MEAN) return FLCE_ERR_ARG;
  if (!(softcap >= 0.0f) || !std::isfinite(softcap)) return FLCE_ERR_ARG;
  // the token-weighted micro-batch scale is a token fraction n_mb / n_total
  // (1.0 for 'sum'), so it is finite and never negative
  if (!std::isfinite(mb_scale) || !(mb_scale >= 0.0f)) return FLCE_ERR_ARG;
  if (reduction == FLCE_MEAN && num_label_tokens > 0) return FLCE_ERR_ARG;
  if (!loss || !num_tokens || !W) return FLCE_ERR_ARG;
  if (N > 0 && (!h || !labels)) return FLCE_ERR_ARG;
  if (backward && (!dW || (N > 0 && !dH))) return FLCE_ERR_ARG;
  flce::Plan p;
  if (!flce::make_plan(N, H, V, dtype, &p, backward, grad_dtype, gather)) return FLCE_ERR_ARG;
  const size_t es = p.elem, gs = p.grad_elem;
  if (backward) {
    if (overlaps(dH, size_t(N) * H * gs, h, size_t(N) * H * es)) return FLCE_ERR_ARG;
    if (overlaps(dW, size_t(V) * H * gs, W, size_t(V) * H * es)) return FLCE_ERR_ARG;
    if (overlaps(dH, size_t(N) * H * gs, dW, size_t(V) * H * gs)) return FLCE_ERR_ARG;
    if (overlaps(dH, size_t(N) * H * gs, W, size_t(V) * H * es)) return FLCE_ERR_ARG;
    if (overlaps(dW, size_t(V) * H * gs, h, size_t(N) * H * es)) return FLCE_ERR_ARG;
    // nor anything else the call reads or writes: dW holds intermediate values
    // from the forward on, before the labels, the scalars and the workspace
    // are done with
    const std::pair<const void*, size_t> other[] = {
        {labels, size_t(N) * sizeof(int64_t)}, {loss, sizeof(float)},
        {num_tokens, sizeof(int64_t)}, {status, sizeof(int32_t)},
        {lse_out, size_t(N) * sizeof(float)}, {workspace, workspace_bytes}};
    for (const auto& o : other)
      if (overlaps(dW, size_t(V) * H * gs, o.first, o.second) ||
          overlaps(dH, size_t(N) * H * gs, o.first, o.second))
        return FLCE_ERR_ARG;
  }
  const uintptr_t mask = dtype == FLCE_BF16 ? 15u : 3u;
  if (dtype == FLCE_BF16 && !flce::bf16_shape_ok(N, p.H, V)) return FLCE_ERR_UNSUPPORTED;
  if (misaligned(W, mask) || (N > 0 && misaligned(h, mask))) return FLCE_ERR_UNSUPPORTED;
  // the bf16 kernels write gradients in 16-byte (float32: 4 x 4-byte) runs
  const uintptr_t gmask = dtype == FLCE_BF16 ? 15u : 3u;
  if (backward && (misaligned(dW, gmask) || (N > 0 && misaligned(dH, gmask))))
    return FLCE_ERR_UNSUPPORTED;
  if (!workspace) return FLCE_ERR_WORKSPACE;
  if (misaligned(workspace, 255u)) return FLCE_ERR_WORKSPACE;
  if (workspace_bytes < (workspace_need ? workspace_need : p.total)) return FLCE_ERR_WORKSPACE;
  return FLCE_OK;
}

}  // namespace

int flce::check_grad_args(const void* h, const void* W, const int64_t* labels, int64_t N,
                          int64_t H, int64_t V, float softcap, int reduction,
                          int64_t num_label_tokens, const float* loss, const int64_t* num_tokens,
                          const void* dH, const void* dW, int dtype, float mb_scale,
                          const void* workspace, size_t workspace_bytes, const void* status,
                          const void* lse_out, size_t workspace_need) {
  return check_common(h, W, labels, N, H, V, softcap, reduction, num_label_tokens, loss,
                      num_tokens, dH, dW, dtype, dtype, mb_scale, workspace, workspace_bytes,
                      true, -1, status, lse_out, workspace_need);
}

extern "C" {

int flce_check_args(const void* h, const void* W, const int64_t* labels,
                    int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                    float softcap, int reduction, int64_t num_label_tokens,
                    float* loss, int64_t* num_tokens, void* dH, void* dW,
                    void* stream, int dtype, float mb_scale, int accumulate_dW,
                    void* workspace, size_t workspace_bytes, int32_t* status,
                    float* lse_out) {
  return flce_check_args_ex(h, W, labels, N, H, V, ignore_index, softcap, reduction,
                            num_label_tokens, loss, num_tokens, dH, dW, stream, dtype, mb_scale,
                            accumulate_dW, workspace, workspace_bytes, status, lse_out, dtype);
}

int flce_check_args_ex(const void* h, const void* W, const int64_t* labels,
                       int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                       float softcap, int reduction, int64_t num_label_tokens,
                       float* loss, int64_t* num_tokens, void* dH, void* dW,
                       void* stream, int dtype, float mb_scale, int accumulate_dW,
                       void* workspace, size_t workspace_bytes, int32_t* status,
                       float* lse_out, int grad_dtype) {
  (void)ignore_index; (void)stream; (void)accumulate_dW;
  return check_common(h, W, labels, N, H, V, softcap, reduction, num_label_tokens, loss,
                      num_tokens, dH, dW, dtype, grad_dtype, mb_scale, workspace,
                      workspace_bytes, true, -1, status, lse_out);
}

int flce_forward_check_args(const void* h, const void* W, const int64_t* labels,
                            int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                            float softcap, int reduction, int64_t num_label_tokens,
                            float* loss, int64_t* num_tokens, void* stream, int dtype,
                            float mb_scale, void* workspace, size_t workspace_bytes,
                            int32_t* status, float* lse_out) {
  (void)ignore_index; (void)stream; (void)status; (void)lse_out;
  return check_common(h, W, labels, N, H, V, softcap, reduction, num_label_tokens, loss,
                      num_tokens, nullptr, nullptr, dtype, dtype, mb_scale, workspace,
                      workspace_bytes, false);
}

int flce_forward_logits_check_args(const void* h, const void* W, const int64_t* labels,
                                   int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                                   float softcap, int reduction, int64_t num_label_tokens,
                                   float* loss, int64_t* num_tokens, void* stream, int dtype,
                                   float mb_scale, void* workspace, size_t workspace_bytes,
                                   int32_t* status, float* lse_out, void* logits,
                                   int64_t ld_logits, int logits_dtype) {
  (void)ignore_index; (void)stream;
  if (logits_dtype != FLCE_F32 && logits_dtype != FLCE_BF16) return FLCE_ERR_ARG;
  if (V > 0 && (ld_logits < V || ld_logits > (int64_t(1) << 31))) return FLCE_ERR_ARG;
  if (N > 0 && !logits) return FLCE_ERR_ARG;
  // the buffer's element count (N - 1) * ld + V stays below 2^60
  if (N > 0 && V > 0 && V <= (int64_t(1) << 31) &&
      N - 1 > ((int64_t(1) << 60) - V) / ld_logits)
    return FLCE_ERR_ARG;
  // the logits come out in the tokens' own order: this entry does not gather
  const int st = check_common(h, W, labels, N, H, V, softcap, reduction, num_label_tokens, loss,
                              num_tokens, nullptr, nullptr, dtype, dtype, mb_scale, workspace,
                              workspace_bytes, false, 0);
  if (st == FLCE_ERR_ARG) return st;            // sizes are valid from here on
  if (N > 0) {
    // the logits buffer, [N][ld_logits] up to its last stored element, is an
    // output of its own: it may overlap no input, no other output and no scratch
    const size_t es = logits_dtype == FLCE_BF16 ? 2 : 4;
    const size_t nl = (size_t(N - 1) * size_t(ld_logits) + size_t(V)) * es;
    const size_t ein = dtype == FLCE_BF16 ? 2 : 4;
    if (overlaps(logits, nl, h, size_t(N) * H * ein) ||
        overlaps(logits, nl, W, size_t(V) * H * ein) ||
        overlaps(logits, nl, labels, size_t(N) * sizeof(int64_t)) ||
        overlaps(logits, nl, loss, sizeof(float)) ||
        overlaps(logits, nl, num_tokens, sizeof(int64_t)) ||
        overlaps(logits, nl, status, sizeof(int32_t)) ||
        overlaps(logits, nl, lse_out, size_t(N) * sizeof(float)) ||
        overlaps(logits, nl, workspace, workspace_bytes))
      return FLCE_ERR_ARG;
    if (st == FLCE_OK || st == FLCE_ERR_WORKSPACE)
      if (misaligned(logits, es - 1)) return FLCE_ERR_UNSUPPORTED;
  }
  return st;
}

const char* flce_status_string(int s) {
  switch (s) {
    case FLCE_OK: return "FLCE_OK";
    case FLCE_ERR_ARG: return "FLCE_ERR_ARG: invalid argument";
    case FLCE_ERR_UNSUPPORTED: return "FLCE_ERR_UNSUPPORTED: unsupported shape or alignment";
    case FLCE_ERR_WORKSPACE: return "FLCE_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case FLCE_ERR_HIP: return "FLCE_ERR_HIP: HIP runtime error";
    case FLCE_ERR_LABEL: return "FLCE_ERR_LABEL: non-ignored label outside [0, V)";
    case FLCE_ERR_SCRATCH:
      return "FLCE_ERR_SCRATCH: the problem needs more than the fixed scratch of the "
             "no-allocation entry point";
    default: return "FLCE: unknown status";
  }
}

}  // extern "C"
