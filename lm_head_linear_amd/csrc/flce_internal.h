// Internal launch interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "flce_plan.h"

namespace flce {

// Kernel kinds, for per-kernel timing.
enum Kind : int {
  kLabelScan = 0,
  kLseFwd = 1,
  kLseMerge = 2,
  kLossFinal = 3,
  kGradLogits = 4,
  kGemmDW = 5,
  kGemmDH = 6,
  kFill = 7,
  kProbsToGrad = 8,
  kDhReduce = 9,
  kGather = 10,
  kGemmDWDH = 11,     // dH's tiles and then dW's, in one grid
  kPadCopy = 12,      // row copies of a call at a padded hidden width
  kNumKinds = 13,
};

// Everything one call needs on the device side.
struct Args {
  const void* h;
  const void* W;
  const int64_t* labels;
  int64_t N, H, V;
  int64_t ignore_index;
  float softcap;
  int reduction;
  int64_t num_label_tokens;
  float* loss;
  int64_t* num_tokens;
  void* dH;
  void* dW;
  float mb_scale;
  int accumulate_dW;
  int32_t* status;
  float* lse_out;
  // optional logits output of the forward: [N][ld_logits], FLCE_F32 or FLCE_BF16
  void* logits;
  int64_t ld_logits;
  int logits_dtype;
  // carved workspace
  Scalars* sc;
  float2* part;
  float* zt;
  float* lse;
  double* tok_loss;  // [N] per-token loss by original position (summed in order)
  void* g;        // G^T chunk [vchunk][ldg]
  float* dh_acc;  // [N][H] (bf16 path with several chunks)
  float* dh_part; // [dh_segs][M][H] split-K partial products of dH (or null)
  float* dw_acc;  // [V][H] float32 dW running sum (no-recompute, several chunks)
  // compact plan: the tokens gathered, non-ignored ones first (see Plan)
  int32_t* idx;   // original position of gathered token r
  int64_t* yc;    // its label
  int32_t* bcnt;  // kept tokens per gather block
  void* hc;       // its hidden row, bf16 [N][H]
  int64_t* ccnt;  // no-recompute variant: live tokens of each token chunk, for
                  // the forward ([n_tok_chunks]) and then for the backward
};

// Launch hook: the C-ABI layer brackets launches with timing events.
struct Launcher {
  hipStream_t stream;
  void (*before)(int kind, hipStream_t s);
  void (*after)(int kind, hipStream_t s);
  void pre(int kind) const { if (before) before(kind, stream); }
  void post(int kind) const { if (after) after(kind, stream); }
};

// Common kernels (dtype independent).
hipError_t launch_empty(const Plan& p, const Args& a, const Launcher& L);
hipError_t launch_label_scan(const Plan& p, const Args& a, const Launcher& L);
hipError_t launch_merge_and_loss(const Plan& p, const Args& a, const Launcher& L);
// The merge for tokens [t0, t0 + nt) (t0 a multiple of 32), and the final
// loss sum over all tokens' blocks.
hipError_t launch_merge(const Plan& p, const Args& a, int64_t t0, int64_t nt, const Launcher& L);
hipError_t launch_loss_final(const Plan& p, const Args& a, const Launcher& L);
hipError_t launch_zero_bytes(void* ptr, size_t bytes, const Launcher& L);
// rows x width elements of `elem` bytes (2 or 4) at dst (row stride ld_dst):
// the first `cols` of each row from src (row stride ld_src), the rest zero.
hipError_t launch_copy_rows(const void* src, int64_t ld_src, void* dst, int64_t ld_dst,
                            int64_t rows, int64_t cols, int64_t width, size_t elem,
                            const Launcher& L);
// Compact plan, first on the stream: the label scan (as launch_label_scan),
// then the tokens gathered, the non-ignored ones first (positions, labels,
// the hidden rows of the first `rows` of them: the kept ones, or all N),
// ignored tokens given a zero loss and their dH rows zeroed (a.dH non-null).
hipError_t launch_scan_gather(const Plan& p, const Args& a, bool all_rows, const Launcher& L);
// No-recompute variant after the gather: the live tokens of every token chunk
// of nc gathered rows, for the forward (all N, or the kept ones) and for the
// backward (the kept ones).
hipError_t launch_chunk_counts(const Plan& p, const Args& a, bool all_rows, const Launcher& L);
// The merge of a gathered token chunk: tokens [t0, t0 + *count) of the
// gathered order, losses and lse_out scattered to original positions.
hipError_t launch_merge_gathered(const Plan& p, const Args& a, int64_t t0, int64_t nt,
                                 const int64_t* count, const Launcher& L);

// bf16 MFMA path.
hipError_t bf16_forward(const Plan& p, const Args& a, const Launcher& L);
hipError_t bf16_backward_chunk(const Plan& p, const Args& a, int64_t chunk, const Launcher& L);
// No-recompute variant, token chunk c: the forward that keeps the
// probabilities, then (after the chunk's merge) G in place and dW, dH.
hipError_t bf16_nr_forward_chunk(const Plan& p, const Args& a, int64_t c, const Launcher& L);
hipError_t bf16_nr_backward_chunk(const Plan& p, const Args& a, int64_t c, const Launcher& L);

// float32 path.
hipError_t f32_forward(const Plan& p, const Args& a, const Launcher& L);
hipError_t f32_backward_chunk(const Plan& p, const Args& a, int64_t chunk, const Launcher& L);

}  // namespace flce
