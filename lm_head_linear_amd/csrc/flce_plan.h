// Host-side problem plan for fused linear cross-entropy: tile counts, the
// backward vocabulary chunk and the carving of the caller's workspace.
// HIP-free so that it builds and is unit-tested on a machine without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>

namespace flce {

// Tile edge of the bf16 MFMA kernels (tokens x vocab and vocab/tokens x hidden).
constexpr int64_t kTileBF16 = 256;
// Tokens per workgroup of the gather of non-ignored tokens.
constexpr int64_t kGatherBlock = 1024;
// Tile edge of the float32 kernels.
constexpr int64_t kTileF32 = 64;
// Elements of one chunk of the logit gradient G^T: up to kChunkElems, or up
// to a sixteenth of the bytes of float32 logits (N V 4 / 16) when that is
// more, but never more than kMaxChunkElems. Larger chunks mean fewer passes
// over the float32 dH running sum.
constexpr int64_t kChunkElems = int64_t(1) << 27;
constexpr int64_t kMaxChunkElems = int64_t(1) << 29;
// The bf16 GEMMs address an operand tile with 32-bit byte offsets from the
// tile base: up to 255 rows of a K-contiguous operand, 2 * ld bytes apart.
// ld (H, or the no-recompute G row length) must keep that below 2^32.
constexpr int64_t kMaxLdBF16 = int64_t(1) << 22;
// Workgroups of one GEMM launch (256 x 256 tiles) must fit a grid dimension.
constexpr int64_t kMaxTiles = (int64_t(1) << 31) - 1;
// Split-K of the dH GEMM: when its M x Nn output has fewer than kSplitTiles
// tiles of 256 x 256 (half the CUs), its K (vocabulary rows) is split into
// up to kMaxSplits segments of at least kMinSplitK, one workgroup per
// (tile, segment), whose float32 partial products a fixed-order reduction
// then adds up.
constexpr int64_t kSplitTiles = 128;
constexpr int64_t kMaxSplits = 4;
constexpr int64_t kMinSplitK = 2048;

// The segment length (a multiple of 64) for a dH GEMM with an M x Nn output
// and K = k, or 0 when it is not split; *segs gets the segment count.
inline int64_t dh_split(int64_t M, int64_t Nn, int64_t k, int64_t* segs) {
  const int64_t tiles = ((M + 255) / 256) * ((Nn + 255) / 256);
  int64_t s = tiles > 0 ? 256 / tiles : 0;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s > k / kMinSplitK) s = k / kMinSplitK;
  if (tiles >= kSplitTiles || s < 2) { *segs = 1; return 0; }
  int64_t kseg = (k + s - 1) / s;
  kseg = (kseg + 63) / 64 * 64;
  *segs = (k + kseg - 1) / kseg;
  return *segs > 1 ? kseg : 0;
}

// Whether the bf16 shapes fit the kernels' index arithmetic.
inline bool bf16_shape_ok(int64_t N, int64_t H, int64_t V) {
  if (H > kMaxLdBF16) return false;
  const int64_t tn = (N + 255) / 256, tv = (V + 255) / 256, th = (H + 255) / 256;
  return tn * tv <= kMaxTiles && tn * th <= kMaxTiles && tv * th <= kMaxTiles;
}

// Scalars shared by the kernels of one call (first 256 bytes of the workspace).
struct Scalars {
  int64_t n_valid;    // non-ignored tokens
  int64_t n_bad;      // non-ignored tokens whose label is outside [0, V)
  double c64;         // loss = c64 * sum of per-token losses
  float c32;          // the same factor for the gradient epilogue
  int32_t pad0;
  double reserved[4];
};

struct Plan {
  int64_t N = 0, H = 0, V = 0;
  int dtype = 0;
  int grad_dtype = 0;        // dtype of dH and dW
  int g_parts = 1;           // 2: G kept as a bf16 hi + lo pair (float32 gradients)
  int64_t tile = 0;     // tile edge for this dtype
  int64_t n_tok_tiles = 0;   // ceil(N / tile)
  int64_t n_voc_tiles = 0;   // ceil(V / tile), forward partials per token
  int64_t ld_part = 0;       // tokens per partial row (multiple of tile)
  int64_t ldg = 0;           // leading dimension of G^T (tokens, multiple of 8)
  int64_t vchunk = 0;        // vocabulary rows per backward chunk
  int64_t n_chunks = 0;
  int64_t n_loss_blocks = 0; // blocks of 32 tokens of the fixed-order loss sum
  bool backward = true;      // plan includes the gradient buffers
  // No-recompute variant: tokens in chunks of `nc`; per chunk the forward
  // stores the probabilities relative to each tile's max, P'[t][v] bf16 with
  // row length `vp`, in the G buffer, which then becomes G in place.
  bool nr = false;
  int64_t nc = 0, n_tok_chunks = 0, vp = 0;
  bool need_dh_acc = false;  // float32 dH accumulator needed (bf16, >1 chunk)
  // No-recompute variant with several token chunks: dW is added up over the
  // chunks in a float32 [V][H] running sum at off_dwacc, rounded to bf16 once.
  bool need_dw_acc = false;
  // bf16 inputs (bf16 or float32 gradients): the tokens are gathered first,
  // the non-ignored ones in order and then the ignored ones (a permutation),
  // and the call runs over the gathered order: the backward over the first
  // n_valid (the kept tokens; an ignored token's G is zero, so its recompute,
  // dW and dH products are exact zeros), the forward over them too, or over
  // all N when per-token lse is asked for. The workspace then holds each
  // gathered token's original position (int32 [N]), label (int64 [N]) and
  // hidden row (bf16 [N][H]), and per-block counts of the gather (int32
  // [n_gather_blocks]); the partials, lse and target logits are indexed in
  // the gathered order, the per-token losses by original position.
  bool compact = false;
  int64_t n_gather_blocks = 0;
  // Split-K of the dH GEMM (bf16 gradients): segments of dh_kseg vocabulary
  // rows (0: not split), at most dh_segs of them per launch, each writing a
  // float32 [M][H] partial product at off_dhpart.
  int64_t dh_kseg = 0, dh_segs = 1;
  size_t elem = 0;           // bytes per element of h/W/G
  size_t grad_elem = 0;      // bytes per element of dH/dW
  // bf16 with a hidden size h_in that is not a multiple of 8 (the kernels
  // load and store 16-byte runs of a row): the call runs at the padded width
  // H = round_up(h_in, 8), on a zero-padded copy of W (off_wp), gathered rows
  // padded the same way (or, without the gather, a padded copy of h at
  // off_hp), and (with gradients) dW and dH computed at that width (off_dwp,
  // off_dhp) and copied out to the caller's h_in columns.
  int64_t h_in = 0;
  bool pad_h = false;
  size_t off_wp = 0, off_hp = 0, off_dwp = 0, off_dhp = 0;
  // byte offsets into the workspace
  size_t off_scalars = 0, off_part = 0, off_zt = 0, off_lse = 0, off_tokloss = 0,
         off_g = 0, off_dhacc = 0, off_dhpart = 0, off_dwacc = 0, off_idx = 0, off_yc = 0,
         off_hc = 0, off_bcnt = 0, off_ccnt = 0, total = 0;
};

// Builds the plan; returns false for invalid sizes or dtypes. A forward-only
// plan (backward = false) carves no logit-gradient chunk and no dH
// accumulator, so its workspace is the forward's alone. grad_dtype < 0 means
// the input dtype; float32 gradients for bf16 inputs keep G as a hi + lo pair
// of bf16 chunks (half as many vocabulary rows per chunk) and need no dH
// accumulator (dH itself is float32). bf16 gradients for float32 inputs are
// refused.
// `gather` (bf16 only): gather the non-ignored tokens first (see
// Plan::compact); < 0 means the default, which gathers for a forward-only
// plan and for bf16 gradients. The logits-returning forward and the
// allocation-free one do not gather.
bool make_plan(int64_t N, int64_t H, int64_t V, int dtype, Plan* p, bool backward = true,
               int grad_dtype = -1, int gather = -1);

// Plan of the no-recompute variant (bf16 only): token chunks of
// `token_chunk` tokens (rounded up to the tile; <= 0: min(N, 8192) rounded
// up), each with a [nc][roundup(V, 256)] bf16 buffer of probabilities that
// becomes that chunk's G, and with more than one chunk a float32 [V][H]
// running sum of dW.
bool make_plan_nr(int64_t N, int64_t H, int64_t V, int dtype, int64_t token_chunk, Plan* p);

// The synchronous checks of the entry points with gradients (dtype gradients),
// the workspace required to hold workspace_need bytes (0: the recompute
// plan's size) instead of the recompute plan's: used by the no-recompute
// variant, whose workspace differs.
int check_grad_args(const void* h, const void* W, const int64_t* labels, int64_t N, int64_t H,
                    int64_t V, float softcap, int reduction, int64_t num_label_tokens,
                    const float* loss, const int64_t* num_tokens, const void* dH, const void* dW,
                    int dtype, float mb_scale, const void* workspace, size_t workspace_bytes,
                    const void* status, const void* lse_out, size_t workspace_need);

}  // namespace flce
