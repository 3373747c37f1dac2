// Small kernels shared by both dtypes: label scan, log-sum-exp merge with the
// per-token loss, the deterministic float64 loss sum, and fills.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/flce.h"
#include "flce_internal.h"

namespace flce {
namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;

// One workgroup counts the non-ignored tokens (exact integers) and the
// non-ignored labels outside [0, V), then fixes the loss/gradient scale c:
//   'sum'  : mb_scale / T if T > 0, else mb_scale
//   'mean' : mb_scale / max(n, 1)   (empty target set -> loss 0, not NaN)
// and num_tokens = n for 'sum', 0 for 'mean'.
__global__ __launch_bounds__(1024) void k_label_scan(
    const int64_t* __restrict__ labels, int64_t N, int64_t V, int64_t ignore_index,
    int reduction, int64_t T, float mb_scale, Scalars* __restrict__ sc,
    int64_t* __restrict__ num_tokens, int32_t* __restrict__ status) {
  __shared__ long long s_valid[16], s_bad[16];
  long long nv = 0, nb = 0;
  for (int64_t i = threadIdx.x; i < N; i += blockDim.x) {
    const int64_t y = labels[i];
    const bool valid = y != ignore_index;
    nv += valid ? 1 : 0;
    nb += (valid && (y < 0 || y >= V)) ? 1 : 0;
  }
  for (int off = 32; off > 0; off >>= 1) {
    nv += __shfl_xor(nv, off);
    nb += __shfl_xor(nb, off);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { s_valid[w] = nv; s_bad[w] = nb; }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long n = 0, bad = 0;
    for (int i = 0; i < int(blockDim.x >> 6); ++i) { n += s_valid[i]; bad += s_bad[i]; }
    double c;
    if (reduction == FLCE_SUM) c = T > 0 ? double(mb_scale) / double(T) : double(mb_scale);
    else c = double(mb_scale) / double(n > 1 ? n : 1);
    sc->n_valid = n;
    sc->n_bad = bad;
    sc->c64 = c;
    sc->c32 = float(c);
    *num_tokens = reduction == FLCE_SUM ? n : 0;
    if (status) *status = bad ? FLCE_ERR_LABEL : FLCE_OK;
  }
}

// Per token: merge the per-vocab-tile (max m_j, sum_j of exp(x - m_j))
// partials into lse = M + log(sum_j s_j exp(m_j - M)) and form the token
// loss lse - z'_target on non-ignored tokens (NaN for an out-of-range label,
// 0 on ignored ones), written in float64 at the token's original position
// (perm[t], or t without a gather). A block handles kMergeTokens tokens; its
// 8 thread groups each merge every 8th tile of them (online max/rescale),
// then the groups are combined in a fixed order. With `count` (a device
// count) only the first *count tokens are merged.
constexpr int kMergeTokens = 32;

__global__ __launch_bounds__(256) void k_lse_merge(
    const float2* __restrict__ part, int64_t n_tiles, int64_t ld_part,
    const float* __restrict__ zt, const int64_t* __restrict__ labels, int64_t N,
    const int64_t* __restrict__ count, int64_t V, int64_t ignore_index,
    float* __restrict__ lse, float* __restrict__ lse_out, double* __restrict__ tok_loss,
    const int32_t* __restrict__ perm) {
  __shared__ float2 grp[8][kMergeTokens];
  if (count) {
    const int64_t c = *count;
    N = c < N ? c : N;
  }
  if (int64_t(blockIdx.x) * kMergeTokens >= N) return;
  const int tk = threadIdx.x % kMergeTokens, g = threadIdx.x / kMergeTokens;
  const int64_t t = int64_t(blockIdx.x) * kMergeTokens + tk;
  float M = -INFINITY, S = 0.f;
  auto merge = [&](float2 q) {
    if (q.x > M) {
      S = (M == -INFINITY ? 0.f : S * exp2f((M - q.x) * kLog2e)) + q.y;
      M = q.x;
    } else {
      S += q.y * exp2f((q.x - M) * kLog2e);
    }
  };
  if (t < N) {
    // tiles g, g + 8, ... in order; four loads in flight before they are merged
    int64_t j = g;
    for (; j + 24 < n_tiles; j += 32) {
      float2 q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) q[u] = part[(j + 8 * u) * ld_part + t];
#pragma unroll
      for (int u = 0; u < 4; ++u) merge(q[u]);
    }
    for (; j < n_tiles; j += 8) merge(part[j * ld_part + t]);
  }
  grp[g][tk] = make_float2(M, S);
  __syncthreads();
  if (g == 0 && t < N) {
    float Mx = -INFINITY;
    for (int i = 0; i < 8; ++i) Mx = fmaxf(Mx, grp[i][tk].x);
    float St = 0.f;
    for (int i = 0; i < 8; ++i)
      if (grp[i][tk].x != -INFINITY) St += grp[i][tk].y * exp2f((grp[i][tk].x - Mx) * kLog2e);
    const float l = Mx + log2f(St) * kLn2;
    const int64_t orig = perm ? int64_t(perm[t]) : t;
    lse[t] = l;
    if (lse_out) lse_out[orig] = l;
    const int64_t y = labels[t];
    double ell = 0.0;
    if (y != ignore_index) ell = (y < 0 || y >= V) ? double(NAN) : double(l) - double(zt[t]);
    tok_loss[orig] = ell;
  }
}

// loss = c * (sum of the per-token losses) in float64, in a fixed order that
// depends only on the original token positions: blocks of 32 tokens summed
// in order, the block sums strided over 256 threads, then a tree. NaN when a
// label was invalid.
__global__ __launch_bounds__(256) void k_loss_final(const double* __restrict__ tok_loss,
                                                    int64_t N, const Scalars* __restrict__ sc,
                                                    float* __restrict__ loss) {
  __shared__ double red[256];
  const int64_t nb = (N + kMergeTokens - 1) / kMergeTokens;
  double s = 0.0;
  for (int64_t b = threadIdx.x; b < nb; b += 256) {
    double sb = 0.0;
    for (int i = 0; i < kMergeTokens; ++i) {
      const int64_t t = b * kMergeTokens + i;
      sb += t < N ? tok_loss[t] : 0.0;
    }
    s += sb;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (int(threadIdx.x) < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = sc->n_bad ? NAN : float(sc->c64 * red[0]);
}

__global__ void k_empty(float* loss, int64_t* num_tokens, int32_t* status) {
  *loss = 0.f;
  *num_tokens = 0;
  if (status) *status = FLCE_OK;
}

__global__ __launch_bounds__(256) void k_zero16(uint4* __restrict__ p, int64_t n16) {
  const uint4 z = {0u, 0u, 0u, 0u};
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += int64_t(gridDim.x) * 256)
    p[i] = z;
}

__global__ __launch_bounds__(256) void k_zero1(unsigned char* __restrict__ p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    p[i] = 0;
}

// ---- the tokens gathered, the non-ignored ones first ----------------------
// Ignored tokens have G = 0: their recomputed logits, dW and dH products are
// exact zeros, so the call runs over the gathered order, the kept tokens
// first. Block b of kGatherBlock tokens first counts its kept tokens; then
// every block finds the count before it and each token's rank (wave
// ballots): a kept token goes to its rank among the kept ones, an ignored
// one to n_valid plus its rank among the ignored ones. The hidden rows follow
// in a copy kernel.
constexpr int kGatherThreads = int(kGatherBlock);

__global__ __launch_bounds__(kGatherThreads) void k_gather_count(
    const int64_t* __restrict__ labels, int64_t N, int64_t ignore_index,
    int32_t* __restrict__ bcnt) {
  __shared__ int32_t wsum[kGatherThreads / 64];
  const int64_t t = int64_t(blockIdx.x) * kGatherThreads + threadIdx.x;
  const bool keep = t < N && labels[t] != ignore_index;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned long long m = __ballot(keep);
  if (lane == 0) wsum[w] = __popcll(m);
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t s = 0;
    for (int i = 0; i < kGatherThreads / 64; ++i) s += wsum[i];
    bcnt[blockIdx.x] = s;
  }
}

__global__ __launch_bounds__(kGatherThreads) void k_gather_tokens(
    const int64_t* __restrict__ labels, int64_t N, int64_t ignore_index,
    const int32_t* __restrict__ bcnt, const Scalars* __restrict__ sc,
    int32_t* __restrict__ idx, int64_t* __restrict__ yc, double* __restrict__ tok_loss) {
  __shared__ int64_t part[kGatherThreads / 64];
  __shared__ int32_t wsum[kGatherThreads / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // kept tokens of the blocks before this one
  int64_t s = 0;
  for (int64_t i = threadIdx.x; i < blockIdx.x; i += kGatherThreads) s += bcnt[i];
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) part[w] = s;
  const int64_t t = int64_t(blockIdx.x) * kGatherThreads + threadIdx.x;
  const int64_t y = t < N ? labels[t] : ignore_index;
  const bool keep = t < N && y != ignore_index;
  const unsigned long long m = __ballot(keep);
  if (lane == 0) wsum[w] = __popcll(m);
  __syncthreads();
  if (t >= N) return;
  int64_t before = __popcll(m & ((1ull << lane) - 1));       // kept tokens before t
  for (int i = 0; i < kGatherThreads / 64; ++i) before += part[i] + (i < w ? wsum[i] : 0);
  const int64_t pos = keep ? before : sc->n_valid + (t - before);
  idx[pos] = int32_t(t);
  yc[pos] = y;
  if (!keep) tok_loss[t] = 0.0;           // not merged when the forward skips it
}

// The label scan and the token gather in one workgroup, for N up to
// kScanGatherMax tokens (one launch instead of three). In a pass of kScanPass
// tokens every thread counts a group of kScanPer consecutive ones (their
// flags staged in LDS from coalesced loads), so a pass needs one exclusive
// scan over the workgroup of the groups' counts: the kept tokens in the low
// 32 bits, the kept ones with a label outside [0, V) in the high 32 (neither
// sum reaches 2^32). With more than one pass, a first sweep counts the
// tokens for the totals. From the totals it fixes the scale c and num_tokens
// as k_label_scan does, and it places each token as k_gather_tokens does: a
// kept one at its rank among the kept ones, an ignored one at n_valid plus
// its rank among the ignored ones.
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 8;
constexpr int64_t kScanPass = int64_t(kScanThreads) * kScanPer;
constexpr int64_t kScanGatherMax = 8 * kScanPass;
constexpr uint64_t kLow32 = 0xffffffffull;

// Exclusive prefix sum over the workgroup of x (one value per thread) and the
// total, through the 16 wave sums in `wsum`.
__device__ __forceinline__ uint64_t block_exclusive_scan(uint64_t x, uint64_t* wsum,
                                                         uint64_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint64_t inc = x;
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  uint64_t before = 0, all = 0;
  for (int i = 0; i < kScanThreads / 64; ++i) {
    before += i < w ? wsum[i] : 0;
    all += wsum[i];
  }
  __syncthreads();                                 // wsum is reused by the next scan
  *total = all;
  return before + inc - x;
}

__global__ __launch_bounds__(kScanThreads) void k_scan_gather(
    const int64_t* __restrict__ labels, int64_t N, int64_t V, int64_t ignore_index,
    int reduction, int64_t T, float mb_scale, Scalars* __restrict__ sc,
    int64_t* __restrict__ num_tokens, int32_t* __restrict__ status, int32_t* __restrict__ idx,
    int64_t* __restrict__ yc, double* __restrict__ tok_loss) {
  __shared__ uint64_t wsum[kScanThreads / 64];
  // a pass's flags in token order (bit 0 kept, bit 1 a kept one with a bad
  // label), and per group of kScanPer tokens its kept mask and the kept
  // tokens of the pass before it: loads and stores run in token order across
  // the threads (coalesced), the scan over the groups
  __shared__ __attribute__((aligned(16))) unsigned char flag[kScanPass];
  __shared__ unsigned char gmask[kScanThreads];
  __shared__ uint32_t gpref[kScanThreads];
  const int tid = threadIdx.x;
  const bool one_pass = N <= kScanPass;
  uint64_t totals = 0;                             // kept | bad << 32, all tokens
  if (!one_pass) {
    uint64_t c = 0;
    for (int64_t t = tid; t < N; t += kScanThreads) {
      const int64_t y = labels[t];
      if (y != ignore_index) c += (y < 0 || y >= V) ? (uint64_t(1) << 32) + 1 : 1;
    }
    block_exclusive_scan(c, wsum, &totals);
  }
  int64_t kept_before_pass = 0;
  for (int64_t p0 = 0; p0 < N; p0 += kScanPass) {
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) {
      const int64_t t = p0 + u * kScanThreads + tid;
      const int64_t y = t < N ? labels[t] : ignore_index;
      flag[u * kScanThreads + tid] = y != ignore_index ? ((y < 0 || y >= V) ? 3 : 1) : 0;
    }
    __syncthreads();
    // group tid: tokens p0 + kScanPer tid ...
    const uint2 f8 = *reinterpret_cast<const uint2*>(flag + tid * kScanPer);
    unsigned keep = 0;
    uint64_t c = 0;
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) {
      const unsigned fu = ((u < 4 ? f8.x : f8.y) >> (8 * (u & 3))) & 0xffu;
      keep |= (fu & 1u) << u;
      c += (fu & 1u) + (uint64_t(fu >> 1) << 32);
    }
    uint64_t pass_totals = 0;
    const uint64_t before = block_exclusive_scan(c, wsum, &pass_totals);
    gmask[tid] = (unsigned char)keep;
    gpref[tid] = uint32_t(before & kLow32);
    if (one_pass) totals = pass_totals;
    const int64_t n = int64_t(totals & kLow32);
    __syncthreads();
    // token p0 + i, i = u kScanThreads + tid: its rank among the kept ones
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) {
      const int i = u * kScanThreads + tid;
      const int64_t t = p0 + i;
      if (t < N) {
        const int g = i / kScanPer, r = i % kScanPer;
        const bool k = flag[i] & 1u;
        const int64_t kept = kept_before_pass + gpref[g] + __builtin_popcount(gmask[g] & ((1u << r) - 1u));
        const int64_t pos = k ? kept : n + (t - kept);
        idx[pos] = int32_t(t);
        yc[pos] = labels[t];
        if (!k) tok_loss[t] = 0.0;        // not merged when the forward skips it
      }
    }
    kept_before_pass += int64_t(pass_totals & kLow32);
    __syncthreads();                               // the staging is rewritten by the next pass
  }
  if (tid == 0) {
    const int64_t n = int64_t(totals & kLow32), bad = int64_t(totals >> 32);
    double c;
    if (reduction == FLCE_SUM) c = T > 0 ? double(mb_scale) / double(T) : double(mb_scale);
    else c = double(mb_scale) / double(n > 1 ? n : 1);
    sc->n_valid = n;
    sc->n_bad = bad;
    sc->c64 = c;
    sc->c32 = float(c);
    *num_tokens = reduction == FLCE_SUM ? n : 0;
    if (status) *status = bad ? FLCE_ERR_LABEL : FLCE_OK;
  }
}

// The dH rows (g16 16-byte pieces each) of the ignored tokens, gathered rows
// n_valid .. N-1, zeroed: the compact backward never writes them. Grid-stride
// over the launch.
__device__ __forceinline__ void zero_ignored_rows(const int32_t* __restrict__ idx, int64_t N,
                                                  const Scalars* __restrict__ sc, int64_t g16,
                                                  uint4* __restrict__ dH) {
  if (!dH) return;
  const int64_t kept = sc->n_valid;
  const int64_t total = (N - kept) * g16;
  const uint4 z = {0u, 0u, 0u, 0u};
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * 256) {
    const int64_t r = i / g16;
    dH[int64_t(idx[kept + r]) * g16 + (i - r * g16)] = z;
  }
}

// hc[r] = h[idx[r]] for the first `rows` gathered rows (*rows_dev, or all
// N), in 16-byte pieces (h8 per row); then the dH rows of the ignored tokens
// zeroed (dH null: no gradients).
__global__ __launch_bounds__(256) void k_gather_rows(const uint4* __restrict__ h, int64_t h8,
                                                     const int32_t* __restrict__ idx,
                                                     const int64_t* __restrict__ rows_dev,
                                                     int64_t rows, uint4* __restrict__ hc,
                                                     const Scalars* __restrict__ sc,
                                                     int64_t g16, uint4* __restrict__ dH) {
  const int64_t total = (rows_dev ? *rows_dev : rows) * h8;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * 256) {
    const int64_t r = i / h8;
    hc[i] = h[int64_t(idx[r]) * h8 + (i - r * h8)];
  }
  zero_ignored_rows(idx, rows, sc, g16, dH);
}

// k_gather_rows for hidden rows of h_in bf16 values (h_in % 8 != 0), stored
// at the padded width hp with the pad columns zero.
__global__ __launch_bounds__(256) void k_gather_rows_pad(const uint16_t* __restrict__ h,
                                                         int64_t h_in, int64_t hp,
                                                         const int32_t* __restrict__ idx,
                                                         const int64_t* __restrict__ rows_dev,
                                                         int64_t rows, uint16_t* __restrict__ hc,
                                                         const Scalars* __restrict__ sc,
                                                         int64_t g16, uint4* __restrict__ dH) {
  const int64_t total = (rows_dev ? *rows_dev : rows) * hp;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * 256) {
    const int64_t r = i / hp, c = i - r * hp;
    hc[i] = c < h_in ? h[int64_t(idx[r]) * h_in + c] : uint16_t(0);
  }
  zero_ignored_rows(idx, rows, sc, g16, dH);
}

// Row copy between widths: row r of dst (stride ld_dst) gets the first `cols`
// elements of row r of src (stride ld_src) and zeros up to `width`.
template <class T>
__global__ __launch_bounds__(256) void k_copy_rows(const T* __restrict__ src, int64_t ld_src,
                                                   T* __restrict__ dst, int64_t ld_dst,
                                                   int64_t rows, int64_t cols, int64_t width) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y)
    for (int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x; c < width;
         c += int64_t(gridDim.x) * 256)
      dst[r * ld_dst + c] = c < cols ? src[r * ld_src + c] : T(0);
}

// Live tokens of each chunk of nc gathered rows: cnt[c] for the forward (the
// first `fwd` gathered rows: the kept ones, or all), cnt[nch + c] for the
// backward (the kept ones).
__global__ void k_chunk_counts(const Scalars* __restrict__ sc, int64_t N, int all, int64_t nc,
                               int64_t nch, int64_t* __restrict__ cnt) {
  const int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (c >= nch) return;
  const int64_t kept = sc->n_valid, fwd = all ? N : kept;
  auto clamp = [&](int64_t x) { return x < 0 ? int64_t(0) : (x > nc ? nc : x); };
  cnt[c] = clamp(fwd - c * nc);
  cnt[nch + c] = clamp(kept - c * nc);
}

}  // namespace

hipError_t launch_empty(const Plan&, const Args& a, const Launcher& L) {
  L.pre(kFill);
  hipLaunchKernelGGL(k_empty, dim3(1), dim3(1), 0, L.stream, a.loss, a.num_tokens, a.status);
  L.post(kFill);
  return hipGetLastError();
}

hipError_t launch_label_scan(const Plan& p, const Args& a, const Launcher& L) {
  L.pre(kLabelScan);
  hipLaunchKernelGGL(k_label_scan, dim3(1), dim3(1024), 0, L.stream, a.labels, p.N, p.V,
                     a.ignore_index, a.reduction, a.num_label_tokens, a.mb_scale, a.sc,
                     a.num_tokens, a.status);
  L.post(kLabelScan);
  return hipGetLastError();
}

hipError_t launch_merge(const Plan& p, const Args& a, int64_t t0, int64_t nt, const Launcher& L) {
  L.pre(kLseMerge);
  hipLaunchKernelGGL(k_lse_merge, dim3(unsigned((nt + kMergeTokens - 1) / kMergeTokens)), dim3(256),
                     0, L.stream, a.part, p.n_voc_tiles, p.ld_part, a.zt, a.labels + t0, nt,
                     nullptr, p.V, a.ignore_index, a.lse, a.lse_out ? a.lse_out + t0 : nullptr,
                     a.tok_loss + t0, nullptr);
  L.post(kLseMerge);
  return hipGetLastError();
}

hipError_t launch_chunk_counts(const Plan& p, const Args& a, bool all_rows, const Launcher& L) {
  L.pre(kGather);
  hipLaunchKernelGGL(k_chunk_counts, dim3(unsigned((p.n_tok_chunks + 63) / 64)), dim3(64), 0,
                     L.stream, a.sc, p.N, all_rows ? 1 : 0, p.nc, p.n_tok_chunks, a.ccnt);
  L.post(kGather);
  return hipGetLastError();
}

hipError_t launch_merge_gathered(const Plan& p, const Args& a, int64_t t0, int64_t nt,
                                 const int64_t* count, const Launcher& L) {
  L.pre(kLseMerge);
  hipLaunchKernelGGL(k_lse_merge, dim3(unsigned((nt + kMergeTokens - 1) / kMergeTokens)), dim3(256),
                     0, L.stream, a.part, p.n_voc_tiles, p.ld_part, a.zt, a.yc + t0, nt, count,
                     p.V, a.ignore_index, a.lse, a.lse_out, a.tok_loss, a.idx + t0);
  L.post(kLseMerge);
  return hipGetLastError();
}

hipError_t launch_merge_and_loss(const Plan& p, const Args& a, const Launcher& L) {
  hipError_t e;
  if (p.compact) {
    // over the gathered order: the kept tokens (or all when the per-token
    // lse is asked for), losses and lse scattered to the original positions
    L.pre(kLseMerge);
    hipLaunchKernelGGL(k_lse_merge, dim3(unsigned((p.N + kMergeTokens - 1) / kMergeTokens)),
                       dim3(256), 0, L.stream, a.part, p.n_voc_tiles, p.ld_part, a.zt, a.yc, p.N,
                       a.lse_out ? nullptr : &a.sc->n_valid, p.V, a.ignore_index, a.lse,
                       a.lse_out, a.tok_loss, a.idx);
    L.post(kLseMerge);
    e = hipGetLastError();
  } else {
    e = launch_merge(p, a, 0, p.N, L);
  }
  if (e != hipSuccess) return e;
  return launch_loss_final(p, a, L);
}

hipError_t launch_loss_final(const Plan& p, const Args& a, const Launcher& L) {
  L.pre(kLossFinal);
  hipLaunchKernelGGL(k_loss_final, dim3(1), dim3(256), 0, L.stream, a.tok_loss, p.N, a.sc,
                     a.loss);
  L.post(kLossFinal);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const void* src, int64_t ld_src, void* dst, int64_t ld_dst,
                            int64_t rows, int64_t cols, int64_t width, size_t elem,
                            const Launcher& L) {
  if (rows <= 0 || width <= 0) return hipSuccess;
  if (elem != 2 && elem != 4) return hipErrorInvalidValue;
  const int64_t gx = (width + 255) / 256;
  const dim3 grid(unsigned(gx < 64 ? gx : 64), unsigned(rows < 16384 ? rows : 16384));
  L.pre(kPadCopy);
  if (elem == 2)
    hipLaunchKernelGGL(k_copy_rows<uint16_t>, grid, dim3(256), 0, L.stream,
                       static_cast<const uint16_t*>(src), ld_src, static_cast<uint16_t*>(dst),
                       ld_dst, rows, cols, width);
  else
    hipLaunchKernelGGL(k_copy_rows<uint32_t>, grid, dim3(256), 0, L.stream,
                       static_cast<const uint32_t*>(src), ld_src, static_cast<uint32_t*>(dst),
                       ld_dst, rows, cols, width);
  L.post(kPadCopy);
  return hipGetLastError();
}

hipError_t launch_zero_bytes(void* ptr, size_t bytes, const Launcher& L) {
  if (bytes == 0) return hipSuccess;
  L.pre(kFill);
  if ((reinterpret_cast<uintptr_t>(ptr) & 15u) == 0 && (bytes & 15u) == 0) {
    const int64_t n16 = int64_t(bytes / 16);
    int64_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_zero16, dim3(unsigned(blocks)), dim3(256), 0, L.stream,
                       reinterpret_cast<uint4*>(ptr), n16);
  } else {
    int64_t blocks = (int64_t(bytes) + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_zero1, dim3(unsigned(blocks)), dim3(256), 0, L.stream,
                       reinterpret_cast<unsigned char*>(ptr), int64_t(bytes));
  }
  L.post(kFill);
  return hipGetLastError();
}

hipError_t launch_scan_gather(const Plan& p, const Args& a, bool all_rows, const Launcher& L) {
  if (p.N <= kScanGatherMax) {
    L.pre(kLabelScan);
    hipLaunchKernelGGL(k_scan_gather, dim3(1), dim3(kScanThreads), 0, L.stream, a.labels, p.N,
                       p.V, a.ignore_index, a.reduction, a.num_label_tokens, a.mb_scale, a.sc,
                       a.num_tokens, a.status, a.idx, a.yc, a.tok_loss);
    L.post(kLabelScan);
  } else {
    const hipError_t e = launch_label_scan(p, a, L);
    if (e != hipSuccess) return e;
    const unsigned nb = unsigned(p.n_gather_blocks);
    L.pre(kGather);
    hipLaunchKernelGGL(k_gather_count, dim3(nb), dim3(kGatherThreads), 0, L.stream, a.labels,
                       p.N, a.ignore_index, a.bcnt);
    hipLaunchKernelGGL(k_gather_tokens, dim3(nb), dim3(kGatherThreads), 0, L.stream, a.labels,
                       p.N, a.ignore_index, a.bcnt, a.sc, a.idx, a.yc, a.tok_loss);
    L.post(kGather);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the hidden rows, then the dH rows of the ignored tokens zeroed
  const int64_t* rows_dev = all_rows ? nullptr : &a.sc->n_valid;
  const int64_t g16 = a.dH ? p.H * int64_t(p.grad_elem) / 16 : 0;   // 16-byte pieces per dH row
  uint4* dH = static_cast<uint4*>(a.dH);
  L.pre(kGather);
  if (p.pad_h) {
    int64_t blocks = (p.N * p.H + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_gather_rows_pad, dim3(unsigned(blocks)), dim3(256), 0, L.stream,
                       static_cast<const uint16_t*>(a.h), p.h_in, p.H, a.idx, rows_dev, p.N,
                       static_cast<uint16_t*>(a.hc), a.sc, g16, dH);
  } else {
    const int64_t h8 = p.H / 8;
    int64_t blocks = (p.N * h8 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_gather_rows, dim3(unsigned(blocks)), dim3(256), 0, L.stream,
                       static_cast<const uint4*>(a.h), h8, a.idx, rows_dev, p.N,
                       static_cast<uint4*>(a.hc), a.sc, g16, dH);
  }
  L.post(kGather);
  return hipGetLastError();
}

}  // namespace flce
