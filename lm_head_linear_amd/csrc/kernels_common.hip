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
// partials into lse = M + log(sum_j s_j exp(m_j - M)), form the token loss
// lse - z'_target on non-ignored tokens (NaN for an out-of-range label), and
// sum the block's tokens in float64 in a fixed order. A block handles
// kMergeTokens tokens; its 8 thread groups each merge every 8th tile of them
// (online max/rescale), then the groups are combined in a fixed order.
constexpr int kMergeTokens = 32;

__global__ __launch_bounds__(256) void k_lse_merge(
    const float2* __restrict__ part, int64_t n_tiles, int64_t ld_part,
    const float* __restrict__ zt, const int64_t* __restrict__ labels, int64_t N,
    int64_t V, int64_t ignore_index, float* __restrict__ lse, float* __restrict__ lse_out,
    double* __restrict__ lsum) {
  __shared__ float2 grp[8][kMergeTokens];
  __shared__ double red[kMergeTokens];
  const int tk = threadIdx.x % kMergeTokens, g = threadIdx.x / kMergeTokens;
  const int64_t t = int64_t(blockIdx.x) * kMergeTokens + tk;
  float M = -INFINITY, S = 0.f;
  if (t < N) {
    for (int64_t j = g; j < n_tiles; j += 8) {
      const float2 q = part[j * ld_part + t];
      if (q.x > M) {
        S = (M == -INFINITY ? 0.f : S * exp2f((M - q.x) * kLog2e)) + q.y;
        M = q.x;
      } else {
        S += q.y * exp2f((q.x - M) * kLog2e);
      }
    }
  }
  grp[g][tk] = make_float2(M, S);
  __syncthreads();
  if (g == 0) {
    double ell = 0.0;
    if (t < N) {
      float Mx = -INFINITY;
      for (int i = 0; i < 8; ++i) Mx = fmaxf(Mx, grp[i][tk].x);
      float St = 0.f;
      for (int i = 0; i < 8; ++i)
        if (grp[i][tk].x != -INFINITY) St += grp[i][tk].y * exp2f((grp[i][tk].x - Mx) * kLog2e);
      const float l = Mx + log2f(St) * kLn2;
      lse[t] = l;
      if (lse_out) lse_out[t] = l;
      const int64_t y = labels[t];
      if (y != ignore_index) ell = (y < 0 || y >= V) ? double(NAN) : double(l) - double(zt[t]);
    }
    red[tk] = ell;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int i = 0; i < kMergeTokens; ++i) s += red[i];
    lsum[blockIdx.x] = s;
  }
}

// loss = c * sum(lsum) in float64, fixed order; NaN when a label was invalid.
__global__ __launch_bounds__(256) void k_loss_final(const double* __restrict__ lsum, int64_t nb,
                                                    const Scalars* __restrict__ sc,
                                                    float* __restrict__ loss) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < nb; i += 256) s += lsum[i];
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
                     0, L.stream, a.part, p.n_voc_tiles, p.ld_part, a.zt, a.labels + t0, nt, p.V,
                     a.ignore_index, a.lse, a.lse_out ? a.lse_out + t0 : nullptr,
                     a.lsum + t0 / kMergeTokens);
  L.post(kLseMerge);
  return hipGetLastError();
}

hipError_t launch_merge_and_loss(const Plan& p, const Args& a, const Launcher& L) {
  hipError_t e = launch_merge(p, a, 0, p.N, L);
  if (e != hipSuccess) return e;
  return launch_loss_final(p, a, L);
}

hipError_t launch_loss_final(const Plan& p, const Args& a, const Launcher& L) {
  L.pre(kLossFinal);
  hipLaunchKernelGGL(k_loss_final, dim3(1), dim3(256), 0, L.stream, a.lsum, p.n_loss_blocks,
                     a.sc, a.loss);
  L.post(kLossFinal);
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

}  // namespace flce
