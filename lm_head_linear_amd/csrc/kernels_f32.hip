// float32 path: the same passes as the bf16 path with float32 operands,
// float32 logit gradient and float32 gradients. Plain LDS-tiled FMA tiles
// (64 x 64 per workgroup, 4 x 4 per thread): on gfx950 the float32 matrix-core
// rate equals the float32 vector rate, so matrix cores buy nothing here.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/flce.h"
#include "flce_internal.h"

namespace flce {
namespace {

constexpr int kT = 64;    // tile edge
constexpr int kBK = 16;   // K step
constexpr float kLog2e = 1.4426950408889634f;

// Operand element (row, k) = p[row * sr + k * sk]; zero outside rows x K.
struct Op {
  const float* p;
  int64_t sr, sk, rows, K;
};

// Thread (tx, ty) = (tid % 16, tid / 16) owns tile rows ty + 16 a and
// columns tx + 16 b (a, b < 4).
__device__ __forceinline__ void tile_gemm(const Op& A, const Op& B, int64_t m0, int64_t n0,
                                          int64_t K, float (&acc)[4][4],
                                          float (*As)[kT + 1], float (*Bs)[kT + 1]) {
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
  for (int64_t k0 = 0; k0 < K; k0 += kBK) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 256 * e;
      const int mm = idx & 63, kk = idx >> 6;
      const int64_t gm = m0 + mm, gn = n0 + mm, gk = k0 + kk;
      As[kk][mm] = (gm < A.rows && gk < A.K) ? A.p[gm * A.sr + gk * A.sk] : 0.f;
      Bs[kk][mm] = (gn < B.rows && gk < B.K) ? B.p[gn * B.sr + gk * B.sk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = As[kk][ty + 16 * a];
#pragma unroll
      for (int b = 0; b < 4; ++b) bv[b] = Bs[kk][tx + 16 * b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(av[a], bv[b], acc[a][b]);
    }
    __syncthreads();
  }
}

// Forward: tile rows = vocab ids, columns = tokens; per (vocab tile, token)
// the max and the sum of exponentials, plus the target logit. With `logits`
// non-null the tile's logits are also stored token-major, out[t][v] with row
// length ld_logits, float32 or (bf16_out) bf16 rounded to nearest even.
__global__ __launch_bounds__(256) void k_f32_lse(const float* __restrict__ W,
                                                 const float* __restrict__ h,
                                                 const int64_t* __restrict__ labels, int64_t N,
                                                 int64_t H, int64_t V, int64_t ignore_index,
                                                 float softcap, float2* __restrict__ part,
                                                 int64_t ld_part, float* __restrict__ zt,
                                                 void* __restrict__ logits, int64_t ld_logits,
                                                 int bf16_out) {
  __shared__ float As[kBK][kT + 1], Bs[kBK][kT + 1];
  __shared__ float Cs[kT][kT + 1];
  const int64_t m0 = int64_t(blockIdx.x) * kT, n0 = int64_t(blockIdx.y) * kT;
  Op A{W, H, 1, V, H}, B{h, H, 1, N, H};
  float acc[4][4];
  tile_gemm(A, B, m0, n0, H, acc, As, Bs);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      float z = acc[a][b];
      if (softcap > 0.f) z = softcap * tanhf(z / softcap);
      Cs[ty + 16 * a][tx + 16 * b] = z;
    }
  __syncthreads();
  if (logits) {
    // consecutive threads take consecutive vocabulary ids of one token row
    for (int idx = tid; idx < kT * kT; idx += 256) {
      const int tl = idx / kT, vl = idx % kT;
      const int64_t t = n0 + tl, v = m0 + vl;
      if (t < N && v < V) {
        const float z = Cs[vl][tl];
        if (bf16_out)
          static_cast<__bf16*>(logits)[t * ld_logits + v] = __bf16(z);
        else
          static_cast<float*>(logits)[t * ld_logits + v] = z;
      }
    }
  }
  if (tid < kT) {
    const int64_t t = n0 + tid;
    const int rows = int((V - m0) < kT ? (V - m0) : kT);
    float m = -INFINITY;
    for (int r = 0; r < rows; ++r) m = fmaxf(m, Cs[r][tid]);
    float s = 0.f;
    for (int r = 0; r < rows; ++r) s += exp2f((Cs[r][tid] - m) * kLog2e);
    if (t < ld_part) part[int64_t(blockIdx.x) * ld_part + t] = make_float2(m, s);
    if (t < N) {
      const int64_t y = labels[t];
      if (y != ignore_index && y >= m0 && y < m0 + rows) zt[t] = Cs[int(y - m0)][tid];
    }
  }
}

// Backward step 1: G^T[v - v0][t] (float32) for one vocabulary chunk.
__global__ __launch_bounds__(256) void k_f32_grad(const float* __restrict__ W,
                                                  const float* __restrict__ h,
                                                  const int64_t* __restrict__ labels,
                                                  const float* __restrict__ lse,
                                                  const Scalars* __restrict__ sc, int64_t N,
                                                  int64_t H, int64_t V, int64_t ignore_index,
                                                  float softcap, int64_t v0, int64_t vcur,
                                                  int64_t ldg, float* __restrict__ gt) {
  __shared__ float As[kBK][kT + 1], Bs[kBK][kT + 1];
  const int64_t m0 = int64_t(blockIdx.x) * kT, n0 = int64_t(blockIdx.y) * kT;
  Op A{W + v0 * H, H, 1, vcur, H}, B{h, H, 1, N, H};
  float acc[4][4];
  tile_gemm(A, B, m0, n0, H, acc, As, Bs);
  const float c = sc->c32;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int64_t t = n0 + tx + 16 * b;
    if (t >= ldg) continue;
    int64_t y = ignore_index;
    bool valid = false;
    float l = 0.f, coef = 0.f;
    if (t < N) {
      y = labels[t];
      if (y != ignore_index) {
        valid = true;
        coef = (y < 0 || y >= V) ? NAN : c;
        l = lse[t];
      }
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int64_t m = m0 + ty + 16 * a;
      if (m >= vcur) continue;
      float z = acc[a][b], d = 1.f;
      if (softcap > 0.f) {
        const float th = tanhf(z / softcap);
        z = softcap * th;
        d = 1.f - th * th;
      }
      const float p = expf(z - l);
      const float oh = (v0 + m == y) ? 1.f : 0.f;
      gt[m * ldg + t] = valid ? (p - oh) * coef * d : 0.f;
    }
  }
}

// Backward step 2: dW[v0 + m][n] (+)= sum_t G^T[m][t] h[t][n].
__global__ __launch_bounds__(256) void k_f32_dw(const float* __restrict__ gt,
                                                const float* __restrict__ h, int64_t N,
                                                int64_t H, int64_t ldg, int64_t v0, int64_t vcur,
                                                int accumulate, float* __restrict__ dW) {
  __shared__ float As[kBK][kT + 1], Bs[kBK][kT + 1];
  const int64_t m0 = int64_t(blockIdx.x) * kT, n0 = int64_t(blockIdx.y) * kT;
  Op A{gt, ldg, 1, vcur, N}, B{h, 1, H, H, N};
  float acc[4][4];
  tile_gemm(A, B, m0, n0, N, acc, As, Bs);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t m = m0 + ty + 16 * a, n = n0 + tx + 16 * b;
      if (m < vcur && n < H) {
        const int64_t idx = (v0 + m) * H + n;
        dW[idx] = accumulate ? dW[idx] + acc[a][b] : acc[a][b];
      }
    }
}

// Backward step 3: dH[t][n] (+)= sum_v G^T[v][t] W[v0 + v][n], chunks in order.
__global__ __launch_bounds__(256) void k_f32_dh(const float* __restrict__ gt,
                                                const float* __restrict__ W, int64_t N,
                                                int64_t H, int64_t ldg, int64_t v0, int64_t vcur,
                                                int first, float* __restrict__ dH) {
  __shared__ float As[kBK][kT + 1], Bs[kBK][kT + 1];
  const int64_t m0 = int64_t(blockIdx.x) * kT, n0 = int64_t(blockIdx.y) * kT;
  Op A{gt, 1, ldg, N, vcur}, B{W + v0 * H, 1, H, H, vcur};
  float acc[4][4];
  tile_gemm(A, B, m0, n0, vcur, acc, As, Bs);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t m = m0 + ty + 16 * a, n = n0 + tx + 16 * b;
      if (m < N && n < H) {
        const int64_t idx = m * H + n;
        dH[idx] = first ? acc[a][b] : dH[idx] + acc[a][b];
      }
    }
}

unsigned cdiv(int64_t a, int64_t b) { return unsigned((a + b - 1) / b); }

}  // namespace

hipError_t f32_forward(const Plan& p, const Args& a, const Launcher& L) {
  L.pre(kLseFwd);
  hipLaunchKernelGGL(k_f32_lse, dim3(cdiv(p.V, kT), cdiv(p.N, kT)), dim3(256), 0, L.stream,
                     static_cast<const float*>(a.W), static_cast<const float*>(a.h), a.labels,
                     p.N, p.H, p.V, a.ignore_index, a.softcap, a.part, p.ld_part, a.zt,
                     a.logits, a.ld_logits, int(a.logits_dtype == FLCE_BF16));
  L.post(kLseFwd);
  return hipGetLastError();
}

hipError_t f32_backward_chunk(const Plan& p, const Args& a, int64_t chunk, const Launcher& L) {
  const int64_t v0 = chunk * p.vchunk;
  const int64_t vcur = (p.V - v0) < p.vchunk ? (p.V - v0) : p.vchunk;
  float* gt = static_cast<float*>(a.g);
  L.pre(kGradLogits);
  hipLaunchKernelGGL(k_f32_grad, dim3(cdiv(vcur, kT), cdiv(p.ldg, kT)), dim3(256), 0, L.stream,
                     static_cast<const float*>(a.W), static_cast<const float*>(a.h), a.labels,
                     a.lse, a.sc, p.N, p.H, p.V, a.ignore_index, a.softcap, v0, vcur, p.ldg, gt);
  L.post(kGradLogits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  L.pre(kGemmDW);
  hipLaunchKernelGGL(k_f32_dw, dim3(cdiv(vcur, kT), cdiv(p.H, kT)), dim3(256), 0, L.stream, gt,
                     static_cast<const float*>(a.h), p.N, p.H, p.ldg, v0, vcur, a.accumulate_dW,
                     static_cast<float*>(a.dW));
  L.post(kGemmDW);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  L.pre(kGemmDH);
  hipLaunchKernelGGL(k_f32_dh, dim3(cdiv(p.N, kT), cdiv(p.H, kT)), dim3(256), 0, L.stream, gt,
                     static_cast<const float*>(a.W), p.N, p.H, p.ldg, v0, vcur,
                     chunk == 0 ? 1 : 0, static_cast<float*>(a.dH));
  L.post(kGemmDH);
  return hipGetLastError();
}

}  // namespace flce
