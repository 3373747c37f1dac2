// bf16 path on CDNA4 matrix cores (gfx950).
//
// One GEMM main loop serves every contraction of the step:
//   forward   Z^T tile = W[v-tile] . h[t-tile]^T        (K = H)
//   recompute Z^T tile, then the logit-gradient epilogue (K = H)
//   dW chunk  = G^T[chunk] . h                          (K = tokens)
//   dH       += G[:, chunk] . W[chunk]                  (K = vocab chunk)
// Workgroup tile 256 x 256, K step 64, four waves of 128 x 128 each built from
// v_mfma_f32_32x32x16_bf16 (fp32 accumulate). Operands are staged through LDS
// in a K-contiguous, XOR-swizzled layout, double buffered; an operand that is
// stored with its M/N dimension contiguous is transposed 8x8 in registers on
// its way into LDS, so the MFMA loop never changes.
//
// Tiles are computed with the vocabulary on the M side and tokens on the N
// side for the logit tiles: a lane then owns one token column and 64 vocab
// values of it, so the per-token max / sum-exp reductions of the forward
// epilogue stay inside the lane (plus one swap between the two half-waves
// and one exchange between the two waves of a column).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/flce.h"
#include "flce_internal.h"

namespace flce {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kBM = 256;
constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kTileBytes = kBM * kBK * 2;  // one operand, one stage: 32 KiB
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  // Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
  return __builtin_bit_cast(uint16_t, __bf16(f));
}

// An operand of the GEMM. Stored either [rows][K] (K contiguous, "N" form)
// or [K][rows] (rows contiguous, "T" form), with `ld` elements between
// consecutive stored rows. Rows >= `rows` and k >= `K` read as zero.
struct Operand {
  const uint16_t* ptr;
  int64_t ld;
  int64_t rows;
  int64_t K;
};

// ---- global -> registers -> LDS -------------------------------------------
// LDS tile layout: 256 rows x 64 k (128 B per row) as 8 chunks of 16 B; the
// chunk c of row r is stored at chunk position c ^ (r & 7).

// N form: thread loads rows (tid>>3) + 32 i, k chunk (tid & 7).
__device__ __forceinline__ void load_n(u32x4 (&r)[8], const Operand& op, int64_t row0,
                                       int64_t k0, int tid) {
  const int c = tid & 7, rr = tid >> 3;
  const int64_t gk = k0 + 8 * c;
  const bool kok = gk < op.K;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t gr = row0 + rr + 32 * i;
    if (kok && gr < op.rows)
      r[i] = *reinterpret_cast<const u32x4*>(op.ptr + gr * op.ld + gk);
    else
      r[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void store_n(char* lds, const u32x4 (&r)[8], int tid) {
  const int c = tid & 7, rr = tid >> 3;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = rr + 32 * i;
    *reinterpret_cast<u32x4*>(lds + (row * 8 + (c ^ (row & 7))) * 16) = r[i];
  }
}

// T form: thread owns k rows 8*(tid&7) + i (i < 8) and 8 consecutive stored
// columns starting at 8*(tid>>3).
__device__ __forceinline__ void load_t(u32x4 (&r)[8], const Operand& op, int64_t row0,
                                       int64_t k0, int tid) {
  const int kb = tid & 7, mb = tid >> 3;
  const int64_t gm = row0 + 8 * mb;
  const bool mok = gm < op.rows;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t gk = k0 + 8 * kb + i;
    if (mok && gk < op.K)
      r[i] = *reinterpret_cast<const u32x4*>(op.ptr + gk * op.ld + gm);
    else
      r[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

// 8x8 transpose of 16-bit values: output m holds the 8 k values of column m.
__device__ __forceinline__ void store_t(char* lds, const u32x4 (&r)[8], int tid) {
  const int kb = tid & 7, mb = tid >> 3;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x = r[2 * e][m >> 1];
      const uint32_t y = r[2 * e + 1][m >> 1];
      o[e] = (m & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
    }
    const int row = 8 * mb + m;
    *reinterpret_cast<u32x4*>(lds + (row * 8 + (kb ^ (row & 7))) * 16) = o;
  }
}

__device__ __forceinline__ bf16x8 read_frag(const char* lds, int row, int chunk) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(lds + (row * 8 + (chunk ^ (row & 7))) * 16);
  return __builtin_bit_cast(bf16x8, v);
}

// ---- tile scheduling --------------------------------------------------------
// Workgroups are handed to the 8 XCDs round-robin. Give each XCD a contiguous
// range of tiles, and order tiles within a range in groups of `group_m`
// M-tiles so that the workgroups resident on one XCD share operand tiles in
// that XCD's L2.
__device__ __forceinline__ void tile_coords(int64_t M, int64_t Nn, int group_m, int64_t& m0,
                                            int64_t& n0) {
  const int64_t num_m = (M + kBM - 1) / kBM, num_n = (Nn + kBM - 1) / kBM;
  const int64_t total = num_m * num_n;
  const int64_t b = blockIdx.x;
  const int64_t q = total / 8, rem = total % 8, x = b % 8, local = b / 8;
  const int64_t tile = x * q + (x < rem ? x : rem) + local;
  const int64_t per_group = int64_t(group_m) * num_n;
  const int64_t g = tile / per_group;
  const int64_t first_m = g * group_m;
  const int64_t gs = (num_m - first_m) < group_m ? (num_m - first_m) : group_m;
  const int64_t in = tile - g * per_group;
  m0 = (first_m + in % gs) * kBM;
  n0 = (in / gs) * kBM;
}

// Element (i, j, r) of the accumulators of a wave sits at tile row
// wm*128 + i*32 + 8*(r/4) + 4*(lane/32) + r%4 and tile column
// wn*128 + j*32 + lane%32 (the 32x32 MFMA output layout).
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) {
  return wn * 128 + j * 32 + (lane & 31);
}

template <bool AT, bool BT, class Epi>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(Operand A, Operand B, int64_t M,
                                                      int64_t Nn, int64_t K, int group_m,
                                                      Epi epi) {
  __shared__ __attribute__((aligned(16))) char smem[4 * kTileBytes];
  int64_t m0, n0;
  tile_coords(M, Nn, group_m, m0, n0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ra[8], rb[8];
  const int64_t nk = (K + kBK - 1) / kBK;
  if (AT) load_t(ra, A, m0, 0, tid); else load_n(ra, A, m0, 0, tid);
  if (BT) load_t(rb, B, n0, 0, tid); else load_n(rb, B, n0, 0, tid);
  if (AT) store_t(smem, ra, tid); else store_n(smem, ra, tid);
  if (BT) store_t(smem + kTileBytes, rb, tid); else store_n(smem + kTileBytes, rb, tid);
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const char* sa = smem + (kt & 1) * 2 * kTileBytes;
    const char* sb = sa + kTileBytes;
    const bool more = kt + 1 < nk;
    if (more) {
      const int64_t k1 = (kt + 1) * kBK;
      if (AT) load_t(ra, A, m0, k1, tid); else load_n(ra, A, m0, k1, tid);
      if (BT) load_t(rb, B, n0, k1, tid); else load_n(rb, B, n0, k1, tid);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 af[4], bfr[4];
      const int ch = 2 * s + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = read_frag(sa, wm * 128 + i * 32 + (lane & 31), ch);
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = read_frag(sb, wn * 128 + j * 32 + (lane & 31), ch);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      char* da = smem + ((kt + 1) & 1) * 2 * kTileBytes;
      if (AT) store_t(da, ra, tid); else store_n(da, ra, tid);
      if (BT) store_t(da + kTileBytes, rb, tid); else store_n(da + kTileBytes, rb, tid);
    }
    __syncthreads();
  }
  epi(acc, m0, n0, wm, wn, lane, smem);
}

__device__ __forceinline__ float softcap_fwd(float z, float s, float inv_s) {
  return s * tanhf(z * inv_s);
}

// ---- forward epilogue: per (vocab tile, token) max and sum-exp ------------
// Tile rows are vocabulary ids (relative to v_off), columns are tokens.
struct EpiLse {
  const int64_t* labels;
  int64_t N, V, ignore_index;
  float softcap, inv_softcap;
  float2* part;  // [n_voc_tiles][ld_part]: (max m, sum of exp(x - m)) of the tile
  int64_t ld_part;
  float* zt;     // target logit (softcapped), one writer per non-ignored token

  __device__ __forceinline__ void operator()(f32x16 (&acc)[4][4], int64_t m0, int64_t n0, int wm,
                                             int wn, int lane, char* smem) const {
    const int half = lane >> 5;
    const int64_t vbase = m0 + wm * 128;
    float mx[4], sm[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t = n0 + acc_col(wn, j, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float z = acc[i][j][r];
          if (softcap > 0.f) z = softcap_fwd(z, softcap, inv_softcap);
          const int64_t v = m0 + acc_row(wm, i, r, lane);
          acc[i][j][r] = v < V ? z : -INFINITY;
        }
      // target logit: the one lane holding (y_t, t) writes it
      const int64_t y = t < N ? labels[t] : ignore_index;
      if (y != ignore_index && y >= vbase && y < vbase + 128 && y < V) {
        const int d = int(y - vbase);
        const int ti = d >> 5, w = d & 31;
        if (((w >> 2) & 1) == half) {
          const int tr = ((w >> 3) << 2) | (w & 3);
          float val = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) val = (i == ti && r == tr) ? acc[i][j][r] : val;
          zt[t] = val;
        }
      }
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[i][j][r]);
      m = fmaxf(m, __shfl_xor(m, 32));
      float s = 0.f;
      if (m != -INFINITY) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s += __builtin_amdgcn_exp2f((acc[i][j][r] - m) * kLog2e);
      }
      s += __shfl_xor(s, 32);
      mx[j] = m;
      sm[j] = s;
    }
    // combine the two waves (wm = 0, 1) that share the token columns
    float2* buf = reinterpret_cast<float2*>(smem);
    if (wm == 1 && half == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) buf[wn * 128 + j * 32 + lane] = make_float2(mx[j], sm[j]);
    }
    __syncthreads();
    if (wm == 0 && half == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float2 o = buf[wn * 128 + j * 32 + lane];
        const float Mx = fmaxf(mx[j], o.x);
        float S = 0.f;
        if (mx[j] != -INFINITY) S += sm[j] * __builtin_amdgcn_exp2f((mx[j] - Mx) * kLog2e);
        if (o.x != -INFINITY) S += o.y * __builtin_amdgcn_exp2f((o.x - Mx) * kLog2e);
        const int64_t t = n0 + acc_col(wn, j, lane);
        if (t < ld_part) part[(m0 / kBM) * ld_part + t] = make_float2(Mx, S);
      }
    }
  }
};

// ---- backward epilogue: the logit gradient G^T for one vocabulary chunk ----
// G[t, v] = c * valid_t * (exp(z'_tv - lse_t) - [v = y_t]) * dz'/dz, stored
// bf16 as G^T[v - v0][t]. Tile rows are chunk-relative vocab ids.
struct EpiGrad {
  const int64_t* labels;
  const float* lse;
  const Scalars* sc;
  int64_t N, V, ignore_index, v0, vcur, ldg;
  float softcap, inv_softcap;
  uint16_t* gt;

  __device__ __forceinline__ void operator()(f32x16 (&acc)[4][4], int64_t m0, int64_t n0, int wm,
                                             int wn, int lane, char*) const {
    const float c = sc->c32;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t = n0 + acc_col(wn, j, lane);
      int64_t y = ignore_index;
      float l = 0.f, coef = 0.f;
      bool valid = false;
      if (t < N) {
        y = labels[t];
        if (y != ignore_index) {
          valid = true;
          coef = (y < 0 || y >= V) ? NAN : c;
          l = lse[t];
        }
      }
      const bool tok = t < ldg;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + acc_row(wm, i, r, lane);
          float z = acc[i][j][r];
          float d = 1.f;
          if (softcap > 0.f) {
            const float th = tanhf(z * inv_softcap);
            z = softcap * th;
            d = 1.f - th * th;
          }
          const float p = __builtin_amdgcn_exp2f((z - l) * kLog2e);
          const float oh = (v0 + m == y) ? 1.f : 0.f;
          const float g = valid ? (p - oh) * coef * d : 0.f;
          if (tok && m < vcur) gt[m * ldg + t] = f32_to_bf16(g);
        }
    }
  }
};

// ---- dW epilogue: rows v0 + m of dW, bf16, optionally accumulated ---------
struct EpiDW {
  uint16_t* dW;
  int64_t H, v0, vcur;
  int accumulate;

  __device__ __forceinline__ void operator()(f32x16 (&acc)[4][4], int64_t m0, int64_t n0, int wm,
                                             int wn, int lane, char*) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + acc_col(wn, j, lane);
      if (n >= H) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + acc_row(wm, i, r, lane);
          if (m < vcur) {
            const int64_t idx = (v0 + m) * H + n;
            float x = acc[i][j][r];
            if (accumulate) x += bf16_to_f32(dW[idx]);
            dW[idx] = f32_to_bf16(x);
          }
        }
    }
  }
};

// ---- dH epilogue: accumulate over vocabulary chunks in a fixed order ------
struct EpiDH {
  uint16_t* dH;
  float* acc32;  // [N][H] float32 running sum (unused with a single chunk)
  int64_t N, H;
  int first, last;

  __device__ __forceinline__ void operator()(f32x16 (&acc)[4][4], int64_t m0, int64_t n0, int wm,
                                             int wn, int lane, char*) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + acc_col(wn, j, lane);
      if (n >= H) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + acc_row(wm, i, r, lane);
          if (m < N) {
            const int64_t idx = m * H + n;
            float x = acc[i][j][r];
            if (!first) x += acc32[idx];
            if (last) dH[idx] = f32_to_bf16(x);
            else acc32[idx] = x;
          }
        }
    }
  }
};

int64_t n_tiles(int64_t M, int64_t Nn) { return ((M + kBM - 1) / kBM) * ((Nn + kBM - 1) / kBM); }

}  // namespace

hipError_t bf16_forward(const Plan& p, const Args& a, const Launcher& L) {
  const uint16_t* W = static_cast<const uint16_t*>(a.W);
  const uint16_t* h = static_cast<const uint16_t*>(a.h);
  Operand A{W, p.H, p.V, p.H};
  Operand B{h, p.H, p.N, p.H};
  EpiLse e{a.labels, p.N, p.V, a.ignore_index, a.softcap,
           a.softcap > 0.f ? 1.f / a.softcap : 0.f, a.part, p.ld_part, a.zt};
  L.pre(kLseFwd);
  hipLaunchKernelGGL((k_gemm<false, false, EpiLse>), dim3(unsigned(n_tiles(p.V, p.N))),
                     dim3(kThreads), 0, L.stream, A, B, p.V, p.N, p.H, 4, e);
  L.post(kLseFwd);
  return hipGetLastError();
}

hipError_t bf16_backward_chunk(const Plan& p, const Args& a, int64_t chunk, const Launcher& L) {
  const uint16_t* W = static_cast<const uint16_t*>(a.W);
  const uint16_t* h = static_cast<const uint16_t*>(a.h);
  uint16_t* gt = static_cast<uint16_t*>(a.g);
  const int64_t v0 = chunk * p.vchunk;
  const int64_t vcur = (p.V - v0) < p.vchunk ? (p.V - v0) : p.vchunk;

  // 1) recompute the logits of the chunk and form G^T[vcur][ldg]
  {
    Operand A{W + v0 * p.H, p.H, vcur, p.H};
    Operand B{h, p.H, p.N, p.H};
    EpiGrad e{a.labels, a.lse, a.sc, p.N, p.V, a.ignore_index, v0, vcur, p.ldg, a.softcap,
              a.softcap > 0.f ? 1.f / a.softcap : 0.f, gt};
    L.pre(kGradLogits);
    hipLaunchKernelGGL((k_gemm<false, false, EpiGrad>), dim3(unsigned(n_tiles(vcur, p.N))),
                       dim3(kThreads), 0, L.stream, A, B, vcur, p.N, p.H, 4, e);
    L.post(kGradLogits);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // 2) dW[v0:v0+vcur] = G^T . h   (M = vcur, N = H, K = tokens)
  {
    Operand A{gt, p.ldg, vcur, p.N};           // [vcur][ldg], K contiguous
    Operand B{h, p.H, p.H, p.N};               // h [N][H]: [K][cols], T form
    EpiDW e{static_cast<uint16_t*>(a.dW), p.H, v0, vcur, a.accumulate_dW};
    L.pre(kGemmDW);
    hipLaunchKernelGGL((k_gemm<false, true, EpiDW>), dim3(unsigned(n_tiles(vcur, p.H))),
                       dim3(kThreads), 0, L.stream, A, B, vcur, p.H, p.N, 4, e);
    L.post(kGemmDW);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // 3) dH (+)= G[:, chunk] . W[chunk]   (M = tokens, N = H, K = vcur)
  {
    Operand A{gt, p.ldg, p.N, vcur};           // G^T [K = vcur][rows = tokens], T form
    Operand B{W + v0 * p.H, p.H, p.H, vcur};   // W chunk [K = vcur][cols = H], T form
    EpiDH e{static_cast<uint16_t*>(a.dH), a.dh_acc, p.N, p.H, chunk == 0 ? 1 : 0,
            chunk == p.n_chunks - 1 ? 1 : 0};
    L.pre(kGemmDH);
    hipLaunchKernelGGL((k_gemm<true, true, EpiDH>), dim3(unsigned(n_tiles(p.N, p.H))),
                       dim3(kThreads), 0, L.stream, A, B, p.N, p.H, vcur, 4, e);
    L.post(kGemmDH);
    return hipGetLastError();
  }
}

}  // namespace flce
