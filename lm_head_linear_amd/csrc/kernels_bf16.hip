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
#include "gemm_index.h"

namespace flce {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kBM = gemm::kBM;
constexpr int kThreads = 256;
constexpr int kTileBytes = kBM * gemm::kBK * 2;  // one operand, one stage: 32 KiB
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  // Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
  return __builtin_bit_cast(uint16_t, __bf16(f));
}

using gemm::Geom;
using gemm::kBK;
using gemm::kLoadsPerOperand;
using gemm::swz_n;
using gemm::swz_t;

// An operand of the GEMM: a pointer and its geometry (see gemm_index.h).
struct Operand {
  const uint16_t* ptr;
  Geom g;
};

// Per-thread state of one operand's direct-to-LDS loads: a wave-uniform tile
// base advanced by `kstep` bytes per K tile, and one 32-bit byte offset per
// load (see gemm::direct_lane for the layout and the edge clamping).
struct DirectLoads {
  const char* base;
  int64_t kstep;
  uint32_t off[kLoadsPerOperand];
};

template <int FORM>
__device__ __forceinline__ DirectLoads setup_direct(const Operand& op, int64_t row0, int wave,
                                                    int lane) {
  DirectLoads d;
  d.base = reinterpret_cast<const char*>(op.ptr + gemm::direct_base(FORM, op.g, row0));
  d.kstep = gemm::direct_kstep(FORM, op.g) * 2;
#pragma unroll
  for (int q = 0; q < kLoadsPerOperand; ++q)
    d.off[q] = uint32_t(gemm::direct_lane(FORM, op.g, row0, wave, lane, q) * 2);
  return d;
}

// Issue one K tile of direct loads into an LDS tile (32 KiB): load q of wave
// w fills LDS bytes [(8w + q) KiB, +1 KiB), lane l writing 16 B at 16 l.
__device__ __forceinline__ void issue_direct(const DirectLoads& d, int64_t kt, char* lds,
                                             int wave) {
  const char* b = d.base + kt * d.kstep;
#pragma unroll
  for (int q = 0; q < kLoadsPerOperand; ++q)
    __builtin_amdgcn_global_load_lds(
        b + d.off[q], (__attribute__((address_space(3))) void*)(lds + (8 * wave + q) * 1024), 16,
        0, 0);
}

// Register path for a partial last K tile: zero-filled past K (and past the
// matrix edge), then stored into the same LDS layout.
template <int FORM>
__device__ __forceinline__ void load_tail(u32x4 (&r)[8], const Operand& op, int64_t row0,
                                          int64_t k0, int tid) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int64_t off;
    const bool ok = gemm::tail_src(FORM, op.g, row0, k0, tid + 256 * i, off);
    r[i] = ok ? *reinterpret_cast<const u32x4*>(op.ptr + off) : u32x4{0u, 0u, 0u, 0u};
  }
}

template <int FORM>
__device__ __forceinline__ void store_tail(char* lds, const u32x4 (&r)[8], int tid) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<u32x4*>(lds + gemm::tail_lds_pos(FORM, tid + 256 * i) * 16) = r[i];
}

// MFMA fragment of 32 rows (block b of the wave's 128) for K substep s.
template <int FORM>
__device__ __forceinline__ bf16x8 read_frag(const char* lds, int row_base, int s, int lane) {
  if (FORM == 0) {
    const int row = row_base + (lane & 31);
    const int c = 2 * s + (lane >> 5);
    const u32x4 v = *reinterpret_cast<const u32x4*>(lds + (row * 8 + (c ^ swz_n(row))) * 16);
    return __builtin_bit_cast(bf16x8, v);
  } else {
    typedef __attribute__((ext_vector_type(4))) short s16x4;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int g = lane >> 4, i = lane & 15;
    const int col = row_base + 16 * (g & 1) + 4 * (i & 3);
    s16x4 h[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int k = 16 * s + 8 * (g >> 1) + 4 * r + (i >> 2);
      const int off = (k * 32 + ((col >> 3) ^ swz_t(k))) * 16 + ((col >> 2) & 1) * 8;
      h[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + off));
    }
    typedef __attribute__((ext_vector_type(8))) short s16x8;
    const s16x8 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
    return __builtin_bit_cast(bf16x8, v);
  }
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

// vmcnt(0), other counters untouched (gfx9 s_waitcnt encoding).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int FA, int FB>
__device__ __forceinline__ void compute_tile(f32x16 (&acc)[4][4], const char* sa, const char* sb,
                                             int wm, int wn, int lane) {
  // let the scheduler interleave the fragment reads with the MFMAs
  __builtin_amdgcn_iglp_opt(0);
  bf16x8 af[2][4], bfr[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) af[0][i] = read_frag<FA>(sa, wm * 128 + i * 32, 0, lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) bfr[0][j] = read_frag<FB>(sb, wn * 128 + j * 32, 0, lane);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int cur = s & 1, nxt = cur ^ 1;
    if (s < 3) {
#pragma unroll
      for (int i = 0; i < 4; ++i) af[nxt][i] = read_frag<FA>(sa, wm * 128 + i * 32, s + 1, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[nxt][j] = read_frag<FB>(sb, wn * 128 + j * 32, s + 1, lane);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
  }
}

// One full K step: start the direct loads of tile kt+1 into the other LDS
// buffers, then multiply tile kt. The buffers are __restrict__ so the
// compiler can tell the direct-to-LDS writes of tile kt+1 from the reads of
// tile kt and does not wait for the former before the latter; the real
// dependency is the explicit vmcnt(0) + barrier at the top of the next step.
template <int FA, int FB>
__device__ __forceinline__ void k_step(f32x16 (&acc)[4][4], const DirectLoads& da,
                                       const DirectLoads& db, int64_t kt, int64_t nfull,
                                       int wave, int wm, int wn, int lane,
                                       const char* __restrict__ ca, const char* __restrict__ cb,
                                       char* __restrict__ na, char* __restrict__ nb) {
  if (kt + 1 < nfull) {
    issue_direct(da, kt + 1, na, wave);
    issue_direct(db, kt + 1, nb, wave);
  }
  compute_tile<FA, FB>(acc, ca, cb, wm, wn, lane);
}

template <int FA, int FB, class Epi>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(Operand A, Operand B, int64_t M,
                                                      int64_t Nn, int64_t K, int group_m,
                                                      Epi epi) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * kTileBytes];
  char* const lds_a0 = smem;
  char* const lds_b0 = smem + kTileBytes;
  char* const lds_a1 = smem + 2 * kTileBytes;
  char* const lds_b1 = smem + 3 * kTileBytes;
  int64_t m0, n0;
  gemm::tile_coords(blockIdx.x, M, Nn, group_m, m0, n0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const DirectLoads da = setup_direct<FA>(A, m0, wave, lane);
  const DirectLoads db = setup_direct<FB>(B, n0, wave, lane);
  const int64_t nfull = K / kBK;               // K tiles loaded directly
  const int64_t nk = (K + kBK - 1) / kBK;      // plus a zero-filled partial tile

  if (nfull > 0) {
    issue_direct(da, 0, lds_a0, wave);
    issue_direct(db, 0, lds_b0, wave);
  }
  for (int64_t kt = 0; kt < nfull; ++kt) {
    wait_vmem();
    __syncthreads();
    const bool odd = kt & 1;
    k_step<FA, FB>(acc, da, db, kt, nfull, wave, wm, wn, lane, odd ? lds_a1 : lds_a0,
                   odd ? lds_b1 : lds_b0, odd ? lds_a0 : lds_a1, odd ? lds_b0 : lds_b1);
  }
  if (nk > nfull) {
    // The partial last K tile goes through registers, zero-filled past K. Its
    // LDS buffers were last read two steps ago, behind the last barrier.
    char* la = (nfull & 1) ? lds_a1 : lds_a0;
    char* lb = (nfull & 1) ? lds_b1 : lds_b0;
    u32x4 ta[8], tb[8];
    load_tail<FA>(ta, A, m0, nfull * kBK, tid);
    load_tail<FB>(tb, B, n0, nfull * kBK, tid);
    store_tail<FA>(la, ta, tid);
    store_tail<FB>(lb, tb, tid);
    __syncthreads();
    compute_tile<FA, FB>(acc, la, lb, wm, wn, lane);
  }
  __syncthreads();
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

// ---- backward epilogue: the logit gradient G for one vocabulary chunk ----
// G[t, v] = c * valid_t * (exp(z'_tv - lse_t) - [v = y_t]) * dz'/dz, stored
// bf16 token-major as G[t][v - v0] (row length ldgv). Tile rows are
// chunk-relative vocab ids, columns tokens. Each wave stages its 128 x 128
// block in its own 32 KiB of LDS as [token][vocab] (a lane packs its 4
// consecutive vocab values into 8 bytes; 8-byte slots XOR-swizzled by token),
// then writes whole 16-byte runs of a token row to global memory.
struct EpiGrad {
  const int64_t* labels;
  const float* lse;
  const Scalars* sc;
  int64_t N, V, ignore_index, v0, vcur, ldgv;
  float softcap, inv_softcap;
  uint16_t* g;

  __device__ __forceinline__ void operator()(f32x16 (&acc)[4][4], int64_t m0, int64_t n0, int wm,
                                             int wn, int lane, char* smem) const {
    const float c = sc->c32;
    const int half = lane >> 5;
    char* reg = smem + (wm + 2 * wn) * kTileBytes;   // this wave's 32 KiB
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tl = j * 32 + (lane & 31);             // token within the wave block
      const int64_t t = n0 + wn * 128 + tl;
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
      // target column relative to this wave's first vocab row (or out of range)
      const int64_t ydiff = y - (v0 + m0 + wm * 128);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          uint32_t packed[2];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rq + e;
            const int vl = i * 32 + 8 * rq + 4 * half + e;   // vocab within the wave block
            float z = acc[i][j][r];
            float d = 1.f;
            if (softcap > 0.f) {
              const float th = tanhf(z * inv_softcap);
              z = softcap * th;
              d = 1.f - th * th;
            }
            const float p = __builtin_amdgcn_exp2f((z - l) * kLog2e);
            const float oh = (ydiff == vl) ? 1.f : 0.f;
            const float gv = valid ? (p - oh) * coef * d : 0.f;
            const uint32_t b = f32_to_bf16(gv);
            if (e & 1) packed[e >> 1] |= b << 16;
            else packed[e >> 1] = b;
          }
          const int slot = (i * 8 + 2 * rq + half) ^ (tl & 31);
          *reinterpret_cast<uint2*>(reg + tl * 256 + slot * 8) = make_uint2(packed[0], packed[1]);
        }
    }
    __syncthreads();
    // read back 16-byte runs of token rows and store them
#pragma unroll 4
    for (int q = 0; q < 32; ++q) {
      const int idx = q * 64 + lane;
      const int tl = idx >> 4, ch = idx & 15, x = tl & 31;
      u32x4 v = *reinterpret_cast<const u32x4*>(reg + tl * 256 + (((2 * ch) ^ x) & ~1) * 8);
      if (x & 1) v = u32x4{v[2], v[3], v[0], v[1]};
      const int64_t t = n0 + wn * 128 + tl;
      const int64_t vl = m0 + wm * 128 + 8 * ch;
      if (t < N && vl < vcur) *reinterpret_cast<u32x4*>(g + t * ldgv + vl) = v;
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

const uint16_t* buf_ptr(const Args& a, int buf) {
  return buf == gemm::kBufW ? static_cast<const uint16_t*>(a.W)
       : buf == gemm::kBufH ? static_cast<const uint16_t*>(a.h)
                            : static_cast<const uint16_t*>(a.g);
}

// A T-form operand is read in 16-byte column chunks: it needs rows % 8 == 0.
bool launch_ok(const gemm::Launch& l) {
  if (l.fa == gemm::kFormT && (l.a.rows % 8 != 0 || l.a.rows < 8)) return false;
  if (l.fb == gemm::kFormT && (l.b.rows % 8 != 0 || l.b.rows < 8)) return false;
  return l.M > 0 && l.Nn > 0 && l.K > 0;
}

template <int FA, int FB, class Epi>
hipError_t run_gemm(const gemm::Launch& l, const Args& a, const Epi& e, int kind,
                    const Launcher& L) {
  if (!launch_ok(l)) return hipErrorInvalidValue;
  Operand A{buf_ptr(a, l.buf_a) + l.off_a, l.a};
  Operand B{buf_ptr(a, l.buf_b) + l.off_b, l.b};
  L.pre(kind);
  hipLaunchKernelGGL((k_gemm<FA, FB, Epi>), dim3(unsigned(gemm::num_tiles(l.M, l.Nn))),
                     dim3(kThreads), 0, L.stream, A, B, l.M, l.Nn, l.K, gemm::kGroupM, e);
  L.post(kind);
  return hipGetLastError();
}

}  // namespace

hipError_t bf16_forward(const Plan& p, const Args& a, const Launcher& L) {
  const gemm::Launch l = gemm::forward_launch(p);
  EpiLse e{a.labels, p.N, p.V, a.ignore_index, a.softcap,
           a.softcap > 0.f ? 1.f / a.softcap : 0.f, a.part, p.ld_part, a.zt};
  return run_gemm<gemm::kFormN, gemm::kFormN>(l, a, e, kLseFwd, L);
}

hipError_t bf16_backward_chunk(const Plan& p, const Args& a, int64_t chunk, const Launcher& L) {
  const int64_t v0 = chunk * p.vchunk;
  const int64_t vcur = gemm::chunk_rows(p, chunk);
  uint16_t* g = static_cast<uint16_t*>(a.g);
  // 1) recompute the logits of the chunk and form G[N][vchunk]
  EpiGrad eg{a.labels, a.lse, a.sc, p.N, p.V, a.ignore_index, v0, vcur, p.vchunk, a.softcap,
             a.softcap > 0.f ? 1.f / a.softcap : 0.f, g};
  hipError_t err = run_gemm<gemm::kFormN, gemm::kFormN>(gemm::backward_launch(p, chunk, 0), a,
                                                         eg, kGradLogits, L);
  if (err != hipSuccess) return err;
  // 2) dW[v0:v0+vcur] = G^T . h
  EpiDW ew{static_cast<uint16_t*>(a.dW), p.H, v0, vcur, a.accumulate_dW};
  err = run_gemm<gemm::kFormT, gemm::kFormT>(gemm::backward_launch(p, chunk, 1), a, ew, kGemmDW,
                                             L);
  if (err != hipSuccess) return err;
  // 3) dH (+)= G[:, chunk] . W[chunk]
  EpiDH eh{static_cast<uint16_t*>(a.dH), a.dh_acc, p.N, p.H, chunk == 0 ? 1 : 0,
           chunk == p.n_chunks - 1 ? 1 : 0};
  return run_gemm<gemm::kFormN, gemm::kFormT>(gemm::backward_launch(p, chunk, 2), a, eh, kGemmDH,
                                              L);
}

}  // namespace flce
