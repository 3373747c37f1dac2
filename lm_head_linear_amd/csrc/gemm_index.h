// Index arithmetic of the bf16 GEMM kernels: tile scheduling, the operand
// descriptions of every launch, and the global addresses of the operand loads.
// Shared verbatim by the HIP kernels and by the host-side bounds checker the
// CPU tests run, so the checker exercises exactly the kernels' arithmetic.
#pragma once

#include <cstdint>

#include "flce_plan.h"

#if defined(__HIPCC__)
#define FLCE_HD __host__ __device__ __forceinline__
#else
#define FLCE_HD inline
#endif

namespace flce {
namespace gemm {

constexpr int kBM = 256;                // tile edge (M and N)
constexpr int kBK = 32;                 // K step
constexpr int kStages = 4;              // LDS stages (prefetch distance kStages - 1)
constexpr int kLoadsPerOperand = 4;     // 16-byte loads per thread per operand per K tile
constexpr int kTailLoads = 4;           // register loads per thread for a partial K tile
constexpr int kGroupM = 4;              // M tiles per raster group

enum Form : int { kFormN = 0, kFormT = 1 };
enum Buf : int { kBufW = 0, kBufH = 1, kBufG = 2 };

// Geometry of one operand. N form: stored [rows][K] (K contiguous); T form:
// stored [K][rows] (rows contiguous). `ld` = elements between stored rows.
// A T-form operand needs rows % 8 == 0 (16-byte column chunks).
struct Geom {
  int64_t ld, rows, K;
};

// One GEMM launch: C[M][Nn] = A . B^T over K, A and B given as (buffer,
// element offset, geometry, form).
struct Launch {
  int64_t M, Nn, K;
  int fa, fb;
  int buf_a, buf_b;
  int64_t off_a, off_b;
  Geom a, b;
};

// The three launches of backward chunk c (0: logit gradient, 1: dW, 2: dH),
// or the forward launch (c < 0).
inline Launch forward_launch(const Plan& p) {
  return Launch{p.V, p.N, p.H, kFormN, kFormN, kBufW, kBufH, 0, 0,
                Geom{p.H, p.V, p.H}, Geom{p.H, p.N, p.H}};
}

inline int64_t chunk_rows(const Plan& p, int64_t c) {
  const int64_t v0 = c * p.vchunk;
  return (p.V - v0) < p.vchunk ? (p.V - v0) : p.vchunk;
}

inline Launch backward_launch(const Plan& p, int64_t c, int which) {
  const int64_t v0 = c * p.vchunk, vcur = chunk_rows(p, c);
  if (which == 0)  // Z^T[chunk] = W[chunk] . h^T, then the gradient epilogue
    return Launch{vcur, p.N, p.H, kFormN, kFormN, kBufW, kBufH, v0 * p.H, 0,
                  Geom{p.H, vcur, p.H}, Geom{p.H, p.N, p.H}};
  // G is stored token-major, G[t][v - v0] with row length vchunk (a multiple
  // of 8; columns from vcur to the row end are never multiplied into a
  // stored output).
  if (which == 1)  // dW[chunk] = G[:, chunk]^T . h  (K = tokens)
    return Launch{vcur, p.H, p.N, kFormT, kFormT, kBufG, kBufH, 0, 0,
                  Geom{p.vchunk, p.vchunk, p.N}, Geom{p.H, p.H, p.N}};
  // dH += G[:, chunk] . W[chunk]  (K = chunk rows)
  return Launch{p.N, p.H, vcur, kFormN, kFormT, kBufG, kBufW, 0, v0 * p.H,
                Geom{p.vchunk, p.N, vcur}, Geom{p.H, p.H, vcur}};
}

inline int64_t num_tiles(int64_t M, int64_t Nn) {
  return ((M + kBM - 1) / kBM) * ((Nn + kBM - 1) / kBM);
}

// Workgroups are handed to the 8 XCDs round-robin. Give each XCD a contiguous
// range of tiles, and order tiles within a range in groups of `group_m`
// M-tiles so that the workgroups resident on one XCD share operand tiles in
// that XCD's L2.
FLCE_HD void tile_coords(int64_t b, int64_t M, int64_t Nn, int group_m, int64_t& m0,
                         int64_t& n0) {
  const int64_t num_m = (M + kBM - 1) / kBM, num_n = (Nn + kBM - 1) / kBM;
  const int64_t total = num_m * num_n;
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

// LDS swizzles. N form: 256 rows x 32 k, 64 B per row, 4 chunks of 16 B;
// logical chunk c of row r at position c ^ swz_n(r). T form: 32 k-rows x 256
// columns, 512 B per k-row, 32 chunks; logical chunk c of k-row k at
// c ^ swz_t(k). Both were chosen by measuring the LDS bank-conflict counter
// on gfx950 for the fragment read patterns: zero conflicts.
FLCE_HD int swz_n(int r) { return (r >> 2) & 3; }
FLCE_HD int swz_t(int k) { return (0xCA60 >> (4 * (k & 3))) & 15; }  // {0,6,10,12}[k%4]

// Direct-to-LDS loads: element offset of the tile base (k = 0) from the
// operand pointer, elements to advance per K tile, and the element offset of
// load q of (wave, lane) from the tile base. Load q of wave w fills LDS bytes
// [(4w + q) KiB, +1 KiB), lane l writing 16 B at 16 l, so a lane fetches the
// logical chunk that the swizzle puts at its LDS position. Rows (N form) or
// column chunks (T form) past the edge are clamped to the last valid one:
// their products land outside the output and are never stored.
FLCE_HD int64_t direct_base(int form, const Geom& g, int64_t row0) {
  return form == kFormN ? row0 * g.ld : row0;
}
FLCE_HD int64_t direct_kstep(int form, const Geom& g) {
  return form == kFormN ? int64_t(kBK) : int64_t(kBK) * g.ld;
}
FLCE_HD int64_t direct_lane(int form, const Geom& g, int64_t row0, int wave, int lane, int q) {
  if (form == kFormN) {
    const int lr = 16 * (4 * wave + q) + (lane >> 2);
    const int c = (lane & 3) ^ swz_n(lr);
    int64_t r = row0 + lr;
    if (r > g.rows - 1) r = g.rows - 1;
    return (r - row0) * g.ld + 8 * c;
  }
  const int kr = 2 * (4 * wave + q) + (lane >> 5);
  const int c = (lane & 31) ^ swz_t(kr);
  int64_t col = 8 * c;
  if (row0 + col > g.rows - 8) col = g.rows - 8 - row0;
  return kr * g.ld + col;
}

// Register path of a partial last K tile: thread tid's load i covers
// z = tid + 256 i (i < kTailLoads). Returns whether it reads memory (else it
// stores zeros) and the element offset from the operand pointer.
FLCE_HD bool tail_src(int form, const Geom& g, int64_t row0, int64_t k0, int z, int64_t& off) {
  if (form == kFormN) {  // z -> (row z / 4, chunk z % 4)
    const int64_t gr = row0 + (z >> 2), gk = k0 + 8 * (z & 3);
    off = gr * g.ld + gk;
    return gr < g.rows && gk < g.K;
  }
  const int64_t gk = k0 + (z >> 5), gm = row0 + 8 * (z & 31);  // (k-row z / 32, chunk z % 32)
  off = gk * g.ld + gm;
  return gk < g.K && gm < g.rows;
}

// LDS chunk position (16-byte units) of the tail element z.
FLCE_HD int tail_lds_pos(int form, int z) {
  return form == kFormN ? (z >> 2) * 4 + ((z & 3) ^ swz_n(z >> 2))
                        : (z >> 5) * 32 + ((z & 31) ^ swz_t(z >> 5));
}

}  // namespace gemm
}  // namespace flce
