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
constexpr int kBK = 32;                 // K per MFMA step (one 16x16x32 MFMA deep)
constexpr int kGroupM = 4;              // M tiles per raster group

enum Form : int { kFormN = 0, kFormT = 1 };

// K per LDS stage tile. With both operands K-contiguous (N form) a stage
// tile holds 64 k, so each row contributes a whole 128-byte cache line to
// every direct load: rows of 64 bytes (half lines) stream at about 60% of
// the rate of whole lines into a CU. A T-form operand already loads runs of
// 512 bytes; there a 32-k stage tile spreads the LDS writes evenly over the
// MFMA steps, which measured faster. Stages: 2 of 64 k (128 KiB of LDS);
// with a transposed operand 5 of 32 k (160 KiB, a barrier every other step).
FLCE_HD constexpr int stage_k(int fa, int fb) { return (fa == kFormN && fb == kFormN) ? 64 : 32; }
FLCE_HD constexpr int num_stages(int fa, int fb) {
  return stage_k(fa, fb) == 64 ? 2 : 5;
}
// 16-byte direct loads per thread per operand per stage tile (256 rows x sk
// x 2 bytes over 256 threads), and register loads for a partial tile.
FLCE_HD constexpr int loads_per_operand(int sk) { return sk / 8; }
FLCE_HD constexpr int tail_loads(int sk) { return sk / 8; }
// Operand buffers: W, h, the logit gradient G, and the hidden rows of the
// non-ignored tokens gathered in order (the backward of a compact plan).
enum Buf : int { kBufW = 0, kBufH = 1, kBufG = 2, kBufHc = 3 };

// Geometry of one operand. N form: stored [rows][K] (K contiguous); T form:
// stored [K][rows] (rows contiguous). `ld` = elements between stored rows.
// A T-form operand needs rows % 8 == 0 (16-byte column chunks).
// blk != 0: the operand is stored in 32-wide blocks instead (the logit
// gradient G): a token-by-vocabulary matrix kept as [vocab / 32][tokens][32],
// blk elements per block (tokens x 32). As an N-form operand (rows = tokens,
// K = vocabulary, 32-k stages) each row of a stage tile is then 64 bytes of
// one 16-KiB-aligned run of 256 rows; as a T-form operand (K = tokens, rows =
// vocabulary) each k-row is 8 runs of 64 bytes, the k-rows of a block
// adjacent. ld is then 32.
struct Geom {
  int64_t ld, rows, K;
  int64_t blk = 0;
};

// Element (t, v) of a blocked token-by-vocabulary matrix.
FLCE_HD int64_t blocked_offset(int64_t t, int64_t v, int64_t blk) {
  return (v >> 5) * blk + t * 32 + (v & 31);
}

// One GEMM launch: C[M][Nn] = A . B^T over K, A and B given as (buffer,
// element offset, geometry, form).
struct Launch {
  int64_t M, Nn, K;
  int fa, fb;
  int buf_a, buf_b;
  int64_t off_a, off_b;
  Geom a, b;
};

// The forward launch, and the three launches of backward chunk c (0: logit
// gradient, 1: dW, 2: dH). With float32 gradients for bf16 inputs G is a
// pair of bf16 chunks, hi then lo, each vchunk x ldg elements; `part` picks
// the one a dW or dH launch reads. A compact plan reads the gathered rows
// (the non-ignored tokens first) instead of h; its token dimension (N of the
// forward and gradient launches, K of dW, M of dH) is then cut on the device
// to the non-ignored count (the forward's only without per-token lse), and
// the sizes here are the upper bound N.
inline Launch forward_launch(const Plan& p) {
  return Launch{p.V, p.N, p.H, kFormN, kFormN, kBufW, p.compact ? kBufHc : kBufH, 0, 0,
                Geom{p.H, p.V, p.H}, Geom{p.H, p.N, p.H}};
}

inline int64_t chunk_rows(const Plan& p, int64_t c) {
  const int64_t v0 = c * p.vchunk;
  return (p.V - v0) < p.vchunk ? (p.V - v0) : p.vchunk;
}

// Elements per 32-column block of the blocked G chunk: its token rows (ldg,
// a multiple of 8) times 32.
inline int64_t g_block(const Plan& p) { return p.ldg * 32; }

// Vocabulary chunks whose probabilities the forward keeps, so that their G
// is formed without recomputing their logits: chunks 0 .. n-1. When dW is the
// call's to overwrite (not added to), chunks 0 .. n-2 go into the part of dW
// that no backward chunk writes before it has used them, and chunk n-1 into
// the G buffer (the recompute of chunk n is the first to write it); otherwise
// n = 1 and chunk 0 goes into the G buffer. Chunk j's probabilities (then
// its G, formed in place) take vchunk x ldg bf16 (the G chunk's blocked
// layout) at byte offset off[j] of dW, the chunks one after another in
// order and ending at the top of dW (rounded down to 256 bytes): each past
// the rows of chunks 0 .. j, which the dH + dW launches of those chunks write
// before or while its G is read. Chunk 0 lowest is what lets the most fit:
// the higher a chunk sits, the more rows may be written below it.
constexpr int kMaxKept = 4;
struct Kept {
  int n = 1;                       // chunks kept: 0 .. n-1
  int64_t off[kMaxKept] = {};      // byte offset into dW of chunk j's G (j < n - 1)
  // where chunk j's G lives: the G buffer or dW
  bool in_dw(int j) const { return j < n - 1; }
};

inline Kept kept_chunks(const Plan& p, bool dw_free) {
  Kept k;
  if (!dw_free || !p.backward || p.g_parts != 1 || p.nr || !p.compact || p.N <= 0) return k;
  const int64_t region = p.vchunk * p.H * 2;      // bytes of one chunk's rows of dW
  const int64_t bytes = p.vchunk * p.ldg * 2;     // bytes of one chunk's G (a multiple of 256)
  const int64_t top = p.V * p.H * 2 / 256 * 256;  // dW's bytes, rounded down
  // m chunks in dW (the last kept one in the G buffer, so m < n_chunks):
  // chunk j at top - (m - j) bytes must start past the rows of chunks 0 .. j
  for (int m = kMaxKept - 1; m >= 1; --m) {
    if (m >= p.n_chunks) continue;
    bool fits = top - m * bytes >= 0;
    for (int j = 0; fits && j < m; ++j) fits = top - (m - j) * bytes >= (j + 1) * region;
    if (!fits) continue;
    for (int j = 0; j < m; ++j) k.off[j] = top - (m - j) * bytes;
    k.n = m + 1;
    return k;
  }
  return k;
}

inline Launch backward_launch(const Plan& p, int64_t c, int which, int part = 0) {
  const int64_t v0 = c * p.vchunk, vcur = chunk_rows(p, c);
  const int64_t g_off = int64_t(part) * p.vchunk * p.ldg;
  const int hb = p.compact ? kBufHc : kBufH;
  if (which == 0)  // Z^T[chunk] = W[chunk] . h^T, then the gradient epilogue
    return Launch{vcur, p.N, p.H, kFormN, kFormN, kBufW, hb, v0 * p.H, 0,
                  Geom{p.H, vcur, p.H}, Geom{p.H, p.N, p.H}};
  // G is stored blocked (g_block(p) elements per 32 vocabulary columns; see
  // Geom): G[t][v - v0] at blocked_offset(t, v - v0, g_block(p)). Columns
  // from vcur to vchunk are never multiplied into a stored output.
  const int64_t blk = g_block(p);
  if (which == 1)  // dW[chunk] = G[:, chunk]^T . h  (K = tokens)
    return Launch{vcur, p.H, p.N, kFormT, kFormT, kBufG, hb, g_off, 0,
                  Geom{32, p.vchunk, p.N, blk}, Geom{p.H, p.H, p.N}};
  // dH += G[:, chunk] . W[chunk]  (K = chunk rows)
  return Launch{p.N, p.H, vcur, kFormN, kFormT, kBufG, kBufW, g_off, v0 * p.H,
                Geom{32, p.N, vcur, blk}, Geom{p.H, p.H, vcur}};
}

// No-recompute variant, token chunk c: tokens [t0, t0 + nt) with t0 = c nc.
// 0: forward over the whole vocabulary (probabilities stored in the G
// buffer, vp columns blocked by 32); 1: dW (+)= G^T . h[chunk] (K = the
// chunk's tokens); 2: dH[chunk] = G . W (K = V, complete in one launch).
inline int64_t nr_chunk_tokens(const Plan& p, int64_t c) {
  const int64_t t0 = c * p.nc;
  return (p.N - t0) < p.nc ? (p.N - t0) : p.nc;
}

// The chunk's probabilities / G are blocked like the G chunk of the recompute
// path (see Geom), nc token rows per 32-column block.
inline int64_t nr_block(const Plan& p) { return p.nc * 32; }

inline Launch nr_launch(const Plan& p, int64_t c, int which) {
  const int64_t t0 = c * p.nc, nt = nr_chunk_tokens(p, c);
  const int hb = p.compact ? kBufHc : kBufH;      // the gathered rows
  if (which == 0)
    return Launch{p.V, nt, p.H, kFormN, kFormN, kBufW, hb, 0, t0 * p.H,
                  Geom{p.H, p.V, p.H}, Geom{p.H, nt, p.H}};
  if (which == 1)
    return Launch{p.V, p.H, nt, kFormT, kFormT, kBufG, hb, 0, t0 * p.H,
                  Geom{32, p.vp, nt, nr_block(p)}, Geom{p.H, p.H, nt}};
  return Launch{nt, p.H, p.V, kFormN, kFormT, kBufG, kBufW, 0, 0,
                Geom{32, nt, p.V, nr_block(p)}, Geom{p.H, p.H, p.V}};
}

FLCE_HD int64_t num_tiles(int64_t M, int64_t Nn) {
  return ((M + kBM - 1) / kBM) * ((Nn + kBM - 1) / kBM);
}

// Element offset that moves an operand's origin to k = k0 (k0 a multiple of
// 32, so a blocked operand moves by whole blocks or block rows).
FLCE_HD int64_t k_origin(int form, const Geom& g, int64_t k0) {
  if (form == kFormN) return g.blk ? (k0 >> 5) * g.blk : k0;
  return g.blk ? k0 * 32 : k0 * g.ld;
}

// Segment z (workgroup index y) of a launch split along K into segments of
// kseg (a multiple of 64): operand origins moved to k0 = z kseg and K cut to
// the segment. Each segment's products go to a partial output of their own.
inline Launch split_segment(const Launch& l, int64_t kseg, int64_t z) {
  Launch s = l;
  const int64_t k0 = z * kseg;
  s.K = (l.K - k0) < kseg ? (l.K - k0) : kseg;
  s.off_a += k_origin(l.fa, l.a, k0);
  s.off_b += k_origin(l.fb, l.b, k0);
  s.a.K = s.K;
  s.b.K = s.K;
  return s;
}

// Workgroups are handed to the 8 XCDs round-robin. Give each XCD a contiguous
// range of tiles, and order tiles within a range in groups of `group_m`
// M-tiles so that the workgroups resident on one XCD share operand tiles in
// that XCD's L2. An XCD's range then covers a contiguous run of M-tiles;
// spread_m (with the M-tile count a multiple of 8) deals the M-tiles to the
// XCDs in turn instead (XCD x gets x, x + 8, ...), for a launch whose first
// M-tiles carry more work: every XCD gets its share of them, and the sharing
// within an XCD is unchanged.
FLCE_HD void tile_coords(int64_t b, int64_t M, int64_t Nn, int group_m, int64_t& m0,
                         int64_t& n0, bool spread_m = false) {
  const int64_t num_m = (M + kBM - 1) / kBM, num_n = (Nn + kBM - 1) / kBM;
  const int64_t total = num_m * num_n;
  const int64_t q = total / 8, rem = total % 8, x = b % 8, local = b / 8;
  const int64_t tile = x * q + (x < rem ? x : rem) + local;
  const int64_t per_group = int64_t(group_m) * num_n;
  const int64_t g = tile / per_group;
  const int64_t first_m = g * group_m;
  const int64_t gs = (num_m - first_m) < group_m ? (num_m - first_m) : group_m;
  const int64_t in = tile - g * per_group;
  int64_t mt = first_m + in % gs;
  if (spread_m && num_m % 8 == 0) {
    const int64_t per = num_m / 8;
    mt = (mt % per) * 8 + mt / per;
  }
  m0 = mt * kBM;
  n0 = (in / gs) * kBM;
}

// LDS layout of one stage tile of an operand. N form: 256 rows x sk k,
// 2 sk bytes per row, sk / 8 chunks of 16 B; logical chunk c of row r at
// position c ^ swz_n(r), the chunk index XORed with bits 1.. of the row. A
// fragment read (16 consecutive rows, one chunk per 16-lane group) then
// reads without LDS bank conflicts, for 64 k (8 chunks per row) and for 32 k
// (4 chunks): the gfx950 bank-conflict counter reads 0 for both read
// patterns, against 4 conflict cycles per read with the 32-k chunk XORed with
// bits 2-3 of the row instead. T form: sk k-rows x 256 columns, 512 B per
// k-row, 32 chunks; logical chunk c of k-row k at c ^ swz_t(k). A transposed
// fragment read (8 bytes per lane) serves 32 lanes at a time, two 16-lane
// groups whose k-rows are 8 apart, each reading 2 chunks of 4 consecutive
// k-rows: the k % 4 term puts one group on 8 distinct bank quads, and the
// XOR 2 on k & 8 puts the other on the 8 quads left, so each half of the
// read covers the 256-byte bank window once. The counter reads 0 for this
// pattern, against 2 conflict cycles per read with the k % 4 term alone.
FLCE_HD int swz_n(int r, int sk) { return sk == 64 ? (r >> 1) & 7 : (r >> 1) & 3; }
FLCE_HD int swz_t(int k) {      // {0,6,10,12}[k % 4], XOR 2 when k & 8
  return ((0xCA60 >> (4 * (k & 3))) & 15) ^ ((k >> 2) & 2);
}

// Where the fragment reads find an element. N form: the 16-byte chunk (8 k
// values) c of row r. T form: byte offset of the 4 columns [col, col + 4) of
// k-row k (col % 4 == 0).
FLCE_HD int lds_chunk_n(int r, int c, int sk) { return r * (sk / 8) + (c ^ swz_n(r, sk)); }
FLCE_HD int lds_byte_t(int k, int col) {
  return (k * 32 + ((col >> 3) ^ swz_t(k))) * 16 + ((col >> 2) & 1) * 8;
}

// Direct-to-LDS loads: element offset of the tile base (k = 0) from the
// operand pointer, elements to advance per stage tile, and the element
// offset of load q of (wave, lane) from the tile base. With L =
// loads_per_operand(sk), load q of wave w fills LDS bytes [(L w + q) KiB,
// +1 KiB), lane l writing 16 B at 16 l, so a lane fetches the logical chunk
// that the swizzle puts at its LDS position: in the N form 1024 / (2 sk) rows
// of 2 sk bytes per load, in the T form 2 k-rows of 512 B. Rows (N form) or
// column chunks (T form) past the edge are clamped to the last valid one:
// their products land outside the output and are never stored.
FLCE_HD int64_t direct_base(int form, const Geom& g, int64_t row0) {
  if (form == kFormN) return row0 * g.ld;
  return g.blk ? (row0 >> 5) * g.blk : row0;      // row0 is a multiple of 256
}
FLCE_HD int64_t direct_kstep(int form, const Geom& g, int sk) {
  if (form == kFormN) return g.blk ? int64_t(sk >> 5) * g.blk : int64_t(sk);
  return int64_t(sk) * g.ld;
}
FLCE_HD int64_t direct_lane(int form, const Geom& g, int64_t row0, int wave, int lane, int q,
                            int sk) {
  const int L = loads_per_operand(sk);
  if (form == kFormN) {
    const int cpr = sk / 8;                           // chunks per row
    const int lr = (64 / cpr) * (L * wave + q) + lane / cpr;
    const int c = (lane % cpr) ^ swz_n(lr, sk);
    int64_t r = row0 + lr;
    if (r > g.rows - 1) r = g.rows - 1;
    return (r - row0) * g.ld + 8 * c;
  }
  const int kr = 2 * (L * wave + q) + (lane >> 5);
  const int c = (lane & 31) ^ swz_t(kr);
  int64_t col = 8 * c;
  if (row0 + col > g.rows - 8) col = g.rows - 8 - row0;
  return g.blk ? (col >> 5) * g.blk + kr * 32 + (col & 31) : kr * g.ld + col;
}

// Register path of a partial last stage tile: thread tid's load i covers
// z = tid + 256 i (i < tail_loads(sk)). Returns whether it reads memory
// (else it stores zeros) and the element offset from the operand pointer.
FLCE_HD bool tail_src(int form, const Geom& g, int64_t row0, int64_t k0, int z, int sk,
                      int64_t& off) {
  if (form == kFormN) {  // z -> (row z / cpr, chunk z % cpr)
    const int cpr = sk / 8;
    const int64_t gr = row0 + z / cpr, gk = k0 + 8 * (z % cpr);
    off = g.blk ? blocked_offset(gr, gk, g.blk) : gr * g.ld + gk;
    return gr < g.rows && gk < g.K;
  }
  const int64_t gk = k0 + (z >> 5), gm = row0 + 8 * (z & 31);  // (k-row z / 32, chunk z % 32)
  off = g.blk ? blocked_offset(gk, gm, g.blk) : gk * g.ld + gm;
  return gk < g.K && gm < g.rows;
}

// LDS chunk position (16-byte units) of the tail element z.
FLCE_HD int tail_lds_pos(int form, int z, int sk) {
  return form == kFormN ? lds_chunk_n(z / (sk / 8), z % (sk / 8), sk)
                        : lds_byte_t(z >> 5, 8 * (z & 31)) / 16;
}

}  // namespace gemm
}  // namespace flce
