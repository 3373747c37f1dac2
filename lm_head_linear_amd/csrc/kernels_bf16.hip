// bf16 path on CDNA4 matrix cores (gfx950).
//
// One GEMM main loop serves every contraction of the step:
//   forward   Z^T tile = W[v-tile] . h[t-tile]^T        (K = H)
//   recompute Z^T tile, then the logit-gradient epilogue (K = H)
//   dW chunk  = G^T[chunk] . h                          (K = tokens)
//   dH       += G[:, chunk] . W[chunk]                  (K = vocab chunk)
// Workgroup tile 256 x 256, four waves of 128 x 128 each built from
// v_mfma_f32_16x16x32_bf16 (fp32 accumulate; 64 of them per wave and 32-k
// step). Of the two bf16 matrix instructions this one holds a higher clock
// under the chip's power limit at the same issue rate. Operands go
// global -> LDS with direct-to-LDS loads (no registers) into XOR-swizzled
// stages: 2 stages of 64 k when both operands are K-contiguous, 5 of 32 k
// when either is transposed (dW, dH). A K-contiguous operand's fragments are
// read with ds_read_b128; one stored with its M/N dimension contiguous is read
// with the gfx950
// transpose read ds_read_b64_tr_b16, so no operand is ever transposed in
// registers or in memory.
//
// Tiles are computed with the vocabulary on the M side and tokens on the N
// side for the logit tiles: a lane then owns 8 token columns and 32 vocab
// values of each, so the per-token max / sum-exp reductions of the forward
// epilogue stay inside the lane (plus two exchanges among the four lanes of a
// column and one between the two waves of a column).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "../../include/flce.h"
#include "flce_internal.h"
#include "gemm_index.h"

namespace flce {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kBM = gemm::kBM;
constexpr int kThreads = 256;
constexpr int kWaveScratch = 32768;               // LDS bytes per wave in the epilogues
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  // Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
  return __builtin_bit_cast(uint16_t, __bf16(f));
}
// Two values rounded to nearest even and packed (lo = a) in one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 v = {__bf16(a), __bf16(b)};
  return __builtin_bit_cast(uint32_t, v);
}

using gemm::Geom;
using gemm::kBK;

// An operand of the GEMM: a pointer and its geometry (see gemm_index.h).
struct Operand {
  const uint16_t* ptr;
  Geom g;
};

// Per-thread state of one operand's direct-to-LDS loads: a wave-uniform tile
// base advanced by `kstep` bytes per stage tile, and one 32-bit byte offset
// per load (see gemm::direct_lane for the layout and the edge clamping).
template <int L>
struct DirectLoads {
  const char* base;
  int64_t kstep;
  uint32_t off[L];
};

template <int FORM, int SK>
__device__ __forceinline__ DirectLoads<gemm::loads_per_operand(SK)> setup_direct(
    const Operand& op, int64_t row0, int wave, int lane) {
  constexpr int L = gemm::loads_per_operand(SK);
  DirectLoads<L> d;
  d.base = reinterpret_cast<const char*>(op.ptr + gemm::direct_base(FORM, op.g, row0));
  d.kstep = gemm::direct_kstep(FORM, op.g, SK) * 2;
#pragma unroll
  for (int q = 0; q < L; ++q)
    d.off[q] = uint32_t(gemm::direct_lane(FORM, op.g, row0, wave, lane, q, SK) * 2);
  return d;
}

// Issue one stage tile of direct loads into an LDS tile (256 x SK bf16): load
// q of wave w fills LDS bytes [(L w + q) KiB, +1 KiB), lane l writing 16 B at
// 16 l.
template <int L>
__device__ __forceinline__ void issue_direct(const DirectLoads<L>& d, int64_t kt, char* lds,
                                             int wave) {
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass instantiates templates without gfx950 builtins
  const char* b = d.base + kt * d.kstep;
#pragma unroll
  for (int q = 0; q < L; ++q)
    __builtin_amdgcn_global_load_lds(
        b + d.off[q], (__attribute__((address_space(3))) void*)(lds + (L * wave + q) * 1024), 16,
        0, 0);
#else
  (void)d, (void)kt, (void)lds, (void)wave;
#endif
}

// Load q (0 .. L-1) of issue_direct alone.
template <int L>
__device__ __forceinline__ void issue_one(const DirectLoads<L>& d, int64_t kt, char* lds, int wave,
                                          int q) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(
      d.base + kt * d.kstep + d.off[q],
      (__attribute__((address_space(3))) void*)(lds + (L * wave + q) * 1024), 16, 0, 0);
#else
  (void)d, (void)kt, (void)lds, (void)wave, (void)q;
#endif
}

// Per-token inputs of an epilogue, staged in LDS past the pipeline stages:
// W 4-byte words per token (W = 1 for float, 2 for int64) of the workgroup's
// 256 token columns n0 .. n0 + 255 (clamped to the last of n tokens), loaded
// with direct-to-LDS loads when the kernel starts, so that their latency
// passes under the K loop instead of stalling the epilogue. Thread tid of
// wave w issues word e = q * 256 + tid of pass q into lds[4 e].
template <int W>
__device__ __forceinline__ void stage_tokens(char* lds, const void* src, int64_t n0, int64_t n,
                                             int wave, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int q = 0; q < W; ++q) {
    const int e = q * 256 + wave * 64 + lane;
    const int64_t t = n0 + e / W;
    const char* p = static_cast<const char*>(src) + ((t < n ? t : n - 1) * W + e % W) * 4;
    __builtin_amdgcn_global_load_lds(
        p, (__attribute__((address_space(3))) void*)(lds + (q * 256 + wave * 64) * 4), 4, 0, 0);
  }
#else
  (void)lds, (void)src, (void)n0, (void)n, (void)wave, (void)lane;
#endif
}

// Register path for a partial last stage tile: zero-filled past K (and past
// the matrix edge), then stored into the same LDS layout.
template <int FORM, int SK>
__device__ __forceinline__ void load_tail(u32x4 (&r)[gemm::tail_loads(SK)], const Operand& op,
                                          int64_t row0, int64_t k0, int tid) {
#pragma unroll
  for (int i = 0; i < gemm::tail_loads(SK); ++i) {
    int64_t off;
    const bool ok = gemm::tail_src(FORM, op.g, row0, k0, tid + 256 * i, SK, off);
    r[i] = ok ? *reinterpret_cast<const u32x4*>(op.ptr + off) : u32x4{0u, 0u, 0u, 0u};
  }
}

template <int FORM, int SK>
__device__ __forceinline__ void store_tail(char* lds, const u32x4 (&r)[gemm::tail_loads(SK)],
                                           int tid) {
#pragma unroll
  for (int i = 0; i < gemm::tail_loads(SK); ++i)
    *reinterpret_cast<u32x4*>(lds + gemm::tail_lds_pos(FORM, tid + 256 * i, SK) * 16) = r[i];
}

// MFMA fragment of 16 rows (row_base .. row_base + 15 of the tile) for the
// 32-wide K part p (0 .. SK/32 - 1) of a stage tile: lane l holds row
// row_base + l % 16 at k = 32 p + 8 (l / 16) + 0..7. Both operands use the
// same k order, which is all the product needs.
template <int FORM, int SK>
__device__ __forceinline__ bf16x8 read_frag(const char* lds, int row_base, int p, int lane) {
  if (FORM == 0) {
    const int row = row_base + (lane & 15);
    const int c = 4 * p + (lane >> 4);
    const u32x4 v = *reinterpret_cast<const u32x4*>(lds + gemm::lds_chunk_n(row, c, SK) * 16);
    return __builtin_bit_cast(bf16x8, v);
  } else {
    // Lane i of a 16-lane group receives element i % 4 of the 8-byte chunks
    // read by lanes 4e + i / 4 (e = 0..3): lane i reads k-row base + i / 4 at
    // columns 4 (i % 4) .. + 3, so lane i gets column i at k-rows base + 0..3.
    typedef __attribute__((ext_vector_type(4))) short s16x4;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int g = lane >> 4, i = lane & 15;
    const int col = row_base + 4 * (i & 3);
    s16x4 h[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int k = 32 * p + 8 * g + 4 * r + (i >> 2);
      h[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + gemm::lds_byte_t(k, col)));
    }
    typedef __attribute__((ext_vector_type(8))) short s16x8;
    const s16x8 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
    return __builtin_bit_cast(bf16x8, v);
  }
}

// A wave's accumulators: 8 x 8 blocks of 16 x 16, four values per lane.
// Element (i, j, r) sits at tile row wm*128 + i*16 + 4*(lane/16) + r and
// tile column wn*128 + j*16 + lane%16 (the 16x16 MFMA output layout), so a
// lane holds 4 consecutive rows of each block and the four lanes l, l ^ 16,
// l ^ 32, l ^ 48 share its columns.
typedef f32x4 Acc[8][8];

__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * 128 + i * 16 + 4 * (lane >> 4) + r;
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) {
  return wn * 128 + j * 16 + (lane & 15);
}

// Max and sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 that share an
// accumulator column, with the gfx950 lane swaps (VALU, no LDS round trip).
// permlane16_swap(x, x) yields x of lanes l & ~16 and l | 16, and
// permlane32_swap(x, x) those of lanes l & ~32 and l | 32, in that order in
// every lane, so all four lanes get the same bits.
__device__ __forceinline__ float col_max4(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
#endif
  return x;
}
__device__ __forceinline__ float col_sum4(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(b[0]) + __uint_as_float(b[1]);
#endif
  return x;
}

// Waits of the K loop (gfx9 s_waitcnt encoding: vmcnt bits [3:0] and
// [15:14], expcnt [6:4], lgkmcnt [11:8]; a field at its maximum does not
// wait).
__device__ __forceinline__ void wait_vm24() { __builtin_amdgcn_s_waitcnt(0x4F78); }   // vmcnt(24)
__device__ __forceinline__ void wait_vm16() { __builtin_amdgcn_s_waitcnt(0x4F70); }   // vmcnt(16)
__device__ __forceinline__ void wait_vm8() { __builtin_amdgcn_s_waitcnt(0x0F78); }    // vmcnt(8)
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }    // vmcnt(0)
__device__ __forceinline__ void wait_vm0_lgkm0() { __builtin_amdgcn_s_waitcnt(0x0070); }

// Workgroup barrier for the K loop. Unlike __syncthreads() it implies no
// memory fence or wait: the waits that order the pipeline are explicit
// before it. The empty asm statements keep the compiler from moving memory
// accesses across it, the scheduling barriers keep MFMAs on their side.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// MFMA fragments of one step (32 k) for the wave's 128 x 128 block: 32-wide
// part `part` of a stage tile, 8 row blocks of each operand.
struct StepFrags {
  bf16x8 a[8], b[8];
};

template <int FA, int FB, int SK>
__device__ __forceinline__ void read_step(StepFrags& f, const char* sa, const char* sb, int part,
                                          int wm, int wn, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.a[i] = read_frag<FA, SK>(sa, wm * 128 + i * 16, part, lane);
#pragma unroll
  for (int j = 0; j < 8; ++j) f.b[j] = read_frag<FB, SK>(sb, wn * 128 + j * 16, part, lane);
}

__device__ __forceinline__ void mfma_step(Acc& acc, const StepFrags& f) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Scheduling hints for a step of dH (K-contiguous G, transposed W): its 64
// MFMAs, the fragment reads of the next step after the first MFMAs (all in
// the first half of the step), and the NLOADS direct loads one after every
// second MFMA of the second half, so everything issues under the MFMAs.
template <int FA, int FB, int NLOADS>
__device__ __forceinline__ void interleave_hints() {
  constexpr int kReads = (FA == 0 ? 8 : 16) + (FB == 0 ? 8 : 16);
#pragma unroll
  for (int q = 0; q < 64; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // MFMA
    const bool load = q >= 32 && q % 2 == 0 && (q - 32) / 2 < NLOADS;
    if (NLOADS > 0 && load) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
    if (q < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
  }
}

// One MFMA step: optionally start the direct loads of a stage tile into its
// (free) stage, read the fragments of the next step (32-wide part
// `next_part` of the stage tile at na/nb) and multiply the current step,
// whose fragments were read during the previous one. The stages are
// __restrict__ so the compiler does not order the direct-to-LDS writes
// against the reads; the real dependencies are the waits and the barriers.
//
// The forward/gradient GEMMs (both operands K-contiguous, 16 loads on every
// other step) and dW (both transposed, 8 loads per step) issue the step as 16
// chunks of 4 MFMAs, fenced by scheduling barriers: the fragment reads of the
// next step in chunks 0..7 (row block c of each operand in chunk c, after the
// first chunk's MFMAs, so that their wait for the current fragments does not
// include the new reads), and the direct loads one per chunk (A and B
// alternating) or one per chunk of the second half. Left to scheduling hints,
// the compiler bunched 14 of the 16 loads of the K-contiguous steps back to
// back. dH measured faster with the hints.
template <int FA, int FB, int SK, bool LOADS, int L>
__device__ __forceinline__ void k_step(Acc& acc, const StepFrags& cur, StepFrags& nxt,
                                       const DirectLoads<L>& da, const DirectLoads<L>& db,
                                       int64_t load_tile, const char* __restrict__ na,
                                       const char* __restrict__ nb, int next_part,
                                       char* __restrict__ la, char* __restrict__ lb, int wave,
                                       int wm, int wn, int lane) {
  if constexpr (FA != FB) {
    if (LOADS) {
      issue_direct<L>(da, load_tile, la, wave);
      issue_direct<L>(db, load_tile, lb, wave);
    }
    read_step<FA, FB, SK>(nxt, na, nb, next_part, wm, wn, lane);
    mfma_step(acc, cur);
    interleave_hints<FA, FB, LOADS ? 2 * L : 0>();
  } else {
    constexpr bool kNN = FA == 0;
    static_assert(2 * L == (kNN ? 16 : 8), "one load per chunk (of the second half)");
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int i = c >> 1;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = 4 * (c & 1) + jj;
        acc[i][j] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.a[i], cur.b[j], acc[i][j], 0, 0, 0);
      }
      if (c == 0) __builtin_amdgcn_sched_barrier(0);
      if (c < 8) {
        nxt.a[c] = read_frag<FA, SK>(na, wm * 128 + c * 16, next_part, lane);
        nxt.b[c] = read_frag<FB, SK>(nb, wn * 128 + c * 16, next_part, lane);
      }
      if (LOADS) {
        if (kNN) {
          if (c & 1) issue_one<L>(db, load_tile, lb, wave, c >> 1);
          else       issue_one<L>(da, load_tile, la, wave, c >> 1);
        } else if (c >= 8) {
          const int q = c - 8;
          if (q < L) issue_one<L>(da, load_tile, la, wave, q);
          else       issue_one<L>(db, load_tile, lb, wave, q - L);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The K loop of one tile: acc += A[m0 .. m0 + 255][0, K) . B[n0 .. n0 + 255][0, K)^T
// through the LDS stages at smem: a partial last stage tile first (through
// registers), then the pipelined full stage tiles. Every wave leaves it
// behind a barrier, with no load in flight.
template <int FA, int FB>
__device__ __forceinline__ void k_loop(Acc& acc, const Operand& A, const Operand& B, int64_t K,
                                       int64_t m0, int64_t n0, char* smem, int tid, int lane,
                                       int wave, int wm, int wn) {
  constexpr int SK = gemm::stage_k(FA, FB);
  constexpr int kStages = gemm::num_stages(FA, FB);
  constexpr int L = gemm::loads_per_operand(SK);
  constexpr int kTileBytes = kBM * SK * 2;          // one operand, one stage

  const DirectLoads<L> da = setup_direct<FA, SK>(A, m0, wave, lane);
  const DirectLoads<L> db = setup_direct<FB, SK>(B, n0, wave, lane);
  const int64_t nfull = K / SK;                // stage tiles loaded directly
  const int64_t nk = (K + SK - 1) / SK;        // plus a zero-filled partial tile

  auto st_a = [&](int64_t t) { return smem + (t % kStages) * 2 * kTileBytes; };
  auto st_b = [&](int64_t t) { return smem + (t % kStages) * 2 * kTileBytes + kTileBytes; };
  if (nk > nfull) {
    // The partial last stage tile goes through registers, zero-filled past K,
    // into stage 0, and is multiplied first, before the pipelined loop, whose
    // prologue then reuses the stage (behind the barrier). Placed after the
    // loop instead, it made the register allocator shuffle the 64
    // accumulator tuples through copies and spills inside the loop.
    char* la = st_a(0);
    char* lb = st_b(0);
    u32x4 ta[gemm::tail_loads(SK)], tb[gemm::tail_loads(SK)];
    load_tail<FA, SK>(ta, A, m0, nfull * SK, tid);
    load_tail<FB, SK>(tb, B, n0, nfull * SK, tid);
    store_tail<FA, SK>(la, ta, tid);
    store_tail<FB, SK>(lb, tb, tid);
    __syncthreads();
    StepFrags ft;
#pragma unroll
    for (int part = 0; part < SK / 32; ++part) {
      read_step<FA, FB, SK>(ft, la, lb, part, wm, wn, lane);
      mfma_step(acc, ft);
    }
    __syncthreads();
  }
  if (nfull > 0) {
    const int64_t last = nfull - 1;
    StepFrags f[2];
    if constexpr (SK == 64) {
      // Two stages of 64 k, two MFMA steps (the two 32-wide halves) per stage
      // tile; stage tile t lives in stage t % 2 and the fragments of a step
      // are read during the step before it. Even step (first half of tile
      // t): multiply it, read the second half; no wait, no barrier. Odd step
      // (second half): wait until this wave's loads of tile t+1 have landed
      // and its reads of tile t have returned, then a barrier -- tile t+1 is
      // published and no wave reads tile t's stage any more -- so the loads
      // of tile t+2 go into it; read the first half of tile t+1. A tile's
      // loads thus have two steps to land. Every odd step issues one tile
      // (past the last one it re-loads the last into the free stage), so
      // the body has no branches for the scheduler to stop at.
      issue_direct<L>(da, 0, st_a(0), wave);
      issue_direct<L>(db, 0, st_b(0), wave);
      issue_direct<L>(da, last > 0 ? 1 : 0, st_a(1), wave);
      issue_direct<L>(db, last > 0 ? 1 : 0, st_b(1), wave);
      wait_vm16();                                 // tile 0 landed
      stage_barrier();
      read_step<FA, FB, SK>(f[0], st_a(0), st_b(0), 0, wm, wn, lane);
      for (int64_t t = 0; t < nfull; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        k_step<FA, FB, SK, false>(acc, f[0], f[1], da, db, 0, st_a(t), st_b(t), 1, nullptr,
                                  nullptr, wave, wm, wn, lane);
        __builtin_amdgcn_sched_barrier(0);
        wait_vm0_lgkm0();
        stage_barrier();
        const int64_t lt = t + 2 < last ? t + 2 : last;
        k_step<FA, FB, SK, true>(acc, f[1], f[0], da, db, lt, st_a(t + 1), st_b(t + 1), 0,
                                 st_a(t), st_b(t), wave, wm, wn, lane);
      }
    } else {
      // Five stages of 32 k, one MFMA step per stage tile; tile t lives in
      // stage t % 5, is loaded 4 steps ahead and its fragments are read
      // during step t-1. Every step issues exactly one tile (past the last
      // one it re-loads the last into a free stage), so the number of loads
      // in flight at each wait is the same and the body has no branches for
      // the scheduler to stop at. A barrier only at even steps: the barrier
      // at the top of even step k publishes tiles k+1 and k+2 (only tile k+3
      // may still be in flight) and frees the stages of all tiles up to k,
      // whose fragments were read before it; step k loads tile k+4 into the
      // stage of tile k-1 and the odd step k+1 loads tile k+5 into the stage
      // of tile k. Stage indices advance by one per step in wave-uniform
      // registers (5 is not a power of two). With the LDS bank conflicts of
      // the transposed and 32-k reads removed, five stages measured faster
      // than four with a barrier per step for dH too (its launch 4% faster).
      static_assert(kStages == 5, "five stages of 32 k");
      auto next_stage = [](int x) { return x == kStages - 1 ? 0 : x + 1; };
#pragma unroll
      for (int t = 0; t < kStages - 1; ++t) {
        issue_direct<L>(da, t < last ? t : last, st_a(t), wave);
        issue_direct<L>(db, t < last ? t : last, st_b(t), wave);
      }
      wait_vm24();                                 // tile 0 landed (three more in flight)
      stage_barrier();
      read_step<FA, FB, SK>(f[0], st_a(0), st_b(0), 0, wm, wn, lane);
      int s_read = 1, s_load = kStages - 1;        // stages of tiles k+1 and k+4
      int64_t kt = 0;
      // two steps per iteration: the even one with the barrier, then the odd one
      for (; kt + 1 < nfull; kt += 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int64_t k = kt + u;
          __builtin_amdgcn_sched_barrier(0);
          if (u == 0) {
            wait_vm8();                            // all but the newest tile landed
            stage_barrier();
          }
          const int64_t lt = k + kStages - 1;
          char* sa = smem + s_read * 2 * kTileBytes;
          char* la = smem + s_load * 2 * kTileBytes;
          k_step<FA, FB, SK, true>(acc, f[u], f[u ^ 1], da, db, lt < last ? lt : last, sa,
                                   sa + kTileBytes, 0, la, la + kTileBytes, wave, wm, wn, lane);
          s_read = next_stage(s_read);
          s_load = next_stage(s_load);
        }
      }
      if (kt < nfull) {                            // odd number of steps: the last one (even)
        wait_vm8();
        stage_barrier();
        const int64_t lt = kt + kStages - 1;
        char* sa = smem + s_read * 2 * kTileBytes;
        char* la = smem + s_load * 2 * kTileBytes;
        k_step<FA, FB, SK, true>(acc, f[0], f[1], da, db, lt < last ? lt : last, sa,
                                 sa + kTileBytes, 0, la, la + kTileBytes, wave, wm, wn, lane);
      }
    }
    // the re-loads past the last tile may still be in flight
    wait_vm0();
    stage_barrier();
  }
}

// Which dimension of a launch is cut on the device to the count at `dyn`
// (the non-ignored tokens of a compact plan): none, M, N or K. The grid is
// sized for the launch's sizes (an upper bound); a cut M or N makes the tile
// raster run over the live tiles, and the workgroups past them leave at once,
// before any load.
enum Dyn : int { kDynNone = 0, kDynM = 1, kDynN = 2, kDynK = 3 };

// Whether an epilogue asks for the raster that deals M-tiles to the XCDs in
// turn (gemm::tile_coords): one whose first M-tiles do more work.
template <class E, class = void>
struct SpreadM : std::false_type {};
template <class E>
struct SpreadM<E, std::void_t<decltype(E::kSpreadM)>> : std::bool_constant<E::kSpreadM> {};

// LDS bytes of a GEMM's stages (reused by its epilogue: 32 KiB per wave).
template <int FA, int FB>
constexpr int stage_bytes() {
  return gemm::num_stages(FA, FB) * 2 * kBM * gemm::stage_k(FA, FB) * 2;
}

// One workgroup tile of a GEMM launch: workgroup `bid` of the launch's tile
// raster (and K segment `seg` of a split launch), with the LDS at smem: the
// stages, then the epilogue's per-token inputs.
template <int FA, int FB, class Epi, bool BA, int SEGS, bool SPLITK, int DYN>
__device__ __forceinline__ void gemm_tile(char* smem, int64_t bid, int seg, Operand A,
                                          Operand B, int64_t M, int64_t Nn, int64_t K,
                                          int group_m, Epi epi, int64_t a2_off,
                                          const int64_t* dyn) {
  // BA: operand A is the blocked G (gemm::Geom). Fixing blk at compile time
  // for the dense operands lets the address arithmetic drop the blocked case.
  // SEGS = 2: a second K loop over A shifted by a2_off elements (the lo half
  // of a split G) against the same B, into the same accumulators, so the
  // tile is (A + A2) . B^T with one epilogue.
  // SPLITK: the GEMM is split along K into segments of a2_off (a multiple of
  // 64); this workgroup takes segment `seg` and its epilogue writes a partial
  // product.
  static_assert(SEGS == 1 || SEGS == 2, "one or two K segments");
  static_assert(!(SPLITK && SEGS == 2), "a split GEMM has one K segment per workgroup");
  if constexpr (!BA) A.g.blk = 0;
  B.g.blk = 0;
  if constexpr (SPLITK) {
    epi.select_segment(seg);
    const int64_t k0 = int64_t(seg) * a2_off;
    K = (K - k0) < a2_off ? (K - k0) : a2_off;
    A.ptr += gemm::k_origin(FA, A.g, k0);
    B.ptr += gemm::k_origin(FB, B.g, k0);
    A.g.K = K;
    B.g.K = K;
  }
  constexpr int SK = gemm::stage_k(FA, FB);
  constexpr int kStages = gemm::num_stages(FA, FB);
  constexpr int L = gemm::loads_per_operand(SK);
  constexpr int kSmemBytes = stage_bytes<FA, FB>();      // 128 or 160 KiB
  static_assert(kSmemBytes >= 4 * kWaveScratch, "epilogue staging");
  static_assert(kBK == 32 && (SK == 32 || SK == 64), "MFMA steps of 32 k");
  static_assert(2 * L == (SK == 64 ? 16 : 8), "waitcnt immediates");
  static_assert(SK == 64 ? kStages == 2 : kStages == 5, "pipeline depth");
  if constexpr (DYN == kDynM || DYN == kDynN) {
    // The raster runs over the live tiles: the workgroups past them leave at
    // once, and the live ones are spread over all XCDs (a raster over the
    // launch's upper bound would leave the XCDs that own the dead tiles idle).
    const int64_t d = *dyn;
    if constexpr (DYN == kDynM) {
      M = d < M ? d : M;
      epi.N = M;                                   // the epilogue's token rows
    } else {
      Nn = d < Nn ? d : Nn;
      epi.N = Nn;                                  // the epilogue's token columns
    }
    if (bid >= gemm::num_tiles(M, Nn)) return;
  }
  int64_t m0, n0;
  gemm::tile_coords(bid, M, Nn, group_m, m0, n0, SpreadM<Epi>::value);
  if constexpr (DYN == kDynK) {
    const int64_t d = *dyn;
    K = d < K ? d : K;                             // past the count: zero-filled
    A.g.K = K;
    B.g.K = K;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  // first in the queue, so every later counted wait of the pipeline covers it
  epi.stage(smem + kSmemBytes, n0, wave, lane);

  Acc acc;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

  k_loop<FA, FB>(acc, A, B, K, m0, n0, smem, tid, lane, wave, wm, wn);
  if constexpr (SEGS == 2)
    k_loop<FA, FB>(acc, Operand{A.ptr + a2_off, A.g}, B, K, m0, n0, smem, tid, lane, wave, wm, wn);
  __syncthreads();
  epi(acc, m0, n0, wm, wn, lane, smem, smem + kSmemBytes);
}

// A GEMM launch over dense operands (the forward and gradient GEMMs): one
// workgroup per tile. The stages are one __shared__ array: with a second LDS
// object the compiler can no longer tell the direct-to-LDS writes of one
// stage from the reads of another and serialises the pipeline.
template <int FA, int FB, class Epi, int DYN>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(Operand A, Operand B, int64_t M,
                                                      int64_t Nn, int64_t K, int group_m,
                                                      Epi epi, const int64_t* dyn) {
  __shared__ __attribute__((aligned(1024))) char smem[stage_bytes<FA, FB>() + Epi::kTokBytes];
  gemm_tile<FA, FB, Epi, false, 1, false, DYN>(smem, blockIdx.x, 0, A, B, M, Nn, K, group_m, epi,
                                               0, dyn);
}

// Two independent GEMMs of one backward chunk in one grid: the n1 workgroups
// of the first (padded to a multiple of 8, so the XCD raster of the second
// stays aligned) and then those of the second. The dH GEMM goes first: with
// the kept tokens only, its tiles may fill its last round of workgroups only
// in part, and the shorter dW tiles behind it fill the rest instead of the
// next launch starting on an idle chip. One LDS array serves both.
// SPLIT1: the first GEMM is split along K into segments of off1 rows, its
// n1 = t1 x segments workgroups segment by segment (workgroup b: segment
// b / t1, tile b % t1), each writing a partial product of its own.
// SEGS = 2 (float32 gradients): both GEMMs run their K loop over the hi part
// of G and then over the lo part, off1 (= off2) elements further.
template <int FA1, int FB1, class Epi1, int DYN1, bool SPLIT1, int FA2, int FB2, class Epi2,
          int DYN2, int SEGS>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_pair(
    int64_t n1p, int64_t t1, int64_t n1, int64_t off1, Operand A1, Operand B1, int64_t M1,
    int64_t N1, int64_t K1, Epi1 e1, Operand A2, Operand B2, int64_t M2, int64_t N2, int64_t K2,
    Epi2 e2, int64_t off2, const int64_t* dyn) {
  static_assert(!(SPLIT1 && SEGS == 2), "a split GEMM has one K segment per workgroup");
  constexpr int kB1 = stage_bytes<FA1, FB1>() + Epi1::kTokBytes;
  constexpr int kB2 = stage_bytes<FA2, FB2>() + Epi2::kTokBytes;
  __shared__ __attribute__((aligned(1024))) char smem[kB1 > kB2 ? kB1 : kB2];
  const int64_t b = blockIdx.x;
  if (b < n1p) {
    if (b >= n1) return;
    if constexpr (SPLIT1) {
      const int64_t seg = b / t1;
      gemm_tile<FA1, FB1, Epi1, true, 1, true, DYN1>(smem, b - seg * t1, int(seg), A1, B1, M1,
                                                     N1, K1, gemm::kGroupM, e1, off1, dyn);
    } else {
      gemm_tile<FA1, FB1, Epi1, true, SEGS, false, DYN1>(smem, b, 0, A1, B1, M1, N1, K1,
                                                         gemm::kGroupM, e1, off1, dyn);
    }
  } else {
    gemm_tile<FA2, FB2, Epi2, true, SEGS, false, DYN2>(smem, b - n1p, 0, A2, B2, M2, N2, K2,
                                                       gemm::kGroupM, e2, off2, dyn);
  }
}

// tanh(x) = 1 - 2 / (exp(2x) + 1), from the hardware exp2 and reciprocal.
// Exact limits +-1 for large |x|; absolute error a few 1e-7, which the
// softcap scale s turns into a logit error of a few s * 1e-7.
__device__ __forceinline__ float tanh_fast(float x) {
  const float e = __builtin_amdgcn_exp2f(x * (2.f * kLog2e));
  return 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);
}

// XOR swizzle of the 8-byte slots of a staged token row (32 slots, 256 bytes,
// one bank window): 2 b(t) with b(t) the 4-bit token t % 16 with its two
// halves swapped. Even, so the 16-byte runs read back stay whole. A staging
// write of 32 lanes (two 16-lane groups g, g + 1, 16 tokens each) covers all
// 64 banks once (g goes to bit 0, b(t) to bits 1..4), and so does a 16-lane
// read of 4 chunks of 4 consecutive tokens (the token's two low bits land
// above the chunk's).
__device__ __forceinline__ int token_swizzle(int tl) {
  return 8 * (tl & 3) + 2 * ((tl >> 2) & 3);
}

// ---- token-major logits output of the forward --------------------------
// Kinds of logits output of the forward epilogue.
enum LogitsOut : int { kNoLogits = 0, kLogitsF32 = 1, kLogitsBF16 = 2 };

// Stores the tile's logits (rows vocabulary ids, columns tokens, masked rows
// v >= V never stored) row-major by token: out[t][v], row length ld, as
// float32 or as bf16 rounded to nearest even. Each wave stages its block in
// its own 32 KiB of LDS as [token][vocab]: bf16 all 128 vocabulary rows in
// one pass (8-byte slots, as in store_token_major), float32 64 rows (row
// blocks i of 16, four per pass) per pass (16-byte slots holding a lane's 4
// consecutive vocabulary values, XOR-swizzled by token), then writes 16-byte
// runs of token rows. A run that would cross V,
// and every run when `vec` is 0 (destination or row length not 16-byte
// aligned), is written element by element. Ends with a barrier, so the
// caller may reuse the LDS at once.
template <int OUT>
__device__ __forceinline__ void store_logits(const Acc& acc, char* smem, int wm, int wn, int lane,
                                             void* out, int64_t ld, int vec, int64_t m0,
                                             int64_t n0, int64_t N, int64_t V) {
  constexpr bool F32 = OUT == kLogitsF32;
  constexpr int kPasses = F32 ? 2 : 1;
  constexpr int kRun = F32 ? 4 : 8;                // elements per 16-byte run
  const int g = lane >> 4;
  char* reg = smem + (wm + 2 * wn) * kWaveScratch;
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    if (ps) __syncthreads();                       // the previous pass has been read
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tl = j * 16 + (lane & 15);
#pragma unroll
      for (int ii = 0; ii < 8 / kPasses; ++ii) {
        const int i = ii + ps * (8 / kPasses);
        const f32x4 v = acc[i][j];
        if (F32) {
          const int slot = (ii * 4 + g) ^ (tl & 15);
          *reinterpret_cast<u32x4*>(reg + tl * 256 + slot * 16) =
              u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                    __float_as_uint(v[3])};
        } else {
          const int slot = (i * 4 + g) ^ token_swizzle(tl);
          *reinterpret_cast<uint2*>(reg + tl * 256 + slot * 8) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int q = 0; q < 32; ++q) {
      const int idx = q * 64 + lane;
      const int tl = idx >> 4, ch = idx & 15;
      u32x4 v;
      if (F32) {
        v = *reinterpret_cast<const u32x4*>(reg + tl * 256 + (ch ^ (tl & 15)) * 16);
      } else {
        v = *reinterpret_cast<const u32x4*>(reg + tl * 256 + ((2 * ch) ^ token_swizzle(tl)) * 8);
      }
      const int64_t t = n0 + wn * 128 + tl;
      const int64_t vl = m0 + wm * 128 + (F32 ? ps * 64 + 4 * ch : 8 * ch);
      if (t < N && vl < V) {
        if (vec && vl + kRun <= V) {
          char* dst = static_cast<char*>(out) + (t * ld + vl) * (F32 ? 4 : 2);
          *reinterpret_cast<u32x4*>(dst) = v;
        } else {
          const int n = int(V - vl < kRun ? V - vl : kRun);
          for (int e = 0; e < n; ++e) {
            if (F32)
              static_cast<uint32_t*>(out)[t * ld + vl + e] = v[e];
            else
              static_cast<uint16_t*>(out)[t * ld + vl + e] = uint16_t(v[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    }
  }
  __syncthreads();
}

// ---- token-major bf16 stores of a tile held in the accumulators ----------
// The tile's rows are vocabulary ids, its columns tokens; the destination is
// row-major by token, dst[t][v] with row length ld, or (BLOCKED) blocked,
// dst[blocked_offset(t, v, blk)]. Each wave stages its
// 128 x 128 block in its own 32 KiB of LDS as [token][vocab] (a lane packs
// its 4 consecutive vocab values of a block into 8 bytes; 8-byte slots
// XOR-swizzled by token), then writes whole 16-byte runs of token rows; columns t >= nt and
// rows v >= nv are not written. LO stores the residual v - bf16(v) instead
// of v (the low half of a bf16 pair). Optionally one element per token
// column j of the lane is replaced after staging: patch->pos[j] >= 0 is its
// byte offset in the wave's staging area (target_slot) and patch->val[j] its
// value. The caller separates a second use of the staging area with a
// barrier.
struct TargetPatch {
  int pos[8];
  float val[8];
};

// Byte offset, in a wave's staging area, of row d (0..127, the wave's own
// rows) of token column tl: the 8-byte slot d / 4 of the token row, swizzled.
__device__ __forceinline__ int target_slot(int d, int tl) {
  return tl * 256 + (((d >> 2) ^ token_swizzle(tl)) * 8) + 2 * (d & 3);
}

// The value of accumulator element (i, j, r) is get(i, j, r): the element
// itself, or a function of it formed as it is staged.
template <bool LO, bool PATCH = false, bool BLOCKED = false, class Get>
__device__ __forceinline__ void store_token_major(const Get& get, char* smem, int wm, int wn,
                                                  int lane, uint16_t* dst, int64_t ld,
                                                  int64_t m0, int64_t n0, int64_t nt,
                                                  int64_t nv, const TargetPatch* patch = nullptr,
                                                  int64_t blk = 0) {
  const int g = lane >> 4;
  char* reg = smem + (wm + 2 * wn) * kWaveScratch;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int tl = j * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = get(i, j, e);
        if (LO) v[e] -= bf16_to_f32(f32_to_bf16(v[e]));
      }
      const uint32_t lo = pack_bf16x2(v[0], v[1]);
      const uint32_t hi = pack_bf16x2(v[2], v[3]);
      const int slot = (i * 4 + g) ^ token_swizzle(tl);
      *reinterpret_cast<uint2*>(reg + tl * 256 + slot * 8) = make_uint2(lo, hi);
    }
  }
  if (PATCH) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (patch->pos[j] >= 0) {
        float v = patch->val[j];
        if (LO) v -= bf16_to_f32(f32_to_bf16(v));
        *reinterpret_cast<uint16_t*>(reg + patch->pos[j]) = f32_to_bf16(v);
      }
  }
  __syncthreads();
  if constexpr (BLOCKED) {
    // Blocked destination (dst[blocked_offset(t, v, blk)]): store q covers
    // vocabulary block q / 8 of the wave (32 columns) for 16 tokens, one
    // contiguous KiB.
#pragma unroll 4
    for (int q = 0; q < 32; ++q) {
      const int tl = (q & 7) * 16 + (lane >> 2), ch = (q >> 3) * 4 + (lane & 3);
      const u32x4 v =
          *reinterpret_cast<const u32x4*>(reg + tl * 256 + ((2 * ch) ^ token_swizzle(tl)) * 8);
      const int64_t t = n0 + wn * 128 + tl;
      const int64_t vl = m0 + wm * 128 + 8 * ch;
      if (t < nt && vl < nv)
        *reinterpret_cast<u32x4*>(dst + gemm::blocked_offset(t, vl, blk)) = v;
    }
  } else {
#pragma unroll 4
    for (int q = 0; q < 32; ++q) {
      const int idx = q * 64 + lane;
      const int tl = idx >> 4, ch = idx & 15;
      const u32x4 v =
          *reinterpret_cast<const u32x4*>(reg + tl * 256 + ((2 * ch) ^ token_swizzle(tl)) * 8);
      const int64_t t = n0 + wn * 128 + tl;
      const int64_t vl = m0 + wm * 128 + 8 * ch;
      if (t < nt && vl < nv) *reinterpret_cast<u32x4*>(dst + t * ld + vl) = v;
    }
  }
}

// ---- forward epilogue: per (vocab tile, token) max and sum-exp ------------
// Tile rows are vocabulary ids, columns are tokens.
// SOFTCAP selects the s * tanh(z / s) variant at compile time; OUT, whether
// the logits z' themselves are also stored (the float32 values the max and
// sum are formed from). PC: the tiles of the first pc_rows vocabulary rows
// also keep their probabilities relative to the tile max M of each token,
// P' = exp(z' - M) <= 1, as bf16 in the blocked layout of the backward's G
// chunk (pblk elements per 32 rows): the rows of backward chunk j (pc_vchunk
// rows each) at probs<j>, so that the backward can form those chunks' G from
// them instead of recomputing their logits. The partials are formed exactly
// as without PC; P' is formed again from the logits in the accumulators once
// the tile max is known.
template <bool SOFTCAP, int OUT = kNoLogits, bool PC = false>
struct EpiLse {
  static_assert(!(PC && OUT != kNoLogits), "kept probabilities or stored logits, not both");
  const int64_t* labels;
  int64_t N, V, ignore_index;
  float softcap, inv_softcap;
  float2* part;  // [n_voc_tiles][ld_part]: (max m, sum of exp(x - m)) of the tile
  int64_t ld_part;
  float* zt;     // target logit (softcapped), one writer per non-ignored token
  void* logits;  // OUT != kNoLogits: [N][ld_logits]
  int64_t ld_logits;
  int vec;       // 16-byte runs of the logits rows are aligned
  // PC: where each kept chunk's G goes (chunks 0 .. 3; separate fields, not an
  // array, so that the epilogue's copy stays in registers)
  uint16_t* probs0 = nullptr;
  uint16_t* probs1 = nullptr;
  uint16_t* probs2 = nullptr;
  uint16_t* probs3 = nullptr;
  int64_t pc_rows = 0, pblk = 0, pc_vchunk = 1;
  static_assert(gemm::kMaxKept == 4, "one field per kept chunk");
  // the tiles of the kept rows store more: deal the vocabulary tiles to the XCDs
  static constexpr bool kSpreadM = PC;

  static constexpr int kTokBytes = 2048;          // the tile's labels
  __device__ __forceinline__ void stage(char* tok, int64_t n0, int wave, int lane) const {
    stage_tokens<2>(tok, labels, n0, N, wave, lane);
  }

  __device__ __forceinline__ void operator()(Acc& acc, int64_t m0, int64_t n0, int wm, int wn,
                                             int lane, char* smem, const char* tok) const {
    const int64_t* lab = reinterpret_cast<const int64_t*>(tok);
    const int g = lane >> 4;
    const int64_t vbase = m0 + wm * 128;
    const bool pc = PC && m0 < pc_rows;          // the whole workgroup agrees
    float mx[8], sm[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t t = n0 + acc_col(wn, j, lane);
      // the lane's 32 logits of the column, softcapped and masked past V, in
      // registers of their own (the accumulators are not written back unless
      // the logits are stored)
      float z[8][4];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = acc[i][j][r];
          if (SOFTCAP) x = softcap * tanh_fast(x * inv_softcap);
          const int64_t v = m0 + acc_row(wm, i, r, lane);
          z[i][r] = v < V ? x : -INFINITY;
          if (OUT != kNoLogits) acc[i][j][r] = z[i][r];
        }
      // target logit: the one lane holding (y_t, t) writes it
      const int64_t y = t < N ? lab[acc_col(wn, j, lane)] : ignore_index;
      if (y != ignore_index && y >= vbase && y < vbase + 128 && y < V) {
        const int d = int(y - vbase);
        const int ti = d >> 4, tr = d & 3;
        if (((d >> 2) & 3) == g) {
          float val = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) val = (i == ti && r == tr) ? z[i][r] : val;
          zt[t] = val;
        }
      }
      // max and sum in four independent chains (r), then combined over the
      // lane's values and the four lanes of the column
      float mq[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) mq[r] = fmaxf(mq[r], z[i][r]);
      const float m = col_max4(fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3])));
      // sum of exp(z - m) = sum of 2^(z log2 e - m log2 e), one fma per element
      float s = 0.f;
      if (m != -INFINITY) {
        const float mb = m * kLog2e;
        float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sq[r] += __builtin_amdgcn_exp2f(fmaf(z[i][r], kLog2e, -mb));
        s = (sq[0] + sq[1]) + (sq[2] + sq[3]);
      }
      mx[j] = m;
      sm[j] = col_sum4(s);
    }
    if (OUT != kNoLogits)
      store_logits<OUT>(acc, smem, wm, wn, lane, logits, ld_logits, vec, m0, n0, N, V);
    // combine the two waves (wm = 0, 1) that share the token columns
    float2* buf = reinterpret_cast<float2*>(smem);
    float* wmax = reinterpret_cast<float*>(smem + 2048);    // PC: [2][256] wave maxima
    if (PC && pc && g == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) wmax[wm * 256 + wn * 128 + j * 16 + lane] = mx[j];
    }
    if (wm == 1 && g == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) buf[wn * 128 + j * 16 + lane] = make_float2(mx[j], sm[j]);
    }
    __syncthreads();
    if (wm == 0 && g == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float2 o = buf[wn * 128 + j * 16 + lane];
        const float Mx = fmaxf(mx[j], o.x);
        float S = 0.f;
        if (mx[j] != -INFINITY) S += sm[j] * __builtin_amdgcn_exp2f((mx[j] - Mx) * kLog2e);
        if (o.x != -INFINITY) S += o.y * __builtin_amdgcn_exp2f((o.x - Mx) * kLog2e);
        const int64_t t = n0 + acc_col(wn, j, lane);
        if (t < ld_part) part[(m0 / kBM) * ld_part + t] = make_float2(Mx, S);
      }
    }
    if (PC && pc) {
      // P' = exp(z' - M), M the tile max of the column (both waves' maxima),
      // formed again from the logits in the accumulators as it is staged
      float mb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float o = wmax[(1 - wm) * 256 + wn * 128 + j * 16 + (lane & 15)];
        mb[j] = fmaxf(mx[j], o) * kLog2e;
      }
      __syncthreads();                             // the maxima are read; staging reuses LDS
      auto prob = [&](int i, int j, int r) {
        float x = acc[i][j][r];
        if (SOFTCAP) x = softcap * tanh_fast(x * inv_softcap);
        return mb[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(fmaf(x, kLog2e, -mb[j]));
      };
      // the kept chunk of this tile (the chunk edges are tile edges)
      const int64_t j = m0 / pc_vchunk, jr0 = j * pc_vchunk;
      uint16_t* dst = j == 0 ? probs0 : j == 1 ? probs1 : j == 2 ? probs2 : probs3;
      const int64_t jrows = V - jr0 < pc_vchunk ? V - jr0 : pc_vchunk;
      store_token_major<false, false, true>(prob, smem, wm, wn, lane, dst, 0, m0 - jr0, n0, N,
                                            jrows, nullptr, pblk);
    }
  }
};

// ---- backward epilogue: the logit gradient G for one vocabulary chunk ----
// G[t, v] = c * valid_t * (exp(z'_tv - lse_t) - [v = y_t]) * dz'/dz, stored
// bf16 in 32-column blocks, G[t][v - v0] at blocked_offset(t, v - v0, gblk)
// (see gemm::Geom: whole cache lines for the dW and dH loads that read it
// back). Tile rows are chunk-relative vocab ids, columns tokens. G is formed
// in float32 in place of the logits, then stored through store_token_major. SPLIT (float32
// gradients) stores two bf16 chunks, G_hi = bf16(G) at g and
// G_lo = bf16(G - G_hi) at g + lo_off.
template <bool SOFTCAP, bool SPLIT>
struct EpiGrad {
  const int64_t* labels;
  const float* lse;
  const float* zt;   // the forward's float32 target logits
  const Scalars* sc;
  int64_t N, V, ignore_index, v0, vcur, gblk;   // gblk: elements per block of G
  float softcap, inv_softcap;
  uint16_t* g;
  int64_t lo_off;   // elements from the hi to the lo chunk (SPLIT)

  // the tile's labels, lse and target logits
  static constexpr int kTokBytes = 4096;
  __device__ __forceinline__ void stage(char* tok, int64_t n0, int wave, int lane) const {
    stage_tokens<2>(tok, labels, n0, N, wave, lane);
    stage_tokens<1>(tok + 2048, lse, n0, N, wave, lane);
    stage_tokens<1>(tok + 3072, zt, n0, N, wave, lane);
  }

  // Every element is first formed as if it were not the target:
  // c exp(z' - lse) dz'/dz = exp2(z' log2 e + log2 c - lse log2 e) dz'/dz, the
  // scale folded into the exponent (c = 0 for ignored tokens gives exact
  // zeros, a NaN scale for a bad label NaN). The one target element of a
  // token in this block is then replaced in the staged tile by
  // c (exp(z'_y - lse) - 1) dz'/dz from the forward's target logit, which is
  // the same float32 value the GEMM recomputes.
  __device__ __forceinline__ void operator()(Acc& acc, int64_t m0, int64_t n0, int wm, int wn,
                                             int lane, char* smem, const char* tok) const {
    const int64_t* lab = reinterpret_cast<const int64_t*>(tok);
    const float* lse_t = reinterpret_cast<const float*>(tok + 2048);
    const float* zt_t = reinterpret_cast<const float*>(tok + 3072);
    const float c = sc->c32;
    const int lg = lane >> 4;                           // the lane's row group
    const int64_t vbase = v0 + m0 + wm * 128;           // global vocab id of block row 0
    TargetPatch tp;
    float bias[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tl = j * 16 + (lane & 15);             // token within the wave block
      const int64_t t = n0 + wn * 128 + tl;
      // Every token's lse is known (ignored ones too) and columns past N hold
      // the logits of token N-1 (staged lse clamped the same way), so
      // exp(z' - lse) <= 1 everywhere.
      const float l = lse_t[wn * 128 + tl];
      float coef = 0.f;
      tp.pos[j] = -1;
      tp.val[j] = 0.f;
      if (t < N) {
        const int64_t y = lab[wn * 128 + tl];
        if (y != ignore_index) {
          coef = (y < 0 || y >= V) ? NAN : c;
          if (y >= vbase && y < vbase + 128) {
            const int d = int(y - vbase);
            if (((d >> 2) & 3) == lg) {
              const float z = zt_t[wn * 128 + tl];
              float dd = 1.f;
              if (SOFTCAP) {
                const float th = z * inv_softcap;
                dd = 1.f - th * th;
              }
              tp.pos[j] = target_slot(d, tl);
              tp.val[j] = (__builtin_amdgcn_exp2f((z - l) * kLog2e) - 1.f) * coef * dd;
            }
          }
        }
      }
      bias[j] = log2f(coef) - l * kLog2e;
    }
    // G of element (i, j, r), from the logit in the accumulator
    auto grad = [&](int i, int j, int r) {
      const float z = acc[i][j][r];
      if (SOFTCAP) {
        const float th = tanh_fast(z * inv_softcap);
        return __builtin_amdgcn_exp2f(fmaf(softcap * th, kLog2e, bias[j])) * (1.f - th * th);
      }
      return __builtin_amdgcn_exp2f(fmaf(z, kLog2e, bias[j]));
    };
    if (!SPLIT) {
      // formed as it is staged, never written back to the accumulators
      store_token_major<false, true, true>(grad, smem, wm, wn, lane, g, 0, m0, n0, N, vcur, &tp,
                                           gblk);
      return;
    }
    // two stores of the same values (hi, then lo): form them once, in place
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = grad(i, j, r);
    auto held = [&](int i, int j, int r) { return acc[i][j][r]; };
    store_token_major<false, true, true>(held, smem, wm, wn, lane, g, 0, m0, n0, N, vcur, &tp,
                                         gblk);
    __syncthreads();                                   // the staging area is reused
    store_token_major<true, true, true>(held, smem, wm, wn, lane, g + lo_off, 0, m0, n0, N, vcur,
                                        &tp, gblk);
  }
};

// ---- forward epilogue of the no-recompute variant ------------------------
// As EpiLse, and it also keeps the probabilities: with the tile max Mx of
// each token shared by the two waves of its column, it stores
// P'[t][v] = exp(z'_tv - Mx) (<= 1) as bf16 at blocked_offset(t, v, pblk),
// and the partial (Mx, sum of P') of the tile. G follows later without
// recomputing the logits: G = c (P' exp(Mx - lse) - [v = y]) dz'/dz.
template <bool SOFTCAP>
struct EpiLseP {
  const int64_t* labels;
  int64_t N, V, ignore_index;
  float softcap, inv_softcap;
  float2* part;  // [n_voc_tiles][ld_part]: (max, sum of exp(x - max)) of the tile
  int64_t ld_part;
  float* zt;     // target logit (softcapped), one writer per non-ignored token
  uint16_t* probs;  // blocked, pblk elements per 32 vocabulary columns
  int64_t pblk;

  static constexpr int kTokBytes = 2048;          // the tile's labels
  __device__ __forceinline__ void stage(char* tok, int64_t n0, int wave, int lane) const {
    stage_tokens<2>(tok, labels, n0, N, wave, lane);
  }

  __device__ __forceinline__ void operator()(Acc& acc, int64_t m0, int64_t n0, int wm, int wn,
                                             int lane, char* smem, const char* tok) const {
    const int64_t* lab = reinterpret_cast<const int64_t*>(tok);
    const int g = lane >> 4;
    const int64_t vbase = m0 + wm * 128;
    float mx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t t = n0 + acc_col(wn, j, lane);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float z = acc[i][j][r];
          if (SOFTCAP) z = softcap * tanh_fast(z * inv_softcap);
          const int64_t v = m0 + acc_row(wm, i, r, lane);
          acc[i][j][r] = v < V ? z : -INFINITY;
        }
      const int64_t y = t < N ? lab[acc_col(wn, j, lane)] : ignore_index;
      if (y != ignore_index && y >= vbase && y < vbase + 128 && y < V) {
        const int d = int(y - vbase);
        const int ti = d >> 4, tr = d & 3;
        if (((d >> 2) & 3) == g) {
          float val = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) val = (i == ti && r == tr) ? acc[i][j][r] : val;
          zt[t] = val;
        }
      }
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, acc[i][j][r]);
      mx[j] = col_max4(m);
    }
    // the tile max of each token column, from both waves that hold it
    float* xb = reinterpret_cast<float*>(smem);      // [2][256] maxima, then [256] sums
    if (g == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) xb[wm * 256 + wn * 128 + j * 16 + lane] = mx[j];
    }
    __syncthreads();
    float sm[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float Mx = fmaxf(mx[j], xb[(1 - wm) * 256 + wn * 128 + j * 16 + (lane & 15)]);
      mx[j] = Mx;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p =
              Mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((acc[i][j][r] - Mx) * kLog2e);
          acc[i][j][r] = p;
          s += p;
        }
      sm[j] = col_sum4(s);
    }
    __syncthreads();                                  // maxima read before the sums reuse xb
    if (wm == 1 && g == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) xb[wn * 128 + j * 16 + lane] = sm[j];
    }
    __syncthreads();
    if (wm == 0 && g == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t t = n0 + acc_col(wn, j, lane);
        if (t < ld_part)
          part[(m0 / kBM) * ld_part + t] = make_float2(mx[j], sm[j] + xb[wn * 128 + j * 16 + lane]);
      }
    }
    __syncthreads();                                  // sums read before the staging reuses LDS
    auto held = [&](int i, int j, int r) { return acc[i][j][r]; };
    store_token_major<false, false, true>(held, smem, wm, wn, lane, probs, 0, m0, n0, N, V,
                                          nullptr, pblk);
  }
};

// G in place of the stored probabilities of nt tokens (the first *count
// ones when `count` is given) and the vocabulary columns [0, nv) of a chunk
// whose column v is vocabulary id vbase + v:
//   G[t][v] = c valid_t (P'[t][v] exp(M_tv - lse_t) - [vbase + v = y_t]) dz'/dz
// with M_tv the max of v's vocabulary tile for token t (the forward partial).
// The target element is formed from the float32 target logit instead:
// c (exp(z'_ty - lse_t) - 1) dz'/dz. With a softcap, dz'/dz = 1 - (z'/s)^2 and
// z' = M + ln P' elsewhere. The buffer is blocked (gemm::blocked_offset, blk
// elements per 32 columns); in block b (blockIdx.y, then strided), thread i
// converts the 8 consecutive elements of run i of the block's used part
// [nt tokens][4 runs], so a wave reads and writes one contiguous KiB.
template <bool SOFTCAP>
__global__ __launch_bounds__(256) void k_probs_to_grad(
    uint16_t* __restrict__ gp, int64_t blk, int64_t nt, const int64_t* __restrict__ count,
    int64_t vbase, int64_t nv, int64_t V, const float2* __restrict__ part, int64_t ld_part,
    const float* __restrict__ lse, const float* __restrict__ zt,
    const int64_t* __restrict__ labels, int64_t ignore_index, const Scalars* __restrict__ sc,
    float inv_softcap) {
  if (count) {
    const int64_t c = *count;
    nt = c < nt ? c : nt;
  }
  const int64_t rem = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (rem >= nt * 4) return;
  const int64_t t = rem >> 2;
  const int64_t y = labels[t];
  const float coef = y == ignore_index ? 0.f : ((y < 0 || y >= V) ? NAN : sc->c32);
  const float l = lse[t];
  const int64_t nb = (nv + 31) / 32;
  for (int64_t b = blockIdx.y; b < nb; b += gridDim.y) {
    const int64_t v0 = b * 32 + (rem & 3) * 8;
    uint16_t* run = gp + b * blk + t * 32 + (rem & 3) * 8;
    const float M = part[((vbase + v0) / kBM) * ld_part + t].x;
    const float scale = __builtin_amdgcn_exp2f((M - l) * kLog2e);
    const u32x4 in = *reinterpret_cast<const u32x4*>(run);
    float g[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w = in[e >> 1];
      const float pv = bf16_to_f32(uint16_t((e & 1) ? (w >> 16) : (w & 0xFFFF)));
      const int64_t v = v0 + e;
      float x;
      if (vbase + v == y) {
        const float z = zt[t];
        x = (__builtin_amdgcn_exp2f((z - l) * kLog2e) - 1.f) * coef;
        if (SOFTCAP) {
          const float th = z * inv_softcap;
          x *= 1.f - th * th;
        }
      } else {
        x = pv * scale * coef;
        if (SOFTCAP && pv > 0.f) {
          const float th = (M + __logf(pv)) * inv_softcap;
          x *= 1.f - th * th;
        }
      }
      g[e] = v < nv ? x : 0.f;
    }
    *reinterpret_cast<u32x4*>(run) = u32x4{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]),
                                           pack_bf16x2(g[4], g[5]), pack_bf16x2(g[6], g[7])};
  }
}

// ---- row-major epilogues staged through LDS ---------------------------------
// A wave's 128 x 128 float32 block goes out in 4 passes of 32 rows (row blocks
// 2P and 2P + 1 of 16): the lane values are written to the wave's LDS scratch
// as [32][128] float32 (the four 64-byte column quarters of a 256-byte bank
// window permuted by row / 4, which puts the four 16-lane groups of a write on
// different banks), then read back as float4 runs of 4 consecutive columns of
// one row, which the caller's functor stores. Before the staging of each pass
// the functor may issue its own global loads for that pass (prefetch), so
// their latency overlaps the LDS traffic.
__device__ __forceinline__ int staged_col(int row, int col) {
  return col ^ (((row >> 2) & 3) << 4);
}

template <class Pass>
__device__ __forceinline__ void staged_rows(Acc& acc, int wm, int wn, int lane, char* smem,
                                            Pass& pass) {
  float* reg = reinterpret_cast<float*>(smem + (wm + 2 * wn) * kWaveScratch);
  pass.prefetch(0, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i + 1 < 4) pass.prefetch(i + 1, lane);     // in flight while block i is staged
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * h + 4 * (lane >> 4) + r;
          reg[row * 128 + staged_col(row, j * 16 + (lane & 15))] = acc[2 * i + h][j][r];
        }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int idx = q * 64 + lane, row = idx >> 5, c4 = idx & 31;
      const float4 v = *reinterpret_cast<const float4*>(reg + row * 128 + staged_col(row, 4 * c4));
      pass.store(i, q, row, 4 * c4, v);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ---- dW epilogue: rows v0 + m of dW, bf16, optionally added to ------------
template <bool ACCUM>
struct EpiDW {
  uint16_t* dW;
  int64_t H, v0, vcur;

  struct Pass {
    const EpiDW& e;
    int64_t r0, c0;   // global (chunk-relative row, column) of the wave block
    __device__ __forceinline__ void prefetch(int, int) {}
    __device__ __forceinline__ void store(int i, int, int row, int col, float4 v) {
      const int64_t m = r0 + i * 32 + row, n = c0 + col;
      if (m >= e.vcur || n >= e.H) return;
      uint16_t* p = e.dW + (e.v0 + m) * e.H + n;
      if (ACCUM) {
        const uint2 o = *reinterpret_cast<const uint2*>(p);
        v.x += bf16_to_f32(uint16_t(o.x)); v.y += bf16_to_f32(uint16_t(o.x >> 16));
        v.z += bf16_to_f32(uint16_t(o.y)); v.w += bf16_to_f32(uint16_t(o.y >> 16));
      }
      *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
    }
  };

  static constexpr int kTokBytes = 0;             // no per-token inputs
  __device__ __forceinline__ void stage(char*, int64_t, int, int) const {}

  __device__ __forceinline__ void operator()(Acc& acc, int64_t m0, int64_t n0, int wm, int wn,
                                             int lane, char* smem, const char*) const {
    Pass pass{*this, m0 + wm * 128, n0 + wn * 128};
    staged_rows(acc, wm, wn, lane, smem, pass);
  }
};

// ---- float32 dW epilogue (float32 gradients for bf16 inputs) -------------
template <bool ACCUM>
struct EpiDW32 {
  float* dW;
  int64_t H, v0, vcur;

  struct Pass {
    const EpiDW32& e;
    int64_t r0, c0;   // global (chunk-relative row, column) of the wave block
    __device__ __forceinline__ void prefetch(int, int) {}
    __device__ __forceinline__ void store(int i, int, int row, int col, float4 v) {
      const int64_t m = r0 + i * 32 + row, n = c0 + col;
      if (m >= e.vcur || n >= e.H) return;
      float4* p = reinterpret_cast<float4*>(e.dW + (e.v0 + m) * e.H + n);
      if (ACCUM) {
        const float4 o = *p;
        v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
      }
      *p = v;
    }
  };

  static constexpr int kTokBytes = 0;             // no per-token inputs
  __device__ __forceinline__ void stage(char*, int64_t, int, int) const {}

  __device__ __forceinline__ void operator()(Acc& acc, int64_t m0, int64_t n0, int wm, int wn,
                                             int lane, char* smem, const char*) const {
    Pass pass{*this, m0 + wm * 128, n0 + wn * 128};
    staged_rows(acc, wm, wn, lane, smem, pass);
  }
};

// ---- dW of the no-recompute variant, summed over token chunks in float32 --
// SRC: 0 nothing to add, 1 the bf16 dW already in memory (accumulate_dW),
// 2 the float32 running sum of the earlier chunks. DST: 1 bf16 dW, rounded to
// nearest even once, at the last chunk; 2 the float32 running sum. The
// running sums of the next row block are loaded while the current one is
// staged, as in the dH epilogue.
template <int SRC, int DST>
struct EpiDWAcc {
  uint16_t* dW;
  float* acc32;  // [V][H] float32 running sum
  int64_t H, vcur;

  struct Pass {
    const EpiDWAcc& e;
    int64_t r0, c0;
    float4 prev[2][16];
    __device__ __forceinline__ void prefetch(int i, int lane) {
      if (SRC != 2) return;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int idx = q * 64 + lane, row = idx >> 5, c4 = idx & 31;
        const int64_t m = r0 + i * 32 + row, n = c0 + 4 * c4;
        prev[i & 1][q] = (m < e.vcur && n < e.H)
                             ? *reinterpret_cast<const float4*>(e.acc32 + m * e.H + n)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    __device__ __forceinline__ void store(int i, int q, int row, int col, float4 v) {
      const int64_t m = r0 + i * 32 + row, n = c0 + col;
      if (m >= e.vcur || n >= e.H) return;
      if (SRC == 1) {
        const uint2 o = *reinterpret_cast<const uint2*>(e.dW + m * e.H + n);
        v.x += bf16_to_f32(uint16_t(o.x)); v.y += bf16_to_f32(uint16_t(o.x >> 16));
        v.z += bf16_to_f32(uint16_t(o.y)); v.w += bf16_to_f32(uint16_t(o.y >> 16));
      } else if (SRC == 2) {
        const float4 o = prev[i & 1][q];
        v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
      }
      if (DST == 1)
        *reinterpret_cast<uint2*>(e.dW + m * e.H + n) =
            make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
      else
        *reinterpret_cast<float4*>(e.acc32 + m * e.H + n) = v;
    }
  };

  static constexpr int kTokBytes = 0;             // no per-token inputs
  __device__ __forceinline__ void stage(char*, int64_t, int, int) const {}

  __device__ __forceinline__ void operator()(Acc& acc, int64_t m0, int64_t n0, int wm, int wn,
                                             int lane, char* smem, const char*) const {
    Pass pass{*this, m0 + wm * 128, n0 + wn * 128, {}};
    staged_rows(acc, wm, wn, lane, smem, pass);
  }
};

// ---- dH epilogue: accumulate over vocabulary chunks in a fixed order ------
// FIRST: no running sum to add; LAST: store bf16 dH instead of the float32
// running sum. MAPACC: the running sum is the float32 dH output itself, so
// its rows, too, are the tokens' original positions (row_map).
template <bool FIRST, bool LAST, bool MAPACC = false>
struct EpiDH {
  uint16_t* dH;
  float* acc32;  // [N][H] float32 running sum (unused with a single chunk)
  int64_t N, H;
  // compact plan: the bf16 row m of dH goes to row row_map[m] (null: m)
  const int32_t* row_map = nullptr;

  struct Pass {
    const EpiDH& e;
    int64_t r0, c0;
    float4 prev[2][16];  // the running sums of row blocks i and i + 1
    __device__ __forceinline__ void prefetch(int i, int lane) {
      if (FIRST) return;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int idx = q * 64 + lane, row = idx >> 5, c4 = idx & 31;
        const int64_t m = r0 + i * 32 + row, n = c0 + 4 * c4;
        const int64_t ma = MAPACC ? int64_t(e.row_map[m < e.N ? m : 0]) : m;
        prev[i & 1][q] = (m < e.N && n < e.H)
                             ? *reinterpret_cast<const float4*>(e.acc32 + ma * e.H + n)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    __device__ __forceinline__ void store(int i, int q, int row, int col, float4 v) {
      const int64_t m = r0 + i * 32 + row, n = c0 + col;
      if (m >= e.N || n >= e.H) return;
      if (!FIRST) {
        const float4 o = prev[i & 1][q];
        v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
      }
      if (LAST) {
        const int64_t mo = e.row_map ? int64_t(e.row_map[m]) : m;
        *reinterpret_cast<uint2*>(e.dH + mo * e.H + n) =
            make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
      } else {
        const int64_t ma = MAPACC ? int64_t(e.row_map[m]) : m;
        *reinterpret_cast<float4*>(e.acc32 + ma * e.H + n) = v;
      }
    }
  };

  static constexpr int kTokBytes = 0;             // no per-token inputs
  __device__ __forceinline__ void stage(char*, int64_t, int, int) const {}

  __device__ __forceinline__ void operator()(Acc& acc, int64_t m0, int64_t n0, int wm, int wn,
                                             int lane, char* smem, const char*) const {
    Pass pass{*this, m0 + wm * 128, n0 + wn * 128, {}};
    staged_rows(acc, wm, wn, lane, smem, pass);
  }
};

// ---- split-K dH: one K segment's float32 partial product -----------------
// The workgroups of K segment s (the s-th run of dH tiles of a split
// k_gemm_pair) store their tiles of G . W over that segment's K range into
// part + s * seg_stride, [rows][H] float32; k_dh_reduce adds the segments up.
struct EpiDHPart {
  float* part;
  int64_t N, H;          // rows written (a compact plan cuts N on the device), columns
  int64_t seg_stride;    // elements per segment's partial product (launch rows * H)

  static constexpr int kTokBytes = 0;             // no per-token inputs
  __device__ __forceinline__ void stage(char*, int64_t, int, int) const {}
  // the workgroup's K segment (called by the split GEMM tile before the K loop)
  __device__ __forceinline__ void select_segment(int seg) { part += int64_t(seg) * seg_stride; }

  __device__ __forceinline__ void operator()(Acc& acc, int64_t m0, int64_t n0, int wm, int wn,
                                             int lane, char* smem, const char* tok) const {
    EpiDH<true, false>{nullptr, part, N, H, nullptr}(acc, m0, n0, wm, wn, lane, smem, tok);
  }
};

// The split-K partial products of dH added up in a fixed order (segment 0
// first), after the float32 running sum of the earlier vocabulary chunks
// when there is one (PRIOR), stored as the new running sum or, for the last
// chunk, as bf16 dH rounded to nearest even (BF16OUT). Four consecutive
// elements per thread; n4 = elements / 4, stride = elements per segment.
template <bool PRIOR, bool BF16OUT>
__global__ __launch_bounds__(256) void k_dh_reduce(const float* __restrict__ part, int segs,
                                                   int64_t n4, int64_t stride,
                                                   const float* prior, float* out32,
                                                   uint16_t* out16, int64_t H,
                                                   const int64_t* __restrict__ rows_dyn,
                                                   const int32_t* __restrict__ row_map) {
  // a compact plan: only the first *rows_dyn rows, the bf16 row m at row_map[m]
  if (rows_dyn) {
    const int64_t n4d = *rows_dyn * (H / 4);
    n4 = n4d < n4 ? n4d : n4;
  }
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n4;
       i += int64_t(gridDim.x) * 256) {
    float4 v = PRIOR ? reinterpret_cast<const float4*>(prior)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int z = 0; z < segs; ++z) {
      const float4 q = reinterpret_cast<const float4*>(part + z * stride)[i];
      v.x += q.x; v.y += q.y; v.z += q.z; v.w += q.w;
    }
    if (BF16OUT) {
      int64_t o = i;
      if (row_map) {
        const int64_t m = i / (H / 4);
        o = int64_t(row_map[m]) * (H / 4) + (i - m * (H / 4));
      }
      reinterpret_cast<uint2*>(out16)[o] = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
    } else {
      reinterpret_cast<float4*>(out32)[i] = v;
    }
  }
}

hipError_t launch_dh_reduce(const float* part, int64_t segs, int64_t n, const float* prior,
                            float* out32, uint16_t* out16, const Launcher& L, int64_t H,
                            const int64_t* rows_dyn = nullptr, const int32_t* row_map = nullptr) {
  const int64_t n4 = n / 4;
  const int64_t want = (n4 + 255) / 256;
  const dim3 grid(unsigned(want < 4096 ? want : 4096));
  L.pre(kDhReduce);
  if (prior && out16)
    hipLaunchKernelGGL((k_dh_reduce<true, true>), grid, dim3(256), 0, L.stream, part, int(segs),
                       n4, n, prior, out32, out16, H, rows_dyn, row_map);
  else if (prior)
    hipLaunchKernelGGL((k_dh_reduce<true, false>), grid, dim3(256), 0, L.stream, part, int(segs),
                       n4, n, prior, out32, out16, H, rows_dyn, row_map);
  else if (out16)
    hipLaunchKernelGGL((k_dh_reduce<false, true>), grid, dim3(256), 0, L.stream, part, int(segs),
                       n4, n, prior, out32, out16, H, rows_dyn, row_map);
  else
    hipLaunchKernelGGL((k_dh_reduce<false, false>), grid, dim3(256), 0, L.stream, part,
                       int(segs), n4, n, prior, out32, out16, H, rows_dyn, row_map);
  L.post(kDhReduce);
  return hipGetLastError();
}

const uint16_t* buf_ptr(const Args& a, int buf) {
  return buf == gemm::kBufW  ? static_cast<const uint16_t*>(a.W)
       : buf == gemm::kBufH  ? static_cast<const uint16_t*>(a.h)
       : buf == gemm::kBufHc ? static_cast<const uint16_t*>(a.hc)
                             : static_cast<const uint16_t*>(a.g);
}

// A T-form operand is read in 16-byte column chunks: it needs rows % 8 == 0.
// The per-lane load offsets are 32-bit byte offsets from the tile base: at
// most min(255, rows - 1) rows of ld elements plus 64 k for a K-contiguous
// operand, 63 k-rows of ld elements plus the row length for a T-form one.
// The tile count must fit the grid.
bool operand_offsets_fit(int form, const gemm::Geom& g) {
  const int64_t reach = form == gemm::kFormN ? (g.rows - 1 < 255 ? g.rows - 1 : 255) * g.ld + 64
                        : g.blk ? 7 * g.blk + 64 * 32
                                : 63 * g.ld + g.rows;
  return reach >= 0 && 2 * reach + 16 <= int64_t(0xFFFFFFFF);
}

bool launch_ok(const gemm::Launch& l) {
  if (l.fa == gemm::kFormT && (l.a.rows % 8 != 0 || l.a.rows < 8)) return false;
  if (l.fb == gemm::kFormT && (l.b.rows % 8 != 0 || l.b.rows < 8)) return false;
  if (!operand_offsets_fit(l.fa, l.a) || !operand_offsets_fit(l.fb, l.b)) return false;
  if (gemm::num_tiles(l.M, l.Nn) > kMaxTiles) return false;
  return l.M > 0 && l.Nn > 0 && l.K > 0;
}

template <int FA, int FB, int DYN = kDynNone, class Epi>
hipError_t run_gemm(const gemm::Launch& l, const Args& a, const Epi& e, int kind,
                    const Launcher& L, const int64_t* dyn = nullptr) {
  if (!launch_ok(l)) return hipErrorInvalidValue;
  if (l.a.blk != 0 || l.b.blk != 0) return hipErrorInvalidValue;
  if ((DYN != kDynNone) != (dyn != nullptr)) return hipErrorInvalidValue;
  Operand A{buf_ptr(a, l.buf_a) + l.off_a, l.a};
  Operand B{buf_ptr(a, l.buf_b) + l.off_b, l.b};
  L.pre(kind);
  hipLaunchKernelGGL((k_gemm<FA, FB, Epi, DYN>), dim3(unsigned(gemm::num_tiles(l.M, l.Nn))),
                     dim3(kThreads), 0, L.stream, A, B, l.M, l.Nn, l.K, gemm::kGroupM, e, dyn);
  L.post(kind);
  return hipGetLastError();
}

// Two GEMMs whose A operand is the blocked G in one grid (k_gemm_pair): the
// first launch's tiles (SPLIT1: times its segs1 K segments of kseg1), padded
// to a multiple of 8 workgroups, then the second's. SEGS = 2: both over G's
// hi part and then its lo part, lo_off elements further.
template <int FA1, int FB1, int DYN1, int FA2, int FB2, int DYN2, bool SPLIT1 = false,
          int SEGS = 1, class Epi1, class Epi2>
hipError_t run_gemm_pair(const gemm::Launch& l1, const Epi1& e1, const gemm::Launch& l2,
                         const Epi2& e2, const Args& a, int kind, const Launcher& L,
                         const int64_t* dyn, int64_t kseg1 = 0, int64_t segs1 = 1,
                         int64_t lo_off = 0) {
  static_assert(SEGS == 1 || SEGS == 2, "one or two K segments");
  if ((SEGS == 2) != (lo_off != 0)) return hipErrorInvalidValue;
  if (!launch_ok(l1) || !launch_ok(l2)) return hipErrorInvalidValue;
  if (l1.a.blk == 0 || l1.b.blk != 0 || l2.a.blk == 0 || l2.b.blk != 0)
    return hipErrorInvalidValue;
  if (((DYN1 != kDynNone) || (DYN2 != kDynNone)) != (dyn != nullptr)) return hipErrorInvalidValue;
  // SPLIT1: kseg1 a multiple of 64 (whole stage tiles), every segment non-empty
  if (SPLIT1 && (kseg1 <= 0 || kseg1 % 64 != 0 || segs1 < 1 || (segs1 - 1) * kseg1 >= l1.K))
    return hipErrorInvalidValue;
  const int64_t t1 = gemm::num_tiles(l1.M, l1.Nn);
  const int64_t n1 = t1 * (SPLIT1 ? segs1 : 1);
  const int64_t n1p = (n1 + 7) / 8 * 8;
  const int64_t total = n1p + gemm::num_tiles(l2.M, l2.Nn);
  if (total > kMaxTiles) return hipErrorInvalidValue;
  const Operand A1{buf_ptr(a, l1.buf_a) + l1.off_a, l1.a}, B1{buf_ptr(a, l1.buf_b) + l1.off_b, l1.b};
  const Operand A2{buf_ptr(a, l2.buf_a) + l2.off_a, l2.a}, B2{buf_ptr(a, l2.buf_b) + l2.off_b, l2.b};
  L.pre(kind);
  hipLaunchKernelGGL((k_gemm_pair<FA1, FB1, Epi1, DYN1, SPLIT1, FA2, FB2, Epi2, DYN2, SEGS>),
                     dim3(unsigned(total)), dim3(kThreads), 0, L.stream, n1p, t1, n1,
                     SPLIT1 ? kseg1 : lo_off, A1, B1, l1.M, l1.Nn, l1.K, e1, A2, B2, l2.M,
                     l2.Nn, l2.K, e2, lo_off, dyn);
  L.post(kind);
  return hipGetLastError();
}

}  // namespace

namespace {
template <int OUT>
hipError_t bf16_forward_out(const Plan& p, const Args& a, const Launcher& L) {
  const gemm::Launch l = gemm::forward_launch(p);
  const int esz = OUT == kLogitsF32 ? 4 : 2;
  const int vec = OUT != kNoLogits && reinterpret_cast<uintptr_t>(a.logits) % 16 == 0 &&
                  (a.ld_logits * esz) % 16 == 0;
  // a compact plan: the gathered tokens and their labels; only the kept ones
  // (a device count) when no per-token lse is asked for
  const int64_t* lab = p.compact ? a.yc : a.labels;
  const int64_t* nv = (p.compact && !a.lse_out) ? &a.sc->n_valid : nullptr;
  constexpr int NF = gemm::kFormN;
  if constexpr (OUT == kNoLogits) {
    if (p.compact && p.backward && p.g_parts == 1) {
      // the probabilities of the first backward chunks are kept (their G is
      // formed from them, without recomputing their logits): when dW is not
      // added to, all but the last of them in dW's free rows, the last (or,
      // otherwise, chunk 0 alone) in the G buffer
      const gemm::Kept kept = gemm::kept_chunks(p, !a.accumulate_dW);
      auto run = [&](auto e) {
        auto at = [&](int j) -> uint16_t* {
          if (kept.in_dw(j))
            return reinterpret_cast<uint16_t*>(static_cast<char*>(a.dW) + kept.off[j]);
          return j == kept.n - 1 ? static_cast<uint16_t*>(a.g) : nullptr;
        };
        e.probs0 = at(0);
        e.probs1 = at(1);
        e.probs2 = at(2);
        e.probs3 = at(3);
        e.pc_rows = kept.n * p.vchunk < p.V ? kept.n * p.vchunk : p.V;
        e.pc_vchunk = p.vchunk;
        e.pblk = gemm::g_block(p);
        return nv ? run_gemm<NF, NF, kDynN>(l, a, e, kLseFwd, L, nv)
                  : run_gemm<NF, NF>(l, a, e, kLseFwd, L);
      };
      if (a.softcap > 0.f)
        return run(EpiLse<true, kNoLogits, true>{lab, p.N, p.V, a.ignore_index, a.softcap,
                                                 1.f / a.softcap, a.part, p.ld_part, a.zt,
                                                 nullptr, 0, 0});
      return run(EpiLse<false, kNoLogits, true>{lab, p.N, p.V, a.ignore_index, 0.f, 0.f, a.part,
                                                p.ld_part, a.zt, nullptr, 0, 0});
    }
  }
  if (a.softcap > 0.f) {
    EpiLse<true, OUT> e{lab, p.N, p.V, a.ignore_index, a.softcap, 1.f / a.softcap, a.part,
                        p.ld_part, a.zt, a.logits, a.ld_logits, vec};
    return nv ? run_gemm<NF, NF, kDynN>(l, a, e, kLseFwd, L, nv)
              : run_gemm<NF, NF>(l, a, e, kLseFwd, L);
  }
  EpiLse<false, OUT> e{lab, p.N, p.V, a.ignore_index, 0.f, 0.f, a.part, p.ld_part, a.zt,
                       a.logits, a.ld_logits, vec};
  return nv ? run_gemm<NF, NF, kDynN>(l, a, e, kLseFwd, L, nv)
            : run_gemm<NF, NF>(l, a, e, kLseFwd, L);
}
}  // namespace

hipError_t bf16_forward(const Plan& p, const Args& a, const Launcher& L) {
  if (!a.logits) return bf16_forward_out<kNoLogits>(p, a, L);
  if (a.logits_dtype == FLCE_F32) return bf16_forward_out<kLogitsF32>(p, a, L);
  return bf16_forward_out<kLogitsBF16>(p, a, L);
}

// Float32 gradients for bf16 inputs: G as a bf16 hi + lo pair; dW and dH
// each take one GEMM whose K loop runs over the hi part and then the lo part
// into the same float32 accumulators, added into the float32 outputs chunk by
// chunk in a fixed order.
hipError_t bf16_backward_chunk_f32grad(const Plan& p, const Args& a, int64_t chunk,
                                       const Launcher& L) {
  // over the kept tokens, gathered in order (their count n_valid on the
  // device); dH is its own float32 running sum at the tokens' positions
  if (!p.compact) return hipErrorInvalidValue;
  const int64_t v0 = chunk * p.vchunk;
  const int64_t vcur = gemm::chunk_rows(p, chunk);
  uint16_t* g = static_cast<uint16_t*>(a.g);
  const int64_t lo_off = p.vchunk * p.ldg;
  const int64_t* nv = &a.sc->n_valid;
  constexpr int NF = gemm::kFormN, TF = gemm::kFormT;
  const gemm::Launch lg = gemm::backward_launch(p, chunk, 0);
  hipError_t err;
  if (a.softcap > 0.f) {
    const EpiGrad<true, true> eg{a.yc, a.lse, a.zt, a.sc, p.N, p.V, a.ignore_index, v0, vcur,
                                 gemm::g_block(p), a.softcap, 1.f / a.softcap, g, lo_off};
    err = run_gemm<NF, NF, kDynN>(lg, a, eg, kGradLogits, L, nv);
  } else {
    const EpiGrad<false, true> eg{a.yc, a.lse, a.zt, a.sc, p.N, p.V, a.ignore_index, v0, vcur,
                                  gemm::g_block(p), 0.f, 0.f, g, lo_off};
    err = run_gemm<NF, NF, kDynN>(lg, a, eg, kGradLogits, L, nv);
  }
  if (err != hipSuccess) return err;
  // dH (its float32 output is its own running sum, rows at the tokens'
  // positions) and dW, each over G's hi and lo parts, in one grid
  float* dW = static_cast<float*>(a.dW);
  float* dH = static_cast<float*>(a.dH);
  const gemm::Launch lw = gemm::backward_launch(p, chunk, 1, 0);
  const gemm::Launch lh = gemm::backward_launch(p, chunk, 2, 0);
  auto pair = [&](auto edh) {
    if (a.accumulate_dW)
      return run_gemm_pair<NF, TF, kDynM, TF, TF, kDynK, false, 2>(
          lh, edh, lw, EpiDW32<true>{dW, p.H, v0, vcur}, a, kGemmDWDH, L, nv, 0, 1, lo_off);
    return run_gemm_pair<NF, TF, kDynM, TF, TF, kDynK, false, 2>(
        lh, edh, lw, EpiDW32<false>{dW, p.H, v0, vcur}, a, kGemmDWDH, L, nv, 0, 1, lo_off);
  };
  if (chunk == 0) return pair(EpiDH<true, false, true>{nullptr, dH, p.N, p.H, a.idx});
  return pair(EpiDH<false, false, true>{nullptr, dH, p.N, p.H, a.idx});
}

hipError_t bf16_backward_chunk(const Plan& p, const Args& a, int64_t chunk, const Launcher& L) {
  if (p.g_parts == 2) return bf16_backward_chunk_f32grad(p, a, chunk, L);
  // bf16 gradients: the plan is compact, the backward runs over the
  // non-ignored tokens gathered in order (their labels, lse, target logits
  // and rows), with their count n_valid read on the device
  if (!p.compact) return hipErrorInvalidValue;
  const int64_t v0 = chunk * p.vchunk;
  const int64_t vcur = gemm::chunk_rows(p, chunk);
  const int64_t* nv = &a.sc->n_valid;
  constexpr int NF = gemm::kFormN, TF = gemm::kFormT;
  // 1) G[n_valid][vchunk]: for the chunks whose probabilities the forward
  // kept (in dW's free rows, the last of them in the G buffer), from them, in
  // place; the others by recomputing the chunk's logits into the G buffer.
  // The dH and dW launches below read G where it was formed.
  const gemm::Kept kept = gemm::kept_chunks(p, !a.accumulate_dW);
  Args ag = a;
  if (kept.in_dw(int(chunk))) ag.g = static_cast<char*>(a.dW) + kept.off[chunk];
  uint16_t* g = static_cast<uint16_t*>(ag.g);
  const gemm::Launch lg = gemm::backward_launch(p, chunk, 0);
  hipError_t err;
  if (chunk < kept.n) {
    const int64_t nb = (vcur + 31) / 32;
    const dim3 grid(unsigned((p.N * 4 + 255) / 256), unsigned(nb < 512 ? nb : 512));
    L.pre(kProbsToGrad);
    if (a.softcap > 0.f)
      hipLaunchKernelGGL(k_probs_to_grad<true>, grid, dim3(256), 0, L.stream, g,
                         gemm::g_block(p), p.N, nv, v0, vcur, p.V, a.part, p.ld_part, a.lse,
                         a.zt, a.yc, a.ignore_index, a.sc, 1.f / a.softcap);
    else
      hipLaunchKernelGGL(k_probs_to_grad<false>, grid, dim3(256), 0, L.stream, g,
                         gemm::g_block(p), p.N, nv, v0, vcur, p.V, a.part, p.ld_part, a.lse,
                         a.zt, a.yc, a.ignore_index, a.sc, 0.f);
    L.post(kProbsToGrad);
    err = hipGetLastError();
  } else if (a.softcap > 0.f) {
    const EpiGrad<true, false> eg{a.yc, a.lse, a.zt, a.sc, p.N, p.V, a.ignore_index, v0, vcur,
                                  gemm::g_block(p), a.softcap, 1.f / a.softcap, g, 0};
    err = run_gemm<NF, NF, kDynN>(lg, a, eg, kGradLogits, L, nv);
  } else {
    const EpiGrad<false, false> eg{a.yc, a.lse, a.zt, a.sc, p.N, p.V, a.ignore_index, v0, vcur,
                                   gemm::g_block(p), 0.f, 0.f, g, 0};
    err = run_gemm<NF, NF, kDynN>(lg, a, eg, kGradLogits, L, nv);
  }
  if (err != hipSuccess) return err;
  // 2) dW[v0:v0+vcur] = G^T . h (K = the kept tokens) and 3) dH (+)= G . W[chunk]
  // (rows of the kept tokens, chunks in order, scattered to their positions
  // when stored as bf16)
  uint16_t* dW = static_cast<uint16_t*>(a.dW);
  uint16_t* dH = static_cast<uint16_t*>(a.dH);
  const gemm::Launch lw = gemm::backward_launch(p, chunk, 1);
  const gemm::Launch lh = gemm::backward_launch(p, chunk, 2);
  const bool first = chunk == 0, last = chunk == p.n_chunks - 1;
  if (p.dh_kseg) {
    // few dH output tiles: dH split along K, then dW, in one grid, and the
    // segments' partial products added up in a fixed order afterwards
    const int64_t segs = (lh.K + p.dh_kseg - 1) / p.dh_kseg;
    const EpiDHPart ep{a.dh_part, p.N, p.H, p.N * p.H};
    if (a.accumulate_dW)
      err = run_gemm_pair<NF, TF, kDynM, TF, TF, kDynK, true>(
          lh, ep, lw, EpiDW<true>{dW, p.H, v0, vcur}, ag, kGemmDWDH, L, nv, p.dh_kseg, segs);
    else
      err = run_gemm_pair<NF, TF, kDynM, TF, TF, kDynK, true>(
          lh, ep, lw, EpiDW<false>{dW, p.H, v0, vcur}, ag, kGemmDWDH, L, nv, p.dh_kseg, segs);
    if (err != hipSuccess) return err;
    return launch_dh_reduce(a.dh_part, segs, p.N * p.H, first ? nullptr : a.dh_acc,
                            last ? nullptr : a.dh_acc, last ? dH : nullptr, L, p.H, nv, a.idx);
  }
  // dH's tiles and then dW's in one grid
  auto pair = [&](auto edh) {
    if (a.accumulate_dW)
      return run_gemm_pair<NF, TF, kDynM, TF, TF, kDynK>(
          lh, edh, lw, EpiDW<true>{dW, p.H, v0, vcur}, ag, kGemmDWDH, L, nv);
    return run_gemm_pair<NF, TF, kDynM, TF, TF, kDynK>(
        lh, edh, lw, EpiDW<false>{dW, p.H, v0, vcur}, ag, kGemmDWDH, L, nv);
  };
  if (first && last) return pair(EpiDH<true, true>{dH, a.dh_acc, p.N, p.H, a.idx});
  if (first) return pair(EpiDH<true, false>{dH, a.dh_acc, p.N, p.H, a.idx});
  if (last) return pair(EpiDH<false, true>{dH, a.dh_acc, p.N, p.H, a.idx});
  return pair(EpiDH<false, false>{dH, a.dh_acc, p.N, p.H, a.idx});
}

}  // namespace flce

namespace flce {

// The no-recompute variant runs over the gathered tokens (the kept ones
// first): token chunk c is gathered rows [c nc, c nc + nc), of which the
// first ccnt[c] take part in the forward and the first ccnt[nch + c] in the
// backward (device counts).
hipError_t bf16_nr_forward_chunk(const Plan& p, const Args& a, int64_t c, const Launcher& L) {
  const int64_t t0 = c * p.nc, nt = gemm::nr_chunk_tokens(p, c);
  const gemm::Launch l = gemm::nr_launch(p, c, 0);
  uint16_t* probs = static_cast<uint16_t*>(a.g);
  const int64_t* cf = a.ccnt + c;
  constexpr int NF = gemm::kFormN;
  if (a.softcap > 0.f) {
    EpiLseP<true> e{a.yc + t0, nt, p.V, a.ignore_index, a.softcap, 1.f / a.softcap, a.part,
                    p.ld_part, a.zt, probs, gemm::nr_block(p)};
    return run_gemm<NF, NF, kDynN>(l, a, e, kLseFwd, L, cf);
  }
  EpiLseP<false> e{a.yc + t0, nt, p.V, a.ignore_index, 0.f, 0.f, a.part, p.ld_part, a.zt,
                   probs, gemm::nr_block(p)};
  return run_gemm<NF, NF, kDynN>(l, a, e, kLseFwd, L, cf);
}

hipError_t bf16_nr_backward_chunk(const Plan& p, const Args& a, int64_t c, const Launcher& L) {
  const int64_t t0 = c * p.nc, nt = gemm::nr_chunk_tokens(p, c);
  const int64_t* cb = a.ccnt + p.n_tok_chunks + c;     // the chunk's kept tokens
  uint16_t* g = static_cast<uint16_t*>(a.g);
  // 1) G in place of the probabilities
  const int64_t nb = (p.V + 31) / 32;
  const dim3 grid(unsigned((nt * 4 + 255) / 256), unsigned(nb < 512 ? nb : 512));
  const int64_t blk = gemm::nr_block(p);
  L.pre(kProbsToGrad);
  if (a.softcap > 0.f)
    hipLaunchKernelGGL(k_probs_to_grad<true>, grid, dim3(256), 0, L.stream, g, blk, nt, cb,
                       int64_t(0), p.V, p.V, a.part, p.ld_part, a.lse, a.zt, a.yc + t0,
                       a.ignore_index, a.sc, 1.f / a.softcap);
  else
    hipLaunchKernelGGL(k_probs_to_grad<false>, grid, dim3(256), 0, L.stream, g, blk, nt, cb,
                       int64_t(0), p.V, p.V, a.part, p.ld_part, a.lse, a.zt, a.yc + t0,
                       a.ignore_index, a.sc, 0.f);
  L.post(kProbsToGrad);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // 2) dW (+)= G^T . h[chunk] (K = the chunk's kept tokens); over several
  // token chunks the sum is kept in float32 and rounded to bf16 once, at the
  // last chunk. 3) dH[chunk] = G . W over the whole vocabulary, the rows
  // stored at the tokens' original positions (or, with few dH tiles, split
  // along K into partial products). Both in one grid, dH's workgroups first.
  uint16_t* dW = static_cast<uint16_t*>(a.dW);
  uint16_t* dH = static_cast<uint16_t*>(a.dH);
  const int32_t* rmap = a.idx + t0;
  const gemm::Launch lw = gemm::nr_launch(p, c, 1);
  const gemm::Launch lh = gemm::nr_launch(p, c, 2);
  constexpr int T = gemm::kFormT, NF = gemm::kFormN;
  const EpiDH<true, true> edh{dH, nullptr, nt, p.H, rmap};
  const int64_t segs = p.dh_kseg ? (lh.K + p.dh_kseg - 1) / p.dh_kseg : 1;
  auto dw = [&](auto epi) {
    if (p.dh_kseg)
      return run_gemm_pair<NF, T, kDynM, T, T, kDynK, true>(
          lh, EpiDHPart{a.dh_part, nt, p.H, nt * p.H}, lw, epi, a, kGemmDWDH, L, cb, p.dh_kseg,
          segs);
    return run_gemm_pair<NF, T, kDynM, T, T, kDynK>(lh, edh, lw, epi, a, kGemmDWDH, L, cb);
  };
  if (!p.need_dw_acc) {
    err = a.accumulate_dW ? dw(EpiDW<true>{dW, p.H, 0, p.V}) : dw(EpiDW<false>{dW, p.H, 0, p.V});
  } else if (c == 0) {
    err = a.accumulate_dW ? dw(EpiDWAcc<1, 2>{dW, a.dw_acc, p.H, p.V})
                          : dw(EpiDWAcc<0, 2>{dW, a.dw_acc, p.H, p.V});
  } else if (c < p.n_tok_chunks - 1) {
    err = dw(EpiDWAcc<2, 2>{dW, a.dw_acc, p.H, p.V});
  } else {
    err = dw(EpiDWAcc<2, 1>{dW, a.dw_acc, p.H, p.V});
  }
  if (err != hipSuccess || !p.dh_kseg) return err;
  // few dH output tiles: its K segments (run in the grid above) added up in
  // a fixed order
  return launch_dh_reduce(a.dh_part, segs, nt * p.H, nullptr, nullptr, dH, L, p.H, cb, rmap);
}

}  // namespace flce
