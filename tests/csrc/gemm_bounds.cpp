// Host-side check of every global address the bf16 GEMM kernels load, using
// the kernels' own index arithmetic (gemm_index.h) and the library's planner.
// For each problem shape: every launch (forward, and the three launches of
// every backward chunk), every workgroup, wave, lane and load. Direct loads
// are affine in the stage tile, so the first and the last full stage tile are
// checked.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../lm_head_linear_amd/csrc/gemm_index.h"

using namespace flce;
using namespace flce::gemm;

static long failures = 0;

static void fail(const char* what, int64_t a, int64_t b, int64_t c) {
  if (failures < 20) std::printf("FAIL %s (%lld %lld %lld)\n", what, (long long)a, (long long)b, (long long)c);
  ++failures;
}

static int64_t alloc_of(const Plan& p, int buf) {
  if (buf == kBufG) return p.nr ? p.nc * p.vp : p.g_parts * p.vchunk * p.ldg;
  return buf == kBufW ? p.V * p.H : p.N * p.H;
}

static void check_operand(const Plan& p, const Launch& l, int which, int64_t row0) {
  const int sk = stage_k(l.fa, l.fb), nl = loads_per_operand(sk), ntail = tail_loads(sk);
  const int form = which == 0 ? l.fa : l.fb;
  const Geom& g = which == 0 ? l.a : l.b;
  const int64_t base_off = which == 0 ? l.off_a : l.off_b;
  const int64_t alloc = alloc_of(p, which == 0 ? l.buf_a : l.buf_b);
  if (form == kFormT && (g.rows % 8 != 0 || g.rows < 8)) fail("T-form rows % 8", g.rows, 0, 0);
  const int64_t nfull = l.K / sk, nk = (l.K + sk - 1) / sk;
  const int64_t tb = direct_base(form, g, row0), ks = direct_kstep(form, g, sk);
  for (int wave = 0; wave < 4; ++wave)
    for (int lane = 0; lane < 64; ++lane)
      for (int q = 0; q < nl; ++q) {
        const int64_t lo = direct_lane(form, g, row0, wave, lane, q, sk);
        if (lo < 0 || lo * 2 > int64_t(0xFFFFFFFFll) - 16) fail("lane offset", lo, row0, q);
        if (nfull == 0) continue;
        for (int64_t kt : {int64_t(0), nfull - 1}) {
          const int64_t e = base_off + tb + kt * ks + lo;
          if (e < 0 || e + 8 > alloc) fail("direct load out of bounds", e, alloc, kt);
        }
      }
  if (nk > nfull)
    for (int z = 0; z < 256 * ntail; ++z) {
      int64_t off;
      if (tail_src(form, g, row0, nfull * sk, z, sk, off)) {
        const int64_t e = base_off + off;
        if (e < 0 || e + 8 > alloc) fail("tail load out of bounds", e, alloc, z);
      }
      const int pos = tail_lds_pos(form, z, sk);
      if (pos < 0 || pos >= 256 * ntail) fail("tail lds position", pos, z, 0);
    }
}

// The LDS side of the direct loads: on an interior tile (no clamping), the
// element each lane fetches must be the one the fragment reads look for at
// the LDS position the lane writes, and the positions must cover the stage
// tile exactly once.
static void check_lds_layout() {
  const int64_t ld = 4096;
  for (int sk : {32, 64})
    for (int form : {int(kFormN), int(kFormT)}) {
      const Geom g{ld, 1 << 20, 1 << 20};
      const int nl = loads_per_operand(sk);
      std::vector<char> hit(size_t(kBM) * sk * 2 / 16, 0);
      for (int wave = 0; wave < 4; ++wave)
        for (int lane = 0; lane < 64; ++lane)
          for (int q = 0; q < nl; ++q) {
            const int64_t pos = (nl * wave + q) * 64 + lane;   // 16-byte LDS chunk written
            if (pos < 0 || pos >= int64_t(hit.size())) { fail("lds chunk range", pos, q, lane); continue; }
            if (hit[size_t(pos)]++) fail("lds chunk written twice", pos, q, lane);
            const int64_t off = direct_lane(form, g, 0, wave, lane, q, sk);
            const int64_t a = off / ld, b = off % ld;          // (row, k) or (k-row, column)
            const int64_t want = form == kFormN ? lds_chunk_n(int(a), int(b / 8), sk)
                                                : lds_byte_t(int(a), int(b)) / 16;
            if (form == kFormN && (a >= kBM || b >= sk || b % 8)) fail("N element", a, b, q);
            if (form == kFormT && (a >= sk || b >= kBM || b % 8)) fail("T element", a, b, q);
            if (want != pos) fail("lds position mismatch", sk, pos, want);
          }
      for (size_t i = 0; i < hit.size(); ++i)
        if (!hit[i]) fail("lds chunk never written", sk, int64_t(i), form);
      // tail path: a bijection onto the same positions
      std::vector<char> th(hit.size(), 0);
      for (int z = 0; z < 256 * tail_loads(sk); ++z) {
        const int pos = tail_lds_pos(form, z, sk);
        if (pos < 0 || pos >= int(th.size()) || th[size_t(pos)]++) fail("tail position", sk, z, pos);
      }
    }
}

// The transposed fragment read (ds_read_b64_tr_b16, 8 bytes per lane) of a
// T-form stage tile: lane i of 16-lane group g reads k-row 8 g + 4 r + i / 4 at
// columns row_base + 4 (i % 4) .. + 3. Each 32-lane half of the read (served
// together, the LDS's 64 four-byte banks at once) covers every bank once: the
// bank-conflict counter on gfx950 reads 0 for this layout.
static void check_lds_banks_t() {
  for (int r = 0; r < 2; ++r)
    for (int rb = 0; rb < kBM; rb += 16)
      for (int half = 0; half < 2; ++half) {
        int banks[64] = {0};
        for (int lane = 32 * half; lane < 32 * half + 32; ++lane) {
          const int g = lane >> 4, i = lane & 15;
          const int byte = lds_byte_t(8 * g + 4 * r + (i >> 2), rb + 4 * (i & 3));
          for (int w = 0; w < 2; ++w) banks[(byte / 4 + w) % 64]++;
        }
        for (int b = 0; b < 64; ++b)
          if (banks[b] != 1) fail("transposed read bank", r, rb, b);
      }
}

// Same predicate as the library's launch check: the 32-bit lane offsets fit.
static bool offsets_fit(int form, const Geom& g) {
  const int64_t reach = form == kFormN ? (g.rows - 1 < 255 ? g.rows - 1 : 255) * g.ld + 64
                        : g.blk ? 7 * g.blk + 64 * 32
                                : 63 * g.ld + g.rows;
  return reach >= 0 && 2 * reach + 16 <= int64_t(0xFFFFFFFF);
}

// The blocked geometry (the logit gradient G) fetches, for every lane, load
// and stage tile, the same logical element as the dense geometry of the same
// matrix, and its tail path reads the same elements. Dense: G[t][v] at
// t * ld + v; blocked: at blocked_offset(t, v, blk).
static void check_blocked_matches_dense() {
  const int64_t T = 700, Vc = 1024, ld = Vc, blk = 704 * 32;   // 704: T rounded up to 8
  auto dense_tv = [&](int64_t e, int64_t& t, int64_t& v) { t = e / ld; v = e % ld; };
  auto blocked_tv = [&](int64_t e, int64_t& t, int64_t& v) {
    v = (e / blk) * 32 + (e % blk) % 32;
    t = (e % blk) / 32;
  };
  const int sk = 32;
  // N form (dH: rows = tokens, K = vocabulary) and T form (dW: K = tokens,
  // rows = vocabulary)
  for (int form : {int(kFormN), int(kFormT)}) {
    const Geom gd = form == kFormN ? Geom{ld, T, Vc} : Geom{ld, Vc, T};
    const Geom gb = form == kFormN ? Geom{32, T, Vc, blk} : Geom{32, Vc, T, blk};
    const int64_t rows = form == kFormN ? T : Vc, K = form == kFormN ? Vc : T;
    for (int64_t row0 = 0; row0 < rows; row0 += kBM)
      for (int64_t kt : {int64_t(0), int64_t(1), K / sk - 1}) {
        for (int wave = 0; wave < 4; ++wave)
          for (int lane = 0; lane < 64; ++lane)
            for (int q = 0; q < loads_per_operand(sk); ++q) {
              const int64_t ed = direct_base(form, gd, row0) + kt * direct_kstep(form, gd, sk) +
                                 direct_lane(form, gd, row0, wave, lane, q, sk);
              const int64_t eb = direct_base(form, gb, row0) + kt * direct_kstep(form, gb, sk) +
                                 direct_lane(form, gb, row0, wave, lane, q, sk);
              int64_t t1, v1, t2, v2;
              dense_tv(ed, t1, v1);
              blocked_tv(eb, t2, v2);
              if (t1 != t2 || v1 != v2) fail("blocked load differs from dense", form, t1 * ld + v1, t2 * ld + v2);
            }
        for (int z = 0; z < 256 * tail_loads(sk); ++z) {
          int64_t od, ob;
          const bool vd = tail_src(form, gd, row0, kt * sk, z, sk, od);
          const bool vb = tail_src(form, gb, row0, kt * sk, z, sk, ob);
          if (vd != vb) { fail("blocked tail validity", form, z, kt); continue; }
          if (!vd) continue;
          int64_t t1, v1, t2, v2;
          dense_tv(od, t1, v1);
          blocked_tv(ob, t2, v2);
          if (t1 != t2 || v1 != v2) fail("blocked tail differs from dense", form, z, kt);
        }
      }
  }
}

static void check_launch(const Plan& p, const Launch& l, bool spread_m = false) {
  if (!offsets_fit(l.fa, l.a) || !offsets_fit(l.fb, l.b)) fail("offsets exceed 32 bits", l.M, l.Nn, l.K);
  const int64_t nt = num_tiles(l.M, l.Nn);
  const int64_t num_m = (l.M + kBM - 1) / kBM;
  std::vector<char> seen(size_t(nt), 0);
  for (int64_t b = 0; b < nt; ++b) {
    int64_t m0, n0;
    tile_coords(b, l.M, l.Nn, kGroupM, m0, n0, spread_m);
    if (m0 < 0 || m0 >= l.M || n0 < 0 || n0 >= l.Nn || m0 % kBM || n0 % kBM) {
      fail("tile out of range", b, m0, n0);
      continue;
    }
    char& s = seen[size_t((n0 / kBM) * num_m + m0 / kBM)];
    if (s) fail("tile visited twice", b, m0, n0);
    s = 1;
    check_operand(p, l, 0, m0);
    check_operand(p, l, 1, n0);
  }
}

// The segments of a split-K dH launch: every segment's loads in bounds, and
// the segments cover K exactly once in order.
static int64_t n_split_segments = 0;
static void check_split(const Plan& p, const Launch& l) {
  if (!p.dh_kseg) return;
  if (p.dh_kseg % 64) fail("segment length", p.dh_kseg, l.K, 0);
  const int64_t segs = (l.K + p.dh_kseg - 1) / p.dh_kseg;
  if (segs > p.dh_segs) fail("more segments than carved", segs, p.dh_segs, l.K);
  int64_t covered = 0;
  for (int64_t z = 0; z < segs; ++z) {
    const Launch s = split_segment(l, p.dh_kseg, z);
    if (s.K <= 0 || s.K > p.dh_kseg) fail("segment size", z, s.K, l.K);
    covered += s.K;
    check_launch(p, s);
    ++n_split_segments;
  }
  if (covered != l.K) fail("segments do not cover K", covered, l.K, segs);
}

// The chunks whose probabilities the forward keeps: chunks 0 .. n-2 in dW's
// free rows, chunk n-1 in the G buffer (a chunk that exists, so the
// recompute of chunk n is the first to write that buffer). Chunk j's G
// (vchunk x ldg bf16) in dW lies inside dW, 256-byte aligned, clear of the
// rows of chunks 0 .. j (written by their dH + dW launches before or while it
// is read) and of every other kept chunk. The G reads of chunk j's launches
// are within vchunk x ldg elements of its base (check_launch), so they stay
// inside that range too.
static int64_t n_kept_extra = 0;
static void check_kept(const Plan& p) {
  const Kept k = kept_chunks(p, true);
  const Kept none = kept_chunks(p, false);
  if (none.n != 1 || none.in_dw(0)) fail("chunks kept in dW while dW is added to", none.n, p.N, p.V);
  if (k.n < 1 || k.n > kMaxKept || k.n > p.n_chunks) fail("kept count", k.n, p.n_chunks, 0);
  if (k.in_dw(k.n - 1)) fail("the last kept chunk is not in the G buffer", k.n, 0, 0);
  const int64_t dw_bytes = p.V * p.H * 2, bytes = p.vchunk * p.ldg * 2;
  for (int j = 0; j < k.n; ++j) {
    if (!k.in_dw(j)) continue;
    const int64_t lo = k.off[j], hi = lo + bytes;
    if (lo % 256) fail("kept chunk alignment", j, lo, 0);
    if (lo < 0 || hi > dw_bytes) fail("kept chunk outside dW", j, lo, dw_bytes);
    for (int c = 0; c <= j && c < p.n_chunks; ++c) {
      const int64_t r0 = c * p.vchunk * p.H * 2, r1 = r0 + chunk_rows(p, c) * p.H * 2;
      if (lo < r1 && r0 < hi) fail("kept chunk overlaps rows written before it is read", j, c, lo);
    }
    for (int q = 0; q < k.n; ++q)
      if (q != j && k.in_dw(q) && lo < k.off[q] + bytes && k.off[q] < hi)
        fail("kept chunks overlap", j, q, lo);
    ++n_kept_extra;
  }
}

int main(int argc, char** argv) {
  // N H V [vchunk]
  struct Shape { int64_t N, H, V, vc; };
  std::vector<Shape> shapes = {
      {1, 8, 1, 0},        {1, 8, 2, 0},        {3, 8, 7, 0},       {257, 64, 257, 0},
      {600, 264, 1500, 512}, {513, 136, 777, 256}, {1000, 512, 3000, 1024},
      {255, 8, 255, 0},    {257, 8, 300, 256},  {8, 8, 8, 0},       {7, 16, 513, 256},
      {300, 136, 1000, 0}, {700, 128, 1500, 512}, {1024, 256, 4096, 0}, {1100, 128, 2000, 0},
      {100, 16, 1, 0},     {100, 16, 2, 0},     {333, 64, 1024, 0},  {256, 64, 512, 0},
      {2048, 1024, 32000, 0}, {4096, 4096, 131072, 0}, {8192, 4096, 131072, 0},
      {8192, 3584, 256000, 0}, {16384, 4096, 131072, 0},
      // few dH output tiles: split-K segments, ragged last segment, several chunks
      {300, 136, 9000, 0}, {600, 264, 20000, 4096}, {2048, 1024, 33000, 0}};
  check_lds_layout();
  check_lds_banks_t();
  check_blocked_matches_dense();
  std::printf("lds layout and blocked G: %s\n", failures ? "FAILURES" : "ok");
  if (argc == 5) shapes = {{std::atoll(argv[1]), std::atoll(argv[2]), std::atoll(argv[3]), std::atoll(argv[4])}};
  for (const Shape& s : shapes) {
    if (s.vc > 0) {
      char buf[32];
      std::snprintf(buf, sizeof buf, "%lld", (long long)s.vc);
      setenv("FLCE_VCHUNK", buf, 1);
    } else {
      unsetenv("FLCE_VCHUNK");
    }
    for (int grad : {1, 0}) {       // bf16 gradients, then float32 gradients (G hi + lo)
      Plan p;
      if (!make_plan(s.N, s.H, s.V, 1, &p, true, grad)) { fail("plan", s.N, s.H, s.V); continue; }
      check_launch(p, forward_launch(p));
      check_launch(p, forward_launch(p), true);     // the raster that deals M-tiles to XCDs
      check_kept(p);
      for (int64_t c = 0; c < p.n_chunks; ++c) {
        check_launch(p, backward_launch(p, c, 0));
        for (int part = 0; part < p.g_parts; ++part)
          for (int w = 1; w < 3; ++w) check_launch(p, backward_launch(p, c, w, part));
        check_split(p, backward_launch(p, c, 2));
      }
    }
    for (int64_t tc : {int64_t(0), int64_t(256), int64_t(1000)}) {   // no-recompute variant
      Plan q;
      if (!make_plan_nr(s.N, s.H, s.V, 1, tc, &q)) { fail("plan nr", s.N, s.H, tc); continue; }
      for (int64_t c = 0; c < q.n_tok_chunks; ++c) {
        for (int w = 0; w < 3; ++w) check_launch(q, nr_launch(q, c, w));
        check_split(q, nr_launch(q, c, 2));
      }
    }
    Plan p;
    make_plan(s.N, s.H, s.V, 1, &p);
    std::printf("shape N=%lld H=%lld V=%lld chunk=%lld chunks=%lld: %s\n", (long long)s.N,
                (long long)s.H, (long long)s.V, (long long)p.vchunk, (long long)p.n_chunks,
                failures ? "FAILURES" : "ok");
  }
  if (failures == 0)
    std::printf("all loads in bounds (%lld split-K segments, %lld chunks kept in dW)\n",
                (long long)n_split_segments, (long long)n_kept_extra);
  return failures ? 1 : 0;
}
