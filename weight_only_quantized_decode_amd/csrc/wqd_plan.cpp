// Packed sizes, validation and launch planning (host only, no HIP).
#include "wqd_plan.h"

namespace wqd {

int packed_sizes(int fmt, int64_t N, int64_t K, PackedSizes* out) {
  if (!fmt_ok(fmt) || N < 1 || K < 1) return kEArg;
  if (fmt == kFmtW4 ? (K % kGroup) != 0 : (K % 8) != 0) return kEShape;
  if (N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return kEShape;
  PackedSizes p;
  p.NB = ceil_div(N, kTileRows);
  p.KT = ceil_div(K, tile_k(fmt));
  p.G4 = 0;
  p.w_bytes = size_t(p.NB) * size_t(p.KT) * kTileBytes;
  if (fmt == kFmtBF16) {
    p.s_bytes = 0;
    p.z_bytes = 0;
  } else if (fmt == kFmtFP8) {
    p.s_bytes = size_t(p.NB) * kTileRows * sizeof(float);
    p.z_bytes = 0;
  } else {
    p.G4 = ceil_div(K / kGroup, kScaleQuad);
    p.s_bytes = size_t(p.NB) * size_t(p.G4) * kTileRows * kScaleQuad * 2;  // fp16 [NB][G4][16][4]
    p.z_bytes = size_t(p.NB) * size_t(p.G4) * kTileRows * 2;               // 4 nibbles [NB][G4][16]
  }
  *out = p;
  return kOK;
}

int plan_gemv(int fmt, int64_t M, int64_t N, int64_t K, GemvPlan* out) {
  PackedSizes ps;
  int st = packed_sizes(fmt, N, K, &ps);
  if (st != kOK) return st;
  if (M < 1) return kEArg;
  GemvPlan g{};
  g.NB = ps.NB;
  g.KT = ps.KT;
  g.mrows = int(M < kGemvMaxM ? M : kGemvMaxM);
  g.nchunks = int(ceil_div(M, kGemvMaxM));
  // Fewer than two 16-row blocks per compute unit (256 CUs): spread K over 8
  // wavefronts per workgroup to keep more loads in flight (LDS allows it for
  // up to 2 activation rows).
  g.waves = (g.NB < 512 && g.mrows <= 2) ? 8 : 4;
  *out = g;
  return kOK;
}

// Wavefronts per workgroup: the fewest whose shares fit the preferred length
// (32 tiles; 16 for BF16, whose tiles carry a quarter of the K of W4A16), then
// doubled while the launch has fewer wavefronts than the target (8 per
// compute unit; 16 for BF16) and each still gets at least one group of 4
// tiles.  Fewer, longer shares amortise each wavefront's start (its x sums
// and first loads).  Measured on the 70B and 7B shapes.  Three or more rows,
// and two W4A16 rows, keep shares of at most 16 tiles (registers).
int plan_bcast(int fmt, int64_t M, int64_t N, int64_t K, BcastPlan* out) {
  PackedSizes ps;
  int st = packed_sizes(fmt, N, K, &ps);
  if (st != kOK) return st;
  if (M < 1) return kEArg;
  if (M > (fmt == kFmtW4 ? kBcastMaxMW4 : kBcastMaxM)) return kEUnsupported;
  auto share = [&](int w) { return ceil_div(ps.KT, 4 * int64_t(w)) * 4; };
  const int64_t pref = fmt == kFmtBF16 ? 16 : 32;
  const int64_t cap = (M >= 3 || (fmt == kFmtW4 && M == 2)) ? 16 : 32;
  const int64_t target = fmt == kFmtBF16 ? 4096 : 2048;
  int w = 4;
  while (w < 16 && share(w) > (pref < cap ? pref : cap)) w *= 2;
  if (share(w) > cap) return kEUnsupported;
  while (w < 16 && ps.NB * w < target && ceil_div(ps.KT, 4) >= 2 * w) w *= 2;
  BcastPlan p{};
  p.NB = ps.NB;
  p.KT = ps.KT;
  p.waves = w;
  p.per_wave = int(share(w));
  p.groups = p.per_wave <= 16 ? 4 : 8;
  *out = p;
  return kOK;
}

// Wavefronts per workgroup as for the broadcast kernel: the fewest whose
// shares hold at most 32 tiles, doubled while the launch has fewer than 2048
// wavefronts and each keeps at least one group of 4 tiles.
constexpr int64_t kComputeUnits = 256;  // MI355X

int plan_mc(int fmt, int64_t M, int64_t N, int64_t K, McPlan* out) {
  PackedSizes ps;
  int st = packed_sizes(fmt, N, K, &ps);
  if (st != kOK) return st;
  if (M < 1) return kEArg;
  if (M > kMcMaxM || M * K * 2 >= (int64_t(1) << 31)) return kEUnsupported;
  auto share = [&](int w) { return ceil_div(ps.KT, 4 * int64_t(w)) * 4; };
  // Two 16-row blocks per wavefront halve the x reads per weight byte.  Measured
  // on the 70B shapes: a clear gain for W4A16 (whose x bytes per weight byte
  // are the highest) and for long K, neutral to slightly negative for short-K
  // FP8; below 128 blocks the launch gets too few wavefronts.
  // From 9 rows (up to 16) FP8 takes two row blocks as well, and FP8 / W4A16
  // keep the fewest wavefronts whose shares fit (measured on 8192^2 and
  // 4096^2: 5-12% faster than doubling them).
  const bool wide = M > kGemvMaxM && fmt != kFmtBF16;
  int rb = ps.NB >= 128 && (fmt == kFmtW4 || ps.KT >= 256 || wide) ? 2 : 1;
  // Three row blocks when that lowers the most row blocks any compute unit
  // carries (one workgroup per unit is the aim: a unit running two takes
  // their time end to end): 640 blocks (a 10240-row matrix) give 214
  // workgroups of three instead of 320 of two.  Not with 16 wavefronts,
  // whose 128 registers three row blocks do not fit.
  if (rb == 2 && share(8) <= 32 &&
      ceil_div(ceil_div(ps.NB, 3), kComputeUnits) * 3 < ceil_div(ceil_div(ps.NB, 2), kComputeUnits) * 2)
    rb = 3;
  const int64_t units = ceil_div(ps.NB, rb);
  int w = 4;
  while (w < 16 && share(w) > 32) w *= 2;
  if (share(w) > 32) return kEUnsupported;
  while (!wide && w < (rb == 3 ? 8 : 16) && units * w < 2048 / rb && ceil_div(ps.KT, 4) >= 2 * w) w *= 2;
  McPlan p{};
  p.NB = ps.NB;
  p.KT = ps.KT;
  p.waves = w;
  p.per_wave = int(share(w));
  p.rb = rb;
  *out = p;
  return kOK;
}

// Skinny kernel: consumer wavefronts per workgroup and row blocks per consumer
// from (7, 2), (7, 1), (4, 2), (5, 2) (x chunks shared by 14, 7, 8 or 10 row
// blocks; 10 fills the compute units for N = 10240 with 4 splits); a
// ring of 8 weight tiles per row block; x chunks of 4 tiles (2 for W4A16 from
// 17 rows and for everything from 33, whose chunks would otherwise need up to
// 200 KiB of LDS), three buffers.  K is
// split so that the launch has about as many workgroups as compute units
// (S = units / groups: a second workgroup on only some units would make them
// the tail), keeping every split at least 2 rings long and at most 8 splits
// (each adds M * N * 8 bytes of partial traffic).  The configuration whose
// workgroups fill whole multiples of the compute units best wins; near ties
// go to the earlier one (measured on the 70B shapes).

static int plan_skinny_with(int fmt, int64_t M, const PackedSizes& ps, int waves, int rb, int64_t S, SkPlan* out) {
  SkPlan p{};
  p.NB = ps.NB;
  p.KT = ps.KT;
  p.mf = int(ceil_div(M, 16));
  p.rb = rb;
  p.waves = waves;
  p.ring = 8;
  p.ct = (fmt == kFmtW4 && p.mf >= 2) || p.mf >= 3 ? 2 : 4;
  p.nx = 3;
  p.groups = ceil_div(p.NB, int64_t(p.waves) * p.rb);
  const int64_t body = p.ring;
  if (S < 1) {
    S = kComputeUnits / p.groups;
    const int64_t max_s = p.KT / (2 * body);
    if (S > max_s) S = max_s;
    if (S > 8) S = 8;
    if (S < 1) S = 1;
  }
  const int64_t per = ceil_div(ceil_div(p.KT, S), body) * body;
  p.per_split = int(per);
  p.S = int(ceil_div(p.KT, per));
  *out = p;
  return kOK;
}

int plan_skinny(int fmt, int64_t M, int64_t N, int64_t K, SkPlan* out) {
  PackedSizes ps;
  int st = packed_sizes(fmt, N, K, &ps);
  if (st != kOK) return st;
  if (M < 1) return kEArg;
  if (M > kSkMaxM || M * K * 2 >= (int64_t(1) << 31)) return kEUnsupported;
  if (K % tile_k(fmt) != 0) return kEUnsupported;
  if (ps.s_bytes >= (size_t(1) << 31) || ps.z_bytes >= (size_t(1) << 31)) return kEUnsupported;
  SkPlan p{};
  if (fmt == kFmtW4 && M > 16 && ps.KT >= 128) {
    // W4A16 from 17 rows on long K: the dequantisation and group corrections
    // make the kernel compute-heavy and more resident wavefronts pay
    // (measured on 8192 x 28672 at 17-64 rows, 17-27% faster than the
    // choice below): two x row blocks take 4 consumers with twice the
    // splits (two workgroups per compute unit), three or four take 7
    // consumers of two row blocks (one workgroup per compute unit).
    if (ceil_div(M, 16) == 2) {
      const int64_t groups = ceil_div(ps.NB, int64_t(8));
      int64_t S = 2 * kComputeUnits / groups;
      const int64_t max_s = ps.KT / 16;
      S = S > 8 ? 8 : S;
      S = S > max_s ? max_s : S;
      plan_skinny_with(fmt, M, ps, 4, 2, S < 1 ? 1 : S, &p);
    } else {
      plan_skinny_with(fmt, M, ps, 7, 2, 0, &p);
    }
    p.ws_bytes = p.S > 1 ? size_t(p.S) * size_t(M) * size_t(N) * sizeof(float) : 0;
    *out = p;
    return kOK;
  }
  double best = -1.0;
  for (const auto& cfg : kSkCfg) {
    SkPlan q;
    plan_skinny_with(fmt, M, ps, cfg[0], cfg[1], 0, &q);
    const int64_t W = q.groups * q.S;
    const double fill = double(W) / double(ceil_div(W, kComputeUnits) * kComputeUnits);
    if (fill > best + 0.02) {
      best = fill;
      p = q;
    }
  }
  p.ws_bytes = p.S > 1 ? size_t(p.S) * size_t(M) * size_t(N) * sizeof(float) : 0;
  *out = p;
  return kOK;
}

// Tiled kernel (above kGmMinM rows, where it measured faster than the LDS
// matrix-core kernel on the 70B verify shapes once N gives at least kGmMinNBN
// column blocks).  Tile heights: 64 rows (4 wavefronts for BF16 / FP8, 8 for
// W4A16) or, with wm = 2, 256 rows of 8 wavefronts (BF16 / FP8) or 128 rows
// (W4A16).  Height and K split come from time models fitted to the kernel on
// the 7B and 70B projection shapes (W = tiles x splits workgroups, cps chunks
// of 64 k (128 for W4A16) per workgroup, S splits):
//  * BF16 / FP8: t = c0 + cps x (a + b x fill) x L + S x M x N x 8 B / bw,
//    where fill is the share of real rows in the padded tiles and L = 1 for
//    W <= 256, else r x ceil(W / 256) (r < 1 for 64-row tiles, which run two
//    workgroups per compute unit side by side); the last term, for S > 1, is
//    the float32 partials written and read once.  Fitted constants below
//    (c0 in us, a and b in us per chunk, bw in TB/s); on the fitting sweep
//    the modelled choice came within 1.3% of the best measured one in total.
//  * W4A16: ceil(W / 256) rounds of cps chunks at 1.33 us (64 rows) or 2.26
//    (128 rows) per chunk, plus partials at about 4 TB/s.
// The cheapest S from 1 to 8 (each split at least 4 chunks) wins, within 2%
// the smaller S; between heights the taller one needs a 2% margin.
struct GmCost {
  double c0, a, b, r, bw;
};
static constexpr GmCost kGmCost[2][2] = {
    {{7.7, 0.771, 0.0, 0.941, 4.37}, {10.5, 1.649, 0.498, 1.103, 5.38}},   // BF16: 64 / 256 rows
    {{8.4, 0.469, 0.079, 0.912, 4.49}, {11.4, 1.23, 0.394, 1.13, 6.16}},  // FP8
};
// One tile shape (wm) of the tiled kernel: its padded rows, x-sum bytes and
// the K split of least modelled time (returned in *t_us).
static int plan_gemm_wm(int fmt, int64_t M, int64_t N, int64_t K, const PackedSizes& ps, int wm, GmPlan* out,
                        double* t_us) {
  GmPlan p{};
  p.NB = ps.NB;
  p.KT = ps.KT;
  p.wm = wm;
  const bool wide = wm == 2;  // 128-row wavefront tiles
  const int64_t rows = !wide ? 64 : fmt == kFmtW4 ? 128 : 256;  // per workgroup
  p.NBN = ceil_div(p.NB, 16);
  p.MB = ceil_div(M, rows);
  p.Mp = p.MB * rows;
  p.nchunks = fmt == kFmtW4 ? p.KT : ceil_div(K, 64);
  if (fmt == kFmtW4 && p.KT * p.Mp * 4 >= (int64_t(1) << 31)) return kEUnsupported;
  p.xs_bytes = fmt == kFmtW4 ? (size_t(p.KT) * size_t(p.Mp) * sizeof(float) + 255) / 256 * 256 : 0;
  const int64_t tiles = p.NBN * p.MB;
  const double mn8 = double(M) * double(N) * 8.0;  // one split's partials, bytes
  const double fill = double(M) / double(p.Mp);
  const int64_t max_s = p.nchunks / 4 < 1 ? 1 : (p.nchunks / 4 > 8 ? 8 : p.nchunks / 4);
  double best = 0.0;
  int64_t S = 1;
  for (int64_t s = 1; s <= max_s; ++s) {
    const int64_t cps = ceil_div(p.nchunks, s), se = ceil_div(p.nchunks, cps);
    const int64_t rounds = ceil_div(tiles * se, kComputeUnits);
    double t;
    if (fmt == kFmtW4) {
      t = double(rounds) * double(cps) * (wide ? 2.26 : 1.33) + (se > 1 ? double(se) * mn8 / 4.0e6 : 0.0);
    } else {
      const GmCost& c = kGmCost[fmt == kFmtFP8][wide];
      const double L = rounds == 1 ? 1.0 : c.r * double(rounds);
      t = c.c0 + double(cps) * (c.a + c.b * fill) * L + (se > 1 ? double(se) * mn8 / (c.bw * 1.0e6) : 0.0);
    }
    if (s == 1 || t < 0.98 * best) {
      best = t;
      S = se;
    }
  }
  p.cps = ceil_div(p.nchunks, S);
  p.S = int(ceil_div(p.nchunks, p.cps));
  p.ws_bytes = p.xs_bytes + (p.S > 1 ? size_t(p.S) * size_t(M) * size_t(N) * sizeof(float) : 0);
  if (fmt == kFmtW4 && p.S == 1 && p.NBN > 8) {
    // tail split: the column blocks from nbn1 (a multiple of 8, so that
    // every XCD keeps whole column blocks) run as S2 K splits after the
    // others, filling the last round that whole tiles would leave part idle
    // (the 70B gate at 1024 rows: 896 tiles, 3.5 rounds); their partials
    // take a small second launch.  Rounds on the busiest XCD (32 compute
    // units, one workgroup each).
    const double k = wide ? 2.26 : 1.33;
    const int64_t per_cu = kComputeUnits / 8;
    for (int64_t nbn1 = 8; nbn1 < p.NBN; nbn1 += 8) {
      const int64_t r1 = ceil_div(nbn1 / 8 * p.MB, per_cu);
      for (int s2 = 2; s2 <= 4; ++s2) {
        const int64_t cps2 = ceil_div(p.nchunks, int64_t(s2));
        if (ceil_div(p.nchunks, cps2) != s2 || cps2 < 4) continue;
        const int64_t r2 = ceil_div(ceil_div(p.NBN - nbn1, int64_t(8)) * p.MB * s2, per_cu);
        const double nt = double(N - nbn1 * 256);
        const double t = (double(r1) * double(p.nchunks) + double(r2) * double(cps2)) * k +
                         double(s2) * double(M) * nt * 8.0 / 4.0e6 + 4.0;
        if (t < 0.98 * best) {
          best = t;
          p.nbn1 = nbn1;
          p.S2 = s2;
          p.cps2 = int(cps2);
        }
      }
    }
    if (p.S2 > 0)
      p.ws_bytes = p.xs_bytes + size_t(p.S2) * size_t(M) * size_t(N - p.nbn1 * 256) * sizeof(float);
  }
  *out = p;
  *t_us = best;
  return kOK;
}

// The tiled kernel with both operands staged in LDS (wm = 3; BF16 and FP8):
// 256 x 256 tiles, one workgroup per compute unit, chunks of one packed tile
// along K (32 k BF16, 64 k FP8).  Time model t = c0 + cps * a * rounds + the
// split partials (written and read once at bw), fitted by least squares to
// the kernel on the 70B q, gate and down shapes at 192-1024 rows (rms error
// ~10% BF16, ~4% FP8).
struct GlCost {
  double c0, a, bw;
};
static constexpr GlCost kGlCost[2] = {
    {13.0, 0.89, 3.75},   // BF16
    {12.07, 1.53, 5.15},  // FP8
};
constexpr int64_t kGlMinM = 192;

// FP8 tile shapes of the LDS-staged kernel: (weight row blocks per wavefront,
// wavefront rows of 64 rows) and the time of one of its 64-k chunks relative
// to the 256 x 256 tile's.
struct GlShape {
  int rbw, lwr;
  double f;
};
#ifndef WQD_GL_F72
#define WQD_GL_F72 0.93
#endif
#ifndef WQD_GL_BF16_F74
#define WQD_GL_BF16_F74 0.965
#endif
#ifndef WQD_GL_FORCE_SHAPE
static constexpr GlShape kGlShapes[] = {{8, 4, 1.0}, {7, 4, 0.95}, {7, 2, WQD_GL_F72}};
static constexpr GlShape kGlShapesBf16[] = {{8, 4, 1.0}, {7, 4, WQD_GL_BF16_F74}};
#else
static constexpr GlShape kGlShapes[] = {WQD_GL_FORCE_SHAPE};  // measurement builds only
static constexpr GlShape kGlShapesBf16[] = {WQD_GL_FORCE_SHAPE};
#endif

static int plan_gemm_lds(int fmt, int64_t M, int64_t N, int64_t K, const PackedSizes& ps, GmPlan* out,
                         double* t_us) {
  if (fmt != kFmtBF16 && fmt != kFmtFP8) return kEUnsupported;
  // fitted and measured from 192 rows (below, most of a 256-row tile is padding)
  if (M < kGlMinM) return kEUnsupported;
  // K a whole number of tiles (no x piece of a tile lies past K)
  if (K % tile_k(fmt) != 0) return kEUnsupported;
  // weight offsets of 32 row blocks stay below 2^31
  if (32 * ps.KT * kTileBytes >= (int64_t(1) << 31)) return kEUnsupported;
  GmPlan p{};
  p.NB = ps.NB;
  p.KT = ps.KT;
  p.wm = 3;
  p.nchunks = p.KT;
  const double mn8 = double(M) * double(N) * 8.0;
  const int64_t max_s = p.nchunks / 8 < 1 ? 1 : (p.nchunks / 8 > 8 ? 8 : p.nchunks / 8);
  const GlCost& gc = kGlCost[fmt == kFmtFP8];
  // the tile shape that fills the compute units' rounds best and the K split
  const GlShape* shapes = fmt == kFmtFP8 ? kGlShapes : kGlShapesBf16;
  const int nshapes = fmt == kFmtFP8 ? int(sizeof(kGlShapes) / sizeof(kGlShapes[0]))
                                     : int(sizeof(kGlShapesBf16) / sizeof(kGlShapesBf16[0]));
  double best = 0.0;
  int64_t S = 1;
  GlShape pick = shapes[0];
  bool first = true;
  for (int h = 0; h < nshapes; ++h) {
    const GlShape& sh = shapes[h];
    // column block j runs on XCD j % 8 (workgroups are dispatched round-robin
    // over the 8 XCDs and the kernel maps them so), so the busiest XCD holds
    // ceil(NBN / 8) column blocks' workgroups for its 32 compute units
    const int64_t nbn_xcd = ceil_div(ceil_div(p.NB, int64_t(8 / sh.lwr * sh.rbw)), int64_t(8));
    const int64_t per_xcd = nbn_xcd * ceil_div(M, int64_t(64 * sh.lwr));
    for (int64_t s = 1; s <= max_s; ++s) {
      const int64_t cps = ceil_div(p.nchunks, s), se = ceil_div(p.nchunks, cps);
      const int64_t rounds = ceil_div(per_xcd * se, kComputeUnits / 8);
      const double t =
          gc.c0 + double(cps) * gc.a * sh.f * double(rounds) + (se > 1 ? double(se) * mn8 / (gc.bw * 1.0e6) : 0.0);
      if (first || t < 0.98 * best) {
        best = t;
        S = se;
        pick = sh;
        first = false;
      }
    }
  }
  p.rbw = pick.rbw;
  p.lwr = pick.lwr;
  p.NBN = ceil_div(p.NB, int64_t(8 / pick.lwr * pick.rbw));
  p.MB = ceil_div(M, int64_t(64 * pick.lwr));
  p.Mp = p.MB * 64 * pick.lwr;
  p.cps = ceil_div(p.nchunks, S);
  p.S = int(ceil_div(p.nchunks, p.cps));
  p.ws_bytes = p.S > 1 ? size_t(p.S) * size_t(M) * size_t(N) * sizeof(float) : 0;
  *out = p;
  *t_us = best;
  return kOK;
}

int plan_gemm(int fmt, int64_t M, int64_t N, int64_t K, GmPlan* out) {
  PackedSizes ps;
  int st = packed_sizes(fmt, N, K, &ps);
  if (st != kOK) return st;
  if (M < 1) return kEArg;
  if (M * K * 2 >= (int64_t(1) << 31)) return kEUnsupported;
#ifdef WQD_GEMM_FORCE_WM
  {
    // measurement builds only: one tile shape regardless of the models
    double t = 0.0;
    GmPlan pf;
    const int wf = WQD_GEMM_FORCE_WM;
    if ((wf == 3 ? plan_gemm_lds(fmt, M, N, K, ps, &pf, &t) : plan_gemm_wm(fmt, M, N, K, ps, wf, &pf, &t)) == kOK) {
      *out = pf;
      return kOK;
    }
  }
#endif
  double t1 = 0.0, t2 = 0.0, t3 = 0.0;
  GmPlan p3;
  const bool lds_ok = plan_gemm_lds(fmt, M, N, K, ps, &p3, &t3) == kOK;
  // 64-row tiles or the taller ones, whichever the model puts faster (within
  // 2%: 64).  Taller tiles read each weight chunk for more rows (W4A16: half
  // the dequantisation per multiply) but pad M and quantise the launch into
  // rounds more coarsely (W4A16 on the 70B shapes: 4-14% faster for gate /
  // down from 512 rows and q from 768, up to 12% slower where the rounds fall
  // badly, e.g. gate at 384 rows).
  GmPlan p1, p2;
  st = plan_gemm_wm(fmt, M, N, K, ps, 1, &p1, &t1);
  if (st != kOK) return st;
  GmPlan best = p1;
  double tb = t1;
  if (plan_gemm_wm(fmt, M, N, K, ps, 2, &p2, &t2) == kOK && t2 < 0.98 * tb) {
    best = p2;
    tb = t2;
  }
  if (lds_ok && t3 < 0.98 * tb) best = p3;
  *out = best;
  return kOK;
}

// Tiles per chunk of the matrix-core kernel: the staged x chunk is 16 KiB
// (16 * BMS rows), at most 8 tiles.
static int mfma_tpc(int fmt, int bms) {
  const int raw = 8192 / (16 * bms * tile_k(fmt));
  return raw > 8 ? 8 : (raw < 1 ? 1 : raw);
}

int plan_mfma(int fmt, int64_t M, int64_t N, int64_t K, MfmaPlan* out) {
  PackedSizes ps;
  int st = packed_sizes(fmt, N, K, &ps);
  if (st != kOK) return st;
  if (M < 1) return kEArg;
  MfmaPlan p{};
  p.BMS = M <= 16 ? 1 : M <= 32 ? 2 : 4;
  p.BNT = (M > 64 && fmt != kFmtBF16) ? 2 : 1;
  p.TPC = mfma_tpc(fmt, p.BMS);
  p.NB = ps.NB;
  p.KT = ps.KT;
  p.NBB = ceil_div(p.NB, 4 * p.BNT);
  p.MB = ceil_div(M, 16 * p.BMS);
  p.chunks = ceil_div(p.KT, p.TPC);
  const int64_t wgs = p.NBB * p.MB;
  const int64_t target = 512;  // two workgroups per compute unit
  int64_t S = wgs >= target ? 1 : ceil_div(target, wgs);
  // every split keeps at least 4 chunks
  const int64_t max_s = p.chunks / 4 > 1 ? p.chunks / 4 : 1;
  if (S > max_s) S = max_s;
  if (S > 16) S = 16;
  p.chunks_per_split = ceil_div(p.chunks, S);
  S = ceil_div(p.chunks, p.chunks_per_split);
  p.S = int(S);
  p.ws_bytes = p.S > 1 ? size_t(p.S) * size_t(M) * size_t(N) * sizeof(float) : 0;
  *out = p;
  return kOK;
}

int choose_path(int fmt, int64_t M, int64_t N, int64_t K, Choice* out) {
  Choice c{};
  int st = plan_gemv(fmt, M, N, K, &c.gemv);
  if (st != kOK) return st;
  const int64_t bcast_first = fmt == kFmtW4 ? 1 : 4;
  const bool sk_ok = plan_skinny(fmt, M, N, K, &c.sk) == kOK;
  // up to 8 rows the skinny kernel pays off where its shares are long (its
  // start and, with a K split, the second launch are amortised), measured
  // on the 70B shapes: gate/up from 2 rows, down at 8
  const bool sk_long = sk_ok && c.sk.per_split >= 48 && (c.sk.S == 1 || M >= kGemvMaxM);
  // FP8 at 4 rows: the skinny kernel ahead of the broadcast one where its
  // shares are long (70B gate/up 82.7 -> 74.4 us; at 2 and 3 rows the
  // broadcast kernel is as fast or faster, measured on the same box)
  const bool sk_first = fmt == kFmtFP8 && M >= 4 && sk_long;
  if (!sk_first && M <= bcast_first && plan_bcast(fmt, M, N, K, &c.bcast) == kOK) {
    c.path = kPathBcast;
  } else if (M <= kGemvMaxM && sk_long) {
    c.path = kPathSkinny;
  } else if (M <= kGemvMaxM && plan_mc(fmt, M, N, K, &c.mc) == kOK) {
    c.path = kPathMc;
  } else if (M <= kGemvMaxM && plan_bcast(fmt, M, N, K, &c.bcast) == kOK) {
    c.path = kPathBcast;
  } else if (M <= kGemvMaxM) {
    c.path = kPathStaged;
  } else if (M <= kMcMaxM && N <= 8192 && K <= 8192 && sk_ok && c.sk.S > 1 &&
             plan_mc(fmt, M, N, K, &c.mc) == kOK) {
    // 9 to 16 rows on matrices up to 8192 x 8192 that the skinny kernel would
    // split: the streaming matrix-core kernel needs no second launch
    // (measured on 8192^2 and 4096^2: 10-35% faster for FP8 and W4A16)
    c.path = kPathMc;
  } else if (M <= kSkMaxM && sk_ok) {
    c.path = kPathSkinny;
  } else if (M > kGmMinM && ceil_div(N, int64_t(256)) >= kGmMinNBN && plan_gemm(fmt, M, N, K, &c.gm) == kOK) {
    c.path = c.gm.wm == 3 ? kPathGemmLds : kPathGemm;
  } else {
    st = plan_mfma(fmt, M, N, K, &c.mfma);
    if (st != kOK) return st;
    c.path = kPathMfma;
  }
  *out = c;
  return kOK;
}

int workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, size_t* out) {
  Choice c;
  int st = choose_path(fmt, M, N, K, &c);
  if (st != kOK) return st;
  *out = c.path == kPathMfma     ? c.mfma.ws_bytes
         : c.path == kPathSkinny ? c.sk.ws_bytes
         : c.path == kPathGemm || c.path == kPathGemmLds ? c.gm.ws_bytes
                                 : 0;
  return kOK;
}

// W8A8 LDS-staged form: from this many rows; per-chunk cost model and the
// relative chunk times of its tile shapes.
#ifndef WQD_W8_LDS_MIN_M
#define WQD_W8_LDS_MIN_M 256
#endif
constexpr int64_t kW8LdsMinM = WQD_W8_LDS_MIN_M;
static constexpr GlCost kW8Cost = {12.0, 1.53, 5.15};
#ifndef WQD_W8_FORCE_SHAPE
static constexpr GlShape kW8Shapes[] = {{8, 4, 1.0}, {7, 4, 0.95}, {7, 2, 0.93}};
#else
static constexpr GlShape kW8Shapes[] = {WQD_W8_FORCE_SHAPE};  // measurement builds only
#endif

int plan_w8a8(int64_t M, int64_t N, int64_t K, W8Plan* out) {
  PackedSizes ps;
  int st = packed_sizes(kFmtFP8, N, K, &ps);
  if (st != kOK) return st;
  if (M < 1) return kEArg;
  if (K % 16 != 0) return kEShape;  // activation codes move in 16-byte pieces
  if (M * K >= (int64_t(1) << 31) - 16) return kEUnsupported;
  W8Plan p{};
  p.NB = ps.NB;
  p.KT = ps.KT;
  if (M <= 32) {
    p.mf = 2, p.wr = 1;
  } else if (M <= 64) {
    p.mf = 4, p.wr = 1;
  } else {
    p.mf = 8, p.wr = 1;
  }
  p.nchunks = ceil_div(p.KT, 2);  // 128-k chunks
  if (M >= kW8LdsMinM && K % 128 == 0 && 32 * p.KT * kTileBytes < (int64_t(1) << 31)) {
    // the LDS-staged form: the tile shape and K split by the busiest XCD's
    // rounds (as for the weight-only FP8 LDS-staged kernel)
    const double mn8 = double(M) * double(N) * 8.0;
    const int64_t max_s = p.nchunks / 4 < 1 ? 1 : (p.nchunks / 4 > 8 ? 8 : p.nchunks / 4);
    double best = 0.0, fill = 0.0;
    bool first = true;
    for (const GlShape& sh : kW8Shapes) {
      const int64_t nbn = ceil_div(p.NB, int64_t(8 / sh.lwr * sh.rbw)), mb = ceil_div(M, int64_t(64 * sh.lwr));
      const int64_t per_xcd = ceil_div(nbn, int64_t(8)) * mb;
      for (int64_t s = 1; s <= max_s; ++s) {
        const int64_t cps = ceil_div(p.nchunks, s), se = ceil_div(p.nchunks, cps);
        const int64_t rounds = ceil_div(per_xcd * se, kComputeUnits / 8);
        const double t = kW8Cost.c0 + double(cps) * kW8Cost.a * sh.f * double(rounds) +
                         (se > 1 ? double(se) * mn8 / (kW8Cost.bw * 1.0e6) : 0.0);
        if (first || t < 0.98 * best) {
          best = t;
          first = false;
          p.rbw = sh.rbw;
          p.lwr = sh.lwr;
          p.NBN = nbn;
          p.MB = mb;
          p.cps = cps;
          p.S = int(se);
          fill = double(per_xcd * se) / double(rounds * (kComputeUnits / 8));
        }
      }
    }
    // where the rounds are not nearly full (e.g. the 70B gate at 768 rows:
    // 3/4), the 4-wavefront register-operand tiles measured faster
    if (fill >= 0.9) {
      p.lds = 1;
      p.ws_bytes = p.S > 1 ? size_t(p.S) * size_t(M) * size_t(N) * sizeof(float) : 0;
      *out = p;
      return kOK;
    }
    p.rbw = p.lwr = 0;
  }
  const int64_t bm = 16 * int64_t(p.mf) * p.wr;
  p.NBN = ceil_div(p.NB, 16);  // 256-column blocks
  p.MB = ceil_div(M, bm);
  // fill at least one round of the 256 compute units (two workgroups each
  // for the 4-wavefront tiles), each split at least 4 chunks, at most 8 splits
  const int64_t tiles = ceil_div(p.NBN, 8) * 8 * p.MB;
  const int64_t target = p.wr == 1 ? 512 : 256;
  int64_t S = tiles >= target ? 1 : ceil_div(target, tiles);
  const int64_t max_s = p.nchunks / 4 > 1 ? p.nchunks / 4 : 1;
  if (S > max_s) S = max_s;
  if (S > 8) S = 8;
  p.cps = ceil_div(p.nchunks, S);
  S = ceil_div(p.nchunks, p.cps);
  p.S = int(S);
  p.ws_bytes = p.S > 1 ? size_t(p.S) * size_t(M) * size_t(N) * sizeof(float) : 0;
  *out = p;
  return kOK;
}

int plan_act_quant(int64_t M, int64_t K, int* parts) {
  if (M < 1 || K < 1) return kEArg;
  if (K % 16 != 0) return kEShape;
  if (M * K >= (int64_t(1) << 40)) return kEUnsupported;
  // ranges of at least 32 KiB of x per part (8 loads in flight per thread)
  const int64_t n16 = M * K / 8;
  int64_t g = ceil_div(n16, 2048);
  if (g > kActQuantParts) g = kActQuantParts;
  *parts = int(g < 1 ? 1 : g);
  return kOK;
}

#ifndef WQD_ATTN_TARGET_GROUPS
#define WQD_ATTN_TARGET_GROUPS 256
#endif
constexpr int64_t kAttnTargetGroups = WQD_ATTN_TARGET_GROUPS;  // workgroups of 4 wavefronts per launch
constexpr int64_t kAttnWavesPerSplit = 4;

int plan_attn(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D, AttnPlan* out, bool fp8_kv) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Lmax < 1) return kEArg;
  if (D != 128 || Hq % Hkv != 0 || Hq / Hkv > 16 || Lmax % 32 != 0) return kEShape;
  if (Lmax * 128 * 2 >= (int64_t(1) << 31) || B > 65535 || Hkv > 65535 || Hq > 65535) return kEUnsupported;
  AttnPlan p{};
  p.Lmax = Lmax;
  p.Hq = int(Hq);
  p.Hkv = int(Hkv);
  // about one workgroup of 4 wavefronts per compute unit (long streams per
  // wavefront measured faster than more, shorter splits), each wavefront at
  // least 2 steps; a step is 32 positions of a bf16 cache, 64 of an FP8 one
  // (the same 16 KiB of keys and values)
  const int64_t step = fp8_kv ? 64 : 32;
  const int64_t pairs = B * Hkv;
  const int64_t steps = ceil_div(Lmax, step);
  int64_t S = ceil_div(kAttnTargetGroups, pairs);
  const int64_t max_s = steps / (2 * kAttnWavesPerSplit) > 1 ? steps / (2 * kAttnWavesPerSplit) : 1;
  if (S > max_s) S = max_s;
  p.chunk = int(step * ceil_div(steps, S));
  p.S = int(ceil_div(Lmax, p.chunk));
  p.fp8_kv = fp8_kv ? 1 : 0;
  p.ws_bytes = p.S > 1 ? size_t(B) * size_t(Hq) * size_t(p.S) * (2 + 128) * sizeof(float) : 0;
  *out = p;
  return kOK;
}

int plan_chain_call(int fmt, int64_t M, int64_t N, int64_t K, bool swiglu, ChainCall* out) {
  PackedSizes ps;
  int st = packed_sizes(fmt, N, K, &ps);
  if (st != kOK) return st;
  if (M < 1) return kEArg;
  if (M > kChainMaxM) return kEUnsupported;
  if (swiglu && N % 16 != 0) return kEShape;
  if (ps.NB >= (int64_t(1) << 31) || ceil_div(ps.KT, kChainWaves) > (int64_t(1) << 20)) return kEUnsupported;
  ChainCall c{};
  c.N = N;
  c.K = K;
  c.KT = ps.KT;
  c.G4 = fmt == kFmtW4 ? ps.G4 : 0;
  c.per_wave = int(ceil_div(ps.KT, 8 * int64_t(kChainWaves)) * 8);
  c.nb = int(ps.NB);
  c.ni = int(ceil_div(ps.NB, kChainRB));
  c.swiglu = swiglu ? 1 : 0;
  c.wait_for = -1;
  *out = c;
  return kOK;
}

size_t chain_workspace_bytes(int64_t ncalls) {
  return chain_counters_offset(ncalls) + size_t(ncalls) * kChainCounters * kChainCounterStride * sizeof(int);
}

}  // namespace wqd
