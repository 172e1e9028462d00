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

int workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, size_t* out) {
  GemvPlan g;
  int st = plan_gemv(fmt, M, N, K, &g);
  if (st != kOK) return st;
  *out = 0;
  return kOK;
}

}  // namespace wqd
