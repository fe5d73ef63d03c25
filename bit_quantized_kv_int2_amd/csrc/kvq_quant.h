// Device-side quantiser and cache addressing shared by the bulk pack and the
// append kernels (internal). The rule is the one kv_quantize_pack documents:
// min/max in fp32 (-0 below +0), s = fp16((max - min) / (2^b - 1)) with an
// IEEE fp32 division, z = fp16(min), code = clamp(rint((x - z) / s), 0, 2^b - 1) from
// the stored fp16 s and z, code 0 when s == 0.
#pragma once

#include "kvq_internal.h"

namespace kvq {
namespace {

struct Geo {
  int H, Lp, max_pages, paged;
  const int32_t* table;
  // index of the 64-token chunk holding token t of (b, h)
  __device__ long chunk(int b, int h, int t) const {
    if (!paged) return ((long)b * H + h) * (Lp / kPage) + t / kPage;
    return (long)table[(long)b * max_pages + t / kPage] * H + h;
  }
  // written extent of a sequence: whole padded length, or whole pages
  __device__ int extent(int L) const { return paged ? ((L + kPage - 1) / kPage) * kPage : Lp; }
};

__device__ inline uint16_t f16_bits(float x) {
  _Float16 h = (_Float16)x;  // v_cvt_f16_f32, round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ inline float f16_val(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }

// token-wise pair of token t, channel group j (ng groups per token)
__device__ inline long pair_token(const Geo& g, int b, int h, int t, int j, int ng) {
  return ((g.chunk(b, h, t) * kPage + t % kPage) * ng + j) * 2;
}
__device__ inline long pair_channel(const Geo& g, int b, int h, int t, int d) {
  if (!g.paged) return (((long)b * g.H + h) * (g.Lp / kGroup) + t / kGroup) * (long)kHeadDim * 2 + d * 2;
  int t0 = (t / kGroup) * kGroup;
  return (g.chunk(b, h, t0) * kHeadDim + d) * 2;
}

__device__ inline int encode(float x, float S, float Z, int qmax) {
  if (S == 0.0f) return 0;
  float diff = x - Z;
  float t = __fdiv_rn(diff, S);
  float r = rintf(t);
  r = fminf(fmaxf(r, 0.0f), (float)qmax);
  return (int)r;
}

}  // namespace
}  // namespace kvq
