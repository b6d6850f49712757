// Device side of the counter-based dropout mask (struct Drop in kernels.h).
#pragma once
#include "common.h"
#include "kernels.h"

namespace mtb {

// the four words of counter group g (elements 4g .. 4g+3)
MTB_DEV u32x4 drop_words(const Drop& d, uint64_t g) {
  return philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), d.site, d.offset, d.k0, d.k1);
}

MTB_DEV float drop_keep(const Drop& d, uint32_t w) { return w >= d.thr ? d.scale : 0.0f; }

// multiplier (0 or 1 / (1 - p)) of flat element i
MTB_DEV float drop_mul(const Drop& d, uint64_t i) {
  const u32x4 w = drop_words(d, i >> 2);
  const uint32_t j = (uint32_t)i & 3u;
  const uint32_t r = j == 0 ? w[0] : j == 1 ? w[1] : j == 2 ? w[2] : w[3];
  return drop_keep(d, r);
}

// multipliers of the 4 elements 4g .. 4g+3
MTB_DEV void drop_mul4(const Drop& d, uint64_t g, float (&m)[4]) {
  const u32x4 w = drop_words(d, g);
  m[0] = drop_keep(d, w[0]);
  m[1] = drop_keep(d, w[1]);
  m[2] = drop_keep(d, w[2]);
  m[3] = drop_keep(d, w[3]);
}

// v[e] *= multiplier of element i + e, e < 8 (i % 4 == 0)
MTB_DEV void drop_apply8(const Drop& d, uint64_t i, float (&v)[8]) {
  float m[4];
  drop_mul4(d, i >> 2, m);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] *= m[e];
  drop_mul4(d, (i >> 2) + 1, m);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[4 + e] *= m[e];
}

}  // namespace mtb
