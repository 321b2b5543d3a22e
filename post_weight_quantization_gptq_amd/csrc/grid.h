// The asymmetric min-max grid of the sweep, shared with the export kernels.
#pragma once
#include "common.h"

struct Grid {
  float s, r, z;
};

// Asymmetric min-max grid over values with minimum mn and maximum mx; every
// step in fp32 exactly as specified (0 always inside the range).
__device__ __forceinline__ Grid grid_from(float mn, float mx, float maxq) {
  const float lo = fminf(mn, 0.f), hi = fmaxf(mx, 0.f);
  Grid g;
  if (hi == lo) {
    g.s = 1.f;
    g.r = 1.f;
    g.z = 0.f;
    return g;
  }
  g.s = (hi - lo) / maxq;
  g.r = 1.f / g.s;
  const float zr = __fadd_rn(__fmul_rn(-lo, g.r), 0.f);
  g.z = fminf(fmaxf(rintf(zr), 0.f), maxq);
  return g;
}

