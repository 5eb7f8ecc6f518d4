// Rotary position embedding helpers shared by the prefill and backward kernels (internal
// header).  RoFormer form: the pair of dimensions (2t, 2t+1) of the vector at position p
// turns by the angle p * theta^(-2t/d); f_t = theta^(-2t/d) / (2 pi) in 2^-64 units
// (PrefillArgs::rope_f).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "polar_mfma.h"

namespace polar {

// RoPE rotation angle of pair t at position pos: revolutions = frac(pos * f_t) taken
// exactly from the 64-bit fixed-point product, then the hardware sine and cosine, whose
// argument is in revolutions (the rotated values are rounded to bf16 afterwards, far
// coarser than their error).
__device__ __forceinline__ void rope_cs(uint64_t f, int pos, float &c, float &s) {
  const uint32_t hi = (uint32_t)(((uint64_t)(uint32_t)pos * f) >> 32);
  const float rev = (float)hi * 2.3283064365386963e-10f;
  s = __builtin_amdgcn_sinf(rev);
  c = __builtin_amdgcn_cosf(rev);
}

// Dims dim0 .. dim0 + 3 (dim0 even) of a gradient at position pos turned by the transposed
// rotation, the opposite angle: (g0, g1) -> (g0 c + g1 s, g1 c - g0 s).
__device__ __forceinline__ f32x4 unrotate4(f32x4 w, int dim0, int pos, const uint64_t *f) {
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    float c, sn;
    rope_cs(f[dim0 / 2 + m], pos, c, sn);
    const float g0 = w[2 * m], g1 = w[2 * m + 1];
    w[2 * m] = fmaf(g0, c, g1 * sn);
    w[2 * m + 1] = fmaf(g1, c, -(g0 * sn));
  }
  return w;
}

}  // namespace polar
