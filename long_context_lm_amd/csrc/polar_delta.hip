// In-place gated-delta memory step for gfx950 (the recurrent memory stream).
//
// The ATMA technical summary (gist.science), section 2.2, performs the recurrent memory
// update in place, so states are never gathered into a batch and scattered back; section
// 2.1 L2-normalises the memory's keys and queries.  Rule (gated delta rule, one token):
//   k <- k/|k|, q <- q/|q|;   S' = alpha S (I - beta k k^T) + beta v k^T;   o = S' q
// rewritten as  u = beta (v - alpha S k),  S' = alpha S + u k^T,  o = alpha S q + u (k.q),
// so the 64 x 64 fp32 state is read once and written once where it lives in the pool.
//
// A 256-thread workgroup updates one (sequence, head) state at a time, NS in a row: thread
// t owns row i = t/4 of the state and the 16 columns 16*(t%4)..+15, held in registers
// between the read and the write, and the next state is loaded while the current one is
// updated.  Row sums (S k, S q) and the dots (k.k, q.q, k.q) reduce over the 4 threads of
// a row with lane shuffles in a fixed order.
#include "polar_kernels.h"

namespace polar {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Sum over the 4 lanes of a quad with DPP quad permutes (lane order fixed: (x0+x1)+(x2+x3)
// in every lane).
__device__ __forceinline__ float quad_sum(float x) {
  const int xi = __float_as_int(x);
  x += __int_as_float(__builtin_amdgcn_update_dpp(xi, xi, 0xB1, 0xF, 0xF, false));   // 1,0,3,2
  const int yi = __float_as_int(x);
  return x + __int_as_float(__builtin_amdgcn_update_dpp(yi, yi, 0x4E, 0xF, 0xF, false));  // 2,3,0,1
}

// 16 consecutive elements as floats.
__device__ __forceinline__ void load16(const float *p, float *x) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 w = *(const f32x4 *)(p + 4 * j);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * j + e] = w[e];
  }
}
__device__ __forceinline__ void load16(const uint16_t *p, float *x) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const u32x4 w = *(const u32x4 *)(p + 8 * j);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * j + 2 * e] = __uint_as_float(w[e] << 16);
      x[8 * j + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
}
__device__ __forceinline__ float load1(const float *p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t *p) {
  return __uint_as_float((uint32_t)*p << 16);
}

// One (sequence, head) state at a time per workgroup, NS states per workgroup in a row: the
// next state's slot, state row and vectors are loaded while the current one is updated.
template <class E>
struct DeltaLoad {
  float s[16], q[16], k[16];
  float v, alpha, beta;
  int ok;
  float *S;
};

template <class E, int NS>
__global__ void __launch_bounds__(256) polar_delta_step_kernel(DeltaArgs a) {
  constexpr int D = kHeadDim;
  const int t = threadIdx.x, i = t >> 2, c = t & 3;
  const int units = a.B * a.H;
  auto load = [&](int unit, DeltaLoad<E> &L) {
    const int b = unit / a.H, h = unit % a.H;
    const size_t bh = (size_t)b * a.H + h;
    const int slot = a.slots[b];
    L.ok = slot >= 0 && slot < a.num_slots;
    L.S = a.pool + ((size_t)(L.ok ? slot : 0) * a.H + h) * D * D + i * D + 16 * c;
    if (L.ok) load16(L.S, L.s);
    load16((const E *)a.q + bh * D + 16 * c, L.q);
    load16((const E *)a.k + bh * D + 16 * c, L.k);
    L.v = load1((const E *)a.v + bh * D + i);
    L.alpha = a.alpha[bh];
    L.beta = a.beta[bh];
  };
  auto update = [&](int unit, DeltaLoad<E> &L) {
    const size_t bh = (size_t)unit;                      // unit = b * H + h
    if (!L.ok) {                                         // skipped sequence: zero output
      if (c == 0) a.out[bh * D + i] = 0.f;
      return;
    }
    float kk = 0.f, qq = 0.f, kq = 0.f, sk = 0.f, sq = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      kk = fmaf(L.k[j], L.k[j], kk);
      qq = fmaf(L.q[j], L.q[j], qq);
      kq = fmaf(L.k[j], L.q[j], kq);
      sk = fmaf(L.s[j], L.k[j], sk);
      sq = fmaf(L.s[j], L.q[j], sq);
    }
    kk = quad_sum(kk);
    qq = quad_sum(qq);
    kq = quad_sum(kq);
    sk = quad_sum(sk);
    sq = quad_sum(sq);
    const float rk = a.normalize ? rsqrtf(kk + 1e-12f) : 1.0f;
    const float rq = a.normalize ? rsqrtf(qq + 1e-12f) : 1.0f;
    const float u = L.beta * (L.v - L.alpha * sk * rk);
    const float uk = u * rk;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 w = {fmaf(L.alpha, L.s[4 * j], uk * L.k[4 * j]),
                       fmaf(L.alpha, L.s[4 * j + 1], uk * L.k[4 * j + 1]),
                       fmaf(L.alpha, L.s[4 * j + 2], uk * L.k[4 * j + 2]),
                       fmaf(L.alpha, L.s[4 * j + 3], uk * L.k[4 * j + 3])};
      *(f32x4 *)(L.S + 4 * j) = w;
    }
    if (c == 0) a.out[bh * D + i] = L.alpha * sq * rq + u * (kq * rk * rq);
  };
  const int u0 = blockIdx.x * NS;
  DeltaLoad<E> L[2];
  if (u0 < units) load(u0, L[0]);
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    const int u = u0 + n;
    if (u >= units) break;
    if (n + 1 < NS && u + 1 < units) load(u + 1, L[(n + 1) & 1]);
    update(u, L[n & 1]);
  }
}

}  // namespace

#ifndef POLAR_DELTA_NS
#define POLAR_DELTA_NS 4
#endif

hipError_t launch_delta_step(int dtype, const DeltaArgs &a, hipStream_t stream) {
  constexpr int NS = POLAR_DELTA_NS;
  const long long units = (long long)a.B * a.H;
  if (units <= 0) return hipSuccess;
  const dim3 grid((unsigned)((units + NS - 1) / NS));
  if (dtype == 1)
    hipLaunchKernelGGL((polar_delta_step_kernel<uint16_t, NS>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((polar_delta_step_kernel<float, NS>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace polar
