// In-place gated-delta memory step for gfx950 (the recurrent memory stream).
//
// The ATMA technical summary (gist.science), section 2.2, performs the recurrent memory
// update in place, so states are never gathered into a batch and scattered back; section
// 2.1 L2-normalises the memory's keys and queries.  Rule (gated delta rule, one token):
//   k <- k/|k|, q <- q/|q|;   S' = alpha S (I - beta k k^T) + beta v k^T;   o = S' q
// rewritten as  u = beta (v - alpha S k),  S' = alpha S + u k^T,  o = alpha S q + u (k.q),
// so the 64 x 64 fp32 state is read once and written once where it lives in the pool.
//
// One workgroup per (sequence, head): thread t owns row i = t/4 of the state and the 16
// columns 16*(t%4)..+15, held in registers between the read and the write.  Row sums
// (S k, S q) and the dots (k.k, q.q, k.q) reduce over the 4 threads of a row with lane
// shuffles in a fixed order.
#include "polar_kernels.h"

namespace polar {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1);
  return x + __shfl_xor(x, 2);
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

template <class E>
__global__ void __launch_bounds__(256) polar_delta_step_kernel(DeltaArgs a) {
  constexpr int D = kHeadDim;
  const int b = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int t = threadIdx.x, i = t >> 2, c = t & 3;
  const size_t bh = (size_t)b * a.H + h;
  const int slot = a.slots[b];
  if (slot < 0 || slot >= a.num_slots) {               // skipped sequence: zero output
    if (c == 0) a.out[bh * D + i] = 0.f;
    return;
  }
  float *S = a.pool + ((size_t)slot * a.H + h) * D * D + i * D + 16 * c;
  float s[16], q[16], k[16];
  load16(S, s);
  load16((const E *)a.q + bh * D + 16 * c, q);
  load16((const E *)a.k + bh * D + 16 * c, k);
  const float v = load1((const E *)a.v + bh * D + i);
  const float alpha = a.alpha[bh], beta = a.beta[bh];

  float kk = 0.f, qq = 0.f, kq = 0.f, sk = 0.f, sq = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    kk = fmaf(k[j], k[j], kk);
    qq = fmaf(q[j], q[j], qq);
    kq = fmaf(k[j], q[j], kq);
    sk = fmaf(s[j], k[j], sk);
    sq = fmaf(s[j], q[j], sq);
  }
  kk = quad_sum(kk);
  qq = quad_sum(qq);
  kq = quad_sum(kq);
  sk = quad_sum(sk);
  sq = quad_sum(sq);
  const float rk = a.normalize ? 1.0f / sqrtf(kk + 1e-12f) : 1.0f;
  const float rq = a.normalize ? 1.0f / sqrtf(qq + 1e-12f) : 1.0f;
  const float u = beta * (v - alpha * sk * rk);
  const float uk = u * rk;
#pragma unroll
  for (int j = 0; j < 16; ++j) s[j] = fmaf(alpha, s[j], uk * k[j]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 w = {s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]};
    *(f32x4 *)(S + 4 * j) = w;
  }
  if (c == 0) a.out[bh * D + i] = alpha * sq * rq + u * (kq * rk * rq);
}

}  // namespace

hipError_t launch_delta_step(int dtype, const DeltaArgs &a, hipStream_t stream) {
  const long long blocks = (long long)a.B * a.H;
  if (blocks <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(polar_delta_step_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(polar_delta_step_kernel<float>, dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace polar
