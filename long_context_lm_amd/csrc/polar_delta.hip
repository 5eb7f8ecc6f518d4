// In-place gated-delta memory step for gfx950 (the recurrent memory stream).
//
// The ATMA technical summary (gist.science), section 2.2, performs the recurrent memory
// update in place, so states are never gathered into a batch and scattered back; section
// 2.1 L2-normalises the memory's keys and queries.  Rule (gated delta rule, one token):
//   k <- k/|k|, q <- q/|q|;   S' = alpha S (I - beta k k^T) + beta v k^T;   o = S' q
// rewritten as  u = beta (v - alpha S k),  S' = alpha S + u k^T,  o = alpha S q + u (k.q),
// so the 64 x 64 fp32 state is read once and written once where it lives in the pool.
//
// A 256-thread workgroup updates one (sequence, head) state at a time, NS in a row, and
// loads the next state while the current one is updated.  The state is read as 1024
// 16-byte chunks in address order, chunk 256 j + t to thread t, so each load instruction
// of a wave covers one contiguous kilobyte: thread t holds columns 4 (t%16)..+3 of rows
// 16 j + t/16 (j = 0..3), in registers between the read and the write.  A row then lives
// in one 16-lane DPP row, and the row sums (S k, S q) and the dots (k.k, q.q, k.q) reduce
// over those 16 lanes in a fixed order that leaves the same value in all of them.
#include "polar_kernels.h"

namespace polar {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Sum over the 16 lanes of a DPP row: quad butterflies, then the half-row and row mirrors.
// Every lane computes ((x0+x1)+(x2+x3)) + ... in the same pairing, so all 16 lanes hold
// the same bits.
template <int kCtrl>
__device__ __forceinline__ float dpp_sum_step(float x) {
  const int xi = __float_as_int(x);
  return x + __int_as_float(__builtin_amdgcn_update_dpp(xi, xi, kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x = dpp_sum_step<0xB1>(x);    // quad_perm 1,0,3,2
  x = dpp_sum_step<0x4E>(x);    // quad_perm 2,3,0,1
  x = dpp_sum_step<0x141>(x);   // row_half_mirror: quads 0<->1, 2<->3
  return dpp_sum_step<0x140>(x);  // row_mirror: halves 0<->1
}

// 4 consecutive elements as floats.
__device__ __forceinline__ void load4(const float *p, float *x) {
  const f32x4 w = *(const f32x4 *)p;
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = w[e];
}
__device__ __forceinline__ void load4(const uint16_t *p, float *x) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 w = *(const u32x2 *)p;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    x[2 * e] = __uint_as_float(w[e] << 16);
    x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
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
  f32x4 s[4];          // rows 16 j + t/16, columns 4 (t%16)..+3
  float q[4], k[4], v[4];
  float alpha, beta;
  int ok;
  float *S;
};

template <class E, int NS>
__global__ void __launch_bounds__(256) polar_delta_step_kernel(DeltaArgs a) {
  constexpr int D = kHeadDim;
  const int t = threadIdx.x, r0 = t >> 4, c0 = 4 * (t & 15);
  const int units = a.B * a.H;
  auto load = [&](int unit, DeltaLoad<E> &L) {
    const int b = unit / a.H, h = unit % a.H;
    const size_t bh = (size_t)b * a.H + h;
    const int slot = a.slots[b];
    L.ok = slot >= 0 && slot < a.num_slots;
    L.S = a.pool + ((size_t)(L.ok ? slot : 0) * a.H + h) * D * D + 4 * t;
    if (L.ok) {
#pragma unroll
      for (int j = 0; j < 4; ++j) L.s[j] = *(const f32x4 *)(L.S + 1024 * j);
    }
    load4((const E *)a.q + bh * D + c0, L.q);
    load4((const E *)a.k + bh * D + c0, L.k);
#pragma unroll
    for (int j = 0; j < 4; ++j) L.v[j] = load1((const E *)a.v + bh * D + 16 * j + r0);
    L.alpha = a.alpha[bh];
    L.beta = a.beta[bh];
  };
  auto update = [&](int unit, DeltaLoad<E> &L) {
    const size_t bh = (size_t)unit;                      // unit = b * H + h
    const bool writer = (t & 15) == 0;
    if (!L.ok) {                                         // skipped sequence: zero output
      if (writer) {
#pragma unroll
        for (int j = 0; j < 4; ++j) a.out[bh * D + 16 * j + r0] = 0.f;
      }
      return;
    }
    float kk = 0.f, qq = 0.f, kq = 0.f, sk[4], sq[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kk = fmaf(L.k[e], L.k[e], kk);
      qq = fmaf(L.q[e], L.q[e], qq);
      kq = fmaf(L.k[e], L.q[e], kq);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sk[j] = 0.f;
      sq[j] = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sk[j] = fmaf(L.s[j][e], L.k[e], sk[j]);
        sq[j] = fmaf(L.s[j][e], L.q[e], sq[j]);
      }
      sk[j] = row16_sum(sk[j]);
      sq[j] = row16_sum(sq[j]);
    }
    kk = row16_sum(kk);
    qq = row16_sum(qq);
    kq = row16_sum(kq);
    const float rk = a.normalize ? rsqrtf(kk + 1e-12f) : 1.0f;
    const float rq = a.normalize ? rsqrtf(qq + 1e-12f) : 1.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float u = L.beta * (L.v[j] - L.alpha * sk[j] * rk);
      const float uk = u * rk;
      f32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = fmaf(L.alpha, L.s[j][e], uk * L.k[e]);
      *(f32x4 *)(L.S + 1024 * j) = w;
      if (writer) a.out[bh * D + 16 * j + r0] = L.alpha * sq[j] * rq + u * (kq * rk * rq);
    }
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

hipError_t launch_delta_step(int dtype, const DeltaArgs &a, hipStream_t stream) {
  constexpr int NS = 4;   // states per workgroup
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
