// Device building blocks shared by the Polar Attention kernels on gfx950 (CDNA4):
// MFMA element traits for bf16 and fp32 inputs, wave-half exchanges, fast exp2.
//
// MFMA register layouts used throughout (wave64):
//  * 32x32 output (v_mfma_f32_32x32x16_bf16 / v_mfma_f32_32x32x2_f32): lane l holds
//    column l%32 and rows 8*(r/4) + 4*(l/32) + r%4 for its 16 accumulators r.
//  * 16x16 output (v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x4_f32): lane l holds
//    column l%16 and rows 4*(l/16) + r for its 4 accumulators r.
//  * A and B operands: lane l supplies KPL consecutive contraction slots of row (A) or
//    column (B) l%32 (resp. l%16) in slot group l/32 (resp. l/16).  The kernels only rely
//    on A and B using the same slot numbering, so any contraction order is correct.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace polar {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x from this lane and from lane l^32, combined in the same order in every lane.
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}
// The value lane l^32 holds (exact).
__device__ __forceinline__ float half_other(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0] == __float_as_int(x) ? r[1] : r[0]);
}
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

// Position of key k32 (0..31 inside a 32-key block) in a transposed V row: the kpl keys
// that one lane feeds to one P.V MFMA sit next to each other.  Lane group g of MFMA t
// supplies slots e = 0..kpl-1 for keys 8*(i/4) + 4*g + i%4 with i = t*kpl + e (the keys
// that the score MFMA left in that lane).  The same order serves any 32-long
// contraction whose B operand comes straight out of a 32x32 MFMA result.
template <int KPL>
__device__ __forceinline__ int vpos32(int k32) {
  const int a = k32 >> 3, gg = (k32 >> 2) & 1, cc = k32 & 3;
  const int i = 4 * a + cc;
  return (i / KPL) * (2 * KPL) + gg * KPL + (i % KPL);
}

// The four bf16 A-operand fragments of a 64-key tile stored as swizzled key rows in LDS,
// read transposed with ds_read_b64_tr_b16: fragment j (key block j/2, half j%2) is the pair
// of 8-byte reads at rows 16 j (from lane address lo) and 16 j + 8 (from hi; the two
// addresses differ where the swizzle of the row differs), row pitch 128 bytes.
// The reads are issued in one asm block that waits for them before it ends.  Through the
// builtin, the compiler cannot tell these reads from the tiles still being written by
// buffer_load ... lds and first waits for every load in flight, including the tile fetched
// ahead in the same step; the tile read here was published by an earlier barrier.
// (Outputs are early-clobber: none may take an address register while reads are pending.)
__device__ __forceinline__ void tr_read_tile(uint32_t lo, uint32_t hi, bf16x8 f[4]) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  s16x4 r0, r1, r2, r3, r4, r5, r6, r7;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:2048\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:2048\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:4096\n\t"
      "ds_read_b64_tr_b16 %5, %9 offset:4096\n\t"
      "ds_read_b64_tr_b16 %6, %8 offset:6144\n\t"
      "ds_read_b64_tr_b16 %7, %9 offset:6144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(lo), "v"(hi));
  f[0] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
  f[1] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r2, r3, 0, 1, 2, 3, 4, 5, 6, 7));
  f[2] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r4, r5, 0, 1, 2, 3, 4, 5, 6, 7));
  f[3] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r6, r7, 0, 1, 2, 3, 4, 5, 6, 7));
}
// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// bf16 inputs: 8 contraction slots per lane per MFMA, fp32 accumulation.
struct Bf16 {
  using elem_t = uint16_t;                 // storage (bit pattern)
  using frag_t = bf16x8;
  static constexpr int kpl = 8;
  static constexpr int vec = 8;            // elements per 16-byte global access

  __device__ static __forceinline__ f32x16 mma32(frag_t a, frag_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 mma16(frag_t a, frag_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag_t load(const elem_t *p) {
    return *reinterpret_cast<const frag_t *>(p);
  }
  __device__ static __forceinline__ frag_t zero() {
    u32x4 z = {0u, 0u, 0u, 0u};
    return __builtin_bit_cast(frag_t, z);
  }
  // Round kpl probabilities to bf16 (nearest-even) for the P.V product.
  __device__ static __forceinline__ frag_t pack(const float *x) {
    frag_t r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
    return r;
  }
  // S += sum p, Q += sum p^2 over the rounded probabilities (dot2 per pair).
  __device__ static __forceinline__ void stats(frag_t f, float &S, float &Q) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bf16x2 pr;
      pr[0] = f[2 * e];
      pr[1] = f[2 * e + 1];
      S = __builtin_amdgcn_fdot2_f32_bf16(pr, one, S, false);
      Q = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, Q, false);
    }
  }
};

// fp32 inputs: 1 contraction slot per lane per MFMA; probabilities stay fp32.
struct F32 {
  using elem_t = float;
  using frag_t = float;
  static constexpr int kpl = 1;
  static constexpr int vec = 4;

  __device__ static __forceinline__ f32x16 mma32(frag_t a, frag_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 mma16(frag_t a, frag_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag_t load(const elem_t *p) { return *p; }
  __device__ static __forceinline__ frag_t zero() { return 0.0f; }
  __device__ static __forceinline__ frag_t pack(const float *x) { return x[0]; }
  __device__ static __forceinline__ void stats(frag_t f, float &S, float &Q) {
    S += f;
    Q = fmaf(f, f, Q);
  }
};

}  // namespace polar
