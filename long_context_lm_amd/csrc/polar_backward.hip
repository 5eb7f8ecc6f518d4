// Backward pass of the causal Polar Attention prefill for gfx950 (bf16 inputs, fp32
// gradients).
//
// The forward is section 2.1 of the ATMA technical summary (gist.science), "Polar
// Attention: A Three-Channel Decomposition", as fused in section 2.2.  Differentiating it
// row by row (row i of head h, c = beta_h * tau(i+1), l_j = c <q_i, k_j>, p = softmax(l)):
//   du    = (I - dir dir^T) d_dir / |u| + d_attn             (dir = u/|u|)
//   th    = tanh(ln n_eff) = (n^2-1)/(n^2+1);  gc = d_count . w_h
//   dgate = d_gate + gc th;  dn = d_n_eff + gc gate 4n/(n^2+1)^2
//   dm    = dgate gate (1-gate)                              (gate = sigmoid(m - floor))
//   A     = d_lse + 2 n dn - u . du;   E = -2 n^2 dn         (n_eff = 1/sum p^2)
//   dl_j  = p_j (v_j . du + A + E p_j) + [j = j*] dm         (j* = first arg-max key)
//   dq_i  = c sum_j dl_j k_j;  dk_j = sum_i c dl_ij q_i;  dv_j = sum_i p_ij du_i
//   dbeta = sum_i [tau (q_i . sum_j dl_ij k_j) - dm (tau/sqrt(d)) sqrt(2 ln n)],
//   dnull_bias = -sum_i dm,   dcount_vec = sum_i d_count_i gate th.
// d_attn is the cotangent of the plain softmax read-out u = sum_j p_j v_j (the softmax
// arm).  u . du = u . d_attn in exact arithmetic (the direction part is orthogonal to u);
// the prep kernel takes it of the rounded du the other kernels read.  p is recomputed
// from the saved log-sum-exp, so no T x T quantity is stored.
//
// Kernels, in launch order:
//  1. prep:  one 16-lane group per row: du (bf16) and the row scalars.
//  2. dq:    one wave per 32 rows of a head (lane = query, as in the forward): per 64-key
//            tile S^T = K Q^T and dP^T = V du^T on MFMA, dl on the VALU, then
//            dq^T += K^T dl^T with K^T from a transposed LDS tile.
//  3. dk/dv: one wave per 32 keys (lane = key), keys and values resident in registers;
//            a workgroup owns two key blocks (i and its mirror, for causal balance) and
//            walks, from the last one down, every query tile of the G heads sharing the KV
//            head that can see their keys.  S' = Q K^T and dP' = du V^T on MFMA (the row's
//            c applied on the VALU), then dv^T += du^T P and dk^T += Q^T dS with du^T and
//            Q^T from transposed tiles.
//            Each key has one owner, so dk and dv need no atomics.
//  4. parameter gradients: fixed-order two-level reductions over rows.
#include <type_traits>

#include "polar_kernels.h"
#include "polar_mfma.h"
#include "polar_rope.h"

namespace polar {
namespace {

constexpr int kD = kHeadDim;
constexpr int kBufferFlags = 0x00020000;   // gfx9 buffer resource word 3 (raw dword access)
constexpr int kDqWaves = 8;
constexpr int kDkvWaves = 4;
constexpr int kDkvDepth = 1;      // query tiles in flight ahead of the compute
constexpr int kDkvSplitMax = 2;   // workgroups sharing one key block (by heads)
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
using F = bf16x8;

// Keys row i sees: i + 1, or min(i + 1, W) under a sliding window W.
__device__ __forceinline__ int keys_seen(int row, int window) {
  return window > 0 ? min(row + 1, window) : row + 1;
}

__device__ __forceinline__ float tau_of(int n, float inv_log_train) {
  return inv_log_train > 0.f ? fmaxf(1.0f, logf((float)n) * inv_log_train) : 1.0f;
}

__device__ __forceinline__ const uint16_t *lds_at(const uint16_t *base, uint32_t off) {
  asm volatile("" : "+v"(off));
  return reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(base) + off);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Interleave two rows' 4 bf16 values (two dwords each) into 4 dwords: dword e holds
// element e of the first row in its low half and of the second row in its high half.
__device__ __forceinline__ uint32_t pair_word(u32x2 w0, u32x2 w1, int e) {
  return (e & 1) ? ((w0[e >> 1] >> 16) | (w1[e >> 1] & 0xFFFF0000u))
                 : ((w0[e >> 1] & 0xFFFFu) | (w1[e >> 1] << 16));
}

// Gradient rows leave as whole 256-byte rows with non-temporal stores: a wave stages its
// 32 rows (held in the 32x32 MFMA accumulator layout: lane l has row l % 32, dims
// 32 db + 8 j4 + 4 (l / 32) + e in register 4 j4 + e of block db) in a wave-private LDS
// area of 32 x kRowPitch floats, then stores four whole rows per instruction.  Whole lines
// bypass the L2, so the launch does not end on a write-back of its outputs.
constexpr int kRowPitch = kD + 4;
__device__ __forceinline__ void stage_rows(float *st, const f32x16 (&acc)[2], float scale,
                                           int lane) {
  float *row = st + (lane & 31) * kRowPitch + 4 * (lane >> 5);
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[db][4 * j4 + e] * scale;
      *(f32x4 *)(row + db * 32 + 8 * j4) = v;
    }
}
// row_ptr(r): destination of row r (0..31) or NULL to skip it; fix(v, r, dim0): the four
// values of row r from dim0 on, as stored.
template <class RowPtr, class Fix>
__device__ __forceinline__ void store_rows(const float *st, int lane, RowPtr row_ptr, Fix fix) {
  const int cc = (lane & 15) * 4;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (lane >> 4);
    float *dst = row_ptr(r);
    if (dst)
      __builtin_nontemporal_store(fix(*(const f32x4 *)(st + r * kRowPitch + cc), r, cc),
                                  (f32x4 *)(dst + cc));
  }
}

// ------------------------------------------------------------------ 1. per-row prep
__global__ void __launch_bounds__(256) polar_bwd_prep_kernel(BwdArgs a) {
  const int tid = threadIdx.x, l16 = tid & 15;
  const long long nrows = (long long)a.B * a.T * a.Hq;
  const long long R = (long long)blockIdx.x * 16 + (tid >> 4);
  const bool ok = R < nrows;
  const long long Rc = ok ? R : nrows - 1;
  const int h = (int)(Rc % a.Hq);
  const int i = (int)((Rc / a.Hq) % a.T);
  const size_t e0 = (size_t)Rc * kD + 4 * l16;
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  const f32x4 dir = *(const f32x4 *)(a.dir + e0);
  const f32x4 cd = a.c_dir ? *(const f32x4 *)(a.c_dir + e0) : z4;
  const f32x4 cc = a.c_count ? *(const f32x4 *)(a.c_count + e0) : z4;
  const f32x4 w = a.c_count ? *(const f32x4 *)(a.count_vec + (size_t)h * kD + 4 * l16) : z4;
  const f32x4 ca = a.c_attn ? *(const f32x4 *)(a.c_attn + e0) : z4;
  float dd = 0.f, gc = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    dd = fmaf(dir[c], cd[c], dd);
    gc = fmaf(cc[c], w[c], gc);
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    dd += __shfl_xor(dd, m);
    gc += __shfl_xor(gc, m);
  }
  const float U = a.u_norm[Rc], n = a.n_eff[Rc], gate = a.gate[Rc], lse = a.lse[Rc];
  const float inv = U > 0.f ? 1.0f / U : 0.f;
  const float beta = a.beta ? a.beta[h] : 8.0f;
  const int nk = keys_seen(i, a.window);
  const float tau = tau_of(nk, a.inv_log_train);
  const float c = beta * tau;
  // du as the MFMA kernels read it (bf16), and u . du of that rounded value: the row
  // constant -u . du then cancels the value term's sum over keys exactly as it does in
  // exact arithmetic (where it is -u . d_u, the direction part being orthogonal to u),
  // instead of leaving the rounding of du times the mean logit and key.
  bf16x4 o1;
  float ud = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float du = (cd[k] - dir[k] * dd) * inv + ca[k];
    o1[k] = (__bf16)du;
    ud = fmaf(dir[k], (float)o1[k], ud);
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) ud += __shfl_xor(ud, m);
  const float n2 = n * n;
  const float th = (n2 - 1.f) / (n2 + 1.f);
  const float dth_dn = 4.f * n / ((n2 + 1.f) * (n2 + 1.f));
  const float dgate = (a.c_gate ? a.c_gate[Rc] : 0.f) + gc * th;
  const float dn = (a.c_n_eff ? a.c_n_eff[Rc] : 0.f) + gc * gate * dth_dn;
  const float dm = dgate * gate * (1.f - gate);
  const float A = (a.c_lse ? a.c_lse[Rc] : 0.f) + 2.f * n * dn - U * ud;
  const float E = -2.f * n2 * dn;
  if (!ok) return;
  *(bf16x4 *)(a.du + e0) = o1;
  if (l16 == 0) {
    const f32x4 r0 = {c * kLog2e, lse * kLog2e, c * A, c * E};
    const f32x4 r1 = {A, E, dm, __int_as_float(a.arg_max[Rc])};
    const float fl =
        a.null_floor ? -dm * tau * 0.125f * sqrtf(2.f * logf((float)nk)) : 0.f;
    const f32x4 rp = {0.f, -dm, gate * th, fl};
    *(f32x4 *)(a.rows + 8 * Rc) = r0;
    *(f32x4 *)(a.rows + 8 * Rc + 4) = r1;
    *(f32x4 *)(a.rp + 4 * Rc) = rp;
  }
}

// ------------------------------------------------------------------ 2. dq
// kWin: the sliding-window instance (the causal one keeps the code it had without it).
template <int kWaves, bool kWin>
__global__ void __launch_bounds__(64 * kWaves) polar_bwd_dq_kernel(BwdArgs a) {
  constexpr int kThreads = 64 * kWaves;
  constexpr int KT = 64, KROW = 72, TROW = 72;
  constexpr int NTASK = 512;                        // 16-byte chunks (or pair tasks) per tile
  constexpr int NPER = (NTASK + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][KT * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[2][kD * TROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g32 = lane >> 5, c32 = lane & 31;
  const int n_hc = a.G / a.hb;
  const int NY = a.Hkv * n_hc;
  int id = blockIdx.x;
  const int b = id % a.B;
  id /= a.B;
  const int y = id % NY;
  const int rb = a.n_row_blocks - 1 - id / NY;
  const int g = y / n_hc, hc = y % n_hc;
  const int h = g * a.G + hc * a.hb + (wave % a.hb);
  const int WR = (kWaves / a.hb) * 32;
  const int row0 = rb * WR;
  const int wrow0 = row0 + (wave / a.hb) * 32;
  const int wg_last = min(row0 + WR, a.T) - 1;
  const int w_last = wrow0 < a.T ? min(wrow0 + 32, a.T) - 1 : -1;
  const int ntiles = wg_last / KT + 1;
  const int row = wrow0 + c32;
  const bool valid = row < a.T;

  const size_t row_bytes = (size_t)a.Hkv * kD * 2;
  const size_t kv_base = ((size_t)b * a.T * a.Hkv + g) * kD;
  const int kv_bytes = (int)(((size_t)a.T * a.Hkv - g) * kD * 2);
  const auto krsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const uint16_t *)a.k + kv_base), 0, kv_bytes, kBufferFlags);
  const auto vrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const uint16_t *)a.v + kv_base), 0, kv_bytes, kBufferFlags);

  // Row scalars; rows past T get p = 0 (lse2 = +inf) and zero coefficients.
  const size_t rr = ((size_t)b * a.T + (valid ? row : 0)) * a.Hq + h;
  float cl2 = 1.f, lse2 = INFINITY, A = 0.f, E = 0.f, dm = 0.f;
  int js = 0;
  if (valid) {
    const f32x4 r0 = *(const f32x4 *)(a.rows + 8 * rr);
    const f32x4 r1 = *(const f32x4 *)(a.rows + 8 * rr + 4);
    cl2 = r0[0];
    lse2 = r0[1];
    A = r1[0];
    E = r1[1];
    dm = r1[2];
    js = min(max(__float_as_int(r1[3]), 0), a.T - 1);   // memory-safe on a corrupt table
  }
  // Q and du fragments: B operands of S^T = K Q^T and dP^T = V du^T.
  F qf[4], df[4];
  {
    const uint16_t *qp = (const uint16_t *)a.q + rr * kD + g32 * 8;
    const uint16_t *dp = a.du + rr * kD + g32 * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qf[ks] = valid ? *(const F *)(qp + ks * 16) : Bf16::zero();
      df[ks] = valid ? *(const F *)(dp + ks * 16) : Bf16::zero();
    }
  }
  f32x16 o[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

  // Staging: K and V rows as 16-byte chunks; K^T from 2-key x 4-dim tasks whose pairs of
  // keys land in one LDS word of the transposed tile.
  u32x4 kst[NPER], vst[NPER];
  u32x2 tst[NPER][2];
  auto stage_load = [&](int t) {
    const int key0 = t * KT;
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      const int ch = min(tid + kThreads * j, NTASK - 1);
      const int key = ch >> 3, part = ch & 7;
      const int off = (int)((size_t)(key0 + key) * row_bytes) + part * 16;
      kst[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krsrc, off, 0, 0));
      vst[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrsrc, off, 0, 0));
      const int kp = ch & 31, dg = ch >> 5;
#pragma unroll
      for (int r = 0; r < 2; ++r)
        tst[j][r] = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                       krsrc, (int)((size_t)(key0 + 2 * kp + r) * row_bytes) + dg * 8, 0, 0));
    }
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      const int ch = tid + kThreads * j;
      if (NPER * kThreads != NTASK && ch >= NTASK) continue;
      const int key = ch >> 3, part = ch & 7;
      *(u32x4 *)&Ks[buf][key * KROW + part * 8] = kst[j];
      *(u32x4 *)&Vs[buf][key * KROW + part * 8] = vst[j];
      const int kp = ch & 31, dg = ch >> 5;
      const int pos = ((2 * kp) >> 5) * 32 + vpos32<8>((2 * kp) & 31);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *(uint32_t *)&Kt[buf][(dg * 4 + e) * TROW + pos] = pair_word(tst[j][0], tst[j][1], e);
    }
  };

  const uint32_t k_lane = (uint32_t)((c32 * KROW + g32 * 8) * 2);
  const uint32_t t_lane = (uint32_t)((c32 * TROW + g32 * 8) * 2);
  constexpr uint32_t KBUF = KT * KROW * 2, TBUF = kD * TROW * 2;

  // Under a sliding window the first tile is the one holding the workgroup's first
  // visible key, and a wave skips the tiles wholly before its own first one.
  const int W = kWin ? a.window : 0;
  const int t_first = W > 0 ? max(0, row0 - W + 1) / KT : 0;
  const int w_first = W > 0 ? wrow0 - W + 1 : 0;
  stage_load(t_first);
  stage_store(0);
  __syncthreads();
  for (int t = t_first; t < ntiles; ++t) {
    const int buf = (t - t_first) & 1;
    const bool more = t + 1 < ntiles;
    if (more) stage_load(t + 1);
    const int key0 = t * KT;
    if (key0 <= w_last && key0 + KT - 1 >= w_first) {
      const uint16_t *Kb = lds_at(&Ks[0][0], k_lane + buf * KBUF);
      const uint16_t *Vb = lds_at(&Vs[0][0], k_lane + buf * KBUF);
      const f32x16 zero = {};
      f32x16 S[2], P[2];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const F ka = *(const F *)(Kb + kb * 32 * KROW + ks * 16);
          S[kb] = Bf16::mma32(ka, qf[ks], ks == 0 ? zero : S[kb]);
          const F va = *(const F *)(Vb + kb * 32 * KROW + ks * 16);
          P[kb] = Bf16::mma32(va, df[ks], ks == 0 ? zero : P[kb]);
        }
      // Tiles wholly below the wave's first row need no mask; the branch is per wave, so
      // the mask's compares and selects stay out of the other tiles' code.
      F dl[2][2];
      auto dlogits = [&](auto masked) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          float x[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float s = S[kb][r];
            if constexpr (decltype(masked)::value) {
              const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * g32 + (r & 3);
              if (key > row || (W > 0 && key <= row - W)) s = -INFINITY;
            }
            const float p = fast_exp2(fmaf(s, cl2, -lse2));
            x[r] = p * (P[kb][r] + fmaf(E, p, A));
          }
          dl[kb][0] = Bf16::pack(x);
          dl[kb][1] = Bf16::pack(x + 8);
        }
      };
      if (key0 + KT - 1 > wrow0 || (W > 0 && key0 <= wrow0 + 31 - W))
        dlogits(std::true_type{});
      else
        dlogits(std::false_type{});
      const uint16_t *Tb = lds_at(&Kt[0][0], t_lane + buf * TBUF);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            const F ta = *(const F *)(Tb + db * 32 * TROW + kb * 32 + tt * 16);
            o[db] = Bf16::mma32(ta, dl[kb][tt], o[db]);
          }
    }
    if (more) stage_store(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: the arg-max key's share of dl, the dbeta row term, dq = c * sum dl k.
  if (valid && dm != 0.f) {
    const uint16_t *kr = (const uint16_t *)a.k + (((size_t)b * a.T + js) * a.Hkv + g) * kD;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const u32x2 w = *(const u32x2 *)(kr + db * 32 + 8 * j4 + 4 * g32);
        o[db][4 * j4 + 0] = fmaf(dm, bf16_lo(w[0]), o[db][4 * j4 + 0]);
        o[db][4 * j4 + 1] = fmaf(dm, bf16_hi(w[0]), o[db][4 * j4 + 1]);
        o[db][4 * j4 + 2] = fmaf(dm, bf16_lo(w[1]), o[db][4 * j4 + 2]);
        o[db][4 * j4 + 3] = fmaf(dm, bf16_hi(w[1]), o[db][4 * j4 + 3]);
      }
  }
  const float tau = tau_of(keys_seen(valid ? row : 0, a.window), a.inv_log_train);
  if (a.d_beta) {
    float qd = 0.f;
    if (valid) {
      const uint16_t *qr = (const uint16_t *)a.q + rr * kD;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const u32x2 w = *(const u32x2 *)(qr + db * 32 + 8 * j4 + 4 * g32);
          qd = fmaf(bf16_lo(w[0]), o[db][4 * j4 + 0], qd);
          qd = fmaf(bf16_hi(w[0]), o[db][4 * j4 + 1], qd);
          qd = fmaf(bf16_lo(w[1]), o[db][4 * j4 + 2], qd);
          qd = fmaf(bf16_hi(w[1]), o[db][4 * j4 + 3], qd);
        }
    }
    qd = half_sum(qd);
    if (valid && g32 == 0) a.rp[4 * rr] = tau * qd;
  }
  // dq = c o, through the wave's staging area (the tile buffers are free after the loop's
  // last barrier; every staged load went through registers).
  __shared__ __attribute__((aligned(16))) float Ost[kWaves][32 * kRowPitch];
  stage_rows(Ost[wave], o, (a.beta ? a.beta[h] : 8.0f) * tau, lane);
  __syncthreads();
  // Under RoPE, dq with respect to the unrotated q: each row turned back at its position.
  store_rows(
      Ost[wave], lane,
      [&](int r) -> float * {
        const int qrow = wrow0 + r;
        return qrow < a.T ? a.dq + (((size_t)b * a.T + qrow) * a.Hq + h) * kD : nullptr;
      },
      [&](f32x4 v, int r, int dim0) {
        return a.rope ? unrotate4(v, dim0, wrow0 + r, a.rope_f) : v;
      });
}

// ------------------------------------------------------------------ 3. dk / dv
// kRope: the instance that turns dk back by the transposed rotation (its own instance, so
// that the others keep their registers).
template <int kWaves, int kDepth, bool kWin, bool kRope>
__global__ void __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
polar_bwd_dkv_kernel(BwdArgs a) {
  constexpr int kThreads = 64 * kWaves;
  static_assert(kThreads == 256, "one staging task per thread");
  constexpr int KB = 32 * kWaves;                   // keys per key block
  constexpr int QROW = 72, TROW = 40;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][32 * QROW];   // q rows
  __shared__ __attribute__((aligned(16))) uint16_t Cs[2][32 * QROW];   // du rows
  __shared__ __attribute__((aligned(16))) uint16_t Qt[2][kD * TROW];   // q^T
  __shared__ __attribute__((aligned(16))) uint16_t Dt[2][kD * TROW];   // du^T
  // Row scalars: cl2, lse2, c*A, c*E, dm, arg-max key (bits).
  __shared__ __attribute__((aligned(16))) float Sc[2][6][32];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g32 = lane >> 5, c32 = lane & 31;
  // Causal balance: a workgroup owns key blocks i and nkb-1-i, whose query-tile counts
  // add up to the same total for every i.  Workgroups are dealt to the 8 XCDs
  // round-robin by block index; each XCD gets a contiguous range of (sequence, KV head,
  // pair) units, pair fastest, so the workgroups of one (sequence, KV head) share an L2
  // and, all walking the query tiles top-down, read each tile at about the same time.
  const int nblk = gridDim.x;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int unit = xcd * (nblk >> 3) + min(xcd, nblk & 7) + local;
  const int npair = (a.n_key_blocks + 1) >> 1;
  const int pair = (unit % (npair * a.hsplit)) / a.hsplit;
  const int hpart = unit % a.hsplit;
  const int bg = unit / (npair * a.hsplit);
  // With hsplit > 1 the G query heads of the group are shared by hsplit workgroups: the
  // first writes dk/dv, the others partials that a follow-up kernel adds in, in order.
  const int GH = a.G / a.hsplit;                    // heads walked by this workgroup
  const int hbase = hpart * GH;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int nrt = (a.T + 31) / 32;
  const int rs = a.Hq * kD * 2;                     // bytes between rows of q / du
  // Step s walks row tile rt_hi - s / GH: the last one that sees the key block (the last
  // of the sequence, or under a sliding window W the one holding row k0 + KB - 2 + W),
  // down to the key block's own.
  const int W = kWin ? a.window : 0;
  int rt_hi = nrt - 1;

  // Loop-invariant per-thread buffer offsets; the row tile and head move the resource
  // base, so rows past T fall outside the resource and load zeros.
  const int rw = tid >> 3, part = tid & 7, rp = tid & 15, dg = tid >> 4;
  const int voff_c = rw * rs + part * 16;
  const int voff_p0 = 2 * rp * rs + dg * 8;
  const int voff_p1 = voff_p0 + rs;
  const int voff_s = (tid & 31) * a.Hq * 32 + (tid >> 5) * 16;   // r0 (tid < 32) or r1

  // Staged query-side data of one step: q and du row chunks, q and du pair tasks, and
  // (threads < 64) one row record.  kDepth sets are in flight.
  struct Stage {
    u32x4 qst, cst;
    u32x2 qtst[2], dtst[2];
    f32x4 sst;
  };
  Stage st[kDepth];
  auto stage_load = [&](Stage &R, int s) {
    u32x4 &qst = R.qst, &cst = R.cst;
    u32x2 *qtst = R.qtst, *dtst = R.dtst;
    f32x4 &sst = R.sst;
    const int r0row = (rt_hi - s / GH) * 32;
    const int h = g * a.G + hbase + s % GH;
    const size_t row0 = ((size_t)b * a.T + r0row) * a.Hq + h;
    const int nbytes = (int)(((size_t)(a.T - r0row) * a.Hq - h) * kD * 2);
    const auto qr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const uint16_t *)a.q + row0 * kD), 0, nbytes, kBufferFlags);
    const auto dr = __builtin_amdgcn_make_buffer_rsrc((void *)(a.du + row0 * kD), 0, nbytes,
                                                      kBufferFlags);
    qst = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, voff_c, 0, 0));
    cst = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(dr, voff_c, 0, 0));
    qtst[0] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(qr, voff_p0, 0, 0));
    qtst[1] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(qr, voff_p1, 0, 0));
    dtst[0] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(dr, voff_p0, 0, 0));
    dtst[1] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(dr, voff_p1, 0, 0));
    if (tid < 64) {
      const int sbytes = (int)(((size_t)(a.T - r0row) * a.Hq - h) * 32);
      const auto sr = __builtin_amdgcn_make_buffer_rsrc((void *)(a.rows + row0 * 8), 0, sbytes,
                                                        kBufferFlags);
      sst = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, voff_s, 0, 0));
    }
  };
  // Rows past T: p = 0 (lse2 = +inf), zero coefficients, no arg-max key.
  auto stage_store = [&](Stage &R, int buf, int s) {
    const u32x4 &qst = R.qst, &cst = R.cst;
    const u32x2 *qtst = R.qtst, *dtst = R.dtst;
    f32x4 &sst = R.sst;
    if (tid < 64 && (rt_hi - s / GH) * 32 + (tid & 31) >= a.T) {
      const f32x4 pad0 = {1.f, INFINITY, 0.f, 0.f};
      const f32x4 pad1 = {0.f, 0.f, 0.f, __int_as_float(-1)};
      sst = tid < 32 ? pad0 : pad1;
    }
    *(u32x4 *)&Qs[buf][rw * QROW + part * 8] = qst;
    *(u32x4 *)&Cs[buf][rw * QROW + part * 8] = cst;
    const int pos = vpos32<8>(2 * rp);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      *(uint32_t *)&Qt[buf][(dg * 4 + e) * TROW + pos] = pair_word(qtst[0], qtst[1], e);
      *(uint32_t *)&Dt[buf][(dg * 4 + e) * TROW + pos] = pair_word(dtst[0], dtst[1], e);
    }
    if (tid < 32) {
#pragma unroll
      for (int q = 0; q < 4; ++q) Sc[buf][q][tid] = sst[q];
    } else if (tid < 64) {
      Sc[buf][4][tid - 32] = sst[2];
      Sc[buf][5][tid - 32] = sst[3];
    }
  };

  const uint32_t q_lane = (uint32_t)((c32 * QROW + g32 * 8) * 2);
  const uint32_t t_lane = (uint32_t)((c32 * TROW + g32 * 8) * 2);
  constexpr uint32_t QBUF = 32 * QROW * 2, TBUF = kD * TROW * 2;

  for (int half = 0; half < 2; ++half) {
    const int kblk = half == 0 ? pair : a.n_key_blocks - 1 - pair;
    if (half == 1 && kblk == pair) break;            // odd count: the middle block once
    const int k0 = kblk * KB;
    rt_hi = W > 0 ? min(nrt - 1, (k0 + KB - 2 + W) / 32) : nrt - 1;
    const int kw0 = k0 + wave * 32;
    const int key = kw0 + c32;
    const bool kvalid = key < a.T;

    F kf[4], vf[4];
    {
      const size_t kb = (((size_t)b * a.T + (kvalid ? key : 0)) * a.Hkv + g) * kD + g32 * 8;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        kf[ks] = kvalid ? *(const F *)((const uint16_t *)a.k + kb + ks * 16) : Bf16::zero();
        vf[ks] = kvalid ? *(const F *)((const uint16_t *)a.v + kb + ks * 16) : Bf16::zero();
      }
      // Settle these loads here, on every path into the key loop, so the loop's first
      // MFMA does not wait on the staging loads issued in the same step.
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    }
    f32x16 dK[2], dV[2];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dK[db][r] = 0.f;
        dV[db][r] = 0.f;
      }

    const int nsteps = (rt_hi + 1 - k0 / 32) * GH;
    // Pipeline: step s computes from LDS buffer s&1; at its end, step s+1's staged set is
    // stored to the other buffer and refilled with step s+1+kDepth, so every load has
    // kDepth steps to arrive.  The step loop is unrolled by kDepth to keep set indices
    // compile-time constants.
#pragma unroll
    for (int u = 0; u < kDepth; ++u)
      if (u < nsteps) stage_load(st[u], u);
    if (nsteps > 0) stage_store(st[0], 0, 0);
    if (kDepth < nsteps) stage_load(st[0], kDepth);
    __syncthreads();
    for (int s0 = 0; s0 < nsteps; s0 += kDepth) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        const int s = s0 + u;
        if (s >= nsteps) break;
        const int buf = s & 1;
        const int r0row = (rt_hi - s / GH) * 32;
        if (r0row + 31 >= kw0 && kw0 < a.T && (W == 0 || r0row <= kw0 + 30 + W)) {
          const uint16_t *Qb = lds_at(&Qs[0][0], q_lane + buf * QBUF);
          const uint16_t *Cb = lds_at(&Cs[0][0], q_lane + buf * QBUF);
          // The arg-max key of row c32, read ahead of the products that hide its latency.
          const int jl = __float_as_int(Sc[buf][5][c32]);
          const f32x16 zero = {};
          f32x16 S, P;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            S = Bf16::mma32(*(const F *)(Qb + ks * 16), kf[ks], ks == 0 ? zero : S);
            P = Bf16::mma32(*(const F *)(Cb + ks * 16), vf[ks], ks == 0 ? zero : P);
          }
          // Query tiles wholly below the wave's keys need no mask (branch per wave).
          float pv[16], dsv[16];
          auto probs = [&](auto masked) {
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
              const int ri0 = 8 * a4 + 4 * g32;
              const f32x4 cl = *(const f32x4 *)&Sc[buf][0][ri0];
              const f32x4 ls = *(const f32x4 *)&Sc[buf][1][ri0];
              const f32x4 ac = *(const f32x4 *)&Sc[buf][2][ri0];
              const f32x4 ec = *(const f32x4 *)&Sc[buf][3][ri0];
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const int r = 4 * a4 + c;
                float p = fast_exp2(fmaf(S[r], cl[c], -ls[c]));
                if constexpr (decltype(masked)::value) {
                  const int row = r0row + ri0 + c;
                  if (row < key || (W > 0 && row - W >= key)) p = 0.f;
                }
                pv[r] = p;
                // c dl / p = c (du . v_j) + c A + c E p, with c = cl ln 2.
                dsv[r] = p * fmaf(cl[c] * kLn2, P[r], fmaf(ec[c], p, ac[c]));
              }
            }
          };
          if (r0row < kw0 + 31 || (W > 0 && r0row + 31 - W >= kw0))
            probs(std::true_type{});
          else
            probs(std::false_type{});
          // Rows whose arg-max key belongs to this wave (rare): add c*dm at that key.
          if (__ballot(jl >= kw0 && jl < kw0 + 32) != 0) {
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
              const int ri0 = 8 * a4 + 4 * g32;
              const f32x4 jv = *(const f32x4 *)&Sc[buf][5][ri0];
              const f32x4 dmv = *(const f32x4 *)&Sc[buf][4][ri0];
              const f32x4 cl = *(const f32x4 *)&Sc[buf][0][ri0];
#pragma unroll
              for (int c = 0; c < 4; ++c)
                if (__float_as_int(jv[c]) == key) dsv[4 * a4 + c] += dmv[c] * cl[c] * kLn2;
            }
          }
          const F pp0 = Bf16::pack(pv), pp1 = Bf16::pack(pv + 8);
          const F dp0 = Bf16::pack(dsv), dp1 = Bf16::pack(dsv + 8);
          const uint16_t *Db = lds_at(&Dt[0][0], t_lane + buf * TBUF);
          const uint16_t *Tb = lds_at(&Qt[0][0], t_lane + buf * TBUF);
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            dV[db] = Bf16::mma32(*(const F *)(Db + db * 32 * TROW), pp0, dV[db]);
            dK[db] = Bf16::mma32(*(const F *)(Tb + db * 32 * TROW), dp0, dK[db]);
            dV[db] = Bf16::mma32(*(const F *)(Db + db * 32 * TROW + 16), pp1, dV[db]);
            dK[db] = Bf16::mma32(*(const F *)(Tb + db * 32 * TROW + 16), dp1, dK[db]);
          }
        }
        if (s + 1 < nsteps) {
          Stage &nx = st[(u + 1) % kDepth];                // constant once unrolled
          stage_store(nx, buf ^ 1, s + 1);
          if (s + 1 + kDepth < nsteps) stage_load(nx, s + 1 + kDepth);
        }
        __syncthreads();
      }
    }

    if (kvalid) {
      const size_t ob = (((size_t)b * a.T + key) * a.Hkv + g) * kD;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const int d0 = db * 32 + 8 * j4 + 4 * g32;
          f32x4 kv, vv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kv[e] = dK[db][4 * j4 + e];
            vv[e] = dV[db][4 * j4 + e];
          }
          // Under RoPE, dk with respect to the unrotated k (partials too: the turn is
          // linear, so the partial add sums turned vectors).
          if constexpr (kRope) kv = unrotate4(kv, d0, key, a.rope_f);
          const size_t pofs = (size_t)(hpart - 1) * a.B * a.T * a.Hkv * kD;
          *(f32x4 *)((hpart == 0 ? a.dk : a.dk_part + pofs) + ob + d0) = kv;
          *(f32x4 *)((hpart == 0 ? a.dv : a.dv_part + pofs) + ob + d0) = vv;
        }
    }
  }
}

// dk += the partials of the other head groups of the dk/dv kernel, in a fixed order.
__global__ void __launch_bounds__(256) polar_bwd_dkv_add_kernel(BwdArgs a) {
  const size_t n4 = (size_t)a.B * a.T * a.Hkv * kD / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    f32x4 k = ((const f32x4 *)a.dk)[i], v = ((const f32x4 *)a.dv)[i];
    for (int p = 0; p < a.hsplit - 1; ++p) {
      k = k + ((const f32x4 *)a.dk_part)[p * n4 + i];
      v = v + ((const f32x4 *)a.dv_part)[p * n4 + i];
    }
    ((f32x4 *)a.dk)[i] = k;
    ((f32x4 *)a.dv)[i] = v;
  }
}

// ------------------------------------------------------------------ 4. parameter grads
// Stage 1: workgroup (chunk p, head h) sums its rows in a fixed order.
__global__ void __launch_bounds__(256) polar_bwd_param_kernel(BwdArgs a) {
  const int p = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int dim = tid & 63, sub = tid >> 6;
  const long long nr = (long long)a.B * a.T;
  const long long chunk = (nr + a.n_part - 1) / a.n_part;
  const long long lo = (long long)p * chunk;
  const long long hi = min(nr, lo + chunk);
  float dw = 0.f, dbeta = 0.f, dbias = 0.f;
  // Rows in a fixed order; four rows' loads are issued before their sums.
  long long rho = lo + sub;
  for (; rho + 12 < hi; rho += 16) {
    f32x4 rp[4];
    float cc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t rr = (size_t)(rho + 4 * u) * a.Hq + h;
      rp[u] = *(const f32x4 *)(a.rp + 4 * rr);
      cc[u] = a.c_count ? a.c_count[rr * kD + dim] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      dw = fmaf(rp[u][2], cc[u], dw);
      dbeta += rp[u][0] + rp[u][3];
      dbias += rp[u][1];
    }
  }
  for (; rho < hi; rho += 4) {
    const size_t rr = (size_t)rho * a.Hq + h;
    const f32x4 rp = *(const f32x4 *)(a.rp + 4 * rr);
    if (a.c_count) dw = fmaf(rp[2], a.c_count[rr * kD + dim], dw);
    dbeta += rp[0] + rp[3];
    dbias += rp[1];
  }
  __shared__ float red[4][66];
  red[sub][dim] = dw;
  if (dim == 0) {
    red[sub][64] = dbeta;
    red[sub][65] = dbias;
  }
  __syncthreads();
  if (tid < 66)
    a.part[((size_t)h * a.n_part + p) * kPartStride + tid] =
        (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
}

// Stage 2: one workgroup per head adds the chunks in order.
__global__ void __launch_bounds__(128) polar_bwd_param_final_kernel(BwdArgs a) {
  const int h = blockIdx.x, tid = threadIdx.x;
  if (tid >= 66) return;
  float s = 0.f;
  const float *pp = a.part + (size_t)h * a.n_part * kPartStride + tid;
  int p = 0;
  for (; p + 8 <= a.n_part; p += 8) {                // loads issued ahead, sums in order
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = pp[(size_t)(p + u) * kPartStride];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += x[u];
  }
  for (; p < a.n_part; ++p) s += pp[(size_t)p * kPartStride];
  if (tid < 64) {
    if (a.d_count_vec) a.d_count_vec[(size_t)h * kD + tid] = s;
  } else if (tid == 64) {
    if (a.d_beta) a.d_beta[h] = s;
  } else {
    if (a.d_null_bias) a.d_null_bias[h] = s;
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int n_parts(int B, int T) {
  const long long nr = (long long)B * T;
  return (int)max(1LL, min(256LL, (nr + 255) / 256));
}

}  // namespace

size_t bwd_ws_bytes(int B, int T, int Hq, int Hkv) {
  const size_t nrows = (size_t)B * T * Hq;
  return align256(nrows * kD * 2) + align256(nrows * 32) + align256(nrows * 16) +
         align256((size_t)Hq * n_parts(B, T) * kPartStride * 4) +
         2 * align256((size_t)(kDkvSplitMax - 1) * B * T * Hkv * kD * 4);
}

void bwd_ws_layout(BwdArgs &a, void *ws) {
  const size_t nrows = (size_t)a.B * a.T * a.Hq;
  char *p = (char *)ws;
  a.du = (uint16_t *)p;
  p += align256(nrows * kD * 2);
  a.rows = (float *)p;
  p += align256(nrows * 32);
  a.rp = (float *)p;
  p += align256(nrows * 16);
  a.part = (float *)p;
  p += align256((size_t)a.Hq * n_parts(a.B, a.T) * kPartStride * 4);
  a.dk_part = (float *)p;
  p += align256((size_t)(kDkvSplitMax - 1) * a.B * a.T * a.Hkv * kD * 4);
  a.dv_part = (float *)p;
  a.n_part = n_parts(a.B, a.T);
}

int bwd_rows_per_block(int hb) { return (kDqWaves / hb) * 32; }
int bwd_keys_per_block() { return 32 * kDkvWaves; }
int bwd_head_split(int G) {
  for (int s = kDkvSplitMax; s > 1; s >>= 1)
    if (G % s == 0) return s;
  return 1;
}

// Zero fill by a kernel rather than hipMemsetAsync, so that a caller may capture the call in
// a graph (a memset node there is avoided on purpose).
__global__ void __launch_bounds__(256) polar_zero_kernel(float *p, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
    p[i] = 0.f;
}

hipError_t launch_zero(float *p, long long n, hipStream_t stream) {
  if (!p || n <= 0) return hipSuccess;
  const long long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(polar_zero_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)),
                     dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream) {
  const long long nrows = (long long)a.B * a.T * a.Hq;
  if (nrows <= 0) return hipSuccess;
  hipLaunchKernelGGL(polar_bwd_prep_kernel, dim3((unsigned)((nrows + 15) / 16)), dim3(256), 0,
                     stream, a);
  const long long dq_blocks = (long long)a.n_row_blocks * a.Hkv * (a.G / a.hb) * a.B;
  const long long dkv_blocks =
      (long long)((a.n_key_blocks + 1) / 2) * a.hsplit * a.Hkv * a.B;
  const dim3 gq((unsigned)dq_blocks), bq(64 * kDqWaves);
  const dim3 gk((unsigned)dkv_blocks), bk(64 * kDkvWaves);
  if (a.window > 0) {
    hipLaunchKernelGGL((polar_bwd_dq_kernel<kDqWaves, true>), gq, bq, 0, stream, a);
    if (a.rope)
      hipLaunchKernelGGL((polar_bwd_dkv_kernel<kDkvWaves, kDkvDepth, true, true>), gk, bk, 0,
                         stream, a);
    else
      hipLaunchKernelGGL((polar_bwd_dkv_kernel<kDkvWaves, kDkvDepth, true, false>), gk, bk, 0,
                         stream, a);
  } else {
    hipLaunchKernelGGL((polar_bwd_dq_kernel<kDqWaves, false>), gq, bq, 0, stream, a);
    if (a.rope)
      hipLaunchKernelGGL((polar_bwd_dkv_kernel<kDkvWaves, kDkvDepth, false, true>), gk, bk, 0,
                         stream, a);
    else
      hipLaunchKernelGGL((polar_bwd_dkv_kernel<kDkvWaves, kDkvDepth, false, false>), gk, bk,
                         0, stream, a);
  }
  if (a.hsplit > 1) {
    const long long n4 = (long long)a.B * a.T * a.Hkv * kD / 4;
    hipLaunchKernelGGL(polar_bwd_dkv_add_kernel, dim3((unsigned)min((n4 + 255) / 256, 8192LL)),
                       dim3(256), 0, stream, a);
  }
  if (a.d_beta || a.d_null_bias || a.d_count_vec) {
    hipLaunchKernelGGL(polar_bwd_param_kernel, dim3(a.n_part, a.Hq), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(polar_bwd_param_final_kernel, dim3(a.Hq), dim3(128), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace polar
