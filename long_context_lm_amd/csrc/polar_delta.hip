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
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, xi, kCtrl, 0xF, 0xF, false));
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

// ---------------------------------------------------------------------------------------
// The memory stream over a sequence: the same step for tokens t = 0..T-1 in order, the
// state held in registers from its single read to its single write, o_t for every token.
//
// A workgroup of 4 waves owns one half (32 rows of d_v) of one (sequence, head) state; the
// rows of the gated delta rule are independent given k, q and the row's v, so the two
// halves need no communication.  Wave w holds rows 8 w .. 8 w + 7 of its half, lane l
// columns 8 (l % 8) .. + 7 of row 8 w + l / 8: the row sums S k and S q reduce over the 8
// lanes of a DPP half-row.  Tokens pass through LDS in chunks of C: the workgroup loads a
// chunk's q and k (64 dims), v (its 32 rows), alpha and beta (256 / C threads per token),
// L2-normalises q and k there (the step's x / sqrt(x.x + 1e-12)) and forms k.q once per
// token; the next chunk's loads are issued before the current chunk is walked.  The walk
// is the step's arithmetic, u = beta (v - alpha S k), o = alpha S q + u (k.q),
// S' = alpha S + u k^T, token after token.  Tokens past the end of the sequence are staged
// as alpha = 1, beta = 0, k = q = v = 0, which leaves S bit-for-bit unchanged, so every
// chunk is walked in full.  o is identical in the 8 lanes of a row; over 8 tokens lane
// c keeps the o of token c and writes it to LDS, and the chunk leaves in 128-byte rows.
// Sum over the 8 lanes of a DPP half-row (every lane gets the same bits).
__device__ __forceinline__ float row8_sum(float x) {
  x = dpp_sum_step<0xB1>(x);    // quad_perm 1,0,3,2
  x = dpp_sum_step<0x4E>(x);    // quad_perm 2,3,0,1
  return dpp_sum_step<0x141>(x);  // row_half_mirror: quads 0<->1, 2<->3
}
// Sum over groups of N (2, 4 or 8) neighbouring lanes.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if (N >= 2) x = dpp_sum_step<0xB1>(x);
  if (N >= 4) x = dpp_sum_step<0x4E>(x);
  if (N >= 8) x = dpp_sum_step<0x141>(x);
  return x;
}

struct SeqTok {
  float alpha, beta, kq, pad;
};

// N consecutive elements of E, held raw between the global load and the conversion.
template <class E, int N>
struct RawVec {
  static constexpr int kWords = N * (int)sizeof(E) / 4;
  static_assert(kWords % 2 == 0, "8-byte granules");
  uint32_t w[kWords];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = 0u;
  }
  __device__ __forceinline__ void load(const E *p) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    if constexpr (kWords % 4 == 0) {
#pragma unroll
      for (int i = 0; i < kWords / 4; ++i) {
        const u32x4 x = *((const u32x4 *)p + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[4 * i + e] = x[e];
      }
    } else {
#pragma unroll
      for (int i = 0; i < kWords / 2; ++i) {
        const u32x2 x = *((const u32x2 *)p + i);
        w[2 * i] = x[0];
        w[2 * i + 1] = x[1];
      }
    }
  }
  __device__ __forceinline__ void to_f32(float *x) const {
#pragma unroll
    for (int i = 0; i < kWords; ++i) {
      if constexpr (sizeof(E) == 2) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      } else {
        x[i] = __uint_as_float(w[i]);
      }
    }
  }
};

template <class E, int C>
__global__ void __launch_bounds__(256) polar_delta_seq_kernel(DeltaSeqArgs a) {
  constexpr int D = kHeadDim;
  constexpr int TPT = 256 / C;        // staging threads per token
  constexpr int DPT = D / TPT;        // q and k dims per staging thread
  constexpr int VPT = 32 / TPT;       // v rows per staging thread
  constexpr int OP = 36;              // o row pitch in LDS (16-byte aligned, spreads banks)
  static_assert(C % 8 == 0 && TPT >= 2 && TPT <= 8, "chunk of 32..128 tokens");
  __shared__ __attribute__((aligned(16))) float ks[C][D], qs[C][D], vs[C][32], os[C][OP];
  __shared__ __attribute__((aligned(16))) SeqTok tk[C];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = blockIdx.x & 1, bh = blockIdx.x >> 1;
  const int b = bh / a.H, h = bh % a.H;
  const int slot = a.slots[b];
  const bool ok = slot >= 0 && slot < a.num_slots;      // uniform over the workgroup
  const int rl = wave * 8 + (lane >> 3), cg = lane & 7;   // walk: row in the half, columns
  const int tt = tid / TPT, tq = tid % TPT;               // staging: token, part

  float S[8];
  float *const sp =
      a.pool + (((size_t)(ok ? slot : 0) * a.H + h) * D + half * 32 + rl) * D + cg * 8;
  if (ok) {
    const f32x4 s0 = *(const f32x4 *)sp, s1 = *(const f32x4 *)(sp + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      S[e] = s0[e];
      S[4 + e] = s1[e];
    }
  }

  RawVec<E, DPT> rq, rk;
  RawVec<E, VPT> rv;
  rq.zero();
  rk.zero();
  rv.zero();
  float al = 1.f, be = 0.f;
  auto fetch = [&](int c0) {
    const int t = c0 + tt;
    if (t < a.T) {
      const size_t tok = ((size_t)b * a.T + t) * a.H + h;
      rq.load((const E *)a.q + tok * D + DPT * tq);
      rk.load((const E *)a.k + tok * D + DPT * tq);
      rv.load((const E *)a.v + tok * D + half * 32 + VPT * tq);
      al = a.alpha[tok];
      be = a.beta[tok];
    }
  };
  auto stage = [&](int c0) {
    const bool live = c0 + tt < a.T;    // uniform over each group of TPT lanes
    float qf[DPT], kf[DPT], vf[VPT];
    rq.to_f32(qf);
    rk.to_f32(kf);
    rv.to_f32(vf);
    float kk = 0.f, qq = 0.f, kq = 0.f;
#pragma unroll
    for (int e = 0; e < DPT; ++e) {
      kk = fmaf(kf[e], kf[e], kk);
      qq = fmaf(qf[e], qf[e], qq);
      kq = fmaf(kf[e], qf[e], kq);
    }
    kk = group_sum<TPT>(kk);
    qq = group_sum<TPT>(qq);
    kq = group_sum<TPT>(kq);
    const float rk = a.normalize ? rsqrtf(kk + 1e-12f) : 1.0f;
    const float rq = a.normalize ? rsqrtf(qq + 1e-12f) : 1.0f;
    // A padded token's registers hold an earlier token (or zeros): select, never scale.
#pragma unroll
    for (int i = 0; i < DPT / 4; ++i) {
      f32x4 kw, qw;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kw[e] = live ? kf[4 * i + e] * rk : 0.0f;
        qw[e] = live ? qf[4 * i + e] * rq : 0.0f;
      }
      *(f32x4 *)&ks[tt][DPT * tq + 4 * i] = kw;
      *(f32x4 *)&qs[tt][DPT * tq + 4 * i] = qw;
    }
#pragma unroll
    for (int i = 0; i < VPT / 4; ++i) {
      f32x4 vw;
#pragma unroll
      for (int e = 0; e < 4; ++e) vw[e] = live ? vf[4 * i + e] : 0.0f;
      *(f32x4 *)&vs[tt][VPT * tq + 4 * i] = vw;
    }
    if (tq == 0) tk[tt] = live ? SeqTok{al, be, kq * rk * rq, 0.f} : SeqTok{1.f, 0.f, 0.f, 0.f};
    // Every load of this chunk has been consumed: no global load is in flight past here.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  };

  fetch(0);
  for (int c0 = 0; c0 < a.T; c0 += C) {
    stage(c0);
    __syncthreads();
    if (c0 + C < a.T) fetch(c0 + C);          // lands while this chunk is walked
    if (ok) {
      for (int t0 = 0; t0 < C; t0 += 8) {
        float osel = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int t = t0 + j;
          const f32x4 k0 = *(const f32x4 *)&ks[t][cg * 8];
          const f32x4 k1 = *(const f32x4 *)&ks[t][cg * 8 + 4];
          const f32x4 q0 = *(const f32x4 *)&qs[t][cg * 8];
          const f32x4 q1 = *(const f32x4 *)&qs[t][cg * 8 + 4];
          const SeqTok tok = tk[t];
          const float vr = vs[t][rl];
          float sk0 = 0.f, sk1 = 0.f, sq0 = 0.f, sq1 = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sk0 = fmaf(S[e], k0[e], sk0);
            sk1 = fmaf(S[4 + e], k1[e], sk1);
            sq0 = fmaf(S[e], q0[e], sq0);
            sq1 = fmaf(S[4 + e], q1[e], sq1);
          }
          const float sk = row8_sum(sk0 + sk1), sq = row8_sum(sq0 + sq1);
          const float u = tok.beta * (vr - tok.alpha * sk);
          const float o = tok.alpha * sq + u * tok.kq;
          osel = cg == j ? o : osel;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            S[e] = fmaf(u, k0[e], tok.alpha * S[e]);
            S[4 + e] = fmaf(u, k1[e], tok.alpha * S[4 + e]);
          }
        }
        os[t0 + cg][rl] = osel;
      }
    }
    __syncthreads();
    // The chunk's outputs: TPT threads per token, VPT floats each.
    if (c0 + tt < a.T) {
      float *op = a.out + (((size_t)b * a.T + c0 + tt) * a.H + h) * D + half * 32 + VPT * tq;
#pragma unroll
      for (int i = 0; i < VPT / 4; ++i)
        *(f32x4 *)(op + 4 * i) =
            ok ? *(const f32x4 *)&os[tt][VPT * tq + 4 * i] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  if (ok) {
    *(f32x4 *)sp = f32x4{S[0], S[1], S[2], S[3]};
    *(f32x4 *)(sp + 4) = f32x4{S[4], S[5], S[6], S[7]};
  }
}

}  // namespace

hipError_t launch_delta_sequence(int dtype, const DeltaSeqArgs &a, hipStream_t stream) {
  constexpr int C = 64;   // tokens per chunk
  const long long wgs = 2LL * a.B * a.H;
  if (wgs <= 0 || a.T <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL((polar_delta_seq_kernel<uint16_t, C>), dim3((unsigned)wgs), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((polar_delta_seq_kernel<float, C>), dim3((unsigned)wgs), dim3(256), 0,
                       stream, a);
  return hipGetLastError();
}

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
