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

#include <type_traits>


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
// A workgroup of 4 waves owns one (sequence, head) state.  Lane l of wave w holds columns
// CPL (l % LPR) .. + CPL - 1 of row CPL w + l / LPR (CPL = 16 columns, LPR = 4 lanes per
// row): the row sums S k and S q reduce over the LPR lanes of a DPP quad.  Tokens pass
// through LDS in chunks of C: the workgroup loads a chunk's q, k and v (64 dims each),
// alpha and beta (256 / C threads per token), L2-normalises q and k there (the step's
// x / sqrt(x.x + 1e-12)) and forms k.q once per token; the next chunk's loads are issued
// before the current chunk is walked.  Sixteen columns per lane keep the per-token
// overhead (two DPP steps per row sum, the scalars u and o) small beside the three
// multiply-adds per state element; the arithmetic, not LDS, bounds the walk.
//
// The walk takes tokens in groups of 8 and defers the gate: with g_j the product of the
// group's alpha up to token j and S = g_j R, the step u = beta (v - alpha S k),
// o = alpha S q + u (k.q), S' = alpha S + u k^T becomes
//   u = beta v - (beta g_j) (R k),   o = g_j (R q) + u (k.q),   R' = R + (u / g_j) k^T,
// one multiply-add per state element per token instead of a multiply and a multiply-add;
// S = g_7 R is restored at the end of the group.  The step's value is unchanged up to fp32
// rounding.  A group where a running gate product leaves [2^-64, 2^64] (or is not a
// number) takes the step as written, so no input overflows the deferred form.
//
// Tokens past the end of the sequence are staged as alpha = 1, beta = 0, k = q = v = 0,
// which leaves the state bit-for-bit unchanged, so every chunk is walked in full.  o is
// identical in the LPR lanes of a row; over a group lane c keeps the o of tokens c, c + 4,
// writes them to LDS, and the chunk leaves in 256-byte rows.

// Sum over groups of N (2, 4 or 8) neighbouring lanes.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if (N >= 2) x = dpp_sum_step<0xB1>(x);
  if (N >= 4) x = dpp_sum_step<0x4E>(x);
  if (N >= 8) x = dpp_sum_step<0x141>(x);
  return x;
}

// Per-token constants of the walk.  Deferred form: c1 = beta g, g, rg = 1 / g.  Step as
// written: c1 = beta alpha, g = alpha, rg unused.  vs holds beta v in both.
struct SeqTok {
  float c1, g, rg, kq;
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

template <class E, int C, int CPL>
__global__ void __launch_bounds__(256) polar_delta_seq_kernel(DeltaSeqArgs a) {
  constexpr int D = kHeadDim;
  constexpr int LPR = D / CPL;        // lanes per state row (the row sums reduce over them)
  constexpr int RW = 4 * CPL;         // state rows per workgroup (4 waves, a row per lane)
  constexpr int NP = D / RW;          // workgroups per state
  constexpr int NSL = 8 / LPR;        // tokens of a group whose o one lane keeps
  constexpr int TPT = 256 / C;        // staging threads per token
  constexpr int DPT = D / TPT;        // q and k dims per staging thread
  constexpr int VPT = RW / TPT;       // v rows per staging thread
  constexpr int OP = RW + 4;          // o row pitch in LDS (16-byte aligned, spreads banks)
  static_assert(C % 8 == 0 && TPT >= 2 && TPT <= 8 && VPT >= 4, "chunk of 32..128 tokens");
  static_assert(CPL == 8 || CPL == 16, "8 or 16 columns per lane");
  __shared__ __attribute__((aligned(16))) float ks[C][D], qs[C][D], vs[C][RW], os[C][OP];
  __shared__ __attribute__((aligned(16))) SeqTok tk[C];
  __shared__ int direct[C / 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = blockIdx.x % NP, bh = blockIdx.x / NP;
  const int b = bh / a.H, h = bh % a.H;
  const int slot = a.slots[b];
  const bool ok = slot >= 0 && slot < a.num_slots;      // uniform over the workgroup
  const int cg = lane % LPR;                              // walk: columns CPL cg .. + CPL-1
  const int rw = wave * CPL + lane / LPR;                 // walk: row in the workgroup
  const int tt = tid / TPT, tq = tid % TPT;               // staging: token, part

  float S[CPL];
  float *const sp =
      a.pool + (((size_t)(ok ? slot : 0) * a.H + h) * D + part * RW + rw) * D + cg * CPL;
  if (ok) {
#pragma unroll
    for (int c = 0; c < CPL / 4; ++c) {
      const f32x4 x = *(const f32x4 *)(sp + 4 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) S[4 * c + e] = x[e];
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
      rv.load((const E *)a.v + tok * D + part * RW + VPT * tq);
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
    const float alive = live ? al : 1.0f, blive = live ? be : 0.0f;
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
      for (int e = 0; e < 4; ++e) vw[e] = live ? blive * vf[4 * i + e] : 0.0f;
      *(f32x4 *)&vs[tt][VPT * tq + 4 * i] = vw;
    }
    // The group of 8 tokens holding token tt lies in 8 TPT consecutive lanes of this wave
    // (token j of the group at lanes base + j TPT): the gate products g_j and the group's
    // g_7 are formed in the same order in every lane.
    const int j = tt & 7, base = (lane / (8 * TPT)) * (8 * TPT);
    float g = 1.0f, g7 = 1.0f;
    bool tame = true;                       // every running product in [2^-64, 2^64]
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float ai = __shfl(alive, base + i * TPT);
      g7 *= ai;
      g = i <= j ? g7 : g;
      tame = tame && g7 >= 0x1p-64f && g7 <= 0x1p64f;   // false for a NaN gate
    }
    const bool dir = !tame;
    if (tq == 0) {
      const float kqn = live ? kq * rk * rq : 0.0f;
      tk[tt] = dir ? SeqTok{blive * alive, alive, 0.0f, kqn}
                   : SeqTok{blive * g, g, 1.0f / g, kqn};
      if (j == 0) direct[tt >> 3] = dir ? 1 : 0;
    }
    // Every load of this chunk has been consumed: no global load is in flight past here.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  };

  // One group of 8 tokens from token t0 of the chunk.
  struct Tok {
    f32x4 k[CPL / 4], q[CPL / 4];
    SeqTok c;
    float bv;
  };
  auto read_tok = [&](int t, Tok &x) {
#pragma unroll
    for (int c = 0; c < CPL / 4; ++c) {
      x.k[c] = *(const f32x4 *)&ks[t][cg * CPL + 4 * c];
      x.q[c] = *(const f32x4 *)&qs[t][cg * CPL + 4 * c];
    }
    x.c = tk[t];
    x.bv = vs[t][rw];
  };
  auto walk_group = [&](int t0, auto deferred) {
    constexpr bool kDeferred = decltype(deferred)::value;
    float osel[NSL], g7 = 1.0f;
#pragma unroll
    for (int n = 0; n < NSL; ++n) osel[n] = 0.f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      Tok cur;
      read_tok(t0 + jj, cur);
      float sk0 = 0.f, sk1 = 0.f, sq0 = 0.f, sq1 = 0.f;
#pragma unroll
      for (int c = 0; c < CPL / 4; c += 2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sk0 = fmaf(S[4 * c + e], cur.k[c][e], sk0);
          sk1 = fmaf(S[4 * c + 4 + e], cur.k[c + 1][e], sk1);
          sq0 = fmaf(S[4 * c + e], cur.q[c][e], sq0);
          sq1 = fmaf(S[4 * c + 4 + e], cur.q[c + 1][e], sq1);
        }
      const float sk = group_sum<LPR>(sk0 + sk1), sq = group_sum<LPR>(sq0 + sq1);
      const float u = fmaf(-cur.c.c1, sk, cur.bv);
      const float o = fmaf(cur.c.g, sq, u * cur.c.kq);
      osel[jj / LPR] = cg == jj % LPR ? o : osel[jj / LPR];
      if constexpr (kDeferred) {
        const float w = u * cur.c.rg;
#pragma unroll
        for (int c = 0; c < CPL / 4; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) S[4 * c + e] = fmaf(w, cur.k[c][e], S[4 * c + e]);
      } else {
#pragma unroll
        for (int c = 0; c < CPL / 4; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            S[4 * c + e] = fmaf(u, cur.k[c][e], cur.c.g * S[4 * c + e]);
      }
      g7 = cur.c.g;
    }
    if constexpr (kDeferred) {
#pragma unroll
      for (int e = 0; e < CPL; ++e) S[e] *= g7;
    }
#pragma unroll
    for (int n = 0; n < NSL; ++n) os[t0 + n * LPR + cg][rw] = osel[n];
  };

  fetch(0);
  for (int c0 = 0; c0 < a.T; c0 += C) {
    stage(c0);
    __syncthreads();
    if (c0 + C < a.T) fetch(c0 + C);          // lands while this chunk is walked
    if (ok) {
      for (int t0 = 0; t0 < C; t0 += 8) {
        if (__builtin_amdgcn_readfirstlane(direct[t0 >> 3]))
          walk_group(t0, std::false_type{});
        else
          walk_group(t0, std::true_type{});
      }
    }
    __syncthreads();
    // The chunk's outputs: TPT threads per token, VPT floats each.
    if (c0 + tt < a.T) {
      float *op = a.out + (((size_t)b * a.T + c0 + tt) * a.H + h) * D + part * RW + VPT * tq;
#pragma unroll
      for (int i = 0; i < VPT / 4; ++i)
        *(f32x4 *)(op + 4 * i) =
            ok ? *(const f32x4 *)&os[tt][VPT * tq + 4 * i] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  if (ok) {
#pragma unroll
    for (int c = 0; c < CPL / 4; ++c)
      *(f32x4 *)(sp + 4 * c) = f32x4{S[4 * c], S[4 * c + 1], S[4 * c + 2], S[4 * c + 3]};
  }
}

}  // namespace

hipError_t launch_delta_sequence(int dtype, const DeltaSeqArgs &a, hipStream_t stream) {
  constexpr int C = 32;     // tokens per chunk (34 KB of LDS)
  constexpr int CPL = 16;   // state columns per lane: one workgroup per state
  const long long wgs = (long long)(kHeadDim / (4 * CPL)) * a.B * a.H;
  if (wgs <= 0 || a.T <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL((polar_delta_seq_kernel<uint16_t, C, CPL>), dim3((unsigned)wgs),
                       dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((polar_delta_seq_kernel<float, C, CPL>), dim3((unsigned)wgs), dim3(256),
                       0, stream, a);
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
