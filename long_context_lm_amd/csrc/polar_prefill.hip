// Fused causal Polar Attention prefill for gfx950.
//
// Follows the fused kernel of the ATMA technical summary (gist.science), section 2.2
// "Hardware-Software Codesign": participation ratios are computed online in O(block)
// memory with streaming accumulators and squared correction factors, so the T x T
// scores never exist in memory.  The arithmetic per row is section 2.1's direction and
// magnitude channels (definitions in include/polar.h).
//
// Work decomposition (one workgroup = 4 waves = 256 threads):
//  * a workgroup owns `hb` query heads that share one KV head (GQA) and a block of rows;
//    each wave owns 32*QB consecutive rows of one of those heads;
//  * K and V tiles of 64 keys are staged global -> registers -> LDS, double buffered, so
//    every K/V byte brought on chip serves all `hb` heads and all rows of the block;
//  * S^T = K Q^T runs on MFMA with K from LDS and Q resident in registers.  The 32x32
//    output puts one query per lane (column) and 16 keys per lane, so the row statistics
//    need one cross-half exchange per tile and the probabilities are already laid out as
//    the B operand of O^T = V^T P^T, whose V^T operand is read from a transposed LDS tile;
//  * online statistics per row, in log2 units x = beta*tau*log2(e)*<q,k>:
//      running reference M (raised lazily when the tile maximum exceeds it by > 8),
//      S = sum 2^(x-M), Q = sum 2^(2(x-M)), u = sum 2^(x-M) v, and the exact row maximum.
//    Raising the reference rescales S and u by 2^(M_old-M_new) and Q by its square, the
//    squared correction factor of section 2.2;
//  * epilogue: n_eff = S^2/Q, lse, the floor gate, dir = u/|u|, count.
#include "polar_kernels.h"
#include "polar_mfma.h"

namespace polar {
namespace {

constexpr int kD = kHeadDim;
constexpr int kKT = 64;          // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLazyTheta = 8.0f;

template <class TR> struct LdsCfg;
template <> struct LdsCfg<Bf16> { static constexpr int krow = 72, vrow = 72; };  // 144 B rows
template <> struct LdsCfg<F32> { static constexpr int krow = 68, vrow = 65; };

// Position of key k32 (0..31 inside a 32-key block) in a transposed V row: the kpl keys
// that one lane feeds to one P.V MFMA sit next to each other.  Lane group g of MFMA t
// supplies slots e = 0..kpl-1 for keys 8*(i/4) + 4*g + i%4 with i = t*kpl + e (the keys
// that the score MFMA left in that lane).
template <int KPL>
__device__ __forceinline__ int vpos32(int k32) {
  const int a = k32 >> 3, gg = (k32 >> 2) & 1, cc = k32 & 3;
  const int i = 4 * a + cc;
  return (i / KPL) * (2 * KPL) + gg * KPL + (i % KPL);
}

template <class TR, int QB>
__global__ void __launch_bounds__(kThreads) polar_prefill_kernel(PrefillArgs a) {
  using E = typename TR::elem_t;
  using F = typename TR::frag_t;
  constexpr int KPL = TR::kpl, KSTEP = 2 * KPL, NKS = kD / KSTEP, NT = 16 / KPL;
  constexpr int KROW = LdsCfg<TR>::krow, VROW = LdsCfg<TR>::vrow;
  constexpr int VEC = TR::vec;                       // elements per 16-byte chunk
  constexpr int CPR = kD / VEC;                      // chunks per key row
  constexpr int NCH = kKT * CPR / kThreads;          // chunks per thread per tile
  __shared__ __attribute__((aligned(16))) E Ks[2][kKT * KROW];
  __shared__ __attribute__((aligned(16))) E Vs[2][kD * VROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g32 = lane >> 5, c32 = lane & 31;

  // Heaviest row blocks first; consecutive blocks cycle over (KV head, batch).
  const int n_hc = a.G / a.hb;
  const int NY = a.Hkv * n_hc;
  int id = blockIdx.x;
  const int b = id % a.B;
  id /= a.B;
  const int y = id % NY;
  const int rb = a.n_row_blocks - 1 - id / NY;
  const int g = y / n_hc, hc = y % n_hc;
  const int h = g * a.G + hc * a.hb + (wave % a.hb);
  const int WR = (kWaves / a.hb) * 32 * QB;
  const int row0 = rb * WR;
  const int wrow0 = row0 + (wave / a.hb) * 32 * QB;
  const int wg_last = min(row0 + WR, a.T) - 1;
  const int w_last = wrow0 < a.T ? min(wrow0 + 32 * QB, a.T) - 1 : -1;
  const int ntiles = wg_last / kKT + 1;

  const size_t kv_stride = (size_t)a.Hkv * kD;     // elements between consecutive keys
  const E *__restrict__ kbase = (const E *)a.k + ((size_t)b * a.T * a.Hkv + g) * kD;
  const E *__restrict__ vbase = (const E *)a.v + ((size_t)b * a.T * a.Hkv + g) * kD;

  // Per-row logit scales: natural units and log2 units.
  const float beta = a.beta ? a.beta[h] : 8.0f;
  float cnat[QB], cl2[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wrow0 + qb * 32 + c32;
    const float tau =
        a.inv_log_train > 0.f ? fmaxf(1.0f, logf((float)(row + 1)) * a.inv_log_train) : 1.0f;
    cnat[qb] = beta * tau;
    cl2[qb] = cnat[qb] * kLog2e;
  }

  // Q fragments (B operand of S^T = K Q^T), resident for the whole key loop.
  F qf[QB][NKS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wrow0 + qb * 32 + c32;
    const bool ok = row < a.T;
    const E *qp = (const E *)a.q + (((size_t)b * a.T + (ok ? row : 0)) * a.Hq + h) * kD + g32 * KPL;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[qb][ks] = ok ? TR::load(qp + ks * KSTEP) : TR::zero();
  }

  f32x16 o[QB][2];
  float Mref[QB], smax[QB], Ssum[QB], Qsum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.f;
    Mref[qb] = -INFINITY;
    smax[qb] = -INFINITY;
    Ssum[qb] = 0.f;
    Qsum[qb] = 0.f;
  }

  // ---- K/V staging: global -> registers -> LDS (V transposed) ----
  u32x4 kst[NCH], vst[NCH];
  auto stage_load = [&](int t) {
    const int key0 = t * kKT;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ch = tid + kThreads * j;
      const int key = ch / CPR, part = ch % CPR;
      const u32x4 z = {0u, 0u, 0u, 0u};
      kst[j] = (key0 + key < a.T)
                   ? *(const u32x4 *)(kbase + (size_t)(key0 + key) * kv_stride + part * VEC)
                   : z;
    }
    if constexpr (KPL == 8) {
      // bf16: thread takes keys (2p, 2p+1) x 8 dims so a pair lands in one LDS word.
      const int p = tid / CPR, part = tid % CPR;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int key = 2 * p + j;
        const u32x4 z = {0u, 0u, 0u, 0u};
        vst[j] = (key0 + key < a.T)
                     ? *(const u32x4 *)(vbase + (size_t)(key0 + key) * kv_stride + part * VEC)
                     : z;
      }
    } else {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int ch = tid + kThreads * j;
        const int key = ch / CPR, part = ch % CPR;
        const u32x4 z = {0u, 0u, 0u, 0u};
        vst[j] = (key0 + key < a.T)
                     ? *(const u32x4 *)(vbase + (size_t)(key0 + key) * kv_stride + part * VEC)
                     : z;
      }
    }
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ch = tid + kThreads * j;
      const int key = ch / CPR, part = ch % CPR;
      *(u32x4 *)&Ks[buf][key * KROW + part * VEC] = kst[j];
    }
    if constexpr (KPL == 8) {
      const int p = tid / CPR, part = tid % CPR;
      const int key = 2 * p;
      const int pos = (key >> 5) * 32 + vpos32<KPL>(key & 31);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w0 = vst[0][e >> 1], w1 = vst[1][e >> 1];
        const uint32_t word = (e & 1) ? ((w0 >> 16) | (w1 & 0xFFFF0000u))
                                      : ((w0 & 0xFFFFu) | (w1 << 16));
        *(uint32_t *)&Vs[buf][(part * 8 + e) * VROW + pos] = word;
      }
    } else {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int ch = tid + kThreads * j;
        const int key = ch / CPR, part = ch % CPR;
        const int pos = (key >> 5) * 32 + vpos32<KPL>(key & 31);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Vs[buf][(part * 4 + e) * VROW + pos] = __uint_as_float(vst[j][e]);
      }
    }
  };

  stage_load(0);
  stage_store(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool has_next = t + 1 < ntiles;
    if (has_next) stage_load(t + 1);
    const int key0 = t * kKT;
    if (key0 <= w_last) {
      const E *Kt = Ks[buf];
      const E *Vt = Vs[buf];
      // S^T = K Q^T for two 32-key blocks.
      f32x16 s[QB][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const F ka = TR::load(Kt + (kb * 32 + c32) * KROW + ks * KSTEP + g32 * KPL);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][kb] = TR::mma32(ka, qf[qb][ks], s[qb][kb]);
        }
      }
      const bool need_mask = key0 + kKT - 1 > wrow0;
      F pf[QB][2][NT];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int row = wrow0 + qb * 32 + c32;
        if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * g32 + (r & 3);
              if (key > row) s[qb][kb][r] = -INFINITY;
            }
        }
        float mx = s[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
        mx = half_max(mx);
        smax[qb] = fmaxf(smax[qb], mx);
        const float mt = mx * cl2[qb];
        if (mt > Mref[qb] + kLazyTheta) {
          const float alpha = fast_exp2(Mref[qb] - mt);
          Ssum[qb] *= alpha;
          Qsum[qb] *= alpha * alpha;
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
          Mref[qb] = mt;
        }
        const float negM = -Mref[qb];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          float pv[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) pv[r] = fast_exp2(fmaf(s[qb][kb][r], cl2[qb], negM));
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            pf[qb][kb][tt] = TR::pack(pv + tt * KPL);
            TR::stats(pf[qb][kb][tt], Ssum[qb], Qsum[qb]);
          }
        }
      }
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            const F va = TR::load(Vt + (db * 32 + c32) * VROW + kb * 32 + tt * KSTEP + g32 * KPL);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) o[qb][db] = TR::mma32(va, pf[qb][kb][tt], o[qb][db]);
          }
    }
    if (has_next) stage_store(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  const float bias = a.null_bias ? a.null_bias[h] : 0.0f;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wrow0 + qb * 32 + c32;
    const float St = half_sum(Ssum[qb]);
    const float Qt = half_sum(Qsum[qb]);
    float nrm = 0.f;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) nrm = fmaf(o[qb][db][r], o[qb][db][r], nrm);
    nrm = half_sum(nrm);
    if (row < a.T) {
      const float neff = St * St / Qt;
      const float lse = (Mref[qb] + log2f(St)) * kLn2;
      const float m_nat = smax[qb] * cnat[qb];
      float floor_ = bias;
      if (a.null_floor) floor_ += cnat[qb] * 0.125f * sqrtf(2.0f * logf((float)(row + 1)));
      const float gate = 1.0f / (1.0f + expf(floor_ - m_nat));
      const float n2 = neff * neff;
      const float th = (n2 - 1.0f) / (n2 + 1.0f);
      const float inv = nrm > 0.f ? rsqrtf(nrm) : 0.f;
      const size_t obase = ((size_t)b * a.T + row) * a.Hq + h;
      float *dp = a.dir + obase * kD;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const int dim0 = db * 32 + 8 * j4 + 4 * g32;
          f32x4 val;
#pragma unroll
          for (int c = 0; c < 4; ++c) val[c] = o[qb][db][4 * j4 + c] * inv;
          *(f32x4 *)(dp + dim0) = val;
        }
      if (a.count) {
        const float cg = gate * th;
        const float *wp = a.count_vec + (size_t)h * kD;
        float *cp = a.count + obase * kD;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            const int dim0 = db * 32 + 8 * j4 + 4 * g32;
            const f32x4 w = *(const f32x4 *)(wp + dim0);
            *(f32x4 *)(cp + dim0) = w * cg;
          }
      }
      if (g32 == 0) {
        a.n_eff[obase] = neff;
        if (a.gate) a.gate[obase] = gate;
        if (a.lse) a.lse[obase] = lse;
      }
    }
  }
}

constexpr int kQbBf16 = 2;
constexpr int kQbF32 = 1;

}  // namespace

int prefill_heads_per_block(int G) {
  if (G % 4 == 0) return 4;
  if (G % 2 == 0) return 2;
  return 1;
}

int prefill_rows_per_block(int dtype, int hb) {
  const int qb = dtype == 1 ? kQbBf16 : kQbF32;
  return (kWaves / hb) * 32 * qb;
}

hipError_t launch_prefill(int dtype, const PrefillArgs &a, hipStream_t stream) {
  const int NY = a.Hkv * (a.G / a.hb);
  const long long blocks = (long long)a.n_row_blocks * NY * a.B;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)blocks), block(kThreads);
  if (dtype == 1)
    hipLaunchKernelGGL((polar_prefill_kernel<Bf16, kQbBf16>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((polar_prefill_kernel<F32, kQbF32>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace polar
