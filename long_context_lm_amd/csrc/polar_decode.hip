// GQA-grouped paged decode of Polar Attention for gfx950.
//
// Follows the decode kernel of the ATMA technical summary (gist.science), section 2.2
// "Hardware-Software Codesign": the kernel reads paged KV cache blocks directly, and the
// query heads that share a KV head are served together, so each K/V byte is read from
// HBM once for all of them (the pages' 4x traffic saving at 16 query / 4 KV heads).
//
// Split kernel: one wave per (sequence b, KV head g, chunk of up to 16 query heads, split
// of consecutive pages).  Per 64-token page:
//   * the K page is read straight from HBM into MFMA A fragments (16 B per lane),
//     S^T = K Q^T on 16x16 MFMA with the group's queries as the 16 columns;
//   * masked keys (past seq_len, or a page id outside the pool) get -inf;
//   * online max / sum / sum-of-squares with a lazily raised reference, as in prefill;
//   * the V page is read once, transposed through LDS, and O^T += V^T P^T on MFMA.
// Each split writes (reference, max score, S, Q, u[64]) per query head to the workspace.
// Combine kernel: one workgroup per (b, query head) merges the splits with factors
// 2^(M_s-R) (squared for Q), each wave a contiguous share of them, and applies the
// direction / count epilogue with n = seq_len.
#include <mutex>

#include "polar_kernels.h"
#include "polar_mfma.h"

namespace polar {
namespace {

constexpr int kD = kHeadDim;
constexpr int kP = kPageSize;
constexpr int kEntry = 68;        // floats per (b, head, split) partial
constexpr float kLazyTheta = 8.0f;
constexpr int kTargetWaves = 4096;
// Splits shorter than kMinPagesPerSplit pages are used only to reach kMinWaves: at B = 1,
// L = 256K, 512 splits of 8 pages per KV head took 46.7 us (split + combine) against 49.3
// with 1024 of 4 and 60.7 with 256 of 16; at B = 16, 64 splits of 64 pages stay (32 of 128
// were 1% slower).
constexpr int kMinWaves = 2048;
constexpr int kMinPagesPerSplit = 8;
constexpr int kCombineWaves = 16;   // waves per (b, head) merge

template <class TR> struct DecCfg;
template <> struct DecCfg<Bf16> { static constexpr int vrow = 72; };
template <> struct DecCfg<F32> { static constexpr int vrow = 65; };

// Position of page key k (0..63) in a transposed V row: the kpl keys one lane feeds to one
// 16x16 P.V MFMA are adjacent.  Lane group j (= lane/16) of MFMA t supplies slots
// e = 0..kpl-1 for keys 16*(i/4) + 4*j + i%4 with i = t*kpl + e.
template <int KPL>
__device__ __forceinline__ int vpos64(int k) {
  const int kb = k >> 4, j = (k >> 2) & 3, r = k & 3;
  const int i = 4 * kb + r;
  return (i / KPL) * (4 * KPL) + j * KPL + (i % KPL);
}

__device__ __forceinline__ float quarter_max(float x) {   // over lanes l, l^16, l^32, l^48
  x = fmaxf(x, __shfl_xor(x, 16));
  return half_max(x);
}
__device__ __forceinline__ float quarter_sum(float x) {
  x = x + __shfl_xor(x, 16);
  return half_sum(x);
}

template <class TR>
__global__ void __launch_bounds__(64) polar_decode_split_kernel(DecodeArgs a) {
  using E = typename TR::elem_t;
  using F = typename TR::frag_t;
  constexpr int KPL = TR::kpl, KSTEP = 4 * KPL, NKS = kD / KSTEP, NT = 16 / KPL;
  constexpr int VROW = DecCfg<TR>::vrow;
  __shared__ __attribute__((aligned(16))) E Vs[kD * VROW];

  const int lane = threadIdx.x, g16 = lane >> 4, c16 = lane & 15;
  const int split = blockIdx.x;
  const int g = blockIdx.y / a.n_hchunk, hc = blockIdx.y % a.n_hchunk;
  const int b = blockIdx.z;
  const int hcol = hc * 16 + c16;                     // query head inside the group
  const bool col_ok = hcol < a.G;
  const int h = g * a.G + (col_ok ? hcol : 0);

  const int L = min(max(a.seq_lens[b], 1), a.max_seq_len);
  const int npages = (L + kP - 1) / kP;
  const int p_begin = split * a.pages_per_split;
  const int p_end = min(p_begin + a.pages_per_split, npages);

  const float beta = a.beta ? a.beta[h] : 8.0f;
  const float tau =
      a.inv_log_train > 0.f ? fmaxf(1.0f, logf((float)L) * a.inv_log_train) : 1.0f;
  const float cl2 = beta * tau * kLog2e;

  F qf[NKS];
  {
    const E *qp = (const E *)a.q + ((size_t)b * a.Hq + h) * kD + g16 * KPL;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = col_ok ? TR::load(qp + ks * KSTEP) : TR::zero();
  }

  f32x4 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) o[db][r] = 0.f;
  float Mref = -INFINITY, smax = -INFINITY, Ssum = 0.f, Qsum = 0.f;

  const size_t page_elems = (size_t)kP * kD;
  for (int p = p_begin; p < p_end; ++p) {
    const int phys = a.page_table[(size_t)b * a.stride + p];
    const bool valid = phys >= 0 && phys < a.num_pages;
    const int key0 = p * kP;
    const size_t off = ((size_t)(valid ? phys : 0) * a.Hkv + g) * page_elems;
    const E *kp = (const E *)a.k_cache + off;
    const E *vp = (const E *)a.v_cache + off;

    // S^T = K Q^T, four 16-key blocks.
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s[kb][r] = 0.f;
      if (valid) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const F ka = TR::load(kp + (kb * 16 + c16) * kD + ks * KSTEP + g16 * KPL);
          s[kb] = TR::mma16(ka, qf[ks], s[kb]);
        }
      }
    }
    // V page -> LDS, transposed (all lanes).  Previous page's reads are complete.
    __syncthreads();
    if (valid) {
      if constexpr (KPL == 8) {
        const int dpart = lane & 3, quad = lane >> 2;      // 16 dims x 4 keys per lane
        u32x4 raw[4][2];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          // keys past the sequence end are zeroed: the page tail may hold any bits
          const bool live = key0 + 4 * quad + c < L;
#pragma unroll
          for (int ch = 0; ch < 2; ++ch) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            raw[c][ch] =
                live ? *(const u32x4 *)(vp + (4 * quad + c) * kD + dpart * 16 + ch * 8) : z;
          }
        }
        const int pos = vpos64<KPL>(4 * quad);
#pragma unroll
        for (int dd = 0; dd < 16; ++dd) {
          const int ch = dd >> 3, w = (dd & 7) >> 1, hi = dd & 1;
          uint32_t word[2];
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const uint32_t a0 = raw[2 * pr][ch][w], a1 = raw[2 * pr + 1][ch][w];
            word[pr] = hi ? ((a0 >> 16) | (a1 & 0xFFFF0000u)) : ((a0 & 0xFFFFu) | (a1 << 16));
          }
          uint2 wv = make_uint2(word[0], word[1]);
          *(uint2 *)&Vs[(dpart * 16 + dd) * VROW + pos] = wv;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int ch = lane + 64 * j;
          const int key = ch >> 4, part = ch & 15;
          const u32x4 z = {0u, 0u, 0u, 0u};
          const u32x4 x = key0 + key < L ? *(const u32x4 *)(vp + key * kD + part * 4) : z;
          const int pos = vpos64<KPL>(key);
#pragma unroll
          for (int e = 0; e < 4; ++e) Vs[(part * 4 + e) * VROW + pos] = __uint_as_float(x[e]);
        }
      }
    }
    __syncthreads();

    // Mask keys past the sequence end and whole invalid pages.
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + kb * 16 + 4 * g16 + r;
        if (!valid || key >= L) s[kb][r] = -INFINITY;
      }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = quarter_max(mx);
    smax = fmaxf(smax, mx);
    const float mt = mx * cl2;
    if (mt > Mref + kLazyTheta) {
      const float alpha = fast_exp2(Mref - mt);
      Ssum *= alpha;
      Qsum *= alpha * alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[db][r] *= alpha;
      Mref = mt;
    }
    const float negM = Mref == -INFINITY ? 0.f : -Mref;
    float pv[16];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[kb * 4 + r] = fast_exp2(fmaf(s[kb][r], cl2, negM));
    F pf[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      pf[t] = TR::pack(pv + t * KPL);
      TR::stats(pf[t], Ssum, Qsum);
    }
    if (valid) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const F va = TR::load(&Vs[(db * 16 + c16) * VROW + t * KSTEP + g16 * KPL]);
          o[db] = TR::mma16(va, pf[t], o[db]);
        }
    }
  }

  const float St = quarter_sum(Ssum);
  const float Qt = quarter_sum(Qsum);
  if (col_ok) {
    float *e = a.ws + (((size_t)b * a.Hq + h) * a.n_split + split) * kEntry;
    if (g16 == 0) {
      e[0] = Mref;
      e[1] = smax;
      e[2] = St;
      e[3] = Qt;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) *(f32x4 *)(e + 4 + db * 16 + 4 * g16) = o[db];
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// One workgroup of kCombineWaves waves per (sequence, query head).  All threads find the
// reference R = max of the splits' references (and the row maximum); then wave w merges a
// contiguous share of the splits: lanes own splits for the scalar weights 2^(M_s - R),
// and the value merge walks them 64 at a time, each split's weight read from a lane
// register, into four independent accumulators.  The waves' partial sums are added in a
// fixed order, so the result does not depend on timing.
__global__ void __launch_bounds__(64 * kCombineWaves) polar_decode_combine_kernel(DecodeArgs a) {
  constexpr int NW = kCombineWaves;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pair = blockIdx.x;
  const int b = pair / a.Hq, h = pair % a.Hq;
  const int n = a.n_split;
  const float *e = a.ws + (size_t)pair * n * kEntry;
  __shared__ float red[NW][2];
  __shared__ float part[NW][2 + kD];
  float R = -INFINITY, smax = -INFINITY;
  for (int s = tid; s < n; s += 64 * NW) {
    R = fmaxf(R, e[s * kEntry + 0]);
    smax = fmaxf(smax, e[s * kEntry + 1]);
  }
  R = wave_max(R);
  smax = wave_max(smax);
  if (lane == 0) {
    red[wave][0] = R;
    red[wave][1] = smax;
  }
  __syncthreads();
  R = red[0][0];
  smax = red[0][1];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    R = fmaxf(R, red[i][0]);
    smax = fmaxf(smax, red[i][1]);
  }

  const int per = (n + NW - 1) / NW;
  const int s_begin = min(n, wave * per), s_end = min(n, s_begin + per);
  float S = 0.f, Q = 0.f, u0 = 0.f, u1 = 0.f, u2 = 0.f, u3 = 0.f;
  for (int s0 = s_begin; s0 < s_end; s0 += 64) {
    const int s = s0 + lane;
    float w = 0.f;
    if (s < s_end) {
      const float Ms = e[s * kEntry + 0];
      w = Ms == -INFINITY ? 0.f : fast_exp2(Ms - R);
      S = fmaf(e[s * kEntry + 2], w, S);
      Q = fmaf(e[s * kEntry + 3], w * w, Q);
    }
    const int cnt = min(64, s_end - s0);
    const float *us = e + (size_t)s0 * kEntry + 4 + lane;
    int j = 0;
    for (; j + 8 <= cnt; j += 8) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = us[(j + i) * kEntry];
      u0 = fmaf(x[0], __shfl(w, j + 0), u0);
      u1 = fmaf(x[1], __shfl(w, j + 1), u1);
      u2 = fmaf(x[2], __shfl(w, j + 2), u2);
      u3 = fmaf(x[3], __shfl(w, j + 3), u3);
      u0 = fmaf(x[4], __shfl(w, j + 4), u0);
      u1 = fmaf(x[5], __shfl(w, j + 5), u1);
      u2 = fmaf(x[6], __shfl(w, j + 6), u2);
      u3 = fmaf(x[7], __shfl(w, j + 7), u3);
    }
    for (; j < cnt; ++j) u0 = fmaf(us[j * kEntry], __shfl(w, j), u0);
  }
  S = wave_sum(S);
  Q = wave_sum(Q);
  part[wave][2 + lane] = (u0 + u1) + (u2 + u3);
  if (lane == 0) {
    part[wave][0] = S;
    part[wave][1] = Q;
  }
  __syncthreads();
  if (wave != 0) return;
  S = part[0][0];
  Q = part[0][1];
  float u = part[0][2 + lane];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    S += part[i][0];
    Q += part[i][1];
    u += part[i][2 + lane];
  }
  const int L = min(max(a.seq_lens[b], 1), a.max_seq_len);
  const float beta = a.beta ? a.beta[h] : 8.0f;
  const float tau =
      a.inv_log_train > 0.f ? fmaxf(1.0f, logf((float)L) * a.inv_log_train) : 1.0f;
  const float cnat = beta * tau;
  const float nrm = wave_sum(u * u);
  const float neff = S * S / Q;
  const float lse = (R + log2f(S)) * kLn2;
  const float m_nat = smax * cnat;
  float floor_ = a.null_bias ? a.null_bias[h] : 0.0f;
  if (a.null_floor) floor_ += cnat * 0.125f * sqrtf(2.0f * logf((float)L));
  const float gate = 1.0f / (1.0f + expf(floor_ - m_nat));
  const float n2 = neff * neff;
  const float th = (n2 - 1.0f) / (n2 + 1.0f);
  const float inv = nrm > 0.f ? rsqrtf(nrm) : 0.f;
  const size_t ob = (size_t)b * a.Hq + h;
  a.dir[ob * kD + lane] = u * inv;
  if (a.count) a.count[ob * kD + lane] = gate * th * a.count_vec[(size_t)h * kD + lane];
  if (lane == 0) {
    a.n_eff[ob] = neff;
    if (a.gate) a.gate[ob] = gate;
    if (a.lse) a.lse[ob] = lse;
  }
}

}  // namespace

DecodeGrid decode_grid(int B, int Hq, int Hkv, int max_seq_len) {
  DecodeGrid d;
  const int G = Hq / Hkv;
  d.n_hchunk = (G + 15) / 16;
  const int npages = (max_seq_len + kP - 1) / kP;
  const long long pairs = (long long)(B > 0 ? B : 1) * Hkv * d.n_hchunk;
  long long ns = (kTargetWaves + pairs - 1) / pairs;
  if (ns > npages / kMinPagesPerSplit)
    ns = std::max((kMinWaves + pairs - 1) / pairs, (long long)(npages / kMinPagesPerSplit));
  if (ns > npages) ns = npages;
  if (ns < 1) ns = 1;
  d.pages_per_split = (int)((npages + ns - 1) / ns);
  d.n_split = (npages + d.pages_per_split - 1) / d.pages_per_split;
  return d;
}

// Scratch of the allocation-free decode entry point: the split partials live in this
// device array instead of a caller workspace.  Each GPU the library runs on holds its own
// copy until the process ends; every call on that GPU shares it.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in): the device address is
// looked up once per device with hipGetSymbolAddress and kept.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

hipError_t noalloc_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *per_device[kMaxDevices];
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void *p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with dev current
    if (err != hipSuccess) return err;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

size_t decode_ws_bytes(int B, int Hq, int Hkv, int max_seq_len) {
  const DecodeGrid d = decode_grid(B, Hq, Hkv, max_seq_len);
  return (size_t)B * Hq * d.n_split * kEntry * sizeof(float);
}

hipError_t launch_decode(int dtype, const DecodeArgs &a, hipStream_t stream) {
  if (a.B <= 0) return hipSuccess;
  dim3 grid(a.n_split, a.Hkv * a.n_hchunk, a.B), block(64);
  if (dtype == 1)
    hipLaunchKernelGGL((polar_decode_split_kernel<Bf16>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((polar_decode_split_kernel<F32>), grid, block, 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int pairs = a.B * a.Hq;
  hipLaunchKernelGGL(polar_decode_combine_kernel, dim3(pairs), dim3(64 * kCombineWaves), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace polar
