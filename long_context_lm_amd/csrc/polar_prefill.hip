// Fused causal Polar Attention prefill for gfx950.
//
// Follows the fused kernel of the ATMA technical summary (gist.science), section 2.2
// "Hardware-Software Codesign": participation ratios are computed online in O(block)
// memory with streaming accumulators and squared correction factors, so the T x T
// scores never exist in memory.  The arithmetic per row is section 2.1's direction and
// magnitude channels (definitions in include/polar.h).
//
// Work decomposition (one workgroup = kWaves waves: 8 for bf16, or 16 for the paged split
// instance; 4 for fp32):
//  * a workgroup owns `hb` query heads that share one KV head (GQA) and a block of rows;
//    each wave owns 32*QB consecutive rows of one of those heads;
//  * K and V tiles of 64 keys are staged into LDS through a ring of two or four slots,
//    so every K/V byte brought on chip serves all `hb` heads and all rows of the block.
//    bf16 tiles go
//    global -> LDS directly (buffer loads with the LDS destination), row-major with a
//    16-byte chunk swizzle, and V^T fragments come from the transposing LDS read; fp32
//    tiles, and bf16 keys that still need RoPE, pass through registers (V transposed);
//  * S^T = K Q^T runs on MFMA with K from LDS and Q resident in registers.  The 32x32
//    output puts one query per lane (column) and 16 keys per lane, so the row statistics
//    need one cross-half exchange per tile and the probabilities are already laid out as
//    the B operand of O^T = V^T P^T;
//  * online statistics per row, in log2 units x = beta*tau*log2(e)*<q,k>:
//      running reference M (raised lazily when the tile maximum exceeds it by > 8),
//      S = sum 2^(x-M), Q = sum 2^(2(x-M)), u = sum 2^(x-M) v, and the exact row maximum.
//    Raising the reference rescales S and u by 2^(M_old-M_new) and Q by its square, the
//    squared correction factor of section 2.2;
//  * epilogue: n_eff = S^2/Q, lse, the floor gate, dir = u/|u|, count;
//  * training instances (kModeSave, kModeSaveWin) also keep, per lane, the first key attaining
//    the lane's running maximum score and write |u| and that key (the row's arg-max) for
//    the backward pass, and, when asked, the softmax read-out u itself;
//  * variant instances add a sliding window, RoPE and the plain softmax output: q is
//    rotated as it is loaded, and K either arrives rotated (kModeVariant, rotated once by
//    polar_rope_keys_kernel) or is rotated while each tile is staged through registers
//    (kModeVariantRot); tiles that every row sees whole take the pipelined path;
//  * paged instances (kMode == kModePaged) serve chunked prefill over a paged KV cache: the
//    rows are C new tokens at positions start_pos[b].., and a 64-key tile is one page,
//    read through the page table (pages with invalid ids are masked out);
//  * mixed instances (kMode == kModeMix) compute as the plain ones and write the sum of
//    the three streams of section 2.1, dir + count + memory, instead of dir and count.
#include <mutex>

#include "polar_kernels.h"
#include "polar_mfma.h"
#include "polar_rope.h"

namespace polar {
namespace {

constexpr int kD = kHeadDim;
constexpr int kKTBf16 = 64;   // keys per tile (bf16 instances): one page of the paged cache
constexpr float kLazyTheta = 8.0f;
// Task queues of a ticketed launch; its counter set has one more word, the completion count.
constexpr int kTicketQueues = 15;
// The running reference before any visible key: finite, so that -M needs no select, and so
// low that the first visible tile always raises it (the rescale factor is then 0).
constexpr float kNoRef = -3.0e38f;
constexpr int kBufferFlags = 0x00020000;   // gfx9 buffer resource word 3 (raw dword access)

// Direct (bf16) tiles hold 16-byte chunk c of key row r at slot c ^ tile_swz(r) of the
// row's 128 bytes.  The LDS serves 256 bytes (64 four-byte banks) per cycle:
//  * a K fragment read (ds_read_b128) covers one chunk of 16 consecutive rows per cycle,
//    and the 8 rows of each parity get 8 distinct slots, so the 16 lanes hit 16 distinct
//    16-byte bank groups;
//  * a V^T fragment read (ds_read_b64_tr_b16) covers 4 chunks of 4 consecutive rows per
//    32 lanes; rows two apart differ in bit 2 of the swizzle, so their chunk sets land in
//    different halves of the row's bank groups.
// Rows r and r + 8 (r & 8 == 0) differ by slot bit 1: tile_swz(r + 8) == tile_swz(r) ^ 2.
__device__ __forceinline__ int tile_swz(int r) { return ((r >> 2) & 3) | ((r & 2) << 1); }

template <class TR> struct LdsCfg;
template <> struct LdsCfg<Bf16> {
  static constexpr int kt = kKTBf16, krow = 72, vrow = kKTBf16 + 8;
};
template <> struct LdsCfg<F32> { static constexpr int kt = 64, krow = 68, vrow = 65; };

constexpr int kModePlain = 0, kModeSave = 1, kModeVariant = 2, kModePaged = 3;
// Variant whose keys still need RoPE (no rotated copy): they are rotated while staged
// through registers, so this mode keeps the register staging path.
constexpr int kModeVariantRot = 4;
// Plain prefill writing dir + count + memory as one output (a.mixed).
constexpr int kModeMix = 5;
// The training instance under a sliding window (its own instance, so that the causal
// training forward keeps the code it had without the window).
constexpr int kModeSaveWin = 6;

// The rotated pair, with the contraction spelled out so that every place that rotates a
// key rounds the same way: (x0 c - x1 s, x0 s + x1 c).
__device__ __forceinline__ float rot_re(float x0, float x1, float c, float s) {
  return fmaf(x0, c, -(x1 * s));
}
__device__ __forceinline__ float rot_im(float x0, float x1, float c, float s) {
  return fmaf(x0, s, x1 * c);
}

// kLean: each tile's scores are used in the step that issues them (see kAhead below).  Lean
// instances are held to 128 registers (four waves per SIMD), the training instances with
// their arg-max tracking included.
template <class TR, int QB, int kWaves, int kMode, bool kLean>
__global__ void __launch_bounds__(64 * kWaves, kLean ? 4 : 1)
    polar_prefill_kernel(PrefillArgs a) {
  constexpr bool kSave = kMode == kModeSave || kMode == kModeSaveWin;
  constexpr bool kVar = kMode == kModeVariant || kMode == kModeVariantRot;
  constexpr bool kPaged = kMode == kModePaged;
  constexpr bool kMix = kMode == kModeMix;
  // The sliding window: variant instances, and the windowed training instance (which takes
  // q and k already rotated when RoPE is on).
  constexpr bool kWin = kVar || kMode == kModeSaveWin;
  // Instances that can also write the softmax read-out u (a.attn, when non-NULL).
  constexpr bool kAttn = kVar || kSave;
  static_assert(!kPaged || LdsCfg<TR>::kt == kPageSize, "a key tile is one page");
  constexpr int kThreads = 64 * kWaves;
  constexpr int kKT = LdsCfg<TR>::kt;                // keys per tile
  constexpr int NKB = kKT / 32;                      // 32-key MFMA blocks per tile
  using E = typename TR::elem_t;
  using F = typename TR::frag_t;
  constexpr int KPL = TR::kpl, KSTEP = 2 * KPL, NKS = kD / KSTEP, NT = 16 / KPL;
  constexpr int KROW = LdsCfg<TR>::krow, VROW = LdsCfg<TR>::vrow;
  constexpr int VEC = TR::vec;                       // elements per 16-byte chunk
  constexpr int CPR = kD / VEC;                      // chunks per key row
  // bf16 tiles go global -> LDS directly (buffer_load ... lds), unpadded, with the 16-byte
  // chunks of key row k stored in slot order chunk ^ (k & 7) so that fragment reads spread
  // over the banks; K fragments are read as rows, V^T fragments with the transposing
  // ds_read_b64_tr_b16.  Other instances stage through registers into padded tiles (V
  // transposed on the way).
  // Split instance (paged, lean, 16 waves): waves w and w + 8 own the same rows and head;
  // the first eight take the first half of the fully visible tiles, the other eight the
  // rest, and the halves merge through LDS at the end.
  constexpr bool kSplit = kPaged && kLean && kWaves == 16;
  constexpr int kRowWaves = kSplit ? 8 : kWaves;     // waves that own distinct rows
  constexpr bool kDirect =
      KPL == 8 && kMode != kModeVariantRot && kKT == 64 && (kWaves == 8 || kSplit);
  static_assert(!kSplit || QB == 1, "split instance: one query block per wave");
  constexpr int kSlotBytes = kDirect ? 2 * kKT * kD * (int)sizeof(E)
                                     : (kKT * KROW + kD * VROW) * (int)sizeof(E);
  // Tile t + kDepth is loaded during step t; the ring holds tiles t .. t + kDepth.  Direct
  // loads cost no registers, so they run further ahead than the register staging.
  // Scores run two tiles ahead of their probabilities, so that no vector instruction waits
  // on a recent MFMA result.  Lean instances use each tile's scores in the step that issues
  // them: with one score buffer instead of three they fit 128 registers, two workgroups
  // share each CU (four waves per SIMD), and the other workgroup's waves, whose barriers
  // fall elsewhere, cover the score MFMAs' latency.
  static_assert(!kLean || kDirect, "lean instances stage direct tiles");
  constexpr int kAhead = kLean ? 0 : 2;
  constexpr int kDepth = kDirect ? kAhead + 1 : 3;
  constexpr int kSlots = kDepth + 1;
  static_assert(kAhead == 0 || kAhead == 2, "scores in the same step or two tiles ahead");
  static_assert(kDepth >= kAhead + 1 && 2 * (kDepth - kAhead - 1) < 16, "loads in flight < 16");
  // The split merge reuses the rings' LDS after the last barrier: no tile load may still be
  // in flight then, which holds when each step waits for all of its loads (one tile ahead).
  static_assert(!kSplit || kDepth == 1, "split instance loads one tile ahead");
  constexpr int kXchBytes = 8 * 36 * 64 * (int)sizeof(float);   // split merge: 36 values/lane
  constexpr int kRingBytes = kSlots * kSlotBytes;
  // Lean instances (plain, training, mixed, variant) write their vector outputs as whole
  // 256-byte rows with non-temporal stores: each wave's 32 rows go through LDS (the registers hold 16-byte pieces of 32
  // rows), in the ring's space once every tile load has landed.  Whole lines bypass the
  // L2, so the launch does not end on a write-back of the outputs: at B = 8, T = 2K
  // 125 -> 117 us.  (Non-temporal stores of the 16-byte pieces were 60% slower; whole rows
  // through the L2 gained nothing.)
  constexpr bool kRowStores = kLean && (kMode == kModePlain || kSave ||
                                        kMode == kModeMix || kMode == kModeVariant);
  constexpr int kOutPitch = kD + 4;                 // floats per staged row (spreads banks)
  constexpr int kOutBytes = kRowStores ? kWaves * 32 * kOutPitch * (int)sizeof(float) : 0;
  constexpr int kBase = kSplit ? (2 * kRingBytes > kXchBytes ? 2 * kRingBytes : kXchBytes)
                               : kRingBytes;
  constexpr int kSmemBytes = kBase > kOutBytes ? kBase : kOutBytes;
  __shared__ __attribute__((aligned(128))) char smem[kSmemBytes];
  auto Ks = reinterpret_cast<E (*)[kKT * KROW]>(smem);
  auto Vs = reinterpret_cast<E (*)[kD * VROW]>(smem + 4 * kKT * KROW * sizeof(E));

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = kSplit ? (wave >> 3) : 0;          // split instance: key-range half
  const int wv = kSplit ? (wave & 7) : wave;         // row-owning wave index
  char *const gsmem = smem + grp * kRingBytes;       // this half's ring
  const int g32 = lane >> 5, c32 = lane & 31;

  // Heaviest row blocks first; consecutive blocks cycle over (batch, KV head), the
  // task's group.  With tickets, workgroups take tasks in the order they start rather
  // than in workgroup order, from queues of their own groups: the hardware deals
  // workgroups to the eight XCDs round robin, so a workgroup's grid position fixes its
  // group (and the K/V its XCD's L2 holds); it takes the next row block of its queue
  // (the groups g with g % Q equal to its own), heaviest first, and once that queue is
  // empty, the next of the other queues in turn.  An XCD that runs faster then starts its
  // next workgroups sooner and takes more of its groups' work, and at the end the light
  // tail of the others, instead of idling while the slowest XCD finishes its fixed share.
  const int n_hc = a.G / a.hb;
  const int NY = a.Hkv * n_hc;
  // Only the plain lean instance is ever launched with tickets (the others keep exactly
  // the code they had without them).
  constexpr bool kTicketed = kMode == kModePlain && kLean;
  __shared__ int s_task;
  int id = blockIdx.x;
  if (kTicketed && a.ticket) {
    if (tid == 0) {
      const int GY = a.B * NY;                           // groups
      const int Q = min(GY, kTicketQueues);              // queues
      const int home = (int)(blockIdx.x % (unsigned)GY) % Q;
      int task = (int)blockIdx.x;        // unreachable fallback: a repeat writes equal values
      for (int i = 0; i < Q; ++i) {
        const int q = (home + i) % Q;
        const int cnt = (GY - q + Q - 1) / Q;              // groups q, q + Q, ...
        const unsigned j = atomicAdd(a.ticket + q, 1u);
        if (j < (unsigned)(cnt * a.n_row_blocks)) {
          task = (int)(j / cnt) * GY + q + Q * (int)(j % cnt);
          break;
        }
      }
      s_task = task;
    }
    __syncthreads();
    id = s_task;
  }
  const int b = id % a.B;
  id /= a.B;
  const int y = id % NY;
  const int rb = a.n_row_blocks - 1 - id / NY;
  const int g = y / n_hc, hc = y % n_hc;
  const int h = g * a.G + hc * a.hb + (wv % a.hb);
  const int WR = (kRowWaves / a.hb) * 32 * QB;
  const int row0 = rb * WR;
  const int wrow0 = row0 + (wv / a.hb) * 32 * QB;
  // Row r of this sequence sits at position pbase + r (pbase = 0 outside paged instances).
  const int pbase = kPaged ? min(max(a.start_pos[b], 0), a.max_seq_len - a.T) : 0;
  const int wg_last = min(row0 + WR, a.T) - 1;
  const int w_last = wrow0 < a.T ? pbase + min(wrow0 + 32 * QB, a.T) - 1 : -1;
  const int ntiles = (pbase + wg_last) / kKT + 1;

  // K and V rows of this (b, g) through buffer resources sized to the sequence, so loads
  // of keys >= T return zeros without a branch.
  const size_t kv_row_bytes = (size_t)a.Hkv * kD * sizeof(E);
  const size_t kv_base = ((size_t)b * a.T * a.Hkv + g) * kD;
  const int kv_bytes = (int)(((size_t)a.T * a.Hkv - g) * kD * sizeof(E));
  const E *const kbase = (const E *)a.k + kv_base, *const vbase = (const E *)a.v + kv_base;
  const auto krsrc = __builtin_amdgcn_make_buffer_rsrc((void *)kbase, 0, kv_bytes, kBufferFlags);
  const auto vrsrc = __builtin_amdgcn_make_buffer_rsrc((void *)vbase, 0, kv_bytes, kBufferFlags);

  // Per-row logit scales: natural units and log2 units.
  const float beta = a.beta ? a.beta[h] : 8.0f;
  float cnat[QB], cl2[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wrow0 + qb * 32 + c32;
    const int nk = (kWin && a.window > 0) ? min(row + 1, a.window) : pbase + row + 1;
    const float tau =
        a.inv_log_train > 0.f ? fmaxf(1.0f, logf((float)nk) * a.inv_log_train) : 1.0f;
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
    if constexpr (kVar) {
      if (a.rope) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          if constexpr (KPL == 8) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              float c, sn;
              rope_cs(a.rope_f[ks * 8 + g32 * 4 + m], row, c, sn);
              const float x0 = (float)qf[qb][ks][2 * m], x1 = (float)qf[qb][ks][2 * m + 1];
              qf[qb][ks][2 * m] = (__bf16)rot_re(x0, x1, c, sn);
              qf[qb][ks][2 * m + 1] = (__bf16)rot_im(x0, x1, c, sn);
            }
          } else {
            // fp32: lanes l and l^32 hold the two elements of pair ks.
            float c, sn;
            rope_cs(a.rope_f[ks], row, c, sn);
            const float x = qf[qb][ks], other = half_other(x);
            qf[qb][ks] = x * c + (g32 ? other * sn : -other * sn);
          }
        }
      }
    }
  }

  f32x16 o[QB][2];
  float Mref[QB], smax[QB], Ssum[QB], Qsum[QB];
  float lbest[QB];                          // kSave: this lane's best score so far
  int lkey[QB];                             // kSave: first key attaining it
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.f;
    Mref[qb] = kNoRef;
    smax[qb] = -INFINITY;
    lbest[qb] = -INFINITY;
    lkey[qb] = 0;
    Ssum[qb] = 0.f;
    Qsum[qb] = 0.f;
  }

  // ---- K/V staging: global -> registers -> LDS (V transposed) ----
  // K: 16-byte chunks, copied as is.  V (bf16): tasks of 2 keys x 4 dims (two 8-byte loads)
  // so every thread of a 512-thread workgroup does one V task and one K chunk per tile, and
  // each pair of keys lands in one LDS word of the transposed tile.  Keys vary fastest
  // across lanes, which keeps the transposed writes on distinct banks.  V (fp32): 16-byte
  // chunks scattered element by element.
  constexpr int KTASKS = kKT * CPR;
  constexpr int VDIMS = KPL == 8 ? 4 : VEC;          // dims per V task
  constexpr int VKEYS = KPL == 8 ? 2 : 1;            // keys per V task
  constexpr int VKG = kKT / VKEYS;                   // V tasks per dim group
  constexpr int VTASKS = VKG * (kD / VDIMS);
  constexpr int NK = (KTASKS + kThreads - 1) / kThreads;
  constexpr int NV = (VTASKS + kThreads - 1) / kThreads;
  typedef uint32_t vchunk_t __attribute__((ext_vector_type(KPL == 8 ? 2 : 4)));
  u32x4 kst[NK];
  vchunk_t vst[NV][VKEYS];
  int staged_key0 = 0;                               // variant: position of the staged tile
  // This wave's part of a direct tile in LDS (uniform: one scalar register).
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(lds_addr(gsmem) + wv * 1024);
  int tok[kSlots];                                   // paged: slot holds a valid page
#pragma unroll
  for (int i = 0; i < kSlots; ++i) tok[i] = 1;
  auto stage_load = [&](int t) {
    const int key0 = t * kKT;
    staged_key0 = key0;
    // Tile source: rows of this (b, g) in place, or (paged) one page of the pools.
    auto rk = krsrc, rv = vrsrc;
    int base = (int)((size_t)key0 * kv_row_bytes), rstride = (int)kv_row_bytes;
    if constexpr (kPaged) {
      const int npg = min(a.stride, (pbase + a.T + kPageSize - 1) / kPageSize);
      // A scalar load (the index is uniform): it does not count against vmcnt, which the
      // direct tiles' wait relies on.
      const int tu = __builtin_amdgcn_readfirstlane(t);
      const int page =
          tu < npg ? a.page_table[(size_t)__builtin_amdgcn_readfirstlane(b) * a.stride + tu] : -1;
      const bool pok = page >= 0 && page < a.num_pages;
      tok[t % kSlots] = pok;
      const size_t pe = ((size_t)(pok ? page : 0) * a.Hkv + g) * kPageSize * kD;
      const int nb = pok ? kPageSize * kD * (int)sizeof(E) : 0;
      rk = __builtin_amdgcn_make_buffer_rsrc((void *)((const E *)a.k + pe), 0, nb, kBufferFlags);
      rv = __builtin_amdgcn_make_buffer_rsrc((void *)((const E *)a.v + pe), 0, nb, kBufferFlags);
      base = 0;
      rstride = kD * (int)sizeof(E);
    }
    if constexpr (kDirect) {
      // Wave w moves keys 8w..8w+7 of K and of V: lane l takes key 8w + l/8 and the chunk
      // that belongs in slot l%8 of that row, and the hardware writes lane l's 16 bytes at
      // the wave's LDS base + 16 l.  The lane's offset inside a tile is fixed: the tile's
      // start moves the (scalar) buffer resource instead, whose size still ends at the
      // sequence's last key, so keys past it read zeros.  The LDS destination is uniform.
      if constexpr (!kPaged) {
        const int toff = key0 * (int)kv_row_bytes;
        const int rem = max(kv_bytes - toff, 0);
        rk = __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)kbase + toff), 0, rem,
                                               kBufferFlags);
        rv = __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)vbase + toff), 0, rem,
                                               kBufferFlags);
      }
      const int key = 8 * wv + (lane >> 3);
      const int loff = key * rstride + (((lane & 7) ^ tile_swz(key)) << 4);
      const uint32_t dst = wave_lds + (uint32_t)((t % kSlots) * kSlotBytes);
      using lds_void = __attribute__((address_space(3))) void *;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void)(uintptr_t)dst, 16, loff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (lds_void)(uintptr_t)(dst + kKT * kD * sizeof(E)), 16, loff, 0, 0, 0);
      return;
    }
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int ch = min(tid + kThreads * j, KTASKS - 1);
      const int key = ch / CPR, part = ch % CPR;
      kst[j] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, base + key * rstride + part * 16, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int ti = min(tid + kThreads * j, VTASKS - 1);
      const int part = ti / VKG;
#pragma unroll
      for (int r = 0; r < VKEYS; ++r) {
        const int key = (ti % VKG) * VKEYS + r;
        const int off = base + key * rstride + part * VDIMS * (int)sizeof(E);
        if constexpr (KPL == 8)
          vst[j][r] = __builtin_bit_cast(vchunk_t,
                                         __builtin_amdgcn_raw_buffer_load_b64(rv, off, 0, 0));
        else
          vst[j][r] = __builtin_bit_cast(vchunk_t,
                                         __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
      }
    }
  };
  auto stage_store = [&](int slot, int vslot) {
    if constexpr (kDirect) {
      // The tiles go straight to LDS.  Wait until this wave's loads of the tile needed next
      // (t + 1 + kAhead after step t) have landed: every call issues two loads (K and V)
      // per tile, so those of the kDepth - kAhead - 1 tiles after it may still be in
      // flight.  The caller's barrier then publishes the tile.
      __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * (kDepth - kAhead - 1)));
      return;
    }
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int ch = tid + kThreads * j;
      const int key = ch / CPR, part = ch % CPR;
      if constexpr (kVar) {
        if (a.rope && !a.k_rotated) {
          // Rotate the staged chunk: pairs (2t, 2t+1) of key position staged_key0 + key.
          const int pos = staged_key0 + key;
#pragma unroll
          for (int m = 0; m < (KPL == 8 ? 4 : 2); ++m) {
            float c, sn, x0, x1;
            if constexpr (KPL == 8) {
              rope_cs(a.rope_f[part * 4 + m], pos, c, sn);
              x0 = __uint_as_float(kst[j][m] << 16);
              x1 = __uint_as_float(kst[j][m] & 0xFFFF0000u);
              const bf16x2 r = {(__bf16)rot_re(x0, x1, c, sn), (__bf16)rot_im(x0, x1, c, sn)};
              kst[j][m] = __builtin_bit_cast(uint32_t, r);
            } else {
              rope_cs(a.rope_f[part * 2 + m], pos, c, sn);
              x0 = __uint_as_float(kst[j][2 * m]);
              x1 = __uint_as_float(kst[j][2 * m + 1]);
              kst[j][2 * m] = __float_as_uint(rot_re(x0, x1, c, sn));
              kst[j][2 * m + 1] = __float_as_uint(rot_im(x0, x1, c, sn));
            }
          }
        }
      }
      if (NK * kThreads == KTASKS || ch < KTASKS)
        *(u32x4 *)&Ks[slot][key * KROW + part * VEC] = kst[j];
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int ti = tid + kThreads * j;
      if (NV * kThreads != VTASKS && ti >= VTASKS) continue;
      const int part = ti / VKG;
      const int key = (ti % VKG) * VKEYS;
      const int pos = (key >> 5) * 32 + vpos32<KPL>(key & 31);
      if constexpr (KPL == 8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w0 = vst[j][0][e >> 1], w1 = vst[j][1][e >> 1];
          const uint32_t word = (e & 1) ? ((w0 >> 16) | (w1 & 0xFFFF0000u))
                                        : ((w0 & 0xFFFFu) | (w1 << 16));
          *(uint32_t *)&Vs[vslot][(part * 4 + e) * VROW + pos] = word;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Vs[vslot][(part * 4 + e) * VROW + pos] = __uint_as_float(vst[j][0][e]);
      }
    }
  };

  // Per-lane LDS read offsets.  The per-step base passes through an empty asm so the
  // compiler materialises one address per step and folds the fragment offsets inside a
  // tile into the instructions' immediate fields.
  const uint32_t k_lane = (uint32_t)((c32 * KROW + g32 * KPL) * sizeof(E));
  const uint32_t v_lane = (uint32_t)((c32 * VROW + g32 * KPL) * sizeof(E));
  constexpr uint32_t KSLOT = kKT * KROW * sizeof(E), VSLOT = kD * VROW * sizeof(E);
  // Direct tiles: byte offsets of this lane's fragments inside a slot.  K fragment (kb, ks):
  // key kb*32 + c32, chunk 2 ks + g32.  V^T fragment (kb, tt, db), half h: lane i of 16-lane
  // group G reads 4 dims of key kb*32 + 16 tt + 8 h + 4 (G/2) + i/4 and, transposed, holds
  // dim 32 db + (lane % 32) of keys ... + 4 (lane / 32) + 0..3, the slot order of P.  The
  // swizzle of a row depends on its index mod 16, so one offset serves every kb and tt;
  // the h = 1 rows (8 further on) have slot bit 1 flipped: address bit 5 (slot and ring
  // bases are multiples of 128 bytes, the LDS array starts at address 0).
  // The K offsets of the four chunk pairs differ only in slot bits 1 and 2: chunk 2 ks + g32
  // sits at kofs0 ^ (32 ks).
  static_assert(kSlotBytes % 128 == 0 && kRingBytes % 128 == 0, "row-aligned slots");
  uint32_t kofs0, vofs[2];
  {
    const int sw = tile_swz(c32);
    kofs0 = (uint32_t)(c32 * 128 + ((g32 ^ sw) << 4));
    const int G4 = lane >> 4, i = lane & 15;
    const int krow = 4 * (G4 >> 1) + (i >> 2);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int chunk = 4 * db + 2 * (G4 & 1) + ((i & 3) >> 1);
      vofs[db] = (uint32_t)(kKT * kD * sizeof(E) + krow * 128 + ((chunk ^ tile_swz(krow)) << 4) +
                            (i & 1) * 8);
    }
  }
  auto lds_at = [](const E *base, uint32_t off) {
    asm volatile("" : "+v"(off));
    return reinterpret_cast<const E *>(reinterpret_cast<const char *>(base) + off);
  };
  // K fragment row addresses of the four chunk pairs, (kofs0 ^ 32 ks) + slot base, each
  // formed by one instruction in the step that uses it (no per-slot addresses are held
  // across the loop; the kb offset stays an immediate of the reads).  The slot base is a
  // multiple of 128, so ks = 2, 3 flip bit 6 of the ks = 0, 1 addresses (inline operands
  // only: 96 would be a literal).
  using lds_frag = const __attribute__((address_space(3))) F *;
  auto k_addrs = [&](const char *sb, lds_frag (&kp)[4]) {
    uint32_t a0, a1, a2, a3;
    const uint32_t base = lds_addr(sb);
    asm volatile("v_add_u32 %0, %1, %2" : "=v"(a0) : "s"(base), "v"(kofs0));
    asm volatile("v_xad_u32 %0, %1, 32, %2" : "=v"(a1) : "v"(kofs0), "s"(base));
    asm volatile("v_xor_b32 %0, 64, %1" : "=v"(a2) : "v"(a0));
    asm volatile("v_xor_b32 %0, 64, %1" : "=v"(a3) : "v"(a1));
    kp[0] = (lds_frag)(uintptr_t)a0;
    kp[1] = (lds_frag)(uintptr_t)a1;
    kp[2] = (lds_frag)(uintptr_t)a2;
    kp[3] = (lds_frag)(uintptr_t)a3;
  };

  // ---- per-tile building blocks ----
  struct Scores { f32x16 v[QB][NKB]; };
  struct Probs { F v[QB][NKB][NT]; };
  // S^T = K Q^T for the two 32-key blocks of a tile.
  // Independent accumulation chains are issued round-robin (a dependent MFMA waits for
  // its predecessor's result).
  auto score = [&](int slot, Scores &S) {
    const f32x16 zero = {};
    if constexpr (kDirect) {
      static_assert(NKS == 4, "a direct key row is four chunk pairs");
      lds_frag kpa[4];
      k_addrs(gsmem + slot * kSlotBytes, kpa);
      // One 32-key block's chain after the other, so that the maximum over the first block
      // runs beside the second block's MFMAs: 8.74 ms at T = 64K against 8.81 with the two
      // chains interleaved.  The split paged instance keeps them interleaved (1.36 ms
      // against 1.37 for a 4096-token chunk).
#pragma unroll
      for (int i = 0; i < NKS * NKB; ++i) {
        const int kb = kPaged ? i % NKB : i / NKS, ks = kPaged ? i / NKB : i % NKS;
        const F ka = kpa[ks][kb * 32 * 128 / (int)sizeof(F)];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          S.v[qb][kb] = TR::mma32(ka, qf[qb][ks], ks == 0 ? zero : S.v[qb][kb]);
      }
    } else {
    const E *Kt = lds_at(&Ks[0][0], k_lane + slot * KSLOT);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const F ka = TR::load(Kt + kb * 32 * KROW + ks * KSTEP);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          S.v[qb][kb] = TR::mma32(ka, qf[qb][ks], ks == 0 ? zero : S.v[qb][kb]);
      }
    }
    if constexpr (kPaged) {
      if (!tok[slot]) {                               // a page with an invalid id
        // The empty volatile statement keeps this rare path a branch: if-converted, it
        // costs one select per score of every tile.
        asm volatile("");
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) S.v[qb][kb][r] = -INFINITY;
      }
    }
  };
  // Causal mask: key > row -> -inf.
  auto mask = [&](Scores &S, int key0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = wrow0 + qb * 32 + c32;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * g32 + (r & 3);
          bool masked = key > pbase + row;
          if constexpr (kWin) masked = masked || (a.window > 0 && key <= row - a.window);
          if (masked) S.v[qb][kb][r] = -INFINITY;
        }
    }
  };
  // Row maximum of a tile's raw scores (both wave halves hold the same row).
  auto tile_max = [&](const Scores &S, int qb) {
    float mx = S.v[qb][0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S.v[qb][kb][r]);
    return half_max(mx);
  };
  // kSave: keep the lowest key attaining this lane's maximum.  Tiles arrive in key order
  // and a lane's registers in increasing key order, so a strict improvement picks the
  // first occurrence.  Lanes rarely improve after the first tiles.
  auto track = [&](const Scores &S, int qb, int key0) {
    if constexpr (kSave) {
      float mx = S.v[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S.v[qb][kb][r]);
      if (mx > lbest[qb]) {
        asm volatile("");     // a branch, not selects: lanes rarely improve after a few tiles
        // The offset of the lowest register holding the maximum, as a small literal (one
        // select per register), then the lane's base key added once.
        int off = 0;
#pragma unroll
        for (int kb = NKB - 1; kb >= 0; --kb)
#pragma unroll
          for (int r = 15; r >= 0; --r)
            if (S.v[qb][kb][r] == mx) off = kb * 32 + 8 * (r >> 2) + (r & 3);
        lbest[qb] = mx;
        lkey[qb] = key0 + 4 * g32 + off;
      }
    }
  };
  // Raise the reference when the tile maximum passes it by more than the lazy threshold:
  // u and S scale by 2^(M_old - M_new), Q by the square of that factor.
  auto raise_ref = [&](int qb, float mt) {
    if (mt > Mref[qb] + kLazyTheta) {
      const float alpha = fast_exp2(Mref[qb] - mt);
      const float alpha2 = alpha * alpha;
      Ssum[qb] *= alpha;
      Qsum[qb] *= alpha2;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
      Mref[qb] = mt;
    }
  };
  // p = 2^(x - M), rounded for the P.V product (and the matrix statistics).
  auto probs = [&](const Scores &S, Probs &P) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float negM = -Mref[qb];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float pv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) pv[r] = fast_exp2(fmaf(S.v[qb][kb][r], cl2[qb], negM));
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) P.v[qb][kb][tt] = TR::pack(pv + tt * KPL);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) TR::stats(P.v[qb][kb][tt], Ssum[qb], Qsum[qb]);
      }
    }
  };
  // O^T += V^T P^T
  auto pv_mma = [&](int slot, const Probs &P) {
    if constexpr (kDirect && !kPaged) {
      // One asm block per 32-dimension half (see tr_read_tile).  The paged instance keeps
      // the builtin below: with the block's full LDS wait it was 4% slower, as the wait
      // also covers the page-id load issued at the start of the step.
      static_assert(NKB == 2 && NT == 2, "a direct tile is two 32-key blocks of two halves");
      const char *sb = gsmem + slot * kSlotBytes;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        F va[4];
        const uint32_t lo = lds_addr(sb) + vofs[db];
        tr_read_tile(lo, (lo ^ 32u) + 8 * 128, va);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              o[qb][db] = TR::mma32(va[2 * kb + tt], P.v[qb][kb][tt], o[qb][db]);
      }
      return;
    }
    if constexpr (kDirect) {
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      using lds_v4 = __attribute__((address_space(3))) s16x4 *;
      const uint32_t sbase = lds_addr(gsmem + slot * kSlotBytes);
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        uint32_t lo = sbase + vofs[db];
        asm volatile("" : "+v"(lo));
        const uint32_t hi = (lo ^ 32u) + 8 * 128;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            const uint32_t r0 = (kb * 32 + 16 * tt) * 128;
            const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(uintptr_t)(lo + r0));
            const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(uintptr_t)(hi + r0));
            const F va = __builtin_bit_cast(F, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) o[qb][db] = TR::mma32(va, P.v[qb][kb][tt], o[qb][db]);
          }
      }
      return;
    }
    const E *Vt = lds_at(&Vs[0][0], v_lane + slot * VSLOT);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const F va = TR::load(Vt + db * 32 * VROW + kb * 32 + tt * KSTEP);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][db] = TR::mma32(va, P.v[qb][kb][tt], o[qb][db]);
        }
  };

  // ---- software-pipelined key loop ----
  // On gfx950 a wave waiting to issue an MFMA also holds back VALU issue of the other wave
  // on its SIMD, so matrix and vector work overlap inside each wave's own instruction
  // stream.  With scores two tiles ahead (8-wave instances), step t issues the scores of
  // tile t+2 (MFMA) beside tile t's probabilities (VALU), then tile t's P.V product beside
  // the maximum of tile t+1, whose scores were issued a whole step earlier, so no VALU
  // instruction waits on a recent MFMA result; K and V use four LDS slots (tile t+3 is
  // stored while tiles t..t+2 are live).  Lean instances take each tile whole in one step
  // (scores, maximum, probabilities, P.V) and leave the overlap to the other workgroup on
  // the CU; two slots.  Tiles fully below the workgroup's first row need no mask;
  // the diagonal tiles run one at a time.
  // Tiles [tf0, tf1) are seen whole by every row of the workgroup and take this pipelined
  // path; the others are masked one at a time.  With a sliding window the loop starts at
  // the first tile any row can see (t0) and the fully visible range starts at tf0.
  const int t0 = (kWin && a.window > 0) ? max(0, row0 - a.window + 1) / kKT : 0;
  const int tf1 = min((pbase + row0 + 1) / kKT, ntiles);
  const int tf0 = (kWin && a.window > 0)
                      ? min(tf1, (max(0, wg_last - a.window + 1) + kKT - 1) / kKT)
                      : t0;

  // Split instance: the first half owns tiles [t0, tm), the second [tm, ntiles).
  const int tm = kSplit ? tf1 / 2 : t0;
  const int tb = (kSplit && grp) ? tm : t0;
  if constexpr (kDirect) {
    // Every step issues one tile's loads, past the sequence end too (they read zeros), so
    // the count of loads in flight after any tile is fixed.
    for (int j = tb; j < tb + kDepth; ++j) stage_load(j);
    stage_store(0, 0);
  } else {
    for (int j = t0; j < t0 + 3 && j < ntiles; ++j) {
      stage_load(j);
      stage_store(j % 4, j % 4);
    }
  }
  __syncthreads();

  Scores Sa, Sb, Sc;
  Probs P;
  auto first_max = [&](const Scores &Sx, int key0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      track(Sx, qb, key0);
      const float mx = tile_max(Sx, qb);
      smax[qb] = fmaxf(smax[qb], mx);
      raise_ref(qb, mx * cl2[qb]);
    }
  };
  // One masked tile (window edges, diagonal, keys past the sequence).
  auto masked_step = [&](int t) {
    const bool stage = kDirect || t + 3 < ntiles;
    if (stage) stage_load(t + kDepth);
    const int key0 = t * kKT;
    bool live = key0 <= w_last;
    if constexpr (kWin) live = live && (a.window == 0 || key0 + kKT > wrow0 - a.window + 1);
    if (live) {
      score(t % kSlots, Sa);
      mask(Sa, key0);
      first_max(Sa, key0);
      probs(Sa, P);
      pv_mma(t % kSlots, P);
    }
    if (stage) stage_store((t + 3) % kSlots, (t + 3) % kSlots);
    __syncthreads();
  };

  int t = t0;
  for (; t < tf0; ++t) masked_step(t);

  if (kAhead > 0 && tf1 > tf0) {
    score(tf0 % kSlots, Sa);
    first_max(Sa, tf0 * kKT);
  }
  if (kAhead == 2 && tf1 > tf0 + 1) score((tf0 + 1) % kSlots, Sb);

  auto pipe_step = [&](int t, Scores &S0, Scores &S1, Scores &S2) {
    const bool stage = kDirect || t + 3 < ntiles;
    stage_load(t + kDepth);  // unconditional: loads past the sequence return zeros
    score((t + 2) % kSlots, S2);
    probs(S0, P);
    pv_mma(t % kSlots, P);
    const bool next_full = t + 1 < tf1;
    float mxs[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mxs[qb] = tile_max(S1, qb);
    if (next_full) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) track(S1, qb, (t + 1) * kKT);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      smax[qb] = next_full ? fmaxf(smax[qb], mxs[qb]) : smax[qb];
      raise_ref(qb, next_full ? mxs[qb] * cl2[qb] : -INFINITY);
    }
    if (stage) stage_store((t + 3) % kSlots, (t + 3) % kSlots);
    __syncthreads();
  };

  if constexpr (kSplit) {
    // Both halves take the same number of barrier steps (WG-uniform); a half past its last
    // tile only waits.
    const int te = grp ? ntiles : tm;
    const int nsteps = max(tm - t0, ntiles - tm);
    for (int s = 0; s < nsteps; ++s) {
      const int tt = tb + s;
      if (tt < te) {
        stage_load(tt + kDepth);
        const int key0 = tt * kKT;
        const bool full = tt < tf1;
        if (full || key0 <= w_last) {
          score(tt % kSlots, Sa);
          if (!full) mask(Sa, key0);
          first_max(Sa, key0);
          probs(Sa, P);
          pv_mma(tt % kSlots, P);
        }
      }
      stage_store(0, 0);
      __syncthreads();
    }
    t = ntiles;
  } else if constexpr (kAhead == 0) {
    // Each tile's scores, maximum, probabilities and P.V in one step; the waves of the
    // other workgroup on the CU cover the score MFMAs' latency.
    for (; t < tf1; ++t) {
      stage_load(t + kDepth);
      score(t % kSlots, Sa);
      first_max(Sa, t * kKT);
      probs(Sa, P);
      pv_mma(t % kSlots, P);
      stage_store(0, 0);
      __syncthreads();
    }
  } else {
    while (t < tf1) {
      pipe_step(t, Sa, Sb, Sc);
      if (++t >= tf1) break;
      pipe_step(t, Sb, Sc, Sa);
      if (++t >= tf1) break;
      pipe_step(t, Sc, Sa, Sb);
      ++t;
    }
  }
  for (; t < ntiles; ++t) masked_step(t);

  if constexpr (kSplit) {
    // Merge the halves: the second writes (u, M, max, S, Q) per lane, the first rescales
    // both to the larger reference and adds.  Every tile load has landed and been read
    // before the last step's barrier, so the rings' LDS is free.
    float *x = reinterpret_cast<float *>(smem) + wv * 36 * 64 + lane;
    if (grp) {
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[(db * 16 + r) * 64] = o[0][db][r];
      x[32 * 64] = Mref[0];
      x[33 * 64] = smax[0];
      x[34 * 64] = Ssum[0];
      x[35 * 64] = Qsum[0];
    }
    __syncthreads();
    if (grp) return;
    const float M1 = x[32 * 64], M0 = Mref[0];
    const float M = fmaxf(M0, M1);
    const float a0 = fast_exp2(M0 - M);
    const float a1 = fast_exp2(M1 - M);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[0][db][r] = o[0][db][r] * a0 + x[(db * 16 + r) * 64] * a1;
    smax[0] = fmaxf(smax[0], x[33 * 64]);
    Ssum[0] = Ssum[0] * a0 + x[34 * 64] * a1;
    Qsum[0] = Qsum[0] * (a0 * a0) + x[35 * 64] * (a1 * a1);
    Mref[0] = M;
  }

  // ---- epilogue ----
  if constexpr (kRowStores) {
    // The last step issued loads of a tile past the end: let them land before the ring's
    // space is reused.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
  }
  const float bias = a.null_bias ? a.null_bias[h] : 0.0f;
  // Row stores: per-row factors of the staged u (1/|u|, gate tanh(ln n_eff), 1/S).
  float rinv[QB], cgate[QB], rinvs[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    rinv[qb] = 0.f;
    cgate[qb] = 0.f;
    rinvs[qb] = 0.f;
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
      const int nk = (kWin && a.window > 0) ? min(row + 1, a.window) : pbase + row + 1;
      if (a.null_floor) floor_ += cnat[qb] * 0.125f * sqrtf(2.0f * logf((float)nk));
      const float gate = 1.0f / (1.0f + expf(floor_ - m_nat));
      const float n2 = neff * neff;
      const float th = (n2 - 1.0f) / (n2 + 1.0f);
      const float inv = nrm > 0.f ? rsqrtf(nrm) : 0.f;
      const size_t obase = ((size_t)b * a.T + row) * a.Hq + h;
      if constexpr (kRowStores) {
        // u itself: dir, attn and mixed are u times a per-row factor, applied at the store.
        float *ep = reinterpret_cast<float *>(smem) + (wv * 32 + c32) * kOutPitch;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            const int dim0 = db * 32 + 8 * j4 + 4 * g32;
            f32x4 val;
#pragma unroll
            for (int c = 0; c < 4; ++c) val[c] = o[qb][db][4 * j4 + c];
            *(f32x4 *)(ep + dim0) = val;
          }
        rinv[qb] = inv;
        if constexpr (kAttn) rinvs[qb] = 1.0f / St;
      } else if constexpr (kMix) {
        // The three streams summed: u/|u| + gate tanh(ln n_eff) w_h + memory.
        const float cg = a.count_vec ? gate * th : 0.f;
        const float *wp = a.count_vec ? a.count_vec + (size_t)h * kD : nullptr;
        const float *mp = a.memory ? a.memory + obase * kD : nullptr;
        float *xp = a.mixed + obase * kD;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            const int dim0 = db * 32 + 8 * j4 + 4 * g32;
            const f32x4 w = a.count_vec ? *(const f32x4 *)(wp + dim0) : f32x4{0.f, 0.f, 0.f, 0.f};
            const f32x4 m = a.memory ? *(const f32x4 *)(mp + dim0) : f32x4{0.f, 0.f, 0.f, 0.f};
            f32x4 val;
#pragma unroll
            for (int c = 0; c < 4; ++c) val[c] = (o[qb][db][4 * j4 + c] * inv + cg * w[c]) + m[c];
            *(f32x4 *)(xp + dim0) = val;
          }
      } else {
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
      }
      if constexpr (kAttn && !kRowStores) {
        if (a.attn) {
          const float is = 1.0f / St;
          float *ap = a.attn + obase * kD;
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
              const int dim0 = db * 32 + 8 * j4 + 4 * g32;
              f32x4 val;
#pragma unroll
              for (int c = 0; c < 4; ++c) val[c] = o[qb][db][4 * j4 + c] * is;
              *(f32x4 *)(ap + dim0) = val;
            }
        }
      }
      if constexpr (kRowStores) cgate[qb] = (!kMix || a.count_vec) ? gate * th : 0.f;
      if (!kMix && !kRowStores && a.count) {
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
      if constexpr (kSave) {
        // Arg-max over the two wave halves: larger score, then lower key.
        const float ob = __shfl_xor(lbest[qb], 32);
        const int ok = __shfl_xor(lkey[qb], 32);
        const int key = (ob > lbest[qb] || (ob == lbest[qb] && ok < lkey[qb])) ? ok : lkey[qb];
        if (g32 == 0) {
          a.u_norm[obase] = sqrtf(nrm) / St;
          a.arg_max[obase] = key;
        }
      }
      if (g32 == 0) {
        a.n_eff[obase] = neff;
        if (a.gate) a.gate[obase] = gate;
        if (a.lse) a.lse[obase] = lse;
      }
    }
  }
  if constexpr (kRowStores) {
    // Four whole rows per store: lane l writes dims 4 (l % 16) .. + 3 of row 4 i + l / 16;
    // count is gate tanh(ln n_eff) (held by the row's own lane) times the head's vector.
    static_assert(!kRowStores || QB == 1, "row stores: one query block per wave");
    __syncthreads();
    const float *ep = reinterpret_cast<const float *>(smem) + wv * 32 * kOutPitch;
    const int rq = lane >> 4, cc = (lane & 15) * 4;
    const bool wcount = kMix ? a.count_vec != nullptr : a.count != nullptr;
    bool wattn = false;
    if constexpr (kAttn) wattn = a.attn != nullptr;
    const f32x4 w4 = wcount ? *(const f32x4 *)(a.count_vec + (size_t)h * kD + cc)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + rq;
      const float cgr = __shfl(cgate[0], r), invr = __shfl(rinv[0], r);
      float isr = 0.f;
      if constexpr (kAttn) isr = __shfl(rinvs[0], r);
      if (wrow0 + r < a.T) {
        const size_t ob = (((size_t)b * a.T + wrow0 + r) * a.Hq + h) * kD + cc;
        const f32x4 u4 = *(const f32x4 *)(ep + r * kOutPitch + cc);
        const f32x4 dv = u4 * invr;
        if constexpr (kAttn) {
          if (wattn) __builtin_nontemporal_store(u4 * isr, (f32x4 *)(a.attn + ob));
        }
        if constexpr (kMix) {
          // The three streams summed: u/|u| + gate tanh(ln n_eff) w_h + memory.
          const f32x4 m = a.memory ? *(const f32x4 *)(a.memory + ob) : f32x4{0.f, 0.f, 0.f, 0.f};
          f32x4 val;
#pragma unroll
          for (int c = 0; c < 4; ++c) val[c] = (dv[c] + cgr * w4[c]) + m[c];
          __builtin_nontemporal_store(val, (f32x4 *)(a.mixed + ob));
        } else {
          __builtin_nontemporal_store(dv, (f32x4 *)(a.dir + ob));
          if (wcount) __builtin_nontemporal_store(w4 * cgr, (f32x4 *)(a.count + ob));
        }
      }
    }
  }
  // Every workgroup has taken its task once the completion count reaches the grid: the
  // last one to finish leaves the counters at zero for the next launch on this slot.
  if (kTicketed && a.ticket && tid == 0) {
    if (atomicAdd(a.ticket + kTicketQueues, 1u) == gridDim.x - 1) {
#pragma unroll
      for (int q = 0; q <= kTicketQueues; ++q) atomicExch(a.ticket + q, 0u);
    }
  }
}

// One 16-byte chunk (part) of a row at position pos turned by RoPE: 4 pairs for bf16, 2 for
// fp32, with the staging's arithmetic (rope_cs, the same explicit FMAs, one rounding to the
// storage type), so every place that rotates a vector gets the same values.
template <class E>
__device__ __forceinline__ u32x4 rotate_chunk(u32x4 w, int part, int pos, const uint64_t *f) {
  if constexpr (sizeof(E) == 2) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float c, sn;
      rope_cs(f[part * 4 + m], pos, c, sn);
      const float x0 = __uint_as_float(w[m] << 16), x1 = __uint_as_float(w[m] & 0xFFFF0000u);
      const bf16x2 r = {(__bf16)rot_re(x0, x1, c, sn), (__bf16)rot_im(x0, x1, c, sn)};
      w[m] = __builtin_bit_cast(uint32_t, r);
    }
  } else {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float c, sn;
      rope_cs(f[part * 2 + m], pos, c, sn);
      const float x0 = __uint_as_float(w[2 * m]), x1 = __uint_as_float(w[2 * m + 1]);
      w[2 * m] = __float_as_uint(rot_re(x0, x1, c, sn));
      w[2 * m + 1] = __float_as_uint(rot_im(x0, x1, c, sn));
    }
  }
  return w;
}

// Key rotation ahead of the variant prefill: one thread per 16-byte chunk of a key row, so
// the attention kernel sees the keys it would have rotated while staging them.
template <class E>
__global__ void __launch_bounds__(256) polar_rope_keys_kernel(PrefillArgs a, E *k_out) {
  constexpr int kVec = 16 / (int)sizeof(E);            // elements per chunk
  constexpr int kChunks = kD / kVec;                   // chunks per key row
  const long long n = (long long)a.B * a.T * a.Hkv * kChunks;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (long long)gridDim.x * 256) {
    const int part = (int)(i % kChunks);
    const long long row = i / kChunks;                 // (b * T + pos) * Hkv + g
    const int pos = (int)((row / a.Hkv) % a.T);
    const u32x4 w = *(const u32x4 *)((const E *)a.k + row * kD + part * kVec);
    *(u32x4 *)(k_out + row * kD + part * kVec) = rotate_chunk<E>(w, part, pos, a.rope_f);
  }
}

// q [B,T,Hq,d] and k [B,T,Hkv,d] rotated in one launch (the training arm with RoPE): the
// chunks of q first, then those of k.
template <class E>
__global__ void __launch_bounds__(256) polar_rope_qk_kernel(RopeQk r) {
  constexpr int kVec = 16 / (int)sizeof(E);
  constexpr int kChunks = kD / kVec;
  const long long nq = (long long)r.B * r.T * r.Hq * kChunks;
  const long long n = nq + (long long)r.B * r.T * r.Hkv * kChunks;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (long long)gridDim.x * 256) {
    const bool isq = i < nq;
    const long long j = isq ? i : i - nq;
    const int H = isq ? r.Hq : r.Hkv;
    const int part = (int)(j % kChunks);
    const long long row = j / kChunks;                 // (b * T + pos) * H + h
    const int pos = (int)((row / H) % r.T);
    const E *src = (const E *)(isq ? r.q : r.k) + row * kD + part * kVec;
    E *dst = (E *)(isq ? r.q_out : r.k_out) + row * kD + part * kVec;
    *(u32x4 *)dst = rotate_chunk<E>(*(const u32x4 *)src, part, pos, r.rope_f);
  }
}

constexpr int kQbBf16 = 1;
constexpr int kQbF32 = 1;
constexpr int kWavesBf16 = 8;
constexpr int kWavesF32 = 4;
// The lean instances pay off once the grid holds two workgroups per CU (256 CUs); with one
// per CU the pipelined instances keep their two waves per SIMD busier.
constexpr long long kLeanMinWorkgroups = 512;

}  // namespace

int prefill_heads_per_block(int G) {
  if (G % 4 == 0) return 4;
  if (G % 2 == 0) return 2;
  return 1;
}

PrefillShape prefill_shape(int dtype, const PrefillArgs &a) {
  if (dtype != 1) return {0, (kWavesF32 / a.hb) * 32 * kQbF32};
  const int rows = (kWavesBf16 / a.hb) * 32 * kQbBf16;
  // Launches whose keys are already rotated (direct tiles) may be lean.
  const bool direct_mode = !(a.rope && !a.k_rotated);
  const long long wgs = (long long)((a.T + rows - 1) / rows) * a.Hkv * (a.G / a.hb) * a.B;
  if (direct_mode && wgs >= kLeanMinWorkgroups) return {1, rows};
  // Paged launches with fewer workgroups split each row block's keys over two halves of a
  // 16-wave workgroup: four waves per SIMD instead of two.
  if (a.paged) return {2, rows};
  return {0, rows};
}

hipError_t launch_rope_qk(int dtype, const RopeQk &r, hipStream_t stream) {
  const long long n = (long long)r.B * r.T * (r.Hq + r.Hkv) * (kD / (dtype == 1 ? 8 : 4));
  if (n <= 0) return hipSuccess;
  const long long need = (n + 255) / 256;
  const unsigned blocks = (unsigned)(need < 65536 ? need : 65536);
  if (dtype == 1)
    hipLaunchKernelGGL((polar_rope_qk_kernel<uint16_t>), dim3(blocks), dim3(256), 0, stream, r);
  else
    hipLaunchKernelGGL((polar_rope_qk_kernel<float>), dim3(blocks), dim3(256), 0, stream, r);
  return hipGetLastError();
}

hipError_t launch_rope_keys(int dtype, const PrefillArgs &a, void *k_out, hipStream_t stream) {
  const long long n = (long long)a.B * a.T * a.Hkv * (kD / (dtype == 1 ? 8 : 4));
  if (n <= 0) return hipSuccess;
  const long long need = (n + 255) / 256;
  const unsigned blocks = (unsigned)(need < 65536 ? need : 65536);
  if (dtype == 1)
    hipLaunchKernelGGL((polar_rope_keys_kernel<uint16_t>), dim3(blocks), dim3(256), 0, stream, a,
                       (uint16_t *)k_out);
  else
    hipLaunchKernelGGL((polar_rope_keys_kernel<float>), dim3(blocks), dim3(256), 0, stream, a,
                       (float *)k_out);
  return hipGetLastError();
}

// Task counters for launches that hand out row blocks by ticket: one set (the queue
// counters and the completion count) per launch, in a ring of kTicketSlots sets per
// device, each set back at zero when its launch ends.  A slot comes round again after
// kTicketSlots further launches on the device; only launches that far apart and still
// running concurrently (a graph replayed beside itself on another stream, say) could share
// one.
constexpr int kTicketSlots = 1024;
static __device__ __align__(256) unsigned prefill_tickets[kTicketSlots][kTicketQueues + 1];

// The launches that take tasks by ticket: plain prefills of at least eight workgroups per
// CU slot (T = 64K: 1.7% faster).  Below that the atomic at each workgroup's start costs
// more than the tail it saves (2K and 16K forwards: 3-7% slower), and the variant
// instances measured 1.5% slower with tickets at 64K, so they keep the grid order.
constexpr long long kTicketMinWorkgroups = 4096;

hipError_t ticket_slot(unsigned **slot) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static unsigned *base[kMaxDevices];
  static unsigned next[kMaxDevices];
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!base[dev]) {
    void *p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(prefill_tickets));   // with dev current
    if (err != hipSuccess) return err;
    base[dev] = (unsigned *)p;
  }
  *slot = base[dev] + (kTicketQueues + 1) * (next[dev]++ % kTicketSlots);
  return hipSuccess;
}

hipError_t launch_prefill(int dtype, const PrefillArgs &args, hipStream_t stream) {
  const int NY = args.Hkv * (args.G / args.hb);
  const long long blocks = (long long)args.n_row_blocks * NY * args.B;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  PrefillArgs a = args;
  a.ticket = nullptr;
  if (blocks >= kTicketMinWorkgroups && dtype == 1 && a.lean == 1 && !a.paged && !a.variant &&
      a.u_norm == nullptr) {
    hipError_t err = ticket_slot(&a.ticket);
    if (err != hipSuccess) return err;
  }
  dim3 grid((unsigned)blocks);
  const int mode = a.paged ? kModePaged
                 : a.variant ? ((a.rope && !a.k_rotated) ? kModeVariantRot : kModeVariant)
                 : a.mixed ? kModeMix
                 : a.u_norm == nullptr ? kModePlain
                 : (a.window > 0 ? kModeSaveWin : kModeSave);
  const dim3 bb(64 * kWavesBf16), bf(64 * kWavesF32);
  if (dtype == 1 && a.lean == 2) {
    if (mode != kModePaged) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((polar_prefill_kernel<Bf16, 1, 16, kModePaged, true>), grid,
                       dim3(1024), 0, stream, a);
  } else if (dtype == 1 && a.lean) {
    if (mode == kModePlain)
      hipLaunchKernelGGL((polar_prefill_kernel<Bf16, 1, kWavesBf16, kModePlain, true>), grid,
                         bb, 0, stream, a);
    else if (mode == kModeVariant)
      hipLaunchKernelGGL((polar_prefill_kernel<Bf16, 1, kWavesBf16, kModeVariant, true>), grid,
                         bb, 0, stream, a);
    else if (mode == kModePaged)
      hipLaunchKernelGGL((polar_prefill_kernel<Bf16, 1, kWavesBf16, kModePaged, true>), grid,
                         bb, 0, stream, a);
    else if (mode == kModeSave)
      hipLaunchKernelGGL((polar_prefill_kernel<Bf16, 1, kWavesBf16, kModeSave, true>), grid,
                         bb, 0, stream, a);
    else if (mode == kModeSaveWin)
      hipLaunchKernelGGL((polar_prefill_kernel<Bf16, 1, kWavesBf16, kModeSaveWin, true>), grid,
                         bb, 0, stream, a);
    else if (mode == kModeMix)
      hipLaunchKernelGGL((polar_prefill_kernel<Bf16, 1, kWavesBf16, kModeMix, true>), grid,
                         bb, 0, stream, a);
    else
      return hipErrorInvalidConfiguration;   // prefill_shape never picks it for other modes
  } else if (dtype == 1) {
    if (mode == kModePlain)
      hipLaunchKernelGGL((polar_prefill_kernel<Bf16, kQbBf16, kWavesBf16, kModePlain, false>),
                         grid, bb, 0, stream, a);
    else if (mode == kModeSave)
      hipLaunchKernelGGL((polar_prefill_kernel<Bf16, kQbBf16, kWavesBf16, kModeSave, false>),
                         grid, bb, 0, stream, a);
    else if (mode == kModeSaveWin)
      hipLaunchKernelGGL((polar_prefill_kernel<Bf16, kQbBf16, kWavesBf16, kModeSaveWin, false>),
                         grid, bb, 0, stream, a);
    else if (mode == kModeMix)
      hipLaunchKernelGGL((polar_prefill_kernel<Bf16, kQbBf16, kWavesBf16, kModeMix, false>),
                         grid, bb, 0, stream, a);
    else if (mode == kModeVariant)
      hipLaunchKernelGGL((polar_prefill_kernel<Bf16, kQbBf16, kWavesBf16, kModeVariant, false>),
                         grid, bb, 0, stream, a);
    else if (mode == kModeVariantRot)
      hipLaunchKernelGGL(
          (polar_prefill_kernel<Bf16, kQbBf16, kWavesBf16, kModeVariantRot, false>), grid, bb, 0,
          stream, a);
    else
      hipLaunchKernelGGL((polar_prefill_kernel<Bf16, kQbBf16, kWavesBf16, kModePaged, false>),
                         grid, bb, 0, stream, a);
  } else {
    if (a.lean) return hipErrorInvalidConfiguration;
    if (mode == kModePlain)
      hipLaunchKernelGGL((polar_prefill_kernel<F32, kQbF32, kWavesF32, kModePlain, false>), grid,
                         bf, 0, stream, a);
    else if (mode == kModeSave)
      hipLaunchKernelGGL((polar_prefill_kernel<F32, kQbF32, kWavesF32, kModeSave, false>), grid,
                         bf, 0, stream, a);
    else if (mode == kModeSaveWin)
      hipLaunchKernelGGL((polar_prefill_kernel<F32, kQbF32, kWavesF32, kModeSaveWin, false>),
                         grid, bf, 0, stream, a);
    else if (mode == kModeMix)
      hipLaunchKernelGGL((polar_prefill_kernel<F32, kQbF32, kWavesF32, kModeMix, false>), grid,
                         bf, 0, stream, a);
    else if (mode == kModeVariant || mode == kModeVariantRot)   // fp32 always stages K itself
      hipLaunchKernelGGL((polar_prefill_kernel<F32, kQbF32, kWavesF32, kModeVariant, false>),
                         grid, bf, 0, stream, a);
    else
      hipLaunchKernelGGL((polar_prefill_kernel<F32, kQbF32, kWavesF32, kModePaged, false>), grid,
                         bf, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace polar
