// Launch descriptors shared by the C-ABI layer and the HIP kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace polar {

constexpr int kHeadDim = 64;    // d supported by this version
constexpr int kPageSize = 64;   // tokens per KV page supported by this version

struct PrefillArgs {
  const void *q, *k, *v;                  // [B,T,Hq,d], [B,T,Hkv,d] x2
  const float *beta, *null_bias, *count_vec;
  float *dir, *count, *n_eff, *gate, *lse;
  float *u_norm;                          // [B,T,Hq] |u| for the backward pass, or NULL
  int32_t *arg_max;                       // [B,T,Hq] first key of the row maximum (with u_norm)
  // Softmax read-out sum p v [B,T,Hq,d], or NULL (variant and training instances):
  float *attn;
  // Variant modes (variant instances only):
  int variant;                            // 1: launch the variant instance
  int window;                             // W >= 1: row i sees keys i-W+1..i; 0: all
  int rope;                               // 1: rotate q and k by RoPE on load
  int k_rotated;                          // 1: k is already rotated (rotate q only)
  uint64_t rope_f[kHeadDim / 2];          // revolutions per position of pair t, 2^-64 units
  int B, T, Hq, Hkv, G;                   // G = Hq / Hkv
  int hb;                                 // query heads per workgroup (divides G, <= 4)
  int lean;                               // 1: lean instance, 2: paged split (prefill_shape)
  int n_row_blocks;                       // ceil(T / rows per workgroup)
  float inv_log_train;                    // 1/ln(train_len) with the length temperature, else 0
  int null_floor;                         // 1: add the extreme-value term to the floor
  // Paged chunk instances: q holds C = T rows per sequence at positions start_pos[b]..;
  // k and v are the page pools [num_pages,Hkv,kPageSize,d] read through page_table.
  int paged;
  const int32_t *page_table;              // [B,stride]
  const int32_t *start_pos;               // [B]
  int stride, num_pages, max_seq_len;
  // Mixed output (section 2.1's out = content + count + memory): when non-NULL, the kernel
  // writes mixed = dir + count + memory [B,T,Hq,d] instead of dir and count; memory may be
  // NULL (no memory stream).
  float *mixed;
  const float *memory;
  // Task and completion counters of this launch ([2], zero on entry, zero again when the
  // last workgroup ends), or NULL: workgroup i then takes row block task i.
  unsigned *ticket;
};

// dtype: 0 = f32, 1 = bf16 (same numbering as polar_dtype).
int prefill_heads_per_block(int G);
// Which prefill instance runs a (0 pipelined, 1 lean, 2 paged split) and its rows per
// workgroup.  Reads dtype and a.B, a.T, a.Hkv, a.G, a.hb, a.paged, a.rope, a.k_rotated.
struct PrefillShape {
  int lean, rows;
};
PrefillShape prefill_shape(int dtype, const PrefillArgs &a);
hipError_t launch_prefill(int dtype, const PrefillArgs &a, hipStream_t stream);
// Rotates the keys a.k [B,T,Hkv,d] by RoPE at positions 0..T-1 into k_out (same layout),
// with exactly the arithmetic the prefill's staging applies.
hipError_t launch_rope_keys(int dtype, const PrefillArgs &a, void *k_out, hipStream_t stream);
// The training arm with RoPE: q [B,T,Hq,d] and k [B,T,Hkv,d] rotated into q_out, k_out
// (rope_f as in PrefillArgs).  The backward kernels turn dq and dk back themselves
// (BwdArgs::rope).
struct RopeQk {
  const void *q, *k;
  void *q_out, *k_out;
  int B, T, Hq, Hkv;
  uint64_t rope_f[kHeadDim / 2];
};
hipError_t launch_rope_qk(int dtype, const RopeQk &r, hipStream_t stream);

struct DecodeArgs {
  const void *q;                          // [B,Hq,d]
  const void *k_cache, *v_cache;          // [num_pages,Hkv,page,d]
  const int32_t *page_table;              // [B,stride]
  const int32_t *seq_lens;                // [B]
  const float *beta, *null_bias, *count_vec;
  float *dir, *count, *n_eff, *gate, *lse;
  float *ws;                              // split partials
  int B, Hq, Hkv, G, num_pages, stride, max_seq_len;
  int n_split, pages_per_split, n_hchunk; // split-KV grid
  float inv_log_train;
  int null_floor;
};

struct DecodeGrid {
  int n_split, pages_per_split, n_hchunk;
};
DecodeGrid decode_grid(int B, int Hq, int Hkv, int max_seq_len);
size_t decode_ws_bytes(int B, int Hq, int Hkv, int max_seq_len);
hipError_t launch_decode(int dtype, const DecodeArgs &a, hipStream_t stream);
// The allocation-free decode's static scratch: its size, and its device address on the
// current device (looked up on the first call on each device).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
hipError_t noalloc_scratch(void **ptr);

// Writes a chunk of new keys/values into the page pools.
struct AppendArgs {
  const void *k_new, *v_new;              // [B,C,Hkv,d]
  void *k_cache, *v_cache;                // [num_pages,Hkv,kPageSize,d]
  const int32_t *page_table, *start_pos;
  int B, C, Hkv, stride, num_pages, max_seq_len;
  int row_bytes;                          // d * element size
};
hipError_t launch_kv_append(const AppendArgs &a, hipStream_t stream);

// In-place gated-delta memory step (states [num_slots,H,d,d] fp32, d = kHeadDim).
struct DeltaArgs {
  float *pool;
  const int32_t *slots;                   // [B]
  const void *q, *k, *v;                  // [B,H,d]
  const float *alpha, *beta;              // [B,H]
  float *out;                             // [B,H,d]
  int B, H, num_slots, normalize;
};
hipError_t launch_delta_step(int dtype, const DeltaArgs &a, hipStream_t stream);
// The memory stream over T tokens per sequence (states [num_slots,H,d,d] fp32, in place).
struct DeltaSeqArgs {
  float *pool;
  const int32_t *slots;                   // [B]
  const void *q, *k, *v;                  // [B,T,H,d]
  const float *alpha, *beta;              // [B,T,H]
  float *out;                             // [B,T,H,d]
  int B, T, H, num_slots, normalize;
};
hipError_t launch_delta_sequence(int dtype, const DeltaSeqArgs &a, hipStream_t stream);

// Backward pass of the causal prefill (bf16 inputs).  Per-row quantities (float4 each;
// r0 and r1 of a row are adjacent in `rows`):
//   r0 = {c*log2(e), lse*log2(e), c*A, c*E}   r1 = {A, E, dm, arg-max key (int bits)}
//   rp = {dbeta contribution of the dq kernel, -dm, gate*tanh(ln n_eff), floor term of dbeta}
// with c = beta*tau and dl_j = p_j (v_j.du + A + E p_j) + [j = arg-max] dm (the u . du
// inside A taken of the bf16 du the kernels read).
struct BwdArgs {
  const void *q, *k, *v;                  // bf16 [B,T,Hq,d], [B,T,Hkv,d] x2
  const float *beta, *null_bias, *count_vec;
  const float *dir, *n_eff, *gate, *lse;  // forward outputs
  const float *u_norm;                    // forward residuals
  const int32_t *arg_max;
  const float *c_dir, *c_count, *c_n_eff, *c_gate, *c_lse;   // cotangents (NULL = 0)
  const float *c_attn;                    // cotangent of the read-out u = sum p v (NULL = 0)
  float *dq, *dk, *dv;                    // fp32 [B,T,Hq,d], [B,T,Hkv,d] x2
  float *d_beta, *d_null_bias, *d_count_vec;
  uint16_t *du;                           // workspace: bf16 du [B,T,Hq,d]
  float *rows;                            // workspace: per-row r0, r1 (8 floats)
  float *rp;                              // workspace: per-row float4
  float *part;                            // workspace: [Hq][n_part][kPartStride]
  float *dk_part, *dv_part;               // workspace: dk, dv of head groups 1..hsplit-1
  int B, T, Hq, Hkv, G;
  int hb, n_row_blocks;                   // dq kernel: heads per workgroup, row blocks
  int n_key_blocks;                       // dk/dv kernel: key blocks per (b, KV head)
  int hsplit;                             // dk/dv kernel: workgroups per key block (divides G)
  int n_part;                             // parameter reduction: row chunks per head
  float inv_log_train;
  int null_floor;
  int window;                             // W >= 1: row i sees keys i-W+1..i; 0: all
  // 1: q and k are RoPE-rotated (rope_f as in PrefillArgs); dq and dk leave the kernels
  // turned back by the transposed rotation.
  int rope;
  uint64_t rope_f[kHeadDim / 2];
};
constexpr int kPartStride = 68;           // dw[64], dbeta, dbias, pad

size_t bwd_ws_bytes(int B, int T, int Hq, int Hkv);
void bwd_ws_layout(BwdArgs &a, void *ws);  // sets du, rows, rp, part, dk/dv parts, n_part
int bwd_rows_per_block(int hb);
int bwd_keys_per_block();
int bwd_head_split(int G);                // workgroups sharing one key block (divides G)
hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream);
// p[0..n) = 0 with a kernel (capturable in a graph, unlike a memset node).
hipError_t launch_zero(float *p, long long n, hipStream_t stream);

}  // namespace polar
