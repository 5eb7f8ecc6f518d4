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
  int B, T, Hq, Hkv, G;                   // G = Hq / Hkv
  int hb;                                 // query heads per workgroup (divides G, <= 4)
  int n_row_blocks;                       // ceil(T / rows per workgroup)
  float inv_log_train;                    // 1/ln(train_len) with the length temperature, else 0
  int null_floor;                         // 1: add the extreme-value term to the floor
};

// dtype: 0 = f32, 1 = bf16 (same numbering as polar_dtype).
int prefill_heads_per_block(int G);
int prefill_rows_per_block(int dtype, int hb);
hipError_t launch_prefill(int dtype, const PrefillArgs &a, hipStream_t stream);

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

}  // namespace polar
