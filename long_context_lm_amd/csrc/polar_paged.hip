// Paged KV cache maintenance for gfx950: append a chunk of new keys and values.
//
// The decode kernel of the ATMA technical summary (gist.science), section 2.2, reads keys
// and values from paged cache blocks; this is the write side.  Token t of sequence b lands
// at logical position s + t, with s = start_pos[b] clamped to [0, max_seq_len - C] exactly
// as the chunked prefill clamps it: page page_table[b, pos / 64], slot pos % 64, for every
// KV head (page-major pools [num_pages, Hkv, 64, d]).  Pure data movement: one
// 16-byte chunk per thread and grid-stride loop, coalesced on both sides (a (page, head)
// block is 64 contiguous rows).
#include "polar_kernels.h"

namespace polar {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) polar_kv_append_kernel(AppendArgs a) {
  const int cpr = a.row_bytes / 16;                          // 16-byte chunks per row
  const long long total = (long long)a.B * a.C * a.Hkv * cpr;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * 256) {
    const int part = (int)(idx % cpr);
    long long r = idx / cpr;
    const int g = (int)(r % a.Hkv);
    r /= a.Hkv;
    const int t = (int)(r % a.C);
    const int b = (int)(r / a.C);
    const int pos = min(max(a.start_pos[b], 0), a.max_seq_len - a.C) + t;
    const int page = a.page_table[(size_t)b * a.stride + pos / kPageSize];
    if (page < 0 || page >= a.num_pages) continue;
    const size_t src = (((size_t)b * a.C + t) * a.Hkv + g) * a.row_bytes + part * 16;
    const size_t dst =
        (((size_t)page * a.Hkv + g) * kPageSize + pos % kPageSize) * a.row_bytes + part * 16;
    *(u32x4 *)((char *)a.k_cache + dst) = *(const u32x4 *)((const char *)a.k_new + src);
    *(u32x4 *)((char *)a.v_cache + dst) = *(const u32x4 *)((const char *)a.v_new + src);
  }
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs &a, hipStream_t stream) {
  const long long total = (long long)a.B * a.C * a.Hkv * (a.row_bytes / 16);
  if (total <= 0) return hipSuccess;
  const long long blocks = min((total + 255) / 256, 65536LL);
  hipLaunchKernelGGL(polar_kv_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace polar
