// C-ABI entry points of libpolar: argument validation, launch geometry, dispatch.
// Every check runs before any HIP call, so errors are reported without a GPU and
// nothing is launched or written on an error.
#include <stdarg.h>
#include <stdio.h>
#include <math.h>

#include "../../include/polar.h"
#include "polar_kernels.h"

namespace {

thread_local char g_last_error[512] = "";

polar_status fail(polar_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

polar_status check_params(const polar_params *p, polar_dtype dt, const polar_outputs *out) {
  if (!p) return fail(POLAR_ERR_NULL_POINTER, "params is NULL");
  if (!out) return fail(POLAR_ERR_NULL_POINTER, "outputs is NULL");
  if (dt != POLAR_DTYPE_F32 && dt != POLAR_DTYPE_BF16)
    return fail(POLAR_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (p->n_q_heads < 1 || p->n_kv_heads < 1)
    return fail(POLAR_ERR_BAD_SHAPE, "head counts must be >= 1 (Hq=%d, Hkv=%d)", p->n_q_heads,
                p->n_kv_heads);
  if (p->n_q_heads % p->n_kv_heads != 0)
    return fail(POLAR_ERR_BAD_SHAPE, "Hq (%d) is not a multiple of Hkv (%d)", p->n_q_heads,
                p->n_kv_heads);
  if (p->head_dim != polar::kHeadDim)
    return fail(POLAR_ERR_UNSUPPORTED, "head_dim %d unsupported (only %d)", p->head_dim,
                polar::kHeadDim);
  if (p->flags & ~(uint32_t)(POLAR_FLAG_LENGTH_TEMP | POLAR_FLAG_NULL_FLOOR))
    return fail(POLAR_ERR_UNSUPPORTED, "unknown flag bits 0x%x", p->flags);
  if ((p->flags & POLAR_FLAG_LENGTH_TEMP) && p->train_len < 2)
    return fail(POLAR_ERR_BAD_SHAPE, "train_len must be >= 2 with LENGTH_TEMP (got %d)",
                p->train_len);
  return POLAR_OK;
}

// Output pointers are checked only for non-empty calls (empty tensors may be NULL).
polar_status check_outputs(const polar_params *p, const polar_outputs *out) {
  if (!out->dir) return fail(POLAR_ERR_NULL_POINTER, "outputs.dir is NULL");
  if (!out->n_eff) return fail(POLAR_ERR_NULL_POINTER, "outputs.n_eff is NULL");
  if (out->count && !p->count_vec)
    return fail(POLAR_ERR_NULL_POINTER, "outputs.count requested but params.count_vec is NULL");
  if (!aligned16(out->dir) || (out->count && !aligned16(out->count)) ||
      (out->count && !aligned16(p->count_vec)))
    return fail(POLAR_ERR_MISALIGNED, "dir, count and count_vec must be 16-byte aligned");
  return POLAR_OK;
}

float inv_log_train(const polar_params *p) {
  return (p->flags & POLAR_FLAG_LENGTH_TEMP) ? (float)(1.0 / log((double)p->train_len)) : 0.f;
}

// RoPE frequencies of the kernels: revolutions per position of pair t, rounded to 2^-64
// units (< 1/(2 pi), so they fit); all zero when theta == 0.
void fill_rope_f(uint64_t *f, float theta) {
  for (int t = 0; t < polar::kHeadDim / 2; ++t) {
    f[t] = 0;
    if (theta > 0.f) {
      const long double r = powl((long double)theta, -2.0L * t / polar::kHeadDim) /
                            (2.0L * 3.14159265358979323846264338327950288L);
      f[t] = (uint64_t)(r * 18446744073709551616.0L + 0.5L);
    }
  }
}

polar_status check_variant(const polar_variant *var) {
  if (!var) return POLAR_OK;
  if (var->window < 0) return fail(POLAR_ERR_BAD_SHAPE, "window (%d) must be >= 0", var->window);
  if (!(var->rope_theta >= 0.f) || !isfinite(var->rope_theta) ||
      (var->rope_theta > 0.f && var->rope_theta <= 1.f))
    return fail(POLAR_ERR_BAD_SHAPE, "rope_theta must be 0 or a finite value > 1");
  return POLAR_OK;
}

// Rotates q [B,T,Hq,d] and k [B,T,Hkv,d] of type dt by RoPE into q_out and k_out, with
// polar_attn_fwd_variant's rounding.
hipError_t rotate_qk(polar_dtype dt, const void *q, const void *k, void *q_out, void *k_out,
                     int B, int T, int Hq, int Hkv, float theta, hipStream_t stream) {
  polar::RopeQk r{};
  r.q = q;
  r.k = k;
  r.q_out = q_out;
  r.k_out = k_out;
  r.B = B;
  r.T = T;
  r.Hq = Hq;
  r.Hkv = Hkv;
  fill_rope_f(r.rope_f, theta);
  return polar::launch_rope_qk((int)dt, r, stream);
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

struct PagedSrc {
  const int32_t *page_table, *start_pos;
  int stride, num_pages, max_seq_len;
};

polar_status prefill(const polar_params *p, polar_dtype dt, int32_t B, int32_t T, const void *q,
                     const void *k, const void *v, const polar_outputs *out,
                     const polar_saved *saved, const polar_variant *var, void *stream,
                     const PagedSrc *paged = nullptr, float *mixed = nullptr,
                     const float *memory = nullptr) {
  polar_status st = check_params(p, dt, out);
  if (st != POLAR_OK) return st;
  if (var) {
    st = check_variant(var);
    if (st != POLAR_OK) return st;
    if (var->attn && !aligned16(var->attn))
      return fail(POLAR_ERR_MISALIGNED, "variant attn output must be 16-byte aligned");
    if (var->workspace && !aligned16(var->workspace))
      return fail(POLAR_ERR_MISALIGNED, "variant workspace must be 16-byte aligned");
  }
  if (B < 0 || T < 0) return fail(POLAR_ERR_BAD_SHAPE, "B (%d) and T (%d) must be >= 0", B, T);
  if (B == 0 || T == 0) return POLAR_OK;
  st = check_outputs(p, out);
  if (st != POLAR_OK) return st;
  if (!q || !k || !v) return fail(POLAR_ERR_NULL_POINTER, "q, k and v must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(POLAR_ERR_MISALIGNED, "q, k and v must be 16-byte aligned");
  if (saved) {
    if (!saved->u_norm || !saved->arg_max)
      return fail(POLAR_ERR_NULL_POINTER, "saved.u_norm and saved.arg_max must be non-NULL");
    if (!out->gate || !out->lse)
      return fail(POLAR_ERR_NULL_POINTER, "training forward needs outputs.gate and outputs.lse");
  }

  // K/V rows are addressed with 32-bit byte offsets (one tile past the end included).
  const long long elt = dt == POLAR_DTYPE_BF16 ? 2 : 4;
  if (!paged && ((long long)T + 64) * p->n_kv_heads * polar::kHeadDim * elt >= 0x7fffffffLL)
    return fail(POLAR_ERR_BAD_SHAPE, "T*Hkv too large for one sequence (T=%d, Hkv=%d)", T,
                p->n_kv_heads);

  polar::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = p->beta;
  a.null_bias = p->null_bias;
  a.count_vec = p->count_vec;
  a.dir = out->dir;
  a.count = out->count;
  a.n_eff = out->n_eff;
  a.gate = out->gate;
  a.lse = out->lse;
  a.mixed = mixed;
  a.memory = memory;
  a.u_norm = saved ? saved->u_norm : nullptr;
  a.arg_max = saved ? saved->arg_max : nullptr;
  a.attn = var ? var->attn : nullptr;
  a.window = var ? var->window : 0;
  a.rope = (var && var->rope_theta > 0.f) ? 1 : 0;
  // The training forward takes its window in the training instance (and its q and k
  // already rotated, see polar_attn_fwd_train_variant).
  a.variant = (!saved && (a.attn || a.window > 0 || a.rope)) ? 1 : 0;
  if (saved && a.rope)
    return fail(POLAR_ERR_UNSUPPORTED, "the training forward takes no rotation here");
  // Keys rotated once into the caller's workspace instead of in every staging workgroup.
  void *k_rot = nullptr;
  if (a.rope && var->workspace) {
    const size_t need = (size_t)B * T * p->n_kv_heads * polar::kHeadDim * (size_t)elt;
    if (var->workspace_bytes < need)
      return fail(POLAR_ERR_WORKSPACE_TOO_SMALL, "variant workspace has %zu bytes, needs %zu",
                  var->workspace_bytes, need);
    k_rot = var->workspace;
  }
  a.paged = paged ? 1 : 0;
  a.page_table = paged ? paged->page_table : nullptr;
  a.start_pos = paged ? paged->start_pos : nullptr;
  a.stride = paged ? paged->stride : 0;
  a.num_pages = paged ? paged->num_pages : 0;
  a.max_seq_len = paged ? paged->max_seq_len : 0;
  fill_rope_f(a.rope_f, a.rope ? var->rope_theta : 0.f);
  a.B = B;
  a.T = T;
  a.Hq = p->n_q_heads;
  a.Hkv = p->n_kv_heads;
  a.G = a.Hq / a.Hkv;
  a.hb = polar::prefill_heads_per_block(a.G);
  a.k_rotated = k_rot ? 1 : 0;          // the keys are rotated into k_rot before the launch
  const polar::PrefillShape shape = polar::prefill_shape((int)dt, a);
  a.lean = shape.lean;
  a.n_row_blocks = (T + shape.rows - 1) / shape.rows;
  a.inv_log_train = inv_log_train(p);
  a.null_floor = (p->flags & POLAR_FLAG_NULL_FLOOR) ? 1 : 0;
  const long long blocks = (long long)a.n_row_blocks * a.Hkv * (a.G / a.hb) * B;
  if (blocks > 0x7fffffffLL)
    return fail(POLAR_ERR_BAD_SHAPE, "problem too large for one launch (%lld workgroups)", blocks);
  hipError_t err = hipSuccess;
  if (k_rot) {
    err = polar::launch_rope_keys((int)dt, a, k_rot, (hipStream_t)stream);
    if (err != hipSuccess) return fail(POLAR_ERR_HIP, "key rotation launch: %s", hipGetErrorString(err));
    a.k = k_rot;
  }
  err = polar::launch_prefill((int)dt, a, (hipStream_t)stream);
  if (err != hipSuccess) return fail(POLAR_ERR_HIP, "prefill launch: %s", hipGetErrorString(err));
  return POLAR_OK;
}

// Shape limits of the backward: 32-bit byte offsets over q/du rows and K/V rows.
bool bwd_shape_ok(int32_t B, int32_t T, int32_t Hq, int32_t Hkv) {
  const long long d2 = polar::kHeadDim * 2;
  return ((long long)T + 64) * Hq * d2 < 0x7fffffffLL &&
         ((long long)T + 64) * Hkv * d2 < 0x7fffffffLL &&
         (long long)B * T * Hq < (1LL << 34);
}

}  // namespace

extern "C" {

polar_status polar_attn_fwd(const polar_params *p, polar_dtype dt, int32_t B, int32_t T,
                            const void *q, const void *k, const void *v,
                            const polar_outputs *out, void *stream) {
  return prefill(p, dt, B, T, q, k, v, out, nullptr, nullptr, stream);
}

polar_status polar_attn_fwd_mixed(const polar_params *p, polar_dtype dt, int32_t B, int32_t T,
                                  const void *q, const void *k, const void *v,
                                  const float *memory, float *mixed, const polar_outputs *out,
                                  void *stream) {
  if (!out) return fail(POLAR_ERR_NULL_POINTER, "outputs is NULL");
  if (out->dir || out->count)
    return fail(POLAR_ERR_UNSUPPORTED,
                "outputs.dir and outputs.count must be NULL: the mixed output replaces them");
  if (B > 0 && T > 0) {
    if (!mixed) return fail(POLAR_ERR_NULL_POINTER, "mixed is NULL");
    if (!aligned16(mixed) || (memory && !aligned16(memory)))
      return fail(POLAR_ERR_MISALIGNED, "mixed and memory must be 16-byte aligned");
    if (p && p->count_vec && !aligned16(p->count_vec))
      return fail(POLAR_ERR_MISALIGNED, "count_vec must be 16-byte aligned");
  }
  polar_outputs o = *out;
  o.dir = mixed;             // validated as the vector output
  return prefill(p, dt, B, T, q, k, v, &o, nullptr, nullptr, stream, nullptr, mixed, memory);
}

size_t polar_variant_workspace_bytes(const polar_params *p, polar_dtype dt, int32_t B,
                                     int32_t T) {
  if (!p || B < 0 || T < 0 || p->n_kv_heads < 1 ||
      (dt != POLAR_DTYPE_BF16 && dt != POLAR_DTYPE_F32))
    return 0;
  return (size_t)B * T * p->n_kv_heads * polar::kHeadDim * (dt == POLAR_DTYPE_BF16 ? 2 : 4);
}

polar_status polar_attn_fwd_variant(const polar_params *p, const polar_variant *var,
                                    polar_dtype dt, int32_t B, int32_t T, const void *q,
                                    const void *k, const void *v, const polar_outputs *out,
                                    void *stream) {
  return prefill(p, dt, B, T, q, k, v, out, nullptr, var, stream);
}

polar_status polar_attn_fwd_train(const polar_params *p, polar_dtype dt, int32_t B, int32_t T,
                                  const void *q, const void *k, const void *v,
                                  const polar_outputs *out, const polar_saved *saved,
                                  void *stream) {
  if (!saved) return fail(POLAR_ERR_NULL_POINTER, "saved is NULL");
  return prefill(p, dt, B, T, q, k, v, out, saved, nullptr, stream);
}

size_t polar_train_variant_workspace_bytes(const polar_params *p, const polar_variant *var,
                                           polar_dtype dt, int32_t B, int32_t T) {
  if (!p || B < 0 || T < 0 || p->n_kv_heads < 1 || p->n_q_heads < 1 ||
      (dt != POLAR_DTYPE_BF16 && dt != POLAR_DTYPE_F32) || check_variant(var) != POLAR_OK)
    return 0;
  if (!var || var->rope_theta == 0.f) return 0;
  return (size_t)B * T * (p->n_q_heads + p->n_kv_heads) * polar::kHeadDim *
         (dt == POLAR_DTYPE_BF16 ? 2 : 4);
}

polar_status polar_attn_fwd_train_variant(const polar_params *p, const polar_variant *var,
                                          polar_dtype dt, int32_t B, int32_t T, const void *q,
                                          const void *k, const void *v,
                                          const polar_outputs *out, const polar_saved *saved,
                                          void *stream) {
  if (!saved) return fail(POLAR_ERR_NULL_POINTER, "saved is NULL");
  polar_status st = check_variant(var);
  if (st != POLAR_OK) return st;
  if (var && var->attn && !aligned16(var->attn))
    return fail(POLAR_ERR_MISALIGNED, "variant attn output must be 16-byte aligned");
  // The window and the read-out go to the training instance; a rotation is done here,
  // into the workspace.
  polar_variant w{};
  w.window = var ? var->window : 0;
  w.attn = var ? var->attn : nullptr;
  const float theta = var ? var->rope_theta : 0.f;
  if (theta == 0.f) return prefill(p, dt, B, T, q, k, v, out, saved, &w, stream);
  st = check_params(p, dt, out);
  if (st != POLAR_OK) return st;
  if (B < 0 || T < 0) return fail(POLAR_ERR_BAD_SHAPE, "B (%d) and T (%d) must be >= 0", B, T);
  if (B == 0 || T == 0) return POLAR_OK;
  if (!q || !k || !v) return fail(POLAR_ERR_NULL_POINTER, "q, k and v must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(POLAR_ERR_MISALIGNED, "q, k and v must be 16-byte aligned");
  if (!var->workspace) return fail(POLAR_ERR_NULL_POINTER, "RoPE needs var.workspace");
  if (!aligned16(var->workspace))
    return fail(POLAR_ERR_MISALIGNED, "variant workspace must be 16-byte aligned");
  const size_t need = polar_train_variant_workspace_bytes(p, var, dt, B, T);
  if (var->workspace_bytes < need)
    return fail(POLAR_ERR_WORKSPACE_TOO_SMALL, "variant workspace has %zu bytes, needs %zu",
                var->workspace_bytes, need);
  const size_t qbytes =
      (size_t)B * T * p->n_q_heads * polar::kHeadDim * (dt == POLAR_DTYPE_BF16 ? 2 : 4);
  char *qr = (char *)var->workspace, *kr = qr + qbytes;
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = rotate_qk(dt, q, k, qr, kr, B, T, p->n_q_heads, p->n_kv_heads, theta, s);
  if (e != hipSuccess) return fail(POLAR_ERR_HIP, "rotation launch: %s", hipGetErrorString(e));
  return prefill(p, dt, B, T, qr, kr, v, out, saved, &w, stream);
}

size_t polar_bwd_workspace_bytes(const polar_params *p, int32_t B, int32_t T) {
  if (!p || B < 1 || T < 1 || p->n_kv_heads < 1 || p->n_q_heads < 1 ||
      p->n_q_heads % p->n_kv_heads != 0 || !bwd_shape_ok(B, T, p->n_q_heads, p->n_kv_heads))
    return 0;
  return polar::bwd_ws_bytes(B, T, p->n_q_heads, p->n_kv_heads);
}

// The backward, with the variant's window and rotation (var may be NULL).
static polar_status bwd_impl(const polar_params *p, const polar_variant *var, polar_dtype dt,
                             int32_t B, int32_t T, const void *q, const void *k, const void *v,
                             const polar_outputs *fwd, const polar_saved *saved,
                             const polar_cotangents *cot, const polar_grads *grads,
                             void *workspace, size_t workspace_bytes, void *stream) {
  polar_status st = check_params(p, dt, fwd);
  if (st != POLAR_OK) return st;
  st = check_variant(var);
  if (st != POLAR_OK) return st;
  if (var && var->attn)
    return fail(POLAR_ERR_UNSUPPORTED,
                "the backward takes no var.attn (the read-out's gradient is cot.attn)");
  const int window = var ? var->window : 0;
  const float theta = var ? var->rope_theta : 0.f;
  if (dt != POLAR_DTYPE_BF16)
    return fail(POLAR_ERR_UNSUPPORTED, "the backward pass takes bf16 inputs only");
  if (!saved || !cot || !grads)
    return fail(POLAR_ERR_NULL_POINTER, "saved, cot and grads must be non-NULL");
  if (B < 0 || T < 0) return fail(POLAR_ERR_BAD_SHAPE, "B (%d) and T (%d) must be >= 0", B, T);
  if (cot->count && !p->count_vec)
    return fail(POLAR_ERR_NULL_POINTER, "cot.count given but params.count_vec is NULL");
  const int Hq = p->n_q_heads;
  if (B == 0 || T == 0) {
    hipStream_t zs = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (grads->d_beta && e == hipSuccess) e = polar::launch_zero(grads->d_beta, Hq, zs);
    if (grads->d_null_bias && e == hipSuccess) e = polar::launch_zero(grads->d_null_bias, Hq, zs);
    if (grads->d_count_vec && e == hipSuccess)
      e = polar::launch_zero(grads->d_count_vec, (long long)Hq * p->head_dim, zs);
    if (e != hipSuccess) return fail(POLAR_ERR_HIP, "zero fill: %s", hipGetErrorString(e));
    return POLAR_OK;
  }
  if (!q || !k || !v) return fail(POLAR_ERR_NULL_POINTER, "q, k and v must be non-NULL");
  if (!fwd->dir || !fwd->n_eff || !fwd->gate || !fwd->lse)
    return fail(POLAR_ERR_NULL_POINTER, "fwd.dir, fwd.n_eff, fwd.gate and fwd.lse are required");
  if (!saved->u_norm || !saved->arg_max)
    return fail(POLAR_ERR_NULL_POINTER, "saved.u_norm and saved.arg_max must be non-NULL");
  if (!grads->dq || !grads->dk || !grads->dv)
    return fail(POLAR_ERR_NULL_POINTER, "grads.dq, grads.dk and grads.dv are required");
  if (!workspace) return fail(POLAR_ERR_NULL_POINTER, "workspace is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(fwd->dir) ||
      !aligned16(grads->dq) || !aligned16(grads->dk) || !aligned16(grads->dv) ||
      (cot->dir && !aligned16(cot->dir)) || (cot->count && !aligned16(cot->count)) ||
      (cot->attn && !aligned16(cot->attn)) || (cot->count && !aligned16(p->count_vec)))
    return fail(POLAR_ERR_MISALIGNED,
                "q, k, v, fwd.dir, cot.dir, cot.count, cot.attn, count_vec, dq, dk, dv must be "
                "16-byte aligned");
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(POLAR_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (!bwd_shape_ok(B, T, Hq, p->n_kv_heads))
    return fail(POLAR_ERR_BAD_SHAPE, "T*Hq too large for the backward (B=%d, T=%d, Hq=%d)", B,
                T, Hq);
  const size_t base = polar::bwd_ws_bytes(B, T, Hq, p->n_kv_heads);
  const size_t qbytes = (size_t)B * T * Hq * polar::kHeadDim * 2;
  const size_t kbytes = (size_t)B * T * p->n_kv_heads * polar::kHeadDim * 2;
  const size_t need = theta > 0.f ? align256(base) + align256(qbytes) + kbytes : base;
  if (workspace_bytes < need)
    return fail(POLAR_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed",
                workspace_bytes, need);

  hipStream_t s = (hipStream_t)stream;
  if (theta > 0.f) {
    // The kernels run on the rotated q and k, held after the backward's own workspace.
    char *qr = (char *)workspace + align256(base);
    char *kr = qr + align256(qbytes);
    hipError_t e = rotate_qk(dt, q, k, qr, kr, B, T, Hq, p->n_kv_heads, theta, s);
    if (e != hipSuccess) return fail(POLAR_ERR_HIP, "rotation launch: %s", hipGetErrorString(e));
    q = qr;
    k = kr;
  }

  polar::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = p->beta;
  a.null_bias = p->null_bias;
  a.count_vec = p->count_vec;
  a.dir = fwd->dir;
  a.n_eff = fwd->n_eff;
  a.gate = fwd->gate;
  a.lse = fwd->lse;
  a.u_norm = saved->u_norm;
  a.arg_max = saved->arg_max;
  a.c_dir = cot->dir;
  a.c_count = cot->count;
  a.c_n_eff = cot->n_eff;
  a.c_gate = cot->gate;
  a.c_lse = cot->lse;
  a.c_attn = cot->attn;
  a.dq = grads->dq;
  a.dk = grads->dk;
  a.dv = grads->dv;
  a.d_beta = grads->d_beta;
  a.d_null_bias = grads->d_null_bias;
  a.d_count_vec = grads->d_count_vec;
  a.B = B;
  a.T = T;
  a.Hq = Hq;
  a.Hkv = p->n_kv_heads;
  a.G = a.Hq / a.Hkv;
  a.hb = polar::prefill_heads_per_block(a.G);
  const int rows = polar::bwd_rows_per_block(a.hb);
  a.n_row_blocks = (T + rows - 1) / rows;
  const int keys = polar::bwd_keys_per_block();
  a.n_key_blocks = (T + keys - 1) / keys;
  a.hsplit = polar::bwd_head_split(a.G);
  a.inv_log_train = inv_log_train(p);
  a.null_floor = (p->flags & POLAR_FLAG_NULL_FLOOR) ? 1 : 0;
  a.window = window;
  a.rope = theta > 0.f ? 1 : 0;
  fill_rope_f(a.rope_f, theta);
  polar::bwd_ws_layout(a, workspace);
  const long long dq_blocks = (long long)a.n_row_blocks * a.Hkv * (a.G / a.hb) * B;
  const long long dkv_blocks = (long long)((a.n_key_blocks + 1) / 2) * a.hsplit * a.Hkv * B;
  if (dq_blocks > 0x7fffffffLL || dkv_blocks > 0x7fffffffLL)
    return fail(POLAR_ERR_BAD_SHAPE, "problem too large for one launch");
  // With RoPE the dq and dk/dv kernels turn their outputs back by the transposed rotation,
  // so the gradients are with respect to the unrotated q and k.
  hipError_t err = polar::launch_bwd(a, s);
  if (err != hipSuccess) return fail(POLAR_ERR_HIP, "backward launch: %s", hipGetErrorString(err));
  return POLAR_OK;
}

polar_status polar_attn_bwd(const polar_params *p, polar_dtype dt, int32_t B, int32_t T,
                            const void *q, const void *k, const void *v,
                            const polar_outputs *fwd, const polar_saved *saved,
                            const polar_cotangents *cot, const polar_grads *grads,
                            void *workspace, size_t workspace_bytes, void *stream) {
  return bwd_impl(p, nullptr, dt, B, T, q, k, v, fwd, saved, cot, grads, workspace,
                  workspace_bytes, stream);
}

polar_status polar_attn_bwd_variant(const polar_params *p, const polar_variant *var,
                                    polar_dtype dt, int32_t B, int32_t T, const void *q,
                                    const void *k, const void *v, const polar_outputs *fwd,
                                    const polar_saved *saved, const polar_cotangents *cot,
                                    const polar_grads *grads, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  return bwd_impl(p, var, dt, B, T, q, k, v, fwd, saved, cot, grads, workspace,
                  workspace_bytes, stream);
}

size_t polar_bwd_variant_workspace_bytes(const polar_params *p, const polar_variant *var,
                                         int32_t B, int32_t T) {
  const size_t base = polar_bwd_workspace_bytes(p, B, T);
  if (base == 0 || check_variant(var) != POLAR_OK) return 0;
  if (!var || var->rope_theta == 0.f) return base;
  const size_t qbytes = (size_t)B * T * p->n_q_heads * polar::kHeadDim * 2;
  const size_t kbytes = (size_t)B * T * p->n_kv_heads * polar::kHeadDim * 2;
  return align256(base) + align256(qbytes) + kbytes;
}

size_t polar_decode_workspace_bytes(const polar_params *p, int32_t B, int32_t max_seq_len) {
  if (!p || B < 1 || max_seq_len < 1 || p->n_kv_heads < 1 ||
      p->n_q_heads < 1 || p->n_q_heads % p->n_kv_heads != 0)
    return 0;
  return polar::decode_ws_bytes(B, p->n_q_heads, p->n_kv_heads, max_seq_len);
}

}  // extern "C"

namespace {

// The paged decode; with no_alloc the split partials go to the library's static scratch
// (workspace and workspace_bytes are ignored) instead of the caller's workspace.
polar_status decode(const polar_params *p, polar_dtype dt, int32_t B, const void *q,
                    const void *k_cache, const void *v_cache, int32_t num_pages,
                    int32_t page_size, const int32_t *page_table, int32_t page_table_stride,
                    const int32_t *seq_lens, int32_t max_seq_len, void *workspace,
                    size_t workspace_bytes, const polar_outputs *out, void *stream,
                    bool no_alloc) {
  polar_status st = check_params(p, dt, out);
  if (st != POLAR_OK) return st;
  if (B < 0) return fail(POLAR_ERR_BAD_SHAPE, "B (%d) must be >= 0", B);
  if (page_size != polar::kPageSize)
    return fail(POLAR_ERR_UNSUPPORTED, "page_size %d unsupported (only %d)", page_size,
                polar::kPageSize);
  if (B == 0) return POLAR_OK;
  st = check_outputs(p, out);
  if (st != POLAR_OK) return st;
  if (!q || !k_cache || !v_cache || !page_table || !seq_lens || (!no_alloc && !workspace))
    return fail(POLAR_ERR_NULL_POINTER,
                no_alloc ? "q, k_cache, v_cache, page_table and seq_lens must be non-NULL"
                         : "q, k_cache, v_cache, page_table, seq_lens and workspace must be "
                           "non-NULL");
  if (num_pages < 1) return fail(POLAR_ERR_BAD_SHAPE, "num_pages (%d) must be >= 1", num_pages);
  if (max_seq_len < 1)
    return fail(POLAR_ERR_BAD_SHAPE, "max_seq_len (%d) must be >= 1", max_seq_len);
  const int need_pages = (max_seq_len + page_size - 1) / page_size;
  if (page_table_stride < need_pages)
    return fail(POLAR_ERR_BAD_SHAPE, "page_table_stride (%d) < ceil(max_seq_len/page_size) (%d)",
                page_table_stride, need_pages);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (!no_alloc && !aligned16(workspace)))
    return fail(POLAR_ERR_MISALIGNED, "q, caches and workspace must be 16-byte aligned");
  const size_t need = polar::decode_ws_bytes(B, p->n_q_heads, p->n_kv_heads, max_seq_len);
  if (no_alloc && need > polar::kNoAllocScratchBytes)
    return fail(POLAR_ERR_WORKSPACE_TOO_SMALL,
                "this decode needs %zu bytes of split partials; the static scratch of the "
                "allocation-free entry point holds %zu (use polar_attn_decode_paged with a "
                "workspace)", need, polar::kNoAllocScratchBytes);
  if (!no_alloc && workspace_bytes < need)
    return fail(POLAR_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed",
                workspace_bytes, need);

  const polar::DecodeGrid grid =
      polar::decode_grid(B, p->n_q_heads, p->n_kv_heads, max_seq_len);
  if ((long long)p->n_kv_heads * grid.n_hchunk > 65535 || B > 65535)
    return fail(POLAR_ERR_BAD_SHAPE, "grid too large (B=%d, Hkv*chunks=%lld)", B,
                (long long)p->n_kv_heads * grid.n_hchunk);
  if (no_alloc) {
    // Every argument has been checked; now the scratch's address on this device.
    const hipError_t e = polar::noalloc_scratch(&workspace);
    if (e != hipSuccess)
      return fail(POLAR_ERR_HIP, "scratch lookup: %s", hipGetErrorString(e));
  }
  polar::DecodeArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.beta = p->beta;
  a.null_bias = p->null_bias;
  a.count_vec = p->count_vec;
  a.dir = out->dir;
  a.count = out->count;
  a.n_eff = out->n_eff;
  a.gate = out->gate;
  a.lse = out->lse;
  a.ws = (float *)workspace;
  a.B = B;
  a.Hq = p->n_q_heads;
  a.Hkv = p->n_kv_heads;
  a.G = a.Hq / a.Hkv;
  a.num_pages = num_pages;
  a.stride = page_table_stride;
  a.max_seq_len = max_seq_len;
  a.n_split = grid.n_split;
  a.pages_per_split = grid.pages_per_split;
  a.n_hchunk = grid.n_hchunk;
  a.inv_log_train = inv_log_train(p);
  a.null_floor = (p->flags & POLAR_FLAG_NULL_FLOOR) ? 1 : 0;
  hipError_t err = polar::launch_decode((int)dt, a, (hipStream_t)stream);
  if (err != hipSuccess) return fail(POLAR_ERR_HIP, "decode launch: %s", hipGetErrorString(err));
  return POLAR_OK;
}

}  // namespace

extern "C" {

polar_status polar_attn_decode_paged(const polar_params *p, polar_dtype dt, int32_t B,
                                     const void *q, const void *k_cache, const void *v_cache,
                                     int32_t num_pages, int32_t page_size,
                                     const int32_t *page_table, int32_t page_table_stride,
                                     const int32_t *seq_lens, int32_t max_seq_len,
                                     void *workspace, size_t workspace_bytes,
                                     const polar_outputs *out, void *stream) {
  return decode(p, dt, B, q, k_cache, v_cache, num_pages, page_size, page_table,
                page_table_stride, seq_lens, max_seq_len, workspace, workspace_bytes, out,
                stream, false);
}

polar_status polar_attn_decode_paged_noalloc(const polar_params *p, polar_dtype dt, int32_t B,
                                             const void *q, const void *k_cache,
                                             const void *v_cache, int32_t num_pages,
                                             int32_t page_size, const int32_t *page_table,
                                             int32_t page_table_stride, const int32_t *seq_lens,
                                             int32_t max_seq_len, const polar_outputs *out,
                                             void *stream) {
  return decode(p, dt, B, q, k_cache, v_cache, num_pages, page_size, page_table,
                page_table_stride, seq_lens, max_seq_len, nullptr, 0, out, stream, true);
}

polar_status polar_kv_append(const polar_params *p, polar_dtype dt, int32_t B, int32_t C,
                             const void *k_new, const void *v_new, void *k_cache,
                             void *v_cache, int32_t num_pages, int32_t page_size,
                             const int32_t *page_table, int32_t page_table_stride,
                             const int32_t *start_pos, int32_t max_seq_len, void *stream) {
  if (!p) return fail(POLAR_ERR_NULL_POINTER, "params is NULL");
  if (dt != POLAR_DTYPE_F32 && dt != POLAR_DTYPE_BF16)
    return fail(POLAR_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (p->n_kv_heads < 1) return fail(POLAR_ERR_BAD_SHAPE, "Hkv must be >= 1");
  if (p->head_dim != polar::kHeadDim)
    return fail(POLAR_ERR_UNSUPPORTED, "head_dim %d unsupported (only %d)", p->head_dim,
                polar::kHeadDim);
  if (page_size != polar::kPageSize)
    return fail(POLAR_ERR_UNSUPPORTED, "page_size %d unsupported (only %d)", page_size,
                polar::kPageSize);
  if (B < 0 || C < 0) return fail(POLAR_ERR_BAD_SHAPE, "B (%d) and C (%d) must be >= 0", B, C);
  if (B == 0 || C == 0) return POLAR_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !page_table || !start_pos)
    return fail(POLAR_ERR_NULL_POINTER, "tensors, page_table and start_pos must be non-NULL");
  if (num_pages < 1) return fail(POLAR_ERR_BAD_SHAPE, "num_pages (%d) must be >= 1", num_pages);
  if (max_seq_len < C)
    return fail(POLAR_ERR_BAD_SHAPE, "max_seq_len (%d) < C (%d)", max_seq_len, C);
  if (page_table_stride < (max_seq_len + page_size - 1) / page_size)
    return fail(POLAR_ERR_BAD_SHAPE, "page_table_stride (%d) < ceil(max_seq_len/page_size)",
                page_table_stride);
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(POLAR_ERR_MISALIGNED, "k_new, v_new and the pools must be 16-byte aligned");
  polar::AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_table = page_table;
  a.start_pos = start_pos;
  a.B = B;
  a.C = C;
  a.Hkv = p->n_kv_heads;
  a.stride = page_table_stride;
  a.num_pages = num_pages;
  a.max_seq_len = max_seq_len;
  a.row_bytes = polar::kHeadDim * (dt == POLAR_DTYPE_BF16 ? 2 : 4);
  hipError_t err = polar::launch_kv_append(a, (hipStream_t)stream);
  if (err != hipSuccess) return fail(POLAR_ERR_HIP, "append launch: %s", hipGetErrorString(err));
  return POLAR_OK;
}

polar_status polar_attn_prefill_paged(const polar_params *p, polar_dtype dt, int32_t B,
                                      int32_t C, const void *q, const void *k_cache,
                                      const void *v_cache, int32_t num_pages, int32_t page_size,
                                      const int32_t *page_table, int32_t page_table_stride,
                                      const int32_t *start_pos, int32_t max_seq_len,
                                      const polar_outputs *out, void *stream) {
  polar_status st = check_params(p, dt, out);
  if (st != POLAR_OK) return st;
  if (page_size != polar::kPageSize)
    return fail(POLAR_ERR_UNSUPPORTED, "page_size %d unsupported (only %d)", page_size,
                polar::kPageSize);
  if (B < 0 || C < 0) return fail(POLAR_ERR_BAD_SHAPE, "B (%d) and C (%d) must be >= 0", B, C);
  if (B == 0 || C == 0) return POLAR_OK;
  if (!page_table || !start_pos)
    return fail(POLAR_ERR_NULL_POINTER, "page_table and start_pos must be non-NULL");
  if (num_pages < 1) return fail(POLAR_ERR_BAD_SHAPE, "num_pages (%d) must be >= 1", num_pages);
  if (max_seq_len < C)
    return fail(POLAR_ERR_BAD_SHAPE, "max_seq_len (%d) < C (%d)", max_seq_len, C);
  if (page_table_stride < (max_seq_len + page_size - 1) / page_size)
    return fail(POLAR_ERR_BAD_SHAPE, "page_table_stride (%d) < ceil(max_seq_len/page_size)",
                page_table_stride);
  const PagedSrc src{page_table, start_pos, page_table_stride, num_pages, max_seq_len};
  return prefill(p, dt, B, C, q, k_cache, v_cache, out, nullptr, nullptr, stream, &src);
}

namespace {
// Checks shared by the step and the sequence entry points.
polar_status delta_params_ok(const polar_delta_params *p, polar_dtype dt) {
  if (!p) return fail(POLAR_ERR_NULL_POINTER, "params is NULL");
  if (dt != POLAR_DTYPE_F32 && dt != POLAR_DTYPE_BF16)
    return fail(POLAR_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (p->n_heads < 1) return fail(POLAR_ERR_BAD_SHAPE, "n_heads must be >= 1");
  if (p->key_dim != polar::kHeadDim || p->value_dim != polar::kHeadDim)
    return fail(POLAR_ERR_UNSUPPORTED, "key_dim and value_dim must be %d", polar::kHeadDim);
  if (p->flags & ~(uint32_t)POLAR_DELTA_NORMALIZE_QK)
    return fail(POLAR_ERR_UNSUPPORTED, "unknown flag bits 0x%x", p->flags);
  return POLAR_OK;
}
}  // namespace

polar_status polar_delta_step(const polar_delta_params *p, polar_dtype dt, int32_t B,
                              float *state_pool, int32_t num_slots, const int32_t *slots,
                              const void *q, const void *k, const void *v, const float *alpha,
                              const float *beta, float *out, void *stream) {
  if (polar_status st = delta_params_ok(p, dt)) return st;
  if (B < 0) return fail(POLAR_ERR_BAD_SHAPE, "B (%d) must be >= 0", B);
  if (B == 0) return POLAR_OK;
  if (!state_pool || !slots || !q || !k || !v || !alpha || !beta || !out)
    return fail(POLAR_ERR_NULL_POINTER, "all tensors must be non-NULL");
  if (num_slots < 1) return fail(POLAR_ERR_BAD_SHAPE, "num_slots (%d) must be >= 1", num_slots);
  if ((long long)B * p->n_heads > 0x7fffffffLL)
    return fail(POLAR_ERR_BAD_SHAPE, "B*H too large for one launch");
  if (!aligned16(state_pool) || !aligned16(q) || !aligned16(k) || !aligned16(out))
    return fail(POLAR_ERR_MISALIGNED, "state_pool, q, k and out must be 16-byte aligned");
  polar::DeltaArgs a;
  a.pool = state_pool;
  a.slots = slots;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.out = out;
  a.B = B;
  a.H = p->n_heads;
  a.num_slots = num_slots;
  a.normalize = (p->flags & POLAR_DELTA_NORMALIZE_QK) ? 1 : 0;
  hipError_t err = polar::launch_delta_step((int)dt, a, (hipStream_t)stream);
  if (err != hipSuccess) return fail(POLAR_ERR_HIP, "delta step launch: %s", hipGetErrorString(err));
  return POLAR_OK;
}

polar_status polar_delta_sequence(const polar_delta_params *p, polar_dtype dt, int32_t B,
                                  int32_t T, float *state_pool, int32_t num_slots,
                                  const int32_t *slots, const void *q, const void *k,
                                  const void *v, const float *alpha, const float *beta,
                                  float *out, void *stream) {
  if (polar_status st = delta_params_ok(p, dt)) return st;
  if (B < 0 || T < 0) return fail(POLAR_ERR_BAD_SHAPE, "B (%d) and T (%d) must be >= 0", B, T);
  if (B == 0 || T == 0) return POLAR_OK;
  if (!state_pool || !slots || !q || !k || !v || !alpha || !beta || !out)
    return fail(POLAR_ERR_NULL_POINTER, "all tensors must be non-NULL");
  if (num_slots < 1) return fail(POLAR_ERR_BAD_SHAPE, "num_slots (%d) must be >= 1", num_slots);
  if (2LL * B * p->n_heads > 0x7fffffffLL)
    return fail(POLAR_ERR_BAD_SHAPE, "B*H too large for one launch");
  if ((long long)B * T * p->n_heads > (1LL << 56))
    return fail(POLAR_ERR_BAD_SHAPE, "B*T*H too large");
  if (!aligned16(state_pool) || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
      !aligned16(out))
    return fail(POLAR_ERR_MISALIGNED, "state_pool, q, k, v and out must be 16-byte aligned");
  polar::DeltaSeqArgs a;
  a.pool = state_pool;
  a.slots = slots;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.out = out;
  a.B = B;
  a.T = T;
  a.H = p->n_heads;
  a.num_slots = num_slots;
  a.normalize = (p->flags & POLAR_DELTA_NORMALIZE_QK) ? 1 : 0;
  hipError_t err = polar::launch_delta_sequence((int)dt, a, (hipStream_t)stream);
  if (err != hipSuccess)
    return fail(POLAR_ERR_HIP, "delta sequence launch: %s", hipGetErrorString(err));
  return POLAR_OK;
}

const char *polar_status_str(polar_status s) {
  switch (s) {
    case POLAR_OK: return "ok";
    case POLAR_ERR_NULL_POINTER: return "null pointer";
    case POLAR_ERR_BAD_SHAPE: return "bad shape";
    case POLAR_ERR_UNSUPPORTED: return "unsupported";
    case POLAR_ERR_MISALIGNED: return "misaligned pointer";
    case POLAR_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case POLAR_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char *polar_last_error(void) { return g_last_error; }

int32_t polar_abi_version(void) { return POLAR_ABI_VERSION; }

}  // extern "C"
