// C ABI of libjetlong: argument validation and dispatch (include/jetlong.h).
//
// Every argument is checked before any HIP call; a failing call enqueues
// nothing and leaves a message for jl_last_error() on the calling thread.
#include <math.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>

#include "../../include/jetlong.h"
#include "jl_launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return JL_OK;
  return fail(JL_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool supported_dim(int d) { return d == 64 || d == 128; }
bool supported_dtype(int t) { return t == JL_F32 || t == JL_BF16; }

int check_common(int dtype, int Hq, int Hkv, int head_dim, int w_pretrained, int w0,
                 double theta, float scale) {
  if (!supported_dtype(dtype)) return fail(JL_ERR_UNSUPPORTED, "dtype %d not supported (JL_F32 or JL_BF16)", dtype);
  if (!supported_dim(head_dim)) return fail(JL_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (Hq < 1 || Hkv < 1) return fail(JL_ERR_INVALID_ARG, "Hq=%d and Hkv=%d must be >= 1", Hq, Hkv);
  if (Hq % Hkv) return fail(JL_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (w_pretrained < 1) return fail(JL_ERR_INVALID_ARG, "w_pretrained=%d must be >= 1", w_pretrained);
  if (w0 < 0) return fail(JL_ERR_INVALID_ARG, "w0=%d must be >= 0", w0);
  if (!(theta > 0.0) || !isfinite(theta)) return fail(JL_ERR_INVALID_ARG, "rope_theta must be finite and > 0");
  if (!(scale >= 0.f) || !isfinite(scale)) return fail(JL_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  return JL_OK;
}

float resolve_scale(float scale, int head_dim) {
  return scale == 0.f ? static_cast<float>(1.0 / sqrt(static_cast<double>(head_dim))) : scale;
}

}  // namespace

extern "C" {

int64_t jl_bifocal_group_size(int64_t L, int64_t w_pretrained) {
  if (L < 0 || w_pretrained < 1) {
    fail(JL_ERR_INVALID_ARG, "group_size needs L >= 0 and w_pretrained >= 1");
    return JL_ERR_INVALID_ARG;
  }
  const int64_t g = L / w_pretrained + (L % w_pretrained != 0);
  return g < 1 ? 1 : g;
}

size_t jl_bifocal_prefill_workspace_size(int dtype, int B, int total_k, int max_seqlen_k, int Hq,
                                         int Hkv, int head_dim) {
  if (!supported_dtype(dtype) || !supported_dim(head_dim) || B < 0 || total_k < 0 ||
      max_seqlen_k < 0 || Hq < 1 || Hkv < 1)
    return 0;
  if (dtype == JL_BF16) return jl::prefill_ws_bytes_bf16(B, total_k, max_seqlen_k, Hkv, head_dim);
  return jl::prefill_ws_bytes_f32(max_seqlen_k, head_dim);
}

size_t jl_bifocal_prefill_ie_workspace_size(int dtype, int B, int total_q, int total_k, int max_seqlen_k, int Hq,
                                            int Hkv, int head_dim) {
  if (!supported_dtype(dtype) || !supported_dim(head_dim) || B < 0 || total_q < 0 || total_k < 0 ||
      max_seqlen_k < 0 || Hq < 1 || Hkv < 1)
    return 0;
  return jl::prefill_ie_ws_bytes(dtype == JL_BF16, B, total_q, total_k, max_seqlen_k, Hq, Hkv, head_dim);
}

}  // extern "C"

namespace {

// Checks a full prefill argument list and fills `c`; JL_OK with c.B == 0 or
// c.total_q == 0 means there is nothing to launch.
// bf16 prefill: the attention kernel addresses one KV head's rotated keys
// and V^T tiles with 32-bit byte offsets below 2^31, i.e. padded keys
// (roundup64(total_k) + 64 B) times 2 head_dim bytes.
int check_bf16_key_span(int dtype, int B, int total_k, int head_dim) {
  if (dtype != JL_BF16) return JL_OK;
  const int64_t tpad = (static_cast<int64_t>(total_k) + 63) / 64 * 64 + 64LL * B;
  if (tpad * head_dim * 2 > INT32_MAX)
    return fail(JL_ERR_UNSUPPORTED, "bf16 prefill of %lld padded keys x head_dim %d exceeds 2^31 bytes per KV head",
                static_cast<long long>(tpad), head_dim);
  return JL_OK;
}

int prefill_args(const void* q, const void* k, const void* v, void* o, float* lse, int dtype,
                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int total_q,
                 int total_k, int max_seqlen_q, int max_seqlen_k, int Hq, int Hkv, int head_dim,
                 int w_pretrained, int w0, double rope_theta, float softmax_scale, const void* workspace,
                 size_t workspace_bytes, jl::PrefillCall* c, bool ie = false) {
  *c = jl::PrefillCall{};
  int st = check_common(dtype, Hq, Hkv, head_dim, w_pretrained, w0, rope_theta, softmax_scale);
  if (st != JL_OK) return st;
  if (B < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(JL_ERR_INVALID_ARG, "sizes must be non-negative");
  if (total_q > total_k) return fail(JL_ERR_INVALID_ARG, "total_q=%d exceeds total_k=%d", total_q, total_k);
  if (max_seqlen_q > max_seqlen_k) return fail(JL_ERR_INVALID_ARG, "max_seqlen_q exceeds max_seqlen_k");
  if (B == 0 || total_q == 0) return JL_OK;
  st = check_bf16_key_span(dtype, B, total_k, head_dim);
  if (st != JL_OK) return st;
  if (!q || !k || !v || !o) return fail(JL_ERR_INVALID_ARG, "q, k, v and o must be non-null");
  if (!cu_seqlens_q) return fail(JL_ERR_INVALID_ARG, "cu_seqlens_q must be non-null");
  if (!cu_seqlens_k && total_k != total_q) return fail(JL_ERR_INVALID_ARG, "cu_seqlens_k is NULL but total_k != total_q");
  if (max_seqlen_k < 1) return fail(JL_ERR_INVALID_ARG, "max_seqlen_k must be >= 1 for a non-empty batch");
  const size_t need = ie ? jl_bifocal_prefill_ie_workspace_size(dtype, B, total_q, total_k, max_seqlen_k, Hq, Hkv, head_dim)
                        : jl_bifocal_prefill_workspace_size(dtype, B, total_k, max_seqlen_k, Hq, Hkv, head_dim);
  if (!workspace) return fail(JL_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (workspace_bytes < need) return fail(JL_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(JL_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  c->q = q; c->k = k; c->v = v; c->o = o; c->lse = lse;
  c->cu_q = cu_seqlens_q;
  c->cu_k = cu_seqlens_k ? cu_seqlens_k : cu_seqlens_q;
  c->B = B; c->total_q = total_q; c->total_k = total_k;
  c->max_q = max_seqlen_q; c->max_k = max_seqlen_k;
  c->Hq = Hq; c->Hkv = Hkv; c->D = head_dim;
  c->w_pretrained = w_pretrained; c->w0 = w0;
  c->theta = rope_theta;
  c->scale = resolve_scale(softmax_scale, head_dim);
  c->ws = const_cast<void*>(workspace);
  return JL_OK;
}

}  // namespace

extern "C" {

int jl_bifocal_prefill_ex(const void* q, const void* k, const void* v, void* o, float* lse, int dtype,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                          int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int Hq,
                          int Hkv, int head_dim, int w_pretrained, int w0, double rope_theta,
                          float softmax_scale, void* workspace, size_t workspace_bytes,
                          void* stream, unsigned flags) {
  if (flags & ~static_cast<unsigned>(JL_FLAG_PREROTATED)) return fail(JL_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  jl::PrefillCall c;
  const int st = prefill_args(q, k, v, o, lse, dtype, cu_seqlens_q, cu_seqlens_k, B, total_q, total_k,
                              max_seqlen_q, max_seqlen_k, Hq, Hkv, head_dim, w_pretrained, w0,
                              rope_theta, softmax_scale, workspace, workspace_bytes, &c);
  if (st != JL_OK || c.B == 0) return st;
  c.prerot = (flags & JL_FLAG_PREROTATED) != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = dtype == JL_BF16 ? jl::launch_prefill_bf16_prepare(c, s) : jl::launch_prefill_f32_prepare(c, s);
  if (e != hipSuccess) return hip_status(e, "jl_bifocal_prefill prepare launch");
  e = dtype == JL_BF16 ? jl::launch_prefill_bf16_attend(c, s) : jl::launch_prefill_f32_attend(c, s);
  return hip_status(e, "jl_bifocal_prefill attend launch");
}

int jl_bifocal_prefill_ie(const void* q, const void* k, const void* v, void* o, float* lse, int dtype,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int total_q,
                          int total_k, int max_seqlen_q, int max_seqlen_k, int Hq, int Hkv, int head_dim,
                          int w_pretrained, int w0, double rope_theta, float softmax_scale, void* workspace,
                          size_t workspace_bytes, void* stream, unsigned flags) {
  if (flags & ~static_cast<unsigned>(JL_FLAG_PREROTATED)) return fail(JL_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  jl::PrefillCall c;
  const int st = prefill_args(q, k, v, o, lse, dtype, cu_seqlens_q, cu_seqlens_k, B, total_q, total_k,
                              max_seqlen_q, max_seqlen_k, Hq, Hkv, head_dim, w_pretrained, w0,
                              rope_theta, softmax_scale, workspace, workspace_bytes, &c, true);
  if (st != JL_OK || c.B == 0) return st;
  c.prerot = (flags & JL_FLAG_PREROTATED) != 0;
  return hip_status(jl::launch_prefill_ie(c, dtype == JL_BF16, static_cast<hipStream_t>(stream)),
                    "jl_bifocal_prefill_ie launch");
}

int jl_bifocal_prefill_prepare_ex(const void* k, const void* v, int dtype, const int32_t* cu_seqlens_k,
                                  int B, int total_k, int max_seqlen_k, int Hkv, int head_dim,
                                  int w_pretrained, double rope_theta, void* workspace,
                                  size_t workspace_bytes, void* stream, unsigned flags) {
  if (flags & ~static_cast<unsigned>(JL_FLAG_PREROTATED)) return fail(JL_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  int st = check_common(dtype, Hkv, Hkv, head_dim, w_pretrained, 0, rope_theta, 0.f);
  if (st != JL_OK) return st;
  if (B < 0 || total_k < 0 || max_seqlen_k < 0) return fail(JL_ERR_INVALID_ARG, "sizes must be non-negative");
  if (B == 0 || total_k == 0) return JL_OK;
  st = check_bf16_key_span(dtype, B, total_k, head_dim);
  if (st != JL_OK) return st;
  if (!k || !v || !cu_seqlens_k) return fail(JL_ERR_INVALID_ARG, "k, v and cu_seqlens_k must be non-null");
  if (max_seqlen_k < 1) return fail(JL_ERR_INVALID_ARG, "max_seqlen_k must be >= 1 for a non-empty batch");
  const size_t need = jl_bifocal_prefill_workspace_size(dtype, B, total_k, max_seqlen_k, Hkv, Hkv, head_dim);
  if (!workspace) return fail(JL_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (workspace_bytes < need) return fail(JL_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(JL_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  jl::PrefillCall c{};
  c.k = k; c.v = v; c.cu_k = cu_seqlens_k;
  c.B = B; c.total_k = total_k; c.max_k = max_seqlen_k;
  c.Hq = Hkv; c.Hkv = Hkv; c.D = head_dim;
  c.w_pretrained = w_pretrained;
  c.theta = rope_theta;
  c.ws = workspace;
  c.prerot = (flags & JL_FLAG_PREROTATED) != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == JL_BF16 ? jl::launch_prefill_bf16_prepare(c, s) : jl::launch_prefill_f32_prepare(c, s);
  return hip_status(e, "jl_bifocal_prefill_prepare launch");
}

int jl_bifocal_prefill_attend_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                 int B, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                                 int Hq, int Hkv, int head_dim, int w_pretrained, int w0,
                                 double rope_theta, float softmax_scale, const void* workspace,
                                 size_t workspace_bytes, void* stream, unsigned flags) {
  if (flags & ~static_cast<unsigned>(JL_FLAG_PREROTATED)) return fail(JL_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  jl::PrefillCall c;
  const int st = prefill_args(q, k, v, o, lse, dtype, cu_seqlens_q, cu_seqlens_k, B, total_q, total_k,
                              max_seqlen_q, max_seqlen_k, Hq, Hkv, head_dim, w_pretrained, w0,
                              rope_theta, softmax_scale, workspace, workspace_bytes, &c);
  if (st != JL_OK || c.B == 0) return st;
  c.prerot = (flags & JL_FLAG_PREROTATED) != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == JL_BF16 ? jl::launch_prefill_bf16_attend(c, s) : jl::launch_prefill_f32_attend(c, s);
  return hip_status(e, "jl_bifocal_prefill_attend launch");
}

size_t jl_bifocal_decode_workspace_size(int dtype, int B, int max_L, int Hq, int Hkv, int head_dim) {
  if (!supported_dtype(dtype) || !supported_dim(head_dim) || B < 0 || max_L < 0 || Hq < 1 || Hkv < 1)
    return 0;
  return jl::decode_ws_bytes(B, max_L, Hq, Hkv, head_dim);
}

}  // extern "C"

namespace {

// Checks the arguments every decode entry point shares and fills `c`
// (workspace, table and partial-state pointers are left to the caller).
int decode_args(const void* q, const void* k_cache, const void* v_cache, int64_t stride_b, int64_t stride_s,
                int64_t stride_h, void* o, float* lse, int dtype, const int32_t* seq_L, int B, int max_L, int Hq,
                int Hkv, int head_dim, int w_pretrained, int w0, double rope_theta, float softmax_scale,
                unsigned flags, jl::DecodeCall* c) {
  *c = jl::DecodeCall{};
  if (flags & ~static_cast<unsigned>(JL_FLAG_PREROTATED)) return fail(JL_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  int st = check_common(dtype, Hq, Hkv, head_dim, w_pretrained, w0, rope_theta, softmax_scale);
  if (st != JL_OK) return st;
  if (Hq / Hkv > 16) return fail(JL_ERR_UNSUPPORTED, "decode supports up to 16 query heads per KV head (got %d)", Hq / Hkv);
  if (B < 0 || max_L < 0) return fail(JL_ERR_INVALID_ARG, "sizes must be non-negative");
  if (B == 0) return JL_OK;
  if (max_L < 1) return fail(JL_ERR_INVALID_ARG, "max_L must be >= 1");
  if (!q || !k_cache || !v_cache || !o || !seq_L) return fail(JL_ERR_INVALID_ARG, "q, caches, o and seq_L must be non-null");
  if (stride_b < 0 || stride_s < head_dim || stride_h < head_dim)
    return fail(JL_ERR_INVALID_ARG, "cache strides must be >= head_dim (got b=%lld s=%lld h=%lld)",
                static_cast<long long>(stride_b), static_cast<long long>(stride_s), static_cast<long long>(stride_h));
  if (dtype == JL_BF16 && (stride_b % 8 || stride_s % 8 || stride_h % 8))
    return fail(JL_ERR_INVALID_ARG, "bf16 cache strides must be multiples of 8 elements (16-byte rows)");
  if ((dtype == JL_BF16 && (reinterpret_cast<uintptr_t>(k_cache) % 16 || reinterpret_cast<uintptr_t>(v_cache) % 16 ||
                            reinterpret_cast<uintptr_t>(q) % 16)))
    return fail(JL_ERR_INVALID_ARG, "bf16 q and caches must be 16-byte aligned");
  c->q = q; c->kc = k_cache; c->vc = v_cache;
  c->sb = stride_b; c->ss = stride_s; c->sh = stride_h;
  c->o = o; c->lse = lse; c->seq_L = seq_L;
  c->B = B; c->max_L = max_L; c->Hq = Hq; c->Hkv = Hkv; c->D = head_dim;
  c->w_pretrained = w_pretrained; c->w0 = w0;
  c->theta = rope_theta;
  c->scale = resolve_scale(softmax_scale, head_dim);
  c->prerot = (flags & JL_FLAG_PREROTATED) != 0;
  return JL_OK;
}

int check_workspace(const void* workspace, size_t workspace_bytes, size_t need) {
  if (!workspace) return fail(JL_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (workspace_bytes < need) return fail(JL_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(JL_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return JL_OK;
}

}  // namespace

extern "C" {

int jl_bifocal_decode_ex(const void* q, const void* k_cache, const void* v_cache, int64_t stride_b,
                         int64_t stride_s, int64_t stride_h, void* o, float* lse, int dtype,
                         const int32_t* seq_L, int B, int max_L, int Hq, int Hkv, int head_dim,
                         int w_pretrained, int w0, double rope_theta, float softmax_scale,
                         void* workspace, size_t workspace_bytes, void* stream, unsigned flags) {
  jl::DecodeCall c;
  int st = decode_args(q, k_cache, v_cache, stride_b, stride_s, stride_h, o, lse, dtype, seq_L, B, max_L, Hq, Hkv,
                       head_dim, w_pretrained, w0, rope_theta, softmax_scale, flags, &c);
  if (st != JL_OK || c.B == 0) return st;
  st = check_workspace(workspace, workspace_bytes,
                       jl_bifocal_decode_workspace_size(dtype, B, max_L, Hq, Hkv, head_dim));
  if (st != JL_OK) return st;
  c.ws = workspace;
  return hip_status(jl::launch_decode(c, dtype == JL_BF16, static_cast<hipStream_t>(stream)),
                    "jl_bifocal_decode launch");
}

size_t jl_bifocal_rope_table_size(int max_pos, int head_dim) {
  if (max_pos < 0 || !supported_dim(head_dim)) return 0;
  return jl::rope_table_bytes(max_pos, head_dim);
}

int jl_bifocal_rope_table(int max_pos, int head_dim, double rope_theta, void* table, size_t table_bytes,
                          void* stream) {
  if (!supported_dim(head_dim)) return fail(JL_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (max_pos < 0) return fail(JL_ERR_INVALID_ARG, "max_pos must be non-negative");
  if (!(rope_theta > 0.0) || !isfinite(rope_theta)) return fail(JL_ERR_INVALID_ARG, "rope_theta must be finite and > 0");
  if (max_pos == 0) return JL_OK;
  const size_t need = jl::rope_table_bytes(max_pos, head_dim);
  if (!table) return fail(JL_ERR_INVALID_ARG, "table is NULL (%zu bytes needed)", need);
  if (table_bytes < need) return fail(JL_ERR_INVALID_ARG, "table has %zu bytes, %zu needed", table_bytes, need);
  if (reinterpret_cast<uintptr_t>(table) % 256) return fail(JL_ERR_INVALID_ARG, "table must be 256-byte aligned");
  return hip_status(jl::launch_rope_table_full(table, max_pos, head_dim, rope_theta, static_cast<hipStream_t>(stream)),
                    "jl_bifocal_rope_table launch");
}

size_t jl_bifocal_decode_with_table_workspace_size(int dtype, int B, int max_L, int Hq, int Hkv, int head_dim) {
  if (!supported_dtype(dtype) || !supported_dim(head_dim) || B < 0 || max_L < 0 || Hq < 1 || Hkv < 1)
    return 0;
  return jl::decode_part_bytes(dtype == JL_BF16, B, max_L, Hq, Hkv, head_dim);
}

int jl_bifocal_decode_with_table(const void* q, const void* k_cache, const void* v_cache, int64_t stride_b,
                                 int64_t stride_s, int64_t stride_h, void* o, float* lse, int dtype,
                                 const int32_t* seq_L, int B, int max_L, int Hq, int Hkv, int head_dim,
                                 int w_pretrained, int w0, float softmax_scale, const void* table,
                                 size_t table_bytes, int table_rows, void* workspace, size_t workspace_bytes,
                                 void* stream, unsigned flags) {
  jl::DecodeCall c;
  int st = decode_args(q, k_cache, v_cache, stride_b, stride_s, stride_h, o, lse, dtype, seq_L, B, max_L, Hq, Hkv,
                       head_dim, w_pretrained, w0, 1.0, softmax_scale, flags, &c);
  if (st != JL_OK || c.B == 0) return st;
  if (!table) return fail(JL_ERR_INVALID_ARG, "table must be non-null");
  if (table_rows < max_L) return fail(JL_ERR_INVALID_ARG, "table covers %d positions, max_L = %d", table_rows, max_L);
  if (table_bytes < jl::rope_table_bytes(table_rows, head_dim))
    return fail(JL_ERR_INVALID_ARG, "table has %zu bytes, %d rows need %zu", table_bytes, table_rows,
                jl::rope_table_bytes(table_rows, head_dim));
  if (reinterpret_cast<uintptr_t>(table) % 256) return fail(JL_ERR_INVALID_ARG, "table must be 256-byte aligned");
  st = check_workspace(workspace, workspace_bytes,
                       jl_bifocal_decode_with_table_workspace_size(dtype, B, max_L, Hq, Hkv, head_dim));
  if (st != JL_OK) return st;
  c.ws = workspace;
  c.table = table;
  c.table_rows = table_rows;
  return hip_status(jl::launch_decode(c, dtype == JL_BF16, static_cast<hipStream_t>(stream)),
                    "jl_bifocal_decode_with_table launch");
}

int jl_bifocal_decode_with_table_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                         int64_t stride_b, int64_t stride_s, int64_t stride_h, void* o, float* lse,
                                         int dtype, const int32_t* seq_L, int B, int max_L, int Hq, int Hkv,
                                         int head_dim, int w_pretrained, int w0, float softmax_scale,
                                         const void* table, size_t table_bytes, int table_rows, void* stream,
                                         unsigned flags) {
  jl::DecodeCall c;
  int st = decode_args(q, k_cache, v_cache, stride_b, stride_s, stride_h, o, lse, dtype, seq_L, B, max_L, Hq, Hkv,
                       head_dim, w_pretrained, w0, 1.0, softmax_scale, flags, &c);
  if (st != JL_OK || c.B == 0) return st;
  if (!table) return fail(JL_ERR_INVALID_ARG, "table must be non-null");
  if (table_rows < max_L) return fail(JL_ERR_INVALID_ARG, "table covers %d positions, max_L = %d", table_rows, max_L);
  if (table_bytes < jl::rope_table_bytes(table_rows, head_dim))
    return fail(JL_ERR_INVALID_ARG, "table has %zu bytes, %d rows need %zu", table_bytes, table_rows,
                jl::rope_table_bytes(table_rows, head_dim));
  if (reinterpret_cast<uintptr_t>(table) % 256) return fail(JL_ERR_INVALID_ARG, "table must be 256-byte aligned");
  const size_t need = jl::decode_part_bytes(dtype == JL_BF16, B, max_L, Hq, Hkv, head_dim);
  if (need > jl::decode_scratch_bytes())
    return fail(JL_ERR_UNSUPPORTED,
                "no-allocation decode: these sizes need %zu bytes of partial states, the device scratch holds %zu",
                need, jl::decode_scratch_bytes());
  void* scr = nullptr;
  const hipError_t e = jl::decode_scratch(&scr);
  if (e != hipSuccess) return hip_status(e, "jl_bifocal_decode_with_table_noalloc scratch lookup");
  c.table = table;
  c.table_rows = table_rows;
  c.part = static_cast<float*>(scr);
  return hip_status(jl::launch_decode(c, dtype == JL_BF16, static_cast<hipStream_t>(stream)),
                    "jl_bifocal_decode_with_table_noalloc launch");
}

int jl_bifocal_decode_key_rows(const int32_t* seq_L, int B, int max_L, int Hkv, int w_pretrained, int w0,
                               unsigned flags, int32_t* rows_out, void* stream) {
  if (flags & ~static_cast<unsigned>(JL_FLAG_PREROTATED)) return fail(JL_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  if (B < 0 || max_L < 0 || Hkv < 1) return fail(JL_ERR_INVALID_ARG, "need B >= 0, max_L >= 0, Hkv >= 1");
  if (w_pretrained < 1 || w0 < 0) return fail(JL_ERR_INVALID_ARG, "need w_pretrained >= 1 and w0 >= 0");
  if (B == 0 || max_L == 0) return JL_OK;
  if (!seq_L || !rows_out) return fail(JL_ERR_INVALID_ARG, "seq_L and rows_out must be non-null");
  return hip_status(jl::launch_decode_key_rows(seq_L, B, max_L, Hkv, w_pretrained, w0,
                                               (flags & JL_FLAG_PREROTATED) != 0, rows_out,
                                               static_cast<hipStream_t>(stream)),
                    "jl_bifocal_decode_key_rows launch");
}

int jl_bifocal_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int dtype,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                       int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int Hq,
                       int Hkv, int head_dim, int w_pretrained, int w0, double rope_theta,
                       float softmax_scale, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return jl_bifocal_prefill_ex(q, k, v, o, lse, dtype, cu_seqlens_q, cu_seqlens_k, B, total_q, total_k,
                               max_seqlen_q, max_seqlen_k, Hq, Hkv, head_dim, w_pretrained, w0, rope_theta,
                               softmax_scale, workspace, workspace_bytes, stream, 0u);
}

int jl_bifocal_prefill_prepare(const void* k, const void* v, int dtype, const int32_t* cu_seqlens_k,
                               int B, int total_k, int max_seqlen_k, int Hkv, int head_dim,
                               int w_pretrained, double rope_theta, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return jl_bifocal_prefill_prepare_ex(k, v, dtype, cu_seqlens_k, B, total_k, max_seqlen_k, Hkv, head_dim,
                                       w_pretrained, rope_theta, workspace, workspace_bytes, stream, 0u);
}

int jl_bifocal_prefill_attend(const void* q, const void* k, const void* v, void* o, float* lse,
                              int dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int B, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                              int Hq, int Hkv, int head_dim, int w_pretrained, int w0,
                              double rope_theta, float softmax_scale, const void* workspace,
                              size_t workspace_bytes, void* stream) {
  return jl_bifocal_prefill_attend_ex(q, k, v, o, lse, dtype, cu_seqlens_q, cu_seqlens_k, B, total_q, total_k,
                                      max_seqlen_q, max_seqlen_k, Hq, Hkv, head_dim, w_pretrained, w0,
                                      rope_theta, softmax_scale, workspace, workspace_bytes, stream, 0u);
}

int jl_bifocal_decode(const void* q, const void* k_cache, const void* v_cache, int64_t stride_b,
                      int64_t stride_s, int64_t stride_h, void* o, float* lse, int dtype,
                      const int32_t* seq_L, int B, int max_L, int Hq, int Hkv, int head_dim,
                      int w_pretrained, int w0, double rope_theta, float softmax_scale,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return jl_bifocal_decode_ex(q, k_cache, v_cache, stride_b, stride_s, stride_h, o, lse, dtype, seq_L, B, max_L,
                              Hq, Hkv, head_dim, w_pretrained, w0, rope_theta, softmax_scale, workspace,
                              workspace_bytes, stream, 0u);
}

int jl_bifocal_remote_positions(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                                int total_q, int w_pretrained, int32_t* pos_out, int32_t* f_out,
                                int32_t* G_out, void* stream) {
  if (B < 0 || total_q < 0) return fail(JL_ERR_INVALID_ARG, "sizes must be non-negative");
  if (w_pretrained < 1) return fail(JL_ERR_INVALID_ARG, "w_pretrained must be >= 1");
  if (B == 0) return JL_OK;
  if (!cu_seqlens_q) return fail(JL_ERR_INVALID_ARG, "cu_seqlens_q must be non-null");
  if (!pos_out && !f_out && !G_out) return fail(JL_ERR_INVALID_ARG, "no output given");
  return hip_status(jl::launch_remote_positions(cu_seqlens_q, cu_seqlens_k ? cu_seqlens_k : cu_seqlens_q,
                                                B, total_q, w_pretrained, pos_out, f_out, G_out,
                                                static_cast<hipStream_t>(stream)),
                    "jl_bifocal_remote_positions launch");
}

int jl_bifocal_tile_classes(int Lq, int L, int w0, int BM, int BN, uint8_t* cls_out, void* stream) {
  if (Lq < 0 || L < 0 || Lq > L) return fail(JL_ERR_INVALID_ARG, "need 0 <= Lq <= L");
  if (w0 < 0) return fail(JL_ERR_INVALID_ARG, "w0 must be >= 0");
  if (BM < 1 || BN < 1 || BM > 4096 || BN > 4096) return fail(JL_ERR_INVALID_ARG, "BM and BN must lie in [1, 4096]");
  if (Lq == 0) return JL_OK;
  if (!cls_out) return fail(JL_ERR_INVALID_ARG, "cls_out must be non-null");
  return hip_status(jl::launch_tile_classes(Lq, L, w0, BM, BN, cls_out, static_cast<hipStream_t>(stream)),
                    "jl_bifocal_tile_classes launch");
}

int jl_bifocal_prefill_tile_shape(int dtype, int Hq, int Hkv, int head_dim, int* BM, int* BN) {
  if (!BM || !BN) return fail(JL_ERR_INVALID_ARG, "BM and BN must be non-null");
  if (!supported_dtype(dtype)) return fail(JL_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
  if (!supported_dim(head_dim)) return fail(JL_ERR_UNSUPPORTED, "head_dim %d not supported", head_dim);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(JL_ERR_INVALID_ARG, "Hq must be a positive multiple of Hkv");
  if (dtype == JL_BF16) {
    jl::prefill_bf16_tile_shape(Hq / Hkv, BM, BN);
  } else {
    *BM = 64;
    *BN = 32;
  }
  return JL_OK;
}

const char* jl_status_string(int code) {
  switch (code) {
    case JL_OK: return "ok";
    case JL_ERR_INVALID_ARG: return "invalid argument";
    case JL_ERR_UNSUPPORTED: return "unsupported configuration";
    case JL_ERR_WORKSPACE: return "workspace missing or too small";
    case JL_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* jl_last_error(void) { return g_last_error; }

const char* jl_version(void) { return "0.1.0"; }

}  // extern "C"
