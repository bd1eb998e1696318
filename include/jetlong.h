/*
 * jetlong.h — C ABI of the MI355X (gfx950) dynamic bifocal RoPE attention
 * library (libjetlong.so).
 *
 * The method: "Jet-Long: Efficient Long-Context Extension with Dynamic
 * Bifocal RoPE" (gist.science technical summaries of arXiv 2607.07740).
 *   - Section "Dynamic Bifocal RoPE": a causal query/key pair whose distance
 *     is below the local window w0 is scored with classic RoPE at the true
 *     positions; every farther pair is scored with RoPE at the grouped
 *     positions f(x) = floor(x / G), G = max(1, ceil(L / w_pretrained)),
 *     recomputed from the current sequence length L (eq. G, eq. f).
 *   - Section "Inference Efficiency Mechanisms": the KV cache keeps the base
 *     keys at their exact absolute positions and is never rewritten; the
 *     rotation that the remote branch needs is applied on the fly.
 *
 * Readings taken where the pages are silent:
 *   RoPE: theta_k = theta^(-2k/d), rotate-half pairing (dims k and k + d/2);
 *   the remote branch rotates every token by f of its own absolute position
 *   (no extra offset); the local window holds distances 0 .. w0-1 (w0 = 0
 *   makes every pair remote); softmax scale 1/sqrt(d) unless given; GQA query
 *   head h reads KV head h / (Hq / Hkv); in decode L counts the new token.
 *
 * Conventions shared by every entry point
 *   Memory:   the caller allocates and frees every buffer (inputs, outputs,
 *             workspace).  Pointers marked "device" must be device memory of
 *             the current HIP device.  The library allocates nothing and
 *             keeps no device state between calls, with one exception:
 *             jl_bifocal_decode_with_table_noalloc works in a fixed static
 *             device array of its own (see there).
 *   Streams:  `stream` is a hipStream_t passed as void* (NULL = the default
 *             stream).  Work is only enqueued; nothing synchronises the host.
 *             The host never reads device arguments such as cu_seqlens.
 *   Errors:   every argument is checked before any HIP call; on failure the
 *             call returns a negative jl_status, enqueues nothing and records
 *             a message for jl_last_error().  A launch failure returns
 *             JL_ERR_HIP.  A device fault surfaces at the caller's next
 *             synchronisation.  No C++ exception crosses this interface.
 *   dtype:    JL_F32 (float) or JL_BF16 (bfloat16, round-to-nearest-even on
 *             output).  The RoPE angles and their cos/sin are formed in fp64
 *             and rounded once to fp32.
 *             JL_F32: rotation, products, softmax and accumulation in fp32.
 *             JL_BF16: the matrix-core operands are IEEE half (f16), every
 *             product is accumulated in fp32:
 *               prefill - each key is rotated once in fp32 and stored as
 *                 half; values are converted to half (exact for bf16 in
 *                 range); queries are rotated in fp32, scaled by
 *                 softmax_scale * log2(e) and rounded to half; the
 *                 probabilities are rounded to half, and each row's sum of
 *                 them is formed per 64-key tile by a tree of packed-half
 *                 adds (relative error below 2^-11 per level) before it is
 *                 added to the fp32 running sum; maxima, exponentials and
 *                 rescaling run in fp32.
 *               decode - each key is converted to half and rotated in
 *                 packed-half arithmetic from a half copy of its cos/sin row;
 *                 the query as in prefill; P V runs on the bf16 matrix cores
 *                 with P split into a bf16 high and low part (about 16
 *                 significant bits) against the exact bf16 values; softmax
 *                 and accumulation in fp32.  With JL_FLAG_PREROTATED and
 *                 w0 >= max_L (every key inside the window: plain RoPE
 *                 attention over a RoPE cache) Q K^T runs on the bf16 matrix
 *                 cores straight from the stored keys, the scaled query
 *                 rounded to bf16.
 *   Range (JL_BF16): half holds magnitudes below 65520.  Supported inputs:
 *             |k_e| < 46300 for every key element (each rotated component
 *             then stays below its pair's norm, < 65504), |v_e| < 65504 for
 *             prefill values, |q_e| * softmax_scale * log2(e) < 46300 for
 *             queries; decode values are not limited.  A rotated key, value
 *             or scaled query outside half range is replaced by NaN (decode:
 *             its scores become infinite or NaN and the head's result is set
 *             to NaN), so the outputs that attend it come out NaN, never as
 *             a wrong finite value; other rows of the same sequence and KV
 *             head may be NaN too.
 *   head_dim: 64 or 128.  Hq must be a multiple of Hkv.
 *   Limits:   sequence lengths < 2^31; positions are int32.  bf16 prefill
 *             (prepare and attend): (roundup64(total_k) + 64 B) * head_dim
 *             * 2 must not exceed 2^31 - 1 (about 8.4M keys per call at
 *             head_dim 128), else JL_ERR_UNSUPPORTED.
 */
#ifndef JETLONG_H
#define JETLONG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  JL_OK = 0,
  JL_ERR_INVALID_ARG = -1, /* null pointer, negative size, Hq % Hkv != 0 ... */
  JL_ERR_UNSUPPORTED = -2, /* head_dim, dtype or size outside what is built */
  JL_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required    */
  JL_ERR_HIP = -4          /* a HIP call failed (launch, device query)      */
} jl_status;

typedef enum { JL_F32 = 0, JL_BF16 = 1 } jl_dtype;

/* Tile class codes of jl_bifocal_tile_classes (low two bits) and the flag
 * bit for a tile that also holds pairs with the key after the query. */
enum { JL_TILE_SKIP = 0, JL_TILE_LOCAL = 1, JL_TILE_REMOTE = 2, JL_TILE_STRADDLE = 3,
       JL_TILE_DIAG = 4 };

/* Group size G = max(1, ceil(L / w_pretrained)) in exact integer arithmetic
 * ("Dynamic Bifocal RoPE", eq. G).  Host only.  Returns G >= 1, or
 * JL_ERR_INVALID_ARG when L < 0 or w_pretrained < 1. */
int64_t jl_bifocal_group_size(int64_t L, int64_t w_pretrained);

/* Bytes of device workspace jl_bifocal_prefill needs for these sizes, or 0 on
 * invalid sizes.  total_k = number of packed key rows (cu_seqlens_k[B]). */
size_t jl_bifocal_prefill_workspace_size(int dtype, int B, int total_k, int max_seqlen_k,
                                         int Hq, int Hkv, int head_dim);

/* Packed variable-length causal prefill ("Dynamic Bifocal RoPE"; the
 * "Inclusion-Exclusion Attention Merge" of the pages reaches the same result
 * by three merged passes; this library routes each key tile instead).
 *
 *   q   device [total_q, Hq, head_dim]   dtype   raw (un-rotated) queries
 *   k,v device [total_k, Hkv, head_dim]  dtype   raw keys / values, read only
 *   o   device [total_q, Hq, head_dim]   dtype   output
 *   lse device [Hq, total_q] float or NULL: natural-log log-sum-exp per row
 *   cu_seqlens_q device int32 [B+1]: sequence b owns query rows
 *       cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1.
 *   cu_seqlens_k device int32 [B+1] or NULL (= cu_seqlens_q).  Sequence b
 *       has L_b = cu_seqlens_k[b+1]-cu_seqlens_k[b] keys at positions
 *       0 .. L_b-1 and its Lq_b queries sit at the last Lq_b positions
 *       (L_b - Lq_b .. L_b - 1; a chunk of a longer prefill); Lq_b <= L_b is
 *       required.  G_b is computed from L_b on the device.
 *   max_seqlen_q / max_seqlen_k: upper bounds of Lq_b / L_b.  A sequence
 *       that breaks Lq_b <= L_b, Lq_b <= max_seqlen_q or L_b <= max_seqlen_k
 *       (lengths live on the device and are not checked on the host) is left
 *       unwritten in o and lse; the inclusion-exclusion route leaves its rows
 *       unspecified.
 *   w_pretrained >= 1, w0 >= 0, rope_theta > 0.
 *   softmax_scale: 0 selects 1/sqrt(head_dim).
 *   workspace: device, >= jl_bifocal_prefill_workspace_size(...) bytes,
 *       256-byte aligned; contents need not be initialised.
 */
int jl_bifocal_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                       int dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       int B, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                       int Hq, int Hkv, int head_dim, int w_pretrained, int w0,
                       double rope_theta, float softmax_scale,
                       void* workspace, size_t workspace_bytes, void* stream);

/* The two stages jl_bifocal_prefill runs, for callers that attend several
 * query batches (or several w0 values) to one prepared key set, or that time
 * the stages apart.
 *
 * jl_bifocal_prefill_prepare reads k, v and cu_seqlens_k (meanings as above)
 * and fills `workspace` with the cos/sin table of positions 0 ..
 * max_seqlen_k-1 and, for JL_BF16, every key rotated once at its position p
 * and once at f(p) plus the values in the transposed layout the MFMA kernel
 * reads (the "Dynamic Bifocal RoPE" rotations, eq. G / eq. f; inputs stay
 * untouched).  The workspace size is
 * jl_bifocal_prefill_workspace_size(dtype, B, total_k, max_seqlen_k, Hq, Hkv,
 * head_dim) for the Hq later used.
 *
 * jl_bifocal_prefill_attend runs the attention over a workspace prepared by
 * a call with the same k, v, dtype, cu_seqlens_k, B, total_k, max_seqlen_k,
 * Hkv, head_dim, w_pretrained and rope_theta (not checked: a mismatch gives
 * wrong results, not a fault), with the other arguments as in
 * jl_bifocal_prefill. */
int jl_bifocal_prefill_prepare(const void* k, const void* v, int dtype, const int32_t* cu_seqlens_k,
                               int B, int total_k, int max_seqlen_k, int Hkv, int head_dim,
                               int w_pretrained, double rope_theta, void* workspace,
                               size_t workspace_bytes, void* stream);
int jl_bifocal_prefill_attend(const void* q, const void* k, const void* v, void* o, float* lse,
                              int dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int B, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                              int Hq, int Hkv, int head_dim, int w_pretrained, int w0,
                              double rope_theta, float softmax_scale, const void* workspace,
                              size_t workspace_bytes, void* stream);

/* Flag bits of the *_ex entry points. */
enum { JL_FLAG_PREROTATED = 1 };

/* The same prefill calls with flags.  JL_FLAG_PREROTATED: q and k arrive
 * already rotated at their true positions (R(p) q, R(p) k: the usual RoPE
 * cache layout), everything else as above.  Local pairs are then scored on
 * the stored vectors as they are; remote pairs apply the correction rotation
 * R(f(p) - p) to both sides on the fly ("Inference Efficiency Mechanisms",
 * correction rotation; "Dynamic Bifocal RoPE", eq. f), and the inputs stay
 * untouched.  A workspace prepared with the flag must be attended with it.
 * Unknown flag bits: JL_ERR_INVALID_ARG.  flags = 0 is exactly the call
 * without _ex. */
int jl_bifocal_prefill_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                          int dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          int B, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                          int Hq, int Hkv, int head_dim, int w_pretrained, int w0,
                          double rope_theta, float softmax_scale,
                          void* workspace, size_t workspace_bytes, void* stream, unsigned flags);
int jl_bifocal_prefill_prepare_ex(const void* k, const void* v, int dtype, const int32_t* cu_seqlens_k,
                                  int B, int total_k, int max_seqlen_k, int Hkv, int head_dim,
                                  int w_pretrained, double rope_theta, void* workspace,
                                  size_t workspace_bytes, void* stream, unsigned flags);
int jl_bifocal_prefill_attend_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                 int B, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                                 int Hq, int Hkv, int head_dim, int w_pretrained, int w0,
                                 double rope_theta, float softmax_scale, const void* workspace,
                                 size_t workspace_bytes, void* stream, unsigned flags);

/* The same prefill result by the pages' own route, the inclusion-exclusion
 * attention merge ("Inference Efficiency Mechanisms"): three attention passes
 * with fp32 output and LSE, (1) the pairs closer than w0 rotated at their
 * true positions, (2) every causal pair rotated at the grouped positions
 * f(p), (3) the pairs closer than w0 at f(p), then per row
 *   O = (w1 O1 + w2 O2 - w3 O3) / (w1 + w2 - w3), w_i = exp(LSE_i - M),
 *   M = max(LSE_1, LSE_2), LSE = M + log(w1 + w2 - w3).
 * Arguments, flags and error behaviour as jl_bifocal_prefill_ex; the
 * workspace (256-byte aligned, caller-owned, scratch between calls) must
 * hold jl_bifocal_prefill_ie_workspace_size(...) bytes: the prefill
 * workspace plus three fp32 [total_q, Hq, head_dim] rows and three fp32
 * [Hq, total_q] LSE buffers.  It exists to compare against the tile-routed
 * jl_bifocal_prefill: it does about the work of a full causal pass plus two
 * window passes, and the difference w2 - w3 cancels when a row's grouped-
 * position mass sits inside the window. */
size_t jl_bifocal_prefill_ie_workspace_size(int dtype, int B, int total_q, int total_k,
                                            int max_seqlen_k, int Hq, int Hkv, int head_dim);
int jl_bifocal_prefill_ie(const void* q, const void* k, const void* v, void* o, float* lse,
                          int dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          int B, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                          int Hq, int Hkv, int head_dim, int w_pretrained, int w0,
                          double rope_theta, float softmax_scale,
                          void* workspace, size_t workspace_bytes, void* stream, unsigned flags);

/* Bytes of device workspace jl_bifocal_decode needs, or 0 on invalid sizes. */
size_t jl_bifocal_decode_workspace_size(int dtype, int B, int max_L, int Hq, int Hkv,
                                        int head_dim);

/* One new query per sequence against an untouched KV cache ("Inference
 * Efficiency Mechanisms": base keys stay at their absolute positions; the
 * rotation each key needs is applied in registers, the cache is never
 * written).
 *
 *   q   device [B, Hq, head_dim] dtype, raw query of the newest token
 *   k_cache, v_cache device, dtype, raw keys/values; element (b, s, h, e) at
 *       offset b*stride_b + s*stride_s + h*stride_h + e (strides in elements,
 *       head_dim contiguous, same strides for both caches).  Read only.
 *   o   device [B, Hq, head_dim] dtype output; lse device [B, Hq] float or NULL
 *   seq_L device int32 [B]: keys valid in sequence b, the new token included
 *       (1 <= seq_L[b] <= max_L); the query sits at position seq_L[b]-1.
 *       A sequence outside that range (the lengths live on the device and
 *       are not checked on the host) is left unwritten in o and lse.
 *   workspace: device, >= jl_bifocal_decode_workspace_size(...) bytes.
 */
int jl_bifocal_decode(const void* q, const void* k_cache, const void* v_cache,
                      int64_t stride_b, int64_t stride_s, int64_t stride_h,
                      void* o, float* lse, int dtype, const int32_t* seq_L, int B, int max_L,
                      int Hq, int Hkv, int head_dim, int w_pretrained, int w0,
                      double rope_theta, float softmax_scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/* jl_bifocal_decode with flags.  JL_FLAG_PREROTATED: q holds R(L-1) q and the
 * key cache holds R(j) k_j (keys rotated at their absolute positions, the
 * cache layout the pages keep); local keys are used as stored and remote keys
 * get the correction rotation R(f(j) - j) in registers as they stream by, so
 * the cache is never rewritten ("Inference Efficiency Mechanisms").  flags =
 * 0 is exactly jl_bifocal_decode. */
int jl_bifocal_decode_ex(const void* q, const void* k_cache, const void* v_cache,
                         int64_t stride_b, int64_t stride_s, int64_t stride_h,
                         void* o, float* lse, int dtype, const int32_t* seq_L, int B, int max_L,
                         int Hq, int Hkv, int head_dim, int w_pretrained, int w0,
                         double rope_theta, float softmax_scale,
                         void* workspace, size_t workspace_bytes, void* stream, unsigned flags);

/* Prepared cos/sin table for jl_bifocal_decode_with_table: the angles p *
 * theta_k of positions p = 0 .. max_pos-1 (theta_k = theta^(-2k/d)), formed
 * in fp64; fp32 (cos, sin) rows [max_pos][head_dim/2], then, 256-byte
 * aligned, half rows [max_pos][head_dim] holding (cos, cos, sin, sin) of
 * each frequency pair.  It depends only on max_pos, head_dim and theta, so a
 * caller builds it once (as a RoPE cos/sin cache) and reuses it for every
 * decode step.  jl_bifocal_rope_table_size returns its bytes (0 on invalid
 * sizes); jl_bifocal_rope_table fills caller-owned device memory (256-byte
 * aligned, >= that size) on `stream`. */
size_t jl_bifocal_rope_table_size(int max_pos, int head_dim);
int jl_bifocal_rope_table(int max_pos, int head_dim, double rope_theta, void* table, size_t table_bytes,
                          void* stream);

/* jl_bifocal_decode_ex over a prepared table instead of building the cos/sin
 * rows it reads on every call ("Inference Efficiency Mechanisms": the
 * rotations are applied on the fly; the cos/sin values themselves do not
 * depend on the call).  table: device, from jl_bifocal_rope_table with the
 * same head_dim and the rope_theta wanted (not checked: a different theta
 * gives a different, valid-looking result), covering table_rows >= max_L
 * positions; table_bytes its size.  It is read only (and not read at all by a
 * bf16 pre-rotated call with w0 >= max_L).  workspace: device, 256-byte
 * aligned, >= jl_bifocal_decode_with_table_workspace_size(...) bytes (the
 * partial states of the key-range splits).  Everything else, including
 * flags, as jl_bifocal_decode_ex. */
size_t jl_bifocal_decode_with_table_workspace_size(int dtype, int B, int max_L, int Hq, int Hkv,
                                                   int head_dim);
int jl_bifocal_decode_with_table(const void* q, const void* k_cache, const void* v_cache,
                                 int64_t stride_b, int64_t stride_s, int64_t stride_h,
                                 void* o, float* lse, int dtype, const int32_t* seq_L, int B,
                                 int max_L, int Hq, int Hkv, int head_dim, int w_pretrained, int w0,
                                 float softmax_scale, const void* table, size_t table_bytes,
                                 int table_rows, void* workspace, size_t workspace_bytes,
                                 void* stream, unsigned flags);

/* jl_bifocal_decode_with_table for callers that cannot allocate memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument, and the call allocates nothing.  The
 * partial states live in a device array inside the library, one per GPU,
 * held until the process ends: at most 64 MiB, i.e. B * Hq * splits *
 * slots * (head_dim + 2) * 4 bytes, the size
 * jl_bifocal_decode_with_table_workspace_size reports; larger sizes return
 * JL_ERR_UNSUPPORTED before anything is enqueued.  Every call on one GPU
 * shares that array, so calls that overlap on one GPU (different streams,
 * or host threads) race and give wrong results; calls in order on one
 * stream are safe.  The first call on a device looks up the array's device
 * address (no allocation); a failure there returns JL_ERR_HIP.  Arguments,
 * results and flags otherwise as jl_bifocal_decode_with_table. */
int jl_bifocal_decode_with_table_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                         int64_t stride_b, int64_t stride_s, int64_t stride_h,
                                         void* o, float* lse, int dtype, const int32_t* seq_L, int B,
                                         int max_L, int Hq, int Hkv, int head_dim, int w_pretrained,
                                         int w0, float softmax_scale, const void* table,
                                         size_t table_bytes, int table_rows, void* stream,
                                         unsigned flags);

/* Debug export of the bf16 decode's integer map ("Dynamic Bifocal RoPE",
 * eq. G / eq. f): for sequence b (seq_L device int32 [B]) and key j <
 * seq_L[b], rows_out[b * max_L + j] (device int32 [B, max_L]) receives the
 * cos/sin row the bf16 split kernel rotates key j with, computed by the same
 * device code and key walk as that kernel for these B, max_L and Hkv: j if
 * the key is within w0 of the query at seq_L[b]-1, else f(j) = floor(j / G);
 * with JL_FLAG_PREROTATED 0 for a local key and ~(j - f(j)) (the correction
 * R(f(j) - j): row j - f(j) with sin negated, stored bit-inverted) for a
 * remote one.  Entries j >= seq_L[b], and sequences outside 1 .. max_L, are
 * not written. */
int jl_bifocal_decode_key_rows(const int32_t* seq_L, int B, int max_L, int Hkv, int w_pretrained,
                               int w0, unsigned flags, int32_t* rows_out, void* stream);

/* Integer position map of a packed batch, exactly as the prefill kernels use
 * it (eq. G, eq. f).  Device outputs: pos_out/f_out int32 [total_q] (query
 * position and its remote position), G_out int32 [B].  cu_seqlens_k may be
 * NULL (= cu_seqlens_q). */
int jl_bifocal_remote_positions(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                                int total_q, int w_pretrained, int32_t* pos_out, int32_t* f_out,
                                int32_t* G_out, void* stream);

/* Tile classes the prefill kernels use, for one sequence of Lq queries at
 * positions L-Lq .. L-1 against L keys, in BM x BN blocks (1 <= BM, BN <=
 * 4096).  cls_out: device uint8 [ceil(Lq/BM), ceil(L/BN)], row-major. */
int jl_bifocal_tile_classes(int Lq, int L, int w0, int BM, int BN, uint8_t* cls_out,
                            void* stream);

/* Query-block height and key-tile width the bf16 prefill kernel routes on,
 * for a given GQA ratio Hq/Hkv (so tests can compare its tile map). */
int jl_bifocal_prefill_tile_shape(int dtype, int Hq, int Hkv, int head_dim, int* BM, int* BN);

/* Static description of a status code. */
const char* jl_status_string(int code);

/* Detail of the last failing call on this host thread ("" if none). */
const char* jl_last_error(void);

/* Library version, e.g. "0.1.0". */
const char* jl_version(void);

#ifdef __cplusplus
}
#endif
#endif /* JETLONG_H */
