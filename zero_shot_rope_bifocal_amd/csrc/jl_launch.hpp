// Host-side launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace jl {

// Arguments of one prefill call after validation (device pointers).
struct PrefillCall {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int B, total_q, total_k, max_q, max_k;
  int Hq, Hkv, D;
  int w_pretrained, w0;
  double theta;
  float scale;
  void* ws;
  bool prerot;  // q and k arrive rotated at their true positions
};

struct DecodeCall {
  const void* q;
  const void* kc;
  const void* vc;
  int64_t sb, ss, sh;
  void* o;
  float* lse;
  const int32_t* seq_L;
  int B, max_L, Hq, Hkv, D;
  int w_pretrained, w0;
  double theta;
  float scale;
  void* ws;
  bool prerot;  // q and the key cache arrive rotated at their true positions
  const void* table;  // prepared cos/sin table (rope_table_bytes layout) or null: built in ws
  int table_rows;     // positions the prepared table covers
  float* part;        // partial states, or null: in ws after the table
};

// Workspace layouts (bytes).
size_t prefill_ws_bytes_bf16(int B, int total_k, int max_k, int Hkv, int D);
size_t prefill_ws_bytes_f32(int max_k, int D);
size_t decode_ws_bytes(int B, int max_L, int Hq, int Hkv, int D);
// Partial states of one decode call (what a prepared-table decode needs).
size_t decode_part_bytes(bool bf16, int B, int max_L, int Hq, int Hkv, int D);
// A full cos/sin table of positions [0, npos): fp32 rows [npos][D/2] float2,
// then (256-byte aligned) the half rows [npos][D] of the decode key rotation.
size_t rope_table_bytes(int npos, int D);
hipError_t launch_rope_table_full(void* table, int npos, int D, double theta, hipStream_t s);
// Device scratch of the no-allocation decode: its size, and this device's
// address of it (looked up once per device, then cached).
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** out);
// The signed table rows the bf16 split kernel rotates keys with, [B][max_L].
hipError_t launch_decode_key_rows(const int32_t* seq_L, int B, int max_L, int Hkv, int w_pretrained, int w0,
                                  bool prerot, int32_t* out, hipStream_t s);
int decode_num_splits(int B, int max_L, int Hkv);

// Query-block height / key-tile width of the bf16 prefill kernel.
void prefill_bf16_tile_shape(int ratio, int* BM, int* BN);

// tab16 (optional): the same rows in half, entry kp of a row = (cos, cos,
// sin, sin) of frequencies 2kp and 2kp + 1.
hipError_t launch_rope_table(float2* tab, int npos, int D, double theta, hipStream_t s, uint16_t* tab16 = nullptr);
// Same table, writing only the rows a decode reads: those below
// min(w_pretrained, npos) (every remote position), each sequence's window
// [seq_L[b] - w0, seq_L[b]) and its query rows.  With tab16 given the fp32
// rows are written for the query rows alone (the bf16 split kernel rotates
// keys from the half rows).
hipError_t launch_rope_table_rows(float2* tab, int npos, int D, double theta, const int32_t* seq_L, int B,
                                  int w0, int w_pretrained, hipStream_t s, uint16_t* tab16 = nullptr);
// Prefill in two stages on one workspace: prepare (cos/sin table; for bf16
// also the rotated key copies and transposed values) and attend.
hipError_t launch_prefill_bf16_prepare(const PrefillCall& c, hipStream_t s);
hipError_t launch_prefill_bf16_attend(const PrefillCall& c, hipStream_t s);
hipError_t launch_prefill_f32_prepare(const PrefillCall& c, hipStream_t s);
hipError_t launch_prefill_f32_attend(const PrefillCall& c, hipStream_t s);
hipError_t launch_decode(const DecodeCall& c, bool bf16, hipStream_t s);

// Inclusion-exclusion route to the same prefill result: three attention
// passes with fp32 output rows [total_q][Hq][D] and LSE [Hq][total_q], then a
// merge.  The passes read the workspace of a finished prepare.
enum IePass : int { kIeWindowLocal = 1, kIeFullRemote = 2, kIeWindowRemote = 3 };
hipError_t launch_prefill_bf16_ie_pass(const PrefillCall& c, int pass, float* o, float* lse, hipStream_t s);
hipError_t launch_prefill_f32_ie_pass(const PrefillCall& c, int pass, float* o, float* lse, hipStream_t s);
// Workspace of the merged route: the prefill workspace, then three fp32 O
// and three LSE buffers.
size_t prefill_ie_ws_bytes(bool bf16, int B, int total_q, int total_k, int max_k, int Hq, int Hkv, int D);
hipError_t launch_prefill_ie(const PrefillCall& c, bool bf16, hipStream_t s);
hipError_t launch_remote_positions(const int32_t* cu_q, const int32_t* cu_k, int B, int total_q,
                                   int w_pretrained, int32_t* pos, int32_t* f, int32_t* G,
                                   hipStream_t s);
hipError_t launch_tile_classes(int Lq, int L, int w0, int BM, int BN, uint8_t* out, hipStream_t s);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace jl
