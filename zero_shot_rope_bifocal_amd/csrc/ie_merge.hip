// The pages' own route to the bifocal prefill result: three plain attention
// passes merged by their log-sum-exp statistics.
//
// "Jet-Long: Efficient Long-Context Extension with Dynamic Bifocal RoPE",
// section "Inference Efficiency Mechanisms" (inclusion-exclusion attention
// merge).  With s1 the LSE of the window pass at the true positions, s2 that
// of the full causal pass at the grouped positions and s3 that of the window
// pass at the grouped positions, M = max(s1, s2) and w_i = exp(s_i - M):
//   O = (w1 O1 + w2 O2 - w3 O3) / (w1 + w2 - w3),  LSE = M + log(w1 + w2 - w3).
// The window pairs enter through pass 1 and leave pass 2 through pass 3; the
// difference w2 - w3 cancels when most of a row's grouped-position mass lies
// inside the window.  The tile-routed kernels never form that difference.
#include "jl_device.hpp"
#include "jl_launch.hpp"

namespace jl {

namespace {

// One thread = 4 features of one (token, head) row.
template <typename OutT, int D>
__global__ __launch_bounds__(256) void ie_merge_kernel(const float* __restrict__ o1, const float* __restrict__ o2,
                                                       const float* __restrict__ o3, const float* __restrict__ s1,
                                                       const float* __restrict__ s2, const float* __restrict__ s3,
                                                       OutT* __restrict__ o, float* __restrict__ lse, int total_q,
                                                       int Hq) {
  constexpr int TPR = D / 4;  // threads per row
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = t / TPR;  // tok * Hq + h
  if (row >= static_cast<int64_t>(total_q) * Hq) return;
  const int c = static_cast<int>(t % TPR) * 4;
  const int64_t tok = row / Hq;
  const int h = static_cast<int>(row % Hq);
  const int64_t li = static_cast<int64_t>(h) * total_q + tok;
  const float a = s1[li], b = s2[li], e = s3[li];
  const float M = fmaxf(a, b);
  const float w1 = expf(a - M), w2 = expf(b - M), w3 = expf(e - M);
  const float den = w1 + w2 - w3;
  const float inv = 1.f / den;
  const float4 x1 = *reinterpret_cast<const float4*>(o1 + row * D + c);
  const float4 x2 = *reinterpret_cast<const float4*>(o2 + row * D + c);
  const float4 x3 = *reinterpret_cast<const float4*>(o3 + row * D + c);
  const float r0 = (w1 * x1.x + w2 * x2.x - w3 * x3.x) * inv;
  const float r1 = (w1 * x1.y + w2 * x2.y - w3 * x3.y) * inv;
  const float r2 = (w1 * x1.z + w2 * x2.z - w3 * x3.z) * inv;
  const float r3 = (w1 * x1.w + w2 * x2.w - w3 * x3.w) * inv;
  if constexpr (sizeof(OutT) == 4) {
    *reinterpret_cast<float4*>(o + row * D + c) = make_float4(r0, r1, r2, r3);
  } else {
    *reinterpret_cast<uint2*>(o + row * D + c) = make_uint2(pack_bf16x2(r0, r1), pack_bf16x2(r2, r3));
  }
  if (lse && c == 0) lse[li] = M + logf(den);
}

template <typename OutT>
hipError_t launch_merge(const PrefillCall& c, const float* o1, const float* o2, const float* o3, const float* s1,
                        const float* s2, const float* s3, hipStream_t s) {
  const int64_t threads = static_cast<int64_t>(c.total_q) * c.Hq * (c.D / 4);
  const unsigned blocks = static_cast<unsigned>((threads + 255) / 256);
  OutT* o = static_cast<OutT*>(c.o);
  if (c.D == 128)
    hipLaunchKernelGGL((ie_merge_kernel<OutT, 128>), dim3(blocks), dim3(256), 0, s, o1, o2, o3, s1, s2, s3, o, c.lse,
                       c.total_q, c.Hq);
  else
    hipLaunchKernelGGL((ie_merge_kernel<OutT, 64>), dim3(blocks), dim3(256), 0, s, o1, o2, o3, s1, s2, s3, o, c.lse,
                       c.total_q, c.Hq);
  return hipGetLastError();
}

size_t base_ws_bytes(bool bf16, int B, int total_k, int max_k, int Hkv, int D) {
  return align_up(bf16 ? prefill_ws_bytes_bf16(B, total_k, max_k, Hkv, D) : prefill_ws_bytes_f32(max_k, D), 256);
}

}  // namespace

size_t prefill_ie_ws_bytes(bool bf16, int B, int total_q, int total_k, int max_k, int Hq, int Hkv, int D) {
  const size_t orow = align_up(static_cast<size_t>(total_q) * Hq * D * sizeof(float), 256);
  const size_t lrow = align_up(static_cast<size_t>(total_q) * Hq * sizeof(float), 256);
  return base_ws_bytes(bf16, B, total_k, max_k, Hkv, D) + 3 * orow + 3 * lrow;
}

hipError_t launch_prefill_ie(const PrefillCall& c, bool bf16, hipStream_t s) {
  if (c.B == 0 || c.total_q == 0) return hipSuccess;
  const size_t orow = align_up(static_cast<size_t>(c.total_q) * c.Hq * c.D * sizeof(float), 256);
  const size_t lrow = align_up(static_cast<size_t>(c.total_q) * c.Hq * sizeof(float), 256);
  char* w = static_cast<char*>(c.ws) + base_ws_bytes(bf16, c.B, c.total_k, c.max_k, c.Hkv, c.D);
  float* o[3];
  float* l[3];
  for (int i = 0; i < 3; ++i) {
    o[i] = reinterpret_cast<float*>(w + i * orow);
    l[i] = reinterpret_cast<float*>(w + 3 * orow + i * lrow);
  }
  hipError_t e = bf16 ? launch_prefill_bf16_prepare(c, s) : launch_prefill_f32_prepare(c, s);
  const int passes[3] = {kIeWindowLocal, kIeFullRemote, kIeWindowRemote};
  for (int i = 0; i < 3 && e == hipSuccess; ++i)
    e = bf16 ? launch_prefill_bf16_ie_pass(c, passes[i], o[i], l[i], s)
             : launch_prefill_f32_ie_pass(c, passes[i], o[i], l[i], s);
  if (e != hipSuccess) return e;
  return bf16 ? launch_merge<uint16_t>(c, o[0], o[1], o[2], l[0], l[1], l[2], s)
              : launch_merge<float>(c, o[0], o[1], o[2], l[0], l[1], l[2], s);
}

}  // namespace jl
