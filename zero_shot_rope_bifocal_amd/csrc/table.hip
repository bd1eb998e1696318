// cos/sin table and integer debug exports.
//
// "Jet-Long: Efficient Long-Context Extension with Dynamic Bifocal RoPE",
// section "Dynamic Bifocal RoPE": eq. G (group size from the current length)
// and eq. f (remote position = floor(x / G)).
#include "jl_device.hpp"
#include "jl_launch.hpp"

namespace jl {

// (cos, sin)(p * theta_k) for p in [0, npos), k in [0, D/2), theta_k =
// theta^(-2k/D), rounded once to fp32.  Layout: float2 tab[p * (D/2) + k].
// A thread owns one frequency and a run of kRun consecutive positions: the
// first angle and the one-step rotation come from fp64 sincos, the rest of
// the run from the fp64 rotation recurrence (cos, sin)(a + t) =
// (cos a cos t - sin a sin t, sin a cos t + cos a sin t), whose error after
// kRun steps stays near 1e-14, far below the fp32 rounding of the table.  The
// table thus keeps full fp32 accuracy at positions near 2^17, where an fp32
// angle would be off by ~1e-2 rad.
//
// With seq_L given (decode), only rows a decode can read are written: rows
// below `remote_rows` (every remote position f(j) < w_pretrained) and each
// sequence's local window [L_b - w0, L_b).  With tab16 given, the same rows
// are also written as half: entry kp of row p holds (cos, cos, sin, sin) of
// frequencies 2kp and 2kp + 1, the operand order of a packed-half rotation.
constexpr int kRun = 32;

__global__ void rope_table_kernel(float2* __restrict__ tab, uint16_t* __restrict__ tab16, int npos, int half,
                                  double theta, double neg2_over_d, const int32_t* __restrict__ seq_L, int B,
                                  int w0, int remote_rows) {
  const int k = threadIdx.x % half;
  const int run = blockIdx.x * (blockDim.x / half) + threadIdx.x / half;
  const int p0 = run * kRun;
  if (p0 >= npos) return;
  const int pend = min(npos, p0 + kRun);
  bool all = seq_L == nullptr || pend <= remote_rows;
  if (!all) {
    bool any = p0 < remote_rows;
    for (int b = 0; b < B && !any; ++b) {
      const int Lb = seq_L[b];
      any = Lb - w0 < pend && Lb > p0;
    }
    if (!any) return;
  }
  const double inv = pow(theta, neg2_over_d * k);
  double s, c, s1, c1;
  sincos(static_cast<double>(p0) * inv, &s, &c);
  sincos(inv, &s1, &c1);
  for (int p = p0; p < pend; ++p) {
    bool need = all || p < remote_rows;
    for (int b = 0; b < B && !need; ++b) need = p >= seq_L[b] - w0 && p < seq_L[b];
    if (need) tab[static_cast<int64_t>(p) * half + k] = make_float2(static_cast<float>(c), static_cast<float>(s));
    if (tab16) {
      // frequencies k and k + 1 sit in neighbouring lanes; the even lane
      // writes the pair's 8-byte entry (every lane of the wave takes part in
      // the exchange, so it stays outside the `need` branch)
      const uint32_t cs = pack_f16x2(static_cast<float>(c), static_cast<float>(s));
      const uint32_t odd = __shfl_down(cs, 1);
      if (need && !(k & 1))
        *reinterpret_cast<uint2*>(tab16 + (static_cast<int64_t>(p) * (half / 2) + k / 2) * 4) =
            make_uint2((cs & 0xffffu) | (odd << 16), (cs >> 16) | (odd & 0xffff0000u));
    }
    const double cn = c * c1 - s * s1;
    s = s * c1 + c * s1;
    c = cn;
  }
}

hipError_t launch_rope_table(float2* tab, int npos, int D, double theta, hipStream_t s, uint16_t* tab16) {
  return launch_rope_table_rows(tab, npos, D, theta, nullptr, 0, 0, npos, s, tab16);
}

hipError_t launch_rope_table_rows(float2* tab, int npos, int D, double theta, const int32_t* seq_L, int B,
                                  int w0, int remote_rows, hipStream_t s, uint16_t* tab16) {
  const int half = D / 2;
  if (npos <= 0) return hipSuccess;
  const int runs = (npos + kRun - 1) / kRun;
  const int per_block = 256 / half;
  hipLaunchKernelGGL(rope_table_kernel, dim3((runs + per_block - 1) / per_block), dim3(per_block * half), 0, s,
                     tab, tab16, npos, half, theta, -2.0 / static_cast<double>(D), seq_L, B, w0, remote_rows);
  return hipGetLastError();
}

// Query positions, remote positions and per-sequence G of a packed batch:
// sequence b has L_b keys and its Lq_b queries at the last Lq_b positions.
__global__ void remote_positions_kernel(const int32_t* __restrict__ cu_q,
                                        const int32_t* __restrict__ cu_k, int B, int total_q,
                                        int w_pretrained, int32_t* __restrict__ pos,
                                        int32_t* __restrict__ f, int32_t* __restrict__ Gout) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < B && Gout) Gout[t] = group_size(cu_k[t + 1] - cu_k[t], w_pretrained);
  if (t >= total_q) return;
  int lo = 0, hi = B - 1;  // last b with cu_q[b] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int L = cu_k[b + 1] - cu_k[b];
  const int Lq = cu_q[b + 1] - cu_q[b];
  const int p = (L - Lq) + (t - cu_q[b]);
  const int G = group_size(L, w_pretrained);
  if (pos) pos[t] = p;
  if (f) f[t] = p / G;
}

hipError_t launch_remote_positions(const int32_t* cu_q, const int32_t* cu_k, int B, int total_q,
                                   int w_pretrained, int32_t* pos, int32_t* f, int32_t* G,
                                   hipStream_t s) {
  const int n = total_q > B ? total_q : B;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(remote_positions_kernel, dim3((n + 255) / 256), dim3(256), 0, s, cu_q, cu_k,
                     B, total_q, w_pretrained, pos, f, G);
  return hipGetLastError();
}

// The classifier the prefill kernels route on, over one sequence's blocks.
__global__ void tile_classes_kernel(int Lq, int L, int w0, int BM, int BN, int nqb, int nkb,
                                    uint8_t* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(nqb) * nkb) return;
  const int a = static_cast<int>(idx / nkb);
  const int bk = static_cast<int>(idx % nkb);
  const int q_off = L - Lq;
  const int i0 = q_off + a * BM;
  const int i1 = min(q_off + Lq, i0 + BM) - 1;
  const int j0 = bk * BN;
  const int j1 = min(L, j0 + BN) - 1;
  out[idx] = static_cast<uint8_t>(classify_tile(i0, i1, j0, j1, w0));
}

hipError_t launch_tile_classes(int Lq, int L, int w0, int BM, int BN, uint8_t* out,
                               hipStream_t s) {
  const int nqb = (Lq + BM - 1) / BM;
  const int nkb = (L + BN - 1) / BN;
  const int64_t n = static_cast<int64_t>(nqb) * nkb;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(tile_classes_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                     0, s, Lq, L, w0, BM, BN, nqb, nkb, out);
  return hipGetLastError();
}

}  // namespace jl
