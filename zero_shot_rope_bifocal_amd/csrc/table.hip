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
// With seq_L given (decode), only rows a decode can read are written.  Work
// items (one run of kRun rows for one frequency; a wavefront holds whole
// runs): items [0, n0) cover the rows below `rows0` (every remote position
// f(j) < w_pretrained); items n0 + b * nw + r run r of sequence b's local
// window [max(L_b - w0, rows0), L_b), skipped when sequence b - 1 has the
// same length; items n0 + B * nw + b the two rows its query is rotated with,
// L_b - 1 and f(L_b - 1).  With q32_only set (the bf16 decode, whose keys
// read the half rows only) the fp32 rows are written for the query rows
// alone.  With tab16 given, the same rows are also written as half: entry kp
// of row p holds (cos, cos, sin, sin) of frequencies 2kp and 2kp + 1, the
// operand order of a packed-half rotation.  Runs start at multiples of kRun,
// so a row that two items write (overlapping windows) gets the same bits.
constexpr int kRun = 32;

__global__ void rope_table_kernel(float2* __restrict__ tab, uint16_t* __restrict__ tab16, int npos, int half,
                                  double theta, double neg2_over_d, const int32_t* __restrict__ seq_L, int B,
                                  int w0, int rows0, int nw, int w_pretrained, int q32_only) {
  const int k = threadIdx.x % half;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * (blockDim.x / half) + threadIdx.x / half;
  const int n0 = (rows0 + kRun - 1) / kRun;
  int p0 = 0, hi = rows0;
  if (item < n0) {
    p0 = static_cast<int>(item) * kRun;
  } else {
    if (!seq_L) return;
    const int64_t wi = item - n0;
    const int b = static_cast<int>(wi < static_cast<int64_t>(B) * nw ? wi / nw : wi - static_cast<int64_t>(B) * nw);
    if (b >= B) return;
    const int Lb = seq_L[b];
    if (Lb < 1 || Lb > npos) return;  // a sequence the decode leaves unwritten
    if (wi >= static_cast<int64_t>(B) * nw) {
      // the query's rows, fp32 only; without q32_only the other items hold
      // them, except row L_b - 1 when the window is empty
      const double inv = pow(theta, neg2_over_d * k);
      const int rows[2] = {Lb - 1, (Lb - 1) / group_size(Lb, w_pretrained)};
      for (int i = 0; i < 2; ++i) {
        if (!q32_only && (rows[i] < rows0 || w0 > 0)) continue;
        double sv, cv;
        sincos(static_cast<double>(rows[i]) * inv, &sv, &cv);
        tab[static_cast<int64_t>(rows[i]) * half + k] = make_float2(static_cast<float>(cv), static_cast<float>(sv));
      }
      return;
    }
    if (b > 0 && seq_L[b - 1] == Lb) return;
    const int lo = max(Lb - w0, rows0);
    hi = Lb;
    if (lo >= hi) return;
    p0 = lo / kRun * kRun + static_cast<int>(wi % nw) * kRun;
  }
  if (p0 >= hi) return;
  const int pend = min(hi, p0 + kRun);
  const double inv = pow(theta, neg2_over_d * k);
  double s, c, s1, c1;
  sincos(static_cast<double>(p0) * inv, &s, &c);
  sincos(inv, &s1, &c1);
  for (int p = p0; p < pend; ++p) {
    if (!q32_only) tab[static_cast<int64_t>(p) * half + k] = make_float2(static_cast<float>(c), static_cast<float>(s));
    if (tab16) {
      // frequencies k and k + 1 sit in neighbouring lanes of one run; the
      // even lane writes the pair's 8-byte entry
      const uint32_t cs = pack_f16x2(static_cast<float>(c), static_cast<float>(s));
      const uint32_t odd = __shfl_down(cs, 1);
      if (!(k & 1))
        *reinterpret_cast<uint2*>(tab16 + (static_cast<int64_t>(p) * (half / 2) + k / 2) * 4) =
            make_uint2((cs & 0xffffu) | (odd << 16), (cs >> 16) | (odd & 0xffff0000u));
    }
    const double cn = c * c1 - s * s1;
    s = s * c1 + c * s1;
    c = cn;
  }
}

namespace {
hipError_t launch_table(float2* tab, int npos, int D, double theta, const int32_t* seq_L, int B, int w0, int rows0,
                        int w_pretrained, hipStream_t s, uint16_t* tab16) {
  const int half = D / 2;
  const int per_block = 256 / half;
  const int n0 = (rows0 + kRun - 1) / kRun;
  // runs of one window from its aligned start
  const int nw = seq_L ? ((w0 < npos ? w0 : npos) + kRun - 1) / kRun + 1 : 0;
  const int64_t items = n0 + (static_cast<int64_t>(nw) + 1) * (seq_L ? B : 0);
  const int64_t blocks = (items + per_block - 1) / per_block;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>(blocks)), dim3(per_block * half), 0, s, tab, tab16,
                     npos, half, theta, -2.0 / static_cast<double>(D), seq_L, B, w0, rows0, nw, w_pretrained,
                     seq_L && tab16 ? 1 : 0);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_rope_table(float2* tab, int npos, int D, double theta, hipStream_t s, uint16_t* tab16) {
  if (npos <= 0) return hipSuccess;
  return launch_table(tab, npos, D, theta, nullptr, 0, 0, npos, 1, s, tab16);
}

hipError_t launch_rope_table_rows(float2* tab, int npos, int D, double theta, const int32_t* seq_L, int B,
                                  int w0, int w_pretrained, hipStream_t s, uint16_t* tab16) {
  if (npos <= 0 || B <= 0) return hipSuccess;
  return launch_table(tab, npos, D, theta, seq_L, B, w0, w_pretrained < npos ? w_pretrained : npos, w_pretrained, s,
                      tab16);
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
