// fp32 prefill of dynamic bifocal RoPE attention (VALU, gfx950).
//
// "Jet-Long: Efficient Long-Context Extension with Dynamic Bifocal RoPE",
// section "Dynamic Bifocal RoPE": pairs closer than w0 use classic RoPE at the
// true positions, the others RoPE at f(x) = floor(x / G) (eq. G, eq. f).
//
// This is the full-precision variant: every product runs in fp32 FMA.  Each
// key tile is rotated on the fly, in LDS, at both angle sets (true position
// and grouped position) straight from the raw keys, so no rotated copy of K
// is ever stored.  One workgroup = one wavefront = 64 query rows of one head;
// the 64 rows read the same rotated tile (LDS broadcast) and each lane picks,
// per key, the local or the remote pair of vectors by its own distance.
#include "jl_device.hpp"
#include "jl_launch.hpp"

namespace jl {

namespace {

constexpr int kRows = 64;
constexpr int kBN = 32;

struct Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const float2* tab;
  int B, total_q, Hq, Hkv, ratio, nqb, max_q, max_k;
  int w_pretrained, w0;
  float scale_log2;
  int prerot;  // q and k arrive rotated at their true positions
  // 0: the routed result.  Window passes of the inclusion-exclusion merge,
  // only pairs closer than w0: 1 rotated at the true positions, 2 at the
  // grouped ones.  (Its full pass is mode 0 with w0 = 0.)
  int mode;
};

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(Params p) {
  constexpr int H = D / 2;
  constexpr int QSTR = D + 1;  // odd stride: one bank per lane
  __shared__ float sQl[kRows * QSTR];
  __shared__ float sQr[kRows * QSTR];
  __shared__ float sKl[kBN * D];
  __shared__ float sKr[kBN * D];
  __shared__ float sV[kBN * D];

  const int t = threadIdx.x;
  const int qb = p.nqb - 1 - static_cast<int>(blockIdx.x);  // heaviest first
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int hkv = h / p.ratio;
  const int qbeg = p.cu_q[b];
  const int Lq = p.cu_q[b + 1] - qbeg;
  const int kbeg = p.cu_k[b];
  const int L = p.cu_k[b + 1] - kbeg;
  // sequences that break the documented contract are left unwritten
  if (Lq < 0 || Lq > L || L > p.max_k || Lq > p.max_q) return;
  if (qb * kRows >= Lq) return;
  const int q_off = L - Lq;
  const int G = group_size(L, p.w_pretrained);
  const int i0 = q_off + qb * kRows;
  const int i1 = min(q_off + Lq, i0 + kRows) - 1;
  const int qi = i0 + t;
  const bool qvalid = qi <= i1;

  // this lane's query row, rotated at p and f(p)
  {
    const int pl = qvalid ? qi : 0;
    const RotRow rl = rot_row(pl, pl, p.prerot);
    const RotRow rr = rot_row(pl / G, pl, p.prerot);
    const float* src = p.q + (static_cast<int64_t>(qbeg + (qvalid ? qi - q_off : 0)) * p.Hq + h) * D;
    for (int kk = 0; kk < H; ++kk) {
      const float x1 = qvalid ? src[kk] : 0.f;
      const float x2 = qvalid ? src[kk + H] : 0.f;
      float2 cl = p.tab[static_cast<int64_t>(rl.row) * H + kk];
      float2 cr = p.tab[static_cast<int64_t>(rr.row) * H + kk];
      cl.y *= rl.sgn;
      cr.y *= rr.sgn;
      sQl[t * QSTR + kk] = x1 * cl.x - x2 * cl.y;
      sQl[t * QSTR + kk + H] = x2 * cl.x + x1 * cl.y;
      sQr[t * QSTR + kk] = x1 * cr.x - x2 * cr.y;
      sQr[t * QSTR + kk + H] = x2 * cr.x + x1 * cr.y;
    }
  }

  float acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float* qlrow = &sQl[t * QSTR];
  const float* qrrow = &sQr[t * QSTR];

  const int nkt = i1 / kBN + 1;
  const int kt0 = p.mode ? max(0, i0 - p.w0 + 1) / kBN : 0;
  for (int kt = kt0; kt < nkt; ++kt) {
    const int j0 = kt * kBN;
    __syncthreads();
    // rotate the raw key tile at both angle sets into LDS
    for (int idx = t; idx < kBN * H; idx += 64) {
      const int jj = idx / H;
      const int kk = idx % H;
      const int j = j0 + jj;
      float l1 = 0.f, l2 = 0.f, r1 = 0.f, r2 = 0.f;
      if (j < L) {
        const float* src = p.k + (static_cast<int64_t>(kbeg + j) * p.Hkv + hkv) * D;
        const float x1 = src[kk];
        const float x2 = src[kk + H];
        const RotRow rl = rot_row(j, j, p.prerot);
        const RotRow rr = rot_row(j / G, j, p.prerot);
        float2 cl = p.tab[static_cast<int64_t>(rl.row) * H + kk];
        float2 cr = p.tab[static_cast<int64_t>(rr.row) * H + kk];
        cl.y *= rl.sgn;
        cr.y *= rr.sgn;
        l1 = x1 * cl.x - x2 * cl.y;
        l2 = x2 * cl.x + x1 * cl.y;
        r1 = x1 * cr.x - x2 * cr.y;
        r2 = x2 * cr.x + x1 * cr.y;
      }
      sKl[jj * D + kk] = l1;
      sKl[jj * D + kk + H] = l2;
      sKr[jj * D + kk] = r1;
      sKr[jj * D + kk + H] = r2;
    }
    for (int idx = t; idx < kBN * D; idx += 64) {
      const int jj = idx / D;
      const int e = idx % D;
      const int j = j0 + jj;
      sV[idx] = j < L ? p.v[(static_cast<int64_t>(kbeg + j) * p.Hkv + hkv) * D + e] : 0.f;
    }
    __syncthreads();

    float s[kBN];
    float mx = -INFINITY;
    for (int jj = 0; jj < kBN; ++jj) {
      const int j = j0 + jj;
      float sc = -INFINITY;
      const bool in_window = qi - j < p.w0;
      if (j <= qi && j < L && (p.mode == 0 || in_window)) {
        const bool local = p.mode == 0 ? in_window : p.mode == 1;
        const float* qv = local ? qlrow : qrrow;
        const float* kv = local ? &sKl[jj * D] : &sKr[jj * D];
        float dot = 0.f;
#pragma unroll 16
        for (int e = 0; e < D; ++e) dot = fmaf(qv[e], kv[e], dot);
        sc = dot * p.scale_log2;
      }
      s[jj] = sc;
      mx = fmaxf(mx, sc);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] *= alpha;
    for (int jj = 0; jj < kBN; ++jj) {
      const float pj = s[jj] == -INFINITY ? 0.f : exp2f(s[jj] - m_new);
      l_run += pj;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(pj, sV[jj * D + e], acc[e]);
    }
    m_run = m_new;
  }

  if (qvalid) {
    const int64_t tok = qbeg + qi - q_off;
    float* dst = p.o + (tok * p.Hq + h) * D;
    // only a window pass with w0 = 0 sees no key at all: O = 0, LSE = -inf
    const bool empty = !(l_run > 0.f);
    const float inv = empty ? 0.f : 1.f / l_run;
#pragma unroll
    for (int e = 0; e < D; ++e) dst[e] = acc[e] * inv;
    if (p.lse) p.lse[static_cast<int64_t>(h) * p.total_q + tok] = empty ? -INFINITY : (m_run + log2f(l_run)) * kLn2;
  }
}

}  // namespace

size_t prefill_ws_bytes_f32(int max_k, int D) {
  return align_up(static_cast<size_t>(max_k) * (D / 2) * sizeof(float2), 256);
}

hipError_t launch_prefill_f32_prepare(const PrefillCall& c, hipStream_t s) {
  if (c.B == 0 || c.total_k == 0) return hipSuccess;
  return launch_rope_table(static_cast<float2*>(c.ws), c.max_k, c.D, c.theta, s);
}

static Params make_params(const PrefillCall& c) {
  Params p{};
  p.q = static_cast<const float*>(c.q);
  p.k = static_cast<const float*>(c.k);
  p.v = static_cast<const float*>(c.v);
  p.o = static_cast<float*>(c.o);
  p.lse = c.lse;
  p.cu_q = c.cu_q;
  p.cu_k = c.cu_k;
  p.tab = static_cast<const float2*>(c.ws);
  p.B = c.B;
  p.total_q = c.total_q;
  p.Hq = c.Hq;
  p.Hkv = c.Hkv;
  p.ratio = c.Hq / c.Hkv;
  p.nqb = (c.max_q + kRows - 1) / kRows;
  p.max_q = c.max_q;
  p.max_k = c.max_k;
  p.w_pretrained = c.w_pretrained;
  p.w0 = c.w0;
  p.scale_log2 = c.scale * kLog2e;
  p.prerot = c.prerot ? 1 : 0;
  return p;
}

static hipError_t launch(const Params& p, int D, hipStream_t s) {
  const dim3 grid(p.nqb, p.Hq, p.B);
  if (D == 128) hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, s, p);
  else hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prefill_f32_attend(const PrefillCall& c, hipStream_t s) {
  if (c.total_q == 0 || c.B == 0) return hipSuccess;
  return launch(make_params(c), c.D, s);
}

hipError_t launch_prefill_f32_ie_pass(const PrefillCall& c, int pass, float* o, float* lse, hipStream_t s) {
  if (c.total_q == 0 || c.B == 0) return hipSuccess;
  Params p = make_params(c);
  p.o = o;
  p.lse = lse;
  if (pass == kIeFullRemote) p.w0 = 0;
  else p.mode = pass == kIeWindowLocal ? 1 : 2;
  return launch(p, c.D, s);
}

}  // namespace jl
