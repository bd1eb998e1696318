// bf16 prefill of dynamic bifocal RoPE attention on gfx950 MFMA.
//
// "Jet-Long: Efficient Long-Context Extension with Dynamic Bifocal RoPE",
// section "Dynamic Bifocal RoPE" (local window w0 with classic RoPE, remote
// pairs at f(x) = floor(x / G), eq. G / eq. f) and section "Inference
// Efficiency Mechanisms" (the pages reach the routed result by an
// inclusion-exclusion merge of three FlashAttention passes; here each key
// tile is routed instead, and only tiles that straddle the window edge form
// both logit sets).
//
// Two kernels per call, both on the caller's stream:
//  1. prep: every key row is rotated once at its true position p and once at
//     f(p) (head-major rows padded per sequence to a multiple of 64) and V is
//     laid out transposed per head, [d][key], so that the PV product can read
//     8 keys of one feature as two 8-byte LDS reads.  The raw K/V inputs are
//     only read.
//  Operand precision: the MFMA operands (rotated Q and K, P, V) are IEEE
//  half, accumulation is fp32.  bf16 inputs convert to half exactly (within
//  +-65504), and rotation keeps each pair's norm, while a rotated value
//  rounded back to bf16 would carry 8x the rounding error of half (8 vs 11
//  significant bits) at the same MFMA rate.
//  2. attention: one workgroup = 8 wavefronts = one KV head x HPW query heads
//     x (32 * 8 / HPW) query positions.  S^T = K Q^T runs on
//     v_mfma_f32_32x32x16_f16 with the rotated key tile (LDS) as A and the
//     query (registers, rotated at p and f(p) in the prologue from the fp32
//     cos/sin table) as B; the accumulator layout puts one query per lane, so
//     the online softmax needs one cross-half exchange, and the same registers
//     become the B operand of O^T = V^T P^T.
#include "jl_device.hpp"
#include "jl_launch.hpp"

namespace jl {

namespace {

constexpr int kBN = 64;     // keys per tile
constexpr int kWaves = 8;   // wavefronts per workgroup
constexpr int kThreads = kWaves * 64;

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const float2* tab;  // [max_k][D/2]
  uint16_t* kr;       // [Hkv][tpad][D]  keys rotated at f(p), half
  uint16_t* kl;       // [Hkv][tpad][D]  keys rotated at p, half
  uint16_t* vt;       // [Hkv][D][tpad]  values, transposed, half
  int64_t tpad;
  int B, total_q, Hq, Hkv, ratio, ngroups, nqb, max_q, max_k;
  int w_pretrained, w0;
  float scale_log2;   // softmax scale * log2(e)
};

// First padded key row of sequence b: rows of different sequences never
// share a 64-row tile, and every sequence owns its tail rows up to the next
// multiple of 64.
__device__ __forceinline__ int64_t key_row_offset(const int32_t* cu_k, int b) {
  return (static_cast<int64_t>(cu_k[b]) + 63) / 64 * 64 + 64LL * b;
}

// ---------------------------------------------------------------- prep pass
// grid (tpad / 64, Hkv, D / 16), 64 threads; thread = one padded key row and
// one 1/(D/16) slice of the features.
template <int D>
__global__ __launch_bounds__(64) void prep_kernel(Params p) {
  constexpr int H = D / 2;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 64 + threadIdx.x;
  const int hk = blockIdx.y;
  const int c = blockIdx.z;  // K: elements c*8..+7 and H+c*8..+7; V: c*16..+15
  if (r >= p.tpad) return;
  int lo = 0, hi = p.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (key_row_offset(p.cu_k, mid) <= r) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int64_t pos64 = r - key_row_offset(p.cu_k, b);
  const int L = p.cu_k[b + 1] - p.cu_k[b];
  if (L < 0 || L > p.max_k) return;
  if (pos64 < 0 || pos64 >= ((static_cast<int64_t>(L) + 63) & ~63LL)) return;  // gap rows
  const int pos = static_cast<int>(pos64);
  uint16_t* kl_row = p.kl + (static_cast<int64_t>(hk) * p.tpad + r) * D;
  uint16_t* kr_row = p.kr + (static_cast<int64_t>(hk) * p.tpad + r) * D;
  uint16_t* vt_col = p.vt + static_cast<int64_t>(hk) * D * p.tpad + r;
  if (pos < L) {
    const int64_t tok = p.cu_k[b] + pos;
    const int G = group_size(L, p.w_pretrained);
    const int fp = pos / G;
    const uint16_t* src = p.k + (tok * p.Hkv + hk) * D;
    const uint4 a = *reinterpret_cast<const uint4*>(src + c * 8);
    const uint4 bb = *reinterpret_cast<const uint4*>(src + H + c * 8);
    const uint32_t xa[4] = {a.x, a.y, a.z, a.w};
    const uint32_t xb[4] = {bb.x, bb.y, bb.z, bb.w};
    uint32_t la[4], lb[4], ra[4], rb[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      float l1[2], l2[2], r1[2], r2[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int kk = c * 8 + e2 * 2 + hh;
        const float x1 = bf16_bits_to_float(static_cast<uint16_t>(xa[e2] >> (16 * hh)));
        const float x2 = bf16_bits_to_float(static_cast<uint16_t>(xb[e2] >> (16 * hh)));
        const float2 cl = p.tab[static_cast<int64_t>(pos) * H + kk];
        const float2 cr = p.tab[static_cast<int64_t>(fp) * H + kk];
        l1[hh] = x1 * cl.x - x2 * cl.y;
        l2[hh] = x2 * cl.x + x1 * cl.y;
        r1[hh] = x1 * cr.x - x2 * cr.y;
        r2[hh] = x2 * cr.x + x1 * cr.y;
      }
      la[e2] = pack_f16x2(l1[0], l1[1]);
      lb[e2] = pack_f16x2(l2[0], l2[1]);
      ra[e2] = pack_f16x2(r1[0], r1[1]);
      rb[e2] = pack_f16x2(r2[0], r2[1]);
    }
    *reinterpret_cast<uint4*>(kl_row + c * 8) = make_uint4(la[0], la[1], la[2], la[3]);
    *reinterpret_cast<uint4*>(kl_row + H + c * 8) = make_uint4(lb[0], lb[1], lb[2], lb[3]);
    *reinterpret_cast<uint4*>(kr_row + c * 8) = make_uint4(ra[0], ra[1], ra[2], ra[3]);
    *reinterpret_cast<uint4*>(kr_row + H + c * 8) = make_uint4(rb[0], rb[1], rb[2], rb[3]);
    const uint16_t* vs = p.v + (tok * p.Hkv + hk) * D + c * 16;
    const uint4 v0 = *reinterpret_cast<const uint4*>(vs);
    const uint4 v1 = *reinterpret_cast<const uint4*>(vs + 8);
    const uint32_t vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float x = bf16_bits_to_float(static_cast<uint16_t>(vv[e >> 1] >> (16 * (e & 1))));
      vt_col[static_cast<int64_t>(c * 16 + e) * p.tpad] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
    }
  } else {
    const uint4 z = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(kl_row + c * 8) = z;
    *reinterpret_cast<uint4*>(kl_row + H + c * 8) = z;
    *reinterpret_cast<uint4*>(kr_row + c * 8) = z;
    *reinterpret_cast<uint4*>(kr_row + H + c * 8) = z;
#pragma unroll
    for (int e = 0; e < 16; ++e) vt_col[static_cast<int64_t>(c * 16 + e) * p.tpad] = 0;
  }
}

// ---------------------------------------------------------------- attention

template <int D, int HPW>
__global__ __launch_bounds__(kThreads) void attn_kernel(Params p) {
  constexpr int RB = kWaves / HPW;  // 32-row blocks per query head
  constexpr int ROWS = 32 * RB;     // query positions per workgroup
  constexpr int KS = D / 16;        // k-steps of QK^T
  constexpr int MB = D / 32;        // 32-feature blocks of O^T
  constexpr int H = D / 2;
  constexpr int KSTR = D + 8;       // LDS row stride of key tiles (elements)
  constexpr int VSTR = kBN + 4;     // LDS row stride of V^T tiles (elements)
  constexpr int KCH = kBN * D / 8;  // 16-byte chunks per key tile
  constexpr int KPT = (KCH + kThreads - 1) / kThreads;
  constexpr int VCH = D * kBN / 8;
  constexpr int VPT = (VCH + kThreads - 1) / kThreads;

  __shared__ __attribute__((aligned(16))) uint16_t sKr[2][kBN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sKl[2][kBN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;

  // heaviest query blocks first; consecutive ids cycle over the KV heads so
  // that one XCD keeps revisiting the same head's tiles
  const int units = p.B * p.Hkv * p.ngroups;
  const int id = blockIdx.x;
  const int qb = p.nqb - 1 - id / units;
  int rest = id % units;
  const int hkv = rest % p.Hkv;
  rest /= p.Hkv;
  const int grp = rest % p.ngroups;
  const int b = rest / p.ngroups;

  const int qbeg = p.cu_q[b];
  const int Lq = p.cu_q[b + 1] - qbeg;
  const int L = p.cu_k[b + 1] - p.cu_k[b];
  // sequences that break the documented contract are left unwritten
  if (Lq < 0 || Lq > L || L > p.max_k || Lq > p.max_q) return;
  if (qb * ROWS >= Lq) return;
  const int q_off = L - Lq;
  const int G = group_size(L, p.w_pretrained);
  const int i0 = q_off + qb * ROWS;
  const int i1 = min(q_off + Lq, i0 + ROWS) - 1;
  const int64_t krow0 = key_row_offset(p.cu_k, b);

  const int hs = w % HPW;
  const int rb = w / HPW;
  const int h = hkv * p.ratio + grp * HPW + hs;
  const int r32 = lane & 31;
  const int g = lane >> 5;
  const int qi = i0 + rb * 32 + r32;
  const bool qvalid = qi <= i1;

  // ---- query fragments rotated at p (local) and f(p) (remote)
  f16x8 qlf[KS], qrf[KS];
  {
    float x[KS][8];
    if (qvalid) {
      const uint16_t* src = p.q + (static_cast<int64_t>(qbeg + qi - q_off) * p.Hq + h) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 u = *reinterpret_cast<const uint4*>(src + ks * 16 + g * 8);
        const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          x[ks][e] = bf16_bits_to_float(static_cast<uint16_t>(uu[e >> 1] >> (16 * (e & 1))));
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[ks][e] = 0.f;
    }
    const int pl = qvalid ? qi : 0;
    const int pr = pl / G;
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = ks * 16 + g * 8 + e;
        const float2 cl = p.tab[static_cast<int64_t>(pl) * H + kk];
        const float2 cr = p.tab[static_cast<int64_t>(pr) * H + kk];
        const float x1 = x[ks][e];
        const float x2 = x[ks + KS / 2][e];
        qlf[ks][e] = static_cast<_Float16>(x1 * cl.x - x2 * cl.y);
        qlf[ks + KS / 2][e] = static_cast<_Float16>(x2 * cl.x + x1 * cl.y);
        qrf[ks][e] = static_cast<_Float16>(x1 * cr.x - x2 * cr.y);
        qrf[ks + KS / 2][e] = static_cast<_Float16>(x2 * cr.x + x1 * cr.y);
      }
    }
  }

  // ---- tile loader (global -> registers -> LDS), double buffered
  const uint16_t* kr_base = p.kr + static_cast<int64_t>(hkv) * p.tpad * D;
  const uint16_t* kl_base = p.kl + static_cast<int64_t>(hkv) * p.tpad * D;
  const uint16_t* vt_base = p.vt + static_cast<int64_t>(hkv) * D * p.tpad;
  uint4 rk[KPT], rkl[KPT], rv[VPT];

  auto tile_class = [&](int kt) {
    const int j0 = kt * kBN;
    return classify_tile(i0, i1, j0, min(L, j0 + kBN) - 1, p.w0);
  };
  auto issue = [&](int kt, int cls) {
    const int64_t row0 = krow0 + static_cast<int64_t>(kt) * kBN;
    const int base = cls & 3;
    if (base != kLocal) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int c = tid + i * kThreads;
        if (c < KCH)
          rk[i] = *reinterpret_cast<const uint4*>(kr_base + (row0 + c / (D / 8)) * D + (c % (D / 8)) * 8);
      }
    }
    if (base != kRemote) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int c = tid + i * kThreads;
        if (c < KCH)
          rkl[i] = *reinterpret_cast<const uint4*>(kl_base + (row0 + c / (D / 8)) * D + (c % (D / 8)) * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * kThreads;
      if (c < VCH)
        rv[i] = *reinterpret_cast<const uint4*>(vt_base + static_cast<int64_t>(c / (kBN / 8)) * p.tpad + row0 + (c % (kBN / 8)) * 8);
    }
  };
  auto commit = [&](int buf, int cls) {
    const int base = cls & 3;
    if (base != kLocal) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int c = tid + i * kThreads;
        if (c < KCH) *reinterpret_cast<uint4*>(&sKr[buf][(c / (D / 8)) * KSTR + (c % (D / 8)) * 8]) = rk[i];
      }
    }
    if (base != kRemote) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int c = tid + i * kThreads;
        if (c < KCH) *reinterpret_cast<uint4*>(&sKl[buf][(c / (D / 8)) * KSTR + (c % (D / 8)) * 8]) = rkl[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * kThreads;
      if (c < VCH) {
        uint16_t* dst = &sV[buf][(c / (kBN / 8)) * VSTR + (c % (kBN / 8)) * 8];
        reinterpret_cast<uint2*>(dst)[0] = make_uint2(rv[i].x, rv[i].y);
        reinterpret_cast<uint2*>(dst)[1] = make_uint2(rv[i].z, rv[i].w);
      }
    }
  };

  // ---- main loop
  float m_run = -INFINITY;  // running max, log2 domain
  float l_run = 0.f;
  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;

  const int nkt = i1 / kBN + 1;
  int cls = tile_class(0);
  issue(0, cls);
  commit(0, cls);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    int ncls = 0;
    if (kt + 1 < nkt) {
      ncls = tile_class(kt + 1);
      issue(kt + 1, ncls);
    }
    const int base = cls & 3;
    const int j0 = kt * kBN;
    const bool need_mask = (cls & kDiag) || (j0 + kBN > L);

    f32x16 sr[2], sl[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) { sr[kb][r] = 0.f; sl[kb][r] = 0.f; }
    if (base != kLocal) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const f16x8 a = *reinterpret_cast<const f16x8*>(&sKr[buf][(kb * 32 + r32) * KSTR + ks * 16 + g * 8]);
          sr[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qrf[ks], sr[kb], 0, 0, 0);
        }
    }
    if (base != kRemote) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const f16x8 a = *reinterpret_cast<const f16x8*>(&sKl[buf][(kb * 32 + r32) * KSTR + ks * 16 + g * 8]);
          sl[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qlf[ks], sl[kb], 0, 0, 0);
        }
    }

    // routing, masking, scaling (lane = one query; register r = one key)
    float t[2][16];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kj = j0 + kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
        float s;
        if (base == kRemote) s = sr[kb][r];
        else if (base == kLocal) s = sl[kb][r];
        else s = (qi - kj < p.w0) ? sl[kb][r] : sr[kb][r];
        s *= p.scale_log2;
        if (need_mask && (kj > qi || kj >= L)) s = -INFINITY;
        t[kb][r] = s;
        mx = fmaxf(mx, s);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        t[kb][r] = exp2f(t[kb][r] - m_new);
        rs += t[kb][r];
      }
    rs += __shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][r] *= alpha;

    // P^T fragments: k-step ks2 covers tile keys ks2*16 .. ks2*16+15
    f16x8 pf[4];
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[ks2][e] = static_cast<_Float16>(t[ks2 >> 1][(ks2 & 1) * 8 + e]);

    // O^T += V^T P^T; A slot s of lane half g holds key ks2*16 + (s/4)*8 + g*4 + s%4,
    // the same key the P^T slot s holds
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int ks2 = 0; ks2 < 4; ++ks2) {
        const uint16_t* vr = &sV[buf][(mb * 32 + r32) * VSTR + ks2 * 16 + g * 4];
        const uint2 lo = *reinterpret_cast<const uint2*>(vr);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
        const uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
        const f16x8 a = __builtin_bit_cast(f16x8, u);
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[ks2], acc[mb], 0, 0, 0);
      }

    if (kt + 1 < nkt) commit(buf ^ 1, ncls);
    __syncthreads();
    cls = ncls;
  }

  // ---- epilogue: lane holds query qi, features mb*32 + (r/4)*8 + g*4 + r%4
  if (qvalid) {
    const float inv = 1.f / l_run;
    const int64_t tok = qbeg + qi - q_off;
    uint16_t* dst = p.o + (tok * p.Hq + h) * D;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = mb * 32 + q4 * 8 + g * 4;
        const uint32_t w0v = pack_bf16x2(acc[mb][q4 * 4 + 0] * inv, acc[mb][q4 * 4 + 1] * inv);
        const uint32_t w1v = pack_bf16x2(acc[mb][q4 * 4 + 2] * inv, acc[mb][q4 * 4 + 3] * inv);
        *reinterpret_cast<uint2*>(dst + d) = make_uint2(w0v, w1v);
      }
    if (p.lse && g == 0) p.lse[static_cast<int64_t>(h) * p.total_q + tok] = (m_run + log2f(l_run)) * kLn2;
  }
}

int heads_per_wg(int ratio) { return ratio % 4 == 0 ? 4 : (ratio % 2 == 0 ? 2 : 1); }

template <int D, int HPW>
hipError_t launch_attn(const Params& prm, int nqb, hipStream_t s) {
  const int units = prm.B * prm.Hkv * prm.ngroups;
  const int64_t blocks = static_cast<int64_t>(nqb) * units;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_kernel<D, HPW>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, prm);
  return hipGetLastError();
}

}  // namespace

void prefill_bf16_tile_shape(int ratio, int* BM, int* BN) {
  *BM = 32 * kWaves / heads_per_wg(ratio);
  *BN = kBN;
}

static int64_t prefill_tpad(int B, int total_k) {
  return (static_cast<int64_t>(total_k) + 63) / 64 * 64 + 64LL * B;
}

size_t prefill_ws_bytes_bf16(int B, int total_k, int max_k, int Hkv, int D) {
  const size_t tab = align_up(static_cast<size_t>(max_k) * (D / 2) * sizeof(float2), 256);
  const size_t rows = static_cast<size_t>(prefill_tpad(B, total_k)) * Hkv * D * sizeof(uint16_t);
  return tab + 3 * align_up(rows, 256);
}

hipError_t launch_prefill_bf16(const PrefillCall& c, hipStream_t s) {
  if (c.total_q == 0 || c.B == 0) return hipSuccess;
  const int64_t tpad = prefill_tpad(c.B, c.total_k);
  char* ws = static_cast<char*>(c.ws);
  const size_t tab_bytes = align_up(static_cast<size_t>(c.max_k) * (c.D / 2) * sizeof(float2), 256);
  const size_t rows = align_up(static_cast<size_t>(tpad) * c.Hkv * c.D * sizeof(uint16_t), 256);
  Params p{};
  p.q = static_cast<const uint16_t*>(c.q);
  p.k = static_cast<const uint16_t*>(c.k);
  p.v = static_cast<const uint16_t*>(c.v);
  p.o = static_cast<uint16_t*>(c.o);
  p.lse = c.lse;
  p.cu_q = c.cu_q;
  p.cu_k = c.cu_k;
  p.tab = reinterpret_cast<const float2*>(ws);
  p.kr = reinterpret_cast<uint16_t*>(ws + tab_bytes);
  p.kl = reinterpret_cast<uint16_t*>(ws + tab_bytes + rows);
  p.vt = reinterpret_cast<uint16_t*>(ws + tab_bytes + 2 * rows);
  p.tpad = tpad;
  p.B = c.B;
  p.total_q = c.total_q;
  p.Hq = c.Hq;
  p.Hkv = c.Hkv;
  p.ratio = c.Hq / c.Hkv;
  const int hpw = heads_per_wg(p.ratio);
  p.ngroups = p.ratio / hpw;
  const int rows_per_wg = 32 * kWaves / hpw;
  p.nqb = (c.max_q + rows_per_wg - 1) / rows_per_wg;
  p.max_q = c.max_q;
  p.max_k = c.max_k;
  p.w_pretrained = c.w_pretrained;
  p.w0 = c.w0;
  p.scale_log2 = c.scale * kLog2e;

  hipError_t e = launch_rope_table(reinterpret_cast<float2*>(ws), c.max_k, c.D, c.theta, s);
  if (e != hipSuccess) return e;
  if (c.total_k > 0) {
    const dim3 pg(static_cast<unsigned>((tpad + 63) / 64), c.Hkv, c.D / 16);
    if (c.D == 128) hipLaunchKernelGGL(prep_kernel<128>, pg, dim3(64), 0, s, p);
    else hipLaunchKernelGGL(prep_kernel<64>, pg, dim3(64), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (c.D == 128) {
    if (hpw == 4) return launch_attn<128, 4>(p, p.nqb, s);
    if (hpw == 2) return launch_attn<128, 2>(p, p.nqb, s);
    return launch_attn<128, 1>(p, p.nqb, s);
  }
  if (hpw == 4) return launch_attn<64, 4>(p, p.nqb, s);
  if (hpw == 2) return launch_attn<64, 2>(p, p.nqb, s);
  return launch_attn<64, 1>(p, p.nqb, s);
}

}  // namespace jl
