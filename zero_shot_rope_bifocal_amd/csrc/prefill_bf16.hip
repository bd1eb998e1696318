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
//     laid out transposed per head and 64-key tile, [tile][d][64 keys], with
//     each 16-key group in the k-slot order of the PV MFMA, so that one A
//     fragment (8 keys of one feature) is one 16-byte LDS read.  Every K and
//     V^T tile is then one contiguous 64 x d block.  The raw K/V inputs are
//     only read.
//  Operand precision: the MFMA operands (rotated Q and K, P, V) are IEEE
//  half, accumulation is fp32.  bf16 inputs convert to half exactly (within
//  +-65504), and rotation keeps each pair's norm, while a rotated value
//  rounded back to bf16 would carry 8x the rounding error of half (8 vs 11
//  significant bits) at the same MFMA rate.  A rotated key, value or scaled
//  query that half cannot hold is stored as NaN, so the rows that use it
//  come out NaN rather than finite and wrong.
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
constexpr int kWaves = 8;   // 32-row blocks per workgroup
#ifndef JL_PREFILL_NRB
#define JL_PREFILL_NRB 1
#endif

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
  uint16_t* vt;       // [Hkv][tpad / 64][D][64]  values, transposed per 64-key tile, half
  int64_t tpad;
  int B, total_q, Hq, Hkv, ratio, ngroups, nqb, max_q, max_k;
  int w_pretrained, w0;
  float scale_log2;   // softmax scale * log2(e)
  int prerot;         // q and k arrive rotated at their true positions
  float* o32;         // fp32 output rows of a merge pass (MODE != kModeBifocal)
  int band_remote;    // window pass at the grouped positions (kModeWindow)
};

// What one attention launch computes.  kModeBifocal is the routed result.
// The other two are passes of the inclusion-exclusion merge, with fp32
// output: kModeFull is plain causal attention over every key with one
// rotation (the caller passes w0 = 0, so every pair takes the grouped
// positions); kModeWindow keeps only the pairs closer than w0, rotated at
// the true positions, or at the grouped ones when band_remote is set (the
// caller then points kl at the grouped key copy).
enum : int { kModeBifocal = 0, kModeFull = 1, kModeWindow = 2 };

// First padded key row of sequence b: rows of different sequences never
// share a 64-row tile, and every sequence owns its tail rows up to the next
// multiple of 64.
__device__ __forceinline__ int64_t key_row_offset(const int32_t* cu_k, int b) {
  return (static_cast<int64_t>(cu_k[b]) + 63) / 64 * 64 + 64LL * b;
}

// ---------------------------------------------------------------- prep pass
// grid (tpad / 64, Hkv), 4 * D threads: a workgroup covers 64 padded key
// rows of one KV head; wavefront c takes one 1/(D/16) slice of the features
// of every row (lane = row), so the D/16 slices of a row are read and
// written together.
template <int D>
__global__ __launch_bounds__(4 * D) void prep_kernel(Params p) {
  constexpr int H = D / 2;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 64 + (threadIdx.x & 63);
  const int hk = blockIdx.y;
  const int c = threadIdx.x >> 6;  // K: elements c*8..+7 and H+c*8..+7; V: c*16..+15
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
  // V^T column of this key: inside each 16-key group the quads are stored in
  // the order 0, 2, 1, 3, which is the order the PV MFMA's k slots take them
  const int64_t rq = (r >> 2) & 3;
  const int64_t vcol = (r & ~15LL) | (((rq == 1) ? 2 : (rq == 2) ? 1 : rq) << 2) | (r & 3);
  uint16_t* vt_col = p.vt + static_cast<int64_t>(hk) * D * p.tpad + (r >> 6) * (D * 64) + (vcol & 63);
  if (pos < L) {
    const int64_t tok = p.cu_k[b] + pos;
    const int G = group_size(L, p.w_pretrained);
    const int fp = pos / G;
    // keys at p and at f(p) (or, for a pre-rotated cache, as stored and with
    // the correction rotation R(f(p) - p))
    const RotRow rl = rot_row(pos, pos, p.prerot);
    const RotRow rr = rot_row(fp, pos, p.prerot);
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
        float2 cl = p.tab[static_cast<int64_t>(rl.row) * H + kk];
        float2 cr = p.tab[static_cast<int64_t>(rr.row) * H + kk];
        cl.y *= rl.sgn;
        cr.y *= rr.sgn;
        l1[hh] = x1 * cl.x - x2 * cl.y;
        l2[hh] = x2 * cl.x + x1 * cl.y;
        r1[hh] = x1 * cr.x - x2 * cr.y;
        r2[hh] = x2 * cr.x + x1 * cr.y;
      }
      la[e2] = pack_f16x2_or_nan(l1[0], l1[1]);
      lb[e2] = pack_f16x2_or_nan(l2[0], l2[1]);
      ra[e2] = pack_f16x2_or_nan(r1[0], r1[1]);
      rb[e2] = pack_f16x2_or_nan(r2[0], r2[1]);
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
      vt_col[(c * 16 + e) * 64] = __builtin_bit_cast(uint16_t, half_or_nan(x));
    }
  } else {
    const uint4 z = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(kl_row + c * 8) = z;
    *reinterpret_cast<uint4*>(kl_row + H + c * 8) = z;
    *reinterpret_cast<uint4*>(kr_row + c * 8) = z;
    *reinterpret_cast<uint4*>(kr_row + H + c * 8) = z;
#pragma unroll
    for (int e = 0; e < 16; ++e) vt_col[(c * 16 + e) * 64] = 0;
  }
}

// ---------------------------------------------------------------- attention
//
// A workgroup covers one KV head, HPW of its query heads and 256 / HPW query
// positions; NW = 8 / NRB wavefronts each own one head and NRB blocks of 32
// positions.  With NRB = 2 every K / V fragment read from LDS feeds two MFMAs
// (one per row block), which halves LDS traffic per FLOP; the wave then runs
// alone on its SIMD with up to 512 registers.

constexpr int kVSTR = kBN + 8;  // LDS row stride of V^T tiles (elements, 16-byte rows)

// Per-thread registers of one prefetched tile (global -> registers -> LDS):
// CPT 16-byte chunks of each of K (remote), K (local) and V^T.
template <int CPT>
struct TileRegs {
  uint4 kr[CPT], kl[CPT], v[CPT];
};

// Where one lane's part of a tile comes from and goes: buffer resources over
// one KV head's rotated key copies and V^T tiles (the tile's byte offset is
// a scalar, the lane's byte offset inside the tile a constant), and the
// lane's element offsets inside an LDS key / V^T tile.  Lane tid moves the
// CPT consecutive chunks tid*CPT .. (always inside one LDS row).
struct TileSrc {
  __amdgpu_buffer_rsrc_t kr, kl, vt;
  uint32_t voff;  // bytes
  uint32_t lk, lv;  // LDS elements
};
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint16_t* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buf16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
template <int D, int NT>
__device__ __forceinline__ TileSrc tile_src(const uint16_t* kr_base, const uint16_t* kl_base, const uint16_t* vt_base,
                                            int64_t tpad, int tid) {
  constexpr int CPT = D * kBN / 8 / NT;
  const int c0 = tid * CPT;
  TileSrc s;
  s.kr = head_rsrc(kr_base, tpad * D * 2);
  s.kl = head_rsrc(kl_base, tpad * D * 2);
  s.vt = head_rsrc(vt_base, tpad * D * 2);
  s.voff = static_cast<uint32_t>(c0) * 16u;
  s.lk = static_cast<uint32_t>((c0 / (D / 8)) * (D + 8) + (c0 % (D / 8)) * 8);
  s.lv = static_cast<uint32_t>((c0 / (kBN / 8)) * kVSTR + (c0 % (kBN / 8)) * 8);
  return s;
}
template <int D>
__device__ __forceinline__ uint32_t tile_soff(int64_t row0) { return static_cast<uint32_t>(row0 * (D * 2)); }

template <int D, int NT>
__device__ __forceinline__ void load_tile(TileRegs<D * kBN / 8 / NT>& t, const TileSrc& s, uint32_t soff, int cls) {
  constexpr int CPT = D * kBN / 8 / NT;
  const int base = cls & 3;
  if (base != kLocal) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) t.kr[i] = buf16(s.kr, s.voff + i * 16, soff);
  }
  if (base != kRemote) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) t.kl[i] = buf16(s.kl, s.voff + i * 16, soff);
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) t.v[i] = buf16(s.vt, s.voff + i * 16, soff);
}

template <int D, int NT>
__device__ __forceinline__ void store_tile(const TileRegs<D * kBN / 8 / NT>& t, uint16_t* sKr, uint16_t* sKl,
                                           uint16_t* sV, int cls, const TileSrc& s) {
  constexpr int CPT = D * kBN / 8 / NT;
  const int base = cls & 3;
  if (base != kLocal) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) *reinterpret_cast<uint4*>(sKr + s.lk + i * 8) = t.kr[i];
  }
  if (base != kRemote) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) *reinterpret_cast<uint4*>(sKl + s.lk + i * 8) = t.kl[i];
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) *reinterpret_cast<uint4*>(sV + s.lv + i * 8) = t.v[i];
}

// load_tile / store_tile for a tile class known at compile time: inside the
// fast loops every load is unconditional, so the staging registers carry no
// control-flow merge (whose register copies would wait for the loads at once).
template <int D, int NT, int BASE>
__device__ __forceinline__ void load_tile_c(TileRegs<D * kBN / 8 / NT>& t, const TileSrc& s, uint32_t soff) {
  constexpr int CPT = D * kBN / 8 / NT;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    if constexpr (BASE != kLocal) t.kr[i] = buf16(s.kr, s.voff + i * 16, soff);
    if constexpr (BASE != kRemote) t.kl[i] = buf16(s.kl, s.voff + i * 16, soff);
    t.v[i] = buf16(s.vt, s.voff + i * 16, soff);
  }
}

template <int D, int NT, int BASE>
__device__ __forceinline__ void store_tile_c(const TileRegs<D * kBN / 8 / NT>& t, uint16_t* sKr, uint16_t* sKl,
                                             uint16_t* sV, const TileSrc& s) {
  constexpr int CPT = D * kBN / 8 / NT;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    if constexpr (BASE != kLocal) *reinterpret_cast<uint4*>(sKr + s.lk + i * 8) = t.kr[i];
    if constexpr (BASE != kRemote) *reinterpret_cast<uint4*>(sKl + s.lk + i * 8) = t.kl[i];
    *reinterpret_cast<uint4*>(sV + s.lv + i * 8) = t.v[i];
  }
}

// Raw bf16 query fragment of this lane (features ks*16 + g*8 + e), or zeros.
template <int D>
__device__ __forceinline__ void load_query(float (&x)[D / 16][8], const uint16_t* src, bool valid, int g) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (valid) u = *reinterpret_cast<const uint4*>(src + ks * 16 + g * 8);
    const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[ks][e] = bf16_bits_to_float(static_cast<uint16_t>(uu[e >> 1] >> (16 * (e & 1))));
  }
}

// Rotates this lane's query fragment by `rot` (table row and sign of sin, see
// rot_row) and scales it by c = softmax_scale * log2(e), so that the MFMA
// accumulators come out as log2-domain logits.
template <int D>
__device__ __forceinline__ void rotate_query(f16x8 (&out)[D / 16], const float (&x)[D / 16][8],
                                             const float2* __restrict__ tab, RotRow rot, int g, float c) {
  constexpr int KS = D / 16;
  const float2* row = tab + static_cast<int64_t>(rot.row) * (D / 2);
#pragma unroll
  for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float2 cs = row[ks * 16 + g * 8 + e];
      cs.y *= rot.sgn;
      const float x1 = x[ks][e], x2 = x[ks + KS / 2][e];
      out[ks][e] = half_or_nan((x1 * cs.x - x2 * cs.y) * c);
      out[ks + KS / 2][e] = half_or_nan((x2 * cs.x + x1 * cs.y) * c);
    }
}

// Value of lane l ^ 32 combined with lane l's own (max or sum), on the VALU.
__device__ __forceinline__ float xhalf_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// P^T (half) from log2-domain scores already relative to the row's running
// max; returns this lane's sum of the rounded probabilities (they are what
// P V multiplies), as a pairwise tree of packed half adds.  The tree is cheap
// next to the other wavefront's MFMAs (the f16 dot instructions that would
// sum in fp32 share the matrix pipeline and stall behind them); each level
// rounds to half, a relative error below 2^-11 per level, unbiased, against
// the bf16 rounding of the output.  A sum that overflows half comes out
// infinite, which the fast path's check catches; on the slow path every
// probability is at most 1.
__device__ __forceinline__ float lane_probs(const float (&t)[2][16], f16x8 (&pf)[4]) {
#pragma unroll
  for (int ks2 = 0; ks2 < 4; ++ks2)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      pf[ks2][e] = static_cast<_Float16>(__builtin_amdgcn_exp2f(t[ks2 >> 1][(ks2 & 1) * 8 + e]));
  f16x2 h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f16x2 a = {pf[i >> 1][(i & 1) * 4 + 0], pf[i >> 1][(i & 1) * 4 + 1]};
    const f16x2 b = {pf[i >> 1][(i & 1) * 4 + 2], pf[i >> 1][(i & 1) * 4 + 3]};
    h[i] = a + b;
  }
#pragma unroll
  for (int st = 4; st >= 1; st >>= 1)
#pragma unroll
    for (int i = 0; i < st; ++i) h[i] = h[i] + h[i + st];
  return static_cast<float>(h[0][0]) + static_cast<float>(h[0][1]);
}
// Row sum of P^T (both lane halves).
__device__ __forceinline__ float probs(const float (&t)[2][16], f16x8 (&pf)[4]) {
  return xhalf_sum(lane_probs(t, pf));
}

// O^T += V^T P^T for NRB row blocks: every V^T fragment (one 16-byte LDS read:
// each 16-key group of a V^T row is stored in the MFMA k-slot order by the
// prep pass) feeds NRB MFMAs.  Same read-ahead schedule as qk().
template <int D, int NRB>
__device__ __forceinline__ void pv(const uint16_t* __restrict__ v_lane, const f16x8 (&pf)[NRB][4],
                                   f32x16 (&acc)[NRB][D / 32]) {
  constexpr int MB = D / 32;
  constexpr int NF = 4 * MB;  // fragments: (k-step, feature block), feature block fastest
  constexpr int PF = 4;       // fragments read ahead of the MFMAs (measured best of 4 / 8 / all)
  f16x8 a[PF];
#pragma unroll
  for (int f = 0; f < PF; ++f)
    a[f] = *reinterpret_cast<const f16x8*>(v_lane + (f % MB) * 32 * kVSTR + (f / MB) * 16);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const f16x8 cur = a[f % PF];
    if (f + PF < NF)
      a[f % PF] = *reinterpret_cast<const f16x8*>(v_lane + ((f + PF) % MB) * 32 * kVSTR + ((f + PF) / MB) * 16);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
      acc[rb][f % MB] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur, pf[rb][f / MB], acc[rb][f % MB], 0, 0, 0);
  }
  // keep the read-ahead the loop above describes: PF reads, then one read per
  // MFMA, then the last MFMAs (the scheduler otherwise trades it for
  // registers and waits on every read)
  __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
  for (int f = 0; f < NF - PF; ++f) {
    __builtin_amdgcn_sched_group_barrier(0x008, NRB, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NRB * PF, 0);
}

// S^T of a 64-key tile for NRB row blocks (two 32-key blocks each); the
// accumulators start at `init`.  Every K fragment feeds NRB MFMAs.  The
// schedule keeps LDS reads PF fragments ahead of the MFMAs that consume them,
// so the read latency hides behind MFMA work instead of stalling each MFMA.
template <int D, int NRB>
__device__ __forceinline__ void qk(const uint16_t* __restrict__ k_lane, const f16x8 (&qf)[NRB][D / 16],
                                   const float (&init)[NRB], f32x16 (&sc)[NRB][2]) {
  constexpr int KSTR = D + 8;
  constexpr int KS = D / 16;
  constexpr int NF = 2 * KS;  // fragments per tile: (key block, k-step)
  constexpr int PF = 4;       // fragments read ahead of the MFMAs (measured best of 4 / 8 / all)
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[rb][kb][r] = init[rb];
  f16x8 a[PF];
#pragma unroll
  for (int f = 0; f < PF; ++f) a[f] = *reinterpret_cast<const f16x8*>(k_lane + (f & 1) * 32 * KSTR + (f >> 1) * 16);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const f16x8 cur = a[f % PF];
    if (f + PF < NF)
      a[f % PF] = *reinterpret_cast<const f16x8*>(k_lane + ((f + PF) & 1) * 32 * KSTR + ((f + PF) >> 1) * 16);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
      sc[rb][f & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur, qf[rb][f >> 1], sc[rb][f & 1], 0, 0, 0);
  }
  // keep the read-ahead the loop above describes: PF reads, then one read per
  // MFMA, then the last MFMAs (the scheduler otherwise trades it for
  // registers and waits on every read)
  __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
  for (int f = 0; f < NF - PF; ++f) {
    __builtin_amdgcn_sched_group_barrier(0x008, NRB, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NRB * PF, 0);
}

// Fast path of an unmasked tile scored with one rotation (all-remote, or
// all-local with the local rotations).  The score accumulators start at
// -m_run, so they come out relative to the running max and the
// probabilities follow at once.  If any lane's sum of them exceeds 2^12
// (some row's max may have risen by 7 or more, log2; an infinite or NaN sum
// included) the tile is left to the slow path, which recomputes it, and
// nothing is changed.  Otherwise every probability and partial sum is at
// most 2^12, well inside half range (half keeps its relative precision at
// any magnitude), the stale max stands and O needs no rescale.
template <int D, int NRB>
__device__ __forceinline__ bool tile_fast(const uint16_t* __restrict__ kr_lane,
                                          const uint16_t* __restrict__ v_lane,
                                          const f16x8 (&qrf)[NRB][D / 16], f32x16 (&acc)[NRB][D / 32],
                                          const float (&m_run)[NRB], float (&l_run)[NRB]) {
  float init[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) init[rb] = -m_run[rb];
  f32x16 sc[NRB][2];
  qk<D, NRB>(kr_lane, qrf, init, sc);
  f16x8 pf[NRB][4];
  float ls[NRB];
  bool grow = false;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    float t[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) t[kb][r] = sc[rb][kb][r];
    ls[rb] = lane_probs(t, pf[rb]);
    grow = grow || !(ls[rb] <= 4096.f);
  }
  if (__any(grow)) return false;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) l_run[rb] += xhalf_sum(ls[rb]);
  pv<D, NRB>(v_lane, pf, acc);
  return true;
}

// General tile (any class, optional mask) with an exact running-max update.
// USE_R / USE_L select which logit sets the tile needs (remote / local / both
// when it straddles the window edge); MASK adds the causal and
// end-of-sequence mask.  Lane (r32, g) holds query qi[rb]; accumulator
// register r of key block kb holds key j0g + kb*32 + (r/4)*8 + r%4 (j0g =
// tile start + g*4).  PAIRS keeps only some pairs: kPairsAll, kPairsRemote
// (distance >= w0) or kPairsWindow (distance < w0); with a selection a row may
// stay empty over a tile (running max -inf), which is guarded.
enum : int { kPairsAll = 0, kPairsRemote = 1, kPairsWindow = 2 };
template <int D, int NRB, bool USE_R, bool USE_L, bool MASK, int PAIRS = kPairsAll>
__device__ __forceinline__ void tile_slow(const uint16_t* __restrict__ kr_lane,
                                          const uint16_t* __restrict__ kl_lane,
                                          const uint16_t* __restrict__ v_lane,
                                          const f16x8 (&qrf)[NRB][D / 16], const f16x8 (&qlf)[NRB][D / 16],
                                          f32x16 (&acc)[NRB][D / 32], float (&m_run)[NRB], float (&l_run)[NRB],
                                          const int (&qi)[NRB], int j0g, int L, int w0) {
  float zero[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) zero[rb] = 0.f;
  f32x16 sr[NRB][2], sl[NRB][2];
  if constexpr (USE_R) qk<D, NRB>(kr_lane, qrf, zero, sr);
  if constexpr (USE_L) qk<D, NRB>(kl_lane, qlf, zero, sl);
  f16x8 pf[NRB][4];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    float t[2][16];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kj = j0g + kb * 32 + (r >> 2) * 8 + (r & 3);
        float s;
        if constexpr (USE_R && USE_L) s = (qi[rb] - kj < w0) ? sl[rb][kb][r] : sr[rb][kb][r];
        else if constexpr (USE_R) s = sr[rb][kb][r];
        else s = sl[rb][kb][r];
        if constexpr (MASK) s = (kj > qi[rb] || kj >= L) ? -INFINITY : s;
        if constexpr (PAIRS == kPairsWindow) s = (qi[rb] - kj >= w0) ? -INFINITY : s;
        if constexpr (PAIRS == kPairsRemote) s = (qi[rb] - kj < w0) ? -INFINITY : s;
        t[kb][r] = s;
        mx = fmaxf(mx, s);
      }
    mx = xhalf_max(mx);
    const float m_new = fmaxf(m_run[rb], mx);
    float m_use = m_new;
    if constexpr (PAIRS != kPairsAll) m_use = m_new == -INFINITY ? 0.f : m_new;  // empty so far: p = 0, no NaN
    const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_use);
    l_run[rb] *= alpha;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][mb][r] *= alpha;
    m_run[rb] = m_new;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) t[kb][r] -= m_use;
    l_run[rb] += probs(t, pf[rb]);
  }
  pv<D, NRB>(v_lane, pf, acc);
}

template <int D, int HPW, int NRB, int MODE>
__global__ __launch_bounds__(64 * 8 / NRB) void attn_kernel(Params p) {
  constexpr bool BAND = MODE == kModeWindow;
  constexpr int NW = 8 / NRB;       // wavefronts per workgroup
  constexpr int NT = NW * 64;       // threads per workgroup
  constexpr int ROWS = 32 * 8 / HPW;  // query positions per workgroup
  constexpr int WROWS = 32 * NRB;   // query positions per wavefront
  constexpr int KS = D / 16;        // k-steps of QK^T
  constexpr int MB = D / 32;        // 32-feature blocks of O^T
  constexpr int KSTR = D + 8;       // LDS row stride of key tiles (elements)
  static_assert(NW % HPW == 0, "each wavefront owns one query head");

  __shared__ __attribute__((aligned(16))) uint16_t sKr[2][kBN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sKl[2][kBN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * kVSTR];

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
  const int pb = w / HPW;
  const int h = hkv * p.ratio + grp * HPW + hs;
  const int r32 = lane & 31;
  const int g = lane >> 5;
  int qi[NRB];
  bool qvalid[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    qi[rb] = i0 + pb * WROWS + rb * 32 + r32;
    qvalid[rb] = qi[rb] <= i1;
  }

  // ---- query fragments rotated at f(p); the local ones are built after the
  // all-remote tiles so that they do not occupy registers during them
  f16x8 qrf[NRB][KS], qlf[NRB][KS];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int pl = qvalid[rb] ? qi[rb] : 0;
    const uint16_t* qsrc = p.q + (static_cast<int64_t>(qbeg + (qvalid[rb] ? qi[rb] - q_off : 0)) * p.Hq + h) * D;
    float x[KS][8];
    load_query<D>(x, qsrc, qvalid[rb], g);
    rotate_query<D>(qrf[rb], x, p.tab, rot_row(pl / G, pl, p.prerot), g, p.scale_log2);
  }

  const uint16_t* kr_base = p.kr + static_cast<int64_t>(hkv) * p.tpad * D;
  const uint16_t* kl_base = p.kl + static_cast<int64_t>(hkv) * p.tpad * D;
  const uint16_t* vt_base = p.vt + static_cast<int64_t>(hkv) * D * p.tpad;
  const TileSrc tsrc = tile_src<D, NT>(kr_base, kl_base, vt_base, p.tpad, tid);
  const int kr_off = r32 * KSTR + g * 8;
  const int v_off = r32 * kVSTR + g * 8;

  float m_run[NRB], l_run[NRB];  // running max (log2 domain, possibly stale by < 8), sum
  f32x16 acc[NRB][MB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[rb][mb] = f32x16{};
  }

  const int nkt = i1 / kBN + 1;
  // tiles [0, nrem) are all-remote; classes never return to remote later
  int nrem = 0;
  while (nrem < nkt && (classify_tile(i0, i1, nrem * kBN, min(L, nrem * kBN + kBN) - 1, p.w0) & 3) == kRemote) ++nrem;
  auto cls_of = [&](int kt) { return classify_tile(i0, i1, kt * kBN, min(L, kt * kBN + kBN) - 1, p.w0); };

  // a window pass starts at the first tile that holds a pair inside w0
  const int kt0 = BAND ? nrem : 0;
  TileRegs<D * kBN / 8 / NT> tr;
  int cls;
  if constexpr (BAND) {
    cls = 0;
    if (kt0 < nkt) {
      cls = cls_of(kt0);
      load_tile<D, NT>(tr, tsrc, tile_soff<D>(krow0 + static_cast<int64_t>(kt0) * kBN), cls);
      store_tile<D, NT>(tr, sKr[kt0 & 1], sKl[kt0 & 1], sV[kt0 & 1], cls, tsrc);
    }
  } else {
    cls = cls_of(0);
    load_tile<D, NT>(tr, tsrc, tile_soff<D>(krow0), cls);
    store_tile<D, NT>(tr, sKr[0], sKl[0], sV[0], cls, tsrc);
  }
  __syncthreads();

  // ---- all-remote tiles: remote query only.  The inner loop is the fast
  // path; a tile it declines (first tile, a large max increase, a masked
  // tile) is redone by the slow path, which then re-enters the fast loop.
  // The next tile's global loads are issued at the top of every iteration,
  // before the current tile is computed, and stored to LDS after it.
  int kt = kt0;
  int ncls = 0;
  while (!BAND && kt < nrem) {
    // fast loop over tiles whose successor is all-remote as well
    bool in_flight = false;  // loads of tile kt + 1 already issued
    for (; kt + 1 < nrem; ++kt) {
      const int buf = kt & 1;
      load_tile_c<D, NT, kRemote>(tr, tsrc, tile_soff<D>(krow0 + static_cast<int64_t>(kt + 1) * kBN));
      in_flight = true;
      if ((cls & kDiag) || kt * kBN + kBN > L) break;
      if (!tile_fast<D, NRB>(sKr[buf] + kr_off, sV[buf] + v_off, qrf, acc, m_run, l_run)) break;
      store_tile_c<D, NT, kRemote>(tr, sKr[buf ^ 1], sKl[buf ^ 1], sV[buf ^ 1], tsrc);
      in_flight = false;
      __syncthreads();
      cls = cls_of(kt + 1);
    }
    // tile kt: one the fast path declined or that needs a mask (the loads of
    // tile kt + 1 are in flight), or the last all-remote tile
    const int buf = kt & 1;
    ncls = kt + 1 < nkt ? cls_of(kt + 1) : 0;
    const bool masked = (cls & kDiag) || kt * kBN + kBN > L;
    bool done = false;
    if (!in_flight) {
      if (kt + 1 < nkt)
        load_tile<D, NT>(tr, tsrc, tile_soff<D>(krow0 + static_cast<int64_t>(kt + 1) * kBN), ncls);
      if (!masked) done = tile_fast<D, NRB>(sKr[buf] + kr_off, sV[buf] + v_off, qrf, acc, m_run, l_run);
    }
    if (!done) {
      const int j0g = kt * kBN + g * 4;
      if (masked)
        tile_slow<D, NRB, true, false, true>(sKr[buf] + kr_off, sKl[buf] + kr_off, sV[buf] + v_off, qrf, qlf, acc,
                                             m_run, l_run, qi, j0g, L, p.w0);
      else
        tile_slow<D, NRB, true, false, false>(sKr[buf] + kr_off, sKl[buf] + kr_off, sV[buf] + v_off, qrf, qlf, acc,
                                              m_run, l_run, qi, j0g, L, p.w0);
    }
    if (kt + 1 < nkt) store_tile<D, NT>(tr, sKr[buf ^ 1], sKl[buf ^ 1], sV[buf ^ 1], ncls, tsrc);
    __syncthreads();
    cls = ncls;
    ++kt;
  }

  // ---- window-edge and local tiles: the local query joins (slow path)
  if (nrem < nkt) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int pl = qvalid[rb] ? qi[rb] : 0;
      const uint16_t* qsrc = p.q + (static_cast<int64_t>(qbeg + (qvalid[rb] ? qi[rb] - q_off : 0)) * p.Hq + h) * D;
      float x[KS][8];
      load_query<D>(x, qsrc, qvalid[rb], g);
      const int pa = BAND && p.band_remote ? pl / G : pl;
      rotate_query<D>(qlf[rb], x, p.tab, rot_row(pa, pl, p.prerot), g, p.scale_log2);
    }
    // window-edge tiles need both logit sets
    int nloc = nrem;
    while (nloc < nkt && (cls_of(nloc) & 3) != kLocal) ++nloc;
    for (kt = nrem; kt < nloc; ++kt) {
      const int buf = kt & 1;
      ncls = 0;
      if (kt + 1 < nkt) {
        ncls = cls_of(kt + 1);
        load_tile<D, NT>(tr, tsrc, tile_soff<D>(krow0 + static_cast<int64_t>(kt + 1) * kBN), ncls);
      }
      const int j0g = kt * kBN + g * 4;
      const uint16_t* krl = sKr[buf] + kr_off;
      const uint16_t* kll = sKl[buf] + kr_off;
      const uint16_t* vl = sV[buf] + v_off;
      if constexpr (BAND) {
        if ((cls & kDiag) || kt * kBN + kBN > L)
          tile_slow<D, NRB, false, true, true, kPairsWindow>(krl, kll, vl, qrf, qlf, acc, m_run, l_run, qi, j0g, L,
                                                             p.w0);
        else
          tile_slow<D, NRB, false, true, false, kPairsWindow>(krl, kll, vl, qrf, qlf, acc, m_run, l_run, qi, j0g, L,
                                                              p.w0);
      } else {
        if ((cls & kDiag) || kt * kBN + kBN > L)
          tile_slow<D, NRB, true, true, true>(krl, kll, vl, qrf, qlf, acc, m_run, l_run, qi, j0g, L, p.w0);
        else
          tile_slow<D, NRB, true, true, false>(krl, kll, vl, qrf, qlf, acc, m_run, l_run, qi, j0g, L, p.w0);
      }
      if (kt + 1 < nkt) store_tile<D, NT>(tr, sKr[buf ^ 1], sKl[buf ^ 1], sV[buf ^ 1], ncls, tsrc);
      __syncthreads();
      cls = ncls;
    }
    // all-local tiles: one rotation again, so the fast path as for the
    // remote tiles (only the local query is live from here on)
    while (kt < nkt) {
      bool in_flight = false;
      for (; kt + 1 < nkt; ++kt) {
        const int buf = kt & 1;
        load_tile_c<D, NT, kLocal>(tr, tsrc, tile_soff<D>(krow0 + static_cast<int64_t>(kt + 1) * kBN));
        in_flight = true;
        if ((cls & kDiag) || kt * kBN + kBN > L) break;
        if (!tile_fast<D, NRB>(sKl[buf] + kr_off, sV[buf] + v_off, qlf, acc, m_run, l_run)) break;
        store_tile_c<D, NT, kLocal>(tr, sKr[buf ^ 1], sKl[buf ^ 1], sV[buf ^ 1], tsrc);
        in_flight = false;
        __syncthreads();
        cls = cls_of(kt + 1);
      }
      const int buf = kt & 1;
      ncls = kt + 1 < nkt ? cls_of(kt + 1) : 0;
      const bool masked = (cls & kDiag) || kt * kBN + kBN > L;
      bool done = false;
      if (!in_flight && !masked) done = tile_fast<D, NRB>(sKl[buf] + kr_off, sV[buf] + v_off, qlf, acc, m_run, l_run);
      if (!done) {
        const int j0g = kt * kBN + g * 4;
        if (masked)
          tile_slow<D, NRB, false, true, true, BAND ? kPairsWindow : kPairsAll>(
              sKr[buf] + kr_off, sKl[buf] + kr_off, sV[buf] + v_off, qrf, qlf, acc, m_run, l_run, qi, j0g, L, p.w0);
        else
          tile_slow<D, NRB, false, true, false, BAND ? kPairsWindow : kPairsAll>(
              sKr[buf] + kr_off, sKl[buf] + kr_off, sV[buf] + v_off, qrf, qlf, acc, m_run, l_run, qi, j0g, L, p.w0);
      }
      if (kt + 1 < nkt) store_tile_c<D, NT, kLocal>(tr, sKr[buf ^ 1], sKl[buf ^ 1], sV[buf ^ 1], tsrc);
      __syncthreads();
      cls = ncls;
      ++kt;
    }
  }

  // ---- epilogue: lane holds query qi[rb], features mb*32 + (r/4)*8 + g*4 + r%4
  if constexpr (MODE != kModeBifocal) {
    // merge pass: fp32 rows; a window pass with w0 = 0 holds no pair at all
    // (O = 0, LSE = -inf)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      if (!qvalid[rb]) continue;
      const bool empty = !(l_run[rb] > 0.f);
      const float inv = empty ? 0.f : 1.f / l_run[rb];
      const int64_t tok = qbeg + qi[rb] - q_off;
      float* dst = p.o32 + (tok * p.Hq + h) * D;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<float4*>(dst + mb * 32 + q4 * 8 + g * 4) =
              make_float4(acc[rb][mb][q4 * 4 + 0] * inv, acc[rb][mb][q4 * 4 + 1] * inv,
                          acc[rb][mb][q4 * 4 + 2] * inv, acc[rb][mb][q4 * 4 + 3] * inv);
      if (g == 0)
        p.lse[static_cast<int64_t>(h) * p.total_q + tok] = empty ? -INFINITY : (m_run[rb] + log2f(l_run[rb])) * kLn2;
    }
    return;
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    if (!qvalid[rb]) continue;
    const float inv = 1.f / l_run[rb];
    const int64_t tok = qbeg + qi[rb] - q_off;
    uint16_t* dst = p.o + (tok * p.Hq + h) * D;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = mb * 32 + q4 * 8 + g * 4;
        const uint32_t w0v = pack_bf16x2(acc[rb][mb][q4 * 4 + 0] * inv, acc[rb][mb][q4 * 4 + 1] * inv);
        const uint32_t w1v = pack_bf16x2(acc[rb][mb][q4 * 4 + 2] * inv, acc[rb][mb][q4 * 4 + 3] * inv);
        // non-temporal: O (1 GiB at 128K) is written once and larger than
        // any cache; left dirty in the caches it is written back in the
        // middle of whatever kernel runs next
        __builtin_nontemporal_store(u32x2{w0v, w1v}, reinterpret_cast<u32x2*>(dst + d));
      }
    if (p.lse && g == 0) p.lse[static_cast<int64_t>(h) * p.total_q + tok] = (m_run[rb] + log2f(l_run[rb])) * kLn2;
  }
}

int heads_per_wg(int ratio) { return ratio % 4 == 0 ? 4 : (ratio % 2 == 0 ? 2 : 1); }

// Row blocks per wavefront of the attention kernel (1: 8 waves of 32 rows;
// 2: 4 waves of 64 rows).
constexpr int kNRB = JL_PREFILL_NRB;

template <int D, int HPW, int MODE>
hipError_t launch_attn(const Params& prm, int nqb, hipStream_t s) {
  const int units = prm.B * prm.Hkv * prm.ngroups;
  const int64_t blocks = static_cast<int64_t>(nqb) * units;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_kernel<D, HPW, kNRB, MODE>), dim3(static_cast<unsigned>(blocks)), dim3(64 * 8 / kNRB), 0,
                     s, prm);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_attn_mode(const Params& p, int D, hipStream_t s) {
  const int hpw = heads_per_wg(p.ratio);
  if (D == 128) {
    if (hpw == 4) return launch_attn<128, 4, MODE>(p, p.nqb, s);
    if (hpw == 2) return launch_attn<128, 2, MODE>(p, p.nqb, s);
    return launch_attn<128, 1, MODE>(p, p.nqb, s);
  }
  if (hpw == 4) return launch_attn<64, 4, MODE>(p, p.nqb, s);
  if (hpw == 2) return launch_attn<64, 2, MODE>(p, p.nqb, s);
  return launch_attn<64, 1, MODE>(p, p.nqb, s);
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

static Params make_params(const PrefillCall& c) {
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
  p.prerot = c.prerot ? 1 : 0;
  return p;
}

hipError_t launch_prefill_bf16_prepare(const PrefillCall& c, hipStream_t s) {
  if (c.B == 0 || c.total_k == 0) return hipSuccess;
  const Params p = make_params(c);
  hipError_t e = launch_rope_table(static_cast<float2*>(c.ws), c.max_k, c.D, c.theta, s);
  if (e != hipSuccess) return e;
  const dim3 pg(static_cast<unsigned>((p.tpad + 63) / 64), c.Hkv);
  if (c.D == 128) hipLaunchKernelGGL(prep_kernel<128>, pg, dim3(4 * 128), 0, s, p);
  else hipLaunchKernelGGL(prep_kernel<64>, pg, dim3(4 * 64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16_attend(const PrefillCall& c, hipStream_t s) {
  if (c.total_q == 0 || c.B == 0) return hipSuccess;
  return launch_attn_mode<kModeBifocal>(make_params(c), c.D, s);
}

hipError_t launch_prefill_bf16_ie_pass(const PrefillCall& c, int pass, float* o, float* lse, hipStream_t s) {
  if (c.total_q == 0 || c.B == 0) return hipSuccess;
  Params p = make_params(c);
  p.o32 = o;
  p.lse = lse;
  if (pass == kIeFullRemote) {
    p.w0 = 0;
    return launch_attn_mode<kModeFull>(p, c.D, s);
  }
  if (pass == kIeWindowRemote) {
    p.band_remote = 1;
    p.kl = p.kr;
  }
  return launch_attn_mode<kModeWindow>(p, c.D, s);
}

}  // namespace jl
