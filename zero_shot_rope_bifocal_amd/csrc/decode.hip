// Split-K decode of dynamic bifocal RoPE attention on gfx950.
//
// "Jet-Long: Efficient Long-Context Extension with Dynamic Bifocal RoPE",
// section "Inference Efficiency Mechanisms": the KV cache holds the base keys
// at their exact absolute positions and is never rewritten; the rotation the
// bifocal scoring needs is applied on the fly to the active query and to each
// key as it is read, in registers.  Section "Dynamic Bifocal RoPE": a key
// closer to the query than w0 is scored with classic RoPE, every other key
// with RoPE at f(x) = floor(x / G), G from the current length L (eq. G, f).
//
// Kernel 1 (split).  bf16: grid (sequence x KV-head group, splits), 8
// wavefronts per workgroup; the workgroup owns one key range of one sequence
// for up to 8 KV heads (one wavefront per head when Hkv >= 8), so each 2 KB
// cache row is one contiguous read and all waves share cos/sin rows.  Each
// wavefront streams 32-key blocks and keeps its own online-softmax state for
// all query heads of its GQA group; every cache byte is read once.
//   * a lane loads 4 x 16 bytes of one key in the A-operand layout of
//     v_mfma_f32_16x16x32_f16 (rotate-half partners in the same lane),
//     rotates them at the key's own angle (j if local, f(j) if remote) from
//     the fp32 cos/sin table, and Q K^T for the whole head group is one chain
//     of D/32 MFMAs per 16 keys (rotated operands in IEEE half: 11
//     significant bits, bf16 inputs convert exactly; fp32 accumulation);
//   * the V block is staged row-major in the wavefront's own LDS slice and
//     read back with transposing LDS reads as the B operand of
//     v_mfma_f32_16x16x32_bf16; the probabilities stay in the registers Q K^T
//     left them in (that is already the A-operand layout), split into a bf16
//     high and low part so that P V keeps ~16 bits of P on exact bf16 V.
//   fp32: the same stream with the products on the VALU (4 wavefronts).
// Kernel 2 (combine): log-sum-exp merge of the per-wavefront partials.
#include "jl_device.hpp"
#include "jl_launch.hpp"

namespace jl {

namespace {

constexpr int kWaves = 8;  // bf16 split kernel: one workgroup = 8 wavefronts
constexpr int kWavesF32 = 4;
constexpr int kBlk = 16;  // keys per wavefront step

struct Params {
  const void* q;
  const void* kc;
  const void* vc;
  int64_t sb, ss, sh;
  float* part;  // [B][Hq][nsplit][slots][D + 2]  (O unnormalised, m (log2), l)
  const int32_t* seq_L;
  const float2* tab;
  const _Float16* tab16;  // the same rows in half, (cos, cos, sin, sin) per frequency pair
  int B, Hq, Hkv, ratio, nsplit, kps, max_L;
  int wph;    // wavefronts per KV head in a workgroup (bf16 split kernel)
  int slots;  // partial states per (sequence, head, split)
  int w_pretrained, w0;
  float scale_log2;
  int prerot;  // q and the key cache arrive rotated at their true positions
};

template <int D>
__device__ __forceinline__ float* part_ptr(const Params& p, int b, int h, int split, int w) {
  return p.part + ((((static_cast<int64_t>(b) * p.Hq + h) * p.nsplit + split) * p.slots + w) * (D + 2));
}

// ---------------------------------------------------------------- bf16

// Key-block of the bf16 split kernel: 16 keys per wavefront step.
constexpr int kKB = 16;

// XOR swizzle of the 16-byte chunks of V-block row `key` (D/8 chunks per
// row): the transposing read of 32 lanes covers 8 rows x 32 bytes, and the
// swizzle places those 8 pieces on 8 different 32-byte bank slots of the
// 256-byte bank space (D = 128: one row spans all of it; D = 64: rows of one
// parity share half of it).
template <int D>
__device__ __forceinline__ int vswz(int key) {
  if constexpr (D == 128) return (key & 7) * 2;
  else return ((key >> 1) & 3) * 2;
}

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): within each 16-lane
// group, element j of lane i's result is element i % 4 of the 8 bytes
// addressed by lane 4*j + i/4 of that group.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) const void*)p));
}

// 16 bytes per lane from global memory straight into LDS (gfx950
// global_load_lds_dwordx4): lane l writes lds_base + 16*l; lds_base must be
// the same in every lane.  Counted by vmcnt like any other load.
__device__ __forceinline__ void load_lds16(const void* gsrc, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(gsrc),
                                   (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 0);
#endif
}

// Maximum of v over the lanes l, l ^ 16 (v_permlane16_swap: rows of 16
// lanes trade places) and over l, l ^ 32 (v_permlane32_swap), on the VALU.
__device__ __forceinline__ float xrow16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xrow32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xrow_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Loop-invariant state of one wavefront of the bf16 split kernel.
template <int D>
struct SplitCtx {
  const uint16_t* kc;  // this (sequence, KV head)'s key rows
  const uint16_t* vc;
  const float2* tab;
  const _Float16* tab16;
  const uint16_t* klane;     // kc + col*ss + g*8: this lane's K piece of block row 0
  const uint16_t* vlane[2];  // vc + (lane/CPR)*ss + swizzled chunk, for (t*RPI) % 8 = 0 / 4
  const f16x8* ql;     // LDS: query fragments rotated at qpos, [t][g][head]
  uint16_t* vblk;      // LDS: this wave's V block
  int64_t ss;
  int qpos, kend, w0, G, col, g, lane, qcol, nr;
  float invG;
  int tr_addr[D / 16];  // transposed-read LDS element offsets per 16-feature block
};

// Running state: O block nb in lane (col, g) holds feature nb*16 + col of
// heads g*4 + rr; m (log2 domain) of head `col`, and the part of its l from
// the keys of lane group g (summed over g after the last block).
template <int D>
struct SplitState {
  f32x4 o[D / 16];
  float m, l;
};

// One 16-key block starting at j0 (wave-uniform).  q0 = j0 / G, r0 = j0 % G.
// TAIL: the block may run past kend; rows are clamped to kend-1 and their
// probabilities are zero.
template <int D, int NR, bool TAIL, bool PR>
__device__ __forceinline__ void split_block(const SplitCtx<D>& c, const f16x8 (&qrf)[D / 32],
                                            SplitState<D>& st, int j0, int q0, int r0) {
  constexpr int NT = D / 32;
  constexpr int HT = NT / 2;
  constexpr int H = D / 2;
  constexpr int NB = D / 16;
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;  // V rows per LDS-load instruction
  const int col = c.col, g = c.g;

  // ---- K in the A layout (lane = key j0 + col, features t*32 + g*8 ..) and
  // the V block (row-major, chunk-swizzled) straight into LDS
  const int jk = j0 + col;
  const int jkr = TAIL ? min(jk, c.kend - 1) : jk;
  // non-tail addresses: a per-lane base plus the wave-uniform row offset
  const uint16_t* krow = TAIL ? c.kc + jkr * c.ss + g * 8 : c.klane + j0 * c.ss;
  uint4 kr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) kr[t] = *reinterpret_cast<const uint4*>(krow + t * 32);
#pragma unroll
  for (int t = 0; t < kKB / RPI; ++t) {
    const uint16_t* src;
    if constexpr (TAIL) {
      const int key = t * RPI + c.lane / CPR;
      const int jv = min(j0 + key, c.kend - 1);
      src = c.vc + jv * c.ss + ((c.lane % CPR) ^ vswz<D>(key)) * 8;
    } else {
      src = c.vlane[(t * RPI / 4) & 1] + (j0 + t * RPI) * c.ss;
    }
    load_lds16(src, c.vblk + t * 512);
  }

  // ---- rotate each key at its own angle: j if within w0 of the query,
  // else f(j) = j / G = q0 + (r0 + col) / G.  The small quotient is exact in
  // fp32: (n + 1/2) / G lies at least 1/(2G) from an integer and the product
  // with the rounded reciprocal errs by under (G + 16) 2^-23 / G.  Rows past
  // kend (tail only) read table row 0.
  // PR (pre-rotated cache): local keys are used as stored (row 0: cos 1,
  // sin 0) and remote keys get R(f(j) - j), i.e. row j - f(j) with sin negated
  const bool klocal = c.qpos - jk < c.w0;
  int kpos;
  if constexpr (TAIL) {
    const int fj = jk / c.G;
    kpos = jk < c.kend ? (klocal ? (PR ? 0 : jk) : (PR ? jk - fj : fj)) : 0;
  } else {
    const int frem = c.G < (1 << 20) ? q0 + static_cast<int>((static_cast<float>(r0 + col) + 0.5f) * c.invG)
                                     : jk / c.G;
    kpos = klocal ? (PR ? 0 : jk) : (PR ? jk - frem : frem);
  }
  const float ksgn = PR && !klocal ? -1.f : 1.f;
  // rotation in packed half: the bf16 key converts to half exactly, the half
  // cos/sin carry at most 2^-12 absolute error, and the result is rounded to
  // half for the MFMA either way
  f16x8 a[NT];
  const uint4* cs8 = reinterpret_cast<const uint4*>(c.tab16 + (static_cast<int64_t>(kpos) * (H / 2) + g * 4) * 4);
  const f16x2 sgn2 = {static_cast<_Float16>(ksgn), static_cast<_Float16>(ksgn)};
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    const uint4 ca = cs8[t * 8], cb = cs8[t * 8 + 1];  // frequency pairs e2 = 0, 1 and 2, 3
    const uint32_t cw[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const f16x2 cc = __builtin_bit_cast(f16x2, cw[2 * e2]);
      f16x2 sn = __builtin_bit_cast(f16x2, cw[2 * e2 + 1]);
      if constexpr (PR) sn = sn * sgn2;
      const uint32_t u1[4] = {kr[t].x, kr[t].y, kr[t].z, kr[t].w};
      const uint32_t u2[4] = {kr[t + HT].x, kr[t + HT].y, kr[t + HT].z, kr[t + HT].w};
      const uint32_t w1 = u1[e2], w2 = u2[e2];
      const f16x2 x1 = {static_cast<_Float16>(__uint_as_float(w1 << 16)), static_cast<_Float16>(__uint_as_float(w1 & 0xffff0000u))};
      const f16x2 x2 = {static_cast<_Float16>(__uint_as_float(w2 << 16)), static_cast<_Float16>(__uint_as_float(w2 & 0xffff0000u))};
      const f16x2 o1 = x1 * cc - x2 * sn;
      const f16x2 o2 = x2 * cc + x1 * sn;
      a[t][2 * e2] = o1[0];
      a[t][2 * e2 + 1] = o1[1];
      a[t + HT][2 * e2] = o2[0];
      a[t + HT][2 * e2 + 1] = o2[1];
    }
  }

  // ---- S = K_rot Q_sel^T: lane (col = head, g) holds keys j0 + g*4 + rr
  const bool all_remote = c.qpos - (j0 + kKB - 1) >= c.w0;
  const bool all_local = c.qpos - j0 < c.w0;
  f32x4 sr = {0.f, 0.f, 0.f, 0.f}, sl = {0.f, 0.f, 0.f, 0.f};
  if (!all_local) {
#pragma unroll
    for (int t = 0; t < NT; ++t) sr = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], qrf[t], sr, 0, 0, 0);
  }
  if (!all_remote) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      sl = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], c.ql[(t * 4 + g) * NR + c.qcol], sl, 0, 0, 0);
  }
  // one logit set per key: outside the window edge the other set was not
  // formed and is zero
  float sv[4];
  if (all_remote || all_local) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) sv[rr] = sr[rr] + sl[rr];
  } else {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) sv[rr] = c.qpos - (j0 + g * 4 + rr) < c.w0 ? sl[rr] : sr[rr];
  }
  if constexpr (TAIL) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      if (j0 + g * 4 + rr >= c.kend) sv[rr] = -INFINITY;
  }

  // ---- online softmax with a lazy maximum: m only moves when a score
  // exceeds it by more than 2^8 (so exp2(s - m) <= 256); O and l are
  // rescaled then, on a wave-uniform branch.  Each lane checks its own four
  // scores; the head's maximum over the block (lanes col, col + 16, + 32,
  // + 48) is formed only on that branch.
  const float lmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  if (__any(lmax > st.m + 8.f)) {
    const float bmax = xrow32_max(xrow16_max(lmax));
    const bool grow = bmax > st.m + 8.f;
    const float m_new = grow ? bmax : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
    st.m = m_new;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float ar;
      if constexpr (NR <= 4) ar = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), rr));
      else ar = __shfl(alpha, g * 4 + rr);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) st.o[nb][rr] *= ar;
    }
  }
  float pv[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) pv[rr] = __builtin_amdgcn_exp2f(sv[rr] - st.m);
  st.l += (pv[0] + pv[1]) + (pv[2] + pv[3]);  // this lane's keys; the head's sum is formed at the end
  // P as a bf16 high part plus a bf16 low part: on exact bf16 V the product
  // keeps ~16 bits of P
  const uint32_t h01 = pack_bf16x2(pv[0], pv[1]), h23 = pack_bf16x2(pv[2], pv[3]);
  const uint32_t l01 = pack_bf16x2(pv[0] - __uint_as_float(h01 << 16), pv[1] - __uint_as_float(h01 & 0xffff0000u));
  const uint32_t l23 = pack_bf16x2(pv[2] - __uint_as_float(h23 << 16), pv[3] - __uint_as_float(h23 & 0xffff0000u));
  const i16x4 phi = __builtin_bit_cast(i16x4, make_uint2(h01, h23));
  const i16x4 plo = __builtin_bit_cast(i16x4, make_uint2(l01, l23));

  // ---- O += P V on MFMA (v_mfma_f32_16x16x16_bf16): A = P (head x 16
  // keys; lane (col, g) holds keys g*4 .. g*4+3 of head col, exactly where
  // Q K^T left them), B = V (16 keys x 16 features) from one transposing
  // LDS read
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const i16x4 bv = lds_read_tr16(c.vblk + c.tr_addr[nb]);
    st.o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, bv, st.o[nb], 0, 0, 0);
    st.o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, bv, st.o[nb], 0, 0, 0);
  }
}

template <int D, int NR, bool PR>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void split_bf16_kernel(Params p) {
  constexpr int NT = D / 32;    // QK^T MFMAs per 16 keys (32 features each)
  constexpr int HT = NT / 2;    // first-half feature groups
  constexpr int H = D / 2;
  constexpr int NB = D / 16;    // PV MFMAs per 16 keys (16 features each)
  static_assert(NR <= 16, "one MFMA column per query head");
  __shared__ __attribute__((aligned(16))) uint16_t sV[kWaves][kKB * D];  // per-wave V block
  // B fragments of the query heads rotated at qpos (needed only by key
  // blocks that reach into the local window): [wave][t][g][head]
  __shared__ f16x8 sQl[kWaves][NT * 4 * NR];

  // one workgroup = one key range of one sequence for `hw` KV heads, `wph`
  // wavefronts per head: with 8 KV heads every wave streams its own 256-byte
  // slice of the same 2 KB cache rows, and all waves read the same cos/sin rows
  const int hw = kWaves / p.wph;
  const int hgrp = blockIdx.x % (p.Hkv / hw);
  const int b = blockIdx.x / (p.Hkv / hw);
  const int split = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hkv = hgrp * hw + wid / p.wph;
  const int w = wid % p.wph;  // this wave's slot among the waves of its head
  const int L = p.seq_L[b];
  if (L < 1 || L > p.max_L) return;  // outside the documented contract: left unwritten
  const int G = group_size(L, p.w_pretrained);
  const int qpos = L - 1;
  const int kbeg = split * p.kps;
  const int kend = min(L, kbeg + p.kps);

  SplitCtx<D> c;
  c.col = lane & 15;  // QK: B column = query head slot, A row = key; PV: feature in block
  c.g = lane >> 4;    // 16-lane group: QK feature group / PV key group
  c.lane = lane;
  c.kc = static_cast<const uint16_t*>(p.kc) + b * p.sb + hkv * p.sh;
  c.vc = static_cast<const uint16_t*>(p.vc) + b * p.sb + hkv * p.sh;
  c.tab = p.tab;
  c.tab16 = p.tab16;
  c.ql = sQl[wid];
  c.vblk = sV[wid];
  c.ss = p.ss;
  c.qpos = qpos;
  c.kend = kend;
  c.w0 = p.w0;
  c.G = G;
  c.invG = 1.f / static_cast<float>(G);
  c.qcol = min(c.col, NR - 1);  // columns >= NR compute unused heads
  c.klane = c.kc + c.col * p.ss + c.g * 8;
  {
    // the chunk swizzle depends on the block row modulo 8 only
    constexpr int CPR = D / 8;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int key = x * 4 + lane / CPR;
      c.vlane[x] = c.vc + (lane / CPR) * p.ss + ((lane % CPR) ^ vswz<D>(key)) * 8;
    }
  }
  const int col = c.col, g = c.g;

  // query fragments for all heads of the group, rotated at qpos and f(qpos),
  // with the softmax scale (log2 domain) folded in
  f16x8 qrf[NT];
  {
    float x[NT][8];
    if (col < p.ratio) {
      const uint16_t* src = static_cast<const uint16_t*>(p.q) +
                            (static_cast<int64_t>(b) * p.Hq + hkv * p.ratio + col) * D;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint4 u = *reinterpret_cast<const uint4*>(src + t * 32 + g * 8);
        const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[t][e] = bf16_bits_to_float(static_cast<uint16_t>(uu[e >> 1] >> (16 * (e & 1))));
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[t][e] = 0.f;
    }
    const RotRow rl = rot_row(qpos, qpos, PR);
    const RotRow rr = rot_row(qpos / G, qpos, PR);
    const float sc = p.scale_log2;
    f16x8 ql[NT];
#pragma unroll
    for (int t = 0; t < HT; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = t * 32 + g * 8 + e;
        float2 cl = p.tab[static_cast<int64_t>(rl.row) * H + kk];
        float2 cr = p.tab[static_cast<int64_t>(rr.row) * H + kk];
        cl.y *= rl.sgn;
        cr.y *= rr.sgn;
        const float x1 = x[t][e], x2 = x[t + HT][e];
        ql[t][e] = static_cast<_Float16>((x1 * cl.x - x2 * cl.y) * sc);
        ql[t + HT][e] = static_cast<_Float16>((x2 * cl.x + x1 * cl.y) * sc);
        qrf[t][e] = static_cast<_Float16>((x1 * cr.x - x2 * cr.y) * sc);
        qrf[t + HT][e] = static_cast<_Float16>((x2 * cr.x + x1 * cr.y) * sc);
      }
    if (col < NR) {
#pragma unroll
      for (int t = 0; t < NT; ++t) sQl[wid][(t * 4 + g) * NR + col] = ql[t];
    }
  }

  // transposed-read address of lane (g, col): the 4 features nb*16 +
  // 4*(col%4) .. of key g*4 + col/4; 16-byte chunk ch of a row sits at
  // position ch ^ vswz(row)
  {
    const int tr_row = g * 4 + (col >> 2);
    const int tr_half = (col & 1) * 4;
    const int tr_c = (col >> 1) & 1;
    const int tr_x = vswz<D>(tr_row);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) c.tr_addr[nb] = tr_row * D + ((nb * 2 + tr_c) ^ tr_x) * 8 + tr_half;
  }

  SplitState<D> st;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) st.o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;

  // blocks j0 = kbeg + w*16 + n*step; j0 / G tracked as quotient + remainder
  const int step = p.wph * kKB;
  const int qs = step / G, rs = step % G;
  int j0 = kbeg + w * kKB;
  int q0 = j0 / G, r0 = j0 % G;
  for (; j0 + kKB <= kend; j0 += step) {
    split_block<D, NR, false, PR>(c, qrf, st, j0, q0, r0);
    q0 += qs;
    r0 += rs;
    if (r0 >= G) { r0 -= G; ++q0; }
  }
  if (j0 < kend) split_block<D, NR, true, PR>(c, qrf, st, j0, q0, r0);

  st.l = xrow_sum(st.l);

  // ---- this wavefront's partial state: O feature nb*16 + col of head
  // g*4 + rr in register rr; m and l of head hh in lane hh
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int hh = g * 4 + rr;
    if (hh < p.ratio) {
      float* dst = part_ptr<D>(p, b, hkv * p.ratio + hh, split, w);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) dst[nb * 16 + col] = st.o[nb][rr];
    }
  }
  if (g == 0 && col < p.ratio) {
    float* dst = part_ptr<D>(p, b, hkv * p.ratio + col, split, w);
    dst[D] = st.m;
    dst[D + 1] = st.l;
  }
}

// ---------------------------------------------------------------- fp32

template <int D, int NR>
__global__ __launch_bounds__(kWavesF32 * 64) void split_f32_kernel(Params p) {
  constexpr int NT = D / 32;
  constexpr int HT = NT / 2;
  constexpr int H = D / 2;
  constexpr int EPL = D / 64;
  __shared__ float sQ[2][NR][D];  // [0] rotated at qpos, [1] at f(qpos)

  const int hkv = blockIdx.x % p.Hkv;
  const int b = blockIdx.x / p.Hkv;
  const int split = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int L = p.seq_L[b];
  if (L < 1 || L > p.max_L) return;  // outside the documented contract: left unwritten
  const int G = group_size(L, p.w_pretrained);
  const int qpos = L - 1;
  const int kbeg = split * p.kps;
  const int kend = min(L, kbeg + p.kps);
  const int col = lane & 15;
  const int g = lane >> 4;
  const float* kc = static_cast<const float*>(p.kc) + b * p.sb + hkv * p.sh;
  const float* vc = static_cast<const float*>(p.vc) + b * p.sb + hkv * p.sh;

  for (int idx = threadIdx.x; idx < NR * H; idx += kWavesF32 * 64) {
    const int hh = idx / H;
    const int kk = idx % H;
    const bool hv = hh < p.ratio;
    const float* src = static_cast<const float*>(p.q) + (static_cast<int64_t>(b) * p.Hq + hkv * p.ratio + (hv ? hh : 0)) * D;
    const float x1 = hv ? src[kk] : 0.f, x2 = hv ? src[kk + H] : 0.f;
    const RotRow rl = rot_row(qpos, qpos, p.prerot);
    const RotRow rr = rot_row(qpos / G, qpos, p.prerot);
    float2 cl = p.tab[static_cast<int64_t>(rl.row) * H + kk];
    float2 cr = p.tab[static_cast<int64_t>(rr.row) * H + kk];
    cl.y *= rl.sgn;
    cr.y *= rr.sgn;
    sQ[0][hh][kk] = x1 * cl.x - x2 * cl.y;
    sQ[0][hh][kk + H] = x2 * cl.x + x1 * cl.y;
    sQ[1][hh][kk] = x1 * cr.x - x2 * cr.y;
    sQ[1][hh][kk + H] = x2 * cr.x + x1 * cr.y;
  }
  __syncthreads();

  float m_run[NR], l_run[NR], oacc[NR][EPL];
#pragma unroll
  for (int hh = 0; hh < NR; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) oacc[hh][e] = 0.f;
  }

  for (int j0 = kbeg + w * kBlk; j0 < kend; j0 += kWavesF32 * kBlk) {
    const int jk = j0 + col;  // this lane's key
    const bool kval = jk < kend;
    const bool klocal = qpos - jk < p.w0;
    const RotRow kr_ = rot_row(klocal ? jk : jk / G, jk, p.prerot);
    const int kpos = kval ? kr_.row : 0;
    const float ksgn = kr_.sgn;
    float kv[NT][8];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) kv[t][e] = kval ? kc[jk * p.ss + t * 32 + g * 8 + e] : 0.f;
#pragma unroll
    for (int t = 0; t < HT; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 cs = p.tab[static_cast<int64_t>(kpos) * H + t * 32 + g * 8 + e];
        const float sn = cs.y * ksgn;
        const float x1 = kv[t][e], x2 = kv[t + HT][e];
        kv[t][e] = x1 * cs.x - x2 * sn;
        kv[t + HT][e] = x2 * cs.x + x1 * sn;
      }
    const float* qsel = klocal ? &sQ[0][0][0] : &sQ[1][0][0];
    float s[NR];
#pragma unroll
    for (int hh = 0; hh < NR; ++hh) {
      float part = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fmaf(kv[t][e], qsel[hh * D + t * 32 + g * 8 + e], part);
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      s[hh] = kval ? part * p.scale_log2 : -INFINITY;
    }
#pragma unroll
    for (int hh = 0; hh < NR; ++hh) {
      float bm = s[hh];
      bm = fmaxf(bm, __shfl_xor(bm, 1));
      bm = fmaxf(bm, __shfl_xor(bm, 2));
      bm = fmaxf(bm, __shfl_xor(bm, 4));
      bm = fmaxf(bm, __shfl_xor(bm, 8));
      const float m_new = fmaxf(m_run[hh], bm);
      const float alpha = exp2f(m_run[hh] - m_new);
      s[hh] = exp2f(s[hh] - m_new);
      float bs = s[hh];
      bs += __shfl_xor(bs, 1);
      bs += __shfl_xor(bs, 2);
      bs += __shfl_xor(bs, 4);
      bs += __shfl_xor(bs, 8);
      l_run[hh] = l_run[hh] * alpha + bs;
      m_run[hh] = m_new;
#pragma unroll
      for (int e = 0; e < EPL; ++e) oacc[hh][e] *= alpha;
    }
#pragma unroll
    for (int m = 0; m < kBlk; ++m) {
      const int jv = j0 + m;
      float vf[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) vf[e] = jv < kend ? vc[jv * p.ss + lane * EPL + e] : 0.f;
#pragma unroll
      for (int hh = 0; hh < NR; ++hh) {
        const float pm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s[hh]), m));
#pragma unroll
        for (int e = 0; e < EPL; ++e) oacc[hh][e] = fmaf(pm, vf[e], oacc[hh][e]);
      }
    }
  }

#pragma unroll
  for (int hh = 0; hh < NR; ++hh) {
    if (hh >= p.ratio) break;
    float* dst = part_ptr<D>(p, b, hkv * p.ratio + hh, split, w);
#pragma unroll
    for (int e = 0; e < EPL; ++e) dst[lane * EPL + e] = oacc[hh][e];
    if (lane == 0) {
      dst[D] = m_run[hh];
      dst[D + 1] = l_run[hh];
    }
  }
}

// ---------------------------------------------------------------- combine

// Log-sum-exp merge of the partial states of one (sequence, query head):
// weights 2^(m_s - M) are formed once, then each thread sums one feature
// over the partials (coalesced reads).
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(const float* __restrict__ part, int nparts, void* o,
                                                    float* lse, int bf16, const int32_t* __restrict__ seq_L,
                                                    int Hq, int max_L) {
  constexpr int kMaxParts = 1024;
  __shared__ float sw[kMaxParts];
  __shared__ float sred[D / 64];
  __shared__ float sM, sden;
  const int bh = blockIdx.x;  // b * Hq + h
  const int t = threadIdx.x;
  const int L = seq_L[bh / Hq];
  if (L < 1 || L > max_L) return;  // outside the documented contract: left unwritten, as in the split kernel
  const float* pp = part + static_cast<int64_t>(bh) * nparts * (D + 2);
  float mx = -INFINITY;
  for (int s = t; s < nparts; s += D) mx = fmaxf(mx, pp[s * (D + 2) + D]);
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((t & 63) == 0) sred[t >> 6] = mx;
  __syncthreads();
  if (t == 0) {
    float M = sred[0];
    for (int i = 1; i < D / 64; ++i) M = fmaxf(M, sred[i]);
    sM = M;
  }
  __syncthreads();
  const float M = sM;
  float den = 0.f;
  for (int s = t; s < nparts; s += D) {
    const float ms = pp[s * (D + 2) + D];
    const float wgt = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    sw[s] = wgt;
    den += wgt * pp[s * (D + 2) + D + 1];
  }
  for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
  __syncthreads();
  if ((t & 63) == 0) sred[t >> 6] = den;
  __syncthreads();
  if (t == 0) {
    float dd = 0.f;
    for (int i = 0; i < D / 64; ++i) dd += sred[i];
    sden = dd;
  }
  __syncthreads();
  float num = 0.f;
  for (int s = 0; s < nparts; ++s) num = fmaf(sw[s], pp[s * (D + 2) + t], num);
  const float r = num / sden;
  if (bf16) static_cast<uint16_t*>(o)[static_cast<int64_t>(bh) * D + t] = float_to_bf16_bits(r);
  else static_cast<float*>(o)[static_cast<int64_t>(bh) * D + t] = r;
  if (lse && t == 0) lse[bh] = (M + log2f(sden)) * kLn2;
}

template <int D, int NR>
void launch_split(const Params& p, bool bf16, hipStream_t s) {
  if (bf16) {
    const int hw = kWaves / p.wph;
    if (p.prerot)
      hipLaunchKernelGGL((split_bf16_kernel<D, NR, true>), dim3(p.B * (p.Hkv / hw), p.nsplit), dim3(kWaves * 64), 0, s, p);
    else
      hipLaunchKernelGGL((split_bf16_kernel<D, NR, false>), dim3(p.B * (p.Hkv / hw), p.nsplit), dim3(kWaves * 64), 0, s, p);
  } else {
    hipLaunchKernelGGL((split_f32_kernel<D, NR>), dim3(p.B * p.Hkv, p.nsplit), dim3(kWavesF32 * 64), 0, s, p);
  }
}

template <int D>
void launch_split_d(const Params& p, int ratio, bool bf16, hipStream_t s) {
  if (ratio <= 1) launch_split<D, 1>(p, bf16, s);
  else if (ratio <= 2) launch_split<D, 2>(p, bf16, s);
  else if (ratio <= 4) launch_split<D, 4>(p, bf16, s);
  else if (ratio <= 8) launch_split<D, 8>(p, bf16, s);
  else launch_split<D, 16>(p, bf16, s);
}

int keys_per_split(int max_L, int nsplit) {
  const int per = (max_L + nsplit - 1) / nsplit;
  return (per + 63) / 64 * 64;
}

}  // namespace

// Key-range splits per (sequence, KV head): about 16384 streaming
// wavefronts in all (four per slot at the split kernel's 4 waves per SIMD),
// each split at least 256 keys, and at most 128 splits (the combine merges up
// to 1024 partial states).
int decode_num_splits(int B, int max_L, int Hkv) {
  int hw = 1;
  while (hw < kWaves && Hkv % (hw * 2) == 0) hw *= 2;
  const int64_t waves = static_cast<int64_t>(B) * Hkv * (kWaves / hw);
  int64_t ns = (16384 + waves - 1) / waves;
  const int64_t cap = (static_cast<int64_t>(max_L) + 255) / 256;
  if (ns > cap) ns = cap;
  if (ns > 128) ns = 128;
  if (ns < 1) ns = 1;
  return static_cast<int>(ns);
}

size_t decode_ws_bytes(int B, int max_L, int Hq, int Hkv, int D) {
  const int ns = decode_num_splits(B, max_L, Hkv);
  const size_t tab = align_up(static_cast<size_t>(max_L) * (D / 2) * sizeof(float2), 256);
  const size_t tab16 = align_up(static_cast<size_t>(max_L) * D * sizeof(_Float16), 256);
  const size_t part = static_cast<size_t>(B) * Hq * ns * kWaves * (D + 2) * sizeof(float);  // slots <= kWaves
  return tab + tab16 + align_up(part, 256);
}

hipError_t launch_decode(const DecodeCall& c, bool bf16, hipStream_t s) {
  if (c.B == 0) return hipSuccess;
  const int ns = decode_num_splits(c.B, c.max_L, c.Hkv);
  char* ws = static_cast<char*>(c.ws);
  const size_t tab = align_up(static_cast<size_t>(c.max_L) * (c.D / 2) * sizeof(float2), 256);
  const size_t tab16 = align_up(static_cast<size_t>(c.max_L) * c.D * sizeof(_Float16), 256);
  uint16_t* t16 = reinterpret_cast<uint16_t*>(ws + tab);
  Params p{};
  p.q = c.q;
  p.kc = c.kc;
  p.vc = c.vc;
  p.sb = c.sb;
  p.ss = c.ss;
  p.sh = c.sh;
  p.part = reinterpret_cast<float*>(ws + tab + tab16);
  p.seq_L = c.seq_L;
  p.tab = reinterpret_cast<const float2*>(ws);
  p.tab16 = reinterpret_cast<const _Float16*>(t16);
  p.B = c.B;
  p.Hq = c.Hq;
  p.Hkv = c.Hkv;
  p.ratio = c.Hq / c.Hkv;
  p.nsplit = ns;
  p.kps = keys_per_split(c.max_L, ns);
  p.max_L = c.max_L;
  {
    int hw = 1;  // KV heads per bf16 workgroup: largest power of two dividing Hkv, at most 8
    while (hw < kWaves && c.Hkv % (hw * 2) == 0) hw *= 2;
    p.wph = kWaves / hw;
  }
  p.slots = bf16 ? p.wph : kWavesF32;
  p.w_pretrained = c.w_pretrained;
  p.w0 = c.w0;
  p.scale_log2 = c.scale * kLog2e;
  p.prerot = c.prerot ? 1 : 0;
  // rows a decode reads: remote positions (all below w_pretrained) and each
  // sequence's local window; a pre-rotated cache reads row 0 and the
  // correction rows j - f(j), which cover the whole range
  uint16_t* t16w = bf16 ? t16 : nullptr;  // the half rows feed the bf16 split kernel only
  hipError_t e = c.prerot ? launch_rope_table(reinterpret_cast<float2*>(ws), c.max_L, c.D, c.theta, s, t16w)
                          : launch_rope_table_rows(reinterpret_cast<float2*>(ws), c.max_L, c.D, c.theta, c.seq_L, c.B,
                                                   c.w0, c.w_pretrained, s, t16w);
  if (e != hipSuccess) return e;
  const int ratio = c.Hq / c.Hkv;
  if (c.D == 128) launch_split_d<128>(p, ratio, bf16, s);
  else launch_split_d<64>(p, ratio, bf16, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nparts = ns * p.slots;
  if (c.D == 128)
    hipLaunchKernelGGL(combine_kernel<128>, dim3(c.B * c.Hq), dim3(128), 0, s, p.part, nparts, c.o, c.lse, bf16 ? 1 : 0,
                       c.seq_L, c.Hq, c.max_L);
  else
    hipLaunchKernelGGL(combine_kernel<64>, dim3(c.B * c.Hq), dim3(64), 0, s, p.part, nparts, c.o, c.lse, bf16 ? 1 : 0,
                       c.seq_L, c.Hq, c.max_L);
  return hipGetLastError();
}

}  // namespace jl
