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
#include <algorithm>
#include <mutex>

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
  int plain;   // bf16, pre-rotated, every key inside the window (kKeyPlain)
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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load_lds16(const void* gsrc, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  // cache policy 2 = nt: the cache is streamed once per call (the K rows
  // are loaded non-temporal too), which measured ~2.4% faster than cached
  // loads at 16 x 128K
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(gsrc),
                                   (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 2);
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

// Blocks of one wavefront: j0 = kbeg + w*16 + n*step over its key range,
// with j0 / G tracked as a quotient q0 and remainder r0 (no integer division
// in the loop).  The debug export of the key rows walks the same blocks.
struct KeyBlocks {
  int j0, q0, r0, qs, rs, step, G;
  __device__ __forceinline__ KeyBlocks(int kbeg, int w, int wph, int G_) : G(G_) {
    step = wph * 16;
    qs = step / G;
    rs = step % G;
    j0 = kbeg + w * 16;
    q0 = j0 / G;
    r0 = j0 % G;
  }
  __device__ __forceinline__ void next() {
    j0 += step;
    q0 += qs;
    r0 += rs;
    if (r0 >= G) {
      r0 -= G;
      ++q0;
    }
  }
};

// Table row and sign of sin with which the bf16 split kernel rotates key
// jk = j0 + col (col < 16) of a block that starts at j0 = q0 * G + r0: j if the
// key is within w0 of the query at qpos, else f(j) = j / G (eq. f).  Outside
// the tail, f(j) = q0 + (r0 + col) / G with the small quotient taken in fp32:
// (n + 1/2) / G lies at least 1/(2G) from an integer and the product with the
// rounded reciprocal errs by under (G + 16) 2^-23 / G, so the truncation is
// exact for G < 2^20 (above, an integer division).  In a tail block
// (TAIL) keys at or past kend read row 0.  PR (pre-rotated cache): a local
// key is used as stored (row 0: cos 1, sin 0), a remote one gets the
// correction R(f(j) - j), i.e. row j - f(j) with sin negated.
template <bool PR, bool TAIL>
__device__ __forceinline__ RotRow split_key_rot(int jk, int col, int q0, int r0, int G, float invG, int qpos,
                                                int w0, int kend) {
  const bool klocal = qpos - jk < w0;
  int fj;
  if constexpr (TAIL) fj = jk / G;
  else fj = G < (1 << 20) ? q0 + static_cast<int>((static_cast<float>(r0 + col) + 0.5f) * invG) : jk / G;
  int row = klocal ? (PR ? 0 : jk) : (PR ? jk - fj : fj);
  if constexpr (TAIL) row = jk < kend ? row : 0;
  return RotRow{row, PR && !klocal ? -1.f : 1.f};
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
  int tr_base;  // transposed-read LDS element offset of 16-feature block 0 (block nb: tr_base ^ 16 nb)
};

// Running state: O block nb in lane (col, g) holds feature nb*16 + col of
// heads g*4 + rr; m (log2 domain) of head `col`, and the part of its l from
// the keys of lane group g (summed over g after the last block).
template <int D>
struct SplitState {
  f32x4 o[D / 16];
  float m, l;
  bool bad;  // some key of this lane's head scored -inf: an input outside half range
};

// How the bf16 split kernel treats the keys it streams.  kKeyRaw: raw keys,
// rotated at j or f(j) from the half cos/sin rows.  kKeyPre: a pre-rotated
// cache, local keys used as stored and remote keys corrected by R(f(j) - j).
// kKeyPlain: a pre-rotated cache with every key inside the window (w0 >=
// max_L), i.e. plain RoPE attention over a RoPE cache: no table, no key
// rotation, Q K^T straight from the stored bf16 keys on the bf16 MFMA.
enum : int { kKeyRaw = 0, kKeyPre = 1, kKeyPlain = 2 };

// The K rows of one full 16-key block in the A layout (lane = key j0 + col,
// features t*32 + g*8 ..).  The block walk issues the next block's K rows and
// V block (by DMA into the wave's other LDS buffer) while the current block
// is computed; the cos/sin rows (L2 hits) are loaded by each block itself.
template <int D>
struct BlockLoads {
  uint4 kr[D / 32];
};

// Issues the loads of the full block at j0 from HBM: V into vdst (the wave's
// LDS buffer for that block), then K, so that waiting for K waits for both.
template <int D>
__device__ __forceinline__ void issue_block_loads(const SplitCtx<D>& c, BlockLoads<D>& L, int j0, uint16_t* vdst) {
  constexpr int NT = D / 32;
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;  // V rows per LDS-load instruction
#pragma unroll
  for (int t = 0; t < kKB / RPI; ++t)
    load_lds16(c.vlane[(t * RPI / 4) & 1] + (j0 + t * RPI) * c.ss, vdst + t * 512);
  const uint16_t* krow = c.klane + j0 * c.ss;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(krow + t * 32));
    L.kr[t] = make_uint4(x[0], x[1], x[2], x[3]);
  }
}

// The transposing reads of a block's V (one per 16-feature block) in one
// asm statement that waits for them itself: the compiler would otherwise
// wait for every outstanding load into LDS (the next block's V) before each
// of them, since it cannot tell the wave's two V buffers apart.  The caller
// guarantees that this buffer's loads are complete (they were issued before
// the K loads the block already waited for).
__device__ __forceinline__ void lds_read_tr16_all(i16x4 (&o)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}
__device__ __forceinline__ void lds_read_tr16_all(i16x4 (&o)[4], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}

// One 16-key block starting at j0 (wave-uniform).  q0 = j0 / G, r0 = j0 % G.
// TAIL: the block may run past kend; rows are clamped to kend-1 and their
// probabilities are zero.
// PFM (prefetched, full blocks): the block's K rows arrived in L and its V
// block in vcur, both issued one block earlier, and only its cos/sin rows are
// loaded here; once its keys are consumed (after the rotation; after Q K^T
// for plain keys) the K rows and V block of the block at nj0 are issued into
// L and vnext when has_next.  Otherwise (the tail block) the block issues
// all its own loads and waits for them.
template <int D, int NR, bool TAIL, int KM, bool PFM = false>
__device__ __forceinline__ void split_block(const SplitCtx<D>& c, const f16x8 (&qrf)[D / 32],
                                            SplitState<D>& st, int j0, int q0, int r0,
                                            BlockLoads<D>* L = nullptr, uint16_t* vcur = nullptr,
                                            bool has_next = false, int nj0 = 0, int nq0 = 0, int nr0 = 0,
                                            uint16_t* vnext = nullptr) {
  constexpr int NT = D / 32;
  constexpr int HT = NT / 2;
  constexpr int H = D / 2;
  constexpr int NB = D / 16;
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;  // V rows per LDS-load instruction
  constexpr bool PR = KM == kKeyPre;
  const int col = c.col, g = c.g;

  // ---- loads of the block, all issued before the first wait: the cos/sin
  // rows of the keys' angles (they depend on j only), the V block
  // (row-major, chunk-swizzled) straight into LDS, and K in the A layout
  // (lane = key j0 + col, features t*32 + g*8 ..).  Loads into LDS and into
  // registers share one counter that the compiler cannot split, so the
  // first use of K waits for all of them: issued together, the block pays
  // one memory latency instead of one per group.
  const int jk = j0 + col;
  const int jkr = TAIL ? min(jk, c.kend - 1) : jk;
  RotRow krot{0, 1.f};
  uint4 cst[HT][2];
  uint4 kr[NT];
  if constexpr (KM != kKeyPlain) {
    krot = split_key_rot<PR, TAIL>(jk, col, q0, r0, c.G, c.invG, c.qpos, c.w0, c.kend);
    const uint4* cs8 =
        reinterpret_cast<const uint4*>(c.tab16 + (static_cast<int64_t>(krot.row) * (H / 2) + g * 4) * 4);
#pragma unroll
    for (int t = 0; t < HT; ++t) {
      cst[t][0] = cs8[t * 8];      // frequency pairs e2 = 0, 1
      cst[t][1] = cs8[t * 8 + 1];  // e2 = 2, 3
    }
  }
  if constexpr (PFM) {
    static_assert(!TAIL, "the tail block loads for itself");
#pragma unroll
    for (int t = 0; t < NT; ++t) kr[t] = L->kr[t];
  } else {
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
  // non-tail addresses: a per-lane base plus the wave-uniform row offset
  const uint16_t* krow = TAIL ? c.kc + jkr * c.ss + g * 8 : c.klane + j0 * c.ss;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(krow + t * 32));
    kr[t] = make_uint4(x[0], x[1], x[2], x[3]);
  }
  __builtin_amdgcn_sched_barrier(0);
  }

  f16x8 a[NT];
  if constexpr (KM != kKeyPlain) {
  // ---- rotate each key at its own angle (split_key_rot) in packed half:
  // the bf16 key converts to half exactly, the half cos/sin carry at most
  // 2^-12 absolute error, and the result is rounded to half for the MFMA
  // either way.  A key outside half range turns into +-inf here, its scores
  // into +-inf or NaN (never finite); NaN and +inf poison the head's sums by
  // themselves, -inf is caught below.
  const f16x2 sgn2 = {static_cast<_Float16>(krot.sgn), static_cast<_Float16>(krot.sgn)};
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    const uint4 ca = cst[t][0], cb = cst[t][1];
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
  }
  if constexpr (PFM && KM != kKeyPlain) {
    if (has_next) {
      __builtin_amdgcn_sched_barrier(0);
      issue_block_loads<D>(c, *L, nj0, vnext);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- S = K_rot Q_sel^T: lane (col = head, g) holds keys j0 + g*4 + rr
  const bool all_remote = c.qpos - (j0 + kKB - 1) >= c.w0;
  const bool all_local = c.qpos - j0 < c.w0;
  f32x4 sr = {0.f, 0.f, 0.f, 0.f}, sl = {0.f, 0.f, 0.f, 0.f};
  if constexpr (KM == kKeyPlain) {
    // every key local: the stored bf16 key is the A operand as loaded
#pragma unroll
    for (int t = 0; t < NT; ++t)
      sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[t]), __builtin_bit_cast(bf16x8, qrf[t]),
                                                   sl, 0, 0, 0);
    if constexpr (PFM) {
      if (has_next) {
        __builtin_amdgcn_sched_barrier(0);
        issue_block_loads<D>(c, *L, nj0, vnext);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else if (!all_local) {
#pragma unroll
    for (int t = 0; t < NT; ++t) sr = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], qrf[t], sr, 0, 0, 0);
  }
  if (KM != kKeyPlain && !all_remote) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      sl = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], c.ql[(t * 4 + g) * NR + c.qcol], sl, 0, 0, 0);
  }
  // one logit set per key: outside the window edge the other set was not
  // formed and is zero
  float sv[4];
  if (KM == kKeyPlain || all_remote || all_local) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) sv[rr] = sr[rr] + sl[rr];
  } else {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) sv[rr] = c.qpos - (j0 + g * 4 + rr) < c.w0 ? sl[rr] : sr[rr];
  }
  if constexpr (KM != kKeyPlain) {
    // a finite in-range key never scores -inf; one that does was outside
    // half range (see above) and makes its head's result NaN at the end
    const float lmin = fminf(fminf(sv[0], sv[1]), fminf(sv[2], sv[3]));
    st.bad = st.bad || lmin == -INFINITY;
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
  if constexpr (PFM) {
    // the other V buffer is being filled for the next block meanwhile
    i16x4 bv[NB];
    uint32_t ad[NB];
    const uint32_t vb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) const uint16_t*)((__attribute__((address_space(3))) const void*)vcur)));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) ad[nb] = vb + 2u * static_cast<uint32_t>(c.tr_base ^ (nb << 4));
    lds_read_tr16_all(bv, ad);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      st.o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, bv[nb], st.o[nb], 0, 0, 0);
      st.o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, bv[nb], st.o[nb], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const i16x4 bv = lds_read_tr16(c.vblk + (c.tr_base ^ (nb << 4)));
      st.o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, bv, st.o[nb], 0, 0, 0);
      st.o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, bv, st.o[nb], 0, 0, 0);
    }
  }
}

template <int D, int NR, int KM>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void split_bf16_kernel(Params p) {
  constexpr bool PR = KM == kKeyPre;
  constexpr int NT = D / 32;    // QK^T MFMAs per 16 keys (32 features each)
  constexpr int HT = NT / 2;    // first-half feature groups
  constexpr int H = D / 2;
  constexpr int NB = D / 16;    // PV MFMAs per 16 keys (16 features each)
  static_assert(NR <= 16, "one MFMA column per query head");
  // per-wave V blocks: two buffers for the prefetching walk; with more than 8
  // query heads per KV head the local query fragments take the LDS that the
  // second buffer would (two workgroups per CU must fit in 160 KB), and the
  // walk loads each block for itself
  constexpr int NVB = NR <= 8 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint16_t sV[kWaves][NVB][kKB * D];
  // B fragments of the query heads rotated at qpos (needed only by key
  // blocks that reach into the local window): [wave][t][g][head]
  __shared__ f16x8 sQl[kWaves][NT * 4 * NR];

  // one workgroup = one key range of one sequence for `hw` KV heads, `wph`
  // wavefronts per head: with 8 KV heads every wave streams its own 256-byte
  // slice of the same 2 KB cache rows, and all waves read the same cos/sin rows
  const int hw = kWaves / p.wph;
  // workgroup -> (sequence, head group, key range).  Workgroups go to the 8
  // XCDs in turn (id mod 8); when the ranges divide by 8, XCD x takes ranges
  // x * ns/8 .. of every sequence, so each XCD's L2 holds the cos/sin rows
  // of its own eighth of the positions only.
  const int units = p.B * (p.Hkv / hw);
  const int id = blockIdx.x;
  int unit, split;
  if (p.nsplit % 8 == 0) {
    const int k = id / 8;
    unit = k % units;
    split = (id % 8) * (p.nsplit / 8) + k / units;
  } else {
    unit = id % units;
    split = id / units;
  }
  const int hgrp = unit % (p.Hkv / hw);
  const int b = unit / (p.Hkv / hw);
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
  c.vblk = sV[wid][0];
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
    const float sc = p.scale_log2;
    if constexpr (KM == kKeyPlain) {
      // stored query (already rotated at qpos), scaled, as a bf16 operand
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        bf16x8 qb;
#pragma unroll
        for (int e = 0; e < 8; ++e) qb[e] = static_cast<__bf16>(x[t][e] * sc);
        qrf[t] = __builtin_bit_cast(f16x8, qb);
      }
    } else {
      const RotRow rl = rot_row(qpos, qpos, PR);
      const RotRow rr = rot_row(qpos / G, qpos, PR);
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
          ql[t][e] = half_or_nan((x1 * cl.x - x2 * cl.y) * sc);
          ql[t + HT][e] = half_or_nan((x2 * cl.x + x1 * cl.y) * sc);
          qrf[t][e] = half_or_nan((x1 * cr.x - x2 * cr.y) * sc);
          qrf[t + HT][e] = half_or_nan((x2 * cr.x + x1 * cr.y) * sc);
        }
      if (col < NR) {
#pragma unroll
        for (int t = 0; t < NT; ++t) sQl[wid][(t * 4 + g) * NR + col] = ql[t];
      }
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
    // block nb's chunk is (2 nb + tr_c) ^ tr_x with tr_x even, i.e. 2 (nb ^ tr_x / 2) + tr_c: the
    // block index enters the element offset as 16 (nb ^ tr_x / 2), on bits no other term uses
    c.tr_base = tr_row * D + (tr_c * 8 + tr_half) + (tr_x / 2) * 16;
  }

  SplitState<D> st;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) st.o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
  st.bad = false;

  // full blocks: each one's loads are issued while the previous block is
  // computed; then the tail block, which loads for itself
  KeyBlocks kb(kbeg, w, p.wph, G);
  if constexpr (NVB == 1) {
    for (; kb.j0 + kKB <= kend; kb.next()) split_block<D, NR, false, KM>(c, qrf, st, kb.j0, kb.q0, kb.r0);
  } else if (kb.j0 + kKB <= kend) {
    BlockLoads<D> L;
    int buf = 0;
    issue_block_loads<D>(c, L, kb.j0, sV[wid][0]);
    for (;;) {
      KeyBlocks nb = kb;
      nb.next();
      const bool has_next = nb.j0 + kKB <= kend;
      split_block<D, NR, false, KM, true>(c, qrf, st, kb.j0, kb.q0, kb.r0, &L, sV[wid][buf], has_next, nb.j0, nb.q0,
                                          nb.r0, sV[wid][(buf ^ 1) % NVB]);
      kb = nb;
      buf ^= 1;
      if (!has_next) break;
    }
  }
  if (kb.j0 < kend) split_block<D, NR, true, KM>(c, qrf, st, kb.j0, kb.q0, kb.r0);

  if (st.bad) st.l = __builtin_nanf("");
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
// the weights 2^(m_s - M) are formed once into LDS; then the kCombThreads /
// D thread groups each sum every NG-th partial state for one feature, with
// four independent accumulators so that several loads are in flight, and
// the group sums are added in LDS.
constexpr int kCombThreads = 512;
constexpr int kMaxParts = 1024;
template <int D>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(const float* __restrict__ part, int nparts, void* o,
                                                               float* lse, int bf16, const int32_t* __restrict__ seq_L,
                                                               int Hq, int max_L) {
  constexpr int NW = kCombThreads / 64;
  constexpr int NG = kCombThreads / D;
  __shared__ float sw[kMaxParts];
  __shared__ float sred_m[NW], sred_d[NW];
  __shared__ float sacc[NG][D];
  const int bh = blockIdx.x;  // b * Hq + h
  const int t = threadIdx.x;
  const int L = seq_L[bh / Hq];
  if (L < 1 || L > max_L) return;  // outside the documented contract: left unwritten, as in the split kernel
  const float* pp = part + static_cast<int64_t>(bh) * nparts * (D + 2);
  float mx = -INFINITY;
  for (int s = t; s < nparts; s += kCombThreads) mx = fmaxf(mx, pp[s * (D + 2) + D]);
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((t & 63) == 0) sred_m[t >> 6] = mx;
  __syncthreads();
  float M = sred_m[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) M = fmaxf(M, sred_m[i]);
  float den = 0.f;
  for (int s = t; s < nparts; s += kCombThreads) {
    const float ms = pp[s * (D + 2) + D];
    const float wgt = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    sw[s] = wgt;
    den += wgt * pp[s * (D + 2) + D + 1];
  }
  for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
  if ((t & 63) == 0) sred_d[t >> 6] = den;
  __syncthreads();
  const int f = t % D, gi = t / D;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int s = gi;
  for (; s + 3 * NG < nparts; s += 4 * NG) {
    a0 = fmaf(sw[s], pp[s * (D + 2) + f], a0);
    a1 = fmaf(sw[s + NG], pp[(s + NG) * (D + 2) + f], a1);
    a2 = fmaf(sw[s + 2 * NG], pp[(s + 2 * NG) * (D + 2) + f], a2);
    a3 = fmaf(sw[s + 3 * NG], pp[(s + 3 * NG) * (D + 2) + f], a3);
  }
  for (; s < nparts; s += NG) a0 = fmaf(sw[s], pp[s * (D + 2) + f], a0);
  sacc[gi][f] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  if (t >= D) return;
  float num = 0.f;
#pragma unroll
  for (int i = 0; i < NG; ++i) num += sacc[i][t];
  float dd = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) dd += sred_d[i];
  const float r = num / dd;
  if (bf16) static_cast<uint16_t*>(o)[static_cast<int64_t>(bh) * D + t] = float_to_bf16_bits(r);
  else static_cast<float*>(o)[static_cast<int64_t>(bh) * D + t] = r;
  if (lse && t == 0) lse[bh] = (M + log2f(dd)) * kLn2;
}

// Debug export: the signed table row the bf16 split kernel rotates each key
// with (split_key_rot over the same KeyBlocks walk), row r with sin negated
// stored as ~r.  One thread per (split, wave slot, key column) of sequence
// blockIdx.y; keys past L_b are not written.
template <bool PR>
__global__ void key_rows_kernel(const int32_t* __restrict__ seq_L, int max_L, int nsplit, int kps, int wph,
                                int w_pretrained, int w0, int32_t* __restrict__ out) {
  const int b = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int col = idx % 16;
  const int w = (idx / 16) % wph;
  const int split = idx / (16 * wph);
  if (split >= nsplit) return;
  const int L = seq_L[b];
  if (L < 1 || L > max_L) return;
  const int G = group_size(L, w_pretrained);
  const float invG = 1.f / static_cast<float>(G);
  const int qpos = L - 1;
  const int kbeg = split * kps;
  const int kend = min(L, kbeg + kps);
  int32_t* dst = out + static_cast<int64_t>(b) * max_L;
  KeyBlocks kb(kbeg, w, wph, G);
  for (; kb.j0 + kKB <= kend; kb.next()) {
    const RotRow r = split_key_rot<PR, false>(kb.j0 + col, col, kb.q0, kb.r0, G, invG, qpos, w0, kend);
    dst[kb.j0 + col] = r.sgn < 0.f ? ~r.row : r.row;
  }
  if (kb.j0 < kend && kb.j0 + col < kend) {
    const RotRow r = split_key_rot<PR, true>(kb.j0 + col, col, kb.q0, kb.r0, G, invG, qpos, w0, kend);
    dst[kb.j0 + col] = r.sgn < 0.f ? ~r.row : r.row;
  }
}

template <int D, int NR>
void launch_split(const Params& p, bool bf16, hipStream_t s) {
  if (bf16) {
    const int hw = kWaves / p.wph;
    const dim3 grid(p.B * (p.Hkv / hw) * p.nsplit);
    if (p.plain)
      hipLaunchKernelGGL((split_bf16_kernel<D, NR, kKeyPlain>), grid, dim3(kWaves * 64), 0, s, p);
    else if (p.prerot)
      hipLaunchKernelGGL((split_bf16_kernel<D, NR, kKeyPre>), grid, dim3(kWaves * 64), 0, s, p);
    else
      hipLaunchKernelGGL((split_bf16_kernel<D, NR, kKeyRaw>), grid, dim3(kWaves * 64), 0, s, p);
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

// Key-range splits per (sequence, KV head).  The bf16 split kernel runs two
// 8-wavefront workgroups per CU (4 waves per SIMD), i.e. 512 at once on the
// 256 CUs of gfx950; the grid is sized to fill that once and no more (one
// round, no tail: at 16 x 128K, 32 splits ran in 1.40 ms against 1.42, 1.45
// and 1.59 ms for 64, 128 and 256).  Each split keeps at least 256 keys and
// the combine merges at most 1024 partial states per head.
constexpr int kResidentSplitGroups = 512;
int decode_num_splits(int B, int max_L, int Hkv) {
  int hw = 1;
  while (hw < kWaves && Hkv % (hw * 2) == 0) hw *= 2;
  const int64_t units = static_cast<int64_t>(B) * (Hkv / hw);  // workgroups per split
  int64_t ns = kResidentSplitGroups / std::max<int64_t>(units, 1);
  const int64_t cap_keys = (static_cast<int64_t>(max_L) + 255) / 256;
  // partial states per head: ns * (kWaves / hw) on the bf16 path, ns *
  // kWavesF32 on the fp32 one
  const int64_t cap_parts = kMaxParts / std::max(kWaves / hw, kWavesF32);
  ns = std::min(ns, std::min(cap_keys, cap_parts));
  return static_cast<int>(std::max<int64_t>(ns, 1));
}

// KV heads per bf16 split workgroup: the largest power of two dividing Hkv,
// at most 8; each head then has 8 / hw wavefronts (partial-state slots).
static int split_waves_per_head(int Hkv) {
  int hw = 1;
  while (hw < kWaves && Hkv % (hw * 2) == 0) hw *= 2;
  return kWaves / hw;
}

size_t decode_part_bytes(bool bf16, int B, int max_L, int Hq, int Hkv, int D) {
  const int ns = decode_num_splits(B, max_L, Hkv);
  const int slots = bf16 ? split_waves_per_head(Hkv) : kWavesF32;
  return align_up(static_cast<size_t>(B) * Hq * ns * slots * (D + 2) * sizeof(float), 256);
}

size_t rope_table_bytes(int npos, int D) {
  return align_up(static_cast<size_t>(npos) * (D / 2) * sizeof(float2), 256) +
         align_up(static_cast<size_t>(npos) * D * sizeof(_Float16), 256);
}

size_t decode_ws_bytes(int B, int max_L, int Hq, int Hkv, int D) {
  const size_t part = std::max(decode_part_bytes(true, B, max_L, Hq, Hkv, D),
                               decode_part_bytes(false, B, max_L, Hq, Hkv, D));
  return rope_table_bytes(max_L, D) + part;
}

hipError_t launch_rope_table_full(void* table, int npos, int D, double theta, hipStream_t s) {
  const size_t tab = align_up(static_cast<size_t>(npos) * (D / 2) * sizeof(float2), 256);
  return launch_rope_table(static_cast<float2*>(table), npos, D, theta, s,
                           reinterpret_cast<uint16_t*>(static_cast<char*>(table) + tab));
}

bool decode_is_plain(const DecodeCall& c, bool bf16) { return bf16 && c.prerot && c.w0 >= c.max_L; }

hipError_t launch_decode(const DecodeCall& c, bool bf16, hipStream_t s) {
  if (c.B == 0) return hipSuccess;
  const int ns = decode_num_splits(c.B, c.max_L, c.Hkv);
  const bool plain = decode_is_plain(c, bf16);
  // cos/sin rows: the caller's prepared table (rows 0 .. table_rows-1), or
  // the front of the workspace, built here
  char* ws = static_cast<char*>(c.ws);
  const int npos = c.table ? c.table_rows : c.max_L;
  char* tbase = c.table ? static_cast<char*>(const_cast<void*>(c.table)) : ws;
  const size_t tab = align_up(static_cast<size_t>(npos) * (c.D / 2) * sizeof(float2), 256);
  uint16_t* t16 = reinterpret_cast<uint16_t*>(tbase + tab);
  Params p{};
  p.q = c.q;
  p.kc = c.kc;
  p.vc = c.vc;
  p.sb = c.sb;
  p.ss = c.ss;
  p.sh = c.sh;
  p.part = c.part ? c.part : reinterpret_cast<float*>(ws + (c.table ? 0 : rope_table_bytes(c.max_L, c.D)));
  p.seq_L = c.seq_L;
  p.tab = reinterpret_cast<const float2*>(tbase);
  p.tab16 = reinterpret_cast<const _Float16*>(t16);
  p.B = c.B;
  p.Hq = c.Hq;
  p.Hkv = c.Hkv;
  p.ratio = c.Hq / c.Hkv;
  p.nsplit = ns;
  p.kps = keys_per_split(c.max_L, ns);
  p.max_L = c.max_L;
  p.wph = split_waves_per_head(c.Hkv);
  p.slots = bf16 ? p.wph : kWavesF32;
  if (ns * p.slots > kMaxParts) return hipErrorInvalidValue;  // excluded by decode_num_splits
  p.w_pretrained = c.w_pretrained;
  p.w0 = c.w0;
  p.scale_log2 = c.scale * kLog2e;
  p.prerot = c.prerot ? 1 : 0;
  p.plain = plain ? 1 : 0;
  hipError_t e = hipSuccess;
  if (!c.table && !plain) {
    // rows a decode reads: remote positions (all below w_pretrained) and each
    // sequence's local window; a pre-rotated cache reads row 0 and the
    // correction rows j - f(j), which cover the whole range
    uint16_t* t16w = bf16 ? t16 : nullptr;  // the half rows feed the bf16 split kernel only
    e = c.prerot ? launch_rope_table(reinterpret_cast<float2*>(ws), c.max_L, c.D, c.theta, s, t16w)
                 : launch_rope_table_rows(reinterpret_cast<float2*>(ws), c.max_L, c.D, c.theta, c.seq_L, c.B, c.w0,
                                          c.w_pretrained, s, t16w);
    if (e != hipSuccess) return e;
  }
  const int ratio = c.Hq / c.Hkv;
  if (c.D == 128) launch_split_d<128>(p, ratio, bf16, s);
  else launch_split_d<64>(p, ratio, bf16, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nparts = ns * p.slots;
  if (c.D == 128)
    hipLaunchKernelGGL(combine_kernel<128>, dim3(c.B * c.Hq), dim3(kCombThreads), 0, s, p.part, nparts, c.o, c.lse,
                       bf16 ? 1 : 0, c.seq_L, c.Hq, c.max_L);
  else
    hipLaunchKernelGGL(combine_kernel<64>, dim3(c.B * c.Hq), dim3(kCombThreads), 0, s, p.part, nparts, c.o, c.lse,
                       bf16 ? 1 : 0, c.seq_L, c.Hq, c.max_L);
  return hipGetLastError();
}

// Partial states of jl_bifocal_decode_with_table_noalloc, for callers that
// cannot allocate: a file-scope device array, one per GPU the library runs on,
// held until the process ends.  Host code must not use the array's name as a
// device address; it takes the address hipGetSymbolAddress returns, looked up
// once per device (with that device current) and kept.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t decode_scratch_bytes() { return kScratchBytes; }

hipError_t decode_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_key_rows(const int32_t* seq_L, int B, int max_L, int Hkv, int w_pretrained, int w0,
                                  bool prerot, int32_t* out, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const int ns = decode_num_splits(B, max_L, Hkv);
  const int kps = keys_per_split(max_L, ns);
  const int wph = split_waves_per_head(Hkv);
  const int threads = ns * wph * 16;
  const dim3 grid((threads + 255) / 256, B);
  if (prerot)
    hipLaunchKernelGGL(key_rows_kernel<true>, grid, dim3(256), 0, s, seq_L, max_L, ns, kps, wph, w_pretrained, w0, out);
  else
    hipLaunchKernelGGL(key_rows_kernel<false>, grid, dim3(256), 0, s, seq_L, max_L, ns, kps, wph, w_pretrained, w0,
                       out);
  return hipGetLastError();
}

}  // namespace jl
