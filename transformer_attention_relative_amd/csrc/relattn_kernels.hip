// Fused relative-position attention forward for gfx950 (MI355X).
//
// Sources (page title, then passage):
//   [RPE]  "Relative Position Embeddings, in depth: Shaw, Transformer-XL,
//          T5 buckets and DeBERTa ..." (aicassindra.com)
//   [T5B]  "T5 Relative-Position Bias" (liminalml.com)
//   [DRPE] "DeBERTa > Relative Position Encoding" (mbrenndoerfer.com)
//
// Design (a workgroup = NW wave64s; a wave owns QB blocks of 32 query rows
// of one (b, h)):
//   * Key/value tiles (64 rows) go straight from global memory into an LDS
//     ring of stages (global_load_lds_dwordx4), 16-byte chunks XOR-swizzled
//     per row; no register staging, so the next tiles are in flight while
//     the current one is used.
//   * Scores are produced transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16,
//     or v_mfma_f32_32x32x2f32 for float32): a lane owns one query row and 16
//     keys of each 32-key block, so the row max needs one lane^32 exchange per
//     tile and the output rescale is a per-lane scalar.  One K fragment read
//     from LDS feeds the QB query blocks of the wave.
//   * The output is accumulated transposed, O^T = V^T P^T: P leaves the score
//     accumulator directly as the B operand; the V^T A operand comes from the
//     row-major V tile through ds_read_b64_tr_b16 (LDS transpose read).
//   * Online softmax in the exp2 domain with scale*log2(e) folded into one
//     FMA; a row's reference max is only moved (and the output rescaled) on
//     an exact path taken by a block whose lane sum of P exceeds 2^20.
//   * The relative term never exists as an L x L array: per (query block,
//     key tile) it is a per-row constant folded into the exponent (saturated
//     T5 buckets, clipped Shaw / DeBERTa offsets) or it is written into the
//     MFMA accumulator before q.k is accumulated on top (near-diagonal
//     tiles).  Masked entries enter that accumulator as -inf.
//   * T5 bucket ids come from host-computed integer thresholds; no log runs
//     on the GPU ([T5B]: saturation starts at the lower edge of the last bin).
//   * Shaw's value term: each offset strictly inside the clip window belongs
//     to exactly one key of a row, so its bin holds that key's probability;
//     near tiles scatter those probabilities into a per-wave bin tile that is
//     multiplied by a_V with one more MFMA; the two clipped bins take the rest
//     of the row mass at the end ([RPE] Shaw section).
//   * DeBERTa near blocks compute the content-to-position band (Kr rows x Q)
//     and the position-to-content band (Qr rows x K) with MFMA and gather
//     them through per-wave LDS; far blocks reduce to a per-row constant plus
//     a per-key constant ([DRPE]: every offset beyond +-k uses a boundary
//     row), the latter formed in bfloat16 as K times the boundary Qr row by
//     MFMA.
//   * Transformer-XL blocks compute q.E over their 63 distances the same way,
//     with the bias terms u.k_j and v.E[r] added as float32 constants ([RPE]
//     Transformer-XL section); ALiBi adds slope * distance.
//   * Decode-like T5 / ALiBi shapes split each workgroup's key range over two
//     halves of four waves, merged through LDS at the end.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "relattn_internal.hpp"

namespace relattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define RA_NEG_INF (-__builtin_inff())
#define RA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Orders this wave's LDS writes before its later LDS reads (lanes of the same
// wave read what other lanes wrote).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// s_waitcnt vmcnt(N) (gfx9 encoding, expcnt/lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// ----------------------------------------------------------------------------
// Index functions (shared by the index kernel and the fused kernel)
// ----------------------------------------------------------------------------

// T5 bucket of offset = key - query ([RPE] T5 section; [T5B]).  thr[m] is the
// smallest distance whose within-direction slot is >= exact + m (thr[0] ==
// exact); the thresholds come from the host, so no logarithm runs here.
// Entries from nthr on hold INT32_MAX, so with at most 16 thresholds the
// count is a fixed run of compares against uniform (scalar) values.
__device__ __forceinline__ int t5_bucket_dev(int offset, int slots, int exact, int bidir,
                                             int nthr, const int32_t* thr) {
  int base = 0, dist;
  if (bidir) {
    base = offset > 0 ? slots : 0;
    dist = offset < 0 ? -offset : offset;
  } else {
    dist = offset < 0 ? -offset : 0;
  }
  int m = 0;
  if (nthr <= 16) {
#pragma unroll
    for (int t = 1; t < 16; ++t) m += dist >= thr[t] ? 1 : 0;
  } else {
    for (int t = 1; t < nthr; ++t) m += dist >= thr[t] ? 1 : 0;
  }
  return dist < exact ? base + dist : base + exact + m;
}

// Shaw row: clip(key - query, -k, k) + k ([RPE] Shaw section).
__device__ __forceinline__ int shaw_row_dev(int offset, int k) {
  return min(max(offset, -k), k) + k;
}

// DeBERTa clip-and-shift of x = i - j ([DRPE] "The Relative Position Formula").
__device__ __forceinline__ int deberta_delta_dev(int x, int k) {
  return min(max(x, -k), k - 1) + k;
}

__global__ void relattn_index_kernel(IndexArgs a) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < a.n; e += stride) {
    const int qp = a.q_pos[e], kp = a.k_pos[e];
    int r;
    if (a.kind == 0) {
      r = t5_bucket_dev(kp - qp, a.t5_slots, a.t5_exact, a.t5_bidir, a.t5_nthr, a.t5_thr);
    } else if (a.kind == 1) {
      r = shaw_row_dev(kp - qp, a.clip_k);
    } else if (a.kind == 3) {
      r = abs(kp - qp);  // ALiBi distance
    } else if (a.kind == 4) {
      r = qp - kp;       // Transformer-XL: row of the relative encodings
    } else {
      r = a.which == 0 ? deberta_delta_dev(qp - kp, a.clip_k) : deberta_delta_dev(kp - qp, a.clip_k);
    }
    a.out[e] = r;
  }
}

// ----------------------------------------------------------------------------
// MFMA helpers and fragments
// ----------------------------------------------------------------------------

__device__ __forceinline__ f32x16 mma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x2 cvt2(float x, float y) {
  f32x2 v = {x, y};
  return __builtin_convertvector(v, bf16x2);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(f32x16 s, int base) {
  bf16x2 c0 = cvt2(s[base + 0], s[base + 1]), c1 = cvt2(s[base + 2], s[base + 3]);
  bf16x2 c2 = cvt2(s[base + 4], s[base + 5]), c3 = cvt2(s[base + 6], s[base + 7]);
  bf16x8 r = {c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
  return r;
}

// Sum of the 8 bf16 values with v_dot2c_f32_bf16 (two per instruction).
__device__ __forceinline__ float sum_bf16x8(bf16x8 p, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){p[0], p[1]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){p[2], p[3]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){p[4], p[5]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){p[6], p[7]}, one, acc, false);
  return acc;
}

// max of three (v_max3_f32).  The library is compiled without NaN support
// (-fno-honor-nans): scores are finite or -inf, and with NaNs possible every
// fmaxf operand would first be quieted by an extra v_max.
__device__ __forceinline__ float vmax3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Max of the 16 scores a lane holds for one 32-key block (two chains).
__device__ __forceinline__ float max16(const f32x16& x) {
  float m0 = vmax3(x[0], x[1], x[2]), m1 = vmax3(x[3], x[4], x[5]);
  m0 = vmax3(m0, x[6], x[7]);
  m1 = vmax3(m1, x[8], x[9]);
  m0 = vmax3(m0, x[10], x[11]);
  m1 = vmax3(m1, x[12], x[13]);
  return vmax3(m0, m1, vmax3(x[14], x[15], x[15]));
}

// The lane index, computed by instructions the compiler may not move: values
// derived from it inside a loop stay inside that loop instead of being
// hoisted (and kept live) across the whole kernel.
__device__ __forceinline__ int opaque_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// max(x[l], x[l ^ 32]) in every lane l without going through LDS:
// v_permlane32_swap on (x, x) exchanges the high half of the first copy with
// the low half of the second, so one result holds the low half's values in
// both halves and the other the high half's.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float lo = __uint_as_float(r[0]), hi = __uint_as_float(r[1]);
  return vmax3(lo, hi, hi);
}

// In the 32x32 accumulator layout, register i of a lane in half hh holds
// row 8*(i/4) + 4*hh + (i%4) of the lane's column.
__device__ __forceinline__ int acc_row(int i, int hh) { return 8 * (i >> 2) + 4 * hh + (i & 3); }

// Slot permutations of the LDS tile rows: chunk c of K row r (CPR 16-byte
// chunks per row) is stored in slot c ^ swz_k<CPR>(r), chunk c of V row r in
// slot c ^ swz_v<CPR>(r).  The masks are GF(2)-linear in the row bits.
// swz_k: the K fragment reads (16 or 32 consecutive lanes reading 16 bytes
// from consecutive rows) touch every bank once per cycle whether a cycle
// serves 256 or 512 bytes.  swz_v: the V transpose reads (32 or 64 lanes
// reading 8 bytes from 4 or 8 consecutive rows) do the same, and the mask
// depends on the row's low 3 bits only, so every V read of a tile is one
// per-lane offset plus an immediate.
template <int CPR>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (CPR == 4) return (((r >> 2) ^ (r >> 4)) & 1) | (((r >> 3) & 1) << 1);
  else if constexpr (CPR == 8)
    return ((r >> 3) & 1) | (((r >> 2) & 1) << 1) | ((((r >> 1) ^ (r >> 2) ^ (r >> 4)) & 1) << 2);
  else return ((r ^ (r >> 4)) & 1) | (((r >> 3) & 1) << 1) | (((r >> 2) & 1) << 2) | (((r >> 1) & 1) << 3);
}
template <int CPR, bool BF>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (BF && CPR == 8) return (((r >> 1) ^ (r >> 2)) & 1) << 2;
  else return 0;
}

// A row-major table row as an MFMA operand (A row or B column): bf16 chunk t
// holds elements 16t + 8hh .. +7; fp32 element t is d-index t + (d/2)*hh.
template <bool BF, int D>
struct TableFrag;
template <int D>
struct TableFrag<true, D> {
  bf16x8 v[D / 16];
  __device__ __forceinline__ void load(const bf16* row, int hh) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) v[t] = *reinterpret_cast<const bf16x8*>(row + 16 * t + 8 * hh);
  }
  // a row of a swizzled LDS K tile; off[t] = byte offset of chunk t (see KOffsets)
  __device__ __forceinline__ void load_lds(const char* base, const int* off) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) v[t] = *reinterpret_cast<const bf16x8*>(base + off[t]);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) v[t] = {};
  }
};
template <int D>
struct TableFrag<false, D> {
  float v[D / 2];
  __device__ __forceinline__ void load(const float* row, int hh) {
#pragma unroll
    for (int t = 0; t < D / 8; ++t) {
      f32x4 x = *reinterpret_cast<const f32x4*>(row + (D / 2) * hh + 4 * t);
      v[4 * t + 0] = x[0]; v[4 * t + 1] = x[1]; v[4 * t + 2] = x[2]; v[4 * t + 3] = x[3];
    }
  }
  __device__ __forceinline__ void load_lds(const char* base, const int* off) {
#pragma unroll
    for (int t = 0; t < D / 8; ++t) {
      f32x4 x = *reinterpret_cast<const f32x4*>(base + off[t]);
      v[4 * t + 0] = x[0]; v[4 * t + 1] = x[1]; v[4 * t + 2] = x[2]; v[4 * t + 3] = x[3];
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int t = 0; t < D / 2; ++t) v[t] = 0.f;
  }
};

// a.b over the head dimension, accumulated from zero (the first MFMA takes
// the inline constant 0 as its accumulator input)
template <bool BF, int D>
__device__ __forceinline__ f32x16 mma_frag0(const TableFrag<BF, D>& a, const TableFrag<BF, D>& b) {
  f32x16 c;
  if constexpr (BF) {
    c = mma_bf16(a.v[0], b.v[0], f32x16{});
#pragma unroll
    for (int t = 1; t < D / 16; ++t) c = mma_bf16(a.v[t], b.v[t], c);
  } else {
    c = mma_f32(a.v[0], b.v[0], f32x16{});
#pragma unroll
    for (int t = 1; t < D / 2; ++t) c = mma_f32(a.v[t], b.v[t], c);
  }
  return c;
}

template <bool BF, int D>
__device__ __forceinline__ f32x16 mma_frag(const TableFrag<BF, D>& a, const TableFrag<BF, D>& b, f32x16 c) {
  if constexpr (BF) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) c = mma_bf16(a.v[t], b.v[t], c);
  } else {
#pragma unroll
    for (int t = 0; t < D / 2; ++t) c = mma_f32(a.v[t], b.v[t], c);
  }
  return c;
}

// Per-lane byte offsets into the K and V tiles, fixed for the whole key loop
// (a tile read is its stage base + one of these + an immediate).
//   k[t]: the 16-byte chunk t of the lane's K fragment row lq (the MFMA A
//         row) of a 32-key block; bf16 chunk t holds head dims 16t + 8hh ..,
//         float32 chunk t holds head dims 4t + (d/2)hh ..
//   v[db] (bf16): the V^T fragment (A operand of O^T = V^T P^T) for head-dim
//         block db, read with ds_read_b64_tr_b16.  The transpose read gives
//         lane (group G = lane/16, index i) the elements e = 0..3 of the
//         8-byte chunks addressed by lanes 16G + 4e + i/4, each at position
//         i%4.  So lane (G, e, j) addresses key 16cc + 8*half + 4*(G/2) + e
//         at head dims 32db + 16*(G%2) + 4j .. +3, and every lane receives
//         the 4 keys of its MFMA k-slots at head dim 32db + lane%32 -- the
//         same key order as P in the score accumulator.
//   v[0] (float32): key 4hh + (cc%4) + 8(cc/4) of a 32-key block at head dim
//         lq (plus 32db and the key offsets as immediates).
template <bool BF, int D>
struct KOffsets {
  static constexpr int ESZ = BF ? 2 : 4, ROWB = D * ESZ, CPR = ROWB / 16;
  static constexpr int NK = BF ? D / 16 : D / 8;
  static constexpr int NV = BF ? D / 32 : 1;
  int k[NK], v[NV];
  __device__ __forceinline__ void init(int lane) {
    const int lq = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int t = 0; t < NK; ++t) {
      const int chunk = BF ? 2 * t + hh : (D / 8) * hh + t;
      k[t] = lq * ROWB + ((chunk ^ swz_k<CPR>(lq)) * 16);
    }
    if constexpr (BF) {
      const int G = lane >> 4, e = (lane & 15) >> 2, j = lane & 3;
      const int kl = 4 * (G >> 1) + e;
#pragma unroll
      for (int db = 0; db < NV; ++db) {
        const int c = 4 * db + 2 * (G & 1) + (j >> 1);
        v[db] = kl * ROWB + ((c ^ swz_v<CPR, BF>(kl)) * 16) + 8 * (j & 1);
      }
    } else {
      v[0] = 4 * hh * ROWB + lq * 4;
    }
  }
};

template <int D>
__device__ __forceinline__ bf16x8 load_vt_frag(const char* vtile, int cc, const int vo) {
  constexpr int ROWB = D * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((RA_LDS i16x4*)(vtile + vo + (16 * cc) * ROWB));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((RA_LDS i16x4*)(vtile + vo + (16 * cc + 8) * ROWB));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// float32 V element: key 32kb + acc_row(cc, hh), head dim 32db + lq.
template <int D>
__device__ __forceinline__ float load_v_f32(const char* vtile, int kb, int cc, int db, const int vo) {
  constexpr int ROWB = D * 4;
  return *reinterpret_cast<const float*>(vtile + vo + (32 * kb + 8 * (cc >> 2) + (cc & 3)) * ROWB + 128 * db);
}

// One 16-byte global -> LDS copy per lane (global_load_lds_dwordx4): lane l
// writes LDS bytes lds_base + 16*l .. +15; lds_base must be wave-uniform.
// The copy takes its LDS address from m0.  It is issued from inline assembly
// that saves m0, sets it, issues the copy and restores it, so m0 holds the
// compiler's value again when the block ends (no register the compiler
// reserves is clobbered).  Assembly rather than __builtin_amdgcn_global_load_lds:
// the compiler cannot tell the copies of the next tile from the tile being
// read, and with the builtin it waits for every copy in flight
// (s_waitcnt vmcnt(0)) before each LDS transpose read of V, which serialises
// the copies with the compute.  The kernel orders the copies itself
// (s_waitcnt vmcnt for the copies of the tile about to be read, then a
// workgroup barrier before any wave reads it).
__device__ __forceinline__ void lds_dma16(const void* gptr, const char* lds_base) {
  const uint32_t m0v = (uint32_t)(uintptr_t)(const RA_LDS char*)lds_base;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0"
      : "=&s"(saved)
      : "v"(gptr), "s"(m0v)
      : "memory");
}

// Same copy with a wave-uniform 64-bit global base and a per-lane 32-bit
// offset (the scalar-base form: the per-tile address update is scalar).
__device__ __forceinline__ void lds_dma16_s(const char* gbase, int goff, const char* lds_base) {
  const uint32_t m0v = (uint32_t)(uintptr_t)(const RA_LDS char*)lds_base;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0"
      : "=&s"(saved)
      : "v"(goff), "s"(gbase), "s"(m0v)
      : "memory");
}

// Direct global -> LDS loads of one K tile and one V tile.  Instruction `ins`
// of a tile covers rows ins*RPI .. +RPI-1; lane l fills LDS slot l of that
// 1 KiB block: row ins*RPI + l/CPR, slot l%CPR, which holds chunk
// slot ^ swz(row).  The per-lane offsets are fixed; a tile that runs past
// the last key re-reads the last key for those rows (in bounds; the keys are
// masked).  Both swizzles read row bits 0..4 only, so when a wave's
// successive instructions are a multiple of 32 rows apart their per-lane
// offsets repeat: one (K, V) offset pair per lane then serves every
// instruction, and the row step goes into the wave-uniform base.
template <bool BF, int D, int NW>
struct TileDma {
  static constexpr int ESZ = BF ? 2 : 4, ROWB = D * ESZ, CPR = ROWB / 16;
  static constexpr int RPI = 64 / CPR, IPT = kBK / RPI, IPW = (IPT + NW - 1) / NW;
  static constexpr int LPW = 2 * IPW;  // load instructions per wave per tile
  static constexpr bool REPEAT = (NW * RPI) % 32 == 0;
  static constexpr int NOFF = REPEAT ? 1 : IPW;
  int ko[NOFF], vo[NOFF];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int r = 0; r < NOFF; ++r) {
      const int row = (wave + r * NW) * RPI + lane / CPR, slot = lane % CPR;
      ko[r] = row * ROWB + ((slot ^ swz_k<CPR>(row)) * 16);
      vo[r] = row * ROWB + ((slot ^ swz_v<CPR, BF>(row)) * 16);
    }
  }
  __device__ __forceinline__ void issue(const char* Kg, const char* Vg, int Lk, int k0, char* stage,
                                        int tile_bytes, int wave, int lane) const {
    if (k0 + kBK <= Lk) {
      const char* kb = Kg + (size_t)k0 * ROWB;
      const char* vb = Vg + (size_t)k0 * ROWB;
#pragma unroll
      for (int r = 0; r < IPW; ++r) {
        const int ins = wave + r * NW;
        const int o = REPEAT ? 0 : r;
        const int step = REPEAT ? r * NW * RPI * ROWB : 0;  // bytes of the row step
        if (IPT % NW == 0 || ins < IPT) {  // wave < NW
          lds_dma16_s(kb + step, ko[o], stage + ins * 1024);
          lds_dma16_s(vb + step, vo[o], stage + tile_bytes + ins * 1024);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < IPW; ++r) {
        const int ins = wave + r * NW;
        const int o = REPEAT ? 0 : r;
        const int step = REPEAT ? r * NW * RPI * ROWB : 0;
        if (IPT % NW == 0 || ins < IPT) {  // wave < NW
          const int row = ins * RPI + lane / CPR;
          const int grow = min(k0 + row, Lk - 1);
          const long long shift = (long long)(grow - row) * ROWB + step;  // may be negative
          lds_dma16(Kg + shift + ko[o], stage + ins * 1024);
          lds_dma16(Vg + shift + vo[o], stage + tile_bytes + ins * 1024);
        }
      }
    }
  }
};

// ----------------------------------------------------------------------------
// The fused forward kernel
// ----------------------------------------------------------------------------

// A block whose lane partial row sum of P exceeds this (or is infinite)
// goes through the exact path: its raw scores are recomputed, the reference
// max moves to the block's max and the running state is rescaled.
constexpr float kSumLimit = 0x1p20f;

// Exponent offset c*b - m_ref of a row; a row with no reference yet (no
// visible key so far) gets a huge finite offset, so every visible score of
// its first block overflows to +inf (and takes the exact path) while hidden
// scores stay -inf (p = 0).  Finite on purpose: -inf + inf would be NaN,
// which the library's no-NaN arithmetic does not look for.
__device__ __forceinline__ float ref_offset(float cb, float m_ref) {
  return m_ref == RA_NEG_INF ? 0x1p100f : cb - m_ref;
}

// DeBERTa blocks whose offsets are all clipped use one Qr row for every pair,
// so their position-to-content term k_j.Qr[d] is a per-key constant.  In
// bfloat16 the kernel forms it itself: K times a B operand whose every
// column is that Qr row, four more MFMAs on the block's K fragment (exact
// products, float32 sums).  In float32 the constants come from
// relattn_colc_kernel (float32 dot products) and enter the score accumulator
// through one MFMA: A holds the key's constants, B selects the side for
// every query.  Transformer-XL's u.k_j takes the same key-constant MFMA with
// bfloat16 hi + lo pairs.
template <bool BF>
struct KeyConst;
template <>
struct KeyConst<true> {
  bf16x8 v;  // lanes of half 0: {hi0, lo0, hi1, lo1, 0, 0, 0, 0} of key lq
  __device__ __forceinline__ void load(const void* colc, size_t base, int key, int hh) {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(reinterpret_cast<const bf16*>(colc) + (base + key) * 4);
    const bf16 z = (bf16)0.f;
    v = hh == 0 ? bf16x8{x[0], x[1], x[2], x[3], z, z, z, z} : bf16x8{};
  }
  // side-0 constant c0 and side-1 constant c1 of key lq, each as a bf16
  // hi + lo pair
  __device__ __forceinline__ void set(float c0, float c1, int hh) {
    const bf16 h0 = (bf16)c0, h1 = (bf16)c1;
    const bf16 l0 = (bf16)(c0 - (float)h0), l1 = (bf16)(c1 - (float)h1);
    const bf16 z = (bf16)0.f;
    v = hh == 0 ? bf16x8{h0, l0, h1, l1, z, z, z, z} : bf16x8{};
  }
};
template <>
struct KeyConst<false> {
  float v;  // k-slot hh: the key's side-hh constant
  __device__ __forceinline__ void load(const void* colc, size_t base, int key, int hh) {
    v = reinterpret_cast<const float*>(colc)[(base + key) * 2 + hh];
  }
  __device__ __forceinline__ void set(float c0, float c1, int hh) { v = hh == 0 ? c0 : c1; }
};

// c + (the side's constant of row lq) in every column; a row is a key of the
// score block (DeBERTa, Transformer-XL u.k_j, ALiBi) or a distance of a band
// block (Transformer-XL v.E[r])
template <bool BF>
__device__ __forceinline__ f32x16 mma_keyconst(const KeyConst<BF>& kc, int side, int hh,
                                               f32x16 c = f32x16{}) {
  if constexpr (BF) {
    const bf16 one = (bf16)1.f, z = (bf16)0.f;
    bf16x8 sel = {};
    if (hh == 0) sel = side == 0 ? bf16x8{one, one, z, z, z, z, z, z} : bf16x8{z, z, one, one, z, z, z, z};
    return mma_bf16(kc.v, sel, c);
  } else {
    return mma_f32(kc.v, hh == side ? 1.f : 0.f, c);
  }
}

// Work item of the workgroup dispatched at position i of n.  The dispatcher
// sends workgroup i to XCD i % 8 and, within the XCD, its k-th workgroup
// (k = i / 8) to CU k % 32, a second round of workgroups taking the CUs'
// second slots in the same order.  With two slots per CU and m workgroups
// on an XCD, 32 < m <= 64, the workgroups at k < m - 32 and k >= 32 share
// a CU while those at m - 32 <= k < 32 run alone.  Items come in order of
// decreasing work (t = 0 the heaviest of the XCD's items): the heaviest
// 64 - m run alone, and each shared CU pairs one of the next heaviest with
// one of the lightest (measured on the padded T5 encoder: 20.1 -> 17.6 us).
// Otherwise positions map to items in order.
__device__ __forceinline__ int dispatch_to_item(int i, int n, int cu_slots) {
  const int x = i % kNumXcd, k = i / kNumXcd;
  const int m = (n - x + kNumXcd - 1) / kNumXcd;  // workgroups on this XCD
  int t = k;
  if (cu_slots == 2 && m > kCuPerXcd && m <= 2 * kCuPerXcd) {
    if (k < m - kCuPerXcd) t = k + 2 * kCuPerXcd - m;    // shared CU, heavier item
    else if (k < kCuPerXcd) t = k - (m - kCuPerXcd);     // alone
    else t = kCuPerXcd + m - 1 - k;                      // shared CU, lighter item
  }
  return t * kNumXcd + x;
}

// The sequence at place `place` when sequences are ordered by valid length
// (clamped to [0, Lk]) in whole key tiles, most first, ties in index order,
// and its valid length as given.  One wave: lane j holds sequence j
// (B <= 64); wave-uniform result.
__device__ __forceinline__ int2 seq_by_length(const int32_t* len, int B, int Lk, int place) {
  const int ln = threadIdx.x & 63;
  const int given = ln < B ? len[ln] : 0;
  const int tiles = ln < B ? (min(max(given, 0), Lk) + kBK - 1) / kBK : -1;
  int mine = 0;
  for (int j = 0; j < B; ++j) {
    const int tj = __builtin_amdgcn_readlane(tiles, j);
    mine += (tj > tiles || (tj == tiles && j < ln)) ? 1 : 0;
  }
  const unsigned long long hit = __ballot(ln < B && mine == place);
  const int b = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
  return make_int2(b, __builtin_amdgcn_readlane(given, b));
}

// Workgroups per CU the register budget is set for: two, except where the
// LDS of a 128-wide head already allows only one (Shaw, DeBERTa, TXL), which
// then gets the whole register file.
template <int KIND, bool BF, int D, int QB, int NW>
__global__ __launch_bounds__(64 * NW, (D > 64 && KIND != 0 && KIND != 3) ? 1 : 8 / NW)
void relattn_fwd_kernel(FwdArgs a) {
  static_assert(QB == 1 || QB == 2, "one or two query blocks per wave");
  // KS = 2: waves 0 .. NW/2-1 and NW/2 .. NW-1 are two halves over the same
  // query rows, each with half of the workgroup's key tiles (key_split)
  constexpr int KS = key_split(KIND, NW);
  constexpr int NWQ = NW / KS;        // waves over distinct query rows
  static_assert(KS == 1 || QB == 1, "a key split runs one query block per wave");
  using T = typename std::conditional<BF, bf16, float>::type;
  using QFrag = TableFrag<BF, D>;
  constexpr int NKB = kBK / 32;       // 32-key blocks per tile
  constexpr int NDB = D / 32;         // 32-wide head-dim blocks of the output
  constexpr int RW = 32 * QB;         // query rows per wave
  constexpr int BQ = RW * NWQ;        // query rows per workgroup
  constexpr int NS = num_stages(KIND, BF, D);
  // Four stages go in pairs: one wait, one barrier and two tile copies per
  // two tiles (the copies of tiles r+2 and r+3 at even r), so each copy
  // has two tiles of work to land in
  constexpr bool PAIR = NS == 4;
  // ring stage of tile r (r >= 0)
  auto stage_of = [](const int r) -> int { return (int)((unsigned)r % (unsigned)NS); };
  constexpr int AHEAD = PAIR ? 2 : NS - 1;  // tiles copied before the loop
  using Dma = TileDma<BF, D, NWQ>;    // the waves of one half share a tile's copies
  constexpr int ROWB = Dma::ROWB;     // bytes per K / V row
  constexpr int LPW = Dma::LPW;       // load instructions per wave per tile
  constexpr bool EVEN_LOADS = (Dma::IPT % NWQ) == 0;
  constexpr float NEG_INF = RA_NEG_INF;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const LdsLayout L = lds_layout(KIND, BF, D, QB, NW, a.clip_k, a.lut_n);
  float* relf = reinterpret_cast<float*>(smem + L.rel_off);
  // this wave's ring of key/value stages (one per key-split half)

  // ---- work item -------------------------------------------------------------
  // Work items in order of decreasing work: the query-tile rank is the
  // major index, heaviest (latest causal) tiles first, so every XCD starts
  // its longest items first.  (head, split) is the minor index, so when
  // B*H*splits is a multiple of 8 every item of one (head, split) lands on
  // the same XCD and shares its L2.  Without a causal mask and with
  // per-sequence valid lengths, the sequences, longest first, are the major
  // index instead, and the dispatch positions are rearranged so that the
  // heaviest items get a CU to themselves (see dispatch_to_item).
  const int per_rank = a.B * a.H * a.n_splits;
  int item = blockIdx.x;
  int seq_len = -1;  // the sequence's valid length when read here
  // (one query block per wave: the two-block kernels are chosen for many
  // workgroups per CU, where the order matters little and registers are short)
  if (QB == 1 && a.sort_items) {
    item = dispatch_to_item(blockIdx.x, a.grid, a.cu_slots);
    // sequences ordered by valid length (the whole work of a workgroup
    // without a causal mask), sequence-major
    const int per_pair = a.H * a.n_splits;
    const int per_seq = a.n_qtiles * per_pair;
    const int place = item / per_seq;
    const int r = item - place * per_seq;
    const int2 bl = seq_by_length(a.kv_valid_len, a.B, a.Lk, place);
    seq_len = bl.y;
    item = (r / per_pair) * per_rank + bl.x * per_pair + r % per_pair;
  }
  const int rank = item / per_rank;
  const int rest = item - rank * per_rank;
  const int bh = rest / a.n_splits;
  const int split = rest - bh * a.n_splits;
  const int qt = a.n_qtiles - 1 - rank;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;

  const int tid = threadIdx.x;
  // the wave index is uniform across the wave; say so, so that everything
  // derived from it (positions, tile classes) lives in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = KS == 2 ? wave / NWQ : 0;    // key-split half
  const int wq = wave - half * NWQ;             // wave within the half
  const int lane = tid & 63;
  const int lq = lane & 31, hh = lane >> 5;
  const int q0 = qt * BQ;
  const int wrow0 = q0 + wq * RW;
  const int pw_min = a.q_pos_offset + wrow0;
  const bool wave_active = wrow0 < a.Lq;
  const int pw_max_real = a.q_pos_offset + min(wrow0 + RW, a.Lq) - 1;
  int qrow[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) qrow[qb] = wrow0 + 32 * qb + lq;
  char* const sbase = smem + half * NS * L.stage_bytes;
  // the part of a workgroup's key-tile range [kb, ke) this wave's half runs:
  // the first ceil(n / 2) tiles for half 0, the rest for half 1
  auto half_range = [&](int& kb, int& ke) {
    if constexpr (KS == 2) {
      const int n0 = (ke - kb + 1) >> 1;
      if (half == 0) ke = kb + n0;
      else kb += n0;
    }
  };

  // p = exp2(c * s + (c * b - m_ref)): one FMA per score, c = scale*log2(e),
  // b the block's per-row constant, m_ref the row's reference (log2 units)
  const float c = a.scale_log2;
  const T* Qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * a.Lq * D;
  const char* Kg = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.k) + (size_t)bh * a.Lk * D);
  const char* Vg = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.v) + (size_t)bh * a.Lk * D);
  const int wg_pos_max = a.q_pos_offset + min(q0 + BQ, a.Lq) - 1;
  const int ck = a.clip_k;

  // ---- the first key/value tile copies go out before anything else when
  // their keys are known at launch (no per-sequence valid length, or an
  // unsplit key range, which starts at key 0), so they overlap every load of
  // the prologue.  Tiles past a short valid length are read for nothing and
  // never used (the loop's in-order waits only wait longer).  A split key
  // range under a valid length starts at a tile that depends on it, so its
  // first copies wait for it.
  const int causal_end = a.causal ? min(a.Lk, wg_pos_max + 1) : a.Lk;
  // Key tile of loop step r over the tile range [kb, ke).  ALiBi visits the
  // tiles nearest the diagonal first: from the tile of the workgroup's
  // middle query position down to kb, then upward from there; under a
  // distance penalty a row's scores then mostly fall from tile to tile, so
  // its reference rarely has to move.  The other kinds run upward.
  const int wg_mid_tile = ((a.q_pos_offset + q0 + wg_pos_max) >> 1) >> 6;  // floor division
  static_assert(kBK == 64, "wg_mid_tile divides by 64");
  auto tile_at = [&](const int r, const int kb, const int ke) -> int {
    if constexpr (KIND == 3) {
      const int kc = min(max(wg_mid_tile, kb), ke - 1);
      return r <= kc - kb ? kc - r : kb + r;
    }
    return kb + r;
  };
  // ALiBi's order needs the exact tile range, so its early copies wait for
  // a per-sequence valid length
  // (with a key split, a valid length moves the halves' boundary, so the
  // early copies wait for it too)
  const bool early_copies =
      (KIND == 3 || KS == 2) ? a.kv_valid_len == nullptr
                             : (a.n_splits == 1 || a.kv_valid_len == nullptr);
  // Only the first tile goes out here; the others follow the register loads
  // below.  Memory loads retire in order, so a wait for those registers
  // would otherwise also wait for every tile issued before them (with four
  // stages, three tiles of every workgroup at once at kernel start).
  int early_n0 = 0, early_beg0 = 0;
  if (early_copies) {
    const int n_kt0 = (causal_end + kBK - 1) / kBK;
    const int per0 = (n_kt0 + a.n_splits - 1) / a.n_splits;
    early_beg0 = min(n_kt0, split * per0);
    int early_end0 = min(n_kt0, early_beg0 + per0);
    half_range(early_beg0, early_end0);
    early_n0 = early_end0 - early_beg0;
    if (early_n0 > 0) {
      Dma dma;
      dma.init(wq, lane);
      dma.issue(Kg, Vg, a.Lk, tile_at(0, early_beg0, early_beg0 + early_n0) * kBK, sbase,
                L.tile_bytes, wq, lane);
    }
  }

  // ---- register loads (valid length, Q fragments, the kind's small tables)
  const int kv_valid = seq_len >= 0 ? seq_len
                       : (a.kv_valid_len ? __builtin_amdgcn_readfirstlane(a.kv_valid_len[b]) : a.Lk);
  QFrag qf[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (qrow[qb] < a.Lq) qf[qb].load(Qg + (size_t)qrow[qb] * D, hh);
    else qf[qb].zero();
  }
  // T5: distinct offset-table entries per thread fetched early (the table
  // holds lut_stride + 3 distinct offsets; 4 x 64 x NW covers 1024 of them
  // with 4 waves)
  constexpr int LUT_EARLY = 4;
  float lut_early[LUT_EARLY];
  float bias_left = 0.f, bias_right = 0.f;          // T5 saturated buckets / scale
  constexpr int SHAW_RB = 3;                          // blocks of 32 a_K rows (k <= 32)
  TableFrag<BF, D> krow[KIND == 1 ? SHAW_RB : 1];     // Shaw a_K rows / DeBERTa Kr rows
  // Shaw bf16: a_V rows 1 .. 2k-1 in 16-byte chunks, read row-major
  // (coalesced) here and written transposed into LDS by the prologue
  constexpr int AVT_CH = (63 * (D / 8) + 64 * NW - 1) / (64 * NW);
  bf16x8 avt_ch[KIND == 1 && BF ? AVT_CH : 1];
  // Shaw: a_V rows 0 and 2k for this wave's epilogue copy, element e = lane
  // + 64 * c of [row 0 | row 2k] (read with the other register loads, so no
  // later step waits for memory)
  constexpr int AVE = (2 * D + 63) / 64;
  T av_end[KIND == 1 ? AVE : 1];
  if constexpr (KIND == 0) {
    const float* tab = reinterpret_cast<const float*>(a.table);
#pragma unroll
    for (int i = 0; i < LUT_EARLY; ++i) {
      const int x = tid + i * 64 * NW;
      lut_early[i] = 0.f;
      if (x < a.lut_n) {
        const int bk = t5_bucket_dev(a.lut_lo + x, a.t5_slots, a.t5_exact, a.t5_bidir, a.t5_nthr, a.t5_thr);
        lut_early[i] = tab[bk * a.H + h];
      }
    }
    const int bl = t5_bucket_dev(-(1 << 30), a.t5_slots, a.t5_exact, a.t5_bidir, a.t5_nthr, a.t5_thr);
    const int br = t5_bucket_dev(1 << 30, a.t5_slots, a.t5_exact, a.t5_bidir, a.t5_nthr, a.t5_thr);
    const float inv_scale = 1.f / a.scale;
    bias_left = tab[bl * a.H + h] * inv_scale;
    bias_right = tab[br * a.H + h] * inv_scale;
  } else if constexpr (KIND == 1) {
    const T* ak = reinterpret_cast<const T*>(a.table);
    const int nrow = 2 * ck + 1;
#pragma unroll
    for (int rb = 0; rb < SHAW_RB; ++rb)
      if (rb * 32 < nrow) krow[rb].load(ak + (size_t)min(rb * 32 + lq, nrow - 1) * D, hh);
    if constexpr (BF) {
      const bf16* av = reinterpret_cast<const bf16*>(a.table2);
      const int nch = (2 * ck - 1) * (D / 8);
#pragma unroll
      for (int c = 0; c < AVT_CH; ++c) {
        const int e = tid + c * 64 * NW;
        avt_ch[c] = bf16x8{};
        if (e < nch) avt_ch[c] = *reinterpret_cast<const bf16x8*>(av + (size_t)(e / (D / 8) + 1) * D + 8 * (e % (D / 8)));
      }
    }
    {
      const T* av = reinterpret_cast<const T*>(a.table2);
#pragma unroll
      for (int c = 0; c < AVE; ++c) {
        const int e = lane + 64 * c;
        av_end[c] = e < 2 * D ? av[(size_t)(e < D ? 0 : 2 * ck) * D + (e % D)] : (T)0.f;
      }
    }
  } else if constexpr (KIND == 2) {
    const T* kr = reinterpret_cast<const T*>(a.table);
    const int u = (lq == 1) ? 2 * ck - 1 : 0;
    krow[0].load(kr + ((size_t)u * a.H + h) * D, hh);
  }
  // ALiBi: the head's slope in raw-score units per unit of distance, and the
  // in-block key term of blocks whose keys all lie at or before every query
  // (side 0: -slope * (key - the block's first key)) or at or after it
  // (side 1: +slope * (key - first key)); the rest of the bias is a per-row
  // constant of the block
  float alibi_s = 0.f;
  KeyConst<BF> alibi_kc;
  if constexpr (KIND == 3) {
    alibi_s = reinterpret_cast<const float*>(a.table)[h] / a.scale;
    alibi_kc.set(-alibi_s * (float)lq, alibi_s * (float)lq, hh);
  }
  const int kv_lim = max(0, min(a.Lk, kv_valid));
  const int kv_end = min(kv_lim, causal_end);
  const int n_kt = kv_end > 0 ? (kv_end + kBK - 1) / kBK : 0;
  const int per_split = (n_kt + a.n_splits - 1) / a.n_splits;
  int kt_begin = min(n_kt, split * per_split);
  int kt_end = min(n_kt, kt_begin + per_split);
  // loop steps of the workgroup (every wave runs them all and meets every
  // tile barrier; with a key split, half 1 idles after its last tile when it
  // has one tile fewer than half 0)
  const int n_steps = KS == 2 ? (kt_end - kt_begin + 1) >> 1 : kt_end - kt_begin;
  half_range(kt_begin, kt_end);
  const int n_my = kt_end - kt_begin;

  // ---- the rest of the early tile copies, once the registers' loads (and
  // the first tile) have landed
  if constexpr (NS > 2) {
    if (early_copies && early_n0 > 1) {
      wait_vmcnt<0>();
      Dma dma;
      dma.init(wq, lane);
#pragma unroll
      for (int s = 1; s < AHEAD; ++s)
        if (s < early_n0)
          dma.issue(Kg, Vg, a.Lk, tile_at(s, early_beg0, early_beg0 + early_n0) * kBK,
                    sbase + s * L.stage_bytes, L.tile_bytes, wq, lane);
    }
  }

  // ---- per-kind prologue (LDS tables) ---------------------------------------
  float shaw_right[QB];                              // Shaw: q.(a_K[2k] - a_K[0])
  float shaw_base[QB];                               // Shaw: q.a_K[0], left out of every logit
  float crow_lo[QB], crow_hi[QB];                    // DeBERTa: q.Kr[0], q.Kr[2k-1]
  float* arel = nullptr; // Shaw: this wave's relative-key logits
  T* wbins = nullptr;    // Shaw: this wave's bin rows, [32 * QB][bin slots]
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) shaw_right[qb] = shaw_base[qb] = crow_lo[qb] = crow_hi[qb] = 0.f;

  if constexpr (KIND == 0) {
    // four copies of bias[offset]/scale, copy c shifted by c entries:
    // entry x of the table goes to copy c at position x - c
    const float inv_scale = 1.f / a.scale;
    const int nx = L.lut_stride + 3;
    auto put4 = [&](const int x, const float val) {
#pragma unroll
      for (int cpy = 0; cpy < 4; ++cpy) {
        const int y = x - cpy;
        if (y >= 0 && y < L.lut_stride) relf[cpy * L.lut_stride + y] = val;
      }
    };
#pragma unroll
    for (int i = 0; i < LUT_EARLY; ++i) {
      const int x = tid + i * 64 * NW;
      if (x < nx) put4(x, lut_early[i] * inv_scale);
    }
    const float* tab = reinterpret_cast<const float*>(a.table);
    for (int x = tid + LUT_EARLY * 64 * NW; x < nx; x += 64 * NW) {
      float val = 0.f;
      if (x < a.lut_n) {
        const int bk = t5_bucket_dev(a.lut_lo + x, a.t5_slots, a.t5_exact, a.t5_bidir, a.t5_nthr, a.t5_thr);
        val = tab[bk * a.H + h] * inv_scale;
      }
      put4(x, val);
    }
  } else if constexpr (KIND == 1) {
    // arel[row][r] = q.a_K[r] - q.a_K[0], r = 0..2k, by MFMA over blocks of
    // 32 table rows; subtracting the r = 0 value is softmax-neutral and
    // makes every key beyond -k contribute exactly zero.
    arel = reinterpret_cast<float*>(smem + L.rel_off + wave * L.arel_wave_bytes);
    wbins = reinterpret_cast<T*>(smem + L.rel_off + L.wscr_off + wave * L.wscr_wave_bytes);
    const int nrow = 2 * ck + 1;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float base0 = 0.f;
#pragma unroll
      for (int rb = 0; rb < SHAW_RB; ++rb) {
        if (rb * 32 >= nrow) break;
        const f32x16 acc = mma_frag0<BF, D>(krow[rb], qf[qb]);
        if (rb == 0) base0 = __shfl(acc[0], lq);  // row 0 sits in lane lq, register 0
        if (rb == 0) shaw_base[qb] = base0;
        // table rows past 2k land in the row's padding slot 2k+1
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = min(rb * 32 + acc_row(i, hh), nrow);
          arel[(32 * qb + lq) * L.arel_stride + r] = acc[i] - base0;
        }
      }
    }
    // bin rows start (and are kept) at zero; this lane clears its half of
    // each of its rows
    {
      const int nbin = shaw_bin_slots(ck);
      constexpr int EPV = 16 / sizeof(T);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        f32x4* zp = reinterpret_cast<f32x4*>(wbins + (32 * qb + lq) * shaw_bin_stride(ck, (int)sizeof(T)) + hh * (nbin / 2));
        for (int x = 0; x < nbin / 2 / EPV; ++x) zp[x] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    // this wave's copy of a_V rows 0 and 2k, read by its epilogue
    {
      T* ends = reinterpret_cast<T*>(smem + L.rel_off + L.avend_off) + wave * 2 * D;
#pragma unroll
      for (int c = 0; c < AVE; ++c)
        if (lane + 64 * c < 2 * D) ends[lane + 64 * c] = av_end[c];
    }
    wave_lds_fence();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) shaw_right[qb] = arel[(32 * qb + lq) * L.arel_stride + 2 * ck];
    if constexpr (BF) {
      // a_V^T for the in-window bins: avt[d][s] = a_V[s][d], s = 1 .. 2k-1
      const int nb = shaw_bin_slots(ck);
      T* avt = reinterpret_cast<T*>(smem + L.rel_off + L.avt_off);
      const int nch = (2 * ck - 1) * (D / 8);
#pragma unroll
      for (int c = 0; c < AVT_CH; ++c) {
        const int e = tid + c * 64 * NW;
        if (e < nch) {
          const int r = e / (D / 8), d0 = 8 * (e % (D / 8));
#pragma unroll
          for (int q = 0; q < 8; ++q) avt[(d0 + q) * nb + r + 1] = avt_ch[c][q];
        }
      }
      // slot 0 and slots 2k .. nb-1 (the out-of-window slots and the padding)
      // meet zero rows
      const int npad = nb - 2 * ck;
      for (int e = tid; e < D * (npad + 1); e += 64 * NW) {
        const int dd = e / (npad + 1), x = e % (npad + 1);
        avt[dd * nb + (x == 0 ? 0 : 2 * ck - 1 + x)] = (T)0.f;
      }
    }
  } else if constexpr (KIND == 2) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const f32x16 acc = mma_frag0<BF, D>(krow[0], qf[qb]);
      crow_lo[qb] = __shfl(acc[0], lq);
      crow_hi[qb] = __shfl(acc[1], lq);
    }
    if constexpr (BF) {
      // the head's clipped Qr rows Qr[0] and Qr[2k-1], one 16-byte chunk per
      // thread (read after the first tile's barrier)
      constexpr int NCH = D / 8;
      if (tid < 2 * NCH) {
        const int row = tid < NCH ? 0 : 2 * ck - 1, c8 = tid % NCH;
        const T* src = reinterpret_cast<const T*>(a.table2) + ((size_t)row * a.H + h) * D + 8 * c8;
        *reinterpret_cast<f32x4*>(smem + L.rel_off + L.qr_off + (tid / NCH) * D * 2 + 16 * c8) =
            *reinterpret_cast<const f32x4*>(src);
      }
    }
  }

  // ---- start streaming the first key tiles of a split key range ------------
  if (!early_copies) {
    Dma dma;
    dma.init(wq, lane);
#pragma unroll
    for (int s = 0; s < AHEAD; ++s)
      if (s < n_my)
        dma.issue(Kg, Vg, a.Lk, tile_at(s, kt_begin, kt_end) * kBK, sbase + s * L.stage_bytes,
                  L.tile_bytes, wq, lane);
  }

  // ---- band-row ring (DeBERTa Kr, Transformer-XL E): ring index
  // v = u - ring_c0 of the row index before clamping, u = query - key + k
  // (DeBERTa's clip-and-shift) or u = query - key (TXL's distance).  Tile kt
  // reads v in [-64 kt, 319 - 64 kt]; slot = v mod kRingRows holds the
  // clamped row of this head, chunk c of slot s at byte s*128 +
  // 16*(c ^ swz_k<8>(s)).
  constexpr bool KR_RING = band_ring(KIND, BF, D, NW);
  const int ring_k = KIND == 2 ? ck : 0;                     // u - (query - key)
  const int ring_rows = KIND == 2 ? 2 * ck : ck;             // rows of the table
  const int ring_c0 = a.q_pos_offset + q0 + ring_k - 63;
  char* ring = smem + L.rel_off + L.ring_off;
  auto ring_slot = [&](const int v) -> int {
    const int m = v % kRingRows;
    return m < 0 ? m + kRingRows : m;
  };
  // copy the 64 rows v0 .. v0+63 (v0 a multiple of 64): 8 copies of 8 rows,
  // copy `ins` issued by wave ins % NW
  auto ring_fill = [&](const int v0, const int ln) {
    if constexpr (KR_RING) {
      const T* kr = reinterpret_cast<const T*>(a.table);
      const int s0 = ring_slot(v0);
#pragma unroll
      for (int ins = wave; ins < 8; ins += NW) {
        const int row = 8 * ins + (ln >> 3), slot = ln & 7;
        const int u = min(max(ring_c0 + v0 + row, 0), ring_rows - 1);
        const int chunk = slot ^ swz_k<8>(row);
        lds_dma16(kr + ((size_t)u * a.H + h) * D + 8 * chunk, ring + (s0 + 8 * ins) * 128);
      }
    }
  };
  if constexpr (KR_RING) {
    if (n_my > 0) {
#pragma unroll
      for (int g = 0; g < 5; ++g) ring_fill(-64 * kt_begin + 64 * g, lane);
    }
  }

  // ---- running state ------------------------------------------------------
  // m_ref: the row's reference max in log2 units (both lane halves agree);
  // -inf until the row has seen a visible key.  p = exp2(s - m_ref) is used
  // as is while every block keeps its lane sums below kSumLimit.
  f32x16 o[QB][NDB];
  float m_ref[QB], l_run[QB], lr_run[QB], win_run[QB];
  // Transformer-XL (encoding rows from the LDS ring): a wave visits its key
  // blocks in ascending order, so the first half of a block's band (distances
  // T0 .. T0+31) is the second half of the next block's; it stays in
  // registers, tagged with its T0
  constexpr bool TXL_CARRY = KIND == 4 && KR_RING;
  f32x16 txl_half[1];
  int txl_t0 = -(1 << 30);  // no block yet
  // DeBERTa (same kernel): the first half of the Qr rows of the wave's next
  // key block (distances T0 - 32 ..), requested right after this block's
  // band gathers, so its latency hides behind this block's softmax and
  // P V; tagged with the T0 of the block it serves
  constexpr bool QR_NEXT = KIND == 2 && KR_RING;
  TableFrag<BF, D> qr_next;
  int qr_t0 = -(1 << 30);
  // ... and this block's first half, the next block's second half (the
  // next block's T0 is this one's minus 32), tagged with that T0.  Every
  // near block after the first thus reads one new half from memory, early
  // (requested once the block's band gathers are done, which leaves the
  // eight-wave kernel 7 registers in scratch instead of 21 at the same
  // speed); measured on DeBERTa k=512 it runs 1.5% faster than reading the
  // second half at the block's start.
  TableFrag<BF, D> qr_carry;
  int qr_ct0 = -(1 << 30);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[qb][db] = {};
    m_ref[qb] = NEG_INF;
    l_run[qb] = 0.f;         // this lane's partial row sum
    lr_run[qb] = 0.f;        // Shaw: partial mass of keys at offset >= k
    win_run[qb] = 0.f;       // Shaw: partial mass of keys inside the clip window
  }

  // Shaw: apply the pending bins of query block qb (o += a_V^T W^T), then
  // clear them.  Wave-uniform; a no-op when no bin was written since the
  // last flush.
  bool bins_dirty[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) bins_dirty[qb] = false;
  auto flush_bins = [&](const int qb) {
    if constexpr (KIND == 1) {
      if (!bins_dirty[qb]) return;
      bins_dirty[qb] = false;
      const int ln = opaque_lane();
      const int lq = ln & 31, hh = ln >> 5;
      const int nbin = shaw_bin_slots(ck);
      T* wrow = wbins + (32 * qb + lq) * shaw_bin_stride(ck, (int)sizeof(T));
      wave_lds_fence();
      // the mass inside the window, summed from the bins themselves (the
      // two out-of-window slots left out)
      float win = 0.f;
      if constexpr (BF) {
        const bf16* avt = reinterpret_cast<const bf16*>(smem + L.rel_off + L.avt_off);
        for (int cb = 0; cb < nbin / 16; ++cb) {
          const bf16x8 wf = *reinterpret_cast<const bf16x8*>(wrow + 16 * cb + 8 * hh);
          win = sum_bf16x8(wf, win);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(avt + (32 * db + lq) * nbin + 16 * cb + 8 * hh);
            o[qb][db] = mma_bf16(vf, wf, o[qb][db]);
          }
        }
        if (hh == 0) win -= (float)wrow[0] + (float)wrow[2 * ck];
      } else {
        const float* av = reinterpret_cast<const float*>(a.table2);
        for (int cb = 0; cb < nbin / 2; ++cb) {
          const int rr = 2 * cb + hh;
          const bool in_win = rr >= 1 && rr < 2 * ck;
          const float wv = wrow[rr];
          win += in_win ? wv : 0.f;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const float vv = in_win ? av[(size_t)rr * D + 32 * db + lq] : 0.f;
            o[qb][db] = mma_f32(vv, wv, o[qb][db]);
          }
        }
      }
      win_run[qb] += win;
      wave_lds_fence();
      constexpr int EPV = 16 / sizeof(T);
      f32x4* zp = reinterpret_cast<f32x4*>(wrow + hh * (nbin / 2));
      for (int x = 0; x < nbin / 2 / EPV; ++x) zp[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // Tile classes (wave-uniform):
  //   0: every block far from the diagonal band (the relative term is a
  //      per-row constant, plus a per-key constant for DeBERTa; ALiBi: every
  //      key on one side of every query, the bias linear in the key), no
  //      mask;
  //   1: T5, every block inside the bucket table's range, no mask;
  //   2: anything else (band terms, masks, Shaw bins);
  //   3: nothing to do for this wave (past its causal reach).
  // Runs of equal class go through a loop of their own, so the lean loops
  // are not burdened with the registers of the general one.
  auto tile_class = [&](const int r) -> int {
    if (KS == 2 && r >= n_my) return 3;  // this half has no tile at step r
    const int k0 = tile_at(r, kt_begin, kt_end) * kBK;
    if (!wave_active || (a.causal && k0 > pw_max_real)) return 3;
    bool far_all = true, near_all = true;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int pq_min = pw_min + 32 * qb, pq_max = pq_min + 31;
      const int omin = k0 - pq_max, omax = k0 + kBK - 1 - pq_min;  // key - query
      bool far;
      if constexpr (KIND == 0) far = omax <= -a.t5_lsat || omin >= a.t5_rsat;
      else if constexpr (KIND == 1) far = omin >= ck || omax <= -ck;
      else if constexpr (KIND == 2) far = -omax >= ck || -omin <= -ck;
      else if constexpr (KIND == 3) far = omax <= 0 || omin >= 0;  // ALiBi: every key on one side
      else far = false;  // Transformer-XL: the encodings are never clipped
      far_all = far_all && far;
      near_all = near_all && !far;
    }
    // no block of the tile touches the causal diagonal or the end of the keys
    const bool unmasked = !(a.causal && k0 + kBK - 1 > pw_min) && (k0 + kBK <= kv_lim);
    if (unmasked && far_all) return 0;
    if (KIND == 0 && unmasked && near_all) return 1;
    return 2;
  };

  auto run_tile = [&](auto cls_tag, const int r, const int ln) {
    constexpr int CLS = decltype(cls_tag)::value;
    // per-lane values, from the loop's own lane index (see opaque_lane)
    const int lane = ln, lq = ln & 31, hh = ln >> 5;
    int pos[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) pos[qb] = pw_min + 32 * qb + lq;
    KOffsets<BF, D> ko;
    ko.init(lane);
    const int kt = tile_at(r, kt_begin, kt_end);
    if constexpr (PAIR) {
      // at even r: tiles r and r+1 landed for every wave, every wave is
      // done with tiles r-2 and r-1
      if ((r & 1) == 0) {
        wait_vmcnt<0>();
        __syncthreads();
      }
    } else {
      if constexpr (NS >= 3 && EVEN_LOADS) {
        // tiles newer than r that may still be in flight: min(NS - 2, n_my - 1 - r)
        const int newer = min(NS - 2, n_my - 1 - r);
        if (newer >= 1) wait_vmcnt<LPW>();
        else wait_vmcnt<0>();
      } else {
        wait_vmcnt<0>();
      }
    }
    const int k0 = kt * kBK;
    // The tile's row constants from global memory, requested before the
    // workgroup barrier so that their latency overlaps the wait for the other
    // waves (they are first read after it).
    //   per-key constants of the tile's keys: DeBERTa k_j.Qr[0] / k_j.Qr[2k-1]
    //   (clipped blocks), Transformer-XL u.k_j;
    //   Transformer-XL v.E[r] of the band rows of the tile's blocks: block kb
    //   of one query block reads the distance rows T0 + 32 tb + m, T0 = T0t -
    //   32 kb (tb = 0, 1; m = lane), so entry t = 1 - kb + tb holds rows T0t +
    //   32 (t - 1) + m (hidden negative distances read row 0)
    constexpr bool KEYC = KIND == 4 || (KIND == 2 && !BF);  // per-key constants from the pre-pass
    KeyConst<BF> kc[KEYC ? NKB : 1];
    // DeBERTa bfloat16: q.k_j + k_j.Qr[side row] for a block whose offsets
    // are all clipped to one side: K (A) times Q^T (B) on top of K times the
    // side's Qr row in every column (B, read from LDS)
    auto clipped_scores = [&](const TableFrag<BF, D>& kf, const int qb, const int side) -> f32x16 {
      TableFrag<BF, D> rf;
      rf.load(reinterpret_cast<const T*>(smem + L.rel_off + L.qr_off) + side * D, hh);
      return mma_frag<BF, D>(kf, qf[qb], mma_frag0<BF, D>(kf, rf));
    };
    KeyConst<BF> venc[KIND == 4 ? NKB + 1 : 1];
    if constexpr (KEYC && CLS != 3) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) kc[kb].load(a.colc, (size_t)bh * a.Lk, min(k0 + 32 * kb + lq, a.Lk - 1), hh);
    }
    if constexpr (KIND == 4 && CLS != 3) {
      static_assert(QB == 1, "Transformer-XL runs one query block per wave");
      const int T0t = pw_min - k0 - 31;
#pragma unroll
      for (int t = 0; t <= NKB; ++t)
        venc[t].load(a.colc2, (size_t)h * ck, min(max(T0t + 32 * (t - 1) + lq, 0), ck - 1), hh);
    }
    if constexpr (!PAIR) __syncthreads();  // tile r landed for every wave; every wave is done with tile r-1
    // The constants above are the only memory reads still in flight: wait
    // for them here, before the copies below are issued.  Copies go through
    // inline assembly the compiler does not track, and its own wait before
    // the first use of the constants would count only its loads and so also
    // wait for those copies (measured on Transformer-XL with memory: 303 ->
    // 296 us)
    if constexpr (KEYC && CLS != 3) wait_vmcnt<0>();
    // Lean tiles in bfloat16 run as a software pipeline (below); T5 with two
    // query blocks per wave or 128-wide heads keeps the step loop (the
    // pipeline's extra live registers spill there).  Shaw's tiles with
    // blocks inside the clip window run in the pipeline too (64-wide heads):
    // their blocks take the relative-key logits as the accumulator's
    // initial value, the masks, and the bins after the softmax
    constexpr bool SHAW_NEAR_PIPE = KIND == 1 && CLS == 2 && BF && QB == 1 && D <= 64;
    constexpr bool PIPE = (CLS != 2 || SHAW_NEAR_PIPE) && CLS != 3 && BF && KIND != 4 &&
                          !(KIND == 0 && (QB == 2 || D > 64));
    // copies of the tile NS - 1 ahead into the stage of tile r - 1 (free:
    // every wave has passed the barrier above)
    auto issue_next = [&]() {
      if constexpr (PAIR) {
        if ((r & 1) == 0 && r + 2 < n_my) {
          constexpr bool KEEP = QB == 1 && D <= 64;
          Dma dma;
          dma.init(wq, KEEP ? lane : opaque_lane());
#pragma unroll
          for (int t = 2; t < 4; ++t)
            if (r + t < n_my)
              dma.issue(Kg, Vg, a.Lk, tile_at(r + t, kt_begin, kt_end) * kBK,
                        sbase + stage_of(r + t) * L.stage_bytes, L.tile_bytes, wq, lane);
        }
      } else if (r + NS - 1 < n_my) {
        // copy offsets: kept in registers across tiles with one query block
        // per wave; recomputed from a fresh lane id where registers are
        // short (two query blocks, 128-wide heads, DeBERTa's four-wave
        // variant)
        constexpr bool KEEP = QB == 1 && D <= 64 && !(KIND == 2 && NW == 4);
        Dma dma;
        dma.init(wq, KEEP ? lane : opaque_lane());
        dma.issue(Kg, Vg, a.Lk, tile_at(r + NS - 1, kt_begin, kt_end) * kBK,
                  sbase + stage_of(r + NS - 1) * L.stage_bytes, L.tile_bytes, wq, lane);
      }
    };
    // a pipelined tile issues them after its first scores, so that its
    // first MFMAs do not wait for the copies' address arithmetic
    if constexpr (!PIPE) issue_next();
    // the next tile's 64 new Kr rows (they replace rows no tile reads again)
    if constexpr (KR_RING) {
      if (r + 1 < n_my) ring_fill(-64 * (kt + 1), lane);
    }
    if constexpr (CLS == 3) return;
    const char* ktile = sbase + stage_of(r) * L.stage_bytes;
    const char* vtile = ktile + L.tile_bytes;

    // ---- the tile's query blocks (wave-uniform) ----
    float b_tile[QB];  // per-row constant of the tile's far blocks (raw score units)
    bool near[QB], far_right[QB];
    int deb_side[QB];  // DeBERTa / ALiBi: 0 far-left tile, 1 far-right tile, -1 mixed
    const float* lutp[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      b_tile[qb] = 0.f;
      near[qb] = far_right[qb] = false;
      deb_side[qb] = -1;
      lutp[qb] = nullptr;
      const int pq_min = pw_min + 32 * qb, pq_max = pq_min + 31;
      const int omin = k0 - pq_max, omax = k0 + kBK - 1 - pq_min;  // key - query
      if constexpr (KIND == 0) {
        if (omax <= -a.t5_lsat) b_tile[qb] = bias_left;
        else if (omin >= a.t5_rsat) b_tile[qb] = bias_right;
        else {
          near[qb] = true;
          const int x0 = k0 - pos[qb] - a.lut_lo;  // table index of this lane's first key
          const int cp = x0 & 3;
          lutp[qb] = relf + cp * L.lut_stride + (x0 - cp);
        }
      } else if constexpr (KIND == 1) {
        if (omin >= ck) {
          b_tile[qb] = shaw_right[qb];
          far_right[qb] = true;
        } else if (omax > -ck) {
          near[qb] = true;
        }
      } else if constexpr (KIND == 2) {
        if (-omax >= ck) { deb_side[qb] = 0; b_tile[qb] = crow_hi[qb]; }       // every query - key >= k
        else if (-omin <= -ck) { deb_side[qb] = 1; b_tile[qb] = crow_lo[qb]; } // every query - key <= -k
      } else if constexpr (KIND == 3) {
        if (omax <= 0) deb_side[qb] = 0;       // every key at or before every query
        else if (omin >= 0) deb_side[qb] = 1;  // every key at or after every query
      }
    }
    // exponent offsets c*b - m_ref of the tile's blocks
    float off[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) off[qb] = ref_offset(c * b_tile[qb], m_ref[qb]);

    // One step of 32 keys (block kb of the tile) for the query blocks in the
    // bit mask QM: scores, softmax, P V.  A K fragment and a V fragment read
    // from LDS feed every query block of the step.  Class 2 runs one query
    // block per step so that fewer values are live.
    auto step = [&](auto qm_tag, const int kb) {
      constexpr int QM = decltype(qm_tag)::value;
      const int j0 = k0 + 32 * kb;
      // T5 / ALiBi: a block of a mixed tile whose keys are all hidden from
      // every row of its query blocks (past the causal diagonal or the valid
      // keys) would only add zeros: skip it (causal ALiBi, 4096 tokens: 172
      // -> 168 us; the band kinds' code ran as fast or slower with the
      // branch, DeBERTa 292 -> 297 us, Transformer-XL 293 -> 302 us)
      if constexpr (CLS == 2 && (KIND == 0 || KIND == 3)) {
        bool live = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          if ((QM >> qb) & 1) live = live || ((!a.causal || j0 <= pw_min + 32 * qb + 31) && j0 < kv_lim);
        if (!live) return;
      }

      // DeBERTa, per block: 0 / 1 every offset clipped on one side, -1 band
      auto deb_block_side = [&](const int qb) -> int {
        const int pq_min = pw_min + 32 * qb, pq_max = pq_min + 31;
        const int tmin = pq_min - (j0 + 31), tmax = pq_max - j0;  // query - key over the block
        return tmin >= ck ? 0 : (tmax <= -ck ? 1 : -1);
      };
      // ALiBi, per block: 0 / 1 every key on one side, -1 across the diagonal
      auto alibi_side = [&](const int qb) -> int {
        if (CLS == 0) return deb_side[qb];
        const int pq_min = pw_min + 32 * qb;
        return j0 + 31 <= pq_min ? 0 : (j0 >= pq_min + 31 ? 1 : -1);
      };
      // per-row constant of this block (raw score units)
      auto b_block = [&](const int qb) -> float {
        if constexpr (KIND == 2) {
          if (CLS == 2) {
            const int side = deb_block_side(qb);
            return side == 0 ? crow_hi[qb] : (side == 1 ? crow_lo[qb] : 0.f);
          }
        }
        if constexpr (KIND == 3) {
          // slope * |key - query| = slope * (query - j0) - slope * (key - j0)
          // left of the diagonal, the negation of both terms right of it
          const int side = alibi_side(qb);
          const float dist = (float)(pos[qb] - j0);
          return side == 0 ? alibi_s * dist : (side == 1 ? -alibi_s * dist : 0.f);
        }
        return b_tile[qb];
      };

      // raw scores of query block qb: relative term (except a per-row
      // constant) + q.k; hidden keys -inf
      auto scores = [&](const int qb, const TableFrag<BF, D>& kf) -> f32x16 {
        const int pq_min = pw_min + 32 * qb;
        f32x16 s;
        if constexpr (KIND == 0) {
          if (CLS == 1 || (CLS == 2 && near[qb])) {
            f32x16 init;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 x = *reinterpret_cast<const f32x4*>(lutp[qb] + 32 * kb + 8 * g + 4 * hh);
              init[4 * g + 0] = x[0]; init[4 * g + 1] = x[1];
              init[4 * g + 2] = x[2]; init[4 * g + 3] = x[3];
            }
            s = mma_frag<BF, D>(kf, qf[qb], init);
          } else {
            s = mma_frag0<BF, D>(kf, qf[qb]);
          }
        } else if constexpr (KIND == 1) {
          if (CLS == 2 && near[qb]) {
            const float* ar = arel + (32 * qb + lq) * L.arel_stride;
            const int obase = j0 + 4 * hh - pos[qb];  // offset of register 0's key
            f32x16 init;
#pragma unroll
            for (int i = 0; i < 16; ++i) init[i] = (float)ar[shaw_row_dev(obase + acc_row(i, 0), ck)];
            s = mma_frag<BF, D>(kf, qf[qb], init);
          } else {
            s = mma_frag0<BF, D>(kf, qf[qb]);
          }
        } else if constexpr (KIND == 3) {
          const int side = alibi_side(qb);
          if (side >= 0) {
            s = mma_keyconst<BF>(alibi_kc, side, hh);
            s = mma_frag<BF, D>(kf, qf[qb], s);
          } else {
            // a block across the diagonal: the whole bias, per element
            const int obase = j0 + 4 * hh - pos[qb];  // offset of register 0's key
            f32x16 init;
#pragma unroll
            for (int i = 0; i < 16; ++i) init[i] = alibi_s * (float)abs(obase + acc_row(i, 0));
            s = mma_frag<BF, D>(kf, qf[qb], init);
          }
        } else if constexpr (KIND == 4) {
          // (q + v).E[i - j] for the block's 63 distances by MFMA (rows
          // E[T0 + m], columns = queries), stored [query][m] in the wave's
          // LDS tile and read back along each query's diagonal
          // the band's MFMAs and stores at raised wave priority in the
          // eight-wave kernel (see DeBERTa below; Transformer-XL with
          // memory 288.4 -> 278.3 us)
          if constexpr (KR_RING) __builtin_amdgcn_s_setprio(2);
          float* band = relf + wave * L.deb_wave_floats;
          const T* enc = reinterpret_cast<const T*>(a.table);
          const int T0 = pq_min - j0 - 31;  // band index m <-> query - key = T0 + m
          // half tb: v.E[T0 + 32 tb + m] (the position bias, a per-row
          // constant of the band) + q.E[T0 + 32 tb + m]
          auto band_half = [&](const int tb, const TableFrag<BF, D>& ef) -> f32x16 {
            return mma_frag<BF, D>(ef, qf[qb], mma_keyconst<BF>(venc[1 - kb + tb], 0, hh));
          };
          f32x16 half[2];
          if constexpr (TXL_CARRY) {
            // the previous block's first half is this block's second half
            const bool carried = txl_t0 == T0 + 32;
            {
              TableFrag<BF, D> ef;
              ef.load_lds(ring + ring_slot(T0 - ring_c0) * 128, ko.k);
              half[0] = band_half(0, ef);
            }
            if (carried) {
              half[1] = txl_half[0];
            } else {
              TableFrag<BF, D> ef;
              ef.load_lds(ring + ring_slot(T0 + 32 - ring_c0) * 128, ko.k);
              half[1] = band_half(1, ef);
            }
            txl_half[0] = half[0];
            txl_t0 = T0;
          } else {
            TableFrag<BF, D> ef[2];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {  // negative distances are hidden keys: any row serves
              if constexpr (KR_RING) {
                ef[tb].load_lds(ring + ring_slot(T0 + 32 * tb - ring_c0) * 128, ko.k);
              } else {
                ef[tb].load(enc + ((size_t)min(max(T0 + 32 * tb + lq, 0), ck - 1) * a.H + h) * D, hh);
              }
            }
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) half[tb] = band_half(tb, ef[tb]);
          }
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            float* dst = band + lq * kCbandStride + 32 * tb + 4 * hh;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 x = {half[tb][4 * g], half[tb][4 * g + 1], half[tb][4 * g + 2], half[tb][4 * g + 3]};
              *reinterpret_cast<f32x4*>(dst + 8 * g) = x;
            }
          }
          if constexpr (KR_RING) __builtin_amdgcn_s_setprio(0);
          wave_lds_fence();
          f32x16 init;
          {
            const float* crow = band + lq * (kCbandStride + 1) + 31;
#pragma unroll
            for (int i = 0; i < 16; ++i) init[i] = crow[-acc_row(i, hh)];
          }
          wave_lds_fence();  // the next block overwrites the tile
          // + u.k_j (the content bias, a per-key constant) + q.k_j
          s = mma_frag<BF, D>(kf, qf[qb], mma_keyconst<BF>(kc[kb], 0, hh, init));
        } else {
          const int side = CLS == 0 ? deb_side[qb] : deb_block_side(qb);
          if (side >= 0) {
            // k_j.Qr[0] (side 0) or k_j.Qr[2k-1] (side 1) for every query
            if constexpr (BF) {
              s = clipped_scores(kf, qb, side);
            } else {
              s = mma_keyconst<BF>(kc[kb], side, hh);
              s = mma_frag<BF, D>(kf, qf[qb], s);
            }
          } else {
            // one 32 x kCbandStride float tile per wave, used first for the
            // content-to-position band, then for the position-to-content band
            float* band = relf + wave * L.deb_wave_floats;
            // In the eight-wave kernel the content-to-position band's MFMAs
            // and stores run at raised wave priority: they start the
            // block's dependency chain, and the other wave of the SIMD fills
            // in behind them (k=512: 268.4 -> 261.5 us; keeping the priority
            // through the position-to-content band as well gains nothing,
            // 267.9 us)
            if constexpr (KR_RING) __builtin_amdgcn_s_setprio(2);
            const T* kr = reinterpret_cast<const T*>(a.table);
            const T* qr = reinterpret_cast<const T*>(a.table2);
            const int T0 = pq_min - j0 - 31;  // band index m <-> query - key = T0 + m
            // Qr rows delta(-(T0 + 32 nb + lane)) (the position-to-content
            // band's A operand); the first half may have been requested by
            // the previous block
            TableFrag<BF, D> bfr[2];
            if (QR_NEXT && qr_t0 == T0) bfr[0] = qr_next;
            else bfr[0].load(qr + ((size_t)deberta_delta_dev(-(T0 + lq), ck) * a.H + h) * D, hh);
            if (QR_NEXT && qr_ct0 == T0) bfr[1] = qr_carry;
            else bfr[1].load(qr + ((size_t)deberta_delta_dev(-(T0 + 32 + lq), ck) * a.H + h) * D, hh);
            // content-to-position: rows Kr[delta(T0 + m)], columns = queries,
            // stored [query][m]
            TableFrag<BF, D> af[2];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
              if constexpr (KR_RING) {
                // rows u = T0 + 32 tb + lane + k: 32 consecutive ring slots
                af[tb].load_lds(ring + ring_slot(T0 + 32 * tb + ck - ring_c0) * 128, ko.k);
              } else {
                af[tb].load(kr + ((size_t)deberta_delta_dev(T0 + 32 * tb + lq, ck) * a.H + h) * D, hh);
              }
            }
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
              const f32x16 acc = mma_frag0<BF, D>(af[tb], qf[qb]);
              float* dst = band + lq * kCbandStride + 32 * tb + 4 * hh;
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const f32x4 x = {acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
                *reinterpret_cast<f32x4*>(dst + 8 * g) = x;
              }
            }
            if constexpr (KR_RING) __builtin_amdgcn_s_setprio(0);
            wave_lds_fence();
            // key j0 + jl of query row lq sits at m = lq - jl + 31
            float cg[16];
            {
              const float* crow = band + lq * (kCbandStride + 1) + 31;
#pragma unroll
              for (int i = 0; i < 16; ++i) cg[i] = crow[-acc_row(i, hh)];
            }
            // position-to-content: rows n <-> query - key = T0 + n (Qr row
            // delta(key - query), the A operand), columns = keys (the K
            // fragment as the B operand); register 4g + e of a lane holds n =
            // 32 nb + 8g + 4hh + e of its key, so the tile [key][n] takes one
            // 16-byte store per four registers.  The tile is the one the
            // reads above used (they precede these writes in the wave's LDS
            // order).
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
              const f32x16 acc = mma_frag0<BF, D>(bfr[nb], kf);
              float* dst = band + lq * kCbandStride + 32 * nb + 4 * hh;
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const f32x4 x = {acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
                *reinterpret_cast<f32x4*>(dst + 8 * g) = x;
              }
            }
            if constexpr (QR_NEXT) {
              qr_carry = bfr[0];
              qr_ct0 = T0 - 32;
            }
            wave_lds_fence();
            // key j0 + jl of query row lq sits at n = lq - jl + 31
            f32x16 init;
            {
              const float* prow = band + lq + 31;
#pragma unroll
              for (int i = 0; i < 16; ++i) init[i] = cg[i] + prow[acc_row(i, hh) * (kCbandStride - 1)];
            }
            wave_lds_fence();  // the next block overwrites the tile
            if constexpr (QR_NEXT) {
              // the next key block's first half: distances T0 - 32 + lane
              qr_next.load(qr + ((size_t)deberta_delta_dev(-(T0 - 32 + lq), ck) * a.H + h) * D, hh);
              qr_t0 = T0 - 32;
            }
            s = mma_frag<BF, D>(kf, qf[qb], init);
          }
        }
        // masks: hidden keys become -inf (only on blocks that touch the
        // causal diagonal or the end of the valid keys)
        if constexpr (CLS == 2) {
          if ((a.causal && j0 + 31 > pq_min) || (j0 + 32 > kv_lim)) {
            // register i holds key j0 + acc_row(i, hh) = j0 + 4hh + acc_row(i, 0);
            // it is visible iff acc_row(i, 0) <= last - j0 - 4hh
            const int last = a.causal ? min(kv_lim - 1, pos[qb]) : kv_lim - 1;
            const int lim = last - j0 - 4 * hh;
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (acc_row(i, 0) > lim) s[i] = NEG_INF;
          }
        }
        return s;
      };

      using PFrag = typename std::conditional<BF, bf16x8, float>::type;
      PFrag pf[QB][BF ? 2 : 1];
      f32x16 s[QB];
      float lsum[QB];
      // p = exp2(mul * s + add) in place of s, its bfloat16 copy for the P V
      // product, the lane sum
      auto softmax = [&](const int qb, const float mul, const float add) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[qb][i] = fast_exp2(fmaf(s[qb][i], mul, add));
        float ls = 0.f;
        if constexpr (BF) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            pf[qb][h2] = pack_bf16x8(s[qb], 8 * h2);
            ls = sum_bf16x8(pf[qb][h2], ls);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) ls += s[qb][i];
        }
        lsum[qb] = ls;
      };

      // Scores of every query block of the step, their softmax, then one
      // wave-wide check: the whole step stays one scheduling region, so the
      // MFMAs of one query block overlap the exponentials of the other.  One
      // K fragment read from LDS feeds the query blocks; the exact path reads
      // its own copy, so nothing of the fast path stays live for it.
      {
        TableFrag<BF, D> kf;
        kf.load_lds(ktile + 32 * kb * ROWB, ko.k);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if (!((QM >> qb) & 1)) continue;
          s[qb] = scores(qb, kf);
        }
      }
      // One query block per wave leaves registers to spare: the V^T
      // fragments of the step are read before the softmax, so their LDS
      // latency hides behind it instead of sitting between it and P V.
      // (not in DeBERTa's eight-wave kernel, which spends these registers on
      // the requested Qr rows)
      constexpr bool EARLY_V = BF && QB == 1 && D <= 64 && !QR_NEXT;
      bf16x8 vpre[EARLY_V ? 2 : 1][EARLY_V ? NDB : 1];
      if constexpr (EARLY_V) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int db = 0; db < NDB; ++db) vpre[h2][db] = load_vt_frag<D>(vtile, 2 * kb + h2, ko.v[db]);
      }
      bool bad = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (!((QM >> qb) & 1)) continue;
        softmax(qb, c, (KIND == 3 || (KIND == 2 && CLS == 2)) ? ref_offset(c * b_block(qb), m_ref[qb])
                                                              : off[qb]);
        bad = bad || lsum[qb] > kSumLimit;
      }
      if (__builtin_expect(__any(bad), 0)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if (!((QM >> qb) & 1)) continue;
          if (!__any(lsum[qb] > kSumLimit)) continue;
          // exact path: scores in log2 units, the row max, rescale of the
          // running state
          TableFrag<BF, D> kf2;
          kf2.load_lds(ktile + 32 * kb * ROWB, ko.k);
          s[qb] = scores(qb, kf2);
          const float cb = c * b_block(qb);
#pragma unroll
          for (int i = 0; i < 16; ++i) s[qb][i] = fmaf(s[qb][i], c, cb);
          const float mn = fmaxf(m_ref[qb], max_halves(max16(s[qb])));
          const float alpha = mn == NEG_INF ? 1.f : fast_exp2(m_ref[qb] - mn);
          if constexpr (KIND == 1) flush_bins(qb);  // bins hold p at the old reference
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[qb][db] *= alpha;
          l_run[qb] *= alpha;
          lr_run[qb] *= alpha;
          win_run[qb] *= alpha;
          m_ref[qb] = mn;
          const float mu = mn == NEG_INF ? 0.f : mn;
          softmax(qb, 1.f, -mu);
          off[qb] = ref_offset(c * b_tile[qb], m_ref[qb]);
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (!((QM >> qb) & 1)) continue;
        l_run[qb] += lsum[qb];

        // Shaw: keys past the window go to bin 2k; keys inside it to their
        // own bin: scattered into the wave's bin tile (one row per query),
        // which is then multiplied by a_V with MFMA
        if constexpr (KIND == 1) {
          if (far_right[qb]) {
            lr_run[qb] += lsum[qb];
          } else if (CLS == 2 && near[qb]) {
            // keys inside the window: their probability goes to the row's
            // own bin (each offset belongs to exactly one key of a row, so a
            // bin is assigned once); the bins are multiplied by a_V when the
            // row is done or before its running state is rescaled
            // Branch-free: the key at offset o stores to slot clamp(o + k,
            // 0, 2k), so keys outside the window land in the slots 0 and 2k
            // (never read as bins); the window's mass is summed from the
            // bins when they are applied
            T* wrow = wbins + (32 * qb + lq) * shaw_bin_stride(ck, (int)sizeof(T));
            const int obase = j0 + 4 * hh - pos[qb];  // offset of register 0's key
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int slot = min(max(obase + ck + acc_row(i, 0), 0), 2 * ck);
              if constexpr (BF) wrow[slot] = pf[qb][i >> 3][i & 7];
              else wrow[slot] = s[qb][i];
            }
            // keys at offset >= k (later keys, all hidden under a causal
            // mask) take bin 2k
            if (!a.causal) {
              float lr = 0.f;
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                float pv;
                if constexpr (BF) pv = (float)pf[qb][i >> 3][i & 7];
                else pv = s[qb][i];
                lr += obase + acc_row(i, 0) >= ck ? pv : 0.f;
              }
              lr_run[qb] += lr;
            }
            bins_dirty[qb] = true;
          }
        }
      }

      // O^T += V^T P^T over these 32 keys
      if constexpr (BF) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            bf16x8 vf;
            if constexpr (EARLY_V) vf = vpre[h2][db];
            else vf = load_vt_frag<D>(vtile, 2 * kb + h2, ko.v[db]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              if ((QM >> qb) & 1) o[qb][db] = mma_bf16(vf, pf[qb][h2], o[qb][db]);
          }
      } else {
#pragma unroll
        for (int cc = 0; cc < 16; ++cc)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const float vv = load_v_f32<D>(vtile, kb, cc, db, ko.v[0]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              if ((QM >> qb) & 1) o[qb][db] = mma_f32(vv, s[qb][cc], o[qb][db]);
          }
      }
    };

    // Lean tiles (classes 0 and 1) in bfloat16: a software pipeline over
    // the tile's NKB*QB blocks of 32 keys x 32 query rows (block g: key
    // block g / QB, query block g % QB).  The code of block g holds the
    // scores of block g+1 and the P V product of block g-1 beside block g's
    // exponentials: none depends on the others, so the MFMAs run while the
    // vector ALU computes the softmax, within one wave.
    auto pipe_tile = [&]() {
      constexpr int NB = NKB * QB;
      // raw scores of block g: the in-block relative term + q.k
      auto block_scores = [&](const int g, const TableFrag<BF, D>& kf) -> f32x16 {
        const int kb = g / QB, qb = g % QB;
        if constexpr (KIND == 0) {
          if constexpr (CLS == 1) {
            f32x16 init;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const f32x4 x = *reinterpret_cast<const f32x4*>(lutp[qb] + 32 * kb + 8 * q4 + 4 * hh);
              init[4 * q4 + 0] = x[0]; init[4 * q4 + 1] = x[1];
              init[4 * q4 + 2] = x[2]; init[4 * q4 + 3] = x[3];
            }
            return mma_frag<BF, D>(kf, qf[qb], init);
          } else {
            return mma_frag0<BF, D>(kf, qf[qb]);
          }
        } else if constexpr (KIND == 1 && CLS == 2) {
          const int j0 = k0 + 32 * kb;
          f32x16 x;
          if (near[qb]) {
            const float* ar = arel + (32 * qb + lq) * L.arel_stride;
            const int obase = j0 + 4 * hh - pos[qb];  // offset of register 0's key
            f32x16 init;
#pragma unroll
            for (int i = 0; i < 16; ++i) init[i] = (float)ar[shaw_row_dev(obase + acc_row(i, 0), ck)];
            x = mma_frag<BF, D>(kf, qf[qb], init);
          } else {
            x = mma_frag0<BF, D>(kf, qf[qb]);
          }
          // hidden keys -inf (blocks that touch the causal diagonal or the
          // end of the valid keys)
          const int pq_min = pw_min + 32 * qb;
          if ((a.causal && j0 + 31 > pq_min) || (j0 + 32 > kv_lim)) {
            const int last = a.causal ? min(kv_lim - 1, pos[qb]) : kv_lim - 1;
            const int lim = last - j0 - 4 * hh;
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (acc_row(i, 0) > lim) x[i] = NEG_INF;
          }
          return x;
        } else if constexpr (KIND == 2) {
          return clipped_scores(kf, qb, deb_side[qb]);
        } else if constexpr (KIND == 3) {
          return mma_frag<BF, D>(kf, qf[qb], mma_keyconst<BF>(alibi_kc, deb_side[qb], hh));
        } else {
          return mma_frag0<BF, D>(kf, qf[qb]);
        }
      };
      // per-row constant of block g (raw score units)
      auto block_b = [&](const int g) -> float {
        const int kb = g / QB, qb = g % QB;
        if constexpr (KIND == 3) {
          const float dist = (float)(pos[qb] - (k0 + 32 * kb));
          return deb_side[qb] == 0 ? alibi_s * dist : -alibi_s * dist;
        }
        return b_tile[qb];
      };
      auto block_off = [&](const int g) -> float {
        if constexpr (KIND == 3) return ref_offset(c * block_b(g), m_ref[g % QB]);
        return off[g % QB];
      };
      // p = exp2(mul * x + add) in place, its bfloat16 copy, the lane sum
      auto smax = [&](f32x16& x, bf16x8 (&pb)[2], const float mul, const float add) -> float {
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = fast_exp2(fmaf(x[i], mul, add));
        float ls = 0.f;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          pb[h2] = pack_bf16x8(x, 8 * h2);
          ls = sum_bf16x8(pb[h2], ls);
        }
        return ls;
      };
      f32x16 sc[2];
      bf16x8 pb[2][2];
      bf16x8 vf[2][NDB];  // V^T fragments of the key block of the pending P V
      // One query block per wave and 64-wide heads leave registers to spare:
      // the K fragment of the second key block is read with the first one's
      // and the V^T fragments of the last key block with the previous
      // block's, so no MFMA of the tile waits for its LDS read, and the
      // block's instructions are ordered explicitly: its LDS reads first,
      // then each MFMA followed by a few vector instructions (measured on
      // the causal 4096-token Shaw workload: 195 -> 191 us; 128-wide heads
      // ran slower with it)
      constexpr bool KPRE = QB == 1 && NKB == 2 && D <= 64;
      bf16x8 vl[KPRE ? 2 : 1][KPRE ? NDB : 1];  // V^T fragments of the last key block
      auto load_v = [&](const int kb) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int db = 0; db < NDB; ++db) vf[h2][db] = load_vt_frag<D>(vtile, 2 * kb + h2, ko.v[db]);
      };
      auto pv = [&](const int g) {
        const int qb = g % QB;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            bf16x8 vv = vf[h2][db];
            if constexpr (KPRE) if (g == NB - 1) vv = vl[h2][db];
            o[qb][db] = mma_bf16(vv, pb[g & 1][h2], o[qb][db]);
          }
      };
      TableFrag<BF, D> kpre;
      {
        TableFrag<BF, D> kf;
        kf.load_lds(ktile, ko.k);
        if constexpr (KPRE) kpre.load_lds(ktile + 32 * ROWB, ko.k);
        sc[0] = block_scores(0, kf);
      }
      issue_next();
#pragma unroll
      for (int g = 0; g < NB; ++g) {
        const int kb = g / QB, qb = g % QB;
        if (g >= 1 && (g - 1) % QB == 0) load_v((g - 1) / QB);
        if constexpr (KPRE) {
          if (g == NB - 1) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
              for (int db = 0; db < NDB; ++db) vl[h2][db] = load_vt_frag<D>(vtile, 2 * (NKB - 1) + h2, ko.v[db]);
          }
        }
        if (g + 1 < NB) {
          if constexpr (KPRE) {
            sc[(g + 1) & 1] = block_scores(g + 1, kpre);
          } else {
            TableFrag<BF, D> kf;
            kf.load_lds(ktile + 32 * ((g + 1) / QB) * ROWB, ko.k);
            sc[(g + 1) & 1] = block_scores(g + 1, kf);
          }
        }
        float ls = smax(sc[g & 1], pb[g & 1], c, block_off(g));
        if (g >= 1) pv(g - 1);
        if constexpr (KPRE) {
          // scheduling groups (masks: 0x100 LDS reads, 0x002 | 0x400 vector
          // and transcendental instructions, 0x008 MFMA)
          __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
          __builtin_amdgcn_sched_group_barrier(0x402, 8, 0);
#pragma unroll
          for (int i = 0; i < 10; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x402, 5, 0);
          }
        }
        if (__builtin_expect(__any(ls > kSumLimit), 0)) {
          // exact path: the block's scores in log2 units, the row max, the
          // rescale of the running state, the softmax again
          TableFrag<BF, D> kf2;
          kf2.load_lds(ktile + 32 * kb * ROWB, ko.k);
          f32x16 x = block_scores(g, kf2);
          const float cb = c * block_b(g);
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = fmaf(x[i], c, cb);
          const float mn = fmaxf(m_ref[qb], max_halves(max16(x)));
          const float alpha = mn == NEG_INF ? 1.f : fast_exp2(m_ref[qb] - mn);
          if constexpr (KIND == 1) flush_bins(qb);  // bins hold p at the old reference
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[qb][db] *= alpha;
          l_run[qb] *= alpha;
          lr_run[qb] *= alpha;
          win_run[qb] *= alpha;
          m_ref[qb] = mn;
          ls = smax(x, pb[g & 1], 1.f, -(mn == NEG_INF ? 0.f : mn));
          off[qb] = ref_offset(c * b_tile[qb], m_ref[qb]);
        }
        l_run[qb] += ls;
        if constexpr (KIND == 1) {
          if (far_right[qb]) lr_run[qb] += ls;
        }
        if constexpr (KIND == 1 && CLS == 2) {
          if (near[qb]) {
            // keys inside the window: their probability to the row's own bin
            // (slot clamp(offset + k, 0, 2k): keys outside the window land
            // in the unread slots 0 and 2k); keys at offset >= k, only
            // without a causal mask, to bin 2k
            T* wrow = wbins + (32 * qb + lq) * shaw_bin_stride(ck, (int)sizeof(T));
            const int obase = k0 + 32 * kb + 4 * hh - pos[qb];  // offset of register 0's key
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int slot = min(max(obase + ck + acc_row(i, 0), 0), 2 * ck);
              wrow[slot] = pb[g & 1][i >> 3][i & 7];
            }
            if (!a.causal) {
              float lr = 0.f;
#pragma unroll
              for (int i = 0; i < 16; ++i)
                lr += obase + acc_row(i, 0) >= ck ? (float)pb[g & 1][i >> 3][i & 7] : 0.f;
              lr_run[qb] += lr;
            }
            bins_dirty[qb] = true;
          }
        }
      }
      if constexpr (QB == 1 && !KPRE) load_v(NKB - 1);
      pv(NB - 1);
    };

    if constexpr (PIPE) {
      pipe_tile();
    } else if constexpr (CLS != 2) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) step(std::integral_constant<int, (1 << QB) - 1>{}, kb);
    } else {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) step(std::integral_constant<int, 1>{}, kb);
      if constexpr (QB > 1) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) step(std::integral_constant<int, 2>{}, kb);
      }
    }
  };

  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C3 = std::integral_constant<int, 3>;
  int r = 0;
  while (r < n_steps) {
    const int cls = tile_class(r);
    const int ln = opaque_lane();
    if constexpr (QR_NEXT) {
      if (cls != 2) {
        // no near block follows within this run: drop the requested Qr rows
        qr_t0 = -(1 << 30);
        qr_next.zero();
        qr_ct0 = -(1 << 30);
        qr_carry.zero();
      }
    }
    if (cls == 0) {
      do { run_tile(C0{}, r, ln); ++r; } while (r < n_steps && tile_class(r) == 0);
    } else if (cls == 1) {
      if constexpr (KIND == 0) {
        do { run_tile(C1{}, r, ln); ++r; } while (r < n_steps && tile_class(r) == 1);
      }
    } else if (cls == 2) {
      do { run_tile(C2{}, r, ln); ++r; } while (r < n_steps && tile_class(r) == 2);
    } else {
      do { run_tile(C3{}, r, ln); ++r; } while (r < n_steps && tile_class(r) == 3);
    }
  }

  // ---- epilogue -------------------------------------------------------------
  wait_vmcnt<0>();  // no tile load may still be writing LDS when the wave ends
  if constexpr (KS == 2) {
    // The halves meet: half 1 hands its running state (per lane: the output
    // registers, the reference, the partial row sum; lane l of wave wq + NWQ
    // holds the same query row and head dims as lane l of wave wq) to half 0
    // through the stage memory, which no wave reads any more.  Half 0 moves
    // both to the larger reference, 2^(m - M) each, and adds them.
    constexpr int XS = 16 * NDB + 4;  // floats per lane
    float* xs = reinterpret_cast<float*>(smem) + (size_t)(wq * 64 + lane) * XS;
    __syncthreads();  // every wave is done with its stages
    if (half == 1) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4*>(xs + 16 * db + 4 * g) =
              f32x4{o[0][db][4 * g], o[0][db][4 * g + 1], o[0][db][4 * g + 2], o[0][db][4 * g + 3]};
      *reinterpret_cast<f32x4*>(xs + 16 * NDB) = f32x4{m_ref[0], l_run[0], 0.f, 0.f};
    }
    __syncthreads();
    if (half == 1) return;
    const f32x4 ml = *reinterpret_cast<const f32x4*>(xs + 16 * NDB);
    const float mb = ml[0], lb = ml[1];
    const float M = fmaxf(m_ref[0], mb);
    if (M != NEG_INF) {
      const float wa = m_ref[0] == NEG_INF ? 0.f : fast_exp2(m_ref[0] - M);
      const float wb = mb == NEG_INF ? 0.f : fast_exp2(mb - M);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(xs + 16 * db + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[0][db][4 * g + e] = wa * o[0][db][4 * g + e] + wb * x[e];
        }
      l_run[0] = wa * l_run[0] + wb * lb;
      m_ref[0] = M;
    }
  }
  if (!wave_active) return;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
    if constexpr (KIND == 1) {
      flush_bins(qb);
      // bins 0 and 2k take the row mass not held by the in-window bins
      const float lr_tot = lr_run[qb] + __shfl_xor(lr_run[qb], 32);
      const float w_in = win_run[qb] + __shfl_xor(win_run[qb], 32);
      const float w0 = l_tot - w_in - lr_tot;
      // register 4g + q of a lane holds head dim 32 db + 8 g + 4 hh + q: four
      // consecutive elements of each end row, one vector read each
      using T4 = typename std::conditional<BF, bf16x4, f32x4>::type;
      const T* ends = reinterpret_cast<const T*>(smem + L.rel_off + L.avend_off) + wave * 2 * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dd = 32 * db + 8 * g + 4 * hh;
          const T4 e0 = *reinterpret_cast<const T4*>(ends + dd);
          const T4 e1 = *reinterpret_cast<const T4*>(ends + D + dd);
#pragma unroll
          for (int q = 0; q < 4; ++q) o[qb][db][4 * g + q] += w0 * (float)e0[q] + lr_tot * (float)e1[q];
        }
    }
    if (qrow[qb] >= a.Lq) continue;
    // the row's reference on the logits' own scale (Shaw leaves q.a_K[0] out
    // of every logit, a softmax-neutral shift)
    const float m_row = KIND == 1 ? m_ref[qb] + c * shaw_base[qb] : m_ref[qb];
    if (a.n_splits == 1) {
      // sum_j exp(logit_j) = l_tot * 2^m_row
      if (a.lse != nullptr && hh == 0)
        a.lse[(size_t)bh * a.Lq + qrow[qb]] =
            l_tot > 0.f ? (__log2f(l_tot) + m_row) * 0.6931471805599453f : NEG_INF;
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      T* og = reinterpret_cast<T*>(a.out) + ((size_t)bh * a.Lq + qrow[qb]) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dd = 32 * db + 8 * g + 4 * hh;
          if constexpr (BF) {
            const bf16x2 y0 = cvt2(o[qb][db][4 * g] * inv, o[qb][db][4 * g + 1] * inv);
            const bf16x2 y1 = cvt2(o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv);
            const bf16x4 y = {y0[0], y0[1], y1[0], y1[1]};
            *reinterpret_cast<bf16x4*>(og + dd) = y;
          } else {
            const f32x4 y = {o[qb][db][4 * g] * inv, o[qb][db][4 * g + 1] * inv,
                             o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv};
            *reinterpret_cast<f32x4*>(og + dd) = y;
          }
        }
    } else {
      const size_t row = ((size_t)split * a.B * a.H + bh) * a.Lq + qrow[qb];
      float* po = a.part_o + row * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dd = 32 * db + 8 * g + 4 * hh;
          const f32x4 y = {o[qb][db][4 * g], o[qb][db][4 * g + 1], o[qb][db][4 * g + 2], o[qb][db][4 * g + 3]};
          *reinterpret_cast<f32x4*>(po + dd) = y;
        }
      if (hh == 0) {
        const f32x2 ml = {l_tot > 0.f ? m_row : NEG_INF, l_tot};
        *reinterpret_cast<f32x2*>(a.part_ml + row * 2) = ml;
      }
    }
  }
}

// Merge split-KV partials: each split holds an unnormalised output and its
// (max, sum) in the exp2 domain; rescale to the common max and normalise.
// One thread per 4 output elements of a row; the (max, sum) pairs and the
// output chunks of every split are requested together (MS splits at most,
// MS a multiple of 4), so the merge costs one memory round trip.
template <bool BF, int D, int MS>
__global__ __launch_bounds__(256) void relattn_combine_kernel(CombineArgs a) {
  using T = typename std::conditional<BF, bf16, float>::type;
  const int64_t nrow = (int64_t)a.BH * a.Lq;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = idx / (D / 4);
  const int ch = (int)(idx % (D / 4));
  if (row >= nrow) return;
  f32x2 ml[MS];
  f32x4 po[MS];
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    if (s < a.n_splits) {
      const size_t r = (size_t)s * nrow + row;
      ml[s] = *reinterpret_cast<const f32x2*>(a.part_ml + r * 2);
      po[s] = *reinterpret_cast<const f32x4*>(a.part_o + r * D + 4 * ch);
    } else {
      ml[s] = f32x2{RA_NEG_INF, 0.f};
      po[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  float M = RA_NEG_INF;
#pragma unroll
  for (int s = 0; s < MS; ++s) M = fmaxf(M, ml[s][0]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float Lsum = 0.f;
  if (M != RA_NEG_INF) {
#pragma unroll
    for (int s = 0; s < MS; ++s) {
      // splits that saw no visible key hold (-inf, 0): weight 0
      const float w = ml[s][1] > 0.f ? fast_exp2(ml[s][0] - M) : 0.f;
      Lsum += w * ml[s][1];
      acc += w * po[s];
    }
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  if (a.lse != nullptr && ch == 0)
    a.lse[row] = Lsum > 0.f ? (__log2f(Lsum) + M) * 0.6931471805599453f : RA_NEG_INF;
  T* og = reinterpret_cast<T*>(a.out) + row * D + 4 * ch;
  if constexpr (BF) {
    const bf16x2 y0 = cvt2(acc[0] * inv, acc[1] * inv), y1 = cvt2(acc[2] * inv, acc[3] * inv);
    const bf16x4 y = {y0[0], y0[1], y1[0], y1[1]};
    *reinterpret_cast<bf16x4*>(og) = y;
  } else {
    const f32x4 y = acc * inv;
    *reinterpret_cast<f32x4*>(og) = y;
  }
}

// Row constants in float32 for the score terms that reduce to one value per
// key or per relative distance:
//   DeBERTa  k_j.Qr[0][h] and k_j.Qr[2k-1][h] (the position-to-content term
//            of blocks whose offsets are all clipped, [DRPE]);
//   TXL      u_h.k_j per key and v_h.E[r, h] per distance r ([RPE]
//            Transformer-XL: the global content and position biases).
// bfloat16 inputs store each constant as a bf16 hi + lo pair ({hi0, lo0, hi1,
// lo1} per entry); float32 inputs store the float pair.  A row of d elements
// is CPR 16-byte chunks; CPR consecutive lanes take one row (lane c its chunk
// c), so a wave reads 64 / CPR whole rows, one contiguous run per load when
// the rows are adjacent, and the partial dot products meet by lane exchanges.
// Grid: x = blocks of kColcPasses * 256 / CPR rows of one group (each lane
// group takes kColcPasses rows, requested together), y = groups (strided
// when there are more groups than the grid's y extent), z = job; no lane
// divides.  A job without a second vector multiplies by zeros.
constexpr int kColcPasses = 4;  // Transformer-XL with memory: 293.7 -> 288.5 us with the 3-D grid
template <bool BF, int D>
__global__ __launch_bounds__(256) void relattn_colc_kernel(ColcArgs a) {
  using T = typename std::conditional<BF, bf16, float>::type;
  constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = D / EPV;         // chunks per row (4 .. 16)
  static_assert(CPR >= 2 && CPR <= 64 && (CPR & (CPR - 1)) == 0, "chunks per row");
  constexpr int RPB = 256 / CPR;       // rows per workgroup and pass
  constexpr int NP = kColcPasses;      // passes: rows r, r + RPB, ... of one lane group
  const ColcJob& j = a.job[blockIdx.z];
  const int c = threadIdx.x % CPR;
  const int r0 = blockIdx.x * RPB * NP + threadIdx.x / CPR;  // first row within the group
  for (int g = blockIdx.y; g < j.G; g += gridDim.y) {  // wave-uniform
    const int h = g % j.H;
    const f32x4 ax = *reinterpret_cast<const f32x4*>(reinterpret_cast<const T*>(j.a0) + (size_t)h * D + c * EPV);
    f32x4 bx = {};
    if (j.a1) bx = *reinterpret_cast<const f32x4*>(reinterpret_cast<const T*>(j.a1) + (size_t)h * D + c * EPV);
    // the pass rows' chunks are requested together; a row past the last
    // computes nothing and stores nothing, but its lanes stay for the
    // exchanges
    f32x4 kx[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int r = r0 + p * RPB;
      kx[p] = {};
      if (r < j.R)
        kx[p] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const T*>(j.x) +
                                                ((int64_t)g * j.x_sg + (int64_t)r * j.x_sr) * D + c * EPV);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int r = r0 + p * RPB;
      const T* ke = reinterpret_cast<const T*>(&kx[p]);
      const T* ae = reinterpret_cast<const T*>(&ax);
      const T* be = reinterpret_cast<const T*>(&bx);
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        s0 = fmaf((float)ke[e], (float)ae[e], s0);
        s1 = fmaf((float)ke[e], (float)be[e], s1);
      }
      // sum over the CPR lanes of the row (a fixed order, so the result
      // does not depend on the launch)
#pragma unroll
      for (int m = 1; m < CPR; m <<= 1) {
        s0 += __shfl_xor(s0, m);
        s1 += __shfl_xor(s1, m);
      }
      if (r < j.R && c == 0) {
        const int64_t idx = (int64_t)g * j.R + r;
        if constexpr (BF) {
          const bf16 h0 = (bf16)s0, h1 = (bf16)s1;
          const bf16x4 y = {h0, (bf16)(s0 - (float)h0), h1, (bf16)(s1 - (float)h1)};
          reinterpret_cast<bf16x4*>(j.out)[idx] = y;
        } else {
          reinterpret_cast<f32x2*>(j.out)[idx] = f32x2{s0, s1};
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Host-side launch helpers (called from relattn_api.cpp)
// ----------------------------------------------------------------------------

// Device scratch of relattn_fwd_noalloc: the workspace (split-KV partials,
// row constants) of callers that cannot allocate.  Each GPU the library runs
// on holds its own copy until the process ends.  In host code `scratch` is a
// host-side stand-in for the symbol, not a device address: its address on a
// device comes from hipGetSymbolAddress with that device current, kept per
// device, and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

template <int KIND, bool BF, int D, int QB, int NW>
static hipError_t launch_fwd_t(const FwdArgs& a, int grid, int lds, hipStream_t st) {
  auto kfn = relattn_fwd_kernel<KIND, BF, D, QB, NW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, dim3(grid), dim3(64 * NW), lds, st, a);
  return hipGetLastError();
}

bool fwd_variant_built(int kind, bool bf, int d, Variant v) {
  if (d == 128) return bf && v.qb == 1 && v.nw == 4;
  if ((kind == 0 || kind == 3) && v.nw == 8) return bf && v.qb == 1;  // key split
  if ((kind == 2 || kind == 4) && bf && d == 64) return v.qb == 1 && (v.nw == 8 || v.nw == 4);
  if (kind == 2 || kind == 4) return v.qb == 1 && v.nw == 4;  // kinds 0, 1, 3 below
  return v.nw == 4 && (v.qb == 1 || (v.qb == 2 && bf && kind != 1));
}

hipError_t launch_fwd(int kind, bool bf, int d, Variant v, const FwdArgs& a, int grid, int lds,
                      hipStream_t st) {
#define RA_CASE(K, B, DD, QBV, NWV)                                     \
  if (kind == K && bf == B && d == DD && v.qb == QBV && v.nw == NWV) \
    return launch_fwd_t<K, B, DD, QBV, NWV>(a, grid, lds, st);
#define RA_DT(K, QBV, NWV)                                                        \
  RA_CASE(K, true, 64, QBV, NWV) RA_CASE(K, true, 32, QBV, NWV) RA_CASE(K, false, 64, QBV, NWV) \
  RA_CASE(K, false, 32, QBV, NWV)
  RA_DT(0, 1, 4) RA_DT(1, 1, 4) RA_DT(2, 1, 4) RA_DT(3, 1, 4) RA_DT(4, 1, 4)
  RA_CASE(2, true, 64, 1, 8) RA_CASE(4, true, 64, 1, 8)
  RA_CASE(0, true, 64, 1, 8) RA_CASE(0, true, 32, 1, 8) RA_CASE(3, true, 64, 1, 8)
  RA_CASE(3, true, 32, 1, 8)
  RA_CASE(0, true, 128, 1, 4) RA_CASE(1, true, 128, 1, 4) RA_CASE(2, true, 128, 1, 4)
  RA_CASE(3, true, 128, 1, 4) RA_CASE(4, true, 128, 1, 4)
  RA_CASE(0, true, 64, 2, 4) RA_CASE(0, true, 32, 2, 4)
  RA_CASE(3, true, 64, 2, 4) RA_CASE(3, true, 32, 2, 4)
#undef RA_DT
#undef RA_CASE
  return hipErrorInvalidValue;
}

template <bool BF, int D>
static void launch_combine_t(const CombineArgs& a, int grid, hipStream_t st) {
  if (a.n_splits <= 8) hipLaunchKernelGGL((relattn_combine_kernel<BF, D, 8>), dim3(grid), dim3(256), 0, st, a);
  else if (a.n_splits <= 16) hipLaunchKernelGGL((relattn_combine_kernel<BF, D, 16>), dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((relattn_combine_kernel<BF, D, kMaxSplits>), dim3(grid), dim3(256), 0, st, a);
}

hipError_t launch_combine(bool bf, int d, const CombineArgs& a, hipStream_t st) {
  const int64_t threads = (int64_t)a.BH * a.Lq * (d / 4);
  const int grid = (int)((threads + 255) / 256);
  if (bf && d == 128) launch_combine_t<true, 128>(a, grid, st);
  else if (bf && d == 64) launch_combine_t<true, 64>(a, grid, st);
  else if (bf && d == 32) launch_combine_t<true, 32>(a, grid, st);
  else if (!bf && d == 64) launch_combine_t<false, 64>(a, grid, st);
  else launch_combine_t<false, 32>(a, grid, st);
  return hipGetLastError();
}

hipError_t launch_colc(bool bf, int d, const ColcArgs& a, hipStream_t st) {
  int rmax = 0, gmax = 0;
  for (int jb = 0; jb < a.njobs; ++jb) {
    rmax = std::max(rmax, (int)a.job[jb].R);
    gmax = std::max(gmax, (int)a.job[jb].G);
  }
  if (a.njobs == 0 || rmax == 0 || gmax == 0) return hipSuccess;
  const int rpb = 256 / (d * (bf ? 2 : 4) / 16) * kColcPasses;  // rows per workgroup
  const dim3 grid((rmax + rpb - 1) / rpb, std::min(gmax, 65535), a.njobs);
  if (bf && d == 128) hipLaunchKernelGGL((relattn_colc_kernel<true, 128>), grid, dim3(256), 0, st, a);
  else if (bf && d == 64) hipLaunchKernelGGL((relattn_colc_kernel<true, 64>), grid, dim3(256), 0, st, a);
  else if (bf && d == 32) hipLaunchKernelGGL((relattn_colc_kernel<true, 32>), grid, dim3(256), 0, st, a);
  else if (!bf && d == 64) hipLaunchKernelGGL((relattn_colc_kernel<false, 64>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((relattn_colc_kernel<false, 32>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_index(const IndexArgs& a, hipStream_t st) {
  int64_t blocks = (a.n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(relattn_index_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace relattn
