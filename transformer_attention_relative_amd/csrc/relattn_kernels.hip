// Fused relative-position attention forward for gfx950 (MI355X).
//
// Sources (page title, then passage):
//   [RPE]  "Relative Position Embeddings, in depth: Shaw, Transformer-XL,
//          T5 buckets and DeBERTa ..." (aicassindra.com)
//   [T5B]  "T5 Relative-Position Bias" (liminalml.com)
//   [DRPE] "DeBERTa > Relative Position Encoding" (mbrenndoerfer.com)
//
// Design (one workgroup = 4 wave64s = 128 query rows of one (b, h)):
//   * Scores are produced transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (bf16) or v_mfma_f32_32x32x2f32 (fp32): a
//     lane then owns one query row and 16 keys of each 32-key block, so the
//     row max / row sum need one cross-lane exchange (lane ^ 32) per tile
//     and the per-row rescale of the output is a per-lane scalar.
//   * The output is accumulated transposed too, O^T = V^T P^T, so P leaves
//     the score accumulator directly as the B operand (no LDS round trip).
//     V is staged in LDS transposed for that reason.
//   * The relative term never exists as an L x L array: for each (wave,
//     key tile) it is either a per-row constant folded into the softmax
//     exponent (saturated T5 buckets, clipped Shaw / DeBERTa offsets) or it
//     is written into the MFMA accumulator *before* q.k is accumulated on
//     top (near-diagonal tiles).  Masked entries enter that accumulator as
//     -inf, so masking costs nothing in the MFMA loop.
//   * T5 bucket ids come from host-computed integer thresholds; no log is
//     evaluated on the GPU ([T5B]: saturation starts at the lower edge of
//     the last bin).
//   * Shaw's value term uses the offset-binned softmax mass: every offset
//     strictly inside the clip window belongs to exactly one key per row, so
//     its mass is that key's probability; the two clipped bins take the
//     remainder ([RPE] Shaw section).
//   * DeBERTa near tiles compute the content-to-position band (Kr rows x Q)
//     and the position-to-content band (K x Qr rows) with MFMA and gather
//     them through per-wave LDS; far tiles reduce to a per-row constant plus
//     a per-key constant ([DRPE] clip-and-shift: every offset beyond +-k uses
//     a boundary row).
#include <hip/hip_runtime.h>

#include "relattn_internal.hpp"

namespace relattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define RA_NEG_INF (-__builtin_inff())

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void wave_lds_fence() {
  // Orders this wave's LDS writes before its later LDS reads (other lanes of
  // the same wave read what a lane wrote).
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ----------------------------------------------------------------------------
// Index functions (shared by the index kernel and the fused kernel)
// ----------------------------------------------------------------------------

// T5 bucket of offset = key - query ([RPE] T5 section; [T5B]).  thr[m] is the
// smallest distance whose within-direction slot is >= exact + m (thr[0] ==
// exact); the thresholds come from the host, so no logarithm runs here.
__device__ __forceinline__ int t5_bucket_dev(int offset, int slots, int exact, int bidir,
                                             int nthr, const int32_t* thr) {
  int base = 0, dist;
  if (bidir) {
    base = offset > 0 ? slots : 0;
    dist = offset < 0 ? -offset : offset;
  } else {
    dist = offset < 0 ? -offset : 0;
  }
  if (dist < exact) return base + dist;
  int m = 0;
  for (int t = 1; t < nthr; ++t) m += dist >= thr[t] ? 1 : 0;
  return base + exact + m;
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
    } else {
      r = a.which == 0 ? deberta_delta_dev(qp - kp, a.clip_k) : deberta_delta_dev(kp - qp, a.clip_k);
    }
    a.out[e] = r;
  }
}

// ----------------------------------------------------------------------------
// MFMA wrappers
// ----------------------------------------------------------------------------

__device__ __forceinline__ f32x16 mma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(f32x16 s, int base) {
  f32x2 p0 = {s[base + 0], s[base + 1]}, p1 = {s[base + 2], s[base + 3]};
  f32x2 p2 = {s[base + 4], s[base + 5]}, p3 = {s[base + 6], s[base + 7]};
  bf16x2 c0 = __builtin_convertvector(p0, bf16x2), c1 = __builtin_convertvector(p1, bf16x2);
  bf16x2 c2 = __builtin_convertvector(p2, bf16x2), c3 = __builtin_convertvector(p3, bf16x2);
  bf16x8 r = {c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
  return r;
}

// In the 32x32 accumulator layout, register i of a lane in half hh holds
// row 8*(i/4) + 4*hh + (i%4) of the lane's column.
__device__ __forceinline__ int acc_row(int i, int hh) { return 8 * (i >> 2) + 4 * hh + (i & 3); }

// Row-table fragment: the A operand row (or B operand column) `row` of a
// table whose rows are `d` contiguous elements.  bf16: elements
// 16t + 8hh .. +7 for chunk t; fp32: element t + (d/2)*hh.
template <bool BF, int D>
struct TableFrag;
template <int D>
struct TableFrag<true, D> {
  bf16x8 v[D / 16];
  __device__ __forceinline__ void load(const bf16* row, int hh) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) v[t] = *reinterpret_cast<const bf16x8*>(row + 16 * t + 8 * hh);
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
};

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

// ----------------------------------------------------------------------------
// The fused forward kernel
// ----------------------------------------------------------------------------

template <int KIND, bool BF, int D>
__global__ __launch_bounds__(kThreads, 2) void relattn_fwd_kernel(FwdArgs a) {
  using T = typename std::conditional<BF, bf16, float>::type;
  constexpr int NKB = kBK / 32;  // 32-key blocks per tile
  constexpr int NDB = D / 32;    // 32-wide head-dim blocks of the output
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const LdsLayout L = lds_layout(KIND, BF, D, a.clip_k, a.lut_n);
  T* Ks = reinterpret_cast<T*>(smem + L.k_off);
  T* Vs = reinterpret_cast<T*>(smem + L.v_off);
  float* rel = reinterpret_cast<float*>(smem + L.rel_off);

  // ---- work item (XCD-aware: consecutive logical ids share an L2) ----------
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int lid = (nblk % 8 == 0) ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
  const int per_bh = a.n_qtiles * a.n_splits;
  const int bh = lid / per_bh;
  const int rest = lid - bh * per_bh;
  const int qt = a.n_qtiles - 1 - rest / a.n_splits;  // heavy (late) tiles first
  const int split = rest % a.n_splits;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, hh = lane >> 5;
  const int q0 = qt * kBQ;
  const int wrow0 = q0 + wave * kWaveRows;       // first row of this wave
  const int qrow = wrow0 + lq;                    // this lane's query row
  const int pos = a.q_pos_offset + qrow;          // its absolute position
  const int pw_min = a.q_pos_offset + wrow0;
  const int pw_max = pw_min + kWaveRows - 1;
  const bool wave_active = wrow0 < a.Lq;
  const int pw_max_real = a.q_pos_offset + min(wrow0 + kWaveRows, a.Lq) - 1;

  int kv_lim = a.Lk;
  if (a.kv_valid_len) kv_lim = max(0, min(kv_lim, a.kv_valid_len[b]));
  const int wg_pos_max = a.q_pos_offset + min(q0 + kBQ, a.Lq) - 1;
  const int kv_end = a.causal ? min(kv_lim, wg_pos_max + 1) : kv_lim;
  const int n_kt = kv_end > 0 ? (kv_end + kBK - 1) / kBK : 0;
  const int per_split = (n_kt + a.n_splits - 1) / a.n_splits;
  const int kt_begin = min(n_kt, split * per_split);
  const int kt_end = min(n_kt, kt_begin + per_split);

  const float c = a.scale_log2;
  const size_t qkv_head = (size_t)bh;
  const T* Qg = reinterpret_cast<const T*>(a.q) + qkv_head * a.Lq * D;
  const T* Kg = reinterpret_cast<const T*>(a.k) + qkv_head * a.Lk * D;
  const T* Vg = reinterpret_cast<const T*>(a.v) + qkv_head * a.Lk * D;

  // ---- Q fragment (B operand of S^T = K Q^T), held for the whole loop ------
  TableFrag<BF, D> qf;
  if (qrow < a.Lq) {
    qf.load(Qg + (size_t)qrow * D, hh);
  } else {
#pragma unroll
    for (int t = 0; t < (BF ? D / 16 : D / 2); ++t) qf.v[t] = {};
  }

  // ---- per-kind prologue -----------------------------------------------------
  float bias_left_raw = 0.f, bias_right_raw = 0.f;  // T5 saturated buckets / scale
  float shaw_right = 0.f;                            // Shaw: q.(a_K[2k] - a_K[0])
  float crow_lo = 0.f, crow_hi = 0.f;                // DeBERTa: q.Kr[0], q.Kr[2k-1]
  float* arel = nullptr;
  float* slog = nullptr;
  float* cband = nullptr;
  float* pband = nullptr;
  const int ck = a.clip_k;

  if constexpr (KIND == 0) {
    const float* tab = reinterpret_cast<const float*>(a.table);
    const float inv_scale = 1.f / a.scale;
    for (int e = tid; e < a.lut_n; e += kThreads) {
      const int bk = t5_bucket_dev(a.lut_lo + e, a.t5_slots, a.t5_exact, a.t5_bidir, a.t5_nthr, a.t5_thr);
      rel[e] = tab[bk * a.H + h] * inv_scale;
    }
    const int bl = t5_bucket_dev(-(1 << 30), a.t5_slots, a.t5_exact, a.t5_bidir, a.t5_nthr, a.t5_thr);
    const int br = t5_bucket_dev(1 << 30, a.t5_slots, a.t5_exact, a.t5_bidir, a.t5_nthr, a.t5_thr);
    bias_left_raw = tab[bl * a.H + h] * inv_scale;
    bias_right_raw = tab[br * a.H + h] * inv_scale;
  } else if constexpr (KIND == 1) {
    // arel[q][r] = q.a_K[r] - q.a_K[0] for r in 0..2k, by MFMA over blocks of
    // 32 table rows; subtracting the r = 0 value is softmax-neutral and makes
    // every key beyond -k contribute exactly zero.
    arel = rel + wave * L.wave_rel_floats;
    slog = arel + kWaveRows * L.arel_stride;
    const T* ak = reinterpret_cast<const T*>(a.table);
    const int nrow = 2 * ck + 1;
    float base0 = 0.f;
    for (int rb = 0; rb * 32 < nrow; ++rb) {
      TableFrag<BF, D> af;
      af.load(ak + (size_t)min(rb * 32 + lq, nrow - 1) * D, hh);
      f32x16 acc = {};
      acc = mma_frag<BF, D>(af, qf, acc);
      if (rb == 0) base0 = __shfl(acc[0], lq);  // row 0 sits in lane lq, register 0
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = rb * 32 + acc_row(i, hh);
        if (r < nrow) arel[lq * L.arel_stride + r] = acc[i] - base0;
      }
    }
    for (int r = hh; r < L.slog_stride; r += 2) slog[lq * L.slog_stride + r] = RA_NEG_INF;
    wave_lds_fence();
    shaw_right = arel[lq * L.arel_stride + 2 * ck];
  } else {
    cband = rel + wave * L.wave_rel_floats;
    pband = cband + kWaveRows * L.cband_stride;
    const T* kr = reinterpret_cast<const T*>(a.table);
    TableFrag<BF, D> af;
    const int u = (lq == 1) ? 2 * ck - 1 : 0;
    af.load(kr + ((size_t)u * a.H + h) * D, hh);
    f32x16 acc = {};
    acc = mma_frag<BF, D>(af, qf, acc);
    crow_lo = __shfl(acc[0], lq);
    crow_hi = __shfl(acc[1], lq);
  }

  // ---- K/V tile staging (global -> registers -> LDS) -----------------------
  constexpr int VEC = BF ? 8 : 4;                 // elements per 16-byte load
  constexpr int K_CHUNKS = kBK * D / VEC;
  constexpr int K_PER_T = (K_CHUNKS + kThreads - 1) / kThreads;
  constexpr int V_UNITS = BF ? (kBK / 2) * (D / 8) : kBK * D / 4;
  constexpr int V_PER_T = (V_UNITS + kThreads - 1) / kThreads;
  u32x4 kreg[K_PER_T];
  u32x4 vreg[V_PER_T][BF ? 2 : 1];

  auto load_tile = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int r = 0; r < K_PER_T; ++r) {
      const int id = tid + r * kThreads;
      const int key = id / (D / VEC), ch = id % (D / VEC);
      u32x4 x = {};
      if (id < K_CHUNKS && k0 + key < a.Lk)
        x = *reinterpret_cast<const u32x4*>(Kg + (size_t)(k0 + key) * D + ch * VEC);
      kreg[r] = x;
    }
#pragma unroll
    for (int r = 0; r < V_PER_T; ++r) {
      const int id = tid + r * kThreads;
      if constexpr (BF) {
        const int pr = id / (D / 8), ch = id % (D / 8);
        u32x4 x0 = {}, x1 = {};
        if (id < V_UNITS) {
          if (k0 + 2 * pr < a.Lk) x0 = *reinterpret_cast<const u32x4*>(Vg + (size_t)(k0 + 2 * pr) * D + ch * 8);
          if (k0 + 2 * pr + 1 < a.Lk) x1 = *reinterpret_cast<const u32x4*>(Vg + (size_t)(k0 + 2 * pr + 1) * D + ch * 8);
        }
        vreg[r][0] = x0;
        vreg[r][1] = x1;
      } else {
        const int key = id / (D / 4), ch = id % (D / 4);
        u32x4 x = {};
        if (id < V_UNITS && k0 + key < a.Lk)
          x = *reinterpret_cast<const u32x4*>(Vg + (size_t)(k0 + key) * D + ch * 4);
        vreg[r][0] = x;
      }
    }
  };
  auto store_tile = [&](int buf) {
    T* ks = Ks + buf * kBK * L.k_stride;
#pragma unroll
    for (int r = 0; r < K_PER_T; ++r) {
      const int id = tid + r * kThreads;
      const int key = id / (D / VEC), ch = id % (D / VEC);
      if (id < K_CHUNKS) *reinterpret_cast<u32x4*>(ks + key * L.k_stride + ch * VEC) = kreg[r];
    }
    if constexpr (BF) {
      T* vt = Vs + buf * D * L.v_stride;
#pragma unroll
      for (int r = 0; r < V_PER_T; ++r) {
        const int id = tid + r * kThreads;
        const int pr = id / (D / 8), ch = id % (D / 8);
        if (id < V_UNITS) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t lo = (vreg[r][0][e >> 1] >> (16 * (e & 1))) & 0xffffu;
            const uint32_t hi = (vreg[r][1][e >> 1] >> (16 * (e & 1))) & 0xffffu;
            *reinterpret_cast<uint32_t*>(vt + (ch * 8 + e) * L.v_stride + 2 * pr) = lo | (hi << 16);
          }
        }
      }
    } else {
      T* vs = Vs + buf * kBK * L.v_stride;
#pragma unroll
      for (int r = 0; r < V_PER_T; ++r) {
        const int id = tid + r * kThreads;
        const int key = id / (D / 4), ch = id % (D / 4);
        if (id < V_UNITS) *reinterpret_cast<u32x4*>(vs + key * L.v_stride + ch * 4) = vreg[r][0];
      }
    }
  };

  // ---- running state ------------------------------------------------------
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = {};
  float m_run = RA_NEG_INF;  // raw-score running max (shared by both halves)
  float l_run = 0.f;         // this lane's partial row sum
  float lr_run = 0.f;        // Shaw: partial mass of keys at offset >= k

  if (kt_begin < kt_end) {
    load_tile(kt_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int buf = (kt - kt_begin) & 1;
    const bool has_next = kt + 1 < kt_end;
    if (has_next) load_tile(kt + 1);
    const int k0 = kt * kBK;

    if (wave_active && k0 <= (a.causal ? pw_max_real : 0x7fffffff)) {
      const T* ks = Ks + buf * kBK * L.k_stride;
      f32x16 s[NKB];
      float b_raw = 0.f;
      bool shaw_near = false, shaw_far_right = false;

      // (1) relative term into the accumulator, or into b_raw
      if constexpr (KIND == 0) {
        const int omin = k0 - pw_max, omax = k0 + kBK - 1 - pw_min;
        if (omax <= -a.t5_lsat) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) s[kb] = {};
          b_raw = bias_left_raw;
        } else if (omin >= a.t5_rsat) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) s[kb] = {};
          b_raw = bias_right_raw;
        } else {
          const float* lut = rel + (k0 - pos - a.lut_lo);
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] = lut[32 * kb + acc_row(i, hh)];
        }
      } else if constexpr (KIND == 1) {
        const int omin = k0 - pw_max, omax = k0 + kBK - 1 - pw_min;
        if (omax <= -ck) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) s[kb] = {};
        } else if (omin >= ck) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) s[kb] = {};
          b_raw = shaw_right;
          shaw_far_right = true;
        } else {
          shaw_near = true;
          const float* ar = arel + lq * L.arel_stride;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] = ar[shaw_row_dev(k0 + 32 * kb + acc_row(i, hh) - pos, ck)];
        }
      } else {
        const int tmin = pw_min - (k0 + kBK - 1), tmax = pw_max - k0;  // t = query - key
        if (tmin >= ck || tmax <= -ck) {
          const int side = tmin >= ck ? 0 : 1;
          b_raw = side == 0 ? crow_hi : crow_lo;
          const float* cc = a.colc + ((size_t)side * a.B * a.H + bh) * a.Lk_pad + k0;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              f32x4 x = *reinterpret_cast<const f32x4*>(cc + 32 * kb + 8 * g + 4 * hh);
              s[kb][4 * g + 0] = x[0]; s[kb][4 * g + 1] = x[1];
              s[kb][4 * g + 2] = x[2]; s[kb][4 * g + 3] = x[3];
            }
        } else {
          const T* kr = reinterpret_cast<const T*>(a.table);
          const T* qr = reinterpret_cast<const T*>(a.table2);
          // content-to-position band: rows t = T0 + m, m in [0, 32 + kBK - 1)
          const int T0 = pw_min - (k0 + kBK - 1);
#pragma unroll
          for (int tb = 0; tb < NKB + 1; ++tb) {
            TableFrag<BF, D> af;
            const int u = deberta_delta_dev(T0 + 32 * tb + lq, ck);
            af.load(kr + ((size_t)u * a.H + h) * D, hh);
            f32x16 acc = {};
            acc = mma_frag<BF, D>(af, qf, acc);
            float* dst = cband + lq * L.cband_stride + 32 * tb + 4 * hh;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              f32x4 x = {acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
              *reinterpret_cast<f32x4*>(dst + 8 * g) = x;
            }
          }
          // position-to-content band per 32-key block: columns n, t = T1 + n,
          // Qr row delta(key, query) = clip(-t) + k; scattered to [query][key]
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            TableFrag<BF, D> kf;
            kf.load(ks + (32 * kb + lq) * L.k_stride, hh);
            const int T1 = pw_min - (k0 + 32 * kb) - 31;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
              const int n = 32 * nb + lq;
              TableFrag<BF, D> bf;
              const int u = deberta_delta_dev(-(T1 + n), ck);
              bf.load(qr + ((size_t)u * a.H + h) * D, hh);
              f32x16 acc = {};
              acc = mma_frag<BF, D>(kf, bf, acc);
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int jl = acc_row(i, hh);
                const int sq = n + jl - 31;
                if (sq >= 0 && sq < 32) pband[sq * L.pband_stride + 32 * kb + jl] = acc[i];
              }
            }
          }
          wave_lds_fence();
          const float* crow = cband + lq * L.cband_stride + (pos - pw_min) + (kBK - 1);
          const float* prow = pband + lq * L.pband_stride;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int jt = 32 * kb + acc_row(i, hh);
              s[kb][i] = crow[-jt] + prow[jt];
            }
          wave_lds_fence();  // the next tile overwrites both bands
        }
      }

      // (2) masks: -inf enters the accumulator before q.k is added
      const bool need_mask = (a.causal && k0 + kBK - 1 > pw_min) || (k0 + kBK > kv_lim);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = k0 + 32 * kb + acc_row(i, hh);
            if (j >= kv_lim || (a.causal && j > pos)) s[kb][i] = RA_NEG_INF;
          }
      }

      // (3) S^T += K Q^T
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        TableFrag<BF, D> kf;
        kf.load(ks + (32 * kb + lq) * L.k_stride, hh);
        s[kb] = mma_frag<BF, D>(kf, qf, s[kb]);
      }

      // (4) Shaw: remember the logits of keys strictly inside the clip window
      float lr_tile = 0.f;
      if constexpr (KIND == 1) {
        if (shaw_near) {
          float* sl = slog + lq * L.slog_stride;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int off = k0 + 32 * kb + acc_row(i, hh) - pos;
              if (off > -ck && off < ck) sl[off + ck - 1] = s[kb][i] * c;
            }
        }
      }

      // (5) online softmax (exp2 domain; scale*log2e folded into one FMA)
      float mx = RA_NEG_INF;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx + b_raw);
      const float m_use = (m_new == RA_NEG_INF) ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_use) * c);
      const float off = (b_raw - m_use) * c;
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(s[kb][i], c, off));
          s[kb][i] = p;
          lsum += p;
        }
      if constexpr (KIND == 1) {
        if (shaw_far_right) {
          lr_tile = lsum;
        } else if (shaw_near) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (k0 + 32 * kb + acc_row(i, hh) - pos >= ck) lr_tile += s[kb][i];
        }
        lr_run = lr_run * alpha + lr_tile;
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;

      // (6) O^T += V^T P^T
      if constexpr (BF) {
        const T* vt = Vs + buf * D * L.v_stride;
#pragma unroll
        for (int cc = 0; cc < kBK / 16; ++cc) {
          const bf16x8 pf = pack_bf16x8(s[cc >> 1], 8 * (cc & 1));
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const T* vr = vt + (32 * db + lq) * L.v_stride + 16 * cc + 4 * hh;
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + 8);
            const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            o[db] = mma_bf16(vf, pf, o[db]);
          }
        }
      } else {
        const T* vs = Vs + buf * kBK * L.v_stride;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int cc = 0; cc < 16; ++cc) {
            const int key = 32 * kb + acc_row(cc, hh);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
              o[db] = mma_f32(vs[key * L.v_stride + 32 * db + lq], s[kb][cc], o[db]);
          }
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------
  if (!wave_active) return;
  float l_tot = l_run + __shfl_xor(l_run, 32);
  const float m_use = (m_run == RA_NEG_INF) ? 0.f : m_run;

  if constexpr (KIND == 1) {
    // value term: bins inside the clip window hold single-key masses; bin 0
    // and bin 2k take what remains of the row mass.
    const T* av = reinterpret_cast<const T*>(a.table2);
    const float lr_tot = lr_run + __shfl_xor(lr_run, 32);
    const float* sl = slog + lq * L.slog_stride;
    const int nin = 2 * ck - 1;  // bins 1 .. 2k-1
    float wsum = 0.f;
    if constexpr (BF) {
      for (int cc = 0; cc * 16 < nin; ++cc) {
        float w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 16 * cc + 8 * hh + e;
          w[e] = r < nin ? fast_exp2(sl[r] - m_use * c) : 0.f;
          wsum += w[e];
        }
        f32x16 tmp = {w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7]};
        const bf16x8 wf = pack_bf16x8(tmp, 0);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          bf16x8 vf;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 16 * cc + 8 * hh + e;
            vf[e] = r < nin ? av[(size_t)(r + 1) * D + 32 * db + lq] : (bf16)0.f;
          }
          o[db] = mma_bf16(vf, wf, o[db]);
        }
      }
    } else {
      for (int cc = 0; cc * 2 < nin; ++cc) {
        const int r = 2 * cc + hh;
        const float w = r < nin ? fast_exp2(sl[r] - m_use * c) : 0.f;
        wsum += w;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const float vv = r < nin ? av[(size_t)(r + 1) * D + 32 * db + lq] : 0.f;
          o[db] = mma_f32(vv, w, o[db]);
        }
      }
    }
    const float w_in = wsum + __shfl_xor(wsum, 32);
    const float w0 = l_tot - w_in - lr_tot;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int dd = 32 * db + acc_row(i, hh);
        o[db][i] += w0 * (float)av[dd] + lr_tot * (float)av[(size_t)(2 * ck) * D + dd];
      }
  }

  if (qrow >= a.Lq) return;
  if (a.n_splits == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T* og = reinterpret_cast<T*>(a.out) + ((size_t)bh * a.Lq + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * db + 8 * g + 4 * hh;
        if constexpr (BF) {
          f32x2 x0 = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv};
          f32x2 x1 = {o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
          bf16x2 y0 = __builtin_convertvector(x0, bf16x2), y1 = __builtin_convertvector(x1, bf16x2);
          bf16x4 y = {y0[0], y0[1], y1[0], y1[1]};
          *reinterpret_cast<bf16x4*>(og + dd) = y;
        } else {
          f32x4 y = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(og + dd) = y;
        }
      }
  } else {
    const size_t row = ((size_t)split * a.B * a.H + bh) * a.Lq + qrow;
    float* po = a.part_o + row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * db + 8 * g + 4 * hh;
        f32x4 y = {o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
        *reinterpret_cast<f32x4*>(po + dd) = y;
      }
    if (hh == 0) {
      f32x2 ml = {l_tot > 0.f ? m_use * c : RA_NEG_INF, l_tot};
      *reinterpret_cast<f32x2*>(a.part_ml + row * 2) = ml;
    }
  }
}

// Merge split-KV partials: each split holds an unnormalised output and its
// (max, sum) in the exp2 domain; rescale to the common max and normalise.
template <bool BF, int D>
__global__ __launch_bounds__(256) void relattn_combine_kernel(CombineArgs a) {
  using T = typename std::conditional<BF, bf16, float>::type;
  const int64_t nrow = (int64_t)a.BH * a.Lq;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = idx / (D / 4);
  const int ch = (int)(idx % (D / 4));
  if (row >= nrow) return;
  float M = RA_NEG_INF;
  for (int s = 0; s < a.n_splits; ++s) M = fmaxf(M, a.part_ml[((size_t)s * nrow + row) * 2]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float Lsum = 0.f;
  if (M != RA_NEG_INF) {
    for (int s = 0; s < a.n_splits; ++s) {
      const size_t r = (size_t)s * nrow + row;
      const float ms = a.part_ml[r * 2], ls = a.part_ml[r * 2 + 1];
      if (!(ls > 0.f)) continue;
      const float w = fast_exp2(ms - M);
      Lsum += w * ls;
      const f32x4 x = *reinterpret_cast<const f32x4*>(a.part_o + r * D + 4 * ch);
      acc += w * x;
    }
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  T* og = reinterpret_cast<T*>(a.out) + row * D + 4 * ch;
  if constexpr (BF) {
    f32x2 x0 = {acc[0] * inv, acc[1] * inv}, x1 = {acc[2] * inv, acc[3] * inv};
    bf16x2 y0 = __builtin_convertvector(x0, bf16x2), y1 = __builtin_convertvector(x1, bf16x2);
    bf16x4 y = {y0[0], y0[1], y1[0], y1[1]};
    *reinterpret_cast<bf16x4*>(og) = y;
  } else {
    f32x4 y = acc * inv;
    *reinterpret_cast<f32x4*>(og) = y;
  }
}

// DeBERTa per-key constants for tiles whose offsets are all clipped:
// colc[0][bh][j] = k_j . Qr[0][h] (key far before the query: d(j,i) = 0),
// colc[1][bh][j] = k_j . Qr[2k-1][h] (key far after it).  Keys in the
// padding up to Lk_pad get 0.
template <bool BF, int D>
__global__ __launch_bounds__(256) void relattn_colc_kernel(ColcArgs a) {
  using T = typename std::conditional<BF, bf16, float>::type;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.BH * a.Lk_pad;
  if (idx >= total) return;
  const int bh = (int)(idx / a.Lk_pad), j = (int)(idx % a.Lk_pad);
  const int h = bh % a.H;
  float s0 = 0.f, s1 = 0.f;
  if (j < a.Lk) {
    const T* kr = reinterpret_cast<const T*>(a.k) + ((size_t)bh * a.Lk + j) * D;
    const T* q0 = reinterpret_cast<const T*>(a.qr) + (size_t)h * D;
    const T* q1 = reinterpret_cast<const T*>(a.qr) + ((size_t)(2 * a.clip_k - 1) * a.H + h) * D;
#pragma unroll 8
    for (int e = 0; e < D; ++e) {
      const float kv = (float)kr[e];
      s0 = fmaf(kv, (float)q0[e], s0);
      s1 = fmaf(kv, (float)q1[e], s1);
    }
  }
  a.colc[(size_t)bh * a.Lk_pad + j] = s0;
  a.colc[((size_t)a.BH + bh) * a.Lk_pad + j] = s1;
}

// ----------------------------------------------------------------------------
// Host-side launch helpers (called from relattn_api.cpp)
// ----------------------------------------------------------------------------

template <int KIND, bool BF, int D>
static hipError_t launch_fwd_t(const FwdArgs& a, int grid, int lds, hipStream_t st) {
  auto kfn = relattn_fwd_kernel<KIND, BF, D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, dim3(grid), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_fwd(int kind, bool bf, int d, const FwdArgs& a, int grid, int lds, hipStream_t st) {
#define RA_CASE(K, B, DD) \
  if (kind == K && bf == B && d == DD) return launch_fwd_t<K, B, DD>(a, grid, lds, st);
  RA_CASE(0, true, 64) RA_CASE(0, true, 32) RA_CASE(0, false, 64) RA_CASE(0, false, 32)
  RA_CASE(1, true, 64) RA_CASE(1, true, 32) RA_CASE(1, false, 64) RA_CASE(1, false, 32)
  RA_CASE(2, true, 64) RA_CASE(2, true, 32) RA_CASE(2, false, 64) RA_CASE(2, false, 32)
#undef RA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_combine(bool bf, int d, const CombineArgs& a, hipStream_t st) {
  const int64_t threads = (int64_t)a.BH * a.Lq * (d / 4);
  const int grid = (int)((threads + 255) / 256);
  if (bf && d == 64) hipLaunchKernelGGL((relattn_combine_kernel<true, 64>), dim3(grid), dim3(256), 0, st, a);
  else if (bf && d == 32) hipLaunchKernelGGL((relattn_combine_kernel<true, 32>), dim3(grid), dim3(256), 0, st, a);
  else if (!bf && d == 64) hipLaunchKernelGGL((relattn_combine_kernel<false, 64>), dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((relattn_combine_kernel<false, 32>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_colc(bool bf, int d, const ColcArgs& a, hipStream_t st) {
  const int64_t threads = (int64_t)a.BH * a.Lk_pad;
  const int grid = (int)((threads + 255) / 256);
  if (bf && d == 64) hipLaunchKernelGGL((relattn_colc_kernel<true, 64>), dim3(grid), dim3(256), 0, st, a);
  else if (bf && d == 32) hipLaunchKernelGGL((relattn_colc_kernel<true, 32>), dim3(grid), dim3(256), 0, st, a);
  else if (!bf && d == 64) hipLaunchKernelGGL((relattn_colc_kernel<false, 64>), dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((relattn_colc_kernel<false, 32>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_index(const IndexArgs& a, hipStream_t st) {
  int64_t blocks = (a.n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(relattn_index_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace relattn
