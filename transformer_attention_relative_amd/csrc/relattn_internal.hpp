// Internal definitions shared by the host launcher and the gfx950 kernels.
// Not part of the public ABI (include/relattn.h is).
#pragma once

#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define RELATTN_HD __host__ __device__
#else
#define RELATTN_HD
#endif

namespace relattn {

// ---- work decomposition -------------------------------------------------
// One workgroup = 4 wave64s; each wave owns 32 consecutive query rows, so a
// workgroup covers a 128-row query tile of one (batch, head).  Keys are
// streamed in tiles of kBK rows through LDS.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveRows = 32;
constexpr int kBQ = kWaveRows * kWaves;  // 128 query rows per workgroup
constexpr int kBK = 64;                  // keys per tile

// ---- limits checked by the host before launch -----------------------------
constexpr int kT5MaxThr = 128;   // slots - exact <= 128  (num_buckets <= 256)
constexpr int kT5MaxLut = 4096;  // entries of the per-head offset -> bias table
constexpr int kShawMaxK = 32;
constexpr int kMaxSplits = 32;

// Kernel argument block (passed by value).
struct FwdArgs {
  const void *q, *k, *v;
  void *out;
  const void *table, *table2;
  const int32_t *kv_valid_len;
  float *part_o;   // split-KV partial outputs  [n_splits][B*H][Lq][d]
  float *part_ml;  // split-KV row stats        [n_splits][B*H][Lq][2] (m*c, l)
  float *colc;     // DeBERTa per-key constants [2][B*H][Lk_pad]
  int32_t B, H, Lq, Lk, Lk_pad;
  int32_t q_pos_offset, causal;
  int32_t clip_k;
  float scale;      // multiplies the raw score
  float scale_log2; // scale * log2(e)
  int32_t n_qtiles, n_splits;
  // T5 bucket thresholds and the offset lookup table geometry
  int32_t t5_slots, t5_exact, t5_bidir, t5_nthr;
  int32_t t5_lsat, t5_rsat;  // offsets <= -lsat / >= rsat share one bucket
  int32_t lut_lo, lut_n;     // table covers offsets lut_lo .. lut_lo+lut_n-1
  int32_t t5_thr[kT5MaxThr];
};

struct IndexArgs {
  const int32_t *q_pos, *k_pos;
  int32_t *out;
  int64_t n;
  int32_t kind, which, clip_k;
  int32_t t5_slots, t5_exact, t5_bidir, t5_nthr;
  int32_t t5_thr[kT5MaxThr];
};

struct CombineArgs {
  const float *part_o, *part_ml;
  void *out;
  int32_t BH, Lq, n_splits;
};

struct ColcArgs {
  const void *k, *qr;
  float *colc;
  int32_t BH, H, Lk, Lk_pad, clip_k;
};

// ---- LDS layout ------------------------------------------------------------
// K tile:  bf16 [kBK][d + 8]  (row stride keeps 16-byte rows, staggers banks)
//          fp32 [kBK][d + 4]
// V tile:  bf16 transposed [d][kBK + 4] (the PV product contracts over keys,
//          so each lane reads 4-key runs of one head-dim row)
//          fp32 row-major [kBK][d + 4]
// Both double-buffered.  After them, per kind:
//   T5      float lut[lut_n]
//   SHAW    per wave: float arel[32][2k+1], float slog[32][2k-1]
//   DEBERTA per wave: float cband[32][kBK + 36], float pband[32][kBK + 4]
struct LdsLayout {
  int k_off, v_off, rel_off, total;
  int k_stride, v_stride;       // elements
  int wave_rel_floats;          // per-wave floats of the kind region
  int arel_stride, slog_stride; // SHAW
  int cband_stride, pband_stride; // DEBERTA
};

RELATTN_HD inline LdsLayout lds_layout(int kind, bool bf16, int d, int clip_k, int lut_n) {
  LdsLayout L{};
  const int esz = bf16 ? 2 : 4;
  L.k_stride = bf16 ? d + 8 : d + 4;
  L.v_stride = bf16 ? kBK + 4 : d + 4;
  const int k_bytes = 2 * kBK * L.k_stride * esz;
  const int v_bytes = bf16 ? 2 * d * L.v_stride * esz : 2 * kBK * L.v_stride * esz;
  L.k_off = 0;
  L.v_off = k_bytes;
  L.rel_off = (k_bytes + v_bytes + 15) & ~15;
  int rel_bytes = 0;
  if (kind == 0) {
    rel_bytes = lut_n * 4;
  } else if (kind == 1) {
    L.arel_stride = 2 * clip_k + 1;
    L.slog_stride = 2 * clip_k - 1 > 0 ? 2 * clip_k - 1 : 1;
    L.wave_rel_floats = kWaveRows * (L.arel_stride + L.slog_stride);
    rel_bytes = kWaves * L.wave_rel_floats * 4;
  } else {
    L.cband_stride = kBK + 36;   // 32 + kBK - 1 band rows, padded to a 16-byte multiple
    L.pband_stride = kBK + 4;
    L.wave_rel_floats = kWaveRows * (L.cband_stride + L.pband_stride);
    rel_bytes = kWaves * L.wave_rel_floats * 4;
  }
  L.total = L.rel_off + ((rel_bytes + 15) & ~15);
  return L;
}

}  // namespace relattn
