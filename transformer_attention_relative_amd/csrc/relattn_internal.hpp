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
// A workgroup is NW wave64s; each wave owns QB blocks of 32 consecutive query
// rows of one (batch, head).  Keys stream through LDS in tiles of kBK rows.
constexpr int kBK = 64;        // keys per tile
constexpr int kBlockRows = 32; // query rows per MFMA block

// ---- limits checked by the host before launch -----------------------------
constexpr int kT5MaxThr = 128;   // slots - exact <= 128  (num_buckets <= 256)
constexpr int kT5MaxLut = 4096;  // entries of the per-head offset -> bias table
constexpr int kShawMaxK = 32;
constexpr int kMaxSplits = 32;
constexpr int kNumXcd = 8;        // MI355X: 8 XCDs of 32 CUs
constexpr int kCuPerXcd = 32;
constexpr int kMaxSortSeqs = 64;  // sequences a workgroup orders by valid length (one wave)
constexpr int kLdsPerCU = 160 * 1024;
// device scratch of relattn_fwd_noalloc (one array per GPU, fixed size)
constexpr size_t kScratchBytes = size_t(16) << 20;

// Kernel argument block (passed by value).
struct FwdArgs {
  const void *q, *k, *v;
  void *out;
  const void *table, *table2;
  const int32_t *kv_valid_len;
  float *part_o;   // split-KV partial outputs  [n_splits][B*H][Lq][d]
  float *part_ml;  // split-KV row stats        [n_splits][B*H][Lq][2] (log2 max, sum)
  const void *colc; // per-key constants [B*H][Lk] x 8 bytes (relattn_colc_kernel):
                    // DeBERTa k_j.Qr[0], k_j.Qr[2k-1]; Transformer-XL u.k_j
  const void *colc2; // Transformer-XL per-distance constants v.E[r] [H][clip_k] x 8 bytes
  float *lse;       // [B*H][Lq] row log-sum-exp (natural log) or NULL
  int32_t B, H, Lq, Lk;
  int32_t q_pos_offset;  // query row 0 minus key row 0 (absolute positions; may be < 0)
  int32_t causal;
  int32_t clip_k;
  float scale;      // multiplies the raw score
  float scale_log2; // scale * log2(e)
  int32_t n_qtiles, n_splits;
  int32_t grid;          // workgroups of this launch
  int32_t cu_slots;      // workgroups of this launch one CU holds at once
  int32_t sort_items;    // order work by sequence valid length (non-causal, B <= 64)
  // T5 bucket thresholds and the offset lookup table geometry
  int32_t t5_slots, t5_exact, t5_bidir, t5_nthr;
  int32_t t5_lsat, t5_rsat;  // offsets <= -lsat / >= rsat share one bucket
  int32_t lut_lo, lut_n;     // table covers offsets lut_lo .. lut_lo+lut_n-1
  int32_t t5_thr[kT5MaxThr];  // entries from t5_nthr on hold INT32_MAX
};

struct IndexArgs {
  const int32_t *q_pos, *k_pos;
  int32_t *out;
  int64_t n;
  int32_t kind, which, clip_k;
  int32_t t5_slots, t5_exact, t5_bidir, t5_nthr;
  int32_t t5_thr[kT5MaxThr];  // entries from t5_nthr on hold INT32_MAX
};

// One job of relattn_colc_kernel: for g < G, r < R, entry g*R + r of `out`
// holds (x_gr . a0_h, x_gr . a1_h) in float32 (8 bytes: a bf16 hi + lo pair
// per constant for bf16 inputs, the float pair for float32), where
// x_gr = x + (g * x_sg + r * x_sr) * d, h = g % H, a0_h = a0 + h * d,
// a1_h = a1 + h * d (a1 may be NULL: the second constant is 0).
struct ColcJob {
  const void *x, *a0, *a1;
  void *out;
  int64_t x_sg, x_sr;
  int32_t G, R, H;
};

struct ColcArgs {
  ColcJob job[2];
  int32_t njobs;  // 1 or 2
};

struct CombineArgs {
  const float *part_o, *part_ml;
  void *out;
  float *lse;  // [BH][Lq] or NULL
  int32_t BH, Lq, n_splits;
};

// Kernel variant: waves per workgroup and 32-row query blocks per wave.
struct Variant {
  int nw, qb;
};

// Key/value stages in flight (global -> LDS ring depth) per kind.
RELATTN_HD constexpr int num_stages(int kind, bool bf16, int d) {
  return d > 64 ? 2 : ((kind == 0 || kind == 3) ? (bf16 ? 4 : 3) : 2);
}

// Key split inside a workgroup: T5 and ALiBi workgroups of eight waves are
// two halves of four waves over the same query rows, each running half of
// the workgroup's key tiles with its own stage ring (decode-like shapes,
// where four-wave workgroups leave one wave per SIMD); 1 = no split.
RELATTN_HD constexpr int key_split(int kind, int nw) {
  return ((kind == 0 || kind == 3) && nw == 8) ? 2 : 1;
}

// Shaw bin slots of a query row: slot s holds the probability of the key at
// offset s - k for the offsets strictly inside the clip window (s = 1 ..
// 2k-1, the a_V row index); slots 0 and 2k take the keys at offsets <= -k
// and >= k (overwritten, never read as bins); padded to whole MFMA
// contraction chunks.
RELATTN_HD constexpr int shaw_bin_slots(int clip_k) { return ((2 * clip_k + 1) + 15) / 16 * 16; }

// Row stride (elements) of the Shaw bin rows in LDS: the slots plus 16 bytes,
// an odd multiple of 16 bytes, so that the per-lane bin stores of the 32
// rows of a block spread over 16 bank groups instead of 4.
RELATTN_HD constexpr int shaw_bin_stride(int clip_k, int esz) {
  return shaw_bin_slots(clip_k) + (((shaw_bin_slots(clip_k) * esz / 16) % 2 == 0) ? 16 / esz : 0);
}

// ---- LDS layout ------------------------------------------------------------
// Stage s holds the K tile then the V tile of one key tile, each kBK rows of
// d elements (with a key split, each half has its own ring of stages, half h
// at h * stages * stage_bytes), each kBK rows of
// d elements, row-major; 16-byte chunks are XOR-swizzled within a row
// (chunk c of row r sits in slot c ^ (r & 7)) so that column reads of
// consecutive rows hit different banks.  After the stages, per kind:
//   T5      float lut4[4][lut_stride]: four copies of bias[offset]*log2(e),
//           copy c shifted by c entries, so any 4 consecutive offsets are one
//           aligned 16-byte read
//   SHAW    per wave: float arel[rows][2k+2] (q.a_K[r] - q.a_K[0]); per
//           wave: bin rows [rows][bin_slots] (input dtype), one per query
//           row of the wave; bf16 only: a_V^T [d][bin_slots] (column s =
//           a_V row s for s = 1 .. 2k-1, zero elsewhere); per wave: a_V
//           rows 0 and 2k [2][d] (input dtype)
//   DEBERTA per wave: float band[32][kCbandStride], the content-to-position
//           band [query][m] and then the position-to-content band [key][n];
//           bf16, d = 64, 8 waves: the Kr ring [kRingRows][d] (rows
//           XOR-swizzled like the K tiles); bf16: the head's clipped Qr rows
//           Qr[0] and Qr[2k-1] [2][d]
//   TXL     per wave: float band[32][kCbandStride], the position band
//           [query][m]; bf16, d = 64, 8 waves: the E ring, as DeBERTa's
constexpr int kCbandStride = 68;  // 64 band columns, padded: rows stay 16-byte aligned and
                                  // a query's diagonal (stride 69) hits distinct banks

struct LdsLayout {
  int stage_bytes, tile_bytes, rel_off, total;
  int lut_stride;
  int arel_stride, arel_wave_bytes, wscr_off, wscr_wave_bytes, avt_off, avend_off;
  int deb_wave_floats;
  int ring_off;  // DeBERTa / TXL bf16, d = 64, 8 waves: ring of band rows (kRingRows x 128 B)
  int qr_off;    // DeBERTa bf16: the clipped Qr rows [2][d]
};

// The band rows of a workgroup of 8 waves x 32 query rows (DeBERTa's Kr
// rows of the content-to-position band, Transformer-XL's encodings E): a
// tile of 64 keys reads 320 consecutive rows, the next tile 64 rows below
// them, so a ring of 384 rows holds one tile's rows and the next tile's new
// ones.
constexpr int kRingRows = 384;
RELATTN_HD constexpr bool band_ring(int kind, bool bf16, int d, int nw) {
  return (kind == 2 || kind == 4) && bf16 && d == 64 && nw == 8;
}

RELATTN_HD inline LdsLayout lds_layout(int kind, bool bf16, int d, int qb, int nw, int clip_k,
                                       int lut_n) {
  LdsLayout L{};
  const int esz = bf16 ? 2 : 4;
  L.tile_bytes = kBK * d * esz;
  L.stage_bytes = 2 * L.tile_bytes;
  L.rel_off = key_split(kind, nw) * num_stages(kind, bf16, d) * L.stage_bytes;
  int rel_bytes = 0;
  if (kind == 0) {
    // stride = 16 (mod 64) floats: four lanes reading the four copies at one
    // aligned position land in different bank groups
    L.lut_stride = ((lut_n + 3) + 63 - 16) / 64 * 64 + 16;
    rel_bytes = 4 * L.lut_stride * 4;
  } else if (kind == 1) {
    const int rows = kBlockRows * qb;
    const int nbin = shaw_bin_slots(clip_k);
    // even stride: a row read at offset (const - row) walks 33 banks per row
    L.arel_stride = 2 * clip_k + 2;
    L.arel_wave_bytes = (rows * L.arel_stride * 4 + 15) / 16 * 16;  // float32
    L.wscr_off = nw * L.arel_wave_bytes;
    L.wscr_wave_bytes = rows * shaw_bin_stride(clip_k, esz) * esz;
    L.avt_off = L.wscr_off + nw * L.wscr_wave_bytes;
    L.avend_off = L.avt_off + (bf16 ? d * nbin * 2 : 0);
    rel_bytes = L.avend_off + nw * 2 * d * esz;  // per wave: a_V rows 0 and 2k
  } else if (kind == 2 || kind == 4) {
    L.deb_wave_floats = kBlockRows * kCbandStride;
    rel_bytes = nw * L.deb_wave_floats * 4;
    if (band_ring(kind, bf16, d, nw)) {
      L.ring_off = rel_bytes;
      rel_bytes += kRingRows * d * 2;
    }
    if (kind == 2 && bf16) {
      L.qr_off = rel_bytes;
      rel_bytes += 2 * d * 2;
    }
  }  // ALIBI: nothing beyond the stages
  L.total = L.rel_off + ((rel_bytes + 15) & ~15);
  return L;
}

}  // namespace relattn
