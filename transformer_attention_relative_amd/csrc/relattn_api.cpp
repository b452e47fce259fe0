// Host side of the C ABI declared in include/relattn.h: argument
// validation (before any HIP call), T5 bucket thresholds, workspace
// sizing, split-KV planning and kernel dispatch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "relattn.h"
#include "relattn_internal.hpp"

namespace relattn {
hipError_t launch_fwd(int kind, bool bf, int d, Variant v, const FwdArgs& a, int grid, int lds,
                      hipStream_t st);
bool fwd_variant_built(int kind, bool bf, int d, Variant v);
hipError_t launch_combine(bool bf, int d, const CombineArgs& a, hipStream_t st);
hipError_t launch_colc(bool bf, int d, const ColcArgs& a, hipStream_t st);
hipError_t launch_index(const IndexArgs& a, hipStream_t st);
hipError_t scratch_address(void** ptr);
}  // namespace relattn

using namespace relattn;

static_assert(kScratchBytes == RELATTN_NOALLOC_SCRATCH_BYTES,
              "the device scratch array and the header disagree on its size");

namespace {

thread_local std::string g_last_error;

relattn_status fail(relattn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

relattn_status ok() {
  g_last_error.clear();
  return RELATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kNumCU = 256;  // MI355X compute units (split-KV planning only)

// Within-direction T5 slot of a distance, evaluated as on the pages
// ([RPE] "T5: one scalar per head, looked up by bucket"): float64 logarithm
// ratio, truncated, capped at the last slot.
int t5_slot_fp64(int64_t dist, int slots, int exact, int max_distance) {
  if (dist < exact) return (int)dist;
  const double frac = std::log((double)dist / (double)exact) /
                      std::log((double)max_distance / (double)exact);
  const double scaled = frac * (double)(slots - exact);
  const int64_t slot = (int64_t)exact + (int64_t)scaled;
  return slot > slots - 1 ? slots - 1 : (int)slot;
}

struct T5Plan {
  int slots, exact, nthr, lsat, rsat, lut_lo, lut_n;
  int thr[kT5MaxThr];
};

relattn_status t5_plan(int num_buckets, int max_distance, int bidirectional, int wave_rows, T5Plan* P) {
  if (num_buckets < 2 || num_buckets > 256)
    return fail(RELATTN_ERR_INVALID, "T5 num_buckets=%d outside [2, 256]", num_buckets);
  const int slots = bidirectional ? num_buckets / 2 : num_buckets;
  const int exact = slots / 2;
  if (exact < 1)
    return fail(RELATTN_ERR_INVALID, "T5 num_buckets=%d leaves no exact-distance slot", num_buckets);
  if (max_distance <= exact)
    return fail(RELATTN_ERR_INVALID, "T5 max_distance=%d must exceed the exact range %d",
                max_distance, exact);
  P->slots = slots;
  P->exact = exact;
  P->nthr = slots - exact;
  if (P->nthr > kT5MaxThr) return fail(RELATTN_ERR_UNSUPPORTED, "too many T5 log slots");
  // thr[m] = smallest distance whose slot reaches exact + m.  The slot is
  // monotone in the distance and reaches the last slot by max_distance, so
  // a binary search over [exact, max_distance] finds each threshold.
  P->thr[0] = exact;
  for (int m = 1; m < P->nthr; ++m) {
    int64_t lo = exact, hi = max_distance;
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (t5_slot_fp64(mid, slots, exact, max_distance) >= exact + m) hi = mid;
      else lo = mid + 1;
    }
    P->thr[m] = (int)lo;
  }
  P->lsat = P->thr[P->nthr - 1];
  P->rsat = bidirectional ? P->lsat : 0;
  const int W = wave_rows + kBK - 1;  // offsets spanned by one wave's tile
  P->lut_lo = -P->lsat - W;
  P->lut_n = P->lsat + P->rsat + 2 * W + 1;
  return RELATTN_OK;
}

struct Plan {
  bool bf;
  bool colc;  // the row-constant pre-pass runs before the forward kernel
  float scale;
  Variant var;
  int n_qtiles, n_splits, grid, lds, cu_slots;
  size_t off_part_o, off_part_ml, off_colc, off_colc2, ws_bytes;
  T5Plan t5;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

relattn_status plan_problem(const relattn_params* p, Plan* P) {
  if (!p) return fail(RELATTN_ERR_INVALID, "params is NULL");
  if (p->kind < 0 || p->kind > 4) return fail(RELATTN_ERR_INVALID, "unknown kind %d", p->kind);
  if (p->dtype != RELATTN_FP32 && p->dtype != RELATTN_BF16)
    return fail(RELATTN_ERR_INVALID, "unknown dtype %d", p->dtype);
  if (p->B < 1 || p->H < 1 || p->Lq < 1 || p->Lk < 1)
    return fail(RELATTN_ERR_INVALID, "B, H, Lq, Lk must be >= 1 (got %d %d %d %d)",
                p->B, p->H, p->Lq, p->Lk);
  if (p->d < 1) return fail(RELATTN_ERR_INVALID, "d=%d must be >= 1", p->d);
  if (p->d != 32 && p->d != 64 && !(p->d == 128 && p->dtype == RELATTN_BF16))
    return fail(RELATTN_ERR_UNSUPPORTED, "d=%d (built: 32, 64; 128 in bfloat16)", p->d);
  if ((int64_t)p->B * p->H > (1 << 24)) return fail(RELATTN_ERR_UNSUPPORTED, "B*H too large");
  if (p->Lq > (1 << 26) || p->Lk > (1 << 26))
    return fail(RELATTN_ERR_UNSUPPORTED, "sequence length above 2^26");
  if (p->q_pos_offset < 0) return fail(RELATTN_ERR_INVALID, "q_pos_offset=%d < 0", p->q_pos_offset);
  if ((int64_t)p->q_pos_offset + p->Lq > (1 << 28))
    return fail(RELATTN_ERR_UNSUPPORTED, "query positions above 2^28");
  if (p->k_pos_offset < 0) return fail(RELATTN_ERR_INVALID, "k_pos_offset=%d < 0", p->k_pos_offset);
  if ((int64_t)p->k_pos_offset + p->Lk > (1 << 28))
    return fail(RELATTN_ERR_UNSUPPORTED, "key positions above 2^28");
  if (!(p->scale >= 0.f) || std::isinf(p->scale))
    return fail(RELATTN_ERR_INVALID, "scale must be finite and >= 0 (0 = default)");
  if (!p->table) return fail(RELATTN_ERR_INVALID, "table is NULL");
  if (p->lse && (reinterpret_cast<uintptr_t>(p->lse) & 3))
    return fail(RELATTN_ERR_INVALID, "lse must be 4-byte aligned");
  if (p->kind == RELATTN_ALIBI && (reinterpret_cast<uintptr_t>(p->table) & 3))
    return fail(RELATTN_ERR_INVALID, "ALiBi slopes must be 4-byte aligned");
  if (p->kind == RELATTN_SHAW || p->kind == RELATTN_DEBERTA || p->kind == RELATTN_TXL) {
    if (!p->table2) return fail(RELATTN_ERR_INVALID, "table2 is NULL");
    if (!aligned16(p->table) || !aligned16(p->table2))
      return fail(RELATTN_ERR_INVALID, "tables must be 16-byte aligned");
    if (p->clip_k < 1) return fail(RELATTN_ERR_INVALID, "clip_k=%d must be >= 1", p->clip_k);
    if (p->kind == RELATTN_SHAW && p->clip_k > kShawMaxK)
      return fail(RELATTN_ERR_UNSUPPORTED, "Shaw clip_k=%d above %d", p->clip_k, kShawMaxK);
    if (p->kind == RELATTN_DEBERTA && p->clip_k > 65536)
      return fail(RELATTN_ERR_UNSUPPORTED, "DeBERTa clip_k=%d above 65536", p->clip_k);
  }
  if (p->kind == RELATTN_TXL) {
    // causal, and a relative-encoding row for every distance a query can see
    if (!p->causal) return fail(RELATTN_ERR_INVALID, "Transformer-XL attention must be causal");
    const int64_t far = (int64_t)p->q_pos_offset + p->Lq - 1 - p->k_pos_offset;
    if (far >= p->clip_k)
      return fail(RELATTN_ERR_INVALID, "Transformer-XL encodings have %d rows; distances up to %lld are visible",
                  p->clip_k, (long long)far);
  }
  P->bf = p->dtype == RELATTN_BF16;
  const float dflt = p->kind == RELATTN_DEBERTA ? 1.f / std::sqrt(3.f * p->d) : 1.f / std::sqrt((float)p->d);
  P->scale = p->scale > 0.f ? p->scale : dflt;

  // Kernel variant: 4 waves.  DeBERTa: 32 rows per wave (its near-block band
  // tile takes 8.5 KiB of LDS per wave; two workgroups fit a CU).  T5 /
  // ALiBi: 64 rows per wave when there are enough workgroups to fill two per
  // CU (one LDS fragment then feeds two MFMAs) and the LDS fits two
  // workgroups per CU, else 32 rows per wave.  float32 always uses 32 rows
  // per wave (its fragments are twice as large).
  const int BH = p->B * p->H;
  auto lds_for = [&](Variant v, int* total, int* lut_n) -> relattn_status {
    *lut_n = 0;
    if (p->kind == RELATTN_T5) {
      relattn_status s = t5_plan(p->num_buckets, p->max_distance, p->bidirectional,
                                 kBlockRows * v.qb, &P->t5);
      if (s != RELATTN_OK) return s;
      if (P->t5.lut_n > kT5MaxLut)
        return fail(RELATTN_ERR_UNSUPPORTED, "T5 saturation distance %d too large for the LDS table",
                    P->t5.lsat);
      *lut_n = P->t5.lut_n;
    }
    *total = lds_layout(p->kind, P->bf, p->d, v.qb, v.nw, p->clip_k, *lut_n).total;
    return RELATTN_OK;
  };
  Variant var = Variant{4, 1};
  // DeBERTa / Transformer-XL bf16, d = 64: eight waves share one ring of
  // band rows in LDS (DeBERTa with a narrow clip window has few band blocks
  // and keeps two four-wave workgroups per CU)
  if (((p->kind == RELATTN_DEBERTA && p->clip_k >= 64) || p->kind == RELATTN_TXL) && P->bf &&
      p->d == 64)
    var = Variant{8, 1};
  int lds_total = 0, lut_n = 0;
  // (Shaw keeps one query block per wave: with its per-row float32
  // relative-key logits, two blocks would leave one workgroup per CU, and one
  // block per wave measured as fast as two on the causal 4096-token workload)
  if ((p->kind == RELATTN_T5 || p->kind == RELATTN_ALIBI) && P->bf && p->d <= 64) {
    const int64_t wgs2 = (int64_t)BH * ((p->Lq + 4 * 64 - 1) / (4 * 64));
    int t2 = 0;
    if (wgs2 >= 2 * kNumCU && lds_for(Variant{4, 2}, &t2, &lut_n) == RELATTN_OK &&
        t2 <= kLdsPerCU / 2)
      var = Variant{4, 2};
  }
  if ((p->kind == RELATTN_T5 || p->kind == RELATTN_ALIBI) && P->bf && p->d <= 64 &&
      p->Lq > kBlockRows && var.qb == 1) {
    // Decode-like shapes with several query blocks (a block of cached
    // queries against a long key range): four-wave workgroups would leave
    // one wave per SIMD, so each workgroup takes eight waves as two halves
    // over the same query rows, each half running half of the key tiles
    const int64_t wgs4 = (int64_t)BH * ((p->Lq + 4 * kBlockRows - 1) / (4 * kBlockRows));
    int t8 = 0;
    if (wgs4 < kNumCU && lds_for(Variant{8, 1}, &t8, &lut_n) == RELATTN_OK && t8 <= kLdsPerCU)
      var = Variant{8, 1};
  }
  relattn_status ls = lds_for(var, &lds_total, &lut_n);
  if (ls != RELATTN_OK) return ls;
  if (lds_total > kLdsPerCU && p->kind == RELATTN_SHAW && !P->bf) {
    // float32 Shaw with a wide clip window: two waves per workgroup
    var = Variant{2, 1};
    ls = lds_for(var, &lds_total, &lut_n);
    if (ls != RELATTN_OK) return ls;
  }
  if (!fwd_variant_built(p->kind, P->bf, p->d, var)) return fail(RELATTN_ERR_UNSUPPORTED, "no kernel variant");
  P->var = var;
  const int BQ = kBlockRows * var.qb * var.nw / key_split(p->kind, var.nw);  // query rows per workgroup
  P->n_qtiles = (p->Lq + BQ - 1) / BQ;
  const int64_t wgs = (int64_t)BH * P->n_qtiles;
  // keys visible to the last query row (causal): key index j sees rows with
  // q_pos_offset + i >= k_pos_offset + j
  const int64_t qoff = (int64_t)p->q_pos_offset - p->k_pos_offset;
  const int64_t kv_reach =
      p->causal ? std::max<int64_t>(0, std::min<int64_t>(p->Lk, qoff + p->Lq)) : p->Lk;
  const int64_t kt = (kv_reach + kBK - 1) / kBK;
  int splits = 1;
  // Split the key range only when there are fewer workgroups than CUs
  // (decode-like shapes); the partials cost an extra HBM round trip.  A
  // query tile of one block (a decode step) aims at two workgroups per CU;
  // more rows per tile aim at one (each split then writes as many partial
  // rows, and a 128-query step over 4096 keys ran 7% faster with 4 splits
  // than with 8, a one-token step 7% slower)
  if (wgs < kNumCU && kt >= 8) {
    const int64_t per_cu = std::min<int64_t>(p->Lq, BQ) <= kBlockRows ? 2 : 1;
    int64_t want = (per_cu * kNumCU + wgs - 1) / wgs;
    want = std::min<int64_t>(want, kt / 4);
    want = std::min<int64_t>(want, kMaxSplits);
    splits = (int)std::max<int64_t>(1, want);
  }
  P->n_splits = splits;
  const int64_t grid = wgs * splits;
  if (grid > 0x7fffffff) return fail(RELATTN_ERR_UNSUPPORTED, "grid too large");
  P->grid = (int)grid;
  if (lds_total > kLdsPerCU) return fail(RELATTN_ERR_UNSUPPORTED, "LDS need %d B above 160 KiB", lds_total);
  P->lds = lds_total;
  // workgroups a CU holds at once: LDS, and the register budget the kernels
  // are built for (two workgroups, one for 128-wide Shaw, DeBERTa and
  // Transformer-XL and for eight-wave workgroups)
  {
    const int by_regs = (p->d > 64 && p->kind != RELATTN_T5 && p->kind != RELATTN_ALIBI) ? 1 : 8 / var.nw;
    const int by_lds = lds_total > 0 ? kLdsPerCU / lds_total : by_regs;
    P->cu_slots = std::max(1, std::min(by_regs, by_lds));
  }

  // the row-constant pre-pass (Transformer-XL; DeBERTa in float32: bfloat16
  // DeBERTa forms its per-key constants with MFMA inside the forward kernel)
  // runs one lane per 16-byte chunk of every (head, key) row and every
  // (head, encoding row)
  const bool colc = p->kind == RELATTN_TXL || (p->kind == RELATTN_DEBERTA && !P->bf);
  P->colc = colc;
  if (colc &&
      ((int64_t)BH * p->Lk + (p->kind == RELATTN_TXL ? (int64_t)p->H * p->clip_k : 0)) *
              (p->d * (P->bf ? 2 : 4) / 16) >= ((int64_t)1 << 31))
    return fail(RELATTN_ERR_UNSUPPORTED, "B*H*Lk too large for the row-constant pass");
  size_t off = 0;
  P->off_part_o = P->off_part_ml = P->off_colc = P->off_colc2 = 0;
  if (splits > 1) {
    P->off_part_o = off;
    off = align256(off + (size_t)splits * BH * p->Lq * p->d * sizeof(float));
    P->off_part_ml = off;
    off = align256(off + (size_t)splits * BH * p->Lq * 2 * sizeof(float));
  }
  if (colc) {
    // per-key constants, 8 bytes per (head, key)
    P->off_colc = off;
    off = align256(off + (size_t)BH * p->Lk * 8);
  }
  if (p->kind == RELATTN_TXL) {
    // per-distance constants v.E[r], 8 bytes per (head, encoding row)
    P->off_colc2 = off;
    off = align256(off + (size_t)p->H * p->clip_k * 8);
  }
  P->ws_bytes = off;
  return RELATTN_OK;
}

}  // namespace

extern "C" {

int32_t relattn_abi_version(void) { return RELATTN_ABI_VERSION; }

const char* relattn_status_str(relattn_status s) {
  switch (s) {
    case RELATTN_OK: return "ok";
    case RELATTN_ERR_INVALID: return "invalid argument";
    case RELATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case RELATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case RELATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* relattn_last_error(void) { return g_last_error.c_str(); }

relattn_status relattn_t5_thresholds(int32_t num_buckets, int32_t max_distance, int32_t bidirectional,
                                     int32_t* thr, int32_t cap, int32_t* count) {
  T5Plan P;
  relattn_status s = t5_plan(num_buckets, max_distance, bidirectional, kBlockRows, &P);
  if (s != RELATTN_OK) return s;
  if (count) *count = P.nthr;
  if (thr)
    for (int m = 0; m < P.nthr && m < cap; ++m) thr[m] = P.thr[m];
  return ok();
}

relattn_status relattn_workspace_bytes(const relattn_params* p, size_t* bytes) {
  if (!bytes) return fail(RELATTN_ERR_INVALID, "bytes is NULL");
  Plan P;
  relattn_status s = plan_problem(p, &P);
  if (s != RELATTN_OK) return s;
  *bytes = P.ws_bytes;
  return ok();
}

}  // extern "C"

namespace {

relattn_status check_tensors(const void* q, const void* k, const void* v, const void* out) {
  if (!q || !k || !v || !out) return fail(RELATTN_ERR_INVALID, "q, k, v and out must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(RELATTN_ERR_INVALID, "q, k, v and out must be 16-byte aligned");
  return RELATTN_OK;
}

// Enqueue the kernels of one planned call; `workspace` holds at least
// P.ws_bytes bytes (checked by the caller).
relattn_status enqueue(const relattn_params* p, const Plan& P, const void* q, const void* k,
                       const void* v, void* out, void* workspace, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  FwdArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.table = p->table; a.table2 = p->table2;
  a.kv_valid_len = p->kv_valid_len;
  a.lse = p->lse;
  a.B = p->B; a.H = p->H; a.Lq = p->Lq; a.Lk = p->Lk;
  // the kernels see positions relative to key row 0 (may be negative)
  a.q_pos_offset = p->q_pos_offset - p->k_pos_offset;
  a.causal = p->causal ? 1 : 0;
  a.clip_k = p->clip_k;
  a.scale = P.scale;
  a.scale_log2 = P.scale * 1.4426950408889634f;
  a.n_qtiles = P.n_qtiles;
  a.n_splits = P.n_splits;
  a.grid = P.grid;
  a.cu_slots = P.cu_slots;
  // without a causal mask a workgroup's work is its sequence's valid length
  a.sort_items = (p->kv_valid_len != nullptr && !p->causal && p->B > 1 && p->B <= kMaxSortSeqs) ? 1 : 0;
  if (P.n_splits > 1) {
    a.part_o = reinterpret_cast<float*>(ws + P.off_part_o);
    a.part_ml = reinterpret_cast<float*>(ws + P.off_part_ml);
  }
  if (p->kind == RELATTN_T5) {
    a.t5_slots = P.t5.slots; a.t5_exact = P.t5.exact;
    a.t5_bidir = p->bidirectional ? 1 : 0; a.t5_nthr = P.t5.nthr;
    a.t5_lsat = P.t5.lsat; a.t5_rsat = P.t5.rsat;
    a.lut_lo = P.t5.lut_lo; a.lut_n = P.t5.lut_n;
    for (int m = 0; m < kT5MaxThr; ++m) a.t5_thr[m] = m < P.t5.nthr ? P.t5.thr[m] : INT32_MAX;
  }
  hipError_t e = hipSuccess;
  if (P.colc) {
    const size_t esz = P.bf ? 2 : 4;
    const char* t2 = reinterpret_cast<const char*>(p->table2);
    ColcArgs ca;
    std::memset(&ca, 0, sizeof ca);
    a.colc = ws + P.off_colc;
    // rows of K: key j of head bh at k + (bh * Lk + j) * d
    ColcJob& kj = ca.job[0];
    kj.x = k; kj.out = ws + P.off_colc;
    kj.x_sg = p->Lk; kj.x_sr = 1; kj.G = p->B * p->H; kj.R = p->Lk; kj.H = p->H;
    if (p->kind == RELATTN_DEBERTA) {
      // k_j.Qr[0][h] and k_j.Qr[2k-1][h] (Qr [2k, H, d])
      kj.a0 = t2;
      kj.a1 = t2 + (size_t)(2 * p->clip_k - 1) * p->H * p->d * esz;
      ca.njobs = 1;
    } else {
      // u_h.k_j (table2 row 0 = u [H, d]) and v_h.E[r, h] (table2 row 1 = v;
      // E [clip_k, H, d]: row r of head h at E + (r * H + h) * d)
      kj.a0 = t2;
      kj.a1 = nullptr;
      ColcJob& ej = ca.job[1];
      ej.x = p->table; ej.a0 = t2 + (size_t)p->H * p->d * esz; ej.a1 = nullptr;
      ej.out = ws + P.off_colc2;
      ej.x_sg = 1; ej.x_sr = p->H; ej.G = p->H; ej.R = p->clip_k; ej.H = p->H;
      ca.njobs = 2;
      a.colc2 = ws + P.off_colc2;
    }
    e = launch_colc(P.bf, p->d, ca, st);
    if (e != hipSuccess) return fail(RELATTN_ERR_HIP, "row-constant launch: %s", hipGetErrorString(e));
  }
  e = launch_fwd(p->kind, P.bf, p->d, P.var, a, P.grid, P.lds, st);
  if (e != hipSuccess) return fail(RELATTN_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  if (P.n_splits > 1) {
    CombineArgs cb{a.part_o, a.part_ml, out, p->lse, p->B * p->H, p->Lq, P.n_splits};
    e = launch_combine(P.bf, p->d, cb, st);
    if (e != hipSuccess) return fail(RELATTN_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

relattn_status relattn_fwd(const relattn_params* p, const void* q, const void* k, const void* v,
                           void* out, void* workspace, size_t workspace_bytes, void* stream) {
  Plan P;
  relattn_status s = plan_problem(p, &P);
  if (s != RELATTN_OK) return s;
  s = check_tensors(q, k, v, out);
  if (s != RELATTN_OK) return s;
  if (P.ws_bytes > 0 && (!workspace || workspace_bytes < P.ws_bytes))
    return fail(RELATTN_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", P.ws_bytes,
                workspace_bytes, workspace ? "" : ", NULL");
  if (workspace && !aligned16(workspace)) return fail(RELATTN_ERR_INVALID, "workspace must be 16-byte aligned");
  return enqueue(p, P, q, k, v, out, workspace, stream);
}

relattn_status relattn_fwd_noalloc(const relattn_params* p, const void* q, const void* k,
                                   const void* v, void* out, void* stream) {
  Plan P;
  relattn_status s = plan_problem(p, &P);
  if (s != RELATTN_OK) return s;
  s = check_tensors(q, k, v, out);
  if (s != RELATTN_OK) return s;
  if (P.ws_bytes > kScratchBytes)
    return fail(RELATTN_ERR_WORKSPACE,
                "problem needs %zu bytes of workspace; the fixed device scratch of "
                "relattn_fwd_noalloc holds %zu (use relattn_fwd with a workspace)",
                P.ws_bytes, kScratchBytes);
  void* ws = nullptr;
  if (P.ws_bytes > 0) {
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess)
      return fail(RELATTN_ERR_HIP, "device scratch address: %s", hipGetErrorString(e));
  }
  return enqueue(p, P, q, k, v, out, ws, stream);
}

relattn_status relattn_rel_index(const relattn_params* p, const int32_t* q_pos, const int32_t* k_pos,
                                 int64_t n, int32_t which, int32_t* idx_out, void* stream) {
  if (!p) return fail(RELATTN_ERR_INVALID, "params is NULL");
  if (p->kind < 0 || p->kind > 4) return fail(RELATTN_ERR_INVALID, "unknown kind %d", p->kind);
  if (n < 0) return fail(RELATTN_ERR_INVALID, "n=%lld < 0", (long long)n);
  if (which != 0 && which != 1) return fail(RELATTN_ERR_INVALID, "which=%d not 0 or 1", which);
  if (which == 1 && p->kind != RELATTN_DEBERTA)
    return fail(RELATTN_ERR_INVALID, "which=1 exists only for DeBERTa");
  IndexArgs a;
  std::memset(&a, 0, sizeof a);
  if (p->kind == RELATTN_T5) {
    T5Plan P;
    relattn_status s = t5_plan(p->num_buckets, p->max_distance, p->bidirectional, kBlockRows, &P);
    if (s != RELATTN_OK) return s;
    a.t5_slots = P.slots; a.t5_exact = P.exact; a.t5_bidir = p->bidirectional ? 1 : 0;
    a.t5_nthr = P.nthr;
    for (int m = 0; m < kT5MaxThr; ++m) a.t5_thr[m] = m < P.nthr ? P.thr[m] : INT32_MAX;
  } else if (p->kind == RELATTN_SHAW || p->kind == RELATTN_DEBERTA) {
    if (p->clip_k < 1) return fail(RELATTN_ERR_INVALID, "clip_k=%d must be >= 1", p->clip_k);
  }
  if (n == 0) return ok();
  if (!q_pos || !k_pos || !idx_out) return fail(RELATTN_ERR_INVALID, "NULL position or output pointer");
  a.q_pos = q_pos; a.k_pos = k_pos; a.out = idx_out; a.n = n;
  a.kind = p->kind; a.which = which; a.clip_k = p->clip_k;
  hipError_t e = launch_index(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RELATTN_ERR_HIP, "index launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
