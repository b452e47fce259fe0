/*
 * relattn.h -- C ABI of the fused relative-position attention forward for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (page title, then the passage):
 *   [RPE]  "Relative Position Embeddings, in depth: Shaw, Transformer-XL,
 *          T5 buckets and DeBERTa ..." (aicassindra.com)
 *   [T5B]  "T5 Relative-Position Bias" (liminalml.com)
 *   [DRPE] "DeBERTa > Relative Position Encoding" (mbrenndoerfer.com)
 *
 * One call computes, for every (batch b, head h, query row i):
 *
 *   out[b,h,i,:] = sum_j softmax_j(s_ij) * value_ij
 *
 * over the keys j that are visible to row i, where, with absolute query
 * position p_i = q_pos_offset + i and absolute key position
 * t_j = k_pos_offset + j,
 *
 *   T5      s_ij = scale * q_i.k_j + table[bucket(t_j - p_i), h]
 *           value_ij = v_j
 *           bucket(): [RPE] "T5: one scalar per head, looked up by bucket"
 *           and [T5B] (offset = key - query; bidirectional splits the
 *           buckets by direction; causal bucketing clamps forward offsets
 *           to distance 0).  The bias is added after scaling.
 *   SHAW    s_ij = scale * q_i.(k_j + a_K[r_ij]),  r_ij = clip(t_j - p_i, -k, k) + k
 *           value_ij = v_j + a_V[r_ij]
 *           [RPE] "Shaw et al.: learned vectors on keys and values".
 *   DEBERTA s_ij = scale * (q_i.k_j + q_i.Kr[d(p_i, t_j), h] + k_j.Qr[d(t_j, p_i), h])
 *           d(x, y) = clip(x - y, -k, k - 1) + k, value_ij = v_j
 *           [DRPE] "The Relative Position Formula" (clip-and-shift index,
 *           2k rows); [RPE] "DeBERTa: disentangled content and position"
 *           (content-to-position plus position-to-content, scale 1/sqrt(3d)).
 *   ALIBI   s_ij = scale * q_i.k_j + slope[h] * |t_j - p_i|,  value_ij = v_j
 *           [RPE] "ALiBi and RoPE: the two endpoints" (T5 with the table
 *           removed: a fixed slope per head times the distance, no maximum
 *           distance).  The slope carries its sign: a negative slope
 *           penalises distance.
 *   TXL     s_ij = scale * ((q_i + u_h).k_j + (q_i + v_h).E[p_i - t_j, h]),
 *           value_ij = v_j.  [RPE] "Transformer-XL: four terms and two global
 *           biases": content keys against the query plus the global content
 *           bias u, projected relative encodings E = W_KR R(i - j) against
 *           the query plus the global position bias v.  Causal only (the
 *           cached segment precedes the queries); E has one row per distance
 *           0 .. clip_k - 1 and must cover every visible distance.  The bias
 *           terms u.k_j (one per key) and v.E[r] (one per distance) are
 *           formed in float32 by a pre-pass over K and E and added to the
 *           score as constants; q.k_j and q.E[r] come from the inputs as
 *           given (nothing is rounded before a product).
 *
 * Offset conventions (documented because mixing them swaps past and future,
 * [RPE] "Failure modes"): T5 and Shaw index by key - query; DeBERTa's
 * d(i, j) takes query - key.
 *
 * Visibility: key j is hidden when causal != 0 and t_j > p_i, and when
 * kv_valid_len != NULL and j >= kv_valid_len[b] (a key index, not a
 * position).
 *
 * Key positions: every term depends on positions only through t_j - p_i,
 * so a cache whose oldest keys were dropped is described by k_pos_offset
 * alone, and nothing stored needs rewriting ([RPE] "Kernels and the KV
 * cache": offset-only biases survive eviction).  Lq = 1 with
 * q_pos_offset = the new token's position is one decode step ([T5B],
 * cached decoding).  Masking is independent of
 * bucketing ([T5B]): a forward offset that maps to bucket 0 is still hidden
 * under the causal mask.  A row with no visible key produces zeros.
 *
 * Neither the L x L bias nor any L x L x d tensor is written to memory: the
 * relative term is formed inside the tile loop ([RPE] "Kernels and the KV
 * cache: where the choice bites").
 *
 * Conventions for every entry point
 *   - Ownership: the caller owns all buffers.  The library allocates no
 *     device memory and keeps no state between calls; calls are re-entrant.
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t passed as
 *     void*, NULL = the null stream) and the call returns without waiting.
 *   - Validation: every argument is checked on the host before anything is
 *     enqueued; on failure nothing is launched and a status is returned.
 *     relattn_last_error() then describes the failure (thread-local).
 *   - Launch failures reported by the HIP runtime return RELATTN_ERR_HIP.
 */
#ifndef RELATTN_H
#define RELATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: relattn_params gained k_pos_offset and lse; kinds RELATTN_ALIBI, RELATTN_TXL */
#define RELATTN_ABI_VERSION 2

typedef enum {
    RELATTN_T5 = 0,
    RELATTN_SHAW = 1,
    RELATTN_DEBERTA = 2,
    RELATTN_ALIBI = 3,
    RELATTN_TXL = 4
} relattn_kind;

typedef enum {
    RELATTN_FP32 = 0,   /* float32 inputs, float32 arithmetic, float32 output   */
    RELATTN_BF16 = 1    /* bfloat16 inputs, float32 accumulation, bf16 output     */
} relattn_dtype;

typedef enum {
    RELATTN_OK = 0,
    RELATTN_ERR_INVALID = 1,      /* malformed argument (null pointer, bad size) */
    RELATTN_ERR_UNSUPPORTED = 2,  /* well-formed but outside what is built      */
    RELATTN_ERR_WORKSPACE = 3,    /* workspace missing or smaller than needed   */
    RELATTN_ERR_HIP = 4           /* the HIP runtime reported an error          */
} relattn_status;

/*
 * Problem description.  Tensor layouts (all row-major and contiguous):
 *   q, out : [B, H, Lq, d]      k, v : [B, H, Lk, d]      element type = dtype
 *   T5      table  : float32 [num_buckets, H]       table2 : unused (NULL)
 *   SHAW    table  : a_K [2*clip_k + 1, d] (dtype)  table2 : a_V, same shape;
 *           shared by all heads ([RPE] Shaw section)
 *   DEBERTA table  : Kr [2*clip_k, H, d] (dtype)    table2 : Qr, same shape
 *   ALIBI   table  : float32 slopes [H]             table2 : unused (NULL)
 *   TXL     table  : E [clip_k, H, d] (dtype)       table2 : [2, H, d] (dtype):
 *           row 0 = u, row 1 = v
 * Device pointers must be 16-byte aligned (ALiBi slopes: 4-byte).
 */
typedef struct {
    int32_t kind;            /* relattn_kind                                     */
    int32_t dtype;           /* relattn_dtype                                    */
    int32_t B, H, Lq, Lk, d; /* d in {32, 64}, and 128 for BF16                    */
    const void *table;       /* device pointer, see above                        */
    const void *table2;      /* device pointer, see above                        */
    int32_t num_buckets;     /* T5: total buckets (2..256)                       */
    int32_t max_distance;    /* T5: distance where log buckets end (> exact range) */
    int32_t bidirectional;   /* T5: nonzero = split buckets by direction         */
    int32_t clip_k;          /* SHAW (1..32) / DEBERTA (1..65536): clip k;
                                TXL: rows of the relative encodings E          */
    int32_t q_pos_offset;    /* absolute position of query row 0 (>= 0)
                                ([T5B], cached decoder)                         */
    int32_t k_pos_offset;    /* absolute position of key row 0 (>= 0)          */
    int32_t causal;          /* nonzero: hide keys after the query's position    */
    const int32_t *kv_valid_len; /* device int32 [B] or NULL: keys j >= len hidden */
    float scale;             /* 0 = default: 1/sqrt(d) (T5, SHAW, ALIBI), 1/sqrt(3d)
                                (DEBERTA)                                       */
    float *lse;              /* device float32 [B, H, Lq] or NULL: written with
                                log(sum over visible j of exp(s_ij)) (natural
                                log), -inf for a row with no visible key.  Two
                                calls over disjoint key ranges (k_pos_offset
                                places each) merge exactly: out = (e^lse1 out1 +
                                e^lse2 out2) / (e^lse1 + e^lse2)               */
} relattn_params;

/*
 * Fused forward.  q, k, v, out: device pointers as described above.
 * workspace: device buffer of at least relattn_workspace_bytes() bytes
 * (may be NULL when that size is 0); its contents on entry do not matter and
 * on return are unspecified.  Two calls that share a workspace must be
 * ordered on one stream.
 * Returns RELATTN_OK once all kernels are enqueued.
 */
relattn_status relattn_fwd(const relattn_params *p, const void *q, const void *k,
                           const void *v, void *out, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Fused forward that allocates nothing, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same computation, arguments (minus the
 * workspace) and errors as relattn_fwd.  The workspace is a fixed array of
 * RELATTN_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held
 * until the process ends; a problem whose relattn_workspace_bytes() exceeds
 * it returns RELATTN_ERR_WORKSPACE and launches nothing.  The array's device
 * address is looked up once per device, on the first call made with that
 * device current (the stream must belong to the current device).  Every
 * call on one GPU shares that GPU's array and it keeps the last call's
 * contents: calls that overlap in time on one GPU (other streams, other
 * threads) race and must be ordered by the caller.  No part of the array
 * needs to start at zero.  The call itself allocates nothing (no hipMalloc,
 * no allocating library routine).
 */
#define RELATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
relattn_status relattn_fwd_noalloc(const relattn_params *p, const void *q, const void *k,
                                   const void *v, void *out, void *stream);

/* Bytes of device workspace relattn_fwd needs for this problem: the split-KV
 * partial results of decode-like shapes; for DEBERTA in FP32 the per-key
 * position-to-content constants of clipped blocks (8 bytes per key and
 * head; in BF16 the kernel forms them itself); for TXL the per-distance
 * constants v.E[r] (8 bytes per encoding row and head) and, in FP32, the
 * per-key constants u.k_j (8 bytes per key and head). */
relattn_status relattn_workspace_bytes(const relattn_params *p, size_t *bytes);

/*
 * Relative index of n (query position, key position) pairs, computed by the
 * same device index functions the fused kernel uses:
 *   which = 0: T5 bucket(k_pos - q_pos) | SHAW clip(k_pos - q_pos, -k, k) + k |
 *              DEBERTA d(q_pos, k_pos) | ALIBI |k_pos - q_pos| |
 *              TXL q_pos - k_pos (the row of E)
 *   which = 1: DEBERTA d(k_pos, q_pos) (position-to-content index); other
 *              kinds reject it.
 * Only kind and the kind's index parameters of *p are read (shapes and
 * tables are ignored).  q_pos, k_pos: device int32 [n]; idx_out: device
 * int32 [n].  n may be 0 (nothing is launched).
 */
relattn_status relattn_rel_index(const relattn_params *p, const int32_t *q_pos,
                                 const int32_t *k_pos, int64_t n, int32_t which,
                                 int32_t *idx_out, void *stream);

/*
 * T5 bucket thresholds as the kernels use them (host computation, no GPU):
 * thr[m] for m = 0 .. slots - exact - 1 is the smallest distance whose
 * within-direction slot is >= exact + m, evaluated with the pages' float64
 * logarithm formula.  *count receives slots - exact; at most `cap` entries
 * are written.
 */
relattn_status relattn_t5_thresholds(int32_t num_buckets, int32_t max_distance,
                                     int32_t bidirectional, int32_t *thr,
                                     int32_t cap, int32_t *count);

const char *relattn_status_str(relattn_status s);
const char *relattn_last_error(void);
int32_t relattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RELATTN_H */
