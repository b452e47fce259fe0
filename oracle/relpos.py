"""Float64 CPU oracle: relative-position attention forward, written from the pages.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg use it.

Sources (each function names the passage it follows):
  [RPE]   "Relative Position Embeddings, in depth: Shaw, Transformer-XL, T5
          buckets and DeBERTa ..." (aicassindra.com)
  [T5B]   "T5 Relative-Position Bias" (liminalml.com)
  [DRPE]  "DeBERTa > Relative Position Encoding" (mbrenndoerfer.com)

Everything is materialised on purpose (index matrices, bias / relative
logits, scores, probabilities), one (batch, head) at a time, in float64 from
the already-rounded inputs.  Library primitives used as single steps: matrix
products, ``take_along_axis`` gathers, ``np.add.at`` scatter-adds, ``exp``.

Readings taken where the pages leave a step open (also listed in the design
notes of the repository):
  * T5 logits are q.k * scale plus the bias; the bias itself is not scaled.
  * T5 table layout is [num_buckets, H].
  * Shaw: the page leaves the scaling implicit; the whole q.(k + a_K) is
    multiplied by scale.
  * DeBERTa: c2p = q_i . Kr[delta(i,j)], p2c = k_j . Qr[delta(j,i)], the sum
    of the three terms times 1/sqrt(3d), d = head dimension.
  * ALiBi ([RPE] "ALiBi and RoPE: the two endpoints": T5 without a learned
    table, a fixed slope per head times the distance): bias = slope[h] *
    |key position - query position|, added after scaling like T5's bias;
    the slope carries its sign (negative slopes penalise distance).
  * Transformer-XL ([RPE] "Transformer-XL: four terms and two global
    biases"): logit = scale * ((q_i + u).k_j + (q_i + v).E[i - j]) with E the
    projected relative encodings W_KR R(i - j) of one head, one row per
    distance i - j >= 0 (table [rows, H, d]), u and v the global content and
    position biases (table2 [2, H, d]); the whole sum is scaled by 1/sqrt(d)
    as for Shaw.  It is causal (the memory segment precedes the queries) and
    E must have a row for every visible distance.
  * Keys sit at absolute positions k_pos_offset + j; queries at
    q_pos_offset + i.  Padding masks key *index* j >= n_valid.
  * A row with no visible key has output 0.

Parity pins: every function here is pinned by tests under ``tests/``
(page-printed values, closed forms, library reductions, brute force).
The bf16 rounding of P inside the GPU kernel is not modelled here (this
oracle keeps float64 throughout); it is covered by the tolerance.
"""

from __future__ import annotations

import math

import numpy as np

KINDS = ("t5", "shaw", "deberta", "alibi", "txl")


# --------------------------------------------------------------------------
# Index functions
# --------------------------------------------------------------------------

def _t5_slots(num_buckets: int, max_distance: int, bidirectional: bool):
    """Slot count after the direction split and the exact-range size.

    [RPE] "T5: one scalar per head, looked up by bucket": bidirectional
    attention gives half of the buckets to keys after the query; inside a
    half (or the whole table, causal) the first half of the slots are exact
    distances.  Degenerate settings (no exact slot, or a maximum distance
    that does not exceed the exact range, which would make the log ratio
    undefined or negative) are rejected.
    """
    slots = num_buckets // 2 if bidirectional else num_buckets
    exact = slots // 2
    if exact < 1:
        raise ValueError("num_buckets too small: no exact-distance slot")
    if max_distance <= exact:
        raise ValueError("max_distance must exceed the exact range")
    return slots, exact


def t5_bucket(offset: int, bidirectional: bool = True, num_buckets: int = 32,
              max_distance: int = 128) -> int:
    """T5 bucket of one offset, offset = key position - query position.

    [RPE] "T5: one scalar per head, looked up by bucket" (the bucketing
    function and its worked example); [T5B] (the direction split, the
    causal clamp of forward offsets to distance 0, the saturation rule).
    Steps: split direction, take the distance, exact slot if small, else a
    log-spaced slot between the exact range and max_distance, saturating at
    the last slot.  Evaluated in float64 as on the pages.
    """
    slots, exact = _t5_slots(num_buckets, max_distance, bidirectional)
    offset = int(offset)
    if bidirectional:
        base = slots if offset > 0 else 0
        dist = -offset if offset < 0 else offset
    else:
        base = 0
        dist = -offset if offset < 0 else 0
    if dist < exact:
        return base + dist
    frac = math.log(dist / exact) / math.log(max_distance / exact)
    slot = exact + int(frac * (slots - exact))
    if slot > slots - 1:
        slot = slots - 1
    return base + slot


def t5_bucket_array(offsets, bidirectional: bool = True, num_buckets: int = 32,
                    max_distance: int = 128) -> np.ndarray:
    """``t5_bucket`` applied elementwise (once per distinct offset, scattered)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    uniq, inv = np.unique(offsets, return_inverse=True)
    vals = np.array([t5_bucket(int(o), bidirectional, num_buckets, max_distance)
                     for o in uniq], dtype=np.int64)
    return vals[inv].reshape(offsets.shape)


def shaw_index(offset, clip_k: int):
    """Shaw table row for offset = key - query.

    [RPE] "Shaw et al.: learned vectors on keys and values": the offset j - i
    is clipped to [-k, k], giving 2k + 1 rows; row = clipped offset + k.
    """
    if clip_k < 1:
        raise ValueError("clip_k must be >= 1")
    o = np.asarray(offset, dtype=np.int64)
    return np.minimum(np.maximum(o, -clip_k), clip_k) + clip_k


def deberta_delta(i_minus_j, k: int):
    """DeBERTa clip-and-shift index delta for a signed distance i - j.

    [DRPE] "The Relative Position Formula": three cases -- index 0 when
    i - j <= -k, index 2k - 1 when i - j >= k, otherwise i - j + k -- which
    gives 2k rows ("Why 2k Embeddings?").
    """
    if k < 1:
        raise ValueError("k must be >= 1")
    x = np.asarray(i_minus_j, dtype=np.int64)
    return np.where(x <= -k, 0, np.where(x >= k, 2 * k - 1, x + k)).astype(np.int64)


def skew(qe: np.ndarray) -> np.ndarray:
    """Music-Transformer skew of qe[..., i, r] (r embeds distance r - (L-1)).

    [RPE] "The skewing trick": prepend a zero column, reinterpret the
    [L, L+1] buffer as [L+1, L], drop the first row.  For j <= i the result
    holds query i against distance j - i; entries above the diagonal are
    not relative logits.
    """
    qe = np.asarray(qe)
    L = qe.shape[-2]
    if qe.shape[-1] != L:
        raise ValueError("skew expects a square [..., L, L] input")
    lead = qe.shape[:-2]
    padded = np.concatenate([np.zeros(lead + (L, 1), dtype=qe.dtype), qe], axis=-1)
    return padded.reshape(lead + (L + 1, L))[..., 1:, :]


def rel_index_matrices(kind: str, Lq: int, Lk: int, *, q_pos_offset: int = 0,
                       k_pos_offset: int = 0, num_buckets: int = 32,
                       max_distance: int = 128, bidirectional: bool = True,
                       clip_k: int = 0, rows=None):
    """Integer index matrices [n_rows, Lk] for one kind.

    Returns ``idx`` (T5 bucket / Shaw row / DeBERTa delta(i, j) / ALiBi
    distance |key - query|) and, for DeBERTa, ``idx2`` = delta(j, i) used by
    the position-to-content term.
    Offsets use absolute positions q_pos_offset + i and k_pos_offset + j;
    [T5B] (cached decoder paragraph) requires absolute query positions.
    """
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    qpos = q_pos_offset + rows
    kpos = k_pos_offset + np.arange(Lk)
    key_minus_query = kpos[None, :] - qpos[:, None]
    if kind == "t5":
        return {"idx": t5_bucket_array(key_minus_query, bidirectional,
                                       num_buckets, max_distance)}
    if kind == "shaw":
        return {"idx": shaw_index(key_minus_query, clip_k)}
    if kind == "deberta":
        return {"idx": deberta_delta(-key_minus_query, clip_k),
                "idx2": deberta_delta(key_minus_query, clip_k)}
    if kind == "alibi":
        return {"idx": np.abs(key_minus_query)}
    if kind == "txl":
        return {"idx": -key_minus_query}        # distance i - j, the row of E
    raise ValueError(f"unknown kind {kind!r}")


# --------------------------------------------------------------------------
# Attention forward
# --------------------------------------------------------------------------

def _default_scale(kind: str, d: int) -> float:
    # [RPE] DeBERTa section: three summed terms -> sqrt(3d); the others use
    # the ordinary 1/sqrt(d).
    return 1.0 / math.sqrt(3 * d) if kind == "deberta" else 1.0 / math.sqrt(d)


def relattn_forward_head(q, k, v, kind: str, h: int, table=None, table2=None, *,
                         num_buckets: int = 32, max_distance: int = 128,
                         bidirectional: bool = True, clip_k: int = 0,
                         q_pos_offset: int = 0, k_pos_offset: int = 0,
                         causal: bool = False, n_valid=None, scale=None,
                         rows=None, return_lse: bool = False):
    """Forward pass of one (batch, head): q [Lq, d], k/v [Lk, d] -> [n, d].

    Steps (float64, everything materialised):
      1. offsets key - query from absolute positions;
      2. index matrix ([RPE] T5 / Shaw sections, [DRPE] formula);
      3. relative term:
         T5      bias[i, j] = table[bucket, h]                  ([RPE] T5)
         Shaw    R[i, j] = (Q a_K^T)[i, row(i, j)]   ([RPE] Shaw, "workable
                 form": Q times the 2k+1 vectors, gathered by clipped offset)
         DeBERTa R[i, j] = (Q Kr_h^T)[i, delta(i,j)] + (K Qr_h^T)[j, delta(j,i)]
                                                ([RPE] DeBERTa; [DRPE])
         ALiBi   bias[i, j] = slope[h] * distance    ([RPE] ALiBi and RoPE)
         TXL     (q_i + u).k_j + (q_i + v).E[i - j]  ([RPE] Transformer-XL:
                 (a)+(c) against content keys, (b)+(d) against the projected
                 relative encodings)
      4. logits: T5 / ALiBi q.k*scale + bias; Shaw/DeBERTa (q.k + R)*scale;
      5. masks: causal hides keys after the query's position; padding hides
         key index j >= n_valid ([T5B]: masking is separate from bucketing);
      6. softmax over visible keys;
      7. output P V; Shaw adds sum_j p_ij a_V[row(i, j)] ([RPE] Shaw).
    ``rows`` selects query rows (all by default), for sampled comparisons.
    ``return_lse`` also returns each row's log of the sum over visible keys
    of exp(logit) (-inf for a row with no visible key).
    """
    if kind not in KINDS:
        raise ValueError(f"unknown kind {kind!r}")
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Lq, d = q.shape
    Lk = k.shape[0]
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    if scale is None or scale == 0:
        scale = _default_scale(kind, d)
    qr = q[rows]
    qpos = q_pos_offset + rows
    kpos = k_pos_offset + np.arange(Lk)
    idx = rel_index_matrices(kind, Lq, Lk, q_pos_offset=q_pos_offset,
                             k_pos_offset=k_pos_offset, num_buckets=num_buckets,
                             max_distance=max_distance, bidirectional=bidirectional,
                             clip_k=clip_k, rows=rows)
    content = qr @ k.T
    if kind == "t5":
        tab = np.asarray(table, dtype=np.float64)
        bias = tab[idx["idx"], h]
        logits = content * scale + bias
    elif kind == "alibi":
        slope = float(np.asarray(table, dtype=np.float64).reshape(-1)[h])
        logits = content * scale + slope * idx["idx"]
    elif kind == "txl":
        if not causal:
            raise ValueError("Transformer-XL attention is causal")
        enc = np.asarray(table, dtype=np.float64)[:, h, :]     # [rows, d]
        u, vb = np.asarray(table2, dtype=np.float64)[:, h, :]  # [d] each
        dist = idx["idx"]
        vis = dist >= 0
        if np.any(dist[vis] >= enc.shape[0]):
            raise ValueError("relative encoding table too short for the visible distances")
        terms_ac = (qr + u) @ k.T
        pos_all = (qr + vb) @ enc.T                            # [n, rows]
        terms_bd = np.take_along_axis(pos_all, np.clip(dist, 0, enc.shape[0] - 1), axis=1)
        logits = (terms_ac + terms_bd) * scale
    elif kind == "shaw":
        a_k = np.asarray(table, dtype=np.float64)
        rel_keys = qr @ a_k.T                       # [n, 2k+1]
        rel = np.take_along_axis(rel_keys, idx["idx"], axis=1)
        logits = (content + rel) * scale
    else:
        kr = np.asarray(table, dtype=np.float64)[:, h, :]   # [2k, d]
        qrel = np.asarray(table2, dtype=np.float64)[:, h, :]
        c2p_all = qr @ kr.T                         # [n, 2k]
        p2c_all = k @ qrel.T                        # [Lk, 2k]
        c2p = np.take_along_axis(c2p_all, idx["idx"], axis=1)
        p2c = p2c_all[np.arange(Lk)[None, :], idx["idx2"]]
        logits = (content + c2p + p2c) * scale

    visible = np.ones(logits.shape, dtype=bool)
    if causal:
        visible &= kpos[None, :] <= qpos[:, None]
    if n_valid is not None:
        visible &= (np.arange(Lk) < int(n_valid))[None, :]
    logits = np.where(visible, logits, -np.inf)

    any_visible = visible.any(axis=1)
    rowmax = np.where(any_visible, logits.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(visible, np.exp(logits - rowmax[:, None]), 0.0)
    denom = e.sum(axis=1)
    p = np.where(any_visible[:, None], e / np.where(any_visible, denom, 1.0)[:, None], 0.0)

    out = p @ v
    if kind == "shaw":
        a_v = np.asarray(table2, dtype=np.float64)
        mass = np.zeros((len(rows), a_v.shape[0]))
        np.add.at(mass, (np.arange(len(rows))[:, None].repeat(Lk, 1), idx["idx"]), p)
        out = out + mass @ a_v
    if return_lse:
        lse = np.where(any_visible, rowmax + np.log(np.where(any_visible, denom, 1.0)), -np.inf)
        return out, lse
    return out


def relattn_forward(q, k, v, kind: str, table=None, table2=None, *,
                    num_buckets: int = 32, max_distance: int = 128,
                    bidirectional: bool = True, clip_k: int = 0,
                    q_pos_offset: int = 0, k_pos_offset: int = 0,
                    causal: bool = False, kv_valid_len=None, scale=None,
                    heads=None, rows=None, return_lse: bool = False):
    """Batched forward: q [B, H, Lq, d], k/v [B, H, Lk, d] -> float64.

    ``heads`` (list of (b, h)) and ``rows`` restrict the work for sampled
    comparisons; the result then has shape [len(heads), len(rows), d].
    Otherwise the result is [B, H, Lq, d].  Tables: T5 [num_buckets, H];
    Shaw a_K, a_V [2k+1, d]; DeBERTa Kr, Qr [2k, H, d]; ALiBi slopes [H].
    ``return_lse`` also returns the row log-sum-exp ([B, H, Lq], or
    [len(heads), len(rows)]).
    """
    q = np.asarray(q)
    B, H, Lq, d = q.shape
    kw = dict(num_buckets=num_buckets, max_distance=max_distance,
              bidirectional=bidirectional, clip_k=clip_k,
              q_pos_offset=q_pos_offset, k_pos_offset=k_pos_offset,
              causal=causal, scale=scale, rows=rows, return_lse=True)
    lens = None if kv_valid_len is None else np.asarray(kv_valid_len).reshape(-1)
    n_rows = Lq if rows is None else len(rows)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    out = np.zeros((len(pairs), n_rows, d), dtype=np.float64)
    lse = np.zeros((len(pairs), n_rows), dtype=np.float64)
    for t, (b, h) in enumerate(pairs):
        nv = None if lens is None else int(lens[b])
        out[t], lse[t] = relattn_forward_head(q[b, h], k[b, h], v[b, h], kind, h,
                                              table, table2, n_valid=nv, **kw)
    if heads is None:
        out = out.reshape(B, H, n_rows, d)
        lse = lse.reshape(B, H, n_rows)
    return (out, lse) if return_lse else out


# --------------------------------------------------------------------------
# Brute-force twin (tiny sizes only)
# --------------------------------------------------------------------------

def relattn_forward_bruteforce(q, k, v, kind: str, h: int, table=None, table2=None,
                               *, num_buckets: int = 32, max_distance: int = 128,
                               bidirectional: bool = True, clip_k: int = 0,
                               q_pos_offset: int = 0, k_pos_offset: int = 0,
                               causal: bool = False, n_valid=None,
                               scale=None) -> np.ndarray:
    """Pair-by-pair loops with the naive materialised tensors, one head.

    [RPE] Shaw: the naive form builds an L x L x d tensor of a_K (and a_V)
    per pair; [DRPE] module: the position embeddings are looked up into an
    [Lq, Lk, d] tensor per pair.  Scalar ``t5_bucket`` per pair.  Plain
    Python loops and ``math.exp``; meant for L <= 16.
    """
    q = [list(map(float, row)) for row in np.asarray(q, dtype=np.float64)]
    k = [list(map(float, row)) for row in np.asarray(k, dtype=np.float64)]
    v = [list(map(float, row)) for row in np.asarray(v, dtype=np.float64)]
    Lq, Lk, d = len(q), len(k), len(q[0])
    if scale is None or scale == 0:
        scale = _default_scale(kind, d)

    def dot(a, b):
        s = 0.0
        for x, y in zip(a, b):
            s += x * y
        return s

    pair_key = pair_val = pair_kr = pair_qr = None
    if kind == "shaw":
        a_k = np.asarray(table, dtype=np.float64)
        a_v = np.asarray(table2, dtype=np.float64)
        pair_key = [[None] * Lk for _ in range(Lq)]
        pair_val = [[None] * Lk for _ in range(Lq)]
        for i in range(Lq):
            for j in range(Lk):
                off = (k_pos_offset + j) - (q_pos_offset + i)
                r = max(-clip_k, min(clip_k, off)) + clip_k
                pair_key[i][j] = list(map(float, a_k[r]))
                pair_val[i][j] = list(map(float, a_v[r]))
    elif kind == "deberta":
        kr = np.asarray(table, dtype=np.float64)[:, h, :]
        qrl = np.asarray(table2, dtype=np.float64)[:, h, :]
        pair_kr = [[None] * Lk for _ in range(Lq)]
        pair_qr = [[None] * Lk for _ in range(Lq)]
        for i in range(Lq):
            for j in range(Lk):
                dist = (q_pos_offset + i) - (k_pos_offset + j)
                pair_kr[i][j] = list(map(float, kr[int(deberta_delta(dist, clip_k))]))
                pair_qr[i][j] = list(map(float, qrl[int(deberta_delta(-dist, clip_k))]))

    out = np.zeros((Lq, d))
    for i in range(Lq):
        logits = []
        for j in range(Lk):
            pi, pj = q_pos_offset + i, k_pos_offset + j
            if causal and pj > pi:
                continue
            if n_valid is not None and j >= n_valid:
                continue
            if kind == "t5":
                b = t5_bucket(pj - pi, bidirectional, num_buckets, max_distance)
                s = dot(q[i], k[j]) * scale + float(np.asarray(table)[b, h])
            elif kind == "alibi":
                s = dot(q[i], k[j]) * scale + float(np.asarray(table).reshape(-1)[h]) * abs(pj - pi)
            elif kind == "txl":
                enc_row = list(map(float, np.asarray(table, dtype=np.float64)[pi - pj, h]))
                u = list(map(float, np.asarray(table2, dtype=np.float64)[0, h]))
                vb = list(map(float, np.asarray(table2, dtype=np.float64)[1, h]))
                s = (dot([a + b for a, b in zip(q[i], u)], k[j])
                     + dot([a + b for a, b in zip(q[i], vb)], enc_row)) * scale
            elif kind == "shaw":
                s = dot(q[i], [a + b for a, b in zip(k[j], pair_key[i][j])]) * scale
            else:
                s = (dot(q[i], k[j]) + dot(q[i], pair_kr[i][j])
                     + dot(k[j], pair_qr[i][j])) * scale
            logits.append((j, s))
        if not logits:
            continue
        mx = max(s for _, s in logits)
        weights = [(j, math.exp(s - mx)) for j, s in logits]
        z = sum(w for _, w in weights)
        for j, w in weights:
            p = w / z
            vec = v[j] if kind != "shaw" else [a + b for a, b in zip(v[j], pair_val[i][j])]
            for c in range(d):
                out[i, c] += p * vec[c]
    return out
