"""Oracle against library routines, the skew trick, brute force and invariants.

  [RPE]  "Relative Position Embeddings, in depth" (aicassindra.com)
  [T5B]  "T5 Relative-Position Bias" (liminalml.com)
  [DRPE] "DeBERTa > Relative Position Encoding" (mbrenndoerfer.com)
"""

import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from tests import long_cache

ATOL = 1e-10


def _sdpa(q, k, v, mask=None, scale=None):
    """torch's reference attention on the CPU in float64 (math path)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q)[None, None], t(k)[None, None], t(v)[None, None],
        attn_mask=None if mask is None else t(mask)[None, None], scale=scale)
    return out[0, 0].numpy()


def _rand(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


def _mask_add(Lq, Lk, q_off=0, causal=False, n_valid=None):
    m = np.zeros((Lq, Lk))
    qpos = q_off + np.arange(Lq)[:, None]
    kpos = np.arange(Lk)[None, :]
    if causal:
        m = np.where(kpos > qpos, -np.inf, m)
    if n_valid is not None:
        m = np.where(kpos >= n_valid, -np.inf, m)
    return m


# ---------------------------------------------------------------- reductions

@pytest.mark.parametrize("causal,n_valid,q_off", [(False, None, 0), (True, None, 0),
                                                  (False, 13, 0), (True, None, 40)])
def test_zero_tables_reduce_to_plain_attention(causal, n_valid, q_off):
    rng = np.random.default_rng(1)
    Lq, Lk, d = 17, 23 if not causal else 17 + q_off, 16
    q, k, v = _rand(rng, Lq, d), _rand(rng, Lk, d), _rand(rng, Lk, d)
    mask = _mask_add(Lq, Lk, q_off, causal, n_valid)
    want = _sdpa(q, k, v, mask, 1 / math.sqrt(d))
    want_deb = _sdpa(q, k, v, mask, 1 / math.sqrt(3 * d))   # [RPE] DeBERTa: sqrt(3d)
    common = dict(q_pos_offset=q_off, causal=causal, n_valid=n_valid)
    got = oracle.relattn_forward_head(q, k, v, "t5", 0, np.zeros((32, 1)), **common)
    np.testing.assert_allclose(got, want, atol=ATOL)
    z = np.zeros((9, d))
    got = oracle.relattn_forward_head(q, k, v, "shaw", 0, z, z, clip_k=4, **common)
    np.testing.assert_allclose(got, want, atol=ATOL)
    z = np.zeros((10, 1, d))
    got = oracle.relattn_forward_head(q, k, v, "deberta", 0, z, z, clip_k=5, **common)
    np.testing.assert_allclose(got, want_deb, atol=ATOL)
    got = oracle.relattn_forward_head(q, k, v, "alibi", 0, np.zeros(1), **common)
    np.testing.assert_allclose(got, want, atol=ATOL)


@pytest.mark.parametrize("bidir", [True, False])
def test_t5_equals_sdpa_with_dense_bias(bidir):
    # [RPE] "Kernels and the KV cache": a dense float mask carrying the bias
    # through the library's attention gives the same result.
    rng = np.random.default_rng(2)
    Lq, Lk, d, H, h = 40, 300, 32, 3, 2
    q, k, v = _rand(rng, Lq, d), _rand(rng, Lk, d), _rand(rng, Lk, d)
    table = _rand(rng, 32, H, s=0.5)
    q_off = 200
    idx = oracle.rel_index_matrices("t5", Lq, Lk, q_pos_offset=q_off, bidirectional=bidir)["idx"]
    mask = table[idx, h] + _mask_add(Lq, Lk, q_off, causal=not bidir)
    want = _sdpa(q, k, v, mask, 1 / math.sqrt(d))
    got = oracle.relattn_forward_head(q, k, v, "t5", h, table, bidirectional=bidir,
                                      q_pos_offset=q_off, causal=not bidir)
    np.testing.assert_allclose(got, want, atol=ATOL)


def test_t5_constant_table_is_invisible():
    # softmax shift invariance: one constant per head changes nothing.
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 20, 8), _rand(rng, 20, 8), _rand(rng, 20, 8)
    table = np.full((32, 2), 0.37)
    got = oracle.relattn_forward_head(q, k, v, "t5", 1, table)
    np.testing.assert_allclose(got, _sdpa(q, k, v, None, 1 / math.sqrt(8)), atol=ATOL)


@pytest.mark.parametrize("causal", [True, False])
def test_shaw_gather_equals_skew_path(causal):
    # [RPE] "The skewing trick": the causal relative logits from the
    # pad-reshape-slice trick equal the clipped gather; for the encoder the
    # trick runs a second time on the mirrored problem.
    rng = np.random.default_rng(4)
    L, d, kc = 12, 8, 3
    q, k, v = _rand(rng, L, d), _rand(rng, L, d), _rand(rng, L, d)
    a_k = _rand(rng, 2 * kc + 1, d, s=0.5)
    # E[r] embeds distance r - (L - 1)
    E = np.stack([a_k[min(max(r - (L - 1), -kc), kc) + kc] for r in range(L)])
    lower = oracle.skew(q @ E.T)
    # mirrored problem: reversed queries, E'[r] embeds distance (L - 1) - r
    Em = np.stack([a_k[min(max((L - 1) - r, -kc), kc) + kc] for r in range(L)])
    upper = oracle.skew(q[::-1] @ Em.T)[::-1, ::-1]
    rel = np.tril(lower) + np.triu(upper, 1)
    scale = 1 / math.sqrt(d)
    mask = rel * scale + _mask_add(L, L, causal=causal)
    want = _sdpa(q, k, v, mask, scale)
    zeros = np.zeros_like(a_k)
    got = oracle.relattn_forward_head(q, k, v, "shaw", 0, a_k, zeros, clip_k=kc, causal=causal)
    np.testing.assert_allclose(got, want, atol=ATOL)


def test_shaw_equal_key_rows_invisible_and_value_rows_shift():
    rng = np.random.default_rng(5)
    L, d, kc = 15, 8, 2
    q, k, v = _rand(rng, L, d), _rand(rng, L, d), _rand(rng, L, d)
    base = _sdpa(q, k, v, _mask_add(L, L, causal=True), 1 / math.sqrt(d))
    a_k = np.tile(_rand(rng, 1, d), (2 * kc + 1, 1))
    c = _rand(rng, 1, d)
    a_v = np.tile(c, (2 * kc + 1, 1))
    got = oracle.relattn_forward_head(q, k, v, "shaw", 0, a_k, a_v, clip_k=kc, causal=True)
    np.testing.assert_allclose(got, base + c, atol=ATOL)


def test_shaw_uniform_attention_closed_form():
    # Q = K = 0 gives uniform weights over visible keys, so the value-side
    # term is the average of a_V rows over the clipped offsets seen.
    rng = np.random.default_rng(6)
    L, d, kc = 11, 4, 3
    z = np.zeros((L, d))
    v = _rand(rng, L, d)
    a_k = _rand(rng, 2 * kc + 1, d)
    a_v = _rand(rng, 2 * kc + 1, d)
    got = oracle.relattn_forward_head(z, z, v, "shaw", 0, a_k, a_v, clip_k=kc, causal=True)
    for i in range(L):
        n = i + 1
        want = v[: i + 1].mean(0)
        counts = np.zeros(2 * kc + 1)
        for off in range(-i, 1):
            counts[max(off, -kc) + kc] += 1
        want = want + (counts / n) @ a_v
        np.testing.assert_allclose(got[i], want, atol=ATOL)


def test_masking_independence():
    # [T5B]: masking is checked on its own -- entries of masked keys must
    # not influence anything.
    rng = np.random.default_rng(7)
    Lq, Lk, d = 9, 30, 8
    q, k, v = _rand(rng, Lq, d), _rand(rng, Lk, d), _rand(rng, Lk, d)
    q_off, n_valid = 12, 19     # visible: keys <= 12 + i and < 19
    k2, v2 = k.copy(), v.copy()
    k2[19:] = 1e3 * _rand(rng, Lk - 19, d)
    v2[19:] = -7.0
    tabs = {"t5": (_rand(rng, 32, 1), None),
            "shaw": (_rand(rng, 7, d), _rand(rng, 7, d)),
            "deberta": (_rand(rng, 8, 1, d), _rand(rng, 8, 1, d))}
    for kind, (t1, t2) in tabs.items():
        kw = dict(clip_k=3 if kind == "shaw" else 4, q_pos_offset=q_off, causal=True,
                  n_valid=n_valid, bidirectional=False)
        a = oracle.relattn_forward_head(q, k, v, kind, 0, t1, t2, **kw)
        b = oracle.relattn_forward_head(q, k2, v2, kind, 0, t1, t2, **kw)
        assert np.array_equal(a, b), kind
        # also: future keys (positions > query) under causal
        k3, v3 = k.copy(), v.copy()
        k3[q_off + Lq:] = 55.0
        v3[q_off + Lq:] = 55.0
        c = oracle.relattn_forward_head(q, k3, v3, kind, 0, t1, t2, **kw)
        assert np.array_equal(a, c), kind


def test_fully_masked_rows_are_zero():
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 4, 8), _rand(rng, 6, 8), _rand(rng, 6, 8)
    got = oracle.relattn_forward_head(q, k, v, "t5", 0, _rand(rng, 32, 1), n_valid=0)
    assert np.array_equal(got, np.zeros_like(got))


def test_position_shift_leaves_output_unchanged():
    # [RPE] "Choosing a scheme": shifting the input by a constant leaves the
    # attention pattern unchanged.
    rng = np.random.default_rng(9)
    q, k, v = _rand(rng, 10, 8), _rand(rng, 14, 8), _rand(rng, 14, 8)
    cases = {"t5": (_rand(rng, 32, 1), None, {}),
             "alibi": (_rand(rng, 1), None, {}),
             "shaw": (_rand(rng, 9, 8), _rand(rng, 9, 8), dict(clip_k=4)),
             "deberta": (_rand(rng, 10, 1, 8), _rand(rng, 10, 1, 8), dict(clip_k=5))}
    for kind, (t1, t2, kw) in cases.items():
        a = oracle.relattn_forward_head(q, k, v, kind, 0, t1, t2, q_pos_offset=3, **kw)
        b = oracle.relattn_forward_head(q, k, v, kind, 0, t1, t2, q_pos_offset=903,
                                        k_pos_offset=900, **kw)
        np.testing.assert_allclose(a, b, atol=1e-12)


def test_rows_selection_matches_full():
    rng = np.random.default_rng(10)
    q, k, v = _rand(rng, 2, 3, 21, 8), _rand(rng, 2, 3, 21, 8), _rand(rng, 2, 3, 21, 8)
    kr, qr = _rand(rng, 8, 3, 8), _rand(rng, 8, 3, 8)
    full = oracle.relattn_forward(q, k, v, "deberta", kr, qr, clip_k=4, causal=True)
    part = oracle.relattn_forward(q, k, v, "deberta", kr, qr, clip_k=4, causal=True,
                                  heads=[(1, 2), (0, 1)], rows=[0, 5, 20])
    np.testing.assert_allclose(part[0], full[1, 2, [0, 5, 20]], atol=1e-13)
    np.testing.assert_allclose(part[1], full[0, 1, [0, 5, 20]], atol=1e-13)


@pytest.mark.parametrize("kind", ["t5", "shaw", "deberta", "alibi", "txl"])
def test_batched_valid_lengths_equal_truncated_keys(kind):
    """The batched forward's per-sequence lengths ([T5B]: the padding mask
    hides key index j >= n_b of sequence b) against the same computation on
    each sequence's keys cut to its length, with no mask at all.  B != H and
    every length differs, so taking the length of the wrong sequence (or a
    head's index for a sequence's) changes the result."""
    rng = np.random.default_rng(31)
    B, H, Lq, Lk, d, clip = 3, 2, 9, 14, 8, 3
    q, k, v = _rand(rng, B, H, Lq, d), _rand(rng, B, H, Lk, d), _rand(rng, B, H, Lk, d)
    causal, q_off = (True, 10) if kind == "txl" else (False, 4)
    if kind == "t5":
        t1, t2 = _rand(rng, 32, H), None
    elif kind == "alibi":
        t1, t2 = _rand(rng, H, s=0.3), None
    elif kind == "txl":
        t1, t2 = _rand(rng, q_off + Lq, H, d), _rand(rng, 2, H, d)
    elif kind == "shaw":
        t1, t2 = _rand(rng, 2 * clip + 1, d), _rand(rng, 2 * clip + 1, d)
    else:
        t1, t2 = _rand(rng, 2 * clip, H, d), _rand(rng, 2 * clip, H, d)
    lens = np.array([5, 14, 1])
    kw = dict(clip_k=clip, q_pos_offset=q_off, causal=causal)
    got, lse = oracle.relattn_forward(q, k, v, kind, t1, t2, kv_valid_len=lens,
                                      return_lse=True, **kw)
    for b in range(B):
        n = int(lens[b])
        for h in range(H):
            want, wl = oracle.relattn_forward_head(q[b, h], k[b, h, :n], v[b, h, :n], kind, h,
                                                   t1, t2, return_lse=True, **kw)
            np.testing.assert_allclose(got[b, h], want, atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse[b, h], wl, atol=1e-12, rtol=0)
    # and the lengths do matter: the sequences differ from the unmasked run
    full = oracle.relattn_forward(q, k, v, kind, t1, t2, **kw)
    assert np.abs(full[0] - got[0]).max() > 1e-3 and np.abs(full[2] - got[2]).max() > 1e-3
    np.testing.assert_allclose(full[1], got[1], atol=1e-12, rtol=0)


# -------------------------------------------------------------- brute force

@settings(max_examples=60, deadline=None)
@given(kind=st.sampled_from(["t5", "shaw", "deberta", "alibi", "txl"]),
       Lq=st.integers(1, 9), Lk=st.integers(1, 12), d=st.sampled_from([2, 4, 8]),
       q_off=st.integers(0, 40), k_off=st.integers(0, 40), causal=st.booleans(),
       bidir=st.booleans(), nb=st.sampled_from([4, 8, 16, 32, 64]),
       md=st.sampled_from([8, 20, 128]), clip=st.integers(1, 6),
       n_valid=st.one_of(st.none(), st.integers(0, 12)), seed=st.integers(0, 10_000))
def test_vectorised_equals_bruteforce(kind, Lq, Lk, d, q_off, k_off, causal, bidir, nb,
                                      md, clip, n_valid, seed):
    slots = nb // 2 if bidir else nb
    if kind == "t5" and md <= slots // 2:
        md = slots
    rng = np.random.default_rng(seed)
    H, h = 2, seed % 2
    q, k, v = _rand(rng, Lq, d), _rand(rng, Lk, d), _rand(rng, Lk, d)
    if kind == "t5":
        t1, t2 = _rand(rng, nb, H), None
    elif kind == "alibi":
        t1, t2 = _rand(rng, H, s=0.3), None
    elif kind == "txl":
        causal = True
        rows = max(1, q_off + Lq - k_off)
        t1, t2 = _rand(rng, rows, H, d), _rand(rng, 2, H, d)
    elif kind == "shaw":
        t1, t2 = _rand(rng, 2 * clip + 1, d), _rand(rng, 2 * clip + 1, d)
    else:
        t1, t2 = _rand(rng, 2 * clip, H, d), _rand(rng, 2 * clip, H, d)
    kw = dict(num_buckets=nb, max_distance=md, bidirectional=bidir, clip_k=clip,
              q_pos_offset=q_off, k_pos_offset=k_off, causal=causal, n_valid=n_valid)
    a = oracle.relattn_forward_head(q, k, v, kind, h, t1, t2, **kw)
    b = oracle.relattn_forward_bruteforce(q, k, v, kind, h, t1, t2, **kw)
    np.testing.assert_allclose(a, b, atol=1e-11, rtol=0)


# -------------------------------------------------------------------- ALiBi

@pytest.mark.parametrize("causal", [False, True])
def test_alibi_is_t5_with_a_linear_table(causal):
    # [RPE] "ALiBi and RoPE": ALiBi is T5 without a learned table, a slope per
    # head times the distance.  Inside T5's exact range (distance < 8 at
    # bidirectional 32/128, < 16 causal) a T5 table whose exact slots hold
    # slope * distance gives the same logits, so the outputs agree.
    rng = np.random.default_rng(21)
    H, d = 3, 8
    L = 8                                        # every |offset| <= 7
    q, k, v = _rand(rng, L, d), _rand(rng, L, d), _rand(rng, L, d)
    slopes = np.array([-0.5, 0.25, -0.0625])
    table = np.zeros((32, H))
    bidir = not causal
    for dist in range(8):
        if bidir:
            table[dist] = slopes * dist           # keys at or before the query
            table[16 + dist] = slopes * dist      # keys after it
        else:
            table[dist] = slopes * dist           # causal: bucket = distance
    for h in range(H):
        a = oracle.relattn_forward_head(q, k, v, "alibi", h, slopes, causal=causal,
                                        q_pos_offset=4, k_pos_offset=4)
        b = oracle.relattn_forward_head(q, k, v, "t5", h, table, bidirectional=bidir,
                                        causal=causal, q_pos_offset=4, k_pos_offset=4)
        np.testing.assert_allclose(a, b, atol=1e-13)


def test_alibi_dense_bias_matches_sdpa():
    # the bias materialised as an L x L float mask, through torch's attention
    rng = np.random.default_rng(22)
    Lq, Lk, d = 11, 19, 8
    q, k, v = _rand(rng, Lq, d), _rand(rng, Lk, d), _rand(rng, Lk, d)
    slope = -0.37
    qpos = 30 + np.arange(Lq)[:, None]
    kpos = 25 + np.arange(Lk)[None, :]
    mask = slope * np.abs(kpos - qpos)
    want = _sdpa(q, k, v, mask, 1 / math.sqrt(d))
    got = oracle.relattn_forward_head(q, k, v, "alibi", 0, np.array([slope]),
                                      q_pos_offset=30, k_pos_offset=25)
    np.testing.assert_allclose(got, want, atol=1e-12)


def test_alibi_steep_penalty_reads_the_key_at_distance_zero():
    # a large negative slope leaves only the key at the query's own position
    rng = np.random.default_rng(23)
    L, d = 12, 8
    q, k, v = _rand(rng, L, d), _rand(rng, L, d), _rand(rng, L, d)
    got = oracle.relattn_forward_head(q, k, v, "alibi", 0, np.array([-200.0]))
    np.testing.assert_allclose(got, v, atol=1e-12)


# ------------------------------------------------------- row log-sum-exp

def test_lse_equals_torch_logsumexp():
    # zero tables: the logits are q.k * scale, so the row LSE is torch's
    # logsumexp over the visible keys
    rng = np.random.default_rng(24)
    Lq, Lk, d = 9, 15, 8
    q, k, v = _rand(rng, Lq, d), _rand(rng, Lk, d), _rand(rng, Lk, d)
    mask = _mask_add(Lq, Lk, 3, True, 12)
    logits = torch.from_numpy(q @ k.T / math.sqrt(d) + mask)
    want = torch.logsumexp(logits, dim=1).numpy()
    _, got = oracle.relattn_forward_head(q, k, v, "t5", 0, np.zeros((32, 1)), q_pos_offset=3,
                                         causal=True, n_valid=12, return_lse=True)
    np.testing.assert_allclose(got, want, atol=1e-12)
    _, none = oracle.relattn_forward_head(q, k, v, "t5", 0, np.zeros((32, 1)), n_valid=0,
                                          return_lse=True)
    assert np.all(np.isneginf(none))


@pytest.mark.parametrize("kind", ["t5", "shaw", "deberta", "alibi"])
def test_two_key_segments_merge_by_lse(kind):
    # keys split in two contiguous ranges, each placed by k_pos_offset: the
    # two partial results merge exactly by their row LSE ([RPE] "Kernels and
    # the KV cache": offset-only terms need no rewriting when a cache is cut)
    rng = np.random.default_rng(25)
    Lq, Lk, d, cut = 7, 20, 8, 9
    q, k, v = _rand(rng, Lq, d), _rand(rng, Lk, d), _rand(rng, Lk, d)
    t1, t2, kw = {"t5": (_rand(rng, 32, 1), None, {}),
                  "shaw": (_rand(rng, 9, d), _rand(rng, 9, d), dict(clip_k=4)),
                  "deberta": (_rand(rng, 10, 1, d), _rand(rng, 10, 1, d), dict(clip_k=5)),
                  "alibi": (np.array([-0.3]), None, {})}[kind]
    common = dict(q_pos_offset=13, causal=True, return_lse=True, **kw)
    full, lf = oracle.relattn_forward_head(q, k, v, kind, 0, t1, t2, **common)
    o1, l1 = oracle.relattn_forward_head(q, k[:cut], v[:cut], kind, 0, t1, t2, **common)
    o2, l2 = oracle.relattn_forward_head(q, k[cut:], v[cut:], kind, 0, t1, t2,
                                         k_pos_offset=cut, **common)
    m = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - m), np.exp(l2 - m)
    merged = (w1[:, None] * o1 + w2[:, None] * o2) / (w1 + w2)[:, None]
    np.testing.assert_allclose(merged, full, atol=1e-12)
    np.testing.assert_allclose(m + np.log(w1 + w2), lf, atol=1e-12)


# --------------------------------------------------------- Transformer-XL

def test_txl_position_terms_equal_the_skew():
    # [RPE] Transformer-XL: terms (b)+(d) are (q_i + v) against the projected
    # relative encodings "followed by the same skew".  With content keys at
    # zero only those terms remain; the page's pad / reshape / slice of
    # (Q + v) E_s^T, E_s[r] = the encoding of key - query = r - (L - 1), gives
    # the same causal logits as the oracle's gather by distance i - j.
    rng = np.random.default_rng(31)
    L, d, H, h = 9, 8, 2, 1
    q, v = _rand(rng, L, d), _rand(rng, L, d)
    k = np.zeros((L, d))
    enc = _rand(rng, L, H, d)                  # enc[r] encodes distance i - j = r
    uv = _rand(rng, 2, H, d)
    e_skew = enc[::-1, h, :]                   # row r <-> i - j = L - 1 - r
    s = oracle.skew((q + uv[1, h]) @ e_skew.T) / math.sqrt(d)
    mask = np.where(np.tril(np.ones((L, L))) > 0, s, -np.inf)
    want = _sdpa(q, k, v, mask, 1 / math.sqrt(d))
    got = oracle.relattn_forward_head(q, k, v, "txl", h, enc, uv, causal=True)
    np.testing.assert_allclose(got, want, atol=1e-12)


def test_txl_content_bias_is_a_per_key_term():
    # E = 0 and v = 0: only (q_i + u).k_j remains, i.e. plain attention plus
    # scale * u.k_j for every row, as a dense mask through torch's attention
    rng = np.random.default_rng(32)
    Lq, Lk, d, H = 7, 12, 8, 1
    q, k, v = _rand(rng, Lq, d), _rand(rng, Lk, d), _rand(rng, Lk, d)
    uv = np.zeros((2, H, d))
    uv[0, 0] = _rand(rng, d)
    kpos, qpos = np.arange(Lk)[None, :], 5 + np.arange(Lq)[:, None]
    mask = np.where(kpos <= qpos, np.broadcast_to((k @ uv[0, 0]) / math.sqrt(d), (Lq, Lk)), -np.inf)
    want = _sdpa(q, k, v, mask, 1 / math.sqrt(d))
    got = oracle.relattn_forward_head(q, k, v, "txl", 0, np.zeros((Lk + 5, H, d)), uv,
                                      q_pos_offset=5, causal=True)
    np.testing.assert_allclose(got, want, atol=1e-12)
    # and with u = 0 as well: plain causal attention
    got0 = oracle.relattn_forward_head(q, k, v, "txl", 0, np.zeros((Lk + 5, H, d)),
                                       np.zeros((2, H, d)), q_pos_offset=5, causal=True)
    want0 = _sdpa(q, k, v, np.where(kpos <= qpos, 0.0, -np.inf), 1 / math.sqrt(d))
    np.testing.assert_allclose(got0, want0, atol=1e-12)


def test_txl_shift_and_table_checks():
    rng = np.random.default_rng(33)
    q, k, v = _rand(rng, 6, 8), _rand(rng, 10, 8), _rand(rng, 10, 8)
    enc, uv = _rand(rng, 12, 1, 8), _rand(rng, 2, 1, 8)
    a = oracle.relattn_forward_head(q, k, v, "txl", 0, enc, uv, q_pos_offset=4, causal=True)
    b = oracle.relattn_forward_head(q, k, v, "txl", 0, enc, uv, q_pos_offset=504,
                                    k_pos_offset=500, causal=True)
    np.testing.assert_allclose(a, b, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.relattn_forward_head(q, k, v, "txl", 0, enc, uv, q_pos_offset=4)   # not causal
    with pytest.raises(ValueError):
        oracle.relattn_forward_head(q, k, v, "txl", 0, enc[:5], uv, q_pos_offset=4, causal=True)


# The long key-cache case of the GPU tests reduces each output row to sums of
# the softmax weights over (j >> 19, j mod 5) classes; that reduction against
# the full oracle, at a cache within one class group and one spanning two.
@pytest.mark.parametrize("Lk", [5000, 600000])
@pytest.mark.parametrize("kind", ["t5", "alibi"])
def test_long_cache_closed_form_equals_the_oracle(kind, Lk):
    tab = long_cache.table(kind)
    Lq = 2
    qpos0 = Lk - Lq
    rng = np.random.default_rng(9)
    q = rng.standard_normal((Lq, long_cache.D))
    k = np.zeros((Lk, long_cache.D))
    v = long_cache.values(np.arange(Lk))
    for h in range(2):
        want = oracle.relattn_forward_head(q, k, v, kind, h, tab, None, causal=True,
                                           q_pos_offset=qpos0, **long_cache.T5_PARAMS)
        for i in range(Lq):
            got = long_cache.expected(kind, tab, Lk, qpos0 + i, h)
            assert np.abs(got - want[i]).max() < 1e-12, (kind, Lk, h, i)
