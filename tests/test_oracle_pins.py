"""Pins of the float64 oracle to what the pages and the mathematics fix.

Nothing here touches the HIP library.  Sources:
  [RPE]  "Relative Position Embeddings, in depth" (aicassindra.com)
  [T5B]  "T5 Relative-Position Bias" (liminalml.com)
  [DRPE] "DeBERTa > Relative Position Encoding" (mbrenndoerfer.com)
"""

import os

import numpy as np
import pytest

import oracle
from tests.closed_forms import t5_bucket_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_t5_rows():
    rows = []
    with open(os.path.join(GOLDEN, "t5_bucket_pages.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            mode, rng, bucket, nb, md = line.split()[:5]
            if ":" in rng:
                a, b = map(int, rng.split(":"))
            else:
                a = b = int(rng)
            rows.append((mode == "bi", a, b, bucket, int(nb), int(md), line))
    return rows


@pytest.mark.parametrize("row", _golden_t5_rows(), ids=lambda r: r[-1].split("[")[0].strip())
def test_t5_bucket_page_values(row):
    bidir, a, b, bucket, nb, md, _ = row
    for off in range(a, b + 1):
        got = oracle.t5_bucket(off, bidir, nb, md)
        if bucket == "*":          # exact range: bucket equals the distance
            want = abs(off) if bidir else -off
        elif bucket.startswith("+"):   # same as the mirrored left value plus a shift
            want = oracle.t5_bucket(-off, bidir, nb, md) + int(bucket[1:])
        else:
            want = int(bucket)
        assert got == want, (off, got, want)


def test_t5_bidirectional_bucket_16_never_selected():
    # [T5B]: with 32 buckets, bidirectional slot 16 is unreachable (offset
    # +0 belongs to the left half, and +1 maps to 17).
    got = oracle.t5_bucket_array(np.arange(-5000, 5001), True, 32, 128)
    assert 16 not in set(got.tolist())
    assert set(got.tolist()) == set(range(32)) - {16}


def test_t5_two_token_sign_test():
    # [RPE] "Failure modes": a two-token sequence distinguishes past and
    # future.  Query 0 vs key 1 is offset +1 -> 16 + 1; query 1 vs key 0 is
    # offset -1 -> 1.
    idx = oracle.rel_index_matrices("t5", 2, 2, bidirectional=True)["idx"]
    assert idx[0, 1] == 17 and idx[1, 0] == 1 and idx[0, 0] == 0 and idx[1, 1] == 0


@pytest.mark.parametrize("nb,md", [(8, 16), (16, 64), (32, 128), (32, 256), (64, 128),
                                   (64, 512), (128, 1024), (32, 4096), (30, 100)])
@pytest.mark.parametrize("bidir", [True, False])
def test_t5_bucket_equals_exact_integer_closed_form(nb, md, bidir):
    # The page's float64 log formula against an exact integer criterion
    # (no logarithm); they must agree on every offset used by the kernels.
    offs = np.arange(-8192, 8193)
    got = oracle.t5_bucket_array(offs, bidir, nb, md)
    want = np.array([t5_bucket_exact(int(o), bidir, nb, md) for o in offs])
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(int(offs[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_t5_monotone_and_saturating():
    for bidir in (True, False):
        left = [oracle.t5_bucket(-dd, bidir) for dd in range(0, 3000)]
        assert all(x <= y for x, y in zip(left, left[1:]))
        assert left[-1] == (15 if bidir else 31)


def test_t5_rejects_degenerate_parameters():
    with pytest.raises(ValueError):
        oracle.t5_bucket(-5, True, 2, 128)       # one slot per half, no exact range
    with pytest.raises(ValueError):
        oracle.t5_bucket(-5, True, 32, 8)        # max distance inside exact range


def test_t5_cached_absolute_positions_matrix():
    # [T5B] cached decoder: the query keeps its absolute position.
    idx = oracle.rel_index_matrices("t5", 1, 129, q_pos_offset=128,
                                    bidirectional=False)["idx"]
    assert idx[0, 124] == 4
    idx0 = oracle.rel_index_matrices("t5", 1, 129, q_pos_offset=0,
                                     bidirectional=False)["idx"]
    assert idx0[0, 124] == 0


def test_deberta_delta_boundaries():
    # [DRPE] "The Relative Position Formula": -k -> 0, 0 -> k, k-1 -> 2k-1,
    # clamped beyond; 2k rows in all ("Why 2k Embeddings?").
    for k in (1, 2, 5, 16, 512):
        assert oracle.deberta_delta(-k, k) == 0
        assert oracle.deberta_delta(0, k) == k
        assert oracle.deberta_delta(k - 1, k) == 2 * k - 1
        assert oracle.deberta_delta(-k - 7, k) == 0
        assert oracle.deberta_delta(k, k) == 2 * k - 1
        assert oracle.deberta_delta(10 * k, k) == 2 * k - 1
        vals = oracle.deberta_delta(np.arange(-3 * k, 3 * k), k)
        assert vals.min() == 0 and vals.max() == 2 * k - 1
        assert len(np.unique(vals)) == 2 * k


def test_deberta_printed_relative_matrix():
    want = np.loadtxt(os.path.join(GOLDEN, "deberta_relpos_L6.txt"), dtype=np.int64)
    k = 512
    idx = oracle.rel_index_matrices("deberta", 6, 6, clip_k=k)
    # before clipping and shifting: delta - k recovers i - j inside the clip
    assert np.array_equal(idx["idx"] - k, want)
    # antisymmetry of i - j: entry (i, j) is minus entry (j, i)
    assert np.array_equal(idx["idx2"] - k, -want)
    assert np.array_equal(want, -want.T)


def test_shaw_index_boundaries():
    # [RPE] Shaw: offset j - i clipped to [-k, k] -> 2k + 1 rows.
    for k in (1, 4, 16):
        assert oracle.shaw_index(-k, k) == 0
        assert oracle.shaw_index(0, k) == k
        assert oracle.shaw_index(k, k) == 2 * k
        assert oracle.shaw_index(-k - 100, k) == 0
        assert oracle.shaw_index(k + 100, k) == 2 * k
    idx = oracle.rel_index_matrices("shaw", 3, 3, clip_k=1)["idx"]
    # query 0 vs key 2 is offset +2 -> clipped to +1 -> row 2
    assert idx[0, 2] == 2 and idx[2, 0] == 0 and idx[1, 1] == 1


def test_index_shift_invariance():
    # [RPE] "Choosing a scheme": shifting every position by a constant must
    # leave the pattern unchanged -- here, every index.
    for kind, kw in (("t5", dict(bidirectional=True)), ("t5", dict(bidirectional=False)),
                     ("shaw", dict(clip_k=3)), ("deberta", dict(clip_k=4))):
        a = oracle.rel_index_matrices(kind, 9, 11, q_pos_offset=2, k_pos_offset=0, **kw)
        b = oracle.rel_index_matrices(kind, 9, 11, q_pos_offset=1002, k_pos_offset=1000, **kw)
        for key in a:
            assert np.array_equal(a[key], b[key])


def test_skew_identity_L6_d8():
    # [RPE] "The skewing trick": for j <= i the skewed product holds query i
    # against distance j - i, i.e. q_i . E[j - i + L - 1].
    rng = np.random.default_rng(0)
    L, d = 6, 8
    q, E = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    s = oracle.skew(q @ E.T)
    for i in range(L):
        for j in range(L):
            if j <= i:
                assert np.isclose(s[i, j], q[i] @ E[j - i + L - 1], rtol=0, atol=1e-12)
            elif j == i + 1:
                assert s[i, j] == 0.0                      # the padded zero column
            else:
                # above the diagonal: the next query row against a shifted distance
                assert np.isclose(s[i, j], q[i + 1] @ E[j - i - 2], rtol=0, atol=1e-12)
