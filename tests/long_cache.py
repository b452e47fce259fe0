"""The long key-cache case of the GPU tests, in closed form (tests only).

A decoder's last steps over a very long cache: K = 0, so the logit of key j
is the relative term alone (T5 bucket bias, ALiBi distance penalty), and
V[j, c] = (((j >> 19) + c) mod 13 + j mod 5) / 64, exact in bfloat16, which
changes from one key to the next and every 2^19 keys.  Each output row is
then sum_j w_j V[j] / sum_j w_j with w_j the softmax weights, which reduces
to sums of w over the (j >> 19, j mod 5) classes.  The weights come from the
oracle's own indices; beyond 4096 positions T5 uses the bucket the oracle
gives the farthest offset (one bucket serves every offset past max_distance).
"""

import numpy as np

import oracle

D = 64
T5_PARAMS = dict(num_buckets=32, max_distance=128, bidirectional=False)


def values(rows):
    """Rows `rows` of V of one head, [len(rows), 64] float64."""
    j = np.asarray(rows, dtype=np.int64)[:, None]
    c = np.arange(D, dtype=np.int64)[None, :]
    return ((((j >> 19) + c) % 13) + j % 5) / 64.0


def table(kind):
    """Two heads: head 0 puts nearly all weight on the last few keys, head 1
    spreads it over the whole cache."""
    if kind == "t5":
        b = np.arange(32, dtype=np.float64)
        h0 = np.where(b < 16, 20.0 - 0.5 * b, np.where(b < 31, 4.0 - 0.1 * (b - 16), 0.0))
        h1 = np.where(b < 16, 1.0 - 0.05 * b, np.where(b < 31, 0.5 - 0.02 * (b - 16), 0.0))
        return np.stack([h0, h1], axis=1).astype(np.float32)
    return np.array([-0.5, -2.0 ** -22], dtype=np.float32)


def expected(kind, tab, Lk, qpos, h):
    """Output row [64] (float64) of the query at absolute position qpos
    (keys at positions 0 .. Lk-1, causal)."""
    off = np.arange(Lk, dtype=np.int64) - qpos          # key - query
    vis = off <= 0
    if kind == "t5":
        reach = -4096
        near = off >= reach
        bucket = np.empty(Lk, dtype=np.int64)
        bucket[near] = oracle.t5_bucket_array(off[near], **T5_PARAMS)
        far = oracle.t5_bucket(int(off[0]), T5_PARAMS["bidirectional"], T5_PARAMS["num_buckets"],
                               T5_PARAMS["max_distance"])
        assert far == oracle.t5_bucket(reach - 1, T5_PARAMS["bidirectional"],
                                       T5_PARAMS["num_buckets"], T5_PARAMS["max_distance"])
        bucket[~near] = far
        logit = tab[bucket, h].astype(np.float64)
    else:
        logit = float(tab[h]) * np.abs(off).astype(np.float64)
    logit = np.where(vis, logit, -np.inf)
    w = np.exp(logit - logit[vis].max())
    j = np.arange(Lk, dtype=np.int64)
    ng = (Lk >> 19) + 1
    S = np.bincount((j >> 19) * 5 + j % 5, weights=w, minlength=5 * ng).reshape(ng, 5)
    g = np.arange(ng)[:, None, None]
    m = np.arange(5)[None, :, None]
    c = np.arange(D)[None, None, :]
    vals = (((g + c) % 13) + m) / 64.0                  # [group, residue, column]
    return (S[:, :, None] * vals).sum(axis=(0, 1)) / S.sum()
