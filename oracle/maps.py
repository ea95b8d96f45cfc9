"""Relation maps phi(i, j) of [RPA] §3.2 ("Relative-Position Attention").

[RPA] lists three map families: identity (row = offset + N - 1), clipped
(row = clip(offset, -D, D) + D) and bucketed (offsets split into consecutive
ordered buckets).  [RPA] §5.1 "Mechanisms" names the two bucketed maps of the
evaluated mechanisms only by their origin (T5's 32 bidirectional buckets with
maximum distance 128; DeBERTa-v3's 256 logarithmic buckets with maximum
position 512) and prints no formula.  They are written here from their
standard definitions, evaluated EXACTLY with integer arithmetic (no floating
logarithm), so that no rounding decides a bucket boundary.

Parity unpinned against the pages for the two bucket formulas (the pages do
not print them); tests pin them by exact integer facts and structure.
"""

import functools

import numpy as np


@functools.lru_cache(maxsize=None)
def _t5_lut(maxn, num_buckets, max_distance, bidirectional):
    """Bucket (without the sign half) of every magnitude n in [0, maxn].

    For n >= max_exact the bucket is max_exact + k with k the largest integer
    satisfying  k <= span * log(n / max_exact) / log(max_distance / max_exact),
    evaluated exactly as  max_distance**k * max_exact**span
                          <= n**span * max_exact**k   (integers only).
    """
    nb = num_buckets // 2 if bidirectional else num_buckets
    max_exact = nb // 2
    span = nb - max_exact
    lut = np.zeros(maxn + 1, dtype=np.int64)
    k = 0
    for n in range(maxn + 1):
        if n < max_exact:
            lut[n] = n
            continue
        # k is nondecreasing in n: continue the search from the previous value
        while max_distance ** (k + 1) * max_exact ** span <= n ** span * max_exact ** (k + 1):
            k += 1
            if max_exact + k >= nb - 1:
                break
        lut[n] = min(max_exact + k, nb - 1)
    return lut


def t5_bucket(x, num_buckets=32, max_distance=128, bidirectional=True):
    """T5 relative-position bucket of signed offsets ``x`` (the T5 argument is
    memory position minus query position).  Returns an int64 array."""
    x = np.asarray(x, dtype=np.int64)
    if bidirectional:
        half = num_buckets // 2
        ret = (x > 0).astype(np.int64) * half
        n = np.abs(x)
    else:
        ret = np.zeros_like(x)
        n = -np.minimum(x, 0)
    maxn = int(n.max()) if n.size else 0
    lut = _t5_lut(maxn, num_buckets, max_distance, bool(bidirectional))
    return ret + lut[n]


@functools.lru_cache(maxsize=None)
def _log_lut(maxn, bucket_size, max_position):
    """DeBERTa bucket magnitude of every n in [0, maxn].

    n <= mid keeps n.  Otherwise mid + k with k the smallest integer satisfying
    k >= (mid - 1) * log(n / mid) / log((max_position - 1) / mid), evaluated
    exactly as  (max_position-1)**k * mid**(mid-1) >= n**(mid-1) * mid**k.
    """
    mid = bucket_size // 2
    top = max_position - 1
    lut = np.arange(maxn + 1, dtype=np.int64)
    k = 0
    c = mid ** (mid - 1)
    for n in range(mid + 1, maxn + 1):
        rhs = n ** (mid - 1)
        while top ** k * c < rhs * mid ** k:  # k is nondecreasing in n
            k += 1
        lut[n] = mid + k
    return lut


def log_bucket(x, bucket_size=256, max_position=512):
    """DeBERTa-v3 logarithmic bucket of signed offsets ``x`` (int64 array).

    Offsets with |x| <= bucket_size/2 keep their value; larger ones map to
    sign(x) * (mid + ceil((mid-1) * log(|x|/mid) / log((max_position-1)/mid))).
    """
    x = np.asarray(x, dtype=np.int64)
    a = np.abs(x)
    maxn = int(a.max()) if a.size else 0
    lut = _log_lut(maxn, int(bucket_size), int(max_position))
    return np.sign(x) * lut[a]


def map_rows(mp, x):
    """Relation row for signed map arguments ``x`` under map ``mp`` ([RPA] §3.2)."""
    x = np.asarray(x, dtype=np.int64)
    kind = mp["kind"]
    if kind == "identity":
        return x + int(mp["offset"])
    if kind == "clipped":
        c = int(mp["clip"])
        return np.clip(x, -c, c) + c
    if kind == "t5":
        return t5_bucket(x, mp["num_buckets"], mp["max_distance"], mp["bidirectional"])
    if kind == "log":
        bs = int(mp["bucket_size"])
        return np.clip(log_bucket(x, bs, mp["max_position"]) + bs, 0, 2 * bs - 1)
    if kind == "explicit":
        c = int(mp["clip"])
        rows = np.asarray(mp["rows"], dtype=np.int64)
        return rows[np.clip(x, -c, c) + c]
    raise ValueError(kind)


def relation_rows(spec, term, N=None):
    """N x N matrix rho[i, j] = phi(i, j) for table ``term`` in {"aq", "ak", "bias"}.

    The offset is delta = i - j ([RPA] §4.1 "Reachable Projection Ranges");
    each table reads its map at sign * delta (sign = -1 for maps written in
    j - i, as Shaw's, T5's and DeBERTa's position-to-content term are).
    """
    N = spec["N"] if N is None else N
    idx = np.arange(N, dtype=np.int64)
    delta = idx[:, None] - idx[None, :]
    return map_rows(spec["map"], spec["signs"][term] * delta)
