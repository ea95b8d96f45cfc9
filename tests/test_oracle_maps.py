"""Pins of the oracle's relation maps ([RPA] §3.2 map families, §5.1 mechanisms)."""

import math
import os

import numpy as np
import pytest

from oracle.maps import t5_bucket, log_bucket, map_rows, relation_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([int(t) for t in line.split()])
    return rows


def test_t5_golden_ranges():
    for lo, hi, bucket in _load("t5_buckets.txt"):
        x = np.arange(lo, hi + 1)
        assert np.all(t5_bucket(x) == bucket), (lo, hi, bucket)


def test_t5_integer_closed_form():
    # 8 ln(n/8)/ln 16 = log2(n^2) - 6, so the large-offset bucket is
    # 8 + floor(log2(n^2)) - 6 = 2 + bit_length(n^2) - 1, capped at 15.
    x = np.arange(-20000, 20001)
    got = t5_bucket(x)
    n = np.abs(x)
    want = np.empty_like(x)
    for idx, nv in enumerate(n.tolist()):
        if nv < 8:
            b = nv
        else:
            b = min(8 + (nv * nv).bit_length() - 1 - 6, 15)
        want[idx] = b + (16 if x[idx] > 0 else 0)
    assert np.array_equal(got, want)


def test_t5_structure():
    x = np.arange(-5000, 5001)
    b = t5_bucket(x)
    assert set(np.unique(b).tolist()) == set(range(32)) - {16}  # bucket 16 never used
    for r in range(32):
        xs = x[b == r]
        if xs.size:
            assert xs.max() - xs.min() + 1 == xs.size  # one contiguous interval
    # saturation: constant for |x| >= 91, not for 90
    assert np.all(b[x >= 91] == 31) and np.all(b[x <= -91] == 15)
    assert t5_bucket(np.array([90]))[0] == 30 and t5_bucket(np.array([-90]))[0] == 14


def test_t5_float_definition_agrees_off_ties():
    # The standard definition evaluated with floating logarithms agrees with
    # the exact evaluation wherever the argument of floor is not an integer.
    n = np.arange(8, 20000, dtype=np.float64)
    val = np.log(n / 8.0) / np.log(128.0 / 8.0) * 8.0
    off_tie = np.abs(val - np.round(val)) > 1e-9
    fl = np.minimum(8 + np.floor(val), 15).astype(np.int64)
    ex = t5_bucket(-n.astype(np.int64))
    assert np.array_equal(fl[off_tie], ex[off_tie])


def test_log_bucket_golden():
    for x, bucket, row in _load("deberta_buckets.txt"):
        assert log_bucket(np.array([x]))[0] == bucket, x
        assert map_rows({"kind": "log", "bucket_size": 256, "max_position": 512},
                        np.array([x]))[0] == row, x


def test_log_bucket_structure():
    x = np.arange(-20000, 20001)
    b = log_bucket(x)
    assert np.array_equal(b, -log_bucket(-x))  # odd
    small = np.abs(x) <= 128
    assert np.array_equal(b[small], x[small])
    assert np.all(np.diff(b) >= 0)  # nondecreasing
    rows = np.clip(b + 256, 0, 511)
    assert set(np.unique(rows).tolist()) == set(range(512))
    assert np.all(rows[x >= 506] == 511) and rows[x == 505][0] == 510
    assert np.all(rows[x <= -512] == 0) and rows[x == -511][0] == 1


def test_log_bucket_float_definition_agrees_off_ties():
    n = np.arange(129, 20000, dtype=np.float64)
    val = np.log(n / 128.0) / np.log(511.0 / 128.0) * 127.0
    off_tie = np.abs(val - np.round(val)) > 1e-9
    fl = (128 + np.ceil(val)).astype(np.int64)
    ex = log_bucket(n.astype(np.int64))
    assert np.array_equal(fl[off_tie], ex[off_tie])


def test_identity_and_clipped_maps():
    spec = {"N": 9, "map": {"kind": "identity", "offset": 8}, "signs": {"aq": 1}}
    rho = relation_rows(spec, "aq")
    i, j = np.meshgrid(np.arange(9), np.arange(9), indexing="ij")
    assert np.array_equal(rho, i - j + 8)  # [RPA] §3.2: r = delta + N - 1
    spec = {"N": 9, "map": {"kind": "clipped", "clip": 2}, "signs": {"aq": -1}}
    rho = relation_rows(spec, "aq")
    assert np.array_equal(rho, np.clip(j - i, -2, 2) + 2)
    # clipping at >= N - 1 is the identity map shifted by the clip
    spec = {"N": 9, "map": {"kind": "clipped", "clip": 8}, "signs": {"aq": 1}}
    assert np.array_equal(relation_rows(spec, "aq"), i - j + 8)


@pytest.mark.parametrize("x", [0, 3, -3, 100])
def test_explicit_map(x):
    mp = {"kind": "explicit", "clip": 2, "rows": [4, 3, 2, 1, 0]}
    want = [4, 3, 2, 1, 0][min(max(x, -2), 2) + 2]
    assert map_rows(mp, np.array([x]))[0] == want
