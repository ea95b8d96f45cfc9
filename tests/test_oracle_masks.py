"""Pins of the oracle's segment masks (padding and packed sequences) and of
its attention dropout ([RPA] appendix "Masks, packing, and dropout").

  * Philox4x32-10 against the generator's published known-answer vectors;
  * the dropout mask's kept fraction against its probability (binomial
    bound), and p = 0 changes nothing;
  * per-pair brute force with segments and dropout;
  * central finite differences with a fixed dropout mask and segments;
  * packed sequences equal the sequences run one by one, a padding mask
    equals the unpadded problem with zero rows appended;
  * averaged over seeds, dropout leaves O unbiased.
"""

import copy
import math
import os

import numpy as np
import pytest

import oracle
from oracle.philox import keep_mask, philox4x32
from synth import make_mixed, make_problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    n = 0
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            v = [int(t, 16) for t in line.split()]
            got = philox4x32(v[0], v[1], v[2], v[3], v[4], v[5])
            assert [int(x) for x in got] == v[6:10]
            n += 1
    assert n == 3


@pytest.mark.parametrize("p8", [0, 26, 128, 255])
def test_keep_fraction(p8):
    N = 512
    keep = keep_mask(N, 3, p8, 0x123456789ABCDEF)
    frac = keep.mean()
    want = 1.0 - p8 / 256.0
    sd = math.sqrt(want * (1 - want) / keep.size)
    assert abs(frac - want) <= 6 * sd + 1e-12, (frac, want)
    # each byte position of each word is used, and masks differ by slice
    assert not np.array_equal(keep, keep_mask(N, 4, p8, 0x123456789ABCDEF)) or p8 == 0


def _tiny_mixed(N, causal, seed=5, terms=("aq", "ak", "bias", "u", "v")):
    spec, arr = make_mixed(list(terms), 2, 2, N, "f32", seed, causal=causal, clip=3)
    spec = copy.deepcopy(spec)
    spec["d"] = 4
    for key in ("q", "k", "v", "do", "aq", "ak", "u", "v_bias"):
        if key in arr:
            arr[key] = arr[key][..., :4].copy() * (3.0 if key in ("aq", "ak") else 1.0)
    return spec, arr


SEGS = {"packed": [[(0, 4), (4, 9), (9, 11)], [(0, 7), (7, 11)]],
        "padded": [[(0, 8)], [(0, 11)]],
        "gaps": [[(1, 5), (6, 10)], [(0, 3), (5, 11)]]}


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("segs", sorted(SEGS) + [None])
@pytest.mark.parametrize("p8", [0, 77])
def test_bruteforce_masks_and_dropout(segs, p8, causal):
    spec, arr = _tiny_mixed(11, causal)
    spec["segments"] = None if segs is None else SEGS[segs]
    if p8:
        spec["dropout"] = {"p8": p8, "seed": 0xDEADBEEF12345}
    ref = oracle.brute_forward_backward(spec, arr)
    got = oracle.forward_backward(spec, arr)
    for key in ref:
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-10, atol=1e-12, err_msg=key)


def _loss(spec, arr):
    o, _ = oracle.forward(spec, arr)
    return float(np.sum(o * arr["do"]))


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences_masks_and_dropout(causal):
    spec, arr = _tiny_mixed(7, causal, seed=9)
    spec["segments"] = [[(0, 3), (3, 6)], [(1, 7)]]
    spec["dropout"] = {"p8": 64, "seed": 77}
    grads = oracle.forward_backward(spec, arr)
    inputs = {"dq": "q", "dk": "k", "dv": "v", "daq": "aq", "dak": "ak", "dbias": "bias",
              "du": "u", "dv_bias": "v_bias"}
    eps = 1e-6
    rng = np.random.default_rng(0)
    for gk, name in inputs.items():
        x = arr[name]
        for fi in rng.choice(x.size, min(x.size, 25), replace=False):
            idx = np.unravel_index(fi, x.shape)
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(spec, arr)
            x[idx] = old - eps
            lm = _loss(spec, arr)
            x[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grads[gk][idx]) <= 1e-6 * max(1.0, abs(fd)), (gk, idx, fd,
                                                                          grads[gk][idx])


@pytest.mark.parametrize("causal", [False, True])
def test_packed_equals_separate(causal):
    # two sequences packed into one row of B = 1 give each sequence's own
    # result: offsets inside a sequence are i - j either way
    lens = (9, 14)
    spec, arr = make_problem(kind="shaw", B=1, H=2, N=sum(lens), dtype="f32", seed=3,
                             causal=causal, clip=5, shared_table=False)
    spec = dict(spec, segments=[[(0, lens[0]), (lens[0], sum(lens))]])
    packed = oracle.forward_backward(spec, arr)
    daq = np.zeros_like(packed["daq"])
    start = 0
    for n in lens:
        sub = {k: (v[:, :, start:start + n].copy() if v.ndim == 4 else v) for k, v in arr.items()}
        one = oracle.forward_backward(dict(spec, N=n, segments=None), sub)
        for key in ("o", "dq", "dk", "dv"):
            np.testing.assert_allclose(packed[key][:, :, start:start + n], one[key], rtol=1e-12,
                                       atol=1e-13, err_msg=key)
        daq += one["daq"]
        start += n
    np.testing.assert_allclose(packed["daq"], daq, rtol=1e-12, atol=1e-13)


def test_padding_equals_unpadded():
    # a padding mask of length 10 in a row of 16: the first 10 tokens match the
    # unpadded problem; padded tokens have O = 0, L = -inf and no gradient
    spec, arr = make_problem(kind="t5", B=1, H=2, N=16, dtype="f32", seed=4)
    spec = dict(spec, scale=0.25, segments=[[(0, 10)]])
    full = oracle.forward_backward(spec, arr)
    sub = {k: (v[:, :, :10].copy() if v.ndim == 4 else v) for k, v in arr.items()}
    one = oracle.forward_backward(dict(spec, N=10, segments=None), sub)
    for key in ("o", "dq", "dk", "dv"):
        np.testing.assert_allclose(full[key][:, :, :10], one[key], rtol=1e-12, atol=1e-13)
        assert np.all(full[key][:, :, 10:] == 0), key
    assert np.all(np.isneginf(full["lse"][:, :, 10:]))
    np.testing.assert_allclose(full["dbias"], one["dbias"], rtol=1e-12, atol=1e-13)


def test_dropout_unbiased():
    # E[keep * scale] = 1: O averaged over seeds approaches the O of no dropout
    spec, arr = make_problem(kind="shaw", B=1, H=1, N=48, dtype="f32", seed=6, clip=5)
    base = oracle.forward(spec, arr)[0]
    acc = np.zeros_like(base)
    n = 300
    for s in range(n):
        acc += oracle.forward(dict(spec, dropout={"p8": 64, "seed": 1000 + s}), arr)[0]
    err = np.abs(acc / n - base).mean()
    spread = np.abs(oracle.forward(dict(spec, dropout={"p8": 64, "seed": 1}), arr)[0] - base).mean()
    assert err < 0.15 * spread, (err, spread)


def test_dropout_zero_probability_is_identity():
    spec, arr = _tiny_mixed(9, False)
    ref = oracle.forward_backward(spec, arr)
    got = oracle.forward_backward(dict(spec, dropout={"p8": 0, "seed": 5}), arr)
    for key in ref:
        np.testing.assert_array_equal(got[key], ref[key])
