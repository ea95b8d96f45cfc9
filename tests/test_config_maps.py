"""Each input recipe's relation maps against the configuration text itself.

The recipes in ``synth`` carry the direction of every map in ``spec["signs"]``
and the oracle, the brute force and the library descriptor all read it there.
These tests write each configuration's map out in plain numpy from its own
wording -- Shaw indexes R by clamp(j - i, -16, 16) + 16; T5 buckets the
argument j - i; DeBERTa's content-to-position term reads Kr at the bucket of
i - j and the position-to-content term Qr at the bucket of j - i; the causal
Transformer-XL map is i - j, the Conformer one i - j + N - 1 -- and require
the oracle's relation rows and the library's expanded rows to equal them.  A
flipped sign in a recipe fails here.

The two bucket functions are taken from outside the oracle: T5 buckets from
the hand-derived ranges in ``golden/t5_buckets.txt``, DeBERTa buckets from
their floating-point definition (which agrees with exact evaluation for every
offset below 16384; see test_oracle_maps.py).  The mechanisms are those of
"Fast and Exact Relative-Position Attention via Structure-Aware Kernels"
(arXiv 2611.01182), §5.1 "Mechanisms".
"""

import math
import os

import numpy as np
import pytest

import oracle
import relative_position_attention_amd as rpa
from synth import BENCH_SHAPES, CONFIGS, make_problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

needs_lib = pytest.mark.skipif(not os.path.exists(rpa.library_path()),
                               reason="librelpos.so not built")


def _t5_from_golden(x):
    """T5 bucket of argument x (key index minus query index), from the
    hand-derived ranges."""
    x = np.asarray(x, dtype=np.int64)
    out = np.full(x.shape, -1, dtype=np.int64)
    with open(os.path.join(GOLDEN, "t5_buckets.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            lo, hi, b = (int(t) for t in line.split())
            out[(x >= lo) & (x <= hi)] = b
    assert np.all(out >= 0), "offset outside the golden ranges"
    return out


def _deberta_row(x):
    """clamp(bkt(x) + 256, 0, 511) with the DeBERTa-v3 log bucket (256
    buckets, maximum position 512) evaluated in floating point."""
    x = np.asarray(x, dtype=np.int64)
    a = np.abs(x).astype(np.float64)
    big = 128 + np.ceil(127.0 * np.log(np.maximum(a, 1.0) / 128.0) / np.log(511.0 / 128.0))
    bkt = np.where(a <= 128, x, np.sign(x) * big.astype(np.int64))
    return np.clip(bkt + 256, 0, 511)


def _ij(N):
    i = np.arange(N, dtype=np.int64)[:, None]
    j = np.arange(N, dtype=np.int64)[None, :]
    return i, j


def _text_maps(kind, spec):
    """Map of every table, written from the configuration text, as a function
    of (i, j); entries of masked pairs (causal, j > i) are not compared."""
    N = spec["N"]
    i, j = _ij(N)
    if kind == "shaw":
        c = spec["map"]["clip"]
        return {"aq": np.clip(j - i, -c, c) + c}
    if kind == "t5":
        return {"bias": _t5_from_golden(j - i)}
    if kind == "deberta":
        return {"aq": _deberta_row(i - j), "ak": _deberta_row(j - i)}
    if kind == "txl":
        return {"aq": (i - j) if spec["causal"] else (i - j + N - 1)}
    raise ValueError(kind)


# (recipe, kind, N used here): configurations 1-5 and the four 8K bench
# shapes at lengths past every saturation radius (T5 91, DeBERTa 512, Shaw 256)
CASES = [("cfg1", CONFIGS[1], 128), ("cfg2", CONFIGS[2], 300), ("cfg3", CONFIGS[3], 1100),
         ("cfg4", CONFIGS[4], 300), ("cfg5", CONFIGS[5], 300)] + \
        [(f"bench-{k}", BENCH_SHAPES[k], 700 if k != "deberta" else 1100) for k in BENCH_SHAPES]

# what each configuration states besides its maps: terms, table rows at the
# length used here, scale tau, shared table, causal mask
EXPECT = {
    "shaw": lambda N, c: (["aq"], 2 * c + 1, 1.0 / 8.0, True),
    "t5": lambda N, c: (["bias"], 32, 1.0, False),
    "deberta": lambda N, c: (["aq", "ak"], 512, 1.0 / math.sqrt(3 * 64), False),
    "txl": lambda N, c: (["aq", "u", "v"], None, 1.0 / 8.0, False),
}


def _recipe(kw, N):
    kw = dict(kw, B=1, H=2, N=N)
    return make_problem(**kw)[0]


@pytest.mark.parametrize("label,kw,N", CASES, ids=[c[0] for c in CASES])
def test_recipe_matches_configuration_text(label, kw, N):
    spec = _recipe(kw, N)
    kind = kw["kind"]
    terms, rows, tau, shared = EXPECT[kind](N, kw.get("clip", 16))
    assert sorted(spec["terms"]) == sorted(terms)
    if rows is None:  # Transformer-XL: N rows causal, 2N - 1 otherwise
        rows = N if spec["causal"] else 2 * N - 1
    assert spec["rows"] == rows
    assert math.isclose(spec["scale"], tau, rel_tol=1e-15)
    assert bool(spec["aq_shared"]) == shared
    assert spec["causal"] == bool(kw.get("causal", False))
    if label == "cfg1":
        assert kw["clip"] == 16 and spec["dtype"] == "f32"
    if label == "bench-shaw":
        assert kw["clip"] == 256
    visible = np.tril(np.ones((N, N), bool)) if spec["causal"] else np.ones((N, N), bool)
    for term, want in _text_maps(kind, spec).items():
        got = oracle.relation_rows(spec, term)
        assert np.array_equal(got[visible], want[visible]), (label, term)


@needs_lib
@pytest.mark.parametrize("label,kw,N", CASES, ids=[c[0] for c in CASES])
def test_library_rows_match_configuration_text(label, kw, N):
    # the descriptor the binding builds from the recipe: the host plan's
    # expanded rows beta(s), s = delta + D, must be the text's map at the
    # offset delta = i - j
    spec = _recipe(kw, N)
    prob = rpa.Problem(spec)
    D = prob.sizes()["delta"]
    maps = _text_maps(kw["kind"], spec)
    i, j = _ij(N)
    delta = i - j
    for which, term in enumerate(("aq", "ak", "bias")):
        if term not in maps:
            continue
        beta = np.array(rpa.plan_rows(prob, which))
        want = maps[term]
        vis = (delta >= 0) if spec["causal"] else np.ones_like(delta, bool)
        got = beta[np.clip(delta, -D, D) + D]
        assert np.array_equal(got[vis], want[vis]), (label, term)
