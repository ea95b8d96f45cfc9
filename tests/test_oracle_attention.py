"""Pins of the fp64 oracle's forward and backward.

Each check ties the oracle to something other than itself:
  * per-pair brute force (the eager gather reference style of [RPA] §5.1),
  * central finite differences of the forward for every input,
  * torch fp64 autograd of torch's own scaled_dot_product_attention where the
    relation terms vanish (a library routine), and of the forward otherwise,
  * closed forms (uniform attention, N = 1, causal first row),
  * invariants stated by the method: a constant bias changes nothing; the
    bias gradient sums to zero (rows of dS sum to zero, [RPA] App. B.1);
    the query-table gradient summed over rows is zero; Eq. (6) summed over
    queries equals the bias gradient ([RPA] App. B.1, table-gradient lemma).
"""

import copy
import math

import numpy as np
import pytest
import torch

import oracle
from synth import make_problem

GRAD_KEYS = ("dq", "dk", "dv", "daq", "dak", "dbias", "du", "dv_bias")
INPUT_OF = {"dq": "q", "dk": "k", "dv": "v", "daq": "aq", "dak": "ak", "dbias": "bias",
            "du": "u", "dv_bias": "v_bias"}

SMALL_MAPS = {
    # small-parameter versions of the bucketed maps, so tiny N reaches their
    # logarithmic and saturated regions
    "t5": {"kind": "t5", "num_buckets": 8, "max_distance": 12, "bidirectional": True},
    "deberta": {"kind": "log", "bucket_size": 8, "max_position": 16},
}


def tiny(kind, N, d=4, B=1, H=2, causal=False, seed=0, small_map=True, table_gain=None):
    spec, arr = make_problem(kind, B, H, N, "f32", seed, causal=causal, clip=3)
    spec = copy.deepcopy(spec)
    spec["d"] = d
    for key in ("q", "k", "v", "do", "aq", "ak", "u", "v_bias"):
        if key in arr:
            arr[key] = arr[key][..., :d].copy()
    gain = {"deberta": 30.0, "txl": 3.0}.get(kind, 1.0) if table_gain is None else table_gain
    for key in ("aq", "ak"):
        if key in arr:
            arr[key] = arr[key] * gain
    for key in ("u", "v_bias"):
        if key in arr:
            arr[key] = arr[key] * 25.0
    if small_map and kind in SMALL_MAPS:
        spec["map"] = dict(SMALL_MAPS[kind])
        if kind == "t5":
            spec["rows"] = 8
            arr["bias"] = arr["bias"][:8].copy()
        else:
            spec["rows"] = 16
            arr["aq"] = arr["aq"][:16].copy()
            arr["ak"] = arr["ak"][:16].copy()
    return spec, arr


CASES = [
    ("shaw", False), ("shaw", True), ("t5", False), ("t5", True),
    ("deberta", False), ("deberta", True), ("txl", False), ("txl", True),
]


@pytest.mark.parametrize("kind,causal", CASES)
def test_bruteforce_matches_vectorised(kind, causal):
    spec, arr = tiny(kind, N=11, d=3, B=2, H=2, causal=causal, seed=7)
    ref = oracle.brute_forward_backward(spec, arr)
    got = oracle.forward_backward(spec, arr)
    for key in ref:
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-10, atol=1e-12, err_msg=key)


def _loss(spec, arr):
    o, _ = oracle.forward(spec, arr)
    return float(np.sum(o * arr["do"]))


@pytest.mark.parametrize("kind,causal", CASES)
def test_finite_differences(kind, causal):
    spec, arr = tiny(kind, N=6, d=3, B=1, H=2, causal=causal, seed=11)
    grads = oracle.forward_backward(spec, arr)
    eps = 1e-5
    rng = np.random.default_rng(3)
    for gk in GRAD_KEYS:
        if gk not in grads:
            continue
        x = arr[INPUT_OF[gk]]
        flat_idx = np.arange(x.size)
        if x.size > 40:
            flat_idx = rng.choice(x.size, 40, replace=False)
        for fi in flat_idx:
            idx = np.unravel_index(fi, x.shape)
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(spec, arr)
            x[idx] = old - eps
            lm = _loss(spec, arr)
            x[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grads[gk][idx]) <= 1e-6 * max(1.0, abs(fd)), (gk, idx, fd, grads[gk][idx])


def _torch_forward(spec, arr, t):
    """Forward of the score formula in torch fp64, for autograd (N x N per slice)."""
    B, H, N = spec["B"], spec["H"], spec["N"]
    tau = spec["scale"]
    outs = []
    i = torch.arange(N)
    delta = (i[:, None] - i[None, :]).numpy()
    rows = {term: torch.from_numpy(oracle.map_rows(spec["map"], spec["signs"][term] * delta))
            for term in ("aq", "ak", "bias") if term in spec["terms"]}
    for b in range(B):
        for h in range(H):
            q, k, v = t["q"][b, h], t["k"][b, h], t["v"][b, h]
            qc = q + t["u"][h] if "u" in t else q
            s = qc @ k.T
            if "aq" in t:
                a = t["aq"] if spec["aq_shared"] else t["aq"][:, h]
                qp = q + t["v_bias"][h] if "v_bias" in t else q
                s = s + torch.einsum("id,ijd->ij", qp, a[rows["aq"]])
            if "ak" in t:
                s = s + torch.einsum("jd,ijd->ij", k, t["ak"][:, h][rows["ak"]])
            if "bias" in t:
                s = s + t["bias"][:, h][rows["bias"]]
            s = tau * s
            if spec["causal"]:
                s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), -math.inf)
            outs.append(torch.softmax(s, dim=-1) @ v)
    return torch.stack(outs).reshape(B, H, N, -1)


@pytest.mark.parametrize("kind,causal", CASES)
def test_torch_autograd_backward(kind, causal):
    # real map parameters; N spans the T5 saturation (91) and DeBERTa's log region (>128)
    spec, arr = tiny(kind, N=150, d=8, B=1, H=2, causal=causal, seed=5, small_map=False)
    names = [n for n in ("q", "k", "v", "aq", "ak", "bias", "u", "v_bias") if n in arr]
    t = {n: torch.tensor(arr[n], dtype=torch.float64, requires_grad=True) for n in names}
    o = _torch_forward(spec, arr, t)
    (o * torch.tensor(arr["do"])).sum().backward()
    got = oracle.forward_backward(spec, arr)
    np.testing.assert_allclose(got["o"], o.detach().numpy(), rtol=1e-10, atol=1e-12)
    for gk, name in INPUT_OF.items():
        if gk in got:
            np.testing.assert_allclose(got[gk], t[name].grad.numpy(), rtol=1e-9, atol=1e-10,
                                       err_msg=gk)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_relation_terms_reduce_to_sdpa(causal):
    # zero tables and biases reproduce plain softmax attention (library routine)
    for kind in ("shaw", "t5", "deberta", "txl"):
        spec, arr = tiny(kind, N=40, d=16, B=2, H=2, causal=causal, seed=9, small_map=False)
        for key in ("aq", "ak", "bias", "u", "v_bias"):
            if key in arr:
                arr[key] = np.zeros_like(arr[key])
        got = oracle.forward_backward(spec, arr)
        q, k, v = (torch.tensor(arr[n], requires_grad=True) for n in ("q", "k", "v"))
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal,
                                                             scale=spec["scale"])
        o.backward(torch.tensor(arr["do"]))
        np.testing.assert_allclose(got["o"], o.detach().numpy(), rtol=1e-10, atol=1e-12)
        for gk, t in (("dq", q), ("dk", k), ("dv", v)):
            np.testing.assert_allclose(got[gk], t.grad.numpy(), rtol=1e-9, atol=1e-11)


def test_uniform_attention_closed_form():
    for causal in (False, True):
        spec, arr = tiny("shaw", N=9, d=4, B=1, H=1, causal=causal, seed=2)
        arr["q"][:] = 0.0
        arr["k"][:] = 0.0
        arr["aq"][:] = 0.0
        o, lse = oracle.forward(spec, arr)
        v = arr["v"][0, 0]
        for i in range(9):
            cnt = i + 1 if causal else 9
            np.testing.assert_allclose(o[0, 0, i], v[:cnt].mean(axis=0), rtol=1e-13)
            assert abs(lse[0, 0, i] - math.log(cnt)) < 1e-13


def test_single_token():
    for kind in ("shaw", "t5", "deberta", "txl"):
        spec, arr = tiny(kind, N=1, d=4, B=1, H=2, seed=4)
        g = oracle.forward_backward(spec, arr)
        np.testing.assert_allclose(g["o"], arr["v"], rtol=1e-14)
        np.testing.assert_allclose(g["dv"], arr["do"], rtol=1e-14)
        for key in ("dq", "dk", "daq", "dak", "dbias", "du", "dv_bias"):
            if key in g:
                assert np.max(np.abs(g[key])) < 1e-14, key


def test_causal_first_row():
    spec, arr = tiny("txl", N=12, d=4, B=1, H=2, causal=True, seed=6)
    g = oracle.forward_backward(spec, arr)
    np.testing.assert_allclose(g["o"][:, :, 0], arr["v"][:, :, 0], rtol=1e-14)


def test_constant_bias_changes_nothing():
    spec, arr = tiny("t5", N=30, d=8, B=2, H=2, seed=8, small_map=False)
    base = oracle.forward_backward(spec, arr)
    arr2 = dict(arr)
    arr2["bias"] = arr["bias"] * 0.0 + np.array([[0.7, -1.3]])  # constant per head
    arr3 = dict(arr)
    arr3["bias"] = arr["bias"] * 0.0
    a = oracle.forward_backward(spec, arr2)
    b = oracle.forward_backward(spec, arr3)
    for key in ("o", "dq", "dk", "dv", "dbias"):
        np.testing.assert_allclose(a[key], b[key], rtol=1e-9, atol=1e-12, err_msg=key)
    # and adding a per-head constant to a non-constant bias changes nothing either
    arr4 = dict(arr)
    arr4["bias"] = arr["bias"] + np.array([[2.5, -0.25]])
    c = oracle.forward_backward(spec, arr4)
    for key in ("o", "dq", "dk", "dv", "dbias"):
        np.testing.assert_allclose(c[key], base[key], rtol=1e-9, atol=1e-12, err_msg=key)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_sum_invariants(causal):
    # rows of dS sum to zero ([RPA] App. B.1), hence sum_r db_r = 0 and
    # sum_r dA^Q_r = sum_i (q_i + v) sum_j G_ij = 0.
    spec, arr = tiny("t5", N=64, d=8, B=2, H=3, causal=causal, seed=12, small_map=False)
    g = oracle.forward_backward(spec, arr)
    assert np.max(np.abs(g["dbias"].sum(axis=0))) < 1e-12
    for kind in ("shaw", "deberta", "txl"):
        spec, arr = tiny(kind, N=64, d=8, B=2, H=3, causal=causal, seed=12, small_map=False)
        g = oracle.forward_backward(spec, arr)
        assert np.max(np.abs(g["daq"].sum(axis=0))) < 1e-11, kind


def test_dzq_row_sums_equal_bias_gradient():
    # [RPA] App. B.1, table-gradient lemma step 4: sum_i dZ^Q[i, r] = db_r.
    # With A^Q present and a bias on the same map, the bias gradient equals the
    # row sums of the query relation gradient (here: TXL's v term reads it).
    spec, arr = tiny("shaw", N=40, d=8, B=1, H=1, seed=14)
    spec = copy.deepcopy(spec)
    spec["terms"] = ["aq", "bias"]
    spec["signs"]["bias"] = spec["signs"]["aq"]
    arr = dict(arr)
    arr["bias"] = np.random.default_rng(1).standard_normal((spec["rows"], 1))
    g = oracle.forward_backward(spec, arr)
    # dA^Q of a constant query q' = q + e direction: use the identity
    # sum_i dZ^Q[i, r] * 1 = db_r by evaluating dA^Q against an all-ones query column
    arr2 = dict(arr)
    arr2["q"] = arr["q"].copy()
    spec2 = copy.deepcopy(spec)
    spec2["terms"] = ["aq", "bias", "v"]
    arr2["v_bias"] = np.zeros((1, spec["d"]))
    g2 = oracle.forward_backward(spec2, arr2)
    # dv = sum_r (sum_i dZ^Q[i,r]) a_r must equal sum_r db_r a_r
    a = arr["aq"]
    np.testing.assert_allclose(g2["dv_bias"][0], g["dbias"][:, 0] @ a, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_noncontiguous_map_bruteforce(causal):
    # a map giving delta and -delta the same row ([RPA] "Atomic fallback"
    # names such maps): the vectorised scatter by row equals the per-pair
    # brute force for every term
    from synth import make_mixed
    spec, arr = make_mixed(["aq", "ak", "bias", "u", "v"], 1, 2, 9, "f32", 5, causal=causal,
                           clip=3)
    spec = copy.deepcopy(spec)
    spec["map"] = {"kind": "explicit", "clip": 3, "rows": [3, 2, 1, 0, 1, 2, 3]}
    spec["rows"] = 4
    for key in ("aq", "ak", "bias"):
        arr[key] = arr[key][:4].copy()
    ref = oracle.brute_forward_backward(spec, arr)
    got = oracle.forward_backward(spec, arr)
    for key in ref:
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-10, atol=1e-12, err_msg=key)


@pytest.mark.parametrize("kind,causal", CASES)
def test_query_rows_match_bruteforce(kind, causal):
    # the row-sampled oracle (for sequences too long for N x N) against the
    # per-pair brute force: O, L and dQ of every row, in an order that is not
    # the rows' own
    spec, arr = tiny(kind, N=11, d=3, B=2, H=2, causal=causal, seed=9)
    ref = oracle.brute_forward_backward(spec, arr)
    rows = [10, 0, 5, 1, 9, 2, 8, 3, 7, 4, 6]
    for b in range(2):
        for h in range(2):
            o, lse, dq = oracle.query_rows(spec, arr, b, h, rows)
            np.testing.assert_allclose(o, ref["o"][b, h][rows], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(lse, ref["lse"][b, h][rows], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(dq, ref["dq"][b, h][rows], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("kind,causal", CASES)
def test_query_rows_match_slices_real_maps(kind, causal):
    # the same at the mechanisms' own maps and a length past their
    # saturation radii (Shaw clip 16, T5 91, DeBERTa's log region), against
    # the full-slice oracle
    spec, arr = make_problem(kind, 1, 1, 300, "f32", 11, causal=causal, clip=16)
    full = oracle.slice_forward_backward(spec, arr, 0, 0)
    rows = [299, 0, 1, 150, 16, 17, 91, 92, 200, 298]
    o, lse, dq = oracle.query_rows(spec, arr, 0, 0, rows)
    np.testing.assert_allclose(o, full["o"][rows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, full["lse"][rows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dq, full["dq"][rows], rtol=1e-10, atol=1e-12)
