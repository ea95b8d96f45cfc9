"""GPU parity at the configurations' full sizes and at the 8K bench shapes,
in the launch configuration the bench times (bf16 outputs written in fp32 so
the comparison measures the kernels).  The fp64 oracle materialises N x N per
(batch, head), so it runs on sampled slices: every computed slice's O, dQ,
dK, dV are compared element by element, and the per-head table gradients of a
head whose every batch slice was computed are compared whole."""

import numpy as np
import pytest

import oracle
from synth import BENCH_SHAPES, make_config, make_problem
from gpu_util import GRAD_KEYS, TOL, errors, run_library

pytestmark = pytest.mark.gpu


def _head_cols(key, arr, h, spec):
    if key in ("dq", "dk", "dv", "o"):
        raise KeyError(key)
    if key == "daq" and spec["aq_shared"]:
        return arr
    if key in ("daq", "dak"):
        return arr[:, h]
    if key == "dbias":
        return arr[:, h]
    return arr[h]  # du, dv_bias: [H, d]


def _compare(spec, got, slices, table_heads, label):
    tol_abs, tol_rel = TOL[spec["dtype"]]
    heads = sorted({h for _, h in slices})
    batches = sorted({b for b, _ in slices})
    ref = oracle.forward_backward(spec, spec["_arrays"], heads=heads, batches=batches)
    bad = []
    for b, h in slices:
        for key in ("o", "dq", "dk", "dv"):
            ma, rl = errors(got[key][b, h], ref[key][b, h])
            line = f"{label} b{b}h{h} {key:7s} max_abs={ma:.3e} rel_l2={rl:.3e}"
            print(line, flush=True)
            if not (ma <= tol_abs and rl <= tol_rel):
                bad.append(line)
    for h in table_heads:
        for key in GRAD_KEYS[3:]:
            if key not in ref:
                continue
            ma, rl = errors(_head_cols(key, got[key], h, spec), _head_cols(key, ref[key], h, spec))
            line = f"{label} h{h} {key:7s} max_abs={ma:.3e} rel_l2={rl:.3e}"
            print(line, flush=True)
            if not (ma <= tol_abs and rl <= tol_rel):
                bad.append(line)
    assert not bad, "\n".join(bad)


def _problem(spec, arr):
    spec = dict(spec)
    spec["_arrays"] = arr
    return spec


@pytest.mark.parametrize("idx,slices,table_heads", [
    (2, [(0, 0), (1, 0), (2, 0), (3, 0), (3, 15)], [0]),   # T5 B4 H16 N2048
    (3, [(0, 0), (1, 0), (1, 11)], [0]),                   # DeBERTa B2 H12 N4096
    (4, [(0, 0), (0, 7)], [0, 7]),                         # TXL causal B1 H8 N8192
])
def test_config_full_size(idx, slices, table_heads):
    spec, arr = make_config(idx)
    print(f"[full] cfg{idx} B={spec['B']} H={spec['H']} N={spec['N']}", flush=True)
    got = run_library(spec, arr)
    _compare(_problem(spec, arr), got, slices, table_heads, f"cfg{idx}")


def test_config5_full_size():
    # Conformer-style TXL, N = 16384: one head (its table gradients are whole:
    # B = 1)
    spec, arr = make_config(5)
    print(f"[full] cfg5 B={spec['B']} H={spec['H']} N={spec['N']}", flush=True)
    got = run_library(spec, arr)
    _compare(_problem(spec, arr), got, [(0, 3)], [3], "cfg5")


@pytest.mark.parametrize("name", ["shaw", "t5", "deberta", "txl"])
def test_bench_shape(name):
    spec, arr = make_problem(**BENCH_SHAPES[name])
    print(f"[full] bench {name} B={spec['B']} H={spec['H']} N={spec['N']}", flush=True)
    got = run_library(spec, arr)
    if name == "txl":
        slices, heads = [(0, 5)], [5]
    elif name == "deberta":
        slices, heads = [(0, 2), (1, 2)], [2]
    else:
        slices, heads = [(1, 9)], []
    _compare(_problem(spec, arr), got, slices, heads, f"bench-{name}")


@pytest.mark.parametrize("name", ["shaw", "deberta", "txl"])
def test_bench_shape_bf16_outputs(name):
    # the descriptor's bf16 output mode (O, dQ, dK, dV stored in bf16, D
    # taken from the rounded O) at the bench's full size, against the oracle
    # at the bf16 tolerances
    spec, arr = make_problem(**BENCH_SHAPES[name])
    print(f"[full] bench {name} bf16 outputs B={spec['B']} H={spec['H']} N={spec['N']}", flush=True)
    got = run_library(spec, arr, out_dtype="bf16")
    slices, heads = {"deberta": ([(0, 2), (1, 2)], [2]), "txl": ([(0, 5)], [5])}.get(name, ([(1, 9)], []))
    _compare(_problem(spec, arr), got, slices, heads, f"bench-{name}-bf16out")


def test_bench_shaw_table_gradient():
    # the Shaw table is shared by all heads: its gradient sums every slice, so
    # it is checked whole on a one-slice problem of the bench's map and length
    kw = dict(BENCH_SHAPES["shaw"], B=1, H=1)
    spec, arr = make_problem(**kw)
    got = run_library(spec, arr)
    _compare(_problem(spec, arr), got, [(0, 0)], [0], "bench-shaw-1slice")


@pytest.mark.parametrize("idx,slices,table_heads", [
    (4, [(0, 0), (0, 7)], [0, 7]),                         # TXL causal B1 H8 N8192
    (5, [(0, 3)], [3]),                                    # TXL B1 H8 N16384
])
def test_config_full_size_in_tile(idx, slices, table_heads):
    # the same configurations with in-tile relation products ([RPA] §6,
    # Table 7 row "Projections"): no stored projections or offset gradients
    spec, arr = make_config(idx)
    spec = dict(spec, in_tile=True)
    print(f"[full] cfg{idx} in-tile B={spec['B']} H={spec['H']} N={spec['N']}", flush=True)
    got = run_library(spec, arr)
    _compare(_problem(spec, arr), got, slices, table_heads, f"cfg{idx}-in-tile")
