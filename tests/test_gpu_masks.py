"""GPU parity of the segment masks (padding masks, packed variable-length
sequences) and of attention dropout ([RPA] appendix "Masks, packing, and
dropout") against the fp64 oracle, through the C ABI, at the bf16 and fp32
tolerances, for every mechanism, causal and not.  The layouts leave whole
128-token workgroups outside every segment (all-padding rows), segments
that start and end inside tiles, and segments shorter than a tile."""

import copy

import numpy as np
import pytest
import torch

import oracle
from synth import make_problem, scaled_config
from gpu_util import check, run_library

pytestmark = pytest.mark.gpu

N = 700
LAYOUTS = {
    # packed sequences in both rows, the second row ending in padding
    "packed": [[(0, 150), (150, 420), (420, 700)], [(0, 333), (333, 690)]],
    # padding masks: 300 and 700 valid tokens (row 0 leaves workgroups 3-5
    # with padding queries only)
    "padded": [[(0, 300)], [(0, 700)]],
    # short sequences and gaps of padding between them
    "gaps": [[(5, 40), (64, 65), (100, 260), (400, 641)], [(0, 17), (17, 600)]],
}


def _problem(kind, dtype, causal, seed, n=N):
    # (the Shaw table is drawn N(0, 0.25) here: with unit variance, the causal
    # recipe's largest dQ and table-gradient elements carry bf16 errors of
    # 2-3e-2 absolute at rel-L2 2e-3, masks and dropout or not)
    spec, arr = make_problem(kind=kind, B=2, H=2, N=n, dtype=dtype, seed=seed, causal=causal,
                             clip=40, d_model=128, table_std=0.5 if kind == "shaw" else 1.0)
    spec = copy.deepcopy(spec)
    if kind == "t5" and dtype == "f32":
        spec["scale"] = 0.125  # (see test_f32_several_groups)
    return spec, arr


def _case(label, spec, arr):
    print(f"[masks] {label}: B={spec['B']} H={spec['H']} N={spec['N']} dtype={spec['dtype']} "
          f"causal={spec['causal']} segments={spec.get('segments') is not None} "
          f"dropout={spec.get('dropout')}", flush=True)
    got = run_library(spec, arr)
    ref = oracle.forward_backward(spec, arr)
    check(spec, got, ref, label=label)
    return got, ref


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["shaw", "t5", "deberta", "txl"])
@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_segments_bf16(layout, kind, causal):
    spec, arr = _problem(kind, "bf16", causal, 41)
    spec["segments"] = LAYOUTS[layout]
    got, ref = _case(f"seg-{layout}-{kind}-bf16-c{int(causal)}", spec, arr)
    # padding queries: O = 0 and L = -inf exactly
    for b, segs in enumerate(spec["segments"]):
        pad = np.ones(N, bool)
        for s0, s1 in segs:
            pad[s0:s1] = False
        assert np.all(got["o"][b][:, pad] == 0)
        assert np.all(np.isneginf(got["lse"][b][:, pad]))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["shaw", "t5", "deberta", "txl"])
def test_segments_f32(kind, causal):
    spec, arr = _problem(kind, "f32", causal, 42)
    spec["segments"] = LAYOUTS["gaps"]
    _case(f"seg-gaps-{kind}-f32-c{int(causal)}", spec, arr)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["shaw", "t5", "deberta", "txl"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dropout(kind, dtype, causal):
    spec, arr = _problem(kind, dtype, causal, 43)
    spec["dropout"] = {"p8": 26, "seed": 0x5EED0000 + 7 * len(kind)}
    _case(f"drop-{kind}-{dtype}-c{int(causal)}", spec, arr)


@pytest.mark.parametrize("kind", ["shaw", "t5", "deberta", "txl"])
def test_segments_and_dropout(kind):
    spec, arr = _problem(kind, "bf16", False, 44)
    spec["segments"] = LAYOUTS["packed"]
    spec["dropout"] = {"p8": 77, "seed": 0x0123456789ABCDEF}
    _case(f"seg+drop-{kind}", spec, arr)


def test_dropout_seed_changes_mask_and_repeats_bits():
    spec, arr = _problem("shaw", "bf16", False, 45)
    spec["dropout"] = {"p8": 64, "seed": 99}
    a = run_library(spec, arr)
    b = run_library(spec, arr)
    c = run_library(dict(spec, dropout={"p8": 64, "seed": 100}), arr)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    assert not np.array_equal(a["o"], c["o"])


def test_packed_config3_recipe():
    # configuration 3's DeBERTa recipe at N = 4096 packed as three documents
    # (one batch row, two heads), every slice compared
    spec, arr = scaled_config(3, B=1, H=2, N=4096)
    spec = dict(spec, segments=[[(0, 1000), (1000, 3000), (3000, 4096)]])
    _case("cfg3-packed-4096", spec, arr)
