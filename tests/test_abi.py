"""The C ABI library: loads without a GPU, exports every declared symbol, and
its host-only plan (validation, saturation radius, bucket copies) agrees with
the oracle's maps.  No compute call is made here."""

import copy
import os
import re

import numpy as np
import pytest

import oracle
import relative_position_attention_amd as rpa
from synth import CONFIGS, BENCH_SHAPES, make_problem, scaled_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "relpos.h")

needs_lib = pytest.mark.skipif(not os.path.exists(rpa.library_path()),
                               reason="librelpos.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(relpos_\w+)\s*\(", text)))


@needs_lib
def test_exports_every_declared_symbol():
    lib = rpa.library()
    names = declared_functions()
    assert len(names) >= 8
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(rpa.EXPORTED_SYMBOLS)


def _spec_small(idx, N):
    spec, _ = scaled_config(idx, B=1, H=2, N=N)
    return spec


@needs_lib
@pytest.mark.parametrize("idx,delta", [(1, 16), (2, 91), (3, 512)])
def test_saturation_radius(idx, delta):
    spec = make_problem(**dict(CONFIGS[idx], B=1, H=2))[0] if idx != 3 else \
        scaled_config(3, B=1, H=1, N=4096)[0]
    sz = rpa.Problem(spec).sizes()
    assert sz["delta"] == delta
    assert sz["expanded_rows"] == 2 * delta + 1


@needs_lib
@pytest.mark.parametrize("idx,N", [(4, 300), (5, 300)])
def test_identity_delta(idx, N):
    spec = _spec_small(idx, N)
    sz = rpa.Problem(spec).sizes()
    assert sz["delta"] == N - 1


@needs_lib
@pytest.mark.parametrize("idx,N", [(1, 128), (2, 2048), (2, 50), (3, 4096), (3, 300), (4, 257),
                                   (5, 129)])
def test_expanded_rows_match_oracle_maps(idx, N):
    # the host plan's bucket copies ([RPA] App. B.1): beta(s) = phi(s - D)
    spec = _spec_small(idx, N)
    prob = rpa.Problem(spec)
    D = prob.sizes()["delta"]
    s = np.arange(2 * D + 1)
    for which, term in enumerate(("aq", "ak", "bias")):
        if term not in spec["terms"]:
            continue
        got = np.array(rpa.plan_rows(prob, which))
        want = oracle.map_rows(spec["map"], spec["signs"][term] * (s - D))
        if spec["causal"]:
            want = np.where(s - D < 0, -1, want)
        assert np.array_equal(got, want), term


@needs_lib
def test_all_configs_plan():
    for idx in CONFIGS:
        spec = make_problem(**dict(CONFIGS[idx], B=1, H=1, N=64))[0]
        full = dict(spec, B=CONFIGS[idx]["B"], H=CONFIGS[idx]["H"], N=CONFIGS[idx]["N"])
        if spec["map"]["kind"] == "identity":
            N = full["N"]
            full["rows"] = N if spec["causal"] else 2 * N - 1
            full["map"] = dict(spec["map"], offset=0 if spec["causal"] else N - 1)
        sz = rpa.Problem(full).sizes()
        assert sz["z_bytes"] > 0 and sz["bwd_ws_bytes"] > sz["fwd_ws_bytes"]
    for name in BENCH_SHAPES:
        spec = dict(make_problem(**dict(BENCH_SHAPES[name], N=64))[0])
        assert rpa.Problem(spec).sizes()["z_bytes"] > 0


def _err(spec, **over):
    spec = copy.deepcopy(spec)
    prob = rpa.Problem(spec)
    for k, v in over.items():
        if k.startswith("map_"):
            setattr(prob.desc.map, k[4:], v)
        elif k in ("B", "H", "N", "d"):
            setattr(prob.shape, k, v)
        else:
            setattr(prob.desc, k, v)
    with pytest.raises(rpa.RelposError) as ei:
        rpa.plan_sizes(prob)
    return ei.value.code


@needs_lib
def test_validation_errors():
    spec = _spec_small(1, 128)
    assert _err(spec, d=32) == -2                      # head dim != 64: UNSUPPORTED
    assert _err(spec, abi_version=7) == -7             # ABI
    assert _err(spec, N=0) == -1                       # empty problems are refused
    assert _err(spec, B=0) == -1
    assert _err(spec, H=0) == -1
    assert _err(spec, N=(1 << 22) + 1) == -2          # longer than 2^22: UNSUPPORTED
    assert _err(spec, terms=1 << 7) == -1              # unknown term bit
    assert _err(spec, terms=16) == -1                  # V without AQ
    assert _err(spec, dtype=5) == -1
    assert _err(spec, sign_q=0) == -1
    assert _err(spec, num_rows=20) == -3               # clip 16 needs 33 rows: UNSUPPORTED_MAP
    assert _err(spec, aq_row_stride=66) == -4          # rows not 16-byte: MISALIGNED
    assert _err(spec, map_kind=9) == -1
    assert _err(spec, scale=float("inf")) == -1


@needs_lib
@pytest.mark.parametrize("rows", [[3, 2, 1, 0, 1, 2, 3], [2, 0, 3, 1, 0, 2, 3]],
                         ids=["symmetric", "scattered"])
def test_noncontiguous_map_plan(rows):
    # maps whose table rows are not one interval of offsets (delta and -delta
    # sharing a row, or rows scattered over the offsets; [RPA] "Atomic
    # fallback") are planned like any other: the expanded rows are the map
    # itself, beta(s) = phi(s - D)
    spec = copy.deepcopy(_spec_small(1, 64))
    c = 3
    spec["map"] = {"kind": "explicit", "clip": c, "rows": rows}
    spec["rows"] = 4
    prob = rpa.Problem(spec)
    D = prob.sizes()["delta"]
    s = np.arange(2 * D + 1)
    want = oracle.map_rows(spec["map"], spec["signs"]["aq"] * (s - D))
    assert rpa.plan_rows(prob, 0) == list(want)


@needs_lib
def test_explicit_contiguous_map_accepted():
    spec = copy.deepcopy(_spec_small(1, 64))
    c = 3
    spec["map"] = {"kind": "explicit", "clip": c, "rows": [0, 0, 1, 2, 3, 3, 4]}
    spec["rows"] = 5
    prob = rpa.Problem(spec)
    D = prob.sizes()["delta"]
    got = rpa.plan_rows(prob, 0)
    s = np.arange(2 * D + 1)
    want = oracle.map_rows(spec["map"], spec["signs"]["aq"] * (s - D))
    assert list(want) == got


@needs_lib
def test_strerror():
    assert rpa.strerror(0) == "success"
    assert rpa.strerror(-5) == "buffer too small"


@needs_lib
def test_stage_events_validation():
    # instrumentation hook: host-only validation, no GPU call
    import ctypes
    lib = rpa.library()
    assert lib.relpos_set_stage_events(None, 0) == 0
    arr = (ctypes.c_void_p * 9)()
    assert lib.relpos_set_stage_events(arr, 9) == -1
    assert lib.relpos_set_stage_events(None, 2) == -1
    assert lib.relpos_set_stage_events(arr, 0) == 0


def test_t5_descriptors_take_split_operands():
    # the T5 configuration (tau = 1, unit-variance inputs) meets the bf16
    # tolerances only with split operands; the parity harness and the bench
    # must build its descriptor that way, and the others with single operands
    import bench
    from gpu_util import split_operands_for
    spec2 = make_problem(**dict(CONFIGS[2], N=64))[0]
    assert "split_operands" not in spec2  # not an input-recipe property
    assert rpa.Problem(spec2, split_operands=split_operands_for(spec2)).desc.split_operands == 1
    for name in BENCH_SHAPES:
        spec = make_problem(**dict(BENCH_SHAPES[name], N=64))[0]
        want = 1 if name == "t5" else 0
        assert bench.bench_problem(rpa, name, spec, "f32").desc.split_operands == want, name
        assert int(split_operands_for(spec)) == want, name
    for idx in (1, 3, 4, 5):
        spec = make_problem(**dict(CONFIGS[idx], N=64))[0]
        assert not split_operands_for(spec), idx


@needs_lib
def test_in_tile_plan_is_linear_in_n():
    # [RPA] §6 / Table 7 "Projections": with in-tile products nothing
    # quadratic is stored.  Transformer-XL (identity map over 2N - 1 offsets):
    # the stored plan's projections and offset-gradient buffer grow as N^2,
    # the in-tile plan's buffers as N.
    sizes = {}
    for N in (2048, 4096, 8192):
        spec = _spec_small(5, N)
        st = rpa.Problem(spec).sizes()
        it = rpa.Problem(dict(spec, in_tile=True)).sizes()
        sizes[N] = (st, it)
        D = it["delta"]
        assert D >= N + 3 and D % 16 == 15          # every pair in the band, aligned windows
        assert it["expanded_rows"] == 2 * D + 1
    assert sizes[8192][0]["z_bytes"] / sizes[2048][0]["z_bytes"] > 14.0   # ~16x: quadratic
    for key in ("z_bytes", "bwd_ws_bytes", "bwd_ws_bytes_noz"):
        r_it = sizes[8192][1][key] / sizes[2048][1][key]
        assert r_it < 4.5, (key, r_it)               # ~4x: linear
        assert sizes[8192][1][key] < sizes[8192][0][key] / 10, key


@needs_lib
def test_in_tile_plan_past_the_slice_limit():
    # non-causal Transformer-XL at N = 32768: a stored projection slice needs
    # more than 2^31 bytes (rejected); the in-tile plan has no such slice
    spec = _spec_small(5, 32768)
    with pytest.raises(rpa.RelposError) as ei:
        rpa.Problem(spec).sizes()
    assert ei.value.code == -2
    sz = rpa.Problem(dict(spec, in_tile=True)).sizes()
    assert sz["z_bytes"] < 64 * 2**20


@needs_lib
def test_in_tile_validation():
    txl = _spec_small(4, 300)
    assert _err(dict(txl, in_tile=True), in_tile=2) == -1          # not 0/1
    assert _err(dict(txl, in_tile=True), reserved0=1) == -1
    f32 = _spec_small(1, 128)                                       # fp32 Shaw
    assert _err(dict(f32, in_tile=True)) == -2
    t5 = _spec_small(2, 256)                                        # bias only: no projections
    assert _err(dict(t5, in_tile=True)) == -2
    deb = _spec_small(3, 300)                                       # A^K
    assert _err(dict(deb, in_tile=True)) == -2
    # masks and dropout compose with in-tile products, split operands with them do not
    rpa.Problem(dict(txl, in_tile=True, segments=[[(0, 300)]])).sizes()
    rpa.Problem(dict(txl, in_tile=True, dropout={"p8": 10, "seed": 1})).sizes()
    assert _err(dict(txl, in_tile=True, segments=[[(0, 300)]]), split_operands=1) == -2
