"""The host plan (plan.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.

plan.cpp is plain C++ with no HIP call, so g++ builds it with the sanitizers
beside a small driver (plan_host_check.cpp) that plans every descriptor case
below: the five configurations and the four bench shapes at full size, scaled
and edge shapes, explicit and unidirectional maps, term combinations, the
validation errors and the per-slice size limit.  Every case must run clean,
and its return code and buffer sizes must equal what the built library's
relpos_plan_sizes reports for the same descriptor.  Also here: host-only
checks of the per-slice size limit ([RPA] §4.1 "Reachable Projection Ranges":
a query group of an identity map reaches N + G - 1 rows, so its slice grows
as N^2)."""

import copy
import ctypes
import os
import shutil
import struct
import subprocess

import pytest

import relative_position_attention_amd as rpa
from synth import BENCH_SHAPES, CONFIGS, make_mixed, make_problem, scaled_config

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "relative_position_attention_amd", "csrc")

needs_lib = pytest.mark.skipif(not os.path.exists(rpa.library_path()),
                               reason="librelpos.so not built")


def _full(kw):
    spec = make_problem(**dict(kw, B=1, H=1, N=64))[0]
    spec = dict(spec, B=kw["B"], H=kw["H"], N=kw["N"])
    if spec["map"]["kind"] == "identity":
        N = spec["N"]
        spec["rows"] = N if spec["causal"] else 2 * N - 1
        spec["map"] = dict(spec["map"], offset=0 if spec["causal"] else N - 1)
    return spec


def _txl(N, causal, dtype="bf16", terms=("aq", "u", "v")):
    spec = make_problem(kind="txl", B=1, H=8, N=64, dtype=dtype, seed=0, causal=causal,
                        d_model=128)[0]
    spec = dict(spec, N=N, rows=N if causal else 2 * N - 1, terms=list(terms),
                map={"kind": "identity", "offset": 0 if causal else N - 1})
    return spec


def _edit(prob, **over):
    for k, v in over.items():
        if k.startswith("map_"):
            setattr(prob.desc.map, k[4:], v)
        elif k in ("B", "H", "N", "d"):
            setattr(prob.shape, k, v)
        else:
            setattr(prob.desc, k, v)
    return prob


def cases():
    """(label, Problem) for every plan case."""
    out = []
    for idx, kw in CONFIGS.items():
        out.append((f"cfg{idx}", rpa.Problem(_full(kw))))
    for name, kw in BENCH_SHAPES.items():
        out.append((f"bench-{name}", rpa.Problem(_full(kw))))
    for idx, N in ((1, 1), (2, 2), (2, 300), (3, 1100), (4, 700), (5, 129), (3, 17)):
        out.append((f"cfg{idx}-N{N}", rpa.Problem(scaled_config(idx, B=1, H=2, N=N)[0])))
    for kind in ("shaw", "t5", "deberta", "txl"):
        for causal in (False, True):
            spec = make_problem(kind=kind, B=2, H=2, N=600, dtype="f32", seed=1, causal=causal,
                                clip=40, d_model=128)[0]
            out.append((f"{kind}-f32-c{int(causal)}", rpa.Problem(spec)))
    for terms in (["ak"], ["aq", "bias"], ["bias", "u"], ["aq", "ak", "bias", "u", "v"]):
        for causal in (False, True):
            spec = make_mixed(terms, 1, 2, 200, "f32", 1, causal=causal)[0]
            out.append(("+".join(terms) + f"-c{int(causal)}", rpa.Problem(spec)))
    base = make_problem(kind="shaw", B=1, H=2, N=300, dtype="bf16", seed=7, clip=8,
                        shared_table=False)[0]
    ex = copy.deepcopy(base)
    ex["map"] = {"kind": "explicit", "clip": 8,
                 "rows": [0, 0, 0, 1, 1, 2, 3, 4, 5, 6, 7, 8, 8, 9, 10, 10, 10]}
    ex["rows"] = 11
    out.append(("explicit", rpa.Problem(ex)))
    sym = copy.deepcopy(base)
    sym["map"] = {"kind": "explicit", "clip": 3, "rows": [3, 2, 1, 0, 1, 2, 3]}
    sym["rows"] = 4
    out.append(("explicit-symmetric", rpa.Problem(sym)))
    uni = copy.deepcopy(make_problem(kind="t5", B=1, H=2, N=300, dtype="bf16", seed=2,
                                     causal=True)[0])
    uni["map"]["bidirectional"] = False
    out.append(("t5-unidirectional", rpa.Problem(uni)))
    small = copy.deepcopy(make_problem(kind="deberta", B=1, H=2, N=300, dtype="bf16", seed=3)[0])
    small["map"] = {"kind": "log", "bucket_size": 32, "max_position": 128}
    small["rows"] = 64
    out.append(("deberta-b32", rpa.Problem(small)))
    # validation errors (each a copy of configuration 1's descriptor)
    c1 = scaled_config(1, B=1, H=2, N=128)[0]
    for label, over in (("d32", dict(d=32)), ("abi", dict(abi_version=7)), ("N0", dict(N=0)),
                        ("term-bit", dict(terms=1 << 7)), ("v-alone", dict(terms=16)),
                        ("dtype", dict(dtype=5)), ("sign", dict(sign_q=0)),
                        ("rows", dict(num_rows=20)), ("stride", dict(aq_row_stride=66)),
                        ("map-kind", dict(map_kind=9)), ("scale", dict(scale=float("inf"))),
                        ("N-max", dict(N=(1 << 22) + 1)), ("clip-neg", dict(map_clip=-1))):
        out.append((label, _edit(rpa.Problem(copy.deepcopy(c1)), **over)))
    # per-slice size limit: accepted just below, rejected above
    out.append(("txl-nc-32000", rpa.Problem(_txl(32000, False))))
    out.append(("txl-nc-32768", rpa.Problem(_txl(32768, False))))
    out.append(("txl-c-46000", rpa.Problem(_txl(46000, True))))
    out.append(("txl-c-47000", rpa.Problem(_txl(47000, True))))
    out.append(("id-bias-f32-24000", rpa.Problem(_txl(24000, False, "f32", ("aq", "bias")))))
    # in-tile products: the Transformer-XL configurations, a clipped map, N = 1,
    # past the stored path's slice limit, with masks and dropout, and refusals
    for label, spec in (("it-cfg4", _full(CONFIGS[4])), ("it-cfg5", _full(CONFIGS[5])),
                        ("it-shaw", scaled_config(1, B=2, H=2, N=700, dtype="bf16")[0]),
                        ("it-txl-N1", _txl(1, False)), ("it-txl-nc-32768", _txl(32768, False)),
                        ("it-txl-c-47000", _txl(47000, True)),
                        ("it-seg-drop", dict(_txl(700, True), segments=[[(0, 700)]],
                                             dropout={"p8": 9, "seed": 3})),
                        ("it-deberta", _full(CONFIGS[3])),
                        ("it-f32", scaled_config(1, B=1, H=2, N=128)[0])):
        out.append((label, rpa.Problem(dict(spec, in_tile=True))))
    out.append(("it-split-seg", _edit(rpa.Problem(dict(_txl(300, False), in_tile=True,
                                                       segments=[[(0, 300)]])),
                                      split_operands=1)))
    out.append(("it-flag-2", _edit(rpa.Problem(dict(_txl(300, False), in_tile=True)), in_tile=2)))
    return out


def _write_cases(path, items):
    with open(path, "wb") as fh:
        for _, prob in items:
            sh = prob.shape
            fh.write(struct.pack("<4i", sh.B, sh.H, sh.N, sh.d))
            fh.write(ctypes.string_at(ctypes.addressof(prob.desc), ctypes.sizeof(prob.desc)))
            rows = list(prob.spec["map"]["rows"]) if prob.spec["map"]["kind"] == "explicit" else []
            fh.write(struct.pack("<i", len(rows)))
            if rows:
                fh.write(struct.pack(f"<{len(rows)}i", *rows))


def _library_line(prob):
    try:
        s = rpa.plan_sizes(prob)
    except rpa.RelposError as e:
        return f"{e.code}"
    return (f"0 {s['delta']} {s['expanded_rows']} {s['z_bytes']} {s['fwd_ws_bytes']} "
            f"{s['bwd_ws_bytes']} {s['num_groups']}")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_plan_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_host_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "plan.cpp"), os.path.join(HERE, "plan_host_check.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    items = cases()
    path = str(tmp_path / "cases.bin")
    _write_cases(path, items)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe, path], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stderr[-4000:]
    assert "runtime error" not in res.stderr, res.stderr[-4000:]
    lines = res.stdout.strip().splitlines()
    assert len(lines) == len(items)
    codes = {label: int(line.split()[0]) for (label, _), line in zip(items, lines)}
    for label in ("d32", "N-max"):
        assert codes[label] == -2, label
    assert codes["abi"] == -7 and codes["rows"] == -3 and codes["stride"] == -4
    for label in ("N0", "term-bit", "v-alone", "dtype", "sign", "map-kind", "scale", "clip-neg"):
        assert codes[label] == -1, label
    assert codes["txl-nc-32000"] == 0 and codes["txl-nc-32768"] == -2
    assert codes["txl-c-46000"] == 0 and codes["txl-c-47000"] == -2
    assert codes["id-bias-f32-24000"] == -2
    for label in ("it-cfg4", "it-cfg5", "it-shaw", "it-txl-N1", "it-txl-nc-32768",
                  "it-txl-c-47000", "it-seg-drop"):
        assert codes[label] == 0, label
    for label in ("it-deberta", "it-f32", "it-split-seg"):
        assert codes[label] == -2, label
    assert codes["it-flag-2"] == -1
    if os.path.exists(rpa.library_path()):
        for (label, prob), line in zip(items, lines):
            assert _library_line(prob) == line, label


@needs_lib
def test_slice_limit_in_bytes():
    # an identity map's query slice holds N rows of about N + 128 entries:
    # 2-byte entries pass at N = 32000 (2.06e9 bytes) and fail at 32768
    # (2.16e9); fp32 offset gradients with a bias (4-byte entries) fail at
    # N = 24000 (2.3e9 bytes), which 2-byte entries would pass
    ok = rpa.plan_sizes(rpa.Problem(_txl(32000, False)))
    assert ok["z_bytes"] > 8 * 32000 * 32000 * 2
    for spec in (_txl(32768, False), _txl(24000, False, "f32", ("aq", "bias"))):
        with pytest.raises(rpa.RelposError) as ei:
            rpa.plan_sizes(rpa.Problem(spec))
        assert ei.value.code == -2
        assert "2^31" in rpa.library().relpos_last_error().decode()
    assert rpa.plan_sizes(rpa.Problem(_txl(24000, False, "bf16", ("aq",))))["delta"] == 23999
