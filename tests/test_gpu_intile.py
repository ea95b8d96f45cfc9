"""GPU parity of the in-tile relation products ([RPA] §6 "Limitations",
Table 7 row "Projections": every tile computes its own relation products,
nothing quadratic is stored) against the fp64 oracle, through the C ABI.
The oracle is the same plain definition as for the stored projections: the
mode changes where the products are computed, not what is computed.
Shapes span several 128-query workgroups and end in ragged tiles."""

import copy

import numpy as np
import pytest
import torch

import oracle
import relative_position_attention_amd as rpa
from synth import make_problem
from gpu_util import check, run_library, to_device, TOL

pytestmark = pytest.mark.gpu


def _problem(kind, causal, seed, N=700, B=2, H=2):
    spec, arr = make_problem(kind=kind, B=B, H=H, N=N, dtype="bf16", seed=seed, causal=causal,
                             clip=40, d_model=128, table_std=0.5 if kind == "shaw" else 1.0)
    spec = copy.deepcopy(spec)
    spec["in_tile"] = True
    return spec, arr


def _forward(spec, arr, out_dtype="f32"):
    prob = rpa.Problem(spec, out_dtype=out_dtype)
    t = to_device(spec, arr)
    o, lse, _ = rpa.attn_fwd(prob, t, retain=False)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["txl", "shaw"])
@pytest.mark.parametrize("N", [700, 1])
def test_intile_forward(kind, causal, N):
    spec, arr = _problem(kind, causal, 51 + N, N=N)
    print(f"[intile] fwd {kind} causal={causal} N={N}", flush=True)
    o, lse = _forward(spec, arr)
    ref = oracle.forward(spec, arr)
    tol_abs, tol_rel = TOL["bf16"]
    for key, got in (("o", o), ("lse", lse)):
        want = ref[key] if isinstance(ref, dict) else (ref[0] if key == "o" else ref[1])
        ma = float(np.max(np.abs(got - want)))
        rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
        print(f"  {key} max_abs={ma:.3e} rel_l2={rel:.3e}", flush=True)
        assert ma <= tol_abs and rel <= tol_rel


def test_intile_matches_stored_projections():
    # the same problem with and without stored projections: both exact to
    # the bf16 contract, and close to each other
    spec, arr = _problem("txl", True, 61, N=1000)
    o1, l1 = _forward(spec, arr)
    spec0 = dict(spec, in_tile=False)
    o0, l0 = _forward(spec0, arr)
    assert float(np.max(np.abs(o1 - o0))) < 2e-2
    assert float(np.max(np.abs(l1 - l0))) < 2e-2


def test_intile_rejects_key_table():
    spec, arr = make_problem(kind="deberta", B=1, H=2, N=200, dtype="bf16", seed=3, causal=False,
                             d_model=128)
    spec = dict(spec, in_tile=True)
    with pytest.raises(rpa.RelposError) as e:
        _forward(spec, arr)
    assert e.value.code == -2
