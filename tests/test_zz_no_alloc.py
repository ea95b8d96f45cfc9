"""relpos_project_noalloc (the allocation-free projection, for callers that
cannot allocate device memory) against relpos_project through the C ABI.

Two calls in a row share the library's static scratch, the second on a
smaller problem; each call's projections feed relpos_attn_fwd and
relpos_attn_bwd, whose outputs must equal, bit for bit, those computed from
relpos_project's projections (same kernels, same inputs).  The size check is
host-only and runs without a GPU."""

import ctypes

import numpy as np
import pytest
import torch

import relative_position_attention_amd as rpa
from synth import make_problem, scaled_config
from gpu_util import split_operands_for, to_device


def _txl_wide(N, H):
    spec = make_problem(kind="txl", B=1, H=8, N=64, dtype="bf16", seed=0, causal=False,
                        d_model=128)[0]
    return dict(spec, N=N, H=H, rows=2 * N - 1, map={"kind": "identity", "offset": N - 1})


def test_noalloc_rejects_oversized_workspace():
    # an identity map over 2N - 1 offsets with 16 heads needs 16 x 63999 x 64 x 2
    # bytes of expanded table, above the 64 MiB scratch: refused before any
    # device call
    prob = rpa.Problem(_txl_wide(32000, 16))
    assert rpa.plan_sizes(prob)["fwd_ws_bytes"] > 64 << 20
    lib = rpa.library()
    z = ctypes.c_void_p(256)
    rc = lib.relpos_project_noalloc(ctypes.byref(prob.desc), ctypes.byref(prob.shape),
                                    ctypes.byref(rpa.binding._Tensors()), z, 1 << 40, None)
    assert rc == -5
    assert "static scratch" in lib.relpos_last_error().decode()


def _outputs(prob, t, z):
    o, lse, _ = rpa.attn_fwd(prob, t, z=z)
    g = rpa.attn_bwd(prob, t, o, lse, t["do"], z=z)
    torch.cuda.synchronize()
    res = {"o": o, "lse": lse}
    res.update(g)
    return {k: v.cpu() for k, v in res.items()}


@pytest.mark.gpu
def test_noalloc_matches_project_twice():
    # first call: DeBERTa recipe (two tables, bucketed maps); second call,
    # smaller: Shaw recipe with a shared table, so the scratch holds the first
    # call's larger contents when the second runs
    problems = [scaled_config(3, B=2, H=3, N=700), scaled_config(1, B=1, H=2, N=200)]
    for k, (spec, arr) in enumerate(problems):
        print(f"[noalloc] call {k}: B={spec['B']} H={spec['H']} N={spec['N']} "
              f"dtype={spec['dtype']}", flush=True)
        prob = rpa.Problem(spec, out_dtype="f32", split_operands=split_operands_for(spec))
        t = to_device(spec, arr)
        sz = rpa.plan_sizes(prob)
        z_ref = rpa.project(prob, t)
        z_new = torch.zeros(max(sz["z_bytes"], 256), dtype=torch.uint8, device="cuda")
        rpa.project_noalloc(prob, t, z_new)
        torch.cuda.synchronize()
        ref = _outputs(prob, t, z_ref)
        got = _outputs(prob, t, z_new)
        for key in ref:
            assert torch.equal(ref[key], got[key]), (k, key)
        assert np.isfinite(got["o"].numpy()).all()
