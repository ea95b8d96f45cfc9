"""CPU checks of the bench's work models: the reduction stages' byte model
(reachable offset-gradient entries per token, the band rows 1 .. 2D-1 of
the expanded map) against a brute-force count over every (query, key) pair,
and the credited FLOPs of a causal problem against a count of visible pairs."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _entries(N, D, causal, key_side):
    """Distinct (token, expanded row s) band entries, s = clip(i - j, -D, D) + D
    restricted to 1 .. 2D - 1, counted pair by pair."""
    seen = set()
    for i in range(N):
        for j in range(N):
            if causal and j > i:
                continue
            s = max(-D, min(D, i - j)) + D
            if 1 <= s <= 2 * D - 1:
                seen.add((j if key_side else i, s))
    return len(seen)


@pytest.mark.parametrize("N,D,causal", [(1, 1, False), (17, 4, False), (40, 7, True),
                                        (33, 40, False), (29, 28, True), (64, 0, False)])
@pytest.mark.parametrize("terms", [["aq"], ["bias"], ["aq", "ak"], ["aq", "u", "v"]])
def test_reduction_bytes_brute_force(N, D, causal, terms):
    B, H = 2, 3
    spec = {"B": B, "H": H, "N": N, "causal": causal, "terms": terms}
    q, k = bench.reduction_bytes(spec, D)
    tok = B * H * N * 64 * 8  # fp32 partial read + fp32 output written
    q_tok = tok if "aq" in terms else 0
    k_tok = tok if ("ak" in terms or "u" in terms) else 0
    q_reads = ("aq" in terms) + 1  # every term list here has a query-side entry
    q_size = 4 if "bias" in terms else 2
    k_reads = 2 if "ak" in terms else 0
    assert q == q_tok + q_reads * B * H * _entries(N, D, causal, False) * q_size
    assert k == k_tok + k_reads * B * H * _entries(N, D, causal, True) * 2


def test_causal_credit_counts_visible_pairs():
    spec = {"B": 1, "H": 1, "N": 10, "d": 64, "causal": True, "terms": [], "rows": 0}
    fwd, bwd = bench.credited_flops(spec)
    visible = sum(i + 1 for i in range(10))
    assert fwd == pytest.approx(4 * 64 * visible)
    assert bwd == pytest.approx(2 * fwd)
    assert bench.pair_flops(spec) == pytest.approx(2 * 64 * visible)


def test_bench_calls_only_defined_names():
    # every bare name bench.py calls is defined somewhere in it (a function,
    # an import or an assignment) or is a builtin: a deleted helper fails here
    # instead of in the timed run
    import ast
    import builtins
    src = open(os.path.join(ROOT, "bench.py")).read()
    tree = ast.parse(src)
    defined = set(dir(builtins))
    for node in ast.walk(tree):
        if isinstance(node, (ast.FunctionDef, ast.ClassDef)):
            defined.add(node.name)
            defined.update(a.arg for a in node.args.args + node.args.kwonlyargs) if isinstance(node, ast.FunctionDef) else None
        elif isinstance(node, (ast.Import, ast.ImportFrom)):
            defined.update((a.asname or a.name).split(".")[0] for a in node.names)
        elif isinstance(node, ast.Name) and isinstance(node.ctx, ast.Store):
            defined.add(node.id)
        elif isinstance(node, ast.arg):
            defined.add(node.arg)
    called = {n.func.id for n in ast.walk(tree) if isinstance(n, ast.Call) and isinstance(n.func, ast.Name)}
    assert called <= defined, sorted(called - defined)
