"""Per-pair brute force, for tiny inputs only (pure Python loops, fp64).

This is the eager reference style of [RPA] §5.1 "Correctness": the relation
vector of every query-key pair is gathered individually and the score built
pair by pair.  Gradients are accumulated pair by pair with the chain rule
written out directly on the score of each pair (no relation-row reduction),
so this module checks the vectorised oracle's gathers and scatters.
"""

import math

import numpy as np

from .maps import map_rows
from .philox import philox4x32, keep_scale


def _row(spec, term, i, j):
    return int(map_rows(spec["map"], np.array([spec["signs"][term] * (i - j)]))[0])


def _visible(spec, b, i, j):
    """Pair (i, j) of batch element b under the causal and segment masks."""
    if spec["causal"] and j > i:
        return False
    segs = spec.get("segments")
    if segs is None:
        return True
    return any(start <= i < end and start <= j < end for start, end in segs[b])


def _kept(spec, bh, i, j):
    """Dropout factor of pair (i, j): 0 if dropped, else the keep scale (one
    Philox call per pair, the byte of the pair picked out of its block)."""
    dr = spec.get("dropout")
    if dr is None:
        return 1.0
    words = philox4x32(j >> 2, i >> 2, bh, 0, dr["seed"] & 0xFFFFFFFF, dr["seed"] >> 32)
    byte = (int(words[i & 3]) >> (8 * (j & 3))) & 0xFF
    return keep_scale(dr["p8"]) if byte >= dr["p8"] else 0.0


def brute_forward_backward(spec, arrays):
    B, H, N, d = spec["B"], spec["H"], spec["N"], spec["d"]
    tau = float(spec["scale"])
    terms = spec["terms"]
    R = spec.get("rows", 0)
    out = {k: np.zeros((B, H, N, d)) for k in ("o", "dq", "dk", "dv")}
    out["lse"] = np.zeros((B, H, N))
    if "aq" in terms:
        out["daq"] = np.zeros((R, d)) if spec["aq_shared"] else np.zeros((R, H, d))
    if "ak" in terms:
        out["dak"] = np.zeros((R, H, d))
    if "bias" in terms:
        out["dbias"] = np.zeros((R, H))
    if "u" in terms:
        out["du"] = np.zeros((H, d))
    if "v" in terms:
        out["dv_bias"] = np.zeros((H, d))

    def dot(a, b):
        return float(sum(x * y for x, y in zip(a, b)))

    for b in range(B):
        for h in range(H):
            q = arrays["q"][b, h]
            k = arrays["k"][b, h]
            v = arrays["v"][b, h]
            do = arrays["do"][b, h]
            u = arrays["u"][h] if "u" in terms else np.zeros(d)
            vb = arrays["v_bias"][h] if "v" in terms else np.zeros(d)

            def aq_row(r):
                return arrays["aq"][r] if spec["aq_shared"] else arrays["aq"][r, h]

            S = [[-math.inf] * N for _ in range(N)]
            for i in range(N):
                for j in range(N):
                    if not _visible(spec, b, i, j):
                        continue
                    val = dot(q[i] + u, k[j])
                    if "aq" in terms:
                        val += dot(q[i] + vb, aq_row(_row(spec, "aq", i, j)))
                    if "ak" in terms:
                        val += dot(k[j], arrays["ak"][_row(spec, "ak", i, j), h])
                    if "bias" in terms:
                        val += arrays["bias"][_row(spec, "bias", i, j), h]
                    S[i][j] = tau * val
            P = [[0.0] * N for _ in range(N)]
            X = [[_kept(spec, b * H + h, i, j) for j in range(N)] for i in range(N)]
            for i in range(N):
                m = max(S[i])
                if m == -math.inf:  # no visible key: O = 0, L = -inf
                    out["lse"][b, h, i] = -math.inf
                    continue
                tot = sum(math.exp(s - m) for s in S[i])
                out["lse"][b, h, i] = m + math.log(tot)
                for j in range(N):
                    P[i][j] = math.exp(S[i][j] - m) / tot
                for j in range(N):
                    out["o"][b, h, i] += P[i][j] * X[i][j] * v[j]
            o = out["o"][b, h]
            for i in range(N):
                Di = dot(do[i], o[i])
                for j in range(N):
                    if P[i][j] == 0.0:
                        continue
                    out["dv"][b, h, j] += P[i][j] * X[i][j] * do[i]
                    dS = P[i][j] * (X[i][j] * dot(do[i], v[j]) - Di)
                    g = tau * dS
                    # d/dq_i and d/dk_j of the content term (q_i + u) . k_j
                    out["dq"][b, h, i] += g * k[j]
                    out["dk"][b, h, j] += g * (q[i] + u)
                    if "u" in terms:
                        out["du"][h] += g * k[j]
                    if "aq" in terms:
                        r = _row(spec, "aq", i, j)
                        a = aq_row(r)
                        out["dq"][b, h, i] += g * a
                        if spec["aq_shared"]:
                            out["daq"][r] += g * (q[i] + vb)
                        else:
                            out["daq"][r, h] += g * (q[i] + vb)
                        if "v" in terms:
                            out["dv_bias"][h] += g * a
                    if "ak" in terms:
                        r = _row(spec, "ak", i, j)
                        out["dk"][b, h, j] += g * arrays["ak"][r, h]
                        out["dak"][r, h] += g * k[j]
                    if "bias" in terms:
                        out["dbias"][_row(spec, "bias", i, j), h] += g
    return out
