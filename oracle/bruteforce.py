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


def _row(spec, term, i, j):
    return int(map_rows(spec["map"], np.array([spec["signs"][term] * (i - j)]))[0])


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
                    if spec["causal"] and j > i:
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
            for i in range(N):
                m = max(S[i])
                tot = sum(math.exp(s - m) for s in S[i])
                out["lse"][b, h, i] = m + math.log(tot)
                for j in range(N):
                    P[i][j] = math.exp(S[i][j] - m) / tot
                for j in range(N):
                    out["o"][b, h, i] += P[i][j] * v[j]
            o = out["o"][b, h]
            for i in range(N):
                Di = dot(do[i], o[i])
                for j in range(N):
                    if P[i][j] == 0.0:
                        continue
                    out["dv"][b, h, j] += P[i][j] * do[i]
                    dS = P[i][j] * (dot(do[i], v[j]) - Di)
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
