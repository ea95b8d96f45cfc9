"""Plain-definition fp64 forward and backward ([RPA] §3, App. B.1).

For one (batch, head) slice with queries q_i, keys k_j, values v_j the score is
the unified additive form of [RPA] §3.2 Eq. (4), with the two Transformer-XL
query biases written out as in the configurations' score formula:

    S_ij = tau * ( (q_i + u) . k_j
                   + (q_i + v) . A^Q[phi_Q(i, j)]
                   + k_j . A^K[phi_K(i, j)]
                   + b[phi_b(i, j)] )  + M_ij

(absent terms are zero; M_ij = -inf for j > i under the causal mask, and
for pairs in different segments under a segment mask).  Then
P = softmax_row(S), O = P V and L_i = log sum_j exp(S_ij) ([RPA] §3.1 Eq. (1)).

Masks and dropout ([RPA] appendix "Masks, packing, and dropout", which names
padding masks, packed variable-length sequences and attention dropout without
formulas; the readings here):
  * segments: spec["segments"][b] lists disjoint token intervals [start, end)
    of batch element b.  A pair is visible iff both tokens lie in the same
    segment; tokens in no segment are padding.  One segment [0, L_b) is a
    padding mask of length L_b; several segments in one row are packed
    sequences.  Offsets stay delta = i - j (both tokens index the same row).
    A query with no visible key has O = 0, L = -inf and no gradient.
  * dropout: spec["dropout"] = {"p8": p8, "seed": seed} drops pair (i, j)
    with probability p8 / 256 by the counter-based mask of ``philox`` and
    scales the kept probabilities by 1 / (1 - p8 / 256): O = P~ V with
    P~ = P * keep * scale, while L stays the logsumexp of S.  Backward:
    dV = P~^T dO, dP = (dO V^T) * keep * scale, D_i = <dO_i, O_i>,
    dS = P * (dP - D) (D_i = sum_j P_ij dP_ij still holds).

Backward ([RPA] App. B.1, the dV/dS lemma): dV = P^T dO, dP = dO V^T,
D_i = <dO_i, O_i>, dS = P * (dP - D).  With G = tau * dS the relation
gradients follow [RPA] §3.2 Eq. (6) (one row of dZ per pair, by map row) and
the matrix products of the App. B.1 table-gradient lemma:

    dZ^Q[i, r] = sum_{j: phi_Q(i,j) = r} G_ij      dQ = G K + dZ^Q A^Q
    dZ^K[j, r] = sum_{i: phi_K(i,j) = r} G_ij      dK = G^T (Q + u) + dZ^K A^K
    dA^Q = (dZ^Q)^T (Q + v)      dA^K = (dZ^K)^T K      db[r] = sum_{phi_b = r} G
    du = sum_ij G_ij k_j         dv = sum_i (dZ^Q A^Q)_i

Table gradients are summed over the batch (and over heads for a table shared
by all heads).  Everything is float64.
"""

import numpy as np

from .maps import map_rows, relation_rows
from .philox import keep_mask, keep_scale


def _has(spec, term):
    return term in spec["terms"]


def _aq(spec, arrays, h):
    a = arrays["aq"]
    return a if spec["aq_shared"] else a[:, h, :]


def _rows(spec, term, rows):
    """Cached relation rows of ``term``; masked (causal) pairs get row 0, which
    they never contribute to (their P and dS are zero, [RPA] App. B.1)."""
    if term not in rows:
        rho = relation_rows(spec, term)
        if spec["causal"]:
            rho[np.triu_indices(spec["N"], 1)] = 0
        rows[term] = rho
    return rows[term]


def slice_scores(spec, arrays, b, h, rows=None):
    """Score matrix S (fp64, N x N) of slice (b, h), with the relation-row
    matrices used to build it.  ``rows`` caches ``relation_rows`` results."""
    N = spec["N"]
    tau = float(spec["scale"])
    q = arrays["q"][b, h]
    k = arrays["k"][b, h]
    rows = {} if rows is None else rows
    qc = q + arrays["u"][h] if _has(spec, "u") else q
    s = qc @ k.T
    if _has(spec, "aq"):
        _rows(spec, "aq", rows)
        a = _aq(spec, arrays, h)
        qp = q + arrays["v_bias"][h] if _has(spec, "v") else q
        zfull = qp @ a.T  # [N, R]: Z^Q of Eq. (5), every row
        s += np.take_along_axis(zfull, rows["aq"], axis=1)
    if _has(spec, "ak"):
        _rows(spec, "ak", rows)
        a = arrays["ak"][:, h, :]
        zfull = k @ a.T  # [N, R]: Z^K of Eq. (5)
        # term (i, j) = Z^K[j, phi_K(i, j)]
        s += np.take_along_axis(zfull.T, rows["ak"], axis=0)
    if _has(spec, "bias"):
        _rows(spec, "bias", rows)
        s += arrays["bias"][:, h][rows["bias"]]
    s *= tau
    if spec["causal"]:
        s[np.triu_indices(N, 1)] = -np.inf
    seg = segment_ids(spec, b)
    if seg is not None:
        s[(seg[:, None] != seg[None, :]) | (seg[:, None] < 0)] = -np.inf
    return s, rows


def segment_ids(spec, b):
    """Segment index of every token of batch element b (-1: padding), or None
    without a segment mask."""
    if spec.get("segments") is None:
        return None
    ids = np.full(spec["N"], -1, dtype=np.int64)
    for k, (start, end) in enumerate(spec["segments"][b]):
        assert 0 <= start <= end <= spec["N"] and np.all(ids[start:end] < 0), "bad segments"
        ids[start:end] = k
    return ids


def dropout_of(spec, b, h):
    """(keep mask, scale) of slice (b, h), or None without dropout."""
    dr = spec.get("dropout")
    if dr is None:
        return None
    return keep_mask(spec["N"], b * spec["H"] + h, dr["p8"], dr["seed"]), keep_scale(dr["p8"])


def slice_forward(spec, arrays, b, h, rows=None):
    """O (N x d) and natural-log L (N) of slice (b, h) ([RPA] §3.1 Eq. (1)),
    with the softmax P (before dropout).  A row with no visible key has P = 0,
    O = 0 and L = -inf."""
    s, rows = slice_scores(spec, arrays, b, h, rows)
    m = s.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)  # rows with no visible key
    e = np.exp(s - m)
    ssum = e.sum(axis=1, keepdims=True)
    p = e / np.where(ssum > 0, ssum, 1.0)
    dr = dropout_of(spec, b, h)
    pd = p if dr is None else p * dr[0] * dr[1]
    o = pd @ arrays["v"][b, h]
    with np.errstate(divide="ignore"):
        lse = (m + np.log(ssum))[:, 0]
    return o, lse, p, rows


def slice_forward_backward(spec, arrays, b, h, rows=None):
    """Forward and backward of one slice.  Returns a dict with o, lse, dq, dk,
    dv and this slice's contributions to the table gradients."""
    tau = float(spec["scale"])
    o, lse, p, rows = slice_forward(spec, arrays, b, h, rows)
    q = arrays["q"][b, h]
    k = arrays["k"][b, h]
    v = arrays["v"][b, h]
    do = arrays["do"][b, h]
    N = spec["N"]
    R = spec.get("rows", 0)
    out = {"o": o, "lse": lse}
    dr = dropout_of(spec, b, h)
    pd = p if dr is None else p * dr[0] * dr[1]
    out["dv"] = pd.T @ do                      # dV = P~^T dO
    dp = do @ v.T                              # dP = dO V^T
    if dr is not None:
        dp = dp * dr[0] * dr[1]                # through the dropout mask
    dd = np.sum(do * o, axis=1, keepdims=True)  # D_i = <dO_i, O_i>
    ds = p * (dp - dd)                         # dS = P * (dP - D)
    g = tau * ds                               # every term of S carries tau
    del p, pd, dp, ds
    dq = g @ k
    kc = k
    dk = g.T @ (q + arrays["u"][h] if _has(spec, "u") else q)
    if _has(spec, "u"):
        out["du"] = g.sum(axis=0) @ kc           # sum_ij G_ij k_j
    if _has(spec, "aq"):
        a = _aq(spec, arrays, h)
        # Eq. (6): dZ^Q[i, r] = sum over j with phi_Q(i, j) = r of G_ij
        flat = (np.arange(N)[:, None] * R + rows["aq"]).ravel()
        dzq = np.bincount(flat, weights=g.ravel(), minlength=N * R).reshape(N, R)
        qp = q + arrays["v_bias"][h] if _has(spec, "v") else q
        dq += dzq @ a
        out["daq"] = dzq.T @ qp
        if _has(spec, "v"):
            out["dv_bias"] = dzq.sum(axis=0) @ a
    if _has(spec, "ak"):
        a = arrays["ak"][:, h, :]
        # Eq. (6): dZ^K[j, r] = sum over i with phi_K(i, j) = r of G_ij
        flat = (np.arange(N)[None, :] * R + rows["ak"]).ravel()
        dzk = np.bincount(flat, weights=g.ravel(), minlength=N * R).reshape(N, R)
        dk += dzk @ a
        out["dak"] = dzk.T @ k
    if _has(spec, "bias"):
        out["dbias"] = np.bincount(rows["bias"].ravel(), weights=g.ravel(), minlength=R)
    out["dq"] = dq
    out["dk"] = dk
    return out


def query_rows(spec, arrays, b, h, qidx):
    """O, L and dQ of the query rows ``qidx`` of slice (b, h), for sequences
    too long for the N x N slice.  The same definitions as
    ``slice_forward_backward``, evaluated on those rows only: a row's
    softmax, its D_i = <dO_i, O_i> and dQ_i = sum_j G_ij k_j + sum_r
    dZ^Q[i, r] A^Q[r] involve that row alone ([RPA] App. B.1).  Without
    segment masks or dropout."""
    assert spec.get("segments") is None and spec.get("dropout") is None
    N = spec["N"]
    tau = float(spec["scale"])
    qidx = np.asarray(qidx, dtype=np.int64)
    n = qidx.size
    jdx = np.arange(N, dtype=np.int64)
    delta = qidx[:, None] - jdx[None, :]
    masked = delta < 0 if spec["causal"] else np.zeros_like(delta, dtype=bool)

    def rho(term):
        r = map_rows(spec["map"], spec["signs"][term] * delta)
        r[masked] = 0  # masked pairs contribute nothing; any valid row serves
        return r

    q = arrays["q"][b, h][qidx]
    k = arrays["k"][b, h]
    v = arrays["v"][b, h]
    do = arrays["do"][b, h][qidx]
    s = (q + arrays["u"][h] if _has(spec, "u") else q) @ k.T
    if _has(spec, "aq"):
        a = _aq(spec, arrays, h)
        rq = rho("aq")
        qp = q + arrays["v_bias"][h] if _has(spec, "v") else q
        s += np.take_along_axis(qp @ a.T, rq, axis=1)
    if _has(spec, "ak"):
        zk = k @ arrays["ak"][:, h, :].T  # Z^K [N, R]
        s += zk[jdx[None, :], rho("ak")]  # Z^K[j, phi_K(i, j)]
    if _has(spec, "bias"):
        s += arrays["bias"][:, h][rho("bias")]
    s *= tau
    s[masked] = -np.inf
    m = s.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m)
    ssum = e.sum(axis=1, keepdims=True)
    p = e / np.where(ssum > 0, ssum, 1.0)
    o = p @ v
    with np.errstate(divide="ignore"):
        lse = (m + np.log(ssum))[:, 0]
    dd = np.sum(do * o, axis=1, keepdims=True)
    g = tau * p * (do @ v.T - dd)
    dq = g @ k
    if _has(spec, "aq"):
        R = spec["rows"]
        flat = (np.arange(n)[:, None] * R + rq).ravel()
        dzq = np.bincount(flat, weights=g.ravel(), minlength=n * R).reshape(n, R)
        dq += dzq @ a
    return o, lse, dq


def _empty_grads(spec):
    B, H, N, d = spec["B"], spec["H"], spec["N"], spec["d"]
    R = spec.get("rows", 0)
    z = {"o": np.zeros((B, H, N, d)), "lse": np.zeros((B, H, N)),
         "dq": np.zeros((B, H, N, d)), "dk": np.zeros((B, H, N, d)),
         "dv": np.zeros((B, H, N, d))}
    if _has(spec, "aq"):
        z["daq"] = np.zeros((R, d)) if spec["aq_shared"] else np.zeros((R, H, d))
    if _has(spec, "ak"):
        z["dak"] = np.zeros((R, H, d))
    if _has(spec, "bias"):
        z["dbias"] = np.zeros((R, H))
    if _has(spec, "u"):
        z["du"] = np.zeros((H, d))
    if _has(spec, "v"):
        z["dv_bias"] = np.zeros((H, d))
    return z


def forward_backward(spec, arrays, heads=None, batches=None):
    """Full forward + backward over the slices (b in ``batches``, h in ``heads``;
    default all).  Returns full-shape arrays; slices not computed stay zero, and
    table gradients hold only the computed slices' contributions."""
    heads = range(spec["H"]) if heads is None else heads
    batches = range(spec["B"]) if batches is None else batches
    res = _empty_grads(spec)
    rows = {}
    for h in heads:
        for b in batches:
            r = slice_forward_backward(spec, arrays, b, h, rows)
            for key in ("o", "lse", "dq", "dk", "dv"):
                res[key][b, h] = r[key]
            if "daq" in r:
                if spec["aq_shared"]:
                    res["daq"] += r["daq"]
                else:
                    res["daq"][:, h] += r["daq"]
            if "dak" in r:
                res["dak"][:, h] += r["dak"]
            if "dbias" in r:
                res["dbias"][:, h] += r["dbias"]
            if "du" in r:
                res["du"][h] += r["du"]
            if "dv_bias" in r:
                res["dv_bias"][h] += r["dv_bias"]
    return res


def forward(spec, arrays):
    """O [B,H,N,d] and L [B,H,N] (natural log)."""
    B, H = spec["B"], spec["H"]
    o = np.zeros((B, H, spec["N"], spec["d"]))
    lse = np.zeros((B, H, spec["N"]))
    rows = {}
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h], _, rows = slice_forward(spec, arrays, b, h, rows)
    return o, lse


def backward(spec, arrays):
    """All gradients (recomputes the forward; the oracle keeps nothing)."""
    res = forward_backward(spec, arrays)
    return {key: val for key, val in res.items() if key not in ("o", "lse")}

