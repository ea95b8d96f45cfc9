"""Problem recipes: the five parity configurations and the 8K-token bench shapes.

A problem is ``(spec, arrays)``.  ``spec`` is a plain dict describing the
mechanism; ``arrays`` maps names to float64 numpy arrays holding values that
are exactly representable in the problem's dtype.

spec keys
---------
name, B, H, N, d           sizes; inputs are [B, H, N, d] row-major
dtype                      "f32" or "bf16" (inputs, tables, u, v, dO)
causal                     bool; masks pairs with key index j > query index i
scale                      tau, multiplies the whole score (bias terms included)
map                        relation map, applied to sign * (i - j):
    {"kind": "identity", "offset": o}                  row = x + o
    {"kind": "clipped", "clip": D}                     row = clip(x, -D, D) + D
    {"kind": "t5", "num_buckets", "max_distance", "bidirectional"}
    {"kind": "log", "bucket_size", "max_position"}     DeBERTa-style log buckets,
                                                       row = clip(bkt(x)+bs, 0, 2bs-1)
    {"kind": "explicit", "clip": c, "rows": [...]}     row = rows[clip(x,-c,c)+c]
signs                      {"aq": +-1, "ak": +-1, "bias": +-1}
terms                      subset of ["aq", "ak", "bias", "u", "v"]
rows                       R, rows of every relation table
aq_shared                  True if A^Q is one [R, d] table shared by all heads

arrays
------
q, k, v, do   [B, H, N, d]
aq, ak        [R, H, d]  (aq is [R, d] when aq_shared)
bias          [R, H]
u, v_bias     [H, d]
"""

import math

import numpy as np

D_HEAD = 64


def round_to_dtype(x, dtype):
    """Round float64 values once, to nearest-even, to ``dtype``; return float64."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        m, e = np.frexp(x)  # x = m * 2**e, 0.5 <= |m| < 1
        # bf16 keeps 8 significant bits: scale the significand to [128, 256).
        r = np.rint(m * 256.0)  # numpy rint rounds half to even
        return np.ldexp(r, e - 8)
    raise ValueError(dtype)


def _normal(rng, shape, std=1.0):
    return rng.standard_normal(shape) * std


def _sinusoid(positions, d_model):
    """Sinusoidal embedding of (signed) integer positions, [len(positions), d_model]."""
    pos = np.asarray(positions, dtype=np.float64)[:, None]
    k2 = np.arange(0, d_model, 2, dtype=np.float64)[None, :]
    ang = pos / np.power(10000.0, k2 / d_model)
    pe = np.empty((pos.shape[0], d_model), dtype=np.float64)
    pe[:, 0::2] = np.sin(ang)
    pe[:, 1::2] = np.cos(ang)
    return pe


def make_problem(kind, B, H, N, dtype, seed, *, causal=False, clip=16, qkv_std=1.0,
                 table_std=1.0, bias_std=0.5, d_model=None, name=None, shared_table=True):
    """Build one problem of mechanism ``kind`` in {"shaw", "t5", "deberta", "txl"}."""
    d = D_HEAD
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, H, N, d), qkv_std)
    k = _normal(rng, (B, H, N, d), qkv_std)
    v = _normal(rng, (B, H, N, d), qkv_std)
    do = _normal(rng, (B, H, N, d), 1.0)
    arrays = {"q": q, "k": k, "v": v, "do": do}
    spec = {"name": name or kind, "B": B, "H": H, "N": N, "d": d, "dtype": dtype,
            "causal": bool(causal), "signs": {"aq": 1, "ak": 1, "bias": 1},
            "aq_shared": False}
    if kind == "shaw":
        # Shaw et al.: q_i . R[clip(j - i, -D, D) + D], one table shared by all heads.
        R = 2 * clip + 1
        spec.update(scale=1.0 / math.sqrt(d), map={"kind": "clipped", "clip": clip},
                    terms=["aq"], rows=R, aq_shared=bool(shared_table))
        spec["signs"]["aq"] = -1
        arrays["aq"] = _normal(rng, (R, d) if shared_table else (R, H, d), table_std)
    elif kind == "t5":
        R = 32
        spec.update(scale=1.0, map={"kind": "t5", "num_buckets": 32, "max_distance": 128,
                                    "bidirectional": True},
                    terms=["bias"], rows=R)
        spec["signs"]["bias"] = -1  # bucket of (j - i)
        arrays["bias"] = _normal(rng, (R, H), bias_std)
    elif kind == "deberta":
        bs, mp = 256, 512
        R = 2 * bs
        dm = d_model or H * d
        rel = _normal(rng, (R, dm), 0.02)
        wk = _normal(rng, (dm, H * d), 0.02)
        wq = _normal(rng, (dm, H * d), 0.02)
        spec.update(scale=1.0 / math.sqrt(3 * d),
                    map={"kind": "log", "bucket_size": bs, "max_position": mp},
                    terms=["aq", "ak"], rows=R)
        spec["signs"]["aq"] = 1   # c2p: q_i . Kr[row(i - j)]
        spec["signs"]["ak"] = -1  # p2c: k_j . Qr[row(j - i)]
        arrays["aq"] = (rel @ wk).reshape(R, H, d)
        arrays["ak"] = (rel @ wq).reshape(R, H, d)
    elif kind == "txl":
        dm = d_model or H * d
        if causal:
            R = N
            positions = np.arange(0, N)
            mp = {"kind": "identity", "offset": 0}
        else:
            R = 2 * N - 1
            positions = np.arange(0, R) - (N - 1)
            mp = {"kind": "identity", "offset": N - 1}
        wr = _normal(rng, (dm, H * d), 0.02)
        u = _normal(rng, (H, d), 0.02)
        vb = _normal(rng, (H, d), 0.02)
        pe = _sinusoid(positions, dm)
        spec.update(scale=1.0 / math.sqrt(d), map=mp, terms=["aq", "u", "v"], rows=R)
        arrays["aq"] = (pe @ wr).reshape(R, H, d)
        arrays["u"] = u
        arrays["v_bias"] = vb
    else:
        raise ValueError(kind)
    for key in list(arrays):
        arrays[key] = round_to_dtype(arrays[key], dtype)
    return spec, arrays


def make_mixed(terms, B, H, N, dtype, seed, *, causal=False, clip=16, term_std=0.5):
    """A problem with any subset of the relation terms over one clipped map
    (row = clip(x, -clip, clip) + clip of the signed offset), for the term
    combinations no single mechanism uses: per-head tables, bias, u and v all
    N(0, term_std^2), so each term moves the scores visibly at tau = 1/8."""
    d = D_HEAD
    rng = np.random.default_rng(seed)
    arrays = {name: _normal(rng, (B, H, N, d), 1.0) for name in ("q", "k", "v", "do")}
    R = 2 * clip + 1
    spec = {"name": "mixed-" + "+".join(terms), "B": B, "H": H, "N": N, "d": d,
            "dtype": dtype, "causal": bool(causal), "signs": {"aq": 1, "ak": -1, "bias": 1},
            "aq_shared": False, "scale": 1.0 / math.sqrt(d),
            "map": {"kind": "clipped", "clip": clip}, "terms": list(terms), "rows": R}
    if "aq" in terms:
        arrays["aq"] = _normal(rng, (R, H, d), term_std)
    if "ak" in terms:
        arrays["ak"] = _normal(rng, (R, H, d), term_std)
    if "bias" in terms:
        arrays["bias"] = _normal(rng, (R, H), term_std)
    if "u" in terms:
        arrays["u"] = _normal(rng, (H, d), term_std)
    if "v" in terms:
        arrays["v_bias"] = _normal(rng, (H, d), term_std)
    for key in list(arrays):
        arrays[key] = round_to_dtype(arrays[key], dtype)
    return spec, arrays


# The five parity configurations (seed = configuration number).
CONFIGS = {
    1: dict(kind="shaw", B=1, H=2, N=128, dtype="f32", seed=1, clip=16,
            name="cfg1_shaw_fp32"),
    2: dict(kind="t5", B=4, H=16, N=2048, dtype="bf16", seed=2, bias_std=0.5,
            name="cfg2_t5"),
    3: dict(kind="deberta", B=2, H=12, N=4096, dtype="bf16", seed=3, d_model=768,
            name="cfg3_deberta"),
    4: dict(kind="txl", B=1, H=8, N=8192, dtype="bf16", seed=4, causal=True, d_model=512,
            name="cfg4_txl_causal"),
    5: dict(kind="txl", B=1, H=8, N=16384, dtype="bf16", seed=5, causal=False,
            d_model=512, qkv_std=1.0 / math.sqrt(D_HEAD), name="cfg5_conformer_txl"),
}

# The 8K-token attention-level bench shapes (16K-token budget: B = 2, H = 12).
BENCH_SHAPES = {
    "shaw": dict(kind="shaw", B=2, H=12, N=8192, dtype="bf16", seed=101, clip=256,
                 name="bench_shaw_8k"),
    "t5": dict(kind="t5", B=2, H=12, N=8192, dtype="bf16", seed=102, bias_std=0.5,
               name="bench_t5_8k"),
    "deberta": dict(kind="deberta", B=2, H=12, N=8192, dtype="bf16", seed=103,
                    d_model=768, name="bench_deberta_8k"),
    "txl": dict(kind="txl", B=1, H=8, N=8192, dtype="bf16", seed=104, causal=True,
                d_model=512, name="bench_txl_causal_8k"),
}


def make_config(idx):
    """The parity configuration ``idx`` (1..5) at its full size."""
    return make_problem(**CONFIGS[idx])


def scaled_config(idx, *, B=None, H=None, N=None, seed=None, **over):
    """Configuration ``idx``'s recipe at other sizes (same dtype, map and tables)."""
    kw = dict(CONFIGS[idx])
    if B is not None:
        kw["B"] = B
    if H is not None:
        kw["H"] = H
    if N is not None:
        kw["N"] = N
    if seed is not None:
        kw["seed"] = seed
    kw.update(over)
    kw["name"] = f"{kw['name']}_B{kw['B']}H{kw['H']}N{kw['N']}"
    return make_problem(**kw)


def make_bench(name):
    return make_problem(**BENCH_SHAPES[name])
