"""ctypes binding of include/relpos.h (argument marshalling only)."""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "librelpos.so"

EXPORTED_SYMBOLS = (
    "relpos_plan_sizes", "relpos_plan_rows", "relpos_project", "relpos_attn_fwd",
    "relpos_attn_bwd", "relpos_strerror", "relpos_last_error", "relpos_abi_version",
    "relpos_set_stage_events", "relpos_project_noalloc",
)

ABI_VERSION = 4
MAP_KIND = {"identity": 0, "clipped": 1, "t5": 2, "log": 3, "explicit": 4}
DTYPE = {"f32": 0, "bf16": 1}
TERM = {"aq": 1, "ak": 2, "bias": 4, "u": 8, "v": 16}


class RelposError(RuntimeError):
    def __init__(self, code, where, detail=""):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} ({code}) {detail}".strip())


class _Map(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("clip", ctypes.c_int32),
                ("identity_offset", ctypes.c_int32), ("num_buckets", ctypes.c_int32),
                ("max_distance", ctypes.c_int32), ("bidirectional", ctypes.c_int32),
                ("bucket_size", ctypes.c_int32), ("max_position", ctypes.c_int32),
                ("explicit_rows", ctypes.POINTER(ctypes.c_int32))]


class _Desc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("terms", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("num_rows", ctypes.c_int32), ("sign_q", ctypes.c_int32),
                ("sign_k", ctypes.c_int32), ("sign_b", ctypes.c_int32),
                ("split_operands", ctypes.c_int32), ("map", _Map),
                ("aq_row_stride", ctypes.c_int64), ("aq_head_stride", ctypes.c_int64),
                ("ak_row_stride", ctypes.c_int64), ("ak_head_stride", ctypes.c_int64),
                ("bias_row_stride", ctypes.c_int64), ("bias_head_stride", ctypes.c_int64),
                ("segmented", ctypes.c_int32), ("dropout_p8", ctypes.c_int32),
                ("dropout_seed", ctypes.c_uint64), ("in_tile", ctypes.c_int32),
                ("reserved0", ctypes.c_int32)]


class _Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32)]


class _Tensors(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("q", "k", "v", "aq", "ak", "bias", "u", "vbias",
                                                "seg")]


class _Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dq", "dk", "dv", "daq", "dak", "dbias", "du",
                                                "dvbias")]


class _Sizes(ctypes.Structure):
    _fields_ = [("z_bytes", ctypes.c_size_t), ("fwd_ws_bytes", ctypes.c_size_t),
                ("fwd_ws_bytes_noz", ctypes.c_size_t), ("bwd_ws_bytes", ctypes.c_size_t),
                ("bwd_ws_bytes_noz", ctypes.c_size_t), ("delta", ctypes.c_int32),
                ("expanded_rows", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("num_groups", ctypes.c_int32)]


_LIB = None


def library_path():
    return os.environ.get("RELPOS_LIBRARY", os.path.join(HERE, LIB_NAME))


def library():
    """The loaded HIP library; raises if it was not built."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"HIP library {path} not built: run "
                               "`python -m relative_position_attention_amd.build`")
        lib = ctypes.CDLL(path)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        lib.relpos_plan_sizes.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Shape),
                                          ctypes.POINTER(_Sizes)]
        lib.relpos_plan_rows.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Shape), i32,
                                         ctypes.POINTER(ctypes.c_int32), i32]
        lib.relpos_project.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Shape),
                                       ctypes.POINTER(_Tensors), vp, ctypes.c_size_t, vp,
                                       ctypes.c_size_t, vp]
        lib.relpos_project_noalloc.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Shape),
                                               ctypes.POINTER(_Tensors), vp, ctypes.c_size_t, vp]
        lib.relpos_attn_fwd.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Shape),
                                        ctypes.POINTER(_Tensors), vp, ctypes.c_size_t, vp, vp,
                                        vp, ctypes.c_size_t, vp]
        lib.relpos_attn_bwd.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Shape),
                                        ctypes.POINTER(_Tensors), vp, ctypes.c_size_t, vp, vp,
                                        vp, ctypes.POINTER(_Grads), vp, ctypes.c_size_t, vp]
        lib.relpos_strerror.restype = ctypes.c_char_p
        lib.relpos_strerror.argtypes = [ctypes.c_int]
        lib.relpos_last_error.restype = ctypes.c_char_p
        lib.relpos_last_error.argtypes = []
        lib.relpos_abi_version.restype = ctypes.c_int
        lib.relpos_set_stage_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32]
        if lib.relpos_abi_version() != ABI_VERSION:
            raise RuntimeError("librelpos.so ABI version mismatch")
        _LIB = lib
    return _LIB


def strerror(code):
    try:
        return library().relpos_strerror(code).decode()
    except RuntimeError:
        return "unknown"


def _check(code, where):
    if code < 0:
        raise RelposError(code, where, library().relpos_last_error().decode())
    return code


class Problem:
    """Descriptor and shape of one attention problem.

    ``spec`` uses the keys of the synthetic-problem recipes: B, H, N, d,
    dtype, causal, scale, map, signs, terms, rows, aq_shared, and optionally
    segments (per batch row a list of token intervals [start, end); the
    tensors then carry "seg", see segment_bounds) and dropout
    ({"p8": drop probability in 1/256, "seed": 64-bit Philox key}) and
    in_tile (True: relation products computed inside the tiles, nothing
    quadratic stored; bf16 inputs with the A^Q term).  ``out_dtype``
    is the dtype of O, dQ, dK, dV ("f32" or "bf16").  ``split_operands``
    sets the descriptor field of that name (bf16 inputs only): P and the
    score gradient enter their MFMA products as bf16 hi + lo pairs, which a
    strongly peaked softmax needs (T5 at tau = 1 with unit-variance inputs).
    """

    def __init__(self, spec, out_dtype=None, split_operands=False):
        self.spec = spec
        self.out_dtype = out_dtype or spec["dtype"]
        d = _Desc()
        d.abi_version = ABI_VERSION
        d.terms = sum(TERM[t] for t in spec["terms"])
        d.causal = int(bool(spec["causal"]))
        d.scale = float(spec["scale"])
        d.dtype = DTYPE[spec["dtype"]]
        d.out_dtype = DTYPE[self.out_dtype]
        d.num_rows = int(spec.get("rows", 0))
        signs = spec.get("signs", {})
        d.sign_q = int(signs.get("aq", 1))
        d.sign_k = int(signs.get("ak", 1))
        d.sign_b = int(signs.get("bias", 1))
        d.split_operands = int(bool(split_operands))
        d.segmented = int(spec.get("segments") is not None)
        d.in_tile = int(bool(spec.get("in_tile", False)))
        dr = spec.get("dropout")
        if dr is not None:
            d.dropout_p8 = int(dr["p8"])
            d.dropout_seed = int(dr["seed"]) & 0xFFFFFFFFFFFFFFFF
        mp = spec["map"]
        d.map.kind = MAP_KIND[mp["kind"]]
        d.map.clip = int(mp.get("clip", 0))
        d.map.identity_offset = int(mp.get("offset", 0))
        d.map.num_buckets = int(mp.get("num_buckets", 0))
        d.map.max_distance = int(mp.get("max_distance", 0))
        d.map.bidirectional = int(bool(mp.get("bidirectional", False)))
        d.map.bucket_size = int(mp.get("bucket_size", 0))
        d.map.max_position = int(mp.get("max_position", 0))
        self._rows = None
        if mp["kind"] == "explicit":
            rows = list(mp["rows"])
            self._rows = (ctypes.c_int32 * len(rows))(*rows)
            d.map.explicit_rows = ctypes.cast(self._rows, ctypes.POINTER(ctypes.c_int32))
        H = spec["H"]
        if "aq" in spec["terms"]:
            if spec.get("aq_shared"):
                d.aq_row_stride, d.aq_head_stride = 64, 0
            else:
                d.aq_row_stride, d.aq_head_stride = H * 64, 64
        if "ak" in spec["terms"]:
            d.ak_row_stride, d.ak_head_stride = H * 64, 64
        if "bias" in spec["terms"]:
            d.bias_row_stride, d.bias_head_stride = H, 1
        self.desc = d
        self.shape = _Shape(spec["B"], spec["H"], spec["N"], spec.get("d", 64))

    def sizes(self):
        return plan_sizes(self)


def plan_sizes(problem):
    s = _Sizes()
    _check(library().relpos_plan_sizes(ctypes.byref(problem.desc), ctypes.byref(problem.shape),
                                       ctypes.byref(s)), "relpos_plan_sizes")
    return {name: getattr(s, name) for name, _ in _Sizes._fields_}


def plan_rows(problem, which):
    sz = plan_sizes(problem)
    buf = (ctypes.c_int32 * sz["expanded_rows"])()
    n = _check(library().relpos_plan_rows(ctypes.byref(problem.desc),
                                          ctypes.byref(problem.shape), int(which), buf,
                                          sz["expanded_rows"]), "relpos_plan_rows")
    return list(buf[:n])


def segment_bounds(segments, B, N):
    """The descriptor's segment-bound layout (int32 [B, N, 2]) of per-row
    segment lists: token t of a segment [start, end) carries (start, end),
    a token in no segment (padding) carries the empty (0, 0)."""
    import numpy as np
    out = np.zeros((B, N, 2), dtype=np.int32)
    for b in range(B):
        for start, end in segments[b]:
            if not (0 <= start <= end <= N):
                raise ValueError(f"segment ({start}, {end}) outside [0, {N}]")
            out[b, start:end, 0] = start
            out[b, start:end, 1] = end
    return out


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _tensors(problem, t):
    spec = problem.spec
    need = ["q", "k", "v"] + [n for n in ("aq", "ak", "bias", "u") if n in spec["terms"]]
    if "v" in spec["terms"]:
        need.append("v_bias")
    for name in need:
        x = t[name]
        if not x.is_cuda or not x.is_contiguous():
            raise ValueError(f"tensor {name} must be a contiguous device tensor")
    ts = _Tensors()
    ts.q, ts.k, ts.v = t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr()
    if "aq" in spec["terms"]:
        ts.aq = t["aq"].data_ptr()
    if "ak" in spec["terms"]:
        ts.ak = t["ak"].data_ptr()
    if "bias" in spec["terms"]:
        ts.bias = t["bias"].data_ptr()
    if "u" in spec["terms"]:
        ts.u = t["u"].data_ptr()
    if "v" in spec["terms"]:
        ts.vbias = t["v_bias"].data_ptr()
    if spec.get("segments") is not None:
        seg = t["seg"]
        if not seg.is_cuda or not seg.is_contiguous():
            raise ValueError("tensor seg must be a contiguous device tensor")
        ts.seg = seg.data_ptr()
    return ts


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _empty_bytes(n, device):
    import torch
    return torch.empty(max(int(n), 256), dtype=torch.uint8, device=device)


def _out_torch_dtype(problem):
    import torch
    return torch.float32 if problem.out_dtype == "f32" else torch.bfloat16


def project(problem, t, z=None, ws=None):
    """Retained projections ([RPA] Table 9 "Projection"); returns z (bytes)."""
    sz = plan_sizes(problem)
    dev = t["q"].device
    z = _empty_bytes(sz["z_bytes"], dev) if z is None else z
    ws = _empty_bytes(sz["fwd_ws_bytes"], dev) if ws is None else ws
    _check(library().relpos_project(ctypes.byref(problem.desc), ctypes.byref(problem.shape),
                                    ctypes.byref(_tensors(problem, t)), _ptr(z), z.numel(),
                                    _ptr(ws), ws.numel(), _stream()), "relpos_project")
    return z


def project_noalloc(problem, t, z):
    """relpos_project_noalloc: the projection into the caller's z with the
    library's static scratch as workspace (no workspace argument)."""
    _check(library().relpos_project_noalloc(ctypes.byref(problem.desc),
                                            ctypes.byref(problem.shape),
                                            ctypes.byref(_tensors(problem, t)), _ptr(z),
                                            z.numel(), _stream()), "relpos_project_noalloc")
    return z


def attn_fwd(problem, t, z=None, retain=True, o=None, lse=None, ws=None):
    """Forward.  Returns (O, L, z); with retain the projections are computed
    into z (kept for the backward), else into the workspace."""
    import torch
    sz = plan_sizes(problem)
    dev = t["q"].device
    B, H, N = problem.spec["B"], problem.spec["H"], problem.spec["N"]
    if z is None and retain:
        z = project(problem, t)
    if o is None:
        o = torch.empty((B, H, N, 64), dtype=_out_torch_dtype(problem), device=dev)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if ws is None and z is None:
        ws = _empty_bytes(sz["fwd_ws_bytes_noz"], dev)
    # with retained projections the forward needs no workspace
    _check(library().relpos_attn_fwd(ctypes.byref(problem.desc), ctypes.byref(problem.shape),
                                     ctypes.byref(_tensors(problem, t)), _ptr(z),
                                     0 if z is None else z.numel(), _ptr(o), _ptr(lse),
                                     _ptr(ws), 0 if ws is None else ws.numel(), _stream()),
           "relpos_attn_fwd")
    return o, lse, z


def empty_grads(problem, device):
    import torch
    spec = problem.spec
    B, H, N = spec["B"], spec["H"], spec["N"]
    R = spec.get("rows", 0)
    od = _out_torch_dtype(problem)
    g = {n: torch.empty((B, H, N, 64), dtype=od, device=device) for n in ("dq", "dk", "dv")}
    f32 = torch.float32
    if "aq" in spec["terms"]:
        shape = (R, 64) if spec.get("aq_shared") else (R, H, 64)
        g["daq"] = torch.empty(shape, dtype=f32, device=device)
    if "ak" in spec["terms"]:
        g["dak"] = torch.empty((R, H, 64), dtype=f32, device=device)
    if "bias" in spec["terms"]:
        g["dbias"] = torch.empty((R, H), dtype=f32, device=device)
    if "u" in spec["terms"]:
        g["du"] = torch.empty((H, 64), dtype=f32, device=device)
    if "v" in spec["terms"]:
        g["dv_bias"] = torch.empty((H, 64), dtype=f32, device=device)
    return g


def attn_bwd(problem, t, o, lse, dout, z=None, grads=None, ws=None):
    """Backward; returns a dict of gradients (dq, dk, dv and the table grads)."""
    sz = plan_sizes(problem)
    dev = t["q"].device
    grads = empty_grads(problem, dev) if grads is None else grads
    if ws is None:
        ws = _empty_bytes(sz["bwd_ws_bytes"] if z is not None else sz["bwd_ws_bytes_noz"], dev)
    gr = _Grads()
    gr.dq, gr.dk, gr.dv = (grads[n].data_ptr() for n in ("dq", "dk", "dv"))
    for cname, key in (("daq", "daq"), ("dak", "dak"), ("dbias", "dbias"), ("du", "du"),
                       ("dvbias", "dv_bias")):
        if key in grads:
            setattr(gr, cname, grads[key].data_ptr())
    _check(library().relpos_attn_bwd(ctypes.byref(problem.desc), ctypes.byref(problem.shape),
                                     ctypes.byref(_tensors(problem, t)), _ptr(z),
                                     0 if z is None else z.numel(), _ptr(o), _ptr(lse),
                                     _ptr(dout), ctypes.byref(gr), _ptr(ws), ws.numel(),
                                     _stream()), "relpos_attn_bwd")
    return grads


def set_stage_events(events):
    """Register torch.cuda.Event objects (up to 8) that the following entry
    points on this thread record around their kernels (instrumentation; see
    relpos_set_stage_events in include/relpos.h).  [] clears."""
    import torch
    handles = []
    for ev in events:
        if ev.cuda_event == 0:  # torch creates the HIP event on first record
            ev.record(torch.cuda.current_stream())
        handles.append(ev.cuda_event)
    arr = (ctypes.c_void_p * max(1, len(handles)))(*handles)
    _check(library().relpos_set_stage_events(arr, len(handles)), "relpos_set_stage_events")
