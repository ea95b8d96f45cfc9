"""Benchmark: forward / backward of exact relative-position attention at 8K
tokens for the four mechanisms, on one MI355X.

One step = for each mechanism (Shaw clipped 256, T5 buckets, DeBERTa c2p+p2c,
Transformer-XL causal) at its 8192-token shape: relpos_project +
relpos_attn_fwd (the forward) and relpos_attn_bwd (the backward, retained
projections), inputs resident in HBM.  Prints one JSON line.

Timing follows the pages' appendix "Kernel benchmarks": a 512 MiB device
write flushes the caches before every forward and every backward sample;
each pass and kernel is reported as the median (with min and max) of the
timed steps, measured with HIP events on the launch stream; GPU clocks,
power and temperature are recorded: amd-smi before the GPU is touched, the
GPU's sysfs hwmon files before and after the timed region.

Useful FLOPs follow the credit of "Fast and Exact Relative-Position Attention
via Structure-Aware Kernels" (§5.1 evaluation setup, throughput paragraph):
forward 4 B H N^2 d + 2 B H N R d per projected table (none for T5), backward
twice the forward; the attention part of a causal problem is credited for the
visible pairs only.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--mechs shaw,t5,...]
                    [--no-cpu-baseline]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MI355X_BF16_DENSE_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 FLOP/clk
MI355X_HBM_GBPS = 8000.0
MECHS = ("shaw", "t5", "deberta", "txl")


def credited_flops(spec):
    """(forward, backward) useful FLOPs of one problem."""
    B, H, N, d = spec["B"], spec["H"], spec["N"], spec["d"]
    attn = 4.0 * B * H * N * N * d
    if spec["causal"]:
        attn *= (N + 1) / (2.0 * N)
    nproj = sum(1 for t in ("aq", "ak") if t in spec["terms"])
    R = spec.get("rows", 0)
    fwd = attn + nproj * 2.0 * B * H * N * R * d
    return fwd, 2.0 * fwd


def pair_flops(spec):
    """2 d FLOPs per visible (query, key) pair: one N x N x d product."""
    B, H, N, d = spec["B"], spec["H"], spec["N"], spec["d"]
    f = 2.0 * B * H * N * N * d
    if spec["causal"]:
        f *= (N + 1) / (2.0 * N)
    return f


KERNEL_SOURCE = {"attn_fwd": "fwd_fast.hip", "bwd_q": "bwd_q_fast.hip", "bwd_k": "bwd_k_fast.hip"}


def measured_traffic(kernel, mech):
    """HBM bytes per launch of `kernel` for mechanism `mech` from the committed
    rocprofv3 counter summary (profiles/traffic_*.json), if that summary was
    taken on the current kernel source (same SHA-256); else None."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "relative_position_attention_amd", "csrc")
    h = hashlib.sha256()
    for f in [os.path.join(csrc, KERNEL_SOURCE[kernel])] + sorted(glob.glob(os.path.join(csrc, "*.hpp"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    digest = h.hexdigest()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json"))):
        with open(path) as fh:
            rec = json.load(fh)
        if rec.get("kernel") == f"{kernel} ({mech})" and rec.get("source_sha256") == digest:
            return rec["hbm_bytes_per_launch"]
    return None


def reduction_bytes(spec, delta):
    """HBM bytes the query and the key reduction move by design, per call.

    Each offset-gradient entry dZ~[i, s] in the band rows 1 .. 2D-1 that token
    i reaches is read once by each kernel that consumes it: the finalize
    kernel (dQ += dZ~ A~, only with a table on that side) and the partials
    kernel (the table- and bias-gradient chunk sums); with a table term on
    that side (A^Q; A^K or u) the fp32 dQ / dK partial is read and the dQ / dK
    output (fp32 here) written, else the pass writes the output itself and
    the stage moves no token bytes.  Entries are 2 bytes (bf16, or fp16 for
    the Transformer-XL v term), 4 with a scalar bias.  Table tiles, boundary
    sums and chunk partials are not counted."""
    import numpy as np
    B, H, N, D = spec["B"], spec["H"], spec["N"], delta
    causal, terms = spec["causal"], spec["terms"]
    i = np.arange(N, dtype=np.int64)

    def band(dmin, dmax):
        lo = np.maximum(np.clip(dmin, -D, D) + D, 1)
        hi = np.minimum(np.clip(dmax, -D, D) + D, 2 * D - 1)
        return int(np.maximum(hi - lo + 1, 0).sum())

    q_entries = band(np.zeros(N, np.int64) if causal else i - (N - 1), i)
    k_entries = band(np.zeros(N, np.int64) if causal else -i, (N - 1) - i)
    tok = B * H * N * 64 * (4 + 4)
    q_tok = tok if "aq" in terms else 0
    k_tok = tok if ("ak" in terms or "u" in terms) else 0
    q_reads = ("aq" in terms) + any(t in terms for t in ("aq", "bias", "v"))
    q_size = 4 if "bias" in terms else 2
    k_reads = 2 if "ak" in terms else 0
    return (q_tok + q_reads * B * H * q_entries * q_size,
            k_tok + k_reads * B * H * k_entries * 2)


def measured_stage_traffic(stage):
    """HBM bytes per call of a reduction stage, e.g. "query reduction (txl)",
    from the committed rocprofv3 counter summary
    (profiles/traffic_reductions_n8192.json), if it was taken on the current
    reduction sources; else None."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "relative_position_attention_amd", "csrc")
    h = hashlib.sha256()
    for f in [os.path.join(csrc, "reduce_fast.hip"), os.path.join(csrc, "aux.hip")] + \
            sorted(glob.glob(os.path.join(csrc, "*.hpp"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    path = os.path.join(ROOT, "profiles", "traffic_reductions_n8192.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != h.hexdigest():
        return None
    st = rec.get("stages", {}).get(stage)
    return st["hbm_bytes_per_call"] if st else None


# Algorithmic MFMA work of each attention kernel, in N x N x d products:
# forward QK^T, PV; query pass QK^T, dO V^T, dS K; key pass QK^T, dO V^T,
# P^T dO, dS^T Q (the operand splits for peaked softmax are not counted).
KERNEL_PRODUCTS = {"attn_fwd": 2, "bwd_q": 3, "bwd_k": 4}


def bench_problem(rpa, name, spec, out_dtype):
    """Descriptor of a bench shape.  T5 at tau = 1 takes split operands (P and
    the score gradient as bf16 hi + lo pairs in their MFMA products), which
    its peaked softmax needs to meet the bf16 tolerances; the other
    mechanisms take single bf16 operands."""
    return rpa.Problem(spec, out_dtype=out_dtype, split_operands=name == "t5")


class MechRun:
    """Device inputs and preallocated outputs of one mechanism."""

    def __init__(self, name, torch, rpa, synth):
        self.name = name
        spec, arr = synth.make_bench(name)
        self.spec = spec
        dt = torch.bfloat16
        self.t = {k: torch.from_numpy(v).to(dt).cuda() for k, v in arr.items()}
        del arr
        # outputs in fp32: the configuration the parity tests check
        self.prob = bench_problem(rpa, name, spec, "f32")
        sz = rpa.plan_sizes(self.prob)
        self.sizes = sz
        dev = self.t["q"].device
        B, H, N = spec["B"], spec["H"], spec["N"]
        self.z = torch.empty(max(sz["z_bytes"], 256), dtype=torch.uint8, device=dev)
        self.ws_f = torch.empty(max(sz["fwd_ws_bytes"], 256), dtype=torch.uint8, device=dev)
        self.ws_b = torch.empty(max(sz["bwd_ws_bytes"], 256), dtype=torch.uint8, device=dev)
        self.o = torch.empty((B, H, N, 64), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        self.grads = rpa.empty_grads(self.prob, dev)
        self.fwd_flops, self.bwd_flops = credited_flops(spec)
        self.pair_flops = pair_flops(spec)
        self.red_bytes = reduction_bytes(spec, sz["delta"])

    def project(self, rpa):
        rpa.project(self.prob, self.t, z=self.z, ws=self.ws_f)

    def attn(self, rpa):
        rpa.attn_fwd(self.prob, self.t, z=self.z, o=self.o, lse=self.lse)

    def backward(self, rpa):
        rpa.attn_bwd(self.prob, self.t, self.o, self.lse, self.t["do"], z=self.z,
                     grads=self.grads, ws=self.ws_b)


def peak_memory(run, torch, rpa, out_dtype):
    """Peak device MiB beyond the inputs of a forward and of a backward that
    allocate their own buffers, with O, dQ, dK, dV in `out_dtype` (the
    library itself never allocates; [RPA] §5.2 "Memory footprint" counts the
    device memory allocated beyond the inputs)."""
    prob = bench_problem(rpa, run.name, run.spec, out_dtype)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    o, lse, z = rpa.attn_fwd(prob, run.t, retain=True)
    torch.cuda.synchronize()
    fwd = (torch.cuda.max_memory_allocated() - base) / 2**20
    base2 = torch.cuda.memory_allocated()  # inputs + O + L + retained z
    base2 -= z.numel()  # the retained projections count against the backward
    torch.cuda.reset_peak_memory_stats()
    g = rpa.attn_bwd(prob, run.t, o, lse, run.t["do"], z=z)
    torch.cuda.synchronize()
    bwd = (torch.cuda.max_memory_allocated() - base2) / 2**20
    del o, lse, z, g
    torch.cuda.empty_cache()
    return fwd, bwd


def visible_pairs(spec):
    """Visible (query, key) pairs of one (batch, head) slice, summed over the
    batch rows: N^2 (causal: N (N + 1) / 2) without segments, else the sum
    over segments of len^2 (causal: len (len + 1) / 2)."""
    N = spec["N"]
    segs = spec.get("segments")
    if segs is None:
        return spec["B"] * (N * (N + 1) / 2.0 if spec["causal"] else float(N) * N)
    tot = 0.0
    for row in segs:
        for s0, s1 in row:
            n = s1 - s0
            tot += n * (n + 1) / 2.0 if spec["causal"] else float(n) * n
    return tot


def time_variant(label, spec, arr, torch, rpa, split, steps, warmup, flush, retain=True,
                 out_dtype="f32"):
    """Forward (projection + attention, or attention alone recomputing the
    projections) and backward of one problem variant, median ms over `steps`
    flushed samples, with credited TFLOP/s over its visible pairs and the
    peak MiB beyond the inputs of each pass."""
    dt = torch.bfloat16
    t = {k: torch.from_numpy(v).to(dt).cuda() for k, v in arr.items()}
    if spec.get("segments") is not None:
        t["seg"] = torch.from_numpy(rpa.segment_bounds(spec["segments"], spec["B"],
                                                       spec["N"])).cuda()
    prob = rpa.Problem(spec, out_dtype=out_dtype, split_operands=split)
    B, H, N, d = spec["B"], spec["H"], spec["N"], spec["d"]
    pairs = visible_pairs(spec) * H
    nproj = sum(1 for x in ("aq", "ak") if x in spec["terms"])
    fwd_flops = 4.0 * pairs * d + nproj * 2.0 * B * H * N * spec.get("rows", 0) * d
    sz = rpa.plan_sizes(prob)
    z = torch.empty(max(sz["z_bytes"], 256), dtype=torch.uint8, device="cuda") if retain else None
    ws_f = torch.empty(max(sz["fwd_ws_bytes"] if retain else sz["fwd_ws_bytes_noz"], 256),
                       dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(max(sz["bwd_ws_bytes"] if retain else sz["bwd_ws_bytes_noz"], 256),
                       dtype=torch.uint8, device="cuda")
    o = torch.empty((B, H, N, 64), dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16,
                    device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    grads = rpa.empty_grads(prob, torch.device("cuda"))
    stream = torch.cuda.current_stream()

    def fwd():
        if retain:
            rpa.project(prob, t, z=z, ws=ws_f)
            rpa.attn_fwd(prob, t, z=z, o=o, lse=lse)
        else:
            rpa.attn_fwd(prob, t, z=None, retain=False, o=o, lse=lse, ws=ws_f)

    def bwd():
        rpa.attn_bwd(prob, t, o, lse, t["do"], z=z, grads=grads, ws=ws_b)

    for _ in range(warmup):
        fwd()
        bwd()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for e4 in ev:
        flush.fill_(1.0)
        e4[0].record(stream)
        fwd()
        e4[1].record(stream)
        flush.fill_(2.0)
        e4[2].record(stream)
        bwd()
        e4[3].record(stream)
    torch.cuda.synchronize()

    def med(xs):
        xs = sorted(xs)
        n = len(xs)
        return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])

    f_ms = med([e[0].elapsed_time(e[1]) for e in ev])
    b_ms = med([e[2].elapsed_time(e[3]) for e in ev])
    # peak memory beyond the inputs (the library allocates nothing itself)
    torch.cuda.synchronize()
    del z, ws_f, ws_b, o, lse, grads
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    o2, l2, z2 = rpa.attn_fwd(prob, t, retain=retain)
    torch.cuda.synchronize()
    f_mib = (torch.cuda.max_memory_allocated() - base) / 2**20
    base2 = torch.cuda.memory_allocated() - (z2.numel() if z2 is not None else 0)
    torch.cuda.reset_peak_memory_stats()
    g2 = rpa.attn_bwd(prob, t, o2, l2, t["do"], z=z2)
    torch.cuda.synchronize()
    b_mib = (torch.cuda.max_memory_allocated() - base2) / 2**20
    del o2, l2, z2, g2, t
    torch.cuda.empty_cache()
    return {"variant": label, "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
            "fwd_tflops": round(fwd_flops / f_ms / 1e9, 2),
            "bwd_tflops": round(2 * fwd_flops / b_ms / 1e9, 2),
            "fwd_peak_mib": round(f_mib, 1), "bwd_peak_mib": round(b_mib, 1)}


def extras(torch, rpa, synth, flush, steps=5, warmup=2):
    """The path's other modes at the 8K Shaw shape (B = 2, H = 12, clip 256):
    the same call with retained projections as the reference row, packed
    sequences (four documents of 2048 tokens per row, segment mask),
    padding (row lengths 8192 and 5000), attention dropout (26/256), a map
    whose rows are not contiguous offset intervals (|delta| clipped at 256,
    delta and -delta sharing a row), projections recomputed in both
    passes instead of retained, and bf16 outputs.  Credited FLOPs count
    visible pairs."""
    import copy
    spec0, arr0 = synth.make_bench("shaw")
    out = []
    out.append(time_variant("retained (reference)", spec0, arr0, torch, rpa, False, steps, warmup,
                            flush))
    packed = dict(spec0, segments=[[(k * 2048, (k + 1) * 2048) for k in range(4)]] * 2)
    out.append(time_variant("packed 4 x 2048", packed, arr0, torch, rpa, False, steps, warmup,
                            flush))
    padded = dict(spec0, segments=[[(0, 8192)], [(0, 5000)]])
    out.append(time_variant("padded 8192 / 5000", padded, arr0, torch, rpa, False, steps, warmup,
                            flush))
    drop = dict(spec0, dropout={"p8": 26, "seed": 12345})
    out.append(time_variant("dropout 26/256", drop, arr0, torch, rpa, False, steps, warmup, flush))
    sym = copy.deepcopy(spec0)
    c = spec0["map"]["clip"]
    sym["map"] = {"kind": "explicit", "clip": c, "rows": [abs(x) for x in range(-c, c + 1)]}
    sym["rows"] = c + 1
    arr_sym = dict(arr0, aq=arr0["aq"][: c + 1].copy())
    out.append(time_variant("non-contiguous map |delta|", sym, arr_sym, torch, rpa, False, steps,
                            warmup, flush))
    out.append(time_variant("recomputed projections", spec0, arr0, torch, rpa, False, steps,
                            warmup, flush, retain=False))
    out.append(time_variant("bf16 outputs (O, dQ, dK, dV)", spec0, arr0, torch, rpa, False, steps,
                            warmup, flush, out_dtype="bf16"))
    return {"shape": "shaw B2 H12 N8192 clip 256, bf16", "rows": out,
            "in_tile_rows": in_tile_rows(torch, rpa, synth, flush, steps, warmup)}


def in_tile_rows(torch, rpa, synth, flush, steps=5, warmup=2):
    """In-tile relation products ([RPA] §6, Table 7 row "Projections"): the
    Transformer-XL shapes (identity map: stored projections are quadratic)
    with stored and with in-tile products, time and peak MiB of each."""
    rows = []
    for label, spec_arr in (("txl B1 H8 N8192 causal", synth.make_bench("txl")),
                            ("txl B1 H8 N16384 non-causal", synth.make_config(5))):
        spec, arr = spec_arr
        rows.append(time_variant(label + ", stored", spec, arr, torch, rpa, False, steps, warmup,
                                 flush))
        rows.append(time_variant(label + ", in-tile", dict(spec, in_tile=True), arr, torch, rpa,
                                 False, steps, warmup, flush))
    return rows


def cpu_baseline(mechs):
    """The fp64 oracle on one (batch, head) slice of each mechanism's bench
    shape, timed on the host; credited FLOPs of those slices per second."""
    import oracle
    import synth
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [os.cpu_count() or 1])
    except Exception:
        threads = os.cpu_count() or 1
    total_s, total_flops, rounds = 0.0, 0.0, 0
    problems = {}
    # whole rounds over the mechanisms until at least 10 s of oracle work
    while rounds < 4 and (rounds == 0 or total_s < 10.0):
        for name in mechs:
            if name not in problems:
                kw = dict(synth.BENCH_SHAPES[name])
                problems[name] = synth.make_problem(**dict(kw, B=1, H=1))
            spec, arr = problems[name]
            t0 = time.perf_counter()
            oracle.slice_forward_backward(spec, arr, 0, 0)
            total_s += time.perf_counter() - t0
            f, b = credited_flops(spec)
            total_flops += f + b
        rounds += 1
    return {"value": total_flops / total_s / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{rounds} x one (batch, head) slice of each of {','.join(mechs)} at N=8192, "
                      f"fp64 forward+backward ({total_s:.1f} s)"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def smi_state():
    """Clocks, power and temperature of GPU 0 as amd-smi reports them: the
    numeric fields whose names mention a clock, power or temperature, or the
    tool's error.  Runs amd-smi as a child process, so it is called only
    before this process touches the GPU."""
    import subprocess
    err = "not run"
    for cmd in (["amd-smi", "metric", "-g", "0", "-p", "-c", "-t", "--json"],
                ["rocm-smi", "--showtemp", "--showpower", "--showclocks", "--json"]):
        try:
            res = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
        except (OSError, subprocess.TimeoutExpired) as e:
            err = str(e)
            continue
        if res.returncode != 0:
            err = (res.stderr or res.stdout).strip()[-200:]
            continue
        try:
            data = json.loads(res.stdout)
        except ValueError:
            err = res.stdout.strip()[-200:]
            continue
        out = {}

        def walk(x, path):
            if len(out) >= 40:
                return
            if isinstance(x, dict):
                for k, v in x.items():
                    walk(v, path + [str(k)])
            elif isinstance(x, list):
                for k, v in enumerate(x):
                    walk(v, path + [str(k)])
            else:
                name = "/".join(path)
                low = name.lower()
                if any(t in low for t in ("clk", "clock", "power", "temp")) and x != "N/A":
                    out[name] = x
        walk(data, [])
        return {"tool": cmd[0], "fields": out}
    return {"tool": None, "error": err}


def sysfs_state():
    """Current shader clock, power and temperatures of the first AMD GPU from
    its sysfs hwmon files (plain file reads, so it runs while this process
    holds the GPU)."""
    import glob
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            with open(os.path.join(dev, "vendor")) as fh:
                if fh.read().strip() != "0x1002":
                    continue
        except OSError:
            continue
        for hw in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*"))):
            for f in sorted(glob.glob(os.path.join(hw, "*_input")) +
                            glob.glob(os.path.join(hw, "power*_average"))):
                name = os.path.basename(f)
                try:
                    with open(f) as fh:
                        val = int(fh.read().strip())
                except (OSError, ValueError):
                    continue
                label = name
                lf = f.replace("_input", "_label").replace("_average", "_label")
                if os.path.exists(lf):
                    try:
                        with open(lf) as fh:
                            label = fh.read().strip() + " (" + name + ")"
                    except OSError:
                        pass
                if name.startswith("freq"):
                    out[label] = f"{val / 1e6:.0f} MHz"
                elif name.startswith("power"):
                    out[label] = f"{val / 1e6:.1f} W"
                elif name.startswith("temp"):
                    out[label] = f"{val / 1e3:.1f} C"
        sclk = os.path.join(dev, "pp_dpm_sclk")
        if os.path.exists(sclk):
            try:
                with open(sclk) as fh:
                    cur = [ln.strip() for ln in fh if "*" in ln]
                if cur:
                    out["pp_dpm_sclk"] = cur[0]
            except OSError:
                pass
        if out:
            return out
    return {"error": "no readable AMD GPU hwmon files"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--mechs", default=",".join(MECHS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-memory", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-gpu-state", action="store_true",
                    help="skip amd-smi (e.g. under a profiler that preloads into child programs)")
    ap.add_argument("--in-tile-only", action="store_true",
                    help="time only the in-tile rows (stored vs in-tile products at the "
                         "Transformer-XL shapes) and print them as one JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): this library has no "
              "multi-GPU path; heads and batch slices shard with no communication and "
              "the table gradients need one all-reduce",
              file=sys.stderr)
        sys.exit(2)
    # amd-smi is a child program: read it before this process touches the GPU
    smi = smi_state() if not args.no_gpu_state else {"tool": None, "error": "skipped"}
    import torch

    import relative_position_attention_amd as rpa
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    rpa.library()  # fails loudly if the HIP library is missing
    if args.in_tile_only:
        flush = torch.empty(512 * 2**20 // 4, dtype=torch.float32, device="cuda")
        rows = in_tile_rows(torch, rpa, synth, flush, max(1, args.steps), args.warmup)
        print(json.dumps({"in_tile_rows": rows, "steps": args.steps, "warmup": args.warmup}))
        return
    mechs = [m for m in args.mechs.split(",") if m]
    runs = [MechRun(m, torch, rpa, synth) for m in mechs]
    stream = torch.cuda.current_stream()

    mem = {}
    if not args.no_memory:
        for r in runs:
            mem[r.name] = {od: peak_memory(r, torch, rpa, od) for od in ("f32", "bf16")}

    # Cache flush before every timed forward and backward sample ([RPA]
    # appendix "Kernel benchmarks": an L2 flush before each sample): a write
    # over 512 MiB, twice the 256 MB last-level cache, so that no pass finds
    # its inputs or the projections left in cache by the one before
    flush = torch.empty(512 * 2**20 // 4, dtype=torch.float32, device=runs[0].t["q"].device)

    for _ in range(args.warmup):
        for r in runs:
            flush.fill_(0.0)
            r.project(rpa)
            r.attn(rpa)
            flush.fill_(0.0)
            r.backward(rpa)
    torch.cuda.synchronize()

    def new_events(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    # per (step, mechanism): python-level marks around the projection, and
    # the library's stage events around each kernel (relpos_set_stage_events)
    marks = [[(ev_list_p, new_events(2), new_events(6)) for ev_list_p in
              [new_events(2) for _ in runs]] for _ in range(args.steps)]
    for row in marks:  # create every HIP event before the timed region
        for pe, fe, be in row:
            for e in pe + fe + be:
                e.record(stream)
    state_before = sysfs_state()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for step in range(args.steps):
        for k, r in enumerate(runs):
            pe, fe, be = marks[step][k]
            flush.fill_(float(step))
            pe[0].record(stream)
            r.project(rpa)
            pe[1].record(stream)
            rpa.set_stage_events(fe)
            r.attn(rpa)
            rpa.set_stage_events([])
            flush.fill_(float(step))
            rpa.set_stage_events(be)
            r.backward(rpa)
            rpa.set_stage_events([])
    t_end.record(stream)
    torch.cuda.synchronize()
    state_after = sysfs_state()
    wall_ms = t_start.elapsed_time(t_end) / args.steps

    def stats(fn):
        """Median, min and max over the timed steps."""
        xs = sorted(fn(m) for m in marks)
        n = len(xs)
        med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
        return med, xs[0], xs[-1]

    # time of each step's passes (the flushes between them excluded)
    step_ms = [sum(m[k][0][0].elapsed_time(m[k][1][1]) + m[k][2][0].elapsed_time(m[k][2][5])
                   for k in range(len(runs))) for m in marks]
    ms_per_step = sum(step_ms) / len(step_ms)

    def r4(x):
        return round(x, 4)

    per = {}
    kernels = []  # (median ms, mechanism, kernel)
    reductions = []  # (median ms, mechanism, stage, bytes)
    step_flops = 0.0
    for k, r in enumerate(runs):
        proj = stats(lambda m: m[k][0][0].elapsed_time(m[k][0][1]))
        fwd = stats(lambda m: m[k][0][0].elapsed_time(m[k][1][1]))
        attn = stats(lambda m: m[k][1][0].elapsed_time(m[k][1][1]))
        bwd = stats(lambda m: m[k][2][0].elapsed_time(m[k][2][5]))
        kq = stats(lambda m: m[k][2][1].elapsed_time(m[k][2][2]))
        kk = stats(lambda m: m[k][2][3].elapsed_time(m[k][2][4]))
        rq = stats(lambda m: m[k][2][2].elapsed_time(m[k][2][3]))
        rk = stats(lambda m: m[k][2][4].elapsed_time(m[k][2][5]))
        kernels += [(attn[0], r, "attn_fwd"), (kq[0], r, "bwd_q"), (kk[0], r, "bwd_k")]
        reductions += [(rq[0], r, "query reduction", r.red_bytes[0]),
                       (rk[0], r, "key reduction", r.red_bytes[1])]
        step_flops += r.fwd_flops + r.bwd_flops
        d = {
            "shape": {x: r.spec[x] for x in ("B", "H", "N", "causal")},
            "fwd_ms": r4(fwd[0]), "bwd_ms": r4(bwd[0]),
            "fwd_ms_min_max": [r4(fwd[1]), r4(fwd[2])],
            "bwd_ms_min_max": [r4(bwd[1]), r4(bwd[2])],
            "project_ms": r4(proj[0]), "attn_kernel_ms": r4(attn[0]),
            "fwd_tflops": round(r.fwd_flops / fwd[0] / 1e9, 2),
            "bwd_tflops": round(r.bwd_flops / bwd[0] / 1e9, 2),
            "fwd_pct_peak": round(100 * r.fwd_flops / fwd[0] / 1e9 / MI355X_BF16_DENSE_TFLOPS, 2),
            "bwd_pct_peak": round(100 * r.bwd_flops / bwd[0] / 1e9 / MI355X_BF16_DENSE_TFLOPS, 2),
            "kernel_ms": {"attn_fwd": r4(attn[0]), "bwd_q": r4(kq[0]), "bwd_k": r4(kk[0])},
            "kernel_ms_min_max": {"attn_fwd": [r4(attn[1]), r4(attn[2])],
                                  "bwd_q": [r4(kq[1]), r4(kq[2])],
                                  "bwd_k": [r4(kk[1]), r4(kk[2])]},
            "kernel_mfma_tflops": {
                name: round(KERNEL_PRODUCTS[name] * r.pair_flops / ms[0] / 1e9, 2)
                for name, ms in (("attn_fwd", attn), ("bwd_q", kq), ("bwd_k", kk))},
            "reduce_ms": {"query": r4(rq[0]), "key": r4(rk[0])},
            "reduce_bytes": {"query": r.red_bytes[0], "key": r.red_bytes[1]},
            "reduce_gbps": {"query": round(r.red_bytes[0] / rq[0] / 1e6, 1) if r.red_bytes[0] else None,
                            "key": round(r.red_bytes[1] / rk[0] / 1e6, 1) if r.red_bytes[1] else None},
        }
        if r.name in mem:
            d["fwd_peak_mib"] = round(mem[r.name]["f32"][0], 1)
            d["bwd_peak_mib"] = round(mem[r.name]["f32"][1], 1)
            d["fwd_peak_mib_bf16_out"] = round(mem[r.name]["bf16"][0], 1)
            d["bwd_peak_mib_bf16_out"] = round(mem[r.name]["bf16"][1], 1)
        per[r.name] = d

    # Dominant kernel: the single attention kernel (forward, query pass or key
    # pass) with the longest median launch, timed live with the library's
    # stage events on the launch stream; its algorithmic MFMA FLOPs per launch
    # over that duration.
    dom_ms, dom, dom_kernel = max(kernels, key=lambda x: x[0])
    achieved = KERNEL_PRODUCTS[dom_kernel] * dom.pair_flops / dom_ms / 1e9
    roofline = {"bound": "mfma", "kernel": f"{dom_kernel} ({dom.name})",
                "median_launch_ms": round(dom_ms, 4),
                "flops_per_launch": KERNEL_PRODUCTS[dom_kernel] * dom.pair_flops,
                "achieved": round(achieved, 2), "peak": MI355X_BF16_DENSE_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MI355X_BF16_DENSE_TFLOPS, 4),
                "traffic": measured_traffic(dom_kernel, dom.name)}
    if roofline["traffic"] is not None:
        roofline["traffic_unit"] = ("bytes per launch (rocprofv3 FETCH_SIZE, WRITE_SIZE, "
                                    "copy-calibrated; from the profiles/traffic_*.json summary "
                                    "taken on the current kernel source)")
        roofline["traffic_tb_per_s"] = round(roofline["traffic"] / dom_ms / 1e9, 3)

    # HBM-bound stages: the offset-gradient reductions that produce the
    # table and bias gradients (dR / dBias), timed live with the stage events
    # around them (median over the steps); the slowest one against the HBM peak
    red_ms, red_run, red_stage, red_b = max(reductions, key=lambda x: x[0])
    hbm = {"bound": "hbm", "stage": f"{red_stage} ({red_run.name})",
           "kernels": "finalize + partials + fold (+ bias / v / u sums)",
           "median_ms": round(red_ms, 4), "bytes_per_call": red_b,
           "achieved": round(red_b / red_ms / 1e6, 1), "peak": MI355X_HBM_GBPS,
           "unit": "GB/s", "frac": round(red_b / red_ms / 1e6 / MI355X_HBM_GBPS, 4),
           "traffic": measured_stage_traffic(f"{red_stage} ({red_run.name})")}
    if hbm["traffic"] is not None:
        hbm["traffic_unit"] = ("bytes per call (rocprofv3 FETCH_SIZE, WRITE_SIZE, copy-calibrated; "
                               "from profiles/traffic_reductions_n8192.json, taken on the current "
                               "reduction sources)")
        hbm["traffic_gbps"] = round(hbm["traffic"] / red_ms / 1e6, 1)

    value = step_flops / ms_per_step / 1e9
    out = {
        "metric": "fwd/bwd ms + TFLOP/s (% bf16 MFMA peak) per mechanism at N=8K; peak MiB",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "relpos attention fwd+bwd at N=8192: " + ", ".join(
            f"{r.name} B{r.spec['B']} H{r.spec['H']}{' causal' if r.spec['causal'] else ''}"
            for r in runs), "mechanisms": mechs, "d": 64},
        "timing": {"per_pass": "median (min, max) over the timed steps, HIP events on the "
                               "launch stream", "flush": "512 MiB device write before every "
                               "forward and every backward sample",
                   "ms_per_step": "mean over the steps of the passes' own time (flushes "
                                  "excluded)", "wall_ms_per_step_with_flushes": round(wall_ms, 4)},
        "gpu_state": {"amd_smi_at_start": smi, "sysfs_before_timed": state_before,
                      "sysfs_after_timed": state_after},
        "mechanisms": per,
        "roofline": roofline,
        "hbm": hbm,
    }
    if not args.no_extras:
        del runs
        torch.cuda.empty_cache()
        out["extras"] = extras(torch, rpa, synth, flush)
        runs = None
    if not args.no_cpu_baseline:
        del runs
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(mechs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
