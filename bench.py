"""Benchmark of the MXFP8 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the hot path over one batch of synthetic input held
in HBM.  The default workload is the headline one: the bf16 -> MXFP8 dim0 +
dim1 cast of a 16384 x 16384 matrix with heavy-tailed rows, with both scale
sets written in the 128x4 blocked layout by the same launch.  Other workloads
(for profiling):
  square16384_3launch  the same result from three launches: the cast with
             plain scales, then mx_scales_to_blocked on each scale set;
  moe16640   cast of (16640, 5120) activations writing the row scales in the
             M-grouped blocked layout itself (4 groups along M, offsets on
             the device);
  moe16640_2launch  the same from the plain cast + the M-grouped layout;
  moe16640_both  the same cast writing the column scales K-grouped as well
             (the weight-gradient GEMM's layout), in one launch;
  moe16640_both_2launch  the same from the M-grouped cast + the K-grouped
             layout of its plain column scales;
  kgroups    K-grouped layouts of (5120, 512), (8192, 4096), (2048, 4096)
             scale tensors (4 groups along K), the three launches timed as
             one step;
  experts16  dim1 cast of (16, 8192, 5120) expert weights with each
             expert's scales written in the blocked layout by the same launch;
  experts16_2launch  the same from the plain 3D cast + mx_scales_to_blocked;
  rowwise16384  the row-wise fp8 cast (one bf16 scale per row) of the same
             16384 x 16384 input;
  tensorwise16384  the tensor-wise fp8 cast (one bf16 scale, two-stage amax)
             of the same input;
  gemm16640  the MX-scaled GEMM that consumes the casts: M = 16640, N =
             8192, K = 5120, bf16 out (TFLOP/s against the MFMA roofline);
  ggemm16640 the same grouped along M (4 groups, per-group weights);
  kggemm16640  the weight-gradient GEMM grouped along K: 4 outputs of
             (8192, 5120), K = the 16640 tokens split in 4 groups;
  cast_blocked, cast_grouped, cast_plain  the blocked-scale cast, the cast
             with both scale sets grouped (4 equal groups of rows), or the
             plain-scale cast, at any --rows --cols (default 16384 x 16384;
             N(0,1) input drawn on the GPU);
  copy       a plain device-to-device copy of 1 GiB (counter calibration).

Each workload's calls are validated once through the Python binding; the
timed loop then calls the same C-ABI entry points with their arguments
marshalled in advance, so the host keeps ahead of the GPU.

The default run also measures, before the headline's warm-up, the other
workloads of the hot path (the `configs` object: the plain-scale call
mx_cast_dim0_dim1 at 16384 x 16384, the MoE casts with M-grouped and with
both scale sets grouped, the three K-grouped layouts and the 3D expert cast;
each its back-to-back mean over 100 launches, after at least 20 steps and
25 ms of warm-up, and its cold-cache median over 20; --no-extras skips
them).

Prints exactly one JSON line on stdout; progress goes to stderr.  The
`roofline` object is for the dominant kernel (the cast): algorithmic bytes per
launch divided by its average duration from HIP events recorded on the stream
it runs on.  `cpu_baseline` times the CPU oracle on the same input (rank 0,
one GPU) and checks every output byte against the GPU's.  `cold_cache` times
further steps one by one, each after a 512 MiB write and a 512 MiB read of
other buffers, which evict the 256 MB Infinity Cache and the L2 (median;
--cold-launches 0 skips it): the timed loop itself runs steps back to back,
so a step may find part of the previous step's data still cached.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fp8_precision_quantization_amd as mx  # noqa: E402
from fp8_precision_quantization_amd import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_FP8_PEAK_TFLOPS = 5000.0   # dense fp8 MFMA, MI355X
METRIC = "achieved HBM GB/s (% of MI355X peak) for bf16→MXFP8 dim0+dim1 cast"
CAST_SOURCES = ["fp8_precision_quantization_amd/csrc/mx_cast.hip",
                "fp8_precision_quantization_amd/csrc/mx_device.h"]
COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "cast_square16384_counters.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pad(v, m):
    return -(-v // m) * m


def to_dev_bf16(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def cast_bytes(rows, cols):
    """Algorithmic bytes of the dim0+dim1 cast: read 2 B, write 1 + 1 B per
    element, plus one e8m0 byte per 32 elements in each direction."""
    return rows * cols * 2 + 2 * rows * cols + 2 * (rows * cols // 32)


def blocked_bytes(rows, cols, batch=1):
    return batch * (rows * cols + pad(rows, 128) * pad(cols, 4))


def code_of(text):
    """C/C++ source with its comments removed and each line's trailing
    blanks dropped, empty lines skipped: what the compiler sees, so that a
    change to a comment leaves the digest as it was."""
    out, i, n = [], 0, len(text)
    while i < n:
        ch = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif ch in "\"'":
            j = i + 1
            while j < n and text[j] != ch:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(ch)
            i += 1
    lines = ("".join(out)).split("\n")
    return "\n".join(l.rstrip() for l in lines if l.strip())


def sources_digest(read=None):
    """First 16 hex digits of sha256 over the code (comments stripped) of the
    cast kernel's sources, in order; read(path) -> text, default the files."""
    h = hashlib.sha256()
    for p in CAST_SOURCES:
        if read is None:
            with open(os.path.join(ROOT, p), encoding="utf-8") as f:
                text = f.read()
        else:
            text = read(p)
        h.update(code_of(text).encode("utf-8"))
    return h.hexdigest()[:16]


def counter_traffic():
    """HBM bytes per cast launch from the committed counter summary, or None
    when it is missing or was taken on different kernel sources."""
    try:
        text = open(COUNTER_SUMMARY).read()
    except OSError:
        return None
    m_sha = re.search(r"kernel_sources_sha256:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != sources_digest():
        return None
    return float(m_b.group(1))


FLUSH_BYTES = 512 << 20


def cold_cache(step, step_bytes, launches, scale, unit, peak, dev):
    """Each step preceded, outside its timing, by a write of one 512 MiB
    buffer and a read of another: the write evicts the 256 MB Infinity Cache
    and the L2, the read then evicts the write's dirty lines (their
    write-back happens before the step) and leaves only clean, unrelated
    lines.  One event pair per step on the current stream; the median."""
    log("cold-cache timing: %d steps, each after a %d MiB write and a %d MiB read"
        % (launches, FLUSH_BYTES >> 20, FLUSH_BYTES >> 20))
    wbuf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    rbuf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    sink = torch.empty(launches, dtype=torch.int64, device=dev)
    torch.cuda.synchronize(dev)
    for i, (e0, e1) in enumerate(pairs):
        wbuf.fill_(i)
        torch.sum(rbuf, dim=0, out=sink[i])
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize(dev)
    us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in pairs)[launches // 2]
    achieved = step_bytes / (us * 1e-6) / scale
    del wbuf, rbuf
    return {"flush_bytes": 2 * FLUSH_BYTES, "steps": launches, "step_us_median": round(us, 2),
            "achieved": round(achieved, 1), "unit": unit, "frac": round(achieved / peak, 4)}


class Timer:
    """Kernel time from HIP events on torch's current stream (the stream the
    library launches on).

    whole_step=True: the step is the timed operation alone, so one event pair
    around the whole timed region gives its average duration (region / steps)
    and the launches run back to back.  Otherwise a pair of events brackets
    each timed launch inside the step (a timed event record between two
    kernels costs a few microseconds, so this is kept to steps with several
    launches, where one of them must be isolated).  Events are created before
    the timed steps so that the loop stays cheap on the host."""

    def __init__(self, whole_step=False):
        self.whole_step = whole_step
        self.events = []
        self.used = 0
        self.region = None

    def reserve(self, n):
        if self.whole_step:
            return
        while len(self.events) < n:
            self.events.append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
        self.used = 0

    def __enter__(self):
        if self.whole_step:
            return self
        if self.used == len(self.events):
            self.reserve(self.used + 64)
            self.used = len(self.events) - 64
        self.events[self.used][0].record()
        return self

    def __exit__(self, *exc):
        if self.whole_step:
            return
        self.events[self.used][1].record()
        self.used += 1

    def clear(self):
        self.used = 0

    def start_region(self):
        self.region = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        self.region[0].record()

    def end_region(self, steps):
        self.region[1].record()
        self.steps = steps

    def mean_ms(self):
        if self.whole_step:
            return self.region[0].elapsed_time(self.region[1]) / self.steps
        pairs = self.events[:self.used]
        return sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)


def c_call(name, *args, stream_at_call=False):
    """A C-ABI entry point with its arguments marshalled once (tensors become
    device pointers, plus torch's current stream), for the timed loops; the
    Python binding of the same name validates the same call during set-up.
    stream_at_call: look torch's current stream up at each call instead (so
    that the call can be captured into a graph, whose capture runs on a
    stream of its own).  The returned call keeps its tensors alive: a tensor
    known to it only by its address would go back to torch's allocator once
    the set-up returns, and the next allocation (the cold-cache buffers, say)
    could take it over."""
    f = getattr(mx.lib(), name)
    conv = [ctypes.c_void_p(a.data_ptr()) if isinstance(a, torch.Tensor) else a for a in args]
    keep = [a for a in args if isinstance(a, torch.Tensor)]
    if stream_at_call:
        def call():
            rc = f(*conv, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise mx.MxError(rc, name)
    else:
        conv.append(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))

        def call():
            rc = f(*conv)
            if rc != 0:
                raise mx.MxError(rc, name)
    call.tensors = keep
    return call


def oracle_leg(nbytes, sample, run, compare):
    """The CPU oracle timed on the host's cores: run() computes the oracle's
    outputs (timed), compare(result) returns {name: mismatched bytes} against
    the GPU's outputs (not timed)."""
    import oracle
    t0 = time.perf_counter()
    res = run(oracle)
    dt = time.perf_counter() - t0
    bad = compare(res)
    ok = not any(bad.values())
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": "%s, %.1f s wall" % (sample, dt), "matches_gpu": bool(ok),
            **({} if ok else {"mismatched_bytes": bad})}


def moe_single_thread(bits, ends, sample_rows=1024):
    """One thread of the oracle on the first 1024 rows of the MoE input (the
    same cast and M-grouped layout, the groups cut at the sample's end)."""
    import oracle
    cores = oracle.num_threads()
    part = np.ascontiguousarray(bits[:sample_rows])
    e = np.minimum(ends, sample_rows).astype(np.int32)
    r, c = part.shape
    oracle.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        _, s0 = oracle.cast_dim0(part)
        oracle.cast_dim1(part)
        g, _ = oracle.to_blocked_grouped(s0, e, 0)
        dt = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(cores)
    nbytes = r * c * 4 + r * (c // 32) + g.size
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s",
            "sample": "the first %d rows, one thread, %.2f s" % (sample_rows, dt)}


def n_bad(gpu, ref):
    g = gpu.cpu().numpy().reshape(-1)
    r = np.asarray(ref).reshape(-1)
    return int(np.count_nonzero(g != r)) if g.shape == r.shape else -1


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
_SQUARE = {}


def square_input(dev, n=16384):
    """The heavy-tailed (n, n) input (host bits and device copy), drawn once
    per process and shared by the workloads that cast it."""
    if n not in _SQUARE:
        log("generating %dx%d heavy-tailed bf16 input" % (n, n))
        bits = workloads.heavy_tailed_rows(n, n, seed=2)
        _SQUARE[n] = (bits, to_dev_bf16(bits, dev))
    return _SQUARE[n]


def setup_square(dev, n=16384, fused=True):
    bits, x = square_input(dev, n)
    q0 = torch.empty((n, n), dtype=torch.uint8, device=dev)
    q1 = torch.empty((n, n), dtype=torch.uint8, device=dev)
    b0 = torch.empty((pad(n, 128), pad(n // 32, 4)), dtype=torch.uint8, device=dev)
    b1 = torch.empty_like(b0)
    timer = Timer(whole_step=fused)
    if fused:
        mx.mx_cast_dim0_dim1_blocked(x, out=(q0, b0, q1, b1), raw=True)
        cast = c_call("mx_cast_dim0_dim1_blocked", x, n, n, q0, b0, q1, b1)

        def step():
            with timer:
                cast()

        # one launch reads X and writes both codes and both blocked scale sets
        kern_bytes = 4 * n * n + 2 * pad(n, 128) * pad(n // 32, 4)
        step_bytes = kern_bytes
        kern_name = "cast dim0+dim1, blocked scales"
    else:
        s0 = torch.empty((n, n // 32), dtype=torch.uint8, device=dev)
        s1 = torch.empty((n, n // 32), dtype=torch.uint8, device=dev)

        mx.mx_cast_dim0_dim1(x, out=(q0, s0, q1, s1), raw=True)
        mx.mx_scales_to_blocked(s0, out=b0, raw=True)
        cast = c_call("mx_cast_dim0_dim1", x, n, n, q0, s0, q1, s1)
        lay0 = c_call("mx_scales_to_blocked", s0, 1, n, n // 32, b0)
        lay1 = c_call("mx_scales_to_blocked", s1, 1, n, n // 32, b1)

        def step():
            with timer:
                cast()
            lay0()
            lay1()

        kern_bytes = cast_bytes(n, n)
        step_bytes = cast_bytes(n, n) + 2 * blocked_bytes(n, n // 32)
        kern_name = "cast dim0+dim1"

    def cpu_baseline():
        # the oracle on the whole input (a few seconds on the host's cores)
        import oracle
        t0 = time.perf_counter()
        r_q0, r_s0 = oracle.cast_dim0(bits)
        r_q1, r_s1 = oracle.cast_dim1(bits)
        r_b0 = oracle.to_blocked(r_s0)
        r_b1 = oracle.to_blocked(r_s1)
        dt = time.perf_counter() - t0
        nbytes = 4 * n * n + r_b0.size + r_b1.size
        bad = {name: int(np.count_nonzero(g != r)) for name, g, r in (
            ("q_row", q0.cpu().numpy(), r_q0), ("q_col", q1.cpu().numpy(), r_q1),
            ("s_row_blocked", b0.cpu().numpy().reshape(-1), r_b0),
            ("s_col_blocked", b1.cpu().numpy().reshape(-1), r_b1))}
        ok = not any(bad.values())
        cores = oracle.num_threads()
        # one thread on the 1024 x 1024 workload (with special tiles)
        small = workloads.square_with_special_tiles()
        oracle.set_num_threads(1)
        t1 = time.perf_counter()
        s_q0, s_s0 = oracle.cast_dim0(small)
        s_q1, s_s1 = oracle.cast_dim1(small)
        s_b = oracle.to_blocked(s_s0).size + oracle.to_blocked(s_s1).size
        dt1 = time.perf_counter() - t1
        oracle.set_num_threads(cores)
        return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": cores,
                "kind": "oracle",
                "sample": "the whole %dx%d input (dim0+dim1 cast, both scale sets in the blocked "
                          "layout), %.1f s wall" % (n, n, dt),
                "matches_gpu": bool(ok),
                **({} if ok else {"mismatched_bytes": bad}),
                "single_thread": {"value": round((4 * 1024 * 1024 + s_b) / dt1 / 1e9, 3), "unit": "GB/s",
                                  "sample": "1024x1024 with special tiles, one thread, %.2f s" % dt1}}

    config = {"workload": "mx_cast_dim0_dim1%s %dx%d bf16 (heavy-tailed rows), both scale sets "
                          "in the 128x4 blocked layout%s"
                          % ("_blocked" if fused else "", n, n,
                             "" if fused else " by two mx_scales_to_blocked launches"),
              "rows": n, "cols": n, "block": 32, "elem": "e4m3", "scale": "e8m0"}
    return step, step_bytes, timer, kern_bytes, kern_name, cpu_baseline, config


def setup_square_plain(dev, n=16384):
    """mx_cast_dim0_dim1 alone: both codes and both scale sets in the plain
    row-major layout, one call per step (at this shape the call enqueues the
    blocked-scale cast and the in-place conversion of its scales to rows)."""
    bits, x = square_input(dev, n)
    q0 = torch.empty((n, n), dtype=torch.uint8, device=dev)
    q1 = torch.empty((n, n), dtype=torch.uint8, device=dev)
    s0 = torch.empty((n, n // 32), dtype=torch.uint8, device=dev)
    s1 = torch.empty((n, n // 32), dtype=torch.uint8, device=dev)
    mx.mx_cast_dim0_dim1(x, out=(q0, s0, q1, s1), raw=True)
    cast = c_call("mx_cast_dim0_dim1", x, n, n, q0, s0, q1, s1)
    timer = Timer(whole_step=True)

    def step():
        with timer:
            cast()

    nb = cast_bytes(n, n)

    def cpu_baseline():
        def run(o):
            return o.cast_dim0(bits) + o.cast_dim1(bits)

        def compare(r):
            return {"q_row": n_bad(q0, r[0]), "s_row": n_bad(s0, r[1]), "q_col": n_bad(q1, r[2]),
                    "s_col": n_bad(s1, r[3])}
        return oracle_leg(nb, "the whole %dx%d input (dim0+dim1 cast, plain scales)" % (n, n), run, compare)

    config = {"workload": "mx_cast_dim0_dim1 %dx%d bf16 (heavy-tailed rows), plain row-major scales" % (n, n),
              "rows": n, "cols": n, "block": 32, "elem": "e4m3", "scale": "e8m0"}
    return step, nb, timer, nb, "cast dim0+dim1, plain scales (one call)", cpu_baseline, config


def setup_square_3launch(dev):
    return setup_square(dev, fused=False)


def setup_moe(dev, fused=True):
    bits, ends = workloads.moe_activations()
    rows, cols = bits.shape
    x = to_dev_bf16(bits, dev)
    offs = torch.from_numpy(ends).to(dev)
    q0 = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    q1 = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
    s1 = torch.empty((cols, rows // 32), dtype=torch.uint8, device=dev)
    g = len(ends)
    out = torch.empty((rows + 128 * g, pad(cols // 32, 4)), dtype=torch.uint8, device=dev)
    starts = torch.empty(g + 1, dtype=torch.int64, device=dev)
    timer = Timer(whole_step=fused)
    if fused:
        mx.mx_cast_dim0_dim1_mgrouped(x, offs, out=(q0, out, q1, s1), out_group_starts=starts, raw=True)
        cast = c_call("mx_cast_dim0_dim1_mgrouped", x, rows, cols, offs, g, q0, out, starts, q1, s1)

        def step():
            with timer:
                cast()

        # read X; write both code matrices, the grouped row scales, the plain
        # column scales and the starts
        kb = rows * cols * 4 + out.numel() + s1.numel() + 8 * (g + 1)
        nb = kb
        name = "cast dim0+dim1, M-grouped row scales"
        label = "mx_cast_dim0_dim1_mgrouped %dx%d bf16, M-grouped blocked row scales (%d groups)"
    else:
        s0 = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
        mx.mx_cast_dim0_dim1(x, out=(q0, s0, q1, s1), raw=True)
        mx.mx_scales_to_blocked_grouped(s0, offs, 0, out=out, out_group_starts=starts, raw=True)
        cast = c_call("mx_cast_dim0_dim1", x, rows, cols, q0, s0, q1, s1)
        lay = c_call("mx_scales_to_blocked_grouped", s0, rows, cols // 32, offs, g, 0, out, starts)

        def step():
            with timer:
                cast()
            lay()

        kb = cast_bytes(rows, cols)
        nb = cast_bytes(rows, cols) + rows * (cols // 32) + out.numel()
        name = "cast dim0+dim1"
        label = "mx_cast_dim0_dim1 %dx%d bf16 + M-grouped blocked layout (%d groups)"

    def cpu_baseline():
        def run(o):
            r_q0, r_s0 = o.cast_dim0(bits)
            r_q1, r_s1 = o.cast_dim1(bits)
            return r_q0, r_q1, r_s1, o.to_blocked_grouped(r_s0, ends, 0)

        def compare(r):
            r_q0, r_q1, r_s1, (r_g, r_st) = r
            return {"q_row": n_bad(q0, r_q0), "q_col": n_bad(q1, r_q1), "s_col": n_bad(s1, r_s1),
                    "s_row_mgrouped": n_bad(out, r_g), "starts": n_bad(starts, r_st)}
        leg = oracle_leg(nb, "the whole %dx%d input (dim0+dim1 cast, M-grouped blocked row scales)"
                         % (rows, cols), run, compare)
        leg["single_thread"] = moe_single_thread(bits, ends)
        return leg

    config = {"workload": label % (rows, cols, g), "rows": rows, "cols": cols, "groups": g}
    return step, nb, timer, kb, name, cpu_baseline, config


def setup_moe_2launch(dev):
    return setup_moe(dev, fused=False)


def setup_moe_both(dev, fused=True):
    """The MoE activations with both scale sets grouped: M-grouped row scales
    (forward GEMM) and K-grouped column scales (weight-gradient GEMM)."""
    bits, ends = workloads.moe_activations()
    rows, cols = bits.shape
    x = to_dev_bf16(bits, dev)
    offs = torch.from_numpy(ends).to(dev)
    g = len(ends)
    u8 = dict(dtype=torch.uint8, device=dev)
    q0 = torch.empty((rows, cols), **u8)
    q1 = torch.empty((cols, rows), **u8)
    s0g = torch.empty((rows + 128 * g, pad(cols // 32, 4)), **u8)
    s1g = torch.empty((pad(cols, 128), pad(rows // 32, 4) + 4 * g), **u8)
    rs = torch.empty(g + 1, dtype=torch.int64, device=dev)
    cs = torch.empty(g + 1, dtype=torch.int64, device=dev)
    timer = Timer(whole_step=fused)
    if fused:
        mx.mx_cast_dim0_dim1_grouped_blocked(x, offs, out=(q0, s0g, q1, s1g), out_row_starts=rs,
                                             out_col_starts=cs, raw=True)
        cast = c_call("mx_cast_dim0_dim1_grouped_blocked", x, rows, cols, offs, g, q0, s0g, rs, q1, s1g, cs)

        def step():
            with timer:
                cast()

        kb = rows * cols * 4 + s0g.numel() + s1g.numel() + 16 * (g + 1)
        nb = kb
        name = "cast dim0+dim1, M- and K-grouped scales"
        label = ("mx_cast_dim0_dim1_grouped_blocked %dx%d bf16, M-grouped row scales and K-grouped column "
                 "scales (%d groups)")
    else:
        s1 = torch.empty((cols, rows // 32), **u8)
        kends = torch.from_numpy(ends // 32).to(dev)
        mx.mx_cast_dim0_dim1_mgrouped(x, offs, out=(q0, s0g, q1, s1), out_group_starts=rs, raw=True)
        mx.mx_scales_to_blocked_grouped(s1, kends, 1, out=s1g, out_group_starts=cs, raw=True)
        cast = c_call("mx_cast_dim0_dim1_mgrouped", x, rows, cols, offs, g, q0, s0g, rs, q1, s1)
        lay = c_call("mx_scales_to_blocked_grouped", s1, cols, rows // 32, kends, g, 1, s1g, cs)

        def step():
            with timer:
                cast()
            lay()

        kb = rows * cols * 4 + s0g.numel() + s1.numel() + 8 * (g + 1)
        nb = kb + s1.numel() + s1g.numel()
        name = "cast dim0+dim1, M-grouped row scales"
        label = "mx_cast_dim0_dim1_mgrouped %dx%d bf16 + K-grouped layout of the column scales (%d groups)"

    def cpu_baseline():
        def run(o):
            r_q0, r_s0 = o.cast_dim0(bits)
            r_q1, r_s1 = o.cast_dim1(bits)
            return r_q0, r_q1, o.to_blocked_grouped(r_s0, ends, 0), o.to_blocked_grouped(r_s1, ends // 32, 1)

        def compare(r):
            r_q0, r_q1, (r_g0, r_rs), (r_g1, r_cs) = r
            return {"q_row": n_bad(q0, r_q0), "q_col": n_bad(q1, r_q1), "s_row_mgrouped": n_bad(s0g, r_g0),
                    "s_col_kgrouped": n_bad(s1g, r_g1), "row_starts": n_bad(rs, r_rs),
                    "col_starts": n_bad(cs, r_cs)}
        return oracle_leg(nb, "the whole %dx%d input (dim0+dim1 cast, M-grouped row and K-grouped column "
                          "scales)" % (rows, cols), run, compare)

    config = {"workload": label % (rows, cols, g), "rows": rows, "cols": cols, "groups": g}
    return step, nb, timer, kb, name, cpu_baseline, config


def setup_moe_both_2launch(dev):
    return setup_moe_both(dev, fused=False)


def setup_kgroups(dev):
    items = []
    for shape in workloads.K_GROUP_SHAPES:
        s, ends = workloads.k_group_scales(shape)
        r, c = shape
        g = len(ends)
        items.append((torch.from_numpy(s).to(dev), torch.from_numpy(ends).to(dev),
                      torch.empty((pad(r, 128), pad(c, 4) + 4 * g), dtype=torch.uint8, device=dev),
                      torch.empty(g + 1, dtype=torch.int64, device=dev)))
    # the step is the three layouts back to back, timed as a whole (events
    # between launches of a few microseconds each would weigh on them)
    timer = Timer(whole_step=True)

    calls = []
    for s, offs, out, starts in items:
        mx.mx_scales_to_blocked_grouped(s, offs, 1, out=out, out_group_starts=starts, raw=True)
        calls.append(c_call("mx_scales_to_blocked_grouped", s, s.shape[0], s.shape[1], offs, offs.numel(), 1,
                            out, starts, stream_at_call=True))

    def step():
        with timer:
            for call in calls:
                call()

    nb = sum(s.numel() + out.numel() for s, _, out, _ in items)

    def cpu_baseline():
        host = [(s.cpu().numpy(), offs.cpu().numpy()) for s, offs, _, _ in items]

        def run(o):
            return [o.to_blocked_grouped(s, e, 1) for s, e in host]

        def compare(r):
            bad = {}
            for (_, _, out, starts), (r_out, r_st), shape in zip(items, r, workloads.K_GROUP_SHAPES):
                bad["%dx%d" % shape] = n_bad(out, r_out) + n_bad(starts, r_st)
            return bad
        return oracle_leg(nb, "all three scale tensors", run, compare)

    config = {"workload": "K-grouped blocked layout of e8m0 scales %s, 4 groups each"
                          % (list(workloads.K_GROUP_SHAPES),),
              # the three launches last ~20 us together, less than the host
              # takes to issue them: measured as replays of a captured graph
              "graph_steps": 20,
              "metric": "achieved HBM GB/s (% of MI355X peak) for the K-grouped 128x4 blocked layout of e8m0 "
                        "scales",
              "dtype": "u8"}
    return step, nb, timer, nb, "K-grouped layouts (three launches)", cpu_baseline, config


def device_expert_weights(experts, n, k, dev, seed=5):
    """(experts, n, k) bf16 drawn on the device with the expert-weight recipe
    (N(0, 0.02^2), a seeded 1% of the elements times 100): the same
    distribution as workloads.expert_weight, other values (torch's device
    generator), in a fraction of the host's time."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    w = torch.empty((experts, n, k), dtype=torch.bfloat16, device=dev)
    for e in range(experts):
        a = torch.randn((n, k), generator=g, device=dev) * 0.02
        a = torch.where(torch.rand((n, k), generator=g, device=dev) < 0.01, a * 100.0, a)
        w[e] = a.to(torch.bfloat16)
    return w


def setup_experts(dev, experts=16, n=8192, k=5120, fused=True, device_inputs=False):
    if device_inputs:
        w = device_expert_weights(experts, n, k, dev)
    else:
        log("generating (%d, %d, %d) expert weights" % (experts, n, k))
        w = torch.empty((experts, n, k), dtype=torch.bfloat16, device=dev)
        for e in range(experts):
            w[e] = to_dev_bf16(workloads.expert_weight(e, n, k), dev)
    q = torch.empty((experts, k, n), dtype=torch.uint8, device=dev)
    out = torch.empty((experts, pad(k, 128), pad(n // 32, 4)), dtype=torch.uint8, device=dev)
    timer = Timer(whole_step=fused)
    if fused:
        mx.mx_cast_dim1_3d_blocked(w, out=(q, out), raw=True)
        cast = c_call("mx_cast_dim1_3d_blocked", w, experts, n, k, q, out)

        def step():
            with timer:
                cast()

        cb = experts * n * k * 3 + out.numel()
        nb = cb
        name = "cast dim1 3D, blocked scales"
    else:
        s = torch.empty((experts, k, n // 32), dtype=torch.uint8, device=dev)

        mx.mx_cast_dim1_3d(w, out=(q, s), raw=True)
        mx.mx_scales_to_blocked(s, out=out, raw=True)
        cast = c_call("mx_cast_dim1_3d", w, experts, n, k, q, s)
        lay = c_call("mx_scales_to_blocked", s, experts, k, n // 32, out)

        def step():
            with timer:
                cast()
            lay()

        cb = experts * n * k * 3 + experts * n * k // 32
        nb = cb + blocked_bytes(k, n // 32, experts)
        name = "cast dim1 3D"

    def cpu_baseline(sample=2):
        # a bounded sample: the first two experts (of the same workload)
        host = [workloads.expert_weight(e, n, k) for e in range(sample)]

        def run(o):
            outs = []
            for we in host:
                r_q, r_s = o.cast_dim1(we)
                outs.append((r_q, o.to_blocked(r_s)))
            return outs

        def compare(r):
            return {"expert %d" % e: n_bad(q[e], r_q) + n_bad(out[e], r_b) for e, (r_q, r_b) in enumerate(r)}
        per_expert = nb // experts
        return oracle_leg(per_expert * sample, "the first %d of the %d experts (dim1 cast and blocked scales of "
                          "each (%d, %d) expert)" % (sample, experts, n, k), run, compare)
    if device_inputs:
        cpu_baseline = None
    config = {"workload": "%s (%d, %d, %d) bf16 + per-expert blocked scale layout%s%s"
                          % ("mx_cast_dim1_3d_blocked" if fused else "mx_cast_dim1_3d", experts, n, k,
                             "" if fused else " by mx_scales_to_blocked",
                             " (weights drawn on the device)" if device_inputs else ""),
              "experts": experts, "n": n, "k": k,
              "metric": "achieved HBM GB/s (% of MI355X peak) for the bf16->MXFP8 dim1 cast of 3D expert weights"}
    return step, nb, timer, cb, name, cpu_baseline, config


def setup_experts_2launch(dev):
    return setup_experts(dev, fused=False)


def setup_rowwise(dev, n=16384):
    bits, x = square_input(dev, n)
    q = torch.empty((n, n), dtype=torch.uint8, device=dev)
    s = torch.empty(n, dtype=torch.int16, device=dev)
    timer = Timer(whole_step=True)

    mx.mx_quantize_fp8_rowwise(x, out=(q, s), raw=True)
    cast = c_call("mx_quantize_fp8_rowwise", x, n, n, q, s)

    def step():
        with timer:
            cast()

    nb = 3 * n * n + 2 * n   # read bf16, write e4m3fn, write one bf16 scale per row

    def cpu_baseline():
        # the oracle on the whole input (a few seconds on the host's cores)
        import oracle
        t0 = time.perf_counter()
        r_q, r_s = oracle.quantize_fp8_rowwise(bits)
        dt = time.perf_counter() - t0
        ok = np.array_equal(q.cpu().numpy(), r_q) and np.array_equal(s.cpu().numpy().view(np.uint16), r_s)
        return {"value": round(nb / dt / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
                "kind": "oracle",
                "sample": "the whole %dx%d input (row-wise fp8 cast), %.1f s wall" % (n, n, dt),
                "matches_gpu": bool(ok)}

    config = {"workload": "mx_quantize_fp8_rowwise %dx%d bf16 (heavy-tailed rows), one bf16 scale per row"
                          % (n, n), "rows": n, "cols": n, "elem": "e4m3fn", "scale": "bf16 per row",
              "metric": "achieved HBM GB/s (% of MI355X peak) for the bf16->fp8 row-wise cast"}
    return step, nb, timer, nb, "row-wise fp8 cast", cpu_baseline, config


def setup_tensorwise(dev, n=16384):
    bits, x = square_input(dev, n)
    q = torch.empty((n, n), dtype=torch.uint8, device=dev)
    s = torch.empty(1, dtype=torch.int16, device=dev)
    ws = torch.empty(mx.mx_tensorwise_workspace_bytes(n * n), dtype=torch.uint8, device=dev)
    timer = Timer(whole_step=True)

    mx.mx_quantize_fp8_tensorwise(x, out=(q, s), workspace=ws, raw=True)
    cast = c_call("mx_quantize_fp8_tensorwise", x, n * n, q, s, ws, ws.numel())

    def step():
        with timer:
            cast()

    # the amax pass must end before any element is converted and the input
    # does not fit on chip: it is read twice (2 + 2 B), codes written (1 B)
    nb = 5 * n * n + 2

    def cpu_baseline():
        import oracle
        t0 = time.perf_counter()
        r_q, r_s = oracle.quantize_fp8_tensorwise(bits)
        dt = time.perf_counter() - t0
        ok = np.array_equal(q.cpu().numpy(), r_q) and int(s.cpu().numpy().view(np.uint16)[0]) == r_s
        return {"value": round(nb / dt / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
                "kind": "oracle",
                "sample": "the whole %dx%d input (tensor-wise fp8 cast), %.1f s wall" % (n, n, dt),
                "matches_gpu": bool(ok)}

    config = {"workload": "mx_quantize_fp8_tensorwise %dx%d bf16 (heavy-tailed rows), one bf16 scale, "
                          "two-stage amax" % (n, n), "rows": n, "cols": n, "elem": "e4m3fn",
              "scale": "bf16 per tensor",
              "metric": "achieved HBM GB/s (% of MI355X peak) for the bf16->fp8 tensor-wise cast"}
    return step, nb, timer, nb, "tensor-wise fp8 cast (amax + cast launches)", cpu_baseline, config


def _mx_host(rows, k, seed):
    """Seeded random finite e4m3 codes and e8m0 scales (2^-9 .. 2^8)."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, size=(rows, k), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x7E
    s = rng.integers(118, 136, size=(rows, k // 32), dtype=np.uint8)
    return q, s


def _mx_operands(rows, k, seed, dev):
    q, s = _mx_host(rows, k, seed)
    return torch.from_numpy(q).to(dev), torch.from_numpy(s).to(dev)


GEMM_SAMPLE_ROWS = 32


def gemm_oracle_leg(c_rows, parts, n, k, what):
    """The oracle's fp64 GEMM on a bounded sample: the first
    GEMM_SAMPLE_ROWS rows of A against all of B, summed over `parts`
    ((qa, sa, qb, sb) host operands whose products add up to those rows of
    C), timed on the host; the GPU's rows `c_rows` (bf16) must lie within
    2^-10 of the sum of |products| plus half a bf16 ulp."""
    import oracle
    t0 = time.perf_counter()
    want = 0.0
    absum = 0.0
    for qa, sa, qb, sb in parts:
        c, ab = oracle.mx_gemm(qa, sa, qb, sb)
        want = want + c
        absum = absum + ab
    dt = time.perf_counter() - t0
    got = c_rows.float().cpu().numpy().astype(np.float64)
    tol = 2.0 ** -10 * absum + np.abs(want) * 2.0 ** -8 + 1e-30
    bad = int(np.count_nonzero(np.abs(got - want) > tol))
    flops = 2 * GEMM_SAMPLE_ROWS * n * k
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%s: the first %d rows of C (%d x %d x %d), fp64, %.1f s wall"
                      % (what, GEMM_SAMPLE_ROWS, GEMM_SAMPLE_ROWS, n, k, dt),
            "matches_gpu": bad == 0, **({} if bad == 0 else {"outside_tolerance": bad})}


def setup_gemm(dev, grouped=False, m=16640, n=8192, k=5120):
    log("generating MX operands")
    qa_h, sa_h = _mx_host(m, k, 101)
    qa, sa = torch.from_numpy(qa_h).to(dev), torch.from_numpy(sa_h).to(dev)
    # scales in the blocked layouts the GEMM reads (arranged before timing)
    if grouped:
        _, ends = workloads.moe_activations()
        g = len(ends)
        hb = [_mx_host(n, k, 200 + i) for i in range(g)]
        qb = torch.from_numpy(np.stack([o[0] for o in hb])).to(dev)
        sb = mx.mx_scales_to_blocked(torch.from_numpy(np.stack([o[1] for o in hb])).to(dev), raw=True)
        offs = torch.from_numpy(ends).to(dev)
        sa = mx.mx_scales_to_blocked_grouped(sa, offs, 0, raw=True)[0]
        # the sampled rows lie in group 0 (1440 rows)
        assert ends[0] >= GEMM_SAMPLE_ROWS
        sample_b = hb[0]
    else:
        sample_b = _mx_host(n, k, 102)
        qb, sb = torch.from_numpy(sample_b[0]).to(dev), torch.from_numpy(sample_b[1]).to(dev)
        sa = mx.mx_scales_to_blocked(sa, raw=True)
        sb = mx.mx_scales_to_blocked(sb, raw=True)
    c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    timer = Timer(whole_step=True)
    if grouped:
        mx.mx_grouped_gemm_mxfp8(qa, sa, qb, sb, offs, out=c)
        call = c_call("mx_grouped_gemm_mxfp8", qa, sa, qb, sb, offs, g, m, n, k, c, 1)
    else:
        mx.mx_gemm_mxfp8(qa, sa, qb, sb, out=c)
        call = c_call("mx_gemm_mxfp8", qa, sa, qb, sb, m, n, k, c, 1)

    def step():
        with timer:
            call()

    flops = 2 * m * n * k

    def cpu_baseline():
        r = GEMM_SAMPLE_ROWS
        return gemm_oracle_leg(c[:r], [(qa_h[:r], sa_h[:r], sample_b[0], sample_b[1])], n, k,
                               "grouped along M, group 0" if grouped else "dense")

    config = {"workload": "%s M=%d N=%d K=%d, e4m3 x e4m3 with e8m0 block scales (blocked layout), bf16 out%s"
                          % ("mx_grouped_gemm_mxfp8" if grouped else "mx_gemm_mxfp8", m, n, k,
                             ", 4 groups along M" if grouped else ""),
              "m": m, "n": n, "k": k, "unit": "TFLOP/s", "bound": "mfma", "peak": MFMA_FP8_PEAK_TFLOPS,
              "metric": "achieved TFLOP/s of the MX-scaled %sGEMM (%% of MI355X dense fp8 MFMA peak)"
                        % ("grouped " if grouped else ""),
              "dtype": "e4m3",
              "flops": flops}
    return step, flops, timer, flops, "MX GEMM" + (" grouped" if grouped else ""), cpu_baseline, config


def setup_ggemm(dev):
    return setup_gemm(dev, grouped=True)


def setup_kggemm(dev, m=8192, n=5120, k=16640):
    """The MoE weight-gradient GEMM: dW_g (8192, 5120) = dY_g^T X_g over each
    group's tokens, the 16640 tokens split as the MoE workload splits them."""
    log("generating MX operands")
    _, ends = workloads.moe_activations()
    g = len(ends)
    offs = torch.from_numpy(ends).to(dev)
    kends = torch.from_numpy(ends // 32).to(dev)
    qa_h, sa_h = _mx_host(m, k, 111)
    qb_h, sb_h = _mx_host(n, k, 112)
    qa, sa = torch.from_numpy(qa_h).to(dev), torch.from_numpy(sa_h).to(dev)
    qb, sb = torch.from_numpy(qb_h).to(dev), torch.from_numpy(sb_h).to(dev)
    sa = mx.mx_scales_to_blocked_grouped(sa, kends, 1, raw=True)[0]
    sb = mx.mx_scales_to_blocked_grouped(sb, kends, 1, raw=True)[0]
    c = torch.empty((g, m, n), dtype=torch.bfloat16, device=dev)
    timer = Timer(whole_step=True)
    mx.mx_kgrouped_gemm_mxfp8(qa, sa, qb, sb, offs, out=c)
    call = c_call("mx_kgrouped_gemm_mxfp8", qa, sa, qb, sb, offs, g, m, n, k, c, 1)

    def step():
        with timer:
            call()

    flops = 2 * m * n * k

    def cpu_baseline():
        # the first rows of every group's output: per group, its K range
        r = GEMM_SAMPLE_ROWS
        legs = []
        lo = 0
        for gi, e in enumerate(ends):
            hi = min(max(int(e), lo), k)
            kl, kh = lo // 32, hi // 32
            legs.append(gemm_oracle_leg(c[gi, :r], [(qa_h[:r, 32 * kl:32 * kh], sa_h[:r, kl:kh],
                                                    qb_h[:, 32 * kl:32 * kh], sb_h[:, kl:kh])], n, 32 * (kh - kl),
                                        "group %d" % gi))
            lo = hi
        secs = sum(float(re.search(r"([0-9.]+) s wall", leg["sample"]).group(1)) for leg in legs)
        ok = all(leg["matches_gpu"] for leg in legs)
        return {"value": round(2 * r * n * k / max(secs, 1e-9) / 1e12, 6), "unit": "TFLOP/s",
                "cores": legs[0]["cores"], "kind": "oracle",
                "sample": "the first %d rows of each of the %d outputs (%d x %d, each over its group's K range), "
                          "fp64, %.1f s wall" % (r, len(legs), r, n, secs),
                "matches_gpu": ok}

    config = {"workload": "mx_kgrouped_gemm_mxfp8 M=%d N=%d K=%d tokens in %d groups along K, e4m3 x e4m3 with "
                          "e8m0 block scales (K-grouped blocked layout), bf16 out" % (m, n, k, g),
              "m": m, "n": n, "k": k, "groups": g, "unit": "TFLOP/s", "bound": "mfma",
              "peak": MFMA_FP8_PEAK_TFLOPS,
              "metric": "achieved TFLOP/s of the MX-scaled GEMM grouped along K (% of MI355X dense fp8 MFMA peak)",
              "dtype": "e4m3", "flops": flops}
    return step, flops, timer, flops, "MX GEMM grouped along K", cpu_baseline, config


def _device_normal_bf16(rows, cols, seed, dev):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return torch.randn((rows, cols), generator=g, device=dev).to(torch.bfloat16)


def setup_cast_shape(dev, rows=16384, cols=16384, grouped=False, plain=False):
    """The dim0+dim1 cast at any shape (--rows, --cols), N(0,1) input drawn
    on the device: blocked scales, (grouped) 4 equal groups of rows with both
    scale sets grouped, or (plain) plain row-major scales."""
    x = _device_normal_bf16(rows, cols, 7, dev)
    u8 = dict(dtype=torch.uint8, device=dev)
    q0 = torch.empty((rows, cols), **u8)
    q1 = torch.empty((cols, rows), **u8)
    timer = Timer(whole_step=True)
    if grouped:
        g = 4
        offs = torch.tensor([rows // g * (i + 1) // 32 * 32 for i in range(g - 1)] + [rows], dtype=torch.int32,
                            device=dev)
        s0 = torch.empty((rows + 128 * g, pad(cols // 32, 4)), **u8)
        s1 = torch.empty((pad(cols, 128), pad(rows // 32, 4) + 4 * g), **u8)
        rs = torch.empty(g + 1, dtype=torch.int64, device=dev)
        cs = torch.empty(g + 1, dtype=torch.int64, device=dev)
        mx.mx_cast_dim0_dim1_grouped_blocked(x, offs, out=(q0, s0, q1, s1), out_row_starts=rs, out_col_starts=cs,
                                             raw=True)
        call = c_call("mx_cast_dim0_dim1_grouped_blocked", x, rows, cols, offs, g, q0, s0, rs, q1, s1, cs)
        nb = rows * cols * 4 + s0.numel() + s1.numel() + 16 * (g + 1)
        label = "mx_cast_dim0_dim1_grouped_blocked %dx%d bf16 N(0,1), 4 equal groups, both scale sets grouped"
        name = "cast dim0+dim1, M- and K-grouped scales"
    elif plain:
        s0 = torch.empty((rows, cols // 32), **u8)
        s1 = torch.empty((cols, rows // 32), **u8)
        mx.mx_cast_dim0_dim1(x, out=(q0, s0, q1, s1), raw=True)
        call = c_call("mx_cast_dim0_dim1", x, rows, cols, q0, s0, q1, s1)
        nb = cast_bytes(rows, cols)
        label = "mx_cast_dim0_dim1 %dx%d bf16 N(0,1), plain row-major scales"
        name = "cast dim0+dim1, plain scales (one call)"
    else:
        s0 = torch.empty((pad(rows, 128), pad(cols // 32, 4)), **u8)
        s1 = torch.empty((pad(cols, 128), pad(rows // 32, 4)), **u8)
        mx.mx_cast_dim0_dim1_blocked(x, out=(q0, s0, q1, s1), raw=True)
        call = c_call("mx_cast_dim0_dim1_blocked", x, rows, cols, q0, s0, q1, s1)
        nb = rows * cols * 4 + s0.numel() + s1.numel()
        label = "mx_cast_dim0_dim1_blocked %dx%d bf16 N(0,1), both scale sets in the 128x4 blocked layout"
        name = "cast dim0+dim1, blocked scales"

    def step():
        with timer:
            call()

    config = {"workload": label % (rows, cols), "rows": rows, "cols": cols}
    return step, nb, timer, nb, name, None, config


def setup_copy(dev, nbytes=1 << 30):
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    timer = Timer(whole_step=True)

    def step():
        with timer:
            b.copy_(a)

    config = {"workload": "device copy of %d bytes (counter calibration)" % nbytes}
    return step, 2 * nbytes, timer, 2 * nbytes, "copy", None, config


WORKLOADS = {"square16384": setup_square, "square16384_3launch": setup_square_3launch,
             "square16384_plain": setup_square_plain,
             "moe16640": setup_moe, "moe16640_2launch": setup_moe_2launch, "kgroups": setup_kgroups, "rowwise16384": setup_rowwise,
             "tensorwise16384": setup_tensorwise, "moe16640_both": setup_moe_both,
             "moe16640_both_2launch": setup_moe_both_2launch, "gemm16640": setup_gemm, "ggemm16640": setup_ggemm, "kggemm16640": setup_kggemm,
             "experts16": setup_experts, "experts16_2launch": setup_experts_2launch, "copy": setup_copy,
             "cast_blocked": setup_cast_shape,
             "cast_grouped": lambda dev, **kw: setup_cast_shape(dev, grouped=True, **kw),
             "cast_plain": lambda dev, **kw: setup_cast_shape(dev, plain=True, **kw)}


# Further workloads measured by the default run (one entry each under
# "configs"): the plain-scale call the headline's fused call replaces, the
# MoE activation casts with grouped scales, the K-grouped layouts and the 3D
# expert-weight cast.  They run before the headline's warm-up.
EXTRAS = (
    ("square16384_plain", setup_square_plain),
    ("moe16640", setup_moe),
    ("moe16640_both", setup_moe_both),
    ("kgroups", setup_kgroups),
    ("experts16", lambda dev: setup_experts(dev, device_inputs=True)),
)


def graph_step_us(step, graph_steps, steps, dev):
    """Mean time of a step replayed from a captured graph of `graph_steps`
    steps (one event pair around steps // graph_steps replays): the GPU runs
    the launches back to back, whatever the host's time to issue them."""
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(graph_steps):
            step()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize(dev)
    reps = max(1, steps // graph_steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize(dev)
    us = e0.elapsed_time(e1) * 1e3 / (reps * graph_steps)
    del g
    return us, reps * graph_steps


def measure_extra(name, setup, dev, warmup=20, steps=100, cold=20):
    """Back-to-back mean over `steps` launches (one event pair around them,
    after `warmup`; replays of a captured graph for workloads whose launches
    are shorter than the host's time to issue them) and the cold-cache
    median over `cold` more, for one workload; its buffers are released
    afterwards."""
    step, step_bytes, timer, kern_bytes, kern_name, _, config = setup(dev)
    scale = 1e12 if config.get("unit") == "TFLOP/s" else 1e9
    unit = config.get("unit", "GB/s")
    peak = config.get("peak", HBM_PEAK_GBS)
    graph_steps = config.get("graph_steps", 0)
    # warm-up: at least `warmup` steps and 25 ms of them, so that a workload
    # measured first still runs at the GPU's steady clocks
    timer.reserve(warmup + steps)
    t0 = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t0 < 0.025:
        for _ in range(10):
            step()
        done += 10
        torch.cuda.synchronize(dev)
        timer.clear()
    timer.clear()
    if graph_steps:
        us, steps = graph_step_us(step, graph_steps, steps, dev)
    else:
        timer.start_region()
        for _ in range(steps):
            step()
        timer.end_region(steps)
        torch.cuda.synchronize(dev)
        us = timer.mean_ms() * 1e3
    achieved = kern_bytes / (us * 1e-6) / scale
    timer.reserve(cold)
    c = cold_cache(step, step_bytes, cold, scale, unit, peak, dev)
    log("%s: %.2f us, %.1f %s (%.1f%%); cold %.2f us" % (name, us, achieved, unit, 100 * achieved / peak,
                                                         c["step_us_median"]))
    return {"workload": config["workload"], "kernel": kern_name, "kernel_us": round(us, 2),
            "achieved": round(achieved, 1), "unit": unit, "frac": round(achieved / peak, 4),
            ("algorithmic_flops" if unit == "TFLOP/s" else "algorithmic_bytes"): kern_bytes,
            "cold_us_median": c["step_us_median"], "cold_frac": c["frac"], "steps": steps, "warmup": done,
            **({"graph_steps": graph_steps} if graph_steps else {})}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="square16384", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rows", type=int, default=None, help="rows of the cast_blocked / cast_grouped / cast_plain workloads")
    ap.add_argument("--cols", type=int, default=None, help="cols of the cast_blocked / cast_grouped / cast_plain workloads")
    ap.add_argument("--cold-launches", type=int, default=50,
                    help="steps timed one by one after cache-evicting traffic (0: skip)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the further workloads the default run measures before the headline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the cast and layout kernels run on one GPU's "
              "share and no multi-GPU path is built; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    mx.lib()

    shape = {k: v for k, v in (("rows", args.rows), ("cols", args.cols)) if v is not None}
    if shape and args.workload not in ("cast_blocked", "cast_grouped", "cast_plain"):
        print("--rows / --cols apply to the cast_blocked, cast_grouped and cast_plain workloads only",
              file=sys.stderr)
        sys.exit(2)
    step, step_bytes, timer, kern_bytes, kern_name, cpu_fn, config = WORKLOADS[args.workload](dev, **shape)
    extras = None
    if args.workload == "square16384" and not args.no_extras:
        # Measured first: they also bring the GPU out of its idle clocks (a
        # process's first ~15-20 ms of launches, or the first after an idle
        # second, run ~4% slower whatever they touch), so that a short
        # warm-up of the headline reads its steady state.
        extras = {}
        for name, setup in EXTRAS:
            extras[name] = measure_extra(name, setup, dev)
            torch.cuda.synchronize(dev)
            torch.cuda.empty_cache()
    timer.reserve(args.warmup + args.steps)
    torch.cuda.synchronize(dev)
    log("warmup %d steps" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    timer.clear()

    log("timing %d steps" % args.steps)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    timer.start_region()
    for _ in range(args.steps):
        step()
    timer.end_region(args.steps)
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    scale = 1e12 if config.get("unit") == "TFLOP/s" else 1e9
    unit = config.pop("unit", "GB/s")
    metric = config.pop("metric", METRIC)
    dtype = config.pop("dtype", "bf16")
    bound = config.pop("bound", "hbm")
    config.pop("graph_steps", None)
    peak = config.pop("peak", HBM_PEAK_GBS)
    value = step_bytes / (ms_per_step * 1e-3) / scale
    kern_ms = timer.mean_ms()
    achieved = kern_bytes / (kern_ms * 1e-3) / scale
    log("step %.2f us, %s %.2f us = %.1f %s" % (ms_per_step * 1e3, kern_name, kern_ms * 1e3, achieved, unit))

    traffic = counter_traffic() if args.workload == "square16384" else None
    roofline = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4),
                "traffic": traffic,
                "kernel": kern_name, "kernel_us": round(kern_ms * 1e3, 2),
                ("algorithmic_flops" if unit == "TFLOP/s" else "algorithmic_bytes"): kern_bytes}
    if traffic is not None:
        # not measured by this run: the committed counter summary's figure,
        # used only while the kernel sources it was taken on are unchanged
        roofline["traffic_source"] = ("rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE, stored in profiles/%s "
                                      "(kernel sources digest %s)" % (os.path.basename(COUNTER_SUMMARY),
                                                                       sources_digest()))

    cold = None
    if args.cold_launches > 0:
        timer.reserve(args.cold_launches)   # steps that time a launch inside keep recording
        cold = cold_cache(step, step_bytes, args.cold_launches, scale, unit, peak, dev)

    cpu = None
    if cpu_fn is not None and not args.no_cpu_baseline:
        log("timing the CPU oracle on a slice")
        cpu = cpu_fn()

    line = {"metric": metric, "value": round(value, 1), "unit": unit, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic", "config": config, "roofline": roofline, "cpu_baseline": cpu,
            "cold_cache": cold}
    if extras is not None:
        line["configs"] = extras
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
