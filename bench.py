#!/usr/bin/env python3
"""Throughput of the row-reduce hot path on one MI355X, as achieved HBM GB/s.

One step runs every large workload once, in this order, each on its own
buffers with inputs already resident in HBM:

  fused      fused residual add + RMSNorm, bf16 I/O, 8192 x 4096
  rms_bf16   RMSNorm bf16, 8192 x 4096 (the fused workload's x and gamma)
  sm_wave    softmax fp32 -> fp32, 16384 x 1024 (a wavefront per row)
  sm_vocab   softmax bf16 -> fp32, 256 x 152064 (a row per 1024-lane workgroup)
  sm_causal  softmax fp32 -> fp32, 28*4096 x 4096, causal -inf mask (a workgroup per row)

value = algorithmic bytes of one step (each input read once, each output
written once, gamma once) / measured time of one step.  Every workload but
the 3.76 GB causal softmax has ROTATE copies of its buffers, and step k uses
copy k mod ROTATE, so between two uses of a buffer more than the 256 MB
last-level cache has streamed through and every kernel starts cold (the
causal softmax's own footprint is 15 times that cache).  The fused op updates
its residual in place each step; that changes the values, not the work.

Two timed regions of K steps each, on the launch stream: the first has HIP
events only around the K steps and gives the value; the second records an
event between operations and gives each operation's average duration (the
breakdown and the roofline of the dominant operation, the one with the
largest share of the step).

cpu_baseline: the fp64 CPU oracle, timed on the host cores over the same
workloads (all rows by default; --cpu-fraction takes the first rows of each),
reported in the same unit.  parity: the GPU outputs of the same run against
those oracle outputs, per operation, at the test suite's bars.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s and % of MI355X peak, RMSNorm 8192x4096 bf16 + softmax rows"
PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, published
# The kernel of a launch is the library's device code plus the launch plan
# (both recorded beside the counters and compared).
PLAN_KEYS = ("variant_name", "waves_per_row", "rows_per_group", "vecs_per_lane", "vec_elems",
             "block_threads")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sm_causal_softmax_block.json")

OPS = ("fused", "rms_bf16", "sm_wave", "sm_vocab", "sm_causal")
ROTATE = 4   # buffer copies of every workload but sm_causal


def code_object_sha(lib_path=None):
    """Hash of the device code the library carries: the instructions, kernel
    descriptors and metadata notes of the gfx950 code objects in its
    .hip_fatbin section, read without loading the library.  Comments,
    host-only edits and the linker's placement of device variables (whose
    order in .bss varies from build to build) leave it unchanged; any kernel
    change changes it."""
    if lib_path is None:
        from row_reduction_rmsnorm_amd import binding
        lib_path = binding.LIB_PATH
    h = hashlib.sha256()
    for name, body in device_code_sections(fatbin_bytes(lib_path)):
        h.update(name + b"\0" + len(body).to_bytes(8, "little") + body)
    return h.hexdigest()[:16]


def _elf_sections(data):
    """(name, type, offset, size) of every section of a 64-bit ELF image."""
    import struct
    if data[:4] != b"\x7fELF" or data[4] != 2:
        raise ValueError("not a 64-bit ELF image")
    shoff = struct.unpack_from("<Q", data, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    heads = [struct.unpack_from("<IIQQQQ", data, shoff + i * shentsize) for i in range(shnum)]
    names = heads[shstrndx][4]
    out = []
    for name, typ, _, _, off, size in heads:
        end = data.index(b"\0", names + name)
        out.append((data[names + name:end], typ, off, size))
    return out


def device_code_sections(fatbin):
    """(name, contents) of the .text, .rodata and .note sections of every
    amdgcn code object in an offload-bundle blob, in bundle order."""
    import struct
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    out = []
    pos = fatbin.find(magic)
    while pos >= 0:
        count = struct.unpack_from("<Q", fatbin, pos + len(magic))[0]
        at = pos + len(magic) + 8
        for _ in range(count):
            off, size, tlen = struct.unpack_from("<QQQ", fatbin, at)
            triple = fatbin[at + 24:at + 24 + tlen]
            at += 24 + tlen
            if b"amdgcn" in triple and size > 0:
                co = fatbin[pos + off:pos + off + size]
                for name, typ, soff, ssize in _elf_sections(co):
                    if name in (b".text", b".rodata", b".note"):
                        out.append((triple + b":" + name, co[soff:soff + ssize]))
        pos = fatbin.find(magic, pos + 1)
    if not out:
        raise ValueError("no amdgcn code object in the bundle")
    return out


def fatbin_bytes(lib_path):
    """The .hip_fatbin ELF section of a shared library (its offload bundles)."""
    import struct
    with open(lib_path, "rb") as f:
        data = f.read()
    if data[:4] != b"\x7fELF" or data[4] != 2:
        raise ValueError(f"{lib_path}: not a 64-bit ELF file")
    shoff = struct.unpack_from("<Q", data, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)

    def section(i):
        return struct.unpack_from("<IIQQQQ", data, shoff + i * shentsize)

    names = section(shstrndx)[4]
    for i in range(shnum):
        name, _, _, _, off, size = section(i)
        end = data.index(b"\0", names + name)
        if data[names + name:end] == b".hip_fatbin":
            return data[off:off + size]
    raise ValueError(f"{lib_path}: no .hip_fatbin section")


def algorithmic_bytes(op, M, N):
    """Read each input once, write each output once, gamma once."""
    if op == "fused":
        return 4 * M * N * 2 + N * 2
    if op == "rms_bf16":
        return 2 * M * N * 2 + N * 2
    if op == "rms_f32":
        return 2 * M * N * 4 + N * 4
    if op == "sm_wave" or op == "sm_causal":
        return M * N * (4 + 4)
    if op == "sm_vocab":
        return M * N * (2 + 4)
    raise KeyError(op)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def setup(torch, dev):
    """bufs[name]: the workload's first buffer set (with M, N) and, under
    "sets", all its copies (set 0 first).  Copies hold the same values at
    other addresses."""
    import workloads
    import row_reduction_rmsnorm_amd as rr
    bufs = {}
    t0 = time.time()
    w = workloads.make("fused")
    x = w.arrays["x"].to(dev)
    g = w.arrays["gamma"].to(dev)
    r = w.arrays["residual"].to(dev)
    bufs["fused"] = [dict(x=x.clone(), r=r.clone(), g=g, y=torch.empty_like(x), M=w.M, N=w.N,
                          eps=w.eps, r0=w.arrays["residual"]) for _ in range(ROTATE)]
    # copies of x of their own, so the RMSNorm never finds the fused op's input in a cache
    bufs["rms_bf16"] = [dict(x=x.clone(), g=g, y=torch.empty_like(x), M=w.M, N=w.N, eps=w.eps)
                        for _ in range(ROTATE)]
    del x, r
    for name in ("sm_wave", "sm_vocab", "sm_causal"):
        w = workloads.make(name)
        xs = w.arrays["x"].to(dev)
        n = 1 if name == "sm_causal" else ROTATE
        sets = []
        for i in range(n):
            xi = xs if i == n - 1 else xs.clone()
            y = torch.empty(xs.shape, dtype=torch.float32, device=dev)
            sets.append(dict(x=xi, y=y, ws=rr.softmax_workspace(xi, torch.float32), M=w.M, N=w.N))
        bufs[name] = sets
    for name in list(bufs):
        sets = bufs[name]
        bufs[name] = dict(sets[0], sets=sets)
    torch.cuda.synchronize()
    log(f"[bench] inputs generated and resident in HBM ({time.time() - t0:.1f} s)")
    return bufs


def make_ops(rr, bufs):
    """name -> fn(k): the operation on buffer set k mod (number of sets)."""
    def pick(name, k):
        sets = bufs[name]["sets"]
        return sets[k % len(sets)]

    def fused(k):
        b = pick("fused", k)
        rr.rr_fused_add_rmsnorm(b["y"], b["r"], b["x"], b["g"], b["eps"])

    def rms(k):
        b = pick("rms_bf16", k)
        rr.rr_rmsnorm(b["y"], b["x"], b["g"], b["eps"])

    def softmax(name):
        def run(k):
            b = pick(name, k)
            rr.rr_softmax_rows(b["y"], b["x"], b["ws"])
        return run

    return {"fused": fused, "rms_bf16": rms, "sm_wave": softmax("sm_wave"),
            "sm_vocab": softmax("sm_vocab"), "sm_causal": softmax("sm_causal")}


def sanity(torch, bufs):
    """Cheap checks after the first step (torch arithmetic, no oracle): the new
    residual is bf16(x + r0) and softmax rows sum to one."""
    f = bufs["fused"]
    rows = slice(0, 64)
    expect = (f["x"][rows].cpu() + f["r0"][rows])
    assert torch.equal(f["r"][rows].cpu(), expect), "fused residual mismatch"
    for name in ("sm_wave", "sm_vocab", "sm_causal"):
        s = bufs[name]["y"][:64].double().sum(dim=1)
        err = float((s - 1).abs().max())
        assert err < 1e-4, f"{name}: row sums off by {err}"


def cpu_baseline(torch, rr, ops, bufs, fraction):
    """Time the fp64 oracle on the first ceil(M * fraction) rows of every
    workload; returns the equivalent GB/s over the same algorithmic bytes.

    Outside the timed calls, the oracle's outputs also serve as the parity
    check of this run: each operation is run once more on buffer set 0 (the
    fused op, which updates its residual in place on every step, on a fresh
    copy of the original residual) and its output on those rows is compared
    with them at the bars of tests/compare.py.  Returns (baseline, parity)."""
    import numpy as np
    import oracle
    from tests import compare
    total_t = 0.0
    total_b = 0
    parts = []
    parity = {}

    def check(name, fn, bar):
        try:
            parity[name] = dict(fn(), bar=bar, ok=True)
        except AssertionError as e:
            parity[name] = dict(bar=bar, ok=False, error=str(e))
            log(f"[bench] PARITY FAILURE {name}: {e}")

    for name in OPS:
        b = bufs[name]
        M, N = b["M"], b["N"]
        m = max(1, int(math.ceil(M * fraction)))
        xs = b["x"][:m].float().cpu().double().numpy()
        if name == "fused":
            rs = b["r0"][:m].double().numpy()
            g = b["g"].float().cpu().double().numpy()
            t0 = time.perf_counter()
            h_ref, y_ref = oracle.fused_add_rmsnorm(xs, rs, g, b["eps"], "bf16")
            dt = time.perf_counter() - t0
            r_gpu = b["r0"][:m].to(b["x"].device)
            y_gpu = torch.empty_like(r_gpu)
            rr.rr_fused_add_rmsnorm(y_gpu, r_gpu, b["x"][:m], b["g"], b["eps"])
            torch.cuda.synchronize()
            check(name, lambda: {"residual": compare.check_bf16_exact(r_gpu, h_ref, "fused residual"),
                                 "y": compare.check_bf16(y_gpu, y_ref, "fused y")},
                  "residual bit-exact; y <= 1 bf16 ulp")
            del h_ref, y_ref, r_gpu, y_gpu
        elif name == "rms_bf16":
            g = b["g"].float().cpu().double().numpy()
            t0 = time.perf_counter()
            ref = oracle.rmsnorm(xs, g, b["eps"])
            dt = time.perf_counter() - t0
            ops[name](0)
            torch.cuda.synchronize()
            check(name, lambda: compare.check_bf16(b["y"][:m], ref, name), "<= 1 bf16 ulp")
            del ref
        else:
            t0 = time.perf_counter()
            ref = oracle.softmax(xs)
            dt = time.perf_counter() - t0
            ops[name](0)
            torch.cuda.synchronize()
            check(name, lambda: compare.check_softmax(b["y"][:m], xs, ref, name),
                  f"max |g - r| <= {compare.SOFTMAX_F32_ATOL:g} per probability; rows sum to 1 within "
                  f"{compare.SOFTMAX_ROWSUM_ATOL:g}")
            del ref
        nb = algorithmic_bytes(name, m, N)
        total_t += dt
        total_b += nb
        parts.append(f"{name} {m}/{M} rows")
        del xs
    base = {
        "value": round(total_b / total_t / 1e9, 3),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"{'all' if fraction >= 1 else f'the first {fraction:.4g}'} of the rows of every workload "
                   f"({', '.join(parts)}); "
                   f"{total_b / 1e9:.3f} GB algorithmic, {total_t:.2f} s on the host"),
        "seconds": round(total_t, 3),
    }
    return base, parity


def measure_extras(torch, rr, dev, K, bufs):
    """Operations outside the step, each timed on its own: K launches between
    two events, after a warm-up launch, each launch on the next of several
    copies of its buffers, so that (as in the step) more than the 256 MB
    last-level cache streams through between two uses of a copy and every
    launch starts cold.  The operations: the 64 x 3584 fp32 RMSNorm and the
    256 x 5120 fp32 LayerNorm (latency cases on 256 CUs, reported as time and
    rows/s, also as a HIP graph of K launches, which removes the host's
    launch cost), LayerNorm bf16 8192 x 4096 (the RMSNorm workload's shape,
    for bandwidth), the attention-score softmax through the causal rule (only
    the kept keys are read: row i of a head reads i + 1 keys and writes all
    4096), log-softmax on the vocabulary logits, rows that are not whole
    vectors (a 50257-wide vocabulary softmax; an RMSNorm, a LayerNorm and a
    fused add + RMSNorm of 4097), and the
    vocabulary softmax at decode-size row counts (1, 16, 48 rows of 152064
    bf16 -> fp32: the split path, two kernels)."""
    import numpy as np
    import workloads
    out = {}

    def timed(name, fn, nbytes, M, sets=1, graph=False):
        """fn(k) runs the operation on copy k mod sets."""
        fn(0)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for k in range(K):
            fn((k + 1) % sets)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / K * 1e3
        out[name] = {"us": round(us, 2), "bytes": nbytes, "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "rows_per_s": round(M / (us * 1e-6), 1), "buffer_sets": sets,
                     "cold": sets > 1 or nbytes > (512 << 20)}
        if graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for k in range(K):
                    fn(k % sets)
            g.replay()
            torch.cuda.synchronize()
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            gus = a.elapsed_time(b) / K * 1e3
            out[name].update({"graph_us": round(gus, 2),
                              "graph_GBps": round(nbytes / (gus * 1e-6) / 1e9, 1),
                              "graph_rows_per_s": round(M / (gus * 1e-6), 1)})

    def copies(t, n):
        return [t] + [t.clone() for _ in range(n - 1)]

    def sets_for(nbytes):
        """Copies so that more than 256 MB streams between two uses of one."""
        return max(2, int(math.ceil((300 << 20) / nbytes)) + 1)

    # latency cases (tiny footprints; the cache keeps them, the graph figure
    # is the device's time per launch)
    w = workloads.make("rms_f32")
    x, g = w.arrays["x"].to(dev), w.arrays["gamma"].to(dev)
    y = torch.empty_like(x)
    timed("rms_f32_64x3584", lambda k: rr.rr_rmsnorm(y, x, g, w.eps), algorithmic_bytes("rms_f32", w.M, w.N),
          w.M, graph=True)
    w = workloads.make("layernorm")
    x, g, bt = (w.arrays[k].to(dev) for k in ("x", "gamma", "beta"))
    y = torch.empty_like(x)
    timed("layernorm_f32_256x5120", lambda k: rr.rr_layernorm(y, x, g, bt, w.eps),
          2 * w.M * w.N * 4 + 2 * w.N * 4, w.M, graph=True)
    # the floor for the two latency-bound shapes: a kernel that writes one
    # value (torch's fill), timed the same way
    one = torch.empty(1, device=dev)
    timed("launch_floor_fill_1_value", lambda k: one.fill_(1.0), 4, 1, graph=True)
    del x, g, bt, y

    rng = np.random.default_rng(0)
    M, N = 8192, 4096
    nb = 2 * M * N * 2 + 2 * N * 2
    n = sets_for(nb)
    xs = copies(workloads.to_dtype(rng.standard_normal((M, N), dtype=np.float32), "bf16").to(dev), n)
    ys = [torch.empty_like(xs[0]) for _ in range(n)]
    g = workloads.to_dtype(workloads.gamma_vector(N, 1), "bf16").to(dev)
    bt = workloads.to_dtype(workloads.gamma_vector(N, 2) - 1.0, "bf16").to(dev)
    timed("layernorm_bf16_8192x4096", lambda k: rr.rr_layernorm(ys[k], xs[k], g, bt, 1e-5), nb, M, sets=n)
    del xs, ys, g, bt

    b = bufs["sm_causal"]
    M, N = b["M"], b["N"]
    kept = int(np.minimum(N, np.arange(M) % 4096 + 1).sum())
    causal = rr.make_softmax_opts(causal_period=4096, causal_offset=0)
    timed("causal_softmax_f32_114688x4096_kept_keys_only",
          lambda k: rr.rr_softmax_rows_ex(b["y"], b["x"], causal, None), kept * 4 + M * N * 4, M)
    sets = bufs["sm_vocab"]["sets"]
    lg = rr.make_softmax_opts(log_output=True)
    timed("log_softmax_bf16_f32_256x152064",
          lambda k: rr.rr_softmax_rows_ex(sets[k]["y"], sets[k]["x"], lg, sets[k]["ws"]),
          sets[0]["M"] * sets[0]["N"] * (2 + 4), sets[0]["M"], sets=len(sets))

    # rows that are not whole vectors (contiguous rows of an odd width, every
    # row at its own offset): cut at aligned addresses
    M, N = 256, 50257                     # a 50257-entry vocabulary
    nb = M * N * (2 + 4)
    n = sets_for(nb)
    xs = copies(workloads.to_dtype(rng.standard_normal((M, N), dtype=np.float32), "bf16").to(dev), n)
    ys = [torch.empty((M, N), dtype=torch.float32, device=dev) for _ in range(n)]
    timed("softmax_bf16_f32_256x50257_rows_cut", lambda k: rr.rr_softmax_rows(ys[k], xs[k], None), nb, M, sets=n)
    del xs, ys
    M, N = 8192, 4097
    nb = 2 * M * N * 2 + N * 2
    n = sets_for(nb)
    xs = copies(workloads.to_dtype(rng.standard_normal((M, N), dtype=np.float32), "bf16").to(dev), n)
    ys = [torch.empty_like(xs[0]) for _ in range(n)]
    g = workloads.to_dtype(workloads.gamma_vector(N, 3), "bf16").to(dev)
    timed("rmsnorm_bf16_8192x4097_rows_cut", lambda k: rr.rr_rmsnorm(ys[k], xs[k], g, 1e-6), nb, M, sets=n)
    bt = workloads.to_dtype(workloads.gamma_vector(N, 4) - 1.0, "bf16").to(dev)
    timed("layernorm_bf16_8192x4097_rows_cut", lambda k: rr.rr_layernorm(ys[k], xs[k], g, bt, 1e-5),
          nb + N * 2, M, sets=n)
    # the fused op rewrites its residual in place: each copy's residual
    # drifts from call to call, which does not change the work
    rs = [workloads.to_dtype(rng.standard_normal((M, N), dtype=np.float32), "bf16").to(dev) for _ in range(n)]
    timed("fused_add_rmsnorm_bf16_8192x4097_rows_cut",
          lambda k: rr.rr_fused_add_rmsnorm(ys[k], rs[k], xs[k], g, 1e-6), 2 * nb - N * 2, M, sets=n)
    del xs, ys, g, bt, rs

    # the vocabulary softmax at decode-size row counts: few long rows split
    # over many workgroups (statistics pass, then the normalising pass)
    full = bufs["sm_vocab"]["x"]
    N = full.shape[1]
    for M in (1, 16, 48):
        nb = M * N * (2 + 4)
        n = sets_for(nb)
        xs = [full[(i * M) % 256:(i * M) % 256 + M].clone() if (i * M) % 256 + M <= 256 else full[:M].clone()
              for i in range(n)]
        ys = [torch.empty((M, N), dtype=torch.float32, device=dev) for _ in range(n)]
        ws = rr.softmax_workspace(xs[0], torch.float32)
        plan = rr.rr_query_plan(rr.RR_OP_SOFTMAX, M, N, rr.RR_BF16, rr.RR_F32)
        timed(f"softmax_bf16_f32_{M}x{N}_split", lambda k: rr.rr_softmax_rows(ys[k], xs[k], ws), nb, M, sets=n,
              graph=True)
        out[f"softmax_bf16_f32_{M}x{N}_split"].update(
            {"plan": plan["variant_name"], "chunks_per_row": plan["chunks_per_row"],
             "read_once_bytes": nb, "two_pass_bytes": M * N * (2 + 2 + 4)})
        del xs, ys, ws
    return out


def measure_copy_reference(torch, rr, dev, ops, bufs, reps=15):
    """Each step operation against a streaming copy that moves the same bytes
    (the library's rr_stream_copy: half the bytes read, half written, 16-byte
    non-temporal accesses, no reduction), both timed the same way: one launch
    between two events, after writing 512 MiB elsewhere so that neither finds
    its data in a cache; median of `reps`.  At these sizes a kernel's fixed
    start-up and drain time is a visible share of its duration, so this, not
    8 TB/s, is the practical bar for each size.  (torch's own copy_, abs and
    neg move the same bytes 10-40% slower than this copy, so they are not
    used as the bar.)"""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)

    def cold_us(fn):
        ts = []
        for _ in range(reps):
            flush.zero_()
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        ts.sort()
        return ts[len(ts) // 2]

    out = {}
    for name in OPS:
        nb = algorithmic_bytes(name, bufs[name]["M"], bufs[name]["N"])
        n = nb // 8                      # fp32 elements read (and written)
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        copy_us = cold_us(lambda: rr.rr_stream_copy(dst, src))
        op_us = cold_us(lambda: ops[name](0))
        del src, dst
        out[name] = {"bytes": nb, "op_us": round(op_us, 2), "op_GBps": round(nb / (op_us * 1e-6) / 1e9, 1),
                     "copy_us": round(copy_us, 2), "copy_GBps": round(nb / (copy_us * 1e-6) / 1e9, 1),
                     "op_vs_copy": round(copy_us / op_us, 3)}
    del flush
    return out


def causal_plan(rr):
    p = rr.rr_query_plan(rr.RR_OP_SOFTMAX, 114688, 4096, rr.RR_F32, rr.RR_F32)
    return {k: p[k] for k in PLAN_KEYS}


def traffic_for(per_launch_ok, rr):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, if it was taken on the device
    code and the launch plan as they are now."""
    if not per_launch_ok or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("code_object_sha") != code_object_sha() or t.get("plan") != causal_plan(rr):
        return None
    return t.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-fraction", type=float, default=1.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 512 MiB read + 512 MiB write pass (for counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "rows are independent, so a multi-GPU run is the same kernel on each GPU's share of "
              "the rows with no exchange, and only the one-GPU run is measured here.", file=sys.stderr)
        sys.exit(2)

    import torch
    import row_reduction_rmsnorm_amd as rr
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rr.lib()
    bufs = setup(torch, dev)
    ops = make_ops(rr, bufs)

    if args.calibrate_copy:
        # the library's streaming copy (the diagnostics build) of a known size,
        # 512 MiB read and 512 MiB written with the same 16-byte non-temporal
        # accesses the kernels use, for counter calibration; its dispatches
        # are told apart from the size-matched copies below by their grid
        # (32768 workgroups of 1024 lanes)
        src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            rr.rr_stream_copy(dst, src)
        torch.cuda.synchronize()
        del src, dst

    # warmup (the first step is checked)
    for i in range(args.warmup):
        for name in OPS:
            ops[name](i)
        if i == 0:
            torch.cuda.synchronize()
            sanity(torch, bufs)
    torch.cuda.synchronize()

    K = args.steps
    stream = torch.cuda.current_stream(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)

    # timed region 1: K whole steps, events only around them -> the value
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(K):
        for name in OPS:
            ops[name](k)
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / K

    # timed region 2: K more steps with an event between operations -> the
    # per-operation durations (the event records add a little time of their
    # own, so these are slight overestimates of the kernel times)
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(len(OPS) + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    for k in range(K):
        marks[k][0].record(stream)
        for j, name in enumerate(OPS):
            ops[name](k)
            marks[k][j + 1].record(stream)
    torch.cuda.synchronize()
    per_op_all = {name: sorted(marks[k][j].elapsed_time(marks[k][j + 1]) for k in range(K))
                  for j, name in enumerate(OPS)}
    per_op_ms = {name: sum(v) / K for name, v in per_op_all.items()}
    step_bytes = sum(algorithmic_bytes(n, bufs[n]["M"], bufs[n]["N"]) for n in OPS)
    value = step_bytes / (ms_step * 1e-3) / 1e9

    breakdown = {}
    for name in OPS:
        nb = algorithmic_bytes(name, bufs[name]["M"], bufs[name]["N"])
        t = per_op_ms[name]
        breakdown[name] = {"M": bufs[name]["M"], "N": bufs[name]["N"], "bytes": nb,
                           "us": round(t * 1e3, 2), "GBps": round(nb / (t * 1e-3) / 1e9, 1),
                           "us_median": round(per_op_all[name][K // 2] * 1e3, 2),
                           "us_min": round(per_op_all[name][0] * 1e3, 2),
                           "frac_peak": round(nb / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                           "rows_per_s": round(bufs[name]["M"] / (t * 1e-3), 1)}
    dom = max(OPS, key=lambda n: per_op_ms[n])
    dom_bytes = algorithmic_bytes(dom, bufs[dom]["M"], bufs[dom]["N"])
    achieved = dom_bytes / (per_op_ms[dom] * 1e-3) / 1e9
    plan = rr.rr_query_plan(rr.RR_OP_SOFTMAX, bufs[dom]["M"], bufs[dom]["N"], rr.RR_F32, rr.RR_F32) \
        if dom.startswith("sm_") else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic_for(dom == "sm_causal", rr),
                "kernel": dom, "bytes_per_launch": dom_bytes,
                "us_per_launch": round(per_op_ms[dom] * 1e3, 2),
                "plan": plan["variant_name"] if plan else None}

    extras = measure_extras(torch, rr, dev, K, bufs)
    copy_ref = measure_copy_reference(torch, rr, dev, ops, bufs)
    # the same-size streaming copy beside the dominant operation (cold, one
    # launch between events; the op's own cold figure is in size_matched_copy)
    roofline["same_size_copy_GBps"] = copy_ref[dom]["copy_GBps"]

    cpu = parity = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        cpu, parity = cpu_baseline(torch, rr, ops, bufs, args.cpu_fraction)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "one step = fused add+RMSNorm bf16 8192x4096 + RMSNorm bf16 8192x4096 + "
                        "softmax f32 16384x1024 + softmax bf16->f32 256x152064 + "
                        "causal softmax f32 114688x4096",
            "io_dtypes": "bf16 norms; softmax f32->f32, bf16->f32",
            "bytes_per_step": step_bytes,
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "breakdown": breakdown,
        "extras": extras,
        "size_matched_copy": copy_ref,
        "device": torch.cuda.get_device_name(dev),
        "code_object_sha": code_object_sha(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
