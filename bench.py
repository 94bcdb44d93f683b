"""Benchmark of the triangle multiplicative update on one MI355X.

One step = the whole update in both directions (outgoing, then incoming:
projection kernel, contraction kernel, epilogue kernel each) over the
n3605_4ch workload: N = 3605 residues in 4 chains (1200/1000/800/605), the
complex size that page 1 ("Os numeros") folds on four GPUs; c_z = c = 128,
bf16, synthetic seeded inputs already resident in HBM.  The metric is pair
updates per second over the whole job: 2 * N^2 per step / seconds per step.

Two timed loops of K steps each:
  1. the public entry points trimul_outgoing + trimul_incoming, wall clock
     between device synchronizations -> `value`, `ms_per_step`;
  2. the same kernels launched one by one through trimul_tile_operands /
     trimul_tile (identical kernels, launch shapes and buffers) with HIP events
     between them on the launch stream -> per-kernel average durations, the
     roofline of the dominant kernel (the contraction, matrix-core bound) and
     the HBM rates of the projection and epilogue kernels.
The CPU baseline times the float64 oracle's three phases on bounded blocks of
the same workload on the host cores and extrapolates (projection and epilogue
scale with N^2, contraction with N^3).

Prints exactly one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 matrix peak (the fp32 path's contraction instructions)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
C = 128
C_Z = 128
def k1_bytes_per_pair(elt):
    """z in the storage type + mask + a, b in the storage type."""
    return C_Z * elt + 1 + 2 * C * elt


def k3_bytes_per_pair(elt):
    """x (fp32) + z in the storage type + mask + out (fp32)."""
    return C * 4 + C_Z * elt + 1 + C_Z * 4


K1_BYTES_PER_PAIR = k1_bytes_per_pair(2)   # bf16: 769
K3_BYTES_PER_PAIR = k3_bytes_per_pair(2)   # bf16: 1281
K1_FLOPS_PER_PAIR = 4 * C * C_Z * 2
K3_FLOPS_PER_PAIR = 2 * C_Z * C * 2


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def traffic_from_profile(kernel_src):
    """L2-miss bytes per contraction launch from the committed counter summary
    (the L2's FETCH_SIZE and WRITE_SIZE, calibrated on a plain copy; they
    include reads served by the Infinity Cache, so they bound the DRAM traffic
    from above), or None when the summary is absent or the kernel source
    changed since."""
    path = os.path.join(ROOT, "profiles", "k2_contract_n3605_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"source sha256: ([0-9a-f]{64})", text)
    m_b = re.search(r"L2-miss bytes per launch: ([0-9.eE+]+)", text)
    if not m_sha or not m_b:
        return None
    sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    return float(m_b.group(1)) if sha == m_sha.group(1) else None


def measured_ceilings():
    """Achievable peaks measured on this GPU model by the peaks mode (the
    committed summary profiles/peaks_mi355x.md): the bf16 matrix-core loop and
    the streaming kernels at the projection's and epilogue's byte mixes."""
    path = os.path.join(ROOT, "profiles", "peaks_mi355x.md")
    if not os.path.exists(path):
        return {}
    out = {}
    for m in re.finditer(r"ceiling (\w+) (GB/s|TFLOP/s): ([0-9.]+)", open(path).read()):
        out[m.group(1)] = float(m.group(3))
    return out


def blas_threads():
    """Threads of the BLAS library numpy's products run on."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        return os.cpu_count()


def host_cpu(blas_threads):
    """The host the oracle ran on: CPU model, logical CPUs visible to this
    process, and the BLAS thread count the oracle's products used."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "usable_cpus": usable,
            "blas_threads": int(blas_threads)}


def cpu_baseline(work, block_rows):
    """Oracle phase rates on blocks of the workload, extrapolated to the job.

    projection: the a/b operands of a block of `block_rows` rows (all columns);
    contraction: that row block against 4 x block_rows operand rows over all N
    k values (flop-rate measurement); epilogue: a block_rows x block_rows
    block of pairs.  Projection and epilogue scale with N^2 pairs, the
    contraction with 2 N^3 c flops.
    """
    import numpy as np
    import oracle
    import workloads as wl
    threads = blas_threads()
    n = work.n
    rb = block_rows
    w = wl.weights_f64(wl.make_weights(work.c_z, work.c, work.seed, work.dtype))
    z = wl.make_pair_tensor(n, work.c_z, work.seed, work.dtype, "cpu", rows=range(0, rb),
                            chains=wl.chain_ids(work), offsets=wl.chain_offsets(work)).double().numpy()
    m = np.ones((rb, n), np.uint8)
    t0 = time.perf_counter()
    a, b = oracle.project(z, m, w, quant=True)
    t1 = time.perf_counter()
    b4 = np.concatenate([b] * 4)
    x = oracle.contract_rows(a, b4)
    t2 = time.perf_counter()
    oracle.finish(x[:, :rb], z[:, :rb], m[:, :rb], w)
    t3 = time.perf_counter()
    t_proj = (t1 - t0) * (n * n) / (rb * n)
    t_con = (t2 - t1) * (2.0 * n ** 3 * C) / (2.0 * rb * 4 * rb * n * C)
    t_epi = (t3 - t2) * (n * n) / (rb * rb)
    t_dir = t_proj + t_con + t_epi
    return {
        "value": (2 * n * n) / (2 * t_dir),
        "unit": "pair-updates/s",
        "cores": int(threads),
        "kind": "oracle",
        "host": host_cpu(threads),
        "sample": (f"float64 oracle phases on blocks of {work.name}: projection of {rb}x{n} pairs "
                   f"{t1 - t0:.2f}s, contraction {rb}x{4 * rb}x{n}x128 {t2 - t1:.2f}s, epilogue {rb}x{rb} "
                   f"pairs {t3 - t2:.2f}s; extrapolated (projection, epilogue x N^2; contraction x N^3) "
                   f"to {t_dir:.0f}s per direction"),
    }


def bench_tile(work, args, dev):
    """The per-device step of the tiled form: operand chunks for one tile
    (K1), the k-contraction over all chunks in ring order (K2) and the
    epilogue (K3), timed per kernel with HIP events on the launch stream.
    The rate is the tile's pair updates over K2 + K3 (the chunks of a real
    grid arrive from other devices); K1 is reported separately."""
    import torch

    import pair_representation_amd as pra
    import workloads as wl

    t = work.tile
    log(f"[bench] generating {work.name} (N={work.n}) on the GPU")
    z, mask, wts = wl.make_inputs(work, dev)
    w = pra.Weights(wts, pra.BF16 if work.dtype == "bf16" else pra.F32, device=dev)
    ld = (t["chunk"] + 63) // 64 * 64
    rows, cols = t["n_rows"], t["n_cols"]
    res = {}
    for d, name in ((pra.OUTGOING, "outgoing"), (pra.INCOMING, "incoming")):
        a_ops = [pra.new_operand(rows, ld, w.torch_dtype, dev) for _ in range(t["n_chunks"])]
        b_ops = [pra.new_operand(cols, ld, w.torch_dtype, dev) for _ in range(t["n_chunks"])]
        x = pra.new_xacc(rows, cols, dev)
        out = torch.empty((rows, cols, C_Z), dtype=torch.float32, device=dev)
        chunks = [(c * t["chunk"], t["chunk"], a_ops[c], b_ops[c]) for c in range(t["n_chunks"])]

        def run(ev=None):
            if ev is not None:
                ev[0].record()
            for c in range(t["n_chunks"]):
                pra.tile_operands(w, d, z, mask, t["row_off"], rows, t["col_off"], cols, c * t["chunk"],
                                  t["chunk"], ld, a_out=a_ops[c], b_out=b_ops[c])
            if ev is not None:
                ev[1].record()
            pra.tile(w, work.n, t["row_off"], rows, t["col_off"], cols, chunks, pra.TILE_FIRST, x)
            if ev is not None:
                ev[2].record()
            pra.tile(w, work.n, t["row_off"], rows, t["col_off"], cols, [], pra.TILE_LAST, x, z, mask, out)
            if ev is not None:
                ev[3].record()

        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        evs = []
        for _ in range(args.steps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            run(ev)
            evs.append(ev)
        torch.cuda.synchronize()
        k = [sum(ev[i].elapsed_time(ev[i + 1]) for ev in evs) / len(evs) * 1e-3 for i in range(3)]
        flops = 2.0 * rows * cols * t["chunk"] * t["n_chunks"] * C
        res[name] = {"tile_pair_updates_per_s": rows * cols / (k[1] + k[2]),
                     "k1_operands_ms": k[0] * 1e3, "k2_contract_ms": k[1] * 1e3, "k3_epilogue_ms": k[2] * 1e3,
                     "k2_TFLOP/s": flops / k[1] / 1e12, "k2_frac": flops / k[1] / 1e12 / PEAK_BF16_TFLOPS}
        del a_ops, b_ops, x, out, chunks
        torch.cuda.empty_cache()
    both = 2 * rows * cols / sum(res[nm]["k2_contract_ms"] + res[nm]["k3_epilogue_ms"] for nm in res) * 1e3
    return {"metric": "TriMul tile pair-updates/s over contraction + epilogue (operand chunks timed apart)",
            "value": both, "unit": "pair-updates/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "dtype": work.dtype, "data": "synthetic",
            "config": {"workload": work.name, "n": work.n, "tile": t}, "directions": res}


def bench_chunked(work, args, dev):
    """The memory-bounded forward (trimul_forward_chunked) on a grid whose
    whole-grid workspace does not fit beside z and the output: both
    directions, timed with HIP events on the launch stream around each call.
    Reports pair updates per second, the device memory held (z, mask, out and
    the workspace) against the whole-grid path's, and the contraction's
    matrix-core rate over the whole call (a lower bound: the call also runs
    the projections, rebuilt per row block, and the epilogue)."""
    import torch

    import pair_representation_amd as pra
    import workloads as wl

    n = work.n
    cb = work.chunked
    log(f"[bench] generating {work.name} (N={n}) on the GPU")
    z, mask, wts = wl.make_inputs(work, dev)
    w = pra.Weights(wts, pra.BF16 if work.dtype == "bf16" else pra.F32, device=dev)
    blocks = (cb["row_block"], cb["col_block"], cb["k_block"])
    ws = torch.empty(pra.chunked_workspace_bytes(w, n, *blocks), dtype=torch.uint8, device=dev)
    out = torch.empty((n, n, C_Z), dtype=torch.float32, device=dev)
    res = {}
    for d, name in ((pra.OUTGOING, "outgoing"), (pra.INCOMING, "incoming")):
        for _ in range(args.warmup):
            pra.forward_chunked(z, mask, w, d, *blocks, workspace=ws, out=out)
        torch.cuda.synchronize()
        evs = []
        for _ in range(args.steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record()
            pra.forward_chunked(z, mask, w, d, *blocks, workspace=ws, out=out)
            e[1].record()
            evs.append(e)
        torch.cuda.synchronize()
        t = sum(e[0].elapsed_time(e[1]) for e in evs) / len(evs) * 1e-3
        res[name] = {"ms": t * 1e3, "pair_updates_per_s": n * n / t,
                     "contraction_TFLOP/s_over_call": 2.0 * n ** 3 * C / t / 1e12}
        log(f"[bench] {name}: {t * 1e3:.1f} ms")
    io = z.numel() * z.element_size() + mask.numel() + out.numel() * 4
    t_both = sum(r["ms"] for r in res.values()) * 1e-3
    return {"metric": "TriMul pair-updates/s, memory-bounded form (both directions)", "value": 2 * n * n / t_both,
            "unit": "pair-updates/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": t_both * 1e3, "higher_is_better": True, "dtype": work.dtype, "data": "synthetic",
            "config": {"workload": work.name, "n": n, "blocks": dict(cb)},
            "device_bytes": {"z_mask_out": io, "workspace": ws.numel(), "total": io + ws.numel(),
                             "whole_grid_path_total": io + pra.workspace_bytes(w, n),
                             "device_total": torch.cuda.get_device_properties(dev).total_memory},
            "directions": res}


def bench_backward(work, args, dev):
    """Backward of the contraction step (trimul_tile_backward) on the whole
    N x N grid as one tile and one chunk: dA = dX B and dB = dX^T A per
    channel from the workload's outgoing operands (K1 on the seeded z) and a
    seeded gradient dX, timed with HIP events on the launch stream around the
    entry point (its relayout kernels and two contractions).  The rate counts
    the N^2 pair gradients of x per call; the roofline is the two contractions'
    4 N^3 c flop over the whole call (a lower bound for the contraction
    kernels; the per-kernel split is in the committed rocprofv3 summary)."""
    import torch

    import pair_representation_amd as pra
    import workloads as wl

    n = work.n
    log(f"[bench] generating {work.name} (N={n}) on the GPU")
    z, mask, wts = wl.make_inputs(work, dev)
    w = pra.Weights(wts, pra.BF16 if work.dtype == "bf16" else pra.F32, device=dev)
    kp = (n + 63) // 64 * 64
    a_pl, b_pl = pra.tile_operands(w, pra.OUTGOING, z, mask, 0, n, 0, n, 0, n, kp)
    del z
    g = torch.Generator(device=dev).manual_seed(12345)
    dx = torch.randn(pra.xacc_shape(n, n), generator=g, device=dev)
    chunks = [(0, n, a_pl, b_pl)]
    da = [pra.new_xacc(n, n, dev)]
    db = [pra.new_xacc(n, n, dev)]
    ws = torch.empty(pra.tile_backward_workspace_bytes(w, n, n, chunks), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        pra.tile_backward(w, n, n, chunks, dx, da, db, ws)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} backward calls")
    evs = []
    for _ in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        pra.tile_backward(w, n, n, chunks, dx, da, db, ws)
        e[1].record()
        evs.append(e)
    torch.cuda.synchronize()
    t = sum(e[0].elapsed_time(e[1]) for e in evs) / len(evs) * 1e-3
    flops = 4.0 * n * n * n * C
    rec = {
        "metric": "TriMul contraction-backward pair-gradients/s (dA, dB) at N=3605, c=128 bf16 (1 GPU)",
        "value": n * n / t, "unit": "pair-gradients/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": work.dtype, "data": "synthetic (workload operands from the seeded z; seeded N(0,1) dX)",
        "config": {"workload": work.name, "n": n, "part": "contraction backward, one tile, one chunk"},
        "roofline": {"bound": "mfma", "kernel": "trimul_tile_backward (relayouts + two contractions)",
                     "achieved": flops / t / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops / t / 1e12 / PEAK_BF16_TFLOPS, "traffic": None,
                     "algorithmic_per_launch": f"4*N^3*c = {flops:.4e} flop", "avg_launch_ms": t * 1e3},
        "cpu_baseline": None,
    }
    del da, db, ws, dx, a_pl, b_pl
    torch.cuda.empty_cache()
    if args.cpu_rows > 0:
        rec["cpu_baseline"] = cpu_baseline_backward(work, args.cpu_rows)
    return rec


def cpu_baseline_backward(work, block_rows, block_k=128):
    """The oracle's contraction gradients (numpy float64 matmul on all host
    cores) on a block: dA for block_rows rows of a seeded dX against block_k
    columns of a full-height b (2 * block_rows * N * block_k * c flop),
    extrapolated to both gradients of the whole grid (4 N^3 c flop)."""
    import numpy as np

    import oracle

    n = work.n
    r = np.random.default_rng(5)
    b = r.standard_normal((n, block_k, C))
    dx = r.standard_normal((block_rows, n, C))
    a_blk = np.zeros((block_rows, block_k, C))
    t0 = time.perf_counter()
    oracle.contract_rows_vjp(a_blk, b, dx)
    t_blk = time.perf_counter() - t0
    scale = (n / block_rows) * (n / block_k) * 2.0
    t_full = t_blk * scale
    return {"value": n * n / t_full, "unit": "pair-gradients/s", "cores": os.cpu_count(), "kind": "oracle",
            "host": host_cpu(blas_threads()),
            "sample": f"oracle.contract_rows_vjp: {block_rows} rows of dX against {block_k} k-columns of a "
                      f"{n}-row b ({t_blk:.2f}s), extrapolated x{scale:.0f} to both gradients of the "
                      f"{n}x{n} grid ({t_full:.0f}s)"}


def bench_epilogue_backward(work, args, dev):
    """Backward of the epilogue (trimul_epilogue_backward) on the whole N x N
    grid as one tile: x is the workload's real contraction result (K1 + K2 on
    the seeded z, outgoing) and dout a seeded N(0,1) gradient; timed with HIP
    events on the launch stream around the entry point (transpose of the two
    matrices, the per-pair kernel, the two reduction kernels).  The rate counts
    the N^2 pairs per call; the roofline is HBM: per pair the kernel reads x
    (512 B), z (256 B bf16), the mask (1 B) and dout (512 B) and writes dx and
    dz (512 B each), 2305 B, while its six 128 x 128 products (196608 flop per
    pair) need a quarter of that time at the matrix-core peak."""
    import torch

    import pair_representation_amd as pra
    import workloads as wl

    n = work.n
    log(f"[bench] generating {work.name} (N={n}) on the GPU")
    z, mask, wts = wl.make_inputs(work, dev)
    w = pra.Weights(wts, pra.BF16 if work.dtype == "bf16" else pra.F32, device=dev)
    kp = (n + 63) // 64 * 64
    a_pl, b_pl = pra.tile_operands(w, pra.OUTGOING, z, mask, 0, n, 0, n, 0, n, kp)
    x = pra.new_xacc(n, n, dev)
    pra.tile(w, n, 0, n, 0, n, [(0, n, a_pl, b_pl)], pra.TILE_FIRST, x)
    del a_pl, b_pl
    torch.cuda.empty_cache()
    g = torch.Generator(device=dev).manual_seed(23456)
    dout = torch.randn((n, n, C_Z), generator=g, device=dev)
    dx = pra.new_xacc(n, n, dev)
    dz = torch.empty((n, n, C_Z), dtype=torch.float32, device=dev)
    grads = {k: torch.empty(shp, dtype=torch.float32, device=dev) for k, shp in pra.EPILOGUE_GRAD_SHAPES.items()}
    ws = torch.empty(pra.epilogue_backward_workspace_bytes(w), dtype=torch.uint8, device=dev)

    def call():
        pra.epilogue_backward(w, n, 0, n, 0, n, x, z, mask, dout, dx, dz, grads, ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} epilogue-backward calls")
    evs = []
    for _ in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        call()
        e[1].record()
        evs.append(e)
    torch.cuda.synchronize()
    t = sum(e[0].elapsed_time(e[1]) for e in evs) / len(evs) * 1e-3
    per_pair = 512 + (256 if work.dtype == "bf16" else 512) + 1 + 512 + 512 + 512
    nbytes = float(per_pair) * n * n
    rec = {
        "metric": "TriMul epilogue-backward pairs/s (dx, gate-path dz, parameter gradients) at N=3605, c=128 bf16 "
                  "(1 GPU)",
        "value": n * n / t, "unit": "pairs/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": work.dtype, "data": "synthetic (x from the workload's own contraction; seeded N(0,1) dout)",
        "config": {"workload": work.name, "n": n, "part": "epilogue backward, one tile"},
        "roofline": {"bound": "hbm", "kernel": "trimul_epilogue_backward (whole call)",
                     "achieved": nbytes / t / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": nbytes / t / 1e9 / PEAK_HBM_GBS, "traffic": None,
                     "algorithmic_per_launch": f"{per_pair} B/pair * N^2 = {nbytes:.4e} B", "avg_launch_ms": t * 1e3},
        "cpu_baseline": None,
    }
    del x, dout, dx, dz, ws, z, mask
    torch.cuda.empty_cache()
    if args.cpu_rows > 0:
        rec["cpu_baseline"] = cpu_baseline_epilogue_backward(work, wts)
    return rec


def bench_layer_backward(work, args, dev):
    """The whole layer's backward on the N x N grid as one tile and one
    k-chunk, from a forward run once (operands a, b and the contraction
    result x kept) and a seeded N(0,1) dL/dout: epilogue backward (dL/dx, the
    gate's dL/dz, its parameters), contraction backward (dL/da, dL/db) and
    both projection sides (their dL/dz added, their parameters), timed per part
    with HIP events on the launch stream.  The rate counts the N^2 pairs per
    backward pass; the roofline line is the contraction backward's (its two
    matrix-core contractions, 4 N^3 c flop), the dominant part."""
    import torch

    import pair_representation_amd as pra
    import workloads as wl

    n = work.n
    log(f"[bench] generating {work.name} (N={n}) on the GPU")
    z, mask, wts = wl.make_inputs(work, dev)
    w = pra.Weights(wts, pra.BF16 if work.dtype == "bf16" else pra.F32, device=dev)
    kp = (n + 63) // 64 * 64
    a_pl, b_pl = pra.tile_operands(w, pra.OUTGOING, z, mask, 0, n, 0, n, 0, n, kp)
    x = pra.new_xacc(n, n, dev)
    pra.tile(w, n, 0, n, 0, n, [(0, n, a_pl, b_pl)], pra.TILE_FIRST, x)
    chunks = [(0, n, a_pl, b_pl)]
    g = torch.Generator(device=dev).manual_seed(34567)
    dout = torch.randn((n, n, C_Z), generator=g, device=dev)
    dx = pra.new_xacc(n, n, dev)
    dz = torch.empty((n, n, C_Z), dtype=torch.float32, device=dev)
    da, db = [pra.new_xacc(n, n, dev)], [pra.new_xacc(n, n, dev)]
    g_epi = {k: torch.empty(shp, dtype=torch.float32, device=dev) for k, shp in pra.EPILOGUE_GRAD_SHAPES.items()}
    g_proj = {k: torch.empty(shp, dtype=torch.float32, device=dev) for k, shp in pra.PROJECTION_GRAD_SHAPES.items()}
    g_proj["ln_in_w"], g_proj["ln_in_b"] = g_epi["ln_in_w"], g_epi["ln_in_b"]
    ws_e = torch.empty(pra.epilogue_backward_workspace_bytes(w), dtype=torch.uint8, device=dev)
    ws_c = torch.empty(pra.tile_backward_workspace_bytes(w, n, n, chunks), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        pra.epilogue_backward(w, n, 0, n, 0, n, x, z, mask, dout, dx, dz, g_epi, ws_e)
        if ev is not None:
            ev[1].record()
        pra.tile_backward(w, n, n, chunks, dx, da, db, ws_c)
        if ev is not None:
            ev[2].record()
        for k in ("w_a_proj", "w_a_gate", "w_b_proj", "w_b_gate"):
            g_proj[k].zero_()
        pra.tile_operands_backward(w, pra.OUTGOING, z, mask, 0, n, 0, n, 0, n, da=da[0], db=db[0], dz=dz,
                                   grads=g_proj, accumulate=True, workspace=ws_e)
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} layer-backward passes")
    evs = []
    for _ in range(args.steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        step(ev)
        evs.append(ev)
    torch.cuda.synchronize()
    parts = [sum(ev[i].elapsed_time(ev[i + 1]) for ev in evs) / len(evs) * 1e-3 for i in range(3)]
    t = sum(parts)
    flops = 4.0 * n * n * n * C
    return {
        "metric": "TriMul layer-backward pairs/s (all gradients: z and the ten parameters) at N=3605, c=128 bf16 "
                  "(1 GPU)",
        "value": n * n / t, "unit": "pairs/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": work.dtype, "data": "synthetic (forward on the workload's seeded z; seeded N(0,1) dL/dout)",
        "config": {"workload": work.name, "n": n, "part": "whole-layer backward, one tile, one chunk"},
        "parts_ms": {"epilogue_backward": parts[0] * 1e3, "contraction_backward": parts[1] * 1e3,
                     "projection_backward": parts[2] * 1e3},
        "roofline": {"bound": "mfma", "kernel": "contraction backward (relayouts + two contractions)",
                     "achieved": flops / parts[1] / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops / parts[1] / 1e12 / PEAK_BF16_TFLOPS, "traffic": None,
                     "algorithmic_per_launch": f"4*N^3*c = {flops:.4e} flop", "avg_launch_ms": parts[1] * 1e3},
        "cpu_baseline": None,
    }


ATOM_WORKLOAD = {"name": "atoms_b8_n28840_h4", "batch": 8, "n_atoms": 28840, "heads": 4, "keep": 0.9}


def bench_atom_attention(args, dev):
    """Window-batched atom attention (trimul_atom_window_attention) on 8
    sequences of 28840 atoms (8 atoms per residue of the 3605-residue
    workload), 4 heads of 32, a bf16 pair bias per window and 90% of the atoms
    kept, timed with HIP events on the launch stream.  The rate counts
    query-atom outputs (all heads) per second; the roofline is HBM: q, k, v
    and the mask read once, the bias read once, the output written once (k
    and v are read by four windows each, from L2)."""
    import torch

    import pair_representation_amd as pra

    cfg = ATOM_WORKLOAD
    bsz, n, heads = cfg["batch"], cfg["n_atoms"], cfg["heads"]
    nw = (n + 31) // 32
    g = torch.Generator(device=dev).manual_seed(45678)
    q, k, v = (torch.randn((bsz, n, heads, 32), generator=g, device=dev).to(torch.bfloat16) for _ in range(3))
    bias = torch.randn((bsz, nw, heads, 32, 128), generator=g, device=dev).to(torch.bfloat16)
    mask = (torch.rand((bsz, n), generator=g, device=dev) < cfg["keep"]).to(torch.uint8)
    out = torch.empty((bsz, n, heads, 32), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        pra.atom_window_attention(q, k, v, bias, mask, out=out)
    torch.cuda.synchronize()
    evs = []
    for _ in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        pra.atom_window_attention(q, k, v, bias, mask, out=out)
        e[1].record()
        evs.append(e)
    torch.cuda.synchronize()
    t = sum(e[0].elapsed_time(e[1]) for e in evs) / len(evs) * 1e-3
    nbytes = float(3 * bsz * n * heads * 32 * 2 + bsz * nw * heads * 32 * 128 * 2 + bsz * n + bsz * n * heads * 32 * 4)
    flops = 2.0 * 2 * bsz * nw * heads * 32 * 128 * 32
    rec = {
        "metric": "Atom window-attention query-atoms/s (32 x 128 windows, 4 heads of 32, pair bias) (1 GPU)",
        "value": bsz * n / t, "unit": "query-atoms/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q, k, v and bias; 90% of atoms kept)",
        "config": {"workload": cfg["name"], "batch": bsz, "n_atoms": n, "heads": heads, "head_dim": 32,
                   "windows": f"{nw} x 32 queries x 128 keys per sequence"},
        "roofline": {"bound": "hbm", "kernel": "ka_window_attention", "achieved": nbytes / t / 1e9,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": nbytes / t / 1e9 / PEAK_HBM_GBS, "traffic": None,
                     "algorithmic_per_launch": f"{nbytes:.4e} B", "avg_launch_ms": t * 1e3,
                     "matrix_core_TFLOP/s": flops / t / 1e12},
        "cpu_baseline": None,
    }
    if args.cpu_rows > 0:
        rec["cpu_baseline"] = cpu_baseline_atom_attention(cfg)
    return rec


def cpu_baseline_atom_attention(cfg, n_sample=28840):
    """oracle.atom_attention.window_attention (numpy float64) on one seeded
    sequence of n_sample atoms, extrapolated to the workload's query atoms."""
    import numpy as np

    from oracle import atom_attention as aa

    r = np.random.default_rng(7)
    heads = cfg["heads"]
    q, k, v = (r.standard_normal((1, n_sample, heads, 32)) for _ in range(3))
    bias = r.standard_normal((1, aa.n_windows(n_sample), heads, 32, 128))
    mask = (r.random((1, n_sample)) < cfg["keep"]).astype(np.uint8)
    t0 = time.perf_counter()
    aa.window_attention(q, k, v, bias, mask)
    dt = time.perf_counter() - t0
    rate = n_sample / dt
    total = cfg["batch"] * cfg["n_atoms"]
    return {"value": rate, "unit": "query-atoms/s", "cores": os.cpu_count(), "kind": "oracle",
            "host": host_cpu(blas_threads()),
            "sample": f"oracle window_attention on one sequence of {n_sample} atoms ({dt:.2f}s); the "
                      f"{total} query atoms of the workload would take {total / rate:.0f}s"}


def cpu_baseline_epilogue_backward(work, wts, block=65536, blocks=4):
    """oracle.finish_vjp (numpy float64 on the host cores) on ``blocks``
    blocks of ``block`` seeded pairs, extrapolated to the N^2 pairs."""
    import numpy as np

    import oracle

    r = np.random.default_rng(6)
    wref = {k: v.double().cpu().numpy() for k, v in wts.items()}
    t_sum = 0.0
    for _ in range(blocks):
        x = r.standard_normal((block, C))
        zz = r.standard_normal((block, C_Z))
        m = (r.random(block) < 0.9).astype(np.uint8)
        d = r.standard_normal((block, C_Z))
        t0 = time.perf_counter()
        oracle.finish_vjp(x, zz, m, wref, d)
        t_sum += time.perf_counter() - t0
    rate = block * blocks / t_sum
    n = work.n
    return {"value": rate, "unit": "pairs/s", "cores": os.cpu_count(), "kind": "oracle",
            "host": host_cpu(blas_threads()),
            "sample": f"oracle.finish_vjp on {blocks} blocks of {block} seeded pairs ({t_sum:.2f}s); the "
                      f"{n}x{n} grid would take {n * n / rate:.0f}s"}


CONTRACTION_SHAPES = ((3605, 3605, 3605), (3584, 3456, 3605), (3584, 3605, 3605), (3605, 3456, 3605),
                      (3840, 3840, 3605))


def bench_contraction_shapes(args, dev):
    """The contraction kernel alone (trimul_tile with one chunk, FIRST) on
    rows x cols x k shapes around the n3605_4ch grid: the full grid, the same
    grid cut to whole 256 x 384 tiles (3584 x 3456), each ragged edge alone,
    and the grid padded to whole tiles (3840 x 3840).  Operands come from K1
    on a seeded 3840-residue pair tensor; medians of HIP-event timings on the
    launch stream.  The differences give what the ragged tile column and row
    cost against their share of the work."""
    import torch

    import pair_representation_amd as pra
    import workloads as wl

    n = 3840
    z = wl.make_pair_tensor(n, C_Z, 7, "bf16", dev)
    mask = torch.ones((n, n), dtype=torch.uint8, device=dev)
    w = pra.Weights(wl.make_weights(C_Z, C, 7, "bf16"), pra.BF16, device=dev)
    res = []
    for (m, nc, k) in CONTRACTION_SHAPES:
        ld = (k + 63) // 64 * 64
        a, b = pra.tile_operands(w, pra.OUTGOING, z, mask, 0, m, 0, nc, 0, k, ld)
        x = pra.new_xacc(m, nc, dev)
        ch = [(0, k, a, b)]
        for _ in range(max(args.warmup, 1)):
            pra.tile(w, n, 0, m, 0, nc, ch, pra.TILE_FIRST, x)
        torch.cuda.synchronize()
        evs = []
        for _ in range(args.steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record()
            pra.tile(w, n, 0, m, 0, nc, ch, pra.TILE_FIRST, x)
            e[1].record()
            evs.append(e)
        torch.cuda.synchronize()
        ts = sorted(e[0].elapsed_time(e[1]) for e in evs)
        t = ts[len(ts) // 2] * 1e-3
        fl = 2.0 * m * nc * k * C
        res.append({"rows": m, "cols": nc, "k": k, "ms": t * 1e3, "TFLOP/s": fl / t / 1e12,
                    "frac": fl / t / 1e12 / PEAK_BF16_TFLOPS})
        log(f"[shapes] {m} x {nc} x {k}: {t * 1e3:.3f} ms, {fl / t / 1e12:.0f} TFLOP/s")
        del a, b, x
        torch.cuda.empty_cache()
    return {"mode": "contraction-shapes", "metric": "contraction kernel time by tile shape", "dtype": "bf16",
            "data": "synthetic (seeded 3840-residue pair tensor)", "steps": args.steps, "shapes": res}


STREAM_MIXES = (("read", 1, 0), ("write", 0, 1), ("copy", 1, 1), ("k1_mix_1r_2w", 1, 2), ("k3_mix_3r_2w", 3, 2))


def bench_peaks(args, dev):
    """Achievable peaks on this GPU (libtrimul_peaks.so): the bf16
    matrix-core loop (no memory traffic; each wave also reads the shader
    clock and the real-time counter, giving the clock it ran at) and streaming
    kernels at the byte mixes of the projection (1 read : 2 written) and
    epilogue (3 : 2) kernels, plus plain read, write and copy; each streaming
    launch moves about 6 GiB (far beyond the 256 MB last-level cache) and is
    run as a grid-stride loop (plain or non-temporal accesses, 4 or 8
    elements in flight per thread, 4 to 32 work-groups per CU) and in a
    one-shot form (one element per thread over a covering grid, plain or
    non-temporal), the best average reported per mix.  Times are HIP events
    on the launch stream."""
    import ctypes

    import torch

    from pair_representation_amd import build as pbuild

    if not os.path.exists(pbuild.PEAKS_LIB):
        raise RuntimeError(f"{pbuild.PEAKS_LIB} is missing: build it with `python -m pair_representation_amd.build`")
    L = ctypes.CDLL(pbuild.PEAKS_LIB)
    vp = ctypes.c_void_p
    L.peaks_mfma.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp]
    L.peaks_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_longlong, vp,
                               ctypes.c_int, vp]
    L.peaks_wall_clock_khz.restype = ctypes.c_int
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    khz = L.peaks_wall_clock_khz()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            fn()
            e[1].record(stream)
            evs.append(e)
        torch.cuda.synchronize()
        return sum(e[0].elapsed_time(e[1]) for e in evs) / reps * 1e-3

    out = {"cus": cus, "wall_clock_khz": khz}
    # matrix-core loop: one 8-wave work-group per CU, sized to run ~40 ms
    blocks, iters = cus, 120000
    sink = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    clk = torch.zeros(blocks * 8 * 2, dtype=torch.int64, device=dev)

    def mfma():
        st = L.peaks_mfma(blocks, iters, vp(sink.data_ptr()), vp(clk.data_ptr()), sp)
        if st != 0:
            raise RuntimeError(f"peaks_mfma: hip error {st}")

    t = timed(mfma, 3)
    flops = float(blocks) * 8 * iters * 8 * 32768
    c = clk.view(-1, 2).double()
    clock_ghz = float(c[:, 0].sum() / c[:, 1].sum()) * khz * 1e-6 if khz > 0 else None
    out["mfma_bf16"] = {"TFLOP/s": flops / t / 1e12, "frac_of_2500": flops / t / 1e12 / PEAK_BF16_TFLOPS,
                        "ms": t * 1e3, "shader_clock_GHz": clock_ghz,
                        "kernel": "peak_mfma: 8 independent 32x32x16 bf16 chains per wave, 2 waves per SIMD"}
    log(f"[peaks] mfma {out['mfma_bf16']['TFLOP/s']:.0f} TFLOP/s at {clock_ghz} GHz")
    # streaming kernels
    total = 6 << 30
    u32sink = torch.zeros(4, dtype=torch.int32, device=dev)
    res = {}
    for name, r, w in STREAM_MIXES:
        units = total // (16 * (r + w))
        src = torch.empty(max(r, 1) * units * 16, dtype=torch.uint8, device=dev) if r else None
        if src is not None:
            src.fill_(7)
        dst = torch.empty(w * units * 16, dtype=torch.uint8, device=dev) if w else None
        best = None
        forms = [(v, pc) for v in range(4) for pc in (4, 8, 16, 32)] + [(4, 0), (5, 0)]
        for variant, per_cu in forms:
            nb = cus * max(per_cu, 1)

            def run():
                st = L.peaks_stream(r, w, variant, vp(src.data_ptr() if src is not None else 0),
                                    vp(dst.data_ptr() if dst is not None else 0), units,
                                    vp(u32sink.data_ptr()), nb, sp)
                if st != 0:
                    raise RuntimeError(f"peaks_stream: hip error {st}")

            tt = timed(run, 5)
            gbs = (r + w) * units * 16 / tt / 1e9
            if best is None or gbs > best["GB/s"]:
                best = {"GB/s": gbs, "frac_of_8000": gbs / PEAK_HBM_GBS, "ms": tt * 1e3,
                        "blocks": (units + 255) // 256 if variant >= 4 else nb,
                        "form": "one element per thread" if variant >= 4 else
                                f"{8 if variant & 2 else 4} elements per thread and step",
                        "nontemporal": bool(variant & 1),
                        "bytes_read": r * units * 16, "bytes_written": w * units * 16}
        res[name] = best
        log(f"[peaks] {name}: {best['GB/s']:.0f} GB/s ({best['blocks']} blocks)")
        del src, dst
        torch.cuda.empty_cache()
    out["stream"] = res
    # the runtime's own device copy (torch copy_ -> HIP's copy kernel), for reference
    nb = 3 << 30
    a_t = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b_t = torch.empty_like(a_t)
    tt = timed(lambda: b_t.copy_(a_t), 5)
    out["runtime_copy"] = {"GB/s": 2 * nb / tt / 1e9, "frac_of_8000": 2 * nb / tt / 1e9 / PEAK_HBM_GBS,
                           "ms": tt * 1e3, "bytes_read": nb, "bytes_written": nb}
    log(f"[peaks] runtime copy: {out['runtime_copy']['GB/s']:.0f} GB/s")
    del a_t, b_t
    torch.cuda.empty_cache()
    return {"mode": "peaks", "metric": "achievable peaks (matrix-core loop, streaming kernels)", **out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="n3605_4ch")
    ap.add_argument("--cpu-rows", type=int, default=256, help="row block for the CPU baseline (0 = skip)")
    ap.add_argument("--mode", default="bench",
                    choices=["bench", "copy", "peaks", "contraction-shapes", "backward", "epilogue-backward", "layer-backward", "atom-attention"],
                    help="copy: a plain 1 GiB device copy by the streaming probe kernel (counter calibration); "
                         "peaks: achievable matrix-core and streaming peaks (libtrimul_peaks.so); "
                         "contraction-shapes: the contraction kernel on whole-tile and ragged shapes; "
                         "backward: the contraction step's gradients (trimul_tile_backward); "
                         "epilogue-backward: the epilogue's gradients (trimul_epilogue_backward); "
                         "layer-backward: every gradient of the layer (the three backward entry points); "
                         "atom-attention: window-batched atom attention (trimul_atom_window_attention)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(collectives and sharding are out of scope); use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import pair_representation_amd as pra
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.mode == "copy":
        # a plain copy of known size through the streaming probe kernel of
        # libtrimul_peaks.so (one 16-byte load and one 16-byte store per
        # lane), for calibrating the FETCH_SIZE / WRITE_SIZE counters
        import ctypes

        from pair_representation_amd import build as pbuild
        L = ctypes.CDLL(pbuild.PEAKS_LIB)
        vp = ctypes.c_void_p
        L.peaks_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_longlong, vp,
                                   ctypes.c_int, vp]
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        sink = torch.zeros(4, dtype=torch.int32, device=dev)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        for _ in range(3):
            st = L.peaks_stream(1, 1, 0, vp(src.data_ptr()), vp(dst.data_ptr()), nbytes // 16, vp(sink.data_ptr()),
                                cus * 8, vp(torch.cuda.current_stream(dev).cuda_stream))
            if st != 0:
                raise RuntimeError(f"peaks_stream: hip error {st}")
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "kernel": "stream_rw<1, 1, 4, false>", "bytes_read_per_launch": nbytes,
                          "bytes_written_per_launch": nbytes, "launches": 3}), flush=True)
        return
    if args.mode == "atom-attention":
        print(json.dumps(bench_atom_attention(args, dev)), flush=True)
        return
    if args.mode == "peaks":
        print(json.dumps(bench_peaks(args, dev)), flush=True)
        return
    if args.mode == "contraction-shapes":
        print(json.dumps(bench_contraction_shapes(args, dev)), flush=True)
        return
    work = wl.WORKLOADS[args.workload]
    if args.mode == "backward":
        print(json.dumps(bench_backward(work, args, dev)), flush=True)
        return
    if args.mode == "epilogue-backward":
        print(json.dumps(bench_epilogue_backward(work, args, dev)), flush=True)
        return
    if args.mode == "layer-backward":
        print(json.dumps(bench_layer_backward(work, args, dev)), flush=True)
        return
    if work.tile:
        print(json.dumps(bench_tile(work, args, dev)), flush=True)
        return
    if work.chunked:
        print(json.dumps(bench_chunked(work, args, dev)), flush=True)
        return
    n = work.n
    log(f"[bench] generating {work.name} (N={n}) on the GPU")
    z, mask, wts = wl.make_inputs(work, dev)
    w = pra.Weights(wts, pra.BF16 if work.dtype == "bf16" else pra.F32, device=dev)
    ws = pra.new_workspace(w, n, dev)
    out_o = torch.empty((n, n, C_Z), dtype=torch.float32, device=dev)
    out_i = torch.empty_like(out_o)
    # the workspace of the entry points, viewed as the buffers the kernels use:
    # a and b operands (operand layout), then the contraction result
    kp = (n + 63) // 64 * 64
    td = w.torch_dtype
    op_bytes = pra.tile_operand_bytes(w, n, kp)
    plane = (op_bytes + 255) // 256 * 256
    xbytes = pra.tile_xacc_bytes(w, n, n)
    a_pl = ws[:op_bytes].view(td).view(pra.operand_shape(n, kp))
    b_pl = ws[plane:plane + op_bytes].view(td).view(pra.operand_shape(n, kp))
    x = ws[2 * plane:2 * plane + xbytes].view(torch.float32).view(pra.xacc_shape(n, n))
    torch.cuda.synchronize()

    def step_api():
        pra.outgoing(z, mask, w, workspace=ws, out=out_o)
        pra.incoming(z, mask, w, workspace=ws, out=out_i)

    def step_kernels(ev=None):
        for d, out in ((pra.OUTGOING, out_o), (pra.INCOMING, out_i)):
            if ev is not None:
                ev[d][0].record()
            pra.tile_operands(w, d, z, mask, 0, n, 0, n, 0, n, kp, a_out=a_pl, b_out=b_pl)
            if ev is not None:
                ev[d][1].record()
            pra.tile(w, n, 0, n, 0, n, [(0, n, a_pl, b_pl)], pra.TILE_FIRST, x)
            if ev is not None:
                ev[d][2].record()
            pra.tile(w, n, 0, n, 0, n, [], pra.TILE_LAST, x, z, mask, out)
            if ev is not None:
                ev[d][3].record()

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step_api()
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps (entry points)")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_api()
    torch.cuda.synchronize()
    t_api = (time.perf_counter() - t0) / args.steps

    log(f"[bench] timing {args.steps} steps (per-kernel events)")
    for _ in range(args.warmup):
        step_kernels()
    torch.cuda.synchronize()
    durs = {"k1": [], "k2": [], "k3": []}
    t0 = time.perf_counter()
    all_ev = []
    for _ in range(args.steps):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(2)]
        step_kernels(ev)
        all_ev.append(ev)
    torch.cuda.synchronize()
    t_kern = (time.perf_counter() - t0) / args.steps
    for ev in all_ev:
        for d in range(2):
            durs["k1"].append(ev[d][0].elapsed_time(ev[d][1]) * 1e-3)
            durs["k2"].append(ev[d][1].elapsed_time(ev[d][2]) * 1e-3)
            durs["k3"].append(ev[d][2].elapsed_time(ev[d][3]) * 1e-3)
    avg = {k: sum(v) / len(v) for k, v in durs.items()}
    per_dir = {}
    for d, name in ((0, "outgoing"), (1, "incoming")):
        t_dir = [ev[d][0].elapsed_time(ev[d][3]) * 1e-3 for ev in all_ev]
        per_dir[name] = {"pair_updates_per_s": n * n / (sum(t_dir) / len(t_dir)),
                         "ms_median": 1e3 * sorted(t_dir)[len(t_dir) // 2], "ms_min": 1e3 * min(t_dir)}

    pairs = n * n
    k2_flops = 2.0 * n * n * n * C
    k2_tflops = k2_flops / avg["k2"] / 1e12
    # the contraction's peak in its own arithmetic type
    k2_peak = PEAK_BF16_TFLOPS if work.dtype == "bf16" else PEAK_FP32_TFLOPS
    elt = 2 if work.dtype == "bf16" else 4
    k1_bpp, k3_bpp = k1_bytes_per_pair(elt), k3_bytes_per_pair(elt)
    k1_gbs = k1_bpp * pairs / avg["k1"] / 1e9
    k3_gbs = k3_bpp * pairs / avg["k3"] / 1e9
    traffic = traffic_from_profile(os.path.join(ROOT, "pair_representation_amd", "csrc", "k2_contract.hip"))
    ceil = measured_ceilings()

    def vs_ceiling(rate, key):
        return None if key not in ceil else {"ceiling": ceil[key], "frac_of_ceiling": rate / ceil[key],
                                             "ceiling_source": f"profiles/peaks_mi355x.md ({key})"}

    value = 2 * pairs / t_api
    rec = {
        "metric": "TriMul pair-updates/s and MFMA util % at N=3605,c_z=128 bf16 (1 GPU)",
        "value": value,
        "unit": "pair-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_api * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": work.dtype,
        "data": "synthetic (seeded z ~ N(0,1) + inter-chain offset vectors, Xavier-normal weights)",
        "config": {"workload": work.name, "n": n, "c_z": C_Z, "c": C, "chains": list(work.chains),
                   "directions": ["outgoing", "incoming"], "pair_updates_per_step": 2 * pairs},
        "mfma_util_pct": 100.0 * k2_tflops / k2_peak,
        "roofline": {
            "bound": "mfma",
            "kernel": "k2_contract (channel-batched k-contraction)",
            "achieved": k2_tflops,
            "peak": k2_peak,
            "unit": "TFLOP/s",
            "frac": k2_tflops / k2_peak,
            "traffic": traffic,
            "traffic_kind": "L2-miss (fabric) bytes per launch: L2 FETCH_SIZE and WRITE_SIZE calibrated on a plain "
                            "copy; includes Infinity-Cache hits, so an upper bound on DRAM bytes",
            "algorithmic_per_launch": f"2*N^3*c = {k2_flops:.4e} flop",
            "avg_launch_ms": avg["k2"] * 1e3,
            "vs_measured_mfma_loop": vs_ceiling(k2_tflops, "mfma_bf16"),
        },
        "kernels": {
            "k1_project": {"avg_ms": avg["k1"] * 1e3, "bound": "hbm", "GB/s": k1_gbs,
                           "frac": k1_gbs / PEAK_HBM_GBS, "bytes_per_pair": k1_bpp,
                           "TFLOP/s": K1_FLOPS_PER_PAIR * pairs / avg["k1"] / 1e12,
                           "vs_measured_stream": vs_ceiling(k1_gbs, "k1_mix_1r_2w")},
            "k2_contract": {"avg_ms": avg["k2"] * 1e3, "bound": "mfma", "TFLOP/s": k2_tflops,
                            "frac": k2_tflops / k2_peak},
            "k3_epilogue": {"avg_ms": avg["k3"] * 1e3, "bound": "hbm", "GB/s": k3_gbs,
                            "frac": k3_gbs / PEAK_HBM_GBS, "bytes_per_pair": k3_bpp,
                            "TFLOP/s": K3_FLOPS_PER_PAIR * pairs / avg["k3"] / 1e12,
                            "vs_measured_stream": vs_ceiling(k3_gbs, "k3_mix_3r_2w")},
            "per_kernel_loop_ms_per_step": t_kern * 1e3,
        },
        "per_direction": per_dir,
        "cpu_baseline": None,
    }
    n_valid = int(wl.residue_mask(work).sum())
    if n_valid < n:
        # the same time counted over the pairs of unmasked residues only
        # (padding and masked residues still cost their share of the work)
        rec["valid_view"] = {"n_valid": n_valid, "valid_pair_updates_per_s": value * (n_valid / n) ** 2}
    del ws, out_o, out_i, z, mask
    torch.cuda.empty_cache()
    if args.cpu_rows > 0:
        log(f"[bench] CPU oracle baseline on a {args.cpu_rows}-row block")
        rec["cpu_baseline"] = cpu_baseline(work, args.cpu_rows)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
