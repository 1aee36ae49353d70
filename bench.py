"""Benchmark of the block-quantized matmul hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic
Qwen2.5-7B-shaped inputs (weights N(0, 0.02) quantized to Q4_K, activations
N(0, 1)):

  decode  : mq_gemv Q4_K ffn_up 18944x3584 and ffn_down 3584x18944 at M=1
  prefill : mq_quantize_act 512x3584, then mq_gemm (MMQ) with the Q4_K
            ffn_up 18944x3584, attn_q 3584x3584, attn_k and attn_v 512x3584

Inputs are resident in HBM before timing starts.  Each GEMV weight is kept in
several copies, and consecutive steps rotate through them, so every GEMV launch
reads its weights from HBM and not from the 256 MB last-level cache.  Each step
is recorded once into a HIP graph (one graph per weight copy); the timed region
replays exactly --steps of them, bracketed by HIP events on the launch stream.
Per-kernel times come from graphs of one kernel's launches back to back.

Printed JSON line (one GPU):
  value        Q4_K GEMV weight GB/s: GGUF payload bytes of the two decode
               GEMVs / their summed kernel time
  mmq_prefill_tops   2*M*N*K of the four MMQ launches / their kernel time
  roofline     the Q4_K GEMV against 8 TB/s HBM and against a plain read of the
               same bytes with the same workgroup count (libmq_measure.so):
               achieved = algorithmic bytes (payload + x + y) per launch / mean
               launch time; traffic = HBM bytes per launch from the committed
               rocprofv3 FETCH_SIZE / WRITE_SIZE summary under profiles/, null
               once any kernel source differs from the ones it was taken on
  roofline_mmq the ffn_up MMQ against 5.0 POP/s (dense int8; the fp6 block dots cost
               what the int8 ones do), with the
               matrix-unit busy fraction and clock from the committed counters
  warm_cache   the decode GEMVs with one weight copy (weights resident in the
               last-level cache): labelled, never the value
  c5_14b       Qwen2.5-14B layer mix at M=1 (GEMV) and M=2048 (quantize + MMQ)
  secondary    Q6_K vocab-head and Q8_0 GEMV GB/s, other types, the quantizer
  cpu_baseline the CPU oracle (as written) on the same decode weights, on all
               host cores (rows split over processes) and on one thread, with
               the CPU model; plus oracle times for the head GEMV, the M=512 MMQ
               and quantize_act on stated samples.  Runs before the GPU is used.

--counters skips timing: every kernel of the step runs a few times eagerly,
next to a plain 256 MiB device copy that calibrates the HBM byte counters.
"""

import argparse
import json
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
INT8_PEAK_TOPS = 5000.0
LLC_BYTES = 256 * 2 ** 20
COPY_REF_BYTES = 256 * 2 ** 20

Q8_0, Q4_K, Q6_K = 8, 12, 14
REPACKED = 0x100   # type flag of the layout mq_repack writes (Q4_K: the MMQ plane)
ROW_TILED = 0x200  # type flag of Q4_K's row-tiled layout (the long-row GEMV)
DECODE = [("ffn_up", 18944, 3584), ("ffn_down", 3584, 18944)]
PREFILL_M = 512
PREFILL = [("ffn_up", 18944, 3584), ("attn_q", 3584, 3584), ("attn_k", 512, 3584), ("attn_v", 512, 3584)]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20, help="timed replays of the step graph")
    p.add_argument("--warmup", type=int, default=3, help="untimed replays before timing")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--counters", action="store_true",
                   help="no timing: launch each kernel of the step a few times eagerly, plus a plain "
                        "device copy of known size, for rocprofv3 --pmc passes")
    return p.parse_args()


def kernel_sources_sha256():
    """sha256 over every kernel source of libmq (all of csrc/, in name order)."""
    import hashlib
    import os
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "block_quantized_matmul_mq_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def recorded_fields(summary):
    """`key: value` fields of a committed rocprofv3 summary under profiles/, or {}.

    A summary records the sha256 of the kernel sources it was taken on; once any
    source changes, its figures no longer describe the kernels and {} is returned.
    """
    import os
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        lines = open(os.path.join(root, "profiles", summary)).read().splitlines()
    except OSError:
        return {}
    fields = dict(line.split(": ", 1) for line in lines if ": " in line and not line.startswith((" ", "#")))
    if fields.get("kernel_source_sha256") != kernel_sources_sha256():
        return {}
    return fields


def recorded_traffic(summary):
    v = recorded_fields(summary).get("traffic_bytes_per_launch")
    return int(v) if v is not None else None


def copies_for(nbytes):
    """Copies so that one rotation reads at least twice the last-level cache."""
    return max(2, -(-2 * LLC_BYTES // nbytes))


# Arrays the CPU-baseline workers read (set before the worker processes fork).
_CPU = {}


def _cpu_work(task):
    """One piece of oracle work: (kind, lo, hi) rows (or columns) of a workload."""
    import oracle
    from threadpoolctl import threadpool_limits
    kind, lo, hi = task
    with threadpool_limits(limits=1):
        if kind == "gemv_up":
            oracle.gemv(_CPU["w_up"][lo:hi], Q4_K, _CPU["x_up"], hi - lo, 3584)
        elif kind == "gemv_down":
            oracle.gemv(_CPU["w_down"][lo:hi], Q4_K, _CPU["x_down"], hi - lo, 18944)
        elif kind == "gemv_head":
            oracle.gemv(_CPU["head"][lo:hi], Q6_K, _CPU["x_head"], hi - lo, 3584)
        elif kind == "mmq":
            q, d = _CPU["q8"]
            oracle.mmq(_CPU["w_up"][lo:hi], Q4_K, q, d, hi - lo, 3584)
        elif kind == "quantize":
            oracle.quantize_act(_CPU["X"][lo:hi])
    return 0


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w_up, w_down, x_up, x_down, X):
    """The oracle, as written, on the host cores: the decode GEMV pair (the line's value is
    the all-core rate), and the head GEMV, the M=512 MMQ and quantize_act on stated samples.

    All cores: the rows (columns for the MMQ) are split evenly over one worker process per
    core, each running the oracle with one BLAS thread; one thread: the same calls in this
    process.  Median of 3 runs each.  Called before the GPU is touched, so the workers fork
    from a process that has not initialised HIP."""
    import multiprocessing
    import os

    from block_quantized_matmul_mq_amd import synth
    import oracle

    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(affinity, 16))   # the host share of one GPU is 16 cores
    head_rows = 8192                      # sample of the 152064-row Q6_K head
    mmq_cols = 2048                       # sample of the 18944 ffn_up columns, all 512 rows
    _CPU.update(w_up=w_up, w_down=w_down, x_up=x_up, x_down=x_down, X=X,
                head=synth.quantized_weight(Q6_K, head_rows, 3584, 2, 0),
                x_head=synth.activations(1, 3584, 2)[0])
    q, d, _ = oracle.quantize_act(X)
    _CPU["q8"] = (q, d)

    def split(kind, n, parts):
        edges = np.linspace(0, n, parts + 1).astype(int)
        return [(kind, int(a), int(b)) for a, b in zip(edges[:-1], edges[1:]) if b > a]

    def median_time(run):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            run()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    workloads = {
        "gemv_pair": [("gemv_up", 18944), ("gemv_down", 3584)],
        "gemv_head": [("gemv_head", head_rows)],
        "mmq": [("mmq", mmq_cols)],
        "quantize": [("quantize", X.shape[0])],
    }
    one, allc = {}, {}
    for name, parts in workloads.items():
        one[name] = median_time(lambda: [_cpu_work((k, 0, n)) for k, n in parts])
    ctx = multiprocessing.get_context("fork")
    with ctx.Pool(workers) as pool:
        for name, parts in workloads.items():
            tasks = [t for k, n in parts for t in split(k, n, workers)]
            pool.map(_cpu_work, tasks)   # warm the workers
            allc[name] = median_time(lambda: pool.map(_cpu_work, tasks, chunksize=1))
    _CPU.clear()

    pair_bytes = w_up.nbytes + w_down.nbytes
    head_bytes = head_rows * 3584 // 256 * 210
    mmq_ops = 2 * X.shape[0] * mmq_cols * 3584
    qa_bytes = X.nbytes

    def rates(t):
        return {"gemv_pair_GBps": round(pair_bytes / t["gemv_pair"] / 1e9, 4),
                "gemv_q6_K_head_GBps": round(head_bytes / t["gemv_head"] / 1e9, 4),
                "mmq_q4_K_M512_GOPs": round(mmq_ops / t["mmq"] / 1e9, 3),
                "quantize_act_GBps_in": round(qa_bytes / t["quantize"] / 1e9, 4),
                "seconds": {k: round(v, 4) for k, v in t.items()}}

    return {
        "value": round(pair_bytes / allc["gemv_pair"] / 1e9, 4), "unit": "GB/s", "cores": workers,
        "kind": "oracle",
        "sample": (f"numpy f64 oracle GEMV over the full Q4_K ffn_up 18944x3584 + ffn_down 3584x18944 "
                   f"weights, rows split over {workers} worker processes with 1 BLAS thread each, median "
                   f"of 3; also on 1 thread, and the Q6_K head GEMV on {head_rows} of 152064 rows, the "
                   f"Q4_K MMQ at M=512 on {mmq_cols} of 18944 columns, quantize_act on 512x3584"),
        "cpu_model": _cpu_model(), "host_cpus_in_affinity": affinity,
        "all_cores": rates(allc), "one_thread": rates(one),
    }


class GraphTimer:
    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream

    def per_launch_us(self, launches, replays, warmup=2):
        """Record `launches` (callables, one kernel each) into a graph; time `replays` replays."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for fn in launches:
                fn()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        s = torch.cuda.current_stream()
        start.record(s)
        for _ in range(replays):
            g.replay()
        end.record(s)
        torch.cuda.synchronize()
        return 1000.0 * start.elapsed_time(end) / (replays * len(launches))


def load_measure_lib():
    import ctypes
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "block_quantized_matmul_mq_amd",
                        "libmq_measure.so")
    lib = ctypes.CDLL(path)
    lib.mq_measure_read.restype = ctypes.c_int
    lib.mq_measure_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p]
    lib.mq_measure_sink_words.restype = ctypes.c_size_t
    lib.mq_measure_sink_words.argtypes = [ctypes.c_int, ctypes.c_int]
    return lib


# Qwen2.5-14B layer mix: (name, type, N, K, uses per layer); q and o, k and v, gate and up
# share a shape
C5 = [("attn_q_o", Q4_K, 5120, 5120, 2), ("attn_k_v", Q4_K, 1024, 5120, 2),
      ("ffn_gate_up", Q4_K, 13824, 5120, 2), ("ffn_down", Q6_K, 5120, 13824, 1)]
C5_M = 2048


def c5_layer_mix(torch, mq, synth, timer, to_dev, dev, reps):
    """Per-shape GEMV (M = 1, weights rotated past the last-level cache) and quantize + MMQ
    (M = 2048) times for the 14B layer mix, and one layer's totals: q, k, v, o, gate, up,
    down, with the activation planes the layer quantizes (3 of 2048 x 5120, 1 of 2048 x
    13824)."""
    out = {}
    X = {K: torch.from_numpy(synth.activations(C5_M, K, 4, tensor_index=20 + i)).to(dev)
         for i, K in enumerate((5120, 13824))}
    Xq = {K: mq.quantize_act(X[K]) for K in X}
    t_quant = {K: timer.per_launch_us([lambda K=K: mq.quantize_act(X[K], Xq[K])] * 4, reps) for K in X}
    layer_gemv_us = layer_mmq_us = 0.0
    layer_bytes = layer_ops = 0
    for i, (name, qt, N, K, uses) in enumerate(C5):
        raw = synth.quantized_weight(qt, N, K, 4, i)
        nb = mq.weight_bytes(qt, N, K)
        wc = [to_dev(raw) for _ in range(copies_for(nb))]
        del raw
        x = torch.from_numpy(synth.activations(1, K, 4, tensor_index=30 + i)[0]).to(dev)
        y = torch.empty(N, dtype=torch.float32, device=dev)
        g_us = timer.per_launch_us([lambda W=W: mq.gemv(W, qt, x, N, K, y=y) for W in wc], reps)
        gk = mq.last_kernel()
        tiled_us = None
        if qt == Q4_K and mq.repack_bytes(Q4_K | ROW_TILED, N, K):
            # Q4_K's row-tiled layout, kept instead of the GGUF payload when its GEMV is faster
            # (every copy read once first, as for the 7B decode weights)
            wt = [mq.repack(W, Q4_K | ROW_TILED, N, K) for W in wc]
            for W in wt:
                mq.gemv(W, Q4_K | ROW_TILED, x, N, K, y=y)
            tiled_us = timer.per_launch_us([lambda W=W: mq.gemv(W, Q4_K | ROW_TILED, x, N, K, y=y) for W in wt],
                                           reps)
            del wt
        Y = torch.empty((C5_M, N), dtype=torch.float32, device=dev)
        sc = torch.zeros(max(mq.gemm_scratch_bytes(qt, C5_M, N, K), 256), dtype=torch.uint8, device=dev)
        m_us = timer.per_launch_us([lambda W=W: mq.gemm(W, qt, Xq[K], C5_M, N, K, Y=Y, scratch=sc) for W in wc[:2]],
                                   reps)
        m_kernel = mq.last_kernel()
        plane_us = None
        if qt == Q4_K:   # the MMQ plane, kept instead of the GGUF payload when its product is faster
            wp = [mq.repack(W, Q4_K, N, K) for W in wc[:2]]
            sp = torch.zeros(max(mq.gemm_scratch_bytes(Q4_K | REPACKED, C5_M, N, K), 256), dtype=torch.uint8,
                             device=dev)
            plane_us = timer.per_launch_us([lambda W=W: mq.gemm(W, Q4_K | REPACKED, Xq[K], C5_M, N, K, Y=Y, scratch=sp)
                                            for W in wp], reps)
            del wp, sp
        ops = 2 * C5_M * N * K
        out[f"{name}_{N}x{K}"] = {"type": "q4_K" if qt == Q4_K else "q6_K", "uses_per_layer": uses,
                                  "gemv_M1_us": round(g_us, 3), "gemv_M1_GBps": round(nb / g_us / 1e3, 1),
                                  "gemv_kernel": gk, "mmq_M2048_us": round(m_us, 3),
                                  "mmq_M2048_TOPS": round(ops / m_us / 1e6, 2), "mmq_kernel": m_kernel}
        if plane_us is not None:
            out[f"{name}_{N}x{K}"].update({"mmq_plane_M2048_us": round(plane_us, 3),
                                           "mmq_plane_M2048_TOPS": round(ops / plane_us / 1e6, 2)})
            m_us = min(m_us, plane_us)
        if tiled_us is not None:
            out[f"{name}_{N}x{K}"].update({"gemv_row_tiled_M1_us": round(tiled_us, 3),
                                           "gemv_row_tiled_M1_GBps": round(nb / tiled_us / 1e3, 1)})
            g_us = min(g_us, tiled_us)
        layer_gemv_us += uses * g_us
        layer_mmq_us += uses * m_us
        layer_bytes += uses * nb
        layer_ops += uses * ops
        del wc, Y, sc
    q_us = 3 * t_quant[5120] + t_quant[13824]
    out["quantize_act_M2048_us"] = {"K5120": round(t_quant[5120], 3), "K13824": round(t_quant[13824], 3)}
    out["layer"] = {"gemv_M1_us": round(layer_gemv_us, 2), "gemv_M1_GBps": round(layer_bytes / layer_gemv_us / 1e3, 1),
                    "prefill_M2048_us": round(layer_mmq_us + q_us, 2),
                    "prefill_M2048_TOPS": round(layer_ops / (layer_mmq_us + q_us) / 1e6, 2),
                    "note": "q, k, v, o, gate, up, down; kernel times summed (each Q4_K GEMV in the faster of its "
                            "GGUF payload and row-tiled layout, each Q4_K product in the faster of its GGUF payload "
                            "and MMQ plane), quantize_act included at M=2048"}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the kernels are "
              "single-GPU and no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)

    from block_quantized_matmul_mq_amd import synth

    # ---- host inputs (seeded), and the CPU baseline before the GPU is touched ----
    w_host = {name: synth.quantized_weight(Q4_K, N, K, 1, i) for i, (name, N, K) in enumerate(DECODE)}
    for i, (name, N, K) in enumerate(PREFILL[1:]):
        w_host[name] = synth.quantized_weight(Q4_K, N, K, 3, i + 1)
    x_dec = {name: synth.activations(1, K, 1, tensor_index=10 + i)[0] for i, (name, N, K) in enumerate(DECODE)}
    X_pre = synth.activations(PREFILL_M, 3584, 3)
    cpu = None
    if not args.no_cpu_baseline and not args.counters:
        cpu = cpu_baseline(w_host["ffn_up"], w_host["ffn_down"], x_dec["ffn_up"], x_dec["ffn_down"], X_pre)

    import ctypes

    import torch
    from block_quantized_matmul_mq_amd import mq

    dev = torch.device("cuda:0")
    mq.init(0)
    timer = GraphTimer(torch, torch.cuda.current_stream())

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).to(dev)

    # ---- inputs, resident in HBM ----
    ncopy = copies_for(mq.weight_bytes(Q4_K, 18944, 3584))
    copies = {name: [to_dev(w_host[name]) for _ in range(ncopy)] for name, _, _ in DECODE}
    w_pre = {name: to_dev(w_host[name]) for name, _, _ in PREFILL[1:]}
    x_dev = {k: torch.from_numpy(v).to(dev) for k, v in x_dec.items()}
    y_dev = {name: torch.empty(N, dtype=torch.float32, device=dev) for name, N, _ in DECODE}
    X_dev = torch.from_numpy(X_pre).to(dev)
    Xq = torch.empty(mq.act_bytes(PREFILL_M, 3584), dtype=torch.uint8, device=dev)
    Y_dev = {name: torch.empty((PREFILL_M, N), dtype=torch.float32, device=dev) for name, N, _ in PREFILL}
    scratch = {name: torch.zeros(max(mq.gemm_scratch_bytes(Q4_K, PREFILL_M, N, K),
                                     mq.gemm_scratch_bytes(Q4_K | REPACKED, PREFILL_M, N, K), 256),
                                 dtype=torch.uint8, device=dev) for name, N, K in PREFILL}
    # Q4_K's MMQ plane (mq_repack, a one-time transform at load time) of every prefill weight;
    # the ffn_up plane is rotated past the last-level cache like its GGUF copies
    nplane = copies_for(mq.repack_bytes(Q4_K, 18944, 3584))
    planes = {"ffn_up": [mq.repack(copies["ffn_up"][c % ncopy], Q4_K, 18944, 3584) for c in range(nplane)]}
    for name, N, K in PREFILL[1:]:
        planes[name] = [mq.repack(w_pre[name], Q4_K, N, K)]
    torch.cuda.synchronize()

    kernel_names = {}

    # Decode weights with rows of more than 16 super-blocks (ffn_down) are also held in Q4_K's
    # row-tiled layout (mq_repack, a one-time transform at load time, of every rotated copy);
    # each keeps the layout whose GEMV is faster, chosen once at load time from a few timed
    # graph replays, as for the prefill weights below.
    tiled = {name: [mq.repack(W, Q4_K | ROW_TILED, N, K) for W in copies[name]]
             for name, N, K in DECODE if mq.repack_bytes(Q4_K | ROW_TILED, N, K)}
    torch.cuda.synchronize()

    def gemv_on(name, N, K, c, lay):
        W, qt = (tiled[name][c], Q4_K | ROW_TILED) if lay == "row_tiled" else (copies[name][c], Q4_K)

        def fn():
            mq.gemv(W, qt, x_dev[name], N, K, y=y_dev[name])
            kernel_names[f"gemv_{name}"] = mq.last_kernel()
        return fn

    # (every copy is read once first -- the first replays after writing the new copies run
    # slow -- and the layouts are timed in two alternating rounds, the best of each kept)
    gemv_layout, gemv_each = {}, {}
    for name, N, K in DECODE:
        lays = ("gguf", "row_tiled") if name in tiled else ("gguf",)
        for lay in lays:
            for c in range(ncopy):
                gemv_on(name, N, K, c, lay)()
        torch.cuda.synchronize()
        best = {}
        for _ in range(2):
            for lay in lays:
                us = timer.per_launch_us([gemv_on(name, N, K, c, lay) for c in range(ncopy)], 5)
                best[lay] = min(us, best.get(lay, us))
                gemv_each[f"{name}_{lay}"] = {"us": round(best[lay], 3), "kernel": mq.last_kernel(),
                                              "GBps": round(mq.weight_bytes(Q4_K, N, K) / best[lay] / 1e3, 1)}
        gemv_layout[name] = min(lays, key=best.get)

    def gemv_launch(name, N, K, c):
        return gemv_on(name, N, K, c, gemv_layout[name])

    def quant_launch():
        mq.quantize_act(X_dev, Xq)

    def mmq_on(name, N, K, c, lay):
        if lay == "plane":
            W, qt = planes[name][c % len(planes[name])], Q4_K | REPACKED
        else:
            W, qt = (copies["ffn_up"][c % ncopy] if name == "ffn_up" else w_pre[name]), Q4_K

        def fn():
            mq.gemm(W, qt, Xq, PREFILL_M, N, K, Y=Y_dev[name], scratch=scratch[name])
            kernel_names[f"mmq_{name}"] = mq.last_kernel()
        return fn

    # Each prefill weight keeps the layout whose product is faster at M = 512 (GGUF payload
    # or MMQ plane), chosen once at load time from a few timed graph replays, as a serving
    # engine would; the timed step then runs the chosen kernels.
    mq.quantize_act(X_dev, Xq)
    layout_us = {}
    layout = {}
    for name, N, K in PREFILL:
        layout_us[name] = {lay: timer.per_launch_us([mmq_on(name, N, K, c, lay) for c in range(4)], 5)
                           for lay in ("gguf", "plane")}
        layout[name] = min(layout_us[name], key=layout_us[name].get)

    def mmq_launch(name, N, K, c):
        return mmq_on(name, N, K, c, layout[name])

    def step_launches(c):
        out = [gemv_launch(name, N, K, c) for name, N, K in DECODE]
        out.append(quant_launch)
        out += [mmq_launch(name, N, K, c) for name, N, K in PREFILL]
        return out

    if args.counters:
        # reference copy: 256 MiB read + 256 MiB written, to calibrate FETCH_SIZE / WRITE_SIZE
        ref_src = torch.empty(COPY_REF_BYTES, dtype=torch.uint8, device=dev)
        ref_dst = torch.empty_like(ref_src)
        for _ in range(3):
            ref_dst.copy_(ref_src)
        for c in range(min(ncopy, 4)):
            for fn in step_launches(c):
                fn()
        torch.cuda.synchronize()
        print(json.dumps({"counters_run": True, "copy_ref_bytes": COPY_REF_BYTES,
                          "gemv_payload_bytes": {n: mq.weight_bytes(Q4_K, N, K) for n, N, K in DECODE},
                          "kernel_names": kernel_names}), flush=True)
        return

    # eager warmup (also sets the kernel names), then one graph per weight copy: graph c is
    # one step (one pass of the hot path) on copy c
    for c in range(ncopy):
        for fn in step_launches(c):
            fn()
    torch.cuda.synchronize()
    step_graphs = []
    for c in range(ncopy):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for fn in step_launches(c):
                fn()
        step_graphs.append(g)
    for i in range(args.warmup):
        step_graphs[i % ncopy].replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(s)
    for i in range(args.steps):
        step_graphs[(args.warmup + i) % ncopy].replay()
    t_end.record(s)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    del step_graphs

    # per-kernel times: each kernel alone, its launches back to back in a graph
    reps = max(2, args.steps // 2)
    avg_us = {}
    for name, N, K in DECODE:
        avg_us[f"gemv_{name}"] = timer.per_launch_us([gemv_launch(name, N, K, c) for c in range(ncopy)], reps)
    avg_us["quantize_act"] = timer.per_launch_us([quant_launch] * 8, reps)
    mmq_both = {}
    for name, N, K in PREFILL:
        for lay in ("gguf", "plane"):
            us = timer.per_launch_us([mmq_on(name, N, K, c, lay) for c in range(4)], reps)
            mmq_both[f"{name}_{lay}"] = {"us": round(us, 3), "kernel": mq.last_kernel(),
                                         "TOPS": round(2 * PREFILL_M * N * K / us / 1e6, 2)}
        avg_us[f"mmq_{name}"] = mmq_both[f"{name}_{layout[name]}"]["us"]
        for fn in (mmq_launch(name, N, K, 0),):
            fn()

    # plain-read ceiling: the same rotated ffn_up copies read by a kernel that only reads,
    # with the workgroup count of the GEMV (one per CU) and with the best of a few counts
    meas = load_measure_lib()

    def plain_read_gbps(tensors, nbytes, grids=(256, 512, 1024, 2048)):
        out = {}
        for grid in grids:
            sink = torch.empty(meas.mq_measure_sink_words(grid, 1024), dtype=torch.int32, device=dev)

            def read_launch(W, grid=grid, sink=sink):
                rc = meas.mq_measure_read(ctypes.c_void_p(W.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                          grid, 1024, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
                if rc:
                    raise RuntimeError(f"plain-read kernel refused ({rc})")
            us = timer.per_launch_us([lambda W=W: read_launch(W) for W in tensors], reps)
            out[grid] = nbytes / us / 1e3
        return out

    up_bytes = mq.weight_bytes(Q4_K, 18944, 3584)
    read_gbps = plain_read_gbps(copies["ffn_up"], up_bytes)
    plain_read = max(read_gbps.values())

    # warm cache (labelled, never the value): one weight copy, resident in the last-level cache
    warm = {}
    for name, N, K in DECODE:
        us = timer.per_launch_us([gemv_launch(name, N, K, 0)] * 8, reps)
        warm[f"gemv_{name}_us"] = round(us, 3)
        warm[f"gemv_{name}_GBps"] = round(mq.weight_bytes(Q4_K, N, K) / us / 1e3, 1)
    warm["note"] = ("weights resident in the 256 MB last-level cache (one copy, launches back to back); "
                    "every other GEMV figure rotates copies past it")

    gemv_bytes = sum(mq.weight_bytes(Q4_K, N, K) for _, N, K in DECODE)
    # algorithmic bytes of one GEMV launch: GGUF payload + f32 x + f32 y (the same for both shapes)
    gemv_alg_bytes = mq.weight_bytes(Q4_K, 18944, 3584) + 4 * (18944 + 3584)
    gemv_s = sum(avg_us[f"gemv_{n}"] for n, _, _ in DECODE) * 1e-6
    gemv_gbps = gemv_bytes / gemv_s / 1e9
    gemv_alg_gbps = len(DECODE) * gemv_alg_bytes / gemv_s / 1e9
    mmq_ops = sum(2 * PREFILL_M * N * K for _, N, K in PREFILL)
    mmq_s = sum(avg_us[f"mmq_{n}"] for n, _, _ in PREFILL) * 1e-6
    mmq_tops = mmq_ops / mmq_s / 1e12
    up_gbps = mq.weight_bytes(Q4_K, 18944, 3584) / (avg_us["gemv_ffn_up"] * 1e-6) / 1e9
    down_gbps = mq.weight_bytes(Q4_K, 3584, 18944) / (avg_us["gemv_ffn_down"] * 1e-6) / 1e9
    mmq_up_tops = 2 * PREFILL_M * 18944 * 3584 / (avg_us["mmq_ffn_up"] * 1e-6) / 1e12
    mmq_rec = recorded_fields("mmq_q4k_512x18944x3584_counters.txt")

    result = {
        "metric": "Q4_K GEMV weight GB/s at M=1 + MMQ prefill TOPS at M=512 (7B shapes)",
        "value": round(gemv_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "step": (f"one pass of the hot path (2 decode GEMVs, quantize_act, 4 MMQs) replayed from a HIP graph; "
                 f"consecutive steps rotate through {ncopy} weight copies; exactly `steps` passes are timed"),
        "config": {
            "workload": "Qwen2.5-7B Q4_K: decode GEMV ffn_up 18944x3584 + ffn_down 3584x18944 (M=1, f32 x); "
                        "prefill M=512: quantize_act 512x3584 + MMQ ffn_up/attn_q/attn_k/attn_v",
            "M_decode": 1, "M_prefill": PREFILL_M, "weight_copies_rotated": ncopy,
            "parallelism": "single GPU",
        },
        "mmq_prefill_tops": round(mmq_tops, 2),
        "mmq_dtype": ("exact block dots: on Q4_K's MMQ plane fp6 (e2m3) x fp6 MFMA, weight codes c/2 and activation "
                      "codes as two digits h/2, l/2 with block scales 2^5, 2^1 (f32 results); on the GGUF payload "
                      "int8 MFMA (i32 results); f32 scales through bf16 hi/lo matrix products"),
        "gemv_layouts": {"chosen": gemv_layout, "note": "per decode weight, the faster of the GGUF payload and "
                         "Q4_K's row-tiled layout (a permutation of its blocks: the same bytes, the same results bit "
                         "for bit; rows of more than 16 super-blocks only), chosen once at load time",
                         "each": gemv_each},
        "mmq_layouts": {"chosen": layout, "note": "per weight, the faster of the GGUF payload and the MMQ plane "
                        "at M=512, chosen once at load time", "each": mmq_both},
        "roofline": {"bound": "hbm", "achieved": round(gemv_alg_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gemv_alg_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": recorded_traffic("gemv_q4k_7b_ffn_hbm_traffic.txt"),
                     "plain_read_GBps": round(plain_read, 1),
                     "frac_of_plain_read": round(gemv_alg_gbps / plain_read, 4),
                     "plain_read_by_workgroups": {str(g): round(v, 1) for g, v in read_gbps.items()},
                     "algorithmic_bytes_per_launch": gemv_alg_bytes,
                     "kernel": f"{kernel_names['gemv_ffn_up']} (ffn_up) + {kernel_names['gemv_ffn_down']} (ffn_down)",
                     "ffn_up_GBps": round(up_gbps, 1), "ffn_down_GBps": round(down_gbps, 1)},
        "roofline_mmq": {"bound": "mfma", "achieved": round(mmq_up_tops, 2), "peak": INT8_PEAK_TOPS,
                         "unit": "TOP/s", "frac": round(mmq_up_tops / INT8_PEAK_TOPS, 4),
                         "traffic": (int(mmq_rec["traffic_bytes_per_launch"])
                                     if "traffic_bytes_per_launch" in mmq_rec else None),
                         "mfma_busy_frac": (float(mmq_rec["mfma_busy_frac"]) if "mfma_busy_frac" in mmq_rec
                                            else None),
                         "sclk_MHz": float(mmq_rec["sclk_MHz"]) if "sclk_MHz" in mmq_rec else None,
                         "kernel": f"{kernel_names['mmq_ffn_up']} ffn_up M=512 18944x3584"},
        "kernel_avg_us": {lab: round(v, 3) for lab, v in avg_us.items()},
        "kernel_names": kernel_names,
        "warm_cache": warm,
    }

    result["c5_14b"] = c5_layer_mix(torch, mq, synth, timer, to_dev, dev, reps)

    if not args.no_secondary:
        sec = {}
        head = synth.quantized_weight(Q6_K, 152064, 3584, 2, 0)
        hb = mq.weight_bytes(Q6_K, 152064, 3584)
        hcop = [to_dev(head) for _ in range(copies_for(hb))]
        del head
        xh = torch.from_numpy(synth.activations(1, 3584, 2)[0]).to(dev)
        yh = torch.empty(152064, dtype=torch.float32, device=dev)
        us = timer.per_launch_us([lambda W=W: mq.gemv(W, Q6_K, xh, 152064, 3584, y=yh) for W in hcop], reps)
        pr = max(plain_read_gbps(hcop, hb, grids=(256, 512, 1024)).values())
        sec["gemv_q6_K_head_152064x3584"] = {"us": round(us, 3), "GBps": round(hb / us / 1e3, 1),
                                             "frac": round(hb / us / 1e3 / 8000.0, 4), "plain_read_GBps": round(pr, 1),
                                             "frac_of_plain_read": round(hb / us / 1e3 / pr, 4)}
        # small-M product on the head: M = 8 rows (a speculative-verify batch), q8 activations
        Xh = torch.from_numpy(synth.activations(8, 3584, 2, tensor_index=5)).to(dev)
        Xhq = mq.quantize_act(Xh)
        Yh = torch.empty((8, 152064), dtype=torch.float32, device=dev)
        sch = torch.zeros(max(mq.gemm_scratch_bytes(Q6_K, 8, 152064, 3584), 256), dtype=torch.uint8, device=dev)
        us = timer.per_launch_us([lambda W=W: mq.gemm(W, Q6_K, Xhq, 8, 152064, 3584, Y=Yh, scratch=sch)
                                  for W in hcop], reps)
        sec["mmq_q6_K_head_M8_152064x3584"] = {"us": round(us, 3), "weight_GBps": round(hb / us / 1e3, 1),
                                               "TOPS": round(2 * 8 * 152064 * 3584 / us / 1e6, 2),
                                               "kernel": mq.last_kernel()}
        # the same head in the repacked layout (224-byte slots): bytes read are the slots
        rb = mq.repack_bytes(Q6_K, 152064, 3584)
        rcop = [mq.repack(W, Q6_K, 152064, 3584) for W in hcop]
        del hcop
        torch.cuda.synchronize()
        us = timer.per_launch_us([lambda W=W: mq.gemv(W, Q6_K | mq.REPACKED, xh, 152064, 3584, y=yh)
                                  for W in rcop], reps)
        sec["gemv_q6_K_head_repacked_152064x3584"] = {"us": round(us, 3), "GBps": round(rb / us / 1e3, 1),
                                                      "kernel": mq.last_kernel()}
        us = timer.per_launch_us([lambda W=W: mq.gemm(W, Q6_K | mq.REPACKED, Xhq, 8, 152064, 3584, Y=Yh,
                                                      scratch=sch) for W in rcop], reps)
        sec["mmq_q6_K_head_M8_repacked_152064x3584"] = {"us": round(us, 3), "weight_GBps": round(rb / us / 1e3, 1),
                                                        "kernel": mq.last_kernel()}
        del rcop
        for N, K, tag in [(18944, 3584, "7B_ffn_up_shape"), (4864, 896, "0.5B_ffn_up")]:
            w8 = synth.quantized_weight(Q8_0, N, K, 0, 0)
            nb = mq.weight_bytes(Q8_0, N, K)
            wc = [to_dev(w8) for _ in range(copies_for(nb))]
            x8 = torch.from_numpy(synth.activations(1, K, 0)[0]).to(dev)
            y8 = torch.empty(N, dtype=torch.float32, device=dev)
            us = timer.per_launch_us([lambda W=W: mq.gemv(W, Q8_0, x8, N, K, y=y8) for W in wc], reps)
            pr = max(plain_read_gbps(wc, nb - nb % 16, grids=(256, 512, 1024)).values())
            sec[f"gemv_q8_0_{tag}_{N}x{K}"] = {"us": round(us, 3), "GBps": round(nb / us / 1e3, 1),
                                               "frac": round(nb / us / 1e3 / 8000.0, 4),
                                               "plain_read_GBps": round(pr, 1),
                                               "frac_of_plain_read": round(nb / us / 1e3 / pr, 4)}
            del wc
        # the other types of the eligibility list on the 7B ffn_up shape: GEMV at M = 1 (weights
        # rotated past the last-level cache) and the prefill product at M = 512
        N7, K7 = 18944, 3584
        for qt, tag in [(mq.Q5_K, "q5_K"), (mq.Q4_0, "q4_0"), (mq.Q4_1, "q4_1"), (mq.Q5_0, "q5_0"),
                        (mq.Q5_1, "q5_1")]:
            wt = synth.quantized_weight(qt, N7, K7, 1, 50 + qt)
            nb = mq.weight_bytes(qt, N7, K7)
            wc = [to_dev(wt) for _ in range(copies_for(nb))]
            del wt
            xt = x_dev["ffn_up"]
            yt = torch.empty(N7, dtype=torch.float32, device=dev)
            us = timer.per_launch_us([lambda W=W: mq.gemv(W, qt, xt, N7, K7, y=yt) for W in wc], reps)
            gk = mq.last_kernel()
            Yt = torch.empty((PREFILL_M, N7), dtype=torch.float32, device=dev)
            sct = torch.zeros(max(mq.gemm_scratch_bytes(qt, PREFILL_M, N7, K7), 256), dtype=torch.uint8, device=dev)
            us_m = timer.per_launch_us([lambda W=W: mq.gemm(W, qt, Xq, PREFILL_M, N7, K7, Y=Yt, scratch=sct)
                                        for W in wc[:4]], reps)
            sec[f"{tag}_7B_ffn_up_{N7}x{K7}"] = {
                "gemv_us": round(us, 3), "gemv_GBps": round(nb / us / 1e3, 1), "gemv_kernel": gk,
                "mmq_M512_us": round(us_m, 3), "mmq_M512_TOPS": round(2 * PREFILL_M * N7 * K7 / us_m / 1e6, 2),
                "mmq_kernel": mq.last_kernel()}
            del wc, Yt, sct
        # gate and up (18944 x 3584 Q4_K each) as two products, or as one 37888-row product
        gate = copies["ffn_up"][0]
        upw = to_dev(synth.quantized_weight(Q4_K, N7, K7, 1, 60))
        gu = torch.cat([gate, upw])
        ncg = copies_for(2 * mq.weight_bytes(Q4_K, N7, K7))
        gus = [gu] + [gu.clone() for _ in range(ncg - 1)]
        pairs = [(gate, upw)] + [(g[:gate.numel()], g[gate.numel():]) for g in gus[1:]]
        ygu = torch.empty(2 * N7, dtype=torch.float32, device=dev)
        xg = x_dev["ffn_up"]
        us_sep = timer.per_launch_us([lambda a=a, b=b: (mq.gemv(a, Q4_K, xg, N7, K7, y=ygu[:N7]),
                                                        mq.gemv(b, Q4_K, xg, N7, K7, y=ygu[N7:])) for a, b in pairs],
                                     reps)
        us_cat = timer.per_launch_us([lambda g=g: mq.gemv(g, Q4_K, xg, 2 * N7, K7, y=ygu) for g in gus], reps)
        Ygu = torch.empty((PREFILL_M, 2 * N7), dtype=torch.float32, device=dev)
        Yg, Yu = (torch.empty((PREFILL_M, N7), dtype=torch.float32, device=dev) for _ in range(2))
        scg = torch.zeros(max(mq.gemm_scratch_bytes(Q4_K, PREFILL_M, 2 * N7, K7),
                              mq.gemm_scratch_bytes(Q4_K, PREFILL_M, N7, K7), 256), dtype=torch.uint8, device=dev)
        mm_sep = timer.per_launch_us([lambda: (mq.gemm(gate, Q4_K, Xq, PREFILL_M, N7, K7, Y=Yg, scratch=scg),
                                               mq.gemm(upw, Q4_K, Xq, PREFILL_M, N7, K7, Y=Yu, scratch=scg))] * 2,
                                     reps)
        mm_cat = timer.per_launch_us([lambda: mq.gemm(gu, Q4_K, Xq, PREFILL_M, 2 * N7, K7, Y=Ygu, scratch=scg)] * 2,
                                     reps)
        sec["q4_K_gate_up_7B"] = {"gemv_two_launches_us": round(us_sep, 3), "gemv_one_37888_row_launch_us": round(us_cat, 3),
                                  "mmq_M512_two_launches_us": round(mm_sep, 3),
                                  "mmq_M512_one_37888_row_launch_us": round(mm_cat, 3)}
        del gus, pairs, gu, upw
        qa_bytes = PREFILL_M * 3584 * 4
        sec["quantize_act_512x3584"] = {"us": round(avg_us["quantize_act"], 3),
                                        "GBps_in": round(qa_bytes / avg_us["quantize_act"] / 1e3, 1)}
        result["secondary"] = sec

    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
