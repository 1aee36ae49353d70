"""Benchmark of the block-quantized matmul hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic
Qwen2.5-7B-shaped inputs (weights N(0, 0.02) quantized to Q4_K, activations
N(0, 1)):

  decode  : mq_gemv Q4_K ffn_up 18944x3584 and ffn_down 3584x18944 at M=1
  prefill : mq_quantize_act 512x3584, then mq_gemm (int8 MMQ) with the Q4_K
            ffn_up 18944x3584, attn_q 3584x3584, attn_k and attn_v 512x3584

Inputs are resident in HBM before timing starts.  Each GEMV weight is kept in
several copies that the steps rotate through, so every GEMV launch reads its
weights from HBM and not from the 256 MB last-level cache.

Printed JSON line (rank 0, one GPU):
  value     = Q4_K GEMV weight GB/s: GGUF payload bytes of the two decode
              GEMVs / their summed kernel time (HIP events on the launch stream)
  mmq_prefill_tops = 2*M*N*K of the four MMQ launches / their kernel time
  roofline / roofline_mmq = the GEMV against 8 TB/s HBM, the MMQ against
              5.0 POP/s dense int8 MFMA
  cpu_baseline = the CPU oracle's GEMV on the same ffn_up + ffn_down weights
"""

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
INT8_PEAK_TOPS = 5000.0

DECODE = [("ffn_up", 18944, 3584), ("ffn_down", 3584, 18944)]
PREFILL_M = 512
PREFILL = [("ffn_up", 18944, 3584), ("attn_q", 3584, 3584), ("attn_k", 512, 3584), ("attn_v", 512, 3584)]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--copies", type=int, default=8, help="rotated copies of each GEMV weight")
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


def cpu_baseline(w_up, w_down, x_up, x_down):
    """The oracle (as written, single thread) on the full decode pair, median of 3."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limit = None
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.gemv(w_up, 12, x_up, 18944, 3584)
        oracle.gemv(w_down, 12, x_down, 3584, 18944)
        times.append(time.perf_counter() - t0)
    if limit is not None:
        limit.unregister()
    t = float(np.median(times))
    nbytes = w_up.nbytes + w_down.nbytes
    return {"value": nbytes / t / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "numpy f64 oracle GEMV over the full Q4_K ffn_up 18944x3584 + ffn_down "
                      f"3584x18944 weights, 1 thread, median of 3 ({t:.2f} s per pair)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the kernels are "
              "single-GPU and no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_quantized_matmul_mq_amd import mq, synth

    dev = torch.device("cuda:0")
    mq.init(0)
    stream = torch.cuda.current_stream()

    # ---- inputs, resident in HBM ----
    w_host = {name: synth.quantized_weight(12, N, K, 1, i) for i, (name, N, K) in enumerate(DECODE)}
    for i, (name, N, K) in enumerate(PREFILL[1:]):
        w_host[name] = synth.quantized_weight(12, N, K, 3, i + 1)
    x_dec = {name: synth.activations(1, K, 1, tensor_index=10 + i)[0] for i, (name, N, K) in enumerate(DECODE)}
    X_pre = synth.activations(PREFILL_M, 3584, 3)

    copies = {name: [torch.from_numpy(w_host[name].reshape(-1)).to(dev) for _ in range(args.copies)]
              for name, _, _ in DECODE}
    w_pre = {name: torch.from_numpy(w_host[name].reshape(-1)).to(dev) for name, _, _ in PREFILL[1:]}
    x_dev = {k: torch.from_numpy(v).to(dev) for k, v in x_dec.items()}
    y_dev = {name: torch.empty(N, dtype=torch.float32, device=dev) for name, N, _ in DECODE}
    X_dev = torch.from_numpy(X_pre).to(dev)
    Xq = torch.empty(mq.act_bytes(PREFILL_M, 3584), dtype=torch.uint8, device=dev)
    Y_dev = {name: torch.empty((PREFILL_M, N), dtype=torch.float32, device=dev) for name, N, _ in PREFILL}
    torch.cuda.synchronize()

    labels = [f"gemv_{n}" for n, _, _ in DECODE] + ["quantize_act"] + [f"mmq_{n}" for n, _, _ in PREFILL]
    kernel_names = {}

    def step(i, events=None):
        c = i % args.copies
        k = 0

        def mark():
            nonlocal k
            if events is not None:
                events[k].record(stream)
            k += 1

        for name, N, K in DECODE:
            mark()
            mq.gemv(copies[name][c], 12, x_dev[name], N, K, y=y_dev[name])
            kernel_names[f"gemv_{name}"] = mq.last_kernel()
        mark()
        mq.quantize_act(X_dev, Xq)
        for name, N, K in PREFILL:
            mark()
            W = copies["ffn_up"][c] if name == "ffn_up" else w_pre[name]
            mq.gemm(W, 12, Xq, PREFILL_M, N, K, Y=Y_dev[name])
            kernel_names[f"mmq_{name}"] = mq.last_kernel()
        mark()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    nev = len(labels) + 1
    all_events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, all_events[i])
    t_end.record(stream)
    torch.cuda.synchronize()

    total_ms = t_start.elapsed_time(t_end)
    per = {lab: [] for lab in labels}
    for ev in all_events:
        for j, lab in enumerate(labels):
            per[lab].append(ev[j].elapsed_time(ev[j + 1]))
    avg_us = {lab: 1000.0 * float(np.mean(v)) for lab, v in per.items()}

    gemv_bytes = sum(mq.weight_bytes(12, N, K) for _, N, K in DECODE)
    gemv_s = sum(avg_us[f"gemv_{n}"] for n, _, _ in DECODE) * 1e-6
    gemv_gbps = gemv_bytes / gemv_s / 1e9
    mmq_ops = sum(2 * PREFILL_M * N * K for _, N, K in PREFILL)
    mmq_s = sum(avg_us[f"mmq_{n}"] for n, _, _ in PREFILL) * 1e-6
    mmq_tops = mmq_ops / mmq_s / 1e12
    up_bytes = mq.weight_bytes(12, 18944, 3584)
    up_gbps = up_bytes / (avg_us["gemv_ffn_up"] * 1e-6) / 1e9
    mmq_up_tops = 2 * PREFILL_M * 18944 * 3584 / (avg_us["mmq_ffn_up"] * 1e-6) / 1e12

    result = {
        "metric": "Q4_K GEMV weight GB/s at M=1 + MMQ prefill TOPS at M=512 (7B shapes)",
        "value": round(gemv_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "Qwen2.5-7B Q4_K: decode GEMV ffn_up 18944x3584 + ffn_down 3584x18944 (M=1, f32 x); "
                        "prefill M=512: quantize_act 512x3584 + int8 MMQ ffn_up/attn_q/attn_k/attn_v",
            "M_decode": 1, "M_prefill": PREFILL_M, "weight_copies_rotated": args.copies,
            "parallelism": "single GPU",
        },
        "mmq_prefill_tops": round(mmq_tops, 2),
        "mmq_dtype": "i8 x i8 -> i32 block dots, f32 scales",
        "roofline": {"bound": "hbm", "achieved": round(gemv_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gemv_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "gemv Q4_K (ffn_up + ffn_down)",
                     "ffn_up_GBps": round(up_gbps, 1)},
        "roofline_mmq": {"bound": "mfma", "achieved": round(mmq_up_tops, 2), "peak": INT8_PEAK_TOPS,
                         "unit": "TOP/s", "frac": round(mmq_up_tops / INT8_PEAK_TOPS, 4), "traffic": None,
                         "kernel": "mmq Q4_K ffn_up M=512 18944x3584"},
        "kernel_avg_us": {lab: round(v, 3) for lab, v in avg_us.items()},
        "kernel_names": kernel_names,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w_host["ffn_up"], w_host["ffn_down"], x_dec["ffn_up"],
                                              x_dec["ffn_down"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
