#!/usr/bin/env python3
"""Throughput of the tiled GEMM+ReLU on one MI355X, through the tile_gemm C ABI.

One step = one tile_gemm call on the measured workload (default: M=N=K=8192,
bf16 operands drawn from normal(0, 1/sqrt(K)), alpha=0.5, ReLU on, fp32 D),
inputs already resident in HBM.  Prints one JSON line with the throughput in
TFLOP/s (2MNK/t), the roofline position of the GEMM kernel, a parity check of
the output against the oracle on the CPU-baseline sample, and the oracle's own
throughput on the host cores.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--kernel-id ID]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "TFLOP/s (2MNK/t) bf16 GEMM+ReLU at 8192³; % of dense MFMA peak"
# MI355X dense peaks (no sparsity): 256 CUs at 2.4 GHz
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3, "e4m3": 5033.2, "e5m2": 5033.2}
TRAFFIC_FILE = ROOT / "profiles" / "traffic.json"
SOURCES = ["dense_tiled_gemm_tile_amd/csrc/gemm_kernels.hip", "dense_tiled_gemm_tile_amd/csrc/tile_math.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in SOURCES:
        h.update((ROOT / rel).read_bytes())
    return h.hexdigest()[:16]


def traffic_for(workload: str, kernel_id: int):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source; otherwise None."""
    if not TRAFFIC_FILE.exists():
        return None
    data = json.loads(TRAFFIC_FILE.read_text())
    entry = data.get(workload)
    if not entry or entry.get("source_hash") != kernel_source_hash() or entry.get("kernel_id") != kernel_id:
        return None
    return entry.get("hbm_bytes_per_launch")


def copy_calibration(nbytes: int) -> None:
    """A plain device copy of known size, run under the counter profiler to scale
    FETCH_SIZE / WRITE_SIZE."""
    import torch

    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 3}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="square_8192_bf16_relu")
    ap.add_argument("--kernel-id", type=int, default=-1)
    ap.add_argument("--splits", type=int, default=1,
                    help="split K into this many ranges (tile_gemm_splitk, 0 = automatic; workspace allocated "
                         "up front)")
    ap.add_argument("--epilogue", choices=["pointwise", "softmax"], default="pointwise",
                    help="pointwise alpha/ReLU (tile_gemm) or a row softmax over N (tile_gemm_softmax)")
    ap.add_argument("--out-dtype", choices=["f32", "bf16", "f16"], default="f32",
                    help="element type of D (bf16/f16: fp32 epilogue rounded on the way out)")
    ap.add_argument("--block-scales", action="store_true",
                    help="8-bit workloads: seeded block scales (one exponent per 32 k of every A row and B "
                         "column) through tile_gemm_scaled")
    ap.add_argument("--cpu-cols", type=int, default=4096,
                    help="output columns the CPU-baseline oracle computes (all rows, full K)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the GEMM shards into independent column panels, one per GPU, with no exchange)",
              file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return 0

    import torch

    import dense_tiled_gemm_tile_amd as tg
    import seeded_inputs as si

    w = si.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    A_st, B_st = si.workload_operands(w)
    A, B = A_st.to(dev), B_st.to(dev)
    out_torch = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[args.out_dtype]
    D = si.out_storage(w.M, w.batch * w.N, w.ldd).to(out_torch).to(dev)
    if w.batch == 1:
        Av, Bv, Dv = A[:, :w.K], B[:, :w.K].t(), D[:, :w.M].t()
        plan = tg.plan_for(Av, Bv, Dv, args.kernel_id)
        launch = tg.gemm
        if args.epilogue == "softmax":
            def launch(A_, B_, D_, alpha, relu, stream=None, kernel_id=-1):
                return tg.gemm_softmax(A_, B_, D_, alpha, stream=stream, kernel_id=kernel_id)
        if args.block_scales:
            if w.dtype not in ("e4m3", "e5m2"):
                print("--block-scales needs an 8-bit workload", file=sys.stderr)
                return 2
            sc_a_np = si.block_scales(w.M, w.K, w.seed_a + 50)
            sc_b_np = si.block_scales(w.N, w.K, w.seed_b + 50)
            sc_a, sc_b = torch.from_numpy(sc_a_np).to(dev), torch.from_numpy(sc_b_np).to(dev)

            def launch(A_, B_, D_, alpha, relu, stream=None, kernel_id=-1):
                return tg.gemm_scaled(A_, B_, D_, sc_a, sc_b, alpha, relu, stream=stream, kernel_id=kernel_id)
        if args.splits != 1:
            ws = torch.empty(max(tg.splitk_workspace_bytes(w.M, w.N, args.splits), 16), dtype=torch.uint8,
                             device=dev)

            def launch(A_, B_, D_, alpha, relu, stream=None, kernel_id=-1):
                return tg.gemm_splitk(A_, B_, D_, alpha, relu, splits=args.splits, workspace=ws, stream=stream,
                                      kernel_id=kernel_id)
    else:
        # stacked matrices: (batch, M, K), (batch, K, N), (batch, M, N) views
        Av = A.view(w.batch, w.M, w.lda)[:, :, :w.K]
        Bv = B.view(w.batch, w.N, w.ldb)[:, :, :w.K].transpose(1, 2)
        Dv = D.view(w.batch, w.N, w.ldd)[:, :, :w.M].transpose(1, 2)
        plan = tg.plan_for_batched(Av, Bv, Dv, args.kernel_id)
        launch = tg.gemm_batched
    stream = torch.cuda.current_stream(dev)
    if launch is tg.gemm:
        # the plain product: marshal the arguments once, so that small
        # products are timed on the GPU and not on Python's call overhead
        bound = tg.bound_gemm(Av, Bv, Dv, w.alpha, w.relu, stream=stream, kernel_id=args.kernel_id)

        def launch(*_args, **_kw):
            bound()

    for _ in range(args.warmup):
        launch(Av, Bv, Dv, w.alpha, w.relu, stream=stream, kernel_id=args.kernel_id)
    torch.cuda.synchronize()
    # one event before every launch and one after the last, all on the stream
    # the kernel runs on: the whole-region average is the launch duration used
    # for the throughput and the roofline, the per-launch median is reported too
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i].record(stream)
        launch(Av, Bv, Dv, w.alpha, w.relu, stream=stream, kernel_id=args.kernel_id)
    ev[args.steps].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0].elapsed_time(ev[args.steps]) / args.steps
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    median_ms = per[len(per) // 2] if len(per) % 2 else 0.5 * (per[len(per) // 2 - 1] + per[len(per) // 2])
    tflops = w.flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "lda": w.lda, "ldb": w.ldb,
                   "ldd": w.ldd, "alpha": w.alpha, "relu": w.relu, "dist": w.dist,
                   "out_dtype": args.out_dtype, "batch": w.batch, "splits": args.splits,
                   "epilogue": args.epilogue,  # softmax: kernel_id below is the pointwise plan
                   "block_scales": bool(args.block_scales),
                   # with block scales tile_gemm_scaled picks among the instances that apply them
                   "kernel_id": None if args.block_scales else plan.kernel_id,
                   "staged": bool(plan.staged),  # A and B copied into aligned rows first (one more launch)
                   "tile": f"{plan.block_m}x{plan.block_n}x{plan.block_k}", "grid": plan.grid,
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "median_ms_per_launch": round(median_ms, 4),
        "wall_s_timed_region": round(wall, 4),
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "traffic": traffic_for(w.name if args.out_dtype == "f32" else f"{w.name}:out_{args.out_dtype}",
                                   plan.kernel_id),
        },
    }

    if not args.no_cpu_baseline:
        import numpy as np

        import oracle

        threads = oracle.default_threads()
        if args.epilogue == "softmax":
            # whole rows (every n) for rows m < rows
            rows = max(1, min(w.M, args.cpu_cols * 8))
            ms = np.repeat(np.arange(rows, dtype=np.int64)[None, :], w.N, axis=0).reshape(-1)
            ns = np.repeat(np.arange(w.N, dtype=np.int64), rows)
            t0 = time.perf_counter()
            ref, mag = oracle.gemm_entries(w.M, w.N, w.K, w.alpha, False, si.bits(A_st), w.lda, si.bits(B_st),
                                           w.ldb, w.dtype, ms, ns, threads=threads)
            cpu_s = time.perf_counter() - t0
            cpu_flops = 2.0 * rows * w.N * w.K
            ref, mag = ref.reshape(w.N, rows), mag.reshape(w.N, rows)
            cols = w.N
        else:
            cols = min(args.cpu_cols, w.N)  # of the first matrix of a batch
            t0 = time.perf_counter()
            extra = {}
            if args.block_scales:
                extra = dict(scale_a=sc_a_np, lds_a=sc_a_np.shape[1], scale_b=sc_b_np, lds_b=sc_b_np.shape[1])
            ref, mag = oracle.gemm(w.M, w.N, w.K, w.alpha, w.relu, si.bits(A_st), w.lda, si.bits(B_st), w.ldb,
                                   w.dtype, n0=0, n1=cols, threads=threads, **extra)
            cpu_s = time.perf_counter() - t0
            cpu_flops = 2.0 * w.M * cols * w.K
        result["cpu_baseline"] = {
            "value": round(cpu_flops / cpu_s / 1e12, 6),
            "unit": "TFLOP/s",
            "cores": threads,
            "kind": "oracle",
            "sample": (f"rows m < {rows}, every n, of the {w.M}x{w.N}x{w.K} logits (full K), fp64; "
                       f"{cpu_s:.2f} s wall" if args.epilogue == "softmax" else
                       f"output columns n < {cols} of the {w.M}x{w.N}x{w.K} workload"
                       f"{' (first product of the batch)' if w.batch > 1 else ''} (all m, full K), "
                       f"fp64; {cpu_s:.2f} s wall"),
        }
        if args.epilogue == "softmax":
            sub = D[:w.N, :rows]
            if args.out_dtype == "f32":
                d = sub.double().cpu().numpy()
            else:
                d = oracle.decode(sub.contiguous().view(torch.int16).cpu().numpy().view(np.uint16), args.out_dtype)
            ok, ratio = oracle.check_softmax(d, ref, mag, w.K, args.out_dtype)
        elif args.out_dtype == "f32":
            d = D[:cols, :w.M].double().cpu().numpy()
            ok, ratio = oracle.check(d, ref, mag, w.K)
        else:
            raw = D[:cols, :w.M].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            d = oracle.decode(raw, args.out_dtype)
            ok, ratio = oracle.check_out(d, ref, mag, w.K, args.out_dtype)
        result["parity"] = {"entries": int(d.size), "ok": bool(ok and not np.isnan(d).any()),
                            "worst_err_over_tol": round(ratio, 5)}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
