#!/usr/bin/env python3
"""Throughput of the tiled GEMM+ReLU on one MI355X, through the tile_gemm C ABI.

One step = one tile_gemm call on the measured workload (default: M=N=K=8192,
bf16 operands drawn from normal(0, 1/sqrt(K)), alpha=0.5, ReLU on, fp32 D),
inputs already resident in HBM.  Prints one JSON line with the throughput in
TFLOP/s (2MNK/t), the roofline position of the GEMM kernel, a parity check of
the output against the oracle on the CPU-baseline sample, and the oracle's own
throughput on the host cores.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--kernel-id ID]

The defaults (W = 50, K = 100) time the settled clock; with a short warmup
(W = 5, K = 20) the timed region still covers most of the power controller's
settling after an idle GPU, and the average runs about 5-8 % slower than the
per-launch median the line also reports.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "TFLOP/s (2MNK/t) bf16 GEMM+ReLU at 8192³; % of dense MFMA peak"
# MI355X dense peaks (no sparsity): 256 CUs at 2.4 GHz
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3, "e4m3": 5033.2, "e5m2": 5033.2, "e2m1": 10066.3,
               "e2m3": 10066.3, "e3m2": 10066.3}
ELEM_BYTES = {"bf16": 2, "f16": 2, "f32": 4, "e4m3": 1, "e5m2": 1, "e2m1": 0.5, "e2m3": 0.75, "e3m2": 0.75}
COUNTERS_FILE = ROOT / "profiles" / "counters.json"
PROFILES = ROOT / "profiles"
KERNEL_SOURCES = ROOT / "dense_tiled_gemm_tile_amd" / "csrc"
XCDS, SIMDS, SPEC_GHZ = 8, 1024, 2.4  # MI355X: 8 XCDs, 256 CUs x 4 SIMDs, 2.4 GHz peak engine clock


def kernel_sources(kernel_name: str) -> list[Path]:
    """The device sources one compiled kernel is built from (its instance unit
    and the headers every kernel unit includes)."""
    family = {"gemm_wide_kernel": ["gemm_wide.h", "gemm_wide16.hip", "gemm_wide32.hip", "gemm_wide8.hip",
                                   "gemm_wide4.hip", "gemm_wide6.hip"],
              "gemm_wide_m16_kernel": ["gemm_wide_m16.hip"], "gemm_stream_kernel": ["gemm_stream.hip"], "gemm_kernel": ["gemm_rs.hip"],
              "gemm_kslice_kernel": ["gemm_kslice.hip"],
              "splitk_reduce_kernel": ["gemm_aux.hip"], "stage_rows_kernel": ["gemm_aux.hip"]}
    base = ["gemm_common.h", "tile_math.h", "kernel_table.h"]
    for key, files in family.items():
        if f"::{key}<" in kernel_name or kernel_name.startswith(f"{key}<"):
            return [KERNEL_SOURCES / f for f in base + files]
    return sorted(p for p in KERNEL_SOURCES.iterdir() if p.suffix in (".hip", ".h"))


def kernel_source_hash(kernel_name: str = "") -> str:
    """Hash of the device sources of one kernel (all of them when unnamed)."""
    h = hashlib.sha256()
    for path in kernel_sources(kernel_name):
        h.update(path.name.encode())
        h.update(path.read_bytes())
    return h.hexdigest()[:16]


def counters_for(key: str, kernel_id: int):
    """The committed counter summary of this workload's kernel, if it was taken
    on the current sources of that kernel and the same instance; else None."""
    if not COUNTERS_FILE.exists():
        return None
    entry = json.loads(COUNTERS_FILE.read_text()).get(key)
    if (not entry or entry.get("kernel_id") != kernel_id
            or entry.get("source_hash") != kernel_source_hash(entry.get("kernel", ""))):
        return None
    return entry


def _csv_rows(path: Path) -> list[dict]:
    import csv

    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _per_dispatch(pmc_dir: Path, kernel: str) -> list[dict]:
    """Counter values and duration of every dispatch of `kernel` in one
    rocprofv3 --pmc output directory."""
    by = {}
    for r in _csv_rows(next(pmc_dir.rglob("*counter_collection.csv"))):
        if r["Kernel_Name"] != kernel:
            continue
        d = by.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["duration_s"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    return [by[k] for k in sorted(by)]


def summarize_profile(prof: Path, key: str, flops: float, alg_bytes: float, peak: float, command: str) -> dict:
    """Turn one workload's rocprofv3 outputs (kernel trace, counter passes
    pmc_A/pmc_B/pmc_FETCH_SIZE/pmc_WRITE_SIZE, and the copy calibration next
    to it) into a counters.json entry and a Markdown summary under profiles/.
    Dispatch 1 of each counter pass is the first launch in its process (cold
    TLBs and caches) and is left out of the means."""
    stats = _csv_rows(next((prof / "trace").rglob("*kernel_stats.csv")))
    top = max(stats, key=lambda r: float(r["TotalDurationNs"]))
    kernel = top["Name"]
    avg_ns = float(top["AverageNs"])
    warm = lambda rows: rows[1:] if len(rows) > 1 else rows
    a = warm(_per_dispatch(prof / "pmc_A", kernel))
    b = warm(_per_dispatch(prof / "pmc_B", kernel))
    mean = lambda rows, c: sum(r[c] for r in rows) / len(rows)
    clocks = [r["GRBM_GUI_ACTIVE"] / XCDS / r["duration_s"] / 1e9 for r in a]
    busy = [r["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * r["GRBM_GUI_ACTIVE"] / XCDS) for r in a]
    frac = [bz * ck / SPEC_GHZ for bz, ck in zip(busy, clocks)]
    frac_time = [flops / r["duration_s"] / 1e12 / peak for r in a]
    copy = prof.parent
    scale = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = [r for r in _csv_rows(next((copy / f"copy_{c}").rglob("*counter_collection.csv")))
                if r["Counter_Name"] == c]
        # the largest dispatches of the calibration run are the 256 MiB copies
        vals = sorted(float(r["Counter_Value"]) for r in rows)[-3:]
        scale[c] = 268435456 / (1024 * sum(vals) / len(vals))
    fetch = mean(warm(_per_dispatch(prof / "pmc_FETCH_SIZE", kernel)), "FETCH_SIZE")
    write = mean(warm(_per_dispatch(prof / "pmc_WRITE_SIZE", kernel)), "WRITE_SIZE")
    rd, wr = fetch * 1024 * scale["FETCH_SIZE"], write * 1024 * scale["WRITE_SIZE"]
    mops = [c for c in a[0] if c.startswith("SQ_INSTS_VALU_MFMA_MOPS_")]
    mfma_flops = sum(mean(a, c) for c in mops) * 512
    # GRBM_GUI_ACTIVE covers more than the dispatch itself (the counter window
    # opens before the first wave and closes after the last), which only
    # matters for short kernels: no clock or busy fraction below 50 us
    short = avg_ns < 50e3
    entry = {
        "kernel": kernel, "source_hash": kernel_source_hash(kernel),
        "sources": [p.name for p in kernel_sources(kernel)],
        "trace_average_ns": round(avg_ns), "trace_calls": int(top["Calls"]),
        "effective_sclk_ghz": None if short else round(sum(clocks) / len(clocks), 3),
        "mfma_busy_frac": None if short else round(sum(busy) / len(busy), 4),
        "mfma_util_pct_rocprof": round(mean(b, "MfmaUtil"), 2) if b and "MfmaUtil" in b[0] else None,
        "frac_from_counters": None if short else round(sum(frac) / len(frac), 4),
        "frac_from_duration": round(sum(frac_time) / len(frac_time), 4),
        "mfma_flops_counted": mfma_flops, "flops_2mnk": flops,
        "mfma_insts": mean(a, "SQ_INSTS_MFMA"), "valu_insts": mean(a, "SQ_INSTS_VALU"),
        "salu_insts": mean(a, "SQ_INSTS_SALU"), "lds_bank_conflict_cycles": mean(a, "SQ_LDS_BANK_CONFLICT"),
        "lds_insts": mean(b, "SQ_INSTS_LDS") if b and "SQ_INSTS_LDS" in b[0] else None,
        "read_bytes": round(rd), "write_bytes": round(wr), "hbm_bytes_per_launch": round(rd + wr),
        "algorithmic_bytes": alg_bytes, "fetch_scale": round(scale["FETCH_SIZE"], 4),
        "write_scale": round(scale["WRITE_SIZE"], 4),
        "per_dispatch": [{"ms": round(r["duration_s"] * 1e3, 4), "sclk_ghz": round(ck, 3), "mfma_busy": round(bz, 4)}
                         for r, ck, bz in zip(a, clocks, busy)],
    }
    name = re.sub(r"[^A-Za-z0-9]+", "_", kernel.split("(")[0].replace("void tg::", "")).strip("_")
    md = PROFILES / f"{name}__{key.replace(':', '_')}.md"
    entry["summary"] = str(md.relative_to(ROOT))
    lines = [
        f"# `{kernel}` — {key}", "",
        f"Kernel trace (`rocprofv3 --kernel-trace --stats`): {entry['trace_calls']} dispatches, average "
        f"{avg_ns:.0f} ns, min {float(top['MinNs']):.0f} ns, max {float(top['MaxNs']):.0f} ns; "
        f"{flops / avg_ns / 1e3:.1f} TFLOP/s at the average (2MNK/t), {flops / avg_ns / 1e3 / peak:.4f} of "
        f"the {peak} TFLOP/s dense peak.", "",
        "Counters per dispatch (the first launch of each counter run left out)" + (
            "; the kernel is shorter than 50 us, so the clock and busy columns, which divide by the "
            "GRBM_GUI_ACTIVE window (longer than the dispatch), are not meaningful here:" if short else ":"), "",
        "| dispatch ms | effective SCLK GHz (GRBM_GUI_ACTIVE / 8 XCDs / duration) | MFMA busy "
        "(SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8)) | busy x SCLK / 2.4 GHz | 2MNK / t / peak |",
        "|---|---|---|---|---|",
    ]
    for r, ck, bz, fr, ft in zip(a, clocks, busy, frac, frac_time):
        lines.append(f"| {r['duration_s'] * 1e3:.3f} | {ck:.3f} | {bz:.4f} | {fr:.4f} | {ft:.4f} |")
    lines += [
        "", "| quantity | value |", "|---|---|",
        f"| MFMA instructions (SQ_INSTS_MFMA) | {entry['mfma_insts']:.4g} |",
        f"| MFMA flops counted (MOPS x 512) / 2MNK | {mfma_flops / flops:.4f} |",
        f"| rocprof MfmaUtil (%) | {entry['mfma_util_pct_rocprof']} |",
        f"| VALU instructions incl. MFMA (SQ_INSTS_VALU) | {entry['valu_insts']:.4g} |",
        f"| SALU instructions (SQ_INSTS_SALU) | {entry['salu_insts']:.4g} |",
        f"| LDS instructions (SQ_INSTS_LDS) | {entry['lds_insts']} |",
        f"| LDS bank-conflict cycles (SQ_LDS_BANK_CONFLICT) | {entry['lds_bank_conflict_cycles']:.4g} |",
        f"| FETCH_SIZE x {scale['FETCH_SIZE']:.3f} (read bytes / launch) | {rd:.4g} |",
        f"| WRITE_SIZE x {scale['WRITE_SIZE']:.3f} (written bytes / launch) | {wr:.4g} |",
        f"| algorithmic bytes (A, B read once, D written once) | {alg_bytes:.4g} |", "",
        "FETCH_SIZE and WRITE_SIZE are scaled by what the same counters read for a plain 256 MiB device "
        "copy (`bench.py --copy-calibration 268435456`).", "",
        "Commands (from /tmp with TMPDIR=/tmp; `$R` is the repository root, `$O` the output folder):", "",
        "```",
        f"rocprofv3 --kernel-trace --stats --output-format csv -d $O/trace -o run -- python3 $R/bench.py {command} "
        "--steps 20 --warmup 5 --no-cpu-baseline",
        f"rocprofv3 --pmc {' '.join(sorted(k for k in a[0] if k != 'duration_s'))} --output-format csv -d $O/pmc_A "
        f"-o run -- python3 $R/bench.py {command} --steps 3 --warmup 1 --no-cpu-baseline",
        f"rocprofv3 --pmc {' '.join(sorted(k for k in b[0] if k != 'duration_s'))} --output-format csv -d $O/pmc_B "
        f"-o run -- python3 $R/bench.py {command} --steps 3 --warmup 1 --no-cpu-baseline" if b else "",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d $O/pmc_FETCH_SIZE -o run -- python3 $R/bench.py {command} "
        "--steps 3 --warmup 1 --no-cpu-baseline   (then WRITE_SIZE the same way)",
        "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $O/../copy_FETCH_SIZE -o run -- python3 $R/bench.py "
        "--copy-calibration 268435456   (then WRITE_SIZE the same way)",
        "```", "",
    ]
    md.write_text("\n".join(line for line in lines if line is not None) + "\n")
    data = json.loads(COUNTERS_FILE.read_text()) if COUNTERS_FILE.exists() else {}
    data[key] = {"kernel_id": None, **entry}
    COUNTERS_FILE.write_text(json.dumps(data, indent=1, sort_keys=True) + "\n")
    return data[key]


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
    # defaults long enough for the power controller to settle: after an idle
    # GPU the 8192^3 launches run 0.83 ms, then 1.0-1.07 ms, and only after
    # about 30 launches (25 ms of load) their steady 0.80 ms
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
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
                    help="8- and 4-bit workloads: seeded block scales (one exponent per 32 k of every A row and "
                         "B column) through tile_gemm_scaled")
    ap.add_argument("--cpu-cols", type=int, default=4096,
                    help="output columns the CPU-baseline oracle computes (all rows, full K)")
    ap.add_argument("--staged", action="store_true",
                    help="single products through tile_gemm_staged (mode -1) with a workspace allocated up front "
                         "through torch: misaligned rows are first copied into aligned rows when that pays")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="host only: summarise the rocprofv3 outputs in DIR (trace/, pmc_*/; the copy calibration "
                         "in DIR/..) of this workload into profiles/ and profiles/counters.json")
    ap.add_argument("--profile-kernel-id", type=int, default=None,
                    help="with --summarize-profile: the instance the profiled run launched")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the GEMM shards into independent column panels, one per GPU, with no exchange)",
              file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return 0
    if args.summarize_profile:
        import seeded_inputs as si

        w = si.WORKLOADS[args.workload]
        os_ = {"f32": 4, "bf16": 2, "f16": 2}[args.out_dtype]
        es = ELEM_BYTES[w.dtype]
        alg = float(w.batch * ((w.M * w.K + w.K * w.N) * es + w.M * w.N * os_))
        key = w.name if args.out_dtype == "f32" else f"{w.name}:out_{args.out_dtype}"
        cmd = f"--workload {w.name}" + (f" --out-dtype {args.out_dtype}" if args.out_dtype != "f32" else "")
        entry = summarize_profile(Path(args.summarize_profile), key, w.flops, alg, PEAK_TFLOPS[w.dtype], cmd)
        if args.profile_kernel_id is not None:
            data = json.loads(COUNTERS_FILE.read_text())
            data[key]["kernel_id"] = args.profile_kernel_id
            COUNTERS_FILE.write_text(json.dumps(data, indent=1, sort_keys=True) + "\n")
        print(json.dumps({k: entry[k] for k in ("kernel", "effective_sclk_ghz", "mfma_busy_frac",
                                                "frac_from_counters", "frac_from_duration", "summary")}))
        return 0

    import torch

    import dense_tiled_gemm_tile_amd as tg
    import seeded_inputs as si

    w = si.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    A_st, B_st = si.workload_operands(w)
    A, B = A_st.to(dev), B_st.to(dev)
    kv = w.K  # storage columns holding K
    if w.dtype == "e2m1":  # packed pairs: torch's two-element storage type
        A, B, kv = A.view(torch.float4_e2m1fn_x2), B.view(torch.float4_e2m1fn_x2), w.K // 2
    raw = w.dtype in ("e2m3", "e3m2")  # 6-bit: no torch type, raw pointers and element strides
    out_torch = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[args.out_dtype]
    D = si.out_storage(w.M, w.batch * w.N, w.ldd).to(out_torch).to(dev)
    if raw:
        if w.batch != 1 or args.staged or args.splits != 1 or args.epilogue != "pointwise":
            print("6-bit workloads: plain and block-scaled single products only", file=sys.stderr)
            return 2
        code, ocode = tg.DTYPE_CODES[w.dtype], tg.DTYPE_CODES[args.out_dtype]
        Av = Bv = Dv = None
        lib = tg.load_library()
        s_ptr = torch.cuda.current_stream(dev).cuda_stream
        if args.block_scales:
            sc_a_np = si.block_scales(w.M, w.K, w.seed_a + 50, dtype=w.dtype)
            sc_b_np = si.block_scales(w.N, w.K, w.seed_b + 50, dtype=w.dtype)
            sc_a, sc_b = torch.from_numpy(sc_a_np).to(dev), torch.from_numpy(sc_b_np).to(dev)
            fn, fargs = lib.tile_gemm_scaled, (w.M, w.N, w.K, float(w.alpha), int(w.relu), A.data_ptr(), w.lda,
                                               sc_a.data_ptr(), sc_a_np.shape[1], B.data_ptr(), w.ldb,
                                               sc_b.data_ptr(), sc_b_np.shape[1], D.data_ptr(), w.ldd, code, ocode,
                                               s_ptr, args.kernel_id)
            plan = tg.query_plan_scaled(w.M, w.N, w.K, code, A.data_ptr(), w.lda, sc_a.data_ptr(), sc_a_np.shape[1],
                                        B.data_ptr(), w.ldb, sc_b.data_ptr(), sc_b_np.shape[1], D.data_ptr(), w.ldd,
                                        ocode, args.kernel_id)
        else:
            fn, fargs = lib.tile_gemm_out, (w.M, w.N, w.K, float(w.alpha), int(w.relu), A.data_ptr(), w.lda,
                                            B.data_ptr(), w.ldb, D.data_ptr(), w.ldd, code, ocode, s_ptr,
                                            args.kernel_id)
            plan = tg.query_plan(w.M, w.N, w.K, code, A.data_ptr(), w.lda, B.data_ptr(), w.ldb, D.data_ptr(), w.ldd,
                                 args.kernel_id, ocode)

        def launch(*_args, **_kw):
            rc = fn(*fargs)
            if rc != 0:
                raise tg.TileGemmError(rc, tg.strerror(rc))
    elif w.batch == 1:
        Av, Bv, Dv = A[:, :kv], B[:, :kv].t(), D[:, :w.M].t()
        plan = tg.plan_for(Av, Bv, Dv, args.kernel_id)
        launch = tg.gemm
        if args.epilogue == "softmax":
            def launch(A_, B_, D_, alpha, relu, stream=None, kernel_id=-1):
                return tg.gemm_softmax(A_, B_, D_, alpha, stream=stream, kernel_id=kernel_id)
        if args.block_scales:
            if w.dtype not in ("e4m3", "e5m2", "e2m1"):
                print("--block-scales needs an 8- or 4-bit workload", file=sys.stderr)
                return 2
            sc_a_np = si.block_scales(w.M, w.K, w.seed_a + 50, dtype=w.dtype)
            sc_b_np = si.block_scales(w.N, w.K, w.seed_b + 50, dtype=w.dtype)
            sc_a, sc_b = torch.from_numpy(sc_a_np).to(dev), torch.from_numpy(sc_b_np).to(dev)

            def launch(A_, B_, D_, alpha, relu, stream=None, kernel_id=-1):
                return tg.gemm_scaled(A_, B_, D_, sc_a, sc_b, alpha, relu, stream=stream, kernel_id=kernel_id)
        if args.staged:
            ws_bytes = max(tg.staged_workspace_bytes(w.M, w.N, w.K, tg.DTYPE_CODES[w.dtype]), 256)
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
            plan = tg.query_plan_staged(w.M, w.N, w.K, tg.DTYPE_CODES[w.dtype], Av.data_ptr(), w.lda, Bv.data_ptr(),
                                        w.ldb, Dv.data_ptr(), w.ldd, tg.DTYPE_CODES[args.out_dtype] if args.out_dtype
                                        != "f32" else tg.F32, ws.data_ptr(), ws_bytes, -1)

            def launch(A_, B_, D_, alpha, relu, stream=None, kernel_id=-1):
                return tg.gemm_staged(A_, B_, D_, alpha, relu, workspace=ws, mode=-1, stream=stream)
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
    # the timed region: one event before the first launch and one after the
    # last, both on the stream the kernel runs on, and the launches back to
    # back between them; the region average is the launch duration used for
    # the throughput and the roofline.  A second, untimed-for-throughput pass
    # with an event between every two launches gives the per-launch median
    # (those events add a gap per launch, which matters for short kernels).
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        launch(Av, Bv, Dv, w.alpha, w.relu, stream=stream, kernel_id=args.kernel_id)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for i in range(args.steps):
        ev[i].record(stream)
        launch(Av, Bv, Dv, w.alpha, w.relu, stream=stream, kernel_id=args.kernel_id)
    ev[args.steps].record(stream)
    torch.cuda.synchronize()
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
                   # A and B copied into aligned rows of a workspace first (one more launch)
                   "staged": bool(plan.staged),
                   "workspace_bytes": (ws_bytes if args.staged else None),
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
            "traffic": None,
        },
    }
    # counters from the committed rocprofv3 summary of this kernel (null when
    # the kernel sources changed since they were taken)
    key = w.name if args.out_dtype == "f32" else f"{w.name}:out_{args.out_dtype}"
    cnt = None if (args.staged or args.block_scales or args.splits != 1 or args.epilogue != "pointwise") else \
        counters_for(key, plan.kernel_id)
    if cnt:
        result["roofline"]["traffic"] = cnt.get("hbm_bytes_per_launch")
    result["counters"] = None if not cnt else {
        "effective_sclk_ghz": cnt.get("effective_sclk_ghz"),
        "mfma_busy_frac": cnt.get("mfma_busy_frac"),
        "frac_from_counters": cnt.get("frac_from_counters"),
        "summary": cnt.get("summary"),
    }

    if not args.no_cpu_baseline:
        import numpy as np

        import oracle

        threads = oracle.default_threads()
        cores = oracle.affinity_cores()
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
            "cores": cores,
            "threads": threads,
            "cpu_quota": oracle.cpu_quota(),
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
