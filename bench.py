#!/usr/bin/env python
"""Benchmark of the emulated fp64 GEMM (Ozaki scheme II through int8 MFMA) on one MI355X.

One step = one ozk_dgemm_ex call on the largest single-GPU fp64 GEMM workload: 8192 x 8192
x 8192 with entries (U(0,1) - 0.5) exp(4 N(0,1)) (seed 3, the wide-dynamic-range case),
r = 16 moduli and the norm (Cauchy-Schwarz) row/column scaling, the configuration that
reaches normwise 1e-15 against the exact product with the fewest moduli (the max rule
needs r = 18 there: `--scaling max --r 18`).  A step is the whole hot path: column
scaling of B, deconstruction of A and B, 16 int8 MFMA products with the residue epilogue,
CRT reconstruction.  Inputs are resident in HBM before timing starts.  `value` is
emulated fp64 TFLOP/s = 2 m n k / t.

Also reported on the same JSON line:
  roofline      the dominant kernel (batched int8 MFMA products with the residue
                epilogue) timed inside the timed steps, one HIP event pair per launch
                recorded by the launch itself: r * 2 * m * n * kp int8 ops per launch
                against the 5.0 POP/s dense int8 MFMA peak; HBM traffic per launch from
                the committed rocprofv3 counter summary when it matches the kernel source
                (made by `--counters` under two `rocprofv3 --pmc` passes, then
                `--traffic-summary FETCH_DIR WRITE_DIR`).
  cpu_baseline  the CPU oracle (numpy; its matrix products on every BLAS thread) on a
                sampled block of 256 x 1024 outputs of the same workload, with the time of
                each phase (scaling, residues, modular products, CRT).
  extras        native fp64 DGEMM (torch.matmul), the 4096^3 square workload (r sweep
                12..18 under both scaling rules, deconstruction HBM GB/s), the wide-range
                workload at r = 16..20 under both rules, the GEMV and FP4-limb engines, and
                the emulated SpMV of the 7-point Poisson operator on a 256^3 grid.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--r 16] [--scaling norm|max]
                       [--no-cpu-baseline] [--no-extras]
       python bench.py --counters            (launches only, for rocprofv3 --pmc)
       python bench.py --traffic-summary FETCH_DIR WRITE_DIR
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("emulated FP64 GEMM TFLOP/s and % int8-MFMA peak; deconstruction/GEMV HBM GB/s")
PEAK_INT8_TOPS = 5000.0     # dense int8 MFMA, TOP/s
PEAK_FP4_TFLOPS = 10100.0   # dense FP4 MFMA
PEAK_HBM_GBS = 8000.0
# The timed workload: the wide-dynamic-range fp64 GEMM.
M = N = K = 8192
SEED = 3
PHI = 4.0
DEFAULT_R = 16
DEFAULT_SCALING = "norm"
# The square workload reported among the extras.
SQ = 4096
SQ_SEED = 2
SQ_PHI = 0.5


def _source_digest(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "fp64_gemm_emulation_ozk_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _time_events(fn, reps: int, stream, warm_ms: float = 80.0, warm_fn=None) -> float:
    """Average milliseconds per call of fn over reps calls, HIP events on `stream`, after
    calling warm_fn (default fn) back to back for at least warm_ms (the board's clocks take
    some 50-65 ms of load to settle after a change of workload).  A fn that may run only
    reps times (one that consumes per-call state) passes an equivalent warm_fn."""
    import torch

    if warm_ms > 0:
        warm = fn if warm_fn is None else warm_fn
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < warm_ms:
            warm()
            torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / reps


TRAFFIC_PATH = os.path.join(ROOT, "profiles", "traffic_dgemm_8192_r16_norm.json")
COPY_BYTES = 1 << 30   # calibration copy (elementwise negation): 1 GiB read + 1 GiB written


def _traffic(kernel: str, digest: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on this
    exact kernel source; else None."""
    try:
        with open(TRAFFIC_PATH) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = data.get("kernels", {}).get(kernel)
    if not ent or ent.get("source_digest") != digest:
        return None
    return ent.get("hbm_bytes_per_launch")


# Kernels summarised from the counter passes: key -> (kernel-name substring, sources).
COUNTER_KERNELS = {
    "gemm_i8_residues": ("gemm_i8_pairs_kernel<1", ["gemm_i8.hip"]),
    "deconstruct_pair": ("deconstruct_pair_kernel", ["deconstruct.hip"]),
    "norm_partials_cols": ("norm_partials_cols_kernel", ["deconstruct.hip"]),
    "exps_norm": ("exps_norm_kernel", ["deconstruct.hip"]),
    "residues_rows_fused": ("residues_rows_fused_kernel", ["deconstruct.hip"]),
    "residues_cols": ("residues_cols_kernel", ["deconstruct.hip"]),
    "crt": ("crt_kernel<16", ["crt.hip"]),
}


# Kernels of the other engines, summarised when the counter workload ran them
# (`--counters all`): key -> (kernel-name substring, sources, algorithmic bytes per launch).
COUNTER_KERNELS_EXTRA = {
    "gemv_digits_1col": ("gemv_digits_kernel<1, 1, true>", ["gemv_digits.hip"], 8 * 32768 * 32768),
    "gemv_digits_8cols": ("gemv_digits_kernel<7, 1, true>", ["gemv_digits.hip"], 8 * 32768 * 32768),
    "gemv_fly_32cols": ("gemv_fly_kernel<false, 0, 14, 2, true>", ["gemv.hip"],
                        8 * 32768 * 32768),
    "gemv_stored_1col": ("gemv_stored_kernel", ["gemv.hip"], 14 * 32768 * 32768),
    "fp4_gemm": ("fp4_gemm_kernel", ["fp4limb.hip"], None),
    "fp4awe_gemm": ("awe_gemm_kernel", ["fp4awe.hip"], None),
    "fp4awe4_gemm": ("awe4_gemm_kernel", ["fp4awe4.hip"], None),
    # full kernel names: "::pack_rows_kernel(" is the 9-product packer alone
    "fp4_pack_rows": ("::pack_rows_kernel(", ["fp4limb.hip", "fp4_pack.h"],
                      8192 * 8192 * (1 + 1.5)),
    "fp4_pack_cols": ("::pack_cols_kernel(", ["fp4limb.hip", "fp4_pack.h"],
                      8192 * 8192 * (1 + 1.5)),
    "fp4awe_pack_rows": ("awe_pack_rows_kernel(", ["fp4awe.hip", "fp4_pack.h"],
                         8192 * 8192 * (1 + 3)),
    "fp4awe_pack_cols": ("awe_pack_cols_kernel(", ["fp4awe.hip", "fp4_pack.h"],
                         8192 * 8192 * (1 + 3)),
    "fp4awe4_pack_rows_int4": ("awe4_pack_rows_kernel<true>(", ["fp4awe4.hip", "fp4_pack.h"],
                               8192 * 8192 * (1 + 2)),
    "fp4awe4_pack_cols_int8": ("awe4_pack_cols_kernel<false>(", ["fp4awe4.hip", "fp4_pack.h"],
                               8192 * 8192 * (1 + 2)),
    "spmv_rows_r14": ("spmv_residues_kernel<true, 14>", ["spmv.hip"], None),
}


def run_counter_workload(extra: bool = False) -> int:
    """Launches profiled by the rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE, or
    instruction and utilisation counters): a plain device copy of COPY_BYTES
    (calibration), then two default steps (their kernels: column norms of B, the paired
    deconstruction of A and B, the residue GEMM, CRT) and each operand's deconstruction on
    its own.  With `extra`, also one call of each other engine at its workload size: the
    32768^2 GEMV at r = 14 (digits path at 1 and 8 columns, residue path at 32, stored
    planes at 1), the 8192^3 INT8 product through FP4 limbs and the emulated SpMV of the
    256^3 Poisson operator at r = 14 (so that every crt_kernel<16> launch is a DGEMM
    step's).  Nothing is timed."""
    import torch

    import fp64_gemm_emulation_ozk_amd as ozk
    import ozk_inputs

    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 8, dtype=torch.float64, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.neg(src, out=dst)     # one plain streaming read and write of COPY_BYTES
    torch.cuda.synchronize()
    del src, dst
    a, b = ozk_inputs.gemm_operands(M, N, K, seed=SEED, dist="phi", phi=PHI)
    da, db = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    del a, b
    r, rule = DEFAULT_R, DEFAULT_SCALING
    out = torch.empty((M, N), dtype=torch.float64, device=dev)
    ws = torch.empty(ozk.ozk_dgemm_workspace_size(M, N, K, r), dtype=torch.uint8, device=dev)
    for _ in range(2):
        ozk.ozk_dgemm_ex(da, db, r, rule, out=out, workspace=ws)
    # each operand's deconstruction on its own (the step runs them in one launch)
    ozk.ozk_deconstruct_ex(da, 0, r, rule)
    ozk.ozk_deconstruct_ex(db, 1, r, rule, k_budget=K)
    torch.cuda.synchronize()
    del da, db, out, ws
    torch.cuda.empty_cache()
    if extra:
        import numpy as np

        mg = 32768
        ga = ozk_inputs.uniform_matrix_device((mg, mg), 4, dev)
        x_all = torch.from_numpy(ozk_inputs.uniform_matrix(np.random.default_rng(4),
                                                           (mg, 32))).to(dev)
        planes, exps = ozk.ozk_deconstruct(ga, 0, 14, k_budget=mg)
        for nrhs in (1, 8, 32):
            ozk.ozk_dgemv(ga, x_all[:, :nrhs].contiguous(), 14, mode=0, a_exps=exps)
        ozk.ozk_dgemv(None, x_all[:, :1].contiguous(), 14, mode=1, a_planes=planes, a_exps=exps)
        torch.cuda.synchronize()
        del ga, planes, x_all
        torch.cuda.empty_cache()
        ia, ib = (torch.from_numpy(t).to(dev) for t in ozk_inputs.int8_operands(8192, 8192, 8192,
                                                                                 seed=5))
        ozk.ozk_int8gemm_fp4limb(ia, ib)
        ozk.ozk_int8gemm_fp4awe(ia, ib)
        ozk.ozk_int4int8gemm_fp4awe(ia, ib)     # A read as int4 (low nibbles)
        torch.cuda.synchronize()
        del ia, ib
        rp, ci, v = ozk_inputs.poisson_7pt_csr(256)
        drp, dci, dv = (torch.from_numpy(t).to(dev) for t in (rp, ci, v))
        xs = torch.from_numpy(ozk_inputs.uniform_matrix(np.random.default_rng(7),
                                                        (256 ** 3, 1))[:, 0]).to(dev)
        ozk.ozk_spmv_csr(drp, dci, dv, xs, 14, 7)
        torch.cuda.synchronize()
    print("counter workload done", flush=True)
    return 0


def _counter_means(run_dir: str, counter: str) -> dict:
    """Mean per-dispatch value of `counter` for each kernel name in a rocprofv3 csv run."""
    import csv
    import glob

    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    acc = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                acc.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def traffic_summary(fetch_dir: str, write_dir: str, out_path: str | None = None) -> int:
    """Turn the two counter passes into per-launch HBM bytes, scaled by what the same
    counters read for the calibration copy, and write out_path (default TRAFFIC_PATH)."""
    out_path = out_path or TRAFFIC_PATH
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")

    def pick(table, sub):
        hits = [v for k, v in table.items() if sub in k]
        if not hits:
            raise SystemExit(f"kernel {sub!r} not found among {sorted(table)[:8]}")
        return sum(hits) / len(hits)

    copy_f, copy_w = pick(fetch, "neg_kernel"), pick(write, "neg_kernel")   # KiB per dispatch
    f_fac = COPY_BYTES / (copy_f * 1024.0)
    w_fac = COPY_BYTES / (copy_w * 1024.0)
    data = {"what": "L2-to-fabric bytes per launch (HBM or MALL) from rocprofv3 FETCH_SIZE and "
                    "WRITE_SIZE (KiB per dispatch), each scaled by the factor that maps the "
                    "same counter on a plain 1 GiB device copy to 1 GiB",
            "commands": [
                "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv "
                "-d <out>/fetch -o out -- python3 <repo>/bench.py --counters",
                "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv "
                "-d <out>/write -o out -- python3 <repo>/bench.py --counters",
                "python3 bench.py --traffic-summary <out>/fetch <out>/write"],
            "calibration": {"copy_bytes": COPY_BYTES, "fetch_kib": copy_f, "write_kib": copy_w,
                            "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)},
            "kernels": {}}
    for key, (sub, srcs) in COUNTER_KERNELS.items():
        fb = pick(fetch, sub) * 1024.0 * f_fac
        wb = pick(write, sub) * 1024.0 * w_fac
        data["kernels"][key] = {"kernel": sub, "fetch_bytes": round(fb), "write_bytes": round(wb),
                                "hbm_bytes_per_launch": round(fb + wb),
                                "source_digest": _source_digest(srcs)}
    for key, (sub, srcs, algo) in COUNTER_KERNELS_EXTRA.items():
        if not any(sub in k for k in fetch) or not any(sub in k for k in write):
            continue
        fb = pick(fetch, sub) * 1024.0 * f_fac
        wb = pick(write, sub) * 1024.0 * w_fac
        ent = {"kernel": sub, "fetch_bytes": round(fb), "write_bytes": round(wb),
               "hbm_bytes_per_launch": round(fb + wb), "source_digest": _source_digest(srcs)}
        if algo:
            ent["algorithmic_bytes"] = algo
            ent["traffic_over_algorithmic"] = round((fb + wb) / algo, 3)
        data["kernels"][key] = ent
    with open(out_path, "w") as fh:
        json.dump(data, fh, indent=1)
        fh.write("\n")
    print(json.dumps(data, indent=1))
    return 0


def pmc_summary(run_dir: str, out_json: str) -> int:
    """Per-kernel mean per dispatch of every counter found in a rocprofv3 --pmc csv run
    (kernel names shortened to their template head), written to out_json."""
    import csv
    import glob
    import re

    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    acc = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                name = re.sub(r"\(.*$", "", re.sub(r"ozk::\(anonymous namespace\)::|^void ", "",
                                                  row["Kernel_Name"]))[:80]
                ent = acc.setdefault(name, {})
                ent.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
                ent.setdefault("_ns", {})[row["Dispatch_Id"]] = (
                    int(row["End_Timestamp"]) - int(row["Start_Timestamp"]))
    out = {"what": "per-dispatch means of rocprofv3 --pmc counters, per kernel", "kernels": {}}
    for name, ent in acc.items():
        ns = ent.pop("_ns")
        row = {c: round(sum(v) / len(v), 1) for c, v in ent.items()}
        row["dispatches"] = len(ns)
        row["mean_duration_us"] = round(sum(ns.values()) / len(ns) / 1e3, 1)
        out["kernels"][name] = row
    with open(out_json, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out, indent=1))
    return 0


TME_COUNTERS = ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_WAVES",
                "GRBM_GUI_ACTIVE"]
TME_PATH = os.path.join(ROOT, "profiles", "tme_counters.json")
# Kernels whose instruction counts calibrate the time model: key -> (kernel-name
# substring, unit the counts are divided by, number of units per dispatch, moduli).
TME_KERNELS = {
    "decon_rows_wide_4096_r16": ("residues_rows_fused_kernel<true, true, 256, 2, false>",
                                 "element", 4096 * 4096, 16),
    "decon_rows_narrow_32768_r14": ("residues_rows_fused_kernel<false, true, 1024, 4, false>",
                                    "element", 32768 * 32768, 14),
    "decon_cols_wide_4096_r16": ("residues_cols_kernel<true, false>", "element", 4096 * 4096,
                                 16),
    "gemv_fly_32768_r14_32cols": ("gemv_fly_kernel<false, 0, 14, 2, true>", "element of A",
                                  32768 * 32768, 14),
    "gemv_digits_32768_r14_1col": ("gemv_digits_kernel<1, 1, true>", "element of A", 32768 * 32768, 14),
    "gemv_digits_32768_r14_8cols": ("gemv_digits_kernel<7, 1, true>", "element of A", 32768 * 32768, 14),
    "gemv_stored_32768_r14_1col": ("gemv_stored_kernel", "element of A", 32768 * 32768, 14),
    "crt_4096_r16": ("crt_kernel<16", "output", 4096 * 4096, 16),
    "gemm_i8_4096_r16": ("gemm_i8_pairs_kernel<1,", "output x modulus", 4096 * 4096 * 16,
                         16),
}


def run_tme_workload() -> int:
    """Launches profiled by the time-model counter pass (instruction counts only; nothing
    is timed): two DGEMM steps of the 4096^3 r=16 workload and each operand's
    deconstruction on its own, then the 32768^2 r=14 GEMV
    workload's deconstruction and one on-the-fly call for 1, 8 and 32 columns and one
    stored-plane call for 1 column."""
    import numpy as np
    import torch

    import fp64_gemm_emulation_ozk_amd as ozk
    import ozk_inputs

    dev = torch.device("cuda:0")
    a, b = ozk_inputs.gemm_operands(SQ, SQ, SQ, seed=SQ_SEED, dist="phi", phi=SQ_PHI)
    da, db = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    out = torch.empty((SQ, SQ), dtype=torch.float64, device=dev)
    ws = torch.empty(ozk.ozk_dgemm_workspace_size(SQ, SQ, SQ, 16), dtype=torch.uint8, device=dev)
    for _ in range(2):
        ozk.ozk_dgemm(da, db, 16, out=out, workspace=ws)
    ozk.ozk_deconstruct(da, 0, 16)
    ozk.ozk_deconstruct(db, 1, 16, k_budget=SQ)
    torch.cuda.synchronize()
    del da, db, out, ws
    mg, r = 32768, 14
    ga = ozk_inputs.uniform_matrix_device((mg, mg), 4, dev)
    x_all = torch.from_numpy(ozk_inputs.uniform_matrix(np.random.default_rng(4), (mg, 32))).to(dev)
    planes, exps = ozk.ozk_deconstruct(ga, 0, r, k_budget=mg)
    for nrhs in (1, 8, 32):
        dx = x_all[:, :nrhs].contiguous()
        ozk.ozk_dgemv(ga, dx, r, mode=0, a_exps=exps)
    ozk.ozk_dgemv(None, x_all[:, :1].contiguous(), r, mode=1, a_planes=planes, a_exps=exps)
    torch.cuda.synchronize()
    print("time-model counter workload done", flush=True)
    return 0


def tme_summary(run_dir: str) -> int:
    """Per-dispatch instruction counts of the calibration kernels from one rocprofv3 --pmc
    pass over the TME_COUNTERS, and the per-unit figures the time model uses (vector
    instructions x 64 lanes per element per modulus = c_q)."""
    means = {c: _counter_means(run_dir, c) for c in TME_COUNTERS}
    data = {"what": "rocprofv3 --pmc " + " ".join(TME_COUNTERS) + " over `bench.py "
                    "--tme-counters`; instruction counts are per wave (64 lanes)",
            "commands": [
                "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc " + " ".join(TME_COUNTERS) +
                " --output-format csv -d <out> -o out -- python3 <repo>/bench.py --tme-counters",
                "python3 bench.py --tme-summary <out>"],
            "kernels": {}}
    for key, (sub, unit, units, r) in TME_KERNELS.items():
        ent = {"kernel": sub, "unit": unit, "units_per_dispatch": units, "r": r}
        for c in TME_COUNTERS:
            hits = [v for k, v in means[c].items() if sub in k]
            ent[c] = round(sum(hits) / len(hits), 1) if hits else None
        valu, mfma = ent["SQ_INSTS_VALU"], ent["SQ_INSTS_MFMA"]
        if valu is not None and mfma is not None:
            vec = max(valu - mfma, 0.0)
            ent["vector_lane_ops_per_unit"] = round(vec * 64 / units, 3)
            ent["vector_lane_ops_per_unit_per_modulus"] = round(vec * 64 / units / r, 3)
            ent["mfma_per_unit"] = round(mfma / units, 6)
        data["kernels"][key] = ent
    with open(TME_PATH, "w") as fh:
        json.dump(data, fh, indent=1)
        fh.write("\n")
    print(json.dumps(data, indent=1))
    return 0


P_FP64 = 78.6e12          # fp64 FLOP/s (datasheet, vector and matrix)
P_VALU = 256 * 4 * 16 * 2.4e9   # vector lane-operations per second: 256 CUs x 4 SIMDs x 16 lanes


def tme_model(extras: dict, hbm: dict) -> dict | None:
    """Page 1's four-term time model instantiated on this GPU: T = max(T_tensor, T_HBM) +
    T_recon + T_decon, with T_decon = c_q r N / P_int the per-input deconstruction term.
    Instruction counts come from the committed counter pass (profiles/tme_counters.json:
    vector lane-operations and MFMA instructions per element, per kernel); rates are the
    datasheet ones (int8 MFMA 5.0 POP/s, HBM 8 TB/s, vector lane-operations 39.3 T/s).
    Returns the threshold OI* = c_q r P_fp64 / (8 P_int), the per-element instruction
    budget below which an on-the-fly GEMV can stream at memory speed, and
    model-versus-measured times of the GEMV paths and the 4096^3 DGEMM step.

    Each case also carries `model_calibrated_ms`: the same four terms with the ceilings
    this GPU reaches in place of the datasheet rates: the tensor term at the rate the
    4096^3 step's residue products reach (they run under the board's power limit), HBM
    terms at the measured read-only (streams of A) or copy rate (the deconstruction and
    the CRT, which read and write), each of those two terms the larger of its vector-issue
    and its memory time."""
    try:
        with open(TME_PATH) as fh:
            cal = json.load(fh)["kernels"]
    except (OSError, ValueError, KeyError):
        return None
    p_i8 = PEAK_INT8_TOPS * 1e12
    bw = PEAK_HBM_GBS * 1e9

    def k(key, field):
        return cal[key][field]

    cq = k("decon_rows_narrow_32768_r14", "vector_lane_ops_per_unit_per_modulus")
    r14 = 14
    out = {"c_q_residue_path_narrow": cq,
           "c_q_residue_path_wide": k("decon_rows_wide_4096_r16",
                                      "vector_lane_ops_per_unit_per_modulus"),
           "P_int_lane_ops_per_s": P_VALU, "P_fp64_flops": P_FP64,
           "oi_star_flop_per_byte_r14": round(cq * r14 * P_FP64 / (8 * P_VALU), 2),
           "fp64_ridge_flop_per_byte": round(P_FP64 / 8e12, 2),
           "max_lane_ops_per_element_for_memory_speed": {
               "at_8_TBs": round(8 * P_VALU / 8e12, 1),
               "at_measured_read_bw": round(8 * P_VALU / (hbm["hbm_read_gbs"] * 1e9), 1)},
           "digits_path_lane_ops_per_element": k("gemv_digits_32768_r14_1col",
                                                 "vector_lane_ops_per_unit")}
    n_a = 32768.0 * 32768.0
    rows = []
    sq = extras.get("square_4096")
    # measured ceilings (None where the run did not measure them)
    p_i8_cal = (16 * 2.0 * SQ ** 3 / (sq["step_r16_max"]["products_ms"] * 1e-3)
                if sq else None)
    bw_read = hbm.get("hbm_read_gbs", 0.0) * 1e9 or None
    bw_copy = hbm.get("hbm_copy_gbs", 0.0) * 1e9 or None
    g = extras.get("gemv_32768")
    if g:
        by = {run["nrhs"]: run for run in g["runs"]}

        def model(key, hbm_bytes, mfma_ops_per_inst):
            t_t = cal[key]["mfma_per_unit"] * n_a * mfma_ops_per_inst / p_i8
            t_h = hbm_bytes / bw
            t_d = cal[key]["vector_lane_ops_per_unit"] * n_a / P_VALU
            return t_t, t_h, t_d

        # int8 operations per MFMA instruction of each kernel: 16 x 16 x 64 (digits),
        # 16 x 16 x 32 (residues on the fly), 32 x 32 x 32 (stored planes), times 2
        cases = [("on the fly, digits, 1 col", "gemv_digits_32768_r14_1col", 8 * n_a,
                  by.get(1, {}).get("on_the_fly_cached_exps", {}).get("ms"), 32768.0),
                 ("on the fly, digits, 8 cols", "gemv_digits_32768_r14_8cols", 8 * n_a,
                  by.get(8, {}).get("on_the_fly_cached_exps", {}).get("ms"), 32768.0),
                 ("on the fly, residues, 32 cols", "gemv_fly_32768_r14_32cols", 8 * n_a,
                  by.get(32, {}).get("on_the_fly_cached_exps", {}).get("ms"), 16384.0),
                 ("stored planes, 1 col", "gemv_stored_32768_r14_1col", r14 * n_a,
                  by.get(1, {}).get("stored_planes", {}).get("ms"), 65536.0)]
        for name, key, hbm_bytes, measured, ops_inst in cases:
            t_t, t_h, t_d = model(key, hbm_bytes, ops_inst)
            row = {"case": f"GEMV 32768^2 r=14, {name}", "T_tensor_ms": round(t_t * 1e3, 3),
                   "T_hbm_ms": round(t_h * 1e3, 3), "T_decon_ms": round(t_d * 1e3, 3),
                   "model_ms": round((max(t_t, t_h) + t_d) * 1e3, 3),
                   "measured_ms": measured}
            if p_i8_cal and bw_read:
                t_tc = t_t * p_i8 / p_i8_cal
                t_hc = hbm_bytes / bw_read
                row["model_calibrated_ms"] = round((max(t_tc, t_hc) + t_d) * 1e3, 3)
            rows.append(row)
        for nrhs in (1, 8, 32):
            if nrhs in by:
                rows.append({"case": f"GEMV 32768^2 native fp64, {nrhs} col",
                             "T_hbm_ms": round(8 * n_a / bw * 1e3, 3),
                             "model_ms": round(8 * n_a / bw * 1e3, 3),
                             "measured_ms": by[nrhs]["native_fp64"]["ms"]})
    # DGEMM step: products on the matrix cores, deconstruction of A (rows) and B
    # (columns), CRT per output; HBM bytes are small next to the tensor term.
    if sq:
        t_t = 16 * 2.0 * SQ * SQ * SQ / p_i8
        t_d = (k("decon_rows_wide_4096_r16", "vector_lane_ops_per_unit") +
               k("decon_cols_wide_4096_r16", "vector_lane_ops_per_unit")) * SQ * SQ / P_VALU
        t_r = k("crt_4096_r16", "vector_lane_ops_per_unit") * SQ * SQ / P_VALU
        case = {"case": "DGEMM 4096^3 r=16 (max rule)", "T_tensor_ms": round(t_t * 1e3, 3),
                "T_decon_ms": round(t_d * 1e3, 3), "T_recon_ms": round(t_r * 1e3, 3),
                "model_ms": round((t_t + t_d + t_r) * 1e3, 3),
                "measured_ms": sq["step_r16_max"]["ms"],
                "measured_phases_ms": {
                    "products": sq["step_r16_max"]["products_ms"],
                    "deconstruct_rows": sq["deconstruct_rows"]["ms"],
                    "deconstruct_cols": sq["deconstruct_cols"]["ms"]}}
        if p_i8_cal and bw_copy:
            nn = float(SQ * SQ)
            # bytes: rows 8 + 16 per element; columns a maxima pass (8) + 8 + 16; CRT
            # 16 residues in, 8 out per output
            t_dc = max(t_d, (24 + 32) * nn / bw_copy)
            t_rc = max(t_r, 24 * nn / bw_copy)
            case["model_calibrated_ms"] = round((t_t * p_i8 / p_i8_cal + t_dc + t_rc) * 1e3, 3)
        rows.append(case)
    out["cases"] = rows
    return out


def measure_gemv(reps: int, stream) -> dict:
    """The 32768 x 32768 GEMV / low-batch GEMV workload at r = 14: A U(-1,1) (seed 4, drawn
    on the GPU), X U(-1,1) with 1, 8 and 32 columns.  GB/s counts the algorithmic bytes of
    A streamed per call (8 per element on the fly, r per element from stored planes)."""
    import numpy as np
    import torch

    import fp64_gemm_emulation_ozk_amd as ozk
    import ozk_inputs

    mg, kg, r = 32768, 32768, 14
    dev = torch.device("cuda:0")
    da = ozk_inputs.uniform_matrix_device((mg, kg), 4, dev)
    x_all = torch.from_numpy(ozk_inputs.uniform_matrix(np.random.default_rng(4), (kg, 32))).to(dev)
    elems = float(mg) * kg
    out = {"workload": f"A {mg}x{kg} U(-1,1), X {kg}x{{1,8,32}} U(-1,1), r={r}"}
    planes, exps = ozk.ozk_deconstruct(da, 0, r, k_budget=kg)
    dec = lambda: ozk.ozk_deconstruct(da, 0, r, k_budget=kg, planes=planes, exps=exps)
    dec()
    ms = _time_events(dec, reps, stream)
    out["deconstruct_A"] = {"ms": round(ms, 4), "gbs": round((8 + r) * elems / ms / 1e6, 1),
                            "bytes_per_elem": 8 + r}
    rows = []
    for nrhs in (1, 8, 32):
        dx = x_all[:, :nrhs].contiguous()
        y = torch.empty((mg, nrhs), dtype=torch.float64, device=dev)
        res = {"nrhs": nrhs}
        nat = lambda: torch.matmul(da, dx, out=y)
        nat()
        t = _time_events(nat, reps, stream)
        res["native_fp64"] = {"ms": round(t, 4), "gbs": round(8 * elems / t / 1e6, 1)}
        ws0 = torch.empty(ozk.ozk_dgemv_workspace_size(mg, kg, nrhs, r, 0), dtype=torch.uint8,
                          device=dev)
        fly = lambda: ozk.ozk_dgemv(da, dx, r, mode=0, a_exps=exps, out=y, workspace=ws0)
        fly()
        t = _time_events(fly, reps, stream)
        res["on_the_fly_cached_exps"] = {"ms": round(t, 4), "gbs": round(8 * elems / t / 1e6, 1),
                                         "frac_hbm": round(8 * elems / t / 1e6 / PEAK_HBM_GBS, 4)}
        fly2 = lambda: ozk.ozk_dgemv(da, dx, r, mode=0, out=y, workspace=ws0)
        fly2()
        t = _time_events(fly2, reps, stream)
        res["on_the_fly_with_exps_pass"] = {"ms": round(t, 4)}
        ws1 = torch.empty(ozk.ozk_dgemv_workspace_size(mg, kg, nrhs, r, 1), dtype=torch.uint8,
                          device=dev)
        st = lambda: ozk.ozk_dgemv(None, dx, r, mode=1, a_planes=planes, a_exps=exps, out=y,
                                   workspace=ws1)
        st()
        t = _time_events(st, reps, stream)
        res["stored_planes"] = {"ms": round(t, 4), "gbs": round(r * elems / t / 1e6, 1),
                                "frac_hbm": round(r * elems / t / 1e6 / PEAK_HBM_GBS, 4)}
        rows.append(res)
    out["runs"] = rows
    del da, planes
    torch.cuda.empty_cache()
    return out


def measure_wide_range(reps: int, stream, da, db) -> dict:
    """The wide-dynamic-range workload: 8192^3 with entries (U(0,1) - 0.5) exp(4 N(0,1))
    (seed 3), r = 16..20 under both scaling rules, next to native fp64 DGEMM.  rel is the
    normwise distance to the native product (its own rounding error is far below the
    emulation's at small r).  The GPU tests fix the accuracy against the exact product:
    1e-15 normwise needs r = 18 under the max rule and r = 16 under the norm rule."""
    import torch

    import fp64_gemm_emulation_ozk_amd as ozk

    n = da.shape[0]
    dev = da.device
    flops = 2.0 * n * n * n
    ref = torch.matmul(da, db)
    nat = lambda: torch.matmul(da, db, out=ref)
    t_nat = _time_events(nat, reps, stream)
    ref_n = torch.linalg.norm(ref)
    out = torch.empty_like(ref)
    ws = torch.empty(ozk.ozk_dgemm_workspace_size(n, n, n, 20), dtype=torch.uint8, device=dev)
    res = {"workload": f"DGEMM {n}^3, entries (U-0.5)*exp(4*N(0,1)), seed 3",
           "native_fp64": {"ms": round(t_nat, 4), "tflops": round(flops / t_nat / 1e9, 2)},
           "runs": []}
    for rr in range(16, 21):
        row = {"r": rr}
        for rule in ("max", "norm"):
            f = lambda: ozk.ozk_dgemm_ex(da, db, rr, rule, out=out, workspace=ws)
            f()
            t = _time_events(f, reps, stream)
            row[rule] = {"ms": round(t, 4), "tflops": round(flops / t / 1e9, 2),
                         "rel_vs_native": float(torch.linalg.norm(out - ref) / ref_n)}
        res["runs"].append(row)
    by_r = {row["r"]: row for row in res["runs"]}
    res["same_accuracy_1e-15"] = {
        "max_rule_r18_ms": by_r[18]["max"]["ms"], "norm_rule_r16_ms": by_r[16]["norm"]["ms"],
        "speedup": round(by_r[18]["max"]["ms"] / by_r[16]["norm"]["ms"], 3)}
    del ref, out, ws
    torch.cuda.empty_cache()
    return res


def measure_spmv(reps: int, stream) -> dict:
    """Emulated SpMV on the 7-point Poisson operator of a 256^3 grid (16.8 M rows, 117 M
    entries, x U(-1,1) seed 7) at r = 14 and 16, next to the vendor fp64 CSR product
    (torch.sparse.mm of the CSR tensor and x as one column).  GB/s counts the bytes a
    single pass over the operator needs (8 B value + 4 B column per entry, 4 B row offset
    and 8 B each of x and y per row), the same numerator for both."""
    import numpy as np
    import torch

    import fp64_gemm_emulation_ozk_amd as ozk
    import ozk_inputs

    n = 256
    dev = torch.device("cuda:0")
    rp, ci, v = ozk_inputs.poisson_7pt_csr(n)
    rows = n ** 3
    nnz = int(rp[-1])
    drp, dci, dv = (torch.from_numpy(t).to(dev) for t in (rp, ci, v))
    del rp, ci, v
    x = torch.from_numpy(ozk_inputs.uniform_matrix(np.random.default_rng(7), (rows, 1))[:, 0]
                         ).to(dev)
    y = torch.empty(rows, dtype=torch.float64, device=dev)
    algo = 12.0 * nnz + 20.0 * rows
    res = {"workload": f"7-point Poisson operator, {n}^3 grid ({rows} rows, {nnz} entries), "
                       "x U(-1,1)", "bytes_per_call": algo}
    try:
        a_csr = torch.sparse_csr_tensor(drp, dci, dv, size=(rows, rows))
        x2 = x[:, None].contiguous()
        # the vendor sparse library's CSR product (torch.mv on a CSR tensor takes a far
        # slower generic path on this build)
        nat = lambda: torch.sparse.mm(a_csr, x2)
        yn = nat()[:, 0]
        t = _time_events(nat, reps, stream)
        res["native_fp64"] = {"ms": round(t, 4), "gbs": round(algo / t / 1e6, 1),
                              "what": "torch.sparse.mm (vendor CSR SpMM, one column)"}
    except RuntimeError as exc:   # not every build ships the sparse path
        res["native_fp64"] = {"error": str(exc)[:200]}
        yn = None
    for r in (14, 16):
        ws = torch.empty(ozk.ozk_spmv_csr_workspace_size(rows, rows, r), dtype=torch.uint8,
                         device=dev)
        f = lambda: ozk.ozk_spmv_csr(drp, dci, dv, x, r, 7, out=y, workspace=ws)
        f()
        t = _time_events(f, reps, stream)
        ent = {"ms": round(t, 4), "gbs": round(algo / t / 1e6, 1),
               "frac_hbm": round(algo / t / 1e6 / PEAK_HBM_GBS, 4)}
        if yn is not None:
            ent["rel_vs_native"] = float(torch.linalg.norm(y - yn) / torch.linalg.norm(yn))
            if "ms" in res["native_fp64"]:
                ent["speed_vs_native"] = round(res["native_fp64"]["ms"] / t, 3)
        res[f"emulated_r{r}"] = ent
        del ws
    del drp, dci, dv, x, y
    torch.cuda.empty_cache()
    return res


def measure_fp4(reps: int, stream) -> dict:
    """The exact INT8 x INT8 product of 8192^3 int8 operands (uniform in [-128, 127],
    seed 5) through 9 FP4 GEMMs, against the 10.1 PFLOP/s dense FP4 MFMA peak."""
    import numpy as np
    import torch

    import fp64_gemm_emulation_ozk_amd as ozk
    import ozk_inputs

    n = 8192
    dev = torch.device("cuda:0")
    a, b = ozk_inputs.int8_operands(n, n, n, seed=5)
    ia, ib = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    c = torch.empty((n, n), dtype=torch.int32, device=dev)
    ws = torch.empty(ozk.ozk_int8gemm_fp4limb_workspace_size(n, n, n), dtype=torch.uint8,
                     device=dev)
    f = lambda: ozk.ozk_int8gemm_fp4limb(ia, ib, out=c, workspace=ws)
    f()
    t = _time_events(f, reps, stream)
    pa = ozk.ozk_fp4limb_pack(ia, 0)
    pb = ozk.ozk_fp4limb_pack(ib, 1)
    ldpb = pa.shape[-1]
    pack = lambda: (ozk.ozk_fp4limb_pack(ia, 0, planes=pa), ozk.ozk_fp4limb_pack(ib, 1, planes=pb))
    pack()
    tp = _time_events(pack, reps, stream)
    fp4_flops = 9 * 2.0 * n * n * (2 * ldpb)
    out = {"workload": f"int8 {n}x{n}x{n} uniform [-128,127], seed 5",
           "ms": round(t, 4), "pack_ms": round(tp, 4),
           "fp4_tflops_incl_pack": round(fp4_flops / t / 1e9, 1),
           "gemm_ms_excl_pack": round(t - tp, 4),
           "fp4_tflops_gemm": round(fp4_flops / (t - tp) / 1e9, 1),
           "frac_fp4_peak_gemm": round(fp4_flops / (t - tp) / 1e9 / PEAK_FP4_TFLOPS, 4),
           "int8_equiv_tops": round(2.0 * n ** 3 / t / 1e9, 1)}
    # the 6-product engine (weights 1, 29, 37; limb and pairwise-sum planes)
    ws6 = torch.empty(ozk.ozk_int8gemm_fp4awe_workspace_size(n, n, n), dtype=torch.uint8,
                      device=dev)
    f6 = lambda: ozk.ozk_int8gemm_fp4awe(ia, ib, out=c, workspace=ws6)
    f6()
    t6 = _time_events(f6, reps, stream)
    qa = ozk.ozk_fp4awe_pack(ia, 0)
    qb = ozk.ozk_fp4awe_pack(ib, 1)
    pack6 = lambda: (ozk.ozk_fp4awe_pack(ia, 0, planes=qa), ozk.ozk_fp4awe_pack(ib, 1, planes=qb))
    pack6()
    tp6 = _time_events(pack6, reps, stream)
    fl6 = 6 * 2.0 * n * n * n
    out["six_products"] = {
        "what": "6 FP4 plane products (weights 1, 29, 37; limb and pairwise-sum planes)",
        "ms": round(t6, 4), "pack_ms": round(tp6, 4), "gemm_ms_excl_pack": round(t6 - tp6, 4),
        "fp4_tflops_gemm": round(fl6 / (t6 - tp6) / 1e9, 1),
        "frac_fp4_peak_gemm": round(fl6 / (t6 - tp6) / 1e9 / PEAK_FP4_TFLOPS, 4),
        "int8_equiv_tops": round(2.0 * n ** 3 / t6 / 1e9, 1),
        "speedup_vs_nine": round(t / t6, 3)}
    # the 4-product INT4 x INT8 engine (limb weight 5) on int4 A (uniform in [-8, 7])
    a4, b4 = ozk_inputs.int4_int8_operands(n, n, n, seed=5)
    ja, jb = torch.from_numpy(a4).to(dev), torch.from_numpy(b4).to(dev)
    del a4, b4
    ws4 = torch.empty(ozk.ozk_int4int8gemm_fp4awe_workspace_size(n, n, n), dtype=torch.uint8,
                      device=dev)
    f4 = lambda: ozk.ozk_int4int8gemm_fp4awe(ja, jb, out=c, workspace=ws4)
    f4()
    t4 = _time_events(f4, reps, stream)
    ra = ozk.ozk_fp4awe4_pack(ja, 0, True)
    rb = ozk.ozk_fp4awe4_pack(jb, 1, False)
    pack4 = lambda: (ozk.ozk_fp4awe4_pack(ja, 0, True, planes=ra),
                     ozk.ozk_fp4awe4_pack(jb, 1, False, planes=rb))
    pack4()
    tp4 = _time_events(pack4, reps, stream)
    f6i4 = lambda: ozk.ozk_int8gemm_fp4awe(ja, jb, out=c, workspace=ws6)
    t6i4 = _time_events(f6i4, reps, stream)
    fl4 = 4 * 2.0 * n * n * n
    out["int4_x_int8_four_products"] = {
        "what": ("int4 A uniform in [-8, 7] x int8 B, seed 5: 4 FP4 plane products (limb "
                 "weight 5, points 0, inf, 1, 1/2)"),
        "ms": round(t4, 4), "pack_ms": round(tp4, 4), "gemm_ms_excl_pack": round(t4 - tp4, 4),
        "fp4_tflops_gemm": round(fl4 / (t4 - tp4) / 1e9, 1),
        "frac_fp4_peak_gemm": round(fl4 / (t4 - tp4) / 1e9 / PEAK_FP4_TFLOPS, 4),
        "int8_equiv_tops": round(2.0 * n ** 3 / t4 / 1e9, 1),
        "six_product_engine_same_operands_ms": round(t6i4, 4),
        "speedup_vs_six": round(t6i4 / t4, 3)}
    del ja, jb, ws4, ra, rb
    try:
        torch._int_mm(ia, ib)
        ti = _time_events(lambda: torch._int_mm(ia, ib), reps, stream)
        out["vendor_int8_gemm"] = {"ms": round(ti, 4), "tops": round(2.0 * n ** 3 / ti / 1e9, 1)}
    except RuntimeError as exc:
        out["vendor_int8_gemm"] = {"error": str(exc)[:200]}
    del ia, ib, c, ws, pa, pb, ws6, qa, qb
    torch.cuda.empty_cache()
    return out


def measure_hbm_rates(stream) -> dict:
    """What plain streaming reaches on this GPU, as context for the HBM rooflines: a device
    copy of 2 GiB (torch, read + write bytes), a read-only reduction of 2 GiB (torch sum,
    read bytes) and a write-only fill of 2 GiB."""
    import torch

    dev = torch.device("cuda:0")
    out = {}
    src = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    t = _time_events(lambda: dst.copy_(src), 5, stream)
    out["hbm_copy_gbs"] = round(2.0 * src.numel() / t / 1e6, 1)
    del dst
    x = src.view(torch.float64)
    acc = torch.empty((), dtype=torch.float64, device=dev)
    torch.sum(x, dim=0, out=acc)
    t = _time_events(lambda: torch.sum(x, dim=0, out=acc), 5, stream)
    out["hbm_read_gbs"] = round(src.numel() / t / 1e6, 1)
    t = _time_events(lambda: src.fill_(7), 5, stream)
    out["hbm_write_gbs"] = round(src.numel() / t / 1e6, 1)
    del src, x
    torch.cuda.empty_cache()
    out["what"] = ("a 2 GiB device copy, a 2 GiB read-only reduction and a 2 GiB fill "
                   "(write only), torch")
    return out


def measure_square_4096(reps: int, stream) -> dict:
    """The square workload: 4096^3 with entries (U(0,1) - 0.5) exp(0.5 N(0,1)) (seed 2).
    The step at r = 16 (max rule) with its residue products timed inside it, native fp64
    DGEMM and the vendor int8 GEMM on the same sizes, the r sweep 12..18 under both
    scaling rules (time and normwise distance to the native product), and each
    operand's deconstruction alone in HBM GB/s (algorithmic bytes: 8 B read + r B
    written per element, + 8 B for the column maxima pass of B)."""
    import torch

    import fp64_gemm_emulation_ozk_amd as ozk
    import ozk_inputs

    n = SQ
    dev = torch.device("cuda:0")
    a, b = ozk_inputs.gemm_operands(n, n, n, seed=SQ_SEED, dist="phi", phi=SQ_PHI)
    da, db = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    del a, b
    flops = 2.0 * n * n * n
    out = torch.empty((n, n), dtype=torch.float64, device=dev)
    ws = torch.empty(ozk.ozk_dgemm_workspace_size(n, n, n, 18), dtype=torch.uint8, device=dev)
    res = {"workload": f"DGEMM {n}^3, entries (U-0.5)*exp({SQ_PHI}*N(0,1)), seed {SQ_SEED}"}
    for _ in range(20):
        ozk.ozk_dgemm(da, db, 16, out=out, workspace=ws)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        e1.record(stream)
    it = iter(ev)

    def timed():
        e0, e1 = next(it)
        ozk.ozk_dgemm_ex_timed(da, db, 16, e0, e1, "max", out=out, workspace=ws)

    t = _time_events(timed, reps, stream, warm_fn=lambda: ozk.ozk_dgemm_ex(
        da, db, 16, "max", out=out, workspace=ws))
    prod_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / reps
    ops = 16 * 2.0 * n * n * n
    res["step_r16_max"] = {"ms": round(t, 4), "tflops": round(flops / t / 1e9, 2),
                           "products_ms": round(prod_ms, 4),
                           "products_frac_int8_peak": round(ops / prod_ms / 1e9 /
                                                            PEAK_INT8_TOPS, 4)}
    ref = torch.matmul(da, db)
    t = _time_events(lambda: torch.matmul(da, db, out=ref), reps, stream)
    res["native_fp64"] = {"ms": round(t, 4), "tflops": round(flops / t / 1e9, 2)}
    try:
        ia = torch.randint(-128, 128, (n, n), dtype=torch.int8, device=dev)
        ib = torch.randint(-128, 128, (n, n), dtype=torch.int8, device=dev)
        torch._int_mm(ia, ib)
        t = _time_events(lambda: torch._int_mm(ia, ib), reps, stream)
        res["vendor_int8_gemm"] = {"what": "torch._int_mm on one 4096^3 int8 product",
                                   "ms": round(t, 4), "tops": round(flops / t / 1e9, 1),
                                   "ours_per_modulus_ms": round(prod_ms / 16, 4)}
        del ia, ib
    except RuntimeError as exc:  # not every build ships the int8 path
        res["vendor_int8_gemm"] = {"error": str(exc)[:200]}
    ref_n = torch.linalg.norm(ref)
    sweep = []
    for rr in range(12, 19):
        row = {"r": rr}
        for rule in ("max", "norm"):
            f = lambda: ozk.ozk_dgemm_ex(da, db, rr, rule, out=out, workspace=ws)
            f()
            t = _time_events(f, reps, stream)
            row[rule] = {"ms": round(t, 4), "tflops": round(flops / t / 1e9, 2),
                         "rel_vs_native": float(torch.linalg.norm(out - ref) / ref_n)}
        sweep.append(row)
    res["r_sweep"] = sweep
    del ws, out, ref
    r = 16
    planes_a, exps_a = ozk.ozk_deconstruct(da, 0, r)
    planes_b, exps_b = ozk.ozk_deconstruct(db, 1, r, k_budget=n)
    dec = lambda: ozk.ozk_deconstruct(da, 0, r, planes=planes_a, exps=exps_a)
    dec()
    t = _time_events(dec, reps, stream)
    res["deconstruct_rows"] = {"ms": round(t, 4), "bytes": (8 + r) * n * n,
                               "gbs": round((8 + r) * n * n / t / 1e6, 1),
                               "frac_hbm": round((8 + r) * n * n / t / 1e6 / PEAK_HBM_GBS, 4)}
    decb = lambda: ozk.ozk_deconstruct(db, 1, r, k_budget=n, planes=planes_b, exps=exps_b)
    decb()
    t = _time_events(decb, reps, stream)
    res["deconstruct_cols"] = {"ms": round(t, 4), "bytes": (16 + r) * n * n,
                               "gbs": round((16 + r) * n * n / t / 1e6, 1),
                               "note": "column maxima pass (8 B per element) + residues "
                                       "(8 + r B per element)"}
    del da, db, planes_a, planes_b
    torch.cuda.empty_cache()
    return res


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(a, b, r: int, rule: str) -> dict:
    """The oracle, as it stands, on a sampled block of the timed workload: rows 0, 32, 64,
    ... of C (256 rows) by columns 0, 8, 16, ... (1024 columns), 262144 outputs, each phase
    timed.  Exponents come from the full rows of A and columns of B, so the block equals
    the same block of the whole product.  The modular products run in float64 BLAS on all
    of its threads; the other phases are numpy and Python integers on one thread."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import ozaki2

    k = a.shape[1]
    rows = np.arange(0, a.shape[0], 32)
    cols = np.arange(0, b.shape[1], 8)
    phases = {}
    t0 = time.perf_counter()
    ar, bc = a[rows], b[:, cols]
    e = ozaki2.exponents(ar, r, k, 0, "a", rule)
    f = ozaki2.exponents(bc, r, k, 1, "b", rule)
    t1 = time.perf_counter()
    pla = ozaki2.residue_planes(ar, e, r, 0)
    plb = ozaki2.residue_planes(bc, f, r, 1)
    t2 = time.perf_counter()
    prods = ozaki2.modular_products(pla, plb)
    t3 = time.perf_counter()
    ozaki2.reconstruct(prods, r, e, f)
    t4 = time.perf_counter()
    phases = {"scaling_s": round(t1 - t0, 3), "residues_s": round(t2 - t1, 3),
              "modular_products_s": round(t3 - t2, 3), "crt_s": round(t4 - t3, 3)}
    dt = t4 - t0
    flops = 2.0 * len(rows) * len(cols) * k
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max(blas) if blas else 1
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 3), "phases": phases, "cpu_model": _cpu_model(),
            "host_logical_cpus": os.cpu_count(),
            "sample": f"{len(rows)} x {len(cols)} block of C (every 32nd row, every 8th "
                      f"column) of the {M}x{N}x{K} workload, r={r}, {rule} scaling; rate = "
                      f"2 * outputs * k / time, i.e. the whole product's rate at this "
                      f"per-output cost; numpy, modular products on {threads} BLAS threads, "
                      f"other phases on one thread"}


def _percentiles(ms: list) -> dict:
    """Median, 10th and 90th percentile of a list of times (ms), and their count."""
    import numpy as np

    v = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(v)), 4), "p10": round(float(np.percentile(v, 10)), 4),
            "p90": round(float(np.percentile(v, 90)), 4), "n": int(v.size)}


def hold(seconds: float, what: str, step, da, db, r: int, rule: str) -> int:
    """Run one workload back to back for `seconds` (for external power and clock readings)
    and print the mean time per call."""
    import numpy as np
    import torch

    import fp64_gemm_emulation_ozk_amd as ozk
    import ozk_inputs

    dev = da.device
    if what == "dgemm":
        call, name = step, f"DGEMM step {M}^3 r={r} {rule} rule"
    elif what == "products":
        pa = ozk.ozk_deconstruct_ex(da, 0, r, scaling=rule)[0]
        pb = ozk.ozk_deconstruct_ex(db, 1, r, scaling=rule)[0]
        res = ozk.ozk_modular_residues(pa, pb, r)
        call = lambda: ozk.ozk_modular_residues(pa, pb, r, out=res)
        name = f"residue products {M}^3 r={r}"
    elif what in ("fp4limb", "fp4awe4"):
        del da, db
        torch.cuda.empty_cache()
        gen = ozk_inputs.int8_operands if what == "fp4limb" else ozk_inputs.int4_int8_operands
        ia, ib = (torch.from_numpy(t).to(dev) for t in gen(M, M, M, seed=5))
        out = torch.empty((M, M), dtype=torch.int32, device=dev)
        if what == "fp4limb":
            ws = torch.empty(ozk.ozk_int8gemm_fp4limb_workspace_size(M, M, M), dtype=torch.uint8,
                             device=dev)
            call = lambda: ozk.ozk_int8gemm_fp4limb(ia, ib, out=out, workspace=ws)
            name = f"INT8 {M}^3 through 9 FP4 products"
        else:
            ws = torch.empty(ozk.ozk_int4int8gemm_fp4awe_workspace_size(M, M, M),
                             dtype=torch.uint8, device=dev)
            call = lambda: ozk.ozk_int4int8gemm_fp4awe(ia, ib, out=out, workspace=ws)
            name = f"INT4 x INT8 {M}^3 through 4 FP4 products"
    else:
        del da, db
        torch.cuda.empty_cache()
        nrhs, mg, rg = int(what[4:]), 32768, 14
        ga = ozk_inputs.uniform_matrix_device((mg, mg), 4, dev)
        x = torch.from_numpy(ozk_inputs.uniform_matrix(np.random.default_rng(4), (mg, 32)))
        x = x.to(dev)[:, :nrhs].contiguous()
        planes, exps = ozk.ozk_deconstruct(ga, 0, rg, k_budget=mg)[:2]
        del planes
        torch.cuda.empty_cache()
        ws = torch.empty(ozk.ozk_dgemv_workspace_size(mg, mg, nrhs, rg, 0), dtype=torch.uint8,
                         device=dev)
        y = torch.empty((mg, nrhs), dtype=torch.float64, device=dev)
        call = lambda: ozk.ozk_dgemv(ga, x, rg, mode=0, a_exps=exps, out=y, workspace=ws)
        name = f"GEMV {mg}^2 r={rg} on the fly, {nrhs} columns"
    call()
    torch.cuda.synchronize()
    print(f"hold start: {name}", flush=True)
    t0, done = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(25):
            call()
        torch.cuda.synchronize()
        done += 25
    dt = time.perf_counter() - t0
    print(f"hold done: {done} calls, {dt / done * 1e3:.3f} ms each", flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # Untimed warm-up: after an idle spell the board needs some 50-65 ms of this load before
    # its clocks settle, so the default covers that.
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--r", type=int, default=DEFAULT_R)
    ap.add_argument("--scaling", choices=("max", "norm"), default=DEFAULT_SCALING,
                    help="scaling rule of the timed step (norm: per-line 2-norm, the "
                         "headline; max: per-line maximum, needs r = 18 for 1e-15 here)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-gemv", action="store_true")
    ap.add_argument("--no-fp4", action="store_true")
    ap.add_argument("--no-wide", action="store_true",
                    help="skip the wide-range r = 16..20 sweep under both rules")
    ap.add_argument("--no-spmv", action="store_true",
                    help="skip the emulated SpMV (Poisson 256^3) extra")
    ap.add_argument("--no-square", action="store_true",
                    help="skip the 4096^3 square workload extra")
    ap.add_argument("--counters", nargs="?", const="dgemm", choices=("dgemm", "all"),
                    help="only launch the kernels the counter passes profile (all: also the "
                         "GEMV, FP4-limb and SpMV engines)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("DIR", "OUT_JSON"),
                    help="per-kernel means of every counter of a rocprofv3 --pmc csv run")
    ap.add_argument("--traffic-summary", nargs="+", metavar="DIR",
                    help="FETCH_DIR WRITE_DIR [OUT_JSON]: write the HBM traffic summary from "
                         "two rocprofv3 --pmc csv runs")
    ap.add_argument("--tme-counters", action="store_true",
                    help="only launch the kernels the time-model counter pass profiles")
    ap.add_argument("--hold", type=float, metavar="SECONDS",
                    help="run one workload back to back for SECONDS and print its mean time "
                         "(a steady load for reading the board's power and clocks with amd-smi)")
    ap.add_argument("--hold-workload", default="dgemm",
                    choices=("dgemm", "products", "gemv1", "gemv8", "gemv32", "fp4limb",
                             "fp4awe4"),
                    help="what --hold runs: the timed step, its residue products alone, the "
                         "32768^2 GEMV on the fly (r = 14, cached exponents) with 1/8/32 columns, "
                         "or the 8192^3 INT8 (9 FP4 products) or INT4 x INT8 (4) product")
    ap.add_argument("--tme-summary", metavar="DIR",
                    help="write the time-model instruction counts from a rocprofv3 --pmc run")
    args = ap.parse_args()
    if args.traffic_summary:
        if len(args.traffic_summary) not in (2, 3):
            ap.error("--traffic-summary takes FETCH_DIR WRITE_DIR [OUT_JSON]")
        return traffic_summary(*args.traffic_summary)
    if args.tme_summary:
        return tme_summary(args.tme_summary)
    if args.pmc_summary:
        return pmc_summary(*args.pmc_summary)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the emulation "
              "path is built and measured on a single MI355X; multi-GPU runs are not "
              "supported.", file=sys.stderr)
        return 2

    import torch

    import fp64_gemm_emulation_ozk_amd as ozk
    import ozk_inputs

    if not os.path.exists(ozk.LIB_PATH):
        from fp64_gemm_emulation_ozk_amd.build import build_library
        build_library()
    if args.counters:
        return run_counter_workload(extra=args.counters == "all")
    if args.tme_counters:
        return run_tme_workload()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    r = args.r
    rule = args.scaling

    a, b = ozk_inputs.gemm_operands(M, N, K, seed=SEED, dist="phi", phi=PHI)
    da = torch.from_numpy(a).to(dev)
    db = torch.from_numpy(b).to(dev)
    out = torch.empty((M, N), dtype=torch.float64, device=dev)
    ws = torch.empty(ozk.ozk_dgemm_workspace_size(M, N, K, r), dtype=torch.uint8, device=dev)
    step = lambda: ozk.ozk_dgemm_ex(da, db, r, rule, out=out, workspace=ws)

    if args.hold:
        return hold(args.hold, args.hold_workload, step, da, db, r, rule)

    for _ in range(args.warmup):
        step()
    # The timed steps record one HIP event pair around the residue products of each step
    # (ozk_dgemm_ex_timed), so the dominant kernel is timed inside the timed region.
    gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for ga, gb in gev:          # create the events before the timed region
        ga.record(stream)
        gb.record(stream)
    counter = iter(range(args.steps))

    def timed_step():
        i = next(counter)
        ozk.ozk_dgemm_ex_timed(da, db, r, gev[i][0], gev[i][1], rule, out=out, workspace=ws)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_events = _time_events(timed_step, args.steps, stream, warm_ms=0)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_per_step = max(ms_events, 1e-9)
    value = 2.0 * M * N * K / (ms_per_step * 1e-3) / 1e12
    gemm_ms = sum(ga.elapsed_time(gb) for ga, gb in gev) / args.steps
    # the same steps without the two event records, for comparison
    plain_ms = _time_events(step, args.steps, stream)
    # distribution of single steps (one event pair each, after the timed region) and of
    # the residue-product launches inside the timed steps
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for ea, eb in sev:
        ea.record(stream)
        step()
        eb.record(stream)
    torch.cuda.synchronize()
    step_dist = _percentiles([ea.elapsed_time(eb) for ea, eb in sev])
    gemm_dist = _percentiles([ga.elapsed_time(gb) for ga, gb in gev])

    # Sanity: normwise distance to native fp64 (not a parity check; tests do that).
    ref = torch.matmul(da, db)
    rel = float(torch.linalg.norm(out - ref) / torch.linalg.norm(ref))
    kp = ozk.ozk_planes_ld(K)
    kp = (kp + 127) // 128 * 128          # the step pads K to whole 128-byte rows
    ops = r * 2.0 * M * N * kp
    achieved = ops / (gemm_ms * 1e-3) / 1e12
    digest = _source_digest(["gemm_i8.hip"])
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_INT8_TOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_INT8_TOPS, 4),
                "traffic": _traffic("gemm_i8_residues", digest),
                "kernel": "gemm_i8_pairs_kernel<residues> (v_mfma_i32_16x16x64_i8)",
                "kernel_ms": round(gemm_ms, 4), "ops_per_launch": ops,
                "ops_unit": "int8 multiply-adds x 2 (TOP/s reported in the TFLOP/s slot)",
                "timed": "inside the timed steps, one HIP event pair per launch",
                "source_digest": digest}

    extras = {"wall_ms_per_step": round(wall_ms, 4), "normwise_vs_native_fp64": rel,
              "ms_per_step_without_gemm_events": round(plain_ms, 4),
              "emulated_pct_int8_peak": round(r * value / PEAK_INT8_TOPS * 100, 2),
              "products_ms": round(gemm_ms, 4),
              "step_phases": "column scaling of B, paired deconstruction of A and B, "
                             "residue products, CRT",
              "step_ms_distribution": step_dist, "products_ms_distribution": gemm_dist}
    reps = max(args.steps // 2, 5)
    nat_ms = _time_events(lambda: torch.matmul(da, db, out=ref), reps, stream)
    extras["native_fp64_dgemm"] = {"ms": round(nat_ms, 4),
                                   "tflops": round(2.0 * M * N * K / nat_ms / 1e9, 2),
                                   "emulated_speedup": round(nat_ms / ms_per_step, 3)}
    del ref
    if not args.no_extras:
        planes_a, exps_a = ozk.ozk_deconstruct_ex(da, 0, r, rule)
        planes_b, exps_b = ozk.ozk_deconstruct_ex(db, 1, r, rule, k_budget=K)
        dec = lambda: ozk.ozk_deconstruct_ex(da, 0, r, rule, planes=planes_a, exps=exps_a)
        dec()
        dec_ms = _time_events(dec, reps, stream)
        extras["deconstruct_rows"] = {
            "ms": round(dec_ms, 4), "bytes": (8 + r) * M * K,
            "gbs": round((8 + r) * M * K / dec_ms / 1e6, 1),
            "frac_hbm": round((8 + r) * M * K / dec_ms / 1e6 / PEAK_HBM_GBS, 4)}
        decb = lambda: ozk.ozk_deconstruct_ex(db, 1, r, rule, k_budget=K, planes=planes_b,
                                              exps=exps_b)
        decb()
        decb_ms = _time_events(decb, reps, stream)
        extras["deconstruct_cols"] = {
            "ms": round(decb_ms, 4), "bytes": (8 + 8 + r) * K * N,
            "gbs": round((8 + 8 + r) * K * N / decb_ms / 1e6, 1),
            "note": "norm (or maxima) pass over B (8 B per element) + residues "
                    "(8 + r B per element)"}
        del planes_a, planes_b, ws, out
        torch.cuda.empty_cache()
        hbm = measure_hbm_rates(stream)
        extras["hbm_rates"] = hbm
        if not args.no_wide:
            extras["wide_range_8192"] = measure_wide_range(reps, stream, da, db)
        if not args.no_square:
            extras["square_4096"] = measure_square_4096(reps, stream)
        if not args.no_gemv:
            extras["gemv_32768"] = measure_gemv(reps, stream)
        if not args.no_fp4:
            extras["fp4limb_int8gemm_8192"] = measure_fp4(reps, stream)
        if not args.no_spmv:
            extras["spmv_poisson_256"] = measure_spmv(reps, stream)
        model = tme_model(extras, hbm)
        if model is not None:
            extras["tme_model"] = model

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": f"emulated DGEMM {M}x{N}x{K}, entries (U-0.5)*exp({PHI}*N(0,1)), "
                               f"seed {SEED}, r={r} moduli, {rule} row/column scaling",
                   "m": M, "n": N, "k": K, "r": r, "scaling": rule,
                   "compute": "int8 MFMA + fp64 VALU"},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(a, b, r, rule)
    line["extras"] = extras
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
