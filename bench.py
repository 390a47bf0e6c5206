"""Benchmark of the fine-grained FP8 hot path on one MI355X.

One step = the whole path on the 4096^3 workload, inputs resident in HBM:
  1. 1x128 E4M3 quantization of the bf16 activation A [4096,4096]   (fgq_quantize_act_1x128)
  2. 128x128 E4M3 quantization of the bf16 weight B [4096,4096]      (fgq_quantize_weight_128x128)
  3. block-scaled FP8 GEMM C = A_q (x) B_q, bf16 C [4096,4096]       (fgq_gemm_fp8_blockscaled)
value = 2*M*N*K / step time (TFLOP/s of the whole step).  The dominant kernel is the GEMM:
its roofline entry divides its algorithmic flops by its own average duration (HIP events on
the stream it runs on) and compares with the dense FP8 MFMA peak.  The standalone
activation quantizer is measured on X [16384,7168] (rotating buffers so the 256 MB
Infinity Cache cannot serve the input) against the HBM peak.  The CPU oracle is timed on the
same 4096^3 workload (a few seconds on the host's threads; cpu_baseline), and the GPU step's
outputs are compared with its result there.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA (no sparsity)
PEAK_F16_TFLOPS = 2500.0     # MI355X dense FP16 MFMA (the instruction the GEMM issues)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
METRIC = "block-scaled FP8 GEMM TFLOP/s (% FP8 MFMA peak); quantize GB/s (% HBM)"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {   # the sources each profiled kernel is built from (for staleness checks)
    "gemm": ["fine_grained_block_fgq_amd/csrc/gemm.hip",
             "fine_grained_block_fgq_amd/csrc/gemm_common.hpp",
             "fine_grained_block_fgq_amd/csrc/fgq_device.hpp"],
    "quant_act": ["fine_grained_block_fgq_amd/csrc/quant.hip",
                  "fine_grained_block_fgq_amd/csrc/fgq_device.hpp"],
}


def source_hash(kind):
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(key, kind):
    """HBM bytes per launch from the committed counter summary, or None when the kernel's
    source changed since the counters were taken."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(key)
    if not rec or rec.get("source_sha256") != source_hash(kind):
        return None
    return rec["bytes_per_launch"]


def summarize(ktrace_dir, fetch_dir, write_dir, mfma_dir=None):
    """Write the profile summaries under profiles/ from rocprofv3 csv output directories:
    a --kernel-trace --stats run of bench.py, and --pmc FETCH_SIZE / --pmc WRITE_SIZE runs of
    `bench.py --mode profile` (which includes a 512 MiB copy used to calibrate both counters),
    and optionally a --pmc SQ_INSTS_MFMA run of the same (MFMA instruction count per GEMM
    against 2*M*N*K / 16384 flop per 16x16x32 instruction)."""
    import csv
    import glob

    def rows(d, suffix):
        f = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
        if not f:
            raise SystemExit(f"no *{suffix} under {d}")
        with open(f[0]) as fh:
            return list(csv.DictReader(fh))

    def short(name):
        for k in ("gemm_fp8_blockscaled_narrow_kernel", "gemm_fp8_blockscaled_ksplit_kernel",
                  "splitk_reduce_kernel", "gemm_fp8_blockscaled_kernel",
                  "gemm_nvfp4_kernel", "nvfp4_quant_kernel", "nvfp4_amax_kernel",
                  "quant_act_1x128_kernel", "quant_weight_128x128_kernel",
                  "vectorized_elementwise_kernel"):
            if k in name:
                tags = ""
                if "ScaleIn<true>" in name or "ScaleUE8M0" in name:
                    tags += "+ue8m0"
                if k == "gemm_fp8_blockscaled_kernel" and ", true, true>" in name:
                    tags += "+fused"
                return k + tags
        return name[:60]

    os.makedirs(PROFILES, exist_ok=True)
    # kernel durations
    trace = rows(ktrace_dir, "kernel_trace.csv")
    groups = {}
    for r in trace:
        key = (short(r["Kernel_Name"]), int(r["Grid_Size_X"] if "Grid_Size_X" in r else r.get("Grid_Size", 0)))
        groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = [f"{'kernel':40s} {'grid':>9s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for (name, grid), d in sorted(groups.items()):
        lines.append(f"{name:40s} {grid:9d} {len(d):6d} {sum(d)/len(d)/1e3:9.2f} {min(d)/1e3:9.2f} {max(d)/1e3:9.2f}")
    stats = "\n".join(lines)
    # counters
    def counter(d, cname):
        acc = {}
        for r in rows(d, "counter_collection.csv"):
            if r["Counter_Name"] != cname:
                continue
            acc.setdefault((short(r["Kernel_Name"]), int(r["Grid_Size"])), []).append(float(r["Counter_Value"]))
        return acc
    fetch_l, write_l = counter(fetch_dir, "FETCH_SIZE"), counter(write_dir, "WRITE_SIZE")
    # the 512 MiB elementwise dispatches are the fill of the copy's source (writes only)
    # followed by the copies (read + write 512 MiB each): calibrate on the copies
    fk = ("vectorized_elementwise_kernel", 33554432)
    copy_fetch = sorted(fetch_l[fk])[1:]          # drop the fill
    copy_write = sorted(write_l[fk])
    fetch = {k: sum(v) / len(v) for k, v in fetch_l.items()}
    write = {k: sum(v) / len(v) for k, v in write_l.items()}
    fetch[fk] = sum(copy_fetch) / len(copy_fetch)
    write[fk] = copy_write[len(copy_write) // 2]
    copy_bytes = 512 * 2**20
    fetch_scale = copy_bytes / (fetch[fk] * 1024)
    write_scale = copy_bytes / (write[fk] * 1024)
    traffic = {}
    out = ["rocprofv3 byte counters per dispatch (KiB), scaled by the 512 MiB copy calibration",
           f"calibration: copy FETCH_SIZE {fetch[fk]:.1f} KiB -> x{fetch_scale:.3f}; "
           f"WRITE_SIZE {write[fk]:.1f} KiB -> x{write_scale:.3f}",
           f"{'kernel':40s} {'grid':>9s} {'FETCH_KiB':>12s} {'WRITE_KiB':>12s} {'HBM_MB(scaled)':>15s}"]
    for k in sorted(fetch):
        if k not in write:
            continue
        b = fetch[k] * 1024 * fetch_scale + write[k] * 1024 * write_scale
        out.append(f"{k[0]:40s} {k[1]:9d} {fetch[k]:12.1f} {write[k]:12.1f} {b/1e6:15.2f}")
        if k == ("gemm_fp8_blockscaled_kernel", 262144):
            traffic["gemm_fp8_blockscaled 4096^3 bf16"] = {"source_sha256": source_hash("gemm"),
                                                          "bytes_per_launch": b}
        qa = [kk for kk in fetch if kk[0] == "quant_act_1x128_kernel"]
        if qa and k == max(qa, key=lambda kk: kk[1]):   # the [16384,7168] launch
            traffic["quant_act_1x128 16384x7168"] = {"source_sha256": source_hash("quant_act"),
                                                     "bytes_per_launch": b}
    with open(os.path.join(PROFILES, "kernel_stats_bench_step.txt"), "w") as f:
        f.write("command: cd /tmp && export TMPDIR=/tmp; rocprofv3 --kernel-trace --stats -f csv "
                "-d <dir> -o run -- python3 bench.py --gpus 1 --steps 20 --warmup 5\n"
                "summary: python3 bench.py --summarize <ktrace dir> <fetch dir> <write dir>\n\n")
        f.write(stats + "\n")
        g = groups.get(("gemm_fp8_blockscaled_kernel", 262144))
        if g:
            avg = sum(g) / len(g) / 1e3
            tf = 2.0 * 4096 ** 3 / (avg * 1e-6) / 1e12
            f.write(f"\n4096^3 bf16 GEMM (grid 262144): {len(g)} launches, average {avg:.2f} us = "
                    f"{tf:.1f} TFLOP/s = {tf / PEAK_FP8_TFLOPS:.4f} of the {PEAK_FP8_TFLOPS:.0f} "
                    f"TFLOP/s dense FP8 peak ({tf / PEAK_F16_TFLOPS:.4f} of the f16 peak)\n")
    with open(os.path.join(PROFILES, "hbm_traffic_counters.txt"), "w") as f:
        f.write("commands: rocprofv3 --pmc FETCH_SIZE -f csv -d <dir> -o run -- python3 bench.py "
                "--mode profile ; rocprofv3 --pmc WRITE_SIZE -f csv -d <dir> -o run -- python3 "
                "bench.py --mode profile\n\n")
        f.write("\n".join(out) + "\n")
    with open(os.path.join(PROFILES, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    if mfma_dir:
        mf = counter(mfma_dir, "SQ_INSTS_MFMA")
        mlines = ["rocprofv3 --pmc SQ_INSTS_MFMA per dispatch (median over dispatches); a 16x16x32 "
                  "f16 MFMA is 16384 flop, so the GEMM's count x 16384 should equal 2*M*N*K",
                  f"{'kernel':40s} {'grid':>9s} {'SQ_INSTS_MFMA':>14s} {'x16384 flop':>14s}"]
        for k in sorted(mf):
            v = sorted(mf[k])[len(mf[k]) // 2]
            mlines.append(f"{k[0]:40s} {k[1]:9d} {v:14.0f} {v * 16384:14.4g}")
        mlines.append(f"2*4096^3 = {2 * 4096**3:.4g} flop")
        with open(os.path.join(PROFILES, "mfma_count_counters.txt"), "w") as f:
            f.write("command: rocprofv3 --pmc SQ_INSTS_MFMA -f csv -d <dir> -o run -- python3 "
                    "bench.py --mode profile\n\n")
            f.write("\n".join(mlines) + "\n")
        print("\n".join(mlines))
    print(stats)
    print("\n".join(out))


# two rocprofv3 --pmc passes over `bench.py --mode profile` (8 SQ counters and one GRBM
# counter each, the most one pass collects)
SQ_PASSES = [
    "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU "
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_VALU GRBM_GUI_ACTIVE",
    "SQ_INSTS_MFMA SQ_INSTS_VALU_CVT SQ_INSTS_LDS SQ_INSTS_SALU SQ_ACTIVE_INST_LDS "
    "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_ACTIVE_INST_ANY GRBM_GUI_ACTIVE",
]


def summarize_sq(dirs):
    """Instruction mix and unit activity of the 4096^3 GEMM dispatch from the SQ counter passes
    (medians over its dispatches): MFMA busy as a fraction of the 1024 SIMDs' cycles
    (GRBM_GUI_ACTIVE counts each of the 8 XCDs), instructions per MFMA, and wait / LDS rates."""
    import csv
    import glob
    vals = {}
    for d in dirs:
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not f:
            raise SystemExit(f"no counter_collection.csv under {d}")
        with open(f[0]) as fh:
            for r in csv.DictReader(fh):
                if "gemm_fp8_blockscaled_kernel" in r["Kernel_Name"] and \
                        int(r["Grid_Size"]) == 262144 and "ScaleInILb1" not in r["Kernel_Name"]:
                    vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    m = {k: sorted(v)[len(v) // 2] for k, v in vals.items()}
    need = ["GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU"]
    if any(k not in m for k in need):
        raise SystemExit(f"missing counters: {[k for k in need if k not in m]}")
    xcd_cycles = m["GRBM_GUI_ACTIVE"] / 8
    mf = m["SQ_INSTS_MFMA"]
    lines = ["4096^3 GEMM dispatch (gemm_fp8_blockscaled_kernel, 256x128 tiles, bf16 C): "
             "SQ counters, median over its dispatches",
             f"{'counter':32s} {'value':>16s}"]
    lines += [f"{k:32s} {v:16.0f}" for k, v in sorted(m.items())]
    lines += ["",
              f"cycles per XCD (GRBM_GUI_ACTIVE/8)       {xcd_cycles:12.0f}",
              f"MFMA busy / (1024 SIMDs x cycles)        {m['SQ_VALU_MFMA_BUSY_CYCLES'] / (xcd_cycles * 1024):12.3f}",
              f"VALU instructions per MFMA               {m['SQ_INSTS_VALU'] / mf:12.2f}"]
    if "SQ_INSTS_VALU_CVT" in m:
        lines.append(f"conversions per MFMA                     {m['SQ_INSTS_VALU_CVT'] / mf:12.2f}")
    if "SQ_INSTS_LDS" in m:
        lines.append(f"LDS instructions per MFMA                {m['SQ_INSTS_LDS'] / mf:12.2f}")
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in m:
        lines.append(f"MFMA cycles with a VALU op co-issued     "
                     f"{m['SQ_VALU_MFMA_COEXEC_CYCLES'] / m['SQ_VALU_MFMA_BUSY_CYCLES']:12.3f}")
    if "SQ_WAVE_CYCLES" in m:
        for k in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU"):
            if k in m:
                lines.append(f"{k + ' / SQ_WAVE_CYCLES':41s}{m[k] / m['SQ_WAVE_CYCLES']:12.3f}")
    if "SQ_LDS_IDX_ACTIVE" in m and "SQ_LDS_BANK_CONFLICT" in m:
        lines.append(f"LDS bank-conflict cycles / LDS active    "
                     f"{m['SQ_LDS_BANK_CONFLICT'] / m['SQ_LDS_IDX_ACTIVE']:12.3f}")
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, "sq_counters_gemm_4096.txt"), "w") as f:
        f.write("commands: cd /tmp && export TMPDIR=/tmp; for each counter set P of bench.py's "
                "SQ_PASSES: rocprofv3 --pmc P -f csv -d <dir> -o run -- python3 bench.py --mode "
                "profile\nsummary: python3 bench.py --summarize-sq <dir 1> <dir 2>\n\n")
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def to_dev_bf16(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def quant_act_bytes(M, K):
    return 2 * M * K + M * K + 4 * M * (K // 128)


def quant_weight_bytes(K, N):
    return 2 * K * N + K * N + 4 * (K // 128) * (N // 128)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


NVFP4_ORACLE_ROWS = 128   # rows of the 4096^3 NVFP4 GEMM the (slower) NVFP4 oracle computes


def tolerance(C_ref, S, bf16):
    """|C - C_ref| bound of the parity tests: 1e-5*sum|ab| + 1e-6, plus one bf16 ulp of the
    reference for bf16 output"""
    tol = 1e-5 * S + 1e-6
    if bf16:
        mag = np.maximum(np.abs(C_ref) + tol, 2.0 ** -126)
        tol = tol + 2.0 ** (np.floor(np.log2(mag)) - 7)
    return tol


def next_rows_baseline(A, B, C_ref, S, nxt, nt):
    """The oracle on the fused-epilogue, UE8M0 and NVFP4 variants of the 4096^3 step, timed,
    and the GPU's outputs of each checked against it (codes and scales bit for bit, GEMM
    outputs as a fraction of the tolerance)."""
    import oracle
    out = {}
    bits, Cq, sC = nxt["fused"]
    t0 = time.perf_counter()
    rq, rs = oracle.quantize_act(bits, nt)
    t1 = time.perf_counter()
    C = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    out["fused_epilogue"] = {
        "sample": "oracle 1x128 quantization of the fused call's own bf16 C (all 4096 rows); "
                  "C against the fp64 GEMM of the main leg",
        "quantize_seconds": round(t1 - t0, 3),
        "codes_bit_exact": bool(np.array_equal(Cq, rq)),
        "scales_bit_exact": bool(np.array_equal(sC.view(np.uint32), rs.view(np.uint32))),
        "gemm_max_error_over_tolerance": float(np.max(np.abs(C - C_ref) / tolerance(C_ref, S, True))),
    }
    gAq, geA, gBq, geB, gC = nxt["ue8m0"]
    M, K = A.shape
    N = B.shape[1]
    t0 = time.perf_counter()
    Aq, eA = oracle.quantize_act_ue8m0(A, nt)
    Bq, eB = oracle.quantize_weight_ue8m0(B, nt)
    t1 = time.perf_counter()
    Cu, Su = oracle.gemm_f64(Aq, oracle.ue8m0_decode(eA), Bq, oracle.ue8m0_decode(eB), nt)
    t2 = time.perf_counter()
    out["ue8m0"] = {
        "value": 2.0 * M * N * K / (t2 - t1) / 1e12, "unit": "TFLOP/s",
        "sample": f"whole 4096^3 step: UE8M0 quantize A and B ({t1 - t0:.2f} s), fp64 GEMM of "
                  f"all rows ({t2 - t1:.2f} s)",
        "codes_bit_exact": bool(np.array_equal(gAq, Aq) and np.array_equal(gBq, Bq)),
        "scales_bit_exact": bool(np.array_equal(geA, eA) and np.array_equal(geB, eB)),
        "gemm_max_error_over_tolerance": float(np.max(np.abs(gC - Cu) / tolerance(Cu, Su, True))),
    }
    del Cu, Su
    gA4, gsA4, ggA, gB4, gsB4, ggB, gC4 = nxt["nvfp4"]
    rows = gC4.shape[0]
    t0 = time.perf_counter()
    A4, sA4, gA = oracle.quantize_nvfp4(A)
    B4, sB4, gB = oracle.quantize_nvfp4(np.ascontiguousarray(B.T))
    t1 = time.perf_counter()
    C4, S4 = oracle.gemm_nvfp4_f64(A4, sA4, gA, B4, sB4, gB, nt, rows=(0, rows))
    t2 = time.perf_counter()
    C4, S4 = C4[:rows], S4[:rows]
    out["nvfp4"] = {
        "value": 2.0 * rows * N * K / (t2 - t1) / 1e12, "unit": "TFLOP/s",
        "sample": f"NVFP4 quantize of A and B^T [4096,4096] ({t1 - t0:.2f} s, one thread), fp64 "
                  f"GEMM of the first {rows} rows ({t2 - t1:.2f} s)",
        "codes_bit_exact": bool(np.array_equal(gA4, A4) and np.array_equal(gB4, B4)),
        "scales_bit_exact": bool(np.array_equal(gsA4, sA4) and np.array_equal(gsB4, sB4)
                                 and ggA.view(np.uint32)[0] == np.float32(gA).view(np.uint32)
                                 and ggB.view(np.uint32)[0] == np.float32(gB).view(np.uint32)),
        "gemm_max_error_over_tolerance": float(np.max(np.abs(gC4 - C4) / tolerance(C4, S4, True))),
    }
    return out


def cpu_baseline(A, B, step_out=None, next_out=None):
    """The oracle as it stands (scalar C, all host threads over independent rows) on the
    4096^3 workload: quantize A and B, then the fp64 GEMM for all rows.  With the GPU step's
    own outputs (codes, scales, bf16 C, computed on the GPU from the same bf16 inputs), the
    same run also reports their agreement with the oracle's: codes and scales bit for bit,
    and the largest GEMM error as a fraction of the tolerance 1e-5*sum|ab| + 1e-6 (+ one bf16
    ulp of the reference)."""
    import oracle
    nt = oracle.threads()
    t0 = time.perf_counter()
    Aq, sA = oracle.quantize_act(A, nt)
    Bq, sB = oracle.quantize_weight(B, nt)
    t1 = time.perf_counter()
    M, K = A.shape
    N = B.shape[1]
    C_ref, S = oracle.gemm_f64(Aq, sA, Bq, sB, nt)
    t2 = time.perf_counter()
    parity = None
    if step_out is not None:
        gAq, gsA, gBq, gsB, gC = step_out
        tol = tolerance(C_ref, S, True)
        parity = {
            "codes_bit_exact": bool(np.array_equal(gAq, Aq) and np.array_equal(gBq, Bq)),
            "scales_bit_exact": bool(np.array_equal(gsA.view(np.uint32), sA.view(np.uint32))
                                     and np.array_equal(gsB.view(np.uint32), sB.view(np.uint32))),
            "gemm_max_error_over_tolerance": float(np.max(np.abs(gC - C_ref) / tol)),
        }
    nxt = None if next_out is None else next_rows_baseline(A, B, C_ref, S, next_out, nt)
    return {
        "value": 2.0 * M * N * K / (t2 - t1) / 1e12,
        "unit": "TFLOP/s",
        "cores": nt,
        "host_cpus": os.cpu_count(),
        "cores_note": "threads the oracle ran on: the host's CPUs capped at 16, the CPU share "
                      "of one GPU on the measuring box",
        "kind": "oracle",
        "sample": f"whole 4096^3 step: oracle quantize A and B ({t1 - t0:.2f} s) then fp64 "
                  f"dequantize-matmul of all {M} rows ({t2 - t1:.2f} s); value = GEMM flops "
                  f"/ GEMM time",
        "quantize_GBps": (quant_act_bytes(M, K) + quant_weight_bytes(K, N)) / (t1 - t0) / 1e9,
        "seconds": t2 - t0,
        "cpu_model": cpu_model(),
        "parity_of_the_gpu_step": parity,
        "next_rows": nxt,
    }


def time_weight_quantizer(torch, fgq, W, Wq, sW, stream, reps):
    """The 128x128 weight quantizer on a large weight (the prefill workload's W [16384,7168]),
    rotating over two buffer sets (704 MB, beyond the 256 MB Infinity Cache): per launch
    between two events, and back to back."""
    Ws, Wqs, sWs = [W, W.clone()], [Wq, torch.empty_like(Wq)], [sW, torch.empty_like(sW)]
    for r in range(16):
        fgq.fgq_quantize_weight_128x128(Ws[r % 2], Wqs[r % 2], sWs[r % 2], stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for r, (a, b) in enumerate(ev):
        a.record(stream)
        fgq.fgq_quantize_weight_128x128(Ws[r % 2], Wqs[r % 2], sWs[r % 2], stream)
        b.record(stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for r in range(8):
        fgq.fgq_quantize_weight_128x128(Ws[r % 2], Wqs[r % 2], sWs[r % 2], stream)
    e1.record(stream)
    torch.cuda.synchronize()
    K, N = W.shape
    byt = quant_weight_bytes(K, N)
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    gbs = byt / (us * 1e-6) / 1e9
    bgbs = byt / (e0.elapsed_time(e1) / 8 * 1e-3) / 1e9
    log(f"weight quant [{K},{N}]: {us:.1f} us = {gbs:.0f} GB/s per launch, {bgbs:.0f} GB/s "
        f"back to back")
    return {"workload": f"weight quantize W [{K},{N}] bf16 -> E4M3 + fp32 [{K // 128},{N // 128}]",
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "us": round(us, 2),
            "back_to_back_GBps": round(bgbs, 1), "back_to_back_frac": round(bgbs / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": byt}


def step_outputs(torch, fgq, A, B, dev):
    """The outputs of one more pass of each timed 4096^3 step, on the same resident inputs, for
    the oracle comparison: the FP8 step (codes, scales, bf16 C), the fused GEMM + quantization
    of C, the UE8M0 step and the NVFP4 step (C of its first rows only).  Taken after every
    timed region, so that the host copies do not leave the GPU idle (and its clock lowered)
    before a measurement."""
    M, K = A.shape
    N = B.shape[1]

    def host(t):
        return t.cpu().numpy()

    def host_f64(t):
        return t.float().cpu().numpy().astype(np.float64)

    Aq, sA = fgq.fgq_quantize_act_1x128(A)
    Bq, sB = fgq.fgq_quantize_weight_128x128(B)
    C = fgq.fgq_gemm_fp8_blockscaled(Aq, sA, Bq, sB)
    step_out = [host(Aq), host(sA), host(Bq), host(sB), host_f64(C)]
    Cq = torch.empty((M, N), dtype=torch.uint8, device=dev)
    sC = torch.empty((M, N // 128), dtype=torch.float32, device=dev)
    fgq.fgq_gemm_fp8_blockscaled_quant(Aq, sA, Bq, sB, C, Cq, sC)
    nxt = {"fused": [host(C.view(torch.int16)).view(np.uint16), host(Cq), host(sC)]}
    qA, eA = fgq.fgq_quantize_act_1x128_ue8m0(A)
    qB, eB = fgq.fgq_quantize_weight_128x128_ue8m0(B)
    fgq.fgq_gemm_fp8_blockscaled_ue8m0(qA, eA, qB, eB, C)
    nxt["ue8m0"] = [host(qA), host(eA), host(qB), host(eB), host_f64(C)]
    A4, sA4, gA4 = fgq.fgq_quantize_nvfp4(A)
    B4, sB4, gB4 = fgq.fgq_quantize_nvfp4(B.t().contiguous())
    fgq.fgq_gemm_nvfp4(A4, sA4, gA4, B4, sB4, gB4, C)
    nxt["nvfp4"] = [host(A4), host(sA4), host(gA4), host(B4), host(sB4), host(gB4),
                    host_f64(C[:NVFP4_ORACLE_ROWS])]
    return step_out, nxt


def profile_pass(torch, fgq, synth, dev, reps=3):
    """Kernels of the hot path, a few launches each, for rocprofv3 counter runs:
    the 4096^3 step (quantize A, quantize B, GEMM), the [16384,7168] activation quantizer
    and a 512 MiB copy whose byte counts calibrate FETCH_SIZE/WRITE_SIZE."""
    A_bits, B_bits, _ = synth.workload_inputs("sq4096")
    A, B = to_dev_bf16(A_bits, torch), to_dev_bf16(B_bits, torch)
    Aq, sA = fgq.fgq_quantize_act_1x128(A)
    Bq, sB = fgq.fgq_quantize_weight_128x128(B)
    C = torch.empty((4096, 4096), dtype=torch.bfloat16, device=dev)
    X_bits, _, _ = synth.workload_inputs("actq")
    X = to_dev_bf16(X_bits, torch)
    Xq = torch.empty(X.shape, dtype=torch.uint8, device=dev)
    sX = torch.empty((X.shape[0], X.shape[1] // 128), dtype=torch.float32, device=dev)
    src = torch.ones(128 << 20, dtype=torch.float32, device=dev)   # 512 MiB
    dst = torch.empty_like(src)
    for _ in range(reps):
        fgq.fgq_quantize_act_1x128(A, Aq, sA)
        fgq.fgq_quantize_weight_128x128(B, Bq, sB)
        fgq.fgq_gemm_fp8_blockscaled(Aq, sA, Bq, sB, C)
        fgq.fgq_quantize_act_1x128(X, Xq, sX)
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log("profile pass done")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    # a cold GPU needs ~30 ms of this work to reach its steady clock (the first steps run
    # ~25% slower), so before the --warmup steps the step is run until at least this much
    # GPU time has passed, whatever --warmup says (reported as settle_ms / settle_steps)
    ap.add_argument("--settle-ms", type=float, default=200.0)
    ap.add_argument("--quant-reps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="write profiles/ summaries from rocprofv3 csv output and exit")
    ap.add_argument("--summarize-sq", nargs="+", metavar="DIR",
                    help="write profiles/sq_counters_gemm_4096.txt from the SQ counter passes "
                         "(SQ_PASSES) of --mode profile and exit")
    ap.add_argument("--mode", choices=["bench", "profile"], default="bench",
                    help="profile: a short pass for hardware-counter runs -- the GEMM, both "
                         "quantizers and a plain 512 MiB copy (torch.mul by 1) as the "
                         "calibration of the byte counters; prints no JSON")
    args = ap.parse_args()
    if args.summarize:
        summarize(*args.summarize)
        return
    if args.summarize_sq:
        summarize_sq(args.summarize_sq)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path has no multi-GPU stage here "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import fine_grained_block_fgq_amd as fgq
    from fine_grained_block_fgq_amd import calib as fgq_calib
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(2)
    fgq.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.mode == "profile":
        profile_pass(torch, fgq, synth, dev)
        return

    # ---- the step workload: 4096^3, A N(0,1), B N(0,0.02), bf16 C -----------------------
    w = synth.WORKLOADS["sq4096"]
    M, N, K = w.M, w.N, w.K
    log(f"generating {w.name} inputs")
    A_bits, B_bits, _ = synth.workload_inputs("sq4096")
    A = to_dev_bf16(A_bits, torch)
    B = to_dev_bf16(B_bits, torch)
    Aq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sA = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    Bq = torch.empty((K, N), dtype=torch.uint8, device=dev)
    sB = torch.empty((K // 128, N // 128), dtype=torch.float32, device=dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        fgq.fgq_quantize_act_1x128(A, Aq, sA, stream)
        fgq.fgq_quantize_weight_128x128(B, Bq, sB, stream)
        if ev is not None:
            ev[0].record(stream)
        fgq.fgq_gemm_fp8_blockscaled(Aq, sA, Bq, sB, C, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    # clock settle: batches of steps between two events until the GPU time adds up to
    # --settle-ms (measured, not assumed from a step count)
    settle_ms, settle_steps = 0.0, 0
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    while settle_ms < args.settle_ms:
        s0.record(stream)
        for _ in range(50):
            step()
        s1.record(stream)
        torch.cuda.synchronize()
        settle_ms += s0.elapsed_time(s1)
        settle_steps += 50
    log(f"clock settle: {settle_steps} steps, {settle_ms:.1f} ms of GPU time")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: exactly `steps` steps; HIP events on the launch stream bracket each GEMM
    # (the dominant kernel; events between every kernel would add their own gaps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    gm_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    # the two quantizers of the step, each between its own events (outside the timed steps)
    qev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(50)]
    for e in qev:
        e[0].record(stream)
        fgq.fgq_quantize_act_1x128(A, Aq, sA, stream)
        e[1].record(stream)
        fgq.fgq_quantize_weight_128x128(B, Bq, sB, stream)
        e[2].record(stream)
    torch.cuda.synchronize()
    qa_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in qev]))
    qw_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in qev]))
    lib = fgq.load()
    sp = stream.cuda_stream

    def b2b_ms(call, *args, n=40):
        """mean duration of n back-to-back launches of a C entry point between two events
        (the events around every short launch, and the binding's per-call checks, read high)"""
        if call(*args) != 0:
            raise RuntimeError(f"{call.__name__} refused the arguments")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            call(*args)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    qa_b2b = b2b_ms(lib.fgq_quantize_act_1x128, A.data_ptr(), Aq.data_ptr(), sA.data_ptr(), M, K,
                    sp)
    qw_b2b = b2b_ms(lib.fgq_quantize_weight_128x128, B.data_ptr(), Bq.data_ptr(), sB.data_ptr(),
                    K, N, sp)
    gm_all = np.array([e[0].elapsed_time(e[1]) for e in evs])
    flops = 2.0 * M * N * K
    gemm_tflops = flops / (gm_ms * 1e-3) / 1e12
    # measured ceiling: f16 MFMAs only (the partials' instruction), two waves per SIMD on
    # every CU, ~1 ms per launch, at the same (warm) clock
    props = torch.cuda.get_device_properties(dev)
    ncu = props.multi_processor_count
    cal_out = torch.empty((2 * ncu * 512,), dtype=torch.float32, device=dev)
    cal_iters = 2000
    fgq_calib.fgq_calib_mfma_f16(cal_out, 2 * ncu, cal_iters, stream)
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(10)]
    for a, b in cev:
        a.record(stream)
        cal_flops = fgq_calib.fgq_calib_mfma_f16(cal_out, 2 * ncu, cal_iters, stream)
        b.record(stream)
    torch.cuda.synchronize()
    mfma_ceiling = cal_flops / (float(np.median([a.elapsed_time(b) for a, b in cev])) * 1e-3) / 1e12
    # the same for the FP8 MFMAs (16x16x128 f8f6f4), which the GEMM does not use: what the
    # FP8 matrix cores reach here, for context next to the 5.0 PFLOP/s datasheet peak
    fgq_calib.fgq_calib_mfma_fp8(cal_out, 2 * ncu, cal_iters // 2, stream)
    for a, b in cev:
        a.record(stream)
        cal_flops8 = fgq_calib.fgq_calib_mfma_fp8(cal_out, 2 * ncu, cal_iters // 2, stream)
        b.record(stream)
    torch.cuda.synchronize()
    mfma8_ceiling = cal_flops8 / (float(np.median([a.elapsed_time(b) for a, b in cev])) * 1e-3) / 1e12
    del cal_out
    log(f"MFMA-only ceilings: 16x16x32 f16 {mfma_ceiling:.0f}, 16x16x128 fp8 "
        f"{mfma8_ceiling:.0f} TFLOP/s")
    log(f"step {ms_per_step:.4f} ms | quant A {qa_ms*1e3:.1f} us  quant B {qw_ms*1e3:.1f} us  "
        f"GEMM {gm_ms*1e3:.1f} us = {gemm_tflops:.0f} TFLOP/s")

    # ---- fused epilogue: GEMM + 1x128 quantization of C in one launch, against the two
    # launches it replaces (GEMM with bf16 C, then the activation quantizer over C) --------
    Cq = torch.empty((M, N), dtype=torch.uint8, device=dev)
    sC = torch.empty((M, N // 128), dtype=torch.float32, device=dev)
    reps = max(10, args.steps // 2)
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    for r in range(reps + 3):
        e = fev[r - 3] if r >= 3 else None
        if e is not None:
            e[0].record(stream)
        fgq.fgq_gemm_fp8_blockscaled_quant(Aq, sA, Bq, sB, C, Cq, sC, stream=stream)
        if e is not None:
            e[1].record(stream)
        fgq.fgq_gemm_fp8_blockscaled(Aq, sA, Bq, sB, C, stream=stream)
        if e is not None:
            e[2].record(stream)
        fgq.fgq_quantize_act_1x128(C, Cq, sC, stream)
        if e is not None:
            e[3].record(stream)
    torch.cuda.synchronize()
    fused_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in fev]))
    sep_ms = float(np.mean([e[1].elapsed_time(e[3]) for e in fev]))
    log(f"fused GEMM+quant {fused_ms*1e3:.1f} us vs GEMM then quantize {sep_ms*1e3:.1f} us")
    del Cq, sC

    # ---- the same step on UE8M0 (power-of-two exponent byte) scales ----------------------
    eA = torch.empty((M, K // 128), dtype=torch.uint8, device=dev)
    eB = torch.empty((K // 128, N // 128), dtype=torch.uint8, device=dev)
    uev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    for r in range(reps + 3):
        e = uev[r - 3] if r >= 3 else None
        if e is not None:
            e[0].record(stream)
        fgq.fgq_quantize_act_1x128_ue8m0(A, Aq, eA, stream)
        if e is not None:
            e[1].record(stream)
        fgq.fgq_quantize_weight_128x128_ue8m0(B, Bq, eB, stream)
        if e is not None:
            e[2].record(stream)
        fgq.fgq_gemm_fp8_blockscaled_ue8m0(Aq, eA, Bq, eB, C, stream=stream)
        if e is not None:
            e[3].record(stream)
    torch.cuda.synchronize()
    ue_ms = [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in uev])) for i in range(3)]
    ue_act_b2b = b2b_ms(lib.fgq_quantize_act_1x128_ue8m0, A.data_ptr(), Aq.data_ptr(),
                        eA.data_ptr(), M, K, sp)
    log(f"ue8m0: quant A {ue_ms[0]*1e3:.1f} us  quant B {ue_ms[1]*1e3:.1f} us  "
        f"GEMM {ue_ms[2]*1e3:.1f} us")
    del eA, eB

    # ---- NVFP4: the same shapes with E2M1 codes, per-16 E4M3 and global fp32 scales; the
    # weight is quantized from its [N, K] transpose ----------------------------------------
    Bt = B.t().contiguous()
    A4 = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    sA4 = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    gA4 = torch.empty((fgq.FGQ_NVFP4_GLOBAL_FLOATS,), dtype=torch.float32, device=dev)
    B4 = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    sB4 = torch.empty((N, K // 16), dtype=torch.uint8, device=dev)
    gB4 = torch.empty((fgq.FGQ_NVFP4_GLOBAL_FLOATS,), dtype=torch.float32, device=dev)
    nev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    for r in range(reps + 3):
        e = nev[r - 3] if r >= 3 else None
        if e is not None:
            e[0].record(stream)
        fgq.fgq_quantize_nvfp4(A, A4, sA4, gA4, stream)
        if e is not None:
            e[1].record(stream)
        fgq.fgq_quantize_nvfp4(Bt, B4, sB4, gB4, stream)
        if e is not None:
            e[2].record(stream)
        fgq.fgq_gemm_nvfp4(A4, sA4, gA4, B4, sB4, gB4, C, stream=stream)
        if e is not None:
            e[3].record(stream)
    torch.cuda.synchronize()
    nv_ms = [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in nev])) for i in range(3)]
    nv_act_b2b = b2b_ms(lib.fgq_quantize_nvfp4, A.data_ptr(), A4.data_ptr(), sA4.data_ptr(),
                        gA4.data_ptr(), M, K, sp)
    log(f"nvfp4: quant A {nv_ms[0]*1e3:.1f} us  quant B {nv_ms[1]*1e3:.1f} us  "
        f"GEMM {nv_ms[2]*1e3:.1f} us")
    del Bt, A4, sA4, gA4, B4, sB4, gB4
    # algorithmic bytes of one activation quantization in each format
    ue8_act_bytes = 2 * M * K + M * K + M * (K // 128)
    nv4_act_bytes = 2 * M * K + M * K // 2 + M * K // 16 + 4

    # ---- standalone activation quantizer, X [16384,7168] (rotating buffers) -------------
    wq = synth.WORKLOADS["actq"]
    Mq, Kq = wq.M, wq.K
    X_bits, _, _ = synth.workload_inputs("actq")
    nbuf = 4
    Xs = [to_dev_bf16(X_bits, torch) for _ in range(nbuf)]
    Xqs = [torch.empty((Mq, Kq), dtype=torch.uint8, device=dev) for _ in range(nbuf)]
    sXs = [torch.empty((Mq, Kq // 128), dtype=torch.float32, device=dev) for _ in range(nbuf)]
    for r in range(8 * nbuf):   # warm again after the host-side input generation
        i = r % nbuf
        fgq.fgq_quantize_act_1x128(Xs[i], Xqs[i], sXs[i], stream)
    torch.cuda.synchronize()
    qev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.quant_reps)]
    for r, (e0, e1) in enumerate(qev):
        i = r % nbuf
        e0.record(stream)
        fgq.fgq_quantize_act_1x128(Xs[i], Xqs[i], sXs[i], stream)
        e1.record(stream)
    torch.cuda.synchronize()
    q_ms = float(np.mean([a.elapsed_time(b) for a, b in qev]))
    # back to back: 4 rounds over the buffers between two events (each launch's ramp-up
    # overlaps the previous one's drain, as in a stream of quantizations)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for r in range(4 * nbuf):
        i = r % nbuf
        fgq.fgq_quantize_act_1x128(Xs[i], Xqs[i], sXs[i], stream)
    e1.record(stream)
    torch.cuda.synchronize()
    qb_ms = e0.elapsed_time(e1) / (4 * nbuf)
    # measured ceiling: a streaming kernel with the same traffic (16 bytes read, 8 written per
    # lane) over the same rotating buffers, per launch and back to back
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.quant_reps)]
    for r, (a, b) in enumerate(sev):
        i = r % nbuf
        a.record(stream)
        s_bytes = fgq_calib.fgq_calib_stream(Xs[i], Xqs[i], stream)
        b.record(stream)
    e0.record(stream)
    for r in range(4 * nbuf):
        fgq_calib.fgq_calib_stream(Xs[r % nbuf], Xqs[r % nbuf], stream)
    e1.record(stream)
    torch.cuda.synchronize()
    s_gbs = s_bytes / (float(np.mean([a.elapsed_time(b) for a, b in sev])) * 1e-3) / 1e9
    sb_gbs = s_bytes / (e0.elapsed_time(e1) / (4 * nbuf) * 1e-3) / 1e9
    log(f"same-traffic stream: {s_gbs:.0f} GB/s per launch, {sb_gbs:.0f} GB/s back to back")
    q_bytes = quant_act_bytes(Mq, Kq)
    q_gbs = q_bytes / (q_ms * 1e-3) / 1e9
    qb_gbs = q_bytes / (qb_ms * 1e-3) / 1e9
    log(f"act quant [16384,7168]: {q_ms*1e3:.1f} us = {q_gbs:.0f} GB/s per launch; "
        f"{qb_ms*1e3:.1f} us = {qb_gbs:.0f} GB/s back to back")
    # the NVFP4 quantizer on the same rotating X [16384,7168] (two passes over X: the tensor
    # amax, then the coding pass; algorithmic bytes count X once)
    del Xqs, sXs
    X4q = torch.empty((Mq, Kq // 2), dtype=torch.uint8, device=dev)
    X4s = torch.empty((Mq, Kq // 16), dtype=torch.uint8, device=dev)
    X4g = torch.empty((fgq.FGQ_NVFP4_GLOBAL_FLOATS,), dtype=torch.float32, device=dev)
    for r in range(4 * nbuf):
        fgq.fgq_quantize_nvfp4(Xs[r % nbuf], X4q, X4s, X4g, stream)
    torch.cuda.synchronize()
    nqev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(args.quant_reps)]
    for r, (a, b) in enumerate(nqev):
        a.record(stream)
        fgq.fgq_quantize_nvfp4(Xs[r % nbuf], X4q, X4s, X4g, stream)
        b.record(stream)
    e0.record(stream)
    for r in range(4 * nbuf):
        fgq.fgq_quantize_nvfp4(Xs[r % nbuf], X4q, X4s, X4g, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    nq_ms = float(np.mean([a.elapsed_time(b) for a, b in nqev]))
    nqb_ms = e0.elapsed_time(e1) / (4 * nbuf)
    nq_bytes = 2 * Mq * Kq + Mq * Kq // 2 + Mq * Kq // 16 + 4
    log(f"nvfp4 quant [16384,7168]: {nq_ms*1e3:.1f} us per launch = "
        f"{nq_bytes / (nq_ms * 1e-3) / 1e9:.0f} GB/s; {nqb_ms*1e3:.1f} us back to back")
    del Xs, X4q, X4s, X4g

    # ---- the other GEMM workloads (parity-test shapes; reported, not the headline) -------
    gemm_cfgs = {}
    for name in ("tiny", "skinny", "prefill"):
        wc = synth.WORKLOADS[name]
        Mc, Nc, Kc = wc.M, wc.N, wc.K
        Ab, Bb, _ = synth.workload_inputs(name)
        Ac, Bc = to_dev_bf16(Ab, torch), to_dev_bf16(Bb, torch)
        Acq, sAc = fgq.fgq_quantize_act_1x128(Ac, stream=stream)
        Bcq, sBc = fgq.fgq_quantize_weight_128x128(Bc, stream=stream)
        if name == "prefill":
            wq_stats = time_weight_quantizer(torch, fgq, Bc, Bcq, sBc, stream, args.quant_reps)
        del Ac, Bc
        out_dt = torch.bfloat16 if wc.out_dtype == "bf16" else torch.float32
        Cc = torch.empty((Mc, Nc), dtype=out_dt, device=dev)
        n = 20 if name == "prefill" else 200
        # one checked call through the binding, then the C entry point with the same
        # arguments, so that the binding's per-call Python checks (several us) do not set
        # the pace of the small shapes
        fgq.fgq_gemm_fp8_blockscaled(Acq, sAc, Bcq, sBc, Cc, stream=stream)
        code = fgq.FGQ_OUT_BF16 if out_dt == torch.bfloat16 else fgq.FGQ_OUT_F32
        # the HBM-bound skinny shape rotates over copies of its operands totalling >= 512 MB,
        # so the 256 MB Infinity Cache cannot serve them; the others run on one set
        sets = [(Acq, sAc, Bcq, sBc)]
        if name == "skinny":
            per = Acq.numel() + Bcq.numel() + 4 * (sAc.numel() + sBc.numel())
            sets += [tuple(t.clone() for t in sets[0]) for _ in range(-(-(512 << 20) // per) - 1)]
        raw = [(a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(), Cc.data_ptr(), Mc, Nc,
                Kc, code, stream.cuda_stream) for a, sa, b, sb in sets]
        lib = fgq.load()
        if lib.fgq_gemm_fp8_blockscaled(*raw[0]) != 0:
            raise RuntimeError(f"GEMM {name}: the C entry point refused the arguments")
        for r in range(60 if name == "prefill" else 4000):   # ~50 ms: back to the steady clock
            lib.fgq_gemm_fp8_blockscaled(*raw[r % len(raw)])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for r in range(n):
            lib.fgq_gemm_fp8_blockscaled(*raw[r % len(raw)])
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        fl = 2.0 * Mc * Nc * Kc
        byt = Mc * Kc + Kc * Nc + 4 * Mc * (Kc // 128) + 4 * (Kc // 128) * (Nc // 128) \
            + Mc * Nc * (2 if out_dt == torch.bfloat16 else 4)
        gemm_cfgs[name] = {"M": Mc, "N": Nc, "K": Kc, "out": wc.out_dtype,
                           "operand_sets": len(raw),
                           "us_back_to_back": round(us, 2),
                           "TFLOPs": round(fl / (us * 1e-6) / 1e12, 1),
                           "frac_fp8_peak": round(fl / (us * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
                           "algorithmic_GBps": round(byt / (us * 1e-6) / 1e9, 1),
                           "frac_hbm_peak": round(byt / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        log(f"GEMM {name} {Mc}x{Nc}x{Kc}: {us:.1f} us back to back")
        del Acq, sAc, Bcq, sBc, Cc, sets, raw

    out = {
        "metric": METRIC,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": round(settle_ms, 1),
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 operands, exact f16 MFMA, fp32 accumulate (bf16 in/out)",
        "data": "synthetic (Philox4x32-10 seed 0): A N(0,1), B N(0,0.02)",
        "config": {"workload": "4096^3 step: quantize A 1x128 + quantize B 128x128 + "
                               "block-scaled FP8 GEMM, bf16 C",
                   "M": M, "N": N, "K": K, "out": "bf16"},
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                   "compute_units": props.multi_processor_count,
                   "memory_GiB": round(props.total_memory / 2**30, 1)},
        "roofline": {
            "bound": "mfma",
            "kernel": "gemm_fp8_blockscaled_kernel 4096^3 bf16 out",
            "achieved": round(gemm_tflops, 1),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
            "traffic": profiled_traffic("gemm_fp8_blockscaled 4096^3 bf16", "gemm"),
            "algorithmic_bytes": int(M * K + K * N + 4 * M * (K // 128)
                                     + 4 * (K // 128) * (N // 128) + 2 * M * N),
            "frac_f16_peak": round(gemm_tflops / PEAK_F16_TFLOPS, 4),
            "median_us": round(float(np.median(gm_all)) * 1e3, 2),
            "min_us": round(float(gm_all.min()) * 1e3, 2),
            "mfma_only_ceiling": round(mfma_ceiling, 1),
            "frac_of_mfma_only_ceiling": round(gemm_tflops / mfma_ceiling, 4),
            "fp8_mfma_only_ceiling": round(mfma8_ceiling, 1),
            "note": "partials use f16 MFMAs on exactly converted E4M3 operands: the gfx950 FP8 "
                    "MFMA's own sum misses the 1e-5*sum|ab| tolerance (9.7x over it on the tiny "
                    "workload's codes, tests/test_gpu_fp8_mfma.py); frac_f16_peak is against the "
                    "2500 TFLOP/s dense f16 peak of the instruction used, "
                    "fp8_mfma_only_ceiling is what the unused FP8 MFMAs reach here",
        },
        "kernels_us": {"quantize_act_4096x4096": round(qa_ms * 1e3, 2),
                       "quantize_weight_4096x4096": round(qw_ms * 1e3, 2),
                       "gemm_4096^3": round(gm_ms * 1e3, 2),
                       "quantize_act_4096x4096_back_to_back": round(qa_b2b * 1e3, 2),
                       "quantize_weight_4096x4096_back_to_back": round(qw_b2b * 1e3, 2),
                       "note": "back_to_back: 40 launches of the C entry point between two "
                               "events on the same 50 MB of buffers, which the 256 MB Infinity "
                               "Cache holds (the HBM-bound quantizer figures are under quantize "
                               "and quantize_weight)"},
        "quantize": {
            "workload": "activation quantize X [16384,7168] bf16 -> E4M3 + fp32 [16384,56]",
            "bound": "hbm",
            "achieved": round(q_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(q_gbs / PEAK_HBM_GBS, 4),
            "us": round(q_ms * 1e3, 2),
            "back_to_back_GBps": round(qb_gbs, 1),
            "back_to_back_frac": round(qb_gbs / PEAK_HBM_GBS, 4),
            "stream_ceiling_GBps": round(s_gbs, 1),
            "frac_of_stream_ceiling": round(q_gbs / s_gbs, 4),
            "back_to_back_frac_of_stream_ceiling": round(qb_gbs / sb_gbs, 4),
            "algorithmic_bytes": q_bytes,
            "traffic": profiled_traffic("quant_act_1x128 16384x7168", "quant_act"),
        },
        "quantize_weight": wq_stats,
        "quantize_nvfp4": {
            "workload": "NVFP4 quantize X [16384,7168] bf16 -> E2M1 [16384,3584] + E4M3 "
                        "[16384,448] + fp32 global (rotating inputs, 940 MB)",
            "bound": "hbm",
            "us": round(nq_ms * 1e3, 2),
            "achieved": round(nq_bytes / (nq_ms * 1e-3) / 1e9, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(nq_bytes / (nq_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "us_back_to_back": round(nqb_ms * 1e3, 2),
            "back_to_back_frac": round(nq_bytes / (nqb_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": nq_bytes,
            "note": "two passes over X (the tensor amax precedes every block's coding); the "
                    "algorithmic bytes count X once",
        },
        "fused_epilogue": {
            "workload": "4096^3 GEMM + 1x128 E4M3 quantization of its bf16 C",
            "fused_us": round(fused_ms * 1e3, 2),
            "separate_us": round(sep_ms * 1e3, 2),
            "saved_us": round((sep_ms - fused_ms) * 1e3, 2),
            "fused_tflops": round(flops / (fused_ms * 1e-3) / 1e12, 1),
            "fused_frac_fp8_peak": round(flops / (fused_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
        },
        "ue8m0": {
            "workload": "the 4096^3 step on UE8M0 exponent-byte scales",
            "quantize_act_us": round(ue_ms[0] * 1e3, 2),
            "quantize_act_frac_hbm_peak": round(ue8_act_bytes / (ue_ms[0] * 1e-3) / 1e9
                                                / PEAK_HBM_GBS, 4),
            "quantize_act_us_back_to_back": round(ue_act_b2b * 1e3, 2),
            "quantize_act_back_to_back_frac": round(ue8_act_bytes / (ue_act_b2b * 1e-3) / 1e9
                                                    / PEAK_HBM_GBS, 4),
            "quantize_act_back_to_back_note": "same buffers (Infinity Cache resident)",
            "quantize_weight_us": round(ue_ms[1] * 1e3, 2),
            "gemm_us": round(ue_ms[2] * 1e3, 2),
            "gemm_tflops": round(flops / (ue_ms[2] * 1e-3) / 1e12, 1),
            "gemm_frac_fp8_peak": round(flops / (ue_ms[2] * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "gemm_frac_f16_peak": round(flops / (ue_ms[2] * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
        },
        "nvfp4": {
            "workload": "the 4096^3 step in NVFP4 (E2M1, per-16 E4M3 + fp32 global scales)",
            "quantize_act_us": round(nv_ms[0] * 1e3, 2),
            "quantize_act_frac_hbm_peak": round(nv4_act_bytes / (nv_ms[0] * 1e-3) / 1e9
                                                / PEAK_HBM_GBS, 4),
            "quantize_act_us_back_to_back": round(nv_act_b2b * 1e3, 2),
            "quantize_act_back_to_back_frac": round(nv4_act_bytes / (nv_act_b2b * 1e-3) / 1e9
                                                    / PEAK_HBM_GBS, 4),
            "quantize_act_back_to_back_note": "same buffers (Infinity Cache resident)",
            "quantize_weight_us": round(nv_ms[1] * 1e3, 2),
            "gemm_us": round(nv_ms[2] * 1e3, 2),
            "gemm_tflops": round(flops / (nv_ms[2] * 1e-3) / 1e12, 1),
            "gemm_frac_fp8_peak": round(flops / (nv_ms[2] * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "gemm_frac_f16_peak": round(flops / (nv_ms[2] * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
        },
        "gemm_configs": gemm_cfgs,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the 4096^3 workload")
        step_out, next_out = step_outputs(torch, fgq, A, B, dev)
        out["cpu_baseline"] = cpu_baseline(A_bits, B_bits, step_out, next_out)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
