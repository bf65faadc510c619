#!/usr/bin/env python3
"""Benchmark of the fused linear log-prob on one MI355X.

Default workload: linear_logp forward + backward at N = 16384 tokens, D = 4096,
V = 32000, bf16 operands, 2048-token chunks, FP32 dW table, no bias, mean-loss
upstream g = -1/N (the fused linear cross-entropy benchmark of Liger-Kernel
PR #1324, "Benchmark results": one complete forward + backward training
operation). A step is one forward + backward producing logp, lse, dH and dW
(including the table's zero fill) through the C ABI on synthetic
device-resident inputs. Both paths are gated against the oracle and timed:
`fused` (linear_logp_fwd_bwd, one call, reported as `value` by default) and
`split` (linear_logp_fwd then linear_logp_bwd, reported beside it). Other
workloads (--workload) are parity-test shapes and the logits-only log-prob.

Prints ONE JSON line (throughput, roofline of the dominant kernel from live
per-kernel HIP-event timing, and the FP64 oracle timed on a bounded sample on
the host cores). Progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402
from cross_entropy_lm_amd import accounting as A  # noqa: E402

# MI355X published peaks (dense): bf16/fp16 MFMA 2.5 PFLOP/s, fp32 MFMA 157.3
# TFLOP/s, HBM3E 8 TB/s.
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0

METRIC = "fwd+bwd tokens/s linear_logp N16384 D4096 V32000 bf16; % MFMA peak"
# Liger FLCE BF16 at this workload (Liger-Kernel PR #1324, "Full all-dtype
# comparison"): another machine's figure, context only.
PAGES_TOKENS_PER_S = 18263.8

WORKLOADS = {w.name: w for w in [synth.FLCE, synth.FLCE_F16, synth.FLCE_F32, synth.RL_DEFAULT,
                                 synth.BIAS_BIGV, synth.TINY, synth.LOGITS]}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """The library's kernel sources and the build script that sets their
    compiler flags (either changes the kernels the counters measured)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "cross_entropy_lm_amd", "csrc"))):
        with open(os.path.join(ROOT, "cross_entropy_lm_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    with open(os.path.join(ROOT, "cross_entropy_lm_amd", "build.py"), "rb") as fh:
        h.update(b"build.py" + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 PMC summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


# launch-trace kinds of the library -> the names of their kernels (one name
# per role); "vendor_gemm" is the vendor library's GEMM of gemm_reference
PMC_KERNELS = {"dh_dw": ("dh_dw_kernel",), "dlogits": ("dlogits_kernel",),
               "fwd_lse": ("lse_partial_kernel", "lse_q_kernel"), "dh_dw_fwd": ("dh_dw_fwd_kernel",),
               "dh_dw_dlogits": ("dh_dw_dlogits_kernel",), "rows_fwd": ("rows_fwd_kernel",),
               "rows_bwd": ("rows_bwd_kernel",), "vendor_gemm": ("Cijk_",),
               # the two forward roles apart: over the batch (linear_logp_fwd), and
               # the single call's first chunk
               "lse_partial": ("lse_partial_kernel",), "lse_q": ("lse_q_kernel",)}
COPY_BYTES = 1 << 30  # bytes read (and written) by one calibration copy


def kernel_ident(name: str) -> str:
    """The unqualified function name of a kernel as rocprofv3 writes it:
    mangled (_ZN3llp12_GLOBAL__N_114dlogits_kernelI...) or demangled (whose
    template arguments the demangler may garble), or a plain symbol."""
    if name.startswith("_ZN"):
        i, last = 3, ""
        while i < len(name) and name[i].isdigit():
            j = i
            while name[j].isdigit():
                j += 1
            n = int(name[i:j])
            last, i = name[j:j + n], j + n
        return last
    head = re.split(r"[<(]", name.replace("(anonymous namespace)", "_"), maxsplit=1)[0]
    return head.split("::")[-1].split(" ")[-1]


def kernel_matcher(kind: str):
    """Predicate on rocprofv3 kernel names: the kernels of a launch kind."""
    pats = PMC_KERNELS[kind]
    if kind == "vendor_gemm":
        return lambda n: any(p in n for p in pats)
    return lambda n: kernel_ident(n) in pats


def pmc_per_dispatch(path: str, match) -> tuple[float, int]:
    """Mean per dispatch of one rocprofv3 counter CSV's value over the
    dispatches whose kernel name matches; rows of one dispatch are summed."""
    import csv
    import collections

    per = collections.defaultdict(float)
    with open(path) as f:
        for r in csv.DictReader(f):
            if match(r["Kernel_Name"]):
                per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no matching dispatch in {path}")
    return sum(per.values()) / len(per), len(per)


def summarize_pmc(args):
    """profiles/pmc_<kernel>_<workload>.json from four rocprofv3 --pmc CSVs:
    FETCH_SIZE and WRITE_SIZE of the bench run, and of --copy-calibration runs
    (a plain device copy of COPY_BYTES), whose readings give the scale from the
    counters' units to bytes."""
    fetch, write, cfetch, cwrite = args.summarize_pmc
    is_k = kernel_matcher(args.pmc_kernel)
    is_copy = lambda n: "copyBuffer" in n or "copy_kernel" in n  # noqa: E731
    f_val, f_n = pmc_per_dispatch(fetch, is_k)
    w_val, w_n = pmc_per_dispatch(write, is_k)
    cf_val, _ = pmc_per_dispatch(cfetch, is_copy)
    cw_val, _ = pmc_per_dispatch(cwrite, is_copy)
    kf, kw = COPY_BYTES / cf_val, COPY_BYTES / cw_val
    out = {
        "kernel": args.pmc_kernel, "workload": args.workload, "source_hash": kernel_source_hash(),
        "fetch_size_per_dispatch": f_val, "write_size_per_dispatch": w_val, "dispatches": [f_n, w_n],
        "copy_calibration": {"bytes": COPY_BYTES, "fetch_size": cf_val, "write_size": cw_val,
                             "bytes_per_fetch_unit": kf, "bytes_per_write_unit": kw},
        "hbm_read_bytes_per_launch": f_val * kf, "hbm_write_bytes_per_launch": w_val * kw,
        "hbm_bytes_per_launch": f_val * kf + w_val * kw,
    }
    print(json.dumps(out, indent=1))


def summarize_mfma(args):
    """MFMA-pipe utilisation and clock per launch kind from one rocprofv3
    --pmc run of SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE. rocprofv3
    writes each counter summed over its instances: MFMA busy cycles over the
    1024 SIMDs, GUI-active cycles over the 8 XCDs. Per dispatch: clock =
    (GUI-active / 8) / duration; MFMA utilisation = busy / ((GUI-active / 8)
    x 1024 SIMDs), rocprofv3's MfmaUtil. A 16-bit MFMA retires 1024 flop per
    busy SIMD cycle and an fp32 one 64 (the dense peaks 2.5 PFLOP/s and
    157.3 TFLOP/s over 1024 SIMDs at 2.4 GHz), so busy x that figure is the
    flop the pipes executed."""
    import csv
    import collections

    per = collections.defaultdict(dict)
    meta = {}
    with open(args.summarize_mfma) as f:
        for r in csv.DictReader(f):
            d = r["Dispatch_Id"]
            per[d][r["Counter_Name"]] = per[d].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            meta[d] = (r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    fpc = 64 if WORKLOADS[args.workload].dtype == "f32" else 1024  # flop per busy SIMD cycle
    out = {"source_hash": kernel_source_hash(), "workload": args.workload, "flop_per_busy_cycle": fpc,
           "kernels": {}}
    for kind in PMC_KERNELS:
        match = kernel_matcher(kind)
        ds = [d for d in per if match(meta[d][0]) and "SQ_VALU_MFMA_BUSY_CYCLES" in per[d]]
        if not ds:
            continue
        n = len(ds)
        busy = sum(per[d]["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds) / n
        gui = sum(per[d]["GRBM_GUI_ACTIVE"] for d in ds) / n / 8
        ns = sum(meta[d][1] for d in ds) / n
        out["kernels"][kind] = {
            "dispatches": n, "avg_duration_us": ns / 1e3, "mfma_busy_cycles": busy, "gui_active_cycles_per_xcd": gui,
            "clock_ghz": gui / ns, "mfma_util_pct": 100.0 * busy / (gui * 1024), "mfma_flop_executed": busy * fpc,
            "tflops_at_that_clock_and_util": busy * fpc / (ns * 1e-9) / 1e12}
    print(json.dumps(out, indent=1))


def copy_calibration(torch):
    """One plain device copy of COPY_BYTES (a reference for the PMC byte counters)."""
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES}), flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


# ----------------------------------------------------------------------------- linear
PATHS = {
    "fused": "linear_logp_fwd_bwd: one call, upstream g known at forward time (3 N x V x D contractions)",
    "split": "linear_logp_fwd then linear_logp_bwd with the forward's lse (4 N x V x D contractions)",
}


def time_steps(step, args, torch, llp, stream, per_step=None):
    """W untimed steps, then K steps bracketed by HIP events on the launch
    stream (one more event between consecutive steps); returns (ms per step,
    {kind: (total ms, launches)}) and fills `per_step` with the K step times."""
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    llp.llp_trace_enable(True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    llp.llp_trace_enable(False)
    if per_step is not None:
        per_step[:] = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    return ev[0].elapsed_time(ev[-1]) / args.steps, llp.llp_trace_read()


def step_stats(times):
    """Median, 20th and 80th percentile of per-step times (ms)."""
    if not times:
        return None
    q = np.percentile(np.asarray(times, dtype=np.float64), [50, 20, 80])
    return {"median": float(q[0]), "p20": float(q[1]), "p80": float(q[2]), "samples": len(times)}


def measure_ceilings(torch):
    """Same-box ceilings from the microbenchmarks in libllp_ceilings.so (None
    if that library is not built): the MFMA rate of back-to-back bf16 MFMAs on
    register operands, and the HBM streaming rates of a 16-byte-per-lane copy
    (read + write) and read, each the best of 3 timed runs after one warm-up."""
    import ctypes

    path = os.path.join(ROOT, "cross_entropy_lm_amd", "libllp_ceilings.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.llpc_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.llpc_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.llpc_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.llpc_read_out_len.argtypes = [ctypes.c_int64]
    lib.llpc_read_out_len.restype = ctypes.c_int64
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def best(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return min(ts)

    def ok(st):
        if st != 0:
            raise RuntimeError(f"ceilings microbenchmark failed (hipError {st})")

    blocks, iters = 2048, 30000
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    ms = best(lambda: ok(lib.llpc_mfma_loop(blocks, iters, ctypes.c_void_p(out.data_ptr()), sp)))
    mfma = blocks * 4 * iters * 8 * 32768 / (ms * 1e-3) / 1e12
    nbytes = 1 << 31
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    ms_c = best(lambda: ok(lib.llpc_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                         nbytes, sp)))
    red = torch.empty(lib.llpc_read_out_len(nbytes), dtype=torch.int32, device="cuda:0")
    ms_r = best(lambda: ok(lib.llpc_read(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(red.data_ptr()),
                                         sp)))
    del src, dst, red, out
    return {"mfma_loop_tflops": mfma, "copy_GBps": 2 * nbytes / (ms_c * 1e-3) / 1e9,
            "read_GBps": nbytes / (ms_r * 1e-3) / 1e9,
            "what": "same-box microbenchmarks (libllp_ceilings.so): back-to-back v_mfma_f32_32x32x16_bf16 on "
                    "register operands (2048 workgroups x 4 waves x 30000 x 8 MFMAs); a 2 GiB 16-byte-per-lane "
                    "copy (read + write bytes) and read; best of 3 runs"}


def kernel_table(tr, steps, step_flops):
    """Per launch kind: time per step, launches, average launch time and (for
    the contractions) TFLOP/s = the kind's algorithmic flop per step / its time
    per step, i.e. the average launch's flop over the average launch time."""
    kernels = {}
    for k, (tms, cnt) in tr.items():
        if cnt == 0:
            continue
        kernels[k] = {"ms_per_step": tms / steps, "launches_per_step": cnt / steps, "avg_launch_ms": tms / cnt}
        if step_flops.get(k):
            kernels[k]["tflops"] = step_flops[k] / (tms / steps * 1e-3) / 1e12
            kernels[k]["flop_per_launch"] = step_flops[k] / (cnt / steps)
    return kernels


def dw_group(N, D, V, C, K, esize, fused, table_f32=True):
    """Chunks per dW contraction (G), the library's rule (its workspace plan):
    with an FP32 table, dW and K >= 2, the single call and (for small chunks:
    16-bit operands, fewer than 128 dH tiles; or 16-bit operands with
    D % 8 == 0) the two-call path accumulate dW once per group of G chunks:
    G = 2, for small chunks up to 4096 group columns and 1 GiB of group
    buffer, at most K, then balanced: ceil(K / ceil(K / G))."""
    few = esize == 2 and -(-C // 256) * -(-D // 256) < 128
    ld = -(-C // 8) * 8
    lim = 0x7FFFFFF0
    pairable = esize == 2 and D % 8 == 0 and V * D * esize < lim and V * 2 * ld * esize < lim
    if not (table_f32 and K >= 2 and (fused or few or pairable)):
        return 1
    g = 2
    if few:
        g = max(g, min(4096 // ld, (1 << 30) // (V * ld * esize)))
    g = min(g, K)
    return -(-K // -(-K // g))  # as many groups as g needs, of balanced sizes


def schedule(N, D, V, C, K, esize, fused, table_f32=True):
    """(working chunk, chunks, chunks per dW group, dH per group) of the
    library's backward schedule with dW requested: with two or more chunks in
    the plan's group (from the shapes alone, whatever the table's dtype) and
    dH on the layout without W^T, a group runs as one working chunk of G C
    tokens (no further grouping); otherwise the caller's chunks in groups of
    G (an FP32 table's rule)."""
    gp = dw_group(N, D, V, C, K, esize, fused, True)
    ld = -(-C // 8) * 8
    lim = 0x7FFFFFF0
    kmajor = esize == 2 and D % 8 == 0 and V * D * esize < lim and V * max(gp * ld, 2 * ld) * esize < lim
    if gp >= 2 and kmajor:
        Cw = min(gp * C, N)
        return Cw, -(-N // Cw), 1, False
    G = dw_group(N, D, V, C, K, esize, fused, table_f32)
    small = esize == 2 and C % 8 == 0 and -(-C // 256) * -(-D // 256) < 128
    return C, K, G, G > 1 and small and kmajor


def chunk_step_flops(N, D, V, C, K, overlap, G=1, group_dh=False, fused=True):
    """Algorithmic flop per step of each contraction launch kind of the
    chunked part of a path: chunk k's logits tile (the single call's forward,
    fwd_lse; the backward's dlogits recompute, dlogits), dH and (its share of)
    dW each cost 2 C_k V D. With overlap, chunk k + 1's logits tiles ride in
    chunk k's dH / dW launch (dh_dw_fwd; dh_dw_dlogits) and only chunk 0's
    logits tile has a launch of its own; with groups of G chunks, the dW of a
    group runs in the launch of its last chunk; with group_dh (small chunks)
    the dH of a group runs there too, and a launch left with neither dH nor
    dW carries logits tiles only."""
    ck = [min(C, N - k * C) for k in range(K)]
    f = 2 * V * D
    lk, ok = ("fwd_lse", "dh_dw_fwd") if fused else ("dlogits", "dh_dw_dlogits")
    out = {lk: 0, "dh_dw": 0, ok: 0}
    for k in range(K):
        kg = k - k % G
        end = k % G == G - 1 or k == K - 1
        grp = sum(ck[kg:k + 1]) if end else 0
        dw = f * grp
        dh = f * grp if group_dh else f * ck[k]
        if overlap:
            if k == 0:
                out[lk] += f * ck[0]
            if k + 1 < K:
                if dh == 0 and dw == 0:
                    out[lk] += f * ck[k + 1]
                else:
                    out[ok] += dh + dw + f * ck[k + 1]
            else:
                out["dh_dw"] += dh + dw
        else:
            out[lk] += f * ck[k]
            out["dh_dw"] += dh + dw
    return out


def fused_step_flops(N, D, V, C, K, overlap, G=1, group_dh=False):
    """Contraction flop per launch kind of the single call (6 V D per token)."""
    return chunk_step_flops(N, D, V, C, K, overlap, G, group_dh, fused=True)


def split_step_flops(N, D, V, C, K, overlap, G=1, group_dh=False):
    """Contraction flop per launch kind of linear_logp_fwd (one forward over
    the batch, fwd_lse) then linear_logp_bwd (8 V D per token)."""
    out = chunk_step_flops(N, D, V, C, K, overlap, G, group_dh, fused=False)
    out["fwd_lse"] = 2 * N * V * D
    return out


def run_linear(w, args, torch, llp):
    dev = torch.device("cuda:0")
    chunk = args.chunk if args.chunk is not None else w.chunk
    tdt = torch.float32 if args.table == "f32" else {"bf16": torch.bfloat16, "f16": torch.float16,
                                                      "f32": torch.float32}[w.dtype]
    log(f"generating {w.name} on the device")
    d = synth.make_linear_t(w, dev)
    N, D, V = w.N, w.D, w.V
    op_dt = llp.dtype_code(d["h"].dtype)
    C = llp.linear_logp_chunk_rows(N, V, chunk)
    K = llp.linear_logp_num_chunks(N, V, chunk)
    logp = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    dH = torch.empty((N, D), dtype=d["h"].dtype, device=dev)
    dW = torch.empty((V, D), dtype=tdt, device=dev)
    db = torch.empty((V,), dtype=tdt, device=dev) if w.bias else None
    ws_f = torch.empty(max(1, llp.linear_logp_fwd_workspace_size(N, D, V, op_dt)), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(1, llp.linear_logp_bwd_workspace_size(N, D, V, op_dt, chunk, True, True, w.bias, True)),
                       dtype=torch.uint8, device=dev)
    ws_x = torch.empty(max(1, llp.linear_logp_fwd_bwd_workspace_size(N, D, V, op_dt, chunk, True, True, w.bias,
                                                                     True)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def split_step():
        llp.linear_logp_fwd(d["h"], d["W"], d["b"], d["t"], logp=logp, lse=lse, workspace=ws_f)
        llp.linear_logp_bwd(d["h"], d["W"], d["b"], d["t"], d["g"], lse, True, True, w.bias, chunk=chunk,
                            dH=dH, dW=dW, db=db, workspace=ws_b)

    def fused_step():
        llp.linear_logp_fwd_bwd(d["h"], d["W"], d["b"], d["t"], d["g"], True, True, w.bias, chunk=chunk,
                                logp=logp, lse=lse, dH=dH, dW=dW, db=db, workspace=ws_x)

    # correctness gate before timing (and the CPU baseline on the same sample), for both paths
    cpu = None
    accuracy = {}
    for name, step in (("split", split_step), ("fused", fused_step)):
        step()
        torch.cuda.synchronize()
        if not args.no_gate or not args.no_cpu_baseline:
            cpu, accuracy[name] = oracle_sample(w, args, logp, dH, dW, cpu, name)

    # peak device memory of one single call above its inputs: the wrapper
    # allocates the outputs and the workspace (the library allocates nothing)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    outs = llp.linear_logp_fwd_bwd(d["h"], d["W"], d["b"], d["t"], d["g"], True, True, w.bias, chunk=chunk,
                                   dW_dtype=tdt)
    torch.cuda.synchronize()
    peak_extra = torch.cuda.max_memory_allocated() - base
    out_bytes = sum(x.numel() * x.element_size() for x in outs if x is not None)
    del outs
    memory = {"peak_extra_bytes": peak_extra, "workspace_bytes": ws_x.numel(), "output_bytes": out_bytes,
              "what": "torch.cuda.max_memory_allocated above the inputs during one linear_logp_fwd_bwd "
                      "call that allocates its outputs (logp, lse, dH, dW" + (", db" if w.bias else "") +
                      ") and workspace; the library itself allocates nothing"}
    log(f"peak extra memory {peak_extra / 2**20:.1f} MiB = workspace {ws_x.numel() / 2**20:.1f} MiB + "
        f"outputs {out_bytes / 2**20:.1f} MiB")

    flops8 = A.linear_fwd_bwd_flops(N, D, V)
    exec_flops = {"fused": A.linear_model_flops(N, D, V), "split": flops8}
    peak = PEAK_TFLOPS[w.dtype]
    results = {}
    # the single call overlaps the next chunk's forward with 16-bit operands
    # (D % 8 == 0) and an FP32 table (an operand-dtype table keeps separate
    # launches), and runs dW once per group of G chunks with an FP32 table
    # (K >= 2); small chunks with C % 8 == 0 take dH per group too
    esz = 4 if w.dtype == "f32" else 2
    Cw, Kw, G, group_dh = schedule(N, D, V, C, K, esz, True, args.table == "f32")
    overlap = w.dtype in ("bf16", "f16") and Kw >= 2 and D % 8 == 0 and args.table == "f32"
    # the backward of the two-call path overlaps alike (the next chunk's dlogits recompute)
    sCw, sKw, sG, s_gdh = schedule(N, D, V, C, K, esz, False, args.table == "f32")
    s_overlap = w.dtype in ("bf16", "f16") and sKw >= 2 and D % 8 == 0 and args.table == "f32"
    for name, step, sf in (
            ("split", split_step, split_step_flops(N, D, V, sCw, sKw, s_overlap, sG, s_gdh)),
            ("fused", fused_step, fused_step_flops(N, D, V, Cw, Kw, overlap, G, group_dh))):
        log(f"{name}: warmup {args.warmup}, timed {args.steps} steps (C={C}, K={K})")
        per_step = []
        ms, tr = time_steps(step, args, torch, llp, stream, per_step)
        kernels = kernel_table(tr, args.steps, sf)
        mfma = {k: v for k, v in kernels.items() if "tflops" in v}
        results[name] = {
            "ms_per_step": ms, "tokens_per_s": A.tokens_per_s(N, ms), "step_ms": step_stats(per_step),
            # the flop this path executes: 3 contractions (single call) or 4 (split)
            "executed_flop_per_step": exec_flops[name],
            "pct_mfma_peak": 100.0 * exec_flops[name] / (ms * 1e-3) / (peak * 1e12),
            "dominant": max(mfma, key=lambda k: mfma[k]["ms_per_step"]), "kernels": kernels}
        if name == "fused":
            # not executed work: the four contractions of a forward + backward
            # that recomputes the logits, over this path's time
            results[name]["pct_mfma_peak_8vd_equivalent"] = 100.0 * flops8 / (ms * 1e-3) / (peak * 1e12)
    # same-box reference: the vendor GEMM (hipBLASLt through torch.matmul) on
    # the forward logits shape, logits written to HBM, no epilogue
    Wt_ = d["W"].t()
    hmat = d["h"]
    for _ in range(2):
        z = torch.matmul(hmat, Wt_)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        z = torch.matmul(hmat, Wt_)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_gemm = e0.elapsed_time(e1) / 3
    del z
    gemm_ref = {"ms": ms_gemm, "tflops": 2 * N * V * D / (ms_gemm * 1e-3) / 1e12,
                "what": f"torch.matmul h [{N},{D}] x W^T -> [{N},{V}] logits ({w.dtype}), vendor GEMM, no epilogue"}
    ceil = measure_ceilings(torch)
    main = results[args.path]
    other = "split" if args.path == "fused" else "fused"
    dom = main["dominant"]
    achieved = main["kernels"][dom]["tflops"]
    roof = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": achieved / peak, "traffic": traffic_from_profiles(dom, w.name)}
    if ceil is not None and w.dtype in ("bf16", "f16"):
        # the same box's sustained 16-bit MFMA rate (no memory traffic)
        roof["measured_ceiling"] = ceil["mfma_loop_tflops"]
        roof["frac_of_measured"] = achieved / ceil["mfma_loop_tflops"]
    tokens_s = main["tokens_per_s"]
    return {
        "metric": METRIC if w.name == "flce_bf16" else f"fwd+bwd tokens/s linear_logp {w.name}",
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": tokens_s / PAGES_TOKENS_PER_S if w.name == "flce_bf16" and args.table == "f32" else None,
        "vs_baseline_ref": "Liger FLCE BF16 18263.8 tokens/s (Liger-Kernel PR #1324; other hardware, context)",
        "dtype": w.dtype,
        "data": "synthetic (seeded counter-based generator; random-init weights)",
        "config": {"workload": w.name, "N": N, "D": D, "V": V, "chunk": C, "chunks": K,
                   "working_chunk": (Cw if args.path == "fused" else sCw),
                   "chunks_per_dW": (G if args.path == "fused" else sG), "dH_vocab_parts": -(-V // (8192 if w.dtype == "f32" else 32768)),
                   "bias": w.bias, "g": w.g, "dW_table": args.table, "outputs": "logp,lse,dH,dW" +
                   (",db" if w.bias else ""), "path": PATHS[args.path]},
        "pct_mfma_peak": main["pct_mfma_peak"],
        "pct_mfma_peak_basis": f"{main['executed_flop_per_step']:.4e} flop executed per step "
                               f"({'6' if args.path == 'fused' else '8'} V D per token)",
        **({"pct_mfma_peak_8vd_equivalent": main["pct_mfma_peak_8vd_equivalent"]} if args.path == "fused" else {}),
        "memory": memory,
        **({"accuracy": accuracy[args.path]} if args.path in accuracy else {}),
        "step_ms": main["step_ms"],
        "roofline": roof,
        "kernels": main["kernels"],
        "gemm_reference": gemm_ref,
        **({"ceilings": ceil} if ceil is not None else {}),
        other: {"path": PATHS[other], **results[other],
                **({"accuracy": accuracy[other]} if other in accuracy else {})},
        **({"cpu_baseline": {k: v for k, v in cpu.items() if not k.startswith("_")}}
           if cpu is not None and not args.no_cpu_baseline else {}),
    }


def oracle_sample(w, args, logp, dH, dW, prev=None, label=""):
    """FP64 oracle forward + backward (logp, dH, dW) on the first S tokens,
    timed on the host cores once; each path's logp and dH rows are gated
    against it, and the accuracy diagnostics of dH (and of dW when the sample
    is the whole batch) are returned with the CPU baseline."""
    from oracle import linear_logp as O

    S = min(args.cpu_sample_tokens, w.N)
    if prev is None:
        rows = np.arange(S)
        log(f"oracle sample: {S} tokens (host generation first)")
        host = synth.make_linear_np(w, rows=rows)
        t0 = time.perf_counter()
        rlogp, _ = O.linear_logp_fwd(host["h64"], host["W64"], host["b64"], host["t"])
        rdH, rdW, rdb = O.linear_logp_bwd(host["h64"], host["W64"], host["b64"], host["t"], host["g64"], True,
                                          True, w.bias)
        dt = time.perf_counter() - t0
        log(f"oracle {dt:.1f} s")
        prev = {"value": S / dt, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
                "sample": f"first {S} tokens of {w.name}: FP64 numpy oracle forward + backward (logp, dH, dW)"
                          f"{' + db' if w.bias else ''}, {dt:.2f} s",
                "cpu": cpu_model(), "nproc": os.cpu_count(),
                "_ref": (rlogp, rdH, rdW if S == w.N else None)}
    rlogp, rdH, rdW = prev["_ref"]
    gl = logp[:S].double().cpu().numpy()
    gh = dH[:S].double().cpu().numpy()
    tl = {"f32": (1e-5, 5e-4)}.get(w.dtype, (5e-3, 5e-2))
    tg = {"f32": (1e-5, 5e-4)}.get(w.dtype, (5e-4, 2e-2))
    ok_l = np.all(np.abs(gl - rlogp) <= tl[0] + tl[1] * np.abs(rlogp))
    ok_h = np.all(np.abs(gh - rdH) <= tg[0] + tg[1] * np.abs(rdH))
    if not args.no_gate and not (ok_l and ok_h):
        raise SystemExit(f"correctness gate failed ({label}): logp ok={ok_l} dH ok={ok_h}")
    log(f"gate ok ({label}: logp, dH on {S} tokens)")
    acc = {"dH": synth.accuracy(gh, rdH, w.dtype)}
    if rdW is not None:
        acc["dW"] = synth.accuracy(dW.double().cpu().numpy(), rdW, torch_dtype_name(dW.dtype))
    acc["reference"] = f"FP64 oracle on tokens [0, {S}), the upstream g the path receives"
    log(f"accuracy ({label}): dH max err / max {acc['dH']['max_err_over_max']:.2e}, "
        f"{acc['dH']['pct_correctly_rounded']:.4f}% correctly rounded")
    return prev, acc


def torch_dtype_name(dt) -> str:
    return {"torch.float32": "f32", "torch.bfloat16": "bf16", "torch.float16": "f16"}[str(dt)]


# ----------------------------------------------------------------------------- logits only
def run_logits(w, args, torch, llp):
    from oracle import linear_logp as O

    dev = torch.device("cuda:0")
    log(f"generating {w.name} on the device")
    d = synth.make_logits_t(w, dev)
    N, V = w.N, w.V
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    logp = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    dl = torch.empty_like(d["logits"])

    def step():
        llp.logp_fwd(d["logits"], d["t"], logp=logp, lse=lse)
        llp.logp_bwd(d["logits"], d["t"], d["g"], lse, dlogits=dl)

    step()
    torch.cuda.synchronize()
    peak_extra = torch.cuda.max_memory_allocated() - base
    S = min(args.cpu_sample_tokens, 64)
    rows = np.arange(S)
    host = synth.make_logits_rows_np(w, rows)
    t0 = time.perf_counter()
    rlogp, _ = O.logp_fwd(host["logits64"], host["t"])
    rd = O.logp_bwd(host["logits64"], host["t"], host["g64"])
    dt = time.perf_counter() - t0
    gl = logp[:S].double().cpu().numpy()
    gd = dl[:S].double().cpu().numpy()
    acc = {"dlogits": synth.accuracy(gd, rd, w.dtype), "reference": f"FP64 oracle on rows [0, {S})"}
    log(f"accuracy: dlogits max err / max {acc['dlogits']['max_err_over_max']:.2e}, "
        f"{acc['dlogits']['pct_correctly_rounded']:.4f}% correctly rounded")
    if not args.no_gate:
        if not (np.all(np.abs(gl - rlogp) <= 5e-3 + 5e-2 * np.abs(rlogp))
                and np.all(np.abs(gd - rd) <= 5e-4 + 2e-2 * np.abs(rd))):
            raise SystemExit("correctness gate failed (logits-only)")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    llp.llp_trace_enable(True)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    llp.llp_trace_enable(False)
    tr = llp.llp_trace_read()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    e0, e1 = ev[0], ev[-1]  # reused by the references below
    per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    nbytes = {"rows_fwd": N * V * 2, "rows_bwd": 2 * N * V * 2}
    kernels = {}
    for k, (tms, cnt) in tr.items():
        if cnt:
            kernels[k] = {"ms_per_step": tms / args.steps, "avg_launch_ms": tms / cnt,
                          "GBps": nbytes[k] / (tms / cnt * 1e-3) / 1e9}
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    total = A.logits_only_bytes(N, V, 2)
    ceil = measure_ceilings(torch)
    roof = {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["GBps"], "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": kernels[dom]["GBps"] / PEAK_HBM_GBS,
            "traffic": traffic_from_profiles(dom, w.name)}
    if ceil is not None:
        # the same box's streaming rate for this kernel's access mix
        roof["measured_ceiling"] = ceil["copy_GBps"] if dom == "rows_bwd" else ceil["read_GBps"]
        roof["frac_of_measured"] = kernels[dom]["GBps"] / roof["measured_ceiling"]
    out = {
        "metric": "fwd+bwd logits-only logp N32768 V151936 bf16; GB/s",
        "value": total / (ms * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded counter-based generator)",
        "config": {"workload": w.name, "N": N, "V": V, "peak_extra_bytes": peak_extra},
        "step_ms": step_stats(per_step),
        "roofline": roof,
        "kernels": kernels,
        **({"ceilings": ceil} if ceil is not None else {}),
        "accuracy": acc,
        "cpu_baseline": {"value": S * V * 3 * 2 / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                         "sample": f"first {S} rows: FP64 numpy oracle logp + dlogits, {dt:.2f} s",
                         "cpu": cpu_model(), "nproc": os.cpu_count()},
    }
    def copy_reference(dst):
        # same-box reference: a plain device copy of the same bytes (one read
        # and one write of the logits, what rows_bwd moves), into a buffer
        # whose contents are no longer needed
        for _ in range(2):
            dst.copy_(d["logits"])
        e0.record(stream)
        for _ in range(args.steps):
            dst.copy_(d["logits"])
        e1.record(stream)
        torch.cuda.synchronize()
        ms_copy = e0.elapsed_time(e1) / args.steps
        out["copy_reference"] = {"ms": ms_copy, "GBps": 2 * N * V * 2 / (ms_copy * 1e-3) / 1e9,
                                 "what": "torch copy_ of the logits into a same-size buffer (1 read + 1 write)"}

    if args.no_lse_free:
        copy_reference(dl)
        return out
    # the backward for a caller that kept no lse: the row is reduced, then
    # written (two reads, one write); its dlogits equal the saved-lse ones bit for bit
    dl2 = torch.empty_like(dl)
    llp.logp_bwd(d["logits"], d["t"], d["g"], None, dlogits=dl2)
    torch.cuda.synchronize()
    same = bool(torch.equal(dl.view(torch.int16), dl2.view(torch.int16)))
    if not same and not args.no_gate:
        raise SystemExit("correctness gate failed (logits-only backward without lse)")
    e0.record(stream)
    for _ in range(args.steps):
        llp.logp_bwd(d["logits"], d["t"], d["g"], None, dlogits=dl2)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_nolse = e0.elapsed_time(e1) / args.steps
    out["bwd_without_lse"] = {"ms": ms_nolse, "GBps": 3 * N * V * 2 / (ms_nolse * 1e-3) / 1e9,
                              "bytes": "2 reads + 1 write of the logits", "bitwise_equal_to_saved_lse": same}
    copy_reference(dl2)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="flce_bf16", choices=sorted(WORKLOADS))
    ap.add_argument("--chunk", type=int, default=None, help="tokens per backward chunk (default: the workload's)")
    ap.add_argument("--table", default="f32", choices=["f32", "op"], help="dW table dtype")
    ap.add_argument("--path", default="fused", choices=["fused", "split"],
                    help="path reported as `value` (the other is timed too and reported beside it)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=16384)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gate", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run one plain device copy of 1 GiB (reference for PMC byte counters)")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="print the HBM traffic summary of --pmc-kernel from rocprofv3 counter CSVs")
    ap.add_argument("--pmc-kernel", default="dh_dw", choices=sorted(PMC_KERNELS))
    ap.add_argument("--summarize-mfma", metavar="CSV",
                    help="print MFMA utilisation and clock per launch kind from a rocprofv3 counter CSV of "
                         "SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE")
    ap.add_argument("--no-lse-free", action="store_true",
                    help="logits-only workload: leave out the extra timing of the backward without a saved lse "
                         "(so that every rows_bwd dispatch of a profiled run is the saved-lse one)")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.summarize_mfma:
        summarize_mfma(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU layout is a "
              "design note, not a measured path.", file=sys.stderr)
        sys.exit(2)
    import torch

    from cross_entropy_lm_amd import llp

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    llp.lib()  # fail loudly if the HIP library is missing
    w = WORKLOADS[args.workload]
    if isinstance(w, synth.LogitsWorkload):
        out = run_logits(w, args, torch, llp)
    else:
        out = run_linear(w, args, torch, llp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
