"""Benchmark of the decomposed int8 matmul on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config sweep13b] [--extra q_proj,decode1,decode4,decode16]

One step = one whole int8_matmul call (activation pass: outlier detection,
row quantization and compaction; int8 MFMA GEMM; fp16 outlier MFMA; fused
dequant epilogue) on inputs already resident in HBM.  The weight is
prepared once before timing (int8_prepare_weight; its time is reported
separately: the first call, and in ``prepare_weight`` the steady-state rate
of 10 more calls against HBM bandwidth).  Prints one JSON line.

* headline   -- the LLaMA-13B-shaped sweep workload at t = 6 (4096 tokens,
               5120 -> 13824), the largest single-GPU workload; ``extra``
               holds the same measurement, in the same process, for the 7B
               q_proj prefill (4096^3) and the M = 1 and M = 16 decode calls
               (8192 -> 28672), so both halves of the metric (% int8 MFMA
               peak, % HBM bandwidth) are timed in one run.
* value      -- effective TOPS = 2*M*N*K / (wall time of K steps / K).
* weights    -- every workload cycles through enough prepared weight copies
               (at least 768 MiB in all, so three times the 256 MB MALL) that
               each call reads its weight from HBM, as a model's layers do.
* roofline   -- the matmul kernel alone: algorithmic work per launch divided by
               its average duration, read from the HIP events its dispatch
               stamps (int8_matmul_profiled) over K calls run right after
               the timed region, on the same stream and inputs.  Prefill shapes are
               bound by the int8 MFMA peak (5.0 POP/s dense), decode shapes
               by HBM (8 TB/s); traffic comes from the committed rocprofv3
               FETCH_SIZE / WRITE_SIZE counters when they match the current
               kernel sources, else null.
* warm-up    -- W calls, continued until it has lasted at least 50 ms
               (warmup_calls_run says how many ran): the clocks need that long
               under load to settle, and value is the steady-state rate.
* other_entry_points -- the headline workload through int8_linear (with a
               bias) and int8_column_absmax, after the timed region.
* per_call   -- median and minimum of per-call times (HIP events around each
               whole call, and the kernel's own stamps), from passes after
               the timed region.
* ceilings   -- after the timed regions, the practical ceilings of this GPU
               from the probe library (libint8mm_ceilings.so): the int8 MFMA
               issue rate on random and on zero operands, and the read rate of
               a 2 GiB contiguous-chunk stream; roofline.frac_of_measured_ceiling
               sets each matmul kernel against the matching one.
* cpu_baseline -- the CPU oracle (oracle/, unchanged) timed on this host: on a
               row sample of the headline workload with all BLAS threads, and
               single-threaded on the tiny and the M = 16 decode workloads; the
               host's CPU count and the BLAS build are reported beside it.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TOPS of decomposed int8 matmul; % int8 MFMA peak / % HBM BW"
WARMUP_MIN_S = 0.05  # shortest warm-up: clocks settle within tens of milliseconds
PEAK_INT8_TOPS = 5000.0    # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_FP16_TOPS = 2500.0    # MI355X dense fp16 MFMA, 2.5 PFLOP/s
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, 8 TB/s
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["gemm_prefill.hip", "gemm_decode.hip", "device_common.h"]

WORKLOAD_TEXT = {
    "tiny": "tiny 16x1024x1024 (2 planted outlier columns)",
    "q_proj": "LLaMA-7B q_proj prefill, 4096 tokens, 4096->4096 (6 planted outlier columns)",
    "ffn_up": "LLaMA-7B FFN up prefill, 2048 tokens, 4096->11008 (20 planted outlier columns)",
    "ffn_down": "LLaMA-7B FFN down prefill, 2048 tokens, 11008->4096 (55 planted outlier columns)",
    "decode1": "decode M=1, 8192->28672, pre-quantized weight (8 planted outlier columns)",
    "decode4": "decode M=4, 8192->28672, pre-quantized weight (8 planted outlier columns)",
    "decode16": "decode M=16, 8192->28672, pre-quantized weight (8 planted outlier columns)",
    "sweep13b": "LLaMA-13B-shaped prefill, 4096 tokens, 5120->13824, 51 Student-t(3) columns",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "int8_quantized_matmul_col_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


class HipEvents:
    """Raw hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        self.hip.hipEventSynchronize(b)
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, e: int) -> None:
        self.hip.hipEventDestroy(e)


def committed_traffic(config: str, src_hash: str):
    """HBM bytes per launch of the matmul kernel from the committed rocprofv3
    counter runs, if they were taken on the current kernel sources."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(config)
    if not ent or ent.get("kernel_source_hash") != src_hash:
        return None
    return ent.get("hbm_bytes_per_launch")


COPY_CAL_BYTES = 256 << 20   # bytes read (and written) by one calibration copy
COPY_KERNEL_TAG = "neg"


def _pmc_means(run_dir: str, counter: str):
    """Mean value of `counter` per dispatch, keyed by kernel name, from a
    rocprofv3 --pmc run directory (csv output)."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    acc = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def ingest_pmc(config: str, fetch_dir: str, write_dir: str) -> int:
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the matmul kernel, each
    scaled by known bytes / counter of the copy-like calibration kernel that
    ran in the same process."""
    import workloads
    case = workloads.config_case(config)
    # the Y-output instantiation timed by the bench (MODE 0), not the int32-C
    # one that the |O| probe before the timed region runs
    kname = "k_gemm_decode" if case.M <= 16 else "k_gemm_prefill"
    kpat = re.compile(r"k_gemm_decode<\d+, 0, \d+>" if case.M <= 16 else r"k_gemm_prefill<0>")
    fetch = _pmc_means(fetch_dir, "FETCH_SIZE")
    write = _pmc_means(write_dir, "WRITE_SIZE")

    def pick(d, tag):
        if tag == COPY_KERNEL_TAG:
            keys = [k for k in d if tag in k]
        else:
            keys = [k for k in d if kpat.search(k)]
        if not keys:
            raise SystemExit(f"no kernel matching {tag!r} in {sorted(d)}")
        return max(keys, key=lambda k: d[k]) if tag == COPY_KERNEL_TAG else keys[0]

    kf, kw = pick(fetch, kname), pick(write, kname)
    cf, cw = pick(fetch, COPY_KERNEL_TAG), pick(write, COPY_KERNEL_TAG)
    f_scale = COPY_CAL_BYTES / (fetch[cf] * 1024.0)
    w_scale = COPY_CAL_BYTES / (write[cw] * 1024.0)
    rd = fetch[kf] * 1024.0 * f_scale
    wr = write[kw] * 1024.0 * w_scale
    path = os.path.join(PROFILES, "traffic.json")
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data[config] = {
        "kernel": kname,
        "kernel_source_hash": kernel_source_hash(),
        "fetch_kib_per_dispatch": round(fetch[kf], 1),
        "write_kib_per_dispatch": round(write[kw], 1),
        "copy_fetch_kib": round(fetch[cf], 1),
        "copy_write_kib": round(write[cw], 1),
        "copy_bytes": COPY_CAL_BYTES,
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "hbm_read_bytes_per_launch": round(rd),
        "hbm_write_bytes_per_launch": round(wr),
        "hbm_bytes_per_launch": round(rd + wr),
    }
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(data[config]))
    return 0


def _blas_info():
    """BLAS threads in use and the BLAS build numpy links."""
    import numpy as np
    threads, build = os.cpu_count() or 1, "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        if info:
            threads = max(i.get("num_threads", 1) for i in info)
            build = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in info)
    except Exception:  # pragma: no cover
        pass
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        build = f"{blas.get('name')} {blas.get('version')} ({build})"
    except Exception:  # pragma: no cover
        pass
    return int(threads), build


def _time_oracle(X, Wq, s, threshold, n_max, budget_s):
    import numpy as np
    from oracle import int8mm_ref as ref
    ref.int8_matmul_ref(X, Wq, s, threshold)  # warm-up
    times = []
    t_start = time.perf_counter()
    while len(times) < n_max and (time.perf_counter() - t_start) < budget_s:
        t0 = time.perf_counter()
        ref.int8_matmul_ref(X, Wq, s, threshold)
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), len(times)


def cpu_baseline(case, threshold: float, single_cases=(), budget_s: float = 15.0):
    """The oracle, as it stands, on this host: one warm-up call then timed
    calls until about `budget_s` seconds (at most 3, median).  The headline
    workload is sampled by rows with all BLAS threads (the unit is work per
    second, so it scales); `single_cases` ((name, case) pairs, whole) are
    timed with one BLAS thread."""
    from oracle import int8mm_ref as ref
    threads, build = _blas_info()
    M = case.M
    rows = M if M * case.K * case.N <= 4096 * 5120 * 13824 // 4 else M // 8
    X = case.X[:rows]
    Wq, s = ref.prepare_weight_ref(case.W)
    med, n = _time_oracle(X, Wq, s, threshold, 3, budget_s)
    out = {
        "value": 2.0 * rows * case.N * case.K / med / 1e12,
        "unit": "TOPS",
        "cores": int(threads),
        "host_cpus": os.cpu_count(),
        "blas": build,
        "kind": "oracle",
        "sample": f"{rows} of {M} rows x K={case.K} x N={case.N}, threshold {threshold}; "
                  f"median of {n} timed calls after 1 warm-up ({med:.3f} s each); "
                  f"{threads} BLAS threads",
        "single_thread": {},
    }
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    for name, c in single_cases:
        Wq1, s1 = ref.prepare_weight_ref(c.W)
        if threadpool_limits is not None:
            with threadpool_limits(limits=1):
                med1, n1 = _time_oracle(c.X, Wq1, s1, c.threshold, 3, budget_s)
        else:  # pragma: no cover
            med1, n1 = _time_oracle(c.X, Wq1, s1, c.threshold, 3, budget_s)
        out["single_thread"][name] = {
            "value": 2.0 * c.M * c.N * c.K / med1 / 1e12, "unit": "TOPS", "cores": 1,
            "seconds_per_call": round(med1, 4),
            "sample": f"whole workload {c.M}x{c.K}x{c.N}, median of {n1} timed calls after 1 warm-up"}
    return out


# Prepared weight bytes every workload cycles through: three times the 256 MB
# MALL, so that each call reads its weight from HBM.
ROTATE_BYTES = 3 * 256 * 2 ** 20
MAX_COPIES = 64


def measure(mm, lib, ev, dev, case, t, steps, warmup, rotate=None, others=False,
            copy_calibration=False):
    """One workload: weight preparation, warm-up, the timed region of
    `steps` whole calls, then the kernel-stamped and per-call passes.
    Returns the measurement as a dict."""
    import numpy as np
    import torch

    M, K, N = case.M, case.K, case.N
    X = torch.from_numpy(case.X).to(dev)
    W = torch.from_numpy(case.W).to(dev)
    ldk = mm.int8_weight_ld(K)
    wq_bytes = mm.int8_weight_bytes(N, K)
    n_copies = rotate if rotate else max(1, -(-ROTATE_BYTES // wq_bytes))
    n_copies = min(n_copies, MAX_COPIES)
    p0, p1 = ev.create(), ev.create()
    stream = torch.cuda.current_stream(dev).cuda_stream
    ev.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    ev.hip.hipEventRecord(p0, stream)
    Wq, s = mm.int8_prepare_weight(W)
    ev.hip.hipEventRecord(p1, stream)
    prepare_ms = ev.elapsed_ms(p0, p1)
    # steady-state rate of the one-time weight quantization (the first call
    # above includes the first launch of the kernel): 10 more calls into a
    # second buffer, HBM bytes = W read + Wq written + scales written
    Wq2, s2 = torch.empty_like(Wq), torch.empty_like(s)
    ev.hip.hipEventRecord(p0, stream)
    for _ in range(10):
        mm.int8_prepare_weight(W, out=(Wq2, s2))
    ev.hip.hipEventRecord(p1, stream)
    prep_rep_ms = ev.elapsed_ms(p0, p1) / 10
    if not (torch.equal(Wq2, Wq) and torch.equal(s2, s)):
        raise RuntimeError("int8_prepare_weight is not deterministic")
    del Wq2, s2
    prep_bytes = N * K * 2 + Wq.numel() + N * 4
    prepare = {"first_call_ms": round(prepare_ms, 4), "ms": round(prep_rep_ms, 4),
               "bytes": prep_bytes, "GB/s": round(prep_bytes / (prep_rep_ms * 1e-3) / 1e9, 1),
               "peak_GB/s": PEAK_HBM_GBS,
               "frac": round(prep_bytes / (prep_rep_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
               "timing": "HIP events around 10 back-to-back calls after the first"}
    weights = [(Wq, s)] + [(Wq.clone(), s.clone()) for _ in range(n_copies - 1)]
    del W
    Y = torch.empty((M, N), dtype=torch.float16, device=dev)
    ws = mm.workspace_for(M, K, N, dev)
    nO_probe = mm.int8_matmul_stages(X, Wq, s, threshold=t, want_c=True)["n_outliers"]
    n_out = int(nO_probe.item())
    del nO_probe
    torch.cuda.synchronize()

    fn = lib.int8_matmul
    fn_prof = lib.int8_matmul_profiled
    ws_ptr, ws_bytes = ws.data_ptr(), ws.numel()
    args_w = [(w.data_ptr(), sc.data_ptr()) for (w, sc) in weights]
    xp, yp = X.data_ptr(), Y.data_ptr()

    def step(i):
        wp, sp = args_w[i % len(args_w)]
        st = fn(xp, M, K, wp, sp, N, float(t), yp, ws_ptr, ws_bytes, stream)
        if st != 0:
            raise mm.Int8mmError("int8_matmul", st)

    def step_prof(i, e0, e1):
        wp, sp = args_w[i % len(args_w)]
        st = fn_prof(xp, M, K, wp, sp, N, float(t), yp, ws_ptr, ws_bytes, stream, e0, e1)
        if st != 0:
            raise mm.Int8mmError("int8_matmul_profiled", st)

    # W untimed warm-up calls, continued (untimed) until the warm-up has
    # lasted WARMUP_MIN_S: the GPU's clocks need several milliseconds of
    # sustained work to settle, and the rate reported is the steady one
    w0 = time.perf_counter()
    n_warm = 0
    while n_warm < warmup or time.perf_counter() - w0 < WARMUP_MIN_S:
        step(n_warm)
        n_warm += 1
        if n_warm >= warmup and n_warm % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    # timed region: K plain calls
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps

    # the same K calls again through int8_matmul_profiled: the matmul kernel's
    # dispatch stamps a pair of HIP events per call (kept out of the timed
    # region above, since the event packets add time between launches)
    evs = [(ev.create(), ev.create()) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step_prof(i, *evs[i])
    torch.cuda.synchronize()
    kern_ms = [ev.elapsed_ms(a, b) for (a, b) in evs]
    kern_avg = float(np.mean(kern_ms))
    # and once more with a HIP event pair around each whole call, for the
    # per-call median and minimum (the events add gaps: not the timed value)
    torch.cuda.synchronize()
    for i in range(steps):
        ev.hip.hipEventRecord(evs[i][0], stream)
        step(i)
        ev.hip.hipEventRecord(evs[i][1], stream)
    torch.cuda.synchronize()
    call_ms = [ev.elapsed_ms(a, b) for (a, b) in evs]
    for a, b in evs:
        ev.destroy(a)
        ev.destroy(b)
    per_call = {"call_ms_median": round(float(np.median(call_ms)), 5),
                "call_ms_min": round(float(np.min(call_ms)), 5),
                "kernel_ms_median": round(float(np.median(kern_ms)), 5),
                "kernel_ms_min": round(float(np.min(kern_ms)), 5),
                "timing": f"HIP events per call over {steps} calls after the timed region"}
    ev.destroy(p0)
    ev.destroy(p1)
    if not torch.isfinite(Y).all().item():
        raise RuntimeError("non-finite output")
    if copy_calibration:
        src = torch.ones(COPY_CAL_BYTES // 2, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    res = {}
    if others:
        # the other entry points on the same workload, after the timed region:
        # the layer forward with a bias (int8_linear) in rounds interleaved
        # with int8_matmul (so that both see the same clock), and the column
        # maxima (int8_column_absmax)
        bias = (torch.arange(N, device=dev, dtype=torch.float32) % 7 - 3).to(torch.float16) / 8
        lin, cmx = lib.int8_linear, lib.int8_column_absmax
        cm = torch.empty((K,), dtype=torch.float16, device=dev)

        def step_lin(i):
            wp, sp = args_w[i % len(args_w)]
            st = lin(xp, M, K, wp, sp, N, bias.data_ptr(), float(t), yp, ws_ptr, ws_bytes, stream)
            if st != 0:
                raise mm.Int8mmError("int8_linear", st)

        def step_cmx(i):
            st = cmx(xp, M, K, cm.data_ptr(), ws_ptr, ws_bytes, stream)
            if st != 0:
                raise mm.Int8mmError("int8_column_absmax", st)

        def timed(f, n):
            torch.cuda.synchronize()
            a = time.perf_counter()
            for i in range(n):
                f(i)
            torch.cuda.synchronize()
            return (time.perf_counter() - a) * 1e3 / n

        n_round = max(1, min(steps, 20))
        mm_ms, lin_ms = [], []
        for _ in range(4):
            mm_ms.append(timed(step, n_round))
            lin_ms.append(timed(step_lin, n_round))
        colmax_ms = timed(step_cmx, steps)
        res["other_entry_points"] = {
            "int8_linear_ms": round(float(np.median(lin_ms)), 5),
            "int8_matmul_ms_same_rounds": round(float(np.median(mm_ms)), 5),
            "int8_column_absmax_ms": round(colmax_ms, 5),
            "column_absmax_GB/s": round(M * K * 2 / (colmax_ms * 1e-3) / 1e9, 1),
            "timing": (f"wall clock; int8_linear (with a bias) and int8_matmul in 4 interleaved "
                       f"rounds of {n_round} calls (medians), int8_column_absmax over "
                       f"{steps} calls; all after the timed region")}

    ops = 2.0 * M * N * K
    value = ops / (ms_per_step * 1e-3) / 1e12
    decode = M <= mm.INT8MM_DECODE_MAX_M
    src_hash = kernel_source_hash()
    if decode:
        # matmul kernel algorithmic bytes: Wq + a_w + Xq + a_x + Y
        alg_bytes = N * K + 4 * N + M * K + 4 * M + 2 * M * N
        achieved = alg_bytes / (kern_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "algorithmic_bytes_per_launch": alg_bytes}
        call_gbs = alg_bytes / (ms_per_step * 1e-3) / 1e9
        res["whole_call_hbm"] = {"GB/s": round(call_gbs, 1), "frac": round(call_gbs / PEAK_HBM_GBS, 4)}
    else:
        achieved = ops / (kern_avg * 1e-3) / 1e12
        peak = PEAK_FP16_TOPS if n_out == K else PEAK_INT8_TOPS
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "algorithmic_ops_per_launch": ops}
    # the committed counters were taken at the workload's own threshold (another
    # threshold changes |O| and, past three fp16 steps, the kernel's branch)
    roof["traffic"] = committed_traffic(case.name, src_hash) if t == case.threshold else None
    roof["kernel"] = "k_gemm_decode" if decode else "k_gemm_prefill"
    roof["kernel_ms"] = round(kern_avg, 5)
    roof["kernel_timing"] = (f"HIP events stamped by the {roof['kernel']} dispatch, mean of {steps} "
                             "calls run right after the timed region")
    res.update({
        "value": round(value, 2),
        "unit": "TOPS",
        "ms_per_step": round(ms_per_step, 5),
        "warmup_calls_run": n_warm,
        "config": {"workload": WORKLOAD_TEXT.get(case.name, case.name), "name": case.name,
                   "M": M, "K": K, "N": N, "threshold": t, "n_outliers": n_out,
                   "weight_copies": n_copies,
                   "weight_bytes_rotated": n_copies * wq_bytes,
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "per_call": per_call,
        "prepare_weight_ms": round(prepare_ms, 4),
        "prepare_weight": prepare,
    })
    del weights, X, Y, ws
    torch.cuda.empty_cache()
    return res


PROBE_LIB = os.path.join(ROOT, "int8_quantized_matmul_col_amd", "libint8mm_ceilings.so")


def measure_ceilings(torch, dev) -> dict:
    """The practical ceilings on this GPU (after the timed regions): the int8
    MFMA issue rate on random and on zero operands, and the HBM read rate of a
    contiguous-chunk stream over 2 GiB (beyond the 256 MB MALL)."""
    if not os.path.exists(PROBE_LIB):
        raise SystemExit(f"{PROBE_LIB} missing: run __graft_entry__.build()")
    pl = ctypes.CDLL(PROBE_LIB)
    pl.int8mm_probe_mfma_i8.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)]
    pl.int8mm_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)]
    g = torch.Generator().manual_seed(7)
    rnd = torch.randint(-128, 128, (65536,), dtype=torch.int8, generator=g).to(dev)
    zero = torch.zeros(65536, dtype=torch.int8, device=dev)
    blocks = 256 * 4  # four workgroups of 4 waves per CU: 4 waves per SIMD
    out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    res = {}
    for name, src in (("random", rnd), ("zero", zero)):
        v = ctypes.c_double()
        st = pl.int8mm_probe_mfma_i8(ctypes.c_void_p(src.data_ptr()), blocks, 2000,
                                     ctypes.c_void_p(out.data_ptr()), ctypes.byref(v))
        if st != 0:
            raise SystemExit(f"MFMA probe failed: HIP error {st}")
        res[f"mfma_i8_{name}_operands_TOPS"] = round(v.value / 1e12, 1)
    rb = 2 << 30
    buf = torch.ones(rb // 4, dtype=torch.int32, device=dev)
    rblocks = 2048
    rout = torch.empty(rblocks * 256, dtype=torch.int32, device=dev)
    v = ctypes.c_double()
    st = pl.int8mm_probe_read(ctypes.c_void_p(buf.data_ptr()), rb, rblocks,
                              ctypes.c_void_p(rout.data_ptr()), ctypes.byref(v))
    if st != 0:
        raise SystemExit(f"read probe failed: HIP error {st}")
    res["hbm_read_GB/s"] = round(v.value / 1e9, 1)
    del buf
    # the same stream over four rotating copies of 224 MiB (the decode
    # weight's size), one per launch, back to back: the rate a decode-sized
    # read reaches with its launch ramp and tail
    pl.int8mm_probe_read_copies.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_void_p,
                                            ctypes.POINTER(ctypes.c_double)]
    cb, copies = 224 << 20, 4
    buf = torch.ones(cb * copies // 4, dtype=torch.int32, device=dev)
    best = 0.0
    for nb in (256, 512):
        v = ctypes.c_double()
        st = pl.int8mm_probe_read_copies(ctypes.c_void_p(buf.data_ptr()), cb, copies, nb,
                                         ctypes.c_void_p(rout.data_ptr()), ctypes.byref(v))
        if st != 0:
            raise SystemExit(f"read probe failed: HIP error {st}")
        best = max(best, v.value)
    res["hbm_read_224MiB_GB/s"] = round(best / 1e9, 1)
    res["method"] = ("int8mm_probe_mfma_i8: 4 waves per SIMD, 16 independent "
                     "v_mfma_i32_32x32x32_i8 accumulators each, 2000 iterations; "
                     "int8mm_probe_read: 2048 workgroups, each a contiguous chunk of 2 GiB, "
                     "8 x 16-byte loads per lane in flight; int8mm_probe_read_copies: the same "
                     "kernel over 4 rotating 224 MiB copies (the decode weight's size), one per "
                     "launch, 256 or 512 workgroups, the better (libint8mm_ceilings.so)")
    del buf
    torch.cuda.empty_cache()
    return res


def frac_of_ceiling(roof: dict, ceil: dict):
    if roof["unit"] == "GB/s":
        return round(roof["achieved"] / ceil["hbm_read_GB/s"], 4)
    if roof["peak"] >= 4999.0:  # int8 MFMA peak: against the random-operand rate
        return round(roof["achieved"] / ceil["mfma_i8_random_operands_TOPS"], 4)
    return None


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="sweep13b")
    ap.add_argument("--extra", default="q_proj,decode1,decode4,decode16",
                    help="workloads measured after the headline in the same run ('none': only "
                         "the headline)")
    ap.add_argument("--threshold", type=float, default=None)
    ap.add_argument("--rotate", type=int, default=None,
                    help="weight copies cycled through (default: at least 768 MiB of weights, "
                         "so that every call reads its weight from HBM)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the MFMA / HBM ceiling probes run after the timed regions")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a copy-like elementwise kernel (torch.neg) over "
                         f"{COPY_CAL_BYTES >> 20} MiB so HBM counters can be scaled to known bytes")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="CPU only: read two rocprofv3 --pmc runs of this script (FETCH_SIZE, then "
                         "WRITE_SIZE, both with --copy-calibration and --extra none) and record "
                         "the matmul kernel's HBM bytes per launch in profiles/traffic.json")
    args = ap.parse_args()
    if args.ingest_pmc:
        return ingest_pmc(args.config, *args.ingest_pmc)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import int8_quantized_matmul_col_amd as mm
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = mm.load()
    ev = HipEvents()

    case = workloads.config_case(args.config)
    t = case.threshold if args.threshold is None else args.threshold
    log(f"[bench] {args.config}: M={case.M} K={case.K} N={case.N} t={t}")
    head = measure(mm, lib, ev, dev, case, t, args.steps, args.warmup, args.rotate, others=True,
                   copy_calibration=args.copy_calibration)
    log(f"[bench] {args.config}: {head['ms_per_step']} ms per call, kernel "
        f"{head['roofline']['kernel_ms']} ms, frac {head['roofline']['frac']}")

    extra = {}
    cases = {args.config: case}
    names = [] if args.extra in ("", "none") else [n for n in args.extra.split(",") if n]
    for name in names:
        if name == args.config:
            continue
        c = cases[name] = workloads.config_case(name)
        log(f"[bench] extra {name}: M={c.M} K={c.K} N={c.N} t={c.threshold}")
        r = measure(mm, lib, ev, dev, c, c.threshold, args.steps, args.warmup, args.rotate)
        r["metric"] = METRIC
        extra[name] = r
        log(f"[bench] {name}: {r['ms_per_step']} ms per call, kernel {r['roofline']['kernel_ms']} ms, "
            f"frac {r['roofline']['frac']}")

    ceilings = None
    if not args.no_ceilings:
        log("[bench] measuring the MFMA and HBM ceilings ...")
        ceilings = measure_ceilings(torch, dev)
        for roof in [head["roofline"]] + [r["roofline"] for r in extra.values()]:
            roof["frac_of_measured_ceiling"] = frac_of_ceiling(roof, ceilings)
            if roof["unit"] == "GB/s":
                # against a stream of the decode weight's size (ramp and tail included)
                roof["frac_of_224MiB_read"] = round(
                    roof["achieved"] / ceilings["hbm_read_224MiB_GB/s"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        singles = []
        for name in ("tiny", "decode16"):
            singles.append((name, cases.get(name) or workloads.config_case(name)))
        cpu = cpu_baseline(case, t, singles)

    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_calls_run": head["warmup_calls_run"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded N(0,1) activations with planted outlier columns, N(0,0.02) weights)",
        "config": head["config"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "per_call": head["per_call"],
        "prepare_weight_ms": head["prepare_weight_ms"],
        "prepare_weight": head["prepare_weight"],
        "other_entry_points": head.get("other_entry_points"),
        "extra": extra,
        "ceilings": ceilings,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
