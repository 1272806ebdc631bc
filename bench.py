"""Benchmark of the decomposed int8 matmul on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config q_proj] [--threshold T]

One step = one whole int8_matmul call (activation pass: outlier detection,
row quantization and compaction; int8 MFMA GEMM; fp16 outlier MFMA; fused
dequant epilogue) on inputs already resident in HBM.  The weight is
prepared once before timing (int8_prepare_weight; its time is reported
separately).  Prints one JSON line.

* value     -- effective TOPS = 2*M*N*K / (wall time of K steps / K).
* roofline  -- the matmul kernel alone: algorithmic work per launch divided by
               its average duration, read from HIP events recorded on the
               launch stream around every timed launch.  Prefill shapes are
               bound by the int8 MFMA peak (5.0 POP/s dense), decode shapes
               by HBM (8 TB/s); traffic comes from the committed rocprofv3
               FETCH_SIZE / WRITE_SIZE counters when they match the current
               kernel sources, else null.
* cpu_baseline -- the CPU oracle (oracle/, unchanged) timed on this host on
               the same workload (or a row sample of it for the largest
               ones), in the same unit.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TOPS of decomposed int8 matmul; % int8 MFMA peak / % HBM BW"
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


def cpu_baseline(case, threshold: float, budget_s: float = 20.0):
    """The oracle, as it stands, on this host: one warm-up call then timed
    calls until about `budget_s` seconds (at most 5).  Very large workloads
    are sampled by rows (the unit is work per second, so it scales)."""
    import numpy as np
    from oracle import int8mm_ref as ref
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    M = case.M
    rows = M if M * case.K * case.N <= 4096 * 5120 * 13824 // 2 else M // 4
    X = case.X[:rows]
    Wq, s = ref.prepare_weight_ref(case.W)
    ref.int8_matmul_ref(X, Wq, s, threshold)  # warm-up
    times = []
    t_start = time.perf_counter()
    while len(times) < 5 and (time.perf_counter() - t_start) < budget_s:
        t0 = time.perf_counter()
        ref.int8_matmul_ref(X, Wq, s, threshold)
        times.append(time.perf_counter() - t0)
    med = float(np.median(times))
    return {
        "value": 2.0 * rows * case.N * case.K / med / 1e12,
        "unit": "TOPS",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{rows} of {M} rows x K={case.K} x N={case.N}, threshold {threshold}; "
                  f"median of {len(times)} timed calls after 1 warm-up ({med:.3f} s each); "
                  f"numpy/OpenBLAS with {threads} threads",
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="q_proj")
    ap.add_argument("--threshold", type=float, default=None)
    ap.add_argument("--rotate", type=int, default=None,
                    help="weight copies cycled through (default: enough to exceed the 256 MB MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import int8_quantized_matmul_col_amd as mm
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = mm.load()

    case = workloads.config_case(args.config)
    t = case.threshold if args.threshold is None else args.threshold
    M, K, N = case.M, case.K, case.N
    log(f"[bench] {args.config}: M={M} K={K} N={N} t={t}")

    X = torch.from_numpy(case.X).to(dev)
    W = torch.from_numpy(case.W).to(dev)
    ldk = mm.int8_weight_ld(K)
    wq_bytes = N * ldk
    n_copies = args.rotate if args.rotate else max(1, -(-3 * 256 * 2 ** 20 // wq_bytes))
    n_copies = min(n_copies, 8)
    ev = HipEvents()
    p0, p1 = ev.create(), ev.create()
    stream = torch.cuda.current_stream(dev).cuda_stream
    ev.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    ev.hip.hipEventRecord(p0, stream)
    Wq, s = mm.int8_prepare_weight(W)
    ev.hip.hipEventRecord(p1, stream)
    prepare_ms = ev.elapsed_ms(p0, p1)
    weights = [(Wq, s)] + [(Wq.clone(), s.clone()) for _ in range(n_copies - 1)]
    del W
    Y = torch.empty((M, N), dtype=torch.float16, device=dev)
    ws = mm.workspace_for(M, K, N, dev)
    nO_probe = mm.int8_matmul_stages(X, Wq, s, threshold=t, want_c=True)["n_outliers"]
    n_out = int(nO_probe.item())
    del nO_probe
    torch.cuda.synchronize()

    fn = lib.int8_matmul_profiled
    ws_ptr, ws_bytes = ws.data_ptr(), ws.numel()
    args_w = [(w.data_ptr(), sc.data_ptr()) for (w, sc) in weights]
    xp, yp = X.data_ptr(), Y.data_ptr()

    def step(i, e0, e1):
        wp, sp = args_w[i % len(args_w)]
        st = fn(xp, M, K, wp, sp, N, float(t), yp, ws_ptr, ws_bytes, stream, e0, e1)
        if st != 0:
            raise mm.Int8mmError("int8_matmul_profiled", st)

    for i in range(args.warmup):
        step(i, None, None)
    torch.cuda.synchronize()

    evs = [(ev.create(), ev.create()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, *evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kern_ms = [ev.elapsed_ms(a, b) for (a, b) in evs]
    kern_avg = float(np.mean(kern_ms))
    for a, b in evs:
        ev.destroy(a)
        ev.destroy(b)
    ev.destroy(p0)
    ev.destroy(p1)
    assert torch.isfinite(Y).all().item() or args.config == "tiny", "non-finite output"

    ops = 2.0 * M * N * K
    value = ops / (ms_per_step * 1e-3) / 1e12
    decode = M <= mm.INT8MM_DECODE_MAX_M
    src_hash = kernel_source_hash()
    if decode:
        # matmul kernel algorithmic bytes: Wq + a_w + Xq + a_x + Y
        alg_bytes = N * K + 4 * N + M * K + 4 * M + 2 * M * N
        achieved = alg_bytes / (kern_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = ops / (kern_avg * 1e-3) / 1e12
        peak = PEAK_FP16_TOPS if n_out == K else PEAK_INT8_TOPS
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    roof["traffic"] = committed_traffic(args.config, src_hash)
    roof["kernel"] = "k_gemm_decode" if decode else "k_gemm_prefill"
    roof["kernel_ms"] = round(kern_avg, 5)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        cpu = cpu_baseline(case, t)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded N(0,1) activations with planted outlier columns, N(0,0.02) weights)",
        "config": {"workload": WORKLOAD_TEXT.get(args.config, args.config), "name": args.config,
                   "M": M, "K": K, "N": N, "threshold": t, "n_outliers": n_out,
                   "weight_copies": n_copies, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "prepare_weight_ms": round(prepare_ms, 4),
        "kernel_source_hash": src_hash,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
