#!/usr/bin/env python3
"""Attn-QAT forward + backward throughput on one MI355X.

One step is the whole hot path on one batch of synthetic input already resident
in HBM: attnqat_fwd (operand fake-quant, statistics pass, quantized-P output
pass) followed by attnqat_bwd (operand preparation, rowsum(dO*O) preprocess,
dK/dV kernel, dQ kernel). The default workload is the kernel-timing shape of
the FastVideo kernel commit message: 6 heads x 31,200 tokens, head dim 128,
B = 1, NVFP4 fake quantization of Q, K, V and P.

Throughput is credited FLOPs (4 Nq Nk D B H forward, 2.5x that backward) per
second. The JSON line also carries the roofline of the dominant kernel (its
algorithmic FLOPs per launch over its mean launch time, timed with HIP events on
the kernel's stream inside the timed region) and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense BF16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_FP4_TFLOPS = 10100.0  # dense FP4 MFMA peak of MI355X
METRIC = "Attn-QAT fwd+bwd ms & TFLOP/s (% BF16 MFMA peak), H=6 N=31200 d=128"

# Algorithmic FLOPs per (query, key) pair and head dimension unit, per kernel:
# products the method needs at least once. fwd_out: S and P V (4 d);
# bwd_dkdv: S, dV, dP, dK (8 d); bwd_dq: dQ only (2 d), its S and dP are
# recomputation; fwd_lse: none (it recomputes S for the statistics). EXEC
# counts the products each kernel runs.
ALGO_PER_PAIR = {"fwd_out": 4, "bwd_dkdv": 8, "bwd_dq": 2, "fwd_lse": 0}
EXEC_PER_PAIR = {"fwd_out": 4, "bwd_dkdv": 8, "bwd_dq": 6, "fwd_lse": 2}
# Algorithmic HBM bytes per launch of the memory-bound kernels (square
# problems): fake quantization and the transposed copies read and write each
# bf16 element once (4 B); the preprocess reads O and dO and writes D (4 d + 4
# B per query row).
ALGO_BYTES = {
    "fq_axis_d": lambda bh, n, d: 4 * bh * n * d,
    "fq_axis_n": lambda bh, n, d: 4 * bh * n * d,
    "transpose_perm": lambda bh, n, d: 4 * bh * n * d,
    "bwd_pre": lambda bh, n, d: (4 * d + 4) * bh * n,
}


PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash():
    """Hash of the kernel and library sources, to tie counter summaries to the
    code they were taken from."""
    d = os.path.join(ROOT, "quantization_aware_attention_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h", ".cpp")):
            h.update(name.encode())
            with open(os.path.join(d, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, quant, kernel, src_hash):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE/WRITE_SIZE
    summary of this workload, or None when there is none or the sources have
    changed since the counters were taken."""
    path = os.path.join(PROFILES, f"attn_step_{workload}_hbm_bytes.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = [json.loads(line[6:]) for line in f if line.startswith("json: ")]
    if not rec:
        return None
    rec = rec[-1]
    if rec.get("kernel_source_sha256_16") != src_hash or rec.get("quant") != quant:
        return None
    return rec.get("bytes_per_launch", {}).get(kernel)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3,
                    help="synthetic workload id (see synthetic.WORKLOADS)")
    ap.add_argument("--quant", default="qkvp", help="quantized operands, e.g. qkvp or none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sparse", action="store_true",
                    help="skip the block-sparse VSA step at its own configuration")
    ap.add_argument("--main-only", action="store_true",
                    help="time the metric's step only (no standalone kernels, variants, other "
                         "workloads, probes or CPU oracle)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the timing of the other workloads (tiny, DiT, tail)")
    ap.add_argument("--cpu-rows", type=int, default=8192,
                    help="query rows of head 0 in the CPU-oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run one plain 1 GiB device copy (a kernel "
                         "of known traffic for scaling HBM byte counters)")
    ap.add_argument("--power", action="store_true",
                    help="after the timed steps, sample board power and shader clocks "
                         "(amd-smi) while the MFMA probe, the forward and the backward each "
                         "run in a loop (about 20 s)")
    return ap.parse_args()


def cpu_baseline(bits, w, rows, mask):
    """Time the fp64 oracle on the sub-problem: `rows` query rows of head 0
    against all keys, forward and backward."""
    import numpy as np
    from oracle import attention as oatt
    from synthetic import f32_from_bf16_bits
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    q = f32_from_bf16_bits(bits["q"][0, 0, :rows]).astype(np.float64)
    k = f32_from_bf16_bits(bits["k"][0, 0]).astype(np.float64)
    v = f32_from_bf16_bits(bits["v"][0, 0]).astype(np.float64)
    do = f32_from_bf16_bits(bits["do"][0, 0, :rows]).astype(np.float64)
    t0 = time.perf_counter()
    qq, kq, vq = oatt.quantize_operands(q, k, v, mask)
    O, L = oatt.head_forward(qq, kq, vq, w.sm_scale, mask)
    oatt.head_backward(qq, kq, vq, do, O, L, w.sm_scale, mask)
    dt = time.perf_counter() - t0
    flops = 4.0 * rows * w.N * w.D * 3.5
    full_flops = sum(w.credited_flops())
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"fwd+bwd of {rows} query rows of head 0 against all {w.N} keys "
                      f"(credited {flops / 1e9:.1f} GFLOP), fp64 numpy oracle",
            "extrapolated_full_workload_s": round(dt * full_flops / flops, 1),
            "extrapolation": "linear in query rows and heads (rows are independent)",
            "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(),
            "blas_threads": int(threads)}


def _cpu_model():
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:  # pragma: no cover
        pass
    return None


def machine_probes(torch, dev):
    """Dense BF16 MFMA rate and shader clock under that load (probe kernel),
    and the bandwidth of a plain 1 GiB device copy after a cache flush."""
    import ctypes
    from quantization_aware_attention_amd.build import PROBE_PATH
    out = {}
    if os.path.exists(PROBE_PATH):
        lib = ctypes.CDLL(PROBE_PATH)
        fn = lib.aq_probe_mfma_peak
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                       ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                       ctypes.c_void_p]
        blocks = 1024  # four workgroups of four waves per CU: four waves per SIMD
        sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
        stamps = torch.zeros(4, dtype=torch.int64, device=dev)
        tf, mhz = ctypes.c_double(), ctypes.c_double()
        best = (0.0, 0.0)
        # about a second of warm-up calls first: the shader clock takes a
        # while to settle (2.2 GHz in the first calls, 2.4 GHz after)
        t_warm = time.perf_counter()
        while time.perf_counter() - t_warm < 1.0:
            fn(blocks, 20000, sink.data_ptr(), stamps.data_ptr(), ctypes.byref(tf),
               ctypes.byref(mhz), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        for it in (50000, 50000, 50000):
            rc = fn(blocks, it, sink.data_ptr(), stamps.data_ptr(), ctypes.byref(tf),
                    ctypes.byref(mhz), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc == 0 and tf.value > best[0]:
                best = (tf.value, mhz.value)
        out["mfma_bf16_tflops_measured"] = round(best[0], 1)
        out["clock_mhz_under_mfma"] = round(best[1], 0)
        del sink, stamps
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    times = []
    for i in range(4):
        flush.fill_(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = float(sorted(times[1:])[1])
    out["hbm_copy_gbs"] = round(2.0 * (1 << 30) / (ms * 1e-3) / 1e9, 1)
    out["hbm_copy_note"] = "1 GiB device-to-device copy (read + write bytes) after a 1 GiB flush"
    del flush, src, dst
    return out


def time_configs(qaa, torch, np, dev, skip):
    from synthetic import WORKLOADS, make_inputs
    res = {}
    for cid, masks in ((1, (15,)), (2, (15,)), (4, (15, 0))):
        if cid == skip:
            continue
        w = WORKLOADS[cid]
        bits = make_inputs(cid)
        t = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(dev)
             for k, v in bits.items()}
        del bits
        o, lse = torch.empty_like(t["q"]), torch.empty(w.shape[:3], dtype=torch.float32, device=dev)
        g = [torch.empty_like(t["q"]) for _ in range(3)]
        f_fwd, f_bwd = w.credited_flops()
        for mask in masks:
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(10)]
            for i in range(13):
                e = ev[i - 3] if i >= 3 else None
                if e:
                    e[0].record()
                qaa.fwd(t["q"], t["k"], t["v"], w.sm_scale, mask, out=o, lse=lse)
                if e:
                    e[1].record()
                qaa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], w.sm_scale, mask,
                        dq=g[0], dk=g[1], dv=g[2])
                if e:
                    e[2].record()
            torch.cuda.synchronize()
            fm = float(np.median([a.elapsed_time(b) for a, b, _ in ev]))
            bm = float(np.median([b.elapsed_time(c) for _, b, c in ev]))
            tf_f, tf_b = f_fwd / (fm * 1e-3) / 1e12, f_bwd / (bm * 1e-3) / 1e12
            tf = (f_fwd + f_bwd) / ((fm + bm) * 1e-3) / 1e12
            res[f"{w.name}/{'qkvp' if mask == 15 else 'none'}"] = {
                "shape": list(w.shape), "steps": 10, "stat": "median",
                "fwd_ms": round(fm, 4), "bwd_ms": round(bm, 4), "ms_per_step": round(fm + bm, 4),
                "fwd_tflops": round(tf_f, 1), "bwd_tflops": round(tf_b, 1),
                "tflops": round(tf, 1), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        del t, o, lse, g
        torch.cuda.empty_cache()
    return res


def copy_calibration(torch, dev):
    """One plain 1 GiB device-to-device copy, a kernel of known traffic (1 GiB
    read, 1 GiB written) against which HBM byte counters are scaled."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    return 1 << 30


def device_info(torch):
    """Name, architecture, compute units and the HIP runtime of device 0."""
    prop = torch.cuda.get_device_properties(0)
    return {"name": torch.cuda.get_device_name(0) or None,
            "arch": getattr(prop, "gcnArchName", None),
            "compute_units": prop.multi_processor_count,
            "memory_gib": round(prop.total_memory / 2 ** 30, 1),
            "hip_runtime": torch.version.hip}


def board_power(torch, phases, secs=5.0):
    """Board power and shader clocks read with amd-smi about every 0.5 s while
    each phase (name, callable) runs in a loop on a second thread, after 1.5 s
    of warm-up."""
    import re
    import shutil
    import subprocess
    import threading
    smi = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"

    def read():
        r = subprocess.run([smi, "metric", "-p", "-c", "--json"], capture_output=True,
                           text=True, timeout=30)
        if r.returncode != 0:
            return [], []
        pw = re.findall(r'"socket_power":\s*\{\s*"value":\s*(\d+)', r.stdout)
        ck = re.findall(r'"gfx_\d+":\s*\{\s*"clk":\s*\{\s*"value":\s*(\d+)', r.stdout)
        return [int(x) for x in pw], [int(x) for x in ck]

    pw0, _ = read()
    out = {"tool": "amd-smi metric -p -c", "idle_socket_power_w": pw0[0] if pw0 else None}
    for name, fn in phases:
        stop = threading.Event()

        def loop():
            while not stop.is_set():
                fn()
                torch.cuda.synchronize()

        th = threading.Thread(target=loop)
        th.start()
        time.sleep(1.5)
        pws, cks = [], []
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < secs:
            a, b = read()
            pws += a
            cks += b
            time.sleep(0.5)
        stop.set()
        th.join()
        out[name] = {"samples": len(pws),
                     "socket_power_w": [min(pws), max(pws)] if pws else None,
                     "gfx_clock_mhz_mean": round(sum(cks) / len(cks)) if cks else None,
                     "gfx_clock_mhz_range": [min(cks), max(cks)] if cks else None}
        print(f"[bench] power {name}: {out[name]}", file=sys.stderr, flush=True)
    return out


def mfma_probe_fn(torch, dev):
    """One call of the MFMA-only probe kernel (about 2.7e12 FLOPs), or None."""
    import ctypes
    from quantization_aware_attention_amd.build import PROBE_PATH
    if not os.path.exists(PROBE_PATH):
        return None
    lib = ctypes.CDLL(PROBE_PATH)
    fn = lib.aq_probe_mfma_peak
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                   ctypes.c_void_p]
    sink = torch.empty(1024 * 256, dtype=torch.float32, device=dev)
    stamps = torch.zeros(4, dtype=torch.int64, device=dev)
    tf, mhz = ctypes.c_double(), ctypes.c_double()

    def run():
        fn(1024, 10000, sink.data_ptr(), stamps.data_ptr(), ctypes.byref(tf), ctypes.byref(mhz),
           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return run


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the Attn-QAT "
                                   "kernel is measured at one GPU's share of the workload; "
                                   "multi-GPU runs are not supported", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import quantization_aware_attention_amd as qaa
    from synthetic import WORKLOADS, make_inputs, sha256_hex

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    qaa.load()
    w = WORKLOADS[args.workload]
    mask = qaa.parse_mask(args.quant) if args.quant != "none" else 0
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    bits = make_inputs(args.workload)
    hashes = {k: sha256_hex(v)[:16] for k, v in bits.items()}
    t = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(dev) for k, v in bits.items()}
    print(f"[bench] inputs {w.name} {w.shape} generated in {time.perf_counter() - t_gen:.1f}s",
          file=sys.stderr, flush=True)
    kv_idx = None
    if w.topk:
        kv_idx = qaa.block_select(t["q"], t["k"], w.topk, w.block_tokens)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    B, H, N, D = w.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    p = qaa.make_problem(q, k, w.sm_scale, mask, v=v, o=o, do=do, dq=dq, dk=dk, dv=dv,
                         kv_block_idx=kv_idx)
    import ctypes
    L = qaa.lib()
    ws_f = torch.empty(L.attnqat_fwd_workspace_bytes(ctypes.byref(p)), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(L.attnqat_bwd_workspace_bytes(ctypes.byref(p)), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev:
            ev[0].record()
        qaa.fwd(q, k, v, w.sm_scale, mask, kv_idx, out=o, lse=lse, workspace=ws_f,
                validate_index=False)
        if ev:
            ev[1].record()
        qaa.bwd(q, k, v, o, lse, do, w.sm_scale, mask, kv_idx, dq=dq, dk=dk, dv=dv, workspace=ws_b,
                validate_index=False)
        if ev:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    qaa.profile_enable(True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = qaa.profile_read()
    qaa.profile_enable(False)
    fwd_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in evs]))
    bwd_ms = float(np.mean([b.elapsed_time(c) for _, b, c in evs]))
    ms_step = wall * 1e3 / args.steps
    f_fwd, f_bwd = w.credited_flops()
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12

    pairs = float(B * H) * N * N * ((w.topk / (-(-N // w.block_tokens))) if w.topk else 1.0)
    kernels = {}
    for name, (tot, cnt) in kern.items():
        avg = tot / cnt
        e = {"ms_per_launch": round(avg, 4), "launches_per_step": cnt / args.steps,
             "ms_per_step": round(tot / args.steps, 4)}
        if name in ALGO_BYTES:
            nbytes = ALGO_BYTES[name](B * H, N, D)
            e["algo_gbs"] = round(nbytes / (avg * 1e-3) / 1e9, 1)
        if name in EXEC_PER_PAIR:
            e["exec_tflops"] = round(EXEC_PER_PAIR[name] * pairs * D / (avg * 1e-3) / 1e12, 1)
            e["algo_tflops"] = round(ALGO_PER_PAIR[name] * pairs * D / (avg * 1e-3) / 1e12, 1)
        kernels[name] = e
    dom = max(kern.items(), key=lambda kv: kv[1][0])[0]
    dom_avg = kern[dom][0] / kern[dom][1]
    src_hash = kernel_source_hash()
    traffic = measured_traffic(w.name, args.quant, dom, src_hash)
    if dom in ALGO_PER_PAIR:
        achieved = ALGO_PER_PAIR[dom] * pairs * D / (dom_avg * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "ms_per_launch": round(dom_avg, 4),
                "algo_flops_per_launch": ALGO_PER_PAIR[dom] * pairs * D}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": None, "traffic": traffic, "ms_per_launch": round(dom_avg, 4)}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "D": D,
                   "quant": args.quant, "sm_scale": w.sm_scale,
                   "topk": w.topk or None},
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 1),
        "bwd_tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 1),
        "frac_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roof, "kernels": kernels, "input_sha256_16": hashes,
        "kernel_source_sha256_16": src_hash,
        "device": device_info(torch),
    }
    # Standalone fake quantization of one input (HBM-bound): 4 bytes per
    # element (2 read, 2 written), along d (Q's layout) and along tokens (V's).
    if args.power:
        def fwd_only():
            qaa.fwd(q, k, v, w.sm_scale, mask, kv_idx, out=o, lse=lse, workspace=ws_f,
                    validate_index=False)

        def bwd_only():
            qaa.bwd(q, k, v, o, lse, do, w.sm_scale, mask, kv_idx, dq=dq, dk=dk, dv=dv,
                    workspace=ws_b, validate_index=False)
        probe = mfma_probe_fn(torch, dev)
        phases = ([("mfma_probe", probe)] if probe else []) + [("forward", fwd_only),
                                                               ("backward", bwd_only)]
        out["board_power"] = board_power(torch, phases)
    if args.main_only:
        if args.copy_calibration:
            out["copy_calibration_bytes"] = copy_calibration(torch, dev)
        out["cpu_baseline"] = None
        print(json.dumps(out), flush=True)
        return
    # Machine probes first: the MFMA-only rate and clock, and the copy rate.
    out["machine"] = machine_probes(torch, dev)
    # Every launch below follows a 1 GiB fill of a scratch buffer (outside the
    # timed events), which evicts the 256 MB last-level cache and the L2s, so
    # the GB/s are HBM figures, not cache figures.
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    fq_out = torch.empty_like(q)
    fq = {}
    for axis, x in (("d", q), ("n", v)):
        for _ in range(2):
            qaa.fakequant(x, axis, out=fq_out)
        torch.cuda.synchronize()
        qaa.profile_enable(True)
        for i in range(20):
            flush.fill_(i)
            qaa.fakequant(x, axis, out=fq_out)
        torch.cuda.synchronize()
        (tot, cnt), = qaa.profile_read().values()
        qaa.profile_enable(False)
        ms = tot / cnt
        gbs = 4.0 * x.numel() / (ms * 1e-3) / 1e9
        fq[f"axis_{axis}"] = {"ms_per_launch": round(ms, 4), "algo_gbs": round(gbs, 1),
                              "frac_hbm": round(gbs / PEAK_HBM_GBS, 3), "cache": "flushed"}
    out["fakequant_standalone"] = fq
    # The backward preprocess (Dl = rowsum(dO * O)), timed inside whole
    # backward calls that each follow a flush: its O and dO are not resident.
    qaa.profile_enable(True)
    for i in range(10):
        flush.fill_(i)
        qaa.bwd(q, k, v, o, lse, do, w.sm_scale, mask, kv_idx, dq=dq, dk=dk, dv=dv,
                workspace=ws_b, validate_index=False)
    torch.cuda.synchronize()
    rec = qaa.profile_read()
    qaa.profile_enable(False)
    tot, cnt = rec["bwd_pre"]
    ms = tot / cnt
    gbs = ALGO_BYTES["bwd_pre"](B * H, N, D) / (ms * 1e-3) / 1e9
    out["bwd_pre_flushed"] = {"ms_per_launch": round(ms, 4), "algo_gbs": round(gbs, 1),
                              "frac_hbm": round(gbs / PEAK_HBM_GBS, 3)}
    # VSA coarse branch and gated combination on the same tensors (128-token
    # blocks): its kernels are passes over the token tensors, reported as
    # algorithmic GB/s (bf16 bytes each pass must move) next to HBM peak.
    gate = torch.randn_like(q)
    vq, vk, vv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    vo = torch.empty_like(o)
    for _ in range(2):
        qaa.vsa_fwd(q, k, v, gate, o, w.sm_scale, out=vo)
        qaa.vsa_bwd(q, k, v, gate, do, vq, vk, vv, w.sm_scale)
    torch.cuda.synchronize()
    qaa.profile_enable(True)
    for i in range(10):
        flush.fill_(i)
        qaa.vsa_fwd(q, k, v, gate, o, w.sm_scale, out=vo)
        flush.fill_(i + 1)
        qaa.vsa_bwd(q, k, v, gate, do, vq, vk, vv, w.sm_scale)
    torch.cuda.synchronize()
    rec = qaa.profile_read()
    qaa.profile_enable(False)
    tok = 2.0 * B * H * D  # bytes per token row of one bf16 tensor
    vbytes = {"vsa_pool": tok * 3 * N, "vsa_combine": tok * 3 * N, "vsa_gate_reduce": tok * 3 * N,
              "vsa_grad_add": tok * 6 * N}
    vs = {}
    for name, (tot, cnt) in rec.items():
        ms = tot / cnt
        e = {"ms_per_launch": round(ms, 4), "launches_per_step": cnt / 10}
        if name in vbytes:
            e["algo_gbs"] = round(vbytes[name] / (ms * 1e-3) / 1e9, 1)
            e["frac_hbm"] = round(e["algo_gbs"] / PEAK_HBM_GBS, 3)
        vs[name] = e
    out["vsa_coarse"] = {"kernels": vs, "cache": "flushed before each call",
                         "ms_per_step": round(sum(v["ms_per_launch"] * v["launches_per_step"]
                                                  for v in vs.values()), 4)}
    del gate, vq, vk, vv, vo, flush
    # Real-FP4 inference forward (MXFP4 operands on the scaled FP4 matrix
    # instruction) on the same inputs: 4 B H N^2 D credited FLOPs per forward,
    # against the dense FP4 peak.
    mo = torch.empty_like(q)
    ml = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    for _ in range(2):
        qaa.mxfp4_fwd(q, k, v, w.sm_scale, out=mo, lse=ml)
    torch.cuda.synchronize()
    qaa.profile_enable(True)
    for _ in range(5):
        qaa.mxfp4_fwd(q, k, v, w.sm_scale, out=mo, lse=ml)
    torch.cuda.synchronize()
    rec = qaa.profile_read()
    qaa.profile_enable(False)
    mk = {name: round(tot / cnt, 4) for name, (tot, cnt) in rec.items()}
    mfwd = sum(mk.values())
    mflops = 4.0 * B * H * N * N * D
    # The kernel is bound by vector work, not by the FP4 matrix rate. Its
    # compiled loops issue, per 32 scores of a lane, ~26 instructions in pass
    # 1 (maxima) and in pass 2 104 full-rate ones (FMA, add for l, maxima,
    # addresses), 32 exponentials (two issue slots each) and 16 FP4
    # conversions (~2.5 slots): ~7.3 slots of a 64-lane instruction per
    # score, each 4 cycles on one of the 1,024 SIMDs, at the clock the MFMA
    # probe measures (or 2.4 GHz). That floor is reported beside the time.
    clk = (out.get("machine") or {}).get("clock_mhz_under_mfma") or 2400.0
    valu_ms = B * H * N * N * 7.3 / 64 * 4 / 1024 / (clk * 1e6) * 1e3
    out["mxfp4_infer"] = {
        "kernels_ms": mk, "fwd_ms": round(mfwd, 4),
        "tflops": round(mflops / (mfwd * 1e-3) / 1e12, 1),
        "frac_fp4_peak": round(mflops / (mfwd * 1e-3) / 1e12 / PEAK_FP4_TFLOPS, 4),
        "valu_floor_ms": round(valu_ms, 3),
        "frac_valu_floor": round(valu_ms / mk.get("mx_fwd", mfwd), 3)}
    del mo, ml
    # Variants of the P quantizer on the same inputs, reported beside the
    # metric (which is the normalised reading with the plain STE) and credited
    # the same FLOPs: the row-max-relative P and the additive straight-through
    # output O_ste = P Vq, which the backward then takes as its o.
    if mask & qaa.QUANT_P:
        rm = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        os_ = torch.empty_like(o)
        variants = {}

        def time_variant(name, fwd_kw, bwd_o, bwd_kw):
            pr = qaa.make_problem(q, k, w.sm_scale, mask, v=v, o=o, do=do, dq=dq, dk=dk, dv=dv,
                                  kv_block_idx=kv_idx, **bwd_kw)
            ws_bv = torch.empty(L.attnqat_bwd_workspace_bytes(ctypes.byref(pr)),
                                dtype=torch.uint8, device=dev)

            def step(ev=None):
                if ev:
                    ev[0].record()
                qaa.fwd(q, k, v, w.sm_scale, mask, kv_idx, out=o, lse=lse, workspace=ws_f,
                        **fwd_kw)
                if ev:
                    ev[1].record()
                qaa.bwd(q, k, v, bwd_o, lse, do, w.sm_scale, mask, kv_idx, dq=dq, dk=dk, dv=dv,
                        workspace=ws_bv, **bwd_kw)
                if ev:
                    ev[2].record()

            for _ in range(2):
                step()
            nv = max(1, min(args.steps, 5))
            evv = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nv)]
            torch.cuda.synchronize()
            for i in range(nv):
                step(evv[i])
            torch.cuda.synchronize()
            vf = float(np.mean([a.elapsed_time(b) for a, b, _ in evv]))
            vb = float(np.mean([b.elapsed_time(c) for _, b, c in evv]))
            tf = (f_fwd + f_bwd) / ((vf + vb) * 1e-3) / 1e12
            variants[name] = {"steps": nv, "fwd_ms": round(vf, 4), "bwd_ms": round(vb, 4),
                              "ms_per_step": round(vf + vb, 4), "tflops": round(tf, 1),
                              "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
            del ws_bv

        rmk = dict(p_mode=qaa.P_ROWMAX, row_max=rm)
        time_variant("p_rowmax", rmk, o, rmk)
        time_variant("ste_delta", dict(o_ste=os_), os_, {})
        out["variants"] = variants
        del rm, os_
    # The block-sparse VSA step at its own configuration (12 heads x 32,768
    # tokens, 256 blocks of 128 tokens, top-26 key blocks per query block):
    # coarse selection, quantized fine branch and gated coarse branch, forward
    # and backward; credited FLOPs are the dense ones scaled by the density.
    if not args.no_sparse and args.workload != 5:
        w5 = WORKLOADS[5]
        b5 = make_inputs(5)
        t5 = {k_: torch.from_numpy(v_.view(np.int16)).view(torch.bfloat16).to(dev) for k_, v_ in b5.items()}
        del b5
        g5 = torch.randn_like(t5["q"])
        o5f, o5 = torch.empty_like(t5["q"]), torch.empty_like(t5["q"])
        l5 = torch.empty(w5.shape[:3], dtype=torch.float32, device=dev)
        d5 = [torch.empty_like(t5["q"]) for _ in range(3)]
        ev5 = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(5)]
        for i in range(7):
            e = ev5[i - 2] if i >= 2 else None
            if e:
                e[0].record()
            idx5 = qaa.block_select(t5["q"], t5["k"], w5.topk, w5.block_tokens)
            if e:
                e[1].record()
            qaa.fwd(t5["q"], t5["k"], t5["v"], w5.sm_scale, mask, idx5, out=o5f, lse=l5,
                    validate_index=False)
            qaa.vsa_fwd(t5["q"], t5["k"], t5["v"], g5, o5f, w5.sm_scale, out=o5)
            if e:
                e[2].record()
            qaa.bwd(t5["q"], t5["k"], t5["v"], o5f, l5, t5["do"], w5.sm_scale, mask, idx5,
                    dq=d5[0], dk=d5[1], dv=d5[2], validate_index=False)
            qaa.vsa_bwd(t5["q"], t5["k"], t5["v"], g5, t5["do"], d5[0], d5[1], d5[2], w5.sm_scale)
            if e:
                e[3].record()
        torch.cuda.synchronize()
        sel = float(np.mean([a_.elapsed_time(b_) for a_, b_, _, _ in ev5]))
        f5 = float(np.mean([b_.elapsed_time(c_) for _, b_, c_, _ in ev5]))
        bw5 = float(np.mean([c_.elapsed_time(d_) for _, _, c_, d_ in ev5]))
        cf, cb = w5.credited_flops()
        out["sparse_vsa"] = {
            "workload": w5.name, "shape": list(w5.shape), "topk": w5.topk, "steps": 5,
            "select_ms": round(sel, 4), "fwd_ms": round(f5, 4), "bwd_ms": round(bw5, 4),
            "ms_per_step": round(sel + f5 + bw5, 4),
            "credited_tflops": round((cf + cb) / ((sel + f5 + bw5) * 1e-3) / 1e12, 1)}
        del t5, g5, o5f, o5, l5, d5
    # Quantization off on the same inputs (plain attention; the forward is the
    # single-pass kernel), credited the same FLOPs.
    if mask:
        pr0 = qaa.make_problem(q, k, w.sm_scale, 0, v=v, o=o, do=do, dq=dq, dk=dk, dv=dv,
                               kv_block_idx=kv_idx)
        ws0 = torch.empty(L.attnqat_bwd_workspace_bytes(ctypes.byref(pr0)), dtype=torch.uint8,
                          device=dev)
        ev0 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(5)]
        for i in range(7):
            e = ev0[i - 2] if i >= 2 else None
            if e:
                e[0].record()
            qaa.fwd(q, k, v, w.sm_scale, 0, kv_idx, out=o, lse=lse, workspace=ws_f)
            if e:
                e[1].record()
            qaa.bwd(q, k, v, o, lse, do, w.sm_scale, 0, kv_idx, dq=dq, dk=dk, dv=dv, workspace=ws0)
            if e:
                e[2].record()
        torch.cuda.synchronize()
        vf = float(np.mean([a_.elapsed_time(b_) for a_, b_, _ in ev0]))
        vb = float(np.mean([b_.elapsed_time(c_) for _, b_, c_ in ev0]))
        tf = (f_fwd + f_bwd) / ((vf + vb) * 1e-3) / 1e12
        out.setdefault("variants", {})["quant_off"] = {
            "steps": 5, "fwd_ms": round(vf, 4), "bwd_ms": round(vb, 4),
            "ms_per_step": round(vf + vb, 4), "tflops": round(tf, 1),
            "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        del ws0
    # The other workloads, each on its own synthetic inputs (the DiT layer of
    # 12 heads x 25,088 tokens, the 16,411-token tail case with every quantizer
    # on and off, and the tiny case): forward and backward ms, credited
    # TFLOP/s and the fraction of the BF16 peak.
    if not args.no_configs:
        del ws_f, ws_b
        out["configs"] = time_configs(qaa, torch, np, dev, args.workload)
    if args.copy_calibration:
        out["copy_calibration_bytes"] = copy_calibration(torch, dev)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(bits, w, args.cpu_rows, mask)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
