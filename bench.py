#!/usr/bin/env python3
"""Throughput of FlashJoLT compression on one MI355X: compressed KV tokens per second.

Workload (LLaMA-3.1-8B-shaped long context): 32 layers in groups of 4, 8 KV heads, d_head 128,
T = 65536 prefill tokens, fp16 K and V, FlashJoLT (oversample 10, one power iteration, q_cap by
Eq. (5) = 512), token ranks 8..512 and feature ranks 8..128 in steps of 8, residual bits
{0, 2, 4, 8}, one byte budget for all 16 cells (default 2x).  Synthetic power-law cache
(spectral exponent 1 for K, 0.5 for V, N(0, 0.02) noise, 4 outlier key channels), generated on
the GPU before timing.  One step = one jolt_compress call over the whole cache: spectra, the
allocation table and bisection, the fit and the rotated residual.  value = T / (seconds per step).

The JSON line also carries the roofline of the dominant kernel, measured live with the library's
HIP-event stage profiler on its own stream, and the CPU oracle timed on a bounded sample.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--ratio", type=float, default=2.0)
    ap.add_argument("--tokens", type=int, default=65536)
    ap.add_argument("--cpu-tokens", type=int, default=16384, help="tokens of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dtype", default="f16", choices=["f16", "bf16"])
    ap.add_argument("--compare-modes", nargs="?", const="mistral7b", choices=["mistral7b", "llama2_13b"],
                    help="report FlashJoLT against exact JoLT on the Mistral-7B-shaped cache (T = 1024, the "
                         "default) or the LLaMA-2-13B-shaped one (T = 4096): compression time and relative "
                         "reconstruction error of K and V at 2x and 3x")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the HBM byte counters)")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="print a per-kernel summary of a rocprofv3 --kernel-trace --output-format csv directory")
    ap.add_argument("--traffic-from", nargs=5, metavar=("KERNEL", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="KERNEL: project_gemm, residual_encode or reconstruct (with '@tag' for another workload); then "
                         "rocprofv3 --pmc csv directories (FETCH_SIZE / WRITE_SIZE of this bench and of "
                         "--calibrate-copy): add the kernel to profiles/traffic.json and print a summary")
    return ap.parse_args()


# HIP-event records per stage cover this many kernel launches (K and V cells in separate launches)
LAUNCHES_PER_RECORD = {"sketch_gemm": 2, "project_gemm": 2, "feature_gram": 2}

# the dominant kernel of the workload: the projection P^T = Q^T X (fp32 Q in two fp16 planes
# times the fp16 cache read token-major), one launch over the 8 K cells and one over the 8 V cells,
# each split 4-fold along K = T; the launch shape is set by the library's sequencing, hence api.cpp
# among the sources whose change invalidates the counters
# Kernels whose HBM traffic is read from rocprofv3 counters: the kernel, how to find its dispatches
# (its grid for the 8B shape, or the largest grid of that kernel) and the sources its code and launch
# come from (the counters stand only while these hash the same).
TRAFFIC_KERNELS = {
    "project_gemm": {"name": "gemm_dma_kernel<0, 2, 1, 3, 8, 3, 4, 2, false, false>", "grid": 3 * 16 * 512 * 8 * 4,
                     "sources": ["kv_cache_compression_layer_amd/csrc/gemm_dma.hip",
                                 "kv_cache_compression_layer_amd/csrc/gemm_core.hpp",
                                 "kv_cache_compression_layer_amd/csrc/dma.hpp",
                                 "kv_cache_compression_layer_amd/csrc/common.hpp",
                                 "kv_cache_compression_layer_amd/csrc/api.cpp"]},
    "residual_encode": {"name": "encode_dma_kernel<0, 8, 2, 2>", "grid": None,
                        "sources": ["kv_cache_compression_layer_amd/csrc/codec.hip",
                                    "kv_cache_compression_layer_amd/csrc/gemm_core.hpp",
                                    "kv_cache_compression_layer_amd/csrc/dma.hpp",
                                    "kv_cache_compression_layer_amd/csrc/common.hpp",
                                    "kv_cache_compression_layer_amd/csrc/api.cpp"]},
    # the whole-cache reconstruct (the largest grid of the kernel; the decode measurement launches it per group)
    "reconstruct": {"name": "decode_dma_kernel<0, 8>", "grid": None,
                    "sources": ["kv_cache_compression_layer_amd/csrc/codec.hip",
                                "kv_cache_compression_layer_amd/csrc/dma.hpp",
                                "kv_cache_compression_layer_amd/csrc/common.hpp",
                                "kv_cache_compression_layer_amd/csrc/api.cpp"]},
}


def _rows(d, fname):
    import csv
    with open(os.path.join(d, fname)) as f:
        return list(csv.DictReader(f))


def summarize_profile(d):
    """Per (kernel, grid) call count and durations from a kernel-trace csv directory."""
    import collections
    rows = _rows(d, "run_kernel_trace.csv")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    # each compress call starts by generating Omega: launches from the second call on are the steady
    # state (the first call's first launches pay one-time costs: code load, first touch of buffers)
    starts = [int(r["Start_Timestamp"]) for r in rows if "omega_kernel" in r["Kernel_Name"]]
    t_steady = starts[1] if len(starts) > 1 else 0
    agg = collections.defaultdict(list)
    steady = collections.defaultdict(list)
    other = [0.0, 0]
    for r in rows:
        ms = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
        if "jolt::" not in r["Kernel_Name"]:  # input generation and torch glue outside the library
            other[0] += ms
            other[1] += 1
            continue
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        agg[(r["Kernel_Name"], grid)].append(ms)
        if int(r["Start_Timestamp"]) >= t_steady:
            steady[(r["Kernel_Name"], grid)].append(ms)
    tot = sum(sum(v) for v in agg.values())
    out = ["library kernels: %.2f ms over %d dispatches (other kernels of the process: %.2f ms over %d)"
           % (tot, sum(len(v) for v in agg.values()), other[0], other[1]),
           "steady_avg_ms: launches from the second compress call on",
           "%9s %6s %10s %13s %10s %12s  %s" % ("total_ms", "calls", "avg_ms", "steady_avg_ms", "share", "grid_items",
                                               "kernel")]
    for (name, grid), v in sorted(agg.items(), key=lambda kv: -sum(kv[1]))[:30]:
        nm = name.replace("jolt::(anonymous namespace)::", "")
        nm = nm if len(nm) <= 90 else nm[:87] + "..."
        sv = steady.get((name, grid), [])
        sa = "%13.4f" % (sum(sv) / len(sv)) if sv else "%13s" % "-"
        out.append("%9.3f %6d %10.4f %s %9.1f%% %12d  %s" % (sum(v), len(v), sum(v) / len(v), sa, 100 * sum(v) / tot,
                                                              grid, nm))
    return "\n".join(out)


def traffic_from(key, fetch, write, cfetch, cwrite):
    """HBM bytes per launch of a kernel (key: a TRAFFIC_KERNELS stage, optionally '@<tag>' for another
    workload): FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for a plain copy of known size."""
    stage = key.split("@")[0]
    tk = TRAFFIC_KERNELS[stage]

    def counter(d, pick):
        vals = [float(r["Counter_Value"]) for r in _rows(d, "run_counter_collection.csv") if pick(r)]
        return sum(vals) / len(vals), len(vals)
    grid = tk["grid"]
    if grid is None:
        grid = max(int(r["Grid_Size"]) for r in _rows(fetch, "run_counter_collection.csv")
                   if tk["name"] in r["Kernel_Name"])
    is_k = lambda r: tk["name"] in r["Kernel_Name"] and int(r["Grid_Size"]) == grid
    is_copy = lambda r: "copyBuffer" in r["Kernel_Name"] or "copy" in r["Kernel_Name"].lower()
    f_kib, nf = counter(fetch, is_k)
    w_kib, nw = counter(write, is_k)
    cf_kib, _ = counter(cfetch, is_copy)
    cw_kib, _ = counter(cwrite, is_copy)
    fscale = COPY_BYTES / (cf_kib * 1024.0)
    wscale = COPY_BYTES / (cw_kib * 1024.0)
    bytes_per_launch = f_kib * 1024.0 * fscale + w_kib * 1024.0 * wscale
    ent = {"kernel": tk["name"], "grid_items": grid, "sources": tk["sources"],
           "source_hash": source_hash(tk["sources"]), "fetch_kib": f_kib, "write_kib": w_kib,
           "fetch_scale": fscale, "write_scale": wscale, "bytes_per_launch": bytes_per_launch,
           "dispatches": [nf, nw]}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    t = {}
    if os.path.exists(path):
        with open(path) as f:
            t = json.load(f)
    t[key] = ent
    with open(path, "w") as f:
        json.dump(t, f, indent=1)
    return ("kernel %s (grid %d work-items), %d/%d dispatches\n"
            "FETCH_SIZE %.0f KiB/dispatch x scale %.4f (copy of %d bytes read %.0f KiB)\n"
            "WRITE_SIZE %.0f KiB/dispatch x scale %.4f (copy of %d bytes wrote %.0f KiB)\n"
            "HBM bytes per launch: %.4g (read %.4g, write %.4g)"
            % (ent["kernel"], grid, nf, nw, f_kib, fscale, COPY_BYTES, cf_kib, w_kib, wscale, COPY_BYTES, cw_kib,
               bytes_per_launch, f_kib * 1024 * fscale, w_kib * 1024 * wscale))


COPY_BYTES = 1 << 30


def calibrate_copy():
    """Three launches of torch's elementwise copy over 1 GiB: the byte counters of a profiler read
    on this kernel give the scale between counter units and bytes moved."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}), flush=True)


FP64_PEAK_TFLOPS = 78.6


def stage_models(T, L, H, D, G, ell, picks, c):
    """Algorithmic flops and HBM bytes of every stage of one compress call over the whole cache
    (each operand read once, each output written once; split-precision planes and padding not
    counted), with the peak of the units the stage runs on: 'mfma' (fp16/bf16 matrix cores: the
    products of the sketch, projection, Gram and fit), 'fp64' (fp64 Gram, eigensolvers, Cholesky)."""
    GH, M, R = G * H, G * H * D, G * H * T
    n = 2 * (L // G)                        # cells
    kmax = max(p["rT"] for p in picks)      # the fit products run every cell at the largest pick
    kd = max(p["rd"] for p in picks)
    f4 = 4.0
    m = {}

    def add(name, flops, byts, unit):
        m[name] = {"flops": float(flops), "bytes": float(byts), "unit": unit}

    add("feature_gram", 2.0 * R * D * D * n, T * M * c * n, "mfma")
    # two sketches: Y = X Omega, Y = X Z (fp32 Y written in two layouts)
    add("sketch_gemm", 2 * 2.0 * T * M * ell * n, 2 * (T * M * c + 2 * f4 * T * ell + f4 * M * ell) * n, "mfma")
    # 16-bit planes of Q_0^T, Z^T and Y^T (fp32 read, two fp16 planes written)
    add("split_planes", 0.0, (2 * T * ell + M * ell) * 8.0 * n, "mfma")
    # two projections (P^T = Q_0^T X, P'^T = Y^T X; K split 4-fold, partials written)
    add("project_gemm", 2 * 2.0 * T * M * ell * n, 2 * (T * M * c + f4 * T * ell + 4 * f4 * ell * M) * n, "mfma")
    add("project_reduce", 0.0, 2 * (4 * f4 * ell * M + 2 * f4 * ell * M) * n, "mfma")
    # two tall Grams (T ell^2 each, symmetric), one apply Q_0^T = R^-T Y^T (T ell^2, triangular),
    # two Cholesky factorisations and triangular inverses (2 ell^3 / 3 each)
    add("cholqr_tall", (3.0 * T * ell * ell + 4.0 * ell ** 3 / 3) * n, (3 * f4 * T * ell + f4 * T * ell) * n, "mfma")
    add("cholqr_z", (2.0 * M * ell * ell + 2.0 * ell ** 3 / 3) * n, 3 * f4 * M * ell * n, "mfma")
    add("basis_apply", 1.0 * M * ell * ell * n, 2 * f4 * M * ell * n, "mfma")
    add("gram64", 1.0 * ell * ell * M * n, f4 * ell * M * n, "fp64")
    add("eigvals_B", (4.0 * ell ** 3 / 3) * n, 8.0 * ell * ell * n, "fp64")
    add("allocate", 0.0, 0.0, "fp64")
    # fit: eigenvectors, W~ = W R^-T, U_T^T = W~^T Y^T, Y_p = W~^T P'^T
    add("fit_token_factor", (2.0 * kmax * ell * ell + 2.0 * T * ell * kmax + 2.0 * kmax * ell * M) * n,
        (f4 * T * ell + f4 * kmax * T + f4 * ell * M + 2 * f4 * kmax * M) * n, "mfma")
    add("fit_feature_factor", 2.0 * kmax * GH * D * D * n, 2 * f4 * kmax * M * n, "mfma")
    add("fit_core", 2.0 * kmax * GH * D * kd * n, (f4 * kmax * M + f4 * GH * kmax * kd) * n, "mfma")
    add("put_factors", 0.0, sum((T * p["rT"] + D * p["rd"] + GH * p["rT"] * p["rd"]) * (f4 + c) for p in picks), "mfma")
    add("residual_operand", sum(2.0 * GH * D * p["rT"] * p["rd"] for p in picks), sum(8.0 * GH * D * (D + p["rT"]) for p in picks),
        "mfma")
    enc_f = sum(2.0 * R * (D + p["rT"]) * D for p in picks if p["bits"] > 0)
    enc_b = sum(R * D * c + T * p["rT"] * c + R * D * p["bits"] / 8.0 + f4 * R for p in picks if p["bits"] > 0)
    add("residual_encode", enc_f, enc_b, "mfma")
    return m


def stage_table(stages, models, dtype):
    """Per stage: time, algorithmic work, achieved rates and both roofline fractions; the binding
    roof is the one the stage's arithmetic intensity points to."""
    out = {}
    for name, (ms, cnt) in stages.items():
        mdl = models.get(name)
        if mdl is None:
            out[name] = {"ms": round(ms, 3), "records": cnt}
            continue
        s = ms / 1e3
        peak = MFMA_PEAK_TFLOPS[dtype] if mdl["unit"] == "mfma" else FP64_PEAK_TFLOPS
        tf = mdl["flops"] / s / 1e12 if s > 0 else 0.0
        gb = mdl["bytes"] / s / 1e9 if s > 0 else 0.0
        ridge = peak * 1e12 / (HBM_PEAK_GBS * 1e9)
        ai = mdl["flops"] / mdl["bytes"] if mdl["bytes"] > 0 else float("inf")
        out[name] = {"ms": round(ms, 3), "gflop": round(mdl["flops"] / 1e9, 2), "gbyte": round(mdl["bytes"] / 1e9, 3),
                     "tflops": round(tf, 2), "gbs": round(gb, 1), "flop_frac": round(tf / peak, 4),
                     "hbm_frac": round(gb / HBM_PEAK_GBS, 4), "peak_unit": mdl["unit"],
                     "bound": ("mfma" if mdl["unit"] == "mfma" else "fp64") if ai >= ridge else "hbm"}
    return out


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(stage):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel is unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            t = json.load(f)
        ent = t.get(stage)
        if not ent or ent.get("source_hash") != source_hash(ent["sources"]):
            return None
        return ent["bytes_per_launch"]
    except Exception:
        return None


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_info():
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
    except Exception:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(K, V, groups, cfgd, sample_T):
    """The oracle (numpy fp64, multithreaded BLAS) on the first layer group, first sample_T
    tokens; scaled to the full workload's tokens/s."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    G = groups[1] - groups[0]
    sub_k = K[:, :G, :, :sample_T].contiguous()
    sub_v = V[:, :G, :, :sample_T].contiguous()
    if sub_k.dtype.itemsize == 2 and str(sub_k.dtype) == "torch.bfloat16":
        kn, vn = sub_k.view(dtype=__import__("torch").uint16).cpu().numpy(), sub_v.view(dtype=__import__("torch").uint16).cpu().numpy()
    else:
        kn, vn = sub_k.cpu().numpy(), sub_v.cpu().numpy()
    eps2 = {int(b): float(v) for b, v in enumerate(cfgd["eps2"])}
    p = dict(mode="flash", oversample=10, power_iters=1, qcap=None, rT_grid=cfgd["rT"], rd_grid=cfgd["rd"],
             bits=cfgd["bits"], eps2=eps2, target_ratio=cfgd["ratio"])
    t0 = time.time()
    r = oracle.compress(kn, vn, [0, G], cfgd["dtype"], p)
    dt = time.time() - t0
    n_groups = len(groups) - 1
    value = sample_T / (dt * n_groups)
    host = {"nproc": os.cpu_count(), "cpu_model": _cpu_model(), "blas": _blas_info()}
    return {"value": value, "unit": "tokens/s", "cores": int(threads), "kind": "oracle", "host": host,
            "sample": f"oracle compress of layer group 0 (K and V cells) on the first {sample_T} tokens "
                      f"({dt:.1f} s); scaled as {sample_T} tokens / ({dt:.1f} s x {n_groups} groups); "
                      f"status {r['status']}"}


def compare_modes(shape="mistral7b"):
    """FlashJoLT against exact JoLT on one cache (the pages compare them at 1024-token context): per
    budget and mode, the time of one jolt_compress (median of 5 after a warm-up, HIP events) and the
    relative Frobenius error of the whole K and V caches after jolt_reconstruct.  Shapes: Mistral-7B
    (32 layers, 8 KV heads, T = 1024, bits {2, 4, 8}) or LLaMA-2-13B (40 layers, 40 KV heads, T = 4096,
    bits {1, 2, 3, 4}); FlashJoLT's token ranks run to q_cap of Eq. (5), exact ones to T."""
    import torch
    import synth
    from kv_cache_compression_layer_amd import jolt
    torch.cuda.set_device(0)
    if shape == "llama2_13b":
        L, H, T, D, G, bits = 40, 40, 4096, 128, 4, [1, 2, 3, 4]
        title = "LLaMA-2-13B-shaped KV cache, 40 layers (groups of 4) x 40 KV heads x T=4096"
    else:
        L, H, T, D, G, bits = 32, 8, 1024, 128, 4, [2, 4, 8]
        title = "Mistral-7B-shaped KV cache, 32 layers (groups of 4) x 8 KV heads x T=1024"
    groups = list(range(0, L + 1, G))
    K, V = synth.power_law(n_seq=1, L=L, H=H, T=T, D=D, group=G, alpha_k=1.0, alpha_v=1.0, noise_var=0.02,
                           n_outliers=4, dtype="f16", seed=0, device="cuda")
    e = jolt.eps2(D)
    eps2 = {b: float(e[b]) for b in range(9)}
    rows = {}
    for C in (2.0, 3.0):
        for mode, name in ((jolt.EXACT, "exact"), (jolt.FLASH, "flash")):
            probe = jolt.Config(1, L, H, T, D, jolt.F16, groups, jolt.FLASH, [8], [8], bits, C)
            q = probe.token_spectrum_len() - 1
            rT = list(range(8, (T if mode == jolt.EXACT else q) + 1, 8))
            cfg = jolt.Config(1, L, H, T, D, jolt.F16, groups, mode, rT, list(range(8, D + 1, 8)), bits, C,
                              eps2=eps2)
            ws = torch.empty(cfg.workspace_bytes(), dtype=torch.uint8, device="cuda")
            out = torch.empty(cfg.output_bytes(), dtype=torch.uint8, device="cuda")
            jolt.compress(K, V, cfg, out=out, ws=ws)
            torch.cuda.synchronize()
            times = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                blob, picks, lam = jolt.compress(K, V, cfg, out=out, ws=ws)
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            Ko, Vo = torch.empty_like(K), torch.empty_like(V)
            jolt.reconstruct(blob, cfg, picks, Ko, Vo, ws=ws)
            torch.cuda.synchronize()
            err = [float(torch.linalg.vector_norm((O.float() - X.float())) / torch.linalg.vector_norm(X.float()))
                   for O, X in ((Ko, K), (Vo, V))]
            rows[f"{name}_{C:g}x"] = {"ms": round(sorted(times)[2], 3), "err_K": round(err[0], 5),
                                      "err_V": round(err[1], 5),
                                      "token_ranks_K": [p["rT"] for p in picks[0::2]],
                                      "token_ranks_V": [p["rT"] for p in picks[1::2]]}
            del ws, out, Ko, Vo
    for C in ("2x", "3x"):
        ex, fl = rows[f"exact_{C}"], rows[f"flash_{C}"]
        rows[f"gap_{C}"] = {"dK": round(fl["err_K"] - ex["err_K"], 5), "dV": round(fl["err_V"] - ex["err_V"], 5),
                            "time_ratio_exact_over_flash": round(ex["ms"] / fl["ms"], 3)}
    print(json.dumps({"workload": title + " x d_head 128, f16, synthetic (power law, exponent 1)", "modes": rows}),
          flush=True)


def decode_measure(jolt, torch, blob, cfg, picks, T, L, H, D, G, dt, reps=20):
    """One decode step of one layer (32 query heads over 8 KV heads, RoPE base 500000): the fused
    attention over the compressed cells (jolt_decode_attention on a prepared layer state; also with
    the per-layer preparation in every call) against reconstruct-then-attend (jolt_reconstruct of the layer's group, its share per
    layer, then RoPE on the dense keys and scaled dot-product attention in torch).  Memory: the layer's
    compressed bytes plus the fused path's workspace against the dense K and V the other path holds."""
    import math
    st = torch.cuda.current_stream()
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    nq = 4 * H
    rope = jolt.rope_table(D, 500000.0, T)
    g = torch.Generator(device="cuda").manual_seed(0)
    q = torch.randn(nq, D, device="cuda", generator=g) * 0.5
    out = torch.empty(nq, D, device="cuda")
    res = {}
    for layer in (0, L - 1):
        gi = layer // G
        gp = [picks[2 * gi], picks[2 * gi + 1]]
        nb = jolt.load().jolt_decode_attention_workspace_bytes(ctypes.byref(cfg.desc), jolt._picks_array(picks), 0,
                                                               layer, nq)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        jolt.decode_attention(blob, cfg, picks, 0, layer, q, rope=rope, out=out, ws=ws)
        torch.cuda.synchronize()
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(st)
        for _ in range(reps):
            jolt.decode_attention(blob, cfg, picks, 0, layer, q, rope=rope, out=out, ws=ws)
        e1.record(st)
        for _ in range(reps):
            jolt.decode_attention(blob, cfg, picks, 0, layer, q, rope=rope, out=out, ws=ws, reuse_prepared=True)
        e2.record(st)
        torch.cuda.synchronize()
        fused_prep = e0.elapsed_time(e1) / reps
        fused = e1.elapsed_time(e2) / reps
        # reconstruct-then-attend: the group's cells decoded densely, then one layer attended
        gcfg = jolt.Config(1, G, H, T, D, cfg.desc.dtype, [0, G], jolt.FLASH, [8], [8], [2], 2.0)
        Kg = torch.empty(1, G, H, T, D, dtype=tdt, device="cuda")
        Vg = torch.empty_like(Kg)
        gws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")  # the two cells' backbone slices
        jolt.reconstruct(blob, gcfg, gp, Kg, Vg, ws=gws)
        # position-only RoPE factors in the cache dtype (a serving loop keeps them): k cos + rot(k) sin
        cos2 = torch.cat([rope[..., 0], rope[..., 0]], dim=-1).to(tdt)
        sin2 = torch.cat([-rope[..., 1], rope[..., 1]], dim=-1).to(tdt)
        qt = q.to(tdt).view(H, nq // H, D).transpose(1, 2).contiguous()  # [H][D][G]
        scale = 1.0 / math.sqrt(D)

        def attend():
            # decode attention on the dense layer: RoPE on the keys, scores by batched products over the
            # KV heads (grouped queries side by side), softmax over tokens in fp32, weighted values
            Kl, Vl = Kg[0, layer - gi * G], Vg[0, layer - gi * G]
            Kr = torch.addcmul(Kl * cos2, Kl.roll(D // 2, dims=-1), sin2)
            s = torch.bmm(Kr, qt)                                            # [H][T][G]
            p = torch.softmax(s.float() * scale, dim=1).to(tdt).transpose(1, 2).contiguous()
            return torch.bmm(p, Vl)                                          # [H][G][D]
        attend()
        torch.cuda.synchronize()
        r0, r1, r2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        r0.record(st)
        for _ in range(reps):
            jolt.reconstruct(blob, gcfg, gp, Kg, Vg, ws=gws)
        r1.record(st)
        for _ in range(reps):
            attend()
        r2.record(st)
        torch.cuda.synchronize()
        rec_g = r0.elapsed_time(r1) / reps
        att = r1.elapsed_time(r2) / reps
        dense_layer = 2 * H * T * D * 2
        comp_layer = (gp[0]["bytes"] + gp[1]["bytes"]) / G
        res[f"layer{layer}"] = {
            "picks_kv": [[p["rT"], p["rd"], p["bits"]] for p in gp],
            "fused_ms": round(fused, 4),
            "fused_with_prepare_ms": round(fused_prep, 4),
            "reconstruct_group_ms": round(rec_g, 4),
            "reconstruct_then_attend_ms": round(rec_g / G + att, 4),
            "attend_dense_ms": round(att, 4),
            "fused_vs_reconstruct_then_attend": round(fused / (rec_g / G + att), 3),
            "kv_bytes_dense": dense_layer,
            "kv_bytes_fused": int(comp_layer + nb),
            "memory_ratio": round(dense_layer / (comp_layer + nb), 3),
        }
        del Kg, Vg, gws, ws
    return res


def main():
    a = parse()
    if a.compare_modes:
        compare_modes(a.compare_modes)
        return
    if a.calibrate_copy:
        calibrate_copy()
        return
    if a.summarize_profile:
        print(summarize_profile(a.summarize_profile))
        return
    if a.traffic_from:
        print(traffic_from(*a.traffic_from))
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (the path shards by cell "
              f"across GPUs by design, but only the one-GPU kernel is built and measured)", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    from kv_cache_compression_layer_amd import jolt

    torch.cuda.set_device(0)
    T, L, H, D, G = a.tokens, 32, 8, 128, 4
    groups = list(range(0, L + 1, G))
    dt = {"f16": jolt.F16, "bf16": jolt.BF16}[a.dtype]
    t0 = time.time()
    K, V = synth.power_law(n_seq=1, L=L, H=H, T=T, D=D, group=G, alpha_k=1.0, alpha_v=0.5, noise_var=0.02,
                           n_outliers=4, dtype=a.dtype, seed=0, device="cuda")
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    rd = list(range(8, D + 1, 8))
    bits = [2, 4, 8]
    eps2 = jolt.eps2(D)
    # token ranks 8 .. q_cap (Eq. (5): 512 at 2x and T = 65536)
    probe = jolt.Config(1, L, H, T, D, dt, groups, jolt.FLASH, [8], rd, bits, a.ratio)
    qcap = probe.token_spectrum_len() - 1
    rT = list(range(8, qcap + 1, 8))
    cfg = jolt.Config(1, L, H, T, D, dt, groups, jolt.FLASH, rT, rd, bits, a.ratio, oversample=10, power_iters=1,
                      eps2={b: eps2[b] for b in range(9)})
    ws = torch.empty(cfg.workspace_bytes(), dtype=torch.uint8, device="cuda")
    out = torch.empty(cfg.output_bytes(), dtype=torch.uint8, device="cuda")
    for _ in range(a.warmup):
        blob, picks, lam = jolt.compress(K, V, cfg, out=out, ws=ws)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.time()
    e0.record(st)
    for _ in range(a.steps):
        blob, picks, lam = jolt.compress(K, V, cfg, out=out, ws=ws)
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.time() - w0
    ms_step = e0.elapsed_time(e1) / a.steps
    value = T / (ms_step / 1e3)

    # live per-stage timing (HIP events on the library's stream), one extra call
    jolt.profile(True)
    jolt.compress(K, V, cfg, out=out, ws=ws)
    torch.cuda.synchronize()
    stages = jolt.profile_read()
    jolt.profile(False)
    ell = min(qcap + 10, T, G * H * D)
    models = stage_models(T, L, H, D, G, ell, picks, 2)
    table = stage_table(stages, models, a.dtype)
    # The dominant kernel: the stage with the largest time.  Its rate is its algorithmic work over its
    # summed launch time (HIP events on the library's stream); per-launch time = that sum / launches.
    name = max((k for k in table if "gflop" in table[k]), key=lambda k: table[k]["ms"])
    ent, mdl = table[name], models[name]
    launches = stages[name][1] * LAUNCHES_PER_RECORD.get(name, 1)
    if ent["bound"] == "hbm":
        roof = {"bound": "hbm", "achieved": ent["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ent["hbm_frac"]}
    else:
        pk = MFMA_PEAK_TFLOPS[a.dtype] if mdl["unit"] == "mfma" else FP64_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": ent["tflops"], "peak": pk, "unit": "TFLOP/s", "frac": ent["flop_frac"]}
    roof["traffic"] = traffic_for(name)
    roof["kernel"] = name
    roof["launch_ms"] = round(stages[name][0] / launches, 4)
    roof["launches"] = launches

    # dense reconstruction of the whole cache from the blob (jolt_reconstruct, asynchronous on torch's
    # stream): the blob is read once and the cache written once
    Ko, Vo = torch.empty_like(K), torch.empty_like(V)
    jolt.reconstruct(blob, cfg, picks, Ko, Vo, ws=ws)
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(st)
    for _ in range(3):
        jolt.reconstruct(blob, cfg, picks, Ko, Vo, ws=ws)
    r1.record(st)
    torch.cuda.synchronize()
    rec_ms = r0.elapsed_time(r1) / 3
    rec_bytes = float(sum(p["bytes"] for p in picks)) + 2.0 * L * H * T * D * 2
    rec_traffic = traffic_for("reconstruct")
    reconstruct = {"ms": round(rec_ms, 3), "gbyte": round(rec_bytes / 1e9, 3),
                   "gbs": round(rec_bytes / (rec_ms / 1e3) / 1e9, 1),
                   "hbm_frac": round(rec_bytes / (rec_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                   "traffic": None if rec_traffic is None else round(rec_traffic)}
    del Ko, Vo
    decode = decode_measure(jolt, torch, blob, cfg, picks, T, L, H, D, G, a.dtype)
    cpu = None
    if not a.no_cpu_baseline:
        cpu = cpu_baseline(K, V, groups, {"eps2": [float(x) for x in eps2], "rT": rT, "rd": rd, "bits": bits,
                                           "ratio": a.ratio, "dtype": a.dtype}, min(a.cpu_tokens, T))
    total_bytes = sum(p["bytes"] for p in picks)
    dense = 2 * L * H * T * D * 2
    line = {
        "metric": "compressed KV tokens/s (FlashJoLT, 8B-shape); % MFMA / HBM peak",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": a.dtype,
        "data": "synthetic",
        "config": {"workload": f"LLaMA-3.1-8B-shaped KV cache, 32 layers (groups of 4) x 8 KV heads x "
                               f"T={T} x d_head 128, {a.dtype}, FlashJoLT (p=10, 1 power iteration, q_cap={qcap}), "
                               f"budget {a.ratio}x",
                   "global_batch": 1, "seq_len": T, "parallelism": "single GPU", "target_ratio": a.ratio,
                   "achieved_ratio": round(dense / max(total_bytes, 1), 3), "lambda": lam,
                   "picks": [[p["rT"], p["rd"], p["bits"]] for p in picks]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "stages": table,
        "reconstruct": reconstruct,
        "decode_attention": decode,
        "wall_s_timed": round(wall, 3),
        "input_gen_s": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
