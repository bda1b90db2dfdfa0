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
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the HBM byte counters)")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="print a per-kernel summary of a rocprofv3 --kernel-trace --output-format csv directory")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 --pmc csv directories (FETCH_SIZE / WRITE_SIZE of this bench and of "
                         "--calibrate-copy): write profiles/traffic.json for the dominant kernel and print a summary")
    return ap.parse_args()


# the dominant kernel of the workload: the projection P^T = Q^T X (fp32 Q in two fp16 planes
# times the fp16 cache), one launch over the 16 cells
# (one launch covers all 16 cells, split 4-fold along K = T; the launch shape is set by the
# library's sequencing, hence api.cpp among the sources whose change invalidates the counters)
TRAFFIC_KERNEL = {"stage": "project_gemm", "name": "gemm_dma_kernel<0, 2, 1, 3, 8, 3, 4, 2>", "cells_per_launch": 16,
                  "splits": 4,
                  "sources": ["kv_cache_compression_layer_amd/csrc/gemm_dma.hip",
                              "kv_cache_compression_layer_amd/csrc/gemm_core.hpp",
                              "kv_cache_compression_layer_amd/csrc/common.hpp",
                              "kv_cache_compression_layer_amd/csrc/api.cpp"]}


def project_grid(cells, splits=1, ell=522, M=4096):
    """Work-items of a projection launch over `cells` cells as the profiler reports them
    (192 x 256 tiles of 512 threads, one block per tile, K split and cell)."""
    tiles = -(-ell // 192) * -(-M // 256)
    return tiles * 512 * cells * splits


def _rows(d, fname):
    import csv
    with open(os.path.join(d, fname)) as f:
        return list(csv.DictReader(f))


def summarize_profile(d):
    """Per (kernel, grid) call count and durations from a kernel-trace csv directory."""
    import collections
    rows = _rows(d, "run_kernel_trace.csv")
    agg = collections.defaultdict(list)
    other = [0.0, 0]
    for r in rows:
        ms = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
        if "jolt::" not in r["Kernel_Name"]:  # input generation and torch glue outside the library
            other[0] += ms
            other[1] += 1
            continue
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        agg[(r["Kernel_Name"], grid)].append(ms)
    tot = sum(sum(v) for v in agg.values())
    out = ["library kernels: %.2f ms over %d dispatches (other kernels of the process: %.2f ms over %d)"
           % (tot, sum(len(v) for v in agg.values()), other[0], other[1]),
           "%9s %6s %10s %10s %12s  %s" % ("total_ms", "calls", "avg_ms", "share", "grid_items", "kernel")]
    for (name, grid), v in sorted(agg.items(), key=lambda kv: -sum(kv[1]))[:30]:
        nm = name.replace("jolt::(anonymous namespace)::", "")
        nm = nm if len(nm) <= 90 else nm[:87] + "..."
        out.append("%9.3f %6d %10.4f %9.1f%% %12d  %s" % (sum(v), len(v), sum(v) / len(v), 100 * sum(v) / tot, grid, nm))
    return "\n".join(out)


def traffic_from(fetch, write, cfetch, cwrite):
    """HBM bytes per launch of the dominant kernel: FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for a plain copy of known size."""
    def counter(d, pick):
        vals = [float(r["Counter_Value"]) for r in _rows(d, "run_counter_collection.csv") if pick(r)]
        return sum(vals) / len(vals), len(vals)
    grid = project_grid(TRAFFIC_KERNEL["cells_per_launch"], TRAFFIC_KERNEL["splits"])
    is_k = lambda r: TRAFFIC_KERNEL["name"] in r["Kernel_Name"] and int(r["Grid_Size"]) == grid
    is_copy = lambda r: "copyBuffer" in r["Kernel_Name"] or "copy" in r["Kernel_Name"].lower()
    f_kib, nf = counter(fetch, is_k)
    w_kib, nw = counter(write, is_k)
    cf_kib, _ = counter(cfetch, is_copy)
    cw_kib, _ = counter(cwrite, is_copy)
    fscale = COPY_BYTES / (cf_kib * 1024.0)
    wscale = COPY_BYTES / (cw_kib * 1024.0)
    bytes_per_launch = f_kib * 1024.0 * fscale + w_kib * 1024.0 * wscale
    ent = {"kernel": TRAFFIC_KERNEL["name"], "grid_items": grid, "sources": TRAFFIC_KERNEL["sources"],
           "source_hash": source_hash(TRAFFIC_KERNEL["sources"]), "fetch_kib": f_kib, "write_kib": w_kib,
           "fetch_scale": fscale, "write_scale": wscale, "bytes_per_launch": bytes_per_launch,
           "dispatches": [nf, nw]}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    t = {}
    if os.path.exists(path):
        with open(path) as f:
            t = json.load(f)
    t[TRAFFIC_KERNEL["stage"]] = ent
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


def kernel_models(T, L, H, D, G, ell, picks, dtype_bytes):
    """Algorithmic flops / bytes per launch of the measured stages (see the design notes)."""
    GH, M = G * H, G * H * D
    cells_per_launch = (L // G)            # K cells or V cells of one launch
    n_cells = 2 * cells_per_launch
    m = {}
    # Y^T = Omega^T X^T and Y^T = Z^T X^T: 2 T M ell flops per cell, X read once
    m["sketch_gemm"] = {"flops": 2.0 * T * M * ell * cells_per_launch, "launches_per_record": 2,
                        "bytes": (T * M * dtype_bytes + 4.0 * ell * T) * cells_per_launch}
    # P^T = Q^T X: same contraction; reads X and fp32 Q once, writes P in both layouts
    m["project_gemm"] = {"flops": 2.0 * T * M * ell * n_cells, "launches_per_record": 1,
                         "bytes": (T * M * dtype_bytes + 4.0 * ell * T + 2 * 4.0 * ell * M) * n_cells}
    # fused residual encode: one launch over the cells with b > 0
    flops = 0.0
    byts = 0.0
    for p in picks:
        if p["bits"] == 0:
            continue
        R = GH * T
        flops += 2.0 * R * (D + p["rT"]) * D
        byts += R * D * dtype_bytes + T * p["rT"] * dtype_bytes + R * D * p["bits"] / 8.0 + 4.0 * R
    m["residual_encode"] = {"flops": flops, "bytes": byts, "launches_per_record": 1}
    # feature Gram: 2 R D^2 per cell, X read once
    m["feature_gram"] = {"flops": 2.0 * GH * T * D * D * n_cells, "launches_per_record": 1,
                         "bytes": GH * T * D * dtype_bytes * n_cells}
    # per-(l,h) transpose of the cache: read + write once
    m["transpose_x"] = {"flops": 0.0, "launches_per_record": 2, "bytes": 2.0 * GH * T * D * dtype_bytes * cells_per_launch}
    return m


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
    return {"value": value, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle compress of layer group 0 (K and V cells) on the first {sample_T} tokens "
                      f"({dt:.1f} s); scaled as {sample_T} tokens / ({dt:.1f} s x {n_groups} groups); "
                      f"status {r['status']}"}


def main():
    a = parse()
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
    rT = list(range(8, 513, 8))
    rd = list(range(8, D + 1, 8))
    bits = [2, 4, 8]
    eps2 = jolt.eps2(D)
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
    ell = min(512 + 10, T)
    models = kernel_models(T, L, H, D, G, ell, picks, 2)
    # The profiled call is one compress call; rates use the stage's algorithmic work over its summed
    # launch time, the per-launch duration is that sum over the number of launches.
    best = None
    for name, (ms, cnt) in stages.items():
        if name in models and cnt > 0:
            if best is None or ms > best[1]:
                best = (name, ms, cnt)
    roof = None
    if best:
        name, ms, cnt = best
        mdl = models[name]
        # the stage was recorded cnt times, each record covering launches_per_record launches of
        # the modelled work over the whole cell batch
        nl = cnt * mdl["launches_per_record"]
        flop_rate = mdl["flops"] * nl / (ms / 1e3) / 1e12
        byte_rate = mdl["bytes"] * nl / (ms / 1e3) / 1e9
        pl_ms = ms / nl
        ai = mdl["flops"] / max(mdl["bytes"], 1.0)
        ridge = MFMA_PEAK_TFLOPS[a.dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
        if ai >= ridge:
            roof = {"bound": "mfma", "achieved": round(flop_rate, 2), "peak": MFMA_PEAK_TFLOPS[a.dtype],
                    "unit": "TFLOP/s", "frac": round(flop_rate / MFMA_PEAK_TFLOPS[a.dtype], 4)}
        else:
            roof = {"bound": "hbm", "achieved": round(byte_rate, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(byte_rate / HBM_PEAK_GBS, 4)}
        roof["traffic"] = traffic_for(name)
        roof["kernel"] = name
        roof["launch_ms"] = round(pl_ms, 4)
        roof["launches"] = nl
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
                               f"T={T} x d_head 128, {a.dtype}, FlashJoLT (p=10, 1 power iteration, q_cap=512), "
                               f"budget {a.ratio}x",
                   "global_batch": 1, "seq_len": T, "parallelism": "single GPU", "target_ratio": a.ratio,
                   "achieved_ratio": round(dense / max(total_bytes, 1), 3), "lambda": lam,
                   "picks": [[p["rT"], p["rd"], p["bits"]] for p in picks]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "stages_ms": {k: round(v[0], 3) for k, v in stages.items()},
        "wall_s_timed": round(wall, 3),
        "input_gen_s": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
