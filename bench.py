#!/usr/bin/env python3
"""Routed tokens/s of the MoE routing path on one MI355X.

One step = one moe_switch_layer call, a Switch-Base-shaped layer forward on a
fixed synthetic batch (T = 8192 tokens = 16 x 512, d_model = 768, N = 128
experts, top-1 softmax, capacity factor 1.25 -> 80 slots per expert, ReLU
expert FFN d_ff = 3072 with bf16 weights): router weight preparation, route
with load statistics (f, P, aux loss) and capacity prefix sums, capacity
slots + permute-dispatch, grouped expert FFN, gate-scaled inverse-permute
combine with the residual.  All inputs are resident in HBM before the timed
region.

value = T / (time of prepare + route + dispatch + combine) per step, the
"routed tokens/s (route + dispatch + combine)" metric; the expert FFN runs
inside every step but is excluded from that time and reported separately.
Stage times come from HIP events that the library records on its stream at
the stage boundaries (moe_layer_params.stage_events).

Also printed (same JSON line):
  roofline      the dominant kernel of the metric region against its MI355X
                roofline, with the counter-measured HBM traffic when the
                committed profile matches the current kernel source;
  cpu_baseline  the CPU oracle timed on this host on full batches of the same
                workload (route + stats + dispatch + combine).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
CSRC = os.path.join(ROOT, "load_balanced_expert_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--cf", type=float, default=1.25)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 256 MiB device copy (HBM counter calibration)")
    return p.parse_args()


# Sources that decide each kernel's code and launch shape; a committed counter
# profile is used only while these are unchanged.
KERNEL_SOURCES = {
    "route": ("route.hip", "common.hpp", "prefix.hpp", "kernels.hpp", "api.hip"),
    "dispatch": ("dispatch.hip", "common.hpp", "prefix.hpp", "kernels.hpp", "api.hip"),
    "combine": ("combine.hip", "common.hpp", "kernels.hpp", "api.hip"),
    "ffn": ("ffn.hip", "common.hpp", "kernels.hpp", "api.hip"),
}


def kernel_source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch from profiles/<kernel>_<workload>_counters.md, if that
    summary was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    m_tr = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_tr or m_hash.group(1) != src_hash:
        return None
    return float(m_tr.group(1))


def cpu_baseline(spec, inp, cap, seconds: float):
    """The oracle (float64 numpy) on full batches of the workload, repeated for ~`seconds`."""
    import numpy as np
    from oracle import dispatch as OD
    from oracle import expert as OE
    from oracle import router as OR
    from oracle import stats as OS
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    x64 = OR.decode_hidden(inp.x)
    passes = 0
    t0 = time.perf_counter()
    while True:
        r = OR.route(inp.x, inp.w_r, 1)
        OS.switch_stats(r.counts, r.prob_sum, spec.T, spec.alpha)
        dm = OD.dispatch_maps(r.idx, spec.N, cap)
        D = OD.dispatch_rows(inp.x, dm)
        OE.combine(x64, OR.decode_hidden(D), r.gate, dm.token_to_row)
        passes += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    return {"value": passes * spec.T / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{passes} full batches of T={spec.T} (route+stats+dispatch+combine in float64 numpy, "
                      f"identity expert output fed to combine) in {el:.1f} s; BLAS threads={threads}, "
                      f"host affinity cores={len(os.sched_getaffinity(0))}"}


def copy_calibration():
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n, "launches": 5}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); multi-GPU runs are not part of "
              "this path's measurement", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    import load_balanced_expert_amd as M
    import workloads as W

    dev = "cuda:0"
    spec = W.SWITCH_BASE
    T, d, N, k = spec.T, spec.d, spec.N, 1
    cap = M.capacity(T, N, args.cf)
    inp = W.switch_inputs(spec, args.seed)
    w1, w2 = W.all_expert_weights(spec, args.seed)

    def dev_t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x = dev_t(inp.x)
    w_r = dev_t(inp.w_r)
    W1 = dev_t(w1)
    W2 = dev_t(w2)
    del w1, w2
    rows_bound = min(T * k, cap * N)
    lo = M.allocate_layer_outputs(T, d, N, k, rows_bound, x.dtype, True, dev)
    torch.cuda.synchronize()

    def step(ev=None):
        M.switch_layer(x, w_r, k=k, capacity=cap, alpha=spec.alpha, w1=W1, w2=W2, outputs=lo, stage_events=ev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for evs in events:          # creates the HIP events; the library re-records them inside each step
        for e in evs:
            e.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    st = np.array([[events[i][j].elapsed_time(events[i][j + 1]) for j in range(5)]
                   for i in range(args.steps)])  # ms
    names = ["router_prepare", "route", "dispatch", "expert_ffn", "combine"]
    stage_ms = {n: float(np.mean(st[:, j])) for j, n in enumerate(names)}
    metric_ms = stage_ms["router_prepare"] + stage_ms["route"] + stage_ms["dispatch"] + stage_ms["combine"]
    value = T / (metric_ms * 1e-3)
    rows = int(lo.expert_offsets[N].item())

    # dominant single-kernel stage of the metric region
    dom = max(("route", "dispatch", "combine"), key=lambda s_: stage_ms[s_])
    t_s = stage_ms[dom] * 1e-3
    if dom == "route":
        flops = 3 * 2.0 * T * d * N                    # bf16x3 products on bf16 matrix cores
        alg_bytes = T * d * 2 + 3 * N * d * 2 + T * k * 8 + N * 8
        traffic = committed_traffic("route", "switch_base", kernel_source_hash(KERNEL_SOURCES["route"]))
        roof = {"kernel": "k_route_fused (bf16x3 MFMA router + softmax/top-1, histogram, statistics, capacity prefix)",
                "bound": "mfma", "achieved": flops / t_s / 1e12, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": flops / t_s / 1e12 / BF16_PEAK_TFLOPS, "traffic": traffic,
                "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": alg_bytes,
                "hbm_frac_of_same_launch": alg_bytes / t_s / 1e9 / HBM_PEAK_GBS}
    elif dom == "dispatch":
        alg_bytes = T * k * 4 + 2 * rows * d * 2 + T * k * 9
        traffic = committed_traffic("dispatch", "switch_base", kernel_source_hash(KERNEL_SOURCES["dispatch"]))
        roof = {"kernel": "k_disp_rank_copy (token-order slots, maps, permute copy)", "bound": "hbm",
                "achieved": alg_bytes / t_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": alg_bytes / t_s / 1e9 / HBM_PEAK_GBS, "traffic": traffic,
                "algorithmic_bytes_per_launch": alg_bytes}
    else:
        alg_bytes = rows * d * 2 + 2 * T * d * 2 + T * k * 8
        traffic = committed_traffic("combine", "switch_base", kernel_source_hash(KERNEL_SOURCES["combine"]))
        roof = {"kernel": "k_combine_vec (gather expert rows, gate, residual)", "bound": "hbm",
                "achieved": alg_bytes / t_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": alg_bytes / t_s / 1e9 / HBM_PEAK_GBS, "traffic": traffic,
                "algorithmic_bytes_per_launch": alg_bytes}
    roof["avg_launch_us"] = t_s * 1e6
    roof["stage"] = dom

    # the expert FFN stage (outside the metric): weight streaming from HBM bounds it
    d_ff = spec.d_ff
    t_ffn = stage_ms["expert_ffn"] * 1e-3
    ffn_bytes = 2 * N * d * d_ff * 2 + 2 * rows * (d + d_ff) * 2
    ffn_flops = 2 * 2.0 * rows * d * d_ff
    t1 = committed_traffic("ffn1", "switch_base", kernel_source_hash(KERNEL_SOURCES["ffn"]))
    t2 = committed_traffic("ffn2", "switch_base", kernel_source_hash(KERNEL_SOURCES["ffn"]))
    ffn_roof = {"kernel": "k_grouped_gemm<true> + k_grouped_gemm<false> (bf16 MFMA grouped GEMMs)", "bound": "hbm",
                "achieved": ffn_bytes / t_ffn / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ffn_bytes / t_ffn / 1e9 / HBM_PEAK_GBS,
                "traffic": (t1 + t2) if (t1 is not None and t2 is not None) else None,
                "algorithmic_bytes_per_stage": ffn_bytes, "algorithmic_flops_per_stage": ffn_flops,
                "mfma_frac_bf16": ffn_flops / t_ffn / 1e12 / BF16_PEAK_TFLOPS, "stage_us": t_ffn * 1e6}

    alg_metric_bytes = (T * d * 2 + N * d * 4 + T * k * 8) + (T * k * 4 * 3) + 2 * rows * d * 2 + \
        (rows * d * 2 + 2 * T * d * 2 + T * k * 8)
    out = {
        "metric": "routed tokens/sec (route+dispatch+combine) at T=8192,N=128; % HBM roofline",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 x, fp32-accurate router (bf16x3 MFMA), bf16 expert FFN",
        "data": "synthetic (seeded normals, random-init router and expert weights)",
        "config": {"workload": "switch_base: T=8192 (16x512), d_model=768, N=128 experts, top-1 softmax, "
                               f"capacity factor {args.cf} (capacity {cap}), ReLU expert FFN d_ff=3072",
                   "global_batch": T, "capacity": cap, "parallelism": "single GPU"},
        "metric_ms_per_step": metric_ms, "stage_ms": stage_ms,
        "hbm_roofline_frac_of_metric_region": alg_metric_bytes / (metric_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes_metric_region": alg_metric_bytes,
        "dropped_tokens": int(lo.drop_mask.sum().item()), "aux_loss": float(lo.aux.item()),
        "roofline": roof,
        "expert_ffn_roofline": ffn_roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(spec, inp, cap, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
