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

value = T / (time of route + dispatch + combine) per step, the "routed
tokens/s (route + dispatch + combine)" metric; the expert FFN runs inside
every step but is excluded from that time and reported separately.  Times
come from HIP events (created without the system-scope fence, so recording
them does not write back the caches) that the library records on its stream
after the dispatch and after the FFN of every step: the metric region of a
step is the span from its FFN end to the next step's dispatch end.  A short
extra run with all six stage events gives the per-stage breakdown.

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
    p.add_argument("--workload", default="switch_base",
                   choices=["switch_base", "lossfree", "balanced", "switch_c", "qb_demo", "backward"],
                   help="switch_base (default) is the headline; the others report the other configurations")
    return p.parse_args()


# Sources that decide each kernel's code and launch shape; a committed counter
# profile is used only while these are unchanged.
KERNEL_SOURCES = {
    "route": ("route.hip", "common.hpp", "dpp.hpp", "prefix.hpp", "kernels.hpp", "api.hip"),
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


def committed_trace_us(stage: str):
    """Average duration of the stage's kernel in profiles/kernels_switch_base_trace.md, if that trace
    was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, "kernels_switch_base_trace.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    key = {"route": "route", "dispatch": "dispatch", "combine": "combine"}[stage]
    m_hash = re.search(r"source_sha256_16\(" + key + r"\):\s*([0-9a-f]+)", text)
    if not m_hash or m_hash.group(1) != kernel_source_hash(KERNEL_SOURCES[key]):
        return None
    pat = {"route": r"k_route_fused[^|]*\|\s*\d+\s*\|\s*([0-9.]+)", "dispatch": r"k_disp_rank_copy[^|]*\|\s*\d+\s*\|\s*([0-9.]+)",
           "combine": r"k_combine_vec[^|]*\|\s*\d+\s*\|\s*([0-9.]+)"}[stage]
    m = re.search(pat, text)
    return float(m.group(1)) if m else None


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


def _cpu_baseline_child(cf: float, seed: int, seconds: float):
    """Entry of the oracle-timing child process: prints the cpu_baseline JSON object."""
    import workloads as W
    from oracle import dispatch as OD
    spec = W.SWITCH_BASE
    inp = W.switch_inputs(spec, seed)
    print(json.dumps(cpu_baseline(spec, inp, OD.capacity(spec.T, spec.N, cf), seconds)), flush=True)


def cpu_baseline_process(cf: float, seed: int, seconds: float, threads=None):
    """The oracle timed in a child process; threads=1 pins every BLAS / OpenMP pool to one
    thread through the environment, set before numpy is imported."""
    import subprocess
    env = dict(os.environ)
    if threads is not None:
        for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS",
                  "NUMEXPR_NUM_THREADS"):
            env[v] = str(threads)
    code = f"import bench; bench._cpu_baseline_child({cf!r}, {seed!r}, {seconds!r})"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    if r.returncode != 0:
        raise RuntimeError(f"oracle timing failed:\n{r.stderr[-2000:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


class HipEvents:
    """Timing events from the HIP runtime torch already loaded, created with
    hipEventDisableSystemFence: recording them skips the system-scope cache
    writeback and invalidation that a default event performs, which would
    otherwise add several microseconds to every measured span."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        paths = sorted(set(re.findall(r"(/\S*libamdhip64\.so[.\d]*)", open("/proc/self/maps").read())))
        if not paths:
            raise RuntimeError("HIP runtime not loaded")
        self.ct = ctypes
        self.hip = ctypes.CDLL(paths[0])
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        e = self.ct.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.ct.c_uint(self.DISABLE_SYSTEM_FENCE)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return _Ev(e.value)

    def record(self, e, stream):
        self.hip.hipEventRecord(self.ct.c_void_p(e.cuda_event), self.ct.c_void_p(stream))

    def ms(self, a, b):
        f = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(f), self.ct.c_void_p(a.cuda_event),
                                        self.ct.c_void_p(b.cuda_event)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value


class _Ev:
    """A raw hipEvent_t in the shape the binding's stage_events expects."""
    def __init__(self, handle):
        self.cuda_event = handle


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

    if args.workload != "switch_base":
        {"lossfree": bench_lossfree, "balanced": bench_balanced, "switch_c": bench_switch_c,
         "qb_demo": bench_qb_demo, "backward": bench_backward}[args.workload](args)
        return

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
    rows_bound = M.dispatch_rows(T, k, N, cap)   # capacity-padded buffer
    lo = M.allocate_layer_outputs(T, d, N, k, rows_bound, x.dtype, True, dev)
    torch.cuda.synchronize()

    def step(ev=None, capacity=cap, outputs=lo):
        M.switch_layer(x, w_r, k=k, capacity=capacity, alpha=spec.alpha, w1=W1, w2=W2, outputs=outputs,
                       stage_events=ev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    he = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream

    def timed_region(nsteps, capacity, outputs):
        """Per step only two events, after dispatch ([3]) and after the expert FFN ([4]).  The metric
        region of step i is the span from its FFN end to the dispatch end of step i + 1 (its combine,
        then the route and dispatch of the next step: the same work on the same inputs), so one event
        sits inside each measured region; the FFN is e3(i) -> e4(i)."""
        ev3 = [he.create() for _ in range(nsteps + 1)]
        ev4 = [he.create() for _ in range(nsteps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(nsteps + 1):
            step([None, None, None, ev3[i], ev4[i], None], capacity, outputs)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        region = np.array([he.ms(ev4[i], ev3[i + 1]) for i in range(nsteps)])   # ms
        ffn = np.array([he.ms(ev3[i], ev4[i]) for i in range(nsteps)])
        return region, ffn, wall

    region, ffn, wall = timed_region(args.steps, cap, lo)
    metric_ms = float(np.mean(region))
    value = T / (metric_ms * 1e-3)
    rows = int(lo.expert_rows.sum().item())   # kept rows

    # The region above holds one event record, and the GPU idles a few microseconds after each.
    # The same work with no event inside: `nq` whole steps between two events, less `nq` runs of
    # the same expert FFN (on the last step's dispatched rows) between two events; five
    # alternating rounds, the median kept.
    def no_event_region(nq, rounds=5):
        est = []
        for _ in range(rounds):
            a0, a1, b0, b1 = (he.create() for _ in range(4))
            torch.cuda.synchronize()
            he.record(a0, stream)
            for _ in range(nq):
                step()
            he.record(a1, stream)
            torch.cuda.synchronize()
            he.record(b0, stream)
            for _ in range(nq):
                M.expert_ffn(lo.dispatched, lo.expert_offsets, W1, W2, cap, out=lo.y, expert_rows=lo.expert_rows)
            he.record(b1, stream)
            torch.cuda.synchronize()
            est.append((he.ms(a0, a1) - he.ms(b0, b1)) / nq)
        return float(np.median(est)), [float(e) for e in est]

    ne_ms, ne_all = no_event_region(max(args.steps, 20))

    # Stage breakdown: a separate short run with all six stage events.  Every span also carries the
    # cost of the event packets around it; the span between two events with nothing between them
    # ([0] -> [1]: the router weight is prepared outside the step) measures that cost, and each
    # kernel's time is its span minus that.
    nb = min(args.steps, 20)
    evs = [[he.create() for _ in range(6)] for _ in range(nb)]
    for i in range(nb):
        step(evs[i])
    torch.cuda.synchronize()
    st = np.array([[he.ms(evs[i][j], evs[i][j + 1]) for j in range(5)] for i in range(nb)])
    names = ["events_only", "route", "dispatch", "expert_ffn", "combine"]
    stage_ms = {n_: float(np.mean(st[:, j])) for j, n_ in enumerate(names)}
    null_ms = stage_ms["events_only"]

    # cold cache: every step starts after a 1 GiB write that evicts L2 and the 256 MB last-level cache;
    # route + dispatch ([1] -> [3]) and combine ([4] -> [5]) spans, measured the same way warm
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    ncold = min(args.steps, 20)

    def spans(cold):
        out_ = []
        for i in range(ncold):
            if cold:
                flush.fill_(i & 0xFF)
            ev = [he.create() for _ in range(6)]
            step(ev)
            torch.cuda.synchronize()
            out_.append(he.ms(ev[1], ev[3]) + he.ms(ev[4], ev[5]))
        return float(np.mean(out_))

    warm_same = spans(False)
    cold_ms = spans(True)
    del flush

    # the expert FFN on packed weights (moe_expert_weights_pack, done once for weights that stay fixed
    # across calls; bit-identical outputs): its stage span beside the plain one, and the pack's time
    P1, P2 = torch.empty_like(W1), torch.empty_like(W2)
    pk = [he.create() for _ in range(2)]
    he.record(pk[0], stream)
    M.pack_expert_weights(W1, P1)
    M.pack_expert_weights(W2, P2)
    he.record(pk[1], stream)
    torch.cuda.synchronize()
    pack_ms = he.ms(pk[0], pk[1])
    lo_p = M.allocate_layer_outputs(T, d, N, k, rows_bound, x.dtype, True, dev)

    def step_packed(ev=None):
        M.switch_layer(x, w_r, k=k, capacity=cap, alpha=spec.alpha, w1=P1, w2=P2, outputs=lo_p, stage_events=ev,
                       weights_packed=True)

    for _ in range(3):
        step_packed()
    evp = [[he.create() for _ in range(6)] for _ in range(nb)]
    for i in range(nb):
        step_packed(evp[i])
    torch.cuda.synchronize()
    ffn_packed_ms = float(np.mean([he.ms(evp[i][3], evp[i][4]) for i in range(nb)]))
    ffn_plain_span_ms = stage_ms["expert_ffn"]
    del P1, P2, lo_p

    # capacity factor 1.0 (64 slots per expert): same timing as the headline
    cap10 = M.capacity(T, N, 1.0)
    lo10 = M.allocate_layer_outputs(T, d, N, k, M.dispatch_rows(T, k, N, cap10), x.dtype, True, dev)
    for _ in range(3):
        step(None, cap10, lo10)
    region10, _, _ = timed_region(min(args.steps, 30), cap10, lo10)
    rows10 = int(lo10.expert_rows.sum().item())

    # a plain device copy of the metric region's byte count (half read, half written): the
    # practical ceiling of a streaming kernel on this part
    alg_metric_bytes = (T * d * 2 + N * d * 4 + T * k * 8) + (T * k * 4 * 3) + 2 * rows * d * 2 + \
        (rows * d * 2 + 2 * T * d * 2 + T * k * 8)
    csrc_t = torch.empty(alg_metric_bytes // 2, dtype=torch.uint8, device=dev)
    cdst_t = torch.empty_like(csrc_t)
    copy_ms = _timed(he, stream, lambda: cdst_t.copy_(csrc_t), 20, 3, torch)[0]
    copy_gbs = alg_metric_bytes / (copy_ms * 1e-3) / 1e9
    del csrc_t, cdst_t

    # dominant kernel of the metric region, timed by the event span around it.  The span also holds
    # the event packets' cost (an empty pair measures up to `null_ms`), so it is an upper bound on the
    # kernel's duration and the fraction below a lower bound; the kernel trace (profiles/) lies between
    # the span and the span less an empty pair.
    dom = max(("route", "dispatch", "combine"), key=lambda s_: stage_ms[s_])
    t_s = stage_ms[dom] * 1e-3
    if dom == "route":
        method_flops = 2.0 * T * d * N                   # h = x . W_r, the method's fp32 product
        issued_flops = 3 * method_flops                  # three bf16 products (exact bf16x3 split of W_r)
        nch = (T + 31) // 32
        alg_bytes = T * d * 2 + N * d * 4 + T * k * 8 + nch * N * 4
        traffic = committed_traffic("route", "switch_base", kernel_source_hash(KERNEL_SOURCES["route"]))
        roof = {"kernel": "k_route_fused (W_r split in registers, bf16x3 MFMA router, softmax, top-1, histogram, "
                          "chunk counts and super-chunk sums)",
                "bound": "hbm", "achieved": alg_bytes / t_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": alg_bytes / t_s / 1e9 / HBM_PEAK_GBS, "traffic": traffic,
                "algorithmic_bytes_per_launch": alg_bytes,
                "method_flops_per_launch": method_flops,
                "mfma_frac_of_bf16_peak_on_method_flops": method_flops / t_s / 1e12 / BF16_PEAK_TFLOPS,
                "issued_bf16x3_flops_per_launch": issued_flops,
                "issued_bf16_tflops": issued_flops / t_s / 1e12,
                "why_hbm": "at bf16 peak the method's flops take 0.64 us, its bytes 1.63 us at 8 TB/s"}
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
    roof["event_span_us"] = stage_ms[dom] * 1e3
    roof["empty_event_pair_us"] = null_ms * 1e3
    roof["span_less_empty_pair_us"] = (stage_ms[dom] - null_ms) * 1e3
    roof["trace_avg_us"] = committed_trace_us(dom)
    roof["stage"] = dom

    # the expert FFN stage (outside the metric): weight streaming from HBM bounds it
    d_ff = spec.d_ff
    t_ffn = float(np.mean(ffn)) * 1e-3
    ffn_bytes = 2 * N * d * d_ff * 2 + 2 * rows * (d + d_ff) * 2
    ffn_flops = 2 * 2.0 * rows * d * d_ff
    t1 = committed_traffic("ffn1", "switch_base", kernel_source_hash(KERNEL_SOURCES["ffn"]))
    t2 = committed_traffic("ffn2", "switch_base", kernel_source_hash(KERNEL_SOURCES["ffn"]))
    ffn_roof = {"kernel": "k_grouped_gemm_stream<8, true, false> + k_grouped_gemm_stream<8, false, false> (bf16 MFMA grouped GEMMs on the plain weight layout; k_grouped_gemm where the shapes do not fit the stream kernel)", "bound": "hbm",
                "achieved": ffn_bytes / t_ffn / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ffn_bytes / t_ffn / 1e9 / HBM_PEAK_GBS,
                "traffic": (t1 + t2) if (t1 is not None and t2 is not None) else None,
                "algorithmic_bytes_per_stage": ffn_bytes, "algorithmic_flops_per_stage": ffn_flops,
                "mfma_frac_bf16": ffn_flops / t_ffn / 1e12 / BF16_PEAK_TFLOPS, "stage_us": t_ffn * 1e6}

    alg10 = (T * d * 2 + N * d * 4 + T * k * 8) + (T * k * 4 * 3) + 2 * rows10 * d * 2 + \
        (rows10 * d * 2 + 2 * T * d * 2 + T * k * 8)
    ms10 = float(np.mean(region10))
    out = {
        "metric": "routed tokens/sec (route+dispatch+combine) at T=8192,N=128; % HBM roofline",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 x, fp32-accurate router (bf16x3 MFMA), bf16 expert FFN",
        "data": "synthetic (seeded normals, random-init router and expert weights)",
        "config": {"workload": "switch_base: T=8192 (16x512), d_model=768, N=128 experts, top-1 softmax, "
                               f"capacity factor {args.cf} (capacity {cap}), ReLU expert FFN d_ff=3072",
                   "global_batch": T, "capacity": cap, "parallelism": "single GPU"},
        "metric_ms_per_step": metric_ms, "metric_ms_p10_p90": [float(np.percentile(region, 10)),
                                                               float(np.percentile(region, 90))],
        "region_without_events": {"value": T / (ne_ms * 1e-3), "ms_per_step": ne_ms, "rounds_ms": ne_all,
                                  "how": "whole steps between two events, less the same number of expert FFN runs "
                                         "between two events (median of 5 alternating rounds); the headline region "
                                         "also holds one event record"},
        "expert_ffn_ms": t_ffn * 1e3, "stage_ms_event_spans": stage_ms,
        "hbm_roofline_frac_of_metric_region": alg_metric_bytes / (metric_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "copy_ceiling_gbs": copy_gbs,
        "frac_of_copy_ceiling": alg_metric_bytes / (metric_ms * 1e-3) / 1e9 / copy_gbs,
        "algorithmic_bytes_metric_region": alg_metric_bytes,
        "cold_cache": {"value": T / (cold_ms * 1e-3), "ms_per_step": cold_ms,
                       "warm_same_spans_value": T / (warm_same * 1e-3), "warm_same_spans_ms": warm_same,
                       "how": "route+dispatch and combine event spans of steps that each start after a 1 GiB "
                              "write (L2 and the 256 MB last-level cache evicted); warm_same_spans is the same "
                              "measurement without the write"},
        "capacity_factor_1_0": {"value": T / (ms10 * 1e-3), "metric_ms_per_step": ms10, "capacity": cap10,
                                "hbm_roofline_frac_of_metric_region":
                                    alg10 / (ms10 * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                "dropped_tokens": int(lo10.drop_mask.sum().item())},
        "dropped_tokens": int(lo.drop_mask.sum().item()), "aux_loss": float(lo.aux.item()),
        "roofline": roof,
        "expert_ffn_roofline": ffn_roof,
        "expert_ffn_packed_weights": {"stage_span_ms": ffn_packed_ms, "plain_stage_span_ms": ffn_plain_span_ms,
                                      "pack_ms_once": pack_ms,
                                      "how": "the same layer with w1 and w2 rewritten once by moe_expert_weights_pack "
                                             "(bit-identical outputs); expert stage event spans, 20 steps each"},
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline_process(args.cf, args.seed, args.cpu_seconds)
        one = cpu_baseline_process(args.cf, args.seed, args.cpu_seconds / 2, threads=1)
        cb["single_thread"] = {"value": one["value"], "unit": one["unit"], "cores": 1, "sample": one["sample"]}
        out["cpu_baseline"] = cb
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------------------------
# The other configurations (one JSON line each; not the headline)
def _dev(a, torch, np, dev="cuda:0"):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def _timed(he, stream, fn, steps, warmup, torch):
    """ms per call of fn over `steps` back-to-back calls between two events."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = he.create(), he.create()
    t0 = time.perf_counter()
    he.record(a, stream)
    for _ in range(steps):
        fn()
    he.record(b, stream)
    torch.cuda.synchronize()
    return he.ms(a, b) / steps, (time.perf_counter() - t0) * 1e3 / steps


def _cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def bench_lossfree(args):
    """16 micro-batches of 4096 tokens, d=2048, n=256, k=8, sigmoid: route with the Loss-Free bias,
    expert counts and score sums, global-batch accumulation and the bias update, micro-batch after
    micro-batch, each micro-batch one moe_route_lossfree launch.  The same loop as route followed
    by moe_stats is timed beside it."""
    import numpy as np
    import torch
    import load_balanced_expert_amd as M
    import workloads as W
    spec = W.LOSSFREE
    inp = W.lossfree_inputs(spec, args.seed)
    T, d, n, k = spec.T, spec.d, spec.N, spec.k
    xs = [_dev(inp.micro_batch(t), torch, np) for t in range(spec.micro_batches)]
    w_r = _dev(inp.w_r, torch, np)
    dev = "cuda:0"
    bias = torch.zeros(n, dtype=torch.float32, device=dev)
    gc = torch.zeros(n, dtype=torch.int64, device=dev)
    gt = torch.zeros(1, dtype=torch.int64, device=dev)
    routs = [M.route(xs[0], w_r, k, score="sigmoid", bias=bias) for _ in range(spec.micro_batches)]
    souts = [M.stats(T, k, routs[0].counts, routs[0].prob_sum) for _ in range(spec.micro_batches)]
    torch.cuda.synchronize()
    he = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream

    def one_pass():
        for t in range(spec.micro_batches):
            M.route_lossfree(xs[t], w_r, k, bias, spec.gamma, global_counts=gc, global_tokens=gt, out=routs[t])

    def one_pass_two_calls():
        for t in range(spec.micro_batches):
            r = M.route(xs[t], w_r, k, score="sigmoid", bias=b2, out=routs[t])
            M.stats(T, k, r.counts, r.prob_sum, global_counts=gc2, global_tokens=gt2, bias=b2, gamma=spec.gamma,
                    out=souts[t])

    steps = max(1, args.steps // 10)
    b2, gc2, gt2 = bias.clone(), gc.clone(), gt.clone()
    ms2 = _timed(he, stream, one_pass_two_calls, steps, max(1, args.warmup // 5), torch)[0]
    ms, wall_ms = _timed(he, stream, one_pass, steps, max(1, args.warmup // 5), torch)
    tokens = spec.micro_batches * T
    value = tokens / (ms * 1e-3)
    # the fused route kernel alone, back to back, on a bias of its own
    r0, b3 = routs[0], bias.clone()
    t_route = _timed(he, stream, lambda: M.route_lossfree(xs[0], w_r, k, b3, spec.gamma, out=r0), 30, 3, torch)[0]
    method_flops = 2.0 * T * d * n       # the fp32 router product of the method
    alg_bytes = T * d * 2 + d * n * 4 + T * k * 8 + n * 8
    t_r = t_route * 1e-3
    out = {
        "metric": "routed tokens/sec (Loss-Free biased top-k route + expert counts + global batch + bias update)",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": max(1, args.warmup // 5),
        "ms_per_step": ms, "wall_ms_per_step": wall_ms, "higher_is_better": True, "scaling": "weak",
        "route_then_stats_ms_per_step": ms2,
        "vs_baseline": None, "dtype": "bf16 x, fp32-accurate router (bf16x3 MFMA), fp32 bias state",
        "data": "synthetic (4 cluster means ~N(0,4) per dim + N(0,1) noise, one cluster per micro-batch)",
        "config": {"workload": "lossfree: 16 micro-batches x 4096 tokens, d_model=2048, n=256, k=8, sigmoid, "
                               "gamma=1e-3", "global_batch": tokens, "parallelism": "single GPU"},
        # bound: the larger of the method's bytes at 8 TB/s (2.4 us) and its flops at bf16 peak (1.7 us)
        "roofline": {"kernel": "k_route_fused (bf16x3 MFMA router, sigmoid, biased top-8, histogram, score sums, "
                               "bias update)",
                     "bound": "hbm", "achieved": alg_bytes / t_r / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": alg_bytes / t_r / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "avg_launch_us": t_route * 1e3, "algorithmic_bytes_per_launch": alg_bytes,
                     "method_flops_per_launch": method_flops,
                     "mfma_frac_of_bf16_peak_on_method_flops": method_flops / t_r / 1e12 / BF16_PEAK_TFLOPS,
                     "issued_bf16x3_flops_per_launch": 3 * method_flops,
                     "timing": "stand-alone moe_route_lossfree calls back to back between two events"},
        "final_bias_range": [float(bias.min().item()), float(bias.max().item())],
    }
    if not args.no_cpu_baseline:
        from oracle import router as OR
        from oracle import stats as OS
        t0 = time.perf_counter()
        b = np.zeros(n, np.float32)
        done = 0
        while time.perf_counter() - t0 < args.cpu_seconds and done < spec.micro_batches:
            x = inp.micro_batch(done)
            r = OR.route(x, inp.w_r, k, score="sigmoid", bias=b)
            b = OS.lossfree_update(b, r.counts, T, k, spec.gamma)
            done += 1
        el = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": done * T / el, "unit": "tokens/s", "cores": int(_cpu_threads()),
                               "kind": "oracle", "sample": f"{done} micro-batches of 4096 tokens in {el:.1f} s"}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def bench_balanced(args):
    """m=4096, n=64, k=4: QB duals (5 iterations from beta = 0) then the exact completion."""
    import numpy as np
    import torch
    import load_balanced_expert_amd as M
    import workloads as W
    spec = W.BALANCED
    s_np = W.balanced_scores(spec, args.seed)
    m, n, k = spec.m, spec.n, spec.k
    s = _dev(s_np, torch, np)
    beta = torch.zeros(n, dtype=torch.float32, device="cuda:0")
    he = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    res = {}

    def solve(iters, exact):
        beta.zero_()
        return M.balance_duals(s, k, beta, iters=iters, exact=exact)

    t_exact = _timed(he, stream, lambda: solve(5, True), 20, 3, torch)[0]
    info = solve(5, True).info
    torch.cuda.synchronize()
    t_qb20 = _timed(he, stream, lambda: solve(20, False), 20, 3, torch)[0]
    t_qb1 = _timed(he, stream, lambda: solve(1, False), 20, 3, torch)[0]
    per_iter = (t_qb20 - t_qb1) / 19
    bytes_iter = 2 * m * n * 4
    out = {
        "metric": "balanced assignments/sec (QB duals, 5 iterations, + exact completion to the LP optimum)",
        "value": m / (t_exact * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": 20, "warmup": 3,
        "ms_per_step": t_exact, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32 scores and duals, fp64 completion potentials",
        "data": "synthetic (s = per-expert offset ~N(0,1.5^2) + N(0,1) noise)",
        "config": {"workload": "balanced: m=4096, n=64, k=4, exactly 256 tokens per expert",
                   "parallelism": "single GPU"},
        "augmentations": int(info[1].item()), "qb_iteration_us": per_iter * 1e3,
        "roofline": {"kernel": "k_qb_rows + k_qb_cols (one QB iteration)", "bound": "hbm",
                     "achieved": bytes_iter / (per_iter * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": bytes_iter / (per_iter * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": bytes_iter, "avg_launch_us": per_iter * 1e3,
                     "note": "s (1 MiB) stays in the caches; the iteration is latency-bound"},
    }
    if not args.no_cpu_baseline:
        from oracle import balance as OB
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < args.cpu_seconds:
            _, beta0, _ = OB.qb_solve(s_np, k, 5)
            OB.ssp_complete(s_np, k, beta0)
            done += 1
        el = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": done * m / el, "unit": "tokens/s", "cores": int(_cpu_threads()),
                               "kind": "oracle", "sample": f"{done} full solves (QB 5 + SSP completion) in {el:.1f} s"}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def bench_qb_demo(args):
    """The quantile-balancing demo of the optimal-assignment page: m=100000, n=256, k=8,
    s = U(0,1) + U(0,1)_n, T=5 rounds of the interpolated 1 - k/n quantiles from beta = 0,
    then the biased top-k; max / min / mean violation before and after."""
    import numpy as np
    import torch
    import load_balanced_expert_amd as M
    import workloads as W
    m, n, k, T = 100000, 256, 8, 5
    s_np = W.uniform_offset_scores(m, n, args.seed)
    s = _dev(s_np, torch, np)
    beta = torch.zeros(n, dtype=torch.float32, device="cuda:0")
    he = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream

    def solve(iters):
        beta.zero_()
        return M.balance_duals(s, k, beta, iters=iters, quantile=True)

    t_solve = _timed(he, stream, lambda: solve(T), 20, 3, torch)[0]
    out_solve = solve(T)
    torch.cuda.synchronize()
    counts_after = out_solve.counts.cpu().numpy()
    t_1 = _timed(he, stream, lambda: solve(1), 20, 3, torch)[0]
    t_0 = _timed(he, stream, lambda: solve(0), 20, 3, torch)[0]
    per_iter = (t_solve - t_1) / (T - 1)
    plain = torch.topk(s, k, dim=1).indices
    counts_before = torch.bincount(plain.reshape(-1), minlength=n).cpu().numpy()

    def vio(c):
        # each expert's load share against the balanced share 1/n: largest excess (MaxVio),
        # smallest, mean absolute
        excess = (c / c.sum()) / (1.0 / n) - 1.0
        return [float(excess.max()), float(excess.min()), float(np.mean(np.abs(excess)))]

    bytes_iter = 2 * m * n * 4   # the row pass reads s, the column pass its transposed copy
    out = {
        "metric": "quantile-balanced assignments/sec (T=5 interpolated-quantile QB rounds + biased top-k)",
        "value": m / (t_solve * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": 20, "warmup": 3,
        "ms_per_step": t_solve, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32 scores and duals",
        "data": "synthetic (s = U(0,1) + U(0,1)_n, the demo's recipe)",
        "config": {"workload": "qb_demo: m=100000, n=256, k=8, T=5", "parallelism": "single GPU"},
        "load_violation_before": vio(counts_before), "load_violation_after": vio(counts_after),
        "qb_iteration_us": per_iter * 1e3, "transpose_and_topk_us": t_0 * 1e3,
        "roofline": {"kernel": "k_qb_rows + k_qb_cols (one quantile QB iteration)", "bound": "hbm",
                     "achieved": bytes_iter / (per_iter * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": bytes_iter / (per_iter * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": bytes_iter, "avg_launch_us": per_iter * 1e3},
    }
    if not args.no_cpu_baseline:
        from oracle import balance as OB
        t0 = time.perf_counter()
        OB.qb_quantile_solve(s_np, k, T)
        el = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": m / el, "unit": "tokens/s", "cores": int(_cpu_threads()), "kind": "oracle",
                               "sample": f"one full solve (T=5 quantile rounds + top-k, numpy) in {el:.1f} s"}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def bench_switch_c(args):
    """T=65536, d=1024, N=2048, top-1, cf 1.25, ReLU FFN d_ff=4096 (34.4 GB of bf16 expert weights, drawn on
    the GPU from a seeded generator), timed like the headline."""
    import numpy as np
    import torch
    import load_balanced_expert_amd as M
    import workloads as W
    spec = W.SWITCH_C
    T, d, N, k, d_ff = spec.T, spec.d, spec.N, 1, spec.d_ff
    cap = M.capacity(T, N, args.cf)
    inp = W.switch_inputs(spec, args.seed)
    x = _dev(inp.x, torch, np)
    w_r = _dev(inp.w_r, torch, np)
    g = torch.Generator(device="cuda:0")
    g.manual_seed(args.seed)
    W1 = torch.empty((N, d_ff, d), dtype=torch.bfloat16, device="cuda:0")
    W2 = torch.empty((N, d, d_ff), dtype=torch.bfloat16, device="cuda:0")
    for w in (W1, W2):
        for e0 in range(0, N, 256):   # in slices, to bound the fp32 temporary
            w[e0:e0 + 256] = (torch.randn(w[e0:e0 + 256].shape, generator=g, device="cuda:0") * spec.w_std).to(
                torch.bfloat16)
    rows_bound = M.dispatch_rows(T, k, N, cap)   # capacity-padded buffer
    lo = M.allocate_layer_outputs(T, d, N, k, rows_bound, x.dtype, True, "cuda:0")
    torch.cuda.synchronize()
    he = HipEvents()

    def step(ev=None):
        M.switch_layer(x, w_r, k=k, capacity=cap, alpha=spec.alpha, w1=W1, w2=W2, outputs=lo, stage_events=ev)

    steps = max(2, min(args.steps, 10))
    for _ in range(max(1, min(args.warmup, 3))):
        step()
    torch.cuda.synchronize()
    ev3 = [he.create() for _ in range(steps + 1)]
    ev4 = [he.create() for _ in range(steps + 1)]
    t0 = time.perf_counter()
    for i in range(steps + 1):
        step([None, None, None, ev3[i], ev4[i], None])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region = np.array([he.ms(ev4[i], ev3[i + 1]) for i in range(steps)])
    ffn = np.array([he.ms(ev3[i], ev4[i]) for i in range(steps)])
    metric_ms = float(np.mean(region))
    rows = int(lo.expert_rows.sum().item())   # kept rows
    alg_metric_bytes = (T * d * 2 + N * d * 4 + T * k * 8) + (T * k * 4 * 3) + 2 * rows * d * 2 + \
        (rows * d * 2 + 2 * T * d * 2 + T * k * 8)
    method_flops = 2.0 * T * d * N      # the fp32 router product of the method (issued: 3x, bf16x3)
    t_ffn = float(np.mean(ffn)) * 1e-3
    ffn_bytes = 2 * N * d * d_ff * 2 + 2 * rows * (d + d_ff) * 2
    out = {
        "metric": "routed tokens/sec (route+dispatch+combine) at T=65536,N=2048; % HBM roofline",
        "value": T / (metric_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": max(1, min(args.warmup, 3)), "ms_per_step": wall * 1e3 / (steps + 1), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 x, fp32-accurate router (bf16x3 MFMA), bf16 expert FFN",
        "data": "synthetic (seeded normals; expert weights drawn on the GPU)",
        "config": {"workload": "switch_c: T=65536, d_model=1024, N=2048 experts, top-1 softmax, capacity factor "
                               f"{args.cf} (capacity {cap}), ReLU expert FFN d_ff=4096", "global_batch": T,
                   "capacity": cap, "parallelism": "single GPU"},
        "metric_ms_per_step": metric_ms, "expert_ffn_ms": t_ffn * 1e3,
        "hbm_roofline_frac_of_metric_region": alg_metric_bytes / (metric_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "router_method_tflops_if_metric_were_router_only": method_flops / (metric_ms * 1e-3) / 1e12,
        "dropped_tokens": int(lo.drop_mask.sum().item()),
        "expert_ffn_roofline": {"bound": "hbm", "achieved": ffn_bytes / t_ffn / 1e9, "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": ffn_bytes / t_ffn / 1e9 / HBM_PEAK_GBS,
                                "algorithmic_bytes_per_stage": ffn_bytes},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def bench_backward(args):
    """The Switch-Base layer's backward (moe_switch_layer_backward) at the forward's saved values:
    T=8192, d=768, N=128, top-1, cf 1.25, ReLU FFN d_ff=3072, fp32 upstream gradient."""
    import numpy as np
    import torch
    import load_balanced_expert_amd as M
    import workloads as W
    spec = W.SWITCH_BASE
    T, d, N, d_ff = spec.T, spec.d, spec.N, spec.d_ff
    cap = M.capacity(T, N, args.cf)
    inp = W.switch_inputs(spec, args.seed)
    w1, w2 = W.all_expert_weights(spec, args.seed)
    x, w_r, W1, W2 = (_dev(a, torch, np) for a in (inp.x, inp.w_r, w1, w2))
    del w1, w2
    dout = torch.randn((T, d), generator=torch.Generator(device="cuda:0").manual_seed(args.seed), device="cuda:0")
    fwd = M.switch_layer(x, w_r, k=1, capacity=cap, alpha=spec.alpha, w1=W1, w2=W2)
    g = M.switch_layer_backward(x, w_r, W1, W2, fwd, dout, capacity=cap, alpha=spec.alpha)
    torch.cuda.synchronize()
    he = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    steps = max(3, min(args.steps, 20))
    ms, wall_ms = _timed(he, stream, lambda: M.switch_layer_backward(x, w_r, W1, W2, fwd, dout, capacity=cap,
                                                                      alpha=spec.alpha, out=g), steps, 2, torch)
    rows = int(fwd.expert_rows.sum().item())
    # bytes the method must move: both weight sets read (data gradients), both weight gradients
    # written in fp32, the rows' activations and gradients, the router's operands
    wbytes = 2 * N * d * d_ff * 2 + 2 * N * d * d_ff * 4
    abytes = rows * (d * 2 * 3 + d_ff * 2 * 3 + d * 4 * 2) + T * d * (4 * 2 + 2 * 2) + 2 * d * N * 4 + T * N * 4 * 2
    alg = wbytes + abytes
    flops = 4 * 2.0 * rows * d * d_ff + 3 * 2.0 * T * d * N
    out = {
        "metric": "backward tokens/sec (Switch-Base layer: router, balancing loss, expert FFN, dispatch/combine)",
        "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": 2,
        "ms_per_step": ms, "wall_ms_per_step": wall_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32 gradients; bf16 expert operands with fp32 accumulation; fp32 router",
        "data": "synthetic (seeded normals; upstream gradient ~N(0,1))",
        "config": {"workload": f"backward: T=8192, d_model=768, N=128, top-1, capacity factor {args.cf} "
                               f"(capacity {cap}), ReLU FFN d_ff=3072", "parallelism": "single GPU"},
        "roofline": {"kernel": "whole backward (all launches)", "bound": "hbm",
                     "achieved": alg / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_step": alg, "algorithmic_flops_per_step": flops,
                     "mfma_frac_bf16": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
