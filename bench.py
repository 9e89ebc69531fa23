#!/usr/bin/env python3
"""Benchmark of the chunked selective-scan backward on one MI355X.

Workload: Mamba-2 chunked SSD backward, b=4, T=4096, H=32, P=64, N=128, G=1,
chunk length 64, bf16 storage with float32 accumulation; seeded synthetic
inputs already resident in HBM.  One step is one complete backward
(ssd_chunk_bwd: both stages, every kernel) over the batch.

Before the --warmup steps, the workload's steps run untimed for --settle-ms of
wall time (default 100 ms), so that the timed steps see the GPU at its steady
clocks rather than ramping up from idle.

Prints one JSON line with the metric (tokens/s = b*T per second of wall time
over exactly --steps steps, bracketed by device synchronisation), the
roofline of the dominant kernel (algorithmic bytes per launch over its average
launch time, from HIP events on the launch stream), and the float64 oracle
timed on the host on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, published (counts packed FP32 FMA)
METRIC = "scan-backward tokens/s (B·T/s) at Mamba-2 bf16 shape; % of HBM/MFMA roofline"
WORKLOAD = "mamba2_chunk"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w, elem=2, state_elem=2):
    """Compulsory HBM bytes per launch of each kernel and of the whole path.

    Every input read once, every output written once; the stored chunk states
    count once written (state scans) and once read (chunk gradients).
    """
    b, T, H, P, N, G, L, M = w["b"], w["T"], w["H"], w["P"], w["N"], w["G"], w["L"], w.get("M", 1)
    nc = -(-T // L)
    big_x = b * T * M * H * P * elem       # x (or v), dy, dx (or dv) each
    big_bc = b * T * M * G * N * elem      # B, C, dB, dC each
    small = b * T * H * 4                  # dt (or da), d_dt (or d_da) each
    state32 = b * H * P * N * 4            # s0, ds_final, d_s0 each
    states = b * nc * H * P * N * state_elem  # stored S or dS
    scans = 2 * big_x + 2 * big_bc + 2 * small + 3 * state32 + 2 * states
    grads = 3 * big_x + 4 * big_bc + 2 * small + 2 * states
    path = 3 * big_x + 4 * big_bc + 2 * small + 3 * state32
    return {"state_scans": scans, "chunk_grads": grads, "path": path}


_CSRC = "selective_state_space_vjp_amd/csrc/"
_COMMON = (_CSRC + "ssd_common.cuh", _CSRC + "common.cuh")
# the sources each profiled kernel is built from (a counter summary is valid
# for the kernel as long as these files are unchanged)
KERNEL_SOURCES = {
    # (the build script too: it sets this file's scheduling strategy)
    "ssd_chunk16_kernel": (_CSRC + "ssd_chunk16.hip",) + _COMMON + ("selective_state_space_vjp_amd/_build.py",),
    "ssd_chunk_bwd_kernel": (_CSRC + "ssd_chunk.hip",) + _COMMON,
    "ssd_state_scan_kernel": (_CSRC + "ssd_chunk.hip",) + _COMMON,
    "ssd_blocked_bwd_kernel": (_CSRC + "ssd_blocked.hip",) + _COMMON,
}


def sources_sha256(kernel_name):
    """sha256 over a kernel's sources, in order (identifies the kernel a counter run measured)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel_name]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def traffic_from_profile(kernel_name):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the kernel's current sources; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_name}.json")
    if kernel_name not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        if rec.get("sources_sha256") != sources_sha256(kernel_name):
            return None
        return float(rec["bytes_per_launch"])
    except Exception:
        return None


def machine_info():
    """What the numbers were measured on."""
    import torch

    p = torch.cuda.get_device_properties(0)
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        rocm = None
    return {"gpu": torch.cuda.get_device_name(0), "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count, "hip_runtime": torch.version.hip, "rocm": rocm,
            "torch": torch.__version__}


def rel_maxabs(got, ref):
    """max |got - ref| / max |ref| over one tensor (the parity tests' measure)."""
    import numpy as np

    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return num / den if den > 0 else num


def _first(c, n=1):
    return {k: (v[:n] if hasattr(v, "ndim") and v.ndim >= 3 else v) for k, v in c.items()}


def _oracle_ssm(c, w, nthreads):
    """The float64 oracle's backward on the (already sliced) inputs c; returns (seconds, outputs)."""
    import oracle

    t0 = time.perf_counter()
    if w["form"] == "raw":
        ref = oracle.raw_seq_bwd(c["v"], c["da"], c["B"], c["C"], c["s0"], c["dy"], c["ds_final"], nthreads=nthreads)
    else:
        ref = oracle.mamba_seq_bwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["s0"], c["dy"], c["ds_final"],
                                   nthreads=nthreads)
    return time.perf_counter() - t0, ref


def _head_slice(c, w, nh):
    """The first nh heads of batch element 0 (per-head B/C follow the heads when G = H)."""
    out = _first(c)
    hk = ("v", "dy") if w["form"] == "raw" else ("x", "dy")
    for k in hk:
        out[k] = out[k][..., :nh, :]
    for k in ("dt", "da"):
        if k in out:
            out[k] = out[k][..., :nh]
    if "A" in out and w["form"] != "raw":
        out["A"] = out["A"][:nh]
    for k in ("s0", "ds_final"):
        out[k] = out[k][:, :nh]
    if w["G"] == w["H"]:
        for k in ("B", "C"):
            out[k] = out[k][..., :nh, :]
    return out


def cpu_baseline(inp_bf16, w):
    """The float64 oracle on one of the b sequences (all heads, all T steps), on
    every host core; also on one core over the first heads of that sequence.
    Returns (record, oracle outputs for batch element 0)."""
    import oracle

    threads = oracle.default_threads()
    sec, ref = _oracle_ssm(_first(inp_bf16), w, threads)
    nh = max(1, w["H"] // 8)
    sec1, _ = _oracle_ssm(_head_slice(inp_bf16, w, nh), w, 1)
    rec = {"value": w["T"] / sec, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"1 of {w['b']} sequences (T={w['T']}, all {w['H']} heads), float64 store-all "
                     f"sequential reverse recurrence, {sec:.2f} s",
           "one_core": {"value": w["T"] * nh / w["H"] / sec1, "unit": "tokens/s", "cores": 1,
                        "sample": f"heads 0..{nh - 1} of that sequence, {sec1:.2f} s, scaled by {nh}/{w['H']} "
                                  f"of the heads"}}
    return rec, ref


def kda_cpu_baseline(c, w):
    """The float64 oracle on batch element 0, qk head 0 and its value heads (all T
    steps), threaded over the value heads, and on one core over one value head.
    Returns (record, oracle outputs of that slice)."""
    import oracle

    threads = oracle.default_threads()
    grp = w["HV"] // w["H"]
    sl = {k: c[k][:1, :, :1] for k in ("q", "k")}
    sl.update({k: c[k][:1, :, :grp] for k in ("v", "beta", "g", "do")})
    t0 = time.perf_counter()
    ref = oracle.kda_bwd(sl["q"], sl["k"], sl["v"], sl["beta"], sl["g"], c["S0"][:1, :grp], sl["do"], None,
                         scale=c["scale"], nthreads=threads)
    sec = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.kda_bwd(sl["q"], sl["k"], sl["v"][:, :, :1], sl["beta"][:, :, :1], sl["g"][:, :, :1], c["S0"][:1, :1],
                   sl["do"][:, :, :1], None, scale=c["scale"], nthreads=1)
    sec1 = time.perf_counter() - t0
    seqs = w["b"] * w["HV"]  # (batch, value head) sequences of the workload
    rec = {"value": w["b"] * w["T"] * grp / seqs / sec, "unit": "tokens/s", "cores": min(threads, grp),
           "kind": "oracle",
           "sample": f"batch element 0, qk head 0 and its {grp} value heads (T={w['T']}), float64 store-all "
                     f"reverse recurrence, {sec:.2f} s; scaled by the {grp}/{seqs} share of the "
                     f"(batch, value head) sequences",
           "one_core": {"value": w["b"] * w["T"] / seqs / sec1, "unit": "tokens/s", "cores": 1,
                        "sample": f"value head 0 of that slice, {sec1:.2f} s, scaled by 1/{seqs}"}}
    return rec, ref


def kda_flops(w):
    """Algorithmic flops per launch: 5KV per (token, value head) for the forward
    recompute (exp-gate scaling, k^T S_dec, rank-1 update) and 15KV for the
    backward (q-do outer product, S_t do, dS r, dS^T a, S_dec dr, k-dr update,
    rowsum(S_dec dS), gate scaling), counting an FMA as 2."""
    per = w["b"] * w["T"] * w["HV"] * w["K"] * w["V"]
    return {"ckpt": 5 * per, "bwd": 20 * per}


def bench_kda(args, dev):
    import numpy as np
    import torch

    from selective_state_space_vjp_amd import binding, synth

    w = dict(synth.WORKLOADS["kda"])
    inp = synth.workload_inputs("kda")
    c = {k: (v.astype(np.float32).astype(np.float64) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(torch.float32).to(dev).contiguous()
         for k, v in inp.items() if isinstance(v, np.ndarray)}
    call = binding.DeltaCall(t["q"], t["k"], t["v"], t["beta"], t["g"], t["S0"], t["do"], None, scale=inp["scale"])
    del inp
    stages = (binding.DELTA_CKPT, binding.DELTA_BWD, binding.DELTA_REDUCE)
    settle([lambda s=s: call.stage(s) for s in stages], args.settle_ms)
    for _ in range(args.warmup):
        for s in stages:
            call.stage(s)
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        for j, s in enumerate(stages):
            call.stage(s)
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    ms = [sum(e[j].elapsed_time(e[j + 1]) for e in ev) / K for j in range(3)]
    tokens = w["b"] * w["T"]
    fl = kda_flops(w)
    # per (token, value head, 32-column slice): dq_e, dk_e and dg partial rows and one dbeta partial
    part_bytes = w["b"] * w["T"] * w["HV"] * (w["V"] // 32) * (3 * w["K"] + 1) * 4
    # the reduction reads the partials, writes dq, dk ([b,T,H,K]), dg ([b,T,HV,K]) and dbeta
    red_bytes = part_bytes + 4 * (2 * w["b"] * w["T"] * w["H"] * w["K"] + w["b"] * w["T"] * w["HV"] * (w["K"] + 1))
    phases = {
        "ckpt": {"kernel": "delta_fwd_ckpt_kernel", "ms": ms[0], "flops": fl["ckpt"],
                 "TFLOPs": fl["ckpt"] / (ms[0] * 1e9)},
        "bwd": {"kernel": "delta_bwd_kernel", "ms": ms[1], "flops": fl["bwd"], "TFLOPs": fl["bwd"] / (ms[1] * 1e9)},
        "reduce": {"kernel": "delta_reduce_kernel", "ms": ms[2], "bytes": red_bytes,
                   "GBps": red_bytes / (ms[2] * 1e6)},
    }
    dom = phases["bwd"]
    roofline = {"bound": "alu", "achieved": round(dom["TFLOPs"], 2), "peak": FP32_VECTOR_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(dom["TFLOPs"] / FP32_VECTOR_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": dom["kernel"], "algorithmic_flops_per_launch": dom["flops"],
                "avg_launch_ms": round(dom["ms"], 4)}
    line = {
        "metric": METRIC, "value": round(tokens / (ms_per_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "kda", "batch": w["b"], "seqlen": w["T"], "qk_heads": w["H"], "v_heads": w["HV"],
                   "dk": w["K"], "dv": w["V"]},
        "roofline": roofline,
        "phases": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                   for k, v in phases.items()},
    }
    line["seed"] = w["seed"]
    line["machine"] = machine_info()
    line["timing"] = "back-to-back steps (nothing between the library calls); warm infinity cache"
    line["settle_ms"] = args.settle_ms
    if not args.no_cpu_baseline:
        line["cpu_baseline"], ref = kda_cpu_baseline(c, w)
        grp = w["HV"] // w["H"]
        o = call.out
        got = {"dq": o["dq"][:1, :, :1], "dk": o["dk"][:1, :, :1], "dv": o["dv"][:1, :, :grp],
               "dg": o["dg"][:1, :, :grp], "dbeta": o["dbeta"][:1, :, :grp]}
        line["rel_maxabs"] = {k: float(f"{rel_maxabs(v.double().cpu().numpy(), ref[k]):.3e}") for k, v in got.items()}
        line["rel_maxabs_sample"] = "batch element 0, qk head 0 and its value heads, against the float64 oracle"
    print(json.dumps(line), flush=True)


MALL_FLUSH_BYTES = 512 << 20  # twice the 256 MB infinity cache


def settle(step_fns, ms):
    """Run the workload's steps untimed for `ms` of wall time before the warm-up
    steps.  An idle MI355X needs a few tens of milliseconds of load to reach its
    steady clocks (measured: 20 timed steps after 5 warm-up steps from idle run
    about 12 % slower than after 30 ms or more of settling, and no faster after
    100 ms than after 30 ms), which the warm-up steps alone (about a millisecond
    at the default workload) do not cover."""
    import torch

    if ms <= 0:
        return
    t_end = time.perf_counter() + ms / 1e3
    while time.perf_counter() < t_end:
        for f in step_fns:
            f()
        torch.cuda.synchronize()


def cold_cache_steps(step_fns, n, dev):
    """Per-step times with the infinity cache evicted before every step: a
    512 MiB buffer is overwritten between steps (outside the timed events), so
    each step starts with none of its inputs cached, as after other layers'
    traffic.  step_fns are the step's stages; returns the median ms of each
    stage and of the whole step."""
    import torch

    scratch = torch.empty(MALL_FLUSH_BYTES, dtype=torch.uint8, device=dev)
    per = []
    for i in range(n):
        scratch.fill_(i & 0xFF)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(step_fns) + 1)]
        evs[0].record()
        for k, f in enumerate(step_fns):
            f()
            evs[k + 1].record()
        torch.cuda.synchronize()
        per.append([evs[k].elapsed_time(evs[k + 1]) for k in range(len(step_fns))])
    del scratch
    med = lambda v: sorted(v)[len(v) // 2]
    stages = [med([p[k] for p in per]) for k in range(len(step_fns))]
    return stages, med([sum(p) for p in per])


def bench_fwd(args, dev):
    """The chunked forward (ssd_chunk_fwd: y and the final state) at the Mamba-2
    chunked workload shape: one step is one forward over the batch."""
    import numpy as np
    import torch

    from selective_state_space_vjp_amd import binding, synth

    w = dict(synth.WORKLOADS["mamba2_chunk"])
    inp = synth.workload_inputs("mamba2_chunk")
    c = synth.as_dtype(inp, "bf16", "mamba")
    del inp

    def dt_(a, dtype=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32).to(dtype).to(dev).contiguous()

    bf = torch.bfloat16
    x, B, C = dt_(c["x"], bf), dt_(c["B"], bf), dt_(c["C"], bf)
    dt, A, s0 = dt_(c["dt"]), dt_(c["A"]), dt_(c["s0"])
    desc = binding.ssd_desc(x, B, w["L"], binding.FORM_MAMBA2)
    ws = torch.empty(max(binding.ssd_chunk_fwd_workspace(desc), 1), dtype=torch.uint8, device=dev)
    out = {"y": torch.empty_like(x), "s_final": torch.empty_like(s0)}

    def step():
        binding.ssd_chunk_fwd(x, dt, A, B, C, s0, chunk_len=w["L"], out=out, workspace=ws)

    settle([step], args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):  # per-call times: the same K calls again, with events around each
        ev[i][0].record()
        step()
        ev[i][1].record()
    torch.cuda.synchronize()
    call_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    b, T, H, P, N, G = w["b"], w["T"], w["H"], w["P"], w["N"], w["G"]
    # compulsory HBM bytes: x, B, C, dt read and y written once, s0 read and s_final written
    fwd_bytes = 2 * b * T * H * P * 2 + 2 * b * T * G * N * 2 + b * T * H * 4 + 2 * b * H * P * N * 4
    gbps = fwd_bytes / (call_ms * 1e6)
    line = {
        "metric": "scan-forward tokens/s (B·T/s) at Mamba-2 bf16 shape; % of HBM roofline", "value":
        round(b * T / (ms_per_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "mamba2_fwd", "batch": b, "seqlen": T, "heads": H, "headdim": P, "dstate": N,
                   "ngroups": G, "chunk_len": w["L"], "form": "mamba2", "accumulate": "fp32"},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "ssd_fwd_scores_kernel + ssd_fwd_walk_kernel (one ssd_chunk_fwd call)",
                     "algorithmic_bytes_per_launch": fwd_bytes, "avg_launch_ms": round(call_ms, 4)},
    }
    _, cold_ms = cold_cache_steps([step], min(K, 20), dev)
    line["cold_cache"] = {"flush_bytes": MALL_FLUSH_BYTES, "ms_per_step": round(cold_ms, 4),
                          "tokens_per_s": round(b * T / (cold_ms / 1e3), 1),
                          "note": "median per-step event time, infinity cache evicted before each step"}
    line["seed"] = w["seed"]
    line["machine"] = machine_info()
    line["timing"] = "back-to-back steps (nothing between the library calls); warm infinity cache"
    line["settle_ms"] = args.settle_ms
    if not args.no_cpu_baseline:
        import oracle

        threads = oracle.default_threads()
        c0 = {k: (v[:1] if hasattr(v, "ndim") and v.ndim >= 3 else v) for k, v in c.items()}
        t0 = time.perf_counter()
        oracle.mamba_seq_fwd(c0["x"], c0["dt"], c0["A"], c0["B"], c0["C"], c0["s0"], nthreads=threads)
        sec = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": T / sec, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                                "sample": f"1 of {b} sequences (T={T}, all {H} heads), float64 sequential "
                                          f"forward recurrence, {sec:.2f} s"}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed steps for this much wall time before the warm-up steps (GPU clock settle)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD,
                    choices=("mamba2_chunk", "mimo_chunk", "kda", "mamba2_fwd", "mamba2_seq_small", "mamba1_seq"),
                    help="mamba2_chunk (default, the headline line), mimo_chunk (rank-4 MIMO, RAW form), "
                         "kda (gated delta rule, b=2 T=4096 H=16 HV=32 K=V=128, fp32), mamba2_fwd (the "
                         "chunked forward at the mamba2_chunk shape), or the sequential path's small fp32 "
                         "workloads mamba2_seq_small (b=1 T=64 H=2 P=4 N=8) and mamba1_seq (b=2 T=256 D=64 N=16)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        log("bench.py measures one GPU: the library runs on a single MI355X and launches no multi-GPU work "
            "(the backward would shard by batch and B/C group, with no exchange between GPUs).")
        sys.exit(2)

    import numpy as np
    import torch

    from selective_state_space_vjp_amd import binding, synth

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        # a plain 1 GiB device copy: the reference for the HBM byte counters
        # (FETCH_SIZE / WRITE_SIZE of a known transfer) and the rate a pure
        # streaming kernel reaches on this GPU (read + write bytes / time)
        n = 1 << 28  # 2^28 float32 = 1 GiB
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        ms = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dst.copy_(src)
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        fill = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dst.fill_(1.0)
            e1.record()
            torch.cuda.synchronize()
            fill.append(e0.elapsed_time(e1))
        med = sorted(ms)[2]
        print(json.dumps({"calibrate_copy_bytes": n * 4, "copies": 6, "copy_ms_median": round(med, 4),
                          "copy_GBps": round(2 * n * 4 / (med * 1e6), 1),
                          "fill_GBps": round(n * 4 / (sorted(fill)[2] * 1e6), 1),
                          "machine": machine_info()}), flush=True)
        return
    if args.workload == "kda":
        return bench_kda(args, dev)
    if args.workload == "mamba2_fwd":
        return bench_fwd(args, dev)
    if args.workload in ("mamba2_seq_small", "mamba1_seq"):
        return bench_seq(args, dev)
    w = dict(synth.WORKLOADS[args.workload])
    w.setdefault("M", 1)
    inp = synth.workload_inputs(args.workload)
    raw = w["form"] == "raw"
    c = synth.as_dtype(inp, "bf16", "raw" if raw else "mamba")

    def dt_(a, dtype=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32).to(dtype).to(dev).contiguous()

    bf = torch.bfloat16
    if raw:  # pre-scaled (v, da) form: no A
        xv, dy, B, C = dt_(c["v"], bf), dt_(c["dy"], bf), dt_(c["B"], bf), dt_(c["C"], bf)
        dtda, A = dt_(c["da"]), None
    else:
        xv, dy, B, C = dt_(c["x"], bf), dt_(c["dy"], bf), dt_(c["B"], bf), dt_(c["C"], bf)
        dtda, A = dt_(c["dt"]), dt_(c["A"])
    s0, dsf = dt_(c["s0"]), dt_(c["ds_final"])
    call = binding.SsdCall(xv, dtda, A, B, C, s0, dy, dsf, chunk_len=w["L"])
    del inp
    # the kernel the library dispatches the per-chunk backward to at this shape
    if w["L"] * w["M"] > 64:
        grads_kernel = "ssd_blocked_bwd_kernel"
    elif (w["P"], w["N"], w["L"], w["M"]) == (64, 128, 64, 1):
        grads_kernel = "ssd_chunk16_kernel"  # bf16, 16 waves
    else:
        grads_kernel = "ssd_chunk_bwd_kernel"

    settle([call.states, call.grads], args.settle_ms)
    for _ in range(args.warmup):
        call.states()
        call.grads()
    torch.cuda.synchronize()

    K = args.steps
    # the timed steps: nothing but the library calls between the two syncs
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        call.states()
        call.grads()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    # per-stage times: the same K steps again, with events around each stage
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        ev[i][0].record()
        call.states()
        ev[i][1].record()
        call.grads()
        ev[i][2].record()
    torch.cuda.synchronize()
    scans_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    grads_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    tokens = w["b"] * w["T"]
    value = tokens / (ms_per_step / 1e3)

    ab = algorithmic_bytes(w)
    phases = {
        "state_scans": {"kernel": "ssd_state_scan_kernel", "ms": scans_ms, "bytes": ab["state_scans"],
                        "GBps": ab["state_scans"] / (scans_ms * 1e6)},
        "chunk_grads": {"kernel": grads_kernel, "ms": grads_ms, "bytes": ab["chunk_grads"],
                        "GBps": ab["chunk_grads"] / (grads_ms * 1e6)},
    }
    dom_name = max(phases, key=lambda k: phases[k]["ms"])
    dom = phases[dom_name]
    traffic = traffic_from_profile(dom["kernel"])
    roofline = {"bound": "hbm", "achieved": round(dom["GBps"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom["GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom["kernel"],
                "algorithmic_bytes_per_launch": dom["bytes"], "avg_launch_ms": round(dom["ms"], 4)}

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "batch": w["b"], "seqlen": w["T"], "heads": w["H"], "headdim": w["P"],
                   "dstate": w["N"], "ngroups": w["G"], "chunk_len": w["L"], "mimo_rank": w["M"],
                   "form": w["form"], "accumulate": "fp32"},
        "roofline": roofline,
        "phases": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                   for k, v in phases.items()},
        "path_roofline": {"algorithmic_bytes": ab["path"], "achieved_GBps": round(ab["path"] / (ms_per_step * 1e6), 1),
                          "frac": round(ab["path"] / (ms_per_step * 1e6) / HBM_PEAK_GBS, 4)},
    }
    (cold_scans, cold_grads), cold_ms = cold_cache_steps([call.states, call.grads], min(K, 20), dev)
    line["cold_cache"] = {"flush_bytes": MALL_FLUSH_BYTES, "ms_per_step": round(cold_ms, 4),
                          "tokens_per_s": round(tokens / (cold_ms / 1e3), 1),
                          "state_scans_ms": round(cold_scans, 4), "chunk_grads_ms": round(cold_grads, 4),
                          "note": "median per-step event times, infinity cache evicted before each step"}
    line["seed"] = w["seed"]
    line["machine"] = machine_info()
    line["settle_ms"] = args.settle_ms
    line["timing"] = ("ms_per_step: wall clock over back-to-back steps (nothing between the library calls), "
                      "warm infinity cache, after settle_ms of untimed steps and the warm-up steps; "
                      "cold_cache: every step after a 512 MiB write")
    if not args.no_cpu_baseline:
        line["cpu_baseline"], ref = cpu_baseline(c, w)
        line["rel_maxabs"] = {k: float(f"{rel_maxabs(v[:1].double().cpu().numpy(), ref[k]):.3e}")
                              for k, v in call.out.items()}
        line["rel_maxabs_sample"] = "batch element 0, every output element, against the float64 oracle"
    print(json.dumps(line), flush=True)


def bench_seq(args, dev):
    """The sequential backward (ssm_scan_bwd) on one of the small fp32 workloads:
    tokens/s only; these are latency-bound correctness configurations, so no
    roofline claim is made."""
    import numpy as np
    import torch

    from selective_state_space_vjp_amd import binding, synth

    w = dict(synth.WORKLOADS[args.workload])
    inp = synth.workload_inputs(args.workload)
    c = synth.as_dtype(inp, "f32", "mamba")
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(torch.float32).to(dev).contiguous()
         for k, v in c.items() if isinstance(v, np.ndarray)}
    call = binding.ScanCall(t["x"], t["dt"], t["A"], t["B"], t["C"], t["s0"], t["dy"], t["ds_final"])
    settle([call.run], args.settle_ms)
    for _ in range(args.warmup):
        call.run()
    torch.cuda.synchronize()
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        call.run()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / K
    tokens = w["b"] * w["T"]
    line = {
        "metric": "sequential scan-backward tokens/s (B·T/s)", "value": round(tokens / (ms_per_step / 1e3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "batch": w["b"], "seqlen": w["T"], "heads": w["H"], "headdim": w["P"],
                   "dstate": w["N"], "ngroups": w["G"], "decay": "per_state" if w["per_state"] else "per_head"},
        "roofline": None,
        "roofline_note": "latency-bound correctness configuration (a few thousand tokens): no roofline claim",
        "seed": w["seed"], "machine": machine_info(),
        "timing": "back-to-back steps (nothing between the library calls)", "settle_ms": args.settle_ms,
    }
    if not args.no_cpu_baseline:
        import oracle

        threads = oracle.default_threads()
        t0 = time.perf_counter()
        ref = oracle.mamba_seq_bwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["s0"], c["dy"], c["ds_final"],
                                   nthreads=threads)
        sec = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": tokens / sec, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                                "sample": f"the whole workload, float64 store-all reverse recurrence, {sec:.3f} s"}
        line["rel_maxabs"] = {k: float(f"{rel_maxabs(v.double().cpu().numpy(), ref[k]):.3e}")
                              for k, v in call.out.items()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
