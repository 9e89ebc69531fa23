"""Helpers for the GPU parity tests: move synthetic inputs to the device in the
workload dtype and run the float64 oracle on exactly the values the GPU got."""
import numpy as np
import torch

BIG_MAMBA = ("x", "B", "C", "dy")
BIG_RAW = ("v", "B", "C", "dy")

TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_device(d, dtype, big):
    """float64 numpy dict -> torch tensors on cuda:0 (big tensors in `dtype`)."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for k, v in d.items():
        if not isinstance(v, np.ndarray):
            out[k] = v
            continue
        t = torch.from_numpy(np.ascontiguousarray(v)).to(torch.float32)
        if k in big:
            t = t.to(tdt)
        out[k] = t.to("cuda:0").contiguous()
    return out


def to_numpy(t):
    return t.detach().to(torch.float64).cpu().numpy()


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
