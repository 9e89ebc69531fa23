"""Seeded synthetic inputs for the scan-backward workloads.

This module only draws random numbers; it holds none of the method's
arithmetic.  Both the HIP path and the float64 oracle are fed from it (the
oracle gets the same values, upcast to float64 after any bf16 rounding).

Conventions
-----------
* ``N(mu, var)``: the second argument is a variance.
* Draws are float64 from ``numpy.random.default_rng(seed)`` in a fixed order:
  Mamba forms: x (or v), dt_raw, A, B, C, s0, dy, ds_final (then the MIMO decay
  scale); KDA: q, k, v, beta-logit, g-logit, do.
* ``dt`` is the raw, pre-softplus value: dt_raw ~ N(-2, 0.5), so that
  softplus(dt_raw) is the step size the workloads describe.
* bf16 casts are round-to-nearest-even (torch's ``.to(torch.bfloat16)``).

Workloads (shapes follow the pages' tensor definitions; see ``WORKLOADS``):
  mamba2_seq_small  Mamba-2 scan, b=1 T=64 H=2 P=4 N=8 G=1, fp32
  mamba1_seq        Mamba-1 scan with per-state decay, b=2 T=256 D=64 N=16, fp32
  mamba2_chunk      Mamba-2 chunked SSD, b=4 T=4096 H=32 P=64 N=128 G=1 L=64, bf16
  mimo_chunk        Mamba-3 MIMO chunked SSD, b=2 T=4096 H=32 P=64 N=128 M=4 L=64, bf16
  kda               gated delta rule, b=2 T=4096 H=16 HV=32 K=V=128, fp32
"""
from __future__ import annotations

import math

import numpy as np

WORKLOADS = {
    "mamba2_seq_small": dict(form="mamba", b=1, T=64, H=2, P=4, N=8, G=1, per_state=False, dtype="f32", seed=1000),
    "mamba1_seq": dict(form="mamba", b=2, T=256, H=64, P=1, N=16, G=1, per_state=True, dtype="f32", seed=1001),
    "mamba2_chunk": dict(form="mamba", b=4, T=4096, H=32, P=64, N=128, G=1, L=64, per_state=False,
                         dtype="bf16", seed=1002),
    "mimo_chunk": dict(form="raw", b=2, T=4096, M=4, H=32, P=64, N=128, G=32, L=64, dtype="bf16", seed=1003),
    "kda": dict(form="kda", b=2, T=4096, H=16, HV=32, K=128, V=128, dtype="f32", seed=1004),
}


def _normal(rng, shape, mean=0.0, var=1.0):
    return rng.standard_normal(size=shape) * math.sqrt(var) + mean


def mamba_inputs(b, T, H, P, N, G=1, per_state=False, seed=0, zero_s0=False, zero_seed=False):
    """x, dt (raw), A, B, C, s0, dy, ds_final as float64 arrays.

    x, dy, ds_final ~ N(0,1); dt ~ N(-2,0.5); A = -exp(U(0, ln 16)) per head
    (per (head, state) if ``per_state``); B, C ~ N(0, 1/N); s0 ~ N(0, 0.1).
    """
    rng = np.random.default_rng(seed)
    d = {}
    d["x"] = _normal(rng, (b, T, H, P))
    d["dt"] = _normal(rng, (b, T, H), -2.0, 0.5)
    d["A"] = -np.exp(rng.uniform(0.0, math.log(16.0), size=(H, N) if per_state else (H,)))
    d["B"] = _normal(rng, (b, T, G, N), 0.0, 1.0 / N)
    d["C"] = _normal(rng, (b, T, G, N), 0.0, 1.0 / N)
    d["s0"] = _normal(rng, (b, H, P, N), 0.0, 0.1)
    d["dy"] = _normal(rng, (b, T, H, P))
    d["ds_final"] = _normal(rng, (b, H, P, N))
    if zero_s0:
        d["s0"][:] = 0.0
    if zero_seed:
        d["ds_final"][:] = 0.0
    return d


def raw_inputs(b, T, M, H, P, N, G, seed=0):
    """v, da, B, C, s0, dy, ds_final for the pre-scaled (v, da) rank-M form.

    v ~ N(0,1); B, C ~ N(0, 1/N); da = -delta * exp(U(0, ln 16)) per (b, t, h)
    with delta = softplus(N(-2, 0.5)); s0 ~ N(0, 0.1); dy, ds_final ~ N(0,1).
    """
    rng = np.random.default_rng(seed)
    d = {}
    d["v"] = _normal(rng, (b, T, M, H, P))
    z = _normal(rng, (b, T, H), -2.0, 0.5)
    # the workload's step-size distribution: delta = softplus(z)
    delta = np.logaddexp(0.0, z)
    d["B"] = _normal(rng, (b, T, M, G, N), 0.0, 1.0 / N)
    d["C"] = _normal(rng, (b, T, M, G, N), 0.0, 1.0 / N)
    d["s0"] = _normal(rng, (b, H, P, N), 0.0, 0.1)
    d["dy"] = _normal(rng, (b, T, M, H, P))
    d["ds_final"] = _normal(rng, (b, H, P, N))
    d["da"] = -delta * np.exp(rng.uniform(0.0, math.log(16.0), size=(b, T, H)))
    return d


def kda_inputs(b, T, H, HV, K, V, seed=0, nonzero_state=False):
    """q, k (rows L2-normalised), v, beta, g, S0, do for the gated delta rule.

    q, k rows ~ N(0,1) then unit L2 norm; v, do ~ N(0,1); beta = sigmoid(N(0,1));
    g = -softplus(N(0,1)) per (b, t, hv, k); S0 = 0 unless ``nonzero_state``
    (then N(0, 0.1), used only by tests of the initial-state gradient).
    """
    rng = np.random.default_rng(seed)
    d = {}
    q = _normal(rng, (b, T, H, K))
    k = _normal(rng, (b, T, H, K))
    d["q"] = q / np.linalg.norm(q, axis=-1, keepdims=True)
    d["k"] = k / np.linalg.norm(k, axis=-1, keepdims=True)
    d["v"] = _normal(rng, (b, T, HV, V))
    d["beta"] = 1.0 / (1.0 + np.exp(-_normal(rng, (b, T, HV))))
    d["g"] = -np.logaddexp(0.0, _normal(rng, (b, T, HV, K)))
    d["do"] = _normal(rng, (b, T, HV, V))
    d["S0"] = _normal(rng, (b, HV, K, V), 0.0, 0.1) if nonzero_state else np.zeros((b, HV, K, V))
    d["scale"] = 1.0 / math.sqrt(K)
    return d


def workload_inputs(name, **overrides):
    """Inputs for one of ``WORKLOADS`` (shape keys may be overridden)."""
    w = dict(WORKLOADS[name])
    w.update(overrides)
    if w["form"] == "mamba":
        return mamba_inputs(w["b"], w["T"], w["H"], w["P"], w["N"], w["G"], w["per_state"], w["seed"])
    if w["form"] == "raw":
        return raw_inputs(w["b"], w["T"], w["M"], w["H"], w["P"], w["N"], w["G"], w["seed"])
    return kda_inputs(w["b"], w["T"], w["H"], w["HV"], w["K"], w["V"], w["seed"])


def round_bf16(a):
    """Round a float64 array to bf16 (round-to-nearest-even) and return it as float64."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


# tensors that travel in the "big" dtype (bf16 workloads); the rest stay fp32
BIG_MAMBA = ("x", "B", "C", "dy")
BIG_RAW = ("v", "B", "C", "dy")


def as_dtype(d, dtype, form="mamba"):
    """Round the big tensors to bf16 when dtype == 'bf16' and every tensor to fp32.

    Returns float64 arrays holding exactly the values the GPU receives.
    """
    big = BIG_MAMBA if form == "mamba" else BIG_RAW
    out = {}
    for key, val in d.items():
        if not isinstance(val, np.ndarray):
            out[key] = val
        elif dtype == "bf16" and key in big:
            out[key] = round_bf16(val)
        else:
            out[key] = val.astype(np.float32).astype(np.float64)
    return out
