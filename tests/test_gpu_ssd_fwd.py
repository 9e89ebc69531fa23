"""GPU parity of ssd_chunk_fwd (chunked SSD forward: y and the final state)
through the C ABI.

* Mamba-2 form against the float64 sequential oracle, fp32 (1e-4) and bf16
  (2e-2), at sizes spanning several chunks with a shorter last chunk, one or
  two 16-column p tiles per workgroup, odd and even numbers of 16-wide state
  tiles, several groups and chunk lengths below 64;
* RAW (v, da) rank-M form against the oracle, including ranks whose steps
  straddle 16-row tiles (M = 3, 32) and one step per chunk (M = 64);
* the full bf16 workload (b=4, T=4096, H=32, P=64, N=128) in the launch
  configuration the benchmark times: batch element 0 against the oracle, the
  whole batch through y_{T-1} = C_{T-1} . s_final;
* two chained calls (s_final of the first as s0 of the second) equal one call;
* edge cases: T = 0 (s_final = s0), T = 1, s0 absent, s_final not requested,
  determinism.
"""
import numpy as np
import pytest
import torch

import oracle
from _helpers import rel_maxabs
from gpu_common import BIG_MAMBA, BIG_RAW, TOL, announce, to_device, to_numpy
from selective_state_space_vjp_amd import binding as bd
from selective_state_space_vjp_amd import synth

pytestmark = pytest.mark.gpu


def _gpu_m2(inp, dtype, L, s0=True):
    t = to_device(inp, dtype, BIG_MAMBA)
    out = bd.ssd_chunk_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["s0"] if s0 else None, chunk_len=L)
    torch.cuda.synchronize()
    return {k: to_numpy(v) for k, v in out.items()}


def _oracle_m2(inp, dtype, s0=True):
    c = synth.as_dtype(inp, dtype, "mamba")
    y, sf = oracle.mamba_seq_fwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["s0"] if s0 else None)
    return {"y": y, "s_final": sf}


def _compare(got, ref, tol, keys=("y", "s_final")):
    errs = {k: rel_maxabs(got[k], ref[k]) for k in keys if ref[k].size}
    print("[rel_maxabs]", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert errs and max(errs.values()) < tol, errs
    return errs


M2_SHAPES = [
    # b, T, H, P, N, G, L
    (2, 200, 4, 32, 32, 2, 64),
    (1, 130, 2, 64, 128, 1, 64),
    (2, 96, 4, 16, 48, 4, 16),
    (1, 77, 3, 48, 16, 1, 32),
    (1, 64, 8, 64, 64, 2, 48),
    (1, 150, 2, 32, 80, 1, 64),
    (2, 70, 2, 96, 112, 2, 64),
    # large heads: N = 128 (the largest state) with P = 160 and P = 256
    (1, 80, 2, 160, 128, 1, 64),
    (1, 100, 2, 256, 128, 1, 64),
]


@pytest.mark.parametrize("shape", M2_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mamba2_form_parity(shape, dtype):
    b, T, H, P, N, G, L = shape
    announce(f"ssd fwd mamba2 {dtype} {shape}")
    inp = synth.mamba_inputs(b, T, H, P, N, G, False, seed=sum(shape))
    _compare(_gpu_m2(inp, dtype, L), _oracle_m2(inp, dtype), TOL[dtype])


@pytest.mark.parametrize("shape", [(1, 200, 3, 64, 128, 1, 64), (2, 130, 2, 32, 32, 2, 32)])
@pytest.mark.parametrize("regime", ["no_decay", "weak_decay_long_steps"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decay_regimes(shape, regime, dtype):
    """A = 0 (plain running sums of the inputs) and A = -0.01 with steps of
    about 4 (slow decay, growing states), against the default inputs' fast
    decay."""
    b, T, H, P, N, G, L = shape
    announce(f"ssd fwd mamba2 {dtype} {shape} {regime}")
    inp = synth.mamba_inputs(b, T, H, P, N, G, False, seed=sum(shape) + 7)
    if regime == "no_decay":
        inp["A"][:] = 0.0
    else:
        inp["A"][:] = -0.01
        inp["dt"] = inp["dt"] + 6.0
    _compare(_gpu_m2(inp, dtype, L), _oracle_m2(inp, dtype), TOL[dtype])


RAW_SHAPES = [
    # b, T, M, H, P, N, G, L
    (1, 64, 4, 2, 32, 32, 2, 16),
    (2, 100, 2, 4, 16, 32, 4, 32),
    (1, 48, 1, 4, 32, 16, 1, 64),
    (1, 40, 4, 2, 16, 16, 1, 16),
    (1, 90, 4, 2, 64, 128, 2, 64),
    (1, 50, 3, 2, 32, 32, 1, 16),
    (1, 9, 32, 2, 16, 32, 1, 64),
    (1, 5, 64, 1, 16, 16, 1, 64),
]


@pytest.mark.parametrize("shape", RAW_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_raw_mimo_form_parity(shape, dtype):
    b, T, M, H, P, N, G, L = shape
    announce(f"ssd fwd raw {dtype} {shape}")
    inp = synth.raw_inputs(b, T, M, H, P, N, G, seed=sum(shape))
    c = synth.as_dtype(inp, dtype, "raw")
    y, sf = oracle.raw_seq_fwd(c["v"], c["da"], c["B"], c["C"], c["s0"])
    t = to_device(inp, dtype, BIG_RAW)
    out = bd.ssd_chunk_fwd(t["v"], t["da"], None, t["B"], t["C"], t["s0"], chunk_len=L)
    torch.cuda.synchronize()
    got = {k: to_numpy(v) for k, v in out.items()}
    _compare(got, {"y": y, "s_final": sf}, TOL[dtype])


def test_full_bf16_workload_batch0_and_last_row_identity():
    w = synth.WORKLOADS["mamba2_chunk"]
    announce("ssd fwd bf16 full workload b=4 T=4096 H=32 P=64 N=128 L=64")
    inp = synth.workload_inputs("mamba2_chunk")
    got = _gpu_m2(inp, "bf16", w["L"])
    c = synth.as_dtype(inp, "bf16", "mamba")
    # whole batch: the last output row reads the final state, y_{T-1}[h,p] = sum_n C_{T-1}[g,n] s_final[h,p,n]
    hpg = w["H"] // w["G"]
    Cl = np.repeat(c["C"][:, -1], hpg, axis=1)  # [b, H, N]
    pred = np.einsum("bhn,bhpn->bhp", Cl, got["s_final"])
    assert rel_maxabs(got["y"][:, -1], pred) < TOL["bf16"]
    # batch element 0 against the oracle
    c0 = {k: (v[:1] if isinstance(v, np.ndarray) and v.ndim >= 3 else v) for k, v in c.items()}
    y, sf = oracle.mamba_seq_fwd(c0["x"], c0["dt"], c0["A"], c0["B"], c0["C"], c0["s0"])
    _compare({k: v[:1] for k, v in got.items()}, {"y": y, "s_final": sf}, TOL["bf16"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_two_chained_calls_equal_one(dtype):
    b, T, T1, H, P, N, G, L = 1, 192, 100, 4, 64, 128, 1, 64
    announce(f"ssd fwd chaining {dtype} T={T} split at {T1}")
    inp = synth.mamba_inputs(b, T, H, P, N, G, False, seed=78)
    one = _gpu_m2(inp, dtype, L)
    head = {k: inp[k][:, :T1] for k in ("x", "dt", "B", "C")}
    tail = {k: inp[k][:, T1:] for k in ("x", "dt", "B", "C")}
    g1 = _gpu_m2({**head, "A": inp["A"], "s0": inp["s0"]}, dtype, L)
    g2 = _gpu_m2({**tail, "A": inp["A"], "s0": g1["s_final"]}, dtype, L)
    chained = {"y": np.concatenate([g1["y"], g2["y"]], axis=1), "s_final": g2["s_final"]}
    _compare(chained, one, 1e-5 if dtype == "f32" else TOL["bf16"])


@pytest.mark.parametrize("T,L", [(10, 64), (1, 16), (64, 64), (65, 64)])
def test_short_sequences(T, L):
    announce(f"ssd fwd short T={T} L={L}")
    inp = synth.mamba_inputs(1, T, 2, 16, 32, 1, False, seed=T)
    _compare(_gpu_m2(inp, "f32", L), _oracle_m2(inp, "f32"), TOL["f32"])


def test_without_initial_state():
    announce("ssd fwd s0 absent")
    inp = synth.mamba_inputs(2, 100, 2, 32, 64, 1, False, seed=5)
    _compare(_gpu_m2(inp, "f32", 64, s0=False), _oracle_m2(inp, "f32", s0=False), TOL["f32"])


def test_empty_sequence_returns_initial_state():
    announce("ssd fwd T=0")
    inp = synth.mamba_inputs(2, 0, 2, 16, 16, 1, False, seed=1)
    got = _gpu_m2(inp, "f32", 16)
    assert got["y"].size == 0
    assert np.array_equal(got["s_final"], inp["s0"].astype(np.float32).astype(np.float64))


def test_final_state_not_requested():
    announce("ssd fwd without s_final")
    inp = synth.mamba_inputs(1, 80, 2, 32, 32, 1, False, seed=6)
    t = to_device(inp, "f32", BIG_MAMBA)
    out = bd.ssd_chunk_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["s0"], chunk_len=64, want_final=False)
    torch.cuda.synchronize()
    assert out["s_final"] is None
    _compare({"y": to_numpy(out["y"])}, _oracle_m2(inp, "f32"), TOL["f32"], keys=("y",))


def test_deterministic_across_runs():
    announce("ssd fwd determinism bf16")
    inp = synth.mamba_inputs(2, 256, 8, 64, 128, 1, False, seed=4)
    a = _gpu_m2(inp, "bf16", 64)
    b = _gpu_m2(inp, "bf16", 64)
    for k in ("y", "s_final"):
        assert np.array_equal(a[k], b[k]), k
