"""GPU parity of ssm_scan_bwd (sequential reverse recurrence) against the
float64 oracle, through the C ABI.

Covers both workloads of this path (Mamba-2 small, Mamba-1 per-state), random
shapes with several groups and ragged checkpoint segments, bf16 storage,
s0 = NULL and ds_final = NULL (zeros), an empty sequence, bitwise equality
across checkpoint intervals (the llama.cpp page's checkpoint-every-K
requirement) and run-to-run determinism.
"""
import numpy as np
import pytest
import torch

import oracle
from _helpers import rel_maxabs
from gpu_common import BIG_MAMBA, TOL, announce, to_device, to_numpy
from selective_state_space_vjp_amd import binding as bd
from selective_state_space_vjp_amd import synth

pytestmark = pytest.mark.gpu
OUTS = ("dx", "d_dt", "dB", "dC", "d_s0")


def _gpu(inp, dtype, ckpt=0, null=()):
    """The sequential backward on the GPU; tensors named in `null` are passed as NULL."""
    t = to_device(inp, dtype, BIG_MAMBA)
    for k in null:
        t[k] = None
    out = bd.ssm_scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["s0"], t["dy"], t["ds_final"],
                          ckpt_every=ckpt)
    torch.cuda.synchronize()
    return {k: to_numpy(v) for k, v in out.items()}


def _oracle(inp, dtype):
    c = synth.as_dtype(inp, dtype, "mamba")
    return oracle.mamba_seq_bwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["s0"], c["dy"], c["ds_final"])


def _compare(got, ref, tol):
    errs = {k: rel_maxabs(got[k], ref[k]) for k in OUTS if ref[k].size}
    print("[rel_maxabs]", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert errs and max(errs.values()) < tol, errs
    return errs


@pytest.mark.parametrize("name", ["mamba2_seq_small", "mamba1_seq"])
def test_workload_parity_fp32(name):
    announce(f"scan_seq workload {name}")
    inp = synth.workload_inputs(name)
    _compare(_gpu(inp, "f32"), _oracle(inp, "f32"), TOL["f32"])


@pytest.mark.parametrize("shape", [
    (2, 37, 4, 20, 5, 2, False, 8),    # P not a multiple of the per-thread block, ragged segment
    (1, 100, 6, 3, 16, 3, True, 7),    # Mamba-1 branch with groups
    (3, 65, 2, 33, 64, 1, False, 16),  # several p groups, N = one wave
    (1, 9, 1, 1, 1, 1, False, 4),
])
def test_random_shapes_fp32(shape):
    b, T, H, P, N, G, per_state, K = shape
    announce(f"scan_seq shape {shape}")
    inp = synth.mamba_inputs(b, T, H, P, N, G, per_state, seed=sum(shape))
    _compare(_gpu(inp, "f32", K), _oracle(inp, "f32"), TOL["f32"])


@pytest.mark.parametrize("per_state", [False, True])
@pytest.mark.parametrize("regime", ["no_decay", "weak_decay_long_steps"])
def test_decay_regimes_fp32(per_state, regime):
    """A = 0 (plain running sums) and A = -0.01 with steps of about 4 (slow
    decay, growing states), for the per-head (Mamba-2) and per-state (Mamba-1)
    decay; the default inputs cover fast decay."""
    announce(f"scan_seq decay {regime} per_state={per_state}")
    inp = synth.mamba_inputs(2, 70, 3, 8, 16, 1, per_state, seed=29)
    if regime == "no_decay":
        inp["A"][:] = 0.0
    else:
        inp["A"][:] = -0.01
        inp["dt"] = inp["dt"] + 6.0
    _compare(_gpu(inp, "f32", 8), _oracle(inp, "f32"), TOL["f32"])


def test_bf16_storage():
    announce("scan_seq bf16 small")
    inp = synth.workload_inputs("mamba2_seq_small")
    _compare(_gpu(inp, "bf16"), _oracle(inp, "bf16"), TOL["bf16"])


def test_empty_sequence_returns_seed():
    announce("scan_seq T=0")
    inp = synth.mamba_inputs(2, 0, 2, 4, 8, 1, False, seed=3)
    got = _gpu(inp, "f32")
    assert np.array_equal(got["d_s0"], inp["ds_final"].astype(np.float32).astype(np.float64))
    assert got["dx"].size == 0


def test_checkpoint_interval_is_bitwise_invisible():
    announce("scan_seq checkpoint K in {1, 16, 64, T}")
    inp = synth.mamba_inputs(2, 200, 4, 8, 16, 2, False, seed=9)
    runs = [_gpu(inp, "f32", K) for K in (1, 16, 64, 200)]
    for r in runs[1:]:
        for k in OUTS:
            assert np.array_equal(r[k], runs[0][k]), k


def test_deterministic_across_runs():
    announce("scan_seq determinism")
    inp = synth.workload_inputs("mamba1_seq")
    a = _gpu(inp, "f32")
    b = _gpu(inp, "f32")
    for k in OUTS:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("per_state", [False, True])
@pytest.mark.parametrize("null", [("s0",), ("ds_final",), ("s0", "ds_final")])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_null_initial_state_and_seed(per_state, null, dtype):
    """s0 = NULL and ds_final = NULL mean zeros (the header's contract)."""
    announce(f"scan_seq NULL {null} per_state={per_state} {dtype}")
    inp = synth.mamba_inputs(2, 75, 4, 8, 16, 2, per_state, seed=41 + len(null))
    zeroed = dict(inp)
    for k in null:
        zeroed[k] = np.zeros_like(inp[k])
    _compare(_gpu(inp, dtype, 16, null=null), _oracle(zeroed, dtype), TOL[dtype])
