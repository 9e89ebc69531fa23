"""GPU parity of ssd_chunk_bwd on long fused chunks (L*M > 64 rows: the
row-blocked chunk kernels), through the C ABI.

* RAW (v, da) rank-M form against the float64 oracle in fp32 (1e-4) and bf16
  (2e-2): two and four 64-row blocks, several heads per B/C group (group sums
  over heads), a shorter last chunk, the generic and the compile-time shapes;
* the full rank-4 MIMO workload (b=2, T=4096, M=4, H=32, P=64, N=128, G=32,
  L=64, bf16) in the launch configuration of the library's default plan,
  every batch element against the oracle and the whole batch through the
  identity <dB, B> = <dv, v> of the exact VJP (y and the final state are
  bilinear in (v, B) apart from the s0 term, which depends on neither);
* s0 = NULL and ds_final = NULL (zeros), in both dtypes;
* edge cases: T = 1, a single short chunk, T = 0, determinism.
"""
import numpy as np
import pytest
import torch

import oracle
from _helpers import rel_maxabs
from gpu_common import BIG_RAW, TOL, announce, to_device, to_numpy
from selective_state_space_vjp_amd import binding as bd
from selective_state_space_vjp_amd import synth

pytestmark = pytest.mark.gpu
RAW_OUTS = ("dv", "d_da", "dB", "dC", "d_s0")


def _gpu_raw(inp, dtype, L, null=()):
    """The chunked backward on the GPU; tensors named in `null` are passed as NULL."""
    t = to_device(inp, dtype, BIG_RAW)
    for k in null:
        t[k] = None
    out = bd.ssd_chunk_bwd(t["v"], t["da"], None, t["B"], t["C"], t["s0"], t["dy"], t["ds_final"], chunk_len=L)
    torch.cuda.synchronize()
    return {k: to_numpy(v) for k, v in out.items()}


def _oracle_raw(inp, dtype):
    c = synth.as_dtype(inp, dtype, "raw")
    return oracle.raw_seq_bwd(c["v"], c["da"], c["B"], c["C"], c["s0"], c["dy"], c["ds_final"])


def _compare(got, ref, keys, tol):
    errs = {k: rel_maxabs(got[k], ref[k]) for k in keys if ref[k].size}
    print("[rel_maxabs]", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert errs and max(errs.values()) < tol, errs
    return errs


BLOCKED_SHAPES = [
    # b, T, M, H, P, N, G, L        fused chunk L*M
    (1, 128, 4, 2, 32, 32, 2, 32),   # 128: two blocks, one head per group
    (1, 200, 4, 4, 16, 32, 2, 64),   # 256: four blocks, two heads per group, last chunk of 8 steps
    (2, 96, 2, 2, 64, 128, 2, 64),   # 128: the compile-time P=64, N=128 instance
    (1, 130, 4, 2, 64, 128, 1, 64),  # 256: P=64, N=128, two heads per group, last chunk of 2 steps
    (1, 72, 4, 3, 48, 16, 3, 48),    # 192: three blocks, odd sizes, last chunk of 24 steps
    (1, 80, 4, 2, 128, 64, 1, 64),   # 256: the largest head dim (P = 128) supported in both dtypes
]


@pytest.mark.parametrize("shape", [(1, 80, 4, 2, 128, 128, 1, 64)])
def test_blocked_largest_bf16_shape(shape):
    """P = N = 128: the largest state the row-blocked path supports (bf16 only)."""
    b, T, M, H, P, N, G, L = shape
    announce(f"ssd blocked raw bf16 largest {shape}")
    inp = synth.raw_inputs(b, T, M, H, P, N, G, seed=11)
    _compare(_gpu_raw(inp, "bf16", L), _oracle_raw(inp, "bf16"), RAW_OUTS, TOL["bf16"])


@pytest.mark.parametrize("shape", [(1, 130, 4, 2, 64, 128, 1, 64), (1, 128, 4, 2, 32, 32, 2, 32)])
@pytest.mark.parametrize("regime", ["no_decay", "slow_decay"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_blocked_decay_regimes(shape, regime, dtype):
    """da = 0 (no decay: every exp factor is 1) and da = -0.005 per step (slow
    decay over the whole sequence), against the default inputs' fast decay."""
    b, T, M, H, P, N, G, L = shape
    announce(f"ssd blocked raw {dtype} {shape} {regime}")
    inp = synth.raw_inputs(b, T, M, H, P, N, G, seed=5 + sum(shape))
    inp["da"][:] = 0.0 if regime == "no_decay" else -0.005
    _compare(_gpu_raw(inp, dtype, L), _oracle_raw(inp, dtype), RAW_OUTS, TOL[dtype])


@pytest.mark.parametrize("shape", BLOCKED_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_blocked_raw_parity(shape, dtype):
    b, T, M, H, P, N, G, L = shape
    announce(f"ssd blocked raw {dtype} {shape}")
    inp = synth.raw_inputs(b, T, M, H, P, N, G, seed=3 + sum(shape))
    _compare(_gpu_raw(inp, dtype, L), _oracle_raw(inp, dtype), RAW_OUTS, TOL[dtype])


def test_blocked_full_mimo_workload_every_batch_element():
    """The full rank-4 MIMO workload in the library's default plan: every
    output element of each batch element against the oracle (per batch
    element), and the identity <dB, B> = <dv, v> over the whole batch."""
    w = synth.WORKLOADS["mimo_chunk"]
    announce("ssd blocked bf16 full MIMO workload b=2 T=4096 M=4 H=32 P=64 N=128 G=32 L=64")
    inp = synth.workload_inputs("mimo_chunk")
    got = _gpu_raw(inp, "bf16", w["L"])
    c = synth.as_dtype(inp, "bf16", "raw")
    lhs = float(np.sum(got["dB"] * c["B"]))
    rhs = float(np.sum(got["dv"] * c["v"]))
    print("[identity] <dB,B> =", lhs, " <dv,v> =", rhs, flush=True)
    assert abs(lhs - rhs) <= 2e-2 * max(abs(rhs), 1e-30) + 1e-3, (lhs, rhs)
    ref = oracle.raw_seq_bwd(c["v"], c["da"], c["B"], c["C"], c["s0"], c["dy"], c["ds_final"])
    for bi in range(w["b"]):
        announce(f"  batch element {bi}")
        _compare({k: v[bi:bi + 1] for k, v in got.items()}, {k: v[bi:bi + 1] for k, v in ref.items()}, RAW_OUTS,
                 TOL["bf16"])


@pytest.mark.parametrize("shape", [(1, 130, 4, 2, 64, 128, 1, 64), (1, 128, 4, 2, 32, 32, 2, 32)])
@pytest.mark.parametrize("null", [("s0",), ("ds_final",), ("s0", "ds_final")])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_blocked_null_initial_state_and_seed(shape, null, dtype):
    """s0 = NULL and ds_final = NULL mean zeros on the row-blocked path too."""
    b, T, M, H, P, N, G, L = shape
    announce(f"ssd blocked raw {dtype} {shape} NULL {null}")
    inp = synth.raw_inputs(b, T, M, H, P, N, G, seed=13 + sum(shape) + len(null))
    zeroed = dict(inp)
    for k in null:
        zeroed[k] = np.zeros_like(inp[k])
    _compare(_gpu_raw(inp, dtype, L, null=null), _oracle_raw(zeroed, dtype), RAW_OUTS, TOL[dtype])


@pytest.mark.parametrize("T", [1, 10, 64])
def test_blocked_short_sequences(T):
    announce(f"ssd blocked short T={T}")
    inp = synth.raw_inputs(1, T, 4, 2, 32, 32, 1, seed=T)
    _compare(_gpu_raw(inp, "f32", 64), _oracle_raw(inp, "f32"), RAW_OUTS, TOL["f32"])


def test_blocked_empty_sequence_returns_seed():
    announce("ssd blocked T=0")
    inp = synth.raw_inputs(1, 0, 4, 2, 16, 16, 1, seed=2)
    got = _gpu_raw(inp, "f32", 32)
    assert np.array_equal(got["d_s0"], inp["ds_final"].astype(np.float32).astype(np.float64))


def test_blocked_deterministic_across_runs():
    announce("ssd blocked determinism bf16")
    inp = synth.raw_inputs(1, 256, 4, 4, 64, 128, 2, seed=5)
    a = _gpu_raw(inp, "bf16", 64)
    b = _gpu_raw(inp, "bf16", 64)
    for k in RAW_OUTS:
        assert np.array_equal(a[k], b[k]), k
