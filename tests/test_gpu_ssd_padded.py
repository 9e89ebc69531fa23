"""GPU parity of the chunked backward and forward at head dims and state sizes
that are not multiples of 16 (run on a zero-padded copy of the problem).

* the small Mamba-2 workload (b=1, T=64, H=2, P=4, N=8) through the chunked
  path with chunk lengths 16 and 64: against the float64 oracle (fp32 1e-4,
  bf16 2e-2) and against the GPU's own sequential path in fp32 (1e-5);
* odd P and N in the Mamba-2 and RAW rank-M forms, several groups, a short
  last chunk, the row-blocked path (L*M > 64), NULL s0 / ds_final, the dA
  variant, the two-stage split, and the chunked forward.
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
M2_OUTS = ("dx", "d_dt", "dB", "dC", "d_s0")
RAW_OUTS = ("dv", "d_da", "dB", "dC", "d_s0")


def _compare(got, ref, keys, tol):
    errs = {k: rel_maxabs(got[k], ref[k]) for k in keys if ref[k].size}
    print("[rel_maxabs]", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert errs and max(errs.values()) < tol, errs
    return errs


def _chunked(inp, dtype, L, null=(), want_dA=False):
    t = to_device(inp, dtype, BIG_MAMBA)
    for k in null:
        t[k] = None
    out = bd.ssd_chunk_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["s0"], t["dy"], t["ds_final"], chunk_len=L,
                           want_dA=want_dA)
    torch.cuda.synchronize()
    return {k: to_numpy(v) for k, v in out.items()}


def _sequential(inp, dtype):
    t = to_device(inp, dtype, BIG_MAMBA)
    out = bd.ssm_scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["s0"], t["dy"], t["ds_final"])
    torch.cuda.synchronize()
    return {k: to_numpy(v) for k, v in out.items()}


def _oracle(inp, dtype):
    c = synth.as_dtype(inp, dtype, "mamba")
    return oracle.mamba_seq_bwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["s0"], c["dy"], c["ds_final"])


@pytest.mark.parametrize("L", [16, 64])
def test_small_workload_chunked_matches_sequential_and_oracle(L):
    announce(f"padded chunked small Mamba-2 workload (P=4, N=8), L={L}")
    inp = synth.workload_inputs("mamba2_seq_small")
    got = _chunked(inp, "f32", L)
    _compare(got, _sequential(inp, "f32"), M2_OUTS, 1e-5)
    _compare(got, _oracle(inp, "f32"), M2_OUTS, TOL["f32"])
    _compare(_chunked(inp, "bf16", L), _oracle(inp, "bf16"), M2_OUTS, TOL["bf16"])


PAD_SHAPES = [
    # b, T, H, P, N, G, L
    (2, 100, 4, 20, 40, 2, 32),
    (1, 77, 3, 7, 5, 1, 16),
    (1, 130, 2, 50, 120, 1, 64),
    (2, 65, 2, 1, 1, 2, 16),
]


@pytest.mark.parametrize("shape", PAD_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_padded_mamba2_parity(shape, dtype):
    b, T, H, P, N, G, L = shape
    announce(f"padded ssd mamba2 {dtype} {shape}")
    inp = synth.mamba_inputs(b, T, H, P, N, G, False, seed=sum(shape))
    _compare(_chunked(inp, dtype, L), _oracle(inp, dtype), M2_OUTS, TOL[dtype])


@pytest.mark.parametrize("null", [("s0",), ("ds_final",), ("s0", "ds_final")])
def test_padded_null_states(null):
    announce(f"padded ssd NULL {null}")
    inp = synth.mamba_inputs(1, 90, 2, 12, 20, 1, False, seed=31)
    zeroed = dict(inp)
    for k in null:
        zeroed[k] = np.zeros_like(inp[k])
    _compare(_chunked(inp, "f32", 32, null=null), _oracle(zeroed, "f32"), M2_OUTS, TOL["f32"])


def test_padded_dA_and_stage_split():
    announce("padded ssd dA variant and states/grads split")
    inp = synth.mamba_inputs(2, 96, 4, 6, 10, 2, False, seed=37)
    got = _chunked(inp, "f32", 32, want_dA=True)
    ref = _oracle(inp, "f32")
    _compare(got, ref, M2_OUTS + ("dA",), TOL["f32"])
    t = to_device(inp, "f32", BIG_MAMBA)
    call = bd.SsdCall(t["x"], t["dt"], t["A"], t["B"], t["C"], t["s0"], t["dy"], t["ds_final"], chunk_len=32)
    call.states()
    call.grads()
    torch.cuda.synchronize()
    split = {k: to_numpy(v) for k, v in call.out.items()}
    for k in M2_OUTS:
        assert np.array_equal(split[k], got[k]), k


@pytest.mark.parametrize("shape", [(1, 64, 2, 2, 12, 24, 1, 16), (1, 128, 4, 2, 24, 40, 1, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_padded_raw_rank_m_parity(shape, dtype):
    """RAW (v, da) rank-M form; the second shape has a fused chunk of 256 rows
    (the row-blocked kernels) on the padded problem."""
    b, T, M, H, P, N, G, L = shape
    announce(f"padded ssd raw {dtype} {shape}")
    inp = synth.raw_inputs(b, T, M, H, P, N, G, seed=sum(shape))
    t = to_device(inp, dtype, BIG_RAW)
    out = bd.ssd_chunk_bwd(t["v"], t["da"], None, t["B"], t["C"], t["s0"], t["dy"], t["ds_final"], chunk_len=L)
    torch.cuda.synchronize()
    got = {k: to_numpy(v) for k, v in out.items()}
    c = synth.as_dtype(inp, dtype, "raw")
    ref = oracle.raw_seq_bwd(c["v"], c["da"], c["B"], c["C"], c["s0"], c["dy"], c["ds_final"])
    _compare(got, ref, RAW_OUTS, TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_padded_forward(dtype):
    announce(f"padded chunked forward {dtype}")
    inp = synth.mamba_inputs(2, 150, 3, 12, 8, 1, False, seed=41)
    t = to_device(inp, dtype, BIG_MAMBA)
    out = bd.ssd_chunk_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["s0"], chunk_len=64)
    torch.cuda.synchronize()
    c = synth.as_dtype(inp, dtype, "mamba")
    y, sf = oracle.mamba_seq_fwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["s0"])
    _compare({"y": to_numpy(out["y"]), "s_final": to_numpy(out["s_final"])}, {"y": y, "s_final": sf},
             ("y", "s_final"), TOL[dtype])
