"""ssd_chunk_bwd_noalloc (the chunked backward on the library's own device
array, for callers that cannot allocate) against ssd_chunk_bwd, through the C
ABI: two calls in a row, the second with a smaller input (the array keeps
the first call's contents, which the second must not depend on), in both
dtypes and both input forms, the largest workspace the array holds, and the
refusal of a shape whose workspace exceeds it.  The two entry points run the
same kernels on the same inputs, so their outputs must be bitwise equal.
"""
import numpy as np
import pytest
import torch

from gpu_common import BIG_MAMBA, BIG_RAW, announce, to_device
from selective_state_space_vjp_amd import binding as bd
from selective_state_space_vjp_amd import synth

pytestmark = pytest.mark.gpu


def _pair(inp, dtype, L, raw):
    t = to_device(inp, dtype, BIG_RAW if raw else BIG_MAMBA)
    xv, dtda, A = (t["v"], t["da"], None) if raw else (t["x"], t["dt"], t["A"])
    ref = bd.ssd_chunk_bwd(xv, dtda, A, t["B"], t["C"], t["s0"], t["dy"], t["ds_final"], chunk_len=L)
    out = {k: torch.full_like(v, float("nan")) for k, v in ref.items()}
    got = bd.ssd_chunk_bwd_noalloc(xv, dtda, A, t["B"], t["C"], t["s0"], t["dy"], t["ds_final"], chunk_len=L,
                                   out=out)
    torch.cuda.synchronize()
    return got, ref


def _equal(got, ref):
    for k in ref:
        a, b = got[k].cpu(), ref[k].cpu()
        assert torch.equal(a, b), (k, float((a.double() - b.double()).abs().max()))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_call_twice_second_smaller(dtype):
    announce(f"noalloc {dtype}: b=2 T=300 H=8 P=64 N=128, then b=1 T=70 H=3")
    big = synth.mamba_inputs(2, 300, 8, 64, 128, 1, False, seed=21)
    _equal(*_pair(big, dtype, 64, False))
    small = synth.mamba_inputs(1, 70, 3, 64, 128, 1, False, seed=22)
    _equal(*_pair(small, dtype, 64, False))


def test_noalloc_raw_rank4_and_general_shapes():
    announce("noalloc raw rank-4 b=1 T=130 H=2 P=64 N=128, then Mamba-2 b=1 T=96 H=4 P=32 N=32 G=2 L=32")
    _equal(*_pair(synth.raw_inputs(1, 130, 4, 2, 64, 128, 1, seed=23), "bf16", 64, True))
    _equal(*_pair(synth.mamba_inputs(1, 96, 4, 32, 32, 2, False, seed=24), "f32", 32, False))


def test_noalloc_largest_supported_then_refused():
    """One 4096-step sequence of the Mamba-2 head shape (H=32, P=64, N=128,
    bf16) fits the array; twice the tokens do not and are refused before
    anything runs."""
    w = synth.WORKLOADS["mamba2_chunk"]
    announce("noalloc bf16 b=1 T=4096 H=32 P=64 N=128 (largest), then b=2 refused")
    inp = synth.mamba_inputs(1, w["T"], w["H"], w["P"], w["N"], 1, False, seed=25)
    _equal(*_pair(inp, "bf16", w["L"], False))
    t = to_device(synth.mamba_inputs(2, w["T"], w["H"], w["P"], w["N"], 1, False, seed=26), "bf16", BIG_MAMBA)
    out = {"dx": torch.empty_like(t["x"]), "d_dt": torch.empty_like(t["dt"]), "dB": torch.empty_like(t["B"]),
           "dC": torch.empty_like(t["C"]), "d_s0": torch.empty_like(t["s0"])}
    with pytest.raises(bd.SsmVjpError) as e:
        bd.ssd_chunk_bwd_noalloc(t["x"], t["dt"], t["A"], t["B"], t["C"], t["s0"], t["dy"], t["ds_final"],
                                 chunk_len=w["L"], out=out)
    assert e.value.status == bd.EWORKSPACE
    # the refused call enqueued nothing: a following call is still exact
    _equal(*_pair(synth.mamba_inputs(1, 200, 4, 64, 128, 1, False, seed=27), "bf16", 64, False))
