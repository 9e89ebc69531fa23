"""The debug finiteness mode (environment variable SSMVJP_CHECK_FINITE): every
entry point scans the outputs it wrote and returns SSMVJP_ENONFINITE when one
holds a NaN or an infinity.  A NaN is planted in one input element (the host
builds the inputs; the kernels only do arithmetic on it), and the same call
on clean inputs must return OK with outputs identical to the mode off."""
import numpy as np
import pytest
import torch

from gpu_common import BIG_MAMBA, BIG_RAW, announce, to_device
from selective_state_space_vjp_amd import binding as bd
from selective_state_space_vjp_amd import synth

pytestmark = pytest.mark.gpu


def _expect_nonfinite(fn):
    with pytest.raises(bd.SsmVjpError) as e:
        fn()
    assert e.value.status == bd.ENONFINITE


def _same(a, b):
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("case", ["seq_f32", "chunk16_bf16", "chunk_f32", "raw_bf16", "blocked_bf16"])
def test_nonfinite_outputs_are_reported(case, monkeypatch):
    announce(f"finite check {case}")
    raw = case.startswith("raw") or case.startswith("blocked")
    dtype = "bf16" if case.endswith("bf16") else "f32"
    if raw:
        M, L = (4, 64) if case.startswith("blocked") else (2, 16)
        inp = synth.raw_inputs(1, 100, M, 2, 64, 128, 1, seed=3)
    else:
        inp = synth.mamba_inputs(1, 150, 3, 64 if case != "seq_f32" else 8, 128 if case != "seq_f32" else 16, 1,
                                 False, seed=2)
        L = 64 if case == "chunk16_bf16" else 32

    def run(d):
        t = to_device(d, dtype, BIG_RAW if raw else BIG_MAMBA)
        if raw:
            return bd.ssd_chunk_bwd(t["v"], t["da"], None, t["B"], t["C"], t["s0"], t["dy"], t["ds_final"],
                                    chunk_len=L)
        if case == "seq_f32":
            return bd.ssm_scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["s0"], t["dy"], t["ds_final"])
        return bd.ssd_chunk_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["s0"], t["dy"], t["ds_final"],
                                chunk_len=L)

    monkeypatch.delenv("SSMVJP_CHECK_FINITE", raising=False)
    plain = run(inp)
    torch.cuda.synchronize()
    monkeypatch.setenv("SSMVJP_CHECK_FINITE", "1")
    _same(run(inp), plain)
    bad = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    key = "v" if raw else "x"
    bad[key][0, 40, ...] = np.nan
    _expect_nonfinite(lambda: run(bad))
    monkeypatch.delenv("SSMVJP_CHECK_FINITE", raising=False)
    run(bad)  # the mode off: no scan, no error
    torch.cuda.synchronize()


def test_nonfinite_delta_rule_and_forward(monkeypatch):
    announce("finite check delta rule and chunked forward")
    inp = synth.kda_inputs(1, 30, 1, 2, 128, 32, seed=4)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).float().cuda() for k, v in inp.items()
         if isinstance(v, np.ndarray)}
    monkeypatch.setenv("SSMVJP_CHECK_FINITE", "1")
    bd.delta_rule_bwd(t["q"], t["k"], t["v"], t["beta"], t["g"], t["S0"], t["do"], scale=inp["scale"])
    t["do"][0, 7, 1, 3] = float("inf")
    _expect_nonfinite(lambda: bd.delta_rule_bwd(t["q"], t["k"], t["v"], t["beta"], t["g"], t["S0"], t["do"],
                                                scale=inp["scale"]))
    m = to_device(synth.mamba_inputs(1, 130, 2, 64, 128, 1, False, seed=5), "bf16", BIG_MAMBA)
    bd.ssd_chunk_fwd(m["x"], m["dt"], m["A"], m["B"], m["C"], m["s0"], chunk_len=64)
    m["B"][0, 99, 0, 5] = float("nan")
    _expect_nonfinite(lambda: bd.ssd_chunk_fwd(m["x"], m["dt"], m["A"], m["B"], m["C"], m["s0"], chunk_len=64))
    torch.cuda.synchronize()
