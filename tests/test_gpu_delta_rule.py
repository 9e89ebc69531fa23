"""GPU parity of delta_rule_bwd (KDA gated delta-rule backward) through the C ABI.

* random shapes against the float64 oracle (fp32, relative max-abs 1e-4):
  several value slices, GVA groups of 1, 2 and 4, sequences that end inside a
  checkpoint segment, non-zero initial state and final-state gradient;
* T = 1 and T = 0 (dS0 is then the final-state gradient);
* S0 = NULL and dS_final = NULL (zeros);
* the full workload: qk heads 0, 7 and 15 of both batch elements, every
  output (dq, dk, dv, dg, dbeta, dS0) against the oracle;
* the full workload (b=2, T=4096, H=16, HV=32, K=V=128) in the launch
  configuration the benchmark times: batch element 0, qk head 0 (value heads
  0..1) against the oracle on that slice of the inputs, and the whole
  output through the identity <dq, q> = <dv, v> of the exact VJP (both equal
  <do, o> when S0 = 0, since o is linear in q and in (v, S0));
* bitwise determinism across runs.
"""
import numpy as np
import pytest
import torch

import oracle
from _helpers import rel_maxabs
from gpu_common import announce, to_numpy
from selective_state_space_vjp_amd import binding as bd
from selective_state_space_vjp_amd import synth

pytestmark = pytest.mark.gpu
OUTS = ("dq", "dk", "dv", "dg", "dbeta", "dS0")
TOL = 1e-4


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32).to("cuda:0").contiguous()


def _gpu(inp, dSf=None, null_S0=False):
    t = {k: _dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
    if null_S0:
        t["S0"] = None
    out = bd.delta_rule_bwd(t["q"], t["k"], t["v"], t["beta"], t["g"], t["S0"], t["do"],
                            None if dSf is None else _dev(dSf), scale=inp["scale"])
    torch.cuda.synchronize()
    return {k: to_numpy(v) for k, v in out.items() if v is not None}


def _f32(inp):
    return {k: (v.astype(np.float32).astype(np.float64) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}


def _oracle(c, dSf=None):
    return oracle.kda_bwd(c["q"], c["k"], c["v"], c["beta"], c["g"], c["S0"], c["do"], dSf, scale=c["scale"])


def _compare(got, ref, keys=OUTS, tol=TOL):
    errs = {k: rel_maxabs(got[k], ref[k]) for k in keys if ref[k].size}
    print("[rel_maxabs]", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert errs and max(errs.values()) < tol, errs
    return errs


SHAPES = [
    # b, T, H, HV, V, nonzero S0, nonzero dS_final
    (1, 40, 2, 4, 32, False, False),
    (2, 37, 1, 2, 64, True, True),
    (1, 24, 2, 2, 128, True, False),
    (1, 19, 1, 4, 96, False, True),
    (1, 1, 1, 1, 32, True, True),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_delta_rule_parity(shape):
    b, T, H, HV, V, s0, dsf = shape
    announce(f"delta_rule {shape}")
    inp = synth.kda_inputs(b, T, H, HV, 128, V, seed=T + 7 * HV + V, nonzero_state=s0)
    dSf = np.random.default_rng(T).standard_normal((b, HV, 128, V)) if dsf else None
    c = _f32(inp)
    dSf32 = None if dSf is None else dSf.astype(np.float32).astype(np.float64)
    _compare(_gpu(inp, dSf), _oracle(c, dSf32))


@pytest.mark.parametrize("case", ["no_decay", "no_write", "full_write"])
def test_delta_rule_degenerate_gates(case):
    """g = 0 (no decay of the state), beta = 0 (the state never changes: the
    write path of every step is zero) and beta = 1 (each step fully replaces
    the state's component along k), with non-zero S0 and dS_final."""
    announce(f"delta_rule degenerate {case}")
    inp = synth.kda_inputs(1, 40, 2, 4, 128, 64, seed=3, nonzero_state=True)
    if case == "no_decay":
        inp["g"][:] = 0.0
    else:
        inp["beta"][:] = 0.0 if case == "no_write" else 1.0
    dSf = np.random.default_rng(5).standard_normal((1, 4, 128, 64))
    _compare(_gpu(inp, dSf), _oracle(_f32(inp), dSf.astype(np.float32).astype(np.float64)))


def test_delta_rule_empty_sequence():
    announce("delta_rule T=0")
    inp = synth.kda_inputs(2, 0, 1, 2, 128, 32, seed=1)
    dSf = np.random.default_rng(5).standard_normal((2, 2, 128, 32))
    got = _gpu(inp, dSf)
    assert np.array_equal(got["dS0"], dSf.astype(np.float32).astype(np.float64))


def test_delta_rule_full_workload_slice_and_identity():
    w = synth.WORKLOADS["kda"]
    announce("delta_rule full workload b=2 T=4096 H=16 HV=32 K=V=128")
    inp = synth.workload_inputs("kda")
    got = _gpu(inp)
    c = _f32(inp)
    # whole output: <dq, q> = <dv, v> (S0 = 0)
    lhs = float(np.sum(got["dq"] * c["q"]))
    rhs = float(np.sum(got["dv"] * c["v"]))
    print(f"[identity] <dq,q>={lhs:.6e} <dv,v>={rhs:.6e}", flush=True)
    assert abs(lhs - rhs) <= 1e-4 * max(abs(rhs), 1.0), (lhs, rhs)
    # batch element 0, qk head 0 and its value heads against the oracle
    grp = w["HV"] // w["H"]
    nh, nv = 1, grp
    sl = {"q": c["q"][:1, :, :nh], "k": c["k"][:1, :, :nh], "v": c["v"][:1, :, :nv], "beta": c["beta"][:1, :, :nv],
          "g": c["g"][:1, :, :nv], "S0": c["S0"][:1, :nv], "do": c["do"][:1, :, :nv], "scale": c["scale"]}
    ref = _oracle(sl)
    sub = {"dq": got["dq"][:1, :, :nh], "dk": got["dk"][:1, :, :nh], "dv": got["dv"][:1, :, :nv],
           "dg": got["dg"][:1, :, :nv], "dbeta": got["dbeta"][:1, :, :nv], "dS0": got["dS0"][:1, :nv]}
    _compare(sub, ref)


@pytest.mark.parametrize("null_S0,null_dSf", [(True, False), (False, True), (True, True)])
def test_delta_rule_null_state_and_seed(null_S0, null_dSf):
    """S0 = NULL and dS_final = NULL mean zeros (the header's contract)."""
    announce(f"delta_rule NULL S0={null_S0} dS_final={null_dSf}")
    inp = synth.kda_inputs(2, 45, 2, 4, 128, 64, seed=17, nonzero_state=True)
    dSf = np.random.default_rng(19).standard_normal((2, 4, 128, 64))
    c = _f32(inp)
    if null_S0:
        c["S0"] = np.zeros_like(c["S0"])
    got = _gpu(inp, None if null_dSf else dSf, null_S0=null_S0)
    _compare(got, _oracle(c, None if null_dSf else dSf.astype(np.float32).astype(np.float64)))


def test_delta_rule_full_workload_heads_of_every_batch_element():
    """The full workload: qk heads 0, 7 and 15 (each with its value heads) of
    both batch elements against the oracle, every output including dk, dg and
    dbeta, which no identity covers."""
    w = synth.WORKLOADS["kda"]
    announce("delta_rule full workload b=2 T=4096 H=16 HV=32 K=V=128, qk heads 0, 7, 15 of each batch element")
    inp = synth.workload_inputs("kda")
    got = _gpu(inp)
    c = _f32(inp)
    grp = w["HV"] // w["H"]
    picks = [(bi, h) for bi in range(w["b"]) for h in (0, 7, w["H"] - 1)]
    # the picked (batch element, qk head) slices stacked along the batch axis
    def qk(a):
        return np.stack([a[bi, :, h] for bi, h in picks])[:, :, None]

    def vh(a):
        return np.stack([a[bi, :, grp * h:grp * (h + 1)] for bi, h in picks])

    sl = {"q": qk(c["q"]), "k": qk(c["k"]), "v": vh(c["v"]), "beta": vh(c["beta"]), "g": vh(c["g"]),
          "do": vh(c["do"]), "S0": np.stack([c["S0"][bi, grp * h:grp * (h + 1)] for bi, h in picks]),
          "scale": c["scale"]}
    ref = _oracle(sl)
    sub = {"dq": qk(got["dq"]), "dk": qk(got["dk"]), "dv": vh(got["dv"]), "dg": vh(got["dg"]),
           "dbeta": vh(got["dbeta"]), "dS0": np.stack([got["dS0"][bi, grp * h:grp * (h + 1)] for bi, h in picks])}
    for i, (bi, h) in enumerate(picks):
        announce(f"  batch element {bi}, qk head {h}")
        _compare({k: v[i:i + 1] for k, v in sub.items()}, {k: v[i:i + 1] for k, v in ref.items()})


def test_delta_rule_deterministic():
    announce("delta_rule determinism")
    inp = synth.kda_inputs(1, 100, 2, 4, 128, 128, seed=11, nonzero_state=True)
    a = _gpu(inp)
    b = _gpu(inp)
    for k in OUTS:
        assert np.array_equal(a[k], b[k]), k
