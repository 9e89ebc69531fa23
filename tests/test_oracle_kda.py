"""Pins for the KDA gated-delta-rule oracle (oracle.kda_fwd / kda_bwd).

  * a hand-derived two-step worked example (tests/golden/kda_scalar_T2.txt);
  * central finite differences of the float64 forward for all five gradients
    and the initial-state gradient, with a non-zero final-state seed;
  * torch.autograd of an independently written torch forward (F1..F6);
  * homogeneity identities: o is linear in q, and (o, S_T) are jointly linear
    in (v, S0);
  * value columns are independent in the recurrence (a perturbation of one
    column of v changes no other column of o);
  * dropping the residual path from the gated state's gradient (the notes'
    two-path warning) and a wrong GVA head map each fail the FD gate by >= 100x.
"""
import numpy as np
import pytest

import oracle
from _helpers import fd_grads, rel_maxabs, rel_maxabs_probed
from selective_state_space_vjp_amd import synth

FD_GATE = 1e-7
KDA_GRADS = (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"), ("S0", "dS0"))


def _inputs(b, T, H, HV, K, V, seed):
    d = synth.kda_inputs(b, T, H, HV, K, V, seed=seed, nonzero_state=True)
    rng = np.random.default_rng(seed + 1)
    d["dS_final"] = rng.standard_normal(d["S0"].shape)
    return d


def _objective(inp):
    o, Sf = oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["S0"],
                           scale=inp["scale"], nthreads=1)
    return float(np.sum(inp["do"] * o) + np.sum(inp["dS_final"] * Sf))


def _bwd(inp, mutation=oracle.MUT_NONE):
    return oracle.kda_bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["S0"], inp["do"],
                          inp["dS_final"], scale=inp["scale"], mutation=mutation, nthreads=1)


@pytest.mark.parametrize("shape", [(1, 5, 1, 1, 3, 2), (1, 4, 2, 4, 2, 3), (2, 3, 1, 2, 3, 3)])
def test_fd_all_gradients(shape):
    inp = _inputs(*shape, seed=sum(shape))
    fd, counts = fd_grads(_objective, inp, [k for k, _ in KDA_GRADS], eps=1e-5)
    assert all(c > 0 for c in counts.values())
    got = _bwd(inp)
    errs = {g: rel_maxabs_probed(got[g], fd[k]) for k, g in KDA_GRADS}
    assert max(errs.values()) < FD_GATE, errs


def _torch_forward(q, k, v, beta, g, S0, scale):
    """Independent float64 torch forward of F1..F6 with the GVA head map hv -> hv // G."""
    import torch

    b, T, H, K = q.shape
    HV = v.shape[2]
    G = HV // H
    qe = q.repeat_interleave(G, dim=2) * scale
    ke = k.repeat_interleave(G, dim=2)
    S = S0
    outs = []
    for t in range(T):
        Sdec = torch.exp(g[:, t])[..., None] * S
        p = torch.einsum("bhk,bhkv->bhv", ke[:, t], Sdec)
        r = v[:, t] - p
        a = beta[:, t, :, None] * ke[:, t]
        S = Sdec + a[..., None] * r[:, :, None, :]
        outs.append(torch.einsum("bhk,bhkv->bhv", qe[:, t], S))
    return torch.stack(outs, 1), S


def test_autograd_independent_forward():
    import torch

    inp = _inputs(2, 12, 2, 4, 5, 6, seed=8)
    names = tuple(k for k, _ in KDA_GRADS)
    ts = {n: torch.tensor(inp[n], dtype=torch.float64, requires_grad=True) for n in names}
    o, Sf = _torch_forward(ts["q"], ts["k"], ts["v"], ts["beta"], ts["g"], ts["S0"], inp["scale"])
    J = (torch.tensor(inp["do"]) * o).sum() + (torch.tensor(inp["dS_final"]) * Sf).sum()
    auto = torch.autograd.grad(J, [ts[n] for n in names])
    got = _bwd(inp)
    for (k, gname), a in zip(KDA_GRADS, auto):
        assert rel_maxabs(got[gname], a.numpy()) < 1e-12, (k, rel_maxabs(got[gname], a.numpy()))
    o_o, Sf_o = oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["S0"], scale=inp["scale"])
    assert rel_maxabs(o_o, o.detach().numpy()) < 1e-12


def test_homogeneity_identities():
    inp = _inputs(1, 40, 2, 4, 6, 5, seed=12)
    o, Sf = oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["S0"], scale=inp["scale"])
    J = np.sum(inp["do"] * o) + np.sum(inp["dS_final"] * Sf)
    g = _bwd(inp)
    assert np.sum(g["dq"] * inp["q"]) == pytest.approx(np.sum(inp["do"] * o), rel=1e-12)
    assert np.sum(g["dv"] * inp["v"]) + np.sum(g["dS0"] * inp["S0"]) == pytest.approx(J, rel=1e-12)


def test_value_columns_are_independent():
    inp = _inputs(1, 30, 1, 2, 4, 6, seed=14)
    o, _ = oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["S0"], scale=inp["scale"])
    v2 = inp["v"].copy()
    v2[..., 3] += 0.5
    o2, _ = oracle.kda_fwd(inp["q"], inp["k"], v2, inp["beta"], inp["g"], inp["S0"], scale=inp["scale"])
    others = [c for c in range(6) if c != 3]
    assert np.array_equal(o[..., others], o2[..., others])
    assert not np.allclose(o[..., 3], o2[..., 3])


@pytest.mark.parametrize("mutation", [oracle.MUT_DROP_KDR, oracle.MUT_WRONG_GVA])
def test_mutations_are_caught(mutation):
    inp = _inputs(1, 4, 2, 4, 2, 3, seed=31)
    fd, _ = fd_grads(_objective, inp, [k for k, _ in KDA_GRADS], eps=1e-5)
    bad = _bwd(inp, mutation)
    errs = {g: rel_maxabs_probed(bad[g], fd[k]) for k, g in KDA_GRADS}
    assert max(errs.values()) > 100 * FD_GATE, errs


def test_golden_hand_derived_example():
    from test_oracle_mamba import _eval_expr
    import os

    path = os.path.join(os.path.dirname(__file__), "golden", "kda_scalar_T2.txt")
    gi, go = {}, {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        kind, name, idx, expr = line.split(None, 3)
        (gi if kind == "input" else go).setdefault(name, {})[idx] = _eval_expr(expr)

    def seq(d, name, shape):
        return np.array([d[name]["0"], d[name]["1"]]).reshape(shape)
    inp = dict(q=seq(gi, "q", (1, 2, 1, 1)), k=seq(gi, "k", (1, 2, 1, 1)), v=seq(gi, "v", (1, 2, 1, 1)),
               beta=seq(gi, "beta", (1, 2, 1)), g=seq(gi, "g", (1, 2, 1, 1)), S0=np.full((1, 1, 1, 1), gi["S0"]["-"]),
               do=seq(gi, "do", (1, 2, 1, 1)), dS_final=np.full((1, 1, 1, 1), gi["dS_final"]["-"]),
               scale=gi["scale"]["-"])
    o, Sf = oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["S0"], scale=inp["scale"])
    got = _bwd(inp)
    checked = 0
    for t in ("0", "1"):
        ti = int(t)
        for name, val in (("o", o[0, ti, 0, 0]), ("dq", got["dq"][0, ti, 0, 0]), ("dk", got["dk"][0, ti, 0, 0]),
                          ("dv", got["dv"][0, ti, 0, 0]), ("dg", got["dg"][0, ti, 0, 0]),
                          ("dbeta", got["dbeta"][0, ti, 0])):
            assert val == pytest.approx(go[name][t], abs=1e-14), (name, t)
            checked += 1
    assert Sf[0, 0, 0, 0] == pytest.approx(go["S_final"]["-"], abs=1e-14)
    assert got["dS0"][0, 0, 0, 0] == pytest.approx(go["dS0"]["-"], abs=1e-14)
    assert checked == 12
