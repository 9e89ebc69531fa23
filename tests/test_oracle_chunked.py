"""Pins for the chunked SSD oracle (oracle.ssd_chunk_fwd / ssd_chunk_bwd /
ssd_mamba2_bwd) and the rank-M sequential form it re-associates.

  * the chunked forward (K1..K5) equals the sequential rank-M recurrence for
    every chunk length, including 1 (K5 reduces to the diagonal), T, and a
    shorter last chunk;
  * the chunked backward equals the sequential store-all backward to 1e-12;
  * both backwards equal central finite differences of the sequential forward
    and torch.autograd of an independently written torch forward;
  * homogeneity identities; MIMO rank 1 with per-head B/C equals Mamba-2;
  * every dropped d_cumA source, a prefix-sum K1 backward, the triu(0) mask
    and a missing mimo_rank reduction each fail the FD gate by >= 100x.
"""
import numpy as np
import pytest

import oracle
from _helpers import fd_grads, rel_maxabs, rel_maxabs_probed
from selective_state_space_vjp_amd import synth

FD_GATE = 1e-7
RAW_GRADS = (("v", "dv"), ("da", "d_da"), ("B", "dB"), ("C", "dC"), ("s0", "d_s0"))


def _raw_objective(inp):
    y, sf = oracle.raw_seq_fwd(inp["v"], inp["da"], inp["B"], inp["C"], inp["s0"], nthreads=1)
    return float(np.sum(inp["dy"] * y) + np.sum(inp["ds_final"] * sf))


def _chunk_bwd(inp, L, mutation=oracle.MUT_NONE):
    return oracle.ssd_chunk_bwd(inp["v"], inp["da"], inp["B"], inp["C"], inp["s0"], inp["dy"],
                                inp["ds_final"], L, mutation=mutation, nthreads=1)


def _seq_bwd(inp):
    return oracle.raw_seq_bwd(inp["v"], inp["da"], inp["B"], inp["C"], inp["s0"], inp["dy"],
                              inp["ds_final"], nthreads=1)


@pytest.mark.parametrize("M,G,H", [(1, 1, 2), (2, 2, 2), (3, 1, 3), (4, 2, 4)])
@pytest.mark.parametrize("L", [1, 2, 3, 4, 7, 24])
def test_chunked_forward_equals_sequential(M, G, H, L):
    inp = synth.raw_inputs(2, 24, M, H, 3, 4, G, seed=L + 10 * M)
    y_s, sf_s = oracle.raw_seq_fwd(inp["v"], inp["da"], inp["B"], inp["C"], inp["s0"])
    y_c, sf_c = oracle.ssd_chunk_fwd(inp["v"], inp["da"], inp["B"], inp["C"], inp["s0"], L)
    assert rel_maxabs(y_c, y_s) < 1e-12
    assert rel_maxabs(sf_c, sf_s) < 1e-12


@pytest.mark.parametrize("M,G,H", [(1, 1, 2), (2, 2, 2), (4, 1, 4), (2, 2, 4)])
@pytest.mark.parametrize("L", [1, 3, 5, 8, 20])
def test_chunked_backward_equals_sequential(M, G, H, L):
    inp = synth.raw_inputs(2, 20, M, H, 3, 5, G, seed=3 + L + M)
    gs = _seq_bwd(inp)
    gc = _chunk_bwd(inp, L)
    for _, k in RAW_GRADS:
        assert rel_maxabs(gc[k], gs[k]) < 1e-12, (k, rel_maxabs(gc[k], gs[k]))


@pytest.mark.parametrize("M,L", [(1, 4), (2, 3), (3, 8)])
def test_fd_raw_backwards(M, L):
    inp = synth.raw_inputs(1, 8, M, 2, 2, 3, 1, seed=40 + M)
    fd, counts = fd_grads(_raw_objective, inp, [k for k, _ in RAW_GRADS], eps=1e-5)
    assert all(c > 0 for c in counts.values())
    for got in (_seq_bwd(inp), _chunk_bwd(inp, L)):
        errs = {g: rel_maxabs_probed(got[g], fd[k]) for k, g in RAW_GRADS}
        assert max(errs.values()) < FD_GATE, errs


def _torch_raw_forward(v, da, B, C, s0):
    """Independent float64 torch forward of the rank-M recurrence (for autograd)."""
    import torch

    b, T, M, H, P = v.shape
    G = B.shape[3]
    Bh = B.repeat_interleave(H // G, dim=3)
    Ch = C.repeat_interleave(H // G, dim=3)
    s = s0
    ys = []
    for t in range(T):
        s = torch.exp(da[:, t, :, None, None]) * s + torch.einsum("bmhp,bmhn->bhpn", v[:, t], Bh[:, t])
        ys.append(torch.einsum("bhpn,bmhn->bmhp", s, Ch[:, t]))
    return torch.stack(ys, 1), s


@pytest.mark.parametrize("M,G,L", [(1, 1, 8), (4, 2, 16), (2, 1, 5)])
def test_autograd_independent_forward(M, G, L):
    import torch

    inp = synth.raw_inputs(2, 40, M, 4, 3, 6, G, seed=70 + M)
    ts = {k: torch.tensor(v, dtype=torch.float64, requires_grad=k in ("v", "da", "B", "C", "s0"))
          for k, v in inp.items()}
    y, sf = _torch_raw_forward(ts["v"], ts["da"], ts["B"], ts["C"], ts["s0"])
    J = (ts["dy"] * y).sum() + (ts["ds_final"] * sf).sum()
    auto = torch.autograd.grad(J, [ts[k] for k, _ in RAW_GRADS])
    got = _chunk_bwd(inp, L)
    for (k, g), a in zip(RAW_GRADS, auto):
        assert rel_maxabs(got[g], a.numpy()) < 1e-12, (k, rel_maxabs(got[g], a.numpy()))


def test_homogeneity_identities_chunked():
    inp = synth.raw_inputs(1, 64, 2, 4, 4, 8, 2, seed=91)
    y, sf = oracle.raw_seq_fwd(inp["v"], inp["da"], inp["B"], inp["C"], inp["s0"])
    J = np.sum(inp["dy"] * y) + np.sum(inp["ds_final"] * sf)
    g = _chunk_bwd(inp, 16)
    vdv = np.sum(g["dv"] * inp["v"])
    assert vdv + np.sum(g["d_s0"] * inp["s0"]) == pytest.approx(J, rel=1e-12)
    assert np.sum(g["dC"] * inp["C"]) == pytest.approx(np.sum(inp["dy"] * y), rel=1e-12)
    assert np.sum(g["dB"] * inp["B"]) == pytest.approx(vdv, rel=1e-12)


@pytest.mark.parametrize("L", [1, 8, 16, 64, 50])
@pytest.mark.parametrize("G", [1, 2])
def test_mamba2_chunked_equals_sequential(L, G):
    inp = synth.mamba_inputs(2, 64, 4, 3, 5, G, False, seed=17 + L)
    gs = oracle.mamba_seq_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["s0"], inp["dy"],
                              inp["ds_final"])
    gc = oracle.ssd_mamba2_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["s0"], inp["dy"],
                               inp["ds_final"], L)
    for k in ("dx", "d_dt", "dB", "dC", "d_s0"):
        assert rel_maxabs(gc[k], gs[k]) < 1e-12, (k, rel_maxabs(gc[k], gs[k]))


def test_mimo_rank1_per_head_bc_equals_mamba2_form():
    """RAW rank 1 with v = x*delta, da = delta*A_h is the Mamba-2 scan; the chain
    rule back to (x, dt) then gives the Mamba-2 gradients."""
    inp = synth.mamba_inputs(1, 32, 3, 4, 5, 3, False, seed=23)
    delta = np.logaddexp(0.0, inp["dt"])
    v = (inp["x"] * delta[..., None])[:, :, None]
    da = delta * inp["A"][None, None, :]
    raw = _chunk_bwd(dict(v=v, da=da, B=inp["B"][:, :, None], C=inp["C"][:, :, None], s0=inp["s0"],
                          dy=inp["dy"][:, :, None], ds_final=inp["ds_final"]), 8)
    ref = oracle.mamba_seq_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["s0"], inp["dy"],
                               inp["ds_final"])
    assert rel_maxabs(raw["dv"][:, :, 0] * delta[..., None], ref["dx"]) < 1e-12
    assert rel_maxabs(raw["dB"][:, :, 0], ref["dB"]) < 1e-12
    assert rel_maxabs(raw["dC"][:, :, 0], ref["dC"]) < 1e-12
    assert rel_maxabs(raw["d_s0"], ref["d_s0"]) < 1e-12


CHUNK_MUTATIONS = [oracle.MUT_DROP_BLUE_DA, oracle.MUT_DROP_ORANGE_DA, oracle.MUT_DROP_K3_DA,
                   oracle.MUT_DROP_K4_DA, oracle.MUT_PREFIX_K1, oracle.MUT_STRICT_MASK,
                   oracle.MUT_NO_M_REDUCE]


@pytest.mark.parametrize("mutation", CHUNK_MUTATIONS)
def test_chunked_mutations_are_caught(mutation):
    inp = synth.raw_inputs(1, 8, 2, 2, 2, 3, 1, seed=55)
    fd, _ = fd_grads(_raw_objective, inp, [k for k, _ in RAW_GRADS], eps=1e-5)
    bad = _chunk_bwd(inp, 4, mutation)
    errs = {g: rel_maxabs_probed(bad[g], fd[k]) for k, g in RAW_GRADS}
    assert max(errs.values()) > 100 * FD_GATE, errs


@pytest.mark.parametrize("mutation", [oracle.MUT_DROP_DA_PATH, oracle.MUT_ZERO_SEED, oracle.MUT_DROP_SOFTPLUS])
def test_mamba2_chunked_chain_mutations_are_caught(mutation):
    inp = synth.mamba_inputs(1, 12, 2, 2, 3, 1, False, seed=21)
    ref = oracle.mamba_seq_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["s0"], inp["dy"],
                               inp["ds_final"])
    bad = oracle.ssd_mamba2_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["s0"], inp["dy"],
                                inp["ds_final"], 4, mutation=mutation)
    assert max(rel_maxabs(bad[k], ref[k]) for k in ("dx", "d_dt", "dB", "dC", "d_s0")) > 1e-3
