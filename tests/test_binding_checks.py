"""Host-side argument checks of the Python binding.

The C entry points see only pointers, so a tensor of the wrong size would be
read or written out of bounds on the GPU.  The binding must refuse every
mismatch (inputs against the shapes x or v fixes, caller-supplied outputs and
workspaces) before any call into the library.  These run without a GPU: the
shape checks come before the device check, and correctly shaped CPU tensors
are refused because there is no CPU path.
"""
import pytest
import torch

from selective_state_space_vjp_amd import binding as bd

f32, bf16 = torch.float32, torch.bfloat16


def _scan(b=1, T=8, H=2, P=4, N=8, G=1, per_state=False):
    return dict(x=torch.zeros(b, T, H, P), dt=torch.zeros(b, T, H), A=torch.zeros((H, N) if per_state else (H,)),
                B=torch.zeros(b, T, G, N), C=torch.zeros(b, T, G, N), s0=torch.zeros(b, H, P, N),
                dy=torch.zeros(b, T, H, P), ds_final=torch.zeros(b, H, P, N))


def _call_scan(a, **kw):
    return bd.ssm_scan_bwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["s0"], a["dy"], a["ds_final"], **kw)


def test_scan_correct_shapes_refused_only_for_the_device():
    with pytest.raises(ValueError, match="GPU tensor"):
        _call_scan(_scan())


@pytest.mark.parametrize("key,bad", [
    ("C", torch.zeros(1, 8, 1, 4)),        # N differs from B's
    ("C", torch.zeros(2, 8, 1, 8)),        # batch differs from x's
    ("dy", torch.zeros(1, 8, 2, 5)),
    ("dt", torch.zeros(1, 7, 2)),
    ("A", torch.zeros(3)),                 # not [H]
    ("A", torch.zeros(2, 4)),              # per-state A with the wrong N
    ("s0", torch.zeros(1, 2, 4, 9)),
    ("ds_final", torch.zeros(1, 2, 3, 8)),
])
def test_scan_rejects_mismatched_inputs(key, bad):
    a = _scan()
    a[key] = bad
    with pytest.raises(ValueError, match="shape"):
        _call_scan(a)


def test_scan_rejects_mixed_big_dtypes():
    a = _scan()
    a["dy"] = a["dy"].to(bf16)
    with pytest.raises(TypeError):
        _call_scan(a)


def _scan_out(b=1, T=8, H=2, P=4, N=8, G=1):
    return dict(dx=torch.zeros(b, T, H, P), d_dt=torch.zeros(b, T, H), dB=torch.zeros(b, T, G, N),
                dC=torch.zeros(b, T, G, N), d_s0=torch.zeros(b, H, P, N))


@pytest.mark.parametrize("key,bad", [
    ("dx", torch.zeros(1, 8, 2, 3)), ("d_dt", torch.zeros(1, 8, 1)), ("dB", torch.zeros(1, 8, 1, 4)),
    ("dC", torch.zeros(1, 4, 1, 8)), ("d_s0", torch.zeros(1, 2, 4, 4)),
])
def test_scan_rejects_mismatched_out(key, bad):
    out = _scan_out()
    out[key] = bad
    with pytest.raises(ValueError, match="shape"):
        _call_scan(_scan(), out=out)


def test_scan_rejects_incomplete_out_and_wrong_out_dtype():
    out = _scan_out()
    del out["dC"]
    with pytest.raises(ValueError, match="missing"):
        _call_scan(_scan(), out=out)
    out = _scan_out()
    out["d_dt"] = out["d_dt"].to(torch.float64)
    with pytest.raises(TypeError):
        _call_scan(_scan(), out=out)


def _ssd(raw=False, b=1, T=32, M=2, H=2, P=16, N=16, G=1):
    x = torch.zeros(b, T, M, H, P) if raw else torch.zeros(b, T, H, P)
    bc = (b, T, M, G, N) if raw else (b, T, G, N)
    return dict(xv=x, dtda=torch.zeros(b, T, H), A=None if raw else torch.zeros(H), B=torch.zeros(bc),
                C=torch.zeros(bc), s0=torch.zeros(b, H, P, N), dy=torch.zeros_like(x),
                ds_final=torch.zeros(b, H, P, N))


def _call_ssd(a, **kw):
    return bd.ssd_chunk_bwd(a["xv"], a["dtda"], a["A"], a["B"], a["C"], a["s0"], a["dy"], a["ds_final"],
                            chunk_len=16, **kw)


@pytest.mark.parametrize("raw", [False, True])
def test_ssd_correct_shapes_refused_only_for_the_device(raw):
    with pytest.raises(ValueError, match="GPU tensor"):
        _call_ssd(_ssd(raw))


@pytest.mark.parametrize("raw", [False, True])
@pytest.mark.parametrize("key", ["B", "C"])
@pytest.mark.parametrize("axis", [0, 1])
def test_ssd_rejects_B_C_with_another_batch_or_length(raw, key, axis):
    a = _ssd(raw)
    shape = list(a[key].shape)
    shape[axis] += 1
    a[key] = torch.zeros(shape)
    with pytest.raises(ValueError, match="shape"):
        _call_ssd(a)


def test_ssd_rejects_B_C_with_another_rank():
    a = _ssd(True)
    a["C"] = torch.zeros(1, 32, 3, 1, 16)  # M = 3 against v's M = 2
    with pytest.raises(ValueError, match="shape"):
        _call_ssd(a)
    a = _ssd(True)
    a["B"] = torch.zeros(1, 32, 3, 1, 16)
    with pytest.raises(ValueError, match="shape"):
        _call_ssd(a)


@pytest.mark.parametrize("key,bad", [("A", torch.zeros(3)), ("dtda", torch.zeros(1, 32, 3)),
                                     ("dy", torch.zeros(1, 32, 2, 8)), ("s0", torch.zeros(1, 2, 16, 8)),
                                     ("ds_final", torch.zeros(2, 2, 16, 16))])
def test_ssd_rejects_mismatched_inputs(key, bad):
    a = _ssd()
    a[key] = bad
    with pytest.raises(ValueError, match="shape"):
        _call_ssd(a)


@pytest.mark.parametrize("raw", [False, True])
def test_ssd_rejects_mismatched_out(raw):
    a = _ssd(raw)
    names = ("dv", "d_da") if raw else ("dx", "d_dt")
    good = {names[0]: torch.zeros_like(a["xv"]), names[1]: torch.zeros(1, 32, 2), "dB": torch.zeros_like(a["B"]),
            "dC": torch.zeros_like(a["C"]), "d_s0": torch.zeros(1, 2, 16, 16)}
    for key in good:
        out = dict(good)
        t = good[key]
        out[key] = torch.zeros(*t.shape[:-1], t.shape[-1] + 1)
        with pytest.raises(ValueError, match="shape"):
            _call_ssd(a, out=out)


def test_ssd_rejects_noncontiguous_input():
    a = _ssd()
    a["B"] = torch.zeros(1, 32, 2, 16)[:, :, :1, :]  # every other row
    with pytest.raises(ValueError, match="contiguous"):
        _call_ssd(a)


def test_ssd_fwd_rejects_mismatched_B_and_out():
    a = _ssd()
    a["C"] = torch.zeros(1, 31, 1, 16)
    with pytest.raises(ValueError, match="shape"):
        bd.ssd_chunk_fwd(a["xv"], a["dtda"], a["A"], a["B"], a["C"], a["s0"], chunk_len=16)
    a = _ssd()
    with pytest.raises(ValueError, match="shape"):
        bd.ssd_chunk_fwd(a["xv"], a["dtda"], a["A"], a["B"], a["C"], a["s0"], chunk_len=16,
                         out={"y": torch.zeros(1, 32, 2, 8), "s_final": None})


def _kda(b=1, T=8, H=1, HV=2, K=128, V=32):
    return dict(q=torch.zeros(b, T, H, K), k=torch.zeros(b, T, H, K), v=torch.zeros(b, T, HV, V),
                beta=torch.zeros(b, T, HV), g=torch.zeros(b, T, HV, K), S0=torch.zeros(b, HV, K, V),
                d_o=torch.zeros(b, T, HV, V))


def _call_kda(a, **kw):
    return bd.delta_rule_bwd(a["q"], a["k"], a["v"], a["beta"], a["g"], a["S0"], a["d_o"], scale=1.0, **kw)


def test_kda_rejects_mismatched_inputs_and_out():
    with pytest.raises(ValueError, match="GPU tensor"):
        _call_kda(_kda())
    for key, bad in (("k", torch.zeros(1, 8, 1, 64)), ("g", torch.zeros(1, 8, 1, 128)),
                     ("beta", torch.zeros(1, 8, 1)), ("d_o", torch.zeros(1, 8, 2, 16))):
        a = _kda()
        a[key] = bad
        with pytest.raises(ValueError, match="shape"):
            _call_kda(a)
    a = _kda()
    good = dict(dq=torch.zeros(1, 8, 1, 128), dk=torch.zeros(1, 8, 1, 128), dv=torch.zeros(1, 8, 2, 32),
                dg=torch.zeros(1, 8, 2, 128), dbeta=torch.zeros(1, 8, 2), dS0=torch.zeros(1, 2, 128, 32))
    for key in good:
        out = dict(good)
        out[key] = torch.zeros(*good[key].shape[:-1], good[key].shape[-1] + 2)
        with pytest.raises(ValueError, match="shape"):
            _call_kda(a, out=out)
