"""Host-only checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

from selective_state_space_vjp_amd import binding as bd

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ssmvjp.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "return")))


def test_library_exports_every_declared_function():
    declared = _declared_functions()
    assert len(declared) >= 8
    lib = ctypes.CDLL(str(bd.LIB_PATH))
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(bd.EXPORTS)


def test_version_and_status_strings():
    assert bd.version() == "0.1.0"
    assert bd.status_str(bd.EINVAL) == "invalid argument"
    assert bd.status_str(99) == "unknown status"


def _scan(**kw):
    d = dict(batch=1, seqlen=8, nheads=2, headdim=4, dstate=8, ngroups=1, decay=0, dtype=0, ckpt_every=0, reserved=0)
    d.update(kw)
    return bd.ScanDesc(**d)


def _ws(fn, desc):
    n = ctypes.c_size_t(0)
    st = getattr(bd.lib(), fn)(ctypes.byref(desc), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    (dict(), bd.OK),
    (dict(nheads=3, ngroups=2), bd.EINVAL),
    (dict(headdim=0), bd.EINVAL),
    (dict(seqlen=-1), bd.EINVAL),
    (dict(decay=7), bd.EINVAL),
    (dict(dtype=5), bd.EINVAL),
    (dict(reserved=1), bd.EINVAL),
    (dict(ckpt_every=-2), bd.EINVAL),
    (dict(dstate=2048), bd.EUNSUPPORTED),
    (dict(headdim=512, dstate=128), bd.EUNSUPPORTED),
])
def test_scan_descriptor_validation(kw, status):
    st, n = _ws("ssm_scan_bwd_workspace", _scan(**kw))
    assert st == status
    if status == bd.OK:
        assert n > 0


def test_scan_workspace_shrinks_with_checkpointing():
    big = _ws("ssm_scan_bwd_workspace", _scan(seqlen=4096, headdim=64, dstate=128, ckpt_every=1))[1]
    small = _ws("ssm_scan_bwd_workspace", _scan(seqlen=4096, headdim=64, dstate=128, ckpt_every=64))[1]
    assert small < big / 10


def test_scan_rejects_null_pointers_and_small_workspace_without_launching():
    L = bd.lib()
    d = _scan()
    nulls = [None] * 14
    assert L.ssm_scan_bwd(ctypes.byref(d), *nulls, 0, None) == bd.EINVAL
    fake = [ctypes.c_void_p(4096 * (i + 1)) for i in range(13)]
    assert L.ssm_scan_bwd(ctypes.byref(d), *fake, None, 0, None) == bd.EWORKSPACE
    mis = list(fake)
    mis[1] = ctypes.c_void_p(4096 + 2)  # dt misaligned for float32
    ws = ctypes.c_void_p(1 << 20)
    assert L.ssm_scan_bwd(ctypes.byref(d), *mis, ws, 1 << 30, None) == bd.EINVAL


def _ssd(**kw):
    d = dict(batch=1, seqlen=128, nheads=4, headdim=64, dstate=128, ngroups=1, mimo_rank=1, chunk_len=64, form=0,
             dtype=1)
    d.update(kw)
    return bd.SsdDesc(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(), bd.OK),
    (dict(seqlen=100), bd.OK),
    (dict(nheads=3, ngroups=2), bd.EINVAL),
    (dict(form=0, mimo_rank=2), bd.EINVAL),
    (dict(form=3), bd.EINVAL),
    (dict(chunk_len=0), bd.EINVAL),
    # P or N off the 16-multiple: run zero-padded to the next multiple of 16
    # when the padded shape is supported
    (dict(headdim=20), bd.OK),
    (dict(dstate=40), bd.OK),
    (dict(headdim=4, dstate=8, chunk_len=16), bd.OK),
    (dict(headdim=4, dstate=8, chunk_len=64, dtype=0), bd.OK),
    (dict(headdim=120, dstate=128), bd.EUNSUPPORTED),  # padded to P = N = 128: too large at L = 64
    (dict(headdim=20, chunk_len=72), bd.EUNSUPPORTED),  # padding does not cover the chunk length
    (dict(dstate=256), bd.EUNSUPPORTED),
    (dict(headdim=112, dstate=80), bd.EUNSUPPORTED),
    (dict(headdim=128, dstate=128), bd.EUNSUPPORTED),
    (dict(headdim=128, dstate=64), bd.OK),
    (dict(chunk_len=72), bd.EUNSUPPORTED),
    # fused chunks longer than 64 rows (row-blocked kernels): multiples of 64, chunk_len <= 64
    (dict(form=1, mimo_rank=2), bd.OK),
    (dict(form=1, mimo_rank=3), bd.EUNSUPPORTED),  # rows of a step would straddle 64-row blocks
    (dict(form=1, mimo_rank=4, chunk_len=48), bd.OK),
    (dict(form=1, mimo_rank=4, ngroups=4), bd.OK),
    (dict(form=1, mimo_rank=5, chunk_len=16), bd.EUNSUPPORTED),
    (dict(chunk_len=128), bd.EUNSUPPORTED),
    (dict(form=1, mimo_rank=4, headdim=128, dstate=128), bd.OK),
    (dict(form=1, mimo_rank=4, headdim=128, dstate=128, dtype=0), bd.EUNSUPPORTED),
    # byte offsets inside one batch element are 32-bit: here the stored chunk
    # states (4 heads x 16 KiB per chunk) reach 2 GiB at 2^21 steps; the batch
    # size does not enter the bound
    (dict(seqlen=(1 << 21) - 64), bd.OK),
    (dict(seqlen=1 << 21), bd.EUNSUPPORTED),
    (dict(batch=64, seqlen=(1 << 21) - 64), bd.OK),
])
def test_ssd_descriptor_validation(kw, status):
    st, _ = _ws("ssd_chunk_bwd_workspace", _ssd(**kw))
    assert st == status


@pytest.mark.parametrize("kw,status", [
    (dict(), bd.OK),
    (dict(dv=256), bd.OK),
    (dict(seqlen=0), bd.OK),
    (dict(nv_heads=3, nqk_heads=2), bd.EINVAL),
    (dict(dk=0), bd.EINVAL),
    (dict(reserved=1), bd.EINVAL),
    (dict(dk=64), bd.EUNSUPPORTED),   # the kernels hold K = 128 rows of the state
    (dict(dv=48), bd.EUNSUPPORTED),   # V is cut into 32-column slices
])
def test_delta_descriptor_validation(kw, status):
    d = dict(batch=1, seqlen=64, nqk_heads=2, nv_heads=4, dk=128, dv=32, scale=0.25, reserved=0)
    d.update(kw)
    st, _ = _ws("delta_rule_bwd_workspace", bd.DeltaDesc(**d))
    assert st == status


def test_binding_refuses_cpu_tensors():
    import torch

    x = torch.zeros(1, 4, 2, 4)
    with pytest.raises(ValueError, match="GPU tensor"):
        bd.ssm_scan_bwd(x, torch.zeros(1, 4, 2), torch.zeros(2), torch.zeros(1, 4, 1, 8), torch.zeros(1, 4, 1, 8),
                        None, x, None)


def test_delta_rejects_bad_arguments_without_launching():
    # every case returns before anything is enqueued, so no GPU is needed
    L = bd.lib()
    d = bd.DeltaDesc(batch=1, seqlen=16, nqk_heads=1, nv_heads=2, dk=128, dv=32, scale=0.25, reserved=0)
    nulls = [None] * 14
    assert L.delta_rule_bwd(ctypes.byref(d), *nulls, None, 0, None) == bd.EINVAL
    fake = [ctypes.c_void_p(4096 * (i + 1)) for i in range(14)]
    assert L.delta_rule_bwd(ctypes.byref(d), *fake, None, 0, None) == bd.EWORKSPACE
    mis = list(fake)
    mis[2] = ctypes.c_void_p(4096 * 3 + 8)  # v only 8-byte aligned
    assert L.delta_rule_bwd(ctypes.byref(d), *mis, ctypes.c_void_p(1 << 20), 1 << 34, None) == bd.EINVAL
    # the staged entry point validates its stage mask the same way
    ws = ctypes.c_void_p(1 << 20)
    for bad in (0, 8, -1):
        assert L.delta_rule_bwd_stages(ctypes.byref(d), bad, *fake, ws, 1 << 34, None) == bd.EINVAL


def test_ssd_stage_entry_points_validate_like_the_full_call():
    L = bd.lib()
    d = _ssd()
    # NULL inputs (ten pointers incl. the workspace; eleven for the grads stage)
    assert L.ssd_chunk_bwd_states(ctypes.byref(d), *([None] * 10), 0, None) == bd.EINVAL
    assert L.ssd_chunk_bwd_grads(ctypes.byref(d), *([None] * 11), 0, None) == bd.EINVAL


@pytest.mark.parametrize("kw,desc_status,call_status", [
    # supported descriptors reach the NULL-pointer check of the call
    (dict(), bd.OK, bd.EINVAL),
    (dict(form=1, mimo_rank=4), bd.OK, bd.EINVAL),
    (dict(form=1, mimo_rank=3, chunk_len=16), bd.OK, bd.EINVAL),  # steps straddle 16-row tiles
    (dict(headdim=48, dstate=96, dtype=0), bd.OK, bd.EINVAL),
    (dict(headdim=20), bd.OK, bd.EINVAL),  # zero-padded to 32
    (dict(dstate=40), bd.OK, bd.EINVAL),   # zero-padded to 48
    (dict(dstate=250), bd.EUNSUPPORTED, bd.EUNSUPPORTED),  # 256 after padding: over the forward's N <= 128
    (dict(dstate=256), bd.EUNSUPPORTED, bd.EUNSUPPORTED),
    (dict(form=1, mimo_rank=65), bd.EUNSUPPORTED, bd.EUNSUPPORTED),
    (dict(nheads=3, ngroups=2), bd.EINVAL, bd.EINVAL),
    (dict(form=0, mimo_rank=2), bd.EINVAL, bd.EINVAL),
    (dict(chunk_len=0), bd.EINVAL, bd.EINVAL),
    (dict(batch=0), bd.OK, bd.OK),  # nothing to do: no pointer is read
])
def test_ssd_fwd_validates_before_launching(kw, desc_status, call_status):
    L = bd.lib()
    d = _ssd(**kw)
    n = ctypes.c_size_t(0)
    assert L.ssd_chunk_fwd_workspace(ctypes.byref(d), ctypes.byref(n)) == desc_status
    assert L.ssd_chunk_fwd(ctypes.byref(d), *([None] * 8), None, 0, None) == call_status


def test_ssd_fwd_rejects_misaligned_big_tensors():
    L = bd.lib()
    d = _ssd()
    fake = [ctypes.c_void_p(4096 * (i + 1)) for i in range(8)]
    mis = list(fake)
    mis[0] = ctypes.c_void_p(4096 + 8)  # x only 8-byte aligned
    ws = ctypes.c_void_p(1 << 20)
    assert L.ssd_chunk_fwd(ctypes.byref(d), *mis, ws, 1 << 30, None) == bd.EINVAL
    mis = list(fake)
    mis[7] = ctypes.c_void_p(4096 * 8 + 2)  # s_final misaligned for float32
    assert L.ssd_chunk_fwd(ctypes.byref(d), *mis, ws, 1 << 30, None) == bd.EINVAL
    # bf16 needs the scores workspace; float32 needs none
    assert L.ssd_chunk_fwd(ctypes.byref(d), *fake, None, 0, None) == bd.EWORKSPACE
    n = ctypes.c_size_t(0)
    assert L.ssd_chunk_fwd_workspace(ctypes.byref(d), ctypes.byref(n)) == bd.OK
    assert n.value == 1 * 2 * 1 * 16 * 256 * 4  # b * chunks * groups score blocks
    d32 = _ssd(dtype=0)
    assert L.ssd_chunk_fwd_workspace(ctypes.byref(d32), ctypes.byref(n)) == bd.OK and n.value == 0


def test_dA_entry_points_validate_before_launching():
    L = bd.lib()
    fake = [ctypes.c_void_p(4096 * (i + 1)) for i in range(13)]
    ws = ctypes.c_void_p(1 << 20)
    # chunked: dA needs the Mamba-2 form and a dA pointer
    d = _ssd()
    assert L.ssd_chunk_bwd_dA(ctypes.byref(d), *fake, None, ws, 1 << 34, None) == bd.EINVAL
    raw = _ssd(form=1, mimo_rank=2)
    assert L.ssd_chunk_bwd_dA(ctypes.byref(raw), *fake, ctypes.c_void_p(1 << 21), ws, 1 << 34, None) == bd.EINVAL
    assert L.ssd_chunk_bwd_dA(ctypes.byref(d), *([None] * 14), None, 0, None) == bd.EINVAL
    mis = ctypes.c_void_p((1 << 21) + 2)  # dA misaligned for float32
    assert L.ssd_chunk_bwd_dA(ctypes.byref(d), *fake, mis, ws, 1 << 34, None) == bd.EINVAL
    # sequential
    s = _scan()
    assert L.ssm_scan_bwd_dA(ctypes.byref(s), *fake, None, ws, 1 << 34, None) == bd.EINVAL
    assert L.ssm_scan_bwd_dA(ctypes.byref(s), *fake, mis, ws, 1 << 34, None) == bd.EINVAL
    # an empty batch has nothing to write
    assert L.ssm_scan_bwd_dA(ctypes.byref(_scan(batch=0)), *([None] * 14), None, 0, None) == bd.OK


def test_scan_lds_limit_is_the_stated_one():
    """P = N = 128 keeps P*N within 32768 but its state needs 74,304 bytes of
    LDS (over the 64 KiB the header states); P = 64, N = 128 fits."""
    assert _ws("ssm_scan_bwd_workspace", _scan(headdim=128, dstate=128))[0] == bd.EUNSUPPORTED
    assert _ws("ssm_scan_bwd_workspace", _scan(headdim=64, dstate=256))[0] == bd.EUNSUPPORTED
    assert _ws("ssm_scan_bwd_workspace", _scan(headdim=64, dstate=128))[0] == bd.OK


def _lds_bytes(P, N):
    Q = -(-P // min(P, 16))
    return 4 * (P * (N + 1) + 2 * Q * N + -(-(Q * N) // 64))


@pytest.mark.parametrize("P,N", [(1, 16), (4, 8), (16, 256), (33, 64), (64, 128), (96, 96), (128, 128), (20, 500),
                                 (2, 1024), (64, 256), (128, 64)])
def test_scan_header_formula_matches_the_library(P, N):
    Q = -(-P // min(P, 16))
    ok = N <= 1024 and P * N <= 32768 and Q * N <= 1024 and _lds_bytes(P, N) <= 65536
    st = _ws("ssm_scan_bwd_workspace", _scan(headdim=P, dstate=N))[0]
    assert st == (bd.OK if ok else bd.EUNSUPPORTED), (P, N, st)


def test_nonfinite_status_and_debug_workspace(monkeypatch):
    """The debug finiteness mode (SSMVJP_CHECK_FINITE) has its own status, and
    while it is on every workspace query reports 256 more bytes (the scan's
    flag), rounded after the plan's own bytes."""
    assert bd.status_str(bd.ENONFINITE).startswith("non-finite")
    queries = [("ssm_scan_bwd_workspace", _scan()),
               ("ssd_chunk_bwd_workspace", bd.SsdDesc(1, 100, 2, 16, 16, 1, 1, 16, 0, 0)),
               ("ssd_chunk_fwd_workspace", bd.SsdDesc(1, 100, 2, 16, 16, 1, 1, 16, 0, 1)),
               ("delta_rule_bwd_workspace", bd.DeltaDesc(1, 20, 1, 2, 128, 32, 1.0, 0))]
    monkeypatch.delenv("SSMVJP_CHECK_FINITE", raising=False)
    off = [_ws(fn, d) for fn, d in queries]
    monkeypatch.setenv("SSMVJP_CHECK_FINITE", "0")
    assert [_ws(fn, d) for fn, d in queries] == off
    monkeypatch.setenv("SSMVJP_CHECK_FINITE", "1")
    for (fn, d), (st0, n0) in zip(queries, off):
        st, n = _ws(fn, d)
        assert st == st0 == bd.OK
        assert n == (n0 + 255) // 256 * 256 + 256, (fn, n0, n)


def test_debug_mode_still_validates_before_launching(monkeypatch):
    """With the mode on, a workspace sized for the mode off is refused before
    anything is enqueued."""
    monkeypatch.delenv("SSMVJP_CHECK_FINITE", raising=False)
    d = _scan()
    n = _ws("ssm_scan_bwd_workspace", d)[1]
    monkeypatch.setenv("SSMVJP_CHECK_FINITE", "1")
    fake = [ctypes.c_void_p(4096 * (i + 1)) for i in range(13)]
    assert bd.lib().ssm_scan_bwd(ctypes.byref(d), *fake, ctypes.c_void_p(1 << 20), n, None) == bd.EWORKSPACE


def test_padded_workspace_holds_the_padded_problem():
    """A P or N off the 16-multiple needs the padded problem's workspace plus
    the padded copies of the inputs and outputs: more than the next supported
    shape's own workspace."""
    n_pad = _ws("ssd_chunk_bwd_workspace", _ssd(headdim=20, dtype=0))[1]
    n_32 = _ws("ssd_chunk_bwd_workspace", _ssd(headdim=32, dtype=0))[1]
    assert n_pad > n_32
