"""ctypes binding of libssmvjp (C ABI in include/ssmvjp.h).

Argument marshalling only: shape/dtype checks, output and workspace
allocation through torch's caching allocator, and the current HIP stream.
Every step of the computation runs in the HIP kernels; there is no CPU path.
If the library is missing the calls raise.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

LIB_PATH = Path(__file__).resolve().parent / "libssmvjp.so"

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP, ENONFINITE = 0, 1, 2, 3, 4, 5
F32, BF16 = 0, 1
DECAY_PER_HEAD, DECAY_PER_STATE = 0, 1
FORM_MAMBA2, FORM_RAW = 0, 1
DELTA_CKPT, DELTA_BWD, DELTA_REDUCE, DELTA_ALL = 1, 2, 4, 7

_STATUS_FNS = ("ssm_scan_bwd_workspace", "ssm_scan_bwd", "ssm_scan_bwd_dA", "ssd_chunk_bwd_workspace",
               "ssd_chunk_bwd", "ssd_chunk_bwd_dA", "ssd_chunk_bwd_states", "ssd_chunk_bwd_grads", "ssd_chunk_bwd_noalloc",
               "ssd_chunk_fwd_workspace", "ssd_chunk_fwd", "delta_rule_bwd_workspace", "delta_rule_bwd",
               "delta_rule_bwd_stages")
EXPORTS = _STATUS_FNS + ("ssmvjp_status_str", "ssmvjp_version")


class ScanDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("decay", ctypes.c_int32), ("dtype", ctypes.c_int32), ("ckpt_every", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class SsdDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("mimo_rank", ctypes.c_int64), ("chunk_len", ctypes.c_int64),
                ("form", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class DeltaDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nqk_heads", ctypes.c_int64),
                ("nv_heads", ctypes.c_int64), ("dk", ctypes.c_int64), ("dv", ctypes.c_int64),
                ("scale", ctypes.c_float), ("reserved", ctypes.c_int32)]


class SsmVjpError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_str(status)})")


_lib = None


def lib():
    """Load libssmvjp.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(str(LIB_PATH))
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.ssm_scan_bwd_workspace.argtypes = [ctypes.POINTER(ScanDesc), ctypes.POINTER(sz)]
        L.ssm_scan_bwd.argtypes = [ctypes.POINTER(ScanDesc)] + [vp] * 14 + [sz, vp]
        L.ssm_scan_bwd_dA.argtypes = [ctypes.POINTER(ScanDesc)] + [vp] * 15 + [sz, vp]
        L.ssd_chunk_bwd_workspace.argtypes = [ctypes.POINTER(SsdDesc), ctypes.POINTER(sz)]
        L.ssd_chunk_bwd.argtypes = [ctypes.POINTER(SsdDesc)] + [vp] * 14 + [sz, vp]
        L.ssd_chunk_bwd_dA.argtypes = [ctypes.POINTER(SsdDesc)] + [vp] * 15 + [sz, vp]
        L.ssd_chunk_bwd_states.argtypes = [ctypes.POINTER(SsdDesc)] + [vp] * 10 + [sz, vp]
        L.ssd_chunk_bwd_grads.argtypes = [ctypes.POINTER(SsdDesc)] + [vp] * 11 + [sz, vp]
        L.ssd_chunk_bwd_noalloc.argtypes = [ctypes.POINTER(SsdDesc)] + [vp] * 14
        L.ssd_chunk_fwd_workspace.argtypes = [ctypes.POINTER(SsdDesc), ctypes.POINTER(sz)]
        L.ssd_chunk_fwd.argtypes = [ctypes.POINTER(SsdDesc)] + [vp] * 9 + [sz, vp]
        L.delta_rule_bwd_workspace.argtypes = [ctypes.POINTER(DeltaDesc), ctypes.POINTER(sz)]
        L.delta_rule_bwd.argtypes = [ctypes.POINTER(DeltaDesc)] + [vp] * 15 + [sz, vp]
        L.delta_rule_bwd_stages.argtypes = [ctypes.POINTER(DeltaDesc), ctypes.c_int32] + [vp] * 15 + [sz, vp]
        for name in _STATUS_FNS:
            getattr(L, name).restype = ctypes.c_int
        L.ssmvjp_status_str.argtypes = [ctypes.c_int]
        L.ssmvjp_status_str.restype = ctypes.c_char_p
        L.ssmvjp_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(status):
    return lib().ssmvjp_status_str(int(status)).decode()


def version():
    return lib().ssmvjp_version().decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; big tensors are float32 or bfloat16")


def _need(t, name, dtype, shape, device):
    """Check an optional tensor argument (None passes): shape, dtype and layout.
    The device is checked by _on_gpu once every shape has been checked."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(device, *tensors):
    """Every tensor handed to the library lives on the same GPU (there is no CPU path)."""
    if not device.type == "cuda":
        raise ValueError("inputs must be GPU tensors (there is no CPU path)")
    for t in tensors:
        if t is not None and t.device != device:
            raise ValueError(f"a tensor is on {t.device}, expected {device} (there is no CPU path)")


def _check_out(out, spec, device):
    """Every tensor of a caller-supplied ``out`` dict must match what the call writes:
    the kernels see only pointers, so a wrong size would be written out of bounds."""
    for name, (dtype, shape) in spec.items():
        if name not in out or out[name] is None:
            raise ValueError(f"out is missing '{name}'")
        _need(out[name], f"out['{name}']", dtype, shape, device)


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        if not workspace.is_contiguous() or not workspace.is_cuda or workspace.device != device:
            raise ValueError(f"workspace must be a contiguous tensor on {device}")
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def _check(fn, status):
    if status != OK:
        raise SsmVjpError(fn, status)


# --------------------------------------------------------------------------- #
def scan_desc(x, A, B, ckpt_every=0):
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    decay = DECAY_PER_STATE if A.dim() == 2 else DECAY_PER_HEAD
    return ScanDesc(b, T, H, P, N, G, decay, _dtype_code(x), int(ckpt_every), 0)


def ssm_scan_bwd_workspace(desc):
    n = ctypes.c_size_t(0)
    _check("ssm_scan_bwd_workspace", lib().ssm_scan_bwd_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def ssm_scan_bwd(x, dt, A, B, C, s0, dy, ds_final, *, ckpt_every=0, want_dA=False, out=None, workspace=None,
                 stream=None):
    """Sequential selective-scan backward.  Returns dict dx, d_dt, dB, dC, d_s0
    (and dA, shaped like A, with want_dA=True).

    x, dy [b,T,H,P] and B, C [b,T,G,N] are float32 or bfloat16 (all the same);
    dt [b,T,H], A [H] (Mamba-2) or [H,N] (Mamba-1), s0, ds_final [b,H,P,N] float32
    (s0 / ds_final may be None = zeros).
    """
    if x is None or B is None or A is None or x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [b,T,H,P], B [b,T,G,N] and A [H] or [H,N]")
    desc = scan_desc(x, A, B, ckpt_every)
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev, big = x.device, x.dtype
    _need(x, "x", big, (b, T, H, P), dev)
    _need(dy, "dy", big, (b, T, H, P), dev)
    _need(B, "B", big, (b, T, G, N), dev)
    _need(C, "C", big, (b, T, G, N), dev)
    for name, t in (("dt", dt), ("C", C), ("dy", dy)):
        if t is None:
            raise ValueError(f"{name} is required")
    _need(dt, "dt", torch.float32, (b, T, H), dev)
    if A.dim() not in (1, 2):
        raise ValueError("A must be [H] (per-head decay) or [H,N] (per-state decay)")
    _need(A, "A", torch.float32, (H,) if A.dim() == 1 else (H, N), dev)
    _need(s0, "s0", torch.float32, (b, H, P, N), dev)
    _need(ds_final, "ds_final", torch.float32, (b, H, P, N), dev)
    spec = dict(dx=(big, (b, T, H, P)), d_dt=(torch.float32, (b, T, H)), dB=(big, (b, T, G, N)),
                dC=(big, (b, T, G, N)), d_s0=(torch.float32, (b, H, P, N)))
    if out is None:
        out = dict(dx=torch.empty_like(x), d_dt=torch.empty_like(dt), dB=torch.empty_like(B),
                   dC=torch.empty_like(C), d_s0=torch.empty((b, H, P, N), dtype=torch.float32, device=dev))
    _check_out(out, spec, dev)
    _on_gpu(dev, x, dt, A, B, C, s0, dy, ds_final, *out.values())
    ws, wsb = _workspace(ssm_scan_bwd_workspace(desc), dev, workspace)
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(s0), _ptr(dy), _ptr(ds_final), _ptr(out["dx"]),
            _ptr(out["d_dt"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["d_s0"]))
    if want_dA:
        if "dA" not in out:
            out["dA"] = torch.empty_like(A)
        _need(out["dA"], "out['dA']", torch.float32, tuple(A.shape), dev)
        st = lib().ssm_scan_bwd_dA(ctypes.byref(desc), *args, _ptr(out["dA"]), _ptr(ws), wsb, _stream(stream))
        _check("ssm_scan_bwd_dA", st)
    else:
        st = lib().ssm_scan_bwd(ctypes.byref(desc), *args, _ptr(ws), wsb, _stream(stream))
        _check("ssm_scan_bwd", st)
    return out


class ScanCall:
    """A prepared ssm_scan_bwd call on fixed device buffers (for repeated timing):
    arguments are checked once, ``run()`` only enqueues the backward."""

    def __init__(self, x, dt, A, B, C, s0, dy, ds_final, *, ckpt_every=0, stream=None):
        self.out = ssm_scan_bwd(x, dt, A, B, C, s0, dy, ds_final, ckpt_every=ckpt_every, stream=stream)
        self.desc = scan_desc(x, A, B, ckpt_every)
        self.ws, self.wsb = _workspace(ssm_scan_bwd_workspace(self.desc), x.device, None)
        self.stream = stream
        p, o = _ptr, self.out
        self._args = (p(x), p(dt), p(A), p(B), p(C), p(s0), p(dy), p(ds_final), p(o["dx"]), p(o["d_dt"]), p(o["dB"]),
                      p(o["dC"]), p(o["d_s0"]))
        self._keep = (x, dt, A, B, C, s0, dy, ds_final)

    def run(self):
        st = lib().ssm_scan_bwd(ctypes.byref(self.desc), *self._args, _ptr(self.ws), self.wsb, _stream(self.stream))
        _check("ssm_scan_bwd", st)


# --------------------------------------------------------------------------- #
def ssd_desc(xv, B, chunk_len, form):
    if form == FORM_MAMBA2:
        b, T, H, P = xv.shape
        M = 1
        G, N = B.shape[2], B.shape[3]
    else:
        b, T, M, H, P = xv.shape
        G, N = B.shape[3], B.shape[4]
    return SsdDesc(b, T, H, P, N, G, M, int(chunk_len), form, _dtype_code(xv))


def _ssd_inputs(xv, dtda, A, B, C, s0, form, chunk_len):
    """Descriptor of a chunked call after checking every input against the shapes
    x/v fixes: B, C [b,T,G,N] (RAW: [b,T,M,G,N]), dt/da [b,T,H], A [H], states
    [b,H,P,N]."""
    if xv is None or B is None:
        raise ValueError("x/v and B are required")
    if xv.dim() != (4 if form == FORM_MAMBA2 else 5):
        raise ValueError(f"x/v must be {'[b,T,H,P]' if form == FORM_MAMBA2 else '[b,T,M,H,P]'}")
    if B.dim() != xv.dim():
        raise ValueError(f"B must be {'[b,T,G,N]' if form == FORM_MAMBA2 else '[b,T,M,G,N]'}")
    desc = ssd_desc(xv, B, chunk_len, form)
    b, T, H, P, N, G, M = desc.batch, desc.seqlen, desc.nheads, desc.headdim, desc.dstate, desc.ngroups, desc.mimo_rank
    dev, big = xv.device, xv.dtype
    bc = (b, T, G, N) if form == FORM_MAMBA2 else (b, T, M, G, N)
    _need(xv, "x/v", big, tuple(xv.shape), dev)
    _need(B, "B", big, bc, dev)
    _need(C, "C", big, bc, dev)
    _need(dtda, "dt/da", torch.float32, (b, T, H), dev)
    if form == FORM_MAMBA2:
        _need(A, "A", torch.float32, (H,), dev)
    _need(s0, "s0", torch.float32, (b, H, P, N), dev)
    if C is None or dtda is None or (form == FORM_MAMBA2 and A is None):
        raise ValueError("C, dt/da (and A in the Mamba-2 form) are required")
    return desc


def _ssd_grad_spec(desc, xv, form):
    b, T, H, P, N, G, M = (desc.batch, desc.seqlen, desc.nheads, desc.headdim, desc.dstate, desc.ngroups,
                           desc.mimo_rank)
    big = xv.dtype
    bc = (b, T, G, N) if form == FORM_MAMBA2 else (b, T, M, G, N)
    names = ("dx", "d_dt") if form == FORM_MAMBA2 else ("dv", "d_da")
    return {names[0]: (big, tuple(xv.shape)), names[1]: (torch.float32, (b, T, H)), "dB": (big, bc),
            "dC": (big, bc), "d_s0": (torch.float32, (b, H, P, N))}


def ssd_chunk_bwd_workspace(desc):
    n = ctypes.c_size_t(0)
    _check("ssd_chunk_bwd_workspace", lib().ssd_chunk_bwd_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def ssd_chunk_bwd(xv, dtda, A, B, C, s0, dy, ds_final, *, chunk_len, want_dA=False, out=None, workspace=None,
                  stream=None):
    """Chunked SSD backward.

    Mamba-2 form (A given): xv = x [b,T,H,P], dtda = dt [b,T,H] (raw),
    B, C [b,T,G,N]; returns dict dx, d_dt, dB, dC, d_s0 (and dA [H] with
    want_dA=True).
    RAW form (A None): xv = v [b,T,M,H,P], dtda = da [b,T,H], B, C [b,T,M,G,N];
    returns dict dv, d_da, dB, dC, d_s0.
    """
    form = FORM_MAMBA2 if A is not None else FORM_RAW
    desc = _ssd_inputs(xv, dtda, A, B, C, s0, form, chunk_len)
    b, T, H, P, N = desc.batch, desc.seqlen, desc.nheads, desc.headdim, desc.dstate
    dev, big = xv.device, xv.dtype
    if dy is None:
        raise ValueError("dy is required")
    _need(dy, "dy", big, tuple(xv.shape), dev)
    _need(ds_final, "ds_final", torch.float32, (b, H, P, N), dev)
    names = ("dx", "d_dt") if form == FORM_MAMBA2 else ("dv", "d_da")
    if out is None:
        out = {names[0]: torch.empty_like(xv), names[1]: torch.empty_like(dtda), "dB": torch.empty_like(B),
               "dC": torch.empty_like(C), "d_s0": torch.empty((b, H, P, N), dtype=torch.float32, device=dev)}
    _check_out(out, _ssd_grad_spec(desc, xv, form), dev)
    _on_gpu(dev, xv, dtda, A, B, C, s0, dy, ds_final, *out.values())
    ws, wsb = _workspace(ssd_chunk_bwd_workspace(desc), dev, workspace)
    args = (_ptr(xv), _ptr(dtda), _ptr(A), _ptr(B), _ptr(C), _ptr(s0), _ptr(dy), _ptr(ds_final),
            _ptr(out[names[0]]), _ptr(out[names[1]]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["d_s0"]))
    if want_dA:
        if form != FORM_MAMBA2:
            raise ValueError("dA needs the Mamba-2 (x, dt, A) form")
        if "dA" not in out:
            out["dA"] = torch.empty_like(A)
        _need(out["dA"], "out['dA']", torch.float32, (H,), dev)
        st = lib().ssd_chunk_bwd_dA(ctypes.byref(desc), *args, _ptr(out["dA"]), _ptr(ws), wsb, _stream(stream))
        _check("ssd_chunk_bwd_dA", st)
    else:
        st = lib().ssd_chunk_bwd(ctypes.byref(desc), *args, _ptr(ws), wsb, _stream(stream))
        _check("ssd_chunk_bwd", st)
    return out


NOALLOC_SCRATCH_BYTES = 96 << 20  # SSMVJP_NOALLOC_SCRATCH_BYTES


def ssd_chunk_bwd_noalloc(xv, dtda, A, B, C, s0, dy, ds_final, *, chunk_len, out, stream=None):
    """ssd_chunk_bwd on the library's own device array instead of a workspace.

    ``out`` (required: this call allocates nothing) holds the output tensors,
    as returned by ssd_chunk_bwd.  Shapes whose workspace exceeds
    NOALLOC_SCRATCH_BYTES raise (SSMVJP_EWORKSPACE).
    """
    form = FORM_MAMBA2 if A is not None else FORM_RAW
    desc = _ssd_inputs(xv, dtda, A, B, C, s0, form, chunk_len)
    if dy is None or out is None:
        raise ValueError("dy and out are required")
    dev = xv.device
    _need(dy, "dy", xv.dtype, tuple(xv.shape), dev)
    _need(ds_final, "ds_final", torch.float32, (desc.batch, desc.nheads, desc.headdim, desc.dstate), dev)
    _check_out(out, _ssd_grad_spec(desc, xv, form), dev)
    _on_gpu(dev, xv, dtda, A, B, C, s0, dy, ds_final, *out.values())
    names = ("dx", "d_dt") if form == FORM_MAMBA2 else ("dv", "d_da")
    st = lib().ssd_chunk_bwd_noalloc(ctypes.byref(desc), _ptr(xv), _ptr(dtda), _ptr(A), _ptr(B), _ptr(C), _ptr(s0),
                                     _ptr(dy), _ptr(ds_final), _ptr(out[names[0]]), _ptr(out[names[1]]),
                                     _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["d_s0"]), _stream(stream))
    _check("ssd_chunk_bwd_noalloc", st)
    return out


def ssd_chunk_fwd_workspace(desc):
    n = ctypes.c_size_t(0)
    _check("ssd_chunk_fwd_workspace", lib().ssd_chunk_fwd_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def ssd_chunk_fwd(xv, dtda, A, B, C, s0=None, *, chunk_len=64, out=None, want_final=True, workspace=None,
                  stream=None):
    """Chunked SSD forward.  Returns dict y (like xv) and s_final [b,H,P,N] float32.

    Mamba-2 form (A given): xv = x [b,T,H,P], dtda = dt [b,T,H] (raw), B, C [b,T,G,N].
    RAW form (A None): xv = v [b,T,M,H,P], dtda = da [b,T,H], B, C [b,T,M,G,N].
    s0 None = zeros; want_final=False leaves s_final out (None).
    """
    form = FORM_MAMBA2 if A is not None else FORM_RAW
    desc = _ssd_inputs(xv, dtda, A, B, C, s0, form, chunk_len)
    b, T, H, P, N = desc.batch, desc.seqlen, desc.nheads, desc.headdim, desc.dstate
    dev, big = xv.device, xv.dtype
    if out is None:
        out = {"y": torch.empty_like(xv),
               "s_final": torch.empty((b, H, P, N), dtype=torch.float32, device=dev) if want_final else None}
    if out.get("y") is None:
        raise ValueError("out is missing 'y'")
    _need(out["y"], "out['y']", big, tuple(xv.shape), dev)
    _need(out.get("s_final"), "out['s_final']", torch.float32, (b, H, P, N), dev)
    _on_gpu(dev, xv, dtda, A, B, C, s0, out["y"], out.get("s_final"))
    ws, wsb = _workspace(ssd_chunk_fwd_workspace(desc), dev, workspace)
    st = lib().ssd_chunk_fwd(ctypes.byref(desc), _ptr(xv), _ptr(dtda), _ptr(A), _ptr(B), _ptr(C), _ptr(s0),
                             _ptr(out["y"]), _ptr(out["s_final"]), _ptr(ws), wsb, _stream(stream))
    _check("ssd_chunk_fwd", st)
    return out


class SsdCall:
    """A prepared ssd_chunk_bwd call on fixed device buffers (for repeated timing).

    ``run()`` enqueues the whole backward; ``states()`` then ``grads()`` enqueue
    its two stages separately (together they are exactly ``run()``).
    """

    def __init__(self, xv, dtda, A, B, C, s0, dy, ds_final, *, chunk_len, out=None, stream=None):
        self.form = FORM_MAMBA2 if A is not None else FORM_RAW
        self.desc = _ssd_inputs(xv, dtda, A, B, C, s0, self.form, chunk_len)
        d = self.desc
        dev = xv.device
        if dy is None:
            raise ValueError("dy is required")
        _need(dy, "dy", xv.dtype, tuple(xv.shape), dev)
        _need(ds_final, "ds_final", torch.float32, (d.batch, d.nheads, d.headdim, d.dstate), dev)
        names = ("dx", "d_dt") if self.form == FORM_MAMBA2 else ("dv", "d_da")
        if out is None:
            out = {names[0]: torch.empty_like(xv), names[1]: torch.empty_like(dtda), "dB": torch.empty_like(B),
                   "dC": torch.empty_like(C),
                   "d_s0": torch.empty((d.batch, d.nheads, d.headdim, d.dstate), dtype=torch.float32, device=dev)}
        _check_out(out, _ssd_grad_spec(d, xv, self.form), dev)
        _on_gpu(dev, xv, dtda, A, B, C, s0, dy, ds_final, *out.values())
        self.out = out
        self.ws, self.wsb = _workspace(ssd_chunk_bwd_workspace(d), dev, None)
        self.stream = stream
        p = _ptr
        self._in = (p(xv), p(dtda), p(A), p(B), p(C))
        self._s0, self._dy, self._dsf = p(s0), p(dy), p(ds_final)
        self._o = (p(out[names[0]]), p(out[names[1]]), p(out["dB"]), p(out["dC"]))
        self._ds0 = p(out["d_s0"])
        self._keep = (xv, dtda, A, B, C, s0, dy, ds_final)

    def run(self):
        st = lib().ssd_chunk_bwd(ctypes.byref(self.desc), *self._in, self._s0, self._dy, self._dsf, *self._o,
                                 self._ds0, _ptr(self.ws), self.wsb, _stream(self.stream))
        _check("ssd_chunk_bwd", st)

    def states(self):
        st = lib().ssd_chunk_bwd_states(ctypes.byref(self.desc), *self._in, self._s0, self._dy, self._dsf,
                                        self._ds0, _ptr(self.ws), self.wsb, _stream(self.stream))
        _check("ssd_chunk_bwd_states", st)

    def grads(self):
        st = lib().ssd_chunk_bwd_grads(ctypes.byref(self.desc), *self._in, self._dy, *self._o, _ptr(self.ws),
                                       self.wsb, _stream(self.stream))
        _check("ssd_chunk_bwd_grads", st)


# --------------------------------------------------------------------------- #
def delta_desc(q, v, scale):
    b, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    return DeltaDesc(b, T, H, HV, K, V, float(scale), 0)


def delta_rule_bwd_workspace(desc):
    n = ctypes.c_size_t(0)
    _check("delta_rule_bwd_workspace", lib().delta_rule_bwd_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def _delta_args(q, k, v, beta, g, S0, d_o, dS_final, want_dS0, out):
    if q is None or v is None or q.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [b,T,H,K] and v [b,T,HV,V]")
    desc = delta_desc(q, v, 1.0)
    b, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    dev, f32 = q.device, torch.float32
    _need(q, "q", f32, (b, T, H, K), dev)
    _need(k, "k", f32, (b, T, H, K), dev)
    _need(v, "v", f32, (b, T, HV, V), dev)
    _need(beta, "beta", f32, (b, T, HV), dev)
    _need(g, "g", f32, (b, T, HV, K), dev)
    _need(S0, "S0", f32, (b, HV, K, V), dev)
    _need(d_o, "d_o", f32, (b, T, HV, V), dev)
    _need(dS_final, "dS_final", f32, (b, HV, K, V), dev)
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("g", g), ("d_o", d_o)):
        if t is None:
            raise ValueError(f"{name} is required")
    if out is None:
        out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v), dg=torch.empty_like(g),
                   dbeta=torch.empty_like(beta),
                   dS0=torch.empty((b, HV, K, V), dtype=f32, device=dev) if want_dS0 else None)
    _check_out(out, dict(dq=(f32, (b, T, H, K)), dk=(f32, (b, T, H, K)), dv=(f32, (b, T, HV, V)),
                         dg=(f32, (b, T, HV, K)), dbeta=(f32, (b, T, HV))), dev)
    _need(out.get("dS0"), "out['dS0']", f32, (b, HV, K, V), dev)
    _on_gpu(dev, q, k, v, beta, g, S0, d_o, dS_final, *out.values())
    p = _ptr
    args = (p(q), p(k), p(v), p(beta), p(g), p(S0), p(d_o), p(dS_final), p(out["dq"]), p(out["dk"]), p(out["dv"]),
            p(out["dg"]), p(out["dbeta"]), p(out.get("dS0")))
    return desc, out, args


def delta_rule_bwd(q, k, v, beta, g, S0, d_o, dS_final=None, *, scale, want_dS0=True, out=None, workspace=None,
                   stream=None):
    """KDA gated delta-rule backward (float32).  Returns dict dq, dk, dv, dg, dbeta, dS0."""
    desc, out, args = _delta_args(q, k, v, beta, g, S0, d_o, dS_final, want_dS0, out)
    desc.scale = float(scale)
    ws, wsb = _workspace(delta_rule_bwd_workspace(desc), q.device, workspace)
    st = lib().delta_rule_bwd(ctypes.byref(desc), *args, _ptr(ws), wsb, _stream(stream))
    _check("delta_rule_bwd", st)
    return out


class DeltaCall:
    """A prepared delta_rule_bwd call on fixed device buffers (for repeated timing).

    ``run()`` enqueues the whole backward; ``stage(DELTA_CKPT)``,
    ``stage(DELTA_BWD)`` and ``stage(DELTA_REDUCE)`` in that order enqueue its
    three kernels separately (together they are exactly ``run()``).
    """

    def __init__(self, q, k, v, beta, g, S0, d_o, dS_final=None, *, scale, want_dS0=True, out=None, stream=None):
        self.desc, self.out, self._args = _delta_args(q, k, v, beta, g, S0, d_o, dS_final, want_dS0, out)
        self.desc.scale = float(scale)
        self.ws, self.wsb = _workspace(delta_rule_bwd_workspace(self.desc), q.device, None)
        self.stream = stream
        self._keep = (q, k, v, beta, g, S0, d_o, dS_final)

    def stage(self, stages):
        st = lib().delta_rule_bwd_stages(ctypes.byref(self.desc), int(stages), *self._args, _ptr(self.ws), self.wsb,
                                         _stream(self.stream))
        _check("delta_rule_bwd_stages", st)

    def run(self):
        self.stage(DELTA_ALL)
