"""float64 CPU oracle for the selective state-space scan VJP.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and never imports it.

The arithmetic lives in ``ssm_oracle.c`` (plain C, float64, no fast-math); this
module only builds it with gcc, marshals numpy arrays and allocates outputs.

Functions and the passages they follow:

* ``mamba_seq_fwd`` / ``mamba_seq_bwd`` -- the sequential selective scan and its
  store-all reverse recurrence seeded with the final-state gradient
  (llama.cpp PR "S1-31: SSM_SCAN_BACK", the op description and the
  "grad is the WHOLE packed gradient" / store-all paragraphs).  Mamba-2
  (one decay per head) and Mamba-1 (one decay per state).  Besides the page's
  five gradients the backward returns dA, the gradient of the decay
  coefficients (burn-mamba's combined_backward returns the decay gradient
  d_da; dA = sum over batch and time of d_da * delta).
* ``raw_seq_fwd`` / ``raw_seq_bwd`` -- the same recurrence in the pre-scaled
  (v, da) form with a rank-M input per step: the sequential computation that the
  chunked kernels re-associate (burn-mamba "combined_backward.rs", the K3/K4/K5
  recap comments).
* ``ssd_chunk_fwd`` / ``ssd_chunk_bwd`` -- the chunked SSD forward (K1..K5) and
  the recompute backward in the order of burn-mamba's ``combined_backward``:
  K1..K4 recompute, reverse per-chunk BLUE / ORANGE / K4 loop, batched K3, K2,
  K1 backwards and the combine.
* ``ssd_mamba2_bwd`` -- the chunked backward with the Mamba-2 input chain
  (x, dt, A) -> (v = x*softplus(dt), da = softplus(dt)*A).
* ``kda_fwd`` / ``kda_bwd`` -- the KDA gated delta rule: forward F1..F6 (K3
  notes, "反向传播推导") and its reverse-time adjoint, derived from F1..F6 by
  writing each step as a linear map of the previous state, with the gradients
  of q and k summed over the value heads of each qk head.

Parity pins for every function are in ``tests/test_oracle_*.py`` (finite
differences of the float64 forward, closed forms, a hand-derived worked example,
scipy's IIR filter, torch autograd of an independently written forward,
homogeneity identities, sequential/chunked agreement and mutation kill tests).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "ssm_oracle.c"
_LIB = _HERE / "liboracle.so"

# mutation ids, mirrored from ssm_oracle.c
MUT_NONE = 0
MUT_DROP_DA_PATH = 1
MUT_ZERO_SEED = 2
MUT_DROP_Y_TO_DS = 3
MUT_PREV_STATE_IN_DC = 4
MUT_DROP_SOFTPLUS = 5
MUT_DROP_BLUE_DA = 11
MUT_DROP_ORANGE_DA = 12
MUT_DROP_K3_DA = 13
MUT_DROP_K4_DA = 14
MUT_PREFIX_K1 = 15
MUT_STRICT_MASK = 16
MUT_NO_M_REDUCE = 17
MUT_DROP_KDR = 21
MUT_WRONG_GVA = 22


def build(force: bool = True) -> Path:
    """Compile ssm_oracle.c with gcc (-O2, OpenMP, no fast-math)."""
    if not force and _LIB.exists() and _LIB.stat().st_mtime >= _SRC.stat().st_mtime:
        return _LIB
    tmp = _LIB.with_suffix(".so.tmp%d" % os.getpid())
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-o", str(tmp), str(_SRC), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
            build()
        lib = ctypes.CDLL(str(_LIB))
        i64, dp, ci, cd = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.orc_mamba_seq_fwd.argtypes = [i64] * 6 + [ci] + [dp] * 8 + [ci]
        lib.orc_mamba_seq_bwd.argtypes = [i64] * 6 + [ci] + [dp] * 14 + [ci, ci]
        lib.orc_raw_seq_fwd.argtypes = [i64] * 7 + [dp] * 7 + [ci]
        lib.orc_raw_seq_bwd.argtypes = [i64] * 7 + [dp] * 12 + [ci]
        lib.orc_ssd_chunk_fwd.argtypes = [i64] * 8 + [dp] * 7 + [ci]
        lib.orc_ssd_chunk_bwd.argtypes = [i64] * 8 + [dp] * 12 + [ci, ci]
        lib.orc_ssd_mamba2_bwd.argtypes = [i64] * 7 + [dp] * 13 + [ci, ci]
        lib.orc_kda_fwd.argtypes = [i64] * 6 + [cd] + [dp] * 8 + [ci]
        lib.orc_kda_bwd.argtypes = [i64] * 6 + [cd] + [dp] * 14 + [ci, ci]
        for name in ("orc_mamba_seq_fwd", "orc_mamba_seq_bwd", "orc_raw_seq_fwd", "orc_raw_seq_bwd",
                     "orc_ssd_chunk_fwd", "orc_ssd_chunk_bwd", "orc_ssd_mamba2_bwd",
                     "orc_kda_fwd", "orc_kda_bwd"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"oracle {name} failed with code {rc}")


def default_threads():
    """Threads for the oracle: OMP_NUM_THREADS if set, else the CPUs this process may use."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return os.cpu_count() or 1


def _threads(nthreads):
    return int(nthreads) if nthreads else default_threads()


# --------------------------------------------------------------------------- #
# Mamba sequential (x, dt, A, B, C) form
# --------------------------------------------------------------------------- #

def _mamba_dims(x, B, A):
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    per_state = 1 if A.ndim == 2 else 0
    return b, T, H, P, N, G, per_state


def mamba_seq_fwd(x, dt, A, B, C, s0=None, nthreads=0):
    """Return (y [b,T,H,P], s_final [b,H,P,N])."""
    x, dt, A, B, C, s0 = map(_f64, (x, dt, A, B, C, s0))
    b, T, H, P, N, G, ps = _mamba_dims(x, B, A)
    y = np.zeros((b, T, H, P))
    sf = np.zeros((b, H, P, N))
    _check(_load().orc_mamba_seq_fwd(b, T, H, P, N, G, ps, _p(x), _p(dt), _p(A), _p(B), _p(C),
                                     _p(s0), _p(y), _p(sf), _threads(nthreads)), "mamba_seq_fwd")
    return y, sf


def mamba_seq_bwd(x, dt, A, B, C, s0, dy, ds_final, mutation=MUT_NONE, nthreads=0):
    """Return dict dx, d_dt, dB, dC, d_s0 (same shapes as x, dt, B, C, s0) and
    dA (same shape as A)."""
    x, dt, A, B, C, s0, dy, dsf = map(_f64, (x, dt, A, B, C, s0, dy, ds_final))
    b, T, H, P, N, G, ps = _mamba_dims(x, B, A)
    out = dict(dx=np.zeros_like(x), d_dt=np.zeros_like(dt), dB=np.zeros_like(B),
               dC=np.zeros_like(C), d_s0=np.zeros((b, H, P, N)), dA=np.zeros_like(A))
    _check(_load().orc_mamba_seq_bwd(b, T, H, P, N, G, ps, _p(x), _p(dt), _p(A), _p(B), _p(C),
                                     _p(s0), _p(dy), _p(dsf), _p(out["dx"]), _p(out["d_dt"]),
                                     _p(out["dB"]), _p(out["dC"]), _p(out["d_s0"]), _p(out["dA"]),
                                     int(mutation), _threads(nthreads)), "mamba_seq_bwd")
    return out


# --------------------------------------------------------------------------- #
# RAW (v, da) rank-M form: sequential and chunked
# --------------------------------------------------------------------------- #

def _raw_dims(v, B):
    b, T, M, H, P = v.shape
    G, N = B.shape[3], B.shape[4]
    return b, T, M, H, P, N, G


def raw_seq_fwd(v, da, B, C, s0=None, nthreads=0):
    v, da, B, C, s0 = map(_f64, (v, da, B, C, s0))
    b, T, M, H, P, N, G = _raw_dims(v, B)
    y = np.zeros_like(v)
    sf = np.zeros((b, H, P, N))
    _check(_load().orc_raw_seq_fwd(b, T, M, H, P, N, G, _p(v), _p(da), _p(B), _p(C), _p(s0),
                                   _p(y), _p(sf), _threads(nthreads)), "raw_seq_fwd")
    return y, sf


def raw_seq_bwd(v, da, B, C, s0, dy, ds_final, nthreads=0):
    v, da, B, C, s0, dy, dsf = map(_f64, (v, da, B, C, s0, dy, ds_final))
    b, T, M, H, P, N, G = _raw_dims(v, B)
    out = dict(dv=np.zeros_like(v), d_da=np.zeros_like(da), dB=np.zeros_like(B),
               dC=np.zeros_like(C), d_s0=np.zeros((b, H, P, N)))
    _check(_load().orc_raw_seq_bwd(b, T, M, H, P, N, G, _p(v), _p(da), _p(B), _p(C), _p(s0),
                                   _p(dy), _p(dsf), _p(out["dv"]), _p(out["d_da"]), _p(out["dB"]),
                                   _p(out["dC"]), _p(out["d_s0"]), _threads(nthreads)), "raw_seq_bwd")
    return out


def ssd_chunk_fwd(v, da, B, C, s0, chunk_len, nthreads=0):
    v, da, B, C, s0 = map(_f64, (v, da, B, C, s0))
    b, T, M, H, P, N, G = _raw_dims(v, B)
    y = np.zeros_like(v)
    sf = np.zeros((b, H, P, N))
    _check(_load().orc_ssd_chunk_fwd(b, T, M, H, P, N, G, int(chunk_len), _p(v), _p(da), _p(B), _p(C),
                                     _p(s0), _p(y), _p(sf), _threads(nthreads)), "ssd_chunk_fwd")
    return y, sf


def ssd_chunk_bwd(v, da, B, C, s0, dy, ds_final, chunk_len, mutation=MUT_NONE, nthreads=0):
    v, da, B, C, s0, dy, dsf = map(_f64, (v, da, B, C, s0, dy, ds_final))
    b, T, M, H, P, N, G = _raw_dims(v, B)
    out = dict(dv=np.zeros_like(v), d_da=np.zeros_like(da), dB=np.zeros_like(B),
               dC=np.zeros_like(C), d_s0=np.zeros((b, H, P, N)))
    _check(_load().orc_ssd_chunk_bwd(b, T, M, H, P, N, G, int(chunk_len), _p(v), _p(da), _p(B), _p(C),
                                     _p(s0), _p(dy), _p(dsf), _p(out["dv"]), _p(out["d_da"]),
                                     _p(out["dB"]), _p(out["dC"]), _p(out["d_s0"]), int(mutation),
                                     _threads(nthreads)), "ssd_chunk_bwd")
    return out


def ssd_mamba2_bwd(x, dt, A, B, C, s0, dy, ds_final, chunk_len, mutation=MUT_NONE, nthreads=0):
    """Chunked backward in the Mamba-2 (x, dt, A) input form; outputs as mamba_seq_bwd."""
    x, dt, A, B, C, s0, dy, dsf = map(_f64, (x, dt, A, B, C, s0, dy, ds_final))
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    out = dict(dx=np.zeros_like(x), d_dt=np.zeros_like(dt), dB=np.zeros_like(B),
               dC=np.zeros_like(C), d_s0=np.zeros((b, H, P, N)))
    _check(_load().orc_ssd_mamba2_bwd(b, T, H, P, N, G, int(chunk_len), _p(x), _p(dt), _p(A), _p(B),
                                      _p(C), _p(s0), _p(dy), _p(dsf), _p(out["dx"]), _p(out["d_dt"]),
                                      _p(out["dB"]), _p(out["dC"]), _p(out["d_s0"]), int(mutation),
                                      _threads(nthreads)), "ssd_mamba2_bwd")
    return out


# --------------------------------------------------------------------------- #
# KDA gated delta rule
# --------------------------------------------------------------------------- #

def kda_fwd(q, k, v, beta, g, S0=None, scale=1.0, nthreads=0):
    q, k, v, beta, g, S0 = map(_f64, (q, k, v, beta, g, S0))
    b, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    o = np.zeros_like(v)
    Sf = np.zeros((b, HV, K, V))
    _check(_load().orc_kda_fwd(b, T, H, HV, K, V, float(scale), _p(q), _p(k), _p(v), _p(beta), _p(g),
                               _p(S0), _p(o), _p(Sf), _threads(nthreads)), "kda_fwd")
    return o, Sf


def kda_bwd(q, k, v, beta, g, S0, d_o, dS_final=None, scale=1.0, mutation=MUT_NONE, nthreads=0):
    q, k, v, beta, g, S0, d_o, dSf = map(_f64, (q, k, v, beta, g, S0, d_o, dS_final))
    b, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v), dg=np.zeros_like(g),
               dbeta=np.zeros_like(beta), dS0=np.zeros((b, HV, K, V)))
    _check(_load().orc_kda_bwd(b, T, H, HV, K, V, float(scale), _p(q), _p(k), _p(v), _p(beta), _p(g),
                               _p(S0), _p(d_o), _p(dSf), _p(out["dq"]), _p(out["dk"]), _p(out["dv"]),
                               _p(out["dg"]), _p(out["dbeta"]), _p(out["dS0"]), int(mutation),
                               _threads(nthreads)), "kda_bwd")
    return out
