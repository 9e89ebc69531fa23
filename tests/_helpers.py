"""Shared test helpers: error metric and central finite differences."""
import numpy as np


def rel_maxabs(got, ref):
    """max_i |got_i - ref_i| / max_i |ref_i| over one tensor (0/0 -> 0)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert got.size > 0, "empty comparison"
    den = np.max(np.abs(ref))
    num = np.max(np.abs(got - ref))
    if den == 0.0:
        return float(num)
    return float(num / den)


def fd_grads(objective, inputs, keys, eps=1e-5, max_per_key=None, rng=None):
    """Central differences of ``objective(inputs)`` w.r.t. every element of each key.

    Returns (grads, counts): grads[key] has NaN where an element was not probed.
    With ``max_per_key`` a random subset of elements is probed.
    """
    grads, counts = {}, {}
    for key in keys:
        base = inputs[key]
        g = np.full(base.shape, np.nan)
        flat_idx = np.arange(base.size)
        if max_per_key is not None and base.size > max_per_key:
            rng = rng or np.random.default_rng(0)
            flat_idx = rng.choice(base.size, size=max_per_key, replace=False)
        for i in flat_idx:
            idx = np.unravel_index(i, base.shape)
            plus = dict(inputs)
            minus = dict(inputs)
            p = base.copy()
            m = base.copy()
            p[idx] += eps
            m[idx] -= eps
            plus[key] = p
            minus[key] = m
            g[idx] = (objective(plus) - objective(minus)) / (2.0 * eps)
        grads[key] = g
        counts[key] = len(flat_idx)
    return grads, counts


def rel_maxabs_probed(got, fd):
    """rel_maxabs restricted to the probed (non-NaN) elements of an FD gradient."""
    mask = ~np.isnan(fd)
    assert mask.sum() > 0, "no element was probed"
    return rel_maxabs(np.asarray(got)[mask], fd[mask])
