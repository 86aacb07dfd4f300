"""Index maps of the tiled page layout, written from the formulas documented in
include/pkv_spec.h, for tests that read or write raw pool bytes."""
import numpy as np


def k_index(t, c, dtype, D):
    q = D // 4
    j, r = c // q, c % q
    if dtype == "bf16":
        return (r // 8) * 512 + t * 32 + j * 8 + (r % 8)
    return (r // 16) * 1024 + t * 64 + j * 16 + (r % 16)


def v_index(t, c, dtype):
    if dtype == "bf16":
        return ((c // 2) * 4 + t // 4) * 8 + (c % 2) * 4 + (t % 4)
    return ((c // 4) * 4 + t // 4) * 16 + (c % 4) * 4 + (t % 4)


def _grid(D):
    t = np.arange(16)[:, None]
    c = np.arange(D)[None, :]
    return t, c


def detile_k(slab_elems, dtype, D):
    """slab as a flat element array (uint16 for bf16, uint8 for fp8) -> [16, D]."""
    t, c = _grid(D)
    return np.asarray(slab_elems).reshape(-1)[k_index(t, c, dtype, D)]


def detile_v(slab_elems, dtype, D):
    t, c = _grid(D)
    return np.asarray(slab_elems).reshape(-1)[v_index(t, c, dtype)]


def tile_v(rows, dtype, D):
    """[16, D] elements -> flat slab in the V layout."""
    t, c = _grid(D)
    out = np.zeros(16 * D, dtype=np.asarray(rows).dtype)
    out[v_index(t, c, dtype)] = rows
    return out


def tile_k(rows, dtype, D):
    t, c = _grid(D)
    out = np.zeros(16 * D, dtype=np.asarray(rows).dtype)
    out[k_index(t, c, dtype, D)] = rows
    return out
