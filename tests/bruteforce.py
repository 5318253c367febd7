"""A second, deliberately different statement of masked attention, used only to
check the oracle on tiny inputs.

Where the oracle walks each query's key range in C, this builds the whole
query-by-key mask matrix in numpy from the positions, exponentiates the raw
scores without subtracting a maximum (inputs are tiny and well scaled), and
normalises with ``math.fsum``.  It takes dequantised keys and values.
"""
import math

import numpy as np


def mask_matrix(pos, window, key_pos):
    """M[r, j] = 1 when key position key_pos[j] is attended by a query at
    pos[r] with window window[r] (0 = no window)."""
    pos = np.asarray(pos)[:, None]
    window = np.asarray(window)[:, None]
    kp = np.asarray(key_pos)[None, :]
    causal = kp <= pos
    in_window = (window == 0) | (kp > pos - window)
    return causal & in_window


def attend(q, pos, window, key_pos, k_hat, v_hat, scale):
    q = np.asarray(q, dtype=np.float64)
    m = mask_matrix(pos, window, key_pos)
    raw = np.exp((q @ np.asarray(k_hat, dtype=np.float64).T) * scale)
    out = np.zeros((q.shape[0], v_hat.shape[1]))
    for r in range(q.shape[0]):
        w = [raw[r, j] for j in range(len(key_pos)) if m[r, j]]
        vs = [v_hat[j] for j in range(len(key_pos)) if m[r, j]]
        z = math.fsum(w)
        for c in range(v_hat.shape[1]):
            out[r, c] = math.fsum(wi * vi[c] for wi, vi in zip(w, vs)) / z
    return out
