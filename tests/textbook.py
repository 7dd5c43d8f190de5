"""Textbook contiguous attention in numpy fp64, independent of the oracle.

Used only to pin the oracle: with an identity block table, paged decode must
equal ordinary attention over each sequence's contiguous K/V rows.  Stored
values are decoded with torch's own dtype casts, never with the oracle's
decoders.
"""

import numpy as np
import scipy.special
import torch


def to_f64(t) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def attention(q, K, V, scale):
    """q [H, D]; K, V [L, Hkv, D] (float64) -> [H, D] = softmax(scale q K^T) V per head."""
    H, D = q.shape
    L, Hkv, _ = K.shape
    G = H // Hkv
    out = np.zeros((H, D))
    if L == 0:
        return out
    for h in range(H):
        s = scale * (K[:, h // G, :] @ q[h])
        out[h] = scipy.special.softmax(s) @ V[:, h // G, :]
    return out
