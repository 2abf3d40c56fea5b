"""Random-sign Hadamard transform along the head dimension (test infra only).

Source: "FlashAttention-3: Fast & Accurate Attention with Asynchrony &
Low-Precision" (Embodied AI 101 transcript), section "Incoherent Processing for
FP8 Accuracy": queries and keys are multiplied by a random orthogonal matrix
per head, realised as a Hadamard transform with random signs in O(d log d).
The review "FlashAttention-3: почему внимание стало быстрее", section "Метод",
item 3, describes the same step as incoherent processing before quantisation.

Reading (the pages do not fix the matrix): M = diag(s) H_d / sqrt(d), with H_d
the Sylvester-ordered Hadamard matrix of order d (d a power of two) and s a
vector of +-1 per head. A row x becomes x M = H_d (s * x) / sqrt(d) (H_d is
symmetric). M is orthogonal, so (Q M)(K M)^T = Q K^T and attention is
unchanged; V is not rotated.
"""

import numpy as np


def fwht(x):
    """Unnormalised Walsh-Hadamard transform along the last axis, float64.

    Sylvester ordering: the result equals x @ H_d with H_1 = [1],
    H_2n = [[H_n, H_n], [H_n, -H_n]]. Butterflies of span 1, 2, 4, ...
    """
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("Hadamard transform needs a power-of-two length")
    h = 1
    while h < d:
        shp = y.shape[:-1] + (d // (2 * h), 2, h)
        z = y.reshape(shp)
        a = z[..., 0, :].copy()
        b = z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(y.shape)
        h *= 2
    return y


def random_sign_hadamard(x, signs):
    """x M with M = diag(signs) H_d / sqrt(d), applied to the last axis.

    x: [..., H, N, d]; signs: [H, d] of +-1 (one vector per head, shared by Q
    and K of that head). Returns float64.
    """
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64)
    d = x.shape[-1]
    return fwht(x * s[:, None, :]) / np.sqrt(d)
