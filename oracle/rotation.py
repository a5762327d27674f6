"""The seeded random orthogonal rotation of the residual (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: JoLT abstract (arXiv 2607.12550v2), the method sentence: the residual
is rotated by a random orthogonal matrix before low-bit quantization; news
article paragraphs 2 and 4 call it a Johnson-Lindenstrauss rotation that
whitens the residual.

Readings: the rotation acts on the feature axis of every (head, token) residual
vector, y = Q r, so in row form Y = R Q^T and the inverse is R = Y Q.  It is
square (D x D, no dimension reduction) and Haar distributed: A[i, j] is normal
number i*D + j of the rotation stream of ``seed``, and Q is the Q factor of
A's Householder QR with the signs chosen so that diag(R) > 0 (the unique QR with
positive diagonal, which makes Q Haar; Mezzadri, "How to generate random
matrices from the classical compact groups", Notices AMS 2007).  One Q per seed
serves every tensor, so it costs no bytes in the compressed record.
"""
from __future__ import annotations

import numpy as np

from . import rng


def gaussian_matrix(seed: int, D: int) -> np.ndarray:
    return rng.normals(seed, rng.TAG_ROTATION, D * D).reshape(D, D)


def rotation(seed: int, D: int) -> np.ndarray:
    A = gaussian_matrix(seed, D)
    Q, R = np.linalg.qr(A)
    s = np.sign(np.diag(R))
    s[s == 0] = 1.0
    return Q * s
