"""Counter-based random numbers for the codec's own seeded draws (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The pages call for a random orthogonal rotation (JoLT abstract, the sentence
introducing the method) and a randomized SVD (abstract, FlashJoLT sentence) but
fix no generator.  Reading: both sides implement the same published
counter-based generator independently, so a draw is a pure function of
(seed, stream tag, index):

* ``mix64`` is the SplitMix64 output finalizer (Steele, Lea & Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014).
* The stream key is ``mix64(seed XOR tag)``.  Word ``i`` of a stream is the
  ``i``-th output of the standard sequential SplitMix64 generator whose state
  starts at the key: ``mix64(key + (i + 1) * 0x9E3779B97F4A7C15 mod 2^64)``.
* A uniform is ``((word >> 11) + 0.5) * 2^-53``, in the open interval (0, 1).
* Normals come in Box-Muller pairs (Box & Muller 1958): for pair ``k`` with
  uniforms ``u1 = U(2k)``, ``u2 = U(2k+1)`` and ``rad = sqrt(-2 ln u1)``,
  element ``2k`` is ``rad * cos(2 pi u2)`` and element ``2k+1`` is
  ``rad * sin(2 pi u2)``; computed in fp64.
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB

# Stream tags (ASCII "JOLTROT1", "JOLTSKT1").  A per-tensor stream XORs the
# tag with (layer << 8 | kind), kind 0 = K, 1 = V.
TAG_ROTATION = 0x4A4F4C54524F5431
TAG_SKETCH = 0x4A4F4C54534B5431


def mix64(z: int) -> int:
    """SplitMix64 finalizer on a Python int (mod 2^64)."""
    z &= MASK64
    z ^= z >> 30
    z = (z * _M1) & MASK64
    z ^= z >> 27
    z = (z * _M2) & MASK64
    z ^= z >> 31
    return z


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    z ^= z >> np.uint64(30)
    z *= np.uint64(_M1)          # uint64 multiply wraps mod 2^64
    z ^= z >> np.uint64(27)
    z *= np.uint64(_M2)
    z ^= z >> np.uint64(31)
    return z


def stream_key(seed: int, tag: int) -> int:
    return mix64((seed ^ tag) & MASK64)


def tensor_tag(tag: int, layer: int, kind: int) -> int:
    """Per-tensor stream tag: purpose tag XOR (layer << 8 | kind)."""
    return (tag ^ ((layer << 8) | kind)) & MASK64


def sequence(state: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` of sequential SplitMix64 from ``state``.

    Output i is mix64(state + (i + 1) * GAMMA mod 2^64): the generator adds
    GAMMA to its state, then finalizes.
    """
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        st = np.uint64(state & MASK64) + idx * np.uint64(GAMMA)
    return _mix64_np(st)


def words(seed: int, tag: int, start: int, count: int) -> np.ndarray:
    """Words ``start .. start+count-1`` of stream (seed, tag), uint64."""
    return sequence(stream_key(seed, tag), start, count)


def uniforms(seed: int, tag: int, start: int, count: int) -> np.ndarray:
    w = words(seed, tag, start, count)
    return ((w >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def normals(seed: int, tag: int, count: int) -> np.ndarray:
    """Elements ``0 .. count-1`` of the Box-Muller normal stream (fp64)."""
    npairs = (count + 1) // 2
    u = uniforms(seed, tag, 0, 2 * npairs)
    u1 = u[0::2]
    u2 = u[1::2]
    rad = np.sqrt(-2.0 * np.log(u1))
    ang = 2.0 * np.pi * u2
    out = np.empty(2 * npairs, dtype=np.float64)
    out[0::2] = rad * np.cos(ang)
    out[1::2] = rad * np.sin(ang)
    return out[:count]
