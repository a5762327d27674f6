"""Seeded synthetic KV-cache tensors (input generator shared by tests and bench).

This module only makes inputs.  It holds none of the codec's arithmetic and is
the one module that both the HIP path's tests/bench and the CPU oracle use.

The pages measure on real Mistral-7B-v0.3 (GQA, 8 KV heads) and LLaMA-2-13B
(MHA, 40 heads) caches (JoLT abstract, arXiv 2607.12550v2, the results
sentences).  No weights or corpora are available, so these synthetic tensors
stand in for them, with the models' cache shapes (head_dim D = 128):

  X_h = A diag(sigma * c_h) B^T + eps          (h = 0 .. H-1)

* A (T x r0) and B (D x r0) are orthonormal (Q factors of Gaussian matrices),
  r0 = min(96, T, D) rank-1 terms shared by all heads;
* sigma_i = sqrt(T D) * decay^i, so entries are O(1);
* c_h ~ N(0, 1) per head and term (per-head mixing);
* eps ~ N(0, 0.01), read as variance 0.01 (standard deviation 0.1);
* outlier feature channels d in {D/8, 3D/8, 5D/8, 7D/8} (one per group of 32
  features) are multiplied by 8 after the noise is added;
* decay is 0.9 for the single-tensor case and drawn per (layer, kind)
  uniformly from [0.85, 0.95] for whole caches;
* bf16 inputs are generated in fp64 and rounded (fp32, then bf16 nearest-even).

Random numbers come from numpy's PCG64 keyed by (seed, layer, kind, purpose),
so every tensor is reproducible on its own.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

RANK = 96
NOISE_STD = 0.1
OUTLIER_SCALE = 8.0

_P_SIGNAL, _P_DECAY = 0x5EED, 0xDECA


@dataclass(frozen=True)
class CacheConfig:
    name: str
    n_layers: int
    H: int
    T: int
    D: int
    dtype: str                     # "f32" or "bf16"
    ratio: float = 0.0             # byte budget vs bf16; 0 = fixed choice
    method: str = "exact"          # "exact" or "flash"
    outliers: str = "KV"           # kinds that carry outlier channels
    kinds: tuple = (0, 1)
    fixed_choice: tuple = ()       # (r_T, r_D, bits) when ratio == 0
    fixed_decay: float = 0.0       # 0 = draw per (layer, kind)
    bits: tuple = (1, 2, 3, 4)
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def elems(self) -> int:
        return self.H * self.T * self.D


CONFIGS = {
    # single K tensor, fixed ranks and bits
    "single_k_t1024_f32": CacheConfig("single_k_t1024_f32", 1, 8, 1024, 128, "f32",
                                      kinds=(0,), fixed_choice=(256, 64, 2),
                                      fixed_decay=0.9),
    # Mistral-7B-v0.3-shaped GQA cache, 2x budget, exact factors
    "mistral7b_t4096_2x": CacheConfig("mistral7b_t4096_2x", 32, 8, 4096, 128, "bf16",
                                      ratio=2.0),
    # LLaMA-2-13B-shaped MHA cache, 2x budget, outliers in K only
    "llama13b_t4096_2x": CacheConfig("llama13b_t4096_2x", 40, 40, 4096, 128, "bf16",
                                     ratio=2.0, outliers="K"),
    # Mistral-7B shape at 1024 tokens, FlashJoLT vs exact
    "mistral7b_t1024_flash": CacheConfig("mistral7b_t1024_flash", 32, 8, 1024, 128,
                                         "bf16", ratio=2.0, method="flash"),
    # long-context Mistral-7B shape, 3x budget, FlashJoLT encode
    "mistral7b_t32768_3x": CacheConfig("mistral7b_t32768_3x", 32, 8, 32768, 128,
                                       "bf16", ratio=3.0, method="flash"),
}


def round_bf16_f32(x: np.ndarray) -> np.ndarray:
    """fp64/fp32 -> fp32 -> bf16 (nearest-even on the fp32 bits); fp32 result."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _orthonormal(g: np.ndarray) -> np.ndarray:
    q, r = np.linalg.qr(g)
    return q


def decay_for(seed: int, layer: int, kind: int) -> float:
    rng = np.random.default_rng([seed, layer, kind, _P_DECAY])
    return float(rng.uniform(0.85, 0.95))


def tensor(H: int, T: int, D: int, *, seed: int = 0, layer: int = 0, kind: int = 0,
           decay: float = 0.9, outliers: bool = True, dtype: str = "f32",
           noise_std: float = NOISE_STD, rank: int = RANK) -> np.ndarray:
    """One synthetic K or V tensor [H, T, D] as fp32 (bf16-exact if dtype='bf16')."""
    rng = np.random.default_rng([seed, layer, kind, _P_SIGNAL])
    r0 = min(rank, T, D)
    A = _orthonormal(rng.standard_normal((T, r0)))
    B = _orthonormal(rng.standard_normal((D, r0)))
    sigma = np.sqrt(float(T * D)) * decay ** np.arange(r0)
    c = rng.standard_normal((H, r0))
    X = np.empty((H, T, D), dtype=np.float64)
    for h in range(H):
        X[h] = (A * (sigma * c[h])) @ B.T
    X += noise_std * rng.standard_normal((H, T, D))
    if outliers:
        ch = [D // 8, 3 * D // 8, 5 * D // 8, 7 * D // 8]
        X[:, :, ch] *= OUTLIER_SCALE
    if dtype == "bf16":
        return round_bf16_f32(X)
    if dtype == "f32":
        return X.astype(np.float32)
    raise ValueError(dtype)


def config_tensor(cfg: CacheConfig, layer: int, kind: int, T: int | None = None) -> np.ndarray:
    """Tensor (layer, kind) of a cache configuration (optionally at another T)."""
    decay = cfg.fixed_decay if cfg.fixed_decay > 0 else decay_for(cfg.seed, layer, kind)
    out = (kind == 0 and "K" in cfg.outliers) or (kind == 1 and "V" in cfg.outliers)
    return tensor(cfg.H, cfg.T if T is None else T, cfg.D, seed=cfg.seed, layer=layer,
                  kind=kind, decay=decay, outliers=out, dtype=cfg.dtype)


def _config_item(args):
    name, layer, kind = args
    return layer, kind, config_tensor(CONFIGS[name], layer, kind)


def generate(cfg: CacheConfig, items, workers: int = 8):
    """Yield (layer, kind, tensor) for every (layer, kind) in ``items``, made by
    ``workers`` spawned processes (completion order).  Spawned, not forked, so
    the caller may already hold a GPU context."""
    import multiprocessing as mp
    items = [(cfg.name, int(l), int(k)) for l, k in items]
    if workers <= 1 or len(items) <= 1:
        for it in items:
            yield _config_item(it)
        return
    import os
    keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in keys}
    os.environ.update({k: "1" for k in keys})      # one BLAS thread per worker
    try:
        pool = mp.get_context("spawn").Pool(min(workers, len(items)))
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    try:
        yield from pool.imap_unordered(_config_item, items)
    finally:
        # let the workers finish and exit on their own (terminating them
        # makes every worker report an abort)
        pool.close()
        pool.join()
