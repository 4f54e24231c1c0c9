"""Seeded synthetic inputs for the F16-weight products.

This module holds shapes and random numbers only: none of the products'
arithmetic.  The same host arrays feed the oracle and the GPU library.

Recipe (the pages' SmolLM2-135M and Llama-3-8B matrices are not available, so
synthetic matrices of the same shapes and value distribution stand in):

* weights: z ~ N(0,1) drawn as float32 by numpy's PCG64 ``standard_normal``,
  multiplied by float32(0.02) and cast to float16 with numpy's own cast; the
  f16 bit patterns are the weights (row-major ``[rows][k]``, k contiguous);
* activations: float32 N(0,1), ``[n][k]``; the paths under test round them to
  f16 themselves.

Seeds: the 576x576 case draws W then A from ``default_rng(0)``.  Other
matrices use ``default_rng([cfg, layer, mat_id, block])`` per block of 2048
rows (so blocks can be drawn in parallel); activations use
``default_rng([cfg, layer, 100 + group])``.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

MAT_IDS = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6, "logits": 7}

# (rows, k) per matrix, weight row-major with k contiguous.
SMOLLM2_135M = {
    "q": (576, 576), "k": (192, 576), "v": (192, 576), "o": (576, 576),
    "gate": (1536, 576), "up": (1536, 576), "down": (576, 1536),
}
SMOLLM2_135M_LOGITS = (49152, 576)      # tied token_embd
SMOLLM2_135M_LAYERS = 30

LLAMA3_8B = {
    "q": (4096, 4096), "k": (1024, 4096), "v": (1024, 4096), "o": (4096, 4096),
    "gate": (14336, 4096), "up": (14336, 4096), "down": (4096, 14336),
}
LLAMA3_8B_LOGITS = (128256, 4096)

# config ids (seed namespace)
CFG_C1, CFG_135M, CFG_135M_PREFILL, CFG_8B, CFG_8B_PREFILL = 1, 2, 3, 4, 5

PREFILL_N = 512
_BLOCK = 2048


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _f16_from_normal(rng, shape) -> np.ndarray:
    z = rng.standard_normal(shape, dtype=np.float32)
    return (z * np.float32(0.02)).astype(np.float16).view(np.uint16)


def weight(cfg: int, layer: int, mat: str, rows: int, k: int) -> np.ndarray:
    """Seeded F16 weight [rows][k] as uint16 bit patterns."""
    mid = MAT_IDS[mat]
    out = np.empty((rows, k), dtype=np.uint16)
    blocks = [(b, min(b + _BLOCK, rows)) for b in range(0, rows, _BLOCK)]

    def fill(blk):
        b0, b1 = blk
        rng = np.random.default_rng([cfg, layer, mid, b0 // _BLOCK])
        out[b0:b1] = _f16_from_normal(rng, (b1 - b0, k))

    if len(blocks) == 1:
        fill(blocks[0])
    else:
        with _cf.ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, blocks))
    return out


def activation(cfg: int, layer: int, group: int, n: int, k: int) -> np.ndarray:
    """Seeded float32 N(0,1) activations [n][k]."""
    rng = np.random.default_rng([cfg, layer, 100 + group])
    return rng.standard_normal((n, k), dtype=np.float32)


def c1():
    """The 576x576 case: W (f16 bits) then A (f32, 3 columns) from seed 0."""
    rng = np.random.default_rng(0)
    w = _f16_from_normal(rng, (576, 576))
    a = rng.standard_normal((3, 576), dtype=np.float32)
    return w, a


def random_f16(seed, shape, scale: float = 1.0) -> np.ndarray:
    """f16 bit patterns of float32(N(0,1) * scale), for sweeps and edge cases."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(shape, dtype=np.float32)
    return (z * np.float32(scale)).astype(np.float16).view(np.uint16)
