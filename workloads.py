"""Seeded synthetic inputs for the NVFP4 projection path.

This module is shared by the tests, the smoke check and the benchmark; it holds
no arithmetic of the method (no quantizer, no codec, no projection).  It only
draws fp32 weights and bf16 activations with the shapes and distributions of
the 27B-class decode projections: weights ~ N(0, 0.02^2), activations ~ N(0, 1)
rounded to bf16, optionally with a fraction of 16-element weight groups scaled
up to exercise the group-scale range.

Two generators:
  * host (numpy PCG64, ``numpy.random.default_rng(seed)``), used for every case
    the CPU oracle checks in full;
  * device (torch's Philox generator on the GPU, seeded per matrix), used for
    the 64-layer decode-step sweep (23 G weights), where a host draw would take
    minutes; tests copy a device draw back to the host to check it.
"""
from __future__ import annotations

import numpy as np
import torch

WEIGHT_STD = 0.02
GROUP = 16  # weights per scale group along k (the "g16" of nvfp4/g16)

# Projection shapes of one 27B-class decoder layer: (name, n_out, k_in).
LAYER_PROJECTIONS = (
    ("qkv", 12288, 5120),
    ("o", 5120, 6144),
    ("gate", 17408, 5120),
    ("up", 17408, 5120),
    ("down", 5120, 17408),
)
SWEEP_LAYERS = 64
SWEEP_ROWS = (1, 2, 4, 8, 16, 32)


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (torch's round-to-nearest-even), returned as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def draw_weights(rng: np.random.Generator, n: int, k: int, outlier_frac: float = 0.0,
                 outlier_mult: float = 50.0) -> np.ndarray:
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(WEIGHT_STD)
    if outlier_frac > 0.0:
        ngroups = n * k // GROUP
        count = int(round(outlier_frac * ngroups))
        idx = rng.choice(ngroups, size=count, replace=False)
        g = w.reshape(ngroups, GROUP)
        g[idx] *= np.float32(outlier_mult)
    return w


def draw_x(rng: np.random.Generator, rows: int, k: int) -> np.ndarray:
    return bf16_bits(rng.standard_normal((rows, k), dtype=np.float32))


def case(n: int, k: int, rows: int, seed: int, outlier_frac: float = 0.0, dual: bool = False):
    """A generic seeded case.  Draw order: weights (gate then up when dual), then x."""
    rng = np.random.default_rng(seed)
    w = draw_weights(rng, n, k, outlier_frac)
    w2 = draw_weights(rng, n, k, outlier_frac) if dual else None
    x = draw_x(rng, rows, k)
    return {"n": n, "k": k, "rows": rows, "W": w, "W_up": w2, "x": x}


# The four single-call workloads (seed i for workload i).
def tiny(seed: int = 0):
    """1 row, k=512, n=256."""
    return case(256, 512, 1, seed)


def qkv_rows1(seed: int = 1):
    """Fused qkv-like projection, n=12288, k=5120, 1 row."""
    return case(12288, 5120, 1, seed)


def gate_up_rows1(seed: int = 2):
    """Dual gate+up with SiLU, two n=17408, k=5120 matrices, 1 row."""
    return case(17408, 5120, 1, seed, dual=True)


def down_rows8(seed: int = 3):
    """Down projection at verify width: n=5120, k=17408, 8 rows, 1% of groups x50."""
    return case(5120, 17408, 8, seed, outlier_frac=0.01)


# ---- device draws for the decode-step sweep ---------------------------------

def sweep_seed(layer: int, proj_index: int) -> int:
    return 4_000_000 + 16 * layer + proj_index


def draw_weights_device(n: int, k: int, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    w = torch.randn((n, k), generator=g, device=device, dtype=torch.float32)
    return w.mul_(WEIGHT_STD)


def draw_x_device(rows: int, k: int, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((rows, k), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
