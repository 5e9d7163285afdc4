"""Seeded input generators (no method arithmetic).

* GEMM operands: A [M, K] and Bt [N, K] drawn from N(0, 1) with a CPU
  ``torch.Generator`` seeded per (seed, rank, round), rounded to bf16, and
  returned as bf16 bit patterns (uint16).  Both sides take the same bits.
* Completion orders: a seeded Fisher-Yates permutation (numpy's
  ``Generator.permutation``) of a rank's chunk indices.
* Replica sentinel: every replica starts filled with the byte 0xA5, so a
  byte that no round wrote is visible.
"""

import numpy as np
import torch

BASE_SEED = 0x7C0FFEE
SENTINEL = 0xA5


def round_seed(seed: int, rank: int, rnd: int) -> int:
    """A distinct generator seed per (seed, rank, round)."""
    return (seed * 1_000_003 + rank * 65_537 + rnd) & 0x7FFF_FFFF_FFFF_FFFF


def gemm_operands(seed: int, rank: int, rnd: int, M: int, N: int, K: int):
    """(A_bits [M,K], Bt_bits [N,K]) as uint16 bf16 bit patterns."""
    g = torch.Generator(device="cpu")
    g.manual_seed(round_seed(seed, rank, rnd))
    a = torch.randn(M, K, generator=g, dtype=torch.float32).to(torch.bfloat16)
    bt = torch.randn(N, K, generator=g, dtype=torch.float32).to(torch.bfloat16)
    return (a.view(torch.int16).numpy().view(np.uint16).copy(),
            bt.view(torch.int16).numpy().view(np.uint16).copy())


def shuffled_order(seed: int, rank: int, rnd: int, n: int) -> np.ndarray:
    """Seeded Fisher-Yates permutation of range(n) for one rank and round."""
    rng = np.random.Generator(np.random.PCG64(round_seed(seed, rank, rnd)))
    return rng.permutation(n).astype(np.uint32)
