"""Reference for the GEMM producer (oracle side).

The "Triggered Plans" page (*Model*) uses a tiled GEMM as its example
producer: a persistent kernel that stores each tile of ``C = A @ B`` and
marks the tile's chunk ready.  The pages fix no precision; the reading used
here: bf16 inputs, fp32 accumulation, bf16 output.  ``B`` is held as its
transpose ``Bt [N, K]`` (K contiguous), so ``C = A @ Bt.T``.

The reference is the library matmul in fp32 on bf16-rounded inputs.  Its own
pin is a float64 matmul of the same inputs.
"""

import numpy as np
import torch


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def gemm_ref(a_bits: np.ndarray, bt_bits: np.ndarray) -> np.ndarray:
    """C = A @ Bt.T in fp32 (CPU library matmul) from bf16 bit patterns."""
    a = torch.from_numpy(bf16_bits_to_f32(a_bits))
    bt = torch.from_numpy(bf16_bits_to_f32(bt_bits))
    return (a @ bt.T).numpy()


def gemm_ref_f64(a_bits: np.ndarray, bt_bits: np.ndarray) -> np.ndarray:
    a = bf16_bits_to_f32(a_bits).astype(np.float64)
    bt = bf16_bits_to_f32(bt_bits).astype(np.float64)
    return a @ bt.T


def within_tolerance(got: np.ndarray, ref: np.ndarray, rtol: float = 1e-2):
    """Pass test for the GEMM producer: elementwise
    |got - ref| <= rtol * max(|ref|, rms(ref)), and relative Frobenius error
    <= rtol.  Returns (ok, max_scaled_err, frob_rel_err)."""
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    scale = np.maximum(np.abs(ref), rms)
    scaled = np.abs(got - ref) / np.where(scale > 0, scale, 1.0)
    frob = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    worst = float(scaled.max()) if scaled.size else 0.0
    return (worst <= rtol and frob <= rtol), worst, frob
