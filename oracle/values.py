"""Seeded values that the synthetic producers write (oracle side).

The pages fix no input data; their tests only require that every round writes
values distinct from the round before ("Triggered SDMA Plans", *Testing*:
stale-data check over several epochs).  The reading used here: every element
of rank ``rank``'s block in round ``rnd`` at element index ``index`` holds

    k = rank * 2**48 + rnd * 2**32 + index
    h = mix64(k XOR mix64(seed))

where ``mix64`` is the SplitMix64 output function (Steele, Lea & Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014; the constants
are those of Vigna's public-domain ``splitmix64.c``).  From ``h``:

* ``u32`` pattern: the low 32 bits of ``h`` (compared as bits);
* ``u8`` pattern: the low 8 bits of ``h`` (for byte-granular layouts);
* ``bf16`` uniform in [-1, 1): ``u = h >> 41`` (23 bits),
  ``f = (u - 2**22) * 2**-22`` (exact in fp32), bf16 = high half of f's bits.

This module is the oracle's own implementation; the GPU fill kernel carries an
independent one written from the same published definition.
"""

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def mix64_int(x: int) -> int:
    """SplitMix64 output mix of one 64-bit integer (pure Python, exact)."""
    z = x & MASK64
    z = ((z ^ (z >> 30)) * _M1) & MASK64
    z = ((z ^ (z >> 27)) * _M2) & MASK64
    return z ^ (z >> 31)


def splitmix64_stream(seed: int, n: int):
    """The SplitMix64 generator: state += gamma; emit mix64(state)."""
    state = seed & MASK64
    out = []
    for _ in range(n):
        state = (state + GOLDEN_GAMMA) & MASK64
        out.append(mix64_int(state))
    return out


def mix64_np(z: np.ndarray) -> np.ndarray:
    """Vectorised ``mix64`` on uint64 arrays (wrapping multiplies)."""
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= np.uint64(_M1)
        z ^= z >> np.uint64(27)
        z *= np.uint64(_M2)
        z ^= z >> np.uint64(31)
    return z


def element_hash(seed: int, rank: int, rnd: int, index: np.ndarray) -> np.ndarray:
    """h(seed, rank, round, index) for an array of element indices."""
    index = np.asarray(index, dtype=np.uint64)
    if rnd >= (1 << 16) or rank >= (1 << 16):
        raise ValueError("rank and round must fit in 16 bits for this key layout")
    if index.size and int(index.max()) >= (1 << 32):
        raise ValueError("element index must fit in 32 bits for this key layout")
    key = (np.uint64(rank) << np.uint64(48)) | (np.uint64(rnd) << np.uint64(32)) | index
    return mix64_np(key ^ np.uint64(mix64_int(seed)))


def u32_pattern(seed: int, rank: int, rnd: int, index: np.ndarray) -> np.ndarray:
    """Low 32 bits of the element hash, as uint32."""
    return (element_hash(seed, rank, rnd, index) & np.uint64(0xFFFFFFFF)).astype(np.uint32)


def u8_pattern(seed: int, rank: int, rnd: int, index: np.ndarray) -> np.ndarray:
    """Low 8 bits of the element hash, as uint8."""
    return (element_hash(seed, rank, rnd, index) & np.uint64(0xFF)).astype(np.uint8)


def bf16_uniform_bits(seed: int, rank: int, rnd: int, index: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of the uniform [-1, 1) values."""
    h = element_hash(seed, rank, rnd, index)
    u = (h >> np.uint64(41)).astype(np.int64)               # 23 random bits
    f = ((u - (1 << 22)).astype(np.float32) * np.float32(2.0 ** -22))
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def block_bytes(kind: str, seed: int, rank: int, rnd: int, nelem: int, start: int = 0) -> np.ndarray:
    """Bytes of elements [start, start+nelem) of a rank's block, little-endian."""
    idx = np.arange(start, start + nelem, dtype=np.uint64)
    if kind == "u32":
        return u32_pattern(seed, rank, rnd, idx).view(np.uint8)
    if kind == "bf16":
        return bf16_uniform_bits(seed, rank, rnd, idx).view(np.uint8)
    if kind == "u8":
        return u8_pattern(seed, rank, rnd, idx)
    raise ValueError(kind)


ELEM_BYTES = {"u32": 4, "bf16": 2, "u8": 1}
