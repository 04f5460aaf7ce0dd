"""NumPy's own Philox4x64-10 (an implementation independent of the oracle's and the
library's), used by the tests to recompute the uniforms a call draws.

NumPy's Philox advances its counter before producing a block, so block(c) comes from a
generator whose counter is c - 1 (a 256-bit little-endian decrement)."""
import numpy as np


def block(counter, key) -> np.ndarray:
    c = [int(x) for x in counter]
    val = sum(w << (64 * i) for i, w in enumerate(c))
    val = (val - 1) % (1 << 256)
    prev = np.array([(val >> (64 * i)) & ((1 << 64) - 1) for i in range(4)], dtype=np.uint64)
    g = np.random.Philox(counter=prev, key=np.array([int(k) for k in key], dtype=np.uint64))
    return g.random_raw(4).astype(np.uint64)


def word_to_uniform(w: int) -> float:
    """(2 (w >> 12) + 1) 2^-53: an odd 53-bit integer over 2^53, exact in fp64."""
    return (2 * (int(w) >> 12) + 1) / 2.0 ** 53


def uniform(seed: int, c0: int, step: int, stream: int, tag: int) -> float:
    return word_to_uniform(block([c0, step, stream, tag], [seed, 0])[0])
