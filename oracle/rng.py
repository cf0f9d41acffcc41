"""SplitMix64 uniforms for the oracle (test infrastructure only).

SplitMix64 is the generator of Steele, Lea and Flood, "Fast splittable
pseudorandom number generators" (OOPSLA 2014), in the form of Vigna's public
reference implementation: the state advances by the odd constant
0x9E3779B97F4A7C15 and every output is the state passed through a 64-bit
finaliser (xor-shift 30, multiply, xor-shift 27, multiply, xor-shift 31).

Counter form used by the verifier: output number `ctr` (0-based) of a stream
seeded with `seed` is finaliser(seed + (ctr + 1) * 0x9E3779B97F4A7C15 mod 2^64),
so any element can be produced on its own.  A uniform is the top 24 bits of
that output scaled by 2^-24, which lies on the grid {0, 2^-24, ..., 1 - 2^-24}
and is exact in both float32 and float64.

The pages tie reproducibility of sampled outputs to the random seed and the
order in which random numbers are consumed ("EAGLE-3 speculative decoding
review", sections on interpreting losslessness and on lossless versus
numerically identical output); the verifier therefore draws its uniforms from a
counter indexed by (request, position, slot), independent of the outcome.

Pure Python integers: slow and obviously exact.
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def finalise(z: int) -> int:
    """The SplitMix64 output function applied to one 64-bit state."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def splitmix64_output(seed: int, ctr: int) -> int:
    """Output number ctr (0-based) of the SplitMix64 stream seeded with seed."""
    return finalise((seed + (ctr + 1) * GOLDEN_GAMMA) & MASK64)


def splitmix64_stream(seed: int, n: int) -> list:
    """First n outputs of a sequentially stepped SplitMix64 generator."""
    state = seed & MASK64
    out = []
    for _ in range(n):
        state = (state + GOLDEN_GAMMA) & MASK64
        out.append(finalise(state))
    return out


def uniforms_loop(seed: int, counter0: int, n: int) -> np.ndarray:
    """n uniforms u[i] = (output(seed, counter0 + i) >> 40) * 2^-24 as float64,
    one Python integer at a time (small n)."""
    vals = [(splitmix64_output(seed, counter0 + i) >> 40) for i in range(n)]
    return np.asarray(vals, dtype=np.float64) * (2.0 ** -24)


def uniforms(seed: int, counter0: int, n: int) -> np.ndarray:
    """Same values as uniforms_loop, with numpy uint64 arithmetic (which wraps
    modulo 2^64 exactly like the definition) for large n."""
    with np.errstate(over="ignore"):
        ctr = np.arange(n, dtype=np.uint64) + np.uint64((counter0 + 1) & MASK64)
        z = np.uint64(seed & MASK64) + ctr * np.uint64(GOLDEN_GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return (z >> np.uint64(40)).astype(np.float64) * (2.0 ** -24)


def chain_uniforms(seed: int, B: int, k: int, counter0: int = 0) -> np.ndarray:
    """Uniforms for a chain call, shape [B, k+1, 2].

    Slot 0 at position i is the acceptance uniform for draft i; slot 1 is the
    resampling uniform used only at the position where the request stops
    (the first rejection, or the bonus position k).  Flat counter
    ((b * (k+1)) + i) * 2 + slot, offset by counter0.
    """
    return uniforms(seed, counter0, B * (k + 1) * 2).reshape(B, k + 1, 2)


def tree_uniforms(seed: int, B: int, N: int, counter0: int = 0) -> np.ndarray:
    """Uniforms for a tree call, shape [B, N, 2]: slot 0 of node j decides
    node j's test, slot 1 drives the draw if the request stops at node j.
    Flat counter ((b * N) + j) * 2 + slot, offset by counter0 (the chain
    layout with k + 1 = N)."""
    return uniforms(seed, counter0, B * N * 2).reshape(B, N, 2)
