"""CPU ORACLE of the in-graph activation mask -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU leg may
import this module; the product path never does.  Plain numpy, integer work.

Source: the papernotes.org notes on "Communication-Efficient LLM Adaptation
over Decentralized GPU Meshes", "Key design 1" (in-graph activation masking
with a shared pseudo-random generator): at a pipeline boundary the hidden
states h (T tokens x H dimensions) are multiplied by a 0/1 mask m that keeps
K = round((1 - p) H) dimensions of every token; m is a deterministic function
g of the layer index, the optimizer step and the batch, so sender and
receiver rebuild it locally and only the K kept values of each token travel;
the mask is an element-wise product in the graph, so the gradient of h is the
gradient of the masked states times m (the same index set travels back).

Readings where the notes leave the details open (listed in the design notes):
  * exactly K kept dimensions per token, K = floor((1 - p) H + 1/2);
  * token i keeps the K dimensions j with the smallest 64-bit hash
    u(seed, i, j) (ties, not expected, go to the smaller j): a uniformly random
    K-subset when u behaves like a random function;
  * u(seed, i, j) = mix64(seed + (i H + j + 1) gamma), mix64 the output
    function of SplitMix64 (Steele, Lea and Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014), gamma = 0x9E3779B97F4A7C15;
    seed = mix64(mix64(mix64((layer+1) gamma) ^ (step+1) gamma) ^ (batch+1) gamma);
  * kept values travel in ascending order of their dimension index.
"""
from __future__ import annotations

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1


def mix64(z):
    """SplitMix64 output function on uint64 numpy values (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(M2)
    return z ^ (z >> np.uint64(31))


def mix64_int(z: int) -> int:
    """The same function on a Python integer (64-bit wrap)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def seed_of(layer: int, step: int, batch: int) -> int:
    """The mask seed g(layer, step, batch)."""
    s = mix64_int(((layer + 1) * GAMMA) & MASK64)
    s = mix64_int(s ^ (((step + 1) * GAMMA) & MASK64))
    return mix64_int(s ^ (((batch + 1) * GAMMA) & MASK64))


def keep_count(H: int, p: float) -> int:
    """K = floor((1 - p) H + 1/2): kept dimensions per token at mask rate p."""
    return int(np.floor((1.0 - p) * H + 0.5))


def hashes(seed: int, T: int, H: int, rows=None) -> np.ndarray:
    """u(seed, i, j) for the tokens i in `rows` (default all T) and every j < H."""
    rows = np.arange(T, dtype=np.uint64) if rows is None else np.asarray(rows, dtype=np.uint64)
    c = rows[:, None] * np.uint64(H) + np.arange(H, dtype=np.uint64)[None, :] + np.uint64(1)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(seed) + c * np.uint64(GAMMA))


def indices(layer: int, step: int, batch: int, T: int, H: int, K: int, rows=None) -> np.ndarray:
    """Kept dimensions of each token (int32, [len(rows)][K], ascending)."""
    u = hashes(seed_of(layer, step, batch), T, H, rows)
    out = np.empty((u.shape[0], K), dtype=np.int32)
    j = np.arange(H)
    for r in range(u.shape[0]):
        order = np.lexsort((j, u[r]))  # by hash, then by dimension
        out[r] = np.sort(order[:K])
    return out


def mask(idx: np.ndarray, H: int) -> np.ndarray:
    """The 0/1 mask m of an index set."""
    m = np.zeros((idx.shape[0], H), dtype=np.uint8)
    np.put_along_axis(m, idx.astype(np.int64), 1, axis=1)
    return m


def pack(x: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """The kept values of each token, in ascending dimension order."""
    return np.take_along_axis(np.asarray(x), idx.astype(np.int64), axis=1)


def unpack(v: np.ndarray, idx: np.ndarray, H: int) -> np.ndarray:
    """Dense masked states h * m from the kept values (zeros elsewhere)."""
    v = np.asarray(v)
    out = np.zeros((v.shape[0], H), dtype=v.dtype)
    np.put_along_axis(out, idx.astype(np.int64), v, axis=1)
    return out
