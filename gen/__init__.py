"""Seeded synthetic inputs for the spectral-correction optimizer step.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no EMA, SVD, filter, projection or AdamW).  Both the HIP
path's tests/benchmark and the CPU oracle consume the arrays produced here.

Workload recipe (shapes and distributions of the fine-tuning setting described
in "Communication-Efficient LLM Adaptation over Decentralized GPU Meshes",
papernotes.org notes, sections "Key design 2/3" and "Training strategy"):

* a low-rank "slowly drifting" signal S = U0 diag(s0) V0^T with U0, V0 Haar
  orthonormal (QR of a Gaussian, column signs fixed by diag(R) > 0) and a power
  law spectrum s0_i = 1e-2 * i^-1.5, i = 1..r0, r0 = min(m, n) by default;
* initial anchor momentum M0 = S + N(0, 1e-4)   (N(0, x): x is the std-dev);
* each anchor gradient G_anc_k = S + fresh N(0, 1e-4);
* each masked gradient G_mask_k = 0.5 * S + fresh N(0, 1e-3);
* a second shape set, Llama-3-8B blocks, for the 8B-class workloads;
* weights W0 ~ N(0, 0.02).

Values are drawn in float64 and rounded once, round-to-nearest-even, to the
storage dtype (float32; bfloat16 goes float64 -> float32 -> bfloat16, both
RNE).  Every matrix can be regenerated on its own from
``SeedSequence(ENTROPY, spawn_key=(cfg, block, mat, stream, k))``.
"""
from __future__ import annotations

import numpy as np

ENTROPY = 260914339

# stream ids inside a spawn key
S_U0, S_V0, S_M0, S_GANC, S_GMASK, S_W = 0, 1, 2, 3, 4, 5
S_U1, S_V1 = 6, 7  # second signal of the drifting variant (timing workloads only)

# Llama-3.2-1B block shapes, row-major [out, in]
BLOCK_SHAPES = (
    ("q", 2048, 2048),
    ("k", 512, 2048),
    ("v", 512, 2048),
    ("o", 2048, 2048),
    ("gate", 8192, 2048),
    ("up", 8192, 2048),
    ("down", 2048, 8192),
)
N_BLOCKS = 16

# Llama-3-8B block shapes (public model configuration: hidden 4096, 32 query and
# 8 key/value heads of 128, MLP 14336), row-major [out, in]; the 32 blocks'
# fp32 states exceed one GPU, so workloads take a few blocks at a time
BLOCK_SHAPES_8B = (
    ("q", 4096, 4096),
    ("k", 1024, 4096),
    ("v", 1024, 4096),
    ("o", 4096, 4096),
    ("gate", 14336, 4096),
    ("up", 14336, 4096),
    ("down", 4096, 14336),
)

SIGNAL_SCALE = 1e-2
SIGNAL_POWER = 1.5
M0_NOISE = 1e-4
GANC_NOISE = 1e-4
GMASK_SIGNAL = 0.5
GMASK_NOISE = 1e-3
W_STD = 0.02


def rng(cfg: int, block: int, mat: int, stream: int, k: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(ENTROPY, spawn_key=(int(cfg), int(block), int(mat), int(stream), int(k)))
    return np.random.Generator(np.random.PCG64(ss))


def haar(g: np.random.Generator, n: int, r: int) -> np.ndarray:
    """n x r matrix with orthonormal columns, Haar distributed (r <= n)."""
    z = g.standard_normal((n, r))
    q, rr = np.linalg.qr(z)
    sgn = np.sign(np.diag(rr))
    sgn[sgn == 0] = 1.0
    return q * sgn


def spectrum(r0: int) -> np.ndarray:
    i = np.arange(1, r0 + 1, dtype=np.float64)
    return SIGNAL_SCALE * i ** (-SIGNAL_POWER)


def to_f32(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


class MatrixInputs:
    """All synthetic inputs of one weight matrix, regenerated lazily from seeds.

    ``cfg`` / ``block`` / ``mat`` name the matrix; ``r0`` the signal rank.
    Float64 "exact" values are available for tests that need them.
    """

    def __init__(self, cfg: int, block: int, mat: int, m: int, n: int, r0: int | None = None,
                 noise: bool = True):
        self.cfg, self.block, self.mat, self.m, self.n = cfg, block, mat, m, n
        self.r0 = min(m, n) if r0 is None else int(r0)
        self.noise = noise
        self._sig = None

    def factors(self):
        """(U0 [m, r0], s0 [r0], V0 [n, r0]) in float64."""
        if self._sig is None:
            u0 = haar(rng(self.cfg, self.block, self.mat, S_U0), self.m, self.r0)
            v0 = haar(rng(self.cfg, self.block, self.mat, S_V0), self.n, self.r0)
            self._sig = (u0, spectrum(self.r0), v0)
        return self._sig

    def signal(self) -> np.ndarray:
        u0, s0, v0 = self.factors()
        return (u0 * s0) @ v0.T

    def _noise(self, stream: int, k: int, std: float) -> np.ndarray:
        if not self.noise:
            return np.zeros((self.m, self.n))
        return std * rng(self.cfg, self.block, self.mat, stream, k).standard_normal((self.m, self.n))

    def m0(self) -> np.ndarray:
        return self.signal() + self._noise(S_M0, 0, M0_NOISE)

    def g_anc(self, k: int) -> np.ndarray:
        return self.signal() + self._noise(S_GANC, k, GANC_NOISE)

    def g_mask(self, k: int) -> np.ndarray:
        return GMASK_SIGNAL * self.signal() + self._noise(S_GMASK, k, GMASK_NOISE)

    def w0(self) -> np.ndarray:
        return W_STD * rng(self.cfg, self.block, self.mat, S_W, 0).standard_normal((self.m, self.n))


def stored(x64: np.ndarray, dtype: str):
    """Round float64 values to the storage dtype.

    Returns (payload, as_float64): payload is float32 array for 'f32' or the
    uint16 bit patterns for 'bf16'; as_float64 is the exactly representable
    stored value widened back to float64.
    """
    f = to_f32(x64)
    if dtype == "f32":
        return f, f.astype(np.float64)
    if dtype == "bf16":
        b = f32_to_bf16_bits(f)
        return b, bf16_bits_to_f32(b).astype(np.float64)
    raise ValueError(dtype)


# ---- named workloads -------------------------------------------------------

DEFAULT_HP = dict(tau_p=1e-3, alpha=0.3, beta_anc=0.9, lr=2e-5, beta1=0.9, beta2=0.999,
                  eps=1e-8, weight_decay=0.01)


def workload(name: str):
    """Shapes and schedule of a named workload.

    Returns dict(shapes=[(m, n), ...], ids=[(cfg, block, mat), ...],
    steps_per_anchor=int, dtype=str).
    """
    if name == "single_64x48":
        return dict(shapes=[(64, 48)], ids=[(1, 0, 0)], steps_per_anchor=5, dtype="f32")
    if name == "q_proj_2048":
        return dict(shapes=[(2048, 2048)], ids=[(2, 0, 0)], steps_per_anchor=25, dtype="f32")
    if name == "block_1b":
        return dict(shapes=[(m, n) for _, m, n in BLOCK_SHAPES],
                    ids=[(3, 0, i) for i in range(7)], steps_per_anchor=20, dtype="f32")
    if name in ("blocks16_1b", "blocks16_1b_bf16"):
        shapes, ids = [], []
        for b in range(N_BLOCKS):
            for i, (_, m, n) in enumerate(BLOCK_SHAPES):
                shapes.append((m, n))
                ids.append((4 if name == "blocks16_1b" else 5, b, i))
        return dict(shapes=shapes, ids=ids,
                    steps_per_anchor=25 if name == "blocks16_1b" else 1,
                    dtype="f32" if name == "blocks16_1b" else "bf16")
    if name in ("block_8b", "blocks4_8b"):
        nblk = 1 if name == "block_8b" else 4
        shapes, ids = [], []
        for b in range(nblk):
            for i, (_, m, n) in enumerate(BLOCK_SHAPES_8B):
                shapes.append((m, n))
                ids.append((6, b, i))
        return dict(shapes=shapes, ids=ids, steps_per_anchor=25, dtype="f32")
    raise KeyError(name)
