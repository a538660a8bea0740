"""Seeded synthetic inputs generated on the GPU with torch (timing workloads).

Same recipe as ``gen.MatrixInputs`` (see the package docstring) but drawn with
torch's device generator, so the 112-matrix workload is produced in seconds.
Values differ from the host generator's (different random streams); parity
tests use the host generator.  Holds no arithmetic of the method.
"""
from __future__ import annotations

import torch

from . import (ENTROPY, GANC_NOISE, GMASK_NOISE, GMASK_SIGNAL, M0_NOISE, S_GANC, S_GMASK, S_M0,
               S_U0, S_U1, S_V0, S_V1, S_W, SIGNAL_POWER, SIGNAL_SCALE, W_STD)
import math


def _seed(cfg, block, mat, stream, k=0) -> int:
    x = (ENTROPY * 1000003 + cfg) * 1000003 + block
    x = (x * 1000003 + mat) * 1000003 + stream
    x = x * 1000003 + k
    return x % (2 ** 62)


def _gen(device, *key):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*key))
    return g


def _haar(device, key, n, r, max_iter=60):
    """Orthonormal n x r factor: the polar factor Z (Z^T Z)^(-1/2) of a Gaussian
    Z (Haar distributed), by the Newton-Schulz iteration X <- X (3I - X^T X) / 2
    started from Z / (sqrt(n) + sqrt(r)) (spectral norm below sqrt(3)).  Uses
    matrix products only, accurate to float32 rounding."""
    z = torch.randn((n, r), generator=_gen(device, *key), device=device, dtype=torch.float32)
    x = z / (n ** 0.5 + r ** 0.5)
    eye = torch.eye(r, device=device, dtype=torch.float32)
    for _ in range(max_iter):
        g = x.t().contiguous() @ x
        err = torch.linalg.matrix_norm(g - eye).item() / r ** 0.5
        x = 1.5 * x - 0.5 * (x @ g)
        if err < 1e-6:
            break
    return x.contiguous()


class DeviceMatrixInputs:
    """drift = theta > 0: the drifting variant, whose anchor gradient k carries the
    signal cos(k theta) S + sin(k theta) S' (S' an independent signal of the same
    spectrum), so the dominant subspaces turn between anchor updates; theta = 0
    is the fixed-subspace recipe."""

    def __init__(self, cfg, block, mat, m, n, device, dtype=torch.float32, drift=0.0):
        self.key = (cfg, block, mat)
        self.m, self.n = m, n
        self.device = device
        self.dtype = dtype
        self.drift = float(drift)
        r = min(m, n)
        i = torch.arange(1, r + 1, device=device, dtype=torch.float32)
        s0 = SIGNAL_SCALE * i.pow(-SIGNAL_POWER)
        u0 = _haar(device, self.key + (S_U0,), m, r)
        v0 = _haar(device, self.key + (S_V0,), n, r)
        self.signal = ((u0 * s0) @ v0.t().contiguous()).contiguous()
        del u0, v0
        self.signal2 = None
        if self.drift > 0.0:
            u1 = _haar(device, self.key + (S_U1,), m, r)
            v1 = _haar(device, self.key + (S_V1,), n, r)
            self.signal2 = ((u1 * s0) @ v1.t().contiguous()).contiguous()
            del u1, v1

    def _anchor_signal(self, k):
        if self.signal2 is None:
            return self.signal
        a = k * self.drift
        return math.cos(a) * self.signal + math.sin(a) * self.signal2

    def _noise(self, stream, k, std):
        return std * torch.randn((self.m, self.n), generator=_gen(self.device, *self.key, stream, k),
                                 device=self.device, dtype=torch.float32)

    def m0(self):
        return (self.signal + self._noise(S_M0, 0, M0_NOISE)).contiguous()

    def g_anc(self, k):
        return (self._anchor_signal(k) + self._noise(S_GANC, k, GANC_NOISE)).to(
            self.dtype).contiguous()

    def g_mask(self, k):
        return (GMASK_SIGNAL * self.signal + self._noise(S_GMASK, k, GMASK_NOISE)).to(
            self.dtype).contiguous()

    def w0(self):
        return self._noise(S_W, 0, W_STD).to(self.dtype).contiguous()
