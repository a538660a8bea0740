"""CPU fp64 ORACLE of the spectral-correction optimizer step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (``spectral_correction_optimizer_amd``) never imports it and shares no
code with it; the only common module is ``gen`` (seeded random inputs, no
method arithmetic).

Source of every step: the papernotes.org notes on "Communication-Efficient LLM
Adaptation over Decentralized GPU Meshes" (arXiv 2609.14339):

  O1  anchor EMA      -- "Key design 2" (async dual circuit), the EMA equation
                          for the anchor momentum buffer M^anc.
  O2  thin SVD        -- "Key design 3" (spectral-correction optimizer), the
                          SVD M^anc = U S V^T; own one-sided Jacobi in C
                          (oracle/jacobi.c), nothing truncated.
  O3  Tikhonov filter -- "Key design 3", d_i = s_i / (s_i + tau_p).
  O4  two-sided projection and reconstruction -- "Key design 3", the three
                          equations X = U^T G V, X_filt = diag(d) X diag(d),
                          G_filt = U X_filt V^T.
  O5  convex combination -- "Key design 3", G_proj = a G_mask + (1-a) G_filt.
  O6  AdamW           -- the overview ("Overall framework": denoised gradient
                          goes to AdamW) and "Training strategy" (AdamW with
                          peak lr 2e-5); decoupled weight decay as in
                          Loshchilov & Hutter / torch.optim.AdamW.

All arithmetic is float64.  Inputs are the exact values the GPU receives
(float32 or bfloat16) widened to float64.  The stateful driver ``Optimizer``
rounds the tensors the configuration stores in a narrower type (W, m, v,
M_anc) to that type, round-to-nearest-even, at the end of each call.

Readings where the pages are silent (each listed with its reason in the
design notes of the repository):
  * thin SVD, r = min(m, n), nothing truncated;
  * d_i = 0 when s_i + tau_p = 0 (the tau -> 0+ limit);
  * M_anc starts at zero; the SVD is refreshed only when M_anc changes;
  * AdamW: eps outside the square root, bias correction on, decay scaled by
    lr and applied to the pre-step weights, step count advanced per step.

Pins (tests/test_oracle_*.py) tie every function to facts other than itself:
a hand-worked 4x3 case, closed forms, LAPACK singular values, torch's AdamW,
brute force on 2x2, invariants and equivariances.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_jacobi.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle/jacobi.c with gcc into liboracle_jacobi.so."""
    import subprocess
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fPIC", "-shared",
               "-std=c11", "-o", _LIB_PATH + ".tmp", os.path.join(_HERE, "jacobi.c"), "-lm",
               "-lpthread"]
        subprocess.check_call(cmd)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_jacobi_svd.restype = ctypes.c_int
        lib.oracle_jacobi_svd.argtypes = [ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 4 + [
            ctypes.c_int, ctypes.c_int]
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


# ---- O1 ---------------------------------------------------------------------

def ema(M: np.ndarray, G_anc: np.ndarray, beta_anc: float) -> np.ndarray:
    """Anchor momentum EMA: M <- beta_anc * M + (1 - beta_anc) * G_anc."""
    return beta_anc * np.asarray(M, np.float64) + (1.0 - beta_anc) * np.asarray(G_anc, np.float64)


# ---- O2 ---------------------------------------------------------------------

def svd(M: np.ndarray, max_sweeps: int = 100, threads: int | None = None):
    """Thin SVD by fp64 one-sided Jacobi (oracle/jacobi.c).

    Returns (U [m, r], s [r] descending, V [n, r], sweeps); sweeps < 0 means the
    sweep cap was reached before a rotation-free sweep.
    """
    M = np.ascontiguousarray(M, dtype=np.float64)
    m, n = M.shape
    r = min(m, n)
    U = np.zeros((m, r))
    s = np.zeros(r)
    V = np.zeros((n, r))
    if threads is None:
        threads = default_threads()
    sweeps = _load().oracle_jacobi_svd(m, n, M.ctypes.data, U.ctypes.data, s.ctypes.data,
                                       V.ctypes.data, int(max_sweeps), int(threads))
    if sweeps == 0:
        raise MemoryError("oracle_jacobi_svd failed")
    return U, s, V, sweeps


# ---- O3 ---------------------------------------------------------------------

def tikhonov(s: np.ndarray, tau_p: float) -> np.ndarray:
    """d_i = s_i / (s_i + tau_p), with d_i = 0 where s_i + tau_p = 0."""
    s = np.asarray(s, np.float64)
    den = s + tau_p
    out = np.zeros_like(s)
    nz = den != 0.0
    out[nz] = s[nz] / den[nz]
    return out


# ---- O4 ---------------------------------------------------------------------

def project(U: np.ndarray, d: np.ndarray, V: np.ndarray, G: np.ndarray) -> np.ndarray:
    """Two-sided projection, spectral filter and reconstruction.

    X = U^T G V;  X_filt = diag(d) X diag(d);  G_filt = U X_filt V^T.
    Matrix products are numpy (BLAS) float64 matmuls.
    """
    U = np.asarray(U, np.float64)
    V = np.asarray(V, np.float64)
    G = np.asarray(G, np.float64)
    d = np.asarray(d, np.float64)
    X = (U.T @ G) @ V
    X_filt = d[:, None] * X * d[None, :]
    return (U @ X_filt) @ V.T


# ---- O5 ---------------------------------------------------------------------

def combine(G_mask: np.ndarray, G_filt: np.ndarray, alpha: float) -> np.ndarray:
    """G_proj = alpha * G_mask + (1 - alpha) * G_filt."""
    return alpha * np.asarray(G_mask, np.float64) + (1.0 - alpha) * np.asarray(G_filt, np.float64)


# ---- O6 ---------------------------------------------------------------------

def adamw(W, m, v, g, t: int, lr: float, beta1: float, beta2: float, eps: float,
          weight_decay: float):
    """One AdamW update with step count t (>= 1, already advanced).

    m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2;
    m_hat = m / (1 - b1^t);  v_hat = v / (1 - b2^t);
    W <- W - lr wd W - lr m_hat / (sqrt(v_hat) + eps)      (W on the right: pre-step)
    """
    W = np.asarray(W, np.float64)
    g = np.asarray(g, np.float64)
    m = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    W_new = W - lr * weight_decay * W - lr * m_hat / (np.sqrt(v_hat) + eps)
    return W_new, m, v


# ---- storage rounding -----------------------------------------------------------

_BF16_MIN_EXP = -133  # quantum of bfloat16 subnormals: 2^-133


def round_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype (RNE), returned as float64.

    'f64' leaves values untouched; 'f32' rounds to float32; 'bf16' rounds once,
    directly from float64, to bfloat16 (8 significant bits).
    """
    x = np.asarray(x, np.float64)
    if dtype == "f64":
        return x.copy()
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        if not np.all(np.isfinite(x)):
            raise ValueError("non-finite value in bf16 storage rounding")
        _, e = np.frexp(x)  # x = f * 2^e, 0.5 <= |f| < 1
        q = np.ldexp(1.0, np.maximum(e - 8, _BF16_MIN_EXP))
        return np.rint(x / q) * q
    raise ValueError(dtype)


# ---- stateful driver ------------------------------------------------------------

class Optimizer:
    """The optimizer over a list of weight matrices, in float64 with storage rounding.

    hp keys: tau_p, alpha, beta_anc, lr, beta1, beta2, eps, weight_decay.
    w_dtype: storage type of W ('f32', 'bf16' or 'f64'); m, v and M_anc are
    stored as state_dtype ('f32' or 'f64').
    """

    def __init__(self, shapes, hp: dict, w_dtype: str = "f32", state_dtype: str = "f32",
                 threads: int | None = None, max_sweeps: int = 100):
        self.shapes = [tuple(int(a) for a in s) for s in shapes]
        self.hp = dict(hp)
        self.w_dtype = w_dtype
        self.state_dtype = state_dtype
        self.threads = threads
        self.max_sweeps = max_sweeps
        self.t = 0
        self.M = [np.zeros(s) for s in self.shapes]
        self.m = [np.zeros(s) for s in self.shapes]
        self.v = [np.zeros(s) for s in self.shapes]
        self.factors = [None] * len(self.shapes)  # (U, s, V) of the current M
        self.d = [None] * len(self.shapes)
        self.sweeps = [0] * len(self.shapes)
        self.last_filt = [None] * len(self.shapes)
        self.last_proj = [None] * len(self.shapes)

    def set_anchor_momentum(self, i: int, M: np.ndarray):
        self.M[i] = round_storage(M, self.state_dtype)
        self.factors[i] = None

    def _refresh(self, i: int):
        U, s, V, sweeps = svd(self.M[i], self.max_sweeps, self.threads)
        self.factors[i] = (U, s, V)
        self.d[i] = tikhonov(s, self.hp["tau_p"])
        self.sweeps[i] = sweeps

    def anchor_update(self, G_anc_list, defer_refresh: bool = False):
        """O1 then O2/O3 for every matrix.  defer_refresh: mark the factors stale
        instead; the next step (or anchor update) recomputes them from the same
        M, so results are identical and an EMA-only chain of anchor arrivals
        costs no SVD."""
        for i, G in enumerate(G_anc_list):
            self.M[i] = round_storage(ema(self.M[i], G, self.hp["beta_anc"]), self.state_dtype)
            if defer_refresh:
                self.factors[i] = None
            else:
                self._refresh(i)

    def set_tau(self, tau_p: float):
        self.hp["tau_p"] = float(tau_p)
        for i, f in enumerate(self.factors):
            if f is not None:
                self.d[i] = tikhonov(f[1], tau_p)

    def step(self, W_list, G_mask_list):
        """O4, O5, O6 for every matrix; returns the new weights (float64 values of
        the stored type).  G_filt / G_proj of the step are kept in last_filt /
        last_proj."""
        hp = self.hp
        self.t += 1
        out = []
        for i, (W, G) in enumerate(zip(W_list, G_mask_list)):
            if self.factors[i] is None:
                self._refresh(i)
            U, s, V = self.factors[i]
            G = np.asarray(G, np.float64)
            G_filt = project(U, self.d[i], V, G)
            G_proj = combine(G, G_filt, hp["alpha"])
            W_new, m_new, v_new = adamw(W, self.m[i], self.v[i], G_proj, self.t, hp["lr"],
                                        hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"])
            self.m[i] = round_storage(m_new, self.state_dtype)
            self.v[i] = round_storage(v_new, self.state_dtype)
            W_new = round_storage(W_new, self.w_dtype)
            self.last_filt[i] = G_filt
            self.last_proj[i] = G_proj
            out.append(W_new)
        return out


from . import masking  # noqa: E402  (O7: the in-graph activation mask, oracle/masking.py)
