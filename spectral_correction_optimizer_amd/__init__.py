"""Spectral-correction AdamW on AMD MI355X: Python binding of libscopt.

Argument marshalling only: every step of the optimizer runs in the HIP
kernels of ``libscopt.so`` (C ABI in ``include/scopt.h``).  PyTorch supplies
device memory and the current HIP stream.  There is no CPU fallback: if the
library has not been built, importing the binding works but constructing an
optimizer raises ``ScoptError``.

The method (papernotes.org notes on "Communication-Efficient LLM Adaptation
over Decentralized GPU Meshes", "Key design 2" and "Key design 3"): per weight
matrix, an anchor-momentum EMA, a thin SVD of it, the Tikhonov response
d_i = s_i / (s_i + tau_p), the two-sided projection and reconstruction
G_filt = U diag(d) (U^T G V) diag(d) V^T, the combination
G_proj = alpha G + (1 - alpha) G_filt, then AdamW.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first: libscopt then binds to torch's HIP runtime

__all__ = ["SpectralAdamW", "ScoptError", "library_path", "load_library", "EXPORTED_SYMBOLS",
           "mask_keep_count", "mask_seed", "mask_indices", "mask_pack", "mask_unpack"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libscopt.so")
_lib = None

EXPORTED_SYMBOLS = (
    "sc_default_hparams", "sc_opt_create", "sc_opt_destroy", "sc_anchor_update", "sc_refresh",
    "sc_anchor_update_async", "sc_refresh_wait", "sc_refresh_pending", "sc_step", "sc_step_noalloc", "sc_set_lr", "sc_set_tau", "sc_set_state", "sc_get_state", "sc_set_step",
    "sc_get_step", "sc_set_factors", "sc_get_factors", "sc_keep_proj", "sc_get_filtered",
    "sc_set_solve_waves", "sc_set_fused_gram", "sc_set_v_rounds", "sc_set_sweep_stop", "sc_set_quad",
    "sc_get_stats", "sc_get_sweep_counts", "sc_profile", "sc_get_kernel_times", "sc_last_error",
    "sc_mask_keep_count", "sc_mask_seed", "sc_mask_indices", "sc_mask_pack", "sc_mask_unpack",
)

SC_F32, SC_BF16 = 0, 1
STATE_KINDS = {"m_anc": 0, "adam_m": 1, "adam_v": 2}


class ScoptError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libscopt error {code}: {msg}")
        self.code = code


class HParams(ctypes.Structure):
    _fields_ = [("tau_p", ctypes.c_float), ("alpha", ctypes.c_float), ("beta_anc", ctypes.c_float),
                ("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("max_sweeps", ctypes.c_int), ("jacobi_tol", ctypes.c_float),
                ("sync_check", ctypes.c_int), ("warm_start", ctypes.c_int),
                ("precondition", ctypes.c_int)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double), ("flops", ctypes.c_double),
                ("bytes", ctypes.c_double)]


class Stats(ctypes.Structure):
    _fields_ = [("n_mats", ctypes.c_int), ("step", ctypes.c_int64), ("refreshes", ctypes.c_int),
                ("sweeps_max", ctypes.c_int), ("not_converged", ctypes.c_int),
                ("nonfinite_grad", ctypes.c_int), ("nonfinite_anchor", ctypes.c_int),
                ("factor_sweeps_max", ctypes.c_int), ("factor_rejected", ctypes.c_int)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libscopt.so (raises ScoptError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ScoptError(-100, f"{_LIB_PATH} is missing; build it with __graft_entry__.build()")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)
    sig = {
        "sc_default_hparams": (None, [ctypes.POINTER(HParams)]),
        "sc_opt_create": (ctypes.c_int, [ctypes.POINTER(vp), ctypes.c_int, i64p, i64p, ctypes.c_int,
                                         ctypes.c_int, ctypes.POINTER(HParams), ctypes.c_int]),
        "sc_opt_destroy": (ctypes.c_int, [vp]),
        "sc_anchor_update": (ctypes.c_int, [vp, ctypes.POINTER(vp), vp]),
        "sc_refresh": (ctypes.c_int, [vp, vp]),
        "sc_anchor_update_async": (ctypes.c_int, [vp, ctypes.POINTER(vp), vp]),
        "sc_refresh_wait": (ctypes.c_int, [vp, vp]),
        "sc_refresh_pending": (ctypes.c_int, [vp, ctypes.POINTER(ctypes.c_int)]),
        "sc_step": (ctypes.c_int, [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp]),
        "sc_step_noalloc": (ctypes.c_int, [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp]),
        "sc_set_lr": (ctypes.c_int, [vp, ctypes.c_float]),
        "sc_set_tau": (ctypes.c_int, [vp, ctypes.c_float]),
        "sc_set_state": (ctypes.c_int, [vp, ctypes.c_int, ctypes.c_int, vp, vp]),
        "sc_get_state": (ctypes.c_int, [vp, ctypes.c_int, ctypes.c_int, vp, vp]),
        "sc_set_step": (ctypes.c_int, [vp, ctypes.c_int64]),
        "sc_get_step": (ctypes.c_int, [vp, i64p]),
        "sc_set_factors": (ctypes.c_int, [vp, ctypes.c_int, vp, vp, vp, vp]),
        "sc_get_factors": (ctypes.c_int, [vp, ctypes.c_int, vp, vp, vp, vp]),
        "sc_keep_proj": (ctypes.c_int, [vp, ctypes.c_int]),
        "sc_set_solve_waves": (ctypes.c_int, [vp, ctypes.c_int, ctypes.c_int]),
        "sc_set_fused_gram": (ctypes.c_int, [vp, ctypes.c_int]),
        "sc_set_v_rounds": (ctypes.c_int, [vp, ctypes.c_int]),
        "sc_set_sweep_stop": (ctypes.c_int, [vp, ctypes.c_float]),
        "sc_set_quad": (ctypes.c_int, [vp, ctypes.c_int]),
        "sc_get_filtered": (ctypes.c_int, [vp, ctypes.c_int, vp, vp, vp]),
        "sc_get_stats": (ctypes.c_int, [vp, ctypes.POINTER(Stats), ctypes.POINTER(ctypes.c_int)]),
        "sc_get_sweep_counts": (ctypes.c_int, [vp, ctypes.POINTER(ctypes.c_int),
                                               ctypes.POINTER(ctypes.c_int)]),
        "sc_profile": (ctypes.c_int, [vp, ctypes.c_int]),
        "sc_get_kernel_times": (ctypes.c_int, [vp, ctypes.POINTER(KernelTime), ctypes.c_int,
                                               ctypes.POINTER(ctypes.c_int)]),
        "sc_last_error": (ctypes.c_char_p, []),
        "sc_mask_keep_count": (ctypes.c_int, [ctypes.c_int, ctypes.c_float, ctypes.POINTER(ctypes.c_int)]),
        "sc_mask_seed": (ctypes.c_int, [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                        ctypes.POINTER(ctypes.c_uint64)]),
        "sc_mask_indices": (ctypes.c_int, [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                           vp, vp]),
        "sc_mask_pack": (ctypes.c_int, [ctypes.c_int, vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                        vp, vp]),
        "sc_mask_unpack": (ctypes.c_int, [ctypes.c_int, vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                          vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise ScoptError(rc, load_library().sc_last_error().decode())


def default_hparams() -> dict:
    hp = HParams()
    load_library().sc_default_hparams(ctypes.byref(hp))
    return {name: getattr(hp, name) for name, _ in HParams._fields_}


_DT = {torch.float32: SC_F32, torch.bfloat16: SC_BF16}


class SpectralAdamW:
    """Spectral-correction AdamW over a fixed list of weight-matrix shapes.

    shapes: [(rows, cols), ...] of the row-major weights ([out, in]).
    w_dtype: torch.float32 or torch.bfloat16 (storage of W); g_dtype: type of
    G_mask and G_anc.  Keyword hyper-parameters: tau_p, alpha, beta_anc, lr,
    beta1, beta2, eps, weight_decay, max_sweeps, jacobi_tol, sync_check,
    warm_start, precondition.
    """

    def __init__(self, shapes, w_dtype=torch.float32, g_dtype=torch.float32, device=None, **hp):
        lib = load_library()
        self.shapes = [(int(r), int(c)) for r, c in shapes]
        self.n = len(self.shapes)
        if w_dtype not in _DT or g_dtype not in _DT:
            raise ValueError("dtypes must be torch.float32 or torch.bfloat16")
        self.w_dtype, self.g_dtype = w_dtype, g_dtype
        self.device = torch.device(device if device is not None else "cuda")
        if self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        h = HParams()
        lib.sc_default_hparams(ctypes.byref(h))
        for k, v in hp.items():
            if not hasattr(h, k):
                raise TypeError(f"unknown hyper-parameter {k}")
            setattr(h, k, v)
        self.hp = {name: getattr(h, name) for name, _ in HParams._fields_}
        rows = (ctypes.c_int64 * self.n)(*[r for r, _ in self.shapes])
        cols = (ctypes.c_int64 * self.n)(*[c for _, c in self.shapes])
        handle = ctypes.c_void_p()
        _check(lib.sc_opt_create(ctypes.byref(handle), self.n, rows, cols, _DT[w_dtype],
                                 _DT[g_dtype], ctypes.byref(h), self.device.index))
        self._h = handle
        self._lib = lib

    # -- helpers -------------------------------------------------------------------------
    def _stream(self):
        return ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)

    def _ptrs(self, tensors, dtype, what):
        if len(tensors) != self.n:
            raise ValueError(f"{what}: expected {self.n} tensors, got {len(tensors)}")
        arr = (ctypes.c_void_p * self.n)()
        for i, (t, shp) in enumerate(zip(tensors, self.shapes)):
            if t.device != self.device or t.dtype != dtype or tuple(t.shape) != shp or \
                    not t.is_contiguous():
                raise ValueError(f"{what}[{i}] must be a contiguous {dtype} tensor of shape {shp} "
                                 f"on {self.device}, got {t.dtype} {tuple(t.shape)} on {t.device}")
            arr[i] = t.data_ptr()
        return arr

    def _f32(self, idx, t, shape, what):
        if t.device != self.device or t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) \
                or not t.is_contiguous():
            raise ValueError(f"{what} must be a contiguous float32 tensor of shape {tuple(shape)}")
        return ctypes.c_void_p(t.data_ptr())

    # -- the method ----------------------------------------------------------------------
    def anchor_update(self, G_anc):
        """EMA of the anchor momentum with G_anc, then SVD refresh."""
        _check(self._lib.sc_anchor_update(self._h, self._ptrs(G_anc, self.g_dtype, "G_anc"),
                                          self._stream()))

    def refresh(self):
        _check(self._lib.sc_refresh(self._h, self._stream()))

    def anchor_update_async(self, G_anc):
        """EMA with G_anc and SVD refresh beside the following steps, which use the
        previous factors until refresh_wait().  G_anc must stay valid and
        unchanged until then."""
        _check(self._lib.sc_anchor_update_async(self._h, self._ptrs(G_anc, self.g_dtype, "G_anc"),
                                                self._stream()))

    def refresh_wait(self):
        """Complete a pending asynchronous refresh: the current stream waits for it
        and later steps use its factors."""
        _check(self._lib.sc_refresh_wait(self._h, self._stream()))

    def refresh_pending(self) -> bool:
        p = ctypes.c_int()
        _check(self._lib.sc_refresh_pending(self._h, ctypes.byref(p)))
        return bool(p.value)

    def step(self, W, G_mask):
        """One spectral-corrected AdamW step; W is updated in place."""
        _check(self._lib.sc_step(self._h, self._ptrs(W, self.w_dtype, "W"),
                                 self._ptrs(G_mask, self.g_dtype, "G_mask"), self._stream()))

    def step_noalloc(self, W, G_mask):
        """The same step through the allocation-free entry point (intermediates in
        the library's per-GPU scratch array)."""
        _check(self._lib.sc_step_noalloc(self._h, self._ptrs(W, self.w_dtype, "W"),
                                         self._ptrs(G_mask, self.g_dtype, "G_mask"), self._stream()))

    def set_lr(self, lr: float):
        _check(self._lib.sc_set_lr(self._h, float(lr)))

    def set_tau(self, tau_p: float):
        _check(self._lib.sc_set_tau(self._h, float(tau_p)))

    def set_state(self, idx: int, kind: str, src: torch.Tensor):
        _check(self._lib.sc_set_state(self._h, idx, STATE_KINDS[kind],
                                      self._f32(idx, src, self.shapes[idx], kind), self._stream()))

    def get_state(self, idx: int, kind: str) -> torch.Tensor:
        out = torch.empty(self.shapes[idx], dtype=torch.float32, device=self.device)
        _check(self._lib.sc_get_state(self._h, idx, STATE_KINDS[kind],
                                      ctypes.c_void_p(out.data_ptr()), self._stream()))
        return out

    @property
    def step_count(self) -> int:
        t = ctypes.c_int64()
        _check(self._lib.sc_get_step(self._h, ctypes.byref(t)))
        return t.value

    @step_count.setter
    def step_count(self, t: int):
        _check(self._lib.sc_set_step(self._h, int(t)))

    def set_factors(self, idx: int, U: torch.Tensor, s: torch.Tensor, V: torch.Tensor):
        m, n = self.shapes[idx]
        r = min(m, n)
        _check(self._lib.sc_set_factors(self._h, idx, self._f32(idx, U, (m, r), "U"),
                                        self._f32(idx, s, (r,), "s"), self._f32(idx, V, (n, r), "V"),
                                        self._stream()))

    def get_factors(self, idx: int):
        m, n = self.shapes[idx]
        r = min(m, n)
        U = torch.empty((m, r), dtype=torch.float32, device=self.device)
        s = torch.empty((r,), dtype=torch.float32, device=self.device)
        V = torch.empty((n, r), dtype=torch.float32, device=self.device)
        _check(self._lib.sc_get_factors(self._h, idx, ctypes.c_void_p(U.data_ptr()),
                                        ctypes.c_void_p(s.data_ptr()), ctypes.c_void_p(V.data_ptr()),
                                        self._stream()))
        return U, s, V

    def set_solve_waves(self, waves: int = 0, copies: int = 0):
        """Jacobi pair-solve variant: `waves` (1, 2, 4, 8) wavefronts per pair and
        `copies` (1, 2) LDS copies of its Gram; 0 picks by each launch's pair
        count.  All variants give identical results."""
        _check(self._lib.sc_set_solve_waves(self._h, int(waves), int(copies)))

    def set_fused_gram(self, enable: bool = True):
        """Fused rotation apply + next-round pair Gram (default on)."""
        _check(self._lib.sc_set_fused_gram(self._h, 1 if enable else 0))

    def set_v_rounds(self, rounds: int = 2):
        """V-row rotations of the fused sweeps: 2 rounds per pass (default) or 1;
        bit-identical results."""
        _check(self._lib.sc_set_v_rounds(self._h, int(rounds)))

    def set_sweep_stop(self, stop: float = 1e-4):
        """Sweep-stop rule of the Jacobi sweeps (0 = off); a certificate checks
        the result."""
        _check(self._lib.sc_set_sweep_stop(self._h, float(stop)))

    def set_quad(self, mode: int = 1):
        """Quad passes of the Jacobi sweeps (three pair rounds per pass over groups
        of four column blocks): 0 off, 1 (default) where a list's block counts
        allow and its groups fill the GPU, 2 wherever the block counts allow."""
        _check(self._lib.sc_set_quad(self._h, int(mode)))

    def keep_proj(self, enable: bool = True):
        _check(self._lib.sc_keep_proj(self._h, 1 if enable else 0))

    def get_filtered(self, idx: int, proj: bool = False):
        shp = self.shapes[idx]
        gf = torch.empty(shp, dtype=torch.float32, device=self.device)
        gp = torch.empty(shp, dtype=torch.float32, device=self.device) if proj else None
        _check(self._lib.sc_get_filtered(self._h, idx, ctypes.c_void_p(gf.data_ptr()),
                                         ctypes.c_void_p(gp.data_ptr() if gp is not None else None),
                                         self._stream()))
        return (gf, gp) if proj else gf

    def stats(self):
        st = Stats()
        per = (ctypes.c_int * self.n)()
        _check(self._lib.sc_get_stats(self._h, ctypes.byref(st), per))
        d = {name: getattr(st, name) for name, _ in Stats._fields_}
        d["sweeps"] = list(per)
        fac = (ctypes.c_int * self.n)()
        _check(self._lib.sc_get_sweep_counts(self._h, None, fac))
        d["factor_sweeps"] = list(fac)
        return d

    def profile(self, enable: bool = True, serial: bool = False):
        """Enable / disable per-kernel event timing (resets the totals).  serial:
        every kernel alone on the current stream (slower pass); otherwise the
        production schedule, each launch timed on its own stream."""
        _check(self._lib.sc_profile(self._h, (2 if serial else 1) if enable else 0))

    def kernel_times(self):
        """{family: dict(launches, total_ms, flops, bytes)} accumulated since profile(True)."""
        arr = (KernelTime * 64)()
        cnt = ctypes.c_int()
        _check(self._lib.sc_get_kernel_times(self._h, arr, 64, ctypes.byref(cnt)))
        out = {}
        for i in range(min(cnt.value, 64)):
            k = arr[i]
            out[k.name.decode()] = dict(launches=k.launches, total_ms=k.total_ms, flops=k.flops,
                                        bytes=k.bytes)
        return out

    def close(self):
        if getattr(self, "_h", None):
            self._lib.sc_opt_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---- in-graph activation mask ("Key design 1"): stateless calls --------------------

def mask_keep_count(H: int, p: float) -> int:
    """Kept dimensions per token at mask rate p: floor((1 - p) H + 1/2)."""
    k = ctypes.c_int()
    _check(load_library().sc_mask_keep_count(int(H), float(p), ctypes.byref(k)))
    return k.value


def mask_seed(layer: int, step: int, batch: int) -> int:
    """The mask seed of (layer, step, batch)."""
    s = ctypes.c_uint64()
    _check(load_library().sc_mask_seed(int(layer), int(step), int(batch), ctypes.byref(s)))
    return s.value


def _cur_stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def mask_indices(seed: int, T: int, H: int, K: int, device=None) -> "torch.Tensor":
    """Kept dimensions of each of T tokens: int32 [T, K] on the device, ascending."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    _check(load_library().sc_mask_indices(int(seed), int(T), int(H), int(K),
                                          ctypes.c_void_p(idx.data_ptr()), _cur_stream(dev)))
    return idx


def _mask_dt(t):
    if t.dtype == torch.float32:
        return SC_F32
    if t.dtype == torch.bfloat16:
        return SC_BF16
    raise ValueError(f"mask tensors must be float32 or bfloat16, got {t.dtype}")


def mask_pack(x: "torch.Tensor", idx: "torch.Tensor") -> "torch.Tensor":
    """Kept values of each token (x: [T, H] contiguous; idx: int32 [T, K])."""
    T, H = x.shape
    K = idx.shape[1]
    if not (x.is_contiguous() and idx.is_contiguous() and idx.dtype == torch.int32 and idx.shape[0] == T
            and idx.device == x.device):
        raise ValueError("mask_pack: contiguous x [T, H] and int32 idx [T, K] on one device")
    out = torch.empty((T, K), dtype=x.dtype, device=x.device)
    _check(load_library().sc_mask_pack(_mask_dt(x), ctypes.c_void_p(x.data_ptr()),
                                       ctypes.c_void_p(idx.data_ptr()), T, H, K,
                                       ctypes.c_void_p(out.data_ptr()), _cur_stream(x.device)))
    return out


def mask_unpack(packed: "torch.Tensor", idx: "torch.Tensor", H: int) -> "torch.Tensor":
    """Dense [T, H] rows with the packed values at idx and zeros elsewhere."""
    T, K = packed.shape
    if not (packed.is_contiguous() and idx.is_contiguous() and idx.dtype == torch.int32
            and tuple(idx.shape) == (T, K) and idx.device == packed.device):
        raise ValueError("mask_unpack: contiguous packed [T, K] and int32 idx [T, K] on one device")
    out = torch.empty((T, H), dtype=packed.dtype, device=packed.device)
    _check(load_library().sc_mask_unpack(_mask_dt(packed), ctypes.c_void_p(packed.data_ptr()),
                                         ctypes.c_void_p(idx.data_ptr()), T, int(H), K,
                                         ctypes.c_void_p(out.data_ptr()), _cur_stream(packed.device)))
    return out
