"""The C-ABI library without a GPU: it loads, exports every symbol that
include/scopt.h declares, and rejects invalid arguments synchronously with
the documented error codes (validation happens before any GPU work)."""
import ctypes
import os
import re

import pytest

import spectral_correction_optimizer_amd as sco

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "scopt.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sc_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sco.library_path()):
        pytest.skip("libscopt.so not built")
    return sco.load_library()


def test_header_matches_binding():
    assert declared_functions() == sorted(sco.EXPORTED_SYMBOLS)


def test_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_defaults(lib):
    hp = sco.default_hparams()
    assert abs(hp["tau_p"] - 1e-3) < 1e-9 and abs(hp["alpha"] - 0.3) < 1e-7
    assert abs(hp["beta_anc"] - 0.9) < 1e-7 and abs(hp["lr"] - 2e-5) < 1e-12
    assert hp["max_sweeps"] >= 1 and hp["sync_check"] == 1


def _create(lib, n, rows, cols, hp=None, wdt=0, gdt=0, device=0):
    h = ctypes.c_void_p()
    if hp is None:
        hp = sco.HParams()
        lib.sc_default_hparams(ctypes.byref(hp))
    r = (ctypes.c_int64 * max(n, 1))(*rows)
    c = (ctypes.c_int64 * max(n, 1))(*cols)
    rc = lib.sc_opt_create(ctypes.byref(h), n, r, c, wdt, gdt, ctypes.byref(hp), device)
    return rc, h


def test_invalid_arguments(lib):
    assert _create(lib, 0, [1], [1])[0] == -1
    assert _create(lib, 129, [4] * 129, [4] * 129)[0] == -1
    assert _create(lib, 1, [0], [5])[0] == -2
    assert _create(lib, 1, [5], [70000])[0] == -2
    assert _create(lib, 1, [5], [5], wdt=7)[0] == -1
    for field, bad in [("alpha", 1.5), ("tau_p", -1.0), ("eps", 0.0), ("beta1", 1.0),
                       ("max_sweeps", 0), ("beta_anc", -0.1), ("jacobi_tol", 2.0)]:
        hp = sco.HParams()
        lib.sc_default_hparams(ctypes.byref(hp))
        setattr(hp, field, bad)
        rc, _ = _create(lib, 1, [8], [8], hp=hp)
        assert rc == -1, field
        assert lib.sc_last_error().decode()
    h = ctypes.c_void_p()
    assert lib.sc_opt_create(None, 1, None, None, 0, 0, None, 0) == -1
    # calls on a NULL handle
    assert lib.sc_step(None, None, None, None) == -1
    assert lib.sc_anchor_update(None, None, None) == -1
    assert lib.sc_set_lr(None, 1.0) == -1
    assert lib.sc_get_stats(None, None, None) == -1
    assert lib.sc_anchor_update_async(None, None, None) == -1
    assert lib.sc_refresh_wait(None, None) == -1
    assert lib.sc_refresh_pending(None, None) == -1
    assert lib.sc_set_solve_waves(None, 0, 0) == -1
    assert lib.sc_set_fused_gram(None, 1) == -1
    assert lib.sc_set_v_rounds(None, 2) == -1
    assert lib.sc_set_sweep_stop(None, ctypes.c_float(1e-4)) == -1
    assert lib.sc_set_quad(None, 1) == -1
    assert lib.sc_opt_destroy(None) == 0
    # the stateless mask calls validate before any GPU work
    k = ctypes.c_int()
    assert lib.sc_mask_keep_count(2048, 0.95, ctypes.byref(k)) == 0 and k.value == 102
    assert lib.sc_mask_keep_count(0, 0.5, ctypes.byref(k)) == -1
    assert lib.sc_mask_keep_count(8, 1.5, ctypes.byref(k)) == -1
    assert lib.sc_mask_indices(0, 4, 4097, 1, None, None) == -1
    assert lib.sc_mask_indices(0, 4, 64, 65, None, None) == -1
    assert lib.sc_mask_indices(0, -1, 64, 8, None, None) == -1
    assert lib.sc_mask_indices(0, 4, 64, 8, None, None) == -1      # NULL idx
    assert lib.sc_mask_pack(7, None, None, 4, 64, 8, None, None) == -1
    assert lib.sc_mask_unpack(0, None, None, 4, 64, 8, None, None) == -1
    assert lib.sc_mask_indices(0, 0, 64, 8, None, None) == 0       # T = 0: nothing to do


def test_no_device_is_reported(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc, _ = _create(lib, 1, [8], [8])
    assert rc == -5
    assert "device" in lib.sc_last_error().decode()


def test_mask_seed_and_count_match_oracle(lib):
    """The library's host-side mask seed and keep count equal the oracle's."""
    import oracle.masking as mk
    for layer, step, batch in [(0, 0, 0), (3, 10, 7), (2 ** 40, 5, 2 ** 63), (2 ** 64 - 2, 1, 2)]:
        assert sco.mask_seed(layer, step, batch) == mk.seed_of(layer, step, batch)
    for H, p in [(2048, 0.95), (4096, 0.95), (10, 0.25), (8, 0.0), (8, 1.0), (1000, 0.9)]:
        assert sco.mask_keep_count(H, p) == mk.keep_count(H, p)
