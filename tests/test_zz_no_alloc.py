"""The allocation-free step entry point (sc_step_noalloc) against sc_step.

Two handles with identical state take the same steps, one through sc_step and
one through sc_step_noalloc (step intermediates in the library's per-GPU
scratch array); G_filt, G_proj and W must agree to the parity bar (1e-4
relative Frobenius on G_filt / G_proj, 1e-7 on float32 W).  Two calls in a
row, the second on a handle of smaller matrices, so that a second call that
reads stale scratch contents of the first would show.
"""
import numpy as np
import pytest
import torch

import gen
from tests.gpu_harness import relf, say, to_dev, from_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pair(shapes, cfg):
    import spectral_correction_optimizer_amd as sco
    dev = torch.device("cuda")
    ins = [gen.MatrixInputs(cfg, 0, i, *sh) for i, sh in enumerate(shapes)]
    opts, Ws = [], []
    for _ in range(2):
        opt = sco.SpectralAdamW(shapes, device=dev)
        opt.keep_proj(True)
        for i, mi in enumerate(ins):
            opt.set_state(i, "m_anc", to_dev(gen.stored(mi.m0(), "f32")[0], "f32", dev))
        opt.anchor_update([to_dev(gen.stored(mi.g_anc(0), "f32")[0], "f32", dev) for mi in ins])
        opts.append(opt)
        Ws.append([to_dev(gen.stored(mi.w0(), "f32")[0], "f32", dev) for mi in ins])
    return ins, opts, Ws


def _compare(shapes, ins, opts, Ws, k):
    dev = torch.device("cuda")
    G = [to_dev(gen.stored(mi.g_mask(k), "f32")[0], "f32", dev) for mi in ins]
    opts[0].step(Ws[0], G)
    opts[1].step_noalloc(Ws[1], G)
    torch.cuda.synchronize()
    worst = [0.0, 0.0, 0.0]
    bitwise = True
    for i in range(len(shapes)):
        fa, pa = (from_dev(x) for x in opts[0].get_filtered(i, proj=True))
        fb, pb = (from_dev(x) for x in opts[1].get_filtered(i, proj=True))
        wa, wb = from_dev(Ws[0][i]), from_dev(Ws[1][i])
        worst[0] = max(worst[0], relf(fb, fa))
        worst[1] = max(worst[1], relf(pb, pa))
        worst[2] = max(worst[2], float(np.abs(wb - wa).max()))
        bitwise = bitwise and np.array_equal(fa, fb) and np.array_equal(wa, wb)
    say(f"  step {k}: relF G_filt {worst[0]:.2e} G_proj {worst[1]:.2e} max|dW| {worst[2]:.2e} "
        f"bitwise {bitwise}")
    assert worst[0] <= 1e-4 and worst[1] <= 1e-4 and worst[2] <= 1e-7


def test_noalloc_step_matches_step_two_calls_second_smaller():
    big = [(1024, 1024), (256, 1024), (2048, 512), (512, 2048), (300, 200)]
    small = [(96, 64), (64, 160), (40, 40)]
    for shapes, cfg in ((big, 140), (small, 141)):
        say(f"case: sc_step_noalloc vs sc_step on {shapes}")
        ins, opts, Ws = _pair(shapes, cfg)
        for k in range(2):
            _compare(shapes, ins, opts, Ws, k)
        for o in opts:
            o.close()


def test_noalloc_step_rejects_oversized_matrix():
    """A matrix whose intermediates exceed the 128 MiB array (8400 x 4200: two
    4200 x 4200 float32 intermediates, 141 MB): a clear error before any GPU
    work, and the handle's ordinary step still works."""
    import spectral_correction_optimizer_amd as sco
    dev = torch.device("cuda")
    shapes = [(8400, 4200)]
    opt = sco.SpectralAdamW(shapes, device=dev)
    W = [torch.zeros(shapes[0], device=dev)]
    G = [torch.zeros(shapes[0], device=dev)]
    with pytest.raises(sco.ScoptError) as e:
        opt.step_noalloc(W, G)
    say(f"  rejected: {e.value}")
    assert e.value.code == -2 and "scratch" in str(e.value)
    opt.step(W, G)
    torch.cuda.synchronize()
    opt.close()
