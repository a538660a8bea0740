"""GPU parity of the in-graph activation mask ("Key design 1") against the
oracle (oracle/masking.py): kept indices bit-exact, pack and unpack bit-exact,
on small and ragged sizes and at the Llama-3.2-1B boundary size (65536 tokens
= batch 32 x context 2048, H = 2048, mask rate 0.95) on sampled tokens."""
import numpy as np
import pytest
import torch

import oracle.masking as mk
from tests.gpu_harness import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# one-wavefront kernel with 64 / 128 / 256 / 512 candidates per token: (50, 1000, 1),
# (37, 100, 13), (64, 2048, 102), (16, 4096, 205); one workgroup sorting all H:
# (1, 1, 1), (37, 100, 100), (5, 3000, 1500), (8, 2048, 300), (3, 2, 1); more tokens
# than unpack workgroups (9000), so LDS rows are reused, with 16-byte and element stores
@pytest.mark.parametrize("T,H,K", [(1, 1, 1), (37, 100, 0), (37, 100, 100), (37, 100, 13), (64, 2048, 102),
                                   (16, 4096, 205), (5, 3000, 1500), (300, 257, 31), (3, 2, 1),
                                   (50, 1000, 1), (40, 512, 5), (8, 2048, 300), (9000, 64, 3), (9000, 97, 9)])
def test_indices_pack_unpack_exact(T, H, K):
    import spectral_correction_optimizer_amd as sco
    say(f"case: mask T {T} H {H} K {K}")
    layer, step, batch = 5, 1234, 17
    seed = sco.mask_seed(layer, step, batch)
    idx = sco.mask_indices(seed, T, H, K, device="cuda")
    ref = mk.indices(layer, step, batch, T, H, K)
    got = idx.cpu().numpy()
    assert np.array_equal(got, ref)
    x = torch.randn(T, H, device="cuda")
    v = sco.mask_pack(x, idx)
    assert np.array_equal(v.cpu().numpy(), mk.pack(x.cpu().numpy(), ref))
    d = sco.mask_unpack(v, idx, H)
    assert np.array_equal(d.cpu().numpy(), mk.unpack(v.cpu().numpy(), ref, H))
    # bfloat16 payloads move bit for bit
    xb = x.to(torch.bfloat16)
    vb = sco.mask_pack(xb, idx)
    assert torch.equal(vb.view(torch.int16).cpu(), xb.view(torch.int16).cpu()[
        torch.arange(T)[:, None], idx.long().cpu()])
    db = sco.mask_unpack(vb, idx, H)
    ref_b = mk.unpack(vb.view(torch.int16).cpu().numpy(), ref, H)
    assert np.array_equal(db.view(torch.int16).cpu().numpy(), ref_b)


def test_empty_and_backward_reuse():
    """T = 0 queues nothing; with K = 0 unpack writes zeros; the backward of the
    masked map (gradient times m) is unpack(pack(grad)) with the same indices."""
    import spectral_correction_optimizer_amd as sco
    say("case: mask T 0, K 0, backward reuse")
    idx = sco.mask_indices(1, 0, 64, 8, device="cuda")
    assert idx.shape == (0, 8)
    idx0 = sco.mask_indices(1, 4, 64, 0, device="cuda")
    d = sco.mask_unpack(torch.empty(4, 0, device="cuda"), idx0, 64)
    assert torch.count_nonzero(d).item() == 0
    T, H, K = 32, 512, 26
    idx = sco.mask_indices(sco.mask_seed(1, 2, 3), T, H, K, device="cuda")
    x = torch.randn(T, H, device="cuda", dtype=torch.float64).float().requires_grad_(True)
    ti = idx.long()
    y = torch.zeros_like(x).scatter(1, ti, x.gather(1, ti))
    g = torch.randn(T, H, device="cuda")
    y.backward(g)
    back = sco.mask_unpack(sco.mask_pack(g.contiguous(), idx), idx, H)
    assert torch.equal(back, x.grad)


def test_llama_1b_boundary_sampled():
    """65536 tokens x 2048 dims at mask rate 0.95 (K = 102): every token keeps K
    distinct ascending dimensions; 64 sampled tokens (first, last and random)
    equal the oracle's indices, packed values and unpacked rows."""
    import spectral_correction_optimizer_amd as sco
    T, H = 65536, 2048
    K = sco.mask_keep_count(H, 0.95)
    say(f"case: mask 1B boundary T {T} H {H} K {K}")
    layer, step, batch = 7, 100, 3
    idx = sco.mask_indices(sco.mask_seed(layer, step, batch), T, H, K, device="cuda")
    assert idx.shape == (T, K)
    d = torch.diff(idx, dim=1)
    assert bool((d > 0).all()) and int(idx.min()) >= 0 and int(idx.max()) < H
    rows = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(0).integers(0, T, 62)]))
    ref = mk.indices(layer, step, batch, T, H, K, rows=rows)
    assert np.array_equal(idx.cpu().numpy()[rows], ref)
    x = torch.randn(T, H, device="cuda", dtype=torch.bfloat16)
    v = sco.mask_pack(x, idx)
    xr = x.view(torch.int16).cpu().numpy()[rows]
    assert np.array_equal(v.view(torch.int16).cpu().numpy()[rows], mk.pack(xr, ref))
    u = sco.mask_unpack(v, idx, H)
    assert np.array_equal(u.view(torch.int16).cpu().numpy()[rows],
                          mk.unpack(mk.pack(xr, ref), ref, H))
