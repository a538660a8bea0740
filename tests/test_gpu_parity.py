"""GPU parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Seeded synthetic inputs of the workloads' shapes and distributions (gen).
Sizes are chosen so the oracle finishes in seconds while spanning several
GEMM tiles, several Jacobi block pairs and ragged tails.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from tests.gpu_harness import Scenario, relf, say, to_dev, from_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import spectral_correction_optimizer_amd as sco
    sco.load_library()


def test_single_64x48_five_steps():
    """The small single-matrix workload: 64x48 fp32, 1 anchor update, 5 steps.
    W is gated on every element."""
    say("case: 64x48, 1 refresh + 5 steps")
    sc = Scenario([(64, 48)], [(1, 0, 0)], steps=5)
    rep = sc.run()
    Scenario.check(rep)
    assert max(e for _, _, c, e in rep["excluded"]) <= 1e-7


@pytest.mark.parametrize("shape", [(200, 136), (136, 200), (130, 130), (520, 96), (96, 520),
                                   (300, 64), (33, 70), (257, 1), (1, 45)])
def test_ragged_shapes(shape):
    say(f"case: ragged {shape}, 1 refresh + 3 steps")
    sc = Scenario([shape], [(90, 0, 0)], steps=3)
    Scenario.check(sc.run())


def test_group_of_mixed_shapes_two_refreshes():
    """Several matrices of all three shape classes in one handle; the anchor
    arrives every 2 steps."""
    shapes = [(256, 256), (96, 256), (512, 128), (128, 512), (72, 40)]
    say(f"case: group {shapes}, refresh every 2 steps, 5 steps")
    sc = Scenario(shapes, [(91, 0, i) for i in range(len(shapes))], steps=5, anchor_every=2)
    Scenario.check(sc.run())


@pytest.mark.parametrize("tau", [1e-4, 1e-2, 0.0])
def test_tau_values(tau):
    say(f"case: tau {tau}, 192x160")
    sc = Scenario([(192, 160)], [(92, 0, 0)], hp=dict(tau_p=tau), steps=2)
    Scenario.check(sc.run())


def test_alpha_one_is_plain_adamw():
    """alpha = 1: G_proj = G_mask ("pure mask" ablation), the step is AdamW on G_mask."""
    say("case: alpha 1")
    sc = Scenario([(160, 96)], [(93, 0, 0)], hp=dict(alpha=1.0), steps=3)
    Scenario.check(sc.run())


def test_alpha_zero_pure_filtered():
    say("case: alpha 0")
    sc = Scenario([(160, 96)], [(94, 0, 0)], hp=dict(alpha=0.0), steps=2)
    Scenario.check(sc.run())


def test_bf16_weights_and_gradients():
    """bfloat16 W, G_mask and G_anc (float32 states): W within one bf16 ulp."""
    say("case: bf16 W/G, 256x192 and 128x320")
    sc = Scenario([(256, 192), (128, 320)], [(95, 0, 0), (95, 0, 1)], steps=3, w_dtype="bf16",
                  g_dtype="bf16")
    rep = sc.run()
    Scenario.check(rep, w_dtype="bf16")


def test_no_anchor_yet_gives_alpha_g():
    """Before any anchor arrives M_anc = 0, so d = 0, G_filt = 0 and G_proj = alpha G."""
    import spectral_correction_optimizer_amd as sco
    say("case: no anchor")
    dev = torch.device("cuda")
    opt = sco.SpectralAdamW([(96, 64)], device=dev)
    opt.keep_proj(True)
    g = torch.randn(96, 64, device=dev) * 1e-3
    w = torch.randn(96, 64, device=dev) * 0.02
    opt.step([w], [g])
    gf, gp = opt.get_filtered(0, proj=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(gf).item() == 0
    assert torch.allclose(gp, 0.3 * g, rtol=1e-6, atol=0)
    opt.close()


def test_injected_oracle_factors_isolate_projection():
    """Install the oracle's (fp32-rounded) factors, then compare G_filt: this
    isolates the projection / reconstruction GEMM chain from the SVD."""
    import spectral_correction_optimizer_amd as sco
    dev = torch.device("cuda")
    for (m, n) in [(384, 256), (256, 384), (320, 320)]:
        say(f"case: injected factors {m}x{n}")
        mi = gen.MatrixInputs(96, 0, 0, m, n)
        M = gen.stored(mi.m0(), "f32")[1]
        U, s, V, _ = oracle.svd(M)
        U32, s32, V32 = (x.astype(np.float32) for x in (U, s, V))
        G = gen.stored(mi.g_mask(0), "f32")[0]
        opt = sco.SpectralAdamW([(m, n)], device=dev)
        opt.set_factors(0, *(torch.from_numpy(x).to(dev) for x in (U32, s32, V32)))
        w = torch.zeros(m, n, device=dev)
        opt.step([w], [torch.from_numpy(G).to(dev)])
        gf = from_dev(opt.get_filtered(0))
        ref = oracle.project(U32.astype(np.float64), oracle.tikhonov(s32.astype(np.float64), 1e-3),
                             V32.astype(np.float64), G.astype(np.float64))
        err = relf(gf, ref)
        say(f"  relF {err:.3e}")
        assert err < 1e-5
        # exported factors round-trip
        U2, s2, V2 = (x.cpu().numpy() for x in opt.get_factors(0))
        assert np.array_equal(s2, s32) and np.array_equal(U2, U32) and np.array_equal(V2, V32)
        opt.close()


def test_svd_self_consistency():
    """GPU factors reconstruct M and are orthonormal to float32 accuracy."""
    import spectral_correction_optimizer_amd as sco
    dev = torch.device("cuda")
    for (m, n) in [(320, 192), (192, 320), (256, 256), (640, 160), (160, 640)]:
        say(f"case: svd self-check {m}x{n}")
        mi = gen.MatrixInputs(97, 0, 0, m, n)
        pay, M = gen.stored(mi.m0(), "f32")
        opt = sco.SpectralAdamW([(m, n)], device=dev)
        opt.set_state(0, "m_anc", torch.from_numpy(pay).to(dev))
        opt.refresh()
        U, s, V = (x.double().cpu().numpy() for x in opt.get_factors(0))
        r = min(m, n)
        rec = np.linalg.norm((U * s) @ V.T - M) / np.linalg.norm(M)
        ou = np.linalg.norm(U.T @ U - np.eye(r)) / np.sqrt(r)
        ov = np.linalg.norm(V.T @ V - np.eye(r)) / np.sqrt(r)
        s_ref = np.linalg.svd(M, compute_uv=False)
        se = np.abs(np.sort(s)[::-1] - s_ref).max() / s_ref[0]
        say(f"  recon {rec:.2e} orthU {ou:.2e} orthV {ov:.2e} s err {se:.2e} stats {opt.stats()}")
        assert rec < 1e-5 and ou < 1e-5 and ov < 1e-5 and se < 1e-5
        opt.close()


@pytest.mark.parametrize("precondition", [1, 0])
def test_cholesky_preconditioned_shapes(precondition):
    """Operands at least twice as long as wide run their first sweeps on the
    Cholesky factor of the Gram, then polish on A = M V; both settings meet the
    gates, and the factor phase really ran (or did not)."""
    shapes = [(520, 96), (96, 520), (1024, 256), (256, 640), (200, 136)]
    say(f"case: precondition={precondition} {shapes}, refresh every 2 steps, 4 steps")
    sc = Scenario(shapes, [(93, 0, i) for i in range(len(shapes))], steps=4, anchor_every=2)
    rep = sc.run(gpu_hp=dict(precondition=precondition))
    Scenario.check(rep)
    st = rep["stats"]
    say(f"  stats {st}")
    assert st["factor_rejected"] == 0
    assert (st["factor_sweeps_max"] > 0) == bool(precondition)


def test_cholesky_rejected_for_rank_deficient_operand():
    """Warm start from a full-rank anchor's factors, then a rank-8 anchor: the
    operand A = M V_prev has linearly dependent columns, the Gram factorization
    is rejected and the matrix runs the plain sweeps; factors and G_filt still
    agree with the oracle."""
    import spectral_correction_optimizer_amd as sco
    dev = torch.device("cuda")
    shapes = [(384, 96), (96, 384)]
    say(f"case: rank-8 anchors {shapes} after a full-rank refresh, rejected factorization")
    opt = sco.SpectralAdamW(shapes, device=dev)
    full = [gen.MatrixInputs(94, 0, i, m, n) for i, (m, n) in enumerate(shapes)]
    low = [gen.MatrixInputs(94, 1, i, m, n, r0=8, noise=False) for i, (m, n) in enumerate(shapes)]
    for i, mi in enumerate(full):
        opt.set_state(i, "m_anc", to_dev(gen.stored(mi.m0(), "f32")[0], "f32", dev))
    opt.refresh()
    Ms = []
    for i, mi in enumerate(low):
        pay, M = gen.stored(mi.m0(), "f32")
        Ms.append(M)
        opt.set_state(i, "m_anc", to_dev(pay, "f32", dev))
    opt.refresh()
    st = opt.stats()
    say(f"  stats {st}")
    assert st["factor_rejected"] == 2 and st["not_converged"] == 0
    W = [torch.zeros(m, n, device=dev) for m, n in shapes]
    G = [gen.stored(mi.g_mask(0), "f32") for mi in full]
    opt.step(W, [to_dev(p, "f32", dev) for p, _ in G])
    for i, M in enumerate(Ms):
        U, s, V, _ = oracle.svd(M)
        ref = oracle.project(U, oracle.tikhonov(s, opt.hp["tau_p"]), V, G[i][1])
        err = relf(from_dev(opt.get_filtered(i)), ref)
        say(f"  mat {i}: relF G_filt {err:.3e}")
        assert err <= 1e-4
    opt.close()


def test_determinism_bitwise():
    """Two runs on identical inputs give bitwise identical weights."""
    say("case: determinism 192x256 + 256x128")
    outs = []
    for _ in range(2):
        import spectral_correction_optimizer_amd as sco
        dev = torch.device("cuda")
        shapes = [(192, 256), (256, 128)]
        opt = sco.SpectralAdamW(shapes, device=dev)
        ins = [gen.MatrixInputs(98, 0, i, *s) for i, s in enumerate(shapes)]
        for i, mi in enumerate(ins):
            opt.set_state(i, "m_anc", to_dev(gen.stored(mi.m0(), "f32")[0], "f32", dev))
        W = [to_dev(gen.stored(mi.w0(), "f32")[0], "f32", dev) for mi in ins]
        opt.anchor_update([to_dev(gen.stored(mi.g_anc(0), "f32")[0], "f32", dev) for mi in ins])
        for k in range(3):
            opt.step(W, [to_dev(gen.stored(mi.g_mask(k), "f32")[0], "f32", dev) for mi in ins])
        torch.cuda.synchronize()
        outs.append([w.cpu().numpy().copy() for w in W])
        opt.close()
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_checkpoint_resume_bitwise():
    """Save M_anc, m, v, t and the factors after 2 steps; a fresh handle restored
    from them continues bitwise identically to the uninterrupted run."""
    import spectral_correction_optimizer_amd as sco
    say("case: checkpoint / resume 160x224")
    dev = torch.device("cuda")
    shape = (160, 224)
    mi = gen.MatrixInputs(99, 0, 0, *shape)
    g = [to_dev(gen.stored(mi.g_mask(k), "f32")[0], "f32", dev) for k in range(4)]
    a = sco.SpectralAdamW([shape], device=dev)
    a.set_state(0, "m_anc", to_dev(gen.stored(mi.m0(), "f32")[0], "f32", dev))
    Wa = to_dev(gen.stored(mi.w0(), "f32")[0], "f32", dev)
    a.anchor_update([to_dev(gen.stored(mi.g_anc(0), "f32")[0], "f32", dev)])
    a.step([Wa], [g[0]])
    a.step([Wa], [g[1]])
    ck = {k: a.get_state(0, k) for k in ("m_anc", "adam_m", "adam_v")}
    fac = a.get_factors(0)
    t = a.step_count
    Wb = Wa.clone()
    b = sco.SpectralAdamW([shape], device=dev)
    for k, v in ck.items():
        b.set_state(0, k, v)
    b.set_factors(0, *fac)
    b.step_count = t
    for k in (2, 3):
        a.step([Wa], [g[k]])
        b.step([Wb], [g[k]])
    torch.cuda.synchronize()
    assert torch.equal(Wa, Wb)
    a.close()
    b.close()


def test_nonfinite_gradient_flag():
    import spectral_correction_optimizer_amd as sco
    say("case: non-finite flag")
    dev = torch.device("cuda")
    opt = sco.SpectralAdamW([(64, 64)], device=dev)
    g = torch.zeros(64, 64, device=dev)
    g[3, 5] = float("nan")
    w = torch.zeros(64, 64, device=dev)
    st = opt.stats()
    assert st["nonfinite_grad"] == 0
    opt.step([w], [g])
    st = opt.stats()
    assert st["nonfinite_grad"] == 1 and st["step"] == 1
    opt.close()


def test_q_proj_2048_full_config():
    """The single q_proj workload: 2048x2048 fp32, 1 anchor update, 25 steps
    with fresh noise per step, against the oracle in full."""
    say("case: 2048x2048, 1 refresh + 25 steps (oracle ~1 min)")
    sc = Scenario([(2048, 2048)], [(2, 0, 0)], steps=25)
    rep = sc.run(check_every_step=False)
    Scenario.check(rep)


def test_certificate_failure_polishes_that_matrix_alone():
    """Second (warm) refresh with the factor phase: a noiseless power-law anchor
    (condition number about 1.4e3) fails the Gram certificate of A = M V and is
    polished; a long, narrow pure-noise one (condition number about 1.4, short
    dot products in A = M V) passes it and is not.  Only the polished matrix's final Gram is redone, so
    every matrix must still carry its own E: G_filt of all three matrices
    agrees with the oracle."""
    import spectral_correction_optimizer_amd as sco
    dev = torch.device("cuda")
    shapes = [(512, 128), (2048, 64), (256, 256)]
    say(f"case: certificate failure on one of {shapes}")
    ins = [gen.MatrixInputs(95, 0, 0, *shapes[0], noise=False),
           gen.MatrixInputs(95, 0, 1, *shapes[1], r0=0),
           gen.MatrixInputs(95, 0, 2, *shapes[2])]
    opt = sco.SpectralAdamW(shapes, device=dev)
    for i, mi in enumerate(ins):
        opt.set_state(i, "m_anc", to_dev(gen.stored(mi.m0(), "f32")[0], "f32", dev))
    opt.refresh()
    Ms = []
    for i, mi in enumerate(ins):
        pay, M = gen.stored(mi.g_anc(1), "f32")
        Ms.append(M)
        opt.set_state(i, "m_anc", to_dev(pay, "f32", dev))
    opt.refresh()
    st = opt.stats()
    say(f"  stats {st}")
    assert st["not_converged"] == 0 and st["factor_rejected"] == 0
    assert st["sweeps"][0] > st["factor_sweeps"][0] > 0      # factor phase, then polished
    assert st["sweeps"][1] == st["factor_sweeps"][1] > 0     # certified after the factor phase
    W = [torch.zeros(m, n, device=dev) for m, n in shapes]
    G = [gen.stored(mi.g_mask(0), "f32") for mi in ins]
    opt.step(W, [to_dev(p, "f32", dev) for p, _ in G])
    for i, M in enumerate(Ms):
        U, s, V, _ = oracle.svd(M)
        ref = oracle.project(U, oracle.tikhonov(s, opt.hp["tau_p"]), V, G[i][1])
        err = relf(from_dev(opt.get_filtered(i)), ref)
        say(f"  mat {i}: relF G_filt {err:.3e}")
        assert err <= 1e-4
    opt.close()

def test_async_refresh_matches_synchronous_order():
    """Asynchronous anchor updates (sc_anchor_update_async ... sc_refresh_wait)
    give bitwise the weights of the synchronous call order in which the steps
    issued while a refresh was pending come before it: those steps use the
    previous factors, and the refresh itself computes the same factors.  A second
    asynchronous update while one is pending completes the first one."""
    import spectral_correction_optimizer_amd as sco
    say("case: asynchronous refresh vs synchronous order, 192x256 + 512x128 + 128x128")
    dev = torch.device("cuda")
    shapes = [(192, 256), (512, 128), (128, 128)]
    ins = [gen.MatrixInputs(97, 0, i, *sh) for i, sh in enumerate(shapes)]
    GA = [[to_dev(gen.stored(mi.g_anc(k), "f32")[0], "f32", dev) for mi in ins] for k in range(4)]
    G = [[to_dev(gen.stored(mi.g_mask(k), "f32")[0], "f32", dev) for mi in ins] for k in range(7)]

    def run(asynchronous):
        opt = sco.SpectralAdamW(shapes, device=dev)
        for i, mi in enumerate(ins):
            opt.set_state(i, "m_anc", to_dev(gen.stored(mi.m0(), "f32")[0], "f32", dev))
        W = [to_dev(gen.stored(mi.w0(), "f32")[0], "f32", dev) for mi in ins]
        opt.anchor_update(GA[0])
        opt.step(W, G[0])
        if asynchronous:
            opt.anchor_update_async(GA[1])
            opt.step(W, G[1])
            opt.step(W, G[2])
            opt.refresh_wait()
            opt.step(W, G[3])
            opt.anchor_update_async(GA[2])
            opt.step(W, G[4])
            opt.anchor_update_async(GA[3])  # completes the GA[2] refresh first
            opt.step(W, G[5])
            opt.refresh_wait()
            assert not opt.refresh_pending()
        else:
            opt.step(W, G[1])
            opt.step(W, G[2])
            opt.anchor_update(GA[1])
            opt.step(W, G[3])
            opt.step(W, G[4])
            opt.anchor_update(GA[2])
            opt.step(W, G[5])
            opt.anchor_update(GA[3])
        opt.step(W, G[6])
        torch.cuda.synchronize()
        out = [w.cpu().numpy().copy() for w in W]
        st = opt.stats()
        opt.profile(True)
        if asynchronous:
            with pytest.raises(sco.ScoptError):
                opt.anchor_update_async(GA[3])
        opt.profile(False)
        opt.close()
        return out, st

    wa, sa = run(True)
    ws, ss = run(False)
    say(f"  sweeps async {sa['sweeps']} sync {ss['sweeps']}")
    assert sa["not_converged"] == 0 and ss["not_converged"] == 0
    for a, b in zip(wa, ws):
        assert np.array_equal(a, b)


def test_solve_wave_variants_bitwise():
    """The pair solve on one, two, four or eight wavefronts per pair, with one or two LDS
    copies, computes the same rotations in the same order: factors, sweep counts
    and weights agree bit for bit, on shapes with ragged pair blocks, a
    Cholesky-preconditioned operand and both orientations.  Invalid variants are
    rejected."""
    import spectral_correction_optimizer_amd as sco
    say("case: solve variants (waves x copies), 192x256 + 512x128 + 200x333 + 96x1000 + 700x64")
    dev = torch.device("cuda")
    shapes = [(192, 256), (512, 128), (200, 333), (96, 1000), (700, 64)]
    ins = [gen.MatrixInputs(131, 0, i, *sh) for i, sh in enumerate(shapes)]
    GA = [to_dev(gen.stored(mi.g_anc(0), "f32")[0], "f32", dev) for mi in ins]
    G = [to_dev(gen.stored(mi.g_mask(0), "f32")[0], "f32", dev) for mi in ins]

    def run(waves, copies):
        opt = sco.SpectralAdamW(shapes, device=dev)
        opt.set_solve_waves(waves, copies)
        for i, mi in enumerate(ins):
            opt.set_state(i, "m_anc", to_dev(gen.stored(mi.m0(), "f32")[0], "f32", dev))
        W = [to_dev(gen.stored(mi.w0(), "f32")[0], "f32", dev) for mi in ins]
        opt.anchor_update(GA)
        opt.step(W, G)
        torch.cuda.synchronize()
        fac = [[t.cpu().numpy().copy() for t in opt.get_factors(i)] for i in range(len(shapes))]
        out = [w.cpu().numpy().copy() for w in W]
        st = opt.stats()
        if waves == 0:
            for bad in ((3, 0), (-1, 0), (16, 0), (2, 3), (1, 2), (4, -1)):
                with pytest.raises(sco.ScoptError):
                    opt.set_solve_waves(*bad)
        opt.close()
        return fac, out, st

    ref_f, ref_w, ref_s = run(1, 0)
    assert ref_s["not_converged"] == 0
    for waves, copies in ((2, 2), (2, 1), (4, 2), (4, 1), (8, 2), (8, 1), (0, 0)):
        f, w, st = run(waves, copies)
        say(f"  waves {waves} copies {copies}: sweeps {st['sweeps']} (one wave: {ref_s['sweeps']})")
        assert st["sweeps"] == ref_s["sweeps"] and st["factor_sweeps"] == ref_s["factor_sweeps"]
        for a, b in zip(f, ref_f):
            for x, y in zip(a, b):
                assert np.array_equal(x, y)
        for x, y in zip(w, ref_w):
            assert np.array_equal(x, y)


def test_v_rounds_bitwise():
    """The V rows of the fused sweeps updated two rounds per pass (default) and one
    round per pass give bit-identical factors, sweep counts and weights: a cold
    and a warm refresh (Cholesky factor phase and polishing on the tall operands),
    power-of-two block counts from 4 to 16 in one list, a 128-column V (a partial
    256-column chunk), and a block count that is not a power of two (per-round
    path beside the fused ones).  Invalid values are rejected."""
    import spectral_correction_optimizer_amd as sco
    say("case: V rows 1 vs 2 rounds per pass, 256x256 + 512x128 + 128x1024 + 1024x512 + 512x512 + 320x640")
    dev = torch.device("cuda")
    shapes = [(256, 256), (512, 128), (128, 1024), (1024, 512), (512, 512), (320, 640)]
    ins = [gen.MatrixInputs(171, 0, i, *sh) for i, sh in enumerate(shapes)]
    GA = [[to_dev(gen.stored(mi.g_anc(k), "f32")[0], "f32", dev) for mi in ins] for k in range(2)]
    G = [to_dev(gen.stored(mi.g_mask(0), "f32")[0], "f32", dev) for mi in ins]

    def run(rounds):
        opt = sco.SpectralAdamW(shapes, device=dev)
        opt.set_v_rounds(rounds)
        for i, mi in enumerate(ins):
            opt.set_state(i, "m_anc", to_dev(gen.stored(mi.m0(), "f32")[0], "f32", dev))
        W = [to_dev(gen.stored(mi.w0(), "f32")[0], "f32", dev) for mi in ins]
        sweeps = []
        for k in range(2):
            opt.anchor_update(GA[k])
            st = opt.stats()
            sweeps.append((st["sweeps"], st["factor_sweeps"]))
        opt.step(W, G)
        torch.cuda.synchronize()
        fac = [[t.cpu().numpy().copy() for t in opt.get_factors(i)] for i in range(len(shapes))]
        out = [w.cpu().numpy().copy() for w in W]
        st = opt.stats()
        if rounds == 2:
            for bad in (0, 3, -1):
                with pytest.raises(sco.ScoptError):
                    opt.set_v_rounds(bad)
        opt.close()
        return fac, out, sweeps, st

    ref_f, ref_w, ref_sw, ref_s = run(1)
    f, w, sw, st = run(2)
    say(f"  sweeps (total, factor) per refresh: {sw} (one round per pass: {ref_sw})")
    assert ref_s["not_converged"] == 0 and st["not_converged"] == 0
    assert sw == ref_sw
    for a, b in zip(f, ref_f):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
    for x, y in zip(w, ref_w):
        assert np.array_equal(x, y)


def test_fused_gram_matches_unfused():
    """The fused rotation apply + next-round Gram (bfloat16 three-way split) and
    the standalone float32 Gram give the same SVD to float32 accuracy: singular
    values, reconstruction, G_filt within the parity gate and W after a step (on
    the elements the W gate covers, |G_proj| >= 1e-6), on
    power-of-two block counts (fused), others (not fused) and Cholesky-
    preconditioned operands (fused over the factor rows)."""
    import spectral_correction_optimizer_amd as sco
    say("case: fused vs unfused Gram, 256x256 + 512x128 + 320x1024 + 1024x256 + 2048x512 + 96x1000")
    dev = torch.device("cuda")
    shapes = [(256, 256), (512, 128), (320, 1024), (1024, 256), (2048, 512), (96, 1000)]
    ins = [gen.MatrixInputs(151, 0, i, *sh) for i, sh in enumerate(shapes)]
    GA = [to_dev(gen.stored(mi.g_anc(0), "f32")[0], "f32", dev) for mi in ins]
    G = [to_dev(gen.stored(mi.g_mask(0), "f32")[0], "f32", dev) for mi in ins]

    def run(fuse):
        opt = sco.SpectralAdamW(shapes, device=dev)
        opt.set_fused_gram(fuse)
        opt.keep_proj(True)
        for i, mi in enumerate(ins):
            opt.set_state(i, "m_anc", to_dev(gen.stored(mi.m0(), "f32")[0], "f32", dev))
        W = [to_dev(gen.stored(mi.w0(), "f32")[0], "f32", dev) for mi in ins]
        opt.anchor_update(GA)
        opt.step(W, G)
        torch.cuda.synchronize()
        fac = [[t.double().cpu().numpy() for t in opt.get_factors(i)] for i in range(len(shapes))]
        gf = [[t.double().cpu().numpy() for t in opt.get_filtered(i, proj=True)]
              for i in range(len(shapes))]
        out = [w.double().cpu().numpy() for w in W]
        st = opt.stats()
        opt.close()
        return fac, gf, out, st

    fa, gfa, wa, sa = run(True)
    fb, gfb, wb, sb = run(False)
    say(f"  sweeps fused {sa['sweeps']} unfused {sb['sweeps']}")
    assert sa["not_converged"] == 0 and sb["not_converged"] == 0
    for i, (m, n) in enumerate(shapes):
        (Ua, sva, Va), (Ub, svb, Vb) = fa[i], fb[i]
        s_err = np.abs(np.sort(sva)[::-1] - np.sort(svb)[::-1]).max() / svb.max()
        rec = np.linalg.norm((Ua * sva) @ Va.T - (Ub * svb) @ Vb.T) / np.linalg.norm((Ub * svb) @ Vb.T)
        g_rel = np.linalg.norm(gfa[i][0] - gfb[i][0]) / np.linalg.norm(gfb[i][0])
        # W on the elements the parity gate covers: |G_proj| >= 1e-6 (near g = 0
        # the first AdamW update amplifies any G_proj difference by lr / eps)
        keep = np.abs(gfb[i][1]) >= 1e-6
        w_err = np.abs(wa[i] - wb[i])[keep].max()
        say(f"  {m}x{n}: s {s_err:.2e} recon {rec:.2e} G_filt {g_rel:.2e} W {w_err:.2e}")
        assert s_err < 1e-5 and rec < 1e-5 and g_rel < 1e-4 and w_err < 1e-7


def test_sync_check_0_enqueue_only_matches_oracle():
    """The enqueue-only refresh (sync_check = 0: no host polls, a fixed sweep
    budget whose rounds exit at once on converged matrices, the factor phase and
    the polishing of matrices failing the Gram certificate decided on the device)
    against the oracle over two warm refreshes of the three shape classes."""
    shapes = [(520, 96), (96, 520), (1024, 256), (256, 256), (200, 136)]
    say(f"case: sync_check=0 {shapes}, refresh every 2 steps, 4 steps")
    sc = Scenario(shapes, [(132, 0, i) for i in range(len(shapes))], steps=4, anchor_every=2,
                  max_sweeps=16)
    rep = sc.run(gpu_hp=dict(sync_check=0))
    Scenario.check(rep)
    st = rep["stats"]
    say(f"  stats {st}")
    assert st["not_converged"] == 0 and st["factor_rejected"] == 0
    assert st["factor_sweeps_max"] > 0  # the factor phase ran without host decisions


@pytest.mark.parametrize("stop", [0.9, 0.0])
def test_sweep_stop_rule_against_oracle(stop):
    """The sweep-stop rule at 0.9 ends the plain sweeps after a matrix's first
    sweep: the final Gram's certificate rejects them, their sweeps resume and
    their final Gram is redone, and the result still matches the oracle (in the
    factor phase the rule stays capped at 1e-4); with the rule off (0) sweeps end
    only on the convergence threshold.  Cold and warm refreshes of the three
    shape classes."""
    import spectral_correction_optimizer_amd as sco
    shapes = [(256, 256), (128, 512), (512, 128), (1024, 256), (200, 136)]
    say(f"case: sweep stop {stop}, {shapes}, refresh every 2 steps, 4 steps")
    sc = Scenario(shapes, [(181, 0, i) for i in range(len(shapes))], steps=4, anchor_every=2)

    def setup(opt):
        for bad in (-0.1, 1.0, float("nan")):
            with pytest.raises(sco.ScoptError):
                opt.set_sweep_stop(bad)
        opt.set_sweep_stop(stop)

    rep = sc.run(setup=setup)
    Scenario.check(rep)
    st = rep["stats"]
    say(f"  stats {st}")
    assert st["not_converged"] == 0
    # every refresh still ran more than one sweep per matrix
    assert all(min(g) >= 2 for g, _ in rep["sweeps"])


def test_sweep_cap_reports_not_converged():
    """max_sweeps = 1 stops every matrix after one sweep of a cold refresh: the
    stats report each matrix as not converged with one sweep, and a step still
    runs on the partial factors."""
    import spectral_correction_optimizer_amd as sco
    dev = torch.device("cuda")
    shapes = [(256, 192), (128, 320)]
    say(f"case: max_sweeps=1 on {shapes}")
    ins = [gen.MatrixInputs(133, 0, i, *sh) for i, sh in enumerate(shapes)]
    opt = sco.SpectralAdamW(shapes, device=dev, max_sweeps=1)
    for i, mi in enumerate(ins):
        opt.set_state(i, "m_anc", to_dev(gen.stored(mi.m0(), "f32")[0], "f32", dev))
    opt.refresh()
    st = opt.stats()
    say(f"  stats {st}")
    assert st["not_converged"] == len(shapes) and st["sweeps"] == [1] * len(shapes)
    W = [torch.zeros(*sh, device=dev) for sh in shapes]
    opt.step(W, [to_dev(gen.stored(mi.g_mask(0), "f32")[0], "f32", dev) for mi in ins])
    torch.cuda.synchronize()
    assert all(torch.isfinite(w).all().item() for w in W)
    opt.close()


def test_nonfinite_anchor_flag_and_other_matrices_unaffected():
    """A NaN in one matrix's anchor gradient: the anchor flag is raised, that
    matrix stops after its first sweep and is reported as not converged (a NaN
    no longer reads as a converged sweep), and the other matrix of the handle
    still matches the oracle."""
    import spectral_correction_optimizer_amd as sco
    dev = torch.device("cuda")
    shapes = [(192, 128), (160, 96)]
    say(f"case: NaN in the anchor gradient of matrix 1 of {shapes}")
    ins = [gen.MatrixInputs(134, 0, i, *sh) for i, sh in enumerate(shapes)]
    opt = sco.SpectralAdamW(shapes, device=dev)
    ora = oracle.Optimizer(shapes[:1], opt_hp(opt))
    for i, mi in enumerate(ins):
        pay, val = gen.stored(mi.m0(), "f32")
        opt.set_state(i, "m_anc", to_dev(pay, "f32", dev))
        if i == 0:
            ora.set_anchor_momentum(0, val)
    ga = [gen.stored(mi.g_anc(0), "f32") for mi in ins]
    bad = ga[1][0].copy()
    bad[7, 3] = np.nan
    assert opt.stats()["nonfinite_anchor"] == 0
    opt.anchor_update([to_dev(ga[0][0], "f32", dev), to_dev(bad, "f32", dev)])
    ora.anchor_update([ga[0][1]])
    st = opt.stats()
    say(f"  stats {st}")
    assert st["nonfinite_anchor"] == 1 and st["not_converged"] == 1
    assert st["sweeps"][1] == 1
    gm = [gen.stored(mi.g_mask(0), "f32") for mi in ins]
    W = [to_dev(gen.stored(mi.w0(), "f32")[0], "f32", dev) for mi in ins]
    Wo = ora.step([gen.stored(ins[0].w0(), "f32")[1]], [gm[0][1]])
    opt.step(W, [to_dev(p, "f32", dev) for p, _ in gm])
    ef = relf(from_dev(opt.get_filtered(0)), ora.last_filt[0])
    keep = np.abs(ora.last_proj[0]) >= 1e-6
    ew = float(np.abs(from_dev(W[0]) - Wo[0])[keep].max())
    say(f"  matrix 0: relF G_filt {ef:.3e} W {ew:.3e}")
    assert ef <= 1e-4 and ew <= 1e-7
    opt.close()


def opt_hp(opt):
    return {k: opt.hp[k] for k in ("tau_p", "alpha", "beta_anc", "lr", "beta1", "beta2", "eps",
                                   "weight_decay")}


def test_async_refresh_matches_oracle():
    """The asynchronous anchor updates against the oracle run in the synchronous
    order they stand for: steps issued while a refresh is pending use the
    previous factors, so the oracle takes those steps before the anchor update.
    G_filt and G_proj of the steps outside a pending window (reading them back
    completes the refresh) and the weights at the end, which carry every step,
    are compared."""
    import spectral_correction_optimizer_amd as sco
    from tests.gpu_harness import REL_TOL, SMALL_G, W_TOL
    dev = torch.device("cuda")
    shapes = [(192, 256), (512, 128), (128, 128)]
    say(f"case: asynchronous refresh vs the oracle in synchronous order, {shapes}")
    ins = [gen.MatrixInputs(135, 0, i, *sh) for i, sh in enumerate(shapes)]
    GA = [[gen.stored(mi.g_anc(k), "f32") for mi in ins] for k in range(3)]
    G = [[gen.stored(mi.g_mask(k), "f32") for mi in ins] for k in range(6)]
    opt = sco.SpectralAdamW(shapes, device=dev)
    opt.keep_proj(True)
    ora = oracle.Optimizer(shapes, opt_hp(opt))
    W, Wo = [], []
    for i, mi in enumerate(ins):
        pay, val = gen.stored(mi.m0(), "f32")
        opt.set_state(i, "m_anc", to_dev(pay, "f32", dev))
        ora.set_anchor_momentum(i, val)
        pay, val = gen.stored(mi.w0(), "f32")
        W.append(to_dev(pay, "f32", dev))
        Wo.append(val)
    dv = lambda xs: [to_dev(p, "f32", dev) for p, _ in xs]
    hv = lambda xs: [v for _, v in xs]
    worst = [0.0, 0.0]
    small = None

    def step(k, inspect=True):
        # inspect=False while a refresh is pending: reading G_filt back would
        # complete the refresh and switch the next steps to the new factors
        nonlocal Wo, small
        opt.step(W, dv(G[k]))
        Wo = ora.step(Wo, hv(G[k]))
        if small is None:
            small = [np.abs(p) < SMALL_G for p in ora.last_proj]
        if not inspect:
            return
        for i in range(len(shapes)):
            gf, gp = opt.get_filtered(i, proj=True)
            worst[0] = max(worst[0], relf(from_dev(gf), ora.last_filt[i]))
            worst[1] = max(worst[1], relf(from_dev(gp), ora.last_proj[i]))

    # the anchor gradients of an asynchronous update must stay allocated until its
    # refresh is completed (the EMA reads them on the library's own stream)
    ga_dev = [dv(GA[k]) for k in range(3)]
    opt.anchor_update(ga_dev[0])
    ora.anchor_update(hv(GA[0]))
    step(0)
    opt.anchor_update_async(ga_dev[1])   # pending while steps 1 and 2 run
    step(1, inspect=False)
    step(2, inspect=False)
    opt.refresh_wait()
    ora.anchor_update(hv(GA[1]))
    step(3)
    opt.anchor_update_async(ga_dev[2])
    step(4, inspect=False)
    opt.refresh_wait()
    ora.anchor_update(hv(GA[2]))
    step(5)
    torch.cuda.synchronize()
    werr = max(float(np.abs(from_dev(W[i]) - Wo[i])[~small[i]].max()) for i in range(len(shapes)))
    say(f"  worst relF G_filt {worst[0]:.3e} G_proj {worst[1]:.3e} W {werr:.3e}")
    assert worst[0] <= REL_TOL and worst[1] <= REL_TOL and werr <= W_TOL
    assert opt.stats()["not_converged"] == 0
    opt.close()
