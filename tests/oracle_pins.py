"""Pins of the CPU oracle: facts fixed by the pages or by mathematics, not by the
oracle itself.

Each ``pin_*`` takes the oracle module and raises AssertionError when the oracle
disagrees.  They are collected by tests/test_oracle_pins.py and re-run against
deliberately broken copies of the oracle in tests/test_oracle_mutations.py to
show that plausible mistakes (a dropped term, a wrong sign or index, a
transposed operand) are caught.

Page citations refer to the papernotes.org notes on "Communication-Efficient LLM
Adaptation over Decentralized GPU Meshes": "Key design 2" (anchor EMA),
"Key design 3" (SVD, Tikhonov filter, two-sided projection, combination),
"Training strategy" (AdamW, defaults) and "Ablations" (the meaning of the
alpha and tau extremes).
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

EPS53 = 2.0 ** -53


def _frac(a):
    return np.array([[float(Fraction(x)) for x in row] for row in a])


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _haar(seed, n, r):
    q, rr = np.linalg.qr(_rand(seed, n, r))
    return q * np.where(np.diag(rr) < 0, -1.0, 1.0)


def _relf(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def filt(o, M, G, tau):
    """Full filter path of the oracle: SVD, Tikhonov response, projection."""
    U, s, V, _ = o.svd(M, threads=2)
    return o.project(U, o.tikhonov(s, tau), V, G)


# ---- P1: hand-worked 4x3 case (exact rationals) --------------------------------

def pin_worked_4x3(o):
    g = json.load(open(os.path.join(GOLDEN, "worked_4x3.json")))
    M = np.array(g["M"])
    U, s, V, sweeps = o.svd(M, threads=1)
    assert sweeps > 0
    assert np.allclose(s, g["singular_values"], rtol=0, atol=1e-14), s
    d = o.tikhonov(s, g["tau_p"])
    assert np.allclose(d, [float(Fraction(x)) for x in g["d"]], rtol=0, atol=1e-15), d
    G = np.array(g["G_mask"])
    G_filt = o.project(U, d, V, G)
    assert np.allclose(G_filt, _frac(g["G_filt"]), rtol=0, atol=1e-14), G_filt
    G_proj = o.combine(G, G_filt, g["alpha"])
    assert np.allclose(G_proj, _frac(g["G_proj"]), rtol=0, atol=1e-14), G_proj


# ---- P2: AdamW with constant gradient, closed form over T steps ------------------

def pin_adamw_constant_grad(o):
    g = json.load(open(os.path.join(GOLDEN, "worked_4x3.json")))
    a = g["adamw"]
    gp = _frac(g["G_proj"])
    W = np.full(gp.shape, a["W0"])
    m = np.zeros_like(W)
    v = np.zeros_like(W)
    W1 = None
    for t in range(1, a["T"] + 1):
        W, m, v = o.adamw(W, m, v, gp, t, a["lr"], a["beta1"], a["beta2"], a["eps"], a["weight_decay"])
        if t == 1:
            W1 = W.copy()
    c = 1.0 - a["lr"] * a["weight_decay"]
    r = gp / (np.abs(gp) + a["eps"])
    T = a["T"]
    WT = c ** T * a["W0"] - a["lr"] * r * (1.0 - c ** T) / (1.0 - c)
    assert np.allclose(W, WT, rtol=0, atol=1e-14), np.abs(W - WT).max()
    W1ref = c * a["W0"] - a["lr"] * r
    assert np.allclose(W1, W1ref, rtol=0, atol=1e-15)
    # bias-corrected moments equal g and g^2 exactly in exact arithmetic
    assert np.allclose(m / (1 - a["beta1"] ** T), gp, rtol=1e-13, atol=0)
    assert np.allclose(v / (1 - a["beta2"] ** T), gp * gp, rtol=1e-12, atol=0)


# ---- P3: alpha = 1 is plain AdamW on G_mask (torch.optim.AdamW, fp64, CPU) --------

def pin_alpha1_is_torch_adamw(o):
    import torch
    hp = dict(tau_p=1e-3, alpha=1.0, beta_anc=0.9, lr=2e-5, beta1=0.9, beta2=0.999, eps=1e-8,
              weight_decay=0.01)
    m_, n_ = 9, 7
    opt = o.Optimizer([(m_, n_)], hp, w_dtype="f64", state_dtype="f64", threads=1)
    opt.anchor_update([_rand(1, m_, n_) * 1e-2])
    W0 = _rand(2, m_, n_) * 0.02
    p = torch.nn.Parameter(torch.tensor(W0, dtype=torch.float64))
    topt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                             weight_decay=hp["weight_decay"], foreach=False)
    W = W0.copy()
    for k in range(6):
        G = _rand(10 + k, m_, n_) * 1e-3
        W = opt.step([W], [G])[0]
        p.grad = torch.tensor(G, dtype=torch.float64)
        topt.step()
        assert np.allclose(W, p.detach().numpy(), rtol=0, atol=1e-16), np.abs(W - p.detach().numpy()).max()


# ---- P4: tau = 0 and full rank: projectors onto col(M) / row(M) ------------------

def pin_tau0_projectors(o):
    # square, full rank: G_filt = G
    M = _rand(3, 12, 12)
    G = _rand(4, 12, 12)
    assert _relf(filt(o, M, G, 0.0), G) < 1e-12
    # tall: G_filt = M (M^T M)^-1 M^T G (row space is all of R^n)
    M = _rand(5, 15, 6)
    G = _rand(6, 15, 6)
    ref = M @ np.linalg.solve(M.T @ M, M.T @ G)
    assert _relf(filt(o, M, G, 0.0), ref) < 1e-11
    # wide: G_filt = G M^T (M M^T)^-1 M
    M = _rand(7, 5, 13)
    G = _rand(8, 5, 13)
    ref = (G @ M.T) @ np.linalg.solve(M @ M.T, M)
    assert _relf(filt(o, M, G, 0.0), ref) < 1e-11


# ---- P5: tau > 0, exact low rank with known factors (no SVD in the reference) -----

def pin_known_factors(o):
    for (m, n, r0, seed) in [(20, 11, 4, 11), (9, 17, 3, 12), (16, 16, 16, 13)]:
        U0 = _haar(seed, m, r0)
        V0 = _haar(seed + 100, n, r0)
        s0 = np.sort(np.random.default_rng(seed).uniform(0.5, 2.0, r0))[::-1] * 1e-2
        M = (U0 * s0) @ V0.T
        G = _rand(seed + 200, m, n)
        tau = 3e-3
        d0 = s0 / (s0 + tau)
        ref = U0 @ (d0[:, None] * (U0.T @ G @ V0) * d0[None, :]) @ V0.T
        assert _relf(filt(o, M, G, tau), ref) < 1e-11, (m, n, _relf(filt(o, M, G, tau), ref))


# ---- P6: rank one --------------------------------------------------------------

def pin_rank_one(o):
    u = _haar(21, 10, 1)[:, 0]
    v = _haar(22, 7, 1)[:, 0]
    sig, tau = 2.5, 0.7
    M = sig * np.outer(u, v)
    G = _rand(23, 10, 7)
    d = sig / (sig + tau)
    ref = d * d * (u @ G @ v) * np.outer(u, v)
    assert _relf(filt(o, M, G, tau), ref) < 1e-12


# ---- P7: a gradient inside a strong subspace passes nearly unchanged -------------

def pin_strong_subspace(o):
    m, n, k = 40, 30, 5
    U0 = _haar(31, m, n)
    V0 = _haar(32, n, n)
    s = np.concatenate([np.linspace(10.0, 5.0, k), np.linspace(1e-3, 1e-4, n - k)])
    M = (U0 * s) @ V0.T
    C = _rand(33, k, k)
    G = U0[:, :k] @ C @ V0[:, :k].T
    tau = 1e-3
    dk = (s[:k] / (s[:k] + tau)).min()
    err = _relf(filt(o, M, G, tau), G)
    assert err <= 1 - dk * dk + 1e-12, err
    assert err < 1e-3


# ---- P8: bounds and the two tau extremes -----------------------------------------

def pin_bounds_and_limits(o):
    import scipy.linalg
    M = _rand(41, 14, 9)
    G = _rand(42, 14, 9)
    U, s, V, _ = o.svd(M, threads=1)
    for tau in [1e-6, 1e-2, 1.0, 10.0]:
        d = o.tikhonov(s, tau)
        assert np.all(d >= 0) and np.all(d < 1)
        Gf = o.project(U, d, V, G)
        assert np.linalg.norm(Gf) <= d.max() ** 2 * np.linalg.norm(G) * (1 + 1e-12)
    # tau -> infinity: tau^2 G_filt -> (M M^T)^1/2 G (M^T M)^1/2, so G_filt -> 0
    tau = 1e7
    lim = np.real(scipy.linalg.sqrtm(M @ M.T)) @ G @ np.real(scipy.linalg.sqrtm(M.T @ M))
    Gf = o.project(U, o.tikhonov(s, tau), V, G)
    assert _relf(tau * tau * Gf, lim) < 1e-5
    # tau -> 0 with s >> tau: d -> 1
    assert np.all(o.tikhonov(s, 1e-14) > 1 - 1e-12)
    # zero singular value with tau = 0 reads d = 0
    assert o.tikhonov(np.array([0.0, 1.0]), 0.0).tolist() == [0.0, 1.0]


# ---- P9: equivariances -----------------------------------------------------------

def pin_equivariance(o):
    M = _rand(51, 11, 6)
    G = _rand(52, 11, 6)
    tau = 0.3
    F = filt(o, M, G, tau)
    # transpose: ties the wide path (A = M^T) to the tall path
    assert _relf(filt(o, M.T.copy(), G.T.copy(), tau), F.T) < 1e-12
    # orthogonal change of basis on both sides
    QL = _haar(53, 11, 11)
    QR = _haar(54, 6, 6)
    assert _relf(filt(o, QL @ M @ QR.T, QL @ G @ QR.T, tau), QL @ F @ QR.T) < 1e-12
    # scaling M and tau together
    assert _relf(filt(o, 7.0 * M, G, 7.0 * tau), F) < 1e-12
    # linear in G
    G2 = _rand(55, 11, 6)
    assert _relf(filt(o, M, 2.0 * G - 3.0 * G2, tau), 2.0 * F - 3.0 * filt(o, M, G2, tau)) < 1e-12


# ---- P10: SVD against LAPACK and its defining properties -------------------------

def pin_svd_lapack(o):
    for (m, n, seed) in [(37, 23, 61), (23, 37, 62), (30, 30, 63), (64, 48, 64)]:
        M = _rand(seed, m, n)
        U, s, V, sweeps = o.svd(M, threads=3)
        assert sweeps > 0
        r = min(m, n)
        s_ref = np.linalg.svd(M, compute_uv=False)
        assert np.max(np.abs(s - s_ref)) <= 1e-13 * s_ref[0]
        assert np.all(np.diff(s) <= 0)
        assert np.linalg.norm((U * s) @ V.T - M) <= 50 * r * EPS53 * np.linalg.norm(M)
        assert np.linalg.norm(U.T @ U - np.eye(r)) <= 50 * r * EPS53
        assert np.linalg.norm(V.T @ V - np.eye(r)) <= 50 * r * EPS53
        # the filtered gradient does not depend on which valid factors are used
        Ul, sl, Vlt = np.linalg.svd(M, full_matrices=False)
        G = _rand(seed + 1, m, n)
        d, dl = o.tikhonov(s, 0.5), o.tikhonov(sl, 0.5)
        assert _relf(o.project(U, d, V, G), o.project(Ul, dl, Vlt.T, G)) < 1e-12


# ---- P11: brute force on tiny cases -----------------------------------------------

def pin_tiny_cases(o):
    a, b, c, dd = 3.0, -1.0, 2.0, 0.5
    M = np.array([[a, b], [c, dd]])
    S = a * a + b * b + c * c + dd * dd
    D = a * dd - b * c
    root = np.sqrt(S * S - 4 * D * D)
    s_ref = np.sqrt([(S + root) / 2, (S - root) / 2])
    _, s, _, _ = o.svd(M, threads=1)
    assert np.allclose(s, s_ref, rtol=1e-14, atol=0)
    # one column: s = ||M||, U = M / s, V = [1]
    Mc = _rand(71, 6, 1)
    U, s, V, _ = o.svd(Mc, threads=1)
    assert abs(s[0] - np.sqrt((Mc ** 2).sum())) < 1e-14 * s[0]
    assert np.allclose(U[:, 0], Mc[:, 0] / s[0], atol=1e-15) and V[0, 0] == 1.0
    # one row
    Mr = _rand(72, 1, 5)
    U, s, V, _ = o.svd(Mr, threads=1)
    assert abs(s[0] - np.linalg.norm(Mr)) < 1e-14 * s[0] and U[0, 0] == 1.0
    # zero matrix: all singular values zero, d = 0, G_filt = 0
    Z = np.zeros((5, 4))
    U, s, V, _ = o.svd(Z, threads=1)
    assert np.all(s == 0)
    Gf = o.project(U, o.tikhonov(s, 1e-3), V, _rand(73, 5, 4))
    assert np.all(Gf == 0)


# ---- P12: anchor EMA -----------------------------------------------------------

def pin_ema(o):
    M0 = _rand(81, 6, 5)
    G = _rand(82, 6, 5)
    beta = 0.9
    M = M0.copy()
    for _ in range(7):
        M = o.ema(M, G, beta)
    # k updates with a constant anchor gradient: beta^k M0 + (1 - beta^k) G
    assert np.allclose(M, beta ** 7 * M0 + (1 - beta ** 7) * G, rtol=0, atol=1e-14)
    assert np.array_equal(o.ema(M0, G, 0.0), G) and np.array_equal(o.ema(M0, G, 1.0), M0)
    assert o.ema(np.array([2.0]), np.array([4.0]), 0.5)[0] == 3.0


# ---- P13: determinism across thread counts ----------------------------------------

def pin_thread_determinism(o):
    M = _rand(91, 50, 34)
    r1 = o.svd(M, threads=1)
    r5 = o.svd(M, threads=5)
    for a, b in zip(r1[:3], r5[:3]):
        assert np.array_equal(a, b)
    assert r1[3] == r5[3]


# ---- storage rounding -----------------------------------------------------------

def pin_storage_rounding(o):
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8 + 2.0 ** -30), 0.1, 2.0 ** -140])
    got = o.round_storage(x, "bf16")
    # ties to even, above-tie rounds up, 0.1 -> 0x3DCD = 0.10009765625, subnormal quantum 2^-133
    assert got.tolist() == [1.0, 1.0 + 2.0 ** -6, -(1.0 + 2.0 ** -7), 0.10009765625, 0.0]
    assert o.round_storage(np.array([0.1]), "f32")[0] == float(np.float32(0.1))


# ---- the stateful driver: anchor EMA -> refresh -> steps, with storage rounding ------

_WORKED_HP = dict(tau_p=1.0, alpha=0.3, beta_anc=0.75, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                  weight_decay=1e-2)
# an anchor gradient with every row non-zero (the worked M has a zero fourth row)
_WORKED_GANC = [[1.0, 2.0, 0.0], [0.0, -1.0, 1.0], [0.5, 0.0, -2.0], [1.0, 1.0, 1.0]]


def pin_optimizer_driver_worked_4x3(o):
    """``Optimizer`` chains the EMA of "Key design 2", the refresh, the filter and
    projection of "Key design 3" and AdamW in the right order and with the right
    arguments: two anchor arrivals with the same gradient G from M0 give
    M = b^2 M0 + (1 - b^2) G, and M0 is chosen so that this is the hand-worked M;
    the steps then reproduce the hand-worked G_filt, G_proj and the AdamW closed
    form.  An anchor arrival between steps (here one that leaves M in place) does
    not advance the step count."""
    g = json.load(open(os.path.join(GOLDEN, "worked_4x3.json")))
    a = g["adamw"]
    hp = dict(_WORKED_HP)
    assert hp["tau_p"] == g["tau_p"] and hp["alpha"] == g["alpha"] and hp["lr"] == a["lr"]
    b = hp["beta_anc"]
    M = np.array(g["M"])
    Ga = np.array(_WORKED_GANC)
    M0 = (M - (1.0 - b * b) * Ga) / (b * b)
    opt = o.Optimizer([(4, 3)], hp, w_dtype="f64", state_dtype="f64", threads=1)
    opt.set_anchor_momentum(0, M0)
    opt.anchor_update([Ga], defer_refresh=True)
    assert not np.allclose(opt.M[0], M, atol=1e-3)  # one arrival is not there yet
    opt.anchor_update([Ga])
    assert np.allclose(opt.M[0], M, rtol=0, atol=1e-14), opt.M[0]
    U, s, V = opt.factors[0]
    assert np.allclose(s, g["singular_values"], rtol=0, atol=1e-14), s
    assert np.allclose(opt.d[0], [float(Fraction(x)) for x in g["d"]], rtol=0, atol=1e-14)
    assert opt.t == 0
    G = np.array(g["G_mask"])
    gp = _frac(g["G_proj"])
    W = np.full((4, 3), a["W0"])
    c = 1.0 - a["lr"] * a["weight_decay"]
    r = gp / (np.abs(gp) + a["eps"])
    for t in range(1, a["T"] + 1):
        W = opt.step([W], [G])[0]
        assert opt.t == t
        assert np.allclose(opt.last_filt[0], _frac(g["G_filt"]), rtol=0, atol=1e-14)
        assert np.allclose(opt.last_proj[0], gp, rtol=0, atol=1e-14)
        WT = c ** t * a["W0"] - a["lr"] * r * (1.0 - c ** t) / (1.0 - c)
        assert np.allclose(W, WT, rtol=0, atol=1e-14), (t, np.abs(W - WT).max())
        if t == 2:
            opt.anchor_update([M])  # b M + (1 - b) M = M: same factors, t unchanged
            assert opt.t == 2 and np.allclose(opt.M[0], M, rtol=0, atol=1e-14)


def pin_optimizer_deferred_refresh(o):
    """An anchor arrival whose SVD refresh is deferred to the next step gives the
    same weights, bit for bit, as one refreshed at once (the factors are a
    function of M alone), and the deferred chain really uses the new M."""
    rng_ = np.random.default_rng(77)
    shape = (6, 4)
    hp = dict(tau_p=1e-3, alpha=0.3, beta_anc=0.9, lr=2e-5, beta1=0.9, beta2=0.999, eps=1e-8,
              weight_decay=0.01)
    ga = [1e-2 * rng_.standard_normal(shape) for _ in range(3)]
    gm = [1e-3 * rng_.standard_normal(shape) for _ in range(3)]
    W0 = 0.02 * rng_.standard_normal(shape)
    outs = []
    for defer in (False, True, None):
        opt = o.Optimizer([shape], hp, threads=1)
        opt.set_anchor_momentum(0, 1e-2 * np.ones(shape))
        W = W0.copy()
        for k in range(3):
            if defer is not None or k == 0:
                opt.anchor_update([ga[k]], defer_refresh=bool(defer))
            W = opt.step([W], [gm[k]])[0]
        outs.append(W)
    assert np.array_equal(outs[0], outs[1])
    assert not np.array_equal(outs[0], outs[2])  # later anchors do change the result


def _rne_f32(x):
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def _rne_bf16(x):
    """Round float64 to bfloat16 (8 significant bits), nearest-even, on the bit
    pattern: add half of the dropped 45-bit field (minus one unless the kept
    last bit is odd) and clear the field.  Normal numbers only."""
    x = np.asarray(x, np.float64)
    u = x.view(np.uint64)
    keep = (u >> np.uint64(45)) & np.uint64(1)
    u = (u + np.uint64((1 << 44) - 1) + keep) & ~np.uint64((1 << 45) - 1)
    return u.view(np.float64)


def pin_optimizer_storage_rounding(o):
    """After every call, the state the driver stores in a narrower type (M_anc
    after an anchor arrival; m, v and W after a step) is the round-to-nearest-even
    of what the same call computes in float64 from the same stored inputs.  The
    float64 driver is re-seeded with the narrow driver's state before each call."""
    rng_ = np.random.default_rng(123)
    shape = (7, 5)
    hp = dict(tau_p=1e-3, alpha=0.3, beta_anc=0.9, lr=2e-5, beta1=0.9, beta2=0.999, eps=1e-8,
              weight_decay=0.01)
    w_round = {"f32": _rne_f32, "bf16": _rne_bf16}
    assert _rne_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert _rne_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    for wdt in ("f32", "bf16"):
        nar = o.Optimizer([shape], hp, w_dtype=wdt, state_dtype="f32", threads=1)
        wide = o.Optimizer([shape], hp, w_dtype="f64", state_dtype="f64", threads=1)
        M0 = _rne_f32(1e-2 * rng_.standard_normal(shape))
        nar.set_anchor_momentum(0, M0)
        W = w_round[wdt](0.02 * rng_.standard_normal(shape))
        for call in range(6):
            if call in (0, 3):
                Ga = _rne_f32(1e-2 * rng_.standard_normal(shape))
                wide.M[0] = nar.M[0].copy()
                nar.anchor_update([Ga])
                wide.anchor_update([Ga])
                assert np.array_equal(nar.M[0], _rne_f32(wide.M[0])), (wdt, call)
                assert not np.array_equal(nar.M[0], wide.M[0])
                continue
            wide.M[0], wide.m[0], wide.v[0], wide.t = nar.M[0].copy(), nar.m[0].copy(), \
                nar.v[0].copy(), nar.t
            wide.factors[0], wide.d[0] = nar.factors[0], nar.d[0]
            G = _rne_f32(1e-3 * rng_.standard_normal(shape))
            Wn = nar.step([W], [G])[0]
            Ww = wide.step([W], [G])[0]
            assert np.array_equal(nar.m[0], _rne_f32(wide.m[0])), (wdt, call, "m")
            assert np.array_equal(nar.v[0], _rne_f32(wide.v[0])), (wdt, call, "v")
            assert np.array_equal(Wn, w_round[wdt](Ww)), (wdt, call, "W")
            assert not (np.array_equal(nar.v[0], wide.v[0]) and np.array_equal(nar.m[0], wide.m[0]))
            W = Wn


# ---- the in-graph activation mask ("Key design 1") -------------------------------

def pin_mask_keep_count(o):
    """K = round((1 - p) H) kept dimensions per token, ties rounded up (reading)."""
    mk = o.masking
    assert mk.keep_count(2048, 0.95) == 102  # 102.4
    assert mk.keep_count(2048, 0.90) == 205  # 204.8
    assert mk.keep_count(4096, 0.95) == 205  # 204.8
    assert mk.keep_count(10, 0.25) == 8      # 7.5
    assert mk.keep_count(8, 0.0) == 8 and mk.keep_count(8, 1.0) == 0


def _unshift(y, s):
    """Inverse of x -> x ^ (x >> s) on uint64 words."""
    x = y.copy()
    for _ in range(64 // s + 1):
        x = y ^ (x >> np.uint64(s))
    return x


def pin_mask_mixer_inverts(o):
    """The SplitMix64 output function (Steele, Lea and Flood 2014: xor-shifts by 30, 27,
    31 and the odd multipliers 0xBF58476D1CE4E5B9, 0x94D049BB133111EB) is a bijection of
    64-bit words: undoing its steps with the modular inverses of the multipliers
    recovers the input, which fails for a dropped or altered step or constant."""
    mk = o.masking
    z = np.random.default_rng(5).integers(0, 2 ** 63, 2000, dtype=np.uint64) * np.uint64(2) + \
        np.random.default_rng(6).integers(0, 2, 2000, dtype=np.uint64)
    y = mk.mix64(z)
    i1 = np.uint64(pow(0xBF58476D1CE4E5B9, -1, 2 ** 64))
    i2 = np.uint64(pow(0x94D049BB133111EB, -1, 2 ** 64))
    with np.errstate(over="ignore"):
        x = _unshift(y, 31) * i2
        x = _unshift(x, 27) * i1
    x = _unshift(x, 30)
    assert np.array_equal(x, z)
    assert all(mk.mix64_int(int(a)) == int(b) for a, b in zip(z[:64], y[:64]))


def pin_mask_avalanche(o):
    """Flipping any one input bit flips about half of the 64 output bits: the hash
    behaves like a random function, which the uniform-subset reading relies on."""
    mk = o.masking
    z = np.random.default_rng(7).integers(0, 2 ** 63, 4000, dtype=np.uint64)
    y = mk.mix64(z)
    for b in range(64):
        d = y ^ mk.mix64(z ^ np.uint64(1 << b))
        flips = np.unpackbits(d.view(np.uint8)).reshape(-1, 64).sum(axis=1)
        assert 31.0 < flips.mean() < 33.0, (b, flips.mean())


def pin_mask_exact_k(o):
    """Every token keeps exactly K distinct dimensions in [0, H), listed in ascending
    order; K = 0 keeps none and K = H keeps all."""
    mk = o.masking
    for T, H, K in [(5, 64, 16), (3, 100, 0), (3, 100, 100), (2, 2048, 102), (4, 7, 3)]:
        idx = mk.indices(2, 9, 1, T, H, K)
        assert idx.shape == (T, K) and idx.dtype == np.int32
        if K:
            assert (np.diff(idx, axis=1) > 0).all() and idx.min() >= 0 and idx.max() < H
        if K == H:
            assert (idx == np.arange(H)).all()


def pin_mask_nested(o):
    """Smallest-hash selection: the kept set for K1 < K2 lies inside the one for K2."""
    mk = o.masking
    a = mk.indices(4, 1, 0, 8, 256, 12)
    b = mk.indices(4, 1, 0, 8, 256, 40)
    for r in range(8):
        assert set(a[r]).issubset(set(b[r]))


def pin_mask_uniform(o):
    """Over many tokens each dimension is kept with frequency K/H and each pair of
    dimensions with K(K-1)/(H(H-1)) (uniform random K-subsets)."""
    mk = o.masking
    T, H, K = 20000, 32, 8
    m = mk.mask(mk.indices(1, 2, 3, T, H, K), H).astype(np.float64)
    e = T * K / H
    chi2 = (((m.sum(axis=0) - e) ** 2) / e).sum()
    assert chi2 < 75.0, chi2  # 31 degrees of freedom: far beyond the 99.99% point
    co = (m.T @ m) / T
    off = co[~np.eye(H, dtype=bool)]
    assert abs(off.mean() - K * (K - 1) / (H * (H - 1))) < 2e-3


def pin_mask_keys(o):
    """The mask depends on the layer, the step, the batch and the token, and on nothing
    else: equal keys give equal masks, any changed key a different one."""
    mk = o.masking
    base = mk.indices(3, 5, 7, 4, 128, 20)
    assert np.array_equal(base, mk.indices(3, 5, 7, 4, 128, 20))
    for other in [(4, 5, 7), (3, 6, 7), (3, 5, 8)]:
        assert not np.array_equal(base, mk.indices(*other, 4, 128, 20))
    assert not np.array_equal(base[0], base[1])
    # the same token under a longer sequence keeps the same dimensions
    assert np.array_equal(base, mk.indices(3, 5, 7, 9, 128, 20, rows=range(4)))


def pin_mask_pack_unpack(o):
    """pack keeps the K values of each token in ascending dimension order; unpack puts
    them back with zeros elsewhere: unpack(pack(x)) = x * m and pack(unpack(v)) = v."""
    mk = o.masking
    x = _rand(11, 6, 50)
    idx = mk.indices(0, 0, 0, 6, 50, 13)
    m = mk.mask(idx, 50)
    assert (m.sum(axis=1) == 13).all()
    v = mk.pack(x, idx)
    assert v.shape == (6, 13)
    for r in range(6):
        assert np.array_equal(v[r], x[r][np.flatnonzero(m[r])])
    assert np.array_equal(mk.unpack(v, idx, 50), x * m)
    assert np.array_equal(mk.pack(mk.unpack(v, idx, 50), idx), v)


def pin_mask_gradient(o):
    """The mask is an element-wise product in the graph ("Key design 1" gradient
    equation): torch's gradient of h -> h * m, formed by gather and scatter, is the
    upstream gradient times m, which is unpack(pack(upstream)) with the same indices."""
    import torch
    mk = o.masking
    idx = mk.indices(6, 2, 1, 4, 12, 5)
    x = torch.tensor(_rand(12, 4, 12), requires_grad=True)
    ti = torch.tensor(idx, dtype=torch.int64)
    y = torch.zeros_like(x).scatter(1, ti, x.gather(1, ti))
    g = _rand(13, 4, 12)
    y.backward(torch.tensor(g))
    got = x.grad.numpy()
    assert np.array_equal(got, g * mk.mask(idx, 12))
    assert np.array_equal(got, mk.unpack(mk.pack(g, idx), idx, 12))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
