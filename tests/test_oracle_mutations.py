"""Plant plausible mistakes in the CPU oracle and check that the pins catch each.

Every mutation replaces one oracle function by a subtly wrong variant (a
dropped term, a wrong sign or index, a transposed operand, a swapped
coefficient) for the duration of one test; at least one pin of
tests/oracle_pins.py must then fail.
"""
import numpy as np
import pytest

from tests import oracle_pins


def _project_one_sided(U, d, V, G):
    X = (U.T @ G) @ V
    return (U @ (d[:, None] * X)) @ V.T


def _project_transposed_x(U, d, V, G):
    X = (U.T @ G) @ V
    Xf = d[:, None] * X * d[None, :]
    return (U @ Xf.T) @ V.T


def _project_no_filter(U, d, V, G):
    return (U @ ((U.T @ G) @ V)) @ V.T


def _project_d_linear(U, d, V, G):
    X = (U.T @ G) @ V
    sd = np.sqrt(d)
    return (U @ (sd[:, None] * X * sd[None, :])) @ V.T


def _tikhonov_inverted(s, tau):
    s = np.asarray(s, np.float64)
    den = s + tau
    out = np.zeros_like(s)
    nz = den != 0
    out[nz] = tau / den[nz]
    return out


def _tikhonov_double_tau(s, tau):
    s = np.asarray(s, np.float64)
    den = s + 2 * tau
    out = np.zeros_like(s)
    nz = den != 0
    out[nz] = s[nz] / den[nz]
    return out


def _combine_swapped(G, Gf, alpha):
    return (1 - alpha) * np.asarray(G) + alpha * np.asarray(Gf)


def _adamw_no_bias_correction(W, m, v, g, t, lr, b1, b2, eps, wd):
    W = np.asarray(W, np.float64)
    m = b1 * m + (1 - b1) * g
    v = b2 * v + (1 - b2) * g * g
    return W - lr * wd * W - lr * m / (np.sqrt(v) + eps), m, v


def _adamw_unscaled_decay(W, m, v, g, t, lr, b1, b2, eps, wd):
    W = np.asarray(W, np.float64)
    m = b1 * m + (1 - b1) * g
    v = b2 * v + (1 - b2) * g * g
    mh, vh = m / (1 - b1 ** t), v / (1 - b2 ** t)
    return W - wd * W - lr * mh / (np.sqrt(vh) + eps), m, v


def _adamw_eps_inside(W, m, v, g, t, lr, b1, b2, eps, wd):
    W = np.asarray(W, np.float64)
    m = b1 * m + (1 - b1) * g
    v = b2 * v + (1 - b2) * g * g
    mh, vh = m / (1 - b1 ** t), v / (1 - b2 ** t)
    return W - lr * wd * W - lr * mh / np.sqrt(vh + eps), m, v


def _adamw_swapped_betas(W, m, v, g, t, lr, b1, b2, eps, wd):
    W = np.asarray(W, np.float64)
    m = b2 * m + (1 - b2) * g
    v = b1 * v + (1 - b1) * g * g
    mh, vh = m / (1 - b2 ** t), v / (1 - b1 ** t)
    return W - lr * wd * W - lr * mh / (np.sqrt(vh) + eps), m, v


def _ema_swapped(M, G, beta):
    return (1 - beta) * np.asarray(M, np.float64) + beta * np.asarray(G, np.float64)


MUTATIONS = {
    "project_one_sided_d": ("project", _project_one_sided),
    "project_transposed_x": ("project", _project_transposed_x),
    "project_no_filter": ("project", _project_no_filter),
    "project_sqrt_d": ("project", _project_d_linear),
    "tikhonov_inverted": ("tikhonov", _tikhonov_inverted),
    "tikhonov_double_tau": ("tikhonov", _tikhonov_double_tau),
    "combine_swapped": ("combine", _combine_swapped),
    "adamw_no_bias_correction": ("adamw", _adamw_no_bias_correction),
    "adamw_unscaled_decay": ("adamw", _adamw_unscaled_decay),
    "adamw_eps_inside_sqrt": ("adamw", _adamw_eps_inside),
    "adamw_swapped_betas": ("adamw", _adamw_swapped_betas),
    "ema_swapped": ("ema", _ema_swapped),
}


def _svd_swapped_factors(orig):
    def f(M, max_sweeps=100, threads=None):
        U, s, V, sw = orig(M, max_sweeps, threads)
        if U.shape[1] == V.shape[0] == V.shape[1] == U.shape[0]:
            return V, s, U, sw
        return U[::-1].copy(), s, V, sw  # reversed row index
    return f


def _svd_unsorted_vectors(orig):
    def f(M, max_sweeps=100, threads=None):
        U, s, V, sw = orig(M, max_sweeps, threads)
        return U, s[::-1].copy(), V, sw  # values no longer paired with their vectors
    return f


WRAPPERS = {"svd_swapped_or_reversed": _svd_swapped_factors, "svd_unpaired_values": _svd_unsorted_vectors}


def _pins_fail(o):
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, oracle_mod, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(oracle_mod, attr, fn)
    assert _pins_fail(oracle_mod), f"mutation {name} passed every pin"


@pytest.mark.parametrize("name", sorted(WRAPPERS))
def test_svd_mutation_is_caught(name, oracle_mod, monkeypatch):
    monkeypatch.setattr(oracle_mod, "svd", WRAPPERS[name](oracle_mod.svd))
    assert _pins_fail(oracle_mod), f"mutation {name} passed every pin"


# ---- the stateful driver (oracle.Optimizer): call sites and storage rounding -------

def _driver_mutations(o):
    """Plausible mistakes in how ``Optimizer`` chains the steps, each as
    (method name, replacement)."""
    Opt = o.Optimizer
    step_orig = Opt.step

    def anchor_swapped(self, G_anc_list, defer_refresh=False):
        for i, G in enumerate(G_anc_list):
            self.M[i] = o.round_storage(o.ema(G, self.M[i], self.hp["beta_anc"]), self.state_dtype)
            if defer_refresh:
                self.factors[i] = None
            else:
                self._refresh(i)

    def anchor_no_refresh(self, G_anc_list, defer_refresh=False):
        for i, G in enumerate(G_anc_list):
            self.M[i] = o.round_storage(o.ema(self.M[i], G, self.hp["beta_anc"]), self.state_dtype)
            if self.factors[i] is None:
                self._refresh(i)

    def anchor_not_rounded(self, G_anc_list, defer_refresh=False):
        for i, G in enumerate(G_anc_list):
            self.M[i] = o.ema(self.M[i], G, self.hp["beta_anc"])
            if defer_refresh:
                self.factors[i] = None
            else:
                self._refresh(i)

    def anchor_defer_keeps_factors(self, G_anc_list, defer_refresh=False):
        for i, G in enumerate(G_anc_list):
            self.M[i] = o.round_storage(o.ema(self.M[i], G, self.hp["beta_anc"]), self.state_dtype)
            if not defer_refresh or self.factors[i] is None:
                self._refresh(i)

    def anchor_advances_t(self, G_anc_list, defer_refresh=False):
        self.t += 1
        for i, G in enumerate(G_anc_list):
            self.M[i] = o.round_storage(o.ema(self.M[i], G, self.hp["beta_anc"]), self.state_dtype)
            if defer_refresh:
                self.factors[i] = None
            else:
                self._refresh(i)

    def _step_variant(skip):
        def step(self, W_list, G_mask_list):
            hp = self.hp
            self.t += 1
            out = []
            for i, (W, G) in enumerate(zip(W_list, G_mask_list)):
                if self.factors[i] is None:
                    self._refresh(i)
                U, s, V = self.factors[i]
                G = np.asarray(G, np.float64)
                G_filt = o.project(U, self.d[i], V, G)
                G_proj = o.combine(G, G_filt, hp["alpha"])
                W_new, m_new, v_new = o.adamw(W, self.m[i], self.v[i], G_proj, self.t, hp["lr"],
                                              hp["beta1"], hp["beta2"], hp["eps"],
                                              hp["weight_decay"])
                self.m[i] = m_new if skip == "m" else o.round_storage(m_new, self.state_dtype)
                self.v[i] = v_new if skip == "v" else o.round_storage(v_new, self.state_dtype)
                if skip != "W":
                    W_new = o.round_storage(W_new, self.w_dtype)
                self.last_filt[i] = G_filt
                self.last_proj[i] = G_proj
                out.append(W_new)
            return out
        return step

    assert step_orig is not None
    return {
        "driver_ema_args_swapped": ("anchor_update", anchor_swapped),
        "driver_anchor_keeps_old_factors": ("anchor_update", anchor_no_refresh),
        "driver_anchor_momentum_not_rounded": ("anchor_update", anchor_not_rounded),
        "driver_anchor_advances_step_count": ("anchor_update", anchor_advances_t),
        "driver_deferred_refresh_keeps_factors": ("anchor_update", anchor_defer_keeps_factors),
        "driver_m_not_rounded": ("step", _step_variant("m")),
        "driver_v_not_rounded": ("step", _step_variant("v")),
        "driver_w_not_rounded": ("step", _step_variant("W")),
    }


DRIVER_MUTATIONS = ["driver_anchor_advances_step_count", "driver_anchor_keeps_old_factors",
                    "driver_deferred_refresh_keeps_factors",
                    "driver_anchor_momentum_not_rounded", "driver_ema_args_swapped",
                    "driver_m_not_rounded", "driver_v_not_rounded", "driver_w_not_rounded"]


@pytest.mark.parametrize("name", DRIVER_MUTATIONS)
def test_driver_mutation_is_caught(name, oracle_mod, monkeypatch):
    attr, fn = _driver_mutations(oracle_mod)[name]
    monkeypatch.setattr(oracle_mod.Optimizer, attr, fn)
    assert _pins_fail(oracle_mod), f"mutation {name} passed every pin"


def test_driver_mutation_list_is_complete(oracle_mod):
    assert sorted(_driver_mutations(oracle_mod)) == sorted(DRIVER_MUTATIONS)


# ---- the in-graph activation mask ------------------------------------------------

def _mask_mutations(mk):
    """Plausible mistakes in oracle/masking.py, each as (attribute, replacement)."""
    def keep_count_floor(H, p):
        return int(np.floor((1.0 - p) * H))

    def indices_coarse_hash(layer, step, batch, T, H, K, rows=None):
        # ranks by the top 4 bits only: ties go to low dimensions, a biased subset
        u = mk.hashes(mk.seed_of(layer, step, batch), T, H, rows) >> np.uint64(60)
        out = np.empty((u.shape[0], K), dtype=np.int32)
        j = np.arange(H)
        for r in range(u.shape[0]):
            out[r] = np.sort(np.lexsort((j, u[r]))[:K])
        return out

    def indices_unsorted(layer, step, batch, T, H, K, rows=None):
        u = mk.hashes(mk.seed_of(layer, step, batch), T, H, rows)
        out = np.empty((u.shape[0], K), dtype=np.int32)
        j = np.arange(H)
        for r in range(u.shape[0]):
            out[r] = np.lexsort((j, u[r]))[:K]  # kept in hash order, not dimension order
        return out

    seed_of = mk.seed_of if mk is not None else None

    def seed_without_layer(layer, step, batch):
        return seed_of(0, step, batch)

    def mix64_no_second_shift(z):
        z = np.asarray(z, dtype=np.uint64)
        with np.errstate(over="ignore"):
            z = (z ^ (z >> np.uint64(30))) * np.uint64(mk.M1)
            z = z * np.uint64(mk.M2)
        return z ^ (z >> np.uint64(31))

    def unpack_shifted(v, idx, H):
        out = np.zeros((v.shape[0], H), dtype=np.asarray(v).dtype)
        np.put_along_axis(out, np.minimum(idx.astype(np.int64) + 1, H - 1), v, axis=1)
        return out

    return {
        "mask_keep_count_floor": ("keep_count", keep_count_floor),
        "mask_coarse_hash": ("indices", indices_coarse_hash),
        "mask_unsorted_pack_order": ("indices", indices_unsorted),
        "mask_seed_without_layer": ("seed_of", seed_without_layer),
        "mask_mixer_step_dropped": ("mix64", mix64_no_second_shift),
        "mask_unpack_off_by_one": ("unpack", unpack_shifted),
    }


MASK_MUTATIONS = sorted(_mask_mutations(None).keys())


@pytest.mark.parametrize("name", MASK_MUTATIONS)
def test_mask_mutation_is_caught(name, oracle_mod, monkeypatch):
    attr, fn = _mask_mutations(oracle_mod.masking)[name]
    monkeypatch.setattr(oracle_mod.masking, attr, fn)
    assert _pins_fail(oracle_mod), f"mutation {name} passed every pin"
