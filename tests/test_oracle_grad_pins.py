"""Pins of the oracle's gradients (``oracle.backward``) against facts other than itself.

* Central finite differences of the forward oracle, for every element of every input of
  every differentiable variant: a dropped term, a wrong sign or a transposed operand in
  the reverse sweep moves at least one entry by far more than the difference error.
* Causal linear attention (erase gate 0, write gate 1, no decay, zero initial state),
  o = scale tril(Q K^T) V, whose gradients are textbook matrix calculus:
  dV = scale tril(Q K^T)^T dO, dQ = tril(scale dO V^T) K, dK = tril(scale dO V^T)^T Q.
"""
import numpy as np
import pytest

import oracle as O

GRAD_VARIANTS = ["plain", "gdn", "gdn2", "explicit", "gdn2_decay", "kda", "kda_gdn2"]


def tiny_stream(variant, T=5, Dk=3, Dv=2, seed=0):
    """One stream of random inputs in the ranges the workloads use (gains in (0, 1),
    log decays < 0)."""
    rng = np.random.default_rng(seed)
    x = {"q": rng.standard_normal((T, Dk)), "k": rng.standard_normal((T, Dk)) / np.sqrt(Dk),
         "v": rng.standard_normal((T, Dv))}
    if variant in ("gdn2", "gdn2_decay", "kda_gdn2"):
        x["erase"] = rng.uniform(0.2, 0.9, (T, Dk))
        x["write"] = rng.uniform(0.2, 0.9, (T, Dv))
    else:
        x["beta"] = rng.uniform(0.2, 0.9, T)
    if variant in ("gdn", "explicit", "gdn2_decay"):
        x["log_alpha"] = -rng.uniform(0.05, 0.5, T)
    if variant in ("kda", "kda_gdn2"):
        x["log_alpha"] = -rng.uniform(0.05, 0.5, (T, Dk))
    if variant == "explicit":
        x["write_key"] = rng.standard_normal((T, Dk)) / np.sqrt(Dk)
    S0 = rng.standard_normal((Dv, Dk))
    dO = rng.standard_normal((T, Dv))
    dST = rng.standard_normal((Dv, Dk))
    return x, S0, dO, dST


def _loss(x, S0, dO, dST, scale):
    o, S, _ = O.recurrent_stream(x, scale=scale, S0=S0)
    return float(np.sum(o * dO) + np.sum(S * dST))


@pytest.mark.parametrize("variant", GRAD_VARIANTS)
def test_gradients_match_central_differences(variant):
    x, S0, dO, dST = tiny_stream(variant, seed=GRAD_VARIANTS.index(variant))
    scale = 0.7
    g = O.recurrent_stream_grad(x, dO, dST, scale=scale, S0=S0)
    names = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "erase": "derase",
             "write": "dwrite", "log_alpha": "dlog_alpha", "write_key": "dwrite_key"}
    h = 1e-6
    checked = 0
    for key, gname in list(names.items()) + [("S0", "dS0")]:
        base = S0 if key == "S0" else x.get(key)
        if base is None:
            assert gname not in g, gname
            continue
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            vals = []
            for sgn in (1.0, -1.0):
                pert = base.copy()
                pert[idx] += sgn * h
                if key == "S0":
                    vals.append(_loss(x, pert, dO, dST, scale))
                else:
                    vals.append(_loss({**x, key: pert}, S0, dO, dST, scale))
            fd[idx] = (vals[0] - vals[1]) / (2 * h)
        err = np.max(np.abs(g[gname] - fd))
        assert err <= 1e-7 * (1.0 + np.max(np.abs(fd))), (gname, err)
        checked += 1
    assert checked >= 5


@pytest.mark.parametrize("variant", ["gdn", "kda_gdn2"])
def test_checkpointed_sweep_is_the_same(variant):
    x, S0, dO, dST = tiny_stream(variant, T=23, Dk=4, Dv=3, seed=5)
    a = O.recurrent_stream_grad(x, dO, dST, S0=S0)
    b = O.recurrent_stream_grad(x, dO, dST, S0=S0, checkpoint=4)
    assert a.keys() == b.keys()
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_linear_attention_gradients_are_textbook():
    rng = np.random.default_rng(11)
    T, Dk, Dv, scale = 9, 4, 3, 0.5
    Q, K, V = rng.standard_normal((T, Dk)), rng.standard_normal((T, Dk)), rng.standard_normal((T, Dv))
    x = {"q": Q, "k": K, "v": V, "erase": np.zeros((T, Dk)), "write": np.ones((T, Dv))}
    dO = rng.standard_normal((T, Dv))
    g = O.recurrent_stream_grad(x, dO, None, scale=scale)
    M = np.tril(Q @ K.T)
    dM = np.tril(scale * dO @ V.T)
    np.testing.assert_allclose(g["dv"], scale * M.T @ dO, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dq"], dM @ K, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dk"], dM.T @ Q, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dS0"], scale * dO.T @ Q, rtol=1e-12, atol=1e-12)


def test_batched_wrapper_places_streams():
    rng = np.random.default_rng(2)
    B, T, H, Dk, Dv = 2, 6, 3, 3, 2
    x = {"q": rng.standard_normal((B, T, H, Dk)), "k": rng.standard_normal((B, T, H, Dk)),
         "v": rng.standard_normal((B, T, H, Dv)), "beta": rng.uniform(0, 1, (B, T, H)),
         "log_alpha": -rng.uniform(0, 1, (B, T, H))}
    dO = rng.standard_normal((B, T, H, Dv))
    g = O.recurrent_grad(x, dO, None, streams=[(1, 2)])
    one = O.recurrent_stream_grad({k: v[1, :, 2] for k, v in x.items()}, dO[1, :, 2])
    np.testing.assert_array_equal(g["dk"][1, :, 2], one["dk"])
    np.testing.assert_array_equal(g["dlog_alpha"][1, :, 2], one["dlog_alpha"])
    np.testing.assert_array_equal(g["dS0"][1, 2], one["dS0"])
    assert np.all(g["dk"][0] == 0) and np.all(g["dS0"][1, 1] == 0)


PRECOND_VARIANTS = ["gdn", "gdn2", "kda", "plain"]


@pytest.mark.parametrize("variant", PRECOND_VARIANTS)
def test_preconditioner_gradients_match_central_differences(variant):
    """The diagonal preconditioner on the write key (r_t = k_t (.) p_t): dk through both the
    erase and the write key, and dL/dh_init, against central differences of the forward."""
    x, S0, dO, dST = tiny_stream(variant, T=6, seed=40 + PRECOND_VARIANTS.index(variant))
    rng = np.random.default_rng(7)
    pre = dict(rho=0.8, eps=0.1, h_init=rng.uniform(0.1, 0.6, x["k"].shape[1]), t0=3)
    scale = 0.9

    def loss(xx, h_init):
        o, S, _ = O.recurrent_stream(xx, scale=scale, S0=S0, precond=dict(pre, h_init=h_init))
        return float(np.sum(o * dO) + np.sum(S * dST))

    g = O.recurrent_stream_grad(x, dO, dST, scale=scale, S0=S0, precond=pre)
    assert "dwrite_key" not in g
    h = 1e-6
    for key, gname in [("k", "dk"), ("q", "dq"), ("h_init", "dpc_h_init")]:
        base = pre["h_init"] if key == "h_init" else x[key]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            vals = []
            for sgn in (1.0, -1.0):
                pert = base.copy()
                pert[idx] += sgn * h
                vals.append(loss(x, pert) if key == "h_init" else loss({**x, key: pert}, pre["h_init"]))
            fd[idx] = (vals[0] - vals[1]) / (2 * h)
        err = np.max(np.abs(g[gname] - fd))
        assert err <= 1e-7 * (1.0 + np.max(np.abs(fd))), (gname, err)


def test_preconditioner_gradient_of_a_constant_accumulator():
    """rho -> 0 with a zero initial accumulator: p_t = 1 / (k_t^2 + eps) elementwise, so
    r_t = k_t / (k_t^2 + eps) and dr/dk = (eps - k^2) / (k^2 + eps)^2: the chain rule
    reduces to that closed form (rho = 1e-300 leaves the accumulator the current key's
    square to fp64 precision)."""
    rng = np.random.default_rng(3)
    k = rng.standard_normal((5, 4))
    dr = rng.standard_normal((5, 4))
    eps = 0.3
    dk, dh0 = O.precond_grad(k, dr, 1e-300, eps, np.zeros(4), 0)
    np.testing.assert_allclose(dk, dr * (eps - k * k) / (k * k + eps) ** 2, rtol=1e-12, atol=1e-14)
    assert np.all(np.abs(dh0) < 1e-250)


BAND_VARIANTS = ["gdn", "gdn2_decay", "explicit", "plain"]


@pytest.mark.parametrize("variant", BAND_VARIANTS)
def test_chunk_form_gradient_with_exact_t_is_the_recurrence_gradient(variant):
    """band >= C - 1 keeps all of T: the chunk-form gradient equals the reverse sweep of the
    recurrence (two independent derivations)."""
    x, S0, dO, dST = tiny_stream(variant, T=13, Dk=4, Dv=3, seed=60 + BAND_VARIANTS.index(variant))
    a = O.recurrent_stream_grad(x, dO, dST, scale=0.6, S0=S0)
    b = O.chunked_stream_grad(x, dO, dST, chunk=5, band=4, scale=0.6, S0=S0)
    assert a.keys() == b.keys()
    for key in a:
        np.testing.assert_allclose(b[key], a[key], rtol=1e-10, atol=1e-11, err_msg=key)


@pytest.mark.parametrize("band", [0, 1, 2])
@pytest.mark.parametrize("variant", BAND_VARIANTS)
def test_band_gradients_match_central_differences(variant, band):
    """The band-limited T (t_mode ("neumann", band)): every input's gradient against central
    differences of the oracle's chunk form, a ragged last chunk included."""
    x, S0, dO, dST = tiny_stream(variant, T=11, Dk=3, Dv=2, seed=70 + band)
    scale, C = 0.8, 4

    def loss(xx, s0):
        o, S, _ = O.chunked_stream(xx, chunk=C, t_mode=("neumann", band), scale=scale, S0=s0)
        return float(np.sum(o * dO) + np.sum(S * dST))

    g = O.chunked_stream_grad(x, dO, dST, chunk=C, band=band, scale=scale, S0=S0)
    names = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "erase": "derase",
             "write": "dwrite", "log_alpha": "dlog_alpha", "write_key": "dwrite_key"}
    h = 1e-6
    for key, gname in list(names.items()) + [("S0", "dS0")]:
        base = S0 if key == "S0" else x.get(key)
        if base is None:
            continue
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            vals = []
            for sgn in (1.0, -1.0):
                pert = base.copy()
                pert[idx] += sgn * h
                vals.append(loss(x, pert) if key == "S0" else loss({**x, key: pert}, S0))
            fd[idx] = (vals[0] - vals[1]) / (2 * h)
        err = np.max(np.abs(g[gname] - fd))
        assert err <= 1e-7 * (1.0 + np.max(np.abs(fd))), (gname, err)


def test_band_gradient_differs_from_the_recurrence_gradient():
    """A narrow band is a different function: its gradient is not the recurrence's."""
    x, S0, dO, dST = tiny_stream("gdn", T=12, Dk=4, Dv=3, seed=80)
    a = O.recurrent_stream_grad(x, dO, dST, S0=S0)
    b = O.chunked_stream_grad(x, dO, dST, chunk=6, band=1, S0=S0)
    assert O.rel_l2(b["dk"], a["dk"]) > 1e-3
