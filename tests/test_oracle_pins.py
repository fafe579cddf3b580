"""Pins of the fp64 CPU oracle against facts other than itself.

Each test ties the oracle to an exact-rational brute force, a hand-worked example, a
closed form, a textbook special case or an identity stated on the pages, so that a
dropped term, a wrong sign or index, or a transposed operand fails at least one.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import gdr_synth as gs
import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)

VARIANTS = ["plain", "gdn", "gdn2", "pdn", "explicit", "gdn2_decay", "pdn_decay", "kda", "kda_gdn2"]


def small_inputs(variant, B=1, H=2, T=70, Dk=8, Dv=6, seed=7):
    base = {"plain": "plain", "gdn": "gdn", "gdn2": "gdn2", "pdn": "pdn", "explicit": "gdn",
            "gdn2_decay": "gdn2", "pdn_decay": "pdn", "kda": "kda", "kda_gdn2": "gdn2"}[variant]
    over = dict(B=B, H=H, T=T, Dk=Dk, Dv=Dv, seed=seed, dtype="f32")
    if variant == "kda_gdn2":
        over["decay"] = "channel"
    if variant == "explicit":
        over["wkey"] = "explicit"
    if variant.endswith("_decay"):
        over["decay"] = "scalar"
    s = gs.spec(base, **over)
    x = gs.make_inputs(s)
    pc = dict(rho=0.99, eps=1e-3, h0=1.0, t0=0) if s.wkey == "precond" else None
    return s, x, pc


# ----------------------------------------------------------------------------------
# Exact-rational brute force: explicit d x d transition products.
# ----------------------------------------------------------------------------------

def _fr(a):
    return [[Fraction(x) for x in row] for row in a]


def _matmul(A, B):
    return [[sum((A[i][l] * B[l][j] for l in range(len(B))), Fraction(0)) for j in range(len(B[0]))]
            for i in range(len(A))]


def _brute(q, k, v, alpha, e, r, vp, S0):
    """S_t = S_{t-1} M_t + v'_t r_t^T with M_t = Diag(a_t) (I - e_t r_t^T); o_t = S_t q_t.
    ``alpha[t]`` is a scalar (a_t = alpha_t 1) or a list of Dk per-channel decays."""
    Dk = len(k[0])
    S = [row[:] for row in S0]
    outs, Ms = [], []
    for t in range(len(q)):
        a = alpha[t] if isinstance(alpha[t], list) else [alpha[t]] * Dk
        M = [[a[i] * ((1 if i == j else 0) - e[t][i] * r[t][j]) for j in range(Dk)] for i in range(Dk)]
        Ms.append(M)
        S = _matmul(S, M)
        S = [[S[a][j] + vp[t][a] * r[t][j] for j in range(Dk)] for a in range(len(S))]
        outs.append([sum((S[a][j] * q[t][j] for j in range(Dk)), Fraction(0)) for a in range(len(S))])
    return outs, S, Ms


def _rat(rng, shape, den=8):
    return [[Fraction(int(rng.integers(-den, den + 1)), den) for _ in range(shape[1])] for _ in range(shape[0])]


@pytest.mark.parametrize("variant", ["plain", "gated", "channel", "precond", "explicit", "diag"])
def test_brute_force_exact_rationals(variant):
    rng = np.random.default_rng(99 + len(variant))
    T, Dk, Dv = 6, 3, 2
    q, k, v = _rat(rng, (T, Dk)), _rat(rng, (T, Dk)), _rat(rng, (T, Dv))
    beta = [Fraction(int(rng.integers(1, 8)), 8) for _ in range(T)]
    alpha = [Fraction(1)] * T
    if variant == "gated":
        alpha = [Fraction(int(rng.integers(4, 9)), 8) for _ in range(T)]
    if variant == "diag":   # one decay per key channel
        alpha = [[Fraction(int(rng.integers(2, 9)), 8) for _ in range(Dk)] for _ in range(T)]
    S0 = _rat(rng, (Dv, Dk), den=4)
    x = {"q": np.array(q, float), "k": np.array(k, float), "v": np.array(v, float)}
    precond = None
    if variant == "channel":
        b = [[Fraction(int(rng.integers(0, 9)), 8) for _ in range(Dk)] for _ in range(T)]
        w = [[Fraction(int(rng.integers(0, 9)), 8) for _ in range(Dv)] for _ in range(T)]
        e = [[b[t][i] * k[t][i] for i in range(Dk)] for t in range(T)]
        r = k
        vp = [[w[t][i] * v[t][i] for i in range(Dv)] for t in range(T)]
        x["erase"], x["write"] = np.array(b, float), np.array(w, float)
    else:
        e = [[beta[t] * k[t][i] for i in range(Dk)] for t in range(T)]
        vp = [[beta[t] * v[t][i] for i in range(Dv)] for t in range(T)]
        x["beta"] = np.array(beta, float)
        r = k
        if variant == "precond":
            rho, eps, h0, t0 = Fraction(99, 100), Fraction(1, 1000), Fraction(1), 3
            h = [h0] * Dk
            r = []
            for t in range(T):
                h = [rho * h[i] + k[t][i] * k[t][i] for i in range(Dk)]
                corr = 1 - rho ** (t0 + t + 1)
                r.append([k[t][i] / (h[i] / corr + eps) for i in range(Dk)])
            precond = dict(rho=0.99, eps=1e-3, h_init=np.full(Dk, 1.0), t0=t0)
        elif variant == "explicit":
            r = _rat(rng, (T, Dk), den=4)
            x["write_key"] = np.array(r, float)
    if variant == "gated":
        x["log_alpha"] = np.log(np.array([float(a) for a in alpha]))
    if variant == "diag":
        x["log_alpha"] = np.log(np.array([[float(a) for a in row] for row in alpha]))
    outs, S_T, Ms = _brute(q, k, v, alpha, e, r, vp, S0)

    # the unrolled sum: S_T = S_0 prod_t M_t + sum_t v'_t r_t^T prod_{s>t} M_s
    def prod(ms):
        P = [[Fraction(int(i == j)) for j in range(Dk)] for i in range(Dk)]
        for M in ms:
            P = _matmul(P, M)
        return P
    U = _matmul(S0, prod(Ms))
    for t in range(T):
        term = _matmul([[vp[t][a] * r[t][j] for j in range(Dk)] for a in range(Dv)], prod(Ms[t + 1:]))
        U = [[U[a][j] + term[a][j] for j in range(Dk)] for a in range(Dv)]
    assert U == S_T

    o_ref = np.array([[float(z) for z in row] for row in outs])
    S_ref = np.array([[float(z) for z in row] for row in S_T])
    for fn, kw in [(O.recurrent_stream, {}), (O.chunked_stream, {"chunk": 2}),
                   (O.chunked_stream, {"chunk": 4})]:
        o, S, _ = fn(x, S0=np.array(S0, float), precond=precond, **kw)
        np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-12)


def test_hand_worked_golden():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_d2.json")))
    for case in g["cases"]:
        x = {k: np.array(v, float) for k, v in g["inputs"].items()}
        x["log_alpha"] = np.log(np.array(case["alpha"]))
        o, S, _ = O.recurrent_stream(x)
        np.testing.assert_allclose(o, case["o"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(S, case["S"], rtol=0, atol=1e-14)
        o2, S2, _ = O.chunked_stream(x, chunk=2)
        np.testing.assert_allclose(o2, case["o"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(S2, case["S"], rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------------
# Closed forms and special cases.
# ----------------------------------------------------------------------------------

def test_single_token_closed_form():
    """T = 1 from S_0 = 0: o_1 = beta (k . scale q) v  (decay has nothing to act on)."""
    Dk, Dv = 5, 4
    q, k, v = RNG.standard_normal((1, Dk)), RNG.standard_normal((1, Dk)), RNG.standard_normal((1, Dv))
    beta, la, scale = np.array([0.3]), np.array([-0.7]), 0.5
    o, S, _ = O.recurrent_stream({"q": q, "k": k, "v": v, "beta": beta, "log_alpha": la}, scale=scale)
    np.testing.assert_allclose(o[0], beta[0] * scale * (k[0] @ q[0]) * v[0], rtol=1e-14)
    np.testing.assert_allclose(S, beta[0] * np.outer(v[0], k[0]), rtol=1e-14)


@pytest.mark.parametrize("form", ["recurrent", "chunked"])
def test_zero_gain_is_pure_decay(form):
    """beta = 0: S_t = (prod alpha) S_0 and o_t = e^{g_t} S_0 q_t."""
    T, Dk, Dv = 37, 6, 5
    x = {"q": RNG.standard_normal((T, Dk)), "k": RNG.standard_normal((T, Dk)),
         "v": RNG.standard_normal((T, Dv)), "beta": np.zeros(T),
         "log_alpha": -0.2 * RNG.random(T)}
    S0 = RNG.standard_normal((Dv, Dk))
    fn = O.recurrent_stream if form == "recurrent" else (lambda x, **kw: O.chunked_stream(x, chunk=8, **kw))
    o, S, _ = fn(x, S0=S0)
    g = np.cumsum(x["log_alpha"])
    np.testing.assert_allclose(S, np.exp(g[-1]) * S0, rtol=1e-13)
    np.testing.assert_allclose(o, np.exp(g)[:, None] * (x["q"] @ S0.T), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("form", ["recurrent", "chunked"])
def test_equal_channel_decays_are_the_scalar_decay(form):
    """A per-channel decay with every channel equal to log alpha_t is the scalar-gated rule."""
    s, x, _ = small_inputs("gdn", T=45)
    xc = dict(x, log_alpha=np.repeat(x["log_alpha"][..., None], s.Dk, axis=-1))
    S0 = RNG.standard_normal((s.B, s.H, s.Dv, s.Dk)) * 0.3
    f = O.recurrent if form == "recurrent" else (lambda x, **kw: O.chunked(x, chunk=16, **kw))
    o1, S1, _ = f(x, state0=S0)
    o2, S2, _ = f(xc, state0=S0)
    assert O.rel_l2(o2, o1) < 1e-13 and O.rel_l2(S2, S1) < 1e-13


@pytest.mark.parametrize("form", ["recurrent", "chunked"])
def test_zero_gain_is_pure_channel_decay(form):
    """beta = 0 with per-channel decays: S_t = S_0 Diag(exp(G_t)) and o_t = S_0 (exp(G_t) (.) q_t),
    G the cumulative log decay of each channel."""
    T, Dk, Dv = 29, 6, 5
    x = {"q": RNG.standard_normal((T, Dk)), "k": RNG.standard_normal((T, Dk)),
         "v": RNG.standard_normal((T, Dv)), "beta": np.zeros(T),
         "log_alpha": -0.3 * RNG.random((T, Dk))}
    S0 = RNG.standard_normal((Dv, Dk))
    fn = O.recurrent_stream if form == "recurrent" else (lambda x, **kw: O.chunked_stream(x, chunk=8, **kw))
    o, S, _ = fn(x, S0=S0)
    G = np.cumsum(x["log_alpha"], axis=0)
    np.testing.assert_allclose(S, S0 * np.exp(G[-1])[None, :], rtol=1e-13)
    np.testing.assert_allclose(o, (np.exp(G) * x["q"]) @ S0.T, rtol=1e-12, atol=1e-14)


def test_orthonormal_keys_exact_retrieval():
    """beta = 1, alpha = 1, S_0 = 0, orthonormal keys: S k_j = v_j; a rewritten key keeps
    only its latest value (the delta rule replaces, linear attention would add)."""
    d, Dv = 16, 7
    Qm, _ = np.linalg.qr(RNG.standard_normal((d, d)))
    keys = Qm.T                               # rows orthonormal
    order = list(range(d)) + [3, 9]           # keys 3 and 9 are written twice
    vals = RNG.standard_normal((len(order), Dv))
    x = {"q": keys[order], "k": keys[order], "v": vals, "beta": np.ones(len(order))}
    o, S, _ = O.recurrent_stream(x)
    latest = {kj: vals[t] for t, kj in enumerate(order)}
    for j in range(d):
        np.testing.assert_allclose(S @ keys[j], latest[j], atol=1e-12)
    # reading key t right after writing it returns its value
    np.testing.assert_allclose(o, vals, atol=1e-12)
    oc, Sc, _ = O.chunked_stream(x, chunk=4)
    np.testing.assert_allclose(Sc, S, atol=1e-12)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("chunk", [1, 2, 4, 8, 16, 32, 64, 128])
def test_chunked_equals_recurrent(variant, chunk):
    """The chunk form reaches the recurrence exactly (up to rounding), any chunk size,
    ragged tail, non-zero initial state."""
    s, x, pc = small_inputs(variant, T=70)
    S0 = RNG.standard_normal((s.B, s.H, s.Dv, s.Dk)) * 0.3
    if pc is not None:
        pc = dict(pc, h_init=1.0 + RNG.random((s.B, s.H, s.Dk)), t0=5)
    o1, S1, h1 = O.recurrent(x, state0=S0, precond=pc, scale=0.7)
    o2, S2, h2 = O.chunked(x, chunk=chunk, state0=S0, precond=pc, scale=0.7)
    assert O.rel_l2(o2, o1) < 1e-12
    assert O.rel_l2(S2, S1) < 1e-12
    if pc is not None:
        np.testing.assert_array_equal(h1, h2)


# ----------------------------------------------------------------------------------
# The triangular inverse [MMI]: Lemma 3.1, full Neumann, band identity, residual.
# ----------------------------------------------------------------------------------

def _chunk_A(C=64, Dk=16, seed=3):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((C, Dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(C)))
    g = np.cumsum(-0.1 * np.logaddexp(0, rng.standard_normal(C)))
    i, j = np.indices((C, C))
    L = np.where(j < i, (beta[:, None] * k) @ k.T * np.exp(np.where(j < i, g[:, None] - g[None, :], 0)), 0)
    return -L


@pytest.mark.parametrize("C", [8, 16, 32, 64])
def test_lemma_3_1_powers(C):
    """A^n is zero above its n-th subdiagonal; A^C = 0 exactly."""
    A = _chunk_A(C)
    i, j = np.indices((C, C))
    P = np.eye(C)
    for n in range(1, C + 1):
        P = P @ A
        assert np.all(P[i - j < n] == 0.0)
    assert np.all(P == 0.0)


@pytest.mark.parametrize("C", [4, 16, 64])
def test_full_neumann_is_the_inverse(C):
    """N >= C - 1: masked truncated Neumann == forward substitution == triangular solve
    == numpy inverse of (I - A)."""
    A = _chunk_A(C)
    inv = np.linalg.inv(np.eye(C) - A)
    for N in (C - 1, C + 5):
        np.testing.assert_allclose(O.neumann_literal(A, N), inv, atol=1e-12)
    np.testing.assert_allclose(O.forward_substitution(A), inv, atol=1e-12)
    np.testing.assert_allclose(O.tri_inverse(A, "exact"), inv, atol=1e-12)
    np.testing.assert_allclose((np.eye(C) - A) @ O.forward_substitution(A), np.eye(C), atol=1e-12)


@pytest.mark.parametrize("N", [1, 3, 7])
def test_band_of_truncated_series_is_band_of_inverse(N):
    """Lemma 3.1 consequence: band_N(sum_{n<=N} A^n) = band_N((I - A)^-1), and it depends
    only on band_N(A)."""
    C = 64
    A = _chunk_A(C, seed=N)
    i, j = np.indices((C, C))
    band = i - j <= N
    T_exact = O.tri_inverse(A, "exact")
    np.testing.assert_allclose(O.neumann_literal(A, N), np.where(band, T_exact, 0), atol=1e-13)
    A2 = np.where(band, A, np.tril(RNG.standard_normal((C, C)), -1))   # change A outside the band
    np.testing.assert_allclose(O.neumann_literal(A2, N), O.neumann_literal(A, N), atol=1e-13)


@pytest.mark.parametrize("N,S", [(3, 0), (3, 1), (3, 8), (1, 2), (7, 3)])
def test_residual_correction_closed_form(N, S):
    """E = I - (I - A) T0 lives on subdiagonals >= N + 1, so T0 sum_{s<=S} E^s equals the
    inverse on every subdiagonal < (S + 1)(N + 1) and everywhere once that reaches C."""
    C = 64
    A = _chunk_A(C, seed=11)
    i, j = np.indices((C, C))
    T_exact = O.tri_inverse(A, "exact")
    Tr = O.residual_corrected(A, N, S)
    exact_band = (i - j) < (S + 1) * (N + 1)
    np.testing.assert_allclose(np.where(exact_band, Tr, 0), np.where(exact_band, T_exact, 0), atol=1e-12)
    if (S + 1) * (N + 1) >= C:
        np.testing.assert_allclose(Tr, T_exact, atol=1e-12)


def test_sign_of_A_matters():
    """With A = +tril(...) instead of -tril(...) the chunk form leaves the recurrence."""
    s, x, _ = small_inputs("gdn", T=64)
    o1, _, _ = O.recurrent(x)
    import oracle.core as C

    orig = C.tri_inverse
    try:
        C.tri_inverse = lambda A, mode="exact": orig(-A, mode)
        o2, _, _ = O.chunked(x, chunk=16)
    finally:
        C.tri_inverse = orig
    assert O.rel_l2(o2, o1) > 1e-3


# ----------------------------------------------------------------------------------
# Variants: reductions and textbook special cases.
# ----------------------------------------------------------------------------------

def test_channel_gates_equal_to_beta_give_plain_rule():
    s, x, _ = small_inputs("gdn", T=50)
    x2 = dict(x)
    beta = x2.pop("beta")
    x2["erase"] = np.repeat(beta[..., None], s.Dk, axis=-1)
    x2["write"] = np.repeat(beta[..., None], s.Dv, axis=-1)
    o1, S1, _ = O.recurrent(x)
    o2, S2, _ = O.recurrent(x2)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


@pytest.mark.parametrize("decay", [False, True])
def test_zero_erase_is_causal_linear_attention(decay):
    """Erase gate 0, write gate 1: nothing is erased, o = tril(Q K^T (.) Gamma) V
    (linear attention, the offline solve of [PDN section 2a/2c])."""
    T, Dk, Dv = 45, 6, 5
    x = {"q": RNG.standard_normal((T, Dk)), "k": RNG.standard_normal((T, Dk)),
         "v": RNG.standard_normal((T, Dv)), "erase": np.zeros((T, Dk)), "write": np.ones((T, Dv))}
    g = np.zeros(T)
    if decay:
        x["log_alpha"] = -0.3 * RNG.random(T)
        g = np.cumsum(x["log_alpha"])
    i, j = np.indices((T, T))
    Gam = np.where(j <= i, np.exp(np.where(j <= i, g[:, None] - g[None, :], 0)), 0)
    ref = ((x["q"] @ x["k"].T) * Gam) @ x["v"]
    for fn in (O.recurrent_stream, lambda x: O.chunked_stream(x, chunk=16)):
        o, _, _ = fn(x)
        np.testing.assert_allclose(o, ref, atol=1e-12)


def test_precond_accumulator_closed_form():
    """h_t = rho^t h_0 + sum_{s<=t} rho^{t-s} k_s^2 (the prefix sum of [PDN 2b], decayed)."""
    T, Dk, rho = 40, 5, 0.99
    k = RNG.standard_normal((T, Dk))
    h0 = 1.0 + RNG.random(Dk)
    u, hT = O.diag_precond_write_key(k, rho, 1e-3, h0, t0=0)
    for t in (0, 7, T - 1):
        h_t = rho ** (t + 1) * h0 + sum(rho ** (t - s) * k[s] ** 2 for s in range(t + 1))
        hhat = h_t / (1 - rho ** (t + 1))
        np.testing.assert_allclose(u[t], k[t] / (hhat + 1e-3), rtol=1e-13)
    np.testing.assert_allclose(hT, rho ** T * h0 + sum(rho ** (T - 1 - s) * k[s] ** 2 for s in range(T)), rtol=1e-13)
    # split: absorbing the first 15 tokens then continuing with t0 = 15 gives the same keys
    u1, h1 = O.diag_precond_write_key(k[:15], rho, 1e-3, h0, t0=0)
    u2, h2 = O.diag_precond_write_key(k[15:], rho, 1e-3, h1, t0=15)
    np.testing.assert_allclose(np.concatenate([u1, u2]), u, rtol=1e-15)


def test_write_key_equal_to_read_key_is_plain_rule():
    s, x, _ = small_inputs("gdn", T=40)
    x2 = dict(x, write_key=x["k"])
    o1, S1, _ = O.recurrent(x)
    o2, S2, _ = O.recurrent(x2)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


@pytest.mark.parametrize("form", ["recurrent", "chunked"])
def test_exact_preconditioner_is_ridge_regression(form):
    """Write key G_t^-1 k_t with G_t = lambda I + sum_{s<=t} k_s k_s^T, beta = 1, S_0 = 0:
    the recurrence is recursive least squares, so S_t = (sum v k^T) G_t^-1 and
    o_t = S_t q_t -- the exact least-squares recovery of [PDN section 2a]."""
    T, Dk, Dv, lam = 30, 6, 4, 0.5
    q, k, v = RNG.standard_normal((T, Dk)), RNG.standard_normal((T, Dk)), RNG.standard_normal((T, Dv))
    G = lam * np.eye(Dk)
    wk = np.empty((T, Dk))
    ref = np.empty((T, Dv))
    M = np.zeros((Dv, Dk))
    for t in range(T):
        G = G + np.outer(k[t], k[t])
        wk[t] = np.linalg.solve(G, k[t])
        M = M + np.outer(v[t], k[t])
        ref[t] = np.linalg.solve(G.T, M.T).T @ q[t]
    x = {"q": q, "k": k, "v": v, "beta": np.ones(T), "write_key": wk}
    fn = O.recurrent_stream if form == "recurrent" else (lambda x: O.chunked_stream(x, chunk=8))
    o, S, _ = fn(x)
    np.testing.assert_allclose(o, ref, atol=1e-10)


# ----------------------------------------------------------------------------------
# State I/O: decode steps and resumption.
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("variant", ["gdn", "gdn2", "pdn", "kda"])
def test_decode_steps_equal_recurrence(variant):
    s, x, pc = small_inputs(variant, B=2, H=2, T=9)
    o_ref, S_ref, h_ref = O.recurrent(x, precond=pc)
    S = np.zeros((s.B, s.H, s.Dv, s.Dk))
    hcur = np.full((s.B, s.H, s.Dk), 1.0)
    for t in range(s.T):
        xt = {key: val[:, t] for key, val in x.items()}
        p = None if pc is None else dict(pc, h_init=hcur, t0=t)
        o, S, hf = O.decode_step(xt, S, precond=p)
        if hf is not None:
            hcur = hf
        np.testing.assert_allclose(o, o_ref[:, t], atol=1e-13)
    np.testing.assert_allclose(S, S_ref, atol=1e-13)


@pytest.mark.parametrize("variant", ["gdn", "pdn", "kda"])
def test_split_sequence_resume(variant):
    s, x, pc = small_inputs(variant, T=100)
    o, S, h = O.chunked(x, chunk=16, precond=pc)
    cut = 37
    xa = {key: val[:, :cut] for key, val in x.items()}
    xb = {key: val[:, cut:] for key, val in x.items()}
    oa, Sa, ha = O.chunked(xa, chunk=16, precond=pc)
    pb = None if pc is None else dict(pc, h_init=ha, t0=cut)
    ob, Sb, hb = O.chunked(xb, chunk=16, state0=Sa, precond=pb)
    assert O.rel_l2(np.concatenate([oa, ob], axis=1), o) < 1e-13
    assert O.rel_l2(Sb, S) < 1e-13


def test_error_measures():
    a = np.array([3.0, 4.0])
    assert O.rel_l2(a, a) == 0.0
    assert O.rel_l2(np.array([3.0, 4.5]), a) == pytest.approx(0.1)
    assert O.snr_db(np.array([3.0, 4.5]), a) == pytest.approx(20.0)


def test_bf16_rounding_of_generator():
    """The generator's bf16 rounding is round-to-nearest-even on the top 16 bits."""
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 1e-3], dtype=np.float32)
    r = gs.round_to_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                       # tie -> even (mantissa ...0)
    assert r[2] == 1.0 + 4 * 2 ** -8         # tie -> even (rounds up)
    assert r[3] == 1.0
    assert r[4] == -2.5
    assert abs(r[5] - 1e-3) <= 1e-3 * 2 ** -8
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
