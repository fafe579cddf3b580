"""fp64 NumPy oracle of the chunked gated delta rule -- TEST INFRASTRUCTURE ONLY.

Notation.  One (batch, head) stream has tokens t = 1..T with query q_t and key k_t
in R^{Dk} and value v_t in R^{Dv}.  The state S is Dv x Dk and the output is
o_t = S_t (scale * q_t).  Every supported variant is one rank-1 template with an
erase (read) key e_t, a write key r_t, a written value v'_t and a decay: a scalar
alpha_t = exp(log_alpha_t), or one decay per key channel, a_t = exp(log_alpha_t) in
R^{Dk} (the diagonal gate S_{t-1} Diag(a_t) of Kimi Delta Attention):

    S_t = alpha_t S_{t-1} (I - e_t r_t^T) + v'_t r_t^T
    S_t = S_{t-1} Diag(a_t) (I - e_t r_t^T) + v'_t r_t^T        (per-channel decay)

    variant                         alpha_t   e_t          r_t          v'_t
    delta rule                      1         beta k       k            beta v
    scalar-gated delta rule         alpha_t   beta k       k            beta v
    channel gates (erase b, write w) 1 or a_t  b (.) k      k            w (.) v
    diagonal preconditioner (ATK)   1 or a_t  beta k       k (.) p_t    beta v
    explicit write key              1 or a_t  beta k       given        beta v

Sources: the delta rule is the online SGD step on the least-squares loss [PDN
section 1]; alpha_t and beta_t are the decay and gain axes [PDN section 2c]; the
preconditioner applied to the write key, with the read key kept for the prediction
S k, is apply-to-key [PDN section 2a]; its diagonal form is a second-moment prefix
sum [PDN section 2b]; erase and write gates sit on the key and value axes [GDN2].
The chunk form and T = (I - A)^-1 follow [MMI "Declaracao do Problema"].  Page
titles are listed in ``oracle/__init__.py``.

Readings where the pages are silent (each pinned by a test):
* The decay multiplies the old state only; the write term is not decayed.  A
  per-channel decay scales the state's key channels (its columns), before the erase.
* The output reads the state after token t's own update.
* A carries the minus sign: A = -tril_{-1}((E R^T) (.) Gamma), so T = (I + L)^-1.
* Channel gates: the erase gate scales the key in the erase term and the write gate
  scales the value: e = b (.) k, r = k, v' = w (.) v  (*parity unpinned* against the
  Gated DeltaNet-2 model itself: the news item gives the gates' axes, no formula).
* Diagonal preconditioner (decayed, bias-corrected form): h_t = rho h_{t-1} + k_t^2,
  h_0 = h0, hhat_t = h_t / (1 - rho^t) with t the 1-based global token index,
  p_t = 1 / (hhat_t + eps), computed from the stored (possibly bf16-rounded) k.
* A sequence whose length is not a multiple of the chunk size ends with a shorter
  chunk (equivalent to padding with identity transitions).
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np
import scipy.linalg

F64 = np.float64


# --------------------------------------------------------------------------------------
# Variant vectors (the "prologue"): e, r, v' per token of one stream.
# --------------------------------------------------------------------------------------

def diag_precond_write_key(k: np.ndarray, rho: float, eps: float, h_init: np.ndarray,
                           t0: int) -> Tuple[np.ndarray, np.ndarray]:
    """Diagonal second-moment preconditioner applied to the key [PDN section 2b].

    The accumulator of per-channel second moments is a prefix sum over tokens; here in
    its decayed, bias-corrected form.  Returns the write key u_t = k_t (.) p_t for every
    token and the final accumulator h_T.  ``t0`` counts tokens already absorbed into
    ``h_init`` (the bias correction uses the global 1-based index t0 + t).
    """
    k = np.asarray(k, dtype=F64)
    h = np.array(h_init, dtype=F64, copy=True)
    u = np.empty_like(k)
    for t in range(k.shape[0]):
        h = rho * h + k[t] * k[t]
        tg = t0 + t + 1
        hhat = h / (1.0 - rho ** tg)
        u[t] = k[t] / (hhat + eps)
    return u, h


def variant_vectors(x: Dict[str, np.ndarray], *, precond: Optional[dict] = None
                    ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """Per-token (e, r, v', log_alpha, h_final) of ONE stream.

    ``x`` holds 2-D arrays [T, D] (and 1-D [T] gates) for a single (batch, head):
    keys q, k, v and either ``beta`` (scalar gain) or ``erase``/``write`` (channel
    gain); optionally ``log_alpha`` (scalar decay) and ``write_key`` (explicit write
    key).  ``precond`` = dict(rho, eps, h_init, t0) selects the diagonal
    preconditioner for the write key.  ``log_alpha`` is [T] (scalar decay) or [T, Dk]
    (one decay per key channel).
    """
    k = np.asarray(x["k"], dtype=F64)
    v = np.asarray(x["v"], dtype=F64)
    T = k.shape[0]
    if x.get("erase") is not None:
        e = np.asarray(x["erase"], dtype=F64) * k
        vp = np.asarray(x["write"], dtype=F64) * v
    else:
        beta = np.asarray(x["beta"], dtype=F64)
        e = beta[:, None] * k
        vp = beta[:, None] * v
    h_final = None
    if precond is not None:
        r, h_final = diag_precond_write_key(k, precond["rho"], precond["eps"],
                                            precond["h_init"], precond["t0"])
    elif x.get("write_key") is not None:
        r = np.asarray(x["write_key"], dtype=F64)
    else:
        r = k
    la = x.get("log_alpha")
    la = np.zeros(T, dtype=F64) if la is None else np.asarray(la, dtype=F64)
    return e, r, vp, la, h_final


# --------------------------------------------------------------------------------------
# The definition: token-by-token recurrence.
# --------------------------------------------------------------------------------------

def recurrent_stream(x: Dict[str, np.ndarray], *, scale: float = 1.0,
                     S0: Optional[np.ndarray] = None, precond: Optional[dict] = None
                     ) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """One stream, token by token: S <- alpha S; d = v' - S e; S <- S + d r^T; o = S (scale q).

    With a per-channel decay the first step is S <- S Diag(a_t) (column c scaled by a_tc;
    numpy broadcasts the [Dk] row of decays over the rows of S).
    Returns (o [T, Dv], S_T [Dv, Dk], h_T or None).
    """
    e, r, vp, la, h_final = variant_vectors(x, precond=precond)
    q = np.asarray(x["q"], dtype=F64) * scale
    T, Dk = e.shape
    Dv = vp.shape[1]
    S = np.zeros((Dv, Dk), dtype=F64) if S0 is None else np.array(S0, dtype=F64, copy=True)
    o = np.empty((T, Dv), dtype=F64)
    for t in range(T):
        S *= np.exp(la[t])
        d = vp[t] - S @ e[t]
        S += np.outer(d, r[t])
        o[t] = S @ q[t]
    return o, S, h_final


def _stream(x: Dict[str, np.ndarray], b: int, h: int) -> Dict[str, np.ndarray]:
    return {key: (None if val is None else val[b, :, h]) for key, val in x.items()}


def _precond_for(precond: Optional[dict], b: int, h: int, Dk: int) -> Optional[dict]:
    if precond is None:
        return None
    hi = precond.get("h_init")
    h_init = np.full(Dk, precond.get("h0", 1.0), dtype=F64) if hi is None else hi[b, h]
    return dict(rho=precond["rho"], eps=precond["eps"], h_init=h_init,
                t0=precond.get("t0", 0))


def _run(fn, x, *, state0=None, precond=None, streams=None, **kw):
    B, T, H, _ = x["q"].shape
    Dk = x["k"].shape[-1]
    Dv = x["v"].shape[-1]
    o = np.zeros((B, T, H, Dv), dtype=F64)
    S = np.zeros((B, H, Dv, Dk), dtype=F64)
    hf = np.zeros((B, H, Dk), dtype=F64) if precond is not None else None
    todo = streams if streams is not None else [(b, h) for b in range(B) for h in range(H)]
    for (b, h) in todo:
        s0 = None if state0 is None else state0[b, h]
        ob, Sb, hb = fn(_stream(x, b, h), S0=s0, precond=_precond_for(precond, b, h, Dk), **kw)
        o[b, :, h] = ob
        S[b, h] = Sb
        if hf is not None:
            hf[b, h] = hb
    return o, S, hf


def recurrent(x: Dict[str, np.ndarray], *, scale: float = 1.0,
              state0: Optional[np.ndarray] = None, precond: Optional[dict] = None,
              streams=None):
    """The recurrence over [B, T, H, D] inputs.  Returns (o, S_final, h_final).

    ``state0`` is [B, H, Dv, Dk] (zero if None).  ``precond`` = dict(rho, eps, h0 or
    h_init [B, H, Dk], t0).  ``streams`` restricts the work to a list of (b, h) pairs
    (the other entries of the results stay zero).
    """
    return _run(recurrent_stream, x, state0=state0, precond=precond, streams=streams,
                scale=scale)


def decode_step(x: Dict[str, np.ndarray], state: np.ndarray, *, scale: float = 1.0,
                precond: Optional[dict] = None):
    """One token for every stream: inputs [B, H, D] / [B, H]; state [B, H, Dv, Dk].

    Returns (o [B, H, Dv], new state, h_final or None).  Same recurrence with T = 1.
    """
    xt = {key: (None if val is None else np.asarray(val)[:, None]) for key, val in x.items()}
    o, S, hf = recurrent(xt, scale=scale, state0=state, precond=precond)
    return o[:, 0], S, hf


# --------------------------------------------------------------------------------------
# Triangular inverse T = (I - A)^-1 of a strictly lower-triangular A [MMI].
# --------------------------------------------------------------------------------------

def forward_substitution(A: np.ndarray) -> np.ndarray:
    """T = (I - A)^-1 by forward substitution, column by column [MMI "Declaracao do Problema"].

    (I - A) T = I gives, for i > j, T_ij = sum_{l=j}^{i-1} A_il T_lj with T_jj = 1:
    k - 1 sequential steps for a k x k matrix.
    """
    n = A.shape[0]
    T = np.eye(n, dtype=F64)
    for j in range(n):
        for i in range(j + 1, n):
            acc = 0.0
            for l in range(j, i):
                acc += A[i, l] * T[l, j]
            T[i, j] = acc
    return T


def neumann_literal(A: np.ndarray, N: int) -> np.ndarray:
    """Truncated Neumann series with the structural diagonal mask [MMI Metodologia 1, 2].

    T0 = sum_{n=0}^{N} A^n by explicit powers, then entries with i - j > N are set to
    zero (mask M_ij = 1 iff i - j <= N), by selection.
    """
    n = A.shape[0]
    T0 = np.eye(n, dtype=F64)
    P = np.eye(n, dtype=F64)
    for _ in range(N):
        P = P @ A
        T0 = T0 + P
    i, j = np.indices((n, n))
    return np.where(i - j <= N, T0, 0.0)


def residual_corrected(A: np.ndarray, N: int, S: int) -> np.ndarray:
    """Parallel residual correction [MMI Metodologia 3].

    With the masked truncated series T0, E = I - (I - A) T0 and T ~ T0 sum_{s=0}^{S} E^s.
    """
    n = A.shape[0]
    I = np.eye(n, dtype=F64)
    T0 = neumann_literal(A, N)
    E = I - (I - A) @ T0
    acc = I.copy()
    P = I.copy()
    for _ in range(S):
        P = P @ E
        acc = acc + P
    return T0 @ acc


def tri_inverse(A: np.ndarray, mode="exact") -> np.ndarray:
    """T = (I - A)^-1 by one of: "exact" (triangular solve), "fwdsub",
    ("neumann", N) or ("residual", N, S)."""
    if mode == "exact":
        n = A.shape[0]
        return scipy.linalg.solve_triangular(np.eye(n) - A, np.eye(n), lower=True,
                                             unit_diagonal=True)
    if mode == "fwdsub":
        return forward_substitution(A)
    if isinstance(mode, tuple) and mode[0] == "neumann":
        return neumann_literal(A, int(mode[1]))
    if isinstance(mode, tuple) and mode[0] == "residual":
        return residual_corrected(A, int(mode[1]), int(mode[2]))
    raise ValueError(f"unknown tri_inverse mode {mode!r}")


# --------------------------------------------------------------------------------------
# Chunk-parallel form.
# --------------------------------------------------------------------------------------

def chunked_stream(x: Dict[str, np.ndarray], *, chunk: int, t_mode="exact",
                   scale: float = 1.0, S0: Optional[np.ndarray] = None,
                   precond: Optional[dict] = None):
    """One stream in chunk form [MMI "Declaracao do Problema"], step by step.

    For chunk c starting from state S_c, with g the inclusive in-chunk cumulative sum
    of log alpha and Gamma_ij = exp(g_i - g_j) for j <= i:
        L  = tril_{-1}((E R^T) (.) Gamma),  A = -L,  T = (I - A)^-1
        W  = T (e^g (.) E),   U = T V'                       (WY form)
        D  = U - W S_c^T                                     (corrected values)
        O  = (e^g (.) Q) S_c^T + (tril_0(Q R^T) (.) Gamma) D
        S_{c+1} = e^{g_C} S_c + D^T (e^{g_C - g} (.) R)
    Returns (o [T, Dv], S_T, h_T or None).
    """
    e, r, vp, la, h_final = variant_vectors(x, precond=precond)
    if la.ndim == 2:
        return _chunked_stream_channel_decay(e, r, vp, la, h_final, x, chunk=chunk, t_mode=t_mode,
                                             scale=scale, S0=S0)
    q = np.asarray(x["q"], dtype=F64) * scale
    T, Dk = e.shape
    Dv = vp.shape[1]
    S = np.zeros((Dv, Dk), dtype=F64) if S0 is None else np.array(S0, dtype=F64, copy=True)
    o = np.empty((T, Dv), dtype=F64)
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(c0 + chunk, T))
        E, R, V, Q = e[sl], r[sl], vp[sl], q[sl]
        n = E.shape[0]
        g = np.cumsum(la[sl])
        i, j = np.indices((n, n))
        causal = j <= i
        Gam = np.where(causal, np.exp(np.where(causal, g[:, None] - g[None, :], 0.0)), 0.0)
        L = np.where(j < i, (E @ R.T) * Gam, 0.0)
        A = -L
        Tm = tri_inverse(A, t_mode)
        W = Tm @ (np.exp(g)[:, None] * E)
        U = Tm @ V
        D = U - W @ S.T
        P = np.where(causal, (Q @ R.T) * Gam, 0.0)
        o[sl] = (np.exp(g)[:, None] * Q) @ S.T + P @ D
        S = np.exp(g[-1]) * S + D.T @ (np.exp(g[-1] - g)[:, None] * R)
    return o, S, h_final


def _chunked_stream_channel_decay(e, r, vp, la, h_final, x, *, chunk, t_mode, scale, S0):
    """Chunk form with one decay per key channel.  With G the inclusive in-chunk cumulative
    sum of log a (a [n, Dk] array) the pairwise decay of channel c between tokens j <= i is
    exp(G_ic - G_jc), so it moves inside the key products:
        L_ij = sum_c e_ic r_jc exp(G_ic - G_jc)  (j < i),  A = -L,  T = (I - A)^-1
        D    = T (V' - (e^G (.) E) S_c^T)
        P_ij = sum_c q_ic r_jc exp(G_ic - G_jc)  (j <= i)
        O    = (e^G (.) Q) S_c^T + P D
        S_{c+1} = S_c Diag(e^{G_C}) + D^T (e^{G_C - G} (.) R)
    (the same derivation as the scalar chunk form: unroll S_t = S_{t-1} Diag(a_t) + d_t r_t^T
    with d_t = v'_t - S_{t-1} Diag(a_t) e_t over the chunk and collect the d_j terms).
    """
    q = np.asarray(x["q"], dtype=F64) * scale
    T, Dk = e.shape
    Dv = vp.shape[1]
    S = np.zeros((Dv, Dk), dtype=F64) if S0 is None else np.array(S0, dtype=F64, copy=True)
    o = np.empty((T, Dv), dtype=F64)
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(c0 + chunk, T))
        E, R, V, Q = e[sl], r[sl], vp[sl], q[sl]
        n = E.shape[0]
        G = np.cumsum(la[sl], axis=0)
        i, j = np.indices((n, n))
        causal = j <= i
        # exp(G_ic - G_jc) where j <= i, else 0 (the exponent is never formed above the diagonal)
        dG = np.where(causal[:, :, None], G[:, None, :] - G[None, :, :], 0.0)
        Gam = np.where(causal[:, :, None], np.exp(dG), 0.0)
        L = np.where(j < i, np.einsum("ic,jc,ijc->ij", E, R, Gam), 0.0)
        Tm = tri_inverse(-L, t_mode)
        D = Tm @ (V - (np.exp(G) * E) @ S.T)
        P = np.where(causal, np.einsum("ic,jc,ijc->ij", Q, R, Gam), 0.0)
        o[sl] = (np.exp(G) * Q) @ S.T + P @ D
        S = S * np.exp(G[-1])[None, :] + D.T @ (np.exp(G[-1][None, :] - G) * R)
    return o, S, h_final


def chunked(x: Dict[str, np.ndarray], *, chunk: int, t_mode="exact", scale: float = 1.0,
            state0: Optional[np.ndarray] = None, precond: Optional[dict] = None,
            streams=None):
    """Chunk form over [B, T, H, D] inputs.  Returns (o, S_final, h_final)."""
    return _run(chunked_stream, x, state0=state0, precond=precond, streams=streams,
                chunk=chunk, t_mode=t_mode, scale=scale)


# --------------------------------------------------------------------------------------
# Error measures.
# --------------------------------------------------------------------------------------

def rel_l2(x: np.ndarray, ref: np.ndarray) -> float:
    """||x - ref||_2 / ||ref||_2 over the whole tensor (fp64)."""
    x = np.asarray(x, dtype=F64)
    ref = np.asarray(ref, dtype=F64)
    den = np.sqrt(np.sum(ref * ref))
    num = np.sqrt(np.sum((x - ref) ** 2))
    return float(num / den) if den > 0 else float(num)


def snr_db(x: np.ndarray, ref: np.ndarray) -> float:
    """Signal-to-noise ratio in dB, -20 log10(rel-L2) (the single-kernel accuracy
    readout of [MMI "Resultados Experimentais"])."""
    e = rel_l2(x, ref)
    return float("inf") if e == 0 else float(-20.0 * np.log10(e))
