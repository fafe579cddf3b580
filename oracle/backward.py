"""fp64 gradients of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Reverse-mode differentiation of the token-by-token recurrence of ``core.recurrent_stream``
(the pages train these layers but print no backward pass; the gradient is the plain
derivative of the forward definition, taken step by step in reverse).  For one stream,
with the state before token t written S_{t-1}, the decay step Sa = alpha_t S_{t-1}
(or S_{t-1} Diag(a_t)), the corrected value d_t = v'_t - Sa e_t and
S_t = Sa + d_t r_t^T, o_t = S_t (scale q_t).  Given the loss gradients dO and dS_T, the
reverse sweep carries G = dL/dS_t:

    G      += do_t (scale q_t)^T              dq_t  = scale S_t^T do_t
    dd_t    = G r_t                            dr_t  = G^T d_t
    dSa     = G - dd_t e_t^T                   de_t  = -Sa^T dd_t,   dv'_t = dd_t
    scalar decay:      dlog_alpha_t = <dSa, Sa>,                    G <- alpha_t dSa
    per-channel decay: dlog_alpha_tc = sum_v dSa_vc Sa_vc,          G <- dSa Diag(a_t)
    no decay:          G <- dSa

and dS_0 = G at the end.  The variant vectors are then differentiated by the chain rule:
e = beta k | b (.) k, v' = beta v | w (.) v, r = k | given write key.

With the diagonal preconditioner [PDN section 2b] the write key is r_t = k_t (.) p_t,
p_t = 1 / (h_t / b_t + eps), b_t = 1 - rho^(t0 + t + 1), h_t = rho h_{t-1} + k_t (.) k_t
(per channel, h_0 the accumulator given), so dr_t reaches k through p_t as well: with
a_t = -(dr_t (.) k_t (.) p_t (.) p_t) / b_t (dL/dh_t through p_t alone) and the accumulator's
total gradient H_t = a_t + rho H_{t+1} (H_{T+1} = 0: the final accumulator is not part of
the loss), dk_t gets dr_t (.) p_t + 2 k_t (.) H_t and the initial accumulator rho H_1.

Pinned in ``tests/test_oracle_grad_pins.py`` by central finite differences of the forward
oracle (every input element, every variant, the preconditioner included) and by the causal
linear-attention special case, whose gradients are textbook.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .core import F64, _precond_for, _stream, variant_vectors


def precond_grad(k: np.ndarray, dr: np.ndarray, rho: float, eps: float, h_init: np.ndarray,
                 t0: int):
    """Chain rule through the diagonal preconditioner of one stream: given dr = dL/dr_t for
    the write keys r_t = k_t (.) p_t, returns (dL/dk_t through r, dL/dh_init)."""
    k = np.asarray(k, dtype=F64)
    dr = np.asarray(dr, dtype=F64)
    T = k.shape[0]
    # the forward prefix: p_t and b_t of every token
    h = np.array(h_init, dtype=F64, copy=True)
    p = np.empty_like(k)
    bt = np.empty(T, dtype=F64)
    for t in range(T):
        h = rho * h + k[t] * k[t]
        bt[t] = 1.0 - rho ** (t0 + t + 1)
        p[t] = 1.0 / (h / bt[t] + eps)
    dk = np.empty_like(k)
    Ht = np.zeros(k.shape[1], dtype=F64)
    for t in reversed(range(T)):
        Ht = -(dr[t] * k[t] * p[t] * p[t]) / bt[t] + rho * Ht
        dk[t] = dr[t] * p[t] + 2.0 * k[t] * Ht
    return dk, rho * Ht


def recurrent_stream_grad(x: Dict[str, np.ndarray], dO: np.ndarray,
                          dS_T: Optional[np.ndarray] = None, *, scale: float = 1.0,
                          S0: Optional[np.ndarray] = None, checkpoint: int = 0,
                          precond: Optional[dict] = None) -> Dict[str, np.ndarray]:
    """Gradients of one stream's loss with respect to its inputs.

    ``x`` holds one stream's [T, D] / [T] arrays as for ``core.recurrent_stream``; ``dO`` is
    dL/do [T, Dv], ``dS_T`` dL/dS_T [Dv, Dk] (zero if None).  ``checkpoint`` > 0 keeps the
    state only every ``checkpoint`` tokens and recomputes the states in between during the
    reverse sweep (for long sequences); 0 keeps every state.

    Returns dq, dk, dv, dS0 and, as the variant has them, dbeta | (derase, dwrite),
    dlog_alpha ([T] or [T, Dk]) and dwrite_key.  ``precond`` = dict(rho, eps, h_init, t0)
    selects the diagonal preconditioner for the write key; then dpc_h_init (dL/dh_init,
    [Dk]) is returned as well.
    """
    e, r, vp, la, _ = variant_vectors(x, precond=precond)
    q = np.asarray(x["q"], dtype=F64) * scale
    dO = np.asarray(dO, dtype=F64)
    T, Dk = e.shape
    Dv = vp.shape[1]
    chd = la.ndim == 2
    S = np.zeros((Dv, Dk), dtype=F64) if S0 is None else np.array(S0, dtype=F64, copy=True)

    def step(S_prev, t):
        """(Sa, d, S_t) of token t from the state before it."""
        a = np.exp(la[t])
        Sa = S_prev * (a[None, :] if chd else a)
        d = vp[t] - Sa @ e[t]
        return Sa, d, Sa + np.outer(d, r[t])

    # forward sweep: the state before every token (or before every checkpoint-th token)
    seg = checkpoint if checkpoint > 0 else 1
    saved = {}
    for t in range(T):
        if t % seg == 0:
            saved[t] = S.copy()
        S = step(S, t)[2]

    de = np.zeros_like(e)
    dr = np.zeros_like(r)
    dvp = np.zeros_like(vp)
    dq = np.zeros_like(q)
    dla = np.zeros_like(la)
    G = np.zeros((Dv, Dk), dtype=F64) if dS_T is None else np.array(dS_T, dtype=F64, copy=True)
    for s0 in reversed(range(0, T, seg)):
        # states before tokens s0 .. s1 - 1 of this segment
        s1 = min(s0 + seg, T)
        before = [saved[s0]]
        for t in range(s0, s1 - 1):
            before.append(step(before[-1], t)[2])
        for t in reversed(range(s0, s1)):
            S_prev = before[t - s0]
            Sa, d, St = step(S_prev, t)
            G = G + np.outer(dO[t], q[t])
            dq[t] = St.T @ dO[t]
            dd = G @ r[t]
            dr[t] = G.T @ d
            dSa = G - np.outer(dd, e[t])
            de[t] = -(Sa.T @ dd)
            dvp[t] = dd
            if chd:
                dla[t] = np.sum(dSa * Sa, axis=0)
                G = dSa * np.exp(la[t])[None, :]
            else:
                dla[t] = np.sum(dSa * Sa)
                G = dSa * np.exp(la[t])
    dq *= scale   # q above is scale * q

    k = np.asarray(x["k"], dtype=F64)
    v = np.asarray(x["v"], dtype=F64)
    g: Dict[str, np.ndarray] = {"dq": dq, "dS0": G}
    if x.get("erase") is not None:
        b = np.asarray(x["erase"], dtype=F64)
        w = np.asarray(x["write"], dtype=F64)
        dk = b * de
        g["derase"] = k * de
        g["dwrite"] = v * dvp
        g["dv"] = w * dvp
    else:
        beta = np.asarray(x["beta"], dtype=F64)
        dk = beta[:, None] * de
        g["dbeta"] = np.sum(k * de, axis=1) + np.sum(v * dvp, axis=1)
        g["dv"] = beta[:, None] * dvp
    if precond is not None:
        dkp, dh0 = precond_grad(k, dr, precond["rho"], precond["eps"], precond["h_init"], precond["t0"])
        dk = dk + dkp
        g["dpc_h_init"] = dh0
    elif x.get("write_key") is not None:
        g["dwrite_key"] = dr
    else:
        dk = dk + dr
    g["dk"] = dk
    if x.get("log_alpha") is not None:
        g["dlog_alpha"] = dla
    return g


def recurrent_grad(x: Dict[str, np.ndarray], dO: np.ndarray, dS_T: Optional[np.ndarray] = None,
                   *, scale: float = 1.0, state0: Optional[np.ndarray] = None, streams=None,
                   checkpoint: int = 0, precond: Optional[dict] = None) -> Dict[str, np.ndarray]:
    """Gradients over [B, T, H, D] inputs (every stream, or the listed (b, h) pairs; the
    other entries stay zero).  ``dO`` is [B, T, H, Dv], ``dS_T`` [B, H, Dv, Dk] or None.
    ``precond`` = dict(rho, eps, h0 or h_init [B, H, Dk], t0) as for ``core.recurrent``.
    The results have the inputs' shapes; dS0 is [B, H, Dv, Dk], dpc_h_init [B, H, Dk]."""
    B, T, H, _ = x["q"].shape
    Dk = x["k"].shape[-1]
    Dv = x["v"].shape[-1]
    out: Dict[str, np.ndarray] = {}
    todo = streams if streams is not None else [(b, h) for b in range(B) for h in range(H)]
    for (b, h) in todo:
        gb = recurrent_stream_grad(_stream(x, b, h), np.asarray(dO)[b, :, h],
                                   None if dS_T is None else dS_T[b, h], scale=scale,
                                   S0=None if state0 is None else state0[b, h],
                                   checkpoint=checkpoint, precond=_precond_for(precond, b, h, Dk))
        for key, val in gb.items():
            if key not in out:
                shape = {"dS0": (B, H, Dv, Dk), "dpc_h_init": (B, H, Dk)}.get(key, (B, T, H) + val.shape[1:])
                out[key] = np.zeros(shape, dtype=F64)
            if key in ("dS0", "dpc_h_init"):
                out[key][b, h] = val
            else:
                out[key][b, :, h] = val
    return out


def chunked_stream_grad(x: Dict[str, np.ndarray], dO: np.ndarray, dS_T: Optional[np.ndarray] = None,
                        *, chunk: int, band: int, scale: float = 1.0, S0: Optional[np.ndarray] = None,
                        precond: Optional[dict] = None) -> Dict[str, np.ndarray]:
    """Gradients of one stream's loss through the chunk form with the band-limited T
    (``core.chunked_stream`` with t_mode ("neumann", band): T_b = M (.) sum_{n<=band} A^n, M the
    band i - j <= band), scalar or no decay.  The band entries of the truncated series equal
    those of (I - A)^-1 for strictly lower A (Lemma 3.1 of the MatMul-only inversion summary),
    so T_b = M (.) T as functions of A and dA = T^T (M (.) dT_b) T^T on the strictly lower part.
    Everything else is the chain rule through the chunk form's steps, chunk by chunk in reverse:
        o = (e^g (.) Q) S^T + P D,   D = T_b X,   X = V' - (e^g (.) E) S^T,
        S' = e^{g_n} S + D^T (e^{g_n - g} (.) R),   P = causal (.) (Q R^T) (.) Gamma,
        L = strict lower (.) (E R^T) (.) Gamma,     A = -L.
    Returns the same dictionary as ``recurrent_stream_grad``.
    """
    e, r, vp, la, _ = variant_vectors(x, precond=precond)
    if la.ndim != 1:
        raise ValueError("chunked_stream_grad: scalar or no decay only")
    q = np.asarray(x["q"], dtype=F64) * scale
    dO = np.asarray(dO, dtype=F64)
    T, Dk = e.shape
    Dv = vp.shape[1]
    S = np.zeros((Dv, Dk), dtype=F64) if S0 is None else np.array(S0, dtype=F64, copy=True)
    # forward, keeping every chunk's operands
    saved = []
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(c0 + chunk, T))
        E, R, V, Q = e[sl], r[sl], vp[sl], q[sl]
        n = E.shape[0]
        g = np.cumsum(la[sl])
        i, j = np.indices((n, n))
        causal = j <= i
        Gam = np.where(causal, np.exp(np.where(causal, g[:, None] - g[None, :], 0.0)), 0.0)
        L = np.where(j < i, (E @ R.T) * Gam, 0.0)
        Tf = np.linalg.inv(np.eye(n) + L)          # the exact inverse, for the derivative
        Tb = np.where(i - j <= band, Tf, 0.0)       # the band (the forward's T_b)
        Et = np.exp(g)[:, None] * E
        X = V - Et @ S.T
        D = Tb @ X
        P = np.where(causal, (Q @ R.T) * Gam, 0.0)
        saved.append((sl, S.copy(), g, Gam, L, Tf, Tb, Et, X, D, P))
        S = np.exp(g[-1]) * S + D.T @ (np.exp(g[-1] - g)[:, None] * R)
    # reverse
    de = np.zeros_like(e)
    dr = np.zeros_like(r)
    dvp = np.zeros_like(vp)
    dq = np.zeros_like(q)
    dla = np.zeros_like(la)
    G = np.zeros((Dv, Dk), dtype=F64) if dS_T is None else np.array(dS_T, dtype=F64, copy=True)
    for (sl, Sc, g, Gam, L, Tf, Tb, Et, X, D, P) in reversed(saved):
        E, R, Q, dOc = e[sl], r[sl], q[sl], dO[sl]
        n = E.shape[0]
        i, j = np.indices((n, n))
        dg = np.zeros(n)
        gn = g[-1]
        Rb = np.exp(gn - g)[:, None] * R
        Qt = np.exp(g)[:, None] * Q
        # S' = e^{g_n} S + D^T Rb
        dD = Rb @ G.T
        dRb = D @ G
        dg[-1] += np.sum(G * Sc) * np.exp(gn) + np.sum(dRb * Rb)
        dg -= np.sum(dRb * Rb, axis=1)
        dR = np.exp(gn - g)[:, None] * dRb
        dS = np.exp(gn) * G
        # o = Qt S^T + P D
        dQt = dOc @ Sc
        dS = dS + dOc.T @ Qt
        dg += np.sum(dQt * Qt, axis=1)
        dQ = np.exp(g)[:, None] * dQt
        dP = np.where(j <= i, dOc @ D.T, 0.0)
        dD = dD + P.T @ dOc
        # P = causal (.) (Q R^T) (.) Gamma
        dg += np.sum(dP * P, axis=1) - np.sum(dP * P, axis=0)
        dQ = dQ + (dP * Gam) @ R
        dR = dR + (dP * Gam).T @ Q
        # D = T_b X,  X = V' - Et S^T
        dX = Tb.T @ dD
        dTb = np.where(i - j <= band, dD @ X.T, 0.0)
        dL = -np.where(j < i, Tf.T @ dTb @ Tf.T, 0.0)   # A = -L, dA = T^T (M (.) dT_b) T^T
        dvp[sl] = dX
        dEt = -dX @ Sc
        dS = dS - dX.T @ Et
        dg += np.sum(dEt * Et, axis=1)
        dE = np.exp(g)[:, None] * dEt
        # L = strict lower (.) (E R^T) (.) Gamma
        dg += np.sum(dL * L, axis=1) - np.sum(dL * L, axis=0)
        dE = dE + (dL * Gam) @ R
        dR = dR + (dL * Gam).T @ E
        de[sl], dr[sl], dq[sl] = dE, dR, dQ
        dla[sl] = np.cumsum(dg[::-1])[::-1]
        G = dS
    dq *= scale
    k = np.asarray(x["k"], dtype=F64)
    v = np.asarray(x["v"], dtype=F64)
    out: Dict[str, np.ndarray] = {"dq": dq, "dS0": G}
    if x.get("erase") is not None:
        b = np.asarray(x["erase"], dtype=F64)
        w = np.asarray(x["write"], dtype=F64)
        dk = b * de
        out["derase"] = k * de
        out["dwrite"] = v * dvp
        out["dv"] = w * dvp
    else:
        beta = np.asarray(x["beta"], dtype=F64)
        dk = beta[:, None] * de
        out["dbeta"] = np.sum(k * de, axis=1) + np.sum(v * dvp, axis=1)
        out["dv"] = beta[:, None] * dvp
    if precond is not None:
        dkp, dh0 = precond_grad(k, dr, precond["rho"], precond["eps"], precond["h_init"], precond["t0"])
        dk = dk + dkp
        out["dpc_h_init"] = dh0
    elif x.get("write_key") is not None:
        out["dwrite_key"] = dr
    else:
        dk = dk + dr
    out["dk"] = dk
    if x.get("log_alpha") is not None:
        out["dlog_alpha"] = dla
    return out


def chunked_grad(x: Dict[str, np.ndarray], dO: np.ndarray, dS_T: Optional[np.ndarray] = None,
                 *, chunk: int, band: int, scale: float = 1.0, state0: Optional[np.ndarray] = None,
                 streams=None, precond: Optional[dict] = None) -> Dict[str, np.ndarray]:
    """``chunked_stream_grad`` over [B, T, H, D] inputs, laid out as ``recurrent_grad``."""
    B, T, H, _ = x["q"].shape
    Dk = x["k"].shape[-1]
    Dv = x["v"].shape[-1]
    out: Dict[str, np.ndarray] = {}
    todo = streams if streams is not None else [(b, h) for b in range(B) for h in range(H)]
    for (b, h) in todo:
        gb = chunked_stream_grad(_stream(x, b, h), np.asarray(dO)[b, :, h],
                                 None if dS_T is None else dS_T[b, h], chunk=chunk, band=band, scale=scale,
                                 S0=None if state0 is None else state0[b, h],
                                 precond=_precond_for(precond, b, h, Dk))
        for key, val in gb.items():
            if key not in out:
                shape = {"dS0": (B, H, Dv, Dk), "dpc_h_init": (B, H, Dk)}.get(key, (B, T, H) + val.shape[1:])
                out[key] = np.zeros(shape, dtype=F64)
            if key in ("dS0", "dpc_h_init"):
                out[key][b, h] = val
            else:
                out[key][b, :, h] = val
    return out
