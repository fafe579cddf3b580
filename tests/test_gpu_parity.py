"""GPU parity of gdr_chunk_fwd and gdr_recurrent_step against the fp64 CPU oracle.

Every test prints the case it runs (workload, shape, seed, entry point) before touching
the GPU.  Bounds: rel-L2 <= 1e-4 for the fp32 path, <= 2e-2 for the bf16 path.
"""
import numpy as np
import pytest

import gdr_synth as gs
import oracle as O
from _gpu_util import TOL_BF16, TOL_F32, dev, host, precond_opts, run_chunk, torch_dtype

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


def tol(s):
    return TOL_F32 if s.dtype == "f32" else TOL_BF16


def small(variant, dtype="f32", **kw):
    base = {"plain": "plain", "gdn": "gdn", "gdn2": "gdn2", "pdn": "pdn", "explicit": "gdn",
            "gdn2_decay": "gdn2", "pdn_decay": "pdn", "kda": "kda", "kda_gdn2": "gdn2",
            "kda_pdn": "pdn"}[variant]
    over = dict(B=2, H=3, T=150, Dk=64, Dv=48, dtype=dtype, seed=11)
    if variant in ("kda_gdn2", "kda_pdn"):
        over["decay"] = "channel"
    over.update(kw)
    if variant == "explicit":
        over["wkey"] = "explicit"
    if variant.endswith("_decay"):
        over["decay"] = "scalar"
    return gs.spec(base, **over)


# ---------------------------------------------------------------------------------
# The fp32 path
# ---------------------------------------------------------------------------------

def test_plain_fp32_workload():
    """Plain delta rule, B1 H1 T256 d64 fp32, C64: exact T within 1e-4 of the oracle."""
    s = gs.spec("plain")
    announce(f"plain f32 {s}")
    x = gs.make_inputs(s)
    o_ref, S_ref, _ = O.recurrent(x)
    o, S, _ = run_chunk(s, x)
    assert O.rel_l2(host(o), o_ref) <= TOL_F32
    assert O.rel_l2(host(S), S_ref) <= TOL_F32


def test_full_neumann_is_bitwise_exact_fp32():
    """N >= C - 1 runs the same computation as the exact path: bit-identical in fp32."""
    import torch
    s = gs.spec("plain")
    announce("plain f32 neumann N=63,100 vs exact, bitwise")
    x = gs.make_inputs(s)
    o, S, _ = run_chunk(s, x)
    for N in (63, 100):
        oN, SN, _ = run_chunk(s, x, neumann_order=N)
        assert torch.equal(oN, o) and torch.equal(SN, S), N
    o3, _, _ = run_chunk(s, x, neumann_order=3)
    assert not torch.equal(o3, o)


@pytest.mark.parametrize("N", [0, 1, 3, 7])
def test_band_fp32_matches_literal_neumann(N):
    """Band-N T on the GPU vs the oracle's literal sum_{n<=N} A^n with the diagonal mask."""
    s = gs.spec("plain")
    announce(f"plain f32 band N={N}")
    x = gs.make_inputs(s)
    o_ref, S_ref, _ = O.chunked(x, chunk=64, t_mode=("neumann", N))
    o, S, _ = run_chunk(s, x, neumann_order=N)
    assert O.rel_l2(host(o), o_ref) <= TOL_F32
    assert O.rel_l2(host(S), S_ref) <= TOL_F32


@pytest.mark.parametrize("N,S", [(3, 8), (0, 3), (1, 5), (3, 15)])
def test_residual_fp32_matches_oracle(N, S):
    """Band-N start corrected by S residual steps (T0 sum_{s<=S} E^s) vs the oracle's literal
    steps; (0, 3) and (1, 5) differ from the exact inverse by 1.5e-2 and 5e-4 on this data, so
    the check separates them from it.  Exact once (S + 1)(N + 1) >= C: (3, 15)."""
    s = gs.spec("plain")
    announce(f"plain f32 residual N={N} S={S}")
    x = gs.make_inputs(s)
    o_ref, S_ref, _ = O.chunked(x, chunk=64, t_mode=("residual", N, S))
    o, St, _ = run_chunk(s, x, neumann_order=N, residual_steps=S)
    assert O.rel_l2(host(o), o_ref) <= TOL_F32
    assert O.rel_l2(host(St), S_ref) <= TOL_F32
    if (S + 1) * (N + 1) >= 64:
        o_ex, S_ex, _ = O.recurrent(x)
        assert O.rel_l2(host(o), o_ex) <= TOL_F32 and O.rel_l2(host(St), S_ex) <= TOL_F32


@pytest.mark.parametrize("variant,dtype,chunk", [("pdn", "f32", 64), ("gdn", "f32", 32), ("gdn2_decay", "f32", 16),
                                                 ("pdn", "bf16", 64), ("gdn", "bf16", 64)])
def test_residual_variants(variant, dtype, chunk):
    """The residual correction in every gain / decay / write-key combination and chunk size
    (the auto dispatch: the fp32 kernel for fp32 or chunk < 64, the matrix-core kernel for the
    bf16 cases at chunk 64)."""
    s = small(variant, dtype, chunk=chunk, Dk=64 if dtype == "f32" else 128, Dv=48 if dtype == "f32" else 128)
    announce(f"residual N=2 S=4 {variant} {dtype} C{chunk} {s}")
    x = gs.make_inputs(s)
    o_ref, S_ref, _ = O.chunked(x, chunk=chunk, t_mode=("residual", 2, 4), precond=precond_opts(s))
    o, St, _ = run_chunk(s, x, neumann_order=2, residual_steps=4)
    assert O.rel_l2(host(o), o_ref) <= tol(s)
    assert O.rel_l2(host(St), S_ref) <= tol(s)


@pytest.mark.parametrize("variant", ["plain", "gdn", "gdn2", "pdn", "explicit", "gdn2_decay", "pdn_decay",
                                     "kda", "kda_gdn2", "kda_pdn"])
@pytest.mark.parametrize("chunk,Dk,Dv,T", [(64, 64, 48, 150), (16, 32, 16, 37), (32, 128, 128, 200),
                                           (64, 128, 20, 64)])
def test_variants_fp32(variant, chunk, Dk, Dv, T):
    """Every variant, ragged tails, non-zero state, query scale: fp32 within 1e-4."""
    s = small(variant, "f32", Dk=Dk, Dv=Dv, T=T, chunk=chunk)
    announce(f"{variant} f32 C={chunk} Dk={Dk} Dv={Dv} T={T}")
    x = gs.make_inputs(s)
    rng = np.random.default_rng(5)
    S0 = (rng.standard_normal((s.B, s.H, s.Dv, s.Dk)) * 0.2).astype(np.float32)
    pc = precond_opts(s)
    h_in = None
    if pc is not None:
        h_in = (1.0 + rng.random((s.B, s.H, s.Dk))).astype(np.float32)
        pc = dict(pc, h_init=h_in.astype(np.float64), t0=9)
    o_ref, S_ref, h_ref = O.recurrent(x, state0=S0.astype(np.float64), precond=pc, scale=0.8)
    o, S, h = run_chunk(s, x, state_in=S0, pc_h_in=h_in, pc_t0=9 if pc else 0, scale=0.8)
    assert O.rel_l2(host(o), o_ref) <= TOL_F32
    assert O.rel_l2(host(S), S_ref) <= TOL_F32
    if pc is not None:
        assert O.rel_l2(host(h), h_ref) <= 1e-6


def test_exact_preconditioner_ridge_regression_fp32():
    """Explicit write key G_t^-1 k_t, beta = 1: outputs are the ridge-regression predictions."""
    T, Dk, Dv, lam = 96, 16, 16, 0.5
    rng = np.random.default_rng(8)
    q = rng.standard_normal((T, Dk)); k = rng.standard_normal((T, Dk)); v = rng.standard_normal((T, Dv))
    G = lam * np.eye(Dk); M = np.zeros((Dv, Dk)); wk = np.empty((T, Dk)); ref = np.empty((T, Dv))
    for t in range(T):
        G = G + np.outer(k[t], k[t]); wk[t] = np.linalg.solve(G, k[t])
        M = M + np.outer(v[t], k[t]); ref[t] = np.linalg.solve(G.T, M.T).T @ q[t]
    f = lambda a: a.astype(np.float32)[None, :, None]
    x = {"q": f(q), "k": f(k), "v": f(v), "beta": np.ones((1, T, 1), np.float32), "write_key": f(wk)}
    s = gs.spec("gdn", B=1, H=1, T=T, Dk=Dk, Dv=Dv, dtype="f32", decay="none", wkey="explicit")
    announce("ridge regression f32")
    o, _, _ = run_chunk(s, x, chunk=32)
    assert O.rel_l2(host(o)[0, :, 0], ref) <= 1e-3   # fp32 inputs of an ill-conditioned solve


# ---------------------------------------------------------------------------------
# Edge cases, state I/O, determinism, isolation
# ---------------------------------------------------------------------------------

@pytest.mark.parametrize("T", [0, 1, 63, 64, 65])
def test_lengths_edge_cases(T):
    import torch
    s = small("gdn", "f32", T=max(T, 1), B=1, H=2)
    announce(f"gdn f32 T={T}")
    x = gs.make_inputs(s)
    x = {k_: v_[:, :T] for k_, v_ in x.items()}
    rng = np.random.default_rng(1)
    S0 = rng.standard_normal((s.B, s.H, s.Dv, s.Dk)).astype(np.float32)
    s = s.replace(T=T)
    o, S, _ = run_chunk(s, x, state_in=S0)
    if T == 0:
        assert o.numel() == 0
        assert torch.equal(S.cpu(), torch.from_numpy(S0))
        return
    o_ref, S_ref, _ = O.recurrent(x, state0=S0.astype(np.float64))
    assert O.rel_l2(host(o), o_ref) <= TOL_F32
    assert O.rel_l2(host(S), S_ref) <= TOL_F32


@pytest.mark.parametrize("dtype,impl", [("f32", "generic"), ("bf16", "auto")])
def test_split_sequence_resume(dtype, impl):
    """Running T tokens at once == running a prefix, then the rest from its state (and
    preconditioner accumulator): bitwise when the cut is on a chunk boundary."""
    import torch
    s = small("pdn_decay", dtype, T=256, Dk=128, Dv=128, B=1, H=2)
    announce(f"split resume pdn_decay {dtype} {impl}")
    x = gs.make_inputs(s)
    o, S, h = run_chunk(s, x, impl=impl)
    cut = 128
    xa = {k_: v_[:, :cut] for k_, v_ in x.items()}
    xb = {k_: v_[:, cut:] for k_, v_ in x.items()}
    oa, Sa, ha = run_chunk(s.replace(T=cut), xa, impl=impl)
    ob, Sb, hb = run_chunk(s.replace(T=256 - cut), xb, state_in=host(Sa).astype(np.float32),
                           pc_h_in=host(ha).astype(np.float32), pc_t0=cut, impl=impl)
    assert torch.equal(torch.cat([oa, ob], dim=1), o)
    assert torch.equal(Sb, S) and torch.equal(hb, h)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_deterministic(dtype):
    import torch
    s = small("gdn", dtype, Dk=128, Dv=128, T=300)
    announce(f"determinism gdn {dtype}")
    x = gs.make_inputs(s)
    o1, S1, _ = run_chunk(s, x)
    o2, S2, _ = run_chunk(s, x)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nan_stays_in_its_head(dtype):
    s = small("gdn", dtype, Dk=128, Dv=128, T=130, B=2, H=3)
    announce(f"head isolation gdn {dtype}")
    x = gs.make_inputs(s)
    x["v"] = x["v"].copy()
    x["v"][1, 70, 2, 5] = np.nan
    o, S, _ = run_chunk(s, x)
    o, S = host(o), host(S)
    bad = np.zeros((s.B, s.H), bool)
    bad[1, 2] = True
    for b in range(s.B):
        for h in range(s.H):
            if bad[b, h]:
                assert np.isnan(o[b, 70:, h]).any()
                assert np.isfinite(o[b, :64, h]).all()    # chunks before the NaN are clean
            else:
                assert np.isfinite(o[b, :, h]).all() and np.isfinite(S[b, h]).all()


# ---------------------------------------------------------------------------------
# The bf16 path
# ---------------------------------------------------------------------------------

@pytest.mark.parametrize("variant", ["gdn", "gdn2", "pdn", "explicit", "plain", "kda"])
@pytest.mark.parametrize("impl", ["generic", "auto"])
def test_variants_bf16_small(variant, impl):
    s = small(variant, "bf16", Dk=128, Dv=128, T=200, B=2, H=2)
    announce(f"{variant} bf16 {impl} T=200")
    x = gs.make_inputs(s)
    rng = np.random.default_rng(2)
    S0 = (rng.standard_normal((s.B, s.H, s.Dv, s.Dk)) * 0.2).astype(np.float32)
    o_ref, S_ref, _ = O.recurrent(x, state0=S0.astype(np.float64), precond=precond_opts(s))
    o, S, _ = run_chunk(s, x, state_in=S0, impl=impl)
    assert O.rel_l2(host(o), o_ref) <= TOL_BF16
    assert O.rel_l2(host(S), S_ref) <= TOL_BF16


def _sampled(s, x, o, S, streams, precond=None, t_mode=None, blk=64):
    """Oracle on a few (b, h) streams only; compare those streams.  The output error is the
    larger of the whole-stream rel-L2 and the worst rel-L2 over the stream's 64-token blocks
    (a defect confined to one chunk position moves a long stream's norm too little)."""
    if t_mode is None:
        o_ref, S_ref, _ = O.recurrent(x, precond=precond, streams=streams)
    else:
        o_ref, S_ref, _ = O.chunked(x, chunk=s.chunk, t_mode=t_mode, precond=precond, streams=streams)
    o, S = host(o), host(S)
    errs = []
    for (b, h) in streams:
        e_stream = O.rel_l2(o[b, :, h], o_ref[b, :, h])
        e_blk = max(O.rel_l2(o[b, t0:t0 + blk, h], o_ref[b, t0:t0 + blk, h]) for t0 in range(0, o.shape[1], blk))
        errs.append((max(e_stream, e_blk), O.rel_l2(S[b, h], S_ref[b, h])))
    return errs


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["gdn", "gdn2", "pdn"])
def test_full_size_workloads_sampled(name):
    """Full-size workloads in the benchmark's launch configuration; the oracle checks a
    sample of streams end to end."""
    s = gs.spec(name)
    announce(f"full size {name} {s}")
    x = gs.make_inputs(s)
    o, S, _ = run_chunk(s, x)
    streams = [(0, 0), (s.B - 1, s.H - 1), (s.B // 2, 7)]
    for eo, eS in _sampled(s, x, o, S, streams, precond=precond_opts(s)):
        print(f"  rel-L2 out {eo:.3e} state {eS:.3e}", flush=True)
        assert eo <= TOL_BF16 and eS <= TOL_BF16


@pytest.mark.timeout(300)
def test_precond_band3_vs_exact():
    """Preconditioned workload with exact T and with band N = 3: each vs its oracle, and
    the error between the two reported."""
    s = gs.spec("pdn")
    announce(f"pdn exact vs band3 {s}")
    x = gs.make_inputs(s)
    oe, Se, _ = run_chunk(s, x)
    ob, Sb, _ = run_chunk(s, x, neumann_order=3)
    streams = [(0, 0), (3, 15)]
    for eo, eS in _sampled(s, x, ob, Sb, streams, precond=precond_opts(s), t_mode=("neumann", 3)):
        print(f"  band3 vs oracle band3: out {eo:.3e} state {eS:.3e}", flush=True)
        assert eo <= TOL_BF16 and eS <= TOL_BF16
    gpu_gap = O.rel_l2(host(ob), host(oe))
    print(f"  rel-L2(exact, band3) on the GPU, whole output: {gpu_gap:.3e}", flush=True)
    assert gpu_gap > 1e-2   # the band approximation is far from exact on this data


@pytest.mark.timeout(300)
def test_kda_full_size_and_band():
    """Per-key-channel decay at the benchmark's shape (B4 H16 T4096 d128 bf16) on sampled
    streams, exact T and band N = 3 (each against its oracle)."""
    s = gs.spec("kda")
    announce(f"kda full size {s}")
    x = gs.make_inputs(s)
    o, St, _ = run_chunk(s, x)
    streams = [(0, 0), (3, 15)]
    for eo, eS in _sampled(s, x, o, St, streams):
        print(f"  kda exact vs oracle: out {eo:.3e} state {eS:.3e}", flush=True)
        assert eo <= TOL_BF16 and eS <= TOL_BF16
    ob, Sb, _ = run_chunk(s, x, neumann_order=3)
    for eo, eS in _sampled(s, x, ob, Sb, [(1, 3)], t_mode=("neumann", 3)):
        print(f"  kda band3 vs oracle band3: out {eo:.3e} state {eS:.3e}", flush=True)
        assert eo <= TOL_BF16 and eS <= TOL_BF16


@pytest.mark.timeout(300)
def test_precond_residual_full_size():
    """Preconditioned workload at full size with the band-3 start and 8 residual steps (the
    page's defaults) vs the oracle's residual steps on sampled streams; the distance to the
    exact path is reported."""
    s = gs.spec("pdn")
    announce(f"pdn band3 + residual 8 {s}")
    x = gs.make_inputs(s)
    o, St, _ = run_chunk(s, x, neumann_order=3, residual_steps=8)
    streams = [(0, 0), (3, 15)]
    for eo, eS in _sampled(s, x, o, St, streams, precond=precond_opts(s), t_mode=("residual", 3, 8)):
        print(f"  residual vs oracle residual: out {eo:.3e} state {eS:.3e}", flush=True)
        assert eo <= TOL_BF16 and eS <= TOL_BF16
    for eo, eS in _sampled(s, x, o, St, streams, precond=precond_opts(s)):
        print(f"  residual vs exact oracle: out {eo:.3e} state {eS:.3e}", flush=True)


@pytest.mark.timeout(600)
def test_long_prefill_sampled():
    s = gs.spec("long")
    announce(f"long prefill {s}")
    x = gs.make_inputs(s)
    o, S, _ = run_chunk(s, x)
    for eo, eS in _sampled(s, x, o, S, [(0, 0), (0, 31)]):
        print(f"  rel-L2 out {eo:.3e} state {eS:.3e}", flush=True)
        assert eo <= TOL_BF16 and eS <= TOL_BF16


# ---------------------------------------------------------------------------------
# Decode step
# ---------------------------------------------------------------------------------

@pytest.mark.parametrize("variant,dtype,Dk", [("gdn", "bf16", 128), ("gdn", "f32", 64), ("gdn2", "bf16", 128),
                                              ("pdn", "bf16", 128), ("explicit", "f32", 40),
                                              ("gdn", "f32", 100), ("kda", "bf16", 128), ("kda", "f32", 64),
                                              ("kda", "f32", 100)])
def test_steps_equal_chunk_fwd_and_oracle(variant, dtype, Dk):
    """n x gdr_recurrent_step == oracle recurrence == gdr_chunk_fwd over the same tokens."""
    import torch
    import chunked_gated_delta_gdr_amd as G
    s = small(variant, dtype, T=20, Dk=Dk, Dv=Dk, B=3, H=2)
    announce(f"steps {variant} {dtype} Dk={Dk}")
    x = gs.make_inputs(s)
    pc = precond_opts(s)
    o_ref, S_ref, h_ref = O.recurrent(x, precond=pc)
    o_c, S_c, _ = run_chunk(s, x, chunk=16)
    io = torch_dtype(dtype)
    state = torch.zeros((s.B, s.H, s.Dv, s.Dk), dtype=torch.float32, device="cuda")
    h = torch.full((s.B, s.H, s.Dk), s.pc_h0, dtype=torch.float32, device="cuda") if pc else None
    outs = []
    for t in range(s.T):
        xt = {k_: v_[:, t] for k_, v_ in x.items()}
        o_t, _ = G.gdr_recurrent_step(
            dev(xt["q"], io), dev(xt["k"], io), dev(xt["v"], io), state,
            beta=dev(xt.get("beta"), torch.float32), log_alpha=dev(xt.get("log_alpha"), torch.float32),
            erase=dev(xt.get("erase"), io), write=dev(xt.get("write"), io),
            write_key=dev(xt.get("write_key"), io), precond=pc is not None, pc_h_in=h, pc_h_out=h,
            pc_t0=t)
        outs.append(o_t)
    torch.cuda.synchronize()
    o_s = torch.stack(outs, dim=1)
    t_ = tol(s)
    assert O.rel_l2(host(o_s), o_ref) <= t_
    assert O.rel_l2(host(state), S_ref) <= t_
    assert O.rel_l2(host(o_s), host(o_c)) <= t_
    if pc:
        assert O.rel_l2(host(h), h_ref) <= 1e-6


@pytest.mark.timeout(600)
def test_long_decode_batch64():
    """Long-context workload: prefill B1 H32 T32768, replicate its final state to batch 64,
    run 1024 decode steps with inputs pre-staged on the device; the oracle checks batch
    rows 0 and 63 (all heads) over every step, decode-only from the GPU's state."""
    import torch
    import chunked_gated_delta_gdr_amd as G
    s = gs.spec("long")
    announce(f"long decode {s.decode_batch}x{s.decode_steps}")
    x = gs.make_inputs(s)
    _, S, _ = run_chunk(s, x)
    del x
    Bd, steps = s.decode_batch, s.decode_steps
    state = S.expand(Bd, -1, -1, -1).contiguous()
    S0 = host(state[[0, Bd - 1]])
    bf = torch.bfloat16
    ins = [gs.make_decode_inputs(s, t) for t in range(steps)]
    dq = [(dev(d["q"], bf), dev(d["k"], bf), dev(d["v"], bf), dev(d["beta"], torch.float32),
           dev(d["log_alpha"], torch.float32)) for d in ins]
    outs = torch.empty((steps, Bd, s.H, s.Dv), dtype=bf, device="cuda")
    for t in range(steps):
        q, k, v, be, la = dq[t]
        G.gdr_recurrent_step(q, k, v, state, beta=be, log_alpha=la, out=outs[t])
    torch.cuda.synchronize()
    rows = [0, Bd - 1]
    xo = {key: np.stack([d[key][rows] for d in ins], axis=1) for key in ("q", "k", "v", "beta", "log_alpha")}
    o_ref, S_ref, _ = O.recurrent(xo, state0=S0)
    e_o = O.rel_l2(host(outs[:, rows].transpose(0, 1)), o_ref)
    e_S = O.rel_l2(host(state[rows]), S_ref)
    print(f"  decode rel-L2 out {e_o:.3e} state {e_S:.3e}", flush=True)
    assert e_o <= TOL_BF16 and e_S <= TOL_BF16


# ---------------------------------------------------------------------------------
# The bf16 matrix-core kernel, forced (impl="mfma")
# ---------------------------------------------------------------------------------

@pytest.mark.parametrize("variant", ["kda", "kda_gdn2", "kda_pdn"])
@pytest.mark.parametrize("BV", [16, 32])
@pytest.mark.parametrize("chunk,Dk,Dv,T", [(64, 128, 48, 150), (16, 32, 20, 37), (32, 64, 96, 200)])
def test_kda_value_tiles_fp32(variant, BV, chunk, Dk, Dv, T, monkeypatch):
    """Per-channel decay with value tiles of 16 and 32 state rows (forced through
    GDR_GENERIC_BV; ragged last tiles): fp32 within 1e-4 of the recurrence."""
    monkeypatch.setenv("GDR_GENERIC_BV", str(BV))
    s = small(variant, "f32", Dk=Dk, Dv=Dv, T=T, chunk=chunk)
    announce(f"{variant} f32 BV={BV} C={chunk} Dk={Dk} Dv={Dv} T={T}")
    x = gs.make_inputs(s)
    rng = np.random.default_rng(8)
    S0 = (rng.standard_normal((s.B, s.H, s.Dv, s.Dk)) * 0.2).astype(np.float32)
    pc = precond_opts(s)
    h_in = None
    if pc is not None:
        h_in = (1.0 + rng.random((s.B, s.H, s.Dk))).astype(np.float32)
        pc = dict(pc, h_init=h_in.astype(np.float64), t0=5)
    o_ref, S_ref, h_ref = O.recurrent(x, state0=S0.astype(np.float64), precond=pc, scale=0.7)
    o, S, h = run_chunk(s, x, state_in=S0, pc_h_in=h_in, pc_t0=5 if pc else 0, scale=0.7)
    assert O.rel_l2(host(o), o_ref) <= TOL_F32
    assert O.rel_l2(host(S), S_ref) <= TOL_F32
    if pc is not None:
        assert O.rel_l2(host(h), h_ref) <= 1e-6


MFMA_VARIANTS = ["gdn", "plain", "gdn2", "gdn2_decay", "pdn", "pdn_decay", "explicit"]


@pytest.mark.parametrize("variant", MFMA_VARIANTS)
@pytest.mark.parametrize("BV,B,H,T", [(16, 2, 2, 200), (32, 2, 2, 200), (0, 4, 16, 130)])
def test_mfma_variants(variant, BV, B, H, T, monkeypatch):
    """Every variant on the matrix-core kernel with value tiles of 16 and 32 state rows
    (forced through GDR_MFMA_BV; 0 = the library's own choice)."""
    if BV:
        monkeypatch.setenv("GDR_MFMA_BV", str(BV))
    else:
        monkeypatch.delenv("GDR_MFMA_BV", raising=False)
    s = small(variant, "bf16", Dk=128, Dv=128, T=T, B=B, H=H)
    announce(f"mfma {variant} BV={BV} B={B} H={H} T={T}")
    x = gs.make_inputs(s)
    rng = np.random.default_rng(3)
    S0 = (rng.standard_normal((s.B, s.H, s.Dv, s.Dk)) * 0.2).astype(np.float32)
    pc = precond_opts(s)
    h_in = None
    if pc is not None:
        h_in = (1.0 + rng.random((s.B, s.H, s.Dk))).astype(np.float32)
        pc = dict(pc, h_init=h_in.astype(np.float64), t0=70)
    streams = [(0, 0), (B - 1, H - 1), (B // 2, H // 2)]
    o_ref, S_ref, h_ref = O.recurrent(x, state0=S0.astype(np.float64), precond=pc, scale=0.9, streams=streams)
    o, S, h = run_chunk(s, x, state_in=S0, pc_h_in=h_in, pc_t0=70 if pc else 0, scale=0.9, impl="mfma")
    o, S = host(o), host(S)
    for (b, hh) in streams:
        eo = O.rel_l2(o[b, :, hh], o_ref[b, :, hh])
        eS = O.rel_l2(S[b, hh], S_ref[b, hh])
        print(f"  ({b},{hh}) rel-L2 out {eo:.3e} state {eS:.3e}", flush=True)
        assert eo <= TOL_BF16 and eS <= TOL_BF16
    if pc is not None:
        hh = host(h)
        for (b, k_) in streams:
            assert O.rel_l2(hh[b, k_], h_ref[b, k_]) <= 1e-5


@pytest.mark.parametrize("N", [0, 3, 15, 20, 63])
def test_mfma_band(N):
    """Band-limited T on the matrix-core kernel vs the oracle's literal masked Neumann sum."""
    s = small("pdn", "bf16", Dk=128, Dv=128, T=192, B=2, H=2)
    announce(f"mfma band N={N}")
    x = gs.make_inputs(s)
    pc = precond_opts(s)
    mode = "exact" if N >= 63 else ("neumann", N)
    o_ref, S_ref, _ = O.chunked(x, chunk=64, t_mode=mode, precond=pc)
    o, S, _ = run_chunk(s, x, neumann_order=N, impl="mfma")
    eo, eS = O.rel_l2(host(o), o_ref), O.rel_l2(host(S), S_ref)
    print(f"  rel-L2 out {eo:.3e} state {eS:.3e}", flush=True)
    assert eo <= TOL_BF16 and eS <= TOL_BF16


@pytest.mark.parametrize("variant", MFMA_VARIANTS)
@pytest.mark.parametrize("N,S", [(0, 1), (1, 2), (3, 8)])
def test_mfma_residual(variant, N, S):
    """Residual-corrected T (band-N start, S steps) on the matrix-core kernel vs the oracle's
    literal residual steps.  With N = 0, S = 1 the residual T is 4e-2 away from the exact one on
    these inputs, so the GPU must be much closer to the residual than to the exact T."""
    s = small(variant, "bf16", Dk=128, Dv=128, T=200, B=2, H=2)
    announce(f"mfma residual N={N} S={S} {variant}")
    x = gs.make_inputs(s)
    pc = precond_opts(s)
    o_ref, S_ref, _ = O.chunked(x, chunk=64, t_mode=("residual", N, S), precond=pc)
    o, St, _ = run_chunk(s, x, neumann_order=N, residual_steps=S, impl="mfma")
    eo, eS = O.rel_l2(host(o), o_ref), O.rel_l2(host(St), S_ref)
    print(f"  rel-L2 out {eo:.3e} state {eS:.3e}", flush=True)
    assert eo <= TOL_BF16 and eS <= TOL_BF16
    if (N, S) == (0, 1):
        o_ex, _, _ = O.chunked(x, chunk=64, precond=pc)
        ee = O.rel_l2(host(o), o_ex)
        print(f"  distance to the exact T's output {ee:.3e}", flush=True)
        assert 3 * eo < ee


@pytest.mark.parametrize("BV", [16, 32])
def test_mfma_residual_value_tiles(BV, monkeypatch):
    """Both value-tile widths with the residual steps (different helper-wave counts), a start
    state and a partial last chunk."""
    monkeypatch.setenv("GDR_MFMA_BV", str(BV))
    s = small("pdn_decay", "bf16", Dk=128, Dv=128, T=150, B=2, H=3)
    announce(f"mfma residual N=2 S=4 BV={BV}")
    x = gs.make_inputs(s)
    rng = np.random.default_rng(5)
    S0 = (rng.standard_normal((s.B, s.H, s.Dv, s.Dk)) * 0.2).astype(np.float32)
    pc = precond_opts(s)
    o_ref, S_ref, _ = O.chunked(x, chunk=64, t_mode=("residual", 2, 4), precond=pc, state0=S0.astype(np.float64))
    o, St, _ = run_chunk(s, x, state_in=S0, neumann_order=2, residual_steps=4, impl="mfma")
    eo, eS = O.rel_l2(host(o), o_ref), O.rel_l2(host(St), S_ref)
    print(f"  rel-L2 out {eo:.3e} state {eS:.3e}", flush=True)
    assert eo <= TOL_BF16 and eS <= TOL_BF16


def test_mfma_matches_generic_kernel():
    """The two kernels agree with each other (bf16 inputs; fp32 vs bf16-MFMA internals)."""
    s = small("gdn", "bf16", Dk=128, Dv=128, T=333, B=2, H=4)
    announce("mfma vs generic gdn")
    x = gs.make_inputs(s)
    o1, S1, _ = run_chunk(s, x, impl="mfma")
    o2, S2, _ = run_chunk(s, x, impl="generic")
    assert O.rel_l2(host(o1), host(o2)) <= TOL_BF16
    assert O.rel_l2(host(S1), host(S2)) <= TOL_BF16


@pytest.mark.parametrize("T", [0, 1, 64, 65, 127])
def test_mfma_lengths(T):
    import torch
    s = small("gdn", "bf16", Dk=128, Dv=128, T=max(T, 1), B=1, H=2)
    announce(f"mfma gdn T={T}")
    x = gs.make_inputs(s)
    x = {k_: v_[:, :T] for k_, v_ in x.items()}
    rng = np.random.default_rng(4)
    S0 = rng.standard_normal((s.B, s.H, s.Dv, s.Dk)).astype(np.float32)
    s = s.replace(T=T)
    o, S, _ = run_chunk(s, x, state_in=S0, impl="mfma")
    if T == 0:
        assert torch.equal(S.cpu(), torch.from_numpy(S0))
        return
    o_ref, S_ref, _ = O.recurrent(x, state0=S0.astype(np.float64))
    assert O.rel_l2(host(o), o_ref) <= TOL_BF16
    assert O.rel_l2(host(S), S_ref) <= TOL_BF16
