"""GPU parity of gdr_chunk_fwd_ws: T of every chunk formed first (all chunks at once), then the
matrix-core kernel's sequential pass reading it.  Against the fp64 oracle at the bf16 bound
(rel-L2 <= 2e-2 per stream and per 64-token block) and against gdr_chunk_fwd (the same inverse
route with its blocks in another order: close to rounding).  Every test prints its case first.
"""
import numpy as np
import pytest

import gdr_synth as gs
import oracle as O
from _gpu_util import TOL_BF16, host, run_chunk

pytestmark = pytest.mark.gpu

VARIANTS = ["gdn", "plain", "gdn2", "gdn2_decay"]


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


def spec(variant, **kw):
    base = {"gdn": "gdn", "plain": "plain", "gdn2": "gdn2", "gdn2_decay": "gdn2"}[variant]
    over = dict(B=2, H=2, T=200, Dk=128, Dv=128, dtype="bf16", seed=41)
    over.update(kw)
    if variant == "gdn2_decay":
        over["decay"] = "scalar"
    return gs.spec(base, **over)


def check_streams(o, S, o_ref, S_ref, streams, T):
    for (b, h) in streams:
        eo, eS = O.rel_l2(o[b, :, h], o_ref[b, :, h]), O.rel_l2(S[b, h], S_ref[b, h])
        blk = max((O.rel_l2(o[b, t:t + 64, h], o_ref[b, t:t + 64, h]) for t in range(0, T, 64)), default=0.0)
        print(f"  ({b},{h}) rel-L2 out {eo:.3e} state {eS:.3e} worst 64-token block {blk:.3e}", flush=True)
        assert eo <= TOL_BF16 and eS <= TOL_BF16 and blk <= TOL_BF16


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("B,H,T", [(2, 2, 200), (4, 16, 130)])
def test_tpre_variants(variant, B, H, T):
    s = spec(variant, B=B, H=H, T=T)
    announce(f"tpre {variant} B={B} H={H} T={T}")
    x = gs.make_inputs(s)
    rng = np.random.default_rng(5)
    S0 = (rng.standard_normal((s.B, s.H, s.Dv, s.Dk)) * 0.2).astype(np.float32)
    streams = [(0, 0), (B - 1, H - 1), (B // 2, H // 2)]
    o_ref, S_ref, _ = O.recurrent(x, state0=S0.astype(np.float64), scale=0.9, streams=streams)
    o, S, _ = run_chunk(s, x, state_in=S0, scale=0.9, impl="mfma", workspace=True)
    of, Sf, _ = run_chunk(s, x, state_in=S0, scale=0.9, impl="mfma")
    o, S, of, Sf = host(o), host(S), host(of), host(Sf)
    check_streams(o, S, o_ref, S_ref, streams, T)
    gap = O.rel_l2(o, of)
    print(f"  rel-L2(with workspace, without) over every stream: {gap:.3e}", flush=True)
    assert gap <= 5e-3


@pytest.mark.parametrize("T", [0, 1, 63, 64, 65, 127, 128])
def test_tpre_lengths(T):
    s = spec("gdn", T=T)
    announce(f"tpre gdn T={T}")
    x = gs.make_inputs(s)
    o_ref, S_ref, _ = O.recurrent(x)
    o, S, _ = run_chunk(s, x, impl="mfma", workspace=True)
    o, S = host(o), host(S)
    if T > 0:
        assert O.rel_l2(o, o_ref) <= TOL_BF16
    assert O.rel_l2(S, S_ref) <= TOL_BF16 or T == 0


def test_tpre_chunk128_exact():
    """Exact T at chunk 128 (lowered to chunk 64) through the workspace path."""
    s = spec("gdn", T=300, chunk=128)
    announce("tpre gdn chunk 128 exact T=300")
    x = gs.make_inputs(s)
    o_ref, S_ref, _ = O.recurrent(x)
    o, S, _ = run_chunk(s, x, impl="mfma", workspace=True)
    assert O.rel_l2(host(o), o_ref) <= TOL_BF16 and O.rel_l2(host(S), S_ref) <= TOL_BF16


def test_tpre_not_applicable_is_ignored():
    """The preconditioned write key and the band limit run the fused kernel: a workspace given
    there changes nothing, bit for bit."""
    import torch
    for variant, kw in (("pdn", {}), ("gdn", dict(neumann_order=3))):
        s = gs.spec(variant, B=2, H=2, T=150, Dk=128, Dv=128, dtype="bf16", seed=7)
        announce(f"tpre ignored: {variant} {kw}")
        x = gs.make_inputs(s)
        o1, S1, _ = run_chunk(s, x, impl="mfma", workspace=True, **kw)
        o2, S2, _ = run_chunk(s, x, impl="mfma", **kw)
        assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_tpre_deterministic():
    import torch
    s = spec("gdn2", B=2, H=4, T=257)
    announce("tpre gdn2 twice, bitwise")
    x = gs.make_inputs(s)
    o1, S1, _ = run_chunk(s, x, impl="mfma", workspace=True)
    o2, S2, _ = run_chunk(s, x, impl="mfma", workspace=True)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("workload", ["gdn", "gdn2", "long"])
def test_tpre_full_size_sampled(workload):
    s = gs.spec(workload)
    streams = [(0, 0), (s.B - 1, s.H - 1)]
    announce(f"tpre full size {s}, streams {streams}")
    x = gs.make_inputs(s)
    o_ref, S_ref, _ = O.recurrent(x, streams=streams)
    o, S, _ = run_chunk(s, x, workspace=True)
    check_streams(host(o), host(S), o_ref, S_ref, streams, s.T)


# --------------------------------------------------------------------------------------
# Per-channel decay on the matrix-core kernel: operands, T and P prepared for every chunk
# at once, then the sequential pass with the state decayed per channel
# --------------------------------------------------------------------------------------

def kda_spec(**kw):
    over = dict(B=2, H=2, T=200, Dk=128, Dv=128, dtype="bf16", seed=43)
    over.update(kw)
    return gs.spec("kda", **over)


@pytest.mark.parametrize("B,H,T", [(2, 2, 200), (4, 16, 130), (1, 3, 64)])
def test_kda_matrix_cores(B, H, T):
    """Against the fp64 oracle per stream and per 64-token block, and against the fp32 kernel."""
    s = kda_spec(B=B, H=H, T=T)
    announce(f"kda matrix cores B={B} H={H} T={T}")
    x = gs.make_inputs(s)
    rng = np.random.default_rng(6)
    S0 = (rng.standard_normal((s.B, s.H, s.Dv, s.Dk)) * 0.2).astype(np.float32)
    streams = sorted({(0, 0), (B - 1, H - 1), (B // 2, H // 2)})
    o_ref, S_ref, _ = O.recurrent(x, state0=S0.astype(np.float64), scale=0.9, streams=streams)
    o, S, _ = run_chunk(s, x, state_in=S0, scale=0.9, impl="mfma", workspace=True)
    og, Sg, _ = run_chunk(s, x, state_in=S0, scale=0.9, impl="generic")
    o, S, og, Sg = host(o), host(S), host(og), host(Sg)
    check_streams(o, S, o_ref, S_ref, streams, T)
    gap, gapS = O.rel_l2(o, og), O.rel_l2(S, Sg)
    print(f"  rel-L2(matrix cores, fp32 kernel) over every stream: out {gap:.3e} state {gapS:.3e}", flush=True)
    assert gap <= TOL_BF16 and gapS <= TOL_BF16


@pytest.mark.parametrize("T", [0, 1, 63, 64, 65, 127])
def test_kda_matrix_cores_lengths(T):
    s = kda_spec(T=T)
    announce(f"kda matrix cores T={T}")
    x = gs.make_inputs(s)
    rng = np.random.default_rng(7)
    S0 = (rng.standard_normal((s.B, s.H, s.Dv, s.Dk)) * 0.2).astype(np.float32)
    o_ref, S_ref, _ = O.recurrent(x, state0=S0.astype(np.float64))
    o, S, _ = run_chunk(s, x, state_in=S0, impl="mfma", workspace=True)
    o, S = host(o), host(S)
    if T > 0:
        assert O.rel_l2(o, o_ref) <= TOL_BF16
    assert O.rel_l2(S, S_ref) <= TOL_BF16


def test_kda_matrix_cores_chunk128_exact():
    s = kda_spec(T=300, chunk=128)
    announce("kda matrix cores chunk 128 exact T=300")
    x = gs.make_inputs(s)
    o_ref, S_ref, _ = O.recurrent(x)
    o, S, _ = run_chunk(s, x, impl="mfma", workspace=True)
    assert O.rel_l2(host(o), o_ref) <= TOL_BF16 and O.rel_l2(host(S), S_ref) <= TOL_BF16


def test_kda_matrix_cores_need_the_workspace():
    """Without the workspace the per-channel decay stays on the fp32 kernel: asking for the
    matrix cores is refused, the automatic choice runs the fp32 kernel."""
    s = kda_spec(T=70)
    announce("kda: matrix cores without the workspace")
    x = gs.make_inputs(s)
    with pytest.raises(Exception):
        run_chunk(s, x, impl="mfma")
    import torch
    o, S, _ = run_chunk(s, x)
    og, Sg, _ = run_chunk(s, x, impl="generic")
    assert torch.equal(o, og) and torch.equal(S, Sg)


def test_kda_matrix_cores_deterministic():
    import torch
    s = kda_spec(B=2, H=4, T=257)
    announce("kda matrix cores twice, bitwise")
    x = gs.make_inputs(s)
    o1, S1, _ = run_chunk(s, x, impl="mfma", workspace=True)
    o2, S2, _ = run_chunk(s, x, impl="mfma", workspace=True)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.timeout(300)
def test_kda_matrix_cores_full_size_sampled():
    s = gs.spec("kda")
    streams = [(0, 0), (s.B - 1, s.H - 1), (1, 7)]
    announce(f"kda matrix cores full size {s}, streams {streams}")
    x = gs.make_inputs(s)
    o_ref, S_ref, _ = O.recurrent(x, streams=streams)
    o, S, _ = run_chunk(s, x, workspace=True)
    check_streams(host(o), host(S), o_ref, S_ref, streams, s.T)


@pytest.mark.parametrize("strong_chunks", [(1,), (0, 3), ()])
def test_kda_matrix_cores_mixed_routes(strong_chunks):
    """Chunks whose per-channel decay over the chunk falls below 2^-120 take the preparation's
    robust route, the others the fast one: strong decays (log a = -5 U(0, 1) per token and
    channel) in the listed 64-token chunks only, mild ones elsewhere, against the fp64 oracle."""
    s = kda_spec(B=2, H=3, T=256)
    announce(f"kda matrix cores, strong decays in chunks {strong_chunks}")
    x = gs.make_inputs(s)
    rng = np.random.default_rng(11)
    la = np.array(x["log_alpha"], dtype=np.float64)
    for c in strong_chunks:
        la[:, 64 * c:64 * (c + 1)] = -5.0 * rng.random(la[:, 64 * c:64 * (c + 1)].shape)
    x["log_alpha"] = la.astype(np.float32).astype(np.float64)
    streams = [(0, 0), (1, 2)]
    o_ref, S_ref, _ = O.recurrent(x, streams=streams)
    o, S, _ = run_chunk(s, x, impl="mfma", workspace=True)
    check_streams(host(o), host(S), o_ref, S_ref, streams, s.T)
