"""GPU parity of gdr_chunk_bwd against the fp64 oracle's gradients (``oracle.backward``).

The backward computes in fp32 whatever the io dtype (bf16 inputs are widened exactly), so
every gradient is held to the fp32 bound: rel-L2 <= 1e-4 over each gradient tensor.  Every
test prints the case it runs before touching the GPU.
"""
import numpy as np
import pytest

import gdr_synth as gs
import oracle as O
from _gpu_util import TOL_F32, dev, host, torch_dtype

pytestmark = pytest.mark.gpu

GRAD_NAMES = ["dq", "dk", "dv", "dbeta", "derase", "dwrite", "dlog_alpha", "dwrite_key", "dstate_in",
              "dpc_h_in"]


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


def spec(variant, **kw):
    base = {"plain": "plain", "gdn": "gdn", "gdn2": "gdn2", "explicit": "gdn",
            "gdn2_decay": "gdn2", "kda": "kda", "kda_gdn2": "kda", "kda_explicit": "kda",
            "pdn": "pdn", "pdn_decay": "gdn", "pdn_kda": "kda", "pdn_gdn2": "gdn2"}[variant]
    over = dict(B=2, H=2, T=200, Dk=64, Dv=48, dtype="f32", seed=21)
    over.update(kw)
    if variant in ("explicit", "kda_explicit"):
        over["wkey"] = "explicit"
    if variant == "gdn2_decay":
        over["decay"] = "scalar"
    if variant == "kda_gdn2":
        over["gain"] = "channel"
    if variant.startswith("pdn"):
        over["wkey"] = "precond"
    return gs.spec(base, **over)


def run_bwd(s, x, cot, *, state_in=None, d_state_out=True, scale=1.0, chunk=None, pre=None, band=-1):
    import torch
    import chunked_gated_delta_gdr_amd as G
    io = torch_dtype(s.dtype)
    f32 = torch.float32
    pk = {}
    if pre is not None:
        pk = dict(precond=True, pc_h_in=dev(pre.get("h_init"), f32), pc_rho=pre["rho"], pc_eps=pre["eps"],
                  pc_h0=pre.get("h0", 1.0), pc_t0=pre["t0"])
    g = G.gdr_chunk_bwd(
        dev(x["q"], io), dev(x["k"], io), dev(x["v"], io), dev(cot["d_out"], io),
        beta=dev(x.get("beta"), f32), log_alpha=dev(x.get("log_alpha"), f32),
        erase=dev(x.get("erase"), io), write=dev(x.get("write"), io),
        write_key=dev(x.get("write_key"), io), state_in=dev(state_in, f32),
        d_state_out=dev(cot["d_state_out"], f32) if d_state_out else None,
        chunk=chunk or s.chunk, scale=scale, neumann_order=band, **pk)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in g.items()}


def oracle_grads(s, x, cot, *, state_in=None, d_state_out=True, scale=1.0, streams=None,
                 checkpoint=0, pre=None, band=-1):
    dST = cot["d_state_out"] if d_state_out else None
    if band >= 0:   # the chunk form with the band-limited T
        g = O.chunked_grad(x, cot["d_out"], dST, chunk=s.chunk, band=band, scale=scale, state0=state_in,
                           streams=streams, precond=pre)
    else:
        g = O.recurrent_grad(x, cot["d_out"], dST, scale=scale, state0=state_in, streams=streams,
                             checkpoint=checkpoint, precond=pre)
    g["dstate_in"] = g.pop("dS0")
    if "dpc_h_init" in g:
        g["dpc_h_in"] = g.pop("dpc_h_init")
    return g


def compare(got, ref, streams=None, tol=TOL_F32):
    assert set(got) == set(ref), (sorted(got), sorted(ref))
    for name in GRAD_NAMES:
        if name not in ref:
            continue
        a, b = got[name], ref[name]
        if streams is not None:
            if name in ("dstate_in", "dpc_h_in"):
                a = np.stack([a[bb, hh] for bb, hh in streams])
                b = np.stack([b[bb, hh] for bb, hh in streams])
            else:
                a = np.stack([a[bb, :, hh] for bb, hh in streams])
                b = np.stack([b[bb, :, hh] for bb, hh in streams])
        assert np.all(np.isfinite(a)), name
        err = O.rel_l2(a, b)
        print(f"  {name}: rel-L2 {err:.2e}", flush=True)
        assert err <= tol, (name, err)


def state(s, seed=5, amp=0.3):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((s.B, s.H, s.Dv, s.Dk)) * amp).astype(np.float32)


@pytest.mark.parametrize("variant", ["plain", "gdn", "gdn2", "explicit", "gdn2_decay", "kda", "kda_gdn2",
                                     "kda_explicit"])
def test_bwd_variants_fp32(variant):
    s = spec(variant)
    announce(f"bwd {variant} f32 {s}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    got = run_bwd(s, x, cot, state_in=S0, scale=0.8)
    compare(got, oracle_grads(s, x, cot, state_in=S0, scale=0.8))


@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("variant", ["gdn", "gdn2_decay", "kda"])
def test_bwd_chunk_sizes(variant, chunk):
    s = spec(variant, T=77, chunk=chunk)
    announce(f"bwd {variant} f32 chunk {chunk} {s}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    compare(run_bwd(s, x, cot, state_in=S0), oracle_grads(s, x, cot, state_in=S0))


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (100, 40), (98, 42), (32, 16), (16, 200)])
def test_bwd_head_dims(Dk, Dv):
    s = spec("gdn", Dk=Dk, Dv=Dv, T=130)
    announce(f"bwd gdn f32 Dk={Dk} Dv={Dv} {s}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    compare(run_bwd(s, x, cot, state_in=S0), oracle_grads(s, x, cot, state_in=S0))


@pytest.mark.parametrize("variant", ["gdn", "gdn2", "explicit", "kda"])
def test_bwd_bf16(variant):
    s = spec(variant, dtype="bf16", Dk=128, Dv=128, T=200)
    announce(f"bwd {variant} bf16 {s}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    compare(run_bwd(s, x, cot, state_in=S0), oracle_grads(s, x, cot, state_in=S0))


@pytest.mark.parametrize("variant,H", [("gdn", 2), ("kda", 2), ("gdn", 36)])
def test_bwd_unaligned_inputs(variant, H):
    """Queries, keys and dO one element past a 16-byte boundary: the kernels fall back from
    their four-element loads to element loads, with the same gradients (bitwise: the same
    values reach the same products).  H = 36 gives 288 value tiles of 32 rows (the sequential
    kernels' 32-row variant; the smaller shapes run the 16-row one)."""
    import torch
    import chunked_gated_delta_gdr_amd as G
    s = spec(variant, dtype="bf16", Dk=128, Dv=128, T=150, H=H)
    announce(f"bwd {variant} bf16 unaligned q, k, dO {s}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    io, f32 = torch.bfloat16, torch.float32

    def shifted(a):
        t = dev(a, io)
        buf = torch.empty(t.numel() + 1, dtype=io, device=t.device)
        u = buf[1:].view(t.shape)
        u.copy_(t)
        assert u.data_ptr() % 16 != 0
        return u

    def call(q, k, d_out):
        g = G.gdr_chunk_bwd(q, k, dev(x["v"], io), d_out, beta=dev(x.get("beta"), f32),
                            log_alpha=dev(x.get("log_alpha"), f32), state_in=dev(S0, f32),
                            d_state_out=dev(cot["d_state_out"], f32), chunk=s.chunk)
        torch.cuda.synchronize()
        return {n: host(v) for n, v in g.items()}

    got = call(shifted(x["q"]), shifted(x["k"]), shifted(cot["d_out"]))
    ref = call(dev(x["q"], io), dev(x["k"], io), dev(cot["d_out"], io))
    for n in ref:
        assert np.array_equal(got[n], ref[n]), n
    streams = None if H <= 2 else [(0, 0), (1, H - 1)]
    compare(got, oracle_grads(s, x, cot, state_in=S0, streams=streams), streams=streams)


@pytest.mark.parametrize("T", [1, 37, 64, 65])
def test_bwd_short_and_ragged(T):
    s = spec("gdn", T=T)
    announce(f"bwd gdn f32 T={T}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    compare(run_bwd(s, x, cot, state_in=S0), oracle_grads(s, x, cot, state_in=S0))


def test_bwd_zero_state_and_no_state_gradient():
    s = spec("gdn2_decay", T=150)
    announce(f"bwd gdn2_decay f32 no state_in, no d_state_out {s}")
    x, cot = gs.make_inputs(s), gs.make_cotangents(s)
    got = run_bwd(s, x, cot, state_in=None, d_state_out=False)
    compare(got, oracle_grads(s, x, cot, state_in=None, d_state_out=False))


def test_bwd_empty_sequence():
    """T = 0: no token gradients, and dL/dstate_in = dL/dstate_out."""
    s = spec("gdn", T=0)
    announce("bwd gdn f32 T=0")
    x, cot = gs.make_inputs(s), gs.make_cotangents(s)
    got = run_bwd(s, x, cot, state_in=state(s))
    np.testing.assert_array_equal(got["dstate_in"], cot["d_state_out"])
    assert got["dq"].size == 0 and got["dlog_alpha"].size == 0


def test_bwd_is_deterministic():
    s = spec("gdn", T=150)
    announce("bwd gdn f32 twice, bitwise")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    a = run_bwd(s, x, cot, state_in=S0)
    b = run_bwd(s, x, cot, state_in=S0)
    for name in a:
        np.testing.assert_array_equal(a[name], b[name])


def test_bwd_full_size_gdn_sampled():
    """The gdn workload at full size (B4 H16 T4096 d128 bf16): two streams against the oracle
    (checkpointed reverse sweep), every gradient finite everywhere."""
    s = gs.spec("gdn")
    streams = [(0, 0), (3, 15)]
    announce(f"bwd gdn full size {s}, streams {streams}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s, amp=0.1)
    got = run_bwd(s, x, cot, state_in=S0)
    for name, val in got.items():
        assert np.all(np.isfinite(val)), name
    ref = oracle_grads(s, x, cot, state_in=S0, streams=streams, checkpoint=64)
    compare(got, ref, streams=streams)


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (100, 40), (98, 42), (32, 16)])
def test_bwd_kda_head_dims(Dk, Dv):
    s = spec("kda", Dk=Dk, Dv=Dv, T=130)
    announce(f"bwd kda f32 Dk={Dk} Dv={Dv} {s}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    compare(run_bwd(s, x, cot, state_in=S0), oracle_grads(s, x, cot, state_in=S0))


@pytest.mark.parametrize("T", [1, 37, 64, 65])
def test_bwd_kda_short_and_ragged(T):
    s = spec("kda", T=T)
    announce(f"bwd kda f32 T={T}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    compare(run_bwd(s, x, cot, state_in=S0), oracle_grads(s, x, cot, state_in=S0))


def test_bwd_kda_no_state():
    s = spec("kda", T=150)
    announce(f"bwd kda f32 no state_in, no d_state_out {s}")
    x, cot = gs.make_inputs(s), gs.make_cotangents(s)
    compare(run_bwd(s, x, cot, state_in=None, d_state_out=False),
            oracle_grads(s, x, cot, state_in=None, d_state_out=False))


def test_bwd_kda_equal_channels_is_scalar_decay():
    """Per-channel decays that are equal across the channels give the scalar-decay gradients,
    with dlog_alpha (scalar) the channel sum of dlog_alpha (per channel)."""
    s = spec("kda", T=150)
    announce(f"bwd kda equal channels vs gdn {s}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    la = x["log_alpha"][..., 0].copy()
    xc = dict(x, log_alpha=np.ascontiguousarray(np.repeat(la[..., None], s.Dk, axis=-1)))
    xs = dict(x, log_alpha=la)
    gc = run_bwd(s, xc, cot, state_in=S0)
    gsc = run_bwd(spec("gdn", T=150), xs, cot, state_in=S0)
    for name in ("dq", "dk", "dv", "dbeta", "dstate_in"):
        err = O.rel_l2(gc[name], gsc[name])
        print(f"  {name}: rel-L2 {err:.2e}", flush=True)
        assert err <= TOL_F32, (name, err)
    err = O.rel_l2(gc["dlog_alpha"].sum(-1), gsc["dlog_alpha"])
    print(f"  dlog_alpha (channel sum): rel-L2 {err:.2e}", flush=True)
    assert err <= TOL_F32


def test_bwd_full_size_kda_sampled():
    """The kda workload at full size (B4 H16 T4096 d128 bf16): two streams against the oracle
    (checkpointed reverse sweep), every gradient finite everywhere."""
    s = gs.spec("kda")
    streams = [(0, 0), (3, 15)]
    announce(f"bwd kda full size {s}, streams {streams}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s, amp=0.1)
    got = run_bwd(s, x, cot, state_in=S0)
    for name, val in got.items():
        assert np.all(np.isfinite(val)), name
    ref = oracle_grads(s, x, cot, state_in=S0, streams=streams, checkpoint=64)
    compare(got, ref, streams=streams)


def precond_args(s, given=False, seed=9):
    """The workload's preconditioner, or (given) a random accumulator and a later start."""
    if not given:
        return dict(rho=s.pc_rho, eps=s.pc_eps, h0=s.pc_h0, t0=0)
    rng = np.random.default_rng(seed)
    h_init = rng.uniform(0.002, 0.02, (s.B, s.H, s.Dk)).astype(np.float32)
    return dict(rho=0.95, eps=1e-2, h_init=h_init, t0=37)


@pytest.mark.parametrize("given", [False, True])
@pytest.mark.parametrize("variant", ["pdn", "pdn_decay", "pdn_kda", "pdn_gdn2"])
def test_bwd_precond_fp32(variant, given):
    s = spec(variant)
    pre = precond_args(s, given)
    announce(f"bwd {variant} f32 precond {'given accumulator' if given else 'h0'} {s}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    got = run_bwd(s, x, cot, state_in=S0, scale=0.8, pre=pre)
    compare(got, oracle_grads(s, x, cot, state_in=S0, scale=0.8, pre=pre))


@pytest.mark.parametrize("T,chunk", [(1, 64), (37, 16), (65, 32), (130, 64)])
def test_bwd_precond_lengths(T, chunk):
    s = spec("pdn_decay", T=T, chunk=chunk)
    pre = precond_args(s, True)
    announce(f"bwd pdn_decay f32 T={T} chunk {chunk}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    compare(run_bwd(s, x, cot, state_in=S0, pre=pre), oracle_grads(s, x, cot, state_in=S0, pre=pre))


def test_bwd_precond_bf16():
    s = spec("pdn", dtype="bf16", Dk=128, Dv=128, T=200)
    pre = precond_args(s)
    announce(f"bwd pdn bf16 {s}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    compare(run_bwd(s, x, cot, state_in=S0, pre=pre), oracle_grads(s, x, cot, state_in=S0, pre=pre))


def test_bwd_precond_empty_sequence():
    """T = 0: dL/dpc_h_in is zero (the accumulator reaches no output)."""
    s = spec("pdn", T=0)
    announce("bwd pdn f32 T=0")
    x, cot = gs.make_inputs(s), gs.make_cotangents(s)
    got = run_bwd(s, x, cot, state_in=state(s), pre=precond_args(s, True))
    np.testing.assert_array_equal(got["dpc_h_in"], 0.0)
    np.testing.assert_array_equal(got["dstate_in"], cot["d_state_out"])


def test_bwd_full_size_pdn_sampled():
    """The pdn workload at full size (B4 H16 T4096 d128 bf16, preconditioned write key): two
    streams against the oracle (checkpointed reverse sweep), every gradient finite everywhere."""
    s = gs.spec("pdn")
    pre = precond_args(s)
    streams = [(0, 0), (3, 15)]
    announce(f"bwd pdn full size {s}, streams {streams}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s, amp=0.1)
    got = run_bwd(s, x, cot, state_in=S0, pre=pre)
    for name, val in got.items():
        assert np.all(np.isfinite(val)), name
    ref = oracle_grads(s, x, cot, state_in=S0, streams=streams, checkpoint=64, pre=pre)
    compare(got, ref, streams=streams)


@pytest.mark.parametrize("band", [0, 1, 3, 8])
@pytest.mark.parametrize("variant", ["gdn", "gdn2", "plain", "explicit", "pdn_decay"])
def test_bwd_band_fp32(variant, band):
    """The forward with the band-limited T (neumann_order = band) differentiated: against the
    oracle's chunk-form gradient (dA = T^T (M (.) dT_b) T^T)."""
    s = spec(variant, T=150)
    pre = precond_args(s) if variant.startswith("pdn") else None
    announce(f"bwd {variant} f32 band {band} {s}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    got = run_bwd(s, x, cot, state_in=S0, scale=0.9, pre=pre, band=band)
    compare(got, oracle_grads(s, x, cot, state_in=S0, scale=0.9, pre=pre, band=band))


@pytest.mark.parametrize("chunk,T", [(16, 37), (32, 65), (64, 64)])
def test_bwd_band_chunks(chunk, T):
    s = spec("gdn", T=T, chunk=chunk)
    announce(f"bwd gdn f32 band 2 chunk {chunk} T {T}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    compare(run_bwd(s, x, cot, state_in=S0, band=2), oracle_grads(s, x, cot, state_in=S0, band=2))


def test_bwd_band_covering_the_chunk_is_exact():
    """band >= C - 1 keeps all of T: the band path's gradients are the exact path's."""
    s = spec("gdn", T=150)
    announce("bwd gdn f32 band 63 vs exact")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    a = run_bwd(s, x, cot, state_in=S0)
    b = run_bwd(s, x, cot, state_in=S0, band=63)
    for name in a:
        err = O.rel_l2(b[name], a[name])
        print(f"  {name}: rel-L2 {err:.2e}", flush=True)
        assert err <= TOL_F32, (name, err)


def test_bwd_band_bf16():
    s = spec("gdn", dtype="bf16", Dk=128, Dv=128, T=200)
    announce(f"bwd gdn bf16 band 3 {s}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s)
    compare(run_bwd(s, x, cot, state_in=S0, band=3), oracle_grads(s, x, cot, state_in=S0, band=3))


def test_bwd_full_size_gdn_band_sampled():
    """The gdn workload at full size with the band-limited T (N = 3): two streams against the
    oracle's chunk-form gradient, every gradient finite everywhere."""
    s = gs.spec("gdn")
    streams = [(0, 0), (3, 15)]
    announce(f"bwd gdn full size band 3 {s}, streams {streams}")
    x, cot, S0 = gs.make_inputs(s), gs.make_cotangents(s), state(s, amp=0.1)
    got = run_bwd(s, x, cot, state_in=S0, band=3)
    for name, val in got.items():
        assert np.all(np.isfinite(val)), name
    compare(got, oracle_grads(s, x, cot, state_in=S0, streams=streams, band=3), streams=streams)
