"""GPU parity at chunk 128 against the fp64 oracle's chunk form at chunk 128.

The exact T at chunk 128 is the chunk-64 computation regrouped (the block T_ba = T_bb A_ba T_aa
is applied through the state after the chunk's first 64 tokens), so it must match the
oracle's exact chunk-128 form and the recurrence alike.  The band-limited T at chunk 128
keeps T's entries with i - j <= N over the whole 128 x 128 matrix, which includes the corner
that joins the two 64-row halves: it must match the oracle's literal masked Neumann sum at
chunk 128 (and differs from the band at chunk 64).  Every test prints its case first.
Bounds: rel-L2 <= 1e-4 on the fp32 kernel, <= 2e-2 with bf16 operands.
"""
import numpy as np
import pytest

import gdr_synth as gs
import oracle as O
from _gpu_util import TOL_BF16, TOL_F32, host, precond_opts, run_chunk

pytestmark = pytest.mark.gpu

VARIANTS = ["plain", "gdn", "gdn2", "gdn2_decay", "pdn", "pdn_decay", "explicit"]


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


def small(variant, dtype="f32", **kw):
    base = {"plain": "plain", "gdn": "gdn", "gdn2": "gdn2", "gdn2_decay": "gdn2", "pdn": "pdn",
            "pdn_decay": "pdn", "explicit": "gdn"}[variant]
    over = dict(B=2, H=3, T=300, Dk=64, Dv=48, dtype=dtype, seed=31, chunk=128)
    over.update(kw)
    if variant == "explicit":
        over["wkey"] = "explicit"
    if variant.endswith("_decay"):
        over["decay"] = "scalar"
    return gs.spec(base, **over)


def start_state(s, seed=3, amp=0.3):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((s.B, s.H, s.Dv, s.Dk)) * amp).astype(np.float32)


def check(o, S, o_ref, S_ref, bound):
    eo, eS = O.rel_l2(host(o), o_ref), O.rel_l2(host(S), S_ref)
    print(f"  rel-L2 out {eo:.3e} state {eS:.3e}", flush=True)
    assert eo <= bound and eS <= bound


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("N", [0, 3, 15])
def test_band_fp32(variant, N):
    """Band N at chunk 128 on the fp32 kernel, T = 300 (two whole chunks and a 44-token tail),
    with a start state, a query scale and, for the preconditioner, a carried h and offset."""
    s = small(variant)
    announce(f"chunk128 band N={N} {variant} f32 {s}")
    x = gs.make_inputs(s)
    S0 = start_state(s)
    pc = precond_opts(s)
    h_in = None
    if pc is not None:
        h_in = (1.0 + np.random.default_rng(4).random((s.B, s.H, s.Dk))).astype(np.float32)
        pc = dict(pc, h_init=h_in.astype(np.float64), t0=90)
    o_ref, S_ref, _ = O.chunked(x, chunk=128, t_mode=("neumann", N), precond=pc, scale=0.9,
                                state0=S0.astype(np.float64))
    o, S, _ = run_chunk(s, x, state_in=S0, pc_h_in=h_in, pc_t0=90 if pc else 0, scale=0.9, neumann_order=N)
    check(o, S, o_ref, S_ref, TOL_F32)


@pytest.mark.parametrize("T", [1, 40, 64, 65, 100, 128, 129, 192, 200, 256])
def test_band_lengths_fp32(T):
    """Lengths around the half and whole chunk: a lone first half, a partial second half, a
    whole chunk, a chunk and one token."""
    s = small("gdn", T=T)
    announce(f"chunk128 band N=3 gdn f32 T={T}")
    x = gs.make_inputs(s)
    S0 = start_state(s)
    o_ref, S_ref, _ = O.chunked(x, chunk=128, t_mode=("neumann", 3), state0=S0.astype(np.float64))
    o, S, _ = run_chunk(s, x, state_in=S0, neumann_order=3)
    check(o, S, o_ref, S_ref, TOL_F32)


def test_band_is_not_the_chunk64_band():
    """The corner that joins the halves matters: the chunk-128 band differs from the chunk-64
    band by far more than rounding, and the GPU follows the chunk-128 one."""
    s = small("plain", T=256, B=1, H=2)
    announce("chunk128 vs chunk64 band N=3 plain f32")
    x = gs.make_inputs(s)
    o128, _, _ = run_chunk(s, x, neumann_order=3)
    o64, _, _ = run_chunk(s, x, neumann_order=3, chunk=64)
    r128, _, _ = O.chunked(x, chunk=128, t_mode=("neumann", 3))
    r64, _, _ = O.chunked(x, chunk=64, t_mode=("neumann", 3))
    gap = O.rel_l2(r128, r64)
    print(f"  oracle gap chunk 128 vs 64: {gap:.3e}", flush=True)
    assert gap > 1e3 * TOL_F32
    assert O.rel_l2(host(o128), r128) <= TOL_F32
    assert O.rel_l2(host(o64), r64) <= TOL_F32


@pytest.mark.parametrize("variant", ["gdn", "pdn", "gdn2"])
@pytest.mark.parametrize("impl,dtype", [("generic", "f32"), ("auto", "bf16")])
def test_exact(variant, impl, dtype):
    """Exact T at chunk 128 (matrix-core kernel for bf16 at d = 128) vs the oracle's exact
    chunk-128 form and its recurrence."""
    s = small(variant, dtype, Dk=128, Dv=128, T=333, B=2, H=2)
    announce(f"chunk128 exact {variant} {dtype} impl={impl}")
    x = gs.make_inputs(s)
    S0 = start_state(s)
    pc = precond_opts(s)
    o_ref, S_ref, _ = O.chunked(x, chunk=128, state0=S0.astype(np.float64), precond=pc)
    o_rec, _, _ = O.recurrent(x, state0=S0.astype(np.float64), precond=pc)
    assert O.rel_l2(o_ref, o_rec) <= 1e-12
    o, S, _ = run_chunk(s, x, state_in=S0, impl=impl)
    check(o, S, o_ref, S_ref, TOL_F32 if dtype == "f32" else TOL_BF16)


def test_exact_band_127_is_exact():
    """A band limit N >= 127 keeps every entry of a 128-token chunk: the same bits as exact."""
    import torch
    s = small("gdn", "bf16", Dk=128, Dv=128, T=300, B=1, H=2)
    announce("chunk128 N=127, 400 vs exact, bitwise")
    x = gs.make_inputs(s)
    o, S, _ = run_chunk(s, x)
    for N in (127, 400):
        oN, SN, _ = run_chunk(s, x, neumann_order=N)
        assert torch.equal(oN, o) and torch.equal(SN, S), N


@pytest.mark.parametrize("N", [3, 15])
def test_band_bf16_headline_shape(N):
    """Band N at chunk 128 with bf16 inputs at d = 128 (the preconditioned workload's shape per
    stream), on the fp32 kernel."""
    s = small("pdn", "bf16", Dk=128, Dv=128, T=520, B=2, H=2)
    announce(f"chunk128 band N={N} pdn bf16 d128 T=520")
    x = gs.make_inputs(s)
    pc = precond_opts(s)
    o_ref, S_ref, _ = O.chunked(x, chunk=128, t_mode=("neumann", N), precond=pc)
    o, S, _ = run_chunk(s, x, neumann_order=N)
    check(o, S, o_ref, S_ref, TOL_BF16)


@pytest.mark.timeout(300)
def test_band3_full_size_sampled():
    """The preconditioned workload at full size (B4 H16 T4096 d128 bf16) with chunk 128 and
    band N = 3, checked on three streams per 128-token block against the oracle's chunk-128
    band form; also reports its gap to the exact T."""
    s = gs.spec("pdn", chunk=128)
    announce(f"chunk128 band N=3 full size {s}")
    x = gs.make_inputs(s)
    pc = precond_opts(s)
    streams = [(0, 0), (1, 7), (3, 15)]
    o_ref, S_ref, _ = O.chunked(x, chunk=128, t_mode=("neumann", 3), precond=pc, streams=streams)
    o, S, _ = run_chunk(s, x, neumann_order=3)
    oe, _, _ = run_chunk(s, x)
    o, S, oe = host(o), host(S), host(oe)
    for (b, h) in streams:
        eo, eS = O.rel_l2(o[b, :, h], o_ref[b, :, h]), O.rel_l2(S[b, h], S_ref[b, h])
        blk = max(O.rel_l2(o[b, t:t + 128, h], o_ref[b, t:t + 128, h]) for t in range(0, s.T, 128))
        print(f"  ({b},{h}) rel-L2 out {eo:.3e} state {eS:.3e} worst 128-token block {blk:.3e}", flush=True)
        assert eo <= TOL_BF16 and eS <= TOL_BF16 and blk <= 2 * TOL_BF16
    gap = O.rel_l2(o, oe)
    print(f"  GPU rel-L2(exact, band 3) at chunk 128, all streams: {gap:.4f}", flush=True)
    assert gap > 1e-2


def test_backward_exact():
    """The backward at chunk 128 (exact T) equals the chunk-64 backward bit for bit and the
    oracle's gradient of the recurrence."""
    import torch
    import chunked_gated_delta_gdr_amd as G
    from _gpu_util import dev
    s = small("gdn", T=200, B=1, H=2)
    announce(f"chunk128 backward exact gdn f32 {s}")
    x, cot = gs.make_inputs(s), gs.make_cotangents(s)
    f32 = torch.float32

    def bwd(chunk):
        g = G.gdr_chunk_bwd(dev(x["q"], f32), dev(x["k"], f32), dev(x["v"], f32), dev(cot["d_out"], f32),
                            beta=dev(x["beta"], f32), log_alpha=dev(x["log_alpha"], f32),
                            d_state_out=dev(cot["d_state_out"], f32), chunk=chunk)
        torch.cuda.synchronize()
        return g

    g128, g64 = bwd(128), bwd(64)
    for name in g64:
        assert torch.equal(g128[name], g64[name]), name
    ref = O.recurrent_grad(x, cot["d_out"], cot["d_state_out"])
    ref["dstate_in"] = ref.pop("dS0")
    for name in ref:
        err = O.rel_l2(host(g128[name]), ref[name])
        print(f"  {name}: rel-L2 {err:.2e}", flush=True)
        assert err <= TOL_F32
