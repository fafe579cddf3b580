"""gdr_chunk_bwd_noalloc, the backward for callers that cannot allocate device memory (its
workspace is the library's own scratch array), against gdr_chunk_bwd with a caller-owned
workspace: the same kernels on the same inputs, so the gradients must be bit-identical.  Two
calls in a row share the scratch array, the second on a smaller input."""
import numpy as np
import pytest

import gdr_synth as gs
from _gpu_util import dev

pytestmark = pytest.mark.gpu


def _bwd(s, x, cot, S0, noalloc):
    import torch
    import chunked_gated_delta_gdr_amd as G
    io = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    f32 = torch.float32
    pc = s.wkey == "precond"
    g = G.gdr_chunk_bwd(dev(x["q"], io), dev(x["k"], io), dev(x["v"], io), dev(cot["d_out"], io),
                        beta=dev(x.get("beta"), f32), log_alpha=dev(x.get("log_alpha"), f32),
                        precond=pc, pc_rho=s.pc_rho, pc_eps=s.pc_eps, pc_h0=s.pc_h0,
                        state_in=dev(S0), d_state_out=dev(cot["d_state_out"]), chunk=s.chunk, noalloc=noalloc)
    torch.cuda.synchronize()
    return g


def test_noalloc_backward_matches_workspace_backward():
    import torch
    import chunked_gated_delta_gdr_amd as G
    cap = G.gdr_chunk_bwd_noalloc_max_workspace()
    cases = [gs.spec("gdn", B=1, H=4, T=3000, seed=91),                                       # 55 MB of scratch
             gs.spec("pdn", B=2, H=1, T=333, Dk=64, Dv=48, dtype="f32", seed=92)]             # smaller, second
    for s in cases:
        desc = G.make_desc(B=s.B, T=s.T, H=s.H, Dk=s.Dk, Dv=s.Dv, chunk=s.chunk,
                           io_dtype=G.GDR_BF16 if s.dtype == "bf16" else G.GDR_F32,
                           decay=G.GDR_DECAY_SCALAR if s.decay == "scalar" else G.GDR_DECAY_NONE,
                           wkey=G.GDR_WKEY_DIAG_PRECOND if s.wkey == "precond" else G.GDR_WKEY_SAME)
        need = G.gdr_chunk_bwd_workspace_size(desc)
        print(f"\n[case] noalloc backward {s.name} B{s.B} H{s.H} T{s.T} Dk{s.Dk} Dv{s.Dv} {s.dtype}: "
              f"workspace {need} of {cap} bytes", flush=True)
        assert 0 < need <= cap
        x, cot = gs.make_inputs(s), gs.make_cotangents(s)
        S0 = (0.2 * np.random.default_rng(s.seed).standard_normal((s.B, s.H, s.Dv, s.Dk))).astype(np.float32)
        ref = _bwd(s, x, cot, S0, noalloc=False)
        got = _bwd(s, x, cot, S0, noalloc=True)
        assert sorted(got) == sorted(ref)
        for name in ref:
            assert torch.equal(got[name], ref[name]), name
