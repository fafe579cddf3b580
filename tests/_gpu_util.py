"""Helpers shared by the GPU tests: move seeded inputs to the device, call the library
through its binding, and bring results back as fp64 numpy arrays."""
import numpy as np

TOL_F32 = 1e-4    # rel-L2 bound of the fp32 path
TOL_BF16 = 2e-2   # rel-L2 bound of the bf16 path


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def dev(x, dtype=None):
    """numpy float32 (bf16-representable when dtype is bf16) -> device tensor, exactly."""
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")
    return t if dtype is None else t.to(dtype)


def host(t):
    import torch
    return None if t is None else t.detach().to(torch.float64).cpu().numpy()


def precond_opts(s):
    return dict(rho=s.pc_rho, eps=s.pc_eps, h0=s.pc_h0, t0=0) if s.wkey == "precond" else None


def run_chunk(s, x, *, state_in=None, pc_h_in=None, pc_t0=0, neumann_order=-1, residual_steps=0,
              impl="auto", scale=1.0, chunk=None, sync=True, workspace=False):
    """gdr_chunk_fwd on inputs ``x`` (numpy, from gdr_synth).  Returns torch tensors.
    ``workspace``: call gdr_chunk_fwd_ws with a workspace above every layout it may need (64 KB
    per (batch, head, chunk of 64 tokens) for T or the per-channel decay's operands and records,
    plus the sequence split's q~ and three states), filled with garbage first (its contents on
    entry must not matter)."""
    import torch
    import chunked_gated_delta_gdr_amd as G
    io = torch_dtype(s.dtype)
    f32 = torch.float32
    ws = None
    if workspace:
        nch = (s.T + 63) // 64
        nbytes = s.B * s.H * nch * 65536 + s.B * s.T * s.H * 256 + s.B * s.H * 3 * 65536 + 2048
        ws = torch.full((nbytes,), 0x7f, dtype=torch.uint8, device="cuda")
    out = G.gdr_chunk_fwd(
        dev(x["q"], io), dev(x["k"], io), dev(x["v"], io),
        beta=dev(x.get("beta"), f32), log_alpha=dev(x.get("log_alpha"), f32),
        erase=dev(x.get("erase"), io), write=dev(x.get("write"), io),
        write_key=dev(x.get("write_key"), io),
        precond=s.wkey == "precond", pc_h_in=dev(pc_h_in, f32), pc_rho=s.pc_rho, pc_eps=s.pc_eps,
        pc_h0=s.pc_h0, pc_t0=pc_t0,
        state_in=dev(state_in, f32), chunk=chunk or s.chunk, neumann_order=neumann_order,
        residual_steps=residual_steps,
        scale=scale, impl=impl, workspace=ws)
    if sync:
        torch.cuda.synchronize()
    return out
