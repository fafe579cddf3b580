"""ctypes binding of libgdr.so: same names as the C ABI in include/gdr.h."""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))

GDR_OK, GDR_EINVAL, GDR_ENOTSUP, GDR_EHIP = 0, 1, 2, 3
GDR_F32, GDR_BF16 = 0, 1
GDR_GAIN_SCALAR, GDR_GAIN_CHANNEL = 0, 1
GDR_DECAY_NONE, GDR_DECAY_SCALAR, GDR_DECAY_CHANNEL = 0, 1, 2
GDR_WKEY_SAME, GDR_WKEY_DIAG_PRECOND, GDR_WKEY_EXPLICIT = 0, 1, 2
GDR_IMPL_AUTO, GDR_IMPL_GENERIC, GDR_IMPL_MFMA = 0, 1, 2
_IMPL = {"auto": GDR_IMPL_AUTO, "generic": GDR_IMPL_GENERIC, "mfma": GDR_IMPL_MFMA}


class gdr_desc_t(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32), ("gain", ctypes.c_int32), ("decay", ctypes.c_int32),
        ("wkey", ctypes.c_int32),
        ("neumann_order", ctypes.c_int32), ("residual_steps", ctypes.c_int32), ("impl", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("pc_rho", ctypes.c_float), ("pc_eps", ctypes.c_float), ("pc_h0", ctypes.c_float),
        ("pc_t0", ctypes.c_int64),
    ]


class gdr_inputs_t(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("beta", ctypes.c_void_p), ("log_alpha", ctypes.c_void_p),
        ("erase", ctypes.c_void_p), ("write", ctypes.c_void_p),
        ("write_key", ctypes.c_void_p),
        ("pc_h_in", ctypes.c_void_p), ("pc_h_out", ctypes.c_void_p),
    ]


class gdr_grads_t(ctypes.Structure):
    _fields_ = [
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("dbeta", ctypes.c_void_p), ("derase", ctypes.c_void_p), ("dwrite", ctypes.c_void_p),
        ("dlog_alpha", ctypes.c_void_p), ("dwrite_key", ctypes.c_void_p),
        ("dstate_in", ctypes.c_void_p), ("dpc_h_in", ctypes.c_void_p),
    ]


class GdrError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{gdr_status_str(status)}: {msg}")
        self.status = status


_LIB = None


def lib_path() -> str:
    return os.path.join(PKG, "libgdr.so")


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        p = lib_path()
        if not os.path.exists(p):
            raise ImportError(f"{p} is missing: build it with `python -m chunked_gated_delta_gdr_amd.build` "
                              "(there is no fallback implementation)")
        L = ctypes.CDLL(p)
        P = ctypes.POINTER
        L.gdr_chunk_fwd.argtypes = [P(gdr_desc_t), P(gdr_inputs_t), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]
        L.gdr_chunk_fwd.restype = ctypes.c_int
        L.gdr_recurrent_step.argtypes = [P(gdr_desc_t), P(gdr_inputs_t), ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]
        L.gdr_recurrent_step.restype = ctypes.c_int
        L.gdr_validate.argtypes = [P(gdr_desc_t), P(gdr_inputs_t), ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_int]
        L.gdr_validate.restype = ctypes.c_int
        L.gdr_chunk_bwd.argtypes = [P(gdr_desc_t), P(gdr_inputs_t), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, P(gdr_grads_t), ctypes.c_void_p, ctypes.c_uint64,
                                    ctypes.c_void_p]
        L.gdr_chunk_bwd.restype = ctypes.c_int
        L.gdr_chunk_bwd_noalloc.argtypes = [P(gdr_desc_t), P(gdr_inputs_t), ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, P(gdr_grads_t), ctypes.c_void_p]
        L.gdr_chunk_bwd_noalloc.restype = ctypes.c_int
        L.gdr_chunk_bwd_noalloc_max_workspace.argtypes = []
        L.gdr_chunk_bwd_noalloc_max_workspace.restype = ctypes.c_uint64
        L.gdr_chunk_bwd_workspace_size.argtypes = [P(gdr_desc_t)]
        L.gdr_chunk_bwd_workspace_size.restype = ctypes.c_uint64
        L.gdr_validate_bwd.argtypes = [P(gdr_desc_t), P(gdr_inputs_t), ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, P(gdr_grads_t), ctypes.c_void_p, ctypes.c_uint64]
        L.gdr_validate_bwd.restype = ctypes.c_int
        L.gdr_chunk_fwd_impl.argtypes = [P(gdr_desc_t)]
        L.gdr_chunk_fwd_impl.restype = ctypes.c_int
        L.gdr_chunk_fwd_ws.argtypes = [P(gdr_desc_t), P(gdr_inputs_t), ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
        L.gdr_chunk_fwd_ws.restype = ctypes.c_int
        L.gdr_chunk_fwd_workspace_size.argtypes = [P(gdr_desc_t)]
        L.gdr_chunk_fwd_workspace_size.restype = ctypes.c_uint64
        L.gdr_status_str.argtypes = [ctypes.c_int]
        L.gdr_status_str.restype = ctypes.c_char_p
        L.gdr_last_error.argtypes = []
        L.gdr_last_error.restype = ctypes.c_char_p
        L.gdr_abi_version.argtypes = []
        L.gdr_abi_version.restype = ctypes.c_int
        if L.gdr_abi_version() != 5:
            raise ImportError("libgdr ABI version mismatch")
        _LIB = L
    return _LIB


def gdr_status_str(status: int) -> str:
    return lib().gdr_status_str(status).decode()


def gdr_last_error() -> str:
    return lib().gdr_last_error().decode()


def gdr_abi_version() -> int:
    return lib().gdr_abi_version()


def make_desc(*, B, T, H, Dk, Dv, chunk=64, io_dtype=GDR_BF16, gain=GDR_GAIN_SCALAR,
              decay=GDR_DECAY_NONE, wkey=GDR_WKEY_SAME, neumann_order=-1, residual_steps=0,
              impl=GDR_IMPL_AUTO, scale=1.0, pc_rho=0.99, pc_eps=1e-3, pc_h0=1.0,
              pc_t0=0) -> gdr_desc_t:
    return gdr_desc_t(ctypes.sizeof(gdr_desc_t), B, T, H, Dk, Dv, chunk, io_dtype, gain, decay, wkey,
                      neumann_order, residual_steps, impl, scale, pc_rho, pc_eps, pc_h0, pc_t0)


def gdr_validate(desc: gdr_desc_t, inputs: gdr_inputs_t, state_in=None, out=None, state_out=None,
                 for_step: bool = False) -> int:
    """Host-side argument check (no HIP call).  Pointers are ints or None."""
    return lib().gdr_validate(ctypes.byref(desc), ctypes.byref(inputs), state_in, out, state_out,
                              int(for_step))


def gdr_chunk_bwd_workspace_size(desc: gdr_desc_t) -> int:
    return int(lib().gdr_chunk_bwd_workspace_size(ctypes.byref(desc)))


def gdr_chunk_bwd_noalloc_max_workspace() -> int:
    return int(lib().gdr_chunk_bwd_noalloc_max_workspace())


def gdr_validate_bwd(desc: gdr_desc_t, inputs: gdr_inputs_t, state_in=None, d_out=None,
                     d_state_out=None, grads: Optional[gdr_grads_t] = None, workspace=None,
                     workspace_bytes: int = 0) -> int:
    """gdr_chunk_bwd's host-side argument check (no HIP call).  Pointers are ints or None."""
    g = grads if grads is not None else gdr_grads_t()
    return lib().gdr_validate_bwd(ctypes.byref(desc), ctypes.byref(inputs), state_in, d_out, d_state_out,
                                  ctypes.byref(g), workspace, workspace_bytes)


def gdr_chunk_fwd_impl(desc: gdr_desc_t) -> int:
    return lib().gdr_chunk_fwd_impl(ctypes.byref(desc))


# ------------------------------------------------------------------------------------
# torch marshalling
# ------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(name, t, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: device {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _io_code(dtype) -> int:
    torch = _torch()
    if dtype == torch.float32:
        return GDR_F32
    if dtype == torch.bfloat16:
        return GDR_BF16
    raise TypeError(f"unsupported io dtype {dtype} (float32 or bfloat16)")


def _stream(stream, device) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _raise(status: int):
    if status != GDR_OK:
        raise GdrError(status, gdr_last_error())


def gdr_chunk_fwd(q, k, v, *, beta=None, log_alpha=None, erase=None, write=None, write_key=None,
                  precond: bool = False, pc_h_in=None, pc_h_out=None, pc_rho: float = 0.99,
                  pc_eps: float = 1e-3, pc_h0: float = 1.0, pc_t0: int = 0,
                  state_in=None, out=None, state_out=None, return_state: bool = True,
                  chunk: int = 64, neumann_order: int = -1, residual_steps: int = 0,
                  scale: float = 1.0, impl: str = "auto", workspace=None,
                  stream=None) -> Tuple[object, object, object]:
    """Chunked forward on torch tensors (q, k, v [B, T, H, D]).  Returns (out, state_out, pc_h_out).

    Gains: ``beta`` [B, T, H] fp32, or ``erase`` [B, T, H, Dk] and ``write`` [B, T, H, Dv].
    Decay: ``log_alpha`` [B, T, H] fp32 (one per token), [B, T, H, Dk] fp32 (one per key
    channel) or None.  Write key: ``write_key`` [B, T, H, Dk],
    or ``precond=True`` for the diagonal preconditioner (accumulator ``pc_h_in`` [B, H, Dk]
    fp32 or None for ``pc_h0``).  T: exact (``neumann_order`` < 0), the band N
    (``neumann_order`` = N), or that band corrected by ``residual_steps`` residual steps.
    Outputs are allocated when not given; ``state_out`` is allocated only if ``return_state``.
    ``workspace``: a uint8 device tensor of at least ``gdr_chunk_fwd_workspace_size(desc)``
    bytes (gdr_chunk_fwd_ws: T of every chunk formed first, where that applies), or None.
    """
    torch = _torch()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    io = q.dtype
    _io_code(io)
    f32 = torch.float32
    _check("q", q, (B, T, H, Dk), io, dev)
    _check("k", k, (B, T, H, Dk), io, dev)
    _check("v", v, (B, T, H, Dv), io, dev)
    _check("beta", beta, (B, T, H), f32, dev)
    chd = log_alpha is not None and log_alpha.dim() == 4
    _check("log_alpha", log_alpha, (B, T, H, Dk) if chd else (B, T, H), f32, dev)
    _check("erase", erase, (B, T, H, Dk), io, dev)
    _check("write", write, (B, T, H, Dv), io, dev)
    _check("write_key", write_key, (B, T, H, Dk), io, dev)
    _check("state_in", state_in, (B, H, Dv, Dk), f32, dev)
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=io, device=dev)
    _check("out", out, (B, T, H, Dv), io, dev)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, Dv, Dk), dtype=f32, device=dev)
    _check("state_out", state_out, (B, H, Dv, Dk), f32, dev)
    if precond:
        _check("pc_h_in", pc_h_in, (B, H, Dk), f32, dev)
        if pc_h_out is None:
            pc_h_out = torch.empty((B, H, Dk), dtype=f32, device=dev)
        _check("pc_h_out", pc_h_out, (B, H, Dk), f32, dev)
    desc = make_desc(B=B, T=T, H=H, Dk=Dk, Dv=Dv, chunk=chunk, io_dtype=_io_code(io),
                     gain=GDR_GAIN_CHANNEL if erase is not None else GDR_GAIN_SCALAR,
                     decay=(GDR_DECAY_CHANNEL if chd else
                            GDR_DECAY_SCALAR if log_alpha is not None else GDR_DECAY_NONE),
                     wkey=(GDR_WKEY_DIAG_PRECOND if precond else
                           GDR_WKEY_EXPLICIT if write_key is not None else GDR_WKEY_SAME),
                     neumann_order=neumann_order, residual_steps=residual_steps,
                     impl=_IMPL[impl], scale=scale,
                     pc_rho=pc_rho, pc_eps=pc_eps, pc_h0=pc_h0, pc_t0=pc_t0)
    ins = gdr_inputs_t(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha), _ptr(erase), _ptr(write),
                       _ptr(write_key), _ptr(pc_h_in) if precond else None,
                       _ptr(pc_h_out) if precond else None)
    if workspace is None:
        st = lib().gdr_chunk_fwd(ctypes.byref(desc), ctypes.byref(ins), _ptr(state_in), _ptr(out),
                                 _ptr(state_out), _stream(stream, dev))
    else:
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the inputs' device")
        st = lib().gdr_chunk_fwd_ws(ctypes.byref(desc), ctypes.byref(ins), _ptr(state_in), _ptr(out),
                                    _ptr(state_out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream, dev))
    _raise(st)
    return out, state_out, (pc_h_out if precond else None)


def gdr_chunk_fwd_workspace_size(desc) -> int:
    """Bytes of gdr_chunk_fwd_ws's workspace for a descriptor (0 where it does not apply)."""
    return int(lib().gdr_chunk_fwd_workspace_size(ctypes.byref(desc)))


def gdr_recurrent_step(q, k, v, state, *, beta=None, log_alpha=None, erase=None, write=None,
                       write_key=None, precond: bool = False, pc_h_in=None, pc_h_out=None,
                       pc_rho: float = 0.99, pc_eps: float = 1e-3, pc_h0: float = 1.0, pc_t0: int = 0,
                       out=None, scale: float = 1.0, stream=None):
    """One decode token for every stream: q, k [B, H, Dk], v [B, H, Dv], state [B, H, Dv, Dk]
    fp32 updated in place.  Returns (out [B, H, Dv], pc_h_out)."""
    torch = _torch()
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    io = q.dtype
    f32 = torch.float32
    _io_code(io)
    _check("q", q, (B, H, Dk), io, dev)
    _check("k", k, (B, H, Dk), io, dev)
    _check("v", v, (B, H, Dv), io, dev)
    _check("beta", beta, (B, H), f32, dev)
    chd = log_alpha is not None and log_alpha.dim() == 3
    _check("log_alpha", log_alpha, (B, H, Dk) if chd else (B, H), f32, dev)
    _check("erase", erase, (B, H, Dk), io, dev)
    _check("write", write, (B, H, Dv), io, dev)
    _check("write_key", write_key, (B, H, Dk), io, dev)
    _check("state", state, (B, H, Dv, Dk), f32, dev)
    if out is None:
        out = torch.empty((B, H, Dv), dtype=io, device=dev)
    _check("out", out, (B, H, Dv), io, dev)
    if precond:
        _check("pc_h_in", pc_h_in, (B, H, Dk), f32, dev)
        if pc_h_out is None:
            pc_h_out = pc_h_in if pc_h_in is not None else torch.empty((B, H, Dk), dtype=f32, device=dev)
        _check("pc_h_out", pc_h_out, (B, H, Dk), f32, dev)
    desc = make_desc(B=B, T=1, H=H, Dk=Dk, Dv=Dv, chunk=64, io_dtype=_io_code(io),
                     gain=GDR_GAIN_CHANNEL if erase is not None else GDR_GAIN_SCALAR,
                     decay=(GDR_DECAY_CHANNEL if chd else
                            GDR_DECAY_SCALAR if log_alpha is not None else GDR_DECAY_NONE),
                     wkey=(GDR_WKEY_DIAG_PRECOND if precond else
                           GDR_WKEY_EXPLICIT if write_key is not None else GDR_WKEY_SAME),
                     scale=scale, pc_rho=pc_rho, pc_eps=pc_eps, pc_h0=pc_h0, pc_t0=pc_t0)
    ins = gdr_inputs_t(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha), _ptr(erase), _ptr(write),
                       _ptr(write_key), _ptr(pc_h_in) if precond else None,
                       _ptr(pc_h_out) if precond else None)
    st = lib().gdr_recurrent_step(ctypes.byref(desc), ctypes.byref(ins), _ptr(state), _ptr(out),
                                  _stream(stream, dev))
    _raise(st)
    return out, (pc_h_out if precond else None)


def gdr_chunk_bwd(q, k, v, d_out, *, beta=None, log_alpha=None, erase=None, write=None,
                  write_key=None, precond: bool = False, pc_h_in=None, pc_rho: float = 0.99,
                  pc_eps: float = 1e-3, pc_h0: float = 1.0, pc_t0: int = 0,
                  state_in=None, d_state_out=None, want_dstate_in: bool = True,
                  chunk: int = 64, neumann_order: int = -1, scale: float = 1.0, workspace=None,
                  stream=None, noalloc: bool = False) -> dict:
    """Gradients through ``gdr_chunk_fwd`` on torch tensors.  ``d_out`` [B, T, H, Dv] (io dtype)
    and ``d_state_out`` [B, H, Dv, Dk] fp32 (or None) are the loss gradients of the forward's
    outputs.  Returns a dict of fp32 tensors: dq, dk, dv, and as the variant has them dbeta |
    derase, dwrite, dlog_alpha, dwrite_key, dpc_h_in (``precond``), and dstate_in (if
    ``want_dstate_in``).  ``neumann_order`` = N >= 0 differentiates the forward with the
    band-limited T.  The workspace (uint8, gdr_chunk_bwd_workspace_size bytes) is allocated
    when not given.  ``noalloc`` calls gdr_chunk_bwd_noalloc instead, whose workspace is the
    library's own scratch array (no workspace argument; the gradient tensors are still
    allocated here unless the caller marshals the C call itself)."""
    torch = _torch()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    io = q.dtype
    f32 = torch.float32
    _io_code(io)
    _check("q", q, (B, T, H, Dk), io, dev)
    _check("k", k, (B, T, H, Dk), io, dev)
    _check("v", v, (B, T, H, Dv), io, dev)
    _check("d_out", d_out, (B, T, H, Dv), io, dev)
    _check("beta", beta, (B, T, H), f32, dev)
    chd = log_alpha is not None and log_alpha.dim() == 4
    _check("log_alpha", log_alpha, (B, T, H, Dk) if chd else (B, T, H), f32, dev)
    _check("erase", erase, (B, T, H, Dk), io, dev)
    _check("write", write, (B, T, H, Dv), io, dev)
    _check("write_key", write_key, (B, T, H, Dk), io, dev)
    _check("state_in", state_in, (B, H, Dv, Dk), f32, dev)
    _check("d_state_out", d_state_out, (B, H, Dv, Dk), f32, dev)
    if precond:
        _check("pc_h_in", pc_h_in, (B, H, Dk), f32, dev)
    desc = make_desc(B=B, T=T, H=H, Dk=Dk, Dv=Dv, chunk=chunk, io_dtype=_io_code(io),
                     gain=GDR_GAIN_CHANNEL if erase is not None else GDR_GAIN_SCALAR,
                     decay=(GDR_DECAY_CHANNEL if chd else
                            GDR_DECAY_SCALAR if log_alpha is not None else GDR_DECAY_NONE),
                     wkey=(GDR_WKEY_DIAG_PRECOND if precond else
                           GDR_WKEY_EXPLICIT if write_key is not None else GDR_WKEY_SAME),
                     scale=scale, impl=GDR_IMPL_GENERIC, neumann_order=neumann_order,
                     pc_rho=pc_rho, pc_eps=pc_eps, pc_h0=pc_h0, pc_t0=pc_t0)

    def new(shape):
        return torch.empty(shape, dtype=f32, device=dev)

    g = {"dq": new((B, T, H, Dk)), "dk": new((B, T, H, Dk)), "dv": new((B, T, H, Dv))}
    if erase is not None:
        g["derase"] = new((B, T, H, Dk))
        g["dwrite"] = new((B, T, H, Dv))
    else:
        g["dbeta"] = new((B, T, H))
    if log_alpha is not None:
        g["dlog_alpha"] = new((B, T, H, Dk) if chd else (B, T, H))
    if write_key is not None:
        g["dwrite_key"] = new((B, T, H, Dk))
    if want_dstate_in:
        g["dstate_in"] = new((B, H, Dv, Dk))
    if precond:
        g["dpc_h_in"] = new((B, H, Dk))
    grads = gdr_grads_t(*[_ptr(g.get(name)) for name, _ in gdr_grads_t._fields_])
    ins = gdr_inputs_t(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha), _ptr(erase), _ptr(write),
                       _ptr(write_key), _ptr(pc_h_in) if precond else None, None)
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc takes no workspace")
        st = lib().gdr_chunk_bwd_noalloc(ctypes.byref(desc), ctypes.byref(ins), _ptr(state_in), _ptr(d_out),
                                         _ptr(d_state_out), ctypes.byref(grads), _stream(stream, dev))
        _raise(st)
        return g
    nbytes = gdr_chunk_bwd_workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, need {nbytes}")
    st = lib().gdr_chunk_bwd(ctypes.byref(desc), ctypes.byref(ins), _ptr(state_in), _ptr(d_out),
                             _ptr(d_state_out), ctypes.byref(grads), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream, dev))
    _raise(st)
    return g
