"""The C ABI without a GPU: the library loads, exports what include/gdr.h declares, and
rejects malformed calls on the host before anything is launched."""
import ctypes
import os
import re

import pytest

import chunked_gated_delta_gdr_amd as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")

BASE = 1 << 32          # fake, well-aligned, disjoint "device addresses" (never dereferenced)
MB = 1 << 26


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert {"gdr_chunk_fwd", "gdr_recurrent_step", "gdr_validate", "gdr_status_str",
            "gdr_last_error", "gdr_abi_version", "gdr_chunk_fwd_impl"} <= set(names)
    L = G.lib()
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    assert G.gdr_abi_version() == 5
    for s in (G.GDR_OK, G.GDR_EINVAL, G.GDR_ENOTSUP, G.GDR_EHIP):
        assert G.gdr_status_str(s).startswith("GDR_")
    assert "UNKNOWN" in G.gdr_status_str(42)


def test_struct_layout_matches_header():
    # uint32 + 13 int32 + 4 float = 72 bytes, then the int64: 80
    assert ctypes.sizeof(G.gdr_desc_t) == 80
    assert ctypes.sizeof(G.gdr_inputs_t) == 10 * 8
    assert ctypes.sizeof(G.gdr_grads_t) == 10 * 8


def desc(**kw):
    d = dict(B=2, T=100, H=3, Dk=64, Dv=32, chunk=64, io_dtype=G.GDR_BF16)
    d.update(kw)
    return G.make_desc(**d)


def ptrs(n=10):
    return [BASE + i * MB for i in range(n)]


def inputs(**kw):
    p = ptrs()
    d = dict(q=p[0], k=p[1], v=p[2], beta=p[3])
    d.update(kw)
    return G.gdr_inputs_t(**d)


OUT, SIN, SOUT = BASE + 20 * MB, BASE + 21 * MB, BASE + 22 * MB


def check(expect, d=None, ins=None, state_in=None, out=OUT, state_out=SOUT, for_step=False):
    d = d or desc()
    ins = ins or inputs()
    st = G.gdr_validate(d, ins, state_in, out, state_out, for_step)
    assert st == expect, (st, G.gdr_last_error())
    if expect != G.GDR_OK:
        assert G.gdr_last_error() != ""
    return st


def test_valid_call_validates():
    check(G.GDR_OK)
    check(G.GDR_OK, state_in=SIN)
    check(G.GDR_OK, state_in=SOUT)                 # in-place state
    check(G.GDR_OK, state_out=None)
    check(G.GDR_OK, d=desc(T=0), ins=inputs(q=None, k=None, v=None, beta=None), out=None)
    assert G.gdr_last_error() == ""


@pytest.mark.parametrize("field,value,status", [
    ("struct_size", 12, G.GDR_EINVAL),
    ("B", 0, G.GDR_EINVAL), ("H", 0, G.GDR_EINVAL), ("T", -1, G.GDR_EINVAL),
    ("Dk", 0, G.GDR_EINVAL), ("Dv", 0, G.GDR_EINVAL),
    ("Dk", 256, G.GDR_ENOTSUP), ("Dv", 1024, G.GDR_ENOTSUP),
    ("chunk", 0, G.GDR_EINVAL), ("chunk", 256, G.GDR_ENOTSUP), ("chunk", 48, G.GDR_ENOTSUP),
    ("io_dtype", 7, G.GDR_EINVAL), ("gain", 5, G.GDR_EINVAL), ("decay", 3, G.GDR_EINVAL),
    ("wkey", 9, G.GDR_EINVAL), ("impl", 4, G.GDR_EINVAL),
    ("scale", float("nan"), G.GDR_EINVAL), ("scale", float("inf"), G.GDR_EINVAL),
])
def test_bad_descriptor(field, value, status):
    d = desc()
    setattr(d, field, value)
    check(status, d=d)


@pytest.mark.parametrize("N,S,status", [(-1, 1, G.GDR_EINVAL), (3, -1, G.GDR_EINVAL),
                                        (3, 65, G.GDR_ENOTSUP), (3, 8, G.GDR_OK), (-1, 0, G.GDR_OK)])
def test_residual_steps(N, S, status):
    check(status, d=desc(neumann_order=N, residual_steps=S))


def test_channel_decay_descriptor():
    p = ptrs()
    check(G.GDR_EINVAL, d=desc(decay=G.GDR_DECAY_CHANNEL))                     # no log_alpha
    check(G.GDR_OK, d=desc(decay=G.GDR_DECAY_CHANNEL), ins=inputs(log_alpha=p[4]))
    check(G.GDR_EINVAL, d=desc(decay=G.GDR_DECAY_CHANNEL), ins=inputs(log_alpha=p[4]),
          out=p[4] + 2 * 100 * 3 * 4)   # out inside the [B, T, H, Dk] fp32 gates (not [B, T, H])
    check(G.GDR_ENOTSUP, d=desc(decay=G.GDR_DECAY_CHANNEL, neumann_order=3, residual_steps=2),
          ins=inputs(log_alpha=p[4]))
    d = desc(Dk=128, Dv=128, decay=G.GDR_DECAY_CHANNEL)
    assert G.gdr_chunk_fwd_impl(d) == G.GDR_IMPL_GENERIC


def test_residual_correction_kernels():
    """The residual-corrected T runs on the matrix-core kernel at chunk 64 (bf16, d = 128) and on
    the generic kernel otherwise."""
    d = desc(Dk=128, Dv=128, neumann_order=3, residual_steps=8)
    assert G.gdr_chunk_fwd_impl(d) == G.GDR_IMPL_MFMA
    d.impl = G.GDR_IMPL_GENERIC
    assert G.gdr_chunk_fwd_impl(d) == G.GDR_IMPL_GENERIC
    d = desc(Dk=128, Dv=128, neumann_order=3, residual_steps=8, chunk=32)
    assert G.gdr_chunk_fwd_impl(d) == G.GDR_IMPL_GENERIC
    d = desc(Dk=128, Dv=128, neumann_order=3, residual_steps=8, io_dtype=G.GDR_F32)
    assert G.gdr_chunk_fwd_impl(d) == G.GDR_IMPL_GENERIC


@pytest.mark.parametrize("N,S,decay,status", [
    (-1, 0, G.GDR_DECAY_SCALAR, G.GDR_OK), (-1, 0, G.GDR_DECAY_CHANNEL, G.GDR_OK),
    (0, 0, G.GDR_DECAY_SCALAR, G.GDR_OK), (3, 0, G.GDR_DECAY_NONE, G.GDR_OK), (15, 0, G.GDR_DECAY_SCALAR, G.GDR_OK),
    (16, 0, G.GDR_DECAY_SCALAR, G.GDR_ENOTSUP), (126, 0, G.GDR_DECAY_NONE, G.GDR_ENOTSUP),
    (127, 0, G.GDR_DECAY_CHANNEL, G.GDR_OK), (500, 0, G.GDR_DECAY_SCALAR, G.GDR_OK),
    (3, 0, G.GDR_DECAY_CHANNEL, G.GDR_ENOTSUP), (3, 8, G.GDR_DECAY_SCALAR, G.GDR_ENOTSUP),
    (127, 2, G.GDR_DECAY_NONE, G.GDR_ENOTSUP)])
def test_chunk128_descriptor(N, S, decay, status):
    """Chunk 128: exact T (or N >= 127) for every variant; a band limit N <= 15 with scalar or no
    decay; nothing else."""
    p = ptrs()
    la = p[4] if decay != G.GDR_DECAY_NONE else None
    check(status, d=desc(chunk=128, neumann_order=N, residual_steps=S, decay=decay), ins=inputs(log_alpha=la))


def test_chunk128_kernel_choice():
    """The exact T at chunk 128 is the chunk-64 computation regrouped, so it keeps the
    matrix-core kernel; the band-limited T at chunk 128 runs on the fp32 kernel only."""
    assert G.gdr_chunk_fwd_impl(desc(Dk=128, Dv=128, chunk=128)) == G.GDR_IMPL_MFMA
    assert G.gdr_chunk_fwd_impl(desc(Dk=128, Dv=128, chunk=128, neumann_order=200)) == G.GDR_IMPL_MFMA
    assert G.gdr_chunk_fwd_impl(desc(Dk=128, Dv=128, chunk=128, neumann_order=3)) == G.GDR_IMPL_GENERIC
    assert G.gdr_chunk_fwd_impl(desc(Dk=128, Dv=128, chunk=128, neumann_order=3, impl=G.GDR_IMPL_MFMA)) == -1


def test_chunk128_backward():
    """The backward at chunk 128 takes the exact T (its workspace is chunk 64's) and rejects
    the band-limited one."""
    assert G.gdr_chunk_bwd_workspace_size(desc(chunk=128)) == G.gdr_chunk_bwd_workspace_size(desc(chunk=64))
    assert G.gdr_chunk_bwd_workspace_size(desc(chunk=128, neumann_order=3)) == 0
    assert call_validate_bwd(desc(chunk=128)) == G.GDR_OK, G.gdr_last_error()
    d = desc(chunk=128, neumann_order=3)
    ins, gr, a = bwd_args(d)
    assert G.gdr_validate_bwd(d, ins, None, a["d_out"], None, gr, a["workspace"], 1 << 30) == G.GDR_ENOTSUP
    assert "chunk 128" in G.gdr_last_error()


def test_huge_problem_rejected():
    check(G.GDR_ENOTSUP, d=desc(B=1 << 20, T=1 << 20, H=1 << 10))


def test_stream_count_bound():
    """At most 2^19 (batch, head) streams: every launch grid stays within 2^32 work-items and
    the kernels' workgroup indices within 2^24, whatever the head dims."""
    check(G.GDR_OK, d=desc(B=1 << 9, H=1 << 10, T=1, Dk=1, Dv=1))
    check(G.GDR_ENOTSUP, d=desc(B=(1 << 9) + 1, H=1 << 10, T=1, Dk=1, Dv=1))
    assert "streams" in G.gdr_last_error()
    check(G.GDR_ENOTSUP, d=desc(B=65535, H=65535, T=1, Dk=1, Dv=1))


def test_bwd_chunk_count_bound():
    """The backward's per-chunk kernels put the chunks on the grid's x axis: at most 2^22."""
    far = [BASE + i * (1 << 36) for i in range(30)]   # disjoint for tensors up to 64 GiB

    def validate(T):
        d = desc(B=1, H=1, T=T, Dk=1, Dv=1, chunk=16)
        ins = G.gdr_inputs_t(q=far[0], k=far[1], v=far[2], beta=far[3])
        gr = G.gdr_grads_t(dq=far[10], dk=far[11], dv=far[12], dbeta=far[13], dstate_in=far[19])
        return G.lib().gdr_validate_bwd(ctypes.byref(d), ctypes.byref(ins), None, far[9], None, ctypes.byref(gr),
                                        far[24], G.gdr_chunk_bwd_workspace_size(d))

    assert validate((1 << 22) * 16) == G.GDR_OK, G.gdr_last_error()
    assert validate((1 << 22) * 16 + 1) == G.GDR_ENOTSUP
    assert "chunks" in G.gdr_last_error()


def test_pointer_consistency_with_variant():
    p = ptrs()
    check(G.GDR_EINVAL, ins=inputs(beta=None))                                   # gain scalar, no beta
    check(G.GDR_EINVAL, ins=inputs(q=None))
    check(G.GDR_EINVAL, ins=inputs(erase=p[5], write=p[6]))                     # gates with scalar gain
    check(G.GDR_EINVAL, d=desc(gain=G.GDR_GAIN_CHANNEL), ins=inputs(erase=p[5], write=p[6]))  # beta too
    check(G.GDR_OK, d=desc(gain=G.GDR_GAIN_CHANNEL), ins=inputs(beta=None, erase=p[5], write=p[6]))
    check(G.GDR_EINVAL, d=desc(gain=G.GDR_GAIN_CHANNEL), ins=inputs(beta=None, erase=p[5]))
    check(G.GDR_EINVAL, d=desc(decay=G.GDR_DECAY_SCALAR))                       # no log_alpha
    check(G.GDR_OK, d=desc(decay=G.GDR_DECAY_SCALAR), ins=inputs(log_alpha=p[4]))
    check(G.GDR_EINVAL, ins=inputs(log_alpha=p[4]))                             # log_alpha, no decay
    check(G.GDR_EINVAL, d=desc(wkey=G.GDR_WKEY_EXPLICIT))
    check(G.GDR_OK, d=desc(wkey=G.GDR_WKEY_EXPLICIT), ins=inputs(write_key=p[7]))
    check(G.GDR_EINVAL, ins=inputs(write_key=p[7]))
    check(G.GDR_EINVAL, ins=inputs(pc_h_in=p[8]))                               # pc_h without precond
    check(G.GDR_OK, d=desc(wkey=G.GDR_WKEY_DIAG_PRECOND), ins=inputs(pc_h_in=p[8], pc_h_out=p[9]))
    check(G.GDR_EINVAL, out=None)


@pytest.mark.parametrize("field,value", [("pc_rho", 1.0), ("pc_rho", 0.0), ("pc_eps", 0.0),
                                         ("pc_h0", -1.0), ("pc_t0", -3)])
def test_bad_precond_constants(field, value):
    d = desc(wkey=G.GDR_WKEY_DIAG_PRECOND)
    setattr(d, field, value)
    check(G.GDR_EINVAL, d=d)


def test_overlaps_rejected():
    p = ptrs()
    check(G.GDR_EINVAL, out=p[0])                                  # out == q
    check(G.GDR_EINVAL, out=p[2] + 64)                             # out inside v
    check(G.GDR_EINVAL, state_out=p[1])                            # state over k
    check(G.GDR_EINVAL, state_in=SOUT + 1024)                      # partial state overlap
    check(G.GDR_EINVAL, state_out=OUT)                             # state over out
    d = desc(wkey=G.GDR_WKEY_DIAG_PRECOND)
    check(G.GDR_EINVAL, d=d, ins=inputs(pc_h_in=p[8], pc_h_out=p[8]))   # chunk_fwd: no in-place h
    # the step allows the in-place accumulator
    ds = desc(T=1, wkey=G.GDR_WKEY_DIAG_PRECOND)
    check(G.GDR_OK, d=ds, ins=inputs(pc_h_in=p[8], pc_h_out=p[8]), for_step=True)


def test_misaligned_rejected():
    p = ptrs()
    check(G.GDR_EINVAL, ins=inputs(q=p[0] + 1))
    check(G.GDR_EINVAL, ins=inputs(beta=p[3] + 2))
    check(G.GDR_OK, d=desc(io_dtype=G.GDR_BF16), ins=inputs(q=p[0] + 2))
    check(G.GDR_EINVAL, d=desc(io_dtype=G.GDR_F32), ins=inputs(q=p[0] + 2))
    check(G.GDR_EINVAL, state_out=SOUT + 2)


def test_step_contract():
    check(G.GDR_OK, d=desc(T=1), for_step=True)
    check(G.GDR_EINVAL, d=desc(T=2), for_step=True)
    check(G.GDR_EINVAL, d=desc(T=1), state_out=None, for_step=True)
    check(G.GDR_EINVAL, d=desc(T=1), out=None, for_step=True)


def test_entry_points_reject_before_launch():
    """With an invalid descriptor the entry points return before any HIP call, so they can
    be called on a host without a GPU."""
    L = G.lib()
    d = desc(B=0)
    ins = inputs()
    assert L.gdr_chunk_fwd(ctypes.byref(d), ctypes.byref(ins), None, OUT, SOUT, None) == G.GDR_EINVAL
    assert "B = 0" in G.gdr_last_error()
    d = desc(T=1, Dk=300)
    assert L.gdr_recurrent_step(ctypes.byref(d), ctypes.byref(ins), SOUT, OUT, None) == G.GDR_ENOTSUP
    assert L.gdr_chunk_fwd(None, None, None, None, None, None) == G.GDR_EINVAL


def test_impl_choice():
    assert G.gdr_chunk_fwd_impl(desc(impl=G.GDR_IMPL_GENERIC)) == G.GDR_IMPL_GENERIC
    assert G.gdr_chunk_fwd_impl(desc(io_dtype=G.GDR_F32)) == G.GDR_IMPL_GENERIC
    assert G.gdr_chunk_fwd_impl(desc(Dk=128, Dv=128)) == G.GDR_IMPL_MFMA
    assert G.gdr_chunk_fwd_impl(desc(Dk=128, Dv=128, chunk=32)) == G.GDR_IMPL_GENERIC
    assert G.gdr_chunk_fwd_impl(desc(Dk=128, Dv=128, impl=G.GDR_IMPL_GENERIC)) == G.GDR_IMPL_GENERIC
    assert G.gdr_chunk_fwd_impl(desc(Dk=64, impl=G.GDR_IMPL_MFMA)) == -1


# ----------------------------------------------------------------------------------
# gdr_chunk_bwd: workspace size and host-side validation
# ----------------------------------------------------------------------------------

def _al(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("decay,wkey", [(G.GDR_DECAY_SCALAR, G.GDR_WKEY_SAME),
                                        (G.GDR_DECAY_CHANNEL, G.GDR_WKEY_SAME),
                                        (G.GDR_DECAY_CHANNEL, G.GDR_WKEY_DIAG_PRECOND)])
@pytest.mark.parametrize("T,C", [(100, 64), (64, 64), (1, 16), (4096, 32), (0, 64)])
def test_bwd_workspace_size_formula(T, C, decay, wkey):
    d = desc(T=T, chunk=C, decay=decay, wkey=wkey)
    B, H, Dk, Dv = 2, 3, 64, 32
    NC = (T + C - 1) // C
    want = (2 * _al(B * H * NC * Dv * Dk * 4) + 3 * _al(B * T * H * Dv * 4) + 2 * _al(B * H * NC * C * C * 4)
            + _al(B * H * NC * C * Dk * 4))
    if decay == G.GDR_DECAY_CHANNEL:   # the cumulative decays G
        want += _al(B * H * NC * C * Dk * 4)
    if wkey == G.GDR_WKEY_DIAG_PRECOND:   # write keys, p_t, write-key gradients, chunk sums
        want += 3 * _al(B * T * H * Dk * 4) + _al(B * H * NC * Dk * 4)
    assert G.gdr_chunk_bwd_workspace_size(d) == want
    # the band-limited T adds the whole T and dD
    band = want + _al(B * H * NC * C * C * 4) + _al(B * T * H * Dv * 4)
    assert G.gdr_chunk_bwd_workspace_size(desc(T=T, chunk=C, decay=decay, wkey=wkey, neumann_order=3)) == band
    assert G.gdr_chunk_bwd_workspace_size(desc(chunk=48)) == 0


def bwd_args(d, **over):
    """Well-formed, disjoint fake pointers for a backward call of descriptor d."""
    p = [BASE + i * MB for i in range(40)]
    ins = dict(q=p[0], k=p[1], v=p[2])
    if d.gain == G.GDR_GAIN_SCALAR:
        ins["beta"] = p[3]
    else:
        ins["erase"], ins["write"] = p[4], p[5]
    if d.decay != G.GDR_DECAY_NONE:
        ins["log_alpha"] = p[6]
    if d.wkey == G.GDR_WKEY_EXPLICIT:
        ins["write_key"] = p[7]
    gr = dict(dq=p[10], dk=p[11], dv=p[12], dstate_in=p[19])
    if d.gain == G.GDR_GAIN_SCALAR:
        gr["dbeta"] = p[13]
    else:
        gr["derase"], gr["dwrite"] = p[14], p[15]
    if d.decay != G.GDR_DECAY_NONE:
        gr["dlog_alpha"] = p[16]
    if d.wkey == G.GDR_WKEY_EXPLICIT:
        gr["dwrite_key"] = p[17]
    a = dict(state_in=p[8], d_out=p[9], d_state_out=p[18], workspace=p[24],
             workspace_bytes=G.gdr_chunk_bwd_workspace_size(d))
    gr.update(over.pop("grads", {}))
    ins.update(over.pop("ins", {}))
    a.update(over)
    return G.gdr_inputs_t(**ins), G.gdr_grads_t(**gr), a


def call_validate_bwd(d, **over):
    ins, gr, a = bwd_args(d, **over)
    return G.gdr_validate_bwd(d, ins, a["state_in"], a["d_out"], a["d_state_out"], gr, a["workspace"],
                              a["workspace_bytes"])


@pytest.mark.parametrize("gain", [G.GDR_GAIN_SCALAR, G.GDR_GAIN_CHANNEL])
@pytest.mark.parametrize("decay", [G.GDR_DECAY_NONE, G.GDR_DECAY_SCALAR, G.GDR_DECAY_CHANNEL])
@pytest.mark.parametrize("wkey", [G.GDR_WKEY_SAME, G.GDR_WKEY_EXPLICIT, G.GDR_WKEY_DIAG_PRECOND])
def test_bwd_accepts_supported_variants(gain, decay, wkey):
    d = desc(gain=gain, decay=decay, wkey=wkey)
    assert call_validate_bwd(d) == G.GDR_OK, G.gdr_last_error()


@pytest.mark.parametrize("kw", [dict(neumann_order=3, residual_steps=2),
                                dict(neumann_order=3, decay=G.GDR_DECAY_CHANNEL)])
def test_bwd_rejects_unsupported_variants(kw):
    d = desc(**kw)
    ins, gr, a = bwd_args(d)
    assert G.gdr_validate_bwd(d, ins, None, a["d_out"], None, gr, a["workspace"],
                              a["workspace_bytes"]) == G.GDR_ENOTSUP, G.gdr_last_error()


def test_bwd_rejects_missing_and_extra_grads():
    d = desc(decay=G.GDR_DECAY_SCALAR)
    assert call_validate_bwd(d, grads=dict(dk=None)) == G.GDR_EINVAL
    assert "dk" in G.gdr_last_error()
    assert call_validate_bwd(d, grads=dict(dlog_alpha=None)) == G.GDR_EINVAL
    assert call_validate_bwd(d, grads=dict(derase=BASE + 30 * MB)) == G.GDR_EINVAL
    assert call_validate_bwd(desc(), grads=dict(dlog_alpha=BASE + 30 * MB)) == G.GDR_EINVAL
    assert call_validate_bwd(d, grads=dict(dstate_in=None), d_state_out=None, state_in=None) == G.GDR_OK
    assert call_validate_bwd(d, d_out=None) == G.GDR_EINVAL


def test_bwd_workspace_checks():
    d = desc()
    need = G.gdr_chunk_bwd_workspace_size(d)
    assert call_validate_bwd(d, workspace_bytes=need - 1) == G.GDR_EINVAL
    assert "workspace" in G.gdr_last_error()
    assert call_validate_bwd(d, workspace=BASE + 24 * MB + 128) == G.GDR_EINVAL
    assert call_validate_bwd(d, workspace=None) == G.GDR_EINVAL
    # T == 0 needs none
    d0 = desc(T=0)
    assert G.gdr_chunk_bwd_workspace_size(d0) == 0
    ins, gr, a = bwd_args(d0)
    assert G.gdr_validate_bwd(d0, ins, None, None, None, gr, None, 0) == G.GDR_OK, G.gdr_last_error()


def test_bwd_overlap_rules():
    d = desc()
    # an output on an input, on another output, on the workspace
    assert call_validate_bwd(d, grads=dict(dq=BASE + 0 * MB)) == G.GDR_EINVAL
    assert call_validate_bwd(d, grads=dict(dk=BASE + 10 * MB + 64)) == G.GDR_EINVAL
    assert call_validate_bwd(d, grads=dict(dv=BASE + 24 * MB + 4096)) == G.GDR_EINVAL
    assert call_validate_bwd(d, grads=dict(dstate_in=BASE + 18 * MB)) == G.GDR_EINVAL
    # the workspace on an input
    assert call_validate_bwd(d, workspace=BASE + 9 * MB) == G.GDR_EINVAL


def test_bwd_entry_point_rejects_before_launch():
    d = desc()
    ins, gr, a = bwd_args(d, grads=dict(dq=None))
    st = G.lib().gdr_chunk_bwd(ctypes.byref(d), ctypes.byref(ins), None, a["d_out"], None, ctypes.byref(gr),
                               a["workspace"], a["workspace_bytes"], None)
    assert st == G.GDR_EINVAL


def test_bwd_preconditioner_arguments():
    d = desc(wkey=G.GDR_WKEY_DIAG_PRECOND, decay=G.GDR_DECAY_SCALAR)
    assert call_validate_bwd(d) == G.GDR_OK, G.gdr_last_error()
    assert call_validate_bwd(d, ins=dict(pc_h_in=BASE + 31 * MB), grads=dict(dpc_h_in=BASE + 32 * MB)) == G.GDR_OK
    # the backward does not write the final accumulator
    assert call_validate_bwd(d, ins=dict(pc_h_out=BASE + 31 * MB)) == G.GDR_EINVAL
    # dL/dpc_h_in exists only with the preconditioner, and must not overlap an input
    assert call_validate_bwd(desc(), grads=dict(dpc_h_in=BASE + 32 * MB)) == G.GDR_EINVAL
    assert call_validate_bwd(d, ins=dict(pc_h_in=BASE + 31 * MB), grads=dict(dpc_h_in=BASE + 31 * MB)) == G.GDR_EINVAL
    assert "overlaps" in G.gdr_last_error()
    assert call_validate_bwd(d, grads=dict(dpc_h_in=BASE + 32 * MB + 2)) == G.GDR_EINVAL


def test_noalloc_backward_rejects_before_any_hip_call():
    """gdr_chunk_bwd_noalloc: a descriptor whose workspace exceeds the scratch array is refused
    with GDR_ENOTSUP before the library touches the GPU (so this runs without one)."""
    cap = G.gdr_chunk_bwd_noalloc_max_workspace()
    assert cap == 64 << 20
    L = G.lib()
    d = desc(B=4, H=16, T=4096, Dk=128, Dv=128)
    assert G.gdr_chunk_bwd_workspace_size(d) > cap
    ins, gr, a = bwd_args(d)
    st = L.gdr_chunk_bwd_noalloc(ctypes.byref(d), ctypes.byref(ins), None, a["d_out"], None, ctypes.byref(gr), None)
    assert st == G.GDR_ENOTSUP
    assert "no-allocation" in G.gdr_last_error()
    assert L.gdr_chunk_bwd_noalloc(None, ctypes.byref(ins), None, a["d_out"], None, ctypes.byref(gr), None) == G.GDR_EINVAL


def test_forward_workspace_size_and_checks():
    """gdr_chunk_fwd_ws: the workspace is 10 KB per (batch, head, chunk of 64 tokens) where T can
    be formed beforehand (matrix-core kernel, write key k, exact T), 0 elsewhere; a workspace
    that is too small, misaligned or overlapping an argument is rejected before anything runs."""
    d = desc(Dk=128, Dv=128)
    need = G.gdr_chunk_fwd_workspace_size(d)
    al = lambda x: (x + 255) // 256 * 256
    # ten 16 x 16 blocks of T as bf16 pairs per chunk; this batch's 24 value tiles of 32 rows fill
    # at most half of the CUs, so the sequence split adds q~ [B, T, H, 128] bf16 and three states
    assert need == 2 * 3 * 2 * 10240 + al(2 * 100 * 3 * 128 * 2) + 3 * 2 * 3 * 128 * 128 * 4
    big = desc(Dk=128, Dv=128, B=16, H=16)   # 1024 value tiles: no split
    assert G.gdr_chunk_fwd_workspace_size(big) == 16 * 16 * 2 * 10240
    assert G.gdr_chunk_fwd_workspace_size(desc(Dk=128, Dv=128, T=64)) == 2 * 3 * 1 * 10240   # one chunk: no split
    assert G.gdr_chunk_fwd_workspace_size(desc(Dk=128, Dv=128, chunk=128)) == need
    assert G.gdr_chunk_fwd_workspace_size(desc(Dk=128, Dv=128, wkey=G.GDR_WKEY_DIAG_PRECOND)) == 0
    assert G.gdr_chunk_fwd_workspace_size(desc(Dk=128, Dv=128, neumann_order=3)) == 0
    assert G.gdr_chunk_fwd_workspace_size(desc(Dk=128, Dv=128, impl=G.GDR_IMPL_GENERIC)) == 0
    assert G.gdr_chunk_fwd_workspace_size(desc()) == 0   # Dk = 64: the fp32 kernel
    assert G.gdr_chunk_fwd_workspace_size(desc(Dk=128, Dv=128, io_dtype=G.GDR_F32)) == 0
    # per-channel decay (matrix-core kernel through the workspace only): the three decayed operand
    # arrays [B, T, H, 128] bf16, a 15872-byte record and a 4-byte flag per (batch, head, chunk),
    # each section rounded up to 256 bytes
    al = lambda x: (x + 255) // 256 * 256
    kd = desc(Dk=128, Dv=128, decay=G.GDR_DECAY_CHANNEL)
    assert G.gdr_chunk_fwd_workspace_size(kd) == 3 * al(2 * 100 * 3 * 128 * 2) + al(2 * 3 * 2 * 15872) + al(2 * 3 * 2 * 4)
    assert G.gdr_chunk_fwd_workspace_size(desc(Dk=128, Dv=128, decay=G.GDR_DECAY_CHANNEL, T=77)) == \
        3 * al(2 * 77 * 3 * 128 * 2) + al(2 * 3 * 2 * 15872) + al(2 * 3 * 2 * 4)
    assert G.gdr_chunk_fwd_workspace_size(desc(Dk=128, Dv=128, decay=G.GDR_DECAY_CHANNEL, chunk=128)) == \
        G.gdr_chunk_fwd_workspace_size(kd)
    for kw in (dict(neumann_order=3), dict(gain=G.GDR_GAIN_CHANNEL), dict(wkey=G.GDR_WKEY_DIAG_PRECOND),
               dict(wkey=G.GDR_WKEY_EXPLICIT), dict(io_dtype=G.GDR_F32), dict(impl=G.GDR_IMPL_GENERIC)):
        assert G.gdr_chunk_fwd_workspace_size(desc(Dk=128, Dv=128, decay=G.GDR_DECAY_CHANNEL, **kw)) == 0, kw
    assert G.gdr_chunk_fwd_impl(kd) == G.GDR_IMPL_GENERIC   # gdr_chunk_fwd itself: the fp32 kernel
    L = G.lib()
    ins = inputs()
    ws = BASE + 40 * MB

    def call(wptr, nbytes):
        return L.gdr_chunk_fwd_ws(ctypes.byref(d), ctypes.byref(ins), None, OUT, SOUT, wptr, nbytes, None)

    assert call(ws, need - 1) == G.GDR_EINVAL and "workspace" in G.gdr_last_error()
    assert call(ws + 16, need) == G.GDR_EINVAL and "aligned" in G.gdr_last_error()
    assert call(OUT, need) == G.GDR_EINVAL and "overlaps" in G.gdr_last_error()
    assert call(BASE + 1 * MB, need) == G.GDR_EINVAL and "overlaps" in G.gdr_last_error()
