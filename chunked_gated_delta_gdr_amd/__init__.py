"""chunked_gated_delta_gdr_amd -- chunked gated delta rule on AMD MI355X (gfx950).

A thin Python binding over the C ABI of ``libgdr.so`` (declared in ``include/gdr.h``).
The functions here only marshal arguments: they check torch tensors (device, dtype,
contiguity, shapes), fill the descriptor structs and call the library on the current
HIP stream.  Every step of the computation runs in the library's HIP kernels; there is
no CPU or PyTorch fallback, and importing the package fails loudly when the library has
not been built (``python -m chunked_gated_delta_gdr_amd.build``).
"""
from ._binding import (  # noqa: F401
    GDR_OK, GDR_EINVAL, GDR_ENOTSUP, GDR_EHIP,
    GDR_F32, GDR_BF16,
    GDR_GAIN_SCALAR, GDR_GAIN_CHANNEL,
    GDR_DECAY_NONE, GDR_DECAY_SCALAR, GDR_DECAY_CHANNEL,
    GDR_WKEY_SAME, GDR_WKEY_DIAG_PRECOND, GDR_WKEY_EXPLICIT,
    GDR_IMPL_AUTO, GDR_IMPL_GENERIC, GDR_IMPL_MFMA,
    GdrError, gdr_desc_t, gdr_inputs_t, gdr_grads_t,
    lib, lib_path, make_desc,
    gdr_chunk_fwd, gdr_recurrent_step, gdr_validate, gdr_chunk_fwd_impl,
    gdr_chunk_bwd, gdr_chunk_bwd_workspace_size, gdr_validate_bwd, gdr_chunk_bwd_noalloc_max_workspace,
    gdr_chunk_fwd_workspace_size,
    gdr_status_str, gdr_last_error, gdr_abi_version,
)
