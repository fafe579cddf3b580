"""CPU oracle for the chunked gated delta rule -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 NumPy code whose only job is to be obviously correct.  Only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import it; the
GPU library never does, and this package never imports the GPU library.  The two
share no code; only the seeded input generators (``gdr_synth``) serve both.

Sources (titles of the pages the method is described on):

* [PDN]  "Preconditioned DeltaNet: Curvature-aware Sequence Modeling for Linear
         Recurrences" (gist.science summaries, Portuguese and Arabic) -- the delta rule
         as an online SGD step on a least-squares loss (section 1), the exact
         preconditioner and apply-to-key write key (section 2a), the diagonal
         second-moment preconditioner as a prefix sum (section 2b), the DGPS axes
         decay alpha_t / gain beta_t / preconditioner / solve (section 2c).
* [GDN2] "NVIDIA Apresenta Gated DeltaNet-2" (news item), section "Como DeltaNet-2
         Redesenhou a Arquitetura" -- channel-wise erase gate on the key axis and write
         gate on the value axis.
* [MMI]  "Quando o 'Bom o Suficiente' e Otimo: Aproximacao de Inversao de Matriz
         Baseada Apenas em Multiplicacao para Gated DeltaNet Quantizado" (gist.science
         summary) -- chunk-wise form with T = (I - A)^-1, A strictly lower triangular,
         forward substitution ("Declaracao do Problema"); truncated Neumann series and
         Lemma 3.1 (Metodologia 1); structural diagonal mask (Metodologia 2); parallel
         residual correction (Metodologia 3).

Parity status: every public function is pinned by tests under ``tests/`` against
closed forms, exact-rational brute force, textbook special cases or identities the
pages state.  One reading is *parity unpinned* against its source: the Gated
DeltaNet-2 update equations (the news item names the two gates' axes but prints no
formula); the reading used is pinned only against its own special cases.
"""
from .core import (  # noqa: F401
    variant_vectors,
    diag_precond_write_key,
    recurrent,
    recurrent_stream,
    chunked,
    chunked_stream,
    tri_inverse,
    forward_substitution,
    neumann_literal,
    residual_corrected,
    decode_step,
    rel_l2,
    snr_db,
)
from .backward import (  # noqa: F401
    chunked_grad, chunked_stream_grad, precond_grad, recurrent_grad, recurrent_stream_grad,
)
