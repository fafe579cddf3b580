/*
 * gdr.h -- C ABI of the chunked gated delta-rule library for AMD MI355X (gfx950).
 *
 * The library computes, for every (batch b, head h) stream, the linear recurrence
 *
 *     S_t = alpha_t S_{t-1} (I - e_t r_t^T) + v'_t r_t^T,      o_t = S_t (scale q_t)
 *
 * with state S (Dv x Dk), erase (read) key e_t, write key r_t, written value v'_t and
 * scalar decay alpha_t = exp(log_alpha_t).  The variants are chosen by the descriptor:
 *
 *   gain   SCALAR   e = beta k,           v' = beta v        (delta rule / gated delta rule)
 *          CHANNEL  e = erase (.) k,      v' = write (.) v   (erase gate on the key axis,
 *                                                              write gate on the value axis)
 *   decay  NONE     alpha = 1;  SCALAR  alpha_t = exp(log_alpha_t), log_alpha <= 0
 *   wkey   SAME     r = k;  EXPLICIT  r = write_key;
 *          DIAG_PRECOND  r = k (.) p_t with p_t = 1 / (hhat_t + eps),
 *                        h_t = rho h_{t-1} + k_t (.) k_t, hhat_t = h_t / (1 - rho^t),
 *                        t the 1-based global token index (pc_t0 + position + 1).
 *
 * Sources (page titles): the delta rule as an online SGD step on a least-squares loss,
 * and the decay / gain / preconditioner axes -- "Preconditioned DeltaNet: Curvature-aware
 * Sequence Modeling for Linear Recurrences", technical summary sections 1, 2a (apply-to-key
 * write key), 2b (diagonal second-moment preconditioner), 2c (DGPS axes); channel-wise
 * erase and write gates -- "NVIDIA Apresenta Gated DeltaNet-2", section "Como DeltaNet-2
 * Redesenhou a Arquitetura"; chunk-wise evaluation with T = (I - A)^-1 for a strictly
 * lower-triangular A, and the truncated Neumann series with a diagonal band mask --
 * "Quando o 'Bom o Suficiente' e Otimo: Aproximacao de Inversao de Matriz Baseada Apenas
 * em Multiplicacao para Gated DeltaNet Quantizado", "Declaracao do Problema" and
 * "Metodologia" 1-2.
 *
 * Conventions shared by every entry point:
 *  - Layout: q, k, write_key, erase are [B, T, H, Dk]; v, write, out are [B, T, H, Dv];
 *    beta, log_alpha are [B, T, H]; all contiguous, row-major, last index fastest.  The
 *    state is [B, H, Dv, Dk] fp32 (value rows contiguous); the preconditioner accumulator
 *    is [B, H, Dk] fp32.
 *  - Element types: q, k, v, erase, write, write_key and out use io_dtype (fp32 or bf16);
 *    beta, log_alpha, state and pc_h are always fp32.
 *  - Memory: every pointer is a device pointer owned by the caller.  The library never
 *    allocates, frees or keeps a pointer after the call returns.  Scratch memory, where an
 *    entry point uses it, is passed in by the caller (gdr_chunk_bwd_workspace_size,
 *    gdr_chunk_fwd_workspace_size).
 *  - Execution: the work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *    the null stream) and the call returns without synchronising.
 *  - Errors: arguments are validated on the host before anything is enqueued.  On
 *    GDR_EINVAL or GDR_ENOTSUP nothing is launched and nothing is written.  A launch
 *    failure returns GDR_EHIP.  gdr_last_error() gives a thread-local description of the
 *    last non-OK return.  Faults inside a kernel surface at the caller's next
 *    synchronisation, as usual in HIP.
 *  - Determinism: no atomics; results are bitwise reproducible run to run.
 *  - Threads: the library is stateless and reentrant.
 */
#ifndef GDR_H_
#define GDR_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 5

typedef enum {
  GDR_OK = 0,
  GDR_EINVAL = 1,   /* malformed descriptor, missing or overlapping pointer */
  GDR_ENOTSUP = 2,  /* well-formed but outside what the library implements   */
  GDR_EHIP = 3      /* a HIP runtime call failed                             */
} gdr_status_t;

enum { GDR_F32 = 0, GDR_BF16 = 1 };                                     /* io_dtype */
enum { GDR_GAIN_SCALAR = 0, GDR_GAIN_CHANNEL = 1 };                     /* gain     */
enum { GDR_DECAY_NONE = 0, GDR_DECAY_SCALAR = 1, GDR_DECAY_CHANNEL = 2 }; /* decay  */
enum { GDR_WKEY_SAME = 0, GDR_WKEY_DIAG_PRECOND = 1, GDR_WKEY_EXPLICIT = 2 }; /* wkey */
enum { GDR_IMPL_AUTO = 0, GDR_IMPL_GENERIC = 1, GDR_IMPL_MFMA = 2 };    /* impl     */

typedef struct gdr_desc {
  uint32_t struct_size;   /* must equal sizeof(gdr_desc_t) (ABI guard)                    */
  int32_t B, T, H;        /* batch, tokens in this call (1 for gdr_recurrent_step), heads;
                             B, H <= 65535 and B * H <= 2^19 streams (GDR_ENOTSUP beyond:
                             every launch grid then fits HIP's 32-bit work-item counts);
                             the backward also takes at most 2^22 chunks per stream      */
  int32_t Dk, Dv;         /* key and value head dims: 1 <= Dk <= 128, 1 <= Dv <= 512      */
  int32_t chunk;          /* chunk size C in tokens: 16, 32, 64 or 128 (ignored by the
                             step; the inversion summary measures 32, 64 and 128).  At 128
                             the exact T runs as two 64-row blocks, the off-diagonal block
                             T_ba = T_bb A_ba T_aa applied through the state after the first
                             64 tokens (the same product regrouped), on either kernel; a
                             band limit needs N <= 15 (or N >= 127, which is exact), decay
                             NONE or SCALAR and no residual steps, and runs on the generic
                             kernel; other chunk-128 descriptors return GDR_ENOTSUP        */
  int32_t io_dtype;       /* GDR_F32 | GDR_BF16                                            */
  int32_t gain;           /* GDR_GAIN_*                                                    */
  int32_t decay;          /* GDR_DECAY_*                                                   */
  int32_t wkey;           /* GDR_WKEY_*                                                    */
  int32_t neumann_order;  /* < 0: exact T = (I - A)^-1 by blocked forward substitution
                             (substitution inside 4 x 4 diagonal blocks, block products
                             T_21 = T_22 A_21 T_11 between them);
                             N >= 0: T restricted to the band i - j <= N (the masked
                             truncated Neumann series sum_{n<=N} A^n, which equals the band
                             of the exact inverse); N >= C - 1 reproduces the exact path
                             bit for bit in fp32                                           */
  int32_t residual_steps; /* S >= 0, only with neumann_order = N >= 0: when S > 0, T is the
                             parallel residual correction of the band-N start
                             T0 = band_N((I - A)^-1): E = I - (I - A) T0 and
                             T = T0 (I + E + ... + E^S)  (MatMul-only inversion summary,
                             Metodologia 3).  Exact once (S + 1)(N + 1) >= C.  Both
                             kernels implement it (the matrix-core one at chunk 64); not
                             at chunk 128 or with decay CHANNEL (GDR_ENOTSUP)              */
  int32_t impl;           /* GDR_IMPL_AUTO picks the fastest kernel for the shape;
                             GENERIC forces the fp32 VALU kernel; MFMA forces the bf16
                             matrix-core kernel (GDR_ENOTSUP if the shape is outside it)   */
  float scale;            /* query scale (finite)                                          */
  float pc_rho;           /* preconditioner decay rho, 0 < rho < 1 (wkey DIAG_PRECOND)     */
  float pc_eps;           /* preconditioner epsilon, > 0                                   */
  float pc_h0;            /* initial accumulator value when pc_h_in is NULL, >= 0          */
  int64_t pc_t0;          /* tokens already absorbed into pc_h_in (>= 0)                   */
} gdr_desc_t;

typedef struct gdr_inputs {
  const void *q, *k, *v;    /* io_dtype; required                                         */
  const float *beta;        /* [B,T,H] fp32; required iff gain == SCALAR                   */
  const float *log_alpha;   /* decay SCALAR: [B,T,H] fp32 (<= 0), one decay per token;
                               decay CHANNEL: [B,T,H,Dk] fp32 (<= 0), one decay per key
                               channel (S_t = S_{t-1} Diag(a_t) (I - e r^T) + v' r^T, the
                               diagonal gate named beside Kimi Delta Attention in the
                               Preconditioned DeltaNet summary); required iff decay != NONE.
                               The chunked form with CHANNEL runs on the generic kernel and
                               takes no residual correction                               */
  const void *erase;        /* [B,T,H,Dk] io_dtype; required iff gain == CHANNEL           */
  const void *write;        /* [B,T,H,Dv] io_dtype; required iff gain == CHANNEL           */
  const void *write_key;    /* [B,T,H,Dk] io_dtype; required iff wkey == EXPLICIT          */
  const float *pc_h_in;     /* [B,H,Dk] fp32 or NULL (=> every entry pc_h0); DIAG_PRECOND  */
  float *pc_h_out;          /* [B,H,Dk] fp32 or NULL (=> not returned); DIAG_PRECOND.  For
                               gdr_chunk_fwd it must not overlap pc_h_in; for
                               gdr_recurrent_step it may equal pc_h_in (in-place update)   */
} gdr_inputs_t;

/*
 * gdr_chunk_fwd -- chunk-parallel forward pass over T tokens.
 *
 * Per chunk of C tokens, with g the in-chunk inclusive cumulative sum of log_alpha and
 * Gamma_ij = exp(g_i - g_j) (j <= i):
 *     A = -tril_{-1}((E R^T) (.) Gamma),  T = (I - A)^-1  (exact, or its band i - j <= N)
 *     W = T (e^g (.) E),  U = T V',  D = U - W S^T
 *     O = (e^g (.) Q) S^T + (tril(Q R^T) (.) Gamma) D,   S <- e^{g_C} S + D^T (e^{g_C - g} (.) R)
 * (chunk-wise form and T of the MatMul-only inversion summary, "Declaracao do Problema").
 *
 *   state_in   [B,H,Dv,Dk] fp32 initial state, or NULL for zeros.
 *   out        [B,T,H,Dv] io_dtype; must not overlap any input.  May be NULL only if T == 0.
 *   state_out  [B,H,Dv,Dk] fp32 final state, or NULL (not written).  May be the same
 *              pointer as state_in (in-place); any other overlap is rejected.
 *   stream     hipStream_t as void*.
 * T == 0 is valid: state_out receives state_in (or zeros) and pc_h_out receives pc_h_in.
 */
gdr_status_t gdr_chunk_fwd(const gdr_desc_t *desc, const gdr_inputs_t *in,
                           const float *state_in, void *out, float *state_out,
                           void *stream);

/*
 * gdr_chunk_fwd_ws -- gdr_chunk_fwd with caller-owned scratch memory in which T of every
 * chunk is formed first, all chunks at once, before the sequential pass reads it (same
 * results as gdr_chunk_fwd to rounding: the same stable inverse, its blocks in a different
 * order).  T = (I - A)^-1 of each chunk depends only on the chunk's own keys and gates
 * (MatMul-only inversion summary, "Declaracao do Problema"), so forming it apart from the
 * state pass is exact.  It applies where the matrix-core kernel runs with write key k and
 * the exact T (no band limit, no residual steps); elsewhere the workspace is not used.
 * With one decay per key channel (GDR_DECAY_CHANNEL: the diagonal gate the Preconditioned
 * DeltaNet summaries name beside Gated DeltaNet, section 2c) this entry point is the one that
 * runs it on the bf16 matrix cores (bf16, Dk = Dv = 128, chunk 64 or exact 128, scalar gains,
 * write key k, exact T): the workspace then also holds each chunk's decayed keys and queries,
 * P and the per-channel state decay, all formed before the sequential pass; gdr_chunk_fwd
 * runs that descriptor on the fp32 kernel.  Results equal gdr_chunk_fwd's within the bf16
 * bound.  Where the batch's 32-row value tiles (B * H * 4) number at most 128, the sequential
 * pass also splits each sequence in two segments that run at once: the second from a zero
 * state and again as its own transition from the identity.  Their outputs are then corrected
 * by the first segment's final state (linearity of the recurrence in its state).
 *
 *   workspace        device memory of at least gdr_chunk_fwd_workspace_size(desc) bytes,
 *                    256-byte aligned, overlapping no other argument; its contents on entry
 *                    do not matter and are overwritten.  NULL: exactly gdr_chunk_fwd.
 *   workspace_bytes  its size; less than needed returns GDR_EINVAL.
 * Other arguments and errors as gdr_chunk_fwd.
 */
gdr_status_t gdr_chunk_fwd_ws(const gdr_desc_t *desc, const gdr_inputs_t *in,
                              const float *state_in, void *out, float *state_out,
                              void *workspace, uint64_t workspace_bytes, void *stream);

/* Bytes of gdr_chunk_fwd_ws's workspace: 10 KB per (batch, head, chunk of 64 tokens) where it
 * applies (T's ten 16 x 16 blocks on and below the diagonal, each as a pair of bf16 parts); with
 * the sequence split (B * H * 4 <= 128, at least two chunks) also B * T * H * 256 bytes rounded
 * up to 256 (the transition's outputs) and 3 * B * H * 65536 bytes (three fp32 states); 0
 * where it does not (any workspace is then ignored) or for an invalid descriptor.  With the
 * per-channel decay: three [B, T, H, 128] bf16 arrays (the decayed keys and queries), then
 * 15872 bytes and a 4-byte flag per (batch, head, chunk), each section rounded up to 256 bytes
 * (about 64 KB per chunk).  Pure host arithmetic. */
uint64_t gdr_chunk_fwd_workspace_size(const gdr_desc_t *desc);

/*
 * gdr_recurrent_step -- one token for every stream, updating the state in place:
 *     S <- alpha S;  d = v' - S e;  S <- S + d r^T;  o = S (scale q)
 * (one online SGD step of the delta rule, Preconditioned DeltaNet summary section 1; the
 * fixed-size state replaces a growing key-value cache, Gated DeltaNet-2 news item).
 *
 *   desc->T must be 1; inputs are laid out [B,1,H,D] (= [B,H,D]) and [B,1,H].
 *   state      [B,H,Dv,Dk] fp32, read and overwritten.
 *   out        [B,H,Dv] io_dtype; must not overlap any input or the state.
 *   For DIAG_PRECOND the token's global index is pc_t0 + 1 and pc_h_out may equal pc_h_in.
 */
gdr_status_t gdr_recurrent_step(const gdr_desc_t *desc, const gdr_inputs_t *in,
                                float *state, void *out, void *stream);

/*
 * gdr_validate -- the host-side argument check used by both entry points, exposed on its
 * own.  Makes no HIP call.  `for_step` = 1 checks gdr_recurrent_step's contract (then
 * state_out names the in-place state and state_in is ignored), 0 checks gdr_chunk_fwd's.
 */
gdr_status_t gdr_validate(const gdr_desc_t *desc, const gdr_inputs_t *in,
                          const float *state_in, const void *out, const float *state_out,
                          int for_step);

/* Gradients written by gdr_chunk_bwd: fp32 device buffers owned by the caller, laid out
 * like the inputs they belong to.  Every buffer the descriptor's variant has is required. */
typedef struct gdr_grads {
  float *dq;          /* [B,T,H,Dk]                                                       */
  float *dk;          /* [B,T,H,Dk] (through e and, with wkey SAME, through r = k)         */
  float *dv;          /* [B,T,H,Dv]                                                       */
  float *dbeta;       /* [B,T,H]; iff gain == SCALAR, else NULL                            */
  float *derase;      /* [B,T,H,Dk]; iff gain == CHANNEL, else NULL                        */
  float *dwrite;      /* [B,T,H,Dv]; iff gain == CHANNEL, else NULL                        */
  float *dlog_alpha;  /* [B,T,H] if decay == SCALAR, [B,T,H,Dk] if CHANNEL, else NULL       */
  float *dwrite_key;  /* [B,T,H,Dk]; iff wkey == EXPLICIT, else NULL                       */
  float *dstate_in;   /* [B,H,Dv,Dk] or NULL (not written)                                 */
  float *dpc_h_in;    /* [B,H,Dk] dL/dpc_h_in (every entry, also when pc_h_in is NULL: the
                         gradient of the pc_h0 start); wkey DIAG_PRECOND only, or NULL      */
} gdr_grads_t;

/*
 * gdr_chunk_bwd -- gradients of a scalar loss through gdr_chunk_fwd.
 *
 * The pages train these layers (Preconditioned DeltaNet summary: chunk-wise forms are what
 * makes training on GPUs efficient, section 2b; models trained at 340M and 1B parameters,
 * section 4) but give no backward pass.  This is the derivative of the forward above,
 * taken through its chunk-wise form ("Declaracao do Problema" of the MatMul-only inversion
 * summary) in four launches:
 *   1. per chunk, in parallel: T, P, W = T (e^g (.) E) and U = T V';
 *   2. forward state pass (per value tile): D = U - W S^T and the state at every chunk start;
 *   3. reverse sweep over chunks (per value tile): with dS the gradient at the chunk end,
 *        dD = e^{g_C - g} (.) (R dS^T) + scale P^T dO,   dX = T^T dD   (= dV'),
 *        dS <- e^{g_C} dS + scale dO^T (e^g (.) Q) - dX^T (e^g (.) E);
 *   4. per chunk, in parallel: dQ, dE, dR and the gate gradient from the stored states,
 *      the state gradients, D and dX, then the chain rule to the variant's inputs.
 * With per-channel decay (the Diag gate; Kimi Delta Attention in the pages' related-work
 * sections) every e^g above is per key channel: e^g (.) E, e^g (.) Q and e^{g_C - g} (.) R
 * elementwise, e^{g_C} dS scales the state's columns, the pairwise decay sits inside the
 * products over channels (L, P) and over tokens (dQ, dE, dR), and the gate gradient is one
 * per token and channel.
 * With the preconditioned write key (DIAG_PRECOND) two more launches bracket these: a scan
 * per channel that forms the write keys r_t = k_t (.) p_t (fp32) before, and after, the chain
 * rule through p_t: the accumulator's gradient H_t = -(dr_t k_t p_t^2) / b_t + rho H_{t+1}
 * (reverse scan per channel, the final accumulator outside the loss) adds
 * dr_t (.) p_t + 2 k_t (.) H_t to dk and gives dL/dpc_h_in = rho H_1.  The final
 * accumulator (pc_h_out) is not written.
 * All arithmetic is fp32 (inputs in io_dtype are widened once).
 *
 * With the band-limited T (neumann_order = N >= 0) the forward is D = T_b X with T_b the band
 * i - j <= N of T; its derivative adds dT_b = dD X^T = (dD D^T) T_b^-T, masked to the band, and
 * takes dA = T^T (M (.) dT_b) T^T (the band of the truncated series is that of T, so the
 * derivative is that of the band of the inverse) in place of -dX D^T; the sweep keeps dD for
 * it, the preparation both T and T_b.
 *
 * Supported: gain SCALAR | CHANNEL, decay NONE | SCALAR | CHANNEL, wkey SAME | EXPLICIT |
 * DIAG_PRECOND, exact T or the band-limited T (not with decay CHANNEL), no residual steps
 * (neumann_order < 0), chunk 16 | 32 | 64, or 128 with the exact T (the chunk-64 backward of
 * the same function), Dk <= 128, Dv <= 512, io fp32 | bf16; anything else returns
 * GDR_ENOTSUP (desc->impl is ignored).
 *
 *   in, state_in  the forward's inputs and initial state (NULL for zeros), unchanged.
 *   d_out         [B,T,H,Dv] io_dtype: dL/dout.  May be NULL only if T == 0.
 *   d_state_out   [B,H,Dv,Dk] fp32: dL/dstate_out, or NULL for zeros.
 *   grads         the outputs; none may overlap an input, another output or the workspace.
 *   workspace     device memory of at least gdr_chunk_bwd_workspace_size(desc) bytes,
 *                 256-byte aligned, owned by the caller; its contents on entry do not
 *                 matter and on return are unspecified.  May be NULL if that size is 0.
 * Enqueued on `stream`; the workspace and the outputs must stay allocated until the work
 * has run.  Deterministic (no atomics).
 */
gdr_status_t gdr_chunk_bwd(const gdr_desc_t *desc, const gdr_inputs_t *in, const float *state_in,
                           const void *d_out, const float *d_state_out, const gdr_grads_t *grads,
                           void *workspace, uint64_t workspace_bytes, void *stream);

/* Bytes of workspace gdr_chunk_bwd needs for this descriptor (0 if it is rejected or
 * T == 0): the chunk-start states and their gradients (2 B H ceil(T/C) Dv Dk floats), D,
 * dX and U (3 B T H Dv floats), T and P (2 B H ceil(T/C) C^2 floats) and W
 * (B H ceil(T/C) C Dk floats), with decay CHANNEL also the cumulative decays G
 * (B H ceil(T/C) C Dk floats), with wkey DIAG_PRECOND also the write keys, p_t and the
 * write-key gradients (3 B T H Dk floats) and per-chunk sums of the preconditioner's scans
 * (B H ceil(T/C) Dk floats), with neumann_order >= 0 also the whole T (B H ceil(T/C) C^2
 * floats) and dD (B T H Dv floats), each section 256-byte aligned.  No HIP call. */
uint64_t gdr_chunk_bwd_workspace_size(const gdr_desc_t *desc);

/*
 * gdr_chunk_bwd_noalloc -- gdr_chunk_bwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving or training loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, validation, kernels and results as gdr_chunk_bwd, without the workspace: the
 * workspace is a file-scope device array of gdr_chunk_bwd_noalloc_max_workspace() bytes
 * (64 MiB) inside the library, one copy per GPU, held until the process ends.  The call
 * allocates and frees nothing; the first call on a device looks up that device's copy
 * (hipGetSymbolAddress), later calls reuse it.  Descriptors whose
 * gdr_chunk_bwd_workspace_size exceeds the array return GDR_ENOTSUP before anything is
 * launched (at Dk = Dv = 128, C = 64 the workspace is about 290 KB per (batch, head, chunk):
 * some 225 of them, e.g. B = 1, H = 4, T = 3584).  Every call on one GPU shares its array, so
 * calls that overlap in time on one GPU (other streams, other threads) race: order them, e.g.
 * on one stream.  Nothing in the array needs clearing between calls.
 */
gdr_status_t gdr_chunk_bwd_noalloc(const gdr_desc_t *desc, const gdr_inputs_t *in, const float *state_in,
                                   const void *d_out, const float *d_state_out, const gdr_grads_t *grads,
                                   void *stream);

/* Size in bytes of the scratch array gdr_chunk_bwd_noalloc uses (no HIP call). */
uint64_t gdr_chunk_bwd_noalloc_max_workspace(void);

/* gdr_chunk_bwd's argument check on its own (no HIP call). */
gdr_status_t gdr_validate_bwd(const gdr_desc_t *desc, const gdr_inputs_t *in,
                              const float *state_in, const void *d_out, const float *d_state_out,
                              const gdr_grads_t *grads, const void *workspace,
                              uint64_t workspace_bytes);

/* Which kernel gdr_chunk_fwd would launch for this descriptor: GDR_IMPL_GENERIC or
 * GDR_IMPL_MFMA, or a negative value if the descriptor is rejected.  No HIP call. */
int gdr_chunk_fwd_impl(const gdr_desc_t *desc);

const char *gdr_status_str(gdr_status_t status);  /* static string, never NULL          */
const char *gdr_last_error(void);                 /* thread-local; "" after GDR_OK       */
int gdr_abi_version(void);                        /* GDR_ABI_VERSION                     */

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
