// Internal declarations shared by the host layer and the kernels of libgdr.
// Nothing here is part of the public ABI (include/gdr.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr.h"

namespace gdr {

// Everything a kernel launch needs, resolved and validated on the host.
struct ChunkArgs {
  const void *q, *k, *v;
  const float *beta, *log_alpha;
  const void *erase, *write, *write_key;
  const float *pc_h_in;
  float *pc_h_out;
  const float *state_in;
  void *out;
  float *state_out;
  int B, T, H, Dk, Dv, C;
  int gain, decay, wkey, N;   // N < 0: exact T; else band i - j <= N
  int S;                      // residual-correction steps on the band start (0: none)
  float scale, rho, log_rho, eps, h0;
  long long t0;
  // the chunks' T (exact, write key k) formed beforehand, as bf16 pairs row-major,
  // [B, H, chunks][hi, lo][64][64] (gdr_chunk_fwd_ws); null: the matrix-core kernel forms it.
  // With the per-channel decay on the matrix-core kernel: the base of its whole workspace
  const uint16_t *tpre;
  // Sequence split (gdr_chunk_fwd_ws, where the batch's value tiles fill at most half the GPU):
  // seg_split > 0 is the first chunk of the second segment.  The sequential pass then runs
  // three groups of workgroups: the first segment from state_in (its final state S_mid to
  // seg_state[0]), the second from a zero state (outputs to out, final state S_loc to
  // seg_state[1]), and the second again with V' = 0 from the identity (its outputs
  // q~ = scale M q to seg_qt [B,T,H,128] bf16, its final state M to seg_state[2]);
  // a fix-up adds S_mid q~ to the second segment's outputs and forms S_mid M + S_loc.
  int seg_split;
  uint16_t *seg_qt;
  float *seg_state;   // [3][B,H,Dv,Dk]
};

// Backward pass (gdr_chunk_bwd): the forward's arguments plus the incoming gradients, the
// gradient outputs and the workspace sections.
struct BwdArgs {
  ChunkArgs f;
  const void *dout;          // [B,T,H,Dv] io dtype
  const float *dstate_out;   // [B,H,Dv,Dk] or null (zero)
  float *dq, *dk, *dv, *dbeta, *derase, *dwrite, *dla, *dwk, *dstate_in;
  // workspace: states at chunk starts and their gradients [B,H,NC,Dv,Dk], D and dX
  // [B,T,H,Dv], T and P [B,H,NC,C,C], W [B,H,NC,C,Dk], U [B,T,H,Dv]; with per-channel decay
  // also G [B,H,NC,C,Dk], the in-chunk cumulative log2 decay (null otherwise)
  float *h, *dh, *D, *dX, *Tw, *Pw, *Ww, *Uw, *Gw;
  // preconditioned write key: the write keys r = k (.) p and p [B,T,H,Dk] (formed before the
  // other kernels; the kernels read the write key from Rk whenever it is set), the write-key
  // gradients dR [B,T,H,Dk] (null otherwise); dL/dpc_h_in [B,H,Dk] or null
  float *Rk, *Pk, *dRk, *dpc_h_in;
  float *Sg;   // preconditioned write key: per-chunk partial sums of its scans [B,H,NC,Dk]
  // band-limited T (f.N >= 0): Tw holds the band T_b, Tfw the whole inverse T [B,H,NC,C,C];
  // dDw the sweep's dD [B,T,H,Dv] (null otherwise)
  float *Tfw, *dDw;
  int NC;   // chunks per stream
};

// Host launchers (return hipSuccess or the launch error).
hipError_t launch_chunk_generic(const ChunkArgs &a, int io_dtype, hipStream_t s);
hipError_t launch_chunk_mfma(const ChunkArgs &a, hipStream_t s);
unsigned long long chunk_mfma_tpre_bytes(const gdr_desc_t &d);
bool chunk_mfma_supports(const gdr_desc_t &d, const gdr_inputs_t &in, const float *state_in,
                         const void *out, const float *state_out);
// the per-channel decay on the matrix-core kernel (only with gdr_chunk_fwd_ws's workspace)
bool chunk_mfma_kda_supports(const gdr_desc_t &d, const gdr_inputs_t &in, const float *state_in,
                             const void *out, const float *state_out);
hipError_t launch_step(const ChunkArgs &a, int io_dtype, hipStream_t s);
hipError_t launch_bwd_prep_state(const BwdArgs &a, int io_dtype, hipStream_t s);
hipError_t launch_bwd_sweep(const BwdArgs &a, int io_dtype, hipStream_t s);
hipError_t launch_bwd_chunk(const BwdArgs &a, int io_dtype, hipStream_t s);
hipError_t launch_bwd_pc_keys(const BwdArgs &a, int io_dtype, hipStream_t s);
hipError_t launch_bwd_pc_grad(const BwdArgs &a, int io_dtype, hipStream_t s);

// ---------------------------------------------------------------------------------
// Device helpers: storage conversions.  bf16 is stored as uint16_t bit patterns.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ float ld_f(const float *p, long long i) { return p[i]; }
__device__ __forceinline__ float ld_f(const uint16_t *p, long long i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// fp32 -> bf16, round to nearest even (NaN stays NaN): one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// two values packed low | high << 16
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ void st_f(float *p, long long i, float x) { p[i] = x; }
__device__ __forceinline__ void st_f(uint16_t *p, long long i, float x) { p[i] = f32_to_bf16_bits(x); }

}  // namespace gdr
