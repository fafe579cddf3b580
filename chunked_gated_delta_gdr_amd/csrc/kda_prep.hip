// Preparation of the per-key-channel decay forward for the bf16 matrix-core kernel.
//
// With one decay per key channel (S_t = S_{t-1} Diag(a_t)(I - beta_t k_t k_t^T) + beta_t v_t
// k_t^T, the diagonal gate of Kimi Delta Attention that the Preconditioned DeltaNet summaries
// name beside Gated DeltaNet, section 2c) the pairwise decay 2^(G_ic - G_jc) of channel c
// between tokens j <= i of a chunk (G the in-chunk inclusive cumulative log2 decay) sits
// inside the key products, so A and P are no longer a key product times a per-pair scalar.
// Everything of a chunk that does not depend on the state is formed here, for every chunk
// at once (one workgroup per batch, head and chunk), and the matrix-core kernel's sequential
// pass then runs the scalar-gain structure on it with the state decay taken per channel:
//   E~ = 2^G (.) k,  Q~ = 2^G (.) q,  R~ = 2^(G_last - G) (.) k      (bf16, [B, T, H, 128])
//   L_ij = beta_i sum_c k_ic k_jc 2^(G_ic - G_jc), j < i;  A = -L;  T = (I - A)^-1
//   P_ij = sum_c q_ic k_jc 2^(G_ic - G_jc), j <= i
//   gC_c = 2^(G_last,c)
// so that per chunk (chunk form of the MatMul-only inversion summary, "Declaracao do
// Problema"): X = beta (.) (V - E~ S^T), D = T X, O = scale (Q~ S^T + P D) and
// S <- S Diag(gC) + D^T R~.  Every exponent evaluated here is <= 0 except the ones the Gram
// routine keeps inside a diagonal 4 x 4 sub-block.
//
// L and P are fp32 (the per-channel Gram tiles of chd_gram.h: matrix cores below the diagonal
// tiles with the decay split at a reference row, pairwise factors on them), T by the blocked
// forward substitution of tri_blocks.h in fp32.  Per chunk one record of 15872 bytes:
//   T   the ten 16 x 16 blocks on and below the diagonal, block q = ib (ib + 1) / 2 + jb, each
//       as its bf16 hi part then its lo part (T - hi, rounded), 16 rows of 16 (10240 bytes)
//   P   the same ten blocks as single bf16, 16 rows of 16 (5120 bytes)
//   gC  128 fp32 (512 bytes)
// The record is read as 16-byte items u < 992, item u at byte 16 u.
#include "common.h"
#include "tri_blocks.h"
#include "chd_gram.h"

namespace gdr {
namespace {

constexpr int kC = 64;
constexpr int kD = 128;
constexpr int kNT = 512;
constexpr int kLD = kD + 4;   // fp32 row stride of the [token][channel] tiles
constexpr int kLP = kC + 4;   // fp32 row stride of the 64 x 64 tiles
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRecItems = 992;   // 16-byte items of a chunk's record

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float elt(const uint4 &v, int e) {
  const uint32_t w = (&v.x)[e >> 1];
  return bf16_bits_to_f32((e & 1) ? (w >> 16) : (w & 0xffffu));
}
__device__ __forceinline__ uint4 pack8(const float (&x)[8]) {
  return make_uint4(f32x2_to_bf16x2_bits(x[0], x[1]), f32x2_to_bf16x2_bits(x[2], x[3]),
                    f32x2_to_bf16x2_bits(x[4], x[5]), f32x2_to_bf16x2_bits(x[6], x[7]));
}

struct __align__(16) PrepSmem {
  float x[kC][kLD];   // beta (.) k, then q
  float r[kC][kLD];   // k
  float g[kC][kLD];   // log2 decays, then G
  float l[kC][kLP];   // L (A = -L), strictly lower
  float p[kC][kLP];   // P, lower with the diagonal
  float t[kC][kLP];   // T
  float z[32][36];    // the inverse's scratch
  float tot[4][kD];   // sums of the scan's four 16-token segments
};

__global__ __launch_bounds__(kNT, 1) void kda_prep_kernel(ChunkArgs a, uint16_t *qt, uint16_t *et, uint16_t *rt,
                                                          uint16_t *rec) {
  __shared__ PrepSmem sm;
  const int tid = threadIdx.x;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int H = a.H, T = a.T;
  const int nchunks = (T + kC - 1) / kC;
  const int c0 = c * kC, n = min(kC, T - c0);
  const long long tokstride = static_cast<long long>(H) * kD;
  // element offset of (b, c0, h, 0) in the [B, T, H, 128] arrays, and of (b, c0, h) in [B, T, H]
  const long long base = (static_cast<long long>(b) * T * H + h) * kD + static_cast<long long>(c0) * tokstride;
  const long long gate0 = static_cast<long long>(b) * T * H + h + static_cast<long long>(c0) * H;
  const uint16_t *gq = static_cast<const uint16_t *>(a.q) + base;
  const uint16_t *gk = static_cast<const uint16_t *>(a.k) + base;
  const float *gla = a.log_alpha + base;

  // keys and queries: items u = tid + 512 m of 8 bf16 (row u / 16, columns 8 (u % 16) ..);
  // log decays: items w = tid + 512 m of 4 fp32 (row w / 32, columns 4 (w % 32) ..).  Rows past
  // the end of the sequence read the last row and are zeroed (zero keys, no decay, so G stays
  // constant past the chunk's last token).
  uint4 kv[2], qv[2];
  float bt[2];
  float4 lv[4];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int u = tid + kNT * m, row = min(u >> 4, n - 1);
    kv[m] = *reinterpret_cast<const uint4 *>(gk + row * tokstride + 8 * (u & 15));
    qv[m] = *reinterpret_cast<const uint4 *>(gq + row * tokstride + 8 * (u & 15));
    bt[m] = a.beta[gate0 + static_cast<long long>(row) * H];
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int w = tid + kNT * m, row = min(w >> 5, n - 1);
    lv[m] = *reinterpret_cast<const float4 *>(gla + row * tokstride + 4 * (w & 31));
  }
  for (int i = tid; i < kC * kLP; i += kNT) (&sm.t[0][0])[i] = 0.f;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int u = tid + kNT * m, row = u >> 4, col = 8 * (u & 15);
    const bool ok = row < n;
    float kf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) kf[e] = ok ? elt(kv[m], e) : 0.f;
    *reinterpret_cast<float4 *>(&sm.r[row][col]) = make_float4(kf[0], kf[1], kf[2], kf[3]);
    *reinterpret_cast<float4 *>(&sm.r[row][col + 4]) = make_float4(kf[4], kf[5], kf[6], kf[7]);
    const float s = bt[m];
    *reinterpret_cast<float4 *>(&sm.x[row][col]) = make_float4(s * kf[0], s * kf[1], s * kf[2], s * kf[3]);
    *reinterpret_cast<float4 *>(&sm.x[row][col + 4]) = make_float4(s * kf[4], s * kf[5], s * kf[6], s * kf[7]);
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int w = tid + kNT * m, row = w >> 5, col = 4 * (w & 31);
    const float4 v = lv[m];
    *reinterpret_cast<float4 *>(&sm.g[row][col]) =
        row < n ? make_float4(v.x * kLog2e, v.y * kLog2e, v.z * kLog2e, v.w * kLog2e) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __syncthreads();

  // G: inclusive scan over the chunk per channel; thread (segment tid / 128, channel tid % 128)
  // scans its 16 tokens, then adds the sums of the segments before it
  {
    const int ch = tid & (kD - 1), seg = tid >> 7;
    float gl[16], run = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      run += sm.g[16 * seg + i][ch];
      gl[i] = run;
    }
    sm.tot[seg][ch] = run;
    __syncthreads();
    float off = 0.f;
    for (int s = 0; s < seg; ++s) off += sm.tot[s][ch];
#pragma unroll
    for (int i = 0; i < 16; ++i) sm.g[16 * seg + i][ch] = gl[i] + off;
  }
  __syncthreads();

  // the decayed operands of the sequential pass (rows of the chunk only)
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int u = tid + kNT * m, row = u >> 4, col = 8 * (u & 15);
    if (row < n) {
      float fq[8], fe[8], fr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gv = sm.g[row][col + e], gl = sm.g[kC - 1][col + e];
        const float up = ex2(gv), dn = ex2(gl - gv);
        fq[e] = elt(qv[m], e) * up;
        fe[e] = elt(kv[m], e) * up;
        fr[e] = elt(kv[m], e) * dn;
      }
      const long long o = base + row * tokstride + col;
      *reinterpret_cast<uint4 *>(qt + o) = pack8(fq);
      *reinterpret_cast<uint4 *>(et + o) = pack8(fe);
      *reinterpret_cast<uint4 *>(rt + o) = pack8(fr);
    }
  }

  // L, then P over the same decayed key products (the queries replace beta (.) k)
  chd::gram<kD, kLD, kLP>(sm.x, sm.r, sm.g, sm.l, false, tid);
  __syncthreads();
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int u = tid + kNT * m, row = u >> 4, col = 8 * (u & 15);
    const bool ok = row < n;
    float qf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[e] = ok ? elt(qv[m], e) : 0.f;
    *reinterpret_cast<float4 *>(&sm.x[row][col]) = make_float4(qf[0], qf[1], qf[2], qf[3]);
    *reinterpret_cast<float4 *>(&sm.x[row][col + 4]) = make_float4(qf[4], qf[5], qf[6], qf[7]);
  }
  __syncthreads();
  chd::gram<kD, kLD, kLP>(sm.x, sm.r, sm.g, sm.p, true, tid);
  // T = (I - A)^-1 from L (published before the last barrier); ends with a barrier, after which
  // P is complete too
  tri::inverse_blocks<kLP, kLP>(sm.l, sm.t, sm.z, -1, tid);

  uint16_t *const dst = rec + (static_cast<long long>(b * H + h) * nchunks + c) * (kRecItems * 8);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int u = tid + kNT * m;
    if (u < 960) {
      const bool isT = u < 640;
      const int v = isT ? u : u - 640;
      const int q = isT ? v >> 6 : v >> 5;
      const int ib = q < 1 ? 0 : q < 3 ? 1 : q < 6 ? 2 : 3, jb = q - ib * (ib + 1) / 2;
      const int i = 16 * ib + ((v >> 1) & 15), j0 = 16 * jb + 8 * (v & 1);
      const bool lo = isT && ((v >> 5) & 1);
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = j0 + e;
        const float t = (j <= i) ? (isT ? sm.t[i][j] : sm.p[i][j]) : 0.f;
        x[e] = lo ? t - bf16_bits_to_f32(f32_to_bf16_bits(t)) : t;
      }
      *reinterpret_cast<uint4 *>(dst + 8 * u) = pack8(x);
    } else if (u < kRecItems) {
      const int ch = 4 * (u - 960);
      const float4 gl = *reinterpret_cast<const float4 *>(&sm.g[kC - 1][ch]);
      *reinterpret_cast<float4 *>(dst + 8 * u) = make_float4(ex2(gl.x), ex2(gl.y), ex2(gl.z), ex2(gl.w));
    }
  }
}

}  // namespace

hipError_t launch_kda_prep(const ChunkArgs &a, uint16_t *qt, uint16_t *et, uint16_t *rt, uint16_t *rec,
                           hipStream_t s) {
  const int nchunks = (a.T + kC - 1) / kC;
  if (nchunks == 0) return hipSuccess;
  hipLaunchKernelGGL(kda_prep_kernel, dim3(nchunks, a.H, a.B), dim3(kNT), 0, s, a, qt, et, rt, rec);
  return hipGetLastError();
}

}  // namespace gdr
