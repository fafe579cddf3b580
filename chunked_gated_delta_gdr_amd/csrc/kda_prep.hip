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
// Two routes form L and P.  The fast one references every decay to the chunk's start:
// 2^(G_ic - G_jc) = 2^G_ic 2^-G_jc, so with K^ = 2^-G (.) k, L = beta (.) tril_-1(E~ K^T) and
// P = tril(Q~ K^T), products of operands prepared once, on the bf16 matrix cores with each
// operand as a hi / lo pair (X_hi Y_hi + X_lo Y_hi + X_hi Y_lo, about 16 significant bits).
// Its factors stay in range while every channel's cumulative decay over the chunk is at least
// 2^-120 (G >= -120 in log2 units); a chunk that decays further is flagged and formed again by
// the robust route, a second launch that leaves unflagged chunks alone.
//
// Robust route: L and P in fp32, formed together: every decay factor serves both, since they differ only in
// the row operand (beta (.) k against q).  The tiles below the diagonal go to the fp32 matrix
// cores with the decay split at the last row of the column block (both factors <= 1); the
// diagonal tiles stay on the vector ALUs in 4 x 4 sub-blocks, those below the sub-block
// diagonal split the same way, the diagonal sub-blocks one factor per pair (this is the
// per-channel Gram route of the fp32 kernel, chd_gram.h, for two outputs at once).  The key
// channels run in two halves of 64 (keys and queries as bf16 in LDS, G in fp32), the products
// accumulating in registers across them, so a workgroup needs 78 KB of LDS and two share a
// CU.  T follows by the blocked forward substitution of tri_blocks.h in fp32.  Per chunk one
// record of 15872 bytes:
//   T   the ten 16 x 16 blocks on and below the diagonal, block q = ib (ib + 1) / 2 + jb, each
//       as its bf16 hi part then its lo part (T - hi, rounded), 16 rows of 16 (10240 bytes)
//   P   the same ten blocks as single bf16, 16 rows of 16 (5120 bytes)
//   gC  128 fp32 (512 bytes)
// The record is read as 16-byte items u < 992, item u at byte 16 u.
#include "common.h"
#include "tri_blocks.h"

namespace gdr {
namespace {

constexpr int kC = 64;
constexpr int kD = 128;
constexpr int kHC = 64;        // key channels per half
constexpr int kNT = 512;
constexpr int kKL = kHC + 8;   // bf16 row stride of the half key / query tiles (144 bytes)
constexpr int kGL = kHC + 4;   // fp32 row stride of the half G tile
constexpr int kLP = kC + 4;    // fp32 row stride of the 64 x 64 tiles
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRecItems = 992;   // 16-byte items of a chunk's record

typedef float f4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f4v mfma32(short8v a, short8v b, f4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
constexpr float kFastMin = -120.f;   // smallest G (log2 units) the fast route takes
__device__ __forceinline__ f4v mma(float a, float b, f4v c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }
// 2^x by one v_exp_f32 (every kept exponent is <= 0; results below 2^-126 flush to zero, where
// they are negligible against the O(1) terms they join)
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float elt(const uint4 &v, int e) {
  const uint32_t w = (&v.x)[e >> 1];
  return bf16_bits_to_f32((e & 1) ? (w >> 16) : (w & 0xffffu));
}
__device__ __forceinline__ uint4 pack8(const float (&x)[8]) {
  return make_uint4(f32x2_to_bf16x2_bits(x[0], x[1]), f32x2_to_bf16x2_bits(x[2], x[3]),
                    f32x2_to_bf16x2_bits(x[4], x[5]), f32x2_to_bf16x2_bits(x[6], x[7]));
}
// four consecutive bf16 channels as floats (one 8-byte LDS read)
__device__ __forceinline__ float4 ld4b(const uint16_t *p) {
  const uint2 w = *reinterpret_cast<const uint2 *>(p);
  return make_float4(bf16_bits_to_f32(w.x & 0xffffu), bf16_bits_to_f32(w.x >> 16), bf16_bits_to_f32(w.y & 0xffffu),
                     bf16_bits_to_f32(w.y >> 16));
}
__device__ __forceinline__ float4 ld4f(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float dot4(const float4 &x, const float4 &y) {
  return fmaf(x.x, y.x, fmaf(x.y, y.y, fmaf(x.z, y.z, x.w * y.w)));
}
__device__ __forceinline__ float4 mul4(const float4 &x, const float4 &y) {
  return make_float4(x.x * y.x, x.y * y.y, x.z * y.z, x.w * y.w);
}
__device__ __forceinline__ float4 ex24(const float4 &x, const float4 &y) {   // 2^(x - y)
  return make_float4(ex2(x.x - y.x), ex2(x.y - y.y), ex2(x.z - y.z), ex2(x.w - y.w));
}

struct __align__(16) PrepSmem {
  union {
    struct {
      uint16_t k[kC][kKL];   // keys of one half of the channels
      uint16_t q[kC][kKL];   // queries
      float g[kC][kGL];      // log2 decays, then G (in-chunk inclusive cumulative sum)
    } h;
    float t[kC][kLP];        // T, once the Gram products are done
  } u;
  float l[kC][kLP];     // L (A = -L): strictly lower
  float p[kC][kLP];     // P: lower with the diagonal
  float z[32][36];      // the inverse's scratch
  float tot[8][kHC];    // sums of the scan's eight 8-token segments
  float glast[kD];      // G at the chunk's last token, every channel
  float beta[kC];
};

__global__ __launch_bounds__(kNT, 4) void kda_prep_robust_kernel(ChunkArgs a, uint16_t *qt, uint16_t *et,
                                                                 uint16_t *rt, uint16_t *rec, const uint32_t *flags) {
  // only the chunks the fast route flagged
  const int nch = (a.T + kC - 1) / kC;
  if (flags[(static_cast<long long>(blockIdx.z) * a.H + blockIdx.y) * nch + blockIdx.x] == 0) return;
  __shared__ PrepSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 15, kq = lane >> 4;
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

  // This thread's items: keys and queries at row irow, channels 64 hf + ich .. + 7 of half hf;
  // log decays at rows (tid + 512 m) / 16, channels 64 hf + 4 ((tid + 512 m) % 16) .. + 3.  Rows
  // past the end of the sequence read the last row and are zeroed (zero keys, no decay: G stays
  // constant past the chunk's last token).
  const int irow = tid >> 3, ich = 8 * (tid & 7);
  const bool iok = irow < n;
  if (tid < kC) sm.beta[tid] = tid < n ? a.beta[gate0 + static_cast<long long>(tid) * H] : 0.f;

  // Gram accumulators, kept across the two halves.  Waves 0..5: tile `wave` of the six below
  // the diagonal (row by row: (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)); waves 0..3 also the four
  // diagonal 4 x 4 sub-blocks of diagonal tile `wave` (lane: sub-block lane / 16, channels
  // 4 (lane % 16) .. of the half), waves 4..7 the six lower 4 x 4 sub-blocks of diagonal tile
  // wave - 4 (lane: pair lane / 8 < 6, channels 8 (lane % 8) .. of the half).
  f4v oL = {0.f, 0.f, 0.f, 0.f}, oP = {0.f, 0.f, 0.f, 0.f};
  float dL[4][4], dP[4][4];
  const int ut = wave, tib = ut < 1 ? 1 : ut < 3 ? 2 : 3, tjb = ut - (tib - 1) * tib / 2;   // (wave < 6)
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) dL[u][w] = dP[u][w] = 0.f;
  const int sb = lane >> 3;   // (waves 4..7) sub-block pair
  const int pbi = sb < 1 ? 1 : sb < 3 ? 2 : 3, pbj = min(sb - (pbi - 1) * pbi / 2, pbi - 1);

  // (lane offsets in 32 bits from the uniform bases: 64 rows of at most 65535 heads of 128 channels)
  const int tok32 = H * kD;
#pragma unroll 1
  for (int hf = 0; hf < 2; ++hf) {
    uint4 kv, qv;
    float4 lv[2];
    {
      const int o = min(irow, n - 1) * tok32 + kHC * hf + ich;
      kv = *reinterpret_cast<const uint4 *>(gk + o);
      qv = *reinterpret_cast<const uint4 *>(gq + o);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int w = tid + kNT * m;
        lv[m] = *reinterpret_cast<const float4 *>(gla + (min(w >> 4, n - 1) * tok32 + kHC * hf + 4 * (w & 15)));
      }
    }
    if (hf == 1) __syncthreads();   // every read of the first half's tiles done
    *reinterpret_cast<uint4 *>(&sm.u.h.k[irow][ich]) = iok ? kv : make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4 *>(&sm.u.h.q[irow][ich]) = iok ? qv : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int w = tid + kNT * m, row = w >> 4;
      const float4 v = lv[m];
      *reinterpret_cast<float4 *>(&sm.u.h.g[row][4 * (w & 15)]) =
          row < n ? make_float4(v.x * kLog2e, v.y * kLog2e, v.z * kLog2e, v.w * kLog2e) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    {   // G: inclusive scan over the chunk; thread (segment tid / 64 of 8 tokens, channel tid % 64)
      const int ch = tid & (kHC - 1), sg = tid >> 6;
      float gl[8], run = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        run += sm.u.h.g[8 * sg + i][ch];
        gl[i] = run;
      }
      sm.tot[sg][ch] = run;
      __syncthreads();
      float off = 0.f;
      for (int s2 = 0; s2 < sg; ++s2) off += sm.tot[s2][ch];
#pragma unroll
      for (int i = 0; i < 8; ++i) sm.u.h.g[8 * sg + i][ch] = gl[i] + off;
      if (sg == 7) sm.glast[kHC * hf + ch] = gl[7] + off;
    }
    __syncthreads();
    // the decayed operands of the sequential pass, this half's channels (rows of the chunk only)
    if (iok) {
      float fq[8], fe[8], fr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gv = sm.u.h.g[irow][ich + e], gl = sm.u.h.g[kC - 1][ich + e];
        const float up = ex2(gv), dn = ex2(gl - gv);
        fq[e] = elt(qv, e) * up;
        fe[e] = elt(kv, e) * up;
        fr[e] = elt(kv, e) * dn;
      }
      const int o = irow * tok32 + kHC * hf + ich;
      *reinterpret_cast<uint4 *>(qt + base + o) = pack8(fq);
      *reinterpret_cast<uint4 *>(et + base + o) = pack8(fe);
      *reinterpret_cast<uint4 *>(rt + base + o) = pack8(fr);
    }
    // Gram products of this half
    const uint16_t(*K)[kKL] = sm.u.h.k;
    const uint16_t(*Q)[kKL] = sm.u.h.q;
    const float(*Gs)[kGL] = sm.u.h.g;
    if (wave < 6) {
      const int ref = 16 * tjb + 15, i = 16 * tib + col, j = 16 * tjb + col;
      // (K order permuted: sub-step e of block ks takes channel ks + 4 kq + e)
#pragma unroll 2
      for (int ks = 0; ks < kHC; ks += 16) {
            const int kk = ks + 4 * kq;
            const float4 gr = ld4f(&Gs[ref][kk]);
            const float4 fi = ex24(ld4f(&Gs[i][kk]), gr);
            const float4 bj = mul4(ld4b(&K[j][kk]), ex24(gr, ld4f(&Gs[j][kk])));
            const float4 xk = mul4(ld4b(&K[i][kk]), fi), xq = mul4(ld4b(&Q[i][kk]), fi);
        oL = mma(xk.x, bj.x, oL);
        oP = mma(xq.x, bj.x, oP);
        oL = mma(xk.y, bj.y, oL);
        oP = mma(xq.y, bj.y, oP);
        oL = mma(xk.z, bj.z, oL);
        oP = mma(xq.z, bj.z, oP);
        oL = mma(xk.w, bj.w, oL);
        oP = mma(xq.w, bj.w, oP);
      }
    }
    if (wave < 4) {
      // diagonal sub-block kq of diagonal tile `wave`, channels 4 col .. + 3: one factor per pair
      const int i0 = 16 * wave + 4 * kq, ch = 4 * col;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 xk = ld4b(&K[i0 + u][ch]), xq = ld4b(&Q[i0 + u][ch]), gi = ld4f(&Gs[i0 + u][ch]);
#pragma unroll
        for (int w = 0; w <= u; ++w) {
          float4 r = ld4b(&K[i0 + w][ch]);
          if (w < u) r = mul4(r, ex24(gi, ld4f(&Gs[i0 + w][ch])));
          dL[u][w] += dot4(xk, r);
          dP[u][w] += dot4(xq, r);
        }
      }
    } else if (sb < 6) {
      // lower sub-block (pbi, pbj) of diagonal tile wave - 4, channels 8 (lane % 8) .. + 7, the
      // decay split at the last row of the column sub-block
      const int d = wave - 4;
      const int i0 = 16 * d + 4 * pbi, j0 = 16 * d + 4 * pbj, ref = j0 + 3;
#pragma unroll
      for (int cc = 0; cc < 8; cc += 4) {
        const int ch = 8 * (lane & 7) + cc;
        const float4 gr = ld4f(&Gs[ref][ch]);
        float4 rr[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) rr[w] = mul4(ld4b(&K[j0 + w][ch]), ex24(gr, ld4f(&Gs[j0 + w][ch])));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 f = ex24(ld4f(&Gs[i0 + u][ch]), gr);
          const float4 xk = mul4(ld4b(&K[i0 + u][ch]), f), xq = mul4(ld4b(&Q[i0 + u][ch]), f);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            dL[u][w] += dot4(xk, rr[w]);
            dP[u][w] += dot4(xq, rr[w]);
          }
        }
      }
    }
  }

  // sums over the lanes that split the channels of a sub-block
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    if (wave >= 4 && m == 8) break;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        dL[u][w] += __shfl_xor(dL[u][w], m);
        dP[u][w] += __shfl_xor(dP[u][w], m);
      }
  }
  // L (rows scaled by beta) and P to LDS
  if (wave < 6) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * tib + 4 * kq + r, j = 16 * tjb + col;
      sm.l[i][j] = oL[r] * sm.beta[i];
      sm.p[i][j] = oP[r];
    }
  }
  if (wave < 4) {
    if (col == 0) {
      const int i0 = 16 * wave + 4 * kq;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          sm.l[i0 + u][i0 + w] = w < u ? dL[u][w] * sm.beta[i0 + u] : 0.f;
          sm.p[i0 + u][i0 + w] = w <= u ? dP[u][w] : 0.f;
        }
    }
  } else if ((lane & 7) == 0 && sb < 6) {
    const int d = wave - 4;
    const int i0 = 16 * d + 4 * pbi, j0 = 16 * d + 4 * pbj;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        sm.l[i0 + u][j0 + w] = dL[u][w] * sm.beta[i0 + u];
        sm.p[i0 + u][j0 + w] = dP[u][w];
      }
  }
  // the six 4 x 4 blocks above the sub-block diagonal of each diagonal tile hold zeros
  if (tid < 4 * 6 * 16) {
    const int dt = tid / 96, ub = (tid % 96) / 16, en = tid % 16;
    const int ubi = ub < 3 ? 0 : ub < 5 ? 1 : 2;
    const int ubj = ub < 3 ? ub + 1 : ub < 5 ? ub - 1 : 3;
    const int i = 16 * dt + 4 * ubi + (en >> 2), j = 16 * dt + 4 * ubj + (en & 3);
    sm.l[i][j] = 0.f;
    sm.p[i][j] = 0.f;
  }
  __syncthreads();   // L, P complete; every read of the half tiles done (T takes their space)
  for (int i = tid; i < kC * kLP; i += kNT) (&sm.u.t[0][0])[i] = 0.f;
  __syncthreads();
  // T = (I - A)^-1 from L; ends with a barrier
  tri::inverse_blocks<kLP, kLP>(sm.l, sm.u.t, sm.z, -1, tid);

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
        const float t = (j <= i) ? (isT ? sm.u.t[i][j] : sm.p[i][j]) : 0.f;
        x[e] = lo ? t - bf16_bits_to_f32(f32_to_bf16_bits(t)) : t;
      }
      *reinterpret_cast<uint4 *>(dst + 8 * u) = pack8(x);
    } else if (u < kRecItems) {
      const int ch = 4 * (u - 960);
      const float4 gl = ld4f(&sm.glast[ch]);
      *reinterpret_cast<float4 *>(dst + 8 * u) = make_float4(ex2(gl.x), ex2(gl.y), ex2(gl.z), ex2(gl.w));
    }
  }
}

// ------------------------------- the fast route -------------------------------
constexpr int kOL = kHC + 8;   // bf16 row stride of the prepared operand tiles (144 bytes)

struct __align__(16) FastSmem {
  union {
    struct {
      uint16_t e[2][kC][kOL];   // E~ = 2^G (.) k as hi, lo (one half of the channels)
      uint16_t q[2][kC][kOL];   // Q~ = 2^G (.) q
      uint16_t r[2][kC][kOL];   // K^ = 2^-G (.) k
      float g[kC][kGL];         // log2 decays, then G
    } h;
    struct {
      float l[kC][kLP];   // L
      float p[kC][kLP];   // P
      float t[kC][kLP];   // T
      float z[32][36];    // the inverse's scratch
    } f;
  } u;
  float tot[8][kHC];
  float glast[kD];
  float beta[kC];
  int flag;
};

__device__ __forceinline__ short8v ld16(const uint16_t *p) { return *reinterpret_cast<const short8v *>(p); }
__device__ __forceinline__ void split8(const float (&x)[8], uint4 &hi, uint4 &lo) {
  float h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = bf16_bits_to_f32(f32_to_bf16_bits(x[e]));
    l[e] = x[e] - h[e];
  }
  hi = pack8(h);
  lo = pack8(l);
}

__global__ __launch_bounds__(kNT, 4) void kda_prep_fast_kernel(ChunkArgs a, uint16_t *qt, uint16_t *et, uint16_t *rt,
                                                               uint16_t *rec, uint32_t *flags) {
  __shared__ FastSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, l4 = lane >> 4;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int H = a.H, T = a.T;
  const int nchunks = (T + kC - 1) / kC;
  const int c0 = c * kC, n = min(kC, T - c0);
  const long long tokstride = static_cast<long long>(H) * kD;
  const long long base = (static_cast<long long>(b) * T * H + h) * kD + static_cast<long long>(c0) * tokstride;
  const long long gate0 = static_cast<long long>(b) * T * H + h + static_cast<long long>(c0) * H;
  const uint16_t *gq = static_cast<const uint16_t *>(a.q) + base;
  const uint16_t *gk = static_cast<const uint16_t *>(a.k) + base;
  const float *gla = a.log_alpha + base;
  const int tok32 = H * kD;   // (lane offsets in 32 bits: 64 rows of at most 65535 heads of 128 channels)
  // this thread's items, as in the robust route: keys / queries at row irow, channels
  // 64 hf + ich .. + 7; log decays at rows (tid + 512 m) / 16, channels 64 hf + 4 ((tid + 512 m) % 16)
  const int irow = tid >> 3, ich = 8 * (tid & 7);
  const bool iok = irow < n;
  if (tid < kC) sm.beta[tid] = tid < n ? a.beta[gate0 + static_cast<long long>(tid) * H] : 0.f;
  if (tid == 0) sm.flag = 0;

  // the ten 16 x 16 tiles on and below the diagonal: wave w owns tiles w and w + 8 (< 10),
  // tile u < 6 below the diagonal (row by row (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)), u >= 6 the
  // diagonal tile u - 6
  auto tile_rc = [](int u, int &ib, int &jb) {
    if (u >= 6) {
      ib = jb = u - 6;
    } else {
      ib = u < 1 ? 1 : u < 3 ? 2 : 3;
      jb = u - (ib - 1) * ib / 2;
    }
  };
  f4v accL[2], accP[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) accL[s] = accP[s] = f4v{0.f, 0.f, 0.f, 0.f};

#pragma unroll 1
  for (int hf = 0; hf < 2; ++hf) {
    uint4 kv, qv;
    float4 lv[2];
    {
      const int o = min(irow, n - 1) * tok32 + kHC * hf + ich;
      kv = *reinterpret_cast<const uint4 *>(gk + o);
      qv = *reinterpret_cast<const uint4 *>(gq + o);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int w = tid + kNT * m;
        lv[m] = *reinterpret_cast<const float4 *>(gla + (min(w >> 4, n - 1) * tok32 + kHC * hf + 4 * (w & 15)));
      }
    }
    if (hf == 1) __syncthreads();   // every read of the first half's tiles done
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int w = tid + kNT * m, row = w >> 4;
      const float4 v = lv[m];
      *reinterpret_cast<float4 *>(&sm.u.h.g[row][4 * (w & 15)]) =
          row < n ? make_float4(v.x * kLog2e, v.y * kLog2e, v.z * kLog2e, v.w * kLog2e) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    {   // G: inclusive scan over the chunk (segment tid / 64 of 8 tokens, channel tid % 64)
      const int ch = tid & (kHC - 1), sg = tid >> 6;
      float gl[8], run = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        run += sm.u.h.g[8 * sg + i][ch];
        gl[i] = run;
      }
      sm.tot[sg][ch] = run;
      __syncthreads();
      float off = 0.f;
      for (int s2 = 0; s2 < sg; ++s2) off += sm.tot[s2][ch];
#pragma unroll
      for (int i = 0; i < 8; ++i) sm.u.h.g[8 * sg + i][ch] = gl[i] + off;
      if (sg == 7) {
        const float gz = gl[7] + off;   // the smallest G of the channel
        sm.glast[kHC * hf + ch] = gz;
        // (wave 7: one lane per channel) the chunk leaves the fast route's range?
        if (__any(gz < kFastMin) && lane == 0) sm.flag = 1;
      }
    }
    __syncthreads();
    {   // outputs and the prepared operand pairs of this half (item irow, ich .. + 7)
      float fq[8], fe[8], fr[8], fk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gv = sm.u.h.g[irow][ich + e], gl = sm.u.h.g[kC - 1][ich + e];
        const float up = ex2(gv), dn = ex2(gl - gv), rk = ex2(-gv);
        const float kx = iok ? elt(kv, e) : 0.f, qx = iok ? elt(qv, e) : 0.f;
        fq[e] = qx * up;
        fe[e] = kx * up;
        fr[e] = kx * dn;
        fk[e] = kx * rk;
      }
      if (iok) {
        const int o = irow * tok32 + kHC * hf + ich;
        *reinterpret_cast<uint4 *>(qt + base + o) = pack8(fq);
        *reinterpret_cast<uint4 *>(et + base + o) = pack8(fe);
        *reinterpret_cast<uint4 *>(rt + base + o) = pack8(fr);
      }
      uint4 hi, lo;
      split8(fe, hi, lo);
      *reinterpret_cast<uint4 *>(&sm.u.h.e[0][irow][ich]) = hi;
      *reinterpret_cast<uint4 *>(&sm.u.h.e[1][irow][ich]) = lo;
      split8(fq, hi, lo);
      *reinterpret_cast<uint4 *>(&sm.u.h.q[0][irow][ich]) = hi;
      *reinterpret_cast<uint4 *>(&sm.u.h.q[1][irow][ich]) = lo;
      split8(fk, hi, lo);
      *reinterpret_cast<uint4 *>(&sm.u.h.r[0][irow][ich]) = hi;
      *reinterpret_cast<uint4 *>(&sm.u.h.r[1][irow][ich]) = lo;
    }
    __syncthreads();
    // Gram tiles of this half: lane l gives row l % 16 of the A operand (E~ or Q~ rows of block
    // ib) and column l % 16 of the B operand (K^ rows of block jb), K slots 8 (l / 16) .. + 7
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int u = wave + 8 * s;
      if (u < 10) {
        int ib, jb;
        tile_rc(u, ib, jb);
#pragma unroll
        for (int k0 = 0; k0 < kHC; k0 += 32) {
          const int kk = k0 + 8 * l4;
          const short8v bh = ld16(&sm.u.h.r[0][16 * jb + l16][kk]), bl = ld16(&sm.u.h.r[1][16 * jb + l16][kk]);
          const short8v eh = ld16(&sm.u.h.e[0][16 * ib + l16][kk]), el = ld16(&sm.u.h.e[1][16 * ib + l16][kk]);
          const short8v qh = ld16(&sm.u.h.q[0][16 * ib + l16][kk]), ql = ld16(&sm.u.h.q[1][16 * ib + l16][kk]);
          accL[s] = mfma32(eh, bl, mfma32(el, bh, mfma32(eh, bh, accL[s])));
          accP[s] = mfma32(qh, bl, mfma32(ql, bh, mfma32(qh, bh, accP[s])));
        }
      }
    }
  }
  __syncthreads();   // every read of the operand tiles done: L, P, T take their space
  const bool flagged = sm.flag != 0;
  // lane: rows 16 ib + 4 (l / 16) + r, column 16 jb + l % 16 of its tiles
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int u = wave + 8 * s;
    if (u < 10) {
      int ib, jb;
      tile_rc(u, ib, jb);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ib + 4 * l4 + r, j = 16 * jb + l16;
        sm.u.f.l[i][j] = j < i ? accL[s][r] * sm.beta[i] : 0.f;
        sm.u.f.p[i][j] = j <= i ? accP[s][r] : 0.f;
      }
    }
  }
  for (int i = tid; i < kC * kLP; i += kNT) (&sm.u.f.t[0][0])[i] = 0.f;
  if (tid == 0) flags[(static_cast<long long>(b) * H + h) * nchunks + c] = flagged ? 1u : 0u;
  __syncthreads();
  if (flagged) return;   // (workgroup-uniform) the robust route forms this chunk
  // T = (I - A)^-1 from L; ends with a barrier
  tri::inverse_blocks<kLP, kLP>(sm.u.f.l, sm.u.f.t, sm.u.f.z, -1, tid);

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
        const float t = (j <= i) ? (isT ? sm.u.f.t[i][j] : sm.u.f.p[i][j]) : 0.f;
        x[e] = lo ? t - bf16_bits_to_f32(f32_to_bf16_bits(t)) : t;
      }
      *reinterpret_cast<uint4 *>(dst + 8 * u) = pack8(x);
    } else if (u < kRecItems) {
      const int ch = 4 * (u - 960);
      const float4 gl = ld4f(&sm.glast[ch]);
      *reinterpret_cast<float4 *>(dst + 8 * u) = make_float4(ex2(gl.x), ex2(gl.y), ex2(gl.z), ex2(gl.w));
    }
  }
}

}  // namespace

hipError_t launch_kda_prep(const ChunkArgs &a, uint16_t *qt, uint16_t *et, uint16_t *rt, uint16_t *rec,
                           uint32_t *flags, hipStream_t s) {
  const int nchunks = (a.T + kC - 1) / kC;
  if (nchunks == 0) return hipSuccess;
  const dim3 grid(nchunks, a.H, a.B);
  hipLaunchKernelGGL(kda_prep_fast_kernel, grid, dim3(kNT), 0, s, a, qt, et, rt, rec, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kda_prep_robust_kernel, grid, dim3(kNT), 0, s, a, qt, et, rt, rec, flags);
  return hipGetLastError();
}

}  // namespace gdr
