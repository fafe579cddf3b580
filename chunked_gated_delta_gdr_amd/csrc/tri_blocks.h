// Blocked inverse of a chunk's unit lower-triangular matrix, shared by the forward and
// backward kernels (fp32 on the matrix cores).
#pragma once

#include "common.h"

namespace gdr {
namespace tri {

typedef float f4v __attribute__((ext_vector_type(4)));

// one 16 x 16 x 4 fp32 matrix-core step: lane l gives A[l % 16][l / 16] and B[l / 16][l % 16]
// and holds D[4 (l / 16) + r][l % 16], r < 4
__device__ __forceinline__ f4v mma(float a, float b, f4v c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }

// LDS writes of this wave become visible to its own later reads
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// T = (I - A)^-1 for the strictly lower-triangular A = -L of one chunk of up to 64 tokens
// (chunk-wise form of the MatMul-only inversion summary, "Declaracao do Problema"), by a
// workgroup of at least 4 waves, as blocked forward substitution in 16 x 16 blocks on the fp32
// matrix cores.  Each diagonal block D_b = (I - A_bb)^-1 (one wave each): substitution inside
// its four 4 x 4 diagonal sub-blocks, then two levels of block products D <- D + D N_m D, N_m the
// part of A_bb that joins the blocks of the level (the 4 x 4 blocks (1, 0) and (3, 2), then the
// 8 x 8 block (1, 0)), since the inverse of [[P, 0], [M, Q]] has Q^-1 M P^-1 below its diagonal.
// Then T_10 = D_1 A_10 D_0, T_32 = D_3 A_32 D_2 and the lower-left quadrant T_ba = T_b A_ba T_a
// (a, b the 32 x 32 halves) as block products.  Every intermediate is part of the inverse, so no
// factor grows past |T| (unlike the powers of A in a Neumann product form, which dwarf T when
// keys are correlated or gains exceed 1).  Every block is band-masked when it is written (N >= 0
// keeps i - j <= N; N < 0 keeps all): an in-band entry of a product of lower-triangular factors
// reads only in-band entries of them (Lemma 3.1, Metodologia 1), and the same holds for the
// substitution, so the band entries are those of the exact path, bit for bit, and N >= n - 1
// runs the exact path's instructions.  Rows of L past the chunk must be zero (their T rows come
// out unit rows), and the 16 x 16 blocks of Tm above the diagonal must hold zero on entry (they
// are never written).  Zs is 32 x 36 scratch, 16-byte aligned, as are the rows of Tm.  Starts
// reading L without a barrier (the caller publishes it) and ends with a workgroup barrier.
template <int LDL, int LDT>
__device__ __forceinline__ void inverse_blocks(const float (*LP)[LDL], float (*Tm)[LDT], float (*Zs)[36], int N,
                                               int tid) {
  auto keep = [&](int i, int j) { return N < 0 || i - j <= N; };
  const int lane = tid & 63, w = tid >> 6, col = lane & 15, kq = lane >> 4;
  if (w < 4) {   // diagonal block w, from P = A_bb held in the wave's scratch
    const int o = 16 * w;
    float *Pw = &Zs[0][0] + 288 * w;   // 16 x 16, row stride 16
    for (int e = lane; e < 256; e += 64) {
      const int i = e >> 4, j = e & 15;
      Pw[e] = j < i ? -LP[o + i][o + j] : 0.f;
    }
    wave_sync();
    // 4 x 4 sub-blocks: lane (col, kq) forms column col of its sub-block sb = col / 4,
    // x_r = [r == col % 4] + sum_{l < r} P_rl x_l, and keeps rows 4 kq .. 4 kq + 3 of the block
    // diagonal D1 (its accumulator layout: zero unless kq == sb)
    f4v d;
    {
      const int sb = col >> 2, jj = col & 3;
      const float *Ps = Pw + 16 * (4 * sb) + 4 * sb;   // P_rl = Ps[16 r + l]
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float acc = r == jj ? 1.f : 0.f;
#pragma unroll
        for (int l = 0; l < r; ++l) acc = fmaf(Ps[16 * r + l], x[l], acc);
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) d[r] = kq == sb ? x[r] : 0.f;
    }
    // the levels: Z = N_m D (A operand from P's rows, masked; B operand the accumulator of D with
    // the K order 4 kq + s, so a lane's own registers are its B values), then D + D Z (A operand
    // from D's rows, published to the block of Tm first)
#pragma unroll 1
    for (int lev = 0; lev < 2; ++lev) {
#pragma unroll
      for (int r = 0; r < 4; ++r) Tm[o + 4 * kq + r][o + col] = d[r];
      const int rb = lev == 0 ? col >> 2 : col >> 3;   // row block of N_m at this lane's row
      const bool nz = lev == 0 ? ((rb & 1) != 0 && kq == rb - 1) : (rb == 1 && (kq >> 1) == 0);
      wave_sync();
      f4v z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) z = mma(nz ? Pw[16 * col + 4 * kq + s] : 0.f, d[s], z);
#pragma unroll
      for (int s = 0; s < 4; ++s) d = mma(Tm[o + col][o + 4 * kq + s], z[s], d);
      wave_sync();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * kq + r;
      Tm[o + i][o + col] = keep(i, col) ? d[r] : 0.f;
    }
  }
  __syncthreads();
  if (w < 2) {   // Z_p = A_(2p+1, 2p) D_2p, p = w
    const int ro = 32 * w + 16, co = 32 * w;
    f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mma(-LP[ro + col][co + 4 * s + kq], Tm[co + 4 * s + kq][co + col], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) Zs[16 * w + 4 * kq + r][col] = acc[r];
  }
  __syncthreads();
  if (w < 2) {   // T_(2p+1, 2p) = D_(2p+1) Z_p
    const int ro = 32 * w + 16, co = 32 * w;
    f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mma(Tm[ro + col][ro + 4 * s + kq], Zs[16 * w + 4 * s + kq][col], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = ro + 4 * kq + r, j = co + col;
      Tm[i][j] = keep(i, j) ? acc[r] : 0.f;
    }
  }
  __syncthreads();
  const int zi = (w >> 1) & 1, zj = w & 1;   // 16 x 16 tile of the 32 x 32 products (waves 0..3)
  if (w < 4) {   // Z = A_ba T_a (T_a lower: k from 16 zj)
    f4v acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 4 * zj; s < 8; ++s) acc = mma(-LP[32 + 16 * zi + col][4 * s + kq], Tm[4 * s + kq][16 * zj + col], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) Zs[16 * zi + 4 * kq + r][16 * zj + col] = acc[r];
  }
  __syncthreads();
  if (w < 4) {   // T_ba = T_b Z (T_b lower: k below 16 zi + 16)
    f4v acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < 4 * (zi + 1); ++s)
      acc = mma(Tm[32 + 16 * zi + col][32 + 4 * s + kq], Zs[4 * s + kq][16 * zj + col], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 32 + 16 * zi + 4 * kq + r, j = 16 * zj + col;
      Tm[i][j] = keep(i, j) ? acc[r] : 0.f;
    }
  }
  __syncthreads();
}

}  // namespace tri
}  // namespace gdr
