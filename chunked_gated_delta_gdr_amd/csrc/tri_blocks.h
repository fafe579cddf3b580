// Blocked inverse of a chunk's unit lower-triangular matrix, shared by the forward and
// backward kernels.
#pragma once

#include "common.h"

namespace gdr {
namespace tri {

__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float2 ld2(const float *p) { return *reinterpret_cast<const float2 *>(p); }

// T = (I - A)^-1 for the strictly lower-triangular A = -L of one chunk of up to 64 tokens
// (chunk-wise form of the MatMul-only inversion summary, "Declaracao do Problema"), by one
// workgroup of 256 threads, in 16 x 16 blocks.  With D_b = (I - A_bb)^-1 (the four diagonal
// blocks, solved at once, one wave each, by right-looking forward substitution: at step l
// every row i > l adds A_il T_lj, so each entry sums its terms in increasing l),
//   T_10 = D_1 A_10 D_0,  T_32 = D_3 A_32 D_2,  T_ba = T_b A_ba T_a
// where a, b are the 32 x 32 halves (T_a = [D_0 0; T_10 D_1], T_b likewise).  Every entry is
// band-masked as it is written (N >= 0 keeps i - j <= N; N < 0 keeps all): the band of each
// product depends only on the bands of its factors (Lemma 3.1, Metodologia 1), so the band
// entries are those of the exact path, bit for bit, and N >= n - 1 runs exactly the exact
// path's instructions.  Rows of L past the chunk must be zero (their T rows come out unit
// rows), and the 16 x 16 blocks of Tm above the diagonal must hold zero on entry (they are
// never written).  Zs is 32 x 36 scratch.  Threads 0..255 do the work; in a larger workgroup
// the others pass active = false and only take part in the barriers.  Starts reading L
// without a barrier (the caller publishes it) and ends with a workgroup barrier.
template <int LDL, int LDT>
__device__ __forceinline__ void inverse_blocks(const float (*LP)[LDL], float (*Tm)[LDT], float (*Zs)[36], int N,
                                               int tid, bool active = true) {
  auto keep = [&](int i, int j) { return N < 0 || i - j <= N; };
  const int lane = tid & 63, w = tid >> 6;
  if (active) {   // diagonal block w: lane = (block row ii, block columns jq .. jq + 3)
    const int ii = lane >> 2, jq = (lane & 3) * 4;
    const int o = 16 * w, gi = o + ii;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (ii == 0) *reinterpret_cast<float4 *>(&Tm[o][o + jq]) = make_float4(jq == 0 ? 1.f : 0.f, 0.f, 0.f, 0.f);
    // rows of the block are published and read by lanes of this wave only
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int l = 0; l < 15; ++l) {
      const float A_il = l < ii ? -LP[gi][o + l] : 0.f;
      const float4 t = ld4(&Tm[o + l][o + jq]);
      acc[0] = fmaf(A_il, t.x, acc[0]);
      acc[1] = fmaf(A_il, t.y, acc[1]);
      acc[2] = fmaf(A_il, t.z, acc[2]);
      acc[3] = fmaf(A_il, t.w, acc[3]);
      if (ii == l + 1) {
        float r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int jj = jq + u;
          r[u] = jj == ii ? 1.f : (jj < ii && keep(ii, jj)) ? acc[u] : 0.f;
        }
        *reinterpret_cast<float4 *>(&Tm[gi][o + jq]) = make_float4(r[0], r[1], r[2], r[3]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  __syncthreads();
  // two 16 x 16 products at once: thread = (product p, row r, columns c, c + 1)
  const int p = tid >> 7, r = (tid >> 3) & 15, c = (tid & 7) * 2;
  if (active) {   // Z_p = A_(2p+1, 2p) D_2p
    const int ro = 32 * p + 16, co = 32 * p;
    float z0 = 0.f, z1 = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const float av = -LP[ro + r][co + m];
      const float2 d = ld2(&Tm[co + m][co + c]);
      z0 = fmaf(av, d.x, z0);
      z1 = fmaf(av, d.y, z1);
    }
    *reinterpret_cast<float2 *>(&Zs[16 * p + r][c]) = make_float2(z0, z1);
  }
  __syncthreads();
  if (active) {   // T_(2p+1, 2p) = D_(2p+1) Z_p
    const int ro = 32 * p + 16, co = 32 * p;
    float t0v = 0.f, t1v = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const float dv = Tm[ro + r][ro + m];
      const float2 z = ld2(&Zs[16 * p + m][c]);
      t0v = fmaf(dv, z.x, t0v);
      t1v = fmaf(dv, z.y, t1v);
    }
    const int i = ro + r, j = co + c;
    Tm[i][j] = keep(i, j) ? t0v : 0.f;
    Tm[i][j + 1] = keep(i, j + 1) ? t1v : 0.f;
  }
  __syncthreads();
  // 32 x 32 products: thread = (row r2, columns c4 .. c4 + 3)
  const int r2 = tid >> 3, c4 = (tid & 7) * 4;
  if (active) {   // Z = A_ba T_a
    float z[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int m = 0; m < 32; ++m) {
      const float av = -LP[32 + r2][m];
      const float4 t = ld4(&Tm[m][c4]);
      z[0] = fmaf(av, t.x, z[0]);
      z[1] = fmaf(av, t.y, z[1]);
      z[2] = fmaf(av, t.z, z[2]);
      z[3] = fmaf(av, t.w, z[3]);
    }
    *reinterpret_cast<float4 *>(&Zs[r2][c4]) = make_float4(z[0], z[1], z[2], z[3]);
  }
  __syncthreads();
  if (active) {   // T_ba = T_b Z
    float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int m = 0; m < 32; ++m) {
      const float tb = Tm[32 + r2][32 + m];
      const float4 z = ld4(&Zs[m][c4]);
      t[0] = fmaf(tb, z.x, t[0]);
      t[1] = fmaf(tb, z.y, t[1]);
      t[2] = fmaf(tb, z.z, t[2]);
      t[3] = fmaf(tb, z.w, t[3]);
    }
    const int i = 32 + r2;
    float4 o4;
    o4.x = keep(i, c4) ? t[0] : 0.f;
    o4.y = keep(i, c4 + 1) ? t[1] : 0.f;
    o4.z = keep(i, c4 + 2) ? t[2] : 0.f;
    o4.w = keep(i, c4 + 3) ? t[3] : 0.f;
    *reinterpret_cast<float4 *>(&Tm[i][c4]) = o4;
  }
  __syncthreads();
}

}  // namespace tri
}  // namespace gdr
