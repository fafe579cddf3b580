// Gram tiles of one chunk under per-channel (diagonal) decay, shared by the forward and
// backward kernels (fp32; the matrix cores for the tiles below the diagonal).
#pragma once

#include "common.h"

namespace gdr {
namespace chd {

typedef float f4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4v mma(float a, float b, f4v c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }

// 2^x by one v_exp_f32: for the decay factors, whose exponents are <= 0 (or discarded), a
// result below 2^-126 is flushed where exp2f would go on into denormals (then both are
// negligible against the O(1) terms they are summed with); exp2f's range handling costs five
// more instructions per call, and these factors are most of the per-channel decay's work
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ void fma4(float &acc, const float4 &x, const float4 &y) {
  acc = fmaf(x.x, y.x, acc);
  acc = fmaf(x.y, y.y, acc);
  acc = fmaf(x.z, y.z, acc);
  acc = fmaf(x.w, y.w, acc);
}

// LP[i][j] = sum_c X_ic R_jc 2^(G_ic - G_jc) for j < i (j <= i with incl_diag) on the ten
// 16 x 16 tiles on and below the diagonal of a 64-token chunk (the per-channel decay between
// tokens j <= i of the Kimi Delta Attention recurrence, inside the key products); the entries
// of the diagonal tiles above the diagonal are zero, the tiles above are not written.  X, R
// and G (the in-chunk cumulative log2 decay, non-increasing along the chunk, constant past
// its last token) are [64][LD] fp32 rows in LDS, DK channels (zero keys past the chunk and
// past the head dimension).  Every exponent that is evaluated for a kept entry is <= 0:
//  * the six tiles below the diagonal (row block ib > column block jb) go to the matrix
//    cores with the decay split at the last row of block jb, ref = 16 jb + 15, as
//    2^(G_ic - G_ref,c) 2^(G_ref,c - G_jc), each factor in its operand;
//  * the four diagonal tiles stay on the vector ALUs in 4 x 4 sub-blocks: those below the
//    sub-block diagonal split the same way at the last row of their column sub-block (one
//    exponential per operand row and channel), the diagonal sub-blocks take one exponential
//    per pair below their diagonal and none on it.
// Waves 0..3 take matrix tiles wave and wave + 4 and the diagonal sub-blocks of diagonal
// tile `wave`; waves 4..7 the lower sub-blocks of diagonal tile wave - 4 (one wave of each
// kind per SIMD).  512 threads; no barrier inside (the caller publishes X, R, G before and
// LP after).
template <int DK, int LD, int LDP>
__device__ __forceinline__ void gram(const float (*Xs)[LD], const float (*Rs)[LD], const float (*Gs)[LD],
                                     float (*LP)[LDP], bool incl_diag, int tid) {
  const int wave = tid >> 6, lane = tid & 63, col = lane & 15, kq = lane >> 4;
  if (wave < 4) {
    for (int u = wave; u < 6; u += 4) {
      const int ib = u < 1 ? 1 : u < 3 ? 2 : 3, jb = u - (ib - 1) * ib / 2;
      const int ref = 16 * jb + 15, i = 16 * ib + col, j = 16 * jb + col;
      // (K order permuted: sub-step u of block s takes k = s + 4 kq + u, so each lane reads 4
      // consecutive channels with one 16-byte read per operand)
      f4v ap[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll 2
      for (int ks = 0; ks < DK; ks += 16) {
        const int kk = ks + 4 * kq;
        const float4 x = ld4(&Xs[i][kk]), gx = ld4(&Gs[i][kk]), gr = ld4(&Gs[ref][kk]);
        const float4 r = ld4(&Rs[j][kk]), gy = ld4(&Gs[j][kk]);
        ap[0] = mma(x.x * ex2(gx.x - gr.x), r.x * ex2(gr.x - gy.x), ap[0]);
        ap[1] = mma(x.y * ex2(gx.y - gr.y), r.y * ex2(gr.y - gy.y), ap[1]);
        ap[0] = mma(x.z * ex2(gx.z - gr.z), r.z * ex2(gr.z - gy.z), ap[0]);
        ap[1] = mma(x.w * ex2(gx.w - gr.w), r.w * ex2(gr.w - gy.w), ap[1]);
      }
      const f4v acc = ap[0] + ap[1];
#pragma unroll
      for (int r = 0; r < 4; ++r) LP[16 * ib + 4 * kq + r][j] = acc[r];
    }
    // diagonal sub-block lane >> 4 of tile `wave`, 8 channels per lane over 16 adjacent lanes
    // (summed by shuffles)
    const int g = lane & 15, i0 = 16 * wave + 4 * (lane >> 4), c0g = 8 * g;
    float acc[4][4] = {};
    if (c0g < DK) {
#pragma unroll
      for (int cc = 0; cc < 8; cc += 4) {
        const int c = c0g + cc;
        float4 x[4], gi[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          x[u] = ld4(&Xs[i0 + u][c]);
          gi[u] = ld4(&Gs[i0 + u][c]);
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float4 r = ld4(&Rs[i0 + w][c]), gj = ld4(&Gs[i0 + w][c]);
#pragma unroll
          for (int u = w; u < 4; ++u) {
            if (u == w) {
              fma4(acc[u][w], x[u], r);
            } else {
              const float4 dd = make_float4(x[u].x * ex2(gi[u].x - gj.x), x[u].y * ex2(gi[u].y - gj.y),
                                            x[u].z * ex2(gi[u].z - gj.z), x[u].w * ex2(gi[u].w - gj.w));
              fma4(acc[u][w], dd, r);
            }
          }
        }
      }
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w <= u; ++w) acc[u][w] += __shfl_xor(acc[u][w], m);
    if (g == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          LP[i0 + u][i0 + w] = (w < u || (incl_diag && w == u)) ? acc[u][w] : 0.f;
    }
  } else {
    // sub-block sb = lane >> 3 (< 6: row sub-block bi > column sub-block bj) of diagonal tile
    // d, 16 channels per lane over 8 adjacent lanes
    const int d = wave - 4, g = lane & 7, sb = lane >> 3;
    const int bi = sb < 1 ? 1 : sb < 3 ? 2 : 3, bj = min(sb - (bi - 1) * bi / 2, bi - 1);
    const int i0 = 16 * d + 4 * bi, j0 = 16 * d + 4 * bj, ref = j0 + 3, c0g = 16 * g;
    float acc[4][4] = {};
    if (sb < 6 && c0g < DK) {
#pragma unroll 1
      for (int cc = 0; cc < 16; cc += 4) {
        const int c = c0g + cc;
        const float4 gr = ld4(&Gs[ref][c]);
        float4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 xv = ld4(&Xs[i0 + u][c]), gv = ld4(&Gs[i0 + u][c]);
          x[u] = make_float4(xv.x * ex2(gv.x - gr.x), xv.y * ex2(gv.y - gr.y), xv.z * ex2(gv.z - gr.z),
                             xv.w * ex2(gv.w - gr.w));
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float4 rv = ld4(&Rs[j0 + w][c]), gv = ld4(&Gs[j0 + w][c]);
          const float4 r = make_float4(rv.x * ex2(gr.x - gv.x), rv.y * ex2(gr.y - gv.y), rv.z * ex2(gr.z - gv.z),
                                       rv.w * ex2(gr.w - gv.w));
#pragma unroll
          for (int u = 0; u < 4; ++u) fma4(acc[u][w], x[u], r);
        }
      }
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[u][w] += __shfl_xor(acc[u][w], m);
    if (g == 0 && sb < 6) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) LP[i0 + u][j0 + w] = acc[u][w];   // all below the diagonal
    }
  }
  // the six 4 x 4 blocks above the sub-block diagonal of each diagonal tile hold zeros (the
  // products with P read whole diagonal tiles): one entry per thread
  if (tid < 4 * 6 * 16) {
    const int dt = tid / 96, ub = (tid % 96) / 16, en = tid % 16;
    const int ubi = ub < 3 ? 0 : ub < 5 ? 1 : 2;
    const int ubj = ub < 3 ? ub + 1 : ub < 5 ? ub - 1 : 3;
    LP[16 * dt + 4 * ubi + (en >> 2)][16 * dt + 4 * ubj + (en & 3)] = 0.f;
  }
}

}  // namespace chd
}  // namespace gdr
