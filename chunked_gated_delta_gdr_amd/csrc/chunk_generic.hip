// Generic chunk-parallel gated delta-rule forward: fp32 arithmetic on the vector ALUs.
//
// This is the fp32 path (and the fallback for shapes the matrix-core kernel does not
// cover).  One workgroup owns one (batch, head, value tile of BV state rows) and walks
// the sequence chunk by chunk; the state tile stays in LDS for the whole sequence.
//
// Per chunk of n <= C tokens (chunk-wise form and T = (I - A)^-1 of the MatMul-only
// inversion summary, "Declaracao do Problema"):
//   g      inclusive cumulative sum of log alpha inside the chunk
//   L_ij   = exp(g_i - g_j) (e_i . r_j)              for j < i   (A = -L)
//   X      = V' - (e^g (.) E) S^T                      (value tile only)
//   T      = (I - A)^-1: forward substitution inside the four 16 x 16 diagonal blocks, then
//            the off-diagonal blocks as block products.  With a band limit N only entries
//            with i - j <= N are kept (they use only band entries of the factors: Lemma 3.1
//            of the same summary, Metodologia 1-2), so N >= n - 1 runs exactly the same
//            instructions as the exact path.
//            Optionally (S > 0, band start N) the parallel residual correction of the
//            same summary, Metodologia 3: T = T0 sum_{s<=S} E^s, E = I - (I - A) T0.
//   D      = T X                                     (= U - W S^T of the WY form)
//   P_ij   = exp(g_i - g_j) (q_i . r_j)              for j <= i
//   O      = scale ((e^g (.) Q) S^T + P D)
//   S      <- e^{g_n} S + D^T (e^{g_n - g} (.) R)
#include "common.h"
#include "tri_blocks.h"

namespace gdr {
namespace {

constexpr int kThreads = 256;
constexpr int kBV = 16;     // state rows per workgroup
constexpr int kCMax = 64;   // largest chunk
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float2 ld2(const float *p) { return *reinterpret_cast<const float2 *>(p); }
__device__ __forceinline__ void fma4(float &acc, const float4 &x, const float4 &y) {
  acc = fmaf(x.x, y.x, acc);
  acc = fmaf(x.y, y.y, acc);
  acc = fmaf(x.z, y.z, acc);
  acc = fmaf(x.w, y.w, acc);
}

template <typename IO, int DK, bool CHD>
__global__ __launch_bounds__(kThreads) void chunk_generic_kernel(ChunkArgs a) {
  // CHD: one decay per key channel (log_alpha [B, T, H, Dk]).  The pairwise decay of channel
  // c between tokens j <= i is 2^(G_ic - G_jc) with G the in-chunk cumulative log2 decay, so it
  // sits inside the key products: L_ij = sum_c e_ic r_jc 2^(G_ic - G_jc) (P likewise), the
  // state is read through e^G (.) e and e^G (.) q, and the update uses e^{G_C - G} (.) r and
  // S Diag(e^{G_C}).  Every exponent that is kept is <= 0.
  // fp32 row stride of the [token][channel] tiles: 16-byte aligned rows whose starts fall on
  // distinct 16-byte bank groups for 16 consecutive rows (conflict-free 16-byte reads)
  constexpr int LD = DK + 4;
  constexpr int kLoadIt = kCMax * DK / kThreads;   // elements per thread of one staged tile
  const IO *__restrict__ q = static_cast<const IO *>(a.q);
  const IO *__restrict__ k = static_cast<const IO *>(a.k);
  const IO *__restrict__ v = static_cast<const IO *>(a.v);
  const IO *__restrict__ er = static_cast<const IO *>(a.erase);
  const IO *__restrict__ wr = static_cast<const IO *>(a.write);
  const IO *__restrict__ wk = static_cast<const IO *>(a.write_key);
  IO *__restrict__ out = static_cast<IO *>(a.out);

  const int tid = threadIdx.x;
  const int vt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int v0 = vt * kBV;
  const int nv = min(kBV, a.Dv - v0);
  const int Dk = a.Dk, Dv = a.Dv, H = a.H, T = a.T;

  __shared__ __align__(16) float Rs[kCMax][LD];     // write keys r
  __shared__ __align__(16) float Xs[kCMax][LD];     // erase keys e, then queries q
  __shared__ float LP[kCMax][kCMax + 1];            // L (strict lower), then P (lower)
  __shared__ __align__(16) float Tm[kCMax][kCMax + 4];   // T, row-major
  __shared__ __align__(16) float Zs[32][32 + 4];         // block products in flight
  __shared__ __align__(16) float Zb[CHD ? 1 : kCMax][kCMax + 4];   // residual-correction series
  __shared__ __align__(16) float Gs[CHD ? kCMax : 1][CHD ? LD : 4];  // cumulative log2 decays
  __shared__ __align__(16) float Ss[kBV][LD];       // state tile
  __shared__ __align__(16) float Xv[kCMax][kBV];    // X
  __shared__ __align__(16) float Dl[kCMax][kBV];    // D
  __shared__ float gs[kCMax], eg[kCMax], wd[kCMax];

  const long long sh = static_cast<long long>(b) * H + h;  // (b, h) index
  for (int idx = tid; idx < kBV * LD; idx += kThreads) {
    const int r = idx / LD, c = idx % LD;
    float s = 0.f;
    if (a.state_in != nullptr && r < nv && c < Dk) s = a.state_in[(sh * Dv + v0 + r) * Dk + c];
    Ss[r][c] = s;
  }
  // the 16 x 16 blocks of T above the diagonal are never written: zero once
  for (int idx = tid; idx < kCMax * kCMax; idx += kThreads) {
    const int i = idx / kCMax, j = idx % kCMax;
    if ((j >> 4) > (i >> 4)) Tm[i][j] = 0.f;
  }
  float hreg = 0.f;  // preconditioner accumulator of channel `tid`
  if (a.wkey == GDR_WKEY_DIAG_PRECOND && tid < Dk)
    hreg = a.pc_h_in != nullptr ? a.pc_h_in[sh * Dk + tid] : a.h0;

  // thread tiles: 4 x 4 blocks of the C x C products, 2 x 2 blocks of the C x kBV ones
  const int bi = tid >> 4, bj = tid & 15;      // rows 4 bi.., columns 4 bj..
  const int t0 = 2 * (tid >> 3), r0 = 2 * (tid & 7);

  for (int c0 = 0; c0 < T; c0 += a.C) {
    const int n = min(a.C, T - c0);
    // token (b, c0 + t, h) row index in [B, T, H]
    auto tok = [&](int t) -> long long { return (static_cast<long long>(b) * T + c0 + t) * H + h; };
    // Element (t, c) of a [B, T, H, Dk] tensor sits t * H * Dk + c after the chunk's first
    // token row (a 32-bit offset: 64 H Dk < 2^31).  stage() copies rows 0..n-1 of such a tile
    // into dst (zero beyond n and Dk).  Every load reads a valid element (indices clamped into
    // the tile) and the mask is applied afterwards, so the loads carry no branch and all of a
    // tile's loads are in flight together.
    const long long row0 = tok(0);
    const int rstride = H * Dk;
    auto stage = [&](float(*dst)[LD], auto &&load) {
      float x[kLoadIt];
#pragma unroll
      for (int it = 0; it < kLoadIt; ++it) {
        const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
        const int tc = min(t, n - 1), cc = min(c, Dk - 1);
        x[it] = load(tc, tc * rstride + cc);
      }
#pragma unroll
      for (int it = 0; it < kLoadIt; ++it) {
        const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
        if (!(t < n && c < Dk)) x[it] = 0.f;
      }
#pragma unroll
      for (int it = 0; it < kLoadIt; ++it) {
        const int idx = tid + it * kThreads;
        dst[idx / DK][idx % DK] = x[it];
      }
    };
    // LP[i][j] = exp(g_i - g_j) (Xs_i . Rs_j) for j < i (or j <= i), zero above; rows past n
    // hold zero keys, so they come out zero
    auto gram = [&](bool incl_diag) {
      if (bj > bi) return;
      float acc[4][4] = {};
      if constexpr (CHD) {
#pragma unroll 2
        for (int c = 0; c < DK; c += 4) {
          float4 x[4], r[4], gi[4], gj[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            x[u] = ld4(&Xs[4 * bi + u][c]);
            r[u] = ld4(&Rs[4 * bj + u][c]);
            gi[u] = ld4(&Gs[4 * bi + u][c]);
            gj[u] = ld4(&Gs[4 * bj + u][c]);
          }
          // (entries above the diagonal may overflow here; they are discarded below)
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const float4 d = make_float4(x[u].x * exp2f(gi[u].x - gj[w].x), x[u].y * exp2f(gi[u].y - gj[w].y),
                                           x[u].z * exp2f(gi[u].z - gj[w].z), x[u].w * exp2f(gi[u].w - gj[w].w));
              fma4(acc[u][w], d, r[w]);
            }
        }
      } else {
#pragma unroll 4
        for (int c = 0; c < DK; c += 4) {
          float4 x[4], r[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            x[u] = ld4(&Xs[4 * bi + u][c]);
            r[u] = ld4(&Rs[4 * bj + u][c]);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int w = 0; w < 4; ++w) fma4(acc[u][w], x[u], r[w]);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int i = 4 * bi + u, j = 4 * bj + w;
          const float dec = CHD ? 1.f : expf(gs[i] - gs[j]);
          LP[i][j] = (j < i || (incl_diag && j == i)) ? dec * acc[u][w] : 0.f;
        }
    };
    // (Xs_t . Ss_r) for the thread's 2 x 2 block of tokens t0.. and state rows r0..
    // (with per-channel decays: the rows are read as 2^G (.) x)
    auto dot_state = [&](float (&acc)[2][2]) {
#pragma unroll 4
      for (int c = 0; c < DK; c += 4) {
        float4 x0 = ld4(&Xs[t0][c]), x1 = ld4(&Xs[t0 + 1][c]);
        if constexpr (CHD) {
          const float4 g0 = ld4(&Gs[t0][c]), g1 = ld4(&Gs[t0 + 1][c]);
          x0 = make_float4(x0.x * exp2f(g0.x), x0.y * exp2f(g0.y), x0.z * exp2f(g0.z), x0.w * exp2f(g0.w));
          x1 = make_float4(x1.x * exp2f(g1.x), x1.y * exp2f(g1.y), x1.z * exp2f(g1.z), x1.w * exp2f(g1.w));
        }
        const float4 s0 = ld4(&Ss[r0][c]), s1 = ld4(&Ss[r0 + 1][c]);
        fma4(acc[0][0], x0, s0);
        fma4(acc[0][1], x0, s1);
        fma4(acc[1][0], x1, s0);
        fma4(acc[1][1], x1, s1);
      }
    };

    __syncthreads();  // previous chunk done with every buffer
    // write keys (the preconditioned ones are formed from the staged keys below)
    const IO *kc = k + row0 * Dk;
    {
      const IO *src = ((a.wkey == GDR_WKEY_EXPLICIT) ? wk : k) + row0 * Dk;
      stage(Rs, [&](int, int o) { return ld_f(src, o); });
    }
    // erase keys
    if (a.gain == GDR_GAIN_SCALAR) {
      const float *bc = a.beta + row0;
      stage(Xs, [&](int t, int o) { return bc[t * H] * ld_f(kc, o); });
    } else {
      const IO *ec = er + row0 * Dk;
      stage(Xs, [&](int, int o) { return ld_f(ec, o) * ld_f(kc, o); });
    }
    if constexpr (CHD) {
      // per-channel decays: stage, then each channel's inclusive cumulative sum in log2 units
      // (rows past n are zero, so the sums stay flat there)
      const float *lac = a.log_alpha + row0 * Dk;
      stage(Gs, [&](int, int o) { return lac[o]; });
      __syncthreads();
      if (tid < DK) {
        float gv[kCMax];
#pragma unroll
        for (int t = 0; t < kCMax; ++t) gv[t] = Gs[t][tid];
        float g = 0.f;
#pragma unroll
        for (int t = 0; t < kCMax; ++t) {
          g = fmaf(gv[t], kLog2e, g);
          Gs[t][tid] = g;
        }
      }
    }
    // gates: inclusive cumulative sum of log alpha over the chunk (one wave)
    if (tid < kCMax) {
      float g = (a.decay == GDR_DECAY_SCALAR && tid < n) ? a.log_alpha[tok(tid)] : 0.f;
#pragma unroll
      for (int d = 1; d < kCMax; d <<= 1) {
        const float y = __shfl_up(g, d, kCMax);
        if (tid >= d) g += y;
      }
      const float glast = __shfl(g, n - 1, kCMax);
      gs[tid] = g;
      eg[tid] = expf(g);
      wd[tid] = expf(glast - g);
    }
    if (a.wkey == GDR_WKEY_DIAG_PRECOND) {
      // u = k / (h / (1 - rho^t) + eps), h_t = rho h_{t-1} + k_t^2.  The bias corrections of the
      // chunk's tokens first (one thread each), then channel `tid` walks the chunk: its keys
      // are read up front, so only the accumulator chain is serial.
      float *icorr = &Zs[0][0];   // (free until the inverse is built)
      if (tid < kCMax) {
        const float tg = static_cast<float>(a.t0 + c0 + tid + 1);
        icorr[tid] = 1.f / -expm1f(tg * a.log_rho);   // 1 / (1 - rho^t)
      }
      __syncthreads();
      if (tid < Dk) {
        // rows past n hold zero keys (their u comes out zero); the accumulator skips them
        float kv[kCMax];
#pragma unroll
        for (int t = 0; t < kCMax; ++t) kv[t] = Rs[t][tid];
#pragma unroll
        for (int t = 0; t < kCMax; ++t) {
          const float hn = fmaf(a.rho, hreg, kv[t] * kv[t]);
          hreg = t < n ? hn : hreg;
          Rs[t][tid] = kv[t] / fmaf(hreg, icorr[t], a.eps);
        }
      }
    }
    __syncthreads();
    // L (strict lower)
    gram(false);
    // X = V' - (e^g (.) E) S^T on the value tile
    {
      float vp[2][2];   // (loads from clamped indices; entries outside the tile are masked below)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const int t = min(t0 + u, n - 1), r = min(r0 + w, nv - 1);
          const long long vi = tok(t) * Dv + v0 + r;
          const float vv = ld_f(v, vi);
          vp[u][w] = (a.gain == GDR_GAIN_SCALAR) ? a.beta[tok(t)] * vv : ld_f(wr, vi) * vv;
        }
      float acc[2][2] = {};
      dot_state(acc);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const int t = t0 + u, r = r0 + w;
          Xv[t][r] = (t < n && r < nv) ? vp[u][w] - eg[t] * acc[u][w] : 0.f;
        }
    }
    __syncthreads();
    // T = (I - A)^-1 by 16 x 16 blocks (exact, or its band i - j <= N)
    tri::inverse_blocks(LP, Tm, Zs, a.N, tid);
    // Parallel residual correction of the band start T0 (MatMul-only inversion summary,
    // Metodologia 3): E = I - (I - A) T0, Z = I + E (I + E (... (I + E))) with S factors
    // (= sum_{s<=S} E^s), T = T0 Z.  E and Z are strictly lower / unit lower triangular, so
    // each product sums over l < i (l <= i for T0 Z).  Thread: row i, columns jg .. jg + 15;
    // every product is formed in registers and written back after a barrier (E over L, Z
    // in place, T over T0).
    if (CHD ? false : a.S > 0) {
      const int i = tid >> 2, jg = (tid & 3) * 16;
      // the rows of wave w are 16 w .. 16 w + 15, so every sum below ends before l = 16 (w + 1):
      // a wave-uniform bound; the coefficients past the row's own bound are masked to zero
      const int lwave = 16 * ((tid >> 6) + 1);
      float acc[16];
      // acc = sum_{l < lend} (+-Lm[i][l]) Tr[l][jg ..], four rows of Tr per batch of reads
      auto row_product = [&](const auto *Lm, const float(*Tr)[kCMax + 4], int lend, bool neg) {
#pragma unroll
        for (int u = 0; u < 16; ++u) acc[u] = 0.f;
        for (int l0 = 0; l0 < lwave; l0 += 4) {
          float x[4];
          float4 t[4][4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float m = Lm[i][l0 + q];
            x[q] = l0 + q < lend ? (neg ? -m : m) : 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u) t[q][u] = ld4(&Tr[l0 + q][jg + 4 * u]);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              acc[4 * u] = fmaf(x[q], t[q][u].x, acc[4 * u]);
              acc[4 * u + 1] = fmaf(x[q], t[q][u].y, acc[4 * u + 1]);
              acc[4 * u + 2] = fmaf(x[q], t[q][u].z, acc[4 * u + 2]);
              acc[4 * u + 3] = fmaf(x[q], t[q][u].w, acc[4 * u + 3]);
            }
        }
      };
      // E_ij = delta_ij - T0_ij + (A T0)_ij, A = -L
      row_product(LP, Tm, i, true);
      float e[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) e[u] = ((jg + u == i) ? 1.f : 0.f) - Tm[i][jg + u] + acc[u];
      __syncthreads();   // every row of A has been read
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        LP[i][jg + u] = e[u];
        Zb[i][jg + u] = (jg + u == i) ? 1.f : 0.f;
      }
      __syncthreads();
      for (int st = 0; st < a.S; ++st) {   // Z <- I + E Z
        row_product(LP, Zb, i, false);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 16; ++u) Zb[i][jg + u] = ((jg + u == i) ? 1.f : 0.f) + acc[u];
        __syncthreads();
      }
      // T = T0 Z (T0 is lower triangular: l <= i)
      row_product(Tm, Zb, i + 1, false);
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 16; u += 4)
        *reinterpret_cast<float4 *>(&Tm[i][jg + u]) = make_float4(acc[u], acc[u + 1], acc[u + 2], acc[u + 3]);
      __syncthreads();
    }
    // queries replace the erase keys (last read before the barrier above)
    {
      const IO *qc = q + row0 * Dk;
      stage(Xs, [&](int, int o) { return ld_f(qc, o); });
    }
    __syncthreads();
    // D = T X: acc = X_tr; for s < t: acc += T_ts X_sr
    {
      float acc[2][2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float2 x = ld2(&Xv[t0 + u][r0]);
        acc[u][0] = x.x;
        acc[u][1] = x.y;
      }
      for (int s = 0; s < t0; ++s) {
        const float2 x = ld2(&Xv[s][r0]);
        const float a0 = Tm[t0][s], a1 = Tm[t0 + 1][s];
        acc[0][0] = fmaf(a0, x.x, acc[0][0]);
        acc[0][1] = fmaf(a0, x.y, acc[0][1]);
        acc[1][0] = fmaf(a1, x.x, acc[1][0]);
        acc[1][1] = fmaf(a1, x.y, acc[1][1]);
      }
      {   // s = t0 for the second row
        const float2 x = ld2(&Xv[t0][r0]);
        const float a1 = Tm[t0 + 1][t0];
        acc[1][0] = fmaf(a1, x.x, acc[1][0]);
        acc[1][1] = fmaf(a1, x.y, acc[1][1]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) *reinterpret_cast<float2 *>(&Dl[t0 + u][r0]) = make_float2(acc[u][0], acc[u][1]);
    }
    // P (lower incl. diagonal; L is no longer needed)
    gram(true);
    __syncthreads();
    // O = scale ((e^g (.) Q) S^T + P D)
    {
      float acc[2][2] = {};
      dot_state(acc);
      if constexpr (!CHD) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          acc[u][0] *= eg[t0 + u];
          acc[u][1] *= eg[t0 + u];
        }
      }
      for (int j = 0; j <= t0; ++j) {
        const float2 d = ld2(&Dl[j][r0]);
        const float p0 = LP[t0][j], p1 = LP[t0 + 1][j];
        acc[0][0] = fmaf(p0, d.x, acc[0][0]);
        acc[0][1] = fmaf(p0, d.y, acc[0][1]);
        acc[1][0] = fmaf(p1, d.x, acc[1][0]);
        acc[1][1] = fmaf(p1, d.y, acc[1][1]);
      }
      {   // j = t0 + 1 for the second row
        const float2 d = ld2(&Dl[t0 + 1][r0]);
        const float p1 = LP[t0 + 1][t0 + 1];
        acc[1][0] = fmaf(p1, d.x, acc[1][0]);
        acc[1][1] = fmaf(p1, d.y, acc[1][1]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const int t = t0 + u, r = r0 + w;
          if (t < n && r < nv) st_f(out, tok(t) * Dv + v0 + r, a.scale * acc[u][w]);
        }
    }
    if constexpr (CHD) {   // R <- 2^(G_C - G) (.) R for the update (P, its last other use, is done)
#pragma unroll
      for (int it = 0; it < kLoadIt; ++it) {
        const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
        Rs[t][c] *= exp2f(Gs[n - 1][c] - Gs[t][c]);
      }
    }
    __syncthreads();
    // S <- e^{g_n} S + D^T (e^{g_n - g} (.) R): thread (row r, columns c..c+3); rows past nv
    // and columns past Dk stay zero (their D rows and key columns are zero).  Per-channel
    // decays: S Diag(2^{G_C}) + D^T R with R already scaled.
    {
      const float gl = eg[n - 1];
      constexpr int NC4 = DK / 4;
#pragma unroll
      for (int u0 = 0; u0 < kBV * NC4; u0 += kThreads) {
        const int u = u0 + tid;
        if (kBV * NC4 % kThreads != 0 && u >= kBV * NC4) break;
        const int r = u / NC4, c = (u % NC4) * 4;
        const float4 s = ld4(&Ss[r][c]);
        float4 acc = make_float4(gl * s.x, gl * s.y, gl * s.z, gl * s.w);
        if constexpr (CHD) {
          const float4 gc = ld4(&Gs[n - 1][c]);
          acc = make_float4(exp2f(gc.x) * s.x, exp2f(gc.y) * s.y, exp2f(gc.z) * s.z, exp2f(gc.w) * s.w);
        }
        for (int j = 0; j < n; ++j) {
          const float w = Dl[j][r] * wd[j];
          const float4 rr = ld4(&Rs[j][c]);
          acc.x = fmaf(w, rr.x, acc.x);
          acc.y = fmaf(w, rr.y, acc.y);
          acc.z = fmaf(w, rr.z, acc.z);
          acc.w = fmaf(w, rr.w, acc.w);
        }
        *reinterpret_cast<float4 *>(&Ss[r][c]) = acc;
      }
    }
  }
  __syncthreads();
  if (a.state_out != nullptr) {
    for (int idx = tid; idx < kBV * DK; idx += kThreads) {
      const int r = idx / DK, c = idx % DK;
      if (r < nv && c < Dk) a.state_out[(sh * Dv + v0 + r) * Dk + c] = Ss[r][c];
    }
  }
  if (a.wkey == GDR_WKEY_DIAG_PRECOND && a.pc_h_out != nullptr && vt == 0 && tid < Dk)
    a.pc_h_out[sh * Dk + tid] = hreg;
}

template <typename IO, bool CHD>
hipError_t launch_dk(const ChunkArgs &a, hipStream_t s) {
  const dim3 grid((a.Dv + kBV - 1) / kBV, a.H, a.B);
  if (a.Dk <= 32)
    hipLaunchKernelGGL((chunk_generic_kernel<IO, 32, CHD>), grid, dim3(kThreads), 0, s, a);
  else if (a.Dk <= 64)
    hipLaunchKernelGGL((chunk_generic_kernel<IO, 64, CHD>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((chunk_generic_kernel<IO, 128, CHD>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <typename IO>
hipError_t launch_io(const ChunkArgs &a, hipStream_t s) {
  return a.decay == GDR_DECAY_CHANNEL ? launch_dk<IO, true>(a, s) : launch_dk<IO, false>(a, s);
}

}  // namespace

hipError_t launch_chunk_generic(const ChunkArgs &a, int io_dtype, hipStream_t s) {
  return io_dtype == GDR_BF16 ? launch_io<uint16_t>(a, s) : launch_io<float>(a, s);
}

}  // namespace gdr
