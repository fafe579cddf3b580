// Generic chunk-parallel gated delta-rule forward: fp32 arithmetic, products on the fp32
// matrix cores.
//
// This is the fp32 path (and the kernel for every shape and option the bf16 matrix-core
// kernel does not cover).  One workgroup of 8 waves owns one (batch, head, value tile of BV
// state rows) and walks the sequence chunk by chunk; the state tile lives in the waves' MFMA
// accumulators for the whole sequence (16 x 16 tiles), mirrored in LDS for the products that
// read it as an operand.
//
// Per chunk of n <= C tokens (chunk-wise form and T = (I - A)^-1 of the MatMul-only inversion
// summary, "Declaracao do Problema"):
//   g      inclusive cumulative sum of log alpha inside the chunk
//   L_ij   = exp(g_i - g_j) (e_i . r_j)              for j < i   (A = -L)
//   X      = V' - (e^g (.) E) S^T                      (value tile only)
//   T      = (I - A)^-1: forward substitution inside the four 16 x 16 diagonal blocks, then
//            the off-diagonal blocks as block products (tri_blocks.h).  With a band limit N
//            only entries with i - j <= N are kept (they use only band entries of the
//            factors: Lemma 3.1 of the same summary, Metodologia 1-2), so N >= n - 1 runs
//            exactly the same instructions as the exact path.
//            Optionally (S > 0, band start N) the parallel residual correction of the
//            same summary, Metodologia 3: T = T0 sum_{s<=S} E^s, E = I - (I - A) T0.
//   D      = T X                                     (= U - W S^T of the WY form)
//   P_ij   = exp(g_i - g_j) (q_i . r_j)              for j <= i
//   O      = scale ((e^g (.) Q) S^T + P D)
//   S      <- e^{g_n} S + D^T (e^{g_n - g} (.) R)
// Products: v_mfma_f32_16x16x4_f32 (fp32 operands and accumulation; lane l gives A[l % 16]
// [l / 16] and B[l / 16][l % 16] and holds D[4 (l / 16) + r][l % 16], r < 4).  The tiles of
// X, D and O are spread one per wave; the ten C x C tiles on and below the diagonal two per
// wave at most.
//
// Chunk 128 with a band-limited T (N <= 15; the C128 variant): the chunk runs as its two
// 64-row halves a and b in turn, each with the steps above and its own in-chunk cumulative
// decay.  In block form T = [[T_aa, 0], [T_ba, T_bb]], and the band of T_ba is
// band(T_bb A_ba T_aa) (every term of an in-band entry uses in-band factors, Lemma 3.1), which
// for N <= 15 touches only rows 64..79 and columns 48..63.  The chunk's D_b is
// T_bb X_b + T_ba X_a with X_b read from the chunk's start state S_c; the output and the state
// update of half b, read from the state after half a, equal the chunk-128 ones, since
// e^{g} Q_b S_c^T + P_ba D_a = e^{g'} Q_b S_mid^T for any D_a (g' the cumulative decay from the
// start of half b).  So half a also keeps S_c, rows 48..63 of its write keys, X and T_aa and
// its last decays, and half b adds the corner (64 + i, 48 + j), kept where i - j + 16 <= N,
// to the first 16 rows of its D.
#include <cstdlib>

#include "common.h"
#include "tri_blocks.h"
#include "chd_gram.h"

namespace gdr {
namespace {

constexpr int kThreads = 512;   // 8 waves
constexpr int kCMax = 64;       // largest chunk
constexpr float kLog2e = 1.4426950408889634f;

typedef float float4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4v mfma4(float a, float b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ void fma4(float &acc, const float4 &x, const float4 &y) {
  acc = fmaf(x.x, y.x, acc);
  acc = fmaf(x.y, y.y, acc);
  acc = fmaf(x.z, y.z, acc);
  acc = fmaf(x.w, y.w, acc);
}

// sum over k < K of A[i][k] B[k][j] for the lane's row i (row pointer ra) and column j (row
// pointer rb of B^T), both with k contiguous in LDS: the K order is permuted so that sub-step
// u of block s takes k = s + 4 kq + u, and each lane reads its 4 k with one 16-byte read per
// operand; two independent accumulator chains
template <int K>
__device__ __forceinline__ float4v dot_kc(const float *ra, const float *rb, int kq) {
  float4v a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < K; s += 16) {
    const float4 x = ld4(ra + s + 4 * kq), y = ld4(rb + s + 4 * kq);
    a0 = mfma4(x.x, y.x, a0);
    a1 = mfma4(x.y, y.y, a1);
    a0 = mfma4(x.z, y.z, a0);
    a1 = mfma4(x.w, y.w, a1);
  }
  return a0 + a1;
}

// tile u (0..9) of the ten 16 x 16 tiles on and below the diagonal of a 64 x 64 matrix
__device__ __forceinline__ void lower_tile(int u, int &ib, int &jb) {
  ib = u < 1 ? 0 : u < 3 ? 1 : u < 6 ? 2 : 3;
  jb = u - ib * (ib + 1) / 2;
}

template <typename IO, int DK, bool CHD, int BV, bool C128>
__global__ __launch_bounds__(kThreads) void chunk_generic_kernel(ChunkArgs a) {
  static_assert(!C128 || (!CHD && BV == 16), "chunk 128 runs with scalar or no decay on 16-row value tiles");
  // CHD: one decay per key channel (log_alpha [B, T, H, Dk]).  The pairwise decay of channel
  // c between tokens j <= i is 2^(G_ic - G_jc) with G the in-chunk cumulative log2 decay, so it
  // sits inside the key products: L_ij = sum_c e_ic r_jc 2^(G_ic - G_jc) (P likewise; factored
  // into the operands below the diagonal tiles, per pair on them), the state is read through
  // 2^G (.) e and 2^G (.) q, and the update uses
  // 2^(G_C - G) (.) r and S Diag(2^G_C).  Every exponent that is kept is <= 0.
  constexpr int LD = DK + 4;            // fp32 row stride of the [token][channel] tiles
  constexpr int kLoadIt = kCMax * DK / kThreads;
  constexpr int NCB = DK / 16;          // channel blocks
  constexpr int NRB = BV / 16;          // value-row blocks
  constexpr int NTS = NRB * NCB;        // state tiles
  constexpr int NTW = (NTS + 7) / 8;    // state tiles per wave
  constexpr int NXT = 4 * NRB;          // tiles of the C x BV products X, D, O
  const IO *__restrict__ q = static_cast<const IO *>(a.q);
  const IO *__restrict__ k = static_cast<const IO *>(a.k);
  const IO *__restrict__ v = static_cast<const IO *>(a.v);
  const IO *__restrict__ er = static_cast<const IO *>(a.erase);
  const IO *__restrict__ wr = static_cast<const IO *>(a.write);
  const IO *__restrict__ wk = static_cast<const IO *>(a.write_key);
  IO *__restrict__ out = static_cast<IO *>(a.out);

  const int tid = threadIdx.x;
  // XCD-aware tile order: workgroups are dealt to the 8 XCDs in turn, so consecutive logical
  // tiles (the value tiles of one head, which read the same keys, queries and decays) get ids
  // 8 apart and share an XCD's L2
  // (indices in 64 bits: the grid may hold up to 2^24 workgroups, and the host bounds it)
  const uint64_t nvt = gridDim.x, nh = gridDim.y;
  const uint64_t G = nvt * nh * gridDim.z;
  const uint64_t bid = blockIdx.x + nvt * (blockIdx.y + nh * static_cast<uint64_t>(blockIdx.z));
  const uint64_t logical = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int vt = static_cast<int>(logical % nvt), h = static_cast<int>((logical / nvt) % nh),
            b = static_cast<int>(logical / nvt / nh);
  const int v0 = vt * BV;
  const int nv = min(BV, a.Dv - v0);
  const int Dk = a.Dk, Dv = a.Dv, H = a.H, T = a.T;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 15, kq = lane >> 4;
  const bool xwave = wave < NXT;        // owns the (tb, rb) tile of X, D and O
  const int tb = wave & 3, rb = wave >> 2;

  // With per-channel decays (the cumulative decays take a 64 x Dk tile) LDS is tight: D
  // overwrites X once every read of X is done, the inverse's scratch lives in the erase-key
  // tile (dead between X and the queries) and the preconditioner's bias corrections in Zb.
  constexpr bool kTight = CHD;
  __shared__ __align__(16) float Rs[kCMax][LD];     // write keys r
  __shared__ __align__(16) float Xs[kCMax][LD];     // erase keys e, then queries q
  __shared__ float LP[kCMax][kCMax + 1];            // L (then E of the residual), then P
  __shared__ __align__(16) float Tm[kCMax][kCMax + 4];   // T, row-major
  __shared__ __align__(16) float Zs_[kTight ? 1 : 32][36];            // block products in flight
  __shared__ __align__(16) float Zb[CHD ? 1 : kCMax][kCMax + 4];   // residual-correction series
  __shared__ __align__(16) float Gs[CHD ? kCMax : 1][CHD ? LD : 4];  // cumulative log2 decays
  __shared__ __align__(16) float Ss[BV][LD];        // mirror of the state tile
  __shared__ __align__(16) float Xv[kCMax][BV];     // X
  __shared__ __align__(16) float Dl_[kTight ? 1 : kCMax][BV];   // D
  __shared__ float gs[kCMax], eg[kCMax], wd[kCMax];
  float(*const Zs)[36] = kTight ? reinterpret_cast<float(*)[36]>(&Xs[0][0]) : Zs_;
  float(*const Dl)[BV] = kTight ? Xv : Dl_;
  static_assert(!kTight || 32 * 36 <= kCMax * LD, "the inverse's scratch must fit the key tile");
  // chunk 128: what half a hands to half b.  The start state S_c and write-key rows 48..63 take
  // the residual series' buffer (the residual correction is not offered at chunk 128).
  constexpr int kH = C128 ? 16 : 1;
  __shared__ __align__(16) float Taa[kH][kH + 1];   // T_aa rows / columns 48..63
  __shared__ __align__(16) float Xat[kH][C128 ? BV : 1];   // X_a rows 48..63
  __shared__ float Zc[kH][kH + 1];                  // A_ba T_aa, then the band of T_ba
  __shared__ float wdt[kH], ega[1];                 // e^{g_63 - g_j} (j = 48..63), e^{g_63} of half a
  float(*const Ss2)[LD] = reinterpret_cast<float(*)[LD]>(&Zb[0][0]);
  float(*const Rat)[LD] = reinterpret_cast<float(*)[LD]>(&Zb[0][0] + BV * LD);
  static_assert(!C128 || (BV + 16) * LD <= kCMax * (kCMax + 4), "S_c and the key rows must fit the series buffer");

  const long long sh = static_cast<long long>(b) * H + h;  // (b, h) index
  // state tiles of this wave: tile u = wave + 8 m -> value-row block u / NCB, channel block u % NCB
  float4v Sacc[NTW];
#pragma unroll
  for (int m = 0; m < NTW; ++m) {
    const int u = wave + 8 * m;
    const int row = 16 * (u / NCB) + 4 * kq, c = 16 * (u % NCB) + col;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = 0.f;
      if (u < NTS && a.state_in != nullptr && row + r < nv && c < Dk)
        x = a.state_in[(sh * Dv + v0 + row + r) * Dk + c];
      Sacc[m][r] = x;
    }
  }
  for (int idx = tid; idx < BV * LD; idx += kThreads) {
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

  // one of the ten lower 16 x 16 tiles (ib, jb) of a C x C product of lower-triangular
  // factors: sum over k from column block jb to row block ib of (sgnX X)[rows][k] Y[k][cols],
  // X and Y row-major in LDS (row strides LX, LY)
  auto lower_mm = [&](const float *X, int LX, const float *Y, int LY, int u, float sgnX) {
    int ib, jb;
    lower_tile(u, ib, jb);
    float4v acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 16 * jb; k0 < 16 * ib + 16; k0 += 4)
      acc = mfma4(sgnX * X[(16 * ib + col) * LX + k0 + kq], Y[(k0 + kq) * LY + 16 * jb + col], acc);
    return acc;
  };

  const int step = C128 ? kCMax : a.C;
  for (int c0 = 0; c0 < T; c0 += step) {
    const int n = min(step, T - c0);
    // chunk 128: half b of a chunk, or half a with a half b to follow (then n = 64)
    const bool hb = C128 && ((c0 / kCMax) & 1) != 0;
    const bool ha = C128 && !hb && c0 + kCMax < T;
    // token (b, c0 + t, h) row index in [B, T, H]
    auto tok = [&](int t) -> long long { return (static_cast<long long>(b) * T + c0 + t) * H + h; };
    const long long row0 = tok(0);
    const int rstride = H * Dk;

    __syncthreads();  // previous chunk done with every buffer
    if (ha) {   // the chunk's start state, for half b's X
      for (int idx = tid; idx < BV * LD; idx += kThreads) (&Ss2[0][0])[idx] = (&Ss[0][0])[idx];
    }
    {   // write keys (the preconditioned ones are formed from them below), erase keys and, with
        // per-channel decays, the log decays: all loads first (clamped), then the masked stores
      float xr[kLoadIt], xk[kLoadIt], xg[kLoadIt], xl[CHD ? kLoadIt : 1];
      const IO *rsrc = ((a.wkey == GDR_WKEY_EXPLICIT) ? wk : k) + row0 * Dk, *kc = k + row0 * Dk;
      const IO *ec = er + row0 * Dk;
      const float *bc = a.beta + row0;
#pragma unroll
      for (int it = 0; it < kLoadIt; ++it) {
        const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
        const int tc = min(t, n - 1), o = tc * rstride + min(c, Dk - 1);
        xr[it] = ld_f(rsrc, o);
        xk[it] = ld_f(kc, o);
        xg[it] = a.gain == GDR_GAIN_SCALAR ? bc[tc * H] : ld_f(ec, o);
        if constexpr (CHD) xl[it] = a.log_alpha[row0 * Dk + o];
      }
#pragma unroll
      for (int it = 0; it < kLoadIt; ++it) {
        const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
        const bool in = t < n && c < Dk;
        Rs[t][c] = in ? xr[it] : 0.f;
        Xs[t][c] = in ? xg[it] * xk[it] : 0.f;
        if constexpr (CHD) Gs[t][c] = in ? xl[it] : 0.f;
      }
    }
    // gates: inclusive cumulative sum of log alpha over the chunk (one wave; zero without a
    // scalar decay)
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
      float *icorr = kTight ? &Zb[0][0] : &Zs[0][0];   // (free until the inverse is built)
      if (tid < kCMax) {
        const float tg = static_cast<float>(a.t0 + c0 + tid + 1);
        icorr[tid] = 1.f / -expm1f(tg * a.log_rho);   // 1 / (1 - rho^t)
      }
      __syncthreads();
      if (tid < Dk) {
        // rows past n hold zero keys (their u comes out zero); the accumulator skips them.
        // Keys are read 16 at a time ahead of the serial chain.
        for (int t0 = 0; t0 < kCMax; t0 += 16) {
          float kv[16];
#pragma unroll
          for (int t = 0; t < 16; ++t) kv[t] = Rs[t0 + t][tid];
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const float hn = fmaf(a.rho, hreg, kv[t] * kv[t]);
            hreg = t0 + t < n ? hn : hreg;
            Rs[t0 + t][tid] = kv[t] / fmaf(hreg, icorr[t0 + t], a.eps);
          }
        }
      }
    }
    if constexpr (CHD) {
      // each channel's inclusive cumulative sum of log decays in log2 units (rows past n are
      // zero, so the sums stay flat there)
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
    __syncthreads();

    // LP[i][j] = decay_ij (X_i . R_j) for j < i (or j <= i) on the tiles on and below the
    // diagonal; rows past n hold zero keys, so they come out zero
    auto gram = [&](bool incl_diag) {
      if constexpr (CHD) {
        chd::gram<DK, LD>(Xs, Rs, Gs, LP, incl_diag, tid);
      } else {
        for (int u = wave; u < 10; u += 8) {
          int ib, jb;
          lower_tile(u, ib, jb);
          const float4v acc = dot_kc<DK>(&Xs[16 * ib + col][0], &Rs[16 * jb + col][0], kq);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * ib + 4 * kq + r, j = 16 * jb + col;
            LP[i][j] = (j < i || (incl_diag && j == i)) ? expf(gs[i] - gs[j]) * acc[r] : 0.f;
          }
        }
      }
    };
    // the read of the state mirror Sm through row t of Y (E or Q): f e^g_t Y_t, or 2^G_t (.) Y_t
    auto state_read = [&](const float(*Y)[LD], const float(*Sm)[LD], float f, float4v &acc) {
      const int t = 16 * tb + col;
      if constexpr (CHD) {
        // (k order permuted as in dot_kc)
        float4v a1 = {0.f, 0.f, 0.f, 0.f};
        acc = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
        for (int ks = 0; ks < DK; ks += 16) {
          const int kk = ks + 4 * kq;
          const float4 y = ld4(&Y[t][kk]), g = ld4(&Gs[t][kk]), z = ld4(&Sm[16 * rb + col][kk]);
          acc = mfma4(y.x * chd::ex2(g.x), z.x, acc);
          a1 = mfma4(y.y * chd::ex2(g.y), z.y, a1);
          acc = mfma4(y.z * chd::ex2(g.z), z.z, acc);
          a1 = mfma4(y.w * chd::ex2(g.w), z.w, a1);
        }
        acc += a1;
      } else {
        acc = dot_kc<DK>(&Y[t][0], &Sm[16 * rb + col][0], kq);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= C128 ? f * eg[16 * tb + 4 * kq + r] : eg[16 * tb + 4 * kq + r];
      }
    };

    // L (strict lower)
    gram(false);
    if (hb && wave == 7) {
      // Z = A_ba T_aa on the corner: rows 0..15 of half b against rows 48..63 of half a, where
      // A_ij = -e^{g'_i} e^{g_63 - g_j} (e_i . r_j)
      const float4v l = dot_kc<DK>(&Xs[col][0], &Rat[col][0], kq);
#pragma unroll
      for (int r = 0; r < 4; ++r) Zc[4 * kq + r][col] = -eg[4 * kq + r] * wdt[col] * l[r];
      tri::wave_sync();
      float4v z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4) z = mfma4(Zc[col][k0 + kq], Taa[k0 + kq][col], z);
      tri::wave_sync();
#pragma unroll
      for (int r = 0; r < 4; ++r) Zc[4 * kq + r][col] = z[r];
    }
    // X = V' - (e^g (.) E) S^T on the value tile
    if (xwave) {
      float vp[4];   // (loads from clamped indices; entries outside the tile are masked below)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = min(16 * tb + 4 * kq + r, n - 1), rr = min(16 * rb + col, nv - 1);
        const long long vi = tok(t) * Dv + v0 + rr;
        const float vv = ld_f(v, vi);
        vp[r] = (a.gain == GDR_GAIN_SCALAR) ? a.beta[tok(t)] * vv : ld_f(wr, vi) * vv;
      }
      float4v acc;
      if (hb)
        state_read(Xs, Ss2, ega[0], acc);   // half b reads the chunk's start state
      else
        state_read(Xs, Ss, 1.f, acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tb + 4 * kq + r, rr = 16 * rb + col;
        Xv[t][rr] = (t < n && rr < nv) ? vp[r] - acc[r] : 0.f;
      }
    }
    __syncthreads();
    // the queries' loads are issued here, so they are in flight during the inverse; they
    // replace the erase keys in LDS after it
    float xq[kLoadIt];
    {
      const IO *qc = q + row0 * Dk;
#pragma unroll
      for (int it = 0; it < kLoadIt; ++it) {
        const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
        xq[it] = ld_f(qc, min(t, n - 1) * rstride + min(c, Dk - 1));
      }
    }
    // T = (I - A)^-1 by 16 x 16 blocks (exact, or its band i - j <= N)
    tri::inverse_blocks(LP, Tm, Zs, a.N, tid);
    // Parallel residual correction of the band start T0 (MatMul-only inversion summary,
    // Metodologia 3): E = I - (I - A) T0 = I - T0 + A T0, Z = I + E (I + E (... (I + E))) with S
    // factors (= sum_{s<=S} E^s), T = T0 Z.  All factors are lower triangular, so each product
    // is formed on the ten lower tiles, each tile summing over the k-blocks between its
    // column and row blocks; every product is formed in registers and written back after a
    // barrier (E over L, Z in place, T over T0).
    if ((CHD || C128) ? false : a.S > 0) {
      float4v e[2];
      for (int u = wave, m = 0; u < 10; u += 8, ++m) e[m] = lower_mm(&LP[0][0], kCMax + 1, &Tm[0][0], kCMax + 4, u, -1.f);
      __syncthreads();   // every row of A has been read
      for (int u = wave, m = 0; u < 10; u += 8, ++m) {
        int ib, jb;
        lower_tile(u, ib, jb);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * ib + 4 * kq + r, j = 16 * jb + col;
          LP[i][j] = ((i == j) ? 1.f : 0.f) - Tm[i][j] + e[m][r];
        }
      }
      for (int idx = tid; idx < kCMax * kCMax; idx += kThreads) {
        const int i = idx / kCMax, j = idx % kCMax;
        Zb[i][j] = i == j ? 1.f : 0.f;
      }
      __syncthreads();
      for (int st = 0; st < a.S; ++st) {   // Z <- I + E Z
        float4v z[2];
        for (int u = wave, m = 0; u < 10; u += 8, ++m) z[m] = lower_mm(&LP[0][0], kCMax + 1, &Zb[0][0], kCMax + 4, u, 1.f);
        __syncthreads();
        for (int u = wave, m = 0; u < 10; u += 8, ++m) {
          int ib, jb;
          lower_tile(u, ib, jb);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * ib + 4 * kq + r, j = 16 * jb + col;
            Zb[i][j] = ((i == j) ? 1.f : 0.f) + z[m][r];
          }
        }
        __syncthreads();
      }
      // T = T0 Z
      float4v tz[2];
      for (int u = wave, m = 0; u < 10; u += 8, ++m) tz[m] = lower_mm(&Tm[0][0], kCMax + 4, &Zb[0][0], kCMax + 4, u, 1.f);
      __syncthreads();
      for (int u = wave, m = 0; u < 10; u += 8, ++m) {
        int ib, jb;
        lower_tile(u, ib, jb);
#pragma unroll
        for (int r = 0; r < 4; ++r) Tm[16 * ib + 4 * kq + r][16 * jb + col] = tz[m][r];
      }
    }
    {   // queries replace the erase keys (their last reads, L and X, were before the barriers above)
#pragma unroll
      for (int it = 0; it < kLoadIt; ++it) {
        const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
        Xs[t][c] = (t < n && c < Dk) ? xq[it] : 0.f;
      }
    }
    __syncthreads();
    // D = T X (T lower triangular: the sum ends with the row block)
    float4v dacc = {0.f, 0.f, 0.f, 0.f};
    if (xwave) {
      for (int s0 = 0; s0 < 16 * (tb + 1); s0 += 4)
        dacc = mfma4(Tm[16 * tb + col][s0 + kq], Xv[s0 + kq][16 * rb + col], dacc);
      if (hb && tb == 0) {
        // + band(T_ba) X_a: W = T_bb Z on the corner, entry (i, j) being T's (64 + i, 48 + j)
        float4v w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) w = mfma4(Tm[col][k0 + kq], Zc[k0 + kq][col], w);
        tri::wave_sync();
#pragma unroll
        for (int r = 0; r < 4; ++r) Zc[4 * kq + r][col] = 4 * kq + r + 16 - col <= a.N ? w[r] : 0.f;
        tri::wave_sync();
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) dacc = mfma4(Zc[col][k0 + kq], Xat[k0 + kq][16 * rb + col], dacc);
      }
      if constexpr (!kTight) {
#pragma unroll
        for (int r = 0; r < 4; ++r) Dl[16 * tb + 4 * kq + r][16 * rb + col] = dacc[r];
      }
    }
    if (ha && wave >= 4) {   // (16-row value tiles: waves 4..7 hold no tile of X, D or O)
      const int t4 = tid - 256;
      for (int idx = t4; idx < 16 * LD; idx += 256) Rat[idx / LD][idx % LD] = Rs[48 + idx / LD][idx % LD];
      Taa[t4 >> 4][t4 & 15] = Tm[48 + (t4 >> 4)][48 + (t4 & 15)];
      Xat[t4 >> 4][t4 & 15] = Xv[48 + (t4 >> 4)][t4 & 15];
      if (t4 < 16) wdt[t4] = wd[48 + t4];
      if (t4 == 0) ega[0] = eg[kCMax - 1];
    }
    // P (lower incl. diagonal; L is no longer needed)
    gram(true);
    __syncthreads();
    if constexpr (kTight) {   // every read of X is done: D takes its place
      if (xwave) {
#pragma unroll
        for (int r = 0; r < 4; ++r) Dl[16 * tb + 4 * kq + r][16 * rb + col] = dacc[r];
      }
      __syncthreads();
    }
    // O = scale ((e^g (.) Q) S^T + P D)
    if (xwave) {
      float4v acc;
      state_read(Xs, Ss, 1.f, acc);
      for (int j0 = 0; j0 < 16 * (tb + 1); j0 += 4)
        acc = mfma4(LP[16 * tb + col][j0 + kq], Dl[j0 + kq][16 * rb + col], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tb + 4 * kq + r, rr = 16 * rb + col;
        if (t < n && rr < nv) st_f(out, tok(t) * Dv + v0 + rr, a.scale * acc[r]);
      }
    }
    __syncthreads();   // every read of the state mirror is done
    // S <- e^{g_n} S + D^T (e^{g_n - g} (.) R); per-channel decays: S Diag(2^{G_C}) +
    // D^T (2^(G_C - G) (.) R).  Rows of D past n are zero.
    {
      const float gl = eg[n - 1];
#pragma unroll
      for (int m = 0; m < NTW; ++m) {
        const int u = wave + 8 * m;
        if (u >= NTS) continue;
        const int rbs = u / NCB, cbs = u % NCB, c = 16 * cbs + col;
        float4v acc = Sacc[m], acc2 = {0.f, 0.f, 0.f, 0.f};   // two independent chains
        if constexpr (CHD) {
          acc *= chd::ex2(Gs[n - 1][c]);
        } else {
          acc *= gl;
        }
        for (int t0 = 0; t0 < n; t0 += 8) {
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const int t = t0 + 4 * p + kq;
            float am = Dl[t][16 * rbs + col], br = Rs[t][c];
            if constexpr (CHD)
              br *= chd::ex2(Gs[n - 1][c] - Gs[t][c]);
            else
              am *= wd[t];
            if (p == 0)
              acc = mfma4(am, br, acc);
            else
              acc2 = mfma4(am, br, acc2);
          }
        }
        acc += acc2;
        Sacc[m] = acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) Ss[16 * rbs + 4 * kq + r][c] = acc[r];
      }
    }
  }
  if (a.state_out != nullptr) {
#pragma unroll
    for (int m = 0; m < NTW; ++m) {
      const int u = wave + 8 * m;
      const int row = 16 * (u / NCB) + 4 * kq, c = 16 * (u % NCB) + col;
      if (u < NTS && c < Dk) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (row + r < nv) a.state_out[(sh * Dv + v0 + row + r) * Dk + c] = Sacc[m][r];
      }
    }
  }
  if (a.wkey == GDR_WKEY_DIAG_PRECOND && a.pc_h_out != nullptr && vt == 0 && tid < Dk)
    a.pc_h_out[sh * Dk + tid] = hreg;
}

template <typename IO, bool CHD, int BV, bool C128 = false>
hipError_t launch_dk(const ChunkArgs &a, hipStream_t s) {
  const dim3 grid((a.Dv + BV - 1) / BV, a.H, a.B);
  if (a.Dk <= 32)
    hipLaunchKernelGGL((chunk_generic_kernel<IO, 32, CHD, BV, C128>), grid, dim3(kThreads), 0, s, a);
  else if (a.Dk <= 64)
    hipLaunchKernelGGL((chunk_generic_kernel<IO, 64, CHD, BV, C128>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((chunk_generic_kernel<IO, 128, CHD, BV, C128>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// Workgroups own 32 value rows.  With per-channel decays the Gram tiles (the larger part of a
// chunk) do not depend on the value tile, so 32 rows halve their total against 16; 16 rows
// are kept only where 32 would leave CUs without a workgroup.  GDR_GENERIC_BV=16|32
// overrides that choice (tuning and tests).
template <typename IO>
hipError_t launch_io(const ChunkArgs &a, hipStream_t s) {
  // chunk 128 reaches this kernel only with a band limit 0 <= N <= 15 and scalar or no decay
  if (a.C == 2 * kCMax) return launch_dk<IO, false, 16, true>(a, s);
  if (a.decay != GDR_DECAY_CHANNEL) return launch_dk<IO, false, 32>(a, s);
  const char *e = getenv("GDR_GENERIC_BV");
  const int forced = e == nullptr ? 0 : atoi(e);
  const bool wide = forced == 16 || forced == 32
                        ? forced == 32
                        : static_cast<long long>(a.B) * a.H * ((a.Dv + 31) / 32) >= 256;
  return wide ? launch_dk<IO, true, 32>(a, s) : launch_dk<IO, true, 16>(a, s);
}

}  // namespace

hipError_t launch_chunk_generic(const ChunkArgs &a, int io_dtype, hipStream_t s) {
  return io_dtype == GDR_BF16 ? launch_io<uint16_t>(a, s) : launch_io<float>(a, s);
}

}  // namespace gdr
