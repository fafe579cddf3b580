// Backward pass of the chunked gated delta rule: fp32 arithmetic on the vector ALUs.
//
// The pages give no backward; this is the derivative of the chunk-wise forward
// ("Declaracao do Problema" of the MatMul-only inversion summary).  Per chunk of n tokens
// starting from state S (Dv x Dk), with g the in-chunk cumulative log decay,
// Gamma_ij = exp(g_i - g_j), L = tril_{-1}((E R^T) (.) Gamma), T = (I + L)^-1:
//   X = V' - (e^g (.) E) S^T,  D = T X,  P = tril_0((Q R^T) (.) Gamma),
//   O = scale ((e^g (.) Q) S^T + P D),  S' = e^{g_n} S + D^T (e^{g_n - g} (.) R).
// Given dO and dS' (the gradient at the chunk's end, including every later chunk):
//   dD  = e^{g_n - g} (.) (R dS'^T) + scale P^T dO
//   dX  = T^T dD                                   (= dV'; dT = dD X^T gives dL = -dX D^T)
//   dS  = e^{g_n} dS' + scale dO^T (e^g (.) Q) - dX^T (e^g (.) E)
//   dM  = scale (dO D^T) (.) Gamma on j <= i,   dL' = -(dX D^T) (.) Gamma on j < i
//   dQ  = scale e^g (.) (dO S) + dM R
//   dE  = -e^g (.) (dX S) + dL' R
//   dR  = e^{g_n - g} (.) (D dS') + dM^T Q + dL'^T E
//   dg_i = q_i . dQ_i + e_i . dE_i - r_i . dR_i
//          (+ e^{g_n} <dS', S> + sum_j r_j . (e^{g_n - g_j} dS'^T d_j) for i = n)
//   dlog_alpha = in-chunk reverse cumulative sum of dg.
// Four kernels: the chunk preparation (parallel over chunks: T, P, W = T (e^g (.) E),
// U = T V'), the state pass (sequential over chunks, per value tile: D = U - W S^T and the
// state at every chunk start), the reverse sweep (sequential over chunks, per value tile,
// last to first: carries dS, emits dX and the gradient at each chunk's end) and the
// per-chunk pass (parallel over chunks; everything else).
#include "common.h"
#include "tri_blocks.h"

namespace gdr {
namespace {

constexpr int kThreads = 256;
constexpr int kBV = 16;     // state rows per workgroup of the sweep
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
__device__ __forceinline__ float at(const float4 &v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

// g (inclusive cumulative sum of log alpha over tokens 0..n-1, flat past n), e^g and
// e^{g_{n-1} - g} of one chunk; called by the first wave.
__device__ __forceinline__ void chunk_gates(const ChunkArgs &f, long long row0, int n, int lane,
                                            float *gs, float *eg, float *wd) {
  float g = (f.decay == GDR_DECAY_SCALAR && lane < n) ? f.log_alpha[row0 + static_cast<long long>(lane) * f.H] : 0.f;
#pragma unroll
  for (int d = 1; d < kCMax; d <<= 1) {
    const float y = __shfl_up(g, d, kCMax);
    if (lane >= d) g += y;
  }
  const float glast = __shfl(g, n - 1, kCMax);
  gs[lane] = g;
  eg[lane] = expf(g);
  wd[lane] = expf(glast - g);
}

// ---------------------------------------------------------------------------------------
// Chunk preparation: one workgroup per (batch, head, chunk), all chunks at once.  Everything
// of a chunk that does not depend on the state: T = (I + L)^-1 and P (C x C, for the sweep),
// W = T (e^g (.) E) (C x Dk) and U = T V' (C x Dv, for the state pass).
// ---------------------------------------------------------------------------------------
template <typename IO, int DK>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(BwdArgs a) {
  static_assert(DK == 64 || DK == 128, "channel groups of 64");
  constexpr int LD = DK + 4;
  constexpr int NG = DK / 64;
  constexpr int CW = 4 * NG;
  constexpr int kLoadIt = kCMax * DK / kThreads;
  const ChunkArgs &f = a.f;
  const IO *__restrict__ q = static_cast<const IO *>(f.q);
  const IO *__restrict__ k = static_cast<const IO *>(f.k);
  const IO *__restrict__ v = static_cast<const IO *>(f.v);
  const IO *__restrict__ er = static_cast<const IO *>(f.erase);
  const IO *__restrict__ wr = static_cast<const IO *>(f.write);
  const IO *__restrict__ wk = static_cast<const IO *>(f.write_key);

  const int tid = threadIdx.x;
  const int ci = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Dk = f.Dk, Dv = f.Dv, H = f.H, T = f.T, C = f.C;
  const int c0 = ci * C;
  const int n = min(C, T - c0);
  const long long sh = static_cast<long long>(b) * H + h;
  auto tok = [&](int t) -> long long { return (static_cast<long long>(b) * T + c0 + t) * H + h; };
  const long long row0 = tok(0);

  __shared__ __align__(16) float Es[kCMax][LD];   // erase keys e
  __shared__ __align__(16) float Rs[kCMax][LD];   // write keys r
  __shared__ __align__(16) float Xs[kCMax][LD];   // queries, then blocks of V'
  __shared__ float LP[kCMax][kCMax + 1];          // L, then P
  __shared__ __align__(16) float Tm[kCMax][kCMax + 4];
  __shared__ __align__(16) float Zs[32][36];
  __shared__ float gs[kCMax], eg[kCMax], wd[kCMax];

  if (tid < kCMax) chunk_gates(f, row0, n, tid, gs, eg, wd);
  for (int idx = tid; idx < kCMax * kCMax; idx += kThreads) {
    const int i = idx / kCMax, j = idx % kCMax;
    if ((j >> 4) > (i >> 4)) Tm[i][j] = 0.f;
  }
  {   // E, R, Q: all loads first (clamped), then the masked stores
    float xk[kLoadIt], xg[kLoadIt], xr[kLoadIt], xq[kLoadIt];
    const IO *qc = q + row0 * Dk, *kc = k + row0 * Dk, *ec = er + row0 * Dk;
    const IO *rsrc = ((f.wkey == GDR_WKEY_EXPLICIT) ? wk : k) + row0 * Dk;
    const float *bc = f.beta + row0;
#pragma unroll
    for (int it = 0; it < kLoadIt; ++it) {
      const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
      const int tc = min(t, n - 1), o = tc * H * Dk + min(c, Dk - 1);
      xk[it] = ld_f(kc, o);
      xg[it] = f.gain == GDR_GAIN_SCALAR ? bc[tc * H] : ld_f(ec, o);
      xr[it] = ld_f(rsrc, o);
      xq[it] = ld_f(qc, o);
    }
#pragma unroll
    for (int it = 0; it < kLoadIt; ++it) {
      const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
      const bool in = t < n && c < Dk;
      Es[t][c] = in ? xg[it] * xk[it] : 0.f;
      Rs[t][c] = in ? xr[it] : 0.f;
      Xs[t][c] = in ? xq[it] : 0.f;
    }
  }
  __syncthreads();
  // LP[i][j] = exp(g_i - g_j) (X_i . R_j) for j < i (or j <= i), zero elsewhere
  const int bi = tid >> 4, bj = tid & 15;
  auto gram = [&](const float(*X)[LD], bool incl_diag) {
    float acc[4][4] = {};
    if (bj <= bi) {
#pragma unroll 4
      for (int c = 0; c < DK; c += 4) {
        float4 x[4], r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          x[u] = ld4(&X[4 * bi + u][c]);
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
        const bool keep = j < i || (incl_diag && j == i);
        LP[i][j] = keep ? expf(gs[i] - gs[j]) * acc[u][w] : 0.f;
      }
  };
  gram(Es, false);
  __syncthreads();
  tri::inverse_blocks(LP, Tm, Zs, -1, tid);
  gram(Xs, true);
  __syncthreads();
  {   // T and P of the chunk (C x C) for the sweep
    const long long cc = (sh * a.NC + ci) * static_cast<long long>(C * C);
    for (int idx = tid; idx < C * C; idx += kThreads) {
      a.Tw[cc + idx] = Tm[idx / C][idx % C];
      a.Pw[cc + idx] = LP[idx / C][idx % C];
    }
  }
  // thread (ti, cj): rows 4 ti .. 4 ti + 3, columns 64 g + 4 cj .. + 3 of W and U
  const int ti = tid >> 4, cj = tid & 15;
  // acc = T[rows] (Y (.) s) over the thread's columns, with row s of Y scaled by scl(s)
  auto tri_product = [&](const float(*Y)[LD], auto &&scl, float (&acc)[4][CW]) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < CW; ++e) acc[u][e] = 0.f;
    const int send = min(4 * ti + 4, n);
#pragma unroll 4
    for (int s0 = 0; s0 < send; ++s0) {
      float4 y[NG];
      const float sc = scl(s0);
#pragma unroll
      for (int g = 0; g < NG; ++g) y[g] = ld4(&Y[s0][64 * g + 4 * cj]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float tv = sc * Tm[4 * ti + u][s0];   // zero above the diagonal
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[u][4 * g + e] = fmaf(tv, at(y[g], e), acc[u][4 * g + e]);
      }
    }
  };
  {   // W = T (e^g (.) E), [B, H, NC, C, Dk]
    float acc[4][CW];
    tri_product(Es, [&](int s0) { return eg[s0]; }, acc);
    float *Wc = a.Ww + (sh * a.NC + ci) * static_cast<long long>(C) * Dk;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = 4 * ti + u;
      if (t >= n) continue;
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 64 * g + 4 * cj + e;
          if (c < Dk) Wc[static_cast<long long>(t) * Dk + c] = acc[u][4 * g + e];
        }
    }
  }
  // U = T V' by blocks of DK value columns, [B, T, H, Dv]
  for (int vb = 0; vb < Dv; vb += DK) {
    __syncthreads();   // Xs free (P formed / previous block used)
    {
      float xv[kLoadIt], xw[kLoadIt];
      const float *bc = f.beta + row0;
#pragma unroll
      for (int it = 0; it < kLoadIt; ++it) {
        const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
        const int tc = min(t, n - 1);
        const long long o = static_cast<long long>(tc) * H * Dv + min(vb + c, Dv - 1);
        xv[it] = ld_f(v + row0 * Dv, o);
        xw[it] = f.gain == GDR_GAIN_SCALAR ? bc[tc * H] : ld_f(wr + row0 * Dv, o);
      }
#pragma unroll
      for (int it = 0; it < kLoadIt; ++it) {
        const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
        Xs[t][c] = (t < n && vb + c < Dv) ? xw[it] * xv[it] : 0.f;
      }
    }
    __syncthreads();
    float acc[4][CW];
    tri_product(Xs, [&](int) { return 1.f; }, acc);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = 4 * ti + u;
      if (t >= n) continue;
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = vb + 64 * g + 4 * cj + e;
          if (c < Dv) a.Uw[tok(t) * Dv + c] = acc[u][4 * g + e];
        }
    }
  }
}

// ---------------------------------------------------------------------------------------
// State pass: one workgroup per (batch, head, tile of kBV value rows), chunks first to last.
// With W and U of every chunk at hand only the state-dependent part remains:
// D = U - W S^T (saved) and S <- e^{g_n} S + D^T (e^{g_n - g} (.) R); the state at every
// chunk start is saved too.  The next chunk's W, R and U are loaded during this chunk.
// ---------------------------------------------------------------------------------------
template <typename IO, int DK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void bwd_state_kernel(BwdArgs a) {
  constexpr int LD = DK + 4;
  constexpr int kLoadIt = kCMax * DK / kThreads;
  constexpr int kUIt = kCMax * kBV / kThreads;
  const ChunkArgs &f = a.f;
  const IO *__restrict__ k = static_cast<const IO *>(f.k);
  const IO *__restrict__ wk = static_cast<const IO *>(f.write_key);

  const int tid = threadIdx.x;
  const int vt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int v0 = vt * kBV;
  const int nv = min(kBV, f.Dv - v0);
  const int Dk = f.Dk, Dv = f.Dv, H = f.H, T = f.T, C = f.C;
  const long long sh = static_cast<long long>(b) * H + h;

  __shared__ __align__(16) float Ws[kCMax][LD];   // W of the chunk
  __shared__ __align__(16) IO Rs[kCMax][LD];      // write keys (in the io type: exact)
  __shared__ __align__(16) float Ss[kBV][LD];     // state tile
  __shared__ __align__(16) float Dl[kCMax][kBV];  // D, then e^{g_n - g} D
  __shared__ __align__(16) float Us[kCMax][kBV];  // U
  __shared__ float gs[kCMax], eg[kCMax], wd[kCMax];

  for (int idx = tid; idx < kBV * LD; idx += kThreads) {
    const int r = idx / LD, c = idx % LD;
    float s = 0.f;
    if (f.state_in != nullptr && r < nv && c < Dk) s = f.state_in[(sh * Dv + v0 + r) * Dk + c];
    Ss[r][c] = s;
  }
  const IO *rbase = (f.wkey == GDR_WKEY_EXPLICIT) ? wk : k;
  float pw[kLoadIt], pu[kUIt];
  IO pr[kLoadIt];
  // loads of chunk ci into registers (indices clamped into the chunk)
  auto cload = [&](int ci) {
    const int c0 = ci * C, n = min(C, T - c0);
    const long long row0 = (static_cast<long long>(b) * T + c0) * H + h;
    const float *Wc = a.Ww + (sh * a.NC + ci) * static_cast<long long>(C) * Dk;
#pragma unroll
    for (int it = 0; it < kLoadIt; ++it) {
      const int idx = tid + it * kThreads, t = min(idx / DK, n - 1), c = min(idx % DK, Dk - 1);
      pw[it] = Wc[static_cast<long long>(t) * Dk + c];
      pr[it] = rbase[(row0 + static_cast<long long>(t) * H) * Dk + c];
    }
#pragma unroll
    for (int it = 0; it < kUIt; ++it) {
      const int idx = tid + it * kThreads, t = min(idx / kBV, n - 1), r = min(idx % kBV, nv - 1);
      pu[it] = a.Uw[(row0 + static_cast<long long>(t) * H) * Dv + v0 + r];
    }
  };
  const int t0 = 2 * (tid >> 3), r0 = 2 * (tid & 7);
  if (a.NC > 0) cload(0);
  for (int ci = 0; ci < a.NC; ++ci) {
    const int c0 = ci * C;
    const int n = min(C, T - c0);
    auto tok = [&](int t) -> long long { return (static_cast<long long>(b) * T + c0 + t) * H + h; };
    __syncthreads();   // previous chunk done with every buffer
    {   // the state at this chunk's start
      float *hc = a.h + ((sh * a.NC + ci) * Dv + v0) * static_cast<long long>(Dk);
      for (int idx = tid; idx < nv * Dk; idx += kThreads) hc[idx] = Ss[idx / Dk][idx % Dk];
    }
#pragma unroll
    for (int it = 0; it < kLoadIt; ++it) {
      const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
      const bool in = t < n && c < Dk;
      Ws[t][c] = in ? pw[it] : 0.f;
      Rs[t][c] = in ? pr[it] : IO(0);
    }
#pragma unroll
    for (int it = 0; it < kUIt; ++it) {
      const int idx = tid + it * kThreads, t = idx / kBV, r = idx % kBV;
      Us[t][r] = (t < n && r < nv) ? pu[it] : 0.f;
    }
    if (tid < kCMax) chunk_gates(f, tok(0), n, tid, gs, eg, wd);
    __syncthreads();
    if (ci + 1 < a.NC) cload(ci + 1);   // in flight during this chunk's products
    {   // D = U - W S^T on the thread's 2 x 2 block
      float acc[2][2] = {};
#pragma unroll 4
      for (int c = 0; c < DK; c += 4) {
        const float4 x0 = ld4(&Ws[t0][c]), x1 = ld4(&Ws[t0 + 1][c]);
        const float4 s0 = ld4(&Ss[r0][c]), s1 = ld4(&Ss[r0 + 1][c]);
        fma4(acc[0][0], x0, s0);
        fma4(acc[0][1], x0, s1);
        fma4(acc[1][0], x1, s0);
        fma4(acc[1][1], x1, s1);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const int t = t0 + u, r = r0 + w;
          const bool in = t < n && r < nv;
          const float d = Us[t][r] - acc[u][w];
          if (in) a.D[tok(t) * Dv + v0 + r] = d;
          Dl[t][r] = in ? wd[t] * d : 0.f;
        }
    }
    __syncthreads();
    // S <- e^{g_n} S + (e^{g_n - g} (.) D)^T R: thread (row r, columns c .. c + 3)
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
        // rows past n hold zeros, so the sum may run to the next multiple of 8
        for (int j0 = 0; j0 < n; j0 += 8) {
#pragma unroll
          for (int j = j0; j < j0 + 8; ++j) {
            const float w = Dl[j][r];
            acc.x = fmaf(w, ld_f(&Rs[j][c], 0), acc.x);
            acc.y = fmaf(w, ld_f(&Rs[j][c], 1), acc.y);
            acc.z = fmaf(w, ld_f(&Rs[j][c], 2), acc.z);
            acc.w = fmaf(w, ld_f(&Rs[j][c], 3), acc.w);
          }
        }
        *reinterpret_cast<float4 *>(&Ss[r][c]) = acc;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Reverse sweep: one workgroup of kSwThreads per (batch, head, tile of kSwBV value rows),
// chunks last to first.  dS (kSwBV x Dk) stays in LDS.  Two waves per SIMD, so one wave's
// LDS and global latencies overlap the other's arithmetic.
// ---------------------------------------------------------------------------------------
constexpr int kSwBV = 32;
constexpr int kSwThreads = 512;

template <typename IO, int DK>
__global__ __launch_bounds__(kSwThreads) void bwd_sweep_kernel(BwdArgs a) {
  constexpr int LD = DK + 4;
  constexpr int kBV = kSwBV, kThreads = kSwThreads;
  constexpr int kLoadIt = kCMax * DK / kThreads;
  const ChunkArgs &f = a.f;
  const IO *__restrict__ q = static_cast<const IO *>(f.q);
  const IO *__restrict__ k = static_cast<const IO *>(f.k);
  const IO *__restrict__ er = static_cast<const IO *>(f.erase);
  const IO *__restrict__ wk = static_cast<const IO *>(f.write_key);
  const IO *__restrict__ dout = static_cast<const IO *>(a.dout);

  const int tid = threadIdx.x;
  const int vt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int v0 = vt * kBV;
  const int nv = min(kBV, f.Dv - v0);
  const int Dk = f.Dk, Dv = f.Dv, H = f.H, T = f.T, C = f.C;

  __shared__ __align__(16) float Ks[kCMax][LD];     // write keys r, then queries q
  __shared__ __align__(16) float Es[kCMax][LD];     // erase keys e
  __shared__ float Tm[kCMax][kCMax + 1];            // T (unit lower)
  __shared__ float Pm[kCMax][kCMax + 1];            // P (lower)
  __shared__ __align__(16) float dS[kBV][LD];       // gradient at the current chunk's end
  __shared__ __align__(16) float dOs[kCMax][kBV];   // dO
  __shared__ __align__(16) float dDs[kCMax][kBV];   // dD
  __shared__ __align__(16) float Am[kCMax][kBV];    // scale e^g dO
  __shared__ __align__(16) float Bm[kCMax][kBV];    // e^g dX
  __shared__ float gs[kCMax], eg[kCMax], wd[kCMax];

  const long long sh = static_cast<long long>(b) * H + h;
  for (int idx = tid; idx < kBV * LD; idx += kThreads) {
    const int r = idx / LD, c = idx % LD;
    float s = 0.f;
    if (a.dstate_out != nullptr && r < nv && c < Dk) s = a.dstate_out[(sh * Dv + v0 + r) * Dk + c];
    dS[r][c] = s;
  }
  const int t0 = 2 * (tid >> 4), r0 = 2 * (tid & 15);   // 2 x 2 block of the C x kBV tiles

  for (int ci = a.NC - 1; ci >= 0; --ci) {
    const int c0 = ci * C;
    const int n = min(C, T - c0);
    auto tok = [&](int t) -> long long { return (static_cast<long long>(b) * T + c0 + t) * H + h; };
    const long long row0 = tok(0);
    const int rstride = H * Dk;

    __syncthreads();   // previous chunk done with every buffer
    // Every load of the chunk is issued before the first LDS store (indices clamped into the
    // chunk, masks applied afterwards), so they are in flight together: write keys, keys,
    // gains, queries (kept in registers until the write keys are dead), T, P and dO.
    constexpr int kCC = kCMax * kCMax / kThreads, kOIt = kCMax * kBV / kThreads;
    float xr[kLoadIt], xk[kLoadIt], xg[kLoadIt], xq[kLoadIt], xt[kCC], xp[kCC], xo[kOIt];
    {
      const IO *rsrc = ((f.wkey == GDR_WKEY_EXPLICIT) ? wk : k) + row0 * Dk;
      const IO *kc = k + row0 * Dk, *qc = q + row0 * Dk;
      const IO *ec = er + row0 * Dk;
      const float *bc = f.beta + row0;
#pragma unroll
      for (int it = 0; it < kLoadIt; ++it) {
        const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
        const int tc = min(t, n - 1), o = tc * rstride + min(c, Dk - 1);
        xr[it] = ld_f(rsrc, o);
        xk[it] = ld_f(kc, o);
        xg[it] = f.gain == GDR_GAIN_SCALAR ? bc[tc * H] : ld_f(ec, o);
        xq[it] = ld_f(qc, o);
      }
      const long long cc = (sh * a.NC + ci) * static_cast<long long>(C * C);
#pragma unroll
      for (int it = 0; it < kCC; ++it) {
        const int idx = min(tid + it * kThreads, C * C - 1);
        xt[it] = a.Tw[cc + idx];
        xp[it] = a.Pw[cc + idx];
      }
#pragma unroll
      for (int it = 0; it < kOIt; ++it) {
        const int idx = tid + it * kThreads, t = min(idx / kBV, n - 1), r = min(idx % kBV, nv - 1);
        xo[it] = ld_f(dout, tok(t) * Dv + v0 + r);
      }
    }
    if (tid < kCMax) chunk_gates(f, row0, n, tid, gs, eg, wd);
    {   // the gradient at this chunk's end, for the per-chunk pass
      float *dhc = a.dh + ((sh * a.NC + ci) * Dv + v0) * static_cast<long long>(Dk);
      for (int idx = tid; idx < nv * Dk; idx += kThreads) dhc[idx] = dS[idx / Dk][idx % Dk];
    }
#pragma unroll
    for (int it = 0; it < kLoadIt; ++it) {
      const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
      const bool in = t < n && c < Dk;
      Ks[t][c] = in ? xr[it] : 0.f;
      Es[t][c] = in ? xg[it] * xk[it] : 0.f;
    }
#pragma unroll
    for (int it = 0; it < kCC; ++it) {
      const int idx = tid + it * kThreads;
      if (idx < C * C) {
        Tm[idx / C][idx % C] = xt[it];
        Pm[idx / C][idx % C] = xp[it];
      }
    }
#pragma unroll
    for (int it = 0; it < kOIt; ++it) {
      const int idx = tid + it * kThreads, t = idx / kBV, r = idx % kBV;
      dOs[t][r] = (t < n && r < nv) ? xo[it] : 0.f;
    }
    __syncthreads();
    // dD = e^{g_n - g} (.) (R dS^T) + scale P^T dO on the thread's 2 x 2 block
    {
      float acc[2][2] = {};
#pragma unroll 4
      for (int c = 0; c < DK; c += 4) {
        const float4 x0 = ld4(&Ks[t0][c]), x1 = ld4(&Ks[t0 + 1][c]);
        const float4 s0 = ld4(&dS[r0][c]), s1 = ld4(&dS[r0 + 1][c]);
        fma4(acc[0][0], x0, s0);
        fma4(acc[0][1], x0, s1);
        fma4(acc[1][0], x1, s0);
        fma4(acc[1][1], x1, s1);
      }
      float p[2][2] = {};
      // P is zero above the diagonal, and T, P and dO rows past n (up to the next multiple of
      // 8, inside the chunk) hold zeros, so the sums run over whole blocks of 8 rows
      for (int i0 = t0 & ~7; i0 < n; i0 += 8) {
#pragma unroll
        for (int i = i0; i < i0 + 8; ++i) {
          const float2 o = ld2(&dOs[i][r0]);
          const float p0 = Pm[i][t0], p1 = Pm[i][t0 + 1];
          p[0][0] = fmaf(p0, o.x, p[0][0]);
          p[0][1] = fmaf(p0, o.y, p[0][1]);
          p[1][0] = fmaf(p1, o.x, p[1][0]);
          p[1][1] = fmaf(p1, o.y, p[1][1]);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const int t = t0 + u, r = r0 + w;
          dDs[t][r] = (t < n && r < nv) ? fmaf(wd[t], acc[u][w], f.scale * p[u][w]) : 0.f;
        }
    }
    __syncthreads();
    // dX = T^T dD (T unit lower, zero above the diagonal); written out for the per-chunk
    // pass, and folded with e^g into the state-gradient update
    {
      float x[2][2] = {};
      for (int i0 = t0 & ~7; i0 < n; i0 += 8) {
#pragma unroll
        for (int i = i0; i < i0 + 8; ++i) {
          const float2 d = ld2(&dDs[i][r0]);
          const float a0 = Tm[i][t0], a1 = Tm[i][t0 + 1];
          x[0][0] = fmaf(a0, d.x, x[0][0]);
          x[0][1] = fmaf(a0, d.y, x[0][1]);
          x[1][0] = fmaf(a1, d.x, x[1][0]);
          x[1][1] = fmaf(a1, d.y, x[1][1]);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const int t = t0 + u, r = r0 + w;
          const bool in = t < n && r < nv;
          if (in) a.dX[tok(t) * Dv + v0 + r] = x[u][w];
          Bm[t][r] = in ? eg[t] * x[u][w] : 0.f;
          Am[t][r] = in ? f.scale * eg[t] * dOs[t][r] : 0.f;
        }
    }
    // queries replace the write keys (their last read was before the barrier above)
#pragma unroll
    for (int it = 0; it < kLoadIt; ++it) {
      const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
      Ks[t][c] = (t < n && c < Dk) ? xq[it] : 0.f;
    }
    __syncthreads();
    // dS <- e^{g_n} dS + A^T Q - B^T E: thread (row r, columns c .. c + 3)
    {
      const float gl = eg[n - 1];
      constexpr int NC4 = DK / 4;
#pragma unroll
      for (int u0 = 0; u0 < kBV * NC4; u0 += kThreads) {
        const int u = u0 + tid;
        if (kBV * NC4 % kThreads != 0 && u >= kBV * NC4) break;
        const int r = u / NC4, c = (u % NC4) * 4;
        const float4 s = ld4(&dS[r][c]);
        float4 acc = make_float4(gl * s.x, gl * s.y, gl * s.z, gl * s.w);
        for (int j0 = 0; j0 < n; j0 += 8) {
#pragma unroll
          for (int j = j0; j < j0 + 8; ++j) {
            const float am = Am[j][r], bm = Bm[j][r];
            const float4 qq = ld4(&Ks[j][c]), ee = ld4(&Es[j][c]);
            acc.x = fmaf(am, qq.x, fmaf(-bm, ee.x, acc.x));
            acc.y = fmaf(am, qq.y, fmaf(-bm, ee.y, acc.y));
            acc.z = fmaf(am, qq.z, fmaf(-bm, ee.z, acc.z));
            acc.w = fmaf(am, qq.w, fmaf(-bm, ee.w, acc.w));
          }
        }
        *reinterpret_cast<float4 *>(&dS[r][c]) = acc;
      }
    }
  }
  __syncthreads();
  if (a.dstate_in != nullptr) {
    for (int idx = tid; idx < nv * Dk; idx += kThreads) {
      const int r = idx / Dk, c = idx % Dk;
      a.dstate_in[(sh * Dv + v0 + r) * Dk + c] = dS[r][c];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Per-chunk pass: one workgroup per (batch, head, chunk).  Thread (ti, cj) owns tokens
// 4 ti .. 4 ti + 3 and key channels 64 g + 4 cj .. + 3 of the C x Dk gradients, and the
// 4 x 4 block (tokens 4 ti.., tokens 4 cj..) of the C x C ones.
// ---------------------------------------------------------------------------------------
template <typename IO, int DK>
__global__ __launch_bounds__(kThreads) void bwd_chunk_kernel(BwdArgs a) {
  static_assert(DK == 64 || DK == 128, "channel groups of 64");
  constexpr int LD = DK + 4;
  constexpr int NG = DK / 64;      // float4 channel groups per thread
  constexpr int CW = 4 * NG;       // channels per thread
  constexpr int kVB = 16;          // value rows per step of the value loop
  constexpr int LT = kCMax + 4;    // row stride of [value][token] and C x C tiles
  constexpr int kLoadIt = kCMax * DK / kThreads;
  const ChunkArgs &f = a.f;
  const IO *__restrict__ q = static_cast<const IO *>(f.q);
  const IO *__restrict__ k = static_cast<const IO *>(f.k);
  const IO *__restrict__ v = static_cast<const IO *>(f.v);
  const IO *__restrict__ er = static_cast<const IO *>(f.erase);
  const IO *__restrict__ wr = static_cast<const IO *>(f.write);
  const IO *__restrict__ wk = static_cast<const IO *>(f.write_key);
  const IO *__restrict__ dout = static_cast<const IO *>(a.dout);

  const int tid = threadIdx.x;
  const int ci = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Dk = f.Dk, Dv = f.Dv, H = f.H, T = f.T, C = f.C;
  const int c0 = ci * C;
  const int n = min(C, T - c0);
  const int ti = tid >> 4, cj = tid & 15;
  const long long sh = static_cast<long long>(b) * H + h;
  auto tok = [&](int t) -> long long { return (static_cast<long long>(b) * T + c0 + t) * H + h; };
  const long long row0 = tok(0);

  struct TilesA {   // value loop: state rows, their gradients, token tiles by value row
    float S[kVB][LD], dS[kVB][LD], dOT[kVB][LT], dXT[kVB][LT], DT[kVB][LT];
  };
  struct TilesB {   // key products: Q, E, R and the C x C gradients dM, dL'
    float Q[kCMax][LD], E[kCMax][LD], R[kCMax][LD], dM[kCMax][LT], dL[kCMax][LT];
  };
  __shared__ __align__(16) union {
    TilesA A;
    TilesB B;
  } sm;
  __shared__ float gs[kCMax], eg[kCMax], wd[kCMax], dgs[kCMax], vdx[kCMax];
  __shared__ float red[2][kThreads / 64];

  if (tid < kCMax) chunk_gates(f, row0, n, tid, gs, eg, wd);

  float AQ[4][CW], AE[4][CW], AR[4][CW], MP[4][4], ML[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int e = 0; e < CW; ++e) AQ[u][e] = AE[u][e] = AR[u][e] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) MP[u][w] = ML[u][w] = 0.f;
  }
  float sdot = 0.f;   // this thread's share of <dS', S>
  float vsum = 0.f;   // this thread's share of v_t . dX_t (scalar gain), t = tid >> 2
  const float *hc = a.h + (sh * a.NC + ci) * static_cast<long long>(Dv) * Dk;
  const float *dhc = a.dh + (sh * a.NC + ci) * static_cast<long long>(Dv) * Dk;

  // ---- value loop: dO S, dX S, D dS', dO D^T, dX D^T --------------------------------
  // Each block of kVB value rows is loaded into registers one block ahead (indices clamped,
  // masks applied when the registers are written to LDS), so its loads are in flight while
  // the previous block is multiplied.
  constexpr int kSIt = kVB * DK / kThreads;   // state elements per thread and block
  float ps[kSIt], pds[kSIt], po[4], px[4], pd[4], pv[4], pw[4];
  const int lt = tid >> 2, rq = 4 * (tid & 3);   // token-tile element (token lt, rows rq ..)
  auto vload = [&](int vb) {
#pragma unroll
    for (int it = 0; it < kSIt; ++it) {
      const int idx = tid + it * kThreads, r = idx / DK, c = idx % DK;
      const long long o = static_cast<long long>(min(vb + r, Dv - 1)) * Dk + min(c, Dk - 1);
      ps[it] = hc[o];
      pds[it] = dhc[o];
    }
    const int tt = min(lt, n - 1);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long long idx = tok(tt) * Dv + min(vb + rq + u, Dv - 1);
      po[u] = ld_f(dout, idx);
      px[u] = a.dX[idx];
      pd[u] = a.D[idx];
      pv[u] = ld_f(v, idx);
      pw[u] = f.gain == GDR_GAIN_SCALAR ? f.beta[tok(tt)] : ld_f(wr, idx);
    }
  };
  vload(0);
  for (int vb = 0; vb < Dv; vb += kVB) {
    const int nvb = min(kVB, Dv - vb);
    __syncthreads();   // previous tiles consumed
#pragma unroll
    for (int it = 0; it < kSIt; ++it) {
      const int idx = tid + it * kThreads, r = idx / DK, c = idx % DK;
      const bool in = r < nvb && c < Dk;
      const float s = in ? ps[it] : 0.f, ds = in ? pds[it] : 0.f;
      sm.A.S[r][c] = s;
      sm.A.dS[r][c] = ds;
      sdot = fmaf(s, ds, sdot);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = rq + u;
      const bool in = lt < n && r < nvb;
      const float gx = in ? px[u] : 0.f;
      sm.A.dOT[r][lt] = in ? po[u] : 0.f;
      sm.A.dXT[r][lt] = gx;
      sm.A.DT[r][lt] = in ? pd[u] : 0.f;
      if (in) {   // dv (and dwrite) are elementwise in dX
        const long long idx = tok(lt) * Dv + vb + r;
        a.dv[idx] = pw[u] * gx;
        if (f.gain == GDR_GAIN_SCALAR)
          vsum = fmaf(pv[u], gx, vsum);
        else
          a.dwrite[idx] = pv[u] * gx;
      }
    }
    __syncthreads();
    if (vb + kVB < Dv) vload(vb + kVB);
    for (int r = 0; r < nvb; ++r) {
      const float4 o4 = ld4(&sm.A.dOT[r][4 * ti]), x4 = ld4(&sm.A.dXT[r][4 * ti]);
      const float4 d4 = ld4(&sm.A.DT[r][4 * ti]), dj = ld4(&sm.A.DT[r][4 * cj]);
      float4 s[NG], ds[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        s[g] = ld4(&sm.A.S[r][64 * g + 4 * cj]);
        ds[g] = ld4(&sm.A.dS[r][64 * g + 4 * cj]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float ou = at(o4, u), xu = at(x4, u), du = at(d4, u);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          MP[u][w] = fmaf(ou, at(dj, w), MP[u][w]);
          ML[u][w] = fmaf(xu, at(dj, w), ML[u][w]);
        }
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            AQ[u][4 * g + e] = fmaf(ou, at(s[g], e), AQ[u][4 * g + e]);
            AE[u][4 * g + e] = fmaf(xu, at(s[g], e), AE[u][4 * g + e]);
            AR[u][4 * g + e] = fmaf(du, at(ds[g], e), AR[u][4 * g + e]);
          }
      }
    }
  }
  vsum += __shfl_xor(vsum, 1);
  vsum += __shfl_xor(vsum, 2);
  if ((tid & 3) == 0) vdx[tid >> 2] = vsum;

  // ---- key products -------------------------------------------------------------------
  __syncthreads();   // the value-loop tiles are dead (the key tiles share their memory)
  {   // Q, E, R: all loads first (clamped), then the masked LDS stores
    float xq[kLoadIt], xk[kLoadIt], xg[kLoadIt], xr[kLoadIt];
    const IO *qc = q + row0 * Dk, *kc = k + row0 * Dk, *ec = er + row0 * Dk;
    const IO *rsrc = ((f.wkey == GDR_WKEY_EXPLICIT) ? wk : k) + row0 * Dk;
    const float *bc = f.beta + row0;
#pragma unroll
    for (int it = 0; it < kLoadIt; ++it) {
      const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
      const int tc = min(t, n - 1), o = tc * H * Dk + min(c, Dk - 1);
      xq[it] = ld_f(qc, o);
      xk[it] = ld_f(kc, o);
      xg[it] = f.gain == GDR_GAIN_SCALAR ? bc[tc * H] : ld_f(ec, o);
      xr[it] = ld_f(rsrc, o);
    }
#pragma unroll
    for (int it = 0; it < kLoadIt; ++it) {
      const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
      const bool in = t < n && c < Dk;
      sm.B.Q[t][c] = in ? xq[it] : 0.f;
      sm.B.E[t][c] = in ? xg[it] * xk[it] : 0.f;
      sm.B.R[t][c] = in ? xr[it] : 0.f;
    }
  }
  // the decay factors of the state terms, and the C x C gradients
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = 4 * ti + u;
    const float sq = f.scale * eg[t], se = -eg[t], sr = wd[t];
#pragma unroll
    for (int e = 0; e < CW; ++e) {
      AQ[u][e] *= sq;
      AE[u][e] *= se;
      AR[u][e] *= sr;
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int j = 4 * cj + w;
      // (the exponent above the diagonal may overflow; it is discarded)
      const float dec = expf(gs[t] - gs[j]);
      sm.B.dM[t][j] = (j <= t && t < n) ? f.scale * MP[u][w] * dec : 0.f;
      sm.B.dL[t][j] = (j < t && t < n) ? -ML[u][w] * dec : 0.f;
    }
  }
  __syncthreads();
  // lambda: this thread's share of sum_j r_j . (e^{g_n - g_j} dS'^T d_j)
  float lam = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const float4 rr = ld4(&sm.B.R[4 * ti + u][64 * g + 4 * cj]);
#pragma unroll
      for (int e = 0; e < 4; ++e) lam = fmaf(at(rr, e), AR[u][4 * g + e], lam);
    }
  // dQ += dM R, dE += dL' R
  for (int j = 0; j < n; ++j) {
    float4 rr[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) rr[g] = ld4(&sm.B.R[j][64 * g + 4 * cj]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float m = sm.B.dM[4 * ti + u][j], l = sm.B.dL[4 * ti + u][j];
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          AQ[u][4 * g + e] = fmaf(m, at(rr[g], e), AQ[u][4 * g + e]);
          AE[u][4 * g + e] = fmaf(l, at(rr[g], e), AE[u][4 * g + e]);
        }
    }
  }
  // dR += dM^T Q + dL'^T E
  for (int i = 0; i < n; ++i) {
    const float4 m4 = ld4(&sm.B.dM[i][4 * ti]), l4 = ld4(&sm.B.dL[i][4 * ti]);
    float4 qq[NG], ee[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      qq[g] = ld4(&sm.B.Q[i][64 * g + 4 * cj]);
      ee[g] = ld4(&sm.B.E[i][64 * g + 4 * cj]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float m = at(m4, u), l = at(l4, u);
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          AR[u][4 * g + e] = fmaf(m, at(qq[g], e), fmaf(l, at(ee[g], e), AR[u][4 * g + e]));
    }
  }
  // gate gradient per token: q . dQ + e . dE - r . dR over the thread's channels, summed
  // over the 16 lanes that share the tokens
  float pg[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = 4 * ti + u;
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const float4 qq = ld4(&sm.B.Q[t][64 * g + 4 * cj]), ee = ld4(&sm.B.E[t][64 * g + 4 * cj]);
      const float4 rr = ld4(&sm.B.R[t][64 * g + 4 * cj]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(at(qq, e), AQ[u][4 * g + e], acc);
        acc = fmaf(at(ee, e), AE[u][4 * g + e], acc);
        acc = fmaf(-at(rr, e), AR[u][4 * g + e], acc);
      }
    }
    pg[u] = acc;
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1)
#pragma unroll
    for (int u = 0; u < 4; ++u) pg[u] += __shfl_xor(pg[u], m);
  // block sums of <dS', S> and lambda
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    sdot += __shfl_xor(sdot, m);
    lam += __shfl_xor(lam, m);
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = sdot;
    red[1][tid >> 6] = lam;
  }
  if (cj == 0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) dgs[4 * ti + u] = pg[u];
  }
  __syncthreads();
  if (f.decay == GDR_DECAY_SCALAR && tid < kCMax) {
    // dlog_alpha_t = sum_{i >= t} dg_i inside the chunk
    float x = tid < n ? dgs[tid] : 0.f;
    if (tid == n - 1) {
      float st = 0.f, lt = 0.f;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) {
        st += red[0][w];
        lt += red[1][w];
      }
      x += eg[n - 1] * st + lt;
    }
#pragma unroll
    for (int d = 1; d < kCMax; d <<= 1) {
      const float y = __shfl_down(x, d, kCMax);
      if (tid + d < kCMax) x += y;
    }
    if (tid < n) a.dla[tok(tid)] = x;
  }
  // ---- chain rule to the variant's inputs, stores ------------------------------------
  float pk[4] = {0.f, 0.f, 0.f, 0.f};   // k . dE per token (scalar gain)
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = 4 * ti + u;
    if (t >= n) continue;
    const long long rowk = tok(t) * Dk;
    const float bt = f.gain == GDR_GAIN_SCALAR ? f.beta[tok(t)] : 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 64 * g + 4 * cj + e;
        if (c >= Dk) continue;
        const float de = AE[u][4 * g + e], dr = AR[u][4 * g + e];
        const float kk = ld_f(k, rowk + c);
        a.dq[rowk + c] = AQ[u][4 * g + e];
        float dkv;
        if (f.gain == GDR_GAIN_SCALAR) {
          dkv = bt * de;
          pk[u] = fmaf(kk, de, pk[u]);
        } else {
          dkv = ld_f(er, rowk + c) * de;
          a.derase[rowk + c] = kk * de;
        }
        if (f.wkey == GDR_WKEY_EXPLICIT)
          a.dwk[rowk + c] = dr;
        else
          dkv += dr;
        a.dk[rowk + c] = dkv;
      }
  }
  if (f.gain == GDR_GAIN_SCALAR) {
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
#pragma unroll
      for (int u = 0; u < 4; ++u) pk[u] += __shfl_xor(pk[u], m);
    if (cj == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = 4 * ti + u;
        if (t < n) a.dbeta[tok(t)] = pk[u] + vdx[t];
      }
    }
  }
}

template <typename IO>
hipError_t prep_state_io(const BwdArgs &a, hipStream_t s) {
  if (a.NC == 0) return hipSuccess;
  const dim3 gp(a.NC, a.f.H, a.f.B);
  if (a.f.Dk <= 64)
    hipLaunchKernelGGL((bwd_prep_kernel<IO, 64>), gp, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_prep_kernel<IO, 128>), gp, dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 gs((a.f.Dv + kBV - 1) / kBV, a.f.H, a.f.B);
  if (a.f.Dk <= 32)
    hipLaunchKernelGGL((bwd_state_kernel<IO, 32>), gs, dim3(kThreads), 0, s, a);
  else if (a.f.Dk <= 64)
    hipLaunchKernelGGL((bwd_state_kernel<IO, 64>), gs, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_state_kernel<IO, 128>), gs, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <typename IO>
hipError_t sweep_io(const BwdArgs &a, hipStream_t s) {
  const dim3 grid((a.f.Dv + kSwBV - 1) / kSwBV, a.f.H, a.f.B);
  if (a.f.Dk <= 32)
    hipLaunchKernelGGL((bwd_sweep_kernel<IO, 32>), grid, dim3(kSwThreads), 0, s, a);
  else if (a.f.Dk <= 64)
    hipLaunchKernelGGL((bwd_sweep_kernel<IO, 64>), grid, dim3(kSwThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_sweep_kernel<IO, 128>), grid, dim3(kSwThreads), 0, s, a);
  return hipGetLastError();
}

template <typename IO>
hipError_t chunk_io(const BwdArgs &a, hipStream_t s) {
  if (a.NC == 0) return hipSuccess;
  const dim3 grid(a.NC, a.f.H, a.f.B);
  if (a.f.Dk <= 64)
    hipLaunchKernelGGL((bwd_chunk_kernel<IO, 64>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_chunk_kernel<IO, 128>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prep_state(const BwdArgs &a, int io_dtype, hipStream_t s) {
  return io_dtype == GDR_BF16 ? prep_state_io<uint16_t>(a, s) : prep_state_io<float>(a, s);
}

hipError_t launch_bwd_sweep(const BwdArgs &a, int io_dtype, hipStream_t s) {
  return io_dtype == GDR_BF16 ? sweep_io<uint16_t>(a, s) : sweep_io<float>(a, s);
}

hipError_t launch_bwd_chunk(const BwdArgs &a, int io_dtype, hipStream_t s) {
  return io_dtype == GDR_BF16 ? chunk_io<uint16_t>(a, s) : chunk_io<float>(a, s);
}

}  // namespace gdr
