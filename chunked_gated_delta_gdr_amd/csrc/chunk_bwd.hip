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

// W consecutive floats (W = 2 or 4, aligned to 4 W bytes) into registers
template <int W>
__device__ __forceinline__ void ldw(const float *p, float (&x)[W]) {
  if constexpr (W == 4) {
    const float4 v = ld4(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  } else {
    const float2 v = ld2(p);
    x[0] = v.x; x[1] = v.y;
  }
}

// log alpha of token `lane` of the chunk starting at token row row0 (0 past n or without decay)
__device__ __forceinline__ float chunk_log_alpha(const ChunkArgs &f, long long row0, int n, int lane) {
  return (f.decay == GDR_DECAY_SCALAR && lane < n) ? f.log_alpha[row0 + static_cast<long long>(lane) * f.H] : 0.f;
}

// g (inclusive cumulative sum of log alpha over tokens 0..n-1, flat past n), e^g and
// e^{g_{n-1} - g} of one chunk from lane's log alpha `la`; called by the first wave.
__device__ __forceinline__ void chunk_gates_from(float la, int n, int lane, float *gs, float *eg, float *wd) {
  float g = la;
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

__device__ __forceinline__ void chunk_gates(const ChunkArgs &f, long long row0, int n, int lane,
                                            float *gs, float *eg, float *wd) {
  chunk_gates_from(chunk_log_alpha(f, row0, n, lane), n, lane, gs, eg, wd);
}

// ---------------------------------------------------------------------------------------
// Chunk preparation: one workgroup per (batch, head, chunk), all chunks at once.  Everything
// of a chunk that does not depend on the state: T = (I + L)^-1 and P (C x C, for the sweep),
// W = T (e^g (.) E) (C x Dk) and U = T V' (C x Dv, for the state pass).
// ---------------------------------------------------------------------------------------
constexpr int kPrThreads = 512;

template <typename IO, int DK>
__global__ __launch_bounds__(kPrThreads) void bwd_prep_kernel(BwdArgs a) {
  static_assert(DK == 64 || DK == 128, "32 channel groups of 2 or 4");
  constexpr int kThreads = kPrThreads;
  constexpr int LD = DK + 4;
  constexpr int CW = DK / 32;
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
  // thread (ti, cj): rows 4 ti .. 4 ti + 3 and columns 2 cj, 2 cj + 1 of the C x C products;
  // rows 4 ti .. and columns CW cj .. CW cj + CW - 1 of W and U
  const int ti = tid >> 5, cj = tid & 31;
  // LP[i][j] = exp(g_i - g_j) (X_i . R_j) for j < i (or j <= i), zero elsewhere
  auto gram = [&](const float(*X)[LD], bool incl_diag) {
    float acc[4][2] = {};
    if (2 * cj <= 4 * ti + 3) {
#pragma unroll 4
      for (int c = 0; c < DK; c += 4) {
        float4 x[4], r[2];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = ld4(&X[4 * ti + u][c]);
#pragma unroll
        for (int w = 0; w < 2; ++w) r[w] = ld4(&Rs[2 * cj + w][c]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int w = 0; w < 2; ++w) fma4(acc[u][w], x[u], r[w]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int i = 4 * ti + u, j = 2 * cj + w;
        const bool keep = j < i || (incl_diag && j == i);
        LP[i][j] = keep ? expf(gs[i] - gs[j]) * acc[u][w] : 0.f;
      }
  };
  gram(Es, false);
  __syncthreads();
  tri::inverse_blocks(LP, Tm, Zs, -1, tid, tid < 256);
  gram(Xs, true);
  __syncthreads();
  {   // T and P of the chunk (C x C) for the sweep
    const long long cc = (sh * a.NC + ci) * static_cast<long long>(C * C);
    for (int idx = tid; idx < C * C; idx += kThreads) {
      a.Tw[cc + idx] = Tm[idx / C][idx % C];
      a.Pw[cc + idx] = LP[idx / C][idx % C];
    }
  }
  const int ch0 = CW * cj;
  // acc = T[rows] (Y (.) s) over the thread's columns, with row s of Y scaled by scl(s)
  auto tri_product = [&](const float(*Y)[LD], auto &&scl, float (&acc)[4][CW]) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < CW; ++e) acc[u][e] = 0.f;
    const int send = min(4 * ti + 4, n);
#pragma unroll 4
    for (int s0 = 0; s0 < send; ++s0) {
      float y[CW];
      const float sc = scl(s0);
      ldw<CW>(&Y[s0][ch0], y);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float tv = sc * Tm[4 * ti + u][s0];   // zero above the diagonal
#pragma unroll
        for (int e = 0; e < CW; ++e) acc[u][e] = fmaf(tv, y[e], acc[u][e]);
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
      for (int e = 0; e < CW; ++e)
        if (ch0 + e < Dk) Wc[static_cast<long long>(t) * Dk + ch0 + e] = acc[u][e];
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
      for (int e = 0; e < CW; ++e) {
        const int c = vb + ch0 + e;
        if (c < Dv) a.Uw[tok(t) * Dv + c] = acc[u][e];
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
    // S <- e^{g_n} S + (e^{g_n - g} (.) D)^T R: thread (rows r + RS m for m < NR, columns
    // c .. c + 3); each row of R read from LDS serves all NR rows
    {
      const float gl = eg[n - 1];
      constexpr int NC4 = DK / 4;
      constexpr int NR = (kBV * NC4 + kThreads - 1) / kThreads;
      constexpr int RS = kThreads / NC4;
      const int r = tid / NC4, c = (tid % NC4) * 4;
      if (r < RS && r < kBV) {
        float4 acc[NR];
#pragma unroll
        for (int m = 0; m < NR; ++m) {
          const float4 s = r + RS * m < kBV ? ld4(&Ss[r + RS * m][c]) : make_float4(0.f, 0.f, 0.f, 0.f);
          acc[m] = make_float4(gl * s.x, gl * s.y, gl * s.z, gl * s.w);
        }
        // rows past n hold zeros, so the sum may run to the next multiple of 8
        for (int j0 = 0; j0 < n; j0 += 8) {
#pragma unroll
          for (int j = j0; j < j0 + 8; ++j) {
            const float r0f = ld_f(&Rs[j][c], 0), r1f = ld_f(&Rs[j][c], 1);
            const float r2f = ld_f(&Rs[j][c], 2), r3f = ld_f(&Rs[j][c], 3);
#pragma unroll
            for (int m = 0; m < NR; ++m) {
              const float w = Dl[j][min(r + RS * m, kBV - 1)];
              acc[m].x = fmaf(w, r0f, acc[m].x);
              acc[m].y = fmaf(w, r1f, acc[m].y);
              acc[m].z = fmaf(w, r2f, acc[m].z);
              acc[m].w = fmaf(w, r3f, acc[m].w);
            }
          }
        }
#pragma unroll
        for (int m = 0; m < NR; ++m)
          if (r + RS * m < kBV) *reinterpret_cast<float4 *>(&Ss[r + RS * m][c]) = acc[m];
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
  // Loads of chunk ci into registers (indices clamped into the chunk, masks applied when they
  // are written to LDS): write keys, keys, gains, T, P and dO are loaded one chunk ahead, so
  // they are in flight during the previous chunk's products; the queries, needed only after
  // the first two barriers of a chunk, are loaded at its start.
  constexpr int kCC = kCMax * kCMax / kThreads, kOIt = kCMax * kBV / kThreads;
  float xr[kLoadIt], xk[kLoadIt], xg[kLoadIt], xq[kLoadIt], xt[kCC], xp[kCC], xo[kOIt], xla = 0.f;
  const IO *rbase = (f.wkey == GDR_WKEY_EXPLICIT) ? wk : k;
  auto cload = [&](int ci) {
    const int c0 = ci * C, n = min(C, T - c0);
    const long long row0 = (static_cast<long long>(b) * T + c0) * H + h;
    if (tid < kCMax) xla = chunk_log_alpha(f, row0, n, tid);
    const IO *rsrc = rbase + row0 * Dk, *kc = k + row0 * Dk, *ec = er + row0 * Dk;
    const float *bc = f.beta + row0;
#pragma unroll
    for (int it = 0; it < kLoadIt; ++it) {
      const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
      const int tc = min(t, n - 1), o = tc * H * Dk + min(c, Dk - 1);
      xr[it] = ld_f(rsrc, o);
      xk[it] = ld_f(kc, o);
      xg[it] = f.gain == GDR_GAIN_SCALAR ? bc[tc * H] : ld_f(ec, o);
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
      xo[it] = ld_f(dout, (row0 + static_cast<long long>(t) * H) * Dv + v0 + r);
    }
  };
  if (a.NC > 0) cload(a.NC - 1);

  for (int ci = a.NC - 1; ci >= 0; --ci) {
    const int c0 = ci * C;
    const int n = min(C, T - c0);
    auto tok = [&](int t) -> long long { return (static_cast<long long>(b) * T + c0 + t) * H + h; };
    const long long row0 = tok(0);

    __syncthreads();   // previous chunk done with every buffer
    {
      const IO *qc = q + row0 * Dk;
#pragma unroll
      for (int it = 0; it < kLoadIt; ++it) {
        const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
        xq[it] = ld_f(qc, min(t, n - 1) * H * Dk + min(c, Dk - 1));
      }
    }
    if (tid < kCMax) chunk_gates_from(xla, n, tid, gs, eg, wd);
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
    if (ci > 0) cload(ci - 1);   // in flight during this chunk's products
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
    // dS <- e^{g_n} dS + A^T Q - B^T E: thread (rows r + 8 m for m < NR, columns c .. c + 3);
    // each row of Q and E read from LDS serves all NR rows
    {
      const float gl = eg[n - 1];
      constexpr int NC4 = DK / 4;
      constexpr int NR = (kBV * NC4 + kThreads - 1) / kThreads;   // rows per thread
      constexpr int RS = kThreads / NC4;                          // row step between them
      const int r = tid / NC4, c = (tid % NC4) * 4;
      if (r < RS && r < kBV) {
        float4 acc[NR];
#pragma unroll
        for (int m = 0; m < NR; ++m) {
          const float4 s = r + RS * m < kBV ? ld4(&dS[r + RS * m][c]) : make_float4(0.f, 0.f, 0.f, 0.f);
          acc[m] = make_float4(gl * s.x, gl * s.y, gl * s.z, gl * s.w);
        }
        for (int j0 = 0; j0 < n; j0 += 8) {
#pragma unroll
          for (int j = j0; j < j0 + 8; ++j) {
            const float4 qq = ld4(&Ks[j][c]), ee = ld4(&Es[j][c]);
#pragma unroll
            for (int m = 0; m < NR; ++m) {
              const int rr = min(r + RS * m, kBV - 1);
              const float am = Am[j][rr], bm = Bm[j][rr];
              acc[m].x = fmaf(am, qq.x, fmaf(-bm, ee.x, acc[m].x));
              acc[m].y = fmaf(am, qq.y, fmaf(-bm, ee.y, acc[m].y));
              acc[m].z = fmaf(am, qq.z, fmaf(-bm, ee.z, acc[m].z));
              acc[m].w = fmaf(am, qq.w, fmaf(-bm, ee.w, acc[m].w));
            }
          }
        }
#pragma unroll
        for (int m = 0; m < NR; ++m)
          if (r + RS * m < kBV) *reinterpret_cast<float4 *>(&dS[r + RS * m][c]) = acc[m];
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
// Per-chunk pass: one workgroup of kCkThreads per (batch, head, chunk).  Thread (ti, cj)
// owns tokens 4 ti .. 4 ti + 3 and key channels CW cj .. CW cj + CW - 1 of the C x Dk
// gradients, and the 4 x 2 block (tokens 4 ti.., tokens 2 cj..) of the C x C ones.
// ---------------------------------------------------------------------------------------
constexpr int kCkThreads = 512;

template <typename IO, int DK>
__global__ __launch_bounds__(kCkThreads) void bwd_chunk_kernel(BwdArgs a) {
  static_assert(DK == 64 || DK == 128, "32 channel groups of 2 or 4");
  constexpr int kThreads = kCkThreads;
  constexpr int kWaves = kThreads / 64;
  constexpr int LD = DK + 4;
  constexpr int CW = DK / 32;      // channels per thread
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
  const int ti = tid >> 5, cj = tid & 31;
  const int ch0 = CW * cj;   // the thread's first key channel
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
  __shared__ float red[2][kWaves];

  if (tid < kCMax) chunk_gates(f, row0, n, tid, gs, eg, wd);

  float AQ[4][CW], AE[4][CW], AR[4][CW], MP[4][2], ML[4][2];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int e = 0; e < CW; ++e) AQ[u][e] = AE[u][e] = AR[u][e] = 0.f;
#pragma unroll
    for (int w = 0; w < 2; ++w) MP[u][w] = ML[u][w] = 0.f;
  }
  float sdot = 0.f;   // this thread's share of <dS', S>
  float vsum = 0.f;   // this thread's share of v_t . dX_t (scalar gain), t = tid >> 3
  const float *hc = a.h + (sh * a.NC + ci) * static_cast<long long>(Dv) * Dk;
  const float *dhc = a.dh + (sh * a.NC + ci) * static_cast<long long>(Dv) * Dk;

  // ---- value loop: dO S, dX S, D dS', dO D^T, dX D^T --------------------------------
  // Each block of kVB value rows is loaded into registers one block ahead (indices clamped,
  // masks applied when the registers are written to LDS), so its loads are in flight while
  // the previous block is multiplied.
  constexpr int kSIt = kVB * DK / kThreads;   // state elements per thread and block
  float ps[kSIt], pds[kSIt], po[2], px[2], pd[2], pv[2], pw[2];
  const int lt = tid >> 3, rq = 2 * (tid & 7);   // token-tile element (token lt, rows rq, rq + 1)
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
    for (int u = 0; u < 2; ++u) {
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
    for (int u = 0; u < 2; ++u) {
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
#pragma unroll 2
    for (int r = 0; r < nvb; ++r) {
      const float4 o4 = ld4(&sm.A.dOT[r][4 * ti]), x4 = ld4(&sm.A.dXT[r][4 * ti]);
      const float4 d4 = ld4(&sm.A.DT[r][4 * ti]);
      const float2 dj = ld2(&sm.A.DT[r][2 * cj]);
      float s[CW], ds[CW];
      ldw<CW>(&sm.A.S[r][ch0], s);
      ldw<CW>(&sm.A.dS[r][ch0], ds);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float ou = at(o4, u), xu = at(x4, u), du = at(d4, u);
        MP[u][0] = fmaf(ou, dj.x, MP[u][0]);
        MP[u][1] = fmaf(ou, dj.y, MP[u][1]);
        ML[u][0] = fmaf(xu, dj.x, ML[u][0]);
        ML[u][1] = fmaf(xu, dj.y, ML[u][1]);
#pragma unroll
        for (int e = 0; e < CW; ++e) {
          AQ[u][e] = fmaf(ou, s[e], AQ[u][e]);
          AE[u][e] = fmaf(xu, s[e], AE[u][e]);
          AR[u][e] = fmaf(du, ds[e], AR[u][e]);
        }
      }
    }
  }
  vsum += __shfl_xor(vsum, 1);
  vsum += __shfl_xor(vsum, 2);
  vsum += __shfl_xor(vsum, 4);
  if ((tid & 7) == 0) vdx[lt] = vsum;

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
    for (int w = 0; w < 2; ++w) {
      const int j = 2 * cj + w;
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
  for (int u = 0; u < 4; ++u) {
    float rr[CW];
    ldw<CW>(&sm.B.R[4 * ti + u][ch0], rr);
#pragma unroll
    for (int e = 0; e < CW; ++e) lam = fmaf(rr[e], AR[u][e], lam);
  }
  // dQ += dM R, dE += dL' R (rows past n of dM and dL' are zero: whole blocks of 8)
  for (int j0 = 0; j0 < n; j0 += 8) {
#pragma unroll
    for (int j = j0; j < j0 + 8; ++j) {
      float rr[CW];
      ldw<CW>(&sm.B.R[j][ch0], rr);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float m = sm.B.dM[4 * ti + u][j], l = sm.B.dL[4 * ti + u][j];
#pragma unroll
        for (int e = 0; e < CW; ++e) {
          AQ[u][e] = fmaf(m, rr[e], AQ[u][e]);
          AE[u][e] = fmaf(l, rr[e], AE[u][e]);
        }
      }
    }
  }
  // dR += dM^T Q + dL'^T E
  for (int i0 = 0; i0 < n; i0 += 8) {
#pragma unroll
    for (int i = i0; i < i0 + 8; ++i) {
      const float4 m4 = ld4(&sm.B.dM[i][4 * ti]), l4 = ld4(&sm.B.dL[i][4 * ti]);
      float qq[CW], ee[CW];
      ldw<CW>(&sm.B.Q[i][ch0], qq);
      ldw<CW>(&sm.B.E[i][ch0], ee);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float m = at(m4, u), l = at(l4, u);
#pragma unroll
        for (int e = 0; e < CW; ++e) AR[u][e] = fmaf(m, qq[e], fmaf(l, ee[e], AR[u][e]));
      }
    }
  }
  // gate gradient per token: q . dQ + e . dE - r . dR over the thread's channels, summed
  // over the 32 lanes that share the tokens
  float pg[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = 4 * ti + u;
    float qq[CW], ee[CW], rr[CW];
    ldw<CW>(&sm.B.Q[t][ch0], qq);
    ldw<CW>(&sm.B.E[t][ch0], ee);
    ldw<CW>(&sm.B.R[t][ch0], rr);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < CW; ++e) {
      acc = fmaf(qq[e], AQ[u][e], acc);
      acc = fmaf(ee[e], AE[u][e], acc);
      acc = fmaf(-rr[e], AR[u][e], acc);
    }
    pg[u] = acc;
  }
#pragma unroll
  for (int m = 1; m < 32; m <<= 1)
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
      float st = 0.f, lt2 = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        st += red[0][w];
        lt2 += red[1][w];
      }
      x += eg[n - 1] * st + lt2;
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
    for (int e = 0; e < CW; ++e) {
      const int c = ch0 + e;
      if (c >= Dk) continue;
      const float de = AE[u][e], dr = AR[u][e];
      const float kk = ld_f(k, rowk + c);
      a.dq[rowk + c] = AQ[u][e];
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
    for (int m = 1; m < 32; m <<= 1)
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
    hipLaunchKernelGGL((bwd_prep_kernel<IO, 64>), gp, dim3(kPrThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_prep_kernel<IO, 128>), gp, dim3(kPrThreads), 0, s, a);
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
    hipLaunchKernelGGL((bwd_chunk_kernel<IO, 64>), grid, dim3(kCkThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_chunk_kernel<IO, 128>), grid, dim3(kCkThreads), 0, s, a);
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
