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
// Two kernels: the reverse sweep (sequential over chunks, per value tile; carries dS and
// emits dX and the gradient at each chunk's end) and the per-chunk pass (parallel over
// chunks; everything else).  The forward recompute that saves S at each chunk start, D, T
// and P is the generic forward kernel.
#include "common.h"

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
// Reverse sweep: one workgroup per (batch, head, tile of kBV value rows), chunks last to
// first.  dS (kBV x Dk) stays in LDS.
// ---------------------------------------------------------------------------------------
template <typename IO, int DK>
__global__ __launch_bounds__(kThreads) void bwd_sweep_kernel(BwdArgs a) {
  constexpr int LD = DK + 4;
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
  const int t0 = 2 * (tid >> 3), r0 = 2 * (tid & 7);

  for (int ci = a.NC - 1; ci >= 0; --ci) {
    const int c0 = ci * C;
    const int n = min(C, T - c0);
    auto tok = [&](int t) -> long long { return (static_cast<long long>(b) * T + c0 + t) * H + h; };
    const long long row0 = tok(0);
    const int rstride = H * Dk;
    // rows 0..n-1 of a [B, T, H, Dk] tile into dst, zero beyond n and Dk (clamped loads, then
    // the mask)
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

    __syncthreads();   // previous chunk done with every buffer
    {   // the gradient at this chunk's end, for the per-chunk pass
      float *dhc = a.dh + ((sh * a.NC + ci) * Dv + v0) * static_cast<long long>(Dk);
      for (int idx = tid; idx < nv * Dk; idx += kThreads) dhc[idx] = dS[idx / Dk][idx % Dk];
    }
    const IO *kc = k + row0 * Dk;
    {
      const IO *src = ((f.wkey == GDR_WKEY_EXPLICIT) ? wk : k) + row0 * Dk;
      stage(Ks, [&](int, int o) { return ld_f(src, o); });
    }
    if (f.gain == GDR_GAIN_SCALAR) {
      const float *bc = f.beta + row0;
      stage(Es, [&](int t, int o) { return bc[t * H] * ld_f(kc, o); });
    } else {
      const IO *ec = er + row0 * Dk;
      stage(Es, [&](int, int o) { return ld_f(ec, o) * ld_f(kc, o); });
    }
    {
      const long long cc = (sh * a.NC + ci) * static_cast<long long>(C * C);
      for (int idx = tid; idx < C * C; idx += kThreads) {
        Tm[idx / C][idx % C] = a.Tw[cc + idx];
        Pm[idx / C][idx % C] = a.Pw[cc + idx];
      }
    }
    for (int idx = tid; idx < kCMax * kBV; idx += kThreads) {
      const int t = idx / kBV, r = idx % kBV;
      dOs[t][r] = (t < n && r < nv) ? ld_f(dout, tok(t) * Dv + v0 + r) : 0.f;
    }
    if (tid < kCMax) chunk_gates(f, row0, n, tid, gs, eg, wd);
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
      // P is zero above the diagonal, so row t0 + 1 may start at i = t0 too
      for (int i = t0; i < n; ++i) {
        const float2 o = ld2(&dOs[i][r0]);
        const float p0 = Pm[i][t0], p1 = Pm[i][t0 + 1];
        p[0][0] = fmaf(p0, o.x, p[0][0]);
        p[0][1] = fmaf(p0, o.y, p[0][1]);
        p[1][0] = fmaf(p1, o.x, p[1][0]);
        p[1][1] = fmaf(p1, o.y, p[1][1]);
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
      for (int i = t0; i < n; ++i) {
        const float2 d = ld2(&dDs[i][r0]);
        const float a0 = Tm[i][t0], a1 = Tm[i][t0 + 1];
        x[0][0] = fmaf(a0, d.x, x[0][0]);
        x[0][1] = fmaf(a0, d.y, x[0][1]);
        x[1][0] = fmaf(a1, d.x, x[1][0]);
        x[1][1] = fmaf(a1, d.y, x[1][1]);
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
    {
      const IO *qc = q + row0 * Dk;
      stage(Ks, [&](int, int o) { return ld_f(qc, o); });
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
        for (int j = 0; j < n; ++j) {
          const float am = Am[j][r], bm = Bm[j][r];
          const float4 qq = ld4(&Ks[j][c]), ee = ld4(&Es[j][c]);
          acc.x = fmaf(am, qq.x, fmaf(-bm, ee.x, acc.x));
          acc.y = fmaf(am, qq.y, fmaf(-bm, ee.y, acc.y));
          acc.z = fmaf(am, qq.z, fmaf(-bm, ee.z, acc.z));
          acc.w = fmaf(am, qq.w, fmaf(-bm, ee.w, acc.w));
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
  for (int vb = 0; vb < Dv; vb += kVB) {
    const int nvb = min(kVB, Dv - vb);
    __syncthreads();   // previous tiles consumed
    for (int idx = tid; idx < kVB * DK; idx += kThreads) {
      const int r = idx / DK, c = idx % DK;
      float s = 0.f, ds = 0.f;
      if (r < nvb && c < Dk) {
        s = hc[static_cast<long long>(vb + r) * Dk + c];
        ds = dhc[static_cast<long long>(vb + r) * Dk + c];
      }
      sm.A.S[r][c] = s;
      sm.A.dS[r][c] = ds;
      sdot = fmaf(s, ds, sdot);
    }
    {   // thread = (token t, value rows rq .. rq + 3); dv (and dwrite) are elementwise in dX
      const int t = tid >> 2, rq = 4 * (tid & 3);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = rq + u;
        float go = 0.f, gx = 0.f, dd = 0.f;
        if (t < n && r < nvb) {
          const long long idx = tok(t) * Dv + vb + r;
          go = ld_f(dout, idx);
          gx = a.dX[idx];
          dd = a.D[idx];
          const float vv = ld_f(v, idx);
          if (f.gain == GDR_GAIN_SCALAR) {
            a.dv[idx] = f.beta[tok(t)] * gx;
            vsum = fmaf(vv, gx, vsum);
          } else {
            a.dv[idx] = ld_f(wr, idx) * gx;
            a.dwrite[idx] = vv * gx;
          }
        }
        sm.A.dOT[r][t] = go;
        sm.A.dXT[r][t] = gx;
        sm.A.DT[r][t] = dd;
      }
    }
    __syncthreads();
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
  auto stage = [&](float(*dst)[LD], auto &&load) {
    float x[kLoadIt];
#pragma unroll
    for (int it = 0; it < kLoadIt; ++it) {
      const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
      const int tc = min(t, n - 1), cc = min(c, Dk - 1);
      x[it] = load(tc, tc * H * Dk + cc);
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
  const IO *kc = k + row0 * Dk;
  stage(sm.B.Q, [&](int, int o) { return ld_f(q + row0 * Dk, o); });
  if (f.gain == GDR_GAIN_SCALAR) {
    const float *bc = f.beta + row0;
    stage(sm.B.E, [&](int t, int o) { return bc[t * H] * ld_f(kc, o); });
  } else {
    const IO *ec = er + row0 * Dk;
    stage(sm.B.E, [&](int, int o) { return ld_f(ec, o) * ld_f(kc, o); });
  }
  {
    const IO *src = ((f.wkey == GDR_WKEY_EXPLICIT) ? wk : k) + row0 * Dk;
    stage(sm.B.R, [&](int, int o) { return ld_f(src, o); });
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
hipError_t sweep_io(const BwdArgs &a, hipStream_t s) {
  const dim3 grid((a.f.Dv + kBV - 1) / kBV, a.f.H, a.f.B);
  if (a.f.Dk <= 32)
    hipLaunchKernelGGL((bwd_sweep_kernel<IO, 32>), grid, dim3(kThreads), 0, s, a);
  else if (a.f.Dk <= 64)
    hipLaunchKernelGGL((bwd_sweep_kernel<IO, 64>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_sweep_kernel<IO, 128>), grid, dim3(kThreads), 0, s, a);
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

hipError_t launch_bwd_sweep(const BwdArgs &a, int io_dtype, hipStream_t s) {
  return io_dtype == GDR_BF16 ? sweep_io<uint16_t>(a, s) : sweep_io<float>(a, s);
}

hipError_t launch_bwd_chunk(const BwdArgs &a, int io_dtype, hipStream_t s) {
  return io_dtype == GDR_BF16 ? chunk_io<uint16_t>(a, s) : chunk_io<float>(a, s);
}

}  // namespace gdr
