// Backward pass of the chunked gated delta rule: fp32 arithmetic, products on the matrix cores.
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
// per-chunk pass (parallel over chunks; everything else).  Variants, each a compile-time
// flag of the kernels it touches: the per-channel decay (CHD), the preconditioned write key
// (PC: two scans per channel before and after the four kernels) and the band-limited T
// (BAND: dL = -T^T (M (.) dD X^T) T^T in place of -dX D^T).
#include <type_traits>

#include "common.h"
#include "tri_blocks.h"
#include "chd_gram.h"

namespace gdr {
namespace {

// XCD-aware order of a (value tile, head, batch) grid: workgroups are dealt to the 8 XCDs in
// turn, so consecutive logical tiles (the value tiles of one head, which read the same keys
// and gates) get ids 8 apart and share an XCD's L2
// (indices in 64 bits: the grid may hold up to 2^24 workgroups, and the host bounds it)
__device__ __forceinline__ void xcd_tile(int &vt, int &h, int &b) {
  const uint64_t nvt = gridDim.x, nh = gridDim.y;
  const uint64_t G = nvt * nh * gridDim.z;
  const uint64_t bid = blockIdx.x + nvt * (blockIdx.y + nh * static_cast<uint64_t>(blockIdx.z));
  const uint64_t logical = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  vt = static_cast<int>(logical % nvt);
  h = static_cast<int>((logical / nvt) % nh);
  b = static_cast<int>(logical / nvt / nh);
}

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

// fp32 matrix-core product D = A B + C of 16 x 16 x 4 tiles: lane l gives A[l % 16][l / 16] and
// B[l / 16][l % 16] and holds D[4 (l / 16) + r][l % 16], r < 4 (v_mfma_f32_16x16x4_f32)
typedef float float4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4v mfma4(float a, float b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
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

// four consecutive elements of an io (bf16 or fp32) or fp32 array, at an index that is a multiple
// of four from a 16-byte aligned base: one 8- or 16-byte load instead of four
__device__ __forceinline__ void ld4e(const float *p, long long i, float *x) {
  const float4 v = *reinterpret_cast<const float4 *>(p + i);
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
__device__ __forceinline__ void ld4e(const uint16_t *p, long long i, float *x) {
  const uint2 v = *reinterpret_cast<const uint2 *>(p + i);
  x[0] = bf16_bits_to_f32(v.x & 0xffffu); x[1] = bf16_bits_to_f32(v.x >> 16);
  x[2] = bf16_bits_to_f32(v.y & 0xffffu); x[3] = bf16_bits_to_f32(v.y >> 16);
}

// W consecutive floats to LDS: one 16-byte write for W = 4 (p 16-byte aligned), else one write
template <int W>
__device__ __forceinline__ void st_row(float *p, const float *x) {
  if constexpr (W == 4)
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
  else
    p[0] = x[0];
}

// log alpha of token `lane` of the chunk starting at token row row0 (0 past n or without decay)
__device__ __forceinline__ float chunk_log_alpha(const ChunkArgs &f, long long row0, int n, int lane) {
  return (f.decay == GDR_DECAY_SCALAR && lane < n) ? f.log_alpha[row0 + static_cast<long long>(lane) * f.H] : 0.f;
}

// the write key at offset o (token row, channel) of the chunk whose first element is row0k:
// the formed preconditioned key (fp32) with the preconditioner (PC), else k or the explicit
// write key (chosen at compile time: a load inside a run-time branch would have to complete
// before the branch ends)
template <bool PC, typename IO>
__device__ __forceinline__ float ld_wkey(const BwdArgs &a, const IO *rbase, long long row0k, long long o) {
  if constexpr (PC)
    return a.Rk[row0k + o];
  else
    return ld_f(rbase + row0k, o);
}

// the same four at once (ld4e)
template <bool PC, typename IO>
__device__ __forceinline__ void ld_wkey4(const BwdArgs &a, const IO *rbase, long long row0k, long long o, float *x) {
  if constexpr (PC)
    ld4e(a.Rk + row0k, o, x);
  else
    ld4e(rbase + row0k, o, x);
}

// tile u < 10 of the ten 16 x 16 tiles on and below the diagonal of a 64 x 64 matrix
__device__ __forceinline__ void lower_tile10(int u, int &ib, int &jb) {
  ib = u < 1 ? 0 : u < 3 ? 1 : u < 6 ? 2 : 3;
  jb = u - ib * (ib + 1) / 2;
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
// W = T (e^g (.) E) (C x Dk) and U = T V' (C x Dv, for the state pass).  With per-channel
// decay (CHD) also G, the in-chunk cumulative log2 decay of every token and channel, for the
// other three kernels; the Gram tiles take the decay inside their channel sums, W the factor
// 2^G elementwise.
// ---------------------------------------------------------------------------------------
constexpr int kPrThreads = 512;

template <typename IO, int DK, bool CHD, bool PC>
__global__ __launch_bounds__(kPrThreads) void bwd_prep_kernel(BwdArgs a) {
  static_assert(DK == 64 || DK == 128, "32 channel groups of 2 or 4");
  constexpr int kThreads = kPrThreads;
  constexpr int LD = DK + 4;
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
  __shared__ __align__(16) float Xs[kCMax][LD];   // queries (CHD: G), then blocks of V'
  __shared__ float LP[kCMax][kCMax + 1];          // L, then P
  __shared__ __align__(16) float Tm[kCMax][kCMax + 4];
  __shared__ __align__(16) float Zs[32][36];
  __shared__ float gs[kCMax], eg[kCMax], wd[kCMax];

  if (tid < kCMax) chunk_gates(f, row0, n, tid, gs, eg, wd);
  for (int idx = tid; idx < kCMax * kCMax; idx += kThreads) {
    const int i = idx / kCMax, j = idx % kCMax;
    if ((j >> 4) > (i >> 4)) Tm[i][j] = 0.f;
  }
  const IO *qc = q + row0 * Dk;
  {   // E, R, Q (CHD: log alpha): all loads first (clamped), then the masked stores; the keys
      // once when the write key is the key, a scalar gain once per token (lane t of every
      // wave holds token t's, handed to the staged elements by a lane shuffle).  One copy of
      // the loads and stores per case, so that no branch separates the loads (all in flight
      // at once) and no register array is merged across cases.
    const IO *kc = k + row0 * Dk, *ec = er + row0 * Dk;
    const IO *rbase = (f.wkey == GDR_WKEY_EXPLICIT) ? wk : k;
    const int lane = tid & 63;
    auto stage = [&](auto same, auto scalar) __attribute__((always_inline)) {
      constexpr bool kSame = decltype(same)::value, kScalar = decltype(scalar)::value;
      float xk[kLoadIt], xg[kScalar ? 1 : kLoadIt], xr[kSame ? 1 : kLoadIt], xq[kLoadIt];
      const float bl = kScalar ? f.beta[row0 + static_cast<long long>(min(lane, n - 1)) * H] : 0.f;
#pragma unroll
      for (int it = 0; it < kLoadIt; ++it) {
        const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
        const int tc = min(t, n - 1), o = tc * H * Dk + min(c, Dk - 1);
        xk[it] = ld_f(kc, o);
        if constexpr (!kScalar) xg[it] = ld_f(ec, o);
        if constexpr (!kSame) xr[it] = ld_wkey<PC>(a, rbase, row0 * Dk, o);
        xq[it] = CHD ? f.log_alpha[row0 * Dk + o] : ld_f(qc, o);
      }
#pragma unroll
      for (int it = 0; it < kLoadIt; ++it) {
        const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
        const bool in = t < n && c < Dk;
        float g;
        if constexpr (kScalar)
          g = __shfl(bl, t);   // (t < kCMax = 64: a lane of this wave)
        else
          g = xg[it];
        Es[t][c] = in ? g * xk[it] : 0.f;
        if constexpr (kSame)
          Rs[t][c] = in ? xk[it] : 0.f;
        else
          Rs[t][c] = in ? xr[it] : 0.f;
        Xs[t][c] = in ? xq[it] : 0.f;
      }
    };
    const bool rk_same = !PC && f.wkey != GDR_WKEY_EXPLICIT, gsc = f.gain == GDR_GAIN_SCALAR;
    if (rk_same) {
      if (gsc) stage(std::true_type{}, std::true_type{});
      else stage(std::true_type{}, std::false_type{});
    } else {
      if (gsc) stage(std::false_type{}, std::true_type{});
      else stage(std::false_type{}, std::false_type{});
    }
  }
  __syncthreads();
  if constexpr (CHD) {
    // G: cumulative sum of log2 alpha over the chunk per channel (zero past n: flat there),
    // in place of the log alphas, and to the workspace for the other kernels
    if (tid < DK) {   // (all reads first, so they are in flight together)
      float gv[kCMax];
#pragma unroll
      for (int t = 0; t < kCMax; ++t) gv[t] = Xs[t][tid];
      float g = 0.f;
      float *Gc = a.Gw + (sh * a.NC + ci) * static_cast<long long>(C) * Dk;
#pragma unroll
      for (int t = 0; t < kCMax; ++t) {
        g = fmaf(gv[t], kLog2e, g);
        Xs[t][tid] = g;
        if (t < n && tid < Dk) Gc[static_cast<long long>(t) * Dk + tid] = g;
      }
    }
    __syncthreads();
  }
  // fp32 MFMA tiles (lane layout as for mfma4): wave w, lane (col, kq)
  const int wave = tid >> 6, lane = tid & 63, col = lane & 15, kq = lane >> 4;
  // LP[i][j] = exp(g_i - g_j) (X_i . R_j) on the 10 tiles on and below the diagonal (j < i,
  // or j <= i), tile u = wave and wave + 8; the tiles above are never read
  auto gram = [&](const float(*X)[LD], bool incl_diag) {
    for (int u = wave; u < 10; u += 8) {
      const int ib = u < 1 ? 0 : u < 3 ? 1 : u < 6 ? 2 : 3;
      const int jb = u - ib * (ib + 1) / 2;
      const float4v acc = dot_kc<DK>(&X[16 * ib + col][0], &Rs[16 * jb + col][0], kq);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ib + 4 * kq + r, j = 16 * jb + col;
        const bool keep = j < i || (incl_diag && j == i);
        LP[i][j] = keep ? expf(gs[i] - gs[j]) * acc[r] : 0.f;
      }
    }
  };
  if constexpr (CHD)
    chd::gram<DK, LD>(Es, Rs, Xs, LP, false, tid);
  else
    gram(Es, false);
  __syncthreads();
  tri::inverse_blocks(LP, Tm, Zs, -1, tid);
  // T (Y (.) scl) on the tiles (token block ib = wave % 4, channel blocks MT (wave / 4) + m):
  // T is lower triangular, so the sum over tokens s ends with block ib
  constexpr int MT = DK / 32;
  const int ib = wave & 3, cb0 = MT * (wave >> 2);
  auto tri_product = [&](const float(*Y)[LD], auto &&scl, float4v (&acc)[MT]) {
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = float4v{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < 16 * (ib + 1); s0 += 4) {
      // (band-limited T: the band of the inverse, T_b, the forward's T)
      const float at_ = (f.N < 0 || 16 * ib + col - (s0 + kq) <= f.N) ? Tm[16 * ib + col][s0 + kq] : 0.f;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int c = 16 * (cb0 + m) + col;
        acc[m] = mfma4(at_, scl(s0 + kq, c) * Y[s0 + kq][c], acc[m]);
      }
    }
  };
  auto store_w = [&]() {   // W = T (e^g (.) E), [B, H, NC, C, Dk]
    float4v acc[MT];
    if constexpr (CHD)
      tri_product(Es, [&](int s, int c) { return chd::ex2(Xs[s][c]); }, acc);
    else
      tri_product(Es, [&](int s, int) { return eg[s]; }, acc);
    float *Wc = a.Ww + (sh * a.NC + ci) * static_cast<long long>(C) * Dk;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int c = 16 * (cb0 + m) + col;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * ib + 4 * kq + r;
        if (t < n && c < Dk) Wc[static_cast<long long>(t) * Dk + c] = acc[m][r];
      }
    }
  };
  if constexpr (CHD) {
    // W before P: the queries then take the erase keys' place (G stays in Xs for P)
    store_w();
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kLoadIt; ++it) {
      const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
      const float x = ld_f(qc, min(t, n - 1) * H * Dk + min(c, Dk - 1));
      Es[t][c] = (t < n && c < Dk) ? x : 0.f;
    }
    __syncthreads();
    chd::gram<DK, LD>(Es, Rs, Xs, LP, true, tid);
  } else {
    gram(Xs, true);
  }
  __syncthreads();
  {   // T and P of the chunk (C x C) for the sweep (P is zero above the diagonal)
    const long long cc = (sh * a.NC + ci) * static_cast<long long>(C * C);
    for (int idx = tid; idx < C * C; idx += kThreads) {
      const int i = idx / C, j = idx % C;
      a.Tw[cc + idx] = (f.N < 0 || i - j <= f.N) ? Tm[i][j] : 0.f;   // T_b with a band
      if (f.N >= 0) a.Tfw[cc + idx] = Tm[i][j];                       // and the whole inverse
      a.Pw[cc + idx] = j <= i ? LP[i][j] : 0.f;
    }
  }
  if constexpr (!CHD) store_w();
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
    float4v acc[MT];
    tri_product(Xs, [&](int, int) { return 1.f; }, acc);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int c = vb + 16 * (cb0 + m) + col;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * ib + 4 * kq + r;
        if (t < n && c < Dv) a.Uw[tok(t) * Dv + c] = acc[m][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// State pass: one workgroup of kStThreads (8 waves) per (batch, head, tile of kStBV value
// rows), chunks first to last, on the fp32 matrix cores.  With W and U of every chunk at
// hand only the state-dependent part remains: D = U - W S^T (saved) and
// S <- e^{g_n} S + (e^{g_n - g} (.) D)^T R; the state at every chunk start is saved too.  S
// lives in the waves' accumulators (16 x 16 tiles), mirrored in LDS for D's product; wave w
// owns the tile (token block w % 4, value-row block w / 4) of D.  The next chunk's W, R and U
// are loaded during this chunk.  With per-channel decay (CHD) the update is
// S <- S Diag(2^G_n) + D^T (2^(G_n - G) (.) R): the write keys are decayed elementwise as
// they are staged and the state's columns scaled.
// ---------------------------------------------------------------------------------------
constexpr int kStBV = 32;
constexpr int kStThreads = 512;

template <typename IO, int DK, bool CHD, bool PC, bool V4, int BVT>
__global__ __launch_bounds__(kStThreads) void bwd_state_kernel(BwdArgs a) {
  // V4: four consecutive elements per load and per LDS write, as in the reverse sweep
  constexpr int LD = DK + 4;
  constexpr int kBV = BVT, kThreads = kStThreads;   // value rows per workgroup: 32, or 16
  constexpr int kLoadIt = kCMax * DK / kThreads;
  constexpr int kUIt = kCMax * kBV / kThreads;
  constexpr int NCB = DK / 16;
  constexpr int NTS = (kBV / 16) * NCB;
  constexpr int NTW = (NTS + 7) / 8;
  const ChunkArgs &f = a.f;
  const IO *__restrict__ k = static_cast<const IO *>(f.k);
  const IO *__restrict__ wk = static_cast<const IO *>(f.write_key);

  const int tid = threadIdx.x;
  int vt, h, b;
  xcd_tile(vt, h, b);
  const int v0 = vt * kBV;
  const int nv = min(kBV, f.Dv - v0);
  const int Dk = f.Dk, Dv = f.Dv, H = f.H, T = f.T, C = f.C;
  const long long sh = static_cast<long long>(b) * H + h;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 15, kq = lane >> 4;
  const int tb = wave & 3, rb = wave >> 2;

  __shared__ __align__(16) float Ws[kCMax][LD];   // W of the chunk
  __shared__ __align__(16) float Rs[kCMax][LD];   // write keys (CHD: decayed)
  __shared__ __align__(16) float Ss[kBV][LD];     // mirror of the state
  __shared__ __align__(16) float Dl[kCMax][kBV + 4];  // e^{g_n - g} D (rows padded as in the sweep)
  __shared__ __align__(16) float Us[kCMax][kBV];  // U
  __shared__ float gs[kCMax], eg[kCMax], wd[kCMax];
  __shared__ float gcn[CHD ? DK : 1];            // CHD: 2^G_n per channel

  float4v Sacc[NTW];
#pragma unroll
  for (int m = 0; m < NTW; ++m) {
    const int u = wave + 8 * m;
    const int row = 16 * (u / NCB) + 4 * kq, c = 16 * (u % NCB) + col;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = 0.f;
      if (u < NTS && f.state_in != nullptr && row + r < nv && c < Dk)
        x = f.state_in[(sh * Dv + v0 + row + r) * Dk + c];
      Sacc[m][r] = x;
    }
  }
  for (int idx = tid; idx < kBV * LD; idx += kThreads) {
    const int r = idx / LD, c = idx % LD;
    float s = 0.f;
    if (f.state_in != nullptr && r < nv && c < Dk) s = f.state_in[(sh * Dv + v0 + r) * Dk + c];
    Ss[r][c] = s;
  }
  const IO *rbase = (f.wkey == GDR_WKEY_EXPLICIT) ? wk : k;
  constexpr int STEP = V4 ? 4 : 1;   // elements per load
  // (the U tile in fours only when every thread has whole groups of four: kBV = 32)
  constexpr bool V4U = V4 && kUIt % 4 == 0;
  constexpr int STEPU = V4U ? 4 : 1;
  static_assert(!V4 || (kLoadIt % 4 == 0 && DK % 4 == 0), "V4 loads take whole groups of four");
  float pw[kLoadIt], pu[kUIt], pr[kLoadIt];
  // CHD: G of the staged elements, G_n of the thread's channels (the same in every item:
  // kThreads is a multiple of DK; V4: the four channels 4 (tid mod DK/4) + j)
  float pg[CHD ? kLoadIt : 1], pgn[STEP] = {};
  // element `it` of this thread in a chunk's [C][DK] tile and in a [C][kBV] value tile
  auto elem_tc = [&](int it, int &t, int &c) __attribute__((always_inline)) {
    if constexpr (V4) {
      const int iv = tid + (it >> 2) * kThreads;
      t = iv / (DK / 4);
      c = 4 * (iv % (DK / 4)) + (it & 3);
    } else {
      const int idx = tid + it * kThreads;
      t = idx / DK;
      c = idx % DK;
    }
  };
  auto elem_tr = [&](int it, int &t, int &r) __attribute__((always_inline)) {
    if constexpr (V4U) {
      const int iv = tid + (it >> 2) * kThreads;
      t = iv / (kBV / 4);
      r = 4 * (iv % (kBV / 4)) + (it & 3);
    } else {
      const int idx = tid + it * kThreads;
      t = idx / kBV;
      r = idx % kBV;
    }
  };
  // loads of chunk ci into registers (indices clamped into the chunk)
  auto cload = [&](int ci) {
    const int c0 = ci * C, n = min(C, T - c0);
    const long long row0 = (static_cast<long long>(b) * T + c0) * H + h;
    const float *Wc = a.Ww + (sh * a.NC + ci) * static_cast<long long>(C) * Dk;
#pragma unroll
    for (int it = 0; it < kLoadIt; it += STEP) {
      int t, c;
      elem_tc(it, t, c);
      t = min(t, n - 1);
      if constexpr (V4) {
        c = min(c, Dk - 4);
        ld4e(Wc, static_cast<long long>(t) * Dk + c, &pw[it]);
        ld_wkey4<PC>(a, rbase, row0 * Dk, static_cast<long long>(t) * H * Dk + c, &pr[it]);
      } else {
        c = min(c, Dk - 1);
        pw[it] = Wc[static_cast<long long>(t) * Dk + c];
        pr[it] = ld_wkey<PC>(a, rbase, row0 * Dk, static_cast<long long>(t) * H * Dk + c);
      }
    }
    if constexpr (CHD) {
      const float *Gc = a.Gw + (sh * a.NC + ci) * static_cast<long long>(C) * Dk;
#pragma unroll
      for (int it = 0; it < kLoadIt; it += STEP) {
        int t, c;
        elem_tc(it, t, c);
        t = min(t, n - 1);
        if constexpr (V4)
          ld4e(Gc, static_cast<long long>(t) * Dk + min(c, Dk - 4), &pg[it]);
        else
          pg[it] = Gc[static_cast<long long>(t) * Dk + min(c, Dk - 1)];
      }
      if constexpr (V4)
        ld4e(Gc, static_cast<long long>(n - 1) * Dk + min(4 * (tid % (DK / 4)), Dk - 4), pgn);
      else
        pgn[0] = Gc[static_cast<long long>(n - 1) * Dk + min(tid % DK, Dk - 1)];
    }
#pragma unroll
    for (int it = 0; it < kUIt; it += STEPU) {
      int t, r;
      elem_tr(it, t, r);
      t = min(t, n - 1);
      if constexpr (V4U)
        ld4e(a.Uw, (row0 + static_cast<long long>(t) * H) * Dv + v0 + min(r, nv - 4), &pu[it]);
      else
        pu[it] = a.Uw[(row0 + static_cast<long long>(t) * H) * Dv + v0 + min(r, nv - 1)];
    }
  };
  if (a.NC > 0) cload(0);
  for (int ci = 0; ci < a.NC; ++ci) {
    const int c0 = ci * C;
    const int n = min(C, T - c0);
    auto tok = [&](int t) -> long long { return (static_cast<long long>(b) * T + c0 + t) * H + h; };
    __syncthreads();   // previous chunk done with every buffer
    {   // the state at this chunk's start (from the accumulators)
      float *hc = a.h + ((sh * a.NC + ci) * Dv + v0) * static_cast<long long>(Dk);
#pragma unroll
      for (int m = 0; m < NTW; ++m) {
        const int u = wave + 8 * m;
        const int row = 16 * (u / NCB) + 4 * kq, c = 16 * (u % NCB) + col;
        if (u < NTS && c < Dk) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (row + r < nv) hc[static_cast<long long>(row + r) * Dk + c] = Sacc[m][r];
        }
      }
    }
#pragma unroll
    for (int it = 0; it < kLoadIt; it += STEP) {
      int t, c;
      elem_tc(it, t, c);
      const bool in = t < n && c < Dk;
      float w4[STEP], r4[STEP];
#pragma unroll
      for (int j = 0; j < STEP; ++j) {
        w4[j] = in ? pw[it + j] : 0.f;
        if constexpr (CHD)
          r4[j] = in ? pr[it + j] * chd::ex2(pgn[j] - pg[it + j]) : 0.f;
        else
          r4[j] = in ? pr[it + j] : 0.f;
      }
      st_row<STEP>(&Ws[t][c], w4);
      st_row<STEP>(&Rs[t][c], r4);
    }
    if constexpr (CHD) {
      if constexpr (V4) {
        if (tid < DK / 4)
          for (int j = 0; j < 4; ++j) gcn[4 * tid + j] = chd::ex2(pgn[j]);
      } else {
        if (tid < DK) gcn[tid] = chd::ex2(pgn[0]);
      }
    }
#pragma unroll
    for (int it = 0; it < kUIt; it += STEPU) {
      int t, r;
      elem_tr(it, t, r);
      float u4[STEPU];
#pragma unroll
      for (int j = 0; j < STEPU; ++j) u4[j] = (t < n && r + j < nv) ? pu[it + j] : 0.f;
      st_row<STEPU>(&Us[t][r], u4);
    }
    if (tid < kCMax) chunk_gates(f, tok(0), n, tid, gs, eg, wd);
    __syncthreads();
    if (ci + 1 < a.NC) cload(ci + 1);   // in flight during this chunk's products
    if (16 * rb < kBV) {   // D = U - W S^T, tile (tb, rb) (kBV = 16: waves 0..3 only)
      const float4v acc = dot_kc<DK>(&Ws[16 * tb + col][0], &Ss[16 * rb + col][0], kq);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tb + 4 * kq + r, rr = 16 * rb + col;
        const bool in = t < n && rr < nv;
        const float d = Us[t][rr] - acc[r];
        if (in) a.D[tok(t) * Dv + v0 + rr] = d;
        Dl[t][rr] = in ? wd[t] * d : 0.f;
      }
    }
    __syncthreads();
    // S <- e^{g_n} S + (e^{g_n - g} (.) D)^T R on the wave's tiles (rows of Dl past n are zero)
    {
      const float gl = eg[n - 1];
#pragma unroll
      for (int m = 0; m < NTW; ++m) {
        const int u = wave + 8 * m;
        if (u >= NTS) continue;
        const int rbs = u / NCB, cbs = u % NCB;
        float4v acc = Sacc[m] * (CHD ? gcn[16 * cbs + col] : gl), acc2 = {0.f, 0.f, 0.f, 0.f};   // two chains
        // (rows past n of Dl are zero) tokens in blocks of 16, lane quarter kq taking
        // t = m0 + j + 4 kq at step j of the block at m0, two steps per pass: the rows read by
        // one instruction sit 16 banks apart in Rs (row stride DK + 4) and Dl (kBV + 4)
        const int n16 = (n + 15) & ~15;
        for (int i = 0; i < n16; i += 8) {
          const int t = (i & ~15) + ((i >> 2) & 3) + 4 * kq;   // steps (i / 4) mod 4 and the next
          acc = mfma4(Dl[t][16 * rbs + col], Rs[t][16 * cbs + col], acc);
          acc2 = mfma4(Dl[t + 1][16 * rbs + col], Rs[t + 1][16 * cbs + col], acc2);
        }
        acc += acc2;
        Sacc[m] = acc;
        // the LDS mirror for the next chunk's W S^T (its reads of this chunk are done)
#pragma unroll
        for (int r = 0; r < 4; ++r) Ss[16 * rbs + 4 * kq + r][16 * cbs + col] = acc[r];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Reverse sweep: one workgroup of kSwThreads (8 waves) per (batch, head, tile of kSwBV value
// rows), chunks last to first, every product on the fp32 matrix cores (v_mfma_f32_16x16x4_f32,
// lane layout as in the per-chunk pass below).  The gradient dS (kSwBV x Dk) lives in the
// waves' accumulators for the whole sequence (16 x 16 tiles, a few per wave), mirrored in LDS
// for the products that read it as an operand.  Per chunk, wave w owns the 16 x 16 tile
// (token block w % 4, value-row block w / 4) of dD and dX.  With per-channel decay (CHD) the
// keys are decayed elementwise as they are staged (2^(G_n - G) (.) R, 2^G (.) E, 2^G (.) Q)
// and dS <- dS Diag(2^G_n) + ... scales the gradient's columns.
// ---------------------------------------------------------------------------------------
constexpr int kSwBV = 32;
constexpr int kSwThreads = 512;


template <typename IO, int DK, bool CHD, bool PC, bool BAND, bool V4, int BVT>
__global__ __launch_bounds__(kSwThreads) void bwd_sweep_kernel(BwdArgs a) {
  // V4 (Dk and Dv multiples of 4, 16-byte aligned tensors): every staged array is read four
  // consecutive elements per load and written to LDS 16 bytes at a time; a quarter of the
  // load addresses stay live across the chunk, which keeps this kernel out of scratch
  constexpr int LD = DK + 4;
  constexpr int kBV = BVT, kThreads = kSwThreads;   // value rows per workgroup: 32, or 16
  constexpr int kLoadIt = kCMax * DK / kThreads;
  constexpr int NCB = DK / 16;                   // channel blocks
  constexpr int NTS = (kBV / 16) * NCB;          // dS tiles
  constexpr int NTW = (NTS + 7) / 8;             // dS tiles per wave
  const ChunkArgs &f = a.f;
  const IO *__restrict__ q = static_cast<const IO *>(f.q);
  const IO *__restrict__ k = static_cast<const IO *>(f.k);
  const IO *__restrict__ er = static_cast<const IO *>(f.erase);
  const IO *__restrict__ wk = static_cast<const IO *>(f.write_key);
  const IO *__restrict__ dout = static_cast<const IO *>(a.dout);

  const int tid = threadIdx.x;
  int vt, h, b;
  xcd_tile(vt, h, b);
  const int v0 = vt * kBV;
  const int nv = min(kBV, f.Dv - v0);
  const int Dk = f.Dk, Dv = f.Dv, H = f.H, T = f.T, C = f.C;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 15, kq = lane >> 4;
  const int tb = wave & 3, rb = wave >> 2;        // this wave's dD / dX tile

  __shared__ __align__(16) float Ks[kCMax][LD];     // write keys r, then queries q
  __shared__ __align__(16) float Es[kCMax][LD];     // erase keys e
  __shared__ float Tm[kCMax][kCMax + 1];            // T (unit lower)
  __shared__ float Pm[kCMax][kCMax + 1];            // P (lower)
  __shared__ __align__(16) float dS[kBV][LD];       // mirror of the gradient at the chunk's end
  __shared__ __align__(16) float dOs[kCMax][kBV];   // dO
  __shared__ __align__(16) float dDs[kCMax][kBV];   // dD
  // (rows padded to kBV + 4: the dS update reads rows t, t + 4, t + 8, t + 12 in one
  // instruction, on distinct banks)
  __shared__ __align__(16) float Am[kCMax][kBV + 4];    // scale e^g dO
  __shared__ __align__(16) float Bm[kCMax][kBV + 4];    // e^g dX
  __shared__ float gs[kCMax], eg[kCMax], wd[kCMax];
  __shared__ float gcn[CHD ? DK : 1];   // CHD: 2^G_n per channel
  __shared__ float bsm[kCMax];          // scalar gain of the chunk being staged

  const long long sh = static_cast<long long>(b) * H + h;
  // dS tiles of this wave: tile u = wave + 8 m -> value-row block u / NCB, channel block u % NCB
  float4v dSacc[NTW];
#pragma unroll
  for (int m = 0; m < NTW; ++m) {
    const int u = wave + 8 * m;
    const int row = 16 * (u / NCB) + 4 * kq, c = 16 * (u % NCB) + col;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = 0.f;
      if (u < NTS && a.dstate_out != nullptr && row + r < nv && c < Dk)
        x = a.dstate_out[(sh * Dv + v0 + row + r) * Dk + c];
      dSacc[m][r] = x;
    }
  }
  for (int idx = tid; idx < kBV * LD; idx += kThreads) {
    const int r = idx / LD, c = idx % LD;
    float s = 0.f;
    if (a.dstate_out != nullptr && r < nv && c < Dk) s = a.dstate_out[(sh * Dv + v0 + r) * Dk + c];
    dS[r][c] = s;
  }
  // Loads of chunk ci into registers (indices clamped into the chunk, masks applied when they
  // are written to LDS): write keys, keys, gains, T, P, dO and log alpha are loaded one chunk
  // ahead, so they are in flight during the previous chunk's products; the queries, needed
  // only after the first two barriers of a chunk, are loaded at its start.
  constexpr int kCC = kCMax * kCMax / kThreads, kOIt = kCMax * kBV / kThreads;
  float xr[kLoadIt], xk[kLoadIt], xg[kLoadIt], xq[kLoadIt], xt[kCC], xp[kCC], xo[kOIt], xla = 0.f;
  // scalar gain: beta of the next chunk's token tid (tid < C), published to bsm after this
  // chunk's staging has read it (one load per token instead of one per staged element)
  float xb = 0.f;
  // CHD: G of the staged elements and G_n of the thread's channel (the same in every item:
  // kThreads is a multiple of DK), loaded a chunk ahead once this chunk's queries are staged
  float xgv[CHD ? kLoadIt : 1], xgn[V4 ? 4 : 1] = {};
  const IO *rbase = (f.wkey == GDR_WKEY_EXPLICIT) ? wk : k;
  constexpr int STEP = V4 ? 4 : 1;   // elements per load
  // (dO in fours only when every thread has whole groups of four: kBV = 32)
  constexpr bool V4O = V4 && kOIt % 4 == 0;
  constexpr int STEPO = V4O ? 4 : 1;
  static_assert(!V4 || (kLoadIt % 4 == 0 && kCC % 4 == 0 && DK % 4 == 0), "V4 loads take whole groups of four");
  // element `it` of this thread in a chunk's [C][DK] tile (V4: four consecutive channels per
  // group of four elements; the thread's channels are then 4 (tid mod DK/4) + j in every
  // group, as kThreads is a multiple of DK), in a [C][kBV] value tile, in a C x C matrix (flat)
  auto elem_tc = [&](int it, int &t, int &c) __attribute__((always_inline)) {
    if constexpr (V4) {
      const int iv = tid + (it >> 2) * kThreads;
      t = iv / (DK / 4);
      c = 4 * (iv % (DK / 4)) + (it & 3);
    } else {
      const int idx = tid + it * kThreads;
      t = idx / DK;
      c = idx % DK;
    }
  };
  auto elem_tr = [&](int it, int &t, int &r) __attribute__((always_inline)) {
    if constexpr (V4O) {
      const int iv = tid + (it >> 2) * kThreads;
      t = iv / (kBV / 4);
      r = 4 * (iv % (kBV / 4)) + (it & 3);
    } else {
      const int idx = tid + it * kThreads;
      t = idx / kBV;
      r = idx % kBV;
    }
  };
  auto elem_cc = [&](int it) __attribute__((always_inline)) {
    return V4 ? 4 * (tid + (it >> 2) * kThreads) + (it & 3) : tid + it * kThreads;
  };
  // write key = key (no explicit or preconditioned write key): the keys are loaded once
  const bool rk_same = !PC && f.wkey != GDR_WKEY_EXPLICIT;
  // the next chunk's loads, in three groups: keys (and gains), T and P, dO
  auto cload_keys = [&](int ci) {
    const int c0 = ci * C, n = min(C, T - c0);
    const long long row0 = (static_cast<long long>(b) * T + c0) * H + h;
    if (tid < kCMax) {
      xla = chunk_log_alpha(f, row0, n, tid);
      if (f.gain == GDR_GAIN_SCALAR) xb = f.beta[row0 + static_cast<long long>(min(tid, n - 1)) * H];
    }
    const IO *kc = k + row0 * Dk, *ec = er + row0 * Dk;
#pragma unroll
    for (int it = 0; it < kLoadIt; it += STEP) {
      int t, c;
      elem_tc(it, t, c);
      const int tc = min(t, n - 1);
      if constexpr (V4) {
        const int o = tc * H * Dk + min(c, Dk - 4);
        if (!rk_same) ld_wkey4<PC>(a, rbase, row0 * Dk, o, &xr[it]);
        ld4e(kc, o, &xk[it]);
        if (f.gain != GDR_GAIN_SCALAR) ld4e(ec, o, &xg[it]);
      } else {
        const int o = tc * H * Dk + min(c, Dk - 1);
        if (!rk_same) xr[it] = ld_wkey<PC>(a, rbase, row0 * Dk, o);
        xk[it] = ld_f(kc, o);
        if (f.gain != GDR_GAIN_SCALAR) xg[it] = ld_f(ec, o);
      }
    }
  };
  auto cload_tp = [&](int ci) {
    const long long cc = (sh * a.NC + ci) * static_cast<long long>(C * C);
#pragma unroll
    for (int it = 0; it < kCC; it += STEP) {
      if constexpr (V4) {
        const int iv = min(elem_cc(it), C * C - 4);
        ld4e(a.Tw + cc, iv, &xt[it]);
        ld4e(a.Pw + cc, iv, &xp[it]);
      } else {
        const int idx = min(elem_cc(it), C * C - 1);
        xt[it] = a.Tw[cc + idx];
        xp[it] = a.Pw[cc + idx];
      }
    }
  };
  auto cload_do = [&](int ci) {
    const int c0 = ci * C, n = min(C, T - c0);
    const long long row0 = (static_cast<long long>(b) * T + c0) * H + h;
#pragma unroll
    for (int it = 0; it < kOIt; it += STEPO) {
      int t, r;
      elem_tr(it, t, r);
      t = min(t, n - 1);
      if constexpr (V4O)
        ld4e(dout, (row0 + static_cast<long long>(t) * H) * Dv + v0 + min(r, nv - 4), &xo[it]);
      else
        xo[it] = ld_f(dout, (row0 + static_cast<long long>(t) * H) * Dv + v0 + min(r, nv - 1));
    }
  };
  auto cload = [&](int ci) {
    cload_keys(ci);
    cload_tp(ci);
    cload_do(ci);
  };
  auto gload = [&](int ci) {
    const int n = min(C, T - ci * C);
    const float *Gc = a.Gw + (sh * a.NC + ci) * static_cast<long long>(C) * Dk;
#pragma unroll
    for (int it = 0; it < kLoadIt; it += STEP) {
      int t, c;
      elem_tc(it, t, c);
      t = min(t, n - 1);
      if constexpr (V4)
        ld4e(Gc, static_cast<long long>(t) * Dk + min(c, Dk - 4), &xgv[it]);
      else
        xgv[it] = Gc[static_cast<long long>(t) * Dk + min(c, Dk - 1)];
    }
    if constexpr (V4)
      ld4e(Gc, static_cast<long long>(n - 1) * Dk + min(4 * (tid % (DK / 4)), Dk - 4), xgn);
    else
      xgn[0] = Gc[static_cast<long long>(n - 1) * Dk + min(tid % DK, Dk - 1)];
  };
  if (a.NC > 0) {
    cload(a.NC - 1);
    if constexpr (CHD) gload(a.NC - 1);
    if (tid < kCMax) bsm[tid] = xb;
  }

  for (int ci = a.NC - 1; ci >= 0; --ci) {
    const int c0 = ci * C;
    const int n = min(C, T - c0);
    auto tok = [&](int t) -> long long { return (static_cast<long long>(b) * T + c0 + t) * H + h; };
    const long long row0 = tok(0);

    __syncthreads();   // previous chunk done with every buffer
    {
      const IO *qc = q + row0 * Dk;
#pragma unroll
      for (int it = 0; it < kLoadIt; it += STEP) {
        int t, c;
        elem_tc(it, t, c);
        if constexpr (V4)
          ld4e(qc, min(t, n - 1) * H * Dk + min(c, Dk - 4), &xq[it]);
        else
          xq[it] = ld_f(qc, min(t, n - 1) * H * Dk + min(c, Dk - 1));
      }
    }
    if (tid < kCMax) chunk_gates_from(xla, n, tid, gs, eg, wd);
    {   // the gradient at this chunk's end, for the per-chunk pass (from the accumulators)
      float *dhc = a.dh + ((sh * a.NC + ci) * Dv + v0) * static_cast<long long>(Dk);
#pragma unroll
      for (int m = 0; m < NTW; ++m) {
        const int u = wave + 8 * m;
        const int row = 16 * (u / NCB) + 4 * kq, c = 16 * (u % NCB) + col;
        if (u < NTS && c < Dk) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (row + r < nv) dhc[static_cast<long long>(row + r) * Dk + c] = dSacc[m][r];
        }
      }
    }
    // (V4: a lane's four elements are consecutive channels of one row, one 16-byte LDS write;
    // the rows are 16-byte aligned)
#pragma unroll
    for (int it = 0; it < kLoadIt; it += STEP) {
      int t, c;
      elem_tc(it, t, c);
      const bool in = t < n && c < Dk;
      const float gsc = f.gain == GDR_GAIN_SCALAR ? bsm[t] : 0.f;
      float kr[STEP], ke[STEP];
#pragma unroll
      for (int j = 0; j < STEP; ++j) {
        const float r = rk_same ? xk[it + j] : xr[it + j];
        const float g = f.gain == GDR_GAIN_SCALAR ? gsc : xg[it + j];
        if constexpr (CHD) {
          // (exp2f, not the bare hardware 2^x the other kernels use: measured at B4 H16 T4096,
          // the schedule the compiler makes around the single instruction costs this kernel
          // 1.04 -> 1.19 ms)
          kr[j] = in ? r * exp2f(xgn[j] - xgv[it + j]) : 0.f;
          ke[j] = in ? g * xk[it + j] * exp2f(xgv[it + j]) : 0.f;
        } else {
          kr[j] = in ? r : 0.f;
          ke[j] = in ? g * xk[it + j] : 0.f;
        }
      }
      st_row<STEP>(&Ks[t][c], kr);
      st_row<STEP>(&Es[t][c], ke);
    }
    if constexpr (CHD) {
      if constexpr (V4) {
        if (tid < DK / 4)
          for (int j = 0; j < 4; ++j) gcn[4 * tid + j] = exp2f(xgn[j]);
      } else {
        if (tid < DK) gcn[tid] = exp2f(xgn[0]);
      }
    }
#pragma unroll
    for (int it = 0; it < kCC; ++it) {
      const int idx = elem_cc(it);
      if (idx < C * C) {
        Tm[idx / C][idx % C] = xt[it];
        Pm[idx / C][idx % C] = xp[it];
      }
    }
#pragma unroll
    for (int it = 0; it < kOIt; it += STEPO) {
      int t, r;
      elem_tr(it, t, r);
      float o4[STEPO];
#pragma unroll
      for (int j = 0; j < STEPO; ++j) o4[j] = (t < n && r + j < nv) ? xo[it + j] : 0.f;
      st_row<STEPO>(&dOs[t][r], o4);
    }
    __syncthreads();
    // the next chunk's loads, in flight during this chunk's products: T and P here, the keys
    // and dO after the next barrier (a wave's loads hold up its own instruction issue; split
    // between two phases they lengthen each less than they would one)
    if (ci > 0) cload_tp(ci - 1);
    const int tr0 = 16 * tb + 4 * kq;   // the lane's result rows (tokens) of the dD / dX tile
    // dD = e^{g_n - g} (.) (R dS^T) + scale P^T dO, tile (tb, rb); P is zero above the
    // diagonal and T, P, dO rows past n (inside the chunk) are zero (kBV = 16: waves 0..3)
    const bool vtile = 16 * rb < kBV;
    if (vtile) {
      // R dS^T (16-byte operand reads), then P^T dO
      float4v a1[1], a2 = {0.f, 0.f, 0.f, 0.f};
      a1[0] = dot_kc<DK>(&Ks[16 * tb + col][0], &dS[16 * rb + col][0], kq);
      // (i0 < n keeps every row read below C, where T and P were loaded)
      for (int i0 = 16 * tb; i0 < n; i0 += 4)
        a2 = mfma4(Pm[i0 + kq][16 * tb + col], dOs[i0 + kq][16 * rb + col], a2);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tr0 + r, rr = 16 * rb + col;
        const float dd = fmaf(wd[t], a1[0][r], f.scale * a2[r]);
        dDs[t][rr] = (t < n && rr < nv) ? dd : 0.f;
        if (BAND && t < n && rr < nv) a.dDw[tok(t) * Dv + v0 + rr] = dd;   // (band-limited T)
      }
    }
    __syncthreads();
    if (ci > 0) {
      cload_keys(ci - 1);
      cload_do(ci - 1);
    }
    // dX = T^T dD, tile (tb, rb); written out for the per-chunk pass, and folded with e^g
    // into the state-gradient update
    if (vtile) {
      float4v x = {0.f, 0.f, 0.f, 0.f};
      for (int i0 = 16 * tb; i0 < n; i0 += 4)
        x = mfma4(Tm[i0 + kq][16 * tb + col], dDs[i0 + kq][16 * rb + col], x);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tr0 + r, rr = 16 * rb + col;
        const bool in = t < n && rr < nv;
        if (in) a.dX[tok(t) * Dv + v0 + rr] = x[r];
        Bm[t][rr] = in ? eg[t] * x[r] : 0.f;
        Am[t][rr] = in ? f.scale * eg[t] * dOs[t][rr] : 0.f;
      }
    }
    // queries replace the write keys (their last read was before the barrier above)
#pragma unroll
    for (int it = 0; it < kLoadIt; it += STEP) {
      int t, c;
      elem_tc(it, t, c);
      float q4[STEP];
#pragma unroll
      for (int j = 0; j < STEP; ++j)
        q4[j] = (t < n && c < Dk) ? (CHD ? xq[it + j] * exp2f(xgv[it + j]) : xq[it + j]) : 0.f;
      st_row<STEP>(&Ks[t][c], q4);
    }
    if constexpr (CHD) {
      if (ci > 0) gload(ci - 1);   // this chunk's G is no longer needed
    }
    __syncthreads();
    // (the next chunk's gains: this chunk's staging read bsm before the first barrier)
    if (ci > 0 && tid < kCMax) bsm[tid] = xb;
    // dS <- e^{g_n} dS + A^T Q - B^T E on the wave's tiles; rows of A, B past n are zero
    // Tokens in blocks of 16, lane quarter kq taking t = m0 + j + 4 kq at step j of the block
    // at m0: the rows one instruction reads sit 4 apart, i.e. 16 banks apart in Ks and Es (row
    // stride DK + 4) and in Am and Bm (kBV + 4), so each operand read is free of bank
    // conflicts; rows of the last block past n are zero.  With two tiles per wave (DK = 128)
    // both share the channel block (wave + 8 m has the same remainder mod 8), so the two run
    // in one loop: four independent accumulator chains, and one Q and one E read per step.
    {
      const float gl = eg[n - 1];
      const int n16 = (n + 15) & ~15;
      if constexpr (NTW == 2) {
        static_assert(NCB == 8, "two tiles per wave share a channel block");
        const int cbs = wave;
        const float sc = CHD ? gcn[16 * cbs + col] : gl;
        float4v a0 = dSacc[0] * sc, a1 = dSacc[1] * sc;
        float4v b0 = {0.f, 0.f, 0.f, 0.f}, b1 = {0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < n16; i += 4) {
          const int t = (i & ~15) + ((i >> 2) & 3) + 4 * kq;   // block i / 16, step (i / 4) mod 4
          const float qv = Ks[t][16 * cbs + col], ev = Es[t][16 * cbs + col];
          a0 = mfma4(Am[t][col], qv, a0);
          a1 = mfma4(Am[t][16 + col], qv, a1);
          b0 = mfma4(Bm[t][col], ev, b0);
          b1 = mfma4(Bm[t][16 + col], ev, b1);
        }
        dSacc[0] = a0 - b0;
        dSacc[1] = a1 - b1;
        // the LDS mirror for the next chunk's R dS^T (its reads of this chunk are done)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int r = 0; r < 4; ++r) dS[16 * m + 4 * kq + r][16 * cbs + col] = dSacc[m][r];
      } else {
#pragma unroll
        for (int m = 0; m < NTW; ++m) {
          const int u = wave + 8 * m;
          if (u >= NTS) continue;
          const int rbs = u / NCB, cbs = u % NCB;
          float4v acc = dSacc[m] * (CHD ? gcn[16 * cbs + col] : gl), acc2 = {0.f, 0.f, 0.f, 0.f};   // two chains
          for (int i = 0; i < n16; i += 4) {
            const int t = (i & ~15) + ((i >> 2) & 3) + 4 * kq;
            acc = mfma4(Am[t][16 * rbs + col], Ks[t][16 * cbs + col], acc);
            acc2 = mfma4(Bm[t][16 * rbs + col], Es[t][16 * cbs + col], acc2);
          }
          acc -= acc2;
          dSacc[m] = acc;
#pragma unroll
          for (int r = 0; r < 4; ++r) dS[16 * rbs + 4 * kq + r][16 * cbs + col] = acc[r];
        }
      }
    }
  }
  if (a.dstate_in != nullptr) {
#pragma unroll
    for (int m = 0; m < NTW; ++m) {
      const int u = wave + 8 * m;
      const int row = 16 * (u / NCB) + 4 * kq, c = 16 * (u % NCB) + col;
      if (u < NTS && c < Dk) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (row + r < nv) a.dstate_in[(sh * Dv + v0 + row + r) * Dk + c] = dSacc[m][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Per-chunk pass: one workgroup of kCkThreads (8 waves) per (batch, head, chunk); every
// product on the fp32 matrix cores (v_mfma_f32_16x16x4_f32: lane l gives A[l % 16][l / 16]
// and B[l / 16][l % 16], and holds D[4 (l / 16) + r][l % 16], r < 4).  Wave w owns token
// block tb = w % 4 (16 tokens) and channel half hh = w / 4: the 16 x 16 tiles of dQ, dE, dR
// at (tb, channel tiles of that half); the half-0 waves also own the tiles of dO D^T in row
// block tb (on and below the diagonal), the half-1 waves those of dX D^T (with the band-limited
// T (BAND): of dD D^T, every tile, for the band block that replaces -dX D^T).
// With per-channel decay (CHD) the wave's channel tiles are two in each 64-channel half, and
// the key products run over the halves in turn (Q, E, R, G of one half in LDS): the pairwise
// decay 2^(G_ic - G_jc) sits inside the sums over tokens, split at a reference row for the
// blocks off the diagonal (matrix cores, every exponent <= 0) and taken pair by pair on the
// diagonal block; the gate gradient is one per token and channel.
// ---------------------------------------------------------------------------------------
constexpr int kCkThreads = 512;


template <typename IO, int DK, bool CHD, bool PC, bool BAND>
__global__ __launch_bounds__(kCkThreads) void bwd_chunk_kernel(BwdArgs a) {
  static_assert(DK == 64 || DK == 128, "two halves of 16-channel tiles");
  constexpr int kThreads = kCkThreads;
  constexpr int kWaves = kThreads / 64;
  constexpr int LD = DK + 4;
  constexpr int MT = DK / 32;      // channel tiles per wave
  constexpr int kVB = 32;          // value rows per step of the value loop
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
  const int wave = tid >> 6, lane = tid & 63;
  const int tb = wave & 3, hh = wave >> 2;
  const int col = lane & 15, kq = lane >> 4;
  const int tr0 = 16 * tb + 4 * kq;   // first of the lane's 4 result rows (tokens)
  const long long sh = static_cast<long long>(b) * H + h;
  auto tok = [&](int t) -> long long { return (static_cast<long long>(b) * T + c0 + t) * H + h; };
  const long long row0 = tok(0);
  // the lane's channel in its tile m (CHD: tiles 2 hh, 2 hh + 1 of each 64-channel half)
  auto chan = [&](int m) { return CHD ? 16 * (4 * (m >> 1) + 2 * hh + (m & 1)) + col : 16 * (MT * hh + m) + col; };

  struct TilesA {   // value loop: state rows, their gradients, token tiles by value row
    float S[kVB][LD], dS[kVB][LD], dOT[kVB][LT], dXT[kVB][LT], DT[kVB][LT], dDT[kVB][LT];
  };
  struct TilesBand {   // band-limited T: Z = dD D^T, then W1^T; L for T_b^-1; T_b^-1; T; T^T
    float Z[kCMax][LT], Lb[kCMax][LT], Ti[kCMax][LT], Tf[kCMax][LT], TT[kCMax][LT], Zs[32][36];
  };
  struct TilesB {   // key products: Q, E, R and the C x C gradients dM, dL'
    float Q[kCMax][LD], E[kCMax][LD], R[kCMax][LD], dM[kCMax][LT], dL[kCMax][LT];
  };
  constexpr int LC = 68;   // (CHD) row stride of the 64-channel half tiles
  struct TilesC {          // (CHD) key products by channel halves: Q, E, R, G of one half; dM, dL'
    float Q[kCMax][LC], E[kCMax][LC], R[kCMax][LC], G[kCMax][LC], dM[kCMax][LT], dL[kCMax][LT];
  };
  __shared__ __align__(16) union {
    TilesA A;
    std::conditional_t<CHD, TilesC, TilesB> B;
    TilesBand Bd;
  } sm;
  __shared__ float gs[kCMax], eg[kCMax], wd[kCMax], vdx[kCMax];
  __shared__ float dgs[2][kCMax], pks[2][kCMax];
  __shared__ float red[2][kWaves];
  // (CHD) per-thread shares of <dS'_c, S_c> (the thread's channel is tid % DK), and per token
  // block: the channel sums of dg and of r (.) (2^(G_n - G) D dS')
  __shared__ float sdp[CHD ? kThreads : 1], tsum[CHD ? 4 : 1][64], lsum[CHD ? 4 : 1][64];

  if (tid < kCMax) chunk_gates(f, row0, n, tid, gs, eg, wd);

  float4v AQ[MT], AE[MT], AR[MT], MPL[4];
#pragma unroll
  for (int m = 0; m < MT; ++m) AQ[m] = AE[m] = AR[m] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) MPL[jb] = float4v{0.f, 0.f, 0.f, 0.f};
  float sdot = 0.f;   // this thread's share of <dS', S>
  float vsum = 0.f;   // this thread's share of v_t . dX_t (scalar gain), t = tid >> 3
  const float *hc = a.h + (sh * a.NC + ci) * static_cast<long long>(Dv) * Dk;
  const float *dhc = a.dh + (sh * a.NC + ci) * static_cast<long long>(Dv) * Dk;

  // ---- value loop: dO S, dX S, D dS', dO D^T, dX D^T --------------------------------
  // Each block of kVB value rows is loaded into registers one block ahead (indices clamped,
  // masks applied when the registers are written to LDS), so its loads are in flight while
  // the previous block is multiplied.
  constexpr int kSIt = kVB * DK / kThreads;   // state elements per thread and block
  float ps[kSIt], pds[kSIt], po[4], px[4], pd[4], pv[4], pw[4], pdd[4];
  const int lt = tid >> 3, rq = 4 * (tid & 7);   // token-tile element (token lt, rows rq .. rq + 3)
  // band-limited T: the hh = 1 waves form Z = dD D^T (every tile) instead of dX D^T
  constexpr bool band = BAND;
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
      if constexpr (BAND) pdd[u] = a.dDw[idx];
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
      if constexpr (BAND) sm.A.dDT[r][lt] = in ? pdd[u] : 0.f;
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
    // K = kVB value rows in steps of 4 (rows past nvb are zero), lane quarter kq taking row
    // m0 + j + 4 kq at step j of each block of 16: the rows one instruction reads sit 4 apart,
    // 16 banks apart at the row strides DK + 4 and kCMax + 4, free of bank conflicts
#pragma unroll
    for (int ks = 0; ks < kVB; ks += 4) {
      const int kr = (ks & ~15) + ((ks >> 2) & 3) + 4 * kq;
      const float ao = sm.A.dOT[kr][16 * tb + col], ax = sm.A.dXT[kr][16 * tb + col];
      const float ad = sm.A.DT[kr][16 * tb + col];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float bs = sm.A.S[kr][chan(m)], bds = sm.A.dS[kr][chan(m)];
        AQ[m] = mfma4(ao, bs, AQ[m]);
        AE[m] = mfma4(ax, bs, AE[m]);
        AR[m] = mfma4(ad, bds, AR[m]);
      }
      const float am = hh == 0 ? ao : band ? sm.A.dDT[kr][16 * tb + col] : ax;
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
        if (jb <= tb || (band && hh == 1)) MPL[jb] = mfma4(am, sm.A.DT[kr][16 * jb + col], MPL[jb]);
    }
  }
  vsum += __shfl_xor(vsum, 1);
  vsum += __shfl_xor(vsum, 2);
  vsum += __shfl_xor(vsum, 4);
  if ((tid & 7) == 0) vdx[lt] = vsum;

  if constexpr (CHD) {
    // ---- key products, per-channel decay --------------------------------------------------
    constexpr int NH = DK / 64;                   // channel halves
    constexpr int kHIt = kCMax * 64 / kThreads;   // staged elements per thread and half
    auto &B = sm.B;
    __syncthreads();   // the value-loop tiles are dead (the key tiles share their memory)
    sdp[tid] = sdot;
    // dM = scale dO D^T (j <= i), dL' = -dX D^T (j < i) on the tiles on and below the diagonal
    // (the decay, per channel, goes inside the products over tokens below)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tr0 + r;
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        if (jb > tb) continue;
        const int j = 16 * jb + col;
        if (hh == 0)
          B.dM[t][j] = (j <= t && t < n) ? f.scale * MPL[jb][r] : 0.f;
        else
          B.dL[t][j] = (j < t && t < n) ? -MPL[jb][r] : 0.f;
      }
    }
    const IO *qc = q + row0 * Dk, *kc = k + row0 * Dk, *ec = er + row0 * Dk;
    const IO *rbase = (f.wkey == GDR_WKEY_EXPLICIT) ? wk : k;
    const float *bc = f.beta + row0;
    const float *Gc = a.Gw + (sh * a.NC + ci) * static_cast<long long>(C) * Dk;
    float pk[4] = {0.f, 0.f, 0.f, 0.f};   // k . dE over the lane's channels (scalar gain)
    for (int hc = 0; hc < NH; ++hc) {
      {   // Q, E, R, G of channels 64 hc .. 64 hc + 63: loads first (clamped), then masked stores
        float xq[kHIt], xk[kHIt], xg[kHIt], xr[kHIt], xG[kHIt];
#pragma unroll
        for (int it = 0; it < kHIt; ++it) {
          const int idx = tid + it * kThreads, t = idx >> 6, c = 64 * hc + (idx & 63);
          const int tc = min(t, n - 1), cc = min(c, Dk - 1), o = tc * H * Dk + cc;
          xq[it] = ld_f(qc, o);
          xk[it] = ld_f(kc, o);
          xg[it] = f.gain == GDR_GAIN_SCALAR ? bc[tc * H] : ld_f(ec, o);
          xr[it] = ld_wkey<PC>(a, rbase, row0 * Dk, o);
          xG[it] = Gc[static_cast<long long>(tc) * Dk + cc];   // (flat past n)
        }
        __syncthreads();   // the previous half's tiles are consumed
#pragma unroll
        for (int it = 0; it < kHIt; ++it) {
          const int idx = tid + it * kThreads, t = idx >> 6, cl = idx & 63, c = 64 * hc + cl;
          const bool in = t < n && c < Dk;
          B.Q[t][cl] = in ? xq[it] : 0.f;
          B.E[t][cl] = in ? xg[it] * xk[it] : 0.f;
          B.R[t][cl] = in ? xr[it] : 0.f;
          B.G[t][cl] = c < Dk ? xG[it] : 0.f;
        }
      }
      __syncthreads();
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int m = 2 * hc + mm;
        const int cl = 16 * (2 * hh + mm) + col, c = 64 * hc + cl;   // = chan(m)
        float gt[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) gt[r] = B.G[tr0 + r][cl];
        const float gn = B.G[n - 1][cl];
        // the state terms' decays; this lane's share of sum_j r_j (.) (2^(G_n - G_j) (D dS')_j)
        float lam = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = chd::ex2(gt[r]);
          AQ[m][r] *= f.scale * e;
          AE[m][r] *= -e;
          AR[m][r] *= chd::ex2(gn - gt[r]);
          lam = fmaf(B.R[tr0 + r][cl], AR[m][r], lam);
        }
        // dQ += dM R, dE += dL' R with 2^(G_i - G_j): the blocks before block tb through their
        // reference, the row before the block (2^(G_i - G_ref) 2^(G_ref - G_j)), then the
        // diagonal block pair by pair
        if (tb > 0) {
          const float gr = B.G[16 * tb - 1][cl];
          float4v tq = {0.f, 0.f, 0.f, 0.f}, te = {0.f, 0.f, 0.f, 0.f};
          #pragma unroll 1
          for (int j0 = 0; j0 < 16 * tb; j0 += 4) {
            const int jr = j0 + kq;
            const float br = B.R[jr][cl] * chd::ex2(gr - B.G[jr][cl]);
            tq = mfma4(B.dM[16 * tb + col][jr], br, tq);
            te = mfma4(B.dL[16 * tb + col][jr], br, te);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float sc = chd::ex2(gt[r] - gr);
            AQ[m][r] = fmaf(sc, tq[r], AQ[m][r]);
            AE[m][r] = fmaf(sc, te[r], AE[m][r]);
          }
        }
        #pragma unroll 2
        for (int jj = 0; jj < 16; ++jj) {
          const int j = 16 * tb + jj;
          const float rj = B.R[j][cl], gj = B.G[j][cl];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = tr0 + r;
            // (the exponent above the diagonal may overflow; it is discarded)
            const float w = j <= i ? rj * chd::ex2(gt[r] - gj) : 0.f;
            AQ[m][r] = fmaf(B.dM[i][j], w, AQ[m][r]);
            AE[m][r] = fmaf(B.dL[i][j], w, AE[m][r]);
          }
        }
        // dR += dM^T Q + dL'^T E with 2^(G_i - G_j): the blocks after block tb through the
        // block's last row, then the diagonal block pair by pair
        {
          const float gr = B.G[16 * tb + 15][cl];
          float4v tr = {0.f, 0.f, 0.f, 0.f};
          // (i0 < n keeps every row read below 64; rows past n are zero)
          #pragma unroll 1
          for (int i0 = 16 * (tb + 1); i0 < n; i0 += 4) {
            const int ir = i0 + kq;
            const float sc = chd::ex2(B.G[ir][cl] - gr);
            tr = mfma4(B.dM[ir][16 * tb + col], B.Q[ir][cl] * sc, tr);
            tr = mfma4(B.dL[ir][16 * tb + col], B.E[ir][cl] * sc, tr);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) AR[m][r] = fmaf(chd::ex2(gr - gt[r]), tr[r], AR[m][r]);
        }
        #pragma unroll 2
        for (int ii = 0; ii < 16; ++ii) {
          const int i = 16 * tb + ii;
          const float qi = B.Q[i][cl], ei = B.E[i][cl], gi = B.G[i][cl];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = tr0 + r;
            const float w = i >= j ? chd::ex2(gi - gt[r]) : 0.f;
            AR[m][r] = fmaf(fmaf(B.dM[i][j], qi, B.dL[i][j] * ei), w, AR[m][r]);
          }
        }
        // dg_tc = q . dQ + e . dE - r . dR per token and channel; dlog alpha is its reverse
        // cumulative sum along the chunk (rows past n are zero): within the lane's 4 rows, over
        // the 4 lane groups of the channel, over the 4 token blocks (LDS)
        float suf[4];
#pragma unroll
        for (int r = 3; r >= 0; --r) {
          const int t = tr0 + r;
          const float dg = B.Q[t][cl] * AQ[m][r] + B.E[t][cl] * AE[m][r] - B.R[t][cl] * AR[m][r];
          suf[r] = r == 3 ? dg : dg + suf[r + 1];
        }
        float above = 0.f, wtot = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float x = __shfl(suf[0], col + 16 * g);
          wtot += x;
          if (g > kq) above += x;
        }
        lam += __shfl_xor(lam, 16);
        lam += __shfl_xor(lam, 32);
        if (kq == 0) {
          tsum[tb][cl] = wtot;
          lsum[tb][cl] = lam;
        }
        __syncthreads();
        float later = 0.f, lamc = 0.f, sdc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if (w > tb) later += tsum[w][cl];
          lamc += lsum[w][cl];
        }
#pragma unroll
        for (int p = 0; p < kThreads / DK; ++p) sdc += sdp[p * DK + min(c, DK - 1)];
        // the end-of-chunk terms (state decay and 2^(G_n - G) R) enter dg at token n - 1,
        // so every earlier token's sum holds them
        const float tail = above + later + chd::ex2(gn) * sdc + lamc;
        // chain rule to the variant's inputs, stores
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = tr0 + r;
          if (t >= n || c >= Dk) continue;
          const long long rowk = tok(t) * Dk;
          const float de = AE[m][r], dr = AR[m][r];
          a.dla[rowk + c] = suf[r] + tail;
          a.dq[rowk + c] = AQ[m][r];
          float dkv;
          if (f.gain == GDR_GAIN_SCALAR) {
            dkv = f.beta[tok(t)] * de;
            pk[r] = fmaf(ld_f(k, rowk + c), de, pk[r]);
          } else {
            dkv = ld_f(er, rowk + c) * de;
            a.derase[rowk + c] = ld_f(k, rowk + c) * de;
          }
          if (f.wkey != GDR_WKEY_SAME)   // (preconditioned: to the workspace, then through p_t)
            a.dwk[rowk + c] = dr;
          else
            dkv += dr;
          a.dk[rowk + c] = dkv;
        }
      }
    }
    if (f.gain == GDR_GAIN_SCALAR) {
#pragma unroll
      for (int mm2 = 1; mm2 < 16; mm2 <<= 1)
#pragma unroll
        for (int r = 0; r < 4; ++r) pk[r] += __shfl_xor(pk[r], mm2);
      if (col == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) pks[hh][tr0 + r] = pk[r];
      }
      __syncthreads();
      if (tid < n) a.dbeta[tok(tid)] = pks[0][tid] + pks[1][tid] + vdx[tid];
    }
  } else {
    // ---- band-limited T: dL = -T^T (M (.) dT_b) T^T with dT_b = dD X^T = (dD D^T) T_b^-T
    // (X = T_b^-1 D), M the band i - j <= N below the diagonal; T_b^-1 by the shared blocked
    // inverse of T_b, the products as 16 x 16 tiles on the matrix cores (LDS scratch over the
    // key tiles, which are loaded after it)
    float4v dlb[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    if constexpr (BAND) {
      auto &Bd = sm.Bd;
      __syncthreads();   // the value-loop tiles are dead
      if (hh == 1) {
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
          for (int r = 0; r < 4; ++r) Bd.Z[tr0 + r][16 * jb + col] = MPL[jb][r];
      }
      {
        const long long cc = (sh * a.NC + ci) * static_cast<long long>(C * C);
        for (int idx = tid; idx < kCMax * kCMax; idx += kThreads) {
          const int i = idx / kCMax, j = idx % kCMax;
          const bool in = i < C && j < C;
          const float tb_ = in ? a.Tw[cc + i * C + j] : 0.f, tf = in ? a.Tfw[cc + i * C + j] : 0.f;
          Bd.Lb[i][j] = j < i ? tb_ : 0.f;   // T_b = I + Lb: T_b^-1 = (I + Lb)^-1
          Bd.Tf[i][j] = tf;
          Bd.TT[j][i] = tf;
          if ((j >> 4) > (i >> 4)) Bd.Ti[i][j] = 0.f;
        }
      }
      __syncthreads();
      tri::inverse_blocks(Bd.Lb, Bd.Ti, Bd.Zs, -1, tid);   // (ends with a barrier)
      // Zm = M (.) (Z T_b^-T) on every tile (zero above the diagonal and outside the band)
      float4v zt[2];
#pragma unroll
      for (int u2 = 0; u2 < 2; ++u2) {
        const int u = wave + 8 * u2, ib = u >> 2, jb = u & 3;
        zt[u2] = jb <= ib ? dot_kc<kCMax>(&Bd.Z[16 * ib + col][0], &Bd.Ti[16 * jb + col][0], kq)
                          : float4v{0.f, 0.f, 0.f, 0.f};
      }
      __syncthreads();   // every read of Z done
#pragma unroll
      for (int u2 = 0; u2 < 2; ++u2) {
        const int u = wave + 8 * u2, ib = u >> 2, jb = u & 3;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * ib + 4 * kq + r, j = 16 * jb + col;
          Bd.Lb[i][j] = (j < i && i - j <= f.N) ? zt[u2][r] : 0.f;   // (Lb is free: Zm)
        }
      }
      __syncthreads();
      // W1 = Zm T^T, stored transposed (W1T[j][m] = W1[m][j]); only its part below the
      // diagonal is read with a non-zero factor, the rest is zero
#pragma unroll
      for (int u2 = 0; u2 < 2; ++u2) {
        const int u = wave + 8 * u2, ib = u >> 2, jb = u & 3;
        const float4v w = jb <= ib ? dot_kc<kCMax>(&Bd.Lb[16 * ib + col][0], &Bd.Tf[16 * jb + col][0], kq)
                                   : float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) Bd.Z[16 * jb + col][16 * ib + 4 * kq + r] = w[r];
      }
      __syncthreads();
      // dL = -T^T W1 on the ten tiles on and below the diagonal (kept in registers)
#pragma unroll
      for (int u2 = 0; u2 < 2; ++u2) {
        const int u = wave + 8 * u2;
        if (u < 10) {
          int ib, jb;
          lower_tile10(u, ib, jb);
          dlb[u2] = -dot_kc<kCMax>(&Bd.TT[16 * ib + col][0], &Bd.Z[16 * jb + col][0], kq);
        }
      }
    }
    // ---- key products -------------------------------------------------------------------
    __syncthreads();   // the value-loop tiles are dead (the key tiles share their memory)
    {   // Q, E, R: all loads first (clamped), then the masked LDS stores; the keys once when
        // the write key is the key, a scalar gain once per token (lane t holds token t's).  One
        // copy per case, so that no branch separates the loads and no array is merged.
      const IO *qc = q + row0 * Dk, *kc = k + row0 * Dk, *ec = er + row0 * Dk;
      const IO *rbase = (f.wkey == GDR_WKEY_EXPLICIT) ? wk : k;
      auto stage = [&](auto same, auto scalar) __attribute__((always_inline)) {
        constexpr bool kSame = decltype(same)::value, kScalar = decltype(scalar)::value;
        float xq[kLoadIt], xk[kLoadIt], xg[kScalar ? 1 : kLoadIt], xr[kSame ? 1 : kLoadIt];
        const float bl = kScalar ? f.beta[row0 + static_cast<long long>(min(lane, n - 1)) * H] : 0.f;
  #pragma unroll
        for (int it = 0; it < kLoadIt; ++it) {
          const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
          const int tc = min(t, n - 1), o = tc * H * Dk + min(c, Dk - 1);
          xq[it] = ld_f(qc, o);
          xk[it] = ld_f(kc, o);
          if constexpr (!kScalar) xg[it] = ld_f(ec, o);
          if constexpr (!kSame) xr[it] = ld_wkey<PC>(a, rbase, row0 * Dk, o);
        }
  #pragma unroll
        for (int it = 0; it < kLoadIt; ++it) {
          const int idx = tid + it * kThreads, t = idx / DK, c = idx % DK;
          const bool in = t < n && c < Dk;
          float g;
          if constexpr (kScalar)
            g = __shfl(bl, t);   // (t < kCMax = 64: a lane of this wave)
          else
            g = xg[it];
          sm.B.Q[t][c] = in ? xq[it] : 0.f;
          sm.B.E[t][c] = in ? g * xk[it] : 0.f;
          if constexpr (kSame)
            sm.B.R[t][c] = in ? xk[it] : 0.f;
          else
            sm.B.R[t][c] = in ? xr[it] : 0.f;
        }
      };
      const bool rk_same = !PC && f.wkey != GDR_WKEY_EXPLICIT, gsc = f.gain == GDR_GAIN_SCALAR;
      if (rk_same) {
        if (gsc) stage(std::true_type{}, std::true_type{});
        else stage(std::true_type{}, std::false_type{});
      } else {
        if (gsc) stage(std::false_type{}, std::true_type{});
        else stage(std::false_type{}, std::false_type{});
      }
    }
    // the decay factors of the state terms, and the C x C gradients (tiles on and below the
    // diagonal; the products below never read the others)
  #pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tr0 + r;
      const float sq = f.scale * eg[t], se = -eg[t], sr = wd[t];
  #pragma unroll
      for (int m = 0; m < MT; ++m) {
        AQ[m][r] *= sq;
        AE[m][r] *= se;
        AR[m][r] *= sr;
      }
  #pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        if (jb > tb) continue;
        const int j = 16 * jb + col;
        // (the exponent above the diagonal may overflow; it is discarded)
        const float dec = expf(gs[t] - gs[j]);
        if (hh == 0)
          sm.B.dM[t][j] = (j <= t && t < n) ? f.scale * MPL[jb][r] * dec : 0.f;
        else if (!band)
          sm.B.dL[t][j] = (j < t && t < n) ? -MPL[jb][r] * dec : 0.f;
      }
    }
    if constexpr (BAND) {   // dL' = dL (.) Gamma below the diagonal, from the band block's tiles
#pragma unroll
      for (int u2 = 0; u2 < 2; ++u2) {
        const int u = wave + 8 * u2;
        if (u < 10) {
          int ib, jb;
          lower_tile10(u, ib, jb);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * ib + 4 * kq + r, j = 16 * jb + col;
            sm.B.dL[t][j] = (j < t && t < n) ? dlb[u2][r] * expf(gs[t] - gs[j]) : 0.f;
          }
        }
      }
    }
    __syncthreads();
    // lambda: this lane's share of sum_j r_j . (e^{g_n - g_j} dS'^T d_j)
    float lam = 0.f;
  #pragma unroll
    for (int m = 0; m < MT; ++m)
  #pragma unroll
      for (int r = 0; r < 4; ++r) lam = fmaf(sm.B.R[tr0 + r][chan(m)], AR[m][r], lam);
    // dQ += dM R, dE += dL' R over tokens j < 16 (tb + 1)
    for (int j0 = 0; j0 < 16 * (tb + 1); j0 += 4) {
      const int jr = j0 + kq;
      const float am = sm.B.dM[16 * tb + col][jr], al = sm.B.dL[16 * tb + col][jr];
  #pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float br = sm.B.R[jr][chan(m)];
        AQ[m] = mfma4(am, br, AQ[m]);
        AE[m] = mfma4(al, br, AE[m]);
      }
    }
    // dR += dM^T Q + dL'^T E over tokens i >= 16 tb
    for (int i0 = 16 * tb; i0 < kCMax; i0 += 4) {
      const int ir = i0 + kq;
      const float am = sm.B.dM[ir][16 * tb + col], al = sm.B.dL[ir][16 * tb + col];
  #pragma unroll
      for (int m = 0; m < MT; ++m) {
        AR[m] = mfma4(am, sm.B.Q[ir][chan(m)], AR[m]);
        AR[m] = mfma4(al, sm.B.E[ir][chan(m)], AR[m]);
      }
    }
    // per token: q . dQ + e . dE - r . dR (gate) and k . dE (scalar gain) over the lane's
    // channels, summed over the 16 lanes of the row group, then over the two channel halves
    float pg[4], pk[4];
    const long long rowk0 = row0 * Dk;
  #pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tr0 + r;
      float acc = 0.f, acck = 0.f;
  #pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int c = chan(m);
        acc = fmaf(sm.B.Q[t][c], AQ[m][r], acc);
        acc = fmaf(sm.B.E[t][c], AE[m][r], acc);
        acc = fmaf(-sm.B.R[t][c], AR[m][r], acc);
        if (f.gain == GDR_GAIN_SCALAR && t < n && c < Dk)
          acck = fmaf(ld_f(k, rowk0 + static_cast<long long>(t) * H * Dk + c), AE[m][r], acck);
      }
      pg[r] = acc;
      pk[r] = acck;
    }
  #pragma unroll
    for (int mm = 1; mm < 16; mm <<= 1)
  #pragma unroll
      for (int r = 0; r < 4; ++r) {
        pg[r] += __shfl_xor(pg[r], mm);
        pk[r] += __shfl_xor(pk[r], mm);
      }
    if (col == 0) {
  #pragma unroll
      for (int r = 0; r < 4; ++r) {
        dgs[hh][tr0 + r] = pg[r];
        pks[hh][tr0 + r] = pk[r];
      }
    }
    // block sums of <dS', S> and lambda
  #pragma unroll
    for (int mm = 1; mm < 64; mm <<= 1) {
      sdot += __shfl_xor(sdot, mm);
      lam += __shfl_xor(lam, mm);
    }
    if (lane == 0) {
      red[0][wave] = sdot;
      red[1][wave] = lam;
    }
    __syncthreads();
    if (tid < kCMax) {
      if (f.decay == GDR_DECAY_SCALAR) {
        // dlog_alpha_t = sum_{i >= t} dg_i inside the chunk
        float x = tid < n ? dgs[0][tid] + dgs[1][tid] : 0.f;
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
      if (f.gain == GDR_GAIN_SCALAR && tid < n) a.dbeta[tok(tid)] = pks[0][tid] + pks[1][tid] + vdx[tid];
    }
    // ---- chain rule to the variant's inputs, stores ------------------------------------
  #pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tr0 + r;
      if (t >= n) continue;
      const long long rowk = tok(t) * Dk;
      const float bt = f.gain == GDR_GAIN_SCALAR ? f.beta[tok(t)] : 0.f;
  #pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int c = chan(m);
        if (c >= Dk) continue;
        const float de = AE[m][r], dr = AR[m][r];
        a.dq[rowk + c] = AQ[m][r];
        float dkv;
        if (f.gain == GDR_GAIN_SCALAR) {
          dkv = bt * de;
        } else {
          dkv = ld_f(er, rowk + c) * de;
          a.derase[rowk + c] = ld_f(k, rowk + c) * de;
        }
        if (f.wkey != GDR_WKEY_SAME)   // (preconditioned: to the workspace, then through p_t)
          a.dwk[rowk + c] = dr;
        else
          dkv += dr;
        a.dk[rowk + c] = dkv;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Preconditioned write key (diagonal second-moment preconditioner, Preconditioned DeltaNet
// section 2b), per (batch, head, channel).  Forward: the accumulator h_t = rho h_{t-1} + k_t^2
// from pc_h_in (or pc_h0), p_t = 1 / (h_t / b_t + eps) with b_t = 1 - rho^(pc_t0 + t + 1), the
// write key r_t = k_t p_t; r and p go to the workspace.  Backward: with dr_t the write-key
// gradient of the kernels above, the accumulator's gradient H_t = a_t + rho H_{t+1},
// a_t = -(dr_t k_t p_t^2) / b_t (H past the end zero: the final accumulator is not in the
// loss), dk_t += dr_t p_t + 2 k_t H_t, and dL/dpc_h_in = rho H_0.
// Both recurrences are affine, so each runs as two parallel passes over the chunks (one
// workgroup per (chunk, head, batch), one thread per channel): the first takes every chunk's
// own sum from a zero start (the chunk's contribution to the accumulator at its end, or to H
// at its start); the second composes the sums of the chunks before it (after it, for H) into
// its start value, from loads all issued at once, and runs the chunk's tokens from there.
// ---------------------------------------------------------------------------------------
constexpr int kPcThreads = 128;   // channels (Dk <= 128)

__global__ void bwd_zero_kernel(float *p, long long n) {
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}
constexpr int kPcU = 16;          // tokens whose loads are issued together

template <typename IO>
__global__ __launch_bounds__(kPcThreads) void bwd_pc_keys_sum_kernel(BwdArgs a) {
  const ChunkArgs &f = a.f;
  const IO *__restrict__ k = static_cast<const IO *>(f.k);
  const int c = threadIdx.x, ci = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Dk = f.Dk, H = f.H, T = f.T, C = f.C;
  if (c >= Dk) return;
  const int t0 = ci * C, n = min(C, T - t0);
  float acc = 0.f;
  for (int u0 = 0; u0 < n; u0 += kPcU) {
    float kv[kPcU];
#pragma unroll
    for (int u = 0; u < kPcU; ++u)
      kv[u] = ld_f(k, ((static_cast<long long>(b) * T + t0 + min(u0 + u, n - 1)) * H + h) * Dk + c);
#pragma unroll
    for (int u = 0; u < kPcU; ++u)
      if (u0 + u < n) acc = fmaf(f.rho, acc, kv[u] * kv[u]);
  }
  a.Sg[((static_cast<long long>(b) * H + h) * a.NC + ci) * Dk + c] = acc;
}

template <typename IO>
__global__ __launch_bounds__(kPcThreads) void bwd_pc_keys_kernel(BwdArgs a) {
  const ChunkArgs &f = a.f;
  const IO *__restrict__ k = static_cast<const IO *>(f.k);
  const int c = threadIdx.x, ci = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Dk = f.Dk, H = f.H, T = f.T, C = f.C;
  if (c >= Dk) return;
  const long long sh = static_cast<long long>(b) * H + h;
  const int t0 = ci * C, n = min(C, T - t0);
  // the accumulator at this chunk's start: the chunks before it composed (each full, C tokens)
  float acc = f.pc_h_in != nullptr ? f.pc_h_in[sh * Dk + c] : f.h0;
  const float rc = expf(static_cast<float>(C) * f.log_rho);   // rho^C
  for (int j0 = 0; j0 < ci; j0 += kPcU) {
    float sv[kPcU];
#pragma unroll
    for (int u = 0; u < kPcU; ++u) sv[u] = a.Sg[(sh * a.NC + min(j0 + u, ci - 1)) * Dk + c];
#pragma unroll
    for (int u = 0; u < kPcU; ++u)
      if (j0 + u < ci) acc = fmaf(rc, acc, sv[u]);
  }
  for (int u0 = 0; u0 < n; u0 += kPcU) {
    float kv[kPcU];
#pragma unroll
    for (int u = 0; u < kPcU; ++u)
      kv[u] = ld_f(k, ((static_cast<long long>(b) * T + t0 + min(u0 + u, n - 1)) * H + h) * Dk + c);
#pragma unroll
    for (int u = 0; u < kPcU; ++u) {
      const int t = t0 + u0 + u;
      if (u0 + u < n) {
        acc = fmaf(f.rho, acc, kv[u] * kv[u]);
        const float bt = -expm1f(static_cast<float>(f.t0 + t + 1) * f.log_rho);
        const float p = 1.f / (acc / bt + f.eps);
        const long long o = ((static_cast<long long>(b) * T + t) * H + h) * Dk + c;
        a.Pk[o] = p;
        a.Rk[o] = kv[u] * p;
      }
    }
  }
}

// a_t = -(dr_t k_t p_t^2) / b_t of token t (o its element offset)
template <typename IO>
__device__ __forceinline__ float pc_local_grad(const BwdArgs &a, const IO *k, long long o, int t, float &kt,
                                               float &pt, float &gt) {
  kt = ld_f(k, o);
  pt = a.Pk[o];
  gt = a.dRk[o];
  const float bt = -expm1f(static_cast<float>(a.f.t0 + t + 1) * a.f.log_rho);
  return -(gt * kt * pt * pt) / bt;
}

template <typename IO>
__global__ __launch_bounds__(kPcThreads) void bwd_pc_grad_sum_kernel(BwdArgs a) {
  const ChunkArgs &f = a.f;
  const IO *__restrict__ k = static_cast<const IO *>(f.k);
  const int c = threadIdx.x, ci = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Dk = f.Dk, H = f.H, T = f.T, C = f.C;
  if (c >= Dk) return;
  const int t0 = ci * C, n = min(C, T - t0);
  float Hs = 0.f;   // H at the chunk's first token with nothing after the chunk
  for (int u1 = n; u1 > 0; u1 -= kPcU) {   // tokens u1 - kPcU .. u1 - 1 of the chunk, last first
    float av[kPcU];
#pragma unroll
    for (int u = 0; u < kPcU; ++u) {
      const int t = t0 + max(u1 - 1 - u, 0);
      float kt, pt, gt;
      av[u] = pc_local_grad(a, k, ((static_cast<long long>(b) * T + t) * H + h) * Dk + c, t, kt, pt, gt);
    }
#pragma unroll
    for (int u = 0; u < kPcU; ++u)
      if (u1 - 1 - u >= 0) Hs = fmaf(f.rho, Hs, av[u]);
  }
  a.Sg[((static_cast<long long>(b) * H + h) * a.NC + ci) * Dk + c] = Hs;
}

template <typename IO>
__global__ __launch_bounds__(kPcThreads) void bwd_pc_grad_kernel(BwdArgs a) {
  const ChunkArgs &f = a.f;
  const IO *__restrict__ k = static_cast<const IO *>(f.k);
  const int c = threadIdx.x, ci = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Dk = f.Dk, H = f.H, T = f.T, C = f.C, NC = a.NC;
  if (c >= Dk) return;
  const long long sh = static_cast<long long>(b) * H + h;
  const int t0 = ci * C, n = min(C, T - t0);
  // H at the first token after this chunk: the chunks after it composed, last first (every
  // chunk full but the last, of T - (NC - 1) C tokens)
  float Hs = 0.f;
  const float rc = expf(static_cast<float>(C) * f.log_rho);
  const float rl = expf(static_cast<float>(T - (NC - 1) * C) * f.log_rho);
  for (int j1 = NC - 1; j1 > ci; j1 -= kPcU) {   // chunks j1 - kPcU + 1 .. j1, last first
    float sv[kPcU];
#pragma unroll
    for (int u = 0; u < kPcU; ++u) sv[u] = a.Sg[(sh * NC + max(j1 - u, ci + 1)) * Dk + c];
#pragma unroll
    for (int u = 0; u < kPcU; ++u) {
      const int j = j1 - u;
      if (j > ci) Hs = fmaf(j == NC - 1 ? rl : rc, Hs, sv[u]);
    }
  }
  for (int u1 = n; u1 > 0; u1 -= kPcU) {
    float av[kPcU], kv[kPcU], pv[kPcU], gv[kPcU], dk0[kPcU];
#pragma unroll
    for (int u = 0; u < kPcU; ++u) {
      const int t = t0 + max(u1 - 1 - u, 0);
      const long long o = ((static_cast<long long>(b) * T + t) * H + h) * Dk + c;
      av[u] = pc_local_grad(a, k, o, t, kv[u], pv[u], gv[u]);
      dk0[u] = a.dk[o];
    }
#pragma unroll
    for (int u = 0; u < kPcU; ++u) {
      const int t = t0 + u1 - 1 - u;
      if (u1 - 1 - u >= 0) {
        Hs = fmaf(f.rho, Hs, av[u]);
        a.dk[((static_cast<long long>(b) * T + t) * H + h) * Dk + c] = dk0[u] + gv[u] * pv[u] + 2.f * kv[u] * Hs;
      }
    }
  }
  if (ci == 0 && a.dpc_h_in != nullptr) a.dpc_h_in[sh * Dk + c] = f.rho * Hs;
}

// calls fn with std::true_type for the preconditioned write key, std::false_type otherwise
template <typename F>
void launch_pc(const BwdArgs &a, F &&fn) {
  if (a.f.wkey == GDR_WKEY_DIAG_PRECOND)
    fn(std::true_type{});
  else
    fn(std::false_type{});
}

// the kernels' four-element loads (V4): Dk and Dv multiples of 4 and every tensor they read that
// way 16-byte aligned (the workspace sections are 256-byte aligned from the workspace's base)
static bool vec4_ok(const BwdArgs &a) {
  const ChunkArgs &f = a.f;
  if (f.Dk % 4 != 0 || f.Dv % 4 != 0) return false;
  const void *ps[] = {f.q, f.k, f.v, f.erase, f.write, f.write_key, a.dout, a.Tw, a.Pw, a.Gw, a.Rk, a.Ww, a.Uw};
  for (const void *p : ps)
    if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return false;
  return true;
}

// the sequential kernels at Dk = 128: four-element loads when vec4_ok, and 16-row value tiles
// when 32-row ones would give at most 128 workgroups (half the CUs idle)
template <typename F>
void dispatch_v4_bv(const BwdArgs &a, F &&go) {
  const long long tiles32 = static_cast<long long>(a.f.B) * a.f.H * ((a.f.Dv + 31) / 32);
  const bool half = tiles32 <= 128;
  const bool v4 = vec4_ok(a);
  if (half) {
    if (v4) go(std::true_type{}, std::integral_constant<int, 16>{});
    else go(std::false_type{}, std::integral_constant<int, 16>{});
  } else {
    if (v4) go(std::true_type{}, std::integral_constant<int, 32>{});
    else go(std::false_type{}, std::integral_constant<int, 32>{});
  }
}

// launch_pc with a second flag, the band-limited T (never with the per-channel decay: the host
// rejects that combination, and no such kernel is built)
template <bool CHD, typename F>
void launch_var(const BwdArgs &a, F &&fn) {
  launch_pc(a, [&](auto pc) {
    if constexpr (!CHD) {
      if (a.f.N >= 0) {
        fn(pc, std::true_type{});
        return;
      }
    }
    fn(pc, std::false_type{});
  });
}

template <typename IO>
hipError_t prep_state_io(const BwdArgs &a, hipStream_t s) {
  if (a.NC == 0) return hipSuccess;
  const dim3 gp(a.NC, a.f.H, a.f.B);
  const bool chd = a.f.decay == GDR_DECAY_CHANNEL;
  if (a.f.Dk <= 64) {
    if (chd)
      launch_pc(a, [&](auto pc) { hipLaunchKernelGGL((bwd_prep_kernel<IO, 64, true, decltype(pc)::value>), gp, dim3(kPrThreads), 0, s, a); });
    else
      launch_pc(a, [&](auto pc) { hipLaunchKernelGGL((bwd_prep_kernel<IO, 64, false, decltype(pc)::value>), gp, dim3(kPrThreads), 0, s, a); });
  } else {
    if (chd)
      launch_pc(a, [&](auto pc) { hipLaunchKernelGGL((bwd_prep_kernel<IO, 128, true, decltype(pc)::value>), gp, dim3(kPrThreads), 0, s, a); });
    else
      launch_pc(a, [&](auto pc) { hipLaunchKernelGGL((bwd_prep_kernel<IO, 128, false, decltype(pc)::value>), gp, dim3(kPrThreads), 0, s, a); });
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 gs((a.f.Dv + kStBV - 1) / kStBV, a.f.H, a.f.B);   // (Dk <= 64)
  if (a.f.Dk <= 32) {
    if (chd)
      launch_pc(a, [&](auto pc) { hipLaunchKernelGGL((bwd_state_kernel<IO, 32, true, decltype(pc)::value, false, kStBV>), gs, dim3(kStThreads), 0, s, a); });
    else
      launch_pc(a, [&](auto pc) { hipLaunchKernelGGL((bwd_state_kernel<IO, 32, false, decltype(pc)::value, false, kStBV>), gs, dim3(kStThreads), 0, s, a); });
  } else if (a.f.Dk <= 64) {
    if (chd)
      launch_pc(a, [&](auto pc) { hipLaunchKernelGGL((bwd_state_kernel<IO, 64, true, decltype(pc)::value, false, kStBV>), gs, dim3(kStThreads), 0, s, a); });
    else
      launch_pc(a, [&](auto pc) { hipLaunchKernelGGL((bwd_state_kernel<IO, 64, false, decltype(pc)::value, false, kStBV>), gs, dim3(kStThreads), 0, s, a); });
  } else {
    // Dk = 128: 16-row value tiles when 32-row ones would leave half the CUs without a
    // workgroup (at most 128 of them)
    auto go = [&](auto v4c, auto bvc) {
      constexpr bool V = decltype(v4c)::value;
      constexpr int BV = decltype(bvc)::value;
      const dim3 g((a.f.Dv + BV - 1) / BV, a.f.H, a.f.B);
      if (chd)
        launch_pc(a, [&](auto pc) { hipLaunchKernelGGL((bwd_state_kernel<IO, 128, true, decltype(pc)::value, V, BV>), g, dim3(kStThreads), 0, s, a); });
      else
        launch_pc(a, [&](auto pc) { hipLaunchKernelGGL((bwd_state_kernel<IO, 128, false, decltype(pc)::value, V, BV>), g, dim3(kStThreads), 0, s, a); });
    };
    dispatch_v4_bv(a, go);
  }
  return hipGetLastError();
}

template <typename IO>
hipError_t sweep_io(const BwdArgs &a, hipStream_t s) {
  const dim3 grid((a.f.Dv + kSwBV - 1) / kSwBV, a.f.H, a.f.B);   // (Dk <= 64)
  const bool chd = a.f.decay == GDR_DECAY_CHANNEL;
  if (a.f.Dk <= 32) {
    if (chd)
      launch_var<true>(a, [&](auto pc, auto bd) { hipLaunchKernelGGL((bwd_sweep_kernel<IO, 32, true, decltype(pc)::value, decltype(bd)::value, false, kSwBV>), grid, dim3(kSwThreads), 0, s, a); });
    else
      launch_var<false>(a, [&](auto pc, auto bd) { hipLaunchKernelGGL((bwd_sweep_kernel<IO, 32, false, decltype(pc)::value, decltype(bd)::value, false, kSwBV>), grid, dim3(kSwThreads), 0, s, a); });
  } else if (a.f.Dk <= 64) {
    if (chd)
      launch_var<true>(a, [&](auto pc, auto bd) { hipLaunchKernelGGL((bwd_sweep_kernel<IO, 64, true, decltype(pc)::value, decltype(bd)::value, false, kSwBV>), grid, dim3(kSwThreads), 0, s, a); });
    else
      launch_var<false>(a, [&](auto pc, auto bd) { hipLaunchKernelGGL((bwd_sweep_kernel<IO, 64, false, decltype(pc)::value, decltype(bd)::value, false, kSwBV>), grid, dim3(kSwThreads), 0, s, a); });
  } else {
    auto go = [&](auto v4c, auto bvc) {
      constexpr bool V = decltype(v4c)::value;
      constexpr int BV = decltype(bvc)::value;
      const dim3 g((a.f.Dv + BV - 1) / BV, a.f.H, a.f.B);
      if (chd)
        launch_var<true>(a, [&](auto pc, auto bd) { hipLaunchKernelGGL((bwd_sweep_kernel<IO, 128, true, decltype(pc)::value, decltype(bd)::value, V, BV>), g, dim3(kSwThreads), 0, s, a); });
      else
        launch_var<false>(a, [&](auto pc, auto bd) { hipLaunchKernelGGL((bwd_sweep_kernel<IO, 128, false, decltype(pc)::value, decltype(bd)::value, V, BV>), g, dim3(kSwThreads), 0, s, a); });
    };
    dispatch_v4_bv(a, go);
  }
  return hipGetLastError();
}

template <typename IO>
hipError_t chunk_io(const BwdArgs &a, hipStream_t s) {
  if (a.NC == 0) return hipSuccess;
  const dim3 grid(a.NC, a.f.H, a.f.B);
  const bool chd = a.f.decay == GDR_DECAY_CHANNEL;
  if (a.f.Dk <= 64) {
    if (chd)
      launch_var<true>(a, [&](auto pc, auto bd) { hipLaunchKernelGGL((bwd_chunk_kernel<IO, 64, true, decltype(pc)::value, decltype(bd)::value>), grid, dim3(kCkThreads), 0, s, a); });
    else
      launch_var<false>(a, [&](auto pc, auto bd) { hipLaunchKernelGGL((bwd_chunk_kernel<IO, 64, false, decltype(pc)::value, decltype(bd)::value>), grid, dim3(kCkThreads), 0, s, a); });
  } else {
    if (chd)
      launch_var<true>(a, [&](auto pc, auto bd) { hipLaunchKernelGGL((bwd_chunk_kernel<IO, 128, true, decltype(pc)::value, decltype(bd)::value>), grid, dim3(kCkThreads), 0, s, a); });
    else
      launch_var<false>(a, [&](auto pc, auto bd) { hipLaunchKernelGGL((bwd_chunk_kernel<IO, 128, false, decltype(pc)::value, decltype(bd)::value>), grid, dim3(kCkThreads), 0, s, a); });
  }
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

template <typename IO>
hipError_t pc_keys_io(const BwdArgs &a, hipStream_t s) {
  const dim3 grid(a.NC, a.f.H, a.f.B);
  hipLaunchKernelGGL((bwd_pc_keys_sum_kernel<IO>), grid, dim3(kPcThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_pc_keys_kernel<IO>), grid, dim3(kPcThreads), 0, s, a);
  return hipGetLastError();
}

template <typename IO>
hipError_t pc_grad_io(const BwdArgs &a, hipStream_t s) {
  if (a.NC == 0) {   // T = 0: the accumulator reaches no output
    if (a.dpc_h_in == nullptr) return hipSuccess;
    const long long nz = static_cast<long long>(a.f.B) * a.f.H * a.f.Dk;
    hipLaunchKernelGGL(bwd_zero_kernel, dim3(static_cast<unsigned>((nz + 255) / 256)), dim3(256), 0, s,
                       a.dpc_h_in, nz);
    return hipGetLastError();
  }
  const dim3 grid(a.NC, a.f.H, a.f.B);
  hipLaunchKernelGGL((bwd_pc_grad_sum_kernel<IO>), grid, dim3(kPcThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_pc_grad_kernel<IO>), grid, dim3(kPcThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_pc_keys(const BwdArgs &a, int io_dtype, hipStream_t s) {
  return io_dtype == GDR_BF16 ? pc_keys_io<uint16_t>(a, s) : pc_keys_io<float>(a, s);
}

hipError_t launch_bwd_pc_grad(const BwdArgs &a, int io_dtype, hipStream_t s) {
  return io_dtype == GDR_BF16 ? pc_grad_io<uint16_t>(a, s) : pc_grad_io<float>(a, s);
}

}  // namespace gdr
