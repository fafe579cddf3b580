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
//   T      = (I - A)^-1 by forward substitution, column by column; entry order
//            acc = 0; for l = j .. i-1: acc = fma(A_il, T_lj, acc)
//            With a band limit N only entries with i - j <= N are formed (they use only
//            band entries of A: Lemma 3.1 of the same summary, Metodologia 1-2), so
//            N >= n - 1 runs exactly the same instructions as the exact path.
//   D      = T X                                     (= U - W S^T of the WY form)
//   P_ij   = exp(g_i - g_j) (q_i . r_j)              for j <= i
//   O      = scale ((e^g (.) Q) S^T + P D)
//   S      <- e^{g_n} S + D^T (e^{g_n - g} (.) R)
#include "common.h"

namespace gdr {
namespace {

constexpr int kThreads = 256;
constexpr int kBV = 16;     // state rows per workgroup
constexpr int kCMax = 64;   // largest chunk

// dot product of two zero-padded DK-long LDS rows: four partial sums (shorter dependency
// chains; the padding beyond Dk is zero on both sides, so it adds nothing)
template <int DK>
__device__ __forceinline__ float dotrow(const float *x, const float *y) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
  for (int c = 0; c < DK; c += 4) {
    s0 = fmaf(x[c], y[c], s0);
    s1 = fmaf(x[c + 1], y[c + 1], s1);
    s2 = fmaf(x[c + 2], y[c + 2], s2);
    s3 = fmaf(x[c + 3], y[c + 3], s3);
  }
  return (s0 + s1) + (s2 + s3);
}

template <typename IO, int DK>
__global__ __launch_bounds__(kThreads) void chunk_generic_kernel(ChunkArgs a) {
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

  __shared__ float Rs[kCMax][DK + 1];     // write keys r
  __shared__ float Xs[kCMax][DK + 1];     // erase keys e, then queries q
  __shared__ float LT[kCMax][kCMax + 1];  // L (strict lower) | T^T (strict upper) | P (lower)
  __shared__ float Ss[kBV][DK + 1];       // state tile
  __shared__ float Xv[kCMax][kBV];        // X
  __shared__ float Dl[kCMax][kBV];        // D
  __shared__ float gs[kCMax], eg[kCMax], wd[kCMax];

  const long long sh = static_cast<long long>(b) * H + h;  // (b, h) index
  for (int idx = tid; idx < kBV * DK; idx += kThreads) {
    const int r = idx / DK, c = idx % DK;
    float s = 0.f;
    if (a.state_in != nullptr && r < nv && c < Dk) s = a.state_in[(sh * Dv + v0 + r) * Dk + c];
    Ss[r][c] = s;
  }
  float hreg = 0.f;  // preconditioner accumulator of channel `tid`
  if (a.wkey == GDR_WKEY_DIAG_PRECOND && tid < Dk)
    hreg = a.pc_h_in != nullptr ? a.pc_h_in[sh * Dk + tid] : a.h0;

  for (int c0 = 0; c0 < T; c0 += a.C) {
    const int n = min(a.C, T - c0);
    // token (b, c0 + t, h) row index in [B, T, H]
    auto tok = [&](int t) -> long long { return (static_cast<long long>(b) * T + c0 + t) * H + h; };

    __syncthreads();  // previous chunk done with every buffer
    if (tid < n) gs[tid] = (a.decay == GDR_DECAY_SCALAR) ? a.log_alpha[tok(tid)] : 0.f;
    // write keys
    if (a.wkey == GDR_WKEY_DIAG_PRECOND) {
      if (tid < Dk) {
        for (int t = 0; t < n; ++t) {
          const float kk = ld_f(k, tok(t) * Dk + tid);
          hreg = fmaf(a.rho, hreg, kk * kk);
          const float tg = static_cast<float>(a.t0 + c0 + t + 1);
          const float corr = -expm1f(tg * a.log_rho);  // 1 - rho^t
          Rs[t][tid] = kk / (hreg / corr + a.eps);
        }
      } else if (tid < DK) {
        for (int t = 0; t < n; ++t) Rs[t][tid] = 0.f;
      }
    } else {
      const IO *src = (a.wkey == GDR_WKEY_EXPLICIT) ? wk : k;
      for (int idx = tid; idx < n * DK; idx += kThreads) {
        const int t = idx / DK, c = idx % DK;
        Rs[t][c] = c < Dk ? ld_f(src, tok(t) * Dk + c) : 0.f;
      }
    }
    // erase keys
    for (int idx = tid; idx < n * DK; idx += kThreads) {
      const int t = idx / DK, c = idx % DK;
      float e = 0.f;
      if (c < Dk) {
        const float kk = ld_f(k, tok(t) * Dk + c);
        e = (a.gain == GDR_GAIN_SCALAR) ? a.beta[tok(t)] * kk : ld_f(er, tok(t) * Dk + c) * kk;
      }
      Xs[t][c] = e;
    }
    __syncthreads();
    if (tid == 0) {
      float acc = 0.f;
      for (int t = 0; t < n; ++t) {
        acc += gs[t];
        gs[t] = acc;
      }
    }
    __syncthreads();
    if (tid < n) {
      eg[tid] = expf(gs[tid]);
      wd[tid] = expf(gs[n - 1] - gs[tid]);
    }
    // L (strict lower)
    for (int idx = tid; idx < n * n; idx += kThreads) {
      const int i = idx / n, j = idx % n;
      if (j < i) {
        const float dot = dotrow<DK>(Xs[i], Rs[j]);
        LT[i][j] = expf(gs[i] - gs[j]) * dot;
      }
    }
    // X = V' - (e^g (.) E) S^T on the value tile
    for (int idx = tid; idx < n * kBV; idx += kThreads) {
      const int t = idx / kBV, r = idx % kBV;
      float x = 0.f;
      if (r < nv) {
        const float dot = dotrow<DK>(Xs[t], Ss[r]);
        const long long vi = tok(t) * Dv + v0 + r;
        const float vv = ld_f(v, vi);
        const float vp = (a.gain == GDR_GAIN_SCALAR) ? a.beta[tok(t)] * vv : ld_f(wr, vi) * vv;
        x = vp - expf(gs[t]) * dot;
      }
      Xv[t][r] = x;
    }
    __syncthreads();
    // T = (I - A)^-1, T_ij (i > j) stored at LT[j][i].  Right-looking order: thread
    // (row i = tid / 4, columns 16 (tid % 4) .. + 15) adds the term A_il T_lj to T_ij at step
    // l = j .. i - 1, so every entry sums its terms in the same order as column-by-column
    // forward substitution (acc = 0; for l = j .. i-1: acc = fma(A_il, T_lj, acc)), but the
    // steps run over all rows and columns at once; row l + 1 is final after step l and is
    // published before the next step reads it.  Band entries (i - j > N) stay zero.
    {
      static_assert(kThreads == 4 * kCMax, "one thread per (row, 16-column group)");
      const int i = tid >> 2, jg = (tid & 3) * 16;
      float acc[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[q] = 0.f;
      for (int l = 0; l + 1 < n; ++l) {
        if (i > l && i < n) {
          const float A_il = -LT[i][l];
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int j = jg + q;
            if (j <= l && (a.N < 0 || i - j <= a.N)) {
              const float T_lj = (j == l) ? 1.f : LT[j][l];
              acc[q] = fmaf(A_il, T_lj, acc[q]);
            }
          }
        }
        if (i == l + 1) {
#pragma unroll
          for (int q = 0; q < 16; ++q)
            if (jg + q < i) LT[jg + q][i] = acc[q];
        }
        __syncthreads();
      }
    }
    // queries replace the erase keys (last read before the barrier above)
    for (int idx = tid; idx < n * DK; idx += kThreads) {
      const int t = idx / DK, c = idx % DK;
      Xs[t][c] = c < Dk ? ld_f(q, tok(t) * Dk + c) : 0.f;
    }
    __syncthreads();
    // D = T X  (reads the strict upper part of LT)
    for (int idx = tid; idx < n * kBV; idx += kThreads) {
      const int t = idx / kBV, r = idx % kBV;
      float acc = Xv[t][r];
      #pragma unroll 8
      for (int s = 0; s < t; ++s) acc = fmaf(LT[s][t], Xv[s][r], acc);
      Dl[t][r] = acc;
    }
    // P (lower incl. diagonal; disjoint from the strict upper part read above)
    for (int idx = tid; idx < n * n; idx += kThreads) {
      const int i = idx / n, j = idx % n;
      if (j <= i) {
        const float dot = dotrow<DK>(Xs[i], Rs[j]);
        LT[i][j] = expf(gs[i] - gs[j]) * dot;
      }
    }
    __syncthreads();
    // O = scale ((e^g (.) Q) S^T + P D)
    for (int idx = tid; idx < n * kBV; idx += kThreads) {
      const int t = idx / kBV, r = idx % kBV;
      if (r < nv) {
        const float dot = dotrow<DK>(Xs[t], Ss[r]);
        float acc = eg[t] * dot;
        #pragma unroll 8
        for (int j = 0; j <= t; ++j) acc = fmaf(LT[t][j], Dl[j][r], acc);
        st_f(out, tok(t) * Dv + v0 + r, a.scale * acc);
      }
    }
    __syncthreads();
    // S <- e^{g_n} S + D^T (e^{g_n - g} (.) R)
    const float gl = eg[n - 1];
    for (int idx = tid; idx < kBV * DK; idx += kThreads) {
      const int r = idx / DK, c = idx % DK;
      if (r < nv && c < Dk) {
        float acc = gl * Ss[r][c];
        #pragma unroll 8
        for (int j = 0; j < n; ++j) acc = fmaf(Dl[j][r] * wd[j], Rs[j][c], acc);
        Ss[r][c] = acc;
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

template <typename IO>
hipError_t launch_io(const ChunkArgs &a, hipStream_t s) {
  const dim3 grid((a.Dv + kBV - 1) / kBV, a.H, a.B);
  if (a.Dk <= 32)
    hipLaunchKernelGGL((chunk_generic_kernel<IO, 32>), grid, dim3(kThreads), 0, s, a);
  else if (a.Dk <= 64)
    hipLaunchKernelGGL((chunk_generic_kernel<IO, 64>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((chunk_generic_kernel<IO, 128>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_generic(const ChunkArgs &a, int io_dtype, hipStream_t s) {
  return io_dtype == GDR_BF16 ? launch_io<uint16_t>(a, s) : launch_io<float>(a, s);
}

}  // namespace gdr
