// Fused chunk-parallel gated delta-rule forward on the gfx950 matrix cores (bf16 in,
// fp32 accumulate, fp32 state), for Dk = Dv = 128 and chunks of 64 tokens.
//
// One workgroup (8 wave64s) owns one (batch, head, value tile of BV state rows) and
// walks the sequence chunk by chunk.  The state tile S (BV x 128, fp32) lives in MFMA
// accumulator registers for the whole sequence; a bf16 copy in LDS feeds the products
// that read it.  Nothing but the inputs, the output and the final state touches HBM.
//
// Per chunk of 64 tokens (chunk-wise form of the MatMul-only inversion summary,
// "Declaracao do Problema"; the WY correction U - W S^T is evaluated here as
// T (V' - (e^g (.) E) S^T), the same product regrouped so that only one 64 x BV
// right-hand side meets T):
//   g       inclusive cumulative sum of log alpha (kept in log2 units for exp2)
//   L       = tril_{-1}((E R^T) (.) Gamma)                        [MFMA, fp32 in LDS]
//   T       = (I + L)^-1 = (I - A)^-1                             [see below]
//   P       = tril(Q R^T) (.) Gamma                               [MFMA]
//   X       = V' - (e^g (.) E) S^T                                [MFMA + epilogue]
//   D       = T X                                                 [MFMA]
//   O       = scale ((e^g (.) Q) S^T + P D)                       [MFMA]
//   S       <- e^{g_C} S + (e^{g_C - g} (.) D)^T R                [MFMA into the accumulators]
// T is built blockwise: the four 16 x 16 diagonal blocks by forward substitution on the
// vector ALUs (one lane per column), then two merge levels on the matrix cores using
// (I + L)^-1 = [[T_a, 0], [-T_b L_ba T_a, T_b]].  With a band limit N <= 15 (the
// truncated Neumann series with its diagonal mask, same summary, Metodologia 1-2, whose
// band equals the band of the exact inverse by Lemma 3.1) each lane forms its column's N
// sub-diagonal entries by the band-limited substitution instead; a larger N masks the
// exact inverse.
//
// MFMA operand layouts (v_mfma_f32_16x16x32_bf16): lane l supplies row (l % 16) of A
// and column (l % 16) of B, each as 8 consecutive K values starting at 8 * (l / 16);
// the 16 x 16 fp32 result sits in lane l as rows 4 * (l / 16) + r, column l % 16.
// Products that contract over tokens therefore read operands stored token-contiguous
// (R^T, X^T, D^T), which the loaders and epilogues write directly.
#include "common.h"

namespace gdr {
namespace {

typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kC = 64;            // chunk
constexpr int kD = 128;           // Dk = Dv
constexpr int kNW = 8;            // waves per workgroup
constexpr int kNT = kNW * 64;     // threads
constexpr int kLdr = kD + 8;      // bf16 row stride of [64][128] tiles (272 B)
constexpr int kLdc = kC + 8;      // bf16 row stride of [*][64] tiles (144 B)
constexpr int kLda = kC + 4;      // fp32 row stride of L
constexpr float kLog2e = 1.4426950408889634f;

enum : int { kWkSame = 0, kWkPrecond = 1, kWkExplicit = 2 };

template <int BV, bool CHAN, int WK>
struct __align__(16) Smem {
  uint16_t q[kC][kLdr];
  uint16_t k[kC][kLdr];
  uint16_t r[WK != kWkSame ? kC : 1][kLdr];   // write key when it differs from k
  uint16_t e[CHAN ? kC : 1][kLdr];            // erase key b (.) k (channel gain)
  uint16_t rt[kD][kLdc];                      // R^T
  uint16_t t[kC][kLdc];                       // T (bf16)
  uint16_t p[kC][kLdc];                       // P (bf16)
  uint16_t s[BV][kLdr];                       // state copy (bf16)
  uint16_t xt[BV][kLdc];                      // X^T
  uint16_t dt[BV][kLdc];                      // D^T
  uint16_t dt2[BV][kLdc];                     // (e^{g_C - g} D)^T
  float a[kC][kLda];                          // L (fp32)
  float vp[kC][BV + 4];                       // V' tile (fp32)
  float o1[kC][BV + 4];                       // e^g (Q S^T) (fp32)
  float g2[kC], eg[kC], wd[kC], cy[kC], ic[kC], beta[kC];
};

__device__ __forceinline__ float bf(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
// element e (0..7) of 8 bf16 packed in a uint4, as a bit pattern / as fp32
__device__ __forceinline__ uint32_t word(const uint4 &v, int e) {
  const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}
__device__ __forceinline__ float elem(const uint4 &v, int e) { return bf(word(v, e)); }
// 16-byte global load, or zeros when !ok (no select of addresses: the zero is a value)
__device__ __forceinline__ uint4 ldg16(const uint16_t *p, bool ok) {
  uint4 r = make_uint4(0u, 0u, 0u, 0u);
  if (ok) r = *reinterpret_cast<const uint4 *>(p);
  return r;
}
__device__ __forceinline__ uint16_t tobf(float x) { return f32_to_bf16_bits(x); }

__device__ __forceinline__ float4v mfma32(short8v a, short8v b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4v mfma16(short4v a, short4v b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ short8v ld8(const uint16_t *p) {
  return *reinterpret_cast<const short8v *>(p);
}
__device__ __forceinline__ short4v ld4(const uint16_t *p) {
  return *reinterpret_cast<const short4v *>(p);
}
// 4 fp32 from LDS -> 4 bf16
__device__ __forceinline__ short4v ld4f(const float *p) {
  const float4 f = *reinterpret_cast<const float4 *>(p);
  short4v r;
  r[0] = static_cast<short>(tobf(f.x));
  r[1] = static_cast<short>(tobf(f.y));
  r[2] = static_cast<short>(tobf(f.z));
  r[3] = static_cast<short>(tobf(f.w));
  return r;
}
// 4 bf16 down a column (stride ld elements)
__device__ __forceinline__ short4v ld4col(const uint16_t *p, int ld) {
  short4v r;
  r[0] = static_cast<short>(p[0]);
  r[1] = static_cast<short>(p[ld]);
  r[2] = static_cast<short>(p[2 * ld]);
  r[3] = static_cast<short>(p[3 * ld]);
  return r;
}
__device__ __forceinline__ short4v tobf4(float4v v, float s = 1.f) {
  short4v r;
  r[0] = static_cast<short>(tobf(s * v[0]));
  r[1] = static_cast<short>(tobf(s * v[1]));
  r[2] = static_cast<short>(tobf(s * v[2]));
  r[3] = static_cast<short>(tobf(s * v[3]));
  return r;
}

// acc += A[m0.., :K] * B[n0.., :K]^T over K = 32 * nk columns starting at k0; A and B are
// row-major with K contiguous.
__device__ __forceinline__ float4v tile_mma(float4v acc, const uint16_t *A, int lda, const uint16_t *Bm,
                                           int ldb, int m0, int n0, int k0, int nk, int lane) {
  const uint16_t *pa = A + (m0 + (lane & 15)) * lda + k0 + 8 * (lane >> 4);
  const uint16_t *pb = Bm + (n0 + (lane & 15)) * ldb + k0 + 8 * (lane >> 4);
#pragma unroll 4
  for (int kk = 0; kk < nk; ++kk) acc = mfma32(ld8(pa + 32 * kk), ld8(pb + 32 * kk), acc);
  return acc;
}

template <int BV, bool CHAN, bool DECAY, int WK, bool BAND>
__global__ __launch_bounds__(kNT, 1) void chunk_mfma_kernel(ChunkArgs a) {
  constexpr int NVB = BV / 16;         // 16-row blocks of the value tile
  constexpr int NVT = kD / BV;         // value tiles per head
  constexpr int NST = NVB * 8;         // state tiles (16 x 16)
  constexpr int SPW = NST / kNW;       // state tiles per wave
  constexpr int NOT = 4 * NVB;         // output / X / D tiles
  static_assert(NST % kNW == 0, "state tiles must divide among waves");
  __shared__ Smem<BV, CHAN, WK> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15, l4 = lane >> 4;

  // XCD-aware tile order: consecutive logical tiles (the value tiles of one head) land
  // on the same XCD, whose L2 then serves the head's q/k reads to all of them.
  const int G = static_cast<int>(gridDim.x);
  const int bid = static_cast<int>(blockIdx.x);
  const int logical = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int bh = logical / NVT;
  const int vt = logical % NVT;
  const int v0 = vt * BV;
  const int H = a.H, T = a.T;
  const int b = bh / H, h = bh % H;
  const long long tokstride = static_cast<long long>(H) * kD;   // elements between tokens
  const long long head0 = (static_cast<long long>(b) * T * H + h) * kD;  // (b, 0, h, 0)
  const long long gate0 = static_cast<long long>(b) * T * H + h;         // (b, 0, h)

  const uint16_t *gq = static_cast<const uint16_t *>(a.q);
  const uint16_t *gk = static_cast<const uint16_t *>(a.k);
  const uint16_t *gv = static_cast<const uint16_t *>(a.v);
  const uint16_t *gwk = static_cast<const uint16_t *>(a.write_key);
  const uint16_t *ger = static_cast<const uint16_t *>(a.erase);
  const uint16_t *gwr = static_cast<const uint16_t *>(a.write);
  uint16_t *gout = static_cast<uint16_t *>(a.out);

  // ---- one-time LDS init: zero upper blocks of T and P; unit diagonal for band T ----
  for (int idx = tid; idx < kC * kLdc; idx += kNT) {
    const int i = idx / kLdc, j = idx % kLdc;
    (&sm.t[0][0])[idx] = (BAND && i == j) ? tobf(1.f) : 0;
    (&sm.p[0][0])[idx] = 0;
  }

  // ---- state tiles in accumulators ----
  float4v sacc[SPW];
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int st = wave + u * kNW;
    const int vb = st / 8, cb = st % 8;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int v = vb * 16 + 4 * l4 + r, c = cb * 16 + l16;
      float x = 0.f;
      if (a.state_in != nullptr) x = a.state_in[(static_cast<long long>(bh) * kD + v0 + v) * kD + c];
      sacc[u][r] = x;
      sm.s[v][c] = tobf(x);
    }
  }

  // preconditioner accumulator: 4 lanes per channel (token segments of 16)
  const int pc_c = tid >> 2, pc_seg = tid & 3;
  float hcarry = 0.f;
  if (WK == kWkPrecond) hcarry = a.pc_h_in != nullptr ? a.pc_h_in[static_cast<long long>(bh) * kD + pc_c] : a.h0;

  // ---- register prefetch of one chunk ----
  // q, k (and write key / erase gate): units of 8 bf16, 1024 per tensor, 2 per thread
  // v (and write gate) tile: 64 x BV, units of 8 bf16, 8 * BV units
  constexpr int VU = kC * BV / 8;
  uint4 pq[2], pk[2], pr[2], pe[2], pv, pw;
  float pbeta = 0.f, pla = 0.f, pvbeta = 0.f;
  auto prefetch = [&](int c0, int n) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int unit = tid + u * kNT;
      const int t = unit >> 4, col = (unit & 15) * 8;
      const long long off = head0 + static_cast<long long>(c0 + t) * tokstride + col;
      const bool ok = t < n;
      pq[u] = ldg16(gq + off, ok);
      pk[u] = ldg16(gk + off, ok);
      if (WK == kWkExplicit) pr[u] = ldg16(gwk + off, ok);
      if (CHAN) pe[u] = ldg16(ger + off, ok);
    }
    if (tid < VU) {
      const int t = tid / (BV / 8), col = (tid % (BV / 8)) * 8;
      const bool ok = t < n;
      const long long off = head0 + static_cast<long long>(c0 + t) * tokstride + v0 + col;
      pv = ldg16(gv + off, ok);
      if (CHAN) pw = ldg16(gwr + off, ok);
      if (!CHAN) pvbeta = ok ? a.beta[gate0 + static_cast<long long>(c0 + t) * H] : 0.f;
    }
    if (tid < kC) {
      const bool ok = tid < n;
      const long long gi = gate0 + static_cast<long long>(c0 + tid) * H;
      pbeta = (!CHAN && ok) ? a.beta[gi] : 0.f;
      pla = (DECAY && ok) ? a.log_alpha[gi] : 0.f;
    }
  };

  const int nchunks = (T + kC - 1) / kC;
  if (nchunks > 0) prefetch(0, min(kC, T));

  for (int ci = 0; ci < nchunks; ++ci) {
    const int c0 = ci * kC;
    const int n = min(kC, T - c0);
    __syncthreads();  // previous chunk done with every LDS buffer

    // ================= Phase L: prefetched registers -> LDS; gates =================
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int unit = tid + u * kNT;
      const int t = unit >> 4, col = (unit & 15) * 8;
      *reinterpret_cast<uint4 *>(&sm.q[t][col]) = pq[u];
      *reinterpret_cast<uint4 *>(&sm.k[t][col]) = pk[u];
      if (WK == kWkSame) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.rt[col + e][t] = static_cast<uint16_t>(word(pk[u], e));
      } else if (WK == kWkExplicit) {
        *reinterpret_cast<uint4 *>(&sm.r[t][col]) = pr[u];
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.rt[col + e][t] = static_cast<uint16_t>(word(pr[u], e));
      }
      if (CHAN) {
        uint4 ev;
        ev.x = tobf(elem(pe[u], 0) * elem(pk[u], 0)) | (uint32_t(tobf(elem(pe[u], 1) * elem(pk[u], 1))) << 16);
        ev.y = tobf(elem(pe[u], 2) * elem(pk[u], 2)) | (uint32_t(tobf(elem(pe[u], 3) * elem(pk[u], 3))) << 16);
        ev.z = tobf(elem(pe[u], 4) * elem(pk[u], 4)) | (uint32_t(tobf(elem(pe[u], 5) * elem(pk[u], 5))) << 16);
        ev.w = tobf(elem(pe[u], 6) * elem(pk[u], 6)) | (uint32_t(tobf(elem(pe[u], 7) * elem(pk[u], 7))) << 16);
        *reinterpret_cast<uint4 *>(&sm.e[t][col]) = ev;
      }
    }
    if (tid < VU) {
      const int t = tid / (BV / 8), col = (tid % (BV / 8)) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.vp[t][col + e] = CHAN ? elem(pw, e) * elem(pv, e) : pvbeta * elem(pv, e);
    }
    if (wave == 0) {
      // inclusive scan of log2(alpha) over the chunk (padded tokens add 0)
      float g = pla * kLog2e;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_up(g, d, 64);
        if (lane >= d) g += y;
      }
      const float glast = __shfl(g, n - 1, 64);
      const float egv = DECAY ? exp2f(g) : 1.f;
      sm.g2[lane] = g;
      sm.eg[lane] = egv;
      sm.wd[lane] = DECAY ? exp2f(glast - g) : 1.f;
      sm.cy[lane] = CHAN ? egv : pbeta * egv;
      sm.beta[lane] = pbeta;
      if (WK == kWkPrecond) {
        const float tg = static_cast<float>(a.t0 + c0 + lane + 1);
        sm.ic[lane] = 1.f / (-expm1f(tg * a.log_rho));   // 1 / (1 - rho^t)
      }
    }
    // issue the next chunk's loads; they land while this chunk computes
    if (ci + 1 < nchunks) prefetch(c0 + kC, min(kC, T - c0 - kC));
    __syncthreads();

    // ============ Phase U (preconditioner): u = k / (h / (1 - rho^t) + eps) ============
    if (WK == kWkPrecond) {
      // lanes (channel c, segment s) cover tokens 16 s .. 16 s + 15
      const int c = pc_c, s0 = pc_seg * 16;
      const int m = max(0, min(16, n - s0));   // valid tokens of this segment
      float hl[16], kv[16];
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        kv[i] = bf(sm.k[s0 + i][c]);
        if (i < m) acc = fmaf(a.rho, acc, kv[i] * kv[i]);
        hl[i] = acc;
      }
      // carry into segment s: compose the affine maps h -> rho^m h + acc of earlier segments
      float rm = 1.f;
      for (int i = 0; i < m; ++i) rm *= a.rho;
      const int base = lane & ~3;
      float cin = hcarry, cend = hcarry;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float ms = __shfl(rm, base + s, 64);
        const float as = __shfl(acc, base + s, 64);
        if (s < pc_seg) cin = fmaf(ms, cin, as);
        cend = fmaf(ms, cend, as);
      }
      float pw = a.rho;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float u = 0.f;
        if (i < m) {
          const float hv = fmaf(pw, cin, hl[i]);
          u = kv[i] / fmaf(hv, sm.ic[s0 + i], a.eps);
        }
        pw *= a.rho;
        const uint16_t ub = tobf(u);
        sm.r[s0 + i][c] = ub;
        sm.rt[c][s0 + i] = ub;
      }
      hcarry = cend;
      __syncthreads();
    }

    const uint16_t *Ea = CHAN ? &sm.e[0][0] : &sm.k[0][0];                // erase key rows
    const uint16_t *Rr = (WK == kWkSame) ? &sm.k[0][0] : &sm.r[0][0];    // write key rows

    // ================= Phase A: L = tril_{-1}((E R^T) (.) Gamma) =================
    for (int job = wave; job < 10; job += kNW) {
      // lower-triangular tile index -> (ib, jb)
      const int ib = job < 1 ? 0 : job < 3 ? 1 : job < 6 ? 2 : 3;
      const int jb = job - ib * (ib + 1) / 2;
      float4v acc = {0.f, 0.f, 0.f, 0.f};
      acc = tile_mma(acc, Ea, kLdr, Rr, kLdr, ib * 16, jb * 16, 0, 4, lane);
      const int j = jb * 16 + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = ib * 16 + 4 * l4 + r;
        float x = acc[r];
        if (!CHAN) x *= sm.beta[i];
        if (DECAY) x *= exp2f(sm.g2[i] - sm.g2[j]);
        sm.a[i][j] = (j < i) ? x : 0.f;
      }
    }
    __syncthreads();

    // ===== Phase B: diagonal blocks of T (wave 0)  ||  P, X, O1 (other waves) =====
    if (wave == 0) {
      if (!BAND) {
        // lane = (block, column): forward substitution down the column of a 16x16 block
        const int blk = l4, j = l16, o = blk * 16;
        float tv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) tv[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 1; i < 16; ++i) {
          float acc = 0.f;
#pragma unroll
          for (int m = 0; m < i; ++m) acc = fmaf(sm.a[o + i][o + m], tv[m], acc);
          if (i > j) tv[i] = -acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bool keep = (i - j) <= a.N || a.N < 0;
          sm.t[o + i][o + j] = (i >= j && keep) ? tobf(tv[i]) : 0;
        }
      } else {
        // band-limited substitution: lane j forms T_{j+d, j}, d = 1..N (N <= 15)
        const int j = lane;
        float tc[16];
        tc[0] = 1.f;
#pragma unroll
        for (int d = 1; d < 16; ++d) {
          float acc = 0.f;
          if (d <= a.N && j + d < kC) {
#pragma unroll
            for (int m = 0; m < d; ++m) acc = fmaf(-sm.a[j + d][j + m], tc[m], acc);
            sm.t[j + d][j] = tobf(acc);
          }
          tc[d] = acc;
        }
      }
    } else {
      constexpr int NJ = 10 + 2 * NOT;
      for (int job = wave - 1; job < NJ; job += kNW - 1) {
        if (job < 10) {
          // P tile
          const int ib = job < 1 ? 0 : job < 3 ? 1 : job < 6 ? 2 : 3;
          const int jb = job - ib * (ib + 1) / 2;
          float4v acc = {0.f, 0.f, 0.f, 0.f};
          acc = tile_mma(acc, &sm.q[0][0], kLdr, Rr, kLdr, ib * 16, jb * 16, 0, 4, lane);
          const int j = jb * 16 + l16;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = ib * 16 + 4 * l4 + r;
            float x = acc[r];
            if (DECAY) x *= exp2f(sm.g2[i] - sm.g2[j]);
            sm.p[i][j] = (j <= i) ? tobf(x) : 0;
          }
        } else if (job < 10 + NOT) {
          // X tile: X = V' - cy (.) (E S^T), stored transposed
          const int o = job - 10, tb = o / NVB, vb = o % NVB;
          float4v acc = {0.f, 0.f, 0.f, 0.f};
          acc = tile_mma(acc, Ea, kLdr, &sm.s[0][0], kLdr, tb * 16, vb * 16, 0, 4, lane);
          const int v = vb * 16 + l16;
          short4v xv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = tb * 16 + 4 * l4 + r;
            xv[r] = static_cast<short>(tobf(sm.vp[t][v] - sm.cy[t] * acc[r]));
          }
          *reinterpret_cast<short4v *>(&sm.xt[v][tb * 16 + 4 * l4]) = xv;
        } else {
          // O1 tile: e^g (.) (Q S^T)
          const int o = job - 10 - NOT, tb = o / NVB, vb = o % NVB;
          float4v acc = {0.f, 0.f, 0.f, 0.f};
          acc = tile_mma(acc, &sm.q[0][0], kLdr, &sm.s[0][0], kLdr, tb * 16, vb * 16, 0, 4, lane);
          const int v = vb * 16 + l16;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = tb * 16 + 4 * l4 + r;
            sm.o1[t][v] = sm.eg[t] * acc[r];
          }
        }
      }
    }
    __syncthreads();

    if (!BAND) {
      // ============ Phase R1: T_{p,q} = -D_p (L_{p,q} D_q) for (p,q) = (1,0), (3,2) ============
      if (wave < 2) {
        const int p = 1 + 2 * wave, q = p - 1;
        float4v z = {0.f, 0.f, 0.f, 0.f};
        z = mfma16(ld4f(&sm.a[p * 16 + l16][q * 16 + 4 * l4]),
                   ld4col(&sm.t[q * 16 + 4 * l4][q * 16 + l16], kLdc), z);
        float4v tt = {0.f, 0.f, 0.f, 0.f};
        tt = mfma16(ld4(&sm.t[p * 16 + l16][p * 16 + 4 * l4]), tobf4(z), tt);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = p * 16 + 4 * l4 + r, j = q * 16 + l16;
          const bool keep = (i - j) <= a.N || a.N < 0;
          sm.t[i][j] = keep ? tobf(-tt[r]) : 0;
        }
      }
      __syncthreads();
      // ==== Phase R2: T_ba = -T_b (L_ba T_a), rows 32..63, columns 0..31; wave q: 16-col block q ====
      if (wave < 2) {
        const int q = wave;
        float4v z[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          z[s] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            if (u < q) continue;   // T_a[u][q] = 0 above the diagonal
            z[s] = mfma16(ld4f(&sm.a[32 + s * 16 + l16][u * 16 + 4 * l4]),
                          ld4col(&sm.t[u * 16 + 4 * l4][q * 16 + l16], kLdc), z[s]);
          }
        }
        const short4v z0 = tobf4(z[0]), z1 = tobf4(z[1]);
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          float4v tt = {0.f, 0.f, 0.f, 0.f};
          tt = mfma16(ld4(&sm.t[32 + sp * 16 + l16][32 + 4 * l4]), z0, tt);
          if (sp == 1) tt = mfma16(ld4(&sm.t[48 + l16][48 + 4 * l4]), z1, tt);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 32 + sp * 16 + 4 * l4 + r, j = q * 16 + l16;
            const bool keep = (i - j) <= a.N || a.N < 0;
            sm.t[i][j] = keep ? tobf(-tt[r]) : 0;
          }
        }
      }
      __syncthreads();
    }

    // ================= Phase D: D = T X  ->  D^T, (e^{g_C - g} D)^T =================
    for (int o = wave; o < NOT; o += kNW) {
      const int tb = o / NVB, vb = o % NVB;
      float4v acc = {0.f, 0.f, 0.f, 0.f};
      acc = tile_mma(acc, &sm.t[0][0], kLdc, &sm.xt[0][0], kLdc, tb * 16, vb * 16, 0, tb < 2 ? 1 : 2, lane);
      const int v = vb * 16 + l16;
      short4v d1, d2;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tb * 16 + 4 * l4 + r;
        d1[r] = static_cast<short>(tobf(acc[r]));
        d2[r] = static_cast<short>(tobf(sm.wd[t] * acc[r]));
      }
      *reinterpret_cast<short4v *>(&sm.dt[v][tb * 16 + 4 * l4]) = d1;
      *reinterpret_cast<short4v *>(&sm.dt2[v][tb * 16 + 4 * l4]) = d2;
    }
    __syncthreads();

    // ============ Phase H: O = scale (O1 + P D) -> HBM;  S <- e^{g_C} S + D~^T R ============
    for (int o = wave; o < NOT; o += kNW) {
      const int tb = o / NVB, vb = o % NVB;
      float4v acc = {0.f, 0.f, 0.f, 0.f};
      acc = tile_mma(acc, &sm.p[0][0], kLdc, &sm.dt[0][0], kLdc, tb * 16, vb * 16, 0, tb < 2 ? 1 : 2, lane);
      const int v = vb * 16 + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tb * 16 + 4 * l4 + r;
        if (t < n)
          gout[head0 + static_cast<long long>(c0 + t) * tokstride + v0 + v] =
              tobf(a.scale * (sm.o1[t][v] + acc[r]));
      }
    }
    {
      const float gC = DECAY ? sm.eg[kC - 1] : 1.f;   // padded tokens carry alpha = 1
#pragma unroll
      for (int u = 0; u < SPW; ++u) {
        const int st = wave + u * kNW;
        const int vb = st / 8, cb = st % 8;
        float4v acc = sacc[u];
        if (DECAY) acc *= gC;
        acc = tile_mma(acc, &sm.dt2[0][0], kLdc, &sm.rt[0][0], kLdc, vb * 16, cb * 16, 0, 2, lane);
        sacc[u] = acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.s[vb * 16 + 4 * l4 + r][cb * 16 + l16] = tobf(acc[r]);
      }
    }
  }

  // ---- final state and preconditioner accumulator ----
  if (a.state_out != nullptr) {
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int st = wave + u * kNW;
      const int vb = st / 8, cb = st % 8;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = vb * 16 + 4 * l4 + r, c = cb * 16 + l16;
        a.state_out[(static_cast<long long>(bh) * kD + v0 + v) * kD + c] = sacc[u][r];
      }
    }
  }
  if (WK == kWkPrecond && a.pc_h_out != nullptr && vt == 0 && pc_seg == 0)
    a.pc_h_out[static_cast<long long>(bh) * kD + pc_c] = hcarry;
}

template <int BV, bool CHAN, bool DECAY, int WK>
hipError_t launch4(const ChunkArgs &a, hipStream_t s) {
  const int grid = a.B * a.H * (kD / BV);
  const bool band = a.N >= 0 && a.N <= 15;
  if (band)
    hipLaunchKernelGGL((chunk_mfma_kernel<BV, CHAN, DECAY, WK, true>), dim3(grid), dim3(kNT), 0, s, a);
  else
    hipLaunchKernelGGL((chunk_mfma_kernel<BV, CHAN, DECAY, WK, false>), dim3(grid), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

template <int BV>
hipError_t launch_bv(const ChunkArgs &a, hipStream_t s) {
  const bool chan = a.gain == GDR_GAIN_CHANNEL, decay = a.decay == GDR_DECAY_SCALAR;
  const int wk = a.wkey == GDR_WKEY_DIAG_PRECOND ? kWkPrecond : a.wkey == GDR_WKEY_EXPLICIT ? kWkExplicit : kWkSame;
  if (chan) {
    // channel gains with a separate write key exceed the LDS budget (not instantiated)
    return decay ? launch4<BV, true, true, kWkSame>(a, s) : launch4<BV, true, false, kWkSame>(a, s);
  }
  switch (wk) {
    case kWkPrecond:
      return decay ? launch4<BV, false, true, kWkPrecond>(a, s) : launch4<BV, false, false, kWkPrecond>(a, s);
    case kWkExplicit:
      return decay ? launch4<BV, false, true, kWkExplicit>(a, s) : launch4<BV, false, false, kWkExplicit>(a, s);
    default:
      return decay ? launch4<BV, false, true, kWkSame>(a, s) : launch4<BV, false, false, kWkSame>(a, s);
  }
}

}  // namespace

bool chunk_mfma_supports(const gdr_desc_t &d, const gdr_inputs_t &in, const float *state_in, const void *out,
                         const float *state_out) {
  if (d.io_dtype != GDR_BF16 || d.Dk != kD || d.Dv != kD || d.chunk != kC) return false;
  if (d.gain == GDR_GAIN_CHANNEL && d.wkey != GDR_WKEY_SAME) return false;
  const void *p16[] = {in.q, in.k, in.v, in.erase, in.write, in.write_key, out};
  for (const void *p : p16)
    if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return false;
  return true;
}

// Value-tile width: the widest tile that still gives every CU a workgroup.
int chunk_mfma_bv(int B, int H) { return (static_cast<long long>(B) * H * (kD / 32) >= 256) ? 32 : 16; }

hipError_t launch_chunk_mfma(const ChunkArgs &a, hipStream_t s) {
  return chunk_mfma_bv(a.B, a.H) == 32 ? launch_bv<32>(a, s) : launch_bv<16>(a, s);
}

}  // namespace gdr
