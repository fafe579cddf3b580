// Single-token step of the gated delta rule, state updated in place.
//
// For one stream and one token (the online SGD step of the delta rule, Preconditioned
// DeltaNet summary section 1; decay and gain axes, section 2c):
//     S <- alpha S;  d = v' - S e;  S <- S + d r^T;  o = S (scale q)
// Every state row is independent given e, r, q:
//     x_v = S_v . e,  y_v = S_v . q           (old state)
//     d_v = v'_v - alpha x_v
//     o_v = scale (alpha y_v + d_v (r . q))
//     S_v <- alpha S_v + d_v r
// With one decay per key channel (S <- S Diag(a)) the decays move into the vectors:
// x_v = S_v . (a (.) e), y_v = S_v . (a (.) q), d_v = v'_v - x_v, o_v = scale (y_v + d_v (r . q)),
// S_v <- a (.) S_v + d_v r.
// so the kernel makes one pass over the state: one read and one write of every entry,
// which makes it HBM-bound.  One workgroup per (batch, head): its 256 threads cover 16
// rows at a time, 16 lanes per row, each lane holding DK/16 consecutive-in-float4 columns.
#include "common.h"

namespace gdr {
namespace {

constexpr int kThreads = 256;

template <typename IO>
__device__ __forceinline__ void load_vectors(const ChunkArgs &a, long long sh, float *es,
                                             float *rs, float *qs, float *vps, float *as,
                                             float *misc) {
  const IO *q = static_cast<const IO *>(a.q);
  const IO *k = static_cast<const IO *>(a.k);
  const IO *v = static_cast<const IO *>(a.v);
  const IO *er = static_cast<const IO *>(a.erase);
  const IO *wr = static_cast<const IO *>(a.write);
  const IO *wk = static_cast<const IO *>(a.write_key);
  const int tid = threadIdx.x;
  const int Dk = a.Dk, Dv = a.Dv;
  const float beta = (a.gain == GDR_GAIN_SCALAR) ? a.beta[sh] : 1.f;
  for (int c = tid; c < Dk; c += kThreads) {
    const float kk = ld_f(k, sh * Dk + c);
    es[c] = (a.gain == GDR_GAIN_SCALAR) ? beta * kk : ld_f(er, sh * Dk + c) * kk;
    qs[c] = ld_f(q, sh * Dk + c);
    float r = kk;
    if (a.wkey == GDR_WKEY_EXPLICIT) {
      r = ld_f(wk, sh * Dk + c);
    } else if (a.wkey == GDR_WKEY_DIAG_PRECOND) {
      float hh = a.pc_h_in != nullptr ? a.pc_h_in[sh * Dk + c] : a.h0;
      hh = fmaf(a.rho, hh, kk * kk);
      const float corr = -expm1f(static_cast<float>(a.t0 + 1) * a.log_rho);
      r = kk / (hh / corr + a.eps);
      if (a.pc_h_out != nullptr) a.pc_h_out[sh * Dk + c] = hh;  // same thread read it
    }
    rs[c] = r;
    as[c] = (a.decay == GDR_DECAY_CHANNEL) ? expf(a.log_alpha[sh * Dk + c]) : 1.f;
  }
  for (int c = tid; c < Dv; c += kThreads) {
    const float vv = ld_f(v, sh * Dv + c);
    vps[c] = (a.gain == GDR_GAIN_SCALAR) ? beta * vv : ld_f(wr, sh * Dv + c) * vv;
  }
  if (tid == 0) misc[0] = (a.decay == GDR_DECAY_SCALAR) ? expf(a.log_alpha[sh]) : 1.f;
}

// Fast path: Dk == DK (64 or 128), 16-byte aligned state.
template <typename IO, int DK>
__global__ __launch_bounds__(kThreads) void step_kernel(ChunkArgs a) {
  constexpr int F4 = DK / 64;     // float4 per lane per row
  constexpr int kRowsPerPass = kThreads / 16;
  constexpr int kPasses = 4;      // rows in flight per lane
  __shared__ float es[DK], rs[DK], qs[DK], as[DK], vps[512], misc[2];
  const int tid = threadIdx.x;
  const long long sh = static_cast<long long>(blockIdx.y) * a.H + blockIdx.x;
  load_vectors<IO>(a, sh, es, rs, qs, vps, as, misc);
  __syncthreads();
  if (tid < 64) {  // r . q by wave 0
    float p = 0.f;
    for (int c = tid; c < DK; c += 64) p = fmaf(rs[c], qs[c], p);
    for (int m = 32; m >= 1; m >>= 1) p += __shfl_xor(p, m, 64);
    if (tid == 0) misc[1] = p;
  }
  __syncthreads();
  const float alpha = misc[0], rq = misc[1];
  const bool chd = a.decay == GDR_DECAY_CHANNEL;
  const float xs = chd ? 1.f : alpha;   // scale of x and y (per-channel decays sit in e, q)
  const int lane = tid & 15, grp = tid >> 4;
  float4 ef[F4], qf[F4], rf[F4], af[F4];
#pragma unroll
  for (int f = 0; f < F4; ++f) {
    const int c = f * 64 + lane * 4;
    ef[f] = make_float4(es[c], es[c + 1], es[c + 2], es[c + 3]);
    qf[f] = make_float4(qs[c], qs[c + 1], qs[c + 2], qs[c + 3]);
    rf[f] = make_float4(rs[c], rs[c + 1], rs[c + 2], rs[c + 3]);
    af[f] = make_float4(alpha, alpha, alpha, alpha);
    if (chd) {
      af[f] = make_float4(as[c], as[c + 1], as[c + 2], as[c + 3]);
      ef[f] = make_float4(af[f].x * ef[f].x, af[f].y * ef[f].y, af[f].z * ef[f].z, af[f].w * ef[f].w);
      qf[f] = make_float4(af[f].x * qf[f].x, af[f].y * qf[f].y, af[f].z * qf[f].z, af[f].w * qf[f].w);
    }
  }
  float4 *S = reinterpret_cast<float4 *>(a.state_out) + sh * a.Dv * (DK / 4);
  IO *out = static_cast<IO *>(a.out);
  for (int r0 = 0; r0 < a.Dv; r0 += kRowsPerPass * kPasses) {
    float4 sv[kPasses][F4];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int row = r0 + p * kRowsPerPass + grp;
#pragma unroll
      for (int f = 0; f < F4; ++f)
        sv[p][f] = row < a.Dv ? S[row * (DK / 4) + f * 16 + lane] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int row = r0 + p * kRowsPerPass + grp;
      float x = 0.f, y = 0.f;
#pragma unroll
      for (int f = 0; f < F4; ++f) {
        x = fmaf(sv[p][f].x, ef[f].x, x); x = fmaf(sv[p][f].y, ef[f].y, x);
        x = fmaf(sv[p][f].z, ef[f].z, x); x = fmaf(sv[p][f].w, ef[f].w, x);
        y = fmaf(sv[p][f].x, qf[f].x, y); y = fmaf(sv[p][f].y, qf[f].y, y);
        y = fmaf(sv[p][f].z, qf[f].z, y); y = fmaf(sv[p][f].w, qf[f].w, y);
      }
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1) {
        x += __shfl_xor(x, m, 16);
        y += __shfl_xor(y, m, 16);
      }
      if (row < a.Dv) {
        const float d = vps[row] - xs * x;
        if (lane == 0) st_f(out, sh * a.Dv + row, a.scale * fmaf(d, rq, xs * y));
#pragma unroll
        for (int f = 0; f < F4; ++f) {
          float4 s = sv[p][f];
          s.x = fmaf(d, rf[f].x, af[f].x * s.x);
          s.y = fmaf(d, rf[f].y, af[f].y * s.y);
          s.z = fmaf(d, rf[f].z, af[f].z * s.z);
          s.w = fmaf(d, rf[f].w, af[f].w * s.w);
          S[row * (DK / 4) + f * 16 + lane] = s;
        }
      }
    }
  }
}

// Any Dk <= 128, Dv <= 512, any alignment: one thread per state row.
template <typename IO>
__global__ __launch_bounds__(kThreads) void step_kernel_any(ChunkArgs a) {
  __shared__ float es[128], rs[128], qs[128], as[128], vps[512], misc[2];
  const int tid = threadIdx.x;
  const long long sh = static_cast<long long>(blockIdx.y) * a.H + blockIdx.x;
  load_vectors<IO>(a, sh, es, rs, qs, vps, as, misc);
  __syncthreads();
  if (tid == 0) {
    float p = 0.f;
    for (int c = 0; c < a.Dk; ++c) p = fmaf(rs[c], qs[c], p);
    misc[1] = p;
  }
  __syncthreads();
  const float alpha = misc[0], rq = misc[1];
  const bool chd = a.decay == GDR_DECAY_CHANNEL;
  const float xs = chd ? 1.f : alpha;
  IO *out = static_cast<IO *>(a.out);
  for (int row = tid; row < a.Dv; row += kThreads) {
    float *S = a.state_out + (sh * a.Dv + row) * a.Dk;
    float x = 0.f, y = 0.f;
    for (int c = 0; c < a.Dk; ++c) {
      const float ac = chd ? as[c] : 1.f;
      x = fmaf(S[c], ac * es[c], x);
      y = fmaf(S[c], ac * qs[c], y);
    }
    const float d = vps[row] - xs * x;
    st_f(out, sh * a.Dv + row, a.scale * fmaf(d, rq, xs * y));
    for (int c = 0; c < a.Dk; ++c) S[c] = fmaf(d, rs[c], (chd ? as[c] : alpha) * S[c]);
  }
}

template <typename IO>
hipError_t launch_io(const ChunkArgs &a, hipStream_t s) {
  const dim3 grid(a.H, a.B);
  const bool aligned = (reinterpret_cast<uintptr_t>(a.state_out) & 15u) == 0;
  if (aligned && a.Dk == 128)
    hipLaunchKernelGGL((step_kernel<IO, 128>), grid, dim3(kThreads), 0, s, a);
  else if (aligned && a.Dk == 64)
    hipLaunchKernelGGL((step_kernel<IO, 64>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((step_kernel_any<IO>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step(const ChunkArgs &a, int io_dtype, hipStream_t s) {
  return io_dtype == GDR_BF16 ? launch_io<uint16_t>(a, s) : launch_io<float>(a, s);
}

}  // namespace gdr
