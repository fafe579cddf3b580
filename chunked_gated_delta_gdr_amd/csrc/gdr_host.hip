// Host layer of libgdr: argument validation, kernel choice, launch, error reporting.
//
// Validation is a pure host function (no HIP call), so malformed calls are rejected
// before anything is enqueued and can be tested without a GPU.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "common.h"

namespace {

thread_local std::string g_last_error;

gdr_status_t fail(gdr_status_t st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

gdr_status_t ok() {
  g_last_error.clear();
  return GDR_OK;
}

bool log_enabled() {
  static const bool on = [] {
    const char *e = std::getenv("GDR_LOG");
    return e != nullptr && e[0] != '\0' && e[0] != '0';
  }();
  return on;
}

struct Range {
  const char *name;
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(const Range &a, const Range &b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

Range rng(const char *name, const void *p, long double bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{name, lo, p == nullptr ? lo : lo + static_cast<uintptr_t>(bytes)};
}

// Largest element count of any one tensor the library accepts (2^40 elements).
constexpr long double kMaxElems = 1099511627776.0L;
// Largest number of (batch, head) streams per call, and of chunks per stream in the backward
// (whose per-chunk kernels launch one 512-thread workgroup per chunk along the grid's x axis).
constexpr long long kMaxStreams = 1LL << 19;
constexpr long long kMaxBwdChunks = 1LL << 22;

// Sections of gdr_chunk_bwd's workspace (byte offsets, each 256-byte aligned).
struct BwdLayout {
  uint64_t h, dh, D, dX, T, P, W, U, G, R, Pk, dR, Sg, Tf, dD, total;
  int NC;
};

BwdLayout bwd_layout(const gdr_desc_t &d) {
  const uint64_t B = d.B, T = d.T, H = d.H, Dk = d.Dk, Dv = d.Dv, C = d.chunk;
  const uint64_t NC = (T + C - 1) / C;
  auto al = [](uint64_t x) { return (x + 255u) & ~static_cast<uint64_t>(255u); };
  const uint64_t st = al(B * H * NC * Dv * Dk * 4u), tk = al(B * T * H * Dv * 4u), cc = al(B * H * NC * C * C * 4u);
  BwdLayout L{};
  L.h = 0;
  L.dh = st;
  L.D = 2 * st;
  L.dX = L.D + tk;
  L.T = L.dX + tk;
  L.P = L.T + cc;
  L.W = L.P + cc;
  L.U = L.W + al(B * H * NC * C * Dk * 4u);
  L.G = L.U + tk;
  L.R = L.G + (d.decay == GDR_DECAY_CHANNEL ? al(B * H * NC * C * Dk * 4u) : 0u);
  const uint64_t kk = d.wkey == GDR_WKEY_DIAG_PRECOND ? al(B * T * H * Dk * 4u) : 0u;
  L.Pk = L.R + kk;
  L.dR = L.Pk + kk;
  L.Sg = L.dR + kk;
  L.Tf = L.Sg + (d.wkey == GDR_WKEY_DIAG_PRECOND ? al(B * H * NC * Dk * 4u) : 0u);
  const bool band = d.neumann_order >= 0;
  L.dD = L.Tf + (band ? cc : 0u);
  L.total = L.dD + (band ? tk : 0u);
  L.NC = static_cast<int>(NC);
  return L;
}

// Scratch memory of gdr_chunk_bwd_noalloc: a file-scope device array, one copy on every GPU the
// library runs on, kept until the process ends.  In host code its name is a host-side stand-in,
// not a device address: the address of a GPU's copy is taken once per device with
// hipGetSymbolAddress (that device current) and only that pointer is handed to kernels.
constexpr uint64_t kScratchBytes = 64ull << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

gdr_status_t scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GDR_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(GDR_ENOTSUP, "device ordinal %d (max %d)", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(GDR_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDR_OK;
}

}  // namespace

extern "C" {

const char *gdr_status_str(gdr_status_t s) {
  switch (s) {
    case GDR_OK: return "GDR_OK";
    case GDR_EINVAL: return "GDR_EINVAL: invalid argument";
    case GDR_ENOTSUP: return "GDR_ENOTSUP: not supported";
    case GDR_EHIP: return "GDR_EHIP: HIP runtime error";
  }
  return "GDR_UNKNOWN_STATUS";
}

const char *gdr_last_error(void) { return g_last_error.c_str(); }

int gdr_abi_version(void) { return GDR_ABI_VERSION; }

gdr_status_t gdr_validate(const gdr_desc_t *d, const gdr_inputs_t *in, const float *state_in,
                          const void *out, const float *state_out, int for_step) {
  if (d == nullptr || in == nullptr) return fail(GDR_EINVAL, "desc and inputs must be non-NULL");
  if (d->struct_size != sizeof(gdr_desc_t))
    return fail(GDR_EINVAL, "desc->struct_size = %u, expected %zu (ABI mismatch)", d->struct_size,
                sizeof(gdr_desc_t));
  if (d->B < 1 || d->H < 1) return fail(GDR_EINVAL, "B = %d and H = %d must be >= 1", d->B, d->H);
  if (d->B > 65535 || d->H > 65535) return fail(GDR_ENOTSUP, "B = %d, H = %d (max 65535 each)", d->B, d->H);
  // one workgroup per (batch, head, value tile): with up to 8 (matrix-core kernel) or 32 tiles
  // of 512 threads per stream, 2^19 streams keep every grid within 2^32 work-items
  if (static_cast<long long>(d->B) * d->H > kMaxStreams)
    return fail(GDR_ENOTSUP, "B * H = %lld streams (max %lld)", static_cast<long long>(d->B) * d->H, kMaxStreams);
  if (for_step ? d->T != 1 : d->T < 0)
    return fail(GDR_EINVAL, for_step ? "T = %d; gdr_recurrent_step takes exactly one token"
                                     : "T = %d must be >= 0", d->T);
  if (d->Dk < 1 || d->Dv < 1) return fail(GDR_EINVAL, "Dk = %d and Dv = %d must be >= 1", d->Dk, d->Dv);
  if (d->Dk > 128 || d->Dv > 512)
    return fail(GDR_ENOTSUP, "Dk = %d (max 128), Dv = %d (max 512)", d->Dk, d->Dv);
  if (!for_step && d->chunk != 16 && d->chunk != 32 && d->chunk != 64 && d->chunk != 128)
    return fail(d->chunk < 1 ? GDR_EINVAL : GDR_ENOTSUP, "chunk = %d; supported: 16, 32, 64, 128", d->chunk);
  if (d->io_dtype != GDR_F32 && d->io_dtype != GDR_BF16)
    return fail(GDR_EINVAL, "io_dtype = %d", d->io_dtype);
  if (d->gain != GDR_GAIN_SCALAR && d->gain != GDR_GAIN_CHANNEL) return fail(GDR_EINVAL, "gain = %d", d->gain);
  if (d->decay != GDR_DECAY_NONE && d->decay != GDR_DECAY_SCALAR && d->decay != GDR_DECAY_CHANNEL)
    return fail(GDR_EINVAL, "decay = %d", d->decay);
  if (d->wkey != GDR_WKEY_SAME && d->wkey != GDR_WKEY_DIAG_PRECOND && d->wkey != GDR_WKEY_EXPLICIT)
    return fail(GDR_EINVAL, "wkey = %d", d->wkey);
  if (d->impl != GDR_IMPL_AUTO && d->impl != GDR_IMPL_GENERIC && d->impl != GDR_IMPL_MFMA)
    return fail(GDR_EINVAL, "impl = %d", d->impl);
  if (!std::isfinite(d->scale)) return fail(GDR_EINVAL, "scale must be finite");
  if (!for_step) {
    if (d->residual_steps < 0) return fail(GDR_EINVAL, "residual_steps = %d must be >= 0", d->residual_steps);
    if (d->residual_steps > 0 && d->neumann_order < 0)
      return fail(GDR_EINVAL, "residual_steps = %d needs a band start (neumann_order >= 0)", d->residual_steps);
    if (d->residual_steps > 0 && d->decay == GDR_DECAY_CHANNEL)
      return fail(GDR_ENOTSUP, "residual_steps with decay CHANNEL (no room for both in one workgroup's LDS)");
    if (d->residual_steps > 64)
      return fail(GDR_ENOTSUP, "residual_steps = %d (max 64; E^s vanishes once s (N + 1) >= C)",
                  d->residual_steps);
    if (d->chunk == 128 && d->residual_steps > 0)
      return fail(GDR_ENOTSUP, "residual_steps at chunk 128 (the residual correction runs at chunk <= 64)");
    if (d->chunk == 128 && d->neumann_order >= 0 && d->neumann_order < 127) {
      if (d->neumann_order > 15)
        return fail(GDR_ENOTSUP, "chunk 128 with neumann_order = %d (supported: exact, N <= 15, or N >= 127)",
                    d->neumann_order);
      if (d->decay == GDR_DECAY_CHANNEL)
        return fail(GDR_ENOTSUP, "chunk 128 with a band-limited T and decay CHANNEL");
    }
  }

  const long double B = d->B, T = d->T, H = d->H, Dk = d->Dk, Dv = d->Dv;
  if (B * T * H * (Dk > Dv ? Dk : Dv) > kMaxElems || B * H * Dv * Dk > kMaxElems)
    return fail(GDR_ENOTSUP, "problem too large (more than 2^40 elements in one tensor)");
  const long double esz = d->io_dtype == GDR_BF16 ? 2.0L : 4.0L;
  const bool need = d->T > 0;  // tensors indexed by token are only read when T > 0

  // required / forbidden pointers
  if (need && (in->q == nullptr || in->k == nullptr || in->v == nullptr))
    return fail(GDR_EINVAL, "q, k and v are required");
  if (d->gain == GDR_GAIN_SCALAR) {
    if (need && in->beta == nullptr) return fail(GDR_EINVAL, "gain SCALAR needs beta");
    if (in->erase != nullptr || in->write != nullptr)
      return fail(GDR_EINVAL, "erase/write gates given with gain SCALAR");
  } else {
    if (need && (in->erase == nullptr || in->write == nullptr))
      return fail(GDR_EINVAL, "gain CHANNEL needs erase and write");
    if (in->beta != nullptr) return fail(GDR_EINVAL, "beta given with gain CHANNEL");
  }
  if (d->decay != GDR_DECAY_NONE) {
    if (need && in->log_alpha == nullptr) return fail(GDR_EINVAL, "decay SCALAR / CHANNEL needs log_alpha");
  } else if (in->log_alpha != nullptr) {
    return fail(GDR_EINVAL, "log_alpha given with decay NONE");
  }
  if (d->wkey == GDR_WKEY_EXPLICIT) {
    if (need && in->write_key == nullptr) return fail(GDR_EINVAL, "wkey EXPLICIT needs write_key");
  } else if (in->write_key != nullptr) {
    return fail(GDR_EINVAL, "write_key given without wkey EXPLICIT");
  }
  if (d->wkey == GDR_WKEY_DIAG_PRECOND) {
    if (!(d->pc_rho > 0.f && d->pc_rho < 1.f)) return fail(GDR_EINVAL, "pc_rho must be in (0, 1)");
    if (!(d->pc_eps > 0.f) || !std::isfinite(d->pc_eps)) return fail(GDR_EINVAL, "pc_eps must be > 0");
    if (!(d->pc_h0 >= 0.f) || !std::isfinite(d->pc_h0)) return fail(GDR_EINVAL, "pc_h0 must be >= 0");
    if (d->pc_t0 < 0) return fail(GDR_EINVAL, "pc_t0 must be >= 0");
  } else if (in->pc_h_in != nullptr || in->pc_h_out != nullptr) {
    return fail(GDR_EINVAL, "pc_h_in/pc_h_out given without wkey DIAG_PRECOND");
  }
  if ((need || for_step) && out == nullptr) return fail(GDR_EINVAL, "out is required");
  if (for_step && state_out == nullptr) return fail(GDR_EINVAL, "state is required");

  // alignment to the element size
  const uintptr_t ea = d->io_dtype == GDR_BF16 ? 1u : 3u;
  const void *io_ptrs[] = {in->q, in->k, in->v, in->erase, in->write, in->write_key, out};
  for (const void *p : io_ptrs)
    if ((reinterpret_cast<uintptr_t>(p) & ea) != 0) return fail(GDR_EINVAL, "misaligned io pointer");
  const void *f_ptrs[] = {in->beta, in->log_alpha, in->pc_h_in, in->pc_h_out, state_in, state_out};
  for (const void *p : f_ptrs)
    if ((reinterpret_cast<uintptr_t>(p) & 3u) != 0) return fail(GDR_EINVAL, "misaligned fp32 pointer");

  // overlap rules
  const long double ntok = B * T * H;
  const Range r_out = rng("out", out, ntok * Dv * esz);
  const Range inputs[] = {
      rng("q", in->q, ntok * Dk * esz), rng("k", in->k, ntok * Dk * esz),
      rng("v", in->v, ntok * Dv * esz), rng("beta", in->beta, ntok * 4),
      rng("log_alpha", in->log_alpha, ntok * (d->decay == GDR_DECAY_CHANNEL ? Dk : 1) * 4),
      rng("erase", in->erase, ntok * Dk * esz),
      rng("write", in->write, ntok * Dv * esz), rng("write_key", in->write_key, ntok * Dk * esz),
      rng("pc_h_in", in->pc_h_in, B * H * Dk * 4)};
  const Range r_sin = rng("state_in", for_step ? nullptr : state_in, B * H * Dv * Dk * 4);
  const Range r_sout = rng(for_step ? "state" : "state_out", state_out, B * H * Dv * Dk * 4);
  const Range r_hout = rng("pc_h_out", in->pc_h_out, B * H * Dk * 4);
  for (const Range &r : inputs) {
    if (overlap(r_out, r)) return fail(GDR_EINVAL, "out overlaps %s", r.name);
    if (overlap(r_sout, r)) return fail(GDR_EINVAL, "%s overlaps %s", r_sout.name, r.name);
    if (overlap(r_hout, r) && !(for_step && r.lo == r_hout.lo && r.hi == r_hout.hi &&
                                 r.lo == reinterpret_cast<uintptr_t>(in->pc_h_in)))
      return fail(GDR_EINVAL, "pc_h_out overlaps %s", r.name);
  }
  if (overlap(r_out, r_sout)) return fail(GDR_EINVAL, "out overlaps %s", r_sout.name);
  if (overlap(r_out, r_sin)) return fail(GDR_EINVAL, "out overlaps state_in");
  if (overlap(r_out, r_hout)) return fail(GDR_EINVAL, "out overlaps pc_h_out");
  if (overlap(r_hout, r_sout) || overlap(r_hout, r_sin))
    return fail(GDR_EINVAL, "pc_h_out overlaps the state");
  if (overlap(r_sin, r_sout) && !(r_sin.lo == r_sout.lo))
    return fail(GDR_EINVAL, "state_out partially overlaps state_in");
  return ok();
}

// Chunk 128 with the exact T runs as chunk 64: T's block (I - A)^-1 = [[T_aa, 0], [T_ba, T_bb]]
// has T_ba = T_bb A_ba T_aa, so D_b = T_bb (X_b + A_ba D_a), and X_b + A_ba D_a is X_b read from
// the state after the chunk's first 64 tokens.  Chunk 64 computes exactly that product,
// regrouped (the results differ only in rounding).  A band limit N >= 127 keeps every entry.
static gdr_desc_t lower_chunk(const gdr_desc_t &d) {
  gdr_desc_t e = d;
  if (d.chunk == 128 && (d.neumann_order < 0 || d.neumann_order >= 127)) {
    e.chunk = 64;
    e.neumann_order = -1;
  }
  return e;
}

int gdr_chunk_fwd_impl(const gdr_desc_t *dd) {
  if (dd == nullptr || dd->struct_size != sizeof(gdr_desc_t)) return -1;
  const gdr_desc_t dl = lower_chunk(*dd);
  const gdr_desc_t *d = &dl;
  gdr_inputs_t none{};
  const bool mfma = gdr::chunk_mfma_supports(*d, none, nullptr, nullptr, nullptr);
  if (d->impl == GDR_IMPL_GENERIC) return GDR_IMPL_GENERIC;
  if (d->impl == GDR_IMPL_MFMA) return mfma ? GDR_IMPL_MFMA : -1;
  return mfma ? GDR_IMPL_MFMA : GDR_IMPL_GENERIC;
}

static gdr::ChunkArgs make_args(const gdr_desc_t *d, const gdr_inputs_t *in, const float *state_in,
                                void *out, float *state_out) {
  gdr::ChunkArgs a{};
  a.q = in->q; a.k = in->k; a.v = in->v;
  a.beta = in->beta; a.log_alpha = in->log_alpha;
  a.erase = in->erase; a.write = in->write; a.write_key = in->write_key;
  a.pc_h_in = in->pc_h_in; a.pc_h_out = in->pc_h_out;
  a.state_in = state_in; a.out = out; a.state_out = state_out;
  a.B = d->B; a.T = d->T; a.H = d->H; a.Dk = d->Dk; a.Dv = d->Dv; a.C = d->chunk;
  a.gain = d->gain; a.decay = d->decay; a.wkey = d->wkey;
  a.N = d->neumann_order < 0 ? -1 : d->neumann_order;
  a.S = a.N < 0 ? 0 : d->residual_steps;
  a.scale = d->scale;
  a.rho = d->pc_rho; a.log_rho = d->wkey == GDR_WKEY_DIAG_PRECOND ? std::log(d->pc_rho) : 0.f;
  a.eps = d->pc_eps; a.h0 = d->pc_h0; a.t0 = d->pc_t0;
  return a;
}

// the chunk forward with an optional workspace for the precomputed T (null: none)
static gdr_status_t chunk_fwd(const gdr_desc_t *dd, const gdr_inputs_t *in, const float *state_in,
                              void *out, float *state_out, void *ws, uint64_t ws_bytes, void *stream) {
  gdr_status_t st = gdr_validate(dd, in, state_in, out, state_out, 0);
  if (st != GDR_OK) return st;
  const gdr_desc_t dl = lower_chunk(*dd);
  const gdr_desc_t *d = &dl;
  // the per-channel decay runs on the matrix-core kernel only with the workspace
  const bool kda_ok = ws != nullptr && gdr::chunk_mfma_kda_supports(*d, *in, state_in, out, state_out);
  const bool mfma_ok = kda_ok || gdr::chunk_mfma_supports(*d, *in, state_in, out, state_out);
  if (d->impl == GDR_IMPL_MFMA && !mfma_ok)
    return fail(GDR_ENOTSUP, "the MFMA kernel does not cover this descriptor "
                             "(needs bf16, Dk = Dv = 128, chunk 64 or exact chunk 128, 16-byte aligned tensors, "
                             "channel gains only with write key k; a per-channel decay needs scalar gains, write key k, "
                             "exact T and the workspace of gdr_chunk_fwd_ws)");
  const bool use_mfma = mfma_ok && d->impl != GDR_IMPL_GENERIC;
  gdr::ChunkArgs a = make_args(d, in, state_in, out, state_out);
  if (ws != nullptr && use_mfma) {
    const uint64_t need = gdr::chunk_mfma_tpre_bytes(*d);   // (per-channel decay: operands and records)
    if (need > 0) {
      if (ws_bytes < need)
        return fail(GDR_EINVAL, "workspace of %llu bytes, this descriptor needs %llu",
                    static_cast<unsigned long long>(ws_bytes), static_cast<unsigned long long>(need));
      if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(GDR_EINVAL, "workspace must be 256-byte aligned");
      const long double ntok = static_cast<long double>(d->B) * d->T * d->H;
      const long double sbytes = static_cast<long double>(d->B) * d->H * d->Dv * d->Dk * 4;
      const Range r_ws = rng("workspace", ws, static_cast<long double>(need));
      const Range others[] = {
          rng("q", in->q, ntok * d->Dk * 2), rng("k", in->k, ntok * d->Dk * 2), rng("v", in->v, ntok * d->Dv * 2),
          rng("beta", in->beta, ntok * 4),
          rng("log_alpha", in->log_alpha, ntok * 4 * (d->decay == GDR_DECAY_CHANNEL ? d->Dk : 1)),
          rng("erase", in->erase, ntok * d->Dk * 2), rng("write", in->write, ntok * d->Dv * 2),
          rng("out", out, ntok * d->Dv * 2), rng("state_in", state_in, sbytes), rng("state_out", state_out, sbytes)};
      for (const Range &r : others)
        if (overlap(r_ws, r)) return fail(GDR_EINVAL, "workspace overlaps %s", r.name);
      a.tpre = static_cast<const uint16_t *>(ws);
    }
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (log_enabled())
    std::fprintf(stderr, "[gdr] chunk_fwd %s%s B=%d T=%d H=%d Dk=%d Dv=%d C=%d io=%s gain=%d decay=%d wkey=%d N=%d S=%d\n",
                 use_mfma ? "mfma" : "generic", a.tpre != nullptr ? " (T formed beforehand)" : "", d->B, d->T,
                 d->H, d->Dk, d->Dv, d->chunk, d->io_dtype == GDR_BF16 ? "bf16" : "f32", d->gain, d->decay,
                 d->wkey, a.N, a.S);
  const hipError_t e = use_mfma ? gdr::launch_chunk_mfma(a, s) : gdr::launch_chunk_generic(a, d->io_dtype, s);
  if (e != hipSuccess) return fail(GDR_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

gdr_status_t gdr_chunk_fwd(const gdr_desc_t *dd, const gdr_inputs_t *in, const float *state_in,
                           void *out, float *state_out, void *stream) {
  return chunk_fwd(dd, in, state_in, out, state_out, nullptr, 0, stream);
}

uint64_t gdr_chunk_fwd_workspace_size(const gdr_desc_t *dd) {
  if (dd == nullptr || dd->struct_size != sizeof(gdr_desc_t) || dd->B < 1 || dd->H < 1 || dd->T < 0 ||
      (dd->chunk != 16 && dd->chunk != 32 && dd->chunk != 64 && dd->chunk != 128))
    return 0;
  if (dd->impl == GDR_IMPL_GENERIC) return 0;
  const gdr_desc_t dl = lower_chunk(*dd);
  gdr_inputs_t none{};
  if (!gdr::chunk_mfma_supports(dl, none, nullptr, nullptr, nullptr) &&
      !gdr::chunk_mfma_kda_supports(dl, none, nullptr, nullptr, nullptr))
    return 0;
  return gdr::chunk_mfma_tpre_bytes(dl);
}

gdr_status_t gdr_chunk_fwd_ws(const gdr_desc_t *dd, const gdr_inputs_t *in, const float *state_in,
                              void *out, float *state_out, void *workspace, uint64_t workspace_bytes,
                              void *stream) {
  return chunk_fwd(dd, in, state_in, out, state_out, workspace, workspace_bytes, stream);
}

uint64_t gdr_chunk_bwd_workspace_size(const gdr_desc_t *dd) {
  if (dd == nullptr || dd->struct_size != sizeof(gdr_desc_t) || dd->B < 1 || dd->H < 1 || dd->T < 0 ||
      dd->Dk < 1 || dd->Dv < 1 || (dd->chunk != 16 && dd->chunk != 32 && dd->chunk != 64 && dd->chunk != 128))
    return 0;
  const gdr_desc_t dl = lower_chunk(*dd);
  if (dl.chunk == 128) return 0;   // (band-limited T at chunk 128: no backward)
  return bwd_layout(dl).total;
}

gdr_status_t gdr_validate_bwd(const gdr_desc_t *dd, const gdr_inputs_t *in, const float *state_in,
                              const void *d_out, const float *d_state_out, const gdr_grads_t *g,
                              const void *ws, uint64_t ws_bytes) {
  // the forward's own contract, with d_out in the place of out
  gdr_status_t st = gdr_validate(dd, in, state_in, d_out, nullptr, 0);
  if (st != GDR_OK) return fail(st, "forward arguments (d_out checked as out): %s", g_last_error.c_str());
  const gdr_desc_t dl = lower_chunk(*dd);
  const gdr_desc_t *d = &dl;
  if (d->chunk == 128) return fail(GDR_ENOTSUP, "backward of the band-limited T at chunk 128");
  if (g == nullptr) return fail(GDR_EINVAL, "grads must be non-NULL");
  if (in->pc_h_out != nullptr) return fail(GDR_EINVAL, "pc_h_out must be NULL (the backward does not write it)");
  if (g->dpc_h_in != nullptr && d->wkey != GDR_WKEY_DIAG_PRECOND)
    return fail(GDR_EINVAL, "grads->dpc_h_in given without wkey DIAG_PRECOND");
  if ((reinterpret_cast<uintptr_t>(g->dpc_h_in) & 3u) != 0) return fail(GDR_EINVAL, "grads->dpc_h_in misaligned");
  if ((static_cast<long long>(d->T) + d->chunk - 1) / d->chunk > kMaxBwdChunks)
    return fail(GDR_ENOTSUP, "T = %d is %lld chunks of %d (max %lld chunks in the backward)", d->T,
                (static_cast<long long>(d->T) + d->chunk - 1) / d->chunk, d->chunk, kMaxBwdChunks);
  if (d->neumann_order >= 0 && d->residual_steps > 0)
    return fail(GDR_ENOTSUP, "backward of the residual-corrected T (exact or band-limited T only)");
  if (d->neumann_order >= 0 && d->decay == GDR_DECAY_CHANNEL)
    return fail(GDR_ENOTSUP, "backward of the band-limited T with the per-channel decay");
  const bool need = d->T > 0;
  struct Opt {
    const char *name;
    const float *p;
    bool wanted;
    long double elems;
  };
  const long double B = d->B, T = d->T, H = d->H, Dk = d->Dk, Dv = d->Dv, ntok = B * T * H;
  const Opt outs[] = {
      {"dq", g->dq, true, ntok * Dk},
      {"dk", g->dk, true, ntok * Dk},
      {"dv", g->dv, true, ntok * Dv},
      {"dbeta", g->dbeta, d->gain == GDR_GAIN_SCALAR, ntok},
      {"derase", g->derase, d->gain == GDR_GAIN_CHANNEL, ntok * Dk},
      {"dwrite", g->dwrite, d->gain == GDR_GAIN_CHANNEL, ntok * Dv},
      {"dlog_alpha", g->dlog_alpha, d->decay != GDR_DECAY_NONE, d->decay == GDR_DECAY_CHANNEL ? ntok * Dk : ntok},
      {"dwrite_key", g->dwrite_key, d->wkey == GDR_WKEY_EXPLICIT, ntok * Dk},
  };
  for (const Opt &o : outs) {
    if (o.wanted && need && o.p == nullptr) return fail(GDR_EINVAL, "grads->%s is required", o.name);
    if (!o.wanted && o.p != nullptr) return fail(GDR_EINVAL, "grads->%s given but the variant has no such input", o.name);
    if ((reinterpret_cast<uintptr_t>(o.p) & 3u) != 0) return fail(GDR_EINVAL, "grads->%s misaligned", o.name);
  }
  if ((reinterpret_cast<uintptr_t>(g->dstate_in) & 3u) != 0 || (reinterpret_cast<uintptr_t>(d_state_out) & 3u) != 0)
    return fail(GDR_EINVAL, "misaligned fp32 state pointer");
  const uint64_t need_ws = bwd_layout(*d).total;
  if (ws_bytes < need_ws)
    return fail(GDR_EINVAL, "workspace_bytes = %llu, need %llu", static_cast<unsigned long long>(ws_bytes),
                static_cast<unsigned long long>(need_ws));
  if (need_ws > 0 && ws == nullptr) return fail(GDR_EINVAL, "workspace is required");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(GDR_EINVAL, "workspace must be 256-byte aligned");

  // overlap: every output against every input, every other output and the workspace
  const long double esz = d->io_dtype == GDR_BF16 ? 2.0L : 4.0L;
  const Range inputs[] = {
      rng("q", in->q, ntok * Dk * esz), rng("k", in->k, ntok * Dk * esz),
      rng("v", in->v, ntok * Dv * esz), rng("beta", in->beta, ntok * 4),
      rng("log_alpha", in->log_alpha, (d->decay == GDR_DECAY_CHANNEL ? ntok * Dk : ntok) * 4),
      rng("erase", in->erase, ntok * Dk * esz),
      rng("write", in->write, ntok * Dv * esz), rng("write_key", in->write_key, ntok * Dk * esz),
      rng("state_in", state_in, B * H * Dv * Dk * 4), rng("d_out", d_out, ntok * Dv * esz),
      rng("d_state_out", d_state_out, B * H * Dv * Dk * 4), rng("pc_h_in", in->pc_h_in, B * H * Dk * 4)};
  Range written[11];
  int nw = 0;
  for (const Opt &o : outs) written[nw++] = rng(o.name, o.p, o.elems * 4);
  written[nw++] = rng("dstate_in", g->dstate_in, B * H * Dv * Dk * 4);
  written[nw++] = rng("dpc_h_in", g->dpc_h_in, B * H * Dk * 4);
  written[nw++] = rng("workspace", ws, static_cast<long double>(need_ws));
  for (int i = 0; i < nw; ++i) {
    for (const Range &r : inputs)
      if (overlap(written[i], r)) return fail(GDR_EINVAL, "%s overlaps %s", written[i].name, r.name);
    for (int j = i + 1; j < nw; ++j)
      if (overlap(written[i], written[j])) return fail(GDR_EINVAL, "%s overlaps %s", written[i].name, written[j].name);
  }
  return ok();
}

gdr_status_t gdr_chunk_bwd(const gdr_desc_t *dd, const gdr_inputs_t *in, const float *state_in,
                           const void *d_out, const float *d_state_out, const gdr_grads_t *g,
                           void *workspace, uint64_t workspace_bytes, void *stream) {
  gdr_status_t st = gdr_validate_bwd(dd, in, state_in, d_out, d_state_out, g, workspace, workspace_bytes);
  if (st != GDR_OK) return st;
  const gdr_desc_t dl = lower_chunk(*dd);
  const gdr_desc_t *d = &dl;
  const BwdLayout L = bwd_layout(*d);
  char *ws = static_cast<char *>(workspace);
  gdr::BwdArgs b{};
  b.f = make_args(d, in, state_in, nullptr, nullptr);
  b.NC = L.NC;
  if (L.total > 0) {
    b.h = reinterpret_cast<float *>(ws + L.h);
    b.dh = reinterpret_cast<float *>(ws + L.dh);
    b.D = reinterpret_cast<float *>(ws + L.D);
    b.dX = reinterpret_cast<float *>(ws + L.dX);
    b.Tw = reinterpret_cast<float *>(ws + L.T);
    b.Pw = reinterpret_cast<float *>(ws + L.P);
    b.Ww = reinterpret_cast<float *>(ws + L.W);
    b.Uw = reinterpret_cast<float *>(ws + L.U);
    b.Gw = d->decay == GDR_DECAY_CHANNEL ? reinterpret_cast<float *>(ws + L.G) : nullptr;
    if (d->wkey == GDR_WKEY_DIAG_PRECOND) {
      b.Rk = reinterpret_cast<float *>(ws + L.R);
      b.Pk = reinterpret_cast<float *>(ws + L.Pk);
      b.dRk = reinterpret_cast<float *>(ws + L.dR);
      b.Sg = reinterpret_cast<float *>(ws + L.Sg);
    }
    if (d->neumann_order >= 0) {
      b.Tfw = reinterpret_cast<float *>(ws + L.Tf);
      b.dDw = reinterpret_cast<float *>(ws + L.dD);
    }
  }
  b.dout = d_out;
  b.dstate_out = d_state_out;
  b.dq = g->dq; b.dk = g->dk; b.dv = g->dv; b.dbeta = g->dbeta;
  b.derase = g->derase; b.dwrite = g->dwrite; b.dla = g->dlog_alpha; b.dwk = g->dwrite_key;
  b.dstate_in = g->dstate_in;
  const bool pc = d->wkey == GDR_WKEY_DIAG_PRECOND;
  if (pc) b.dwk = b.dRk;   // the write-key gradients go to the workspace, then through p_t
  b.dpc_h_in = g->dpc_h_in;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (log_enabled())
    std::fprintf(stderr, "[gdr] chunk_bwd B=%d T=%d H=%d Dk=%d Dv=%d C=%d io=%s gain=%d decay=%d wkey=%d ws=%llu\n",
                 d->B, d->T, d->H, d->Dk, d->Dv, d->chunk, d->io_dtype == GDR_BF16 ? "bf16" : "f32", d->gain,
                 d->decay, d->wkey, static_cast<unsigned long long>(L.total));
  hipError_t e = hipSuccess;
  if (pc && d->T > 0)   // 0. the preconditioned write keys
    e = gdr::launch_bwd_pc_keys(b, d->io_dtype, s);
  if (e == hipSuccess && d->T > 0)   // 1. forward recompute: T, P, W, U of every chunk, then D and the chunk states
    e = gdr::launch_bwd_prep_state(b, d->io_dtype, s);
  if (e == hipSuccess && (d->T > 0 || g->dstate_in != nullptr))   // 2. reverse sweep
    e = gdr::launch_bwd_sweep(b, d->io_dtype, s);
  if (e == hipSuccess && d->T > 0)   // 3. per-chunk gradients
    e = gdr::launch_bwd_chunk(b, d->io_dtype, s);
  if (e == hipSuccess && pc && (d->T > 0 || g->dpc_h_in != nullptr))   // 4. through the preconditioner
    e = gdr::launch_bwd_pc_grad(b, d->io_dtype, s);
  if (e != hipSuccess) return fail(GDR_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

uint64_t gdr_chunk_bwd_noalloc_max_workspace(void) { return kScratchBytes; }

gdr_status_t gdr_chunk_bwd_noalloc(const gdr_desc_t *d, const gdr_inputs_t *in, const float *state_in,
                                   const void *d_out, const float *d_state_out, const gdr_grads_t *g,
                                   void *stream) {
  // the same validation, kernels and results as gdr_chunk_bwd, with the workspace in this
  // GPU's scratch array; nothing is allocated
  if (d == nullptr || d->struct_size != sizeof(gdr_desc_t))
    return fail(GDR_EINVAL, "desc must be non-NULL with struct_size = %zu", sizeof(gdr_desc_t));
  const uint64_t need = gdr_chunk_bwd_workspace_size(d);
  if (need > kScratchBytes)
    return fail(GDR_ENOTSUP, "the backward needs %llu bytes of workspace; the no-allocation entry point holds %llu",
                static_cast<unsigned long long>(need), static_cast<unsigned long long>(kScratchBytes));
  void *ws = nullptr;
  const gdr_status_t st = scratch_address(&ws);
  if (st != GDR_OK) return st;
  return gdr_chunk_bwd(d, in, state_in, d_out, d_state_out, g, ws, kScratchBytes, stream);
}

gdr_status_t gdr_recurrent_step(const gdr_desc_t *d, const gdr_inputs_t *in, float *state, void *out,
                                void *stream) {
  gdr_status_t st = gdr_validate(d, in, nullptr, out, state, 1);
  if (st != GDR_OK) return st;
  const gdr::ChunkArgs a = make_args(d, in, state, out, state);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (log_enabled())
    std::fprintf(stderr, "[gdr] recurrent_step B=%d H=%d Dk=%d Dv=%d io=%s\n", d->B, d->H, d->Dk, d->Dv,
                 d->io_dtype == GDR_BF16 ? "bf16" : "f32");
  const hipError_t e = gdr::launch_step(a, d->io_dtype, s);
  if (e != hipSuccess) return fail(GDR_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
