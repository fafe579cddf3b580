// Fused chunk-parallel gated delta-rule forward on the gfx950 matrix cores (bf16 in,
// fp32 accumulate, fp32 state), for Dk = Dv = 128 and chunks of 64 tokens.
//
// Per chunk of 64 tokens (chunk-wise form of the MatMul-only inversion summary,
// "Declaracao do Problema"; the WY correction U - W S^T is evaluated as T (V' - e^g E S^T),
// the same product regrouped so only one 64 x 16 right-hand side per value block meets T):
//   g   inclusive cumulative sum of log alpha (log2 units)      Gamma_ij = 2^(g_i - g_j), j <= i
//   A   = -tril_{-1}((E R^T) (.) Gamma),  T = (I - A)^-1        (16 x 16 blocks, see below)
//   P   = tril(Q R^T) (.) Gamma
//   X   = V' - (e^g (.) E) S^T
//   D   = T X
//   O   = scale ((e^g (.) Q) S^T + P D)
//   S  <- e^{g_C} S + (e^{g_C - g} (.) D)^T R
//
// Work split inside one workgroup (8 wave64s; one workgroup per batch, head and value tile
// of BV = 16 or 32 state rows):
//  * value waves (BV / 16 of them) each own 16 state rows.  The transposed state S^T
//    (128 x 16, fp32) lives in that wave's MFMA accumulators for the whole sequence, and
//    every S-dependent product of a chunk is chained through registers: an accumulator
//    tile converted to bf16 is directly the B operand of the next product.  Only these
//    waves store to HBM.
//  * helper waves prepare chunk c + 1 while the value waves run chunk c: they stage the
//    next inputs into LDS from registers prefetched a chunk earlier (only helpers load
//    from HBM), build T and P.  T is formed blockwise: each 16 x 16 diagonal block
//    D = (I - N)^-1 = (I + N)(I + N^2)(I + N^4)(I + N^8) (N strictly lower, so N^16 = 0)
//    on the matrix cores, one block per helper wave, as soon as the chunk is staged; the
//    off-diagonal blocks T_10 = D_1 A_10 D_0, T_32 = D_3 A_32 D_2 and the lower-left
//    quadrant T_ba = T_b A_ba T_a follow in the next phase, beside the P tiles.
//  * With a band limit N >= 0 (the truncated Neumann series with its diagonal mask, same
//    summary, Metodologia 1-2) entries with i - j > N are dropped when T is written; by
//    Lemma 3.1 the band of every product above depends only on the bands of its factors,
//    so the stored band equals the band of the exact inverse.
//  Two barriers per chunk (three with the diagonal preconditioner, whose write keys need a
//  scan over the chunk before A and P can use them).
//
// MFMA operand conventions: v_mfma_f32_16x16x32_bf16 takes in lane l row (l % 16) of A and
// column (l % 16) of B with 8 K-slots each; v_mfma_f32_16x16x16bf16_1k takes 4 K-slots
// (K = 4 (l / 16) + i); the 16 x 16 fp32 result holds rows 4 (l / 16) + r, column l % 16.
// An accumulator tile is therefore the B-operand layout of its K = 16 rows.  For K = 32
// products fed from two accumulator tiles the K-slot order is "split": slots 0..3 are
// rows 4 (l / 16) + r of the first tile, slots 4..7 those of the second, and the A
// operand is gathered from LDS in the same order (against the state the tiles keep their
// channels in an order that makes this the natural order, see the value waves).  A product
// X Y whose factors are both accumulators needs acc(X^T) and acc(Y); transposed copies are
// computed where needed.
#include <cstdlib>
#include <type_traits>

#include "common.h"

namespace gdr {
namespace {

typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kC = 64;          // chunk
constexpr int kD = 128;         // Dk = Dv
constexpr int kNW = 8;          // waves per workgroup
constexpr int kNT = kNW * 64;   // threads
// padded bf16 row strides: 136 bytes (34 banks of 4) for the [64][64] tiles T and P and 72
// bytes (18 banks) for the 32 x 32 block A_ba, so the 16 rows an 8-byte-per-lane access
// touches land on distinct banks
constexpr int kLdc = kC + 4;
constexpr int kLdl = 32 + 4;
constexpr float kLog2e = 1.4426950408889634f;

enum : int { kWkSame = 0, kWkPrecond = 1, kWkExplicit = 2 };

// XOR-swizzled row-major bf16 layouts (16-byte granules), conflict-free for MFMA reads
__device__ __forceinline__ int sw128(int row, int col) {
  return row * 128 + ((((col >> 3) ^ (row & 15))) << 3) + (col & 7);
}

template <int BV, bool CHAN, int WK>
struct __align__(16) Smem {
  uint16_t q[2][kC * kD];                                  // Q
  // 16 bytes apart from a multiple of 512: the value waves read the same offsets of Q and K
  // (or E), and the compiler would otherwise pair those reads into one two-address read whose
  // halves then have to be moved into place
  uint16_t pad_qk[8];
  uint16_t k[2][kC * kD];                                  // K
  uint16_t e[CHAN ? 2 : 1][CHAN ? kC * kD : 8];            // erase key b (.) k
  uint16_t r[WK != kWkSame ? 2 : 1][WK != kWkSame ? kC * kD : 8];   // write key if != k
  uint16_t vp[2][kC][BV + 8];                              // v tile (w (.) v with channel gains)
  uint16_t t[2][kC][kLdc];                                 // T
  uint16_t p[kC][kLdc];                                    // P (one buffer)
  uint16_t lba[32][kLdl];                                  // A_ba = -L_ba (rows 32.., cols ..31)
  uint16_t aod[2][16][20];                                 // A_10, A_32
  float g2[2][kC], eg[2][kC], wd[2][kC], beta[2][kC], ic[2][kC];
};

__device__ __forceinline__ float bf(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
// 2^x by the hardware instruction alone: the arguments are decays between two tokens of a
// chunk (x <= 0 wherever the result is kept); results below the normal range flush to zero
__device__ __forceinline__ float decay2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ uint16_t tobf(float x) { return f32_to_bf16_bits(x); }
__device__ __forceinline__ uint32_t word(const uint4 &v, int e) {
  const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}
__device__ __forceinline__ float elem(const uint4 &v, int e) { return bf(word(v, e)); }

__device__ __forceinline__ short8v ld8(const uint16_t *p) { return *reinterpret_cast<const short8v *>(p); }
// gfx950 transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane j
// receives element j % 4 of the 8-byte rows addressed by lanes 4 i + j / 4, i = 0..3.  If
// lane s of group g addresses M[k0 + 4 g + s / 4][m0 + 4 (s % 4) ..], lane j of group g gets
// M[k0 + 4 g + i][m0 + j]: the K = 16 operand (or accumulator) layout of the block's transpose.
typedef __attribute__((address_space(3))) short4v lds_short4v;
__device__ __forceinline__ short4v ldtr(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(p));
}
__device__ __forceinline__ short4v ld4(const uint16_t *p) { return *reinterpret_cast<const short4v *>(p); }
__device__ __forceinline__ short8v cat(short4v a, short4v b) {
  return short8v{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ float4v mfma32(short8v a, short8v b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// K = 16 product issued as the native gfx950 K = 32 instruction with K-slots 4..7 zero.
// (The legacy v_mfma_f32_16x16x16_bf16 is avoided: its results were read back before
// they were written -- first two result registers stale -- with the wait states the
// compiler inserts for it on gfx950.)
__device__ __forceinline__ float4v mfma16(short4v a, short4v b, float4v c) {
  const short4v z = {0, 0, 0, 0};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(cat(a, z), cat(b, z), c, 0, 0, 0);
}
__device__ __forceinline__ short4v tobf4(float4v v) {
  short4v r;
  const uint32_t lo = f32x2_to_bf16x2_bits(v[0], v[1]), hi = f32x2_to_bf16x2_bits(v[2], v[3]);
  r[0] = static_cast<short>(lo & 0xffff);
  r[1] = static_cast<short>(lo >> 16);
  r[2] = static_cast<short>(hi & 0xffff);
  r[3] = static_cast<short>(hi >> 16);
  return r;
}
__device__ __forceinline__ float4 ld4f(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float4v zero4() { return float4v{0.f, 0.f, 0.f, 0.f}; }
// the 16 x 16 identity as a K = 16 operand (A or B layout: 1.0 where K index == l % 16)
__device__ __forceinline__ short4v ident4(int lane) {
  short4v r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (4 * (lane >> 4) + i == (lane & 15)) ? static_cast<short>(0x3F80) : static_cast<short>(0);
  return r;
}
// One data-parallel-primitive move of a float across lanes (CTRL: the DPP control word; lanes
// with no source, and rows outside ROW_MASK, read 0)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, true));
}
// inclusive prefix sum over the 64 lanes of a wave, in registers: shifts by 1, 2, 4, 8 inside
// each 16-lane row, then the last lane of row 0 (2) added to row 1 (3), then the last lane of
// row 1 (now the total of rows 0-1) added to rows 2 and 3
__device__ __forceinline__ float wave_scan_add(float x) {
  x += dppf<0x111, 0xf>(x);   // row_shr:1
  x += dppf<0x112, 0xf>(x);   // row_shr:2
  x += dppf<0x114, 0xf>(x);   // row_shr:4
  x += dppf<0x118, 0xf>(x);   // row_shr:8
  x += dppf<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
  x += dppf<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}
// lane (lane & ~3) + perm[lane & 3] of a float (quad_perm DPP move, in registers)
template <int PERM>
__device__ __forceinline__ float quadf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), PERM, 0xf, 0xf, false));
}
// keep the scheduler from hoisting the next tile's operand loads above this point
// (bounds register pressure; the hardware still overlaps the independent work)
#define GDR_FENCE() __builtin_amdgcn_sched_barrier(0)

// operand gathers; `l4` = lane / 16
// natural K order, 128-wide swizzled rows: 8 consecutive K from k0 + 8 l4
__device__ __forceinline__ short8v opn128(const uint16_t *a, int row, int k0, int l4) {
  return ld8(a + sw128(row, k0 + 8 * l4));
}
// split-K operand of M^T from a row-major swizzled [K][128] matrix (transposing reads, see
// ldtr): K = k0 + 4 (l / 16) + i and k0 + 16 + 4 (l / 16) + i; the 16 rows of M^T (columns of
// M) are those of state tile cb in the state's channel order (see chan()), so lane l gets
// column chan(16 cb + l % 16): the four lanes of each quad read one 4-column piece
__device__ __forceinline__ short8v optr_state(const uint16_t *a, int cb, int k0, int lane) {
  const int r = 4 * (lane >> 4) + ((lane & 15) >> 2);
  const int c = 32 * (cb >> 1) + 4 * (cb & 1) + 8 * (lane & 3);
  return cat(ldtr(a + sw128(k0 + r, c)), ldtr(a + sw128(k0 + 16 + r, c)));
}
__device__ __forceinline__ short8v opsp(const uint16_t *a, int ld, int row, int k0, int l4) {
  return cat(ld4(a + row * ld + k0 + 4 * l4), ld4(a + row * ld + k0 + 16 + 4 * l4));
}

// D = (I - N)^-1 for a strictly lower 16 x 16 N given as acc(N) and acc(N^T); returns
// acc(D) and, when wanted, acc(D^T).  Doubling: N^16 = 0 so (I - N)^-1 = prod (I + N^(2^k)).
__device__ __forceinline__ void diag_inverse(float4v nA, float4v ntA, float4v &d, float4v *dt, int lane) {
  const short4v n = tobf4(nA), nt = tobf4(ntA);   // B-layout(N), B-layout(N^T)
  const float4v z = zero4();
  const short4v b2 = tobf4(mfma16(nt, n, z)), b2t = tobf4(mfma16(n, nt, z));
  const short4v b4 = tobf4(mfma16(b2t, b2, z)), b4t = tobf4(mfma16(b2, b2t, z));
  const short4v b8t = tobf4(mfma16(b4, b4t, z));
  const int l16 = lane & 15, l4 = lane >> 4;
  float4v id;
#pragma unroll
  for (int r = 0; r < 4; ++r) id[r] = (4 * l4 + r == l16) ? 1.f : 0.f;
  float4v R = nA + id;
  R = mfma16(b2t, tobf4(R), R);
  R = mfma16(b4t, tobf4(R), R);
  R = mfma16(b8t, tobf4(R), R);
  d = R;
  if (dt != nullptr) {
    const short4v b8 = tobf4(mfma16(b4t, b4, z));
    float4v Rt = ntA + id;
    Rt = mfma16(b2, tobf4(Rt), Rt);
    Rt = mfma16(b4, tobf4(Rt), Rt);
    Rt = mfma16(b8, tobf4(Rt), Rt);
    *dt = Rt;
  }
}

template <int BV, bool CHAN, bool DECAY, int WK>
__global__ __launch_bounds__(kNT, 1) void chunk_mfma_kernel(ChunkArgs a) {
  constexpr int NVW = BV / 16;             // value waves
  constexpr int NVT = kD / BV;             // value tiles per head
  constexpr int NHW = kNW - NVW;           // helper waves
  constexpr int NVI = kC * BV / 8;         // V items (8 bf16 each)
  constexpr int LDV = BV + 8;              // padded row stride of the V' tile
  // staging items of 16 bytes: q, k, explicit write key (64 x 128 each), v tile (64 x BV)
  constexpr int NQ = 1024, NK = 1024, NR = (WK == kWkExplicit) ? 1024 : 0;
  constexpr bool SCALED_E = !CHAN;         // E = beta k: beta applied after the product
  // with two value waves, P = tril(Q R^T) is formed by the value waves from the Q operands
  // they already hold for O1 and the R operands: those of Y when R = k and E = beta k (scalar
  // gains), else read beside them (channel gates: R = k, E = b (.) k; a preconditioned or
  // explicit write key: R in its own array); with a single value wave, which would have to
  // keep every R block, the helper waves form it
  constexpr bool kPv = NVW == 2;
  constexpr bool kRq = kPv && (CHAN || WK != kWkSame);   // P's R operands read separately
  __shared__ Smem<BV, CHAN, WK> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a provably wave-uniform (scalar) value: role dispatch below is then a
  // scalar branch, and each role's loop (with its barriers) runs only in its own waves
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, l4 = lane >> 4;
  const bool vwave = wave < NVW;
  const int hw = wave - NVW;               // helper wave index
  const int ht = tid - NVW * 64;           // helper thread index
  const short4v I16 = ident4(lane);

  // XCD-aware tile order: the value tiles of one head land on one XCD (shared L2)
  const int G = static_cast<int>(gridDim.x);
  const int bid = static_cast<int>(blockIdx.x);
  const int logical = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int bh = logical / NVT, vt = logical % NVT, v0 = vt * BV;
  const int H = a.H, T = a.T;
  const int b = bh / H, h = bh % H;
  const long long tokstride = static_cast<long long>(H) * kD;
  const long long head0 = (static_cast<long long>(b) * T * H + h) * kD;
  const long long gate0 = static_cast<long long>(b) * T * H + h;
  const int nchunks = (T + kC - 1) / kC;
  const int N = a.N;
  auto keep = [N](int i, int j) { return N < 0 || i - j <= N; };

  const uint16_t *gq = static_cast<const uint16_t *>(a.q);
  const uint16_t *gk = static_cast<const uint16_t *>(a.k);
  const uint16_t *gv = static_cast<const uint16_t *>(a.v);
  const uint16_t *gwk = static_cast<const uint16_t *>(a.write_key);
  const uint16_t *ger = static_cast<const uint16_t *>(a.erase);
  const uint16_t *gwr = static_cast<const uint16_t *>(a.write);
  uint16_t *gout = static_cast<uint16_t *>(a.out);

  // ---------------- one-time init: zero T (upper blocks stay zero) and P ----------------
  for (int i = tid; i < 2 * kC * kLdc; i += kNT) (&sm.t[0][0][0])[i] = 0;
  for (int i = tid; i < kC * kLdc; i += kNT) (&sm.p[0][0])[i] = 0;

  // Each role runs its own loop with the same barrier sequence, so the compiler allocates
  // registers for one role's loop-carried state at a time.
  if (vwave) {
    // the wave index is a template constant inside the value-wave loop, so every
    // wave-dependent choice below (state rows, the P blocks a wave forms) is static
    auto value_loop = [&](auto wc) {
      constexpr int W = decltype(wc)::value;
      // ---------------- value waves: S^T tiles in accumulators ----------------
      // Tile cb holds S^T[c][v = 16 W + l16] for the channels c = chan(16 cb + 4 l4 + r) =
      // 32 (cb / 2) + 8 l4 + 4 (cb % 2) + r: with this order the bf16 concatenation of tiles
      // 2j and 2j + 1 (the K = 32 B operand of Y and O1) covers channels 32 j + 8 l4 .. + 7 in
      // natural order, so the E / Q / K operands beside it are single 16-byte LDS reads; the
      // update reads R^T in the same order (optr_state) and the state is loaded and stored
      // through it once.
      float4v st[8];
      const int vrow = v0 + 16 * W + l16;   // this lane's state row
      // output element (token l16 of a 16-token block, values 4 l4 .. + 3 of this wave's rows)
      uint16_t *const obase = gout + head0 + static_cast<long long>(l16) * tokstride + v0 + 16 * W + 4 * l4;
      auto chan0 = [&](int cb) { return 32 * (cb >> 1) + 8 * l4 + 4 * (cb & 1); };
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        st[cb] = zero4();
        if (a.state_in != nullptr) {
          const float4 sv = ld4f(a.state_in + (static_cast<long long>(bh) * kD + vrow) * kD + chan0(cb));
          st[cb] = float4v{sv.x, sv.y, sv.z, sv.w};
        }
      }
      for (int c = -1; c < nchunks; ++c) {
        const int cur = c & 1;
        const int c0 = c * kC;
        const int n = min(kC, T - c0);
        short4v x4[4];
        float4v O1[4];
        __syncthreads();   // (1) chunk c staged, T(c) diagonal part ready
        if (c >= 0) {
          // Y = E S^T and O1 = e^g Q S^T for the four 16-token blocks; X = V' - e^g Y.  The
          // operands of block tb + 1 are read while block tb is multiplied.  With kPv the K
          // operands of earlier blocks are kept and the blocks (tb, jb), jb <= tb, of P are
          // formed here, split between the value waves by column block.
          short8v sb[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) sb[j] = cat(tobf4(st[2 * j]), tobf4(st[2 * j + 1]));
          const uint16_t *E = CHAN ? sm.e[cur] : sm.k[cur];
          // one register set per block for the E operands (the wave keeps those of its own P column
          // blocks alive; the others die after their block), double-buffered Q operands
          short8v ev[4][4], qv[2][4];
          short8v kq[2][4];   // kRq: R operands of this wave's two P column blocks
          // kPv: P column blocks are split 5 / 5 tiles between two value waves (blocks 0 and 3 to
          // wave 0, 1 and 2 to wave 1)
          constexpr auto p_owner = [](int jb) { return NVW == 1 ? 0 : (jb == 0 || jb == 3) ? 0 : 1; };
          constexpr auto p_slot = [](int jb) { return NVW == 1 ? jb : (jb < 2 ? 0 : 1); };
          short4v vt[2];
          // Everything a block reads from LDS is read while the previous block is multiplied:
          // LDS reads complete in order, so a read issued inside a block would also wait for
          // the prefetch issued before it.
          float4 egv[2], btv[2];
          float giv[2];
          float4 gjv[4 / NVW];   // kPv: cumulative decay at the columns of this wave's P blocks
          auto load_e = [&](int tb) {
#pragma unroll
            for (int j = 0; j < 4; ++j) ev[tb][j] = opn128(E, tb * 16 + l16, 32 * j, l4);
          };
          auto load_ops = [&](int tb, int slot) {
            if constexpr (!kPv) load_e(tb);
#pragma unroll
            for (int j = 0; j < 4; ++j) qv[slot][j] = opn128(sm.q[cur], tb * 16 + l16, 32 * j, l4);
            // V' block (rows t, columns v) in the accumulator layout, read transposed
            vt[slot] = ldtr(&sm.vp[cur][tb * 16 + 4 * l4 + (l16 >> 2)][16 * W + 4 * (l16 & 3)]);
            if (kRq && p_owner(tb) == W) {
              const uint16_t *Rp = (WK == kWkSame) ? sm.k[cur] : sm.r[cur];
#pragma unroll
              for (int j = 0; j < 4; ++j) kq[p_slot(tb)][j] = opn128(Rp, tb * 16 + l16, 32 * j, l4);
            }
            egv[slot] = ld4f(&sm.eg[cur][tb * 16 + 4 * l4]);
            if (!CHAN) btv[slot] = ld4f(&sm.beta[cur][tb * 16 + 4 * l4]);
            if (kPv) giv[slot] = sm.g2[cur][tb * 16 + l16];
          };
          if constexpr (kPv) {
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
              if (p_owner(jb) == W) gjv[p_slot(jb)] = ld4f(&sm.g2[cur][jb * 16 + 4 * l4]);
          }
          load_ops(0, 0);
          if constexpr (kPv) {
            // the E operands of every block stay live for P anyway: all of them are requested
            // now, so the phase waits for one LDS round trip instead of one per block
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) load_e(tb);
          }
          GDR_FENCE();
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) {
            const int sl = tb & 1;
            if (tb + 1 < 4) load_ops(tb + 1, sl ^ 1);
            GDR_FENCE();   // the prefetch issues before this block's products
            float4v y = zero4(), o = zero4();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              y = mfma32(ev[tb][j], sb[j], y);
              o = mfma32(qv[sl][j], sb[j], o);
            }
            const float4 eg = egv[sl];
            float4v xv;
#pragma unroll
            for (int r = 0; r < 4; ++r) xv[r] = bf(static_cast<uint16_t>(vt[sl][r])) - (&eg.x)[r] * y[r];
            if (!CHAN) {   // V' = beta v and E = beta k: beta applied to the difference
              const float4 bt = btv[sl];
              xv = float4v{bt.x * xv[0], bt.y * xv[1], bt.z * xv[2], bt.w * xv[3]};
            }
            x4[tb] = tobf4(xv);
            O1[tb] = float4v{eg.x * o[0], eg.y * o[1], eg.z * o[2], eg.w * o[3]};
            if constexpr (kPv) {
              // P^T block (jb, tb) = K_jb Q_tb^T: lane holds P[i = tb*16 + l16][j = jb*16 + 4 l4 + r]
              const int i = tb * 16 + l16;
              const float gi = giv[sl];
#pragma unroll
              for (int jb = 0; jb <= tb; ++jb) {
                if (p_owner(jb) != W) continue;
                float4v pt = zero4();
#pragma unroll
                for (int j = 0; j < 4; ++j) pt = mfma32(kRq ? kq[p_slot(jb)][j] : ev[jb][j], qv[sl][j], pt);
                const float4 gj = gjv[p_slot(jb)];
                float4v pv;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const int jj = jb * 16 + 4 * l4 + r;
                  const float x = DECAY ? pt[r] * decay2(gi - (&gj.x)[r]) : pt[r];
                  pv[r] = (jb < tb || jj <= i) ? x : 0.f;   // only the diagonal block is masked
                }
                *reinterpret_cast<short4v *>(&sm.p[i][jb * 16 + 4 * l4]) = tobf4(pv);
              }
            }
            GDR_FENCE();
          }
        }
        __syncthreads();   // (2) T(c), P(c) complete
        if (c >= 0) {
          // every LDS operand of this phase is read up front: T and P blocks, R^T for the update
          const uint16_t *Tm = &sm.t[cur][0][0], *Pm = &sm.p[0][0];
          const uint16_t *Rk = (WK == kWkSame) ? sm.k[cur] : sm.r[cur];
          // (T and P are lower triangular and their upper blocks stay zero in LDS, so the diagonal
          // blocks are read as K = 32 operands together with the zero block beside them)
          const short8v t00 = opsp(Tm, kLdc, l16, 0, l4), t10 = opsp(Tm, kLdc, 16 + l16, 0, l4);
          const short8v t20 = opsp(Tm, kLdc, 32 + l16, 0, l4), t22 = opsp(Tm, kLdc, 32 + l16, 32, l4);
          const short8v t30 = opsp(Tm, kLdc, 48 + l16, 0, l4), t32 = opsp(Tm, kLdc, 48 + l16, 32, l4);
          const short8v p00 = opsp(Pm, kLdc, l16, 0, l4), p10 = opsp(Pm, kLdc, 16 + l16, 0, l4);
          const short8v p20 = opsp(Pm, kLdc, 32 + l16, 0, l4), p22 = opsp(Pm, kLdc, 32 + l16, 32, l4);
          const short8v p30 = opsp(Pm, kLdc, 48 + l16, 0, l4), p32 = opsp(Pm, kLdc, 48 + l16, 32, l4);
          short8v ra[4], rb[4];   // R^T operands of the first half of the update
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            ra[cb] = optr_state(Rk, cb, 0, lane);
            rb[cb] = optr_state(Rk, cb, 32, lane);
          }
          float4 wdv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) wdv[j] = ld4f(&sm.wd[cur][16 * j + 4 * l4]);
          const float gC = DECAY ? sm.eg[cur][kC - 1] : 1.f;

          // D = T X
          const short8v x01 = cat(x4[0], x4[1]), x23 = cat(x4[2], x4[3]);
          float4v D[4];
          D[0] = mfma32(t00, x01, zero4());
          D[1] = mfma32(t10, x01, zero4());
          D[2] = mfma32(t22, x23, mfma32(t20, x01, zero4()));
          D[3] = mfma32(t32, x23, mfma32(t30, x01, zero4()));
          // state update S^T <- e^{g_C} S^T + R^T (wd (.) D), interleaved with O2 = P D
          short4v w4[4], d4[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            w4[j] = tobf4(float4v{wdv[j].x * D[j][0], wdv[j].y * D[j][1], wdv[j].z * D[j][2], wdv[j].w * D[j][3]});
            d4[j] = tobf4(D[j]);
          }
          const short8v w01 = cat(w4[0], w4[1]), w23 = cat(w4[2], w4[3]);
          const short8v d01 = cat(d4[0], d4[1]), d23 = cat(d4[2], d4[3]);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            float4v acc = st[cb];
            if (DECAY) acc *= gC;
            st[cb] = mfma32(rb[cb], w23, mfma32(ra[cb], w01, acc));
            ra[cb] = optr_state(Rk, cb + 4, 0, lane);   // second half, read behind the first
            rb[cb] = optr_state(Rk, cb + 4, 32, lane);
          }
#pragma unroll
          for (int cb = 4; cb < 8; ++cb) {
            float4v acc = st[cb];
            if (DECAY) acc *= gC;
            st[cb] = mfma32(rb[cb - 4], w23, mfma32(ra[cb - 4], w01, acc));
          }
          float4v O2[4];
          // O1 seeds the accumulator: O = scale (O1 + P D)
          O2[0] = mfma32(p00, d01, O1[0]);
          O2[1] = mfma32(p10, d01, O1[1]);
          O2[2] = mfma32(p22, d23, mfma32(p20, d01, O1[2]));
          O2[3] = mfma32(p32, d23, mfma32(p30, d01, O1[3]));
          // output: transpose each 16 x 16 block by an identity product so a lane holds four
          // consecutive values of one token (the four products issue back to back), then 8-byte
          // stores from a per-lane base and uniform offsets; only a partial last chunk masks
          if (a.scale != 1.f) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) O2[tb] = a.scale * O2[tb];
          }
          short4v pk[4];
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) pk[tb] = tobf4(mfma16(tobf4(O2[tb]), I16, zero4()));
          uint16_t *ob = obase + static_cast<long long>(c0) * tokstride;
          if (n == kC) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) *reinterpret_cast<short4v *>(ob + tb * 16 * tokstride) = pk[tb];
          } else {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
              if (tb * 16 + l16 < n) *reinterpret_cast<short4v *>(ob + tb * 16 * tokstride) = pk[tb];
          }
        }
        if (WK == kWkPrecond) __syncthreads();   // (3) write keys of chunk c + 1 formed
      }
      if (a.state_out != nullptr) {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
          *reinterpret_cast<float4 *>(a.state_out + (static_cast<long long>(bh) * kD + vrow) * kD + chan0(cb)) =
              make_float4(st[cb][0], st[cb][1], st[cb][2], st[cb][3]);
      }
    };
    if constexpr (NVW == 1) {
      value_loop(std::integral_constant<int, 0>{});
    } else {
      if (wave == 0) value_loop(std::integral_constant<int, 0>{});
      else value_loop(std::integral_constant<int, 1>{});
    }
    return;
  }

  // ============================== helper waves ==============================
  // One staging point per chunk: every item of chunk c + 1 is written to LDS from registers
  // loaded a full iteration earlier, then the loads of chunk c + 2 are issued.  Items are
  // 16-byte granules in blocks of 64 (one wave-wide load): 16 blocks each of q, k and an
  // explicit write key (64 x 128 bf16), then the blocks of the 64 x BV value tile.  Block
  // s * NHW + hw is slot s of helper wave hw, so everything about a block (source, LDS
  // destination, row / column split) is wave-uniform.  Every slot loads and is staged
  // unconditionally -- a slot past the last block repeats it without storing -- so the
  // registers of a load are first read one iteration after it was issued and the loads of
  // a chunk issue back to back.  Rows past the end of the sequence are read clamped to the
  // last row and zeroed when staged.
  constexpr int NBP = (NQ + NK + NR) / 64;     // blocks of 64 x 128 arrays
  constexpr int NB = NBP + NVI / 64;
  constexpr int NSB = (NB + NHW - 1) / NHW;    // block slots per helper wave
  constexpr int VSH = BV == 32 ? 2 : 1;        // log2(items per value-tile row)
  uint4 pa[NSB], pb[NSB];
#pragma unroll
  for (int s = 0; s < NSB; ++s) pa[s] = pb[s] = make_uint4(0u, 0u, 0u, 0u);
  float gla = 0.f, gbeta = 0.f;                // gates of token `lane` of the staged chunk
  const bool gate_wave = wave == kNW - 1;
  const int tok32 = H * kD;                    // token stride; 64 * tok32 < 2^31 (H <= 65535)
  auto slot_block = [&](int s) { return min(s * NHW + hw, NB - 1); };
  // item u of block blk: row u >> sh, column col0 + (u & msk) * 8
  auto item_rc = [&](int blk, int &t, int &col) {
    const bool isv = blk >= NBP;
    const int u = (isv ? blk - NBP : blk & 15) * 64 + lane;
    t = isv ? u >> VSH : u >> 4;
    col = isv ? (u & (BV / 8 - 1)) * 8 : (u & 15) * 8;
  };

  // Per-slot addressing, fixed for the whole sequence: this lane's item of chunk 0 in global
  // memory (row srow of the chunk) and its LDS byte offset in buffer 0 of its array, so the
  // per-chunk work is a clamp, one multiply-add, the loads and the stores.
  const uint16_t *gsrc[NSB], *gsrc2[NSB];
  int srow[NSB], loff[NSB], lstr[NSB], eoff[NSB];
  char *const smb = reinterpret_cast<char *>(&sm);
#pragma unroll
  for (int s = 0; s < NSB; ++s) {
    const int blk = slot_block(s);
    const bool isv = blk >= NBP;
    const int arr = blk >> 4;
    int t, col;
    item_rc(blk, t, col);
    srow[s] = t;
    const long long g0 = head0 + (isv ? v0 : 0) + col;
    gsrc[s] = (isv ? gv : arr == 0 ? gq : arr == 1 ? gk : gwk) + g0;
    gsrc2[s] = CHAN ? (isv ? gwr : ger) + g0 : gsrc[s];
    uint16_t *d0 = isv ? &sm.vp[0][t][col] : (arr == 0 ? sm.q[0] : arr == 1 ? sm.k[0] : sm.r[0]) + sw128(t, col);
    loff[s] = static_cast<int>(reinterpret_cast<char *>(d0) - smb);
    lstr[s] = isv ? static_cast<int>(sizeof(sm.vp[0])) : kC * kD * 2;
    eoff[s] = static_cast<int>(reinterpret_cast<char *>(sm.e[0] + (CHAN ? sw128(t, col) : 0)) - smb);
  }

  auto load_items = [&](int c) {
    const int c0 = c * kC, nm1 = min(kC, T - c0) - 1;
#pragma unroll
    for (int s = 0; s < NSB; ++s) {
      const long long off = static_cast<long long>(c0 + min(srow[s], nm1)) * tokstride;
      pa[s] = *reinterpret_cast<const uint4 *>(gsrc[s] + off);
      if (CHAN) pb[s] = *reinterpret_cast<const uint4 *>(gsrc2[s] + off);
    }
    const long long gi = gate0 + static_cast<long long>(c0) * H + min(lane, nm1) * H;
    if (DECAY) gla = a.log_alpha[gi];
    if (!CHAN) gbeta = a.beta[gi];
  };
  auto stage_items = [&](int c, int buf) {
    const int n = min(kC, T - c * kC);
#pragma unroll
    for (int s = 0; s < NSB; ++s) {
      const int blk = slot_block(s);
      const bool live = s * NHW + hw < NB;
      const bool isv = blk >= NBP, isk = !isv && (blk >> 4) == 1;
      uint4 x = pa[s];
      if (n < kC) {   // rows past the end of the sequence (read clamped) are zeroed
        const uint32_t m = srow[s] < n ? 0xffffffffu : 0u;
        x = make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
      }
      uint4 xg = x;   // gated copy: erase (.) k, write (.) v
      if (CHAN) {
        xg.x = f32x2_to_bf16x2_bits(elem(pb[s], 0) * elem(x, 0), elem(pb[s], 1) * elem(x, 1));
        xg.y = f32x2_to_bf16x2_bits(elem(pb[s], 2) * elem(x, 2), elem(pb[s], 3) * elem(x, 3));
        xg.z = f32x2_to_bf16x2_bits(elem(pb[s], 4) * elem(x, 4), elem(pb[s], 5) * elem(x, 5));
        xg.w = f32x2_to_bf16x2_bits(elem(pb[s], 6) * elem(x, 6), elem(pb[s], 7) * elem(x, 7));
      }
      if (live) {
        // (component-wise choice: a whole-vector choice by a run-time flag goes through memory)
        const uint4 y = CHAN ? make_uint4(isv ? xg.x : x.x, isv ? xg.y : x.y, isv ? xg.z : x.z, isv ? xg.w : x.w) : x;
        *reinterpret_cast<uint4 *>(smb + loff[s] + buf * lstr[s]) = y;
        if (CHAN && isk) *reinterpret_cast<uint4 *>(smb + eoff[s] + buf * (kC * kD * 2)) = xg;
      }
    }
    // gates: cumulative log decay in log2 units and the quantities derived from it.  Every
    // helper wave loaded the gate registers; all of them take delivery here (so no load is
    // left pending on a path that skips it) and the gate wave forms the scan.
    const float la = gla, bt = gbeta;
    asm volatile("" ::"v"(la), "v"(bt));
    if (gate_wave) {
      const bool ok = lane < n;
      const float beta_t = ok ? bt : 0.f;
      // (a scan in registers: a shuffle through LDS would cost one LDS round trip per step)
      const float g = wave_scan_add(ok ? la * kLog2e : 0.f);
      const float glast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g), n - 1));
      sm.g2[buf][lane] = g;
      sm.eg[buf][lane] = DECAY ? decay2(g) : 1.f;
      sm.wd[buf][lane] = DECAY ? decay2(glast - g) : 1.f;
      sm.beta[buf][lane] = beta_t;
      if (WK == kWkPrecond) {
        const float tg = static_cast<float>(a.t0 + static_cast<long long>(c) * kC + lane + 1);
        sm.ic[buf][lane] = 1.f / (-expm1f(tg * a.log_rho));   // 1 / (1 - rho^t)
      }
    }
  };
  // (E R^T) tile for rows ib, cols jb (trans: the transposed tile), scaled to A = -L
  auto a_tile = [&](int buf, int ib, int jb, bool trans) -> float4v {
    const uint16_t *E = CHAN ? sm.e[buf] : sm.k[buf];
    const uint16_t *R = (WK == kWkSame) ? sm.k[buf] : sm.r[buf];
    const uint16_t *A = trans ? R : E;
    const uint16_t *B = trans ? E : R;
    const int ra = (trans ? jb : ib) * 16 + l16, rb = (trans ? ib : jb) * 16 + l16;
    float4v acc = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma32(opn128(A, ra, 32 * s, l4), opn128(B, rb, 32 * s, l4), acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = trans ? ib * 16 + l16 : ib * 16 + 4 * l4 + r;
      const int j = trans ? jb * 16 + 4 * l4 + r : jb * 16 + l16;
      float x = acc[r];
      if (SCALED_E) x *= sm.beta[buf][i];
      if (DECAY) x *= decay2(sm.g2[buf][i] - sm.g2[buf][j]);
      acc[r] = (j < i) ? -x : 0.f;
    }
    return acc;
  };
  // P tile job (blocks (ib, jb), jb <= ib, numbered row by row), computed transposed
  // (P^T = R Q^T) so each lane writes 4 columns of one row of P
  auto p_tile = [&](int buf, int job) {
    const uint16_t *R = (WK == kWkSame) ? sm.k[buf] : sm.r[buf];
    const int ib = job < 1 ? 0 : job < 3 ? 1 : job < 6 ? 2 : 3;
    const int jb = job - ib * (ib + 1) / 2;
    float4v acc = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = mfma32(opn128(R, jb * 16 + l16, 32 * s, l4), opn128(sm.q[buf], ib * 16 + l16, 32 * s, l4), acc);
    // lane: P[i = ib*16 + l16][j = jb*16 + 4 l4 + r]
    const int i = ib * 16 + l16;
    float4v v;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = jb * 16 + 4 * l4 + r;
      float x = acc[r];
      if (DECAY) x *= decay2(sm.g2[buf][i] - sm.g2[buf][j]);
      v[r] = (j <= i) ? x : 0.f;
    }
    *reinterpret_cast<short4v *>(&sm.p[i][jb * 16 + 4 * l4]) = tobf4(v);
  };
  // write acc(X^T) of the 16 x 16 block (rb, cb) of a row-major [64][kLdc] bf16 matrix as
  // 8-byte rows (lane: row rb*16 + l16, columns cb*16 + 4 l4 .. + 3), band-masked
  auto put_rows = [&](uint16_t *M, int rb, int cb, float4v xt, bool lower_only) {
    const int i = rb * 16 + l16;
    float4v v;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = cb * 16 + 4 * l4 + r;
      v[r] = (keep(i, j) && (!lower_only || j <= i)) ? xt[r] : 0.f;
    }
    *reinterpret_cast<short4v *>(M + i * kLdc + cb * 16 + 4 * l4) = tobf4(v);
  };

  // preconditioner accumulator: helper threads ht < 256 own channels 2 p, 2 p + 1 (p = ht / 4)
  // and tokens 16 s .. 16 s + 15 (s = ht % 4) of a chunk; the four segments of a channel pair
  // are the four lanes of a quad.  The accumulator entering the chunk is kept in all four.
  const bool pc_thread = ht < 256;
  const int pc_p = ht >> 2, pc_seg = ht & 3;
  float hc0 = 0.f, hc1 = 0.f;
  if (WK == kWkPrecond && pc_thread) {
    hc0 = a.pc_h_in != nullptr ? a.pc_h_in[static_cast<long long>(bh) * kD + 2 * pc_p] : a.h0;
    hc1 = a.pc_h_in != nullptr ? a.pc_h_in[static_cast<long long>(bh) * kD + 2 * pc_p + 1] : a.h0;
  }

  if (nchunks > 0) load_items(0);
  for (int c = -1; c < nchunks; ++c) {
    const int cur = c & 1, nxt = (c + 1) & 1;
    const bool have_next = c + 1 < nchunks;

    __syncthreads();   // (1)
    // The two T_ba waves read every operand of their block products (T blocks and A blocks of
    // chunk c, formed before the barrier) ahead of their staging writes: LDS operations of a
    // wave complete in order, so reads issued after the writes would wait for them to drain,
    // while issued first they let the writes drain under the products.
    uint16_t *Tc = &sm.t[cur][0][0];
    const int qb = hw;   // column block of the lower-left quadrant formed by this wave
    // A layout of block (rb, kb) of T; B layout of block (kb, cb) by a transposing read
    auto arow = [&](int rb, int kb) { return ld4(Tc + (rb * 16 + l16) * kLdc + kb * 16 + 4 * l4); };
    auto bcol = [&](int kb, int cb) {
      return ldtr(Tc + (kb * 16 + 4 * l4 + (l16 >> 2)) * kLdc + cb * 16 + 4 * (l16 & 3));
    };
    auto lrow = [&](int s, int u) { return ld4(&sm.lba[s * 16 + l16][u * 16 + 4 * l4]); };
    short4v o_a33, o_b22, o_a22, o_a32, o_a10, o_d, o_a11, o_l00, o_l01, o_l10, o_l11;
    if (c >= 0 && hw < 2) {
      o_a33 = arow(3, 3);
      o_b22 = bcol(2, 2);
      o_a22 = arow(2, 2);
      o_a32 = ld4(&sm.aod[1][l16][4 * l4]);
      o_l01 = lrow(0, 1);
      o_l11 = lrow(1, 1);
      if (qb == 0) {
        o_a10 = ld4(&sm.aod[0][l16][4 * l4]);
        o_d = bcol(0, 0);
        o_a11 = arow(1, 1);
        o_l00 = lrow(0, 0);
        o_l10 = lrow(1, 0);
      } else {
        o_d = bcol(1, 1);
      }
    }
    if (have_next) {
      stage_items(c + 1, nxt);
      if (c + 2 < nchunks) load_items(c + 2);
    }
    if (c >= 0) {
      if (hw < 2) {
        // remaining blocks of T(c): T_10 = D_1 A_10 D_0, T_32 = D_3 A_32 D_2 and column block
        // qb = hw of the lower-left quadrant T_ba = T_b A_ba T_a
        const float4v t32 = mfma16(o_a33, tobf4(mfma16(o_a32, o_b22, zero4())), zero4());
        const short4v t32a = tobf4(mfma16(tobf4(t32), I16, zero4()));   // A layout of T_32
        float4v z0, z1;                                                  // Z = A_ba T_a[:, qb]
        if (qb == 0) {
          const short4v d0 = o_d;
          const float4v t10 = mfma16(o_a11, tobf4(mfma16(o_a10, d0, zero4())), zero4());
          const short4v t10b = tobf4(t10);
          z0 = mfma16(o_l01, t10b, mfma16(o_l00, d0, zero4()));
          z1 = mfma16(o_l11, t10b, mfma16(o_l10, d0, zero4()));
          put_rows(Tc, 1, 0, mfma16(t10b, I16, zero4()), false);
        } else {
          const short4v d1 = o_d;
          z0 = mfma16(o_l01, d1, zero4());
          z1 = mfma16(o_l11, d1, zero4());
          put_rows(Tc, 3, 2, mfma16(tobf4(t32), I16, zero4()), false);
        }
        const short4v z0b = tobf4(z0), z1b = tobf4(z1);
        const float4v tb2 = mfma16(o_a22, z0b, zero4());
        const float4v tb3 = mfma16(o_a33, z1b, mfma16(t32a, z0b, zero4()));
        put_rows(Tc, 2, qb, mfma16(tobf4(tb2), I16, zero4()), false);
        put_rows(Tc, 3, qb, mfma16(tobf4(tb3), I16, zero4()), false);
      }
      // P tiles (10 lower blocks) unless the value waves form them: jobs 8, 9 on the two T_ba
      // waves, 0..7 on the others
      if constexpr (!kPv) {
        if (hw < 2) {
          p_tile(cur, 8 + hw);
        } else {
          p_tile(cur, hw - 2);
          if (hw - 2 + (NHW - 2) < 8) p_tile(cur, hw - 2 + (NHW - 2));
        }
      }
    }
    __syncthreads();   // (2)

    if (WK == kWkPrecond) {
      // write keys of chunk c + 1: u = k / (h / (1 - rho^t) + eps), h_t = rho h_{t-1} + k_t^2
      if (have_next && pc_thread) {
        // this thread: channels 2 p, 2 p + 1, tokens s0 .. s0 + 15 of chunk c + 1 (rows past the
        // end of the sequence were staged as zero and are masked below).  Pass 1 forms the
        // segment's affine map h -> rm h + acc; the four segments' maps are composed across the
        // quad by register moves (an inclusive scan of two steps, then a shift by one); pass 2
        // reruns the segment from its entering accumulator and writes u.  Keys and write keys
        // move as bf16 pairs (4-byte LDS accesses).
        const uint16_t *Kn = sm.k[nxt];
        const int nn = min(kC, T - (c + 1) * kC);
        const int s0 = pc_seg * 16, cp = 2 * pc_p;
        const int m = max(0, min(16, nn - s0));
        float k0[16], k1[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t w = *reinterpret_cast<const uint32_t *>(Kn + sw128(s0 + i, cp));
          k0[i] = bf(w & 0xffffu);
          k1[i] = bf(w >> 16);
        }
        float a0 = 0.f, a1 = 0.f, rm = 1.f;
        if (m == 16) {   // every token present (all but a partial last chunk)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            a0 = fmaf(a.rho, a0, k0[i] * k0[i]);
            a1 = fmaf(a.rho, a1, k1[i] * k1[i]);
          }
          const float r2 = a.rho * a.rho, r4 = r2 * r2, r8 = r4 * r4;
          rm = r8 * r8;
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const bool on = i < m;
            a0 = on ? fmaf(a.rho, a0, k0[i] * k0[i]) : a0;
            a1 = on ? fmaf(a.rho, a1, k1[i] * k1[i]) : a1;
            rm = on ? rm * a.rho : rm;
          }
        }
        // inclusive scan over the quad: F_s = f_s o F_{s-1} = (rm_s R, rm_s A + acc_s)
        {
          const float pr = quadf<0x90>(rm), p0 = quadf<0x90>(a0), p1 = quadf<0x90>(a1);   // lane s - 1
          if (pc_seg >= 1) {
            a0 = fmaf(rm, p0, a0);
            a1 = fmaf(rm, p1, a1);
            rm *= pr;
          }
          const float qr = quadf<0x44>(rm), q0 = quadf<0x44>(a0), q1 = quadf<0x44>(a1);   // lane s - 2
          if (pc_seg >= 2) {
            a0 = fmaf(rm, q0, a0);
            a1 = fmaf(rm, q1, a1);
            rm *= qr;
          }
        }
        // entering accumulator of this segment: F_{s-1}(h_chunk); the next chunk's: F_3(h_chunk)
        const float er = quadf<0x90>(rm), e0 = quadf<0x90>(a0), e1 = quadf<0x90>(a1);
        float h0v = pc_seg == 0 ? hc0 : fmaf(er, hc0, e0);
        float h1v = pc_seg == 0 ? hc1 : fmaf(er, hc1, e1);
        const float lr = quadf<0xff>(rm), l0 = quadf<0xff>(a0), l1 = quadf<0xff>(a1);
        uint16_t *Rn = sm.r[nxt];
        float4 ic4;
        // (the key is rounded to bf16 next, so the hardware reciprocal is accurate enough)
        if (m == 16) {   // no masking: a compare and four selects fewer per token
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if ((i & 3) == 0) ic4 = ld4f(&sm.ic[nxt][s0 + i]);
            const float icv = (&ic4.x)[i & 3];
            h0v = fmaf(a.rho, h0v, k0[i] * k0[i]);
            h1v = fmaf(a.rho, h1v, k1[i] * k1[i]);
            const float u0 = k0[i] * __builtin_amdgcn_rcpf(fmaf(h0v, icv, a.eps));
            const float u1 = k1[i] * __builtin_amdgcn_rcpf(fmaf(h1v, icv, a.eps));
            *reinterpret_cast<uint32_t *>(Rn + sw128(s0 + i, cp)) = f32x2_to_bf16x2_bits(u0, u1);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if ((i & 3) == 0) ic4 = ld4f(&sm.ic[nxt][s0 + i]);
            const float icv = (&ic4.x)[i & 3];
            const bool on = i < m;
            h0v = on ? fmaf(a.rho, h0v, k0[i] * k0[i]) : h0v;
            h1v = on ? fmaf(a.rho, h1v, k1[i] * k1[i]) : h1v;
            const float u0 = k0[i] * __builtin_amdgcn_rcpf(fmaf(h0v, icv, a.eps));
            const float u1 = k1[i] * __builtin_amdgcn_rcpf(fmaf(h1v, icv, a.eps));
            *reinterpret_cast<uint32_t *>(Rn + sw128(s0 + i, cp)) = f32x2_to_bf16x2_bits(on ? u0 : 0.f, on ? u1 : 0.f);
          }
        }
        hc0 = fmaf(lr, hc0, l0);
        hc1 = fmaf(lr, hc1, l1);
      }
      __syncthreads();   // (3)
    }

    if (have_next) {
      const int nb = nxt;
      // off-diagonal blocks of A: A_10, A_32 (for T_10, T_32) and the four blocks of A_ba (jobs
      // 0..5); a wave forms its share together (operands first, then the product chains).  Job
      // q of a batch is job0 + q * jstep; jobs past the last repeat it without storing.
      auto a_jobs = [&](auto njc, int job0, int jstep) {
        constexpr int NJ = decltype(njc)::value;
        const uint16_t *E = CHAN ? sm.e[nb] : sm.k[nb];
        const uint16_t *R = (WK == kWkSame) ? sm.k[nb] : sm.r[nb];
        int ib[NJ], jb[NJ];
        short8v ra[NJ][4], eb[NJ][4];
#pragma unroll
        for (int q = 0; q < NJ; ++q) {
          const int job = min(job0 + q * jstep, 5);
          ib[q] = job == 0 ? 1 : job == 1 ? 3 : 2 + ((job - 2) >> 1);
          jb[q] = job == 0 ? 0 : job == 1 ? 2 : (job - 2) & 1;
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) {
            ra[q][s2] = opn128(R, jb[q] * 16 + l16, 32 * s2, l4);
            eb[q][s2] = opn128(E, ib[q] * 16 + l16, 32 * s2, l4);
          }
        }
        float4v acc[NJ];
#pragma unroll
        for (int q = 0; q < NJ; ++q) acc[q] = zero4();
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
          for (int q = 0; q < NJ; ++q) acc[q] = mfma32(ra[q][s2], eb[q][s2], acc[q]);
        }
#pragma unroll
        for (int q = 0; q < NJ; ++q) {
          const int job = job0 + q * jstep;
          // lane: (E R^T)[i = ib*16 + l16][j = jb*16 + 4 l4 + r], scaled to A = -L (j < i always)
          const int i = ib[q] * 16 + l16;
          const float bi = SCALED_E ? sm.beta[nb][i] : 1.f, gi = sm.g2[nb][i];
          const float4 gj = ld4f(&sm.g2[nb][jb[q] * 16 + 4 * l4]);
          float4v x;
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] = -(DECAY ? acc[q][r] * bi * decay2(gi - (&gj.x)[r]) : acc[q][r] * bi);
          if (job < 6) {
            uint16_t *dst = job < 2 ? &sm.aod[job][l16][4 * l4] : &sm.lba[(ib[q] - 2) * 16 + l16][jb[q] * 16 + 4 * l4];
            *reinterpret_cast<short4v *>(dst) = tobf4(x);
          }
        }
      };
      // With six helpers the two A waves would carry three jobs each against one diagonal
      // inverse per other wave, so waves 0 and 1 (the lightest: their other work is before the
      // second barrier) take jobs 4 and 5 after their inverse.
      constexpr int NOW = NHW - 4;               // waves on A jobs only
      constexpr bool kSplitA = NOW == 2;
      if (hw < 4) {
        // diagonal block hw of T: D = (I - A_pp)^-1
        const float4v n = a_tile(nb, hw, hw, false);
        const float4v nt = mfma16(tobf4(n), I16, zero4());
        float4v d, dt;
        diag_inverse(n, nt, d, &dt, lane);
        put_rows(&sm.t[nb][0][0], hw, hw, dt, true);
        if constexpr (kSplitA) {
          if (hw < 2) a_jobs(std::integral_constant<int, 1>{}, 4 + hw, 1);
        }
      } else if constexpr (kSplitA) {
        a_jobs(std::integral_constant<int, 2>{}, hw - 4, 2);
      } else {
        a_jobs(std::integral_constant<int, (6 + NOW - 1) / NOW>{}, hw - 4, NOW);
      }
    }
  }
  if (WK == kWkPrecond && a.pc_h_out != nullptr && vt == 0 && pc_thread && pc_seg == 0)
  {
    a.pc_h_out[static_cast<long long>(bh) * kD + 2 * pc_p] = hc0;
    a.pc_h_out[static_cast<long long>(bh) * kD + 2 * pc_p + 1] = hc1;
  }
}

template <int BV, bool CHAN, bool DECAY, int WK>
hipError_t launch4(const ChunkArgs &a, hipStream_t s) {
  const int grid = a.B * a.H * (kD / BV);
  hipLaunchKernelGGL((chunk_mfma_kernel<BV, CHAN, DECAY, WK>), dim3(grid), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

template <int BV>
hipError_t launch_bv(const ChunkArgs &a, hipStream_t s) {
  const bool decay = a.decay == GDR_DECAY_SCALAR;
  if (a.gain == GDR_GAIN_CHANNEL)   // channel gains only with the write key equal to the key
    return decay ? launch4<BV, true, true, kWkSame>(a, s) : launch4<BV, true, false, kWkSame>(a, s);
  switch (a.wkey) {
    case GDR_WKEY_DIAG_PRECOND:
      return decay ? launch4<BV, false, true, kWkPrecond>(a, s) : launch4<BV, false, false, kWkPrecond>(a, s);
    case GDR_WKEY_EXPLICIT:
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
  if (d.neumann_order >= 0 && d.residual_steps > 0) return false;
  if (d.decay == GDR_DECAY_CHANNEL) return false;
  const void *p16[] = {in.q, in.k, in.v, in.erase, in.write, in.write_key, out, state_in, state_out};
  for (const void *p : p16)
    if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return false;
  return true;
}

// Value-tile width.  Every workgroup walks its whole sequence, so a call takes about
// (chunks) x (time per chunk) once all workgroups are resident.  With write key k the 32-row
// tile (two value waves forming P from their own operands) has the shorter chunk time and is
// used even when it leaves CUs idle; the other variants keep the widest tile that still gives
// every CU a workgroup.  GDR_MFMA_BV=16|32 overrides (tuning runs).
static int chunk_mfma_bv(const ChunkArgs &a) {
  const char *e = getenv("GDR_MFMA_BV");
  const int forced = e == nullptr ? 0 : atoi(e);
  if (forced == 16 || forced == 32) return forced;
  if (a.wkey == GDR_WKEY_SAME) return 32;
  return (static_cast<long long>(a.B) * a.H * (kD / 32) >= 256) ? 32 : 16;
}

hipError_t launch_chunk_mfma(const ChunkArgs &a, hipStream_t s) {
  return chunk_mfma_bv(a) == 32 ? launch_bv<32>(a, s) : launch_bv<16>(a, s);
}

}  // namespace gdr
