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
//    from HBM), build T and P.  T is formed by blocked forward substitution: each 16 x 16
//    diagonal block D = (I - N)^-1 (one per helper wave, as soon as the chunk is staged) by
//    substitution inside its 4 x 4 diagonal sub-blocks in fp32 and two levels of block
//    products on the matrix cores with every factor carried as a bf16 pair (hi + lo); the
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
  uint16_t t[2][kC][kLdc];                                 // T, bf16 hi part
  uint16_t tl[2][kC][kLdc];                                // T, bf16 lo part (T - hi, rounded)
  uint16_t p[kC][kLdc];                                    // P (one buffer)
  uint16_t lba[32][kLdl], lbal[32][kLdl];                  // A_ba = -L_ba (rows 32.., cols ..31), hi / lo
  uint16_t aod[2][16][20], aodl[2][16][20];                // A_10, A_32, hi / lo
  float g2[2][kC], eg[2][kC], wd[2][kC], beta[2][kC], ic[2][kC];
};

// (per-channel decay on the prepared record) the chunk's state decay per key channel, double
// buffered, in the space of A_ba, which that variant never forms
template <int BV, bool CHAN, int WK>
__device__ __forceinline__ float *gcv_of(Smem<BV, CHAN, WK> &sm, int buf) {
  static_assert(sizeof(Smem<BV, CHAN, WK>::lba) >= 2 * kD * sizeof(float), "per-channel decay buffer");
  return reinterpret_cast<float *>(&sm.lba[0][0]) + buf * kD;
}
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

__device__ __forceinline__ float4v unbf4(short4v v) {
  return float4v{bf(static_cast<uint16_t>(v[0])), bf(static_cast<uint16_t>(v[1])), bf(static_cast<uint16_t>(v[2])),
                 bf(static_cast<uint16_t>(v[3]))};
}

// fp32 values as a bf16 pair: x[0] = bf16(v), x[1] = bf16(v - x[0])
struct Pair {
  short4v h, l;
};
__device__ __forceinline__ Pair split4(float4v v) {
  const short4v h = tobf4(v);
  return Pair{h, tobf4(v - unbf4(h))};
}
// c + X Y for 16 x 16 X, Y held as bf16 pairs (x: the A operand of X, y: the B operand of Y),
// about 16 significant bits each.  The hi / lo pair of X fills the K slots a K = 16 product would
// pad with zeros: X_hi Y_hi + X_lo Y_hi in one instruction, X_hi Y_lo in a second (the X_lo Y_lo
// term, ~2^-16 relative, is dropped).
__device__ __forceinline__ float4v mm2(const Pair &x, const Pair &y, float4v c) {
  return mfma16(x.h, y.l, mfma32(cat(x.h, x.l), cat(y.h, y.h), c));
}
__device__ __forceinline__ float4v mm2(const Pair &x, const Pair &y) { return mm2(x, y, float4v{0.f, 0.f, 0.f, 0.f}); }

// acc(D^T) of D = (I - N)^-1 for a strictly lower 16 x 16 N given in fp32 as acc(N) and acc(N^T),
// by blocked forward substitution (chunk-wise form of the MatMul-only inversion summary,
// "Declaracao do Problema"):
//  * the four 4 x 4 diagonal sub-blocks by substitution in fp32.  Each sub-block sits in one
//    lane quad (in acc(N) quad lane l holds its column l, in acc(N^T) its row l), so the
//    entries of N it needs arrive by quad broadcasts: columns of D1 = blockdiag(sub-block
//    inverses) from acc(N) (x_r = [r == j] + sum_{l < r} N_rl x_l), rows from acc(N^T)
//    (y_r = [r == i] + sum_{l > r} y_l N_lr);
//  * two levels of block products D <- D + D N_m D, N_m the part of N that joins the blocks of
//    the level (the 4 x 4 blocks (1, 0) and (3, 2), then the 8 x 8 block (1, 0)): the inverse of
//    [[P, 0], [M, Q]] has P^-1 and Q^-1 on its diagonal and Q^-1 M P^-1 below it.
// Every intermediate is part of the inverse itself, so no factor grows past |D| (the series
// (I + N)(I + N^2)(I + N^4)(I + N^8) is exact too, but its powers of N are far larger than D
// when keys are correlated or gains exceed 1, and rounded to bf16 they swamp it).
__device__ __forceinline__ float4v diag_inverse_t(float4v n, float4v nt, int lane) {
  const int l16 = lane & 15, l4 = lane >> 4;
  const bool dq = (l16 >> 2) == l4;        // this quad holds a diagonal sub-block
  const int jq = l16 & 3;                  // the lane's column (acc(N)) or row (acc(N^T)) in it
  const float one0 = jq == 0 ? 1.f : 0.f, one1 = jq == 1 ? 1.f : 0.f, one2 = jq == 2 ? 1.f : 0.f,
              one3 = jq == 3 ? 1.f : 0.f;
  float4v d1, dt1;
  {   // columns: N_rl is register r of quad lane l
    const float n10 = quadf<0x00>(n[1]), n20 = quadf<0x00>(n[2]), n30 = quadf<0x00>(n[3]);
    const float n21 = quadf<0x55>(n[2]), n31 = quadf<0x55>(n[3]), n32 = quadf<0xaa>(n[3]);
    const float x0 = one0;
    const float x1 = fmaf(n10, x0, one1);
    const float x2 = fmaf(n21, x1, fmaf(n20, x0, one2));
    const float x3 = fmaf(n32, x2, fmaf(n31, x1, fmaf(n30, x0, one3)));
    d1 = dq ? float4v{x0, x1, x2, x3} : zero4();
  }
  {   // rows: N_lr is register r of quad lane l
    const float n10 = quadf<0x55>(nt[0]), n20 = quadf<0xaa>(nt[0]), n21 = quadf<0xaa>(nt[1]);
    const float n30 = quadf<0xff>(nt[0]), n31 = quadf<0xff>(nt[1]), n32 = quadf<0xff>(nt[2]);
    const float y3 = one3;
    const float y2 = fmaf(y3, n32, one2);
    const float y1 = fmaf(y3, n31, fmaf(y2, n21, one1));
    const float y0 = fmaf(y3, n30, fmaf(y2, n20, fmaf(y1, n10, one0)));
    dt1 = dq ? float4v{y0, y1, y2, y3} : zero4();
  }
  // acc(N_m^T): lane (row l16, column block l4) of N; every factor is split into its bf16 pair
  // once and reused
  const int rb4 = l16 >> 2;
  const bool m1 = (rb4 & 1) != 0 && l4 == rb4 - 1, m2 = (l16 >> 3) == 1 && (l4 >> 1) == 0;
  const Pair ntp = split4(nt);
  const short4v zs = {0, 0, 0, 0};
  const Pair n1p{m1 ? ntp.h : zs, m1 ? ntp.l : zs}, n2p{m2 ? ntp.h : zs, m2 ? ntp.l : zs};
  const Pair d1p = split4(d1), dt1p = split4(dt1);
  const Pair z1p = split4(mm2(n1p, d1p));            // N_1 D_1
  const float4v d2 = mm2(dt1p, z1p, d1);             // D_2 = D_1 + D_1 Z_1
  const float4v dt2 = mm2(z1p, dt1p, dt1);           // D_2^T = D_1^T + Z_1^T D_1^T
  const Pair z2p = split4(mm2(n2p, split4(d2)));     // N_2 D_2
  return mm2(z2p, split4(dt2), dt2);                 // D^T = D_2^T + Z_2^T D_2^T
}

// Role index of the calling wave, wave-uniform (a scalar), so role dispatch is a scalar
// branch.  Waves w and w + 4 share a SIMD; by default the value waves (0, 1) share theirs with
// two staging waves (4, 5).  With channel gains, whose staging (two loads and a product per
// item) is the longest helper phase, two value waves instead share their SIMDs with the two
// T_ba waves (hardware waves 4, 5 take role indices 2, 3) and the four staging waves pair up
// on the other two SIMDs (hardware waves 2, 3, 6, 7): measured 13 % faster there, and slower
// for the other variants, whose T_ba products then compete with the value waves.
template <int NVW, bool CHAN>
__device__ __forceinline__ int role_wave(int tid) {
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  return (NVW == 2 && CHAN) ? ((w & 1) | ((w & 2) << 1) | ((w & 4) >> 1)) : w;
}

// The helper waves' loop, instantiated per role: STG (helpers 2 and up) stage the inputs,
// the others (helpers 0, 1) form T's off-diagonal blocks.  Each instantiation holds only its
// own role's state across iterations, and both run the kernel's barrier sequence.
template <int BV, bool CHAN, bool DECAY, int WK, bool RES, bool STG, bool TP, bool KD, bool SEG>
__device__ __forceinline__ void helper_loop(Smem<BV, CHAN, WK> &sm, const ChunkArgs a) {
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
  constexpr bool kPv = NVW == 2 && !KD;
  constexpr bool kRq = kPv && (CHAN || WK != kWkSame);   // P's R operands read separately

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a provably wave-uniform (scalar) value: role dispatch below is then a
  // scalar branch, and each role's loop (with its barriers) runs only in its own waves
  const int wave = role_wave<NVW, CHAN>(tid);
  const int l16 = lane & 15, l4 = lane >> 4;
  const bool vwave = wave < NVW;
  const int hw = wave - NVW;               // helper wave index
  const int ht = (wave - NVW) * 64 + lane;   // helper thread index
  const short4v I16 = ident4(lane);

  // XCD-aware tile order: the value tiles of one head land on one XCD (shared L2)
  // (the host bounds the grid to 2^22 workgroups, so these fit in 32 bits)
  // With the sequence split the grid holds three groups of the batch's value tiles, in this
  // order (so the first two are resident first): role 0 the first segment, role 1 the second
  // from a zero state, role 2 the second's transition (V' = 0 from the identity)
  // (SEG, a compile-time choice, so the unsplit kernel keeps its constant chunk range)
  const int per = SEG ? static_cast<int>(gridDim.x) / 3 : static_cast<int>(gridDim.x);
  const int role = SEG ? static_cast<int>(blockIdx.x) / per : 0;
  const int local = SEG ? static_cast<int>(blockIdx.x) % per : static_cast<int>(blockIdx.x);
  const int logical = (per % 8 == 0) ? (local % 8) * (per / 8) + local / 8 : local;
  const int bh = logical / NVT, vt = logical % NVT, v0 = vt * BV;
  const int H = a.H, T = a.T;
  const int b = bh / H, h = bh % H;
  const long long tokstride = static_cast<long long>(H) * kD;
  const long long head0 = (static_cast<long long>(b) * T * H + h) * kD;
  const long long gate0 = static_cast<long long>(b) * T * H + h;
  const int nchunks = (T + kC - 1) / kC;
  const int cbeg = (SEG && role != 0) ? a.seg_split : 0;   // this workgroup's chunks
  const int cend = (SEG && role == 0) ? a.seg_split : nchunks;
  const int N = a.N;
  auto keep = [N](int i, int j) { return N < 0 || i - j <= N; };

  const uint16_t *gq = static_cast<const uint16_t *>(a.q);
  const uint16_t *gk = static_cast<const uint16_t *>(a.k);
  const uint16_t *gv = static_cast<const uint16_t *>(a.v);
  const uint16_t *gwk = static_cast<const uint16_t *>(a.write_key);
  const uint16_t *ger = static_cast<const uint16_t *>(a.erase);
  const uint16_t *gwr = static_cast<const uint16_t *>(a.write);
  uint16_t *gout = static_cast<uint16_t *>(a.out);

  // ============================== helper waves ==============================
  // One staging point per chunk: every item of chunk c + 1 is written to LDS from registers
  // loaded a full iteration earlier, then the loads of chunk c + 2 are issued.  Items are
  // 16-byte granules in blocks of 64 (one wave-wide load): 16 blocks each of q, k and an
  // explicit write key (64 x 128 bf16), then the blocks of the 64 x BV value tile.  The two
  // helpers that form T's off-diagonal blocks (hw 0, 1) stage nothing, so their block products
  // never wait behind staging writes (a wave's LDS operations complete in order); the loads'
  // issue (about 160 cycles per 1 KB load, measured) and the LDS writes bound the staging
  // waves' phase.  Block s * NSW + sw is slot s
  // of staging wave sw = hw - 2, so everything about a block (source, LDS destination, row /
  // column split) is wave-uniform.  Every slot loads and is staged
  // unconditionally -- a slot past the last block repeats it without storing -- so the
  // registers of a load are first read one iteration after it was issued and the loads of
  // a chunk issue back to back.  Rows past the end of the sequence are read clamped to the
  // last row and zeroed when staged.
  constexpr int NBP = (NQ + NK + NR) / 64;     // blocks of 64 x 128 arrays
  constexpr int NB = NBP + NVI / 64;
  constexpr int NSW = NHW - 2;                 // staging waves: helpers 2 .. NHW - 1
  constexpr int NSB = (NB + NSW - 1) / NSW;    // block slots per staging wave
  constexpr int VSH = BV == 32 ? 2 : 1;        // log2(items per value-tile row)
  uint4 pa[NSB], pb[NSB];
#pragma unroll
  for (int s = 0; s < NSB; ++s) pa[s] = pb[s] = make_uint4(0u, 0u, 0u, 0u);
  float gla = 0.f, gbeta = 0.f;                // gates of token `lane` of the staged chunk
  const bool gate_wave = wave == kNW - 1;
  const int tok32 = H * kD;                    // token stride; 64 * tok32 < 2^31 (H <= 65535)
  const int sw = hw - 2;
  auto slot_block = [&](int s) __attribute__((always_inline)) { return max(0, min(s * NSW + sw, NB - 1)); };
  // item u of block blk: row u >> sh, column col0 + (u & msk) * 8
  auto item_rc = [&](int blk, int &t, int &col) __attribute__((always_inline)) {
    const bool isv = blk >= NBP;
    const int u = (isv ? blk - NBP : blk & 15) * 64 + lane;
    t = isv ? u >> VSH : u >> 4;
    col = isv ? (u & (BV / 8 - 1)) * 8 : (u & 15) * 8;
  };

  // Per-slot addressing, fixed for the whole sequence: the slot's source array (a wave-uniform
  // choice: 0 q, 1 k, 2 explicit write key, 3 the value tile), this lane's byte offset from the
  // chunk's first row of the head in that array (32 bits: 64 rows of at most 65535 heads of 128
  // channels) and its LDS byte offset in buffer 0.  Per chunk that leaves one scalar base per
  // array, the loads and the stores; a slot's offset is clamped only on a partial last chunk.
  int sarr[NSB], srow[NSB], gofs[NSB], loff[NSB], lstr[NSB], eoff[NSB];
  char *const smb = reinterpret_cast<char *>(&sm);
  const int rowb = static_cast<int>(tokstride) * 2;   // bytes between two tokens' rows
#pragma unroll
  for (int s = 0; s < NSB; ++s) {
    const int blk = slot_block(s);
    const bool isv = blk >= NBP;
    const int arr = blk >> 4;
    int t, col;
    item_rc(blk, t, col);
    sarr[s] = isv ? 3 : arr;
    srow[s] = t;
    gofs[s] = t * rowb + ((isv ? v0 : 0) + col) * 2;
    uint16_t *d0 = isv ? &sm.vp[0][t][col] : (arr == 0 ? sm.q[0] : arr == 1 ? sm.k[0] : sm.r[0]) + sw128(t, col);
    loff[s] = static_cast<int>(reinterpret_cast<char *>(d0) - smb);
    lstr[s] = isv ? static_cast<int>(sizeof(sm.vp[0])) : kC * kD * 2;
    eoff[s] = static_cast<int>(reinterpret_cast<char *>(sm.e[0] + (CHAN ? sw128(t, col) : 0)) - smb);
  }

  auto load_items = [&](int c) __attribute__((always_inline)) {
    const int c0 = c * kC, nm1 = min(kC, T - c0) - 1;
    const long long cb = head0 + static_cast<long long>(c0) * tokstride;   // the chunk's first row
    const char *const bq = reinterpret_cast<const char *>(gq + cb), *const bk = reinterpret_cast<const char *>(gk + cb);
    const char *const bw = reinterpret_cast<const char *>(gwk + cb), *const bv = reinterpret_cast<const char *>(gv + cb);
    const char *const be = reinterpret_cast<const char *>(ger + cb), *const bwv = reinterpret_cast<const char *>(gwr + cb);
#pragma unroll
    for (int s = 0; s < NSB; ++s) {
      // rows past the end of the sequence read the last row (and are zeroed when staged)
      const uint32_t o = static_cast<uint32_t>(gofs[s] - max(0, srow[s] - nm1) * rowb);
      const char *const base = sarr[s] == 0 ? bq : sarr[s] == 1 ? bk : sarr[s] == 2 ? bw : bv;
      pa[s] = *reinterpret_cast<const uint4 *>(base + o);
      if (CHAN) pb[s] = *reinterpret_cast<const uint4 *>((sarr[s] == 3 ? bwv : be) + o);
    }
    const long long gi = gate0 + static_cast<long long>(c0) * H + min(lane, nm1) * H;
    if (DECAY) gla = a.log_alpha[gi];
    if (!CHAN) gbeta = a.beta[gi];
  };
  auto stage_items = [&](int c, int buf) __attribute__((always_inline)) {
    const int n = min(kC, T - c * kC);
#pragma unroll
    for (int s = 0; s < NSB; ++s) {
      const int blk = slot_block(s);
      const bool live = s * NSW + sw < NB;
      const bool isv = blk >= NBP, isk = !isv && (blk >> 4) == 1;
      uint4 x = pa[s];
      if (n < kC) {   // rows past the end of the sequence (read clamped) are zeroed
        const uint32_t m = srow[s] < n ? 0xffffffffu : 0u;
        x = make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
      }
      if (SEG && role == 2 && isv) x = make_uint4(0u, 0u, 0u, 0u);   // the transition: V' = 0
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
  // diagonal block p of A = -L (strictly lower, fp32) as acc(N) and acc(N^T): the two products
  // run on the same operands, and each entry is scaled by exactly the operations of a_tile, so
  // acc(N^T) is the transpose of acc(N) bit for bit
  auto a_diag = [&](int buf, int p, float4v &n, float4v &nt) __attribute__((always_inline)) {
    const uint16_t *E = CHAN ? sm.e[buf] : sm.k[buf];
    const uint16_t *R = (WK == kWkSame) ? sm.k[buf] : sm.r[buf];
    constexpr bool SYM = !CHAN && WK == kWkSame;   // E R^T = K K^T: each tile is its own transpose
    const int row = p * 16 + l16;
    float4v g = zero4(), gt = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const short8v e = opn128(E, row, 32 * s, l4);
      if constexpr (SYM) {
        g = mfma32(e, e, g);
      } else {
        const short8v r = opn128(R, row, 32 * s, l4);
        g = mfma32(e, r, g);
        gt = mfma32(r, e, gt);
      }
    }
    if constexpr (SYM) gt = g;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      {
        const int i = p * 16 + 4 * l4 + r, j = p * 16 + l16;
        float x = g[r];
        if (SCALED_E) x *= sm.beta[buf][i];
        if (DECAY) x *= decay2(sm.g2[buf][i] - sm.g2[buf][j]);
        n[r] = (j < i) ? -x : 0.f;
      }
      {
        const int i = p * 16 + l16, j = p * 16 + 4 * l4 + r;
        float x = gt[r];
        if (SCALED_E) x *= sm.beta[buf][i];
        if (DECAY) x *= decay2(sm.g2[buf][i] - sm.g2[buf][j]);
        nt[r] = (j < i) ? -x : 0.f;
      }
    }
  };
  // P tile job (blocks (ib, jb), jb <= ib, numbered row by row), computed transposed
  // (P^T = R Q^T) so each lane writes 4 columns of one row of P
  auto p_tile = [&](int buf, int job) __attribute__((always_inline)) {
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
  // write acc(X^T) of the 16 x 16 block (rb, cb) of T (buffer buf) as 8-byte rows (lane: row
  // rb*16 + l16, columns cb*16 + 4 l4 .. + 3), band-masked, as the pair (hi, lo): from fp32 values
  // (put_rows) or from the two parts already split (put_rows2; each part exactly bf16)
  auto put_rows2 = [&](int buf, int rb, int cb, float4v xh, float4v xl, bool lower_only) __attribute__((always_inline)) {
    const int i = rb * 16 + l16;
    float4v h, l;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = cb * 16 + 4 * l4 + r;
      const bool on = keep(i, j) && (!lower_only || j <= i);
      h[r] = on ? xh[r] : 0.f;
      l[r] = on ? xl[r] : 0.f;
    }
    *reinterpret_cast<short4v *>(&sm.t[buf][i][cb * 16 + 4 * l4]) = tobf4(h);
    *reinterpret_cast<short4v *>(&sm.tl[buf][i][cb * 16 + 4 * l4]) = tobf4(l);
  };
  auto put_rows = [&](int buf, int rb, int cb, float4v xt, bool lower_only) __attribute__((always_inline)) {
    const Pair x = split4(xt);
    put_rows2(buf, rb, cb, unbf4(x.h), unbf4(x.l), lower_only);
  };
  // acc(X^T) of a pair given in acc(X) (B operand) layout: each part transposed exactly by an
  // identity product
  auto tr2 = [&](const Pair &x, float4v &th, float4v &tl) __attribute__((always_inline)) {
    th = mfma16(x.h, I16, zero4());
    tl = mfma16(x.l, I16, zero4());
  };

  // preconditioner accumulator: the first four staging waves (helpers 2..5); their thread
  // pt = ht - 128 owns channels 2 p, 2 p + 1 (p = pt / 4) and tokens 16 s .. 16 s + 15
  // (s = pt % 4) of a chunk; the four segments of a channel pair are the four lanes of a quad.
  // The accumulator entering the chunk is kept in all four.
  const int pt = ht - 128;
  const bool pc_thread = STG && pt >= 0 && pt < 256;
  const int pc_p = pt >> 2, pc_seg = pt & 3;
  float hc0 = 0.f, hc1 = 0.f;
  if (WK == kWkPrecond && pc_thread) {
    hc0 = a.pc_h_in != nullptr ? a.pc_h_in[static_cast<long long>(bh) * kD + 2 * pc_p] : a.h0;
    hc1 = a.pc_h_in != nullptr ? a.pc_h_in[static_cast<long long>(bh) * kD + 2 * pc_p + 1] : a.h0;
  }

  // (TP) T formed beforehand: the two T_ba waves copy chunk c + 1's pair from the buffer
  // (loaded in the update phase) into T's LDS buffers at the start of the next phase, where
  // they would finish T.  The buffer holds the ten blocks on and below the diagonal (the
  // others stay zero in LDS), block q = ib (ib + 1) / 2 + jb, each as hi then lo, each part
  // 16 rows of 16; item u = 128 m + thread of 16 bytes: block u / 64, part (u / 32) % 2, row
  // (u / 2) % 16, columns 8 (u % 2) .. + 7 of the block.
  // (KD) the per-channel decay's record adds P (items 640..959: block (u - 640) / 32, row
  // ((u - 640) / 2) % 16, columns 8 (u % 2) .., single bf16) and the chunk's per-channel state
  // decay (items 960..991, four fp32 channels each), copied the same way into P's buffer and
  // the per-channel decay buffer (which lives in the unused A_ba space)
  constexpr int kTItems = KD ? 992 : 640;
  constexpr int kTI = TP ? (kTItems + 127) / 128 : 1;
  uint4 tpv[kTI];
  auto tp_load = [&](int c) __attribute__((always_inline)) {
    const uint16_t *src = a.tpre + (static_cast<long long>(bh) * nchunks + c) * (kTItems * 8);
#pragma unroll
    for (int m = 0; m < kTI; ++m)
      if (128 * m + 127 < kTItems || 128 * m + ht < kTItems)
        tpv[m] = *reinterpret_cast<const uint4 *>(src + 8 * (128 * m + ht));
  };
  auto tp_stage = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < kTI; ++m) {
      const int u = 128 * m + ht;
      if (u < 640) {
        const int q = u >> 6;
        const int ib = q < 1 ? 0 : q < 3 ? 1 : q < 6 ? 2 : 3, jb = q - ib * (ib + 1) / 2;
        const int row = 16 * ib + ((u >> 1) & 15), col = 16 * jb + 8 * (u & 1);
        uint16_t *dst = ((u >> 5) & 1) ? &sm.tl[buf][row][col] : &sm.t[buf][row][col];   // 8-byte aligned rows
        *reinterpret_cast<uint2 *>(dst) = make_uint2(tpv[m].x, tpv[m].y);
        *reinterpret_cast<uint2 *>(dst + 4) = make_uint2(tpv[m].z, tpv[m].w);
      } else if (KD && u < 960) {
        const int v = u - 640, q = v >> 5;
        const int ib = q < 1 ? 0 : q < 3 ? 1 : q < 6 ? 2 : 3, jb = q - ib * (ib + 1) / 2;
        uint16_t *dst = &sm.p[16 * ib + ((v >> 1) & 15)][16 * jb + 8 * (v & 1)];
        *reinterpret_cast<uint2 *>(dst) = make_uint2(tpv[m].x, tpv[m].y);
        *reinterpret_cast<uint2 *>(dst + 4) = make_uint2(tpv[m].z, tpv[m].w);
      } else if (KD && u < kTItems) {
        *reinterpret_cast<uint4 *>(&gcv_of(sm, buf)[4 * (u - 960)]) = tpv[m];
      }
    }
  };
  if (STG && cbeg < cend) load_items(cbeg);
  for (int c = cbeg - 1; c < cend; ++c) {
    const int cur = c & 1, nxt = (c + 1) & 1;
    const bool have_next = c + 1 < cend;

    __syncthreads();   // (1)
    // The two T_ba waves read every operand of their block products (T blocks and A blocks of
    // chunk c, formed before the barrier) ahead of their staging writes: LDS operations of a
    // wave complete in order, so reads issued after the writes would wait for them to drain,
    // while issued first they let the writes drain under the products.
    const int qb = hw;   // column block of the lower-left quadrant formed by this wave
    // A layout of block (rb, kb) of T; B layout of block (kb, cb) by a transposing read; every
    // operand as its bf16 pair
    auto arow = [&](int rb, int kb) __attribute__((always_inline)) {
      const int o = (rb * 16 + l16) * kLdc + kb * 16 + 4 * l4;
      return Pair{ld4(&sm.t[cur][0][0] + o), ld4(&sm.tl[cur][0][0] + o)};
    };
    auto bcol = [&](int kb, int cb) __attribute__((always_inline)) {
      const int o = (kb * 16 + 4 * l4 + (l16 >> 2)) * kLdc + cb * 16 + 4 * (l16 & 3);
      return Pair{ldtr(&sm.t[cur][0][0] + o), ldtr(&sm.tl[cur][0][0] + o)};
    };
    auto lrow = [&](int s2, int u) __attribute__((always_inline)) {
      return Pair{ld4(&sm.lba[s2 * 16 + l16][u * 16 + 4 * l4]), ld4(&sm.lbal[s2 * 16 + l16][u * 16 + 4 * l4])};
    };
    auto aodp = [&](int j) __attribute__((always_inline)) { return Pair{ld4(&sm.aod[j][l16][4 * l4]), ld4(&sm.aodl[j][l16][4 * l4])}; };
    Pair o_a33, o_b22, o_a22, o_a32, o_a10, o_d, o_a11, o_l00, o_l01, o_l10, o_l11;
    auto load_ops = [&](auto part) __attribute__((always_inline)) {
      constexpr bool LO = decltype(part)::value;
      auto get = [&](Pair &x, const Pair &v) __attribute__((always_inline)) { (LO ? x.l : x.h) = LO ? v.l : v.h; };
      get(o_a33, arow(3, 3));
      get(o_b22, bcol(2, 2));
      get(o_a22, arow(2, 2));
      get(o_a32, aodp(1));
      get(o_l01, lrow(0, 1));
      get(o_l11, lrow(1, 1));
      if (qb == 0) {
        get(o_a10, aodp(0));
        get(o_d, bcol(0, 0));
        get(o_a11, arow(1, 1));
        get(o_l00, lrow(0, 0));
        get(o_l10, lrow(1, 0));
      } else {
        get(o_d, bcol(1, 1));
      }
    };
    if constexpr (TP) {
      if (!STG && c >= cbeg) tp_stage(cur);
    } else if (!STG && c >= cbeg) {
      load_ops(std::false_type{});
      load_ops(std::true_type{});
    }
    if (STG && have_next) {
      stage_items(c + 1, nxt);
      if (c + 2 < cend) load_items(c + 2);
    }
    if (c >= cbeg) {
      if constexpr (!STG && !TP) {
        // remaining blocks of T(c): T_10 = D_1 A_10 D_0, T_32 = D_3 A_32 D_2 and column block
        // qb = hw of the lower-left quadrant T_ba = T_b A_ba T_a, every product on bf16 pairs
        const Pair t32 = split4(mm2(o_a33, split4(mm2(o_a32, o_b22))));
        float4v t32h, t32l;
        tr2(t32, t32h, t32l);
        const Pair t32a{tobf4(t32h), tobf4(t32l)};   // A layout of T_32
        float4v z0, z1;                              // Z = A_ba T_a[:, qb]
        if (qb == 0) {
          const Pair t10 = split4(mm2(o_a11, split4(mm2(o_a10, o_d))));
          z0 = mm2(o_l01, t10, mm2(o_l00, o_d));
          z1 = mm2(o_l11, t10, mm2(o_l10, o_d));
          float4v th, tl;
          tr2(t10, th, tl);
          put_rows2(cur, 1, 0, th, tl, false);
        } else {
          z0 = mm2(o_l01, o_d);
          z1 = mm2(o_l11, o_d);
          put_rows2(cur, 3, 2, t32h, t32l, false);
        }
        const Pair z0p = split4(z0), z1p = split4(z1);
        const Pair tb2 = split4(mm2(o_a22, z0p));
        const Pair tb3 = split4(mm2(o_a33, z1p, mm2(t32a, z0p)));
        float4v th, tl;
        tr2(tb2, th, tl);
        put_rows2(cur, 2, qb, th, tl, false);
        tr2(tb3, th, tl);
        put_rows2(cur, 3, qb, th, tl, false);
      }
      // P tiles (10 lower blocks) unless the value waves form them (or, KD, the record holds
      // them): jobs 8, 9 on the two T_ba waves, 0..7 on the others
      if constexpr (!kPv && !KD) {
        if constexpr (!STG) {
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

    if constexpr (RES) {
      // Parallel residual correction of the band-limited start T0 = T(c) (MatMul-only
      // inversion summary, Metodologia 3): E = I - (I - A) T0, Z = sum_{s <= S} E^s formed as
      // Z <- I + E Z from Z = I + E, and T = T0 Z.  All are lower triangular, and column block jb
      // of the new Z reads only column block jb of the old one, so a wave keeps one column block
      // of Z in its accumulators through every step with no exchange: helpers 0 and 1 take
      // column blocks 0 and 1, helper 2 blocks 2 and 3.  The tiles of E are shared: published
      // once, as bf16 pairs in A-operand layout, in the Q buffer of chunk c (its last reads were
      // before barrier (2)).  Three barriers: E published (R1), T0 read (R2), T written (R3).
      // (Spreading E's tiles over all six helpers measured slower: the staging helpers, which
      // hold the next chunk's prefetched items, then spill registers.)
      uint16_t *const ebuf = sm.q[cur];
      auto etile = [&](int ib, int kb) __attribute__((always_inline)) {   // 16 x 20 hi, then lo
        return ebuf + (ib * (ib + 1) / 2 + kb) * 640 + l16 * 20 + 4 * l4;
      };
      // the A-operand pair of block (ib, kb) of A (kb <= ib): the diagonal blocks formed again
      // from the chunk's keys, the others as the A jobs left them
      auto aop = [&](int ib, int kb) __attribute__((always_inline)) {
        if (ib == kb) {
          float4v n, nt;
          a_diag(cur, ib, n, nt);
          return split4(nt);
        }
        if (ib == 1) return aodp(0);
        if (ib == 3 && kb == 2) return aodp(1);
        return lrow(ib - 2, kb);
      };
      auto identity = [&]() __attribute__((always_inline)) {
        float4v r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = (4 * l4 + i == l16) ? 1.f : 0.f;
        return r;
      };
      // R1 / R2 / write for the compile-time column blocks J0, J1 (-1: none) of this wave
      auto res_run = [&](auto j0c, auto j1c) __attribute__((always_inline)) {
        constexpr int J0 = decltype(j0c)::value, J1 = decltype(j1c)::value;
        float4v ez[2][4], tz[2][4];
        // R1: the tiles of E in column block JB, E_ij = [i == j] - T0_ij + (A T0)_ij
        auto e_col = [&](auto jbc, float4v(&e_out)[4]) __attribute__((always_inline)) {
          constexpr int JB = decltype(jbc)::value;
#pragma unroll
          for (int ib = JB; ib < 4; ++ib) {
            const Pair t0 = bcol(ib, JB);
            float4v e = -(unbf4(t0.h) + unbf4(t0.l));
            if (ib == JB) e += identity();
#pragma unroll
            for (int kb = JB; kb <= ib; ++kb) e = mm2(aop(ib, kb), bcol(kb, JB), e);
            e_out[ib] = e;
            const Pair ep = split4(e);
            float4v th, tl;
            tr2(ep, th, tl);
            uint16_t *d = etile(ib, JB);
            *reinterpret_cast<short4v *>(d) = tobf4(th);
            *reinterpret_cast<short4v *>(d + 320) = tobf4(tl);
          }
        };
        // R2: Z = I + E, S - 1 steps Z <- I + E Z, then T = T0 Z, on column block JB
        auto z_col = [&](auto jbc, const float4v(&e_in)[4], float4v(&t_out)[4]) __attribute__((always_inline)) {
          constexpr int JB = decltype(jbc)::value;
          Pair ep[4][4];
#pragma unroll
          for (int ib = JB; ib < 4; ++ib)
#pragma unroll
            for (int kb = JB; kb <= ib; ++kb) {
              const uint16_t *t = etile(ib, kb);
              ep[ib][kb] = Pair{ld4(t), ld4(t + 320)};
            }
          float4v z[4];
#pragma unroll
          for (int ib = JB; ib < 4; ++ib) z[ib] = ib == JB ? e_in[ib] + identity() : e_in[ib];
          // the steps take Z rounded to bf16 (E as its pair: E_hi Z + E_lo Z in one 32-deep
          // product): the series' later terms are corrections, and a CPU emulation of this
          // rounding puts T within 1.2e-4 of the fp64 residual-corrected T (3.6e-5 at N = 3,
          // S = 8) against 1e-6 with Z as a pair too, for half the products on the critical
          // wave; T = T0 Z below takes Z as a pair
          for (int st = 1; st < a.S; ++st) {
            short4v zh[4];
#pragma unroll
            for (int kb = JB; kb < 4; ++kb) zh[kb] = tobf4(z[kb]);
#pragma unroll
            for (int ib = JB; ib < 4; ++ib) {
              float4v acc = ib == JB ? identity() : zero4();
#pragma unroll
              for (int kb = JB; kb <= ib; ++kb)
                acc = mfma32(cat(ep[ib][kb].h, ep[ib][kb].l), cat(zh[kb], zh[kb]), acc);
              z[ib] = acc;
            }
          }
          Pair zp[4];
#pragma unroll
          for (int kb = JB; kb < 4; ++kb) zp[kb] = split4(z[kb]);
#pragma unroll
          for (int ib = JB; ib < 4; ++ib) {
            float4v acc = zero4();
#pragma unroll
            for (int kb = JB; kb <= ib; ++kb) acc = mm2(arow(ib, kb), zp[kb], acc);
            t_out[ib] = acc;
          }
        };
        // write: T's column block JB (all ten blocks of T are written; no band mask)
        auto t_put = [&](auto jbc, const float4v(&t_in)[4]) __attribute__((always_inline)) {
          constexpr int JB = decltype(jbc)::value;
#pragma unroll
          for (int ib = JB; ib < 4; ++ib) {
            const Pair tp = split4(t_in[ib]);
            float4v th, tl;
            tr2(tp, th, tl);
            const int i = ib * 16 + l16;
            *reinterpret_cast<short4v *>(&sm.t[cur][i][JB * 16 + 4 * l4]) = tobf4(th);
            *reinterpret_cast<short4v *>(&sm.tl[cur][i][JB * 16 + 4 * l4]) = tobf4(tl);
          }
        };
        if (c >= cbeg) {
          if constexpr (J0 >= 0) e_col(j0c, ez[0]);
          if constexpr (J1 >= 0) e_col(j1c, ez[1]);
        }
        __syncthreads();   // (R1) E published
        if (c >= cbeg) {
          if constexpr (J0 >= 0) z_col(j0c, ez[0], tz[0]);
          if constexpr (J1 >= 0) z_col(j1c, ez[1], tz[1]);
        }
        __syncthreads();   // (R2) every read of T0 done
        if (c >= cbeg) {
          if constexpr (J0 >= 0) t_put(j0c, tz[0]);
          if constexpr (J1 >= 0) t_put(j1c, tz[1]);
        }
        __syncthreads();   // (R3) T(c) complete
      };
      using std::integral_constant;
      if constexpr (!STG) {
        if (hw == 0)
          res_run(integral_constant<int, 0>{}, integral_constant<int, -1>{});
        else
          res_run(integral_constant<int, 1>{}, integral_constant<int, -1>{});
      } else {
        if (hw == 2)
          res_run(integral_constant<int, 2>{}, integral_constant<int, 3>{});
        else
          res_run(integral_constant<int, -1>{}, integral_constant<int, -1>{});
      }
    }

    if (have_next) {
      const int nb = nxt;
      // off-diagonal blocks of A: A_10, A_32 (for T_10, T_32) and the four blocks of A_ba (jobs
      // 0..5); a wave forms its share together (operands first, then the product chains).  Job
      // q of a batch is job0 + q * jstep; jobs past the last repeat it without storing.
      auto a_jobs = [&](auto njc, int job0, int jstep) __attribute__((always_inline)) {
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
            const Pair xp = split4(x);
            uint16_t *dst = job < 2 ? &sm.aod[job][l16][4 * l4] : &sm.lba[(ib[q] - 2) * 16 + l16][jb[q] * 16 + 4 * l4];
            uint16_t *dstl = job < 2 ? &sm.aodl[job][l16][4 * l4] : &sm.lbal[(ib[q] - 2) * 16 + l16][jb[q] * 16 + 4 * l4];
            *reinterpret_cast<short4v *>(dst) = xp.h;
            *reinterpret_cast<short4v *>(dstl) = xp.l;
          }
        }
      };
      // The four diagonal inverses (dependent chains of matrix-core products) run on helpers
      // 2..5, one per SIMD (wave w runs on the SIMD of wave w + 4), the A blocks on the others
      constexpr int NAW = NHW - 4;               // waves on the A blocks
      if constexpr (TP) {
        // (TP) nothing of T to form: the T_ba waves load chunk c + 1's T
        if (!STG) tp_load(c + 1);
      } else if (hw >= 2 && hw < 6) {
        if constexpr (STG) {
          // diagonal block hw - 2 of T: D = (I - A_pp)^-1.  Its chain of dependent products
          // is the longest work of this phase; two of these waves share their SIMDs with the
          // value waves' update, so they take issue priority for it (2-3 % on gdn and pdn;
          // with channel gains the waves sit elsewhere and it makes no difference)
          if (!CHAN) __builtin_amdgcn_s_setprio(3);
          float4v n, nt;
          a_diag(nb, hw - 2, n, nt);
          put_rows(nb, hw - 2, hw - 2, diag_inverse_t(n, nt, lane), true);
          if (!CHAN) __builtin_amdgcn_s_setprio(0);
        }
      } else {
        a_jobs(std::integral_constant<int, (6 + NAW - 1) / NAW>{}, hw < 2 ? hw : hw - 4, NAW);
      }
    }
  }
  if (WK == kWkPrecond && a.pc_h_out != nullptr && vt == 0 && pc_thread && pc_seg == 0)
  {
    a.pc_h_out[static_cast<long long>(bh) * kD + 2 * pc_p] = hc0;
    a.pc_h_out[static_cast<long long>(bh) * kD + 2 * pc_p + 1] = hc1;
  }
}

template <int BV, bool CHAN, bool DECAY, int WK, bool RES, bool TP, bool KD = false, bool SEG = false>
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
  constexpr bool kPv = NVW == 2 && !KD;
  constexpr bool kRq = kPv && (CHAN || WK != kWkSame);   // P's R operands read separately
  __shared__ Smem<BV, CHAN, WK> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a provably wave-uniform (scalar) value: role dispatch below is then a
  // scalar branch, and each role's loop (with its barriers) runs only in its own waves
  const int wave = role_wave<NVW, CHAN>(tid);
  const int l16 = lane & 15, l4 = lane >> 4;
  const bool vwave = wave < NVW;
  const int hw = wave - NVW;               // helper wave index
  const int ht = (wave - NVW) * 64 + lane;   // helper thread index
  const short4v I16 = ident4(lane);

  // XCD-aware tile order: the value tiles of one head land on one XCD (shared L2)
  // (the host bounds the grid to 2^22 workgroups, so these fit in 32 bits)
  // With the sequence split the grid holds three groups of the batch's value tiles, in this
  // order (so the first two are resident first): role 0 the first segment, role 1 the second
  // from a zero state, role 2 the second's transition (V' = 0 from the identity)
  // (SEG, a compile-time choice, so the unsplit kernel keeps its constant chunk range)
  const int per = SEG ? static_cast<int>(gridDim.x) / 3 : static_cast<int>(gridDim.x);
  const int role = SEG ? static_cast<int>(blockIdx.x) / per : 0;
  const int local = SEG ? static_cast<int>(blockIdx.x) % per : static_cast<int>(blockIdx.x);
  const int logical = (per % 8 == 0) ? (local % 8) * (per / 8) + local / 8 : local;
  const int bh = logical / NVT, vt = logical % NVT, v0 = vt * BV;
  const int H = a.H, T = a.T;
  const int b = bh / H, h = bh % H;
  const long long tokstride = static_cast<long long>(H) * kD;
  const long long head0 = (static_cast<long long>(b) * T * H + h) * kD;
  const long long gate0 = static_cast<long long>(b) * T * H + h;
  const int nchunks = (T + kC - 1) / kC;
  const int cbeg = (SEG && role != 0) ? a.seg_split : 0;   // this workgroup's chunks
  const int cend = (SEG && role == 0) ? a.seg_split : nchunks;
  const int N = a.N;
  auto keep = [N](int i, int j) { return N < 0 || i - j <= N; };

  const uint16_t *gq = static_cast<const uint16_t *>(a.q);
  const uint16_t *gk = static_cast<const uint16_t *>(a.k);
  const uint16_t *gv = static_cast<const uint16_t *>(a.v);
  const uint16_t *gwk = static_cast<const uint16_t *>(a.write_key);
  const uint16_t *ger = static_cast<const uint16_t *>(a.erase);
  const uint16_t *gwr = static_cast<const uint16_t *>(a.write);
  uint16_t *gout = (SEG && role == 2) ? a.seg_qt : static_cast<uint16_t *>(a.out);
  // final state: with the sequence split each role's goes to its slot of seg_state
  float *const sout = SEG ? a.seg_state + static_cast<long long>(role) * a.B * a.H * kD * kD : a.state_out;

  // ---------------- one-time init: zero T (upper blocks stay zero) and P ----------------
  for (int i = tid; i < 2 * kC * kLdc; i += kNT) (&sm.t[0][0][0])[i] = (&sm.tl[0][0][0])[i] = 0;
  for (int i = tid; i < kC * kLdc; i += kNT) (&sm.p[0][0])[i] = 0;

  // Each role runs its own loop with the same barrier sequence, so the compiler allocates
  // registers for one role's loop-carried state at a time.
  if (vwave) {
    // the wave index is a template constant inside the value-wave loop, so every wave-dependent
    // choice below (state rows, the P blocks a wave forms) is static
    auto value_loop = [&](auto wc) __attribute__((always_inline)) {
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
      auto chan0 = [&](int cb) __attribute__((always_inline)) { return 32 * (cb >> 1) + 8 * l4 + 4 * (cb & 1); };
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        st[cb] = zero4();
        if (SEG && role == 2) {   // the transition starts from the identity (its rows are unit rows)
#pragma unroll
          for (int r = 0; r < 4; ++r) st[cb][r] = chan0(cb) + r == vrow ? 1.f : 0.f;
        } else if ((!SEG || role == 0) && a.state_in != nullptr) {
          const float4 sv = ld4f(a.state_in + (static_cast<long long>(bh) * kD + vrow) * kD + chan0(cb));
          st[cb] = float4v{sv.x, sv.y, sv.z, sv.w};
        }
      }
      for (int c = cbeg - 1; c < cend; ++c) {
        const int cur = c & 1;
        const int c0 = c * kC;
        const int n = min(kC, T - c0);
        short4v x4[4];
        float4v O1[4];
        __syncthreads();   // (1) chunk c staged, T(c) diagonal part ready
        if (c >= cbeg) {
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
          auto load_e = [&](int tb) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < 4; ++j) ev[tb][j] = opn128(E, tb * 16 + l16, 32 * j, l4);
          };
          auto load_ops = [&](int tb, int slot) __attribute__((always_inline)) {
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
        if constexpr (RES) {   // the residual correction of T(c) on the helpers (see there)
          if (WK == kWkPrecond) __syncthreads();   // (3)
          __syncthreads();   // (R1)
          __syncthreads();   // (R2)
          __syncthreads();   // (R3)
        }
        if (c >= cbeg) {
          // every LDS operand of this phase is read up front: T and P blocks, R^T for the update.
          // T is held as a bf16 pair (hi + lo): the diagonal blocks pack hi and lo into one K = 32
          // operand (the other K half of a diagonal block is zero), the others take one operand
          // per part.  (T and P are lower triangular; their blocks above the diagonal stay zero.)
          const uint16_t *Tm = &sm.t[cur][0][0], *Tl = &sm.tl[cur][0][0], *Pm = &sm.p[0][0];
          const uint16_t *Rk = (WK == kWkSame) ? sm.k[cur] : sm.r[cur];
          auto blk = [&](const uint16_t *M, int rb, int kb) __attribute__((always_inline)) { return ld4(M + (rb * 16 + l16) * kLdc + kb * 16 + 4 * l4); };
          const short8v t00 = cat(blk(Tm, 0, 0), blk(Tl, 0, 0));
          const short8v t10 = cat(blk(Tm, 1, 0), blk(Tm, 1, 1)), t10l = cat(blk(Tl, 1, 0), blk(Tl, 1, 1));
          const short8v t20 = cat(blk(Tm, 2, 0), blk(Tm, 2, 1)), t20l = cat(blk(Tl, 2, 0), blk(Tl, 2, 1));
          const short8v t22 = cat(blk(Tm, 2, 2), blk(Tl, 2, 2));
          const short8v t30 = cat(blk(Tm, 3, 0), blk(Tm, 3, 1)), t30l = cat(blk(Tl, 3, 0), blk(Tl, 3, 1));
          const short8v t32 = cat(blk(Tm, 3, 2), blk(Tm, 3, 3)), t32l = cat(blk(Tl, 3, 2), blk(Tl, 3, 3));
          const short4v q00 = blk(Pm, 0, 0), q22 = blk(Pm, 2, 2);
          const short8v p10 = opsp(Pm, kLdc, 16 + l16, 0, l4);
          const short8v p20 = opsp(Pm, kLdc, 32 + l16, 0, l4);
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
          float4 gcc[KD ? 8 : 1];   // (KD) the state decay of this lane's channels of each tile
          if constexpr (KD) {
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) gcc[cb] = ld4f(&gcv_of(sm, cur)[chan0(cb)]);
          }

          // D = T X  (T_hi X + T_lo X)
          const short8v x01 = cat(x4[0], x4[1]), x23 = cat(x4[2], x4[3]);
          float4v D[4];
          D[0] = mfma32(t00, cat(x4[0], x4[0]), zero4());
          D[1] = mfma32(t10l, x01, mfma32(t10, x01, zero4()));
          D[2] = mfma32(t22, cat(x4[2], x4[2]), mfma32(t20l, x01, mfma32(t20, x01, zero4())));
          D[3] = mfma32(t32l, x23, mfma32(t32, x23, mfma32(t30l, x01, mfma32(t30, x01, zero4()))));
          // state update S^T <- e^{g_C} S^T + R^T (wd (.) D), interleaved with O2 = P D
          short4v w4[4], d4[4], dl4[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            w4[j] = tobf4(float4v{wdv[j].x * D[j][0], wdv[j].y * D[j][1], wdv[j].z * D[j][2], wdv[j].w * D[j][3]});
            const Pair dp = split4(D[j]);
            d4[j] = dp.h;
            dl4[j] = dp.l;
          }
          const short8v w01 = cat(w4[0], w4[1]), w23 = cat(w4[2], w4[3]);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            float4v acc = st[cb];
            if (DECAY) acc *= gC;
            if constexpr (KD) acc = float4v{acc[0] * gcc[cb].x, acc[1] * gcc[cb].y, acc[2] * gcc[cb].z, acc[3] * gcc[cb].w};
            st[cb] = mfma32(rb[cb], w23, mfma32(ra[cb], w01, acc));
            ra[cb] = optr_state(Rk, cb + 4, 0, lane);   // second half, read behind the first
            rb[cb] = optr_state(Rk, cb + 4, 32, lane);
          }
#pragma unroll
          for (int cb = 4; cb < 8; ++cb) {
            float4v acc = st[cb];
            if (DECAY) acc *= gC;
            if constexpr (KD) acc = float4v{acc[0] * gcc[cb].x, acc[1] * gcc[cb].y, acc[2] * gcc[cb].z, acc[3] * gcc[cb].w};
            st[cb] = mfma32(rb[cb - 4], w23, mfma32(ra[cb - 4], w01, acc));
          }
          // O = scale (O1 + P D), D as a bf16 pair (P_00 and P_22 are packed twice against
          // [D_hi; D_lo]); O1 seeds the accumulator
          const short8v d01 = cat(d4[0], d4[1]), d23 = cat(d4[2], d4[3]);
          const short8v dl01 = cat(dl4[0], dl4[1]), dl23 = cat(dl4[2], dl4[3]);
          float4v O2[4];
          O2[0] = mfma32(cat(q00, q00), cat(d4[0], dl4[0]), O1[0]);
          O2[1] = mfma32(p10, dl01, mfma32(p10, d01, O1[1]));
          O2[2] = mfma32(cat(q22, q22), cat(d4[2], dl4[2]), mfma32(p20, dl01, mfma32(p20, d01, O1[2])));
          O2[3] = mfma32(p32, dl23, mfma32(p32, d23, mfma32(p30, dl01, mfma32(p30, d01, O1[3]))));
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
        if (!RES && WK == kWkPrecond) __syncthreads();   // (3) write keys of chunk c + 1 formed
      }
      if (sout != nullptr) {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
          *reinterpret_cast<float4 *>(sout + (static_cast<long long>(bh) * kD + vrow) * kD + chan0(cb)) =
              make_float4(st[cb][0], st[cb][1], st[cb][2], st[cb][3]);
      }
    };
    if constexpr (NVW == 1) value_loop(std::integral_constant<int, 0>{});
    else if (wave == 0) value_loop(std::integral_constant<int, 0>{});
    else value_loop(std::integral_constant<int, 1>{});
    return;
  }

  if (hw >= 2) helper_loop<BV, CHAN, DECAY, WK, RES, true, TP, KD, SEG>(sm, a);
  else helper_loop<BV, CHAN, DECAY, WK, RES, false, TP, KD, SEG>(sm, a);
}

// ---------------------------------------------------------------------------------------
// T = (I - A)^-1 of every chunk at once, for the variants with write key k and the exact
// inverse (gdr_chunk_fwd_ws): one workgroup of four waves per (batch, head, chunk),
// independent of every other chunk, so the whole grid runs in parallel and the sequential
// kernel above only copies T.  The diagonal 16 x 16 blocks by the fused kernel's blocked
// substitution (diag_inverse_t), one per wave; then block forward substitution
// T_ij = D_i sum_{k = j..i-1} A_ik T_kj (MatMul-only inversion summary, "Declaracao do
// Problema": T solves (I - A) T = I) by levels of the block distance i - j (three, two, then
// one block on their own waves), every product on bf16 pairs; the waves exchange blocks through
// LDS in their operand layouts.  Output: the ten blocks on and below the diagonal of T, block
// q = ib (ib + 1) / 2 + jb, each as its hi then lo part of 16 x 16 bf16 row-major:
// [B, H, chunks][10][2][16][16].
// ---------------------------------------------------------------------------------------
constexpr int kTW = 4;   // waves per workgroup of the T kernel

template <bool CHAN, bool DECAY>
__global__ __launch_bounds__(64 * kTW) void chunk_t_kernel(ChunkArgs a, uint16_t *tw) {
  // keys (the write keys), swizzled, then (CHAN) the erase keys b (.) k
  __shared__ __align__(16) uint16_t kbuf[(CHAN ? 2 : 1) * kC * kD];
  __shared__ float g2[kC], bet[kC];
  uint16_t *const ks = kbuf, *const es = kbuf + (CHAN ? kC * kD : 0);
  // Once every product of keys has been formed, the keys' space holds the exchanged 16 x 16
  // blocks, as bf16 pairs in a lane's operand layout (16 bytes per lane): 0..3 acc(D_p^T)
  // (A operands of D_p), 4..7 acc(D_p) (B operands), 8..13 acc(A_ik^T) for (i, k) = (1,0)
  // (2,0) (2,1) (3,0) (3,1) (3,2), 14, 15 acc(T_10), acc(T_21).  (LDS of 16.5 KB per
  // workgroup without channel gains: nine workgroups per CU.)
  static_assert(16 * 64 * sizeof(uint4) == kC * kD * sizeof(uint16_t), "exchange space");
  uint4 (*const xb)[64] = reinterpret_cast<uint4 (*)[64]>(kbuf);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, l4 = lane >> 4;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int H = a.H, T = a.T;
  const int nchunks = (T + kC - 1) / kC;
  const int c0 = c * kC, n = min(kC, T - c0);
  const long long tokstride = static_cast<long long>(H) * kD;
  const long long cb = (static_cast<long long>(b) * T * H + h) * kD + static_cast<long long>(c0) * tokstride;
  const uint16_t *gk = static_cast<const uint16_t *>(a.k) + cb;
  const uint16_t *ger = static_cast<const uint16_t *>(a.erase) + (CHAN ? cb : 0);
  // 1024 items of 16 bytes (item u: row u / 16, columns 8 (u % 16) ..), rows past the end of
  // the sequence read clamped and zeroed
  constexpr int NI = 1024 / (64 * kTW);
  uint4 kv[NI], bv[CHAN ? NI : 1];
#pragma unroll
  for (int m = 0; m < NI; ++m) {
    const int u = 64 * kTW * m + tid, row = min(u >> 4, n - 1);
    kv[m] = *reinterpret_cast<const uint4 *>(gk + row * tokstride + 8 * (u & 15));
    if (CHAN) bv[m] = *reinterpret_cast<const uint4 *>(ger + row * tokstride + 8 * (u & 15));
  }
  if (wv == 0) {   // gates of the chunk's tokens (lane t), as the fused kernel's gate wave forms them
    const long long gi = static_cast<long long>(b) * T * H + h + static_cast<long long>(c0 + min(lane, n - 1)) * H;
    const bool ok = lane < n;
    const float la = DECAY ? a.log_alpha[gi] : 0.f;
    const float bt = CHAN ? 0.f : a.beta[gi];
    g2[lane] = wave_scan_add(ok ? la * kLog2e : 0.f);
    bet[lane] = ok ? bt : 0.f;
  }
#pragma unroll
  for (int m = 0; m < NI; ++m) {
    const int u = 64 * kTW * m + tid, row = u >> 4, col = 8 * (u & 15);
    uint4 x = kv[m];
    if (row >= n) x = make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4 *>(ks + sw128(row, col)) = x;
    if (CHAN) {
      const uint4 w = bv[m];
      *reinterpret_cast<uint4 *>(es + sw128(row, col)) =
          make_uint4(f32x2_to_bf16x2_bits(elem(w, 0) * elem(x, 0), elem(w, 1) * elem(x, 1)),
                     f32x2_to_bf16x2_bits(elem(w, 2) * elem(x, 2), elem(w, 3) * elem(x, 3)),
                     f32x2_to_bf16x2_bits(elem(w, 4) * elem(x, 4), elem(w, 5) * elem(x, 5)),
                     f32x2_to_bf16x2_bits(elem(w, 6) * elem(x, 6), elem(w, 7) * elem(x, 7)));
    }
  }
  __syncthreads();
  const uint16_t *E = CHAN ? es : ks;
  const uint16_t *R = ks;
  constexpr bool SCALED_E = !CHAN;   // E = beta k: beta applied after the product
  // the scaled entry of A = -L at (i, j), j < i, from the raw product x = (E R^T)_ij
  auto a_of = [&](float x, int i, int j) __attribute__((always_inline)) {
    if (SCALED_E) x *= bet[i];
    if (DECAY) x *= decay2(g2[i] - g2[j]);
    return -x;
  };
  const short4v I16 = ident4(lane);
  auto trp = [&](const Pair &x) __attribute__((always_inline)) {   // acc(X^T) of acc(X), exactly
    return Pair{tobf4(mfma16(x.h, I16, zero4())), tobf4(mfma16(x.l, I16, zero4()))};
  };
  auto put = [&](int slot, const Pair &x) __attribute__((always_inline)) {
    xb[slot][lane] = make_uint4(__builtin_bit_cast(uint32_t, short2{x.h[0], x.h[1]}),
                                __builtin_bit_cast(uint32_t, short2{x.h[2], x.h[3]}),
                                __builtin_bit_cast(uint32_t, short2{x.l[0], x.l[1]}),
                                __builtin_bit_cast(uint32_t, short2{x.l[2], x.l[3]}));
  };
  auto get = [&](int slot) __attribute__((always_inline)) {
    const uint4 v = xb[slot][lane];
    const short2 h0 = __builtin_bit_cast(short2, v.x), h1 = __builtin_bit_cast(short2, v.y);
    const short2 l0 = __builtin_bit_cast(short2, v.z), l1 = __builtin_bit_cast(short2, v.w);
    return Pair{short4v{h0.x, h0.y, h1.x, h1.y}, short4v{l0.x, l0.y, l1.x, l1.y}};
  };
  // block (i, j), j <= i: lane (row l16, columns 4 l4 .. + 3) of the pair x = acc(T_ij^T),
  // the 64 lanes' 8 bytes of a part contiguous
  uint16_t *dst = tw + (static_cast<long long>(b * H + h) * nchunks + c) * (10 * 2 * 256);
  auto out = [&](int i, int j, const Pair &x) __attribute__((always_inline)) {
    uint16_t *blk = dst + (i * (i + 1) / 2 + j) * 512 + l16 * 16 + 4 * l4;
    *reinterpret_cast<short4v *>(blk) = x.h;
    *reinterpret_cast<short4v *>(blk + 256) = x.l;
  };
  // A operand of the block (i, k) below the diagonal: acc(A_ik^T) = acc(R_k E_i^T), scaled
  auto aop = [&](int i, int k) __attribute__((always_inline)) {
    float4v x = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) x = mfma32(opn128(R, k * 16 + l16, 32 * s, l4), opn128(E, i * 16 + l16, 32 * s, l4), x);
    float4v y;
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = a_of(x[r], i * 16 + l16, k * 16 + 4 * l4 + r);
    return split4(y);
  };
  const short4v zs = {0, 0, 0, 0};
  {   // wave p: the diagonal block p and its share of the blocks of A below the diagonal
    const int p = wv;
    const int row = p * 16 + l16;
    float4v g = zero4(), gt = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const short8v e = opn128(E, row, 32 * s, l4);
      if constexpr (!CHAN) {
        g = mfma32(e, e, g);
      } else {
        const short8v r = opn128(R, row, 32 * s, l4);
        g = mfma32(e, r, g);
        gt = mfma32(r, e, gt);
      }
    }
    if constexpr (!CHAN) gt = g;
    // blocks of A: wave 0 (1,0) (2,0); wave 1 (2,1) (3,0); wave 2 (3,1); wave 3 (3,2)
    const int n_a = p < 2 ? 2 : 1;
    Pair ap[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int slot = p < 2 ? 2 * p + q : 2 + p;   // 0 1 | 2 3 | 4 | 5
      const int ai = slot < 1 ? 1 : slot < 3 ? 2 : 3;
      const int ak = slot - (ai * (ai - 1)) / 2;
      if (q < n_a) ap[q] = aop(ai, ak);
    }
    __syncthreads();   // every read of the keys done: the exchange space may be written
    float4v nn, nt;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i0 = p * 16 + 4 * l4 + r, j0 = p * 16 + l16;
      nn[r] = j0 < i0 ? a_of(g[r], i0, j0) : 0.f;
      const int i1 = p * 16 + l16, j1 = p * 16 + 4 * l4 + r;
      nt[r] = j1 < i1 ? a_of(gt[r], i1, j1) : 0.f;
    }
    Pair dt = split4(diag_inverse_t(nn, nt, lane));   // acc(D_p^T): rows of D_p
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * l4 + r > l16) dt.h[r] = dt.l[r] = 0;   // (lower triangle kept)
    put(p, dt);
    put(4 + p, trp(dt));
    out(p, p, dt);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      if (q < n_a) put(8 + (p < 2 ? 2 * p + q : 2 + p), ap[q]);
  }
  __syncthreads();
  // level 1: T_10, T_21, T_32 = D_i A_i,i-1 D_i-1 (waves 0, 1, 2)
  if (wv < 3) {
    const int i = wv + 1, j = wv;
    const int aslot = 8 + (i == 1 ? 0 : i == 2 ? 2 : 5);
    const Pair t = split4(mm2(get(i), split4(mm2(get(aslot), get(4 + j)))));
    if (i < 3) put(14 + wv, t);   // T_10, T_21 (T_32 is not read again)
    out(i, j, trp(t));
  }
  __syncthreads();
  // level 2: T_20 = D_2 (A_20 D_0 + A_21 T_10) (wave 0), T_31 = D_3 (A_31 D_1 + A_32 T_21) (wave 1)
  Pair t20{zs, zs};
  if (wv == 0) {
    t20 = split4(mm2(get(2), split4(mm2(get(9), get(4), mm2(get(10), get(14))))));
    out(2, 0, trp(t20));
  } else if (wv == 1) {
    const Pair t31 = split4(mm2(get(3), split4(mm2(get(12), get(5), mm2(get(13), get(15))))));
    out(3, 1, trp(t31));
  }
  // level 3: T_30 = D_3 (A_30 D_0 + A_31 T_10 + A_32 T_20) (wave 0, which holds T_20)
  if (wv == 0) {
    const float4v s = mm2(get(11), get(4), mm2(get(12), get(14), mm2(get(13), t20)));
    out(3, 0, trp(split4(mm2(get(3), split4(s)))));
  }
}

// ---------------------------------------------------------------------------------------
// Sequence split, fix-up.  The state after token t of the second segment is
// S_t = S_mid M_t + S_loc,t (the recurrence is linear in its state; M_t is the transition from
// the segment's start, whose rows evolve as state rows with V' = 0 from the identity), so
// o_t = S_mid (scale M_t q_t) + o_loc,t = S_mid q~_t + o_loc,t and S_end = S_mid M + S_loc.
// ---------------------------------------------------------------------------------------
// out[b, t, h, :] += S_mid q~_t for the second segment's tokens: one workgroup of four waves per
// (ngrp groups of 64 tokens, head, batch; more groups per workgroup amortize loading S_mid when
// there are many); wave w owns state rows 32 w .. + 31 and keeps their columns of
// S_mid^T as bf16 hi / lo B operands; per 16-token block the A operand is q~ (bf16), and the
// 16 x 32 fp32 result goes through LDS so that each lane adds 8 consecutive values of one
// token with one 16-byte read and write of out
__global__ __launch_bounds__(256) void seg_out_fixup_kernel(ChunkArgs a, const float *smid, const uint16_t *qt,
                                                             int t0, int ngrp) {
  __shared__ float tile[4][16][33];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, l4 = lane >> 4;
  const int h = blockIdx.y, b = blockIdx.z;
  const int H = a.H, T = a.T;
  const float *S = smid + (static_cast<long long>(b) * H + h) * kD * kD;   // [v][i]
  short8v bhi[2][4], blo[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const float *p = S + (32 * wave + 16 * j + l16) * kD + 32 * s2 + 8 * l4;
      const float4 x0 = ld4f(p), x1 = ld4f(p + 4);
      const Pair p0 = split4(float4v{x0.x, x0.y, x0.z, x0.w}), p1 = split4(float4v{x1.x, x1.y, x1.z, x1.w});
      bhi[j][s2] = cat(p0.h, p1.h);
      blo[j][s2] = cat(p0.l, p1.l);
    }
  const long long tokstride = static_cast<long long>(H) * kD;
  const long long head0 = (static_cast<long long>(b) * T * H + h) * kD;
  uint16_t *out = static_cast<uint16_t *>(a.out);
#pragma unroll 1
  for (int grp = 0; grp < ngrp; ++grp) {
  const int tb0 = t0 + (static_cast<int>(blockIdx.x) * ngrp + grp) * 64;
  if (tb0 >= T) break;
  // every load of the group's four 16-token blocks is issued first: the A operands (q~ rows
  // tb0 + 16 blk + l16, read clamped past the end) and this lane's 16-byte piece of out for
  // each block (token tb0 + 16 blk + lane / 4, state rows 32 wave + 8 (lane % 4) ..)
  const int tr = lane >> 2, c8 = 8 * (lane & 3);
  short8v av[4][4];
  uint4 ow[4];
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    const long long arow = head0 + static_cast<long long>(min(tb0 + 16 * blk + l16, T - 1)) * tokstride;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) av[blk][s2] = ld8(qt + arow + 32 * s2 + 8 * l4);
    const int t = min(tb0 + 16 * blk + tr, T - 1);
    ow[blk] = *reinterpret_cast<const uint4 *>(out + head0 + static_cast<long long>(t) * tokstride + 32 * wave + c8);
  }
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    const int tt = tb0 + 16 * blk;
    if (tt >= T) break;
    float4v acc[2] = {zero4(), zero4()};
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) acc[j] = mfma32(av[blk][s2], blo[j][s2], mfma32(av[blk][s2], bhi[j][s2], acc[j]));
    // lane: tokens tt + 4 l4 + r, state row 32 wave + 16 j + l16; read back as token lane / 4,
    // rows 32 wave + 8 (lane % 4) .. + 7, added to the piece of out loaded above
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) tile[wave][4 * l4 + r][16 * j + l16] = acc[j][r];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int t = tt + tr;
    if (t < T) {
      const uint4 w = ow[blk];
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = elem(w, e) + tile[wave][tr][c8 + e];
      *reinterpret_cast<uint4 *>(out + head0 + static_cast<long long>(t) * tokstride + 32 * wave + c8) =
          make_uint4(f32x2_to_bf16x2_bits(x[0], x[1]), f32x2_to_bf16x2_bits(x[2], x[3]),
                     f32x2_to_bf16x2_bits(x[4], x[5]), f32x2_to_bf16x2_bits(x[6], x[7]));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  }
}

// state_out = S_mid M + S_loc in fp32: one workgroup per (batch-head, 8 state rows), one thread
// per column; the 8 rows of S_mid sit in LDS, and each thread reads its column of M in slices
// of 32 loads issued back to back (each element of M read once for the 8 rows)
__global__ __launch_bounds__(kD) void seg_state_fixup_kernel(const float *seg_state, float *state_out, long long nbh) {
  __shared__ float rows[8][kD];
  const long long bh = blockIdx.x;
  const int v0 = 8 * static_cast<int>(blockIdx.y), k = threadIdx.x;
  const long long sz = nbh * kD * kD;
  const float *smid = seg_state + bh * kD * kD, *sloc = seg_state + sz + bh * kD * kD, *m = seg_state + 2 * sz + bh * kD * kD;
  float acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    acc[r] = sloc[(v0 + r) * kD + k];
    rows[r][k] = smid[(v0 + r) * kD + k];
  }
  __syncthreads();
  for (int i0 = 0; i0 < kD; i0 += 32) {
    float mv[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) mv[i] = m[(i0 + i) * kD + k];
#pragma unroll
    for (int i = 0; i < 32; ++i)
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[r] = fmaf(rows[r][i0 + i], mv[i], acc[r]);
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) state_out[(bh * kD + v0 + r) * kD + k] = acc[r];
}

template <int BV, bool CHAN, bool DECAY, int WK>
hipError_t launch4(const ChunkArgs &a, hipStream_t s) {
  // <= 2^22 (three groups of the value tiles with the sequence split, which needs <= 128 of them)
  const unsigned grid = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H) * (kD / BV) * (a.seg_split > 0 ? 3u : 1u);
  if (a.S > 0)
    hipLaunchKernelGGL((chunk_mfma_kernel<BV, CHAN, DECAY, WK, true, false>), dim3(grid), dim3(kNT), 0, s, a);
  else if (WK == kWkSame && BV == 32 && a.tpre != nullptr && a.seg_split > 0)
    hipLaunchKernelGGL((chunk_mfma_kernel<BV, CHAN, DECAY, WK, false, WK == kWkSame && BV == 32, false, true>), dim3(grid),
                       dim3(kNT), 0, s, a);
  else if (WK == kWkSame && BV == 32 && a.tpre != nullptr)
    hipLaunchKernelGGL((chunk_mfma_kernel<BV, CHAN, DECAY, WK, false, WK == kWkSame && BV == 32>), dim3(grid), dim3(kNT), 0, s, a);
  else
    hipLaunchKernelGGL((chunk_mfma_kernel<BV, CHAN, DECAY, WK, false, false>), dim3(grid), dim3(kNT), 0, s, a);
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

// Workspace of the per-channel decay on this kernel: the decayed operand arrays E~, Q~, R~
// ([B, T, H, 128] bf16 each), one record per (batch, head, chunk) (T, P and the state decay;
// see kda_prep.hip), then one flag per (batch, head, chunk) (the preparation's route), each
// section 256-byte aligned.
struct KdaWs {
  unsigned long long q, e, r, rec, flags, total;
};
// Sequence split (see ChunkArgs): where the batch's 32-row value tiles number at most 128 (half
// of MI355X's 256 CUs) and the sequence has two chunks or more.  The second segment starts at
// half the chunks when all three groups of workgroups fit on the CUs at once, else at two
// thirds (roles 0 and 1 start first; role 2 takes the CUs that role 1 frees).
constexpr long long kCUs = 256;
int seg_split_of(long long B, long long H, long long T) {
  const long long per = B * H * (kD / 32), nch = (T + kC - 1) / kC;
  if (per * 2 > kCUs || nch < 2) return 0;
  const long long cs = per * 3 <= kCUs ? nch / 2 : (2 * nch + 1) / 3;
  return static_cast<int>(max(1ll, min(cs, nch - 1)));
}
// bytes of T of every chunk, then (sequence split) q~ [B,T,H,128] bf16 and the three states
unsigned long long tpre_t_bytes(long long B, long long T, long long H) {
  return static_cast<unsigned long long>(B * H) * static_cast<unsigned long long>((T + kC - 1) / kC) * (10ull * 2 * 256 * 2);
}
unsigned long long seg_qt_bytes(long long B, long long T, long long H) {
  return (static_cast<unsigned long long>(B * T * H) * kD * 2 + 255ull) & ~255ull;
}

KdaWs kda_ws(long long B, long long T, long long H) {
  auto al = [](unsigned long long x) { return (x + 255ull) & ~255ull; };
  const unsigned long long arr = al(static_cast<unsigned long long>(B * T * H) * kD * 2);
  const unsigned long long nch = static_cast<unsigned long long>((T + kC - 1) / kC);
  KdaWs w;
  w.q = 0;
  w.e = arr;
  w.r = 2 * arr;
  w.rec = 3 * arr;
  w.flags = w.rec + al(static_cast<unsigned long long>(B * H) * nch * (992ull * 16));
  w.total = w.flags + al(static_cast<unsigned long long>(B * H) * nch * 4);
  return w;
}

}  // namespace

hipError_t launch_kda_prep(const ChunkArgs &a, uint16_t *qt, uint16_t *et, uint16_t *rt, uint16_t *rec,
                           uint32_t *flags, hipStream_t s);

// The per-channel decay runs on this kernel only through the workspace (prepared operands):
// bf16, Dk = Dv = 128, chunk 64, scalar gains, write key k, exact T.
bool chunk_mfma_kda_supports(const gdr_desc_t &d, const gdr_inputs_t &in, const float *state_in, const void *out,
                             const float *state_out) {
  if (d.io_dtype != GDR_BF16 || d.Dk != kD || d.Dv != kD || d.chunk != kC) return false;
  if (d.decay != GDR_DECAY_CHANNEL || d.gain != GDR_GAIN_SCALAR || d.wkey != GDR_WKEY_SAME) return false;
  if (d.neumann_order >= 0) return false;
  const void *p16[] = {in.q, in.k, in.v, in.log_alpha, out, state_in, state_out};
  for (const void *p : p16)
    if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return false;
  return true;
}

bool chunk_mfma_supports(const gdr_desc_t &d, const gdr_inputs_t &in, const float *state_in, const void *out,
                         const float *state_out) {
  if (d.io_dtype != GDR_BF16 || d.Dk != kD || d.Dv != kD || d.chunk != kC) return false;
  if (d.gain == GDR_GAIN_CHANNEL && d.wkey != GDR_WKEY_SAME) return false;
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
  if (a.decay == GDR_DECAY_CHANNEL) {
    // prepared operands first (every chunk at once), then the sequential pass as the
    // explicit-write-key variant without a decay, reading T, P and the state decay from the
    // records (the host passes this descriptor here only with its workspace)
    // (an empty sequence needs no workspace: the pass only carries the state through)
    if (a.tpre == nullptr && a.T > 0) return hipErrorInvalidValue;
    const KdaWs w = kda_ws(a.B, a.T, a.H);
    char *ws = reinterpret_cast<char *>(const_cast<uint16_t *>(a.tpre));
    uint16_t *qt = reinterpret_cast<uint16_t *>(ws + w.q), *et = reinterpret_cast<uint16_t *>(ws + w.e);
    uint16_t *rt = reinterpret_cast<uint16_t *>(ws + w.r), *rec = reinterpret_cast<uint16_t *>(ws + w.rec);
    hipError_t e = launch_kda_prep(a, qt, et, rt, rec, reinterpret_cast<uint32_t *>(ws + w.flags), s);
    if (e != hipSuccess) return e;
    ChunkArgs b = a;
    b.q = qt;
    b.k = et;
    b.write_key = rt;
    b.log_alpha = nullptr;
    b.decay = GDR_DECAY_NONE;
    b.wkey = GDR_WKEY_EXPLICIT;
    b.tpre = rec;
    const unsigned grid = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H) * (kD / 32);
    hipLaunchKernelGGL((chunk_mfma_kernel<32, false, false, kWkExplicit, false, true, true>), dim3(grid), dim3(kNT), 0, s,
                       b);
    return hipGetLastError();
  }
  if (a.tpre != nullptr) {   // T of every chunk first (the host passes tpre only where it applies)
    const int nchunks = (a.T + kC - 1) / kC;
    if (nchunks > 0) {
      const dim3 g(nchunks, a.H, a.B);
      uint16_t *tw = const_cast<uint16_t *>(a.tpre);
      const bool decay = a.decay == GDR_DECAY_SCALAR;
      if (a.gain == GDR_GAIN_CHANNEL) {
        if (decay) hipLaunchKernelGGL((chunk_t_kernel<true, true>), g, dim3(64 * kTW), 0, s, a, tw);
        else hipLaunchKernelGGL((chunk_t_kernel<true, false>), g, dim3(64 * kTW), 0, s, a, tw);
      } else {
        if (decay) hipLaunchKernelGGL((chunk_t_kernel<false, true>), g, dim3(64 * kTW), 0, s, a, tw);
        else hipLaunchKernelGGL((chunk_t_kernel<false, false>), g, dim3(64 * kTW), 0, s, a, tw);
      }
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    ChunkArgs b = a;
    const int cs = seg_split_of(a.B, a.H, a.T);
    if (cs > 0) {
      char *ws = reinterpret_cast<char *>(const_cast<uint16_t *>(a.tpre)) + tpre_t_bytes(a.B, a.T, a.H);
      b.seg_split = cs;
      b.seg_qt = reinterpret_cast<uint16_t *>(ws);
      b.seg_state = reinterpret_cast<float *>(ws + seg_qt_bytes(a.B, a.T, a.H));
    }
    hipError_t e = launch_bv<32>(b, s);
    if (e != hipSuccess || cs == 0) return e;
    const int t0 = cs * kC;
    const long long groups = (a.T - t0 + 63) / 64;
    const int ngrp = groups * a.H * a.B >= 4096 ? 4 : 1;
    hipLaunchKernelGGL(seg_out_fixup_kernel, dim3(static_cast<unsigned>((groups + ngrp - 1) / ngrp), a.H, a.B), dim3(256), 0,
                       s, a, b.seg_state, b.seg_qt, t0, ngrp);
    if (a.state_out != nullptr)
      hipLaunchKernelGGL(seg_state_fixup_kernel, dim3(static_cast<unsigned>(a.B * a.H), kD / 8), dim3(kD), 0, s,
                         b.seg_state, a.state_out, static_cast<long long>(a.B) * a.H);
    return hipGetLastError();
  }
  return chunk_mfma_bv(a) == 32 ? launch_bv<32>(a, s) : launch_bv<16>(a, s);
}

// bytes of the precomputed T for gdr_chunk_fwd_ws: its ten lower 16 x 16 blocks as bf16 pairs,
// 10 KB per (batch, head, chunk), where it applies (matrix-core kernel, write key k, exact T,
// no residual steps), else 0
unsigned long long chunk_mfma_tpre_bytes(const gdr_desc_t &d) {
  if (d.decay == GDR_DECAY_CHANNEL) {
    gdr_inputs_t none{};
    return chunk_mfma_kda_supports(d, none, nullptr, nullptr, nullptr) ? kda_ws(d.B, d.T, d.H).total : 0;
  }
  if (d.wkey != GDR_WKEY_SAME || d.neumann_order >= 0 || d.decay == GDR_DECAY_CHANNEL) return 0;
  const unsigned long long tb = tpre_t_bytes(d.B, d.T, d.H);
  if (seg_split_of(d.B, d.H, d.T) == 0) return tb;
  return tb + seg_qt_bytes(d.B, d.T, d.H) + 3ull * d.B * d.H * kD * kD * 4;
}

}  // namespace gdr
