// Prefill intra-chunk attention + inter-chunk fusion on bf16 MFMA (gfx950).
//
// Same arithmetic as the rows kernel (note §5.3 hierarchical softmax; Tide
// Fig. 3): for each selected chunk an independent softmax over its 64 keys,
// weighted by exp(s^ - Lambda); the causal own chunk enters with its exact
// log-mass. Organisation for CDNA4:
//  * A workgroup of W wavefronts (12 for d = 64, 8 for d = 128) owns R query rows:
//    Rq consecutive positions x the G query heads of one kv head. Their
//    selections are counting-sorted in LDS into one row list per chunk, so the
//    work is exactly the (row, chunk) pairs the selection asks for, packed into
//    16-row MFMA tiles.
//  * Chunk u of the workgroup's union is owned by wavefront u mod W, which loads
//    that chunk's K and V^T MFMA fragments straight into registers (from the
//    fragment copy through L2; no LDS staging and no workgroup barrier in the
//    main loop) and runs every tile of the chunk: S^T = K Q^T
//    (v_mfma_f32_16x16x32_bf16, keys on M, rows on N), a column softmax,
//    O^T = V^T P^T.
//  * The local branch is the own chunk (one causal tile per row, normalised in
//    place) or, with a sliding window of W keys, the W/S + 1 chunks the window
//    touches: a first pass over (local chunk, 16-row tile) items records each
//    row's per-chunk maximum and sum, which give the window's log-mass; after
//    Lambda is known a second pass adds exp(s_j - Lambda) v_j of every window
//    key into the row's accumulator.
//  * Contributions are added into the LDS row accumulators with integer atomics
//    in a fixed-point format scaled, row by row, from max|V| over the chunks that
//    row reads (its counted selections and its local chunks).
//    Integer addition is associative, so the result does not depend on which
//    wavefront finishes first: the output is bitwise deterministic.
//  * K and V are first rewritten (k_kv_prep), chunk by chunk, as the MFMA
//    fragments of each lane in lane order (V as V^T with the key order of the
//    MFMA k-slots), so every fragment load of a wavefront is 1 KiB of contiguous
//    memory; the same pass records max|V| per chunk.
//  * Workgroups are numbered kv-head-fastest, so consecutive workgroups (which
//    the dispatcher spreads over the 8 XCDs) give each XCD's L2 a small set of kv
//    heads whose K/V it keeps resident.
//
// MFMA 16x16x32 bf16 lane layout (lane l, g = l/16, c = l%16):
//   A[m = c][k = 8g + j], B[k = 8g + j][n = c], D[m = 4g + r][n = c].
// S^T block kb gives lane l keys 16kb + 4g + r of row c. For the P V product the
// 32 keys of step ks are placed so that k-slot 8g + j holds key 32ks + 4g + j
// (j < 4) or 32ks + 16 + 4g + (j - 4) (j >= 4): exactly the S^T values the lane
// already holds, so P needs no data movement; V^T is stored in that key order.
#include "hils_internal.h"

namespace hils {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct Cfg {
  static constexpr int RMAX = 256;                  // rows per workgroup
  // d = 128: the query rows are read from global memory at tile time and the row
  // lists hold 16-bit entries (the score is read again with the row), so that
  // 256 rows' accumulators fit in LDS: twice the rows per chunk load of 128
  static constexpr bool QG = D == 128;
  static constexpr int AP = D + 2;                  // accumulator row pitch (words, even)
  static constexpr int QP = D + 8;                  // LDS query row pitch (bf16)
  static constexpr int KF = 4 * (D / 32);           // K fragments (uint4) per lane per chunk
  static constexpr int VF = (D / 16) * 2;           // V^T fragments per lane per chunk
  // wavefronts per workgroup: 12 for d = 64 (three per SIMD, in 168 registers),
  // 8 for d = 128 (two per SIMD; its fragments alone take 128 registers)
  static constexpr int THREADS = D == 64 ? 768 : 512;
  static constexpr int WAVES = THREADS / 64;
  static constexpr int CH = (KF + VF) * 64;         // 16-byte words per chunk in the fragment copy
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x combined with its lane^16 and lane^32 partners (v_permlane16/32_swap).
__device__ __forceinline__ float xmax_16_32(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xsum_16_32(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ------------------------------------------------------------------ fragment copy
// Per chunk, the K and V^T MFMA fragments of every lane, in the order the main
// kernel reads them: fragment i of lane l is the 16-byte word i * 64 + l of the
// chunk's block, so one fragment load of a wavefront reads 1 KiB of contiguous
// memory (a direct load of K rows would put the 16 lanes of each quarter-wave on
// 16 different rows and cache lines, and the L1 tag rate would bound the kernel).
// Fragment kb (D/32) + ds of lane (c, g) holds K[16 kb + c][32 ds + 8 g .. + 8];
// fragment KF + 2 db + ks holds feature 16 db + c of the keys in k-slots
// 32 ks + 8 g .. + 8 (the k-slot key order above). Keys at or beyond Tkv are zero.
// vmax[b][g][c] = max |V| over the chunk.
template <int D>
__global__ __launch_bounds__(256) void k_kv_prep(Dims dm, int nct, const uint16_t* __restrict__ K,
                                                 const uint16_t* __restrict__ V,
                                                 uint4* __restrict__ KVf,
                                                 float* __restrict__ vmax) {
  using C = Cfg<D>;
  __shared__ uint16_t ks[kChunk][D + 8];
  __shared__ uint16_t vs[kChunk][D + 8];
  __shared__ float red[4];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const long long kv_stride = (long long)dm.Hkv * D;
  const long long kv_base = ((long long)b * dm.Tcap * dm.Hkv + g) * D;
  float mx = 0.f;
  for (int u = t; u < kChunk * D / 8; u += 256) {
    const int j = u / (D / 8), c8 = u % (D / 8);
    const long long row = (long long)c * kChunk + j;
    const long long off = kv_base + row * kv_stride + c8 * 8;
    const bool in = row < dm.Tkv;
    const uint4 kk = in ? *reinterpret_cast<const uint4*>(K + off) : make_uint4(0, 0, 0, 0);
    const uint4 v = in ? *reinterpret_cast<const uint4*>(V + off) : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(&ks[j][c8 * 8]) = kk;
    *reinterpret_cast<uint4*>(&vs[j][c8 * 8]) = v;
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      mx = fmaxf(mx, fabsf(__uint_as_float(w4[q] << 16)));
      mx = fmaxf(mx, fabsf(__uint_as_float(w4[q] & 0xFFFF0000u)));
    }
  }
  mx = wave_max(mx);
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  uint4* out = KVf + (((long long)b * dm.Hkv + g) * nct + c) * C::CH;
  for (int u = t; u < C::KF * 64; u += 256) {
    const int i = u >> 6, lc = u & 15, lg = (u >> 4) & 3;
    const int kb = i / (D / 32), ds = i % (D / 32);
    out[u] = *reinterpret_cast<const uint4*>(&ks[16 * kb + lc][32 * ds + 8 * lg]);
  }
  for (int u = t; u < C::VF * 64; u += 256) {
    const int i = u >> 6, lg = (u >> 4) & 3, kslot = i & 1;
    const int e = 16 * (i >> 1) + (u & 15);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j0 = 2 * q, j1 = 2 * q + 1;
      const int k0 = 32 * kslot + (j0 < 4 ? 4 * lg + j0 : 16 + 4 * lg + j0 - 4);
      const int k1 = 32 * kslot + (j1 < 4 ? 4 * lg + j1 : 16 + 4 * lg + j1 - 4);
      w[q] = (uint32_t)vs[k0][e] | ((uint32_t)vs[k1][e] << 16);
    }
    out[C::KF * 64 + u] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (t == 0)
    vmax[((long long)b * dm.Hkv + g) * nct + c] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ------------------------------------------------------------------ tiles
template <int D>
struct Frag {
  uint4 k[Cfg<D>::KF];  // k[kb * (D/32) + ds]: K[16kb + c][32ds + 8g .. +8]
  uint4 v[Cfg<D>::VF];  // v[db * 2 + ks]: V^T[16db + c][k-slots 32ks + 8g .. +8]
};

// Fragments of one chunk from its block of the fragment copy (word `base`).
template <int D>
__device__ __forceinline__ void load_frag(Frag<D>& f, const uint4* __restrict__ KVf,
                                          long long base) {
  const uint4* p = KVf + base + (threadIdx.x & 63);
#pragma unroll
  for (int i = 0; i < Cfg<D>::KF; ++i) f.k[i] = p[i * 64];
#pragma unroll
  for (int i = 0; i < Cfg<D>::VF; ++i) f.v[i] = p[(Cfg<D>::KF + i) * 64];
}

template <int D>
__device__ __forceinline__ void load_q(uint4* qv, const uint16_t* Q, long long row, bool valid) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds)
    qv[ds] = valid ? *reinterpret_cast<const uint4*>(Q + row * D + 32 * ds + 8 * g)
                   : make_uint4(0, 0, 0, 0);
}

// Scores, softmax weights and values of one 16-row tile of the causal own chunk:
// keys >= nk (per column) are masked. On return o[db] holds the unnormalised O^T
// block, *z the column sum of the weights and *m2 the column max of the
// log2-domain logits.
template <int D>
__device__ __forceinline__ void tile_core(const Frag<D>& f, const uint4* qv, int nk, float scale2,
                                          floatx4* o, float* z, float* m2) {
  const int g = (threadIdx.x & 63) >> 4;
  floatx4 s[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    s[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
      s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.k[kb * (D / 32) + ds]),
                                                      as_bf16x8(qv[ds]), s[kb], 0, 0, 0);
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (16 * kb + 4 * g + r >= nk) s[kb][r] = -INFINITY;
  float m = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                  fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  m = fmaxf(m, fmaxf(fmaxf(fmaxf(s[2][0], s[2][1]), fmaxf(s[2][2], s[2][3])),
                     fmaxf(fmaxf(s[3][0], s[3][1]), fmaxf(s[3][2], s[3][3]))));
  m = xmax_16_32(m);
  if (m == -INFINITY) m = 0.f;  // padding lane: keeps every value finite
  const float nb = -scale2 * m;
  float zz = 0.f;
  bf16x8 pf[2];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = fast_exp2(fmaf(s[kb][r], scale2, nb));
      zz += e;
      pf[kb >> 1][(kb & 1) * 4 + r] = (__bf16)e;
    }
  *z = xsum_16_32(zz);
  *m2 = m * scale2;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    o[db] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.v[db * 2 + ks]), pf[ks], o[db],
                                                      0, 0, 0);
  }
}

// Weight sums of the fast path that are safe to use.
__device__ __forceinline__ bool z_ok(float z) { return z >= 0x1p-64f && z <= 0x1p64f; }

// Scores, weights and values of one 16-row tile of a selected chunk. Fast path:
// u_j = 2^(s_j scale2) with no running maximum, since the intra-chunk
// normalisation divides any common factor out. The column sum z comes from the
// matrix core as a ones row times the weights, i.e. it is the sum of the bf16
// weights that multiply the values. A column whose sum falls outside
// [2^-64, 2^64], or every column when `fast` is off, takes u_j =
// 2^(s_j scale2 - m2) instead (m2 its log2-domain maximum, so the largest weight
// is 1) before the values are multiplied. The choice is made per column: a row's
// result does not depend on which other rows share its tile.
template <int D>
__device__ __forceinline__ void tile_sel(const Frag<D>& f, const uint4* qv, float scale2, bool fast,
                                         floatx4* o, float* z) {
  floatx4 s[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    s[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
      s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.k[kb * (D / 32) + ds]),
                                                      as_bf16x8(qv[ds]), s[kb], 0, 0, 0);
  }
  bf16x8 pf[2];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      pf[kb >> 1][(kb & 1) * 4 + r] = (__bf16)fast_exp2(s[kb][r] * scale2);
  const __bf16 one = (__bf16)1.0f;
  const bf16x8 ones = {one, one, one, one, one, one, one, one};
  floatx4 zz = floatx4{0.f, 0.f, 0.f, 0.f};
  zz = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[0], zz, 0, 0, 0);
  zz = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[1], zz, 0, 0, 0);
  const bool colbad = !fast || !z_ok(zz[0]);
  if (__builtin_amdgcn_ballot_w64(colbad) != 0) {
    float m = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                    fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    m = fmaxf(m, fmaxf(fmaxf(fmaxf(s[2][0], s[2][1]), fmaxf(s[2][2], s[2][3])),
                       fmaxf(fmaxf(s[3][0], s[3][1]), fmaxf(s[3][2], s[3][3]))));
    m = xmax_16_32(m);
    const float nb = -scale2 * m;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (colbad) pf[kb >> 1][(kb & 1) * 4 + r] = (__bf16)fast_exp2(fmaf(s[kb][r], scale2, nb));
    zz = floatx4{0.f, 0.f, 0.f, 0.f};
    zz = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[0], zz, 0, 0, 0);
    zz = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[1], zz, 0, 0, 0);
  }
  *z = zz[0];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    o[db] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.v[db * 2 + ks]), pf[ks], o[db],
                                                      0, 0, 0);
  }
}

// Sliding-window pass 1: column max (log2 domain, 0 for an empty column) and sum
// of 2^(s scale2 - m2) over the keys klo <= j < khi of the tile's chunk.
template <int D>
__device__ __forceinline__ void tile_stats(const Frag<D>& f, const uint4* qv, int klo, int khi,
                                           float scale2, float* m2, float* z) {
  const int g = (threadIdx.x & 63) >> 4;
  floatx4 s[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    s[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
      s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.k[kb * (D / 32) + ds]),
                                                      as_bf16x8(qv[ds]), s[kb], 0, 0, 0);
  }
  float m = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * kb + 4 * g + r;
      if (j < klo || j >= khi) s[kb][r] = -INFINITY;
      m = fmaxf(m, s[kb][r]);
    }
  m = xmax_16_32(m);
  if (m == -INFINITY) m = 0.f;
  const float nb = -scale2 * m;
  float zz = 0.f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) zz += fast_exp2(fmaf(s[kb][r], scale2, nb));
  *z = xsum_16_32(zz);
  *m2 = m * scale2;
}

// Sliding-window pass 2: o = sum over the keys klo <= j < khi of
// 2^(s_j scale2 - lam2) V_j (lam2 = Lambda log2 e, so every weight is at most 1).
template <int D>
__device__ __forceinline__ void tile_abs(const Frag<D>& f, const uint4* qv, int klo, int khi,
                                         float scale2, float lam2, floatx4* o) {
  const int g = (threadIdx.x & 63) >> 4;
  floatx4 s[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    s[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
      s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.k[kb * (D / 32) + ds]),
                                                      as_bf16x8(qv[ds]), s[kb], 0, 0, 0);
  }
  bf16x8 pf[2];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * kb + 4 * g + r;
      const float e = fast_exp2(fmaf(s[kb][r], scale2, -lam2));
      pf[kb >> 1][(kb & 1) * 4 + r] = (__bf16)(j >= klo && j < khi ? e : 0.f);
    }
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    o[db] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.v[db * 2 + ks]), pf[ks], o[db],
                                                      0, 0, 0);
  }
}

// ------------------------------------------------------------------ main kernel
// Accumulator column of feature 16 db + 4 g + r (the O^T fragment element r of
// block db held by lane group g). The four lane groups of one LDS atomic land 16
// banks apart, so rows that are a few apart (the usual spacing of the rows that
// picked a chunk) do not pile onto the same banks.
__host__ __device__ __forceinline__ int acc_col(int db, int g, int r) {
  return 64 * (db >> 2) + 16 * g + 4 * (db & 3) + r;
}

// misc: [0, 24) the set-up's scans; [kNextChunk] the next selected chunk a
// wavefront claims
constexpr int kNextChunk = 28, kMiscInts = 32;
// Selected chunks of at least kHeavyRows rows come first in the claim order;
// both groups keep ascending chunk order, which the workgroups of a kv head (on
// one XCD) share, so a chunk's fragments serve several of them from L2
constexpr int kHeavyRows = 33;

struct Smem {
  int* acc;       // [R][AP] fixed point (float during the own-chunk phase)
  uint16_t* qs;   // [R][QP] the workgroup's query rows (bf16; none with QG)
  uint32_t* ent;  // row-list entries, chunk-major: rho | k << 16 (16-bit with QG)
  uint16_t* ent16;
  float* lw;      // per entry: its chunk score times log2(e) (none with QG)
  int* rowoff;    // per row: its global row index relative to workgroup row 0
  int* cnt;
  int* off;
  int* cur;
  int* nz;
  float* lown;    // own-chunk log-mass, then the own weight in fixed-point units
  float* lam;     // Lambda times log2(e)
  float* lamx;    // Lambda times log2(e) minus the row's fixed-point shift
  int* fsh;       // per row: fixed-point shift (the row's units are 2^-fsh)
  uint32_t* rvm;  // per row: max |V| over the chunks it reads (float bits)
  float* vx;      // per chunk: max |V| (set-up only; shares off's space)
  int* gmx;       // per (row, group of 8 entries): largest id of the group (set-up
                  // only; shares pm's space)
  float* pm;      // per (row, group of 8 slots): max score and sum of exp(score - max)
  float* pz;
  int* nsel;      // per row: number of terms added to its fixed-point accumulator
  float2* lpart;  // sliding window: per (row, local chunk) max (log2 domain) and sum
  int* misc;
};

// LDS regions, each starting on a 16-byte boundary; nloc = local chunks per row
// kept by the sliding-window pass (0 without a window).
__host__ __device__ inline size_t up16(size_t x) { return (x + 15) & ~(size_t)15; }

template <int D>
__host__ __device__ inline size_t smem_bytes(int R, int K, int ncr, int nloc) {
  constexpr bool QG = Cfg<D>::QG;
  return up16((size_t)R * Cfg<D>::AP * 4) + (QG ? 0 : up16((size_t)R * Cfg<D>::QP * 2)) +
         (QG ? up16((size_t)R * K * 2) : 2 * up16((size_t)R * K * 4)) +
         4 * up16((size_t)(ncr + 1) * 4) + 7 * up16((size_t)R * 4) +
         2 * up16((size_t)R * ((K + 7) / 8) * 4) + up16((size_t)R * nloc * 8) + kMiscInts * 4;
}

template <int D>
__device__ __forceinline__ Smem carve(char* base, int R, int K, int ncr, int nloc) {
  constexpr bool QG = Cfg<D>::QG;
  Smem s;
  s.acc = reinterpret_cast<int*>(base); base += up16((size_t)R * Cfg<D>::AP * 4);
  s.qs = reinterpret_cast<uint16_t*>(base); base += QG ? 0 : up16((size_t)R * Cfg<D>::QP * 2);
  s.ent = reinterpret_cast<uint32_t*>(base);
  s.ent16 = reinterpret_cast<uint16_t*>(base);
  base += QG ? up16((size_t)R * K * 2) : up16((size_t)R * K * 4);
  s.lw = reinterpret_cast<float*>(base); base += QG ? 0 : up16((size_t)R * K * 4);
  s.cnt = reinterpret_cast<int*>(base); base += up16((ncr + 1) * 4);
  s.off = reinterpret_cast<int*>(base);
  s.vx = reinterpret_cast<float*>(base); base += up16((ncr + 1) * 4);
  s.cur = reinterpret_cast<int*>(base); base += up16((ncr + 1) * 4);
  s.nz = reinterpret_cast<int*>(base); base += up16((ncr + 1) * 4);
  s.lown = reinterpret_cast<float*>(base); base += up16(R * 4);
  s.lam = reinterpret_cast<float*>(base); base += up16(R * 4);
  s.lamx = reinterpret_cast<float*>(base); base += up16(R * 4);
  s.fsh = reinterpret_cast<int*>(base); base += up16(R * 4);
  s.rvm = reinterpret_cast<uint32_t*>(base); base += up16(R * 4);
  s.rowoff = reinterpret_cast<int*>(base); base += up16(R * 4);
  s.pm = reinterpret_cast<float*>(base);
  s.gmx = reinterpret_cast<int*>(base); base += up16((size_t)R * ((K + 7) / 8) * 4);
  s.pz = reinterpret_cast<float*>(base); base += up16((size_t)R * ((K + 7) / 8) * 4);
  s.nsel = reinterpret_cast<int*>(base); base += up16(R * 4);
  s.lpart = reinterpret_cast<float2*>(base); base += up16((size_t)R * nloc * 8);
  s.misc = reinterpret_cast<int*>(base);
  return s;
}


// In-place exclusive scan of n ints with kThreads threads; returns the total.
template <int kThreads>
__device__ __forceinline__ int block_exclusive_scan(int* a, int n, int* scratch) {
  constexpr int kWaves = kThreads / 64;
  const int t = threadIdx.x;
  const int seg = (n + kThreads - 1) / kThreads;
  const int lo = min(n, t * seg), hi = min(n, lo + seg);
  int s = 0;
  for (int x = lo; x < hi; ++x) s += a[x];
  const int lane = t & 63, w = t >> 6;
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) scratch[w] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int x = 0; x < kWaves; ++x) {
    const int v = scratch[x];
    before += x < w ? v : 0;
    total += v;
  }
  int run = before + incl - s;
  for (int x = lo; x < hi; ++x) {
    const int v = a[x];
    a[x] = run;
    run += v;
  }
  __syncthreads();
  return total;
}

// Where the workgroup's query rows and scores are read: Q and score point at
// workgroup row 0 (position qi0, head g G); rowoff holds each row's offset in rows.
struct RowSrc {
  const uint16_t* Q;
  const float* score;
};

// Query fragment of workgroup row rho (zero for an empty tile column): from LDS,
// or with QG from global memory (read unconditionally, at a clamped row).
template <int D>
__device__ __forceinline__ void lds_q(uint4* qv, const Smem& sm, const RowSrc& rs, int rho,
                                      bool valid) {
  const int g = (threadIdx.x & 63) >> 4;
  if constexpr (Cfg<D>::QG) {
    const uint16_t* qr = rs.Q + (long long)sm.rowoff[rho] * D + 8 * g;
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
      const uint4 v = *reinterpret_cast<const uint4*>(qr + 32 * ds);
      qv[ds] = valid ? v : make_uint4(0, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
      qv[ds] = valid ? *reinterpret_cast<const uint4*>(sm.qs + rho * Cfg<D>::QP + 32 * ds + 8 * g)
                     : make_uint4(0, 0, 0, 0);
  }
}

// Local-branch work items are the (local chunk, 16-row tile) pairs in chunk
// order; the rows of chunk oc are the positions oc S .. oc S + span - 1 of the
// block (span = S for the own chunk, S + W - 1 for a window of W keys). Each
// wave takes a contiguous run of items so it mostly stays on one chunk.
// Returns false when `item` is past the last one.
__device__ __forceinline__ bool own_item(int item, long long p0, int S, int span, int G, int Rv,
                                         int own_first, int own_last, int* oc_out, int* ra_out,
                                         int* rb_out, int* tl_out) {
  for (int oc = own_first; oc <= own_last; ++oc) {
    const int ra = (int)max(0LL, (long long)oc * S - p0) * G;
    const int rb = (int)min((long long)Rv, ((long long)oc * S + span - p0) * G);
    const int ntile = (rb - ra + 15) / 16;
    if (item < ntile) {
      *oc_out = oc, *ra_out = ra, *rb_out = rb, *tl_out = item;
      return true;
    }
    item -= ntile;
  }
  return false;
}

__device__ __forceinline__ int own_item_count(long long p0, int S, int span, int G, int Rv,
                                              int own_first, int own_last) {
  int n = 0;
  for (int oc = own_first; oc <= own_last; ++oc) {
    const int ra = (int)max(0LL, (long long)oc * S - p0) * G;
    const int rb = (int)min((long long)Rv, ((long long)oc * S + span - p0) * G);
    n += (rb - ra + 15) / 16;
  }
  return n;
}

// Adds one tile's normalised, fused-weighted output to its rows' fixed-point
// accumulators: weight 2^(lw2 - lamx) / z (lw2 = s^ log2 e, lamx = Lambda log2 e
// minus the row's fixed-point shift, so the weight is alpha in the row's units).
// The conversion to an integer is one fma: for |v| < 2^22, v + 1.5 2^23 is a
// float whose bit pattern is 0x4B400000 + round(v). Two neighbouring columns a, b
// share one 64-bit word and one 64-bit integer atomic: the word gains
// bits(b) 2^32 + bits(a), and the sum of such words is exact mod 2^64 whatever the
// order. The offsets (kMagic (2^32 + 1) per added term) are removed at the end.
constexpr float kMagicF = 12582912.0f;  // 1.5 * 2^23
constexpr uint32_t kMagic = 0x4B400000u;

template <int D>
__device__ __forceinline__ void accumulate_fw(const Smem& sm, const floatx4* o, int rho,
                                              float fw) {
  const int gl = (threadIdx.x & 63) >> 4;
  int* ar = sm.acc + rho * Cfg<D>::AP;
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int q = 0; q < 4; q += 2) {
      const uint64_t lo = __float_as_uint(fmaf(o[db][q], fw, kMagicF));
      const uint64_t hi = __float_as_uint(fmaf(o[db][q + 1], fw, kMagicF));
      atomicAdd(reinterpret_cast<unsigned long long*>(ar + acc_col(db, gl, q)),
                (unsigned long long)((hi << 32) | lo));
    }
}

template <int D>
__device__ __forceinline__ void accumulate_tile(const Smem& sm, const floatx4* o, float z, int rho,
                                                float lw2, float lamx) {
  const float fw = fast_exp2(lw2 - lamx) * __builtin_amdgcn_rcpf(z);
  accumulate_fw<D>(sm, o, rho, fw);
}

// Entry word of a chunk's row list: workgroup row (bits 0-15), selection slot
// (bits 16-21), and bit 30 set when the row's values are too large for the
// fast-path weights (max |V| >= 2^50). With QG the entry is 16 bits: row (bits
// 0-7), slot (bits 8-13), slow-path flag (bit 14).
constexpr uint32_t kEntrySlow = 1u << 30;
constexpr uint32_t kEntrySlow16 = 1u << 14;


// Row-list entry e of a chunk, clamped to the last entry so every read is of real
// data (a lane past the end computes a copy of the last row and does not
// accumulate it); reads happen without branches, so they stay in flight. Returns
// the entry's row, its slow-path flag, its chunk score times log2(e) and the
// row's query fragments.
template <int D>
__device__ __forceinline__ void read_entry(const Smem& sm, const RowSrc& rs, int Ksel, int e0,
                                           int n, int e, bool* v, int* rho, bool* slow, float* lw,
                                           float* lm, uint4* q) {
  *v = e < n;
  const int ec = e0 + min(e, n - 1);
  const int g = (threadIdx.x & 63) >> 4;
  if constexpr (Cfg<D>::QG) {
    const uint32_t en = sm.ent16[ec];
    *rho = (int)(en & 0xFFu);
    *slow = (en & 0x4000u) != 0u;
    const long long ro = sm.rowoff[*rho];
    *lw = rs.score[ro * Ksel + ((en >> 8) & 63u)] * kLog2e;
    const uint16_t* qr = rs.Q + ro * D + 8 * g;
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) q[ds] = *reinterpret_cast<const uint4*>(qr + 32 * ds);
  } else {
    const uint32_t en = sm.ent[ec];
    *rho = (int)(en & 0xFFFFu);
    *slow = (en & kEntrySlow) != 0u;
    *lw = sm.lw[ec];
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
      q[ds] = *reinterpret_cast<const uint4*>(sm.qs + *rho * Cfg<D>::QP + 32 * ds + 8 * g);
  }
  *lm = sm.lamx[*rho];
}

// The first tile's entry, query fragments and row normaliser of a chunk (or, for
// a step past the chunk's rows, of any of its entries; such a column does not
// accumulate).
template <int D>
struct TileIn {
  bool v, slow;
  int rho;
  float lw, lm;
  uint4 q[D / 32];
};

// All tiles of one selected chunk c (fragments in f) for the rows that picked
// it, one 16-row tile per step; `in` holds the first tile's entry, read ahead.
// Each step reads the next step's entry, query fragments and row normaliser
// while it runs; the last step reads those of the first tile of chunk cn (the
// chunk this wave claimed next, -1 for none) into `in`, so that the next
// chunk's query reads are issued before its fragment loads and its first score
// products wait only for K, not for the V fragments behind it.
// d = 64 (query rows in LDS): all tiles of chunk c, the first tile's entry read
// when the chunk starts, each step reading the next step's while it runs.
template <int D>
__device__ __forceinline__ void run_chunk_lds(const Frag<D>& f, const Smem& sm, const RowSrc& rs,
                                              int Ksel, int c, float scale2) {
  const int col = threadIdx.x & 15;
  const int e0 = sm.off[c], n = sm.cnt[c];
  const int nstep = (n + 15) / 16;
  bool v, slow;
  int rho;
  float lw, lm;
  uint4 q[D / 32];
  read_entry<D>(sm, rs, Ksel, e0, n, col, &v, &rho, &slow, &lw, &lm, q);
  for (int st = 0; st < nstep; ++st) {
    bool vn, slown;
    int rhon;
    float lwn, lmn;
    uint4 qn[D / 32];
    read_entry<D>(sm, rs, Ksel, e0, n, 16 * (st + 1) + col, &vn, &rhon, &slown, &lwn, &lmn, qn);
    floatx4 o[D / 16];
    float z;
    tile_sel<D>(f, q, scale2, !slow, o, &z);
    if (v) accumulate_tile<D>(sm, o, z, rho, lw, lm);
    v = vn, rho = rhon, slow = slown, lw = lwn, lm = lmn;
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) q[ds] = qn[ds];
  }
}

// nxt: the list index this wave claimed next (valid in lane 0; read at the last
// step, where the next chunk's first tile is read ahead, so the claim's latency
// stays hidden behind the earlier tiles); returns it, wave-uniform.
template <int D>
__device__ __forceinline__ int run_chunk(Frag<D>& f, const uint4* __restrict__ KVf,
                                         long long kvf_base, const Smem& sm, const RowSrc& rs,
                                         int Ksel, int c, int nxt, int nnz, float scale2,
                                         TileIn<D>& in) {
  const int col = threadIdx.x & 15;
  const int e0 = sm.off[c], n = sm.cnt[c];
  const int nstep = (n + 15) / 16;
  int un = nnz, cn = -1;
  for (int st = 0; st < nstep; ++st) {
    TileIn<D> nx;
    int ce0 = e0, cnn = n, ce = 16 * (st + 1) + col;
    if (st + 1 == nstep) {
      un = __builtin_amdgcn_readfirstlane(nxt);
      if (un < nnz) {
        cn = __builtin_amdgcn_readfirstlane(sm.cur[un]);
        ce0 = sm.off[cn], cnn = sm.cnt[cn], ce = col;
      }
    }
    read_entry<D>(sm, rs, Ksel, ce0, cnn, ce, &nx.v, &nx.rho, &nx.slow, &nx.lw, &nx.lm, nx.q);
    floatx4 o[D / 16];
    float z;
    tile_sel<D>(f, in.q, scale2, !in.slow, o, &z);
    // last step: the products of this chunk are done with f, so the next chunk's
    // fragments load while this tile accumulates
    if (cn >= 0) load_frag<D>(f, KVf, kvf_base + (long long)cn * Cfg<D>::CH);
    if (in.v) accumulate_tile<D>(sm, o, z, in.rho, in.lw, in.lm);
    in = nx;
  }
  return un;
}

template <int D, bool SWA>
__global__ __launch_bounds__(Cfg<D>::THREADS) void k_attend_mfma(
    Dims dm, int R, int Rq, int ncr_cap, int nqb, int nct, const uint16_t* __restrict__ Q,
    const uint4* __restrict__ KVf, const float* __restrict__ vmax, const int32_t* __restrict__ idx,
    const float* __restrict__ score, uint16_t* __restrict__ O, float* __restrict__ lse_own,
    float* __restrict__ lse_tot) {
  using C = Cfg<D>;
  constexpr int kThreads = C::THREADS, kWaves = C::WAVES;
  extern __shared__ __align__(16) char smem_raw[];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, col = lane & 15, gl = lane >> 4;
  const int G = dm.G, Ksel = dm.K, S = dm.S;
  // kv head fastest: neighbouring workgroups (spread over XCDs) share few kv heads;
  // query blocks from the last one down, so the blocks with the most candidate
  // chunks (the latest positions) start first and the cheap ones fill in
  const int L = blockIdx.x;
  const int g = L % dm.Hkv, qb = nqb - 1 - (L / dm.Hkv) % nqb, b = L / (dm.Hkv * nqb);
  const int qi0 = qb * Rq;
  const int nq = min(Rq, dm.Tq - qi0);
  const int Rv = nq * G;
  const long long p0 = dm.q_pos0 + qi0;
  const int own_first = (int)(p0 / S), own_last = (int)((p0 + nq - 1) / S);
  const int ncr = own_last;  // selectable chunks lie in [0, own_last)
  // local chunks of the block and the rows each one serves (see own_item)
  const int span = SWA ? S + dm.window - 1 : S;
  const int loc_first = SWA ? (int)(dm.lstart(p0) / S) : own_first;
  const int nloc = SWA ? dm.nlocal_max() : 0;
  Smem sm = carve<D>(smem_raw, R, Ksel, ncr_cap, nloc);
  const long long kvf_base = ((long long)b * dm.Hkv + g) * nct * (long long)C::CH;
  const float* vmx = vmax + ((long long)b * dm.Hkv + g) * nct;
  const float scale2 = dm.scale * kLog2e;
  // global row of workgroup row rho (query position qi0 + rho / G, head g G + rho % G)
  auto row_of = [&](int rho) -> long long {
    return ((long long)b * dm.Tq + qi0 + rho / G) * dm.H + (long long)g * G + rho % G;
  };
  const long long row0 = row_of(0);
  const RowSrc rs{Q + row0 * D, score + row0 * Ksel};

  // own-chunk items of this wave
  const int n_own = own_item_count(p0, S, span, G, Rv, loc_first, own_last);
  const int per_wave = (n_own + kWaves - 1) / kWaves;
  const int item0 = w * per_wave, item_end = min(n_own, item0 + per_wave);
  Frag<D> f;
  int o_oc = 0, o_ra = 0, o_rb = 0, o_tl = 0;
  bool o_have = item0 < item_end && own_item(item0, p0, S, span, G, Rv, loc_first, own_last,
                                             &o_oc, &o_ra, &o_rb, &o_tl);
  // d = 128: the fragments of this wave's first local chunk load during the
  // set-up (measured 2% faster at d = 128, 1% slower at d = 64, whose set-up
  // stages the query rows)
  constexpr bool kEarly = D == 128;
  int fc0 = -1;
  if (kEarly && o_have) {
    load_frag<D>(f, KVf, kvf_base + (long long)o_oc * C::CH);
    fc0 = o_oc;
  }

  // ---- set-up: every global read of the set-up is issued first
  const int kgroups = (Ksel + 7) / 8;  // Rv * kgroups <= kThreads (see plan)
  const bool has_item = t < Rv * kgroups;
  const int it_rho = t / kgroups, it_kg = t % kgroups, it_k0 = it_kg * 8;
  const long long it_pos = p0 + it_rho / G;
  const int it_own = dm.ncand(it_pos);  // the row's candidates: chunks below this
  int cs[8];
  float ss[8];
  {
    const long long r = has_item ? row_of(it_rho) : 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool in = has_item && it_k0 + j < Ksel;
      cs[j] = in ? idx[r * Ksel + it_k0 + j] : -1;
      ss[j] = in ? score[r * Ksel + it_k0 + j] : -INFINITY;
    }
  }
  const int nqv = Rv * (D / 8);  // <= 4 * kThreads (see plan)
  auto ldq = [&](int j) -> uint4 {  // past the end: reload the last piece (in bounds)
    const int x = min(t + j * kThreads, nqv - 1);
    return *reinterpret_cast<const uint4*>(Q + row_of(x / (D / 8)) * D + (x % (D / 8)) * 8);
  };
  auto stq = [&](int j, uint4 v) {
    const int x = t + j * kThreads;
    if (x < nqv) *reinterpret_cast<uint4*>(sm.qs + (x / (D / 8)) * C::QP + (x % (D / 8)) * 8) = v;
  };
  uint4 qv0 = make_uint4(0, 0, 0, 0), qv1 = qv0, qv2 = qv0, qv3 = qv0;
  if constexpr (!C::QG) qv0 = ldq(0), qv1 = ldq(1), qv2 = ldq(2), qv3 = ldq(3);
  const float vpre = t <= own_last ? vmx[t] : 0.f;

  for (int c = t; c <= ncr; c += kThreads) sm.cnt[c] = 0;
  for (int c = t; c <= own_last; c += kThreads) sm.vx[c] = c == t ? vpre : vmx[c];
  for (int rho = t; rho < Rv; rho += kThreads) {
    sm.nsel[rho] = 0;
    sm.rvm[rho] = 0u;
    sm.rowoff[rho] = (rho / G) * dm.H + rho % G;
  }
  if (has_item) {
    int m8 = -1;
#pragma unroll
    for (int j = 0; j < 8; ++j) m8 = max(m8, cs[j]);
    sm.gmx[t] = m8;  // t = it_rho * kgroups + it_kg
  }
  __syncthreads();
  if constexpr (!C::QG) stq(0, qv0), stq(1, qv1), stq(2, qv2), stq(3, qv3);
  // the entries that count (entry_counts: a candidate above every earlier entry
  // of the row); the others lose their score too, so they leave Lambda alone
  uint32_t okm = 0u;
  float rv = 0.f;  // max |V| over the chunks of the row this thread sees
  if (has_item) {
    int prev = -1;
    for (int x = 0; x < it_kg; ++x) prev = max(prev, sm.gmx[it_rho * kgroups + x]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      okm |= entry_counts(cs[j], it_own, prev) ? 1u << j : 0u;
      prev = max(prev, cs[j]);
    }
    if (it_kg == 0)  // the row's local chunks
      for (int c = (int)(dm.lstart(it_pos) / S); c <= (int)(it_pos / S); ++c) rv = fmaxf(rv, sm.vx[c]);
  }
  int nmine = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if ((okm >> j) & 1u) {
      atomicAdd(&sm.cnt[cs[j]], 1);
      rv = fmaxf(rv, sm.vx[cs[j]]);
      ++nmine;
    } else {
      ss[j] = -INFINITY;
    }
  }
  if (has_item) {
    if (nmine) atomicAdd(&sm.nsel[it_rho], nmine);
    atomicMax(&sm.rvm[it_rho], __float_as_uint(rv));  // non-negative floats order as their bits
  }
  __syncthreads();
  for (int c = t; c < ncr; c += kThreads) {
    const int n = sm.cnt[c];
    sm.off[c] = n;
    sm.nz[c] = n >= kHeavyRows ? 1 << 16 : (n > 0 ? 1 : 0);  // heavy and light counts in one word
  }
  __syncthreads();
  block_exclusive_scan<kThreads>(sm.off, ncr, sm.misc);
  const int nzt = block_exclusive_scan<kThreads>(sm.nz, ncr, sm.misc + 12);
  const int nheavy = nzt >> 16, nnz = nheavy + (nzt & 0xFFFF);  // selected chunks
  for (int c = t; c < ncr; c += kThreads) sm.cur[c] = sm.off[c];
  __syncthreads();
  {
    // fast path: weight sums below 2^64 and values below 2^50 keep every partial
    // product of the PV step finite; the row's flag travels in its entries
    const bool slow = has_item && __uint_as_float(sm.rvm[it_rho]) >= 0x1p50f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((okm >> j) & 1u) {
        const int p = atomicAdd(&sm.cur[cs[j]], 1);
        if constexpr (C::QG) {
          sm.ent16[p] = (uint16_t)((uint32_t)it_rho | ((uint32_t)(it_k0 + j) << 8) |
                                   (slow ? kEntrySlow16 : 0u));
        } else {
          sm.ent[p] = (uint32_t)it_rho | ((uint32_t)(it_k0 + j) << 16) | (slow ? kEntrySlow : 0u);
          sm.lw[p] = ss[j] * kLog2e;
        }
      }
  }
  if (has_item) {  // partial log-sum-exp of this group of scores (padding holds -inf)
    float m8 = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) m8 = fmaxf(m8, ss[j]);
    float z8 = 0.f;
    if (m8 > -INFINITY) {
#pragma unroll
      for (int j = 0; j < 8; ++j) z8 += expf(ss[j] - m8);
    }
    sm.pm[t] = m8;
    sm.pz[t] = z8;
  }
  __syncthreads();
  // compacted list of the selected chunks in claim order: the heavy ones, then
  // the rest, each in ascending chunk order (the wavefronts claim them in list
  // order, so the last ones claimed are short and the wavefronts finish together)
  for (int c = t; c < ncr; c += kThreads) {
    const int n = sm.cnt[c], x = sm.nz[c];
    if (n >= kHeavyRows) sm.cur[x >> 16] = c;
    else if (n > 0) sm.cur[nheavy + (x & 0xFFFF)] = c;
  }
  // per-row fixed point: every partial sum of a row is a sub-convex combination
  // of the values of the chunks it reads, so its magnitude is at most that
  // row's max|V| < 2^ex, mapped below 2^21 (each term then fits the one-fma
  // conversion of accumulate_fw); the row's units are 2^-(21 - ex)
  for (int rho = t; rho < Rv; rho += kThreads) {
    int ex = 0;
    frexpf(fmaxf(__uint_as_float(sm.rvm[rho]), 1e-30f), &ex);
    sm.fsh[rho] = 21 - ex;
  }

  // ---- sliding window, pass 1: per (row, local chunk) maximum and sum. Items are
  // taken two at a time when they share a chunk, so two independent tiles run
  // per step (every chunk in loc_first .. own_last has rows, see own_item).
  auto win_next = [&](int& oc, int& ra, int& rb, int& tl) {
    if (16 * ++tl >= rb - ra) {
      ++oc;
      tl = 0;
      ra = (int)max(0LL, (long long)oc * S - p0) * G;
      rb = (int)min((long long)Rv, ((long long)oc * S + span - p0) * G);
    }
  };
  // rows, key bounds and query fragments of the tile (oc, ra, rb, tl); `on` false
  // gives an empty tile
  auto win_tile = [&](bool on, int oc, int ra, int rb, int tl, int* rho, bool* valid, int* klo,
                      int* khi, int* lofs, uint4* qo) {
    *rho = ra + 16 * tl + col;
    *valid = on && *rho < rb;
    const long long pos = p0 + (*valid ? *rho : ra) / G, cb = (long long)oc * S;
    const long long l0 = dm.lstart(pos);
    *klo = *valid ? (int)max(0LL, l0 - cb) : 0;
    *khi = *valid ? (int)min((long long)S, pos - cb + 1) : 0;
    *lofs = oc - (int)(l0 / S);
    lds_q<D>(qo, sm, rs, min(*rho, Rv - 1), *valid);
  };
  if constexpr (SWA) {
    int fc = fc0;  // chunk whose fragments f holds
    int oc = o_oc, ra = o_ra, rb = o_rb, tl = o_tl;
    for (int left = o_have ? item_end - item0 : 0; left > 0;) {
      int oc2 = oc, ra2 = ra, rb2 = rb, tl2 = tl;
      win_next(oc2, ra2, rb2, tl2);
      const bool two = left >= 2 && oc2 == oc;
      if (oc != fc) {
        load_frag<D>(f, KVf, kvf_base + (long long)(oc) * C::CH);
        fc = oc;
      }
      int rho[2], klo[2], khi[2], lofs[2];
      bool valid[2];
      uint4 qo[2][D / 32];
      win_tile(true, oc, ra, rb, tl, &rho[0], &valid[0], &klo[0], &khi[0], &lofs[0], qo[0]);
      win_tile(two, oc2, ra2, rb2, tl2, &rho[1], &valid[1], &klo[1], &khi[1], &lofs[1], qo[1]);
      float m2[2], z[2];
      tile_stats<D>(f, qo[0], klo[0], khi[0], scale2, &m2[0], &z[0]);
      tile_stats<D>(f, qo[1], klo[1], khi[1], scale2, &m2[1], &z[1]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (valid[i] && gl == 0) sm.lpart[rho[i] * nloc + lofs[i]] = make_float2(m2[i], z[i]);
      oc = oc2, ra = ra2, rb = rb2, tl = tl2;
      if (two) win_next(oc, ra, rb, tl);
      left -= two ? 2 : 1;
    }
  }
  // ---- own chunks: causal, normalised (float accumulators for now)
  for (int item = item0, fc = fc0; !SWA && o_have; ) {
    if (o_oc != fc) {
      load_frag<D>(f, KVf, kvf_base + (long long)(o_oc) * C::CH);
      fc = o_oc;
    }
    const int rho = o_ra + 16 * o_tl + col;
    const bool valid = rho < o_rb;
    const int nk = valid ? (int)(p0 + rho / G - (long long)o_oc * S) + 1 : 0;
    uint4 qo[D / 32];
    lds_q<D>(qo, sm, rs, min(rho, Rv - 1), valid);
    floatx4 o[D / 16];
    float z, m2;
    tile_core<D>(f, qo, nk, scale2, o, &z, &m2);
    if (valid) {
      const float inv = __builtin_amdgcn_rcpf(z);
      float* ar = reinterpret_cast<float*>(sm.acc + rho * C::AP);
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q) ar[acc_col(db, gl, q)] = o[db][q] * inv;
      if (gl == 0) sm.lown[rho] = (m2 + __log2f(z)) * kLn2;
    }
    ++item;
    o_have = item < item_end && own_item(item, p0, S, span, G, Rv, loc_first, own_last, &o_oc,
                                         &o_ra, &o_rb, &o_tl);
  }
  __syncthreads();

  // d = 128: the first selected chunk's fragments load during the normaliser and
  // the fixed-point conversion (the window's second pass needs f before that)
  constexpr bool kFirst = kEarly && !SWA;
  if (kFirst && w < nnz) load_frag<D>(f, KVf, kvf_base + (long long)(sm.cur[w]) * C::CH);

  // ---- fusion normaliser per row from the local log-mass and the score partials
  for (int rho = t; rho < Rv; rho += kThreads) {
    float lo;
    if constexpr (SWA) {  // the window's log-mass from its chunks' partials, in chunk order
      const int nl = dm.nlocal(p0 + rho / G);
      const float2* lp = sm.lpart + rho * nloc;
      float m2 = -INFINITY;
      for (int k = 0; k < nl; ++k) m2 = fmaxf(m2, lp[k].x);
      float z = 0.f;
      for (int k = 0; k < nl; ++k) z += lp[k].y * exp2f(lp[k].x - m2);
      lo = (m2 + log2f(z)) * kLn2;
      sm.nsel[rho] += nl;  // one term per local chunk in pass 2
    } else {
      lo = sm.lown[rho];
    }
    float mx = lo;
    for (int kg = 0; kg < kgroups; ++kg) mx = fmaxf(mx, sm.pm[rho * kgroups + kg]);
    float z = expf(lo - mx);
    for (int kg = 0; kg < kgroups; ++kg) {
      const float zg = sm.pz[rho * kgroups + kg];
      if (zg > 0.f) z += zg * expf(sm.pm[rho * kgroups + kg] - mx);
    }
    const float lam = mx + logf(z);
    const int sh = sm.fsh[rho];
    sm.lam[rho] = lam * kLog2e;
    sm.lamx[rho] = lam * kLog2e - (float)sh;
    sm.lown[rho] = ldexpf(expf(lo - lam), sh);
    const long long r = row_of(rho);
    if (lse_own) lse_own[r] = lo;
    if (lse_tot) lse_tot[r] = lam;
  }
  if (t == 0) sm.misc[kNextChunk] = kWaves;  // the chunks after each wave's first
  __syncthreads();
  // own contribution to fixed point: columns 2k, 2k + 1 become the 64-bit word
  // b 2^32 + a of their signed values
  for (int x = t; x < Rv * (D / 2); x += kThreads) {
    const int rho = x / (D / 2), e = 2 * (x % (D / 2));
    int64_t* a = reinterpret_cast<int64_t*>(sm.acc + rho * C::AP + e);
    if constexpr (SWA) {
      *a = 0;
    } else {
      const float2 v = *reinterpret_cast<const float2*>(a);
      const float w = sm.lown[rho];  // rounded to the nearest unit, as the other terms are
      *a = (int64_t)__float2int_rn(v.y * w) * 4294967296LL + (int64_t)__float2int_rn(v.x * w);
    }
  }
  __syncthreads();

  // ---- sliding window, pass 2: exp(s_j - Lambda) v_j of every window key,
  // two tiles per step as in pass 1
  if constexpr (SWA) {
    int oc = 0, ra = 0, rb = 0, tl = 0, fc = -1;
    const bool have = item0 < item_end &&
                      own_item(item0, p0, S, span, G, Rv, loc_first, own_last, &oc, &ra, &rb, &tl);
    for (int left = have ? item_end - item0 : 0; left > 0;) {
      int oc2 = oc, ra2 = ra, rb2 = rb, tl2 = tl;
      win_next(oc2, ra2, rb2, tl2);
      const bool two = left >= 2 && oc2 == oc;
      if (oc != fc) {
        load_frag<D>(f, KVf, kvf_base + (long long)(oc) * C::CH);
        fc = oc;
      }
      int rho[2], klo[2], khi[2], lofs[2];
      bool valid[2];
      uint4 qo[2][D / 32];
      win_tile(true, oc, ra, rb, tl, &rho[0], &valid[0], &klo[0], &khi[0], &lofs[0], qo[0]);
      win_tile(two, oc2, ra2, rb2, tl2, &rho[1], &valid[1], &klo[1], &khi[1], &lofs[1], qo[1]);
      floatx4 o[2][D / 16];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        tile_abs<D>(f, qo[i], klo[i], khi[i], scale2, valid[i] ? sm.lam[rho[i]] : 0.f, o[i]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (valid[i]) accumulate_fw<D>(sm, o[i], rho[i], ldexpf(1.0f, sm.fsh[rho[i]]));
      oc = oc2, ra = ra2, rb = rb2, tl = tl2;
      if (two) win_next(oc, ra, rb, tl);
      left -= two ? 2 : 1;
    }
  }

  // ---- selected chunks: wavefront w starts with chunk w, then claims the next
  // unclaimed one from an LDS counter (chunks hold different numbers of tiles,
  // so a fixed share leaves some wavefronts idle at the end); no barriers. A wave
  // waiting for its chunk's fragments is covered by the other waves of its SIMD
  // (more waves per SIMD measured faster than a second fragment set).
  // With the query rows in global memory (d = 128) a chunk's first tile is read
  // ahead during the previous chunk's last tile (measured 4% faster at the 7B
  // shape); from LDS (d = 64) it is read when the chunk starts (the read-ahead
  // measured 3% slower there).
  if constexpr (C::QG) {
    TileIn<D> tin;
    if (w < nnz) {
      const int c = sm.cur[w];
      read_entry<D>(sm, rs, Ksel, sm.off[c], sm.cnt[c], col, &tin.v, &tin.rho, &tin.slow,
                    &tin.lw, &tin.lm, tin.q);
    }
    // the first chunk's fragments load here (or earlier, see kFirst); every later
    // chunk's during the last tile of the chunk before it
    if (!kFirst && w < nnz) load_frag<D>(f, KVf, kvf_base + (long long)(sm.cur[w]) * C::CH);
    for (int u = w; u < nnz;) {
      int nxt = 0;
      if (lane == 0) nxt = atomicAdd(sm.misc + kNextChunk, 1);  // in flight during the tiles
      u = run_chunk<D>(f, KVf, kvf_base, sm, rs, Ksel, sm.cur[u], nxt, nnz, scale2, tin);
    }
  } else {
    for (int u = w; u < nnz;) {
      if (!kFirst || u != w) load_frag<D>(f, KVf, kvf_base + (long long)(sm.cur[u]) * C::CH);
      int nxt = 0;
      if (lane == 0) nxt = atomicAdd(sm.misc + kNextChunk, 1);  // in flight during the tiles
      run_chunk_lds<D>(f, sm, rs, Ksel, sm.cur[u], scale2);
      u = __builtin_amdgcn_readfirstlane(nxt);
    }
  }
  __syncthreads();

  // ---- write O (bf16, round to nearest even)
  for (int x = t; x < Rv * (D / 8); x += kThreads) {
    const int rho = x / (D / 8), c8 = x % (D / 8);
    const int* ar = sm.acc + rho * C::AP;
    const uint64_t off = (uint64_t)sm.nsel[rho] * ((uint64_t)kMagic * 4294967297ull);
    const int sh = sm.fsh[rho];
    // features 8 c8 .. 8 c8 + 7 are columns acc_col(db, g, 0..3) for g = 2 (c8 & 1),
    // 2 (c8 & 1) + 1 and db = c8 / 2; each pair of columns is one 64-bit word
    const int db = c8 >> 1, g0 = 2 * (c8 & 1);
    uint32_t ow[4];
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int g = g0 + (y >> 1), r = 2 * (y & 1);
      const int64_t xw = (int64_t)(*reinterpret_cast<const uint64_t*>(ar + acc_col(db, g, r)) - off);
      const int a = (int)(uint32_t)xw;
      const int b = (int)((xw - a) >> 32);
      ow[y] = (uint32_t)f32_to_bf16_bits(ldexpf((float)a, -sh)) |
              ((uint32_t)f32_to_bf16_bits(ldexpf((float)b, -sh)) << 16);
    }
    *reinterpret_cast<uint4*>(O + row_of(rho) * D + c8 * 8) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
  }
}

struct Plan {
  int R, Rq, ncr, nqb, nct;
  size_t bytes, kvf_bytes, vmax_bytes;
};

template <int D>
bool plan(const Dims& dm, Plan* p) {
  if (!dm.bf16) return false;
  int r = Cfg<D>::RMAX;
  while (r > 16 && r * dm.K > 4096) r /= 2;
  int rq = r / dm.G;
  if (rq < 1) return false;
  const long long last = dm.q_pos0 + dm.Tq - 1;
  const int ncr = (int)(last / dm.S) + 1;
  const int nloc = dm.window > 0 ? dm.nlocal_max() : 0;
  const size_t limit = 160 * 1024;
  while (rq > 1 && smem_bytes<D>(rq * dm.G, dm.K, ncr, nloc) > limit) rq -= max(1, rq / 8);
  r = rq * dm.G;
  const size_t b = smem_bytes<D>(r, dm.K, ncr, nloc);
  if (b > limit) return false;
  // the set-up gives each thread at most one (row, 8 selections) item and four
  // 16-byte pieces of the query rows
  if (r * ((dm.K + 7) / 8) > Cfg<D>::THREADS) return false;
  if (!Cfg<D>::QG && r * (D / 8) > 4 * Cfg<D>::THREADS) return false;
  p->R = r;
  p->Rq = rq;
  p->ncr = ncr;
  p->nqb = (dm.Tq + rq - 1) / rq;
  p->nct = (int)((last + dm.S) / dm.S);  // chunks holding keys 0..last
  p->bytes = b;
  p->kvf_bytes = (size_t)dm.B * dm.Hkv * p->nct * Cfg<D>::CH * 16;
  p->vmax_bytes = (size_t)dm.B * dm.Hkv * p->nct * 4;
  return true;
}

template <int D>
hipError_t launch_t(const Dims& dm, const Plan& p, const void* Q, const void* K, const void* V,
                    const int32_t* idx, const float* score, void* O, float* lse_own,
                    float* lse_tot, void* ws, hipStream_t st) {
  uint4* kvf = reinterpret_cast<uint4*>(ws);
  float* vmax = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                         ((p.kvf_bytes + 255) & ~(size_t)255));
  hipLaunchKernelGGL((k_kv_prep<D>), dim3(p.nct, dm.Hkv, dm.B), dim3(256), 0, st, dm, p.nct,
                     reinterpret_cast<const uint16_t*>(K), reinterpret_cast<const uint16_t*>(V),
                     kvf, vmax);
  auto kfn = dm.window > 0 ? k_attend_mfma<D, true> : k_attend_mfma<D, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, dim3(dm.B * p.nqb * dm.Hkv), dim3(Cfg<D>::THREADS), p.bytes, st, dm,
                     p.R, p.Rq,
                     p.ncr, p.nqb, p.nct, reinterpret_cast<const uint16_t*>(Q),
                     kvf, vmax, idx, score,
                     reinterpret_cast<uint16_t*>(O), lse_own, lse_tot);
  return hipGetLastError();
}

bool plan_any(const Dims& dm, Plan* p) {
  if (dm.Tq < 64) return false;  // single rows (decode) use the rows kernel
  return dm.d == 64 ? plan<64>(dm, p) : plan<128>(dm, p);
}

}  // namespace

size_t attend_mfma_ws_bytes(const Dims& dm) {
  Plan p;
  if (!plan_any(dm, &p)) return 0;
  return ((p.kvf_bytes + 255) & ~(size_t)255) + p.vmax_bytes;
}

// Launches and returns true when the MFMA path applies (bf16, prefill-sized,
// LDS plan fits); returns false to let the caller use the rows kernel.
bool attend_mfma_try(const Dims& dm, const void* Q, const void* K, const void* V,
                     const int32_t* idx, const float* score, void* O, float* lse_own,
                     float* lse_tot, void* ws, hipStream_t st, hipError_t* err) {
  Plan p;
  if (!plan_any(dm, &p)) return false;
  *err = dm.d == 64 ? launch_t<64>(dm, p, Q, K, V, idx, score, O, lse_own, lse_tot, ws, st)
                    : launch_t<128>(dm, p, Q, K, V, idx, score, O, lse_own, lse_tot, ws, st);
  return true;
}

}  // namespace hils
