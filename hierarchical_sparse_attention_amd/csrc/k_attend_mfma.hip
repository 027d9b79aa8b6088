// Prefill intra-chunk attention + inter-chunk fusion on bf16 MFMA (gfx950).
//
// Same arithmetic as the rows kernel (note §5.3 hierarchical softmax; Tide
// Fig. 3): for each selected chunk an independent softmax over its 64 keys,
// weighted by exp(s^ - Lambda); the causal own chunk enters with its exact
// log-mass. Organisation for CDNA4:
//  * A workgroup (8 wavefronts) owns R query rows: Rq consecutive positions x the
//    G query heads of one kv head. Their selections are counting-sorted in LDS
//    into one row list per chunk, so the work is exactly the (row, chunk) pairs
//    the selection asks for, packed into 16-row MFMA tiles.
//  * Chunk u of the workgroup's union is owned by wavefront u mod 8, which loads
//    that chunk's K and V^T MFMA fragments straight into registers (from L2; no
//    LDS staging and no workgroup barrier in the main loop) and runs every tile
//    of the chunk: S^T = K Q^T (v_mfma_f32_16x16x32_bf16, keys on M, rows on N),
//    a column softmax, O^T = V^T P^T.
//  * Contributions are added into the LDS row accumulators with integer atomics
//    in a fixed-point format scaled from max|V| over the workgroup's chunks.
//    Integer addition is associative, so the result does not depend on which
//    wavefront finishes first: the output is bitwise deterministic.
//  * V is first rewritten (k_vt_prep) chunk by chunk as V^T with the key order of
//    the MFMA k-slots, so each V^T fragment is one 16-byte load; the same pass
//    records max|V| per chunk.
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

constexpr int kThreads = 512;  // 8 wavefronts: two per SIMD
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct Cfg {
  static constexpr int RMAX = D == 64 ? 256 : 128;  // rows per workgroup
  static constexpr int AP = D + 1;                  // accumulator row pitch (words)
  static constexpr int KF = 4 * (D / 32);           // K fragments (uint4) per lane per chunk
  static constexpr int VF = (D / 16) * 2;           // V^T fragments per lane per chunk
  static constexpr bool PREFETCH = D == 64;         // second fragment set in registers
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

// ------------------------------------------------------------------ V^T prepass
// Vt[b][g][c][e][p]: feature e of chunk c in k-slot order p (see above), zero for
// keys at or beyond Tkv; vmax[b][g][c] = max |V| over the chunk.
template <int D>
__global__ __launch_bounds__(256) void k_vt_prep(Dims dm, int nct, const uint16_t* __restrict__ V,
                                                 uint16_t* __restrict__ Vt,
                                                 float* __restrict__ vmax) {
  __shared__ uint16_t vs[kChunk][D + 8];
  __shared__ float red[4];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const long long kv_stride = (long long)dm.Hkv * D;
  const long long kv_base = ((long long)b * dm.Tcap * dm.Hkv + g) * D;
  float mx = 0.f;
  for (int u = t; u < kChunk * D / 8; u += 256) {
    const int j = u / (D / 8), c8 = u % (D / 8);
    const long long row = (long long)c * kChunk + j;
    uint4 v = row < dm.Tkv ? *reinterpret_cast<const uint4*>(V + kv_base + row * kv_stride + c8 * 8)
                           : make_uint4(0, 0, 0, 0);
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
  const long long cbase = (((long long)b * dm.Hkv + g) * nct + c) * (long long)D * kChunk;
  for (int u = t; u < D * 8; u += 256) {
    const int e = u / 8, p8 = u % 8;  // feature e, k-slot run p8*8..p8*8+7
    const int ks = p8 / 4, gg = p8 % 4;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j0 = 2 * q, j1 = 2 * q + 1;
      const int k0 = 32 * ks + (j0 < 4 ? 4 * gg + j0 : 16 + 4 * gg + j0 - 4);
      const int k1 = 32 * ks + (j1 < 4 ? 4 * gg + j1 : 16 + 4 * gg + j1 - 4);
      w[q] = (uint32_t)vs[k0][e] | ((uint32_t)vs[k1][e] << 16);
    }
    *reinterpret_cast<uint4*>(Vt + cbase + (long long)e * kChunk + p8 * 8) =
        make_uint4(w[0], w[1], w[2], w[3]);
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

// Key rows at or beyond Tkv (a partial trailing own chunk) are clamped to the last
// key: they are masked out of the softmax, so only the read must stay in bounds.
template <int D>
__device__ __forceinline__ void load_frag(Frag<D>& f, const uint16_t* K, const uint16_t* Vt,
                                          long long kv_base, long long kv_stride, int chunk,
                                          long long vt_chunk_base, long long Tkv) {
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
      const long long row = min((long long)chunk * kChunk + 16 * kb + c, Tkv - 1);
      f.k[kb * (D / 32) + ds] =
          *reinterpret_cast<const uint4*>(K + kv_base + row * kv_stride + 32 * ds + 8 * g);
    }
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      f.v[db * 2 + ks] = *reinterpret_cast<const uint4*>(
          Vt + vt_chunk_base + (long long)(16 * db + c) * kChunk + 32 * ks + 8 * g);
}

template <int D>
__device__ __forceinline__ void load_q(uint4* qv, const uint16_t* Q, long long row, bool valid) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds)
    qv[ds] = valid ? *reinterpret_cast<const uint4*>(Q + row * D + 32 * ds + 8 * g)
                   : make_uint4(0, 0, 0, 0);
}

// Scores, softmax weights and values of one 16-row tile. keys >= nk are masked
// (causal own chunk; nk = 64 for selected chunks). On return o[db] holds the
// unnormalised O^T block, *z the column sum of the weights and *m2 the column max
// of the log2-domain logits.
template <int D, bool MASK>
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
  if (MASK) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * kb + 4 * g + r >= nk) s[kb][r] = -INFINITY;
  }
  float m = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                  fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  m = fmaxf(m, fmaxf(fmaxf(fmaxf(s[2][0], s[2][1]), fmaxf(s[2][2], s[2][3])),
                     fmaxf(fmaxf(s[3][0], s[3][1]), fmaxf(s[3][2], s[3][3]))));
  m = xmax_16_32(m);
  if (MASK && m == -INFINITY) m = 0.f;  // padding lane: keeps every value finite
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

// ------------------------------------------------------------------ main kernel
struct Smem {
  int* acc;     // [R][AP] fixed point (float during the own-chunk phase)
  uint32_t* ent;
  float* lw;    // fusion log2-weight (s^ - Lambda) log2(e) of each entry
  int* cnt;
  int* off;
  int* cur;
  int* nz;
  float* lown;
  float* lam;
  int* rowid;
  int* misc;
};

template <int D>
__host__ __device__ inline size_t smem_bytes(int R, int K, int ncr) {
  return (size_t)R * Cfg<D>::AP * 4 + (size_t)R * K * 8 + 4 * (size_t)(ncr + 1) * 4 +
         3 * (size_t)R * 4 + 32 * 4;
}

template <int D>
__device__ __forceinline__ Smem carve(char* base, int R, int K, int ncr) {
  Smem s;
  s.acc = reinterpret_cast<int*>(base); base += (size_t)R * Cfg<D>::AP * 4;
  s.ent = reinterpret_cast<uint32_t*>(base); base += (size_t)R * K * 4;
  s.lw = reinterpret_cast<float*>(base); base += (size_t)R * K * 4;
  s.cnt = reinterpret_cast<int*>(base); base += (ncr + 1) * 4;
  s.off = reinterpret_cast<int*>(base); base += (ncr + 1) * 4;
  s.cur = reinterpret_cast<int*>(base); base += (ncr + 1) * 4;
  s.nz = reinterpret_cast<int*>(base); base += (ncr + 1) * 4;
  s.lown = reinterpret_cast<float*>(base); base += R * 4;
  s.lam = reinterpret_cast<float*>(base); base += R * 4;
  s.rowid = reinterpret_cast<int*>(base); base += R * 4;
  s.misc = reinterpret_cast<int*>(base);
  return s;
}

// In-place exclusive scan of n ints with kThreads threads; returns the total.
__device__ __forceinline__ int block_exclusive_scan(int* a, int n, int* scratch) {
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

template <int D>
__global__ __launch_bounds__(kThreads) void k_attend_mfma(
    Dims dm, int R, int Rq, int ncr_cap, int nqb, int nct, const uint16_t* __restrict__ Q,
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ Vt,
    const float* __restrict__ vmax, const int32_t* __restrict__ idx,
    const float* __restrict__ score, uint16_t* __restrict__ O, float* __restrict__ lse_own,
    float* __restrict__ lse_tot) {
  using C = Cfg<D>;
  extern __shared__ __align__(16) char smem_raw[];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, col = lane & 15, gl = lane >> 4;
  const int G = dm.G, Ksel = dm.K, S = dm.S;
  // kv head fastest: neighbouring workgroups (spread over XCDs) share few kv heads
  const int L = blockIdx.x;
  const int g = L % dm.Hkv, qb = (L / dm.Hkv) % nqb, b = L / (dm.Hkv * nqb);
  const int qi0 = qb * Rq;
  const int nq = min(Rq, dm.Tq - qi0);
  const int Rv = nq * G;
  const long long p0 = dm.q_pos0 + qi0;
  const int own_first = (int)(p0 / S), own_last = (int)((p0 + nq - 1) / S);
  const int ncr = own_last;  // selectable chunks: [0, own_last)
  Smem sm = carve<D>(smem_raw, R, Ksel, ncr_cap);
  const long long kv_stride = (long long)dm.Hkv * D;
  const long long kv_base = ((long long)b * dm.Tcap * dm.Hkv + g) * D;
  const long long vt_base = ((long long)b * dm.Hkv + g) * nct * (long long)D * kChunk;
  const float* vmx = vmax + ((long long)b * dm.Hkv + g) * nct;
  const float scale2 = dm.scale * kLog2e;

  // ---- setup: row table and per-chunk row lists (counting sort of the selections)
  for (int c = t; c <= ncr; c += kThreads) sm.cnt[c] = 0;
  for (int rho = t; rho < Rv; rho += kThreads)
    sm.rowid[rho] = (int)(((long long)b * dm.Tq + qi0 + rho / G) * dm.H + (long long)g * G + rho % G);
  __syncthreads();
  for (int rho = t; rho < Rv; rho += kThreads) {
    const long long r = sm.rowid[rho];
    const int own = (int)((p0 + rho / G) / S);
    for (int k = 0; k < Ksel; ++k) {
      const int c = idx[r * Ksel + k];
      if (c >= 0 && c < own) atomicAdd(&sm.cnt[c], 1);
    }
  }
  __syncthreads();
  for (int c = t; c < ncr; c += kThreads) {
    sm.off[c] = sm.cnt[c];
    sm.nz[c] = sm.cnt[c] > 0 ? 1 : 0;
  }
  __syncthreads();
  const int nent = block_exclusive_scan(sm.off, ncr, sm.misc);
  const int nnz = block_exclusive_scan(sm.nz, ncr, sm.misc + 8);
  for (int c = t; c < ncr; c += kThreads) sm.cur[c] = sm.off[c];
  __syncthreads();
  for (int rho = t; rho < Rv; rho += kThreads) {
    const long long r = sm.rowid[rho];
    const int own = (int)((p0 + rho / G) / S);
    for (int k = 0; k < Ksel; ++k) {
      const int c = idx[r * Ksel + k];
      if (c >= 0 && c < own) {
        const int p = atomicAdd(&sm.cur[c], 1);
        sm.ent[p] = (uint32_t)rho | ((uint32_t)k << 16);
      }
    }
  }
  __syncthreads();
  // compacted list of non-empty chunks (chunk c goes to slot nz[c]) and the bound
  // max|V| over every chunk this workgroup reads
  float vm = 0.f;
  for (int c = t; c < ncr; c += kThreads)
    if (sm.cnt[c] > 0) {
      sm.cur[sm.nz[c]] = c;
      vm = fmaxf(vm, vmx[c]);
    }
  for (int c = own_first + t; c <= own_last; c += kThreads) vm = fmaxf(vm, vmx[c]);
  vm = wave_max(vm);
  if (lane == 0) reinterpret_cast<float*>(sm.misc)[16 + w] = vm;
  __syncthreads();
  float vmax_wg = 0.f;
#pragma unroll
  for (int x = 0; x < kWaves; ++x)
    vmax_wg = fmaxf(vmax_wg, reinterpret_cast<float*>(sm.misc)[16 + x]);
  // fixed point: every partial sum is a sub-convex combination of values, so its
  // magnitude is at most max|V| < 2^ex, mapped below 2^29
  int ex = 0;
  frexpf(fmaxf(vmax_wg, 1e-30f), &ex);
  const float fx_scale = ldexpf(1.0f, 29 - ex);
  const float fx_inv = ldexpf(1.0f, ex - 29);

  // ---- own chunks: causal, normalised; items (own chunk, 16-row tile) round robin
  {
    Frag<D> f;
    int loaded = -1;
    int item = 0;
    for (int oc = own_first; oc <= own_last; ++oc) {
      const int ra = (int)max(0LL, (long long)oc * S - p0) * G;
      const int rb = (int)min((long long)Rv, ((long long)oc * S + S - p0) * G);
      const int ntile = (rb - ra + 15) / 16;
      for (int tl = 0; tl < ntile; ++tl, ++item) {
        if (item % kWaves != w) continue;
        if (loaded != oc) {
          load_frag<D>(f, K, Vt, kv_base, kv_stride, oc, vt_base + (long long)oc * D * kChunk, dm.Tkv);
          loaded = oc;
        }
        const int rho = ra + 16 * tl + col;
        const bool valid = rho < rb;
        const long long r = valid ? sm.rowid[rho] : 0;
        const int nk = valid ? (int)(p0 + rho / G - (long long)oc * S) + 1 : 0;
        uint4 qv[D / 32];
        load_q<D>(qv, Q, r, valid);
        floatx4 o[D / 16];
        float z, m2;
        tile_core<D, true>(f, qv, nk, scale2, o, &z, &m2);
        if (valid) {
          const float inv = 1.0f / z;
          float* ar = reinterpret_cast<float*>(sm.acc + rho * C::AP);
#pragma unroll
          for (int db = 0; db < D / 16; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) ar[16 * db + 4 * gl + q] = o[db][q] * inv;
          if (gl == 0) sm.lown[rho] = (m2 + __log2f(z)) * kLn2;
        }
      }
    }
  }
  __syncthreads();

  // ---- fusion normaliser per row; own contribution to fixed point
  for (int rho = t; rho < Rv; rho += kThreads) {
    const long long r = sm.rowid[rho];
    const float lo = sm.lown[rho];
    float mx = lo;
    for (int k = 0; k < Ksel; ++k) mx = fmaxf(mx, score[r * Ksel + k]);
    float z = expf(lo - mx);
    for (int k = 0; k < Ksel; ++k) z += expf(score[r * Ksel + k] - mx);
    const float lam = mx + logf(z);
    sm.lam[rho] = lam;
    const float a = expf(lo - lam) * fx_scale;
    int* ar = sm.acc + rho * C::AP;
    for (int e = 0; e < D; ++e) ar[e] = (int)(__int_as_float(ar[e]) * a);
    if (lse_own) lse_own[r] = lo;
    if (lse_tot) lse_tot[r] = lam;
  }
  __syncthreads();
  for (int e = t; e < nent; e += kThreads) {
    const uint32_t en = sm.ent[e];
    const int rho = (int)(en & 0xFFFFu), k = (int)(en >> 16);
    sm.lw[e] = (score[(long long)sm.rowid[rho] * Ksel + k] - sm.lam[rho]) * kLog2e;
  }
  __syncthreads();

  // ---- selected chunks: chunk u belongs to wavefront u mod 8; no barriers
  {
    Frag<D> f, fn;
    if (w < nnz)
      load_frag<D>(f, K, Vt, kv_base, kv_stride, sm.cur[w],
                   vt_base + (long long)sm.cur[w] * D * kChunk, dm.Tkv);
    for (int u = w; u < nnz; u += kWaves) {
      const int c = sm.cur[u];
      const bool more = u + kWaves < nnz;
      if (C::PREFETCH && more)
        load_frag<D>(fn, K, Vt, kv_base, kv_stride, sm.cur[u + kWaves],
                     vt_base + (long long)sm.cur[u + kWaves] * D * kChunk, dm.Tkv);
      const int e0 = sm.off[c], n = sm.cnt[c];
      const int ntile = (n + 15) / 16;
      uint4 qv[D / 32];
      {
        const bool v0 = col < n;
        const int rho0 = v0 ? (int)(sm.ent[e0 + col] & 0xFFFFu) : 0;
        load_q<D>(qv, Q, v0 ? sm.rowid[rho0] : 0, v0);
      }
      for (int tl = 0; tl < ntile; ++tl) {
        const int e = 16 * tl + col;
        const bool valid = e < n;
        const uint32_t en = valid ? sm.ent[e0 + e] : 0u;
        const int rho = (int)(en & 0xFFFFu);
        const float lw2 = valid ? sm.lw[e0 + e] : 0.f;
        uint4 qc[D / 32];
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds) qc[ds] = qv[ds];
        if (tl + 1 < ntile) {  // prefetch the next tile's query fragments
          const int e1 = e + 16;
          const bool v1 = e1 < n;
          const int rho1 = v1 ? (int)(sm.ent[e0 + e1] & 0xFFFFu) : 0;
          load_q<D>(qv, Q, v1 ? sm.rowid[rho1] : 0, v1);
        }
        floatx4 o[D / 16];
        float z, m2;
        tile_core<D, false>(f, qc, kChunk, scale2, o, &z, &m2);
        if (valid) {
          const float fw = fast_exp2(lw2) / z * fx_scale;
          int* ar = sm.acc + rho * C::AP;
#pragma unroll
          for (int db = 0; db < D / 16; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) atomicAdd(ar + 16 * db + 4 * gl + q, (int)(o[db][q] * fw));
        }
      }
      if (more) {
        if (C::PREFETCH) {
          f = fn;
        } else {
          load_frag<D>(f, K, Vt, kv_base, kv_stride, sm.cur[u + kWaves],
                       vt_base + (long long)sm.cur[u + kWaves] * D * kChunk, dm.Tkv);
        }
      }
    }
  }
  __syncthreads();

  // ---- write O (bf16, round to nearest even)
  for (int x = t; x < Rv * (D / 8); x += kThreads) {
    const int rho = x / (D / 8), c8 = x % (D / 8);
    const int* ar = sm.acc + rho * C::AP + c8 * 8;
    uint32_t ow[4];
#pragma unroll
    for (int y = 0; y < 4; ++y)
      ow[y] = (uint32_t)f32_to_bf16_bits((float)ar[2 * y] * fx_inv) |
              ((uint32_t)f32_to_bf16_bits((float)ar[2 * y + 1] * fx_inv) << 16);
    *reinterpret_cast<uint4*>(O + (long long)sm.rowid[rho] * D + c8 * 8) =
        make_uint4(ow[0], ow[1], ow[2], ow[3]);
  }
}

struct Plan {
  int R, Rq, ncr, nqb, nct;
  size_t bytes, vt_bytes, vmax_bytes;
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
  const size_t limit = 160 * 1024;
  while (rq > 1 && smem_bytes<D>(rq * dm.G, dm.K, ncr) > limit) rq -= max(1, rq / 8);
  r = rq * dm.G;
  const size_t b = smem_bytes<D>(r, dm.K, ncr);
  if (b > limit) return false;
  p->R = r;
  p->Rq = rq;
  p->ncr = ncr;
  p->nqb = (dm.Tq + rq - 1) / rq;
  p->nct = (int)((last + dm.S) / dm.S);  // chunks holding keys 0..last
  p->bytes = b;
  p->vt_bytes = (size_t)dm.B * dm.Hkv * p->nct * D * kChunk * 2;
  p->vmax_bytes = (size_t)dm.B * dm.Hkv * p->nct * 4;
  return true;
}

template <int D>
hipError_t launch_t(const Dims& dm, const Plan& p, const void* Q, const void* K, const void* V,
                    const int32_t* idx, const float* score, void* O, float* lse_own,
                    float* lse_tot, void* ws, hipStream_t st) {
  uint16_t* vt = reinterpret_cast<uint16_t*>(ws);
  float* vmax = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                         ((p.vt_bytes + 255) & ~(size_t)255));
  hipLaunchKernelGGL((k_vt_prep<D>), dim3(p.nct, dm.Hkv, dm.B), dim3(256), 0, st, dm, p.nct,
                     reinterpret_cast<const uint16_t*>(V), vt, vmax);
  auto kfn = k_attend_mfma<D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, dim3(dm.B * p.nqb * dm.Hkv), dim3(kThreads), p.bytes, st, dm, p.R, p.Rq,
                     p.ncr, p.nqb, p.nct, reinterpret_cast<const uint16_t*>(Q),
                     reinterpret_cast<const uint16_t*>(K), vt, vmax, idx, score,
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
  return ((p.vt_bytes + 255) & ~(size_t)255) + p.vmax_bytes;
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
