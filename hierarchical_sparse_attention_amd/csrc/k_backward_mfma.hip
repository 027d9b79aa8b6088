// Training backward of HiLS attention on bf16 MFMA (gfx950), d = 64.
//
// Same gradients as the rows/chunk kernels of k_backward.hip (note §5.3: the
// chunk score enters the forward weights, so the loss gradient reaches the
// query, the summary key, the entropy bias and through the landmark softmax
// (note §5.1) the landmark query and the keys). Per row i with fused weights
// alpha_c = exp(s^_c - Lambda), intra-chunk softmax P, u_j = dO.v_j,
// r_c = sum_j P_j u_j and D = sum_c alpha_c r_c + sum_own w_j u_j = dO.O:
//   selected chunk: ds_j = alpha_c P_j (u_j - r_c), value weight alpha_c P_j,
//                   ds^_c = alpha_c (r_c - D)
//   local branch:   ds_j = w_j (u_j - D), w_j = exp(s_j - Lambda) over its keys
//                   (the own chunk up to the row, or the last W keys)
//   dQ = scale (sum ds_j k_j + sum_c ds^_c k'_c),  dK_j += scale ds_j q,
//   dV_j += weight dO,  dk'_c = scale sum_i ds^_ic q_i,  db'_c = sum_i ds^_ic,
//   ds'_j = p'_j [dk'.(k_j - k'_c) + db' (L' - s'_j - b'_c)],
//   dQl = scale sum_j ds'_j k_j,  dK_j += p'_j dk'_c + scale ds'_j Ql.
//
// Kernels (no floating-point atomics; every sum has a fixed order, so the
// gradients are bitwise reproducible):
//   k_bwd_rowd   : D = dO.O per row from the forward output
//   k_sel_count, k_sel_scan, k_sel_fill: per (b, h, chunk) the rows that
//                  selected the chunk (ascending) as records (position, alpha,
//                  D, slot)
//   k_bwd_kv_mfma: one workgroup per (chunk, kv head); the rows whose local
//                  branch covers keys of the chunk (its own 64 rows, or with a
//                  window of W keys the next S + W - 1 positions) and the rows
//                  that selected it, in 32-row tiles: S^T, U^T on MFMA,
//                  weights and dS through LDS, dK += dS^T Q and dV += A^T dO on
//                  MFMA, ds^ = alpha (r - D) into dk' and db', and each row's
//                  dQ contribution K^T dS^T (+ ds^ k') on MFMA into the row's
//                  slot of a bf16 partial buffer; then the summary and landmark
//                  backward; writes dK, dV, dQl.
//   k_dq_reduce  : dQ = scale * sum of a row's slots in slot order.
// With a Q-Cal scoring query Qs (note §5.4) the chunk scores were computed
// from Qs: dk'_c sums ds^ Qs instead of ds^ q, the partial slots leave out
// ds^ k', and k_dq_reduce forms dQs = scale sum_c ds^_c k'_c from the ds^
// values the key side wrote per (row, slot).
#include <type_traits>

#include "hils_internal.h"

namespace hils {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int D = 64;
constexpr int kLanes = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int KF = 4 * (D / 32);  // row fragments (uint4) of a 64-key chunk per lane

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}
__device__ __forceinline__ floatx4 mfma(uint4 a, uint4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
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
__device__ __forceinline__ float bf(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// MFMA 16x16x32 bf16 lane layout (lane l, g = l / 16, c = l % 16):
//   A[m = c][k = 8g + j], B[k = 8g + j][n = c], D[m = 4g + r][n = c].
// S^T block kb of a chunk gives lane l keys 16 kb + 4g + r of tile row c. For a
// product whose k dimension is the chunk's keys, k-slot 8g + j of step ks holds
// key 32 ks + 4g + j (j < 4) or 32 ks + 16 + 4g + (j - 4) (j >= 4): exactly the
// S^T values the lane holds, so weights need no data movement; K^T is read in
// that key order from LDS (lds_ktfrag).

// ------------------------------------------------------------------ rows
// D = dO . O per row (eight lanes per row, 16-byte loads).
__global__ __launch_bounds__(256) void k_bwd_rowd(long long rows, const uint16_t* __restrict__ O,
                                                  const uint16_t* __restrict__ dO,
                                                  float* __restrict__ ws_D) {
  const long long r = (long long)blockIdx.x * 32 + threadIdx.x / 8;
  const int c8 = threadIdx.x % 8;
  const long long rr = min(r, rows - 1);
  const uint4 ov = *reinterpret_cast<const uint4*>(dO + rr * D + c8 * 8);
  const uint4 yv = *reinterpret_cast<const uint4*>(O + rr * D + c8 * 8);
  const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w}, yw[4] = {yv.x, yv.y, yv.z, yv.w};
  float dd = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    dd = fmaf(__uint_as_float(ow[q] << 16), __uint_as_float(yw[q] << 16),
              fmaf(__uint_as_float(ow[q] & 0xFFFF0000u), __uint_as_float(yw[q] & 0xFFFF0000u), dd));
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) dd += __shfl_xor(dd, o, kLanes);
  if (c8 == 0 && r < rows) ws_D[r] = dd;
}

// dQ = scale * (sum over the row's slots of its dQ partials, fixed slot order):
// slot k < K holds selected chunk idx[k] (written only for valid selections),
// slots K .. K + NL - 1 the local branch's chunks (the first nlocal of them are
// written). Eight lanes per row, 16-byte loads issued together.
template <int KM, bool QCAL>
__global__ __launch_bounds__(256) void k_dq_reduce(Dims dm, long long rows,
                                                   const int32_t* __restrict__ idx,
                                                   const uint16_t* __restrict__ part,
                                                   uint16_t* __restrict__ dQ,
                                                   const float* __restrict__ ws_dsh,
                                                   const float* __restrict__ ksum,
                                                   uint16_t* __restrict__ dQs) {
  const long long r0 = (long long)blockIdx.x * 32 + threadIdx.x / 8;
  const long long r = min(r0, rows - 1);
  const int c8 = threadIdx.x % 8;
  const int Ksel = dm.K, NC = dm.Tkv / dm.S, NS = Ksel + dm.nlocal_max();
  const int pos = (int)((r / dm.H) % dm.Tq);
  const int own = dm.ncand(dm.q_pos0 + pos);           // candidates: chunks below this
  const int nloc = dm.nlocal(dm.q_pos0 + pos);         // written local slots
  const uint16_t* pr = part + r * (long long)NS * D + c8 * 8;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  int seen = -1;  // largest selection id so far (entry_counts)
  for (int k0 = 0; k0 < NS; k0 += KM) {
    uint4 v[KM];
    bool ok[KM];
    int cq[KM];
#pragma unroll
    for (int q = 0; q < KM; ++q) {
      const int k = min(k0 + q, NS - 1);
      cq[q] = k < Ksel ? idx[r * Ksel + k] : -1;
      v[q] = *reinterpret_cast<const uint4*>(pr + (long long)k * D);
    }
#pragma unroll
    for (int q = 0; q < KM; ++q) {
      const int k = min(k0 + q, NS - 1);
      ok[q] = k0 + q < NS &&
              (k < Ksel ? entry_counts(cq[q], min(own, NC), seen) : k - Ksel < nloc);
      if (k0 + q < NS && k < Ksel) seen = max(seen, cq[q]);
    }
#pragma unroll
    for (int q = 0; q < KM; ++q) {
      const uint32_t wv[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += ok[q] ? __uint_as_float(wv[j] << 16) : 0.f;
        acc[2 * j + 1] += ok[q] ? __uint_as_float(wv[j] & 0xFFFF0000u) : 0.f;
      }
    }
  }
  float accs[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) accs[j] = 0.f;
  if constexpr (QCAL) {
    // dQs: ds^ k' over the selected slots in slot order, eight slots' loads at a time
    const long long b = r / ((long long)dm.Tq * dm.H);
    const int h = (int)(r % dm.H);
    constexpr int KS = 8;
    int seen_s = -1;
    for (int k0 = 0; k0 < Ksel; k0 += KS) {
      float dsv[KS];
      float4 ka[KS], kb[KS];
#pragma unroll
      for (int q = 0; q < KS; ++q) {
        const int k = min(k0 + q, Ksel - 1);
        const int c = idx[r * Ksel + k];
        const bool okq = k0 + q < Ksel && entry_counts(c, min(own, NC), seen_s);
        if (k0 + q < Ksel) seen_s = max(seen_s, c);
        dsv[q] = okq ? ws_dsh[r * Ksel + k] : 0.f;
        const float* kp = ksum + (((b * dm.NCcap + (okq ? c : 0)) * dm.H + h) * D + c8 * 8);
        ka[q] = *reinterpret_cast<const float4*>(kp);
        kb[q] = *reinterpret_cast<const float4*>(kp + 4);
      }
#pragma unroll
      for (int q = 0; q < KS; ++q) {
        accs[0] = fmaf(dsv[q], ka[q].x, accs[0]);
        accs[1] = fmaf(dsv[q], ka[q].y, accs[1]);
        accs[2] = fmaf(dsv[q], ka[q].z, accs[2]);
        accs[3] = fmaf(dsv[q], ka[q].w, accs[3]);
        accs[4] = fmaf(dsv[q], kb[q].x, accs[4]);
        accs[5] = fmaf(dsv[q], kb[q].y, accs[5]);
        accs[6] = fmaf(dsv[q], kb[q].z, accs[6]);
        accs[7] = fmaf(dsv[q], kb[q].w, accs[7]);
      }
    }
  }
  if (r0 >= rows) return;
  uint32_t ow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    ow[j] = (uint32_t)f32_to_bf16_bits(acc[2 * j] * dm.scale) |
            ((uint32_t)f32_to_bf16_bits(acc[2 * j + 1] * dm.scale) << 16);
  *reinterpret_cast<uint4*>(dQ + r * D + c8 * 8) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
  if constexpr (QCAL) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      ow[j] = (uint32_t)f32_to_bf16_bits(accs[2 * j] * dm.scale) |
              ((uint32_t)f32_to_bf16_bits(accs[2 * j + 1] * dm.scale) << 16);
    *reinterpret_cast<uint4*>(dQs + r * D + c8 * 8) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
  }
}

// ------------------------------------------------------------------ selection lists
// For every (b, h, chunk c): the rows that selected c (positions ascending) with
// their fusion weight alpha = exp(s^ - Lambda) and D, stored contiguously, so
// that the key side reads its rows' data in one coalesced pass. Built in three
// deterministic passes over blocks of kLBlk positions: per-block counts, an
// exclusive scan per (b, h) in (chunk, block) order, and a fill that ranks each
// selecting position within its block by popcounts of a block bitmap.
// 256 positions per block (8 bitmap words): the fill's LDS (bitmap, staged
// records) then fits three workgroups per compute unit at K = 16, whose phases
// overlap (one 512-position workgroup per compute unit left every barrier and
// round trip exposed)
constexpr int kLBlk = 256;

// A row's K selection entries into registers (KM >= K slots, all reads issued
// together; slots past K repeat entry K - 1 and are never used).
template <int KM>
__device__ __forceinline__ void load_row_ids(const int32_t* __restrict__ ir, int K, int (&cv)[KM]) {
#pragma unroll
  for (int k = 0; k < KM; ++k) cv[k] = ir[min(k, K - 1)];
}

template <int KM>
__global__ __launch_bounds__(256) void k_sel_count(Dims dm, int nblk, const int32_t* __restrict__ idx,
                                                   int* __restrict__ cnt) {
  extern __shared__ int lcnt[];  // [NC]
  const int NC = dm.Tkv / dm.S;
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  for (int x = threadIdx.x; x < NC; x += blockDim.x) lcnt[x] = 0;
  __syncthreads();
  const int i0 = blk * kLBlk, ni = min(kLBlk, dm.Tq - i0);
  // one thread per row: its entries in order, so entry_counts sees the earlier ids
  for (int ii = threadIdx.x; ii < ni; ii += blockDim.x) {
    const int i = i0 + ii;
    const int n = min(dm.ncand(dm.q_pos0 + i), NC);
    int cv[KM];
    load_row_ids<KM>(idx + (((long long)b * dm.Tq + i) * dm.H + h) * dm.K, dm.K, cv);
    int seen = -1;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (k < dm.K && entry_counts(cv[k], n, seen)) atomicAdd(&lcnt[cv[k]], 1);
      seen = max(seen, cv[k]);
    }
  }
  __syncthreads();
  int* out = cnt + ((long long)b * dm.H + h) * NC * nblk;
  for (int c = threadIdx.x; c < NC; c += blockDim.x) out[(long long)c * nblk + blk] = lcnt[c];
}

// In place: cnt[b][h][c][blk] -> offset of the block's entries of chunk c in the
// (b, h) list space; lstart / llen per (b, h, c). Each thread takes a contiguous
// segment, sixteen counts' loads in flight at a time.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void k_sel_scan(Dims dm, int nblk, int* __restrict__ cnt,
                                                           int* __restrict__ lstart,
                                                           int* __restrict__ llen) {
  constexpr int kW = kScanThreads / 64;
  __shared__ int wtot[kW];
  const int NC = dm.Tkv / dm.S;
  const long long bh = (long long)blockIdx.y * dm.H + blockIdx.x;
  int* a = cnt + bh * NC * nblk;
  const int n = NC * nblk;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int seg = (n + kScanThreads - 1) / kScanThreads;
  const int lo = min(n, t * seg), hi = min(n, lo + seg);
  int s = 0;
  for (int x0 = lo; x0 < hi; x0 += 16) {
    int v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = x0 + j < hi ? a[x0 + j] : 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += v[j];
  }
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wtot[w] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int x = 0; x < kW; ++x) {
    before += x < w ? wtot[x] : 0;
    total += wtot[x];
  }
  int run = before + incl - s;
  for (int x0 = lo; x0 < hi; x0 += 16) {
    int v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = x0 + j < hi ? a[x0 + j] : 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (x0 + j < hi) a[x0 + j] = run;
      run += v[j];
    }
  }
  __syncthreads();
  for (int c = t; c < NC; c += kScanThreads) {
    const int st = a[(long long)c * nblk];
    const int en = c + 1 < NC ? a[(long long)(c + 1) * nblk] : total;
    lstart[bh * NC + c] = st;
    llen[bh * NC + c] = en - st;
  }
}

// STAGED (when the block's entries fit in LDS beside the bitmap): the records are
// first placed in LDS in list order (chunk, then rank) as packed (position,
// slot, chunk) words with their weights alpha, and the rows' D, and then written
// out in that order from LDS alone, so consecutive threads write consecutive
// 16-byte records: whole cache lines, where writing each row's records from its
// own thread scatters 16-byte pieces over a line per chunk. Each row's entries
// and scores are read once, all at a time. The records and their places are the
// same either way.
constexpr int kFillThreads = kLBlk;  // one row of the block per thread
template <bool STAGED, int KM>
__global__ __launch_bounds__(kFillThreads) void k_sel_fill(Dims dm, int nblk, const int32_t* __restrict__ idx,
                                                  const float* __restrict__ score,
                                                  const float* __restrict__ lse_tot,
                                                  const float* __restrict__ ws_D,
                                                  const int* __restrict__ off,
                                                  int4* __restrict__ srec) {
  extern __shared__ __align__(16) uint32_t lfill[];
  const int NC = dm.Tkv / dm.S;
  constexpr int W = kLBlk / 32;
  static_assert(W % 4 == 0, "bitmap rows are read 16 bytes at a time");
  static_assert(kLBlk <= 512, "positions are packed in 9 bits");
  uint32_t* lb = lfill;                                   // [NC][W] bitmap of the block
  int* lo = reinterpret_cast<int*>(lfill + (size_t)NC * W);  // [NC] entry offsets
  int* lofl = lo + NC;                                    // STAGED: [NC] block-local offsets
  uint32_t* stage = reinterpret_cast<uint32_t*>(lofl + NC);  // STAGED: [kLBlk * K] entries
  float* salpha = reinterpret_cast<float*>(stage + kLBlk * dm.K);  // STAGED: their alpha
  float* sdr = salpha + kLBlk * dm.K;                     // STAGED: [kLBlk] each row's D
  constexpr int kWv = kFillThreads / 64;
  __shared__ int wtot[kWv];
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const long long bh = (long long)b * dm.H + h;
  for (int x = threadIdx.x; x < NC * W; x += blockDim.x) lb[x] = 0u;
  for (int c = threadIdx.x; c < NC; c += blockDim.x) lo[c] = off[(bh * NC + c) * nblk + blk];
  __syncthreads();
  const int i0 = blk * kLBlk, ni = min(kLBlk, dm.Tq - i0);
  // one thread per row: its entries in order, so entry_counts sees the earlier ids
  for (int ii = threadIdx.x; ii < ni; ii += blockDim.x) {
    const int i = i0 + ii;
    const int n = min(dm.ncand(dm.q_pos0 + i), NC);
    int cv[KM];
    load_row_ids<KM>(idx + (((long long)b * dm.Tq + i) * dm.H + h) * dm.K, dm.K, cv);
    int seen = -1;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (k < dm.K && entry_counts(cv[k], n, seen))
        atomicOr(&lb[cv[k] * W + ii / 32], 1u << (ii % 32));
      seen = max(seen, cv[k]);
    }
  }
  __syncthreads();
  int total = 0;
  if constexpr (STAGED) {
    // block-local entries per chunk (bitmap popcounts), exclusive scan in chunk order
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int seg = (NC + kFillThreads - 1) / kFillThreads;
    const int c0 = min(NC, t * seg), c1 = min(NC, c0 + seg);
    int sum = 0;
    for (int c = c0; c < c1; ++c) {
      int cn = 0;
#pragma unroll
      for (int ww = 0; ww < W; ++ww) cn += __popc(lb[c * W + ww]);
      lofl[c] = cn;
      sum += cn;
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wtot[w] = incl;
    __syncthreads();
    int run = incl - sum;
#pragma unroll
    for (int x = 0; x < kWv; ++x) {
      run += x < w ? wtot[x] : 0;
      total += wtot[x];
    }
    for (int c = c0; c < c1; ++c) {
      const int v = lofl[c];
      lofl[c] = run;
      run += v;
    }
    __syncthreads();
  }
  const long long ebase = bh * (long long)dm.Tq * dm.K;
  for (int ii = threadIdx.x; ii < ni; ii += blockDim.x) {
    const int i = i0 + ii;
    const long long r = ((long long)b * dm.Tq + i) * dm.H + h;
    const int n = min(dm.ncand(dm.q_pos0 + i), NC);
    const int wd = ii / 32;
    // the row's entries, scores, Lambda and D, all reads in flight together
    int cv[KM];
    float sv[KM];
    load_row_ids<KM>(idx + r * dm.K, dm.K, cv);
#pragma unroll
    for (int k = 0; k < KM; ++k) sv[k] = score[r * dm.K + min(k, dm.K - 1)];
    const float lt = lse_tot[r], dr = ws_D[r];
    if constexpr (STAGED) sdr[ii] = dr;
    int seen = -1;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      const int c = cv[k];
      const bool ok = k < dm.K && entry_counts(c, n, seen);
      seen = max(seen, c);
      if (!ok) continue;
      // the chunk's bitmap row in four 16-byte reads (all in flight), then the
      // selected positions before ii counted in registers
      const uint4* row4 = reinterpret_cast<const uint4*>(lb + c * W);
      uint32_t wv[W];
#pragma unroll
      for (int q = 0; q < W / 4; ++q) {
        const uint4 u = row4[q];
        wv[4 * q] = u.x, wv[4 * q + 1] = u.y, wv[4 * q + 2] = u.z, wv[4 * q + 3] = u.w;
      }
      int rank = 0;
#pragma unroll
      for (int ww = 0; ww < W; ++ww)
        rank += ww < wd ? __popc(wv[ww]) : (ww == wd ? __popc(wv[ww] & ((1u << (ii % 32)) - 1u)) : 0);
      const float alpha = expf(sv[k] - lt);
      if constexpr (STAGED) {
        stage[lofl[c] + rank] = (uint32_t)ii | ((uint32_t)k << 9) | ((uint32_t)c << 15);
        salpha[lofl[c] + rank] = alpha;
      } else {
        // one 16-byte record: position, alpha, D, slot
        srec[ebase + lo[c] + rank] = make_int4(i, __float_as_int(alpha), __float_as_int(dr), k);
      }
    }
  }
  if constexpr (STAGED) {
    __syncthreads();
    for (int e = threadIdx.x; e < total; e += blockDim.x) {
      const uint32_t v = stage[e];
      const int ii = (int)(v & 511u), k = (int)((v >> 9) & 63u), c = (int)(v >> 15);
      srec[ebase + lo[c] + (e - lofl[c])] =
          make_int4(i0 + ii, __float_as_int(salpha[e]), __float_as_int(sdr[ii]), k);
    }
  }
}

// ------------------------------------------------------------------ key-side order
// Launch order of the key side's workgroups, index L = (c B + b) Hkv + g: by
// their 32-row tiles (the chunk's own rows and its selecting rows, over the G
// heads), in buckets of log2 of the tile count, the largest bucket first. One
// workgroup; the order within a bucket is free (every workgroup writes only its
// own outputs, so the results do not depend on it).
constexpr int kOrderThreads = 1024;
__global__ __launch_bounds__(kOrderThreads) void k_bwd_order(Dims dm, const int* __restrict__ llen,
                                                            int* __restrict__ order) {
  __shared__ int hist[16], fill[16];
  const int NC = dm.Tkv / dm.S;
  const int n = NC * dm.Hkv * dm.B;
  const int t = threadIdx.x;
  if (t < 16) hist[t] = fill[t] = 0;
  __syncthreads();
  auto bucket = [&](int L) {
    const int g = L % dm.Hkv, b = (L / dm.Hkv) % dm.B, c = L / (dm.Hkv * dm.B);
    int rows = 0;
    for (int hh = 0; hh < dm.G; ++hh)
      rows += kChunk + llen[((long long)b * dm.H + (long long)g * dm.G + hh) * NC + c];
    const int tiles = (rows + 31) / 32;
    return min(15, 31 - __clz(max(tiles, 1)));
  };
  for (int L = t; L < n; L += kOrderThreads) atomicAdd(&hist[bucket(L)], 1);
  __syncthreads();
  for (int L = t; L < n; L += kOrderThreads) {
    const int bk = bucket(L);
    int start = 0;
    for (int x = bk + 1; x < 16; ++x) start += hist[x];
    order[start + atomicAdd(&fill[bk], 1)] = L;
  }
}

// ------------------------------------------------------------------ key side
// One workgroup per (chunk, kv head, batch) with four wavefronts. The chunk's
// own 64 rows (two 32-row tiles) followed by the rows that selected it
// (ascending) form a list of 32-row tiles; wavefront w takes tiles w, w + 4, ...
// and keeps dK, dV for all 64 keys x 64 features in registers; the four partial
// sums are added in a fixed order at the end. A tile's Q and dO rows and its
// weights go to wavefront-private LDS in natural row-major order and come back
// as MFMA operands with k along the rows through the LDS transpose read; the
// next tile's rows are loaded while the current one is computed.
constexpr int kKThreads = 256;
constexpr int kKWaves = kKThreads / 64;
constexpr int kTileRows = 32;
constexpr int TP = D + 8;       // LDS row pitch of 64-wide bf16 tiles
constexpr int TPD = D + 16;     // dS tile: keys, then ds^ in column D, zeros up to D + 15
// a list segment: the own rows (first segment) plus up to 2048 selecting rows
constexpr int kListMax = kChunk + 64 * 32;

typedef short v4s __attribute__((ext_vector_type(4)));
// 16 bytes as a native vector, so that copies of a tile's rows stay in registers
// (copies of HIP's uint4, a struct, went through scratch memory here)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// LDS transpose read (ds_read_b64_tr_b16): in each group of 16 lanes, lane
// 4j + a gives the address of four consecutive 16-bit elements and lane 4a + b
// receives element b of lanes 4j + a, j = 0..3.
__device__ __forceinline__ uint2 lds_tr16(const uint16_t* p) {
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
  uint2 u;
  __builtin_memcpy(&u, &r, 8);
  return u;
}
// MFMA operand with k along the rows of a [32][P] row-major LDS tile: lane
// (c, g) gets m[8g + j][n0 + c], j = 0..7 (k-slot 8g + j = row 8g + j).
template <int P>
__device__ __forceinline__ uint4 lds_kfrag(const uint16_t* m, int n0) {
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
  const uint16_t* p = m + (8 * g + (c >> 2)) * P + n0 + 4 * (c & 3);
  const uint2 lo = lds_tr16(p), hi = lds_tr16(p + 4 * P);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
// four floats to bf16, round to nearest even (packed hardware conversion)
// A operand K^T of a product whose k dimension is the chunk's keys in the
// lane-held order (k-slot 8g + j of step ks = key 32 ks + 4g + j for j < 4,
// 32 ks + 16 + 4g + j - 4 otherwise), from the row-major key tile kc: lane
// (c, g) gets kc[key][n0 + c].
__device__ __forceinline__ uint4 lds_ktfrag(const uint16_t* kc, int ks, int n0) {
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
  const uint16_t* p = kc + (32 * ks + 4 * g + (c >> 2)) * TP + n0 + 4 * (c & 3);
  const uint2 lo = lds_tr16(p), hi = lds_tr16(p + 16 * TP);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}
__device__ __forceinline__ uint2 pack4_bf16(const floatx4& v) {
  const bf16x4 h = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  uint2 u;
  __builtin_memcpy(&u, &h, 8);
  return u;
}

struct KWave {
  uint16_t qs[kTileRows][TP];   // Q rows of the tile
  uint16_t os[kTileRows][TP];   // dO rows of the tile
  uint16_t as[kTileRows][TP];   // value weights [row][key]
  uint16_t dsm[kTileRows][TPD]; // dS [row][key], ds^ of the row in column D
  uint16_t ss[kTileRows][TP];   // scoring-query (Q-Cal) rows of the tile
};
struct KSmem {
  KWave wv[kKWaves];
  uint16_t kc[kChunk][TP];  // the chunk's keys
  int rows[kListMax];       // list segment: position of the row
  float aux[kListMax];      // local rows: D; selecting rows: alpha
  float dvl[kListMax];      // local rows: Lambda; selecting rows: D
  int slotv[kListMax];      // dQ partial slot: selection slot, or K + local chunk
                            // index for local rows; -1 for padding entries
  float dkb[kKWaves][D];    // per-wave dk' partials, then the total
  float dql[kKWaves][D];
  float dbw[kKWaves];
  float qlv[D], kbv[D];
  float sp[kChunk];         // p'_j
  float sdp[kChunk];        // ds'_j
};
static_assert(sizeof(KSmem) <= 160 * 1024, "key-side LDS");
static_assert(sizeof(KWave) >= kChunk * D * sizeof(float), "final reduction buffer");

// A tile's rows are read 8 lanes to a row (one 128-byte line each), so every
// quarter-wave touches two lines; they reach the MFMA operand layout through LDS.
struct KTile {
  u32x4 qc[4], oc[4];  // Q / dO of tile rows 8 i + lane / 8, features 8 (lane % 8) .. + 8
  u32x4 sc[4];         // the scoring query's rows (Q-Cal; zero for own rows)
  float aux[2], dvr[2];
  int rpos[2];   // position of the row, -1 beyond the tile's rows
  int slot[2];
};

template <bool QCAL>
__global__ __launch_bounds__(kKThreads) void k_bwd_kv_mfma(
    Dims dm, const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Qs,
    float* __restrict__ ws_dsh, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ Ql,
    const float* __restrict__ ksum, const float* __restrict__ ent,
    const float* __restrict__ lse_l, const float* __restrict__ lse_tot,
    const uint16_t* __restrict__ dO, const float* __restrict__ ws_D,
    const int* __restrict__ lstart, const int* __restrict__ llen, const int4* __restrict__ srec,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, uint16_t* __restrict__ dQl,
    uint16_t* __restrict__ part, const int* __restrict__ order) {
  extern __shared__ __align__(16) char smem_raw[];
  KSmem& sm = *reinterpret_cast<KSmem*>(smem_raw);
  // the (chunk, kv head, b) of this workgroup, the ones with the most rows first
  // (k_bwd_order): a chunk that most rows selected would otherwise run alone at
  // the end
  const int NC = dm.Tkv / dm.S, G = dm.G;
  const int L = order[blockIdx.x];
  const int g = L % dm.Hkv, b = (L / dm.Hkv) % dm.B, c = L / (dm.Hkv * dm.B);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, col = lane & 15, gl = lane >> 4;
  const float scale2 = dm.scale * kLog2e;
  const float inv_scale = 1.0f / dm.scale;
  const long long kv_stride = (long long)dm.Hkv * D;
  const long long kv_base = ((long long)b * dm.Tcap * dm.Hkv + g) * D;
  const long long key0 = (long long)c * kChunk;
  KWave& wv = sm.wv[w];

  // the chunk's K and V rows as MFMA A fragments, and K in LDS
  uint4 kf[KF], vf[KF];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      const long long off = kv_base + (key0 + 16 * kb + col) * kv_stride + 32 * ds + 8 * gl;
      kf[kb * 2 + ds] = *reinterpret_cast<const uint4*>(K + off);
      vf[kb * 2 + ds] = *reinterpret_cast<const uint4*>(V + off);
    }
  for (int x = t; x < kChunk * D / 8; x += kKThreads) {
    const int j = x / (D / 8), c8 = x % (D / 8);
    *reinterpret_cast<uint4*>(&sm.kc[j][c8 * 8]) =
        *reinterpret_cast<const uint4*>(K + kv_base + (key0 + j) * kv_stride + c8 * 8);
  }
  // columns D + 1 .. D + 15 of the dS tiles stay zero
  for (int x = lane; x < kTileRows * 15; x += kLanes) wv.dsm[x / 15][D + 1 + x % 15] = 0;
  // dK / scale and dV: block [kb][fb] holds keys 16 kb + 4 gl + r x features 16 fb + col
  floatx4 dka[4][4], dva[4][4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) dka[kb][fb] = dva[kb][fb] = floatx4{0.f, 0.f, 0.f, 0.f};

  long long row_base = 0;  // row index of position 0 of the current head
  const long long discard_row = (long long)dm.B * dm.Tq * dm.H * (dm.K + dm.nlocal_max());
  auto load_tile = [&](int e0, int nr, bool own_rows) {
    KTile T;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + min(8 * i + (lane >> 3), nr - 1);
      const long long r = row_base + (long long)sm.rows[e] * dm.H;
      const long long off = r * D + 8 * (lane & 7);
      T.qc[i] = *reinterpret_cast<const u32x4*>(Q + off);
      T.oc[i] = *reinterpret_cast<const u32x4*>(dO + off);
      if constexpr (QCAL)
        T.sc[i] = own_rows ? u32x4{0, 0, 0, 0} : *reinterpret_cast<const u32x4*>(Qs + off);
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const bool v = 16 * hf + col < nr;
      const int e = e0 + min(16 * hf + col, nr - 1);
      const int pos = sm.rows[e];
      T.aux[hf] = v ? sm.aux[e] : 0.f;
      T.dvr[hf] = sm.dvl[e];
      T.slot[hf] = sm.slotv[e];
      T.rpos[hf] = v && T.slot[hf] >= 0 ? pos : -1;
    }
    return T;
  };

  // one 32-row tile; rows beyond nr get zero weights (their Q / dO are a valid row's)
  // own_rows is a compile-time constant (std::true_type / std::false_type), so
  // that the selecting rows' tiles, nearly all of them, are one branch-free body
  auto compute_tile = [&](const KTile& T, auto own_c, floatx4 (&dkq)[4], float& dbp) {
    constexpr bool own_rows = decltype(own_c)::value;
    // the tile's rows to LDS (the scoring query's only for dk'), then the B
    // operands Q / dO of rows 16 hf + c, features 32 ds + 8g .. back from there
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 8 * i + (lane >> 3), c8 = 8 * (lane & 7);
      *reinterpret_cast<u32x4*>(&wv.qs[rr][c8]) = T.qc[i];
      *reinterpret_cast<u32x4*>(&wv.os[rr][c8]) = T.oc[i];
      if constexpr (QCAL)
        if (!own_rows) *reinterpret_cast<u32x4*>(&wv.ss[rr][c8]) = T.sc[i];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      uint4 qf[2], of[2];
#pragma unroll
      for (int ds = 0; ds < 2; ++ds) {
        qf[ds] = *reinterpret_cast<const uint4*>(&wv.qs[16 * hf + col][32 * ds + 8 * gl]);
        of[ds] = *reinterpret_cast<const uint4*>(&wv.os[16 * hf + col][32 * ds + 8 * gl]);
      }
      floatx4 s[4], u[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = u[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < 2; ++ds) {
          s[kb] = mfma(kf[kb * 2 + ds], qf[ds], s[kb]);
          u[kb] = mfma(vf[kb * 2 + ds], of[ds], u[kb]);
        }
      }
      floatx4 a[4], d[4];
      float dsh = 0.f;
      if constexpr (own_rows) {
        // w_j = exp(s_j - Lambda) over the row's local keys lstart .. position
        const float lam2 = T.dvr[hf] * kLog2e, Dr = T.aux[hf];
        const int klo = (int)dm.lstart(max(T.rpos[hf], 0));
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kp = (int)key0 + 16 * kb + 4 * gl + r;
            const float wj = kp <= T.rpos[hf] && kp >= klo
                                 ? __builtin_amdgcn_exp2f(fmaf(s[kb][r], scale2, -lam2)) : 0.f;
            a[kb][r] = wj;
            d[kb][r] = wj * (u[kb][r] - Dr);
          }
      } else {
        float m = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          m = fmaxf(m, fmaxf(fmaxf(s[kb][0], s[kb][1]), fmaxf(s[kb][2], s[kb][3])));
        m = xmax_16_32(m) * scale2;  // scale2 > 0
        float z = 0.f, zu = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            s[kb][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], scale2, -m));
            z += s[kb][r];
            zu = fmaf(s[kb][r], u[kb][r], zu);
          }
        z = xsum_16_32(z);
        zu = xsum_16_32(zu);
        const float iz = 1.0f / z, rc = zu * iz, al = T.aux[hf], cf = al * iz;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = cf * s[kb][r];
            a[kb][r] = p;
            d[kb][r] = p * (u[kb][r] - rc);
          }
        // ds^ = alpha (r - D) of the row: db' here, dk' through the dS tile
        dsh = al * (rc - T.dvr[hf]);
        dbp += dsh;
        if constexpr (QCAL) {
          if (gl == 0 && T.rpos[hf] >= 0)
            ws_dsh[(row_base + (long long)T.rpos[hf] * dm.H) * dm.K + T.slot[hf]] = dsh;
        }
      }
      if (gl == 0) wv.dsm[16 * hf + col][D] = __builtin_bit_cast(uint16_t, (__bf16)dsh);
      uint2 dpk[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        dpk[kb] = pack4_bf16(d[kb]);
        *reinterpret_cast<uint2*>(&wv.as[16 * hf + col][16 * kb + 4 * gl]) = pack4_bf16(a[kb]);
        *reinterpret_cast<uint2*>(&wv.dsm[16 * hf + col][16 * kb + 4 * gl]) = dpk[kb];
      }
      // dQ^T / scale of the row from this chunk: K^T dS^T (+ ds^ k' for a
      // selecting row), to the row's partial slot (lane: features 16 db + 4 gl + r)
      const uint4 pf[2] = {make_uint4(dpk[0].x, dpk[0].y, dpk[1].x, dpk[1].y),
                           make_uint4(dpk[2].x, dpk[2].y, dpk[3].x, dpk[3].y)};
      // a padding row (rpos < 0) stores to the discard row past the partials, so
      // the stores need no branch
      const long long prow =
          T.rpos[hf] >= 0
              ? (row_base + (long long)T.rpos[hf] * dm.H) * (dm.K + dm.nlocal_max()) + T.slot[hf]
              : discard_row;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        floatx4 dq = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) dq = mfma(lds_ktfrag(&sm.kc[0][0], ks, 16 * db), pf[ks], dq);
        if constexpr (!QCAL) {
          // unconditional (a local row has ds^ = 0, and 0 k' + dq = dq exactly), so
          // the read needs no branch and wait of its own
          const float4 kb4 = *reinterpret_cast<const float4*>(&sm.kbv[16 * db + 4 * gl]);
          dq[0] = fmaf(dsh, kb4.x, dq[0]);
          dq[1] = fmaf(dsh, kb4.y, dq[1]);
          dq[2] = fmaf(dsh, kb4.z, dq[2]);
          dq[3] = fmaf(dsh, kb4.w, dq[3]);
        }
        *reinterpret_cast<uint2*>(part + prow * D + 16 * db + 4 * gl) = pack4_bf16(dq);
      }
    }
    __builtin_amdgcn_wave_barrier();
    // dV += A^T dO, dK += dS^T Q over the tile's 32 rows (k dimension = rows)
    uint4 obf[4], qbf[4];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      obf[fb] = lds_kfrag<TP>(&wv.os[0][0], 16 * fb);
      qbf[fb] = lds_kfrag<TP>(&wv.qs[0][0], 16 * fb);
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint4 af = lds_kfrag<TP>(&wv.as[0][0], 16 * kb);
      const uint4 df = lds_kfrag<TPD>(&wv.dsm[0][0], 16 * kb);
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        dva[kb][fb] = mfma(af, obf[fb], dva[kb][fb]);
        dka[kb][fb] = mfma(df, qbf[fb], dka[kb][fb]);
      }
    }
    // dk' / scale += sum over the rows of ds^ q, or of ds^ times the scoring
    // query with Q-Cal (row 0 of this product)
    {
      const uint4 hf5 = lds_kfrag<TPD>(&wv.dsm[0][0], D);
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        // own rows have ds^ = 0: their scoring-query rows are not loaded
        const uint4 qb = QCAL && !own_rows ? lds_kfrag<TP>(&wv.ss[0][0], 16 * fb) : qbf[fb];
        dkq[fb] = mfma(hf5, qb, dkq[fb]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    row_base = (long long)b * dm.Tq * dm.H + h;
    // dk' / scale (lane (col, 0) element 0 of block fb: feature 16 fb + col)
    // and the lane's partial sum of db'
    floatx4 dkq[4];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) dkq[fb] = floatx4{0.f, 0.f, 0.f, 0.f};
    float dbp = 0.f;
    const long long bh = (long long)b * dm.H + h;
    const long long sidx = ((long long)b * dm.NCcap + c) * dm.H + h;
    // the summary backward's per-(chunk, head) inputs, read while the tiles run
    const float lp_h = lse_l[sidx], ent_h = ent[sidx];
    const int LN = llen[bh * NC + c];
    const long long lsrc = bh * (long long)dm.Tq * dm.K + lstart[bh * NC + c];
    // local rows: positions key0 .. key0 + span - 1 (span = S, or S + W - 1 with a
    // window), padded to whole tiles with entries of slot -1
    const int nown = (int)min((long long)(dm.window > 0 ? kChunk + dm.window - 1 : kChunk),
                              (long long)dm.Tq - key0);
    const int nown_pad = (nown + kTileRows - 1) / kTileRows * kTileRows;
    const int kSeg = kListMax - nown_pad;  // > 0: the plan bounds the window
    for (int s0 = 0;; s0 += kSeg) {
      // list segment: the local rows first (first segment only), then
      // selecting rows s0 .. s0 + kSeg of the chunk's list
      const int base = s0 == 0 ? nown_pad : 0;
      const int ns = min(kSeg, LN - s0);
      const int n = base + ns;
      if (s0 == 0 && t < D) {
        sm.kbv[t] = ksum[sidx * D + t];
        sm.qlv[t] = bf(Ql[sidx * D + t]);  // for the summary backward after the tiles
      }
      // the segment's rows into LDS: a round of reads (kSegU per thread for the
      // local rows, kSegR for the selecting rows' records) is issued before any
      // of it is stored, so a segment takes one or two memory round trips
      constexpr int kSegU = 3, kSegR = 8;
      for (int e0 = t; e0 < base; e0 += kKThreads * kSegU) {
        int pp[kSegU];
        float dr[kSegU], lt[kSegU];
#pragma unroll
        for (int u = 0; u < kSegU; ++u) {
          const long long pos = key0 + min(min(e0 + u * kKThreads, base - 1), nown - 1);
          const long long r = row_base + pos * dm.H;
          pp[u] = (int)pos;
          dr[u] = ws_D[r];
          lt[u] = lse_tot[r];
        }
#pragma unroll
        for (int u = 0; u < kSegU; ++u) {
          const int e = e0 + u * kKThreads;
          if (e < base) {
            sm.rows[e] = pp[u];
            sm.aux[e] = dr[u];
            sm.dvl[e] = lt[u];
            sm.slotv[e] = e < nown ? dm.K + (c - (int)(dm.lstart(pp[u]) / kChunk)) : -1;
          }
        }
      }
      for (int e0 = t; e0 < ns; e0 += kKThreads * kSegR) {
        int4 rec[kSegR];
#pragma unroll
        for (int u = 0; u < kSegR; ++u) rec[u] = srec[lsrc + s0 + min(e0 + u * kKThreads, ns - 1)];
#pragma unroll
        for (int u = 0; u < kSegR; ++u) {
          const int e = e0 + u * kKThreads;
          if (e < ns) {
            sm.rows[base + e] = rec[u].x;
            sm.aux[base + e] = __int_as_float(rec[u].y);
            sm.dvl[base + e] = __int_as_float(rec[u].z);
            sm.slotv[base + e] = rec[u].w;
          }
        }
      }
      __syncthreads();
      int e0 = kTileRows * w;
      if (e0 < n) {
        KTile cur = load_tile(e0, min(kTileRows, n - e0), e0 < base);
        for (;;) {
          const int e1 = e0 + kTileRows * kKWaves;
          const bool more = e1 < n;
          const int ep = more ? e1 : e0;
          const KTile nxt = load_tile(ep, min(kTileRows, n - ep), ep < base);
          if (e0 < base) compute_tile(cur, std::true_type{}, dkq, dbp);
          else compute_tile(cur, std::false_type{}, dkq, dbp);
          if (!more) break;
          cur = nxt;
          e0 = e1;
        }
      }
      __syncthreads();
      if (s0 + kSeg >= LN) break;
    }

    // ---- summary and landmark backward of (chunk c, head h)
    // db': sum over the 16 rows (lanes col) of a lane group
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) dbp += __shfl_xor(dbp, o, kLanes);
    if (gl == 0) {
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) sm.dkb[w][16 * fb + col] = dkq[fb][0];
    }
    if (lane == 0) sm.dbw[w] = dbp;
    __syncthreads();
    if (t < D)  // fixed order over the wavefronts
      sm.dkb[0][t] = (((sm.dkb[0][t] + sm.dkb[1][t]) + sm.dkb[2][t]) + sm.dkb[3][t]) * dm.scale;
    __syncthreads();
    if (w == 0) {  // lane j: key j of the chunk
      float s1 = 0.f, t1 = 0.f;
#pragma unroll
      for (int e8 = 0; e8 < D / 8; ++e8) {
        const uint4 kv = *reinterpret_cast<const uint4*>(&sm.kc[lane][8 * e8]);
        const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = 8 * e8 + 2 * q;
          const float k0v = __uint_as_float(kw[q] << 16), k1v = __uint_as_float(kw[q] & 0xFFFF0000u);
          s1 = fmaf(sm.qlv[e], k0v, fmaf(sm.qlv[e + 1], k1v, s1));
          t1 = fmaf(sm.dkb[0][e], k0v - sm.kbv[e], fmaf(sm.dkb[0][e + 1], k1v - sm.kbv[e + 1], t1));
        }
      }
      s1 *= dm.scale;
      const float Lp = lp_h, bias = ent_h;
      const float dbv = ((sm.dbw[0] + sm.dbw[1]) + sm.dbw[2]) + sm.dbw[3];
      const float p1 = expf(s1 - Lp);
      sm.sp[lane] = p1;
      sm.sdp[lane] = p1 * (t1 + dbv * (Lp - s1 - bias));
    }
    __syncthreads();
    {  // dQl = scale sum_j ds'_j k_j: wave w sums keys 16 w .. 16 w + 15
      float acc = 0.f;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) acc = fmaf(sm.sdp[16 * w + jj], bf(sm.kc[16 * w + jj][lane]), acc);
      sm.dql[w][lane] = acc;
    }
    __syncthreads();
    if (t < D)
      dQl[sidx * D + t] = f32_to_bf16_bits(
          (((sm.dql[0][t] + sm.dql[1][t]) + sm.dql[2][t]) + sm.dql[3][t]) * dm.scale);
    // dK_j += p'_j dk' + scale ds'_j Ql: added once, by wavefront 0's accumulators
    if (w == 0) {
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        const float dk_e = sm.dkb[0][16 * fb + col];
        const float ql_e = sm.qlv[16 * fb + col];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 16 * kb + 4 * gl + r;
            dka[kb][fb][r] += sm.sp[j] * dk_e * inv_scale + sm.sdp[j] * ql_e;
          }
      }
    }
    __syncthreads();
  }

  // ---- dK = scale * (sum of the wavefronts' accumulators), dV; each wavefront
  // writes its partial sums to its own LDS region, then a fixed-order sum
  float* red = reinterpret_cast<float*>(&sm.wv[w]);  // [64 keys][64 features]
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          red[(16 * kb + 4 * gl + r) * D + 16 * fb + col] = pass == 0 ? dka[kb][fb][r] : dva[kb][fb][r];
    __syncthreads();
    const float* r0 = reinterpret_cast<const float*>(&sm.wv[0]);
    const float* r1 = reinterpret_cast<const float*>(&sm.wv[1]);
    const float* r2 = reinterpret_cast<const float*>(&sm.wv[2]);
    const float* r3 = reinterpret_cast<const float*>(&sm.wv[3]);
    uint16_t* out = pass == 0 ? dK : dV;
    const float sc = pass == 0 ? dm.scale : 1.0f;
    for (int x = t; x < kChunk * D / 4; x += kKThreads) {
      const int j = x / (D / 4), e = 4 * (x % (D / 4)), o = j * D + e;
      const float4 a0 = *reinterpret_cast<const float4*>(r0 + o);
      const float4 a1 = *reinterpret_cast<const float4*>(r1 + o);
      const float4 a2 = *reinterpret_cast<const float4*>(r2 + o);
      const float4 a3 = *reinterpret_cast<const float4*>(r3 + o);
      const floatx4 v = {(((a0.x + a1.x) + a2.x) + a3.x) * sc, (((a0.y + a1.y) + a2.y) + a3.y) * sc,
                         (((a0.z + a1.z) + a2.z) + a3.z) * sc, (((a0.w + a1.w) + a2.w) + a3.w) * sc};
      *reinterpret_cast<uint2*>(out + kv_base + (key0 + j) * kv_stride + e) = pack4_bf16(v);
    }
    __syncthreads();
  }
}

struct BPlan {
  int nct, nblk;
  bool staged;  // the list fill stages the block's records in LDS
  size_t cnt_bytes, ls_bytes, rec_bytes, part_bytes, order_bytes, fill_smem;
};

bool bwd_plan(const Dims& dm, BPlan* p) {
  if (!dm.bf16 || dm.d != 64 || dm.Tq < 64 || dm.q_pos0 != 0 || dm.Tq != dm.Tkv) return false;
  // the local rows of a chunk and at least one tile of selecting rows fit a list segment
  if (dm.window > 16 * kChunk) return false;
  p->nct = dm.Tkv / dm.S;
  p->nblk = (dm.Tq + kLBlk - 1) / kLBlk;
  const size_t rows = (size_t)dm.B * dm.Tq * dm.H;
  p->cnt_bytes = (size_t)dm.B * dm.H * p->nct * p->nblk * sizeof(int);
  p->ls_bytes = (size_t)dm.B * dm.H * p->nct * sizeof(int);
  p->order_bytes = (size_t)dm.B * dm.Hkv * p->nct * sizeof(int);
  p->rec_bytes = rows * dm.K * sizeof(int4);
  // the dQ partials, then one discard row that padding rows store to
  p->part_bytes = (rows * (dm.K + dm.nlocal_max()) + 1) * D * sizeof(uint16_t);
  p->fill_smem = (size_t)p->nct * (kLBlk / 32 + 1) * sizeof(int);
  const size_t staged = p->fill_smem + (size_t)p->nct * sizeof(int) +
                        (size_t)kLBlk * dm.K * (sizeof(uint32_t) + sizeof(float)) +
                        (size_t)kLBlk * sizeof(float);
  p->staged = staged <= 160 * 1024 && p->nct <= (1 << 17);  // chunk ids packed in 17 bits
  if (p->staged) p->fill_smem = staged;
  return p->fill_smem <= 160 * 1024;
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// The three list passes, with KM >= K register slots per row.
template <int KM>
hipError_t launch_lists(const Dims& dm, const BPlan& p, const int32_t* idx, const float* score,
                        const float* lse_tot, const float* ws_D, int* cnt, int* lstart, int* llen,
                        int4* srec, hipStream_t st) {
  hipLaunchKernelGGL(k_sel_count<KM>, dim3(p.nblk, dm.H, dm.B), dim3(256),
                     (size_t)p.nct * sizeof(int), st, dm, p.nblk, idx, cnt);
  hipLaunchKernelGGL(k_sel_scan, dim3(dm.H, dm.B), dim3(kScanThreads), 0, st, dm, p.nblk, cnt,
                     lstart, llen);
  const void* fk = p.staged ? reinterpret_cast<const void*>(k_sel_fill<true, KM>)
                            : reinterpret_cast<const void*>(k_sel_fill<false, KM>);
  hipError_t e = hipFuncSetAttribute(fk, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)p.fill_smem);
  if (e != hipSuccess) return e;
  if (p.staged)
    hipLaunchKernelGGL((k_sel_fill<true, KM>), dim3(p.nblk, dm.H, dm.B), dim3(kFillThreads),
                       p.fill_smem, st, dm, p.nblk, idx, score, lse_tot, ws_D, cnt, srec);
  else
    hipLaunchKernelGGL((k_sel_fill<false, KM>), dim3(p.nblk, dm.H, dm.B), dim3(kFillThreads),
                       p.fill_smem, st, dm, p.nblk, idx, score, lse_tot, ws_D, cnt, srec);
  return hipGetLastError();
}

}  // namespace

size_t backward_mfma_ws_bytes(const Dims& dm) {
  BPlan p;
  if (!bwd_plan(dm, &p)) return 0;
  return up256(p.cnt_bytes) + 2 * up256(p.ls_bytes) + up256(p.rec_bytes) + up256(p.part_bytes) +
         up256(p.order_bytes);
}

bool backward_mfma_try(const Dims& dm, const void* Q, const void* K, const void* V,
                       const void* Ql, const float* ksum, const float* ent, const float* lse_l,
                       const int32_t* idx, const float* score, const float* lse_tot,
                       const void* O, const void* dO, void* dQ, void* dK, void* dV, void* dQl,
                       const void* Qs, void* dQs, float* ws_D, float* ws_dsh, void* ws_mfma,
                       hipStream_t st, hipError_t* err) {
  BPlan p;
  if (!bwd_plan(dm, &p)) return false;
  char* base = reinterpret_cast<char*>(ws_mfma);
  int* cnt = reinterpret_cast<int*>(base);
  base += up256(p.cnt_bytes);
  int* lstart = reinterpret_cast<int*>(base);
  base += up256(p.ls_bytes);
  int* llen = reinterpret_cast<int*>(base);
  base += up256(p.ls_bytes);
  int4* srec = reinterpret_cast<int4*>(base);
  base += up256(p.rec_bytes);
  uint16_t* part = reinterpret_cast<uint16_t*>(base);
  base += up256(p.part_bytes);
  int* order = reinterpret_cast<int*>(base);
  const long long rows = (long long)dm.B * dm.Tq * dm.H;
  const unsigned rblocks = (unsigned)((rows + 31) / 32);
  const auto* dOh = reinterpret_cast<const uint16_t*>(dO);
  hipLaunchKernelGGL(k_bwd_rowd, dim3(rblocks), dim3(256), 0, st, rows,
                     reinterpret_cast<const uint16_t*>(O), dOh, ws_D);
  hipError_t e = dm.K <= 16 ? launch_lists<16>(dm, p, idx, score, lse_tot, ws_D, cnt, lstart,
                                                llen, srec, st)
                 : dm.K <= 32 ? launch_lists<32>(dm, p, idx, score, lse_tot, ws_D, cnt, lstart,
                                                 llen, srec, st)
                              : launch_lists<64>(dm, p, idx, score, lse_tot, ws_D, cnt, lstart,
                                                 llen, srec, st);
  if (e != hipSuccess) {
    *err = e;
    return true;
  }
  hipLaunchKernelGGL(k_bwd_order, dim3(1), dim3(kOrderThreads), 0, st, dm, llen, order);
  const bool qcal = Qs != nullptr;
  const void* kvk = qcal ? reinterpret_cast<const void*>(k_bwd_kv_mfma<true>)
                         : reinterpret_cast<const void*>(k_bwd_kv_mfma<false>);
  e = hipFuncSetAttribute(kvk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(KSmem));
  if (e != hipSuccess) {
    *err = e;
    return true;
  }
  const auto* Qh = reinterpret_cast<const uint16_t*>(Q);
  const auto* Qsh = qcal ? reinterpret_cast<const uint16_t*>(Qs) : Qh;
#define HILS_KV(QC)                                                                                 \
  hipLaunchKernelGGL(k_bwd_kv_mfma<QC>, dim3(p.nct * dm.Hkv * dm.B), dim3(kKThreads), sizeof(KSmem), \
                     st, dm, Qh, Qsh, ws_dsh, reinterpret_cast<const uint16_t*>(K),                 \
                     reinterpret_cast<const uint16_t*>(V), reinterpret_cast<const uint16_t*>(Ql),   \
                     ksum, ent, lse_l, lse_tot, dOh, ws_D, lstart, llen, srec,                      \
                     reinterpret_cast<uint16_t*>(dK), reinterpret_cast<uint16_t*>(dV),              \
                     reinterpret_cast<uint16_t*>(dQl), part, order)
  if (qcal) HILS_KV(true); else HILS_KV(false);
#undef HILS_KV
  auto* dQh = reinterpret_cast<uint16_t*>(dQ);
  auto* dQsh = reinterpret_cast<uint16_t*>(dQs);
#define HILS_DQ(KM, QC)                                                                          \
  hipLaunchKernelGGL((k_dq_reduce<KM, QC>), dim3(rblocks), dim3(256), 0, st, dm, rows, idx, part, \
                     dQh, ws_dsh, ksum, dQsh)
  if (dm.K + 1 <= 17) {
    if (qcal) HILS_DQ(17, true); else HILS_DQ(17, false);
  } else {
    if (qcal) HILS_DQ(13, true); else HILS_DQ(13, false);
  }
#undef HILS_DQ
  *err = hipGetLastError();
  return true;
}

}  // namespace hils
