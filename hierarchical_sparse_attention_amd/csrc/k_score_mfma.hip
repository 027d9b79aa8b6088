// Chunk scoring and top-K selection on bf16 MFMA (note §5.2: s^_{i,c} =
// q_i.k'_c/sqrt(d) + b'_c, I_i = {c in C_i : rank_desc(s^_{i,c}) < K}).
//
// The summary key k'_c is float32. With q exactly bf16, the dot product is
// computed on matrix cores from a two-term split k' = hi + lo (hi = bf16(k'),
// lo = bf16(k' - hi)): every product q_e * hi_e and q_e * lo_e is exact in
// float32, the MFMA accumulates in float32, and the dropped remainder is below
// 2^-17 |k'_e|, so the score matches a float32 dot product to rounding level.
//
// All bf16 paths (prefill tiles and decode splits) run the same MFMA sequence per
// (row, chunk) element: acc = sum over 32-wide feature steps of q.hi then q.lo,
// then s = acc * scale + ent. An element of an MFMA result depends only on its
// own row of A and column of B, so every path yields bit-identical scores and
// therefore identical selections.
//
// Prefill: one wavefront owns 64 query rows of one head. Candidates are scored
// 64 (d = 128: 32) at a time into LDS (16 x 16 MFMA blocks, rows on M, chunks on
// N); then each lane takes one row and keeps its running top list in registers:
// in groups of 16 candidates, a compare against the list's last score marks the
// few that can enter, and those are inserted with a compare-exchange pass.
// Decode: candidates of a row are split over workgroups; each writes its local
// top-K (rank counting), and the union is ranked by the merge kernel shared with
// the float32 path or by the decode step's slot kernel itself.
#include "hils_internal.h"
#include "mfma_common.h"

namespace hils {
namespace {

constexpr int kSplitM = kSplitMfma;  // candidates per decode workgroup

using mf::as_bf16x8;
using mf::bf16x8;
using mf::floatx4;
using mf::score_block;
using mf::split8;

// Split copy of the summary keys in MFMA fragment order. Per (b, h) the chunks
// come in blocks of 16; block blk holds D/16 fragments of 64 lanes, fragment
// 2 ds + x of lane (c, g) being the hi (x = 0) or lo (x = 1) part of
// k'[16 blk + c][32 ds + 8 g .. + 8] (16 bytes). One fragment load of a
// wavefront is then 1 KiB of contiguous memory. Chunks at or beyond nc are zero.
template <int D>
__device__ __forceinline__ long long ks_frag(const Dims& dm, int nc, int b, int h, int blk) {
  return ((((long long)b * dm.H + h) * ((nc + 15) / 16) + blk) * (D / 16)) * 64;
}

template <int D>
__global__ __launch_bounds__(256) void k_ksplit(Dims dm, int nc, const float* __restrict__ ksum,
                                                uint4* __restrict__ ks) {
  const int nblk = (nc + 15) / 16;
  const long long n = (long long)dm.B * dm.H * nblk * (D / 16) * 64;
  for (long long x = blockIdx.x * 256LL + threadIdx.x; x < n; x += (long long)gridDim.x * 256) {
    const int lane = (int)(x & 63), i = (int)((x >> 6) % (D / 16));
    const long long bhb = (x >> 6) / (D / 16);
    const int blk = (int)(bhb % nblk);
    const long long bh = bhb / nblk;
    const int h = (int)(bh % dm.H), b = (int)(bh / dm.H);
    const int chunk = 16 * blk + (lane & 15), ds = i >> 1;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (chunk < nc) {
      const float* src = ksum + (((long long)b * dm.NCcap + chunk) * dm.H + h) * D + 32 * ds +
                         8 * (lane >> 4);
      const float4 a = *reinterpret_cast<const float4*>(src);
      const float4 bb = *reinterpret_cast<const float4*>(src + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = bb.x; v[5] = bb.y; v[6] = bb.z; v[7] = bb.w;
    }
    bf16x8 hi, lo;
    split8(v, hi, lo);
    uint4 w;
    __builtin_memcpy(&w, (i & 1) ? &lo : &hi, 16);
    ks[x] = w;
  }
}

// Running top-KM list of one row in registers, sorted by (score desc, chunk asc).
// Inserting is one pass with no dependency chain (no dynamic indexing): entry k
// becomes entry k-1 when the candidate beats entry k-1, else the candidate when
// it beats entry k, else stays; a candidate that beats nothing falls off the end.
// Candidates arrive in ascending chunk order and compare strictly, so equal
// scores keep the lower chunk first.
template <int KM>
struct TopList {
  float s[KM];
  int c[KM];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int k = 0; k < KM; ++k) { s[k] = -INFINITY; c[k] = 0x7fffffff; }
  }
  // x enters after every entry it does not beat (strictly greater goes first,
  // so an equal score from a later chunk stays behind). Updated in place from
  // the tail: slot k's new score is the median of x, s[k - 1] and s[k] (the list
  // is descending) and is written while s[k - 1] still holds its old value, so
  // no copy of the list is made; each comparison serves two neighbouring slots.
  __device__ __forceinline__ void insert(float x, int xc) {
    bool gk = x > s[KM - 1];
#pragma unroll
    for (int k = KM - 1; k > 0; --k) {
      const bool gp = x > s[k - 1];
      s[k] = __builtin_amdgcn_fmed3f(x, s[k - 1], s[k]);
      c[k] = gp ? c[k - 1] : (gk ? xc : c[k]);
      gk = gp;
    }
    s[0] = gk ? x : s[0];
    c[0] = gk ? xc : c[0];
  }
};

// Largest v (0 .. 16) over the wavefront, by a binary search on ballots
// (compares and scalar operations, no cross-lane data movement).
__device__ __forceinline__ int wave_max16(int v) {
  int m = 0;
#pragma unroll
  for (int bit = 16; bit > 0; bit >>= 1)
    if (__builtin_amdgcn_ballot_w64(v >= m + bit) != 0) m += bit;
  return m;
}

// Sorts 16 (score, chunk) pairs by (score desc, chunk asc) in registers with a
// bitonic network (80 compare-exchanges at fixed positions).
__device__ __forceinline__ void sort16(float* x, int* xc) {
#pragma unroll
  for (int k = 2; k <= 16; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int l = i ^ j;
        if (l > i) {
          // first = the one that belongs earlier in (score desc, chunk asc)
          const bool desc = (i & k) == 0;
          const bool lbefore = x[l] > x[i] || (x[l] == x[i] && xc[l] < xc[i]);
          const bool sw = desc ? lbefore : !lbefore;
          const float a = x[i], bb = x[l];
          const int ca = xc[i], cb = xc[l];
          x[i] = sw ? bb : a;
          x[l] = sw ? a : bb;
          xc[i] = sw ? cb : ca;
          xc[l] = sw ? ca : cb;
        }
      }
}

// d = 128 with a 16-entry list is held to 3 wavefronts per SIMD (it fits in 168
// registers; left alone the compiler takes 174 and only 2 fit).
template <int D, int KM>
__global__ __launch_bounds__(64, (D == 128 && KM == 16) ? 3 : 1) void k_score_mfma(
    Dims dm, int nc, const uint16_t* __restrict__ Q, const uint4* __restrict__ ks,
    const float* __restrict__ ent, int32_t* __restrict__ idx, float* __restrict__ score) {
  // candidates per block: 32 at d = 128 (a smaller LDS block lets more
  // wavefronts share a compute unit: 0.51 against 0.57 ms at the 7B shape), 64 at
  // d = 64 (where 32 measured 3% slower)
  constexpr int CB = D == 128 ? 32 : 64;
  __shared__ float sS[64][CB + 1];
  const int lane = threadIdx.x, c = lane & 15, g = lane >> 4;
  // 1-D grid, position blocks slowest and longest (latest) first
  const int nqb = (dm.Tq + 63) / 64, L = blockIdx.x;
  const int h = L % dm.H, b = (L / dm.H) % dm.B, K = dm.K;
  const int i0 = (nqb - 1 - L / (dm.H * dm.B)) * 64;
  const int nrows = min(64, dm.Tq - i0);
  const int my_n = lane < nrows ? dm.ncand(dm.q_pos0 + i0 + lane) : 0;
  const int nmax = dm.ncand(dm.q_pos0 + i0 + nrows - 1);

  // A fragments: rows 16mb + c, features 32ds + 8g .. +8
  uint4 qa[4][D / 32];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = 16 * mb + c;
    const bool v = m < nrows;
    const long long off = (((long long)b * dm.Tq + i0 + m) * dm.H + h) * D;
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
      qa[mb][ds] = v ? *reinterpret_cast<const uint4*>(Q + off + 32 * ds + 8 * g) : make_uint4(0, 0, 0, 0);
  }
  TopList<KM> top;
  top.init();
  for (int c0 = 0; c0 < nmax; c0 += CB) {
#pragma unroll
    for (int nb = 0; nb < CB / 16; ++nb) {
      // a column past the candidates reads block 0 (in bounds): its score is
      // never looked at, so the loads need no condition and stay in flight
      // together
      const int chunk = c0 + 16 * nb + c;
      const bool cv = chunk < nmax;
      bf16x8 hi[D / 32], lo[D / 32];
      const uint4* src = ks + ks_frag<D>(dm, nc, b, h, cv ? (c0 >> 4) + nb : 0) + lane;
#pragma unroll
      for (int ds = 0; ds < D / 32; ++ds) {
        hi[ds] = as_bf16x8(src[(2 * ds) * 64]);
        lo[ds] = as_bf16x8(src[(2 * ds + 1) * 64]);
      }
      const float e = ent[((long long)b * dm.NCcap + (cv ? chunk : 0)) * dm.H + h];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const floatx4 acc = score_block<D>(qa[mb], hi, lo);
#pragma unroll
        for (int r = 0; r < 4; ++r) sS[16 * mb + 4 * g + r][16 * nb + c] = fmaf(acc[r], dm.scale, e);
      }
    }
    __syncthreads();
    // lane = row. In sub-blocks of 16 candidates: mark the ones that beat the
    // row's current KM-th score, then insert them (all lanes step together).
    const int lim = min(CB, my_n - c0);
    int sb0 = 0;
    if (c0 == 0) {
      // the row's first 16 candidates fill its empty list in one sort
      float xs[16];
      int xc[16];
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const bool ok = jj < lim;
        xs[jj] = ok ? sS[lane][jj] : -INFINITY;
        xc[jj] = ok ? jj : 0x7fffffff;
      }
      sort16(xs, xc);
#pragma unroll
      for (int k = 0; k < 16 && k < KM; ++k) top.s[k] = xs[k], top.c[k] = xc[k];
      sb0 = 1;
    }
#pragma unroll 1
    for (int sb = sb0; sb < CB / 16; ++sb) {
      const float theta = top.s[KM - 1];
      // the 16 reads are unconditional and combined without short-circuit, so
      // they are all in flight together
      float xv[16];
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) xv[jj] = sS[lane][16 * sb + jj];
      uint32_t mask = 0;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj)
        mask |= ((16 * sb + jj < lim) & (xv[jj] > theta)) ? (1u << jj) : 0u;
      const int todo = wave_max16(__popc(mask));
      // each insert's candidate is read one insert ahead
      int jj = mask ? __ffs(mask) - 1 : 0;
      float x = sS[lane][16 * sb + jj];
      for (int p = 0; p < todo; ++p) {
        const bool have = mask != 0;
        const int cj = jj;
        mask &= mask - 1;
        jj = mask ? __ffs(mask) - 1 : 0;
        const float xn = sS[lane][16 * sb + jj];
        top.insert(have ? x : -INFINITY, c0 + 16 * sb + cj);
        x = xn;
      }
    }
    __syncthreads();
  }
  if (lane >= nrows) return;
  const int cnt = min(K, my_n);
  const long long o = (((long long)b * dm.Tq + i0 + lane) * dm.H + h) * K;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    int rank = 0;
#pragma unroll
    for (int k2 = 0; k2 < KM; ++k2) rank += (k2 < cnt && top.c[k2] < top.c[k]) ? 1 : 0;
    if (k < cnt) {
      idx[o + rank] = top.c[k];
      score[o + rank] = top.s[k];
    }
  }
  for (int k = cnt; k < K; ++k) {
    idx[o + k] = -1;
    score[o + k] = -INFINITY;
  }
}

// GQA group-max selection on matrix cores (note §5.4), G = 2 or 4. A workgroup
// of G wavefronts owns 64 positions of one kv head; wavefront hh scores them for
// query head gk G + hh exactly as the per-head kernel does (same blocks, same
// summary-key reuse) into its own LDS region. The G wavefronts then split the 64
// positions (64 / G each) and rank the candidates by the maximum over the G
// regions with the per-head kernel's register top-K. The selected chunks go to a
// per-position bitmask; a second pass scores the blocks again and every lane
// writes the scores of the (position, chunk) elements it holds whose bit is set.
template <int D, int KM, int G>
__global__ __launch_bounds__(64 * G) void k_score_mfma_group(Dims dm, int nc,
                                                             const uint16_t* __restrict__ Q,
                                                             const uint4* __restrict__ ks,
                                                             const float* __restrict__ ent,
                                                             int32_t* __restrict__ idx,
                                                             float* __restrict__ score) {
  constexpr int PS = 64 / G;  // positions each wavefront selects for
  static_assert(G == 2 || G == 4, "group size");
  extern __shared__ __align__(16) float gsm2[];
  const int t = threadIdx.x, lane = t & 63, hh = t >> 6, c = lane & 15, g = lane >> 4;
  const int nqb = (dm.Tq + 63) / 64, L = blockIdx.x;
  const int gk = L % dm.Hkv, b = (L / dm.Hkv) % dm.B, K = dm.K;
  const int h = gk * G + hh;
  const int i0 = (nqb - 1 - L / (dm.Hkv * dm.B)) * 64;
  const int npos = min(64, dm.Tq - i0);
  const int nmax = dm.ncand(dm.q_pos0 + i0 + npos - 1);
  const int words = (nmax + 31) / 32;
  // LDS: the G score blocks, later reused by the second pass's prefix table
  // (64 x words ints, larger than the blocks past 65 G 32 candidates), then the
  // bitmask; layout as group_mfma_smem sizes it for nc candidates
  float (*sS)[64][65] = reinterpret_cast<float (*)[64][65]>(gsm2);  // [G]
  uint32_t* selb =
      reinterpret_cast<uint32_t*>(gsm2 + max(G * 64 * 65, 64 * ((nc + 31) / 32)));  // [64][words]
  // selecting lane: position sp = hh PS + lane of the block
  const int sp = hh * PS + min(lane, PS - 1);
  const bool sel_lane = lane < PS && sp < npos;
  const int my_n = sel_lane ? dm.ncand(dm.q_pos0 + i0 + sp) : 0;

  uint4 qa[4][D / 32];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = 16 * mb + c;
    const long long off = (((long long)b * dm.Tq + i0 + m) * dm.H + h) * D;
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
      qa[mb][ds] = m < npos ? *reinterpret_cast<const uint4*>(Q + off + 32 * ds + 8 * g) : make_uint4(0, 0, 0, 0);
  }
  // this wavefront's head: scores of candidates c0 .. c0 + 63 for the 64 positions
  // scores of candidates c0 + 16 nb + c for rows 16 mb + 4 g + r, handed per block to f
  auto score_blocks = [&](int c0, auto&& f) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int chunk = c0 + 16 * nb + c;
      const bool cv = chunk < nmax;
      // a column past the candidates reads block 0 (in bounds); its score is
      // never selected, so the loads need no condition
      const uint4* src = ks + ks_frag<D>(dm, nc, b, h, cv ? (c0 >> 4) + nb : 0) + lane;
      bf16x8 hi[D / 32], lo[D / 32];
#pragma unroll
      for (int ds = 0; ds < D / 32; ++ds) {
        hi[ds] = as_bf16x8(src[(2 * ds) * 64]);
        lo[ds] = as_bf16x8(src[(2 * ds + 1) * 64]);
      }
      const float e = ent[((long long)b * dm.NCcap + (cv ? chunk : 0)) * dm.H + h];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const floatx4 a = score_block<D>(qa[mb], hi, lo);
        floatx4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = fmaf(a[r], dm.scale, e);
        f(mb, nb, v);
      }
    }
  };
  // Selection by the group maximum. With KM <= 32 every wavefront ranks all 64
  // positions (lane = position) over its own share of the candidates (16-wide
  // sub-blocks hh, hh + G, ... of each 64-candidate block, in chunk order), and
  // the G sorted lists of a position are merged at the end (the position's top
  // KM lies in the union of its lists' tops): all 64 lanes work where one
  // position per lane over all candidates would keep 64 / G lanes. With KM = 64
  // the G lists do not fit the score blocks' LDS, and each wavefront ranks its
  // own 64 / G positions over all candidates.
  constexpr bool kSplit = KM <= 32;
  const int rp = kSplit ? lane : sp;  // the position this lane ranks
  const int rn = kSplit ? (lane < npos ? dm.ncand(dm.q_pos0 + i0 + lane) : 0) : my_n;
  auto gscore = [&](int j) -> float {
    float v = sS[0][rp][j];
#pragma unroll
    for (int x = 1; x < G; ++x) v = fmaxf(v, sS[x][rp][j]);
    return v;
  };

  TopList<KM> top;
  top.init();
  bool first = true;  // the list's first sub-block is sorted in one go
  for (int c0 = 0; c0 < nmax; c0 += 64) {
    score_blocks(c0, [&](int mb, int nb, const floatx4& v) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sS[hh][16 * mb + 4 * g + r][16 * nb + c] = v[r];
    });
    __syncthreads();
    const int lim = min(64, rn - c0);
#pragma unroll 1
    for (int sb = kSplit ? hh : 0; sb < 4; sb += kSplit ? G : 1) {
      if (first) {
        float xs[16];
        int xc[16];
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) xs[jj] = gscore(16 * sb + jj);  // all in flight together
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const bool ok = 16 * sb + jj < lim;
          xs[jj] = ok ? xs[jj] : -INFINITY;
          xc[jj] = ok ? c0 + 16 * sb + jj : 0x7fffffff;
        }
        sort16(xs, xc);
#pragma unroll
        for (int k = 0; k < 16 && k < KM; ++k) top.s[k] = xs[k], top.c[k] = xc[k];
        first = false;
        continue;
      }
      const float theta = top.s[KM - 1];
      // unconditional reads, combined without short-circuit (all in flight together)
      float xv[16];
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) xv[jj] = gscore(16 * sb + jj);
      uint32_t mask = 0;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj)
        mask |= ((16 * sb + jj < lim) & (xv[jj] > theta)) ? (1u << jj) : 0u;
      const int todo = wave_max16(__popc(mask));
      // each insert's candidate is read one insert ahead
      int jj = mask ? __ffs(mask) - 1 : 0;
      float x = gscore(16 * sb + jj);
      for (int q = 0; q < todo; ++q) {
        const bool have = mask != 0;
        const int cj = jj;
        mask &= mask - 1;
        jj = mask ? __ffs(mask) - 1 : 0;
        const float xn = gscore(16 * sb + jj);
        top.insert(have ? x : -INFINITY, c0 + 16 * sb + cj);
        x = xn;
      }
    }
    __syncthreads();
  }
  if constexpr (kSplit) {
    // the G lists of every position through LDS (the score blocks are free now),
    // then wavefront hh merges those of its positions by (score desc, chunk asc)
    float* ml = reinterpret_cast<float*>(gsm2);            // [G][KM][64]
    int* mi = reinterpret_cast<int*>(gsm2) + G * KM * 64;  // [G][KM][64]
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      ml[(hh * KM + k) * 64 + lane] = top.s[k];
      mi[(hh * KM + k) * 64 + lane] = top.c[k];
    }
    __syncthreads();
    int pk[G];
#pragma unroll
    for (int x = 0; x < G; ++x) pk[x] = 0;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      float bs = -INFINITY;
      int bc = 0x7fffffff, bx = 0;
#pragma unroll
      for (int x = 0; x < G; ++x) {
        const int o = (x * KM + min(pk[x], KM - 1)) * 64 + sp;
        const float vs = pk[x] < KM ? ml[o] : -INFINITY;
        const int vc = pk[x] < KM ? mi[o] : 0x7fffffff;
        const bool better = vs > bs || (vs == bs && vc < bc);
        bs = better ? vs : bs;
        bc = better ? vc : bc;
        bx = better ? x : bx;
      }
      top.s[k] = bs;
      top.c[k] = bc;
#pragma unroll
      for (int x = 0; x < G; ++x) pk[x] += x == bx ? 1 : 0;
    }
    __syncthreads();
  }
  // selected sets: index output for the G heads and the position's bitmask
  const int cnt = min(K, my_n);
  for (int x = t; x < 64 * words; x += 64 * G) selb[x] = 0u;
  __syncthreads();
  if (sel_lane) {
    const long long orow = ((long long)b * dm.Tq + i0 + sp) * dm.H + (long long)gk * G;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      int rank = 0;
#pragma unroll
      for (int k2 = 0; k2 < KM; ++k2) rank += (k2 < cnt && top.c[k2] < top.c[k]) ? 1 : 0;
      if (k < cnt) {
        atomicOr(&selb[sp * words + top.c[k] / 32], 1u << (top.c[k] % 32));
#pragma unroll
        for (int x = 0; x < G; ++x) idx[(orow + x) * K + rank] = top.c[k];
      }
    }
    for (int k = cnt; k < K; ++k)
#pragma unroll
      for (int x = 0; x < G; ++x) {
        idx[(orow + x) * K + k] = -1;
        score[(orow + x) * K + k] = -INFINITY;
      }
  }
  __syncthreads();
  // per (position, bitmask word): selected chunks in the words before it, kept
  // where the first pass's scores were
  int* selp = reinterpret_cast<int*>(gsm2);  // [64][words]
  for (int p = t; p < 64; p += 64 * G) {
    int run = 0;
    for (int x = 0; x < words; ++x) {
      selp[p * words + x] = run;
      run += __popc(selb[p * words + x]);
    }
  }
  __syncthreads();
  // second pass: this head's score of every selected (position, chunk); the
  // bitmask and prefix reads are unconditional, so they are in flight together
  for (int c0 = 0; c0 < nmax; c0 += 64) {
    score_blocks(c0, [&](int mb, int nb, const floatx4& v) {
      const int ch = c0 + 16 * nb + c;
      const int wi = min(ch / 32, words - 1);
      uint32_t wv[4];
      int pre[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = 16 * mb + 4 * g + r;
        wv[r] = selb[pos * words + wi];
        pre[r] = selp[pos * words + wi];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = 16 * mb + 4 * g + r;
        const bool hit = (pos < npos) & (ch < nmax) & (((wv[r] >> (ch % 32)) & 1u) != 0u);
        if (hit)
          score[(((long long)b * dm.Tq + i0 + pos) * dm.H + h) * K + pre[r] +
                __popc(wv[r] & ((1u << (ch % 32)) - 1u))] = v[r];
      }
    });
  }
}

size_t group_mfma_smem(int G, int nmax) {
  const size_t words = (nmax + 31) / 32;
  return std::max<size_t>((size_t)G * 64 * 65, 64 * words) * sizeof(float) +
         64 * words * sizeof(uint32_t);
}

// Decode split: grid (splits, rows); a workgroup of 4 wavefronts scores the
// kSplitM candidates of one row, 32 per wavefront (the row sits in M position 0
// of each 16x16 block; other positions are zero), and writes the split's local
// top-K, ranked in LDS.
template <int D>
__global__ __launch_bounds__(256) void k_score_split_mfma(Dims dm, const uint16_t* __restrict__ Q,
                                                          const float* __restrict__ ksum,
                                                          const float* __restrict__ ent,
                                                          float* __restrict__ ws_s,
                                                          int* __restrict__ ws_i, int nsplit) {
  static_assert(kSplitM == 128, "four wavefronts of 32 candidates");
  __shared__ __align__(16) float ss[kSplitM];
  __shared__ int part[kSplitM];
  const int split = blockIdx.x, r = blockIdx.y;
  const int i = (r / dm.H) % dm.Tq;
  const int n = dm.ncand(dm.q_pos0 + i);
  const int cbase = split * kSplitM;
  mf::split_scores<D, 4>(dm, Q, ksum, ent, r, n, cbase, ss);
  __syncthreads();
  // local rank: invalid candidates hold -inf and sort after every valid one
  // (a valid candidate's rank counts only valid candidates before it)
  const long long o = ((long long)r * nsplit + split) * dm.K;
  mf::split_local_topk_halves<kSplitM>(ss, part, max(0, min(kSplitM, n - cbase)), cbase, dm.K,
                                      ws_s + o, ws_i + o);
}

}  // namespace

bool score_mfma_group_applies(const Dims& dm) {
  const int nmax = dm.ncand(dm.q_pos0 + dm.Tq - 1);
  return dm.bf16 && (dm.G == 2 || dm.G == 4) && group_mfma_smem(dm.G, nmax) <= 160 * 1024;
}

hipError_t launch_score_mfma_group(const Dims& dm, const void* Q, const float* ksum,
                                   const float* ent, int32_t* idx, float* score, void* ws,
                                   hipStream_t st) {
  const int nc = max(1, dm.ncand(dm.q_pos0 + dm.Tq - 1));
  uint4* ks = reinterpret_cast<uint4*>(ws);
  const long long n16 = (long long)dm.B * dm.H * ((nc + 15) / 16) * (dm.d / 16) * 64;
  const int grid = (int)std::min<long long>((n16 + 255) / 256, 4096);
  const size_t smem = group_mfma_smem(dm.G, nc);
  dim3 g3((unsigned)((dm.Tq + 63) / 64) * dm.Hkv * dm.B);
  const auto* Qh = reinterpret_cast<const uint16_t*>(Q);
  hipError_t e = hipSuccess;
#define HILS_GRP(DD, KMM, GG)                                                                  \
  do {                                                                                         \
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_score_mfma_group<DD, KMM, GG>),     \
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);             \
    if (e != hipSuccess) return e;                                                             \
    hipLaunchKernelGGL((k_score_mfma_group<DD, KMM, GG>), g3, dim3(64 * GG), smem, st, dm, nc, \
                       Qh, ks, ent, idx, score);                                               \
  } while (0)
#define HILS_GRP_K(DD)                                                                       \
  do {                                                                                         \
    if (dm.K <= 16) {                                                                          \
      if (dm.G == 2) HILS_GRP(DD, 16, 2); else HILS_GRP(DD, 16, 4);                             \
    } else if (dm.K <= 32) {                                                                   \
      if (dm.G == 2) HILS_GRP(DD, 32, 2); else HILS_GRP(DD, 32, 4);                             \
    } else {                                                                                   \
      if (dm.G == 2) HILS_GRP(DD, 64, 2); else HILS_GRP(DD, 64, 4);                             \
    }                                                                                          \
  } while (0)
  if (dm.d == 64) {
    hipLaunchKernelGGL((k_ksplit<64>), dim3(grid), dim3(256), 0, st, dm, nc, ksum, ks);
    HILS_GRP_K(64);
  } else {
    hipLaunchKernelGGL((k_ksplit<128>), dim3(grid), dim3(256), 0, st, dm, nc, ksum, ks);
    HILS_GRP_K(128);
  }
#undef HILS_GRP_K
#undef HILS_GRP
  return hipGetLastError();
}

size_t score_mfma_prefill_ws_bytes(const Dims& dm) {
  const int nc = max(1, dm.ncand(dm.q_pos0 + dm.Tq - 1));
  return (size_t)dm.B * dm.H * ((nc + 15) / 16) * 16 * 2 * dm.d * sizeof(uint16_t);
}

hipError_t launch_score_mfma_prefill(const Dims& dm, const void* Q, const float* ksum,
                                     const float* ent, int32_t* idx, float* score, void* ws,
                                     hipStream_t st) {
  const int nc = max(1, dm.ncand(dm.q_pos0 + dm.Tq - 1));
  uint4* ks = reinterpret_cast<uint4*>(ws);
  const long long n16 = (long long)dm.B * dm.H * ((nc + 15) / 16) * (dm.d / 16) * 64;
  const int grid = (int)std::min<long long>((n16 + 255) / 256, 4096);
  dim3 g3((unsigned)((dm.Tq + 63) / 64) * dm.H * dm.B);
  const auto* Qh = reinterpret_cast<const uint16_t*>(Q);
  // the register list holds 16, 32 or 64 entries: the smallest that holds K
#define HILS_ROW(DD)                                                                             \
  do {                                                                                           \
    if (dm.K <= 16)                                                                              \
      hipLaunchKernelGGL((k_score_mfma<DD, 16>), g3, dim3(64), 0, st, dm, nc, Qh, ks, ent, idx,   \
                         score);                                                                 \
    else if (dm.K <= 32)                                                                         \
      hipLaunchKernelGGL((k_score_mfma<DD, 32>), g3, dim3(64), 0, st, dm, nc, Qh, ks, ent, idx,   \
                         score);                                                                 \
    else                                                                                         \
      hipLaunchKernelGGL((k_score_mfma<DD, 64>), g3, dim3(64), 0, st, dm, nc, Qh, ks, ent, idx,   \
                         score);                                                                 \
  } while (0)
  if (dm.d == 64) {
    hipLaunchKernelGGL((k_ksplit<64>), dim3(grid), dim3(256), 0, st, dm, nc, ksum, ks);
    HILS_ROW(64);
  } else {
    hipLaunchKernelGGL((k_ksplit<128>), dim3(grid), dim3(256), 0, st, dm, nc, ksum, ks);
    HILS_ROW(128);
  }
#undef HILS_ROW
  return hipGetLastError();
}

hipError_t launch_score_mfma_split(const Dims& dm, const void* Q, const float* ksum,
                                   const float* ent, float* ws_s, int* ws_i, int nsplit,
                                   hipStream_t st) {
  const long long rows = (long long)dm.B * dm.Tq * dm.H;
  if (dm.d == 64)
    hipLaunchKernelGGL((k_score_split_mfma<64>), dim3(nsplit, rows), dim3(256), 0, st, dm,
                       reinterpret_cast<const uint16_t*>(Q), ksum, ent, ws_s, ws_i, nsplit);
  else
    hipLaunchKernelGGL((k_score_split_mfma<128>), dim3(nsplit, rows), dim3(256), 0, st, dm,
                       reinterpret_cast<const uint16_t*>(Q), ksum, ent, ws_s, ws_i, nsplit);
  return hipGetLastError();
}

}  // namespace hils
