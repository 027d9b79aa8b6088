// Intra-chunk attention over the selected chunks plus the local branch (the
// causal own chunk, or a sliding window of the last W keys), fused with the
// inter-chunk softmax (note §5.3 hierarchical softmax; Tide Fig. 3:
// intra-chunk weight exp(s_ij)/Z_{i,c(j)} times inter-chunk share
// exp(s^_{i,c})/Z^_i, with the local branch's exact mass inside Z^_i).
//
// Each (query, chunk) pair is an independent softmax over at most S = 64 keys,
// so the fusion weight of every chunk is known once the local branch's
// log-mass is: w_ij = exp(s_ij - m_ic + s^_ic - Lambda_i); a local key gets
// exp(s_ij - Lambda_i). No online rescaling of outputs is needed.
//
// Rows kernel: one wavefront per (b, i, h). Lane j owns key j for the logits;
// lane e owns output features e (and e+64) for the value sum, with the weights
// broadcast lane-to-lane by v_readlane.
#include <algorithm>

#include "decode_merge.h"
#include "decode_slot.h"
#include "hils_internal.h"

namespace hils {
namespace {

using dec::DecodeCfg;
using dec::SlotRegs;
using dec::slot_compute;
using dec::slot_load;
using dec::cross_sum;
using dec::cross_max;

template <bool BF16, int D>
__device__ __forceinline__ float key_logit(const void* K, long long row_off, const float* q,
                                           float scale) {
  float kr[D];
  load_row<BF16, D>(K, row_off, kr);
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < D; ++e) acc = fmaf(q[e], kr[e], acc);
  return acc * scale;
}

__device__ __forceinline__ float lane_bcast(float v, int j) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}

// acc[x] += sum_{j < nkeys} w_j * V[row0 + j][lane + 64 x], w_j read from lane j.
template <bool BF16, int D>
__device__ __forceinline__ void accumulate_values(const void* V, long long row0_off,
                                                  long long row_stride, float w, int nkeys,
                                                  int lane, float* acc) {
  for (int j = 0; j < nkeys; ++j) {
    const float wj = lane_bcast(w, j);
    if (wj == 0.0f) continue;  // wave-uniform
    const long long off = row0_off + j * row_stride;
#pragma unroll
    for (int x = 0; x < D / kWave; ++x) acc[x] = fmaf(wj, load_elem<BF16>(V, off + lane + kWave * x), acc[x]);
  }
}

template <bool BF16, int D>
__global__ __launch_bounds__(256) void k_attend_rows(Dims dm, const void* __restrict__ Q,
                                                     const void* __restrict__ K,
                                                     const void* __restrict__ V,
                                                     const int32_t* __restrict__ idx,
                                                     const float* __restrict__ score,
                                                     void* __restrict__ O,
                                                     float* __restrict__ lse_own,
                                                     float* __restrict__ lse_tot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int i = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int h = blockIdx.y, b = blockIdx.z;
  if (i >= dm.Tq) return;
  const int g = h / dm.G;
  const long long r = ((long long)b * dm.Tq + i) * dm.H + h;
  const long long pos = dm.q_pos0 + i;
  const int ncand = dm.ncand(pos);
  const long long kv_stride = (long long)dm.Hkv * D;                 // elements between key rows
  const long long kv_base = ((long long)b * dm.Tcap * dm.Hkv + g) * D;  // row 0 of (b, g)

  float q[D];
  load_row<BF16, D>(Q, r * D, q);

  // local branch: keys l0 .. pos, chunk by chunk (one chunk for the own-chunk branch)
  const long long l0 = dm.lstart(pos), c_lo = l0 / kChunk, c_hi = pos / kChunk;
  auto local_logit = [&](long long cc, bool* v) {
    const long long j = cc * dm.S + lane;
    *v = j >= l0 && j <= pos;
    return *v ? key_logit<BF16, D>(K, kv_base + j * kv_stride, q, dm.scale) : -INFINITY;
  };
  float m_loc = -INFINITY, z_loc = 0.0f;  // running max and sum over the local chunks
  for (long long cc = c_lo; cc <= c_hi; ++cc) {
    bool v;
    const float s = local_logit(cc, &v);
    const float m = wave_max(s);
    const float z = wave_sum(v ? expf(s - m) : 0.0f);
    const float mn = fmaxf(m_loc, m);
    z_loc = z_loc * expf(m_loc - mn) + z * expf(m - mn);
    m_loc = mn;
  }
  const float l_own = m_loc + logf(z_loc);

  // inter-chunk normaliser over the counted entries' scores and the own log-mass
  // (lane k holds entry k; see entry_counts)
  const int Ksel = dm.K;
  const int cl = lane < Ksel ? idx[r * Ksel + lane] : -1;
  const bool counted = lane < Ksel && entry_counts(cl, ncand, wave_excl_max(cl, -1));
  const uint64_t cmask = __ballot(counted);
  float sc = -INFINITY;
  if (counted) sc = score[r * Ksel + lane];
  const float mx = fmaxf(wave_max(sc), l_own);
  const float Lambda = mx + logf(wave_sum(lane < Ksel ? expf(sc - mx) : 0.0f) + expf(l_own - mx));

  float acc[D / kWave];
#pragma unroll
  for (int x = 0; x < D / kWave; ++x) acc[x] = 0.0f;
  for (long long cc = c_lo; cc <= c_hi; ++cc) {
    bool v;
    const float s = local_logit(cc, &v);
    accumulate_values<BF16, D>(V, kv_base + cc * dm.S * kv_stride, kv_stride,
                               v ? expf(s - Lambda) : 0.0f,
                               (int)min((long long)kChunk, pos - cc * dm.S + 1), lane, acc);
  }

  for (int k = 0; k < Ksel; ++k) {
    if (((cmask >> k) & 1ull) == 0ull) continue;  // wave-uniform: entries that do not count
    const int c = __builtin_amdgcn_readlane(cl, k);
    const float sh = lane_bcast(sc, k);
    const long long j = (long long)c * dm.S + lane;
    const float s = key_logit<BF16, D>(K, kv_base + j * kv_stride, q, dm.scale);
    const float m = wave_max(s);
    const float lz = m + logf(wave_sum(expf(s - m)));
    const float w = expf(s - lz + sh - Lambda);
    accumulate_values<BF16, D>(V, kv_base + (long long)c * dm.S * kv_stride, kv_stride, w,
                               kChunk, lane, acc);
  }
#pragma unroll
  for (int x = 0; x < D / kWave; ++x) store_elem<BF16>(O, r * D + lane + kWave * x, acc[x]);
  if (lane == 0) {
    if (lse_own) lse_own[r] = l_own;
    if (lse_tot) lse_tot[r] = Lambda;
  }
}

// ---------------------------------------------------------------- decode
// Few query rows (decode): one wavefront per (slot, row): slot k < K attends
// selected chunk idx[k], slots K .. K + NL - 1 the local branch's chunks (its
// keys inside each chunk). Each writes its normalised output and log-mass to
// the workspace; a combine kernel then applies the inter-chunk softmax per row
// in a fixed slot order (a local chunk enters with its exact log-mass, which
// sums to the local branch's).
// float32 slot: lane j owns key j for the logits, lane e features e (+ 64 x).
template <int D>
__device__ __forceinline__ void decode_slot_f32(const Dims& dm, const float* qs, const float* K,
                                                const float* V, long long kv_base, long long key0,
                                                int nk, float* o_out, float* l_out) {
  const int lane = threadIdx.x & (kWave - 1);
  const long long kv_stride = (long long)dm.Hkv * D;
  const bool valid = lane < nk;
  float kr[D];
  load_row<false, D>(K, kv_base + (key0 + min(lane, nk - 1)) * kv_stride, kr);
  float dot = 0.0f;
#pragma unroll
  for (int e = 0; e < D; ++e) dot = fmaf(qs[e], kr[e], dot);
  const float s = valid ? dot * dm.scale : -INFINITY;
  const float m = wave_max(s);
  const float L = m + logf(wave_sum(valid ? expf(s - m) : 0.0f));
  const float p = valid ? expf(s - L) : 0.0f;
  float acc[D / kWave];
#pragma unroll
  for (int x = 0; x < D / kWave; ++x) acc[x] = 0.0f;
  for (int j = 0; j < nk; ++j) {
    const float pj = lane_bcast(p, j);
    const long long row = kv_base + (key0 + j) * kv_stride;
#pragma unroll
    for (int x = 0; x < D / kWave; ++x) acc[x] = fmaf(pj, V[row + lane + kWave * x], acc[x]);
  }
#pragma unroll
  for (int x = 0; x < D / kWave; ++x) o_out[lane + kWave * x] = acc[x];
  if (lane == 0) *l_out = L;
}

// Slot kernel: grid (K + NL, rows), one wavefront per (slot, row); writes the
// slot's normalised output and log-mass (-inf for padding) to the workspace.
// Spreading the slots over workgroups keeps many chunk reads in flight at once.
template <bool BF16, int D>
__global__ __launch_bounds__(64) void k_decode_partial(Dims dm, const void* __restrict__ Q,
                                                       const void* __restrict__ K,
                                                       const void* __restrict__ V,
                                                       const int32_t* __restrict__ idx,
                                                       float* __restrict__ part_o,
                                                       float* __restrict__ part_l) {
  __shared__ __align__(16) uint16_t qh[D];
  __shared__ __align__(16) float qf[D];
  const int slot = blockIdx.x, lane = threadIdx.x;
  const long long r = blockIdx.y;
  const int h = (int)(r % dm.H), i = (int)((r / dm.H) % dm.Tq);
  const int b = (int)(r / ((long long)dm.H * dm.Tq));
  const int g = h / dm.G;
  const long long pos = dm.q_pos0 + i;
  const int ncand = dm.ncand(pos);
  const long long po = r * (dm.K + dm.nlocal_max()) + slot;
  const long long kv_base = ((long long)b * dm.Tcap * dm.Hkv + g) * D;
  const long long kv_stride = (long long)dm.Hkv * D;
  // query and selection read together (unconditionally, indices in bounds); lane
  // l < slot holds the row's earlier entry l, which decides whether this one counts
  const int c = idx[r * dm.K + min(slot, dm.K - 1)];
  const int cprev = lane < min(slot, dm.K) ? idx[r * dm.K + lane] : -1;
#pragma unroll
  for (int x = 0; x < D / kWave; ++x) {
    if (BF16) qh[lane + kWave * x] = reinterpret_cast<const uint16_t*>(Q)[r * D + lane + kWave * x];
    else qf[lane + kWave * x] = reinterpret_cast<const float*>(Q)[r * D + lane + kWave * x];
  }
  long long key0;
  int nk;
  const int prev_max = wave_max_int(cprev);
  if (slot < dm.K) {
    if (!entry_counts(c, ncand, prev_max)) {  // padding or an entry that does not count: no mass
      if (lane == 0) part_l[po] = -INFINITY;
      return;
    }
    key0 = (long long)c * dm.S;
    nk = kChunk;
  } else {  // local chunk l0 / S + slot - K, keys from max(l0, its start) to min(pos, its end)
    const long long l0 = dm.lstart(pos), cc = l0 / kChunk + (slot - dm.K);
    if (cc > pos / kChunk) {
      if (lane == 0) part_l[po] = -INFINITY;
      return;
    }
    key0 = cc * dm.S > l0 ? cc * dm.S : l0;
    nk = (int)(min(pos, cc * dm.S + dm.S - 1) - key0) + 1;
  }
  if (BF16) {
    SlotRegs<D> rg;
    slot_load<D>(rg, reinterpret_cast<const uint16_t*>(K), reinterpret_cast<const uint16_t*>(V),
                 kv_base, kv_stride, key0, nk);
    __syncthreads();
    slot_compute<D>(rg, dm, qh, nk, part_o + po * D, part_l + po);
  } else {
    __syncthreads();
    decode_slot_f32<D>(dm, qf, reinterpret_cast<const float*>(K), reinterpret_cast<const float*>(V),
                       kv_base, key0, nk, part_o + po * D, part_l + po);
  }
}

// Slot kernel of a decode step that merges the split lists itself: grid
// (K + NL, rows), one workgroup of nsplit * KM threads (rounded up to whole
// wavefronts) per (slot, row). A selected slot's workgroup ranks the union of
// the row's lists (every workgroup of the row finds the same K entries), takes
// the entry at its place in chunk order, writes it to idx / score and attends
// to that chunk with its first wavefront, as k_decode_partial does; local slots
// skip the merge. Same outputs as the merge kernel followed by k_decode_partial.
template <bool BF16, int D, int KM, int NL>
__global__ __launch_bounds__(1024) void k_decode_merge_partial(
    Dims dm, const void* __restrict__ Q, const void* __restrict__ K, const void* __restrict__ V,
    const float* __restrict__ ws_s, const int* __restrict__ ws_i, int nsplit,
    int32_t* __restrict__ idx, float* __restrict__ score, float* __restrict__ part_o,
    float* __restrict__ part_l) {
  __shared__ dec::MergeSmem<KM> sm;
  __shared__ __align__(16) uint16_t qh[D];
  __shared__ __align__(16) float qf[D];
  __shared__ int sel_c;
  const int slot = blockIdx.x, t = threadIdx.x, lane = t & (kWave - 1);
  const long long r = blockIdx.y;
  const int h = (int)(r % dm.H), i = (int)((r / dm.H) % dm.Tq);
  const int b = (int)(r / ((long long)dm.H * dm.Tq));
  const int g = h / dm.G;
  const long long pos = dm.q_pos0 + i;
  const int ncand = dm.ncand(pos);
  const long long po = r * (dm.K + dm.nlocal_max()) + slot;
  const long long kv_base = ((long long)b * dm.Tcap * dm.Hkv + g) * D;
  const long long kv_stride = (long long)dm.Hkv * D;
  for (int e = t; e < D; e += blockDim.x) {  // read before any barrier below
    if (BF16) qh[e] = reinterpret_cast<const uint16_t*>(Q)[r * D + e];
    else qf[e] = reinterpret_cast<const float*>(Q)[r * D + e];
  }
  long long key0 = 0;
  int nk = 0;
  bool have = true;
  if (slot < dm.K) {  // uniform over the workgroup
    const int cnt = dec::merge_rank<KM, NL>(dm, r, ncand, ws_s, ws_i, nsplit, kSplitMfma, sm);
    const long long o = r * dm.K;
    if (t < cnt && dec::merge_place<KM>(sm, t, cnt) == slot) {
      const int c = dec::merge_chunk(sm.sel[t]);
      sel_c = c;
      idx[o + slot] = c;
      score[o + slot] = dec::merge_score(sm.sel[t]);
    }
    if (slot >= cnt && t == 0) {
      idx[o + slot] = -1;
      score[o + slot] = -INFINITY;
    }
    __syncthreads();
    // a merged list is ascending with distinct candidate ids: every entry counts
    have = slot < cnt;
    key0 = have ? (long long)sel_c * dm.S : 0;
    nk = kChunk;
  } else {  // local chunk l0 / S + slot - K, keys from max(l0, its start) to min(pos, its end)
    __syncthreads();
    const long long l0 = dm.lstart(pos), cc = l0 / kChunk + (slot - dm.K);
    have = cc <= pos / kChunk;
    key0 = cc * dm.S > l0 ? cc * dm.S : l0;
    nk = (int)(min(pos, cc * dm.S + dm.S - 1) - key0) + 1;
  }
  if (t >= kWave) return;
  if (!have) {
    if (lane == 0) part_l[po] = -INFINITY;
    return;
  }
  if (BF16) {
    SlotRegs<D> rg;
    slot_load<D>(rg, reinterpret_cast<const uint16_t*>(K), reinterpret_cast<const uint16_t*>(V),
                 kv_base, kv_stride, key0, nk);
    slot_compute<D>(rg, dm, qh, nk, part_o + po * D, part_l + po);
  } else {
    decode_slot_f32<D>(dm, qf, reinterpret_cast<const float*>(K), reinterpret_cast<const float*>(V),
                       kv_base, key0, nk, part_o + po * D, part_l + po);
  }
}

// Inter-chunk softmax of one row over its slots in a fixed order (selected slots
// by their chunk score, local slots by their exact log-mass), by one wavefront.
// sc: the row's K selection scores by slot; po / pl: the row's slot outputs
// [NS][D] and log-masses [NS] (-inf for padding). Lane k holds slots k and
// 64 + k. The pointers may be global or LDS: the arithmetic is the same.
template <bool BF16, int D>
__device__ __forceinline__ void combine_row(const Dims& dm, long long r, const float* sc_row,
                                            const float* po, const float* pl_row,
                                            void* __restrict__ O, float* __restrict__ lse_own,
                                            float* __restrict__ lse_tot) {
  constexpr int X = D / kWave;
  constexpr int KF = 48 / X;  // slots whose partials are read in the first round trip
  const int lane = threadIdx.x & (kWave - 1), Ks = dm.K, NS = Ks + dm.nlocal_max();
  // every read is issued before any is used; rows of padding slots were not
  // written and are read only to keep the loads unconditional (weight 0)
  float lg[2], loc[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int k = lane + 64 * u, kc = min(k, NS - 1);
    const float pl = pl_row[kc];
    const float sc = sc_row[min(k, Ks - 1)];
    lg[u] = k >= NS ? -INFINITY : k < Ks ? (pl != -INFINITY ? sc : -INFINITY) : pl;
    loc[u] = k >= Ks && k < NS ? pl : -INFINITY;
  }
  float pv[KF][X];
#pragma unroll
  for (int k = 0; k < KF; ++k)
#pragma unroll
    for (int x = 0; x < X; ++x) pv[k][x] = po[min(k, NS - 1) * D + lane + kWave * x];
  const float ml = wave_max(fmaxf(loc[0], loc[1]));
  const float l_own = ml + logf(wave_sum(expf(loc[0] - ml) + expf(loc[1] - ml)));
  const float mx = wave_max(fmaxf(lg[0], lg[1]));
  const float Lambda = mx + logf(wave_sum(expf(lg[0] - mx) + expf(lg[1] - mx)));
  const float a0 = expf(lg[0] - Lambda), a1 = expf(lg[1] - Lambda);
  float acc[X];
#pragma unroll
  for (int x = 0; x < X; ++x) acc[x] = 0.0f;
#pragma unroll
  for (int k = 0; k < KF; ++k) {
    const float ak = k < NS ? lane_bcast(a0, k) : 0.0f;
    if (ak != 0.0f) {  // wave-uniform; padding and absent slots are skipped
#pragma unroll
      for (int x = 0; x < X; ++x) acc[x] = fmaf(ak, pv[k][x], acc[x]);
    }
  }
  // the remaining slots (more than KF: K > 32 or a long window), eight loads at a time
  for (int k0 = KF; k0 < NS; k0 += 8) {
    float pw[8][X];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int x = 0; x < X; ++x)
        pw[u][x] = po[min(k0 + u, NS - 1) * D + lane + kWave * x];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + u;
      const float ak = k >= NS ? 0.0f : k < 64 ? lane_bcast(a0, k) : lane_bcast(a1, k - 64);
      if (ak != 0.0f) {
#pragma unroll
        for (int x = 0; x < X; ++x) acc[x] = fmaf(ak, pw[u][x], acc[x]);
      }
    }
  }
#pragma unroll
  for (int x = 0; x < X; ++x) store_elem<BF16>(O, r * D + lane + kWave * x, acc[x]);
  if (lane == 0) {
    if (lse_own) lse_own[r] = l_own;
    if (lse_tot) lse_tot[r] = Lambda;
  }
}

// Combine kernel: one wavefront per row (combine_row over the slot partials in
// the workspace).
template <bool BF16, int D>
__global__ __launch_bounds__(64) void k_decode_combine(Dims dm, const float* __restrict__ score,
                                                       const float* __restrict__ part_o,
                                                       const float* __restrict__ part_l,
                                                       void* __restrict__ O,
                                                       float* __restrict__ lse_own,
                                                       float* __restrict__ lse_tot) {
  const long long r = blockIdx.x;
  const long long pb = r * (dm.K + dm.nlocal_max());
  combine_row<BF16, D>(dm, r, score + r * dm.K, part_o + pb * D, part_l + pb, O, lse_own,
                       lse_tot);
}

// One decode row per workgroup, for calls of many rows (batched sequences): the
// row's split lists are merged once (as the merge kernel does), its selected and
// local slots are attended by the workgroup's wavefronts (slot u on wavefront u
// mod waves, as the slot kernel does) into LDS, and the slots are fused from
// LDS by combine_row. Same arithmetic as the merge, slot and combine kernels,
// so the results are the same bit for bit, with no slot partials in global
// memory. Dynamic LDS: the slot outputs [NS][D], log-masses [NS] and the
// selection scores [K]. At d = 128 a slot's key and value rows take 128
// registers, so the workgroup holds at most 512 threads.
template <int D>
constexpr int kRowThreads = D == 128 ? 512 : 1024;
template <bool BF16, int D, int KM, int NL>
__global__ __launch_bounds__(kRowThreads<D>) void k_decode_row(
    Dims dm, const void* __restrict__ Q, const void* __restrict__ K, const void* __restrict__ V,
    const float* __restrict__ ws_s, const int* __restrict__ ws_i, int nsplit,
    int32_t* __restrict__ idx, float* __restrict__ score, void* __restrict__ O,
    float* __restrict__ lse_own, float* __restrict__ lse_tot) {
  __shared__ dec::MergeSmem<KM> sm;
  __shared__ __align__(16) uint16_t qh[D];
  __shared__ __align__(16) float qf[D];
  __shared__ int sel_c[KM];
  extern __shared__ __align__(16) float rdyn[];
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave, nw = blockDim.x / kWave;
  const long long r = blockIdx.x;
  const int h = (int)(r % dm.H), i = (int)((r / dm.H) % dm.Tq);
  const int b = (int)(r / ((long long)dm.H * dm.Tq));
  const int g = h / dm.G;
  const long long pos = dm.q_pos0 + i;
  const int ncand = dm.ncand(pos);
  const int NS = dm.K + dm.nlocal_max();
  float* po = rdyn;             // [NS][D]
  float* pl = po + NS * D;      // [NS]
  float* psc = pl + NS;         // [K]
  const long long kv_base = ((long long)b * dm.Tcap * dm.Hkv + g) * D;
  const long long kv_stride = (long long)dm.Hkv * D;
  for (int e = t; e < D; e += blockDim.x) {  // read before the merge's barriers
    if (BF16) qh[e] = reinterpret_cast<const uint16_t*>(Q)[r * D + e];
    else qf[e] = reinterpret_cast<const float*>(Q)[r * D + e];
  }
  const int cnt = dec::merge_rank<KM, NL>(dm, r, ncand, ws_s, ws_i, nsplit, kSplitMfma, sm);
  const long long o = r * dm.K;
  if (t < cnt) {  // the selected entries in chunk order
    const int p = dec::merge_place<KM>(sm, t, cnt);
    const int c = dec::merge_chunk(sm.sel[t]);
    const float s = dec::merge_score(sm.sel[t]);
    sel_c[p] = c;
    psc[p] = s;
    idx[o + p] = c;
    score[o + p] = s;
  }
  for (int k = cnt + t; k < dm.K; k += blockDim.x) {
    idx[o + k] = -1;
    score[o + k] = -INFINITY;
    psc[k] = -INFINITY;
  }
  __syncthreads();
  for (int slot = w; slot < NS; slot += nw) {  // uniform per wavefront
    long long key0;
    int nk;
    bool have;
    if (slot < dm.K) {  // a merged list is ascending with distinct candidate ids: all count
      have = slot < cnt;
      key0 = have ? (long long)sel_c[slot] * dm.S : 0;
      nk = kChunk;
    } else {  // local chunk l0 / S + slot - K, keys from max(l0, its start) to min(pos, its end)
      const long long l0 = dm.lstart(pos), cc = l0 / kChunk + (slot - dm.K);
      have = cc <= pos / kChunk;
      key0 = cc * dm.S > l0 ? cc * dm.S : l0;
      nk = (int)(min(pos, cc * dm.S + dm.S - 1) - key0) + 1;
    }
    if (!have) {
      if (lane == 0) pl[slot] = -INFINITY;
      continue;
    }
    if (BF16) {
      SlotRegs<D> rg;
      slot_load<D>(rg, reinterpret_cast<const uint16_t*>(K), reinterpret_cast<const uint16_t*>(V),
                   kv_base, kv_stride, key0, nk);
      slot_compute<D>(rg, dm, qh, nk, po + slot * D, pl + slot);
    } else {
      decode_slot_f32<D>(dm, qf, reinterpret_cast<const float*>(K),
                         reinterpret_cast<const float*>(V), kv_base, key0, nk, po + slot * D,
                         pl + slot);
    }
  }
  __syncthreads();
  if (w == 0) combine_row<BF16, D>(dm, r, psc, po, pl, O, lse_own, lse_tot);
}

// The slot kernels (one wavefront per selected or local chunk of a row, no
// fragment copy) serve few query positions; the matrix-core kernel first copies
// the whole cache's K and V into fragment order, which pays only when the rows
// share their chunks. Slots are taken below 64 positions, and beyond while the
// bytes the slots read stay within four times the cache's K and V (measured on
// the 128K cache: 64 to 256 positions of 16 heads, 1.9x to 3.6x faster so).
bool use_decode(const Dims& dm) {
  if (dm.Tq < 64) return true;
  const long long rows = (long long)dm.B * dm.Tq * dm.H;
  if (rows > 65535) return false;  // the slot kernel's grid holds rows in y
  const double slot_keys = (double)rows * (dm.K + dm.nlocal_max()) * dm.S;
  const double cache_keys = (double)dm.B * dm.Tkv * dm.Hkv;
  return slot_keys <= 4.0 * cache_keys;
}

size_t decode_ws_bytes(const Dims& dm) {
  const size_t rows = (size_t)dm.B * dm.Tq * dm.H;
  const size_t n = rows * (dm.K + dm.nlocal_max());
  return ((n * dm.d * sizeof(float) + 255) & ~(size_t)255) + n * sizeof(float);
}

template <bool BF16, int D>
hipError_t launch_decode(const Dims& dm, const void* Q, const void* K, const void* V,
                         const int32_t* idx, const float* score, void* O, float* lse_own,
                         float* lse_tot, void* ws, hipStream_t st) {
  const long long rows = (long long)dm.B * dm.Tq * dm.H;
  const size_t n = (size_t)rows * (dm.K + dm.nlocal_max());
  float* part_o = reinterpret_cast<float*>(ws);
  float* part_l = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                           ((n * D * sizeof(float) + 255) & ~(size_t)255));
  hipLaunchKernelGGL((k_decode_partial<BF16, D>), dim3(dm.K + dm.nlocal_max(), rows), dim3(64), 0,
                     st, dm, Q, K,
                     V, idx, part_o, part_l);
  hipLaunchKernelGGL((k_decode_combine<BF16, D>), dim3(rows), dim3(64), 0, st, dm, score, part_o,
                     part_l, O, lse_own, lse_tot);
  return hipGetLastError();
}

template <bool BF16, int D, int KM, int NL>
hipError_t launch_decode_merged_t(const Dims& dm, const void* Q, const void* K, const void* V,
                                  const float* ws_s, const int* ws_i, int nsplit, int32_t* idx,
                                  float* score, void* O, float* lse_own, float* lse_tot, void* ws,
                                  hipStream_t st) {
  const long long rows = (long long)dm.B * dm.Tq * dm.H;
  const size_t n = (size_t)rows * (dm.K + dm.nlocal_max());
  float* part_o = reinterpret_cast<float*>(ws);
  float* part_l = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                           ((n * D * sizeof(float) + 255) & ~(size_t)255));
  const int nt = std::max(kWave, (nsplit * KM + kWave - 1) / kWave * kWave);
  hipLaunchKernelGGL((k_decode_merge_partial<BF16, D, KM, NL>), dim3(dm.K + dm.nlocal_max(), rows),
                     dim3(nt), 0, st, dm, Q, K, V, ws_s, ws_i, nsplit, idx, score, part_o,
                     part_l);
  hipLaunchKernelGGL((k_decode_combine<BF16, D>), dim3(rows), dim3(64), 0, st, dm, score, part_o,
                     part_l, O, lse_own, lse_tot);
  return hipGetLastError();
}

template <bool BF16, int D, int KM, int NL>
hipError_t launch_decode_row_t(const Dims& dm, const void* Q, const void* K, const void* V,
                               const float* ws_s, const int* ws_i, int nsplit, int32_t* idx,
                               float* score, void* O, float* lse_own, float* lse_tot,
                               hipStream_t st) {
  const long long rows = (long long)dm.B * dm.Tq * dm.H;
  const int NS = dm.K + dm.nlocal_max();
  // enough wavefronts for the merge's list entries and for up to 16 slots at once
  const int nt = std::min(kRowThreads<D>, std::max((nsplit * KM + kWave - 1) / kWave * kWave,
                                                   kWave * std::min(NS, 16)));
  if (nsplit * KM > nt) return hipErrorInvalidValue;
  const size_t smem = ((size_t)NS * D + NS + dm.K) * sizeof(float);
  const void* fn = reinterpret_cast<const void*>(k_decode_row<BF16, D, KM, NL>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_decode_row<BF16, D, KM, NL>), dim3((unsigned)rows), dim3(nt), smem, st,
                     dm, Q, K, V, ws_s, ws_i, nsplit, idx, score, O, lse_own, lse_tot);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_decode_row_d(const Dims& dm, const void* Q, const void* K, const void* V,
                               const float* ws_s, const int* ws_i, int nsplit, int km,
                               int32_t* idx, float* score, void* O, float* lse_own,
                               float* lse_tot, hipStream_t st) {
  const bool nl16 = nsplit <= 16;  // km = 64 holds at most 16 lists
  if (km == 16 && nl16)
    return launch_decode_row_t<BF16, D, 16, 16>(dm, Q, K, V, ws_s, ws_i, nsplit, idx, score, O,
                                                lse_own, lse_tot, st);
  if (km == 16 && nsplit <= 24)
    return launch_decode_row_t<BF16, D, 16, 24>(dm, Q, K, V, ws_s, ws_i, nsplit, idx, score, O,
                                                lse_own, lse_tot, st);
  if (km == 16)
    return launch_decode_row_t<BF16, D, 16, 32>(dm, Q, K, V, ws_s, ws_i, nsplit, idx, score, O,
                                                lse_own, lse_tot, st);
  if (km == 32 && nl16)
    return launch_decode_row_t<BF16, D, 32, 16>(dm, Q, K, V, ws_s, ws_i, nsplit, idx, score, O,
                                                lse_own, lse_tot, st);
  if (km == 32)
    return launch_decode_row_t<BF16, D, 32, 32>(dm, Q, K, V, ws_s, ws_i, nsplit, idx, score, O,
                                                lse_own, lse_tot, st);
  return launch_decode_row_t<BF16, D, 64, 16>(dm, Q, K, V, ws_s, ws_i, nsplit, idx, score, O,
                                              lse_own, lse_tot, st);
}

template <bool BF16, int D>
hipError_t launch_decode_merged_d(const Dims& dm, const void* Q, const void* K, const void* V,
                                  const float* ws_s, const int* ws_i, int nsplit, int km,
                                  int32_t* idx, float* score, void* O, float* lse_own,
                                  float* lse_tot, void* ws, hipStream_t st) {
  const bool nl16 = nsplit <= 16;  // km = 64 holds at most 16 lists
  if (km == 16 && nl16)
    return launch_decode_merged_t<BF16, D, 16, 16>(dm, Q, K, V, ws_s, ws_i, nsplit, idx, score, O,
                                                   lse_own, lse_tot, ws, st);
  if (km == 16 && nsplit <= 24)
    return launch_decode_merged_t<BF16, D, 16, 24>(dm, Q, K, V, ws_s, ws_i, nsplit, idx, score, O,
                                                   lse_own, lse_tot, ws, st);
  if (km == 16)
    return launch_decode_merged_t<BF16, D, 16, 32>(dm, Q, K, V, ws_s, ws_i, nsplit, idx, score, O,
                                                   lse_own, lse_tot, ws, st);
  if (km == 32 && nl16)
    return launch_decode_merged_t<BF16, D, 32, 16>(dm, Q, K, V, ws_s, ws_i, nsplit, idx, score, O,
                                                   lse_own, lse_tot, ws, st);
  if (km == 32)
    return launch_decode_merged_t<BF16, D, 32, 32>(dm, Q, K, V, ws_s, ws_i, nsplit, idx, score, O,
                                                   lse_own, lse_tot, ws, st);
  return launch_decode_merged_t<BF16, D, 64, 16>(dm, Q, K, V, ws_s, ws_i, nsplit, idx, score, O,
                                                 lse_own, lse_tot, ws, st);
}

template <bool BF16, int D>
hipError_t launch_t(const Dims& dm, const void* Q, const void* K, const void* V,
                    const int32_t* idx, const float* score, void* O, float* lse_own,
                    float* lse_tot, hipStream_t st) {
  constexpr int kRowsPerWg = 4;
  dim3 grid((dm.Tq + kRowsPerWg - 1) / kRowsPerWg, dm.H, dm.B);
  hipLaunchKernelGGL((k_attend_rows<BF16, D>), grid, dim3(kRowsPerWg * kWave), 0, st, dm, Q, K,
                     V, idx, score, O, lse_own, lse_tot);
  return hipGetLastError();
}

}  // namespace

bool attend_is_decode(const Dims& dm) { return use_decode(dm); }

hipError_t launch_decode_merged(const Dims& dm, const void* Q, const void* K, const void* V,
                                const float* ws_s, const int* ws_i, int nsplit, int km,
                                int32_t* idx, float* score, void* O, float* lse_own,
                                float* lse_tot, void* ws, hipStream_t st) {
  if (km != 16 && km != 32 && km != 64) return hipErrorInvalidValue;
  if (nsplit < 1 || nsplit > 32 || nsplit * km > 1024) return hipErrorInvalidValue;
  if (dm.bf16)
    return dm.d == 64 ? launch_decode_merged_d<true, 64>(dm, Q, K, V, ws_s, ws_i, nsplit, km, idx,
                                                         score, O, lse_own, lse_tot, ws, st)
                      : launch_decode_merged_d<true, 128>(dm, Q, K, V, ws_s, ws_i, nsplit, km,
                                                          idx, score, O, lse_own, lse_tot, ws, st);
  return dm.d == 64 ? launch_decode_merged_d<false, 64>(dm, Q, K, V, ws_s, ws_i, nsplit, km, idx,
                                                        score, O, lse_own, lse_tot, ws, st)
                    : launch_decode_merged_d<false, 128>(dm, Q, K, V, ws_s, ws_i, nsplit, km, idx,
                                                         score, O, lse_own, lse_tot, ws, st);
}

hipError_t launch_decode_row(const Dims& dm, const void* Q, const void* K, const void* V,
                             const float* ws_s, const int* ws_i, int nsplit, int km, int32_t* idx,
                             float* score, void* O, float* lse_own, float* lse_tot,
                             hipStream_t st) {
  if (km != 16 && km != 32 && km != 64) return hipErrorInvalidValue;
  if (nsplit < 1 || nsplit > 32 || nsplit * km > 1024) return hipErrorInvalidValue;
  if ((long long)dm.B * dm.Tq * dm.H > 0x7fffffffLL) return hipErrorInvalidValue;
  if (dm.bf16)
    return dm.d == 64 ? launch_decode_row_d<true, 64>(dm, Q, K, V, ws_s, ws_i, nsplit, km, idx,
                                                      score, O, lse_own, lse_tot, st)
                      : launch_decode_row_d<true, 128>(dm, Q, K, V, ws_s, ws_i, nsplit, km, idx,
                                                       score, O, lse_own, lse_tot, st);
  return dm.d == 64 ? launch_decode_row_d<false, 64>(dm, Q, K, V, ws_s, ws_i, nsplit, km, idx,
                                                     score, O, lse_own, lse_tot, st)
                    : launch_decode_row_d<false, 128>(dm, Q, K, V, ws_s, ws_i, nsplit, km, idx,
                                                      score, O, lse_own, lse_tot, st);
}

bool decode_row_applies(const Dims& dm, int nsplit, int km) {
  return nsplit * km <= (dm.d == 128 ? kRowThreads<128> : kRowThreads<64>);
}

size_t attend_ws_bytes(const Dims& dm) {
  return use_decode(dm) ? decode_ws_bytes(dm) : attend_mfma_ws_bytes(dm);
}

hipError_t launch_attend_fuse(const Dims& dm, const void* Q, const void* K, const void* V,
                              const int32_t* idx, const float* score, void* O, float* lse_own,
                              float* lse_tot, void* ws, hipStream_t st) {
  if ((long long)dm.B * dm.Tq * dm.H == 0) return hipSuccess;
  // prefill-sized bf16 problems run on matrix cores; single rows (decode) and
  // float32 inputs use the rows kernel
  hipError_t err = hipSuccess;
  if (use_decode(dm)) {
    if (dm.bf16)
      return dm.d == 64 ? launch_decode<true, 64>(dm, Q, K, V, idx, score, O, lse_own, lse_tot, ws, st)
                        : launch_decode<true, 128>(dm, Q, K, V, idx, score, O, lse_own, lse_tot, ws, st);
    return dm.d == 64 ? launch_decode<false, 64>(dm, Q, K, V, idx, score, O, lse_own, lse_tot, ws, st)
                      : launch_decode<false, 128>(dm, Q, K, V, idx, score, O, lse_own, lse_tot, ws, st);
  }
  if (attend_mfma_try(dm, Q, K, V, idx, score, O, lse_own, lse_tot, ws, st, &err)) return err;
  if (dm.bf16) {
    return dm.d == 64 ? launch_t<true, 64>(dm, Q, K, V, idx, score, O, lse_own, lse_tot, st)
                      : launch_t<true, 128>(dm, Q, K, V, idx, score, O, lse_own, lse_tot, st);
  }
  return dm.d == 64 ? launch_t<false, 64>(dm, Q, K, V, idx, score, O, lse_own, lse_tot, st)
                    : launch_t<false, 128>(dm, Q, K, V, idx, score, O, lse_own, lse_tot, st);
}

}  // namespace hils
