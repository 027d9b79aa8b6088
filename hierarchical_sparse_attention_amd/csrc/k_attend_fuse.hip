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
#include "hils_internal.h"

namespace hils {
namespace {

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

  // inter-chunk normaliser over the selected scores and the own log-mass
  const int Ksel = dm.K;
  float sc = -INFINITY;
  if (lane < Ksel) sc = score[r * Ksel + lane];
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
    const int c = idx[r * Ksel + k];  // wave-uniform
    if (c < 0 || c >= ncand) continue;  // pads; ids outside the candidate range are ignored
    const float sh = score[r * Ksel + k];
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
// bf16 key and value rows are read with 16-byte loads in one layout: the wave's
// lanes form NG = 64 / LP groups of LP = d / 8 lanes; group q holds rows
// NV q .. NV q + NV - 1 (NV = d / 8) and lane l % LP of the group the features
// 8 (l % LP) .. + 8 of those rows, so each load instruction reads whole rows.
// Logits: per-lane partial dots summed over the group's lanes; softmax across
// groups; values: per-lane partial outputs summed across groups. Cross-lane
// steps use DPP and permlane swaps.
template <int D>
struct DecodeCfg {
  static constexpr int LP = D / 8;                // lanes per row
  static constexpr int NG = kWave / LP;           // row groups
  static constexpr int NV = kChunk / NG;          // rows per group (16-byte pieces per lane)
};

// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror, row_ror:8
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140,
              kDppRor8 = 0x128;
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// sum over the LP lanes of a group (LP = 8 or 16)
template <int LP>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  if (LP == 16) v += dpp<kDppMirror>(v);
  return v;
}
__device__ __forceinline__ float swap16_32(float x, bool mx) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = mx ? fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1])) : __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return mx ? fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1])) : __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// max / sum across the NG groups (lanes that differ in l / LP)
template <int LP>
__device__ __forceinline__ float cross_max(float v) {
  if (LP == 8) v = fmaxf(v, dpp<kDppRor8>(v));
  return swap16_32(v, true);
}
template <int LP>
__device__ __forceinline__ float cross_sum(float v) {
  if (LP == 8) v += dpp<kDppRor8>(v);
  return swap16_32(v, false);
}

template <int D>
struct SlotRegs {
  uint4 k[DecodeCfg<D>::NV];
  uint4 v[DecodeCfg<D>::NV];
};

template <int D>
__device__ __forceinline__ void slot_load(SlotRegs<D>& x, const uint16_t* K, const uint16_t* V,
                                          long long kv_base, long long kv_stride, long long key0,
                                          int nk) {
  using C = DecodeCfg<D>;
  const int lane = threadIdx.x & (kWave - 1);
  const int j0 = C::NV * (lane / C::LP), f0 = 8 * (lane % C::LP);
#pragma unroll
  for (int m = 0; m < C::NV; ++m) {
    const long long off = kv_base + (key0 + min(j0 + m, nk - 1)) * kv_stride + f0;
    x.k[m] = *reinterpret_cast<const uint4*>(K + off);
    x.v[m] = *reinterpret_cast<const uint4*>(V + off);
  }
}

template <int D>
__device__ __forceinline__ void slot_compute(const SlotRegs<D>& x, const Dims& dm,
                                             const uint16_t* qs, int nk, float* o_out,
                                             float* l_out) {
  using C = DecodeCfg<D>;
  const int lane = threadIdx.x & (kWave - 1);
  const int j0 = C::NV * (lane / C::LP), f0 = 8 * (lane % C::LP);
  const uint4 qv = *reinterpret_cast<const uint4*>(qs + f0);  // this lane's 8 query features
  const uint32_t qa[4] = {qv.x, qv.y, qv.z, qv.w};
  float s[C::NV];
#pragma unroll
  for (int m = 0; m < C::NV; ++m) {
    const uint32_t ka[4] = {x.k[m].x, x.k[m].y, x.k[m].z, x.k[m].w};
    float part = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      part = fmaf(__uint_as_float(qa[k] << 16), __uint_as_float(ka[k] << 16), part);
      part = fmaf(__uint_as_float(qa[k] & 0xFFFF0000u), __uint_as_float(ka[k] & 0xFFFF0000u), part);
    }
    s[m] = group_sum<C::LP>(part);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int m = 0; m < C::NV; ++m) {
    s[m] = j0 + m < nk ? s[m] * dm.scale : -INFINITY;
    mx = fmaxf(mx, s[m]);
  }
  mx = cross_max<C::LP>(mx);
  float z = 0.0f;
#pragma unroll
  for (int m = 0; m < C::NV; ++m) {
    s[m] = expf(s[m] - mx);  // 0 for masked keys
    z += s[m];
  }
  z = cross_sum<C::LP>(z);
  const float L = mx + logf(z);
  const float iz = 1.0f / z;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int m = 0; m < C::NV; ++m) {
    const float pj = s[m] * iz;
    const uint32_t va[4] = {x.v[m].x, x.v[m].y, x.v[m].z, x.v[m].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[2 * k] = fmaf(pj, __uint_as_float(va[k] << 16), acc[2 * k]);
      acc[2 * k + 1] = fmaf(pj, __uint_as_float(va[k] & 0xFFFF0000u), acc[2 * k + 1]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = cross_sum<C::LP>(acc[e]);
  if (lane < C::LP) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o_out[f0 + e] = acc[e];
  }
  if (lane == 0) *l_out = L;
}

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
  // query and selection read together (unconditionally, indices in bounds)
  const int c = idx[r * dm.K + min(slot, dm.K - 1)];
#pragma unroll
  for (int x = 0; x < D / kWave; ++x) {
    if (BF16) qh[lane + kWave * x] = reinterpret_cast<const uint16_t*>(Q)[r * D + lane + kWave * x];
    else qf[lane + kWave * x] = reinterpret_cast<const float*>(Q)[r * D + lane + kWave * x];
  }
  long long key0;
  int nk;
  if (slot < dm.K) {
    if (c < 0 || c >= ncand) {  // padding slot: no mass
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

// Combine kernel: one wavefront per row applies the inter-chunk softmax to the
// slots in a fixed order (selected slots by their chunk score, local slots by
// their exact log-mass). Lane k holds slots k and 64 + k.
template <bool BF16, int D>
__global__ __launch_bounds__(64) void k_decode_combine(Dims dm, const float* __restrict__ score,
                                                       const float* __restrict__ part_o,
                                                       const float* __restrict__ part_l,
                                                       void* __restrict__ O,
                                                       float* __restrict__ lse_own,
                                                       float* __restrict__ lse_tot) {
  constexpr int X = D / kWave;
  constexpr int KF = 48 / X;  // slots whose partials are read in the first round trip
  const long long r = blockIdx.x;
  const int lane = threadIdx.x, Ks = dm.K, NS = Ks + dm.nlocal_max();
  const long long pb = r * NS;
  // every read is issued before any is used; rows of padding slots were not
  // written and are read only to keep the loads unconditional (weight 0)
  float lg[2], loc[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int k = lane + 64 * u, kc = min(k, NS - 1);
    const float pl = part_l[pb + kc];
    const float sc = score[r * Ks + min(k, Ks - 1)];
    lg[u] = k >= NS ? -INFINITY : k < Ks ? (pl != -INFINITY ? sc : -INFINITY) : pl;
    loc[u] = k >= Ks && k < NS ? pl : -INFINITY;
  }
  float pv[KF][X];
#pragma unroll
  for (int k = 0; k < KF; ++k)
#pragma unroll
    for (int x = 0; x < X; ++x) pv[k][x] = part_o[(pb + min(k, NS - 1)) * D + lane + kWave * x];
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
        pw[u][x] = part_o[(pb + min(k0 + u, NS - 1)) * D + lane + kWave * x];
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

bool use_decode(const Dims& dm) { return dm.Tq < 64; }

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
