// Intra-chunk attention over the selected chunks plus the causal own chunk,
// fused with the inter-chunk softmax (note §5.3 hierarchical softmax; Tide
// Fig. 3: intra-chunk weight exp(s_ij)/Z_{i,c(j)} times inter-chunk share
// exp(s^_{i,c})/Z^_i, with the own chunk's exact mass inside Z^_i).
//
// Each (query, chunk) pair is an independent softmax over at most S = 64 keys,
// so the fusion weight of every chunk is known once the own chunk's log-mass
// is: w_ij = exp(s_ij - m_ic + s^_ic - Lambda_i). No online rescaling is needed.
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
  const long long own = pos / dm.S;
  const long long kv_stride = (long long)dm.Hkv * D;                 // elements between key rows
  const long long kv_base = ((long long)b * dm.Tcap * dm.Hkv + g) * D;  // row 0 of (b, g)

  float q[D];
  load_row<BF16, D>(Q, r * D, q);

  // own chunk: keys own*S .. pos (causal)
  const long long j_own = own * dm.S + lane;
  const bool own_valid = j_own <= pos;
  float s_own = -INFINITY;
  if (own_valid) s_own = key_logit<BF16, D>(K, kv_base + j_own * kv_stride, q, dm.scale);
  const float m_own = wave_max(s_own);
  const float l_own = m_own + logf(wave_sum(own_valid ? expf(s_own - m_own) : 0.0f));

  // inter-chunk normaliser over the selected scores and the own log-mass
  const int Ksel = dm.K;
  float sc = -INFINITY;
  if (lane < Ksel) sc = score[r * Ksel + lane];
  const float mx = fmaxf(wave_max(sc), l_own);
  const float Lambda = mx + logf(wave_sum(lane < Ksel ? expf(sc - mx) : 0.0f) + expf(l_own - mx));

  float acc[D / kWave];
#pragma unroll
  for (int x = 0; x < D / kWave; ++x) acc[x] = 0.0f;
  const float w_own = own_valid ? expf(s_own - Lambda) : 0.0f;
  accumulate_values<BF16, D>(V, kv_base + own * dm.S * kv_stride, kv_stride, w_own,
                             (int)(pos - own * dm.S) + 1, lane, acc);

  for (int k = 0; k < Ksel; ++k) {
    const int c = idx[r * Ksel + k];  // wave-uniform
    if (c < 0 || c >= own) continue;  // pads; ids outside the candidate range are ignored
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
// Few query rows (decode): the work is split over (row, slot) pairs so a single
// query still spreads over the chip. Slot k < K attends selected chunk idx[k],
// slot K the causal own chunk. Each pair writes its normalised output and its
// log-mass to the workspace; a combine kernel then applies the inter-chunk
// softmax per row in a fixed slot order.
template <bool BF16, int D>
__global__ __launch_bounds__(64) void k_decode_partial(Dims dm, const void* __restrict__ Q,
                                                       const void* __restrict__ K,
                                                       const void* __restrict__ V,
                                                       const int32_t* __restrict__ idx,
                                                       float* __restrict__ part_o,
                                                       float* __restrict__ part_l) {
  const int slot = blockIdx.x, lane = threadIdx.x;
  const long long r = blockIdx.y;
  const int h = (int)(r % dm.H), i = (int)((r / dm.H) % dm.Tq);
  const int b = (int)(r / ((long long)dm.H * dm.Tq));
  const int g = h / dm.G;
  const long long pos = dm.q_pos0 + i, own = pos / dm.S;
  const long long po = (r * (dm.K + 1) + slot);
  long long key0;
  int nk;
  if (slot < dm.K) {
    const int c = idx[r * dm.K + slot];
    if (c < 0 || c >= own) {  // padding slot
      if (lane == 0) part_l[po] = -INFINITY;
      return;
    }
    key0 = (long long)c * dm.S;
    nk = kChunk;
  } else {
    key0 = own * dm.S;
    nk = (int)(pos - key0) + 1;
  }
  const long long kv_stride = (long long)dm.Hkv * D;
  const long long kv_base = ((long long)b * dm.Tcap * dm.Hkv + g) * D;
  // every load is issued before the softmax: q, the lane's key row, and for
  // o[e] = sum_j p_j V[j][e] (lane = feature) all 64 value rows (rows beyond nk
  // are clamped in bounds and carry p_j = 0)
  float q[D];
  load_row<BF16, D>(Q, r * D, q);
  const bool valid = lane < nk;
  float kr[D];
  load_row<BF16, D>(K, kv_base + (key0 + min(lane, nk - 1)) * kv_stride, kr);
  float vv[kChunk][D / kWave];
#pragma unroll
  for (int j = 0; j < kChunk; ++j) {
    const long long row = key0 + min(j, nk - 1);
#pragma unroll
    for (int x = 0; x < D / kWave; ++x)
      vv[j][x] = load_elem<BF16>(V, kv_base + row * kv_stride + lane + kWave * x);
  }
  float dot = 0.0f;
#pragma unroll
  for (int e = 0; e < D; ++e) dot = fmaf(q[e], kr[e], dot);
  const float s = valid ? dot * dm.scale : -INFINITY;
  const float m = wave_max(s);
  const float L = m + logf(wave_sum(valid ? expf(s - m) : 0.0f));
  const float p = valid ? expf(s - L) : 0.0f;
  float acc[D / kWave];
#pragma unroll
  for (int x = 0; x < D / kWave; ++x) acc[x] = 0.0f;
#pragma unroll
  for (int j = 0; j < kChunk; ++j) {
    const float pj = lane_bcast(p, j);
#pragma unroll
    for (int x = 0; x < D / kWave; ++x) acc[x] = fmaf(pj, vv[j][x], acc[x]);
  }
#pragma unroll
  for (int x = 0; x < D / kWave; ++x) part_o[po * D + lane + kWave * x] = acc[x];
  if (lane == 0) part_l[po] = L;
}

template <bool BF16, int D>
__global__ __launch_bounds__(64) void k_decode_combine(Dims dm, const float* __restrict__ score,
                                                       const float* __restrict__ part_o,
                                                       const float* __restrict__ part_l,
                                                       void* __restrict__ O,
                                                       float* __restrict__ lse_own,
                                                       float* __restrict__ lse_tot) {
  const long long r = blockIdx.x;
  const int lane = threadIdx.x, Ks = dm.K;
  const long long pb = r * (Ks + 1);
  // logits: selected slots use their chunk score, the own slot its exact log-mass
  const float l_own = part_l[pb + Ks];
  float lg = -INFINITY;
  if (lane < Ks && part_l[pb + lane] != -INFINITY) lg = score[r * Ks + lane];
  const float mx = fmaxf(wave_max(lg), l_own);
  const float Lambda = mx + logf(wave_sum(lane < Ks ? expf(lg - mx) : 0.0f) + expf(l_own - mx));
  const float a = lane < Ks ? expf(lg - Lambda) : 0.0f;
  const float a_own = expf(l_own - Lambda);
  float acc[D / kWave];
#pragma unroll
  for (int x = 0; x < D / kWave; ++x) acc[x] = 0.0f;
  for (int k0 = 0; k0 < Ks; k0 += 8) {
    float pv[8][D / kWave];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int x = 0; x < D / kWave; ++x)
        pv[kk][x] = k0 + kk < Ks ? part_o[(pb + k0 + kk) * D + lane + kWave * x] : 0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      // padding slots wrote no partial: their (unwritten) values are never used
      const float ak = k0 + kk < Ks ? lane_bcast(a, k0 + kk) : 0.0f;
      if (ak != 0.0f) {  // wave-uniform
#pragma unroll
        for (int x = 0; x < D / kWave; ++x) acc[x] = fmaf(ak, pv[kk][x], acc[x]);
      }
    }
  }
#pragma unroll
  for (int x = 0; x < D / kWave; ++x) {
    acc[x] = fmaf(a_own, part_o[(pb + Ks) * D + lane + kWave * x], acc[x]);
    store_elem<BF16>(O, r * D + lane + kWave * x, acc[x]);
  }
  if (lane == 0) {
    if (lse_own) lse_own[r] = l_own;
    if (lse_tot) lse_tot[r] = Lambda;
  }
}

bool use_decode(const Dims& dm) { return dm.Tq < 64; }

size_t decode_ws_bytes(const Dims& dm) {
  const size_t rows = (size_t)dm.B * dm.Tq * dm.H;
  const size_t n = rows * (dm.K + 1);
  return ((n * dm.d * sizeof(float) + 255) & ~(size_t)255) + n * sizeof(float);
}

template <bool BF16, int D>
hipError_t launch_decode(const Dims& dm, const void* Q, const void* K, const void* V,
                         const int32_t* idx, const float* score, void* O, float* lse_own,
                         float* lse_tot, void* ws, hipStream_t st) {
  const long long rows = (long long)dm.B * dm.Tq * dm.H;
  const size_t n = (size_t)rows * (dm.K + 1);
  float* part_o = reinterpret_cast<float*>(ws);
  float* part_l = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                           ((n * D * sizeof(float) + 255) & ~(size_t)255));
  hipLaunchKernelGGL((k_decode_partial<BF16, D>), dim3(dm.K + 1, rows), dim3(64), 0, st, dm, Q, K,
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
