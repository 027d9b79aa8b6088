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

size_t attend_ws_bytes(const Dims& dm) { return attend_mfma_ws_bytes(dm); }

hipError_t launch_attend_fuse(const Dims& dm, const void* Q, const void* K, const void* V,
                              const int32_t* idx, const float* score, void* O, float* lse_own,
                              float* lse_tot, void* ws, hipStream_t st) {
  if ((long long)dm.B * dm.Tq * dm.H == 0) return hipSuccess;
  // prefill-sized bf16 problems run on matrix cores; single rows (decode) and
  // float32 inputs use the rows kernel
  hipError_t err = hipSuccess;
  if (attend_mfma_try(dm, Q, K, V, idx, score, O, lse_own, lse_tot, ws, st, &err)) return err;
  if (dm.bf16) {
    return dm.d == 64 ? launch_t<true, 64>(dm, Q, K, V, idx, score, O, lse_own, lse_tot, st)
                      : launch_t<true, 128>(dm, Q, K, V, idx, score, O, lse_own, lse_tot, st);
  }
  return dm.d == 64 ? launch_t<false, 64>(dm, Q, K, V, idx, score, O, lse_own, lse_tot, st)
                    : launch_t<false, 128>(dm, Q, K, V, idx, score, O, lse_own, lse_tot, st);
}

}  // namespace hils
