// Landmark chunk summaries (note §5.1, Proposition 3.1; note §5.2 landmark token).
//
// One wavefront per (batch, chunk, kv head): the chunk's S = 64 keys are
// staged once in LDS (one coalesced pass over HBM) and reused by the G query
// heads of the group. Lane j owns key j for the landmark logits and their
// softmax; lane e owns feature e for the weighted key sum.
#include "hils_internal.h"

namespace hils {
namespace {

template <bool BF16, int D>
__global__ __launch_bounds__(kWave) void k_summarize(Dims dm, const void* __restrict__ K,
                                                      const void* __restrict__ Ql, int c_begin,
                                                      float* __restrict__ ksum,
                                                      float* __restrict__ ent,
                                                      float* __restrict__ lse) {
  __shared__ float kt[kChunk][D + 1];  // +1 pad: lane-per-row reads hit distinct banks
  __shared__ float qs[D];
  __shared__ float pw[kChunk];
  const int c = c_begin + blockIdx.x, g = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;

  constexpr int VE = BF16 ? 8 : 4;  // elements per 16-byte vector
  constexpr int VPR = D / VE;       // vectors per key row
  constexpr int NV = kChunk * VPR / kWave;  // vectors per lane
  static_assert(kChunk * VPR % kWave == 0 && D % kWave == 0, "tile shape");
  // the landmark query of the first head is requested with the keys; each later
  // head's while the previous head is being summarised (the head index is
  // clamped, so the load needs no branch)
  constexpr int QE = D / kWave;
  auto ldql = [&](int hh, float* q) {
    const long long sidx = ((long long)b * dm.NCcap + c) * dm.H + g * dm.G + hh;
#pragma unroll
    for (int k = 0; k < QE; ++k) q[k] = load_elem<BF16>(Ql, sidx * D + lane + k * kWave);
  };
  float qn[QE];
  ldql(0, qn);
  // every 16-byte load of the chunk's keys is issued before any is used
  uint4 raw[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = lane + i * kWave;
    const int j = v / VPR, col = (v % VPR) * VE;
    const long long off =
        (((long long)b * dm.Tcap + (long long)c * kChunk + j) * dm.Hkv + g) * D + col;
    raw[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(K) +
                                             off * (BF16 ? 2 : 4));
  }
  // consumed here, after every key load (nothing is scheduled across the
  // barrier), so the compiler cannot sink the first query load below the keys
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < QE; ++k) asm volatile("" ::"v"(qn[k]));
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = lane + i * kWave;
    const int j = v / VPR, col = (v % VPR) * VE;
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (BF16) {
        kt[j][col + 2 * k] = __uint_as_float(w[k] << 16);
        kt[j][col + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
      } else {
        kt[j][col + k] = __uint_as_float(w[k]);
      }
    }
  }

  for (int hh = 0; hh < dm.G; ++hh) {
    const int h = g * dm.G + hh;
    const long long sidx = ((long long)b * dm.NCcap + c) * dm.H + h;
#pragma unroll
    for (int k = 0; k < QE; ++k) qs[lane + k * kWave] = qn[k];
    ldql(min(hh + 1, dm.G - 1), qn);
    __syncthreads();
    float acc = 0.0f;
#pragma unroll 16
    for (int e = 0; e < D; ++e) acc = fmaf(qs[e], kt[lane][e], acc);
    const float s = acc * dm.scale;             // landmark logit s'_j
    const float m = wave_max(s);
    const float L = m + logf(wave_sum(expf(s - m)));  // log-sum-exp
    const float p = expf(s - L);                // p'_j
    const float H = wave_sum(p * (L - s));      // -sum p log p, each term >= 0
    pw[lane] = p;
    __syncthreads();
    for (int e = lane; e < D; e += kWave) {
      float a = 0.0f;
#pragma unroll 16
      for (int j = 0; j < kChunk; ++j) a = fmaf(pw[j], kt[j][e], a);
      ksum[sidx * D + e] = a;
    }
    if (lane == 0) {
      ent[sidx] = H;
      if (lse) lse[sidx] = L;
    }
    __syncthreads();
  }
}

template <bool BF16, int D>
hipError_t launch_t(const Dims& dm, const void* K, const void* Ql, int c_begin, int c_end,
                    float* ksum, float* ent, float* lse, hipStream_t st) {
  dim3 grid(c_end - c_begin, dm.Hkv, dm.B);
  hipLaunchKernelGGL((k_summarize<BF16, D>), grid, dim3(kWave), 0, st, dm, K, Ql, c_begin, ksum,
                     ent, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_summarize(const Dims& dm, const void* K, const void* Ql, int c_begin, int c_end,
                            float* ksum, float* ent, float* lse_l, hipStream_t st) {
  if (c_end <= c_begin) return hipSuccess;
  if (dm.bf16) {
    return dm.d == 64 ? launch_t<true, 64>(dm, K, Ql, c_begin, c_end, ksum, ent, lse_l, st)
                      : launch_t<true, 128>(dm, K, Ql, c_begin, c_end, ksum, ent, lse_l, st);
  }
  return dm.d == 64 ? launch_t<false, 64>(dm, K, Ql, c_begin, c_end, ksum, ent, lse_l, st)
                    : launch_t<false, 128>(dm, K, Ql, c_begin, c_end, ksum, ent, lse_l, st);
}

}  // namespace hils
