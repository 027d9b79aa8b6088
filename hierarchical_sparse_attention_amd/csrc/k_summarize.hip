// Landmark chunk summaries (note §5.1, Proposition 3.1; note §5.2 landmark token).
//
// One workgroup per (batch, chunk, kv head) of NW (1, 2 or 4, at most G) wavefronts: the
// chunk's S = 64 keys are staged once in LDS (one coalesced pass over HBM) and
// reused by the G query heads of the group, wavefront w taking heads w, w + NW,
// ... Lane j owns key j for the landmark logits and their softmax; lane e owns
// feature e for the weighted key sum.
#include "hils_internal.h"

namespace hils {
namespace {

// Sum or maximum over the 64 lanes with DPP row permutations (quad swaps, then
// the half-row and row mirrors) and the permlane swaps between rows and halves,
// with no LDS round trip. Every lane ends with the same value: each step
// combines a lane's value with its partner's by a commutative operation.
template <bool MAX>
__device__ __forceinline__ float wave_all(float v) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)));
  v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)));
  v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true)));
  v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true)));
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

template <bool BF16, int D, int NW>
__global__ __launch_bounds__(NW * kWave) void k_summarize(Dims dm, const void* __restrict__ K,
                                                                 const void* __restrict__ Ql,
                                                                 int c_begin,
                                                                 float* __restrict__ ksum,
                                                                 float* __restrict__ ent,
                                                                 float* __restrict__ lse) {
  __shared__ float kt[kChunk][D + 1];  // +1 pad: lane-per-row reads hit distinct banks
  __shared__ float qs[NW][D];
  __shared__ float pw[NW][kChunk];
  const int c = c_begin + blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1), w = NW == 1 ? 0 : threadIdx.x / kWave;

  constexpr int VE = BF16 ? 8 : 4;  // elements per 16-byte vector
  constexpr int VPR = D / VE;       // vectors per key row
  constexpr int NV = kChunk * VPR / kWave;  // vectors per lane of one wavefront
  static_assert(kChunk * VPR % kWave == 0 && D % kWave == 0, "tile shape");
  // the landmark query of the wavefront's first head is requested with the
  // keys; each later head's while the previous head is being summarised (the
  // head index is clamped, so the load needs no branch)
  constexpr int QE = D / kWave;
  auto ldql = [&](int hh, float* q) {
    const long long sidx = ((long long)b * dm.NCcap + c) * dm.H + g * dm.G + hh;
#pragma unroll
    for (int k = 0; k < QE; ++k) q[k] = load_elem<BF16>(Ql, sidx * D + lane + k * kWave);
  };
  float qn[QE];
  ldql(min(w, dm.G - 1), qn);
  // the chunk's keys: the NW wavefronts split the 16-byte pieces (vector v of
  // the tile goes to wavefront v % NW); every load is issued before any is used
  uint4 raw[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = lane + i * kWave;
    const int j = v / VPR, col = (v % VPR) * VE;
    const long long off =
        (((long long)b * dm.Tcap + (long long)c * kChunk + j) * dm.Hkv + g) * D + col;
    if (i % NW == w)
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
    if (i % NW != w) continue;
    const int v = lane + i * kWave;
    const int j = v / VPR, col = (v % VPR) * VE;
    const uint32_t wd[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (BF16) {
        kt[j][col + 2 * k] = __uint_as_float(wd[k] << 16);
        kt[j][col + 2 * k + 1] = __uint_as_float(wd[k] & 0xFFFF0000u);
      } else {
        kt[j][col + k] = __uint_as_float(wd[k]);
      }
    }
  }
  __syncthreads();

  // the wavefronts take the heads in rounds; a wavefront past the last head of
  // a round still reaches its barriers (the count is uniform per round)
  for (int h0 = 0; h0 < dm.G; h0 += NW) {
    const int hh = h0 + w;
    const bool act = hh < dm.G;
    const int h = g * dm.G + min(hh, dm.G - 1);
    const long long sidx = ((long long)b * dm.NCcap + c) * dm.H + h;
#pragma unroll
    for (int k = 0; k < QE; ++k) qs[w][lane + k * kWave] = qn[k];
    ldql(min(hh + NW, dm.G - 1), qn);
    __syncthreads();
    // four interleaved partial sums keep the dependent chains short
    float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int e = 0; e < D; e += 4)
#pragma unroll
      for (int u = 0; u < 4; ++u) a4[u] = fmaf(qs[w][e + u], kt[lane][e + u], a4[u]);
    const float s = ((a4[0] + a4[1]) + (a4[2] + a4[3])) * dm.scale;  // landmark logit s'_j
    const float m = wave_all<true>(s);
    const float L = m + logf(wave_all<false>(expf(s - m)));  // log-sum-exp
    const float p = expf(s - L);                              // p'_j
    const float H = wave_all<false>(p * (L - s));             // -sum p log p, terms >= 0
    pw[w][lane] = p;
    __syncthreads();
    if (act) {
      for (int e = lane; e < D; e += kWave) {
        float b4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int j = 0; j < kChunk; j += 4)
#pragma unroll
          for (int u = 0; u < 4; ++u) b4[u] = fmaf(pw[w][j + u], kt[j + u][e], b4[u]);
        ksum[sidx * D + e] = (b4[0] + b4[1]) + (b4[2] + b4[3]);
      }
      if (lane == 0) {
        ent[sidx] = H;
        if (lse) lse[sidx] = L;
      }
    }
    __syncthreads();
  }
}

template <bool BF16, int D>
hipError_t launch_t(const Dims& dm, const void* K, const void* Ql, int c_begin, int c_end,
                    float* ksum, float* ent, float* lse, hipStream_t st) {
  dim3 grid(c_end - c_begin, dm.Hkv, dm.B);
  // one wavefront per query head of the group, at most four
  if (dm.G >= 4)
    hipLaunchKernelGGL((k_summarize<BF16, D, 4>), grid, dim3(4 * kWave), 0, st, dm, K, Ql, c_begin,
                       ksum, ent, lse);
  else if (dm.G >= 2)
    hipLaunchKernelGGL((k_summarize<BF16, D, 2>), grid, dim3(2 * kWave), 0, st, dm, K, Ql, c_begin,
                       ksum, ent, lse);
  else
    hipLaunchKernelGGL((k_summarize<BF16, D, 1>), grid, dim3(kWave), 0, st, dm, K, Ql, c_begin,
                       ksum, ent, lse);
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
