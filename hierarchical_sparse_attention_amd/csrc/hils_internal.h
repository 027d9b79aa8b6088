// Internal declarations shared by the HIP kernels and the C-ABI host layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hils {

constexpr int kWave = 64;   // CDNA wavefront width
constexpr int kChunk = 64;  // supported chunk size S (one key per lane)

// Dimensions after validation and defaulting (see hils_dims in hils.h).
struct Dims {
  int B, Tq, Tkv, Tcap, NCcap, H, Hkv, G, d, S, K;
  bool bf16;
  long long q_pos0;
  float scale;
};

// ---------------------------------------------------------------- numerics
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t v16) {
  return __uint_as_float(v16 << 16);
}

// float32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, long long i) {
  if constexpr (BF16) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  } else {
    return reinterpret_cast<const float*>(p)[i];
  }
}

template <bool BF16>
__device__ __forceinline__ void store_elem(void* p, long long i, float v) {
  if constexpr (BF16) {
    reinterpret_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(v);
  } else {
    reinterpret_cast<float*>(p)[i] = v;
  }
}

// Load N consecutive elements starting at element offset `off` (16-byte aligned)
// into float registers with 16-byte vector loads.
template <bool BF16, int N>
__device__ __forceinline__ void load_row(const void* base, long long off, float* out) {
  if constexpr (BF16) {
    static_assert(N % 8 == 0, "bf16 rows load 8 elements per vector");
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int v = 0; v < N / 8; ++v) {
      uint4 w = p[v];
      uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        out[v * 8 + 2 * k] = __uint_as_float(ws[k] << 16);
        out[v * 8 + 2 * k + 1] = __uint_as_float(ws[k] & 0xFFFF0000u);
      }
    }
  } else {
    static_assert(N % 4 == 0, "f32 rows load 4 elements per vector");
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
#pragma unroll
    for (int v = 0; v < N / 4; ++v) {
      float4 w = p[v];
      out[4 * v] = w.x; out[4 * v + 1] = w.y; out[4 * v + 2] = w.z; out[4 * v + 3] = w.w;
    }
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Chunk score s^ = scale * (q . kbar) + ent in float32 with a fixed operation
// order (sequential fused multiply-adds over the head dimension), shared by
// every scoring kernel so that all of them produce bit-identical scores.
template <int D>
__device__ __forceinline__ float chunk_score(const float* q, const float* kbar, float scale,
                                             float ent) {
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < D; ++e) acc = fmaf(q[e], kbar[e], acc);
  return fmaf(acc, scale, ent);
}

// ---------------------------------------------------------------- launches
hipError_t launch_summarize(const Dims& dm, const void* K, const void* Ql, int c_begin, int c_end,
                            float* ksum, float* ent, float* lse_l, hipStream_t st);

size_t score_topk_ws_bytes(const Dims& dm);
size_t score_mfma_prefill_ws_bytes(const Dims& dm);
hipError_t launch_score_mfma_prefill(const Dims& dm, const void* Q, const float* ksum,
                                     const float* ent, int32_t* idx, float* score, void* ws,
                                     hipStream_t st);
hipError_t launch_score_mfma_split(const Dims& dm, const void* Q, const float* ksum,
                                   const float* ent, float* ws_s, int* ws_i, int nsplit,
                                   hipStream_t st);
hipError_t launch_score_topk(const Dims& dm, const void* Q, const float* ksum, const float* ent,
                             int32_t* idx, float* score, void* ws, hipStream_t st);

size_t attend_ws_bytes(const Dims& dm);
size_t attend_mfma_ws_bytes(const Dims& dm);
bool attend_mfma_try(const Dims& dm, const void* Q, const void* K, const void* V,
                     const int32_t* idx, const float* score, void* O, float* lse_own,
                     float* lse_tot, void* ws, hipStream_t st, hipError_t* err);
hipError_t launch_attend_fuse(const Dims& dm, const void* Q, const void* K, const void* V,
                              const int32_t* idx, const float* score, void* O, float* lse_own,
                              float* lse_tot, void* ws, hipStream_t st);

size_t backward_ws_bytes(const Dims& dm);
hipError_t launch_backward(const Dims& dm, const void* Q, const void* K, const void* V,
                           const void* Ql, const float* ksum, const float* ent, const float* lse_l,
                           const int32_t* idx, const float* score, const float* lse_tot,
                           const void* dO, void* dQ, void* dK, void* dV, void* dQl, void* ws,
                           hipStream_t st);

}  // namespace hils
