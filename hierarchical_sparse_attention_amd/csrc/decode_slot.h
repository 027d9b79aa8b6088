// Shared by the decode attention kernels (slot kernel, fused decode step): one
// wavefront computes the softmax attention of one query row over the keys of one
// chunk (or a part of it) and returns the normalised output and log-mass.
#pragma once

#include "hils_internal.h"

namespace hils {
namespace dec {

__device__ __forceinline__ float lane_bcast(float v, int j) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}

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

}  // namespace dec
}  // namespace hils
