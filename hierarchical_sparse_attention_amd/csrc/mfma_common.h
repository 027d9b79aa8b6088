// Matrix-core chunk scoring shared by the prefill, decode-split and fused decode
// kernels. The summary key k'_c is float32; with q exactly bf16 the dot product
// runs on bf16 MFMAs from a two-term split k' = hi + lo (hi = bf16(k'),
// lo = bf16(k' - hi)). Every (row, chunk) element goes through the same MFMA
// sequence in every kernel, so all of them produce bit-identical scores.
#pragma once

#include "hils_internal.h"

namespace hils {
namespace mf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// hi/lo split of 8 float32 values into two bf16x8 fragments (round to nearest even).
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 h = (__bf16)x[j];
    hi[j] = h;
    lo[j] = (__bf16)(x[j] - (float)h);
  }
}

// Score accumulation for one 16x16 block: sum_ds q.hi + q.lo, fixed order.
template <int D>
__device__ __forceinline__ floatx4 score_block(const uint4* qa, const bf16x8* hi, const bf16x8* lo) {
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[ds]), hi[ds], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[ds]), lo[ds], acc, 0, 0, 0);
  }
  return acc;
}


// Scores of the 32 NW candidates cbase .. of query row r (one row of Q, the
// kv-group-free per-head layout) into ss[0 .. 32 NW): a workgroup of NW
// wavefronts, wavefront w scoring 32 candidates as two 16 x 16 MFMA blocks with
// the row in M position 0. Candidates at or beyond n score -inf. Every global
// read is issued up front and unconditionally (invalid chunks read chunk 0 and
// are discarded), so they share one round trip.
template <int D, int NW>
__device__ __forceinline__ void split_scores(const Dims& dm, const uint16_t* __restrict__ Q,
                                             const float* __restrict__ ksum,
                                             const float* __restrict__ ent, long long r, int n,
                                             int cbase, float* ss) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, c = lane & 15, g = lane >> 4;
  const int h = (int)(r % dm.H), b = (int)(r / ((long long)dm.H * dm.Tq));
  constexpr int NBW = 2;  // 16-candidate blocks per wavefront
  uint4 qraw[D / 32];
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds)
    qraw[ds] = *reinterpret_cast<const uint4*>(Q + r * D + 32 * ds + 8 * g);
  float4 raw[NBW][D / 32][2];
  float ev[NBW];
#pragma unroll
  for (int q = 0; q < NBW; ++q) {
    const int chunk = cbase + 16 * (NBW * w + q) + c;
    const long long row = ((long long)b * dm.NCcap + (chunk < n ? chunk : 0)) * dm.H + h;
    const float* src = ksum + row * D;
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
      raw[q][ds][0] = *reinterpret_cast<const float4*>(src + 32 * ds + 8 * g);
      raw[q][ds][1] = *reinterpret_cast<const float4*>(src + 32 * ds + 8 * g + 4);
    }
    ev[q] = ent[row];
  }
  uint4 qa[D / 32];  // the row sits in M position 0 (lanes with c == 0)
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) qa[ds] = c == 0 ? qraw[ds] : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int q = 0; q < NBW; ++q) {
    const int nb = NBW * w + q;
    const int chunk = cbase + 16 * nb + c;
    const bool cv = chunk < n;
    bf16x8 hi[D / 32], lo[D / 32];
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
      const float4 a = raw[q][ds][0], bb = raw[q][ds][1];
      float v[8] = {a.x, a.y, a.z, a.w, bb.x, bb.y, bb.z, bb.w};
      if (!cv) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.f;
      }
      split8(v, hi[ds], lo[ds]);
    }
    const floatx4 acc = score_block<D>(qa, hi, lo);
    if (g == 0) ss[16 * nb + c] = cv ? fmaf(acc[0], dm.scale, ev[q]) : -INFINITY;
  }
}

// Local top-K of the nvalid scores in ss (candidate cbase + x in slot x, 16-byte
// aligned; slots past nvalid hold -inf), two threads per candidate (2 SPLIT
// threads, every one calls this; reads of ss ordered after its writes): thread t
// counts the entries of half t / SPLIT of the split that come before candidate
// t % SPLIT in (score desc, chunk asc) order, the second half's counts pass
// through part (SPLIT ints of LDS), and a candidate whose rank is below K is
// written to slot `rank` of the list at ws_s / ws_i.
template <int SPLIT>
__device__ __forceinline__ void split_local_topk_halves(const float* ss, int* part, int nvalid,
                                                        int cbase, int K,
                                                        float* __restrict__ ws_s,
                                                        int* __restrict__ ws_i) {
  const int t = threadIdx.x, x = t % SPLIT, half = t / SPLIT;
  const float sv = ss[x];
  int rank = 0;
  const int y0 = half * (SPLIT / 2);
  const float4* s4 = reinterpret_cast<const float4*>(ss + y0);
  float4 v[SPLIT / 8];
#pragma unroll
  for (int j = 0; j < SPLIT / 8; ++j) v[j] = s4[j];
#pragma unroll
  for (int j = 0; j < SPLIT / 8; ++j) {
    const int y = y0 + 4 * j;
    rank += topk_before(v[j].x, y, sv, x) + topk_before(v[j].y, y + 1, sv, x) +
            topk_before(v[j].z, y + 2, sv, x) + topk_before(v[j].w, y + 3, sv, x);
  }
  if (half == 1) part[x] = rank;
  __syncthreads();
  if (half == 0 && x < nvalid) {
    rank += part[x];
    if (rank < K) {
      ws_s[rank] = sv;
      ws_i[rank] = cbase + x;
    }
  }
}

}  // namespace mf
}  // namespace hils
