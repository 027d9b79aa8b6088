// Landmark chunk summaries (note §5.1, Proposition 3.1; note §5.2 landmark token).
//
// bf16 storage: one wavefront per (batch, chunk, kv head) runs both contractions
// on matrix cores for every query head of the group at once (k_summarize_mfma).
// float32 storage: one workgroup per (batch, chunk, kv head) of NW (1, 2 or 4, at
// most G) wavefronts; the chunk's S = 64 keys are staged once in LDS and reused
// by the G query heads of the group, wavefront w taking heads w, w + NW, ...
// Lane j owns key j for the landmark logits and their softmax; lane e owns
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

// ------------------------------------------------------------------ bf16, matrix cores
// MFMA 16x16x32 bf16 lane layout (lane l, n = l % 16, q = l / 16):
//   A[m = n][k = 8q + j], B[k = 8q + j][n = n], D[m = 4q + r][n = n].
// Logits: S^T = K Ql^T with keys on M (four 16-key blocks kb), heads on N (16 per
// round, G used) and features on k, the K operand loaded straight from HBM into
// registers (lane (n, q) reads 16 bytes of key 16 kb + n). The result gives lane
// (n, q) the logits of head n for keys 16 kb + 4q + r, so a head's softmax is a
// reduction over a lane's 16 values and the four lanes n, n+16, n+32, n+48.
// Weighted key sum: ksum = P K with heads on M, features on N and the 64 keys on
// k, in two 32-key steps whose k-slots are ordered so that slot 8q + j is key
// 32 ks + 4q + j (j < 4) or 32 ks + 16 + 4q + j - 4 (j >= 4): exactly the
// probabilities lane (n, q) already holds, so P needs no data movement. P is
// float32; it enters as a two-term bf16 split p = hi + lo (the remainder is below
// 2^-17 p), so every product is exact and the sum is accumulated in float32. The
// K operand of this product has the keys along k, i.e. the chunk's keys
// transposed: the key tile goes through LDS once (row-major, the registers of
// the first product written out) and comes back by the LDS transpose read.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// x combined over the lanes n, n + 16, n + 32, n + 48 (v_permlane16/32_swap).
template <bool MAX>
__device__ __forceinline__ float xlanes4(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// LDS transpose read (ds_read_b64_tr_b16): in each group of 16 lanes, lane
// 4i + a supplies the address of four consecutive 16-bit elements, and lane
// 4a + e receives element e of the four lanes 4i + a, i = 0..3, in order of i.
__device__ __forceinline__ uint2 lds_tr16(const uint16_t* p) {
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
  uint2 u;
  __builtin_memcpy(&u, &r, 8);
  return u;
}

// B operand of the weighted key sum for 32-key step ks and features f0 .. f0 + 15
// from the row-major key tile kt (pitch P): lane (n, q) gets kt[key][f0 + n] for
// the keys of k-slots 8q .. 8q + 7 in the order above.
template <int P>
__device__ __forceinline__ uint4 key_colfrag(const uint16_t* kt, int ks, int f0) {
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const uint16_t* p = kt + (32 * ks + 4 * q + (n >> 2)) * P + f0 + 4 * (n & 3);
  const uint2 lo = lds_tr16(p), hi = lds_tr16(p + 16 * P);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

template <int D>
__global__ __launch_bounds__(kWave) void k_summarize_mfma(Dims dm, const uint16_t* __restrict__ K,
                                                         const uint16_t* __restrict__ Ql,
                                                         int c_begin, float* __restrict__ ksum,
                                                         float* __restrict__ ent,
                                                         float* __restrict__ lse) {
  constexpr int P = D + 8;  // LDS row pitch (bf16): 16-byte rows, transpose reads spread over banks
  __shared__ __align__(16) uint16_t kt[kChunk * P];
  const int c = c_begin + blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, n = lane & 15, q = lane >> 4;
  // keys: lane (n, q) holds K[16 kb + n][32 ds + 8 q .. + 8]; every load issued first
  const long long krow = (long long)dm.Hkv * D;
  const uint16_t* kb0 = K + (((long long)b * dm.Tcap + (long long)c * kChunk) * dm.Hkv + g) * D;
  uint4 ka[4][D / 32];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
      ka[kb][ds] = *reinterpret_cast<const uint4*>(kb0 + (16 * kb + n) * krow + 32 * ds + 8 * q);
  const long long s0 = ((long long)b * dm.NCcap + c) * dm.H + (long long)g * dm.G;
  auto ldql = [&](int h0, uint4* qb) {  // lane (n, q): Ql[head h0 + n][32 ds + 8 q .. + 8]
    const bool v = h0 + n < dm.G;
    const uint16_t* src = Ql + (s0 + (v ? h0 + n : 0)) * D + 8 * q;
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
      const uint4 x = *reinterpret_cast<const uint4*>(src + 32 * ds);
      qb[ds] = v ? x : make_uint4(0, 0, 0, 0);
    }
  };
  uint4 qb[D / 32];
  ldql(0, qb);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
      *reinterpret_cast<uint4*>(kt + (16 * kb + n) * P + 32 * ds + 8 * q) = ka[kb][ds];
  __syncthreads();

  for (int h0 = 0; h0 < dm.G; h0 += 16) {
    floatx4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < D / 32; ++ds)
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[kb][ds]), as_bf16x8(qb[ds]),
                                                        s[kb], 0, 0, 0);
    }
    if (h0 + 16 < dm.G) ldql(h0 + 16, qb);
    // softmax of head h0 + n over its 64 keys, its log-sum-exp and entropy, in
    // the log2 domain (t_j = s'_j log2 e), so each exponential is one hardware exp2
    const float sc2 = dm.scale * kLog2e;
    float m2 = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[kb][r] *= sc2;
        m2 = fmaxf(m2, s[kb][r]);
      }
    m2 = xlanes4<true>(m2);
    float z = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) z += __builtin_amdgcn_exp2f(s[kb][r] - m2);
    const float L2 = m2 + __builtin_amdgcn_logf(xlanes4<false>(z));  // log-sum-exp / ln 2
    float hs = 0.f;
    bf16x8 phi[2], plo[2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float d2 = L2 - s[kb][r];  // >= 0
        const float p = __builtin_amdgcn_exp2f(-d2);  // p'_j
        hs = fmaf(p, d2, hs);                         // -p log2 p
        const __bf16 hi = (__bf16)p;
        phi[kb >> 1][(kb & 1) * 4 + r] = hi;
        plo[kb >> 1][(kb & 1) * 4 + r] = (__bf16)(p - (float)hi);
      }
    const float H = xlanes4<false>(hs) * kLn2;
    const float L = L2 * kLn2;
    const int h = h0 + n;
    if (q == 0 && h < dm.G) {
      ent[s0 + h] = H;
      if (lse) lse[s0 + h] = L;
    }
    // ksum of head h0 + 4q + r, features 16 fb + n
#pragma unroll
    for (int fb = 0; fb < D / 16; ++fb) {
      floatx4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 kf = as_bf16x8(key_colfrag<P>(kt, ks, 16 * fb));
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi[ks], kf, o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo[ks], kf, o, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int hr = h0 + 4 * q + r;
        if (hr < dm.G) ksum[(s0 + hr) * D + 16 * fb + n] = o[r];
      }
    }
  }
}

template <bool BF16, int D>
hipError_t launch_t(const Dims& dm, const void* K, const void* Ql, int c_begin, int c_end,
                    float* ksum, float* ent, float* lse, hipStream_t st) {
  dim3 grid(c_end - c_begin, dm.Hkv, dm.B);
  if constexpr (BF16) {
    hipLaunchKernelGGL((k_summarize_mfma<D>), grid, dim3(kWave), 0, st, dm,
                       static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(Ql), c_begin,
                       ksum, ent, lse);
  } else {
    // float32: one wavefront per query head of the group, at most four
    if (dm.G >= 4)
      hipLaunchKernelGGL((k_summarize<false, D, 4>), grid, dim3(4 * kWave), 0, st, dm, K, Ql,
                         c_begin, ksum, ent, lse);
    else if (dm.G >= 2)
      hipLaunchKernelGGL((k_summarize<false, D, 2>), grid, dim3(2 * kWave), 0, st, dm, K, Ql,
                         c_begin, ksum, ent, lse);
    else
      hipLaunchKernelGGL((k_summarize<false, D, 1>), grid, dim3(kWave), 0, st, dm, K, Ql, c_begin,
                         ksum, ent, lse);
  }
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
