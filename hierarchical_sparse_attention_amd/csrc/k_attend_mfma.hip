// Prefill intra-chunk attention + inter-chunk fusion on bf16 MFMA (gfx950).
//
// Same arithmetic as the rows kernel (note §5.3 hierarchical softmax; Tide
// Fig. 3), organised for matrix cores and K/V reuse:
//  * A workgroup owns R rows (Rq consecutive query positions x the G query heads
//    of one kv head). Their selections are counting-sorted in LDS into one row
//    list per chunk.
//  * The workgroup sweeps the union of selected chunks in ascending order. Each
//    chunk's 64 keys and values are staged once in LDS (double-buffered; V is
//    stored transposed) and shared by every row that selected the chunk: the
//    rows are packed into 16-row MFMA tiles, so the work done is exactly the
//    (row, chunk) pairs the selection asks for.
//  * Per tile: S^T = K Q^T (v_mfma_f32_16x16x32_bf16, keys on M, rows on N), a
//    column softmax over the chunk's 64 keys, then O^T = V^T P'^T where P'
//    already carries the fusion weight exp(s^ - Lambda) / Z. The fp32 row
//    accumulators live in LDS; a per-chunk barrier orders the updates, so each
//    row sums its chunks in ascending chunk order (deterministic output).
//  * The causal own chunk is processed first (normalised), which yields its
//    log-mass; Lambda follows per row and rescales the own-chunk contribution.
//
// MFMA 16x16x32 bf16 lane layout (lane l, g = l/16, c = l%16):
//   A[m = c][k = 8g + j], B[k = 8g + j][n = c], D[m = 4g + r][n = c].
// S^T tile kb gives lane l keys 16kb + 4g + r of row c; for the P V product the
// 32 keys of step ks are ordered so that k-slot 8g + j holds key 32ks + 4g + j
// (j < 4) or 32ks + 16 + 4g + (j - 4) (j >= 4): exactly the S^T values the lane
// already holds, so P' needs no data movement, and V^T is read with the same
// key order.
#include "hils_internal.h"

namespace hils {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct Cfg {
  static constexpr int RMAX = D == 64 ? 256 : 128;  // rows per workgroup
  static constexpr int KP = D + 8;                  // K tile row pitch (bf16)
  static constexpr int VP = kChunk + 8;             // V^T tile row pitch (bf16)
  static constexpr int AP = D + 4;                  // accumulator row pitch (f32)
  static constexpr int KT = kChunk * KP;            // bf16 per K tile
  static constexpr int VT = D * VP;                 // bf16 per V^T tile
  static constexpr int KU = kChunk * D / 8 / 256;   // 16-byte K loads per thread per chunk
  static constexpr int VU = 32 * (D / 8) / 256;     // (key pair, 8 features) units per thread
};

struct Smem {
  float* acc;
  uint16_t* kb;  // two K tiles, KT apart
  uint16_t* vb;  // two V^T tiles, VT apart
  uint32_t* ent;
  int* cnt;
  int* off;
  int* cur;
  int* nz;
  float* lown;
  float* lam;
  int* misc;
};

template <int D>
__host__ __device__ inline size_t smem_bytes(int R, int K, int ncr) {
  using C = Cfg<D>;
  size_t b = 0;
  b += (size_t)R * C::AP * 4;
  b += 2 * (size_t)C::KT * 2 + 2 * (size_t)C::VT * 2;
  b += (size_t)R * K * 4;
  b += 4 * (size_t)(ncr + 1) * 4;
  b += 2 * (size_t)R * 4;
  b += 16 * 4;
  return b;
}

template <int D>
__device__ __forceinline__ Smem carve(char* base, int R, int K, int ncr) {
  using C = Cfg<D>;
  Smem s;
  s.acc = reinterpret_cast<float*>(base);
  base += (size_t)R * C::AP * 4;
  s.kb = reinterpret_cast<uint16_t*>(base);
  base += 2 * C::KT * 2;
  s.vb = reinterpret_cast<uint16_t*>(base);
  base += 2 * C::VT * 2;
  s.ent = reinterpret_cast<uint32_t*>(base);
  base += (size_t)R * K * 4;
  s.cnt = reinterpret_cast<int*>(base); base += (ncr + 1) * 4;
  s.off = reinterpret_cast<int*>(base); base += (ncr + 1) * 4;
  s.cur = reinterpret_cast<int*>(base); base += (ncr + 1) * 4;
  s.nz = reinterpret_cast<int*>(base); base += (ncr + 1) * 4;
  s.lown = reinterpret_cast<float*>(base); base += R * 4;
  s.lam = reinterpret_cast<float*>(base); base += R * 4;
  s.misc = reinterpret_cast<int*>(base);
  return s;
}

// In-place exclusive scan of n ints with 256 threads; returns the total.
__device__ __forceinline__ int block_exclusive_scan(int* a, int n, int* scratch) {
  const int t = threadIdx.x;
  const int seg = (n + 255) / 256;
  const int lo = min(n, t * seg), hi = min(n, lo + seg);
  int s = 0;
  for (int x = lo; x < hi; ++x) s += a[x];
  // inclusive scan of the 256 segment sums: per wave, then across the 4 waves
  const int lane = t & 63, w = t >> 6;
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) scratch[w] = incl;
  __syncthreads();
  int before = 0;
  for (int x = 0; x < w; ++x) before += scratch[x];
  const int total = scratch[0] + scratch[1] + scratch[2] + scratch[3];
  int run = before + incl - s;
  for (int x = lo; x < hi; ++x) {
    const int v = a[x];
    a[x] = run;
    run += v;
  }
  __syncthreads();
  return total;
}

// Load one chunk's K (row-major) and V (to be transposed) into registers.
template <int D>
struct Stage {
  uint4 k[Cfg<D>::KU];
  uint4 v[2 * Cfg<D>::VU];
};

template <int D>
__device__ __forceinline__ void stage_load(Stage<D>& st, const uint16_t* K, const uint16_t* V,
                                  long long kv_base, long long kv_stride, long long key0,
                                  long long Tkv) {
  const int t = threadIdx.x;
#pragma unroll
  for (int x = 0; x < Cfg<D>::KU; ++x) {
    const int u = t + 256 * x;
    const int j = u / (D / 8), c8 = u % (D / 8);
    const long long row = key0 + j;
    st.k[x] = row < Tkv ? *reinterpret_cast<const uint4*>(K + kv_base + row * kv_stride + c8 * 8)
                        : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int x = 0; x < Cfg<D>::VU; ++x) {
    const int u = t + 256 * x;
    const int m = u % 32, dc = u / 32;
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const long long row = key0 + 2 * m + y;
      st.v[2 * x + y] = row < Tkv
                            ? *reinterpret_cast<const uint4*>(V + kv_base + row * kv_stride + dc * 8)
                            : make_uint4(0, 0, 0, 0);
    }
  }
}

template <int D>
__device__ __forceinline__ void stage_store(const Stage<D>& st, uint16_t* kb, uint16_t* vb) {
  using C = Cfg<D>;
  const int t = threadIdx.x;
#pragma unroll
  for (int x = 0; x < C::KU; ++x) {
    const int u = t + 256 * x;
    const int j = u / (D / 8), c8 = u % (D / 8);
    *reinterpret_cast<uint4*>(kb + j * C::KP + c8 * 8) = st.k[x];
  }
#pragma unroll
  for (int x = 0; x < C::VU; ++x) {
    const int u = t + 256 * x;
    const int m = u % 32, dc = u / 32;
    const uint4 a = st.v[2 * x], b = st.v[2 * x + 1];
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
    uint32_t* dst = reinterpret_cast<uint32_t*>(vb + (dc * 8) * C::VP + 2 * m);
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      // features 2*e2 and 2*e2+1 of keys 2m (low halves) and 2m+1 (high halves)
      dst[(2 * e2) * (C::VP / 2)] = (aw[e2] & 0xFFFFu) | (bw[e2] << 16);
      dst[(2 * e2 + 1) * (C::VP / 2)] = (aw[e2] >> 16) | (bw[e2] & 0xFFFF0000u);
    }
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// One 16-row tile against the staged chunk. Lane column c = lane%16 holds row
// `rho` (or none when !valid). mode 0: own chunk (causal, normalised, writes the
// accumulator and returns the log-mass); mode 1: selected chunk (adds
// weight * normalised output; lw = s^ - Lambda).
template <int D>
__device__ __forceinline__ float tile_pass(const uint16_t* kb, const uint16_t* vb, float* acc,
                                  const uint16_t* Q, long long qrow_off, bool valid, int rho,
                                  int nvalid_keys, float scale2, float lw, bool own_mode) {
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
  // B operand: Q^T fragments for this lane's row
  bf16x8 qf[D / 32];
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    uint4 u = valid ? *reinterpret_cast<const uint4*>(Q + qrow_off + 32 * ds + 8 * g)
                    : make_uint4(0, 0, 0, 0);
    qf[ds] = as_bf16x8(u);
  }
  floatx4 s[4];
#pragma unroll
  for (int kbk = 0; kbk < 4; ++kbk) {
    s[kbk] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
      const uint4 a = *reinterpret_cast<const uint4*>(kb + (16 * kbk + c) * C::KP + 32 * ds + 8 * g);
      s[kbk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), qf[ds], s[kbk], 0, 0, 0);
    }
  }
  // column softmax over the chunk's keys (log2 domain)
  float m = -INFINITY;
#pragma unroll
  for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 16 * kbk + 4 * g + r;
      float v = s[kbk][r] * scale2;
      if (key >= nvalid_keys) v = -INFINITY;
      s[kbk][r] = v;
      m = fmaxf(m, v);
    }
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  if (m == -INFINITY) m = 0.f;  // empty column (padding lane): keeps every value finite
  float z = 0.f;
#pragma unroll
  for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = exp2f(s[kbk][r] - m);
      s[kbk][r] = e;
      z += e;
    }
  z += __shfl_xor(z, 16, 64);
  z += __shfl_xor(z, 32, 64);
  const float f = (valid && z > 0.f) ? (own_mode ? 1.0f / z : expf(lw) / z) : 0.0f;
  bf16x8 pf[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pf[ks][j] = (__bf16)(s[2 * ks][j] * f);
      pf[ks][4 + j] = (__bf16)(s[2 * ks + 1][j] * f);
    }
  // O^T = V^T P'^T, 16 features per block
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    floatx4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint16_t* vrow = vb + (16 * db + c) * C::VP + 32 * ks + 4 * g;
      uint4 a;
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
      a.x = lo.x; a.y = lo.y; a.z = hi.x; a.w = hi.y;
      o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), pf[ks], o, 0, 0, 0);
    }
    if (valid) {
      float4* dst = reinterpret_cast<float4*>(acc + rho * C::AP + 16 * db + 4 * g);
      if (own_mode) {
        *dst = make_float4(o[0], o[1], o[2], o[3]);
      } else {
        float4 v = *dst;
        v.x += o[0]; v.y += o[1]; v.z += o[2]; v.w += o[3];
        *dst = v;
      }
    }
  }
  return (m + log2f(z)) * kLn2;  // natural-log mass of the column (own mode)
}

template <int D>
__global__ __launch_bounds__(256) void k_attend_mfma(Dims dm, int R, int Rq, int ncr_cap,
                                                     const uint16_t* __restrict__ Q,
                                                     const uint16_t* __restrict__ K,
                                                     const uint16_t* __restrict__ V,
                                                     const int32_t* __restrict__ idx,
                                                     const float* __restrict__ score,
                                                     uint16_t* __restrict__ O,
                                                     float* __restrict__ lse_own,
                                                     float* __restrict__ lse_tot) {
  using C = Cfg<D>;
  extern __shared__ __align__(16) char smem_raw[];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, col = lane & 15;
  const int G = dm.G, Ksel = dm.K, S = dm.S;
  const int qi0 = blockIdx.x * Rq, g = blockIdx.y, b = blockIdx.z;
  const int nq = min(Rq, dm.Tq - qi0);
  const int Rv = nq * G;
  const long long p0 = dm.q_pos0 + qi0;
  const int own_first = (int)(p0 / S), own_last = (int)((p0 + nq - 1) / S);
  const int ncr = own_last;  // selectable chunks: [0, own_last)
  Smem sm = carve<D>(smem_raw, R, Ksel, ncr_cap);
  const long long kv_stride = (long long)dm.Hkv * D;
  const long long kv_base = ((long long)b * dm.Tcap * dm.Hkv + g) * D;
  const float scale2 = dm.scale * kLog2e;
  auto row_of = [&](int rho) -> long long {
    return (((long long)b * dm.Tq + qi0 + rho / G) * dm.H + (long long)g * G + rho % G);
  };

  // ---- per-chunk row lists (counting sort of the selections)
  for (int c = t; c <= ncr; c += 256) sm.cnt[c] = 0;
  __syncthreads();
  for (int rho = t; rho < Rv; rho += 256) {
    const long long r = row_of(rho);
    const int own = (int)((p0 + rho / G) / S);
    for (int k = 0; k < Ksel; ++k) {
      const int c = idx[r * Ksel + k];
      if (c >= 0 && c < own) atomicAdd(&sm.cnt[c], 1);
    }
  }
  __syncthreads();
  for (int c = t; c < ncr; c += 256) {
    sm.off[c] = sm.cnt[c];
    sm.nz[c] = sm.cnt[c] > 0 ? 1 : 0;
  }
  __syncthreads();
  block_exclusive_scan(sm.off, ncr, sm.misc);
  const int nnz = block_exclusive_scan(sm.nz, ncr, sm.misc + 4);
  for (int c = t; c < ncr; c += 256) sm.cur[c] = sm.off[c];
  __syncthreads();
  for (int rho = t; rho < Rv; rho += 256) {
    const long long r = row_of(rho);
    const int own = (int)((p0 + rho / G) / S);
    for (int k = 0; k < Ksel; ++k) {
      const int c = idx[r * Ksel + k];
      if (c >= 0 && c < own) {
        const int p = atomicAdd(&sm.cur[c], 1);
        sm.ent[p] = (uint32_t)rho | ((uint32_t)k << 16);
      }
    }
  }
  __syncthreads();
  // compacted list of non-empty chunks (fill cursors are no longer needed):
  // chunk c goes to slot nz[c], the exclusive count of non-empty chunks below it
  for (int c = t; c < ncr; c += 256)
    if (sm.cnt[c] > 0) sm.cur[sm.nz[c]] = c;
  __syncthreads();

  // ---- own chunks (causal, normalised)
  Stage<D> st;
  for (int oc = own_first; oc <= own_last; ++oc) {
    stage_load<D>(st, K, V, kv_base, kv_stride, (long long)oc * S, dm.Tkv);
    stage_store<D>(st, sm.kb, sm.vb);
    __syncthreads();
    const int ra = (int)max(0LL, (long long)oc * S - p0) * G;
    const int rb = (int)min((long long)Rv, ((long long)oc * S + S - p0) * G);
    const int ntile = (rb - ra + 15) / 16;
    for (int tl = w; tl < ntile; tl += 4) {
      const int rho = ra + 16 * tl + col;
      const bool valid = rho < rb;
      const long long r = valid ? row_of(rho) : 0;
      const int nk = valid ? (int)(p0 + rho / G - (long long)oc * S) + 1 : 0;
      const float lo = tile_pass<D>(sm.kb, sm.vb, sm.acc, Q, r * D, valid, rho, nk,
                                    scale2, 0.f, true);
      if (valid && lane < 16) sm.lown[rho] = lo;
    }
    __syncthreads();
  }

  // ---- fusion normaliser per row; rescale the own-chunk contribution
  for (int rho = t; rho < Rv; rho += 256) {
    const long long r = row_of(rho);
    const float lo = sm.lown[rho];
    float mx = lo;
    for (int k = 0; k < Ksel; ++k) mx = fmaxf(mx, score[r * Ksel + k]);
    float z = expf(lo - mx);
    for (int k = 0; k < Ksel; ++k) z += expf(score[r * Ksel + k] - mx);
    const float lam = mx + logf(z);
    sm.lam[rho] = lam;
    const float a = expf(lo - lam);
    float* ar = sm.acc + rho * C::AP;
    for (int e = 0; e < D; e += 4) {
      float4 v = *reinterpret_cast<float4*>(ar + e);
      v.x *= a; v.y *= a; v.z *= a; v.w *= a;
      *reinterpret_cast<float4*>(ar + e) = v;
    }
    if (lse_own) lse_own[r] = lo;
    if (lse_tot) lse_tot[r] = lam;
  }
  __syncthreads();

  // ---- selected chunks, ascending, K/V double-buffered
  if (nnz > 0) {
    stage_load<D>(st, K, V, kv_base, kv_stride, (long long)sm.cur[0] * S, dm.Tkv);
    stage_store<D>(st, sm.kb, sm.vb);
  }
  __syncthreads();
  for (int u = 0; u < nnz; ++u) {
    const int c = sm.cur[u];
    const int buf = u & 1;
    if (u + 1 < nnz) stage_load<D>(st, K, V, kv_base, kv_stride, (long long)sm.cur[u + 1] * S, dm.Tkv);
    const int e0 = sm.off[c], n = sm.cnt[c];
    const int ntile = (n + 15) / 16;
    for (int tl = w; tl < ntile; tl += 4) {
      const int e = 16 * tl + col;
      const bool valid = e < n;
      const uint32_t en = valid ? sm.ent[e0 + e] : 0u;
      const int rho = (int)(en & 0xFFFFu), k = (int)(en >> 16);
      const long long r = valid ? row_of(rho) : 0;
      const float lw = valid ? score[r * Ksel + k] - sm.lam[rho] : 0.f;
      tile_pass<D>(sm.kb + buf * C::KT, sm.vb + buf * C::VT, sm.acc, Q, r * D, valid, rho, kChunk, scale2, lw,
                   false);
    }
    if (u + 1 < nnz) stage_store<D>(st, sm.kb + (buf ^ 1) * C::KT, sm.vb + (buf ^ 1) * C::VT);
    __syncthreads();
  }

  // ---- write O (bf16, round to nearest even)
  for (int x = t; x < Rv * (D / 8); x += 256) {
    const int rho = x / (D / 8), c8 = x % (D / 8);
    const float* ar = sm.acc + rho * C::AP + c8 * 8;
    uint4 o;
    uint32_t* ow = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
    for (int y = 0; y < 4; ++y)
      ow[y] = (uint32_t)f32_to_bf16_bits(ar[2 * y]) | ((uint32_t)f32_to_bf16_bits(ar[2 * y + 1]) << 16);
    *reinterpret_cast<uint4*>(O + row_of(rho) * D + c8 * 8) = o;
  }
}

template <int D>
bool plan(const Dims& dm, int* R, int* Rq, int* ncr_cap, size_t* bytes) {
  if (!dm.bf16) return false;
  int r = Cfg<D>::RMAX;
  while (r > 16 && r * dm.K > 4096) r /= 2;
  int rq = r / dm.G;
  if (rq < 1) return false;
  r = rq * dm.G;
  const long long last = dm.q_pos0 + dm.Tq - 1;
  const int ncr = (int)(last / dm.S) + 1;
  const size_t b = smem_bytes<D>(r, dm.K, ncr);
  if (b > 160 * 1024) return false;
  *R = r; *Rq = rq; *ncr_cap = ncr; *bytes = b;
  return true;
}

template <int D>
hipError_t launch_t(const Dims& dm, const void* Q, const void* K, const void* V,
                    const int32_t* idx, const float* score, void* O, float* lse_own,
                    float* lse_tot, hipStream_t st, int R, int Rq, int ncr_cap, size_t bytes) {
  dim3 grid((dm.Tq + Rq - 1) / Rq, dm.Hkv, dm.B);
  auto kfn = k_attend_mfma<D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, grid, dim3(256), bytes, st, dm, R, Rq, ncr_cap,
                     reinterpret_cast<const uint16_t*>(Q), reinterpret_cast<const uint16_t*>(K),
                     reinterpret_cast<const uint16_t*>(V), idx, score,
                     reinterpret_cast<uint16_t*>(O), lse_own, lse_tot);
  return hipGetLastError();
}

}  // namespace

// Returns true and launches when the MFMA path applies (bf16, LDS budget fits).
bool attend_mfma_try(const Dims& dm, const void* Q, const void* K, const void* V,
                     const int32_t* idx, const float* score, void* O, float* lse_own,
                     float* lse_tot, hipStream_t st, hipError_t* err) {
  int R, Rq, ncr;
  size_t bytes;
  if (dm.d == 64) {
    if (!plan<64>(dm, &R, &Rq, &ncr, &bytes)) return false;
    *err = launch_t<64>(dm, Q, K, V, idx, score, O, lse_own, lse_tot, st, R, Rq, ncr, bytes);
    return true;
  }
  if (!plan<128>(dm, &R, &Rq, &ncr, &bytes)) return false;
  *err = launch_t<128>(dm, Q, K, V, idx, score, O, lse_own, lse_tot, st, R, Rq, ncr, bytes);
  return true;
}

}  // namespace hils
