// Internal declarations shared by the HIP kernels and the C-ABI host layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hils {

constexpr int kWave = 64;   // CDNA wavefront width
constexpr int kChunk = 64;  // supported chunk size S (one key per lane)
constexpr int kMaxSel = 64;  // largest supported top-K
constexpr int kMaxWinChunks = 32;  // largest sliding window, in chunks (2048 keys)

// Dimensions after validation and defaulting (see hils_dims in hils.h).
struct Dims {
  int B, Tq, Tkv, Tcap, NCcap, H, Hkv, G, d, S, K;
  bool bf16;
  bool group_sel;  // one chunk set per kv head by the group maximum of the scores
  long long q_pos0;
  float scale;
  int window;  // local branch: 0 = the query's own chunk; W > 0 = the last W keys
  // The helpers below divide by the constant kChunk: the entry points reject any
  // other S, and a constant divisor is a shift where a run-time 64-bit one is a
  // long emulated division. Positions are never negative.
  // first key of the local branch of the query at absolute position pos
  __host__ __device__ __forceinline__ long long lstart(long long pos) const {
    return window > 0 ? (pos >= window ? pos - window + 1 : 0) : pos - pos % kChunk;
  }
  // candidates are the chunks 0 .. ncand(pos) - 1, wholly before the local branch
  __host__ __device__ __forceinline__ int ncand(long long pos) const {
    return (int)(lstart(pos) / kChunk);
  }
  // chunks the local branch of pos touches: lstart(pos) / S .. pos / S
  __host__ __device__ __forceinline__ int nlocal(long long pos) const {
    return (int)(pos / kChunk - lstart(pos) / kChunk) + 1;
  }
  // most local chunks of any query (partial slots per row in the decode and backward paths)
  __host__ __device__ __forceinline__ int nlocal_max() const {
    return window > 0 ? window / kChunk + 1 : 1;
  }
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

// Whether entry k of a row's selection list counts: its id c is a candidate of
// the row (0 <= c < ncand) and larger than every earlier entry of the row
// (prev_max, the largest earlier id; -1 before the first). Padding, ids outside
// the candidates and repeated or out-of-order ids contribute nothing, neither
// output nor score; a list made by the selection (ascending, padding last)
// counts every real entry. Counted entries are distinct, so per-chunk row lists
// built from them hold a row at most once.
__host__ __device__ __forceinline__ bool entry_counts(int c, int ncand, int prev_max) {
  return c >= 0 && c < ncand && c > prev_max;
}

__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}

// Largest value held by the lanes below this one (exclusive prefix maximum
// across the wavefront; `lo` for lane 0).
__device__ __forceinline__ int wave_excl_max(int v, int lo) {
  const int lane = threadIdx.x & 63;
  int x = __shfl_up(v, 1, 64);
  x = lane == 0 ? lo : x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x = max(x, y);
  }
  return x;
}

// Top-K order key: (score descending, chunk id ascending). Branch-free, so rank
// loops keep their loads in flight.
__device__ __forceinline__ bool topk_before(float sa, int ca, float sb, int cb) {
  return (sa > sb) | ((sa == sb) & (ca < cb));
}

// Final top-K of row r from nsplit local lists (split sp covers candidates
// [sp * split_size, (sp + 1) * split_size) and holds min(K, its candidates)
// entries, best first, at ws[(r * nsplit + sp) * K ...]). The global top-K is a
// subset of the union of the local ones, so ranking the union is exact. Every
// thread of the workgroup takes part; es/ec (16-byte aligned) hold nsplit * K
// entries rounded up to a multiple of 32, sel_s/sel_c K. Writes idx ascending by chunk id (padding -1) and score (padding -inf).
__device__ __forceinline__ void topk_merge_row(const Dims& dm, long long r, int n,
                                               const float* ws_s, const int* ws_i, int nsplit,
                                               int split_size, int32_t* idx, float* score,
                                               float* es, int* ec, float* sel_s, int* sel_c) {
  const int t = threadIdx.x, nt = blockDim.x, K = dm.K;
  const int E = nsplit * K, E4 = (E + 31) & ~31;  // es/ec padded to a multiple of 32
  for (int x = t; x < E4; x += nt) {
    const int sp = x / K, k = x % K;
    const int nv = x < E ? min(K, max(0, min(split_size, n - sp * split_size))) : 0;
    const long long o = r * E + min(x, E - 1);  // read unconditionally (in bounds), so
    const float sv = ws_s[o];                   // both loads are in flight together
    const int cv = ws_i[o];
    const bool v = k < nv;
    es[x] = v ? sv : -INFINITY;
    ec[x] = v ? cv : 0x7fffffff;
  }
  __syncthreads();
  const int cnt = min(K, n);
  const float4* es4 = reinterpret_cast<const float4*>(es);
  const int4* ec4 = reinterpret_cast<const int4*>(ec);
  for (int x = t; x < E; x += nt) {
    const float s = es[x];
    const int c = ec[x];
    int rank = 0;
    for (int y0 = 0; y0 < E4 / 4; y0 += 8) {  // 16 LDS reads in flight per step
      float4 a[8];
      int4 ca[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        a[j] = es4[y0 + j];
        ca[j] = ec4[y0 + j];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        rank += topk_before(a[j].x, ca[j].x, s, c) + topk_before(a[j].y, ca[j].y, s, c) +
                topk_before(a[j].z, ca[j].z, s, c) + topk_before(a[j].w, ca[j].w, s, c);
    }
    if (c != 0x7fffffff && rank < cnt) {
      sel_s[rank] = s;
      sel_c[rank] = c;
    }
  }
  __syncthreads();
  const long long o = r * K;
  for (int k = t; k < K; k += nt) {
    if (k < cnt) {
      const int c = sel_c[k];
      int pos = 0;
      for (int k2 = 0; k2 < cnt; ++k2) pos += sel_c[k2] < c;
      idx[o + pos] = c;
      score[o + pos] = sel_s[k];
    } else {
      idx[o + k] = -1;
      score[o + k] = -INFINITY;
    }
  }
}

// Wave-level top-K merge of at most 64 sorted local lists (lane l holds list l in
// registers, best first): K rounds of a wave-wide maximum over the list heads,
// the winning list advancing by one. Keys are 64-bit, (ordered score bits,
// ~chunk id), so larger is better and ties go to the lower chunk id. Lane k ends
// with the round-k winner in (*wh, *wl); returns the number of rounds with a
// winner. KM >= K.
__device__ __forceinline__ uint32_t order_bits(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_float(uint32_t h) {
  return __uint_as_float((h >> 31) ? (h & 0x7FFFFFFFu) : ~h);
}
template <int CTRL>
__device__ __forceinline__ void key_max_dpp(uint32_t& h, uint32_t& l) {
  const uint32_t ph = (uint32_t)__builtin_amdgcn_mov_dpp((int)h, CTRL, 0xF, 0xF, true);
  const uint32_t pl = (uint32_t)__builtin_amdgcn_mov_dpp((int)l, CTRL, 0xF, 0xF, true);
  const bool gt = (ph > h) | ((ph == h) & (pl > l));
  h = gt ? ph : h;
  l = gt ? pl : l;
}
__device__ __forceinline__ void key_max_pair(uint32_t& h, uint32_t& l, uint32_t h0, uint32_t l0,
                                             uint32_t h1, uint32_t l1) {
  const bool gt = (h1 > h0) | ((h1 == h0) & (l1 > l0));
  h = gt ? h1 : h0;
  l = gt ? l1 : l0;
}
__device__ __forceinline__ void key_wave_max(uint32_t& h, uint32_t& l) {
  key_max_dpp<0xB1>(h, l);   // quad_perm [1,0,3,2]
  key_max_dpp<0x4E>(h, l);   // quad_perm [2,3,0,1]
  key_max_dpp<0x141>(h, l);  // row_half_mirror
  key_max_dpp<0x140>(h, l);  // row_mirror
  auto a = __builtin_amdgcn_permlane16_swap(h, h, false, false);
  auto b = __builtin_amdgcn_permlane16_swap(l, l, false, false);
  key_max_pair(h, l, a[0], b[0], a[1], b[1]);
  auto c = __builtin_amdgcn_permlane32_swap(h, h, false, false);
  auto d = __builtin_amdgcn_permlane32_swap(l, l, false, false);
  key_max_pair(h, l, c[0], d[0], c[1], d[1]);
}
template <int KM>
__device__ __forceinline__ int wave_merge_lists(uint32_t (&lh)[KM], uint32_t (&ll)[KM], int K,
                                                uint32_t* wh, uint32_t* wl) {
  const int lane = threadIdx.x & 63;
  int found = 0;
  for (int k = 0; k < K; ++k) {
    uint32_t h = lh[0], l = ll[0];
    key_wave_max(h, l);
    if (h == 0 && l == 0) break;  // every list exhausted (wave-uniform)
    if (lane == k) *wh = h, *wl = l;
    if (lh[0] == h && ll[0] == l) {  // the winning list (keys are unique) drops its head
#pragma unroll
      for (int j = 0; j + 1 < KM; ++j) lh[j] = lh[j + 1], ll[j] = ll[j + 1];
      lh[KM - 1] = 0, ll[KM - 1] = 0;
    }
    ++found;
  }
  return found;
}

// ---------------------------------------------------------------- launches
hipError_t launch_summarize(const Dims& dm, const void* K, const void* Ql, int c_begin, int c_end,
                            float* ksum, float* ent, float* lse_l, hipStream_t st);

size_t score_topk_ws_bytes(const Dims& dm);
size_t score_mfma_prefill_ws_bytes(const Dims& dm);
// bf16 group-max selection on matrix cores (G = 2 or 4); same workspace as prefill
bool score_mfma_group_applies(const Dims& dm);
hipError_t launch_score_mfma_group(const Dims& dm, const void* Q, const float* ksum,
                                   const float* ent, int32_t* idx, float* score, void* ws,
                                   hipStream_t st);
hipError_t launch_score_mfma_prefill(const Dims& dm, const void* Q, const float* ksum,
                                     const float* ent, int32_t* idx, float* score, void* ws,
                                     hipStream_t st);
constexpr int kSplitMfma = 128;  // candidates per workgroup of the bf16 decode scoring
hipError_t launch_score_mfma_split(const Dims& dm, const void* Q, const float* ksum,
                                   const float* ent, float* ws_s, int* ws_i, int nsplit,
                                   hipStream_t st);
hipError_t launch_score_topk(const Dims& dm, const void* Q, const float* ksum, const float* ent,
                             int32_t* idx, float* score, void* ws, hipStream_t st);
// Decode step with the list merge inside the slot kernel: the number of
// candidate splits (and in *km the list capacity, 16, 32 or 64) when the step
// scores by candidate splits and the rank merge holds every list entry, else 0.
int decode_lists_plan(const Dims& dm, int* km);
size_t decode_lists_ws_bytes(const Dims& dm, int nsplit);
// Split scoring only: each split's local top list (score, chunk) into ws_s / ws_i.
hipError_t launch_decode_lists(const Dims& dm, const void* Q, const float* ksum, const float* ent,
                               float* ws_s, int* ws_i, int nsplit, hipStream_t st);

size_t attend_ws_bytes(const Dims& dm);
size_t attend_mfma_ws_bytes(const Dims& dm);
bool attend_mfma_try(const Dims& dm, const void* Q, const void* K, const void* V,
                     const int32_t* idx, const float* score, void* O, float* lse_own,
                     float* lse_tot, void* ws, hipStream_t st, hipError_t* err);
hipError_t launch_attend_fuse(const Dims& dm, const void* Q, const void* K, const void* V,
                              const int32_t* idx, const float* score, void* O, float* lse_own,
                              float* lse_tot, void* ws, hipStream_t st);
// Whether the attention of these rows runs as decode slots (few query rows).
bool attend_is_decode(const Dims& dm);
// Rest of the decode step after launch_decode_lists: per (slot, row) the merge
// of the row's lists and the slot's attention, then the fixed-order combine.
// Writes idx and score (as hils_score_topk would) and O / lse_own / lse_tot;
// ws holds attend_ws_bytes(dm) and must not overlap the lists.
hipError_t launch_decode_merged(const Dims& dm, const void* Q, const void* K, const void* V,
                                const float* ws_s, const int* ws_i, int nsplit, int km,
                                int32_t* idx, float* score, void* O, float* lse_own,
                                float* lse_tot, void* ws, hipStream_t st);
// The same rest of the step with one workgroup per row (merge once, every slot,
// combine in LDS): for calls of many rows. Same outputs bit for bit; needs no
// workspace beyond the lists.
bool decode_row_applies(const Dims& dm, int nsplit, int km);
hipError_t launch_decode_row(const Dims& dm, const void* Q, const void* K, const void* V,
                             const float* ws_s, const int* ws_i, int nsplit, int km, int32_t* idx,
                             float* score, void* O, float* lse_own, float* lse_tot,
                             hipStream_t st);

size_t backward_ws_bytes(const Dims& dm);
size_t backward_mfma_ws_bytes(const Dims& dm);
// bf16, d = 64 prefill backward on matrix cores; returns false when it does not apply.
bool backward_mfma_try(const Dims& dm, const void* Q, const void* K, const void* V,
                       const void* Ql, const float* ksum, const float* ent, const float* lse_l,
                       const int32_t* idx, const float* score, const float* lse_tot,
                       const void* O, const void* dO, void* dQ, void* dK, void* dV, void* dQl,
                       const void* Qs, void* dQs, float* ws_D, float* ws_dsh, void* ws_mfma,
                       hipStream_t st, hipError_t* err);
hipError_t launch_backward(const Dims& dm, const void* Q, const void* K, const void* V,
                           const void* Ql, const float* ksum, const float* ent, const float* lse_l,
                           const int32_t* idx, const float* score, const float* lse_tot,
                           const void* O, const void* dO, void* dQ, void* dK, void* dV,
                           void* dQl, const void* Qs, void* dQs, void* ws, hipStream_t st);

}  // namespace hils
