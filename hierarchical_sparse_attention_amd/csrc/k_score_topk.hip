// Chunk scoring and top-K selection (note §5.2: s^_{i,c} = q_i.k'_c/sqrt(d) + b'_c,
// I_i = {c in C_i : rank_desc(s^_{i,c}) < K}).
//
// Float32 inputs. (bf16 inputs are scored on matrix cores, k_score_mfma.hip; the
// split/merge structure below is shared.) Two kernels share one float32 score
// function (chunk_score), so both produce bit-identical scores and selections:
//  * rows path (prefill): one thread per query row; summaries are staged in LDS
//    in blocks and broadcast to all rows of the workgroup; each thread keeps its
//    row's running top-K list (score desc, chunk id asc) in LDS.
//  * split path (decode, few rows, many candidates): candidates of a row are
//    split over workgroups (one candidate per thread), each workgroup writes its
//    local top-K to the workspace, and a merge kernel ranks the union. The global
//    top-K is a subset of the union of local top-Ks, so the merge is exact.
// The order key is total: (score descending, chunk id ascending).
#include <algorithm>
#include <cfloat>
#include <climits>

#include "decode_merge.h"
#include "hils_internal.h"

namespace hils {
namespace {

constexpr int kBlockChunks = 32;  // summaries staged per LDS block (rows path)
constexpr int kSplit = kSplitMfma;  // candidates per workgroup (split path, both dtypes)
constexpr int kMergeMax = 4096;   // entries the merge kernel ranks in LDS

__host__ __device__ inline int rows_per_wg(int K) { return K <= 16 ? 256 : (K <= 32 ? 128 : 64); }

__device__ __forceinline__ bool before(float sa, int ca, float sb, int cb) {
  return topk_before(sa, ca, sb, cb);
}

template <bool BF16, int D>
__global__ __launch_bounds__(256) void k_score_rows(Dims dm, const void* __restrict__ Q,
                                                    const float* __restrict__ ksum,
                                                    const float* __restrict__ ent,
                                                    int32_t* __restrict__ idx,
                                                    float* __restrict__ score) {
  __shared__ float kb[kBlockChunks][D];
  __shared__ float eb[kBlockChunks];
  __shared__ float ls[4096];
  __shared__ int li[4096];
  const int R = blockDim.x, t = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int K = dm.K;
  const int i = blockIdx.x * R + t;
  const bool valid = i < dm.Tq;
  const int last = min(dm.Tq, (int)(blockIdx.x + 1) * R) - 1;
  const int n = valid ? dm.ncand(dm.q_pos0 + i) : 0;
  const int nmax = dm.ncand(dm.q_pos0 + last);

  float q[D];
  if (valid) {
    load_row<BF16, D>(Q, (((long long)b * dm.Tq + i) * dm.H + h) * D, q);
  } else {
#pragma unroll
    for (int e = 0; e < D; ++e) q[e] = 0.0f;
  }
  int cnt = 0;
  for (int c0 = 0; c0 < nmax; c0 += kBlockChunks) {
    const int nb = min(kBlockChunks, nmax - c0);
    for (int x = t; x < nb * D; x += R) {
      const int cc = x / D, e = x % D;
      kb[cc][e] = ksum[(((long long)b * dm.NCcap + c0 + cc) * dm.H + h) * D + e];
    }
    for (int x = t; x < nb; x += R) eb[x] = ent[((long long)b * dm.NCcap + c0 + x) * dm.H + h];
    __syncthreads();
    const int lim = min(nb, n - c0);
    for (int cc = 0; cc < lim; ++cc) {
      const float s = chunk_score<D>(q, kb[cc], dm.scale, eb[cc]);
      const int c = c0 + cc;
      if (cnt < K || s > ls[(K - 1) * R + t]) {
        int pos = cnt < K ? cnt : K - 1;
        while (pos > 0) {
          const float prev = ls[(pos - 1) * R + t];
          if (!(prev < s)) break;  // equal scores keep the earlier (lower) chunk first
          ls[pos * R + t] = prev;
          li[pos * R + t] = li[(pos - 1) * R + t];
          --pos;
        }
        ls[pos * R + t] = s;
        li[pos * R + t] = c;
        if (cnt < K) ++cnt;
      }
    }
    __syncthreads();
  }
  if (!valid) return;
  const long long o = (((long long)b * dm.Tq + i) * dm.H + h) * K;
  for (int k = 0; k < cnt; ++k) {
    const int c = li[k * R + t];
    int rank = 0;
    for (int k2 = 0; k2 < cnt; ++k2) rank += li[k2 * R + t] < c;
    idx[o + rank] = c;
    score[o + rank] = ls[k * R + t];
  }
  for (int k = cnt; k < K; ++k) {
    idx[o + k] = -1;
    score[o + k] = -INFINITY;
  }
}

// Group-max selection (note §5.4, GQA): the chunk scores of the G query heads of
// a kv head are aggregated by their maximum and the top K of that is the chunk
// set of the whole group. Thread t owns query head g G + t % G of position
// blockIdx.x * (R / G) + t / G, so the G heads of a position sit in neighbouring
// lanes: they take the group maximum with lane shuffles and keep identical lists
// ordered by (group score desc, chunk asc), each carrying its own head's score
// per entry. Summaries of the G heads are staged in LDS in blocks of cpb chunks.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void k_score_group(Dims dm, int cpb, const void* __restrict__ Q,
                                                     const float* __restrict__ ksum,
                                                     const float* __restrict__ ent,
                                                     int32_t* __restrict__ idx,
                                                     float* __restrict__ score) {
  extern __shared__ __align__(16) float gsm[];
  const int R = blockDim.x, t = threadIdx.x, G = dm.G, K = dm.K;
  float* kb = gsm;                                   // [cpb][G][D]
  float* eb = kb + cpb * G * D;                      // [cpb][G]
  float* ls = eb + cpb * G;                          // [K][R] group scores
  float* lh = ls + K * R;                            // [K][R] own head scores
  int* li = reinterpret_cast<int*>(lh + K * R);      // [K][R] chunk ids
  const int g = blockIdx.y, b = blockIdx.z, hh = t % G;
  const int P = R / G;
  const int i = blockIdx.x * P + t / G;
  const bool valid = i < dm.Tq;
  const int h = g * G + hh;
  const int last = min(dm.Tq, (int)(blockIdx.x + 1) * P) - 1;
  const int n = valid ? dm.ncand(dm.q_pos0 + i) : 0;
  const int nmax = dm.ncand(dm.q_pos0 + last);
  float q[D];
  if (valid) {
    load_row<BF16, D>(Q, (((long long)b * dm.Tq + i) * dm.H + h) * D, q);
  } else {
#pragma unroll
    for (int e = 0; e < D; ++e) q[e] = 0.0f;
  }
  int cnt = 0;
  for (int c0 = 0; c0 < nmax; c0 += cpb) {
    const int nb = min(cpb, nmax - c0);
    for (int x = t; x < nb * G * D; x += R) {
      const int cc = x / (G * D), hx = (x / D) % G, e = x % D;
      kb[x] = ksum[(((long long)b * dm.NCcap + c0 + cc) * dm.H + g * G + hx) * D + e];
    }
    for (int x = t; x < nb * G; x += R)
      eb[x] = ent[((long long)b * dm.NCcap + c0 + x / G) * dm.H + g * G + x % G];
    __syncthreads();
    const int lim = min(nb, n - c0);  // equal for the G heads of a position
    for (int cc = 0; cc < lim; ++cc) {
      const float s = chunk_score<D>(q, kb + (cc * G + hh) * D, dm.scale, eb[cc * G + hh]);
      float gs = s;
      for (int o = 1; o < G; o <<= 1) gs = fmaxf(gs, __shfl_xor(gs, o, 64));
      const int c = c0 + cc;
      if (cnt < K || gs > ls[(K - 1) * R + t]) {
        int pos = cnt < K ? cnt : K - 1;
        while (pos > 0) {
          const float prev = ls[(pos - 1) * R + t];
          if (!(prev < gs)) break;  // equal scores keep the earlier (lower) chunk first
          ls[pos * R + t] = prev;
          lh[pos * R + t] = lh[(pos - 1) * R + t];
          li[pos * R + t] = li[(pos - 1) * R + t];
          --pos;
        }
        ls[pos * R + t] = gs;
        lh[pos * R + t] = s;
        li[pos * R + t] = c;
        if (cnt < K) ++cnt;
      }
    }
    __syncthreads();
  }
  if (!valid) return;
  const long long o = (((long long)b * dm.Tq + i) * dm.H + h) * K;
  for (int k = 0; k < cnt; ++k) {
    const int c = li[k * R + t];
    int rank = 0;
    for (int k2 = 0; k2 < cnt; ++k2) rank += li[k2 * R + t] < c;
    idx[o + rank] = c;
    score[o + rank] = lh[k * R + t];
  }
  for (int k = cnt; k < K; ++k) {
    idx[o + k] = -1;
    score[o + k] = -INFINITY;
  }
}

// chunks per LDS block of the group kernel: as many as 32 KiB hold, 1 to 8
int group_cpb(const Dims& dm) {
  return std::max(1, std::min(8, 32768 / (dm.G * (dm.d + 1) * (int)sizeof(float))));
}
size_t group_smem_bytes(const Dims& dm, int R) {
  return ((size_t)group_cpb(dm) * dm.G * (dm.d + 1) + 3 * (size_t)dm.K * R) * sizeof(float);
}

// Split path, stage 1: grid (splits, rows); thread t scores candidate split*256+t.
template <bool BF16, int D>
__global__ __launch_bounds__(kSplit) void k_score_split(Dims dm, const void* __restrict__ Q,
                                                       const float* __restrict__ ksum,
                                                       const float* __restrict__ ent,
                                                       float* __restrict__ ws_s,
                                                       int* __restrict__ ws_i, int nsplit) {
  __shared__ float qs[D];
  __shared__ float ss[kSplit];
  const int split = blockIdx.x, r = blockIdx.y, t = threadIdx.x;
  const int h = r % dm.H, i = (r / dm.H) % dm.Tq, b = r / (dm.H * dm.Tq);
  const int n = dm.ncand(dm.q_pos0 + i);
  const int c = split * kSplit + t;
  for (int e = t; e < D; e += kSplit) qs[e] = load_elem<BF16>(Q, (long long)r * D + e);
  __syncthreads();
  float s = -INFINITY;
  const bool valid = c < n;
  if (valid) {
    float q[D], kr[D];
#pragma unroll
    for (int e = 0; e < D; ++e) q[e] = qs[e];
    const long long sidx = ((long long)b * dm.NCcap + c) * dm.H + h;
    load_row<false, D>(ksum, sidx * D, kr);
    s = chunk_score<D>(q, kr, dm.scale, ent[sidx]);
  }
  ss[t] = s;
  __syncthreads();
  if (!valid) return;
  const int nvalid = min(kSplit, n - split * kSplit);
  int rank = 0;
  for (int t2 = 0; t2 < nvalid; ++t2) rank += before(ss[t2], split * kSplit + t2, s, c);
  if (rank < dm.K) {
    const long long o = ((long long)r * nsplit + split) * dm.K + rank;
    ws_s[o] = s;
    ws_i[o] = c;
  }
}

// Split path, stage 2: one workgroup per row ranks the union of local lists.
__global__ __launch_bounds__(1024) void k_topk_merge(Dims dm, const float* __restrict__ ws_s,
                                                    const int* __restrict__ ws_i, int nsplit,
                                                    int32_t* __restrict__ idx,
                                                    float* __restrict__ score) {
  __shared__ __align__(16) float es[kMergeMax];
  __shared__ __align__(16) int ec[kMergeMax];
  __shared__ float sel_s[64];
  __shared__ int sel_c[64];
  const int r = blockIdx.x;
  const int i = (r / dm.H) % dm.Tq;
  const int n = dm.ncand(dm.q_pos0 + i);
  topk_merge_row(dm, r, n, ws_s, ws_i, nsplit, kSplit, idx, score, es, ec, sel_s, sel_c);
}

// Split path, stage 2 for at most 64 splits: one wavefront per row merges the
// sorted local lists held in registers (lane = split).
template <int KM>
__global__ __launch_bounds__(64) void k_topk_merge_wave(Dims dm, const float* __restrict__ ws_s,
                                                        const int* __restrict__ ws_i, int nsplit,
                                                        int32_t* __restrict__ idx,
                                                        float* __restrict__ score) {
  __shared__ int sel_c[64];
  const int r = blockIdx.x, lane = threadIdx.x, K = dm.K;
  const int i = (r / dm.H) % dm.Tq;
  const int n = dm.ncand(dm.q_pos0 + i);
  const int nv = lane < nsplit ? min(K, max(0, min(kSplit, n - lane * kSplit))) : 0;
  const long long base = ((long long)r * nsplit + min(lane, nsplit - 1)) * K;
  // every load is issued before any is used (in bounds, masked after); the empty
  // asm statements consume each value unconditionally, which keeps the compiler
  // from moving a load into the branch of its select, where each one would wait
  // for the previous
  float sv[KM];
  int cv[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const int jj = min(j, K - 1);
    sv[j] = ws_s[base + jj];
    cv[j] = ws_i[base + jj];
  }
#pragma unroll
  for (int j = 0; j < KM; ++j) asm volatile("" ::"v"(sv[j]), "v"(cv[j]));
  uint32_t lh[KM], ll[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const bool v = j < nv;
    lh[j] = v ? order_bits(sv[j]) : 0u;
    ll[j] = v ? ~(uint32_t)cv[j] : 0u;
  }
  uint32_t wh = 0, wl = 0;
  const int cnt = wave_merge_lists<KM>(lh, ll, K, &wh, &wl);
  const int c = (int)~wl;
  if (lane < cnt) sel_c[lane] = c;
  __builtin_amdgcn_wave_barrier();
  const long long o = (long long)r * K;
  if (lane < cnt) {
    int pos = 0;
    for (int k2 = 0; k2 < cnt; ++k2) pos += sel_c[k2] < c;
    idx[o + pos] = c;
    score[o + pos] = order_float(wh);
  } else if (lane < K) {
    idx[o + lane] = -1;
    score[o + lane] = -INFINITY;
  }
}

// Merge of the per-split top lists by rank, one thread per list entry (at most
// 32 lists of KM slots, ns * KM <= 1024; dec::merge_rank); the K best entries
// are written in chunk order. The same set as the wavefront merge.
template <int KM, int NL>
__global__ __launch_bounds__(1024) void k_topk_merge_rank(Dims dm, const float* __restrict__ ws_s,
                                                          const int* __restrict__ ws_i, int nsplit,
                                                          int32_t* __restrict__ idx,
                                                          float* __restrict__ score) {
  __shared__ dec::MergeSmem<KM> sm;
  const int r = blockIdx.x, t = threadIdx.x, K = dm.K;
  const int i = (r / dm.H) % dm.Tq;
  const int n = dm.ncand(dm.q_pos0 + i);
  const int cnt = dec::merge_rank<KM, NL>(dm, r, n, ws_s, ws_i, nsplit, kSplit, sm);
  const long long o = (long long)r * K;
  if (t < cnt) {
    const int p = dec::merge_place<KM>(sm, t, cnt);
    idx[o + p] = dec::merge_chunk(sm.sel[t]);
    score[o + p] = dec::merge_score(sm.sel[t]);
  } else if (t < K) {
    idx[o + t] = -1;
    score[o + t] = -INFINITY;
  }
}

// No row has a candidate (every query's local branch reaches back to key 0):
// the selection is empty.
__global__ __launch_bounds__(256) void k_sel_empty(long long n, int32_t* __restrict__ idx,
                                                   float* __restrict__ score) {
  for (long long x = (long long)blockIdx.x * 256 + threadIdx.x; x < n;
       x += (long long)gridDim.x * 256) {
    idx[x] = -1;
    score[x] = -INFINITY;
  }
}

int max_candidates(const Dims& dm) {
  if (dm.Tq <= 0) return 0;
  return dm.ncand(dm.q_pos0 + dm.Tq - 1);
}

int split_count(const Dims& dm) { return (max_candidates(dm) + kSplit - 1) / kSplit; }

bool use_split(const Dims& dm) {
  const long long rows = (long long)dm.B * dm.Tq * dm.H;
  const int ns = split_count(dm);
  return rows <= 4096 && ns >= 1 && (long long)ns * dm.K <= kMergeMax;
}

template <bool BF16, int D>
hipError_t launch_t(const Dims& dm, const void* Q, const float* ksum, const float* ent,
                    int32_t* idx, float* score, void* ws, hipStream_t st) {
  if (dm.group_sel && score_mfma_group_applies(dm))
    return launch_score_mfma_group(dm, Q, ksum, ent, idx, score, ws, st);
  if (dm.group_sel && dm.G > 1) {
    const int R = rows_per_wg(dm.K);  // a multiple of every supported G (powers of two <= 64)
    const int P = R / dm.G;
    const size_t smem = group_smem_bytes(dm, R);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_score_group<BF16, D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_score_group<BF16, D>), dim3((dm.Tq + P - 1) / P, dm.Hkv, dm.B),
                       dim3(R), smem, st, dm, group_cpb(dm), Q, ksum, ent, idx, score);
    return hipGetLastError();
  }
  if (use_split(dm)) {
    const int ns = split_count(dm);
    const long long rows = (long long)dm.B * dm.Tq * dm.H;
    float* ws_s = reinterpret_cast<float*>(ws);
    int* ws_i = reinterpret_cast<int*>(ws_s + rows * ns * dm.K);
    hipError_t e;
    if (BF16) {
      e = launch_score_mfma_split(dm, Q, ksum, ent, ws_s, ws_i, ns, st);
    } else {
      hipLaunchKernelGGL((k_score_split<BF16, D>), dim3(ns, rows), dim3(kSplit), 0, st, dm, Q,
                         ksum, ent, ws_s, ws_i, ns);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    const int KMr = dm.K <= 16 ? 16 : (dm.K <= 32 ? 32 : 64);
    if (ns <= 32 && ns * KMr <= 1024) {  // one thread per list entry, ranks by binary search
      const int nt = (ns * KMr + 63) / 64 * 64;
      const bool nl16 = ns <= 16;  // KM = 64 holds at most 16 lists
      if (KMr == 16 && nl16)
        hipLaunchKernelGGL((k_topk_merge_rank<16, 16>), dim3(rows), dim3(nt), 0, st, dm, ws_s,
                           ws_i, ns, idx, score);
      else if (KMr == 16 && ns <= 24)
        hipLaunchKernelGGL((k_topk_merge_rank<16, 24>), dim3(rows), dim3(nt), 0, st, dm, ws_s,
                           ws_i, ns, idx, score);
      else if (KMr == 16)
        hipLaunchKernelGGL((k_topk_merge_rank<16, 32>), dim3(rows), dim3(nt), 0, st, dm, ws_s,
                           ws_i, ns, idx, score);
      else if (KMr == 32 && nl16)
        hipLaunchKernelGGL((k_topk_merge_rank<32, 16>), dim3(rows), dim3(nt), 0, st, dm, ws_s,
                           ws_i, ns, idx, score);
      else if (KMr == 32)
        hipLaunchKernelGGL((k_topk_merge_rank<32, 32>), dim3(rows), dim3(nt), 0, st, dm, ws_s,
                           ws_i, ns, idx, score);
      else
        hipLaunchKernelGGL((k_topk_merge_rank<64, 16>), dim3(rows), dim3(nt), 0, st, dm, ws_s,
                           ws_i, ns, idx, score);
      return hipGetLastError();
    }
    if (ns <= 64) {  // one wavefront per row, lists in registers
      if (dm.K <= 16)
        hipLaunchKernelGGL(k_topk_merge_wave<16>, dim3(rows), dim3(64), 0, st, dm, ws_s, ws_i, ns,
                           idx, score);
      else if (dm.K <= 32)
        hipLaunchKernelGGL(k_topk_merge_wave<32>, dim3(rows), dim3(64), 0, st, dm, ws_s, ws_i, ns,
                           idx, score);
      else
        hipLaunchKernelGGL(k_topk_merge_wave<64>, dim3(rows), dim3(64), 0, st, dm, ws_s, ws_i, ns,
                           idx, score);
      return hipGetLastError();
    }
    const int E = ns * dm.K;  // one thread per entry when they fit in a workgroup
    const int nt = E <= 1024 ? ((E + 63) / 64) * 64 : 1024;
    hipLaunchKernelGGL(k_topk_merge, dim3(rows), dim3(max(nt, 64)), 0, st, dm, ws_s, ws_i, ns,
                       idx, score);
  } else if (BF16) {
    return launch_score_mfma_prefill(dm, Q, ksum, ent, idx, score, ws, st);
  } else {
    const int R = rows_per_wg(dm.K);
    dim3 grid((dm.Tq + R - 1) / R, dm.H, dm.B);
    hipLaunchKernelGGL((k_score_rows<BF16, D>), grid, dim3(R), 0, st, dm, Q, ksum, ent, idx,
                       score);
  }
  return hipGetLastError();
}

}  // namespace

size_t score_topk_ws_bytes(const Dims& dm) {
  if (max_candidates(dm) == 0) return 0;
  if (dm.group_sel && score_mfma_group_applies(dm)) return score_mfma_prefill_ws_bytes(dm);
  if (dm.group_sel && dm.G > 1) return 0;
  if (!use_split(dm)) return dm.bf16 ? score_mfma_prefill_ws_bytes(dm) : 0;
  const long long rows = (long long)dm.B * dm.Tq * dm.H;
  return (size_t)rows * split_count(dm) * dm.K * (sizeof(float) + sizeof(int));
}

int decode_lists_plan(const Dims& dm, int* km) {
  const long long rows = (long long)dm.B * dm.Tq * dm.H;
  if (rows == 0 || max_candidates(dm) == 0) return 0;
  if (dm.group_sel && dm.G > 1) return 0;
  if (!use_split(dm)) return 0;
  const int ns = split_count(dm);
  const int KMr = dm.K <= 16 ? 16 : (dm.K <= 32 ? 32 : 64);
  if (ns > 32 || ns * KMr > 1024) return 0;
  *km = KMr;
  return ns;
}

size_t decode_lists_ws_bytes(const Dims& dm, int nsplit) {
  const long long rows = (long long)dm.B * dm.Tq * dm.H;
  return (size_t)rows * nsplit * dm.K * (sizeof(float) + sizeof(int));
}

hipError_t launch_decode_lists(const Dims& dm, const void* Q, const float* ksum, const float* ent,
                               float* ws_s, int* ws_i, int nsplit, hipStream_t st) {
  if (dm.bf16) return launch_score_mfma_split(dm, Q, ksum, ent, ws_s, ws_i, nsplit, st);
  const long long rows = (long long)dm.B * dm.Tq * dm.H;
  if (dm.d == 64)
    hipLaunchKernelGGL((k_score_split<false, 64>), dim3(nsplit, rows), dim3(kSplit), 0, st, dm,
                       Q, ksum, ent, ws_s, ws_i, nsplit);
  else
    hipLaunchKernelGGL((k_score_split<false, 128>), dim3(nsplit, rows), dim3(kSplit), 0, st, dm,
                       Q, ksum, ent, ws_s, ws_i, nsplit);
  return hipGetLastError();
}

hipError_t launch_score_topk(const Dims& dm, const void* Q, const float* ksum, const float* ent,
                             int32_t* idx, float* score, void* ws, hipStream_t st) {
  if ((long long)dm.B * dm.Tq * dm.H == 0) return hipSuccess;
  if (max_candidates(dm) == 0) {
    const long long n = (long long)dm.B * dm.Tq * dm.H * dm.K;
    hipLaunchKernelGGL(k_sel_empty, dim3((unsigned)std::min<long long>((n + 255) / 256, 4096)),
                       dim3(256), 0, st, n, idx, score);
    return hipGetLastError();
  }
  if (dm.bf16) {
    return dm.d == 64 ? launch_t<true, 64>(dm, Q, ksum, ent, idx, score, ws, st)
                      : launch_t<true, 128>(dm, Q, ksum, ent, idx, score, ws, st);
  }
  return dm.d == 64 ? launch_t<false, 64>(dm, Q, ksum, ent, idx, score, ws, st)
                    : launch_t<false, 128>(dm, Q, ksum, ent, idx, score, ws, st);
}

}  // namespace hils
