// Exact merge of a decode row's per-split top lists by rank (note §5.2 top-K
// over the union of the splits' local top-K lists, which holds the global one).
// Shared by the selection-only merge kernel and the decode step whose slot
// kernel merges the lists itself before it attends.
#pragma once

#include "hils_internal.h"

namespace hils {
namespace dec {

// LDS of one merge: the keys of every list entry ([split][KM]), the selected
// keys in rank order and the number of valid entries.
template <int KM>
struct MergeSmem {
  unsigned long long keys[1024];
  unsigned long long sel[KM];
  int nval;
};

// Row r's lists: split sp covers candidates [sp * split_size, ...) of the row's
// n and holds min(K, its candidates) entries, best first, at
// ws[(r * nsplit + sp) * K ...]. One thread per list entry (thread t is entry
// t % KM of list t / KM; nsplit <= 32, nsplit * KM <= blockDim.x <= 1024). An
// entry's key packs its (score, chunk) order into 64 bits: the score's order
// bits high and the complemented chunk low, so that a larger key comes first
// and equal scores go to the lower chunk; 0 is an empty slot. Its rank in the
// union is its index in its own list plus, for every other list, the number of
// keys above it, found by a branch-free binary search whose steps over all
// lists advance together (their LDS reads are in flight at once). Keys are
// unique, so the ranks below K name the K best entries. NL (16, 24 or 32) bounds
// nsplit; the searches cover NL lists. Every thread of the workgroup must call
// this. Returns cnt = min(K, valid entries); sel[0 .. cnt) holds the selected
// keys by rank, visible to every thread on return.
template <int KM, int NL>
__device__ __forceinline__ int merge_rank(const Dims& dm, long long r, int n,
                                          const float* __restrict__ ws_s,
                                          const int* __restrict__ ws_i, int nsplit, int split_size,
                                          MergeSmem<KM>& sm) {
  const int t = threadIdx.x, K = dm.K;
  const int sp = t / KM, j = t % KM;
  const bool in = sp < nsplit;
  const int nv = in ? min(K, max(0, min(split_size, n - sp * split_size))) : 0;
  const long long src = ((long long)r * nsplit + (in ? sp : 0)) * K + min(j, K - 1);
  const float sv = ws_s[src];
  const int cv = ws_i[src];
  const unsigned long long key =
      j < nv ? ((unsigned long long)order_bits(sv) << 32) | (uint32_t)~(uint32_t)cv : 0ull;
  if (in) sm.keys[t] = key;
  if (t == 0) {
    int tot = 0;
    for (int x = 0; x < nsplit; ++x) tot += min(K, max(0, min(split_size, n - x * split_size)));
    sm.nval = tot;
  }
  __syncthreads();
  if (key != 0ull) {
    int rank = j;
    int pos[NL];  // per list: keys above `key` found so far
#pragma unroll
    for (int x = 0; x < NL; ++x) pos[x] = 0;
#pragma unroll
    for (int step = KM / 2; step > 0; step >>= 1)
#pragma unroll
      for (int x = 0; x < NL; ++x) {  // lists past nsplit read the last list (no branch)
        const unsigned long long a = sm.keys[min(x, nsplit - 1) * KM + pos[x] + step - 1];
        pos[x] += ((x < nsplit) & (a > key)) ? step : 0;
      }
#pragma unroll
    for (int x = 0; x < NL; ++x) {
      const unsigned long long a = sm.keys[min(x, nsplit - 1) * KM + pos[x]];
      rank += ((x < nsplit) & (x != sp)) ? pos[x] + (a > key ? 1 : 0) : 0;
    }
    if (rank < K) sm.sel[rank] = key;
  }
  __syncthreads();
  return min(K, sm.nval);
}

__device__ __forceinline__ int merge_chunk(unsigned long long key) { return (int)~(uint32_t)key; }
__device__ __forceinline__ float merge_score(unsigned long long key) {
  return order_float((uint32_t)(key >> 32));
}

// Place of selected entry t (t < cnt) in the row's list, which is ascending by
// chunk id.
template <int KM>
__device__ __forceinline__ int merge_place(const MergeSmem<KM>& sm, int t, int cnt) {
  const int c = merge_chunk(sm.sel[t]);
  int p = 0;
#pragma unroll
  for (int k = 0; k < KM; ++k)  // all reads in flight; entries past cnt are not counted
    p += (k < cnt) & (merge_chunk(sm.sel[min(k, cnt - 1)]) < c);
  return p;
}

}  // namespace dec
}  // namespace hils
