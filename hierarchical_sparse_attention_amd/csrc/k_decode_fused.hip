// Fused decode step: chunk scoring, top-K selection, intra-chunk attention and
// inter-chunk fusion of a few query rows in one launch (note §5.2 score and top-K
// equations; note §5.3 hierarchical softmax; Tide Fig. 3).
//
// Grid (splits, rows), one workgroup of kFWaves wavefronts per (split, row):
//  1. the workgroup scores its kFSplit candidates with the matrix-core sequence
//     every bf16 scoring kernel uses (so the scores, and the selection, are bit
//     for bit those of the prefill pass) and writes their local top-K list to
//     the workspace;
//  2. it counts itself in on the row's counter (an agent-scope atomic after a
//     release fence); the workgroup that arrives last for the row goes on, the
//     others are done. Nothing waits for anything;
//  3. the last one merges the row's local lists (the global top-K is a subset of
//     their union: an entry's rank is its index in its own list plus the number
//     of keys above it in every other list), writes idx and score, and puts the
//     row's counter back to zero for the next call;
//  4. its wavefronts attend the selected chunks and the local branch's chunks,
//     one slot each (the slot arithmetic of the decode slot kernel), and one
//     wavefront fuses the slots in a fixed order (the combine arithmetic of the
//     decode path), writing O and the log-masses.
#include "decode_slot.h"
#include "hils_internal.h"
#include "mfma_common.h"

namespace hils {
namespace {

constexpr int kFWaves = 8;
constexpr int kFThreads = 64 * kFWaves;
constexpr int kFSplit = 32 * kFWaves;  // candidates per workgroup
constexpr int kMergeKeys = 4096;       // most list entries the last workgroup ranks

struct FPlan {
  int nsplit, KM, NS;
  size_t smem, cnt_bytes, list_bytes;
};

__host__ __device__ inline size_t fup16(size_t x) { return (x + 15) & ~(size_t)15; }

// LDS: split scores | merge keys [nsplit][KM] | selected keys [KM] | slot chunk ids
// and scores [KM] | query row | slot log-masses [NS] | slot outputs [NS][D]
struct FSmem {
  float* ss;
  unsigned long long* keys;
  unsigned long long* sel;
  int* ci;
  float* si;
  uint16_t* qh;
  float* pl;
  float* po;
};

__host__ __device__ inline size_t fsmem_bytes(int nsplit, int KM, int NS, int D) {
  return fup16(kFSplit * 4) + fup16((size_t)nsplit * KM * 8) + fup16((size_t)KM * 8) +
         2 * fup16((size_t)KM * 4) + fup16((size_t)D * 2) + fup16((size_t)NS * 4) +
         fup16((size_t)NS * D * 4);
}

__device__ inline FSmem fcarve(char* p, int nsplit, int KM, int NS, int D) {
  FSmem s;
  s.ss = reinterpret_cast<float*>(p); p += fup16(kFSplit * 4);
  s.keys = reinterpret_cast<unsigned long long*>(p); p += fup16((size_t)nsplit * KM * 8);
  s.sel = reinterpret_cast<unsigned long long*>(p); p += fup16((size_t)KM * 8);
  s.ci = reinterpret_cast<int*>(p); p += fup16((size_t)KM * 4);
  s.si = reinterpret_cast<float*>(p); p += fup16((size_t)KM * 4);
  s.qh = reinterpret_cast<uint16_t*>(p); p += fup16((size_t)D * 2);
  s.pl = reinterpret_cast<float*>(p); p += fup16((size_t)NS * 4);
  s.po = reinterpret_cast<float*>(p);
  return s;
}

// Keys, bounds and liveness of attention slot `slot` of the row at pos: slots
// below K are the selected chunks (ci, -1 for padding), the rest the local
// branch's chunks, keys max(l0, chunk start) .. min(pos, chunk end).
__device__ __forceinline__ bool slot_keys(const Dims& dm, const FSmem& sm, int slot, long long pos,
                                          long long* key0, int* nk) {
  if (slot < dm.K) {
    const int c = sm.ci[slot];
    *key0 = (long long)max(c, 0) * kChunk;
    *nk = kChunk;
    return c >= 0;
  }
  const long long l0 = dm.lstart(pos), cc = l0 / kChunk + (slot - dm.K);
  *key0 = cc * kChunk > l0 ? cc * kChunk : l0;
  *nk = (int)(min(pos, cc * kChunk + kChunk - 1) - *key0) + 1;
  return cc <= pos / kChunk;
}

template <int D>
__global__ __launch_bounds__(kFThreads) void k_decode_fused(
    Dims dm, int nsplit_max, int KM, const uint16_t* __restrict__ Q,
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const float* __restrict__ ksum, const float* __restrict__ ent, int32_t* __restrict__ idx,
    float* __restrict__ score, uint16_t* __restrict__ O, float* __restrict__ lse_own,
    float* __restrict__ lse_tot, unsigned* __restrict__ cnt, float* __restrict__ ws_s,
    int* __restrict__ ws_i) {
  extern __shared__ __align__(16) char fsm_raw[];
  __shared__ int s_last;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int split = blockIdx.x;
  const long long r = blockIdx.y;
  const int Ks = dm.K, NS = Ks + dm.nlocal_max();
  const int h = (int)(r % dm.H), i = (int)((r / dm.H) % dm.Tq);
  const int b = (int)(r / ((long long)dm.H * dm.Tq)), g = h / dm.G;
  const long long pos = dm.q_pos0 + i;
  const int n = dm.ncand(pos);
  const int nsplit = max(1, (n + kFSplit - 1) / kFSplit);
  if (split >= nsplit) return;  // a row with fewer candidates than the longest one
  const FSmem sm = fcarve(fsm_raw, nsplit_max, KM, NS, D);
  const long long lbase = r * (long long)nsplit_max * Ks;

  // ---- 1. this split's scores and its local top-K list
  const int cbase = split * kFSplit;
  if (n > 0) {
    mf::split_scores<D, kFWaves>(dm, Q, ksum, ent, r, n, cbase, sm.ss);
    __syncthreads();
    mf::split_local_topk<kFSplit>(sm.ss, max(0, min(kFSplit, n - cbase)), cbase, Ks,
                                  ws_s + lbase + (long long)split * Ks,
                                  ws_i + lbase + (long long)split * Ks);
  }
  // ---- 2. publish the list and count the split in; the row's last split goes on
  __threadfence();
  __syncthreads();
  if (t == 0) {
    const unsigned old =
        __hip_atomic_fetch_add(cnt + r, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == (unsigned)(nsplit - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();  // the other splits' lists are visible from here on
  // every split of the row has arrived: the counter is ready for the next call
  if (t == 0) __hip_atomic_exchange(cnt + r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- 3. merge. Keys are (order bits of the score, complemented chunk id), larger
  // is better, 0 for an empty slot; each list is sorted descending. Ids outside
  // the candidates cannot come from step 1; they are dropped all the same, so no
  // slot below can read outside the K and V buffers.
  const int E = nsplit * KM;
  for (int x = t; x < E; x += kFThreads) {
    const int sp = x / KM, j = x % KM;
    const int nv = min(Ks, max(0, min(kFSplit, n - sp * kFSplit)));
    const long long src = lbase + (long long)sp * Ks + min(j, Ks - 1);
    const float sv = ws_s[src];
    const int cv = ws_i[src];
    const bool ok = j < nv && cv >= 0 && cv < n;
    sm.keys[x] = ok ? ((unsigned long long)order_bits(sv) << 32) | (uint32_t)~(uint32_t)cv : 0ull;
  }
  for (int x = t; x < Ks; x += kFThreads) sm.sel[x] = 0ull;
  for (int e = t; e < D / 8; e += kFThreads)
    *reinterpret_cast<uint4*>(sm.qh + 8 * e) = *reinterpret_cast<const uint4*>(Q + r * D + 8 * e);
  __syncthreads();
  for (int x = t; x < E; x += kFThreads) {
    const unsigned long long key = sm.keys[x];
    if (key == 0ull) continue;
    const int sp = x / KM;
    int rank = x % KM;
    for (int l = 0; l < nsplit; ++l) {
      const unsigned long long* lk = sm.keys + l * KM;
      int p = 0;  // keys of list l above `key` (branch-free binary search)
      for (int step = KM / 2; step > 0; step >>= 1) p += lk[p + step - 1] > key ? step : 0;
      p += lk[p] > key ? 1 : 0;
      rank += l == sp ? 0 : p;
    }
    if (rank < Ks) sm.sel[rank] = key;
  }
  __syncthreads();
  // the selection in ascending chunk order: idx / score, and the attention slots
  if (t < Ks) {
    const unsigned long long k0 = sm.sel[t];
    const int c = (int)~(uint32_t)k0;
    int p = 0;
    for (int k2 = 0; k2 < Ks; ++k2) {
      const unsigned long long k1 = sm.sel[k2];
      p += (k1 != 0ull && (int)~(uint32_t)k1 < c) ? 1 : 0;
    }
    if (k0 != 0ull) {
      sm.ci[p] = c;
      sm.si[p] = order_float((uint32_t)(k0 >> 32));
    }
  }
  __syncthreads();
  if (t < Ks) {  // entries past the selected count are padding
    const int csel = min(Ks, n);
    const int c = t < csel ? sm.ci[t] : -1;
    const float sv = t < csel ? sm.si[t] : -INFINITY;
    sm.ci[t] = c;
    sm.si[t] = sv;
    idx[r * Ks + t] = c;
    score[r * Ks + t] = sv;
  }
  __syncthreads();

  // ---- 4. slot attention: slot s on wavefront s mod kFWaves. For d = 64 a
  // wavefront loads two slots' keys and values before computing either.
  const long long kv_base = ((long long)b * dm.Tcap * dm.Hkv + g) * D;
  const long long kv_stride = (long long)dm.Hkv * D;
  constexpr int PAIR = D == 64 ? 2 : 1;
  for (int s0 = w; s0 < NS; s0 += PAIR * kFWaves) {
    long long k0[PAIR];
    int nk[PAIR];
    bool live[PAIR];
    dec::SlotRegs<D> rg[PAIR];
#pragma unroll
    for (int u = 0; u < PAIR; ++u) {
      const int slot = s0 + u * kFWaves;
      live[u] = slot < NS && slot_keys(dm, sm, slot, pos, &k0[u], &nk[u]);
      if (!live[u]) k0[u] = 0, nk[u] = 1;  // loads stay in bounds; results unused
      dec::slot_load<D>(rg[u], K, V, kv_base, kv_stride, k0[u], nk[u]);
    }
#pragma unroll
    for (int u = 0; u < PAIR; ++u) {
      const int slot = s0 + u * kFWaves;
      if (slot >= NS) continue;  // wave-uniform
      if (live[u]) {
        dec::slot_compute<D>(rg[u], dm, sm.qh, nk[u], sm.po + slot * D, sm.pl + slot);
      } else if (lane == 0) {
        sm.pl[slot] = -INFINITY;
      }
    }
  }
  __syncthreads();

  // ---- 5. inter-chunk softmax over the slots in slot order (selected slots by
  // their chunk score, local slots by their exact log-mass); lane k holds slots
  // k and 64 + k
  if (w != 0) return;
  constexpr int X = D / kWave;
  float lg[2], loc[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int k = lane + 64 * u;
    const float pl = k < NS ? sm.pl[k] : -INFINITY;
    const float sc = k < Ks ? sm.si[k] : -INFINITY;
    lg[u] = k >= NS ? -INFINITY : k < Ks ? (pl != -INFINITY ? sc : -INFINITY) : pl;
    loc[u] = k >= Ks && k < NS ? pl : -INFINITY;
  }
  const float ml = wave_max(fmaxf(loc[0], loc[1]));
  const float l_own = ml + logf(wave_sum(expf(loc[0] - ml) + expf(loc[1] - ml)));
  const float mx = wave_max(fmaxf(lg[0], lg[1]));
  const float Lambda = mx + logf(wave_sum(expf(lg[0] - mx) + expf(lg[1] - mx)));
  const float a0 = expf(lg[0] - Lambda), a1 = expf(lg[1] - Lambda);
  float acc[X];
#pragma unroll
  for (int x = 0; x < X; ++x) acc[x] = 0.0f;
  for (int k = 0; k < NS; ++k) {
    const float ak = k < 64 ? dec::lane_bcast(a0, k) : dec::lane_bcast(a1, k - 64);
    if (ak != 0.0f) {  // wave-uniform; padding and absent slots are skipped
#pragma unroll
      for (int x = 0; x < X; ++x) acc[x] = fmaf(ak, sm.po[k * D + lane + kWave * x], acc[x]);
    }
  }
#pragma unroll
  for (int x = 0; x < X; ++x) O[r * D + lane + kWave * x] = f32_to_bf16_bits(acc[x]);
  if (lane == 0) {
    if (lse_own) lse_own[r] = l_own;
    if (lse_tot) lse_tot[r] = Lambda;
  }
}

bool fplan(const Dims& dm, FPlan* p) {
  if (!dm.bf16 || dm.group_sel || dm.Tq < 1) return false;
  const long long rows = (long long)dm.B * dm.Tq * dm.H;
  if (rows > 65535) return false;
  const int n = dm.ncand(dm.q_pos0 + dm.Tq - 1);
  p->nsplit = max(1, (n + kFSplit - 1) / kFSplit);
  p->KM = dm.K <= 16 ? 16 : dm.K <= 32 ? 32 : 64;
  p->NS = dm.K + dm.nlocal_max();
  if ((long long)p->nsplit * p->KM > kMergeKeys || p->NS > 128) return false;
  p->smem = fsmem_bytes(p->nsplit, p->KM, p->NS, dm.d);
  if (p->smem > 160 * 1024) return false;
  p->cnt_bytes = ((size_t)rows * sizeof(unsigned) + 255) & ~(size_t)255;
  p->list_bytes = (size_t)rows * p->nsplit * dm.K * sizeof(float);
  return true;
}

template <int D>
hipError_t launch_t(const Dims& dm, const FPlan& p, const void* Q, const void* K, const void* V,
                    const float* ksum, const float* ent, int32_t* idx, float* score, void* O,
                    float* lse_own, float* lse_tot, void* ws, hipStream_t st) {
  char* base = reinterpret_cast<char*>(ws);
  unsigned* cnt = reinterpret_cast<unsigned*>(base);
  float* ws_s = reinterpret_cast<float*>(base + p.cnt_bytes);
  int* ws_i = reinterpret_cast<int*>(base + p.cnt_bytes + ((p.list_bytes + 255) & ~(size_t)255));
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_decode_fused<D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.smem);
  if (e != hipSuccess) return e;
  const long long rows = (long long)dm.B * dm.Tq * dm.H;
  hipLaunchKernelGGL((k_decode_fused<D>), dim3(p.nsplit, (unsigned)rows), dim3(kFThreads), p.smem,
                     st, dm, p.nsplit, p.KM, reinterpret_cast<const uint16_t*>(Q),
                     reinterpret_cast<const uint16_t*>(K), reinterpret_cast<const uint16_t*>(V),
                     ksum, ent, idx, score, reinterpret_cast<uint16_t*>(O), lse_own, lse_tot, cnt,
                     ws_s, ws_i);
  return hipGetLastError();
}

}  // namespace

size_t decode_fused_counter_bytes(const Dims& dm) {
  FPlan p;
  return fplan(dm, &p) ? p.cnt_bytes : 0;
}

size_t decode_fused_ws_bytes(const Dims& dm) {
  FPlan p;
  if (!fplan(dm, &p)) return 0;
  return p.cnt_bytes + 2 * ((p.list_bytes + 255) & ~(size_t)255);
}

bool decode_fused_try(const Dims& dm, const void* Q, const void* K, const void* V,
                      const float* ksum, const float* ent, int32_t* idx, float* score, void* O,
                      float* lse_own, float* lse_tot, void* ws, hipStream_t st, hipError_t* err) {
  FPlan p;
  if (!fplan(dm, &p)) return false;
  *err = dm.d == 64 ? launch_t<64>(dm, p, Q, K, V, ksum, ent, idx, score, O, lse_own, lse_tot, ws, st)
                    : launch_t<128>(dm, p, Q, K, V, ksum, ent, idx, score, O, lse_own, lse_tot, ws,
                                    st);
  return true;
}

}  // namespace hils
