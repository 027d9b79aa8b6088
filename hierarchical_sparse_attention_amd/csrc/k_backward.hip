// Training backward of HiLS attention with the selection held fixed.
//
// The score of each selected chunk enters the forward weights (note §5.3), so
// the gradient of the loss reaches the query, the summary key k'_c, the entropy
// bias b'_c and, through the landmark softmax (note §5.1), the landmark query
// and the chunk's keys. The pages print no gradient formulas; these follow from
// the forward by the chain rule. Per row (b,i,h) with dO_i, fused weight
// alpha_c = exp(s^_c - Lambda), intra-chunk softmax P_cj, u_j = dO_i.v_j and
// r_c = sum_j P_cj u_j:
//   D_i     = sum_c alpha_c r_c + sum_local w_j u_j  (= dO_i . O_i)
//   ds^_c   = alpha_c (r_c - D_i)                  (gradient of the chunk score)
//   ds_cj   = alpha_c P_cj (u_j - r_c)             (selected chunk logits)
//   ds_j    = w_j (u_j - D_i), w_j = exp(s_j - Lambda)  (local branch: the own
//             chunk up to the row, or the last W keys; incl. its log-mass)
//   dQ_i    = scale (sum ds k_j + sum_c ds^_c k'_c)
//   dK_j   += scale ds q_i,  dV_j += (alpha P or w) dO_i
//   dk'_c   = scale sum_i ds^_ic q_i,  db'_c = sum_i ds^_ic
//   ds'_j   = p'_j [dk'.(k_j - k'_c) + db' (L' - s'_j - b'_c)]
//   dQl_c   = scale sum_j ds'_j k_j,  dK_j += p'_j dk'_c + scale ds'_j Ql_c
//
// Kernels (no floating-point atomics; fixed summation orders => deterministic):
//   k_bwd_rows : one wavefront per row -> dQ, ds^ per slot, D_i (workspace)
//   k_sel_bitmap: bit i of word [b,h,c] set when row i selected chunk c (atomicOr
//                 commutes, so the bitmap does not depend on thread order);
//                 k_sel_bitmap_lds builds blocks of it in LDS and writes them once
//   k_bwd_kv   : one workgroup per (chunk, kv head, batch) -> dK, dV, dQl, walking
//                the rows whose local branch covers the chunk's keys and the
//                rows that selected the chunk in ascending order.
#include "hils_internal.h"

namespace hils {
namespace {

__device__ __forceinline__ float bcast(float v, int j) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}

// dot of a row held in "lane e owns feature e + 64x" layout (xs) with a row in
// registers of every lane (row[D]).
template <int D>
__device__ __forceinline__ float dot_bcast(const float* xs, const float* row) {
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < D; ++e) acc = fmaf(bcast(xs[e / kWave], e % kWave), row[e], acc);
  return acc;
}

struct WsLayout {
  size_t dsh, dr, bitmap, mfma, total;
  int words;  // bitmap words per (b, h, c)
};

WsLayout ws_layout(const Dims& dm) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  WsLayout L;
  const size_t rows = (size_t)dm.B * dm.Tq * dm.H;
  L.words = (dm.Tq + 31) / 32;
  L.dsh = 0;
  L.dr = up(rows * dm.K * sizeof(float));
  L.bitmap = L.dr + up(rows * sizeof(float));
  const int NC = dm.Tkv / dm.S;
  L.mfma = L.bitmap + up((size_t)dm.B * dm.H * NC * L.words * sizeof(uint32_t));
  L.total = L.mfma + backward_mfma_ws_bytes(dm);
  return L;
}

template <bool BF16, int D>
__global__ __launch_bounds__(256) void k_bwd_rows(Dims dm, const void* __restrict__ Q,
                                                  const void* __restrict__ K,
                                                  const void* __restrict__ V,
                                                  const float* __restrict__ ksum,
                                                  const int32_t* __restrict__ idx,
                                                  const float* __restrict__ score,
                                                  const float* __restrict__ lse_tot,
                                                  const void* __restrict__ dO,
                                                  void* __restrict__ dQ, void* __restrict__ dQs,
                                                  float* __restrict__ ws_dsh,
                                                  float* __restrict__ ws_D) {
  constexpr int X = D / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int i = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int h = blockIdx.y, b = blockIdx.z;
  if (i >= dm.Tq) return;
  const int g = h / dm.G, Ksel = dm.K;
  const long long r = ((long long)b * dm.Tq + i) * dm.H + h;
  const long long pos = dm.q_pos0 + i;
  const int ncand = dm.ncand(pos);
  const long long l0 = dm.lstart(pos), c_lo = l0 / kChunk, c_hi = pos / kChunk;
  const long long kv_stride = (long long)dm.Hkv * D;
  const long long kv_base = ((long long)b * dm.Tcap * dm.Hkv + g) * D;
  const float tau = dm.scale, Lambda = lse_tot[r];

  float q[D];
  load_row<BF16, D>(Q, r * D, q);
  float go[X];  // dO in lane-e layout
#pragma unroll
  for (int x = 0; x < X; ++x) go[x] = load_elem<BF16>(dO, r * D + lane + kWave * x);

  auto logits = [&](long long c0, int nk, float& s, float& u) {
    s = -INFINITY;
    u = 0.0f;
    if (lane < nk) {
      float row[D];
      const long long off = kv_base + (c0 + lane) * kv_stride;
      load_row<BF16, D>(K, off, row);
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < D; ++e) acc = fmaf(q[e], row[e], acc);
      s = acc * tau;
      load_row<BF16, D>(V, off, row);
      u = dot_bcast<D>(go, row);  // readlane ignores EXEC: inactive lanes still hold dO
    }
  };

  // the local branch's keys of chunk cc: logits, dO.v and whether the lane's key is one
  auto local_logits = [&](long long cc, float& s, float& u) {
    const int nk = (int)min((long long)kChunk, pos - cc * dm.S + 1);
    logits(cc * dm.S, nk, s, u);
    if (cc * dm.S + lane < l0) s = -INFINITY;
    return nk;
  };
  // pass 1: the local branch's share of D (sum of exp(s_j - Lambda) u_j over its
  // keys), per selected chunk r, alpha and intra-chunk log-sum-exp
  float s, u, m;
  float Dsum = 0.0f;
  for (long long cc = c_lo; cc <= c_hi; ++cc) {
    local_logits(cc, s, u);
    Dsum += wave_sum(s > -INFINITY ? expf(s - Lambda) * u : 0.0f);
  }
  float rk = 0.0f, ak = 0.0f, mk = 0.0f;  // lane k holds slot k's values
  // lane k holds entry k and whether it counts (entry_counts)
  const int cl = lane < Ksel ? idx[r * Ksel + lane] : -1;
  const uint64_t cmask =
      __ballot(lane < Ksel && entry_counts(cl, ncand, wave_excl_max(cl, -1)));
  for (int k = 0; k < Ksel; ++k) {
    if (((cmask >> k) & 1ull) == 0ull) continue;  // wave-uniform
    const int c = __builtin_amdgcn_readlane(cl, k);
    logits((long long)c * dm.S, kChunk, s, u);
    m = wave_max(s);
    const float lz = m + logf(wave_sum(expf(s - m)));
    const float rc = wave_sum(expf(s - lz) * u);
    const float a = expf(score[r * Ksel + k] - Lambda);
    Dsum += a * rc;
    if (lane == k) { rk = rc; ak = a; mk = lz; }
  }

  // pass 2: gradients of the logits and of the query; with a scoring query
  // (Q-Cal) the chunk scores' part goes to dQs
  float dq[X], dqs[X];
#pragma unroll
  for (int x = 0; x < X; ++x) dq[x] = dqs[x] = 0.0f;
  auto add_keys = [&](long long c0, int nk, float ds) {
    for (int j = 0; j < nk; ++j) {
      const float dj = bcast(ds, j);
      const long long off = kv_base + (c0 + j) * kv_stride;
#pragma unroll
      for (int x = 0; x < X; ++x) dq[x] = fmaf(tau * dj, load_elem<BF16>(K, off + lane + kWave * x), dq[x]);
    }
  };
  for (long long cc = c_lo; cc <= c_hi; ++cc) {
    const int nk = local_logits(cc, s, u);
    add_keys(cc * dm.S, nk, s > -INFINITY ? expf(s - Lambda) * (u - Dsum) : 0.0f);
  }
  for (int k = 0; k < Ksel; ++k) {
    const int c = __builtin_amdgcn_readlane(cl, k);
    if (((cmask >> k) & 1ull) == 0ull) {  // wave-uniform
      if (lane == 0) ws_dsh[r * Ksel + k] = 0.0f;
      continue;
    }
    const float rc = bcast(rk, k), a = bcast(ak, k), lz = bcast(mk, k);
    logits((long long)c * dm.S, kChunk, s, u);
    add_keys((long long)c * dm.S, kChunk, a * expf(s - lz) * (u - rc));
    const float dsh = a * (rc - Dsum);
    const long long sidx = (((long long)b * dm.NCcap + c) * dm.H + h) * D;
#pragma unroll
    for (int x = 0; x < X; ++x) dqs[x] = fmaf(tau * dsh, ksum[sidx + lane + kWave * x], dqs[x]);
    if (lane == 0) ws_dsh[r * Ksel + k] = dsh;
  }
  if (dQs) {
#pragma unroll
    for (int x = 0; x < X; ++x) store_elem<BF16>(dQs, r * D + lane + kWave * x, dqs[x]);
  } else {
#pragma unroll
    for (int x = 0; x < X; ++x) dq[x] += dqs[x];
  }
#pragma unroll
  for (int x = 0; x < X; ++x) store_elem<BF16>(dQ, r * D + lane + kWave * x, dq[x]);
  if (lane == 0) ws_D[r] = Dsum;
}

__global__ void k_fill_zero(uint32_t* __restrict__ p, long long n) {
  for (long long x = blockIdx.x * (long long)blockDim.x + threadIdx.x; x < n;
       x += (long long)gridDim.x * blockDim.x)
    p[x] = 0u;
}

__global__ void k_sel_bitmap(Dims dm, const int32_t* __restrict__ idx, uint32_t* __restrict__ bm,
                             int words) {
  const long long n = (long long)dm.B * dm.Tq * dm.H;
  const int NC = dm.Tkv / dm.S;
  // one thread per row: its entries in order, so entry_counts sees the earlier ids
  for (long long r = blockIdx.x * (long long)blockDim.x + threadIdx.x; r < n;
       r += (long long)gridDim.x * blockDim.x) {
    const int h = (int)(r % dm.H);
    const int i = (int)((r / dm.H) % dm.Tq);
    const int b = (int)(r / ((long long)dm.H * dm.Tq));
    const int nc = min(dm.ncand(dm.q_pos0 + i), NC);
    int seen = -1;
    for (int k = 0; k < dm.K; ++k) {
      const int c = idx[r * dm.K + k];
      if (entry_counts(c, nc, seen))
        atomicOr(&bm[(((long long)b * dm.H + h) * NC + c) * words + i / 32], 1u << (i % 32));
      seen = max(seen, c);
    }
  }
}

// Same bitmaps built per (block of wpw words = 32 wpw positions, head, batch)
// in LDS and written once: no global atomics and no clearing pass.
__global__ __launch_bounds__(256) void k_sel_bitmap_lds(Dims dm, const int32_t* __restrict__ idx,
                                                        uint32_t* __restrict__ bm, int words,
                                                        int wpw) {
  extern __shared__ uint32_t lb[];  // [NC][wpw]
  const int NC = dm.Tkv / dm.S;
  const int h = blockIdx.y, b = blockIdx.z;
  const int w0 = blockIdx.x * wpw;
  const int nw = min(wpw, words - w0);
  for (int x = threadIdx.x; x < NC * wpw; x += blockDim.x) lb[x] = 0u;
  __syncthreads();
  const int i0 = w0 * 32, ni = min(nw * 32, dm.Tq - i0);
  for (int ii = threadIdx.x; ii < ni; ii += blockDim.x) {  // one thread per row
    const int i = i0 + ii;
    const int nc = min(dm.ncand(dm.q_pos0 + i), NC);
    const int32_t* ir = idx + (((long long)b * dm.Tq + i) * dm.H + h) * dm.K;
    int seen = -1;
    for (int k = 0; k < dm.K; ++k) {
      const int c = ir[k];
      if (entry_counts(c, nc, seen)) atomicOr(&lb[c * wpw + ii / 32], 1u << (ii % 32));
      seen = max(seen, c);
    }
  }
  __syncthreads();
  for (int x = threadIdx.x; x < NC * nw; x += blockDim.x) {
    const int c = x / nw, ww = x % nw;
    bm[(((long long)b * dm.H + h) * NC + c) * words + w0 + ww] = lb[c * wpw + ww];
  }
}

template <bool BF16, int D>
__global__ __launch_bounds__(256) void k_bwd_kv(Dims dm, const void* __restrict__ Q,
                                                const void* __restrict__ Qsc,
                                                const void* __restrict__ K,
                                                const void* __restrict__ V,
                                                const void* __restrict__ Ql,
                                                const float* __restrict__ ksum,
                                                const float* __restrict__ ent,
                                                const float* __restrict__ lse_l,
                                                const int32_t* __restrict__ idx,
                                                const float* __restrict__ score,
                                                const float* __restrict__ lse_tot,
                                                const void* __restrict__ dO,
                                                const float* __restrict__ ws_dsh,
                                                const float* __restrict__ ws_D,
                                                const uint32_t* __restrict__ bm, int words,
                                                void* __restrict__ dK, void* __restrict__ dV,
                                                void* __restrict__ dQl) {
  constexpr int X = D / kWave;
  constexpr int kListMax = 2048;
  __shared__ float kt[kChunk][D + 1];
  __shared__ float vt[kChunk][D + 1];
  __shared__ float red[kChunk][D];
  __shared__ int rowlist[kListMax];
  __shared__ int list_n;
  __shared__ float part[4][D + 1];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int NC = dm.Tkv / dm.S, Ksel = dm.K;
  const float tau = dm.scale;
  const long long kv_stride = (long long)dm.Hkv * D;
  const long long kv_base = ((long long)b * dm.Tcap * dm.Hkv + g) * D;
  const long long key0 = (long long)c * kChunk;

  for (int x = threadIdx.x; x < kChunk * D; x += blockDim.x) {
    const int j = x / D, e = x % D;
    kt[j][e] = load_elem<BF16>(K, kv_base + (key0 + j) * kv_stride + e);
    vt[j][e] = load_elem<BF16>(V, kv_base + (key0 + j) * kv_stride + e);
  }
  __syncthreads();

  float dk[kChunk * X], dv[kChunk * X];  // [j][x]: key j, feature lane + 64x
#pragma unroll
  for (int y = 0; y < kChunk * X; ++y) { dk[y] = 0.0f; dv[y] = 0.0f; }

  // one query row against this chunk's keys; ds and the value weight a per lane j
  // (keys klo <= j < khi of the chunk take part)
  auto row_pass = [&](long long r, bool own_row, int klo, int khi, float sh) {
    float qx[X], gx[X];
#pragma unroll
    for (int x = 0; x < X; ++x) {
      qx[x] = load_elem<BF16>(Q, r * D + lane + kWave * x);
      gx[x] = load_elem<BF16>(dO, r * D + lane + kWave * x);
    }
    float sacc = 0.0f, uacc = 0.0f;
#pragma unroll 8
    for (int e = 0; e < D; ++e) {
      sacc = fmaf(bcast(qx[e / kWave], e % kWave), kt[lane][e], sacc);
      uacc = fmaf(bcast(gx[e / kWave], e % kWave), vt[lane][e], uacc);
    }
    const bool valid = lane >= klo && lane < khi;
    const float s = valid ? sacc * tau : -INFINITY;
    const float Lambda = lse_tot[r];
    float ds, a;
    if (own_row) {
      a = valid ? expf(s - Lambda) : 0.0f;
      ds = a * (uacc - ws_D[r]);
    } else {
      const float m = wave_max(s);
      const float lz = m + logf(wave_sum(expf(s - m)));
      const float p = expf(s - lz);
      const float rc = wave_sum(p * uacc);
      const float alpha = expf(sh - Lambda);
      a = alpha * p;
      ds = a * (uacc - rc);
    }
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const float dsj = bcast(ds, j) * tau, aj = bcast(a, j);
#pragma unroll
      for (int x = 0; x < X; ++x) {
        dk[j * X + x] = fmaf(dsj, qx[x], dk[j * X + x]);
        dv[j * X + x] = fmaf(aj, gx[x], dv[j * X + x]);
      }
    }
  };

  for (int hh = 0; hh < dm.G; ++hh) {
    const int h = g * dm.G + hh;
    float dkb[X];
#pragma unroll
    for (int x = 0; x < X; ++x) dkb[x] = 0.0f;
    float dbs = 0.0f;
    // rows whose local branch covers keys of this chunk: its own rows, or with a
    // window of W keys the positions key0 .. key0 + S + W - 2
    const int span = dm.window > 0 ? kChunk + dm.window - 1 : kChunk;
    for (int i = (int)key0 + w; i < (int)key0 + span && i < dm.Tq; i += 4) {
      const long long r = ((long long)b * dm.Tq + i) * dm.H + h;
      const long long l0 = dm.lstart(dm.q_pos0 + i);
      row_pass(r, true, (int)max(0LL, l0 - key0),
               (int)min((long long)kChunk, dm.q_pos0 + i - key0 + 1), 0.0f);
    }
    // rows that selected this chunk, ascending, in segments of 64 bitmap words
    const uint32_t* bmw = bm + (((long long)b * dm.H + h) * NC + c) * words;
    for (int w0 = (int)((key0 + kChunk) / 32); w0 < words; w0 += kWave) {
      if (w == 0) {
        const uint32_t word = (w0 + lane < words) ? bmw[w0 + lane] : 0u;
        const int cnt = __popc(word);
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int y = __shfl_up(incl, o, kWave);
          if (lane >= o) incl += y;
        }
        int p = incl - cnt;
        uint32_t bits = word;
        while (bits) {
          const int bit = __ffs(bits) - 1;
          bits &= bits - 1;
          rowlist[p++] = (w0 + lane) * 32 + bit;
        }
        if (lane == kWave - 1) list_n = incl;
      }
      __syncthreads();
      const int n = list_n;
      for (int e = w; e < n; e += 4) {
        const int i = rowlist[e];
        const long long r = ((long long)b * dm.Tq + i) * dm.H + h;
        const int v = lane < Ksel ? idx[r * Ksel + lane] : -1;
        const unsigned long long hit = __ballot(v == c);
        if (hit == 0) continue;  // wave-uniform; cannot happen for a consistent bitmap
        const int slot = __ffsll((long long)hit) - 1;
        const float dsh = ws_dsh[r * Ksel + slot];
        row_pass(r, false, 0, kChunk, score[r * Ksel + slot]);
#pragma unroll
        for (int x = 0; x < X; ++x)
          dkb[x] = fmaf(tau * dsh, load_elem<BF16>(Qsc, r * D + lane + kWave * x), dkb[x]);
        dbs += dsh;
      }
      __syncthreads();
    }
    // combine the summary-key gradients of the four waves in a fixed order
#pragma unroll
    for (int x = 0; x < X; ++x) part[w][lane + kWave * x] = dkb[x];
    if (lane == 0) part[w][D] = dbs;
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int x = 0; x < X; ++x)
        dkb[x] = ((part[0][lane + kWave * x] + part[1][lane + kWave * x]) +
                  part[2][lane + kWave * x]) + part[3][lane + kWave * x];
      const float db = ((part[0][D] + part[1][D]) + part[2][D]) + part[3][D];
      const long long sidx = ((long long)b * dm.NCcap + c) * dm.H + h;
      float qlx[X], kbx[X];
#pragma unroll
      for (int x = 0; x < X; ++x) {
        qlx[x] = load_elem<BF16>(Ql, sidx * D + lane + kWave * x);
        kbx[x] = ksum[sidx * D + lane + kWave * x];
      }
      const float L = lse_l[sidx], bias = ent[sidx];
      float s1 = 0.0f, dkd = 0.0f;
#pragma unroll 8
      for (int e = 0; e < D; ++e) {
        const float kje = kt[lane][e];
        s1 = fmaf(bcast(qlx[e / kWave], e % kWave), kje, s1);
        dkd = fmaf(bcast(dkb[e / kWave], e % kWave), kje - bcast(kbx[e / kWave], e % kWave), dkd);
      }
      s1 *= tau;
      const float p1 = expf(s1 - L);
      const float ds1 = p1 * (dkd + db * (L - s1 - bias));
      float gql[X];
#pragma unroll
      for (int x = 0; x < X; ++x) gql[x] = 0.0f;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        const float pj = bcast(p1, j), dsj = bcast(ds1, j);
#pragma unroll
        for (int x = 0; x < X; ++x) {
          gql[x] = fmaf(tau * dsj, kt[j][lane + kWave * x], gql[x]);
          dk[j * X + x] = fmaf(pj, dkb[x], fmaf(tau * dsj, qlx[x], dk[j * X + x]));
        }
      }
#pragma unroll
      for (int x = 0; x < X; ++x) store_elem<BF16>(dQl, sidx * D + lane + kWave * x, gql[x]);
    }
    __syncthreads();
  }

  // reduce the per-wave dK and dV partials in a fixed wave order and store
  for (int pass = 0; pass < 2; ++pass) {
    float* acc = pass == 0 ? dk : dv;
    for (int ww = 0; ww < 4; ++ww) {
      if (w == ww) {
#pragma unroll
        for (int j = 0; j < kChunk; ++j)
#pragma unroll
          for (int x = 0; x < X; ++x)
            red[j][lane + kWave * x] = ww == 0 ? acc[j * X + x] : red[j][lane + kWave * x] + acc[j * X + x];
      }
      __syncthreads();
    }
    void* out = pass == 0 ? dK : dV;
    for (int x = threadIdx.x; x < kChunk * D; x += blockDim.x) {
      const int j = x / D, e = x % D;
      store_elem<BF16>(out, kv_base + (key0 + j) * kv_stride + e, red[j][e]);
    }
    __syncthreads();
  }
}

template <bool BF16, int D>
hipError_t launch_t(const Dims& dm, const void* Q, const void* K, const void* V, const void* Ql,
                    const float* ksum, const float* ent, const float* lse_l, const int32_t* idx,
                    const float* score, const float* lse_tot, const void* O, const void* dO,
                    void* dQ, void* dK, void* dV, void* dQl, const void* Qs, void* dQs, void* ws,
                    hipStream_t st) {
  const WsLayout L = ws_layout(dm);
  char* base = reinterpret_cast<char*>(ws);
  float* dsh = reinterpret_cast<float*>(base + L.dsh);
  float* Dr = reinterpret_cast<float*>(base + L.dr);
  uint32_t* bm = reinterpret_cast<uint32_t*>(base + L.bitmap);
  const int NC = dm.Tkv / dm.S;
  hipError_t err = hipSuccess;
  if (backward_mfma_try(dm, Q, K, V, Ql, ksum, ent, lse_l, idx, score, lse_tot, O, dO, dQ, dK,
                        dV, dQl, Qs, dQs, Dr, dsh, base + L.mfma, st, &err))
    return err;
  // words per bitmap block: as many as 64 KiB of LDS holds, at most 16
  int wpw = 16;
  while (wpw > 1 && (size_t)NC * wpw * 4 > 65536) wpw /= 2;
  if ((size_t)NC * wpw * 4 <= 65536) {
    hipLaunchKernelGGL(k_sel_bitmap_lds, dim3((L.words + wpw - 1) / wpw, dm.H, dm.B), dim3(256),
                       (size_t)NC * wpw * 4, st, dm, idx, bm, L.words, wpw);
  } else {
    const long long nbm = (long long)dm.B * dm.H * NC * L.words;
    hipLaunchKernelGGL(k_fill_zero, dim3(1024), dim3(256), 0, st, bm, nbm);
    hipLaunchKernelGGL(k_sel_bitmap, dim3(1024), dim3(256), 0, st, dm, idx, bm, L.words);
  }
  hipLaunchKernelGGL((k_bwd_rows<BF16, D>), dim3((dm.Tq + 3) / 4, dm.H, dm.B), dim3(256), 0, st,
                     dm, Q, K, V, ksum, idx, score, lse_tot, dO, dQ, dQs, dsh, Dr);
  hipLaunchKernelGGL((k_bwd_kv<BF16, D>), dim3(NC, dm.Hkv, dm.B), dim3(256), 0, st, dm, Q,
                     Qs ? Qs : Q, K, V,
                     Ql, ksum, ent, lse_l, idx, score, lse_tot, dO, dsh, Dr, bm, L.words, dK, dV,
                     dQl);
  return hipGetLastError();
}

}  // namespace

size_t backward_ws_bytes(const Dims& dm) { return ws_layout(dm).total; }

hipError_t launch_backward(const Dims& dm, const void* Q, const void* K, const void* V,
                           const void* Ql, const float* ksum, const float* ent, const float* lse_l,
                           const int32_t* idx, const float* score, const float* lse_tot,
                           const void* O, const void* dO, void* dQ, void* dK, void* dV,
                           void* dQl, const void* Qs, void* dQs, void* ws, hipStream_t st) {
  if ((long long)dm.B * dm.Tq * dm.H == 0) return hipSuccess;
#define HILS_BWD(BF, DD)                                                                      \
  return launch_t<BF, DD>(dm, Q, K, V, Ql, ksum, ent, lse_l, idx, score, lse_tot, O, dO, dQ, \
                          dK, dV, dQl, Qs, dQs, ws, st)
  if (dm.bf16) {
    if (dm.d == 64) HILS_BWD(true, 64);
    HILS_BWD(true, 128);
  }
  if (dm.d == 64) HILS_BWD(false, 64);
  HILS_BWD(false, 128);
#undef HILS_BWD
}

}  // namespace hils
