// HiLS attention — CPU ORACLE. TEST INFRASTRUCTURE ONLY.
//
// A plain, slow, single-threaded fp64 implementation of what the HiLS hot path
// computes. Only the tests, the smoke check and the benchmark's CPU baseline
// load it; the product library never does, and this file shares no code,
// header, table or helper with the HIP path.
//
// Source: "Hierarchical Sparse Attention Done Right: Toward Infinite Context
// Modeling" (arXiv 2607.02980), as summarised on papers.chlience.com
// (page 2 below) and on the Tide summary page (page 4 below):
//   * page 2 §3 (naive block sparse attention): exact chunk mass
//     Z_{i,c} = sum_{j in chunk c} exp(q_i.k_j / sqrt d).
//   * page 2 §5.1 (Proposition 3.1): landmark softmax p_j over the chunk's keys,
//     summary key k'_c = sum p_j k_j, entropy bias b'_c = -sum p_j log p_j.
//   * page 2 §5.2: chunk score s^_{i,c} = q_i.k'_c / sqrt d + b'_c and the
//     top-K set I_i = {c in C_i : rank_desc(s^_{i,c}) < K}.
//   * page 2 §5.3 and page 4 Fig. 3: hierarchical weights — intra-chunk softmax
//     exp(s_ij)/Z_{i,c(j)} times inter-chunk share Z^_{i,c}/Z^_i, Z^_{i,c} =
//     exp(s^_{i,c}), Z^_i summing the selected surrogates plus the exact mass of
//     the local branch.
//
// Readings taken where the pages are silent (each is restated in the tests):
//   * the local branch is, by default (window 0), the query's own chunk up to
//     the query, attended causally with its exact log-sum-exp entering Z^_i;
//     candidates C_i are the complete chunks strictly before it;
//   * with a sliding window of W > 0 tokens (page 2 §5.2 main setting: W = 512)
//     the local branch is the last W keys [max(0, pos - W + 1), pos] and the
//     candidates are the chunks lying wholly before the window's first key
//     (a chunk the window cuts is not a candidate; its keys before the window
//     are not attended);
//   * the landmark query is per query head and attends the S keys of its
//     chunk (not itself); landmark tokens hold no key/value;
//   * ties in the score rank go to the lower chunk index; rows with fewer
//     than K candidates select all of them (idx padded with -1);
//   * a selection list handed to the attention or the backward counts entry k
//     only when its id is a candidate of the row (0 <= c < n_cand) and larger
//     than every earlier entry of the row; any other entry (padding, an id
//     outside the candidates, a repeated or out-of-order id) contributes
//     nothing, neither its output nor its score. Lists made by the selection
//     (ascending, padded last) count every real entry;
//   * the scale 1/sqrt(d) is applied in all three softmaxes (page 4 Fig. 3
//     caption says it is only omitted there for readability).
//
// Backward: the pages give no gradient formulas; the gradients here follow
// from the forward above by the chain rule with the selected indices held
// fixed (page 2 §5.3: the score enters the forward weights so the loss
// gradient reaches k'_c, b'_c and the landmark query; unselected chunks
// receive nothing).
//
// Layouts (row-major, all double): Q [B,Tq,H,d]; K, V [B,Tkv,Hkv,d];
// Ql [B,NC,H,d]; ksum [B,NC,H,d]; ent, lse_l [B,NC,H]; idx int32 and
// score [B,Tq,H,Ksel]; O [B,Tq,H,d]; lse_own, lse_tot, gap [B,Tq,H].
// Query row i sits at absolute position q_pos0 + i and sees keys 0..pos.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

double dot(const double* a, const double* b, int d) {
  double s = 0.0;
  for (int e = 0; e < d; ++e) s += a[e] * b[e];
  return s;
}

// log(sum_j exp(x_j)), max-shifted.
double logsumexp(const std::vector<double>& x) {
  if (x.empty()) return -INFINITY;
  double m = -INFINITY;
  for (double v : x) m = std::max(m, v);
  if (m == -INFINITY) return -INFINITY;
  double s = 0.0;
  for (double v : x) s += std::exp(v - m);
  return m + std::log(s);
}

struct Shape {
  int B, Tq, Tkv, H, Hkv, d, S, NC, Ksel;
  long q_pos0;
  double scale;
  long window;  // local branch: 0 = own chunk, W > 0 = the last W keys
  // first key of the local branch of the query at absolute position pos
  long local_start(long pos) const {
    return window > 0 ? std::max(0L, pos - window + 1) : (pos / S) * S;
  }
  // candidate chunks: 0 .. n_cand(pos) - 1, the chunks wholly before the local branch
  long n_cand(long pos) const { return local_start(pos) / S; }
  const double* q(const double* Q, int b, int i, int h) const {
    return Q + (((long)b * Tq + i) * H + h) * d;
  }
  const double* kv(const double* X, int b, long j, int g) const {
    return X + (((long)b * Tkv + j) * Hkv + g) * d;
  }
  long row(int b, int i, int h) const { return ((long)b * Tq + i) * H + h; }
};

double resolve_scale(double scale, int d) { return scale != 0.0 ? scale : 1.0 / std::sqrt((double)d); }

// Landmark summary of chunk c for query head h (page 2 §5.1, Proposition 3.1):
// s'_j = tau Ql.k_j, p = softmax(s'), k' = sum p_j k_j, b' = -sum p_j log p_j.
// log p_j is written as s'_j - L' with L' = logsumexp(s'), so p_j -> 0 gives 0.
void summary_one(const Shape& sh, const double* K, const double* ql, int b, int c, int g,
                 double* ksum, double* ent, double* lse) {
  const int S = sh.S, d = sh.d;
  std::vector<double> s(S);
  for (int j = 0; j < S; ++j) s[j] = sh.scale * dot(ql, sh.kv(K, b, (long)c * S + j, g), d);
  const double L = logsumexp(s);
  for (int e = 0; e < d; ++e) ksum[e] = 0.0;
  double H = 0.0;
  for (int j = 0; j < S; ++j) {
    const double p = std::exp(s[j] - L);
    const double* k = sh.kv(K, b, (long)c * S + j, g);
    for (int e = 0; e < d; ++e) ksum[e] += p * k[e];
    H -= p * (s[j] - L);
  }
  *ent = H;
  if (lse) *lse = L;
}

// Scores of every candidate chunk for one row (page 2 §5.2).
void row_scores(const Shape& sh, const double* Q, const double* ksum, const double* ent, int b,
                int i, int h, std::vector<double>& out) {
  const long pos = sh.q_pos0 + i;
  const int n = (int)sh.n_cand(pos);
  out.resize(n);
  const double* q = sh.q(Q, b, i, h);
  for (int c = 0; c < n; ++c) {
    const long sidx = ((long)b * sh.NC + c) * sh.H + h;
    out[c] = sh.scale * dot(q, ksum + sidx * sh.d, sh.d) + ent[sidx];
  }
}

// Softmax attention of one query over keys [j0, j1] of kv head g: returns the
// log-sum-exp of the logits and the normalised output o (length d).
double chunk_attend(const Shape& sh, const double* q, const double* K, const double* V, int b,
                    long j0, long j1, int g, double* o, std::vector<double>* probs = nullptr) {
  const int d = sh.d;
  std::vector<double> s;
  for (long j = j0; j <= j1; ++j) s.push_back(sh.scale * dot(q, sh.kv(K, b, j, g), d));
  const double L = logsumexp(s);
  for (int e = 0; e < d; ++e) o[e] = 0.0;
  if (probs) probs->assign(s.size(), 0.0);
  for (long j = j0; j <= j1; ++j) {
    const double p = std::exp(s[j - j0] - L);
    if (probs) (*probs)[j - j0] = p;
    const double* v = sh.kv(V, b, j, g);
    for (int e = 0; e < d; ++e) o[e] += p * v[e];
  }
  return L;
}

// Forward of one row given its selected set: per selected chunk the intra-chunk
// softmax output o_c and log-mass m_c; the local branch's output and log-mass
// (l_own); fusion logits (selected scores plus the local log-mass), their
// log-sum-exp and O.
struct RowFwd {
  std::vector<int> chunks;        // selected chunk ids (pads dropped)
  std::vector<double> logit;      // s^_{i,c} for selected chunks
  std::vector<double> m;          // intra-chunk log-sum-exp per selected chunk
  std::vector<std::vector<double>> o;  // normalised intra-chunk outputs
  double l_own = 0, Lambda = 0;
  std::vector<double> o_own, O;
};

// Entries of a selection list that count (see the readings above): a candidate
// id above every earlier entry of the row. counted[k] says whether entry k does.
void counted_entries(const Shape& sh, const int* idx_row, long pos, std::vector<bool>& counted) {
  counted.assign(sh.Ksel, false);
  const long n = sh.n_cand(pos);
  long seen = -1;  // largest id among the earlier entries
  for (int k = 0; k < sh.Ksel; ++k) {
    const long c = idx_row[k];
    counted[k] = c >= 0 && c < n && c > seen;
    seen = std::max(seen, c);
  }
}

// idx_row / score_row: the row's Ksel selected ids (-1 = pad) and their scores.
void row_forward(const Shape& sh, const double* Q, const double* K, const double* V,
                 const int* idx_row, const double* score_row, int b, int i, int h, RowFwd& f) {
  const int d = sh.d, S = sh.S, g = h / (sh.H / sh.Hkv);
  const long pos = sh.q_pos0 + i;
  const double* q = sh.q(Q, b, i, h);
  std::vector<bool> counted;
  counted_entries(sh, idx_row, pos, counted);
  f.chunks.clear(); f.logit.clear(); f.m.clear(); f.o.clear();
  for (int k = 0; k < sh.Ksel; ++k) {
    const int c = idx_row[k];
    if (!counted[k]) continue;
    f.chunks.push_back(c);
    f.logit.push_back(score_row[k]);
    std::vector<double> oc(d);
    f.m.push_back(chunk_attend(sh, q, K, V, b, (long)c * S, (long)c * S + S - 1, g, oc.data()));
    f.o.push_back(oc);
  }
  f.o_own.assign(d, 0.0);
  f.l_own = chunk_attend(sh, q, K, V, b, sh.local_start(pos), pos, g, f.o_own.data());
  std::vector<double> all(f.logit);
  all.push_back(f.l_own);
  f.Lambda = logsumexp(all);
  f.O.assign(d, 0.0);
  for (size_t k = 0; k < f.chunks.size(); ++k) {
    const double a = std::exp(f.logit[k] - f.Lambda);
    for (int e = 0; e < d; ++e) f.O[e] += a * f.o[k][e];
  }
  const double a_own = std::exp(f.l_own - f.Lambda);
  for (int e = 0; e < d; ++e) f.O[e] += a_own * f.o_own[e];
}

void list_rows(const Shape& sh, long nrows, const long* rows, std::vector<long>& out) {
  out.clear();
  if (rows) {
    out.assign(rows, rows + nrows);
  } else {
    const long n = (long)sh.B * sh.Tq * sh.H;
    out.resize(n);
    for (long r = 0; r < n; ++r) out[r] = r;
  }
}

}  // namespace

extern "C" {

// Landmark summaries for chunks [c_begin, c_end) of every (batch, query head).
// lse_l may be NULL.
void oracle_summarize(int B, int Tkv, int H, int Hkv, int d, int S, int NC, double scale,
                      const double* K, const double* Ql, int c_begin, int c_end, double* ksum,
                      double* ent, double* lse_l) {
  Shape sh{B, 0, Tkv, H, Hkv, d, S, NC, 0, 0, resolve_scale(scale, d), 0};
  const int G = H / Hkv;
  for (int b = 0; b < B; ++b)
    for (int c = c_begin; c < c_end; ++c)
      for (int h = 0; h < H; ++h) {
        const long sidx = ((long)b * NC + c) * H + h;
        summary_one(sh, K, Ql + sidx * d, b, c, h / G, ksum + sidx * d, ent + sidx,
                    lse_l ? lse_l + sidx : nullptr);
      }
}

// Chunk scores and top-K selection (page 2 §5.2). For each listed row
// (flattened (b*Tq+i)*H+h; rows==NULL means all), idx receives the selected
// chunk ids in ascending order padded with -1, score the matching s^ padded
// with -inf, gap the difference between the K-th and (K+1)-th largest score
// (+inf when the row has at most K candidates).
void oracle_score_topk(int B, int Tq, long q_pos0, int H, int d, int S, int NC, int Ksel,
                       double scale, long window, const double* Q, const double* ksum,
                       const double* ent,
                       long nrows, const long* rows, int* idx, double* score, double* gap) {
  Shape sh{B, Tq, 0, H, 0, d, S, NC, Ksel, q_pos0, resolve_scale(scale, d), window};
  std::vector<long> rl;
  list_rows(sh, nrows, rows, rl);
  std::vector<double> s;
  std::vector<int> order;
  for (long r : rl) {
    const int h = (int)(r % H);
    const int i = (int)((r / H) % Tq);
    const int b = (int)(r / ((long)H * Tq));
    row_scores(sh, Q, ksum, ent, b, i, h, s);
    const int n = (int)s.size();
    order.resize(n);
    for (int c = 0; c < n; ++c) order[c] = c;
    // rank by score descending; equal scores go to the lower chunk index
    std::sort(order.begin(), order.end(), [&](int a, int c) {
      if (s[a] != s[c]) return s[a] > s[c];
      return a < c;
    });
    const int take = std::min(n, Ksel);
    std::vector<int> sel(order.begin(), order.begin() + take);
    std::sort(sel.begin(), sel.end());
    for (int k = 0; k < Ksel; ++k) {
      idx[r * Ksel + k] = k < take ? sel[k] : -1;
      score[r * Ksel + k] = k < take ? s[sel[k]] : -INFINITY;
    }
    if (gap) gap[r] = n > Ksel ? s[order[Ksel - 1]] - s[order[Ksel]] : INFINITY;
  }
}

// Group-max selection for GQA (page 2 §5.4): the chunk scores of every query
// head of a kv head are computed as above and aggregated by their maximum over
// the G heads of the group; the top-K of the aggregated scores (equal scores to
// the lower chunk) is the one index set of every head of the group. idx is that
// set in ascending order for each listed row; score is the row's own head score
// of each selected chunk; gap is taken on the aggregated scores.
void oracle_score_topk_group(int B, int Tq, long q_pos0, int H, int Hkv, int d, int S, int NC,
                             int Ksel, double scale, long window, const double* Q,
                             const double* ksum,
                             const double* ent, long nrows, const long* rows, int* idx,
                             double* score, double* gap) {
  Shape sh{B, Tq, 0, H, Hkv, d, S, NC, Ksel, q_pos0, resolve_scale(scale, d), window};
  const int G = H / Hkv;
  std::vector<long> rl;
  list_rows(sh, nrows, rows, rl);
  std::vector<double> own, other, agg;
  std::vector<int> order;
  for (long r : rl) {
    const int h = (int)(r % H);
    const int i = (int)((r / H) % Tq);
    const int b = (int)(r / ((long)H * Tq));
    const int g = h / G;
    row_scores(sh, Q, ksum, ent, b, i, h, own);
    agg = own;
    for (int hh = g * G; hh < g * G + G; ++hh) {
      row_scores(sh, Q, ksum, ent, b, i, hh, other);
      for (size_t c = 0; c < agg.size(); ++c) agg[c] = std::max(agg[c], other[c]);
    }
    const int n = (int)agg.size();
    order.resize(n);
    for (int c = 0; c < n; ++c) order[c] = c;
    std::sort(order.begin(), order.end(), [&](int a, int c) {
      if (agg[a] != agg[c]) return agg[a] > agg[c];
      return a < c;
    });
    const int take = std::min(n, Ksel);
    std::vector<int> sel(order.begin(), order.begin() + take);
    std::sort(sel.begin(), sel.end());
    for (int k = 0; k < Ksel; ++k) {
      idx[r * Ksel + k] = k < take ? sel[k] : -1;
      score[r * Ksel + k] = k < take ? own[sel[k]] : -INFINITY;
    }
    if (gap) gap[r] = n > Ksel ? agg[order[Ksel - 1]] - agg[order[Ksel]] : INFINITY;
  }
}

// Exact log chunk masses log Z_{i,c} (page 2 §3, naive block sparse attention)
// of every candidate chunk; entries of other chunks are -inf. out is [rows][NC].
void oracle_exact_chunk_lse(int B, int Tq, int Tkv, long q_pos0, int H, int Hkv, int d, int S,
                            int NC, double scale, long window, const double* Q, const double* K,
                            long nrows,
                            const long* rows, double* out) {
  Shape sh{B, Tq, Tkv, H, Hkv, d, S, NC, 0, q_pos0, resolve_scale(scale, d), window};
  std::vector<long> rl;
  list_rows(sh, nrows, rows, rl);
  std::vector<double> tmp(d);
  for (long r : rl) {
    const int h = (int)(r % H);
    const int i = (int)((r / H) % Tq);
    const int b = (int)(r / ((long)H * Tq));
    const long n = sh.n_cand(q_pos0 + i);
    for (int c = 0; c < NC; ++c) {
      double v = -INFINITY;
      if (c < n) {
        const double* q = sh.q(Q, b, i, h);
        std::vector<double> s(S);
        for (int j = 0; j < S; ++j)
          s[j] = sh.scale * dot(q, sh.kv(K, b, (long)c * S + j, h / (H / Hkv)), d);
        v = logsumexp(s);
      }
      out[r * NC + c] = v;
    }
  }
}

// Intra-chunk attention over each selected chunk plus the local branch (the
// causal own chunk, or the last `window` keys), fused by the inter-chunk
// softmax (page 2 §5.3, page 4 Fig. 3). lse_own (the local branch's log-mass)
// and lse_tot may be NULL.
void oracle_attend_fuse(int B, int Tq, int Tkv, long q_pos0, int H, int Hkv, int d, int S,
                        int Ksel, double scale, long window, const double* Q, const double* K,
                        const double* V, const int* idx, const double* score, long nrows,
                        const long* rows, double* O, double* lse_own, double* lse_tot) {
  Shape sh{B, Tq, Tkv, H, Hkv, d, S, 0, Ksel, q_pos0, resolve_scale(scale, d), window};
  std::vector<long> rl;
  list_rows(sh, nrows, rows, rl);
  RowFwd f;
  for (long r : rl) {
    const int h = (int)(r % H);
    const int i = (int)((r / H) % Tq);
    const int b = (int)(r / ((long)H * Tq));
    row_forward(sh, Q, K, V, idx + r * Ksel, score + r * Ksel, b, i, h, f);
    for (int e = 0; e < d; ++e) O[r * d + e] = f.O[e];
    if (lse_own) lse_own[r] = f.l_own;
    if (lse_tot) lse_tot[r] = f.Lambda;
  }
}

// Gradients of sum(dO * O) with the selected indices held fixed. The forward is
// recomputed from Q, K, V, Ql (summaries and scores included). With Q-Cal
// (page 2 §5.4) the chunk scores use a separate scoring query Qs (the
// calibrated q^ = q + W_up W_down h, formed by the caller): the scores' part
// of the query gradient then goes to dQs and dQ keeps the token-attention
// part; Qs == NULL means the scores use Q and dQs is not written. row_mask
// [B*Tq*H] selects the rows whose dQ is produced; kv_mask [B*NC*Hkv] selects the
// (chunk, kv head) pairs whose dK, dV rows and whose dQl rows (heads of that
// group) are produced. NULL masks mean everything. Entries outside the masks are
// left untouched. idx must be the selection made from these inputs.
void oracle_backward(int B, int Tq, int Tkv, long q_pos0, int H, int Hkv, int d, int S, int NC,
                     int Ksel, double scale, long window, const double* Q, const double* K,
                     const double* V,
                     const double* Ql, const int* idx, const double* dO,
                     const unsigned char* row_mask, const unsigned char* kv_mask, double* dQ,
                     double* dK, double* dV, double* dQl, const double* Qs, double* dQs) {
  Shape sh{B, Tq, Tkv, H, Hkv, d, S, NC, Ksel, q_pos0, resolve_scale(scale, d), window};
  const double tau = sh.scale;
  const int G = H / Hkv;
  auto kv_on = [&](int b, long c, int g) {
    if (!kv_mask) return true;
    return c < NC && kv_mask[((long)b * NC + c) * Hkv + g] != 0;
  };
  // summaries of every chunk (forward), needed for the scores
  std::vector<double> ksum((long)B * NC * H * d), ent((long)B * NC * H), lse((long)B * NC * H);
  oracle_summarize(B, Tkv, H, Hkv, d, S, NC, scale, K, Ql, 0, NC, ksum.data(), ent.data(),
                   lse.data());
  // gradient accumulators for the summaries (k' and b')
  std::vector<double> dks((long)B * NC * H * d, 0.0), db((long)B * NC * H, 0.0);
  std::vector<double> gK((long)B * Tkv * Hkv * d, 0.0), gV((long)B * Tkv * Hkv * d, 0.0);
  std::vector<double> dq(d), dqs(d);
  RowFwd f;
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < Tq; ++i)
      for (int h = 0; h < H; ++h) {
        const long r = sh.row(b, i, h);
        const int g = h / G;
        const long pos = q_pos0 + i;
        const long l0 = sh.local_start(pos);
        bool need = !row_mask || row_mask[r];
        for (long c = l0 / S; c <= pos / S && !need; ++c) need = kv_on(b, c, g);
        for (int k = 0; k < Ksel && !need; ++k) {
          const int c = idx[r * Ksel + k];
          if (c >= 0 && kv_on(b, c, g)) need = true;
        }
        if (!need) continue;
        // scores of the selected chunks from the summaries (page 2 §5.2), with
        // the scoring query (Q-Cal) when one is given
        const double* q = sh.q(Q, b, i, h);
        const double* qs = Qs ? sh.q(Qs, b, i, h) : q;
        std::vector<double> sc(Ksel);
        std::vector<bool> counted;
        counted_entries(sh, idx + r * Ksel, pos, counted);
        for (int k = 0; k < Ksel; ++k) {
          const int c = idx[r * Ksel + k];
          if (!counted[k]) { sc[k] = -INFINITY; continue; }
          const long sidx = ((long)b * NC + c) * H + h;
          sc[k] = tau * dot(qs, ksum.data() + sidx * d, d) + ent[sidx];
        }
        row_forward(sh, Q, K, V, idx + r * Ksel, sc.data(), b, i, h, f);
        const double* go = dO + r * d;
        const double D = dot(go, f.O.data(), d);
        for (int e = 0; e < d; ++e) dq[e] = dqs[e] = 0.0;
        double* dq_score = Qs ? dqs.data() : dq.data();  // where the score's query gradient goes
        // selected chunks
        for (size_t k = 0; k < f.chunks.size(); ++k) {
          const int c = f.chunks[k];
          const double a = std::exp(f.logit[k] - f.Lambda);
          const double rc = dot(go, f.o[k].data(), d);
          const double dsh = a * (rc - D);  // gradient of the fusion logit s^_{i,c}
          const long sidx = ((long)b * NC + c) * H + h;
          const double* kb = ksum.data() + sidx * d;
          for (int e = 0; e < d; ++e) dq_score[e] += tau * dsh * kb[e];
          for (int e = 0; e < d; ++e) dks[sidx * d + e] += tau * dsh * qs[e];
          db[sidx] += dsh;
          for (int j = 0; j < S; ++j) {
            const long key = (long)c * S + j;
            const double* kj = sh.kv(K, b, key, g);
            const double* vj = sh.kv(V, b, key, g);
            const double p = std::exp(tau * dot(q, kj, d) - f.m[k]);
            const double ds = a * p * (dot(go, vj, d) - rc);
            for (int e = 0; e < d; ++e) dq[e] += tau * ds * kj[e];
            if (kv_on(b, c, g)) {
              double* gk = gK.data() + (((long)b * Tkv + key) * Hkv + g) * d;
              double* gv = gV.data() + (((long)b * Tkv + key) * Hkv + g) * d;
              for (int e = 0; e < d; ++e) gk[e] += tau * ds * q[e];
              for (int e = 0; e < d; ++e) gv[e] += a * p * go[e];
            }
          }
        }
        // local branch: weights w_j = exp(s_j - Lambda); its log-mass is also a fusion logit
        for (long key = l0; key <= pos; ++key) {
          const double* kj = sh.kv(K, b, key, g);
          const double* vj = sh.kv(V, b, key, g);
          const double w = std::exp(tau * dot(q, kj, d) - f.Lambda);
          const double ds = w * (dot(go, vj, d) - D);
          for (int e = 0; e < d; ++e) dq[e] += tau * ds * kj[e];
          if (kv_on(b, key / S, g)) {
            double* gk = gK.data() + (((long)b * Tkv + key) * Hkv + g) * d;
            double* gv = gV.data() + (((long)b * Tkv + key) * Hkv + g) * d;
            for (int e = 0; e < d; ++e) gk[e] += tau * ds * q[e];
            for (int e = 0; e < d; ++e) gv[e] += w * go[e];
          }
        }
        if (!row_mask || row_mask[r]) {
          for (int e = 0; e < d; ++e) dQ[r * d + e] = dq[e];
          if (Qs)
            for (int e = 0; e < d; ++e) dQs[r * d + e] = dqs[e];
        }
      }
  // landmark summaries: k' = sum p'_j k_j, b' = L' - sum p'_j s'_j with p' = softmax(s')
  for (int b = 0; b < B; ++b)
    for (int c = 0; c < NC; ++c)
      for (int h = 0; h < H; ++h) {
        const int g = h / G;
        if (!kv_on(b, c, g)) continue;
        const long sidx = ((long)b * NC + c) * H + h;
        const double* ql = Ql + sidx * d;
        const double* kb = ksum.data() + sidx * d;
        const double* dkb = dks.data() + sidx * d;
        std::vector<double> gql(d, 0.0);
        for (int j = 0; j < S; ++j) {
          const long key = (long)c * S + j;
          const double* kj = sh.kv(K, b, key, g);
          const double s1 = tau * dot(ql, kj, d);
          const double p = std::exp(s1 - lse[sidx]);
          double dk_dot = 0.0;
          for (int e = 0; e < d; ++e) dk_dot += dkb[e] * (kj[e] - kb[e]);
          const double ds1 = p * (dk_dot + db[sidx] * (lse[sidx] - s1 - ent[sidx]));
          for (int e = 0; e < d; ++e) gql[e] += tau * ds1 * kj[e];
          double* gk = gK.data() + (((long)b * Tkv + key) * Hkv + g) * d;
          for (int e = 0; e < d; ++e) gk[e] += p * dkb[e] + tau * ds1 * ql[e];
        }
        for (int e = 0; e < d; ++e) dQl[sidx * d + e] = gql[e];
      }
  for (int b = 0; b < B; ++b)
    for (int c = 0; c < NC; ++c)
      for (int g = 0; g < Hkv; ++g) {
        if (!kv_on(b, c, g)) continue;
        for (int j = 0; j < S; ++j) {
          const long off = (((long)b * Tkv + (long)c * S + j) * Hkv + g) * d;
          for (int e = 0; e < d; ++e) { dK[off + e] = gK[off + e]; dV[off + e] = gV[off + e]; }
        }
      }
  // keys of an incomplete trailing chunk (decode caches) only receive local-branch terms
  const long tail0 = (long)NC * S;
  for (int b = 0; b < B; ++b)
    for (long key = tail0; key < Tkv; ++key)
      for (int g = 0; g < Hkv; ++g) {
        if (kv_mask) continue;
        const long off = (((long)b * Tkv + key) * Hkv + g) * d;
        for (int e = 0; e < d; ++e) { dK[off + e] = gK[off + e]; dV[off + e] = gV[off + e]; }
      }
}

}  // extern "C"
