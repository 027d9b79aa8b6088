/*
 * hils.h — C ABI of the HiLS (Hierarchical Landmark Sparse) attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * The method is the one described in "Hierarchical Sparse Attention Done
 * Right: Toward Infinite Context Modeling" (arXiv 2607.02980); citations below
 * name the papers.chlience.com research note ("note") and the Tide summary page
 * ("Tide") with their section or figure.
 *
 * Conventions shared by every entry point
 *  - Tensors are contiguous, row-major device buffers, 16-byte aligned:
 *      Q, O, dO, dQ     [B, Tq, H, d]            (dtype of the call)
 *      K, V, dK, dV     [B, Tkv_cap, Hkv, d]     (dtype of the call)
 *      Ql, dQl          [B, NC_cap, H, d]        (dtype of the call)
 *      ksum             [B, NC_cap, H, d]        float32
 *      ent, lse_l       [B, NC_cap, H]           float32
 *      idx              [B, Tq, H, K]            int32
 *      score            [B, Tq, H, K]            float32
 *      lse_own, lse_tot [B, Tq, H]               float32
 *    Query row i sits at absolute position q_pos0 + i and sees key rows
 *    0 .. q_pos0 + i. Chunk c covers key rows [c*S, (c+1)*S). Query head h
 *    uses kv head h / (H / Hkv).
 *  - The library never allocates or frees memory and never synchronises.
 *    Every call only enqueues work on `stream` (NULL = the default stream);
 *    results are valid once the caller has synchronised that stream. Scratch
 *    memory comes from the caller's workspace `ws` of at least the size that
 *    hils_workspace_size reports (ws may be NULL when that size is 0).
 *  - Argument errors return before anything is enqueued and leave outputs
 *    untouched; nothing aborts or prints. HILS_ERR_HIP reports a launch error
 *    read back with hipGetLastError.
 *  - Calls are stateless: concurrent calls on different streams are safe as
 *    long as they do not share output or workspace buffers.
 *  - Supported: S = 64, d in {64, 128}, 1 <= K <= 64, H % Hkv == 0,
 *    dtype float32 or bf16 (float32 accumulation everywhere). Other values
 *    of S, d or K return HILS_ERR_UNSUPPORTED.
 */
#ifndef HILS_H_
#define HILS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HILS_OK = 0,
  HILS_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, inconsistent sizes */
  HILS_ERR_UNSUPPORTED = 2,  /* valid but unsupported shape (S, d, K) */
  HILS_ERR_WORKSPACE = 3,    /* ws smaller than hils_workspace_size */
  HILS_ERR_HIP = 4,          /* a kernel launch failed */
  HILS_ERR_SCRATCH = 5       /* hils_score_topk_noalloc: more scratch than the library holds */
} hils_status;

typedef enum { HILS_F32 = 0, HILS_BF16 = 1 } hils_dtype;

/* Chunk selection of hils_score_topk. PER_HEAD: every query head selects its own
 * chunks. GROUP_MAX (note §5.4, GQA): the chunk scores of the G = H/Hkv query
 * heads of a kv head are aggregated by their maximum and the top K of that is
 * the one chunk set of all G heads; requires G to be a power of two. */
typedef enum { HILS_SELECT_PER_HEAD = 0, HILS_SELECT_GROUP_MAX = 1 } hils_select;

/* A hipStream_t passed as an opaque pointer; NULL means the default stream. */
typedef void* hils_stream;

typedef struct {
  int32_t B;        /* batch */
  int32_t Tq;       /* query rows per batch element */
  int32_t Tkv;      /* valid key rows per batch element */
  int32_t Tkv_cap;  /* key rows allocated per batch element in K/V (0 => Tkv) */
  int32_t NC_cap;   /* chunk slots per batch element in Ql/ksum/ent/lse_l (0 => Tkv_cap/S) */
  int32_t H;        /* query heads */
  int32_t Hkv;      /* kv heads, H % Hkv == 0 */
  int32_t d;        /* head dimension (64 or 128) */
  int32_t S;        /* chunk size (64) */
  int32_t K;        /* selected past chunks per (query, head), 1..64 */
  int32_t dtype;    /* hils_dtype of Q, K, V, Ql, O, dO, dQ, dK, dV, dQl */
  int32_t select_mode; /* hils_select of hils_score_topk; 0 for the other calls */
  int64_t q_pos0;   /* absolute position of query row 0; q_pos0 + Tq <= Tkv */
  float scale;      /* softmax scale; 0 => 1/sqrt(d) */
  int32_t window;   /* local branch: 0 = the query's own chunk (keys from its start
                       up to the query); W > 0 = a sliding window of the last W keys
                       (note §5.2 main setting: 512), W a multiple of S, <= 32 S.
                       The same value must be passed to every call of a forward
                       and its backward. */
} hils_dims;

enum {
  HILS_OP_SUMMARIZE = 0,
  HILS_OP_SCORE_TOPK = 1,
  HILS_OP_ATTEND_FUSE = 2,
  HILS_OP_BACKWARD = 3,
  HILS_OP_DECODE = 4
};

/* Bytes of workspace the operation `op` needs for these dims. */
hils_status hils_workspace_size(const hils_dims* dims, int op, size_t* bytes);

/*
 * Landmark summaries (note §5.1, Proposition 3.1; note §5.2 landmark token).
 * For every batch element b, chunk c in [c_begin, c_end) and query head h
 * (kv head g = h / (H/Hkv)), over the S keys j of chunk c:
 *   s'_j = scale * Ql[b,c,h] . K[b,j,g],   lse_l = log sum_j exp(s'_j),
 *   p'_j = exp(s'_j - lse_l),   ksum = sum_j p'_j K[b,j,g],
 *   ent  = -sum_j p'_j log p'_j.
 * Requires 0 <= c_begin <= c_end <= Tkv/S and c_end <= NC_cap. Only those
 * chunk slots are written; lse_l may be NULL (it is needed by hils_backward).
 * Used incrementally by decode: summarise a chunk once it is complete.
 */
hils_status hils_summarize(const hils_dims* dims, const void* K, const void* Ql,
                           int32_t c_begin, int32_t c_end, float* ksum, float* ent,
                           float* lse_l, void* ws, size_t ws_bytes, hils_stream stream);

/*
 * Chunk scoring and top-K selection (note §5.2, score and top-K equations).
 * Q here is the query the scores use: with Q-Cal (note §5.4) pass the
 * calibrated scoring query q^ = q + W_up W_down h (formed by the caller), and
 * the token query q to hils_attend_fuse.
 * Row (b,i,h) at position p = q_pos0+i has candidates c < floor(l_p/S), the
 * complete chunks before its local branch, whose first key l_p is the start of
 * its own chunk floor(p/S)*S (window 0) or max(0, p - W + 1) (window W > 0; a
 * chunk the window cuts is not a candidate), with score
 *   s^_{i,c} = scale * Q[b,i,h] . ksum[b,c,h] + ent[b,c,h]   (float32).
 * The min(K, n_i) best candidates (score descending, equal scores to the
 * lower chunk id) are written to idx in ascending chunk id, padded with -1,
 * and their scores to score, padded with -inf. ksum/ent must hold every
 * candidate chunk of the last row. With dims->select_mode ==
 * HILS_SELECT_GROUP_MAX the ranking uses max over the kv group's query heads
 * of s^ (same order key); idx is then equal for the heads of a group and each
 * head's score holds its own s^ of the selected chunks.
 */
hils_status hils_score_topk(const hils_dims* dims, const void* Q, const float* ksum,
                            const float* ent, int32_t* idx, float* score, void* ws,
                            size_t ws_bytes, hils_stream stream);

/*
 * hils_score_topk without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). Same arguments, semantics and results (bit for bit) as
 * hils_score_topk; its scratch is a static 16 MiB device buffer of the library,
 * one per GPU, held until the process ends (16 MiB covers every shape whose
 * hils_workspace_size(.., HILS_OP_SCORE_TOPK, ..) is at most 16 MiB; larger ones
 * return HILS_ERR_SCRATCH before anything is enqueued). The copy of the current
 * device is used: make the stream's device current. All calls on one GPU share
 * that buffer, so calls that overlap on one GPU (concurrent streams, or host
 * threads) race and must be serialised by the caller; nothing in it needs to
 * start at zero. The call itself allocates nothing.
 */
hils_status hils_score_topk_noalloc(const hils_dims* dims, const void* Q, const float* ksum,
                                    const float* ent, int32_t* idx, float* score,
                                    hils_stream stream);

/*
 * K and V may also be pinned host memory (hipHostMalloc) in hils_summarize and
 * hils_attend_fuse: a decode cache kept off the GPU (the youleyou.com news
 * article on HiLS-Attention, its first section and Q&A: the KV cache of the
 * chunks a query does not select sits in CPU memory). The kernels read it through
 * its device mapping, so a decode step moves only the chunks it selected and
 * its local branch over the host link; the summaries stay in device memory.
 * Pageable host memory returns HILS_ERR_INVALID_ARG.
 */

/*
 * Selection lists passed to hils_attend_fuse and hils_backward. Entry k of a
 * row's list (idx[b,i,h,k], with its score) counts only when its id c is a
 * candidate of the row (0 <= c < n_i, the candidates of hils_score_topk) and
 * is larger than every earlier entry k' < k of the same row. Any other entry
 * (padding -1, an id outside the candidates, a repeated or out-of-order id)
 * contributes nothing: neither its chunk's output nor its score. The lists
 * hils_score_topk writes (ascending, padding last) count every real entry.
 * No input makes a kernel read outside its buffers.
 */

/*
 * Intra-chunk attention and inter-chunk fusion (note §5.3 hierarchical
 * softmax; Tide Fig. 3). For row (b,i,h) at position p:
 *   each counted entry c (see above): o_c = softmax_j(scale q.k_j) V over its S keys;
 *   local branch, keys l_p .. p (l_p as in hils_score_topk: the own chunk's
 *   start, or the sliding window's first key): o_own = softmax over those keys
 *   and its log-mass l_own;
 *   Lambda = log(sum_c exp(score_c) + exp(l_own));
 *   O = sum_c exp(score_c - Lambda) o_c + exp(l_own - Lambda) o_own.
 * Sums over c run over the counted entries.
 * lse_own (l_own) and lse_tot (Lambda) may be NULL; hils_backward needs them.
 */
hils_status hils_attend_fuse(const hils_dims* dims, const void* Q, const void* K,
                             const void* V, const int32_t* idx, const float* score, void* O,
                             float* lse_own, float* lse_tot, void* ws, size_t ws_bytes,
                             hils_stream stream);

/*
 * One decode step of the query rows at positions q_pos0 .. q_pos0 + Tq - 1 (note
 * §5.2 chunk scores and top-K; note §5.3 hierarchical softmax; the note's key
 * result 5 times HiLS decode per token): the selection of hils_score_topk and the
 * attention of hils_attend_fuse in one call, with the same results (bit for
 * bit, idx and score included). For a few rows it enqueues the candidate splits
 * scored into local top-K lists, then one workgroup per (selected or local
 * chunk, row) that merges the row's lists itself and attends to its chunk, then
 * the fusion of the slots; with many rows (128 and more, e.g. sequences decoding
 * together) one workgroup per row merges its lists once, attends every slot and
 * fuses them; in between the merge runs once per row as its own kernel before
 * the slots. ws is one workspace of
 * hils_workspace_size(.., HILS_OP_DECODE, ..) bytes for all of it (it may be
 * larger than either call's alone); its contents do not matter. K and V may be
 * pinned host memory as for hils_attend_fuse; lse_own and lse_tot may be NULL.
 */
hils_status hils_decode(const hils_dims* dims, const void* Q, const void* K, const void* V,
                        const float* ksum, const float* ent, int32_t* idx, float* score, void* O,
                        float* lse_own, float* lse_tot, void* ws, size_t ws_bytes,
                        hils_stream stream);

/*
 * Training backward with the selection held fixed (note §5.3: the chunk
 * score enters the forward weights, so the loss gradient reaches the summary
 * key, the entropy bias and the landmark query; unselected chunks get none).
 * Given dO, writes (overwrites) dQ, dK, dV and dQl: the gradients of
 * sum(dO * O) through the inter-chunk softmax (scores and local log-mass), the
 * intra-chunk softmaxes, the scores (Q, ksum, ent) and the landmark softmax
 * (Ql, K). dK/dV sum over the query heads of each kv head. Inputs are the
 * forward's: Q, K, V, Ql, ksum, ent, lse_l, idx, score, lse_tot and its
 * output O, which gives each row's D = dO . O (the weighted mean of dO . v
 * over everything the row attends to). Q-Cal (note §5.4): when the scores were
 * computed from a separate scoring query, pass it as Qs [B, Tq, H, d]; the
 * summary-key gradient then uses Qs, dQs [B, Tq, H, d] receives the gradient
 * through the chunk scores and dQ only the one through the token attention
 * (the caller back-propagates dQs into its calibration weights and adds it to
 * the query's gradient). Qs and dQs are both NULL (scores from Q, dQ holds
 * both parts) or both set. Requires a prefill layout (q_pos0 == 0,
 * Tq == Tkv, Tkv % S == 0). idx entries count by the rule above, as in the
 * forward. Deterministic: no floating-point atomics.
 */
hils_status hils_backward(const hils_dims* dims, const void* Q, const void* K, const void* V,
                          const void* Ql, const float* ksum, const float* ent,
                          const float* lse_l, const int32_t* idx, const float* score,
                          const float* lse_tot, const void* O, const void* dO, void* dQ,
                          void* dK, void* dV, void* dQl, const void* Qs, void* dQs, void* ws,
                          size_t ws_bytes, hils_stream stream);

/* Static description of a status code. */
const char* hils_status_string(hils_status status);

/* Library version, 100 * major + minor. */
int32_t hils_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HILS_H_ */
