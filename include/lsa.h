/*
 * lsa.h — C ABI of liblsa.so, the MI355X (gfx950) hot path of LongCat Sparse
 * Attention (LSA): index -> select -> attend.
 *
 * The method, as the LongCat pages state it:
 *   - LSA extends DeepSeek Sparse Attention with three indexing mechanisms
 *     ("LongCat-2.0: how Meituan trained a 1.6T coding model without Nvidia GPUs",
 *     molayo1419.me, section "The sparse attention problem at 1M tokens").
 *   - Streaming-aware Indexing (SI) spends part of each query token's selection
 *     budget on a fixed sink and a local sliding window, so that KV reads become
 *     contiguous ("LongCat-Flash-Lite-Sparse" summary, aitrends.kr, sections
 *     "Good to know" and "Technical features", first bullet).
 *   - Hierarchical Indexing (HI) first picks coarse candidate blocks, then
 *     selects fine tokens inside them; it can be switched on at inference (same
 *     page, "Technical features", third bullet; "Training").
 *   - Cross-Layer Indexing (CLI) reuses one index result in several consecutive
 *     layers (same page, second bullet; molayo1419.me, CLI paragraph).
 *   - Attention runs over the selected tokens only, never over all token pairs
 *     ("LongCat-2.0" summary, aitrends.kr, "Technical features").
 * The pages give no formula for the indexer; this library computes the DSA-style
 * score  I[t,s] = scale[s] * sum_h w[t,h] * ReLU(q[t,h] . k[s])  (reading R1).
 *
 * Conventions (all functions):
 *   - Every pointer inside a descriptor is a DEVICE pointer unless stated; every
 *     array is dense row-major with the stated shape unless strides are given.
 *     Tensors read with vector loads (q, w, k, v, scores, kbar) must be 16-byte
 *     aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Work
 *     is enqueued on it; no call synchronises, allocates device memory, or keeps
 *     a pointer after it returns. The library has no mutable global state, apart
 *     from the static per-GPU buffer of lsa_attend_noalloc.
 *   - Query token t of sequence b sits at position p = ctx_len[b] - T + t
 *     (reading R11); ctx_len NULL means every sequence has N visible rows.
 *     Positions s > p are never visible to query t.
 *   - Return value: LSA_OK (0) or a negative status. On a negative status nothing
 *     was enqueued, except LSA_E_HIP (a launch failed; lsa_last_error() tells
 *     which). Argument checks run on the host before any HIP call.
 *   - Determinism: repeated calls on identical inputs give identical bytes (no
 *     floating-point atomics; every reduction has a fixed order).
 */
#ifndef LSA_H
#define LSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LSA_VERSION 1

/* status codes */
#define LSA_OK 0
#define LSA_E_NULL (-1)        /* a required pointer is NULL */
#define LSA_E_SHAPE (-2)       /* a size is out of range or inconsistent */
#define LSA_E_DTYPE (-3)       /* unknown or unsupported dtype code */
#define LSA_E_BUDGET (-4)      /* K < 1, or sink + window > K */
#define LSA_E_ALIGN (-5)       /* a pointer or stride breaks the 16-byte rule */
#define LSA_E_UNSUPPORTED (-6) /* no compiled kernel for this shape (no slow fallback exists) */
#define LSA_E_WORKSPACE (-7)   /* workspace NULL or smaller than the *_workspace_bytes() answer */
#define LSA_E_HIP (-8)         /* a HIP launch failed */

/* element types */
#define LSA_BF16 1
#define LSA_FP8_E4M3FN 2 /* OCP E4M3 without infinities (gfx950 native), max 448 */
#define LSA_F32 3

/* lsa_select workspace states */
#define LSA_WS_UNKNOWN 0
#define LSA_WS_CLEAN 1
#define LSA_WS_PRIMED 2 /* prepared by lsa_index for exactly the scores it wrote */

/* lsa_index modes */
#define LSA_INDEX_TOKENS 0
#define LSA_INDEX_BLOCKS 1

/*
 * lsa_index — indexer scores (the DSA-style indexer the LSA pages build on).
 *
 * TOKENS, flat (kept == NULL): for every query token (b,t) and position s < N
 *   scores[b][t][s] = k_scale[b][s] * sum_h w[b][t][h] * max(0, q[b][t][h] . k[b][s])
 *   for s <= p, and -inf for s > p. k_scale is NULL for bf16 keys (scale 1).
 *   The contraction runs as bf16 x bf16 products with fp32 accumulation; fp8 keys
 *   are widened exactly to bf16.
 *   q_dtype = LSA_FP8_E4M3FN (fp8 keys, D = 128, TOKENS only; reading R27: the DSA
 *   indexer that LSA extends contracts in fp8, molayo1419.me LongCat-2.0 article,
 *   "The sparse attention problem at 1M tokens"): each query row q[b][t][h] is first
 *   quantised as the fp8 key rows are, s_q = max(max_d |q|, 1e-12) / 448 and codes
 *   c = e4m3fn(clamp(q / s_q, -448, 448)) in fp32, round to nearest even, and the score
 *   uses s_q * c in place of q: k_scale * sum_h (w * s_q) * max(0, c . k), computed as
 *   fp8 x fp8 products with fp32 accumulation (the matrix unit adds the 64 products of
 *   one instruction with a truncated alignment: relative error up to about 2^-11 of
 *   the largest product). q_dtype 0 or LSA_BF16: bf16 queries as above.
 * TOKENS, HI fine stage (kept != NULL): column c of query (b,t) stands for position
 *   s = kept[b][t][c / block_size] * block_size + c % block_size, c < n_keep *
 *   block_size; the score is as above. Columns whose kept entry is -1 or outside
 *   [0, N / block_size), or whose position is > p, get -inf.
 * BLOCKS, HI coarse stage: k is the fp32 block-mean cache kbar[b][n_blocks][D]
 *   (from lsa_block_means) and
 *   scores[b][t][j] = max_h w[b][t][h] * max(0, q[b][t][h] . kbar[b][j])
 *   in fp32 for every block j that is complete and visible (j*block_size +
 *   block_size - 1 <= p) and holds at least one position outside the forced set
 *   sink [0,sink) U window [p-window+1, p]; -inf for every other block (reading R9).
 *
 * Priming a selection: with select_ws != NULL, lsa_index also records in
 *   select_ws what the selection would otherwise compute in a first pass over these
 *   scores (per query token, the distribution of the candidate scores: finite scores at
 *   visible positions outside sink [0,sink) and window [p-window+1, p]). The next
 *   lsa_select must read exactly these scores, with the same B, T, N, ctx_len, kept
 *   map, sink and window, causal = 1, and workspace_state = LSA_WS_PRIMED; no other call
 *   may use select_ws in between. select_ws_bytes must be at least the
 *   lsa_select_workspace_bytes() of that call (256-byte aligned workspace). With
 *   select_ws_state = LSA_WS_UNKNOWN the workspace is cleared first (one fill kernel);
 *   LSA_WS_CLEAN skips that (every successful lsa_select leaves its workspace clean).
 *   With the kept map, window >= block_size - 1 is required, as in lsa_select. Rows of
 *   at most 4096 columns need no priming (lsa_select ranks them in one launch from the
 *   scores alone): for them lsa_index only writes the scores, and the protocol above
 *   still holds.
 *   BLOCKS mode primes the coarse HI block selection the same way ("LongCat-Flash-Lite-
 *   Sparse" summary, Technical features, third bullet: coarse blocks first): the
 *   recorded distribution is that of every finite block score, and the next lsa_select
 *   reads these scores with K = the number of blocks to keep, sink = window = 0,
 *   causal = 0, no kept map and workspace_state = LSA_WS_PRIMED (select_ws_bytes: the
 *   lsa_select_workspace_bytes() of that call).
 *
 * Shapes: q bf16 [B][T][H][D]; w fp32 [B][T][H]; k per k_dtype: bf16 or fp8 [B][N][D]
 * (TOKENS) or fp32 [B][n_blocks][D] (BLOCKS); k_scale fp32 [B][N] (fp8 keys only);
 * kept int32 [B][T][n_keep]; scores fp32 [B][T][n_out] with n_out = N (flat),
 * n_keep*block_size (HI fine) or n_blocks (BLOCKS).
 * Supported: TOKENS D in {64,128}, H in {4,8,16,32,64}, k_dtype bf16 or fp8;
 * BLOCKS D in {64,128}, 1 <= H <= 64, k_dtype f32, window >= block_size - 1 (so the
 * incomplete block at p always lies inside the window and never needs fine scoring;
 * LSA_E_UNSUPPORTED otherwise).
 */
typedef struct lsa_index_desc {
    int32_t mode;            /* LSA_INDEX_TOKENS or LSA_INDEX_BLOCKS */
    int32_t B, T, N;         /* sequences, query tokens per sequence, cache rows per sequence */
    const int32_t *ctx_len;  /* [B] visible rows per sequence, or NULL (= N) */
    int32_t H, D;            /* indexer heads and head dim */
    const void *q;           /* bf16 [B][T][H][D] */
    const float *w;          /* fp32 [B][T][H] */
    const void *k;           /* key cache, see above */
    int32_t k_dtype;         /* LSA_BF16, LSA_FP8_E4M3FN (TOKENS) or LSA_F32 (BLOCKS) */
    const float *k_scale;    /* fp32 [B][N] per-token scale for fp8 keys, else NULL */
    const int32_t *kept;     /* HI fine stage: int32 [B][T][n_keep], else NULL */
    int32_t n_keep;          /* kept blocks per query token (HI fine stage) */
    int32_t block_size;      /* HI block size (HI fine stage and BLOCKS) */
    int32_t n_blocks;        /* BLOCKS: block-mean rows per sequence */
    int32_t sink, window;    /* BLOCKS: forced set used for block eligibility;
                                TOKENS with select_ws: the forced set of the selection */
    float *scores;           /* fp32 [B][T][n_out], written in full */
    void *select_ws;         /* optional: workspace of the lsa_select that reads scores */
    size_t select_ws_bytes;
    int32_t select_ws_state; /* LSA_WS_UNKNOWN or LSA_WS_CLEAN: state of select_ws on entry */
    int32_t q_dtype;         /* TOKENS: 0 or LSA_BF16 (bf16 contraction), LSA_FP8_E4M3FN (reading R27) */
} lsa_index_desc;

int32_t lsa_index(const lsa_index_desc *desc, void *stream);

/*
 * lsa_index_select — lsa_index (flat token scores) and lsa_select (causal token selection,
 * the SI budget of a sink, a local window and a top-k fill) as one call: idx receives exactly
 * what lsa_select would select from the scores lsa_index computes ("LongCat-Flash-Lite-Sparse"
 * summary, aitrends.kr, "Good to know" and "Technical features", first bullet; the scores of
 * reading R1). Two paths, by shape. Few query tokens per sequence: the indexer primes the
 * selection (its epilogue counts the candidates per first-level bin where the kernel has
 * one query per workgroup), so the selection skips its first pass over the scores. Prefill
 * (H in {32, 64}, D in {64, 128}, T >= 64, at least 512 groups of four query tokens over
 * the batch, N <= 2^19): each indexer wave scores one whole row and lists every candidate
 * that can still be among the row's fill when it is scored (a running threshold from the
 * row's histogram so far), and the selection ranks only the lists; the scores are written
 * only when desc->scores is given.
 * Arguments: desc as for lsa_index in TOKENS mode without a kept map, with desc->sink and
 * desc->window the forced set and desc->select_ws ignored; desc->scores may be NULL (the
 * scores then live in the workspace); K the budget (1 <= K <= 4096, sink + window <= K); idx
 * int32 [B][T][K] as lsa_select writes it (ascending positions, then -1).
 * Workspace: lsa_index_select_workspace_bytes(desc, K) bytes, 256-byte aligned: on the
 * prefill path the list lengths (4 bytes per row, rounded up to 256) and the lists (8 bytes
 * per row and position: a list may hold the whole row); otherwise the selection workspace,
 * plus the scores when desc->scores is NULL. workspace_state LSA_WS_UNKNOWN clears what
 * must start at zero (one fill kernel; nothing on the prefill path); LSA_WS_CLEAN skips
 * that and is valid after a successful call with the same B, T and N (every call leaves
 * the workspace clean). Calls sharing a workspace must be ordered on one stream.
 * Errors as lsa_index and lsa_select; LSA_E_UNSUPPORTED for BLOCKS mode or a kept map.
 */
size_t lsa_index_select_workspace_bytes(const lsa_index_desc *desc, int32_t K);
int32_t lsa_index_select(const lsa_index_desc *desc, int32_t K, int32_t *idx, void *workspace, size_t workspace_bytes,
                         int32_t workspace_state, void *stream);

/*
 * lsa_block_means — the block summaries of the HI coarse stage: the mean
 * indexer key of each block of block_size consecutive rows,
 *   kbar[b][j][d] = (1/block_size) * sum_{s=j*bs}^{j*bs+bs-1} k_scale[b][s] * k[b][s][d]
 * computed in fp32 (reading R10), for j < n_blocks (n_blocks * block_size <= N).
 * The cost is amortised: it is recomputed only when the cache changes.
 * Shapes: k bf16 or fp8 [B][N][D]; k_scale fp32 [B][N] (fp8) or NULL; kbar fp32
 * [B][n_blocks][D]. Supported: D in {64,128}, block_size >= 1.
 */
typedef struct lsa_block_means_desc {
    int32_t B, N, D;
    const void *k;
    int32_t k_dtype;         /* LSA_BF16 or LSA_FP8_E4M3FN */
    const float *k_scale;
    int32_t block_size;
    int32_t n_blocks;
    float *kbar;
} lsa_block_means_desc;

int32_t lsa_block_means(const lsa_block_means_desc *desc, void *stream);

/*
 * lsa_select — the SI selection of one budget of K positions per query token
 * (LongCat-Flash-Lite-Sparse summary: the selection budget is split into a fixed
 * sink and a local window; the rest is a top-k fill).
 *
 * causal = 1 (token selection): forced F = [0, min(sink, p+1)) U [max(0, p-window+1), p];
 *   candidates = visible columns whose position is not in F and whose score is
 *   finite; fill m = K - |F| candidates by (score descending, position ascending)
 *   (reading R6; -0.0 and +0.0 are equal), or all of them when there are at most m.
 * causal = 0 (block stage of HI, or any plain top-K): sink and window must be 0;
 *   candidates = every column with a finite score; fill m = K.
 * Positions: column c is position c, or with a candidate map (kept != NULL)
 *   kept[b][t][c / block_size] * block_size + c % block_size (entries -1 or
 *   outside [0, N / block_size) make the column no candidate).
 * Output idx int32 [B][T][K]: the selected positions in ascending order, then -1.
 *
 * Workspace: lsa_select_workspace_bytes(desc) bytes of device memory, 256-byte
 * aligned. With workspace_state = LSA_WS_UNKNOWN the call first clears the state it
 * needs (one small fill kernel), so no initial contents are needed. Every successful
 * call leaves that state zeroed; a caller that reuses a workspace for a call with the
 * same B, T and n_cols (or right after lsa_workspace_clear) may pass LSA_WS_CLEAN to
 * skip the clear. LSA_WS_PRIMED: lsa_index already prepared the workspace for these
 * scores (see lsa_index), so the selection skips its first pass over them.
 * Rows of at most 4096 columns are selected by one workgroup per row in a single
 * launch (the row's keys held in LDS); the workspace state is then ignored and left
 * clean. Longer rows take the histogram, filter and resolve passes.
 * Calls that share one workspace must be ordered on one stream.
 * Supported: 1 <= K <= 4096, n_cols >= 1; with a kept map and causal = 1,
 * window >= block_size - 1 (LSA_E_UNSUPPORTED otherwise).
 */
typedef struct lsa_select_desc {
    int32_t B, T, N;         /* N: cache rows (bounds positions and the kept map) */
    const int32_t *ctx_len;  /* [B] or NULL (= N) */
    const float *scores;     /* fp32 [B][T][n_cols] */
    int32_t n_cols;
    const int32_t *kept;     /* optional column -> position map, int32 [B][T][n_keep] */
    int32_t n_keep, block_size;
    int32_t K, sink, window;
    int32_t causal;          /* 1 token selection at p with forced set, 0 plain top-K */
    int32_t *idx;            /* int32 [B][T][K] */
    int32_t workspace_state; /* LSA_WS_UNKNOWN (0), LSA_WS_CLEAN (1) or LSA_WS_PRIMED (2) */
} lsa_select_desc;

size_t lsa_select_workspace_bytes(const lsa_select_desc *desc);
int32_t lsa_select(const lsa_select_desc *desc, void *workspace, size_t workspace_bytes, void *stream);

/*
 * lsa_attend — softmax attention of each query token over its selected rows only
 * ("LongCat-2.0" summary: no attention over all token pairs), for n_layers
 * consecutive layers that share one selection (CLI).
 *
 * For layer l, query (b,t), query head hq, KV head kvh = hq / (Hq/Hkv) (reading R16):
 *   z_s = softmax_scale * q[l][b][t][hq] . K[l][b][s][kvh]   for s in idx[b][t] (s >= 0)
 *   out[l][b][t][hq] = sum_s softmax(z)_s V[l][b][s][kvh];  lse = log sum_s exp(z_s)
 * bf16 inputs, fp32 accumulation and softmax, bf16 or fp32 output.
 * K element (b,s,h,d) is at k[l*layer_stride_k + b*k_stride_b + s*k_stride_n +
 * h*k_stride_h + d] (elements), d < d_qk; V likewise with the v_* strides, d < d_v.
 * MLA latent rows (reading R15) are expressed with strides: v = k, d_qk = 576,
 * d_v = 512, one KV head.
 * idx int32 [B][T][K]: entries -1 or outside [0, N) are skipped; a query token with no
 * valid entry gets out = 0 and lse = -inf.
 * q bf16 [n_layers][B][T][Hq][d_qk] (layer stride layer_stride_q); out [n_layers][B][T]
 * [Hq][d_v] (layer_stride_out); lse fp32 [n_layers][B][T][Hq] (layer_stride_lse) or NULL.
 * n_splits: how many parts the K rows of one query are split into (0 = library
 * choice; clamped to [ceil(K/2048), min(ceil(K/32), 128)]); partial results are merged
 * in a fixed order.
 * Workspace: lsa_attend_workspace_bytes(desc) bytes (may be 0), 256-byte aligned;
 * no initial contents needed.
 * Supported: (d_qk, d_v) in {(128,128), (576,512)}, Hq % Hkv == 0, Hq/Hkv <= 64,
 * 1 <= K <= 262144, strides multiples of 8 elements.
 * Paged caches (block_table != NULL; reading R26: the "LongCat-Flash-Lite-Sparse"
 * summary, "Good to know", deployment bullet, has the model served by an existing engine
 * whose launcher sets the KV cache dtype and memory split; such engines keep KV in pages
 * named by a per-sequence table): K and V of a
 * layer are one pool of num_pages pages of page_size rows, and position s of sequence
 * b lives in pool row r = block_table[b][s / page_size] * page_size + s % page_size,
 * i.e. K element (b,s,h,d) is at k[l*layer_stride_k + r*k_stride_n + h*k_stride_h + d]
 * (k_stride_b, v_stride_b unused). block_table: device int32 [B][max_pages], owned by
 * the caller, read only. A position whose page index is >= max_pages or whose entry is
 * outside [0, num_pages) is skipped like an invalid idx entry. Results equal those of
 * the contiguous layout holding the same rows, bit for bit. Errors: LSA_E_SHAPE for
 * page_size, max_pages or num_pages < 1, or a pool above 2^31 - 1 rows.
 * With block_table == NULL the three sizes are ignored.
 * Shared selection (idx_shared = 1; reading R29, for draft tokens that share one
 * selection, the MTP extension of LSA in the molayo1419.me LongCat-2.0 article, "The
 * sparse attention problem at 1M tokens"): idx is int32 [B][K], one row per sequence,
 * and query token t of sequence b attends over the entries s of idx[b] with
 * s <= p = ctx_len[b] - T + t (ctx_len: device int32 [B], or NULL for N), so no token sees
 * a later position; a token left with no entry gets out = 0 and lse = -inf. With
 * idx_shared = 0, ctx_len is ignored. lsa_select_attend rejects idx_shared
 * (LSA_E_UNSUPPORTED).
 */
typedef struct lsa_attend_desc {
    int32_t B, T, N;
    int32_t Hq, Hkv, d_qk, d_v;
    const void *q;
    const void *k;
    int64_t k_stride_b, k_stride_n, k_stride_h;
    const void *v;
    int64_t v_stride_b, v_stride_n, v_stride_h;
    const int32_t *idx;
    int32_t K;
    float softmax_scale;
    void *out;
    int32_t out_dtype;       /* LSA_BF16 or LSA_F32 */
    float *lse;              /* optional */
    int32_t n_layers;        /* >= 1 */
    int64_t layer_stride_q, layer_stride_k, layer_stride_v, layer_stride_out, layer_stride_lse;
    int32_t n_splits;
    const int32_t *block_table; /* paged caches: int32 [B][max_pages], or NULL (contiguous) */
    int32_t page_size, max_pages, num_pages;
    int32_t idx_shared;         /* 1: idx is [B][K], one selection shared by the T tokens */
    const int32_t *ctx_len;     /* with idx_shared: [B] visible rows, or NULL (= N) */
} lsa_attend_desc;

size_t lsa_attend_workspace_bytes(const lsa_attend_desc *desc);
int32_t lsa_attend(const lsa_attend_desc *desc, void *workspace, size_t workspace_bytes, void *stream);

/*
 * lsa_attend_noalloc — lsa_attend without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). Same descriptor, results bit-identical to lsa_attend with the
 * same n_splits. The split partials go to a static device buffer of the library
 * (32 MiB, one per GPU, held until the process ends; the call allocates nothing). Every
 * call on a GPU shares that GPU's buffer, which keeps the last call's partials: calls that
 * overlap on one GPU (concurrent streams, threads) race and must be ordered by the caller.
 * Errors as lsa_attend; LSA_E_WORKSPACE when lsa_attend_workspace_bytes(desc) exceeds
 * the buffer (fewer splits, n_splits, shrink it); LSA_E_HIP if the buffer's address cannot
 * be found on the stream's device.
 */
int32_t lsa_attend_noalloc(const lsa_attend_desc *desc, void *stream);

/*
 * lsa_select_attend — lsa_select(sel) followed by lsa_attend(att) on the positions it
 * selects, as one chain: the attention workgroups finish the selection themselves
 * (each the part of the index list it attends over), so the index list does not make
 * a round trip through memory between the two. Same pages as lsa_select and
 * lsa_attend (SI budget of sink, window and top-k fill; attention over the selected
 * tokens only).
 * Results: sel->idx and att->out / att->lse are bit-identical to those of the two
 * calls made separately with the same descriptors (and the same n_splits).
 * Requirements: everything lsa_select and lsa_attend require, and: no kept map
 * (sel->kept == NULL); sel and att agree on B, T, N and K; att->idx is NULL or
 * equal to sel->idx (it is ignored: the positions come from the selection).
 * Workspaces: select_ws as for lsa_select (workspace_state applies as there) and
 * attend_ws as for lsa_attend, with their own *_workspace_bytes() sizes; after a
 * successful call select_ws is clean, as after lsa_select.
 * Errors as for the two calls; LSA_E_UNSUPPORTED for a kept map.
 * Speed: every attention workgroup that shares a selection row repeats the row-level
 * part of the selection, which pays off only with four waves a workgroup (more than 48
 * query heads per KV head) and one KV head of one layer per row; for other shapes the
 * call runs the selection's own resolve kernel and then the plain attention (the same
 * results, never slower than the two calls).
 */
int32_t lsa_select_attend(const lsa_select_desc *sel, const lsa_attend_desc *att, void *select_ws,
                          size_t select_ws_bytes, void *attend_ws, size_t attend_ws_bytes, void *stream);

/*
 * lsa_attend_backward — gradients of lsa_attend (one layer, n_layers = 1) with respect to
 * q, K and V, the selection held fixed (reading R28: the pages' LSA is trained with its
 * sparse operators, and those operators are deterministic: molayo1419.me LongCat-2.0
 * article, "The sparse attention problem at 1M tokens" and "Training on 50,000 Chinese
 * ASICs"). With z_s = softmax_scale q . K_s over the valid entries s of idx[b][t],
 * P_s = exp(z_s - lse), dP_s = dout . V_s, D = dout . out and dS_s = P_s (dP_s - D):
 *   dq[b][t][hq]    = softmax_scale sum_s dS_s K[b][s][kvh]
 *   dk[b][s][kvh]   = softmax_scale sum over (t, hq of kvh) selecting s of dS_s q[b][t][hq]
 *   dv[b][s][kvh]   = sum over (t, hq of kvh) selecting s of P_s dout[b][t][hq]
 * fp32 arithmetic from the bf16 inputs; out and lse are the forward's (lsa_attend with
 * the same idx). Every sum runs in a fixed order (query tokens ascending), so results are
 * reproducible bit for bit; no atomics.
 * Layouts: q, out, dout bf16 [B][T][Hq][d]; lse fp32 [B][T][Hq]; k, v as in lsa_attend
 * (strides in elements); idx int32 [B][T][K] as lsa_select writes it (valid entries
 * strictly ascending, then -1; entries outside [0, N) skipped). Outputs fp32: dq
 * [B][T][Hq][d_qk], written in full; dk [B][N][Hkv][d_qk] and dv [B][N][Hkv][d_v], written
 * only at the rows of positions some query selected: every other row keeps what the caller
 * left there, so a buffer zeroed once (at allocation) receives the dense gradient, with zeros
 * at the unselected positions, and the call moves only the selected rows. MLA (d_qk = 576,
 * d_v = 512, v aliasing k, reading R15): dk is the latent row's gradient, dK plus dV on its
 * first 512 columns, and dv is NULL.
 * Workspace: lsa_attend_backward_workspace_bytes(desc), 256-byte aligned, no initial
 * contents: per-tile parts of dq (32 rows a tile) and, with T > 1, per (query token, KV
 * head, selected row) one row of fp32 contributions (d_qk + d_v floats, MLA d_qk). With
 * T = 1 each selected row has a single contribution, which goes straight to dk / dv.
 * Supported: (d_qk, d_v) in {(128, 128), (576, 512)}, Hq % Hkv == 0, Hq / Hkv <= 64,
 * B * T <= 65535, strides multiples of 8 elements; q, k, v, out, dout, dk, dv 16-byte
 * aligned. Errors as for lsa_attend.
 */
typedef struct lsa_attend_bwd_desc {
    int32_t B, T, N;
    int32_t Hq, Hkv, d_qk, d_v;
    const void *q;
    const void *k;
    int64_t k_stride_b, k_stride_n, k_stride_h;
    const void *v;
    int64_t v_stride_b, v_stride_n, v_stride_h;
    const int32_t *idx;
    int32_t K;
    float softmax_scale;
    const void *out;
    const float *lse;
    const void *dout;
    float *dq, *dk, *dv;
} lsa_attend_bwd_desc;

size_t lsa_attend_backward_workspace_bytes(const lsa_attend_bwd_desc *desc);
int32_t lsa_attend_backward(const lsa_attend_bwd_desc *desc, void *workspace, size_t workspace_bytes, void *stream);

/*
 * lsa_index_target — the indexer distillation target and loss for training the indexer
 * (reading R30; the indexer LSA builds on is DSA's, molayo1419.me LongCat-2.0 article,
 * "The sparse attention problem at 1M tokens"). For query token (b,t) and each valid
 * entry j of idx[b][t] (position s = idx[b][t][j] in [0, N)):
 *   target[b][t][j] = (1/Hq) sum_hq exp(softmax_scale q[b][t][hq] . K[b][s][kvh] - lse[b][t][hq])
 *     (the attention distribution of each head, from lsa_attend's lse, averaged over heads)
 *   u_j = softmax over the valid entries of scores[b][t][s] (the indexer scores)
 *   loss[b][t] = sum_j target_j (log target_j - log u_j) over target_j > 0
 *   grad[b][t][j] = u_j - target_j  (d loss / d scores[b][t][s]; the target held fixed)
 * Padding entries get target 0 and grad 0; a token with no valid entry gets loss 0.
 * fp32 arithmetic from the bf16 inputs; sums in a fixed order (reproducible bits).
 * Layouts: q bf16 [B][T][Hq][d_qk]; k as in lsa_attend (d_qk = 576 for MLA latent rows, or
 * 128); idx int32 [B][T][K]; lse fp32 [B][T][Hq]; scores fp32 [B][T][n_cols] (flat
 * indexer scores, column = position, n_cols >= N); target, grad fp32 [B][T][K]; loss fp32
 * [B][T]. No workspace. Supported: d_qk in {128, 576}, Hq % Hkv == 0, Hq / Hkv <= 64,
 * B * T <= 65535, strides multiples of 8 elements, q and k 16-byte aligned.
 */
typedef struct lsa_index_target_desc {
    int32_t B, T, N;
    int32_t Hq, Hkv, d_qk;
    const void *q;
    const void *k;
    int64_t k_stride_b, k_stride_n, k_stride_h;
    const int32_t *idx;
    int32_t K;
    float softmax_scale;
    const float *lse;
    const float *scores;
    int32_t n_cols;
    float *target, *grad, *loss;
} lsa_index_target_desc;

int32_t lsa_index_target(const lsa_index_target_desc *desc, void *stream);

/*
 * lsa_cache_append — the write side of a decode step: T new tokens per sequence enter the
 * caches that lsa_index and lsa_attend read. SI's local window ends at the current token
 * (reading R4), so a step's rows are appended before the step; HI's coarse pass reads one
 * summary per key block ("LongCat-Flash-Lite-Sparse" summary, "Technical features",
 * first and third bullets), brought up to date here when a block's last row is written
 * (reading R25).
 *
 * New token t of sequence b goes to position s = pos0[b] + t (pos0: device int32 [B],
 * the rows already cached; NULL means N - T, i.e. the last T rows). Positions outside
 * [0, N) are skipped (nothing is written for them).
 *   Indexer key, k_new bf16 [B][T][D] (finite values):
 *     k_dtype LSA_FP8_E4M3FN: k_scale[b][s] = max(max_d |k|, 1e-12) / 448 and
 *       k_cache[b][s][d] = e4m3fn(clamp(k[d] / k_scale[b][s], -448, 448)), fp32 with
 *       correctly rounded divisions, round to nearest even (reading R12, the same
 *       quantisation as the fp8 key caches lsa_index reads);
 *     k_dtype LSA_BF16: k_cache[b][s] = k_new[b][t] (copied).
 *   Row sets (n_rows = 0, 1 or 2; e.g. one MLA latent row, or K and V): row_elems bf16
 *     elements of rows_new[i] [B][T][row_elems] are copied to rows_cache[i] +
 *     b*rows_stride_b[i] + s*rows_stride_n[i] (elements).
 *   kbar (optional, fp32 [B][n_blocks][D]): for every block j = s / block_size whose last
 *     row s ((s + 1) % block_size == 0, j < n_blocks) this call writes, kbar[b][j] is
 *     recomputed from the cache exactly as lsa_block_means computes it (same bytes).
 * Shapes: D in {64, 128}; row_elems, strides multiples of 8; k_new, k_cache, rows
 * 16-byte aligned. Errors as for the other calls (LSA_E_UNSUPPORTED for other D).
 */
typedef struct lsa_cache_append_desc {
    int32_t B, T, N, D;
    const int32_t *pos0;        /* [B] rows already cached, or NULL (= N - T) */
    const void *k_new;          /* bf16 [B][T][D] */
    void *k_cache;              /* fp8 or bf16 [B][N][D] */
    int32_t k_dtype;            /* LSA_FP8_E4M3FN or LSA_BF16 */
    float *k_scale;             /* fp32 [B][N] (fp8 keys), else NULL */
    int32_t n_rows;             /* 0, 1 or 2 */
    const void *rows_new[2];    /* bf16 [B][T][row_elems[i]] */
    void *rows_cache[2];        /* bf16 cache rows, strided */
    int64_t row_elems[2], rows_stride_b[2], rows_stride_n[2];
    float *kbar;                /* optional fp32 [B][n_blocks][D] */
    int32_t block_size, n_blocks;
} lsa_cache_append_desc;

int32_t lsa_cache_append(const lsa_cache_append_desc *desc, void *stream);

/* Measurement hook (not part of the method): the next launch of the token indexer kernel
 * made by lsa_index or lsa_index_select on the calling host thread records its start in
 * start_event and its end in stop_event (hipEvent_t handles created with timing enabled,
 * owned by the caller; either may be NULL), taken from the kernel's own dispatch, so the
 * elapsed time between them is the kernel's execution alone, without the launch latency
 * that a separately recorded event pair around the call adds. The hook applies to one
 * launch and is then cleared; NULL, NULL clears it. Calls that launch no token indexer
 * kernel (BLOCKS mode, errors) leave it set. Returns LSA_OK. */
int32_t lsa_index_launch_events(void *start_event, void *stop_event);

/* Measurement hook (not part of the method), as lsa_index_launch_events for the
 * attention: the next lsa_attend, lsa_attend_noalloc or lsa_select_attend call on the
 * calling host thread records the start of its attention kernel's dispatch in
 * start_event and the end of its last kernel's dispatch (the split merge, or the
 * attention itself when it runs one split) in stop_event, so the elapsed time spans the
 * attention and its merge without the launch latency. The hook applies to one call and is
 * then cleared; NULL, NULL clears it; calls that fail before launching leave it set. In
 * lsa_select_attend the selection kernels that run before the attention are not in the
 * span. Returns LSA_OK. */
int32_t lsa_attend_launch_events(void *start_event, void *stop_event);

/* Zero-fill `bytes` of device memory at `ptr` with a fill kernel (for workspaces). */
int32_t lsa_workspace_clear(void *ptr, size_t bytes, void *stream);

/* Static text for a status code; the last error text of the calling thread. */
const char *lsa_status_str(int32_t status);
const char *lsa_last_error(void);
int32_t lsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LSA_H */
