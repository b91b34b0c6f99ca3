// Internal launcher interface between the C ABI (api.cpp) and the HIP kernels.
// Arguments arrive already validated; launchers only pick a specialisation,
// size the grid and enqueue. Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lsa {

struct IndexTokensArgs {
    int B, T, N, H, D;
    const int32_t *ctx_len;
    const uint16_t *q;      // bf16 [B][T][H][D]
    const float *w;         // [B][T][H]
    const void *k;          // bf16 or fp8 [B][N][D]
    bool fp8;
    bool qf8;               // fp8 keys only: query rows quantised to fp8, fp8 x fp8 contraction
    const float *k_scale;   // [B][N] or null
    const int32_t *kept;    // HI fine: [B][T][n_keep] or null
    int n_keep, block_size;
    float *scores;          // [B][T][n_out]
    int n_out;
    uint32_t *sel_hist;     // optional: selection histogram [B*T][kSelBins] to add candidates to
    int sink, window;       // forced set excluded from sel_hist (and from the emitted candidates)
    // optional (four query rows a workgroup, whole rows): every candidate whose score can
    // still be among its row's K - |forced| largest is appended to cand[row] as its 64-bit
    // composite (order key << 32 | ~position); cand_cnt[row] receives the count
    uint64_t *cand;         // [B*T][N]
    uint32_t *cand_cnt;     // [B*T]
    int K;                  // the selection budget (the fill is K - |forced|)
};
hipError_t launch_index_tokens(const IndexTokensArgs &a, hipStream_t s);
// true when the indexer can emit its rows' candidates (a.cand): flat rows scored by the
// kernel that gives each of four waves one whole query row (many query tokens)
bool index_tokens_emits(int B, int T, int N, int H, int D, bool hi);

bool index_tokens_supported(int H, int D, bool hi);
// true when the token kernel for (H, T, hi) builds sel_hist in its epilogue (one query
// per workgroup); otherwise sel_hist must be built by launch_select_hist.
bool index_tokens_fused_hist(int H, int T, bool hi);

struct IndexBlocksArgs {
    int B, T, N, H, D;
    const int32_t *ctx_len;
    const uint16_t *q;
    const float *w;
    const float *kbar;      // [B][n_blocks][D]
    int n_blocks, block_size, sink, window;
    float *scores;          // [B][T][n_blocks]
    uint32_t *sel_hist;     // optional: per (b, t) the first-level histogram of the finite scores
};
hipError_t launch_index_blocks(const IndexBlocksArgs &a, hipStream_t s);
// The next launch_index_tokens kernel launch on this host thread records its start and end
// into these events (taken from the dispatch); null, null: none.
void set_index_launch_events(hipEvent_t start, hipEvent_t stop);
// The next attention call's first kernel launch on this host thread records its start
// into `start`, its last kernel launch its end into `stop` (taken from the dispatches).
void set_attend_launch_events(hipEvent_t start, hipEvent_t stop);

struct BlockMeansArgs {
    int B, N, D;
    const void *k;
    bool fp8;
    const float *k_scale;
    int block_size, n_blocks;
    float *kbar;
};
hipError_t launch_block_means(const BlockMeansArgs &a, hipStream_t s);

// Cache append (the decode step's write side): new token t of sequence b goes to
// position pos0[b] + t (pos0 NULL: N - T); positions outside [0, N) are skipped.
struct CacheAppendArgs {
    int B, T, N, D;
    const int32_t *pos0;
    const uint16_t *k_new;        // bf16 [B][T][D]
    void *k_cache;                // fp8 or bf16 [B][N][D]
    bool fp8;
    float *k_scale;               // [B][N] (fp8)
    int n_rows;                   // row sets copied (0..2)
    const uint16_t *rows_new[2];  // bf16 [B][T][row_elems]
    uint16_t *rows_cache[2];      // bf16, element (b, s, e) at b*stride_b + s*stride_n + e
    int64_t row_elems[2], stride_b[2], stride_n[2];
    float *kbar;                  // optional [B][n_blocks][D]
    int block_size, n_blocks;
};
hipError_t launch_cache_append(const CacheAppendArgs &a, hipStream_t s);

// Backward of the sparse attention for one layer (selection fixed): dq, and the gradients
// of the selected K/V rows summed over the queries that selected them.
struct AttendBwdArgs {
    int B, T, N, Hq, Hkv, K;
    const uint16_t *q;      // bf16 [B][T][Hq][d_qk]
    const uint16_t *k;      // bf16, element (b, s, h, d) at b*ksb + s*ksn + h*ksh + d
    int64_t ksb, ksn, ksh;
    const uint16_t *v;      // bf16 (MLA: v == k, the first 512 columns)
    int64_t vsb, vsn, vsh;
    const int32_t *idx;     // [B][T][K]: valid entries ascending, then -1
    float scale;
    const uint16_t *out;    // bf16 [B][T][Hq][d_v] (forward output)
    const float *lse;       // [B][T][Hq]
    const uint16_t *dout;   // bf16 [B][T][Hq][d_v]
    float *dq;              // [B][T][Hq][d_qk]
    float *dk;              // [B][N][Hkv][d_qk] (MLA: dK + dV on the first d_v columns)
    float *dv;              // [B][N][Hkv][d_v], null for MLA
    bool mla;
};
size_t attend_bwd_workspace_bytes(const AttendBwdArgs &a);

// Indexer distillation target: per query token, the head-averaged attention distribution
// over its selected rows, the indexer's softmax over the same rows, their KL and its
// gradient with respect to the indexer scores.
struct IndexTargetArgs {
    int B, T, N, Hq, Hkv, K, dqk;
    const uint16_t *q;      // bf16 [B][T][Hq][dqk]
    const uint16_t *k;      // bf16, element (b, s, h, d) at b*ksb + s*ksn + h*ksh + d
    int64_t ksb, ksn, ksh;
    const int32_t *idx;     // [B][T][K]
    float scale;
    const float *lse;       // [B][T][Hq]
    const float *scores;    // [B][T][n_cols], column = position
    int n_cols;
    float *target, *grad;   // [B][T][K]
    float *loss;            // [B][T]
};
hipError_t launch_index_target(const IndexTargetArgs &a, hipStream_t s);
hipError_t launch_attend_bwd(const AttendBwdArgs &a, void *ws, hipStream_t s);

struct SelectArgs {
    int B, T, N;
    const int32_t *ctx_len;
    const float *scores;
    int n_cols;
    const int32_t *kept;
    int n_keep, block_size;
    int K, sink, window;
    bool causal;
    bool ws_clean;          // histogram already zero (left so by a same-shape call)
    bool primed;            // histogram already built for these scores (by the indexer)
    bool vec;               // rows 16-byte aligned (n_cols % 4 == 0 and aligned scores)
    int32_t *idx;
};
size_t select_workspace_bytes(int rows, int n_cols, bool kept);
size_t select_zero_bytes(int rows);  // the part of the workspace kept at zero between calls
hipError_t launch_select(const SelectArgs &a, void *ws, hipStream_t s);
// true when launch_select runs the one-launch selection of small rows (n_cols columns):
// it reads no histogram from the workspace (a primed one is not needed) and leaves the
// workspace clean
bool select_small(int n_cols);
// The selection of flat rows from the candidate lists the indexer emitted (cand [rows][N],
// cand_cnt [rows]); one workgroup per row, nothing else in the workspace.
hipError_t launch_select_cand(const SelectArgs &a, const uint64_t *cand, const uint32_t *cand_cnt, hipStream_t s);
bool select_cand_fits(int n_cols);
// Histogram pass alone (the selection's first pass), for an index call that primes a
// selection workspace with a kernel that cannot build it in its epilogue.
hipError_t launch_select_hist(const SelectArgs &a, void *ws, hipStream_t s);
// The selection up to its last pass (the histogram pass unless primed, then the filter
// pass), for an attention launch that resolves the selection itself.
hipError_t launch_select_front(const SelectArgs &a, void *ws, hipStream_t s);

struct AttendArgs {
    int B, T, N, Hq, Hkv, d_qk, d_v;
    const uint16_t *q;
    const uint16_t *k;
    int64_t ksb, ksn, ksh;
    const uint16_t *v;
    int64_t vsb, vsn, vsh;
    const int32_t *idx;
    int K;
    float scale;
    void *out;
    bool out_f32;
    float *lse;
    int L;
    int64_t lsq, lsk, lsv, lso, lsl;
    int n_splits;           // resolved (>= 1)
    const int32_t *bt;      // paged caches: block table [B][max_pages] (pool page of each
    int page_size, max_pages, num_pages;  // logical page), else null; pool of num_pages pages
    bool idx_shared;        // one index row per sequence for all T query tokens, each masked
    const int32_t *ctx_len; // to positions <= its own p = ctx_len[b] - T + t (null: N)
};
constexpr int kAttendMaxSplits = 128;  // split partials merged by one combine workgroup
int attend_default_splits(const AttendArgs &a);
size_t attend_workspace_bytes(const AttendArgs &a);
bool attend_supported(int d_qk, int d_v, int g);
hipError_t launch_attend(const AttendArgs &a, void *ws, hipStream_t s);
// The split-partial buffer of lsa_attend_noalloc: a static device array of this size,
// one per GPU; *ptr receives device dev's copy (looked up once per device).
constexpr size_t kAttendStaticScratchBytes = (size_t)32 << 20;
hipError_t attend_static_scratch(int dev, void **ptr);
// Selection (flat rows, no kept map) and attention on its output in one chain: the
// attention workgroups resolve their own slices of the selection (sa.idx written too).
// a.idx is ignored; sa and a describe the same B, T, N, K.
hipError_t launch_select_attend(const SelectArgs &sa, void *sel_ws, const AttendArgs &a, void *ws, hipStream_t s);

hipError_t launch_clear(void *p, size_t bytes, hipStream_t s);

}  // namespace lsa
